"""The allocation-free pack entry point (bitlinear_pack_weights_noalloc),
called through the C ABI, against the entry point with a caller workspace
(bitlinear_pack_weights): packed bytes and gamma bit-identical, on calls in
a row whose second input is smaller (the library's static scratch keeps the
first call's partial sums), and the decoded codes and gamma against the
oracle ("BitNet b1.58 in Production", "The Mathematical Mechanism", item 1).
"""
from __future__ import annotations

import ctypes as ct

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_gamma, compare_codes, host, log, to_dev, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def blq():
    torch_mod()
    import bitlinear_quant_act_amd as m
    m.load_library()
    return m


def _ptr(t):
    return ct.c_void_p(t.data_ptr())


def test_noalloc_pack_matches_workspace_pack(blq):
    torch = torch_mod()
    lib = blq.load_library()
    stream = ct.c_void_p(torch.cuda.current_stream().cuda_stream)
    # second call smaller than the first: 1024 partial sums, then 19
    for seed, n, k in ((401, 4096, 14336), (402, 300, 1000), (403, 17, 257)):
        tag = "noalloc pack n=%d k=%d" % (n, k)
        log("case", tag)
        w = synth.latent_weights(seed, n, k)
        wd = to_dev(w)
        nbytes = blq.bitlinear_packed_bytes(n, k)
        ws = blq.bitlinear_pack_workspace_bytes(n, k)
        assert ws <= blq.BITLINEAR_PACK_NOALLOC_SCRATCH_BYTES
        p_ref = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        g_ref = torch.zeros(1, dtype=torch.float32, device="cuda")
        work = torch.empty(ws, dtype=torch.uint8, device="cuda")
        p_na = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
        g_na = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
        rc = lib.bitlinear_pack_weights(_ptr(wd), n, k, _ptr(p_ref), nbytes, _ptr(g_ref), _ptr(work), ws, stream)
        assert rc == 0, rc
        rc = lib.bitlinear_pack_weights_noalloc(_ptr(wd), n, k, _ptr(p_na), nbytes, _ptr(g_na), stream)
        assert rc == 0, rc
        torch.cuda.synchronize()
        assert torch.equal(p_na, p_ref), tag
        assert host(g_na)[0].view(np.uint32) == host(g_ref)[0].view(np.uint32), tag
        g_or = oracle.gamma(w)
        q_or = oracle.ternarize(w, g_or)
        same = check_gamma(host(g_na)[0], g_or, tag)
        compare_codes(host(blq.bitlinear_unpack_weights(p_na, n, k)), q_or, w, g_or, same, tag)


def test_noalloc_pack_rejects_bad_arguments(blq):
    torch = torch_mod()
    lib = blq.load_library()
    w = torch.zeros((16, 256), dtype=torch.float32, device="cuda")
    p = torch.empty(blq.bitlinear_packed_bytes(16, 256), dtype=torch.uint8, device="cuda")
    g = torch.empty(1, dtype=torch.float32, device="cuda")
    assert lib.bitlinear_pack_weights_noalloc(None, 16, 256, _ptr(p), p.numel(), _ptr(g), None) == blq.BITLINEAR_E_NULL
    assert lib.bitlinear_pack_weights_noalloc(_ptr(w), 16, 256, _ptr(p), p.numel() - 1, _ptr(g), None) == blq.BITLINEAR_E_SIZE
    assert lib.bitlinear_pack_weights_noalloc(_ptr(w), 0, 256, _ptr(p), p.numel(), _ptr(g), None) == blq.BITLINEAR_E_SHAPE
