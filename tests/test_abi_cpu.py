"""C-ABI checks that need no GPU: the library loads, exports every function
include/bitlinear.h declares, and rejects bad arguments on the host before
any HIP call (so these run on a machine without a device).  Only argument
combinations that fail validation are passed here; no call reaches a launch.
"""
from __future__ import annotations

import ctypes as ct
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")


@pytest.fixture(scope="module")
def blq():
    import bitlinear_quant_act_amd as m
    # a host-sanitized build of the same sources may be named here (see
    # test_sanitizers.py); by default the in-tree library
    m.load_library(os.environ.get("BITLINEAR_TEST_LIB", m.LIB_PATH))
    return m


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("bitlinear_pack_weights", "bitlinear_quant_act", "bitlinear_forward",
              "bitlinear_forward_batched"):
        assert n in names


def test_every_declared_symbol_is_exported(blq):
    lib = blq.load_library()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # and the Python binding exposes the same names
    assert all(hasattr(blq, n) for n in declared_functions())


def test_single_hip_runtime_mapped(blq):
    assert len(blq._mapped_hip_runtimes()) <= 1


def test_version_and_status_strings(blq):
    assert blq.bitlinear_abi_version() == 2
    for s in range(-7, 1):
        assert blq.bitlinear_status_string(s) not in ("", "unknown status")
    assert blq.bitlinear_status_string(12345) == "unknown status"


def test_packed_bytes(blq):
    # 16 x 256 tiles of 1024 bytes
    assert blq.bitlinear_packed_bytes(2048, 2048) == 2048 * 2048 // 4
    assert blq.bitlinear_packed_bytes(1, 1) == 1024
    assert blq.bitlinear_packed_bytes(17, 257) == 2 * 2 * 1024
    assert blq.bitlinear_packed_bytes(57344, 8192) == 57344 * 8192 // 4
    assert blq.bitlinear_packed_bytes(0, 5) == 0
    assert blq.bitlinear_packed_bytes(5, 0) == 0
    assert blq.bitlinear_packed_bytes(5, (1 << 18) + 1) == 0
    assert blq.bitlinear_packed_bytes(5, 1 << 18) > 0
    assert 8 <= blq.bitlinear_pack_workspace_bytes(2048, 2048) <= 8192
    assert blq.bitlinear_pack_workspace_bytes(57344, 8192) == 8192


# fake device addresses: never dereferenced, every call below fails validation
A16 = 0x10000
A8 = 0x10008
A2 = 0x10002


def test_pack_validation(blq):
    lib = blq.load_library()
    nb = blq.bitlinear_packed_bytes(64, 512)
    ws = blq.bitlinear_pack_workspace_bytes(64, 512)
    E = blq
    assert lib.bitlinear_pack_weights(None, 64, 512, A16, nb, A16, A16, ws, None) == E.BITLINEAR_E_NULL
    assert lib.bitlinear_pack_weights(A16, 64, 512, None, nb, A16, A16, ws, None) == E.BITLINEAR_E_NULL
    assert lib.bitlinear_pack_weights(A16, 64, 512, A16, nb, None, A16, ws, None) == E.BITLINEAR_E_NULL
    assert lib.bitlinear_pack_weights(A16, 64, 512, A16, nb, A16, None, ws, None) == E.BITLINEAR_E_NULL
    assert lib.bitlinear_pack_weights(A16, 0, 512, A16, nb, A16, A16, ws, None) == E.BITLINEAR_E_SHAPE
    assert lib.bitlinear_pack_weights(A16, 64, -3, A16, nb, A16, A16, ws, None) == E.BITLINEAR_E_SHAPE
    assert lib.bitlinear_pack_weights(A16, 64, (1 << 18) + 1, A16, nb, A16, A16, ws, None) == E.BITLINEAR_E_SHAPE
    assert lib.bitlinear_pack_weights(A16, 64, 512, A8, nb, A16, A16, ws, None) == E.BITLINEAR_E_ALIGN
    assert lib.bitlinear_pack_weights(A2, 64, 512, A16, nb, A16, A16, ws, None) == E.BITLINEAR_E_ALIGN
    assert lib.bitlinear_pack_weights(A16, 64, 512, A16, nb, A16, A2, ws, None) == E.BITLINEAR_E_ALIGN
    assert lib.bitlinear_pack_weights(A16, 64, 512, A16, nb - 1, A16, A16, ws, None) == E.BITLINEAR_E_SIZE
    assert lib.bitlinear_pack_weights(A16, 64, 512, A16, nb, A16, A16, ws - 1, None) == E.BITLINEAR_E_SIZE


def test_unpack_and_quant_validation(blq):
    lib = blq.load_library()
    E = blq
    assert lib.bitlinear_unpack_weights(None, 4, 4, A16, None) == E.BITLINEAR_E_NULL
    assert lib.bitlinear_unpack_weights(A16, 4, 4, None, None) == E.BITLINEAR_E_NULL
    assert lib.bitlinear_unpack_weights(A16, 0, 4, A16, None) == E.BITLINEAR_E_SHAPE
    assert lib.bitlinear_unpack_weights(A8, 4, 4, A16, None) == E.BITLINEAR_E_ALIGN
    assert lib.bitlinear_quant_act(None, 1, 8, A16, A16, None) == E.BITLINEAR_E_NULL
    assert lib.bitlinear_quant_act(A16, 1, 8, None, A16, None) == E.BITLINEAR_E_NULL
    assert lib.bitlinear_quant_act(A16, 1, 8, A16, None, None) == E.BITLINEAR_E_NULL
    assert lib.bitlinear_quant_act(A16, 0, 8, A16, A16, None) == E.BITLINEAR_E_SHAPE
    assert lib.bitlinear_quant_act(A16, 1, 0, A16, A16, None) == E.BITLINEAR_E_SHAPE
    assert lib.bitlinear_quant_act(A16 + 1, 1, 8, A16, A16, None) == E.BITLINEAR_E_ALIGN
    assert lib.bitlinear_quant_act(A16, 1, 8, A16, A2, None) == E.BITLINEAR_E_ALIGN


@pytest.mark.parametrize("fname", ["bitlinear_forward", "bitlinear_forward_batched"])
def test_forward_validation(blq, fname):
    fn = getattr(blq.load_library(), fname)
    E = blq
    ok = dict(packed=A16, gamma=A16, n=64, k=512, xq=A16, amax=A16, m=1, y=A16, acc=None)

    def call(**kw):
        a = dict(ok, **kw)
        return fn(a["packed"], a["gamma"], a["n"], a["k"], a["xq"], a["amax"], a["m"], a["y"], a["acc"], None)

    for key in ("packed", "gamma", "xq", "amax", "y"):
        assert call(**{key: None, "n": 64}) == E.BITLINEAR_E_NULL, key
    assert call(n=0) == E.BITLINEAR_E_SHAPE
    assert call(k=0) == E.BITLINEAR_E_SHAPE
    assert call(k=(1 << 18) + 1) == E.BITLINEAR_E_SHAPE
    assert call(m=0) == E.BITLINEAR_E_SHAPE
    assert call(packed=A8) == E.BITLINEAR_E_ALIGN
    assert call(y=A2) == E.BITLINEAR_E_ALIGN
    assert call(gamma=A2) == E.BITLINEAR_E_ALIGN
    assert call(acc=A2) == E.BITLINEAR_E_ALIGN
    if fname == "bitlinear_forward":
        assert call(m=17) == E.BITLINEAR_E_UNSUPPORTED
    else:
        assert call(m=(1 << 21) + 1) == E.BITLINEAR_E_UNSUPPORTED


def test_binding_rejects_host_tensors(blq):
    torch = pytest.importorskip("torch")
    w = torch.zeros(16, 256)
    with pytest.raises(ValueError):
        blq.bitlinear_pack_weights(w)


def test_quant_forward_validation(blq):
    lib = blq.load_library()
    fn = lib.bitlinear_quant_forward
    E = blq
    ok = dict(packed=A16, gamma=A16, n=64, k=512, x=A16, m=1, y=A16, acc=None, xq=None, amax=None)

    def call(**kw):
        a = dict(ok, **kw)
        return fn(a["packed"], a["gamma"], a["n"], a["k"], a["x"], a["m"], a["y"], a["acc"], a["xq"], a["amax"], None)

    for key in ("packed", "gamma", "x", "y"):
        assert call(**{key: None}) == E.BITLINEAR_E_NULL, key
    assert call(xq=A16) == E.BITLINEAR_E_NULL          # codes without a'
    assert call(amax=A16) == E.BITLINEAR_E_NULL        # a' without codes
    assert call(n=0) == E.BITLINEAR_E_SHAPE
    assert call(m=0) == E.BITLINEAR_E_SHAPE
    assert call(packed=A8) == E.BITLINEAR_E_ALIGN
    assert call(x=A16 + 1) == E.BITLINEAR_E_ALIGN
    assert call(m=17) == E.BITLINEAR_E_UNSUPPORTED
    assert call(m=16, k=14336) == E.BITLINEAR_E_UNSUPPORTED
    assert lib.bitlinear_quant_forward_supported(1, 2560) == 1
    assert lib.bitlinear_quant_forward_supported(1, 28672) == 1
    assert lib.bitlinear_quant_forward_supported(2, 14336) == 1
    assert lib.bitlinear_quant_forward_supported(8, 14336) == 1
    assert lib.bitlinear_quant_forward_supported(16, 14336) == 0
    assert lib.bitlinear_quant_forward_supported(17, 256) == 0
    assert lib.bitlinear_quant_forward_supported(0, 256) == 0
    # supported sizes are exactly those whose staged codes (padded rows, 16
    # bytes apart) fit 140 KiB of LDS, beside the 16-wave reduction buffer
    for m in range(1, 17):
        for k in (1, 255, 256, 4096, 6912, 8960, 14336, 28672, 40000, 57344):
            staged = m * (((k + 255) // 256) * 256 + 16)
            assert lib.bitlinear_quant_forward_supported(m, k) == (1 if staged <= 140 * 1024 else 0), (m, k)


def test_norm_and_f32_quant_validation(blq):
    lib = blq.load_library()
    E = blq
    f = lib.bitlinear_rmsnorm_quant_act
    assert f(None, None, 1e-6, 1, 8, A16, A16, None) == E.BITLINEAR_E_NULL
    assert f(A16, None, 1e-6, 1, 8, None, A16, None) == E.BITLINEAR_E_NULL
    assert f(A16, None, 1e-6, 1, 8, A16, None, None) == E.BITLINEAR_E_NULL
    assert f(A16, None, 1e-6, 0, 8, A16, A16, None) == E.BITLINEAR_E_SHAPE
    assert f(A16, None, 1e-6, 1, (1 << 18) + 1, A16, A16, None) == E.BITLINEAR_E_SHAPE
    assert f(A16, None, -1.0, 1, 8, A16, A16, None) == E.BITLINEAR_E_VALUE
    assert f(A16, None, float("inf"), 1, 8, A16, A16, None) == E.BITLINEAR_E_VALUE
    assert f(A16, None, float("nan"), 1, 8, A16, A16, None) == E.BITLINEAR_E_VALUE
    assert f(A16 + 1, None, 1e-6, 1, 8, A16, A16, None) == E.BITLINEAR_E_ALIGN
    assert f(A16, A2, 1e-6, 1, 8, A16, A16, None) == E.BITLINEAR_E_ALIGN
    g = lib.bitlinear_quant_act_f32
    assert g(None, 1, 8, A16, A16, None) == E.BITLINEAR_E_NULL
    assert g(A16, 0, 8, A16, A16, None) == E.BITLINEAR_E_SHAPE
    assert g(A2, 1, 8, A16, A16, None) == E.BITLINEAR_E_ALIGN
    h = lib.bitlinear_rmsnorm_quant_forward
    ok = dict(packed=A16, gamma=A16, n=64, k=512, x=A16, gain=None, eps=1e-6, m=1, y=A16, acc=None, xq=None, amax=None)

    def call(**kw):
        a = dict(ok, **kw)
        return h(a["packed"], a["gamma"], a["n"], a["k"], a["x"], a["gain"], a["eps"], a["m"], a["y"], a["acc"],
                 a["xq"], a["amax"], None)

    for key in ("packed", "gamma", "x", "y"):
        assert call(**{key: None}) == E.BITLINEAR_E_NULL, key
    assert call(xq=A16) == E.BITLINEAR_E_NULL
    assert call(n=0) == E.BITLINEAR_E_SHAPE
    assert call(eps=-2.0) == E.BITLINEAR_E_VALUE
    assert call(gain=A2) == E.BITLINEAR_E_ALIGN
    assert call(packed=A8) == E.BITLINEAR_E_ALIGN
    assert call(m=17) == E.BITLINEAR_E_UNSUPPORTED


def test_swiglu_validation(blq):
    fn = blq.load_library().bitlinear_forward_swiglu
    E = blq
    ok = dict(pg=A16, gg=A16, pu=A16, gu=A16, f=64, k=512, xq=A16, amax=A16, m=1, h=A16, acc=None)

    def call(**kw):
        a = dict(ok, **kw)
        return fn(a["pg"], a["gg"], a["pu"], a["gu"], a["f"], a["k"], a["xq"], a["amax"], a["m"], a["h"], a["acc"], None)

    for key in ("pg", "gg", "pu", "gu", "xq", "amax", "h"):
        assert call(**{key: None}) == E.BITLINEAR_E_NULL, key
    assert call(f=0) == E.BITLINEAR_E_SHAPE
    assert call(m=0) == E.BITLINEAR_E_SHAPE
    assert call(k=(1 << 18) + 1) == E.BITLINEAR_E_SHAPE
    assert call(pu=A8) == E.BITLINEAR_E_ALIGN
    assert call(pg=A8) == E.BITLINEAR_E_ALIGN
    assert call(gu=A2) == E.BITLINEAR_E_ALIGN
    assert call(h=A2) == E.BITLINEAR_E_ALIGN
    assert call(m=(1 << 21) + 1) == E.BITLINEAR_E_UNSUPPORTED


def test_fused_ffn_entry_validation(blq):
    lib = blq.load_library()
    E = blq
    f = lib.bitlinear_rmsnorm_quant_forward_swiglu
    ok = dict(pg=A16, gg=A16, pu=A16, gu=A16, f=64, k=512, x=A16, gain=None, eps=1e-6, m=1, h=A16, acc=None,
              xq=None, amax=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["pg"], a["gg"], a["pu"], a["gu"], a["f"], a["k"], a["x"], a["gain"], a["eps"], a["m"], a["h"],
                 a["acc"], a["xq"], a["amax"], None)

    for key in ("pg", "gg", "pu", "gu", "x", "h"):
        assert call(**{key: None}) == E.BITLINEAR_E_NULL, key
    assert call(amax=A16) == E.BITLINEAR_E_NULL
    assert call(f=0) == E.BITLINEAR_E_SHAPE
    assert call(eps=-1.0) == E.BITLINEAR_E_VALUE
    assert call(pu=A8) == E.BITLINEAR_E_ALIGN
    assert call(x=A16 + 1) == E.BITLINEAR_E_ALIGN
    assert call(m=17) == E.BITLINEAR_E_UNSUPPORTED
    g = lib.bitlinear_quant_forward_f32
    ok2 = dict(packed=A16, gamma=A16, n=64, k=512, x=A16, m=1, y=A16, acc=None, xq=None, amax=None)

    def call2(**kw):
        a = dict(ok2, **kw)
        return g(a["packed"], a["gamma"], a["n"], a["k"], a["x"], a["m"], a["y"], a["acc"], a["xq"], a["amax"], None)

    for key in ("packed", "gamma", "x", "y"):
        assert call2(**{key: None}) == E.BITLINEAR_E_NULL, key
    assert call2(xq=A16) == E.BITLINEAR_E_NULL
    assert call2(m=0) == E.BITLINEAR_E_SHAPE
    assert call2(x=A2) == E.BITLINEAR_E_ALIGN
    assert call2(m=17) == E.BITLINEAR_E_UNSUPPORTED
    assert call2(m=16, k=14336) == E.BITLINEAR_E_UNSUPPORTED


# ---------------------------------------------------------------------------
# variant modes: sizes and host-side validation (nothing reaches a launch)
# ---------------------------------------------------------------------------

def test_variant_sizes(blq):
    # binary tiles: 16 x 512 columns in 1024 bytes (one bit per weight)
    assert blq.bitlinear_packed_bytes_binary(2048, 2048) == 2048 * 2048 // 8
    assert blq.bitlinear_packed_bytes_binary(1, 1) == 1024
    assert blq.bitlinear_packed_bytes_binary(17, 257) == 2 * 1 * 1024
    assert blq.bitlinear_packed_bytes_binary(17, 513) == 2 * 2 * 1024
    assert blq.bitlinear_packed_bytes_binary(0, 5) == 0
    # per-tensor quantisation: one launch (no partials) up to 16384 values, at most 1024 partials
    assert blq.bitlinear_quant_act_tensor_workspace_bytes(1, 16384) == 4
    assert blq.bitlinear_quant_act_tensor_workspace_bytes(2, 16384) == 8
    assert blq.bitlinear_quant_act_tensor_workspace_bytes(4096, 28672) <= 4096
    assert blq.bitlinear_quant_act_tensor_workspace_bytes(0, 8) == 0
    assert blq.bitlinear_quant_forward_binary_supported(1, 28672)
    assert not blq.bitlinear_quant_forward_binary_supported(17, 256)


def test_variant_validation(blq):
    lib = blq.load_library()
    E = blq
    ws = blq.bitlinear_quant_act_tensor_workspace_bytes(64, 512)
    q = lib.bitlinear_quant_act_tensor
    assert q(None, 64, 512, A16, A16, A16, ws, None) == E.BITLINEAR_E_NULL
    assert q(A16, 64, 512, A16, A16, None, ws, None) == E.BITLINEAR_E_NULL
    assert q(A16, 0, 512, A16, A16, A16, ws, None) == E.BITLINEAR_E_SHAPE
    assert q(A16, 64, (1 << 18) + 1, A16, A16, A16, ws, None) == E.BITLINEAR_E_SHAPE
    assert q(A16 + 1, 64, 512, A16, A16, A16, ws, None) == E.BITLINEAR_E_ALIGN
    assert q(A16, 64, 512, A16, A2, A16, ws, None) == E.BITLINEAR_E_ALIGN
    assert q(A16, 64, 512, A16, A16, A16, ws - 1, None) == E.BITLINEAR_E_SIZE
    f = lib.bitlinear_forward_tensor_act
    assert f(A16, A16, 64, 1 << 18, A16, A16, 1, A16, None, None) == E.BITLINEAR_E_SHAPE  # |acc| <= 128 k
    assert f(A16, None, 64, 512, A16, A16, 1, A16, None, None) == E.BITLINEAR_E_NULL
    assert f(A16, A16, 64, 512, A16, A16, (1 << 21) + 1, A16, None, None) == E.BITLINEAR_E_UNSUPPORTED
    nb = blq.bitlinear_packed_bytes(64, 512)
    p = lib.bitlinear_pack_weights_rowscale
    assert p(A16, 64, 512, A16, nb, None, None) == E.BITLINEAR_E_NULL
    assert p(A16, 64, 512, A16, nb, A16 + 1, None) == E.BITLINEAR_E_ALIGN
    assert p(A16, 64, 512, A16, nb - 1, A16, None) == E.BITLINEAR_E_SIZE
    r = lib.bitlinear_forward_rowscale
    assert r(A16, None, 64, 512, A16, A16, 1, A16, None, None) == E.BITLINEAR_E_NULL
    assert r(A16, A16 + 1, 64, 512, A16, A16, 1, A16, None, None) == E.BITLINEAR_E_ALIGN
    assert r(A16, A16, 64, 512, A16, A16, 0, A16, None, None) == E.BITLINEAR_E_SHAPE
    bb = blq.bitlinear_packed_bytes_binary(64, 512)
    assert lib.bitlinear_pack_binary(A16, 64, 512, A16, bb - 1, None) == E.BITLINEAR_E_SIZE
    assert lib.bitlinear_pack_binary(A16, 64, 512, A8, bb, None) == E.BITLINEAR_E_ALIGN
    assert lib.bitlinear_unpack_binary(None, 64, 512, A16, None) == E.BITLINEAR_E_NULL
    b = lib.bitlinear_forward_binary
    assert b(A16, None, 64, 512, A16, A16, 1, A16, None, None) == E.BITLINEAR_E_NULL
    assert b(A16, A16, 64, 512, A16, A16, 1, A16, A2, None) == E.BITLINEAR_E_ALIGN
    fb = lib.bitlinear_quant_forward_binary
    assert fb(A16, A16, 64, 512, A16, 17, A16, None, None, None, None) == E.BITLINEAR_E_UNSUPPORTED
    assert fb(A16, A16, 64, 512, A16, 1, A16, None, A16, None, None) == E.BITLINEAR_E_NULL
