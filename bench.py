#!/usr/bin/env python3
"""Benchmark of the BitLinear forward on one MI355X.

One step = one pass of the per-token path over every BitLinear of the
workload, in layer order: bitlinear_quant_act (bf16 -> int8 codes + a') then
bitlinear_forward (m <= 16) or bitlinear_forward_batched (m > 16) per matrix
(decode: the fused bitlinear_quant_forward instead, at one token and wherever
m * k is small; fused_default).  The
weights are packed once before timing (the one-time preparation step);
packing is timed separately and reported under "pack".  The step is captured
once into a HIP graph and replayed; inputs are resident in HBM and the
weights of consecutive steps are not cache-resident (the stack is larger than
the 256 MB last-level cache, or is replicated until it is).

Default run: the largest configuration, the LLaMA-3-8B-shaped stack at 512
tokens per matrix (7.1 T int8 operations per step), as the headline; then the
same stack's decode at 1, 4 and 8 tokens on the same packed weights, each
with its own rate and roofline under "extra_configs".

Prints ONE JSON line:
  value        algorithmic bytes per step / step time (GB/s) for decode
               workloads, or 2*M*N*K per step / step time (TOPS) for the
               batched workload;
  roofline     the dominant kernel (forward) against HBM or int8 MFMA peak,
               from HIP events around graph replays of its launches;
  cpu_baseline the CPU oracle timed on the host cores on a bounded sample.

Usage: python bench.py [--steps K] [--warmup W] [--workload KEY] [--m M]
Workloads: single2048, b2b_decode, l8b_decode, l8b_prefill (default), l70b_layer.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_I8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA, published
MALL_BYTES = 256 << 20         # last-level (Infinity) cache
COLD_BYTES = 1 << 30           # walk at least this many weight bytes between reuses
# sources of the dominant kernel: the counters in profiles/ are used only while these are unchanged
DECODE_SOURCES = ("gemv.hip", "bitlinear_internal.hpp")
LUT_SOURCES = ("gemv_lut.hip", "bitlinear_internal.hpp")
BATCHED_SOURCES = ("gemm.hip", "bitlinear_internal.hpp")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace runs collapsed, so a
    comment edit leaves the hash (and the counters tied to it) unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif text[i] in "\"'":  # string or character literal, copied whole
            q, j = text[i], i + 1
            while j < n and text[j] != q:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "bitlinear_quant_act_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def forward_bytes(m: int, n: int, k: int) -> int:
    """Algorithmic bytes of one forward call: packed weights, int8 codes, a',
    gamma, fp32 outputs."""
    return (n * k + 3) // 4 + m * k + 4 * m + 4 + 4 * m * n


def quant_bytes(m: int, k: int) -> int:
    return 2 * m * k + m * k + 4 * m


# Variant modes of the pages (each a forward of its own, see include/bitlinear.h):
#   tensor128 -- per-tensor activation scale, Q_b = 128 (bitlinear_quant_act_tensor + bitlinear_forward_tensor_act)
#   rowscale  -- one binary16 scale per output row (bitlinear_forward_rowscale)
#   binary    -- 1-bit sign weights with a per-layer scale (bitlinear_forward_binary; fused at m = 1)
MODES = ("tensor128", "rowscale", "binary")

# The fused entry point (the quantisation, or RMSNorm + quantisation, in the
# GEMV prologue) is chosen per matrix: always for one token; for more tokens
# where m * k is at most FUSED_MAX_MK values.  Every workgroup re-quantises
# all m tokens, so the fusion saves a launch but adds m * k of redundant
# prologue work.  Plain, stack GB/s on one box: the 8B stack at m = 8 with
# its 4096-wide matrices fused (m * k = 32768) 1722 against 1645 unfused; at
# m = 4 with the 14336-wide down projection fused as well (57344) 1849
# against 1858; the 2B stack at m = 8 with its 6912-wide down projection
# fused (55296) 748 against 765.  RMSNorm, us per call (fused / quant +
# forward): 2560 x 6912 at m = 2 6.64 / 6.94; 6144 x 4096 at m = 4 9.41 /
# 7.16; 4096 x 14336 at m = 2 10.44 / 9.38.  The SwiGLU block and the variant
# modes: one token only.
FUSED_MAX_MK = {"plain": 32768, "rmsnorm": 13824}
FUSED_MAX_M = 16  # the decode entry points' token limit


def fused_default(variant: str, m: int, k: int) -> bool:
    return m == 1 or (m <= FUSED_MAX_M and m * k <= FUSED_MAX_MK.get(variant, 0))


def mode_forward_bytes(variant: str, m: int, n: int, k: int, fused: bool = False) -> int:
    """Algorithmic bytes of one forward call of a variant mode."""
    if variant == "binary":
        x_bytes = 2 * m * k if fused else m * k + 4 * m
        return (n * k + 7) // 8 + x_bytes + 4 + 4 * m * n
    if variant == "rowscale":
        return (n * k + 3) // 4 + m * k + 4 * m + 2 * n + 4 * m * n
    return (n * k + 3) // 4 + m * k + 4 + 4 + 4 * m * n  # tensor128: one activation scale


class Mat:
    __slots__ = ("layer", "j", "n", "k", "packed", "gamma", "x", "xq", "amax", "y", "q_or", "g_or", "x_np",
                 "gain", "gain_np", "name", "h", "ws", "s16_or")


def pack_weights(wl, torch, blq, oracle_quota, oracle_mod, variant="plain"):
    """Generate, upload and pack every matrix of the workload once (the
    one-time preparation step, timed on the device); the oracle re-derives the
    codes of the first oracle_quota matrices.  Returns ([Mat], pack info)."""
    dev = torch.device("cuda")
    mats = []
    jobs = list(synth.iter_layer_matrices(wl))
    batch = 8
    t_pack = 0.0
    pack_bytes = 0
    oracle_pack = {"seconds": 0.0, "bytes": 0, "matrices": 0}  # the oracle's weight preparation
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for b0 in range(0, len(jobs), batch):
        chunk = jobs[b0:b0 + batch]
        ws = synth.generate_many([(synth.seed_for(wl, l, j, synth.ROLE_WEIGHT), mt.n, mt.k) for l, j, mt in chunk])
        for (layer, j, mt), w in zip(chunk, ws):
            wd = torch.from_numpy(w).to(dev)
            nbytes = (blq.bitlinear_packed_bytes_binary(mt.n, mt.k) if variant == "binary"
                      else blq.bitlinear_packed_bytes(mt.n, mt.k))
            packed = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            gamma = torch.empty(1, dtype=torch.float32, device=dev)
            work = torch.empty(blq.bitlinear_pack_workspace_bytes(mt.n, mt.k), dtype=torch.uint8, device=dev)
            s_bin = np.float32(np.abs(w).astype(np.float64).mean())  # stand-in for a learned layer scale
            if variant == "rowscale":
                gamma = torch.empty(mt.n, dtype=torch.int16, device=dev)  # binary16 row scales
            elif variant == "binary":
                gamma = torch.from_numpy(np.array([s_bin], np.float32)).to(dev)
            torch.cuda.synchronize()
            e0.record()
            if variant == "rowscale":
                blq.bitlinear_pack_weights_rowscale(wd, packed, gamma)
            elif variant == "binary":
                blq.bitlinear_pack_binary(wd, packed)
            else:
                blq.bitlinear_pack_weights(wd, packed, gamma, work)
            e1.record()
            torch.cuda.synchronize()
            t_pack += e0.elapsed_time(e1) * 1e-3
            pack_bytes += 4 * mt.n * mt.k + nbytes
            mat = Mat()
            mat.layer, mat.j, mat.n, mat.k = layer, j, mt.n, mt.k
            mat.name = mt.name
            mat.packed, mat.gamma = packed, gamma
            mat.s16_or = None
            keep_oracle_codes = len(mats) < oracle_quota
            t_or = time.perf_counter()
            if keep_oracle_codes and variant == "binary":
                mat.g_or = s_bin
                mat.q_or = oracle_mod.binarize(w)
            elif keep_oracle_codes and variant == "rowscale":
                mat.g_or = None
                mat.s16_or = oracle_mod.row_scales(w)
                mat.q_or = oracle_mod.ternarize_rows(w, mat.s16_or)
            elif keep_oracle_codes:
                mat.g_or = oracle_mod.gamma(w)
                mat.q_or = oracle_mod.ternarize(w, mat.g_or)
                oracle_mod.pack_canonical(mat.q_or)  # the oracle's own 2-bit layout, timed with the rest
            else:
                mat.g_or = mat.q_or = None
            if keep_oracle_codes:
                oracle_pack["seconds"] += time.perf_counter() - t_or
                oracle_pack["bytes"] += 4 * mt.n * mt.k
                oracle_pack["matrices"] += 1
            mats.append(mat)
            del wd
        del ws
        log("  packed %d/%d matrices" % (min(b0 + batch, len(jobs)), len(jobs)))
    return mats, {"seconds": t_pack, "bytes": pack_bytes, "oracle": oracle_pack}


def attach_activations(mats, wl, m, torch, blq, variant="plain"):
    """Seeded activations of m tokens for every matrix (the activations of
    workload wl at that token count) and the device buffers of one step; the
    host copy is kept where the oracle holds the matrix's codes."""
    dev = torch.device("cuda")
    for mat in mats:
        x = synth.activations_bf16(synth.seed_for(wl, mat.layer, mat.j, synth.ROLE_ACT, extra=m), m, mat.k,
                                   wl.outlier_frac)
        mat.x_np = x if mat.q_or is not None else None
        mat.x = torch.from_numpy(x.view(np.int16)).to(dev)
        mat.xq = torch.empty((m, mat.k), dtype=torch.int8, device=dev)
        mat.amax = torch.empty(1 if variant == "tensor128" else m, dtype=torch.float32, device=dev)
        mat.ws = (torch.empty(max(4, blq.bitlinear_quant_act_tensor_workspace_bytes(m, mat.k)), dtype=torch.uint8,
                              device=dev) if variant == "tensor128" else None)
        mat.y = torch.empty((m, mat.n), dtype=torch.float32, device=dev)
        mat.gain_np = (synth.norm_gain(synth.seed_for(wl, mat.layer, mat.j, synth.ROLE_GAIN), mat.k)
                       if variant == "rmsnorm" or (variant == "swiglu" and mat.name == "gate_up") else None)
        mat.gain = None if mat.gain_np is None else torch.from_numpy(mat.gain_np).to(dev)
        # SwiGLU variant: the gate+up BitLinear writes h [m][n/2] instead of y
        mat.h = (torch.empty((m, mat.n // 2), dtype=torch.float32, device=dev)
                 if variant == "swiglu" and mat.name == "gate_up" else None)


def replicate(mats, replicas):
    """replicas x [Mat]: copies of the packed weights and of every buffer (the
    oracle's codes stay with the first)."""
    reps = [mats]
    for _ in range(1, replicas):
        cp = []
        for mat in mats:
            c = Mat()
            for s in Mat.__slots__:
                setattr(c, s, getattr(mat, s))
            c.packed = mat.packed.clone()
            c.x, c.xq, c.amax, c.y = mat.x.clone(), mat.xq.new_empty(mat.xq.shape), mat.amax.new_empty(mat.amax.shape), \
                mat.y.new_empty(mat.y.shape)
            c.ws = None if mat.ws is None else mat.ws.new_empty(mat.ws.shape)
            c.h = None if mat.h is None else mat.h.new_empty(mat.h.shape)
            c.q_or = None
            cp.append(c)
        reps.append(cp)
    return reps


def _quant(blq, mat, stream):
    if mat.gain is not None:  # RMSNorm ahead of the quantisation
        blq.bitlinear_rmsnorm_quant_act(mat.x, mat.gain, xq=mat.xq, x_absmax=mat.amax, stream=stream)
    else:
        blq.bitlinear_quant_act(mat.x, mat.xq, mat.amax, stream=stream)


def _fused(blq, mat, stream):
    if mat.gain is not None:
        blq.bitlinear_rmsnorm_quant_forward(mat.packed, mat.gamma, mat.n, mat.k, mat.x, mat.gain, y=mat.y, stream=stream)
    else:
        blq.bitlinear_quant_forward(mat.packed, mat.gamma, mat.n, mat.k, mat.x, y=mat.y, stream=stream)


def _swiglu(blq, mat, stream, fused):
    """gate+up BitLinear (the two halves of one packed matrix) with the SwiGLU
    in its epilogue: h = silu(y_gate) * y_up.  fused: the block input's
    RMSNorm and quantisation run in the same launch."""
    f = mat.n // 2
    half = blq.bitlinear_packed_bytes(f, mat.k)
    if fused:
        blq.bitlinear_rmsnorm_quant_forward_swiglu(mat.packed[:half], mat.gamma, mat.packed[half:], mat.gamma, f,
                                                   mat.k, mat.x, mat.gain, h=mat.h, stream=stream)
    else:
        blq.bitlinear_forward_swiglu(mat.packed[:half], mat.gamma, mat.packed[half:], mat.gamma, f, mat.k, mat.xq,
                                     mat.amax, h=mat.h, stream=stream)


def launch_step_swiglu(blq, mats, m, stream, fused):
    """Feed-forward block as one unit, as the pages' transformer block
    computes it: RMSNorm of the block input, gate+up with the SwiGLU fused,
    and the down projection fed by its own layer's h (quantised from fp32).
    With one token each half is one launch.  The attention projections run as
    in the plain step."""
    fwd = blq.bitlinear_forward if m <= blq.BITLINEAR_FORWARD_MAX_M else blq.bitlinear_forward_batched
    h = None
    for mat in mats:
        if mat.name == "gate_up":
            if not fused:
                _quant(blq, mat, stream)
            _swiglu(blq, mat, stream, fused)
            h = mat.h
        elif mat.name == "down":
            if fused:
                blq.bitlinear_quant_forward_f32(mat.packed, mat.gamma, mat.n, mat.k, h, y=mat.y, stream=stream)
            else:
                blq.bitlinear_quant_act_f32(h, mat.xq, mat.amax, stream=stream)
                fwd(mat.packed, mat.gamma, mat.n, mat.k, mat.xq, mat.amax, y=mat.y, stream=stream)
        elif fused:
            _fused(blq, mat, stream)
        else:
            _quant(blq, mat, stream)
            fwd(mat.packed, mat.gamma, mat.n, mat.k, mat.xq, mat.amax, y=mat.y, stream=stream)


def _forward_fn(blq, m, variant):
    if variant == "lut":
        return blq.bitlinear_forward_lut
    return blq.bitlinear_forward if m <= blq.BITLINEAR_FORWARD_MAX_M else blq.bitlinear_forward_batched


def _mode_quant(blq, mat, stream, variant):
    if variant == "tensor128":
        blq.bitlinear_quant_act_tensor(mat.x, mat.xq, mat.amax, mat.ws, stream=stream)
    else:
        _quant(blq, mat, stream)


def _mode_forward(blq, mat, stream, variant):
    if variant == "tensor128":
        blq.bitlinear_forward_tensor_act(mat.packed, mat.gamma, mat.n, mat.k, mat.xq, mat.amax, y=mat.y, stream=stream)
    elif variant == "rowscale":
        blq.bitlinear_forward_rowscale(mat.packed, mat.gamma, mat.n, mat.k, mat.xq, mat.amax, y=mat.y, stream=stream)
    else:
        blq.bitlinear_forward_binary(mat.packed, mat.gamma, mat.n, mat.k, mat.xq, mat.amax, y=mat.y, stream=stream)


def _mode_fused(blq, mat, stream):  # binary weights, quantisation in the decode prologue
    blq.bitlinear_quant_forward_binary(mat.packed, mat.gamma, mat.n, mat.k, mat.x, y=mat.y, stream=stream)


def launch_step(blq, mats, m, stream, fz, variant="plain"):
    """One pass of the per-token path over every matrix, in layer order;
    fz[j]: matrix j of a layer takes the fused quant + forward call."""
    if variant in MODES:
        for mat in mats:
            if fz[mat.j]:
                _mode_fused(blq, mat, stream)
            else:
                _mode_quant(blq, mat, stream, variant)
                _mode_forward(blq, mat, stream, variant)
        return
    if variant == "swiglu":
        return launch_step_swiglu(blq, mats, m, stream, all(fz))
    fwd = _forward_fn(blq, m, variant)
    for mat in mats:
        if fz[mat.j]:
            _fused(blq, mat, stream)
        else:
            _quant(blq, mat, stream)
            fwd(mat.packed, mat.gamma, mat.n, mat.k, mat.xq, mat.amax, y=mat.y, stream=stream)


def launch_kernel_only(blq, mats, m, stream, which, fz, variant="plain"):
    """Launches of one kernel over every matrix: 'quant' (the quantisation of
    the matrices that take it separately), 'main' (each matrix's forward
    call: the fused quant + forward where fz marks it), 'swiglu' (the gate+up
    launches of the SwiGLU variant)."""
    fwd = _forward_fn(blq, m, variant)
    for mat in mats:
        f = fz[mat.j]
        if which == "swiglu":
            if mat.name == "gate_up":
                _swiglu(blq, mat, stream, f)
        elif which == "quant":
            if f:
                continue
            if variant in MODES:
                _mode_quant(blq, mat, stream, variant)
            else:
                _quant(blq, mat, stream)
        elif variant in MODES:
            if f:
                _mode_fused(blq, mat, stream)
            else:
                _mode_forward(blq, mat, stream, variant)
        elif f:
            _fused(blq, mat, stream)
        else:
            fwd(mat.packed, mat.gamma, mat.n, mat.k, mat.xq, mat.amax, y=mat.y, stream=stream)


def swiglu_bytes(m: int, f: int, k: int) -> int:
    """Algorithmic bytes of one gate+up call with the SwiGLU epilogue: both
    packed halves, int8 codes, a', two gammas, fp32 h [m][f]."""
    return 2 * ((f * k + 3) // 4) + m * k + 4 * m + 8 + 4 * m * f


def fused_bytes(m: int, n: int, k: int) -> int:
    """Algorithmic bytes of one fused quant + forward call: packed weights,
    bf16 activations, gamma, fp32 outputs."""
    return (n * k + 3) // 4 + 2 * m * k + 4 + 4 * m * n


def nonzero_fraction(blq, torch, mats, mode):
    """Fraction of non-zero ternary codes over the given matrices, weighted by
    their sizes, decoded from the packed weights on the device."""
    if mode == "binary":
        return 1.0
    nz = total = 0
    for mt in mats:
        codes = blq.bitlinear_unpack_weights(mt.packed, mt.n, mt.k)
        nz += int(torch.count_nonzero(codes))
        total += mt.n * mt.k
        del codes
    return nz / total


def time_graph(torch, stream, fn, replays):
    """Capture fn(stream) once, replay it `replays` times between two HIP
    events on that stream; returns ms per replay."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(replays):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / replays


def cpu_baseline(oracle_mod, reps_mats, m, wl, budget_s, variant="plain"):
    """The oracle (quant + contraction + dequant; with the SwiGLU variant the
    gate+up -> SwiGLU -> fp32 quant -> down chain) over the workload's
    matrices in layer order, on the host cores, until the sample is done or
    the time budget is spent.  Also checks the GPU outputs of the same
    matrices against the oracle's."""
    mats = [mt for mt in reps_mats if mt.q_or is not None]
    done_bytes = 0
    done_ops = 0
    t_total = 0.0
    worst = 0.0
    chain_ok = True
    nmat = 0
    h_prev = None
    up_flips = None      # SwiGLU chain: tokens whose block-input codes took the other neighbour of a tie
    chain_skipped = 0
    rows_used = m
    phase = {"quant": 0.0, "contract": 0.0, "dequant": 0.0}
    for mat in mats:
        t0 = time.perf_counter()
        tie_count = None
        rows = m if m * mat.n * mat.k <= 2e10 else max(1, int(2e10 // (mat.n * mat.k)))
        if variant == "swiglu" and mat.name == "down":
            if h_prev is None:
                break
            rows = h_prev.shape[0]  # the tokens the gate+up sample produced
            xq, amax = oracle_mod.quant_act_f32(h_prev)
        elif mat.gain_np is not None:
            xq, amax, _, xn = oracle_mod.rmsnorm_quant_act(mat.x_np[:rows], mat.gain_np, with_xnorm=True)
            # the kernels fold r into a': a code may take the other neighbour
            # where x_norm * 127 / a' lies within 2^-19 of a tie (relative)
            t = np.abs(xn.astype(np.float64) * (127.0 / amax.astype(np.float64))[:, None])
            near = np.abs(t - np.floor(t) - 0.5) <= 2.0 ** -19 * t
            tie_count = near.sum(axis=1)
            del xn, t
            if variant == "swiglu" and mat.name == "gate_up":
                # the GPU's codes of the block input (bit-identical in the fused
                # kernel): any difference must be the other neighbour of a tie;
                # such a token's h then differs by that code's whole weight, so
                # the down chain below is compared on the other tokens
                import bitlinear_quant_act_amd as blq_mod
                xq_gpu = blq_mod.bitlinear_rmsnorm_quant_act(mat.x[:rows], mat.gain)[0].cpu().numpy()
                diff = xq_gpu != xq
                chain_ok &= bool(np.all(np.abs(xq_gpu[diff].astype(np.int64) - xq[diff].astype(np.int64)) == 1))
                chain_ok &= bool(np.all(near[diff]))
                up_flips = diff.any(axis=1)
                del xq_gpu, diff
            del near
        elif variant == "tensor128":
            xq, gx = oracle_mod.quant_act_tensor(mat.x_np)  # the scale spans every token
            xq = xq[:rows]
        else:
            xq, amax = oracle_mod.quant_act(mat.x_np[:rows])
        t1 = time.perf_counter()
        acc = (oracle_mod.contract_q128(xq, mat.q_or) if variant == "tensor128"
               else oracle_mod.contract(xq, mat.q_or))
        t2 = time.perf_counter()
        if variant == "tensor128":
            y = oracle_mod.dequant_tensor(acc, mat.g_or, gx)
        elif variant == "rowscale":
            y = oracle_mod.dequant_rows(acc, mat.s16_or, amax)
        elif variant == "swiglu" and mat.name == "gate_up":
            f = mat.n // 2
            y_gate = oracle_mod.dequant(acc[:, :f], mat.g_or, amax)
            y_up = oracle_mod.dequant(acc[:, f:], mat.g_or, amax)
            y = oracle_mod.swiglu(y_gate, y_up)
            h_prev = y
        else:
            y = oracle_mod.dequant(acc, mat.g_or, amax)
        t3 = time.perf_counter()
        phase["quant"] += t1 - t0
        phase["contract"] += t2 - t1
        phase["dequant"] += t3 - t2
        t_total += t3 - t0
        rows_used = rows
        done_bytes += (swiglu_bytes(rows, mat.n // 2, mat.k) if variant == "swiglu" and mat.name == "gate_up"
                       else mode_forward_bytes(variant, rows, mat.n, mat.k) if variant in MODES
                       else forward_bytes(rows, mat.n, mat.k))
        done_ops += 2 * rows * mat.n * mat.k
        out = mat.h if mat.h is not None else mat.y
        yg = out[:rows].cpu().numpy().astype(np.float64)
        yo = y.astype(np.float64)
        if variant == "swiglu" and mat.name == "down":
            # the GPU quantises its own h, equal to the oracle's within 1e-5:
            # a code may sit one step away where the oracle's h * s is within
            # that bound of a rounding tie; allow those codes' weight per token
            t = h_prev.astype(np.float64) * (127.0 / amax.astype(np.float64))[:, None]
            ties = (np.abs(np.abs(t - np.floor(t)) - 0.5) <= 1e-5 * np.abs(t) + 1e-6).sum(axis=1)
            allow = ties[:, None] * float(mat.g_or) * amax.astype(np.float64)[:, None] / 127.0
            keep = np.ones(rows, bool) if up_flips is None else ~up_flips
            chain_skipped += int((~keep).sum())
            chain_ok &= bool(np.all(np.abs(yg[keep] - yo[keep]) <= 1e-5 * np.abs(yo[keep]) + allow[keep] * (1 + 1e-5)
                                    + 1e-30))
        else:
            if tie_count is not None and tie_count.any():
                # tokens with a code at a tie: y within 1e-5 plus those codes' weight;
                # the rest enter the relative error below
                tied = tie_count > 0
                d = tie_count[tied][:, None] * float(mat.g_or) * amax.astype(np.float64)[tied][:, None] / 127.0
                if variant == "swiglu":
                    # h = silu(y_g) * y_u: |dh| <= 1.1 |dy_g| (|y_u| + |dy_u|) + |y_g| |dy_u|
                    yu = np.abs(y_up[tied].astype(np.float64))
                    allow = 1.1 * d * (yu + d) + np.abs(y_gate[tied].astype(np.float64)) * d
                else:
                    allow = d
                chain_ok &= bool(np.all(np.abs(yg[tied] - yo[tied]) <= 1e-5 * np.abs(yo[tied]) + allow * (1 + 1e-5)))
                yg, yo = yg[~tied], yo[~tied]
            nz = yo != 0
            if (yg[~nz] != 0).any():
                worst = float("inf")
            if nz.any():
                worst = max(worst, float((np.abs(yg[nz] - yo[nz]) / np.abs(yo[nz])).max()))
        nmat += 1
        if t_total > budget_s and not (variant == "swiglu" and mat.name == "gate_up"):
            break
    return {"seconds": t_total, "bytes": done_bytes, "ops": done_ops, "matrices": nmat, "rows": rows_used,
            "max_rel_err": worst, "chain_ok": chain_ok, "chain_skipped": chain_skipped, "phases": phase}


def default_fused(wl, m, variant):
    """Per matrix j of a layer: whether the step's default takes the fused
    quant + forward call for it (fused_default); the SwiGLU block and the
    binary mode fuse at one token only, the table-lookup kernel and the
    other modes never."""
    if variant == "lut" or variant in ("tensor128", "rowscale"):
        return (False,) * len(wl.matrices)
    if variant in ("swiglu", "binary"):
        return (m == 1,) * len(wl.matrices)
    return tuple(fused_default(variant, m, mt.k) for mt in wl.matrices)


def choose_fused(blq, wl, m, variant, force_fused=False, force_unfused=False):
    """Per matrix j of a layer: whether the step takes the fused quant +
    forward call for it.  The fused call re-quantises the tokens in every
    workgroup, which pays off for a few tokens on short rows (fused_default);
    the others go through quant + forward.  --fused fuses every matrix the
    call supports, --unfused none; the SwiGLU block and the binary mode are
    fused as a whole or not at all."""
    mode = variant if variant in MODES else None
    nmat = len(wl.matrices)
    if force_unfused or variant == "lut" or mode in ("tensor128", "rowscale"):
        return (False,) * nmat
    if mode == "binary":
        return (m == 1 and all(blq.bitlinear_quant_forward_binary_supported(m, mt.k) for mt in wl.matrices),) * nmat
    if variant == "swiglu":
        return ((m == 1 or force_fused) and
                all(blq.bitlinear_quant_forward_supported(m, mt.k) for mt in wl.matrices),) * nmat
    return tuple((fz or force_fused) and blq.bitlinear_quant_forward_supported(m, mt.k)
                 for fz, mt in zip(default_fused(wl, m, variant), wl.matrices))


def measure(torch, blq, wl, m, reps, variant, fz, steps, warmup, eager, nz_frac=None):
    """Time K steps (after W warmup steps) of the per-token path over the
    packed workload, and the dominant kernel on its own; fz[j]: matrix j of a
    layer takes the fused quant + forward call.  Returns the record without
    the CPU baseline."""
    fused = all(fz)                # every matrix fused (the SwiGLU block and the modes: all or none)
    mixed = any(fz) and not fused  # decode: fused where m * k is small, quant + forward elsewhere
    batched = m > blq.BITLINEAR_FORWARD_MAX_M
    mode = variant if variant in MODES else None
    lut = variant == "lut"
    norm = variant == "rmsnorm"
    sw = variant == "swiglu"
    mats0 = reps[0]

    def call_bytes(mt):
        if mode:
            return mode_forward_bytes(mode, m, mt.n, mt.k)
        if sw and mt.name == "gate_up":
            return swiglu_bytes(m, mt.n // 2, mt.k)
        return forward_bytes(m, mt.n, mt.k)

    step_bytes = sum(call_bytes(mt) for mt in mats0)
    quant_mats = [mt for mt in mats0 if not fz[mt.j]]  # the matrices with a separate quantisation launch
    step_quant_bytes = sum(quant_bytes(m, mt.k) for mt in quant_mats)
    step_ops = sum(2 * m * mt.n * mt.k for mt in mats0)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    # One graph holds one step over every replica in turn (one replay = len(reps)
    # steps), so a small workload is not timed as graph-launch overhead.
    graph = None
    if not eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for mats in reps:
                launch_step(blq, mats, m, torch.cuda.current_stream(), fz, variant)
        torch.cuda.synchronize()
    per_run = len(reps)

    def run():
        if eager:
            with torch.cuda.stream(stream):
                for mats in reps:
                    launch_step(blq, mats, m, stream, fz, variant)
        else:
            graph.replay()

    runs_w = max(1, -(-warmup // per_run))
    runs_t = max(1, -(-steps // per_run))
    for _ in range(runs_w):
        run()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    repeat_ms = []
    for _ in range(5):  # the K steps timed five times; `value` is the first timing
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(runs_t):
            run()
        ev1.record()
        torch.cuda.synchronize()
        repeat_ms.append(ev0.elapsed_time(ev1) / (runs_t * per_run))
    steps_timed = runs_t * per_run
    ms_per_step = repeat_ms[0]
    log("%s m=%d: timed %d steps: %.4f ms/step" % (wl.key, m, steps_timed, ms_per_step))

    # Dominant kernel (each matrix's forward call: the forward, or the fused
    # quant + forward): HIP events on its stream around graph replays that
    # hold only that kernel's launches over every matrix of the workload (no
    # event per launch: an event pair costs more than a small kernel).
    # Average launch duration = elapsed / launches.  The quantisation kernel
    # is timed the same way.
    if quant_mats:  # make sure the codes are current for forward-only replays
        with torch.cuda.stream(stream):
            launch_kernel_only(blq, mats0, m, stream, "quant", fz, variant)
        torch.cuda.synchronize()
    replays = max(2, min(10, steps))
    dom = "swiglu" if sw else "main"
    dom_mats = [mt for mt in mats0 if mt.name == "gate_up"] if sw else mats0

    def all_reps(which):
        return lambda st: [launch_kernel_only(blq, mats, m, st, which, fz, variant) for mats in reps]

    dom_ms = time_graph(torch, stream, all_reps(dom), replays) / len(reps)
    fw_avg_us = dom_ms / len(dom_mats) * 1e3
    q_ms = None
    if quant_mats:
        q_ms = time_graph(torch, stream, all_reps("quant"), replays) / len(reps)

    def main_bytes(mt):  # algorithmic bytes of matrix mt's forward call
        f = fz[mt.j]
        return (fused_bytes if f else forward_bytes)(m, mt.n, mt.k) + (4 * mt.k if norm and f else 0)
    if sw:
        # fused: bf16 input and gains instead of codes and a'
        fw_bytes = sum(swiglu_bytes(m, mt.n // 2, mt.k) + ((m * mt.k + 4 * mt.k - 4 * m) if fused else 0)
                       for mt in dom_mats)
        fw_ops = sum(2 * m * mt.n * mt.k for mt in dom_mats)
    elif mode:
        fw_bytes = sum(mode_forward_bytes(mode, m, mt.n, mt.k, fused) for mt in mats0)
        fw_ops = step_ops
    else:
        fw_bytes = sum(main_bytes(mt) for mt in mats0)
        fw_ops = step_ops
    # The isolated replay includes each launch's dispatch gap, so its time per
    # step can exceed the kernel's share of the real step; the kernel's time
    # per step is then bounded by the step itself, and that bound is used.
    kern_ms_step = dom_ms
    capped = kern_ms_step > ms_per_step
    if capped:
        kern_ms_step = ms_per_step
    if batched:
        value = step_ops / (ms_per_step * 1e-3) / 1e12
        unit = "TOPS"
        achieved = fw_ops / (kern_ms_step * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_I8_PEAK_TOPS, "unit": "TOPS",
                "frac": round(achieved / MFMA_I8_PEAK_TOPS, 4)}
    else:
        value = step_bytes / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        achieved = fw_bytes / (kern_ms_step * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    kern = "gemm_mfma_kernel" if batched else "gemv_lds_kernel"
    roof["kernel"] = (("bitlinear_rmsnorm_quant_forward_swiglu (gemv_lds_kernel, RMSNorm prologue, SwiGLU epilogue)"
                       if fused else "bitlinear_forward_swiglu (%s, SwiGLU epilogue)" % kern)
                      if sw else "bitlinear_forward_batched (gemm_mfma_kernel)" if batched else
                      ("bitlinear_rmsnorm_quant_forward (gemv_lds_kernel, RMSNorm + bf16 prologue)" if norm else
                       "bitlinear_quant_forward (gemv_lds_kernel, bf16 prologue)") if fused else
                      ("%s where m*k <= %d, else bitlinear_forward (gemv_lds_kernel)" % (
                          "bitlinear_rmsnorm_quant_forward" if norm else "bitlinear_quant_forward",
                          FUSED_MAX_MK[variant])) if mixed else
                      "bitlinear_forward_lut (gemv_lut_kernel)" if lut else "bitlinear_forward (gemv_lds_kernel)")
    mode_entry = {"tensor128": "bitlinear_forward_tensor_act", "rowscale": "bitlinear_forward_rowscale",
                  "binary": "bitlinear_quant_forward_binary" if fused else "bitlinear_forward_binary"}
    if mode:
        roof["kernel"] = "%s (%s%s)" % (mode_entry[mode], kern, ", bf16 prologue" if fused else "")
    roof["avg_launch_us"] = round(fw_avg_us, 3)
    roof["launches_per_step"] = len(dom_mats)
    roof["kernel_ms_per_step"] = round(dom_ms, 4)
    if mode:
        roof["per_launch"] = "mean over the workload's matrices of %s" % (
            "2*M*N*K" if batched else
            {"tensor128": "ceil(N*K/4)+M*K+8+4*M*N bytes", "rowscale": "ceil(N*K/4)+M*K+4M+2N+4*M*N bytes",
             "binary": "ceil(N*K/8)+%s+4+4*M*N bytes" % ("2*M*K" if fused else "M*K+4M")}[mode])
    elif sw:
        roof["per_launch"] = "mean over the gate+up matrices of %s" % (
            "2*M*2F*K" if batched else "2*ceil(F*K/4)+2*M*K+4K+8+4*M*F bytes" if fused else
            "2*ceil(F*K/4)+M*K+4M+8+4*M*F bytes")
    else:
        fused_call = "ceil(N*K/4)+2*M*K+4K+4+4*M*N bytes" if norm else "ceil(N*K/4)+2*M*K+4+4*M*N bytes"
        roof["per_launch"] = "mean over the workload's matrices of %s" % (
            "2*M*N*K" if batched else fused_call if fused else
            "%s (fused calls) or ceil(N*K/4)+M*K+4M+4+4*M*N bytes (the others)" % fused_call if mixed else
            "ceil(N*K/4)+M*K+4M+4+4*M*N bytes")
    roof["timing"] = ("HIP events around %d graph replays of the kernel's %d launches per step%s" % (
        replays, len(dom_mats),
        "; their time per step (%.4f ms, dispatch gaps included) exceeds the step's, so the kernel's time per "
        "step is taken as the step's" % dom_ms if capped else ""))
    roof["traffic"] = None
    prof = os.path.join(ROOT, "profiles", "counters_%s_m%d%s.json" % (
        wl.key, m, "" if variant == "plain" else "_" + variant))
    if os.path.exists(prof):
        with open(prof) as f:
            c = json.load(f)
        if c.get("kernel_source_hash") == kernel_source_hash(
                BATCHED_SOURCES if batched else LUT_SOURCES if lut else DECODE_SOURCES):
            roof["traffic"] = c.get("hbm_bytes_per_launch")
    if batched and nz_frac is not None:
        # the method's own work: one add or subtract per non-zero weight and token
        roof["frac_nonzero_adds"] = round(achieved * nz_frac / 2 / MFMA_I8_PEAK_TOPS, 4)

    entry = (((("bitlinear_quant_act_tensor + " if mode == "tensor128" else "" if fused else
                "bitlinear_quant_act + ") + mode_entry[mode]) if mode else
             ("gate+up: bitlinear_rmsnorm_quant_forward_swiglu; down: bitlinear_quant_forward_f32; "
              "others: bitlinear_quant_forward") if sw and fused else
             "gate+up: bitlinear_rmsnorm_quant_act + bitlinear_forward_swiglu; down: "
             "bitlinear_quant_act_f32 + " + ("bitlinear_forward_batched" if batched else
                                             "bitlinear_forward") + "; others as plain"
             if sw else
             ("bitlinear_rmsnorm_quant_forward" if norm else "bitlinear_quant_forward") if fused else
             ("%s where m*k <= %d; elsewhere %s + bitlinear_forward" % (
                 "bitlinear_rmsnorm_quant_forward" if norm else "bitlinear_quant_forward", FUSED_MAX_MK[variant],
                 "bitlinear_rmsnorm_quant_act" if norm else "bitlinear_quant_act")) if mixed else
             ("bitlinear_rmsnorm_quant_act + " if norm else "bitlinear_quant_act + ") +
             ("bitlinear_forward_batched" if batched else
              "bitlinear_forward_lut" if lut else "bitlinear_forward")))
    out = {
        "value": round(value, 2 if batched else 1),
        "unit": unit,
        "steps": steps_timed,
        "warmup": runs_w * per_run,
        "ms_per_step": round(ms_per_step, 4),
        "config": {
            "workload": wl.title,
            "key": wl.key,
            "m": m,
            "layers": wl.layers,
            "matrices_per_step": len(mats0),
            "shapes_kxn": ["%dx%d" % (mt.k, mt.n) for mt in wl.matrices],
            "variant": variant,
            "entry_points": entry,
            "launch": ("hip graph, %d kernels per step" % (sum(
                (1 if fz[mt.j] else 2) + (1 if mode == "tensor128" and
                                       blq.bitlinear_quant_act_tensor_workspace_bytes(m, mt.k) > 4 else 0)
                for mt in mats0)) if not eager else "eager"),
            "cold_cache": "weights %.0f MB per step x %d replica(s)" % (
                sum(mt.packed.numel() for mt in mats0) / 1e6, len(reps)),
            "step_bytes": step_bytes,
            "step_ops": step_ops,
        },
        "pct_of_peak": round(100 * value / (MFMA_I8_PEAK_TOPS if batched else HBM_PEAK_GBS), 2),
        "repeats": {"count": len(repeat_ms), "ms_per_step_min": round(min(repeat_ms), 4),
                    "ms_per_step_median": round(float(np.median(repeat_ms)), 4),
                    "ms_per_step_max": round(max(repeat_ms), 4)},
        "roofline": roof,
    }
    if q_ms is not None:
        out["quant_kernel"] = {"avg_launch_us": round(q_ms / len(quant_mats) * 1e3, 3),
                               "gbs": round(step_quant_bytes / (q_ms * 1e-3) / 1e9, 1)}
    if batched:
        if nz_frac is not None:
            out["nonzero_weight_adds"] = {"fraction_nonzero": round(nz_frac, 4), "tops": round(value * nz_frac / 2, 2),
                                          "definition": "nonzero(q) * M * N * K adds per step / time"}
        # the other roof: algorithmic bytes of the step against the HBM peak
        out["hbm_frac_of_step"] = round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    return out


def cpu_record(oracle_mod, mats0, m, wl, budget, variant, pack):
    cb = cpu_baseline(oracle_mod, mats0, m, wl, budget, variant)
    cores = oracle_mod.num_threads()
    batched = m > 16
    if batched:
        v, u = cb["ops"] / cb["seconds"] / 1e12, "TOPS"
    else:
        v, u = cb["bytes"] / cb["seconds"] / 1e9, "GB/s"
    rec = {
        "value": round(v, 4), "unit": u, "cores": cores, "kind": "oracle",
        "sample": "%d of %d matrices in layer order, %d token(s) each: quant + contraction + dequant "
                  "(%.2f s)" % (cb["matrices"], len(mats0), cb["rows"], cb["seconds"]),
        "cpu": _cpu_model(),
        # the sample's time by oracle step, and the oracle's weight
        # preparation (gamma, ternarisation, canonical 2-bit pack) over the
        # matrices it kept codes for
        "phases_seconds": {kk: round(vv, 4) for kk, vv in cb["phases"].items()},
        "pack": {"seconds": round(pack["oracle"]["seconds"], 4), "matrices": pack["oracle"]["matrices"],
                 "gbs_fp32_read": (round(pack["oracle"]["bytes"] / pack["oracle"]["seconds"] / 1e9, 3)
                                   if pack["oracle"]["seconds"] > 0 else None)},
    }
    parity = {"matrices": cb["matrices"], "max_rel_err_y": cb["max_rel_err"],
              "ok": bool(cb["max_rel_err"] <= 1e-5 and cb["chain_ok"])}
    if variant == "swiglu":
        parity["down_chain_ok"] = cb["chain_ok"]
        # tokens whose block-input codes took the other neighbour of an RMSNorm
        # tie (checked above): their h, and so the down chain, are not compared
        parity["down_chain_tokens_after_a_tie"] = cb["chain_skipped"]
    return rec, parity


# Rough rate of the oracle's contraction on 16 host cores (int8 x ternary
# products summed in int64), used only to size its bounded sample.
ORACLE_MACS_PER_S = 2.0e10

# Workload of the default run: the largest configuration (the LLaMA-3-8B-shaped
# stack at 512 tokens per matrix, 7.1 T int8 operations per step), with the
# same stack's decode at 1, 4 and 8 tokens measured on the same packed weights.
DEFAULT_WORKLOAD = "l8b_prefill"
DEFAULT_EXTRA = "l8b_decode"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, choices=sorted(synth.BY_KEY),
                    help="default: %s, plus %s at each of its token counts on the same weights" % (
                        DEFAULT_WORKLOAD, DEFAULT_EXTRA))
    ap.add_argument("--m", type=int, default=None, help="tokens per matrix (default: workload's first)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="default workload without the decode measurements")
    ap.add_argument("--eager", action="store_true", help="launch the step without a HIP graph")
    ap.add_argument("--fused", action="store_true",
                    help="decode: the fused quant + forward entry point for every matrix (default: per matrix, one token or m*k within FUSED_MAX_MK)")
    ap.add_argument("--unfused", action="store_true",
                    help="decode: bitlinear_quant_act + bitlinear_forward instead of bitlinear_quant_forward")
    ap.add_argument("--fused-max-mk", type=int, default=None, metavar="N",
                    help="decode: fuse the quantisation where m * k <= N (plain and RMSNorm; default FUSED_MAX_MK)")
    ap.add_argument("--variant", default="plain", choices=("plain", "rmsnorm", "swiglu", "lut") + MODES,
                    help="rmsnorm: every BitLinear normalises its input first (per-channel gains); "
                         "swiglu: the feed-forward block as a unit (RMSNorm, gate+up with the SwiGLU fused, "
                         "down fed by h); lut: quant + the table-lookup decode forward; tensor128, rowscale, "
                         "binary: the variant modes (per-tensor Q_b = 128 activations, fp16 row scales, "
                         "1-bit sign weights)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work (bound)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--compare-counters", nargs="+", metavar="ARG",
                    help="CPU only: side-by-side SQ counter table of kernels (see compare_counters())")
    ap.add_argument("--summarize", nargs="+", metavar="ARG",
                    help="CPU only: write profiles/ summaries from rocprofv3 CSVs (see summarize())")
    args = ap.parse_args()
    if args.fused_max_mk is not None:
        for v in FUSED_MAX_MK:
            FUSED_MAX_MK[v] = args.fused_max_mk
    if args.summarize:
        summarize(args.summarize)
        return
    if args.compare_counters:
        compare_counters(args.compare_counters)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only (the path is single-device; "
              "--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bitlinear_quant_act_amd as blq
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    blq.load_library()

    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": nbytes, "launches": 3}))
        return

    default_run = args.workload is None
    wl = synth.BY_KEY[args.workload or DEFAULT_WORKLOAD]
    m = args.m if args.m is not None else wl.ms[0]
    variant = args.variant
    lut = variant == "lut"
    mode = variant if variant in MODES else None
    if lut and (m > blq.BITLINEAR_FORWARD_MAX_M or
                not all(blq.bitlinear_forward_lut_supported(mt.k) for mt in wl.matrices)):
        print("bench.py: --variant lut needs m <= %d and every k within the on-chip table "
              "(k <= 9984)" % blq.BITLINEAR_FORWARD_MAX_M, file=sys.stderr)
        sys.exit(2)
    if variant == "swiglu" and not any(mt.name == "gate_up" for mt in wl.matrices):
        print("bench.py: --variant swiglu needs a workload with a gate+up matrix", file=sys.stderr)
        sys.exit(2)
    fused = choose_fused(blq, wl, m, variant, args.fused, args.unfused)
    want_cpu = not args.no_cpu_baseline
    oracle_mod = None
    if want_cpu or default_run:
        import oracle as oracle_mod  # CPU baseline leg only (and its parity check)
        oracle_mod._load()

    total_packed = synth.packed_weight_bytes_2bit(wl)
    if mode == "binary":
        total_packed //= 2  # one bit per weight
    # a step that walks more than 1.5x the last-level cache evicts its own
    # weights before they come round again; smaller workloads are replicated
    # and walked in turn (the reported steps then round up to whole walks)
    replicas = max(1, -(-COLD_BYTES // total_packed)) if total_packed < 1.5 * MALL_BYTES else 1
    log("workload %s m=%d: %d matrices, %.1f MB packed, %d replica(s)" % (
        wl.key, m, wl.layers * len(wl.matrices), total_packed / 1e6, replicas))
    t0 = time.time()
    # the oracle re-derives ternary codes only for the matrices its bounded
    # sample can cover (about cpu_budget seconds of contraction work)
    oracle_quota = 0
    if want_cpu or default_run:
        macs = 0.0
        for _, _, mt in synth.iter_layer_matrices(wl):
            rows = m if m * mt.n * mt.k <= 2e10 else max(1, int(2e10 // (mt.n * mt.k)))
            macs += rows * mt.n * mt.k
            oracle_quota += 1
            if macs > args.cpu_budget * ORACLE_MACS_PER_S:
                break
    mats, pack = pack_weights(wl, torch, blq, oracle_quota, oracle_mod, variant)
    attach_activations(mats, wl, m, torch, blq, variant)
    reps = replicate(mats, replicas)
    log("setup %.1f s" % (time.time() - t0))

    nz = None
    if m > blq.BITLINEAR_FORWARD_MAX_M:
        # the non-zero fraction, read from the packed codes of the first layer's matrices
        nz = nonzero_fraction(blq, torch, mats[:len(wl.matrices)], mode)
    rec = measure(torch, blq, wl, m, reps, variant, fused, args.steps, args.warmup, args.eager, nz)
    out = {
        "metric": "BitLinear GEMV effective HBM GB/s (% of peak); batched int8 TOPS (% MFMA peak)",
        "value": rec.pop("value"),
        "unit": rec.pop("unit"),
        "n_gpus": 1,
        "steps": rec.pop("steps"),
        "warmup": rec.pop("warmup"),
        "ms_per_step": rec.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded N(0,0.02) latent weights, N(0,1) bf16 activations)",
    }
    out.update(rec)
    out["pack"] = {"seconds": round(pack["seconds"], 4),
                   "gbs": round(pack["bytes"] / pack["seconds"] / 1e9, 1) if pack["seconds"] > 0 else None}
    if want_cpu:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"], out["parity_vs_oracle"] = cpu_record(oracle_mod, reps[0], m, wl, args.cpu_budget,
                                                                  variant, pack)
    else:
        out["cpu_baseline"] = None

    if default_run and not args.no_extra:
        # the same stack's decode (the LLaMA-3-8B-shaped decode workload's
        # activations at 1, 4 and 8 tokens) on the same packed weights
        ewl = synth.BY_KEY[DEFAULT_EXTRA]
        out["extra_configs"] = {}
        for me in ewl.ms:
            for r in reps:
                for mat in r:
                    mat.x = mat.xq = mat.amax = mat.y = mat.h = mat.ws = mat.gain = None
            torch.cuda.empty_cache()
            attach_activations(mats, ewl, me, torch, blq, variant)
            ereps = replicate(mats, replicas)
            efused = choose_fused(blq, ewl, me, variant, args.fused, args.unfused)
            sub = measure(torch, blq, ewl, me, ereps, variant, efused, args.steps, args.warmup, args.eager)
            # parity of the same step's outputs against the oracle, on the matrices whose codes it holds
            sub["parity_vs_oracle"] = cpu_record(oracle_mod, ereps[0], me, ewl, 1.0, variant, pack)[1]
            sub["weights"] = "the packed weights of the headline workload (the same seeded stack)"
            out["extra_configs"]["%s_m%d" % (ewl.key, me)] = sub
    print(json.dumps(out), flush=True)


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _counter_avg_kib(path, kernel_pat):
    """Mean per-dispatch value of the one counter in a rocprofv3 counter CSV,
    over dispatches whose kernel name contains kernel_pat."""
    vals = {}
    for r in _read_csv(path):
        if kernel_pat in r["Kernel_Name"]:
            vals.setdefault(r.get("Dispatch_Id", len(vals)), 0.0)
            vals[r.get("Dispatch_Id", len(vals))] += float(r["Counter_Value"])
    if not vals:
        raise SystemExit("no dispatch of %r in %s" % (kernel_pat, path))
    return sum(vals.values()) / len(vals), len(vals)


def _counters_per_dispatch(paths, kernel_pat):
    """Mean per-dispatch value of every counter in rocprofv3 counter CSVs,
    over dispatches whose kernel name contains kernel_pat."""
    out = {}
    for path in paths:
        per = {}
        for r in _read_csv(path):
            if kernel_pat in r["Kernel_Name"]:
                d = per.setdefault(r["Counter_Name"], {})
                d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        for name, d in per.items():
            out[name] = (sum(d.values()) / len(d), len(d))
    return out


def compare_counters(args):
    """Side-by-side counter table of kernels on one workload (CPU only).

    --compare-counters OUT_MD KEY M LABEL=PATTERN=CSV[,CSV...] ... CMDS CMD...
    Every counter is averaged per dispatch of the kernels whose name holds
    PATTERN.  Derived rows divide by the mean weights per launch (N*K over the
    workload's matrices): wave instructions x 64 lanes per weight."""
    out_md, key, m = args[0], args[1], int(args[2])
    sep = args.index("CMDS") if "CMDS" in args else len(args)
    specs = [a.split("=", 2) for a in args[3:sep]]
    cmds = " ".join(args[sep + 1:])
    wl = synth.BY_KEY[key]
    weights = sum(mt.n * mt.k for mt in wl.matrices) / len(wl.matrices)
    cols = []
    for label, pat, csvs in specs:
        cols.append((label, pat, _counters_per_dispatch(csvs.split(","), pat)))
    names = sorted(set().union(*[c[2].keys() for c in cols]))
    lines = ["# Counter comparison: %s, m=%d" % (wl.title, m), "",
             "Commands (run from the repository root on one MI355X):", "", "```", cmds, "```", "",
             "Mean per dispatch over every launch of the kernel in the run (mean weights per launch: %.0f)." % weights,
             "", "| counter | " + " | ".join("%s (`%s`)" % (c[0], c[1]) for c in cols) + " |",
             "|---|" + "---|" * len(cols)]
    for name in names:
        lines.append("| %s | " % name + " | ".join(
            "%.4g" % c[2][name][0] if name in c[2] else "-" for c in cols) + " |")
    for name in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA", "SQ_INSTS_SALU"):
        if all(name in c[2] for c in cols):
            lines.append("| %s x 64 per weight | " % name + " | ".join(
                "%.3f" % (c[2][name][0] * 64 / weights) for c in cols) + " |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize(args):
    """Write profiles/ summaries from rocprofv3 output (CPU only).

    --summarize KEY[:VARIANT] M STATS_CSV FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV COPY_MIB KERNEL_PAT CMD...
    The algorithmic bytes are those of the dominant kernel bench.py times for
    that workload and variant: each matrix's forward call, fused with the
    quantisation where the step's default fuses it (default_fused)."""
    key, m, stats, fetch, write, cfetch, cwrite, copy_mib, pat = args[:9]
    key, _, variant = key.partition(":")
    variant = variant or "plain"
    cmds = " ".join(args[9:])
    m = int(m)
    copy_kib = float(copy_mib) * 1024.0
    cf, _ = _counter_avg_kib(cfetch, "copy")
    cw, _ = _counter_avg_kib(cwrite, "copy")
    f_fetch = copy_kib / cf
    f_write = copy_kib / cw
    kf, nf = _counter_avg_kib(fetch, pat)
    kw, nw = _counter_avg_kib(write, pat)
    traffic = (kf * f_fetch + kw * f_write) * 1024.0
    rows = [r for r in _read_csv(stats)]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    wl = synth.BY_KEY[key]
    if variant == "swiglu":
        mats = [mt for mt in wl.matrices if mt.name == "gate_up"]
        alg = sum(swiglu_bytes(m, mt.n // 2, mt.k) + ((m * mt.k + 4 * mt.k - 4 * m) if m == 1 else 0)
                  for mt in mats) / len(mats)
    elif variant in MODES:  # binary runs fused at m = 1; the other modes unfused
        alg = sum(mode_forward_bytes(variant, m, mt.n, mt.k, variant == "binary" and m == 1)
                  for mt in wl.matrices) / len(wl.matrices)
    else:
        fz = default_fused(wl, m, variant)
        alg = sum((fused_bytes if f else forward_bytes)(m, mt.n, mt.k) + (4 * mt.k if variant == "rmsnorm" and f else 0)
                  for f, mt in zip(fz, wl.matrices)) / len(wl.matrices)
    suffix = "" if variant == "plain" else "_" + variant
    sources = LUT_SOURCES if variant == "lut" else DECODE_SOURCES if m <= 16 else BATCHED_SOURCES
    out = {
        "workload": key, "m": m, "variant": variant, "kernel_pattern": pat,
        "kernel_source_hash": kernel_source_hash(sources),
        "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw, "dispatches": [nf, nw],
        "copy_calibration": {"copy_mib": float(copy_mib), "fetch_kib": cf, "write_kib": cw,
                             "fetch_factor": f_fetch, "write_factor": f_write},
        "hbm_bytes_per_launch": round(traffic), "algorithmic_bytes_per_launch": round(alg),
        "commands": cmds,
    }
    with open(os.path.join(ROOT, "profiles", "counters_%s_m%d%s.json" % (key, m, suffix)), "w") as f:
        json.dump(out, f, indent=1)
    lines = ["# rocprofv3 kernel statistics: %s, m=%d%s" % (wl.title, m, "" if variant == "plain" else
                                                           ", variant " + variant), "",
             "Commands (run from the repository root on one MI355X):", "", "```", cmds, "```", "",
             "| kernel | calls | avg (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        short = name.split("(")[0].replace("void bitlinear::(anonymous namespace)::", "")
        if "<" in name:
            short = name[:name.index("(", name.index(">"))].replace("void bitlinear::(anonymous namespace)::", "")
        lines.append("| %s | %s | %.3f | %.3f | %.3f | %s%% |" % (short, r["Calls"], float(r["AverageNs"]) / 1e3,
                                                                 float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                                                                 "%.3g" % float(r["Percentage"])))
    dom = [r for r in rows if pat in r["Name"]]
    if dom:
        calls = sum(int(r["Calls"]) for r in dom)
        mean_us = sum(int(r["Calls"]) * float(r["AverageNs"]) for r in dom) / calls / 1e3
        lines += ["", "Every instance of `%s` together: %d calls, %.3f us per launch (call-weighted mean of the "
                  "rows above)." % (pat, calls, mean_us)]
    lines += ["", "HBM traffic of `%s` from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), scaled by a plain "
              "device copy of %s MiB measured the same way (factors %.4f / %.4f): %.0f bytes per launch vs "
              "%.0f algorithmic bytes per launch (mean over the workload's matrices)." % (
                  pat, copy_mib, f_fetch, f_write, traffic, alg)]
    with open(os.path.join(ROOT, "profiles", "%s_m%d%s_kernels.md" % (key, m, suffix)), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(out))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
