"""CPU oracle of the BitNet b1.58 BitLinear forward -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the product library never does.  It is a
thin numpy front-end over ``bitlinear_oracle.c`` (plain C, built by
``oracle/build.py``) and shares no code with the HIP library.

Every function follows a passage of the source pages (cited by title and
section in the C file):
  gamma / ternarize   -- "BitNet b1.58 in Production", The Mathematical
                         Mechanism, item 1 (absmean scale, RoundClip);
  pack / unpack       -- "BitNet 1-bit LLM Inference Framework", How the LUT
                         Kernel Works (codes 00 = 0, 01 = +1, 10 = -1);
  quant_act           -- "BitNet b1.58 in Production", item 2 (per-token
                         absmax, Q_b = 127);
  contract            -- item 3 (integer dot product with weights in
                         {-1, 0, 1});
  dequant             -- item 4 (gamma * max|x| / Q_b);
  rmsnorm_quant_act   -- the same page's "bit_linear.py" listing: nn.RMSNorm,
                         then activation_quant of the normalised input;
  swiglu              -- "BitNet 1-bit LLM Inference Framework", "A Deep Look
                         at the BitNet Architecture" (the block's ffn).
Variant modes:
  quant_act_tensor, dequant_tensor, contract_q128
                      -- "BitNet 1-bit LLM Inference Framework", the BitLinear
                         class under "The Core Structure of BitNet b1.58"
                         (one activation scale per tensor, Q_b = 128);
  row_scales, ternarize_rows, dequant_rows, f32_to_f16_bits
                      -- "BitNet-2B-4T: Inside the 2B-Parameter, 4T-Token 1-Bit
                         LLM", "Weight Representation: Ternary + Scale, Not
                         Pure Binary" (one FP16 scale per output channel);
  binarize            -- "BitNet's 1-Bit Transformer: Architecture Breakdown",
                         "Binary Weight Matrices with Learnable Scaling".
All of them are pinned by tests in tests/test_oracle_*.py.
"""
from __future__ import annotations

import ctypes as _ct
import os as _os

import numpy as np

_HERE = _os.path.dirname(_os.path.abspath(__file__))
# BITLINEAR_ORACLE_LIB lets the mutation test load a deliberately broken copy.
_LIB_PATH = _os.environ.get("BITLINEAR_ORACLE_LIB") or _os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = _ct.c_int64
_p = _ct.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _os.path.exists(_LIB_PATH):
        from . import build as _build  # compile on first use (CPU-only, gcc)
        _build.build()
    lib = _ct.CDLL(_LIB_PATH)
    lib.oracle_abs_sum.argtypes = [_p, _i64, _i64, _p]
    lib.oracle_abs_sum.restype = _ct.c_double
    lib.oracle_gamma_from_sum.argtypes = [_ct.c_double, _i64, _i64]
    lib.oracle_gamma_from_sum.restype = _ct.c_float
    lib.oracle_ternarize.argtypes = [_p, _i64, _i64, _ct.c_float, _p]
    lib.oracle_ternarize.restype = None
    lib.oracle_pack_canonical.argtypes = [_p, _i64, _i64, _p]
    lib.oracle_pack_canonical.restype = None
    lib.oracle_unpack_canonical.argtypes = [_p, _i64, _i64, _p]
    lib.oracle_unpack_canonical.restype = _ct.c_int
    lib.oracle_quant_act.argtypes = [_p, _i64, _i64, _p, _p]
    lib.oracle_quant_act.restype = None
    lib.oracle_contract.argtypes = [_p, _p, _i64, _i64, _i64, _p]
    lib.oracle_contract.restype = _ct.c_int
    lib.oracle_contract_pairs.argtypes = [_p, _p, _i64, _p, _p, _i64, _p]
    lib.oracle_contract_pairs.restype = _ct.c_int
    lib.oracle_dequant.argtypes = [_p, _i64, _i64, _ct.c_float, _p, _p]
    lib.oracle_dequant.restype = None
    lib.oracle_quant_act_f32.argtypes = [_p, _i64, _i64, _p, _p]
    lib.oracle_quant_act_f32.restype = None
    lib.oracle_rmsnorm_quant_act.argtypes = [_p, _p, _ct.c_float, _i64, _i64, _p, _p, _p, _p]
    lib.oracle_rmsnorm_quant_act.restype = None
    lib.oracle_swiglu.argtypes = [_p, _p, _i64, _p]
    lib.oracle_swiglu.restype = None
    lib.oracle_quant_act_tensor.argtypes = [_p, _i64, _i64, _p, _p]
    lib.oracle_quant_act_tensor.restype = None
    lib.oracle_dequant_tensor.argtypes = [_p, _i64, _i64, _ct.c_float, _ct.c_float, _p]
    lib.oracle_dequant_tensor.restype = None
    lib.oracle_contract_q128.argtypes = [_p, _p, _i64, _i64, _i64, _p]
    lib.oracle_contract_q128.restype = _ct.c_int
    lib.oracle_f32_to_f16.argtypes = [_ct.c_float]
    lib.oracle_f32_to_f16.restype = _ct.c_uint16
    lib.oracle_f16_to_f32.argtypes = [_ct.c_uint16]
    lib.oracle_f16_to_f32.restype = _ct.c_float
    lib.oracle_row_scales.argtypes = [_p, _i64, _i64, _p]
    lib.oracle_row_scales.restype = None
    lib.oracle_ternarize_rows.argtypes = [_p, _i64, _i64, _p, _p]
    lib.oracle_ternarize_rows.restype = None
    lib.oracle_dequant_rows.argtypes = [_p, _i64, _i64, _p, _p, _p]
    lib.oracle_dequant_rows.restype = None
    lib.oracle_binarize.argtypes = [_p, _i64, _i64, _p]
    lib.oracle_binarize.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = _ct.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


def abs_sum(w: np.ndarray) -> float:
    """binary64 sum of |W| (rows left to right, then rows in order)."""
    w = _c(w, np.float32)
    n, k = w.shape
    rows = np.empty(n, dtype=np.float64)
    return float(_load().oracle_abs_sum(_ptr(w), n, k, _ptr(rows)))


def gamma(w: np.ndarray) -> np.float32:
    """Absmean scale: mean |W| in binary64, rounded once to binary32."""
    w = _c(w, np.float32)
    n, k = w.shape
    return np.float32(_load().oracle_gamma_from_sum(abs_sum(w), n, k))


def gamma_from_sum(s: float, n: int, k: int) -> np.float32:
    return np.float32(_load().oracle_gamma_from_sum(float(s), n, k))


def ternarize(w: np.ndarray, g) -> np.ndarray:
    """int8 [n][k] = Clip(Round(W / (gamma + 1e-5)), -1, 1)."""
    w = _c(w, np.float32)
    n, k = w.shape
    q = np.empty((n, k), dtype=np.int8)
    _load().oracle_ternarize(_ptr(w), n, k, float(np.float32(g)), _ptr(q))
    return q


def pack_canonical(q: np.ndarray) -> np.ndarray:
    """uint8 [n][ceil(k/4)]: 4 codes per byte, least significant field first."""
    q = _c(q, np.int8)
    n, k = q.shape
    out = np.empty((n, (k + 3) // 4), dtype=np.uint8)
    _load().oracle_pack_canonical(_ptr(q), n, k, _ptr(out))
    return out


def unpack_canonical(b: np.ndarray, n: int, k: int) -> np.ndarray:
    b = _c(b, np.uint8)
    if b.size != n * ((k + 3) // 4):
        raise OracleError("packed buffer has the wrong size")
    q = np.empty((n, k), dtype=np.int8)
    rc = _load().oracle_unpack_canonical(_ptr(b), n, k, _ptr(q))
    if rc == -1:
        raise OracleError("invalid 2-bit code 11 in packed weights")
    if rc == -2:
        raise OracleError("non-zero padding field in packed weights")
    return q


def quant_act(x_bits: np.ndarray):
    """(xq int8 [m][k], a' fp32 [m]) from bf16 bit patterns [m][k]."""
    x = _c(x_bits, np.uint16)
    m, k = x.shape
    xq = np.empty((m, k), dtype=np.int8)
    amax = np.empty(m, dtype=np.float32)
    _load().oracle_quant_act(_ptr(x), m, k, _ptr(xq), _ptr(amax))
    return xq, amax


def quant_act_f32(x: np.ndarray):
    """(xq int8 [m][k], a' fp32 [m]) from fp32 activations [m][k]."""
    x = _c(x, np.float32)
    m, k = x.shape
    xq = np.empty((m, k), dtype=np.int8)
    amax = np.empty(m, dtype=np.float32)
    _load().oracle_quant_act_f32(_ptr(x), m, k, _ptr(xq), _ptr(amax))
    return xq, amax


# torch's nn.RMSNorm default eps for binary32 inputs (the machine epsilon)
RMS_EPS = float(np.finfo(np.float32).eps)


def rmsnorm_quant_act(x_bits: np.ndarray, w=None, eps: float = RMS_EPS, with_xnorm: bool = False):
    """RMSNorm (optional gain w [k]) then per-token quantization of the
    normalised input, in the listing's order.
    Returns (xq int8 [m][k], a' fp32 [m], r fp32 [m]), and x_norm fp32 [m][k]
    as a fourth element when with_xnorm."""
    x = _c(x_bits, np.uint16)
    m, k = x.shape
    wp = None
    if w is not None:
        w = _c(w, np.float32)
        if w.shape != (k,):
            raise OracleError("gain must have k entries")
        wp = _ptr(w)
    xq = np.empty((m, k), dtype=np.int8)
    amax = np.empty(m, dtype=np.float32)
    rr = np.empty(m, dtype=np.float32)
    xn = np.empty((m, k), dtype=np.float32) if with_xnorm else None
    _load().oracle_rmsnorm_quant_act(_ptr(x), wp, float(np.float32(eps)), m, k, _ptr(xq), _ptr(amax), _ptr(rr),
                                     _ptr(xn) if with_xnorm else None)
    return (xq, amax, rr, xn) if with_xnorm else (xq, amax, rr)


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = silu(g) * u elementwise (binary64, rounded once to binary32)."""
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    if g.shape != u.shape:
        raise OracleError("gate and up shapes differ")
    h = np.empty(g.shape, dtype=np.float32)
    _load().oracle_swiglu(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def contract(xq: np.ndarray, q: np.ndarray) -> np.ndarray:
    """int32 [m][n] = sum_k xq[m][k] * q[n][k] by add / skip / subtract."""
    xq = _c(xq, np.int8)
    q = _c(q, np.int8)
    m, k = xq.shape
    n, k2 = q.shape
    if k != k2:
        raise OracleError("inner sizes differ")
    acc = np.empty((m, n), dtype=np.int32)
    rc = _load().oracle_contract(_ptr(xq), _ptr(q), m, n, k, _ptr(acc))
    if rc == -1:
        raise OracleError("accumulator bound |acc| <= 127*K violated")
    if rc == -2:
        raise OracleError("weight code outside {-1, 0, 1}")
    return acc


def contract_pairs(xq: np.ndarray, q_rows: np.ndarray, rows: np.ndarray,
                   qrows: np.ndarray) -> np.ndarray:
    """acc for the listed pairs: sum_k xq[rows[p]][k] * q_rows[qrows[p]][k]."""
    xq = _c(xq, np.int8)
    q_rows = _c(q_rows, np.int8)
    rows = _c(rows, np.int64)
    qrows = _c(qrows, np.int64)
    k = xq.shape[1]
    if q_rows.shape[1] != k or rows.shape != qrows.shape:
        raise OracleError("shape mismatch")
    acc = np.empty(rows.shape[0], dtype=np.int32)
    rc = _load().oracle_contract_pairs(_ptr(xq), _ptr(q_rows), k, _ptr(rows), _ptr(qrows),
                                       rows.shape[0], _ptr(acc))
    if rc != 0:
        raise OracleError("contraction check failed (%d)" % rc)
    return acc


def dequant(acc: np.ndarray, g, amax: np.ndarray) -> np.ndarray:
    """fp32 [m][n] = acc * gamma * a' / 127 (binary64, rounded once)."""
    acc = _c(acc, np.int32)
    amax = _c(amax, np.float32)
    m, n = acc.shape
    y = np.empty((m, n), dtype=np.float32)
    _load().oracle_dequant(_ptr(acc), m, n, float(np.float32(g)), _ptr(amax), _ptr(y))
    return y


def forward(x_bits: np.ndarray, w: np.ndarray, g=None) -> dict:
    """Whole path on the CPU: gamma, ternary codes, activation codes, int32
    accumulators and fp32 outputs.  ``g`` overrides gamma (e.g. to ternarize
    with another computation's gamma when the two differ in the last bit)."""
    gm = gamma(w) if g is None else np.float32(g)
    q = ternarize(w, gm)
    xq, amax = quant_act(x_bits)
    acc = contract(xq, q)
    y = dequant(acc, gm, amax)
    return {"gamma": gm, "q": q, "xq": xq, "amax": amax, "acc": acc, "y": y}


# ---------------------------------------------------------------------------
# variant modes
# ---------------------------------------------------------------------------

def quant_act_tensor(x_bits: np.ndarray):
    """V1: (xq int8 [m][k] in [-128, 127], g fp32) with one scale for the
    whole tensor: code = round(clamp((x * 128) / (g + 1e-8), -128, 127)),
    g = max |x| over every element."""
    x = _c(x_bits, np.uint16)
    m, k = x.shape
    xq = np.empty((m, k), dtype=np.int8)
    g = np.empty(1, dtype=np.float32)
    _load().oracle_quant_act_tensor(_ptr(x), m, k, _ptr(xq), _ptr(g))
    return xq, g[0]


def dequant_tensor(acc: np.ndarray, g_w, g_x) -> np.ndarray:
    """V1: fp32 [m][n] = acc * gamma * g / 2^7 (binary64, rounded once)."""
    acc = _c(acc, np.int32)
    m, n = acc.shape
    y = np.empty((m, n), dtype=np.float32)
    _load().oracle_dequant_tensor(_ptr(acc), m, n, float(np.float32(g_w)), float(np.float32(g_x)), _ptr(y))
    return y


def contract_q128(xq: np.ndarray, q: np.ndarray) -> np.ndarray:
    """contract() for codes in [-128, 127] (bound 128 * K)."""
    xq = _c(xq, np.int8)
    q = _c(q, np.int8)
    m, k = xq.shape
    n, k2 = q.shape
    if k != k2:
        raise OracleError("inner sizes differ")
    acc = np.empty((m, n), dtype=np.int32)
    rc = _load().oracle_contract_q128(_ptr(xq), _ptr(q), m, n, k, _ptr(acc))
    if rc == -1:
        raise OracleError("accumulator bound |acc| <= 128*K violated")
    if rc == -2:
        raise OracleError("weight code outside {-1, 0, 1}")
    return acc


def f32_to_f16_bits(v) -> np.ndarray:
    """binary16 bits (round to nearest even) of binary32 values, element-wise."""
    a = np.asarray(v, dtype=np.float32)
    lib = _load()
    return np.array([lib.oracle_f32_to_f16(float(t)) for t in a.ravel()], dtype=np.uint16).reshape(a.shape)


def f16_bits_to_f32(b) -> np.ndarray:
    a = np.asarray(b, dtype=np.uint16)
    lib = _load()
    return np.array([lib.oracle_f16_to_f32(int(t)) for t in a.ravel()], dtype=np.float32).reshape(a.shape)


def row_scales(w: np.ndarray) -> np.ndarray:
    """V2: binary16 bits [n] of each row's absmean (binary64 mean, rounded
    to binary32, then to binary16)."""
    w = _c(w, np.float32)
    n, k = w.shape
    s16 = np.empty(n, dtype=np.uint16)
    _load().oracle_row_scales(_ptr(w), n, k, _ptr(s16))
    return s16


def ternarize_rows(w: np.ndarray, s16: np.ndarray) -> np.ndarray:
    """V2: int8 [n][k] = Clip(Round(W / (s_row + 1e-5)), -1, 1)."""
    w = _c(w, np.float32)
    s16 = _c(s16, np.uint16)
    n, k = w.shape
    if s16.shape != (n,):
        raise OracleError("one scale per row")
    q = np.empty((n, k), dtype=np.int8)
    _load().oracle_ternarize_rows(_ptr(w), n, k, _ptr(s16), _ptr(q))
    return q


def dequant_rows(acc: np.ndarray, s16: np.ndarray, amax: np.ndarray) -> np.ndarray:
    """V2: fp32 [m][n] = acc * s_n * a'_m / 127 (binary64, rounded once)."""
    acc = _c(acc, np.int32)
    s16 = _c(s16, np.uint16)
    amax = _c(amax, np.float32)
    m, n = acc.shape
    y = np.empty((m, n), dtype=np.float32)
    _load().oracle_dequant_rows(_ptr(acc), m, n, _ptr(s16), _ptr(amax), _ptr(y))
    return y


def binarize(w: np.ndarray) -> np.ndarray:
    """V3: int8 [n][k] = -1 where W < 0, else +1."""
    w = _c(w, np.float32)
    n, k = w.shape
    b = np.empty((n, k), dtype=np.int8)
    _load().oracle_binarize(_ptr(w), n, k, _ptr(b))
    return b


def forward_tensor_act(x_bits: np.ndarray, w: np.ndarray) -> dict:
    """V1 path: main-path gamma and codes, per-tensor Q_b = 128 activations."""
    gm = gamma(w)
    q = ternarize(w, gm)
    xq, gx = quant_act_tensor(x_bits)
    acc = contract_q128(xq, q)
    return {"gamma": gm, "q": q, "xq": xq, "gx": gx, "acc": acc, "y": dequant_tensor(acc, gm, gx)}


def forward_rowscale(x_bits: np.ndarray, w: np.ndarray) -> dict:
    """V2 path: per-row FP16 scales and codes, per-token activations."""
    s16 = row_scales(w)
    q = ternarize_rows(w, s16)
    xq, amax = quant_act(x_bits)
    acc = contract(xq, q)
    return {"s16": s16, "q": q, "xq": xq, "amax": amax, "acc": acc, "y": dequant_rows(acc, s16, amax)}


def forward_binary(x_bits: np.ndarray, w: np.ndarray, s) -> dict:
    """V3 path: sign(W) (zero -> +1) with the given per-layer scale s,
    per-token activations."""
    b = binarize(w)
    xq, amax = quant_act(x_bits)
    acc = contract(xq, b)
    return {"b": b, "xq": xq, "amax": amax, "acc": acc, "y": dequant(acc, np.float32(s), amax)}


def num_threads() -> int:
    return int(_load().oracle_num_threads())
