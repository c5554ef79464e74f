"""BitNet b1.58 BitLinear forward on AMD MI355X (gfx950).

A thin ctypes binding over ``libbitlinear.so`` (C ABI in include/bitlinear.h).
Each function has the name of the C entry point it calls and only marshals
arguments: torch tensors supply device pointers and the stream; every step of
the computation runs in the library's HIP kernels.  There is no fallback: if
the library is missing or no GPU is present, calls raise.

    packed, gamma = bitlinear_pack_weights(w_fp32_cuda)          # one time
    xq, amax = bitlinear_quant_act(x_bf16_cuda)                  # per call
    y = bitlinear_forward(packed, gamma, n, k, xq, amax)         # m <= 16
    y = bitlinear_forward_batched(packed, gamma, n, k, xq, amax) # any m
"""
from __future__ import annotations

import ctypes as _ct
import os as _os

# torch first: its HIP runtime (same SONAME) must be the one libbitlinear binds
# to, so that device pointers and streams are shared.
import torch as _torch

_PKG = _os.path.dirname(_os.path.abspath(__file__))
LIB_PATH = _os.path.join(_PKG, "lib", "libbitlinear.so")

BITLINEAR_OK = 0
BITLINEAR_E_NULL = -1
BITLINEAR_E_SHAPE = -2
BITLINEAR_E_ALIGN = -3
BITLINEAR_E_UNSUPPORTED = -4
BITLINEAR_E_SIZE = -5
BITLINEAR_E_HIP = -6
BITLINEAR_E_VALUE = -7
BITLINEAR_FORWARD_MAX_M = 16
# nn.RMSNorm's default eps for binary32 inputs (the machine epsilon)
RMS_EPS = 1.1920928955078125e-07

_lib = None
_i64 = _ct.c_int64
_p = _ct.c_void_p


class BitlinearError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, bitlinear_status_string(status), status))


def _mapped_hip_runtimes():
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
        return sorted(p for p in paths if p.startswith("/"))
    except OSError:
        return []


def load_library(path: str = LIB_PATH):
    """Load libbitlinear.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not _os.path.exists(path):
        raise ImportError("libbitlinear.so not built at %s; run bitlinear_quant_act_amd/build.py "
                          "(or __graft_entry__.build())" % path)
    lib = _ct.CDLL(path)
    runtimes = _mapped_hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes mapped in this process: %s" % runtimes)
    lib.bitlinear_abi_version.argtypes = []
    lib.bitlinear_abi_version.restype = _ct.c_int
    lib.bitlinear_status_string.argtypes = [_ct.c_int]
    lib.bitlinear_status_string.restype = _ct.c_char_p
    lib.bitlinear_packed_bytes.argtypes = [_i64, _i64]
    lib.bitlinear_packed_bytes.restype = _ct.c_size_t
    lib.bitlinear_pack_workspace_bytes.argtypes = [_i64, _i64]
    lib.bitlinear_pack_workspace_bytes.restype = _ct.c_size_t
    lib.bitlinear_pack_weights.argtypes = [_p, _i64, _i64, _p, _ct.c_size_t, _p, _p, _ct.c_size_t, _p]
    lib.bitlinear_pack_weights.restype = _ct.c_int
    lib.bitlinear_pack_weights_noalloc.argtypes = [_p, _i64, _i64, _p, _ct.c_size_t, _p, _p]
    lib.bitlinear_pack_weights_noalloc.restype = _ct.c_int
    lib.bitlinear_unpack_weights.argtypes = [_p, _i64, _i64, _p, _p]
    lib.bitlinear_unpack_weights.restype = _ct.c_int
    lib.bitlinear_quant_act.argtypes = [_p, _i64, _i64, _p, _p, _p]
    lib.bitlinear_quant_act.restype = _ct.c_int
    lib.bitlinear_quant_forward.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p]
    lib.bitlinear_quant_forward.restype = _ct.c_int
    lib.bitlinear_quant_forward_supported.argtypes = [_i64, _i64]
    lib.bitlinear_quant_forward_supported.restype = _ct.c_int
    lib.bitlinear_rmsnorm_quant_act.argtypes = [_p, _p, _ct.c_float, _i64, _i64, _p, _p, _p]
    lib.bitlinear_rmsnorm_quant_act.restype = _ct.c_int
    lib.bitlinear_rmsnorm_quant_forward.argtypes = [_p, _p, _i64, _i64, _p, _p, _ct.c_float, _i64, _p, _p, _p, _p, _p]
    lib.bitlinear_rmsnorm_quant_forward.restype = _ct.c_int
    lib.bitlinear_quant_act_f32.argtypes = [_p, _i64, _i64, _p, _p, _p]
    lib.bitlinear_quant_act_f32.restype = _ct.c_int
    lib.bitlinear_rmsnorm_quant_forward_swiglu.argtypes = [_p, _p, _p, _p, _i64, _i64, _p, _p, _ct.c_float, _i64,
                                                           _p, _p, _p, _p, _p]
    lib.bitlinear_rmsnorm_quant_forward_swiglu.restype = _ct.c_int
    lib.bitlinear_quant_forward_f32.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p]
    lib.bitlinear_quant_forward_f32.restype = _ct.c_int
    lib.bitlinear_forward_swiglu.argtypes = [_p, _p, _p, _p, _i64, _i64, _p, _p, _i64, _p, _p, _p]
    lib.bitlinear_forward_swiglu.restype = _ct.c_int
    lib.bitlinear_quant_act_tensor_workspace_bytes.argtypes = [_i64, _i64]
    lib.bitlinear_quant_act_tensor_workspace_bytes.restype = _ct.c_size_t
    lib.bitlinear_quant_act_tensor.argtypes = [_p, _i64, _i64, _p, _p, _p, _ct.c_size_t, _p]
    lib.bitlinear_quant_act_tensor.restype = _ct.c_int
    lib.bitlinear_pack_weights_rowscale.argtypes = [_p, _i64, _i64, _p, _ct.c_size_t, _p, _p]
    lib.bitlinear_pack_weights_rowscale.restype = _ct.c_int
    lib.bitlinear_packed_bytes_binary.argtypes = [_i64, _i64]
    lib.bitlinear_packed_bytes_binary.restype = _ct.c_size_t
    lib.bitlinear_pack_binary.argtypes = [_p, _i64, _i64, _p, _ct.c_size_t, _p]
    lib.bitlinear_pack_binary.restype = _ct.c_int
    lib.bitlinear_unpack_binary.argtypes = [_p, _i64, _i64, _p, _p]
    lib.bitlinear_unpack_binary.restype = _ct.c_int
    lib.bitlinear_quant_forward_binary.argtypes = [_p, _p, _i64, _i64, _p, _i64, _p, _p, _p, _p, _p]
    lib.bitlinear_quant_forward_binary.restype = _ct.c_int
    lib.bitlinear_quant_forward_binary_supported.argtypes = [_i64, _i64]
    lib.bitlinear_quant_forward_binary_supported.restype = _ct.c_int
    lib.bitlinear_forward_lut_supported.argtypes = [_i64]
    lib.bitlinear_forward_lut_supported.restype = _ct.c_int
    for name in ("bitlinear_forward", "bitlinear_forward_batched", "bitlinear_forward_lut",
                 "bitlinear_forward_tensor_act", "bitlinear_forward_rowscale", "bitlinear_forward_binary"):
        fn = getattr(lib, name)
        fn.argtypes = [_p, _p, _i64, _i64, _p, _p, _i64, _p, _p, _p]
        fn.restype = _ct.c_int
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _stream_handle(stream):
    if stream is None:
        return _torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev(t: "_torch.Tensor", name: str, dtypes, numel=None):
    if not isinstance(t, _torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device (cuda) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if numel is not None and t.numel() < numel:
        raise ValueError("%s holds %d elements, needs %d" % (name, t.numel(), numel))
    return t.data_ptr()


def _check(status: int, where: str):
    if status != BITLINEAR_OK:
        raise BitlinearError(status, where)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def bitlinear_abi_version() -> int:
    return int(load_library().bitlinear_abi_version())


def bitlinear_status_string(status: int) -> str:
    return load_library().bitlinear_status_string(int(status)).decode()


def bitlinear_packed_bytes(n: int, k: int) -> int:
    return int(load_library().bitlinear_packed_bytes(n, k))


def bitlinear_pack_workspace_bytes(n: int, k: int) -> int:
    return int(load_library().bitlinear_pack_workspace_bytes(n, k))


def bitlinear_pack_weights(w, packed=None, gamma=None, workspace=None, stream=None):
    """w: fp32 [n][k] device tensor -> (packed uint8 tensor, gamma fp32 [1])."""
    lib = load_library()
    if w.dim() != 2:
        raise ValueError("w must be [n][k]")
    n, k = w.shape
    nbytes = bitlinear_packed_bytes(n, k)
    wsbytes = bitlinear_pack_workspace_bytes(n, k)
    if nbytes == 0:
        raise BitlinearError(BITLINEAR_E_SHAPE, "bitlinear_pack_weights")
    if packed is None:
        packed = _torch.empty(nbytes, dtype=_torch.uint8, device=w.device)
    if gamma is None:
        gamma = _torch.empty(1, dtype=_torch.float32, device=w.device)
    if workspace is None:
        workspace = _torch.empty(wsbytes, dtype=_torch.uint8, device=w.device)
    rc = lib.bitlinear_pack_weights(
        _dev(w, "w", (_torch.float32,)), n, k,
        _dev(packed, "packed", (_torch.uint8,)), packed.numel() * packed.element_size(),
        _dev(gamma, "gamma", (_torch.float32,), 1),
        _dev(workspace, "workspace", (_torch.uint8, _torch.float64, _torch.int64)),
        workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _check(rc, "bitlinear_pack_weights")
    return packed, gamma


BITLINEAR_PACK_NOALLOC_SCRATCH_BYTES = 8192


def bitlinear_pack_weights_noalloc(w, packed, gamma, stream=None):
    """bitlinear_pack_weights with the library's static device scratch in
    place of a workspace: the caller passes the outputs (packed uint8 with at
    least bitlinear_packed_bytes(n, k) bytes, gamma fp32 [1]); nothing is
    allocated."""
    lib = load_library()
    if w.dim() != 2:
        raise ValueError("w must be [n][k]")
    n, k = w.shape
    rc = lib.bitlinear_pack_weights_noalloc(
        _dev(w, "w", (_torch.float32,)), n, k,
        _dev(packed, "packed", (_torch.uint8,)), packed.numel() * packed.element_size(),
        _dev(gamma, "gamma", (_torch.float32,), 1), _stream_handle(stream))
    _check(rc, "bitlinear_pack_weights_noalloc")
    return packed, gamma


def bitlinear_unpack_weights(packed, n: int, k: int, codes=None, stream=None):
    """Decode packed weights -> int8 [n][k] codes in {-1, 0, 1}."""
    lib = load_library()
    if codes is None:
        codes = _torch.empty((n, k), dtype=_torch.int8, device=packed.device)
    if packed.numel() * packed.element_size() < bitlinear_packed_bytes(n, k):
        raise BitlinearError(BITLINEAR_E_SIZE, "bitlinear_unpack_weights")
    rc = lib.bitlinear_unpack_weights(_dev(packed, "packed", (_torch.uint8,)), n, k,
                                      _dev(codes, "codes", (_torch.int8,), n * k), _stream_handle(stream))
    _check(rc, "bitlinear_unpack_weights")
    return codes


def bitlinear_quant_act(x, xq=None, x_absmax=None, stream=None):
    """x: bf16 [m][k] (or int16/uint16 bit patterns) -> (xq int8 [m][k], a' fp32 [m])."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be [m][k]")
    m, k = x.shape
    if xq is None:
        xq = _torch.empty((m, k), dtype=_torch.int8, device=x.device)
    if x_absmax is None:
        x_absmax = _torch.empty(m, dtype=_torch.float32, device=x.device)
    rc = lib.bitlinear_quant_act(_dev(x, "x", (_torch.bfloat16, _torch.int16, _torch.uint16)), m, k,
                                 _dev(xq, "xq", (_torch.int8,), m * k),
                                 _dev(x_absmax, "x_absmax", (_torch.float32,), m), _stream_handle(stream))
    _check(rc, "bitlinear_quant_act")
    return xq, x_absmax


def bitlinear_rmsnorm_quant_act(x, gain=None, eps: float = RMS_EPS, xq=None, x_absmax=None, stream=None):
    """RMSNorm (optional gain fp32 [k]) then per-token quantisation of
    x bf16 [m][k] -> (xq int8 [m][k], a' fp32 [m]); a' carries 1/rms."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be [m][k]")
    m, k = x.shape
    if xq is None:
        xq = _torch.empty((m, k), dtype=_torch.int8, device=x.device)
    if x_absmax is None:
        x_absmax = _torch.empty(m, dtype=_torch.float32, device=x.device)
    rc = lib.bitlinear_rmsnorm_quant_act(
        _dev(x, "x", (_torch.bfloat16, _torch.int16, _torch.uint16)),
        None if gain is None else _dev(gain, "gain", (_torch.float32,), k), float(eps), m, k,
        _dev(xq, "xq", (_torch.int8,), m * k), _dev(x_absmax, "x_absmax", (_torch.float32,), m),
        _stream_handle(stream))
    _check(rc, "bitlinear_rmsnorm_quant_act")
    return xq, x_absmax


def bitlinear_quant_act_f32(x, xq=None, x_absmax=None, stream=None):
    """x: fp32 [m][k] -> (xq int8 [m][k], a' fp32 [m])."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be [m][k]")
    m, k = x.shape
    if xq is None:
        xq = _torch.empty((m, k), dtype=_torch.int8, device=x.device)
    if x_absmax is None:
        x_absmax = _torch.empty(m, dtype=_torch.float32, device=x.device)
    rc = lib.bitlinear_quant_act_f32(_dev(x, "x", (_torch.float32,)), m, k,
                                     _dev(xq, "xq", (_torch.int8,), m * k),
                                     _dev(x_absmax, "x_absmax", (_torch.float32,), m), _stream_handle(stream))
    _check(rc, "bitlinear_quant_act_f32")
    return xq, x_absmax


def _forward(fname, packed, gamma, n, k, xq, x_absmax, y, acc, stream):
    lib = load_library()
    m = xq.shape[0]
    if xq.dim() != 2 or xq.shape[1] != k:
        raise ValueError("xq must be [m][k]")
    if packed.numel() * packed.element_size() < bitlinear_packed_bytes(n, k):
        raise BitlinearError(BITLINEAR_E_SIZE, fname)
    if y is None:
        y = _torch.empty((m, n), dtype=_torch.float32, device=xq.device)
    rc = getattr(lib, fname)(
        _dev(packed, "packed", (_torch.uint8,)), _dev(gamma, "gamma", (_torch.float32,), 1), n, k,
        _dev(xq, "xq", (_torch.int8,)), _dev(x_absmax, "x_absmax", (_torch.float32,), m), m,
        _dev(y, "y", (_torch.float32,), m * n),
        None if acc is None else _dev(acc, "acc", (_torch.int32,), m * n), _stream_handle(stream))
    _check(rc, fname)
    return y


def bitlinear_forward(packed, gamma, n: int, k: int, xq, x_absmax, y=None, acc=None, stream=None):
    """Decode path (1 <= m <= 16): y fp32 [m][n]; optional exact int32 acc [m][n]."""
    return _forward("bitlinear_forward", packed, gamma, n, k, xq, x_absmax, y, acc, stream)


def bitlinear_forward_swiglu(packed_gate, gamma_gate, packed_up, gamma_up, f: int, k: int, xq, x_absmax,
                             h=None, acc=None, stream=None):
    """Gate and up projections with h = silu(y_gate) * y_up fused into the
    epilogue: h fp32 [m][f]; optional exact int32 acc [m][2f] (gate, up)."""
    lib = load_library()
    m = xq.shape[0]
    if xq.dim() != 2 or xq.shape[1] != k:
        raise ValueError("xq must be [m][k]")
    nb = bitlinear_packed_bytes(f, k)
    for name, pk in (("packed_gate", packed_gate), ("packed_up", packed_up)):
        if pk.numel() * pk.element_size() < nb:
            raise BitlinearError(BITLINEAR_E_SIZE, "bitlinear_forward_swiglu (%s)" % name)
    if h is None:
        h = _torch.empty((m, f), dtype=_torch.float32, device=xq.device)
    rc = lib.bitlinear_forward_swiglu(
        _dev(packed_gate, "packed_gate", (_torch.uint8,)), _dev(gamma_gate, "gamma_gate", (_torch.float32,), 1),
        _dev(packed_up, "packed_up", (_torch.uint8,)), _dev(gamma_up, "gamma_up", (_torch.float32,), 1), f, k,
        _dev(xq, "xq", (_torch.int8,)), _dev(x_absmax, "x_absmax", (_torch.float32,), m), m,
        _dev(h, "h", (_torch.float32,), m * f),
        None if acc is None else _dev(acc, "acc", (_torch.int32,), 2 * m * f), _stream_handle(stream))
    _check(rc, "bitlinear_forward_swiglu")
    return h


# ---------------------------------------------------------------------------
# variant modes
# ---------------------------------------------------------------------------

def _variant_forward(fname, packed, packed_bytes, wscale, wscale_dtype, wscale_n, n, k, xq, ascale, ascale_n, y, acc,
                     stream):
    lib = load_library()
    if xq.dim() != 2 or xq.shape[1] != k:
        raise ValueError("xq must be [m][k]")
    m = xq.shape[0]
    if packed.numel() * packed.element_size() < packed_bytes:
        raise BitlinearError(BITLINEAR_E_SIZE, fname)
    if y is None:
        y = _torch.empty((m, n), dtype=_torch.float32, device=xq.device)
    rc = getattr(lib, fname)(
        _dev(packed, "packed", (_torch.uint8,)), _dev(wscale, "weight scale", wscale_dtype, wscale_n), n, k,
        _dev(xq, "xq", (_torch.int8,), m * k), _dev(ascale, "activation scale", (_torch.float32,), ascale_n), m,
        _dev(y, "y", (_torch.float32,), m * n),
        None if acc is None else _dev(acc, "acc", (_torch.int32,), m * n), _stream_handle(stream))
    _check(rc, fname)
    return y


def bitlinear_quant_act_tensor_workspace_bytes(m: int, k: int) -> int:
    return int(load_library().bitlinear_quant_act_tensor_workspace_bytes(m, k))


def bitlinear_quant_act_tensor(x, xq=None, x_scale=None, workspace=None, stream=None):
    """Per-tensor Q_b = 128 quantisation: x bf16 [m][k] -> (xq int8 [m][k] in
    [-128, 127], g fp32 [1] = max |x| over the tensor)."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be [m][k]")
    m, k = x.shape
    if xq is None:
        xq = _torch.empty((m, k), dtype=_torch.int8, device=x.device)
    if x_scale is None:
        x_scale = _torch.empty(1, dtype=_torch.float32, device=x.device)
    if workspace is None:
        workspace = _torch.empty(max(bitlinear_quant_act_tensor_workspace_bytes(m, k), 4), dtype=_torch.uint8,
                                 device=x.device)
    rc = lib.bitlinear_quant_act_tensor(_dev(x, "x", (_torch.bfloat16, _torch.int16, _torch.uint16)), m, k,
                                        _dev(xq, "xq", (_torch.int8,), m * k),
                                        _dev(x_scale, "x_scale", (_torch.float32,), 1),
                                        _dev(workspace, "workspace", (_torch.uint8, _torch.int32)),
                                        workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _check(rc, "bitlinear_quant_act_tensor")
    return xq, x_scale


def bitlinear_forward_tensor_act(packed, gamma, n: int, k: int, xq, x_scale, y=None, acc=None, stream=None):
    """Forward of per-tensor codes: y = acc * gamma * g / 128 (any m)."""
    return _variant_forward("bitlinear_forward_tensor_act", packed, bitlinear_packed_bytes(n, k), gamma,
                            (_torch.float32,), 1, n, k, xq, x_scale, 1, y, acc, stream)


def bitlinear_pack_weights_rowscale(w, packed=None, scales=None, stream=None):
    """w fp32 [n][k] -> (packed uint8, binary16 scales [n] as int16 bit patterns)."""
    lib = load_library()
    if w.dim() != 2:
        raise ValueError("w must be [n][k]")
    n, k = w.shape
    nbytes = bitlinear_packed_bytes(n, k)
    if nbytes == 0:
        raise BitlinearError(BITLINEAR_E_SHAPE, "bitlinear_pack_weights_rowscale")
    if packed is None:
        packed = _torch.empty(nbytes, dtype=_torch.uint8, device=w.device)
    if scales is None:
        scales = _torch.empty(n, dtype=_torch.int16, device=w.device)
    rc = lib.bitlinear_pack_weights_rowscale(
        _dev(w, "w", (_torch.float32,)), n, k, _dev(packed, "packed", (_torch.uint8,)),
        packed.numel() * packed.element_size(),
        _dev(scales, "scales", (_torch.int16, _torch.uint16, _torch.float16), n), _stream_handle(stream))
    _check(rc, "bitlinear_pack_weights_rowscale")
    return packed, scales


def bitlinear_forward_rowscale(packed, scales, n: int, k: int, xq, x_absmax, y=None, acc=None, stream=None):
    """Forward with one binary16 scale per output row: y = acc * s_row * a' / 127 (any m)."""
    m = xq.shape[0]
    return _variant_forward("bitlinear_forward_rowscale", packed, bitlinear_packed_bytes(n, k), scales,
                            (_torch.int16, _torch.uint16, _torch.float16), n, n, k, xq, x_absmax, m, y, acc, stream)


def bitlinear_packed_bytes_binary(n: int, k: int) -> int:
    return int(load_library().bitlinear_packed_bytes_binary(n, k))


def bitlinear_pack_binary(w, packed=None, stream=None):
    """w fp32 [n][k] -> packed sign bits (uint8 tensor)."""
    lib = load_library()
    if w.dim() != 2:
        raise ValueError("w must be [n][k]")
    n, k = w.shape
    nbytes = bitlinear_packed_bytes_binary(n, k)
    if nbytes == 0:
        raise BitlinearError(BITLINEAR_E_SHAPE, "bitlinear_pack_binary")
    if packed is None:
        packed = _torch.empty(nbytes, dtype=_torch.uint8, device=w.device)
    rc = lib.bitlinear_pack_binary(_dev(w, "w", (_torch.float32,)), n, k, _dev(packed, "packed", (_torch.uint8,)),
                                   packed.numel() * packed.element_size(), _stream_handle(stream))
    _check(rc, "bitlinear_pack_binary")
    return packed


def bitlinear_unpack_binary(packed, n: int, k: int, codes=None, stream=None):
    lib = load_library()
    if codes is None:
        codes = _torch.empty((n, k), dtype=_torch.int8, device=packed.device)
    if packed.numel() * packed.element_size() < bitlinear_packed_bytes_binary(n, k):
        raise BitlinearError(BITLINEAR_E_SIZE, "bitlinear_unpack_binary")
    rc = lib.bitlinear_unpack_binary(_dev(packed, "packed", (_torch.uint8,)), n, k,
                                     _dev(codes, "codes", (_torch.int8,), n * k), _stream_handle(stream))
    _check(rc, "bitlinear_unpack_binary")
    return codes


def bitlinear_forward_binary(packed, scale, n: int, k: int, xq, x_absmax, y=None, acc=None, stream=None):
    """Binary-weight forward: y = acc * s * a' / 127 (any m); scale fp32 [1]."""
    m = xq.shape[0]
    return _variant_forward("bitlinear_forward_binary", packed, bitlinear_packed_bytes_binary(n, k), scale,
                            (_torch.float32,), 1, n, k, xq, x_absmax, m, y, acc, stream)


def bitlinear_quant_forward_binary_supported(m: int, k: int) -> bool:
    return bool(load_library().bitlinear_quant_forward_binary_supported(m, k))


def bitlinear_quant_forward_binary(packed, scale, n: int, k: int, x, y=None, acc=None, xq=None, x_absmax=None,
                                   stream=None):
    """Fused quantisation + binary-weight decode forward (as bitlinear_quant_forward)."""
    lib = load_library()
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be [m][k]")
    m = x.shape[0]
    if packed.numel() * packed.element_size() < bitlinear_packed_bytes_binary(n, k):
        raise BitlinearError(BITLINEAR_E_SIZE, "bitlinear_quant_forward_binary")
    if y is None:
        y = _torch.empty((m, n), dtype=_torch.float32, device=x.device)
    rc = lib.bitlinear_quant_forward_binary(
        _dev(packed, "packed", (_torch.uint8,)), _dev(scale, "scale", (_torch.float32,), 1), n, k,
        _dev(x, "x", (_torch.bfloat16, _torch.int16, _torch.uint16)), m,
        _dev(y, "y", (_torch.float32,), m * n),
        None if acc is None else _dev(acc, "acc", (_torch.int32,), m * n),
        None if xq is None else _dev(xq, "xq", (_torch.int8,), m * k),
        None if x_absmax is None else _dev(x_absmax, "x_absmax", (_torch.float32,), m),
        _stream_handle(stream))
    _check(rc, "bitlinear_quant_forward_binary")
    return y


def bitlinear_forward_lut_supported(k: int) -> bool:
    return bool(load_library().bitlinear_forward_lut_supported(k))


def bitlinear_forward_lut(packed, gamma, n: int, k: int, xq, x_absmax, y=None, acc=None, stream=None):
    """Table-lookup decode forward; same arguments and result as bitlinear_forward."""
    return _forward("bitlinear_forward_lut", packed, gamma, n, k, xq, x_absmax, y, acc, stream)


def bitlinear_forward_batched(packed, gamma, n: int, k: int, xq, x_absmax, y=None, acc=None, stream=None):
    """Batched path (any m): y fp32 [m][n]; optional exact int32 acc [m][n]."""
    return _forward("bitlinear_forward_batched", packed, gamma, n, k, xq, x_absmax, y, acc, stream)


def bitlinear_quant_forward_supported(m: int, k: int) -> bool:
    return bool(load_library().bitlinear_quant_forward_supported(m, k))


def bitlinear_quant_forward(packed, gamma, n: int, k: int, x, y=None, acc=None, xq=None, x_absmax=None,
                            stream=None):
    """Fused activation quantisation + decode forward (1 <= m <= 16, m*k codes
    within the on-chip budget).  x: bf16 [m][k] (or int16 bit patterns).
    Optional outputs: exact int32 acc [m][n]; the codes xq [m][k] and a' [m]
    (pass both or neither).  Returns y fp32 [m][n]."""
    lib = load_library()
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be [m][k]")
    m = x.shape[0]
    if packed.numel() * packed.element_size() < bitlinear_packed_bytes(n, k):
        raise BitlinearError(BITLINEAR_E_SIZE, "bitlinear_quant_forward")
    if y is None:
        y = _torch.empty((m, n), dtype=_torch.float32, device=x.device)
    rc = lib.bitlinear_quant_forward(
        _dev(packed, "packed", (_torch.uint8,)), _dev(gamma, "gamma", (_torch.float32,), 1), n, k,
        _dev(x, "x", (_torch.bfloat16, _torch.int16, _torch.uint16)), m,
        _dev(y, "y", (_torch.float32,), m * n),
        None if acc is None else _dev(acc, "acc", (_torch.int32,), m * n),
        None if xq is None else _dev(xq, "xq", (_torch.int8,), m * k),
        None if x_absmax is None else _dev(x_absmax, "x_absmax", (_torch.float32,), m),
        _stream_handle(stream))
    _check(rc, "bitlinear_quant_forward")
    return y


def bitlinear_rmsnorm_quant_forward(packed, gamma, n: int, k: int, x, gain=None, eps: float = RMS_EPS, y=None,
                                    acc=None, xq=None, x_absmax=None, stream=None):
    """Fused RMSNorm + activation quantisation + decode forward (the support
    rule of bitlinear_quant_forward).  Returns y fp32 [m][n]."""
    lib = load_library()
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be [m][k]")
    m = x.shape[0]
    if packed.numel() * packed.element_size() < bitlinear_packed_bytes(n, k):
        raise BitlinearError(BITLINEAR_E_SIZE, "bitlinear_rmsnorm_quant_forward")
    if y is None:
        y = _torch.empty((m, n), dtype=_torch.float32, device=x.device)
    rc = lib.bitlinear_rmsnorm_quant_forward(
        _dev(packed, "packed", (_torch.uint8,)), _dev(gamma, "gamma", (_torch.float32,), 1), n, k,
        _dev(x, "x", (_torch.bfloat16, _torch.int16, _torch.uint16)),
        None if gain is None else _dev(gain, "gain", (_torch.float32,), k), float(eps), m,
        _dev(y, "y", (_torch.float32,), m * n),
        None if acc is None else _dev(acc, "acc", (_torch.int32,), m * n),
        None if xq is None else _dev(xq, "xq", (_torch.int8,), m * k),
        None if x_absmax is None else _dev(x_absmax, "x_absmax", (_torch.float32,), m),
        _stream_handle(stream))
    _check(rc, "bitlinear_rmsnorm_quant_forward")
    return y


def bitlinear_rmsnorm_quant_forward_swiglu(packed_gate, gamma_gate, packed_up, gamma_up, f: int, k: int, x,
                                           gain=None, eps: float = RMS_EPS, h=None, acc=None, xq=None,
                                           x_absmax=None, stream=None):
    """RMSNorm + quantisation + gate/up projections + SwiGLU in one decode
    launch (m <= 16 within the on-chip budget).  Returns h fp32 [m][f]."""
    lib = load_library()
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be [m][k]")
    m = x.shape[0]
    nb = bitlinear_packed_bytes(f, k)
    for name, pk in (("packed_gate", packed_gate), ("packed_up", packed_up)):
        if pk.numel() * pk.element_size() < nb:
            raise BitlinearError(BITLINEAR_E_SIZE, "bitlinear_rmsnorm_quant_forward_swiglu (%s)" % name)
    if h is None:
        h = _torch.empty((m, f), dtype=_torch.float32, device=x.device)
    rc = lib.bitlinear_rmsnorm_quant_forward_swiglu(
        _dev(packed_gate, "packed_gate", (_torch.uint8,)), _dev(gamma_gate, "gamma_gate", (_torch.float32,), 1),
        _dev(packed_up, "packed_up", (_torch.uint8,)), _dev(gamma_up, "gamma_up", (_torch.float32,), 1), f, k,
        _dev(x, "x", (_torch.bfloat16, _torch.int16, _torch.uint16)),
        None if gain is None else _dev(gain, "gain", (_torch.float32,), k), float(eps), m,
        _dev(h, "h", (_torch.float32,), m * f),
        None if acc is None else _dev(acc, "acc", (_torch.int32,), 2 * m * f),
        None if xq is None else _dev(xq, "xq", (_torch.int8,), m * k),
        None if x_absmax is None else _dev(x_absmax, "x_absmax", (_torch.float32,), m),
        _stream_handle(stream))
    _check(rc, "bitlinear_rmsnorm_quant_forward_swiglu")
    return h


def bitlinear_quant_forward_f32(packed, gamma, n: int, k: int, x, y=None, acc=None, xq=None, x_absmax=None,
                                stream=None):
    """Quantisation of fp32 activations [m][k] fused into the decode forward.
    Returns y fp32 [m][n]."""
    lib = load_library()
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError("x must be [m][k]")
    m = x.shape[0]
    if packed.numel() * packed.element_size() < bitlinear_packed_bytes(n, k):
        raise BitlinearError(BITLINEAR_E_SIZE, "bitlinear_quant_forward_f32")
    if y is None:
        y = _torch.empty((m, n), dtype=_torch.float32, device=x.device)
    rc = lib.bitlinear_quant_forward_f32(
        _dev(packed, "packed", (_torch.uint8,)), _dev(gamma, "gamma", (_torch.float32,), 1), n, k,
        _dev(x, "x", (_torch.float32,)), m, _dev(y, "y", (_torch.float32,), m * n),
        None if acc is None else _dev(acc, "acc", (_torch.int32,), m * n),
        None if xq is None else _dev(xq, "xq", (_torch.int8,), m * k),
        None if x_absmax is None else _dev(x_absmax, "x_absmax", (_torch.float32,), m),
        _stream_handle(stream))
    _check(rc, "bitlinear_quant_forward_f32")
    return y


def bitlinear(x, packed, gamma, n: int, k: int, stream=None):
    """Convenience: run the fastest entry point that fits x (bf16 [m][k])."""
    m = x.shape[0]
    if m == 1 and bitlinear_quant_forward_supported(m, k):
        return bitlinear_quant_forward(packed, gamma, n, k, x, stream=stream)
    xq, amax = bitlinear_quant_act(x, stream=stream)
    if x.shape[0] <= BITLINEAR_FORWARD_MAX_M:
        return bitlinear_forward(packed, gamma, n, k, xq, amax, stream=stream)
    return bitlinear_forward_batched(packed, gamma, n, k, xq, amax, stream=stream)
