"""ctypes binding of libbitnet_mi355x.so: argument marshalling only.

Function names match the C ABI in include/bitnet_mi355x.h.  torch supplies the
device memory (``data_ptr()``) and the stream (``torch.cuda.current_stream()``);
every step of the layer runs in the HIP kernels behind these calls.  If the
library is missing, the first call raises: there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbitnet_mi355x.so")

BITNET_OK = 0
BITNET_F32 = 0
BITNET_BF16 = 1
STATUS = {0: "BITNET_OK", 1: "BITNET_ERR_NULL", 2: "BITNET_ERR_SHAPE", 3: "BITNET_ERR_DTYPE",
          4: "BITNET_ERR_ALIGN", 5: "BITNET_ERR_WORKSPACE", 6: "BITNET_ERR_HIP"}

# exported symbol -> (restype, argtypes); kept in the order of the public header
_P, _I64, _I, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "bitnet_status_string": (ctypes.c_char_p, [_I]),
    "bitnet_packed_bytes": (_SZ, [_I64, _I64]),
    "bitnet_quantize_weights_workspace_bytes": (_SZ, [_I64, _I64]),
    "bitnet_quantize_weights": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "bitnet_quantize_weights_noalloc": (_I, [_P, _I, _I64, _I64, _P, _P, _P]),
    "bitnet_quantize_acts": (_I, [_P, _I, _I64, _I64, _P, _P, _P]),
    "bitnet_ternary_linear": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P, _P]),
    "bitnet_quant_linear": (_I, [_P, _P, _P, _I, _I64, _I64, _I64, _P, _P, _P, _I, _P, _P]),
}



class BitnetMatrix(ctypes.Structure):
    """struct bitnet_matrix of the public header."""
    _fields_ = [("w_packed", ctypes.c_void_p), ("w_scale", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("y", ctypes.c_void_p), ("acc_out", ctypes.c_void_p)]


SIGNATURES["bitnet_ternary_linear_multi"] = (_I, [ctypes.POINTER(BitnetMatrix), _I, _P, _P, _I64,
                                                  _I64, _I, _P])
SIGNATURES["bitnet_quant_linear_multi"] = (_I, [ctypes.POINTER(BitnetMatrix), _I, _P, _I, _I64,
                                                _I64, _P, _P, _I, _P])


class BitnetActPrologue(ctypes.Structure):
    """struct bitnet_act_prologue of the public header."""
    _fields_ = [("up", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float)]


SIGNATURES["bitnet_quantize_acts_ex"] = (_I, [_P, _I, ctypes.POINTER(BitnetActPrologue), _I64,
                                              _I64, _P, _P, _P])
SIGNATURES["bitnet_quant_linear_ex"] = (_I, [ctypes.POINTER(BitnetMatrix), _I, _P, _I,
                                             ctypes.POINTER(BitnetActPrologue), _I64, _I64, _P,
                                             _P, _I, _P])

SIGNATURES["bitnet_t1_packed_bytes"] = (_SZ, [_I64, _I64])
SIGNATURES["bitnet_quantize_weights_t1"] = (_I, [_P, _I, _I64, _I64, _P, _P, _P, _SZ, _P])
SIGNATURES["bitnet_repack_t1"] = (_I, [_P, _I64, _I64, _P, _P])
SIGNATURES["bitnet_ternary_linear_t1"] = (_I, [ctypes.POINTER(BitnetMatrix), _I, _P, _P, _I64,
                                               _I64, _I, _P])
SIGNATURES["bitnet_quant_linear_t1"] = (_I, [ctypes.POINTER(BitnetMatrix), _I, _P, _I,
                                             ctypes.POINTER(BitnetActPrologue), _I64, _I64, _P,
                                             _P, _I, _P])

SIGNATURES["bitnet_prefill_layout_bytes"] = (_SZ, [_I64, _I64])
SIGNATURES["bitnet_repack_prefill"] = (_I, [_P, _I64, _I64, _P, _P])
SIGNATURES["bitnet_ternary_linear_prefill"] = (_I, [ctypes.POINTER(BitnetMatrix), _I, _P, _P,
                                                    _I64, _I64, _I, _P])

SIGNATURES["bitnet_lut_workspace_bytes"] = (_SZ, [_I64, _I64])
SIGNATURES["bitnet_ternary_linear_lut"] = (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I, _P, _P,
                                                _SZ, _P])

_lib = None


class BitnetError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")


def lib() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run python -m ternary_weight_linear_bit_amd.build)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _lib = handle
    return _lib


def _check(fn, status):
    if status != BITNET_OK:
        raise BitnetError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(dt):
    import torch
    if dt == torch.float32:
        return BITNET_F32
    if dt == torch.bfloat16:
        return BITNET_BF16
    raise TypeError(f"unsupported dtype {dt}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous CUDA tensors")


def _expect(t, shape, dtypes, name):
    """Raise ValueError unless tensor t (if given) has this shape and one of these
    dtypes: the kernels write through raw pointers, so a wrong-sized or
    wrong-typed output would be written out of bounds."""
    import torch
    if t is None:
        return
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if tuple(t.shape) != tuple(shape) or t.dtype not in dtypes:
        raise ValueError(f"{name}: expected shape {tuple(shape)} and dtype "
                         f"{' or '.join(str(d) for d in dtypes)}, got {tuple(t.shape)} {t.dtype}")
    _need_cuda(t)


def _floats():
    import torch
    return (torch.float32, torch.bfloat16)


def _check_act_operands(x, x_q, x_scale, up=None, norm_weight=None):
    """x [M, K] fp32/bf16 (2-D), x_q int8 [M, K], x_scale fp32 [M], the prologue's
    up (like x) and norm weight (fp32 [K])."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    m, k = x.shape
    _expect(x, (m, k), _floats(), "x")
    _expect(x_q, (m, k), torch.int8, "x_q")
    _expect(x_scale, (m,), torch.float32, "x_scale")
    _expect(up, (m, k), x.dtype, "up")
    _expect(norm_weight, (k,), torch.float32, "norm_weight")


def _check_scale(w_scale):
    import torch
    if w_scale is not None and (w_scale.numel() < 1 or w_scale.dtype != torch.float32):
        raise ValueError("w_scale must hold at least one float32")
    _need_cuda(w_scale)


def bitnet_packed_bytes(n: int, k: int) -> int:
    return lib().bitnet_packed_bytes(n, k)


def bitnet_quantize_weights(w, packed=None, scale=None, workspace=None, stream=None):
    """w: [N, K] fp32/bf16 -> (packed uint8 [N, K/4], gamma* fp32 [1])."""
    import torch
    _need_cuda(w)
    n, k = w.shape
    dev = w.device
    if packed is None:
        packed = torch.empty((n, k // 4), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=dev)
    ws_bytes = lib().bitnet_quantize_weights_workspace_bytes(n, k)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _expect(w, (n, k), _floats(), "w")
    _expect(packed, (n, k // 4), torch.uint8, "packed")
    _check_scale(scale)
    _need_cuda(workspace)
    _check("bitnet_quantize_weights", lib().bitnet_quantize_weights(
        _ptr(w), _dtype_code(w.dtype), n, k, _ptr(packed), _ptr(scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return packed, scale


def bitnet_quantize_weights_noalloc(w, packed, scale, stream=None):
    """bitnet_quantize_weights with the library's own per-device workspace: the
    caller supplies packed uint8 [N, K/4] and scale fp32 [1]; nothing is allocated."""
    import torch
    _need_cuda(w)
    n, k = w.shape
    _expect(w, (n, k), _floats(), "w")
    _expect(packed, (n, k // 4), torch.uint8, "packed")
    _check_scale(scale)
    _check("bitnet_quantize_weights_noalloc", lib().bitnet_quantize_weights_noalloc(
        _ptr(w), _dtype_code(w.dtype), n, k, _ptr(packed), _ptr(scale), _stream(stream)))
    return packed, scale


def _prologue(x, up, norm_weight, eps):
    """struct bitnet_act_prologue for (up, norm_weight, eps), or None for none."""
    if up is None and norm_weight is None:
        return None
    _need_cuda(up, norm_weight)
    if up is not None and (up.shape != x.shape or up.dtype != x.dtype):
        raise ValueError("up must match x in shape and dtype")
    return ctypes.byref(BitnetActPrologue(0 if up is None else up.data_ptr(),
                                          0 if norm_weight is None else norm_weight.data_ptr(),
                                          float(eps)))


def bitnet_quantize_acts(x, x_q=None, x_scale=None, stream=None, up=None, norm_weight=None,
                         eps=1e-5):
    """x: [M, K] fp32/bf16 -> (x_q int8 [M, K], d fp32 [M]).  With ``up`` x is the
    gate projection (squared-ReLU gating); with ``norm_weight`` the input is
    RMS-normalised (bitnet_quantize_acts_ex)."""
    import torch
    _need_cuda(x)
    m, k = x.shape
    if x_q is None:
        x_q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty(m, dtype=torch.float32, device=x.device)
    _check_act_operands(x, x_q, x_scale, up, norm_weight)
    pro = _prologue(x, up, norm_weight, eps)
    if pro is None:
        _check("bitnet_quantize_acts", lib().bitnet_quantize_acts(
            _ptr(x), _dtype_code(x.dtype), m, k, _ptr(x_q), _ptr(x_scale), _stream(stream)))
    else:
        _check("bitnet_quantize_acts_ex", lib().bitnet_quantize_acts_ex(
            _ptr(x), _dtype_code(x.dtype), pro, m, k, _ptr(x_q), _ptr(x_scale),
            _stream(stream)))
    return x_q, x_scale


def bitnet_ternary_linear(w_packed, w_scale, x_q, x_scale, y=None, y_dtype=None,
                          acc_out=None, stream=None):
    """Packed W [N, K/4] x int8 X [M, K] -> y [M, N] (fp32 or bf16)."""
    import torch
    _need_cuda(w_packed, w_scale, x_q, x_scale, acc_out)
    m, k = x_q.shape
    n = w_packed.shape[0]
    if w_packed.shape[1] * 4 != k:
        raise ValueError("w_packed and x_q disagree on K")
    if y is None:
        y = torch.empty((m, n), dtype=y_dtype or torch.float32, device=x_q.device)
    _expect(w_packed, (n, k // 4), torch.uint8, "w_packed")
    _check_scale(w_scale)
    _expect(x_q, (m, k), torch.int8, "x_q")
    _expect(x_scale, (m,), torch.float32, "x_scale")
    _expect(y, (m, n), _floats(), "y")
    _expect(acc_out, (m, n), torch.int32, "acc_out")
    _check("bitnet_ternary_linear", lib().bitnet_ternary_linear(
        _ptr(w_packed), _ptr(w_scale), _ptr(x_q), _ptr(x_scale), m, n, k, _ptr(y),
        _dtype_code(y.dtype), _ptr(acc_out), _stream(stream)))
    return y


def bitnet_quant_linear(w_packed, w_scale, x, x_q=None, x_scale=None, y=None, y_dtype=None,
                        acc_out=None, stream=None):
    """Act-quant fused into the layer: returns (y, x_q, x_scale)."""
    import torch
    _need_cuda(w_packed, w_scale, x, acc_out)
    m, k = x.shape
    n = w_packed.shape[0]
    if w_packed.shape[1] * 4 != k:
        raise ValueError("w_packed and x disagree on K")
    if x_q is None:
        x_q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty(m, dtype=torch.float32, device=x.device)
    if y is None:
        y = torch.empty((m, n), dtype=y_dtype or torch.float32, device=x.device)
    _check_act_operands(x, x_q, x_scale)
    _expect(w_packed, (n, k // 4), torch.uint8, "w_packed")
    _check_scale(w_scale)
    _expect(y, (m, n), _floats(), "y")
    _expect(acc_out, (m, n), torch.int32, "acc_out")
    _check("bitnet_quant_linear", lib().bitnet_quant_linear(
        _ptr(w_packed), _ptr(w_scale), _ptr(x), _dtype_code(x.dtype), m, n, k, _ptr(x_q),
        _ptr(x_scale), _ptr(y), _dtype_code(y.dtype), _ptr(acc_out), _stream(stream)))
    return y, x_q, x_scale


def _matrices(mats, m, k, dtype, device, row_bytes=None):
    """[(w_packed, w_scale[, y[, acc_out]])] -> ctypes array and the y tensors.
    Every y must be [M, N] of one shared dtype (fp32 or bf16), every acc_out
    int32 [M, N], every w_packed uint8 [N, row_bytes] (K/4 for the 2-bit layout)."""
    import torch
    if not mats:
        raise ValueError("at least one matrix")
    rb = k // 4 if row_bytes is None else row_bytes
    arr = (BitnetMatrix * len(mats))()
    ys = []
    for i, t in enumerate(mats):
        w_packed, w_scale = t[0], t[1]
        n = w_packed.shape[0]
        y = t[2] if len(t) > 2 and t[2] is not None else torch.empty(
            (m, n), dtype=dtype if not ys else ys[0].dtype, device=device)
        acc = t[3] if len(t) > 3 else None
        _expect(w_packed, (n, rb), torch.uint8, f"w_packed[{i}]")
        _check_scale(w_scale)
        _expect(y, (m, n), ys[0].dtype if ys else _floats(), f"y[{i}]")
        _expect(acc, (m, n), torch.int32, f"acc_out[{i}]")
        arr[i] = BitnetMatrix(w_packed.data_ptr(), w_scale.data_ptr(), n,
                              y.data_ptr(), 0 if acc is None else acc.data_ptr())
        ys.append(y)
    return arr, ys


def bitnet_ternary_linear_multi(mats, x_q, x_scale, y_dtype=None, stream=None):
    """Several (w_packed, w_scale[, y[, acc_out]]) sharing x_q -> list of y."""
    import torch
    _need_cuda(x_q, x_scale)
    m, k = x_q.shape
    _expect(x_q, (m, k), torch.int8, "x_q")
    _expect(x_scale, (m,), torch.float32, "x_scale")
    arr, ys = _matrices(mats, m, k, y_dtype or torch.float32, x_q.device)
    dt = _dtype_code(ys[0].dtype)
    _check("bitnet_ternary_linear_multi", lib().bitnet_ternary_linear_multi(
        arr, len(mats), _ptr(x_q), _ptr(x_scale), m, k, dt, _stream(stream)))
    return ys


def bitnet_quant_linear_multi(mats, x, x_q=None, x_scale=None, y_dtype=None, stream=None,
                              up=None, norm_weight=None, eps=1e-5):
    """Quantise x once and apply several matrices: returns (list of y, x_q, x_scale).
    ``up`` / ``norm_weight`` / ``eps``: the input prologue (bitnet_quant_linear_ex)."""
    import torch
    _need_cuda(x)
    m, k = x.shape
    if x_q is None:
        x_q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty(m, dtype=torch.float32, device=x.device)
    _check_act_operands(x, x_q, x_scale, up, norm_weight)
    arr, ys = _matrices(mats, m, k, y_dtype or torch.float32, x.device)
    dt = _dtype_code(ys[0].dtype)
    pro = _prologue(x, up, norm_weight, eps)
    if pro is None:
        _check("bitnet_quant_linear_multi", lib().bitnet_quant_linear_multi(
            arr, len(mats), _ptr(x), _dtype_code(x.dtype), m, k, _ptr(x_q), _ptr(x_scale), dt,
            _stream(stream)))
    else:
        _check("bitnet_quant_linear_ex", lib().bitnet_quant_linear_ex(
            arr, len(mats), _ptr(x), _dtype_code(x.dtype), pro, m, k, _ptr(x_q), _ptr(x_scale),
            dt, _stream(stream)))
    return ys, x_q, x_scale


# ---------------------------------------------------------------------------
# five ternary weights per byte (T1 layout)
# ---------------------------------------------------------------------------

def bitnet_t1_packed_bytes(n: int, k: int) -> int:
    return lib().bitnet_t1_packed_bytes(n, k)


def t1_row_bytes(k: int) -> int:
    """Bytes per row of a T1 matrix (16 * ceil(K / 80))."""
    return lib().bitnet_t1_packed_bytes(1, k)


def bitnet_quantize_weights_t1(w, packed=None, scale=None, workspace=None, stream=None):
    """w: [N, K] fp32/bf16 -> (T1 packed uint8 [N, 16*ceil(K/80)], gamma* fp32 [1])."""
    import torch
    _need_cuda(w)
    n, k = w.shape
    dev = w.device
    if packed is None:
        packed = torch.empty((n, t1_row_bytes(k)), dtype=torch.uint8, device=dev)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=dev)
    ws_bytes = lib().bitnet_quantize_weights_workspace_bytes(n, k)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    _expect(w, (n, k), _floats(), "w")
    _expect(packed, (n, t1_row_bytes(k)), torch.uint8, "packed")
    _check_scale(scale)
    _need_cuda(workspace)
    _check("bitnet_quantize_weights_t1", lib().bitnet_quantize_weights_t1(
        _ptr(w), _dtype_code(w.dtype), n, k, _ptr(packed), _ptr(scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return packed, scale


def bitnet_repack_t1(w_packed, out=None, stream=None):
    """2-bit packed [N, K/4] -> T1 packed [N, 16*ceil(K/80)]."""
    import torch
    _need_cuda(w_packed)
    n, kb = w_packed.shape
    k = 4 * kb
    if out is None:
        out = torch.empty((n, t1_row_bytes(k)), dtype=torch.uint8, device=w_packed.device)
    _expect(w_packed, (n, kb), torch.uint8, "w_packed")
    _expect(out, (n, t1_row_bytes(k)), torch.uint8, "out")
    _check("bitnet_repack_t1", lib().bitnet_repack_t1(_ptr(w_packed), n, k, _ptr(out),
                                                      _stream(stream)))
    return out


def bitnet_ternary_linear_t1(mats, x_q, x_scale, y_dtype=None, stream=None):
    """Several (w_t1, w_scale[, y[, acc_out]]) sharing x_q -> list of y."""
    import torch
    _need_cuda(x_q, x_scale)
    m, k = x_q.shape
    _expect(x_q, (m, k), torch.int8, "x_q")
    _expect(x_scale, (m,), torch.float32, "x_scale")
    arr, ys = _matrices(mats, m, k, y_dtype or torch.float32, x_q.device, t1_row_bytes(k))
    _check("bitnet_ternary_linear_t1", lib().bitnet_ternary_linear_t1(
        arr, len(mats), _ptr(x_q), _ptr(x_scale), m, k, _dtype_code(ys[0].dtype),
        _stream(stream)))
    return ys


def bitnet_quant_linear_t1(mats, x, x_q=None, x_scale=None, y_dtype=None, stream=None, up=None,
                           norm_weight=None, eps=1e-5):
    """bitnet_quant_linear_multi on T1 matrices: returns (list of y, x_q, x_scale)."""
    import torch
    _need_cuda(x)
    m, k = x.shape
    if x_q is None:
        x_q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty(m, dtype=torch.float32, device=x.device)
    _check_act_operands(x, x_q, x_scale, up, norm_weight)
    arr, ys = _matrices(mats, m, k, y_dtype or torch.float32, x.device, t1_row_bytes(k))
    _check("bitnet_quant_linear_t1", lib().bitnet_quant_linear_t1(
        arr, len(mats), _ptr(x), _dtype_code(x.dtype), _prologue(x, up, norm_weight, eps), m, k,
        _ptr(x_q), _ptr(x_scale), _dtype_code(ys[0].dtype), _stream(stream)))
    return ys, x_q, x_scale


def prefill_layout_shape(n: int, k: int):
    """Shape of an N x K matrix in the prefill layout as a uint8 tensor: one row
    per 32 weight rows, ceil(K/128) * 1024 bytes each."""
    return ((n + 31) // 32, ((k + 127) // 128) * 1024)


def bitnet_repack_prefill(w_packed, out=None, stream=None):
    """2-bit packed [N, K/4] -> the prefill layout, uint8 prefill_layout_shape(N, K)."""
    import torch
    _need_cuda(w_packed)
    n, kb = w_packed.shape
    k = 4 * kb
    shape = prefill_layout_shape(n, k)
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=w_packed.device)
    _expect(w_packed, (n, kb), torch.uint8, "w_packed")
    _expect(out, shape, torch.uint8, "out")
    _check("bitnet_repack_prefill", lib().bitnet_repack_prefill(_ptr(w_packed), n, k, _ptr(out),
                                                                _stream(stream)))
    return out


def bitnet_ternary_linear_prefill(mats, x_q, x_scale, y_dtype=None, stream=None):
    """Several (w_prefill, w_scale, N[, y[, acc_out]]) sharing x_q -> list of y; each
    w_prefill in the prefill layout (prefill_layout_shape(N, K))."""
    import torch
    _need_cuda(x_q, x_scale)
    m, k = x_q.shape
    _expect(x_q, (m, k), torch.int8, "x_q")
    _expect(x_scale, (m,), torch.float32, "x_scale")
    if not mats:
        raise ValueError("at least one matrix")
    arr = (BitnetMatrix * len(mats))()
    ys = []
    for i, t in enumerate(mats):
        w, w_scale, n = t[0], t[1], int(t[2])
        y = t[3] if len(t) > 3 and t[3] is not None else torch.empty(
            (m, n), dtype=(y_dtype or torch.float32) if not ys else ys[0].dtype,
            device=x_q.device)
        acc = t[4] if len(t) > 4 else None
        _expect(w, prefill_layout_shape(n, k), torch.uint8, f"w_prefill[{i}]")
        _check_scale(w_scale)
        _expect(y, (m, n), ys[0].dtype if ys else _floats(), f"y[{i}]")
        _expect(acc, (m, n), torch.int32, f"acc_out[{i}]")
        arr[i] = BitnetMatrix(w.data_ptr(), w_scale.data_ptr(), n, y.data_ptr(),
                              0 if acc is None else acc.data_ptr())
        ys.append(y)
    _check("bitnet_ternary_linear_prefill", lib().bitnet_ternary_linear_prefill(
        arr, len(mats), _ptr(x_q), _ptr(x_scale), m, k, _dtype_code(ys[0].dtype),
        _stream(stream)))
    return ys


# ---------------------------------------------------------------------------
# lookup-table contraction
# ---------------------------------------------------------------------------

def bitnet_ternary_linear_lut(w_packed, w_scale, x_q, x_scale, y=None, y_dtype=None,
                              acc_out=None, workspace=None, stream=None):
    """bitnet_ternary_linear by table lookup: packed W [N, K/4] x int8 X [M, K] -> y."""
    import torch
    _need_cuda(w_packed, w_scale, x_q, x_scale, acc_out)
    m, k = x_q.shape
    n = w_packed.shape[0]
    if w_packed.shape[1] * 4 != k:
        raise ValueError("w_packed and x_q disagree on K")
    if y is None:
        y = torch.empty((m, n), dtype=y_dtype or torch.float32, device=x_q.device)
    ws_bytes = lib().bitnet_lut_workspace_bytes(n, k)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x_q.device)
    _expect(w_packed, (n, k // 4), torch.uint8, "w_packed")
    _check_scale(w_scale)
    _expect(x_q, (m, k), torch.int8, "x_q")
    _expect(x_scale, (m,), torch.float32, "x_scale")
    _expect(y, (m, n), _floats(), "y")
    _expect(acc_out, (m, n), torch.int32, "acc_out")
    _need_cuda(workspace)
    _check("bitnet_ternary_linear_lut", lib().bitnet_ternary_linear_lut(
        _ptr(w_packed), _ptr(w_scale), _ptr(x_q), _ptr(x_scale), m, n, k, _ptr(y),
        _dtype_code(y.dtype), _ptr(acc_out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return y



# ---------------------------------------------------------------------------
# decode chain: every stage of a token in one launch
# ---------------------------------------------------------------------------

class BitnetChainStage(ctypes.Structure):
    """struct bitnet_chain_stage of the public header."""
    _fields_ = [("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int), ("y_dtype", ctypes.c_int),
                ("K", ctypes.c_int64), ("mats", ctypes.POINTER(BitnetMatrix)),
                ("count", ctypes.c_int), ("x_q", ctypes.c_void_p), ("x_scale", ctypes.c_void_p)]


class BitnetChain(ctypes.Structure):
    """struct bitnet_chain of the public header."""
    _fields_ = [("plan", ctypes.c_void_p), ("n_stages", ctypes.c_int), ("M", ctypes.c_int),
                ("grid", ctypes.c_int), ("kmax", ctypes.c_int), ("tmax", ctypes.c_int),
                ("ring", ctypes.c_int)]


SIGNATURES["bitnet_prefill_tile"] = (_I, [_I64, ctypes.POINTER(_I64), _I, _I64,
                                          ctypes.POINTER(_I), ctypes.POINTER(_I),
                                          ctypes.POINTER(_I64), ctypes.POINTER(_I64)])
SIGNATURES["bitnet_chain_plan_bytes"] = (_SZ, [_I])
SIGNATURES["bitnet_chain_plan"] = (_I, [ctypes.POINTER(BitnetChainStage), _I, _I64, _P, _SZ,
                                        ctypes.POINTER(BitnetChain)])
SIGNATURES["bitnet_chain_run"] = (_I, [ctypes.POINTER(BitnetChain), _P])
SIGNATURES["bitnet_chain_error"] = (_I, [ctypes.POINTER(BitnetChain), ctypes.POINTER(_I)])


class Chain:
    """A planned decode chain: the device plan, the bitnet_chain handle and the
    tensors it points to (kept alive here)."""

    def __init__(self, plan, handle, keep):
        self.plan = plan
        self.handle = handle
        self._keep = keep


def bitnet_chain_plan(stages, m):
    """stages: list of dicts with x [M, K] (fp32/bf16), mats [(w_packed, w_scale, y[,
    acc_out])], x_q int8 [M, K], x_scale fp32 [M].  Every y must already exist (a
    later stage's x is usually an earlier stage's y).  Returns a Chain."""
    import torch
    n = len(stages)
    arr = (BitnetChainStage * n)()
    keep = []
    device = None
    for i, st in enumerate(stages):
        x, x_q, x_scale = st["x"], st["x_q"], st["x_scale"]
        _need_cuda(x)
        if x.dim() != 2 or x.shape[0] != m:
            raise ValueError(f"stage {i}: x must be [M, K] with M = {m}")
        k = x.shape[1]
        _check_act_operands(x, x_q, x_scale)
        mats = st["mats"]
        if any(len(t) < 3 or t[2] is None for t in mats):
            raise ValueError(f"stage {i}: every matrix needs its output y")
        marr, ys = _matrices(mats, m, k, mats[0][2].dtype, x.device)
        arr[i] = BitnetChainStage(x.data_ptr(), _dtype_code(x.dtype), _dtype_code(ys[0].dtype), k,
                                  marr, len(mats), x_q.data_ptr(), x_scale.data_ptr())
        keep += [x, x_q, x_scale, marr, ys, mats]
        device = x.device
    nbytes = lib().bitnet_chain_plan_bytes(n)
    plan = torch.empty(nbytes, dtype=torch.uint8, device=device)
    handle = BitnetChain()
    _check("bitnet_chain_plan", lib().bitnet_chain_plan(arr, n, m, _ptr(plan), nbytes,
                                                        ctypes.byref(handle)))
    return Chain(plan, handle, keep)


def bitnet_chain_run(chain, stream=None):
    """Enqueue one launch of the whole chain (one token)."""
    _check("bitnet_chain_run", lib().bitnet_chain_run(ctypes.byref(chain.handle), _stream(stream)))


def bitnet_chain_error(chain) -> int:
    """The plan's sticky error word (0 = every run completed its barriers); syncs."""
    e = ctypes.c_int(0)
    _check("bitnet_chain_error", lib().bitnet_chain_error(ctypes.byref(chain.handle),
                                                          ctypes.byref(e)))
    return e.value


def bitnet_prefill_tile(m, ns, k):
    """(tokens per tile, rows per tile, first launch tokens, first launch rows) of the
    prefill kernel for M tokens over matrices with ns rows and inputs of K
    (bitnet_prefill_tile)."""
    arr = (ctypes.c_int64 * len(ns))(*ns)
    bm, bn = ctypes.c_int(0), ctypes.c_int(0)
    first, rows = ctypes.c_int64(0), ctypes.c_int64(0)
    _check("bitnet_prefill_tile", lib().bitnet_prefill_tile(m, arr, len(ns), k, ctypes.byref(bm),
                                                            ctypes.byref(bn), ctypes.byref(first),
                                                            ctypes.byref(rows)))
    return bm.value, bn.value, first.value, rows.value
