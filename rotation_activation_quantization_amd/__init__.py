"""SignRot's online activation path on MI355X: Python binding of libsignrot.

Argument marshalling only: every step of the path runs in the HIP library
(`libsignrot.so`, built in-tree by `build.py`).  Torch supplies device memory
and the current stream; nothing here computes on the CPU, and every call fails
loudly when the library is missing.

The C ABI is declared in include/signrot.h; the functions here keep its names.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsignrot.so")

SIGNROT_OK = 0
SIGNROT_EINVAL = -1
SIGNROT_EUNSUPPORTED_N = -2
SIGNROT_EHIP = -3

_lib = None


class SignRotError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libsignrot.so (raises when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m rotation_activation_quantization_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    L.signrot_supported_n.argtypes = [i64]
    L.signrot_supported_n.restype = ctypes.c_int
    L.signrot_calibrate.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp]
    L.signrot_calibrate.restype = ctypes.c_int
    L.signrot_calibrate_noalloc.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp]
    L.signrot_calibrate_noalloc.restype = ctypes.c_int
    L.signrot_rotate_quant_int4.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, vp]
    L.signrot_rotate_quant_int4.restype = ctypes.c_int
    L.signrot_rotate_quant_int4_outlier.argtypes = [vp, i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp]
    L.signrot_rotate_quant_int4_outlier.restype = ctypes.c_int
    L.signrot_swiglu_rotate_quant_int4.argtypes = [vp, vp, i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp]
    L.signrot_swiglu_rotate_quant_int4.restype = ctypes.c_int
    L.signrot_rotate_quant_int4_zint.argtypes = [vp, i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp]
    L.signrot_rotate_quant_int4_zint.restype = ctypes.c_int
    L.signrot_dequant.argtypes = [vp, vp, vp, i64, i64, vp, vp]
    L.signrot_dequant.restype = ctypes.c_int
    L.signrot_fold_weights.argtypes = [vp, i64, i64, i64, vp, vp, vp]
    L.signrot_fold_weights.restype = ctypes.c_int
    L.signrot_weight_rowsum.argtypes = [vp, i64, i64, i64, vp, vp]
    L.signrot_weight_rowsum.restype = ctypes.c_int
    L.signrot_int4_linear.argtypes = [vp, vp, vp, i64, i64, vp, i64, vp, i64, vp, vp]
    L.signrot_int4_linear.restype = ctypes.c_int
    L.signrot_int4_linear_kernel_name.argtypes = [vp, i64, i64, vp, i64, i64]
    L.signrot_int4_linear_kernel_name.restype = ctypes.c_char_p
    L.signrot_stream_ceiling.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp]
    L.signrot_stream_ceiling.restype = ctypes.c_int
    L.signrot_strerror.argtypes = [ctypes.c_int]
    L.signrot_strerror.restype = ctypes.c_char_p
    L.signrot_last_error.argtypes = []
    L.signrot_last_error.restype = ctypes.c_char_p
    L.signrot_debug_h28.argtypes = [vp]
    L.signrot_debug_h28.restype = ctypes.c_int
    L.signrot_debug_outer.argtypes = [ctypes.c_int, vp]
    L.signrot_debug_outer.restype = ctypes.c_int
    L.signrot_outer_order.argtypes = [i64]
    L.signrot_outer_order.restype = ctypes.c_int
    L.signrot_debug_outer_folded.argtypes = [ctypes.c_int, ctypes.c_int, vp]
    L.signrot_debug_outer_folded.restype = ctypes.c_int
    L.signrot_outer_fold.argtypes = [i64]
    L.signrot_outer_fold.restype = ctypes.c_int
    L.signrot_kernel_name.argtypes = [i64]
    L.signrot_kernel_name.restype = ctypes.c_char_p
    _lib = L
    return L


EXPORTED = (
    "signrot_supported_n",
    "signrot_calibrate",
    "signrot_calibrate_noalloc",
    "signrot_rotate_quant_int4",
    "signrot_rotate_quant_int4_outlier",
    "signrot_rotate_quant_int4_zint",
    "signrot_swiglu_rotate_quant_int4",
    "signrot_dequant",
    "signrot_fold_weights",
    "signrot_weight_rowsum",
    "signrot_int4_linear",
    "signrot_int4_linear_kernel_name",
    "signrot_strerror",
    "signrot_last_error",
    "signrot_debug_h28",
    "signrot_debug_outer",
    "signrot_debug_outer_folded",
    "signrot_outer_order",
    "signrot_outer_fold",
    "signrot_kernel_name",
    "signrot_stream_ceiling",
)


def check(status: int, where: str) -> None:
    if status != SIGNROT_OK:
        L = lib()
        detail = (L.signrot_last_error() or b"").decode() or L.signrot_strerror(status).decode()
        raise SignRotError(status, where, detail)


def supported_n(n: int) -> bool:
    return bool(lib().signrot_supported_n(int(n)))


def kernel_name(n: int) -> str | None:
    r = lib().signrot_kernel_name(int(n))
    return r.decode() if r else None


def outer_order(n: int) -> int:
    """The outer Hadamard order m of n = m * 2^k (1 for n = 2^k, 0 if unsupported)."""
    return int(lib().signrot_outer_order(int(n)))


def debug_outer(m: int):
    """The library's outer factor H_m as an m x m list of +-1 rows (host only)."""
    buf = (ctypes.c_int8 * (m * m))()
    check(lib().signrot_debug_outer(int(m), ctypes.addressof(buf)), "signrot_debug_outer")
    return [list(buf[r * m:(r + 1) * m]) for r in range(m)]


def debug_outer_folded(m: int, fold: int):
    """The library's folded outer factor H_m (x) Syl_{2^fold} (host only)."""
    import numpy as np

    mm = int(m) << int(fold)
    buf = (ctypes.c_int8 * (mm * mm))()
    check(lib().signrot_debug_outer_folded(int(m), int(fold), ctypes.addressof(buf)), "signrot_debug_outer_folded")
    return np.frombuffer(buf, dtype=np.int8).reshape(mm, mm).copy()


def outer_fold(n: int) -> int:
    """Sylvester bits the rotate kernel for n folds into its outer factor."""
    return int(lib().signrot_outer_fold(int(n)))


def debug_h28():
    """The library's own H28 as a 28x28 list of +-1 rows."""
    buf = (ctypes.c_int8 * 784)()
    check(lib().signrot_debug_h28(ctypes.addressof(buf)), "signrot_debug_h28")
    return [list(buf[r * 28:(r + 1) * 28]) for r in range(28)]


def _stream_of(t):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _rows(x):
    """(pointer, tokens, n, ld) of a [T, n] bf16 tensor whose rows are contiguous."""
    import torch

    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a 2-D bfloat16 CUDA tensor")
    if x.shape[1] > 0 and x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    ld = x.stride(0) if x.shape[0] > 1 else max(x.shape[1], (x.shape[1] + 7) // 8 * 8)
    return x.data_ptr(), x.shape[0], x.shape[1], ld


def signrot_calibrate(x):
    """Calibrate on a bf16 batch [T, n] -> (d int8 [n] on the device, c, t, M_c)."""
    import torch

    ptr, t, n, ld = _rows(x)
    d = torch.empty(n, dtype=torch.int8, device=x.device)
    c = ctypes.c_int32()
    tt = ctypes.c_int64()
    m = ctypes.c_float()
    check(lib().signrot_calibrate(ptr, t, n, ld, d.data_ptr(), ctypes.addressof(c), ctypes.addressof(tt),
                                  ctypes.addressof(m), _stream_of(x)), "signrot_calibrate")
    return d, c.value, tt.value, m.value


def signrot_calibrate_noalloc(x, d_out):
    """signrot_calibrate into a caller-provided d (int8 [n] on the device),
    without any allocation in the library -> (c, t, M_c)."""
    import torch

    ptr, t, n, ld = _rows(x)
    if d_out.dtype != torch.int8 or d_out.numel() != n or not d_out.is_contiguous():
        raise ValueError("d_out must be a contiguous int8 tensor of n entries")
    c = ctypes.c_int32()
    tt = ctypes.c_int64()
    m = ctypes.c_float()
    check(lib().signrot_calibrate_noalloc(ptr, t, n, ld, d_out.data_ptr(), ctypes.addressof(c), ctypes.addressof(tt),
                                          ctypes.addressof(m), _stream_of(x)), "signrot_calibrate_noalloc")
    return c.value, tt.value, m.value


def signrot_rotate_quant_int4(x, d, y_out: bool = False, out=None):
    """bf16 [T, n] and d int8 [n] -> (codes u8 [T, n/2], scale f32 [T], zero f32 [T]
    [, y f32 [T, n]]).  `out` may pass preallocated (codes, scale, zero[, y])."""
    import torch

    ptr, t, n, ld = _rows(x)
    if d.dtype != torch.int8 or d.numel() != n or not d.is_contiguous():
        raise ValueError("d must be a contiguous int8 tensor of n entries")
    if out is None:
        codes = torch.empty((t, n // 2), dtype=torch.uint8, device=x.device)
        scale = torch.empty(t, dtype=torch.float32, device=x.device)
        zero = torch.empty(t, dtype=torch.float32, device=x.device)
        y = torch.empty((t, n), dtype=torch.float32, device=x.device) if y_out else None
    else:
        codes, scale, zero = out[:3]
        y = out[3] if len(out) > 3 else None
    check(lib().signrot_rotate_quant_int4(ptr, t, n, ld, d.data_ptr(), codes.data_ptr(), scale.data_ptr(),
                                          zero.data_ptr(), y.data_ptr() if y is not None else None,
                                          _stream_of(x)), "signrot_rotate_quant_int4")
    return (codes, scale, zero, y) if y is not None else (codes, scale, zero)


def signrot_rotate_quant_int4_outlier(x, c: int, sigma: int, y_out: bool = False, out=None):
    """Like signrot_rotate_quant_int4 for d = sigma * (row c of H), given as the
    outlier channel c and sigma = sign(M_c) (what signrot_calibrate returns)."""
    import torch

    ptr, t, n, ld = _rows(x)
    if out is None:
        codes = torch.empty((t, n // 2), dtype=torch.uint8, device=x.device)
        scale = torch.empty(t, dtype=torch.float32, device=x.device)
        zero = torch.empty(t, dtype=torch.float32, device=x.device)
        y = torch.empty((t, n), dtype=torch.float32, device=x.device) if y_out else None
    else:
        codes, scale, zero = out[:3]
        y = out[3] if len(out) > 3 else None
    check(lib().signrot_rotate_quant_int4_outlier(ptr, t, n, ld, int(c), int(sigma), codes.data_ptr(),
                                                  scale.data_ptr(), zero.data_ptr(),
                                                  y.data_ptr() if y is not None else None, _stream_of(x)),
          "signrot_rotate_quant_int4_outlier")
    return (codes, scale, zero, y) if y is not None else (codes, scale, zero)


def signrot_rotate_quant_int4_zint(x, c: int, sigma: int, out=None):
    """The integer zero-point variant: zero = rint(-mn / s) (integral floats),
    codes = clamp(rint(y / s) + zero, 0, 15); d given as (c, sigma)."""
    import torch

    ptr, t, n, ld = _rows(x)
    if out is None:
        codes = torch.empty((t, n // 2), dtype=torch.uint8, device=x.device)
        scale = torch.empty(t, dtype=torch.float32, device=x.device)
        zero = torch.empty(t, dtype=torch.float32, device=x.device)
    else:
        codes, scale, zero = out[:3]
    check(lib().signrot_rotate_quant_int4_zint(ptr, t, n, ld, int(c), int(sigma), codes.data_ptr(),
                                               scale.data_ptr(), zero.data_ptr(), _stream_of(x)),
          "signrot_rotate_quant_int4_zint")
    return codes, scale, zero


def signrot_swiglu_rotate_quant_int4(gate, up, c: int, sigma: int, y_out: bool = False, out=None):
    """The online path on x = bf16(SiLU(gate) * up), the producer fused in:
    gate and up bf16 [T, n] (same row stride) -> (codes, scale, zero[, y])."""
    import torch

    ptr, t, n, ld = _rows(gate)
    uptr, tu, nu, ldu = _rows(up)
    if (tu, nu) != (t, n) or (t > 1 and ldu != ld):
        raise ValueError("gate and up must have the same shape and row stride")
    if out is None:
        codes = torch.empty((t, n // 2), dtype=torch.uint8, device=gate.device)
        scale = torch.empty(t, dtype=torch.float32, device=gate.device)
        zero = torch.empty(t, dtype=torch.float32, device=gate.device)
        y = torch.empty((t, n), dtype=torch.float32, device=gate.device) if y_out else None
    else:
        codes, scale, zero = out[:3]
        y = out[3] if len(out) > 3 else None
    check(lib().signrot_swiglu_rotate_quant_int4(ptr, uptr, t, n, ld, int(c), int(sigma), codes.data_ptr(),
                                                 scale.data_ptr(), zero.data_ptr(),
                                                 y.data_ptr() if y is not None else None, _stream_of(gate)),
          "signrot_swiglu_rotate_quant_int4")
    return (codes, scale, zero, y) if y is not None else (codes, scale, zero)


def signrot_dequant(codes, scale, zero, n: int | None = None):
    """codes u8 [T, n/2], scale/zero f32 [T] -> y_hat f32 [T, n]."""
    import torch

    t = codes.shape[0]
    n = codes.shape[1] * 2 if n is None else int(n)
    y = torch.empty((t, n), dtype=torch.float32, device=codes.device)
    check(lib().signrot_dequant(codes.data_ptr(), scale.data_ptr(), zero.data_ptr(), t, n, y.data_ptr(),
                                _stream_of(codes)), "signrot_dequant")
    return y


def signrot_fold_weights(w, d):
    """Weights bf16 [rows, n] (one row per output feature of x . W^T) and the
    activations' sign vector d -> W' = W . H . D / sqrt(n), float32 [rows, n]."""
    import torch

    ptr, rows, n, ld = _rows(w)
    if d.dtype != torch.int8 or d.numel() != n or not d.is_contiguous():
        raise ValueError("d must be a contiguous int8 tensor of n entries")
    out = torch.empty((rows, n), dtype=torch.float32, device=w.device)
    check(lib().signrot_fold_weights(ptr, rows, n, ld, d.data_ptr(), out.data_ptr(), _stream_of(w)),
          "signrot_fold_weights")
    return out


def signrot_weight_rowsum(w):
    """bf16 [rows, n] -> rowsum f32 [rows], the exact sum of each row."""
    import torch

    ptr, rows, n, ld = _rows(w)
    out = torch.empty(rows, dtype=torch.float32, device=w.device)
    check(lib().signrot_weight_rowsum(ptr, rows, n, ld, out.data_ptr(), _stream_of(w)), "signrot_weight_rowsum")
    return out


def _linear_operands(codes, w):
    import torch

    if codes.dtype != torch.uint8 or codes.dim() != 2 or not codes.is_contiguous():
        raise ValueError("codes must be a contiguous 2-D uint8 tensor")
    ptr, rows, n, ld = _rows(w)
    if codes.shape[1] * 2 != n:
        raise ValueError(f"codes hold {codes.shape[1] * 2} channels, w has {n}")
    return ptr, rows, n, ld


def signrot_int4_linear(codes, scale, zero, w, rowsum, out=None):
    """INT4 activations (codes u8 [T, n/2], scale/zero f32 [T]) times the folded
    weight w bf16 [rows, n] -> f32 [T, rows] = (scale * (q - zero)) . w^T,
    with rowsum = signrot_weight_rowsum(w)."""
    import torch

    wptr, rows, n, ld = _linear_operands(codes, w)
    t = codes.shape[0]
    for name, v, size in (("scale", scale, t), ("zero", zero, t), ("rowsum", rowsum, rows)):
        if v.dtype != torch.float32 or v.numel() != size or not v.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor of {size} entries")
    if out is None:
        out = torch.empty((t, rows), dtype=torch.float32, device=codes.device)
    check(lib().signrot_int4_linear(codes.data_ptr(), scale.data_ptr(), zero.data_ptr(), t, n, wptr, ld,
                                    rowsum.data_ptr(), rows, out.data_ptr(), _stream_of(codes)),
          "signrot_int4_linear")
    return out


def int4_linear_kernel_name(codes, w) -> str | None:
    wptr, rows, n, ld = _linear_operands(codes, w)
    r = lib().signrot_int4_linear_kernel_name(codes.data_ptr(), codes.shape[0], n, wptr, ld, rows)
    return r.decode() if r else None


def signrot_stream_ceiling(x, out=None):
    """The memory-traffic ceiling kernel (a measurement aid: the online path's
    bytes per token, no arithmetic) on bf16 [T, n] -> (u8 [T, n/2], f32 [T],
    f32 [T])."""
    import torch

    ptr, t, n, ld = _rows(x)
    if out is None:
        out = (torch.empty((t, n // 2), dtype=torch.uint8, device=x.device),
               torch.empty(t, dtype=torch.float32, device=x.device),
               torch.empty(t, dtype=torch.float32, device=x.device))
    check(lib().signrot_stream_ceiling(ptr, t, n, ld, out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(),
                                       _stream_of(x)), "signrot_stream_ceiling")
    return out


# short aliases
calibrate = signrot_calibrate
rotate_quant_int4 = signrot_rotate_quant_int4
rotate_quant_int4_outlier = signrot_rotate_quant_int4_outlier
rotate_quant_int4_zint = signrot_rotate_quant_int4_zint
swiglu_rotate_quant_int4 = signrot_swiglu_rotate_quant_int4
dequant = signrot_dequant
fold_weights = signrot_fold_weights
weight_rowsum = signrot_weight_rowsum
int4_linear = signrot_int4_linear
