"""ctypes binding of librsq.so: same names as the C ABI, argument marshalling only.

Tensors are torch tensors on the current HIP device; every call enqueues on
the current torch stream (``torch.cuda.current_stream()``) unless a stream is
given. All arithmetic happens in the library's HIP kernels. A non-zero status
raises ``RsqError`` carrying the library's message.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librsq.so")

RSQ_OK, RSQ_ERR_INVALID_ARG, RSQ_ERR_UNSUPPORTED, RSQ_ERR_WORKSPACE, RSQ_ERR_HIP = range(5)
RSQ_F32, RSQ_BF16 = 0, 1
RSQ_QA_RMSNORM = 1
RSQ_FP4 = 0x100          # bits = 3 | RSQ_FP4: 3-bit codes in the fp4 layout
RSQ_MAX_RANK = 64


class RsqError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: {msg} (status {status})")
        self.status = status


def _load() -> C.CDLL:
    # torch ships its own HIP runtime under the same soname; loading torch
    # first makes librsq.so bind to that one copy (two runtimes in one
    # process do not share the device).
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python rotation_bit_post_amd/build.py` "
            "(there is no fallback implementation)")
    lib = C.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_size_t
    sig = {
        "rsq_version": (i32, []),
        "rsq_status_str": (C.c_char_p, [i32]),
        "rsq_last_error": (C.c_char_p, []),
        "rsq_packed_row_bytes": (sz, [i64, i32]),
        "rsq_site_bytes": (sz, [i64, i32]),
        "rsq_site_prepare": (i32, [vp, vp, i64, i32, vp, vp]),
        "rsq_subspace_correct": (i32, [vp, vp, i32, i64, i64, i64, vp, i32, vp]),
        "rsq_quant_act": (i32, [vp, i32, i64, i64, i64, C.c_uint, vp, f32, i32, vp, vp, vp]),
        "rsq_correct_quant": (i32, [vp, vp, i32, i64, i64, vp, i32, vp, f32, i32, vp, vp, vp]),
        "rsq_qgemm": (i32, [vp, vp, i64, vp, vp, i64, i64, i32, vp, i32, i64, vp, vp]),
        "rsq_qgemm_residual": (i32, [vp, vp, i64, vp, vp, i64, i64, i32, vp, i64, vp, i32, i64, vp]),
        "rsq_layer_fused": (i32, [vp, vp, i32, i64, i64, vp, i32, vp, f32, i32, vp, vp, vp, vp, i64, vp, i32, vp]),
        "rsq_codes_to_fp4": (i32, [vp, i64, i64, vp, vp]),
        "rsq_qgemm_fp4": (i32, [vp, vp, i64, vp, vp, i64, i64, vp, i64, vp, i32, i64, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


LIB = _load()
EXPORTS = ("rsq_version", "rsq_status_str", "rsq_last_error", "rsq_packed_row_bytes", "rsq_site_bytes",
           "rsq_site_prepare", "rsq_subspace_correct", "rsq_quant_act", "rsq_correct_quant", "rsq_qgemm", "rsq_qgemm_residual",
           "rsq_layer_fused", "rsq_codes_to_fp4", "rsq_qgemm_fp4")


def _check(status: int, func: str) -> None:
    if status != RSQ_OK:
        raise RsqError(status, func, LIB.rsq_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return RSQ_BF16
    if t.dtype == torch.float32:
        return RSQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


# ----------------------------------------------------------------- queries
def rsq_version() -> int:
    return LIB.rsq_version()


def rsq_packed_row_bytes(k: int, bits: int) -> int:
    return LIB.rsq_packed_row_bytes(k, bits)


def rsq_site_bytes(d: int, r: int) -> int:
    return LIB.rsq_site_bytes(d, r)


# ---------------------------------------------------------------- compute
def rsq_site_prepare(U, M, site, stream=None) -> None:
    """U: (d, r) float32, M: (r, r) float32, site: uint8 buffer of rsq_site_bytes(d, r)."""
    d, r = U.shape
    _check(LIB.rsq_site_prepare(_ptr(U), _ptr(M), d, r, _ptr(site), _stream(stream)), "rsq_site_prepare")


def rsq_subspace_correct(h_in, h_out, site, r: int, stream=None) -> None:
    """h_out = h_in + ((h_in U) M) U^T per row; h_in, h_out: (n, d) with the same dtype and row stride."""
    n, d = h_in.shape
    _check(LIB.rsq_subspace_correct(_ptr(h_in), _ptr(h_out), _dtype_code(h_in), n, d, h_in.stride(0),
                                    _ptr(site), r, _stream(stream)), "rsq_subspace_correct")


def rsq_quant_act(x, codes, scales, bits: int, rmsnorm: bool = False, norm_w=None, eps: float = 1e-5,
                  stream=None) -> None:
    n, k = x.shape
    flags = RSQ_QA_RMSNORM if rmsnorm else 0
    _check(LIB.rsq_quant_act(_ptr(x), _dtype_code(x), n, k, x.stride(0), flags, _ptr(norm_w), eps, bits,
                             _ptr(codes), _ptr(scales), _stream(stream)), "rsq_quant_act")


def rsq_correct_quant(h_in, h_out, site, r: int, codes, scales, bits: int, norm_w=None, eps: float = 1e-5,
                      stream=None) -> None:
    n, d = h_in.shape
    _check(LIB.rsq_correct_quant(_ptr(h_in), _ptr(h_out), _dtype_code(h_in), n, d, _ptr(site), r, _ptr(norm_w),
                                 eps, bits, _ptr(codes), _ptr(scales), _stream(stream)), "rsq_correct_quant")


def rsq_qgemm(a_codes, a_scales, n: int, w_codes, w_scales, n_out: int, k: int, bits: int, y, acc_out=None,
              stream=None) -> None:
    _check(LIB.rsq_qgemm(_ptr(a_codes), _ptr(a_scales), n, _ptr(w_codes), _ptr(w_scales), n_out, k, bits,
                         _ptr(y), _dtype_code(y), y.stride(0), _ptr(acc_out), _stream(stream)), "rsq_qgemm")


def rsq_qgemm_residual(a_codes, a_scales, n: int, w_codes, w_scales, n_out: int, k: int, bits: int, residual, y,
                       stream=None) -> None:
    """y = dequantised quantised linear + residual (residual may be y itself)."""
    if residual.dtype != y.dtype:
        raise ValueError("residual and y must have the same dtype")
    _check(LIB.rsq_qgemm_residual(_ptr(a_codes), _ptr(a_scales), n, _ptr(w_codes), _ptr(w_scales), n_out, k, bits,
                                  _ptr(residual), residual.stride(0), _ptr(y), _dtype_code(y), y.stride(0),
                                  _stream(stream)), "rsq_qgemm_residual")


def rsq_codes_to_fp4(codes, rows: int, k: int, fp4, stream=None) -> None:
    """Packed int3 rows -> fp4 rows (k / 2 bytes each), the same code values."""
    _check(LIB.rsq_codes_to_fp4(_ptr(codes), rows, k, _ptr(fp4), _stream(stream)), "rsq_codes_to_fp4")


def rsq_qgemm_fp4(a_fp4, a_scales, n: int, w_fp4, w_scales, n_out: int, k: int, y, residual=None, acc_out=None,
                  stream=None) -> None:
    """The 3-bit quantised linear on fp4 codes; residual (optional) may be y itself."""
    if residual is not None and residual.dtype != y.dtype:
        raise ValueError("residual and y must have the same dtype")
    _check(LIB.rsq_qgemm_fp4(_ptr(a_fp4), _ptr(a_scales), n, _ptr(w_fp4), _ptr(w_scales), n_out, k, _ptr(residual),
                             residual.stride(0) if residual is not None else 0, _ptr(y), _dtype_code(y), y.stride(0),
                             _ptr(acc_out), _stream(stream)), "rsq_qgemm_fp4")


def rsq_layer_fused(h_in, h_out, site, r: int, codes, scales, w_codes, w_scales, n_out: int, y, bits: int,
                    norm_w=None, eps: float = 1e-5, stream=None) -> None:
    n, d = h_in.shape
    _check(LIB.rsq_layer_fused(_ptr(h_in), _ptr(h_out), _dtype_code(h_in), n, d, _ptr(site), r, _ptr(norm_w), eps,
                               bits, _ptr(codes), _ptr(scales), _ptr(w_codes), _ptr(w_scales), n_out, _ptr(y),
                               _dtype_code(y), _stream(stream)), "rsq_layer_fused")
