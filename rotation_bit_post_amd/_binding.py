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
RSQ_ROTATE_RIGHT, RSQ_ROTATE_LEFT = 0, 1


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
        "rsq_qgemm_workspace_bytes": (sz, [i64, i64, i64, i32]),
        "rsq_correct_workspace_bytes": (sz, [i64, i64]),
        "rsq_layer_workspace_bytes": (sz, [i64, i64, i64, i32]),
        "rsq_correct_quant": (i32, [vp, vp, i32, i64, i64, vp, i32, vp, f32, i32, vp, vp, vp, sz, vp]),
        "rsq_qgemm": (i32, [vp, vp, i64, vp, vp, i64, i64, i32, vp, i32, i64, vp, vp, sz, vp]),
        "rsq_qgemm_residual": (i32, [vp, vp, i64, vp, vp, i64, i64, i32, vp, i64, vp, i32, i64, vp, sz, vp]),
        "rsq_layer_fused": (i32, [vp, vp, i32, i64, i64, vp, i32, vp, f32, i32, vp, vp, vp, vp, i64, vp, i32, vp, sz,
                                  vp]),
        "rsq_codes_to_fp4": (i32, [vp, i64, i64, vp, vp]),
        "rsq_rotate_weight": (i32, [vp, i64, i64, vp, i32, vp, vp]),
        "rsq_qgemm_fp4": (i32, [vp, vp, i64, vp, vp, i64, i64, vp, i64, vp, i32, i64, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


LIB = _load()
EXPORTS = ("rsq_version", "rsq_status_str", "rsq_last_error", "rsq_packed_row_bytes", "rsq_site_bytes",
           "rsq_qgemm_workspace_bytes", "rsq_correct_workspace_bytes", "rsq_layer_workspace_bytes",
           "rsq_site_prepare", "rsq_subspace_correct", "rsq_quant_act", "rsq_correct_quant", "rsq_qgemm", "rsq_qgemm_residual",
           "rsq_layer_fused", "rsq_codes_to_fp4", "rsq_qgemm_fp4", "rsq_rotate_weight")


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


# ------------------------------------------------------ argument checks
# The C ABI takes raw pointers, sizes and row strides; these checks make sure
# that what a tensor holds matches what the call is told, before the call.
# Every check raises ValueError and runs before anything is enqueued; the
# last one is that every tensor lives on the GPU.
def _req(cond, msg):
    if not cond:
        raise ValueError(msg)


def _rows(name, t, n=None, k=None):
    """A 2-D tensor of rows with unit column stride (n rows, k columns if given)."""
    _req(t is not None and t.dim() == 2, f"{name} must be a 2-D tensor")
    _req(t.stride(1) == 1 or t.shape[1] <= 1, f"{name} must have unit column stride")
    if n is not None:
        _req(t.shape[0] == n, f"{name} has {t.shape[0]} rows, expected {n}")
    if k is not None:
        _req(t.shape[1] == k, f"{name} has {t.shape[1]} columns, expected {k}")


def _buffer(name, t, nbytes, dtype=None):
    """A contiguous tensor of at least nbytes bytes (and of the given dtype)."""
    import torch
    _req(t is not None, f"{name} is missing")
    if dtype is not None:
        _req(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _req(t.is_contiguous(), f"{name} must be contiguous")
    _req(t.numel() * t.element_size() >= nbytes, f"{name} holds {t.numel() * t.element_size()} bytes, "
                                                  f"{nbytes} needed")
    del torch


def _same_layout(a_name, a, b_name, b):
    _req(a.dtype == b.dtype, f"{b_name} must have {a_name}'s dtype ({a.dtype}), got {b.dtype}")
    _req(tuple(a.shape) == tuple(b.shape), f"{b_name} must have {a_name}'s shape {tuple(a.shape)}, got {tuple(b.shape)}")
    _req(a.stride() == b.stride(), f"{b_name} must have {a_name}'s strides {a.stride()}, got {b.stride()}")


def _on_device(**tensors):
    for name, t in tensors.items():
        if t is not None and not isinstance(t, int):
            _req(t.is_cuda, f"{name} must be a device tensor")


def _codes_scales(n, k, bits, codes, scales):
    import torch
    rb = LIB.rsq_packed_row_bytes(k, bits)
    _req(rb > 0, f"no packed layout for k = {k}, bits = {bits}")
    _buffer("codes", codes, n * rb, torch.uint8)
    _buffer("scales", scales, 4 * n, torch.float32)
    return rb


def _norm_weight(norm_w, k):
    import torch
    if norm_w is not None:
        _buffer("norm_w", norm_w, 4 * k, torch.float32)


# -------------------------------------------------------------- workspace
_DEFAULT_WS = {}


def rsq_workspace(nbytes: int, device=None):
    """A zero-filled device workspace of at least nbytes bytes (see include/rsq.h)."""
    import torch
    return torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=device or "cuda")


def _workspace_arg(workspace):
    if workspace is not None:
        import torch
        _req(workspace.dtype == torch.uint8 and workspace.is_contiguous(), "workspace must be contiguous uint8")


def _workspace(workspace, need: int):
    """(pointer, bytes) of the workspace a call passes. With workspace=None a
    zero-filled buffer kept per device is used (grown when a call needs more);
    calls that use it must run on one stream, as for any shared workspace."""
    if workspace is not None:
        return workspace.data_ptr(), workspace.numel()
    if need == 0:
        return None, 0
    import torch
    dev = torch.cuda.current_device()
    ws = _DEFAULT_WS.get(dev)
    if ws is None or ws.numel() < need:
        ws = rsq_workspace(max(need, 1 << 20))
        _DEFAULT_WS[dev] = ws
    return ws.data_ptr(), ws.numel()


# ----------------------------------------------------------------- queries
def rsq_version() -> int:
    return LIB.rsq_version()


def rsq_packed_row_bytes(k: int, bits: int) -> int:
    return LIB.rsq_packed_row_bytes(k, bits)


def rsq_site_bytes(d: int, r: int) -> int:
    return LIB.rsq_site_bytes(d, r)


def rsq_qgemm_workspace_bytes(n: int, n_out: int, k: int, bits: int) -> int:
    return LIB.rsq_qgemm_workspace_bytes(n, n_out, k, bits)


def rsq_correct_workspace_bytes(n: int, d: int) -> int:
    return LIB.rsq_correct_workspace_bytes(n, d)


def rsq_layer_workspace_bytes(n: int, d: int, n_out: int, bits: int) -> int:
    return LIB.rsq_layer_workspace_bytes(n, d, n_out, bits)


# ---------------------------------------------------------------- compute
def rsq_site_prepare(U, M, site, stream=None) -> None:
    """U: (d, r) float32, M: (r, r) float32, site: uint8 buffer of rsq_site_bytes(d, r)."""
    import torch
    _rows("U", U)
    d, r = U.shape
    _buffer("U", U, 4 * d * r, torch.float32)
    _buffer("M", M, 4 * r * r, torch.float32)
    _buffer("site", site, LIB.rsq_site_bytes(d, r), torch.uint8)
    _on_device(U=U, M=M, site=site)
    _check(LIB.rsq_site_prepare(_ptr(U), _ptr(M), d, r, _ptr(site), _stream(stream)), "rsq_site_prepare")


def rsq_subspace_correct(h_in, h_out, site, r: int, stream=None) -> None:
    """h_out = h_in + ((h_in U) M) U^T per row; h_in, h_out: (n, d) with the same dtype and row stride."""
    _rows("h_in", h_in)
    _rows("h_out", h_out)
    _same_layout("h_in", h_in, "h_out", h_out)
    n, d = h_in.shape
    _buffer("site", site, LIB.rsq_site_bytes(d, r))
    _on_device(h_in=h_in, h_out=h_out, site=site)
    _check(LIB.rsq_subspace_correct(_ptr(h_in), _ptr(h_out), _dtype_code(h_in), n, d, h_in.stride(0),
                                    _ptr(site), r, _stream(stream)), "rsq_subspace_correct")


def rsq_quant_act(x, codes, scales, bits: int, rmsnorm: bool = False, norm_w=None, eps: float = 1e-5,
                  stream=None) -> None:
    _rows("x", x)
    n, k = x.shape
    _codes_scales(n, k, bits, codes, scales)
    _norm_weight(norm_w, k)
    _on_device(x=x, codes=codes, scales=scales, norm_w=norm_w)
    flags = RSQ_QA_RMSNORM if rmsnorm else 0
    _check(LIB.rsq_quant_act(_ptr(x), _dtype_code(x), n, k, x.stride(0), flags, _ptr(norm_w), eps, bits,
                             _ptr(codes), _ptr(scales), _stream(stream)), "rsq_quant_act")


def rsq_correct_quant(h_in, h_out, site, r: int, codes, scales, bits: int, norm_w=None, eps: float = 1e-5,
                      workspace=None, stream=None) -> None:
    """Correction + RMSNorm + quantisation; h_in and h_out contiguous (n, d) of one dtype."""
    _rows("h_in", h_in)
    _req(h_in.is_contiguous(), "h_in must be contiguous (rsq_correct_quant takes no row stride)")
    _same_layout("h_in", h_in, "h_out", h_out)
    n, d = h_in.shape
    _buffer("site", site, LIB.rsq_site_bytes(d, r))
    _codes_scales(n, d, bits, codes, scales)
    _norm_weight(norm_w, d)
    _workspace_arg(workspace)
    _on_device(h_in=h_in, h_out=h_out, site=site, codes=codes, scales=scales, norm_w=norm_w, workspace=workspace)
    ws, ws_bytes = _workspace(workspace, LIB.rsq_correct_workspace_bytes(n, d))
    _check(LIB.rsq_correct_quant(_ptr(h_in), _ptr(h_out), _dtype_code(h_in), n, d, _ptr(site), r, _ptr(norm_w),
                                 eps, bits, _ptr(codes), _ptr(scales), ws, ws_bytes, _stream(stream)),
           "rsq_correct_quant")


def _gemm_operands(a_codes, a_scales, n, w_codes, w_scales, n_out, k, bits, y):
    import torch
    rb = LIB.rsq_packed_row_bytes(k, bits)
    _req(rb > 0, f"no packed layout for k = {k}, bits = {bits}")
    _buffer("a_codes", a_codes, n * rb, torch.uint8)
    _buffer("a_scales", a_scales, 4 * n, torch.float32)
    _buffer("w_codes", w_codes, n_out * rb, torch.uint8)
    _buffer("w_scales", w_scales, 4 * n_out, torch.float32)
    _rows("y", y)
    _req(y.shape[0] >= n and y.shape[1] >= n_out, f"y of shape {tuple(y.shape)} cannot hold {n} x {n_out}")


def rsq_qgemm(a_codes, a_scales, n: int, w_codes, w_scales, n_out: int, k: int, bits: int, y, acc_out=None,
              workspace=None, stream=None) -> None:
    import torch
    _gemm_operands(a_codes, a_scales, n, w_codes, w_scales, n_out, k, bits, y)
    if acc_out is not None:
        _buffer("acc_out", acc_out, 4 * n * n_out, torch.int32)
    _workspace_arg(workspace)
    _on_device(a_codes=a_codes, a_scales=a_scales, w_codes=w_codes, w_scales=w_scales, y=y, acc_out=acc_out,
               workspace=workspace)
    ws, ws_bytes = _workspace(workspace, LIB.rsq_qgemm_workspace_bytes(n, n_out, k, bits))
    _check(LIB.rsq_qgemm(_ptr(a_codes), _ptr(a_scales), n, _ptr(w_codes), _ptr(w_scales), n_out, k, bits,
                         _ptr(y), _dtype_code(y), y.stride(0), _ptr(acc_out), ws, ws_bytes, _stream(stream)),
           "rsq_qgemm")


def _residual(residual, y, n, n_out):
    _rows("residual", residual)
    _req(residual.dtype == y.dtype, "residual and y must have the same dtype")
    _req(residual.shape[0] >= n and residual.shape[1] >= n_out,
         f"residual of shape {tuple(residual.shape)} cannot hold {n} x {n_out}")


def rsq_qgemm_residual(a_codes, a_scales, n: int, w_codes, w_scales, n_out: int, k: int, bits: int, residual, y,
                       workspace=None, stream=None) -> None:
    """y = dequantised quantised linear + residual (residual may be y itself)."""
    _gemm_operands(a_codes, a_scales, n, w_codes, w_scales, n_out, k, bits, y)
    _residual(residual, y, n, n_out)
    _workspace_arg(workspace)
    _on_device(a_codes=a_codes, a_scales=a_scales, w_codes=w_codes, w_scales=w_scales, y=y, residual=residual,
               workspace=workspace)
    ws, ws_bytes = _workspace(workspace, LIB.rsq_qgemm_workspace_bytes(n, n_out, k, bits))
    _check(LIB.rsq_qgemm_residual(_ptr(a_codes), _ptr(a_scales), n, _ptr(w_codes), _ptr(w_scales), n_out, k, bits,
                                  _ptr(residual), residual.stride(0), _ptr(y), _dtype_code(y), y.stride(0),
                                  ws, ws_bytes, _stream(stream)), "rsq_qgemm_residual")


def rsq_codes_to_fp4(codes, rows: int, k: int, fp4, stream=None) -> None:
    """Packed int3 rows -> fp4 rows (k / 2 bytes each), the same code values."""
    import torch
    _buffer("codes", codes, rows * LIB.rsq_packed_row_bytes(k, 3), torch.uint8)
    _buffer("fp4", fp4, rows * (k // 2), torch.uint8)
    _on_device(codes=codes, fp4=fp4)
    _check(LIB.rsq_codes_to_fp4(_ptr(codes), rows, k, _ptr(fp4), _stream(stream)), "rsq_codes_to_fp4")


def rsq_qgemm_fp4(a_fp4, a_scales, n: int, w_fp4, w_scales, n_out: int, k: int, y, residual=None, acc_out=None,
                  workspace=None, stream=None) -> None:
    """The 3-bit quantised linear on fp4 codes; residual (optional) may be y itself."""
    import torch
    _gemm_operands(a_fp4, a_scales, n, w_fp4, w_scales, n_out, k, 3 | RSQ_FP4, y)
    if residual is not None:
        _residual(residual, y, n, n_out)
    if acc_out is not None:
        _buffer("acc_out", acc_out, 4 * n * n_out, torch.int32)
    _workspace_arg(workspace)
    _on_device(a_fp4=a_fp4, a_scales=a_scales, w_fp4=w_fp4, w_scales=w_scales, y=y, residual=residual,
               acc_out=acc_out, workspace=workspace)
    ws, ws_bytes = _workspace(workspace, LIB.rsq_qgemm_workspace_bytes(n, n_out, k, 3 | RSQ_FP4))
    _check(LIB.rsq_qgemm_fp4(_ptr(a_fp4), _ptr(a_scales), n, _ptr(w_fp4), _ptr(w_scales), n_out, k, _ptr(residual),
                             residual.stride(0) if residual is not None else 0, _ptr(y), _dtype_code(y), y.stride(0),
                             _ptr(acc_out), ws, ws_bytes, _stream(stream)), "rsq_qgemm_fp4")


def rsq_layer_fused(h_in, h_out, site, r: int, codes, scales, w_codes, w_scales, n_out: int, y, bits: int,
                    norm_w=None, eps: float = 1e-5, workspace=None, stream=None) -> None:
    """One site and its linear: h_in, h_out contiguous (n, d); y contiguous (n, n_out)."""
    import torch
    _rows("h_in", h_in)
    _req(h_in.is_contiguous(), "h_in must be contiguous (rsq_layer_fused takes no row stride)")
    _same_layout("h_in", h_in, "h_out", h_out)
    n, d = h_in.shape
    _buffer("site", site, LIB.rsq_site_bytes(d, r))
    rb = _codes_scales(n, d, bits, codes, scales)
    _norm_weight(norm_w, d)
    _buffer("w_codes", w_codes, n_out * rb, torch.uint8)
    _buffer("w_scales", w_scales, 4 * n_out, torch.float32)
    _rows("y", y, n, n_out)
    _req(y.is_contiguous(), "y must be contiguous (rsq_layer_fused writes rows of n_out)")
    _workspace_arg(workspace)
    _on_device(h_in=h_in, h_out=h_out, site=site, codes=codes, scales=scales, w_codes=w_codes, w_scales=w_scales,
               y=y, norm_w=norm_w, workspace=workspace)
    ws, ws_bytes = _workspace(workspace, LIB.rsq_layer_workspace_bytes(n, d, n_out, bits))
    _check(LIB.rsq_layer_fused(_ptr(h_in), _ptr(h_out), _dtype_code(h_in), n, d, _ptr(site), r, _ptr(norm_w), eps,
                               bits, _ptr(codes), _ptr(scales), _ptr(w_codes), _ptr(w_scales), n_out, _ptr(y),
                               _dtype_code(y), ws, ws_bytes, _stream(stream)), "rsq_layer_fused")


def rsq_rotate_weight(w, r, side: int, out, stream=None) -> None:
    """Offline weight fusion: out = w r (side RSQ_ROTATE_RIGHT, r: k x k) or out = r^T w
    (RSQ_ROTATE_LEFT, r: n x n); w, out: (n, k) float32, contiguous."""
    import torch
    _rows("w", w)
    n, k = w.shape
    _req(side in (RSQ_ROTATE_RIGHT, RSQ_ROTATE_LEFT), f"side = {side} is not RSQ_ROTATE_RIGHT or RSQ_ROTATE_LEFT")
    rd = k if side == RSQ_ROTATE_RIGHT else n
    _buffer("w", w, 4 * n * k, torch.float32)
    _rows("r", r, rd, rd)
    _buffer("r", r, 4 * rd * rd, torch.float32)
    _rows("out", out, n, k)
    _buffer("out", out, 4 * n * k, torch.float32)
    _on_device(w=w, r=r, out=out)
    _check(LIB.rsq_rotate_weight(_ptr(w), n, k, _ptr(r), side, _ptr(out), _stream(stream)), "rsq_rotate_weight")
