"""Python binding of libslope.so, the SLoPe 2:4 sparse linear layer for MI355X.

Argument marshalling only: every function below checks that its tensors are
contiguous device tensors, reads their shapes and dtypes, and calls the C ABI
function of the same name (declared in include/slope.h) on the current HIP
stream.  All computation happens in the library's HIP kernels; there is no
fallback.  If the shared library has not been built, every call raises.

Tensor conventions (see include/slope.h):
  dense matrices      torch.bfloat16, torch.float16 or torch.float32, row-major
  masks               torch.uint8, 1 = kept
  compressed values   [rows, cols/2], same dtype as the dense matrix
  compressed metadata [rows, ceil(cols/32)] torch.int32 holding the uint32 words
  adapter workspace   torch.uint8 (or any dtype) of slope_lowrank_workspace_bytes()
  wgrad workspace     torch.uint8 (or any dtype) of slope_wgrad_workspace_bytes()
  packed operands     torch.uint8 buffers of slope_packed_sparse_bytes() (sparse
                      tile chunks) or slope_packed_tokens_bytes() (token chunks)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "SlopeError", "library", "library_path", "STATUS",
    "slope_version", "slope_compressed_sizes", "slope_lowrank_workspace_bytes",
    "slope_prune24", "slope_prune_nm", "slope_compress24", "slope_double_prune", "slope_spmm_fwd",
    "slope_spmm_bwd_dx", "slope_masked_wgrad", "slope_lowrank_add", "slope_wgrad_workspace_bytes",
    "slope_packed_tokens_bytes", "slope_pack_tokens", "slope_masked_wgrad_packed", "slope_wgrad_split_workspace_bytes",
    "slope_packed_sparse_bytes", "slope_pack_sparse", "slope_spmm_fwd_packed", "slope_spmm_bwd_dx_packed",
    "slope_spmm_fwd_packed_tokens", "slope_spmm_bwd_dx_packed_tokens",
    "slope_decode_workspace_bytes", "slope_spmm_fwd_decode", "slope_spmm_fwd_decode_noalloc",
    "DECODE_NOALLOC_SCRATCH_BYTES", "slope_lowrank_grads_workspace_bytes",
    "slope_lowrank_grads_packed", "slope_adamw", "slope_adamw_double_prune", "AdamWParams",
    "slope_double_prune_packed", "slope_adamw_double_prune_packed", "slope_prune_compress24", "EXPORTED_SYMBOLS",
    "slope_quantize_e4m3", "slope_packed_sparse_e4m3_bytes", "slope_pack_sparse_e4m3", "slope_spmm_e4m3_packed",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libslope.so")

STATUS = {0: "SLOPE_OK", -1: "SLOPE_ERR_INVALID_ARG", -2: "SLOPE_ERR_SHAPE", -3: "SLOPE_ERR_ALIGN",
          -4: "SLOPE_ERR_WORKSPACE", -5: "SLOPE_ERR_HIP", -6: "SLOPE_ERR_UNSUPPORTED"}

_F32, _BF16, _F16 = 0, 1, 2
_i64, _vp, _i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
_P_I64 = ctypes.POINTER(ctypes.c_int64)


class AdamWParams(ctypes.Structure):
    """slope_adamw_params: hyper-parameters of one AdamW update (step counts from 1)."""
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("step", ctypes.c_int64)]


_P_HP = ctypes.POINTER(AdamWParams)

# name -> (restype, argtypes)
_SIGS = {
    "slope_version": (ctypes.c_int, []),
    "slope_status_string": (ctypes.c_char_p, [_i32]),
    "slope_compressed_sizes": (_i32, [_i64, _i64, _P_I64, _P_I64]),
    "slope_lowrank_workspace_bytes": (_i32, [_i64, _i64, _i64, _i64, _P_I64]),
    "slope_prune24": (_i32, [_i32, _vp, _i64, _i64, _vp, _vp, _vp]),
    "slope_compress24": (_i32, [_i32, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "slope_double_prune": (_i32, [_i32, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "slope_spmm_fwd": (_i32, [_i32, _i32, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _vp, _vp]),
    "slope_spmm_bwd_dx": (_i32, [_i32, _i32, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp]),
    "slope_masked_wgrad": (_i32, [_i32, _i32, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _vp, _i32, _vp, _i64, _vp]),
    "slope_wgrad_workspace_bytes": (_i32, [_i64, _i64, _i64, _P_I64]),
    "slope_packed_tokens_bytes": (_i32, [_i64, _i64, _P_I64]),
    "slope_packed_sparse_bytes": (_i32, [_i64, _i64, _P_I64]),
    "slope_decode_workspace_bytes": (_i32, [_i64, _i64, _i64, _i64, _P_I64]),
    "slope_spmm_fwd_decode": (_i32, [_i32, _i32, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _vp,
                                     _vp]),
    "slope_spmm_fwd_decode_noalloc": (_i32, [_i32, _i32, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _vp,
                                             _vp]),
    "slope_pack_sparse": (_i32, [_i32, _vp, _vp, _i64, _i64, _vp, _i64, _vp]),
    "slope_spmm_fwd_packed": (_i32, [_i32, _i32, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _vp,
                                     _vp]),
    "slope_spmm_bwd_dx_packed": (_i32, [_i32, _i32, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _i64,
                                        _vp, _vp]),
    "slope_spmm_fwd_packed_tokens": (_i32, [_i32, _i32, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _vp,
                                            _i64, _vp, _vp, _i64, _vp]),
    "slope_spmm_bwd_dx_packed_tokens": (_i32, [_i32, _i32, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _vp,
                                               _i64, _vp, _vp, _i64, _vp]),
    "slope_lowrank_grads_workspace_bytes": (_i32, [_i64, _i64, _i64, _i64, _P_I64]),
    "slope_lowrank_grads_packed": (_i32, [_i32, _i32, _vp, _vp, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _vp,
                                          _vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i32, _vp]),
    "slope_pack_tokens": (_i32, [_i32, _vp, _i64, _i64, _vp, _i64, _vp]),
    "slope_masked_wgrad_packed": (_i32, [_i32, _i32, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _i32,
                                         _vp, _i64, _vp]),
    "slope_wgrad_split_workspace_bytes": (_i32, [_i64, _i64, _i64, _P_I64]),
    "slope_lowrank_add": (_i32, [_i32, _i32, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _vp]),
    "slope_adamw": (_i32, [_i32, _i32, _vp, _vp, _vp, _vp, _i64, _P_HP, _vp]),
    "slope_adamw_double_prune": (_i32, [_i32, _i32, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _P_HP, _vp, _vp, _vp,
                                        _vp]),
    "slope_double_prune_packed": (_i32, [_i32, _vp, _vp, _i64, _i64, _vp, _i64, _vp]),
    "slope_prune_compress24": (_i32, [_i32, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _vp]),
    "slope_prune_nm": (_i32, [_i32, _vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp]),
    "slope_adamw_double_prune_packed": (_i32, [_i32, _i32, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _P_HP, _vp, _i64,
                                               _vp, _i64, _vp]),
    "slope_quantize_e4m3": (_i32, [_i32, _vp, _i64, _vp, _vp, _vp]),
    "slope_packed_sparse_e4m3_bytes": (_i32, [_i64, _i64, _P_I64]),
    "slope_pack_sparse_e4m3": (_i32, [_i32, _vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp]),
    "slope_spmm_e4m3_packed": (_i32, [_i32, _vp, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp]),
}
EXPORTED_SYMBOLS = tuple(_SIGS)

_lib = None


class SlopeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({_status_text(status)})")


def library() -> ctypes.CDLL:
    """The loaded libslope.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it first "
                               "(python -m sparse_gemm_02_amd.build); there is no fallback path")
        lib = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            f = getattr(lib, name)
            f.restype, f.argtypes = res, args
        _lib = lib
    return _lib


def _status_text(status: int) -> str:
    try:
        return library().slope_status_string(status).decode()
    except Exception:  # pragma: no cover - library missing
        return "?"


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise SlopeError(fn, status)


def _dt(t) -> int:
    """Library dtype code of a tensor (or of a torch dtype)."""
    d = t if isinstance(t, torch.dtype) else t.dtype
    if d == torch.bfloat16:
        return _BF16
    if d == torch.float16:
        return _F16
    if d == torch.float32:
        return _F32
    raise TypeError(f"expected bfloat16, float16 or float32, got {d}")


def _p(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if t.numel() and not t.is_cuda:
        raise ValueError("tensors must live in GPU memory")
    return t.data_ptr() if t.numel() else None


def _nn(t):
    """Pointer of a required tensor (a dummy non-null address for empty ones)."""
    p = _p(t)
    return p if p is not None else 256  # never dereferenced: the size is zero


def _adapter(L, R):
    """(L pointer, R pointer, r) of the adapter arguments.  Factors with no
    elements (K, N or r zero) make the adapter term zero and go as two NULLs; a
    single factor goes through as given, for the library to reject."""
    if L is None and R is None:
        return None, None, 0
    r = int(L.shape[1]) if L is not None else int(R.shape[0])
    if L is not None and R is not None and (L.numel() == 0 or R.numel() == 0):
        return None, None, r
    return _p(L), _p(R), r


def _nb(t):
    """Bytes of a buffer tensor (0 for None)."""
    return t.numel() * t.element_size() if t is not None else 0


def _s(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def slope_version() -> int:
    return library().slope_version()


def slope_compressed_sizes(rows: int, cols: int):
    nv, nm = ctypes.c_int64(), ctypes.c_int64()
    _check("slope_compressed_sizes", library().slope_compressed_sizes(rows, cols, ctypes.byref(nv), ctypes.byref(nm)))
    return nv.value, nm.value


def slope_lowrank_workspace_bytes(T: int, K: int, r: int, N: int) -> int:
    b = ctypes.c_int64()
    _check("slope_lowrank_workspace_bytes", library().slope_lowrank_workspace_bytes(T, K, r, N, ctypes.byref(b)))
    return b.value


def slope_prune24(W, mask, W_s=None, stream=None) -> None:
    rows, cols = W.shape
    _check("slope_prune24", library().slope_prune24(_dt(W), _nn(W), rows, cols, _nn(mask), _p(W_s), _s(stream)))


def slope_prune_nm(W, n, m, mask, W_s=None, stream=None) -> None:
    rows, cols = W.shape
    _check("slope_prune_nm", library().slope_prune_nm(_dt(W), _nn(W), rows, cols, n, m, _nn(mask), _p(W_s),
                                                      _s(stream)))


def slope_compress24(W, mask, values, meta, invalid=None, stream=None) -> None:
    rows, cols = W.shape
    _check("slope_compress24", library().slope_compress24(_dt(W), _nn(W), _nn(mask), rows, cols, _nn(values),
                                                          _nn(meta), _p(invalid), _s(stream)))


def slope_double_prune(values_s, meta_s, N, K, values_dpT, meta_dpT, mask_dpT=None, stream=None) -> None:
    _check("slope_double_prune", library().slope_double_prune(_dt(values_s), _nn(values_s), _nn(meta_s), N, K,
                                                              _nn(values_dpT), _nn(meta_dpT), _p(mask_dpT),
                                                              _s(stream)))


def slope_spmm_fwd(X, values_s, meta_s, N, Y, L=None, R=None, workspace=None, stream=None) -> None:
    T, K = X.shape
    pl, pr, r = _adapter(L, R)
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("slope_spmm_fwd", library().slope_spmm_fwd(_dt(X), _dt(Y), _nn(X), T, K, _nn(values_s), _nn(meta_s), N,
                                                      pl, pr, r, _p(workspace), wb, _nn(Y), _s(stream)))


def slope_spmm_bwd_dx(dY, values_dpT, meta_dpT, K, dX, stream=None) -> None:
    T, N = dY.shape
    _check("slope_spmm_bwd_dx", library().slope_spmm_bwd_dx(_dt(dY), _dt(dX), _nn(dY), T, N, _nn(values_dpT),
                                                            _nn(meta_dpT), K, _nn(dX), _s(stream)))


def slope_wgrad_workspace_bytes(T: int, N: int, K: int) -> int:
    b = ctypes.c_int64()
    _check("slope_wgrad_workspace_bytes", library().slope_wgrad_workspace_bytes(T, N, K, ctypes.byref(b)))
    return b.value


def slope_masked_wgrad(dY, X, meta_s, dW_values, dW_dense=None, accumulate=False, workspace=None,
                       stream=None) -> None:
    T, N = dY.shape
    K = X.shape[1]
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("slope_masked_wgrad", library().slope_masked_wgrad(_dt(dY), _dt(dW_values), _nn(dY), _nn(X), T, N, K,
                                                              _nn(meta_s), _nn(dW_values), _p(dW_dense),
                                                              int(bool(accumulate)), _p(workspace), wb,
                                                              _s(stream)))


def slope_packed_sparse_bytes(rows: int, cols: int) -> int:
    b = ctypes.c_int64()
    _check("slope_packed_sparse_bytes", library().slope_packed_sparse_bytes(rows, cols, ctypes.byref(b)))
    return b.value


def slope_pack_sparse(values, meta, rows, cols, packed, stream=None) -> None:
    nb = packed.numel() * packed.element_size()
    _check("slope_pack_sparse", library().slope_pack_sparse(_dt(values), _nn(values), _nn(meta), rows, cols,
                                                            _nn(packed), nb, _s(stream)))


def slope_spmm_fwd_packed(X, packed_s, N, Y, L=None, R=None, workspace=None, stream=None) -> None:
    T, K = X.shape
    pl, pr, r = _adapter(L, R)
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("slope_spmm_fwd_packed", library().slope_spmm_fwd_packed(_dt(X), _dt(Y), _nn(X), T, K, _nn(packed_s),
                                                                    _nb(packed_s), N, pl, pr, r, _p(workspace),
                                                                    wb, _nn(Y), _s(stream)))


def slope_spmm_fwd_packed_tokens(X, packed_s, N, Y, X_packed, L=None, R=None, workspace=None, stream=None) -> None:
    T, K = X.shape
    pl, pr, r = _adapter(L, R)
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("slope_spmm_fwd_packed_tokens",
           library().slope_spmm_fwd_packed_tokens(_dt(X), _dt(Y), _nn(X), T, K, _nn(packed_s), _nb(packed_s), N, pl,
                                                  pr, r, _p(workspace), wb, _nn(Y), _nn(X_packed), _nb(X_packed),
                                                  _s(stream)))


def slope_decode_workspace_bytes(T: int, K: int, r: int, N: int) -> int:
    b = ctypes.c_int64()
    _check("slope_decode_workspace_bytes", library().slope_decode_workspace_bytes(T, K, r, N, ctypes.byref(b)))
    return b.value


def slope_spmm_fwd_decode(X, packed_s, N, Y, workspace, L=None, R=None, stream=None) -> None:
    T, K = X.shape
    pl, pr, r = _adapter(L, R)
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("slope_spmm_fwd_decode", library().slope_spmm_fwd_decode(_dt(X), _dt(Y), _nn(X), T, K, _nn(packed_s),
                                                                    _nb(packed_s), N, pl, pr, r, _p(workspace),
                                                                    wb, _nn(Y), _s(stream)))


DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20   # SLOPE_DECODE_NOALLOC_SCRATCH_BYTES


def slope_spmm_fwd_decode_noalloc(X, packed_s, N, Y, L=None, R=None, stream=None) -> None:
    """slope_spmm_fwd_decode without a workspace: the library's static scratch."""
    T, K = X.shape
    pl, pr, r = _adapter(L, R)
    _check("slope_spmm_fwd_decode_noalloc", library().slope_spmm_fwd_decode_noalloc(
        _dt(X), _dt(Y), _nn(X), T, K, _nn(packed_s), _nb(packed_s), N, pl, pr, r, _nn(Y), _s(stream)))


def slope_spmm_bwd_dx_packed(dY, packed_dpT, K, dX, L=None, R=None, workspace=None, stream=None) -> None:
    T, N = dY.shape
    pl, pr, r = _adapter(L, R)
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("slope_spmm_bwd_dx_packed", library().slope_spmm_bwd_dx_packed(_dt(dY), _dt(dX), _nn(dY), T, N,
                                                                          _nn(packed_dpT), _nb(packed_dpT), K, pl,
                                                                          pr, r, _p(workspace), wb, _nn(dX),
                                                                          _s(stream)))


def slope_spmm_bwd_dx_packed_tokens(dY, packed_dpT, K, dX, dY_packed, L=None, R=None, workspace=None,
                                    stream=None) -> None:
    T, N = dY.shape
    pl, pr, r = _adapter(L, R)
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("slope_spmm_bwd_dx_packed_tokens",
           library().slope_spmm_bwd_dx_packed_tokens(_dt(dY), _dt(dX), _nn(dY), T, N, _nn(packed_dpT),
                                                     _nb(packed_dpT), K, pl, pr, r, _p(workspace), wb, _nn(dX),
                                                     _nn(dY_packed), _nb(dY_packed), _s(stream)))


def slope_lowrank_grads_workspace_bytes(T: int, K: int, r: int, N: int) -> int:
    b = ctypes.c_int64()
    _check("slope_lowrank_grads_workspace_bytes",
           library().slope_lowrank_grads_workspace_bytes(T, K, r, N, ctypes.byref(b)))
    return b.value


def slope_lowrank_grads_packed(X, dY, X_packed, dY_packed, L, R, workspace, dL, dR, accumulate=False,
                               fwd_workspace=None, bwd_workspace=None, stream=None) -> None:
    T, K = X.shape
    N = dY.shape[1]
    r = int(L.shape[1])
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("slope_lowrank_grads_packed", library().slope_lowrank_grads_packed(
        _dt(X), _dt(dL), _nn(X), _nn(dY), _nn(X_packed), _nb(X_packed), _nn(dY_packed), _nb(dY_packed), T, K, r, N,
        _nn(L), _nn(R), _p(fwd_workspace), _nb(fwd_workspace), _p(bwd_workspace), _nb(bwd_workspace), _p(workspace),
        wb, _nn(dL), _nn(dR), int(bool(accumulate)), _s(stream)))


def slope_packed_tokens_bytes(T: int, C: int) -> int:
    b = ctypes.c_int64()
    _check("slope_packed_tokens_bytes", library().slope_packed_tokens_bytes(T, C, ctypes.byref(b)))
    return b.value


def slope_pack_tokens(M, packed, stream=None) -> None:
    T, C = M.shape
    nb = packed.numel() * packed.element_size()
    _check("slope_pack_tokens", library().slope_pack_tokens(_dt(M), _nn(M), T, C, _nn(packed), nb, _s(stream)))


def slope_wgrad_split_workspace_bytes(T: int, N: int, K: int) -> int:
    b = ctypes.c_int64()
    _check("slope_wgrad_split_workspace_bytes", library().slope_wgrad_split_workspace_bytes(T, N, K, ctypes.byref(b)))
    return b.value


def slope_masked_wgrad_packed(dY_packed, X_packed, T, N, K, meta_s, dW_values, dW_dense=None, accumulate=False,
                              stream=None, in_dtype=None, split_workspace=None) -> None:
    """in_dtype: torch dtype the packed operands hold (the chunks do not record
    it); defaults to dW_values' dtype when that is 16-bit, else bfloat16.
    split_workspace: optional buffer of slope_wgrad_split_workspace_bytes()."""
    if in_dtype is None:
        in_dtype = dW_values.dtype if dW_values.dtype in (torch.bfloat16, torch.float16) else torch.bfloat16
    _check("slope_masked_wgrad_packed", library().slope_masked_wgrad_packed(
        _dt(in_dtype), _dt(dW_values), _nn(dY_packed), _nb(dY_packed), _nn(X_packed), _nb(X_packed), T, N, K,
        _nn(meta_s), _nn(dW_values), _p(dW_dense), int(bool(accumulate)), _p(split_workspace), _nb(split_workspace),
        _s(stream)))


def slope_lowrank_add(X, L, R, workspace, Y, stream=None) -> None:
    T, K = X.shape
    r, N = R.shape
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("slope_lowrank_add", library().slope_lowrank_add(_dt(X), _dt(Y), _nn(X), _nn(L), _nn(R), T, K, r, N,
                                                            _p(workspace), wb, _nn(Y), _s(stream)))


def _hp(step, lr, beta1, beta2, eps, weight_decay):
    return AdamWParams(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), int(step))


def _f32(t):
    if t.dtype != torch.float32:
        raise TypeError(f"optimizer moments must be float32, got {t.dtype}")
    return _nn(t)


def slope_adamw(params, grads, m, v, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
                stream=None) -> None:
    """One AdamW step on params (updated in place) with float32 moments m, v."""
    n = params.numel()
    if grads.numel() != n or m.numel() != n or v.numel() != n:
        raise ValueError("params, grads, m and v must have the same number of elements")
    hp = _hp(step, lr, beta1, beta2, eps, weight_decay)
    _check("slope_adamw", library().slope_adamw(_dt(params), _dt(grads), _nn(params), _nn(grads), _f32(m), _f32(v),
                                                n, ctypes.byref(hp), _s(stream)))


def slope_prune_compress24(W, values, meta, mask=None, packed=None, stream=None) -> None:
    """Magnitude 2:4 prune and compression of W [rows, cols] in one pass, with
    the mask and W_s's tile-chunk form as optional outputs."""
    rows, cols = W.shape
    nb = packed.numel() * packed.element_size() if packed is not None else 0
    _check("slope_prune_compress24", library().slope_prune_compress24(
        _dt(W), _nn(W), rows, cols, _p(mask), _nn(values), _nn(meta), _p(packed), nb, _s(stream)))


def slope_double_prune_packed(values_s, meta_s, N, K, packed_dpT, stream=None) -> None:
    """The double prune of W_s written straight to W_dp^T's tile-chunk form."""
    nb = packed_dpT.numel() * packed_dpT.element_size()
    _check("slope_double_prune_packed", library().slope_double_prune_packed(
        _dt(values_s), _nn(values_s), _nn(meta_s), N, K, _nn(packed_dpT), nb, _s(stream)))


def slope_adamw_double_prune_packed(values_s, meta_s, dW_values, m, v, N, K, packed_s, packed_dpT, step, lr,
                                    beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, stream=None) -> None:
    """AdamW on the compressed values of W_s (in place, and inside its tile
    chunks packed_s), then the double prune of the updated W_s into the tile
    chunks packed_dpT."""
    n = values_s.numel()
    if dW_values.numel() != n or m.numel() != n or v.numel() != n:
        raise ValueError("values_s, dW_values, m and v must have the same number of elements")
    hp = _hp(step, lr, beta1, beta2, eps, weight_decay)
    _check("slope_adamw_double_prune_packed", library().slope_adamw_double_prune_packed(
        _dt(values_s), _dt(dW_values), _nn(values_s), _nn(meta_s), _nn(dW_values), _f32(m), _f32(v), N, K,
        ctypes.byref(hp), _nn(packed_s), packed_s.numel() * packed_s.element_size(), _nn(packed_dpT),
        packed_dpT.numel() * packed_dpT.element_size(), _s(stream)))


def slope_adamw_double_prune(values_s, meta_s, dW_values, m, v, N, K, values_dpT, meta_dpT, step, lr, beta1=0.9,
                             beta2=0.999, eps=1e-8, weight_decay=0.01, mask_dpT=None, stream=None) -> None:
    """AdamW on the compressed values of W_s (in place), then the double prune of the updated W_s."""
    n = values_s.numel()
    if dW_values.numel() != n or m.numel() != n or v.numel() != n:
        raise ValueError("values_s, dW_values, m and v must have the same number of elements")
    hp = _hp(step, lr, beta1, beta2, eps, weight_decay)
    _check("slope_adamw_double_prune", library().slope_adamw_double_prune(
        _dt(values_s), _dt(dW_values), _nn(values_s), _nn(meta_s), _nn(dW_values), _f32(m), _f32(v), N, K,
        ctypes.byref(hp), _nn(values_dpT), _nn(meta_dpT), _p(mask_dpT), _s(stream)))



# ------------------------------------------------------------------ 8-bit (E4M3) variant
# Codes travel as torch.uint8 tensors; scales as one-element torch.float32 tensors.

def slope_quantize_e4m3(M, scale, q, stream=None) -> None:
    """scale[0] <- 448 / amax(|M|); q <- E4M3 codes of M * scale (same shape as M)."""
    if q.dtype != torch.uint8 or q.numel() != M.numel():
        raise ValueError("q must be a uint8 tensor with as many elements as M")
    if scale.dtype != torch.float32:
        raise TypeError("scale must be float32")
    _check("slope_quantize_e4m3", library().slope_quantize_e4m3(_dt(M), _nn(M), M.numel(), _nn(scale), _nn(q),
                                                                _s(stream)))


def slope_packed_sparse_e4m3_bytes(rows: int, cols: int) -> int:
    b = ctypes.c_int64()
    _check("slope_packed_sparse_e4m3_bytes", library().slope_packed_sparse_e4m3_bytes(rows, cols, ctypes.byref(b)))
    return b.value


def slope_pack_sparse_e4m3(values, meta, rows, cols, scale, packed, stream=None) -> None:
    """E4M3 tile chunks of a compressed 16-bit matrix, with its scale in scale[0]."""
    if scale.dtype != torch.float32:
        raise TypeError("scale must be float32")
    _check("slope_pack_sparse_e4m3", library().slope_pack_sparse_e4m3(_dt(values), _nn(values), _nn(meta), rows, cols,
                                                                      _nn(scale), _nn(packed), _nb(packed),
                                                                      _s(stream)))


def slope_spmm_e4m3_packed(Xq, x_scale, packed_w, w_scale, N, Y, stream=None) -> None:
    """Y [T, N] = (Xq . W_q^T) / (x_scale * w_scale) on E4M3 operands."""
    if Xq.dtype != torch.uint8:
        raise TypeError("Xq must hold uint8 E4M3 codes")
    T, K = Xq.shape
    _check("slope_spmm_e4m3_packed", library().slope_spmm_e4m3_packed(_dt(Y), _nn(Xq), _nn(x_scale), T, K,
                                                                      _nn(packed_w), _nb(packed_w), _nn(w_scale), N,
                                                                      _nn(Y), _s(stream)))
