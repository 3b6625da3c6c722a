"""ctypes binding of libfa_mi355x (include/fa_mi355x.h).

Argument marshalling only: every step of the attention computation runs in
the library's HIP kernels.  PyTorch supplies device memory and the stream.
The raw entry points keep the C names (fa_fwd, fa_fwd_strided, ...); `fwd`
is the tensor-level convenience wrapper the tests and the benchmark use.
"""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa_mi355x.so")

FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_DTYPE_F32, FA_DTYPE_BF16 = 0, 1
FA_MASK_NONE, FA_MASK_ADDITIVE, FA_MASK_BOOL = 0, 1, 2

EXPORTS = ("fa_fwd", "fa_fwd_strided", "fa_fwd_strided_noalloc", "fa_fwd_dropout", "fa_fwd_window", "fa_bwd",
           "fa_supported", "fa_bwd_supported", "fa_variant_count", "fa_variant_name", "fa_status_string",
           "fa_last_error", "fa_abi_version")


class FaError(RuntimeError):
    """A non-OK fa_status; `.status` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class FaStrides(ctypes.Structure):
    _fields_ = [("q", ctypes.c_int64 * 3), ("k", ctypes.c_int64 * 3), ("v", ctypes.c_int64 * 3),
                ("o", ctypes.c_int64 * 3), ("mask", ctypes.c_int64 * 3)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library once.  Raises if it has not been built: there is
    no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m flashattention_forward_04_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, i32, vp]
    lib.fa_fwd.restype = i32
    lib.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, i32,
                                   ctypes.POINTER(FaStrides), vp]
    lib.fa_fwd_strided.restype = i32
    lib.fa_fwd_strided_noalloc.argtypes = list(lib.fa_fwd_strided.argtypes)
    lib.fa_fwd_strided_noalloc.restype = i32
    lib.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, i32, f32,
                                   ctypes.c_uint64, ctypes.c_uint64, ctypes.POINTER(FaStrides), vp]
    lib.fa_fwd_dropout.restype = i32
    lib.fa_fwd_window.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, i32, i32,
                                  ctypes.POINTER(FaStrides), vp]
    lib.fa_fwd_window.restype = i32
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32,
                           i32, vp]
    lib.fa_bwd.restype = i32
    lib.fa_supported.argtypes = [i32, i32, i32, i32]
    lib.fa_supported.restype = i32
    lib.fa_bwd_supported.argtypes = [i32, i32, i32, i32]
    lib.fa_bwd_supported.restype = i32
    lib.fa_variant_count.restype = i32
    lib.fa_variant_name.argtypes = [i32]
    lib.fa_variant_name.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [i32]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_abi_version.restype = i32
    _lib = lib
    return lib


# ---- raw entry points, same names and arguments as the C ABI ----

def fa_fwd(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype, mask_kind, hip_stream) -> int:
    return load_library().fa_fwd(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype,
                                 mask_kind, hip_stream)


def fa_fwd_dropout(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype, mask_kind, p_drop, seed,
                   offset, strides, hip_stream) -> int:
    ref = ctypes.byref(strides) if strides is not None else None
    return load_library().fa_fwd_dropout(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype,
                                         mask_kind, p_drop, seed, offset, ref, hip_stream)


def fa_fwd_window(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype, mask_kind, window, strides,
                  hip_stream) -> int:
    ref = ctypes.byref(strides) if strides is not None else None
    return load_library().fa_fwd_window(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype,
                                        mask_kind, window, ref, hip_stream)


def fa_fwd_strided(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype, mask_kind, strides,
                   hip_stream) -> int:
    ref = ctypes.byref(strides) if strides is not None else None
    return load_library().fa_fwd_strided(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype,
                                         mask_kind, ref, hip_stream)


def fa_fwd_strided_noalloc(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype, mask_kind, strides,
                           hip_stream) -> int:
    ref = ctypes.byref(strides) if strides is not None else None
    return load_library().fa_fwd_strided_noalloc(Q, K, V, mask, O, L, B, H_q, H_kv, qL, kL, D, scale, causal, dtype,
                                                 mask_kind, ref, hip_stream)


def fa_bwd(Q, K, V, O, dO, L, mask, Delta, dQ, dK, dV, B, H_q, H_kv, qL, kL, D, scale, causal, dtype, mask_kind,
           hip_stream) -> int:
    return load_library().fa_bwd(Q, K, V, O, dO, L, mask, Delta, dQ, dK, dV, B, H_q, H_kv, qL, kL, D, scale, causal,
                                 dtype, mask_kind, hip_stream)


def fa_supported(dtype, D, mask_kind, causal) -> int:
    return load_library().fa_supported(dtype, D, mask_kind, causal)


def fa_bwd_supported(dtype, D, mask_kind, causal) -> int:
    return load_library().fa_bwd_supported(dtype, D, mask_kind, causal)


def fa_variant_count() -> int:
    return load_library().fa_variant_count()


def fa_variant_name(i) -> str | None:
    r = load_library().fa_variant_name(i)
    return None if r is None else r.decode()


def fa_status_string(s) -> str:
    return load_library().fa_status_string(s).decode()


def fa_last_error() -> str:
    return load_library().fa_last_error().decode()


def fa_abi_version() -> int:
    return load_library().fa_abi_version()


def check(status: int) -> None:
    if status != FA_OK:
        raise FaError(status, f"{fa_status_string(status)}: {fa_last_error()}")


# ---- tensor-level wrapper ----

def _strides3(t):
    s = t.stride()
    return (s[0], s[1], s[2])


def _check_extent(t, shape, strides, name):
    """Every element the library may touch lies inside t's storage."""
    need = 1 + sum((n - 1) * s for n, s in zip(shape, strides))
    have = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
    if need > have:
        raise ValueError(f"fa: {name} buffer too small: needs {need} elements, has {have}")


def fwd(q, k, v, *, mask=None, causal=False, scale=None, out=None, lse=None, stream=None, dropout_p=None, seed=0,
        offset=0, window=None, no_alloc=False):
    """O, L = attention forward on the GPU through libfa_mi355x.

    q [B, H_q, qL, D]; k, v [B, H_kv, kL, D]: bf16 or fp32 CUDA tensors whose
    last axis is contiguous (other axes may be strided views).
    mask: None; a bool/uint8 tensor (nonzero = attend); or an additive tensor
    of q's dtype.  Shape [B, H_q, qL, kL], or broadcast to it with expand()
    (stride-0 axes); its last axis must be contiguous.
    out: optional O destination [B, H_q, qL, D] of q's dtype, any strides
    with a contiguous last axis (a token-major buffer is
    torch.empty(B, qL, H_q, D).transpose(1, 2)).  lse: optional fp32
    [B, H_q, qL] contiguous.  scale defaults to 1/sqrt(D).
    The call is asynchronous on `stream` (default: torch's current stream).
    dropout_p: None, or a rate in [0, 1] for dropout on the attention weights
    under the 64-bit `seed` and counter `offset` (fa_fwd_dropout; bf16 or
    fp32 at every D).
    window: None, or a causal sliding window of that many keys (row i sees
    keys i - window + 1 .. i; fa_fwd_window, causal only).
    no_alloc: call fa_fwd_strided_noalloc (no window or dropout): split
    partials go to the library's static per-GPU scratch; calls that overlap
    on one GPU must be serialised by the caller.
    """
    import torch

    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("fa: q, k, v must be CUDA (HIP) tensors")
    if q.dtype not in (torch.bfloat16, torch.float32) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("fa: q, k, v must all be bf16 or all fp32")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("fa: q, k, v must be 4-D [B, H, L, D]")
    B, Hq, qL, D = q.shape
    Bk, Hkv, kL, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError(f"fa: shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.stride(3) != 1:
            raise ValueError(f"fa: {n} must have a contiguous last axis")
    dtype = FA_DTYPE_BF16 if q.dtype == torch.bfloat16 else FA_DTYPE_F32
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, qL, D), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, qL), dtype=torch.float32, device=q.device)
    if tuple(out.shape) != (B, Hq, qL, D) or out.dtype != q.dtype or out.stride(3) != 1:
        raise ValueError("fa: out must be [B, H_q, qL, D] of q's dtype with a contiguous last axis")
    if tuple(lse.shape) != (B, Hq, qL) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("fa: lse must be a contiguous fp32 [B, H_q, qL] tensor")

    st = FaStrides()
    st.q[:] = _strides3(q)
    st.k[:] = _strides3(k)
    st.v[:] = _strides3(v)
    st.o[:] = _strides3(out)
    _check_extent(q, q.shape, q.stride(), "q")
    _check_extent(k, k.shape, k.stride(), "k")
    _check_extent(v, v.shape, v.stride(), "v")
    _check_extent(out, out.shape, out.stride(), "out")

    mask_kind, mptr = FA_MASK_NONE, None
    if mask is not None:
        if not mask.is_cuda:
            raise ValueError("fa: mask must be a CUDA tensor")
        if mask.dtype in (torch.bool, torch.uint8):
            mask_kind = FA_MASK_BOOL
            if mask.dtype == torch.bool:
                mask = mask.view(torch.uint8)
        elif mask.dtype == q.dtype:
            mask_kind = FA_MASK_ADDITIVE
        else:
            raise ValueError("fa: an additive mask must have q's dtype; a bool mask must be bool or uint8")
        if mask.dim() != 4:
            raise ValueError("fa: mask must be 4-D (use expand() to broadcast)")
        mask = mask.expand(B, Hq, qL, kL)
        if mask.stride(3) != 1:
            raise ValueError("fa: mask must have a contiguous last axis")
        ms = list(_strides3(mask))
        # size-1 axes can take any stride; all-zero strides mean "default" in
        # the ABI, so a fully broadcast mask is given an explicit row stride.
        if ms == [0, 0, 0]:
            if qL == 1:
                ms[2] = kL
            else:
                mask = mask.contiguous()
                ms = list(_strides3(mask))
        st.mask[:] = ms
        _check_extent(mask, mask.shape, mask.stride(), "mask")
        mptr = mask.data_ptr()

    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    if window is not None and dropout_p is not None:
        raise ValueError("fa: window and dropout_p are not combined")
    if no_alloc and (window is not None or dropout_p is not None):
        raise ValueError("fa: no_alloc has no window or dropout variant")
    if no_alloc:
        check(fa_fwd_strided_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), mptr, out.data_ptr(), lse.data_ptr(),
                                     B, Hq, Hkv, qL, kL, D, float(scale), int(bool(causal)), dtype, mask_kind, st,
                                     stream.cuda_stream))
    elif window is not None:
        check(fa_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), mptr, out.data_ptr(), lse.data_ptr(),
                            B, Hq, Hkv, qL, kL, D, float(scale), int(bool(causal)), dtype, mask_kind, int(window),
                            st, stream.cuda_stream))
    elif dropout_p is None:
        check(fa_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), mptr, out.data_ptr(), lse.data_ptr(),
                             B, Hq, Hkv, qL, kL, D, float(scale), int(bool(causal)), dtype, mask_kind, st,
                             stream.cuda_stream))
    else:
        check(fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), mptr, out.data_ptr(), lse.data_ptr(),
                             B, Hq, Hkv, qL, kL, D, float(scale), int(bool(causal)), dtype, mask_kind,
                             float(dropout_p), int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1), st,
                             stream.cuda_stream))
    return out, lse


def bwd(q, k, v, o, do, lse, *, mask=None, causal=False, scale=None, dq=None, dk=None, dv=None, delta=None,
        stream=None):
    """dQ, dK, dV (and Delta = rowsum(dO * O)) of the attention forward pass
    on the GPU through libfa_mi355x (fa_bwd).

    q, o, do [B, H_q, qL, D] and k, v [B, H_kv, kL, D]: contiguous bf16 CUDA
    tensors; o and lse are fwd's outputs for the same q, k, v, mask, scale
    and causal.  mask: None, bool/uint8 (nonzero = attend) or additive of q's
    dtype, contiguous [B, H_q, qL, kL].  Returns (dq, dk, dv, delta).
    """
    import torch

    B, Hq, qL, D = q.shape
    Bk, Hkv, kL, Dk = k.shape
    for t, n, shape in ((q, "q", (B, Hq, qL, D)), (o, "o", (B, Hq, qL, D)), (do, "do", (B, Hq, qL, D)),
                        (k, "k", (B, Hkv, kL, D)), (v, "v", (B, Hkv, kL, D))):
        if not t.is_cuda or t.dtype != q.dtype or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"fa.bwd: {n} must be a contiguous CUDA tensor of shape {shape} and q's dtype")
    if tuple(lse.shape) != (B, Hq, qL) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("fa.bwd: lse must be a contiguous fp32 [B, H_q, qL] tensor")
    dtype = FA_DTYPE_BF16 if q.dtype == torch.bfloat16 else FA_DTYPE_F32
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    delta = torch.empty_like(lse) if delta is None else delta
    for t, ref, n in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv"), (delta, lse, "delta")):
        if t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous():
            raise ValueError(f"fa.bwd: {n} must be contiguous, shaped and typed like {'lse' if n == 'delta' else n[1:]}")
    mask_kind, mptr = FA_MASK_NONE, None
    if mask is not None:
        if mask.dtype in (torch.bool, torch.uint8):
            mask_kind = FA_MASK_BOOL
            if mask.dtype == torch.bool:
                mask = mask.view(torch.uint8)
        elif mask.dtype == q.dtype:
            mask_kind = FA_MASK_ADDITIVE
        else:
            raise ValueError("fa.bwd: an additive mask must have q's dtype; a bool mask must be bool or uint8")
        if tuple(mask.shape) != (B, Hq, qL, kL) or not mask.is_contiguous() or not mask.is_cuda:
            raise ValueError("fa.bwd: mask must be a contiguous CUDA [B, H_q, qL, kL] tensor")
        mptr = mask.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    check(fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), mptr,
                 delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, qL, kL, D, float(scale),
                 int(bool(causal)), dtype, mask_kind, stream.cuda_stream))
    return dq, dk, dv, delta
