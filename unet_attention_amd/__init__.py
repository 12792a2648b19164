"""Python binding of libsdattn (fused UNet attention for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libsdattn.so``.  The raw functions keep the C names and take
integer device pointers and a ``hipStream_t`` (as an int, 0 = default
stream); ``fwd`` / ``cross_fwd`` / ``stream_fwd`` accept torch tensors on
the ROCm device and use torch only for buffers and the current stream.

The library must have been built (``__graft_entry__.build()`` or
``python unet_attention_amd/build.py``); loading fails loudly otherwise --
there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsdattn.so")

SDATTN_OK = 0
SDATTN_ERR_INVALID_ARG = 1
SDATTN_ERR_UNSUPPORTED = 2
SDATTN_ERR_MISALIGNED = 3
SDATTN_ERR_DEVICE = 4
SDATTN_ERR_LAUNCH = 5

SDATTN_DTYPE_F32 = 0
SDATTN_DTYPE_BF16 = 1
SDATTN_DTYPE_BF16_F32OUT = 2
SDATTN_DTYPE_F16 = 3
SDATTN_DTYPE_F16_F32OUT = 4

# Every function the C header declares, with its ctypes signature.
_VP = ctypes.c_void_p
_I = ctypes.c_int
_ATTN_ARGS = [_VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, ctypes.c_float, _I, _VP]
EXPORTS = {
    "sdattn_fwd": (_I, _ATTN_ARGS),
    "sdattn_cross_fwd": (_I, _ATTN_ARGS),
    "sdattn_stream_fwd": (_I, _ATTN_ARGS),
    "sdattn_fwd_strided": (_I, [_VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _I,
                                ctypes.c_float, _I, _VP]),
    "sdattn_group_norm": (_I, [_VP, _VP, _VP, _VP, _I, _I, _I, _I, ctypes.c_float, _I, _I, _VP]),
    "sdattn_cross_max_ctx": (_I, [_I, _I]),
    "sdattn_strerror": (ctypes.c_char_p, [_I]),
    "sdattn_version": (_I, []),
}


class SdattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {sdattn_strerror(status)} (status {status})")


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsdattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(path)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


# ---------------------------------------------------------------------------
# raw C ABI (same names and argument order as include/sdattn.h)

def sdattn_fwd(q, k, v, out, B, H, Lq, Lk, d, scale, dtype, stream):
    return load().sdattn_fwd(q, k, v, out, B, H, Lq, Lk, d, scale, dtype, stream)


def sdattn_cross_fwd(q, ctx_k, ctx_v, out, B, H, Lq, Lctx, d, scale, dtype, stream):
    return load().sdattn_cross_fwd(q, ctx_k, ctx_v, out, B, H, Lq, Lctx, d,
                                   scale, dtype, stream)


def sdattn_stream_fwd(q, k, v, out, B, H, Lq, Lk, d, scale, dtype, stream):
    return load().sdattn_stream_fwd(q, k, v, out, B, H, Lq, Lk, d, scale, dtype, stream)


def sdattn_fwd_strided(q, k, v, out, B, H, Lq, Lk, d, ldq, ldkv, ldo, scale, dtype, stream):
    return load().sdattn_fwd_strided(q, k, v, out, B, H, Lq, Lk, d, ldq, ldkv, ldo,
                                     scale, dtype, stream)


def sdattn_group_norm(x, gamma, beta, y, N, C, HW, G, eps, silu, dtype, stream):
    return load().sdattn_group_norm(x, gamma, beta, y, N, C, HW, G, eps, silu, dtype, stream)


def sdattn_cross_max_ctx(d, dtype):
    return load().sdattn_cross_max_ctx(d, dtype)


def sdattn_strerror(status):
    return load().sdattn_strerror(status).decode()


def sdattn_version():
    return load().sdattn_version()


# ---------------------------------------------------------------------------
# torch tensors in, torch tensors out


def _on_stream(stream, device):
    """(hipStream_t handle, context) for a call: the caller's stream handle
    (an int) or, if None, torch's current stream.  Under the context, torch
    allocates and converts on that same stream, so every temporary and the
    output are ordered before the kernel that reads or writes them (and the
    caching allocator does not hand their memory to other streams early)."""
    import contextlib
    import torch
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream, contextlib.nullcontext()
    ext = torch.cuda.ExternalStream(stream, device=device)
    return stream, torch.cuda.stream(ext)

_ENTRIES = {"auto": "sdattn_fwd", "cross": "sdattn_cross_fwd",
            "stream": "sdattn_stream_fwd"}


def _dtype_code(in_dtype, out_dtype):
    """(sdattn dtype code, output torch dtype) for an input/output pair."""
    import torch
    if in_dtype == torch.float32:
        if out_dtype not in (None, torch.float32):
            raise ValueError("fp32 inputs produce fp32 output")
        return SDATTN_DTYPE_F32, torch.float32
    codes = {torch.bfloat16: (SDATTN_DTYPE_BF16, SDATTN_DTYPE_BF16_F32OUT),
             torch.float16: (SDATTN_DTYPE_F16, SDATTN_DTYPE_F16_F32OUT)}
    if in_dtype not in codes:
        raise ValueError(f"unsupported input dtype {in_dtype}")
    odt = out_dtype or in_dtype
    if odt == in_dtype:
        return codes[in_dtype][0], odt
    if odt == torch.float32:
        return codes[in_dtype][1], odt
    raise ValueError(f"unsupported output dtype {odt}")


def _call(entry, q, k, v, out=None, scale=None, out_dtype=None, stream=None):
    import torch
    dtype_code, odt = _dtype_code(q.dtype, out_dtype)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} != q dtype {q.dtype}")
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous 4-d device tensor [B,H,L,d]")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if tuple(k.shape) != (B, H, Lk, d) or tuple(v.shape) != (B, H, Lk, d):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if out is not None and (out.dtype != odt or tuple(out.shape) != (B, H, Lq, d)
                            or not out.is_contiguous()):
        raise ValueError("out must be a contiguous [B,H,Lq,d] tensor of the output dtype")
    if scale is None:
        scale = float(1.0 / math.sqrt(d))
    fn = getattr(load(), _ENTRIES[entry])
    handle, ctx = _on_stream(stream, q.device)
    with ctx:
        if out is None:
            out = torch.empty((B, H, Lq, d), dtype=odt, device=q.device)
        rc = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                B, H, Lq, Lk, d, scale, dtype_code, handle)
    if rc != SDATTN_OK:
        raise SdattnError(rc, _ENTRIES[entry])
    return out


def fwd(q, k, v, out=None, scale=None, out_dtype=None, stream=None):
    """softmax(scale * Q K^T) V via sdattn_fwd (short-key or streaming kernel)."""
    return _call("auto", q, k, v, out, scale, out_dtype, stream)


def cross_fwd(q, ctx_k, ctx_v, out=None, scale=None, out_dtype=None, stream=None):
    """Cross-attention to a short context via sdattn_cross_fwd."""
    return _call("cross", q, ctx_k, ctx_v, out, scale, out_dtype, stream)


def stream_fwd(q, k, v, out=None, scale=None, out_dtype=None, stream=None):
    """Always the streaming (online-softmax) kernel, via sdattn_stream_fwd."""
    return _call("stream", q, k, v, out, scale, out_dtype, stream)


def fwd_tokens(q, k, v, heads, out=None, scale=None, out_dtype=None, stream=None):
    """Attention on token-major operands via sdattn_fwd_strided.

    q is [B, Lq, C] and k, v are [B, Lk, C] with C = heads * d, each with
    unit column stride and any row stride (so column slices of a fused
    [B, L, 3C] projection work directly); head h is columns [h*d, (h+1)*d).
    Returns (or fills) out as [B, Lq, C].
    """
    import torch
    dtype_code, odt = _dtype_code(q.dtype, out_dtype)
    if k.stride() != v.stride():
        raise ValueError("k and v must have the same strides")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} != q dtype {q.dtype}")
        if not t.is_cuda or t.dim() != 3 or t.stride(2) != 1 or \
                t.stride(0) != t.shape[1] * t.stride(1):
            raise ValueError(f"{name} must be a [B, L, C] device tensor with unit column "
                             "stride and batch stride L * row stride")
    B, Lq, C = q.shape
    Lk = k.shape[1]
    if C % heads:
        raise ValueError(f"C = {C} is not a multiple of heads = {heads}")
    d = C // heads
    if tuple(k.shape) != (B, Lk, C) or tuple(v.shape) != (B, Lk, C):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if out is not None and (out.dtype != odt or tuple(out.shape) != (B, Lq, C)
                            or out.stride(2) != 1 or out.stride(0) != Lq * out.stride(1)):
        raise ValueError("out must be a [B, Lq, C] tensor of the output dtype")
    if scale is None:
        scale = float(1.0 / math.sqrt(d))
    handle, ctx = _on_stream(stream, q.device)
    with ctx:
        if out is None:
            out = torch.empty((B, Lq, C), dtype=odt, device=q.device)
        rc = load().sdattn_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       B, heads, Lq, Lk, d, q.stride(1), k.stride(1),
                                       out.stride(1), scale, dtype_code, handle)
    if rc != SDATTN_OK:
        raise SdattnError(rc, "sdattn_fwd_strided")
    return out


def group_norm(x, gamma, beta, groups, eps=1e-5, silu=False, out=None, out_dtype=None,
               stream=None):
    """GroupNorm (+ SiLU) of a contiguous [N, C, *spatial] device tensor via
    sdattn_group_norm; gamma and beta are [C] (passed as fp32).  out may be
    x itself (in place) when the output dtype equals the input dtype."""
    import torch
    dtype_code, odt = _dtype_code(x.dtype, out_dtype)
    if not x.is_cuda or not x.is_contiguous() or x.dim() < 2:
        raise ValueError("x must be a contiguous [N, C, ...] device tensor")
    N, C = x.shape[0], x.shape[1]
    HW = x.numel() // max(1, N * C)
    if gamma.numel() != C or beta.numel() != C:
        raise ValueError("gamma and beta must have C entries")
    if out is not None and (out.dtype != odt or out.shape != x.shape or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor of x's shape and the output dtype")
    handle, ctx = _on_stream(stream, x.device)
    with ctx:
        # fp32 copies of gamma and beta (when they are not fp32 already) are
        # made on the launch stream, so the kernel runs after them
        g = gamma.to(device=x.device, dtype=torch.float32).contiguous()
        b = beta.to(device=x.device, dtype=torch.float32).contiguous()
        if out is None:
            out = torch.empty(x.shape, dtype=odt, device=x.device)
        rc = load().sdattn_group_norm(x.data_ptr(), g.data_ptr(), b.data_ptr(), out.data_ptr(),
                                      N, C, HW, groups, float(eps), int(bool(silu)), dtype_code,
                                      handle)
    if rc != SDATTN_OK:
        raise SdattnError(rc, "sdattn_group_norm")
    return out
