"""aule_attn: tiled attention forward for AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C-ABI library ``libaule_attn.so`` (declared in
``include/aule_attn.h``). Every step of the computation runs in the library's HIP kernels;
this module only marshals arguments. PyTorch is used for device tensors and streams.

Low-level functions carry the C names (``aule_attn_fwd``, ``aule_attn_fwd_varlen``,
``aule_status_string``, ``aule_last_error``) and take raw device pointers. The tensor-level
wrappers follow the pages' APIs:

* ``flash_attention(q, k, v, causal=True, scale=None)`` — [batch, heads, seq, head_dim]
  tensors, ``causal`` defaulting to True and ``scale`` to 1/sqrt(head_dim), heads_q a
  multiple of heads_kv (jeff.news Aule-Attention article, API bullets; jdon.com
  Aule-Attention article, GQA/MQA examples);
* ``flash_attn_varlen_qkvpacked_func(qkv, cu_seqlens, max_seqlen, ...)`` — packed
  [total_tokens, 3, heads, head_dim] with cumulative ``cu_seqlens``, ``causal`` defaulting
  to False (ewbang.com article on a PyTorch FlashAttention for Turing, signature and
  docstring of the varlen function; its unsupported options raise NotImplementedError);
* ``flash_attention(..., return_lse=True)`` and ``flash_attention_backward(q, k, v, out, dout,
  lse)`` — the per-row log-sum-exp and the gradients (dq, dk, dv), the score matrix
  recomputed in the backward (FlashAttention-T commentary, FAQ 4, training bullet);
  when q, k or v requires grad, ``flash_attention`` records itself for autograd, so
  ``flash_attention(q, k, v, causal=True).sum().backward()`` fills q.grad, k.grad and v.grad
  (the gradient example of the jdon.com Aule-Attention article): the forward runs
  aule_attn_fwd_lse and keeps O and the LSE, the backward runs aule_attn_bwd;
* ``flash_attention_decode(q, k, v, causal=True, scale=None, num_splits=0)`` — a few new
  queries against a key/value cache, split over the key range (FlashAttention-T
  commentary, FAQ 4: the KV cache processed in blocks at inference); causal masking is
  bottom-right aligned. The fp32 workspace is allocated with torch per call unless given.

If the library is missing the import still succeeds, but every call raises: there is no
CPU fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libaule_attn.so")

AULE_DTYPE_F32, AULE_DTYPE_F16, AULE_DTYPE_BF16 = 0, 1, 2
AULE_OK, AULE_ERR_INVALID_ARGUMENT, AULE_ERR_UNSUPPORTED, AULE_ERR_HIP = 0, 1, 2, 3

EXPORTED = ("aule_attn_fwd", "aule_attn_fwd_lse", "aule_attn_bwd", "aule_attn_fwd_varlen",
            "aule_attn_fwd_varlen_mods",
            "aule_attn_fwd_splitkv", "aule_attn_splitkv_workspace_size",
            "aule_attn_fwd_splitkv_noalloc", "aule_status_string", "aule_last_error")

_lib = None


class AuleError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{aule_status_string(status)}: {detail}")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libaule_attn.so (built by ``tiled_attention_02_amd.build``). Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m tiled_attention_02_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    i32, vp, f32 = ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
    lib.aule_attn_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                  ctypes.c_int, vp]
    lib.aule_attn_fwd.restype = ctypes.c_int
    lib.aule_attn_fwd_varlen.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                         ctypes.c_int, vp]
    lib.aule_attn_fwd_varlen.restype = ctypes.c_int
    lib.aule_attn_fwd_varlen_mods.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32,
                                              i32, f32, vp, i32, ctypes.c_int, vp]
    lib.aule_attn_fwd_varlen_mods.restype = ctypes.c_int
    lib.aule_attn_fwd_lse.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                      ctypes.c_int, vp]
    lib.aule_attn_fwd_lse.restype = ctypes.c_int
    lib.aule_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                  i32, f32, ctypes.c_int, vp]
    lib.aule_attn_bwd.restype = ctypes.c_int
    lib.aule_attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                          ctypes.c_int, i32, vp, ctypes.c_size_t, vp]
    lib.aule_attn_fwd_splitkv.restype = ctypes.c_int
    lib.aule_attn_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                  i32, f32, ctypes.c_int, i32, vp]
    lib.aule_attn_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.aule_attn_splitkv_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, ctypes.c_int, i32]
    lib.aule_attn_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.aule_status_string.argtypes = [ctypes.c_int]
    lib.aule_status_string.restype = ctypes.c_char_p
    lib.aule_last_error.argtypes = []
    lib.aule_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ------------------------------------------------------------------ C names

def aule_attn_fwd(q, k, v, o, batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim,
                  causal, scale, dtype, stream=0) -> int:
    """Raw call: device pointers as ints; returns the status code."""
    return load_library().aule_attn_fwd(q, k, v, o, batch, heads_q, heads_kv, seqlen_q,
                                        seqlen_k, head_dim, int(causal), float(scale),
                                        int(dtype), stream)


def aule_attn_fwd_lse(q, k, v, o, lse, batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim,
                      causal, scale, dtype, stream=0) -> int:
    """Raw call: device pointers as ints; returns the status code."""
    return load_library().aule_attn_fwd_lse(q, k, v, o, lse, batch, heads_q, heads_kv, seqlen_q,
                                            seqlen_k, head_dim, int(causal), float(scale),
                                            int(dtype), stream)


def aule_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, batch, heads_q, heads_kv, seqlen_q,
                  seqlen_k, head_dim, causal, scale, dtype, stream=0) -> int:
    """Raw call: device pointers as ints; returns the status code."""
    return load_library().aule_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, batch, heads_q,
                                        heads_kv, seqlen_q, seqlen_k, head_dim, int(causal),
                                        float(scale), int(dtype), stream)


def aule_attn_fwd_varlen(qkv, cu_seqlens, o, num_seqs, total_tokens, max_seqlen, heads,
                         head_dim, causal, scale, dtype, stream=0) -> int:
    """Raw call: device pointers as ints; returns the status code."""
    return load_library().aule_attn_fwd_varlen(qkv, cu_seqlens, o, num_seqs, total_tokens,
                                               max_seqlen, heads, head_dim, int(causal),
                                               float(scale), int(dtype), stream)


def aule_attn_fwd_varlen_mods(qkv, cu_seqlens, o, num_seqs, total_tokens, max_seqlen, heads,
                              head_dim, causal, scale, window_left, window_right, softcap,
                              alibi_slopes, alibi_batch_stride, dtype, stream=0) -> int:
    """Raw call: device pointers as ints (alibi_slopes may be None); returns the status."""
    return load_library().aule_attn_fwd_varlen_mods(
        qkv, cu_seqlens, o, num_seqs, total_tokens, max_seqlen, heads, head_dim, int(causal),
        float(scale), int(window_left), int(window_right), float(softcap), alibi_slopes,
        int(alibi_batch_stride), int(dtype), stream)


def aule_attn_fwd_splitkv(q, k, v, o, batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim,
                          causal, scale, dtype, num_splits, workspace, workspace_bytes,
                          stream=0) -> int:
    """Raw call: device pointers as ints; returns the status code."""
    return load_library().aule_attn_fwd_splitkv(q, k, v, o, batch, heads_q, heads_kv, seqlen_q,
                                                seqlen_k, head_dim, int(causal), float(scale),
                                                int(dtype), int(num_splits), workspace,
                                                int(workspace_bytes), stream)


def aule_attn_fwd_splitkv_noalloc(q, k, v, o, batch, heads_q, heads_kv, seqlen_q, seqlen_k,
                                  head_dim, causal, scale, dtype, num_splits, stream=0) -> int:
    """Raw call: device pointers as ints; the split partials live in the library's own
    device array (nothing is allocated); returns the status code."""
    return load_library().aule_attn_fwd_splitkv_noalloc(q, k, v, o, batch, heads_q, heads_kv,
                                                        seqlen_q, seqlen_k, head_dim, int(causal),
                                                        float(scale), int(dtype), int(num_splits),
                                                        stream)


def aule_attn_splitkv_workspace_size(batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim,
                                     dtype, num_splits=0) -> int:
    return int(load_library().aule_attn_splitkv_workspace_size(batch, heads_q, heads_kv,
                                                               seqlen_q, seqlen_k, head_dim,
                                                               int(dtype), int(num_splits)))


def aule_status_string(status: int) -> str:
    return load_library().aule_status_string(int(status)).decode()


def aule_last_error() -> str:
    return load_library().aule_last_error().decode()


def _check(status: int) -> None:
    if status != AULE_OK:
        raise AuleError(status, aule_last_error())


# ------------------------------------------------------------------ tensor wrappers

def _torch():
    import torch
    return torch


def dtype_code(dtype) -> int:
    torch = _torch()
    codes = {torch.float32: AULE_DTYPE_F32, torch.float16: AULE_DTYPE_F16,
             torch.bfloat16: AULE_DTYPE_BF16}
    if dtype not in codes:
        raise TypeError(f"unsupported dtype {dtype}; use float16, bfloat16 or float32")
    return codes[dtype]


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _need_gpu_tensor(name, t):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _autograd_fn():
    """The torch.autograd.Function that records flash_attention for the backward (built on
    first use so that importing this module does not import torch)."""
    global _FlashAttentionFn
    if _FlashAttentionFn is not None:
        return _FlashAttentionFn
    torch = _torch()

    class FlashAttentionFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, scale):
            out, lse = _forward(q, k, v, causal, scale, None, True)
            ctx.save_for_backward(q, k, v, out, lse)
            ctx.causal, ctx.scale = causal, scale
            ctx.mark_non_differentiable(lse)
            return out, lse

        @staticmethod
        def backward(ctx, dout, _dlse):
            q, k, v, out, lse = ctx.saved_tensors
            if dout is None:
                return None, None, None, None, None
            # autograd may hand over an expanded (stride 0) gradient, e.g. from .sum()
            dq, dk, dv = flash_attention_backward(q, k, v, out, dout.contiguous(), lse,
                                                  causal=ctx.causal, scale=ctx.scale)
            return dq, dk, dv, None, None

    _FlashAttentionFn = FlashAttentionFn
    return FlashAttentionFn


_FlashAttentionFn = None


def flash_attention(q, k, v, causal: bool = True, scale: float | None = None, out=None,
                    return_lse: bool = False):
    """O = softmax(scale * q k^T [+ causal mask]) v for q [B,Hq,N,d], k/v [B,Hkv,Nk,d].
    With ``return_lse`` also returns the fp32 per-row log-sum-exp [B,Hq,N] the backward
    needs: (out, lse). When gradients are enabled and q, k or v requires grad the call is
    recorded for autograd (``out`` must then be None)."""
    torch = _torch()
    if torch.is_grad_enabled() and any(t.requires_grad for t in (q, k, v)):
        if out is not None:
            raise ValueError("out= cannot be used when q, k or v requires grad")
        if scale is None:
            scale = 1.0 / math.sqrt(q.shape[-1])
        o, lse = _autograd_fn().apply(q, k, v, bool(causal), float(scale))
        return (o, lse) if return_lse else o
    return _forward(q, k, v, causal, scale, out, return_lse)


def _forward(q, k, v, causal, scale, out, return_lse):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_gpu_tensor(name, t)
        if t.dim() != 4:
            raise ValueError(f"{name} must be [batch, heads, seq_len, head_dim]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError("k and v must be [batch, heads_kv, seq_len_k, head_dim] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_gpu_tensor("out", out)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    if return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
        st = aule_attn_fwd_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, causal, scale,
                               dtype_code(q.dtype), _stream_handle(q.device))
        _check(st)
        return out, lse
    st = aule_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv,
                       Nq, Nk, d, causal, scale, dtype_code(q.dtype),
                       _stream_handle(q.device))
    _check(st)
    return out


def flash_attention_backward(q, k, v, out, dout, lse, causal: bool = True,
                             scale: float | None = None, grads=None):
    """Gradients (dq, dk, dv) of flash_attention(q, k, v, causal, scale) = out for the output
    gradient dout, from the lse that flash_attention(..., return_lse=True) returned. ``grads``
    may give preallocated (dq, dk, dv) buffers of the shapes and dtype of (q, k, v)."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("lse", lse)):
        _need_gpu_tensor(name, t)
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise TypeError("q, k, v, out and dout must share a dtype")
    if q.dim() != 4 or k.dim() != 4 or tuple(k.shape) != tuple(v.shape):
        raise ValueError("q [B,Hq,N,d], k and v [B,Hkv,Nk,d]")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must have the shape of q")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("lse must be float32 [B, Hq, N]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = grads
        for name, g, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
            _need_gpu_tensor(name, g)
            if g.shape != like.shape or g.dtype != like.dtype:
                raise ValueError(f"{name} must have the shape and dtype of its input")
    st = aule_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                       lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq,
                       Nk, d, causal, scale, dtype_code(q.dtype), _stream_handle(q.device))
    _check(st)
    return dq, dk, dv


def flash_attention_decode(q, k, v, causal: bool = True, scale: float | None = None,
                           num_splits: int = 0, out=None, workspace=None):
    """Attention of q [B,Hq,Nq,d] (a few new queries) against the cache k/v [B,Hkv,Nk,d],
    split over the key range; under ``causal`` query i is position Nk - Nq + i. ``workspace``
    (a uint8 GPU tensor of at least aule_attn_splitkv_workspace_size bytes) is allocated
    here when not given."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need_gpu_tensor(name, t)
        if t.dim() != 4:
            raise ValueError(f"{name} must be [batch, heads, seq_len, head_dim]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError("k and v must be [batch, heads_kv, seq_len_k, head_dim] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dt = dtype_code(q.dtype)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need_gpu_tensor("out", out)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    need = aule_attn_splitkv_workspace_size(B, Hq, Hkv, Nq, Nk, d, dt, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        _need_gpu_tensor("workspace", workspace)
    st = aule_attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq,
                               Hkv, Nq, Nk, d, causal, scale, dt, num_splits,
                               workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                               _stream_handle(q.device))
    _check(st)
    return out


def flash_attn_varlen_qkvpacked_func(qkv, cu_seqlens, max_seqlen, dropout_p=0.0,
                                     softmax_scale=None, causal=False, window_size=(-1, -1),
                                     softcap=0.0, alibi_slopes=None, deterministic=False,
                                     return_attn_probs=False, out=None, validate=False):
    """Varlen attention over packed qkv [total_tokens, 3, heads, head_dim] with int32
    cu_seqlens [batch+1] on the device; returns [total_tokens, heads, head_dim].

    Score modifiers: ``window_size=(left, right)`` sliding window (-1 = unbounded; with
    causal, right must be -1 or 0), ``softcap`` > 0 caps the scaled scores at
    softcap * tanh(x / softcap), ``alibi_slopes`` (fp32 [heads] or [batch, heads] on the
    device) subtracts slope * |i - j|.

    ``max_seqlen`` must be at least the longest sequence: tokens of a sequence past it are
    neither read as keys nor written. ``validate=True`` also checks cu_seqlens against
    total_tokens and max_seqlen, which reads it back to the host (a synchronisation)."""
    torch = _torch()
    if dropout_p != 0.0:
        raise NotImplementedError("dropout is not supported")
    if return_attn_probs:
        raise NotImplementedError("return_attn_probs is not supported")
    _need_gpu_tensor("qkv", qkv)
    if qkv.dim() != 4 or qkv.shape[1] != 3:
        raise ValueError("Bad qkv shape")
    if cu_seqlens is None or cu_seqlens.dim() != 1 or cu_seqlens.dtype != torch.int32:
        raise ValueError("Bad cu_seqlens")
    _need_gpu_tensor("cu_seqlens", cu_seqlens)
    num_seqs = cu_seqlens.shape[0] - 1
    if num_seqs <= 0:
        raise ValueError("Bad batch size")
    T, _, H, d = qkv.shape
    if validate:
        cu = cu_seqlens.cpu()
        if int(cu[0]) != 0 or int(cu[-1]) != T:
            raise ValueError("Token count mismatch")
        lens = cu[1:] - cu[:-1]
        if bool((lens < 0).any()):
            raise ValueError("Bad cu_seqlens")
        if T and int(lens.max()) > int(max_seqlen):
            raise ValueError("max_seqlen is smaller than the longest sequence")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((T, H, d), dtype=qkv.dtype, device=qkv.device)
    wl, wr = (int(window_size[0]), int(window_size[1]))
    if (wl, wr) == (-1, -1) and softcap == 0.0 and alibi_slopes is None:
        st = aule_attn_fwd_varlen(qkv.data_ptr(), cu_seqlens.data_ptr(), out.data_ptr(), num_seqs,
                                  T, int(max_seqlen), H, d, causal, softmax_scale,
                                  dtype_code(qkv.dtype), _stream_handle(qkv.device))
        _check(st)
        return out
    a_ptr, a_stride = None, 0
    if alibi_slopes is not None:
        _need_gpu_tensor("alibi_slopes", alibi_slopes)
        if alibi_slopes.dtype != torch.float32:
            raise ValueError("alibi_slopes must be float32")
        if tuple(alibi_slopes.shape) == (H,):
            a_stride = 0
        elif tuple(alibi_slopes.shape) == (num_seqs, H):
            a_stride = H
        else:
            raise ValueError("alibi_slopes must be [heads] or [batch, heads]")
        a_ptr = alibi_slopes.data_ptr()
    st = aule_attn_fwd_varlen_mods(qkv.data_ptr(), cu_seqlens.data_ptr(), out.data_ptr(),
                                   num_seqs, T, int(max_seqlen), H, d, causal, softmax_scale,
                                   wl, wr, softcap, a_ptr, a_stride, dtype_code(qkv.dtype),
                                   _stream_handle(qkv.device))
    _check(st)
    return out


__all__ = ["aule_attn_fwd", "aule_attn_fwd_lse", "aule_attn_bwd", "aule_attn_fwd_varlen",
           "aule_attn_fwd_varlen_mods",
           "aule_attn_fwd_splitkv", "aule_attn_fwd_splitkv_noalloc", "flash_attention_backward",
           "aule_attn_splitkv_workspace_size", "aule_status_string", "aule_last_error",
           "flash_attention", "flash_attention_decode", "flash_attn_varlen_qkvpacked_func",
           "load_library", "AuleError", "LIB_PATH", "EXPORTED"]
