"""Exact scaled-dot-product attention forward for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libattn.so`` (see ``include/attn.h``).  The
functions carry the C names and only marshal arguments: torch tensors supply device
pointers and the current HIP stream, and every step of the computation runs in the HIP
kernels.  There is no fallback: if the library is not built, or a call is refused, an
exception is raised.

    o, lse = attn_fwd(q, k, v, scale=None, causal=False)
    o, lse = attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    ws = attn_fwd_splitkv(q, k, v, num_splits, ...)
    o, lse = attn_merge(ws, num_splits, B, H, Sq, d)

Tensors are [B, H, S, d] contiguous on the GPU (ragged batches: [H, total, d] with int32
sequence offsets): torch.float32, torch.bfloat16, or FP8
E4M3FN codes (torch.float8_e4m3fn, or torch.uint8 holding the codes).  Outputs are
float32.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import (ATTN_BF16, ATTN_F32, ATTN_FP8_E4M3, ATTN_MAX_SPLITS,  # noqa: F401
                   ATTN_NOALLOC_SCRATCH_BYTES, AttnError)

__all__ = [
    "attn_fwd", "attn_fwd_ex", "attn_fwd_varlen", "attn_fwd_splitkv", "attn_merge", "attn_splitkv_workspace_bytes",
    "attn_fwd_splitkv_noalloc",
    "attn_splitkv_num_splits",
    "attn_block_m", "attn_block_n", "attn_num_workgroups", "attn_kernel_name",
    "attn_tune", "attn_tune_splitkv", "attn_plan_get", "attn_plan_set", "attn_plan_clear", "plan_parts",
    "attn_status_string", "attn_last_hip_error", "dtype_code", "library_path", "AttnError",
]


def library_path() -> str:
    return _lib.LIB_PATH


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return ATTN_FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def ctypes_ptr(t: torch.Tensor) -> int:
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _out(name, t, shape, dtype, device):
    """Check a caller-supplied output tensor before the call: the C ABI gets only a pointer,
    so a tensor of the wrong type, size or device would be written past its end."""
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    return t


def _same_device(device, **tensors):
    for name, t in tensors.items():
        if t.device != device:
            raise ValueError(f"{name} must be on {device}, got {t.device}")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _qkv(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, d]")
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    if tuple(k.shape) != (B, H, Sk, d) or tuple(v.shape) != (B, H, Sk, d):
        raise ValueError("k and v must be [B, H, Sk, d] with q's B, H and d")
    dt = dtype_code(q)
    if dtype_code(k) != dt or dtype_code(v) != dt:
        raise TypeError("q, k and v must share one dtype")
    _same_device(q.device, k=k, v=v)
    return B, H, Sq, Sk, d, dt


def attn_fwd(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """O = softmax(scale * Q K^T [causal mask]) V and the row log-sum-exp, both fp32."""
    B, H, Sq, Sk, d, dt = _qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Sq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _out("out", out, (B, H, Sq, d), torch.float32, q.device)
    _out("lse", lse, (B, H, Sq), torch.float32, q.device)
    st = _lib.load().attn_fwd(ctypes_ptr(q), ctypes_ptr(k), ctypes_ptr(v), ctypes_ptr(out),
                              ctypes_ptr(lse), B, H, Sq, Sk, d, float(scale), int(causal), dt,
                              _stream(stream))
    _lib.check("attn_fwd", st)
    return out, lse


def attn_fwd_ex(q, k, v, scale=None, causal=False, out_dtype=torch.bfloat16, out=None, lse=None,
                stream=None):
    """attn_fwd with O written as ``out_dtype`` (torch.float32 or torch.bfloat16; bf16 is the
    fp32 result rounded to nearest even at the write-back); lse is float32."""
    B, H, Sq, Sk, d, dt = _qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    odt = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}.get(out_dtype)
    if odt is None:
        raise TypeError(f"unsupported output dtype {out_dtype}")
    if out is None:
        out = torch.empty((B, H, Sq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _out("out", out, (B, H, Sq, d), out_dtype, q.device)
    _out("lse", lse, (B, H, Sq), torch.float32, q.device)
    st = _lib.load().attn_fwd_ex(ctypes_ptr(q), ctypes_ptr(k), ctypes_ptr(v), ctypes_ptr(out),
                                 ctypes_ptr(lse), B, H, Sq, Sk, d, float(scale), int(causal), dt,
                                 odt, _stream(stream))
    _lib.check("attn_fwd_ex", st)
    return out, lse


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    scale=None, causal=False, out=None, lse=None, stream=None):
    """attn_fwd over B packed sequences: q [H, total_q, d], k and v [H, total_k, d],
    cu_seqlens_* int32 [B+1] offsets on the GPU; O [H, total_q, d] and lse [H, total_q]
    (float32).  Sequence b uses rows cu[b]:cu[b+1] of every head and its own keys only."""
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [H, total, d]")
    H, total_q, d = q.shape
    total_k = k.shape[1]
    if tuple(k.shape) != (H, total_k, d) or tuple(v.shape) != (H, total_k, d):
        raise ValueError("k and v must be [H, total_k, d] with q's H and d")
    dt = dtype_code(q)
    if dtype_code(k) != dt or dtype_code(v) != dt:
        raise TypeError("q, k and v must share one dtype")
    for c in (cu_seqlens_q, cu_seqlens_k):
        if c.dtype != torch.int32 or c.dim() != 1:
            raise TypeError("cu_seqlens must be 1-D int32 tensors")
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _same_device(q.device, k=k, v=v, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k)
    if out is None:
        out = torch.empty((H, total_q, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    _out("out", out, (H, total_q, d), torch.float32, q.device)
    _out("lse", lse, (H, total_q), torch.float32, q.device)
    st = _lib.load().attn_fwd_varlen(
        ctypes_ptr(q), ctypes_ptr(k), ctypes_ptr(v), ctypes_ptr(out), ctypes_ptr(lse),
        ctypes_ptr(cu_seqlens_q), ctypes_ptr(cu_seqlens_k), B, H, int(max_seqlen_q),
        int(max_seqlen_k), total_q, total_k, d, float(scale), int(causal), dt, _stream(stream))
    _lib.check("attn_fwd_varlen", st)
    return out, lse


def attn_splitkv_num_splits(B, H, Sq, Sk, d, dtype) -> int:
    """Split count for attn_fwd_splitkv chosen from the shape (1: do not split)."""
    return int(_lib.load().attn_splitkv_num_splits(B, H, Sq, Sk, d, int(dtype)))


def attn_splitkv_workspace_bytes(B, H, Sq, d, num_splits) -> int:
    return int(_lib.load().attn_splitkv_workspace_bytes(B, H, Sq, d, num_splits))


def attn_fwd_splitkv(q, k, v, num_splits, scale=None, causal=False, descales=(1.0, 1.0, 1.0),
                     ws=None, stream=None):
    """Per-chunk softmax states (m, l, u) of an n-way key split, in a workspace tensor."""
    B, H, Sq, Sk, d, dt = _qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = attn_splitkv_workspace_bytes(B, H, Sq, d, num_splits)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _same_device(q.device, ws=ws)
    qd, kd, vd = (float(x) for x in descales)
    st = _lib.load().attn_fwd_splitkv(ctypes_ptr(q), ctypes_ptr(k), ctypes_ptr(v), ctypes_ptr(ws),
                                      ws.numel() * ws.element_size(), int(num_splits), B, H, Sq,
                                      Sk, d, float(scale), int(causal), dt, qd, kd, vd,
                                      _stream(stream))
    _lib.check("attn_fwd_splitkv", st)
    return ws


def attn_merge(ws, num_splits, B, H, Sq, d, out=None, lse=None, stream=None):
    """Combine the chunk states of ``ws`` into (O, lse)."""
    dev = ws.device
    if out is None:
        out = torch.empty((B, H, Sq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    _out("out", out, (B, H, Sq, d), torch.float32, dev)
    _out("lse", lse, (B, H, Sq), torch.float32, dev)
    st = _lib.load().attn_merge(ctypes_ptr(ws), ws.numel() * ws.element_size(), int(num_splits),
                                ctypes_ptr(out), ctypes_ptr(lse), B, H, Sq, d, _stream(stream))
    _lib.check("attn_merge", st)
    return out, lse


def attn_fwd_splitkv_noalloc(q, k, v, num_splits, scale=None, causal=False,
                             descales=(1.0, 1.0, 1.0), out=None, lse=None, stream=None):
    """attn_fwd_splitkv + attn_merge in one library call whose chunk states live in the
    library's static device array (the C call allocates nothing; calls that overlap on one
    GPU race).  Returns (O, lse), float32."""
    B, H, Sq, Sk, d, dt = _qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Sq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _out("out", out, (B, H, Sq, d), torch.float32, q.device)
    _out("lse", lse, (B, H, Sq), torch.float32, q.device)
    qd, kd, vd = (float(x) for x in descales)
    st = _lib.load().attn_fwd_splitkv_noalloc(ctypes_ptr(q), ctypes_ptr(k), ctypes_ptr(v),
                                              ctypes_ptr(out), ctypes_ptr(lse), int(num_splits),
                                              B, H, Sq, Sk, d, float(scale), int(causal), dt,
                                              qd, kd, vd, _stream(stream))
    _lib.check("attn_fwd_splitkv_noalloc", st)
    return out, lse


def attn_bwd_workspace_bytes(B, H, Sq, Sk, d, causal=False) -> int:
    return int(_lib.load().attn_bwd_workspace_bytes(B, H, Sq, Sk, d, int(causal)))


def attn_bwd(q, k, v, o, lse, dout, scale=None, causal=False, dq=None, dk=None, dv=None,
             ws=None, stream=None):
    """Gradients (dQ, dK, dV), fp32, of O = attn_fwd(q, k, v) given O, lse and dO (fp32)."""
    B, H, Sq, Sk, d, dt = _qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for name, t, shape in (("o", o, (B, H, Sq, d)), ("dout", dout, (B, H, Sq, d)),
                           ("lse", lse, (B, H, Sq))):
        if tuple(t.shape) != shape or t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 {list(shape)}")
    dev = q.device
    _same_device(dev, o=o, dout=dout, lse=lse)
    if dq is None:
        dq = torch.empty((B, H, Sq, d), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty((B, H, Sk, d), dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty((B, H, Sk, d), dtype=torch.float32, device=dev)
    _out("dq", dq, (B, H, Sq, d), torch.float32, dev)
    _out("dk", dk, (B, H, Sk, d), torch.float32, dev)
    _out("dv", dv, (B, H, Sk, d), torch.float32, dev)
    if ws is None:
        ws = torch.empty(max(attn_bwd_workspace_bytes(B, H, Sq, Sk, d, causal), 16), dtype=torch.uint8,
                         device=dev)
    _same_device(dev, ws=ws)
    st = _lib.load().attn_bwd(ctypes_ptr(q), ctypes_ptr(k), ctypes_ptr(v), ctypes_ptr(o),
                              ctypes_ptr(dout), ctypes_ptr(lse), ctypes_ptr(dq), ctypes_ptr(dk),
                              ctypes_ptr(dv), ctypes_ptr(ws), ws.numel() * ws.element_size(),
                              B, H, Sq, Sk, d, float(scale), int(causal), dt, _stream(stream))
    _lib.check("attn_bwd", st)
    return dq, dk, dv


def attn_bwd_kernel_name(d, dtype, which):
    return _lib.load().attn_bwd_kernel_name(d, dtype, which).decode()


def workspace_views(ws, num_splits, B, H, Sq, d):
    """(m, l, u) views of a split-KV workspace, shaped [n,B,H,Sq], [n,B,H,Sq], [n,B,H,Sq,d]."""
    rows = B * H * Sq
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    ml = num_splits * rows * 4
    f = ws.view(torch.uint8)
    m = f[0:ml].view(torch.float32).view(num_splits, B, H, Sq)
    l_off = up(ml)
    l = f[l_off:l_off + ml].view(torch.float32).view(num_splits, B, H, Sq)
    u_off = l_off + up(ml)
    u = f[u_off:u_off + ml * d].view(torch.float32).view(num_splits, B, H, Sq, d)
    return m, l, u


def attn_block_m(B, H, Sq, Sk, d, causal, dtype, num_splits=0):
    return int(_lib.load().attn_block_m(B, H, Sq, Sk, d, int(causal), dtype, num_splits))


def attn_block_n(d, dtype):
    return int(_lib.load().attn_block_n(d, dtype))


def attn_num_workgroups(B, H, Sq, Sk, d, causal, dtype, num_splits=0):
    return int(_lib.load().attn_num_workgroups(B, H, Sq, Sk, d, int(causal), dtype, num_splits))


def attn_kernel_name(B, H, Sq, Sk, d, causal, dtype, num_splits=0):
    return _lib.load().attn_kernel_name(B, H, Sq, Sk, d, int(causal), dtype, num_splits).decode()


def attn_tune(q, k, v, scale=None, causal=False, reps=10, out=None, lse=None, stream=None):
    """Time every legal launch plan of attn_fwd for this shape (synchronous), keep the best
    for later attn_fwd calls with the same shape; returns the plan id."""
    B, H, Sq, Sk, d, dt = _qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Sq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _out("out", out, (B, H, Sq, d), torch.float32, q.device)
    _out("lse", lse, (B, H, Sq), torch.float32, q.device)
    plan = ctypes.c_int(-1)
    st = _lib.load().attn_tune(ctypes_ptr(q), ctypes_ptr(k), ctypes_ptr(v), ctypes_ptr(out),
                               ctypes_ptr(lse), B, H, Sq, Sk, d, float(scale), int(causal), dt,
                               int(reps), ctypes.byref(plan), _stream(stream))
    _lib.check("attn_tune", st)
    return plan.value


def attn_tune_splitkv(q, k, v, scale=None, causal=False, descales=(1.0, 1.0, 1.0), reps=10,
                      out=None, lse=None, stream=None):
    """Time split counts 1..64 of the split path (synchronous) and keep the best for
    attn_splitkv_num_splits; returns the count."""
    B, H, Sq, Sk, d, dt = _qkv(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Sq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _out("out", out, (B, H, Sq, d), torch.float32, q.device)
    _out("lse", lse, (B, H, Sq), torch.float32, q.device)
    n = ctypes.c_int(-1)
    qd, kd, vd = (float(x) for x in descales)
    st = _lib.load().attn_tune_splitkv(ctypes_ptr(q), ctypes_ptr(k), ctypes_ptr(v), ctypes_ptr(out),
                                       ctypes_ptr(lse), B, H, Sq, Sk, d, float(scale), int(causal),
                                       dt, qd, kd, vd, int(reps), ctypes.byref(n), _stream(stream))
    _lib.check("attn_tune_splitkv", st)
    return n.value


def attn_plan_get(B, H, Sq, Sk, d, causal, dtype) -> int:
    return int(_lib.load().attn_plan_get(B, H, Sq, Sk, d, int(causal), dtype))


def attn_plan_set(B, H, Sq, Sk, d, causal, dtype, plan) -> None:
    _lib.check("attn_plan_set", _lib.load().attn_plan_set(B, H, Sq, Sk, d, int(causal), dtype, int(plan)))


def attn_plan_clear() -> None:
    _lib.load().attn_plan_clear()


def plan_parts(plan: int):
    """(schedule, head_group) of a plan id."""
    return plan & 3, 1 << (plan >> 2)


def attn_status_string(status):
    return _lib.load().attn_status_string(status).decode()


def attn_last_hip_error():
    return int(_lib.load().attn_last_hip_error())
