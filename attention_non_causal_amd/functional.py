"""torch-facing helpers: allocate outputs with torch and call the C ABI.

Marshalling only -- the computation is the library's HIP kernels.  Tensors
are contiguous [B, S, H, d] on a ROCm device; LSE is fp32 [B, H, Sq].

``stream``: None (torch's current stream), a torch stream, or a raw HIP stream
handle (0: the null stream).  Every allocation a helper makes (outputs,
workspaces) and every fill happens on that same stream, so the caching
allocator and the kernels agree on the order of the work.
"""
from __future__ import annotations

import contextlib
import math

from . import _lib


def _on_stream(stream, device):
    """(context manager making `stream` torch's current stream, the stream
    argument to pass to the binding)."""
    import torch
    if stream is None:
        return contextlib.nullcontext(), None
    if isinstance(stream, int):
        ts = torch.cuda.ExternalStream(stream, device=device) if stream else \
            torch.cuda.default_stream(device)
    else:
        ts = stream
    return torch.cuda.stream(ts), ts


def _require(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B,S,H,d]")


def workspace_for(q, k, dtype=None):
    """A workspace tensor for dit_attn_fwd_ws on q's shape (None if none is needed)."""
    import torch
    B, Sq, H, d = q.shape
    Skv = k.shape[1]
    dt = _lib.DIT_DTYPE_BF16 if dtype is None else dtype
    n = _lib.dit_attn_fwd_workspace_size(B, H, Sq, Skv, d, dt)
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n else None


def attention(q, k, v, scale: float | None = None, out=None, lse=None, stream=None,
              workspace="auto"):
    """bf16 non-causal attention: returns (o bf16 [B,Sq,H,d], lse fp32 [B,H,Sq]).

    workspace: "auto" (default) allocates the scratch dit_attn_fwd_ws needs and
    balances the last wave of workgroups; a uint8 device tensor is used as that
    scratch; None calls dit_attn_fwd (no scratch, no split)."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _require(t, torch.bfloat16, n)
    B, Sq, H, d = q.shape
    Skv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ctx, stream = _on_stream(stream, q.device)
    with ctx:
        if out is None:
            out = torch.empty((B, Sq, H, d), dtype=torch.bfloat16, device=q.device)
        if lse is None:
            lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
        if workspace is None:
            _lib.dit_attn_fwd(q, k, v, out, lse, B, H, Sq, Skv, d, scale, _lib.DIT_DTYPE_BF16,
                              stream)
            return out, lse
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError("workspace must be 'auto', None or a uint8 device tensor")
            workspace = workspace_for(q, k)
        n_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _lib.dit_attn_fwd_ws(q, k, v, out, lse, B, H, Sq, Skv, d, scale, _lib.DIT_DTYPE_BF16,
                             workspace, n_bytes, stream)
    return out, lse


def quantize_fp8(x, stream=None):
    """Per-(b, h, 128-token) e4m3 quantisation: returns (x8 uint8 [B,S,H,d],
    scale fp32 [B,H,ceil(S/128)])."""
    import torch
    _require(x, torch.bfloat16, "x")
    B, S, H, d = x.shape
    ctx, stream = _on_stream(stream, x.device)
    with ctx:
        x8 = torch.empty((B, S, H, d), dtype=torch.uint8, device=x.device)
        nblk = (S + _lib.DIT_FP8_BLOCK - 1) // _lib.DIT_FP8_BLOCK
        sc = torch.empty((B, H, nblk), dtype=torch.float32, device=x.device)
        _lib.dit_quant_fp8(x, x8, sc, B, H, S, d, stream)
    return x8, sc


def attention_fp8(q8, q_scale, k8, k_scale, v8, v_scale, scale: float | None = None,
                  out=None, lse=None, stream=None, workspace="auto"):
    """fp8 (e4m3) non-causal attention on quantised inputs from quantize_fp8.

    workspace: as for attention ("auto": dit_attn_fwd_ws with allocated
    scratch; a uint8 device tensor: that scratch; None: dit_attn_fwd)."""
    import torch
    B, Sq, H, d = q8.shape
    Skv = k8.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = _lib.fp8_tensor(q8, q_scale)
    dk = _lib.fp8_tensor(k8, k_scale)
    dv = _lib.fp8_tensor(v8, v_scale)
    ctx, stream = _on_stream(stream, q8.device)
    with ctx:
        if out is None:
            out = torch.empty((B, Sq, H, d), dtype=torch.bfloat16, device=q8.device)
        if lse is None:
            lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q8.device)
        if workspace is None:
            _lib.dit_attn_fwd(dq, dk, dv, out, lse, B, H, Sq, Skv, d, scale,
                              _lib.DIT_DTYPE_FP8_E4M3, stream)
            return out, lse
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError("workspace must be 'auto', None or a uint8 device tensor")
            workspace = workspace_for(q8, k8, _lib.DIT_DTYPE_FP8_E4M3)
        n_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _lib.dit_attn_fwd_ws(dq, dk, dv, out, lse, B, H, Sq, Skv, d, scale,
                             _lib.DIT_DTYPE_FP8_E4M3, workspace, n_bytes, stream)
    return out, lse


def merge(o_parts, lse_parts, out=None, lse=None, stream=None):
    """LSE-merge of partial results (lists of bf16 [B,Sq,H,d] / fp32 [B,H,Sq])."""
    import torch
    B, Sq, H, d = o_parts[0].shape
    ctx, stream = _on_stream(stream, o_parts[0].device)
    with ctx:
        if out is None:
            out = torch.empty_like(o_parts[0])
        if lse is None:
            lse = torch.empty_like(lse_parts[0])
        _lib.dit_attn_merge(o_parts, lse_parts, len(o_parts), out, lse, B, H, Sq, d, stream)
    return out, lse


def attention_acc(q, k, v, out, lse, scale: float | None = None, stream=None,
                  workspace="auto", kv_batch_tokens: int = 0):
    """Merge bf16 attention over the keys k/v into the running result (out,
    lse) over earlier keys (dit_attn_fwd_acc): rows whose lse is -inf have no
    keys yet.  k, v: tensors, or (pointer, Skv) pairs for a block of larger
    tensors whose batches lie kv_batch_tokens tokens apart (0: Skv).
    workspace as for attention."""
    import torch
    _require(q, torch.bfloat16, "q")
    B, Sq, H, d = q.shape
    if isinstance(k, tuple):
        (k, Skv), (v, _) = k, v
    else:
        for t, n in ((k, "k"), (v, "v")):
            _require(t, torch.bfloat16, n)
        Skv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ctx, stream = _on_stream(stream, q.device)
    with ctx:
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError("workspace must be 'auto', None or a uint8 device tensor")
            n = _lib.dit_attn_fwd_workspace_size(B, H, Sq, Skv, d, _lib.DIT_DTYPE_BF16)
            workspace = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
        n_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _lib.dit_attn_fwd_acc(q, k, v, out, lse, B, H, Sq, Skv, d, scale, _lib.DIT_DTYPE_BF16,
                              kv_batch_tokens, workspace, n_bytes, stream)
    return out, lse


def attention_fp8_acc(q8, q_scale, k8, k_scale, v8, v_scale, out, lse,
                      scale: float | None = None, stream=None, workspace="auto"):
    """Merge fp8 attention over one key block (its own e4m3 tensor and block
    scales, from quantize_fp8) into the running result (out, lse) over earlier
    keys (dit_attn_fwd_acc with DIT_DTYPE_FP8_E4M3): rows whose lse is -inf
    have no keys yet.  workspace as for attention."""
    import torch
    B, Sq, H, d = q8.shape
    Skv = k8.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = _lib.fp8_tensor(q8, q_scale)
    dk = _lib.fp8_tensor(k8, k_scale)
    dv = _lib.fp8_tensor(v8, v_scale)
    ctx, stream = _on_stream(stream, q8.device)
    with ctx:
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError("workspace must be 'auto', None or a uint8 device tensor")
            workspace = workspace_for(q8, k8, _lib.DIT_DTYPE_FP8_E4M3)
        n_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _lib.dit_attn_fwd_acc(dq, dk, dv, out, lse, B, H, Sq, Skv, d, scale,
                              _lib.DIT_DTYPE_FP8_E4M3, 0, workspace, n_bytes, stream)
    return out, lse


def ring_share_attention_acc(q, k, v, n_chunks: int, scale: float | None = None, out=None,
                             lse=None, workspace="auto", stream=None):
    """One ring rank's share as a ring loop runs it: the running result starts
    empty (lse = -inf) and each of ``n_chunks`` consecutive KV chunks is merged
    into it as it is processed (dit_attn_fwd_acc on pointer offsets into k/v,
    batches Skv tokens apart, so any B) -- no partial outputs, no separate
    merge.  The reset of lse, the allocations and the launches all run on
    ``stream``."""
    import torch
    B, Sq, H, d = q.shape
    Skv = k.shape[1]
    if Skv % n_chunks:
        raise ValueError("Skv must be a multiple of n_chunks")
    c = Skv // n_chunks
    ctx, stream = _on_stream(stream, q.device)
    with ctx:
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError("workspace must be 'auto', None or a uint8 device tensor")
            n = _lib.dit_attn_fwd_workspace_size(B, H, Sq, c, d, _lib.DIT_DTYPE_BF16)
            workspace = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
        lse.fill_(-math.inf)
        es = k.element_size()
        for i in range(n_chunks):
            off = i * c * H * d * es
            attention_acc(q, (k.data_ptr() + off, c), (v.data_ptr() + off, c), out, lse, scale,
                          stream, workspace, kv_batch_tokens=Skv)
    return out, lse


def ring_share_attention(q, k, v, n_chunks: int, scale: float | None = None, parts=None,
                         out=None, lse=None, stream=None):
    """One ring rank's share of ring attention, run locally: the local queries
    attend to each of ``n_chunks`` consecutive KV chunks (one forward launch
    each, on pointer offsets into k/v, so B must be 1), then the partials are
    merged.  ``parts`` = optional preallocated (o_parts, lse_parts) lists."""
    import torch
    B, Sq, H, d = q.shape
    Skv = k.shape[1]
    if B != 1:
        raise ValueError("KV chunks are pointer offsets: B must be 1")
    if Skv % n_chunks:
        raise ValueError("Skv must be a multiple of n_chunks")
    c = Skv // n_chunks
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ctx, stream = _on_stream(stream, q.device)
    with ctx:
        if parts is None:
            o_parts = [torch.empty_like(q) for _ in range(n_chunks)]
            lse_parts = [torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
                         for _ in range(n_chunks)]
        else:
            o_parts, lse_parts = parts
        es = k.element_size()
        for i in range(n_chunks):
            off = i * c * H * d * es
            _lib.dit_attn_fwd(q, k.data_ptr() + off, v.data_ptr() + off, o_parts[i],
                              lse_parts[i], B, H, Sq, c, d, scale, _lib.DIT_DTYPE_BF16, stream)
        return merge(o_parts, lse_parts, out, lse, stream)
