"""GPU tests of dit_attn_fwd_noalloc (the split forward launch with the
library's static per-GPU scratch instead of a caller workspace), through the C
ABI: its results must equal those of dit_attn_fwd_ws -- the same kernels on the
same split plan, so bit for bit -- on two calls in a row, the second with a
smaller input (the scratch keeps the first call's contents), and match the
fp64 oracle within the bf16 tolerances.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_non_causal_amd import _lib, functional as F, workloads as wl
from tests._gpu import compare, dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


def _outputs(B, Sq, H, d, dev):
    """Outputs poisoned with NaN, so that anything left unwritten shows."""
    o = torch.full((B, Sq, H, d), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=dev)
    return o, lse


def _noalloc(q, k, v, scale):
    B, Sq, H, d = q.shape
    Skv = k.shape[1]
    o, lse = _outputs(B, Sq, H, d, q.device)
    st = _lib.dit_attn_fwd_noalloc_status(q, k, v, o, lse, B, H, Sq, Skv, d, scale,
                                          _lib.DIT_DTYPE_BF16)
    return st, o, lse


def _ws(q, k, v, scale):
    B, Sq, H, d = q.shape
    Skv = k.shape[1]
    o, lse = _outputs(B, Sq, H, d, q.device)
    ws = F.workspace_for(q, k)
    n = 0 if ws is None else ws.numel()
    _lib.dit_attn_fwd_ws(q, k, v, o, lse, B, H, Sq, Skv, d, scale, _lib.DIT_DTYPE_BF16, ws, n)
    return o, lse


def _same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_noalloc_two_calls_bf16():
    """FLUX-like full size (the largest scratch use of the workloads), then a
    smaller split shape: each equal to dit_attn_fwd_ws bit for bit."""
    W = wl.WORKLOADS["flux"]
    say("noalloc bf16 call 1: FLUX-like B1 H24 S16896 d128")
    g = wl.generate(W)
    q, k, v = dev_bf16(g["q"]), dev_bf16(g["k"]), dev_bf16(g["v"])
    n = _lib.dit_attn_fwd_workspace_size(W.B, W.H, W.Sq, W.Skv, W.d)
    say(f"  split scratch {n} bytes of {_lib.DIT_NOALLOC_SCRATCH_BYTES}")
    assert 0 < n <= _lib.DIT_NOALLOC_SCRATCH_BYTES
    st, o1, l1 = _noalloc(q, k, v, W.scale)
    assert st == _lib.DIT_OK
    o1r, l1r = _ws(q, k, v, W.scale)
    torch.cuda.synchronize()
    assert _same(o1, o1r) and _same(l1, l1r)
    rows = wl.sample_rows(W.Sq, 16)
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], W.scale, rows=rows)
    compare(host_f64(o1)[:, rows], host_f64(l1)[:, :, rows], o_ref, l_ref, what="noalloc flux")
    del q, k, v, o1, l1, o1r, l1r

    B, H, Sq, Skv, d = 1, 2, 256, 2048, 128
    say(f"noalloc bf16 call 2: B{B} H{H} Sq{Sq} Skv{Skv} d{d}")
    assert _lib.dit_attn_fwd_workspace_size(B, H, Sq, Skv, d) > 0, "expected to be split"
    g = wl.generate("tiny", seed=6100, B=B, H=H, Sq=Sq, Skv=Skv, d=d)
    q, k, v = dev_bf16(g["q"]), dev_bf16(g["k"]), dev_bf16(g["v"])
    scale = float(np.float32(1 / math.sqrt(d)))
    st, o2, l2 = _noalloc(q, k, v, scale)
    assert st == _lib.DIT_OK
    o2r, l2r = _ws(q, k, v, scale)
    torch.cuda.synchronize()
    assert _same(o2, o2r) and _same(l2, l2r)
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], scale)
    compare(host_f64(o2), host_f64(l2), o_ref, l_ref, what="noalloc small")


def test_noalloc_two_calls_fp8():
    """The fp8 split launch (pieces of 128-row tiles), a larger then a smaller
    shape, each equal to dit_attn_fwd_ws bit for bit."""
    for B, H, Sq, Skv, d, seed in ((1, 6, 1024, 4096, 128, 6200), (1, 2, 256, 2048, 64, 6201)):
        say(f"noalloc fp8 B{B} H{H} Sq{Sq} Skv{Skv} d{d}")
        n = _lib.dit_attn_fwd_workspace_size(B, H, Sq, Skv, d, _lib.DIT_DTYPE_FP8_E4M3)
        assert 0 < n <= _lib.DIT_NOALLOC_SCRATCH_BYTES, n
        g = wl.generate("flux", seed=seed, B=B, H=H, Sq=Sq, Skv=Skv, d=d)
        q8, qs = F.quantize_fp8(dev_bf16(g["q"]))
        k8, ks = F.quantize_fp8(dev_bf16(g["k"]))
        v8, vs = F.quantize_fp8(dev_bf16(g["v"]))
        scale = float(np.float32(1 / math.sqrt(d)))
        o, lse = _outputs(B, Sq, H, d, q8.device)
        st = _lib.dit_attn_fwd_noalloc_status(_lib.fp8_tensor(q8, qs), _lib.fp8_tensor(k8, ks),
                                              _lib.fp8_tensor(v8, vs), o, lse, B, H, Sq, Skv,
                                              d, scale, _lib.DIT_DTYPE_FP8_E4M3)
        assert st == _lib.DIT_OK
        o_r, l_r = F.attention_fp8(q8, qs, k8, ks, v8, vs, scale)
        torch.cuda.synchronize()
        assert _same(o, o_r) and _same(lse, l_r)


def test_noalloc_unsplit_and_errors():
    """A shape with nothing to split never touches the scratch and equals
    dit_attn_fwd; invalid arguments are rejected before any launch."""
    B, H, Sq, Skv, d = 1, 2, 256, 64, 64
    say("noalloc unsplit shape")
    assert _lib.dit_attn_fwd_workspace_size(B, H, Sq, Skv, d) == 0
    g = wl.generate("tiny", seed=6300, B=B, H=H, Sq=Sq, Skv=Skv, d=d)
    q, k, v = dev_bf16(g["q"]), dev_bf16(g["k"]), dev_bf16(g["v"])
    st, o, l = _noalloc(q, k, v, 0.125)
    assert st == _lib.DIT_OK
    o2, l2 = F.attention(q, k, v, 0.125, workspace=None)
    torch.cuda.synchronize()
    assert _same(o, o2) and _same(l, l2)
    assert _lib.dit_attn_fwd_noalloc_status(q, k, None, o, l, B, H, Sq, Skv, d, 0.125) == \
        _lib.DIT_ERR_NULL
    assert _lib.dit_attn_fwd_noalloc_status(q, k, v, o, l, B, H, Sq, Skv, 96, 0.125) == \
        _lib.DIT_ERR_UNSUPPORTED
    assert _lib.dit_attn_fwd_noalloc_status(q, k, v, q, l, B, H, Sq, Skv, d, 0.125) == \
        _lib.DIT_ERR_ALIAS
    torch.cuda.synchronize()
