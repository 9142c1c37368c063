"""GPU tests of dit_attn_fwd_ws (the bf16 forward pass with caller-provided
scratch, which splits the last wave of query tiles over the keys and merges
the pieces), through the C ABI, against the fp64 oracle.

Gates as for dit_attn_fwd: max|dO| <= 1e-2, max|dLSE|
<= 1e-3, relative RMS <= 1e-2; plus agreement with the unsplit launch, bitwise
repeatability, and the workspace error paths.  The split plan depends on the
device's compute-unit count; the shapes below are split on any GPU with at
least 8 compute units (checked in each test).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_non_causal_amd import _lib, functional as F, workloads as wl
from tests import _gpu
from tests._gpu import compare, dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


def _draw(B, H, Sq, Skv, d, seed):
    g = wl.generate("tiny", seed=seed, B=B, H=H, Sq=Sq, Skv=Skv, d=d)
    return g["q"], g["k"], g["v"]


def _ws_call(q, k, v, scale, ws, ws_bytes):
    B, Sq, H, d = q.shape
    Skv = k.shape[1]
    o = torch.empty((B, Sq, H, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    st = _lib.dit_attn_fwd_ws_status(q, k, v, o, lse, B, H, Sq, Skv, d, scale,
                                     _lib.DIT_DTYPE_BF16, ws, ws_bytes)
    return st, o, lse


SPLIT = [
    (1, 2, 256, 2048, 128),   # 4 query tiles, 32 key tiles each
    (2, 3, 300, 1000, 64),    # ragged query and key tails
    (1, 2, 129, 1000, 128),
    (1, 1, 1, 5000, 128),     # one query row, a key tail of 8
]


@pytest.mark.parametrize("B,H,Sq,Skv,d", SPLIT)
def test_ws_split_full_compare(B, H, Sq, Skv, d):
    say(f"fwd_ws split B{B} H{H} Sq{Sq} Skv{Skv} d{d}")
    n = _lib.dit_attn_fwd_workspace_size(B, H, Sq, Skv, d)
    assert n > 0, "this shape is expected to be split"
    q, k, v = _draw(B, H, Sq, Skv, d, seed=3000 + Sq + Skv + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    ws = torch.empty(n, dtype=torch.uint8, device=qd.device)
    st, o, l = _ws_call(qd, kd, vd, scale, ws, n)
    assert st == _lib.DIT_OK
    o_plain, l_plain = F.attention(qd, kd, vd, scale, workspace=None)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn_fwd(q, k, v, scale)
    compare(host_f64(o), host_f64(l), o_ref, l_ref, what=f"split B{B}H{H}Sq{Sq}Skv{Skv}d{d}")
    # against the unsplit launch: both are within the gate of the oracle; the
    # split changes only the summation order
    d_o = np.abs(host_f64(o) - host_f64(o_plain)).max()
    d_l = np.abs(host_f64(l) - host_f64(l_plain)).max()
    say(f"  split vs unsplit: max|dO| {d_o:.2e} max|dLSE| {d_l:.2e}")
    assert d_o <= 2 * _gpu.BF16_O_TOL and d_l <= 2e-3


def test_ws_deterministic():
    say("fwd_ws determinism")
    B, H, Sq, Skv, d = 1, 2, 256, 2048, 128
    q, k, v = _draw(B, H, Sq, Skv, d, seed=3101)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    n = _lib.dit_attn_fwd_workspace_size(B, H, Sq, Skv, d)
    ws = torch.empty(n, dtype=torch.uint8, device=qd.device)
    outs = []
    for i in range(5):
        ws.fill_(i)  # the workspace contents on entry must not matter
        st, o, l = _ws_call(qd, kd, vd, 0.088, ws, n)
        assert st == _lib.DIT_OK
        outs.append((o, l))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])


def test_ws_unsplit_shape_needs_no_workspace():
    """A shape with nothing to split needs no workspace (NULL is fine) and
    gives exactly the result of dit_attn_fwd."""
    say("fwd_ws without a split")
    B, H, Sq, Skv, d = 1, 2, 256, 64, 64
    assert _lib.dit_attn_fwd_workspace_size(B, H, Sq, Skv, d) == 0
    q, k, v = _draw(B, H, Sq, Skv, d, seed=3102)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    st, o, l = _ws_call(qd, kd, vd, 0.125, None, 0)
    assert st == _lib.DIT_OK
    o2, l2 = F.attention(qd, kd, vd, 0.125, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l, l2)


def test_ws_errors():
    say("fwd_ws workspace errors")
    B, H, Sq, Skv, d = 1, 2, 256, 2048, 128
    q, k, v = _draw(B, H, Sq, Skv, d, seed=3103)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    n = _lib.dit_attn_fwd_workspace_size(B, H, Sq, Skv, d)
    assert n > 0
    ws = torch.empty(n + 64, dtype=torch.uint8, device=qd.device)
    assert _ws_call(qd, kd, vd, 0.1, None, 0)[0] == _lib.DIT_ERR_WORKSPACE
    assert _ws_call(qd, kd, vd, 0.1, ws, n - 16)[0] == _lib.DIT_ERR_WORKSPACE
    assert _ws_call(qd, kd, vd, 0.1, ws.data_ptr() + 8, n)[0] == _lib.DIT_ERR_WORKSPACE
    # workspace overlapping an input or an output
    assert _ws_call(qd, kd, vd, 0.1, kd, n)[0] == _lib.DIT_ERR_WORKSPACE
    o = torch.empty((B, Sq, H, d), dtype=torch.bfloat16, device=qd.device)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=qd.device)
    st = _lib.dit_attn_fwd_ws_status(qd, kd, vd, o, lse, B, H, Sq, Skv, d, 0.1,
                                     _lib.DIT_DTYPE_BF16, o, n)
    assert st == _lib.DIT_ERR_WORKSPACE
    torch.cuda.synchronize()


def test_benchmark_shape_is_split():
    """The FLUX-like workload (d = 128: 256-row query tiles, one workgroup per
    CU) leaves a partial last wave (1584 tiles) on this GPU, so the launch
    bench.py times splits it."""
    W = wl.WORKLOADS["flux"]
    n = _lib.dit_attn_fwd_workspace_size(W.B, W.H, W.Sq, W.Skv, W.d)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"flux workspace {n} bytes on {n_cu} compute units")
    tiles = (W.Sq + 255) // 256 * W.H * W.B
    if tiles % n_cu and 2 * (tiles % n_cu) <= n_cu:
        assert n > 0
