"""GPU tests of dit_attn_fwd_acc (the bf16 forward pass over one block of keys
merged into a running result), through the C ABI, against the fp64 oracle
run on all the keys at once.

Gates as for dit_attn_fwd: max|dO| <= 1e-2, max|dLSE| <= 1e-3, relative RMS
<= 1e-2.  Where a block of at most 8 keys makes |O| as large as |V| the O
budget is the bound of the arithmetic: each block's weights rounded to bf16 before P.V (<= 2^-9
relative) and the running O rounded to bf16 after each of the n blocks
(<= 2^-9 |O| each), so |dO| <= (n + 1) 2^-9 max|V|.
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


def _o_tol(v_bits, bounds):
    """1e-2, or, when a block holds at most FEW_KEYS keys (its O can then be
    as large as |V|), the bound of the arithmetic (n + 1) 2^-9 max|V|."""
    n_blocks = len(bounds) - 1
    if min(b - a for a, b in zip(bounds[:-1], bounds[1:])) > _gpu.FEW_KEYS:
        return _gpu.BF16_O_TOL
    vmax = float(np.abs((np.asarray(v_bits, dtype=np.uint16).astype(np.uint32) << 16)
                        .view(np.float32)).max())
    return max(_gpu.BF16_O_TOL, (n_blocks + 1) * 2.0 ** -9 * vmax)


def _acc_blocks(qd, kd, vd, bounds, scale, o, lse):
    """Merge attention over key blocks [bounds[i], bounds[i+1]) into (o, lse):
    each block is a pointer offset into k/v, whose batches lie Skv tokens apart."""
    B, Sq, H, d = qd.shape
    Skv = kd.shape[1]
    es = kd.element_size()
    for a, b in zip(bounds[:-1], bounds[1:]):
        off = a * H * d * es
        F.attention_acc(qd, (kd.data_ptr() + off, b - a), (vd.data_ptr() + off, b - a), o, lse,
                        scale, kv_batch_tokens=Skv)


@pytest.mark.parametrize("B,Sq,bounds,d", [
    (1, 300, [0, 300, 700, 1000], 64),   # uneven blocks with ragged tails
    (1, 129, [0, 64, 1000], 128),        # one block of a single key tile
    (1, 256, [0, 1, 2, 700], 128),       # blocks of one key
    (1, 70, [0, 4000, 8000], 128),       # two long blocks (split launches)
    (2, 100, [0, 300, 700, 1000], 128),  # batches: blocks are strided slices
    (3, 77, [0, 129, 500], 64),
])
def test_acc_blocks_equal_attention_over_all_keys(B, Sq, bounds, d):
    H, Skv = 2, bounds[-1]
    say(f"fwd_acc blocks {bounds} Sq{Sq} d{d}")
    q, k, v = _draw(B, H, Sq, Skv, d, seed=5000 + Sq + Skv + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o = torch.full((B, Sq, H, d), float("nan"), dtype=torch.bfloat16, device=qd.device)
    lse = torch.full((B, H, Sq), -math.inf, dtype=torch.float32, device=qd.device)
    _acc_blocks(qd, kd, vd, bounds, scale, o, lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn_fwd(q, k, v, scale)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, o_tol=_o_tol(v, bounds),
            what=f"acc blocks {bounds} d{d}")


@pytest.mark.parametrize("B,H,Sq,Skv,d", [(2, 3, 300, 333, 64), (1, 2, 256, 2048, 128)])
def test_acc_into_empty_result_is_the_plain_forward(B, H, Sq, Skv, d):
    """With no running result (LSE -inf; its O, here NaN, is never read) the
    call writes exactly what dit_attn_fwd_ws writes (the second shape is split
    over the keys on any GPU with >= 8 CUs, so the merge kernel's path is
    covered too)."""
    say(f"fwd_acc into an empty result B{B} H{H} Sq{Sq} Skv{Skv} d{d}")
    q, k, v = _draw(B, H, Sq, Skv, d, seed=5100 + Skv)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    scale = 0.09
    n = _lib.dit_attn_fwd_workspace_size(B, H, Sq, Skv, d)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device=qd.device)
    o_ref = torch.empty((B, Sq, H, d), dtype=torch.bfloat16, device=qd.device)
    l_ref = torch.empty((B, H, Sq), dtype=torch.float32, device=qd.device)
    _lib.dit_attn_fwd_ws(qd, kd, vd, o_ref, l_ref, B, H, Sq, Skv, d, scale, _lib.DIT_DTYPE_BF16,
                         ws, n)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, -math.inf)
    _lib.dit_attn_fwd_acc(qd, kd, vd, o, lse, B, H, Sq, Skv, d, scale, _lib.DIT_DTYPE_BF16,
                          workspace=ws, workspace_bytes=n)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, l_ref)


def test_acc_equals_merge_of_two_forwards():
    """Merging a block into a result is the two-part dit_attn_merge, except
    that the block's own O is not rounded to bf16 first: before their final
    rounding the two differ by at most that rounding (2^-9 |O_2|, times a
    weight <= 1), and each final rounding moves a value by at most half an ulp
    -- together one ulp, <= 2^-7 |O| for bf16."""
    B, H, Sq, Skv, d = 1, 3, 200, 900, 128
    say("fwd_acc vs fwd + merge")
    q, k, v = _draw(B, H, Sq, Skv, d, seed=5200)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    scale = 0.088
    half = 500
    o1, l1 = F.attention(qd, kd[:, :half].contiguous(), vd[:, :half].contiguous(), scale)
    o2, l2 = F.attention(qd, kd[:, half:].contiguous(), vd[:, half:].contiguous(), scale)
    om, lm = F.merge([o1, o2], [l1, l2])
    oa, la = o1.clone(), l1.clone()
    F.attention_acc(qd, kd[:, half:].contiguous(), vd[:, half:].contiguous(), oa, la, scale)
    torch.cuda.synchronize()
    d_o = np.abs(host_f64(oa) - host_f64(om))
    bound = 2.0 ** -9 * np.abs(host_f64(o2)) + 2.0 ** -7 * np.abs(host_f64(om)) + 1e-6
    assert (d_o <= bound).all(), f"max excess {(d_o - bound).max():.3e}"
    assert np.abs(host_f64(la) - host_f64(lm)).max() <= 1e-5


def test_acc_errors():
    B, H, Sq, Skv, d = 1, 2, 256, 2048, 128
    q, k, v = _draw(B, H, Sq, Skv, d, seed=5300)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o = torch.empty((B, Sq, H, d), dtype=torch.bfloat16, device=qd.device)
    lse = torch.full((B, H, Sq), -math.inf, dtype=torch.float32, device=qd.device)
    n = _lib.dit_attn_fwd_workspace_size(B, H, Sq, Skv, d)
    assert n > 0, "this shape is expected to be split"
    st = _lib.dit_attn_fwd_acc_status(qd, kd, vd, o, lse, B, H, Sq, Skv, d, 0.1,
                                      _lib.DIT_DTYPE_BF16)
    assert st == _lib.DIT_ERR_WORKSPACE
    torch.cuda.synchronize()


def test_wan_ring_share_accumulated_full_size():
    """The Wan-like ring share as a ring loop runs it: 4 KV chunks merged into
    the running result one after another (no partial outputs, no separate
    merge), against the oracle over all 32760 keys on sampled rows."""
    W = wl.WORKLOADS["wan_ring"]
    say("wan ring share (accumulated): generating inputs")
    g = wl.generate("wan_ring")
    q, k, v = dev_bf16(g["q"]), dev_bf16(g["k"]), dev_bf16(g["v"])
    say("wan ring share (accumulated): 4 chunk forwards merged as they run")
    o, l = F.ring_share_attention_acc(q, k, v, W.n_chunks, W.scale)
    torch.cuda.synchronize()
    # the first query tile (256 rows) and 8 more rows
    rows = _gpu.tile_rows(W.Sq, (0,), extra=8)
    say(f"wan ring share (accumulated): oracle on {len(rows)} rows")
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], W.scale, rows=rows)
    compare(host_f64(o)[:, rows], host_f64(l)[:, :, rows], o_ref, l_ref, what="wan_ring_acc")


def test_ring_share_accumulated_on_a_side_stream():
    """ring_share_attention_acc given a stream that is not torch's current one:
    the reset of the running LSE, the workspace and the four launches all run
    on that stream, in order (the output LSE starts out poisoned with NaN)."""
    say("ring share (accumulated) on a side stream")
    g = wl.generate("wan_ring", seed=5400, Sq=300, Skv=2400)
    scale = float(np.float32(1 / math.sqrt(128)))
    q, k, v = dev_bf16(g["q"]), dev_bf16(g["k"]), dev_bf16(g["v"])
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, q.shape[2], q.shape[1]), float("nan"), dtype=torch.float32,
                     device=q.device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    F.ring_share_attention_acc(q, k, v, 4, scale, out=o, lse=lse, stream=s)
    s.synchronize()
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], scale)
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, what="ring acc side stream")


# ------------------------------------------------------------------ fp8

def _fp8_blocks(g, bounds):
    """Quantise Q once and every key block [a, b) of K and V on its own (a ring
    rank quantises each arriving block by itself)."""
    q8, qs = F.quantize_fp8(dev_bf16(g["q"]))
    blocks = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        kb = np.ascontiguousarray(g["k"][:, a:b])
        vb = np.ascontiguousarray(g["v"][:, a:b])
        k8, ks = F.quantize_fp8(dev_bf16(kb))
        v8, vs = F.quantize_fp8(dev_bf16(vb))
        blocks.append((kb, vb, k8, ks, v8, vs))
    return q8, qs, blocks


@pytest.mark.parametrize("B,H,Sq,bounds,d", [
    (1, 2, 300, [0, 700, 1000, 2048], 128),   # a split block (2048 - 1000 keys)
    (2, 3, 129, [0, 129, 500], 64),
    (1, 2, 256, [0, 2048, 4096], 128),        # two split blocks
])
def test_fp8_acc_blocks_against_oracle(B, H, Sq, bounds, d):
    """fp8 key blocks merged into a running result one after another, on
    unit-normal inputs (RMS-normalised Q/K, N(0,1) V):
    * against the oracle over all keys on the unquantised inputs: max|dO| <= 6e-2;
    * against the oracle on the dequantised inputs, per element: the blocks'
      own kernel bounds (tests/test_gpu_fp8.kernel_bound), weighted by each
      block's share exp(LSE_c - M) / sum, plus what the merge adds -- the
      blocks' LSE errors moving the shares (2 delta max_c |O_c|) and the bf16
      rounding of the running O after each block ((n + 1) 2^-9 max_c |O_c|);
      LSE within the blocks' largest LSE bound (tests/test_gpu_fp8.lse_bound;
      the log-sum-exp merge does not enlarge a max-norm error)."""
    from tests.test_gpu_fp8 import dequant, kernel_bound, lse_bound
    Skv = bounds[-1]
    say(f"fp8 acc blocks {bounds} B{B} H{H} Sq{Sq} d{d}")
    g = wl.generate("flux", seed=5500 + Sq + Skv + d, B=B, H=H, Sq=Sq, Skv=Skv, d=d)
    scale = float(np.float32(1 / math.sqrt(d)))
    q8, qs, blocks = _fp8_blocks(g, bounds)
    o = torch.full((B, Sq, H, d), float("nan"), dtype=torch.bfloat16, device=q8.device)
    lse = torch.full((B, H, Sq), -math.inf, dtype=torch.float32, device=q8.device)
    for _, _, k8, ks, v8, vs in blocks:
        F.attention_fp8_acc(q8, qs, k8, ks, v8, vs, o, lse, scale)
    torch.cuda.synchronize()
    og, lg = host_f64(o), host_f64(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], scale)
    compare(og, lg, o_ref, l_ref, o_tol=_gpu.FP8_O_TOL, lse_tol=5e-2, rel_rms=None,
            what=f"fp8 acc {bounds} vs unquantised")
    qd = dequant(g["q"])
    parts = []
    for kb, vb, *_ in blocks:
        kd, vd = dequant(kb), dequant(vb)
        oc, lc = oracle.attn_fwd(qd, kd, vd, scale)
        parts.append((oc, lc, kernel_bound(qd, kd, vd, scale), lse_bound(qd, kd, scale)))
    lse_c = np.stack([p[1] for p in parts])                  # [n, B, H, Sq]
    w = np.exp(lse_c - lse_c.max(0))
    w = (w / w.sum(0)).transpose(0, 1, 3, 2)[..., None]      # [n, B, Sq, H, 1]
    o_c = np.stack([p[0] for p in parts])                    # [n, B, Sq, H, d]
    o_dq = (w * o_c).sum(0)
    l_dq = lse_c.max(0) + np.log(np.exp(lse_c - lse_c.max(0)).sum(0))
    lb = np.stack([p[3] for p in parts]).max(0)               # [B, H, Sq]
    delta = lb.max()
    omax = np.abs(o_c).max(0)
    bound = (w * np.stack([p[2] for p in parts])).sum(0) \
        + (2 * delta + (len(parts) + 1) * 2.0 ** -9) * omax + 1e-6
    err = np.abs(og - o_dq)
    say(f"  vs dequantised: max|dO| {err.max():.3e} (worst err/bound {(err / bound).max():.3f}) "
        f"max|dLSE| {np.abs(lg - l_dq).max():.3e}")
    assert (err <= bound).all(), "fp8 acc: kernel error exceeds its bound"
    assert (np.abs(lg - l_dq) <= lb).all()


def test_fp8_acc_into_empty_result_is_the_plain_forward():
    """With no running result (LSE -inf, O poisoned with NaN and never read)
    the fp8 call writes exactly what dit_attn_fwd_ws writes, plain and split."""
    for B, H, Sq, Skv, d in ((2, 3, 300, 333, 64), (1, 2, 256, 2048, 128)):
        say(f"fp8 acc into an empty result B{B} H{H} Sq{Sq} Skv{Skv} d{d}")
        g = wl.generate("flux", seed=5600 + Skv, B=B, H=H, Sq=Sq, Skv=Skv, d=d)
        q8, qs, [(_, _, k8, ks, v8, vs)] = _fp8_blocks(g, [0, Skv])
        o_ref, l_ref = F.attention_fp8(q8, qs, k8, ks, v8, vs, 0.09)
        o = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(l_ref, -math.inf)
        F.attention_fp8_acc(q8, qs, k8, ks, v8, vs, o, lse, 0.09)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(lse, l_ref)
