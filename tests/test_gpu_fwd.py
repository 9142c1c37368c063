"""GPU parity of the bf16 forward pass (dit_attn_fwd through the C ABI) against
the fp64 oracle on the same seeded bf16 bytes.

Gates: max|dO| <= 1e-2, max|dLSE| <= 1e-3, plus the internal relative-RMS gate
||dO||/||O|| <= 1e-2.  Small shapes are compared element by element over the
whole output (several tiles, ragged tails); the full-size workloads are compared
on a deterministic sample of query rows (all batches and heads, all keys),
launched exactly as bench.py launches them.
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


def run_fwd(q_bits, k_bits, v_bits, scale, Sq_alloc=None):
    B, Sq, H, d = q_bits.shape
    Skv = k_bits.shape[1]
    q, k, v = dev_bf16(q_bits), dev_bf16(k_bits), dev_bf16(v_bits)
    o = torch.empty((B, Sq, H, d), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _lib.dit_attn_fwd(q, k, v, o, lse, B, H, Sq, Skv, d, scale, _lib.DIT_DTYPE_BF16)
    torch.cuda.synchronize()
    return host_f64(o), host_f64(lse)


def _draw(B, H, Sq, Skv, d, seed, norm=False):
    name = "sd3" if norm else "tiny"
    g = wl.generate(name, seed=seed, B=B, H=H, Sq=Sq, Skv=Skv, d=d)
    return g["q"], g["k"], g["v"]


SMALL = [
    (1, 2, 256, 256, 64),      # the tiny workload
    (2, 3, 300, 333, 64),      # several tiles, ragged query and key tails
    (1, 2, 129, 1000, 128),
    (2, 1, 37, 4250 // 4, 64),
    (1, 1, 1, 1, 128),
    (1, 3, 640, 96, 128),
]


@pytest.mark.parametrize("B,H,Sq,Skv,d", SMALL)
def test_fwd_small_full_compare(B, H, Sq, Skv, d):
    say(f"fwd small B{B} H{H} Sq{Sq} Skv{Skv} d{d}")
    q, k, v = _draw(B, H, Sq, Skv, d, seed=1000 + Sq + Skv + d)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, l = run_fwd(q, k, v, scale)
    o_ref, l_ref = oracle.attn_fwd(q, k, v, scale)
    compare(o, l, o_ref, l_ref, o_tol=_gpu.o_tol(v, Skv), what=f"B{B}H{H}Sq{Sq}Skv{Skv}d{d}")


# 1 .. 10 key tiles: with four LDS ring slots (d = 128) the loop runs groups
# of four iterations, then possibly a pair, then the last tile's P V either
# alone (from slot 0 or 2) or by one more iteration: 6, 8 and 10 tiles (321,
# 449..512, 577) take the remaining combinations
@pytest.mark.parametrize("Skv", [1, 2, 63, 64, 65, 127, 128, 129, 255, 257, 321, 449, 512, 577])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_key_length_sweep(Skv, d):
    say(f"fwd Skv sweep Skv{Skv} d{d}")
    q, k, v = _draw(1, 2, 70, Skv, d, seed=2000 + Skv, norm=True)
    o, l = run_fwd(q, k, v, 1 / math.sqrt(d))
    o_ref, l_ref = oracle.attn_fwd(q, k, v, float(np.float32(1 / math.sqrt(d))))
    compare(o, l, o_ref, l_ref, o_tol=_gpu.o_tol(v, Skv), what=f"Skv{Skv}d{d}")


@pytest.mark.parametrize("Sq", [1, 31, 32, 33, 127, 128, 129, 255])
def test_fwd_query_length_sweep(Sq):
    say(f"fwd Sq sweep Sq{Sq}")
    q, k, v = _draw(1, 2, Sq, 200, 128, seed=3000 + Sq)
    o, l = run_fwd(q, k, v, 1 / math.sqrt(128))
    o_ref, l_ref = oracle.attn_fwd(q, k, v, float(np.float32(1 / math.sqrt(128))))
    compare(o, l, o_ref, l_ref, what=f"Sq{Sq}")


# ------------------------------------------------------------ invariants

def test_single_key_returns_value_exactly():
    say("fwd single key")
    q, k, v = _draw(1, 4, 100, 1, 128, seed=41)
    scale = float(np.float32(1 / math.sqrt(128)))
    o, l = run_fwd(q, k, v, scale)
    vf = oracle.bf16_bits_to_f64(v)
    np.testing.assert_array_equal(o, np.broadcast_to(vf, o.shape))
    _, l_ref = oracle.attn_fwd(q, k, v, scale)
    assert np.abs(l - l_ref).max() <= 1e-5 * max(1.0, np.abs(l_ref).max())


def test_constant_v_returns_v():
    say("fwd constant V")
    B, H, Sq, Skv, d = 1, 2, 130, 700, 64
    q, k, _ = _draw(B, H, Sq, Skv, d, seed=42)
    rng = np.random.default_rng(4)
    row = wl.f32_to_bf16_bits(rng.standard_normal((1, 1, H, d)).astype(np.float32) * 4)
    v = np.ascontiguousarray(np.broadcast_to(row, (B, Skv, H, d)))
    o, _ = run_fwd(q, k, v, 0.125)
    vf = np.broadcast_to(oracle.bf16_bits_to_f64(row), o.shape)
    assert (np.abs(o - vf) <= _gpu.bf16_ulp(vf)).all()


def test_zero_query_gives_uniform_weights():
    say("fwd zero Q")
    B, H, Sq, Skv, d = 1, 2, 64, 16896, 128
    _, k, v = _draw(B, H, 1, Skv, d, seed=43)
    q = np.zeros((B, Sq, H, d), dtype=np.uint16)
    o, l = run_fwd(q, k, v, 1 / math.sqrt(128))
    assert np.abs(l - math.log(Skv)).max() <= 1e-5 * math.log(Skv)
    mean = oracle.bf16_bits_to_f64(v).mean(axis=1, keepdims=True)
    assert np.abs(o - mean).max() <= 2e-3


def test_key_permutation_invariance():
    say("fwd key permutation")
    B, H, Sq, Skv, d = 1, 2, 96, 333, 128
    q, k, v = _draw(B, H, Sq, Skv, d, seed=44, norm=True)
    perm = np.random.default_rng(9).permutation(Skv)
    kp, vp = np.ascontiguousarray(k[:, perm]), np.ascontiguousarray(v[:, perm])
    o1, l1 = run_fwd(q, k, v, 0.088)
    o2, l2 = run_fwd(q, kp, vp, 0.088)
    o_ref, l_ref = oracle.attn_fwd(q, k, v, float(np.float32(0.088)))
    compare(o1, l1, o_ref, l_ref, what="keys in order")
    compare(o2, l2, o_ref, l_ref, what="keys permuted")
    # P is rounded to bf16 relative to the running maximum, which depends on the
    # key order, so the two runs may differ by the P-rounding bound of each
    # (2^-9 (max|v| + |O|)) -- not only by fp32 reassociation.  LSE uses the
    # unrounded weights and so differs only by reassociation.
    vmax = np.abs(oracle.bf16_bits_to_f64(v)).max()
    omax = max(np.abs(o1).max(), np.abs(o2).max())
    assert np.abs(o2 - o1).max() <= 2.0 ** -8 * (vmax + omax)
    assert np.abs(l2 - l1).max() <= 1e-5


def test_huge_logits_stay_finite():
    say("fwd huge logits")
    B, H, Sq, Skv, d = 1, 2, 64, 300, 64
    q, k, v = _draw(B, H, Sq, Skv, d, seed=45, norm=True)
    q100 = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(q) * 100)
    o, l = run_fwd(q100, k, v, 0.125)
    o_ref, l_ref = oracle.attn_fwd(q100, k, v, 0.125)
    compare(o, l, o_ref, l_ref, lse_tol=1e-3 * max(1, np.abs(l_ref).max() / 100), rel_rms=None,
            what="Qx100")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("first", [0, 200])
def test_scores_rising_far_above_the_first_tile(d, first):
    """Keys from `first + 64` on are scaled up so that later scores exceed the
    first key tile's row maximum by far more than the weight bound allows: the
    kernel must find the exact row maxima and redo its pass.  Only head 0 is
    scaled, so the workgroups of head 1 keep their single pass."""
    say(f"fwd rising scores d{d} first{first}")
    B, H, Sq, Skv = 1, 2, 300, 700
    q, k, v = _draw(B, H, Sq, Skv, d, seed=47 + d + first, norm=True)
    kf = wl.bf16_bits_to_f32(k).copy()
    kf[:, first + 64:, 0] *= np.float32(12.0)
    k12 = wl.f32_to_bf16_bits(kf)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, l = run_fwd(q, k12, v, scale)
    o_ref, l_ref = oracle.attn_fwd(q, k12, v, scale)
    # scores of head 0 reach ~50 natural units (~70 log2 units) above the
    # first tile's maximum
    compare(o, l, o_ref, l_ref, o_tol=_gpu.few_key_o_tol(v),
            lse_tol=1e-3 * max(1, np.abs(l_ref).max() / 100), rel_rms=None, what=f"rising d{d}")


def test_rising_scores_split_launch():
    """The same through dit_attn_fwd_ws, whose split pieces each have their
    own first tile."""
    say("fwd_ws rising scores")
    B, H, Sq, Skv, d = 1, 2, 256, 2048, 128
    n = _lib.dit_attn_fwd_workspace_size(B, H, Sq, Skv, d)
    q, k, v = _draw(B, H, Sq, Skv, d, seed=48, norm=True)
    kf = wl.bf16_bits_to_f32(k).copy()
    kf[:, 1500:] *= np.float32(12.0)
    k12 = wl.f32_to_bf16_bits(kf)
    scale = float(np.float32(1 / math.sqrt(d)))
    qd, kd, vd = dev_bf16(q), dev_bf16(k12), dev_bf16(v)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=qd.device)
    o, l = F.attention(qd, kd, vd, scale, workspace=ws)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn_fwd(q, k12, v, scale)
    compare(host_f64(o), host_f64(l), o_ref, l_ref, o_tol=_gpu.few_key_o_tol(v),
            lse_tol=1e-3 * max(1, np.abs(l_ref).max() / 100), rel_rms=None, what="rising split")


def test_large_values_with_rising_scores():
    """|V| ~ 2^40 together with scores that rise past the weight bound: the
    accumulators must not overflow in either pass."""
    say("fwd large V, rising scores")
    B, H, Sq, Skv, d = 1, 1, 130, 400, 64
    q, k, v = _draw(B, H, Sq, Skv, d, seed=49, norm=True)
    kf = wl.bf16_bits_to_f32(k).copy()
    kf[:, 100:] *= np.float32(10.0)
    k10 = wl.f32_to_bf16_bits(kf)
    vbig = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(v) * np.float32(2.0 ** 40))
    o, l = run_fwd(q, k10, vbig, 0.125)
    o_ref, l_ref = oracle.attn_fwd(q, k10, vbig, 0.125)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    err = np.abs(o - o_ref).max()
    say(f"  max|dO|/2^40 = {err / 2.0 ** 40:.2e}")
    assert err <= _gpu.few_key_o_tol(vbig)
    assert np.abs(l - l_ref).max() <= 1e-3 * max(1, np.abs(l_ref).max() / 100)


def test_poisoned_tails_and_sentinels():
    """NaN after the last key changes nothing; nothing is written past Sq."""
    say("fwd poisoned tails")
    H, Sq, Skv, d, pad = 2, 150, 200, 128, 64
    q, k, v = _draw(1, H, Sq, Skv, d, seed=46)
    nan = np.uint16(0x7FC0)
    kp = np.full((1, Skv + pad, H, d), nan, dtype=np.uint16)
    vp = kp.copy()
    kp[:, :Skv] = k
    vp[:, :Skv] = v
    dev = _gpu.device()
    qd, kd, vd = dev_bf16(q), dev_bf16(kp), dev_bf16(vp)
    sentinel_o = torch.full((1, Sq + pad, H, d), 7.0, dtype=torch.bfloat16, device=dev)
    sentinel_l = torch.full((1 * H * Sq + pad,), -3.0, dtype=torch.float32, device=dev)
    _lib.dit_attn_fwd(qd, kd, vd, sentinel_o, sentinel_l, 1, H, Sq, Skv, d, 0.088,
                      _lib.DIT_DTYPE_BF16)
    torch.cuda.synchronize()
    o_clean, l_clean = run_fwd(q, k, v, 0.088)
    np.testing.assert_array_equal(host_f64(sentinel_o[:, :Sq]), o_clean)
    np.testing.assert_array_equal(host_f64(sentinel_l[:H * Sq]).reshape(1, H, Sq), l_clean)
    assert (host_f64(sentinel_o[:, Sq:]) == 7.0).all()
    assert (host_f64(sentinel_l[H * Sq:]) == -3.0).all()


def test_deterministic_repeats():
    say("fwd determinism")
    q, k, v = _draw(2, 3, 300, 333, 128, seed=47)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    outs = []
    for _ in range(10):
        o, l = F.attention(qd, kd, vd, 0.088)
        outs.append((o.clone(), l.clone()))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l, outs[0][1])


def test_noncurrent_stream():
    say("fwd on a side stream")
    q, k, v = _draw(1, 2, 256, 256, 64, seed=48)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, l = F.attention(qd, kd, vd, 0.125)
    s.synchronize()
    o_ref, l_ref = oracle.attn_fwd(q, k, v, 0.125)
    compare(host_f64(o), host_f64(l), o_ref, l_ref, what="side stream")


# ------------------------------------------------------- full-size workloads

# FLUX-like d = 128: 256-row query tiles, 66 per head, 1584 in all; on a GPU of
# 256 compute units the last 48 (head 23, tiles 18..65) are split over the
# keys.  The sample holds whole tiles: tile 0 (a main tile of every head),
# tile 18 (split for head 23), tile 65 (split, the last), plus 32 more rows.
WORKLOAD_ROWS = {
    "tiny": None,
    "sd3": None,                                         # every row
    "flux": lambda Sq: _gpu.tile_rows(Sq, (0, 18, 65), extra=32),
    "flux_h3": lambda Sq: _gpu.tile_rows(Sq, (0, 65), extra=64),
}


@pytest.mark.parametrize("name", list(WORKLOAD_ROWS))
def test_workload_parity(name):
    W = wl.WORKLOADS[name]
    say(f"workload {name}: generating inputs")
    g = wl.generate(name)
    q, k, v = dev_bf16(g["q"]), dev_bf16(g["k"]), dev_bf16(g["v"])
    say(f"workload {name}: B{W.B} H{W.H} Sq{W.Sq} Skv{W.Skv} d{W.d} launch")
    o, l = F.attention(q, k, v, W.scale)
    torch.cuda.synchronize()
    pick = WORKLOAD_ROWS[name]
    rows = None if pick is None else pick(W.Sq)
    say(f"workload {name}: oracle on {('all' if rows is None else len(rows))} rows")
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], W.scale, rows=rows)
    og, lg = host_f64(o), host_f64(l)
    if rows is not None:
        og, lg = og[:, rows], lg[:, :, rows]
    compare(og, lg, o_ref, l_ref, what=name)
