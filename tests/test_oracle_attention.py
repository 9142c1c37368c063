"""Pins for the oracle's attention forward and merge.

Nothing here calls the HIP path.  Each test pins the oracle to something other
than itself: an independent pure-Python brute force, a library routine
(torch's float64 scaled_dot_product_attention / logsumexp on the CPU), closed
forms, and invariants of non-causal softmax attention.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_non_causal_amd import workloads as wl
from tests import _brute


def _f64(bits):
    return oracle.bf16_bits_to_f64(bits)


def _rand_bf16(shape, seed):
    return wl.normal_bf16(shape, seed)


@pytest.mark.parametrize("B,H,Sq,Skv,d", [(1, 1, 1, 1, 1), (2, 2, 3, 5, 4), (1, 3, 7, 2, 8),
                                          (2, 1, 4, 9, 3)])
def test_bruteforce_tiny(B, H, Sq, Skv, d):
    q = _rand_bf16((B, Sq, H, d), 1)
    k = _rand_bf16((B, Skv, H, d), 2)
    v = _rand_bf16((B, Skv, H, d), 3)
    scale = 0.37
    o, lse = oracle.attn_fwd(q, k, v, scale)
    ob, lb = _brute.attention(_f64(q).tolist(), _f64(k).tolist(), _f64(v).tolist(), scale)
    np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(lb), rtol=0, atol=1e-12)


def _torch_reference(q, k, v, scale):
    """float64 CPU reference through torch's SDPA and logsumexp."""
    qt = torch.from_numpy(_f64(q)).permute(0, 2, 1, 3).contiguous()   # [B,H,Sq,d]
    kt = torch.from_numpy(_f64(k)).permute(0, 2, 1, 3).contiguous()
    vt = torch.from_numpy(_f64(v)).permute(0, 2, 1, 3).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    logits = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) * scale
    lse = torch.logsumexp(logits, dim=-1)                              # [B,H,Sq]
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


@pytest.mark.parametrize("B,H,Sq,Skv,d", [(2, 3, 130, 257, 64), (1, 2, 65, 33, 128)])
def test_matches_torch_sdpa_f64(B, H, Sq, Skv, d):
    q = _rand_bf16((B, Sq, H, d), 11)
    k = _rand_bf16((B, Skv, H, d), 12)
    v = _rand_bf16((B, Skv, H, d), 13)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attn_fwd(q, k, v, scale)
    ot, lt = _torch_reference(q, k, v, scale)
    np.testing.assert_allclose(o, ot, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lt, rtol=0, atol=1e-12)


def test_row_subset_equals_full():
    B, H, Sq, Skv, d = 2, 3, 40, 50, 16
    q = _rand_bf16((B, Sq, H, d), 21)
    k = _rand_bf16((B, Skv, H, d), 22)
    v = _rand_bf16((B, Skv, H, d), 23)
    o, lse = oracle.attn_fwd(q, k, v, 0.25)
    rows = [39, 0, 17, 5]
    os_, ls = oracle.attn_fwd(q, k, v, 0.25, rows=rows)
    np.testing.assert_array_equal(os_, o[:, rows])
    np.testing.assert_array_equal(ls, lse[:, :, rows])


def test_two_key_closed_form():
    # q . k1 = 2.5, q . k2 = -1.0 (exact in bf16), scale 0.5
    q = np.array([1.0, 0.5, 0.0, 2.0]).reshape(1, 1, 1, 4)
    k = np.array([[0.5, 1.0, 3.0, 0.75], [-1.0, 2.0, 1.0, -0.5]]).reshape(1, 2, 1, 4)
    v = np.array([[1.0, -2.0, 0.25, 4.0], [3.0, 0.5, -1.5, 0.0]]).reshape(1, 2, 1, 4)
    scale = 0.5
    s1, s2 = scale * 2.5, scale * -1.0
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    o_exp = sig(s1 - s2) * v[0, 0, 0] + sig(s2 - s1) * v[0, 1, 0]
    lse_exp = max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2)))
    o, lse = oracle.attn_fwd(q, k, v, scale)
    np.testing.assert_allclose(o[0, 0, 0], o_exp, rtol=0, atol=1e-14)
    assert abs(lse[0, 0, 0] - lse_exp) <= 1e-14


def test_single_key_returns_its_value():
    q = _rand_bf16((2, 5, 3, 8), 31)
    k = _rand_bf16((2, 1, 3, 8), 32)
    v = _rand_bf16((2, 1, 3, 8), 33)
    o, lse = oracle.attn_fwd(q, k, v, 0.3)
    np.testing.assert_array_equal(o, np.broadcast_to(_f64(v), o.shape))
    dots = np.einsum("bihc,bhc->bhi", _f64(q), _f64(k)[:, 0])
    np.testing.assert_allclose(lse, 0.3 * dots, rtol=0, atol=1e-13)


def test_constant_v_returns_v():
    B, H, Sq, Skv, d = 1, 2, 9, 37, 8
    q = _rand_bf16((B, Sq, H, d), 41)
    k = _rand_bf16((B, Skv, H, d), 42)
    row = np.array([0.75, -3.0, 1.5, 0.0, 2.0, -0.125, 10.0, 1.0])
    v = np.broadcast_to(row, (B, Skv, H, d)).copy()
    o, _ = oracle.attn_fwd(_f64(q), _f64(k), v, 0.5)
    np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), rtol=1e-14, atol=1e-14)


def test_zero_query_uniform_weights():
    B, H, Sq, Skv, d = 1, 2, 3, 16896, 4
    q = np.zeros((B, Sq, H, d))
    k = _f64(_rand_bf16((B, Skv, H, d), 51))
    v = _f64(_rand_bf16((B, Skv, H, d), 52))
    o, lse = oracle.attn_fwd(q, k, v, 1.0)
    np.testing.assert_allclose(lse, math.log(16896), rtol=0, atol=1e-12)
    assert abs(math.log(16896) - 9.734832) < 1e-6
    mean = v.mean(axis=1, keepdims=True)
    np.testing.assert_allclose(o, np.broadcast_to(mean, o.shape), rtol=0, atol=1e-13)


def test_rows_of_softmax_sum_to_one():
    # V = identity over keys, so O row i is exactly the probability row P_i.
    B, H, Sq, Skv = 1, 2, 11, 16
    d = Skv
    q = _f64(_rand_bf16((B, Sq, H, d), 61))
    k = _f64(_rand_bf16((B, Skv, H, d), 62))
    v = np.zeros((B, Skv, H, d))
    for j in range(Skv):
        v[0, j, :, j] = 1.0
    o, lse = oracle.attn_fwd(q, k, v, 0.7)
    np.testing.assert_allclose(o.sum(axis=-1), 1.0, rtol=0, atol=1e-13)
    assert (o > 0).all()
    # and P_ij = exp(s_ij - LSE_i)
    s = 0.7 * np.einsum("bihc,bjhc->bhij", q, k)
    p = np.exp(s - lse[..., None])
    np.testing.assert_allclose(o.transpose(0, 2, 1, 3), p, rtol=1e-12, atol=1e-15)


def test_key_permutation_invariance():
    B, H, Sq, Skv, d = 1, 2, 6, 45, 16
    q = _rand_bf16((B, Sq, H, d), 71)
    k = _rand_bf16((B, Skv, H, d), 72)
    v = _rand_bf16((B, Skv, H, d), 73)
    perm = np.random.default_rng(7).permutation(Skv)
    o1, l1 = oracle.attn_fwd(q, k, v, 0.25)
    o2, l2 = oracle.attn_fwd(q, np.ascontiguousarray(k[:, perm]), np.ascontiguousarray(v[:, perm]),
                             0.25)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)


def test_key_shift_changes_only_lse():
    B, H, Sq, Skv, d = 1, 1, 5, 20, 8
    q = _f64(_rand_bf16((B, Sq, H, d), 81))
    k = _f64(_rand_bf16((B, Skv, H, d), 82))
    v = _f64(_rand_bf16((B, Skv, H, d), 83))
    u = np.array([0.5, -1.0, 0.25, 2.0, 0.0, -0.75, 1.0, 0.125])
    o1, l1 = oracle.attn_fwd(q, k, v, 0.5)
    o2, l2 = oracle.attn_fwd(q, k + u, v, 0.5)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    shift = 0.5 * np.einsum("bihc,c->bhi", q, u)
    np.testing.assert_allclose(l2 - l1, shift, rtol=0, atol=1e-12)


def test_huge_logits_stay_finite():
    B, H, Sq, Skv, d = 1, 1, 4, 30, 16
    q = _f64(_rand_bf16((B, Sq, H, d), 91)) * 100.0
    k = _f64(_rand_bf16((B, Skv, H, d), 92))
    v = _f64(_rand_bf16((B, Skv, H, d), 93))
    o, lse = oracle.attn_fwd(q, k, v, 1.0)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    s = np.einsum("bihc,bjhc->bhij", q, k)
    arg = s.argmax(-1)[0, 0]
    np.testing.assert_allclose(o[0, :, 0], v[0, arg, 0], rtol=0, atol=1e-6)
    np.testing.assert_allclose(lse[0, 0], s.max(-1)[0, 0], rtol=1e-12)


# ---------------------------------------------------------------- merge pins

def _split_fwd(q, k, v, scale, bounds):
    parts_o, parts_l = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        o, l = oracle.attn_fwd(q, np.ascontiguousarray(k[:, a:b]), np.ascontiguousarray(v[:, a:b]),
                               scale)
        parts_o.append(o)
        parts_l.append(l)
    return np.stack(parts_o), np.stack(parts_l)


@pytest.mark.parametrize("bounds", [[0, 100], [0, 40, 100], [0, 25, 26, 70, 100],
                                    [0, 7, 14, 21, 28, 35, 42, 49, 56, 63, 70, 77, 84, 91, 96, 98,
                                     100]])
def test_merge_of_split_partials_equals_full(bounds):
    B, H, Sq, Skv, d = 2, 3, 9, 100, 16
    q = _rand_bf16((B, Sq, H, d), 101)
    k = _rand_bf16((B, Skv, H, d), 102)
    v = _rand_bf16((B, Skv, H, d), 103)
    o_full, l_full = oracle.attn_fwd(q, k, v, 0.25)
    po, pl = _split_fwd(q, k, v, 0.25, bounds)
    o, l = oracle.attn_merge(po, pl)
    np.testing.assert_allclose(o, o_full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, l_full, rtol=0, atol=1e-12)


def test_merge_identities():
    B, H, Sq, d = 1, 2, 5, 8
    rng = np.random.default_rng(5)
    o1 = rng.standard_normal((1, B, Sq, H, d))
    l1 = rng.standard_normal((1, B, H, Sq))
    o, l = oracle.attn_merge(o1, l1)
    np.testing.assert_array_equal(o, o1[0])
    np.testing.assert_array_equal(l, l1[0])
    # equal LSEs: plain mean, LSE + ln n
    o3 = rng.standard_normal((3, B, Sq, H, d))
    l3 = np.broadcast_to(l1, (3, B, H, Sq)).copy()
    o, l = oracle.attn_merge(o3, l3)
    np.testing.assert_allclose(o, o3.mean(0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(l, l1[0] + math.log(3), rtol=0, atol=1e-14)
    # order invariance
    l3 = rng.standard_normal((3, B, H, Sq))
    o_a, l_a = oracle.attn_merge(o3, l3)
    o_b, l_b = oracle.attn_merge(o3[::-1].copy(), l3[::-1].copy())
    np.testing.assert_allclose(o_b, o_a, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l_b, l_a, rtol=0, atol=1e-14)
    # a -inf part carries no weight
    l4 = np.concatenate([l3, np.full((1, B, H, Sq), -np.inf)])
    o4 = np.concatenate([o3, rng.standard_normal((1, B, Sq, H, d))])
    o_c, l_c = oracle.attn_merge(o4, l4)
    np.testing.assert_array_equal(o_c, o_a)
    np.testing.assert_array_equal(l_c, l_a)
    # all parts -inf: O = 0, LSE = -inf
    o_d, l_d = oracle.attn_merge(o3, np.full((3, B, H, Sq), -np.inf))
    assert (o_d == 0).all() and np.isneginf(l_d).all()


def test_merge_weights_against_closed_form():
    # two parts with LSE 0 and ln 3: weights 1/4 and 3/4, merged LSE ln 4.
    o2 = np.stack([np.full((1, 1, 1, 2), 1.0), np.full((1, 1, 1, 2), 5.0)])
    l2 = np.array([0.0, math.log(3.0)]).reshape(2, 1, 1, 1)
    o, l = oracle.attn_merge(o2, l2)
    np.testing.assert_allclose(o, 4.0, rtol=0, atol=1e-15)
    assert abs(l[0, 0, 0] - math.log(4.0)) < 1e-15


def test_workload_generator_recipe():
    g = wl.generate("sd3", B=1, H=2, Sq=10, Skv=12)
    q = wl.bf16_bits_to_f32(g["q"]).astype(np.float64)
    # RMS-normalised per (b, s, h): mean of squares ~ 1 (bf16 rounding aside)
    ms = (q ** 2).mean(-1)
    np.testing.assert_allclose(ms, 1.0, rtol=0, atol=2e-2)
    g8 = wl.generate("flux_fp8", H=24, Sq=4, Skv=4)
    assert len(g8["outliers_q"]) == 31 and len(set(g8["outliers_q"])) == 31
    assert not np.array_equal(np.sort(g8["outliers_q"]), np.sort(g8["outliers_k"]))
    # generation is deterministic
    g2 = wl.generate("sd3", B=1, H=2, Sq=10, Skv=12)
    np.testing.assert_array_equal(g["k"], g2["k"])
