"""GPU parity of dit_attn_merge (and of one ring rank's share: chunked forward
launches + merge) against the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_non_causal_amd import _lib, functional as F, workloads as wl
from tests import _gpu
from tests._gpu import compare, dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


def _partials(B, H, Sq, d, n, seed):
    """Random bf16 partial outputs and fp32 LSEs (as a forward pass would emit)."""
    rng = np.random.default_rng(seed)
    o_bits = wl.f32_to_bf16_bits(rng.standard_normal((n, B, Sq, H, d)).astype(np.float32))
    lse = (rng.standard_normal((n, B, H, Sq)) * 3 + 5).astype(np.float32)
    return o_bits, lse


def _run_merge(o_bits, lse, inplace=False):
    n, B, Sq, H, d = o_bits.shape
    parts_o = [dev_bf16(o_bits[i]) for i in range(n)]
    parts_l = [torch.from_numpy(lse[i].copy()).to(_gpu.device()) for i in range(n)]
    if inplace:
        out, out_l = parts_o[0], parts_l[0]
    else:
        out = torch.empty_like(parts_o[0])
        out_l = torch.empty_like(parts_l[0])
    _lib.dit_attn_merge(parts_o, parts_l, n, out, out_l, B, H, Sq, d)
    torch.cuda.synchronize()
    return host_f64(out), host_f64(out_l)


@pytest.mark.parametrize("n,B,H,Sq,d", [(1, 1, 2, 50, 64), (2, 2, 3, 77, 128), (4, 1, 40, 300, 128),
                                        (16, 1, 2, 33, 64), (7, 2, 5, 129, 64)])
def test_merge_matches_oracle(n, B, H, Sq, d):
    say(f"merge n{n} B{B} H{H} Sq{Sq} d{d}")
    o_bits, lse = _partials(B, H, Sq, d, n, seed=100 + n)
    o, l = _run_merge(o_bits, lse)
    o_ref, l_ref = oracle.attn_merge(o_bits, lse)
    # one bf16 rounding of the output plus fp32 accumulation
    assert (np.abs(o - o_ref) <= _gpu.bf16_ulp(o_ref) + 1e-6).all()
    assert np.abs(l - l_ref).max() <= 1e-5 * np.abs(l_ref).max()


def test_merge_single_part_is_identity_and_inplace():
    say("merge n=1 identity, in place")
    o_bits, lse = _partials(1, 3, 100, 128, 1, seed=7)
    o, l = _run_merge(o_bits, lse)
    np.testing.assert_array_equal(o, oracle.bf16_bits_to_f64(o_bits[0]))
    np.testing.assert_array_equal(l, lse[0].astype(np.float64))
    o_bits4, lse4 = _partials(1, 3, 100, 128, 4, seed=8)
    o_a, l_a = _run_merge(o_bits4, lse4)
    o_b, l_b = _run_merge(o_bits4, lse4, inplace=True)
    np.testing.assert_array_equal(o_a, o_b)
    np.testing.assert_array_equal(l_a, l_b)


def test_merge_neg_inf_parts():
    say("merge -inf parts")
    o_bits, lse = _partials(1, 2, 64, 64, 3, seed=9)
    lse[1] = -np.inf
    o, l = _run_merge(o_bits, lse)
    o2, l2 = _run_merge(o_bits[[0, 2]].copy(), lse[[0, 2]].copy())
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)
    lse[:] = -np.inf
    o, l = _run_merge(o_bits, lse)
    assert (o == 0).all() and np.isneginf(l).all()


def _split_forward_and_merge(q_bits, k_bits, v_bits, bounds, scale):
    B, Sq, H, d = q_bits.shape
    q = dev_bf16(q_bits)
    parts_o, parts_l = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        k = dev_bf16(np.ascontiguousarray(k_bits[:, a:b]))
        v = dev_bf16(np.ascontiguousarray(v_bits[:, a:b]))
        o, l = F.attention(q, k, v, scale)
        parts_o.append(o)
        parts_l.append(l)
    o, l = F.merge(parts_o, parts_l)
    torch.cuda.synchronize()
    return host_f64(o), host_f64(l)


@pytest.mark.parametrize("bounds", [[0, 300, 633], [0, 1, 64, 65, 200, 633],
                                    [0, 40, 80, 120, 160, 200, 240, 280, 320, 360, 400, 440,
                                     480, 520, 560, 600, 633]])
def test_split_forward_then_merge_equals_full(bounds):
    say(f"split forward + merge, {len(bounds) - 1} parts")
    g = wl.generate("tiny", seed=77, B=2, H=3, Sq=150, Skv=633, d=128)
    scale = float(np.float32(1 / math.sqrt(128)))
    o, l = _split_forward_and_merge(g["q"], g["k"], g["v"], bounds, scale)
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], scale)
    compare(o, l, o_ref, l_ref, what=f"split{len(bounds) - 1}")


def test_ring_share_small():
    say("ring share small: 4 chunks of 300 + merge")
    g = wl.generate("wan_ring", seed=78, Sq=200, Skv=1200)
    scale = float(np.float32(1 / math.sqrt(128)))
    q, k, v = dev_bf16(g["q"]), dev_bf16(g["k"]), dev_bf16(g["v"])
    o, l = F.ring_share_attention(q, k, v, 4, scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], scale)
    compare(host_f64(o), host_f64(l), o_ref, l_ref, what="ring small")


def test_wan_ring_share_full_size():
    W = wl.WORKLOADS["wan_ring"]
    say("wan ring share: generating inputs")
    g = wl.generate("wan_ring")
    q, k, v = dev_bf16(g["q"]), dev_bf16(g["k"]), dev_bf16(g["v"])
    say("wan ring share: 4 chunk forwards + merge")
    o, l = F.ring_share_attention(q, k, v, W.n_chunks, W.scale)
    torch.cuda.synchronize()
    # the last query tile (254 rows: 8190 = 31 * 256 + 254) and 8 more rows
    rows = _gpu.tile_rows(W.Sq, (31,), extra=8)
    say(f"wan ring share: oracle (full 32760 keys) on {len(rows)} rows")
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], W.scale, rows=rows)
    compare(host_f64(o)[:, rows], host_f64(l)[:, :, rows], o_ref, l_ref, what="wan_ring")


@pytest.mark.parametrize("n,d", [(2, 64), (3, 128), (16, 128)])
def test_merge_larger_than_the_last_level_cache(n, d):
    """A merge that moves more than 256 MB takes the kernel's streaming
    (non-temporal) accesses; a slice of its rows, merged on its own, takes the
    ordinary ones.  The arithmetic is the same, so the two agree bit for bit,
    and the slice matches the oracle (some rows and parts set to -inf)."""
    B, H, Sq = 1, 256 if d == 64 else 128, 3000 if n < 16 else 600
    say(f"large merge n{n} d{d}: {(n + 1) * B * Sq * H * (2 * d + 4) / 1e6:.0f} MB")
    assert (n + 1) * B * Sq * H * (2 * d + 4) > 256 << 20
    dev = _gpu.device()
    gen = torch.Generator(device=dev).manual_seed(4000 + n)
    parts_o = [torch.randn((B, Sq, H, d), device=dev, generator=gen).to(torch.bfloat16)
               for _ in range(n)]
    parts_l = [torch.randn((B, H, Sq), device=dev, generator=gen) * 3 + 5 for _ in range(n)]
    parts_l[0][:, :, 7] = -math.inf
    for p in parts_l:
        p[:, 3, 11] = -math.inf
    o, l = F.merge(parts_o, parts_l)
    s0, s1 = 5, 40  # rows 5..39 of every head: a small merge of its own
    so = [p[:, s0:s1].contiguous() for p in parts_o]
    sl = [p[:, :, s0:s1].contiguous() for p in parts_l]
    o_s, l_s = F.merge(so, sl)
    torch.cuda.synchronize()
    assert torch.equal(o[:, s0:s1].view(torch.int16), o_s.view(torch.int16))
    assert torch.equal(l[:, :, s0:s1], l_s)
    o_bits = np.stack([p.view(torch.int16).cpu().numpy().view(np.uint16) for p in so])
    lse = np.stack([p.cpu().numpy() for p in sl])
    o_ref, l_ref = oracle.attn_merge(o_bits, lse)
    og, lg = host_f64(o_s), host_f64(l_s)
    assert (np.abs(og - o_ref) <= _gpu.bf16_ulp(o_ref) + 1e-6).all()
    fin = np.isfinite(l_ref)
    assert (np.isneginf(lg) == ~fin).all()
    empty_rows = np.broadcast_to((~fin).transpose(0, 2, 1)[..., None], og.shape)
    assert empty_rows.any() and (og[empty_rows] == 0).all()
    assert np.abs(lg[fin] - l_ref[fin]).max() <= 1e-5 * np.abs(l_ref[fin]).max()
