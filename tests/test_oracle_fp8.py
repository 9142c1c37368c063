"""Pins for the oracle's e4m3 codec and per-(b, h, 128-token block) quantiser.

The codec is pinned to the OCP OFP8 E4M3FN definition (values of specific
codes), to round-trip and ordering invariants, and to an independent library
routine: torch's CPU cast to float8_e4m3fn (round-to-nearest-even, which returns
NaN instead of saturating above 464, so it is compared only inside the range).
The quantiser is pinned by closed forms (the block's largest magnitude maps to
+-448 exactly, scale = amax/448), the e4m3 error bound, block independence and
the zero block, and by re-deriving its bytes with torch's cast.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_non_causal_amd import workloads as wl


# OCP OFP8 E4M3FN: exponent bias 7, 3 mantissa bits, no infinities.
SPEC_POINTS = {
    0x00: 0.0,
    0x80: -0.0,
    0x01: 2.0 ** -9,            # smallest subnormal
    0x07: 7 * 2.0 ** -9,        # largest subnormal, 0.875 * 2^-6
    0x08: 2.0 ** -6,            # smallest normal
    0x38: 1.0,
    0x39: 1.125,
    0x40: 2.0,
    0x7E: 448.0,                # largest normal
    0xFE: -448.0,
    0xB8: -1.0,
    0x3F: 1.875,
    0x30: 0.5,
}


def test_decode_spec_points():
    for code, val in SPEC_POINTS.items():
        got = oracle.e4m3_decode(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)
    assert math.isnan(oracle.e4m3_decode(0x7F))
    assert math.isnan(oracle.e4m3_decode(0xFF))


def test_decode_table_matches_torch():
    table = oracle.e4m3_decode_table()
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(table) == nan).all() and nan.sum() == 2
    np.testing.assert_array_equal(table[~nan], ref[~nan])


def test_encode_roundtrip_and_order():
    table = oracle.e4m3_decode_table()
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(table[c]) == c, hex(c)
    pos = table[0:0x7F]
    assert (np.diff(pos) > 0).all()          # strictly increasing magnitudes


def test_encode_ties_to_even_and_saturation():
    table = oracle.e4m3_decode_table()
    for c in range(0, 0x7E):
        mid = 0.5 * (table[c] + table[c + 1])
        expect = c if c % 2 == 0 else c + 1  # even mantissa wins the tie
        assert oracle.e4m3_encode(mid) == expect, hex(c)
        assert oracle.e4m3_encode(-mid) == expect | 0x80
    for x in (448.0, 449.0, 463.999, 464.0, 465.0, 1e6, float("inf")):
        assert oracle.e4m3_encode(x) == 0x7E
        assert oracle.e4m3_encode(-x) == 0xFE
    assert oracle.e4m3_encode(2.0 ** -11) == 0x00   # below half the smallest subnormal
    assert oracle.e4m3_encode(float("nan")) == 0x7F


def test_encode_matches_torch_cast():
    rng = np.random.default_rng(123)
    mags = np.concatenate([
        rng.uniform(0, 464, 20000),
        np.exp(rng.uniform(math.log(2.0 ** -12), math.log(464), 20000)),
    ]).astype(np.float32)
    x = mags * rng.choice([-1.0, 1.0], mags.size).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(t)) for t in x], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref)


def _blocks(S):
    return [(a, min(a + 128, S)) for a in range(0, S, 128)]


def test_quantiser_closed_forms():
    B, S, H, d = 2, 300, 3, 64           # blocks of 128, 128, 44 tokens
    x = wl.normal_bf16((B, S, H, d), 200)
    q, sc = oracle.quant_fp8(x)
    xf = oracle.bf16_bits_to_f64(x)
    assert sc.shape == (B, H, 3)
    table = oracle.e4m3_decode_table()
    for b in range(B):
        for h in range(H):
            for t, (a, e) in enumerate(_blocks(S)):
                blk = xf[b, a:e, h]
                amax = np.abs(blk).max()
                assert sc[b, h, t] == np.float32(np.float32(amax) / np.float32(448.0))
                qb = q[b, a:e, h]
                idx = np.unravel_index(np.abs(blk).argmax(), blk.shape)
                assert qb[idx] in (0x7E, 0xFE)
                deq = table[qb] * float(sc[b, h, t])
                normal = np.abs(blk) * 448.0 / amax >= 2.0 ** -6
                err = np.abs(deq - blk)
                # RNE to 3 mantissa bits: relative error <= 2^-4 (plus fp32 steps)
                assert (err[normal] <= (2.0 ** -4 + 1e-6) * np.abs(blk[normal])).all()
                assert (err[~normal] <= 2.0 ** -10 * amax / 448.0 * 1.0001).all()


def test_quantiser_matches_torch_cast():
    B, S, H, d = 1, 256, 2, 128
    x = wl.generate("flux_fp8", B=B, H=H, Sq=S, Skv=S)["v"]
    q, sc = oracle.quant_fp8(x)
    xf = torch.from_numpy(wl.bf16_bits_to_f32(x))
    for h in range(H):
        for t, (a, e) in enumerate(_blocks(S)):
            blk = xf[0, a:e, h]
            amax = blk.abs().max()
            inv = torch.tensor(448.0, dtype=torch.float32) / amax
            y = blk * inv
            ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            np.testing.assert_array_equal(q[0, a:e, h], ref)
            assert sc[0, h, t] == (amax / torch.tensor(448.0)).item()


def test_quantiser_blocks_are_independent_and_zero_block():
    B, S, H, d = 1, 384, 2, 64
    x = wl.normal_bf16((B, S, H, d), 300)
    q1, s1 = oracle.quant_fp8(x)
    x2 = x.copy()
    x2[0, 128:256, 1] = 0                # zero one block of head 1
    x2[0, 0, 0, 0] = wl.f32_to_bf16_bits(np.float32([1000.0]))[0]  # outlier in block 0, head 0
    q2, s2 = oracle.quant_fp8(x2)
    assert s2[0, 1, 1] == 1.0 and (q2[0, 128:256, 1] == 0).all()
    # untouched blocks keep their bytes and scales
    np.testing.assert_array_equal(q2[0, 128:, 0], q1[0, 128:, 0])
    np.testing.assert_array_equal(q2[0, :128, 1], q1[0, :128, 1])
    np.testing.assert_array_equal(q2[0, 256:, 1], q1[0, 256:, 1])
    assert s2[0, 0, 1] == s1[0, 0, 1] and s2[0, 1, 2] == s1[0, 1, 2]
    assert s2[0, 0, 0] == np.float32(np.float32(1000.0) / np.float32(448.0))


def test_dequant_inverts_within_bound():
    x = wl.generate("flux_fp8", B=1, H=4, Sq=200, Skv=200)["k"]
    q, sc = oracle.quant_fp8(x)
    xr = oracle.dequant_fp8(q, sc)
    xf = oracle.bf16_bits_to_f64(x)
    rel = np.abs(xr - xf) / np.maximum(np.abs(xf), 1e-30)
    big = np.abs(xf) > 0.5
    assert rel[big].max() <= 2.0 ** -4 + 1e-6


def _nonfinite_blocks():
    """bf16 [1, 384, 3, 64]: head 0 block 0 holds NaNs of both signs among
    finite values, head 1 block 1 a +inf and a -inf, head 2 block 2 only NaNs
    and zeros; every other block is finite."""
    x = wl.normal_bf16((1, 384, 3, 64), 310)
    x[0, 3, 0, 5] = 0x7FC0                    # +NaN
    x[0, 70, 0, 0] = 0xFFC1                   # -NaN with a payload
    x[0, 130, 1, 9] = 0x7F80                  # +inf
    x[0, 200, 1, 2] = 0xFF80                  # -inf
    x[0, 256:, 2] = 0
    x[0, 300, 2, 1] = 0x7FC0
    return x


def test_quantiser_nonfinite_input():
    """The quantiser's steps as written decide non-finite input: a NaN fails
    the comparison with amax (no part in it) and encodes as 0x7F; an infinity
    makes amax and the scale +inf, so finite values become signed zeros and the
    infinities (inf * 0 = NaN) 0x7F; a block of zeros and NaNs has amax 0."""
    x = _nonfinite_blocks()
    q, sc = oracle.quant_fp8(x)
    xf = oracle.bf16_bits_to_f64(x)
    # NaN block: the same bytes and scale as with its NaNs replaced by zeros,
    # except 0x7F at the NaNs
    x0 = x.copy()
    x0[0, 3, 0, 5] = 0
    x0[0, 70, 0, 0] = 0
    q0, s0 = oracle.quant_fp8(x0)
    assert sc[0, 0, 0] == s0[0, 0, 0]
    fin = np.isfinite(xf[0, :128, 0])
    assert (q[0, :128, 0][fin] == q0[0, :128, 0][fin]).all()
    assert q[0, 3, 0, 5] == 0x7F and q[0, 70, 0, 0] == 0x7F
    # infinity block: scale +inf, finite values -> signed zeros, infinities -> 0x7F
    assert sc[0, 1, 1] == np.inf
    blk, qb = xf[0, 128:256, 1], q[0, 128:256, 1]
    fin = np.isfinite(blk)
    assert (qb[fin] == np.where(np.signbit(blk[fin]), 0x80, 0x00)).all()
    assert (qb[~fin] == 0x7F).all() and (~fin).sum() == 2
    # zeros and NaNs only: amax = 0, scale 1, all bytes 0
    assert sc[0, 2, 2] == 1.0 and (q[0, 256:, 2] == 0).all()
    # the finite blocks are untouched by their neighbours
    xc = x.copy()
    xc[0, 3, 0, 5] = xc[0, 70, 0, 0] = xc[0, 130, 1, 9] = xc[0, 200, 1, 2] = 0
    xc[0, 256:, 2] = wl.normal_bf16((1, 128, 64), 311)
    qc, scc = oracle.quant_fp8(xc)
    for h, t in ((0, 1), (0, 2), (1, 0), (1, 2), (2, 0), (2, 1)):
        sl = slice(128 * t, 128 * (t + 1))
        assert sc[0, h, t] == scc[0, h, t]
        np.testing.assert_array_equal(q[0, sl, h], qc[0, sl, h])


def test_dequant_closed_form():
    """dequant(q, scale)[b, s, h, c] = decode(q[b, s, h, c]) * scale[b, h, s // 128],
    re-derived with NumPy indexing on codes and scales drawn independently (every
    (b, h, block) has its own scale, so a wrong block, head or batch index shows)."""
    rng = np.random.default_rng(77)
    B, S, H, d = 2, 300, 3, 16
    q = rng.integers(0, 256, size=(B, S, H, d), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x11                 # no NaN codes
    nblk = (S + 127) // 128
    sc = rng.uniform(0.5, 4.0, size=(B, H, nblk)).astype(np.float32)
    got = oracle.dequant_fp8(q, sc)
    table = oracle.e4m3_decode_table()
    blk = np.arange(S) // 128
    scale_bshd = sc.transpose(0, 2, 1)[:, blk, :, None].astype(np.float64)  # [B, S, H, 1]
    np.testing.assert_array_equal(got, table[q] * scale_bshd)
