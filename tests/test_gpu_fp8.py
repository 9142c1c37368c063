"""GPU parity of the fp8 forward pass: dit_quant_fp8 on Q, K, V, then
dit_attn_fwd with DIT_DTYPE_FP8_E4M3, through the C ABI.

Two references, both from the oracle:
* the oracle on the *dequantised* inputs (decode(q8) * block scale) -- this
  isolates the kernel's own error.  The kernel rounds each softmax weight to
  e4m3 before P.V and normalises by the sum of the rounded weights, so O is a
  convex combination with perturbed weights.  A weight enters the rounding as
  P'' = f K P 2^(m_true - m_ref), P = 2^(s - max s) <= 1, with K = 56, f in
  [1, 2) and a reference m_ref at most M = 5 log2 units above the row
  maximum: relative error <= 2^-4 in e4m3's normal range, absolute <= 2^-10
  below it, i.e. <= E = 2^-10 2^M / K in units of P.  So
      |dO_c| <= 2 (2^-4 sum_j P_j |v_jc - O_c| + E sum_j |v_jc - O_c|)
                / ((1 - 2^-4) sum_j P_j) + 2^-8 |O_c| + 1e-6
  (bf16 output rounding included).  It is computed per element from the
  dequantised inputs and must hold everywhere; LSE uses the unrounded weights
  (gate: lse_bound);
* the oracle on the unquantised bf16 inputs -- the contract gate max|dO| <=
  6e-2 on unit-normal inputs (RMS-normalised Q/K, N(0,1) V) at the FLUX-like
  shape.  On the x8-outlier workload the quantisation floor alone is ~1.1, so
  there the kernel is gated against the dequantised reference and the total
  error is reported.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_non_causal_amd import functional as F, workloads as wl
from tests import _gpu
from tests._gpu import FP8_O_TOL, compare, dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


def run_fp8(g, scale, workspace="auto"):
    """The fp8 path as the library's users call it: dit_attn_fwd_ws (which
    splits the last wave of query tiles when the shape leaves one) by default,
    dit_attn_fwd with workspace=None."""
    q, k, v = dev_bf16(g["q"]), dev_bf16(g["k"]), dev_bf16(g["v"])
    q8, qs = F.quantize_fp8(q)
    k8, ks = F.quantize_fp8(k)
    v8, vs = F.quantize_fp8(v)
    o, l = F.attention_fp8(q8, qs, k8, ks, v8, vs, scale, workspace=workspace)
    torch.cuda.synchronize()
    return host_f64(o), host_f64(l)


def dequant(bits):
    return oracle.dequant_fp8(*oracle.quant_fp8(bits))


# absolute rounding error of a weight below e4m3's normal range, in units of
# the row's largest weight: E = 2^-10 * 2^M / K (see the module docstring)
SUBNORMAL_ERR = 2.0 ** -10 * 2.0 ** 5 / 56


def kernel_bound(qd, kd, vd, scale, rows=None):
    """Per-element bound on the kernel's own error (see module docstring),
    computed one (batch, row, head) at a time to bound memory."""
    qs = qd if rows is None else qd[:, rows]
    B, n, H, d = qs.shape
    out = np.empty((B, n, H, d))
    for b in range(B):
        for h in range(H):
            kh, vh = kd[b, :, h], vd[b, :, h]                    # [Skv, d]
            s = qs[b, :, h] @ kh.T * scale                       # [n, Skv]
            p = np.exp(s - s.max(-1, keepdims=True))
            den = p.sum(-1)                                      # [n]
            o = (p @ vh) / den[:, None]                          # [n, d]
            for i0 in range(0, n, 8):                           # 8 rows at a time
                i1 = min(i0 + 8, n)
                dev = np.abs(vh[None] - o[i0:i1, None])         # [rows, Skv, d]
                pw = np.einsum("rj,rjc->rc", p[i0:i1], dev)
                num = 2.0 * (2.0 ** -4 * pw + SUBNORMAL_ERR * dev.sum(1)) / (1 - 2.0 ** -4)
                out[b, i0:i1, h] = num / den[i0:i1, None] + 2.0 ** -8 * np.abs(o[i0:i1]) + 1e-6
    return out


# Accumulation precision of the fp8 matrix instruction's dot products: an
# error of at most this fraction of the sum of the products' magnitudes,
# scale * sum_c |q_c k_c| (test_fp8_single_key_score_precision measures it
# through the public API and finds about 2^-13).
MFMA_FP8_REL = 2.0 ** -12


def lse_bound(qd, kd, scale, rows=None):
    """Per-(batch, head, row) bound on the fp8 kernel's LSE error against the
    oracle on the dequantised inputs: LSE moves by the softmax-weighted average
    of the score errors, each at most MFMA_FP8_REL * scale * sum_c |q_c k_jc|,
    plus 1e-3 for the fp32 exponentials, sums and logarithm."""
    qs = qd if rows is None else qd[:, rows]
    B, n, H, d = qs.shape
    out = np.empty((B, H, n))
    for b in range(B):
        for h in range(H):
            kh = kd[b, :, h]
            s = qs[b, :, h] @ kh.T * scale
            a = np.abs(qs[b, :, h]) @ np.abs(kh).T * scale
            p = np.exp(s - s.max(-1, keepdims=True))
            out[b, h] = 1e-3 + MFMA_FP8_REL * (p * a).sum(-1) / p.sum(-1)
    return out


def check_against_dequant(g, scale, rows=None, what="", workspace="auto"):
    o, l = run_fp8(g, scale, workspace)
    qd, kd, vd = dequant(g["q"]), dequant(g["k"]), dequant(g["v"])
    o_ref, l_ref = oracle.attn_fwd(qd, kd, vd, scale, rows=rows)
    if rows is not None:
        o, l = o[:, rows], l[:, :, rows]
    bound = kernel_bound(qd, kd, vd, scale, rows)
    err = np.abs(o - o_ref)
    say(f"{what}: vs dequantised oracle max|dO|={err.max():.3e} "
        f"(worst err/bound {(err / bound).max():.3f}) max|dLSE|={np.abs(l - l_ref).max():.3e}")
    assert np.isfinite(o).all() and np.isfinite(l).all()
    assert (err <= bound).all(), f"{what}: kernel error exceeds its bound"
    # LSE: the fp8 matrix instruction sums products of very different
    # magnitude (outlier channels) to ~2^-13 of their magnitudes' sum
    lb = lse_bound(qd, kd, scale, rows)
    dl = np.abs(l - l_ref)
    say(f"{what}: worst LSE err/bound {(dl / lb).max():.3f}")
    assert (dl <= lb).all(), f"{what}: LSE error exceeds its bound"
    return o, l


@pytest.mark.parametrize("B,H,Sq,Skv,d", [(1, 2, 256, 256, 128), (2, 3, 300, 333, 64),
                                          (1, 2, 129, 1000, 128), (1, 1, 1, 1, 128),
                                          (1, 2, 70, 65, 64), (2, 1, 128, 127, 128)])
def test_fp8_small_against_dequantised(B, H, Sq, Skv, d):
    say(f"fp8 small B{B} H{H} Sq{Sq} Skv{Skv} d{d}")
    g = wl.generate("flux", seed=700 + Sq + Skv + d, B=B, H=H, Sq=Sq, Skv=Skv, d=d)
    check_against_dequant(g, float(np.float32(1 / math.sqrt(d))), what=f"fp8 B{B}H{H}Sq{Sq}Skv{Skv}d{d}")


@pytest.mark.parametrize("Skv", [1, 2, 63, 64, 65, 128, 129, 255, 257])
def test_fp8_key_length_sweep(Skv):
    say(f"fp8 Skv sweep {Skv}")
    g = wl.generate("flux", seed=800 + Skv, B=1, H=2, Sq=130, Skv=Skv, d=128)
    check_against_dequant(g, float(np.float32(1 / math.sqrt(128))), what=f"fp8 Skv{Skv}")


def test_fp8_block_scales_vary_along_keys():
    """K/V blocks of very different magnitude (per-block scales from 2^-6 to
    2^7) and an all-zero block: every key tile uses its own scales."""
    say("fp8 varying block scales")
    B, H, S, d = 1, 2, 640, 128
    g = wl.generate("flux", seed=901, B=B, H=H, Sq=200, Skv=S, d=d)
    for name, facs in (("k", [1.0, 0.05, 3.0, 0.0, 0.5]), ("v", [100.0, 0.02, 1.0, 7.0, 0.0])):
        x = wl.bf16_bits_to_f32(g[name]).copy()
        for blk, f in enumerate(facs):
            x[:, 128 * blk:128 * (blk + 1)] *= np.float32(f)
        g[name] = wl.f32_to_bf16_bits(x)
    check_against_dequant(g, float(np.float32(1 / math.sqrt(d))), what="fp8 varying scales")


@pytest.mark.parametrize("B,H,Sq,Skv,d", [(1, 2, 256, 2048, 128), (2, 3, 300, 1000, 64),
                                          (1, 1, 1, 5000, 128)])
def test_fp8_split_launch(B, H, Sq, Skv, d):
    """Shapes whose last wave of query tiles is split over the keys: the merged
    O is sum_j P~_j v_j / sum_j P~_j over all keys (each piece's O is weighted
    by its rounded-weight sum), so the per-element bound holds as for the
    unsplit launch; the two launches agree to twice that bound."""
    from attention_non_causal_amd import _lib
    say(f"fp8 split B{B} H{H} Sq{Sq} Skv{Skv} d{d}")
    assert _lib.dit_attn_fwd_workspace_size(B, H, Sq, Skv, d, _lib.DIT_DTYPE_FP8_E4M3) > 0, \
        "this shape is expected to be split"
    g = wl.generate("flux", seed=950 + Sq + Skv + d, B=B, H=H, Sq=Sq, Skv=Skv, d=d)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, l = check_against_dequant(g, scale, what=f"fp8 split B{B}H{H}Sq{Sq}Skv{Skv}d{d}")
    o1, l1 = run_fp8(g, scale, workspace=None)
    qd, kd, vd = dequant(g["q"]), dequant(g["k"]), dequant(g["v"])
    bound = kernel_bound(qd, kd, vd, scale)
    say(f"  split vs unsplit: max|dO| {np.abs(o - o1).max():.2e} max|dLSE| {np.abs(l - l1).max():.2e}")
    assert (np.abs(o - o1) <= 2 * bound).all()
    assert np.abs(l - l1).max() <= 2e-3


def test_fp8_split_deterministic():
    say("fp8 split determinism")
    g = wl.generate("flux", seed=903, B=1, H=2, Sq=256, Skv=2048, d=128)
    o1, l1 = run_fp8(g, 0.088)
    for _ in range(3):
        o2, l2 = run_fp8(g, 0.088)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_fp8_deterministic():
    say("fp8 determinism")
    g = wl.generate("flux", seed=902, B=1, H=3, Sq=256, Skv=500, d=128)
    o1, l1 = run_fp8(g, 0.088)
    for _ in range(3):
        o2, l2 = run_fp8(g, 0.088)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)


def test_fp8_unit_normal_flux_contract():
    """The contract gate: unit-normal FLUX-like inputs, fp8 path vs the oracle
    on the unquantised inputs, max|dO| <= 6e-2 (sampled rows, full keys)."""
    W = wl.WORKLOADS["flux"]
    say("fp8 unit-normal FLUX: generating inputs")
    g = wl.generate(W)
    # whole 128-row query tiles: 0 (a main tile of every head), 36 and 131
    # (split over the keys for head 23 on a GPU of 256 compute units)
    rows = _gpu.tile_rows(W.Sq, (0, 36, 131), tile=128)
    o, l = run_fp8(g, W.scale)
    say("fp8 unit-normal FLUX: oracle on sampled rows")
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], W.scale, rows=rows)
    # the quantisation floor on the same rows (oracle only): attention on the
    # dequantised inputs against attention on the originals
    o_fl, _ = oracle.attn_fwd(dequant(g["q"]), dequant(g["k"]), dequant(g["v"]), W.scale,
                              rows=rows)
    floor_rr = np.sqrt(((o_fl - o_ref) ** 2).sum() / (o_ref ** 2).sum())
    say(f"fp8 unit-normal FLUX: quantisation floor relRMS={floor_rr:.3e} "
        f"max|dO|={np.abs(o_fl - o_ref).max():.3e}")
    compare(o[:, rows], l[:, :, rows], o_ref, l_ref, o_tol=FP8_O_TOL, lse_tol=5e-2,
            rel_rms=1.1 * floor_rr + 5e-3, what="fp8 FLUX unit-normal vs unquantised")


def test_fp8_outlier_flux_kernel_error():
    """The x8-outlier workload: the kernel's error against the dequantised
    reference must stay inside its bound; the total error against the
    unquantised inputs is reported (the quantisation floor is ~1.1)."""
    W = wl.WORKLOADS["flux_fp8"]
    say("fp8 outlier FLUX: generating inputs")
    g = wl.generate(W)
    # the last 128-row query tile (split over the keys for head 23) and 8 more
    rows = _gpu.tile_rows(W.Sq, (131,), tile=128, extra=8)
    o, l = check_against_dequant(g, W.scale, rows=rows, what="fp8 FLUX outliers")
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], W.scale, rows=rows)
    say(f"fp8 FLUX outliers vs unquantised: max|dO|={np.abs(o - o_ref).max():.3e} "
        f"max|dLSE|={np.abs(l - l_ref).max():.3e}")


def test_fp8_single_key_score_precision():
    """With one key the LSE is the score itself, so the fp8 path's LSE minus the
    exact score of the dequantised inputs is the error of the fp8 dot product
    (the matrix instruction's accumulation) plus fp32 rounding.  Inputs: e4m3
    Q/K with 1% x8 outlier channels and a few query rows whose outlier channel
    meets a key outlier (products 64x the others).  The error must stay within
    MFMA_FP8_REL (2^-12) of scale * sum_c |q_c k_c|; the measured ratio is
    printed (about 2^-13)."""
    say("fp8 single-key score precision")
    B, H, Sq, d = 1, 8, 512, 128
    g = wl.generate("flux_fp8", seed=990, B=B, H=H, Sq=Sq, Skv=1, d=d)
    qf = wl.bf16_bits_to_f32(g["q"]).copy()
    kf = wl.bf16_bits_to_f32(g["k"]).copy()
    qf[:, :64, :, 5] *= np.float32(8.0)                       # a channel both carry
    kf[:, :, :, 5] *= np.float32(8.0)
    g["q"], g["k"] = wl.f32_to_bf16_bits(qf), wl.f32_to_bf16_bits(kf)
    scale = float(np.float32(1 / math.sqrt(d)))
    _, l = run_fp8(g, scale)
    qd, kd = dequant(g["q"]), dequant(g["k"])
    s_exact = np.einsum("bqhc,bhc->bhq", qd, kd[:, 0]) * scale
    a = np.einsum("bqhc,bhc->bhq", np.abs(qd), np.abs(kd[:, 0])) * scale
    ratio = np.abs(l - s_exact) / np.maximum(a, 1e-30)
    say(f"  max |dLSE| {np.abs(l - s_exact).max():.3e}; max |dLSE| / (scale sum|q k|) = "
        f"{ratio.max():.3e} = 2^{math.log2(max(ratio.max(), 1e-30)):.1f}")
    assert (np.abs(l - s_exact) <= MFMA_FP8_REL * a + 1e-6 * np.abs(s_exact) + 1e-6).all()
