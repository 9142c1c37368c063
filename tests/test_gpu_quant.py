"""GPU e4m3 quantiser (dit_quant_fp8) against the oracle's quantiser: the bytes
and the fp32 scales must be identical (the arithmetic is fixed step by step)."""
import numpy as np
import pytest
import torch

import oracle
from attention_non_causal_amd import functional as F, workloads as wl
from tests._gpu import dev_bf16, say

pytestmark = pytest.mark.gpu


def _gpu_quant(x_bits):
    x8, sc = F.quantize_fp8(dev_bf16(x_bits))
    torch.cuda.synchronize()
    return x8.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("B,S,H,d", [(1, 256, 2, 64), (2, 300, 3, 128), (1, 1, 1, 64),
                                     (1, 127, 4, 128), (1, 129, 5, 64)])
def test_quant_bit_exact(B, S, H, d):
    say(f"quant B{B} S{S} H{H} d{d}")
    x = wl.generate("flux_fp8", seed=500 + S, B=B, H=H, Sq=S, Skv=S, d=d)["k"]
    q_gpu, s_gpu = _gpu_quant(x)
    q_ref, s_ref = oracle.quant_fp8(x)
    np.testing.assert_array_equal(s_gpu, s_ref)
    np.testing.assert_array_equal(q_gpu, q_ref)


def test_quant_zero_block_and_extremes():
    say("quant zero block / extremes")
    B, S, H, d = 1, 384, 2, 128
    x = wl.normal_bf16((B, S, H, d), 600)
    x[0, 128:256, 0] = 0
    x[0, 256:, 1] = 0x8000                      # negative zeros only
    x[0, 5, 1, 7] = wl.f32_to_bf16_bits(np.float32([3.0e38]))[0]
    x[0, 6, 1, 9] = wl.f32_to_bf16_bits(np.float32([-1.0e-30]))[0]
    q_gpu, s_gpu = _gpu_quant(x)
    q_ref, s_ref = oracle.quant_fp8(x)
    np.testing.assert_array_equal(s_gpu, s_ref)
    np.testing.assert_array_equal(q_gpu, q_ref)


def test_quant_flux_fp8_full_size():
    say("quant flux_fp8 full size (Q, K, V)")
    g = wl.generate("flux_fp8")
    for n in "qkv":
        q_gpu, s_gpu = _gpu_quant(g[n])
        q_ref, s_ref = oracle.quant_fp8(g[n])
        np.testing.assert_array_equal(s_gpu, s_ref)
        np.testing.assert_array_equal(q_gpu, q_ref)


def test_quant_nonfinite_input_matches_oracle():
    """NaNs (both signs, with a payload), infinities and an all-NaN-and-zero
    block: bytes and scales identical to the oracle's (NaN out of amax and
    encoded 0x7F; an infinite amax gives scale +inf and signed zeros)."""
    from tests.test_oracle_fp8 import _nonfinite_blocks
    say("quant non-finite input")
    x = _nonfinite_blocks()
    q_gpu, s_gpu = _gpu_quant(x)
    q_ref, s_ref = oracle.quant_fp8(x)
    np.testing.assert_array_equal(s_gpu, s_ref)
    np.testing.assert_array_equal(q_gpu, q_ref)
