"""The e4m3 quantisation floor at the FLUX-like shape, computed by the oracle
alone (no GPU): attention on dequant(quant(x)) against attention on x, on a
deterministic subset of query rows (all 24 heads, all 16896 keys).

This fixes what any fp8 kernel with per-(head, 128-token block) scales can
reach against the unquantised oracle:
  * unit-normal inputs (RMS-normalised Q/K, N(0,1) V): floor ~3e-3, far inside
    the 6e-2 budget;
  * the x8-outlier inputs: floor ~1.1, because queries whose outlier channel is
    large get very peaked softmax rows whose largest logits move by ~1 under
    e4m3's 2^-4 relative rounding.  The 6e-2 gate therefore cannot apply there;
    the GPU tests gate the kernel's own error against the oracle on the
    dequantised inputs instead and report the total error next to this floor.
"""
import numpy as np
import pytest

import oracle
from attention_non_causal_amd import workloads as wl


def _floor(name, n_rows=16):
    W = wl.WORKLOADS[name]
    g = wl.generate(name)
    rows = wl.sample_rows(W.Sq, n_rows)
    o, l = oracle.attn_fwd(g["q"], g["k"], g["v"], W.scale, rows=rows)
    dq = [oracle.dequant_fp8(*oracle.quant_fp8(g[n])) for n in "qkv"]
    o2, l2 = oracle.attn_fwd(dq[0], dq[1], dq[2], W.scale, rows=rows)
    return np.abs(o2 - o).max(), np.abs(l2 - l).max()


@pytest.mark.slow
def test_fp8_floor_unit_normal_inside_budget():
    do, dl = _floor("flux")
    print(f"unit-normal e4m3 floor: max|dO|={do:.3e} max|dLSE|={dl:.3e}")
    assert do <= 6e-2 / 4


@pytest.mark.slow
def test_fp8_floor_with_outliers_exceeds_budget():
    do, dl = _floor("flux_fp8")
    print(f"outlier e4m3 floor: max|dO|={do:.3e} max|dLSE|={dl:.3e}")
    assert do > 6e-2
