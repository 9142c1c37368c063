"""The bf16 forward pass at the largest K/V the library accepts.

One batch of K (or V) may hold up to 2^32 - 1 bytes: the kernels address it
with 32-bit buffer offsets.  Here B1 H1 with Skv = 2^32 / (2d) - 1 keys (d128:
2^24 - 1, d64: 2^25 - 1), so K and V are each 4 GiB - 2d bytes and the last
tiles sit right below the limit.

Expected values in closed form (no pass over 8 GiB on the CPU): every key row
is the same k0 and every value row the same v0, except a few special keys j
(the first, some in the middle, the very last ones) with their own k_j, v_j.
With s_j = scale q.k_j and N0 = Skv - |J| copies of score s_0:
    LSE = ln(N0 e^s0 + sum_J e^sj),  O = (N0 e^s0 v0 + sum_J e^sj v_j) / e^LSE.
Every query row is a_i u plus noise (u a unit vector, a_i from 1 to 2) and
special key j is k0 + (b_j / scale) u, so its score is ~b_j a_i above the bulk's
(b_j = 30 + 0.4 i): the special keys share the weight (within a factor e^4 of
each other), the ~2^24 bulk keys together hold < 2e-6 of it, and reading any
special key from the wrong place changes the result.  (The bulk is kept
negligible on purpose: 2^24 identical keys add the same increment about a
million times into each fp32 accumulator, whose systematic rounding then
reaches ~3% -- a limit of fp32 accumulation, not of addressing.)  Gates, on the plain and the split
launch: max|dLSE| <= 1e-3, and max|dO| <= max(1e-2, 2^-8 max|V|) -- where one
special key dominates, O is about that key's value, whose bf16 weight and output
roundings are each up to 2^-9 of it (tests/_gpu.few_key_o_tol).  All K/V reads
go through range-checked buffer descriptors.
"""
import math

import numpy as np
import pytest
import torch

from attention_non_causal_amd import _lib, functional as F, workloads as wl
from tests._gpu import host_f64, say

pytestmark = pytest.mark.gpu


def _bf16_round(x: np.ndarray) -> np.ndarray:
    return wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


@pytest.mark.parametrize("d", [128, 64])
def test_fwd_at_the_largest_kv(d):
    B, H, Sq = 1, 1, 37
    Skv = (1 << 32) // (2 * d) - 1          # 2d bytes per key: 2^32 - 2d bytes
    assert (Skv + 1) * H * d * 2 == 1 << 32
    rng = np.random.default_rng(7100)
    scale = float(np.float32(1 / math.sqrt(d)))
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    a = 1 + np.arange(Sq) / (Sq - 1)
    q = _bf16_round(a[:, None] * u[None] + 0.05 * rng.standard_normal((Sq, d)))
    k0 = _bf16_round(rng.standard_normal(d) / 8)
    v0 = _bf16_round(rng.standard_normal(d))
    special = [0, Skv // 4, Skv // 2 + 5, Skv - 64, Skv - 2, Skv - 1]
    kj = {j: _bf16_round(k0 + (30 + 0.4 * i) / scale * u) for i, j in enumerate(special)}
    vj = {j: _bf16_round(rng.standard_normal(d)) for j in special}

    say("max-size K/V: building 2 x 4 GiB on the device")
    dev = torch.device("cuda")
    kd = torch.from_numpy(k0).to(dev).to(torch.bfloat16).expand(Skv, d).contiguous()
    vd = torch.from_numpy(v0).to(dev).to(torch.bfloat16).expand(Skv, d).contiguous()
    for j in special:
        kd[j] = torch.from_numpy(kj[j]).to(dev).to(torch.bfloat16)
        vd[j] = torch.from_numpy(vj[j]).to(dev).to(torch.bfloat16)
    kd = kd.view(B, Skv, H, d)
    vd = vd.view(B, Skv, H, d)
    qd = torch.from_numpy(q).to(dev).to(torch.bfloat16).view(B, Sq, H, d)

    # closed form in fp64 on the same bf16 values
    q64 = q.astype(np.float64)
    s0 = scale * q64 @ k0.astype(np.float64)                        # [Sq]
    sj = np.stack([scale * q64 @ kj[j].astype(np.float64) for j in special], 1)
    n0 = Skv - len(special)
    m = np.maximum(s0, sj.max(1))
    w0 = n0 * np.exp(s0 - m)
    wj = np.exp(sj - m[:, None])
    z = w0 + wj.sum(1)
    lse_ref = m + np.log(z)
    o_ref = (w0[:, None] * v0.astype(np.float64)[None] +
             wj @ np.stack([vj[j].astype(np.float64) for j in special])) / z[:, None]
    # every special key matters: leaving out any one of them moves O
    for i in range(len(special)):
        wk = np.delete(wj, i, 1)
        vk = np.delete(np.stack([vj[j].astype(np.float64) for j in special]), i, 0)
        o_wo = (w0[:, None] * v0.astype(np.float64)[None] + wk @ vk) / (w0 + wk.sum(1))[:, None]
        assert np.abs(o_wo - o_ref).max() > 0.1, f"special key {special[i]} carries no weight"
    assert (w0 / z).max() < 2e-6

    o_tol = max(1e-2, 2.0 ** -8 * max([np.abs(v0).max()] + [np.abs(x).max() for x in vj.values()]))
    for launch in ("plain", "split"):
        say(f"max-size K/V: {launch} launch")
        ws = None if launch == "plain" else F.workspace_for(qd, kd)
        if launch == "split":
            assert ws is not None, "one query tile over 2^24 keys is expected to be split"
        o, lse = F.attention(qd, kd, vd, scale, workspace=ws)
        torch.cuda.synchronize()
        og = host_f64(o)[0, :, 0, :]
        lg = host_f64(lse)[0, 0]
        do = np.abs(og - o_ref).max()
        dl = np.abs(lg - lse_ref).max()
        say(f"  {launch}: max|dO|={do:.3e} max|dLSE|={dl:.3e}")
        assert do <= o_tol and dl <= 1e-3
    del kd, vd
    torch.cuda.empty_cache()
