"""Seeded synthetic inputs for the DiT attention workloads.

This module only *draws* inputs: it holds none of the attention, merge or
quantisation arithmetic, and it is the one piece shared by the HIP path's tests
and the CPU oracle's tests.  It imports neither side.

Workloads (shapes only; tokens are iid synthetic stand-ins, no dataset or
trained weights):

* ``tiny``      B1 H2 d64, Sq=Skv=256 (a 16x16 patch grid)
* ``sd3``       B2 (cond/uncond CFG pair) H24 d64, S = 4096 image + 154 text
                = 4250 tokens, Q/K RMS-normalised per (b, s, h)
* ``flux``      B1 H24 d128, S = 16384 image + 512 text = 16896, Q/K RMS-normed
* ``flux_fp8``  as ``flux``, then 1% of the H*d channels of each of Q, K, V
                (31 channels, drawn independently per tensor) multiplied by 8
                across all tokens, before e4m3 quantisation
* ``flux_h3``   as ``flux`` with H3: what each GPU runs when 8-way Ulysses
                shards the 24 heads ("xDiT 项目概述" sec. 3.2.2: the Ulysses
                dimension splits by heads; sec. 3.2.3 suggests degree 8 on fast
                links)
* ``wan_ring``  B1 H40 d128, a 21x30x52 = 32760-token video sequence seen by one
                of four ring ranks: 8190 local queries against all 32760 keys,
                handled as 4 KV chunks of 8190 whose partials are merged

The pages motivate these shapes: joint text+image/video sequences of tens of
thousands of tokens ("xDiT 项目概述" sec. 2.2), CFG's cond/uncond pair
(sec. 3.3.1), the ring split of the sequence into blocks (sec. 3.2), and seed 42
from the quick-start table of "AMD、Radeon AI PRO R9700S最大4台で...".

Recipe: root ``numpy.random.SeedSequence(seed)`` spawns one child stream per
tensor in the order Q, K, V, outlier-Q, outlier-K, outlier-V.  Values are drawn
as fp32 N(0, 1), optionally RMS-normalised per (b, s, h) in fp32 with eps 1e-6
and no learned weight, optionally given the x8 outlier channels, then rounded to
bf16 with round-to-nearest-even.  The returned arrays hold bf16 bit patterns as
uint16; the same bytes go to the GPU and to the oracle.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

ROOT_SEED = 42


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    Sq: int
    Skv: int
    qk_norm: bool = False
    fp8: bool = False
    outlier_frac: float = 0.0
    n_chunks: int = 1
    description: str = ""

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), as the fp32 value passed to the kernels."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> float:
        """Algorithmic FLOPs of the forward pass: 4*B*H*Sq*Skv*d."""
        return 4.0 * self.B * self.H * self.Sq * self.Skv * self.d

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes the forward pass must move at least once: Q, K, V read, O and
        LSE written (bf16 tensors, fp32 LSE)."""
        return 2 * self.B * self.H * self.d * (2 * self.Sq + 2 * self.Skv) + 4 * self.B * self.H * self.Sq

    @property
    def chunk(self) -> int:
        assert self.Skv % self.n_chunks == 0
        return self.Skv // self.n_chunks


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, 256, 256,
                     description="B1 H2 d64 S256, bf16 N(0,1)"),
    "sd3": Workload("sd3", 2, 24, 64, 4250, 4250, qk_norm=True,
                    description="SD3-like 1024^2 joint attention, B2 H24 d64 S4250"),
    "flux": Workload("flux", 1, 24, 128, 16896, 16896, qk_norm=True,
                     description="FLUX-like 2048^2 joint attention, B1 H24 d128 S16896 bf16"),
    "flux_fp8": Workload("flux_fp8", 1, 24, 128, 16896, 16896, qk_norm=True, fp8=True,
                         outlier_frac=0.01,
                         description="FLUX-like shape, e4m3 per-(head,128-token) scales, "
                                     "1% channels x8"),
    # the shape each GPU runs under 8-way Ulysses (24 heads / 8)
    "flux_h3": Workload("flux_h3", 1, 3, 128, 16896, 16896, qk_norm=True,
                        description="FLUX-like shape, one GPU's share of 8-way Ulysses: "
                                    "B1 H3 d128 S16896 bf16"),
    "wan_ring": Workload("wan_ring", 1, 40, 128, 8190, 32760, n_chunks=4,
                         description="Wan-like video, one ring rank's share: Sq8190 vs "
                                     "Skv32760 in 4 chunks + merge"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even) and return the bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _rms_norm(x: np.ndarray) -> np.ndarray:
    ms = np.mean(np.square(x, dtype=np.float32), axis=-1, keepdims=True, dtype=np.float32)
    return (x / np.sqrt(ms + np.float32(1e-6))).astype(np.float32)


def _outlier_channels(rng: np.random.Generator, H: int, d: int, frac: float) -> np.ndarray:
    n_out = int(math.ceil(frac * H * d))
    return rng.choice(H * d, size=n_out, replace=False)


def _apply_outliers(x: np.ndarray, chans: np.ndarray, factor: float = 8.0) -> np.ndarray:
    B, S, H, d = x.shape
    flat = x.reshape(B, S, H * d)
    flat[:, :, chans] *= np.float32(factor)
    return flat.reshape(B, S, H, d)


def generate(wl: Workload | str, seed: int = ROOT_SEED, *, B=None, H=None, Sq=None,
             Skv=None, d=None):
    """Draw (q, k, v) bf16 bit arrays for a workload.

    Shape overrides let tests draw smaller tensors with the same value
    structure (norm, outliers).  Returns a dict with ``q`` [B,Sq,H,d],
    ``k``/``v`` [B,Skv,H,d] (uint16 bf16 bits) and, for fp8 workloads, the
    outlier channel indices used for each tensor.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    Sq = wl.Sq if Sq is None else Sq
    Skv = wl.Skv if Skv is None else Skv
    d = wl.d if d is None else d
    children = np.random.SeedSequence(seed).spawn(6)
    rq, rk, rv, oq, ok, ov = (np.random.default_rng(c) for c in children)
    q = _normal(rq, (B, Sq, H, d))
    k = _normal(rk, (B, Skv, H, d))
    v = _normal(rv, (B, Skv, H, d))
    if wl.qk_norm:
        q = _rms_norm(q)
        k = _rms_norm(k)
    out = {}
    if wl.outlier_frac > 0:
        cq = _outlier_channels(oq, H, d, wl.outlier_frac)
        ck = _outlier_channels(ok, H, d, wl.outlier_frac)
        cv = _outlier_channels(ov, H, d, wl.outlier_frac)
        q = _apply_outliers(q, cq)
        k = _apply_outliers(k, ck)
        v = _apply_outliers(v, cv)
        out.update(outliers_q=cq, outliers_k=ck, outliers_v=cv)
    out.update(q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v))
    return out


def normal_bf16(shape, seed: int) -> np.ndarray:
    """bf16 bits of fp32 N(0,1) draws from one seeded stream (small test tensors)."""
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    return f32_to_bf16_bits(_normal(rng, shape))


def sample_rows(Sq: int, n: int, seed: int = ROOT_SEED, tile: int = 128) -> np.ndarray:
    """A deterministic set of query rows for sampled checks at full size: the
    first and last rows, rows on both sides of every 4th tile boundary up to n/2,
    and the rest drawn uniformly without replacement."""
    must = {0, Sq - 1}
    for t in range(tile, Sq, tile * 4):
        must.update({t - 1, t})
        if len(must) >= n // 2:
            break
    must = sorted(r for r in must if 0 <= r < Sq)
    rng = np.random.default_rng(np.random.SeedSequence([seed, Sq, n]))
    rest = np.setdiff1d(np.arange(Sq), np.array(must))
    k = max(0, min(n - len(must), rest.size))
    extra = rng.choice(rest, size=k, replace=False) if k else np.array([], dtype=np.int64)
    return np.sort(np.concatenate([np.array(must, dtype=np.int64), extra])).astype(np.int32)
