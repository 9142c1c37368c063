"""Helpers for the GPU tests: move bf16 bit arrays to the device and back, and
compare against the oracle with the stated tolerances."""
import sys

import numpy as np
import torch

BF16_O_TOL = 1e-2      # max |dO|   (bf16 inputs, fp32 accumulation)
BF16_LSE_TOL = 1e-3    # max |dLSE|
REL_RMS_TOL = 1e-2     # internal gate: ||dO||_2 / ||O||_2
FP8_O_TOL = 6e-2       # max |dO| for the fp8 path on unit-normal inputs


def say(msg: str) -> None:
    """Name the case before each GPU step (flushed, so a fault still shows it)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def device():
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    return torch.device("cuda:0")


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device())


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def compare(o_gpu, lse_gpu, o_ref, lse_ref, o_tol=BF16_O_TOL, lse_tol=BF16_LSE_TOL,
            rel_rms=REL_RMS_TOL, what=""):
    """Element-wise comparison; returns (max|dO|, max|dLSE|, rel_rms)."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite O"
    assert np.isfinite(lse_gpu).all(), f"{what}: non-finite LSE"
    do = np.abs(o_gpu - o_ref).max()
    dl = np.abs(lse_gpu - lse_ref).max()
    rr = np.sqrt(((o_gpu - o_ref) ** 2).sum() / max(((o_ref) ** 2).sum(), 1e-300))
    say(f"{what}: max|dO|={do:.3e} max|dLSE|={dl:.3e} relRMS={rr:.3e}")
    assert do <= o_tol, f"{what}: max|dO| {do} > {o_tol}"
    assert dl <= lse_tol, f"{what}: max|dLSE| {dl} > {lse_tol}"
    if rel_rms is not None:
        assert rr <= rel_rms, f"{what}: relative RMS {rr} > {rel_rms}"
    return do, dl, rr


FEW_KEYS = 8  # up to this many keys a row's O can be as large as |V|


def few_key_o_tol(v_bits) -> float:
    """max|dO| budget where few keys (or a softmax so peaked that one key
    dominates) make |O| as large as |V|.

    The kernel rounds each softmax weight P_j to bf16 before P.V (relative
    error <= 2^-9) while the row sum uses the unrounded weights, and rounds O
    to bf16 (<= 2^-9 |O|), so |dO| <= 2^-9 (max_j |v_j| + |O|) <= 2^-8 max|V|.
    The 1e-2 contract tolerance is kept whenever it is the larger.  Only for
    Skv <= FEW_KEYS and for tests built to make one key dominate; everywhere
    else the contract's 1e-2 applies (o_tol)."""
    vmax = float(np.abs((np.asarray(v_bits, dtype=np.uint16).astype(np.uint32) << 16)
                        .view(np.float32)).max())
    return max(BF16_O_TOL, 2.0 ** -8 * vmax)


def tile_rows(Sq: int, tiles, tile: int = 256, extra: int = 0) -> np.ndarray:
    """Query rows of whole query tiles (tile index t: rows t*tile .. t*tile +
    tile - 1, the last one clipped at Sq), plus `extra` rows drawn from the
    rest, sorted."""
    from attention_non_causal_amd import workloads as wl
    rows = set()
    for t in tiles:
        rows.update(range(t * tile, min((t + 1) * tile, Sq)))
    if extra:
        rows.update(int(r) for r in wl.sample_rows(Sq, extra))
    return np.array(sorted(rows), dtype=np.int32)


def o_tol(v_bits, n_keys: int) -> float:
    """The max|dO| gate of a comparison over n_keys keys: the contract's 1e-2,
    or the few-key bound when n_keys <= FEW_KEYS."""
    return few_key_o_tol(v_bits) if n_keys <= FEW_KEYS else BF16_O_TOL


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """One bf16 unit in the last place at |x| (8 significant bits)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)
