"""Race check through the C ABI: the library built with -DDIT_DEBUG_BARRIERS
(libditattn_debugsync.so: each step of the forward kernels' key loop ends with
every memory operation of the wave waited for and a workgroup barrier -- see
debug_sync in csrc/common.hpp) against the normal build, bit for bit.

Both builds do the same arithmetic in the same order; the debug build only
takes away the freedom of a workgroup's waves to run apart and of LDS copies
to land late.  A result that differs between the two would depend on how the
waves interleave: a read of an LDS slot before its copy landed, or a slot
overwritten while another wave still reads it.  Cases: several query and key
tiles with ragged tails, split launches (workspace), the running-result
merge, both head sizes, bf16 and e4m3, and the FLUX-like shape at full size.
"""
import numpy as np
import pytest
import torch

from attention_non_causal_amd import _lib
from attention_non_causal_amd import functional as F
from attention_non_causal_amd import workloads as wl

from ._gpu import dev_bf16, device, say

pytestmark = pytest.mark.gpu


def _inputs(B, H, Sq, Skv, d, seed):
    rng = np.random.default_rng(seed)

    def t(S):
        x = rng.standard_normal((B, S, H, d)).astype(np.float32)
        return torch.from_numpy(x).to(device()).to(torch.bfloat16)

    return t(Sq), t(Skv), t(Skv)


def _both(run, what):
    """run() -> tuple of tensors; compared bit for bit between the builds."""
    say(f"{what}: normal build")
    a = [x.detach().cpu().clone() for x in run()]
    torch.cuda.synchronize()
    with _lib.use_library(_lib.DEBUG_LIB_PATH):
        say(f"{what}: debug-barrier build")
        b = [x.detach().cpu().clone() for x in run()]
        torch.cuda.synchronize()
    for i, (x, y) in enumerate(zip(a, b)):
        assert x.shape == y.shape
        xb = x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)
        yb = y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)
        n = int((xb != yb).sum())
        assert n == 0, f"{what}: output {i} differs in {n} elements between the builds"


def test_debug_build_is_loaded_as_a_separate_library():
    import os
    assert os.path.exists(_lib.DEBUG_LIB_PATH), (
        "libditattn_debugsync.so is missing: __graft_entry__.build() builds it")
    main = _lib.load()
    with _lib.use_library(_lib.DEBUG_LIB_PATH) as dbg:
        assert dbg is not main and _lib.load() is dbg
    assert _lib.load() is main


@pytest.mark.parametrize("B,H,Sq,Skv,d", [(1, 3, 1000, 777, 128), (2, 2, 777, 1000, 64),
                                           (1, 24, 300, 2100, 128)])
def test_bf16_forward_same_bits(B, H, Sq, Skv, d):
    q, k, v = _inputs(B, H, Sq, Skv, d, seed=7 + d + Skv)
    scale = d ** -0.5

    def run():
        ws = F.workspace_for(q, k)
        return F.attention(q, k, v, scale, workspace=ws)

    _both(run, f"bf16 B{B} H{H} Sq{Sq} Skv{Skv} d{d}")


@pytest.mark.parametrize("B,H,Sq,Skv,d", [(1, 3, 1000, 777, 128), (2, 2, 777, 1000, 64),
                                           (1, 24, 300, 2100, 128)])
def test_fp8_forward_same_bits(B, H, Sq, Skv, d):
    q, k, v = _inputs(B, H, Sq, Skv, d, seed=11 + d + Skv)
    scale = d ** -0.5

    def run():
        q8, k8, v8 = F.quantize_fp8(q), F.quantize_fp8(k), F.quantize_fp8(v)
        ws = F.workspace_for(q8[0], k8[0], _lib.DIT_DTYPE_FP8_E4M3)
        return F.attention_fp8(q8[0], q8[1], k8[0], k8[1], v8[0], v8[1], scale, workspace=ws)

    _both(run, f"fp8 B{B} H{H} Sq{Sq} Skv{Skv} d{d}")


def test_bf16_running_result_same_bits():
    B, H, Sq, Skv, d = 1, 4, 600, 1500, 128
    q, k, v = _inputs(B, H, Sq, Skv, d, seed=5)
    scale = d ** -0.5

    def run():
        o = torch.empty_like(q)
        lse = torch.full((B, H, Sq), float("-inf"), device=device())
        for a, b in ((0, 700), (700, Skv)):
            F.attention_acc(q, k[:, a:b].contiguous(), v[:, a:b].contiguous(), o, lse, scale)
        return o, lse

    _both(run, "bf16 running result, two key blocks")


def test_flux_full_size_same_bits():
    W = wl.WORKLOADS["flux"]
    g = wl.generate(W)
    q, k, v = dev_bf16(g["q"]), dev_bf16(g["k"]), dev_bf16(g["v"])
    del g

    def run_bf16():
        return F.attention(q, k, v, W.scale, workspace=F.workspace_for(q, k))

    _both(run_bf16, "FLUX-like bf16, full size")

    def run_fp8():
        q8, k8, v8 = F.quantize_fp8(q), F.quantize_fp8(k), F.quantize_fp8(v)
        ws = F.workspace_for(q8[0], k8[0], _lib.DIT_DTYPE_FP8_E4M3)
        return F.attention_fp8(q8[0], q8[1], k8[0], k8[1], v8[0], v8[1], W.scale, workspace=ws)

    _both(run_fp8, "FLUX-like fp8, full size")
