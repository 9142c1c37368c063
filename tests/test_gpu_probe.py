"""The probes behind `bench.py --mfma-ceiling` and `bench.py --valu-issue`
(libditprobe.so, not part of the attention library) run on the GPU.  The
matrix-core probe returns finite sums: one short launch per instruction kind,
with zero and with N(0,1) operands, where the zero operands must give exact
zeros.  The vector-issue probe returns one positive cycle count per wave, at
least the instructions it issued."""
import ctypes
import os

import numpy as np
import pytest
import torch

from attention_non_causal_amd import build as libbuild

from ._gpu import device, say

pytestmark = pytest.mark.gpu


def _probe():
    assert os.path.exists(libbuild.PROBE_LIB_PATH), "libditprobe.so missing: run build()"
    lib = ctypes.CDLL(libbuild.PROBE_LIB_PATH)
    lib.dit_probe_mfma_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.dit_probe_mfma_ceiling.restype = ctypes.c_int
    lib.dit_probe_valu_issue.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.dit_probe_valu_issue.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("kind", [0, 1])
def test_probe_runs(kind):
    lib = _probe()
    dev = device()
    n_blocks = 8
    out = torch.full((n_blocks * 256,), float("nan"), device=dev)
    zeros = torch.zeros(4096, dtype=torch.int32, device=dev)
    say(f"mfma probe kind {kind}, zero operands")
    assert lib.dit_probe_mfma_ceiling(zeros.data_ptr(), out.data_ptr(), n_blocks, 3, kind, None) == 0
    torch.cuda.synchronize()
    assert (out == 0).all()
    rng = np.random.default_rng(3)
    if kind == 0:
        x = torch.from_numpy(rng.standard_normal(8192).astype(np.float32)).to(torch.bfloat16)
        src = x.view(torch.int16).to(dev).view(torch.int32)
    else:
        src = torch.from_numpy(rng.integers(0, 0x7f, 16384, dtype=np.uint8)).to(dev).view(torch.int32)
    say(f"mfma probe kind {kind}, random operands")
    assert lib.dit_probe_mfma_ceiling(src.data_ptr(), out.data_ptr(), n_blocks, 3, kind, None) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and (out != 0).any()
    assert lib.dit_probe_mfma_ceiling(None, out.data_ptr(), n_blocks, 3, kind, None) != 0


@pytest.mark.parametrize("kind", range(6))
@pytest.mark.parametrize("waves", [4, 8])
def test_valu_issue_probe_runs(kind, waves):
    lib = _probe()
    dev = device()
    n_blocks, iters = 8, 16
    out = torch.zeros(n_blocks * waves, dtype=torch.int64, device=dev)
    say(f"valu issue probe kind {kind}, {waves} waves per workgroup")
    assert lib.dit_probe_valu_issue(out.data_ptr(), n_blocks, waves, iters, kind, None) == 0
    torch.cuda.synchronize()
    cyc = out.cpu().numpy()
    # a wave issues at most one vector instruction per cycle
    assert (cyc >= 16 * iters).all() and (cyc < 10 ** 9).all()
    assert lib.dit_probe_valu_issue(out.data_ptr(), n_blocks, 5, iters, kind, None) != 0
    assert lib.dit_probe_valu_issue(None, n_blocks, waves, iters, kind, None) != 0
