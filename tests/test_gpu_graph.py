"""The library's calls captured into a HIP graph (through torch.cuda.CUDAGraph,
which captures the stream the calls launch on): the header promises that every
call only enqueues work, allocates nothing and never synchronises.

The graph holds the split bf16 forward (forward kernel + split merge), a
two-part merge, the fp8 quantiser with the fp8 split forward, and a chain of
two dit_attn_fwd_acc blocks whose running LSE is reset by a copy (no memset is
recorded).  It is replayed several times with the program's own eager work
and synchronisations in between; every replay must reproduce the eager results
bit for bit (the kernels are deterministic) and match the fp64 oracle: the bf16
outputs within max|dO| <= 1e-2 / max|dLSE| <= 1e-3 of the oracle over all keys,
the fp8 output within its per-element bound against the oracle on the
dequantised inputs.  A second graph holds the Wan-like ring share as a ring
loop runs it (LSE reset by a fill kernel, four dit_attn_fwd_acc chunks) at full
size, each replay checked against the oracle over all 32760 keys.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from attention_non_causal_amd import _lib, functional as F, workloads as wl
from tests import _gpu
from tests._gpu import compare, dev_bf16, host_f64, say

pytestmark = pytest.mark.gpu


def _inputs(B, H, Sq, Skv, d, seed):
    g = wl.generate("tiny", seed=seed, B=B, H=H, Sq=Sq, Skv=Skv, d=d)
    return g, (dev_bf16(g["q"]), dev_bf16(g["k"]), dev_bf16(g["v"]))


def test_graph_replays_match_eager():
    B, H, Sq, Skv, d = 1, 2, 256, 2048, 128
    say("graph capture: inputs and eager results")
    g, (q, k, v) = _inputs(B, H, Sq, Skv, d, seed=6000)
    scale = 0.088
    dev = q.device
    ws = F.workspace_for(q, k)
    assert ws is not None, "this shape is expected to be split"
    half = Skv // 2
    k1, v1 = k[:, :half].contiguous(), v[:, :half].contiguous()
    k2, v2 = k[:, half:].contiguous(), v[:, half:].contiguous()
    nws_half = _lib.dit_attn_fwd_workspace_size(B, H, Sq, half, d)
    ws_half = torch.empty(max(nws_half, 16), dtype=torch.uint8, device=dev)
    neg_inf = torch.full((B, H, Sq), -math.inf, dtype=torch.float32, device=dev)
    nblk = (Skv + 127) // 128

    def bufs():
        return dict(
            o=torch.empty((B, Sq, H, d), dtype=torch.bfloat16, device=dev),
            l=torch.empty((B, H, Sq), dtype=torch.float32, device=dev),
            o1=torch.empty((B, Sq, H, d), dtype=torch.bfloat16, device=dev),
            l1=torch.empty((B, H, Sq), dtype=torch.float32, device=dev),
            o2=torch.empty((B, Sq, H, d), dtype=torch.bfloat16, device=dev),
            l2=torch.empty((B, H, Sq), dtype=torch.float32, device=dev),
            om=torch.empty((B, Sq, H, d), dtype=torch.bfloat16, device=dev),
            lm=torch.empty((B, H, Sq), dtype=torch.float32, device=dev),
            q8=torch.empty((B, Sq, H, d), dtype=torch.uint8, device=dev),
            qs=torch.empty((B, H, (Sq + 127) // 128), dtype=torch.float32, device=dev),
            k8=torch.empty((B, Skv, H, d), dtype=torch.uint8, device=dev),
            ks=torch.empty((B, H, nblk), dtype=torch.float32, device=dev),
            v8=torch.empty((B, Skv, H, d), dtype=torch.uint8, device=dev),
            vs=torch.empty((B, H, nblk), dtype=torch.float32, device=dev),
            of=torch.empty((B, Sq, H, d), dtype=torch.bfloat16, device=dev),
            lf=torch.empty((B, H, Sq), dtype=torch.float32, device=dev),
            oa=torch.empty((B, Sq, H, d), dtype=torch.bfloat16, device=dev),
            la=torch.empty((B, H, Sq), dtype=torch.float32, device=dev),
        )

    ws8 = None

    def work(t):
        nonlocal ws8
        F.attention(q, k, v, scale, out=t["o"], lse=t["l"], workspace=ws)
        F.attention(q, k1, v1, scale, out=t["o1"], lse=t["l1"], workspace=None)
        F.attention(q, k2, v2, scale, out=t["o2"], lse=t["l2"], workspace=None)
        F.merge([t["o1"], t["o2"]], [t["l1"], t["l2"]], out=t["om"], lse=t["lm"])
        for x, x8, xs, S in ((q, t["q8"], t["qs"], Sq), (k, t["k8"], t["ks"], Skv),
                             (v, t["v8"], t["vs"], Skv)):
            _lib.dit_quant_fp8(x, x8, xs, B, H, S, d)
        if ws8 is None:
            ws8 = F.workspace_for(t["q8"], t["k8"], _lib.DIT_DTYPE_FP8_E4M3)
        F.attention_fp8(t["q8"], t["qs"], t["k8"], t["ks"], t["v8"], t["vs"], scale,
                        out=t["of"], lse=t["lf"], workspace=ws8)
        t["la"].copy_(neg_inf)
        F.attention_acc(q, k1, v1, t["oa"], t["la"], scale, workspace=ws_half)
        F.attention_acc(q, k2, v2, t["oa"], t["la"], scale, workspace=ws_half)

    eager = bufs()
    work(eager)
    torch.cuda.synchronize()
    for name in ("o", "om", "of", "oa"):
        assert torch.isfinite(eager[name].float()).all(), name

    say("graph capture: capturing")
    static = bufs()
    work(static)  # warm up on the side stream torch captures on
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work(static)
    torch.cuda.synchronize()

    # the oracle: attention over all keys (the split forward, the merge of the
    # two halves and the accumulated chain all compute it), and the fp8 path's
    # reference on the dequantised inputs with its per-element bound
    from tests.test_gpu_fp8 import dequant, kernel_bound, lse_bound
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], scale)
    qd8, kd8, vd8 = dequant(g["q"]), dequant(g["k"]), dequant(g["v"])
    o8_ref, l8_ref = oracle.attn_fwd(qd8, kd8, vd8, scale)
    bound8 = kernel_bound(qd8, kd8, vd8, scale)
    lbound8 = lse_bound(qd8, kd8, scale)

    def check_oracle(t, what):
        for o_name, l_name in (("o", "l"), ("om", "lm"), ("oa", "la")):
            compare(host_f64(t[o_name]), host_f64(t[l_name]), o_ref, l_ref,
                    what=f"{what} {o_name}")
        err8 = np.abs(host_f64(t["of"]) - o8_ref)
        say(f"{what} of: max|dO| {err8.max():.3e} (worst err/bound {(err8 / bound8).max():.3f})")
        assert (err8 <= bound8).all(), f"{what}: fp8 output outside its bound"
        assert (np.abs(host_f64(t["lf"]) - l8_ref) <= lbound8).all()

    check_oracle(eager, "eager")
    for rep in range(3):
        say(f"graph capture: replay {rep}")
        for t in static.values():  # outputs poisoned between replays
            t.view(torch.uint8).fill_(0xFF)
        other = bufs()  # the program's own eager work in between
        work(other)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in eager:
            a, b = static[name], eager[name]
            same = torch.equal(a.view(torch.uint8), b.view(torch.uint8))
            assert same, f"replay {rep}: {name} differs from the eager result"
        for name in ("o", "om", "of", "oa"):
            assert torch.equal(other[name].view(torch.uint8), eager[name].view(torch.uint8)), name
        check_oracle(static, f"replay {rep}")


def test_graph_wan_ring_share_accumulated_against_oracle():
    """The Wan-like ring share (B1 H40 d128, 8190 queries, 4 chunks of 8190
    keys) captured as a ring loop runs it -- the running LSE reset to -inf by a
    fill kernel, then four dit_attn_fwd_acc launches -- and replayed three
    times with eager work in between; every replay against the oracle over all
    32760 keys on 264 rows (the first query tile and 8 more)."""
    W = wl.WORKLOADS["wan_ring"]
    say("graph wan ring share: generating inputs")
    g = wl.generate(W)
    q, k, v = dev_bf16(g["q"]), dev_bf16(g["k"]), dev_bf16(g["v"])
    dev = q.device
    o = torch.empty_like(q)
    lse = torch.empty((1, W.H, W.Sq), dtype=torch.float32, device=dev)
    n = _lib.dit_attn_fwd_workspace_size(1, W.H, W.Sq, W.chunk, W.d)
    ws = torch.empty(n, dtype=torch.uint8, device=dev) if n else None

    def share():
        F.ring_share_attention_acc(q, k, v, W.n_chunks, W.scale, out=o, lse=lse, workspace=ws)

    share()  # warm up on the side stream torch captures on
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        share()
    torch.cuda.synchronize()
    rows = _gpu.tile_rows(W.Sq, (0,), extra=8)
    say(f"graph wan ring share: oracle on {len(rows)} rows")
    o_ref, l_ref = oracle.attn_fwd(g["q"], g["k"], g["v"], W.scale, rows=rows)
    scratch_o = torch.empty_like(o)
    for rep in range(3):
        say(f"graph wan ring share: replay {rep}")
        o.view(torch.uint8).fill_(0xFF)
        lse.fill_(float("nan"))
        F.attention(q[:, :512].contiguous(), k[:, :512].contiguous(), v[:, :512].contiguous(),
                    W.scale, out=scratch_o[:, :512])  # the program's own eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        compare(host_f64(o)[:, rows], host_f64(lse)[:, :, rows], o_ref, l_ref,
                what=f"graph wan replay {rep}")
