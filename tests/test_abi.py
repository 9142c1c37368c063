"""C-ABI tests that need no GPU: the library loads, exports every function
the public header declares, and rejects every invalid argument with its status
code before any HIP call (fake, never-dereferenced device addresses are used;
no call here reaches a kernel launch)."""
import ctypes
import math
import subprocess

import pytest

from attention_non_causal_amd import _lib
from attention_non_causal_amd._lib import (DIT_DTYPE_BF16, DIT_DTYPE_FP8_E4M3, DIT_ERR_ALIAS,
                                           DIT_ERR_ALIGN, DIT_ERR_NULL, DIT_ERR_SHAPE,
                                           DIT_ERR_UNSUPPORTED, DIT_ERR_VALUE)

G = 1 << 40  # fake device addresses, 1 TiB apart: never overlap by accident
Q, K, V, O, L = 1 * G, 2 * G, 3 * G, 4 * G, 5 * G


def fwd(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Sq=256, Skv=256, d=64, scale=0.125,
        dtype=DIT_DTYPE_BF16):
    return _lib.dit_attn_fwd_status(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype, stream=0)


def test_library_exports_header_functions():
    names = _lib.header_functions()
    assert set(names) == {"dit_attn_fwd", "dit_attn_fwd_workspace_size", "dit_attn_fwd_ws",
                          "dit_attn_fwd_noalloc", "dit_attn_fwd_acc", "dit_attn_merge",
                          "dit_quant_fp8", "dit_status_string", "dit_version"}
    lib = _lib.load()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_side_libraries_export_the_same_interface():
    """The race-check build exports what the header declares, like the
    library; the probe library exports its two entries."""
    from attention_non_causal_amd import build as libbuild

    def exported(path):
        out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                             text=True, check=True).stdout
        return {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(_lib.header_functions()) <= exported(_lib.DEBUG_LIB_PATH)
    assert {"dit_probe_mfma_ceiling", "dit_probe_valu_issue"} <= exported(libbuild.PROBE_LIB_PATH)


def test_version_and_status_strings():
    assert _lib.dit_version() == 10301
    texts = [_lib.dit_status_string(s) for s in range(9)]
    assert len(set(texts)) == 9 and all(texts)
    assert _lib.dit_status_string(99) == "unknown status"
    assert _lib.dit_status_string(-1) == "unknown status"


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), DIT_ERR_NULL), (dict(k=None), DIT_ERR_NULL), (dict(v=None), DIT_ERR_NULL),
    (dict(o=None), DIT_ERR_NULL), (dict(lse=None), DIT_ERR_NULL),
    (dict(dtype=2), DIT_ERR_UNSUPPORTED), (dict(dtype=-1), DIT_ERR_UNSUPPORTED),
    (dict(d=96), DIT_ERR_UNSUPPORTED), (dict(d=256), DIT_ERR_UNSUPPORTED),
    (dict(d=0), DIT_ERR_UNSUPPORTED),
    (dict(B=0), DIT_ERR_SHAPE), (dict(H=0), DIT_ERR_SHAPE), (dict(Sq=0), DIT_ERR_SHAPE),
    (dict(Skv=0), DIT_ERR_SHAPE), (dict(Skv=-5), DIT_ERR_SHAPE),
    (dict(B=1 << 30, H=1 << 30, Sq=1 << 30), DIT_ERR_SHAPE),
    (dict(H=64, Skv=1 << 18, d=128), DIT_ERR_SHAPE),      # 4 GiB of K per batch
    (dict(B=4, H=64, Skv=(1 << 18) - 1, d=128, scale=0.0), DIT_ERR_VALUE),  # just below
    (dict(scale=0.0), DIT_ERR_VALUE), (dict(scale=-0.125), DIT_ERR_VALUE),
    (dict(scale=math.inf), DIT_ERR_VALUE), (dict(scale=math.nan), DIT_ERR_VALUE),
    (dict(q=Q + 8), DIT_ERR_ALIGN), (dict(k=K + 2), DIT_ERR_ALIGN), (dict(v=V + 4), DIT_ERR_ALIGN),
    (dict(o=O + 8), DIT_ERR_ALIGN), (dict(lse=L + 2), DIT_ERR_ALIGN),
    (dict(o=Q + 4096), DIT_ERR_ALIAS), (dict(o=V - 16), DIT_ERR_ALIAS),
    (dict(lse=K + 64), DIT_ERR_ALIAS), (dict(lse=O + 1024), DIT_ERR_ALIAS),
])
def test_fwd_rejects(kw, status):
    assert fwd(**kw) == status


def test_fwd_fp8_descriptor_checks():
    good = [_lib.fp8_tensor(Q, Q + (1 << 30)), _lib.fp8_tensor(K, K + (1 << 30)),
            _lib.fp8_tensor(V, V + (1 << 30))]
    bad_data = _lib.fp8_tensor(None, Q + (1 << 30))
    bad_scale = _lib.fp8_tensor(K, None)
    st = fwd(q=bad_data, k=good[1], v=good[2], dtype=DIT_DTYPE_FP8_E4M3)
    assert st == DIT_ERR_NULL
    st = fwd(q=good[0], k=bad_scale, v=good[2], dtype=DIT_DTYPE_FP8_E4M3)
    assert st == DIT_ERR_NULL
    mis = _lib.fp8_tensor(V, V + (1 << 30) + 2)
    st = fwd(q=good[0], k=good[1], v=mis, dtype=DIT_DTYPE_FP8_E4M3)
    assert st == DIT_ERR_ALIGN
    mis = _lib.fp8_tensor(Q + 8, Q + (1 << 30))
    st = fwd(q=mis, k=good[1], v=good[2], dtype=DIT_DTYPE_FP8_E4M3)
    assert st == DIT_ERR_ALIGN
    # output overlapping a scale array
    st = fwd(q=good[0], k=good[1], v=good[2], o=K + (1 << 30), dtype=DIT_DTYPE_FP8_E4M3)
    assert st == DIT_ERR_ALIAS


def merge(o_parts=None, lse_parts=None, n=2, o=O, lse=L, B=1, H=2, Sq=100, d=64):
    if o_parts is None:
        o_parts = [Q, K]
    if lse_parts is None:
        lse_parts = [V, V + (1 << 20)]
    return _lib.dit_attn_merge_status(o_parts, lse_parts, n, o, lse, B, H, Sq, d, stream=0)


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), DIT_ERR_NULL), (dict(lse=None), DIT_ERR_NULL),
    (dict(o_parts=[Q, None]), DIT_ERR_NULL), (dict(lse_parts=[None, V]), DIT_ERR_NULL),
    (dict(n=0), DIT_ERR_UNSUPPORTED), (dict(n=17, o_parts=[Q] * 17, lse_parts=[V] * 17),
                                       DIT_ERR_UNSUPPORTED),
    (dict(d=32), DIT_ERR_UNSUPPORTED),
    (dict(B=0), DIT_ERR_SHAPE), (dict(Sq=-1), DIT_ERR_SHAPE),
    (dict(B=2, Sq=1 << 15, H=1 << 15), DIT_ERR_SHAPE),  # 2^31 rows: one past the limit
    (dict(o=O + 4), DIT_ERR_ALIGN), (dict(lse=L + 1), DIT_ERR_ALIGN),
    (dict(o_parts=[Q, K + 8]), DIT_ERR_ALIGN),
    (dict(o=K + 256), DIT_ERR_ALIAS),           # partial overlap with part 1
    (dict(lse=V + 64), DIT_ERR_ALIAS),          # partial overlap with lse part 0
    (dict(o=V), DIT_ERR_ALIAS),                 # output O over an LSE input
    (dict(lse=L, o=L - 512), DIT_ERR_ALIAS),    # O and LSE overlap each other
])
def test_merge_rejects(kw, status):
    assert merge(**kw) == status


def test_merge_null_arrays():
    lib = _lib.load()
    assert lib.dit_attn_merge(None, None, 2, O, L, 1, 2, 100, 64, None) == DIT_ERR_NULL


@pytest.mark.parametrize("args,status", [
    ((None, O, L, 1, 2, 256, 64), DIT_ERR_NULL), ((Q, None, L, 1, 2, 256, 64), DIT_ERR_NULL),
    ((Q, O, None, 1, 2, 256, 64), DIT_ERR_NULL),
    ((Q, O, L, 1, 2, 256, 80), DIT_ERR_UNSUPPORTED),
    ((Q, O, L, 0, 2, 256, 64), DIT_ERR_SHAPE), ((Q, O, L, 1, 2, 0, 64), DIT_ERR_SHAPE),
    ((Q + 2, O, L, 1, 2, 256, 64), DIT_ERR_ALIGN), ((Q, O + 8, L, 1, 2, 256, 64), DIT_ERR_ALIGN),
    ((Q, O, L + 2, 1, 2, 256, 64), DIT_ERR_ALIGN),
    ((Q, Q + 1024, L, 1, 2, 256, 64), DIT_ERR_ALIAS), ((Q, O, O + 16, 1, 2, 256, 64),
                                                       DIT_ERR_ALIAS),
])
def test_quant_rejects(args, status):
    assert _lib.dit_quant_fp8_status(*args, stream=0) == status


def test_binding_raises_with_status():
    with pytest.raises(_lib.DitError) as e:
        _lib.dit_attn_fwd(None, K, V, O, L, 1, 2, 256, 256, 64, 0.125, DIT_DTYPE_BF16, stream=0)
    assert e.value.status == DIT_ERR_NULL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(_lib.LibraryNotBuilt):
        _lib.dit_version()


# ------------------------------------------------- workspace entry points

def fwd_ws(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Sq=256, Skv=256, d=64, scale=0.125,
           dtype=DIT_DTYPE_BF16, ws=None, ws_bytes=0):
    return _lib.dit_attn_fwd_ws_status(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype, ws,
                                       ws_bytes, stream=0)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), DIT_ERR_NULL), (dict(lse=None), DIT_ERR_NULL),
    (dict(dtype=2), DIT_ERR_UNSUPPORTED), (dict(d=96), DIT_ERR_UNSUPPORTED),
    (dict(B=0), DIT_ERR_SHAPE), (dict(H=64, Skv=1 << 18, d=128), DIT_ERR_SHAPE),
    (dict(scale=math.nan), DIT_ERR_VALUE), (dict(o=O + 8), DIT_ERR_ALIGN),
    (dict(o=Q), DIT_ERR_ALIAS),
])
def test_fwd_ws_rejects_like_fwd(kw, status):
    """The workspace entry point validates its tensor arguments exactly as
    dit_attn_fwd does, before any HIP call."""
    assert fwd_ws(**kw) == status
    assert fwd(**kw) == status


def fwd_acc(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Sq=256, Skv=256, d=64, scale=0.125,
            dtype=DIT_DTYPE_BF16, kv_batch_tokens=0, ws=None, ws_bytes=0):
    return _lib.dit_attn_fwd_acc_status(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype,
                                        kv_batch_tokens=kv_batch_tokens, workspace=ws,
                                        workspace_bytes=ws_bytes, stream=0)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), DIT_ERR_NULL), (dict(lse=None), DIT_ERR_NULL),
    (dict(dtype=2), DIT_ERR_UNSUPPORTED), (dict(d=96), DIT_ERR_UNSUPPORTED),
    (dict(B=0), DIT_ERR_SHAPE), (dict(H=64, Skv=1 << 18, d=128), DIT_ERR_SHAPE),
    (dict(scale=math.nan), DIT_ERR_VALUE), (dict(o=O + 8), DIT_ERR_ALIGN),
    (dict(o=Q), DIT_ERR_ALIAS), (dict(lse=V), DIT_ERR_ALIAS),
])
def test_fwd_acc_rejects_like_fwd(kw, status):
    """The accumulating entry point validates its arguments as dit_attn_fwd
    does, before any HIP call."""
    assert fwd_acc(**kw) == status


def test_fwd_acc_kv_batch_stride_checks():
    """kv_batch_tokens: 0 (contiguous) or at least Skv; the batches it spreads
    K and V over are part of their extent for the aliasing checks."""
    for kbt in (-1, 255, 1 << 31):
        assert fwd_acc(kv_batch_tokens=kbt) == DIT_ERR_SHAPE
    # B2 H2 d64: K spans (1000 + 256) tokens x 256 bytes; an output placed 600
    # tokens into it overlaps the second batch's keys (but not a contiguous K)
    o_in_k = K + 600 * 2 * 64 * 2
    assert fwd_acc(B=2, o=o_in_k, kv_batch_tokens=1000) == DIT_ERR_ALIAS
    assert fwd_acc(B=2, o=o_in_k) != DIT_ERR_ALIAS


def test_fwd_acc_fp8_checks():
    """fp8 key blocks are tensors of their own: a batch stride is refused
    before the descriptors are even read (fake addresses here); with
    descriptors the fp8 checks of dit_attn_fwd apply."""
    assert fwd_acc(dtype=DIT_DTYPE_FP8_E4M3, kv_batch_tokens=512) == DIT_ERR_UNSUPPORTED
    good = [_lib.fp8_tensor(Q, Q + (1 << 30)), _lib.fp8_tensor(K, K + (1 << 30)),
            _lib.fp8_tensor(V, V + (1 << 30))]
    assert fwd_acc(q=_lib.fp8_tensor(None, Q + (1 << 30)), k=good[1], v=good[2],
                   dtype=DIT_DTYPE_FP8_E4M3) == DIT_ERR_NULL
    assert fwd_acc(q=good[0], k=good[1], v=_lib.fp8_tensor(V, V + (1 << 30) + 2),
                   dtype=DIT_DTYPE_FP8_E4M3) == DIT_ERR_ALIGN
    assert fwd_acc(q=good[0], k=good[1], v=good[2], o=K + 4096,
                   dtype=DIT_DTYPE_FP8_E4M3) == DIT_ERR_ALIAS


def test_workspace_size_argument_checks():
    st, _ = _lib.dit_attn_fwd_workspace_size_status(1, 2, 256, 256, 64)
    assert st in (_lib.DIT_OK, _lib.DIT_ERR_HIP)  # DIT_ERR_HIP: no HIP device here
    lib = _lib.load()
    assert lib.dit_attn_fwd_workspace_size(1, 2, 256, 256, 64, DIT_DTYPE_BF16, None) == DIT_ERR_NULL
    for args, status in [((0, 2, 256, 256, 64, 0), DIT_ERR_SHAPE),
                         ((1, 2, 256, 256, 96, 0), DIT_ERR_UNSUPPORTED),
                         ((1, 2, 256, 256, 64, 5), DIT_ERR_UNSUPPORTED),
                         ((1, 64, 256, 1 << 18, 128, 0), DIT_ERR_SHAPE)]:
        assert _lib.dit_attn_fwd_workspace_size_status(*args)[0] == status
    # the fp8 path plans its split like the bf16 one (on the device's CU count)
    st, _ = _lib.dit_attn_fwd_workspace_size_status(1, 2, 256, 256, 64, DIT_DTYPE_FP8_E4M3)
    assert st in (_lib.DIT_OK, _lib.DIT_ERR_HIP)


def noalloc(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Sq=256, Skv=256, d=64, scale=0.125,
            dtype=DIT_DTYPE_BF16):
    return _lib.dit_attn_fwd_noalloc_status(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype,
                                            stream=0)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), DIT_ERR_NULL), (dict(lse=None), DIT_ERR_NULL),
    (dict(dtype=2), DIT_ERR_UNSUPPORTED), (dict(d=96), DIT_ERR_UNSUPPORTED),
    (dict(B=0), DIT_ERR_SHAPE), (dict(Skv=-1), DIT_ERR_SHAPE),
    (dict(scale=0.0), DIT_ERR_VALUE), (dict(scale=math.nan), DIT_ERR_VALUE),
    (dict(k=K + 2), DIT_ERR_ALIGN), (dict(o=Q + 4096), DIT_ERR_ALIAS),
])
def test_noalloc_rejects_before_any_hip_call(kw, status):
    """dit_attn_fwd_noalloc validates every argument before its first HIP call
    (the device query and the scratch lookup come after), so on a host without
    a GPU an invalid call returns its own status."""
    assert noalloc(**kw) == status


def test_noalloc_scratch_size_constant():
    """The Python constant mirrors DIT_NOALLOC_SCRATCH_BYTES, which covers the
    largest split any shape needs on a GPU of 256 compute units: 512 pieces of
    128 rows x (128 + 2) fp32 (fp8, d = 128)."""
    import re
    text = open(_lib.HEADER_PATH).read()
    m = re.search(r"#define DIT_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.DIT_NOALLOC_SCRATCH_BYTES
    assert _lib.DIT_NOALLOC_SCRATCH_BYTES >= 512 * 128 * 130 * 4
    assert _lib.DIT_NOALLOC_SCRATCH_BYTES >= 256 * 256 * 129 * 4
