"""fp64 CPU oracle for non-causal attention, its log-sum-exp merge and the
per-(head, 128-token block) e4m3 quantiser.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library (``attention_non_causal_amd``) never imports it, and the two share no
code: the arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over
independent output rows), this module only marshals NumPy arrays.

What each function computes, and which page it follows, is stated in
``oracle.c``.  In short:

* ``attn_fwd``   -- softmax(scale * Q K^T) V per (batch, head), plus
  LSE = ln sum_j exp(scale * q . k_j); non-causal, no mask.  Reading of the
  non-causal DiT attention in "xDiT 项目概述" sec. 2.1 (whole-sequence,
  prefill-like, no KV cache).
* ``attn_merge`` -- combine partial (O, LSE) over disjoint key blocks: the
  step ring attention needs ("xDiT 项目概述" sec. 3.2, USP ring dimension).
* ``quant_fp8`` / ``dequant_fp8`` / ``e4m3_encode`` / ``e4m3_decode`` --
  block-scaled OCP e4m3, one fp32 scale per (b, h, 128 tokens); the block-scaled
  format idea of "生成AI推論を速くするための設計ノート" sec. 3, FP8 per
  "AMD、Radeon AI PRO R9700S最大4台で..." (tuning section).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

FP8_BLOCK = 128


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile ``oracle.c`` (or another source) with gcc into a shared library."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
               "-ffp-contract=off", "-fno-fast-math", "-I", _HERE, src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def load_library(path: str):
    """Load an oracle shared library at ``path`` and declare its signatures.
    (Tests also use this to load deliberately broken builds of oracle.c.)"""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = D
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = D
    lib.oracle_e4m3_encode.argtypes = [D]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = I
    lib.oracle_set_num_threads.argtypes = [I]
    lib.oracle_set_num_threads.restype = None
    for name in ("oracle_attn_fwd_f64", "oracle_attn_fwd_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [P, P, P, P, P, I, I, I, I, I, D, P, I]
        fn.restype = I
    lib.oracle_attn_merge.argtypes = [P, P, I, P, P, I, I, I, I]
    lib.oracle_attn_merge.restype = I
    lib.oracle_quant_fp8.argtypes = [P, P, P, I, I, I, I]
    lib.oracle_quant_fp8.restype = I
    lib.oracle_dequant_fp8.argtypes = [P, P, P, I, I, I, I]
    lib.oracle_dequant_fp8.restype = I
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = load_library(_LIB_PATH)
    return _lib


def use_library(lib) -> None:
    """Route the module-level functions through ``lib`` (None: the default)."""
    global _lib
    _lib = lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def attn_fwd(q, k, v, scale: float, rows=None):
    """Attention forward in fp64.

    q: [B,Sq,H,d], k/v: [B,Skv,H,d] -- either uint16 arrays holding bf16 bit
    patterns (decoded exactly) or float64 arrays.  ``scale`` is used as given
    (widened to fp64).  ``rows``: optional sorted-or-not list of query rows to
    compute (all heads, all batches); the outputs then hold only those rows in
    the order given.

    Returns (o [B,n_rows,H,d] float64, lse [B,H,n_rows] float64).
    """
    lib = _load()
    B, Sq, H, d = q.shape
    Skv = k.shape[1]
    assert k.shape == (B, Skv, H, d) and v.shape == (B, Skv, H, d)
    if q.dtype == np.uint16:
        assert k.dtype == np.uint16 and v.dtype == np.uint16
        fn = lib.oracle_attn_fwd_bf16
    else:
        q = np.ascontiguousarray(q, dtype=np.float64)
        k = np.ascontiguousarray(k, dtype=np.float64)
        v = np.ascontiguousarray(v, dtype=np.float64)
        fn = lib.oracle_attn_fwd_f64
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    if rows is None:
        nr = Sq
        rows_arr = None
        rows_ptr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        nr = int(rows_arr.size)
        rows_ptr = _ptr(rows_arr)
    o = np.empty((B, nr, H, d), dtype=np.float64)
    lse = np.empty((B, H, nr), dtype=np.float64)
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Sq, Skv, d,
            float(scale), rows_ptr, nr)
    if rc != 0:
        raise RuntimeError(f"oracle_attn_fwd failed: {rc}")
    return o, lse


def attn_merge(o_parts, lse_parts):
    """Merge n partial results.

    o_parts: [n,B,Sq,H,d] (float64, or uint16 bf16 bits decoded exactly);
    lse_parts: [n,B,H,Sq] (any float dtype, widened to fp64).
    Returns (o [B,Sq,H,d], lse [B,H,Sq]) in float64.
    """
    lib = _load()
    o_parts = np.asarray(o_parts)
    if o_parts.dtype == np.uint16:
        o_parts = bf16_bits_to_f64(o_parts)
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    n, B, Sq, H, d = o_parts.shape
    assert lse_parts.shape == (n, B, H, Sq)
    o = np.empty((B, Sq, H, d), dtype=np.float64)
    lse = np.empty((B, H, Sq), dtype=np.float64)
    rc = lib.oracle_attn_merge(_ptr(o_parts), _ptr(lse_parts), n, _ptr(o), _ptr(lse),
                               B, H, Sq, d)
    if rc != 0:
        raise RuntimeError(f"oracle_attn_merge failed: {rc}")
    return o, lse


def quant_fp8(x_bits: np.ndarray):
    """Quantise bf16 [B,S,H,d] (uint16 bits) to e4m3 bytes + fp32 scales
    [B,H,ceil(S/128)]."""
    lib = _load()
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    B, S, H, d = x_bits.shape
    nblk = (S + FP8_BLOCK - 1) // FP8_BLOCK
    q = np.empty((B, S, H, d), dtype=np.uint8)
    sc = np.empty((B, H, nblk), dtype=np.float32)
    rc = lib.oracle_quant_fp8(_ptr(x_bits), _ptr(q), _ptr(sc), B, H, S, d)
    if rc != 0:
        raise RuntimeError(f"oracle_quant_fp8 failed: {rc}")
    return q, sc


def dequant_fp8(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Inverse of quant_fp8 up to rounding: decode(q) * block scale, fp64."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    B, S, H, d = q.shape
    x = np.empty((B, S, H, d), dtype=np.float64)
    rc = lib.oracle_dequant_fp8(_ptr(q), _ptr(scale), _ptr(x), B, H, S, d)
    if rc != 0:
        raise RuntimeError(f"oracle_dequant_fp8 failed: {rc}")
    return x


def e4m3_decode(code: int) -> float:
    return _load().oracle_e4m3_decode(int(code))


def e4m3_encode(x: float) -> int:
    return int(_load().oracle_e4m3_encode(float(x)))


def e4m3_decode_table() -> np.ndarray:
    """Decoded value of every byte 0..255 (NaN for the two NaN codes)."""
    lib = _load()
    return np.array([lib.oracle_e4m3_decode(c) for c in range(256)], dtype=np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64 (shift into fp32)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
