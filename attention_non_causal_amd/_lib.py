"""ctypes binding of libditattn.so -- argument marshalling only.

The functions keep the C names and argument order of ``include/dit_attn.h``;
tensors may be given as torch tensors (their ``data_ptr()`` is passed) or as
raw integer device addresses.  Every step of the computation runs in the HIP
kernels of the library; there is no other code path.  If the library has not
been built, the first call raises ``LibraryNotBuilt`` -- nothing falls back.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libditattn.so")
DEBUG_LIB_PATH = os.path.join(_PKG, "libditattn_debugsync.so")  # race-check build (tests only)
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "dit_attn.h")

DIT_OK = 0
DIT_ERR_NULL = 1
DIT_ERR_SHAPE = 2
DIT_ERR_UNSUPPORTED = 3
DIT_ERR_ALIGN = 4
DIT_ERR_VALUE = 5
DIT_ERR_ALIAS = 6
DIT_ERR_HIP = 7
DIT_ERR_WORKSPACE = 8

DIT_DTYPE_BF16 = 0
DIT_DTYPE_FP8_E4M3 = 1
DIT_FP8_BLOCK = 128
MAX_MERGE_PARTS = 16
DIT_NOALLOC_SCRATCH_BYTES = 33 << 20


class LibraryNotBuilt(RuntimeError):
    pass


class DitError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class dit_fp8_tensor_t(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


_lib = None


def load():
    """Load libditattn.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _open(LIB_PATH)
    return _lib


@contextlib.contextmanager
def use_library(path):
    """Route every call of this module to another build of the library (the
    race-check variant libditattn_debugsync.so, for the tests) inside the
    block, then back."""
    global _lib
    saved = load()
    _lib = _open(path)
    try:
        yield _lib
    finally:
        _lib = saved


def _open(path):
    if not os.path.exists(path):
        raise LibraryNotBuilt(
            f"{path} is missing: build it with `python -m attention_non_causal_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(path)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.dit_attn_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.dit_attn_fwd.restype = I
    lib.dit_attn_fwd_workspace_size.argtypes = [I, I, I, I, I, I, ctypes.POINTER(ctypes.c_size_t)]
    lib.dit_attn_fwd_workspace_size.restype = I
    lib.dit_attn_fwd_ws.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P, ctypes.c_size_t, P]
    lib.dit_attn_fwd_ws.restype = I
    lib.dit_attn_fwd_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.dit_attn_fwd_noalloc.restype = I
    lib.dit_attn_fwd_acc.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, ctypes.c_longlong, P,
                                     ctypes.c_size_t, P]
    lib.dit_attn_fwd_acc.restype = I
    lib.dit_attn_merge.argtypes = [P, P, I, P, P, I, I, I, I, P]
    lib.dit_attn_merge.restype = I
    lib.dit_quant_fp8.argtypes = [P, P, P, I, I, I, I, P]
    lib.dit_quant_fp8.restype = I
    lib.dit_status_string.argtypes = [I]
    lib.dit_status_string.restype = ctypes.c_char_p
    lib.dit_version.argtypes = []
    lib.dit_version.restype = I
    return lib


def header_functions() -> list[str]:
    """Names of the functions the public header declares."""
    text = open(HEADER_PATH).read()
    return re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(dit_\w+)\s*\(", text, flags=re.M)


def _addr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError(f"cannot take a device address of {type(x).__name__}")


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def _check(status: int) -> None:
    if status != DIT_OK:
        raise DitError(status, dit_status_string(status))


def dit_status_string(status: int) -> str:
    return load().dit_status_string(int(status)).decode()


def dit_version() -> int:
    return load().dit_version()


def fp8_tensor(data, scale) -> dit_fp8_tensor_t:
    """Host descriptor of an e4m3 tensor and its block scales (device addresses)."""
    return dit_fp8_tensor_t(_addr(data), _addr(scale))


def _fwd_operand(x, dtype: int):
    if dtype == DIT_DTYPE_FP8_E4M3 and isinstance(x, dit_fp8_tensor_t):
        return ctypes.cast(ctypes.pointer(x), ctypes.c_void_p)
    return _addr(x)


def dit_attn_fwd_status(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype=DIT_DTYPE_BF16,
                        stream=None) -> int:
    """Call dit_attn_fwd and return its status code (no exception)."""
    args = [_fwd_operand(t, dtype) for t in (q, k, v)]
    return load().dit_attn_fwd(args[0], args[1], args[2], _addr(o), _addr(lse), int(B), int(H),
                               int(Sq), int(Skv), int(d), float(scale), int(dtype),
                               _stream(stream))


def dit_attn_fwd(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype=DIT_DTYPE_BF16,
                 stream=None) -> None:
    """Enqueue the attention forward pass; raises DitError on a bad argument.

    bf16: q, k, v are bf16 device tensors [B,S,H,d].  fp8: q, k, v are
    ``fp8_tensor(data, scale)`` descriptors.  o: bf16 [B,Sq,H,d]; lse: fp32
    [B,H,Sq].  stream: None = torch's current stream, 0 = the null stream."""
    _check(dit_attn_fwd_status(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype, stream))


def dit_attn_fwd_workspace_size_status(B, H, Sq, Skv, d, dtype=DIT_DTYPE_BF16):
    """Call dit_attn_fwd_workspace_size: returns (status, bytes)."""
    n = ctypes.c_size_t(0)
    st = load().dit_attn_fwd_workspace_size(int(B), int(H), int(Sq), int(Skv), int(d),
                                            int(dtype), ctypes.byref(n))
    return st, n.value


def dit_attn_fwd_workspace_size(B, H, Sq, Skv, d, dtype=DIT_DTYPE_BF16) -> int:
    """Bytes of workspace dit_attn_fwd_ws needs for this shape on the current device."""
    st, n = dit_attn_fwd_workspace_size_status(B, H, Sq, Skv, d, dtype)
    _check(st)
    return n


def dit_attn_fwd_ws_status(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype=DIT_DTYPE_BF16,
                           workspace=None, workspace_bytes=0, stream=None) -> int:
    """Call dit_attn_fwd_ws and return its status code (no exception)."""
    args = [_fwd_operand(t, dtype) for t in (q, k, v)]
    return load().dit_attn_fwd_ws(args[0], args[1], args[2], _addr(o), _addr(lse), int(B),
                                  int(H), int(Sq), int(Skv), int(d), float(scale), int(dtype),
                                  _addr(workspace), int(workspace_bytes), _stream(stream))


def dit_attn_fwd_ws(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype=DIT_DTYPE_BF16,
                    workspace=None, workspace_bytes=0, stream=None) -> None:
    """dit_attn_fwd with caller-provided scratch (see the header): the last wave
    of workgroups is split over the keys and merged."""
    _check(dit_attn_fwd_ws_status(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype, workspace,
                                  workspace_bytes, stream))


def dit_attn_fwd_noalloc_status(q, k, v, o, lse, B, H, Sq, Skv, d, scale,
                               dtype=DIT_DTYPE_BF16, stream=None) -> int:
    """Call dit_attn_fwd_noalloc and return its status code (no exception)."""
    args = [_fwd_operand(t, dtype) for t in (q, k, v)]
    return load().dit_attn_fwd_noalloc(args[0], args[1], args[2], _addr(o), _addr(lse), int(B),
                                       int(H), int(Sq), int(Skv), int(d), float(scale),
                                       int(dtype), _stream(stream))


def dit_attn_fwd_noalloc(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype=DIT_DTYPE_BF16,
                         stream=None) -> None:
    """dit_attn_fwd_ws with the library's static per-GPU scratch instead of a
    workspace: allocates nothing (calls overlapping on one GPU race)."""
    _check(dit_attn_fwd_noalloc_status(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype,
                                       stream))


def dit_attn_fwd_acc_status(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype=DIT_DTYPE_BF16,
                            kv_batch_tokens=0, workspace=None, workspace_bytes=0,
                            stream=None) -> int:
    """Call dit_attn_fwd_acc and return its status code (no exception)."""
    args = [_fwd_operand(t, dtype) for t in (q, k, v)]
    return load().dit_attn_fwd_acc(args[0], args[1], args[2], _addr(o), _addr(lse), int(B),
                                   int(H), int(Sq), int(Skv), int(d), float(scale), int(dtype),
                                   int(kv_batch_tokens), _addr(workspace), int(workspace_bytes),
                                   _stream(stream))


def dit_attn_fwd_acc(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype=DIT_DTYPE_BF16,
                     kv_batch_tokens=0, workspace=None, workspace_bytes=0, stream=None) -> None:
    """The forward pass over one key block merged into the running (o, lse)
    (see the header).  fp8: q, k, v are fp8_tensor descriptors and
    kv_batch_tokens must be 0."""
    _check(dit_attn_fwd_acc_status(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype,
                                   kv_batch_tokens, workspace, workspace_bytes, stream))


def dit_attn_merge_status(o_parts, lse_parts, n_parts, o, lse, B, H, Sq, d, stream=None) -> int:
    n = int(n_parts)
    m = max(n, 1)
    po = (ctypes.c_void_p * m)(*[_addr(t) for t in o_parts][:m]) if o_parts is not None else None
    pl = (ctypes.c_void_p * m)(*[_addr(t) for t in lse_parts][:m]) if lse_parts is not None \
        else None
    return load().dit_attn_merge(po, pl, n, _addr(o), _addr(lse), int(B), int(H), int(Sq),
                                 int(d), _stream(stream))


def dit_attn_merge(o_parts, lse_parts, n_parts, o, lse, B, H, Sq, d, stream=None) -> None:
    """Enqueue the LSE-merge of n_parts partial results (lists of device
    tensors/addresses) into o / lse."""
    _check(dit_attn_merge_status(o_parts, lse_parts, n_parts, o, lse, B, H, Sq, d, stream))


def dit_quant_fp8_status(x, x_fp8, scale, B, H, S, d, stream=None) -> int:
    return load().dit_quant_fp8(_addr(x), _addr(x_fp8), _addr(scale), int(B), int(H), int(S),
                                int(d), _stream(stream))


def dit_quant_fp8(x, x_fp8, scale, B, H, S, d, stream=None) -> None:
    """Enqueue the per-(b, h, 128-token) e4m3 quantisation of x into x_fp8 / scale."""
    _check(dit_quant_fp8_status(x, x_fp8, scale, B, H, S, d, stream))
