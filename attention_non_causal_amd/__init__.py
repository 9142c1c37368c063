"""MI355X-native non-causal attention (O + LSE), LSE-merge and e4m3 quantiser
for DiT inference, as hand-written HIP kernels for gfx950 behind a C ABI
(``include/dit_attn.h``).

``_lib``        ctypes binding with the C names (dit_attn_fwd, dit_attn_merge,
                dit_quant_fp8, dit_status_string, dit_version)
``functional``  torch helpers that allocate outputs and call the binding
``workloads``   seeded synthetic inputs (imports neither the binding nor torch)
``build``       hipcc build of libditattn.so

The shared library is loaded on first use; if it has not been built the call
raises ``LibraryNotBuilt`` (there is no fallback path).
"""
from ._lib import (DIT_DTYPE_BF16, DIT_DTYPE_FP8_E4M3, DitError, LibraryNotBuilt,  # noqa: F401
                   dit_attn_fwd, dit_attn_merge, dit_quant_fp8, dit_status_string, dit_version,
                   fp8_tensor)
