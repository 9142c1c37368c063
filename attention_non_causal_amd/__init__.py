"""MI355X-native non-causal attention (O + LSE), LSE-merge and e4m3 quantiser
for DiT inference, as hand-written HIP kernels for gfx950 behind a C ABI."""
