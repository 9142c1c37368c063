// mfma_ceiling.hip -- measurement aid, not part of the attention library: the
// dense matrix-core throughput this chip sustains on given operand data, at
// the clock its power limit allows.  The peak figures (2.5 PFLOP/s bf16,
// 5.0 fp8) assume 2.4 GHz; under a dense MFMA load the part lowers its clock,
// by how much depending on the data the matrix cores switch.  The attention
// kernels' fractions of peak are read against this.
//
// Two waves per SIMD (workgroups of 4 waves, two per CU), each running a loop
// of 16 MFMAs per turn on four accumulators with operands that change every
// instruction (four A and four B fragments per lane, taken from a caller
// buffer, used in rotation).  The 32x32 cases and the first 16x16x32 case
// rotate over the accumulators (no instruction depends on the one before);
// the second 16x16x32 case runs four dependent instructions on each
// accumulator in a row, the pattern the d = 128 bf16 forward kernel is built
// on.
// Built into libditprobe.so by build(); `bench.py --mfma-ceiling` times it.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// kind 0: v_mfma_f32_32x32x16_bf16 (A, B: 8 bf16 per lane);
// kind 1: v_mfma_scale_f32_32x32x64_f8f6f4 with e4m3 operands (32 bytes per lane);
// kind 2: v_mfma_f32_16x16x32_bf16 (A, B: 8 bf16 per lane), accumulators in rotation;
// kind 3: the same, four dependent instructions per accumulator in a row.
template <int KIND>
__global__ __launch_bounds__(256, 2) void mfma_ceiling_kernel(const uint32_t* __restrict__ src,
                                                              float* __restrict__ out, int iters)
{
    const int lane = threadIdx.x & 63;
    // operand fragments: 8 words per fragment and lane (bf16 uses the first 4)
    i32x8 a[4], b[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const uint32_t* pa = src + ((f * 64 + lane) * 8);
        const uint32_t* pb = src + (((4 + f) * 64 + lane) * 8);
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            a[f][w] = (int)pa[w];
            b[f][w] = (int)pb[w];
        }
    }
    f32x16 acc[4] = {};
    f32x4 acc4[4] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const i32x8& x = a[(i + r) & 3];
                const i32x8& y = b[(i + 2 * r + 1) & 3];
                if constexpr (KIND == 2 || KIND == 3) {
                    const u32x4 xa = {(uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]};
                    const u32x4 ya = {(uint32_t)y[0], (uint32_t)y[1], (uint32_t)y[2], (uint32_t)y[3]};
                    // kind 3: accumulator r for the four instructions of turn r
                    f32x4& c = acc4[KIND == 2 ? i : r];
                    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa),
                                                                __builtin_bit_cast(bf16x8, ya), c, 0,
                                                                0, 0);
                    if constexpr (KIND == 3)
                        if (i == 3)
                            __builtin_amdgcn_sched_barrier(0);  // keep each chain together
                } else if constexpr (KIND == 0) {
                    const u32x4 xa = {(uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]};
                    const u32x4 ya = {(uint32_t)y[0], (uint32_t)y[1], (uint32_t)y[2], (uint32_t)y[3]};
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, xa), __builtin_bit_cast(bf16x8, ya), acc[i], 0, 0, 0);
                } else {
                    acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, acc[i], 0, 0, 0, 127, 0,
                                                                              127);
                }
            }
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            s += acc[i][e];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            s += acc4[i][e];
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// Run the probe once on `stream`: n_blocks workgroups of 256 threads, each
// wave doing 16 * iters matrix instructions.  src: 4096 device words of
// operand data (fragments 0-3 are the A operands, 4-7 the B operands, 8 words
// per lane); out: n_blocks * 256 floats.  kind 0: bf16 32x32x16, 1: e4m3
// 32x32x64, 2: bf16 16x16x32 in rotation, 3: bf16 16x16x32 in chains of four.
// Returns the HIP status of the launch.
extern "C" int dit_probe_mfma_ceiling(const void* src, void* out, int n_blocks, int iters, int kind,
                                      void* stream)
{
    if (!src || !out || n_blocks < 1 || iters < 1 || kind < 0 || kind > 3)
        return (int)hipErrorInvalidValue;
    auto* s = static_cast<hipStream_t>(stream);
    const auto* p = static_cast<const uint32_t*>(src);
    auto* o = static_cast<float*>(out);
    if (kind == 0)
        hipLaunchKernelGGL(mfma_ceiling_kernel<0>, dim3(n_blocks), dim3(256), 0, s, p, o, iters);
    else if (kind == 1)
        hipLaunchKernelGGL(mfma_ceiling_kernel<1>, dim3(n_blocks), dim3(256), 0, s, p, o, iters);
    else if (kind == 2)
        hipLaunchKernelGGL(mfma_ceiling_kernel<2>, dim3(n_blocks), dim3(256), 0, s, p, o, iters);
    else
        hipLaunchKernelGGL(mfma_ceiling_kernel<3>, dim3(n_blocks), dim3(256), 0, s, p, o, iters);
    return (int)hipGetLastError();
}
