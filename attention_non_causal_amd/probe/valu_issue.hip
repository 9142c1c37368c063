// valu_issue.hip -- measurement aid, not part of the attention library: how
// many cycles a SIMD spends per wave64 vector instruction of the kinds the
// softmax of the attention kernels issues (exponential, FMA, addition, the
// bf16 and e4m3 packs), with one wave per SIMD and with two.  The forward
// kernels spend about as many vector instructions per score as this chip's
// vector issue can sustain beside the matrix work, so these rates bound them.
//
// Each wave runs `iters` turns of 16 instructions of one kind on 16
// independent registers (no instruction waits for the one before it) and
// times the loop with s_memtime (shader-clock cycles); the caller gets one
// cycle count per wave.  Inputs are finite values; the results are kept live
// and never read.  Built into libditprobe.so by build_probe();
// `bench.py --valu-issue` runs it.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kChains = 16;

// kind 0: v_exp_f32; 1: v_fma_f32; 2: v_add_f32; 3: v_cvt_pk_bf16_f32;
// 4: v_cvt_pk_fp8_f32; 5: v_exp_f32 and v_fma_f32 alternating.
template <int KIND>
__device__ __forceinline__ void one(uint32_t& r, uint32_t c, uint32_t d, int i)
{
    if constexpr (KIND == 5) {
        // (i is a constant once the caller's loop is unrolled)
        if ((i & 1) == 0)
            asm volatile("v_exp_f32 %0, %1" : "=v"(r) : "v"(c));
        else
            asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(r) : "v"(c), "v"(d));
    } else if constexpr (KIND == 0)
        asm volatile("v_exp_f32 %0, %1" : "=v"(r) : "v"(c));
    else if constexpr (KIND == 1)
        asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(r) : "v"(c), "v"(d));
    else if constexpr (KIND == 2)
        asm volatile("v_add_f32 %0, %1, %0" : "+v"(r) : "v"(c));
    else if constexpr (KIND == 3)
        asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(c), "v"(d));
    else
        asm volatile("v_cvt_pk_fp8_f32 %0, %1, %2" : "=v"(r) : "v"(c), "v"(d));
}

template <int KIND>
__global__ void valu_issue_kernel(uint64_t* __restrict__ out, int iters)
{
    uint32_t r[kChains], c[kChains];
#pragma unroll
    for (int i = 0; i < kChains; ++i) {
        r[i] = 0x3f800000u;                          // 1.0f
        c[i] = 0x3e000000u + ((threadIdx.x + i) << 10);  // ~0.125 .. 0.14f
    }
    const uint32_t d = 0x3f000000u;                  // 0.5f
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kChains; ++i)
            one<KIND>(r[i], c[i], d, i);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < kChains; ++i)
        x ^= r[i];
    asm volatile("" ::"v"(x));
    if ((threadIdx.x & 63) == 0)
        out[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = t1 - t0;
}

}  // namespace

// Run the probe once on `stream`: n_blocks workgroups of 64 * waves threads
// (waves = 4: one wave per SIMD, 8: two), each wave `iters` turns of 16
// instructions of `kind` (0 exp, 1 fma, 2 add, 3 bf16 pack, 4 e4m3 pack, 5
// exp and fma alternating).  out: n_blocks * waves device uint64 cycle counts.
// Returns the HIP status of the launch.
extern "C" int dit_probe_valu_issue(void* out, int n_blocks, int waves, int iters, int kind,
                                    void* stream)
{
    if (!out || n_blocks < 1 || (waves != 4 && waves != 8) || iters < 1 || kind < 0 || kind > 5)
        return (int)hipErrorInvalidValue;
    auto* s = static_cast<hipStream_t>(stream);
    auto* o = static_cast<uint64_t*>(out);
    const dim3 grid(n_blocks), block(64 * waves);
    switch (kind) {
    case 0: hipLaunchKernelGGL(valu_issue_kernel<0>, grid, block, 0, s, o, iters); break;
    case 1: hipLaunchKernelGGL(valu_issue_kernel<1>, grid, block, 0, s, o, iters); break;
    case 2: hipLaunchKernelGGL(valu_issue_kernel<2>, grid, block, 0, s, o, iters); break;
    case 3: hipLaunchKernelGGL(valu_issue_kernel<3>, grid, block, 0, s, o, iters); break;
    case 4: hipLaunchKernelGGL(valu_issue_kernel<4>, grid, block, 0, s, o, iters); break;
    default: hipLaunchKernelGGL(valu_issue_kernel<5>, grid, block, 0, s, o, iters); break;
    }
    return (int)hipGetLastError();
}
