// common.hpp -- device-side helpers shared by the gfx950 kernels of this
// library: vector types, MFMA wrappers, global/LDS access and the
// XCD-aware workgroup remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

namespace dit {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// MI355X has 8 XCDs (each with its own L2); consecutive workgroup ids are
// dispatched round-robin over them.  Remap the hardware id so that each XCD
// receives one contiguous range of logical work items: neighbouring query
// tiles of one head then run on the same XCD and share its L2.  Bijective on
// [0, n) for any n.
__device__ __forceinline__ int xcd_remap(int bid, int n)
{
    constexpr int kXcds = 8;
    const int per = n / kXcds;
    const int rem = n % kXcds;
    const int x = bid % kXcds;
    const int local = bid / kXcds;
    return x * per + (x < rem ? x : rem) + local;
}

__device__ __forceinline__ u32x4 ld_global16(const void* p)
{
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void st_global16(void* p, u32x4 v)
{
    *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ u32x4 ld_lds16(const void* p)
{
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x2 ld_lds8(const void* p)
{
    return *reinterpret_cast<const u32x2*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v)
{
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 cat_bf16x8(u32x2 lo, u32x2 hi)
{
    u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8, v);
}

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16).
// Operand layout per lane l: A row (l % 32), B column (l % 32); both hold the
// 8 consecutive k indices 8*(l/32) .. 8*(l/32)+7.
// Result layout: lane l holds column (l % 32); register r holds row
// 8*(r/4) + 4*(l/32) + (r%4).
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_exp_f32 / v_log_f32: base-2 exponential and logarithm.
__device__ __forceinline__ float exp2_fast(float x)
{
    return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float log2_fast(float x)
{
    return __builtin_amdgcn_logf(x);
}

// Swap with the lane 32 positions away (lane l <-> l ^ 32).
__device__ __forceinline__ float xor32(float x)
{
    return __shfl_xor(x, 32, 64);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// Launch through hipLaunchKernel so the launch's own status is returned
// (hipGetLastError would also report errors left by unrelated earlier calls).
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                         Args... args)
{
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<KArgs...> held(static_cast<KArgs>(args)...);
    void* ptrs[sizeof...(KArgs)];
    std::apply([&ptrs](auto&... e) {
        int i = 0;
        ((ptrs[i++] = static_cast<void*>(&e)), ...);
    }, held);
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream);
}

}  // namespace dit
