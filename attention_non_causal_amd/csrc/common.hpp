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

// The value held by lane l ^ 32.  v_permlane32_swap(a, b) swaps the upper 32
// lanes of a with the lower 32 lanes of b; with a = b = x the first result is
// x[l % 32] and the second x[32 + l % 32] in every lane, so the partner's value
// is the second result in the lower half and the first in the upper half.
// (The selection by half is written out explicitly: combining the two results
// directly, e.g. fmaxf(r0, r1), is mis-simplified to r0 by the compiler.)
__device__ __forceinline__ float partner32(float x, bool upper_half)
{
    const int xi = __builtin_bit_cast(int, x);
    const auto p = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
    return __builtin_bit_cast(float, upper_half ? p[0] : p[1]);
}

// LDS byte address of a pointer into a __shared__ object (a constant for the
// object itself).
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane s supplies the
// address of 4 consecutive 16-bit elements; lane i of the group receives, in
// slot j, element (i % 4) of the 4 read by lane 4j + i/4.  With lane s pointing
// at row s/4, columns 4(s%4)..+3 of a row-major tile, lane i gets column i of
// rows 0..3: a 4 x 16 block arrives transposed.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 ld_lds_tr16(const void* p)
{
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// ds_read_b64_tr_b8: the byte analogue -- within each group of 16 lanes, lane
// s supplies the address of 8 consecutive bytes; lane i receives, in byte j,
// byte (i % 8) of the 8 read by lane 2j + i/8.  With lane s pointing at row
// s/2, bytes 8(s%2)..+7 of a row-major tile, lane i gets column i of rows
// 0..7: an 8 x 16 block arrives transposed.
__device__ __forceinline__ u32x2 ld_lds_tr8(const void* p)
{
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) i32x2*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// Buffer resource over [base, base + bytes) for raw (unstrided) buffer loads;
// an access past `bytes` reads zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Copy 16 bytes per lane from buffer offset voff + soff (soff wave-uniform) into
// LDS at lds + 16 * lane (lds wave-uniform): buffer_load_dwordx4 ... lds.
// (Non-template wrappers keep the host compilation away from the builtins.)
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff,
                                              uint32_t soff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                             voff, soff, 0, 0);
}

// Wait until every outstanding vector-memory operation of this wave (including
// global -> LDS copies) has completed.
__device__ __forceinline__ void wait_vmem_all()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Race check.  Built with -DDIT_DEBUG_BARRIERS, the forward kernels end every
// step of their key loop with this: every outstanding memory operation of the
// wave waited for, then a workgroup barrier.  The waves of a workgroup then
// run in lock step and every copy into LDS has landed before anyone goes on,
// so a race between waves (an LDS slot read before its copy landed, or
// overwritten while still read) cannot happen in that build.  The arithmetic
// is the same in both builds, so any difference between their results points
// at such a race (tests/test_gpu_debug_barriers.py compares them bit for bit).
// In the normal build it is empty.
__device__ __forceinline__ void debug_sync()
{
#ifdef DIT_DEBUG_BARRIERS
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
    __syncthreads();
#endif
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// The two bf16 values of a packed pair (low half first), widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w)
{
    return __builtin_bit_cast(float, w << 16);
}

__device__ __forceinline__ float bf16_hi(uint32_t w)
{
    return __builtin_bit_cast(float, w & 0xffff0000u);
}

// Log-sum-exp merge of one row's new result (LSE lse_new, O_new = c_new * acc)
// into a running one (LSE lse_old, O_old): on return O = c_new * acc +
// c_old * O_old and LSE = lse_out, where w = exp(LSE - max) weights each side
// ("xDiT 项目概述" sec. 3.2: the ring combines the partial results of the key
// blocks).  A running LSE of -inf (no keys yet) leaves c_new, c_old = 0 and
// lse_out as they are, so O_old is then never read.
__device__ __forceinline__ void merge_weights(float lse_old, float lse_new, float& c_new,
                                              float& c_old, float& lse_out)
{
    if (!(lse_old > -INFINITY))
        return;
    const float mx = fmaxf(lse_old, lse_new);
    const float w_old = exp2_fast((lse_old - mx) * kLog2e);
    const float w_new = exp2_fast((lse_new - mx) * kLog2e);
    const float inv = 1.f / (w_old + w_new);  // one of the two weights is 1
    c_new *= w_new * inv;
    c_old = w_old * inv;
    lse_out = mx + log2_fast(w_old + w_new) * kLn2;
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
