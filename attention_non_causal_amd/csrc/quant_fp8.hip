// quant_fp8.hip -- per-(b, h, 128-token block) e4m3 quantisation of a bf16
// [B][S][H][d] tensor, for gfx950.
//
// Block-scaled low-precision tensors are a payload plus per-block scales
// ("生成AI推論を速くするための設計ノート" sec. 3); the FP8 attention backend
// of "AMD、Radeon AI PRO R9700S最大4台で..." consumes FP8 activations.  Here
// each (b, h, block of 128 tokens) gets one fp32 scale:
//     amax = max |x|, inv = fp32(448 / amax), x8 = e4m3_rne(fp32(x * inv)),
//     scale = fp32(amax / 448)          (amax == 0: scale = 1, x8 = 0).
// Every step is one correctly rounded fp32 operation (IEEE division, a single
// multiply, the hardware's round-to-nearest-even conversion to OCP e4m3), so
// the bytes are reproducible bit for bit.  |x * inv| <= 448 * (1 + 2^-23), which
// rounds to 448, so no value reaches the saturation range.
//
// Non-finite input: a NaN takes no part in amax and encodes as 0x7F (e4m3's
// NaN, sign cleared); an infinity makes amax, and so the block's scale,
// infinite, which turns every finite value of the block into a (signed) zero
// and the infinity itself (inf * 0) into 0x7F.  A block whose values are all
// zero or NaN has amax = 0: scale 1 and every byte 0.
//
// One workgroup per block: the block's 128 x d bf16 values are read once into
// registers (16-byte loads, consecutive threads on consecutive chunks), the
// magnitude maximum is reduced across the workgroup, and the same registers
// are converted and written.  HBM-bound: 2 bytes in, 1 byte out per element.
#include "common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

constexpr int kBlockTokens = 128;

// bf16 magnitude bits m (sign cleared) as they count towards amax: a NaN
// (above the infinity's 0x7f80) counts as zero.
__device__ __forceinline__ uint32_t amax_mag(uint32_t m)
{
    return m <= 0x7f80u ? m : 0u;
}

// Four e4m3 codes with the sign bit of every NaN code (S.1111.111) cleared,
// so that a NaN encodes as 0x7F whatever the conversion made of its sign (no
// finite code has all seven low bits set).
__device__ __forceinline__ uint32_t nan_codes_positive(uint32_t w)
{
    const uint32_t nan = ((w & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u;
    return w & ~nan;
}

template <int D>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ X,
                                                        uint8_t* __restrict__ X8,
                                                        float* __restrict__ scale, int H, int S,
                                                        int nblk)
{
    constexpr int kChunks = D / 8;                        // 16-byte chunks per token
    constexpr int kPer = kBlockTokens * kChunks / 256;    // chunks per thread
    __shared__ uint32_t red[4];

    const int tid = threadIdx.x;
    const int blk = blockIdx.x % nblk;
    const int bh = blockIdx.x / nblk;
    const int h = bh % H;
    const long b = bh / H;
    const int s0 = blk * kBlockTokens;
    const int ns = min(kBlockTokens, S - s0);
    const long tok = (long)H * D;
    const long base = ((b * S + s0) * H + h) * D;

    u32x4 v[kPer];
    uint32_t amax_bits = 0;  // max of |x| as bf16 magnitude bits (monotone in |x|), NaN left out
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int c = tid + 256 * i;
        const int r = c / kChunks;
        const int cc = c % kChunks;
        v[i] = u32x4{0, 0, 0, 0};
        if (r < ns)
            v[i] = ld_global16(X + base + r * tok + cc * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            amax_bits = max(amax_bits, amax_mag(v[i][e] & 0x7fffu));
            amax_bits = max(amax_bits, amax_mag((v[i][e] >> 16) & 0x7fffu));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, off, 64));
    if ((tid & 63) == 0)
        red[tid >> 6] = amax_bits;
    __syncthreads();
    amax_bits = max(max(red[0], red[1]), max(red[2], red[3]));

    const float amax = __builtin_bit_cast(float, amax_bits << 16);
    float inv = 0.f, sc = 1.f;
    if (amax_bits != 0) {
        inv = 448.0f / amax;
        sc = amax / 448.0f;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int c = tid + 256 * i;
        const int r = c / kChunks;
        const int cc = c % kChunks;
        if (r >= ns)
            continue;
        u32x2 w = {0, 0};
        if (amax_bits != 0) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const uint32_t x0 = v[i][2 * half], x1 = v[i][2 * half + 1];
                const float f0 = __builtin_bit_cast(float, x0 << 16) * inv;
                const float f1 = __builtin_bit_cast(float, x0 & 0xffff0000u) * inv;
                const float f2 = __builtin_bit_cast(float, x1 << 16) * inv;
                const float f3 = __builtin_bit_cast(float, x1 & 0xffff0000u) * inv;
                int packed = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
                packed = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, packed, true);
                w[half] = nan_codes_positive((uint32_t)packed);
            }
        }
        *reinterpret_cast<u32x2*>(X8 + base + r * tok + cc * 8) = w;
    }
    if (tid == 0)
        scale[(long)bh * nblk + blk] = sc;
}

template <int D>
hipError_t launch_quant_d(const void* x, void* x8, float* scale, int B, int H, int S,
                          hipStream_t stream)
{
    const int nblk = (S + kBlockTokens - 1) / kBlockTokens;
    const long blocks = (long)B * H * nblk;
    if (blocks > 0x7fffffffL)
        return hipErrorInvalidConfiguration;
    return launch_kernel(quant_fp8_kernel<D>, dim3((unsigned)blocks), dim3(256), stream, x, x8,
                         scale, H, S, nblk);
}

}  // namespace

hipError_t launch_quant_fp8(const void* x, void* x8, float* scale, int B, int H, int S, int d,
                            hipStream_t stream)
{
    return d == 64 ? launch_quant_d<64>(x, x8, scale, B, H, S, stream)
                   : launch_quant_d<128>(x, x8, scale, B, H, S, stream);
}

}  // namespace dit
