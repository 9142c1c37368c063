// fwd_bf16.hip -- non-causal attention forward pass (O + LSE) in bf16 with
// fp32 accumulation, for gfx950 (CDNA4) MFMA.
//
// What is computed: per (batch, head), O = softmax(scale * Q K^T) V and
// LSE = ln sum_j exp(scale * q . k_j) -- the whole-sequence, cache-free
// attention of DiT inference ("xDiT 项目概述", sec. 2.1), done by a dedicated
// kernel as "生成AI推論を速くするための設計ノート" sec. 5 recommends for an
// attention that dominates.  The kernel reaches the exact result (up to fp32
// rounding order) by a single pass over key tiles with a running maximum and
// running sum (online softmax).
//
// Work decomposition
//   Workgroup = 4 wavefronts = 128 query rows of one (batch, head); each wave
//   owns 32 rows.  Keys stream through LDS in tiles of 64.
//   Per tile and wave:
//     S^T (keys x queries) = K Q^T on v_mfma_f32_32x32x16_bf16: A = K from LDS,
//       B = Q^T held in registers for the whole kernel.  Computing the
//       transpose puts one query per lane column, so a row maximum and row sum
//       are per-lane reductions plus one exchange with lane l^32.
//     Online softmax in the log2 domain: scale*log2(e) is folded into one FMA
//       before v_exp_f32.
//     O^T (channels x queries) += V^T P^T: A = V^T from LDS (stored
//       transposed), B = P^T straight from the S^T accumulator registers -- the
//       k index of each 16-key step is the same permutation of keys for A and B,
//       so no register shuffle is needed.  The per-row rescale factor is a
//       per-lane scalar.
//   Tails: keys >= Skv are loaded as zeros and their scores set to -inf; query
//   rows >= Sq are computed on zero queries and never stored.
#include "common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

template <int D>
struct FwdBf16Cfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBr = 32 * kWaves;   // query rows per workgroup
    static constexpr int kBc = 64;            // keys per tile
    static constexpr int kKStride = D + 8;    // LDS row stride (elements), K tile [kBc][D]
    static constexpr int kVStride = kBc + 4;  // LDS row stride (elements), V^T tile [D][kBc]
    static constexpr int kChunks = D / 8;     // 16-byte chunks per token row
};

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int H, int Sq, int Skv, float scale_log2, int n_qtiles, int n_blocks)
{
    using Cfg = FwdBf16Cfg<D>;
    constexpr int kBc = Cfg::kBc;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kBc * Cfg::kKStride];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * Cfg::kVStride];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 31;   // query column of this lane within the wave
    const int hh = lane >> 5;  // which 8-wide k group this lane feeds

    const int logical = xcd_remap(blockIdx.x, n_blocks);
    const int qt = logical % n_qtiles;
    const int bh = logical / n_qtiles;
    const int h = bh % H;
    const int b = bh / H;

    const long tok = (long)H * D;  // elements between consecutive tokens
    const uint16_t* Qbh = Q + ((long)b * Sq * H + h) * D;
    const uint16_t* Kbh = K + ((long)b * Skv * H + h) * D;
    const uint16_t* Vbh = V + ((long)b * Skv * H + h) * D;

    const int q_row = qt * Cfg::kBr + wave * 32 + n;
    bf16x8 qf[D / 16];
    if (q_row < Sq) {
        const uint16_t* src = Qbh + (long)q_row * tok + 8 * hh;
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            qf[s] = as_bf16x8(ld_global16(src + 16 * s));
    } else {
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            qf[s] = as_bf16x8(u32x4{0, 0, 0, 0});
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
        oacc[mb] = f32x16{};
    float m_run = -INFINITY;  // running max of scale*log2(e)*s
    float l_run = 0.f;        // running sum over this lane's half of the keys

    const int n_kt = (Skv + kBc - 1) / kBc;
    for (int kt = 0; kt < n_kt; ++kt) {
        const int key0 = kt * kBc;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kBc * Cfg::kChunks / Cfg::kThreads; ++i) {
            const int c = tid + i * Cfg::kThreads;
            const int r = c / Cfg::kChunks;
            const int c8 = c % Cfg::kChunks;
            const int key = key0 + r;
            u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
            if (key < Skv) {
                kv = ld_global16(Kbh + (long)key * tok + c8 * 8);
                vv = ld_global16(Vbh + (long)key * tok + c8 * 8);
            }
            *reinterpret_cast<u32x4*>(Ks + r * Cfg::kKStride + c8 * 8) = kv;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                Vt[(c8 * 8 + e) * Cfg::kVStride + r] = (uint16_t)(vv[e / 2] >> (16 * (e % 2)));
        }
        __syncthreads();

        // S^T = K Q^T for two 32-key blocks.
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sacc[kb] = f32x16{};
            const uint16_t* krow = Ks + (32 * kb + n) * Cfg::kKStride + 8 * hh;
#pragma unroll
            for (int s = 0; s < D / 16; ++s)
                sacc[kb] = mfma32x32x16(as_bf16x8(ld_lds16(krow + 16 * s)), qf[s], sacc[kb]);
        }
        if (key0 + kBc > Skv) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key0 + 32 * kb + 8 * (r / 4) + 4 * hh + (r % 4);
                    if (key >= Skv)
                        sacc[kb][r] = -INFINITY;
                }
        }

        float mx = sacc[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mx = fmaxf(mx, sacc[kb][r]);
        mx = fmaxf(mx, xor32(mx));
        const float m_new = fmaxf(m_run, mx * scale_log2);
        const float alpha = exp2_fast(m_run - m_new);
        m_run = m_new;

        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = exp2_fast(__builtin_fmaf(sacc[kb][r], scale_log2, -m_new));
                sacc[kb][r] = p;
                lsum += p;
            }
        l_run = l_run * alpha + lsum;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
            oacc[mb] *= alpha;

        // P^T fragments: 16-key step t takes registers 8*(t%2) .. +7 of block t/2.
        bf16x8 pf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            u32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[j] = pack_bf16x2(sacc[t / 2][8 * (t % 2) + 2 * j], sacc[t / 2][8 * (t % 2) + 2 * j + 1]);
            pf[t] = as_bf16x8(w);
        }

        // O^T += V^T P^T.  For step t, lane slot j is key 16t + 8(j/4) + 4*hh + (j%4).
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb) {
            const uint16_t* vrow = Vt + (32 * mb + n) * Cfg::kVStride + 4 * hh;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bf16x8 vf = cat_bf16x8(ld_lds8(vrow + 16 * t), ld_lds8(vrow + 16 * t + 8));
                oacc[mb] = mfma32x32x16(vf, pf[t], oacc[mb]);
            }
        }
    }

    const float l_tot = l_run + xor32(l_run);
    const float inv_l = 1.f / l_tot;
    if (q_row < Sq) {
        uint16_t* dst = O + ((long)b * Sq * H + h) * D + (long)q_row * tok + 4 * hh;
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(oacc[mb][4 * g + 0] * inv_l, oacc[mb][4 * g + 1] * inv_l);
                w[1] = pack_bf16x2(oacc[mb][4 * g + 2] * inv_l, oacc[mb][4 * g + 3] * inv_l);
                *reinterpret_cast<u32x2*>(dst + 32 * mb + 8 * g) = w;
            }
        if (hh == 0)
            LSE[((long)b * H + h) * Sq + q_row] = (m_run + log2_fast(l_tot)) * kLn2;
    }
}

template <int D>
hipError_t launch_fwd_bf16_d(const FwdArgs& a, hipStream_t stream)
{
    using Cfg = FwdBf16Cfg<D>;
    const int n_qtiles = (a.Sq + Cfg::kBr - 1) / Cfg::kBr;
    const long n_blocks = (long)n_qtiles * a.H * a.B;
    if (n_blocks > 0x7fffffffL)
        return hipErrorInvalidConfiguration;
    const float scale_log2 = a.scale * kLog2e;
    return launch_kernel(fwd_bf16_kernel<D>, dim3((unsigned)n_blocks), dim3(Cfg::kThreads),
                         stream, a.q, a.k, a.v, a.o, a.lse, a.H, a.Sq, a.Skv, scale_log2,
                         n_qtiles, (int)n_blocks);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream)
{
    return a.d == 64 ? launch_fwd_bf16_d<64>(a, stream) : launch_fwd_bf16_d<128>(a, stream);
}

}  // namespace dit
