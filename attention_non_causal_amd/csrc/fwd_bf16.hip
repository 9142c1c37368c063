// fwd_bf16.hip -- non-causal attention forward pass (O + LSE) in bf16 with
// fp32 accumulation, for gfx950 (CDNA4) MFMA.
//
// What is computed: per (batch, head), O = softmax(scale * Q K^T) V and
// LSE = ln sum_j exp(scale * q . k_j) -- the whole-sequence, cache-free
// attention of DiT inference ("xDiT 项目概述", sec. 2.1), done by a dedicated
// kernel as "生成AI推論を速くするための設計ノート" sec. 5 recommends for an
// attention that dominates.  The kernel reaches the exact result (up to fp32
// rounding order) in one pass over key tiles with a running maximum and sum
// (online softmax).
//
// Work decomposition
//   Workgroup = 4 wavefronts = 128 query rows of one (batch, head); each wave
//   owns 32 rows.  Keys stream through LDS in tiles of 64, double-buffered:
//   while a tile is consumed, the next one is copied global -> LDS by
//   global_load_lds_dwordx4 (no VGPR staging), so one barrier per tile
//   separates producer and consumer.
//   Per tile and wave:
//     S^T (keys x queries) = K Q^T on v_mfma_f32_32x32x16_bf16: A = K rows from
//       LDS, B = Q^T held in registers for the whole kernel.  The transpose
//       puts one query per lane column, so a row maximum or sum is a per-lane
//       reduction plus one exchange with lane l^32 (v_permlane32_swap).
//     Online softmax in the log2 domain: scale*log2(e) is folded into one FMA
//       before v_exp_f32.  The output is rescaled only when a row maximum grows
//       by more than 2^8 over the one in use; until then the stale maximum
//       keeps every weight below 2^8, and the final O / sum and LSE are exact
//       for any maximum, so this skips almost all rescale multiplies.
//     O^T (channels x queries) += V^T P^T: A = V^T read from the row-major V
//       tile with ds_read_b64_tr_b16 (LDS transpose read), B = P^T straight from
//       the S^T accumulator registers.  A and B use the same assignment of keys
//       to k slots, so no register shuffle is needed.
//   LDS tiles are XOR-swizzled in 16-byte chunks (chunk c of row r is stored
//   at chunk c ^ (r mod chunks-per-row)), so the 32 rows one MFMA operand read
//   touches spread over all banks.
//   Tails: key indices past Skv are clamped to the last key for loading (so
//   every LDS value is finite) and their scores set to -inf; query rows >= Sq
//   are computed on zero queries and never stored.
#include "common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

template <int D>
struct FwdBf16Cfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBr = 32 * kWaves;                // query rows per workgroup
    static constexpr int kBc = 64;                         // keys per tile
    static constexpr int kChunks = D / 8;                  // 16-byte chunks per key row
    static constexpr int kTileBytes = kBc * D * 2;         // one K or V tile
    static constexpr int kLoads = kTileBytes / (16 * kThreads);  // 16-B loads per thread per tile
    static constexpr float kRescaleThreshold = 8.0f;       // log2 units
};

// Byte offset, inside a swizzled tile, of element (row, col).
template <int D>
__device__ __forceinline__ int swz(int row, int col)
{
    constexpr int kChunks = D / 8;
    return (row * kChunks + ((col >> 3) ^ (row & (kChunks - 1)))) * 16 + (col & 7) * 2;
}

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int H, int Sq, int Skv, float scale_log2, int n_qtiles, int n_blocks)
{
    using Cfg = FwdBf16Cfg<D>;
    constexpr int kBc = Cfg::kBc;
    constexpr int kTile = Cfg::kTileBytes;
    // [buffer][K, V][tile]
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * 2 * kTile];

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

    // ---- producer: this thread's share of a tile copy -------------------
    // Load i of wave w fills LDS chunks [(i*kWaves + w)*64, +64); lane l takes
    // chunk p = that base + l, i.e. row p / kChunks, swizzled column chunk.
    int ld_row[Cfg::kLoads], ld_col[Cfg::kLoads];
#pragma unroll
    for (int i = 0; i < Cfg::kLoads; ++i) {
        const int p = (i * Cfg::kWaves + wave) * 64 + lane;
        const int r = p / Cfg::kChunks;
        ld_row[i] = r;
        ld_col[i] = ((p % Cfg::kChunks) ^ (r & (Cfg::kChunks - 1))) * 8;
    }
    auto issue_tile = [&](int key0, int buf) {
        uint8_t* kdst = smem + (2 * buf) * kTile;
        uint8_t* vdst = kdst + kTile;
#pragma unroll
        for (int i = 0; i < Cfg::kLoads; ++i) {
            const int key = min(key0 + ld_row[i], Skv - 1);
            const long off = (long)key * tok + ld_col[i];
            const int lds_off = (i * Cfg::kWaves + wave) * 1024;
            __builtin_amdgcn_global_load_lds(
                Kbh + off, (__attribute__((address_space(3))) void*)(kdst + lds_off), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(
                Vbh + off, (__attribute__((address_space(3))) void*)(vdst + lds_off), 16, 0, 0);
        }
    };

    const int n_kt = (Skv + kBc - 1) / kBc;
    issue_tile(0, 0);

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
    float m_used = -INFINITY;  // maximum (scale*log2(e) units) the weights are taken against
    float l_run = 0.f;         // running sum over this lane's half of the keys

    // Per-lane coordinates of the V transpose reads: lane group g = lane/16
    // reads rows 16t + 4*hh (+8 for slots 4..7) + (lane%16)/4 at columns
    // 32*mb + 16*(g%2) + 4*(lane%4) .. +3; lane l then holds channel
    // 32*mb + l%32 for 4 consecutive keys.
    const int v_row = 4 * hh + ((lane & 15) >> 2);
    const int v_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    wait_vmem_all();
    __syncthreads();

    for (int kt = 0; kt < n_kt; ++kt) {
        const int buf = kt & 1;
        const int key0 = kt * kBc;
        if (kt + 1 < n_kt)
            issue_tile(key0 + kBc, buf ^ 1);
        const uint8_t* Kt = smem + (2 * buf) * kTile;
        const uint8_t* Vt = Kt + kTile;

        // S^T = K Q^T for two 32-key blocks.
        f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                sacc[kb] = mfma32x32x16(
                    as_bf16x8(ld_lds16(Kt + swz<D>(32 * kb + n, 16 * s + 8 * hh))), qf[s],
                    sacc[kb]);
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
        mx = fmaxf(mx, partner32(mx, hh));
        const float m_tile = mx * scale_log2;
        const bool grow = m_tile > m_used + Cfg::kRescaleThreshold;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? m_tile : m_used;
            const float alpha = exp2_fast(m_used - m_new);
            m_used = m_new;
            l_run *= alpha;
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb)
                oacc[mb] *= alpha;
        }

        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = exp2_fast(__builtin_fmaf(sacc[kb][r], scale_log2, -m_used));
                sacc[kb][r] = p;
                lsum += p;
            }
        l_run += lsum;

        // P^T fragments: 16-key step t takes registers 8*(t%2) .. +7 of block t/2;
        // slot j is key 16t + 8(j/4) + 4*hh + (j%4).
        bf16x8 pf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            u32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[j] = pack_bf16x2(sacc[t / 2][8 * (t % 2) + 2 * j],
                                   sacc[t / 2][8 * (t % 2) + 2 * j + 1]);
            pf[t] = as_bf16x8(w);
        }

        // O^T += V^T P^T; the two transpose reads give slots 0..3 (keys
        // 16t + 4hh + 0..3) and 4..7 (keys 16t + 8 + 4hh + 0..3).
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int mb = 0; mb < D / 32; ++mb) {
                const u32x2 lo = ld_lds_tr16(Vt + swz<D>(16 * t + v_row, 32 * mb + v_col));
                const u32x2 hi = ld_lds_tr16(Vt + swz<D>(16 * t + 8 + v_row, 32 * mb + v_col));
                oacc[mb] = mfma32x32x16(cat_bf16x8(lo, hi), pf[t], oacc[mb]);
            }

        wait_vmem_all();
        __syncthreads();
    }

    const float l_tot = l_run + partner32(l_run, hh);
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
            LSE[((long)b * H + h) * Sq + q_row] = (m_used + log2_fast(l_tot)) * kLn2;
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
