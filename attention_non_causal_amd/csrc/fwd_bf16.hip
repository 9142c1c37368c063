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
//   while a tile is consumed, the next is copied global -> LDS by
//   buffer_load_dwordx4 ... lds (no VGPR staging).  Each lane's buffer offset
//   within a tile is fixed for the whole kernel and the tile's start is a
//   scalar offset, so a full tile costs no vector address arithmetic; the
//   last, partial tile clamps its rows to the last key instead (every LDS value
//   stays finite).  One barrier per tile separates producer and consumer.
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
//   LDS layout: rows of D bf16; the 16-byte chunk c of row r sits at chunk
//   slot c ^ f(r), where f permutes bits of r so that both read patterns are
//   free of bank conflicts -- 16 rows x one chunk (the K operand) and 4 rows
//   x 4 chunks (the transpose read of V) each cover all 64 banks.  Every LDS
//   address is a per-lane base (computed once) plus a compile-time offset.
//   Tails: query rows >= Sq are computed on zero queries and never stored;
//   keys >= Skv get score -inf.
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
    static constexpr int kRowBytes = D * 2;
    static constexpr int kTileBytes = kBc * kRowBytes;     // one K or V tile
    static constexpr int kBufBytes = 2 * kTileBytes;       // K tile then V tile
    static constexpr int kLoads = kTileBytes / (16 * kThreads);  // 16-B loads per thread
    static constexpr int kMB = D / 32;                     // 32-channel output blocks
    static constexpr float kRescaleThreshold = 8.0f;       // log2 units
};

// Chunk slot of chunk c in row r (see the layout note above).
template <int D>
__device__ __forceinline__ int swz_slot(int r, int c)
{
    if constexpr (D == 128) {
        return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
    } else {
        const int u = (r >> 1) & 7;
        return c ^ (((u & 1) << 2) | (u >> 1));
    }
}

template <int D>
__device__ __forceinline__ int lds_byte(int r, int col)
{
    return r * (D * 2) + swz_slot<D>(r, col >> 3) * 16 + (col & 7) * 2;
}

// N transpose reads at per-lane addresses a[i] + OFF, completed before return.
// (Written out so the reads carry no implied dependence on the outstanding
// global -> LDS copies into the other buffer.)
template <int OFF>
__device__ __forceinline__ void tr_read4(u32x2 (&o)[4], const int (&a)[4])
{
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%8\n\t"
        "ds_read_b64_tr_b16 %1, %5 offset:%8\n\t"
        "ds_read_b64_tr_b16 %2, %6 offset:%8\n\t"
        "ds_read_b64_tr_b16 %3, %7 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF)
        : "memory");
}

template <int OFF>
__device__ __forceinline__ void tr_read8(u32x2 (&o)[8], const int (&a)[8])
{
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%16\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:%16\n\t"
        "ds_read_b64_tr_b16 %2, %10 offset:%16\n\t"
        "ds_read_b64_tr_b16 %3, %11 offset:%16\n\t"
        "ds_read_b64_tr_b16 %4, %12 offset:%16\n\t"
        "ds_read_b64_tr_b16 %5, %13 offset:%16\n\t"
        "ds_read_b64_tr_b16 %6, %14 offset:%16\n\t"
        "ds_read_b64_tr_b16 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
          "=&v"(o[6]), "=&v"(o[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "i"(OFF)
        : "memory");
}

template <int D, int OFF>
__device__ __forceinline__ void tr_read(u32x2 (&o)[2 * D / 32], const int (&a)[2 * D / 32])
{
    if constexpr (D == 128)
        tr_read8<OFF>(o, a);
    else
        tr_read4<OFF>(o, a);
}

// Per-thread state of one workgroup's pass over the keys.
template <int D>
struct FwdBf16Tile {
    using Cfg = FwdBf16Cfg<D>;
    static constexpr int kBc = Cfg::kBc;
    static constexpr int kTile = Cfg::kTileBytes;
    static constexpr int kRow = Cfg::kRowBytes;
    static constexpr int kMB = Cfg::kMB;

    uint8_t* smem;
    __amdgpu_buffer_rsrc_t k_rsrc, v_rsrc;
    uint32_t tok_bytes;
    int Skv, n_kt, wave, hh;
    float scale_log2;
    int ld_row[Cfg::kLoads];
    uint32_t ld_voff[Cfg::kLoads];
    bf16x8 qf[D / 16];
    int k_addr[D / 16];
    int v_addr[2 * kMB];
    f32x16 oacc[kMB];
    float m_used;  // maximum (scale*log2(e) units) the weights are taken against
    float l_run;   // running sum over this lane's half of the keys

    // Copy key tile kt_next into LDS buffer BUF (K tile, then V tile).
    template <int BUF>
    __device__ __forceinline__ void issue(int kt_next)
    {
        const int key0 = kt_next * kBc;
        const uint32_t soff = (uint32_t)key0 * tok_bytes;
        uint8_t* base = smem + BUF * Cfg::kBufBytes;
        if (key0 + kBc <= Skv) {
#pragma unroll
            for (int i = 0; i < Cfg::kLoads; ++i) {
                uint8_t* dst = base + (i * Cfg::kWaves + wave) * 1024;
                copy16_to_lds(k_rsrc, dst, ld_voff[i], soff);
                copy16_to_lds(v_rsrc, dst + kTile, ld_voff[i], soff);
            }
        } else {
            // partial tile: rows past the last key re-read the last key
#pragma unroll
            for (int i = 0; i < Cfg::kLoads; ++i) {
                uint8_t* dst = base + (i * Cfg::kWaves + wave) * 1024;
                const int over = max(key0 + ld_row[i] - (Skv - 1), 0);
                const uint32_t vo = ld_voff[i] - (uint32_t)over * tok_bytes;
                copy16_to_lds(k_rsrc, dst, vo, soff);
                copy16_to_lds(v_rsrc, dst + kTile, vo, soff);
            }
        }
    }

    // O^T += V^T P^T for 16-key step T; the reads for half hi give slots 4hi..4hi+3.
    template <int VOFF, int T>
    __device__ __forceinline__ void pv_step(const bf16x8& p)
    {
        u32x2 vf[2 * kMB];
        tr_read<D, VOFF + 16 * T * kRow>(vf, v_addr);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
            oacc[mb] = mfma32x32x16(cat_bf16x8(vf[2 * mb], vf[2 * mb + 1]), p, oacc[mb]);
    }

    // Consume key tile kt from LDS buffer BUF while tile kt+1 is copied into
    // the other buffer.
    template <int BUF>
    __device__ __forceinline__ void step(int kt)
    {
        constexpr int KOFF = BUF * Cfg::kBufBytes;
        constexpr int VOFF = KOFF + kTile;
        const int key0 = kt * kBc;
        if (kt + 1 < n_kt)
            issue<BUF ^ 1>(kt + 1);
        const uint8_t* sm = smem;

        // S^T = K Q^T for two 32-key blocks.
        f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                sacc[kb] = mfma32x32x16(
                    as_bf16x8(ld_lds16(sm + k_addr[s] + KOFF + 32 * kb * kRow)), qf[s], sacc[kb]);
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
            for (int mb = 0; mb < kMB; ++mb)
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
        pv_step<VOFF, 0>(pf[0]);
        pv_step<VOFF, 1>(pf[1]);
        pv_step<VOFF, 2>(pf[2]);
        pv_step<VOFF, 3>(pf[3]);

        wait_vmem_all();
        __syncthreads();
    }
};

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int H, int Sq, int Skv, float scale_log2, int n_qtiles, int n_blocks)
{
    using Cfg = FwdBf16Cfg<D>;
    constexpr int kMB = Cfg::kMB;
    constexpr int kRow = Cfg::kRowBytes;
    // [buffer][K tile, V tile]
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * Cfg::kBufBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int n = lane & 31;   // query column of this lane within the wave
    const int hh = lane >> 5;  // which 8-wide k group this lane feeds

    const int logical = xcd_remap(blockIdx.x, n_blocks);
    const int qt = logical % n_qtiles;
    const int bh = logical / n_qtiles;
    const int h = bh % H;
    const int b = bh / H;
    const long tok = (long)H * D;  // elements between consecutive tokens

    FwdBf16Tile<D> st;
    st.smem = smem;
    st.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    st.hh = hh;
    st.Skv = Skv;
    st.n_kt = (Skv + Cfg::kBc - 1) / Cfg::kBc;
    st.scale_log2 = scale_log2;
    st.tok_bytes = (uint32_t)(tok * 2);
    {
        const uint16_t* Kbh = K + ((long)b * Skv * H + h) * D;
        const uint16_t* Vbh = V + ((long)b * Skv * H + h) * D;
        // Byte extent of this (b, h)'s keys: rows 0 .. Skv-1 (callers guarantee < 2^32).
        const int extent = (int)((uint32_t)(Skv - 1) * st.tok_bytes + kRow);
        st.k_rsrc = make_rsrc(Kbh, extent);
        st.v_rsrc = make_rsrc(Vbh, extent);
    }
    // Copy i of wave w fills LDS chunks [(i*kWaves + w)*64, +64) of a tile; lane
    // l takes chunk p = that base + l, i.e. row p / kChunks at slot p % kChunks,
    // which holds column chunk (p % kChunks) ^ f(row).
#pragma unroll
    for (int i = 0; i < Cfg::kLoads; ++i) {
        const int p = (i * Cfg::kWaves + st.wave) * 64 + lane;
        const int r = p / Cfg::kChunks;
        st.ld_row[i] = r;
        st.ld_voff[i] = (uint32_t)r * st.tok_bytes + swz_slot<D>(r, p % Cfg::kChunks) * 16;
    }
    st.template issue<0>(0);

    const int q_row = qt * Cfg::kBr + st.wave * 32 + n;
    if (q_row < Sq) {
        const uint16_t* src = Q + ((long)b * Sq * H + h) * D + (long)q_row * tok + 8 * hh;
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            st.qf[s] = as_bf16x8(ld_global16(src + 16 * s));
    } else {
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            st.qf[s] = as_bf16x8(u32x4{0, 0, 0, 0});
    }

    // Per-lane LDS bases.  K operand (A of S^T), step s: row n (+32 for the
    // second block), column 16s + 8hh.  V transpose reads, block mb, half hi:
    // lane group g = lane/16 reads row 4hh + 8hi + (lane%16)/4 (+16t) at columns
    // 32mb + 16(g%2) + 4(lane%4) .. +3, so lane l receives channel 32mb + l%32
    // of keys 16t + 8hi + 4hh + 0..3.
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
        st.k_addr[s] = lds_byte<D>(n, 16 * s + 8 * hh);
    {
        const int vr = 4 * hh + ((lane & 15) >> 2);
        const int vc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi)
                st.v_addr[2 * mb + hi] = lds_byte<D>(vr + 8 * hi, 32 * mb + vc);
    }
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
        st.oacc[mb] = f32x16{};
    st.m_used = -INFINITY;
    st.l_run = 0.f;

    wait_vmem_all();
    __syncthreads();

    for (int kt = 0; kt < st.n_kt; kt += 2) {
        st.template step<0>(kt);
        if (kt + 1 < st.n_kt)
            st.template step<1>(kt + 1);
    }

    const float l_tot = st.l_run + partner32(st.l_run, hh);
    const float inv_l = 1.f / l_tot;
    if (q_row < Sq) {
        uint16_t* dst = O + ((long)b * Sq * H + h) * D + (long)q_row * tok + 4 * hh;
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = pack_bf16x2(st.oacc[mb][4 * g + 0] * inv_l, st.oacc[mb][4 * g + 1] * inv_l);
                w[1] = pack_bf16x2(st.oacc[mb][4 * g + 2] * inv_l, st.oacc[mb][4 * g + 3] * inv_l);
                *reinterpret_cast<u32x2*>(dst + 32 * mb + 8 * g) = w;
            }
        if (hh == 0)
            LSE[((long)b * H + h) * Sq + q_row] = (st.m_used + log2_fast(l_tot)) * kLn2;
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
