// fwd_fp8.hip -- non-causal attention forward pass (O + LSE) on e4m3 inputs
// with per-(b, h, 128-token block) fp32 scales, for gfx950 (CDNA4) fp8 MFMA.
//
// The FP8 attention backend of "AMD、Radeon AI PRO R9700S最大4台で..." (quick-start
// flags and tuning section) runs attention on FP8 activations natively; the
// block-scaled format follows "生成AI推論を速くするための設計ノート" sec. 3
// (payload + block scales).  Inputs come from dit_quant_fp8:
//     x[b,s,h,c] ~= e4m3(x8[b,s,h,c]) * scale[b,h,s/128].
// What is computed is the same attention as the bf16 kernel (softmax(scale *
// Q K^T) V and LSE), on the dequantised inputs, with P rounded to e4m3 for P.V.
//
// Work decomposition (mirrors the bf16 kernel): 4 waves x 32 query rows per
// workgroup, 64-key tiles double-buffered in LDS through buffer_load ... lds.
//   S^T = K8 Q8^T on v_mfma_scale_f32_32x32x64_f8f6f4 (unit E8M0 scales); the
//     fp32 block scales are uniform per (query tile, key tile) because both
//     tiles sit inside one 128-token block, so q_scale * k_scale * scale *
//     log2(e) becomes the coefficient of the softmax FMA.
//   Softmax as in the bf16 kernel (log2 domain, lazy rescale with a 2^2
//     threshold, so every weight is <= 4 and stays in e4m3's normal range).
//   O^T += V8^T P^T on the same MFMA.  The V block scale v_s = 2^e * f
//     (f in [1,2)) is split: f and the constant K = 448 / 2^3 go into the
//     exponent (P'' = P * f * K = exp2(s*c - m + log2(f*K)) <= 448, rounded to
//     e4m3), 2^e goes into the MFMA's E8M0 scale of P.  O_acc then collects
//     K * sum_j P~_j v_j with P~ the rounded weights.  O is normalised by the
//     sum of the same rounded weights (so O is a convex combination of the
//     values and a single key returns its value), taken by one more MFMA per
//     tile against an all-ones operand; LSE uses the sum of the unrounded
//     weights, which keeps it exact up to fp32 rounding.
//   P^T operand: the S^T accumulator gives lane (n, half) keys 8q + 4*half +
//     0..3 in register group q; after packing to e4m3 (4 keys per dword), one
//     v_permlane32_swap per pair of groups makes lane half g hold keys
//     16t + 8g + 0..7, matching the V operand read with ds_read_b64_tr_b8 (a
//     16-lane group reads 8 key rows x 16 channels and lane i receives channel
//     i of the 8 rows).
//   LDS rows hold d e4m3 bytes; chunk c of row r sits at slot c ^ h(r) (see
//   fp8_slot) so the 16-row K reads and the 8-row transpose reads are free of
//   bank conflicts.
#include "common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

template <int D>
struct FwdFp8Cfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBr = 32 * kWaves;               // query rows per workgroup
    static constexpr int kBc = 64;                        // keys per tile
    static constexpr int kRowBytes = D;                   // one e4m3 row
    static constexpr int kChunks = D / 16;                // 16-byte chunks per row
    static constexpr int kTileBytes = kBc * kRowBytes;
    static constexpr int kLoads = kTileBytes / (16 * kThreads);
    static constexpr int kMB = D / 32;                    // 32-channel output blocks
    static constexpr int kKSteps = D / 64;                // MFMA k-steps of Q.K^T
    static constexpr float kRescaleThreshold = 2.0f;      // log2 units: weights <= 4
    static constexpr float kPScale = 56.0f;               // 448 / 2^(threshold + 1)
    static constexpr int kScaleBlock = 128;               // tokens per block scale
};

// Chunk slot of chunk c in row r.
template <int D>
__device__ __forceinline__ int fp8_slot(int r, int c)
{
    if constexpr (D == 128) {
        const int u = (r >> 1) & 7;
        return c ^ (((u & 3) << 1) | (u >> 2));
    } else {
        const int u = (r >> 2) & 3;
        return c ^ (((u & 1) << 1) | (u >> 1));
    }
}

template <int D>
__device__ __forceinline__ int fp8_lds_byte(int r, int col)
{
    return r * D + fp8_slot<D>(r, col >> 4) * 16 + (col & 15);
}

__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, f32x16 c, int scale_b)
{
    // format 0 = e4m3 for both operands; E8M0 scale 127 = 1.0 for A
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, scale_b);
}

// Four transpose reads (8 bytes each) at p + t * ROW16, t = 0..3: the V^T
// operand of one 32x32x64 MFMA (keys 16t..16t+15 in dwords 2t, 2t+1).
template <int ROW16>
__device__ __forceinline__ i32x8 tr8_read4(const uint8_t* p)
{
    const u32x2 o0 = ld_lds_tr8(p), o1 = ld_lds_tr8(p + ROW16), o2 = ld_lds_tr8(p + 2 * ROW16),
                o3 = ld_lds_tr8(p + 3 * ROW16);
    return i32x8{(int)o0[0], (int)o0[1], (int)o1[0], (int)o1[1],
                 (int)o2[0], (int)o2[1], (int)o3[0], (int)o3[1]};
}

// Pack 4 fp32 into 4 e4m3 bytes (round to nearest even; inputs <= 448).
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d)
{
    // both halves are written: the old value of the first is irrelevant (an
    // uninitialised register, so the compiler does not zero it first)
    int w;
    asm volatile("" : "=v"(w));
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

template <int D>
struct FwdFp8Tile {
    using Cfg = FwdFp8Cfg<D>;
    static constexpr int kBc = Cfg::kBc;
    static constexpr int kMB = Cfg::kMB;

    uint8_t* kbuf[2];        // K and V tile buffers, each its own LDS object, so the
    uint8_t* vbuf[2];        // compiler sees operand reads never alias a copy in flight
    __amdgpu_buffer_rsrc_t k_rsrc, v_rsrc;
    uint32_t tok_bytes;
    int Skv, kt_end, wave, hh;  // key tiles up to kt_end (exclusive) are processed
    float qc;                // q_scale * scale * log2(e) of this query tile
    const float* ks;         // k scales of this (b, h)
    const float* vs;         // v scales of this (b, h)
    int ld_row[Cfg::kLoads];
    uint32_t ld_voff[Cfg::kLoads];
    i32x8 qf[Cfg::kKSteps];
    int k_addr[Cfg::kKSteps][2];
    int v_addr[kMB];
    f32x16 oacc[kMB];
    float m_used;  // log2-domain maximum the weights are taken against
    float l_run;   // running sum of unrounded weights over this lane's keys
    float lr_run;  // running sum of the e4m3-rounded weights over all keys
    i32x8 ones;    // all-ones e4m3 operand of the rounded-weight sums
    f32x16 rs;     // the last tile's rounded-weight sums (added at the next step)
    float rs_inv;  // and their 1 / (f K)

    template <int BUF>
    __device__ __forceinline__ void issue(int kt_next)
    {
        const int key0 = kt_next * kBc;
        const uint32_t soff = (uint32_t)key0 * tok_bytes;
        if (key0 + kBc <= Skv) {
#pragma unroll
            for (int i = 0; i < Cfg::kLoads; ++i) {
                const int off = (i * Cfg::kWaves + wave) * 1024;
                copy16_to_lds(k_rsrc, kbuf[BUF] + off, ld_voff[i], soff);
                copy16_to_lds(v_rsrc, vbuf[BUF] + off, ld_voff[i], soff);
            }
        } else {
#pragma unroll
            for (int i = 0; i < Cfg::kLoads; ++i) {
                const int off = (i * Cfg::kWaves + wave) * 1024;
                const int over = max(key0 + ld_row[i] - (Skv - 1), 0);
                const uint32_t vo = ld_voff[i] - (uint32_t)over * tok_bytes;
                copy16_to_lds(k_rsrc, kbuf[BUF] + off, vo, soff);
                copy16_to_lds(v_rsrc, vbuf[BUF] + off, vo, soff);
            }
        }
    }

    // The previous tile's rounded-weight sum into lr_run (read one step late,
    // so that no instruction waits on that matrix instruction).
    __device__ __forceinline__ void add_rs()
    {
        // rs is held (all 16 registers) up to here, so none of them is handed
        // to other values while that matrix instruction may still write it
        asm volatile("" ::"v"(rs));
        lr_run += rs[0] * rs_inv;
    }

    template <int BUF>
    __device__ __forceinline__ void step(int kt)
    {
        const int key0 = kt * kBc;
        if (kt + 1 < kt_end)
            issue<BUF ^ 1>(kt + 1);
        add_rs();

        // block scales of this key tile (uniform): both lie in block key0/128
        const int kblk = key0 / Cfg::kScaleBlock;
        const float c = qc * ks[kblk];
        const uint32_t vbits = __builtin_bit_cast(uint32_t, vs[kblk]);
        const int vexp = max((int)((vbits >> 23) & 0xff), 1);          // E8M0 exponent of v_s
        const float vmant = vs[kblk] * __builtin_bit_cast(float, (uint32_t)(254 - vexp) << 23);
        const float lift = log2_fast(vmant * Cfg::kPScale);            // log2(f * K)

        // S^T = K8 Q8^T for two 32-key blocks
        f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int s = 0; s < Cfg::kKSteps; ++s)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const u32x4 lo = ld_lds16(kbuf[BUF] + k_addr[s][0] + 32 * kb * D);
                const u32x4 hi = ld_lds16(kbuf[BUF] + k_addr[s][1] + 32 * kb * D);
                i32x8 a;
                a[0] = (int)lo[0]; a[1] = (int)lo[1]; a[2] = (int)lo[2]; a[3] = (int)lo[3];
                a[4] = (int)hi[0]; a[5] = (int)hi[1]; a[6] = (int)hi[2]; a[7] = (int)hi[3];
                sacc[kb] = mfma_fp8_32x32x64(a, qf[s], sacc[kb], 127);
            }
        // V^T operands of this tile, read while the K Q^T instructions run
        i32x8 va[kMB];
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
            va[mb] = tr8_read4<16 * D>(vbuf[BUF] + v_addr[mb]);
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
        const float m_tile = mx * c;
        const bool grow = m_tile > m_used + Cfg::kRescaleThreshold;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float m_new = grow ? m_tile : m_used;
            const float alpha = exp2_fast(m_used - m_new);
            m_used = m_new;
            l_run *= alpha;
            lr_run *= alpha;
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb)
                oacc[mb] *= alpha;
        }

        // P'' = P * f * K, rounded to e4m3; the LSE sum takes P itself.
        const float m_eff = m_used - lift;
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = exp2_fast(__builtin_fmaf(sacc[kb][r], c, -m_eff));
                sacc[kb][r] = p;
                lsum += p;
            }
        const float inv_fk = __builtin_amdgcn_rcpf(vmant * Cfg::kPScale);
        l_run += lsum * inv_fk;

        // pack: dword q of block kb = keys 32kb + 8q + 4hh + 0..3
        uint32_t pw[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                pw[kb][q] = pack_e4m3x4(sacc[kb][4 * q], sacc[kb][4 * q + 1],
                                        sacc[kb][4 * q + 2], sacc[kb][4 * q + 3]);
        // regroup so lane half g holds keys 16t + 8g + 0..7 in dwords (2t, 2t+1)
        i32x8 pf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                const auto sw = __builtin_amdgcn_permlane32_swap(
                    (int)pw[kb][2 * t2], (int)pw[kb][2 * t2 + 1], false, false);
                pf[2 * (2 * kb + t2)] = sw[0];
                pf[2 * (2 * kb + t2) + 1] = sw[1];
            }

        // O^T += V8^T P''^T, P'' carrying the 2^e part of the V block scale
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
            oacc[mb] = mfma_fp8_32x32x64(va[mb], pf, oacc[mb], vexp);

        // Sum of the rounded weights of this tile: every row of ones^T P''^T
        // holds it (the same value in both lane halves).
        rs = mfma_fp8_32x32x64(ones, pf, f32x16{}, 127);
        rs_inv = inv_fk;

        wait_vmem_all();
        __syncthreads();
    }
};

// Grid: blocks [0, n_main) each take one query tile over all keys; with a
// split launch the remaining tiles are each split into nsplit pieces over
// contiguous ranges of key tiles, which write normalised fp32 O, LSE and the
// log of their rounded-weight sum (the sum O was normalised by) to the
// workspace: ws_o [piece][kBr][D], ws_lse [piece][kBr], ws_lr [piece][kBr].
// The merge weights each piece's O by its rounded-weight sum, so the merged O
// is again sum_j P~_j v_j / sum_j P~_j over all keys.
template <int D>
__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const float* __restrict__ QS, const float* __restrict__ KS, const float* __restrict__ VS,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H, int Sq, int Skv, float scale_log2,
    int n_qtiles, int n_main, int nsplit, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    float* __restrict__ ws_lr, int acc)
{
    using Cfg = FwdFp8Cfg<D>;
    constexpr int kMB = Cfg::kMB;
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[Cfg::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[Cfg::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[Cfg::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[Cfg::kTileBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int n = lane & 31;
    const int hh = lane >> 5;

    const int n_kt = (Skv + Cfg::kBc - 1) / Cfg::kBc;
    int logical, kt0, kt1, piece;
    if ((int)blockIdx.x < n_main) {
        logical = xcd_remap(blockIdx.x, n_main);
        kt0 = 0;
        kt1 = n_kt;
        piece = -1;
    } else {
        piece = blockIdx.x - n_main;
        logical = n_main + piece / nsplit;
        const int part = piece % nsplit;
        kt0 = (int)((long)part * n_kt / nsplit);
        kt1 = (int)((long)(part + 1) * n_kt / nsplit);
    }
    const int qt = logical % n_qtiles;
    const int bh = logical / n_qtiles;
    const int h = bh % H;
    const int b = bh / H;
    const long tok = (long)H * D;  // bytes between consecutive tokens
    const int nqb = (Sq + Cfg::kScaleBlock - 1) / Cfg::kScaleBlock;
    const int nkb = (Skv + Cfg::kScaleBlock - 1) / Cfg::kScaleBlock;

    FwdFp8Tile<D> st;
    st.kbuf[0] = k_lds0;
    st.kbuf[1] = k_lds1;
    st.vbuf[0] = v_lds0;
    st.vbuf[1] = v_lds1;
    st.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    st.hh = hh;
    st.Skv = Skv;
    st.kt_end = kt1;
    st.tok_bytes = (uint32_t)tok;
    // the query tile of 128 rows is exactly query block qt
    st.qc = QS[(long)bh * nqb + qt] * scale_log2;
    st.ks = KS + (long)bh * nkb;
    st.vs = VS + (long)bh * nkb;
    {
        const uint8_t* Kbh = K + ((long)b * Skv * H + h) * D;
        const uint8_t* Vbh = V + ((long)b * Skv * H + h) * D;
        const int extent = (int)((uint32_t)(Skv - 1) * st.tok_bytes + D);
        st.k_rsrc = make_rsrc(Kbh, extent);
        st.v_rsrc = make_rsrc(Vbh, extent);
    }
#pragma unroll
    for (int i = 0; i < Cfg::kLoads; ++i) {
        const int p = (i * Cfg::kWaves + st.wave) * 64 + lane;
        const int r = p / Cfg::kChunks;
        st.ld_row[i] = r;
        st.ld_voff[i] = (uint32_t)r * st.tok_bytes + fp8_slot<D>(r, p % Cfg::kChunks) * 16;
    }
    st.template issue<0>(kt0);

    const int q_row = qt * Cfg::kBr + st.wave * 32 + n;
    if (q_row < Sq) {
        const uint8_t* src = Q + ((long)b * Sq * H + h) * D + (long)q_row * tok + 32 * hh;
#pragma unroll
        for (int s = 0; s < Cfg::kKSteps; ++s) {
            const u32x4 lo = ld_global16(src + 64 * s);
            const u32x4 hi = ld_global16(src + 64 * s + 16);
            st.qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                             (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    } else {
#pragma unroll
        for (int s = 0; s < Cfg::kKSteps; ++s)
            st.qf[s] = i32x8{};
    }

    // K operand (A of S^T), step s: row n (+32 for the second block), bytes
    // 64s + 32hh .. +31 (two chunks).  V transpose reads, block mb: lane group
    // (hh, g2 = (lane/16)%2) reads rows 8hh + (lane%16)/2 (+16t) at channels
    // 32mb + 16g2 + 8(lane%2) .. +7.
#pragma unroll
    for (int s = 0; s < Cfg::kKSteps; ++s)
#pragma unroll
        for (int e = 0; e < 2; ++e)
            st.k_addr[s][e] = fp8_lds_byte<D>(n, 64 * s + 32 * hh + 16 * e);
    {
        const int vr = 8 * hh + ((lane & 15) >> 1);
        const int vc = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
            st.v_addr[mb] = fp8_lds_byte<D>(vr, 32 * mb + vc);
    }
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
        st.oacc[mb] = f32x16{};
    st.m_used = -INFINITY;
    st.l_run = 0.f;
    st.lr_run = 0.f;
    st.rs = f32x16{};
    st.rs_inv = 0.f;
    // e4m3 1.0 in every byte, placed in registers once for the whole kernel
    st.ones = i32x8{0x38383838, 0x38383838, 0x38383838, 0x38383838,
                    0x38383838, 0x38383838, 0x38383838, 0x38383838};
    asm volatile("" : "+v"(st.ones));

    wait_vmem_all();
    __syncthreads();

    for (int kt = kt0; kt < kt1; kt += 2) {
        st.template step<0>(kt);
        if (kt + 1 < kt1)
            st.template step<1>(kt + 1);
    }
    st.add_rs();

    const float l_tot = st.l_run + partner32(st.l_run, hh);
    const float inv = 1.f / (st.lr_run * Cfg::kPScale);
    if (piece >= 0) {
        // partial result of a split tile
        const int r = st.wave * 32 + n;
        float* dst = ws_o + ((long)piece * Cfg::kBr + r) * D + 4 * hh;
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 w = {st.oacc[mb][4 * g + 0] * inv, st.oacc[mb][4 * g + 1] * inv,
                           st.oacc[mb][4 * g + 2] * inv, st.oacc[mb][4 * g + 3] * inv};
                *reinterpret_cast<f32x4*>(dst + 32 * mb + 8 * g) = w;
            }
        if (hh == 0) {
            ws_lse[(long)piece * Cfg::kBr + r] = (st.m_used + log2_fast(l_tot)) * kLn2;
            ws_lr[(long)piece * Cfg::kBr + r] = (st.m_used + log2_fast(st.lr_run)) * kLn2;
        }
    } else if (q_row < Sq) {
        uint16_t* dst = O + ((long)b * Sq * H + h) * D + (long)q_row * tok + 4 * hh;
        float* lse_dst = LSE + ((long)b * H + h) * Sq + q_row;
        const float lse_new = (st.m_used + log2_fast(l_tot)) * kLn2;
        // O = c_new * acc + c_old * O_old; without a running result (acc = 0, or
        // its LSE is -inf) that is the plain normalisation
        float c_new = inv, c_old = 0.f, lse_out = lse_new;
        if (acc)
            merge_weights(*lse_dst, lse_new, c_new, c_old, lse_out);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 o = {st.oacc[mb][4 * g + 0] * c_new, st.oacc[mb][4 * g + 1] * c_new,
                           st.oacc[mb][4 * g + 2] * c_new, st.oacc[mb][4 * g + 3] * c_new};
                u32x2* p = reinterpret_cast<u32x2*>(dst + 32 * mb + 8 * g);
                if (c_old != 0.f) {
                    const u32x2 old = *p;
                    o += c_old * f32x4{bf16_lo(old[0]), bf16_hi(old[0]), bf16_lo(old[1]),
                                       bf16_hi(old[1])};
                }
                *p = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            }
        if (hh == 0)
            *lse_dst = lse_out;
    }
}

template <int D>
FwdSplit plan_d(int B, int H, int Sq, int Skv, int n_cu)
{
    using Cfg = FwdFp8Cfg<D>;
    const long n_blocks = (long)((Sq + Cfg::kBr - 1) / Cfg::kBr) * H * B;
    const long n_kt = (Skv + Cfg::kBc - 1) / Cfg::kBc;
    return plan_split(n_blocks, n_kt, Cfg::kBr, 2, n_cu, D + 2);
}

template <int D>
hipError_t launch_fwd_fp8_d(const FwdArgs& a, const FwdSplit& sp, hipStream_t stream)
{
    using Cfg = FwdFp8Cfg<D>;
    const int n_qtiles = (a.Sq + Cfg::kBr - 1) / Cfg::kBr;
    const long n_blocks = (long)n_qtiles * a.H * a.B;
    if (n_blocks > 0x7fffffffL)
        return hipErrorInvalidConfiguration;
    const float scale_log2 = a.scale * kLog2e;
    const bool split = sp.n_tail > 0;
    const size_t n_rows = split ? (size_t)sp.n_tail * sp.nsplit * Cfg::kBr : 0;
    float* ws_o = split ? static_cast<float*>(a.ws) : nullptr;
    float* ws_lse = split ? ws_o + n_rows * D : nullptr;
    float* ws_lr = split ? ws_lse + n_rows : nullptr;
    const long grid = split ? (long)sp.n_main + (long)sp.n_tail * sp.nsplit : n_blocks;
    hipError_t e = launch_kernel(fwd_fp8_kernel<D>, dim3((unsigned)grid), dim3(Cfg::kThreads),
                                 stream, a.q, a.k, a.v, a.q_scale, a.k_scale, a.v_scale, a.o,
                                 a.lse, a.H, a.Sq, a.Skv, scale_log2, n_qtiles,
                                 split ? sp.n_main : (int)n_blocks, split ? sp.nsplit : 1, ws_o,
                                 ws_lse, ws_lr, a.acc);
    if (e != hipSuccess || !split)
        return e;
    return launch_split_merge(a, sp, Cfg::kBr, n_qtiles, ws_o, ws_lse, ws_lr, stream);
}

}  // namespace

FwdSplit plan_fwd_fp8_split(int B, int H, int Sq, int Skv, int d, int n_cu)
{
    return d == 64 ? plan_d<64>(B, H, Sq, Skv, n_cu) : plan_d<128>(B, H, Sq, Skv, n_cu);
}

hipError_t launch_fwd_fp8(const FwdArgs& a, const FwdSplit& split, hipStream_t stream)
{
    return a.d == 64 ? launch_fwd_fp8_d<64>(a, split, stream)
                     : launch_fwd_fp8_d<128>(a, split, stream);
}

}  // namespace dit
