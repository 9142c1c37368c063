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
// Work decomposition: a workgroup of 8 waves x 32 query rows (256 rows) per
// CU, in two groups of four waves (128 rows each: one query scale block).
// 64-key tiles of K and V stream through a ring of four LDS slots, copied two
// tiles ahead with buffer_load ... lds.
//   S^T = K8 Q8^T on v_mfma_scale_f32_32x32x64_f8f6f4 (unit E8M0 scales); the
//     fp32 block scales are uniform per (query group, key tile) because both
//     sit inside one 128-token block, so q_scale * k_scale * scale * log2(e)
//     becomes the coefficient of the softmax FMA.
//   Softmax in the log2 domain against a per-row reference m that is not
//     reduced per tile: the weights P'' = f K 2^(s c - m) are summed (the sum
//     serves the LSE), and only when a lane's sum over a tile passes 448 (e4m3's
//     largest value; below it no single weight can overflow) is m raised to
//     5 log2 units above that tile's row maximum and the row's accumulators
//     rescaled.  The first tile of a range always raises it.
//   O^T += V8^T P''^T on the same MFMA.  The V block scale v_s = 2^e * f
//     (f in [1,2)) is split: f and the constant K = 56 go into the exponent,
//     2^e into the MFMA's E8M0 scale of P.  O_acc then collects K * sum_j
//     P~_j v_j with P~ the rounded weights.  O is normalised by the sum of the
//     same rounded weights (so O is a convex combination of the values and a
//     single key returns its value), taken by one more MFMA per tile against
//     an all-ones operand; LSE uses the sum of the unrounded weights.
//   P^T operand: the S^T accumulator gives lane (n, half) keys 32kb + 8q +
//     4*half + 0..3 in register group q of block kb; packed to e4m3 in that
//     order (4 keys per dword) it is the B operand as it stands: the V operand
//     read with ds_read_b64_tr_b8 (a 16-lane group reads 8 key rows x 16
//     channels and lane i receives channel i of the 8 rows) picks its rows so
//     that the same keys land in the same k slots.
//   Ping-pong between the two groups: a tile's work is a matrix phase (P.V of
//     the tile before, its rounded-weight sum, K Q^T of this tile: 9 MFMAs)
//     and a vector phase (the softmax of this tile).  Each SIMD holds one wave
//     of each group, and the groups run opposite phases between workgroup
//     barriers: while one wave's MFMAs occupy the matrix core, the other wave
//     issues its vector instructions.  (Run the other way -- each wave
//     alternating long matrix-only and vector-only stretches by itself -- the
//     two kinds of work barely overlapped.)
//   LDS rows hold d e4m3 bytes; chunk c of row r sits at slot c ^ h(r) (see
//   fp8_slot) so the 16-row K reads and the 8-row transpose reads are free of
//   bank conflicts.
#include "common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

template <int D>
struct FwdFp8Cfg {
    static constexpr int kWaves = 8;                      // two groups of four
    static constexpr int kGroupWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kGroupRows = 32 * kGroupWaves;   // 128: one query scale block
    static constexpr int kBr = 32 * kWaves;               // query rows per workgroup
    static constexpr int kBc = 64;                        // keys per tile
    static constexpr int kRowBytes = D;                   // one e4m3 row
    static constexpr int kChunks = D / 16;                // 16-byte chunks per row
    static constexpr int kTileBytes = kBc * kRowBytes;
    // A wave copies 1 KB (64 lanes x 16 bytes) of a tile per tensor: d = 128,
    // every wave 1 KB of K and 1 KB of V; d = 64, waves 0-3 K and 4-7 V.
    static constexpr int kCopyWaves = kTileBytes / 1024;
    static constexpr int kCopiesPerTile = kCopyWaves == kWaves ? 2 : 1;  // per wave
    static constexpr int kMB = D / 32;                    // 32-channel output blocks
    static constexpr int kKSteps = D / 64;                // MFMA k-steps of Q.K^T
    // Tile t of a range sits in ring slot t % 4 and is copied two steps ahead:
    // K(t) is read in step t, V(t) in step t + 1, so the slot it reuses (tile
    // t - 2's) was last read in step t - 1, behind that step's barriers.
    static constexpr int kRing = 4;
    static constexpr int kDist = 2;
    // The weights are P'' = f K 2^(s c - m), K = kPScale, f in [1, 2), with the
    // reference m kRefMargin log2 units above the row maximum when set (so
    // P'' <= 2 * 56 / 32 = 3.5 then); it is raised when a lane's sum of P''
    // over a tile passes kPLimit (448, the largest e4m3 value).
    static constexpr float kRefMargin = 5.0f;
    static constexpr float kPScale = 56.0f;
    static constexpr float kPLimit = 448.0f;
    static constexpr int kScaleBlock = 128;               // tokens per block scale
};

// Chunk slot of chunk c in row r: a permutation of the row's chunks chosen so
// that the 16-row K operand reads and the 8-row V transpose reads (the rows
// that the V addresses below pick) are free of bank conflicts.
template <int D>
__device__ __forceinline__ int fp8_slot(int r, int c)
{
    if constexpr (D == 128) {
        const int u = (r >> 1) & 7;
        return c ^ (((u & 1) << 1) | ((u >> 1) & 1) | (u & 4));
    } else {
        return c ^ ((r >> 2) & 3);
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

// O^T block += A B in place (A scale 1, B scale 2^(scale_b - 127)), as an asm
// statement: the compiler otherwise writes each product to fresh registers and
// keeps the old accumulator alive beside it.  The compiler does not see this as
// an MFMA, so the kernel keeps the wait states itself: the statement opens
// with two (the compiler may set up an operand, such as the scale, with a
// vector move just before it), and acc_wait comes before vector code touches
// the accumulator (tests/test_asm_hazards.py checks the generated code).
__device__ __forceinline__ void mfma_fp8_acc(f32x16& acc, const i32x8& a, const i32x8& b,
                                             int scale_b)
{
    asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                 : "+v"(acc)
                 : "v"(a), "v"(b), "v"(127), "v"(scale_b));
}

// 24 wait states before vector code touches the O accumulators that the asm
// MFMAs may still be writing (a 16-pass MFMA needs 19 after the last one).
// Tied to every block, so no vector access of one is moved above it.
template <int MB>
__device__ __forceinline__ void acc_wait(f32x16 (&acc)[MB])
{
    if constexpr (MB == 4)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
    else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc[0]), "+v"(acc[1]));
}

// D(16x16) = A(16x128 e4m3) B(128x16 e4m3), unit scales.  Operand layout per
// lane l: A row l % 16, B column l % 16, both holding k = 32 (l / 16) .. +31;
// result: lane l holds column l % 16, rows 4 (l / 16) .. +3 in its 4 registers.
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 a, i32x8 b)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4{}, 0, 0, 0, 127, 0, 127);
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

// Wait until at most N vector-memory operations of this wave are outstanding
// (the copies issued last may stay in flight).
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.)
template <int N>
__device__ __forceinline__ void wait_vmem_keep()
{
    static_assert(N >= 0 && N < 16, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | (0x7 << 4) | (0xf << 8));
}

// Copy 16 bytes per lane from buffer offset voff + soff into LDS at lds + 16 *
// lane (buffer_load_dwordx4 ... lds), as an asm statement: the compiler's
// wait-count tracking cannot tell the ring slots apart and would wait for
// copies into other slots before every read, so these copies are not made
// known to it -- the kernel waits for them itself (wait_vmem_keep and the
// barrier after it, before any read of the slot).  rsrc: the four words of a
// raw buffer descriptor, wave-uniform.  (No other instruction of this kernel
// uses M0.)
__device__ __forceinline__ void copy16_to_lds_untracked(u32x4 rsrc, uint32_t lds, uint32_t voff,
                                                        uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 ::"s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory");
}

// The four words of a raw buffer descriptor over [base, base + bytes) (what
// make_rsrc builds): an access past `bytes` reads zeros.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu)),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes), 0x00020000u};
}

// Workgroup barrier that leaves this wave's copies in flight: __syncthreads()
// would first wait for every outstanding memory operation (vmcnt(0)).  The
// wave's own LDS reads are complete before it arrives (lgkmcnt(0)).  The
// scheduling fences keep the compiler from moving any instruction across it:
// each phase's work stays in its phase.
__device__ __forceinline__ void phase_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((0xf) | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int D>
struct FwdFp8Tile {
    using Cfg = FwdFp8Cfg<D>;
    static constexpr int kBc = Cfg::kBc;
    static constexpr int kMB = Cfg::kMB;

    uint8_t* kbuf;           // K and V ring buffers (kRing slots of one tile each)
    uint8_t* vbuf;
    u32x4 k_rsrc, v_rsrc;    // buffer descriptors (SGPRs) of this (b, h)'s K and V
    uint32_t tok_bytes;
    int Skv, kt0, n_it, hh;  // tiles kt0 .. kt0 + n_it - 1 of the keys are processed
    bool copy_k, copy_v;     // the tensors this wave copies a part of
    uint32_t copy_off;       // this wave's 1 KB part of a tile (LDS byte offset)
    uint32_t ld_voff;        // this lane's source offset within a tile
    float qc;                // q_scale * scale * log2(e) of this wave's query group
    const float* ks;         // k scales of this (b, h)
    const float* vs;         // v scales of this (b, h)
    i32x8 qf[Cfg::kKSteps];
    int k_addr[Cfg::kKSteps][2];
    int v_addr[kMB];
    f32x16 oacc[kMB];
    f32x16 sacc[2];  // S^T of the tile whose softmax comes next
    i32x8 pf;        // P''^T (e4m3) of the tile whose P.V comes next
    int p_vexp;      // and the E8M0 exponent of that tile's V block scale
    float m_used;    // log2-domain reference the weights are taken against
    float l_run;     // running sum of unrounded weights over this lane's keys
    float lr_run;    // running sum of the e4m3-rounded weights over all keys
    i32x8 sel;       // e4m3 0/1 operand of the rounded-weight sums (see mfma_phase)
    f32x4 rs;        // the last P.V tile's rounded-weight sums (added at the next softmax)
    float rs_inv;    // and their 1 / (f K)

    // Copy this wave's part of key tile t (absolute index) into ring slot
    // `slot` (wave-uniform).  Rows past the last key lie outside the buffer
    // range and read as zeros (their scores are masked, so they add nothing).
    __device__ __forceinline__ void issue(int slot, int t)
    {
        const uint32_t soff = (uint32_t)(t * kBc) * tok_bytes;
        const uint32_t off = (uint32_t)slot * Cfg::kTileBytes + copy_off;
        if (copy_k)
            copy16_to_lds_untracked(k_rsrc, lds_addr(kbuf) + off, ld_voff, soff);
        if (copy_v)
            copy16_to_lds_untracked(v_rsrc, lds_addr(vbuf) + off, ld_voff, soff);
    }

    // The previous tile's rounded-weight sum into lr_run: this lane's query is
    // in register 0 (lanes with l % 32 < 16) or 1 of the sum (see mfma_phase).
    __device__ __forceinline__ void add_rs()
    {
        lr_run += ((__lane_id() & 16) ? rs[1] : rs[0]) * rs_inv;
    }

    // The weights 2^(s c - m_eff) of the tile's scores s, packed to e4m3 as
    // they are made (pw: dword q of block kb = keys 32kb + 8q + 4hh + 0..3),
    // and their sum.
    __device__ __forceinline__ float weigh_pack(uint32_t (&pw)[2][4], float c, float m_eff) const
    {
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float e[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    e[i] = exp2_fast(__builtin_fmaf(sacc[kb][4 * q + i], c, -m_eff));
                    lsum += e[i];
                }
                pw[kb][q] = pack_e4m3x4(e[0], e[1], e[2], e[3]);
            }
        return lsum;
    }

    // Matrix phase of step j (ring slot j % 4): P.V of tile j-1 (V in the slot
    // before) with its rounded-weight sum, then S^T = K Q^T of tile j.  All of
    // the phase's LDS operand reads are issued before its first MFMA, so the
    // read latency is paid once per phase rather than once per MFMA.
    __device__ __forceinline__ void mfma_phase(int j)
    {
        const bool pv = j >= 1, qk = j < n_it;
        i32x8 va[kMB];
        i32x8 ka[Cfg::kKSteps][2];
        if (pv) {
            const uint8_t* vb = vbuf + ((j + Cfg::kRing - 1) % Cfg::kRing) * Cfg::kTileBytes;
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb)
                va[mb] = tr8_read4<16 * D>(vb + v_addr[mb]);
        }
        if (qk) {
            const uint8_t* kb_ = kbuf + (j % Cfg::kRing) * Cfg::kTileBytes;
#pragma unroll
            for (int s = 0; s < Cfg::kKSteps; ++s)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const u32x4 lo = ld_lds16(kb_ + k_addr[s][0] + 32 * kb * D);
                    const u32x4 hi = ld_lds16(kb_ + k_addr[s][1] + 32 * kb * D);
                    ka[s][kb] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (pv) {
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb)
                mfma_fp8_acc(oacc[mb], va[mb], pf, p_vexp);
            // The tile's rounded-weight sums, by the 16x16x128 MFMA: read with
            // its layout, P''^T (64 keys x 32 queries, lane l: query l % 32, keys
            // 32 (l / 32) .. +31) is 128 "k" x 16 columns, k group g = l / 16
            // holding query c + 16 (g % 2) for column c.  Row r of sel takes the
            // k groups g with g % 2 == r % 2, so output row r of column c sums
            // query c + 16 (r % 2): lane l's own query lands in register 0 when
            // l % 32 < 16, else register 1.
            rs = mfma_fp8_16x16x128(sel, pf);
        }
        if (qk) {
            sacc[0] = f32x16{};
            sacc[1] = f32x16{};
#pragma unroll
            for (int s = 0; s < Cfg::kKSteps; ++s)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    sacc[kb] = mfma_fp8_32x32x64(ka[s][kb], qf[s], sacc[kb], 127);
        }
    }

    // Vector phase: the softmax of tile j (its S^T in sacc) into pf.
    __device__ __forceinline__ void valu_phase(int j)
    {
        add_rs();
        const int key0 = (kt0 + j) * kBc;
        // block scales of this key tile (uniform): both lie in block key0/128
        const int kblk = key0 / Cfg::kScaleBlock;
        const float c = qc * ks[kblk];
        const uint32_t vbits = __builtin_bit_cast(uint32_t, vs[kblk]);
        const int vexp = max((int)((vbits >> 23) & 0xff), 1);          // E8M0 exponent of v_s
        const float vmant = vs[kblk] * __builtin_bit_cast(float, (uint32_t)(254 - vexp) << 23);
        const float lift = log2_fast(vmant * Cfg::kPScale);            // log2(f * K)
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

        // P'' = P * f * K against the reference m_used, packed to e4m3 (a
        // weight past 448 packs to garbage, but then the sum passes the limit
        // and the tile is weighed again); the LSE sum takes P.
        uint32_t pw[2][4];
        float lsum = weigh_pack(pw, c, m_used - lift);
        if (__builtin_amdgcn_ballot_w64(!(lsum <= Cfg::kPLimit))) {
            // Some lane's weights may pass e4m3's range (or this is the range's
            // first tile, whose reference starts far below): raise the reference
            // to kRefMargin above the tile's row maximum, rescale what was
            // accumulated against the old one, and weigh the tile again.  A lane
            // whose reference does not move keeps alpha = 1.
            float mx = sacc[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    mx = fmaxf(mx, sacc[kb][r]);
            mx = fmaxf(mx, partner32(mx, hh));
            const float m_new = fmaxf(m_used, mx * c + Cfg::kRefMargin);
            const float alpha = exp2_fast(m_used - m_new);
            m_used = m_new;
            l_run *= alpha;
            lr_run *= alpha;
            acc_wait(oacc);  // after the last P.V MFMAs on O
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb)
                oacc[mb] *= alpha;
            lsum = weigh_pack(pw, c, m_used - lift);
        }
        const float inv_fk = __builtin_amdgcn_rcpf(vmant * Cfg::kPScale);
        l_run += lsum * inv_fk;

        // P''^T in the k order of the P.V instruction as packed: dword 4 kb + q
        // holds keys 32 kb + 8 q + 4 hh + 0..3, which the V^T reads put in the
        // same k slots (see the V addresses in the kernel)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                pf[4 * kb + q] = (int)pw[kb][q];
        p_vexp = vexp;
        rs_inv = inv_fk;
    }

    // Step j: the matrix phase of tile j, a workgroup barrier, the softmax of
    // tile j, a barrier.  Every wave runs the same steps; group 1 passes one
    // barrier before its first step and group 0 one after its last (s_barrier
    // counts arrivals, not program points), so group 1 runs one phase behind:
    // while one group's MFMAs run, the other's softmax issues.  A step first
    // copies tile j+2 into slot (j+2) % 4; after its matrix phase the wave's
    // own copies of tile j+1 have landed, so past the next barrier (the other
    // group's matrix phase of tile j+1 comes after it at the earliest) the
    // whole tile is in LDS.
    __device__ __forceinline__ void step(int j)
    {
        constexpr int kD = Cfg::kDist;
        if (j + kD < n_it)
            issue((j + kD) % Cfg::kRing, kt0 + j + kD);
        mfma_phase(j);
        if (j + kD < n_it)
            wait_vmem_keep<Cfg::kCopiesPerTile>();
        else
            wait_vmem_keep<0>();
        phase_barrier();
        if (j < n_it)
            valu_phase(j);
        phase_barrier();
        debug_sync();
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
__global__ __launch_bounds__(FwdFp8Cfg<D>::kThreads, 1) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const float* __restrict__ QS, const float* __restrict__ KS, const float* __restrict__ VS,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H, int Sq, int Skv, float scale_log2,
    int n_qtiles, int n_main, int nsplit, float* __restrict__ ws_o, float* __restrict__ ws_lse,
    float* __restrict__ ws_lr, int acc)
{
    using Cfg = FwdFp8Cfg<D>;
    constexpr int kMB = Cfg::kMB;
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds[Cfg::kRing * Cfg::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds[Cfg::kRing * Cfg::kTileBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int n = lane & 31;
    const int hh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool group1 = wave >= Cfg::kGroupWaves;

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
    st.kbuf = k_lds;
    st.vbuf = v_lds;
    st.hh = hh;
    st.Skv = Skv;
    st.kt0 = kt0;
    st.n_it = kt1 - kt0;
    st.tok_bytes = (uint32_t)tok;
    // the query group's 128 rows are exactly query scale block 2 qt + group
    // (a group wholly past Sq has no block: its rows are never stored)
    {
        const int qb = 2 * qt + (group1 ? 1 : 0);
        st.qc = qb < nqb ? QS[(long)bh * nqb + qb] * scale_log2 : 0.f;
    }
    st.ks = KS + (long)bh * nkb;
    st.vs = VS + (long)bh * nkb;
    {
        const uint8_t* Kbh = K + ((long)b * Skv * H + h) * D;
        const uint8_t* Vbh = V + ((long)b * Skv * H + h) * D;
        const int extent = (int)((uint32_t)(Skv - 1) * st.tok_bytes + D);
        st.k_rsrc = rsrc_words(Kbh, (uint32_t)extent);
        st.v_rsrc = rsrc_words(Vbh, (uint32_t)extent);
    }
    {
        // this wave's 1 KB of a tile: LDS chunks part*64 .. part*64 + 63, lane l
        // taking chunk p = part*64 + l (row p / kChunks, chunk slot p % kChunks,
        // which holds column chunk fp8_slot(row, slot))
        const int part = wave % Cfg::kCopyWaves;
        st.copy_k = Cfg::kCopyWaves == Cfg::kWaves || wave < Cfg::kCopyWaves;
        st.copy_v = Cfg::kCopyWaves == Cfg::kWaves || wave >= Cfg::kCopyWaves;
        st.copy_off = (uint32_t)part * 1024;
        const int p = part * 64 + lane;
        const int r = p / Cfg::kChunks;
        st.ld_voff = (uint32_t)r * st.tok_bytes + fp8_slot<D>(r, p % Cfg::kChunks) * 16;
    }
    // the first kDist tiles; later tiles are copied kDist steps ahead
    st.issue(0, kt0);
    if (st.n_it > 1)
        st.issue(1, kt0 + 1);

    const int q_row = qt * Cfg::kBr + wave * 32 + n;
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
    // 64s + 32hh .. +31 (two chunks).  V transpose reads, block mb: lane pair p
    // = (lane%16)/2 of lane group (hh, g2 = (lane/16)%2) reads row
    // 8(p/4) + 4hh + p%4 (+16t) at channels 32mb + 16g2 + 8(lane%2) .. +7, so
    // byte p of read t holds key 16t + 8(p/4) + 4hh + p%4: k slot 32hh + 8t +
    // p of the MFMA, the slot the S^T accumulator layout gives that key's
    // weight when packed in register order (valu_phase), so P^T needs no
    // exchange between lanes.
#pragma unroll
    for (int s = 0; s < Cfg::kKSteps; ++s)
#pragma unroll
        for (int e = 0; e < 2; ++e)
            st.k_addr[s][e] = fp8_lds_byte<D>(n, 64 * s + 32 * hh + 16 * e);
    {
        const int vp = (lane & 15) >> 1;
        const int vr = 8 * (vp >> 2) + 4 * hh + (vp & 3);
        const int vc = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
            st.v_addr[mb] = fp8_lds_byte<D>(vr, 32 * mb + vc);
    }
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
        st.oacc[mb] = f32x16{};
    // a reference far below any score: the first tile's weights overflow to
    // +inf (masked keys give exp2(-inf) = 0, never NaN), which raises it
    st.m_used = -0x1p100f;
    st.l_run = 0.f;
    st.lr_run = 0.f;
    st.rs = f32x4{};
    st.rs_inv = 0.f;
    st.p_vexp = 127;
    st.pf = i32x8{};
    // sel: A operand of the 16x16x128 sums, lane l = row l % 16 at k group
    // l / 16: e4m3 1.0 (0x38) in every byte where (l / 16) % 2 == (l % 16) % 2,
    // else 0; placed in registers once for the whole kernel
    {
        const uint32_t w = (((lane >> 4) ^ lane) & 1) == 0 ? 0x38383838u : 0u;
        st.sel = i32x8{(int)w, (int)w, (int)w, (int)w, (int)w, (int)w, (int)w, (int)w};
        asm volatile("" : "+v"(st.sel));
    }

    wait_vmem_keep<0>();
    __syncthreads();

    // steps 0 .. n_it (two phases each): step n_it holds only the last tile's P.V
    if (group1)
        phase_barrier();
    for (int j = 0; j <= st.n_it; ++j)
        st.step(j);
    if (!group1)
        phase_barrier();
    st.add_rs();
    acc_wait(st.oacc);  // after the last P.V MFMAs on O

    const float l_tot = st.l_run + partner32(st.l_run, hh);
    const float inv = 1.f / (st.lr_run * Cfg::kPScale);
    if (piece >= 0) {
        // partial result of a split tile
        const int r = wave * 32 + n;
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
    return plan_split(n_blocks, n_kt, Cfg::kBr, 1, n_cu, D + 2);
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
