// fwd_bf16.hip -- non-causal attention forward pass (O + LSE) in bf16 with
// fp32 accumulation, for gfx950 (CDNA4) MFMA: head size 64.  (Head size 128
// runs the kernel of fwd_bf16_d128.hip, built on 16x16x32 accumulate chains;
// this one is built on v_mfma_f32_32x32x16_bf16.)
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
//   Each wave owns 32 query rows of one (batch, head); a workgroup holds 4
//   waves (128 rows), and the launch bound asks for two workgroups per CU
//   (the registers and LDS leave room for a third, which the hardware
//   places).  Keys stream through LDS in tiles of 64.  Copies go
//   global -> LDS by buffer_load_dwordx4 ... lds (no VGPR staging); each
//   lane's buffer offset within a tile is fixed for the whole kernel and the
//   tile's start is a scalar offset.  Rows past the last key lie outside the
//   buffer range and read as zeros, so every LDS value stays finite.
//   Per tile and wave the matrix work is
//     S^T (keys x queries) = K Q^T on v_mfma_f32_32x32x16_bf16: A = K rows from
//       LDS, B = Q^T held in registers for the whole kernel.  The transpose
//       puts one query per lane column, so a row maximum or sum is a per-lane
//       reduction plus one exchange with lane l^32 (v_permlane32_swap).
//     O^T (channels x queries) += V^T P^T: A = V^T read from the V tile with
//       ds_read_b64_tr_b16 (LDS transpose read), B = P^T straight from the S^T
//       accumulator registers.  A and B use the same assignment of keys
//       to k slots, so no register shuffle is needed.
//   Software pipeline: iteration j runs the P V product of tile j-1, the K Q^T
//   product of tile j+1 and the softmax of tile j.  The three are independent,
//   so the 16 matrix instructions of an iteration interleave the two
//   products (per 16-key step: its P V instructions, then as many K Q^T ones),
//   and the softmax's vector instructions are spread over the same slots: the
//   vector ALU works in the shadow of the matrix core instead of after it.
//   The slots are fenced (sched_barrier) so the compiler keeps that order.
//   LDS operands are read several slots ahead: V^T fragments one 16-key step
//   ahead, K operands kMB slots ahead (the last group's during the group
//   before), and the first V^T fragments of iteration j+1 during the last
//   group of iteration j, so that no iteration starts by waiting on LDS.
//   Softmax in the log2 domain: scale*log2(e) is folded into one FMA before
//   v_exp_f32.  The weights of a whole pass over the keys are taken against one
//   reference maximum (the first tile's row maximum): the final O / sum and LSE
//   are exact for any reference as long as no weight overflows, so no tile is
//   reduced to its maximum and O is never rescaled.  Should a later score rise
//   so far above the reference that a lane's weight sum for a tile passes
//   2^32, the workgroup computes the exact row maxima of its key range and
//   makes the pass again (see the kernel).
//   LDS: a ring of K and V tile buffers (two slots each; with two or three
//   workgroups per CU a deeper ring was slower), each its own LDS object.  Iteration j reads K(j+1), V(j-1) from
//   slot j while the copies of the tiles that iteration j + kRing/2 reads go
//   into slot j + kRing/2, last read by iteration j - kRing/2: one barrier
//   per kRing/2 iterations.  It sits before the last group of K Q^T
//   instructions (whose operands are in registers by then), once all LDS
//   reads of the iteration are done, so the next iteration's first reads
//   overlap those matrix instructions.  (Separate objects also let the
//   compiler see that the transpose reads never alias an outstanding copy.)
//   K tile layout: rows of D bf16; the 16-byte chunk c of row r sits at chunk
//   slot c ^ f(r), where f permutes bits of r so that the K operand read (16
//   rows x one chunk) covers all 64 banks.  V tile layout: D/32 blocks of 32
//   channels, each 64 keys x 64 bytes, so a transpose read (4 keys x 64 bytes
//   per half-wave) covers all 64 banks with no swizzle, and every V read is one
//   per-lane register plus a constant.  Every LDS address is a per-lane base
//   (computed once) plus a compile-time offset.
//   Tails: query rows >= Sq are computed on zero queries and never stored;
//   keys >= Skv get score -inf.
#include "common.hpp"
#include "launch.hpp"


namespace dit {
namespace {

template <int D>
struct FwdBf16Cfg {
    static_assert(D == 64, "head size 128 runs fwd_bf16_d128.hip");
    static constexpr int kWaves = 4;
    static constexpr int kWgPerCu = 2;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBr = 32 * kWaves;                // query rows per workgroup
    static constexpr int kBc = 64;                         // keys per tile
    static constexpr int kChunks = D / 8;                  // 16-byte chunks per key row
    static constexpr int kRowBytes = D * 2;
    static constexpr int kTileBytes = kBc * kRowBytes;     // one K or V tile
    static constexpr int kLoads = kTileBytes / (16 * kThreads);  // 16-B loads per thread
    static constexpr int kLoadRows = 16 * kThreads / kRowBytes;   // rows one copy covers
    static constexpr int kMB = D / 32;                     // 32-channel output blocks
    static constexpr int kVBlockBytes = kBc * 64;          // V tile: one 32-channel block
    static constexpr int kRing = 2;                        // K and V tile buffers each
    // Bound on one lane's sum of weights of one tile (32 weights), which keeps
    // every weight <= 2^32: O and the sums cannot overflow for |V| < 2^80.
    static constexpr float kWeightSumLimit = 0x1p32f;
};

// Chunk slot of chunk c in row r (see the layout note above).
template <int D>
__device__ __forceinline__ int swz_slot(int r, int c)
{
    const int u = (r >> 1) & 7;
    return c ^ (((u & 1) << 2) | (u >> 1));
}

template <int D>
__device__ __forceinline__ int lds_byte(int r, int col)
{
    return r * (D * 2) + swz_slot<D>(r, col >> 3) * 16 + (col & 7) * 2;
}

// Keep a vector-ALU result where it is computed: an empty asm that reads and
// rewrites it.  Without this the compiler sinks softmax work that feeds only
// the next iteration into that iteration, past the branches at its start, or
// hoists it into an earlier slot.  (Only vector-ALU results are pinned.)
__device__ __forceinline__ void pin(float& x)
{
    asm volatile("" : "+v"(x));
}

__device__ __forceinline__ void pin(uint32_t& x)
{
    asm volatile("" : "+v"(x));
}

__device__ __forceinline__ void pin(u32x4& x)
{
    asm volatile("" : "+v"(x));
}

// The matrix instructions of the tile loop are asm statements: then their
// order against the slot fences is fixed (compiler-generated MFMAs have no such
// ordering and get moved), O stays in accumulation registers (AGPRs) and the
// S^T accumulators, which the softmax reads, in VGPRs.  The compiler does not
// see these as MFMAs, so the kernel keeps the wait states itself: vector code
// reads an S^T block at least two matrix instructions after its last step,
// and touches O only after acc_wait (tests/test_asm_hazards.py checks the
// generated code).
//   O^T block += A B, accumulator in AGPRs.
__device__ __forceinline__ void mfma_o(f32x16& acc, u32x4 a, u32x4 b)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

//   S^T block = A B (first k step) or += A B, accumulator in VGPRs, B (Q^T,
//   loop-invariant) in AGPRs.
__device__ __forceinline__ void mfma_s0(f32x16& acc, u32x4 a, const u32x4& b)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "a"(b));
}

__device__ __forceinline__ void mfma_s(f32x16& acc, u32x4 a, const u32x4& b)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}

// Wait states before vector code touches an O block after the asm MFMAs on it
// (and before the next MFMA after vector code wrote it): 8 per block, the
// blocks waited for one after another (an 8-pass MFMA needs at most 18).
__device__ __forceinline__ void acc_wait(f32x16& acc)
{
    asm volatile("s_nop 7" : "+a"(acc));
}

// 24 wait states before vector code writes an S^T block an MFMA may still be
// producing.
__device__ __forceinline__ void vgpr_wait(f32x16& acc)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}

// Per-thread state of one workgroup's pass over the keys.
template <int D>
struct FwdBf16Tile {
    using Cfg = FwdBf16Cfg<D>;
    static constexpr int kBc = Cfg::kBc;
    static constexpr int kRow = Cfg::kRowBytes;
    static constexpr int kMB = Cfg::kMB;
    static constexpr int kSteps = D / 16;          // k steps of K Q^T
    static constexpr int kSlots = D / 4;           // matrix instructions per iteration
    static constexpr int kVReads = 2 * kMB;        // V^T transpose reads per 16-key step
    static constexpr int kPer = kSlots / 8;        // slots per group of 4 scores
    static constexpr int kHalf = Cfg::kRing / 2;   // iterations per barrier

    // K and V tile buffers (ring slots 0 .. kRing-1), each its own LDS object.
    uint8_t* kobj[Cfg::kRing];
    uint8_t* vobj[Cfg::kRing];
    __amdgpu_buffer_rsrc_t k_rsrc, v_rsrc;
    uint32_t tok_bytes;
    int key_end, wave, hh;   // keys >= key_end are masked (the end of this block's range)
    float scale_log2;
    uint32_t k_voff;         // this lane's source offset in K copy 0 (copy i: + i * kLoadRows rows)
    uint32_t v_voff;         // this lane's source offset in V copy 0 (copy i: + kWaves/4 blocks)
    u32x4 qf[kSteps];        // bf16 operands are carried as raw 32-bit words
    int k_addr[kSteps / 2];  // LDS address in K slot 0; steps s and s + kSteps/2 differ in one bit
    uint32_t v_reg;          // LDS address of this lane's V transpose reads in V slot 0
    f32x16 oacc[kMB];
    f32x16 sacc[2][2];       // [parity][32-key block]: S^T of a tile
    u32x4 pf[2][4];          // [parity][16-key step]: P^T of a tile
    u32x2 vf[kVReads];       // V^T fragments of one 16-key step
    u32x4 kf[kMB];           // K fragments of one group of K Q^T slots
    uint32_t pw[2];          // bf16 pairs of the even group of a 16-key step
    float lsum;              // sum of this lane's weights of the current tile
    float lsum_max;          // largest lsum of the pass (checked against kWeightSumLimit)
    float m_used;  // reference maximum (scale*log2(e) units) of the weights, fixed per pass
    float l_run;   // running sum over this lane's half of the keys

    // Copy tile kt of K (to K ring slot KB) and/or of V (to V slot VB) into LDS;
    // a negative buffer index skips that tensor.  Rows past the last key lie
    // outside the buffer range and read as zeros.
    __device__ __forceinline__ uint8_t* kbuf(int R) const
    {
        return kobj[R];
    }
    __device__ __forceinline__ uint8_t* vbuf(int R) const
    {
        return vobj[R];
    }

    template <int KB, int VB>
    __device__ __forceinline__ void copy_tile(int kt)
    {
        const uint32_t soff = (uint32_t)(kt * kBc) * tok_bytes;
#pragma unroll
        for (int i = 0; i < Cfg::kLoads; ++i) {
            const int off = (i * Cfg::kWaves + wave) * 1024;
            if constexpr (KB >= 0)
                copy16_to_lds(k_rsrc, kbuf(KB) + off, k_voff,
                              soff + (uint32_t)(i * Cfg::kLoadRows) * tok_bytes);
            if constexpr (VB >= 0)
                copy16_to_lds(v_rsrc, vbuf(VB) + off, v_voff, soff + i * (Cfg::kWaves / 4) * 64);
        }
    }

    // LDS address of the K operand of k step s in K slot 0 (see k_addr).
    __device__ __forceinline__ int k_off(int s) const
    {
        return s < kSteps / 2 ? k_addr[s] : (k_addr[s - kSteps / 2] ^ (16 * kSteps));
    }

    // K operand of k step s, 32-key block kb, from K ring slot KB: the per-lane
    // address in slot 0 plus a constant (the slot's distance from slot 0 folds
    // into the instruction's offset field).
    template <int KB>
    __device__ __forceinline__ u32x4 ld_k(int s, int kb) const
    {
        return ld_lds16(kobj[KB] + (k_off(s) - (int)lds_addr(kobj[0]) + 32 * kb * kRow));
    }

    // K operand of K Q^T step q (k step q/2, 32-key block q%2) from K ring slot KB.
    template <int KB, int Q>
    __device__ __forceinline__ void read_k()
    {
        kf[Q % kMB] = ld_k<KB>(Q / 2, Q % 2);
    }

    // Transpose read E (block E/2, half E%2) of 16-key step T from V slot VB:
    // this lane's address in V slot 0 plus a constant, written so that the
    // constant (the slot's distance from slot 0, the block, the keys) folds
    // into the instruction's offset field.  (The fold needs the subtraction in
    // the same basic block as the read: iteration() re-pins v_reg after its
    // branch.)
    template <int VB>
    __device__ __forceinline__ u32x2 ld_v(int T, int E) const
    {
        const int c = (E / 2) * Cfg::kVBlockBytes + (16 * T + 8 * (E % 2)) * 64;
        return ld_lds_tr16(vobj[VB] + ((int)v_reg - (int)lds_addr(vobj[0]) + c));
    }

    template <int VB, int T, int E>
    __device__ __forceinline__ void read_v()
    {
        vf[E] = ld_v<VB>(T, E);
    }

    // The full S^T of one tile from K slot KB into sacc[SP] (prologue only).
    template <int KB, int SP>
    __device__ __forceinline__ void qk_tile()
    {
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const u32x4 a = ld_k<KB>(s, kb);
                if (s == 0)
                    mfma_s0(sacc[SP][kb], a, qf[s]);
                else
                    mfma_s(sacc[SP][kb], a, qf[s]);
            }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            vgpr_wait(sacc[SP][kb]);
    }

    // Softmax of the tile in sacc[P], vector work of slot I.  The weights are
    // 2^(scale*log2(e)*s - m_used) with m_used fixed for the whole pass (see
    // the kernel), so a tile needs no maximum of its own.  Score w is register
    // w%16 of 32-key block w/16; slot I computes weights kW*I .. kW*I + kW-1
    // in place (block 1's from slot 16/kW >= 8 on, well after its last K Q^T
    // step).  Their sum and bf16 pairs come per group of 4 weights, in the
    // group's last slot.
    static constexpr int kW = 32 / kSlots;  // weights per slot

    template <int P, int I>
    __device__ __forceinline__ void softmax_part()
    {
        // re-pinned each slot, so that this slot's weights cannot be hoisted
        // into an earlier one
        pin(m_used);
#pragma unroll
        for (int w = kW * I; w < kW * (I + 1); ++w) {
            float e = exp2_fast(__builtin_fmaf(sacc[P][w / 16][w % 16], scale_log2, -m_used));
            pin(e);
            sacc[P][w / 16][w % 16] = e;
        }
        if constexpr ((kW * (I + 1)) % 4 == 0) {
            // group of weights w0 .. w0+3 complete: its sum, and its two bf16
            // pairs (words 2(G%2), 2(G%2)+1 of the P^T fragment of step t)
            constexpr int w0 = kW * (I + 1) - 4, G = w0 / 4, kb = w0 / 16, r0 = w0 % 16;
            const f32x16& s = sacc[P][kb];
            const float g = (s[r0] + s[r0 + 1]) + (s[r0 + 2] + s[r0 + 3]);
            lsum = G == 0 ? g : lsum + g;
            pin(lsum);
            constexpr int t = w0 / 8;
            if constexpr (G % 2 == 0) {
                pw[0] = pack_bf16x2(s[r0], s[r0 + 1]);
                pw[1] = pack_bf16x2(s[r0 + 2], s[r0 + 3]);
                pin(pw[0]);
                pin(pw[1]);
            } else {
                u32x4 v = {pw[0], pw[1], pack_bf16x2(s[r0], s[r0 + 1]),
                           pack_bf16x2(s[r0 + 2], s[r0 + 3])};
                pin(v);
                pf[P][t] = v;
            }
        }
    }

    // Scores of keys >= key_end in the tile at key0 (in sacc[SP]) -> -inf.
    template <int SP>
    __device__ __forceinline__ void mask_tile(int key0)
    {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            vgpr_wait(sacc[SP][kb]);  // the last K Q^T steps may still run
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = key0 + 32 * kb + 8 * (r / 4) + 4 * hh + (r % 4);
                if (key >= key_end)
                    sacc[SP][kb][r] = -INFINITY;
            }
    }

    // Row maximum (scale*log2(e) units, both lane halves) of the tile in sacc[SP].
    template <int SP>
    __device__ __forceinline__ float tile_max() const
    {
        float m = sacc[SP][0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                m = fmaxf(m, sacc[SP][kb][r]);
        return fmaxf(m, partner32(m, hh)) * scale_log2;
    }

    // One step of the maximum pass: S^T of the tile kt from K slot KB (its
    // copy waited for), the copy of K(kt+1) into slot KB + kRing/2 started.
    template <int KB>
    __device__ __forceinline__ void max_step(int kt, float& m)
    {
        copy_tile<(KB + Cfg::kRing / 2) % Cfg::kRing, -1>(kt + 1);
        qk_tile<KB, 0>();
        const int key0 = kt * kBc;
        if (key0 + kBc > key_end)
            mask_tile<0>(key0);
        m = fmaxf(m, tile_max<0>());
        wait_vmem_all();
        __syncthreads();
    }

    // Slot I of the iteration that reads ring slot R (parity P = R % 2): one
    // matrix instruction, the LDS reads for later slots, and a share of the
    // softmax.  Slots come in groups of 2 kMB, one per 16-key step t of the
    // previous tile:
    //   first kMB: O^T += V^T P^T of step t, block mb (P^T of the previous
    //              tile, V from slot R), all with the same B operand;
    //   last kMB:  S^T += K Q^T for the next tile (K from slot R), K Q^T
    //              instructions kMB t .. kMB t + kMB-1 (k step q/2, 32-key
    //              block q%2), pairs with the same B operand.
    // (Grouping instructions that share an operand was +3.5% against
    // alternating the two products.)
    template <int R, int I>
    __device__ __forceinline__ void slot()
    {
        constexpr int P = R % 2;
        constexpr int t = I / (2 * kMB), i = I % (2 * kMB);
        if constexpr (I == kSlots - kMB) {
            // The group's barrier: every wave's copies so far have landed (so
            // the slots of the next kHalf iterations hold their tiles) and
            // every wave has finished its reads of this group's slots (the
            // last ones were issued in the group before, and the barrier
            // waits for them), which later copies overwrite.  Then step 0 of
            // the next iteration's V^T fragments.
            if constexpr (R % kHalf == kHalf - 1) {
                wait_vmem_all();
                __syncthreads();
            }
#pragma unroll
            for (int e = 0; e < kVReads; ++e)
                vf[e] = ld_v<(R + 1) % Cfg::kRing>(0, e);
        }
        if constexpr (i < kMB) {
            constexpr int mb = i;
            mfma_o(oacc[mb], u32x4{vf[2 * mb][0], vf[2 * mb][1], vf[2 * mb + 1][0], vf[2 * mb + 1][1]},
                   pf[P ^ 1][t]);
            // K operand of this group's K Q^T instruction i, kMB slots ahead
            // (last group: read in the group before)
            if constexpr (t < 3)
                read_k<R, kMB * t + i>();
            if constexpr (t == 3 && i == 0)
                read_k<R, kMB * 3 + kMB - 1>();
        } else {
            constexpr int v = kMB * t + i - kMB, s = v / 2, kb = v % 2;
            if constexpr (s == 0)
                mfma_s0(sacc[P ^ 1][kb], kf[v % kMB], qf[s]);
            else
                mfma_s(sacc[P ^ 1][kb], kf[v % kMB], qf[s]);
            // K operands of the last group, one slot after their registers'
            // last use
            if constexpr (t == 2 && i > kMB)
                read_k<R, kMB * 3 + (i - kMB - 1)>();
        }
        // V^T fragments 2mb, 2mb+1 of step t+1, one slot after step t's block
        // mb consumed them
        if constexpr (i >= 1 && i <= kMB && t + 1 < 4) {
            constexpr int mb = i - 1;
            read_v<R, t + 1, 2 * mb>();
            read_v<R, t + 1, 2 * mb + 1>();
        }
        softmax_part<P, I>();
        __builtin_amdgcn_sched_barrier(0);
    }

    template <int R, int I>
    __device__ __forceinline__ void slots()
    {
        if constexpr (I < kSlots) {
            slot<R, I>();
            slots<R, I + 1>();
        }
    }

    // The P V product of the last tile alone (after an even number of
    // iterations: P^T in pf[1], V in ring slot 0, which vb is).
    __device__ __forceinline__ void drain(const uint8_t* vb)
    {
        constexpr int P = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int e = 0; e < kVReads; ++e)
                vf[e] = ld_lds_tr16(vb + ((int)v_reg - (int)lds_addr(vobj[0]) + (e / 2) * Cfg::kVBlockBytes +
                                          (16 * t + 8 * (e % 2)) * 64));
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb)
                mfma_o(oacc[mb], u32x4{vf[2 * mb][0], vf[2 * mb][1], vf[2 * mb + 1][0], vf[2 * mb + 1][1]},
                       pf[P ^ 1][t]);
        }
    }

    // Iteration kt, reading ring slot R (kt - first tile = R mod kRing): P V
    // of tile kt-1 (V there), K Q^T of tile kt+1 (K there), softmax of tile
    // kt; copies V(kt + kHalf-1), K(kt + kHalf+1) into ring slot R + kHalf,
    // which iteration kt - kHalf read last.  Every kHalf-th iteration waits
    // for the copies and holds the one barrier of its group (in the slot
    // program, see slot()).  On entry vf holds step 0 of this iteration's V^T
    // fragments, read by the iteration before (or before the first one).
    template <int R>
    __device__ __forceinline__ void iteration(int kt)
    {
        constexpr int P = R % 2;
        constexpr int W = (R + kHalf) % Cfg::kRing;
        copy_tile<-1, W>(kt + kHalf - 1);
        copy_tile<W, -1>(kt + kHalf + 1);
        const int key0 = kt * kBc;
        if (key0 + kBc > key_end)
            mask_tile<P>(key0);
        // re-pinned here, in the block of all of this iteration's V reads:
        // then its distance from slot R folds into their offset fields
        pin(v_reg);
        __builtin_amdgcn_sched_barrier(0);
        slots<R, 0>();
        l_run += lsum;
        lsum_max = fmaxf(lsum_max, lsum);
        debug_sync();
    }
};

// Grid: blocks [0, n_main) each take one query tile over all keys; the
// remaining query tiles (the last, partial wave of workgroups a plain launch
// would end with) are each split into nsplit pieces over contiguous ranges of
// key tiles, so they fill the machine instead of leaving most of it idle.  A
// piece writes its normalised fp32 partial O and its LSE to the workspace
// (ws_o [piece][kBr][D], ws_lse [piece][kBr]); launch_split_merge (split.hip)
// combines them with the log-sum-exp merge.
template <int D>
__global__ __launch_bounds__(FwdBf16Cfg<D>::kThreads, FwdBf16Cfg<D>::kWgPerCu) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int H, int Sq, int Skv, float scale_log2, int n_qtiles, int n_main, int nsplit,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, int acc, long kv_bstride)
{
    using Cfg = FwdBf16Cfg<D>;
    constexpr int kMB = Cfg::kMB;
    constexpr int kRow = Cfg::kRowBytes;
    constexpr int kRing = Cfg::kRing;
    constexpr int kHalf = kRing / 2;
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[Cfg::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[Cfg::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[Cfg::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[Cfg::kTileBytes];
    __shared__ int wave_over[Cfg::kWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int n = lane & 31;   // query column of this lane within the wave
    const int hh = lane >> 5;  // which 8-wide k group this lane feeds

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
    const long tok = (long)H * D;  // elements between consecutive tokens

    FwdBf16Tile<D> st;
    st.kobj[0] = k_lds0;
    st.kobj[1] = k_lds1;
    st.vobj[0] = v_lds0;
    st.vobj[1] = v_lds1;
    st.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    st.hh = hh;
    st.key_end = min(kt1 * Cfg::kBc, Skv);
    st.scale_log2 = scale_log2;
    st.tok_bytes = (uint32_t)(tok * 2);
    {
        // batches of K and V lie kv_bstride tokens apart (Skv when contiguous)
        const uint16_t* Kbh = K + ((long)b * kv_bstride * H + h) * D;
        const uint16_t* Vbh = V + ((long)b * kv_bstride * H + h) * D;
        // Byte extent of this (b, h)'s keys: rows 0 .. Skv-1 (callers guarantee < 2^32).
        const int extent = (int)((uint32_t)(Skv - 1) * st.tok_bytes + kRow);
        st.k_rsrc = make_rsrc(Kbh, extent);
        st.v_rsrc = make_rsrc(Vbh, extent);
    }
    // Copy i of wave w fills LDS chunks [(i*kWaves + w)*64, +64) of a tile; lane
    // l takes chunk p = that base + l.
    //   K (row-major, swizzled): row p / kChunks at slot p % kChunks, which holds
    //   column chunk (p % kChunks) ^ f(row).  Copy i covers rows i * kLoadRows
    //   more than copy 0 and, as f() depends only on row bits that the copy
    //   index does not change, the same chunk slots.
    //   V (32-channel blocks of 64 keys x 64 bytes): block p / 256, key
    //   (p / 4) % 64, 16-byte column chunk p % 4 of the block.  Copy i is
    //   kWaves/4 blocks further on.
    {
        const int p = st.wave * 64 + lane;
        const int r = p / Cfg::kChunks;
        st.k_voff = (uint32_t)r * st.tok_bytes + swz_slot<D>(r, p % Cfg::kChunks) * 16;
        st.v_voff = (uint32_t)((p / 4) % 64) * st.tok_bytes + ((p / 256) * 4 + p % 4) * 16;
    }
    // A pass starts with what its first kHalf iterations read: K(kt0) in the
    // last ring slot (the prologue's K Q^T), K(kt0+1) .. K(kt0+kHalf) in
    // slots 0 .. kHalf-1, and V(kt0) in slot 0, where the first iteration's
    // P V (with P = 0) reads finite values.  (The first pass's copies overlap
    // the Q loads.)
    auto pass_copies = [&]() {
        st.template copy_tile<kRing - 1, -1>(kt0);
        st.template copy_tile<0, -1>(kt0 + 1);
        st.template copy_tile<-1, 0>(kt0);
    };
    pass_copies();

    const int q_row = qt * Cfg::kBr + st.wave * 32 + n;
    if (q_row < Sq) {
        const uint16_t* src = Q + ((long)b * Sq * H + h) * D + (long)q_row * tok + 8 * hh;
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            st.qf[s] = ld_global16(src + 16 * s);
    } else {
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            st.qf[s] = u32x4{0, 0, 0, 0};
    }

    // Q^T lives in accumulation registers for the whole kernel (the K Q^T asm
    // takes B from there); moving it once here keeps the compiler from copying
    // it over before every matrix instruction.
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
        asm volatile("" : "+a"(st.qf[s]));

    // Per-lane LDS bases.  K operand (A of S^T), step s: row n (+32 for the
    // second block), column 16s + 8hh.  V transpose reads, block mb, half hi:
    // lane group g = lane/16 reads key 4hh + 8hi + (lane%16)/4 (+16t) of block
    // mb at channels 16(g%2) + 4(lane%4) .. +3, so lane l receives channel
    // 32mb + l%32 of keys 16t + 8hi + 4hh + 0..3.  (The 32 lanes of one
    // half-wave cover 4 keys x 64 contiguous bytes: all 64 banks once.)
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
        st.k_addr[s] = lds_addr(k_lds0) + lds_byte<D>(n, 16 * s + 8 * hh);
    st.v_reg = lds_addr(v_lds0) + (4 * hh + ((lane & 15) >> 2)) * 64 +
               (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
    pin(st.v_reg);
    // Passes over the key range.  The weights of a pass are taken against one
    // reference maximum m_used: O / sum and LSE are exact for any reference
    // as long as no weight overflows, so no tile needs a maximum of its own and
    // O is never rescaled.  The first pass takes the first tile's row maximum.
    // If a later score rises so far above it that some lane's weights for a
    // tile sum past kWeightSumLimit, the workgroup finds the exact row maxima
    // of the range (a K Q^T-only pass) and makes a second pass against them,
    // in which no weight exceeds 1.
    for (int pass = 0;; ++pass) {
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
            st.oacc[mb] = f32x16{};
            acc_wait(st.oacc[mb]);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
            st.pf[1][t] = u32x4{0, 0, 0, 0};
        st.l_run = 0.f;
        st.lsum_max = 0.f;

        wait_vmem_all();
        __syncthreads();
        st.template qk_tile<kRing - 1, 0>();
        if (pass == 0) {
            if (kt0 * Cfg::kBc + Cfg::kBc > st.key_end)
                st.template mask_tile<0>(kt0 * Cfg::kBc);
            st.m_used = st.template tile_max<0>();
        }
        __syncthreads();  // the last ring slot is refilled by iteration kHalf-1
        // step 0 of the first iteration's V^T fragments (later iterations read
        // theirs in the iteration before)
#pragma unroll
        for (int e = 0; e < 2 * kMB; ++e)
            st.vf[e] = st.template ld_v<0>(0, e);

        // One iteration per tile of the range, unrolled over the ring slots
        // (the slot indices are compile-time), then the last tile's P V: by
        // one more iteration if the count is odd (its own tile lies past the
        // range: all keys masked, weights 0), else by drain().
        const int n_it = kt1 - kt0;
        const int n_pad = (n_it + 1) & ~1;
        int i = 0;
        for (; i < n_pad; i += 2) {
            st.template iteration<0>(kt0 + i);
            st.template iteration<1>(kt0 + i + 1);
        }
        // the last iteration's K Q^T result (of a tile past the range) is
        // dead: hold its registers until that matrix instruction is done
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            vgpr_wait(st.sacc[0][kb]);
        if (i == n_it)
            st.drain(st.vobj[0]);

        if (lane == 0)
            wave_over[st.wave] = __builtin_amdgcn_ballot_w64(st.lsum_max > Cfg::kWeightSumLimit) != 0;
        __syncthreads();
        int over = 0;
#pragma unroll
        for (int w = 0; w < Cfg::kWaves; ++w)
            over |= wave_over[w];
        if (!over || pass > 0)
            break;

        // exact row maxima of the range, then the second pass
        float m = -INFINITY;
        st.template copy_tile<0, -1>(kt0);
        wait_vmem_all();
        __syncthreads();
        const int n_mx = (kt1 - kt0 + 1) & ~1;
        for (int i = 0; i < n_mx; i += 2) {
            st.template max_step<0>(kt0 + i, m);
            st.template max_step<kHalf>(kt0 + i + 1, m);
        }
        st.m_used = m;
        pass_copies();
    }
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
        acc_wait(st.oacc[mb]);

    const float l_tot = st.l_run + partner32(st.l_run, hh);
    const float inv_l = 1.f / l_tot;
    if (piece >= 0) {
        // partial result of a split tile: normalised fp32 O and LSE (natural log)
        const int r = st.wave * 32 + n;
        float* dst = ws_o + ((long)piece * Cfg::kBr + r) * D + 4 * hh;
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 w = {st.oacc[mb][4 * g + 0] * inv_l, st.oacc[mb][4 * g + 1] * inv_l,
                           st.oacc[mb][4 * g + 2] * inv_l, st.oacc[mb][4 * g + 3] * inv_l};
                *reinterpret_cast<f32x4*>(dst + 32 * mb + 8 * g) = w;
            }
        if (hh == 0)
            ws_lse[(long)piece * Cfg::kBr + r] = (st.m_used + log2_fast(l_tot)) * kLn2;
    } else if (q_row < Sq) {
        uint16_t* dst = O + ((long)b * Sq * H + h) * D + (long)q_row * tok + 4 * hh;
        float* lse_dst = LSE + ((long)b * H + h) * Sq + q_row;
        const float lse_new = (st.m_used + log2_fast(l_tot)) * kLn2;
        // O = c_new * acc + c_old * O_old; without a running result (acc = 0, or
        // its LSE is -inf) that is the plain normalisation
        float c_new = inv_l, c_old = 0.f, lse_out = lse_new;
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
    using Cfg = FwdBf16Cfg<D>;
    const long n_blocks = (long)((Sq + Cfg::kBr - 1) / Cfg::kBr) * H * B;
    const long n_kt = (Skv + Cfg::kBc - 1) / Cfg::kBc;
    return plan_split(n_blocks, n_kt, Cfg::kBr, Cfg::kWgPerCu, n_cu, D + 1);
}

template <int D>
hipError_t launch_fwd_bf16_d(const FwdArgs& a, const FwdSplit& sp, hipStream_t stream)
{
    using Cfg = FwdBf16Cfg<D>;
    const int n_qtiles = (a.Sq + Cfg::kBr - 1) / Cfg::kBr;
    const long n_blocks = (long)n_qtiles * a.H * a.B;
    if (n_blocks > 0x7fffffffL)
        return hipErrorInvalidConfiguration;
    const float scale_log2 = a.scale * kLog2e;
    const bool split = sp.n_tail > 0;
    float* ws_o = split ? static_cast<float*>(a.ws) : nullptr;
    float* ws_lse = split ? ws_o + (size_t)sp.n_tail * sp.nsplit * Cfg::kBr * D : nullptr;
    const long grid = split ? (long)sp.n_main + (long)sp.n_tail * sp.nsplit : n_blocks;
    hipError_t e = launch_kernel(fwd_bf16_kernel<D>, dim3((unsigned)grid), dim3(Cfg::kThreads),
                                 stream, a.q, a.k, a.v, a.o, a.lse, a.H, a.Sq, a.Skv, scale_log2,
                                 n_qtiles, split ? sp.n_main : (int)n_blocks,
                                 split ? sp.nsplit : 1, ws_o, ws_lse, a.acc,
                                 a.kv_batch_tokens > 0 ? a.kv_batch_tokens : (long)a.Skv);
    if (e != hipSuccess || !split)
        return e;
    return launch_split_merge(a, sp, Cfg::kBr, n_qtiles, ws_o, ws_lse, nullptr, stream);
}

}  // namespace

FwdSplit plan_fwd_bf16_split(int B, int H, int Sq, int Skv, int d, int n_cu)
{
    return d == 64 ? plan_d<64>(B, H, Sq, Skv, n_cu) : plan_fwd_bf16_d128_split(B, H, Sq, Skv, n_cu);
}

hipError_t launch_fwd_bf16(const FwdArgs& a, const FwdSplit& split, hipStream_t stream)
{
    return a.d == 64 ? launch_fwd_bf16_d<64>(a, split, stream)
                     : launch_fwd_bf16_d128(a, split, stream);
}

}  // namespace dit
