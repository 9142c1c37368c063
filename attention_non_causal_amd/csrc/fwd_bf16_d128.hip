// fwd_bf16_d128.hip -- non-causal attention forward pass (O + LSE) in bf16 with
// fp32 accumulation for head size 128, for gfx950 (CDNA4) MFMA.
//
// What is computed: per (batch, head), O = softmax(scale * Q K^T) V and
// LSE = ln sum_j exp(scale * q . k_j) -- the whole-sequence, cache-free
// attention of DiT inference ("xDiT 项目概述", sec. 2.1), done by a dedicated
// kernel as "生成AI推論を速くするための設計ノート" sec. 5 recommends for an
// attention that dominates.  One pass over key tiles with one reference
// maximum per pass (online softmax); the exact result up to fp32 rounding.
//
// This kernel is built around v_mfma_f32_16x16x32_bf16 accumulate chains.  At
// the clock its power limit allows, the chip sustains more dense bf16 work
// with this 16x16 instruction than with the 32x32x16 one, and the most when
// an instruction accumulates onto the result of the one just before it (the
// accumulator is then forwarded inside the matrix core instead of making a
// round trip through the register file): both products are therefore issued
// as chains of instructions on one accumulator.
//
// Work decomposition
//   A workgroup of 8 waves (256 query rows, 32 per wave), one per CU; keys
//   stream through LDS in tiles of 64.  Per wave and tile:
//     S^T (keys x queries) = K Q^T: 16x16 blocks (key block kb = 0..3, query
//       block qb = 0..1), each one chain of 4 instructions over the channels
//       (32 per step): A = K rows from LDS, B = Q^T held in accumulation
//       registers for the whole kernel.  Lane l holds query 16qb + l%16 and
//       keys 16kb + 4(l/16) + 0..3 of a block.
//     O^T (channels x queries) += V^T P^T: 16x16 blocks (channel block cb =
//       0..7, qb), each a chain of 2 instructions over the tile's keys (32 per
//       step).  B = P^T packed straight from the S^T accumulators: for key
//       step t, lane l's 8 k slots 8g .. 8g+7 (g = l/16) hold keys 32t + 4g +
//       0..3 and 32t + 16 + 4g + 0..3 -- its own S^T values of blocks 2t and
//       2t+1.  A = V^T from two LDS transpose reads (ds_read_b64_tr_b16) that
//       fetch exactly those keys for the lane's channel.
//   Software pipeline: iteration j runs P V of tile j-1, K Q^T of tile j+1 and
//   the softmax of tile j, which are independent.  Its 32 slots alternate a
//   P V chain (channel block cb, one query block) and half a K Q^T chain (two
//   channel steps), each with one weight of the softmax and a share of the
//   LDS reads for slots four or eight ahead; fences keep the order.  (The
//   vector work comes in small shares between the matrix instructions so that
//   one wave's instructions overlap its own matrix work; chains of two keep
//   most of the power advantage of longer ones.)
//   Softmax in the log2 domain with one reference maximum per pass (the first
//   tile's row maximum): O / sum and LSE are exact for any reference as long as
//   no weight overflows.  Should a later score rise so far that a lane's
//   weight sum for a tile passes 2^32, the workgroup computes the exact row
//   maxima of its key range and makes the pass again.
//   LDS: a ring of four K and four V tile buffers; iteration j reads K(j+1)
//   and V(j-1) from slot j mod 4 and copies into slot j+2 (last read by
//   iteration j-2): one barrier per two iterations.  K tile: rows of 128 bf16,
//   16-byte chunk c of row r at chunk slot c ^ f(r) so that the 16-row operand
//   reads cover all 64 banks.  V tile: 8 blocks of 16 channels, each 64 keys x
//   32 bytes, so one transpose read (16 keys x 32 bytes per wave) is one
//   contiguous 512-byte run.
//   Tails: query rows >= Sq are computed on zero queries and never stored;
//   keys >= Skv get score -inf.
#include "common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

struct CfgD128 {
    static constexpr int D = 128;
    static constexpr int kWaves = 8;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBr = 32 * kWaves;               // query rows per workgroup
    static constexpr int kBc = 64;                        // keys per tile
    static constexpr int kRowBytes = D * 2;
    static constexpr int kTileBytes = kBc * kRowBytes;    // one K or V tile (16 KB)
    static constexpr int kLoads = kTileBytes / (16 * kThreads);   // 16-B copies per thread
    static constexpr int kLoadRows = 16 * kThreads / kRowBytes;   // K rows one copy covers
    static constexpr int kCB = D / 16;                    // 16-channel blocks of O^T
    static constexpr int kKS = D / 32;                    // channel steps of K Q^T
    static constexpr int kVBlockBytes = kBc * 32;         // V tile: one 16-channel block
    static constexpr int kRing = 4;
    static constexpr int kHalf = kRing / 2;               // iterations per barrier
    static constexpr int kSlots = 4 * kCB;                // slots per iteration
    static constexpr int kCopySlotV = 1;                  // slots that issue the copies
    static constexpr int kCopySlotK = 5;
    static constexpr int kBarrierSlot = 29;               // see slot()
    // Bound on one lane's sum of weights of one tile and query (16 weights),
    // which keeps every weight <= 2^32: O and the sums cannot overflow for
    // |V| < 2^80.
    static constexpr float kWeightSumLimit = 0x1p32f;
};

// Chunk slot of chunk c in K row r: c XOR a permutation of r's low 4 bits
// (row bits 0, 1, 2, 3 to slot bits 0, 2, 1, 3), so 16 consecutive rows at one
// chunk sit in 16 distinct slots.  A K operand read (lane l: row l % 16, plus
// 16 per key block, chunk 4s + l / 16) is then free of bank conflicts; among
// the XOR permutations of this family some are and some are not, as measured
// with SQ_LDS_BANK_CONFLICT on the bare read pattern (row bits to slot bits
// 2, 3, 0, 1, for one, cost 4 extra cycles per read).
__device__ __forceinline__ int k_slot(int r, int c)
{
    return c ^ ((r & 9) | ((r & 2) << 1) | ((r & 4) >> 1));
}

__device__ __forceinline__ int k_lds_byte(int r, int col)
{
    return r * CfgD128::kRowBytes + k_slot(r, col >> 3) * 16 + (col & 7) * 2;
}

// Keep a vector-ALU result where it is computed (see the slot program).
__device__ __forceinline__ void pin(uint32_t& x)
{
    asm volatile("" : "+v"(x));
}

// Have x computed before this point, without redefining it: the compiler
// takes every register an asm statement writes to need a forwarding wait
// state before a vector instruction reads it, so a pin (above) right before
// such a read costs an s_nop.
__device__ __forceinline__ void use(float x)
{
    asm volatile("" ::"v"(x));
}

// The matrix instructions of the tile loop are asm statements, so that their
// order against the slot fences is fixed, O and Q^T stay in accumulation
// registers and S^T in VGPRs.  The compiler does not see them as MFMAs: the
// kernel keeps the wait states itself (vector code touches a block written by
// one at least 16 wait states later; tests/test_asm_hazards.py checks the
// generated code).  An instruction that accumulates onto the block the one
// before it wrote needs none: the matrix core forwards the accumulator.
//   O^T block += A B, accumulator in AGPRs.
__device__ __forceinline__ void mfma_o(f32x4& acc, const u32x4& a, const u32x4& b)
{
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

//   S^T block = A B (first channel step) or += A B; B (Q^T) in AGPRs.
__device__ __forceinline__ void mfma_s0(f32x4& acc, const u32x4& a, const u32x4& b)
{
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "a"(b));
}

__device__ __forceinline__ void mfma_s(f32x4& acc, const u32x4& a, const u32x4& b)
{
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}

// Chains of two in one statement (the compiler would otherwise pad the
// dependence between two asm statements with a wait state it does not need).
//   O^T block += A0 B0 + A1 B1.
__device__ __forceinline__ void mfma_o2(f32x4& acc, const u32x4& a0, const u32x4& b0,
                                        const u32x4& a1, const u32x4& b1)
{
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\t"
                 "v_mfma_f32_16x16x32_bf16 %0, %3, %4, %0"
                 : "+a"(acc) : "v"(a0), "v"(b0), "v"(a1), "v"(b1));
}

//   S^T block = A0 B0 + A1 B1 (first half of a chain; the operands must not
//   share registers with the block, which the first instruction writes).
__device__ __forceinline__ void mfma_s2_first(f32x4& acc, const u32x4& a0, const u32x4& b0,
                                              const u32x4& a1, const u32x4& b1)
{
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0\n\t"
                 "v_mfma_f32_16x16x32_bf16 %0, %3, %4, %0"
                 : "=&v"(acc) : "v"(a0), "a"(b0), "v"(a1), "a"(b1));
}

//   S^T block += A0 B0 + A1 B1.
__device__ __forceinline__ void mfma_s2(f32x4& acc, const u32x4& a0, const u32x4& b0,
                                        const u32x4& a1, const u32x4& b1)
{
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\t"
                 "v_mfma_f32_16x16x32_bf16 %0, %3, %4, %0"
                 : "+v"(acc) : "v"(a0), "a"(b0), "v"(a1), "a"(b1));
}

// The same chains with one exponential between their two instructions: e =
// 2^x, issued while the first instruction runs and before the second, which
// waits for it.  x comes from an instruction one slot earlier, so the
// exponential waits for nothing; e must not share registers with the
// operands, which the second instruction still reads.
__device__ __forceinline__ void mfma_o2_exp(f32x4& acc, const u32x4& a0, const u32x4& b0,
                                            const u32x4& a1, const u32x4& b1, float& e, float x)
{
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %2, %3, %0\n\t"
                 "v_exp_f32 %1, %6\n\t"
                 "v_mfma_f32_16x16x32_bf16 %0, %4, %5, %0"
                 : "+a"(acc), "=&v"(e) : "v"(a0), "v"(b0), "v"(a1), "v"(b1), "v"(x));
}

__device__ __forceinline__ void mfma_s2_first_exp(f32x4& acc, const u32x4& a0, const u32x4& b0,
                                                  const u32x4& a1, const u32x4& b1, float& e,
                                                  float x)
{
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %2, %3, 0\n\t"
                 "v_exp_f32 %1, %6\n\t"
                 "v_mfma_f32_16x16x32_bf16 %0, %4, %5, %0"
                 : "=&v"(acc), "=&v"(e) : "v"(a0), "a"(b0), "v"(a1), "a"(b1), "v"(x));
}

__device__ __forceinline__ void mfma_s2_exp(f32x4& acc, const u32x4& a0, const u32x4& b0,
                                            const u32x4& a1, const u32x4& b1, float& e, float x)
{
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %2, %3, %0\n\t"
                 "v_exp_f32 %1, %6\n\t"
                 "v_mfma_f32_16x16x32_bf16 %0, %4, %5, %0"
                 : "+v"(acc), "=&v"(e) : "v"(a0), "a"(b0), "v"(a1), "a"(b1), "v"(x));
}

// 16 wait states before vector code touches blocks the asm MFMAs may still be
// writing (a 4-pass MFMA needs at most 11).
__device__ __forceinline__ void acc_wait(f32x4& acc)
{
    asm volatile("s_nop 7\n\ts_nop 7" : "+a"(acc));
}

__device__ __forceinline__ void vgpr_wait(f32x4& acc)
{
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(acc));
}

// Lanes l, l^16, l^32 and l^48 hold the same query column: combine their values.
__device__ __forceinline__ float max_over_groups(float x)
{
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float sum_over_groups(float x)
{
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// Per-thread state of one workgroup's pass over the keys.
struct TileD128 {
    using Cfg = CfgD128;
    static constexpr int kBc = Cfg::kBc;
    static constexpr int kCB = Cfg::kCB;
    static constexpr int kKS = Cfg::kKS;
    static constexpr int kRing = Cfg::kRing;
    static constexpr int kHalf = Cfg::kHalf;
    static constexpr int kSlots = Cfg::kSlots;

    uint8_t* kobj[kRing];    // K and V tile buffers (ring slots), each its own LDS object
    uint8_t* vobj[kRing];
    __amdgpu_buffer_rsrc_t k_rsrc, v_rsrc;
    uint32_t tok_bytes;
    int key_end, wave, g;    // keys >= key_end are masked; g = lane / 16
    float scale_log2;
    uint32_t k_voff;         // this lane's source offset in K copy 0 (copy i: + i * kLoadRows rows)
    uint32_t v_voff;         // this lane's source offset in V copy 0 (copy i: + 64 channels)
    u32x4 qf[2][kKS];        // Q^T fragments [qb][channel step] (accumulation registers)
    int k_addr[kKS];         // LDS address of the K operand of channel step s in K slot 0
    uint32_t v_reg;          // LDS address of this lane's V transpose reads in V slot 0
    f32x4 oacc[kCB][2];      // O^T blocks [cb][qb]
    f32x4 sacc[8];           // S^T blocks b = 2 kb + qb (see the slot program)
    u32x4 pf[2][2][2];       // P^T fragments [parity][key step t][qb]
    u32x4 vf[2][2];          // V^T fragments [cb parity][key step t] of one channel block
    u32x4 kf[kKS];           // K fragments [channel step] of one 16-key block
    float lsum[2];           // this lane's weight sums of the current tile, per query block
    float lsum_max[2];       // largest lsum of the pass (checked against kWeightSumLimit)
    float m_used[2];         // reference maximum (scale*log2(e) units), fixed per pass
    float l_run[2];          // running sums over this lane's keys
    float xw;                // argument of the next slot's exponential
    int copy_kt;             // tile of the current iteration (for copies issued in its slots)
    bool partial;            // the current tile has keys >= key_end

    // Copy tile kt of K (to K ring slot KB) and/or of V (to V slot VB) into LDS;
    // a negative index skips that tensor.  Rows past the last key lie outside
    // the buffer range and read as zeros.
    template <int KB, int VB>
    __device__ __forceinline__ void copy_tile(int kt)
    {
        const uint32_t soff = (uint32_t)(kt * kBc) * tok_bytes;
#pragma unroll
        for (int i = 0; i < Cfg::kLoads; ++i) {
            const int off = (i * Cfg::kWaves + wave) * 1024;
            if constexpr (KB >= 0)
                copy16_to_lds(k_rsrc, kobj[KB] + off, k_voff,
                              soff + (uint32_t)(i * Cfg::kLoadRows) * tok_bytes);
            if constexpr (VB >= 0)
                copy16_to_lds(v_rsrc, vobj[VB] + off, v_voff, soff + i * 4 * 32);
        }
    }

    // K operand of channel step s, key block kb, from K ring slot KB: this
    // lane's address in slot 0 plus a constant that folds into the offset field.
    template <int KB>
    __device__ __forceinline__ u32x4 ld_k(int s, int kb) const
    {
        return ld_lds16(kobj[KB] + (k_addr[s] - (int)lds_addr(kobj[0]) + 16 * kb * Cfg::kRowBytes));
    }

    // The K fragments of key block KBLK from K ring slot KB: channel steps
    // 2H, 2H+1 (one half of every S^T chain of the key block).
    template <int KB, int KBLK, int H>
    __device__ __forceinline__ void read_kf()
    {
        kf[2 * H] = ld_k<KB>(2 * H, KBLK);
        kf[2 * H + 1] = ld_k<KB>(2 * H + 1, KBLK);
    }

    // V^T operand of channel block cb, key step t from V ring slot VB: two
    // transpose reads (keys 32t + 4g + 0..3, then 32t + 16 + 4g + 0..3).
    template <int VB>
    __device__ __forceinline__ u32x4 ld_v(int cb, int t) const
    {
        const uint8_t* p = vobj[VB] + ((int)v_reg - (int)lds_addr(vobj[0]) +
                                       cb * Cfg::kVBlockBytes + 32 * t * 32);
        const u32x2 lo = ld_lds_tr16(p), hi = ld_lds_tr16(p + 16 * 32);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
    }

    template <int VB, int CB>
    __device__ __forceinline__ void read_vf()
    {
        vf[CB % 2][0] = ld_v<VB>(CB, 0);
        vf[CB % 2][1] = ld_v<VB>(CB, 1);
    }

    // The full S^T of one tile from K slot KB into sacc (prologue and the
    // maximum pass only).
    template <int KB>
    __device__ __forceinline__ void qk_tile()
    {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            u32x4 a[kKS];
#pragma unroll
            for (int s = 0; s < kKS; ++s)
                a[s] = ld_k<KB>(s, kb);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                mfma_s0(sacc[2 * kb + qb], a[0], qf[qb][0]);
#pragma unroll
                for (int s = 1; s < kKS; ++s)
                    mfma_s(sacc[2 * kb + qb], a[s], qf[qb][s]);
            }
        }
#pragma unroll
        for (int b = 0; b < 8; ++b)
            vgpr_wait(sacc[b]);
    }

    // Argument of weight J (of the order w = 4 b + i, register i of block b =
    // 2 kb + qb) into xw: the scaled score less the reference maximum.
    template <int J>
    __device__ __forceinline__ void weight_arg()
    {
        constexpr int b = J / 4, qb = b % 2, i = J % 4;
        use(m_used[qb]);
        xw = __builtin_fmaf(sacc[b][i], scale_log2, -m_used[qb]);
        use(xw);
    }

    // Softmax of the current tile after the matrix instructions of slot I,
    // whose asm statement computed e = 2^xw, weight I: the weight goes back
    // into its S^T register, the argument of weight I+1 is computed for the
    // next slot, and weight I-1 is folded (its sum and bf16 pair come one slot
    // after its exponential, so that no instruction waits on it).
    template <int P, int I>
    __device__ __forceinline__ void softmax_part(float e)
    {
        constexpr int b = I / 4, i = I % 4;
        use(e);
        sacc[b][i] = e;
        if constexpr (I + 1 < kSlots)
            weight_arg<I + 1>();
        if constexpr (I > 0)
            fold<P, I - 1>();
    }

    // Weight J into lsum and, with the one before it, into P^T: the pair
    // (i - 1, i) of block b = 2 kb + qb is word 2 (kb % 2) + i / 2 of
    // fragment pf[P][kb / 2][qb].
    template <int P, int J>
    __device__ __forceinline__ void fold()
    {
        constexpr int b = J / 4, kb = b / 2, qb = b % 2, i = J % 4;
        const float e = sacc[b][i];
        lsum[qb] = (J == 4 * qb) ? e : lsum[qb] + e;
        use(lsum[qb]);
        if constexpr (i % 2 == 1) {
            uint32_t pk = pack_bf16x2(sacc[b][i - 1], e);
            pin(pk);
            pf[P][kb / 2][qb][2 * (kb % 2) + i / 2] = pk;
        }
    }

    // Scores of keys >= key_end in block b of the current tile (at key0 =
    // copy_kt * kBc) -> -inf.  Register i of block b = 2 kb + qb holds key
    // key0 + 16kb + 4g + i.
    __device__ __forceinline__ void mask_one(int b)
    {
        vgpr_wait(sacc[b]);  // its K Q^T chain may have ended just before
        const int lim = key_end - copy_kt * kBc - 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (16 * (b / 2) + i >= lim)
                sacc[b][i] = -INFINITY;
    }

    template <int b>
    __device__ __forceinline__ void mask_block()
    {
        mask_one(b);
    }

    // Scores of keys >= key_end in the tile at key0 (all of sacc) -> -inf
    // (prologue and the maximum pass).
    __device__ __forceinline__ void mask_tile(int key0)
    {
#pragma unroll
        for (int b = 0; b < 8; ++b)
            vgpr_wait(sacc[b]);
        const int lim = key_end - key0 - 4 * g;
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (16 * (b / 2) + i >= lim)
                    sacc[b][i] = -INFINITY;
    }

    // Row maximum (scale*log2(e) units) of query block qb of the tile in sacc.
    __device__ __forceinline__ float tile_max(int qb) const
    {
        float m = sacc[qb][0];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                m = fmaxf(m, sacc[2 * kb + qb][i]);
        return max_over_groups(m) * scale_log2;
    }

    // One step of the maximum pass: S^T of the tile kt from K slot KB (its
    // copy waited for), the copy of K(kt+1) into slot KB + kHalf started.
    template <int KB>
    __device__ __forceinline__ void max_step(int kt, float (&m)[2])
    {
        copy_tile<(KB + kHalf) % kRing, -1>(kt + 1);
        qk_tile<KB>();
        const int key0 = kt * kBc;
        if (key0 + kBc > key_end)
            mask_tile(key0);
        m[0] = fmaxf(m[0], tile_max(0));
        m[1] = fmaxf(m[1], tile_max(1));
        wait_vmem_all();
        __syncthreads();
    }

    // Slot I of the iteration that reads ring slot R (parity P = R % 2): one
    // chain of two matrix instructions, LDS reads for later slots, and one
    // weight of the softmax of the current tile (weight I, of block I/4).
    //   even I = 2u: O^T += V^T P^T for channel block cb = u/2, query block
    //     u%2 (P^T of the previous tile, V from slot R), over the tile's two
    //     key steps; at the block's first slot, the V^T fragments of block
    //     cb+1 (last block: block 0 of the next iteration, from slot R+1)
    //     into the other fragment buffer first.
    //   odd I: half of an S^T chain (channel steps 2h, 2h+1).  S^T has one
    //     set of registers: block b = 2 kb + qb of the next tile is computed
    //     in slots 4b+5 (h = 0) and 4b+7 (h = 1), right after the softmax of
    //     this tile has finished with block b; the last block wraps into
    //     slots 1 and 3 of the next iteration, so slots 1 and 3 compute block
    //     7 of the current tile.  K fragments (one set): the half h of key
    //     block kb of the next tile (from slot R) is read at slot 8kb + 2 +
    //     2h, right after the last chain half that used the same registers
    //     for key block kb-1.
    // (The reads lead their use by three to four slots; the V^T fragments of
    // the next iteration's block 0 come from slot R+1 at slot 30, behind the
    // barrier of slot 29.)
    template <int R, int I>
    __device__ __forceinline__ void slot()
    {
        constexpr int P = R % 2;
        constexpr int W = (R + kHalf) % kRing;  // ring slot this iteration's copies fill
        constexpr int RN = (R + 1) % kRing;     // ring slot of the next iteration
        if constexpr (I == Cfg::kBarrierSlot) {
            // The pair's barrier: every wave's copies so far have landed (the
            // slots of the next kHalf iterations hold their tiles) and every
            // wave has finished its reads of this iteration's ring slot (the
            // last one came in the slot before; the first reads of slot R+1
            // come after), which later copies overwrite.
            if constexpr (R % kHalf == kHalf - 1) {
                wait_vmem_all();
                __syncthreads();
            }
        }
        if constexpr (I == 6) {
            // block 7 of the current tile is complete (slots 1 and 3)
            if (partial)
                mask_block<7>();
        }
        float e;  // weight I, computed inside the slot's asm statement
        if constexpr (I % 2 == 0) {
            constexpr int u = I / 2, cb = u / 2, qb = u % 2;
            mfma_o2_exp(oacc[cb][qb], vf[cb % 2][0], pf[P ^ 1][0][qb], vf[cb % 2][1],
                        pf[P ^ 1][1][qb], e, xw);
            // (the reads come after the matrix instructions, which then issue
            // without waiting behind them)
            if constexpr (qb == 0 && cb + 1 < kCB)
                read_vf<R, cb + 1>();
            if constexpr (I == kSlots - 2)
                read_vf<RN, 0>();
        } else {
            // block b, half hs: slots 4b+5+2hs (mod 32)
            constexpr int b = I < 5 ? 7 : (I - 5) / 4, hs = I < 5 ? (I - 1) / 2 : ((I - 5) / 2) % 2;
            constexpr int kb = b / 2, qb = b % 2;
            if constexpr (hs == 0)
                mfma_s2_first_exp(sacc[b], kf[0], qf[qb][0], kf[1], qf[qb][1], e, xw);
            else
                mfma_s2_exp(sacc[b], kf[2], qf[qb][2], kf[3], qf[qb][3], e, xw);
        }
        if constexpr (I % 8 == 2 || I % 8 == 4)
            read_kf<R, I / 8, (I % 8) / 4>();
        softmax_part<P, I>(e);
        if constexpr (I == Cfg::kCopySlotV)
            copy_tile<-1, W>(copy_kt + kHalf - 1);
        if constexpr (I == Cfg::kCopySlotK)
            copy_tile<W, -1>(copy_kt + kHalf + 1);
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
    // iterations: P^T in pf[1], V in the ring slot vb).
    __device__ __forceinline__ void drain(const uint8_t* vb)
    {
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
            const uint8_t* p = vb + ((int)v_reg - (int)lds_addr(vobj[0]) + cb * Cfg::kVBlockBytes);
            u32x4 v[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const u32x2 lo = ld_lds_tr16(p + 32 * t * 32), hi = ld_lds_tr16(p + (32 * t + 16) * 32);
                v[t] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                mfma_o(oacc[cb][qb], v[0], pf[1][0][qb]);
                mfma_o(oacc[cb][qb], v[1], pf[1][1][qb]);
            }
        }
    }

    // Iteration kt, reading ring slot R (kt - first tile = R mod kRing): P V
    // of tile kt-1 (V there), K Q^T of tile kt+1 (K there), softmax of tile
    // kt; copies V(kt + kHalf-1), K(kt + kHalf+1) into ring slot R + kHalf,
    // which iteration kt - kHalf read last.  On entry vf[0] holds channel
    // block 0's V^T fragments, kf key block 3's K fragments of tile kt and
    // sacc blocks 0..6 tile kt's S^T, all from the iteration before (or from
    // before the first one).
    template <int R>
    __device__ __forceinline__ void iteration(int kt)
    {
        constexpr int P = R % 2;
        copy_kt = kt;
        partial = kt * kBc + kBc > key_end;
        if (partial) {
#pragma unroll
            for (int b = 0; b < 7; ++b)
                mask_one(b);
        }
        weight_arg<0>();  // the first slot's exponential (after the masking)
        // re-pinned here, in the block of this iteration's reads, so that the
        // slot distances fold into their offset fields
        asm volatile("" : "+v"(v_reg));
        __builtin_amdgcn_sched_barrier(0);
        slots<R, 0>();
        fold<P, kSlots - 1>();
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            l_run[qb] += lsum[qb];
            lsum_max[qb] = fmaxf(lsum_max[qb], lsum[qb]);
        }
        debug_sync();
    }
};

// Grid: blocks [0, n_main) each take one query tile over all keys; the
// remaining query tiles are each split into nsplit pieces over contiguous
// ranges of key tiles, which write their normalised fp32 partial O and LSE to
// the workspace (ws_o [piece][kBr][D], ws_lse [piece][kBr]); launch_split_merge
// (split.hip) combines them.
__global__ __launch_bounds__(CfgD128::kThreads, 1) void fwd_bf16_d128_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int H, int Sq, int Skv, float scale_log2, int n_qtiles, int n_main, int nsplit,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, int acc, long kv_bstride)
{
    using Cfg = CfgD128;
    constexpr int D = Cfg::D;
    constexpr int kCB = Cfg::kCB;
    constexpr int kKS = Cfg::kKS;
    constexpr int kRing = Cfg::kRing;
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[Cfg::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[Cfg::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds2[Cfg::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t k_lds3[Cfg::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[Cfg::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[Cfg::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds2[Cfg::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t v_lds3[Cfg::kTileBytes];
    __shared__ int wave_over[Cfg::kWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c16 = lane & 15;  // query column of this lane within a 16-query block
    const int g = lane >> 4;    // which group of 8 k slots this lane feeds

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

    TileD128 st;
    st.kobj[0] = k_lds0;
    st.kobj[1] = k_lds1;
    st.kobj[2] = k_lds2;
    st.kobj[3] = k_lds3;
    st.vobj[0] = v_lds0;
    st.vobj[1] = v_lds1;
    st.vobj[2] = v_lds2;
    st.vobj[3] = v_lds3;
    st.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    st.g = g;
    st.key_end = min(kt1 * Cfg::kBc, Skv);
    st.scale_log2 = scale_log2;
    st.tok_bytes = (uint32_t)(tok * 2);
    {
        // batches of K and V lie kv_bstride tokens apart (Skv when contiguous)
        const uint16_t* Kbh = K + ((long)b * kv_bstride * H + h) * D;
        const uint16_t* Vbh = V + ((long)b * kv_bstride * H + h) * D;
        // Byte extent of this (b, h)'s keys: rows 0 .. Skv-1 (callers guarantee < 2^32).
        const int extent = (int)((uint32_t)(Skv - 1) * st.tok_bytes + Cfg::kRowBytes);
        st.k_rsrc = make_rsrc(Kbh, extent);
        st.v_rsrc = make_rsrc(Vbh, extent);
    }
    // Copy i of wave w fills LDS chunks [(i*kWaves + w)*64, +64) of a tile; lane
    // l takes chunk p = that base + l.
    //   K (row-major, swizzled): row p / 16 at chunk slot p % 16, which holds
    //   column chunk (p % 16) ^ f(row).  Copy i covers rows i * kLoadRows more
    //   than copy 0 and, as f() depends only on the row's low 4 bits, the same
    //   chunk slots.
    //   V (16-channel blocks of 64 keys x 32 bytes): block p / 128, key
    //   (p / 2) % 64, 16-byte half p % 2 of the block's 32 bytes.  Copy i is
    //   four blocks (64 channels) further on.
    {
        const int p = st.wave * 64 + lane;
        const int r = p / 16;
        st.k_voff = (uint32_t)r * st.tok_bytes + k_slot(r, p % 16) * 16;
        st.v_voff = (uint32_t)((p / 2) % 64) * st.tok_bytes + ((p / 128) * 2 + p % 2) * 16;
    }
    // A pass starts with what its first kHalf iterations read: K(kt0) in the
    // last ring slot (the prologue's K Q^T), K(kt0+1), K(kt0+2) in slots 0, 1,
    // V(kt0) in slot 1, and V(kt0) in slot 0 too, where the first iteration's
    // P V (with P = 0) reads finite values.
    auto pass_copies = [&]() {
        st.template copy_tile<kRing - 1, -1>(kt0);
        st.template copy_tile<0, -1>(kt0 + 1);
        st.template copy_tile<1, -1>(kt0 + 2);
        st.template copy_tile<-1, 1>(kt0);
        st.template copy_tile<-1, 0>(kt0);
    };
    pass_copies();

    // Q^T fragments: query block qb, channel step s: lane l holds query
    // 16qb + l%16 at channels 32s + 8g .. +7.
    const int q_base = qt * Cfg::kBr + st.wave * 32;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int q_row = q_base + 16 * qb + c16;
        if (q_row < Sq) {
            const uint16_t* src = Q + ((long)b * Sq * H + h) * D + (long)q_row * tok + 8 * g;
#pragma unroll
            for (int s = 0; s < kKS; ++s)
                st.qf[qb][s] = ld_global16(src + 32 * s);
        } else {
#pragma unroll
            for (int s = 0; s < kKS; ++s)
                st.qf[qb][s] = u32x4{0, 0, 0, 0};
        }
    }
    // Q^T lives in accumulation registers for the whole kernel (the K Q^T asm
    // takes B from there).
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int s = 0; s < kKS; ++s)
            asm volatile("" : "+a"(st.qf[qb][s]));

    // Per-lane LDS bases.  K operand of channel step s: row l%16 (+16 per key
    // block), columns 32s + 8g .. +7.  V transpose reads: the lane's 16-lane
    // group reads keys 4g + (0..3) (+ the key step's and half's offsets) of a
    // channel block, lane l%16 pointing at key 4g + (l%16)/4, channels
    // 4((l%16)%4) .. +3, so lane l receives channel l%16 of the four keys.
#pragma unroll
    for (int s = 0; s < kKS; ++s)
        st.k_addr[s] = lds_addr(k_lds0) + k_lds_byte(c16, 32 * s + 8 * g);
    st.v_reg = lds_addr(v_lds0) + (4 * g + (c16 >> 2)) * 32 + (c16 & 3) * 8;
    asm volatile("" : "+v"(st.v_reg));

    // Passes over the key range (see the file comment): the first against the
    // first tile's row maxima, a second against the exact row maxima if some
    // weight sum of the first passed kWeightSumLimit.
    for (int pass = 0;; ++pass) {
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                st.oacc[cb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
                acc_wait(st.oacc[cb][qb]);
            }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
                st.pf[1][t][qb] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            st.l_run[qb] = 0.f;
            st.lsum_max[qb] = 0.f;
        }

        wait_vmem_all();
        __syncthreads();
        st.template qk_tile<kRing - 1>();
        if (pass == 0) {
            if (kt0 * Cfg::kBc + Cfg::kBc > st.key_end)
                st.mask_tile(kt0 * Cfg::kBc);
            st.m_used[0] = st.tile_max(0);
            st.m_used[1] = st.tile_max(1);
        }
        // what the first iteration expects from an iteration before it (see
        // iteration()): channel block 0's V^T fragments and key block 3's K
        // fragments of tile kt0 (its slots 1 and 3 compute block 7 of tile
        // kt0 again, to the same values)
        st.template read_vf<0, 0>();
        st.template read_kf<kRing - 1, 3, 0>();
        st.template read_kf<kRing - 1, 3, 1>();
        __syncthreads();  // the last ring slot is refilled by iteration kHalf-1

        // One iteration per tile of the range, unrolled over the ring slots,
        // then the last tile's P V: by one more iteration if the count is odd
        // (its own tile lies past the range: all keys masked, weights 0), else
        // by drain().
        const int n_it = kt1 - kt0;
        const int n_pad = (n_it + 1) & ~1;
        int i = 0;
        for (; i + 4 <= n_pad; i += 4) {
            st.template iteration<0>(kt0 + i);
            st.template iteration<1>(kt0 + i + 1);
            st.template iteration<2>(kt0 + i + 2);
            st.template iteration<3>(kt0 + i + 3);
        }
        if (i < n_pad) {
            st.template iteration<0>(kt0 + i);
            st.template iteration<1>(kt0 + i + 1);
            i += 2;
        }
        // the last iteration's K Q^T results (of a tile past the range) are
        // dead: hold their registers until those matrix instructions are done
#pragma unroll
        for (int b = 0; b < 8; ++b)
            vgpr_wait(st.sacc[b]);
        if (i == n_it)
            st.drain(i % kRing == 0 ? st.vobj[0] : st.vobj[kRing - 2]);

        if (lane == 0)
            wave_over[st.wave] = __builtin_amdgcn_ballot_w64(
                st.lsum_max[0] > Cfg::kWeightSumLimit || st.lsum_max[1] > Cfg::kWeightSumLimit) != 0;
        __syncthreads();
        int over = 0;
#pragma unroll
        for (int w = 0; w < Cfg::kWaves; ++w)
            over |= wave_over[w];
        if (!over || pass > 0)
            break;

        // exact row maxima of the range, then the second pass
        float m[2] = {-INFINITY, -INFINITY};
        st.template copy_tile<0, -1>(kt0);
        wait_vmem_all();
        __syncthreads();
        const int n_mx = (kt1 - kt0 + 1) & ~1;
        for (int j = 0; j < n_mx; j += 2) {
            st.template max_step<0>(kt0 + j, m);
            st.template max_step<Cfg::kHalf>(kt0 + j + 1, m);
        }
        st.m_used[0] = m[0];
        st.m_used[1] = m[1];
        pass_copies();
    }
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
            acc_wait(st.oacc[cb][qb]);

#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float l_tot = sum_over_groups(st.l_run[qb]);
        const float inv_l = 1.f / l_tot;
        const float lse_new = (st.m_used[qb] + log2_fast(l_tot)) * kLn2;
        const int r = st.wave * 32 + 16 * qb + c16;  // row within the query tile
        const int q_row = qt * Cfg::kBr + r;
        if (piece >= 0) {
            // partial result of a split tile: normalised fp32 O and LSE (natural log)
            float* dst = ws_o + ((long)piece * Cfg::kBr + r) * D + 4 * g;
#pragma unroll
            for (int cb = 0; cb < kCB; ++cb)
                *reinterpret_cast<f32x4*>(dst + 16 * cb) = st.oacc[cb][qb] * inv_l;
            if (g == 0)
                ws_lse[(long)piece * Cfg::kBr + r] = lse_new;
        } else if (q_row < Sq) {
            uint16_t* dst = O + ((long)b * Sq * H + h) * D + (long)q_row * tok + 4 * g;
            float* lse_dst = LSE + ((long)b * H + h) * Sq + q_row;
            // O = c_new * acc + c_old * O_old; without a running result (acc = 0,
            // or its LSE is -inf) that is the plain normalisation
            float c_new = inv_l, c_old = 0.f, lse_out = lse_new;
            if (acc)
                merge_weights(*lse_dst, lse_new, c_new, c_old, lse_out);
#pragma unroll
            for (int cb = 0; cb < kCB; ++cb) {
                f32x4 o = st.oacc[cb][qb] * c_new;
                u32x2* p = reinterpret_cast<u32x2*>(dst + 16 * cb);
                if (c_old != 0.f) {
                    const u32x2 old = *p;
                    o += c_old * f32x4{bf16_lo(old[0]), bf16_hi(old[0]), bf16_lo(old[1]),
                                       bf16_hi(old[1])};
                }
                *p = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            }
            if (g == 0)
                *lse_dst = lse_out;
        }
    }
}

}  // namespace

FwdSplit plan_fwd_bf16_d128_split(int B, int H, int Sq, int Skv, int n_cu)
{
    using Cfg = CfgD128;
    const long n_blocks = (long)((Sq + Cfg::kBr - 1) / Cfg::kBr) * H * B;
    const long n_kt = (Skv + Cfg::kBc - 1) / Cfg::kBc;
    return plan_split(n_blocks, n_kt, Cfg::kBr, 1, n_cu, Cfg::D + 1);
}

hipError_t launch_fwd_bf16_d128(const FwdArgs& a, const FwdSplit& sp, hipStream_t stream)
{
    using Cfg = CfgD128;
    const int n_qtiles = (a.Sq + Cfg::kBr - 1) / Cfg::kBr;
    const long n_blocks = (long)n_qtiles * a.H * a.B;
    if (n_blocks > 0x7fffffffL)
        return hipErrorInvalidConfiguration;
    const float scale_log2 = a.scale * kLog2e;
    const bool split = sp.n_tail > 0;
    float* ws_o = split ? static_cast<float*>(a.ws) : nullptr;
    float* ws_lse = split ? ws_o + (size_t)sp.n_tail * sp.nsplit * Cfg::kBr * Cfg::D : nullptr;
    const long grid = split ? (long)sp.n_main + (long)sp.n_tail * sp.nsplit : n_blocks;
    hipError_t e = launch_kernel(fwd_bf16_d128_kernel, dim3((unsigned)grid), dim3(Cfg::kThreads),
                                 stream, a.q, a.k, a.v, a.o, a.lse, a.H, a.Sq, a.Skv, scale_log2,
                                 n_qtiles, split ? sp.n_main : (int)n_blocks,
                                 split ? sp.nsplit : 1, ws_o, ws_lse, a.acc,
                                 a.kv_batch_tokens > 0 ? a.kv_batch_tokens : (long)a.Skv);
    if (e != hipSuccess || !split)
        return e;
    return launch_split_merge(a, sp, Cfg::kBr, n_qtiles, ws_o, ws_lse, nullptr, stream);
}

}  // namespace dit
