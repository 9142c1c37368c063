// split.hip -- the split launch of the forward kernels: planning, and the
// merge of the pieces of split query tiles.
//
// A forward launch runs one workgroup per query tile.  When the number of
// tiles is not a multiple of what the GPU runs at once, the last wave of
// workgroups leaves most of the GPU idle.  The split launch runs the tiles of
// that wave as nsplit pieces over contiguous ranges of key tiles instead (the
// ring dimension of "xDiT 项目概述" sec. 3.2 applied inside one GPU); each piece
// writes its partial result to caller-provided scratch and split_merge_kernel
// combines them with the log-sum-exp merge (the same arithmetic as
// dit_attn_merge).
#include "common.hpp"
#include "launch.hpp"

#include <algorithm>

namespace dit {
namespace {

// Combine the nsplit pieces of each split query tile (rows rows each):
//     LSE = M + ln sum_p exp(LSE_p - M),  M = max_p LSE_p;
//     O = sum_p w_p O_p / sum_p w_p with w_p = exp(W_p - max_p W_p), where W_p
//     is LSE_p, or the piece's own log-weight ws_w (if given) when O_p was
//     normalised by a different sum than the one LSE_p is the log of.
// With acc, the result is then merged into the running (O, LSE) the output
// holds (merge_weights).  One thread per (split tile, row, 4 channels); the
// threads of one row sit in one wave, so every read of the row's LSE comes
// before its write.
template <int D>
__global__ __launch_bounds__(256) void split_merge_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
    const float* __restrict__ ws_w, uint16_t* __restrict__ O, float* __restrict__ LSE, int H,
    int Sq, int rows, int n_qtiles, int n_main, int nsplit, int n_tail, int acc)
{
    constexpr int kChunks = D / 4;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)n_tail * rows * kChunks)
        return;
    const int c = (int)(idx % kChunks);
    const int r = (int)((idx / kChunks) % rows);
    const int t = (int)(idx / ((long)kChunks * rows));
    const int tile = n_main + t;
    const int qt = tile % n_qtiles;
    const int bh = tile / n_qtiles;
    const int h = bh % H;
    const int b = bh / H;
    const int q_row = qt * rows + r;
    if (q_row >= Sq)
        return;
    const long p0 = (long)t * nsplit;
    const float* wo = ws_w ? ws_w : ws_lse;
    float m = -INFINITY, mw = -INFINITY;
    for (int p = 0; p < nsplit; ++p) {
        m = fmaxf(m, ws_lse[(p0 + p) * rows + r]);
        mw = fmaxf(mw, wo[(p0 + p) * rows + r]);
    }
    float lsum = 0.f, wsum = 0.f;
    f32x4 sum_o = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < nsplit; ++p) {
        lsum += exp2_fast((ws_lse[(p0 + p) * rows + r] - m) * kLog2e);
        const float w = exp2_fast((wo[(p0 + p) * rows + r] - mw) * kLog2e);
        const f32x4 o = *reinterpret_cast<const f32x4*>(ws_o + ((p0 + p) * rows + r) * D + 4 * c);
        sum_o += w * o;
        wsum += w;
    }
    float* lse_dst = LSE + ((long)b * H + h) * Sq + q_row;
    const float lse_new = m + log2_fast(lsum) * kLn2;
    float c_new = 1.f / wsum, c_old = 0.f, lse_out = lse_new;
    if (acc)
        merge_weights(*lse_dst, lse_new, c_new, c_old, lse_out);
    u32x2* dst = reinterpret_cast<u32x2*>(O + (((long)b * Sq + q_row) * H + h) * D + 4 * c);
    f32x4 o = c_new * sum_o;
    if (c_old != 0.f) {
        const u32x2 old = *dst;
        o += c_old * f32x4{bf16_lo(old[0]), bf16_hi(old[0]), bf16_lo(old[1]), bf16_hi(old[1])};
    }
    *dst = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    if (c == 0)
        *lse_dst = lse_out;
}

}  // namespace

FwdSplit plan_split(long n_blocks, long n_kt, int rows, int wg_per_cu, int n_cu,
                    int floats_per_row)
{
    FwdSplit sp = {};
    sp.n_main = (int)n_blocks;
    sp.nsplit = 1;
    if (n_cu <= 0 || n_blocks <= 0 || n_blocks > 0x7fffffffL)
        return sp;
    const long slots = (long)wg_per_cu * n_cu;  // workgroups resident at once
    const long rem = n_blocks % slots;
    // split only a last wave that would leave at least half of the machine idle,
    // into pieces of at least 4 key tiles
    long nsplit = rem > 0 ? slots / rem : 0;
    nsplit = std::min({nsplit, n_kt / 4, (long)kMaxSplit});
    if (rem == 0 || 2 * rem > slots || nsplit < 2)
        return sp;
    sp.n_main = (int)(n_blocks - rem);
    sp.nsplit = (int)nsplit;
    sp.n_tail = (int)rem;
    sp.ws_bytes = (size_t)(rem * nsplit) * rows * floats_per_row * sizeof(float);
    return sp;
}

hipError_t launch_split_merge(const FwdArgs& a, const FwdSplit& sp, int rows, int n_qtiles,
                              const float* ws_o, const float* ws_lse, const float* ws_w,
                              hipStream_t stream)
{
    const long n_threads = (long)sp.n_tail * rows * (a.d / 4);
    const dim3 grid((unsigned)((n_threads + 255) / 256)), block(256);
    auto* o = static_cast<uint16_t*>(a.o);
    if (a.d == 64)
        return launch_kernel(split_merge_kernel<64>, grid, block, stream, ws_o, ws_lse, ws_w, o,
                             a.lse, a.H, a.Sq, rows, n_qtiles, sp.n_main, sp.nsplit, sp.n_tail,
                             a.acc);
    return launch_kernel(split_merge_kernel<128>, grid, block, stream, ws_o, ws_lse, ws_w, o,
                         a.lse, a.H, a.Sq, rows, n_qtiles, sp.n_main, sp.nsplit, sp.n_tail,
                         a.acc);
}

}  // namespace dit
