// merge.hip -- log-sum-exp merge of partial attention results over disjoint
// key blocks, for gfx950.
//
// Ring attention splits the key/value sequence into blocks that pass around a
// ring ("xDiT 项目概述" sec. 3.2, USP's ring dimension), so one GPU's queries
// produce one partial (O_c, LSE_c) per block; this kernel combines them:
//     M = max_c LSE_c,  w_c = exp(LSE_c - M),
//     O = sum_c w_c O_c / sum_c w_c,  LSE = M + ln sum_c w_c.
// It is HBM-bound: every byte of the n partial outputs is read once and the
// result written once.  One thread owns one 16-byte chunk (8 channels) of one
// (b, s, h) row; consecutive threads walk consecutive chunks, so each wave's
// loads and stores are contiguous 1 KiB runs.  All threads of a row sit in
// the same wavefront, so an in-place merge (o == o_parts[0]) reads every
// input before any lane of the row writes.
#include <utility>

#include "common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

struct MergeKernelArgs {
    const uint16_t* o_parts[kMaxMergeParts];
    const float* lse_parts[kMaxMergeParts];
};

// NP (the number of parts) is a template argument so that the part loops
// unroll: a lane issues the loads of all NP log-sum-exps and all NP chunks
// before it waits on any of them.  With one 16-byte load in flight per lane
// (a loop whose trip count is only known at run time waits on each part's
// load before it issues the next) the 32 waves a CU can hold keep too few
// bytes in flight to cover HBM latency: the Wan-shape merge ran at 60% of
// the HBM peak that way.
// NT: non-temporal loads and stores, for merges that move more bytes than
// the 256 MB last-level cache (MALL) holds -- streaming them through it only
// evicts other data (Wan-shape merge, 426 MB: +10%); a smaller merge whose
// partial outputs may still sit there keeps ordinary accesses (-8% with NT).
template <int D, int NP, bool NT>
__global__ __launch_bounds__(256) void merge_kernel(MergeKernelArgs p, uint16_t* O, float* LSE,
                                                    int H, int Sq, long n_rows)
{
    constexpr int kChunks = D / 8;
    // 32-bit row arithmetic (the launcher checks that the rows fit): 64-bit
    // divisions by H and Sq would cost more vector instructions than the rest
    // of the kernel
    const unsigned row = blockIdx.x * (256u / kChunks) + threadIdx.x / kChunks;
    const int c = (int)(threadIdx.x % kChunks);
    if (row >= (unsigned)n_rows)
        return;
    const unsigned bs = row / (unsigned)H;
    const unsigned h = row - bs * (unsigned)H;
    const unsigned b = bs / (unsigned)Sq;
    const unsigned s = bs - b * (unsigned)Sq;
    const long lidx = ((long)b * H + h) * Sq + s;

    float lse[NP];
    u32x4 x[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i)
        lse[i] = p.lse_parts[i][lidx];
#pragma unroll
    for (int i = 0; i < NP; ++i)
        x[i] = NT ? __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4*>(p.o_parts[i] + (long)row * D + c * 8))
                  : ld_global16(p.o_parts[i] + (long)row * D + c * 8);

    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < NP; ++i)
        M = fmaxf(M, lse[i]);
    // No branch on M: the chunks are used on every path, so the compiler does
    // not sink their loads behind the wait on the log-sum-exps.  When every
    // part is empty (M = -inf) the weights are exp2(-inf) = 0 and the result
    // is selected as O = 0, LSE = -inf below.
    const bool empty = M == -INFINITY;
    const float m = empty ? 0.f : M;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const float w = exp2_fast((lse[i] - m) * kLog2e);
        L += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += w * __builtin_bit_cast(float, x[i][e] << 16);
            acc[2 * e + 1] += w * __builtin_bit_cast(float, x[i][e] & 0xffff0000u);
        }
    }
    const float inv = 1.f / L;
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        out[e] = empty ? 0u : pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    const float lse_out = empty ? -INFINITY : M + log2_fast(L) * kLn2;
    if (NT)
        __builtin_nontemporal_store(out, reinterpret_cast<u32x4*>(O + (long)row * D + c * 8));
    else
        st_global16(O + (long)row * D + c * 8, out);
    if (c == 0)
        LSE[lidx] = lse_out;
}

template <int D, int NP>
hipError_t launch_merge_np(const MergeKernelArgs& p, const MergeArgs& a, long n_rows,
                           unsigned blocks, hipStream_t stream)
{
    constexpr long kMallBytes = 256l << 20;
    const long bytes = (long)(NP + 1) * n_rows * (D * 2 + 4);
    if (bytes > kMallBytes)
        return launch_kernel(merge_kernel<D, NP, true>, dim3(blocks), dim3(256), stream, p, a.o,
                             a.lse, a.H, a.Sq, n_rows);
    return launch_kernel(merge_kernel<D, NP, false>, dim3(blocks), dim3(256), stream, p, a.o,
                         a.lse, a.H, a.Sq, n_rows);
}

template <int D, int... NP>
hipError_t launch_merge_parts(std::integer_sequence<int, NP...>, const MergeKernelArgs& p,
                              const MergeArgs& a, long n_rows, unsigned blocks,
                              hipStream_t stream)
{
    using Launch = hipError_t (*)(const MergeKernelArgs&, const MergeArgs&, long, unsigned,
                                  hipStream_t);
    static constexpr Launch table[] = {&launch_merge_np<D, NP + 1>...};
    return table[a.n_parts - 1](p, a, n_rows, blocks, stream);
}

template <int D>
hipError_t launch_merge_d(const MergeArgs& a, hipStream_t stream)
{
    if (a.n_parts < 1 || a.n_parts > kMaxMergeParts)
        return hipErrorInvalidValue;
    MergeKernelArgs p = {};
    for (int i = 0; i < a.n_parts; ++i) {
        p.o_parts[i] = (const uint16_t*)a.o_parts[i];
        p.lse_parts[i] = a.lse_parts[i];
    }
    const long n_rows = (long)a.B * a.Sq * a.H;
    if (n_rows > 0x7fffffffL)
        return hipErrorInvalidConfiguration;
    const long blocks = (n_rows + 256 / (D / 8) - 1) / (256 / (D / 8));
    return launch_merge_parts<D>(std::make_integer_sequence<int, kMaxMergeParts>(), p, a, n_rows,
                                 (unsigned)blocks, stream);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream)
{
    return a.d == 64 ? launch_merge_d<64>(a, stream) : launch_merge_d<128>(a, stream);
}

}  // namespace dit
