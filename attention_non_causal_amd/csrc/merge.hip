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
#include "common.hpp"
#include "launch.hpp"

namespace dit {
namespace {

struct MergeKernelArgs {
    const uint16_t* o_parts[kMaxMergeParts];
    const float* lse_parts[kMaxMergeParts];
};

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeKernelArgs p, int n_parts,
                                                    uint16_t* O, float* LSE, int H, int Sq,
                                                    long n_rows)
{
    constexpr int kChunks = D / 8;
    const long gid = (long)blockIdx.x * 256 + threadIdx.x;
    const long row = gid / kChunks;
    const int c = (int)(gid % kChunks);
    if (row >= n_rows)
        return;
    const int h = (int)(row % H);
    const long bs = row / H;
    const int s = (int)(bs % Sq);
    const long b = bs / Sq;
    const long lidx = (b * H + h) * Sq + s;

    float M = -INFINITY;
    for (int i = 0; i < n_parts; ++i)
        M = fmaxf(M, p.lse_parts[i][lidx]);

    u32x4 out = {0, 0, 0, 0};
    float lse_out = -INFINITY;
    if (M != -INFINITY) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float L = 0.f;
        for (int i = 0; i < n_parts; ++i) {
            const float w = exp2_fast((p.lse_parts[i][lidx] - M) * kLog2e);
            const u32x4 x = ld_global16(p.o_parts[i] + row * D + c * 8);
            L += w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += w * __builtin_bit_cast(float, x[e] << 16);
                acc[2 * e + 1] += w * __builtin_bit_cast(float, x[e] & 0xffff0000u);
            }
        }
        const float inv = 1.f / L;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            out[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
        lse_out = M + log2_fast(L) * kLn2;
    }
    st_global16(O + row * D + c * 8, out);
    if (c == 0)
        LSE[lidx] = lse_out;
}

template <int D>
hipError_t launch_merge_d(const MergeArgs& a, hipStream_t stream)
{
    MergeKernelArgs p = {};
    for (int i = 0; i < a.n_parts; ++i) {
        p.o_parts[i] = (const uint16_t*)a.o_parts[i];
        p.lse_parts[i] = a.lse_parts[i];
    }
    const long n_rows = (long)a.B * a.Sq * a.H;
    const long threads = n_rows * (D / 8);
    const long blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffffL)
        return hipErrorInvalidConfiguration;
    return launch_kernel(merge_kernel<D>, dim3((unsigned)blocks), dim3(256), stream, p,
                         a.n_parts, a.o, a.lse, a.H, a.Sq, n_rows);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream)
{
    return a.d == 64 ? launch_merge_d<64>(a, stream) : launch_merge_d<128>(a, stream);
}

}  // namespace dit
