// launch.hpp -- internal launchers behind the C ABI (not part of the public
// header).  Arguments are validated by the caller (api.cpp) before any launch.
#pragma once

#include <hip/hip_runtime.h>

namespace dit {

struct FwdArgs {
    const void* q;         // bf16 [B][Sq][H][d]  or e4m3 bytes for the fp8 path
    const void* k;         // bf16 [B][Skv][H][d] or e4m3
    const void* v;         // bf16 [B][Skv][H][d] or e4m3
    const float* q_scale;  // fp8 path: fp32 [B][H][ceil(Sq/128)]
    const float* k_scale;  // fp8 path: fp32 [B][H][ceil(Skv/128)]
    const float* v_scale;  // fp8 path: fp32 [B][H][ceil(Skv/128)]
    void* o;               // bf16 [B][Sq][H][d]
    float* lse;            // fp32 [B][H][Sq]
    int B, H, Sq, Skv, d;
    float scale;
    void* ws;              // workspace of the split launch (see FwdSplit)
    int acc;               // 1: merge into the running (O, LSE) held in o, lse (bf16 only)
    long kv_batch_tokens;  // tokens between consecutive batches of k, v (bf16 path; 0: Skv)
};

// Split plan of a forward launch (split.hip): the first n_main query tiles run
// over all keys, the last n_tail are split into nsplit pieces over the keys,
// whose partial results need ws_bytes of workspace (n_tail == 0: no split, no
// workspace).
constexpr int kMaxSplit = 16;

struct FwdSplit {
    int n_main, nsplit, n_tail;
    size_t ws_bytes;
};

constexpr int kMaxMergeParts = 16;

struct MergeArgs {
    const void* o_parts[kMaxMergeParts];
    const float* lse_parts[kMaxMergeParts];
    int n_parts;
    void* o;
    float* lse;
    int B, H, Sq, d;
};

// n_blocks query tiles of `rows` rows over n_kt key tiles, wg_per_cu
// workgroups resident per CU; a piece's partial result takes floats_per_row
// fp32 values per row.
FwdSplit plan_split(long n_blocks, long n_kt, int rows, int wg_per_cu, int n_cu,
                    int floats_per_row);
// Merge the pieces: ws_o [piece][rows][d] normalised O, ws_lse [piece][rows]
// natural-log LSE, ws_w [piece][rows] the log of the sum each O was
// normalised by (nullptr: the same as ws_lse).
hipError_t launch_split_merge(const FwdArgs& a, const FwdSplit& sp, int rows, int n_qtiles,
                              const float* ws_o, const float* ws_lse, const float* ws_w,
                              hipStream_t stream);

FwdSplit plan_fwd_bf16_split(int B, int H, int Sq, int Skv, int d, int n_cu);
// head size 128 (fwd_bf16_d128.hip; plan_fwd_bf16_split and launch_fwd_bf16
// dispatch to these)
FwdSplit plan_fwd_bf16_d128_split(int B, int H, int Sq, int Skv, int n_cu);
hipError_t launch_fwd_bf16_d128(const FwdArgs& a, const FwdSplit& split, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdArgs& a, const FwdSplit& split, hipStream_t stream);
FwdSplit plan_fwd_fp8_split(int B, int H, int Sq, int Skv, int d, int n_cu);
hipError_t launch_fwd_fp8(const FwdArgs& a, const FwdSplit& split, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
// The validated forward entry shared by dit_attn_fwd, _ws, _acc and _noalloc
// (api.cpp): with_ws selects the split launch (scratch ws of ws_bytes), acc
// the merge into the running result, kv_batch_tokens the batch distance of k, v.
// resolve_ws (may be null): called for the scratch address, once every other
// argument has been validated and only when the launch is split.
int fwd_entry(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int Sq, int Skv, int d, float scale, int dtype, bool with_ws, void* ws,
              size_t ws_bytes, bool acc, long long kv_batch_tokens, hipStream_t stream,
              void* (*resolve_ws)(int* status));

hipError_t launch_quant_fp8(const void* x, void* x8, float* scale, int B, int H, int S, int d,
                            hipStream_t stream);

}  // namespace dit
