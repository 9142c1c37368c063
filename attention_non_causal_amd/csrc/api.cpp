// api.cpp -- the C ABI of libditattn: argument validation and dispatch.
//
// Every check runs on the host before any HIP call, so an invalid call
// returns its status without touching the device (and can be exercised on a
// machine without a GPU).  The library allocates nothing and never
// synchronises; a valid call only enqueues kernels on the caller's stream.
#include "dit_attn.h"

#include <math.h>
#include <stdint.h>

#include "launch.hpp"

namespace {

constexpr int64_t kMaxBytes = int64_t(1) << 62;
constexpr int64_t kMaxKvBytesPerBatch = (int64_t(1) << 32) - 1;

bool aligned(const void* p, uintptr_t a)
{
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Product of positive factors, or -1 once it exceeds kMaxBytes.
int64_t checked_bytes(std::initializer_list<int64_t> factors)
{
    int64_t n = 1;
    for (int64_t f : factors) {
        if (f <= 0 || n > kMaxBytes / f)
            return -1;
        n *= f;
    }
    return n;
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range(const void* p, int64_t bytes)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + static_cast<uintptr_t>(bytes)};
}

bool overlap(Range a, Range b)
{
    return a.lo < b.hi && b.lo < a.hi;
}

int map_hip(hipError_t e)
{
    return e == hipSuccess ? DIT_OK : DIT_ERR_HIP;
}

}  // namespace

extern "C" {

int dit_version(void)
{
    return DIT_ATTN_VERSION;
}

const char* dit_status_string(int status)
{
    switch (status) {
    case DIT_OK:
        return "ok";
    case DIT_ERR_NULL:
        return "a required pointer is NULL";
    case DIT_ERR_SHAPE:
        return "a dimension is < 1 or a tensor size overflows";
    case DIT_ERR_UNSUPPORTED:
        return "unsupported head dim, dtype or number of parts";
    case DIT_ERR_ALIGN:
        return "a tensor pointer is misaligned (16 bytes; LSE and scales 4 bytes)";
    case DIT_ERR_VALUE:
        return "scale must be finite and > 0";
    case DIT_ERR_ALIAS:
        return "an output overlaps an input";
    case DIT_ERR_HIP:
        return "HIP kernel launch failed";
    case DIT_ERR_WORKSPACE:
        return "workspace missing, too small, misaligned or overlapping a tensor";
    default:
        return "unknown status";
    }
}

}  // extern "C"

namespace {

// Compute units of the current device (the split plan depends on them).
int current_cu_count(int* n_cu)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return DIT_ERR_HIP;
    return DIT_OK;
}

// Shape checks shared by the forward entry points.
int check_fwd_shape(int B, int H, int Sq, int Skv, int d, int dtype)
{
    if (dtype != DIT_DTYPE_BF16 && dtype != DIT_DTYPE_FP8_E4M3)
        return DIT_ERR_UNSUPPORTED;
    if (d != 64 && d != 128)
        return DIT_ERR_UNSUPPORTED;
    const int64_t esz = dtype == DIT_DTYPE_BF16 ? 2 : 1;
    const int64_t q_bytes = checked_bytes({B, Sq, H, d, esz});
    const int64_t kv_bytes = checked_bytes({B, Skv, H, d, esz});
    const int64_t o_bytes = checked_bytes({B, Sq, H, d, 2});
    const int64_t lse_bytes = checked_bytes({B, H, Sq, 4});
    if (q_bytes < 0 || kv_bytes < 0 || o_bytes < 0 || lse_bytes < 0)
        return DIT_ERR_SHAPE;
    if (kv_bytes / B > kMaxKvBytesPerBatch)
        return DIT_ERR_SHAPE;
    return DIT_OK;
}

}  // namespace

namespace dit {

// dit_attn_fwd, dit_attn_fwd_ws, dit_attn_fwd_acc and dit_attn_fwd_noalloc;
// with_ws selects the split launch, acc the merge into the running result held
// in o, lse, and kv_batch_tokens (acc only; 0: Skv) the distance between
// batches of k, v.
int fwd_entry(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int Sq, int Skv, int d, float scale, int dtype, bool with_ws, void* ws,
              size_t ws_bytes, bool acc, long long kv_batch_tokens, hipStream_t stream,
              void* (*resolve_ws)(int* status))
{
    if (!q || !k || !v || !o || !lse)
        return DIT_ERR_NULL;
    if (dtype != DIT_DTYPE_BF16 && dtype != DIT_DTYPE_FP8_E4M3)
        return DIT_ERR_UNSUPPORTED;
    // fp8 key blocks are tensors of their own (with their own block scales):
    // no batch stride
    if (acc && dtype != DIT_DTYPE_BF16 && kv_batch_tokens != 0)
        return DIT_ERR_UNSUPPORTED;
    if (d != 64 && d != 128)
        return DIT_ERR_UNSUPPORTED;

    dit::FwdArgs a = {};
    const int64_t esz = dtype == DIT_DTYPE_BF16 ? 2 : 1;
    const int64_t q_bytes = checked_bytes({B, Sq, H, d, esz});
    const int64_t kv_bytes = checked_bytes({B, Skv, H, d, esz});
    const int64_t o_bytes = checked_bytes({B, Sq, H, d, 2});
    const int64_t lse_bytes = checked_bytes({B, H, Sq, 4});
    if (q_bytes < 0 || kv_bytes < 0 || o_bytes < 0 || lse_bytes < 0)
        return DIT_ERR_SHAPE;
    // K and V of one batch are addressed with 32-bit buffer offsets
    if (kv_bytes / B > kMaxKvBytesPerBatch)
        return DIT_ERR_SHAPE;
    // batches of K and V kv_batch_tokens apart: they span (B-1) * that + Skv tokens
    if (kv_batch_tokens < 0 || (kv_batch_tokens > 0 && kv_batch_tokens < Skv) ||
        kv_batch_tokens > 0x7fffffffLL)
        return DIT_ERR_SHAPE;
    const int64_t kv_span = kv_batch_tokens == 0
                                ? kv_bytes
                                : checked_bytes({(int64_t)(B - 1) * kv_batch_tokens + Skv, H, d, esz});
    if (kv_span < 0)
        return DIT_ERR_SHAPE;
    if (!(isfinite(scale) && scale > 0.f))
        return DIT_ERR_VALUE;

    if (dtype == DIT_DTYPE_BF16) {
        a.q = q;
        a.k = k;
        a.v = v;
    } else {
        const auto* qd = static_cast<const dit_fp8_tensor_t*>(q);
        const auto* kd = static_cast<const dit_fp8_tensor_t*>(k);
        const auto* vd = static_cast<const dit_fp8_tensor_t*>(v);
        if (!qd->data || !qd->scale || !kd->data || !kd->scale || !vd->data || !vd->scale)
            return DIT_ERR_NULL;
        a.q = qd->data;
        a.k = kd->data;
        a.v = vd->data;
        a.q_scale = qd->scale;
        a.k_scale = kd->scale;
        a.v_scale = vd->scale;
        if (!aligned(a.q_scale, 4) || !aligned(a.k_scale, 4) || !aligned(a.v_scale, 4))
            return DIT_ERR_ALIGN;
    }
    if (!aligned(a.q, 16) || !aligned(a.k, 16) || !aligned(a.v, 16) || !aligned(o, 16) ||
        !aligned(lse, 4))
        return DIT_ERR_ALIGN;

    const Range ro = range(o, o_bytes), rl = range(lse, lse_bytes);
    const Range inputs[] = {range(a.q, q_bytes), range(a.k, kv_span), range(a.v, kv_span)};
    for (const Range& in : inputs)
        if (overlap(ro, in) || overlap(rl, in))
            return DIT_ERR_ALIAS;
    if (overlap(ro, rl))
        return DIT_ERR_ALIAS;
    if (dtype == DIT_DTYPE_FP8_E4M3) {
        const int64_t nq = (Sq + DIT_FP8_BLOCK - 1) / DIT_FP8_BLOCK;
        const int64_t nk = (Skv + DIT_FP8_BLOCK - 1) / DIT_FP8_BLOCK;
        const Range scales[] = {range(a.q_scale, int64_t(B) * H * nq * 4),
                                range(a.k_scale, int64_t(B) * H * nk * 4),
                                range(a.v_scale, int64_t(B) * H * nk * 4)};
        for (const Range& sc : scales)
            if (overlap(ro, sc) || overlap(rl, sc))
                return DIT_ERR_ALIAS;
    }

    a.o = o;
    a.lse = lse;
    a.B = B;
    a.H = H;
    a.Sq = Sq;
    a.Skv = Skv;
    a.d = d;
    a.scale = scale;
    a.acc = acc ? 1 : 0;
    a.kv_batch_tokens = (long)kv_batch_tokens;

    dit::FwdSplit split = {};
    if (with_ws) {
        int n_cu = 0;
        const int st = current_cu_count(&n_cu);
        if (st != DIT_OK)
            return st;
        split = dtype == DIT_DTYPE_BF16 ? dit::plan_fwd_bf16_split(B, H, Sq, Skv, d, n_cu)
                                        : dit::plan_fwd_fp8_split(B, H, Sq, Skv, d, n_cu);
        if (split.n_tail > 0) {
            if (ws_bytes < split.ws_bytes)
                return DIT_ERR_WORKSPACE;
            if (resolve_ws) {
                int rs = DIT_OK;
                ws = resolve_ws(&rs);
                if (rs != DIT_OK)
                    return rs;
            }
            if (!ws || !aligned(ws, 16))
                return DIT_ERR_WORKSPACE;
            const Range rw = range(ws, (int64_t)split.ws_bytes);
            for (const Range& in : inputs)
                if (overlap(rw, in))
                    return DIT_ERR_WORKSPACE;
            if (overlap(rw, ro) || overlap(rw, rl))
                return DIT_ERR_WORKSPACE;
            if (dtype == DIT_DTYPE_FP8_E4M3) {
                const int64_t nq = (Sq + DIT_FP8_BLOCK - 1) / DIT_FP8_BLOCK;
                const int64_t nk = (Skv + DIT_FP8_BLOCK - 1) / DIT_FP8_BLOCK;
                if (overlap(rw, range(a.q_scale, int64_t(B) * H * nq * 4)) ||
                    overlap(rw, range(a.k_scale, int64_t(B) * H * nk * 4)) ||
                    overlap(rw, range(a.v_scale, int64_t(B) * H * nk * 4)))
                    return DIT_ERR_WORKSPACE;
            }
            a.ws = ws;
        }
    }
    if (dtype != DIT_DTYPE_BF16)
        return map_hip(dit::launch_fwd_fp8(a, split, stream));
    return map_hip(dit::launch_fwd_bf16(a, split, stream));
}

}  // namespace dit

extern "C" {

int dit_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int Sq, int Skv, int d, float scale, int dtype, hipStream_t stream)
{
    return dit::fwd_entry(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype, false, nullptr, 0,
                          false, 0, stream, nullptr);
}

int dit_attn_fwd_workspace_size(int B, int H, int Sq, int Skv, int d, int dtype, size_t* bytes)
{
    if (!bytes)
        return DIT_ERR_NULL;
    const int st = check_fwd_shape(B, H, Sq, Skv, d, dtype);
    if (st != DIT_OK)
        return st;
    *bytes = 0;
    int n_cu = 0;
    const int hs = current_cu_count(&n_cu);
    if (hs != DIT_OK)
        return hs;
    *bytes = dtype == DIT_DTYPE_BF16 ? dit::plan_fwd_bf16_split(B, H, Sq, Skv, d, n_cu).ws_bytes
                                     : dit::plan_fwd_fp8_split(B, H, Sq, Skv, d, n_cu).ws_bytes;
    return DIT_OK;
}

int dit_attn_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int Sq, int Skv, int d, float scale, int dtype, void* workspace,
                    size_t workspace_bytes, hipStream_t stream)
{
    return dit::fwd_entry(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype, true, workspace,
                          workspace_bytes, false, 0, stream, nullptr);
}

int dit_attn_fwd_acc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int Sq, int Skv, int d, float scale, int dtype,
                     long long kv_batch_tokens, void* workspace, size_t workspace_bytes,
                     hipStream_t stream)
{
    return dit::fwd_entry(q, k, v, o, lse, B, H, Sq, Skv, d, scale, dtype, true, workspace,
                          workspace_bytes, true, kv_batch_tokens, stream, nullptr);
}

int dit_attn_merge(const void* const* o_parts, const float* const* lse_parts, int n_parts,
                   void* o, float* lse, int B, int H, int Sq, int d, hipStream_t stream)
{
    if (!o_parts || !lse_parts || !o || !lse)
        return DIT_ERR_NULL;
    if (n_parts < 1 || n_parts > dit::kMaxMergeParts)
        return DIT_ERR_UNSUPPORTED;
    for (int i = 0; i < n_parts; ++i)
        if (!o_parts[i] || !lse_parts[i])
            return DIT_ERR_NULL;
    if (d != 64 && d != 128)
        return DIT_ERR_UNSUPPORTED;
    const int64_t o_bytes = checked_bytes({B, Sq, H, d, 2});
    const int64_t lse_bytes = checked_bytes({B, H, Sq, 4});
    // the kernel indexes (b, s, h) rows with 32-bit integers
    if (o_bytes < 0 || lse_bytes < 0 || (int64_t)B * Sq * H > INT32_MAX)
        return DIT_ERR_SHAPE;
    if (!aligned(o, 16) || !aligned(lse, 4))
        return DIT_ERR_ALIGN;
    for (int i = 0; i < n_parts; ++i)
        if (!aligned(o_parts[i], 16) || !aligned(lse_parts[i], 4))
            return DIT_ERR_ALIGN;

    // An output may coincide exactly with an input of its own kind (every
    // input of a row is read before that row is written); any other overlap
    // is rejected.
    const Range ro = range(o, o_bytes), rl = range(lse, lse_bytes);
    if (overlap(ro, rl))
        return DIT_ERR_ALIAS;
    for (int i = 0; i < n_parts; ++i) {
        const Range po = range(o_parts[i], o_bytes), pl = range(lse_parts[i], lse_bytes);
        if (overlap(ro, po) && o_parts[i] != o)
            return DIT_ERR_ALIAS;
        if (overlap(rl, pl) && lse_parts[i] != lse)
            return DIT_ERR_ALIAS;
        if (overlap(ro, pl) || overlap(rl, po))
            return DIT_ERR_ALIAS;
    }

    dit::MergeArgs a = {};
    for (int i = 0; i < n_parts; ++i) {
        a.o_parts[i] = o_parts[i];
        a.lse_parts[i] = lse_parts[i];
    }
    a.n_parts = n_parts;
    a.o = o;
    a.lse = lse;
    a.B = B;
    a.H = H;
    a.Sq = Sq;
    a.d = d;
    return map_hip(dit::launch_merge(a, stream));
}

int dit_quant_fp8(const void* x, void* x_fp8, float* scale, int B, int H, int S, int d,
                  hipStream_t stream)
{
    if (!x || !x_fp8 || !scale)
        return DIT_ERR_NULL;
    if (d != 64 && d != 128)
        return DIT_ERR_UNSUPPORTED;
    const int64_t x_bytes = checked_bytes({B, S, H, d, 2});
    const int64_t x8_bytes = checked_bytes({B, S, H, d, 1});
    const int64_t nblk = S > 0 ? (S + DIT_FP8_BLOCK - 1) / DIT_FP8_BLOCK : 0;
    const int64_t sc_bytes = checked_bytes({B, H, nblk, 4});
    if (x_bytes < 0 || x8_bytes < 0 || sc_bytes < 0)
        return DIT_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(x_fp8, 16) || !aligned(scale, 4))
        return DIT_ERR_ALIGN;
    const Range rx = range(x, x_bytes), r8 = range(x_fp8, x8_bytes), rs = range(scale, sc_bytes);
    if (overlap(rx, r8) || overlap(rx, rs) || overlap(r8, rs))
        return DIT_ERR_ALIAS;
    return map_hip(dit::launch_quant_fp8(x, x_fp8, scale, B, H, S, d, stream));
}

}  // extern "C"
