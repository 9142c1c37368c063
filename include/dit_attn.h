/*
 * dit_attn.h -- C ABI of the MI355X (gfx950) non-causal attention library for
 * DiT inference: the attention forward pass (O and log-sum-exp), the
 * log-sum-exp merge of partial results over KV chunks, and the
 * per-(head, 128-token block) e4m3 quantiser that feeds the fp8 forward pass.
 *
 * Where the operations come from
 *   "xDiT 项目概述" (intelliparadigm.com), sec. 2.1: DiT inference runs the
 *   whole token sequence at once (prefill-like, compute-bound), with no KV
 *   cache and no paging -- so attention here is dense, non-causal and takes
 *   contiguous Q/K/V.  Sec. 2.2: sequences are long (tens of thousands of
 *   joint text+image/video tokens).  Sec. 3.2 (USP): the ring dimension splits
 *   the sequence into blocks that travel around a ring of GPUs; one GPU's
 *   share is its queries against one KV block at a time, and the partial
 *   results are combined -- dit_attn_merge is that combination.
 *   "AMD、Radeon AI PRO R9700S最大4台で..." (aisoku.org), tuning section and
 *   quick-start flags: attention runs through a dedicated FP8 attention
 *   backend; FP8 changes outputs, so it is checked against fixed seeds.
 *   "生成AI推論を速くするための設計ノート" sec. 3: a block-scaled low-precision
 *   tensor is a payload plus per-block scales; sec. 5: a dedicated kernel for
 *   an op whose structure a general one does not fit; sec. 4: launches with no
 *   host sync or allocation can be captured into a graph.
 *
 * The attention formula is never printed on those pages; this library computes
 * the plain reading, per batch b and head h:
 *     S   = scale * Q K^T                  (no mask, no bias: non-causal)
 *     O   = softmax_rows(S) V
 *     LSE = ln sum_j exp(S_ij)             (natural log, scale included)
 *
 * Conventions shared by every entry point
 *   Layouts: Q, O [B][Sq][H][d]; K, V [B][Skv][H][d]; all contiguous with d
 *   fastest.  LSE [B][H][Sq] fp32.  bf16 is IEEE bfloat16 bits; e4m3 is OCP
 *   E4M3FN (bias 7, max 448, no infinities).
 *   Ownership: the caller owns every buffer.  The library allocates nothing,
 *   keeps no state between calls (dit_attn_fwd_noalloc aside: its static
 *   scratch array, see there), never synchronises, and only enqueues work on
 *   `stream` (0 = the null stream), so every call can be captured into a HIP
 *   graph.  Calls are thread-safe (dit_attn_fwd_noalloc: see there).
 *   Errors: every argument is validated on the host before any HIP call, so an
 *   invalid call returns its status code without touching the device.  A
 *   launch failure returns DIT_ERR_HIP.  Faults inside a kernel surface, as
 *   for any asynchronous HIP work, at the caller's next synchronisation.
 */
#ifndef DIT_ATTN_H
#define DIT_ATTN_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIT_ATTN_VERSION 10301 /* major*10000 + minor*100 + patch */

enum dit_status {
    DIT_OK = 0,
    DIT_ERR_NULL = 1,        /* a required pointer is NULL                         */
    DIT_ERR_SHAPE = 2,       /* B, H, Sq, Skv or S < 1, a size overflows 2^62 B, or
                                one batch of K (or V) exceeds 2^32 - 1 bytes        */
    DIT_ERR_UNSUPPORTED = 3, /* d not 64/128, unknown dtype, n_parts not in 1..16   */
    DIT_ERR_ALIGN = 4,       /* tensor not 16-byte aligned (LSE/scales: 4-byte)    */
    DIT_ERR_VALUE = 5,       /* scale not finite or not > 0                        */
    DIT_ERR_ALIAS = 6,       /* an output overlaps an input it may not overlap     */
    DIT_ERR_HIP = 7,         /* the HIP launch (or device query) reported an error */
    DIT_ERR_WORKSPACE = 8    /* dit_attn_fwd_ws/_acc: workspace NULL, smaller than
                                dit_attn_fwd_workspace_size, not 16-byte aligned,
                                or overlapping a tensor                            */
};

enum dit_dtype {
    DIT_DTYPE_BF16 = 0,
    DIT_DTYPE_FP8_E4M3 = 1
};

/* Block size (tokens) of the e4m3 per-(b, h, block) scales. */
#define DIT_FP8_BLOCK 128

/* An e4m3 tensor with its block scales, as produced by dit_quant_fp8.
 *   data : device, e4m3 bytes [B][S][H][d]
 *   scale: device, fp32 [B][H][ceil(S/128)]; x[b,s,h,c] ~= e4m3(data) * scale[b,h,s/128]
 * The descriptor itself lives in host memory and is read during the call only. */
typedef struct dit_fp8_tensor {
    const void* data;
    const float* scale;
} dit_fp8_tensor_t;

/*
 * dit_attn_fwd -- non-causal attention forward pass, O and LSE.
 *
 *   dtype == DIT_DTYPE_BF16:     q, k, v are device pointers to bf16 tensors.
 *   dtype == DIT_DTYPE_FP8_E4M3: q, k, v each point to a HOST dit_fp8_tensor_t
 *       describing an e4m3 tensor and its block scales.  Q.K^T and P.V run on
 *       fp8 MFMA with fp32 accumulation; the block scales are applied inside
 *       the kernel; P is rounded to e4m3 (relative to the running row maximum)
 *       before P.V; O is divided by the sum of those rounded weights (so it
 *       stays a convex combination of values), LSE uses the unrounded ones.
 *   o:   device, bf16 [B][Sq][H][d] (fp32 result rounded to nearest even).
 *   lse: device, fp32 [B][H][Sq].
 *   d:   64 or 128.  Sq, Skv >= 1 (any value: tails are masked).  One batch of K
 *        (Skv * H * d elements) must fit in 2^32 - 1 bytes.
 *   scale: the softmax scale (e.g. 1/sqrt(d)), finite and > 0; used as given.
 *   o and lse must not overlap q, k, v or each other (DIT_ERR_ALIAS).
 */
int dit_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int Sq, int Skv, int d, float scale, int dtype,
                 hipStream_t stream);

/*
 * dit_attn_fwd_workspace_size / dit_attn_fwd_ws -- the forward pass with
 * caller-provided scratch, used to balance the last wave of workgroups.
 *
 * A launch of dit_attn_fwd runs one workgroup per query tile (bf16: 256 rows
 * for d = 128, one per compute unit at a time, 128 rows for d = 64, two per
 * compute unit; fp8: 128 rows, two per compute unit); when the number of
 * tiles is not a multiple of what the GPU runs at once, the last wave leaves
 * most of the GPU idle.  dit_attn_fwd_ws
 * runs the leftover tiles split over contiguous ranges of the keys instead
 * (the ring dimension of "xDiT 项目概述" sec. 3.2 applied inside one GPU),
 * writes their partial O and LSE to the workspace and combines them with the
 * log-sum-exp merge (as dit_attn_merge does).  Results equal dit_attn_fwd's
 * up to fp32 rounding order (fp8: and the e4m3 rounding of the weights, which
 * a piece takes against its own running maximum).
 *
 * dit_attn_fwd_workspace_size: *bytes = the workspace the call needs for this
 *   shape on the current HIP device (0 if nothing is split: then workspace may
 *   be NULL).  Shape arguments as for dit_attn_fwd; needs a HIP device
 *   (DIT_ERR_HIP if the device query fails).
 * dit_attn_fwd_ws: arguments as dit_attn_fwd, plus
 *   workspace: device memory of workspace_bytes bytes, 16-byte aligned, owned
 *   by the caller, not overlapping any tensor; its contents on entry do not
 *   matter and on return are unspecified.  Calls that may run concurrently
 *   need separate workspaces.
 *   Errors as dit_attn_fwd, plus DIT_ERR_WORKSPACE.  The required size is
 *   checked against the current device after the other arguments.
 */
int dit_attn_fwd_workspace_size(int B, int H, int Sq, int Skv, int d, int dtype, size_t* bytes);

int dit_attn_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Sq, int Skv, int d, float scale, int dtype,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dit_attn_fwd_noalloc -- dit_attn_fwd_ws without a workspace argument and
 * without any allocation: for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The split launch's scratch is a static device array of
 * DIT_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends (its device address is looked up once per device,
 * on the first split call made with that device current).
 *
 *   Arguments and results as dit_attn_fwd_ws (bf16 or fp8), minus the
 *   workspace.  DIT_NOALLOC_SCRATCH_BYTES covers every shape on a GPU of up to
 *   256 compute units; where a shape's split needs more, the call returns
 *   DIT_ERR_WORKSPACE (and enqueues nothing).
 *   Every call on one GPU shares that GPU's scratch array: calls that may
 *   overlap on one GPU (other streams, other host threads) race and must be
 *   serialised by the caller.  Nothing in the array needs clearing between
 *   calls.
 */
#define DIT_NOALLOC_SCRATCH_BYTES (33u << 20)

int dit_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int Sq, int Skv, int d, float scale, int dtype,
                         hipStream_t stream);

/*
 * dit_attn_fwd_acc -- the forward pass over one block of keys, merged into a
 * running result over the key blocks before it: what a rank of ring attention
 * runs each time a KV block arrives ("xDiT 项目概述" sec. 3.2: the ring
 * dimension splits the sequence into blocks passed around the GPUs, and each
 * GPU combines the partial results), without writing partial outputs or
 * running a separate merge.
 *
 *   Arguments as dit_attn_fwd_ws (workspace rules included: the split launch
 *   is used when dit_attn_fwd_workspace_size is not 0), except:
 *   dtype: DIT_DTYPE_BF16, or DIT_DTYPE_FP8_E4M3 with q, k, v host
 *       dit_fp8_tensor_t descriptors as for dit_attn_fwd; an fp8 key block is
 *       a tensor of its own with its own block scales [B][H][ceil(Skv/128)]
 *       (as dit_quant_fp8 writes them for that block), so kv_batch_tokens
 *       must be 0 for fp8 (DIT_ERR_UNSUPPORTED otherwise).
 *   kv_batch_tokens (bf16): tokens between the starts of consecutive batches
 *       in k and v (0: Skv, contiguous).  With B > 1 the key block is usually a
 *       slice [s0, s0 + Skv) of larger [B][S][H][d] tensors: pass k, v offset
 *       by s0 tokens and kv_batch_tokens = S.  Must be 0 or >= Skv (else
 *       DIT_ERR_SHAPE); the batches' extents are checked for aliasing.
 *   o, lse: on entry the running result (bf16 O, fp32 natural-log LSE) over
 *       the earlier key blocks -- a row whose LSE is -inf has no keys yet and
 *       its O is not read (so a first block needs only LSE set to -inf); on
 *       return the result over those keys and this block's, computed as
 *       dit_attn_merge would merge the two, except that this block's O enters
 *       in fp32 (it is never rounded to bf16 on its own).  Any other LSE value
 *       on entry (NaN, +inf) is not supported.
 *   Errors as dit_attn_fwd_ws.
 */
int dit_attn_fwd_acc(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int Sq, int Skv, int d, float scale, int dtype,
                     long long kv_batch_tokens, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * dit_attn_merge -- combine n partial attention results over disjoint key
 * blocks into the result over their union, per (b, s, h) row:
 *     M   = max_c LSE_c
 *     w_c = exp(LSE_c - M)
 *     O   = sum_c w_c O_c / sum_c w_c,     LSE = M + ln sum_c w_c
 * A part whose LSE is -inf has weight 0; if every part is -inf the row gets
 * O = 0 and LSE = -inf.  Accumulation is fp32.
 *
 *   o_parts, lse_parts: HOST arrays of n_parts device pointers to bf16
 *       [B][Sq][H][d] partial outputs and fp32 [B][H][Sq] partial LSEs
 *       (exactly what dit_attn_fwd writes).
 *   n_parts: 1..16.
 *   B * Sq * H <= 2^31 - 1 rows (DIT_ERR_SHAPE otherwise; the kernel indexes
 *       rows with 32-bit integers, and a larger part exceeds any one GPU's
 *       memory for either head dimension).
 *   o, lse: device outputs in the same layouts.  o may be exactly o_parts[0]
 *       and lse exactly lse_parts[0] (in-place merge); any other overlap of an
 *       output with an input returns DIT_ERR_ALIAS.
 */
int dit_attn_merge(const void* const* o_parts, const float* const* lse_parts, int n_parts,
                   void* o, float* lse, int B, int H, int Sq, int d, hipStream_t stream);

/*
 * dit_quant_fp8 -- per-(b, h, 128-token block) e4m3 quantisation of a bf16
 * tensor [B][S][H][d].  For each block (the last one may hold S mod 128 tokens):
 *     amax  = max |x| over the block's tokens and all d channels
 *     inv   = fp32(448 / amax),  x8 = e4m3_rne(fp32(x * inv))
 *     scale = fp32(amax / 448)                   (amax == 0: scale 1, x8 = 0)
 * Every fp32 step is a single correctly rounded operation, so the output is
 * bit-reproducible.  Non-finite input: a NaN takes no part in amax and encodes
 * as 0x7F; an infinity makes amax and the block's scale +inf, so the block's
 * finite values encode as (signed) zeros and its infinities as 0x7F; a block
 * whose values are all zero or NaN gets scale 1 and all-zero bytes.
 *   x: device bf16 [B][S][H][d];  x_fp8: device e4m3 [B][S][H][d];
 *   scale: device fp32 [B][H][ceil(S/128)].  Outputs must not overlap x.
 */
int dit_quant_fp8(const void* x, void* x_fp8, float* scale, int B, int H, int S, int d,
                  hipStream_t stream);

/* Static text for a status code ("unknown status" for other values). */
const char* dit_status_string(int status);

/* DIT_ATTN_VERSION of the built library. */
int dit_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIT_ATTN_H */
