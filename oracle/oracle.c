/*
 * oracle.c -- plain, slow, fp64 CPU oracle for non-causal multi-head attention
 * (O and log-sum-exp), the log-sum-exp merge of partial results over KV chunks,
 * and the per-(head, 128-token block) e4m3 quantiser.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library.  The product path
 * (the HIP library under attention_non_causal_amd/) never links, loads or calls
 * it, and this file shares no code, header, table or constant with that path.
 *
 * What the pages fix, and what is a reading (the pages never print a formula):
 *  - "xDiT 项目概述" (intelliparadigm.com), sec. 2.1: DiT inference is
 *    prefill-like over the whole token sequence; there is no KV cache and no
 *    paging, so attention is dense and non-causal.  Sec. 3.2 (USP): the ring
 *    dimension splits the sequence into blocks that circulate around a ring, so
 *    one GPU's queries meet the keys one block at a time and the partial results
 *    must be combined -- that combination is the merge below.
 *  - The attention itself is read as textbook scaled-dot-product softmax
 *    attention per head, with no bias, no mask, no dropout (plainest reading).
 *  - LSE is the natural log of sum_j exp(scale * q . k_j), max added back.
 *  - "AMD、Radeon AI PRO R9700S最大4台で..." (aisoku.org), section on tuning:
 *    FP8 runs natively but changes outputs.  The e4m3 format is OCP E4M3FN
 *    (bias 7, max 448, no infinities, NaN = S.1111.111) -- a reading; the page
 *    only says FP8.
 *  - "生成AI推論を速くするための設計ノート" sec. 3: a block-scaled low-precision
 *    tensor is payload + per-block scale; here one fp32 scale per (b, h, block
 *    of 128 tokens).
 *
 * Arithmetic: every sum is fp64 in plain sequential order; bf16 inputs are
 * decoded exactly.  The forward pass is the two-pass definition (max, then
 * sum and weighted sum), not an online/tiled reformulation.
 *
 * Parallelism: OpenMP over independent (b, h, query row) outputs only; no
 * reduction is split across threads, so results do not depend on the thread
 * count.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- number formats ---------------------------------------------------- */

double oracle_bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP OFP8 E4M3FN decode: 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinity. */
double oracle_e4m3_decode(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Round-to-nearest-even to e4m3 with saturation to +-448 for finite values
 * beyond the largest normal.  NaN maps to 0x7F. */
uint8_t oracle_e4m3_encode(double x)
{
    uint8_t sign = 0;
    double a;
    if (isnan(x))
        return 0x7F;
    if (signbit(x)) {
        sign = 0x80;
        a = -x;
    } else {
        a = x;
    }
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: integer multiples of 2^-9; rint() is RNE under the
         * default rounding mode.  A result of 8 is the smallest normal, whose
         * encoding 0x08 is exactly the integer 8. */
        double q = rint(ldexp(a, 9));
        return (uint8_t)(sign | (uint8_t)q);
    }
    {
        int e2;
        double fr = frexp(a, &e2);          /* a = fr * 2^e2, fr in [0.5, 1) */
        int e = e2 - 1;                     /* a = (2*fr) * 2^e, 2*fr in [1, 2) */
        double mant = rint((2.0 * fr - 1.0) * 8.0);
        int code;
        if (mant >= 8.0) {
            mant = 0.0;
            e += 1;
        }
        code = ((e + 7) << 3) | (int)mant;
        if (code > 0x7E)
            code = 0x7E;
        return (uint8_t)(sign | (uint8_t)code);
    }
}

/* ---- forward ----------------------------------------------------------- */

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* One (b, h, query row) of the definition:
 *   s_j = scale * sum_c q[c] k_j[c]
 *   m   = max_j s_j
 *   l   = sum_j exp(s_j - m)
 *   O   = sum_j exp(s_j - m) v_j / l
 *   LSE = m + ln l                                                         */
static void attn_row(const double* qrow, const double* kh, const double* vh,
                     long kv_stride, int Skv, int d, double scale,
                     double* s, double* orow, double* lse_out)
{
    double m = -INFINITY, l = 0.0;
    int j, c;
    for (j = 0; j < Skv; ++j) {
        const double* kj = kh + (long)j * kv_stride;
        double acc = 0.0;
        for (c = 0; c < d; ++c)
            acc += qrow[c] * kj[c];
        s[j] = scale * acc;
        if (s[j] > m)
            m = s[j];
    }
    for (c = 0; c < d; ++c)
        orow[c] = 0.0;
    for (j = 0; j < Skv; ++j) {
        const double* vj = vh + (long)j * kv_stride;
        double p = exp(s[j] - m);
        l += p;
        for (c = 0; c < d; ++c)
            orow[c] += p * vj[c];
    }
    for (c = 0; c < d; ++c)
        orow[c] /= l;
    *lse_out = m + log(l);
}

static double* decode_bf16_array(const uint16_t* x, long n)
{
    double* y = (double*)malloc((size_t)n * sizeof(double));
    long i;
    if (!y)
        return NULL;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        y[i] = oracle_bf16_to_double(x[i]);
    return y;
}

int oracle_attn_fwd_f64(const double* q, const double* k, const double* v,
                        double* o, double* lse,
                        int B, int H, int Sq, int Skv, int d, double scale,
                        const int* rows, int n_rows)
{
    long total;
    long t;
    int nr = rows ? n_rows : Sq;
    int err = 0;
    if (B <= 0 || H <= 0 || Sq <= 0 || Skv <= 0 || d <= 0 || nr < 0)
        return -1;
    if (rows) {
        int i;
        for (i = 0; i < n_rows; ++i)
            if (rows[i] < 0 || rows[i] >= Sq)
                return -1;
    }
    total = (long)B * H * nr;
#pragma omp parallel reduction(| : err)
    {
        double* s = (double*)malloc((size_t)Skv * sizeof(double));
        if (!s) {
            err |= 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (t = 0; t < total; ++t) {
                /* t enumerates (b, r, h) with h fastest. */
                int h = (int)(t % H);
                long br = t / H;
                int r = (int)(br % nr);
                int b = (int)(br / nr);
                int i = rows ? rows[r] : r;
                const double* qrow = q + (((long)b * Sq + i) * H + h) * d;
                const double* kh = k + ((long)b * Skv * H + h) * d;
                const double* vh = v + ((long)b * Skv * H + h) * d;
                double* orow = o + (((long)b * nr + r) * H + h) * d;
                double* l_out = lse + ((long)b * H + h) * nr + r;
                attn_row(qrow, kh, vh, (long)H * d, Skv, d, scale, s, orow, l_out);
            }
            free(s);
        }
    }
    return err ? -2 : 0;
}

int oracle_attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         double* o, double* lse,
                         int B, int H, int Sq, int Skv, int d, double scale,
                         const int* rows, int n_rows)
{
    double *qd, *kd, *vd;
    int rc;
    if (B <= 0 || H <= 0 || Sq <= 0 || Skv <= 0 || d <= 0)
        return -1;
    qd = decode_bf16_array(q, (long)B * Sq * H * d);
    kd = decode_bf16_array(k, (long)B * Skv * H * d);
    vd = decode_bf16_array(v, (long)B * Skv * H * d);
    if (!qd || !kd || !vd) {
        free(qd);
        free(kd);
        free(vd);
        return -2;
    }
    rc = oracle_attn_fwd_f64(qd, kd, vd, o, lse, B, H, Sq, Skv, d, scale, rows, n_rows);
    free(qd);
    free(kd);
    free(vd);
    return rc;
}

/* ---- merge ------------------------------------------------------------- */

/* Combine n partial results (O_c, LSE_c), each the attention of the same
 * queries over a disjoint block of keys:
 *   M   = max_c LSE_c                 (all -inf: O = 0, LSE = -inf)
 *   w_c = exp(LSE_c - M)
 *   O   = sum_c w_c O_c / sum_c w_c
 *   LSE = M + ln sum_c w_c
 * Layouts: o_parts [n][B][Sq][H][d], lse_parts [n][B][H][Sq].             */
int oracle_attn_merge(const double* o_parts, const double* lse_parts, int n,
                      double* o, double* lse, int B, int H, int Sq, int d)
{
    long rows_total, t;
    long o_part_stride, l_part_stride;
    if (n <= 0 || B <= 0 || H <= 0 || Sq <= 0 || d <= 0)
        return -1;
    rows_total = (long)B * Sq * H;
    o_part_stride = rows_total * d;
    l_part_stride = rows_total;
#pragma omp parallel for schedule(static)
    for (t = 0; t < rows_total; ++t) {
        int h = (int)(t % H);
        long bs = t / H;
        int s = (int)(bs % Sq);
        int b = (int)(bs / Sq);
        long lidx = ((long)b * H + h) * Sq + s;
        double M = -INFINITY, L = 0.0;
        int c, e;
        double* orow = o + t * d;
        for (c = 0; c < n; ++c) {
            double x = lse_parts[c * l_part_stride + lidx];
            if (x > M)
                M = x;
        }
        for (e = 0; e < d; ++e)
            orow[e] = 0.0;
        if (M == -INFINITY) {
            lse[lidx] = -INFINITY;
            continue;
        }
        for (c = 0; c < n; ++c) {
            double w = exp(lse_parts[c * l_part_stride + lidx] - M);
            const double* oc = o_parts + c * o_part_stride + t * d;
            L += w;
            for (e = 0; e < d; ++e)
                orow[e] += w * oc[e];
        }
        for (e = 0; e < d; ++e)
            orow[e] /= L;
        lse[lidx] = M + log(L);
    }
    return 0;
}

/* ---- per-(b, h, 128-token block) e4m3 quantiser ------------------------ */

/* For each (b, h, token block t of at most 128 tokens):
 *   amax  = max |x| over the block's tokens and all d channels
 *   inv   = fp32(448 / amax), y = fp32(x * inv), q = sat_rne_e4m3(y)
 *   scale = fp32(amax / 448)            (amax = 0: scale = 1, q = 0)
 * so that x ~= decode(q) * scale.  x is bf16 [B,S,H,d]; q is e4m3 bytes in
 * the same layout; scale is fp32 [B,H,ceil(S/128)].  The fp32 steps are
 * single correctly rounded IEEE operations, written as such here.
 * Non-finite input follows from these steps as written: a NaN fails the
 * comparison with amax and so takes no part in it, and encodes as 0x7F; an
 * infinity makes amax infinite, inv = 0 and scale = +inf, so finite values
 * encode as signed zeros and the infinity (inf * 0 = NaN) as 0x7F.          */
int oracle_quant_fp8(const uint16_t* x, uint8_t* q, float* scale,
                     int B, int H, int S, int d)
{
    int nblk;
    long total, t;
    if (B <= 0 || H <= 0 || S <= 0 || d <= 0)
        return -1;
    nblk = (S + ORACLE_FP8_BLOCK - 1) / ORACLE_FP8_BLOCK;
    total = (long)B * H * nblk;
#pragma omp parallel for schedule(static)
    for (t = 0; t < total; ++t) {
        int blk = (int)(t % nblk);
        long bh = t / nblk;
        int h = (int)(bh % H);
        int b = (int)(bh / H);
        int s0 = blk * ORACLE_FP8_BLOCK;
        int s1 = s0 + ORACLE_FP8_BLOCK < S ? s0 + ORACLE_FP8_BLOCK : S;
        double amax = 0.0;
        volatile float inv, sc;
        int s, c;
        for (s = s0; s < s1; ++s) {
            const uint16_t* row = x + (((long)b * S + s) * H + h) * d;
            for (c = 0; c < d; ++c) {
                double a = fabs(oracle_bf16_to_double(row[c]));
                if (a > amax)
                    amax = a;
            }
        }
        if (amax == 0.0) {
            sc = 1.0f;
            for (s = s0; s < s1; ++s)
                memset(q + (((long)b * S + s) * H + h) * d, 0, (size_t)d);
        } else {
            float famax = (float)amax; /* exact: amax is a bf16 value */
            inv = 448.0f / famax;
            sc = famax / 448.0f;
            for (s = s0; s < s1; ++s) {
                long base = (((long)b * S + s) * H + h) * d;
                for (c = 0; c < d; ++c) {
                    volatile float y = (float)oracle_bf16_to_double(x[base + c]) * inv;
                    q[base + c] = oracle_e4m3_encode((double)y);
                }
            }
        }
        scale[t] = sc;
    }
    return 0;
}

/* Dequantise e4m3 bytes with their block scales back to fp64:
 *   x[b,s,h,c] = decode(q[b,s,h,c]) * scale[b,h,s/128]                      */
int oracle_dequant_fp8(const uint8_t* q, const float* scale, double* x,
                       int B, int H, int S, int d)
{
    int nblk;
    long total, t;
    if (B <= 0 || H <= 0 || S <= 0 || d <= 0)
        return -1;
    nblk = (S + ORACLE_FP8_BLOCK - 1) / ORACLE_FP8_BLOCK;
    total = (long)B * S * H;
#pragma omp parallel for schedule(static)
    for (t = 0; t < total; ++t) {
        int h = (int)(t % H);
        long bs = t / H;
        int s = (int)(bs % S);
        int b = (int)(bs / S);
        double sc = (double)scale[((long)b * H + h) * nblk + s / ORACLE_FP8_BLOCK];
        int c;
        for (c = 0; c < d; ++c)
            x[t * d + c] = oracle_e4m3_decode(q[t * d + c]) * sc;
    }
    return 0;
}
