/*
 * oracle.c -- plain, slow, fp64 CPU reference for hybrid paged GQA attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library's compute path may call, link
 * or load this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header, table or constant with the
 * HIP library.
 *
 * What it computes is the plain definition of softmax attention, restricted by
 * the two masks the pages describe (pegainfer issue "[Model] Gemma 4 M1 12B",
 * Description: local sliding-window attention at head_dim 256 and global
 * attention at head_dim 512, GQA with two KV head counts, paged prefill and
 * decode; Core AI card, section "hybrid-pf64/ bundles": block-GQA head mapping
 * and a decode step whose single query attends the whole grown cache).
 *
 *   query position p (absolute, from 0); query head h; KV head kv = floor(h / g)
 *   visible keys  J(p) = { j : lo(p) <= j <= p },
 *                 lo(p) = 0 (global) or max(0, p - W + 1) (local: the last W
 *                 positions, the current one included)
 *   scores        s_j = scale * sum_d q[p,h,d] * K[j,kv,d]
 *   logsumexp     LSE = m + ln sum_j exp(s_j - m),  m = max_j s_j
 *   output        O[p,h,:] = sum_j exp(s_j - LSE) * V[j,kv,:]
 *
 * The softmax is two-pass (max, then sum) with no online rescaling. Inputs are
 * bfloat16 bit patterns widened exactly to double; all arithmetic is double.
 * K and V are contiguous per row (no pages): row r stores tokens
 * [k_start[r], ctx_len[r]) back to back as [token][kv_head][head_dim].
 *
 * The KV append writes new tokens into the paged cache by the layout's own definition (token t
 * of a row in page page_table[row][t / page_size], slot t % page_size, pool laid out
 * [page][kv_head][slot][head_dim]; the pegainfer "[Model] Gemma 4 M2 26B-A4B" plan asks that page
 * offsets come from one checked place), element by element, with no blocking.
 *
 * The FP8 KV pool (the pegainfer "[Model] Gemma 4 M2 26B-A4B" plan's opt-in FP8 KV pool for the
 * sliding family; the vLLM Gemma 4 recipe's "--kv-cache-dtype fp8") stores each K and V element as
 * one byte in the OCP 8-bit floating-point format E4M3 (sign, 4 exponent bits with bias 7, 3
 * mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; the all-ones exponent with
 * all-ones mantissa is NaN; there are no infinities, so the largest finite magnitude is 448).
 * The pages fix neither the format variant nor the scale granularity; the reading taken here is
 * E4M3 with one scale per tensor: the stored element stands for code_value * k_scale (K) or
 * code_value * v_scale (V). Attention over such a pool is the same definition as above with
 * K and V replaced by those exact values. Writing into it rounds the fp32 quotient x / scale
 * to the nearest E4M3 value, ties to the even code, saturating finite magnitudes above 448 to
 * 448 and keeping NaN (another reading: the pages give no rounding rule).
 *
 * The split-KV routine follows the pegainfer "[Model] Gemma 4 M3 31B" plan's
 * split-KV chunk policy in its plainest reading: cut a row's keys at absolute
 * multiples of the split size, attend each piece on its own, then merge the
 * pieces by their logsumexp. It exists only to check that the merge is exact.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <string.h>

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Value of an E4M3 code, from the format's definition (sign, biased exponent, mantissa). */
static double e4m3_value(uint8_t c)
{
    const int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7)
        return NAN;
    const double mag = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

double oracle_e4m3_value(uint8_t code) { return e4m3_value(code); }

uint8_t oracle_e4m3_encode(float x)
{
    const uint8_t sign = signbit(x) ? 0x80 : 0;
    if (isnan(x))
        return sign | 0x7f;
    const double a = fabs((double)x);
    if (a >= 448.0)
        return sign | 0x7e;
    /* nearest of the finite magnitudes (codes 0x00 .. 0x7e); on a tie the even code */
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c <= 0x7e; ++c) {
        const double d = fabs(e4m3_value((uint8_t)c) - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return sign | (uint8_t)best;
}

void oracle_e4m3_encode_n(int64_t n, const float *x, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode(x[i]);
}

/* First key position visible to a query at position p. */
static int64_t visible_lo(int is_global, int window, int64_t p)
{
    if (is_global)
        return 0;
    int64_t lo = p - (int64_t)window + 1;
    return lo > 0 ? lo : 0;
}

typedef struct {
    int is_global, Hq, Hkv, hd, window;
    double scale;
    int B;
    const int32_t *q_lens, *ctx_lens, *k_starts;
    const uint16_t *q, *k, *v;
    int64_t *q_off;   /* [B+1] first query index of each row */
    int64_t *k_off;   /* [B]   first stored token index of each row */
    int fp8;          /* K and V are E4M3 codes (k8, v8) standing for code_value * k_scale / v_scale */
    const uint8_t *k8, *v8;
    double k_scale, v_scale;
} problem;

static int check_and_index(problem *pb)
{
    if (pb->Hq <= 0 || pb->Hkv <= 0 || pb->hd <= 0 || pb->B < 0)
        return ORACLE_BAD_ARG;
    if (pb->Hq % pb->Hkv != 0)
        return ORACLE_BAD_ARG;
    if (!pb->is_global && pb->window < 1)
        return ORACLE_BAD_ARG;
    pb->q_off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(pb->B + 1));
    pb->k_off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(pb->B + 1));
    if (!pb->q_off || !pb->k_off)
        return ORACLE_NO_MEM;
    int64_t qo = 0, ko = 0;
    for (int r = 0; r < pb->B; ++r) {
        int64_t L = pb->ctx_lens[r], C = pb->q_lens[r], k0 = pb->k_starts ? pb->k_starts[r] : 0;
        if (C < 0 || L < C || k0 < 0 || k0 > L)
            return ORACLE_BAD_ARG;
        if (C > 0 && L < 1)
            return ORACLE_BAD_ARG;
        /* every key a query of this row can see must be stored */
        if (C > 0 && visible_lo(pb->is_global, pb->window, L - C) < k0)
            return ORACLE_MISSING_KEYS;
        pb->q_off[r] = qo;
        pb->k_off[r] = ko;
        qo += C;
        ko += L - k0;
    }
    pb->q_off[pb->B] = qo;
    pb->k_off[pb->B] = ko;
    return ORACLE_OK;
}

static int row_of_query(const problem *pb, int64_t t)
{
    int lo = 0, hi = pb->B - 1;
    while (lo < hi) {              /* last row with q_off[row] <= t */
        int mid = (lo + hi + 1) / 2;
        if (pb->q_off[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

/* Element offset of token j's row (KV head kv) of row r in the contiguous K / V arrays. */
static int64_t key_index(const problem *pb, int r, int64_t j, int kv)
{
    int64_t k0 = pb->k_starts ? pb->k_starts[r] : 0;
    return ((pb->k_off[r] + (j - k0)) * pb->Hkv + kv) * (int64_t)pb->hd;
}

/* Attend keys [a, b] (inclusive) of row r for one query vector; two-pass softmax.
 * Writes the normalised output (hd doubles) and returns the logsumexp. */
static double attend_range(const problem *pb, int r, int kv, const double *qv,
                           int64_t a, int64_t b, double *scores, double *o)
{
    const int hd = pb->hd;
    int64_t n = b - a + 1;
    double m = -INFINITY;
    for (int64_t j = a; j <= b; ++j) {
        double dot = 0.0;
        if (pb->fp8) {
            const uint8_t *kr = pb->k8 + key_index(pb, r, j, kv);
            for (int d = 0; d < hd; ++d)
                dot += qv[d] * (e4m3_value(kr[d]) * pb->k_scale);
        } else {
            const uint16_t *kr = pb->k + key_index(pb, r, j, kv);
            for (int d = 0; d < hd; ++d)
                dot += qv[d] * widen_bf16(kr[d]);
        }
        double s = pb->scale * dot;
        scores[j - a] = s;
        if (s > m)
            m = s;
    }
    double sum = 0.0;
    for (int64_t i = 0; i < n; ++i)
        sum += exp(scores[i] - m);
    double lse = m + log(sum);
    for (int d = 0; d < hd; ++d)
        o[d] = 0.0;
    for (int64_t j = a; j <= b; ++j) {
        double w = exp(scores[j - a] - lse);
        if (pb->fp8) {
            const uint8_t *vr = pb->v8 + key_index(pb, r, j, kv);
            for (int d = 0; d < hd; ++d)
                o[d] += w * (e4m3_value(vr[d]) * pb->v_scale);
        } else {
            const uint16_t *vr = pb->v + key_index(pb, r, j, kv);
            for (int d = 0; d < hd; ++d)
                o[d] += w * widen_bf16(vr[d]);
        }
    }
    return lse;
}

/* Every (query, query head) of the problem, in parallel. */
static int attend_problem(problem *pbp, double *out, double *lse)
{
    problem pb = *pbp;
    const int is_global = pb.is_global, Hq = pb.Hq, Hkv = pb.Hkv, hd = pb.hd, window = pb.window, B = pb.B;
    const int32_t *q_lens = pb.q_lens, *ctx_lens = pb.ctx_lens;
    const uint16_t *q = pb.q;
    int rc = check_and_index(&pb);
    if (rc != ORACLE_OK) {
        free(pb.q_off);
        free(pb.k_off);
        return rc;
    }
    const int g = Hq / Hkv;
    const int64_t T = pb.q_off[B];
    int64_t max_keys = 1;
    for (int r = 0; r < B; ++r)
        if (ctx_lens[r] > max_keys)
            max_keys = ctx_lens[r];
    int failed = 0;
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)max_keys);
        double *qv = (double *)malloc(sizeof(double) * (size_t)hd);
        int ok = scores && qv;
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
        {
#pragma omp for schedule(dynamic, 4)
            for (int64_t item = 0; item < T * Hq; ++item) {
                if (!ok)
                    continue;
                int64_t t = item / Hq;
                int h = (int)(item % Hq);
                int r = row_of_query(&pb, t);
                int64_t p = (int64_t)ctx_lens[r] - q_lens[r] + (t - pb.q_off[r]);
                int kv = h / g;
                for (int d = 0; d < hd; ++d)
                    qv[d] = widen_bf16(q[(t * Hq + h) * (int64_t)hd + d]);
                lse[t * Hq + h] = attend_range(&pb, r, kv, qv, visible_lo(is_global, window, p), p,
                                               scores, out + (t * Hq + h) * (int64_t)hd);
            }
        }
        free(scores);
        free(qv);
    }
    free(pb.q_off);
    free(pb.k_off);
    return failed ? ORACLE_NO_MEM : ORACLE_OK;
}

int oracle_attend(int is_global, int Hq, int Hkv, int hd, int window, double scale,
                  int B, const int32_t *q_lens, const int32_t *ctx_lens, const int32_t *k_starts,
                  const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  double *out, double *lse)
{
    problem pb = {is_global, Hq, Hkv, hd, window, scale, B, q_lens, ctx_lens, k_starts,
                  q, k, v ? v : k, NULL, NULL, 0, NULL, NULL, 1.0, 1.0};
    return attend_problem(&pb, out, lse);
}

int oracle_attend_fp8kv(int is_global, int Hq, int Hkv, int hd, int window, double scale,
                        int B, const int32_t *q_lens, const int32_t *ctx_lens, const int32_t *k_starts,
                        const uint16_t *q, const uint8_t *k, const uint8_t *v, double k_scale, double v_scale,
                        double *out, double *lse)
{
    if (!k || !v || !(k_scale > 0.0) || !(v_scale > 0.0) || isinf(k_scale) || isinf(v_scale))
        return ORACLE_BAD_ARG;
    problem pb = {is_global, Hq, Hkv, hd, window, scale, B, q_lens, ctx_lens, k_starts,
                  q, NULL, NULL, NULL, NULL, 1, k, v, k_scale, v_scale};
    return attend_problem(&pb, out, lse);
}

/* Merge pieces by logsumexp: M = max lse_i, LSE = M + ln sum_i exp(lse_i - M),
 * O = sum_i exp(lse_i - LSE) o_i. Pieces with lse = -inf are empty and skipped; with no
 * non-empty piece O = 0 and LSE = -inf. Returns LSE. */
static double merge_parts(int np, int hd, const double *lse_parts, const double *o_parts, double *o)
{
    double M = -INFINITY;
    for (int i = 0; i < np; ++i)
        if (lse_parts[i] > M)
            M = lse_parts[i];
    for (int d = 0; d < hd; ++d)
        o[d] = 0.0;
    if (M == -INFINITY)
        return -INFINITY;
    double sum = 0.0;
    for (int i = 0; i < np; ++i)
        if (lse_parts[i] != -INFINITY)
            sum += exp(lse_parts[i] - M);
    double L = M + log(sum);
    for (int i = 0; i < np; ++i) {
        if (lse_parts[i] == -INFINITY)
            continue;
        double w = exp(lse_parts[i] - L);
        for (int d = 0; d < hd; ++d)
            o[d] += w * o_parts[i * (int64_t)hd + d];
    }
    return L;
}

int oracle_merge(int64_t n_rows, int n_parts, int hd, const double *lse_parts, const double *o_parts,
                 double *out, double *lse)
{
    if (n_rows < 0 || n_parts < 1 || hd < 1)
        return ORACLE_BAD_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r)
        lse[r] = merge_parts(n_parts, hd, lse_parts + r * n_parts, o_parts + r * n_parts * (int64_t)hd,
                             out + r * (int64_t)hd);
    return ORACLE_OK;
}

int oracle_decode_split(int is_global, int Hq, int Hkv, int hd, int window, double scale,
                        int B, const int32_t *ctx_lens, const int32_t *k_starts,
                        const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        int split_tokens, double *out, double *lse)
{
    if (split_tokens < 1)
        return ORACLE_BAD_ARG;
    int32_t *ones = (int32_t *)malloc(sizeof(int32_t) * (size_t)(B > 0 ? B : 1));
    if (!ones)
        return ORACLE_NO_MEM;
    for (int r = 0; r < B; ++r)
        ones[r] = 1;
    problem pb = {is_global, Hq, Hkv, hd, window, scale, B, ones, ctx_lens, k_starts,
                  q, k, v ? v : k, NULL, NULL, 0, NULL, NULL, 1.0, 1.0};
    int rc = check_and_index(&pb);
    if (rc != ORACLE_OK) {
        free(pb.q_off);
        free(pb.k_off);
        free(ones);
        return rc;
    }
    const int g = Hq / Hkv;
    int64_t max_keys = 1;
    for (int r = 0; r < B; ++r)
        if (ctx_lens[r] > max_keys)
            max_keys = ctx_lens[r];
    int failed = 0;
#pragma omp parallel
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)max_keys);
        double *qv = (double *)malloc(sizeof(double) * (size_t)hd);
        double *part_o = (double *)malloc(sizeof(double) * (size_t)hd);
        int64_t max_parts = max_keys / split_tokens + 2;
        double *lse_parts = (double *)malloc(sizeof(double) * (size_t)max_parts);
        double *o_parts = (double *)malloc(sizeof(double) * (size_t)(max_parts * hd));
        int ok = scores && qv && part_o && lse_parts && o_parts;
        if (!ok) {
#pragma omp atomic write
            failed = 1;
        }
        {
#pragma omp for schedule(dynamic, 1)
            for (int64_t item = 0; item < (int64_t)B * Hq; ++item) {
                if (!ok)
                    continue;
                int r = (int)(item / Hq), h = (int)(item % Hq), kv = h / g;
                int64_t p = (int64_t)ctx_lens[r] - 1;
                int64_t lo = visible_lo(is_global, window, p);
                for (int d = 0; d < hd; ++d)
                    qv[d] = widen_bf16(q[item * (int64_t)hd + d]);
                /* pieces: keys [s*S, (s+1)*S) intersected with [lo, p] */
                int np = 0;
                for (int64_t s = lo / split_tokens; s * split_tokens <= p; ++s) {
                    int64_t a = s * split_tokens, b = a + split_tokens - 1;
                    if (a < lo) a = lo;
                    if (b > p) b = p;
                    lse_parts[np] = attend_range(&pb, r, kv, qv, a, b, scores, o_parts + np * (int64_t)hd);
                    ++np;
                }
                lse[item] = merge_parts(np, hd, lse_parts, o_parts, out + item * (int64_t)hd);
            }
        }
        free(scores);
        free(qv);
        free(part_o);
        free(lse_parts);
        free(o_parts);
    }
    free(pb.q_off);
    free(pb.k_off);
    free(ones);
    return failed ? ORACLE_NO_MEM : ORACLE_OK;
}

int oracle_layer_is_global(int layer, int n_layers)
{
    /* Five local layers, then one global, repeated; the stack must end on a global layer. */
    if (n_layers < 1 || n_layers % 6 != 0 || layer < 0 || layer >= n_layers)
        return -1;
    return (layer + 1) % 6 == 0 ? 1 : 0;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* E4M3 code of the fp32 quotient x / scale (scale > 0). The sign is x's: for a number it is the
 * quotient's sign anyway, and a NaN x stores NaN with its own sign bit. */
static uint8_t encode_quotient(float x, float scale)
{
    if (isnan(x))
        return signbit(x) ? 0xff : 0x7f;
    return oracle_e4m3_encode(x / scale);
}

/* Destination of the new tokens: bf16 pools (k_pool, v_pool) or E4M3 pools (k_pool8, v_pool8) with
 * their scales. */
typedef struct {
    uint16_t *k_pool, *v_pool;
    uint8_t *k_pool8, *v_pool8;
    float k_scale, v_scale;
} append_dst;

static int64_t append_rows(int Hkv, int hd, int page_size, int B, const int32_t *cu_new, const int32_t *ctx_lens,
                           const int32_t *page_table, int pt_stride, int64_t num_pages, int max_new,
                           const uint16_t *k_new, const uint16_t *v_new, const append_dst *dst_pools)
{
    const int fp8 = dst_pools->k_pool8 != NULL;
    int64_t skipped = 0;
    for (int r = 0; r < B; ++r) {
        const int64_t n = (int64_t)cu_new[r + 1] - cu_new[r];
        /* A malformed row fails closed as a whole: more new tokens than the cache holds, or more
         * than the call's declared bound max_new (when max_new >= 0). */
        if ((int64_t)ctx_lens[r] < n || (max_new >= 0 && n > max_new)) {
            skipped += n;
            continue;
        }
        for (int64_t i = 0; i < n; ++i) {
            const int64_t t = (int64_t)ctx_lens[r] - n + i; /* absolute position of the new token */
            const int64_t logical = t < 0 ? -1 : t / page_size;
            if (t < 0 || logical >= pt_stride) {
                ++skipped;
                continue;
            }
            const int64_t page = page_table[(int64_t)r * pt_stride + logical];
            if (page < 0 || page >= num_pages) {
                ++skipped;
                continue;
            }
            const int64_t slot = t % page_size;
            const int64_t src_tok = (int64_t)cu_new[r] + i;
            for (int kv = 0; kv < Hkv; ++kv)
                for (int d = 0; d < hd; ++d) {
                    const int64_t dst = ((page * Hkv + kv) * page_size + slot) * hd + d;
                    const int64_t src = (src_tok * Hkv + kv) * hd + d;
                    if (fp8) {
                        dst_pools->k_pool8[dst] = encode_quotient((float)widen_bf16(k_new[src]), dst_pools->k_scale);
                        if (v_new)
                            dst_pools->v_pool8[dst] =
                                encode_quotient((float)widen_bf16(v_new[src]), dst_pools->v_scale);
                    } else {
                        dst_pools->k_pool[dst] = k_new[src];
                        if (v_new)
                            dst_pools->v_pool[dst] = v_new[src];
                    }
                }
        }
    }
    return skipped;
}

int64_t oracle_kv_append(int Hkv, int hd, int page_size, int B, const int32_t *cu_new, const int32_t *ctx_lens,
                         const int32_t *page_table, int pt_stride, int64_t num_pages, int max_new,
                         const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool, uint16_t *v_pool)
{
    if (Hkv <= 0 || hd <= 0 || page_size <= 0 || B < 0 || pt_stride <= 0 || num_pages <= 0 || !cu_new ||
        !ctx_lens || !page_table || !k_new || !k_pool || (v_new && !v_pool))
        return ORACLE_BAD_ARG;
    const append_dst d = {k_pool, v_pool, NULL, NULL, 1.0f, 1.0f};
    return append_rows(Hkv, hd, page_size, B, cu_new, ctx_lens, page_table, pt_stride, num_pages, max_new, k_new,
                       v_new, &d);
}

int64_t oracle_kv_append_fp8(int Hkv, int hd, int page_size, int B, const int32_t *cu_new, const int32_t *ctx_lens,
                             const int32_t *page_table, int pt_stride, int64_t num_pages, int max_new,
                             const uint16_t *k_new, const uint16_t *v_new, float k_scale, float v_scale,
                             uint8_t *k_pool, uint8_t *v_pool)
{
    if (Hkv <= 0 || hd <= 0 || page_size <= 0 || B < 0 || pt_stride <= 0 || num_pages <= 0 || !cu_new ||
        !ctx_lens || !page_table || !k_new || !k_pool || (v_new && !v_pool) || !(k_scale > 0.0f) ||
        !(v_scale > 0.0f) || isinf(k_scale) || isinf(v_scale))
        return ORACLE_BAD_ARG;
    const append_dst d = {NULL, NULL, k_pool, v_pool, k_scale, v_scale};
    return append_rows(Hkv, hd, page_size, B, cu_new, ctx_lens, page_table, pt_stride, num_pages, max_new, k_new,
                       v_new, &d);
}
