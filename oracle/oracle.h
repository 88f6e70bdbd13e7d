/*
 * oracle.h -- fp64 CPU reference for hybrid paged GQA attention.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg. The HIP library never includes or links it.
 *
 * Arrays hold bfloat16 bit patterns (uint16_t). Row r of a batch has ctx_lens[r]
 * tokens in its cache (the current step's included) and q_lens[r] queries at
 * positions ctx_lens[r] - q_lens[r] + i. Its keys are stored contiguously for
 * tokens [k_starts[r], ctx_lens[r]) (k_starts may be NULL: all from 0) as
 * [token][num_kv_heads][head_dim]; rows follow each other. Queries are
 * [query][num_q_heads][head_dim], rows following each other. v may be NULL or
 * equal to k when V reads the K cache.
 */
#ifndef GATTN_ORACLE_H
#define GATTN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_OK = 0, ORACLE_BAD_ARG = -1, ORACLE_MISSING_KEYS = -2, ORACLE_NO_MEM = -3 };

/* out: [sum q_lens][Hq][hd] doubles; lse: [sum q_lens][Hq] doubles (natural log). */
int oracle_attend(int is_global, int Hq, int Hkv, int hd, int window, double scale,
                  int B, const int32_t *q_lens, const int32_t *ctx_lens, const int32_t *k_starts,
                  const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  double *out, double *lse);

/* One decode query per row, keys cut at absolute multiples of split_tokens, each
 * piece attended alone, pieces merged by logsumexp. out: [B][Hq][hd]; lse: [B][Hq]. */
int oracle_decode_split(int is_global, int Hq, int Hkv, int hd, int window, double scale,
                        int B, const int32_t *ctx_lens, const int32_t *k_starts,
                        const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        int split_tokens, double *out, double *lse);

/* Logsumexp merge of n_parts pieces per row (empty pieces have lse = -inf).
 * lse_parts: [n_rows][n_parts]; o_parts: [n_rows][n_parts][hd]; out: [n_rows][hd]; lse: [n_rows]. */
int oracle_merge(int64_t n_rows, int n_parts, int hd, const double *lse_parts, const double *o_parts,
                 double *out, double *lse);

/* 1 if layer is global, 0 if local, -1 if n_layers is not a whole number of
 * five-local-one-global groups (the stack must end on a global layer). */
int oracle_layer_is_global(int layer, int n_layers);

/* KV append, the plain definition of the paged layout: row r's n_r = cu_new[r+1] - cu_new[r] new
 * tokens sit at positions t = ctx_lens[r] - n_r + i; token t of row r is stored in page
 * page_table[r][t / page_size], slot t % page_size, as pool[page][kv_head][slot][head_dim]. For
 * every such token whose position fits the table and whose page id is in [0, num_pages), copies
 * its [Hkv][hd] K row (and V row when v_new is not NULL) into the pools; all other pool values
 * stay. A row with ctx_lens[r] < n_r, or with n_r > max_new when max_new >= 0 (the call's declared
 * bound on n_r), is malformed and writes nothing (fail closed). Returns the number of tokens
 * skipped (malformed row, position beyond the table, page id out of range), or ORACLE_BAD_ARG. */
int64_t oracle_kv_append(int Hkv, int hd, int page_size, int B, const int32_t *cu_new, const int32_t *ctx_lens,
                         const int32_t *page_table, int pt_stride, int64_t num_pages, int max_new,
                         const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool, uint16_t *v_pool);

/* FP8 KV pool: K and V hold OCP E4M3 codes (one byte per element, same [token][Hkv][hd] layout as
 * above) standing for code_value * k_scale and code_value * v_scale (one scale per tensor, both
 * positive and finite). Same definition and outputs as oracle_attend. */
int oracle_attend_fp8kv(int is_global, int Hq, int Hkv, int hd, int window, double scale,
                        int B, const int32_t *q_lens, const int32_t *ctx_lens, const int32_t *k_starts,
                        const uint16_t *q, const uint8_t *k, const uint8_t *v, double k_scale, double v_scale,
                        double *out, double *lse);

/* Value of an E4M3 code (NaN for 0x7f and 0xff). */
double oracle_e4m3_value(uint8_t code);

/* Nearest E4M3 code to x, ties to the even code; finite magnitudes above 448 give +-448, NaN gives
 * 0x7f with x's sign bit. */
uint8_t oracle_e4m3_encode(float x);
void oracle_e4m3_encode_n(int64_t n, const float *x, uint8_t *out);

/* oracle_kv_append into E4M3 pools: each element is stored as oracle_e4m3_encode of the fp32
 * quotient bf16_value / scale (k_scale for K, v_scale for V); a NaN value stores NaN with its own
 * sign bit. */
int64_t oracle_kv_append_fp8(int Hkv, int hd, int page_size, int B, const int32_t *cu_new, const int32_t *ctx_lens,
                             const int32_t *page_table, int pt_stride, int64_t num_pages, int max_new,
                             const uint16_t *k_new, const uint16_t *v_new, float k_scale, float v_scale,
                             uint8_t *k_pool, uint8_t *v_pool);

/* OpenMP threads the oracle runs with. */
int oracle_threads(void);

#ifdef __cplusplus
}
#endif
#endif
