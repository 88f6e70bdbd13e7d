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

/* OpenMP threads the oracle runs with. */
int oracle_threads(void);

#ifdef __cplusplus
}
#endif
#endif
