/*
 * gattn.h -- hybrid paged GQA attention for AMD Instinct MI355X (gfx950): public C ABI.
 *
 * What the library computes. Gemma-4-style attention for one layer over a paged
 * KV cache, for two layer families (pegainfer issue "[Model] Gemma 4 M1 12B",
 * Description):
 *   - local:  sliding-window attention; a query at position p sees keys
 *             max(0, p - window + 1) .. p (the last `window` positions, itself
 *             included); head_dim 256 and a 1024-token window in Gemma 4 31B;
 *   - global: full causal attention (keys 0 .. p); head_dim 512 with fewer KV
 *             heads (4 against 32 query heads at 31B, Core AI card, section
 *             "hybrid-pf64/ bundles"), optionally with V read from the K cache
 *             ("K and V projection sharing", same Description).
 * Query head h reads KV head floor(h / (num_q_heads / num_kv_heads)) (the
 * block-GQA mapping named in the hybrid-pf64 numerics-gate paragraph). For every
 * (query, query head) the library returns the softmax-weighted sum of V and the
 * natural-log logsumexp of the scaled scores:
 *   s_j = scale * q . k_j,  LSE = ln sum_j exp(s_j),  O = sum_j exp(s_j - LSE) v_j.
 *
 * Data types. bf16 arrays are passed as uint16_t bit patterns (bfloat16,
 * round-to-nearest-even when the library produces them). LSE and split partials
 * are fp32. All arithmetic on the device accumulates in fp32. The opt-in FP8 KV
 * pool (gattn_decode_fp8kv, gattn_kv_append_fp8) holds one-byte E4M3 codes in the
 * same layout, with one scale per tensor.
 *
 * KV pool layout (one pool per layer; K and V have separate pools unless shared):
 *   pool[num_pages][num_kv_heads][page_size][head_dim] bf16, page_size = 16.
 *   Token t of row r lives in page page_table[r * pt_stride + t / 16], slot
 *   t % 16; its (kv_head, d) element sits at element offset
 *   ((page * num_kv_heads + kv_head) * 16 + t % 16) * head_dim + d.
 *   gattn_kv_offset() is the one checked helper that computes this offset (the
 *   pegainfer "[Model] Gemma 4 M2 26B-A4B" plan routes hand-derived page offsets
 *   through a checked helper). A page-table entry is read only if its page holds
 *   a token the call reads; other entries may hold anything, -1 included.
 *
 * Ownership. The caller allocates every buffer (device memory unless noted) and
 * keeps it alive until the work on `stream` has finished. The library never
 * allocates, frees or synchronises, keeps no mutable global state (apart from
 * gattn_decode_noalloc's per-GPU scratch, below), and is safe to call from
 * several host threads. `stream` is a hipStream_t (NULL = the
 * default stream); every call only enqueues work on it.
 *
 * Errors. Argument errors are detected on the host before anything is enqueued
 * and returned as a gattn_status; the call then has no effect. A failed kernel
 * launch returns GATTN_ERR_HIP. Inconsistent data that only the device can see
 * (a context length outside [1, max_ctx] or beyond the page table, a page id
 * outside [0, num_pages) for a page that holds a visible token) never faults:
 * the affected row's outputs are written as NaN (fail closed). No C++
 * exception crosses this interface.
 */
#ifndef GATTN_H
#define GATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GATTN_ABI_VERSION 1
#define GATTN_PAGE_SIZE 16
/* Size of the per-GPU device array that holds gattn_decode_noalloc's split partials. */
#define GATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 * 1024 * 1024)

enum gattn_family { GATTN_LOCAL = 0, GATTN_GLOBAL = 1 };

enum gattn_status {
    GATTN_OK = 0,
    GATTN_ERR_NULL_PTR = 1,             /* a required pointer is NULL */
    GATTN_ERR_BAD_SHAPE = 2,            /* negative or inconsistent sizes */
    GATTN_ERR_UNSUPPORTED = 3,          /* valid but not served: head_dim, page size, group size, ... */
    GATTN_ERR_WORKSPACE_TOO_SMALL = 4,  /* workspace_bytes < gattn_decode_workspace_bytes() */
    GATTN_ERR_BAD_SPLIT = 5,            /* split_tokens not 0 and not a positive multiple of 16 */
    GATTN_ERR_HIP = 6                   /* a HIP launch failed */
};

/*
 * One layer's geometry. Served: head_dim 256 or 512; page_size 16;
 * num_q_heads a multiple of num_kv_heads with group num_q_heads/num_kv_heads
 * between 1 and 16; local layers need window >= 1 (global layers ignore it);
 * kv_shared 0 or 1; scale finite (Gemma 4 uses 1.0; 1/sqrt(head_dim) is the
 * textbook value). Anything else returns GATTN_ERR_UNSUPPORTED or BAD_SHAPE.
 */
typedef struct gattn_layer {
    int32_t family;        /* GATTN_LOCAL or GATTN_GLOBAL */
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t window;        /* local: keys visible to a query, itself included */
    int32_t page_size;     /* must be 16 */
    int32_t kv_shared;     /* 1: V is read from the K pool (v_pool must equal k_pool) */
    float scale;           /* multiplies q . k before the softmax */
} gattn_layer;

/* Library ABI version (GATTN_ABI_VERSION of the build). */
int gattn_abi_version(void);

/* Static text for a gattn_status value. */
const char *gattn_status_str(int status);

/*
 * Layer schedule of a Gemma 4 decoder stack: five local layers then one global
 * layer, repeated, so that the last layer is global (pegainfer "[Model] Gemma 4
 * M3 31B", Description and Acceptance Criteria: 60 layers, five-to-one pattern,
 * final-global-layer assertion). Returns GATTN_LOCAL or GATTN_GLOBAL, or -1 if
 * layer is outside [0, n_layers) or n_layers is not a positive multiple of 6.
 */
int gattn_layer_family(int layer, int n_layers);

/*
 * The checked page-offset helper. Host-only: page_table_host is host memory,
 * [rows][pt_stride] int32. Returns the element offset of element 0 of
 * (row, token, kv_head) in a pool of num_pages pages, or -1 if any index is out
 * of range (row, token beyond the table, kv_head, or a page id outside
 * [0, num_pages)).
 */
int64_t gattn_kv_offset(const gattn_layer *layer, const int32_t *page_table_host, int rows,
                        int pt_stride, int row, int token, int kv_head, int64_t num_pages);

/*
 * Split-KV decode workspace size in bytes for a call with these arguments, or 0
 * if the arguments are invalid. The workspace holds per-split partials
 * (fp32 o[batch][num_q_heads][slots][head_dim] followed by fp32
 * lse[batch][num_q_heads][slots]). When a call needs a single split per row the
 * size is 0 bytes and the workspace pointer may be NULL: the split kernel then
 * writes the outputs itself. The size depends only on the arguments, so a
 * caller can allocate it once for its largest call (fixed-capacity scratch, as
 * the pegainfer "[Model] Gemma 4 M2 26B-A4B" description asks for graph-safe
 * use).
 */
size_t gattn_decode_workspace_bytes(const gattn_layer *layer, int batch, int max_ctx, int split_tokens);

/*
 * Single-token decode with split-KV flash-decoding and a logsumexp combine
 * (pegainfer "[Model] Gemma 4 M3 31B", Proposed Plan: decode graph buckets and
 * split-KV chunk policy; Core AI card, "--metal-sdpa" section: flash-decode
 * kernel with a split factor).
 *
 *   q          [batch][num_q_heads][head_dim] bf16: one query per row, at
 *              position ctx_lens[r] - 1.
 *   k_pool     KV pool (layout above); v_pool likewise, or equal to k_pool when
 *              layer->kv_shared (then V is never read separately).
 *   num_pages  pages in each pool (bounds every page id the device reads).
 *   page_table [batch][pt_stride] int32 (device memory).
 *   ctx_lens   [batch] int32 (device memory): tokens in the cache including the
 *              current one; must be in [1, max_ctx] and fit the page table.
 *   max_ctx    host-side upper bound of ctx_lens; sets the grid, so the call
 *              enqueues the same work for any ctx_lens (HIP-graph capturable).
 *   split_tokens  keys per split, a positive multiple of 16, or 0 for one
 *              split per row. Split boundaries are absolute multiples of
 *              split_tokens from token 0, so results do not depend on the batch.
 *   workspace  at least gattn_decode_workspace_bytes(...) bytes (may be NULL if
 *              that is 0).
 *   out        [batch][num_q_heads][head_dim] bf16.
 *   lse        [batch][num_q_heads] fp32, natural log.
 * Enqueues the split kernel, then (when a row can have several splits) the
 * combine kernel, on `stream`; at head_dim 256 with bf16 pools and two or three
 * split slots per row (a local row's window over 512-token splits, say) one
 * kernel runs all of a row's slots and merges them with the combine's arithmetic,
 * with the same bits. The workspace size is the same either way.
 */
int gattn_decode(const gattn_layer *layer, const uint16_t *q, const uint16_t *k_pool,
                 const uint16_t *v_pool, int64_t num_pages, const int32_t *page_table, int pt_stride,
                 const int32_t *ctx_lens, int batch, int max_ctx, int split_tokens, void *workspace,
                 size_t workspace_bytes, uint16_t *out, float *lse, void *stream);

/*
 * gattn_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. It runs gattn_decode's kernels with the split partials
 * in a fixed device array that the library holds on every GPU it runs on
 * (GATTN_NOALLOC_SCRATCH_BYTES, 64 MiB, kept until the process ends), and it
 * allocates nothing: no hipMalloc, hipFree or allocating library routine.
 * Arguments, outputs, errors and results are exactly gattn_decode's, bit for
 * bit. A call whose partials would not fit the array
 * (gattn_decode_workspace_bytes(...) > GATTN_NOALLOC_SCRATCH_BYTES) returns
 * GATTN_ERR_WORKSPACE_TOO_SMALL with nothing enqueued. All calls on one GPU share
 * that GPU's array and it keeps the last call's contents: calls that overlap on
 * one GPU (other streams or host threads) race, and the caller must order them.
 * The first call on a device looks up that device's array address with the
 * device current and caches it; a failed lookup returns GATTN_ERR_HIP.
 */
int gattn_decode_noalloc(const gattn_layer *layer, const uint16_t *q, const uint16_t *k_pool,
                         const uint16_t *v_pool, int64_t num_pages, const int32_t *page_table, int pt_stride,
                         const int32_t *ctx_lens, int batch, int max_ctx, int split_tokens, uint16_t *out,
                         float *lse, void *stream);

/*
 * gattn_decode over an FP8 KV pool (the pegainfer "[Model] Gemma 4 M2 26B-A4B" plan's opt-in
 * FP8 KV pool for the sliding family; the vLLM Gemma 4 recipe serves with "--kv-cache-dtype
 * fp8"). Halves the bytes a decode step reads.
 *
 *   k_pool, v_pool  [num_pages][num_kv_heads][16][head_dim] bytes (the layout above with
 *              one-byte elements), each an OCP E4M3 code: sign, 4 exponent bits (bias 7), 3
 *              mantissa bits, subnormals at exponent 0, 0x7f / 0xff NaN, no infinities,
 *              largest magnitude 448. With layer->kv_shared, v_pool is NULL or equal to k_pool.
 *   k_scale, v_scale  one positive finite scale per tensor: a stored K code c stands for
 *              value(c) * k_scale, a V code for value(c) * v_scale. With layer->kv_shared, V is
 *              the K cache and uses k_scale (v_scale is ignored).
 * Everything else (q, page table, lengths, split policy, workspace size and layout, outputs,
 * errors, fail-closed rows) is exactly as for gattn_decode; the result is attention over the
 * dequantized K and V. Served for head_dim 256 with separate pools (the local family) and for
 * head_dim 512 with or without K=V (the global family: the vLLM recipe's FP8 cache covers every
 * layer); a head_dim 256 layer with kv_shared returns GATTN_ERR_UNSUPPORTED, a scale that is not
 * positive and finite GATTN_ERR_BAD_SHAPE.
 */
int gattn_decode_fp8kv(const gattn_layer *layer, const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                       float k_scale, float v_scale, int64_t num_pages, const int32_t *page_table, int pt_stride,
                       const int32_t *ctx_lens, int batch, int max_ctx, int split_tokens, void *workspace,
                       size_t workspace_bytes, uint16_t *out, float *lse, void *stream);

/* Most bucket sizes one decode graph set holds. */
#define GATTN_MAX_GRAPH_BUCKETS 16

/* A set of captured decode graphs, one per batch-size bucket (opaque). */
typedef struct gattn_decode_graphs gattn_decode_graphs;

/*
 * Decode graph bucket set (pegainfer "[Model] Gemma 4 M3 31B", Proposed Plan: the decode graph
 * bucket set next to the split-KV chunk policy, and graph workspaces in the memory envelope).
 * Captures, once, one HIP graph of gattn_decode per bucket size b: the call over the first b rows
 * of the fixed buffers given here. A serving loop then refreshes those buffers (queries, page
 * table, lengths) in place and replays the smallest bucket that holds its batch with
 * gattn_decode_graphs_launch, which enqueues the captured kernels with no host-side argument
 * work and no allocation.
 *
 *   layer .. split_tokens, workspace, out, lse  as for gattn_decode, sized for the largest
 *              bucket: q, out [max_b][num_q_heads][head_dim], lse [max_b][num_q_heads],
 *              page_table [max_b][pt_stride], ctx_lens [max_b], workspace at least
 *              gattn_decode_workspace_bytes(layer, max_b, max_ctx, split_tokens) bytes. All
 *              device memory, owned by the caller, which must keep it alive (and at the same
 *              addresses) until gattn_decode_graphs_destroy.
 *   buckets    n_buckets batch sizes, strictly increasing, each >= 1 (host memory, copied);
 *              1 <= n_buckets <= GATTN_MAX_GRAPH_BUCKETS; max_b = buckets[n_buckets - 1].
 *   graphs     receives the set (NULL on any error).
 * The graphs are captured on a private stream of the current device and must be launched on a
 * stream of the same device. Every argument is checked (as gattn_decode checks it, for each
 * bucket) before anything is captured; a failure returns that status with nothing enqueued and
 * nothing kept. A capture or instantiation failure returns GATTN_ERR_HIP.
 */
int gattn_decode_graphs_create(const gattn_layer *layer, const uint16_t *q, const uint16_t *k_pool,
                               const uint16_t *v_pool, int64_t num_pages, const int32_t *page_table, int pt_stride,
                               const int32_t *ctx_lens, int max_ctx, int split_tokens, void *workspace,
                               size_t workspace_bytes, uint16_t *out, float *lse, const int32_t *buckets,
                               int n_buckets, gattn_decode_graphs **graphs);

/*
 * The bucket a batch of `batch` rows runs in: the smallest bucket >= batch, or -1 if batch < 1,
 * batch exceeds the largest bucket or graphs is NULL.
 */
int gattn_decode_graphs_bucket(const gattn_decode_graphs *graphs, int batch);

/*
 * Replays the graph of gattn_decode_graphs_bucket(graphs, batch) on `stream`. Rows batch ..
 * bucket - 1 are computed too, from whatever the fixed buffers hold there: the caller either keeps
 * them valid or sets their lengths to 0, which fails them closed (NaN outputs, no K/V read). The
 * bits of rows 0 .. batch - 1 are those of gattn_decode over those rows alone. Launches of one set
 * share its buffers: launches that overlap (other streams or host threads) race, and the caller
 * orders them. Returns GATTN_ERR_NULL_PTR for a NULL set, GATTN_ERR_BAD_SHAPE when no bucket holds
 * the batch, GATTN_ERR_HIP if the launch fails.
 */
int gattn_decode_graphs_launch(const gattn_decode_graphs *graphs, int batch, void *stream);

/* Frees the set's graphs (after their launches have finished); NULL is ignored. */
void gattn_decode_graphs_destroy(gattn_decode_graphs *graphs);

/*
 * Chunked causal prefill (Core AI card, "Contents": a flash-prefill with a
 * query axis and an intra-chunk causal mask; "hybrid-pf64/ bundles": a prefill
 * entrypoint next to decode). Row r has q_len = cu_q[r+1] - cu_q[r] queries at
 * absolute positions ctx_lens[r] - q_len + i; the chunk's own K/V are already in
 * the pool. Rows with q_len 0 are skipped; q_len 1 rows are legal (a mixed
 * step may send decode rows here).
 *
 *   q          [total_q][num_q_heads][head_dim] bf16, rows back to back.
 *   cu_q       [batch + 1] int32 (device memory), cu_q[0] = 0, nondecreasing.
 *   ctx_lens   [batch] int32 (device memory), ctx_lens[r] >= q_len of row r.
 *   max_q      host-side upper bound of every row's q_len (sets the grid).
 *   out        [total_q][num_q_heads][head_dim] bf16.
 *   lse        [total_q][num_q_heads] fp32, natural log.
 * num_q_heads above 16384 returns GATTN_ERR_UNSUPPORTED (a query tile's span of
 * q is addressed with 32-bit offsets).
 * Fail closed on device-side data (pegainfer "[Model] Gemma 4 M3 31B", Proposed
 * Plan: what is not served fails closed): a row whose q_len exceeds max_q or
 * ctx_lens[r], or whose context runs past the page table, gets NaN O and LSE for
 * every one of its queries; a page id outside [0, num_pages) in a page that a
 * block of 128 query rows reads turns that block's outputs NaN. Nothing is read
 * or written outside the row's own queries and the pool.
 */
int gattn_prefill(const gattn_layer *layer, const uint16_t *q, const uint16_t *k_pool,
                  const uint16_t *v_pool, int64_t num_pages, const int32_t *page_table, int pt_stride,
                  const int32_t *cu_q, const int32_t *ctx_lens, int batch, int max_q, uint16_t *out,
                  float *lse, void *stream);

/*
 * Logsumexp merge of split partials: the combine half of split-KV decoding
 * (pegainfer "[Model] Gemma 4 M3 31B", Proposed Plan: the split-KV chunk policy;
 * Core AI card, "--metal-sdpa" section: a flash-decode kernel with a split
 * factor), exported so that partials produced elsewhere (another split schedule,
 * or other devices' shares of one long context) merge the same way.
 * For each (row, head): M = max over splits of lse_s; LSE = M + ln sum_s
 * exp(lse_s - M); O = sum_s exp(lse_s - LSE) o_s. Splits with lse_s = -inf are
 * empty and are skipped: their o_s may hold anything (stale data, NaN) and never
 * enters the result, though the whole o_part buffer may be read. A row whose
 * splits are all empty gets O = 0 and LSE = -inf; a NaN lse_s makes the (row,
 * head) result NaN. The sums run in a fixed order over split indices, so the
 * result depends only on the (row, head)'s own partials.
 *
 *   o_part     [batch][num_q_heads][num_splits][head_dim] fp32, each split's
 *              output already normalised by its own softmax sum.
 *   lse_part   [batch][num_q_heads][num_splits] fp32.
 *   out        [batch][num_q_heads][head_dim] bf16; lse [batch][num_q_heads] fp32.
 * head_dim must be a positive multiple of 4 and at most 1024.
 */
int gattn_combine(int batch, int num_q_heads, int head_dim, int num_splits, const float *o_part,
                  const float *lse_part, uint16_t *out, float *lse, void *stream);

/*
 * KV append: write the K and V rows of newly computed tokens into their pages,
 * the step just before attention (a decode step adds one token per row, a
 * prefill chunk adds the chunk; the pegainfer "[Model] Gemma 4 M2 26B-A4B" plan
 * routes these page writes through the same checked offsets as the reads). Row
 * r appends n_r = cu_new[r+1] - cu_new[r] tokens at absolute positions
 * ctx_lens[r] - n_r + i, i in [0, n_r): ctx_lens counts the cache after the
 * append, exactly as gattn_decode and gattn_prefill then read it. Token t of
 * row r goes to page page_table[r * pt_stride + t / 16], slot t % 16 (layout
 * above). Only those slots are written; every other pool byte keeps its value.
 *
 *   k_new      [total_new][num_kv_heads][head_dim] bf16, rows back to back in
 *              cu_new order.
 *   v_new      same shape, or NULL when layer->kv_shared (V is the K cache).
 *   k_pool     written; v_pool written, or NULL / equal to k_pool when kv_shared.
 *   num_pages  pages in each pool.
 *   page_table [batch][pt_stride] int32 (device memory).
 *   cu_new     [batch + 1] int32 (device memory), cu_new[0] = 0, nondecreasing.
 *   ctx_lens   [batch] int32 (device memory), ctx_lens[r] >= n_r.
 *   max_new    host-side upper bound of every n_r (sets the grid).
 *   status     optional int32 (device memory, may be NULL). Fail closed: a row
 *              with n_r > ctx_lens[r] or n_r > max_new writes none of its
 *              tokens, a token whose position lies beyond the page table or
 *              whose page id is outside [0, num_pages) is not written, and in
 *              either case the kernel ORs 1 into *status. The caller clears it.
 * Rows with n_r = 0 are skipped. Enqueues one kernel on `stream`.
 */
int gattn_kv_append(const gattn_layer *layer, const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                    uint16_t *v_pool, int64_t num_pages, const int32_t *page_table, int pt_stride,
                    const int32_t *cu_new, const int32_t *ctx_lens, int batch, int max_new, int32_t *status,
                    void *stream);

/*
 * gattn_kv_append into an FP8 KV pool (the layout and codes of gattn_decode_fp8kv). Each new bf16
 * element x is stored as the E4M3 code nearest to the fp32 quotient x / scale (IEEE division;
 * k_scale for K, v_scale for V), ties to the even code; quotients of magnitude 448 or more (and
 * infinities) store +-448, NaN stores NaN (0x7f with x's sign). The pages leave the rounding rule
 * open; this one keeps every finite value finite. Rows, positions, the page table, fail-closed
 * behaviour and status are exactly as for gattn_kv_append (with layer->kv_shared only K is
 * written: v_new NULL, v_pool NULL or k_pool, v_scale ignored). Served for the layers
 * gattn_decode_fp8kv serves; others return GATTN_ERR_UNSUPPORTED, a scale that is not positive
 * and finite GATTN_ERR_BAD_SHAPE.
 */
int gattn_kv_append_fp8(const gattn_layer *layer, const uint16_t *k_new, const uint16_t *v_new, uint8_t *k_pool,
                        uint8_t *v_pool, float k_scale, float v_scale, int64_t num_pages, const int32_t *page_table,
                        int pt_stride, const int32_t *cu_new, const int32_t *ctx_lens, int batch, int max_new,
                        int32_t *status, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* GATTN_H */
