// Internal launch interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gattn {

struct DecodeArgs {
    const uint16_t *q;
    const void *k_pool;  // bf16, or E4M3 bytes for the FP8 kernel
    const void *v_pool;
    const int32_t *page_table;
    const int32_t *ctx_lens;
    float *o_part;     // per-split partials (several splits per row)
    float *lse_part;
    uint16_t *out;     // final outputs (one split per row)
    float *lse;
    int64_t num_pages;
    int pt_stride;
    int num_q_heads, num_kv_heads, group;
    int is_global, window;
    int split_tokens;  // keys per split
    int n_slots;       // splits per row the grid covers
    int max_ctx;
    float scale_log2;  // softmax scale times log2(e) (times k_scale for FP8 pools)
    float v_scale;     // FP8 pools: the V scale (multiplies the normalised output)
};

struct PrefillArgs {
    const uint16_t *q;
    const uint16_t *k_pool;
    const uint16_t *v_pool;
    const int32_t *page_table;
    const int32_t *cu_q;
    const int32_t *ctx_lens;
    uint16_t *out;
    float *lse;
    int64_t num_pages;
    int pt_stride;
    int num_q_heads, num_kv_heads, group;
    int is_global, window;
    int max_q;
    float scale_log2;
};

struct AppendArgs {
    const uint16_t *k_new;
    const uint16_t *v_new;   // null: only K is written (V is the K cache)
    void *k_pool;            // bf16, or E4M3 bytes for the FP8 kernel
    void *v_pool;
    const int32_t *page_table;
    const int32_t *cu_new;
    const int32_t *ctx_lens;
    int32_t *status;         // may be null
    int64_t num_pages;
    int pt_stride;
    int num_kv_heads;
    int max_new;
    float k_scale, v_scale;  // FP8 pools: stored code = E4M3(value / scale)
};

hipError_t launch_kv_append(const AppendArgs &a, int head_dim, int batch, bool fp8, hipStream_t stream);

hipError_t launch_decode_split(const DecodeArgs &a, int head_dim, bool kv_shared, int batch,
                               hipStream_t stream);

// Decode over E4M3 pools (head_dim 256 with separate K and V pools, or head_dim 512).
// Whether the decode launch for this shape merges a row's split slots itself (head_dim 256,
// two or three slots; FP8 pools only for at most one (row, KV head) per CU), so that no
// separate merge follows.
bool decode_merges_slots(int head_dim, bool fp8, int n_slots, int64_t rows_x_kv_heads);

// Decode graph capture (graphs.cpp): begin capturing on a new private stream of the current device;
// end the capture into an instantiated graph (*exec, NULL on failure) and free the stream; launch
// and free an instantiated graph.
hipError_t graph_capture_begin(hipStream_t *s);
hipError_t graph_capture_end(hipStream_t s, void **exec);
hipError_t graph_launch(void *exec, hipStream_t s);
void graph_free(void *exec);

hipError_t launch_decode_split_fp8(const DecodeArgs &a, int head_dim, bool kv_shared, int batch,
                                   hipStream_t stream);

// Which split slots of a row a decode filled (those past its last key hold lse = -inf): with it the
// merge reads only those outputs. ctx_lens null: every slot may be non-empty.
struct CombineRows {
    const int32_t *ctx_lens = nullptr;
    int split_tokens = 0, is_global = 1, window = 0, max_ctx = 0;
};

hipError_t launch_combine(int batch, int num_q_heads, int head_dim, int num_splits, const float *o_part,
                          const float *lse_part, uint16_t *out, float *lse, hipStream_t stream,
                          const CombineRows &rows = CombineRows());

hipError_t launch_prefill(const PrefillArgs &a, int head_dim, bool kv_shared, int batch,
                          hipStream_t stream);

// Device address and size of the current device's copy of the no-allocation decode's scratch
// (looked up on the first call per device, then cached).
hipError_t noalloc_scratch(void **ptr, size_t *bytes);

}  // namespace gattn
