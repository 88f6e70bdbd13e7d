// C ABI of the hybrid paged GQA attention library: argument validation, split
// policy, workspace sizing and kernel dispatch. Every check runs on the host
// before any HIP call, so a rejected call has no effect and needs no device.
#include "../../include/gattn.h"

#include <math.h>

#include <new>

#include "kernels.h"

namespace {

constexpr int kMaxGroup = 16;

constexpr int kMaxPrefillQHeads = 16384;

int check_layer(const gattn_layer *l) {
    if (!l)
        return GATTN_ERR_NULL_PTR;
    if (l->family != GATTN_LOCAL && l->family != GATTN_GLOBAL)
        return GATTN_ERR_UNSUPPORTED;
    if (l->num_q_heads <= 0 || l->num_kv_heads <= 0 || l->head_dim <= 0)
        return GATTN_ERR_BAD_SHAPE;
    if (l->num_q_heads % l->num_kv_heads != 0)
        return GATTN_ERR_BAD_SHAPE;
    const int g = l->num_q_heads / l->num_kv_heads;
    if (g > kMaxGroup)
        return GATTN_ERR_UNSUPPORTED;
    if (l->head_dim != 256 && l->head_dim != 512)
        return GATTN_ERR_UNSUPPORTED;
    if (l->page_size != GATTN_PAGE_SIZE)
        return GATTN_ERR_UNSUPPORTED;
    if (l->family == GATTN_LOCAL && l->window < 1)
        return GATTN_ERR_BAD_SHAPE;
    if (l->kv_shared != 0 && l->kv_shared != 1)
        return GATTN_ERR_BAD_SHAPE;
    if (!isfinite(l->scale))
        return GATTN_ERR_BAD_SHAPE;
    return GATTN_OK;
}

struct SplitPlan {
    int split_tokens;  // keys per split
    int n_slots;       // splits per row the grid covers
};

// Split boundaries are absolute multiples of split_tokens from token 0. A local
// row's window [p - W + 1, p] touches at most ceil((W - 1) / S) + 1 of them, so the
// grid only covers that many; a global row can touch every split up to max_ctx.
int plan_splits(const gattn_layer *l, int max_ctx, int split_tokens, SplitPlan *plan) {
    if (split_tokens < 0 || (split_tokens % GATTN_PAGE_SIZE) != 0)
        return GATTN_ERR_BAD_SPLIT;
    const int64_t mc = max_ctx;
    int64_t S = split_tokens == 0 ? (mc + GATTN_PAGE_SIZE - 1) / GATTN_PAGE_SIZE * GATTN_PAGE_SIZE
                                  : (int64_t)split_tokens;
    int64_t n = (mc + S - 1) / S;
    if (l->family == GATTN_LOCAL) {
        // W consecutive keys starting anywhere touch at most ceil((W - 1) / S) + 1 splits.
        const int64_t touched = ((int64_t)l->window - 1 + S - 1) / S + 1;
        if (touched < n)
            n = touched;
    }
    if (S > (1 << 30) || n > (1 << 20))
        return GATTN_ERR_UNSUPPORTED;
    plan->split_tokens = (int)S;
    plan->n_slots = (int)n;
    return GATTN_OK;
}

size_t workspace_for(const gattn_layer *l, int batch, const SplitPlan &p) {
    if (p.n_slots <= 1)
        return 0;
    return (size_t)batch * (size_t)l->num_q_heads * (size_t)p.n_slots * (size_t)(l->head_dim + 1) * 4u;
}

}  // namespace

extern "C" {

int gattn_abi_version(void) { return GATTN_ABI_VERSION; }

const char *gattn_status_str(int status) {
    switch (status) {
    case GATTN_OK: return "ok";
    case GATTN_ERR_NULL_PTR: return "null pointer";
    case GATTN_ERR_BAD_SHAPE: return "bad shape";
    case GATTN_ERR_UNSUPPORTED: return "unsupported";
    case GATTN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case GATTN_ERR_BAD_SPLIT: return "bad split size";
    case GATTN_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
    }
}

int gattn_layer_family(int layer, int n_layers) {
    if (n_layers <= 0 || n_layers % 6 != 0 || layer < 0 || layer >= n_layers)
        return -1;
    return (layer % 6 == 5) ? GATTN_GLOBAL : GATTN_LOCAL;
}

int64_t gattn_kv_offset(const gattn_layer *layer, const int32_t *page_table_host, int rows, int pt_stride,
                        int row, int token, int kv_head, int64_t num_pages) {
    if (check_layer(layer) != GATTN_OK || !page_table_host || rows <= 0 || pt_stride <= 0)
        return -1;
    if (row < 0 || row >= rows || token < 0 || kv_head < 0 || kv_head >= layer->num_kv_heads)
        return -1;
    const int logical = token / GATTN_PAGE_SIZE;
    if (logical >= pt_stride)
        return -1;
    const int64_t page = page_table_host[(int64_t)row * pt_stride + logical];
    if (page < 0 || page >= num_pages)
        return -1;
    return ((page * layer->num_kv_heads + kv_head) * GATTN_PAGE_SIZE + token % GATTN_PAGE_SIZE) *
           (int64_t)layer->head_dim;
}

size_t gattn_decode_workspace_bytes(const gattn_layer *layer, int batch, int max_ctx, int split_tokens) {
    if (check_layer(layer) != GATTN_OK || batch < 0 || max_ctx < 1)
        return 0;
    SplitPlan p;
    if (plan_splits(layer, max_ctx, split_tokens, &p) != GATTN_OK)
        return 0;
    return workspace_for(layer, batch, p);
}

}  // extern "C"

namespace {

// Decode over bf16 pools, or over E4M3 pools (fp8) with their per-tensor scales.
int decode_impl(const gattn_layer *layer, const uint16_t *q, const void *k_pool, const void *v_pool, bool fp8,
                float k_scale, float v_scale, int64_t num_pages, const int32_t *page_table, int pt_stride,
                const int32_t *ctx_lens, int batch, int max_ctx, int split_tokens, void *workspace,
                size_t workspace_bytes, uint16_t *out, float *lse, void *stream, bool noalloc = false,
                bool check_only = false) {
    int rc = check_layer(layer);
    if (rc != GATTN_OK)
        return rc;
    if (fp8) {
        if (layer->head_dim == 256 && layer->kv_shared)
            return GATTN_ERR_UNSUPPORTED;
        if (!(k_scale > 0.0f) || !isfinite(k_scale))
            return GATTN_ERR_BAD_SHAPE;
        if (layer->kv_shared)
            v_scale = k_scale;  // V is the K cache: its codes carry the K scale
        else if (!(v_scale > 0.0f) || !isfinite(v_scale))
            return GATTN_ERR_BAD_SHAPE;
    }
    if (batch < 0 || max_ctx < 1 || pt_stride < 1 || num_pages < 1)
        return GATTN_ERR_BAD_SHAPE;
    if ((int64_t)pt_stride * GATTN_PAGE_SIZE < (int64_t)max_ctx)
        return GATTN_ERR_BAD_SHAPE;
    if (!q || !k_pool || !page_table || !ctx_lens || !out || !lse)
        return GATTN_ERR_NULL_PTR;
    if (layer->kv_shared) {
        if (v_pool && v_pool != k_pool)
            return GATTN_ERR_BAD_SHAPE;
        v_pool = k_pool;
    } else if (!v_pool) {
        return GATTN_ERR_NULL_PTR;
    }
    SplitPlan plan;
    rc = plan_splits(layer, max_ctx, split_tokens, &plan);
    if (rc != GATTN_OK)
        return rc;
    const size_t need = workspace_for(layer, batch, plan);
    if (noalloc) {
        // the partials go to this device's fixed scratch array (looked up after every check)
        if (need > GATTN_NOALLOC_SCRATCH_BYTES)
            return GATTN_ERR_WORKSPACE_TOO_SMALL;
        if (batch == 0)
            return GATTN_OK;
        if (need > 0 && gattn::noalloc_scratch(&workspace, &workspace_bytes) != hipSuccess)
            return GATTN_ERR_HIP;
    }
    if (need > workspace_bytes)
        return GATTN_ERR_WORKSPACE_TOO_SMALL;
    if (need > 0 && !workspace)
        return GATTN_ERR_NULL_PTR;
    if (batch == 0 || check_only)
        return GATTN_OK;

    gattn::DecodeArgs a{};
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.page_table = page_table;
    a.ctx_lens = ctx_lens;
    a.num_pages = num_pages;
    a.pt_stride = pt_stride;
    a.num_q_heads = layer->num_q_heads;
    a.num_kv_heads = layer->num_kv_heads;
    a.group = layer->num_q_heads / layer->num_kv_heads;
    a.is_global = layer->family == GATTN_GLOBAL;
    a.window = layer->window;
    a.split_tokens = plan.split_tokens;
    a.n_slots = plan.n_slots;
    a.max_ctx = max_ctx;
    a.scale_log2 = layer->scale * 1.4426950408889634f;
    a.v_scale = 1.0f;
    if (fp8) {
        a.scale_log2 *= k_scale;
        a.v_scale = v_scale;
    }
    a.out = out;
    a.lse = lse;
    if (plan.n_slots > 1) {
        const size_t n_o = (size_t)batch * layer->num_q_heads * plan.n_slots * layer->head_dim;
        a.o_part = (float *)workspace;
        a.lse_part = (float *)workspace + n_o;
    }
    hipStream_t s = (hipStream_t)stream;
    const hipError_t e = fp8 ? gattn::launch_decode_split_fp8(a, layer->head_dim, layer->kv_shared != 0, batch, s)
                             : gattn::launch_decode_split(a, layer->head_dim, layer->kv_shared != 0, batch, s);
    if (e != hipSuccess)
        return GATTN_ERR_HIP;
    if (plan.n_slots > 1 &&
        !gattn::decode_merges_slots(layer->head_dim, fp8, plan.n_slots, (int64_t)batch * layer->num_kv_heads)) {
        gattn::CombineRows rows;
        rows.ctx_lens = ctx_lens;
        rows.split_tokens = plan.split_tokens;
        rows.is_global = layer->family == GATTN_GLOBAL;
        rows.window = layer->window;
        rows.max_ctx = max_ctx;
        if (gattn::launch_combine(batch, layer->num_q_heads, layer->head_dim, plan.n_slots, a.o_part,
                                  a.lse_part, out, lse, s, rows) != hipSuccess)
            return GATTN_ERR_HIP;
    }
    return GATTN_OK;
}

}  // namespace

extern "C" {

int gattn_decode(const gattn_layer *layer, const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                 int64_t num_pages, const int32_t *page_table, int pt_stride, const int32_t *ctx_lens,
                 int batch, int max_ctx, int split_tokens, void *workspace, size_t workspace_bytes,
                 uint16_t *out, float *lse, void *stream) {
    return decode_impl(layer, q, k_pool, v_pool, false, 1.0f, 1.0f, num_pages, page_table, pt_stride, ctx_lens,
                       batch, max_ctx, split_tokens, workspace, workspace_bytes, out, lse, stream);
}

int gattn_decode_noalloc(const gattn_layer *layer, const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                         int64_t num_pages, const int32_t *page_table, int pt_stride, const int32_t *ctx_lens,
                         int batch, int max_ctx, int split_tokens, uint16_t *out, float *lse, void *stream) {
    return decode_impl(layer, q, k_pool, v_pool, false, 1.0f, 1.0f, num_pages, page_table, pt_stride, ctx_lens,
                       batch, max_ctx, split_tokens, nullptr, 0, out, lse, stream, true);
}

int gattn_decode_fp8kv(const gattn_layer *layer, const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool,
                       float k_scale, float v_scale, int64_t num_pages, const int32_t *page_table, int pt_stride,
                       const int32_t *ctx_lens, int batch, int max_ctx, int split_tokens, void *workspace,
                       size_t workspace_bytes, uint16_t *out, float *lse, void *stream) {
    return decode_impl(layer, q, k_pool, v_pool, true, k_scale, v_scale, num_pages, page_table, pt_stride, ctx_lens,
                       batch, max_ctx, split_tokens, workspace, workspace_bytes, out, lse, stream);
}

}  // extern "C"

// The decode graph bucket set: one instantiated graph per bucket size, in increasing order.
struct gattn_decode_graphs {
    int n;
    int32_t buckets[GATTN_MAX_GRAPH_BUCKETS];
    void *exec[GATTN_MAX_GRAPH_BUCKETS];
};

extern "C" {

void gattn_decode_graphs_destroy(gattn_decode_graphs *graphs) {
    if (!graphs)
        return;
    for (int i = 0; i < graphs->n; ++i)
        gattn::graph_free(graphs->exec[i]);
    delete graphs;
}

int gattn_decode_graphs_create(const gattn_layer *layer, const uint16_t *q, const uint16_t *k_pool,
                               const uint16_t *v_pool, int64_t num_pages, const int32_t *page_table, int pt_stride,
                               const int32_t *ctx_lens, int max_ctx, int split_tokens, void *workspace,
                               size_t workspace_bytes, uint16_t *out, float *lse, const int32_t *buckets,
                               int n_buckets, gattn_decode_graphs **graphs) {
    if (!graphs)
        return GATTN_ERR_NULL_PTR;
    *graphs = nullptr;
    if (!buckets)
        return GATTN_ERR_NULL_PTR;
    if (n_buckets < 1 || n_buckets > GATTN_MAX_GRAPH_BUCKETS)
        return GATTN_ERR_BAD_SHAPE;
    for (int i = 0; i < n_buckets; ++i)
        if (buckets[i] < 1 || (i > 0 && buckets[i] <= buckets[i - 1]))
            return GATTN_ERR_BAD_SHAPE;
    // every bucket's call is checked before anything is captured
    for (int i = 0; i < n_buckets; ++i) {
        const int rc = decode_impl(layer, q, k_pool, v_pool, false, 1.0f, 1.0f, num_pages, page_table, pt_stride,
                                   ctx_lens, buckets[i], max_ctx, split_tokens, workspace, workspace_bytes, out, lse,
                                   nullptr, false, true);
        if (rc != GATTN_OK)
            return rc;
    }
    gattn_decode_graphs *set = new (std::nothrow) gattn_decode_graphs{};
    if (!set)
        return GATTN_ERR_HIP;
    for (int i = 0; i < n_buckets; ++i) {
        hipStream_t cs = nullptr;
        if (gattn::graph_capture_begin(&cs) != hipSuccess) {
            gattn_decode_graphs_destroy(set);
            return GATTN_ERR_HIP;
        }
        const int rc = decode_impl(layer, q, k_pool, v_pool, false, 1.0f, 1.0f, num_pages, page_table, pt_stride,
                                   ctx_lens, buckets[i], max_ctx, split_tokens, workspace, workspace_bytes, out, lse,
                                   (void *)cs);
        void *exec = nullptr;
        const hipError_t e = gattn::graph_capture_end(cs, &exec);
        if (rc != GATTN_OK || e != hipSuccess) {
            gattn::graph_free(exec);
            gattn_decode_graphs_destroy(set);
            return rc != GATTN_OK ? rc : GATTN_ERR_HIP;
        }
        set->buckets[i] = buckets[i];
        set->exec[i] = exec;
        set->n = i + 1;
    }
    *graphs = set;
    return GATTN_OK;
}

int gattn_decode_graphs_bucket(const gattn_decode_graphs *graphs, int batch) {
    if (!graphs || batch < 1)
        return -1;
    for (int i = 0; i < graphs->n; ++i)
        if (graphs->buckets[i] >= batch)
            return graphs->buckets[i];
    return -1;
}

int gattn_decode_graphs_launch(const gattn_decode_graphs *graphs, int batch, void *stream) {
    if (!graphs)
        return GATTN_ERR_NULL_PTR;
    for (int i = 0; i < graphs->n; ++i)
        if (batch >= 1 && graphs->buckets[i] >= batch)
            return gattn::graph_launch(graphs->exec[i], (hipStream_t)stream) == hipSuccess ? GATTN_OK : GATTN_ERR_HIP;
    return GATTN_ERR_BAD_SHAPE;
}

int gattn_prefill(const gattn_layer *layer, const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool,
                  int64_t num_pages, const int32_t *page_table, int pt_stride, const int32_t *cu_q,
                  const int32_t *ctx_lens, int batch, int max_q, uint16_t *out, float *lse, void *stream) {
    int rc = check_layer(layer);
    if (rc != GATTN_OK)
        return rc;
    if (batch < 0 || max_q < 0 || pt_stride < 1 || num_pages < 1)
        return GATTN_ERR_BAD_SHAPE;
    // a query tile's rows span at most 256 positions x num_q_heads x head_dim bf16, addressed with
    // 32-bit offsets
    if (layer->num_q_heads > kMaxPrefillQHeads)
        return GATTN_ERR_UNSUPPORTED;
    if (!q || !k_pool || !page_table || !cu_q || !ctx_lens || !out || !lse)
        return GATTN_ERR_NULL_PTR;
    if (layer->kv_shared) {
        if (v_pool && v_pool != k_pool)
            return GATTN_ERR_BAD_SHAPE;
        v_pool = k_pool;
    } else if (!v_pool) {
        return GATTN_ERR_NULL_PTR;
    }
    if (batch == 0 || max_q == 0)
        return GATTN_OK;
    gattn::PrefillArgs a{};
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.page_table = page_table;
    a.cu_q = cu_q;
    a.ctx_lens = ctx_lens;
    a.out = out;
    a.lse = lse;
    a.num_pages = num_pages;
    a.pt_stride = pt_stride;
    a.num_q_heads = layer->num_q_heads;
    a.num_kv_heads = layer->num_kv_heads;
    a.group = layer->num_q_heads / layer->num_kv_heads;
    a.is_global = layer->family == GATTN_GLOBAL;
    a.window = layer->window;
    a.max_q = max_q;
    a.scale_log2 = layer->scale * 1.4426950408889634f;
    if (gattn::launch_prefill(a, layer->head_dim, layer->kv_shared != 0, batch, (hipStream_t)stream) !=
        hipSuccess)
        return GATTN_ERR_HIP;
    return GATTN_OK;
}

}  // extern "C"

namespace {

// KV append into bf16 pools, or into E4M3 pools (fp8) with their per-tensor scales.
int append_impl(const gattn_layer *layer, const uint16_t *k_new, const uint16_t *v_new, void *k_pool, void *v_pool,
                bool fp8, float k_scale, float v_scale, int64_t num_pages, const int32_t *page_table, int pt_stride,
                const int32_t *cu_new, const int32_t *ctx_lens, int batch, int max_new, int32_t *status,
                void *stream) {
    int rc = check_layer(layer);
    if (rc != GATTN_OK)
        return rc;
    if (fp8) {
        if (layer->head_dim == 256 && layer->kv_shared)
            return GATTN_ERR_UNSUPPORTED;
        if (!(k_scale > 0.0f) || !isfinite(k_scale))
            return GATTN_ERR_BAD_SHAPE;
        if (layer->kv_shared)
            v_scale = k_scale;  // unused: only K is written
        else if (!(v_scale > 0.0f) || !isfinite(v_scale))
            return GATTN_ERR_BAD_SHAPE;
    }
    if (batch < 0 || max_new < 0 || pt_stride < 1 || num_pages < 1)
        return GATTN_ERR_BAD_SHAPE;
    if (!k_new || !k_pool || !page_table || !cu_new || !ctx_lens)
        return GATTN_ERR_NULL_PTR;
    if (layer->kv_shared) {
        if (v_new || (v_pool && v_pool != k_pool))
            return GATTN_ERR_BAD_SHAPE;
        v_pool = nullptr;
    } else if (!v_new || !v_pool) {
        return GATTN_ERR_NULL_PTR;
    }
    if (batch == 0 || max_new == 0)
        return GATTN_OK;
    gattn::AppendArgs a{};
    a.k_new = k_new;
    a.v_new = layer->kv_shared ? nullptr : v_new;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.page_table = page_table;
    a.cu_new = cu_new;
    a.ctx_lens = ctx_lens;
    a.status = status;
    a.num_pages = num_pages;
    a.pt_stride = pt_stride;
    a.num_kv_heads = layer->num_kv_heads;
    a.max_new = max_new;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    if (gattn::launch_kv_append(a, layer->head_dim, batch, fp8, (hipStream_t)stream) != hipSuccess)
        return GATTN_ERR_HIP;
    return GATTN_OK;
}

}  // namespace

extern "C" {

int gattn_kv_append(const gattn_layer *layer, const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_pool,
                    uint16_t *v_pool, int64_t num_pages, const int32_t *page_table, int pt_stride,
                    const int32_t *cu_new, const int32_t *ctx_lens, int batch, int max_new, int32_t *status,
                    void *stream) {
    return append_impl(layer, k_new, v_new, k_pool, v_pool, false, 1.0f, 1.0f, num_pages, page_table, pt_stride,
                       cu_new, ctx_lens, batch, max_new, status, stream);
}

int gattn_kv_append_fp8(const gattn_layer *layer, const uint16_t *k_new, const uint16_t *v_new, uint8_t *k_pool,
                        uint8_t *v_pool, float k_scale, float v_scale, int64_t num_pages, const int32_t *page_table,
                        int pt_stride, const int32_t *cu_new, const int32_t *ctx_lens, int batch, int max_new,
                        int32_t *status, void *stream) {
    return append_impl(layer, k_new, v_new, k_pool, v_pool, true, k_scale, v_scale, num_pages, page_table, pt_stride,
                       cu_new, ctx_lens, batch, max_new, status, stream);
}

int gattn_combine(int batch, int num_q_heads, int head_dim, int num_splits, const float *o_part,
                  const float *lse_part, uint16_t *out, float *lse, void *stream) {
    if (batch < 0 || num_q_heads <= 0 || num_splits <= 0 || head_dim <= 0)
        return GATTN_ERR_BAD_SHAPE;
    if (head_dim % 4 != 0 || head_dim > 1024)
        return GATTN_ERR_UNSUPPORTED;
    if (!o_part || !lse_part || !out || !lse)
        return GATTN_ERR_NULL_PTR;
    if (batch == 0)
        return GATTN_OK;
    if (gattn::launch_combine(batch, num_q_heads, head_dim, num_splits, o_part, lse_part, out, lse,
                              (hipStream_t)stream) != hipSuccess)
        return GATTN_ERR_HIP;
    return GATTN_OK;
}

}  // extern "C"
