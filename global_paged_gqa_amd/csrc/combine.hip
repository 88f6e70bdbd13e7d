// Logsumexp merge of split-KV partials (the combine half of flash-decoding).
//
// One workgroup per (row, query head), one thread per four output dims. Every thread
// reads the head's split LSEs (uniform addresses) and forms the maximum, the sum of
// exp(lse - M) and the merged LSE itself, in split order, with no cross-thread
// reduction; the merged O is then the exp(lse_s - LSE)-weighted sum of the split
// outputs, again in split order, so the result depends only on the partials.
//
// The splits a decode row touches form a prefix of its slots (the slots past the row's
// last key are empty), so the prefix of non-empty splits is merged branch-free with all
// its loads in flight; any non-empty split after the first empty one (partials produced
// elsewhere) is handled by a slower loop in the same order. An empty split (lse = -inf)
// contributes nothing and its o (possibly stale or NaN) is never read; a NaN lse marks a
// failed split and turns the whole (row, head) result into NaN.
#include "common.h"
#include "kernels.h"

namespace gattn {

namespace {

__global__ __launch_bounds__(256) void combine_kernel(int num_q_heads, int head_dim, int ns,
                                                      const float *o_part, const float *lse_part,
                                                      uint16_t *out, float *lse) {
    const int h = blockIdx.x, b = blockIdx.y;
    const int64_t bh = (int64_t)b * num_q_heads + h;
    const float *lp = lse_part + bh * ns;
    const int d = threadIdx.x * 4;
    const bool owner = d < head_dim;

    // maximum, then the sum against it, in split order (NaN propagates)
    float M = -INFINITY;
    int n_ne = ns;  // length of the prefix of non-empty splits
    for (int s = 0; s < ns; ++s) {
        const float l = lp[s];
        M = nan_max(M, l);
        if (l == -INFINITY && n_ne == ns)
            n_ne = s;
    }
    if (M == -INFINITY) {  // every split empty
        if (owner)
            *(u32x2 *)(out + bh * head_dim + d) = u32x2{0u, 0u};
        if (threadIdx.x == 0)
            lse[bh] = -INFINITY;
        return;
    }
    float total = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float l = lp[s];
        total += (l == -INFINITY) ? 0.f : __expf(l - M);
    }
    const float LSE = M + __logf(total);

    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (owner) {
        const float *op = o_part + bh * ns * head_dim + d;
#pragma unroll 8
        for (int s = 0; s < n_ne; ++s)
            o += __expf(lp[s] - LSE) * *(const f32x4 *)(op + (int64_t)s * head_dim);
        for (int s = n_ne; s < ns; ++s) {
            const float l = lp[s];
            if (l != -INFINITY)
                o += __expf(l - LSE) * *(const f32x4 *)(op + (int64_t)s * head_dim);
        }
        if (M != M)
            o = f32x4{M, M, M, M};
        *(u32x2 *)(out + bh * head_dim + d) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
    if (threadIdx.x == 0)
        lse[bh] = LSE;
}

}  // namespace

hipError_t launch_combine(int batch, int num_q_heads, int head_dim, int num_splits, const float *o_part,
                          const float *lse_part, uint16_t *out, float *lse, hipStream_t stream) {
    const dim3 grid(num_q_heads, batch);
    // one thread per four dims, rounded up to whole waves (head_dim <= 1024)
    const dim3 block(((head_dim / 4 + 63) / 64) * 64);
    int hq = num_q_heads, hd = head_dim, ns = num_splits;
    void *args[] = {&hq, &hd, &ns, (void *)&o_part, (void *)&lse_part, (void *)&out, (void *)&lse};
    return hipLaunchKernel((const void *)combine_kernel, grid, block, args, 0, stream);
}

}  // namespace gattn
