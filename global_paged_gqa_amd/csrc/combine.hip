// Logsumexp merge of split-KV partials (the combine half of flash-decoding).
//
// One workgroup per (row, query head). Every thread reads the head's split LSEs (uniform
// addresses) and forms the maximum, the sum of exp(lse - M) and the merged LSE itself, in
// split order, with no cross-thread reduction. The merged O is the exp(lse_s - LSE)-weighted
// sum of the split outputs: four thread groups of one thread per four dims each take every
// fourth split (group t: splits t, t+4, ...), so four of a long row's partials are read at
// once, and group 0 adds the others' sums in group order. An empty split (lse = -inf)
// contributes nothing and its o (possibly stale or NaN) is never read; a NaN lse marks a failed
// split and turns the whole (row, head) result into NaN. Which splits a group takes depends
// only on the split index, so the result depends only on the row's own partials, not on how
// many slots the call has.
#include "common.h"
#include "kernels.h"

namespace gattn {

namespace {

constexpr int kGroups = 4;

__global__ __launch_bounds__(1024) void combine_kernel(int num_q_heads, int head_dim, int ns, const float *o_part,
                                                       const float *lse_part, uint16_t *out, float *lse) {
    __shared__ f32x4 part[kGroups - 1][256];  // groups 1..3, one entry per four dims (head_dim <= 1024)
    const int h = blockIdx.x, b = blockIdx.y;
    const int64_t bh = (int64_t)b * num_q_heads + h;
    const float *lp = lse_part + bh * ns;
    const int tpg = blockDim.x / kGroups;  // threads per group
    const int grp = threadIdx.x / tpg, t = threadIdx.x % tpg;
    const int d = t * 4;
    const bool owner = d < head_dim;

    // maximum, then the sum against it, in split order (NaN propagates)
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s)
        M = nan_max(M, lp[s]);
    if (M == -INFINITY) {  // every split empty (uniform: the whole workgroup leaves here)
        if (grp == 0 && owner)
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
#pragma unroll 4
        for (int s = grp; s < ns; s += kGroups) {
            const float l = lp[s];
            if (l != -INFINITY)
                o += __expf(l - LSE) * *(const f32x4 *)(op + (int64_t)s * head_dim);
        }
        if (grp > 0)
            part[grp - 1][t] = o;
    }
    __syncthreads();
    if (grp == 0 && owner) {
#pragma unroll
        for (int q = 0; q < kGroups - 1; ++q)
            o += part[q][t];
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
    // kGroups groups of one thread per four dims, each rounded up to whole waves (head_dim <= 1024)
    const dim3 block(kGroups * ((head_dim / 4 + 63) / 64) * 64);
    int hq = num_q_heads, hd = head_dim, ns = num_splits;
    void *args[] = {&hq, &hd, &ns, (void *)&o_part, (void *)&lse_part, (void *)&out, (void *)&lse};
    return hipLaunchKernel((const void *)combine_kernel, grid, block, args, 0, stream);
}

}  // namespace gattn
