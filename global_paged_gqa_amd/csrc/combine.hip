// Logsumexp merge of split-KV partials (the combine half of flash-decoding).
//
// One workgroup per (row, query head). Threads own four output dims each and are
// grouped so several groups walk disjoint subsets of the splits; the group sums and
// the split maxima and sums are reduced in a fixed order, so the result depends
// only on the partials. Empty splits (lse = -inf)
// are skipped without reading their o; a NaN lse marks a failed split and turns
// the whole (row, head) result into NaN.
#include "common.h"
#include "kernels.h"

namespace gattn {

namespace {

__device__ float block_reduce(float v, bool is_max, float *scratch) {
    // wave-level tree, then across waves through LDS; fixed order throughout
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float o = __shfl_xor(v, off);
        v = is_max ? nan_max(v, o) : v + o;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
    __syncthreads();
    if (lane == 0)
        scratch[wave] = v;
    __syncthreads();
    float r = scratch[0];
    for (int w = 1; w < nw; ++w)
        r = is_max ? nan_max(r, scratch[w]) : r + scratch[w];
    return r;
}

__global__ __launch_bounds__(256) void combine_kernel(int num_q_heads, int head_dim, int ns,
                                                      const float *o_part, const float *lse_part,
                                                      uint16_t *out, float *lse) {
    __shared__ float scratch[4];
    __shared__ f32x4 part[256];
    const int h = blockIdx.x, b = blockIdx.y;
    const int64_t bh = (int64_t)b * num_q_heads + h;
    const float *lp = lse_part + bh * ns;

    float m = -INFINITY;
    for (int s = threadIdx.x; s < ns; s += blockDim.x)
        m = nan_max(m, lp[s]);
    const float M = block_reduce(m, true, scratch);

    // thread = (split group sg, four output dims d); the split groups split the splits
    const int dgroups = head_dim / 4;
    const int ngroups = blockDim.x / dgroups;
    const int sg = threadIdx.x / dgroups;
    const int d = (threadIdx.x % dgroups) * 4;
    if (M == -INFINITY) {  // every split empty
        if (sg == 0)
            *(u32x2 *)(out + bh * head_dim + d) = u32x2{0u, 0u};
        if (threadIdx.x == 0)
            lse[bh] = -INFINITY;
        return;
    }
    float sum = 0.f;
    for (int s = threadIdx.x; s < ns; s += blockDim.x) {
        const float l = lp[s];
        sum += (l == -INFINITY) ? 0.f : __expf(l - M);
    }
    const float total = block_reduce(sum, false, scratch);
    const float LSE = M + __logf(total);

    // Branch-free loop so the partial loads of several splits are in flight together; an
    // empty split's o (possibly stale or NaN) is selected out, never multiplied by zero.
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    const float *op = o_part + bh * ns * head_dim + d;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int s = sg; sg < ngroups && s < ns; s += ngroups) {
        const float l = lp[s];
        const f32x4 v = *(const f32x4 *)(op + (int64_t)s * head_dim);
        const bool empty = l == -INFINITY;
        o += empty ? zero : __expf(l - LSE) * v;
    }
    part[threadIdx.x] = o;
    __syncthreads();
    if (sg == 0) {
        for (int k = 1; k < ngroups; ++k)
            o += part[k * dgroups + threadIdx.x];
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
    // 256 threads: as many split groups of head_dim/4 threads as fit (head_dim <= 1024);
    // leftover threads only join the reductions
    const dim3 block(256);
    int hq = num_q_heads, hd = head_dim, ns = num_splits;
    void *args[] = {&hq, &hd, &ns, (void *)&o_part, (void *)&lse_part, (void *)&out, (void *)&lse};
    return hipLaunchKernel((const void *)combine_kernel, grid, block, args, 0, stream);
}

}  // namespace gattn
