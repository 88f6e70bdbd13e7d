// Logsumexp merge of split-KV partials (the combine half of flash-decoding).
//
// The merged output is fixed as an order of operations: split s joins partial sum s % 4, in
// increasing s; the four partial sums are then added in order ((a0 + a1) + a2) + a3.
// Empty splits (lse = -inf, among them every slot past a row's last key) are skipped, so a
// row's result depends only on its own partials, never on how many split slots the batch
// has. One workgroup per (row, query head) computes it with one thread per four output dims
// in each of G thread groups (G = 1, 2 or 4, by slot count: a thread of group p holds the
// partial sums p, p + G, ...), the groups meeting in LDS at the end. A thread issues the
// loads of F of its splits at once (F = 4, 8 or 16, the least that covers the slots, else
// 16 per pass), before the statistics are known, so that up to 16 G splits wait on memory
// once. Neither G nor F changes the result.
//
// Statistics: every wave forms the maximum M of the split LSEs and the sum of
// exp(lse - M) lane-parallel (lane j takes splits j, j + 64, ...), reduced by symmetric
// pairwise steps over the 64 lanes; LSE = M + ln(sum). An empty split never enters the
// result, whatever its o holds (stale data or NaN); a NaN lse marks a failed split and turns
// the whole (row, head) result into NaN.
#include "common.h"
#include "kernels.h"

namespace gattn {

namespace {

constexpr int kSums = 4;  // partial sums of the fixed order
constexpr int kMaxThreads = 512;

// x from lane l ^ 1 (quad_perm 1,0,3,2), l ^ 2 (quad_perm 2,3,0,1), 7 - l within 8 lanes
// (row_half_mirror) and 15 - l within 16 (row_mirror): each pairs lanes symmetrically.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum and NaN-propagating maximum over the 64 lanes: pairwise steps within 16-lane rows,
// then across rows with the lane swaps.
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    return rows_sum4(x);
}

__device__ __forceinline__ float wave_nan_max(float x) {
    x = nan_max(x, dpp<0xB1>(x));
    x = nan_max(x, dpp<0x4E>(x));
    x = nan_max(x, dpp<0x141>(x));
    x = nan_max(x, dpp<0x140>(x));
    float a = x, b = x;
    swap_rows16(a, b);
    float c = nan_max(a, b), d = c;
    swap_halves32(c, d);
    return nan_max(c, d);
}

__device__ __forceinline__ float uniform(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

template <int G, int F>  // thread groups; splits a thread has in flight per pass
__global__ __launch_bounds__(kMaxThreads) void combine_kernel(int num_q_heads, int head_dim, int ns,
                                                              const float *o_part, const float *lse_part,
                                                              uint16_t *out, float *lse, CombineRows rows) {
    constexpr int J = kSums / G;  // partial sums per thread: p, p + G, ...
    static_assert(G * J == kSums && F % J == 0, "sum layout");
    __shared__ f32x4 part[kMaxThreads];  // (G - 1) J C <= 512 for every launch shape
    const int h = blockIdx.x, b = blockIdx.y;
    const int64_t bh = (int64_t)b * num_q_heads + h;
    const float *lp = lse_part + bh * ns;
    const int C = (head_dim / 4 + 63) / 64 * 64;  // threads per group (blockDim.x = G C)
    const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x / C);
    const int c = threadIdx.x - grp * C;
    const int d = 4 * c;
    const bool owner = d < head_dim;
    const int lane = threadIdx.x & 63;
    const float *op = o_part + bh * ns * head_dim + (owner ? d : 0);
    // Slots [0, n_live) may be non-empty. For a decode's partials: the splits from the one holding
    // the row's first visible key to the one holding its last (a row outside [1, max_ctx] fails
    // its splits with NaN, which the statistics over all slots below catch). Outputs are read
    // for those slots only; the skipped ones hold lse = -inf and would add nothing.
    int n_live = ns;
    if (rows.ctx_lens) {
        const int L = rows.ctx_lens[b];
        if (L >= 1 && L <= rows.max_ctx) {
            const int lo = rows.is_global ? 0 : max(0, L - rows.window);
            n_live = min(ns, (L - 1) / rows.split_tokens - lo / rows.split_tokens + 1);
        }
    }

    // this thread's splits s = base + grp + G k (k < F) of a pass, loads issued up front (none
    // past the live slots: the branch is uniform over the wave)
    float lv[F];
    f32x4 ov[F];
    auto load_pass = [&](int base) {
#pragma unroll
        for (int k = 0; k < F; ++k) {
            if (base + grp + G * k < n_live) {
                const int s = base + grp + G * k;
                lv[k] = lp[s];
                ov[k] = *(const f32x4 *)(op + (int64_t)s * head_dim);
            } else {
                lv[k] = -INFINITY;
                ov[k] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    load_pass(0);

    // maximum, then the sum against it (NaN propagates through both); lane j holds the LSE of
    // split j (the first 64 splits), later splits are read again
    const float l0 = lane < ns ? lp[lane] : -INFINITY;
    float M = l0;
    for (int s = lane + 64; s < ns; s += 64)
        M = nan_max(M, lp[s]);
    M = uniform(wave_nan_max(M));
    if (M == -INFINITY) {  // every split empty
        if (owner && grp == 0)
            *(u32x2 *)(out + bh * head_dim + d) = u32x2{0u, 0u};
        if (threadIdx.x == 0)
            lse[bh] = -INFINITY;
        return;
    }
    float e = (l0 == -INFINITY) ? 0.f : __expf(l0 - M);
    for (int s = lane + 64; s < ns; s += 64) {
        const float l = lp[s];
        e += (l == -INFINITY) ? 0.f : __expf(l - M);
    }
    e = wave_sum(e);
    const float LSE = M + __logf(uniform(e));

    // split base + grp + G k joins partial sum (grp + G k) % 4, held here as acc[k % J]
    // (base is a multiple of 4 G ... of G F, and G J = 4)
    f32x4 acc[J];
#pragma unroll
    for (int j = 0; j < J; ++j)
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int base = 0;;) {
#pragma unroll
        for (int k = 0; k < F; ++k) {
            const bool live = base + grp + G * k < n_live && lv[k] != -INFINITY;
            const float w = __expf(lv[k] - LSE);
            // one explicit fma per element, the same in every instantiation
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[k % J][i] = live ? __builtin_fmaf(w, ov[k][i], acc[k % J][i]) : acc[k % J][i];
        }
        base += G * F;
        if (base >= n_live)
            break;
        load_pass(base);
    }

    // partial sum v = grp + G j lives in group grp; group 0 adds a0 + a1 + a2 + a3 in order
    if constexpr (G > 1) {
        if (grp > 0) {
#pragma unroll
            for (int j = 0; j < J; ++j)
                part[((grp - 1) * J + j) * C + c] = acc[j];
        }
        __syncthreads();
    }
    if (grp == 0 && owner) {
        f32x4 o = acc[0];
#pragma unroll
        for (int v = 1; v < kSums; ++v)
            o += (v % G == 0) ? acc[v / G] : part[((v % G - 1) * J + v / G) * C + c];
        if (M != M)
            o = f32x4{M, M, M, M};
        *(u32x2 *)(out + bh * head_dim + d) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
    if (threadIdx.x == 0)
        lse[bh] = LSE;
}

}  // namespace

hipError_t launch_combine(int batch, int num_q_heads, int head_dim, int num_splits, const float *o_part,
                          const float *lse_part, uint16_t *out, float *lse, hipStream_t stream,
                          const CombineRows &rows) {
    const dim3 grid(num_q_heads, batch);
    // one thread per four dims in each group, rounded up to whole waves (head_dim <= 1024);
    // groups and loads in flight by slot count: (1, 4), (1, 8), (2, 8), (2, 16), (4, 16)
    const int per_group = (head_dim / 4 + 63) / 64 * 64;
    const int max_g = kMaxThreads / per_group >= 4 ? 4 : kMaxThreads / per_group >= 2 ? 2 : 1;
    const int ns = num_splits;
    int g = ns <= 8 ? 1 : ns <= 32 ? 2 : 4;
    g = g < max_g ? g : max_g;
    const int f = ns <= 4 * g ? 4 : ns <= 8 * g ? 8 : 16;
    int hq = num_q_heads, hd = head_dim, nsp = num_splits;
    CombineRows r = rows;
    void *args[] = {&hq, &hd, &nsp, (void *)&o_part, (void *)&lse_part, (void *)&out, (void *)&lse, &r};
    const void *k = nullptr;
    if (g == 1)
        k = f == 4 ? (const void *)combine_kernel<1, 4> : f == 8 ? (const void *)combine_kernel<1, 8>
                                                                 : (const void *)combine_kernel<1, 16>;
    else if (g == 2)
        k = f == 4 ? (const void *)combine_kernel<2, 4> : f == 8 ? (const void *)combine_kernel<2, 8>
                                                                 : (const void *)combine_kernel<2, 16>;
    else
        k = f == 4 ? (const void *)combine_kernel<4, 4> : f == 8 ? (const void *)combine_kernel<4, 8>
                                                                 : (const void *)combine_kernel<4, 16>;
    return hipLaunchKernel(k, grid, dim3(g * per_group), args, 0, stream);
}

}  // namespace gattn
