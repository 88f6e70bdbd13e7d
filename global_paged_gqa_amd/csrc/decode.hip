// Split-KV flash-decode for hybrid paged GQA attention on gfx950.
//
// One workgroup = one (row, KV head, split). A split is the keys of one row in
// [s*S, (s+1)*S) intersected with the row's visible range, S = split_tokens
// (the split-KV chunk policy of the pegainfer "[Model] Gemma 4 M3 31B" plan;
// the flash-decode split factor of the Core AI card's "--metal-sdpa" section).
// Local rows only visit the splits that intersect their window, so a row with a
// 32768-token context still reads at most `window` keys (the sliding-window
// tile pruning that page 5's "Three load-bearing facts" #1 credits with a 3-4x
// gain).
//
// Inside the workgroup four waves take the split's pages round-robin. Each wave
// keeps its own online-softmax state for the g query heads that share this KV
// head and merges with the other three at the end through LDS, in a fixed order
// (deterministic, so results are bitwise independent of the batch).
//
// Per page (16 tokens) a wave does, entirely in registers:
//   S^T[16 tok][16 heads] = K[16 tok][hd] . Q^T[hd][16 heads]   (MFMA 16x16x32, bf16)
//   online softmax on S^T columns                                 (VALU + lane swaps)
//   V^T tile = MFMA(V, identity)  -- an exact register transpose of V
//   O^T[hd][16 heads] += V^T[hd][16 tok] . P^T[16 tok][16 heads]  (MFMA 16x16x16, bf16)
// The K/V loads are 16 B per lane straight from the page into the MFMA operand
// layout (each instruction reads 64 contiguous bytes of 16 token rows), with the
// next page's loads in flight while the current page is computed.
#include "common.h"
#include "kernels.h"

namespace gattn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kMergeBytes = 32 * 1024;

template <int HD>
struct PageRegs {
    u32x4 r[HD / 32];
};

template <int HD, bool SHARED>
__global__ __launch_bounds__(kThreads, 1) void decode_split_kernel(DecodeArgs a) {
    constexpr int NS = HD / 32;  // K-steps of 32 dims for QK
    constexpr int NT = HD / 16;  // 16-dim tiles of the output

    constexpr int kQStride = HD + 8;  // padded LDS row (bf16 elements) of one head's query
    __shared__ float sm_o[kMergeBytes / 4];
    __shared__ __attribute__((aligned(16))) uint16_t sm_q[16 * kQStride];
    __shared__ float sm_m[kWaves][16];
    __shared__ float sm_l[kWaves][16];
    __shared__ int sm_bad[kWaves];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c16 = lane & 15;  // MFMA row/column index of this lane
    const int r4 = lane >> 4;   // 16-lane row of this lane
    const int slot = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int g = a.group;
    const int Hq = a.num_q_heads;

    // ---- the row's visible range and this split's share of it
    const int L = a.ctx_lens[b];
    const bool bad_len = (L < 1) || (L > a.max_ctx) || ((L - 1) / kPage >= a.pt_stride);
    int tb = 0, te = 0;
    if (!bad_len) {
        const int p = L - 1;
        const int lo = a.is_global ? 0 : max(0, p - a.window + 1);
        const int64_t S = a.split_tokens;
        const int64_t s_abs = (a.is_global ? 0 : lo / S) + slot;
        tb = (int)max<int64_t>(lo, s_abs * S);
        te = (int)min<int64_t>(L, (s_abs + 1) * S);
    }
    const bool direct = a.n_slots == 1;
    if (!bad_len && tb >= te) {  // split outside the visible range: mark it empty
        if (threadIdx.x < g)
            a.lse_part[((int64_t)b * Hq + kvh * g + threadIdx.x) * a.n_slots + slot] = -INFINITY;
        return;
    }

    const int pg0 = tb / kPage, pg1 = (te - 1) / kPage;
    const int npg = bad_len ? 0 : pg1 - pg0 + 1;
    const int cnt = npg > wave ? (npg - wave + kWaves - 1) / kWaves : 0;

    // ---- Q^T as the B operand, staged once in LDS for the 16 MFMA columns (the g real
    // heads, zeros for the rest); each page reads lane's head c16, 8 dims per K-step.
    for (int e = threadIdx.x; e < 16 * (HD / 8); e += kThreads) {
        const int hn = e / (HD / 8), d8 = (e % (HD / 8)) * 8;
        u32x4 v = {0, 0, 0, 0};
        if (hn < g)
            v = *(const u32x4 *)(a.q + ((int64_t)b * Hq + kvh * g + hn) * HD + d8);
        *(u32x4 *)(sm_q + hn * kQStride + d8) = v;
    }
    __syncthreads();
    const uint16_t *q_lane = sm_q + c16 * kQStride + r4 * 8;
    // Identity blocks for the register transpose: B[(r4, e)][c16] = 1 iff 8*r4 + e == 16*h + c16.
    u32x4 ident[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t w[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            const int e = 2 * e2;
            uint32_t lo = (8 * r4 + e == 16 * h + c16) ? 0x3F80u : 0u;
            uint32_t hi = (8 * r4 + e + 1 == 16 * h + c16) ? 0x3F80u : 0u;
            w[e2] = lo | (hi << 16);
        }
        ident[h] = u32x4{w[0], w[1], w[2], w[3]};
    }

    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    int bad_page = 0;

    const int64_t blk = (int64_t)kPage * HD;  // elements of one (page, KV head) block
    const int lane_off = c16 * HD + r4 * 8;
    const int32_t *pt = a.page_table + (int64_t)b * a.pt_stride;

    auto page_of = [&](int i) { return pg0 + wave + kWaves * i; };
    auto page_id = [&](int i) {  // scalar load of a page id (wave-uniform), checked
        int pid = i < cnt ? pt[page_of(i)] : 0;
        if (pid < 0 || pid >= a.num_pages) {
            bad_page = 1;
            pid = 0;
        }
        return pid;
    };
    auto load_k = [&](PageRegs<HD> &K, int pid) {
        const uint16_t *kp = a.k_pool + ((int64_t)pid * a.num_kv_heads + kvh) * blk + lane_off;
#pragma unroll
        for (int s = 0; s < NS; ++s)
            K.r[s] = *(const u32x4 *)(kp + s * 32);
    };
    auto load_v = [&](PageRegs<HD> &V, int pid) {
        const uint16_t *vp = a.v_pool + ((int64_t)pid * a.num_kv_heads + kvh) * blk + lane_off;
#pragma unroll
        for (int s = 0; s < NS; ++s)
            V.r[s] = *(const u32x4 *)(vp + s * 32);
    };
    // Scores of page i, online-softmax update, rescale of the accumulator; returns P^T
    // (bf16, as the B operand of the PV product) and which of the lane's tokens are valid.
    auto qk_softmax = [&](PageRegs<HD> &K, int i, bool (&valid)[4]) {
        const int t0 = page_of(i) * kPage;
        f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s)
            st = mfma_k32(K.r[s], *(const u32x4 *)(q_lane + s * 32), st);
        // lane holds S^T[token t0 + 4*r4 + e][head c16]; out-of-range tokens are selected
        // out (a NaN in an unused slot never reaches the sums)
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = t0 + 4 * r4 + e;
            valid[e] = t >= tb && t < te;
            const float v = valid[e] ? st[e] * a.scale_log2 : -INFINITY;
            st[e] = v;
            mx = fmaxf(mx, v);
        }
        mx = rows_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        float ps[4], rs = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ps[e] = fast_exp2(st[e] - m_new);
            rs += ps[e];
        }
        rs = rows_sum(rs);
        l_run = l_run * alpha + rs;
        m_run = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int j = 0; j < NT; ++j)
                acc[j] *= alpha;
        }
        return u32x2{pack_bf16x2(ps[0], ps[1]), pack_bf16x2(ps[2], ps[3])};
    };
    // O^T += V^T P^T for page i; V^T comes from an exact MFMA transpose of the V registers.
    auto pv = [&](PageRegs<HD> &V, int i, u32x2 pb, const bool (&valid)[4]) {
        const int t0 = page_of(i) * kPage;
        const bool edge = t0 < tb || t0 + kPage > te;  // page holds tokens outside [tb, te)
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        __builtin_amdgcn_sched_barrier(0);
        if (edge) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                f32x4 vt = mfma_k32(V.r[j >> 1], ident[j & 1], zero);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    vt[e] = valid[e] ? vt[e] : 0.f;
                const u32x2 va = {pack_exact_bf16x2(vt[0], vt[1]), pack_exact_bf16x2(vt[2], vt[3])};
                acc[j] = mfma_k16(va, pb, acc[j]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const f32x4 vt = mfma_k32(V.r[j >> 1], ident[j & 1], zero);
                const u32x2 va = {pack_exact_bf16x2(vt[0], vt[1]), pack_exact_bf16x2(vt[2], vt[3])};
                acc[j] = mfma_k16(va, pb, acc[j]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // Pipeline: page ids two pages ahead, K one page ahead of the math. V is either
    // double-buffered like K (VBUF = 2) or loaded into its single buffer right after the
    // previous page's PV product (VBUF = 1, for the largest register footprint).
    constexpr int VBUF = (SHARED || HD <= 256) ? 2 : 1;
    if (cnt > 0) {
        PageRegs<HD> KA, KB, VA, VB;
        int pid_b = page_id(1);
        {
            const int pid_a = page_id(0);
            load_k(KA, pid_a);
            if (!SHARED)
                load_v(VA, pid_a);
        }
        for (int i = 0; i < cnt; i += 2) {
            const int pid_c = page_id(i + 2);
            bool valid[4];
            // page i in KA/VA; page i+1 goes to KB (and VB, or VA after the PV product)
            if (i + 1 < cnt) {
                load_k(KB, pid_b);
                if (!SHARED && VBUF == 2)
                    load_v(VB, pid_b);
            }
            u32x2 pb = qk_softmax(KA, i, valid);
            pv(SHARED ? KA : VA, i, pb, valid);
            if (i + 1 >= cnt)
                break;
            if (!SHARED && VBUF == 1)
                load_v(VA, pid_b);
            // page i+1 in KB/(VB or VA); page i+2 goes to KA (and VA)
            if (i + 2 < cnt) {
                load_k(KA, pid_c);
                if (!SHARED && VBUF == 2)
                    load_v(VA, pid_c);
            }
            pb = qk_softmax(KB, i + 1, valid);
            pv(SHARED ? KB : (VBUF == 2 ? VB : VA), i + 1, pb, valid);
            if (!SHARED && VBUF == 1 && i + 2 < cnt)
                load_v(VA, pid_c);
            pid_b = page_id(i + 3);
        }
    }

    // ---- merge the four waves (fixed order) and write this split's result
    if (r4 == 0) {
        sm_m[wave][c16] = m_run;
        sm_l[wave][c16] = l_run;
    }
    if (lane == 0)
        sm_bad[wave] = bad_page;
    const bool any_bad = bad_len;
    constexpr int kChunk = kMergeBytes / 4 / (kWaves * HD);  // heads merged per round
    for (int h0 = 0; h0 < g; h0 += kChunk) {
        __syncthreads();
        if (c16 >= h0 && c16 < min(g, h0 + kChunk)) {
            float *dst = sm_o + ((wave * kChunk) + (c16 - h0)) * HD + 4 * r4;
#pragma unroll
            for (int j = 0; j < NT; ++j)
                *(f32x4 *)(dst + 16 * j) = acc[j];
        }
        __syncthreads();
        const bool bad = any_bad || sm_bad[0] || sm_bad[1] || sm_bad[2] || sm_bad[3];
        const int nh = min(g, h0 + kChunk) - h0;
        for (int e = threadIdx.x; e < nh * HD; e += kThreads) {
            const int hn = h0 + e / HD, d = e % HD;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
                M = fmaxf(M, sm_m[w][hn]);
            float lsum = 0.f, o = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float mw = sm_m[w][hn];
                if (mw == -INFINITY)
                    continue;
                const float wt = fast_exp2(mw - M);
                lsum += wt * sm_l[w][hn];
                o += wt * sm_o[(w * kChunk + (hn - h0)) * HD + d];
            }
            o = o / lsum;
            float lse = (M + fast_log2(lsum)) * kLn2;
            if (bad) {
                o = __builtin_nanf("");
                lse = __builtin_nanf("");
            }
            const int64_t bh = (int64_t)b * Hq + kvh * g + hn;
            if (direct) {
                a.out[bh * HD + d] = (uint16_t)bf16_rne(o);
                if (d == 0)
                    a.lse[bh] = lse;
            } else {
                a.o_part[(bh * a.n_slots + slot) * HD + d] = o;
                if (d == 0)
                    a.lse_part[bh * a.n_slots + slot] = lse;
            }
        }
    }
}

template <int HD, bool SHARED>
hipError_t launch(const DecodeArgs &a, dim3 grid, hipStream_t stream) {
    void *args[] = {(void *)&a};
    return hipLaunchKernel((const void *)decode_split_kernel<HD, SHARED>, grid, dim3(kThreads), args, 0,
                           stream);
}

}  // namespace

hipError_t launch_decode_split(const DecodeArgs &a, int head_dim, bool kv_shared, int batch,
                               hipStream_t stream) {
    const dim3 grid(a.n_slots, a.num_kv_heads, batch);
    if (head_dim == 256)
        return kv_shared ? launch<256, true>(a, grid, stream) : launch<256, false>(a, grid, stream);
    if (head_dim == 512)
        return kv_shared ? launch<512, true>(a, grid, stream) : launch<512, false>(a, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace gattn
