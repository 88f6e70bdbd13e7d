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
// Work split inside the workgroup (four waves): a wave owns 256 head dims of
// the pages of its page group. With head_dim 256 there are four page groups of
// one wave each; with head_dim 512 there are two groups of two waves, the pair
// splitting the head dims and adding their partial scores through LDS (one
// barrier per page). Each group keeps its own online-softmax state for the g
// query heads sharing this KV head; the groups merge at the end through LDS in
// a fixed order, so results are bitwise independent of the batch.
//
// Per page (16 tokens) a wave does, in registers:
//   S^T[16 tok][16 heads] = K[16 tok][dims] . Q^T[dims][16 heads]   (MFMA 16x16x32, bf16)
//   online softmax on S^T columns                                     (VALU + lane shuffles)
//   V^T tile = MFMA(V, identity)  -- an exact register transpose of V
//   O^T[dims][16 heads] += V^T[dims][16 tok] . P^T[16 tok][16 heads]  (MFMA 16x16x16, bf16)
// K/V are read 16 B per lane straight from the page into the MFMA operand layout
// (each instruction reads 64 contiguous bytes of 16 token rows), one page ahead
// of the math, through buffer loads whose resource has zero size past the end of
// the wave's page list (no traffic, no fault, no conditional load).
#include "common.h"
#include "kernels.h"

namespace gattn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kDimsPerWave = 256;
constexpr int kMergeBytes = 32 * 1024;
constexpr int kOcc = 2;  // workgroups per CU the register budget is sized for

struct PageRegs {
    u32x4 r[kDimsPerWave / 32];
};

template <int HD, bool SHARED, int OCC>
__global__ __launch_bounds__(kThreads, OCC) void decode_split_kernel(DecodeArgs a) {
    constexpr int DS = HD / kDimsPerWave;      // waves sharing one page (1 or 2)
    constexpr int NGRP = kWaves / DS;          // page groups
    constexpr int NS = kDimsPerWave / 32;      // K-steps of 32 dims for QK, per wave
    constexpr int NT = kDimsPerWave / 16;      // 16-dim output tiles, per wave
    constexpr int kQStride = HD + 8;           // padded LDS row (bf16 elements) of one head's query
    constexpr int kChunk = kMergeBytes / 4 / (NGRP * HD);  // heads merged per round

    __shared__ float sm_o[kMergeBytes / 4];
    __shared__ __attribute__((aligned(16))) uint16_t sm_q[16 * kQStride];
    __shared__ f32x4 sm_s[DS > 1 ? 2 : 1][DS > 1 ? kWaves * 64 : 1];  // partial scores, double-buffered
    __shared__ float sm_m[NGRP][16];
    __shared__ float sm_l[NGRP][16];
    __shared__ int sm_bad[kWaves];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave / DS, dpart = wave % DS;
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
    const int cnt = npg > grp ? (npg - grp + NGRP - 1) / NGRP : 0;  // pages of this group
    const int cnt_max = (npg + NGRP - 1) / NGRP;                       // of the largest group
    // Paired waves meet at a barrier every page, so every wave runs the same trip count.
    const int trips = DS > 1 ? cnt_max : cnt;

    const int64_t blk = (int64_t)kPage * HD;  // elements of one (page, KV head) block
    const uint32_t lane_off = (uint32_t)(c16 * HD + dpart * kDimsPerWave + r4 * 8) * 2u;  // bytes
    const int32_t *pt = a.page_table + (int64_t)b * a.pt_stride;
    const int pg_hi = npg > 0 ? pg1 : 0;  // last page-table entry this workgroup may read
    auto page_of = [&](int i) { return pg0 + grp + NGRP * i; };

    // ---- page ids, 64 at a time in one vector register: lane j holds the id of the group's
    // page 64*k + j. Pages read their id back with readlane, so no page waits on a scalar
    // load; the next 64 ids are fetched one block ahead. Out-of-range indices are clamped to
    // an entry the workgroup owns (their ids are never used).
    auto load_ids = [&](int first) { return pt[min(page_of(first + lane), pg_hi)]; };
    int ids = load_ids(0);
    int ids_next = load_ids(64);

    // ---- Q^T as the B operand, staged once in LDS for the 16 MFMA columns (the g real
    // heads, zeros for the rest); each page reads lane's head c16, 8 dims per K-step.
    constexpr int kQItems = 16 * (HD / 8) / kThreads;
    u32x4 qv[kQItems];
#pragma unroll
    for (int k = 0; k < kQItems; ++k) {
        const int e = threadIdx.x + k * kThreads;
        const int hn = e / (HD / 8), d8 = (e % (HD / 8)) * 8;
        // unconditional load of a valid head, zeroed afterwards for the padding columns
        const u32x4 v = *(const u32x4 *)(a.q + ((int64_t)b * Hq + kvh * g + min(hn, g - 1)) * HD + d8);
        qv[k] = hn < g ? v : u32x4{0, 0, 0, 0};
    }
    const uint16_t *q_lane = sm_q + c16 * kQStride + dpart * kDimsPerWave + r4 * 8;
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

    // Buffer resource of this KV head's block in page i of the group's list. Past the end of
    // the list, or for a page id outside the pool, the resource has zero size: its loads
    // return zeros without touching memory, so every load can be issued unconditionally
    // (which keeps the compiler's wait counts exact across the software pipeline).
    auto page_rsrc = [&](const uint16_t *pool, int i, int ib) {
        const int rel = i - ib;  // 0..65: position in ids (or, past 63, in ids_next)
        int pid = __builtin_amdgcn_readlane(rel >= 64 ? ids_next : ids, rel & 63);
        bool live = i < cnt;
        if (live && (pid < 0 || pid >= a.num_pages)) {
            bad_page = 1;
            live = false;
        }
        if (!live)
            pid = 0;
        const uint16_t *base = pool + ((int64_t)pid * a.num_kv_heads + kvh) * blk;
        return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, live ? (int)(blk * 2) : 0, 0x00020000);
    };
    auto load_regs = [&](PageRegs &R, __amdgpu_buffer_rsrc_t rsrc) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
            R.r[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_off, s * 64, 0));
        __builtin_amdgcn_sched_barrier(0);  // keep the whole page's loads ahead of the math
    };
    // Scores of page i (this wave's dims; with paired waves the two halves are added in a
    // fixed order, low dims first), online-softmax update and rescale of the accumulator.
    // Returns P^T (bf16, the B operand of the PV product) and the lane's valid tokens.
    auto qk_softmax = [&](PageRegs &K, int i, bool (&valid)[4]) {
        const int t0 = page_of(i) * kPage;
        f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s)
            st = mfma_k32(K.r[s], *(const u32x4 *)(q_lane + s * 32), st);
        if (DS > 1) {
            f32x4 *buf = sm_s[i & 1];
            buf[wave * 64 + lane] = st;
            __syncthreads();
            const f32x4 other = buf[(wave ^ 1) * 64 + lane];
            st = dpart == 0 ? st + other : other + st;
        }
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
    auto pv = [&](PageRegs &V, int i, u32x2 pb, const bool (&valid)[4]) {
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
    // One page of the group: its scores (always, so paired waves meet at their barrier),
    // then the softmax update and PV product if the page exists for this group.
    auto page_step = [&](PageRegs &K, PageRegs &V, int i) {
        bool valid[4];
        if (DS > 1 && i >= cnt) {  // dummy trip: only the partial-score exchange
            f32x4 *buf = sm_s[i & 1];
            buf[wave * 64 + lane] = f32x4{0.f, 0.f, 0.f, 0.f};
            __syncthreads();
            return;
        }
        const u32x2 pb = qk_softmax(K, i, valid);
        pv(V, i, pb, valid);
    };

    // ---- pipeline: K one page ahead of the math; V too when there is room (VBUF = 2),
    // otherwise V's single buffer is refilled right after each PV product (VBUF = 1)
    constexpr int VBUF = (SHARED || OCC == 1) ? 2 : 1;
    PageRegs KA, KB, VA, VB;
    load_regs(KA, page_rsrc(a.k_pool, 0, 0));  // unconditional: empty resource when cnt == 0
    if (!SHARED)
        load_regs(VA, page_rsrc(a.v_pool, 0, 0));
#pragma unroll
    for (int k = 0; k < kQItems; ++k) {
        const int e = threadIdx.x + k * kThreads;
        *(u32x4 *)(sm_q + (e / (HD / 8)) * kQStride + (e % (HD / 8)) * 8) = qv[k];
    }
    __syncthreads();

    for (int i = 0; i < trips; i += 2) {
        // page ids: the block of 64 holding page i is `ids`, the following block `ids_next`
        if ((i & 63) == 0 && i > 0) {
            ids = ids_next;
            ids_next = load_ids(i + 64);
        }
        const int ib = i & ~63;  // page index of ids' lane 0
        // page i in KA/VA; page i+1 goes to KB (and VB, or VA after the PV product)
        load_regs(KB, page_rsrc(a.k_pool, i + 1, ib));
        if (!SHARED && VBUF == 2)
            load_regs(VB, page_rsrc(a.v_pool, i + 1, ib));
        page_step(KA, SHARED ? KA : VA, i);
        if (!SHARED && VBUF == 1)
            load_regs(VA, page_rsrc(a.v_pool, i + 1, ib));
        if (i + 1 >= trips)
            break;
        // page i+1 in KB/(VB or VA); page i+2 goes to KA (and VA)
        load_regs(KA, page_rsrc(a.k_pool, i + 2, ib));
        if (!SHARED && VBUF == 2)
            load_regs(VA, page_rsrc(a.v_pool, i + 2, ib));
        page_step(KB, SHARED ? KB : (VBUF == 2 ? VB : VA), i + 1);
        if (!SHARED && VBUF == 1)
            load_regs(VA, page_rsrc(a.v_pool, i + 2, ib));
    }

    // ---- merge the page groups (fixed order) and write this split's result
    if (dpart == 0 && r4 == 0) {
        sm_m[grp][c16] = m_run;
        sm_l[grp][c16] = l_run;
    }
    if (lane == 0)
        sm_bad[wave] = bad_page;
    for (int h0 = 0; h0 < g; h0 += kChunk) {
        __syncthreads();
        if (c16 >= h0 && c16 < min(g, h0 + kChunk)) {
            float *dst = sm_o + (grp * kChunk + (c16 - h0)) * HD + dpart * kDimsPerWave + 4 * r4;
#pragma unroll
            for (int j = 0; j < NT; ++j)
                *(f32x4 *)(dst + 16 * j) = acc[j];
        }
        __syncthreads();
        bool bad = bad_len;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            bad = bad || sm_bad[w];
        const int nh = min(g, h0 + kChunk) - h0;
        for (int e = threadIdx.x; e < nh * HD; e += kThreads) {
            const int hn = h0 + e / HD, d = e % HD;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NGRP; ++w)
                M = fmaxf(M, sm_m[w][hn]);
            float lsum = 0.f, o = 0.f;
#pragma unroll
            for (int w = 0; w < NGRP; ++w) {
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
    return hipLaunchKernel((const void *)decode_split_kernel<HD, SHARED, kOcc>, grid, dim3(kThreads), args, 0,
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
