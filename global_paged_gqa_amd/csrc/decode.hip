// Split-KV flash-decode for hybrid paged GQA attention on gfx950.
//
// One workgroup = one (row, KV head, split). A split is the keys of one row in
// [s*S, (s+1)*S) intersected with the row's visible range, S = split_tokens
// (the split-KV chunk policy of the pegainfer "[Model] Gemma 4 M3 31B" plan;
// the flash-decode split factor of the Core AI card's "--metal-sdpa" section).
// Local rows only visit the splits that intersect their window, so a row with a
// 32768-token context still reads at most `window` keys (the sliding-window
// tile pruning that the vllm-gemma-4-31b skills page, "Three load-bearing facts",
// credits with a 3-4x gain).
//
// Memory path. Decode reads every visible K/V byte exactly once, so it is bound by
// HBM bandwidth. Each page's (page, KV head) block is contiguous in the pool, and it
// is copied global -> LDS with 16-byte-per-lane buffer loads that read 1 KB of
// consecutive bytes per instruction (reading 16 token rows x 64 B per instruction
// straight into MFMA operand registers caps the same gather well below the
// contiguous rate). The loads are non-temporal (every byte is read once) and go
// straight to LDS, holding no registers.
//
// Work split. A split's pages form C page streams (at head_dim 512 four with K = V, two with
// separate pools, one over FP8 pools; two at 256): stream c takes pages c, c+C, c+2C, ... and
// keeps its own online-softmax state over the whole head dimension, and the states fold in stream
// order. A wave streams its pages through its own slice of LDS (two or three K/V units ahead of
// the math, waited for with explicit per-wave load counts, no barriers); a launch shape puts one,
// two or four streams on each wave. Per page (16 tokens), in registers:
//   S^T[16 tok][16 heads] = K[tok][:] . Q^T[:][heads]    (MFMA 16x16x32, A = K read
//                                                         from LDS, B = Q^T in registers)
//   online softmax on S^T columns                         (VALU, lane swaps)
//   O^T[dims][heads] += V^T[dims][tok] . P^T[tok][heads]  (MFMA 16x16x16, A = V^T from
//                        the gfx950 transpose read of the page, B = P^T straight from the
//                        score tile's accumulator layout)
// The g query heads sharing the KV head fill the 16 MFMA columns (padding heads have
// zero queries and are never written). The fold order is fixed, so the result does not
// depend on timing, on the batch or on the launch shape.
//
// FP8 pools (the opt-in FP8 KV pool for the sliding family of the pegainfer "[Model] Gemma 4
// M2 26B-A4B" plan). K and V elements are OCP E4M3 bytes standing for value * k_scale and
// value * v_scale. A page unit is half as many bytes and is staged the same way; each 16-byte
// LDS chunk then holds 16 dims instead of 8. Every code is widened exactly to bf16 in registers
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1: E4M3 values are a subset of bf16), so the MFMAs
// are the bf16 ones:
//   K: one 16-byte chunk read gives a lane two K-steps' operands (dims 64 j + 16 r4 + 0..7 and
//      8..15); Q^T is loaded in the same dim order.
//   V: the same transpose read returns 2-byte elements, now two adjacent dims of four tokens;
//      two byte permutes split them into one 4-token word per dim, so output tile 2T + h holds
//      dims 32 T + 2 c + h.
// k_scale is folded into the score scale and v_scale into the final normalisation.
#include "common.h"
#include "kernels.h"

namespace gattn {

namespace {

constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)

// Four E4M3 codes -> four bf16 values (exact), low word first.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t w) {
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}

// One side of a stream-state fold for one column: R (+) S scales both sides to the larger of their
// reference maxima and adds them (see the kernel below). An empty side (reference -inf) weighs 0.
struct FoldScales {
    float m, a, c;  // the folded reference, R's factor, S's factor
};
__device__ __forceinline__ FoldScales fold_scales(float mr, float ms) {
    const float M = fmaxf(mr, ms);
    return {M, mr == -INFINITY ? 0.f : fast_exp2(mr - M), ms == -INFINITY ? 0.f : fast_exp2(ms - M)};
}
__device__ __forceinline__ float fold1(float r, float s, const FoldScales &f) { return __builtin_fmaf(s, f.c, r * f.a); }

// A value parked in an accumulation register for the length of a page stream: it is touched only
// between streams, so it stays out of the vector registers the page loop works in.
__device__ __forceinline__ float park(float v) {
    float r;
    asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(r) : "v"(v));
    return r;
}
__device__ __forceinline__ float unpark(float r) {
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(r));
    return v;
}

template <int HD, bool SHARED, int W, int kSliceBytes, bool F8 = false, int NS = 1>
__global__ __launch_bounds__(NS * W * 64) void decode_split_kernel(DecodeArgs a) {
    // A split's pages form C page streams: stream c takes pages c, c + C, c + 2C, ... of the split
    // and keeps its own online-softmax state S_c. The states fold in stream order,
    // R = ((S_0 (+) S_1) (+) S_2) (+) S_3 (with two streams S_0 (+) S_1). W waves run the C streams,
    // E = C / W each, one after another: wave w runs streams w E .. w E + E - 1 and folds them in
    // order in its registers. With one stream per wave the waves' states meet in LDS and each output
    // element folds them in wave order; with two streams on each of two waves, wave 0 hands its fold
    // to wave 1 through LDS. Every launch shape thus applies the same operations to the same values,
    // so it gives the same bits. NS > 1: the workgroup takes all NS split slots of its (row, KV
    // head), one group of W waves per slot, and merges them itself.
    // Page streams of a split: four at head_dim 512 with K = V, two with separate K and V pools (whose
    // waves carry twice the bytes per page), one over FP8 pools (whose only launch shape is one wave
    // per split); two at 256.
    constexpr int C = HD == 512 ? (F8 ? 1 : (SHARED ? 4 : 2)) : 2;
    constexpr int E = C / W;                    // streams per wave
    constexpr int kWaves = NS * W;
    constexpr int kThreads = kWaves * 64;
    constexpr int kRingBytes = kWaves * kSliceBytes;
    constexpr int NKS = HD / 32;                // K-steps of 32 dims in a score
    constexpr int NDT = HD / 16;                // 16-dim output tiles
    constexpr int ESZ = F8 ? 1 : 2;             // bytes per K/V element
    constexpr int ROWB = HD * ESZ;              // bytes of a token row
    constexpr int UNIT = kPage * ROWB;          // one page's K (or V), one KV head
    constexpr int UPP = SHARED ? 1 : 2;         // units per page
    constexpr int SUB = kSliceBytes;
    constexpr int NU = SUB / UNIT;              // units in a slice
    constexpr int LPU = UNIT / 1024;            // 1 KB load instructions per unit
    constexpr int CPR = ROWB / 16;              // 16-byte chunks per token row
    // The score of a page is formed as NCH partial products over consecutive quarters (halves at
    // head_dim 256) of the head dims, their steps interleaved, added in a fixed tree.
    constexpr int NCH = HD == 512 ? 4 : 2;
    constexpr int FOLDF = 16 * HD;              // floats of one state's O in LDS (16 columns)
    static_assert(C % W == 0 && (W == 1 || E <= 2), "stream shape");
    static_assert(CPR >= 16 && LPU >= 1, "row shape");
    static_assert(NU >= 2, "decode ring shape");
    static_assert(NU * LPU + 1 <= 63, "vmcnt range");
    static_assert(FOLDF * 4 <= SUB, "state buffers");
    static_assert(NS == 1 || HD == 256, "merged slots");

    __shared__ __attribute__((aligned(1024))) uint8_t ring[kRingBytes];
    constexpr int NFB = E == 1 ? W : (W > 1 ? 2 : 1);  // state buffers in LDS
    __shared__ float sm_fm[NS][NFB][16];   // states in LDS: reference maxima,
    __shared__ float sm_fl[NS][NFB][16];   // sums of the bf16 weights (normalise O),
    __shared__ float sm_flx[NS][NFB][16];  // sums of the fp32 weights (LSE)
    __shared__ int sm_bad[NS][W];
    __shared__ float sm_lse[NS][16];     // merged slots: each slot's LSE per head

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave / W;                   // split slot within the workgroup
    const int pw = wave % W;                    // wave within the slot's group
    const int c16 = lane & 15;  // MFMA row/column index of this lane
    const int r4 = lane >> 4;   // 16-lane row of this lane
    const int slot = NS > 1 ? grp : (int)blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
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
    // A split outside the visible range is empty. On its own it marks its slot and ends; as a
    // slot of a merging workgroup its waves stream nothing and still reach every barrier, and its
    // state gives lse = -inf, which the final merge skips.
    const bool empty = !bad_len && tb >= te;
    if constexpr (NS == 1) {
        if (empty) {
            if (threadIdx.x < g)
                a.lse_part[((int64_t)b * Hq + kvh * g + threadIdx.x) * a.n_slots + slot] = -INFINITY;
            return;
        }
    }
    // (an empty slot's tb may lie past the row's last table entry: it reads entry 0 instead)
    const int pg0 = bad_len || empty ? 0 : tb / kPage;
    const int npg = bad_len || empty ? 0 : (te - 1) / kPage - pg0 + 1;
    // pages of stream c, and the pages of this wave's streams in the order it runs them
    auto stream_pages = [&](int c) { return npg > c ? (npg - c + C - 1) / C : 0; };
    int my_pages = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
        my_pages += stream_pages(pw * E + e);
    // table index of the wave's k-th page (k < my_pages; a larger k lands past the split)
    auto page_of = [&](int k) {
        int c = pw * E;
#pragma unroll
        for (int e = 0; e < E - 1; ++e) {
            const int n = stream_pages(c);
            if (k >= n) {
                k -= n;
                ++c;
            }
        }
        return pg0 + c + k * C;
    };
    const int32_t *pt = a.page_table + (int64_t)b * a.pt_stride;
    const int pg_hi = npg > 0 ? pg0 + npg - 1 : pg0;  // last table entry this workgroup may read

    // ---- this wave's page ids, 64 at a time in one vector register (lane j: the wave's page
    // 64k + j), read back with readlane when a page is issued. Indices past the wave's pages are
    // clamped to an entry the workgroup owns (their ids are never used).
    auto load_ids = [&](int first) { return pt[min(page_of(first + lane), pg_hi)]; };
    int ids = load_ids(0), ids_next = load_ids(64);
    int ids_base = 0;

    // ---- Q^T as the B operand of the score product: lane holds head c16 (zeros past g),
    // dims 32 s + 8 r4 .. +7 (FP8: 64 (s / 2) + 16 r4 + 8 (s % 2) .. +7)
    u32x4 qb[NKS];
    {
        const uint16_t *qp = a.q + ((int64_t)b * Hq + kvh * g + min(c16, g - 1)) * HD + (F8 ? 16 : 8) * r4;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const u32x4 v = *(const u32x4 *)(qp + (F8 ? 64 * (s >> 1) + 8 * (s & 1) : 32 * s));
            qb[s] = c16 < g ? v : u32x4{0, 0, 0, 0};
        }
    }

    // ---- per-lane LDS byte offsets. The swizzle only permutes the low four bits of a chunk
    // index, so operand offsets repeat with a period of 16 chunks (256 bytes) and the rest of
    // each offset is an immediate.
    // K operand (step s): token c16, logical chunk 4 s + r4 -> kbase[s % 4] + 256 (s / 4)
    // (FP8: chunk 4 j + r4 feeds steps 2 j and 2 j + 1)
    uint32_t kbase[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        kbase[j] = (uint32_t)(c16 * ROWB + ((4 * j + r4) ^ dswz(c16)) * 16);
    // V^T operand (dim tile dt): in 16-lane group r4, lane 4r + q supplies token 4 r4 + r,
    // dims 16 dt + 4q .. +3; the lane receives dim 16 dt + c16 of those four tokens.
    // -> vbase[dt % 8] + 256 (dt / 8)
    uint32_t vbase[8];
    {
        const int t = 4 * r4 + (c16 >> 2), q = c16 & 3;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            vbase[j] = (uint32_t)(t * ROWB + ((2 * j + (q >> 1)) ^ dswz(t)) * 16 + 8 * (q & 1));
    }
    // ring fill: instruction i of a unit writes lane's 16 bytes to the slice's chunk position
    // P = 64 i + lane, which holds token P / CPR at chunk slot P % CPR, i.e. that token's chunk
    // (slot ^ dswz(token)) of the page block.
    auto src_off = [&](int i) {
        const int P = 64 * i + lane;
        const int t = P / CPR;
        return (uint32_t)(t * ROWB + ((P % CPR) ^ dswz(t)) * 16);
    };

    f32x4 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f, l_ex = 0.f;
    // E > 1: the state of the wave's earlier streams (wave 0: their fold; wave 1 of two: its
    // first stream, which folds after the earlier waves' streams)
    float sv[E > 1 ? 4 * NDT : 1];  // parked: sv[4 dt + q] is element q of tile dt
    float sv_m = -INFINITY, sv_l = 0.f, sv_lx = 0.f;
    int bad_page = 0;
    uint8_t *const sub = ring + wave * SUB;
    const uint32_t sub_lds = (uint32_t)(uintptr_t)sub;

    // Issue unit u of this wave's page sequence (its page u / UPP; K, or V when u is odd and the
    // pools are separate) into slice slot u % NU. Pages past the wave's share, and page ids
    // outside the pool, get a zero-size buffer resource: their loads write zeros and touch no
    // memory, so the wave always has exactly LPU loads per unit in flight and the waits below
    // stay exact. The slot's previous unit has been read: its LDS reads are waited for first.
    auto issue = [&](int u) {
        const int k = u / UPP;
        if (k - ids_base >= 64) {  // slide the id window
            ids = ids_next;
            ids_base += 64;
            ids_next = load_ids(ids_base + 64);
        }
        int pid = __builtin_amdgcn_readlane(ids, k - ids_base);
        bool live = k < my_pages;
        if (live && (pid < 0 || pid >= a.num_pages)) {
            bad_page = 1;
            live = false;
        }
        if (!live)
            pid = 0;
        const uint8_t *pool = (const uint8_t *)((SHARED || (u & 1) == 0) ? a.k_pool : a.v_pool);
        const u32x4 rs = raw_rsrc(pool + ((int64_t)pid * a.num_kv_heads + kvh) * UNIT, live ? UNIT : 0);
        const uint32_t dst = sub_lds + (uint32_t)((u % NU) * UNIT);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int i = 0; i < LPU; ++i)
            ring_load16<true>(rs, dst + i * 1024, src_off(i));
    };

    // Q and the first page ids are in registers before the stream starts, so that the only
    // vector-memory operations the waits below count are the stream's own loads.
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int u = 0; u < NU; ++u)
        issue(u);

    // The stream is done: the wave's first stream is kept as is, a later one (wave 0 of a
    // single-wave shape) folds into the kept state; the next stream starts afresh.
    auto end_stream = [&](int e) {
        if constexpr (E == 1)
            return;
        else if (e == 0) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sv[4 * dt + q] = park(acc[dt][q]);
            sv_m = m_run;
            sv_l = l_run;
            sv_lx = l_ex;
        } else {
            const FoldScales f = fold_scales(sv_m, m_run);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    sv[4 * dt + q] = park(fold1(unpark(sv[4 * dt + q]), acc[dt][q], f));
            sv_m = f.m;
            sv_l = fold1(sv_l, l_run, f);
            sv_lx = fold1(sv_lx, l_ex, f);
        }
        // a stream's first page overwrites the accumulators; an empty stream's state is zero
        if (stream_pages(pw * E + e + 1) == 0) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        m_run = -INFINITY;
        l_run = 0.f;
        l_ex = 0.f;
    };
    int u = 0;
    int c = pw * E, ip = 0, nc = stream_pages(c);  // the current stream, its page index, its pages
    for (int k = 0; k < my_pages; ++k) {
        if constexpr (E > 1) {
            while (ip == nc) {  // (an empty stream ends at once)
                end_stream(c - pw * E);
                ++c;
                ip = 0;
                nc = stream_pages(c);
            }
        }
        const int t0 = (pg0 + c + ip * C) * kPage;
        // ---- K unit u landed once at most the NU - 1 later units' loads are outstanding
        wait_vmcnt<(NU - 1) * LPU>();
        const uint8_t *ks = sub + (u % NU) * UNIT;
        // the partial chains (chain h: K-steps [h NKS/NCH, (h+1) NKS/NCH)), their steps
        // interleaved so that consecutive MFMAs are independent
        f32x4 ch[NCH];
#pragma unroll
        for (int h = 0; h < NCH; ++h)
            ch[h] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (F8) {
            // chunk j holds the operands of steps 2 j (its low 8 bytes) and 2 j + 1
            u32x4 kc[NKS / 2];
#pragma unroll
            for (int j = 0; j < NKS / 2; ++j)
                kc[j] = *(const u32x4 *)(ks + kbase[j & 3] + 256 * (j >> 2));
#pragma unroll
            for (int i2 = 0; i2 < NKS / NCH; ++i2)
#pragma unroll
                for (int h = 0; h < NCH; ++h) {
                    const int s = h * (NKS / NCH) + i2;
                    const u32x4 w = kc[s >> 1];
                    const u32x2 lo = e4m3x4_to_bf16((s & 1) ? w[2] : w[0]);
                    const u32x2 hi = e4m3x4_to_bf16((s & 1) ? w[3] : w[1]);
                    ch[h] = mfma_k32(u32x4{lo[0], lo[1], hi[0], hi[1]}, qb[s], ch[h]);
                }
        } else {
#pragma unroll
            for (int i2 = 0; i2 < NKS / NCH; ++i2)
#pragma unroll
                for (int h = 0; h < NCH; ++h) {
                    const int s = h * (NKS / NCH) + i2;
                    ch[h] = mfma_k32(*(const u32x4 *)(ks + kbase[s & 3] + 256 * (s >> 2)), qb[s], ch[h]);
                }
        }
        f32x4 st;
        if constexpr (NCH == 4)
            st = (ch[0] + ch[1]) + (ch[2] + ch[3]);
        else
            st = ch[0] + ch[1];
        if (!SHARED)
            issue(u + NU);

        // ---- online softmax; lane holds S^T[token t0 + 4 r4 + e][head c16]. Tokens outside
        // [tb, te) are selected out (a NaN in an unused slot never reaches the sums).
        float mx = -INFINITY;
        if (t0 >= tb && t0 + kPage <= te) {  // interior page: every token visible
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                st[e2] *= a.scale_log2;
                mx = fmaxf(mx, st[e2]);
            }
        } else {
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const int t = t0 + 4 * r4 + e2;
                st[e2] = (t >= tb && t < te) ? st[e2] * a.scale_log2 : -INFINITY;
                mx = fmaxf(mx, st[e2]);
            }
        }
        // Lazy rescale: a column keeps its reference maximum until a score exceeds it by more
        // than 2^8, so P stays below 256 and the accumulators are rescaled only on those pages.
        // O is normalised by the sum of the bf16-rounded weights the PV product uses, so a
        // weight's rounding scales numerator and denominator alike (a single dominant key gives
        // exactly its V row, whatever the reference); the LSE uses the sum of the fp32 weights.
        // Both share the reference maximum. The weights are formed against the current
        // reference while the column maxima are still being reduced, and formed again on the
        // rare pages where a column moves its reference; the sums are taken after the PV
        // product is issued. Only the order of independent work differs from forming them in
        // sequence: the results are the same.
        float ps[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
            ps[e2] = fast_exp2(st[e2] - m_run);
        const float m_new = fmaxf(m_run, rows_max4(mx));
        const bool resc = m_new > m_run + kRescaleLog2;
        float alpha = 1.0f;
        if (__builtin_amdgcn_ballot_w64(resc)) {
            if (resc) {
                alpha = fast_exp2(m_run - m_new);
                m_run = m_new;
            }
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2)
                ps[e2] = fast_exp2(st[e2] - m_run);
            if (ip > 0) {  // a stream's first product starts from zero instead
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    acc[dt] *= alpha;
            }
        }
        const u32x2 pb = {pack_bf16x2(ps[0], ps[1]), pack_bf16x2(ps[2], ps[3])};

        // ---- O^T += V^T P^T over the whole head dimension
        const int uv = SHARED ? u : u + 1;
        if (!SHARED)
            wait_vmcnt<(NU - 1) * LPU>();
        uint8_t *vs = sub + (uv % NU) * UNIT;
        // Tokens outside [tb, te) carry P = 0, but their V slot may hold anything (a NaN, say,
        // and 0 * NaN is NaN): on the split's first and last page their V rows are zeroed in
        // the slice before the product. (With K = V the scores have already been read.)
        if (t0 < tb || t0 + kPage > te) {
#pragma unroll
            for (int r = 0; r < kPage; ++r) {
                const int t = t0 + r;
                if ((t < tb || t >= te) && lane * 16 < ROWB)
                    *(u32x4 *)(vs + r * ROWB + lane * 16) = u32x4{0, 0, 0, 0};
            }
        }
        // (the first page of a stream accumulates onto zero: its accumulators are not read)
        auto pv = [&](bool from_zero) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            if constexpr (F8) {
                // read T: element c16 of the tile is dims 32 T + 2 c16 (low byte) and + 1 of four tokens
#pragma unroll
                for (int T = 0; T < NDT / 2; ++T) {
                    const u32x2 w = tr_read(vs + vbase[T & 7] + 256 * (T >> 3));
                    acc[2 * T] = mfma_k16(e4m3x4_to_bf16(__builtin_amdgcn_perm(w[1], w[0], 0x06040200u)), pb,
                                          from_zero ? z : acc[2 * T]);
                    acc[2 * T + 1] = mfma_k16(e4m3x4_to_bf16(__builtin_amdgcn_perm(w[1], w[0], 0x07050301u)), pb,
                                              from_zero ? z : acc[2 * T + 1]);
                }
            } else {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    acc[dt] = mfma_k16(tr_read(vs + vbase[dt & 7] + 256 * (dt >> 3)), pb, from_zero ? z : acc[dt]);
            }
        };
        if (ip == 0)
            pv(true);
        else
            pv(false);
        const float rs = ((bf16_lo(pb[0]) + bf16_hi(pb[0])) + bf16_lo(pb[1])) + bf16_hi(pb[1]);
        const float rx = ((ps[0] + ps[1]) + ps[2]) + ps[3];
        l_run = l_run * alpha + rows_sum4(rs);
        l_ex = l_ex * alpha + rows_sum4(rx);
        issue(uv + NU);
        u = uv + 1;
        ++ip;
    }
    if constexpr (E > 1) {
        for (; c < pw * E + E - 1; ++c)  // the streams that ended with the last page, or were empty
            end_stream(c - pw * E);
    }
    // No stream load (the zero-filling ones past the wave's pages included) may still be
    // writing LDS when the slices are reused below.
    wait_vmcnt<0>();

    // Wave 0 of a shape with several streams per wave folds its last stream onto the kept state.
    if constexpr (E > 1) {
        if (pw == 0) {
            const FoldScales f = fold_scales(sv_m, m_run);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[dt][q] = fold1(unpark(sv[4 * dt + q]), acc[dt][q], f);
            m_run = f.m;
            l_run = fold1(sv_l, l_run, f);
            l_ex = fold1(sv_lx, l_ex, f);
        }
    }

    // ---- the waves' states meet in LDS (buffers of 16 x HD floats in the slot group's slices,
    // element (column h, dim d) at h HD + d). One stream per wave: every wave publishes its state
    // and the output loop folds them in wave order. Two streams per wave on two waves: wave 0
    // hands its fold to wave 1, which folds its own two streams onto it and publishes the result.
    const bool wave_bad = __builtin_amdgcn_ballot_w64(bad_page) != 0;
    if (lane == 0)
        sm_bad[grp][pw] = wave_bad;
    float *const fb = (float *)(ring + grp * W * SUB);
    // the wave's O into fold buffer j (FP8: tiles 2T and 2T + 1 interleave, element i of each
    // being dim 32 T + 8 r4 + 2 i (+ 1))
    auto put_state = [&](int j) {
        float *dst = fb + j * FOLDF + c16 * HD;
        if (c16 >= g) {  // padding columns: never read
        } else if constexpr (F8) {
#pragma unroll
            for (int T = 0; T < NDT / 2; ++T) {
                const f32x4 ev = acc[2 * T], od = acc[2 * T + 1];
                *(f32x4 *)(dst + 32 * T + 8 * r4) = f32x4{ev[0], od[0], ev[1], od[1]};
                *(f32x4 *)(dst + 32 * T + 8 * r4 + 4) = f32x4{ev[2], od[2], ev[3], od[3]};
            }
        } else {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                *(f32x4 *)(dst + 16 * dt + 4 * r4) = acc[dt];
        }
        if (r4 == 0) {
            sm_fm[grp][j][c16] = m_run;
            sm_fl[grp][j][c16] = l_run;
            sm_flx[grp][j][c16] = l_ex;
        }
    };
    __syncthreads();  // every wave is done with its slice
    if constexpr (E == 1)
        put_state(pw);
#pragma unroll
    for (int w = 1; w < (E == 1 ? 1 : W); ++w) {
        const int j = (w - 1) & 1;
        if (pw == w - 1)
            put_state(j);
        __syncthreads();
        if (pw == w) {
            // R (the earlier waves' fold, from LDS) (+) this wave's streams, in stream order
            const float mp = sm_fm[grp][j][c16];
            const FoldScales f1 = fold_scales(mp, E > 1 ? sv_m : m_run);
            const FoldScales f2 = fold_scales(f1.m, m_run);
            const float *src = fb + j * FOLDF + c16 * HD;
            auto fold_elem = [&](float rp, int dt, int q) {
                if constexpr (E > 1)
                    acc[dt][q] = fold1(fold1(rp, unpark(sv[4 * dt + q]), f1), acc[dt][q], f2);
                else
                    acc[dt][q] = fold1(rp, acc[dt][q], f1);
            };
            if constexpr (F8) {
#pragma unroll
                for (int T = 0; T < NDT / 2; ++T) {
                    const f32x4 x0 = c16 < g ? *(const f32x4 *)(src + 32 * T + 8 * r4) : f32x4{0.f, 0.f, 0.f, 0.f};
                    const f32x4 x1 = c16 < g ? *(const f32x4 *)(src + 32 * T + 8 * r4 + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
                    fold_elem(x0[0], 2 * T, 0);
                    fold_elem(x0[1], 2 * T + 1, 0);
                    fold_elem(x0[2], 2 * T, 1);
                    fold_elem(x0[3], 2 * T + 1, 1);
                    fold_elem(x1[0], 2 * T, 2);
                    fold_elem(x1[1], 2 * T + 1, 2);
                    fold_elem(x1[2], 2 * T, 3);
                    fold_elem(x1[3], 2 * T + 1, 3);
                }
            } else {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const f32x4 x = c16 < g ? *(const f32x4 *)(src + 16 * dt + 4 * r4) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        fold_elem(x[q], dt, q);
                }
            }
            const float lp = sm_fl[grp][j][c16], lxp = sm_flx[grp][j][c16];
            if constexpr (E > 1) {
                l_run = fold1(fold1(lp, sv_l, f1), l_run, f2);
                l_ex = fold1(fold1(lxp, sv_lx, f1), l_ex, f2);
                m_run = f2.m;
            } else {
                l_run = fold1(lp, l_run, f1);
                l_ex = fold1(lxp, l_ex, f1);
                m_run = f1.m;
            }
        }
    }
    // the buffer holding the fold of the streams before the output loop's own folds (E > 1: the
    // one the handover did not read)
    constexpr int JF = E == 1 ? 0 : (W - 1) & 1;
    constexpr int NFOLD = E == 1 ? W : 1;  // states the output loop folds, from buffer JF on
    if constexpr (E > 1) {
        if (pw == W - 1)
            put_state(JF);
    }
    __syncthreads();

    // each slot's result: element e of slot sl by one thread
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
    bool bad = bad_len;
#pragma unroll
    for (int w = 0; w < W; ++w)
        bad = bad || sm_bad[sl][w];
    const float *fin = (const float *)(ring + sl * W * SUB) + JF * FOLDF;
    for (int e = threadIdx.x * 4; e < g * HD; e += kThreads * 4) {
        const int hn = e / HD, d = e % HD;
        float M = sm_fm[sl][JF][hn], lsum = sm_fl[sl][JF][hn], lxsum = sm_flx[sl][JF][hn];
        f32x4 o = *(const f32x4 *)(fin + hn * HD + d);
#pragma unroll
        for (int w = 1; w < NFOLD; ++w) {
            const FoldScales f = fold_scales(M, sm_fm[sl][w][hn]);
            const f32x4 x = *(const f32x4 *)(fin + w * FOLDF + hn * HD + d);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = fold1(o[q], x[q], f);
            lsum = fold1(lsum, sm_fl[sl][w][hn], f);
            lxsum = fold1(lxsum, sm_flx[sl][w][hn], f);
            M = f.m;
        }
        const float inv = F8 ? a.v_scale / lsum : 1.0f / lsum;
        float lse = (M + fast_log2(lxsum)) * kLn2;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = bad ? __builtin_nanf("") : o[i] * inv;
        if (bad)
            lse = __builtin_nanf("");
        const int64_t bh = (int64_t)b * Hq + kvh * g + hn;
        if constexpr (NS > 1) {
            // kept for the merge (this thread read it last)
            *(f32x4 *)((float *)(ring + sl * W * SUB) + JF * FOLDF + hn * HD + d) = o;
            if (d == 0)
                sm_lse[sl][hn] = lse;
        } else if (direct) {
            *(u32x2 *)(a.out + bh * HD + d) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            if (d == 0)
                a.lse[bh] = lse;
        } else {
            *(f32x4 *)(a.o_part + (bh * a.n_slots + slot) * HD + d) = o;
            if (d == 0)
                a.lse_part[bh * a.n_slots + slot] = lse;
        }
    }
    }  // slots
    if constexpr (NS > 1) {
        // The slots merged with the arithmetic of the separate merge (combine.hip) on the same
        // values, so the bits match it: M the largest slot LSE (NaN propagates); the exp-sum as
        // (e0 + e1) + (e2 + e3); LSE = M + ln(sum); O = ((a0 + a1) + a2) + a3 with a_s = w_s o_s
        // by one fma; empty slots (lse = -inf) add zeros.
        static_assert(NS <= 4, "merged slots: the fixed four-sum order");
        __syncthreads();
        for (int e = threadIdx.x * 4; e < g * HD; e += kThreads * 4) {
            const int hn = e / HD, d = e % HD;
            float ls[4], M = -INFINITY;
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                ls[s2] = s2 < NS ? sm_lse[s2][hn] : -INFINITY;
                M = nan_max(M, ls[s2]);
            }
            const int64_t bh = (int64_t)b * Hq + kvh * g + hn;
            if (M == -INFINITY) {  // every slot empty
                *(u32x2 *)(a.out + bh * HD + d) = u32x2{0u, 0u};
                if (d == 0)
                    a.lse[bh] = -INFINITY;
                continue;
            }
            float ex[4];
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
                ex[s2] = ls[s2] == -INFINITY ? 0.f : __expf(ls[s2] - M);
            const float LSE = M + __logf((ex[0] + ex[1]) + (ex[2] + ex[3]));
            f32x4 part[4];
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                part[s2] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (s2 < NS && ls[s2] != -INFINITY) {
                    const float w = __expf(ls[s2] - LSE);
                    const f32x4 os = *(const f32x4 *)((const float *)(ring + s2 * W * SUB) + JF * FOLDF + hn * HD + d);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        part[s2][i] = __builtin_fmaf(w, os[i], 0.f);
                }
            }
            f32x4 o = part[0];
#pragma unroll
            for (int s2 = 1; s2 < 4; ++s2)
                o += part[s2];
            if (M != M)
                o = f32x4{M, M, M, M};
            *(u32x2 *)(a.out + bh * HD + d) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            if (d == 0)
                a.lse[bh] = LSE;
        }
    }
}

// Launch shape per head_dim, measured on the decode workloads of both families. head_dim 512
// (16 KB units): a batch of more than two workgroups per CU runs one wave per workgroup (all page
// streams of its split in turn) with two units in flight, four workgroups per CU, so that a
// batch's (row, KV head, split) items mostly start at once and no CU waits on a partly filled
// last round. With K = V a grid of at most one workgroup per CU (one long row, say) runs the four
// streams on four waves, and up to two workgroups per CU on two waves of two streams each; with
// separate pools a grid of up to two workgroups per CU (a batch of a single-KV-head family) runs
// its two streams on two waves: there one wave working through a split's pages one at a time
// would set the pace. head_dim 256 (8 KB units): the two page streams on two waves with three units each, three
// workgroups per CU, which keeps the window-sized local items (at most 1024 keys) from running
// one page at a time on few waves. Every shape gives the same bits.
template <int HD>
struct DecodeShape;
template <>
struct DecodeShape<512> {
    static constexpr int waves = 1, slice = 32 * 1024;
};
template <>
struct DecodeShape<256> {
    static constexpr int waves = 2, slice = 24 * 1024;
};
constexpr int kNumCUs = 256;

template <int HD, bool SHARED>
hipError_t launch(const DecodeArgs &a, dim3 grid, hipStream_t stream) {
    constexpr int W = DecodeShape<HD>::waves;
    constexpr int SLICE = DecodeShape<HD>::slice;
    void *args[] = {(void *)&a};
    if constexpr (HD == 256) {
        // two or three slots per row (a local row's window over its splits): one workgroup per
        // (row, KV head) runs them all and merges them, in place of the separate merge launch
        if (decode_merges_slots(HD, false, a.n_slots, (int64_t)grid.y * grid.z)) {
            const dim3 rows(1, grid.y, grid.z);
            if (a.n_slots == 2)
                return hipLaunchKernel((const void *)decode_split_kernel<HD, SHARED, W, SLICE, false, 2>, rows,
                                       dim3(2 * W * 64), args, 0, stream);
            return hipLaunchKernel((const void *)decode_split_kernel<HD, SHARED, W, SLICE, false, 3>, rows,
                                   dim3(3 * W * 64), args, 0, stream);
        }
    }
    if constexpr (HD == 512) {
        const int64_t items = (int64_t)grid.x * grid.y * grid.z;
        if constexpr (SHARED) {
            if (items <= kNumCUs)
                return hipLaunchKernel((const void *)decode_split_kernel<HD, SHARED, 4, SLICE>, grid, dim3(4 * 64),
                                       args, 0, stream);
        }
        if (items <= 2 * kNumCUs)
            return hipLaunchKernel((const void *)decode_split_kernel<HD, SHARED, 2, SLICE>, grid, dim3(2 * 64), args,
                                   0, stream);
    }
    return hipLaunchKernel((const void *)decode_split_kernel<HD, SHARED, W, SLICE>, grid, dim3(W * 64), args, 0,
                           stream);
}

}  // namespace

// FP8 pools: only while every (row, KV head) gets its own CU (at most one round of merging
// workgroups). A larger FP8 batch runs the unmerged kernel, whose small workgroups fit four to
// a CU (measured: merged, the 64-row local batch ran 9% slower and the 16-row sweep layer 8%
// faster). Both give the same bits.
bool decode_merges_slots(int head_dim, bool fp8, int n_slots, int64_t rows_x_kv_heads) {
    return head_dim == 256 && n_slots >= 2 && n_slots <= 3 && (!fp8 || rows_x_kv_heads <= kNumCUs);
}

// FP8 pools at head_dim 256 (4 KB units): two page streams of one wave with four units (two pages)
// each. A workgroup then holds 32 KB of LDS and the wave's registers allow two waves per SIMD, so
// four workgroups (eight waves, 128 KB of loads in flight) fit a CU; measured on the local decode
// workload, 8% faster than the bf16 shape's 24 KB slices (three workgroups per CU), with the same
// bits. At head_dim 512 (8 KB units) the bf16 shape: one wave, 32 KB.
hipError_t launch_decode_split_fp8(const DecodeArgs &a, int head_dim, bool kv_shared, int batch,
                                   hipStream_t stream) {
    const dim3 grid(a.n_slots, a.num_kv_heads, batch);
    void *args[] = {(void *)&a};
    const void *k = nullptr;
    int threads = 64;
    if (head_dim == 256 && !kv_shared) {
        if (decode_merges_slots(head_dim, true, a.n_slots, (int64_t)grid.y * grid.z)) {
            const dim3 rows(1, grid.y, grid.z);
            if (a.n_slots == 2)
                return hipLaunchKernel((const void *)decode_split_kernel<256, false, 2, 16 * 1024, true, 2>, rows,
                                       dim3(2 * 2 * 64), args, 0, stream);
            return hipLaunchKernel((const void *)decode_split_kernel<256, false, 2, 16 * 1024, true, 3>, rows,
                                   dim3(3 * 2 * 64), args, 0, stream);
        }
        k = (const void *)decode_split_kernel<256, false, 2, 16 * 1024, true>;
        threads = 128;
    } else if (head_dim == 512) {
        k = kv_shared ? (const void *)decode_split_kernel<512, true, 1, 32 * 1024, true>
                      : (const void *)decode_split_kernel<512, false, 1, 32 * 1024, true>;
    } else {
        return hipErrorInvalidValue;
    }
    return hipLaunchKernel(k, grid, dim3(threads), args, 0, stream);
}

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
