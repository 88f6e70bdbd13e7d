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
// Work split. The W waves of a workgroup (W = 1 for head_dim 512, 2 for 256) run
// independently: wave w takes pages w, w+W, w+2W, ... of the split, streams them through
// its own slice of LDS (two or three K/V units ahead of the math, waited for with explicit
// per-wave load counts, no barriers) and keeps its own online-softmax state over the whole
// head dimension. Per page (16 tokens), in registers:
//   S^T[16 tok][16 heads] = K[tok][:] . Q^T[:][heads]    (MFMA 16x16x32, A = K read
//                                                         from LDS, B = Q^T in registers)
//   online softmax on S^T columns                         (VALU, lane swaps)
//   O^T[dims][heads] += V^T[dims][tok] . P^T[tok][heads]  (MFMA 16x16x16, A = V^T from
//                        the gfx950 transpose read of the page, B = P^T straight from the
//                        score tile's accumulator layout)
// The g query heads sharing the KV head fill the 16 MFMA columns (padding heads have
// zero queries and are never written). At the end the wave states merge through LDS in a
// fixed order, so the result does not depend on timing or on the batch.
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

template <int HD, bool SHARED, int W, int DS, int kSliceBytes, bool F8 = false, int NS = 1>
__global__ __launch_bounds__(NS * W * DS * 64) void decode_split_kernel(DecodeArgs a) {
    // W page streams of DS waves each; a wave streams its share of the head dims of its
    // stream's pages through its own kSliceBytes of LDS. NS > 1: the workgroup takes all NS split
    // slots of its (row, KV head), one group of W * DS waves per slot, and merges them itself.
    constexpr int kWaves = NS * W * DS;
    constexpr int kThreads = kWaves * 64;
    constexpr int kRingBytes = kWaves * kSliceBytes;
    constexpr int NKS = HD / 32 / DS;            // K-steps of 32 dims in the wave's score partial
    constexpr int NDT = HD / 16 / DS;            // 16-dim output tiles of the wave
    constexpr int ESZ = F8 ? 1 : 2;              // bytes per K/V element
    constexpr int SEG = HD / DS;                 // head dims per wave
    constexpr int SEGB = SEG * ESZ;              // bytes of a token row's segment
    constexpr int PAGEB = kPage * HD * ESZ;      // bytes of one page's K (or V), one KV head
    constexpr int UNIT = kPage * SEGB;           // the wave's segment of it
    constexpr int UPP = SHARED ? 1 : 2;          // units per page
    constexpr int SUB = kSliceBytes;
    constexpr int NU = SUB / UNIT;               // units in a slice
    constexpr int LPU = UNIT / 1024;             // 1 KB load instructions per unit
    constexpr int CPR = SEGB / 16;               // 16-byte chunks per segment row
    // The score of a page is always formed as NCH partial products over consecutive quarters
    // (halves at head_dim 256) of the head dims, added in a fixed tree, whatever DS is: a wave
    // holds NCH / DS of them, so the sum, and everything after it, has the same bits for any DS.
    constexpr int NCH = HD == 512 ? 4 : 2;
    constexpr int CPW = NCH / DS;                // partial chains per wave
    static_assert(NCH % DS == 0 && (DS == 1 || W == 1), "dims split shape");
    static_assert(CPR >= 16 && LPU >= 1, "segment shape");
    static_assert(NU >= 2, "decode ring shape");
    static_assert(NU * LPU + 1 <= 63, "vmcnt range");
    static_assert(16 * HD * 4 <= DS * kSliceBytes, "merge buffer");
    static_assert(!F8 || DS == 1, "fp8 pools: whole head dims per wave");
    static_assert(NS == 1 || DS == 1, "merged slots: whole head dims per wave");
    static_assert(NS * W * 16 * HD * 4 <= kRingBytes, "merge buffer (merged slots)");

    __shared__ __attribute__((aligned(1024))) uint8_t ring[kRingBytes];
    __shared__ float sm_m[NS][W][16];
    __shared__ float sm_l[NS][W][16];   // row sums of the bf16 weights (normalise O)
    __shared__ float sm_lx[NS][W][16];  // row sums of the fp32 weights (LSE)
    __shared__ int sm_bad[NS][W];
    __shared__ f32x4 sm_part[2][DS][64];  // score partials of the dim-split waves (double buffer)
    __shared__ float sm_lse[NS][16];      // merged slots: each slot's LSE per head

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave / (W * DS);                            // split slot within the workgroup
    const int pw = (wave % (W * DS)) / DS, dq = wave % DS;      // page stream, head-dim segment
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
    // slot of a merging workgroup its waves stream nothing and still reach every barrier, and the
    // merge below gives it lse = -inf, which the final merge skips.
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
    const int my_pages = npg > pw ? (npg - pw + W - 1) / W : 0;  // this stream's: w, w+W, ...
    const int32_t *pt = a.page_table + (int64_t)b * a.pt_stride;
    const int pg_hi = npg > 0 ? pg0 + npg - 1 : pg0;  // last table entry this workgroup may read

    // ---- this wave's page ids, 64 at a time in one vector register (lane j: the wave's page
    // 64k + j), read back with readlane when a page is issued. Indices past the split are
    // clamped to an entry the workgroup owns (their ids are never used).
    auto load_ids = [&](int first) { return pt[min(pg0 + (first + lane) * W + pw, pg_hi)]; };
    int ids = load_ids(0), ids_next = load_ids(64);
    int ids_base = 0;

    // ---- Q^T as the B operand of the score product: lane holds head c16 (zeros past g),
    // dims SEG dq + 32 s + 8 r4 .. +7 (FP8: 64 (s / 2) + 16 r4 + 8 (s % 2) .. +7)
    u32x4 qb[NKS];
    {
        const uint16_t *qp = a.q + ((int64_t)b * Hq + kvh * g + min(c16, g - 1)) * HD + SEG * dq +
                             (F8 ? 16 : 8) * r4;
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
        kbase[j] = (uint32_t)(c16 * SEGB + ((4 * j + r4) ^ dswz(c16)) * 16);
    // V^T operand (dim tile dt): in 16-lane group r4, lane 4r + q supplies token 4 r4 + r,
    // dims 16 dt + 4q .. +3; the lane receives dim 16 dt + c16 of those four tokens.
    // -> vbase[dt % 8] + 256 (dt / 8)
    uint32_t vbase[8];
    {
        const int t = 4 * r4 + (c16 >> 2), q = c16 & 3;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            vbase[j] = (uint32_t)(t * SEGB + ((2 * j + (q >> 1)) ^ dswz(t)) * 16 + 8 * (q & 1));
    }
    // ring fill: instruction i of a unit writes lane's 16 bytes to the slice's chunk position
    // P = 64 i + lane, which holds token P / CPR at chunk slot P % CPR, i.e. that token's chunk
    // (slot ^ dswz(token)) of the wave's segment of the page block.
    auto src_off = [&](int i) {
        const int P = 64 * i + lane;
        const int t = P / CPR;
        return (uint32_t)(t * HD * ESZ + SEGB * dq + ((P % CPR) ^ dswz(t)) * 16);
    };

    f32x4 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
        acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f, l_ex = 0.f;
    int bad_page = 0;
    uint8_t *const sub = ring + wave * SUB;
    const uint32_t sub_lds = (uint32_t)(uintptr_t)sub;

    // Issue unit u of this wave's stream (its page u / UPP; K, or V when u is odd and the
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
        const u32x4 rs = raw_rsrc(pool + ((int64_t)pid * a.num_kv_heads + kvh) * PAGEB, live ? PAGEB : 0);
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

    int u = 0;
    for (int k = 0; k < my_pages; ++k) {
        const int t0 = (pg0 + k * W + pw) * kPage;
        // ---- K unit u landed once at most the NU - 1 later units' loads are outstanding
        wait_vmcnt<(NU - 1) * LPU>();
        const uint8_t *ks = sub + (u % NU) * UNIT;
        // this wave's partial chains (chain c: its K-steps [c NKS/CPW, (c+1) NKS/CPW)), their
        // steps interleaved so that consecutive MFMAs are independent
        f32x4 ch[CPW];
#pragma unroll
        for (int c = 0; c < CPW; ++c)
            ch[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (F8) {
            // chunk j holds the operands of steps 2 j (its low 8 bytes) and 2 j + 1
            u32x4 kc[NKS / 2];
#pragma unroll
            for (int j = 0; j < NKS / 2; ++j)
                kc[j] = *(const u32x4 *)(ks + kbase[j & 3] + 256 * (j >> 2));
#pragma unroll
            for (int i = 0; i < NKS / CPW; ++i)
#pragma unroll
                for (int c = 0; c < CPW; ++c) {
                    const int s = c * (NKS / CPW) + i;
                    const u32x4 w = kc[s >> 1];
                    const u32x2 lo = e4m3x4_to_bf16((s & 1) ? w[2] : w[0]);
                    const u32x2 hi = e4m3x4_to_bf16((s & 1) ? w[3] : w[1]);
                    ch[c] = mfma_k32(u32x4{lo[0], lo[1], hi[0], hi[1]}, qb[s], ch[c]);
                }
        } else {
#pragma unroll
            for (int i = 0; i < NKS / CPW; ++i)
#pragma unroll
                for (int c = 0; c < CPW; ++c) {
                    const int s = c * (NKS / CPW) + i;
                    ch[c] = mfma_k32(*(const u32x4 *)(ks + kbase[s & 3] + 256 * (s >> 2)), qb[s], ch[c]);
                }
        }
        f32x4 st;
        if constexpr (CPW == 4)
            st = (ch[0] + ch[1]) + (ch[2] + ch[3]);
        else if constexpr (CPW == 2)
            st = ch[0] + ch[1];
        else
            st = ch[0];
        if (!SHARED)
            issue(u + NU);
        if constexpr (DS > 1) {
            // the DS partials meet in LDS; every wave adds them in the same tree
            sm_part[k & 1][dq][lane] = st;
            __syncthreads();
            const f32x4 p0 = sm_part[k & 1][0][lane], p1 = sm_part[k & 1][1][lane];
            if constexpr (DS == 4)
                st = (p0 + p1) + (sm_part[k & 1][2][lane] + sm_part[k & 1][3][lane]);
            else
                st = p0 + p1;
        }

        // ---- online softmax; lane holds S^T[token t0 + 4 r4 + e][head c16]. Tokens outside
        // [tb, te) are selected out (a NaN in an unused slot never reaches the sums).
        float mx = -INFINITY;
        if (t0 >= tb && t0 + kPage <= te) {  // interior page: every token visible
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                st[e] *= a.scale_log2;
                mx = fmaxf(mx, st[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = t0 + 4 * r4 + e;
                st[e] = (t >= tb && t < te) ? st[e] * a.scale_log2 : -INFINITY;
                mx = fmaxf(mx, st[e]);
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
        for (int e = 0; e < 4; ++e)
            ps[e] = fast_exp2(st[e] - m_run);
        const float m_new = fmaxf(m_run, rows_max4(mx));
        const bool resc = m_new > m_run + kRescaleLog2;
        float alpha = 1.0f;
        if (__builtin_amdgcn_ballot_w64(resc)) {
            if (resc) {
                alpha = fast_exp2(m_run - m_new);
                m_run = m_new;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ps[e] = fast_exp2(st[e] - m_run);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                acc[dt] *= alpha;
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
                if ((t < tb || t >= te) && lane * 16 < SEGB)
                    *(u32x4 *)(vs + r * SEGB + lane * 16) = u32x4{0, 0, 0, 0};
            }
        }
        if constexpr (F8) {
            // read T: element c16 of the tile is dims 32 T + 2 c16 (low byte) and + 1 of four tokens
#pragma unroll
            for (int T = 0; T < NDT / 2; ++T) {
                const u32x2 w = tr_read(vs + vbase[T & 7] + 256 * (T >> 3));
                acc[2 * T] = mfma_k16(e4m3x4_to_bf16(__builtin_amdgcn_perm(w[1], w[0], 0x06040200u)), pb, acc[2 * T]);
                acc[2 * T + 1] =
                    mfma_k16(e4m3x4_to_bf16(__builtin_amdgcn_perm(w[1], w[0], 0x07050301u)), pb, acc[2 * T + 1]);
            }
        } else {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                acc[dt] = mfma_k16(tr_read(vs + vbase[dt & 7] + 256 * (dt >> 3)), pb, acc[dt]);
        }
        const float rs = ((bf16_lo(pb[0]) + bf16_hi(pb[0])) + bf16_lo(pb[1])) + bf16_hi(pb[1]);
        const float rx = ((ps[0] + ps[1]) + ps[2]) + ps[3];
        l_run = l_run * alpha + rows_sum4(rs);
        l_ex = l_ex * alpha + rows_sum4(rx);
        issue(uv + NU);
        u = uv + 1;
    }
    // No stream load (the zero-filling ones past the wave's pages included) may still be
    // writing LDS when the slices are reused below.
    wait_vmcnt<0>();

    // ---- merge the page streams' states (fixed order) and write this split's result. The DS
    // waves of a stream hold the same softmax state (the same arithmetic on the same scores)
    // and each contributes its head dims.
    const bool wave_bad = __builtin_amdgcn_ballot_w64(bad_page) != 0;
    if (lane == 0 && dq == 0)
        sm_bad[grp][pw] = wave_bad;
    if (r4 == 0 && dq == 0) {
        sm_m[grp][pw][c16] = m_run;
        sm_l[grp][pw][c16] = l_run;
        sm_lx[grp][pw][c16] = l_ex;
    }
    __syncthreads();  // every wave is done with its slice; the states are visible
    // [NS][W][g][HD] fp32, each stream's acc scaled to its slot's common max
    float *const mo = (float *)ring;
    {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w)
            M = fmaxf(M, sm_m[grp][w][c16]);
        const float cw = m_run == -INFINITY ? 0.f : fast_exp2(m_run - M);
        if (c16 < g) {
            if constexpr (F8) {
                // tiles 2T and 2T + 1 interleave: element i of each is dim 32 T + 8 r4 + 2 i (+ 1)
                float *dst = mo + (((size_t)grp * W + pw) * g + c16) * HD + SEG * dq + 8 * r4;
#pragma unroll
                for (int T = 0; T < NDT / 2; ++T) {
                    const f32x4 e = acc[2 * T] * cw, o = acc[2 * T + 1] * cw;
                    *(f32x4 *)(dst + 32 * T) = f32x4{e[0], o[0], e[1], o[1]};
                    *(f32x4 *)(dst + 32 * T + 4) = f32x4{e[2], o[2], e[3], o[3]};
                }
            } else {
                float *dst = mo + (((size_t)grp * W + pw) * g + c16) * HD + SEG * dq + 4 * r4;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
                    *(f32x4 *)(dst + 16 * dt) = acc[dt] * cw;
            }
        }
    }
    __syncthreads();
    // each slot's result: element e of slot sl by one thread
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) {
    bool bad = bad_len;
#pragma unroll
    for (int w = 0; w < W; ++w)
        bad = bad || sm_bad[sl][w];
    for (int e = threadIdx.x * 4; e < g * HD; e += kThreads * 4) {
        const int hn = e / HD, d = e % HD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w)
            M = fmaxf(M, sm_m[sl][w][hn]);
        float lsum = 0.f, lxsum = 0.f;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float mw = sm_m[sl][w][hn];
            const float cw = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
            lsum += cw * sm_l[sl][w][hn];
            lxsum += cw * sm_lx[sl][w][hn];
            o += *(const f32x4 *)(mo + (((size_t)sl * W + w) * g + hn) * HD + d);
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
            // kept for the merge (in the slot's first stream buffer: this thread read it last)
            *(f32x4 *)(mo + ((size_t)sl * W * g + hn) * HD + d) = o;
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
                    const f32x4 os = *(const f32x4 *)(mo + ((size_t)s2 * W * g + hn) * HD + d);
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

// Launch shape per head_dim: page streams per workgroup and LDS bytes per wave, measured on the
// decode workloads of both families. head_dim 512 (16 KB units): one wave with two units per
// workgroup, four workgroups per CU, so a batch's (row, KV head, split) items mostly start
// at once and no CU waits on a partly filled last round. head_dim 256 (8 KB units): two
// page streams of one wave with three units each, three workgroups per CU, which keeps the
// window-sized local items (at most 1024 keys) from running one page at a time on few waves.
// A head_dim 512 grid of at most one workgroup per CU (one long row, say) would leave each CU
// one wave working through its pages one at a time, so there four waves share every page,
// a quarter of the head dims each (with eight units of 4 KB in flight per wave); up to two
// workgroups per CU (a batch of a single-KV-head family, say) the same with four units per wave,
// so that two workgroups fit a CU's LDS. The score partials are added in the same tree in every
// shape, so all of them give the same bits.
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
                return hipLaunchKernel((const void *)decode_split_kernel<HD, SHARED, W, 1, SLICE, false, 2>, rows,
                                       dim3(2 * W * 64), args, 0, stream);
            return hipLaunchKernel((const void *)decode_split_kernel<HD, SHARED, W, 1, SLICE, false, 3>, rows,
                                   dim3(3 * W * 64), args, 0, stream);
        }
    }
    if constexpr (HD == 512) {
        const int64_t items = (int64_t)grid.x * grid.y * grid.z;
        if (items <= kNumCUs)
            return hipLaunchKernel((const void *)decode_split_kernel<HD, SHARED, 1, 4, 32 * 1024>, grid,
                                   dim3(4 * 64), args, 0, stream);
        if (items <= 2 * kNumCUs)
            return hipLaunchKernel((const void *)decode_split_kernel<HD, SHARED, 1, 4, 16 * 1024>, grid,
                                   dim3(4 * 64), args, 0, stream);
    }
    return hipLaunchKernel((const void *)decode_split_kernel<HD, SHARED, W, 1, SLICE>, grid, dim3(W * 64), args, 0,
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
                return hipLaunchKernel((const void *)decode_split_kernel<256, false, 2, 1, 16 * 1024, true, 2>, rows,
                                       dim3(2 * 2 * 64), args, 0, stream);
            return hipLaunchKernel((const void *)decode_split_kernel<256, false, 2, 1, 16 * 1024, true, 3>, rows,
                                   dim3(3 * 2 * 64), args, 0, stream);
        }
        k = (const void *)decode_split_kernel<256, false, 2, 1, 16 * 1024, true>;
        threads = 128;
    } else if (head_dim == 512) {
        k = kv_shared ? (const void *)decode_split_kernel<512, true, 1, 1, 32 * 1024, true>
                      : (const void *)decode_split_kernel<512, false, 1, 1, 32 * 1024, true>;
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
