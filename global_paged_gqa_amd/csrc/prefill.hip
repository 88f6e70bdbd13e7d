// Chunked causal prefill over the paged KV cache on gfx950 (bf16 MFMA, fp32 softmax).
//
// A chunk's queries attend the cache with the causal mask inside the chunk and the
// sliding window for the local family (Core AI card, "Contents": a flash-prefill
// with a query axis and an intra-chunk causal mask). One workgroup = one (row, KV
// head, query tile) of 128 MFMA rows; the g query heads that share the KV head are
// packed into the rows (row m = query position m / g, head m % g), so every K/V byte
// staged in LDS serves all g heads.
//
// Keys are processed in blocks of 32 tokens (two pages). Each wave owns a set of rows for
// both products, so the softmax weights never leave its registers:
//   QK: S^T[32 tok][rows] = K . Q^T over the whole head_dim (A = K rows read from LDS,
//       B = Q^T kept in registers), then the masked online softmax of those rows;
//   PV: O^T[dims][rows] += V^T . P^T over the whole head_dim, with V^T read from the
//       row-major page by the gfx950 transpose read (ds_read_b64_tr_b16) and P^T taken
//       straight from the score tile's accumulator layout.
// head_dim 512: four waves of 32 rows (32x32x16 MFMA, accumulators in AGPRs; one wave per
// SIMD). head_dim 256: eight waves of 16 rows (16x16x32 MFMA; two waves per SIMD, so the
// hardware overlaps one wave's softmax and waits with the other's matrix work).
// K and V blocks stream through a 128 KB LDS ring filled by direct global->LDS buffer
// loads in the order of their first use. Iteration j computes the scores of block j+1 and
// then the PV product of block j beside the softmax of block j+1. With separate K and V pools
// (head_dim 512) it has two barriers: the one before the scores frees the slot of the V just
// used and the one before the PV product frees the slot of the K just used, so each K unit is
// requested two blocks ahead of its scores. The ring loads are spread between the MFMA groups
// of both products rather than issued in one burst, because a wave stalls on the issue of a
// global->LDS load while the load unit is busy.
//
// The online softmax rescales lazily: a row keeps its reference maximum until a new score
// exceeds it by more than 2^8, so P stays below 256 and the accumulators are rescaled only
// on those (rare) blocks. O is divided by the sum of the bf16-rounded weights the PV product
// uses and the LSE uses the sum of the fp32 weights, both against the same reference, so the
// result is the exact softmax up to rounding.
//
// The key range of a tile is pruned to [first visible key of its first query, its last
// query] (page 5's "Three load-bearing facts" #1: sliding-window tile pruning); pages in a
// block that lie outside it are never read (zero-size buffer resource: zeros, no traffic).
// Workgroups are mapped so that each XCD works through the query tiles of the same (row,
// KV head), heaviest first, sharing that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace gattn {

namespace {

constexpr int kXcds = 8;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRows = 128;          // MFMA rows per workgroup (4 tiles of 32)
constexpr int kTok = 32;            // keys per block (two pages)
constexpr int kRingBytes = 128 * 1024;
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// LDS layout of one unit (the K or the V of one 32-token block): token row t at t * HD * 2
// bytes, its 16-byte chunk c at slot c ^ swz(t & 15). swz is a bit permutation of the low
// four token bits chosen so that (i) the 16 tokens read at one chunk by a K operand load
// hit 16 different 16-byte bank groups and (ii) the four tokens x two chunks of one
// transpose-read lane group hit 8 different ones.
__device__ __forceinline__ int swz(int x) { return ((x & 3) << 1) | ((x >> 2) & 1) | (x & 8); }

// Four K-steps of the score product S^T += K . Q^T in VGPRs. The PV accumulators fill the
// AGPR file, so the score tile must live in VGPRs; the compiler would place any MFMA result
// in AGPRs here, hence assembly. Back-to-back MFMAs accumulating into exactly the same
// registers need no wait states; `first` starts from zero instead of reading S^T.
template <bool first>
__device__ __forceinline__ void qk4(f32x16 &st, u32x4 k0, u32x4 k1, u32x4 k2, u32x4 k3, u32x4 q0, u32x4 q1,
                                    u32x4 q2, u32x4 q3) {
    if (first)
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %5, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %2, %6, %0\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %3, %7, %0\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %4, %8, %0"
            : "=&v"(st)
            : "v"(k0), "v"(k1), "v"(k2), "v"(k3), "v"(q0), "v"(q1), "v"(q2), "v"(q3));
    else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %5, %0\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %2, %6, %0\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %3, %7, %0\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %4, %8, %0"
            : "+v"(st)
            : "v"(k0), "v"(k1), "v"(k2), "v"(k3), "v"(q0), "v"(q1), "v"(q2), "v"(q3));
}

// The wait states an MFMA result needs before a vector instruction may read it (the
// compiler cannot see that qk4 is an MFMA), with margin.
__device__ __forceinline__ void qk_settle(f32x16 &st) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(st));
}

// acc *= al for an accumulator tile held in AGPRs, one register at a time through a single
// VGPR (written in C++ the multiply makes the compiler stage whole tiles in VGPRs). The
// trailing wait states separate the AGPR writes from the next MFMA reading them.
__device__ __forceinline__ void scale_acc(f32x16 &c, float al) {
#pragma unroll
    for (int v = 0; v < 16; v += 4) {
        float x0 = c[v], x1 = c[v + 1], x2 = c[v + 2], x3 = c[v + 3], t;
        asm volatile(
            "v_accvgpr_read_b32 %4, %0\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %0, %4\n\t"
            "v_accvgpr_read_b32 %4, %1\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %1, %4\n\t"
            "v_accvgpr_read_b32 %4, %2\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %2, %4\n\t"
            "v_accvgpr_read_b32 %4, %3\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %3, %4\n\t"
            "s_nop 4"
            : "+a"(x0), "+a"(x1), "+a"(x2), "+a"(x3), "=&v"(t)
            : "v"(al));
        c[v] = x0;
        c[v + 1] = x1;
        c[v + 2] = x2;
        c[v + 3] = x3;
    }
}

template <int HD, bool SHARED>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs a) {
    constexpr int NKS = HD / 16;                     // K-steps of the score product
    constexpr int NDT = HD / 32;                     // 32-dim output tiles (the whole head_dim)
    constexpr int UNIT = kTok * HD * 2;              // bytes of the K (or V) of one block
    constexpr int NU = kRingBytes / UNIT;            // ring depth in units
    constexpr int LPU = UNIT / 16 / kThreads;        // 16-byte loads per lane per unit
    constexpr int PAGE_BYTES = kPage * HD * 2;       // one (page, KV head) block
    // K = V: units that may still be in flight when an iteration starts (the ones it reads have
    // landed). Separate pools keep four units in the ring (two read, two in flight).
    constexpr int AHEAD = NU - 3;
    static_assert(NU >= 4 && LPU % 2 == 0 && (NU - 1) * LPU + 1 <= 63, "ring shape");

    __shared__ __attribute__((aligned(1024))) uint8_t ring[kRingBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n32 = lane & 31, h = lane >> 5;
    const int g = a.group, Hq = a.num_q_heads;

    // ---- XCD-aware work mapping: the dispatcher deals workgroups round-robin over the
    // XCDs, so give XCD x a contiguous run of work items; within a (row, KV head) the query
    // tiles run from the last (most keys) to the first.
    const int nwg = gridDim.x * gridDim.y * gridDim.z;
    const int wid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int xcd = wid % kXcds, per = nwg / kXcds, extra = nwg % kXcds;
    const int item = xcd * per + min(xcd, extra) + wid / kXcds;
    const int qt = gridDim.x - 1 - item % gridDim.x;
    const int kvh = (item / gridDim.x) % gridDim.y;
    const int b = item / (gridDim.x * gridDim.y);

    const int q0 = a.cu_q[b], q_len = a.cu_q[b + 1] - q0;
    const int L = a.ctx_lens[b];
    const int BQ = kRows / g;          // query positions per tile
    const int tile_q = qt * BQ;        // first query of the tile (within the row)
    if (q_len <= 0 || tile_q >= q_len)
        return;
    const int nq = min(BQ, q_len - tile_q);
    const int p_first = L - q_len + tile_q;  // absolute position of the tile's first query
    const int p_last = p_first + nq - 1;
    // Malformed rows (more queries than cached tokens, or a cache beyond the table)
    // produce NaN outputs instead of reading outside the table.
    const bool bad_row = q_len > L || (L - 1) / kPage >= a.pt_stride;
    const int lo = a.is_global ? 0 : max(0, p_first - a.window + 1);  // first key any row sees
    const int kb0 = lo & ~(kTok - 1);                                    // first block's first key
    const int nblk = bad_row ? 0 : (p_last - kb0) / kTok + 1;
    const int pgA = kb0 / kPage;                                         // first page of block 0
    const int npg = bad_row ? 0 : p_last / kPage - pgA + 1;
    const int32_t *pt = a.page_table + (int64_t)b * a.pt_stride;

    // ---- this wave's rows: row m = 32 * wave + n32 is (query position m / g, head m % g)
    const int m_own = 32 * wave + n32;
    const int pos_own = m_own / g;
    const bool ok_own = pos_own < nq;
    const int p_own = p_first + pos_own;

    // ---- Q^T as the B operand: lane holds row n32, dims 16 s + 8 h .. +7 (zeros for padding rows)
    u32x4 qb[NKS];
    {
        const uint16_t *qp =
            a.q + ((int64_t)(q0 + tile_q + (ok_own ? pos_own : 0)) * Hq + kvh * g + m_own % g) * HD + 8 * h;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const u32x4 v = *(const u32x4 *)(qp + 16 * s);
            qb[s] = ok_own ? v : u32x4{0, 0, 0, 0};
        }
    }

    // O^T tiles of this wave's 32 rows over the whole head dimension (AGPRs)
    f32x16 acc[NDT];
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            acc[d][v] = 0.f;
    float m_run = -INFINITY, l_run = 0.f, l_ex = 0.f;
    int bad_page = 0;

    // ---- ring fill: load k of a unit writes LDS chunk position P = k*256 + wave*64 + lane,
    // i.e. token row P / (HD/8), slot P % (HD/8); it fetches the chunk the swizzle puts there.
    // Loads 0 .. LPU/2-1 cover the block's first page, the rest its second.
    auto src_off = [&](int k) {
        const int P = k * kThreads + wave * 64 + lane;
        const int t = P / (HD / 8);
        const int c = (P % (HD / 8)) ^ swz(t & 15);
        return (uint32_t)((t & 15) * HD + c * 8) * 2u;
    };
    // Page ids of the tile's range, 64 per vector register (lane j: page 64*k + j), read back
    // with readlane so that the block loop never waits on a memory load for an id.
    auto load_ids = [&](int first) {
        return bad_row ? 0 : pt[pgA + min(first + lane, max(npg - 1, 0))];
    };
    int ids = load_ids(0), ids_next = load_ids(64);
    int ids_base = 0;  // page index (relative to pgA) of ids' lane 0
    // The ring streams units in the order of their first use. Separate pools: unit 0 is the K
    // of block 0, unit 2j+1 the K of block j+1, unit 2j+2 the V of block j (iteration j reads
    // both). K = V: unit j is block j. Units past the last block, and pages of a block outside
    // [lo, p_last], load zeros with no memory traffic, so that every wave always has exactly
    // LPU loads per unit in flight and the ring waits stay exact.
    struct UnitLoad {
        u32x4 rs[2];   // buffer resources of the block's two pages (zero size: not read)
        uint32_t dst;  // this wave's LDS base for the unit
    };
    // Per page: the page id (two readlanes, no vector select), an unsigned range check, and the
    // page's byte address, all in scalar registers without branches.
    const uint32_t npages32 = (uint32_t)min<int64_t>(a.num_pages, INT32_MAX);
    const uint64_t kbase = (uint64_t)(uintptr_t)(a.k_pool + (int64_t)kvh * kPage * HD);
    const uint64_t vbase = (uint64_t)(uintptr_t)(a.v_pool + (int64_t)kvh * kPage * HD);
    const uint64_t page_stride = (uint64_t)a.num_kv_heads * PAGE_BYTES;  // bytes between pages
    auto prep = [&](int u) {
        const int blk = SHARED ? u : (u == 0 ? 0 : ((u & 1) ? (u + 1) >> 1 : (u >> 1) - 1));
        const bool is_v = !SHARED && u > 0 && (u & 1) == 0;
        if (blk < nblk && 2 * blk + 1 - ids_base >= 96) {  // slide the id window (every 32 blocks)
            ids = ids_next;
            ids_base += 64;
            ids_next = load_ids(ids_base + 64);
        }
        const uint64_t base = is_v ? vbase : kbase;
        UnitLoad ul;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            const int rel = 2 * blk + pp;
            const int pg = pgA + rel;
            const bool in_range = blk < nblk && pg * kPage <= p_last && pg * kPage + kPage - 1 >= lo;
            const int r = (rel - ids_base) & 127;  // 0..127 for pages in range
            const int id_a = __builtin_amdgcn_readlane(ids, r & 63);
            const int id_b = __builtin_amdgcn_readlane(ids_next, r & 63);
            const uint32_t pid = (uint32_t)(r >= 64 ? id_b : id_a);
            const bool valid = pid < npages32;
            const bool live = in_range && valid;
            bad_page |= (int)(in_range && !valid);
            const uint64_t addr = base + (uint64_t)(live ? pid : 0u) * page_stride;
            ul.rs[pp] = u32x4{(uint32_t)addr, (uint32_t)(addr >> 32) & 0xFFFFu, live ? (uint32_t)PAGE_BYTES : 0u,
                              0x00020000u};
        }
        ul.dst = (uint32_t)(uintptr_t)(ring + (u % NU) * UNIT) + (uint32_t)(wave * 64 * 16);
        return ul;
    };
    auto emit = [&](const UnitLoad &ul, int k) {
        ring_load16(ul.rs[k < LPU / 2 ? 0 : 1], ul.dst + k * kThreads * 16, src_off(k));
    };
    auto issue = [&](int u) {
        const UnitLoad ul = prep(u);
#pragma unroll
        for (int k = 0; k < LPU; ++k)
            emit(ul, k);
    };
    auto unit_k = [&](int j) { return SHARED ? j : (j == 0 ? 0 : 2 * j - 1); };  // unit of block j's K
    auto unit_v = [&](int j) { return SHARED ? j : 2 * j + 2; };                // unit of block j's V

    // ---- per-lane LDS offsets of the operand reads
    // K operand (step s): token n32, chunk 2s + h -> n32*HD*2 + 16*((2s + h) ^ swz) =
    // kb[s & 7] + 256 * (s >> 3), the swizzle touching only the low 8 address bits.
    uint32_t kb[8];
    {
        const int sw = swz(n32 & 15);
#pragma unroll
        for (int v = 0; v < 8; ++v)
            kb[v] = (uint32_t)(n32 * HD * 2 + 16 * ((2 * v + h) ^ sw));
    }
    // V^T operand (transpose read i of dim tile dt, page p): in 16-lane group G (G&1: dims
    // 16..31 of the tile, G>>1 = h), lane 4r + q supplies token 16p + 8i + 4h + r, dims 4q .. 4q+3
    // of its 16; the lane receives its dim for those four tokens. The offset repeats every four
    // tiles (256 bytes): vb[i][dt & 3] + 256 * (dt >> 2).
    uint32_t vb[2][4];
    {
        const int G = lane >> 4, gh = G & 1, r = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int tok = 8 * i + 4 * h + r;
                const int c = 4 * d + 2 * gh + (q >> 1);
                vb[i][d] = (uint32_t)(tok * HD * 2 + 16 * (c ^ swz(tok)) + 8 * (q & 1));
            }
    }

    const float scale = a.scale_log2;
    // S^T[32 tok][32 rows] of block j for this wave's rows. Operand reads run one group of four
    // K-steps ahead of the MFMAs; the scheduling fences keep the compiler from hoisting every
    // read of the block (which would not fit beside Q in registers). hook(t) runs after group t
    // (ring loads issued between the MFMA groups).
    auto qk = [&](int j, f32x16 &st, auto hook) {
        const uint8_t *kst = ring + (unit_k(j) % NU) * UNIT;
        auto kread = [&](int s) { return *(const u32x4 *)(kst + kb[s & 7] + 256 * (s >> 3)); };
        u32x4 kf[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            kf[0][i] = kread(i);
#pragma unroll
        for (int t = 0; t < NKS / 4; ++t) {
            if (t + 1 < NKS / 4) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    kf[(t + 1) & 1][i] = kread(4 * (t + 1) + i);
            }
            const u32x4 *kk = kf[t & 1];
            if (t == 0)
                qk4<true>(st, kk[0], kk[1], kk[2], kk[3], qb[0], qb[1], qb[2], qb[3]);
            else
                qk4<false>(st, kk[0], kk[1], kk[2], kk[3], qb[4 * t], qb[4 * t + 1], qb[4 * t + 2], qb[4 * t + 3]);
            hook(t);
            __builtin_amdgcn_sched_barrier(0);
        }
        qk_settle(st);
    };
    // Masked online softmax of block j's scores for this wave's rows (lane holds tokens
    // 8(v/4) + 4h + v%4 of row n32; the other half of the row's 32 tokens is in lane n32 + 32).
    // Lazy rescale: a row keeps its reference maximum until a score exceeds it by more than
    // 2^8, so P stays below 256 and the accumulators are rescaled only on those (rare) blocks.
    // O is normalised by the sum of the bf16-rounded weights the PV product uses (a weight's
    // rounding scales numerator and denominator alike), the LSE by the sum of the fp32 weights.
    // Returns the P^T fragments of the two 16-token K-steps; alpha is the rows' rescale factor.
    auto softmax = [&](int j, f32x16 &st, u32x4 (&pf)[2], float &alpha) {
        // visible iff T <= p_own (causal) and p_own - T < window (local): with the lane's token
        // offsets o(v) = 8(v/4) + 4h + v%4 from T0, that is lim_lo <= o(v) <= lim_hi
        const int T0 = kb0 + j * kTok;
        const int lim_hi = p_own - T0;
        const int lim_lo = a.is_global ? INT32_MIN : p_own - a.window + 1 - T0;
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int o = 8 * (v >> 2) + 4 * h + (v & 3);
            st[v] = (o <= lim_hi && o >= lim_lo) ? st[v] * scale : -INFINITY;
            mx = fmaxf(mx, st[v]);
        }
        const float m_new = fmaxf(m_run, halves_max(mx));
        const bool resc = m_new > m_run + kRescaleLog2;
        alpha = resc ? fast_exp2(m_run - m_new) : 1.0f;
        if (resc)
            m_run = m_new;
        const float mb = m_run == -INFINITY ? 0.f : m_run;
        float ps[16];
#pragma unroll
        for (int v = 0; v < 16; ++v)
            ps[v] = fast_exp2(st[v] - mb);
        float rs = 0.f, rx = 0.f;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            pf[p] = u32x4{pack_bf16x2(ps[8 * p + 0], ps[8 * p + 1]), pack_bf16x2(ps[8 * p + 2], ps[8 * p + 3]),
                          pack_bf16x2(ps[8 * p + 4], ps[8 * p + 5]), pack_bf16x2(ps[8 * p + 6], ps[8 * p + 7])};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                rs += bf16_lo(pf[p][i]) + bf16_hi(pf[p][i]);
                rx += ps[8 * p + 2 * i] + ps[8 * p + 2 * i + 1];
            }
        }
        l_run = l_run * alpha + halves_sum(rs);
        l_ex = l_ex * alpha + halves_sum(rx);
    };
    // O^T += V^T P^T for block j over the whole head dimension, V^T fragments read one tile
    // ahead of the MFMAs. Tokens no row of the tile can see carry P = 0, and their V rows are
    // zeroed in LDS beforehand (clear_edge), so a never-written slot cannot turn 0 * V into a
    // NaN. hook(dt) runs after tile dt.
    auto pv = [&](int j, const u32x4 pf0, const u32x4 pf1, auto hook) {
        const uint8_t *vst = ring + (unit_v(j) % NU) * UNIT;
        auto vread = [&](int dt, int p) {
            const uint32_t o = 256 * (dt >> 2) + p * PAGE_BYTES;
            const u32x2 v0 = tr_read(vst + vb[0][dt & 3] + o);
            const u32x2 v1 = tr_read(vst + vb[1][dt & 3] + o);
            return u32x4{v0[0], v0[1], v1[0], v1[1]};
        };
        u32x4 va0 = vread(0, 0), va1 = vread(0, 1);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            u32x4 na0, na1;
            if (dt + 1 < NDT) {
                na0 = vread(dt + 1, 0);
                na1 = vread(dt + 1, 1);
            }
            acc[dt] = mfma32(va0, pf0, acc[dt]);
            acc[dt] = mfma32(va1, pf1, acc[dt]);
            hook(dt);
            if (dt + 1 < NDT) {
                va0 = na0;
                va1 = na1;
            }
        }
    };
    // Zero the V rows of block j that no row of the tile can see (tokens before lo or past
    // p_last: only the first and last blocks have them). Called with block j's V landed for
    // every wave; returns whether it wrote, in which case the caller synchronises again.
    auto clear_edge = [&](int j) {
        const int T0 = kb0 + j * kTok;
        if (T0 >= lo && T0 + kTok - 1 <= p_last)
            return false;
        uint8_t *vst = ring + (unit_v(j) % NU) * UNIT;
        for (int t = wave; t < kTok; t += kWaves) {
            const int T = T0 + t;
            if (T < lo || T > p_last)
                for (int c = lane; c < HD / 8; c += 64)
                    *(u32x4 *)(vst + t * HD * 2 + c * 16) = u32x4{0, 0, 0, 0};
        }
        return true;
    };
    // Ring loads of one unit spread over the N MFMA groups of a product: group i issues loads
    // [i*LPU/N, (i+1)*LPU/N) of the unit.
    auto spread = [&](const UnitLoad &ul, auto n_groups) {
        constexpr int N = decltype(n_groups)::value;
        return [&ul, &emit](int i) {
#pragma unroll
            for (int k = i * LPU / N; k < (i + 1) * LPU / N; ++k)
                emit(ul, k);
        };
    };
    auto no_hook = [](int) {};

    // Q and the first page ids are in registers before the ring starts, so that inside the
    // block loop the only vector-memory operations in flight are the ring's own loads.
    __builtin_amdgcn_s_waitcnt(0);
    // Separate pools: units 0..3 (K0, K1, V0, K2) before the loop; iteration j then issues the V
    // of block j+1 (unit 2j+4) after its first barrier and the K of block j+3 (unit 2j+5) after
    // the second, so a K unit is loaded two blocks ahead of its scores and a V unit one block
    // and a half ahead of its product. K = V: units 0 .. NU-2, then unit j+NU-1 per iteration.
    constexpr int PRO = SHARED ? NU - 1 : 4;
#pragma unroll
    for (int u = 0; u < PRO; ++u)
        issue(u);
    wait_vmcnt<(PRO - 1) * LPU>();  // unit 0 (the K of block 0) landed for this wave
    __syncthreads();
    f32x16 st;
    u32x4 pf[2];
    float alpha;
    qk(0, st, no_hook);
    softmax(0, st, pf, alpha);

    // Iteration j: the scores of block j+1 (QK), then the PV product of block j interleaved by
    // the scheduler with the softmax of block j+1 (independent MFMA and VALU work).
    for (int j = 0; j < nblk; ++j) {
        f32x16 st1;
        if (SHARED) {
            // unit j+1 landed for this wave; after the barrier for all waves, and unit j-1's slot
            // (read by the previous PV) is free
            wait_vmcnt<AHEAD * LPU>();
            __syncthreads();
            if (clear_edge(j))
                __syncthreads();
            const UnitLoad ul = prep(j + NU - 1);
            qk(j + 1, st1, spread(ul, std::integral_constant<int, NKS / 4>{}));
        } else {
            // the K of block j+1 landed (units 2j+2 and 2j+3 may be in flight); after the barrier
            // for all waves, and the slot of block j-1's V is free
            wait_vmcnt<2 * LPU>();
            __syncthreads();
            const UnitLoad ul = prep(2 * j + 4);
            // The next block's scores are computed even in the last iteration: block nblk lies
            // past every query (fully masked, its units zero-filled), so it changes no state.
            qk(j + 1, st1, spread(ul, std::integral_constant<int, NKS / 4>{}));
        }
        // rescale this wave's rows for block j (factors from its softmax)
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int d = 0; d < NDT; ++d)
                scale_acc(acc[d], alpha);
        }
        u32x4 pf1[2];
        float alpha1;
        if (SHARED) {
            pv(j, pf[0], pf[1], no_hook);
        } else {
            // the V of block j landed (units 2j+3 and 2j+4 may be in flight); after the barrier
            // for all waves, and the slot of block j+1's K (read by the QK above) is free
            wait_vmcnt<2 * LPU>();
            __syncthreads();
            if (clear_edge(j))
                __syncthreads();
            const UnitLoad ul = prep(2 * j + 5);
            pv(j, pf[0], pf[1], spread(ul, std::integral_constant<int, NDT>{}));
        }
        softmax(j + 1, st1, pf1, alpha1);
        pf[0] = pf1[0];
        pf[1] = pf1[1];
        alpha = alpha1;
    }

    // No ring load (the zero-filling ones past the last block included) may still be writing
    // this workgroup's LDS when it ends.
    wait_vmcnt<0>();

    // ---- this wave's rows: normalise and write O, LSE
    const bool bad = bad_row || __builtin_amdgcn_ballot_w64(bad_page) != 0;
    if (!ok_own)
        return;
    const int64_t orow = (int64_t)(q0 + tile_q + pos_own) * Hq + kvh * g + m_own % g;
    if (h == 0)
        a.lse[orow] = bad ? __builtin_nanf("") : (m_run + fast_log2(l_ex)) * kLn2;
    const float inv = 1.0f / l_run;
    uint16_t *op = a.out + orow * HD + 4 * h;
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = bad ? __builtin_nanf("") : acc[d][4 * jj + e] * inv;
            *(u32x2 *)(op + 32 * d + 8 * jj) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        }
}

// Eight-wave variant: the same 128 MFMA rows per workgroup, 16 rows per wave, with the
// 16x16x32 MFMA for both products, so that two waves share each SIMD and the hardware overlaps
// one wave's softmax, loads and waits with the other's matrix work. Per wave and 32-key block:
//   QK: S^T[32 tok][16 rows] as two 16-key tiles (A = K rows from LDS, B = Q^T in registers);
//   softmax of the rows (the row's 32 scores sit in four 16-lane groups: lane swaps);
//   PV: O^T[16 dims][16 rows] += V^T[16 dims][32 tok] . P^T[32 tok][16 rows] per 16-dim tile,
//       V^T from two transpose reads (tokens 4g.. and 16+4g.. of lane group g), P^T straight
//       from the two score tiles.
// K/V stream through the same 128 KB LDS ring (one barrier per block), laid out with dswz.
template <int HD, bool SHARED>
__global__ __launch_bounds__(512, 1) void prefill16_kernel(PrefillArgs a) {
    constexpr int kW = 8;                            // waves
    constexpr int kT = kW * 64;                      // threads
    constexpr int NKS = HD / 32;                     // K-steps of the score product (16x16x32)
    constexpr int NDT = HD / 16;                     // 16-dim output tiles
    constexpr int UNIT = kTok * HD * 2;              // bytes of the K (or V) of one block
    constexpr int NU = kRingBytes / UNIT;            // ring depth in units
    constexpr int LPU = UNIT / 16 / kT;              // 16-byte loads per lane per unit
    constexpr int PAGE_BYTES = kPage * HD * 2;
    constexpr int AHEAD = SHARED ? NU - 3 : NU - 4;
    static_assert(AHEAD >= 0 && LPU % 2 == 0 && (NU - 1) * LPU + 1 <= 63, "ring shape");

    __shared__ __attribute__((aligned(1024))) uint8_t ring[kRingBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c16 = lane & 15, g4 = lane >> 4;
    const int g = a.group, Hq = a.num_q_heads;

    // ---- XCD-aware work mapping (as in the four-wave kernel)
    const int nwg = gridDim.x * gridDim.y * gridDim.z;
    const int wid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int xcd = wid % kXcds, per = nwg / kXcds, extra = nwg % kXcds;
    const int item = xcd * per + min(xcd, extra) + wid / kXcds;
    const int qt = gridDim.x - 1 - item % gridDim.x;
    const int kvh = (item / gridDim.x) % gridDim.y;
    const int b = item / (gridDim.x * gridDim.y);

    const int q0 = a.cu_q[b], q_len = a.cu_q[b + 1] - q0;
    const int L = a.ctx_lens[b];
    const int BQ = kRows / g;
    const int tile_q = qt * BQ;
    if (q_len <= 0 || tile_q >= q_len)
        return;
    const int nq = min(BQ, q_len - tile_q);
    const int p_first = L - q_len + tile_q;
    const int p_last = p_first + nq - 1;
    const bool bad_row = q_len > L || (L - 1) / kPage >= a.pt_stride;
    const int lo = a.is_global ? 0 : max(0, p_first - a.window + 1);
    const int kb0 = lo & ~(kTok - 1);
    const int nblk = bad_row ? 0 : (p_last - kb0) / kTok + 1;
    const int pgA = kb0 / kPage;
    const int npg = bad_row ? 0 : p_last / kPage - pgA + 1;
    const int32_t *pt = a.page_table + (int64_t)b * a.pt_stride;

    // ---- this wave's rows: row m = 16 * wave + c16 is (query position m / g, head m % g)
    const int m_own = 16 * wave + c16;
    const int pos_own = m_own / g;
    const bool ok_own = pos_own < nq;
    const int p_own = p_first + pos_own;

    // ---- Q^T as the B operand: lane holds row c16, dims 32 s + 8 g4 .. +7
    u32x4 qb[NKS];
    {
        const uint16_t *qp =
            a.q + ((int64_t)(q0 + tile_q + (ok_own ? pos_own : 0)) * Hq + kvh * g + m_own % g) * HD + 8 * g4;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const u32x4 v = *(const u32x4 *)(qp + 32 * s);
            qb[s] = ok_own ? v : u32x4{0, 0, 0, 0};
        }
    }

    f32x4 acc[NDT];
#pragma unroll
    for (int d = 0; d < NDT; ++d)
        acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f, l_ex = 0.f;
    int bad_page = 0;

    // ---- ring fill: load k of a unit writes LDS chunk position P = k*512 + wave*64 + lane,
    // i.e. token row P / (HD/8) of the block, slot P % (HD/8); it fetches the chunk dswz puts
    // there. Loads 0 .. LPU/2-1 cover the block's first page, the rest its second.
    auto src_off = [&](int k) {
        const int P = k * kT + wave * 64 + lane;
        const int t = P / (HD / 8);
        const int c = (P % (HD / 8)) ^ dswz(t & 15);
        return (uint32_t)((t & 15) * HD + c * 8) * 2u;
    };
    auto load_ids = [&](int first) {
        return bad_row ? 0 : pt[pgA + min(first + lane, max(npg - 1, 0))];
    };
    int ids = load_ids(0), ids_next = load_ids(64);
    int ids_base = 0;
    const uint32_t npages32 = (uint32_t)min<int64_t>(a.num_pages, INT32_MAX);
    const uint64_t kbase = (uint64_t)(uintptr_t)(a.k_pool + (int64_t)kvh * kPage * HD);
    const uint64_t vbase = (uint64_t)(uintptr_t)(a.v_pool + (int64_t)kvh * kPage * HD);
    const uint64_t page_stride = (uint64_t)a.num_kv_heads * PAGE_BYTES;
    // Units in the order of first use (see the four-wave kernel).
    auto issue = [&](int u) {
        const int blk = SHARED ? u : (u == 0 ? 0 : ((u & 1) ? (u + 1) >> 1 : (u >> 1) - 1));
        const bool is_v = !SHARED && u > 0 && (u & 1) == 0;
        if (blk < nblk && 2 * blk + 1 - ids_base >= 96) {
            ids = ids_next;
            ids_base += 64;
            ids_next = load_ids(ids_base + 64);
        }
        const uint64_t base = is_v ? vbase : kbase;
        u32x4 rs[2];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            const int rel = 2 * blk + pp;
            const int pg = pgA + rel;
            const bool in_range = blk < nblk && pg * kPage <= p_last && pg * kPage + kPage - 1 >= lo;
            const int r = (rel - ids_base) & 127;
            const int id_a = __builtin_amdgcn_readlane(ids, r & 63);
            const int id_b = __builtin_amdgcn_readlane(ids_next, r & 63);
            const uint32_t pid = (uint32_t)(r >= 64 ? id_b : id_a);
            const bool valid = pid < npages32;
            const bool live = in_range && valid;
            bad_page |= (int)(in_range && !valid);
            const uint64_t addr = base + (uint64_t)(live ? pid : 0u) * page_stride;
            rs[pp] = u32x4{(uint32_t)addr, (uint32_t)(addr >> 32) & 0xFFFFu, live ? (uint32_t)PAGE_BYTES : 0u,
                           0x00020000u};
        }
        const uint32_t dst = (uint32_t)(uintptr_t)(ring + (u % NU) * UNIT) + (uint32_t)(wave * 64 * 16);
#pragma unroll
        for (int k = 0; k < LPU; ++k)
            ring_load16(rs[k < LPU / 2 ? 0 : 1], dst + k * kT * 16, src_off(k));
    };
    auto unit_k = [&](int j) { return SHARED ? j : (j == 0 ? 0 : 2 * j - 1); };
    auto unit_v = [&](int j) { return SHARED ? j : 2 * j + 2; };

    // ---- per-lane LDS offsets
    // K operand (key tile kt, step s): key 16 kt + c16, logical chunk 4 s + g4 ->
    // kb[s % 4] + 256 (s / 4) + 16 kt * HD * 2 (the swizzle touches the low four chunk bits)
    uint32_t kb[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        kb[v] = (uint32_t)(c16 * HD * 2 + 16 * ((4 * v + g4) ^ dswz(c16)));
    // V^T operand (dim tile dt, token half th): in 16-lane group g4, lane 4r + q supplies token
    // 16 th + 4 g4 + r, dims 16 dt + 4q .. +3; the lane receives dim 16 dt + c16 of those four
    // tokens -> vb[th][dt % 8] + 256 (dt / 8)
    uint32_t vb[2][8];
    {
        const int r = c16 >> 2, q = c16 & 3;
#pragma unroll
        for (int th = 0; th < 2; ++th)
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const int tok = 16 * th + 4 * g4 + r;
                vb[th][d] = (uint32_t)(tok * HD * 2 + 16 * ((2 * d + (q >> 1)) ^ dswz(tok & 15)) + 8 * (q & 1));
            }
    }

    const float scale = a.scale_log2;
    // scores of block j: tile kt holds keys 16 kt + 4 g4 + i (i = 0..3) of row c16
    auto qk = [&](int j, f32x4 (&st)[2]) {
        const uint8_t *kst = ring + (unit_k(j) % NU) * UNIT;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; s += 2) {
                x = mfma_k32(*(const u32x4 *)(kst + kb[s & 3] + 256 * (s >> 2) + kt * 16 * HD * 2), qb[s], x);
                y = mfma_k32(*(const u32x4 *)(kst + kb[(s + 1) & 3] + 256 * ((s + 1) >> 2) + kt * 16 * HD * 2),
                             qb[s + 1], y);
            }
            st[kt] = x + y;
        }
    };
    auto softmax = [&](int j, f32x4 (&st)[2], u32x4 &pf, float &alpha) {
        const int T0 = kb0 + j * kTok;
        const int lim_hi = p_own - T0;
        const int lim_lo = a.is_global ? INT32_MIN : p_own - a.window + 1 - T0;
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = 16 * kt + 4 * g4 + i;
                st[kt][i] = (o <= lim_hi && o >= lim_lo) ? st[kt][i] * scale : -INFINITY;
                mx = fmaxf(mx, st[kt][i]);
            }
        const float m_new = fmaxf(m_run, rows_max4(mx));
        const bool resc = m_new > m_run + kRescaleLog2;
        alpha = resc ? fast_exp2(m_run - m_new) : 1.0f;
        if (resc)
            m_run = m_new;
        const float mb = m_run == -INFINITY ? 0.f : m_run;
        float ps[8];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ps[4 * kt + i] = fast_exp2(st[kt][i] - mb);
        pf = u32x4{pack_bf16x2(ps[0], ps[1]), pack_bf16x2(ps[2], ps[3]), pack_bf16x2(ps[4], ps[5]),
                   pack_bf16x2(ps[6], ps[7])};
        float rs = 0.f, rx = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rs += bf16_lo(pf[i]) + bf16_hi(pf[i]);
            rx += ps[2 * i] + ps[2 * i + 1];
        }
        l_run = l_run * alpha + rows_sum4(rs);
        l_ex = l_ex * alpha + rows_sum4(rx);
    };
    auto pv = [&](int j, const u32x4 pf) {
        const uint8_t *vst = ring + (unit_v(j) % NU) * UNIT;
        const int T0 = kb0 + j * kTok;
        // keep mask of the lane's eight tokens (all ones inside [lo, p_last])
        u32x4 keep;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            uint32_t k = 0;
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const int e = 2 * w2 + r2;  // element: token 16 (e / 4) + 4 g4 + e % 4
                const int T = T0 + 16 * (e >> 2) + 4 * g4 + (e & 3);
                k |= (T >= lo && T <= p_last) ? (r2 ? 0xFFFF0000u : 0x0000FFFFu) : 0u;
            }
            keep[w2] = k;
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const uint32_t o = 256 * (dt >> 3);
            const u32x2 v0 = tr_read(vst + vb[0][dt & 7] + o);
            const u32x2 v1 = tr_read(vst + vb[1][dt & 7] + o);
            const u32x4 va = u32x4{v0[0], v0[1], v1[0], v1[1]} & keep;
            acc[dt] = mfma_k32(va, pf, acc[dt]);
        }
    };

    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int u = 0; u < NU - 1; ++u)
        issue(u);
    wait_vmcnt<(NU - 2) * LPU>();
    __syncthreads();
    f32x4 st[2];
    u32x4 pf;
    float alpha;
    qk(0, st);
    softmax(0, st, pf, alpha);

    for (int j = 0; j < nblk; ++j) {
        wait_vmcnt<AHEAD * LPU>();
        __syncthreads();
        if (SHARED) {
            issue(j + NU - 1);
        } else {
            issue(2 * j + NU - 1);
            issue(2 * j + NU);
        }
        // block nblk (computed in the last iteration) lies past every query: fully masked
        f32x4 st1[2];
        qk(j + 1, st1);
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int d = 0; d < NDT; ++d)
                acc[d] *= alpha;
        }
        u32x4 pf1;
        float alpha1;
        pv(j, pf);
        softmax(j + 1, st1, pf1, alpha1);
        pf = pf1;
        alpha = alpha1;
    }
    wait_vmcnt<0>();

    const bool bad = bad_row || __builtin_amdgcn_ballot_w64(bad_page) != 0;
    if (!ok_own)
        return;
    const int64_t orow = (int64_t)(q0 + tile_q + pos_own) * Hq + kvh * g + m_own % g;
    if (g4 == 0)
        a.lse[orow] = bad ? __builtin_nanf("") : (m_run + fast_log2(l_ex)) * kLn2;
    const float inv = 1.0f / l_run;
    uint16_t *op = a.out + orow * HD + 4 * g4;
#pragma unroll
    for (int d = 0; d < NDT; ++d) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = bad ? __builtin_nanf("") : acc[d][e] * inv;
        *(u32x2 *)(op + 16 * d) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
}

// head_dim 256 runs the eight-wave kernel (its registers allow two waves per SIMD); head_dim
// 512 needs the whole register file of a SIMD for one wave's 32 rows and runs the four-wave
// kernel. Both were measured on the mixed-step prefill rows of their family.
template <int HD, bool SHARED>
hipError_t launch(const PrefillArgs &a, dim3 grid, hipStream_t stream) {
    void *args[] = {(void *)&a};
    if constexpr (HD == 256)
        return hipLaunchKernel((const void *)prefill16_kernel<HD, SHARED>, grid, dim3(512), args, 0, stream);
    else
        return hipLaunchKernel((const void *)prefill_kernel<HD, SHARED>, grid, dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, int head_dim, bool kv_shared, int batch, hipStream_t stream) {
    const int bq = kRows / a.group;
    const dim3 grid((a.max_q + bq - 1) / bq, a.num_kv_heads, batch);
    if (head_dim == 256)
        return kv_shared ? launch<256, true>(a, grid, stream) : launch<256, false>(a, grid, stream);
    if (head_dim == 512)
        return kv_shared ? launch<512, true>(a, grid, stream) : launch<512, false>(a, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace gattn
