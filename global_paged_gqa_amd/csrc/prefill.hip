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
// Four waves of 32 rows each (32x32x16 MFMA), the O accumulators in AGPRs: 256 of them at
// head_dim 512, 128 at head_dim 256; one wave per SIMD either way (rows per wave set the LDS
// traffic: every wave reads the whole K and V block, so fewer, fatter waves read less).
// K and V blocks stream through a 128 KB LDS ring filled by direct global->LDS buffer
// loads in the order of their first use. Iteration j computes the scores of block j+1 and
// then the PV product of block j with the softmax of block j+1 placed step by step between
// its MFMAs (VALU work beside the matrix core). With separate K and V pools it has two
// barriers: the one before the scores frees the slot of the V just used and the one before
// the PV product frees the slot of the K just used, so each K unit is requested two blocks
// ahead of its scores. The ring loads are spread between the MFMA groups of both products
// rather than issued in one burst, because a wave stalls on the issue of a global->LDS load
// while the load unit is busy. Each wave prepares the buffer resource of one page per unit.
//
// The online softmax rescales lazily: a row keeps its reference maximum until a new score
// exceeds it by more than 2^8, so P stays below 256 and the accumulators are rescaled only
// on those (rare) blocks. O is divided by the sum of the bf16-rounded weights the PV product
// uses and the LSE uses the sum of the fp32 weights, both against the same reference, so the
// result is the exact softmax up to rounding.
//
// The key range of a tile is pruned to [first visible key of its first query, its last
// query] (the sliding-window tile pruning of the vllm-gemma-4-31b skills page, "Three
// load-bearing facts", first item); pages in a
// block that lie outside it are never read (zero-size buffer resource: zeros, no traffic).
// Workgroups take the query tiles of each (row, KV head) heaviest first, dealt round-robin over
// the XCDs so that every XCD gets an equal share of every row.
#include "common.h"
#include "kernels.h"

namespace gattn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// MFMA rows per wave: two 32-row tiles at head_dim 256, one at 512 (the O accumulators fill
// the AGPRs either way); the workgroup's four waves hold kWaves * 32 * row_tiles rows.
constexpr int row_tiles(int hd) { return hd == 256 ? 2 : 1; }
constexpr int kTok = 32;            // keys per block (two pages)
constexpr int kRingBytes = 128 * 1024;
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)

typedef float f32x16 __attribute__((ext_vector_type(16)));

// c + lo(a) * lo(b) + hi(a) * hi(b) for packed bf16 pairs, in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

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

// Two K-steps of the score product (as qk4).
template <bool first>
__device__ __forceinline__ void qk2(f32x16 &st, u32x4 k0, u32x4 k1, u32x4 q0, u32x4 q1) {
    if (first)
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %3, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0"
            : "=&v"(st)
            : "v"(k0), "v"(k1), "v"(q0), "v"(q1));
    else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %3, %0\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0"
            : "+v"(st)
            : "v"(k0), "v"(k1), "v"(q0), "v"(q1));
}

// Two K-steps for two row tiles (A shared, B per tile), the tiles' MFMAs alternating so that
// no MFMA depends on the one issued just before it.
template <bool first>
__device__ __forceinline__ void qk2x2(f32x16 &s0, f32x16 &s1, u32x4 k0, u32x4 k1, u32x4 a0, u32x4 a1, u32x4 b0,
                                      u32x4 b1) {
    if (first)
        asm("v_mfma_f32_32x32x16_bf16 %0, %2, %4, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %1, %2, %6, 0\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %3, %5, %0\n\t"
            "v_mfma_f32_32x32x16_bf16 %1, %3, %7, %1"
            : "=&v"(s0), "=&v"(s1)
            : "v"(k0), "v"(k1), "v"(a0), "v"(a1), "v"(b0), "v"(b1));
    else
        asm("v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\t"
            "v_mfma_f32_32x32x16_bf16 %1, %2, %6, %1\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %3, %5, %0\n\t"
            "v_mfma_f32_32x32x16_bf16 %1, %3, %7, %1"
            : "+v"(s0), "+v"(s1)
            : "v"(k0), "v"(k1), "v"(a0), "v"(a1), "v"(b0), "v"(b1));
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

// Helpers for the rare paths of the block loop (window slides, edge blocks): the lane index
// recomputed and zeros made on the spot, so that the compiler keeps neither live across the
// loop (spilled, their reloads would wait on the ring's loads).
__device__ __forceinline__ int lane_id() {
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}
__device__ __forceinline__ u32x4 fresh_zeros() {
    uint32_t a, b, c, d;
    asm volatile("v_mov_b32 %0, 0\n\tv_mov_b32 %1, 0\n\tv_mov_b32 %2, 0\n\tv_mov_b32 %3, 0"
                 : "=v"(a), "=v"(b), "=v"(c), "=v"(d));
    return u32x4{a, b, c, d};
}

// Page resources of one tile's K/V stream. A ring unit is the K (or V) of one 32-token block,
// two pages; waves [0, W/2) load its first page and waves [W/2, W) its second, so each wave
// prepares one buffer resource per unit. The tile reads pages [pgA, pgA + npg); page rel
// (relative to pgA) is read only if it holds a token in [lo, p_last], i.e. rel in [0, npg)
// past the first r_lo pages, and its id is below num_pages. Any other page gets a zero-size
// resource (its loads return zeros with no memory traffic), and an id out of range inside the
// tile's range flags the tile. Page ids sit 64 per vector register (lane i: page base + i) and
// are read back with readlane; the window slides every 32 blocks.
template <int HD, int W>
struct TilePages {
    static constexpr int PAGE_BYTES = kPage * HD * 2;
    static constexpr int WPP = W / 2;  // waves per page
    const int32_t *pt;                 // the row's page table, from page pgA
    int npg, r_lo;
    uint32_t npages32;
    uint64_t kbase, vbase, page_stride;
    int ids, ids_next, ids_base;
    int bad;

    __device__ int load_ids(int first, int lane) const { return npg > 0 ? pt[min(first + lane, npg - 1)] : 0; }
    __device__ void init(const PrefillArgs &a, int b, int kvh, int pgA, int npg_, int r_lo_, int lane) {
        pt = a.page_table + (int64_t)b * a.pt_stride + pgA;
        npg = npg_;
        r_lo = r_lo_;
        npages32 = (uint32_t)min<int64_t>(a.num_pages, INT32_MAX);
        kbase = (uint64_t)(uintptr_t)(a.k_pool + (int64_t)kvh * kPage * HD);
        vbase = (uint64_t)(uintptr_t)(a.v_pool + (int64_t)kvh * kPage * HD);
        page_stride = (uint64_t)a.num_kv_heads * PAGE_BYTES;  // bytes between pages
        ids = load_ids(0, lane);
        ids_next = load_ids(64, lane);
        ids_base = 0;
        bad = 0;
    }
    // buffer resource of this wave's page of block blk in the K or V pool
    __device__ u32x4 rsrc(int blk, bool is_v, int wave) {
        const int rel = 2 * blk + wave / WPP;
        if (rel < npg && rel - ids_base >= 96) {
            ids = ids_next;
            ids_base += 64;
            ids_next = load_ids(ids_base + 64, lane_id());
            // Wait for the ids here, on this rare path. Left to the compiler, the wait lands
            // after the branch, on every call, and drains the ring loads in flight each time.
            __builtin_amdgcn_s_waitcnt(0);
        }
        const bool in_range = rel >= r_lo && rel < npg;
        const int r = (rel - ids_base) & 127;  // 0..127 for pages in range
        const int id_a = __builtin_amdgcn_readlane(ids, r & 63);
        const int id_b = __builtin_amdgcn_readlane(ids_next, r & 63);
        const uint32_t pid = (uint32_t)(r >= 64 ? id_b : id_a);
        const bool live = in_range && pid < npages32;
        bad |= (int)(in_range && pid >= npages32);
        const uint64_t addr = (is_v ? vbase : kbase) + (uint64_t)(live ? pid : 0u) * page_stride;
        return u32x4{(uint32_t)addr, (uint32_t)(addr >> 32) & 0xFFFFu, live ? (uint32_t)PAGE_BYTES : 0u,
                     0x00020000u};
    }
};

template <int HD, bool SHARED>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs a) {
    constexpr int NKS = HD / 16;                     // K-steps of the score product
    constexpr int NDT = HD / 32;                     // 32-dim output tiles (the whole head_dim)
    constexpr int UNIT = kTok * HD * 2;              // bytes of the K (or V) of one block
    constexpr int NU = kRingBytes / UNIT;            // ring depth in units
    constexpr int LPU = UNIT / 16 / kThreads;        // 16-byte loads per lane per unit
    constexpr int PAGE_BYTES = kPage * HD * 2;       // one (page, KV head) block
    constexpr int RT = row_tiles(HD);                // 32-row tiles per wave
    constexpr int kRows = kWaves * 32 * RT;          // MFMA rows per workgroup
    // K = V: units that may still be in flight when an iteration starts (the ones it reads have
    // landed). Separate pools keep four units in the ring (two read, two in flight).
    constexpr int AHEAD = NU - 3;
    static_assert(NU >= 4 && LPU % 2 == 0 && (NU - 1) * LPU + 1 <= 63, "ring shape");

    __shared__ __attribute__((aligned(1024))) uint8_t ring[kRingBytes];
    __shared__ int sm_bad;  // some wave met a page id out of range

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n32 = lane & 31, h = lane >> 5;
    const int g = a.group, Hq = a.num_q_heads;

    // ---- work order: (row, KV head) pairs in turn, each pair's query tiles from the last (most
    // keys) to the first. The dispatcher deals consecutive workgroups round-robin over the
    // XCDs, so every XCD gets every eighth tile of each pair: equal shares of long and short
    // rows, while an XCD's CUs still stream the K/V of the same one or two pairs through its L2.
    // (Giving each XCD a contiguous run of pairs instead left the XCDs holding the longest rows
    // working for a third longer than the rest.)
    const int wid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    int item = wid;
    // Local tiles all carry about the same work, and neighbouring tiles of a (row, KV head) read
    // nearly the same keys (their windows differ by one tile of queries), so there the tiles go
    // out in runs of four per XCD instead: workgroup wid runs on XCD wid % 8, and each group of
    // 32 consecutive workgroups hands XCD x its items 4x .. 4x+3 (measured: 1% faster).
    if (!a.is_global) {
        constexpr int kRun = 4;
        const int total = gridDim.x * gridDim.y * gridDim.z;
        const int g0 = wid / (8 * kRun) * (8 * kRun);
        if (g0 + 8 * kRun <= total)
            item = g0 + (wid % 8) * kRun + (wid - g0) / 8;
    }
    const int qt = gridDim.x - 1 - item % gridDim.x;
    const int kvh = (item / gridDim.x) % gridDim.y;
    const int b = item / (gridDim.x * gridDim.y);

    if (threadIdx.x == 0)
        sm_bad = 0;
    const int q0 = a.cu_q[b], q_len = a.cu_q[b + 1] - q0;
    const int L = a.ctx_lens[b];
    const int BQ = kRows / g;          // query positions per tile
    const int tile_q = qt * BQ;        // first query of the tile (within the row)
    if (q_len <= 0 || tile_q >= q_len)
        return;
    // A row with more queries than max_q (the bound the grid was sized by) would leave the
    // queries past the last tile unwritten: the row fails closed, each of its tiles writing NaN
    // over every gridDim.x-th block of BQ queries, so that all of them are covered.
    if (q_len > a.max_q) {
        const float qnan = __builtin_nanf("");
        const uint32_t nan2 = pack_bf16x2(qnan, qnan);
        for (int i0 = tile_q; i0 < q_len; i0 += gridDim.x * BQ)
            for (int e = threadIdx.x; e < min(BQ, q_len - i0) * g; e += kThreads) {
                const int64_t orow = (int64_t)(q0 + i0 + e / g) * Hq + kvh * g + e % g;
                a.lse[orow] = qnan;
                for (int d = 0; d < HD; d += 8)
                    *(u32x4 *)(a.out + orow * HD + d) = u32x4{nan2, nan2, nan2, nan2};
            }
        return;
    }
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

    // ---- this wave's rows: tile r holds rows m = 32 (RT wave + r) + n32, each (query position
    // m / g, head m % g)
    auto m_own = [&](int r) { return 32 * (RT * wave + r) + n32; };
    auto pos_own = [&](int r) { return m_own(r) / g; };
    auto ok_own = [&](int r) { return pos_own(r) < nq; };
    int p_own[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
        p_own[r] = p_first + pos_own(r);

    // ---- Q^T as the B operand: lane holds row n32, dims 16 s + 8 h .. +7 (zeros for padding rows).
    // The tile's Q rows are first copied into the ring (still unused) with whole 1 KB loads, row m
    // at m * HD * 2 bytes with its 16-byte chunk c at slot c ^ (m & 31) (a read of 32 rows at one
    // chunk then touches 32 slots), and read into registers after the copy has landed. Loading
    // them straight into registers gathered 32 bytes per row and instruction; every workgroup
    // starts with this load, so it runs while every CU is loading. Rows past the tile's queries
    // lie beyond the buffer range and load zeros.
    u32x4 qb[RT][NKS];
    {
        constexpr int CPRQ = HD / 8;                           // 16-byte chunks per Q row
        constexpr int QLPW = kRows * CPRQ / 64 / kWaves;       // 1 KB loads per wave
        const uint16_t *qbase = a.q + ((int64_t)(q0 + tile_q) * Hq + kvh * g) * HD;
        const uint32_t qbytes = (uint32_t)(((int64_t)(nq - 1) * Hq + g) * HD * 2);
        const u32x4 qrs = raw_rsrc(qbase, qbytes);
        const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
#pragma unroll
        for (int i = 0; i < QLPW; ++i) {
            const int I = i * kWaves + wave;  // instruction: chunk positions 64 I .. 64 I + 63
            const int P = 64 * I + lane;
            const int m = P / CPRQ, c = (P % CPRQ) ^ (m & 31);
            const int pos = m / g, hq = m - pos * g;
            ring_load16(qrs, ring_lds + 1024u * (uint32_t)I,
                        (uint32_t)((((int64_t)pos * Hq + hq) * HD + c * 8) * 2));
        }
    }
    auto q_from_lds = [&]() {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const int m = m_own(r);
#pragma unroll
            for (int s = 0; s < NKS; ++s)
                qb[r][s] = *(const u32x4 *)(ring + m * HD * 2 + (((2 * s + h) ^ (m & 31)) * 16));
        }
    };

    // O^T tiles of this wave's rows over the whole head dimension (AGPRs)
    f32x16 acc[RT][NDT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int d = 0; d < NDT; ++d)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[r][d][v] = 0.f;
    float m_run[RT], l_run[RT], l_ex[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        m_run[r] = -INFINITY;
        l_run[r] = 0.f;
        l_ex[r] = 0.f;
    }

    // ---- ring fill. Wave w loads page w / 2 of each unit: its load k writes the unit's LDS
    // chunk position P = 1024 (w / 2) + 128 k + 64 (w % 2) + lane, i.e. token row P / (HD/8) of
    // the block, slot P % (HD/8), and fetches the chunk the swizzle puts there.
    using Pages = TilePages<HD, kWaves>;
    static_assert(Pages::PAGE_BYTES / 16 == Pages::WPP * 64 * LPU, "one page per wave group");
    Pages pages;
    pages.init(a, b, kvh, pgA, npg, lo / kPage - pgA, lane);
    auto chunk0 = [&](int k) { return (wave / Pages::WPP) * (Pages::PAGE_BYTES / 16) + k * Pages::WPP * 64 +
                                      (wave % Pages::WPP) * 64; };
    auto src_off = [&](int k) {
        const int P = chunk0(k) + lane;
        const int t = P / (HD / 8);
        const int c = (P % (HD / 8)) ^ swz(t & 15);
        return (uint32_t)((t & 15) * HD + c * 8) * 2u;
    };
    // The ring streams units in the order of their first use. Separate pools: unit 0 is the K
    // of block 0, unit 2j+1 the K of block j+1, unit 2j+2 the V of block j (iteration j reads
    // both). K = V: unit j is block j. Units past the last block, and pages of a block outside
    // [lo, p_last], load zeros with no memory traffic, so that every wave always has exactly
    // LPU loads per unit in flight and the ring waits stay exact.
    struct UnitLoad {
        u32x4 rs;      // buffer resource of this wave's page (zero size: not read)
        uint32_t dst;  // LDS address of the unit
    };
    auto prep = [&](int u) {
        const int blk = SHARED ? u : (u == 0 ? 0 : ((u & 1) ? (u + 1) >> 1 : (u >> 1) - 1));
        const bool is_v = !SHARED && u > 0 && (u & 1) == 0;
        return UnitLoad{pages.rsrc(blk, is_v, wave), (uint32_t)(uintptr_t)(ring + (u % NU) * UNIT)};
    };
    auto emit = [&](const UnitLoad &ul, int k) { ring_load16(ul.rs, ul.dst + chunk0(k) * 16, src_off(k)); };
    auto issue = [&](int u) {
        const UnitLoad ul = prep(u);
#pragma unroll
        for (int k = 0; k < LPU; ++k)
            emit(ul, k);
    };
    auto unit_k = [&](int j) { return SHARED ? j : (j == 0 ? 0 : 2 * j - 1); };  // unit of block j's K
    auto unit_v = [&](int j) { return SHARED ? j : 2 * j + 2; };                // unit of block j's V

    // ---- per-lane LDS offsets of the operand reads
    // K operand (step s): token n32, chunk 2s + h -> n32*HD*2 + 16*((2s + h) ^ swz); with
    // v = s & 7 that is krow + ((32 v) ^ kx) + 256 (s >> 3), kx = 16 (h ^ swz) (the swizzle
    // touches only the low 8 address bits), one XOR per read instead of eight offsets held.
    const uint32_t krow = (uint32_t)(n32 * HD * 2);
    const uint32_t kx = (uint32_t)(16 * (h ^ swz(n32 & 15)));
    // One row tile leaves registers for the eight offsets themselves (no VALU work per read);
    // two row tiles need those registers and compute the XOR per read.
    uint32_t ktab[RT == 1 ? 8 : 1];
    if constexpr (RT == 1) {
#pragma unroll
        for (int v = 0; v < 8; ++v)
            ktab[v] = krow + ((32u * v) ^ kx);
    }
    auto koff = [&](int s) -> uint32_t {
        if constexpr (RT == 1)
            return ktab[s & 7] + 256 * (s >> 3);
        else
            return krow + ((32u * (s & 7)) ^ kx) + 256 * (s >> 3);
    };
    // V^T operand (transpose read i of dim tile dt, page p): in 16-lane group G (G&1: dims
    // 16..31 of the tile, G>>1 = h), lane 4r + q supplies token 16p + 8i + 4h + r, dims 4q .. 4q+3
    // of its 16; the lane receives its dim for those four tokens. Its chunk 4 (dt & 3) + k,
    // k = 2 (G&1) + q/2, lands at slot (4 (dt & 3)) ^ (k ^ swz(token)), so the offset is
    // vrow[i] + ((64 (dt & 3)) ^ vx[i]) + 256 (dt >> 2).
    uint32_t vrow[2], vx[2];
    {
        const int G = lane >> 4, gh = G & 1, r = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tok = 8 * i + 4 * h + r;
            vrow[i] = (uint32_t)(tok * HD * 2 + 8 * (q & 1));
            vx[i] = (uint32_t)(16 * ((2 * gh + (q >> 1)) ^ swz(tok)));
        }
    }
    uint32_t vtab[2][RT == 1 ? 4 : 1];
    if constexpr (RT == 1) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int d = 0; d < 4; ++d)
                vtab[i][d] = vrow[i] + ((64u * d) ^ vx[i]);
    }
    // offset of transpose read i of tile dt within its 256-byte group of four tiles
    auto voff = [&](int i, int dt) -> uint32_t {
        if constexpr (RT == 1)
            return vtab[i][dt & 3];
        else
            return vrow[i] + ((64u * (dt & 3)) ^ vx[i]);
    };

    const float scale = a.scale_log2;
    // the bf16 pair (1, 1) in a register: the weight sums take one dot product per pair of weights
    // (an inline constant operand would not be read as a pair of bf16 values)
    const uint32_t ones_bf16x2 = __builtin_amdgcn_readfirstlane(0x3F803F80u);
    // S^T[32 tok][32 rows] of block j for this wave's rows. Operand reads run one group of four
    // K-steps ahead of the MFMAs; the scheduling fences keep the compiler from hoisting every
    // read of the block (which would not fit beside Q in registers). hook(t) runs after group t
    // (ring loads issued between the MFMA groups).
    // With two row tiles each K fragment feeds two MFMAs, so groups are two K-steps (the same
    // MFMA time per group, half the fragment registers).
    auto qk = [&](int j, f32x16 (&st)[RT], auto hook) {
        constexpr int G = 4 / RT;  // K-steps per group
        const uint8_t *kst = ring + (unit_k(j) % NU) * UNIT;
        auto kread = [&](int s) {
            return *(const u32x4 *)(kst + koff(s));
        };
        // KB fragment buffers: reads run KB - 1 groups ahead of their MFMAs
        constexpr int KB = 2;
        u32x4 kf[KB][G];
#pragma unroll
        for (int d = 0; d < KB - 1; ++d)
#pragma unroll
            for (int i = 0; i < G; ++i)
                kf[d][i] = kread(G * d + i);
#pragma unroll
        for (int t = 0; t < NKS / G; ++t) {
            if (t + KB - 1 < NKS / G) {
#pragma unroll
                for (int i = 0; i < G; ++i)
                    kf[(t + KB - 1) % KB][i] = kread(G * (t + KB - 1) + i);
            }
            const u32x4 *kk = kf[t % KB];
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const u32x4 *qq = qb[r] + G * t;
                if constexpr (G == 4) {
                    if (t == 0)
                        qk4<true>(st[r], kk[0], kk[1], kk[2], kk[3], qq[0], qq[1], qq[2], qq[3]);
                    else
                        qk4<false>(st[r], kk[0], kk[1], kk[2], kk[3], qq[0], qq[1], qq[2], qq[3]);
                } else if (r == 0) {
                    // both tiles at once, their MFMAs alternating
                    const u32x4 *qr = qb[1] + G * t;
                    if (t == 0)
                        qk2x2<true>(st[0], st[1], kk[0], kk[1], qq[0], qq[1], qr[0], qr[1]);
                    else
                        qk2x2<false>(st[0], st[1], kk[0], kk[1], qq[0], qq[1], qr[0], qr[1]);
                }
            }
            if ((t + 1) % RT == 0)
                hook(t / RT);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < RT; ++r)
            qk_settle(st[r]);
    };
    // Masked online softmax of block j's scores for this wave's rows (lane holds tokens
    // 8(v/4) + 4h + v%4 of row n32; the other half of the row's 32 tokens is in lane n32 + 32).
    // Lazy rescale: a row keeps its reference maximum until a score exceeds it by more than
    // 2^8, so P stays below 256 and the accumulators are rescaled only on those (rare) blocks.
    // O is normalised by the sum of the bf16-rounded weights the PV product uses (a weight's
    // rounding scales numerator and denominator alike), the LSE by the sum of the fp32 weights.
    // Returns the P^T fragments of the two 16-token K-steps; alpha is the rows' rescale factor.
    // The softmax runs in twelve steps so that the PV loop can place them between its MFMAs
    // (VALU work beside the matrix core): 0-3 the row maximum (four scores each; edge blocks are
    // masked before the steps), 4 the new reference maximum, 5-8 the exponentials, 9-10 the bf16
    // packing and the sums, 11 the row sums' update.
    struct SmState {
        uint32_t vis0, span;  // key offset o(v) is visible iff (uint)(vis0 + o(v) - 4h) <= span
        bool interior;        // every row of the tile sees all 32 keys of the block: no mask
        float mx, mb, rs, rx;
    };
    auto sm_init = [&](int j, SmState &z, int r) {
        // visible iff T <= p_own (causal) and p_own - T < window (local): with the lane's token
        // offsets o(v) = 8(v/4) + 4h + v%4 from T0, that is lim_lo <= o(v) <= lim_hi, which is
        // one unsigned compare, (uint)(o - lim_lo) <= (uint)(lim_hi - lim_lo) (a negative
        // difference wraps above the span; for global rows lim_lo = INT_MIN and the wrap-around
        // arithmetic leaves exactly o <= lim_hi).
        const int T0 = kb0 + j * kTok;
        const int lim_hi = p_own[r] - T0;
        const int lim_lo = a.is_global ? INT32_MIN : p_own[r] - a.window + 1 - T0;
        z.vis0 = (uint32_t)(4 * h) - (uint32_t)lim_lo;
        z.span = (uint32_t)lim_hi - (uint32_t)lim_lo;
        z.interior = T0 + kTok - 1 <= p_first && (a.is_global || T0 >= p_last - a.window + 1);
        z.mx = -INFINITY;
        z.rs = 0.f;
        z.rx = 0.f;
    };
    // Edge blocks: the invisible keys become -inf, all of a row tile's scores at once, behind one
    // uniform branch ahead of the softmax steps. The steps then hold no branch, so the PV product
    // stays one run of MFMAs the scheduler can spread them over (a branch per step cut it into
    // short runs: 2% slower local, 0.7% global, same bits).
    auto sm_mask = [&](const SmState &z, f32x16 &st) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
            st[v] = z.vis0 + (uint32_t)(8 * (v >> 2) + (v & 3)) <= z.span ? st[v] : -INFINITY;
    };
    auto sm_step = [&](int step, SmState &z, f32x16 &st, u32x4 (&pf)[2], float &alpha, int r) {
        if (step < 4) {
            // raw scores (masked beforehand on edge blocks): the scale enters the exponent (step
            // 5-8) and the row maximum (step 4)
#pragma unroll
            for (int v = 4 * step; v < 4 * step + 4; ++v)
                z.mx = fmaxf(z.mx, st[v]);
        } else if (step == 4) {
            // the scale is positive and rounding is monotonic: scale * max(raw) is the maximum of the
            // rounded scaled scores, exactly
            const float m_new = fmaxf(m_run[r], halves_max(z.mx) * scale);
            const bool resc = m_new > m_run[r] + kRescaleLog2;
            // While the reference is still -inf every weight so far was exactly 0, so the
            // accumulators and sums are zero: they need no rescale (alpha 1 leaves the same bits
            // as alpha 0 and keeps the block from the 4 * NDT AGPR round trips of a rescale).
            alpha = resc && m_run[r] != -INFINITY ? fast_exp2(m_run[r] - m_new) : 1.0f;
            if (resc)
                m_run[r] = m_new;
            z.mb = m_run[r] == -INFINITY ? 0.f : m_run[r];
        } else if (step < 9) {
#pragma unroll
            for (int v = 4 * (step - 5); v < 4 * (step - 5) + 4; ++v)
                st[v] = fast_exp2(__builtin_fmaf(st[v], scale, -z.mb));  // the weights replace the scores
        } else if (step < 11) {
            const int q = step - 9;
            pf[q] = u32x4{pack_bf16x2(st[8 * q + 0], st[8 * q + 1]), pack_bf16x2(st[8 * q + 2], st[8 * q + 3]),
                          pack_bf16x2(st[8 * q + 4], st[8 * q + 5]), pack_bf16x2(st[8 * q + 6], st[8 * q + 7])};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                z.rs = dot2_bf16(pf[q][i], ones_bf16x2, z.rs);
                z.rx += st[8 * q + 2 * i] + st[8 * q + 2 * i + 1];
            }
        } else if (step == 11) {
            l_run[r] = l_run[r] * alpha + halves_sum(z.rs);
            l_ex[r] = l_ex[r] * alpha + halves_sum(z.rx);
        }
    };
    // step s of the RT row tiles' softmax: step s / RT of tile s % RT (the tiles' independent
    // chains interleave)
    constexpr int SM_STEPS = 12 * RT;
    auto sm_any = [&](int s, SmState (&z)[RT], f32x16 (&st)[RT], u32x4 (&pf)[RT][2], float (&alpha)[RT]) {
        const int r = s % RT;
        sm_step(s / RT, z[r], st[r], pf[r], alpha[r], r);
    };
    auto softmax = [&](int j, f32x16 (&st)[RT], u32x4 (&pf)[RT][2], float (&alpha)[RT]) {
        SmState z[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r)
            sm_init(j, z[r], r);
        if (!z[0].interior) {
#pragma unroll
            for (int r = 0; r < RT; ++r)
                sm_mask(z[r], st[r]);
        }
#pragma unroll
        for (int s = 0; s < SM_STEPS; ++s)
            sm_any(s, z, st, pf, alpha);
    };
    // O^T += V^T P^T for block j over the whole head dimension, V^T fragments read one tile
    // ahead of the MFMAs. Tokens no row of the tile can see carry P = 0, and their V rows are
    // zeroed in LDS beforehand (clear_edge), so a never-written slot cannot turn 0 * V into a
    // NaN. hook(dt) runs after tile dt.
    auto pv = [&](int j, const u32x4 (&pf)[RT][2], auto hook) {
        const uint8_t *vst = ring + (unit_v(j) % NU) * UNIT;
        auto vread = [&](int dt, int p) {
            const uint32_t o = 256 * (dt >> 2) + p * PAGE_BYTES;
            const u32x2 v0 = tr_read(vst + voff(0, dt) + o);
            const u32x2 v1 = tr_read(vst + voff(1, dt) + o);
            return u32x4{v0[0], v0[1], v1[0], v1[1]};
        };
        // fragments of tile dt in slot dt % PVA, read PVA - 1 tiles ahead of their MFMAs (the K
        // fragments of the score product are dead here, so the registers are free)
        constexpr int PVA = RT == 1 ? 3 : 2;
        u32x4 vf[PVA][2];
#pragma unroll
        for (int d = 0; d < PVA - 1; ++d) {
            vf[d][0] = vread(d, 0);
            vf[d][1] = vread(d, 1);
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            if (dt + PVA - 1 < NDT) {
                vf[(dt + PVA - 1) % PVA][0] = vread(dt + PVA - 1, 0);
                vf[(dt + PVA - 1) % PVA][1] = vread(dt + PVA - 1, 1);
            }
            // the two halves of the 32 tokens accumulate into the same tile: with two row tiles
            // the four MFMAs alternate tiles, so no MFMA waits on the one just before it
#pragma unroll
            for (int r = 0; r < RT; ++r)
                acc[r][dt] = mfma32(vf[dt % PVA][0], pf[r][0], acc[r][dt]);
#pragma unroll
            for (int r = 0; r < RT; ++r)
                acc[r][dt] = mfma32(vf[dt % PVA][1], pf[r][1], acc[r][dt]);
            hook(dt);
            __builtin_amdgcn_sched_barrier(0);
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
        const u32x4 zero = fresh_zeros();
        const int ln = lane_id();
        for (int t = wave; t < kTok; t += kWaves) {
            const int T = T0 + t;
            if (T < lo || T > p_last)
                for (int c = ln; c < HD / 8; c += 64)
                    *(u32x4 *)(vst + t * HD * 2 + c * 16) = zero;
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
    // block loop the only vector-memory operations in flight are the ring's own loads: Q's copy
    // lands in the ring for every wave, each wave reads its rows, and the ring is free again.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    q_from_lds();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
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
    f32x16 st[RT];
    u32x4 pf[RT][2];
    float alpha[RT];
    qk(0, st, no_hook);
    softmax(0, st, pf, alpha);

    // Iteration j: the scores of block j+1 (QK), then the PV product of block j interleaved by
    // the scheduler with the softmax of block j+1 (independent MFMA and VALU work).
    for (int j = 0; j < nblk; ++j) {
        f32x16 st1[RT];
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
#pragma unroll
        for (int r = 0; r < RT; ++r)
            if (__builtin_amdgcn_ballot_w64(alpha[r] != 1.0f)) {
#pragma unroll
                for (int d = 0; d < NDT; ++d)
                    scale_acc(acc[r][d], alpha[r]);
            }
        u32x4 pf1[RT][2];
        float alpha1[RT];
        SmState z[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r)
            sm_init(j + 1, z[r], r);
        if (!z[0].interior) {
#pragma unroll
            for (int r = 0; r < RT; ++r)
                sm_mask(z[r], st1[r]);
        }
        // Softmax of the next block beside the PV tiles: the masking, maxima and exponentials
        // (steps 0-8 of each row tile) spread over tiles 0 .. NDT-2, the packing into pf1 and
        // the sums after the last tile, when pf is no longer read (pf1 can take its registers).
        auto sm_hook = [&](int dt) {
            constexpr int E = 9 * RT;
            if (dt < NDT - 1) {
#pragma unroll
                for (int s = dt * E / (NDT - 1); s < (dt + 1) * E / (NDT - 1); ++s)
                    sm_any(s, z, st1, pf1, alpha1);
            } else {
#pragma unroll
                for (int s = E; s < SM_STEPS; ++s)
                    sm_any(s, z, st1, pf1, alpha1);
            }
        };
        if (SHARED) {
            pv(j, pf, sm_hook);
        } else {
            // the V of block j landed (units 2j+3 and 2j+4 may be in flight); after the barrier
            // for all waves, and the slot of block j+1's K (read by the QK above) is free
            wait_vmcnt<2 * LPU>();
            __syncthreads();
            if (clear_edge(j))
                __syncthreads();
            const UnitLoad ul = prep(2 * j + 5);
            auto loads = spread(ul, std::integral_constant<int, NDT>{});
            pv(j, pf, [&](int dt) {
                loads(dt);
                sm_hook(dt);
            });
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            pf[r][0] = pf1[r][0];
            pf[r][1] = pf1[r][1];
            alpha[r] = alpha1[r];
        }
    }

    // No ring load (the zero-filling ones past the last block included) may still be writing
    // this workgroup's LDS when it ends.
    wait_vmcnt<0>();
    // whether any wave of the tile met a bad page id
    auto bad_tile = [&](int mine) {
        if (mine)
            sm_bad = 1;
        __syncthreads();
        return sm_bad != 0;
    };

    // ---- this wave's rows: normalise O into the ring (no wave reads it any more: bad_tile's
    // barrier follows every wave's last ring read, and wait_vmcnt<0> its last ring load), then
    // write the tile's rows out as whole 16-byte chunks. A lane holds 8-byte pieces of 32
    // different rows, so storing straight from the accumulators would scatter every store over 64
    // cache lines; through LDS, consecutive lanes write consecutive chunks of a row, and the g
    // rows of one query position are contiguous in `out`. Row m of the tile sits at m * HD * 2
    // bytes of the ring with its 16-byte chunk c at slot c ^ (m & 31), so the 32 rows a staging
    // store touches land in 32 different bank groups.
    const bool bad = bad_row || bad_tile(pages.bad);
    uint8_t *const ost = ring;
    static_assert(kRows * HD * 2 <= kRingBytes, "O staging fits the ring");
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int m = m_own(r);
        if (ok_own(r) && h == 0) {
            const int64_t orow = (int64_t)(q0 + tile_q + pos_own(r)) * Hq + kvh * g + m % g;
            a.lse[orow] = bad ? __builtin_nanf("") : (m_run[r] + fast_log2(l_ex[r])) * kLn2;
        }
        const float inv = 1.0f / l_run[r];
        uint8_t *const orow_lds = ost + m * HD * 2 + 8 * h;
#pragma unroll
        for (int d = 0; d < NDT; ++d)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = bad ? __builtin_nanf("") : acc[r][d][4 * jj + e] * inv;
                *(u32x2 *)(orow_lds + ((4 * d + jj) ^ (m & 31)) * 16) =
                    u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            }
    }
    __syncthreads();
    constexpr int CPR = HD / 8;            // 16-byte chunks per row
    constexpr int RPS = kThreads / CPR;    // rows per pass of the workgroup
    const int n_rows = nq * g;             // rows m < nq * g hold real (query, head) pairs
    const int c = threadIdx.x % CPR;
    // m / g by a float reciprocal: m < 256 and g <= 16, so (m + 0.5) / g is at least 1/32 away from
    // an integer and the rounding of 1/g (2^-24 relative) cannot move it across one
    const float inv_g = 1.0f / (float)g;
    for (int m = threadIdx.x / CPR; m < n_rows; m += RPS) {
        const int pos = (int)(((float)m + 0.5f) * inv_g);
        const int64_t orow = (int64_t)(q0 + tile_q + pos) * Hq + kvh * g + (m - pos * g);
        *(u32x4 *)(a.out + orow * HD + c * 8) = *(const u32x4 *)(ost + m * HD * 2 + (c ^ (m & 31)) * 16);
    }
}

template <int HD, bool SHARED>
hipError_t launch(const PrefillArgs &a, dim3 grid, hipStream_t stream) {
    void *args[] = {(void *)&a};
    return hipLaunchKernel((const void *)prefill_kernel<HD, SHARED>, grid, dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, int head_dim, bool kv_shared, int batch, hipStream_t stream) {
    const int bq = kWaves * 32 * row_tiles(head_dim) / a.group;  // query positions per tile
    const dim3 grid((a.max_q + bq - 1) / bq, a.num_kv_heads, batch);
    if (head_dim == 256)
        return kv_shared ? launch<256, true>(a, grid, stream) : launch<256, false>(a, grid, stream);
    if (head_dim == 512)
        return kv_shared ? launch<512, true>(a, grid, stream) : launch<512, false>(a, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace gattn
