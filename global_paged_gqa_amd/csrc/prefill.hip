// Chunked causal prefill over the paged KV cache on gfx950 (bf16 MFMA, fp32 softmax).
//
// A chunk's queries attend the cache with the causal mask inside the chunk and the
// sliding window for the local family (Core AI card, "Contents": a flash-prefill
// with a query axis and an intra-chunk causal mask). One workgroup = one (row,
// KV head, query tile) of 64 or 128 MFMA rows; the g query heads that share the KV head
// are packed into the rows (row m = position m / g, head m % g), so every K/V byte
// staged in LDS serves all g heads.
//
// Each wave owns 16 or 32 rows (one or two 16-row MFMA tiles) and the full head_dim;
// with two tiles every K/V operand read from LDS feeds two MFMAs. K/V pages stream
// through a ring of LDS stages filled by direct global->LDS buffer loads (no
// registers in flight), several pages ahead of the math; one barrier per page.
// The key range of a tile is pruned to [first visible key of its first query, its
// last query]: pages outside the window are never read (page 5's "Three
// load-bearing facts" #1: sliding-window tile pruning).
//
// Per KV page (16 tokens), per wave and 16-row tile:
//   S^T[16 tok][16 rows] = K . Q^T     MFMA 16x16x32; K from LDS (XOR-swizzled rows),
//                                      Q^T in registers
//   causal / window mask, online softmax per row (columns of S^T)
//   O^T[hd][16 rows] += V^T . P^T      MFMA 16x16x16; V^T read from the row-major LDS
//                                      page with the gfx950 transpose read
//                                      (ds_read_b64_tr_b16), P^T straight from S^T's
//                                      accumulator layout
// Workgroups are mapped so that each XCD works through contiguous query tiles of
// the same (row, KV head), which then share that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace gattn {

namespace {

constexpr int kXcds = 8;

// Work split per head dim. head_dim 256: four waves of two 16-row tiles (every K/V operand
// read from LDS feeds two MFMAs), 128 rows per workgroup. head_dim 512: four waves of one
// tile, 64 rows per workgroup, which keeps the 512-dim accumulator and Q^T of a wave in its
// registers with no spill. One wave per SIMD in both.
template <int HD>
struct Shape {
    static constexpr int RT = HD == 256 ? 2 : 1;  // 16-row MFMA tiles per wave
    static constexpr int WAVES = 4;
    static constexpr int THREADS = WAVES * 64;
    static constexpr int ROWS = WAVES * RT * 16;   // MFMA rows per workgroup
};

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

// Byte offset of 16-byte chunk `c` of token row `t` inside one staged (page, KV head)
// block: rows of HD*2 bytes, chunks XOR-swizzled by the token so 16 rows read at the
// same logical chunk land in 16 different bank groups.
template <int HD>
__device__ __forceinline__ uint32_t chunk_off(int t, int c) {
    return (uint32_t)(t * HD * 2 + ((c ^ (t & 15)) << 4));
}

// The ring's direct buffer->LDS loads and the waits on them are written as inline assembly,
// so that the compiler neither orders its own LDS reads behind every in-flight ring load nor
// merges the ring's wait with its own counters: the ring is synchronised by exactly one
// "at most N loads outstanding" wait plus a barrier per page.
//
// 16 bytes per lane from the buffer `rsrc` at byte offset voffset into LDS at lds + 16 * lane
// (M0 holds the LDS base; it is saved and restored around the load).
__device__ __forceinline__ void ring_load16(u32x4 rsrc, uint32_t lds, uint32_t voffset) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voffset), "s"(rsrc), "s"(lds)
        : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Raw buffer resource: base address, no stride, `bytes` in range (0: every load returns
// zeros and touches no memory).
__device__ __forceinline__ u32x4 raw_rsrc(const void *base, uint32_t bytes) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    return u32x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// ds_read_b64_tr_b16 of four V^T tiles, then one wait for all of them. The ring's LDS reads
// are inline assembly as well (their ordering after the page they read is the ring wait plus
// barrier); the "+v" operands of the wait keep every use of a result after it.
__device__ __forceinline__ void tr_read4(u32x2 (&v)[4], const uint8_t *base, uint32_t off0, uint32_t step) {
    const uint32_t a0 = (uint32_t)(uintptr_t)base;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v[k]) : "v"(a0 + (off0 ^ (step * k))));
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}

// Two ds_read_b128 (K operands, `step` apart under the XOR swizzle), then one wait.
__device__ __forceinline__ void k_read2(u32x4 (&v)[2], const uint8_t *base, uint32_t off0, uint32_t step) {
    const uint32_t a0 = (uint32_t)(uintptr_t)base;
#pragma unroll
    for (int k = 0; k < 2; ++k)
        asm volatile("ds_read_b128 %0, %1" : "=v"(v[k]) : "v"(a0 + (off0 ^ (step * k))));
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]));
}

template <int HD, bool SHARED>
__global__ __launch_bounds__(Shape<HD>::THREADS, 1) void prefill_kernel(PrefillArgs a) {
    constexpr int kRT = Shape<HD>::RT;
    constexpr int kThreads = Shape<HD>::THREADS;
    constexpr int kRows = Shape<HD>::ROWS;
    constexpr int NS = HD / 32;                       // K-steps of the score product
    constexpr int NT = HD / 16;                       // 16-dim output tiles
    constexpr int BLOCK = kPage * HD * 2;             // bytes of one (page, KV head) block
    constexpr int STAGE = SHARED ? BLOCK : 2 * BLOCK; // K (and V) of one page
    constexpr int NSTAGE = 128 * 1024 / STAGE;          // ring depth (pages)
    constexpr int LPB = BLOCK / 16 / kThreads;        // 16-byte loads per lane per block
    constexpr int LPP = SHARED ? LPB : 2 * LPB;       // ... per page
    static_assert(NSTAGE >= 3, "ring too shallow");

    __shared__ __attribute__((aligned(1024))) uint8_t ring[NSTAGE][STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c16 = lane & 15, r4 = lane >> 4;
    const int g = a.group, Hq = a.num_q_heads;

    // ---- XCD-aware work mapping: the dispatcher deals workgroups round-robin over the
    // XCDs, so give XCD x a contiguous run of work items (query tile fastest).
    const int nwg = gridDim.x * gridDim.y * gridDim.z;
    const int wid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int xcd = wid % kXcds, per = nwg / kXcds, extra = nwg % kXcds;
    const int item = xcd * per + min(xcd, extra) + wid / kXcds;
    const int qt = item % gridDim.x;
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
    const int lo = a.is_global ? 0 : max(0, p_first - a.window + 1);
    const int pg0 = lo / kPage, pg1 = p_last / kPage;
    const int npg = bad_row ? 0 : pg1 - pg0 + 1;
    const int32_t *pt = a.page_table + (int64_t)b * a.pt_stride;

    // ---- this wave's rows: tile rt, lane c16 -> row m -> (query tile_q + m / g, head m % g)
    int row_pos[kRT], row_head[kRT], p_row[kRT], lo_row[kRT];
    bool row_ok[kRT];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
        const int m = (wave * kRT + rt) * 16 + c16;
        row_pos[rt] = m / g;
        row_head[rt] = m % g;
        row_ok[rt] = row_pos[rt] < nq;
        p_row[rt] = p_first + row_pos[rt];
        lo_row[rt] = a.is_global ? 0 : p_row[rt] - a.window + 1;
    }

    // ---- Q^T as the B operand: lane holds row c16, 8 dims per K-step (zeros for padding rows)
    u32x4 qb[kRT][NS];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
        const uint16_t *qp =
            a.q + ((int64_t)(q0 + tile_q + (row_ok[rt] ? row_pos[rt] : 0)) * Hq + kvh * g + row_head[rt]) * HD + r4 * 8;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const u32x4 v = *(const u32x4 *)(qp + s * 32);
            qb[rt][s] = row_ok[rt] ? v : u32x4{0, 0, 0, 0};
        }
    }

    f32x4 acc[kRT][NT];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
        for (int j = 0; j < NT; ++j)
            acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[kRT], l_run[kRT];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
        m_run[rt] = -INFINITY;
        l_run[rt] = 0.f;
    }
    int bad_page = 0;

    // ---- page i of the tile's range -> its ring stage, via direct buffer->LDS loads. Lane l
    // of load k lands at byte (k * kThreads + wave * 64 + l) * 16 of the block; it fetches
    // the chunk that the swizzled layout puts there. Pages past the range (or with a bad
    // id) use a zero-size resource: zeros, no traffic.
    uint32_t src_off[LPB];
#pragma unroll
    for (int k = 0; k < LPB; ++k) {
        const int P = k * kThreads + wave * 64 + lane;  // chunk position in the block
        const int t = P / (HD / 8);
        const int c = (P % (HD / 8)) ^ (t & 15);
        src_off[k] = (uint32_t)(t * HD + c * 8) * 2u;
    }
    // Page ids of the tile's range, 64 per vector register (lane j: page 64*k + j), read back
    // with readlane so the page loop never waits on a memory load for an id.
    auto load_ids = [&](int first) { return pt[pg0 + min(first + lane, max(npg - 1, 0))]; };
    int ids = load_ids(0), ids_next = load_ids(64);
    int ids_base = 0;  // page index of ids' lane 0
    auto issue_page = [&](int i) {
        int pid = 0;
        bool live = i < npg;
        if (live) {
            const int rel = i - ids_base;  // 0..127
            pid = __builtin_amdgcn_readlane(rel >= 64 ? ids_next : ids, rel & 63);
            if (pid < 0 || pid >= a.num_pages) {
                bad_page = 1;
                live = false;
                pid = 0;
            }
        }
        const int64_t blk = ((int64_t)pid * a.num_kv_heads + kvh) * (kPage * HD);
        const uint32_t dst = (uint32_t)(uintptr_t)ring[i % NSTAGE] + (uint32_t)(wave * 64 * 16);
        const u32x4 rk = raw_rsrc(a.k_pool + blk, live ? BLOCK : 0);
#pragma unroll
        for (int k = 0; k < LPB; ++k)
            ring_load16(rk, dst + k * kThreads * 16, src_off[k]);
        if (!SHARED) {
            const u32x4 rv = raw_rsrc(a.v_pool + blk, live ? BLOCK : 0);
#pragma unroll
            for (int k = 0; k < LPB; ++k)
                ring_load16(rv, dst + BLOCK + k * kThreads * 16, src_off[k]);
        }
    };

    // Per-lane LDS byte offsets of the operand reads, K-step / dim-tile 0. The swizzle is an
    // XOR on bits that the step index does not share with the row base, so step s of the K
    // read is k_base ^ (64 s) and dim tile j of the V transpose read is v_base ^ (32 j).
    const uint32_t k_base = (uint32_t)(c16 * HD * 2) + ((uint32_t)(16 * r4) ^ (uint32_t)(16 * c16));
    const int tok = 4 * r4 + (c16 >> 2), half = (c16 & 3) >> 1;
    const uint32_t v_base = (uint32_t)(tok * HD * 2) + ((uint32_t)(16 * half) ^ (uint32_t)(16 * tok)) +
                            8u * (uint32_t)(c16 & 1);

    const float scale = a.scale_log2;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // Q and the first page ids are in registers before the ring starts, so that inside the
    // page loop the only vector-memory operations in flight are the ring's own loads and the
    // loop's wait below is exact.
    __builtin_amdgcn_s_waitcnt(0);  // (the compiler's own view: nothing of its is in flight)
#pragma unroll
    for (int i = 0; i < NSTAGE - 1; ++i)
        issue_page(i);

    for (int i = 0; i < npg; ++i) {
        // page i landed for this wave once at most the later NSTAGE-2 pages' loads are
        // outstanding; the barrier makes every wave's share visible and also certifies that
        // page i-1's stage has been fully read, so it can be refilled.
        wait_vmcnt<(NSTAGE - 2) * LPP>();
        __syncthreads();
        if (i + NSTAGE - 1 - ids_base >= 64 + 32) {  // slide the id window (every 64 pages)
            ids = ids_next;
            ids_base += 64;
            ids_next = load_ids(ids_base + 64);
        }
        issue_page(i + NSTAGE - 1);
        const uint8_t *kst = ring[i % NSTAGE];
        const uint8_t *vst = SHARED ? kst : kst + BLOCK;

        // S^T[token c16 .. ][row c16] per row tile: A = K[token c16][8 dims] from LDS (shared by
        // both tiles), B = Q^T
        f32x4 st[kRT];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
            st[rt] = zero;
#pragma unroll
        for (int s0 = 0; s0 < NS; s0 += 2) {
            // chunk_off(c16, 4s + r4) == k_base ^ (64 s)
            u32x4 ka[2];
            k_read2(ka, kst, k_base ^ (64u * s0), 64u);
#pragma unroll
            for (int k = 0; k < 2; ++k)
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt)
                    st[rt] = mfma_k32(ka[k], qb[rt][s0 + k], st[rt]);
        }
        // mask + online softmax; lane holds S^T[token t0 + 4*r4 + e][row c16 of tile rt]
        const int t0 = (pg0 + i) * kPage;
        u32x2 pb[kRT];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            float mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = t0 + 4 * r4 + e;
                const bool ok = row_ok[rt] && t <= p_row[rt] && t >= lo_row[rt];
                const float v = ok ? st[rt][e] * scale : -INFINITY;
                st[rt][e] = v;
                mx = fmaxf(mx, v);
            }
            mx = rows_max(mx);
            const float m_new = fmaxf(m_run[rt], mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;  // row with no visible key yet
            const float alpha = fast_exp2(m_run[rt] - m_use);
            float ps[4], rs = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ps[e] = fast_exp2(st[rt][e] - m_use);
                rs += ps[e];
            }
            rs = rows_sum(rs);
            l_run[rt] = l_run[rt] * alpha + rs;
            m_run[rt] = m_new;
            if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[rt][j] *= alpha;
            }
            pb[rt] = u32x2{pack_bf16x2(ps[0], ps[1]), pack_bf16x2(ps[2], ps[3])};
        }

        // V^T tiles with the transpose read: lane a of 16-lane group r4 supplies 4 dims of
        // token 4*r4 + a/4; lane c16 receives dim c16 of tokens 4*r4 .. 4*r4+3. Tokens no
        // row of the tile can see (before the window, past the last query) carry P = 0, and
        // their V (possibly a NaN slot) is selected out rather than multiplied by zero.
        const bool edge = t0 < lo || t0 + kPage - 1 > p_last;
        uint32_t keep[2] = {0xFFFFFFFFu, 0xFFFFFFFFu};
        if (edge) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = t0 + 4 * r4 + e;
                if (t < lo || t > p_last)
                    keep[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
            }
        }
#pragma unroll
        for (int j0 = 0; j0 < NT; j0 += 4) {
            // chunk_off(tok, 2j + h) + 8 * (c16 & 1) == v_base ^ (32 j)
            u32x2 vt[4];
            tr_read4(vt, vst, v_base ^ (32u * j0), 32u);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                u32x2 va = vt[k];
                va[0] &= keep[0];
                va[1] &= keep[1];
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt)
                    acc[rt][j0 + k] = mfma_k16(va, pb[rt], acc[rt][j0 + k]);
            }
        }
    }

    // ---- normalise and write this wave's rows
    const bool bad = bad_row || __builtin_amdgcn_ballot_w64(bad_page) != 0;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
        if (!row_ok[rt])
            continue;
        const int64_t orow = (int64_t)(q0 + tile_q + row_pos[rt]) * Hq + kvh * g + row_head[rt];
        const float inv = 1.0f / l_run[rt];
        uint16_t *op = a.out + orow * HD + 4 * r4;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            f32x4 o = acc[rt][j] * inv;
            if (bad)
                o = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
            *(u32x2 *)(op + 16 * j) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        }
        if (r4 == 0)
            a.lse[orow] = bad ? __builtin_nanf("") : (m_run[rt] + fast_log2(l_run[rt])) * kLn2;
    }
}

template <int HD, bool SHARED>
hipError_t launch(const PrefillArgs &a, dim3 grid, hipStream_t stream) {
    void *args[] = {(void *)&a};
    return hipLaunchKernel((const void *)prefill_kernel<HD, SHARED>, grid, dim3(Shape<HD>::THREADS), args, 0,
                           stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, int head_dim, bool kv_shared, int batch, hipStream_t stream) {
    const int bq = (head_dim == 256 ? Shape<256>::ROWS : Shape<512>::ROWS) / a.group;
    const dim3 grid((a.max_q + bq - 1) / bq, a.num_kv_heads, batch);
    if (head_dim == 256)
        return kv_shared ? launch<256, true>(a, grid, stream) : launch<256, false>(a, grid, stream);
    if (head_dim == 512)
        return kv_shared ? launch<512, true>(a, grid, stream) : launch<512, false>(a, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace gattn
