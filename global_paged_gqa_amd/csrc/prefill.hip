// Chunked causal prefill over the paged KV cache on gfx950 (bf16 MFMA, fp32 softmax).
//
// A chunk's queries attend the cache with the causal mask inside the chunk and the
// sliding window for the local family (Core AI card, "Contents": a flash-prefill
// with a query axis and an intra-chunk causal mask). One workgroup = one (row,
// KV head, query tile). The g query heads that share the KV head are packed into
// the MFMA rows: row m of the tile is (position m / g, head m % g), so every
// K/V byte staged in LDS serves all g heads.
//
// Four waves per workgroup. A wave owns 32 rows (two 16-row MFMA tiles) and 256
// head dims; with head_dim 512 two waves share the rows, splitting the dims, and
// add their partial scores through LDS. The key range of a tile is pruned to
// [first visible key of its first query, its last query]: whole pages outside
// the window are never read (page 5's "Three load-bearing facts" #1: sliding-
// window tile pruning).
//
// Per KV page (16 tokens):
//   S^T[16 tok][32 rows] = K . Q^T      MFMA 16x16x32, K from LDS (XOR-swizzled rows),
//                                       Q^T held in registers
//   causal / window mask, online softmax per row (columns of S^T)
//   O^T[dims][32 rows] += V^T . P^T     MFMA 16x16x16; V^T read from the row-major LDS
//                                       page with the gfx950 transpose read
//                                       (ds_read_b64_tr_b16), P^T straight from S^T's
//                                       accumulator layout
// The next page is fetched into registers while the current one is computed and
// stored into the other LDS stage afterwards (one barrier per page).
#include "common.h"
#include "kernels.h"

namespace gattn {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kDimsPerWave = 256;
constexpr int kRowsPerWave = 32;

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

// LDS byte offset of 16-byte chunk `c` of token row `t` in a page stage: rows are
// HD*2 bytes, chunks XOR-swizzled by the token so that 16 rows read at the same
// logical chunk hit 16 different bank groups.
template <int HD>
__device__ __forceinline__ uint32_t chunk_off(int t, int c) {
    return (uint32_t)(t * HD * 2 + ((c ^ (t & 15)) << 4));
}

template <int HD, bool SHARED>
__global__ __launch_bounds__(kThreads, 1) void prefill_kernel(PrefillArgs a) {
    constexpr int DS = HD / kDimsPerWave;             // waves sharing the rows (1 or 2)
    constexpr int NRG = kWaves / DS;                  // row groups
    constexpr int BM = NRG * kRowsPerWave;            // rows per workgroup
    constexpr int NS = kDimsPerWave / 32;             // K-steps per wave
    constexpr int NT = kDimsPerWave / 16;             // 16-dim output tiles per wave
    constexpr int PAGE_BYTES = kPage * HD * 2;        // one (page, KV head) block
    constexpr int STAGE_BYTES = SHARED ? PAGE_BYTES : 2 * PAGE_BYTES;
    constexpr int CHUNKS = PAGE_BYTES / 16;            // 16-byte chunks per block
    constexpr int LD_PER_THREAD = CHUNKS / kThreads;   // chunks a thread moves per block

    __shared__ __attribute__((aligned(16))) uint8_t sm_kv[2][STAGE_BYTES];
    __shared__ f32x4 sm_x[DS > 1 ? kWaves : 1][DS > 1 ? 2 * 64 : 1];  // partial scores

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = wave / DS, dpart = wave % DS;
    const int c16 = lane & 15, r4 = lane >> 4;
    const int qt = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int g = a.group, Hq = a.num_q_heads;

    const int q0 = a.cu_q[b], q_len = a.cu_q[b + 1] - q0;
    const int L = a.ctx_lens[b];
    const int BQ = BM / g;                 // query positions per tile
    const int tile_q = qt * BQ;            // first query of the tile (within the row)
    if (q_len <= 0 || tile_q >= q_len)
        return;
    const int nq = min(BQ, q_len - tile_q);  // valid queries in the tile
    const int p_first = L - q_len + tile_q;  // absolute position of the tile's first query
    const int p_last = p_first + nq - 1;
    // Malformed rows (query count above the cache length, or cache beyond the table)
    // produce NaN outputs instead of reading outside the table.
    const bool bad_row = q_len > L || (L - 1) / kPage >= a.pt_stride;

    const int lo = a.is_global ? 0 : max(0, p_first - a.window + 1);
    const int pg0 = lo / kPage, pg1 = p_last / kPage;
    const int npg = bad_row ? 0 : pg1 - pg0 + 1;
    const int32_t *pt = a.page_table + (int64_t)b * a.pt_stride;

    // ---- rows of this wave: two 16-row tiles; row m -> (query tile_q + m / g, head m % g)
    int row_pos[2], row_head[2];
    bool row_ok[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int m = rg * kRowsPerWave + rt * 16 + c16;
        row_pos[rt] = m / g;
        row_head[rt] = m % g;
        row_ok[rt] = row_pos[rt] < nq;
    }

    // ---- Q^T as the B operand: lane holds row c16 of each row tile, 8 dims per K-step
    u32x4 qb[2][NS];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int pos = row_ok[rt] ? row_pos[rt] : 0;
        const uint16_t *qp = a.q + ((int64_t)(q0 + tile_q + pos) * Hq + kvh * g + row_head[rt]) * HD +
                             dpart * kDimsPerWave + r4 * 8;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const u32x4 v = *(const u32x4 *)(qp + s * 32);
            qb[rt][s] = row_ok[rt] ? v : u32x4{0, 0, 0, 0};
        }
    }

    f32x4 acc[2][NT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int j = 0; j < NT; ++j)
            acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    int bad_page = 0;

    // ---- staging: every thread moves LD_PER_THREAD 16-byte chunks of K (and V) per page
    u32x4 pk[LD_PER_THREAD], pvr[SHARED ? 1 : LD_PER_THREAD];
    auto fetch = [&](int i) {  // global -> registers, page i of the tile's range (clamped)
        int pid = pt[pg0 + min(i, max(npg - 1, 0))];
        if (pid < 0 || pid >= a.num_pages) {
            if (i < npg)
                bad_page = 1;
            pid = 0;
        }
        const int64_t base = ((int64_t)pid * a.num_kv_heads + kvh) * (kPage * HD);
#pragma unroll
        for (int k = 0; k < LD_PER_THREAD; ++k) {
            const int c = threadIdx.x + k * kThreads;
            pk[k] = *(const u32x4 *)(a.k_pool + base + c * 8);
            if (!SHARED)
                pvr[k] = *(const u32x4 *)(a.v_pool + base + c * 8);
        }
    };
    auto stash = [&](int stage) {  // registers -> LDS stage (swizzled rows)
#pragma unroll
        for (int k = 0; k < LD_PER_THREAD; ++k) {
            const int c = threadIdx.x + k * kThreads;
            const int t = c / (HD / 8), ch = c % (HD / 8);
            *(u32x4 *)(sm_kv[stage] + chunk_off<HD>(t, ch)) = pk[k];
            if (!SHARED)
                *(u32x4 *)(sm_kv[stage] + PAGE_BYTES + chunk_off<HD>(t, ch)) = pvr[k];
        }
    };

    const float scale = a.scale_log2;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    if (npg > 0) {
        fetch(0);
        stash(0);
    }
    __syncthreads();

    for (int i = 0; i < npg; ++i) {
        const int stage = i & 1;
        const uint8_t *kst = sm_kv[stage];
        const uint8_t *vst = SHARED ? kst : sm_kv[stage] + PAGE_BYTES;
        if (i + 1 < npg)
            fetch(i + 1);

        // S^T partial over this wave's dims: A = K[token c16][8 dims] from LDS
        f32x4 st[2] = {zero, zero};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int ch = (dpart * kDimsPerWave + s * 32 + r4 * 8) / 8;
            const u32x4 ka = *(const u32x4 *)(kst + chunk_off<HD>(c16, ch));
            st[0] = mfma_k32(ka, qb[0][s], st[0]);
            st[1] = mfma_k32(ka, qb[1][s], st[1]);
        }
        if (DS > 1) {
            sm_x[wave][lane] = st[0];
            sm_x[wave][64 + lane] = st[1];
            __syncthreads();
            const f32x4 o0 = sm_x[wave ^ 1][lane], o1 = sm_x[wave ^ 1][64 + lane];
            st[0] = dpart == 0 ? st[0] + o0 : o0 + st[0];
            st[1] = dpart == 0 ? st[1] + o1 : o1 + st[1];
        }

        // mask + online softmax; lane holds S^T[token t0 + 4*r4 + e][row c16 of tile rt]
        const int t0 = (pg0 + i) * kPage;
        u32x2 pb[2];
        bool tok_ok[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int p = p_first + row_pos[rt];
            const int lo_r = a.is_global ? 0 : p - a.window + 1;
            float mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = t0 + 4 * r4 + e;
                tok_ok[rt][e] = row_ok[rt] && t <= p && t >= lo_r;
                const float v = tok_ok[rt][e] ? st[rt][e] * scale : -INFINITY;
                st[rt][e] = v;
                mx = fmaxf(mx, v);
            }
            mx = rows_max(mx);
            const float m_new = fmaxf(m_run[rt], mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;  // row with no key yet
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
        // token 4*r4 + a/4; lane c16 receives dim c16 of tokens 4*r4 .. 4*r4+3.
        // Tokens outside every row's range carry P = 0; a NaN slot would still poison the
        // product, so those tokens' V is selected out first.
        const bool edge_tokens = t0 < lo || t0 + kPage - 1 > p_last;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int dim0 = dpart * kDimsPerWave + 16 * j + 4 * (c16 & 3);
            const int tok = 4 * r4 + (c16 >> 2);
            const uint32_t off = chunk_off<HD>(tok, dim0 >> 3) + ((dim0 & 4) << 1);
            i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vst + off));
            u32x2 va = __builtin_bit_cast(u32x2, v);
            if (edge_tokens) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = t0 + 4 * r4 + e;
                    if (t < lo || t > p_last)
                        va[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
                }
            }
            acc[0][j] = mfma_k16(va, pb[0], acc[0][j]);
            acc[1][j] = mfma_k16(va, pb[1], acc[1][j]);
        }

        if (i + 1 < npg)
            stash(stage ^ 1);
        __syncthreads();
    }

    // ---- normalise and write this wave's rows and dims
    bool bad = bad_row;
    bad = bad || __builtin_amdgcn_ballot_w64(bad_page) != 0;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        if (!row_ok[rt])
            continue;
        const int64_t orow = (int64_t)(q0 + tile_q + row_pos[rt]) * Hq + kvh * g + row_head[rt];
        const float inv = 1.0f / l_run[rt];
        uint16_t *op = a.out + orow * HD + dpart * kDimsPerWave + 4 * r4;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            f32x4 o = acc[rt][j] * inv;
            if (bad)
                o = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
            *(u32x2 *)(op + 16 * j) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        }
        if (dpart == 0 && r4 == 0)
            a.lse[orow] = bad ? __builtin_nanf("") : (m_run[rt] + fast_log2(l_run[rt])) * kLn2;
    }
}

template <int HD, bool SHARED>
hipError_t launch(const PrefillArgs &a, dim3 grid, hipStream_t stream) {
    void *args[] = {(void *)&a};
    return hipLaunchKernel((const void *)prefill_kernel<HD, SHARED>, grid, dim3(kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, int head_dim, bool kv_shared, int batch, hipStream_t stream) {
    const int rows = (kWaves / (head_dim / kDimsPerWave)) * kRowsPerWave;
    const int bq = rows / a.group;
    const dim3 grid((a.max_q + bq - 1) / bq, a.num_kv_heads, batch);
    if (head_dim == 256)
        return kv_shared ? launch<256, true>(a, grid, stream) : launch<256, false>(a, grid, stream);
    if (head_dim == 512)
        return kv_shared ? launch<512, true>(a, grid, stream) : launch<512, false>(a, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace gattn
