// Chunked causal prefill over the paged KV cache on gfx950 (bf16 MFMA, fp32 softmax).
//
// A chunk's queries attend the cache with the causal mask inside the chunk and the
// sliding window for the local family (Core AI card, "Contents": a flash-prefill
// with a query axis and an intra-chunk causal mask). One workgroup = one (row, KV
// head, query tile) of 128 MFMA rows; the g query heads that share the KV head are
// packed into the rows (row m = query position m / g, head m % g), so every K/V byte
// staged in LDS serves all g heads.
//
// Keys are processed in blocks of 32 tokens (two pages). Both products use the
// 32x32x16 bf16 MFMA, which runs at the full matrix rate on gfx950 (the 16x16x16 form
// runs at half rate):
//   QK: wave w computes S^T[32 tok][32 rows] = K . Q^T for its own 32 rows over the whole
//       head_dim (A = K from LDS, B = Q^T kept in registers), then the masked online
//       softmax of those rows.
//   P exchange: each wave stores its P^T as bf16 in LDS, already in the lane order of the
//       PV product's B operand, plus the rows' rescale factors.
//   PV: wave w owns head_dim/4 output dims for all 128 rows: O^T[dims][rows] += V^T . P^T,
//       with V^T read from the row-major page by the gfx950 transpose read
//       (ds_read_b64_tr_b16). Every V^T fragment feeds four MFMAs (the four row tiles).
// K and V blocks stream through a 128 KB LDS ring filled by direct global->LDS buffer
// loads several blocks ahead; two barriers per block (one also publishes P).
//
// The online softmax rescales lazily: a row keeps its running maximum until a new score
// exceeds it by more than 2^8, so P stays below 256 and the accumulators are rescaled only
// on those (rare) blocks. The final O = acc / l and LSE = m + log2 l use the same maximum,
// so the result is the exact softmax up to rounding.
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
    constexpr int DW = HD / kWaves;                  // output dims per wave in PV
    constexpr int ND = DW / 32;                      // 32-dim output tiles per wave
    constexpr int UNIT = kTok * HD * 2;              // bytes of the K (or V) of one block
    constexpr int NU = kRingBytes / UNIT;            // ring depth in units
    constexpr int LPU = UNIT / 16 / kThreads;        // 16-byte loads per lane per unit
    constexpr int PAGE_BYTES = kPage * HD * 2;       // one (page, KV head) block
    static_assert(NU >= 3 && LPU % 2 == 0, "ring shape");

    __shared__ __attribute__((aligned(1024))) uint8_t ring[kRingBytes];
    __shared__ __attribute__((aligned(16))) uint8_t p_lds[kWaves * 2 * 64 * 16];  // P^T fragments
    __shared__ float alpha_lds[kRows];
    __shared__ float l_lds[kRows];
    __shared__ int flag_lds[kWaves];

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

    // ---- this wave's score rows (QK / softmax): row m = 32 * wave + n32
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

    f32x16 acc[ND][kWaves];
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int t = 0; t < kWaves; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[d][t][v] = 0.f;
    float m_run = -INFINITY, l_part = 0.f;
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
    // Unit u: block u (K=V) or block u/2, K if u even else V. Units past the last block, and
    // pages of a block outside [lo, p_last], load zeros with no memory traffic, so that every
    // wave always has exactly LPU loads per unit in flight and the ring waits stay exact.
    auto issue = [&](int u) {
        const int blk = SHARED ? u : (u >> 1);
        const bool is_v = !SHARED && (u & 1);
        const uint16_t *pool = is_v ? a.v_pool : a.k_pool;
        if (blk < nblk && 2 * blk + 1 - ids_base >= 96) {  // slide the id window (every 32 blocks)
            ids = ids_next;
            ids_base += 64;
            ids_next = load_ids(ids_base + 64);
        }
        u32x4 rs[2];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            const int rel = 2 * blk + pp;
            const int pg = pgA + rel;
            bool live = blk < nblk && pg * kPage <= p_last && pg * kPage + kPage - 1 >= lo;
            int pid = 0;
            if (live) {
                const int r = rel - ids_base;  // 0..127
                pid = __builtin_amdgcn_readlane(r >= 64 ? ids_next : ids, r & 63);
                if (pid < 0 || pid >= a.num_pages) {
                    bad_page = 1;
                    live = false;
                    pid = 0;
                }
            }
            rs[pp] = raw_rsrc(pool + ((int64_t)pid * a.num_kv_heads + kvh) * (kPage * HD), live ? PAGE_BYTES : 0);
        }
        const uint32_t dst = (uint32_t)(uintptr_t)(ring + (u % NU) * UNIT) + (uint32_t)(wave * 64 * 16);
#pragma unroll
        for (int k = 0; k < LPU; ++k)
            ring_load16(rs[k < LPU / 2 ? 0 : 1], dst + k * kThreads * 16, src_off(k));
    };

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
    // V^T operand (transpose read i of dim tile d, page p): in 16-lane group G (G&1: dims
    // 16..31 of the tile, G>>1 = h), lane 4r + q supplies token 16p + 8i + 4h + r, dims
    // 4q .. 4q+3 of its 16; the lane receives its dim for those four tokens.
    uint32_t vb[2][ND];
    {
        const int G = lane >> 4, gh = G & 1, r = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                const int tok = 8 * i + 4 * h + r;
                const int c = (wave * DW) / 8 + 4 * d + 2 * gh + (q >> 1);
                vb[i][d] = (uint32_t)(tok * HD * 2 + 16 * (c ^ swz(tok)) + 8 * (q & 1));
            }
    }

    const float scale = a.scale_log2;
    // Q and the first page ids are in registers before the ring starts, so that inside the
    // block loop the only vector-memory operations in flight are the ring's own loads.
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int u = 0; u < NU - 1; ++u)
        issue(u);

    for (int blk = 0; blk < nblk; ++blk) {
        const int uk = SHARED ? blk : 2 * blk;
        // unit uk landed for this wave once at most the later NU-2 units' loads are
        // outstanding; the barrier makes every wave's share visible and certifies that the
        // previous block is fully read, so its slot can be refilled.
        wait_vmcnt<(NU - 2) * LPU>();
        __syncthreads();
        issue(uk + NU - 1);
        const uint8_t *kst = ring + (uk % NU) * UNIT;

        // ---- S^T[32 tok][32 rows] for this wave's rows. Operand reads run one group of four
        // K-steps ahead of the MFMAs; the scheduling fences keep the compiler from hoisting
        // every read of the block (which would not fit beside Q in registers).
        f32x16 st;
        auto kread = [&](int s) { return *(const u32x4 *)(kst + kb[s & 7] + 256 * (s >> 3)); };
        u32x4 kf[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            kf[0][i] = kread(i);
#pragma unroll
        for (int j = 0; j < NKS / 4; ++j) {
            if (j + 1 < NKS / 4) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    kf[(j + 1) & 1][i] = kread(4 * (j + 1) + i);
            }
            const u32x4 *kk = kf[j & 1];
            if (j == 0)
                qk4<true>(st, kk[0], kk[1], kk[2], kk[3], qb[0], qb[1], qb[2], qb[3]);
            else
                qk4<false>(st, kk[0], kk[1], kk[2], kk[3], qb[4 * j], qb[4 * j + 1], qb[4 * j + 2], qb[4 * j + 3]);
            __builtin_amdgcn_sched_barrier(0);
        }
        qk_settle(st);

        // ---- masked online softmax of the rows; lane holds tokens 8(v/4) + 4h + v%4
        const int T0 = kb0 + blk * kTok;
        const bool edge = T0 + kTok - 1 > p_first || (!a.is_global && T0 < p_last - a.window + 1);
        float mx = -INFINITY;
        if (edge) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int T = T0 + 8 * (v >> 2) + 4 * h + (v & 3);
                const bool vis = T <= p_own && (a.is_global || p_own - T < a.window);
                st[v] = vis ? st[v] * scale : -INFINITY;
                mx = fmaxf(mx, st[v]);
            }
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                st[v] *= scale;
                mx = fmaxf(mx, st[v]);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const bool resc = m_new > m_run + kRescaleLog2;
        const float alpha = resc ? fast_exp2(m_run - m_new) : 1.0f;
        if (resc)
            m_run = m_new;
        const float mb = m_run == -INFINITY ? 0.f : m_run;
        float ps[16], rs = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            ps[v] = fast_exp2(st[v] - mb);
            rs += ps[v];
        }
        l_part = l_part * alpha + rs;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const u32x4 pk = {pack_bf16x2(ps[8 * p + 0], ps[8 * p + 1]), pack_bf16x2(ps[8 * p + 2], ps[8 * p + 3]),
                              pack_bf16x2(ps[8 * p + 4], ps[8 * p + 5]), pack_bf16x2(ps[8 * p + 6], ps[8 * p + 7])};
            *(u32x4 *)(p_lds + ((wave * 2 + p) * 64 + lane) * 16) = pk;
        }
        const bool any_resc = __builtin_amdgcn_ballot_w64(resc) != 0;
        if (h == 0)
            alpha_lds[m_own] = alpha;
        if (lane == 0)
            flag_lds[wave] = any_resc;

        // ---- V unit (separate pools) and the P exchange
        const int uv = SHARED ? blk : 2 * blk + 1;
        if (!SHARED)
            wait_vmcnt<(NU - 2) * LPU>();
        __syncthreads();
        if (!SHARED)
            issue(uv + NU - 1);
        const uint8_t *vst = ring + (uv % NU) * UNIT;

#pragma unroll
        for (int t = 0; t < kWaves; ++t) {
            if (__builtin_amdgcn_readfirstlane(flag_lds[t])) {
                const float al = alpha_lds[32 * t + n32];
#pragma unroll
                for (int d = 0; d < ND; ++d)
                    scale_acc(acc[d][t], al);
            }
        }
        // Tokens no row of the tile can see (before the window, past the last query) carry
        // P = 0; their V (possibly a never-written slot) is selected out rather than
        // multiplied by zero.
        u32x2 keep[2][2];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                keep[p][i] = u32x2{0xFFFFFFFFu, 0xFFFFFFFFu};
                if (edge) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int T = T0 + 16 * p + 8 * i + 4 * ((lane >> 5) & 1) + r;
                        if (T < lo || T > p_last)
                            keep[p][i][r >> 1] &= (r & 1) ? 0x0000FFFFu : 0xFFFF0000u;
                    }
                }
            }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            u32x4 pf[kWaves];
#pragma unroll
            for (int t = 0; t < kWaves; ++t)
                pf[t] = *(const u32x4 *)(p_lds + ((t * 2 + p) * 64 + lane) * 16);
            auto vread = [&](int d) {
                u32x2 v0 = tr_read(vst + vb[0][d] + p * PAGE_BYTES);
                u32x2 v1 = tr_read(vst + vb[1][d] + p * PAGE_BYTES);
                return u32x4{v0[0], v0[1], v1[0], v1[1]};
            };
            u32x4 vf[2];
            vf[0] = vread(0);
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                if (d + 1 < ND)
                    vf[(d + 1) & 1] = vread(d + 1);
                u32x4 va = vf[d & 1];
                if (edge)
                    va &= u32x4{keep[p][0][0], keep[p][0][1], keep[p][1][0], keep[p][1][1]};
#pragma unroll
                for (int t = 0; t < kWaves; ++t)
                    acc[d][t] = mfma32(va, pf[t], acc[d][t]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // No ring load (the zero-filling ones past the last block included) may still be writing
    // this workgroup's LDS when it ends.
    wait_vmcnt<0>();

    // ---- row sums, LSE (score owners), then normalise and write O (dim owners)
    const bool bad = bad_row || __builtin_amdgcn_ballot_w64(bad_page) != 0;
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    if (h == 0) {
        l_lds[m_own] = l_tot;
        if (ok_own) {
            const int64_t orow = (int64_t)(q0 + tile_q + pos_own) * Hq + kvh * g + m_own % g;
            a.lse[orow] = bad ? __builtin_nanf("") : (m_run + fast_log2(l_tot)) * kLn2;
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kWaves; ++t) {
        const int m = 32 * t + n32;
        const int pos = m / g;
        if (pos >= nq)
            continue;
        const float inv = 1.0f / l_lds[m];
        const int64_t orow = (int64_t)(q0 + tile_q + pos) * Hq + kvh * g + m % g;
        uint16_t *op = a.out + orow * HD + wave * DW + 4 * h;
#pragma unroll
        for (int d = 0; d < ND; ++d)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = bad ? __builtin_nanf("") : acc[d][t][4 * j + e] * inv;
                *(u32x2 *)(op + 32 * d + 8 * j) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            }
    }
}

template <int HD, bool SHARED>
hipError_t launch(const PrefillArgs &a, dim3 grid, hipStream_t stream) {
    void *args[] = {(void *)&a};
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
