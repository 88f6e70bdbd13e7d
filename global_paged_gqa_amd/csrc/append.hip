// KV append on gfx950: the K and V rows of new tokens copied into their pages.
//
// Row r appends n = cu_new[r+1] - cu_new[r] tokens at positions ctx_lens[r] - n + i; token t
// lands in page page_table[r][t / 16], slot t % 16, and its (kv_head) row of head_dim bf16 is
// contiguous in both the source and the (page, kv_head) block of the pool (the paged layout of
// the gattn.h header; the pegainfer "[Model] Gemma 4 M2 26B-A4B" plan's checked page offsets).
// One workgroup copies kTok tokens of one row: each lane owns one 16-byte chunk position of a
// (token, kv_head) row and steps through rows, kUnroll of them loaded before any is stored, so
// every wave reads and writes whole contiguous rows with several loads in flight, and a row's
// page id is looked up once per row. It is a pure copy, bound by HBM bandwidth: 2 * head_dim * 2 bytes read and
// written per (token, kv_head) and pool (K, and V unless V is the K cache).
//
// Into an FP8 (E4M3) pool (the pegainfer "[Model] Gemma 4 M2 26B-A4B" plan's opt-in FP8 KV pool)
// each element is stored as the code nearest to the fp32 quotient value / scale (IEEE division),
// ties to the even code, magnitudes of 448 and above saturating to 448, NaN kept as NaN; a lane's
// 16 source bytes become 8 pool bytes.
#include "common.h"
#include "kernels.h"

namespace gattn {

namespace {

constexpr int kThreads = 256;
constexpr int kTok = 8;     // tokens per workgroup
// rows a lane loads before it stores them (loads in flight): eight 1 KB rows at head_dim 512, four
// 512 B rows at 256 (measured on the mixed step's append: eight at 512 +6%, eight at 256 -5%)
constexpr int unroll(int hd) { return hd == 512 ? 8 : 4; }

// Four bf16 values (two packed words) -> four E4M3 bytes of value / scale, first value lowest:
// the code nearest to the fp32 quotient (IEEE division), ties to the even code, magnitudes of 448
// and above (infinities included) saturating to 448, a NaN value giving sign | 0x7f. The quotients
// are clamped to [-448, 448] and converted by the gfx950 conversion instruction (round to
// nearest even, subnormal codes included, sign of zeros kept); it writes every NaN as 0xff, and a
// NaN reaches it clamped anyway, so NaN bytes are set afterwards, on the rare waves that hold one.
// Checked against the oracle's encoder on every bf16 value.
__device__ __forceinline__ float e4m3_arg(float x, float scale) { return fminf(fmaxf(x / scale, -448.0f), 448.0f); }

__device__ __forceinline__ uint32_t e4m3x4(uint32_t w0, uint32_t w1, float scale) {
    const float x[4] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1)};
    const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_arg(x[0], scale), e4m3_arg(x[1], scale), 0,
                                                                   false);
    uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_arg(x[2], scale), e4m3_arg(x[3], scale),
                                                              (int)lo, true);
    const bool any_nan = (x[0] != x[0]) | (x[1] != x[1]) | (x[2] != x[2]) | (x[3] != x[3]);
    if (__builtin_amdgcn_ballot_w64(any_nan)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (x[i] != x[i])
                code = (code & ~(0xffu << (8 * i))) |
                       (((__builtin_bit_cast(uint32_t, x[i]) >> 24 & 0x80u) | 0x7fu) << (8 * i));
    }
    return code;
}

template <int HD, bool F8>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(AppendArgs a) {
    constexpr int CPR = HD / 8;           // 16-byte chunks per (token, kv_head) row
    constexpr int RPI = kThreads / CPR;   // rows a workgroup copies per step
    constexpr int kUnroll = unroll(HD);
    // At head_dim 256 a workgroup's rows take several passes of the loop below (four with 16 KV
    // heads); reading each source row before its table entry (a token with a bad page id is then
    // read and not written) lets the two loads overlap in every pass (5% on the mixed step's local
    // append). At 512 one pass covers a workgroup of up to four KV heads, and the table entry goes
    // first (the other order measured 1-3% slower).
    constexpr bool kSrcFirst = HD == 256;
    const int r = blockIdx.y;
    const int n0 = a.cu_new[r], n = a.cu_new[r + 1] - n0;
    const int i0 = blockIdx.x * kTok;
    if (i0 >= n)
        return;
    const int L = a.ctx_lens[r];
    // A malformed row (more new tokens than cached ones, or than the max_new bound the grid was
    // sized by, which would leave tokens past the grid unwritten) fails closed as a whole: none
    // of its tokens is written and the row's first workgroup raises the status flag.
    if (n > L || n > a.max_new) {
        if (blockIdx.x == 0 && threadIdx.x == 0 && a.status)
            atomicOr(a.status, 1);
        return;
    }
    const int nt = min(kTok, n - i0);
    const int Hkv = a.num_kv_heads;
    const int rows = nt * Hkv;
    const int32_t *pt = a.page_table + (int64_t)r * a.pt_stride;
    const int c = threadIdx.x % CPR, sub = threadIdx.x / CPR;  // this lane's chunk of its rows
    int bad = 0;
    for (int row0 = sub; row0 < rows; row0 += RPI * kUnroll) {
        u32x4 kv[kUnroll], vv[kUnroll];
        int64_t dst[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int row = row0 + u * RPI;
            dst[u] = -1;
            if (row >= rows)
                continue;
            const int it = row / Hkv, kvh = row - it * Hkv;
            const int t = L - n + i0 + it;  // absolute position of the token
            const int64_t src = ((int64_t)(n0 + i0 + it) * Hkv + kvh) * HD + c * 8;
            if constexpr (kSrcFirst) {
                kv[u] = *(const u32x4 *)(a.k_new + src);
                if (a.v_new)
                    vv[u] = *(const u32x4 *)(a.v_new + src);
            }
            const int pid = (t >> 4) < a.pt_stride ? pt[t >> 4] : -1;
            if (pid < 0 || pid >= a.num_pages) {
                bad = 1;
                continue;
            }
            dst[u] = (((int64_t)pid * Hkv + kvh) * kPage + (t & (kPage - 1))) * HD + c * 8;  // elements (bytes for FP8)
            if constexpr (!kSrcFirst) {
                kv[u] = *(const u32x4 *)(a.k_new + src);
                if (a.v_new)
                    vv[u] = *(const u32x4 *)(a.v_new + src);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (dst[u] < 0)
                continue;
            if constexpr (F8) {
                const u32x4 k = kv[u];
                *(u32x2 *)((uint8_t *)a.k_pool + dst[u]) =
                    u32x2{e4m3x4(k[0], k[1], a.k_scale), e4m3x4(k[2], k[3], a.k_scale)};
                if (a.v_new) {
                    const u32x4 v = vv[u];
                    *(u32x2 *)((uint8_t *)a.v_pool + dst[u]) =
                        u32x2{e4m3x4(v[0], v[1], a.v_scale), e4m3x4(v[2], v[3], a.v_scale)};
                }
            } else {
                *(u32x4 *)((uint16_t *)a.k_pool + dst[u]) = kv[u];
                if (a.v_new)
                    *(u32x4 *)((uint16_t *)a.v_pool + dst[u]) = vv[u];
            }
        }
    }
    if (a.status && __builtin_amdgcn_ballot_w64(bad) && (threadIdx.x & 63) == 0)
        atomicOr(a.status, 1);
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs &a, int head_dim, int batch, bool fp8, hipStream_t stream) {
    const dim3 grid((a.max_new + kTok - 1) / kTok, batch);
    void *args[] = {(void *)&a};
    if (fp8) {
        if (head_dim == 256)
            return hipLaunchKernel((const void *)kv_append_kernel<256, true>, grid, dim3(kThreads), args, 0, stream);
        if (head_dim == 512)
            return hipLaunchKernel((const void *)kv_append_kernel<512, true>, grid, dim3(kThreads), args, 0, stream);
        return hipErrorInvalidValue;
    }
    if (head_dim == 256)
        return hipLaunchKernel((const void *)kv_append_kernel<256, false>, grid, dim3(kThreads), args, 0, stream);
    if (head_dim == 512)
        return hipLaunchKernel((const void *)kv_append_kernel<512, false>, grid, dim3(kThreads), args, 0, stream);
    return hipErrorInvalidValue;
}

}  // namespace gattn
