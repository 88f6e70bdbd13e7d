// Internal device helpers shared by the gfx950 kernels of the attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gattn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kPage = 16;      // tokens per KV page
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D = A * B + C on a 16x16 tile, K = 32, bf16 inputs, fp32 accumulate.
// Lane l holds A row (l % 16) and B column (l % 16), eight K elements each; the
// K grouping by (l / 16, element) is the same for A and B. C/D: lane l holds
// rows 4 * (l / 16) + i (i = 0..3) of column l % 16.
__device__ __forceinline__ f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Same tile shape with K = 16: four K elements per lane.
__device__ __forceinline__ f32x4 mfma_k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 values to a bf16 pair (low, high), round to nearest even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// The bf16 values in the low / high half of a packed pair, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// The ring's direct buffer->LDS loads and the waits on them are inline assembly: the
// compiler sees neither, so it never orders its own LDS reads behind in-flight ring loads;
// a ring is synchronised by explicit "at most N loads outstanding" waits plus barriers.
//
// 16 bytes per lane from the buffer `rsrc` at byte offset voffset into LDS at lds + 16 * lane
// (M0 holds the LDS base; M0 is declared clobbered, so the compiler reloads it only where it
// keeps a value there itself: saving and restoring it around every load cost two scalar
// instructions per load, 2-4% of the hd 512 prefill). STREAM marks the load non-temporal: data
// read exactly once (decode's K/V) then does not displace cached lines, and a page stream
// sustains about 12% more bandwidth than with the default policy.
template <bool STREAM = false>
__device__ __forceinline__ void ring_load16(u32x4 rsrc, uint32_t lds, uint32_t voffset) {
    if (STREAM)
        asm volatile(
            "s_mov_b32 m0, %2\n\t"
            "buffer_load_dwordx4 %0, %1, 0 offen nt lds"
            :
            : "v"(voffset), "s"(rsrc), "s"(lds)
            : "memory", "m0");
    else
        asm volatile(
            "s_mov_b32 m0, %2\n\t"
            "buffer_load_dwordx4 %0, %1, 0 offen lds"
            :
            : "v"(voffset), "s"(rsrc), "s"(lds)
            : "memory", "m0");
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

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// gfx950 transpose read (ds_read_b64_tr_b16). In each 16-lane group, lane 4r + q supplies the
// LDS address of elements 4q .. 4q+3 of row r of a 4 x 16 bf16 tile; lane j of the group
// receives column j: rows 0..3 of element j, row r in 16-bit slot r.
__device__ __forceinline__ u32x2 tr_read(const uint8_t *p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
}

// Max and sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48) with the
// gfx950 lane swaps. v_permlane16_swap exchanges rows 1 and 3 of its first operand with rows 0
// and 2 of its second; with both operands holding x, each lane ends up with its own value in
// one register and its row partner's (lane l^16) in the other. v_permlane32_swap does the same
// for lanes l and l^32. Written as assembly: given two copies of one value, the compiler folds
// the builtins' two results into one. Both reductions are symmetric, so all four lanes of a
// column get the identical value.
__device__ __forceinline__ void swap_rows16(float &a, float &b) {
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_halves32(float &a, float &b) {
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// Max and sum over the two 32-lane halves of a wave (lanes l and l^32).
__device__ __forceinline__ float halves_max(float x) {
    float a = x, b = x;
    swap_halves32(a, b);
    return fmaxf(a, b);
}

__device__ __forceinline__ float halves_sum(float x) {
    float a = x, b = x;
    swap_halves32(a, b);
    return a + b;
}

__device__ __forceinline__ float rows_max4(float x) {
    float a = x, b = x;
    swap_rows16(a, b);
    float c = fmaxf(a, b), d = c;
    swap_halves32(c, d);
    return fmaxf(c, d);
}

__device__ __forceinline__ float rows_sum4(float x) {
    float a = x, b = x;
    swap_rows16(a, b);
    float c = a + b, d = c;
    swap_halves32(c, d);
    return c + d;
}

// LDS layout of a page of K or V (16 token rows of head_dim bf16) staged for MFMA operand
// reads: token row t at t * HD * 2 bytes, its 16-byte chunk c at chunk slot c ^ dswz(t). dswz is a
// bijection of the four token bits whose values for tokens 0..7 (and for 8..15) differ above
// bit 0, so that (i) a K operand read (16 tokens at one chunk) hits 16 different 16-byte bank
// groups and (ii) a transpose read of a 16-dim tile (8 tokens x 2 adjacent chunks in each half
// wave) hits 16. Token rows are multiples of 256 bytes, so only the chunk slot picks the bank.
__device__ __forceinline__ int dswz(int t) { return ((t & 7) << 1) | ((t >> 3) & 1); }

// NaN-propagating max (fmaxf would drop a NaN operand).
__device__ __forceinline__ float nan_max(float a, float b) { return (a > b || a != a) ? a : b; }

}  // namespace gattn
