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

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// Two fp32 values that are exactly representable in bf16: keep their high halves.
__device__ __forceinline__ uint32_t pack_exact_bf16x2(float lo, float hi) {
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo),
                                 0x07060302u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// All-reduce across the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48),
// always combining in the same order so every lane gets the identical value.
__device__ __forceinline__ float rows_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float rows_sum(float x) {
    // (r0 + r1) + (r2 + r3) in every lane (addition commutes exactly)
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// 16 bytes per lane from a buffer straight into LDS: lane l's data lands at lds + 16 * l
// (lds must be wave-uniform). The host compilation pass never sees the builtin, whose
// LDS pointer type has no host meaning.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, void *lds, uint32_t voffset) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds, 16, voffset, 0,
                                             0, 0);
#endif
}

// NaN-propagating max (fmaxf would drop a NaN operand).
__device__ __forceinline__ float nan_max(float a, float b) { return (a > b || a != a) ? a : b; }

}  // namespace gattn
