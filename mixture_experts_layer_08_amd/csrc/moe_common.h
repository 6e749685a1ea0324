// Shared device helpers for the gfx950 MoE kernels: bf16 storage
// conversions, MFMA operand types, wave-level reductions and host-side
// argument checks.  Nothing here is method arithmetic beyond rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf2f(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bit pattern, round to nearest, ties to even; NaN stays NaN
// (v_cvt_pk_bf16_f32, two values per instruction in pack_bf2, lo in the
// low half).
typedef __bf16 bf16x2_pk_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    const bf16x2_pk_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

// Reductions inside aligned groups of `width` lanes (width a power of two
// not above 64).
__device__ __forceinline__ float group_max(float v, int width) {
    for (int o = width >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, width));
    return v;
}
__device__ __forceinline__ float group_sum(float v, int width) {
    for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, width);
    return v;
}

}  // namespace moe

// ----------------------------------------------------------------- host ----
#define MOE_CHECK_LAUNCH()                                       \
    do {                                                         \
        if (hipGetLastError() != hipSuccess) return MOE_ERR_LAUNCH; \
    } while (0)

static inline bool moe_aligned16(const void* p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}
