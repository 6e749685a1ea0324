// 8-bit expert weights: quantisation to e4m3 codes with per-column scales,
// and dequantisation.
//
// [P4] long-context page (2kiu.com/news/5130654) section 3: expert weights
//      kept in 8 bits and turned back into 16-bit floats with a scale that
//      is computed per expert and per dimension (one global scale loses
//      accuracy).  [P1] section 5.2 and [P5] section 5.1: low-bit expert
//      weights for inference.
//
// Format (OCP float8 e4m3: sign, 4 exponent bits with bias 7, 3 mantissa
// bits, largest finite 448, subnormals m * 2^-9): for W [E, K, N] (bf16),
//   scale[e, n] = max_k |W[e, k, n]| / 448   (1 for an all-zero column)
//   code[e, n, k] = e4m3 nearest to W[e, k, n] / scale[e, n] (ties to the
//                   even code; the quotient never exceeds 448 by more than
//                   rounding, which saturates to 448)
// with the fp32 division correctly rounded.  Codes are stored transposed,
// each output column's K codes contiguous, which is the layout the expert
// products read.
#include "moe_common.h"

namespace {

using namespace moe;

// |W| column maxima: one thread per column, rows read in order (coalesced
// across the threads of a block).
__global__ __launch_bounds__(256) void absmax_kernel(const uint16_t* __restrict__ w, int K, int N,
                                                     float* __restrict__ scale) {
    const int e = blockIdx.y;
    const int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    const uint16_t* p = w + (size_t)e * K * N + n;
    float m = 0.f;
    int k = 0;
    for (; k + 8 <= K; k += 8) {  // eight loads in flight
        uint16_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = p[(size_t)(k + u) * N];
#pragma unroll
        for (int u = 0; u < 8; ++u) m = fmaxf(m, fabsf(bf2f(v[u])));
    }
    for (; k < K; ++k) m = fmaxf(m, fabsf(bf2f(p[(size_t)k * N])));
    scale[(size_t)e * N + n] = m > 0.f ? m / 448.0f : 1.0f;
}

// Nearest e4m3 code of a float32 value, ties to the even code; magnitudes
// of 448 and above give 448; NaN gives the NaN code.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = fabsf(v);
    if (a != a) return sign | 0x7Fu;
    if (a >= 448.0f) return sign | 0x7Eu;
    if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9 (code m = value * 2^9)
        return sign | (uint32_t)__builtin_rintf(a * 512.0f);  // rint: ties to even
    }
    // normal: exponent e in [-6, 8], 3 of the 23 mantissa bits kept with
    // round-to-nearest-even on the bit pattern (a carry moves to the exponent)
    const uint32_t ua = __float_as_uint(a);
    const uint32_t ex = (ua >> 23) - 127u + 7u;               // biased e4m3 exponent, 1..15
    const uint32_t m23 = ua & 0x7FFFFFu;
    const uint32_t m3 = (m23 + 0x7FFFFu + ((m23 >> 20) & 1u)) >> 20;  // 0..8
    uint32_t c = (ex << 3) + m3;
    if (c > 0x7Eu) c = 0x7Eu;
    return sign | c;
}

// Codes of a 64 (k) x 64 (n) block: read W rows (n-contiguous), code each
// value with its column's scale, transpose through LDS and write 64 code
// rows of 64 bytes (k-contiguous).
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ w,
                                                       const float* __restrict__ scale, int K,
                                                       int N, uint8_t* __restrict__ q) {
    __shared__ uint32_t tile[64][17];  // [n][k/4], 4 codes per word, padded
    const int e = blockIdx.z;
    const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;  // column tx, rows 4*ty.. step 16
    const int n = n0 + tx;
    const float s = n < N ? scale[(size_t)e * N + n] : 1.f;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        // rows k0 + 16*r4 + 4*ty .. +3: one packed word of 4 consecutive k
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int k = k0 + 16 * r4 + 4 * ty + b;
            uint32_t c = 0;
            if (k < K && n < N) c = e4m3_rne(bf2f(w[((size_t)e * K + k) * N + n]) / s);
            word |= c << (8 * b);
        }
        tile[tx][4 * r4 + ty] = word;
    }
    __syncthreads();
    // write: thread -> code row (column n0 + row), 16 bytes = k words 4*c4 ..
    const int row = threadIdx.x / 4, c4 = threadIdx.x % 4;
    const int nn = n0 + row;
    if (nn >= N) return;
    const int kk = k0 + 16 * c4;
    uint4 v = make_uint4(tile[row][4 * c4], tile[row][4 * c4 + 1], tile[row][4 * c4 + 2],
                         tile[row][4 * c4 + 3]);
    uint8_t* dst = q + ((size_t)e * N + nn) * K + kk;
    if (kk + 16 <= K) {
        *reinterpret_cast<uint4*>(dst) = v;
    } else {
        const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
        for (int b = 0; kk + b < K; ++b) dst[b] = (uint8_t)(ws[b / 4] >> (8 * (b % 4)));
    }
}

// W [E, K, N] fp32 = decode(code[e, n, k]) * scale[e, n], the decode by the
// same conversion the expert products use (e4m3 -> bf16 is exact), the
// product rounded once to fp32.
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ q,
                                                         const float* __restrict__ scale, int K,
                                                         int N, float* __restrict__ w) {
    __shared__ float tile[64][65];  // [k][n]
    const int e = blockIdx.z;
    const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    // read: thread -> code row n0 + row, 16 codes from k0 + 16*c4
    {
        const int row = threadIdx.x / 4, c4 = threadIdx.x % 4;
        const int n = n0 + row;
        const int kk = k0 + 16 * c4;
        uint32_t ws[4] = {0u, 0u, 0u, 0u};
        if (n < N) {
            const uint8_t* src = q + ((size_t)e * N + n) * K + kk;
            if (kk + 16 <= K) {
                const uint4 v = *reinterpret_cast<const uint4*>(src);
                ws[0] = v.x; ws[1] = v.y; ws[2] = v.z; ws[3] = v.w;
            } else {
                for (int b = 0; kk + b < K; ++b) ws[b / 4] |= (uint32_t)src[b] << (8 * (b % 4));
            }
        }
        const float s = n < N ? scale[(size_t)e * N + n] : 0.f;
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
            const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ws[wi], 1.0f, false));
            const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ws[wi], 1.0f, true));
            tile[16 * c4 + 4 * wi + 0][row] = bf_lo(lo) * s;
            tile[16 * c4 + 4 * wi + 1][row] = bf_hi(lo) * s;
            tile[16 * c4 + 4 * wi + 2][row] = bf_lo(hi) * s;
            tile[16 * c4 + 4 * wi + 3][row] = bf_hi(hi) * s;
        }
    }
    __syncthreads();
    const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
    const int n = n0 + tx;
    if (n >= N) return;
    for (int r = ty; r < 64; r += 4) {
        const int k = k0 + r;
        if (k < K) w[((size_t)e * K + k) * N + n] = tile[r][tx];
    }
}

}  // namespace

extern "C" moe_status_t moe_quantize_fp8(void* stream, const void* w, int E, int64_t K, int64_t N,
                                         uint8_t* q, float* scale) {
    if (E < 0 || K < 0 || N < 0) return MOE_ERR_SHAPE;
    if (E > 65535 || K >= ((int64_t)1 << 22) || N >= ((int64_t)1 << 30) ||
        (int64_t)E * K * N >= ((int64_t)1 << 40))
        return MOE_ERR_UNSUPPORTED;
    if (E == 0 || K == 0 || N == 0) return MOE_OK;
    if (!w || !q || !scale) return MOE_ERR_NULL;
    if (K % 16 || !moe_aligned16(q)) return MOE_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(absmax_kernel, dim3((unsigned)((N + 255) / 256), (unsigned)E), dim3(256), 0,
                       st, static_cast<const uint16_t*>(w), (int)K, (int)N, scale);
    MOE_CHECK_LAUNCH();
    hipLaunchKernelGGL(quantize_kernel,
                       dim3((unsigned)((N + 63) / 64), (unsigned)((K + 63) / 64), (unsigned)E),
                       dim3(256), 0, st, static_cast<const uint16_t*>(w), scale, (int)K, (int)N, q);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

extern "C" moe_status_t moe_dequantize_fp8(void* stream, const uint8_t* q, const float* scale,
                                           int E, int64_t K, int64_t N, float* w) {
    if (E < 0 || K < 0 || N < 0) return MOE_ERR_SHAPE;
    if (E > 65535 || K >= ((int64_t)1 << 22) || N >= ((int64_t)1 << 30) ||
        (int64_t)E * K * N >= ((int64_t)1 << 40))
        return MOE_ERR_UNSUPPORTED;
    if (E == 0 || K == 0 || N == 0) return MOE_OK;
    if (!w || !q || !scale) return MOE_ERR_NULL;
    if (K % 16 || !moe_aligned16(q)) return MOE_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(dequantize_kernel,
                       dim3((unsigned)((N + 63) / 64), (unsigned)((K + 63) / 64), (unsigned)E),
                       dim3(256), 0, st, q, scale, (int)K, (int)N, w);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}
