// Weighted combine of each token's expert outputs back to token order.
//
// [P1] LLaMA4-MoE guide (dpshk.com/news/5809432) section 2.4 and [P2] MoE
//      basics page (dpshk.com/news/6005940) section 3.1: a token's output is
//      the weighted sum of the outputs of its selected experts.  A dropped
//      copy (slot < 0) contributes nothing and the remaining weights are
//      not renormalised.
//
// [P1] section 5.2 adds shared experts that every token passes through; their
//      output (one fp32 row per token, computed like a routed expert over all
//      tokens) is the optional addend the sum starts from.
//
// Bandwidth-bound gather: each workgroup owns a few tokens; each lane owns
// 8 columns of the row, reads them from the k fp32 expert rows through
// slot[], accumulates in fp32 and writes the row once (bf16 output is
// rounded once, to nearest-even).
#include "moe_common.h"
#include "internal.h"

namespace {

using namespace moe;

constexpr int kCThreads = 256;
constexpr int kCTok = 4;

// Each lane owns 8 consecutive columns: two 16-byte fp32 reads per expert
// row, one 16-byte bf16 store (or two fp32 stores) per output row.
template <bool BF16_OUT>
__global__ __launch_bounds__(kCThreads) void combine_kernel(const float4* __restrict__ yd,
                                                           const int32_t* __restrict__ slot,
                                                           const float* __restrict__ w,
                                                           const float4* __restrict__ yadd, int64_t T,
                                                           int k, int row_oct, void* __restrict__ y) {
    __shared__ int s_slot[kCTok * MOE_MAX_TOPK];
    __shared__ float s_w[kCTok * MOE_MAX_TOPK];
    const int64_t t0 = (int64_t)blockIdx.x * kCTok;
    int nt = kCTok;
    if (t0 + nt > T) nt = (int)(T - t0);
    for (int q = threadIdx.x; q < nt * k; q += kCThreads) {
        s_slot[q] = slot[t0 * k + q];
        s_w[q] = w ? w[t0 * k + q] : 1.0f;  // no weights: the plain sum (dispatch backward)
    }
    __syncthreads();
    for (int v = threadIdx.x; v < row_oct; v += kCThreads) {
        float4 a0[kCTok], a1[kCTok];
#pragma unroll
        for (int i = 0; i < kCTok; ++i) {  // the sum starts from the addend row (or zero)
            if (yadd && i < nt) {
                a0[i] = yadd[((t0 + i) * row_oct + v) * 2];
                a1[i] = yadd[((t0 + i) * row_oct + v) * 2 + 1];
            } else {
                a0[i] = a1[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        for (int j = 0; j < k; ++j) {
            float4 q0[kCTok], q1[kCTok];
#pragma unroll
            for (int i = 0; i < kCTok; ++i) {  // the row loads of all tokens are in flight together
                const int s = i < nt ? s_slot[i * k + j] : -1;
                if (s >= 0) {
                    q0[i] = yd[((int64_t)s * row_oct + v) * 2];
                    q1[i] = yd[((int64_t)s * row_oct + v) * 2 + 1];
                } else {
                    q0[i] = q1[i] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
#pragma unroll
            for (int i = 0; i < kCTok; ++i) {
                const float wj = i < nt ? s_w[i * k + j] : 0.f;
                a0[i].x = fmaf(wj, q0[i].x, a0[i].x);
                a0[i].y = fmaf(wj, q0[i].y, a0[i].y);
                a0[i].z = fmaf(wj, q0[i].z, a0[i].z);
                a0[i].w = fmaf(wj, q0[i].w, a0[i].w);
                a1[i].x = fmaf(wj, q1[i].x, a1[i].x);
                a1[i].y = fmaf(wj, q1[i].y, a1[i].y);
                a1[i].z = fmaf(wj, q1[i].z, a1[i].z);
                a1[i].w = fmaf(wj, q1[i].w, a1[i].w);
            }
        }
#pragma unroll
        for (int i = 0; i < kCTok; ++i) {
            if (i >= nt) break;
            const int64_t t = t0 + i;
            if (BF16_OUT) {
                static_cast<uint4*>(y)[t * row_oct + v] =
                    make_uint4(pack_bf2(a0[i].x, a0[i].y), pack_bf2(a0[i].z, a0[i].w),
                               pack_bf2(a1[i].x, a1[i].y), pack_bf2(a1[i].z, a1[i].w));
            } else {
                float4* yo = static_cast<float4*>(y) + (t * row_oct + v) * 2;
                yo[0] = a0[i];
                yo[1] = a1[i];
            }
        }
    }
}

// Tokens none of whose copies was kept: their output row is the sum above
// over no expert rows (the addend row, or zero, with w_j * 0 added for each
// j), rounded once to bf16.  The down product with the combine fused writes
// every other token's row.  One thread per token finds the tokens; each
// wave then writes its tokens' rows with all its lanes.
__global__ __launch_bounds__(256) void combine_empty_kernel(const int32_t* __restrict__ slot,
                                                            const float* __restrict__ w,
                                                            const float4* __restrict__ yadd,
                                                            int64_t T, int k, int row_oct,
                                                            uint4* __restrict__ y) {
    const int lane = threadIdx.x % kWave;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    bool empty = t < T;
    for (int j = 0; empty && j < k; ++j)
        if (slot[t * k + j] >= 0) empty = false;
    uint64_t m = __ballot(empty);
    const int64_t tw = t - lane;  // the wave's first token
    while (m) {
        const int64_t tt = tw + __builtin_ctzll(m);
        m &= m - 1;
        for (int v = lane; v < row_oct; v += kWave) {
            float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
            if (yadd) {
                a0 = yadd[(tt * row_oct + v) * 2];
                a1 = yadd[(tt * row_oct + v) * 2 + 1];
            }
            for (int j = 0; j < k; ++j) {
                const float wj = w[tt * k + j];
                a0.x = fmaf(wj, 0.f, a0.x);
                a0.y = fmaf(wj, 0.f, a0.y);
                a0.z = fmaf(wj, 0.f, a0.z);
                a0.w = fmaf(wj, 0.f, a0.w);
                a1.x = fmaf(wj, 0.f, a1.x);
                a1.y = fmaf(wj, 0.f, a1.y);
                a1.z = fmaf(wj, 0.f, a1.z);
                a1.w = fmaf(wj, 0.f, a1.w);
            }
            y[tt * row_oct + v] = make_uint4(pack_bf2(a0.x, a0.y), pack_bf2(a0.z, a0.w),
                                             pack_bf2(a1.x, a1.y), pack_bf2(a1.z, a1.w));
        }
    }
}

}  // namespace

moe_status_t moe_combine_empty(hipStream_t st, const int32_t* slot, const float* topk_w, int64_t T,
                               int64_t H, int k, const float* y_shared, void* y) {
    if (T == 0) return MOE_OK;
    const int64_t grid = (T + 255) / 256;
    hipLaunchKernelGGL(combine_empty_kernel, dim3((unsigned)grid), dim3(256), 0, st, slot, topk_w,
                       reinterpret_cast<const float4*>(y_shared), T, k, (int)(H / 8),
                       static_cast<uint4*>(y));
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

extern "C" moe_status_t moe_combine(void* stream, moe_dtype_t dtype, const void* y_disp,
                                    const int32_t* slot, const float* topk_w, int64_t T, int64_t H,
                                    int k, const float* y_shared, void* y) {
    if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (T < 0 || H <= 0 || k < 1) return MOE_ERR_SHAPE;
    if (k > MOE_MAX_TOPK || H > (1 << 22) || T * k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (H % 8) return MOE_ERR_ALIGN;
    if (T == 0) return MOE_OK;
    if (!y_disp || !slot || !topk_w || !y) return MOE_ERR_NULL;
    if (!moe_aligned16(y_disp)) return MOE_ERR_ALIGN;
    if (!moe_aligned16(y) || (y_shared && !moe_aligned16(y_shared))) return MOE_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int row_oct = (int)(H / 8);
    const int64_t grid = (T + kCTok - 1) / kCTok;
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)grid), dim3(kCThreads), 0, st,
                           static_cast<const float4*>(y_disp), slot, topk_w,
                           reinterpret_cast<const float4*>(y_shared), T, k, row_oct, y);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)grid), dim3(kCThreads), 0, st,
                           static_cast<const float4*>(y_disp), slot, topk_w,
                           reinterpret_cast<const float4*>(y_shared), T, k, row_oct, y);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

// Backward of the row copy: a token's gradient is the sum of the gradients
// of its kept copies (the combine's gather with unit weights), fp32, plus
// the optional addend row (the shared experts' input gradient).
extern "C" moe_status_t moe_dispatch_bwd(void* stream, const float* dx_disp, const int32_t* slot,
                                         int64_t T, int64_t H, int k, const float* dx_add,
                                         float* dx) {
    if (T < 0 || H <= 0 || k < 1) return MOE_ERR_SHAPE;
    if (k > MOE_MAX_TOPK || H > (1 << 22) || T * k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (H % 8) return MOE_ERR_ALIGN;
    if (T == 0) return MOE_OK;
    if (!dx_disp || !slot || !dx) return MOE_ERR_NULL;
    if (!moe_aligned16(dx_disp) || !moe_aligned16(dx) ||
        (dx_add && !moe_aligned16(dx_add)))
        return MOE_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t grid = (T + kCTok - 1) / kCTok;
    hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)grid), dim3(kCThreads), 0, st,
                       reinterpret_cast<const float4*>(dx_disp), slot, (const float*)nullptr,
                       reinterpret_cast<const float4*>(dx_add), T, k, (int)(H / 8),
                       static_cast<void*>(dx));
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}
