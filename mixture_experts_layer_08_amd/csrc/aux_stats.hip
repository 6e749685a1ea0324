// Load-balancing statistics f_i, p_i and L_aux = alpha * E * sum f_i p_i.
//
// [P2] MoE basics page (dpshk.com/news/6005940) section 2.3: f_i is the
//      fraction of assignments sent to expert i, p_i the mean router
//      probability, L_aux = alpha * N * sum_i f_i p_i (worked example: 7 of
//      8 tokens to one expert gives f = 0.875); section 3.1 counts the
//      flattened top-k indices and divides by their number (T * k).
// [P1] LLaMA4-MoE guide (dpshk.com/news/5809432) section 3.2: the same loss.
//
// Up to 65536 probabilities (T * E) one workgroup of 1024 threads counts with
// LDS integer atomics (order-independent) and sums probability columns in a
// fixed order; above that, the one-pass dispatch kernel without its maps
// (dispatch.hip): blocks sum their tokens' columns, the last block to finish
// adds the block sums in block order.  Both bitwise reproducible.
#include "moe_common.h"

namespace {

constexpr int kAuxSmallThreads = 1024;

__global__ __launch_bounds__(kAuxSmallThreads) void aux_small_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ probs, int64_t T, int E, int k,
    float alpha, int32_t* counts, float* f, float* p, float* l_aux) {
    __shared__ int cnt[MOE_MAX_EXPERTS];
    __shared__ double colsum[kAuxSmallThreads];
    __shared__ double fp[MOE_MAX_EXPERTS];
    const int tid = threadIdx.x;
    if (tid < E) cnt[tid] = 0;
    __syncthreads();
    for (int64_t a0 = tid; a0 < T * k; a0 += 8 * kAuxSmallThreads) {
        int ids[8];  // eight loads in flight
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t a = a0 + (int64_t)u * kAuxSmallThreads;
            ids[u] = a < T * k ? idx[a] : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if ((unsigned)ids[u] < (unsigned)E) atomicAdd(&cnt[ids[u]], 1);
    }
    const int rows = kAuxSmallThreads / E;
    const int r = tid / E, e = tid % E;
    float s = 0.f;
    if (r < rows) {
        // sixteen loads in flight, summed in token order
        for (int64_t t0 = r; t0 < T; t0 += 16 * (int64_t)rows) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int64_t t = t0 + (int64_t)u * rows;
                v[u] = t < T ? probs[t * E + e] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) s += v[u];
        }
    }
    colsum[tid] = (r < rows) ? (double)s : 0.0;
    __syncthreads();
    if (tid < E) {
        double acc = 0.0;
        for (int rr = 0; rr < rows; ++rr) acc += colsum[rr * E + tid];
        const double fe = (double)cnt[tid] / ((double)T * k);
        const double pe = acc / (double)T;
        counts[tid] = cnt[tid];
        f[tid] = (float)fe;
        p[tid] = (float)pe;
        fp[tid] = fe * pe;
    }
    __syncthreads();
    if (tid == 0) {
        double acc = 0.0;
        for (int i = 0; i < E; ++i) acc += fp[i];
        *l_aux = (float)((double)alpha * E * acc);
    }
}

}  // namespace

size_t moe_dispatch_ws_bytes(int64_t T, int E, int k);
moe_status_t moe_stats_onepass(void* stream, const int32_t* idx, const float* probs, int64_t T,
                               int E, int k, float alpha, int32_t* counts, float* f, float* p,
                               float* l_aux, void* ws);

extern "C" moe_status_t moe_aux_stats(void* stream, const int32_t* topk_idx, const float* probs,
                                      int64_t T, int E, int k, float alpha, int32_t* counts,
                                      float* f, float* p, float* l_aux, void* ws,
                                      size_t ws_bytes) {
    if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
    if (T >= ((int64_t)1 << 31) / MOE_MAX_TOPK || T * E >= ((int64_t)1 << 31))
        return MOE_ERR_UNSUPPORTED;
    if (!counts || !f || !p || !l_aux) return MOE_ERR_NULL;
    if (T > 0 && (!topk_idx || !probs)) return MOE_ERR_NULL;
    if (T > 0 && (!ws || ws_bytes < moe_dispatch_ws_bytes(T, E, k))) return MOE_ERR_WORKSPACE;
    if (ws && !moe_aligned16(ws)) return MOE_ERR_ALIGN;
    if (T > 0 && T * E <= 65536) {
        hipLaunchKernelGGL(aux_small_kernel, dim3(1), dim3(kAuxSmallThreads), 0,
                           static_cast<hipStream_t>(stream), topk_idx, probs, T, E, k, alpha,
                           counts, f, p, l_aux);
        MOE_CHECK_LAUNCH();
        return MOE_OK;
    }
    return moe_stats_onepass(stream, topk_idx, probs, T, E, k, alpha, counts, f, p, l_aux, ws);
}
