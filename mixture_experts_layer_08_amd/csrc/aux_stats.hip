// Load-balancing statistics f_i, p_i and L_aux = alpha * E * sum f_i p_i.
//
// [P2] MoE basics page (dpshk.com/news/6005940) section 2.3: f_i is the
//      fraction of assignments sent to expert i, p_i the mean router
//      probability, L_aux = alpha * N * sum_i f_i p_i (worked example: 7 of
//      8 tokens to one expert gives f = 0.875); section 3.1 counts the
//      flattened top-k indices and divides by their number (T * k).
// [P1] LLaMA4-MoE guide (dpshk.com/news/5809432) section 3.2: the same loss.
//
// Two launches (one workgroup for up to 65536 probabilities), both in a fixed
// order so results are bitwise reproducible:
//  1. each block takes a contiguous token range, sums probs columns (fp32
//     per thread, fp64 across threads) and counts expert ids with LDS
//     integer atomics (integer sums are order-independent);
//  2. one block adds the per-block partials in block order and finishes
//     f, p and L_aux in fp64.
#include "moe_common.h"

namespace {

constexpr int kAuxThreads = 256;
constexpr int kAuxTokPerBlock = 64;

__global__ __launch_bounds__(kAuxThreads) void aux_partial_kernel(const int32_t* __restrict__ idx,
                                                                 const float* __restrict__ probs,
                                                                 int64_t T, int E, int k,
                                                                 int32_t* __restrict__ ws_cnt,
                                                                 double* __restrict__ ws_sum) {
    __shared__ int cnt[MOE_MAX_EXPERTS];
    __shared__ double colsum[kAuxThreads];
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kAuxTokPerBlock;
    int64_t t1 = t0 + kAuxTokPerBlock;
    if (t1 > T) t1 = T;
    if (tid < E) cnt[tid] = 0;
    __syncthreads();
    for (int64_t a = t0 * k + tid; a < t1 * k; a += kAuxThreads) {
        const unsigned e = (unsigned)idx[a];
        if (e < (unsigned)E) atomicAdd(&cnt[e], 1);
    }
    // column sums: thread (r, e) with r < rows, e < E strides over tokens
    const int rows = kAuxThreads / E;
    const int r = tid / E, e = tid % E;
    float s = 0.f;
    if (r < rows)
        for (int64_t t = t0 + r; t < t1; t += rows) s += probs[t * E + e];
    colsum[tid] = (r < rows) ? (double)s : 0.0;
    __syncthreads();
    if (tid < E) {
        double acc = 0.0;
        for (int rr = 0; rr < rows; ++rr) acc += colsum[rr * E + tid];
        ws_sum[(size_t)blockIdx.x * E + tid] = acc;
        ws_cnt[(size_t)blockIdx.x * E + tid] = cnt[tid];
    }
}

__global__ __launch_bounds__(MOE_MAX_EXPERTS) void aux_final_kernel(
    const int32_t* __restrict__ ws_cnt, const double* __restrict__ ws_sum, int nblocks, int64_t T,
    int E, int k, float alpha, int32_t* counts, float* f, float* p, float* l_aux) {
    __shared__ double fp[MOE_MAX_EXPERTS];
    const int e = threadIdx.x;
    if (e < E) {
        int64_t c = 0;
        double s = 0.0;
        int b = 0;
        for (; b + 8 <= nblocks; b += 8) {  // eight independent loads in flight, summed in order
            int cc[8];
            double ss[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                cc[u] = ws_cnt[(size_t)(b + u) * E + e];
                ss[u] = ws_sum[(size_t)(b + u) * E + e];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                c += cc[u];
                s += ss[u];
            }
        }
        for (; b < nblocks; ++b) {
            c += ws_cnt[(size_t)b * E + e];
            s += ws_sum[(size_t)b * E + e];
        }
        const double fe = T > 0 ? (double)c / ((double)T * k) : 0.0;
        const double pe = T > 0 ? s / (double)T : 0.0;
        counts[e] = (int32_t)c;
        f[e] = (float)fe;
        p[e] = (float)pe;
        fp[e] = fe * pe;
    }
    __syncthreads();
    if (e == 0) {
        double acc = 0.0;
        for (int i = 0; i < E; ++i) acc += fp[i];
        *l_aux = (float)((double)alpha * E * acc);
    }
}

// Small inputs (T*E <= 65536 probabilities): everything in one workgroup.
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

int aux_blocks(int64_t T) { return (int)((T + kAuxTokPerBlock - 1) / kAuxTokPerBlock); }

}  // namespace

size_t moe_aux_ws_bytes(int64_t T, int E) {
    const int nb = aux_blocks(T);
    return (size_t)nb * E * (sizeof(int32_t) + sizeof(double)) + 256;
}

extern "C" moe_status_t moe_aux_stats(void* stream, const int32_t* topk_idx, const float* probs,
                                      int64_t T, int E, int k, float alpha, int32_t* counts,
                                      float* f, float* p, float* l_aux, void* ws,
                                      size_t ws_bytes) {
    if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
    if (T >= ((int64_t)1 << 31) / MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
    if (!counts || !f || !p || !l_aux) return MOE_ERR_NULL;
    if (T > 0 && (!topk_idx || !probs)) return MOE_ERR_NULL;
    const int nb = aux_blocks(T);
    if (nb > 0) {
        if (!ws) return MOE_ERR_WORKSPACE;
        if (ws_bytes < moe_aux_ws_bytes(T, E)) return MOE_ERR_WORKSPACE;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (T > 0 && T * E <= 65536) {
        hipLaunchKernelGGL(aux_small_kernel, dim3(1), dim3(kAuxSmallThreads), 0, st, topk_idx, probs,
                           T, E, k, alpha, counts, f, p, l_aux);
        MOE_CHECK_LAUNCH();
        return MOE_OK;
    }
    // workspace: [nb][E] double sums (8-byte aligned first), then [nb][E] int32 counts
    double* ws_sum = static_cast<double*>(ws);
    int32_t* ws_cnt = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + (size_t)nb * E * 8);
    if (nb > 0) {
        if ((reinterpret_cast<uintptr_t>(ws) & 7u) != 0) return MOE_ERR_ALIGN;
        hipLaunchKernelGGL(aux_partial_kernel, dim3(nb), dim3(kAuxThreads), 0, st, topk_idx, probs, T,
                           E, k, ws_cnt, ws_sum);
        MOE_CHECK_LAUNCH();
    }
    hipLaunchKernelGGL(aux_final_kernel, dim3(1), dim3(MOE_MAX_EXPERTS), 0, st, ws_cnt, ws_sum, nb, T,
                       E, k, alpha, counts, f, p, l_aux);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}
