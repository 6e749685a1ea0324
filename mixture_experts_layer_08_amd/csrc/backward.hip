// Backward of the combine and of the router.
//
// Combine ([P1] LLaMA4-MoE guide, dpshk.com/news/5809432, section 2.4):
// y_t = sum_j w_tj Y[slot_tj] gives, for each kept copy,
//   dY[slot_tj] = w_tj dy_t   and   dw_tj = <dy_t, Y[slot_tj]>,
// and dw_tj = 0 for a dropped copy.
//
// Router ([P5] llama-moe essay, coreui.cn/article/2610641, section 3.1: top-k
// of the softmax, renormalised; [P2] MoE basics page, dpshk.com/news/6005940,
// section 2.3: L_aux = alpha E sum_i f_i P_i with P_i the mean router
// probability; [P4] long-context page, 2kiu.com/news/5130654, section 2:
// Gumbel hard top-k whose soft path q = softmax((l + g) / tau) carries the
// gradient):
//   dp_sel_j = (dw_j - sum_i dw_i w_i) / sum_i p_sel_i      (renormalisation)
//   dp_te   += dl_aux alpha E f_e / T                      (aux statistics;
//                                                            f is a count)
//   dl       = p * (dp - <dp, p>)          (softmax; times 1 / tau for Gumbel)
//   dx      += dl W_r^T,  dW_r = x^T dl,  db_r = sum_t dl
// The top-k choice itself is piecewise constant and passes no gradient.
// Every sum runs in a fixed order, so results are bitwise reproducible.
#include "moe_common.h"

namespace {

using namespace moe;

// --------------------------------------------------------------- combine ----
// One wave per (token, slot) assignment; each lane handles 8 columns per
// step; the dot product is reduced across the wave in a fixed tree order.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const void* __restrict__ dy, const float4* __restrict__ yd, const int32_t* __restrict__ slot,
    const float* __restrict__ w, int64_t A, int k, int row_oct, void* __restrict__ dyd,
    float* __restrict__ dw) {
    const int64_t a = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    if (a >= A) return;
    const int64_t t = a / k;
    const int s = slot[a];
    if (s < 0) {
        if (lane == 0) dw[a] = 0.f;
        return;
    }
    const float wa = w[a];
    float dot = 0.f;
    for (int v = lane; v < row_oct; v += 64) {
        float g[8];
        if (BF16) {
            const uint4 q = static_cast<const uint4*>(dy)[t * row_oct + v];
            g[0] = bf_lo(q.x); g[1] = bf_hi(q.x); g[2] = bf_lo(q.y); g[3] = bf_hi(q.y);
            g[4] = bf_lo(q.z); g[5] = bf_hi(q.z); g[6] = bf_lo(q.w); g[7] = bf_hi(q.w);
        } else {
            const float4 q0 = static_cast<const float4*>(dy)[(t * row_oct + v) * 2];
            const float4 q1 = static_cast<const float4*>(dy)[(t * row_oct + v) * 2 + 1];
            g[0] = q0.x; g[1] = q0.y; g[2] = q0.z; g[3] = q0.w;
            g[4] = q1.x; g[5] = q1.y; g[6] = q1.z; g[7] = q1.w;
        }
        const float4 y0 = yd[((int64_t)s * row_oct + v) * 2];
        const float4 y1 = yd[((int64_t)s * row_oct + v) * 2 + 1];
        dot = fmaf(g[0], y0.x, dot); dot = fmaf(g[1], y0.y, dot);
        dot = fmaf(g[2], y0.z, dot); dot = fmaf(g[3], y0.w, dot);
        dot = fmaf(g[4], y1.x, dot); dot = fmaf(g[5], y1.y, dot);
        dot = fmaf(g[6], y1.z, dot); dot = fmaf(g[7], y1.w, dot);
        if (BF16) {
            static_cast<uint4*>(dyd)[(int64_t)s * row_oct + v] =
                make_uint4(pack_bf2(wa * g[0], wa * g[1]), pack_bf2(wa * g[2], wa * g[3]),
                           pack_bf2(wa * g[4], wa * g[5]), pack_bf2(wa * g[6], wa * g[7]));
        } else {
            float4* o = static_cast<float4*>(dyd) + ((int64_t)s * row_oct + v) * 2;
            o[0] = make_float4(wa * g[0], wa * g[1], wa * g[2], wa * g[3]);
            o[1] = make_float4(wa * g[4], wa * g[5], wa * g[6], wa * g[7]);
        }
    }
    dot = group_sum(dot, 64);
    if (lane == 0) dw[a] = dot;
}

// ---------------------------------------------------------------- router ----
struct RouteBwdParams {
    const float* probs;      // [T, E] p, or q in Gumbel mode
    const int32_t* idx;      // [T, k]
    const float* w;          // [T, k]
    const float* dw;         // [T, k]
    const float* f;          // [E]
    float aux_scale;         // dl_aux * alpha * E / T
    float inv_tau;           // 1, or 1 / tau in Gumbel mode
    int64_t T;
    int E, k;
    float* dl;               // [T, E]
};

// One wave per token, lane e holding expert e (E <= 64); the two sums over
// experts reduce across the wave in a fixed tree order.
__global__ __launch_bounds__(256) void route_bwd_logits_kernel(RouteBwdParams p) {
    const int64_t t = (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
    const int e = threadIdx.x % 64;
    if (t >= p.T) return;
    const int E = p.E, k = p.k;
    const bool live = e < E;
    const float pe = live ? p.probs[t * E + e] : 0.f;
    // S = sum of the selected probabilities, dot = sum_j dw_j w_j (k <= 8 terms,
    // read by every lane in the same order)
    float S = 0.f, dot = 0.f;
    for (int j = 0; j < k; ++j) {
        const int ej = p.idx[t * k + j];
        S += p.probs[t * E + ej];
        dot = fmaf(p.dw[t * k + j], p.w[t * k + j], dot);
    }
    float dpe = live ? p.aux_scale * p.f[e] : 0.f;  // aux statistics' term
    for (int j = 0; j < k; ++j)                       // renormalisation's term
        if (p.idx[t * k + j] == e) dpe += (p.dw[t * k + j] - dot) / S;
    const float sd = group_sum(dpe * pe, 64);
    if (live) p.dl[t * E + e] = pe * (dpe - sd) * p.inv_tau;
}

// dx[t, h] += sum_e dl[t, e] * W_r[h, e].  A block takes 8 tokens; a thread
// takes 8 consecutive columns, holds their W_r values for 8 experts at a
// time in registers and applies them to every token of the block (dl staged
// in LDS), so W_r is read once per 8 tokens.
constexpr int kDxTok = 8;
template <bool BF16>
__global__ __launch_bounds__(256) void route_bwd_dx_kernel(const float* __restrict__ dl,
                                                           const void* __restrict__ w_r,
                                                           int64_t T, int H, int E,
                                                           float* __restrict__ dx) {
    __shared__ float s_dl[kDxTok * MOE_MAX_EXPERTS];
    const int64_t t0 = (int64_t)blockIdx.x * kDxTok;
    int nt = kDxTok;
    if (t0 + nt > T) nt = (int)(T - t0);
    for (int q = threadIdx.x; q < nt * E; q += blockDim.x) s_dl[q] = dl[t0 * E + q];
    __syncthreads();
    for (int h0 = threadIdx.x * 8; h0 < H; h0 += blockDim.x * 8) {
        float acc[kDxTok][8];
#pragma unroll
        for (int i = 0; i < kDxTok; ++i)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[i][c] = 0.f;
        for (int e0 = 0; e0 < E; e0 += 8) {
            const int ne = E - e0 < 8 ? E - e0 : 8;
            float wv[8][8];
            if (ne == 8 && E % 8 == 0) {  // 8 experts of a W_r row: one or two 16-byte loads
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int64_t o = (int64_t)(h0 + c) * E + e0;
                    if (BF16) {
                        const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w_r) + o);
                        wv[c][0] = bf_lo(q.x); wv[c][1] = bf_hi(q.x); wv[c][2] = bf_lo(q.y); wv[c][3] = bf_hi(q.y);
                        wv[c][4] = bf_lo(q.z); wv[c][5] = bf_hi(q.z); wv[c][6] = bf_lo(q.w); wv[c][7] = bf_hi(q.w);
                    } else {
                        const float4 q0 = *reinterpret_cast<const float4*>(static_cast<const float*>(w_r) + o);
                        const float4 q1 = *reinterpret_cast<const float4*>(static_cast<const float*>(w_r) + o + 4);
                        wv[c][0] = q0.x; wv[c][1] = q0.y; wv[c][2] = q0.z; wv[c][3] = q0.w;
                        wv[c][4] = q1.x; wv[c][5] = q1.y; wv[c][6] = q1.z; wv[c][7] = q1.w;
                    }
                }
            } else {
#pragma unroll
                for (int c = 0; c < 8; ++c)
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int64_t o = (int64_t)(h0 + c) * E + e0 + u;
                        wv[c][u] = u < ne ? (BF16 ? bf2f(static_cast<const uint16_t*>(w_r)[o])
                                                  : static_cast<const float*>(w_r)[o])
                                          : 0.f;
                    }
            }
#pragma unroll
            for (int i = 0; i < kDxTok; ++i) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float d = (i < nt && u < ne) ? s_dl[i * E + e0 + u] : 0.f;
#pragma unroll
                    for (int c = 0; c < 8; ++c) acc[i][c] = fmaf(d, wv[c][u], acc[i][c]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kDxTok; ++i) {
            if (i >= nt) continue;
            float4* o = reinterpret_cast<float4*>(dx + (t0 + i) * H + h0);
            float4 v0 = o[0], v1 = o[1];
            v0.x += acc[i][0]; v0.y += acc[i][1]; v0.z += acc[i][2]; v0.w += acc[i][3];
            v1.x += acc[i][4]; v1.y += acc[i][5]; v1.z += acc[i][6]; v1.w += acc[i][7];
            o[0] = v0;
            o[1] = v1;
        }
    }
}

// Partial sums over token chunks: part[b][e][h] = sum_{t in chunk b} x[t, h]
// dl[t, e], and pb[b][e] = sum_{t in chunk b} dl[t, e] (first column block
// only).  One wave per block: lane l takes the 8 consecutive columns h0 =
// blockIdx.y * 512 + 8 l (one 16-byte load of x per token for bf16) and 8
// experts e0.., with dl of the chunk staged in LDS; tokens are summed in
// order, and the chunks in chunk order below.  A lane stores its 8 columns
// of one expert as two 16-byte stores (a wave: 2 KB contiguous).
constexpr int kWpCols = 512;  // columns per block
template <bool BF16>
__global__ __launch_bounds__(64) void route_bwd_wpart_kernel(const void* __restrict__ x,
                                                             const float* __restrict__ dl,
                                                             int64_t T, int H, int E, int tb,
                                                             float* __restrict__ part,
                                                             float* __restrict__ pb) {
    __shared__ float s_dl[64 * 8];
    const int lane = threadIdx.x;
    const int b = blockIdx.x;
    const int h0 = blockIdx.y * kWpCols + lane * 8;
    const int e0 = blockIdx.z * 8;
    const int ne = E - e0 < 8 ? E - e0 : 8;
    const bool live = h0 < H;  // H is a multiple of 8
    const int64_t t0 = (int64_t)b * tb;
    int64_t t1 = t0 + tb;
    if (t1 > T) t1 = T;
    float acc[8][8], accb[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        accb[c] = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[c][u] = 0.f;
    }
    for (int64_t tc = t0; tc < t1; tc += 64) {
        const int n = (int)(t1 - tc < 64 ? t1 - tc : 64);
        __syncthreads();
        for (int q = lane; q < n * 8; q += 64) {
            const int tt = q / 8, c = q % 8;
            s_dl[q] = c < ne ? dl[(tc + tt) * E + e0 + c] : 0.f;
        }
        __syncthreads();
        // x of 16 tokens in flight at once, then their FMAs in token order
        for (int g0 = 0; g0 < n; g0 += 16) {
            uint4 xq[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                xq[v] = make_uint4(0u, 0u, 0u, 0u);
                if (live && g0 + v < n) {
                    if (BF16) {
                        xq[v] = *reinterpret_cast<const uint4*>(
                            static_cast<const uint16_t*>(x) + (tc + g0 + v) * H + h0);
                    }
                }
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                if (g0 + v >= n) break;
                const int tt = g0 + v;
                float xv[8];
                if (BF16) {
                    const uint4 q = xq[v];
                    xv[0] = bf_lo(q.x); xv[1] = bf_hi(q.x); xv[2] = bf_lo(q.y); xv[3] = bf_hi(q.y);
                    xv[4] = bf_lo(q.z); xv[5] = bf_hi(q.z); xv[6] = bf_lo(q.w); xv[7] = bf_hi(q.w);
                } else if (live) {
                    const float* xr = static_cast<const float*>(x) + (tc + tt) * H + h0;
                    const float4 q0 = *reinterpret_cast<const float4*>(xr);
                    const float4 q1 = *reinterpret_cast<const float4*>(xr + 4);
                    xv[0] = q0.x; xv[1] = q0.y; xv[2] = q0.z; xv[3] = q0.w;
                    xv[4] = q1.x; xv[5] = q1.y; xv[6] = q1.z; xv[7] = q1.w;
                } else {
#pragma unroll
                    for (int c = 0; c < 8; ++c) xv[c] = 0.f;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float d = s_dl[tt * 8 + u];
                    accb[u] += d;
#pragma unroll
                    for (int c = 0; c < 8; ++c) acc[c][u] = fmaf(xv[c], d, acc[c][u]);
                }
            }
        }
    }
    if (live) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (u < ne) {
                float4* o = reinterpret_cast<float4*>(part + ((int64_t)b * E + e0 + u) * H + h0);
                o[0] = make_float4(acc[0][u], acc[1][u], acc[2][u], acc[3][u]);
                o[1] = make_float4(acc[4][u], acc[5][u], acc[6][u], acc[7][u]);
            }
    }
    if (blockIdx.y == 0 && lane == 0) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (u < ne) pb[(int64_t)b * E + e0 + u] = accb[u];
    }
}

__global__ __launch_bounds__(256) void route_bwd_wfinal_kernel(const float* __restrict__ part,
                                                               const float* __restrict__ pb,
                                                               int nb, int H, int E,
                                                               float* __restrict__ dw_r,
                                                               float* __restrict__ db_r) {
    // thread i: expert i / H, column i % H (the partials are [nb][E][H])
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < (int64_t)H * E) {
        float s = 0.f;
        int b = 0;
        for (; b + 8 <= nb; b += 8) {  // eight loads in flight, summed in chunk order
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(b + u) * H * E + i];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
        for (; b < nb; ++b) s += part[(int64_t)b * H * E + i];
        dw_r[(i % H) * E + i / H] = s;
    }
    if (db_r && i < E) {
        float s = 0.f;
        for (int b = 0; b < nb; ++b) s += pb[(int64_t)b * E + i];
        db_r[i] = s;
    }
}

// tokens per partial-sum chunk: at most 128 chunks, at least 32 tokens each
int route_chunk(int64_t T) {
    int64_t tb = (T + 127) / 128;
    if (tb < 32) tb = 32;
    return (int)tb;
}

}  // namespace

extern "C" moe_status_t moe_combine_bwd(void* stream, moe_dtype_t dtype, const void* dy,
                                        const void* y_disp, const int32_t* slot,
                                        const float* topk_w, int64_t T, int64_t H, int k,
                                        void* dy_disp, float* dw) {
    if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (T < 0 || H <= 0 || k < 1) return MOE_ERR_SHAPE;
    if (k > MOE_MAX_TOPK || H > (1 << 22) || T * k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (H % 8) return MOE_ERR_ALIGN;
    if (T == 0) return MOE_OK;
    if (!dy || !slot || !topk_w || !dw || !y_disp || !dy_disp) return MOE_ERR_NULL;
    if (!moe_aligned16(dy) || !moe_aligned16(y_disp) || !moe_aligned16(dy_disp)) return MOE_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t A = T * k;
    const unsigned grid = (unsigned)((A + 3) / 4);
    if (dtype == MOE_BF16)
        hipLaunchKernelGGL(combine_bwd_kernel<true>, dim3(grid), dim3(256), 0, st, dy,
                           static_cast<const float4*>(y_disp), slot, topk_w, A, k, (int)(H / 8),
                           dy_disp, dw);
    else
        hipLaunchKernelGGL(combine_bwd_kernel<false>, dim3(grid), dim3(256), 0, st, dy,
                           static_cast<const float4*>(y_disp), slot, topk_w, A, k, (int)(H / 8),
                           dy_disp, dw);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

extern "C" size_t moe_route_bwd_ws_bytes(int64_t T, int64_t H, int E) {
    if (T <= 0 || H <= 0 || E < 1) return 256;
    const int64_t nb = (T + route_chunk(T) - 1) / route_chunk(T);
    return (size_t)nb * (H + 1) * E * sizeof(float) + 256;
}

extern "C" moe_status_t moe_route_bwd(void* stream, moe_dtype_t dtype, moe_route_mode_t mode,
                                      const void* x, const void* w_r, const float* probs,
                                      const int32_t* topk_idx, const float* topk_w,
                                      const float* dw, const float* f, float alpha, float dl_aux,
                                      int64_t T, int64_t H, int E, int k, int64_t seq_len,
                                      float* dlogits, float* dx, float* dw_r, float* db_r,
                                      void* ws, size_t ws_bytes) {
    if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (mode != MOE_ROUTE_SOFTMAX_TOPK && mode != MOE_ROUTE_GUMBEL_HARD) return MOE_ERR_DTYPE;
    if (T < 0 || H <= 0 || E < 1 || k < 1 || k > E) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
    if (T * H >= ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
    if (H % 8) return MOE_ERR_ALIGN;
    if (mode == MOE_ROUTE_GUMBEL_HARD && seq_len < 0) return MOE_ERR_SHAPE;
    if (!dw_r || !w_r) return MOE_ERR_NULL;
    if (T > 0 && (!x || !probs || !topk_idx || !topk_w || !dw || !f || !dlogits)) return MOE_ERR_NULL;
    if (dx && !moe_aligned16(dx)) return MOE_ERR_ALIGN;
    if (T > 0 && (!moe_aligned16(x) || !moe_aligned16(w_r) || (ws && !moe_aligned16(ws))))
        return MOE_ERR_ALIGN;
    if (T > 0 && (!ws || ws_bytes < moe_route_bwd_ws_bytes(T, H, E))) return MOE_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool bf = dtype == MOE_BF16;
    if (T == 0) {  // no tokens: zero gradients (no kernel reads anything)
        hipLaunchKernelGGL(route_bwd_wfinal_kernel, dim3((unsigned)((H * E + 255) / 256)),
                           dim3(256), 0, st, (const float*)nullptr, (const float*)nullptr, 0,
                           (int)H, E, dw_r, db_r);
        MOE_CHECK_LAUNCH();
        return MOE_OK;
    }
    RouteBwdParams p;
    p.probs = probs;
    p.idx = topk_idx;
    p.w = topk_w;
    p.dw = dw;
    p.f = f;
    p.aux_scale = (float)((double)dl_aux * alpha * E / (double)T);
    p.inv_tau = mode == MOE_ROUTE_GUMBEL_HARD ? (float)(1.0 / (1.0 + 1e-4 * (double)seq_len)) : 1.0f;
    p.T = T;
    p.E = E;
    p.k = k;
    p.dl = dlogits;
    hipLaunchKernelGGL(route_bwd_logits_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, p);
    MOE_CHECK_LAUNCH();
    if (dx) {
        const unsigned g = (unsigned)((T + kDxTok - 1) / kDxTok);
        if (bf)
            hipLaunchKernelGGL(route_bwd_dx_kernel<true>, dim3(g), dim3(256), 0, st, dlogits, w_r, T,
                               (int)H, E, dx);
        else
            hipLaunchKernelGGL(route_bwd_dx_kernel<false>, dim3(g), dim3(256), 0, st, dlogits, w_r,
                               T, (int)H, E, dx);
        MOE_CHECK_LAUNCH();
    }
    const int tb = route_chunk(T);
    const int nb = (int)((T + tb - 1) / tb);
    float* part = static_cast<float*>(ws);
    float* pb = part + (size_t)nb * H * E;
    dim3 gw((unsigned)nb, (unsigned)((H + kWpCols - 1) / kWpCols), (unsigned)((E + 7) / 8));
    if (bf)
        hipLaunchKernelGGL(route_bwd_wpart_kernel<true>, gw, dim3(64), 0, st, x, dlogits, T, (int)H,
                           E, tb, part, pb);
    else
        hipLaunchKernelGGL(route_bwd_wpart_kernel<false>, gw, dim3(64), 0, st, x, dlogits, T,
                           (int)H, E, tb, part, pb);
    MOE_CHECK_LAUNCH();
    hipLaunchKernelGGL(route_bwd_wfinal_kernel, dim3((unsigned)((H * E + 255) / 256)), dim3(256), 0,
                       st, part, pb, nb, (int)H, E, dw_r, db_r);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}
