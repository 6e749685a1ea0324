// Expert FFNs as a grouped GEMM over the dispatched rows.
//
// [P2] MoE basics page (dpshk.com/news/6005940) section 2.2: every expert is
//      a full FFN (SwiGLU, GELU, ... kept inside the expert); section 3.1:
//      the GELU expert is Linear(H, I) -> GELU -> Linear(I, H), both biased;
//      section 4.4: merge the tokens of one expert into one large matmul
//      instead of per-token calls.
// [P5] llama-moe essay (coreui.cn/article/2610641) section 2.1: LLaMA's
//      SwiGLU; section 6.3: fused MoE kernels instead of many small matmuls.
// [P3] Loop-MoE page (discosf.com/news/5228035) section 2.1: all experts'
//      weights as one [E, H, I] tensor (the layout taken here).
//
// Design (gfx950): one persistent kernel per product.  The tile list is
// rebuilt on the device from kept[e] (no host round trip): expert e has
// ceil(kept[e] / BM) row tiles times N / BN_out column tiles.  Workgroup b
// sits on XCD b % 8; in round r it takes tile r*G + (b % 8)*(G/8) + b/8, so
// each XCD works through a contiguous run of tiles; runs are ordered expert
// by expert, in groups that cover every row tile of an expert across a few
// column tiles, so the A rows and the B panels a group shares stay in that
// XCD's L2.
//
// Per tile: 4 waves (2 x 2), BK = 64, v_mfma_f32_16x16x32_bf16 with fp32
// accumulators.  A rows are k-contiguous already.  B = W[e] is n-contiguous
// ([K, N] row-major), but an MFMA B operand wants 8 consecutive k per lane,
// so each thread loads an 8 (k) x 8 (n) block as eight 16-byte vectors and
// transposes it in registers; LDS then holds B as [n][k].  LDS is double
// buffered (one barrier per k-step); the next k-step's global loads are in
// flight during the current step's MFMAs.  Epilogues run on the fp32
// accumulators in registers:
//   SwiGLU:  a tile holds matching gate and up columns (its B tile is half
//            W_gate, half W_up), so h = silu(g) * u needs no extra pass;
//   GELU:    h = gelu_erf(acc + b1);   second product: y = acc (+ b2).
// Results are rounded to bf16 and staged through LDS for full-row 16-byte
// stores.  Rows at or beyond kept[e] are read as zeros and never stored.
#include "moe_common.h"

#include <math.h>

namespace {

using namespace moe;

constexpr int kBK = 64;
constexpr int kLdsRow = kBK + 8;  // bf16 per LDS row: 144 bytes, keeps 16-byte alignment
constexpr int kGThreads = 256;

enum { MODE_SWIGLU = 0, MODE_GELU = 1, MODE_DOWN = 2 };

struct GemmArgs {
    const uint16_t* A;      // [E, C, K]
    const uint16_t* B0;     // [E, K, N] gate / W1 / W2
    const uint16_t* B1;     // [E, K, N] up (SwiGLU)
    const uint16_t* bias;   // [E, N] or null
    void* out;              // [E, C, N]: bf16 (first product) or fp32 (second)
    const int32_t* kept;    // [E]
    int E;
    int64_t C;
    int K;
    int N;                  // output columns
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }
__device__ __forceinline__ float gelu_f(float z) {
    return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

// 8x8 bf16 transpose: r[i] holds row i (8 values, 2 per word); returns the
// column j as 8 values (k = 0..7).
__device__ __forceinline__ uint4 transpose_col(const uint4 (&r)[8], int j) {
    uint32_t o[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t* a = reinterpret_cast<const uint32_t*>(&r[2 * w]);
        const uint32_t* b = reinterpret_cast<const uint32_t*>(&r[2 * w + 1]);
        const uint32_t x = a[j >> 1], y = b[j >> 1];
        o[w] = (j & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

template <int BM, int BN, int MODE>
struct Tile {
    static constexpr int BN_OUT = (MODE == MODE_SWIGLU) ? BN / 2 : BN;
    static constexpr int WM = BM / 2, WN = BN / 2;          // per-wave tile
    static constexpr int TM = WM / 16, TN = WN / 16;        // MFMA tiles per wave
    static constexpr int A_VECS = BM * kBK / 8;             // 16-byte vectors per A tile
    static constexpr int A_PER_T = (A_VECS + kGThreads - 1) / kGThreads;
    static constexpr int B_UNITS = (kBK / 8) * (BN / 8);    // 8x8 blocks per B tile
    static constexpr int B_PER_T = (B_UNITS + kGThreads - 1) / kGThreads;
    static constexpr size_t LDS_STAGE = (size_t)(BM + BN) * kLdsRow * 2;
    // second product keeps fp32 outputs; the first rounds h to bf16
    static constexpr int OUT_BYTES = (MODE == MODE_DOWN) ? 4 : 2;
    static constexpr int OUT_PAD = 16 / OUT_BYTES;
    static constexpr size_t LDS_OUT = (size_t)BM * (BN_OUT + OUT_PAD) * OUT_BYTES;
    static constexpr size_t LDS = (2 * LDS_STAGE > LDS_OUT ? 2 * LDS_STAGE : LDS_OUT);
};

template <int BM, int BN, int MODE>
__global__ __launch_bounds__(kGThreads, 1) void grouped_gemm_kernel(GemmArgs g) {
    using TL = Tile<BM, BN, MODE>;
    constexpr int TM = TL::TM, TN = TL::TN;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_pref[MOE_MAX_EXPERTS + 1];
    __shared__ int s_mt[MOE_MAX_EXPERTS];

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int wm = wave / 2, wn = wave % 2;
    const int NT = g.N / TL::BN_OUT;
    if (tid == 0) {
        int cum = 0;
        for (int e = 0; e < g.E; ++e) {
            int kp = g.kept[e];
            if (kp < 0) kp = 0;
            if (kp > g.C) kp = (int)g.C;
            const int mt = (kp + BM - 1) / BM;
            s_mt[e] = mt;
            s_pref[e] = cum;
            cum += mt * NT;
        }
        s_pref[g.E] = cum;
    }
    __syncthreads();
    const int total = s_pref[g.E];
    const int G = gridDim.x;
    const int xcd = blockIdx.x % 8, slot8 = blockIdx.x / 8;

    uint16_t* As[2];
    uint16_t* Bs[2];
    As[0] = reinterpret_cast<uint16_t*>(smem);
    Bs[0] = As[0] + BM * kLdsRow;
    As[1] = Bs[0] + BN * kLdsRow;
    Bs[1] = As[1] + BM * kLdsRow;

    for (int round = 0;; ++round) {
        const int logical = round * G + xcd * (G / 8) + slot8;
        if (logical >= total) break;
        int e = 0;
        while (e + 1 < g.E && s_pref[e + 1] <= logical) ++e;
        const int local = logical - s_pref[e];
        const int mt = s_mt[e];
        int gn = 32 / mt;
        if (gn < 1) gn = 1;
        if (gn > NT) gn = NT;
        const int grp = local / (mt * gn);
        int width = NT - grp * gn;
        if (width > gn) width = gn;
        const int rem = local - grp * mt * gn;
        const int m_tile = rem / width;
        const int n_tile = grp * gn + rem % width;

        int kept = g.kept[e];
        if (kept > g.C) kept = (int)g.C;
        const int m0 = m_tile * BM;
        const int n0 = n_tile * TL::BN_OUT;  // output column base
        const uint16_t* Ab = g.A + ((size_t)e * g.C + m0) * g.K;
        const uint16_t* B0b = g.B0 + (size_t)e * g.K * g.N;
        const uint16_t* B1b = (MODE == MODE_SWIGLU) ? g.B1 + (size_t)e * g.K * g.N : nullptr;

        uint4 ra[TL::A_PER_T];
        uint4 rb[TL::B_PER_T][8];

        auto load_global = [&](int k0) {
#pragma unroll
            for (int i = 0; i < TL::A_PER_T; ++i) {
                const int v = tid + i * kGThreads;
                if (v < TL::A_VECS) {
                    const int row = v / (kBK / 8), kc = v % (kBK / 8);
                    if (m0 + row < kept)
                        ra[i] = *reinterpret_cast<const uint4*>(Ab + (size_t)row * g.K + k0 + kc * 8);
                    else
                        ra[i] = make_uint4(0, 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < TL::B_PER_T; ++i) {
                const int u = tid + i * kGThreads;
                if (u < TL::B_UNITS) {
                    const int kb = u / (BN / 8), nb = u % (BN / 8);
                    const uint16_t* src;
                    if (MODE == MODE_SWIGLU) {
                        const int half = BN / 16;  // 8-column groups per half
                        src = (nb < half) ? B0b + n0 + nb * 8 : B1b + n0 + (nb - half) * 8;
                    } else {
                        src = B0b + n0 + nb * 8;
                    }
                    src += (size_t)(k0 + kb * 8) * g.N;
#pragma unroll
                    for (int r = 0; r < 8; ++r)
                        rb[i][r] = *reinterpret_cast<const uint4*>(src + (size_t)r * g.N);
                }
            }
        };
        auto store_lds = [&](int buf) {
            uint16_t* as = As[buf];
            uint16_t* bs = Bs[buf];
#pragma unroll
            for (int i = 0; i < TL::A_PER_T; ++i) {
                const int v = tid + i * kGThreads;
                if (v < TL::A_VECS) {
                    const int row = v / (kBK / 8), kc = v % (kBK / 8);
                    *reinterpret_cast<uint4*>(as + row * kLdsRow + kc * 8) = ra[i];
                }
            }
#pragma unroll
            for (int i = 0; i < TL::B_PER_T; ++i) {
                const int u = tid + i * kGThreads;
                if (u < TL::B_UNITS) {
                    const int kb = u / (BN / 8), nb = u % (BN / 8);
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        *reinterpret_cast<uint4*>(bs + (nb * 8 + j) * kLdsRow + kb * 8) =
                            transpose_col(rb[i], j);
                }
            }
        };

        f32x4_t acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // B column (LDS row) of this wave's n-tile j
        auto bcol = [&](int j) {
            if (MODE == MODE_SWIGLU) {
                constexpr int q = BN / 4;  // columns per wave per half
                return (j < TN / 2) ? wn * q + j * 16 : BN / 2 + wn * q + (j - TN / 2) * 16;
            }
            return wn * (BN / 2) + j * 16;
        };

        const int nk = g.K / kBK;
        load_global(0);
        store_lds(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) load_global((kt + 1) * kBK);
            const uint16_t* as = As[cur];
            const uint16_t* bs = Bs[cur];
#pragma unroll
            for (int kk = 0; kk < kBK / 32; ++kk) {
                const int koff = kk * 32 + (lane / 16) * 8;
                bf16x8_t af[TM], bfr[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(
                        as + (wm * TL::WM + i * 16 + lane % 16) * kLdsRow + koff));
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bfr[j] = as_bf16x8(*reinterpret_cast<const uint4*>(
                        bs + (bcol(j) + lane % 16) * kLdsRow + koff));
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
            if (kt + 1 < nk) store_lds(cur ^ 1);
            __syncthreads();
        }

        // epilogue: activation in registers, bf16 tile in LDS, row stores
        uint16_t* os = reinterpret_cast<uint16_t*>(smem);
        float* osf = reinterpret_cast<float*>(smem);
        constexpr int ldo = TL::BN_OUT + TL::OUT_PAD;
        const uint16_t* biasb = g.bias ? g.bias + (size_t)e * g.N + n0 : nullptr;
        constexpr int TNO = (MODE == MODE_SWIGLU) ? TN / 2 : TN;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TNO; ++j) {
                int ocol;
                if (MODE == MODE_SWIGLU)
                    ocol = wn * (BN / 4) + j * 16 + lane % 16;
                else
                    ocol = wn * (BN / 2) + j * 16 + lane % 16;
                float bv = 0.f;
                if (MODE != MODE_SWIGLU && biasb) bv = bf2f(biasb[ocol]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int orow = wm * TL::WM + i * 16 + (lane / 16) * 4 + r;
                    float v;
                    if (MODE == MODE_SWIGLU)
                        v = silu_f(acc[i][j][r]) * acc[i][j + TN / 2][r];
                    else if (MODE == MODE_GELU)
                        v = gelu_f(acc[i][j][r] + bv);
                    else
                        v = acc[i][j][r] + bv;
                    if (MODE == MODE_DOWN)
                        osf[orow * ldo + ocol] = v;
                    else
                        os[orow * ldo + ocol] = (uint16_t)f2bf(v);
                }
            }
        }
        __syncthreads();
        constexpr int el_per_vec = 16 / TL::OUT_BYTES;
        constexpr int vec_per_row = TL::BN_OUT / el_per_vec;
        unsigned char* ob = static_cast<unsigned char*>(g.out) +
                            (((size_t)e * g.C + m0) * g.N + n0) * TL::OUT_BYTES;
        for (int v = tid; v < BM * vec_per_row; v += kGThreads) {
            const int row = v / vec_per_row, c = v % vec_per_row;
            if (m0 + row < kept)
                *reinterpret_cast<uint4*>(ob + ((size_t)row * g.N + c * el_per_vec) * TL::OUT_BYTES) =
                    *reinterpret_cast<const uint4*>(smem + ((size_t)row * ldo + c * el_per_vec) *
                                                               TL::OUT_BYTES);
        }
        __syncthreads();
    }
}

// ----------------------------------------------------------- fp32 path ----
// Plain fp32 tiles (16 x 16 outputs per block, K in steps of 16 through LDS);
// meant for small fp32 layers.
template <int MODE>
__global__ __launch_bounds__(256) void ffn_f32_kernel(const float* __restrict__ A,
                                                      const float* __restrict__ B0,
                                                      const float* __restrict__ B1,
                                                      const float* __restrict__ bias,
                                                      float* __restrict__ out,
                                                      const int32_t* __restrict__ keptv, int64_t C,
                                                      int K, int N) {
    __shared__ float as[16][17], b0s[16][17], b1s[16][17];
    const int e = blockIdx.z;
    int kept = keptv[e];
    if (kept > C) kept = (int)C;
    const int m0 = blockIdx.y * 16, n0 = blockIdx.x * 16;
    if (m0 >= kept) return;
    const int ty = threadIdx.x / 16, tx = threadIdx.x % 16;
    const float* Ab = A + (size_t)e * C * K;
    const float* B0b = B0 + (size_t)e * K * N;
    const float* B1b = (MODE == MODE_SWIGLU) ? B1 + (size_t)e * K * N : nullptr;
    float s0 = 0.f, s1 = 0.f;
    for (int k0 = 0; k0 < K; k0 += 16) {
        const int r = m0 + ty, kk = k0 + tx;
        as[ty][tx] = (r < kept && kk < K) ? Ab[(size_t)r * K + kk] : 0.f;
        const int kr = k0 + ty, c = n0 + tx;
        b0s[ty][tx] = (kr < K && c < N) ? B0b[(size_t)kr * N + c] : 0.f;
        if (MODE == MODE_SWIGLU) b1s[ty][tx] = (kr < K && c < N) ? B1b[(size_t)kr * N + c] : 0.f;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            s0 = fmaf(as[ty][q], b0s[q][tx], s0);
            if (MODE == MODE_SWIGLU) s1 = fmaf(as[ty][q], b1s[q][tx], s1);
        }
        __syncthreads();
    }
    const int r = m0 + ty, c = n0 + tx;
    if (r < kept && c < N) {
        float v;
        if (MODE == MODE_SWIGLU)
            v = (s0 / (1.0f + expf(-s0))) * s1;
        else if (MODE == MODE_GELU)
            v = 0.5f * (s0 + bias[(size_t)e * N + c]) *
                (1.0f + erff((s0 + bias[(size_t)e * N + c]) * 0.70710678118654752f));
        else
            v = s0 + (bias ? bias[(size_t)e * N + c] : 0.f);
        out[((size_t)e * C + r) * N + c] = v;
    }
}

int num_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

template <int BM, int BN, int MODE>
moe_status_t launch_gemm(const GemmArgs& a, hipStream_t st) {
    using TL = Tile<BM, BN, MODE>;
    auto kern = grouped_gemm_kernel<BM, BN, MODE>;
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)TL::LDS) != hipSuccess)
        return MOE_ERR_LAUNCH;
    const int64_t max_tiles = (int64_t)a.E * ((a.C + BM - 1) / BM) * (a.N / TL::BN_OUT);
    const int per_cu = TL::LDS <= 80 * 1024 ? 2 : 1;
    int64_t grid = (int64_t)num_cus() * per_cu;
    if (grid > max_tiles) grid = (max_tiles + 7) / 8 * 8;
    grid = grid / 8 * 8;
    if (grid < 8) grid = 8;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kGThreads), TL::LDS, st, a);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

constexpr int kBM = 256;
constexpr int kBN = 128;

}  // namespace

extern "C" moe_status_t moe_expert_ffn(void* stream, moe_dtype_t dtype, moe_act_t act,
                                       const void* x_disp, const int32_t* kept, int E, int64_t C,
                                       int64_t H, int64_t I, const void* w1, const void* w3,
                                       const void* w2, const void* b1, const void* b2, void* h_ws,
                                       void* y_disp) {
    if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (act != MOE_ACT_SWIGLU && act != MOE_ACT_GELU_BIAS) return MOE_ERR_DTYPE;
    if (E < 1 || C < 0 || H <= 0 || I <= 0) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    if (H > (1 << 20) || I > (1 << 20) || C >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (!kept || !w1 || !w2) return MOE_ERR_NULL;
    if (act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_NULL;
    if (act == MOE_ACT_GELU_BIAS && !b1) return MOE_ERR_NULL;
    if (C == 0) return MOE_OK;
    if (!x_disp || !h_ws || !y_disp) return MOE_ERR_NULL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == MOE_F32) {
        const float* X = static_cast<const float*>(x_disp);
        float* Hh = static_cast<float*>(h_ws);
        float* Y = static_cast<float*>(y_disp);
        dim3 g1((unsigned)((I + 15) / 16), (unsigned)((C + 15) / 16), (unsigned)E);
        dim3 g2((unsigned)((H + 15) / 16), (unsigned)((C + 15) / 16), (unsigned)E);
        if (act == MOE_ACT_SWIGLU)
            hipLaunchKernelGGL(ffn_f32_kernel<MODE_SWIGLU>, g1, dim3(256), 0, st, X,
                               static_cast<const float*>(w1), static_cast<const float*>(w3),
                               (const float*)nullptr, Hh, kept, C, (int)H, (int)I);
        else
            hipLaunchKernelGGL(ffn_f32_kernel<MODE_GELU>, g1, dim3(256), 0, st, X,
                               static_cast<const float*>(w1), (const float*)nullptr,
                               static_cast<const float*>(b1), Hh, kept, C, (int)H, (int)I);
        MOE_CHECK_LAUNCH();
        hipLaunchKernelGGL(ffn_f32_kernel<MODE_DOWN>, g2, dim3(256), 0, st, (const float*)Hh,
                           static_cast<const float*>(w2), (const float*)nullptr,
                           static_cast<const float*>(b2), Y, kept, C, (int)I, (int)H);
        MOE_CHECK_LAUNCH();
        return MOE_OK;
    }
    // bf16: K steps of 64; output tiles of 128 (SwiGLU h) or 256 columns
    if (H % kBN || I % kBK) return MOE_ERR_ALIGN;
    if (act == MOE_ACT_SWIGLU ? (I % (kBN / 2)) : (I % kBN)) return MOE_ERR_ALIGN;
    const void* ptrs[] = {x_disp, w1, w3, w2, b1, b2, h_ws, y_disp};
    for (const void* q : ptrs)
        if (q && !moe_aligned16(q)) return MOE_ERR_ALIGN;
    GemmArgs a1;
    a1.A = static_cast<const uint16_t*>(x_disp);
    a1.B0 = static_cast<const uint16_t*>(w1);
    a1.B1 = static_cast<const uint16_t*>(w3);
    a1.bias = act == MOE_ACT_GELU_BIAS ? static_cast<const uint16_t*>(b1) : nullptr;
    a1.out = h_ws;
    a1.kept = kept;
    a1.E = E;
    a1.C = C;
    a1.K = (int)H;
    a1.N = (int)I;
    moe_status_t s = act == MOE_ACT_SWIGLU ? launch_gemm<kBM, kBN, MODE_SWIGLU>(a1, st)
                                           : launch_gemm<kBM, kBN, MODE_GELU>(a1, st);
    if (s != MOE_OK) return s;
    GemmArgs a2 = a1;
    a2.A = static_cast<const uint16_t*>(h_ws);
    a2.B0 = static_cast<const uint16_t*>(w2);
    a2.B1 = nullptr;
    a2.bias = static_cast<const uint16_t*>(b2);
    a2.out = y_disp;
    a2.K = (int)I;
    a2.N = (int)H;
    return launch_gemm<kBM, kBN, MODE_DOWN>(a2, st);
}
