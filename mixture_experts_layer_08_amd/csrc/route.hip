// Router: logits GEMM, softmax, top-k with renormalised weights, and the
// Gumbel hard top-k variant.
//
// [P2] MoE basics page (dpshk.com/news/6005940) section 2.1: score = x . W_r,
//      softmax, keep the top-k; section 3.1: weights renormalised over the k.
// [P5] llama-moe essay (coreui.cn/article/2610641) section 3.1: selected
//      probabilities divided by their sum; router math kept in high precision.
// [P4] long-context page (2kiu.com/news/5130654) sections 2 and 5.2: Gumbel
//      noise on the logits, hard top-k, temperature 1 + 1e-4 * seq_len.
//
// bf16 design (gfx950): the router is HBM-bound (x is read once, W_r is tiny
// and lives in L2), but at E = 32 it is 32 FLOP per byte of x, above what
// fp32 vector FMA sustains at HBM speed, so the product runs on the matrix
// cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  One workgroup of 8
// waves copies W_r into LDS once, in its own [H, E] layout (16-byte loads),
// and reads MFMA B operands from it with gfx950's transpose LDS reads; it
// then walks 16-token tiles.  Each
// wave owns 1/8 of the hidden dimension and streams its x slice straight
// from HBM into A-fragment registers (16 rows x 64 contiguous bytes per
// load); the next tile's loads are issued before the current tile's
// reduction and epilogue so HBM stays busy.  The 8 partial logit tiles are
// summed in LDS in a fixed order, then lane groups of width G = 2^ceil(log2 E)
// hold one token each for the softmax and the k rounds of arg-max.
#include "moe_common.h"

#include <math.h>

namespace {

using namespace moe;

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kTok = 16;          // tokens per tile (MFMA M)
constexpr int kRWaves = 8;        // waves per router workgroup
constexpr int kRThreads = kRWaves * kWave;
constexpr int kMaxKsPerWave = 16; // 16 k-steps of 32 = 512 hidden per wave

struct RouteParams {
    const void* x;
    const void* w_r;
    const float* b_r;
    int64_t T;
    int H;
    int E;
    int k;
    int mode;          // 0 softmax, 1 gumbel
    uint32_t key0, key1;
    float inv_tau;
    int32_t* topk_idx;
    float* topk_w;
    float* probs;
    float* keys;
};

// Philox4x32-10 (Salmon et al., SC'11), counter (c0, c1, 0, 0): word 0.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t k0,
                                                 uint32_t k1) {
    uint32_t c2 = 0, c3 = 0;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    return c0;
}

// g = -log(-log u) with u = (w + 0.5) 2^-32.  For u >= 1/2 the inner log is
// taken as log1p(-(1 - u)) with 1 - u = (~w + 0.5) 2^-32, which keeps full
// relative precision where u is close to 1.
__device__ __forceinline__ float gumbel_from_word(uint32_t w) {
    const float s = 2.3283064365386963e-10f;  // 2^-32
    float nl;
    if (w < 0x80000000u) {
        nl = -logf(((float)w + 0.5f) * s);
    } else {
        nl = -log1pf(-(((float)(~w) + 0.5f) * s));
    }
    return -logf(nl);
}

// Softmax / top-k / renormalisation on a tile of logits in LDS.
// lg: [kTok][ld] fp32 logits (bias not yet added).  Every thread of the
// block must call this (groups exchange values with lane shuffles).
__device__ void route_epilogue(const float* lg, int ld, int64_t t0, const RouteParams& p,
                               int gw) {
    const int tid = threadIdx.x;
    const int per_pass = blockDim.x / gw;
    const int E = p.E, k = p.k;
    for (int pass = 0; pass * per_pass < kTok; ++pass) {
        const int tt = pass * per_pass + tid / gw;
        const int e = tid % gw;
        const int64_t t = t0 + tt;
        const bool tok_ok = (tt < kTok) && (t < p.T);
        const bool valid = tok_ok && (e < E);
        float l = -INFINITY;
        if (valid) {
            l = lg[tt * ld + e];
            if (p.b_r) l += p.b_r[e];
        }
        float key = l;
        float z = l;  // softmax argument
        if (p.mode == 1 && valid) {
            key = l + gumbel_from_word(philox_word0((uint32_t)t, (uint32_t)e, p.key0, p.key1));
            z = key * p.inv_tau;
        }
        // probabilities
        const float m = group_max(z, gw);
        const float ex = valid ? expf(z - m) : 0.f;
        const float s = group_sum(ex, gw);
        const float prob = valid ? ex / s : 0.f;
        if (valid) {
            p.probs[t * E + e] = prob;
            if (p.keys) p.keys[t * E + e] = key;
        }
        // k rounds of arg-max over (key desc, index asc)
        bool taken = !valid;
        float wsum = 0.f;
        int my_sel = -1;
        float my_prob = 0.f;
        for (int j = 0; j < k; ++j) {
            float bv = taken ? -INFINITY : key;
            int bi = taken ? 0x7FFFFFFF : e;
            for (int o = gw >> 1; o > 0; o >>= 1) {
                const float ov = __shfl_xor(bv, o, gw);
                const int oi = __shfl_xor(bi, o, gw);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            const int base = (threadIdx.x % kWave) / gw * gw;
            const float pw = __shfl(prob, base + (bi < gw ? bi : 0), kWave);
            if (e == bi) taken = true;
            wsum += pw;
            if (e == j) {
                my_sel = bi;
                my_prob = pw;
            }
        }
        if (tok_ok && e < k) {
            p.topk_idx[t * k + e] = my_sel;
            p.topk_w[t * k + e] = my_prob / wsum;
        }
    }
}

template <int NTN>
__global__ __launch_bounds__(kRThreads) void route_bf16_kernel(RouteParams p, int ntiles, int gw) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int H = p.H;
    const int nks = H / 32;                    // k-steps of 32
    const int ks_per_wave = nks / kRWaves;     // <= kMaxKsPerWave
    uint4* wlds = reinterpret_cast<uint4*>(smem);                          // [H][16*NTN] bf16
    f32x4_t* red = reinterpret_cast<f32x4_t*>(smem + (size_t)nks * NTN * 1024);  // [8][NTN][64]
    float* lg = reinterpret_cast<float*>(red + kRWaves * NTN * kWave);     // [16][16*NTN]
    constexpr int ld = 16 * NTN;

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const uint16_t* xb = static_cast<const uint16_t*>(p.x);
    const uint16_t* wr = static_cast<const uint16_t*>(p.w_r);

    const int ks0 = wave * ks_per_wave;
    // A fragment of k-step ks for this lane: x[t0 + lane%16][ks*32 + (lane/16)*8 .. +8]
    auto load_tile = [&](uint4 (&a)[kMaxKsPerWave], int tile) {
        int64_t row = (int64_t)tile * kTok + (lane % 16);
        if (row >= p.T) row = p.T - 1;  // clamp: rows past T are never written out
        const uint4* src = reinterpret_cast<const uint4*>(xb + row * H + (lane / 16) * 8);
#pragma unroll
        for (int i = 0; i < kMaxKsPerWave; ++i)
            if (i < ks_per_wave) a[i] = src[(size_t)(ks0 + i) * 4];
    };

    uint4 a_cur[kMaxKsPerWave], a_nxt[kMaxKsPerWave];
    int tile = blockIdx.x;
    if (tile < ntiles) load_tile(a_cur, tile);

    // Stage W_r [H, E] in LDS as [H][16*NTN] (experts past E are zero),
    // 16-byte vectors when E is a multiple of 8.
    constexpr int EP = 16 * NTN;
    if (p.E % 8 == 0) {
        const int vpr = p.E / 8;  // vectors per W_r row
        for (int v = tid; v < H * vpr; v += kRThreads) {
            const int h = v / vpr, c = v % vpr;
            wlds[h * EP / 8 + c] = reinterpret_cast<const uint4*>(wr)[(size_t)h * vpr + c];
        }
        const int padv = (EP - p.E) / 8;
        for (int v = tid; v < H * padv; v += kRThreads) {
            const int h = v / padv, c = v % padv;
            wlds[h * EP / 8 + vpr + c] = make_uint4(0, 0, 0, 0);
        }
    } else {
        uint16_t* w16 = reinterpret_cast<uint16_t*>(wlds);
        for (int v = tid; v < H * EP; v += kRThreads) {
            const int h = v / EP, e = v % EP;
            w16[v] = e < p.E ? wr[(size_t)h * p.E + e] : (uint16_t)0;
        }
    }
    __syncthreads();

    for (; tile < ntiles; tile += gridDim.x) {
        f32x4_t acc[NTN];
#pragma unroll
        for (int n = 0; n < NTN; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kMaxKsPerWave; ++i) {
            if (i < ks_per_wave) {
                const bf16x8_t a = as_bf16x8(a_cur[i]);
#pragma unroll
                for (int n = 0; n < NTN; ++n) {
                    // transpose reads: lane L of each 16-lane group points at
                    // row k0 + L/4, experts 4*(L%4).., and receives expert L of
                    // rows k0..k0+3 (two reads give the 8 k of the B operand)
                    const unsigned char* wb = reinterpret_cast<const unsigned char*>(wlds);
                    i16x4_t v[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int kr = (ks0 + i) * 32 + (lane / 16) * 8 + hh * 4 + (lane % 16) / 4;
                        v[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(
                            wb + (kr * EP + n * 16 + 4 * (lane % 4)) * 2));
                    }
                    const uint2 lo = __builtin_bit_cast(uint2, v[0]);
                    const uint2 hi = __builtin_bit_cast(uint2, v[1]);
                    const bf16x8_t b = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
                    acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[n], 0, 0, 0);
                }
            }
        }
        const int next = tile + gridDim.x;
        if (next < ntiles) load_tile(a_nxt, next);
#pragma unroll
        for (int n = 0; n < NTN; ++n) red[(wave * NTN + n) * kWave + lane] = acc[n];
        __syncthreads();
        // fixed-order sum of the 8 partial tiles -> lg[token][expert]
        for (int q = tid; q < kTok * ld; q += kRThreads) {
            const int tt = q / ld, e = q % ld;
            const int n = e / 16;
            const int l = (tt / 4) * 16 + (e % 16);
            const int r = tt % 4;
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < kRWaves; ++w) s += red[(w * NTN + n) * kWave + l][r];
            lg[tt * ld + e] = s;
        }
        __syncthreads();
        route_epilogue(lg, ld, (int64_t)tile * kTok, p, gw);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kMaxKsPerWave; ++i) a_cur[i] = a_nxt[i];
    }
}

// fp32 router: plain fp32 dot products (small workloads).
__global__ __launch_bounds__(256) void route_f32_kernel(RouteParams p, int ntiles, int gw) {
    __shared__ float lg[kTok * MOE_MAX_EXPERTS];
    const float* x = static_cast<const float*>(p.x);
    const float* w = static_cast<const float*>(p.w_r);
    const int ld = p.E;
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t t0 = (int64_t)tile * kTok;
        for (int q = threadIdx.x; q < kTok * p.E; q += blockDim.x) {
            const int tt = q / p.E, e = q % p.E;
            const int64_t t = t0 + tt;
            float s = 0.f;
            if (t < p.T) {
                const float* xr = x + t * p.H;
                for (int h = 0; h < p.H; ++h) s = fmaf(xr[h], w[(size_t)h * p.E + e], s);
            }
            lg[tt * ld + e] = s;
        }
        __syncthreads();
        route_epilogue(lg, ld, t0, p, gw);
        __syncthreads();
    }
}

int group_width(int E) {
    int g = 1;
    while (g < E) g <<= 1;
    return g;
}

int num_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

template <int NTN>
moe_status_t launch_bf16(const RouteParams& p, hipStream_t st) {
    const int nks = p.H / 32;
    const size_t lds = (size_t)nks * NTN * 1024 + (size_t)kRWaves * NTN * kWave * 16 +
                       (size_t)kTok * 16 * NTN * 4;
    if (lds > 160 * 1024) return MOE_ERR_UNSUPPORTED;
    if (hipFuncSetAttribute((const void*)route_bf16_kernel<NTN>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return MOE_ERR_LAUNCH;
    const int ntiles = (int)((p.T + kTok - 1) / kTok);
    const int per_cu = lds <= 72 * 1024 ? 2 : 1;
    int grid = num_cus() * per_cu;
    if (grid > ntiles) grid = ntiles;
    hipLaunchKernelGGL(route_bf16_kernel<NTN>, dim3(grid), dim3(kRThreads), lds, st, p, ntiles,
                       group_width(p.E));
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

}  // namespace

extern "C" moe_status_t moe_route(void* stream, moe_dtype_t dtype, const void* x, const void* w_r,
                                  const float* b_r, int64_t T, int64_t H, int E, int k,
                                  moe_route_mode_t mode, uint64_t seed, int64_t seq_len,
                                  int32_t* topk_idx, float* topk_w, float* probs, float* keys) {
    if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (mode != MOE_ROUTE_SOFTMAX_TOPK && mode != MOE_ROUTE_GUMBEL_HARD) return MOE_ERR_DTYPE;
    if (T < 0 || H <= 0 || E < 1 || k < 1 || k > E) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
    if (T >= ((int64_t)1 << 31) || H > (1 << 20)) return MOE_ERR_UNSUPPORTED;
    if (mode == MOE_ROUTE_GUMBEL_HARD && seq_len <= 0) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    if (!x || !w_r || !topk_idx || !topk_w || !probs) return MOE_ERR_NULL;
    RouteParams p;
    p.x = x;
    p.w_r = w_r;
    p.b_r = b_r;
    p.T = T;
    p.H = (int)H;
    p.E = E;
    p.k = k;
    p.mode = (int)mode;
    p.key0 = (uint32_t)(seed & 0xFFFFFFFFull);
    p.key1 = (uint32_t)(seed >> 32);
    p.inv_tau = (float)(1.0 / (1.0 + 1e-4 * (double)seq_len));
    p.topk_idx = topk_idx;
    p.topk_w = topk_w;
    p.probs = probs;
    p.keys = keys;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == MOE_F32) {
        if (H % 4) return MOE_ERR_ALIGN;
        const int ntiles = (int)((T + kTok - 1) / kTok);
        int grid = num_cus() * 4;
        if (grid > ntiles) grid = ntiles;
        hipLaunchKernelGGL(route_f32_kernel, dim3(grid), dim3(256), 0, st, p, ntiles,
                           group_width(E));
        MOE_CHECK_LAUNCH();
        return MOE_OK;
    }
    if (H % 256) return MOE_ERR_ALIGN;
    if (H / 32 / kRWaves > kMaxKsPerWave) return MOE_ERR_UNSUPPORTED;
    if (!moe_aligned16(x) || !moe_aligned16(w_r)) return MOE_ERR_ALIGN;
    const int ntn = (E + 15) / 16;
    switch (ntn) {
        case 1: return launch_bf16<1>(p, st);
        case 2: return launch_bf16<2>(p, st);
        case 3: return launch_bf16<3>(p, st);
        default: return launch_bf16<4>(p, st);
    }
}
