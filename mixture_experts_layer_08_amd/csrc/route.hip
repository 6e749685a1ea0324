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
// bf16 design (gfx950): the router is HBM-bound (x is read once; W_r is
// small and stays in L2), but at E = 32 it is 32 FLOP per byte of x, above
// what fp32 vector FMA sustains at HBM speed, so the product runs on the
// matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  Three kernels
// share the epilogue's rules:
//   * fewer 16-token tiles than 8 per compute unit: a k-split kernel puts 8
//     waves on each tile (each 1/8 of the hidden dimension) so that every
//     compute unit streams;
//   * more: each wave owns whole 16-token tiles over the full hidden
//     dimension, so no partial logits cross waves.  The staged kernel (full
//     workgroups, E a multiple of 8, at most 32 experts) passes x and W_r
//     through LDS together in chunks, every load a direct-to-LDS load of
//     whole row segments; the streaming kernel (every other shape) streams
//     x straight into A-operand registers with W_r staged in LDS.
// W_r sits in LDS in its own [H, E] layout and is read as MFMA B operands
// with gfx950's transposing LDS reads; any H that is a multiple of 256
// works.  Softmax, Gumbel noise and the k rounds of arg-max run on the
// accumulators in the MFMA's own layout: lane l holds experts 16 n + l % 16
// of tokens 4 (l / 16) .. +3, so a token's experts sit in one 16-lane row
// and every reduction is a DPP exchange inside the row (ties go to the lower
// expert index).
#include "moe_common.h"

#include <math.h>

#include <type_traits>

namespace {

using namespace moe;

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kTok = 16;          // tokens per tile (MFMA M)
constexpr int kRMaxWaves = 8;     // waves per router workgroup (one tile each at a time)
constexpr int kRMaxThreads = kRMaxWaves * kWave;
constexpr int kKC = 256;          // hidden entries per chunk
constexpr int kKS = kKC / 32;     // MFMA k-steps per chunk
constexpr int kWStageMax = 128 * 1024;  // bytes of LDS for W_r
// the k-split kernel (fewer tiles): 8 waves share each 16-token tile
constexpr int kKWaves = 8;
constexpr int kKThreads = kKWaves * kWave;
constexpr int kMaxKsPerWave = 16;       // k-steps of 32 per wave: H <= 4096

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

// Exchanges inside 16-lane rows by DPP: lanes xor 1 and xor 2 (quad
// permutes), lane i <-> 7 - i inside each half row (half mirror) and
// i <-> 15 - i inside the row (mirror).  After the four, each in turn
// combined with the lane's own partial result, every lane of a row holds the
// row's max, sum or arg-max, computed without LDS traffic.  Every lane of
// the wave must be active.
template <int CTRL>
__device__ __forceinline__ int dpp16(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp16f(float v) {
    return __builtin_bit_cast(float, dpp16<CTRL>(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp16f<0xB1>(v));
    v = fmaxf(v, dpp16f<0x4E>(v));
    v = fmaxf(v, dpp16f<0x141>(v));
    return fmaxf(v, dpp16f<0x140>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp16f<0xB1>(v);
    v += dpp16f<0x4E>(v);
    v += dpp16f<0x141>(v);
    return v + dpp16f<0x140>(v);
}
// the best of (value desc, index asc) with its carried probability
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& bv, int& bi, float& bp) {
    const float ov = dpp16f<CTRL>(bv);
    const int oi = dpp16<CTRL>(bi);
    const float op = dpp16f<CTRL>(bp);
    if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
        bp = op;
    }
}

// Reductions over aligned groups of gw lanes (gw a power of two, uniform):
// the DPP exchanges above inside 16-lane rows, lane shuffles past 16.
__device__ __forceinline__ float group_max_dpp(float v, int gw) {
    if (gw > 1) v = fmaxf(v, dpp16f<0xB1>(v));
    if (gw > 2) v = fmaxf(v, dpp16f<0x4E>(v));
    if (gw > 4) v = fmaxf(v, dpp16f<0x141>(v));
    if (gw > 8) v = fmaxf(v, dpp16f<0x140>(v));
    for (int o = 16; o < gw; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, gw));
    return v;
}
__device__ __forceinline__ float group_sum_dpp(float v, int gw) {
    if (gw > 1) v += dpp16f<0xB1>(v);
    if (gw > 2) v += dpp16f<0x4E>(v);
    if (gw > 4) v += dpp16f<0x141>(v);
    if (gw > 8) v += dpp16f<0x140>(v);
    for (int o = 16; o < gw; o <<= 1) v += __shfl_xor(v, o, gw);
    return v;
}
// the best (value desc, index asc) over the group, in every lane of it
__device__ __forceinline__ void group_argmax_dpp(float& bv, int& bi, int gw) {
    auto take = [&](float ov, int oi) {
        if (ov > bv || (ov == bv && oi < bi)) {
            bv = ov;
            bi = oi;
        }
    };
    if (gw > 1) take(dpp16f<0xB1>(bv), dpp16<0xB1>(bi));
    if (gw > 2) take(dpp16f<0x4E>(bv), dpp16<0x4E>(bi));
    if (gw > 4) take(dpp16f<0x141>(bv), dpp16<0x141>(bi));
    if (gw > 8) take(dpp16f<0x140>(bv), dpp16<0x140>(bi));
    for (int o = 16; o < gw; o <<= 1) take(__shfl_xor(bv, o, gw), __shfl_xor(bi, o, gw));
}

// Softmax / top-k / renormalisation on a tile of logits in LDS.
// lg: [kTok][ld] fp32 logits (bias not yet added).  Every thread of the
// block must call this (groups exchange values by DPP and lane shuffles).
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
        const float m = group_max_dpp(z, gw);
        const float ex = valid ? __expf(z - m) : 0.f;
        const float s = group_sum_dpp(ex, gw);
        const float prob = valid ? ex * __builtin_amdgcn_rcpf(s) : 0.f;
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
            group_argmax_dpp(bv, bi, gw);
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

// Softmax, Gumbel keys, top-k and renormalised weights of one wave's
// 16-token tile, on the accumulators in the MFMA layout: acc[n][i] of lane l
// is the logit of token t0 + 4 (l / 16) + i and expert 16 n + l % 16.
// Gumbel noise of the tile's (token, expert) pairs in the accumulator layout
// (it depends only on the counter (t, e) and the seed, so it is computed while
// the tile's x loads are in flight); zero in softmax mode.
template <int NTN>
__device__ __forceinline__ void tile_noise(float (&gn)[NTN][4], int64_t t0, const RouteParams& p,
                                           int lane) {
    const int c = lane % 16, g = lane / 16;
#pragma unroll
    for (int n = 0; n < NTN; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = t0 + 4 * g + i;
            const int e = 16 * n + c;
            gn[n][i] = (p.mode == 1 && e < p.E && t < p.T)
                           ? gumbel_from_word(philox_word0((uint32_t)t, (uint32_t)e, p.key0, p.key1))
                           : 0.f;
        }
}

template <int NTN>
__device__ __forceinline__ void route_tile_epilogue(const f32x4_t (&acc)[NTN],
                                                    const float (&gn)[NTN][4],
                                                    const float (&bias)[NTN], int64_t t0,
                                                    const RouteParams& p, int lane) {
    const int E = p.E, k = p.k;
    const int c = lane % 16, g = lane / 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + 4 * g + i;
        const bool tok_ok = t < p.T;
        float key[NTN], z[NTN], prob[NTN];
        bool ok[NTN];
        float m = -INFINITY;
#pragma unroll
        for (int n = 0; n < NTN; ++n) {
            const int e = 16 * n + c;
            ok[n] = e < E;
            const float l = acc[n][i] + bias[n];
            key[n] = l;
            z[n] = l;
            if (p.mode == 1) {
                key[n] = l + gn[n][i];
                z[n] = key[n] * p.inv_tau;
            }
            if (!ok[n]) key[n] = z[n] = -INFINITY;
            m = fmaxf(m, z[n]);
        }
        m = row16_max(m);
        float sum = 0.f;
#pragma unroll
        for (int n = 0; n < NTN; ++n) {
            prob[n] = ok[n] ? __expf(z[n] - m) : 0.f;
            sum += prob[n];
        }
        sum = row16_sum(sum);
        const float rs = __builtin_amdgcn_rcpf(sum);
#pragma unroll
        for (int n = 0; n < NTN; ++n) {
            prob[n] = ok[n] ? prob[n] * rs : 0.f;
            if (ok[n] && tok_ok) {
                p.probs[t * E + 16 * n + c] = prob[n];
                if (p.keys) p.keys[t * E + 16 * n + c] = key[n];
            }
        }
        // k rounds of arg-max over (key desc, index asc) across the 16 lanes
        bool taken[NTN];
#pragma unroll
        for (int n = 0; n < NTN; ++n) taken[n] = !ok[n];
        float wsum = 0.f, my_p = 0.f;
        int my_sel = -1;
        for (int j = 0; j < k; ++j) {
            float bv = -INFINITY, bp = 0.f;
            int bi = 0x7FFFFFFF;
#pragma unroll
            for (int n = 0; n < NTN; ++n) {  // this lane's best (lower n: lower index)
                if (!taken[n] && (key[n] > bv || bi == 0x7FFFFFFF)) {
                    bv = key[n];
                    bi = 16 * n + c;
                    bp = prob[n];
                }
            }
            argmax_step<0xB1>(bv, bi, bp);
            argmax_step<0x4E>(bv, bi, bp);
            argmax_step<0x141>(bv, bi, bp);
            argmax_step<0x140>(bv, bi, bp);
#pragma unroll
            for (int n = 0; n < NTN; ++n)
                if (16 * n + c == bi) taken[n] = true;
            wsum += bp;
            if (c == j) {
                my_sel = bi;
                my_p = bp;
            }
        }
        if (tok_ok && c < k) {
            p.topk_idx[t * k + c] = my_sel;
            p.topk_w[t * k + c] = my_p / wsum;
        }
    }
}

// buffer_load_dwordx4 ... lds: each lane's 16 bytes go to LDS at M0 + 16 * lane
// (asm, so the compiler neither tracks nor waits for it: the kernel waits
// with an explicit vmcnt(0) and a barrier before any wave reads the stage).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; nothing else here uses it
__device__ __forceinline__ void w_dma16(i32x4_t rsrc, uint32_t lds_addr, int voffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    rsrc.x = __builtin_amdgcn_readfirstlane(rsrc.x);
    rsrc.y = __builtin_amdgcn_readfirstlane(rsrc.y);
    rsrc.z = __builtin_amdgcn_readfirstlane(rsrc.z);
    rsrc.w = __builtin_amdgcn_readfirstlane(rsrc.w);
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(m0), "v"(voffset), "s"(rsrc)
        : "memory", "m0");
}
#pragma clang diagnostic pop

// W_r rows r0 .. r0 + rows into the LDS stage [rows][EP] bf16 (experts E ..
// EP-1 zero).  E a multiple of 8: direct-to-LDS loads of 16-byte pieces, a
// piece past the expert columns given an offset past the descriptor's range
// (it reads as zero); otherwise element by element through registers.
template <int NTN>
__device__ void stage_w(const RouteParams& p, unsigned char* smem, int r0, int rows) {
    constexpr int EP = 16 * NTN;
    const int tid = threadIdx.x, nthr = blockDim.x, E = p.E;
    const uint16_t* wr = static_cast<const uint16_t*>(p.w_r);
    if (E % 8 == 0) {
        const uint64_t a = reinterpret_cast<uint64_t>(wr);
        i32x4_t rs;
        rs.x = (int)(uint32_t)a;
        rs.y = (int)(uint32_t)(a >> 32) & 0xFFFF;
        rs.z = (int)(uint32_t)((size_t)p.H * E * 2);   // H * E * 2 < 2^27 (checked on the host)
        rs.w = 0x00020000;
        const uint32_t base = (uint32_t)(uintptr_t)(const lds_void_t*)smem;
        const int nbytes = rows * EP * 2;               // a multiple of 1 KB
        for (int o = (tid / kWave) * 1024; o < nbytes; o += (nthr / kWave) * 1024) {
            const int lo = o + (tid % kWave) * 16;        // this lane's LDS byte
            const int row = lo / (EP * 2), c16 = (lo % (EP * 2)) / 16;
            const int voff = c16 * 8 < E ? ((r0 + row) * E + c16 * 8) * 2 : 0x7FFFFFF0;
            w_dma16(rs, base + o, voff);
        }
    } else {
        uint16_t* w16 = reinterpret_cast<uint16_t*>(smem);
        for (int q = tid; q < rows * EP; q += nthr) {
            const int h = q / EP, e = q % EP;
            w16[q] = e < E ? wr[(size_t)(r0 + h) * E + e] : (uint16_t)0;
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The streaming kernel, for many tiles: each wave owns whole 16-token tiles
// (tile t of a wave in round r is (block * waves + wave) + r * grid * waves;
// every wave of a block runs the same number of rounds).  W_r sits in LDS in
// stages of `hs` rows: when one stage holds all of W_r it is loaded once and
// the waves never meet again; otherwise the waves restage at each stage
// boundary of every tile.  The chunk stream runs in groups of three (three
// register buffers, the loads of the chunk three ahead issued as each one is
// used) with uniform control flow: every step issues its load (past the end,
// of the last chunk again, which the caches hold), and the stream is padded
// to a multiple of three with steps whose results are not used, so the
// compiler's waits count all three buffers in flight.
template <int NTN>
__global__ __launch_bounds__(kRMaxThreads, 1) void route_bf16_kernel(RouteParams p, int ntiles,
                                                                    int hs) {
    extern __shared__ __align__(16) unsigned char smem[];   // W_r stage [hs][16 NTN] bf16
    constexpr int EP = 16 * NTN;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int nw = blockDim.x / kWave;
    const int H = p.H;
    const int nch = H / kKC;                    // chunks per tile
    const int chs = hs / kKC;                   // chunks per W_r stage
    const bool restage = chs < nch;
    const int per_round = gridDim.x * nw;
    const int nrounds = (ntiles + per_round - 1) / per_round;
    const int nsteps = nrounds * nch;           // < 2^31 (checked on the host)
    const int npad = (nsteps + 2) / 3 * 3;
    const uint16_t* xb = static_cast<const uint16_t*>(p.x);
    const int tile0 = blockIdx.x * nw + wave;
    if (nsteps == 0) return;

    // A operand of k-step s of chunk ch of round r's tile:
    // x[row][ch*256 + s*32 + (lane/16)*8 .. +8]
    auto load_x = [&](uint4 (&a)[kKS], int gstep) {
        if (gstep > nsteps - 1) gstep = nsteps - 1;
        const int r = gstep / nch, ch = gstep - r * nch;
        int64_t row = (int64_t)(tile0 + r * per_round) * kTok + (lane % 16);
        if (row >= p.T) row = p.T - 1;  // clamp: rows past T are never written out
        const uint4* src = reinterpret_cast<const uint4*>(xb + row * H + ch * kKC + (lane / 16) * 8);
#pragma unroll
        for (int s2 = 0; s2 < kKS; ++s2) a[s2] = src[s2 * 4];
    };

    float bias[NTN];
#pragma unroll
    for (int n = 0; n < NTN; ++n) {
        const int e = 16 * n + lane % 16;
        bias[n] = (p.b_r && e < p.E) ? p.b_r[e] : 0.f;
    }
    uint4 a0[kKS], a1[kKS], a2[kKS];
    load_x(a0, 0);
    load_x(a1, 1);
    load_x(a2, 2);
    stage_w<NTN>(p, smem, 0, restage ? hs : H);
    __syncthreads();
    // blocked sums: each chunk's 256 products are summed in a fresh
    // accumulator and added to the running total, which keeps fp32 rounding
    // of long hidden sizes near that of a 256-term sum
    f32x4_t acc[NTN], tot[NTN];
    float gn[NTN][4];
#pragma unroll
    for (int n = 0; n < NTN; ++n) tot[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    tile_noise<NTN>(gn, (int64_t)tile0 * kTok, p, lane);

    int ch = 0, rnd = 0;   // chunk and round of the current step (wave-uniform)
    // (the marker makes the three inlined steps different code, so the
    // compiler keeps three register buffers instead of merging the steps
    // into one body that copies buffers, which would wait for their loads)
    auto step = [&](auto buf, uint4 (&a)[kKS], int gstep) {
        asm volatile("; x buffer %0" ::"n"(decltype(buf)::value));
        if (restage && ch % chs == 0 && gstep > 0 && gstep < nsteps) {  // uniform
            __syncthreads();
            const int r0 = ch * kKC;
            stage_w<NTN>(p, smem, r0, min(hs, H - r0));
            __syncthreads();
        }
        const unsigned char* wb = smem + (size_t)(ch % chs) * kKC * EP * 2;
#pragma unroll
        for (int n = 0; n < NTN; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < kKS; ++s2) {
            const bf16x8_t av = as_bf16x8(a[s2]);
#pragma unroll
            for (int n = 0; n < NTN; ++n) {
                // transpose reads: lane L of each 16-lane group points at
                // row k0 + L/4, experts 4*(L%4).., and receives expert L of
                // rows k0..k0+3 (two reads give the 8 k of the B operand)
                i16x4_t v[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int kr = s2 * 32 + (lane / 16) * 8 + hh * 4 + (lane % 16) / 4;
                    v[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4_t*)(wb + (kr * EP + n * 16 + 4 * (lane % 4)) * 2));
                }
                const uint2 lo = __builtin_bit_cast(uint2, v[0]);
                const uint2 hi = __builtin_bit_cast(uint2, v[1]);
                const bf16x8_t bv = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[n], 0, 0, 0);
            }
        }
#pragma unroll
        for (int n = 0; n < NTN; ++n) tot[n] += acc[n];
        load_x(a, gstep + 3);
        if (ch == nch - 1 && gstep < nsteps) {
            const int tile = tile0 + rnd * per_round;
            if (tile < ntiles) route_tile_epilogue<NTN>(tot, gn, bias, (int64_t)tile * kTok, p, lane);
#pragma unroll
            for (int n = 0; n < NTN; ++n) tot[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            // the next tile's noise, while its first chunks' loads are in flight
            tile_noise<NTN>(gn, (int64_t)(tile + per_round) * kTok, p, lane);
        }
        if (++ch == nch) {
            ch = 0;
            ++rnd;
        }
    };
    for (int gs = 0; gs < npad; gs += 3) {
        step(std::integral_constant<int, 0>{}, a0, gs);
        step(std::integral_constant<int, 1>{}, a1, gs + 1);
        step(std::integral_constant<int, 2>{}, a2, gs + 2);
    }
}

// buffer_load_dword ... lds: each lane's 4 bytes go to LDS at M0 + 4 * lane.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved; nothing else here uses it
__device__ __forceinline__ void w_dma4(i32x4_t rsrc, uint32_t lds_addr, int voffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    rsrc.x = __builtin_amdgcn_readfirstlane(rsrc.x);
    rsrc.y = __builtin_amdgcn_readfirstlane(rsrc.y);
    rsrc.z = __builtin_amdgcn_readfirstlane(rsrc.z);
    rsrc.w = __builtin_amdgcn_readfirstlane(rsrc.w);
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dword %1, %2, 0 offen lds"
        :
        : "s"(m0), "v"(voffset), "s"(rsrc)
        : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ i32x4_t route_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4_t rs;
    rs.x = (int)(uint32_t)a;
    rs.y = (int)(uint32_t)(a >> 32) & 0xFFFF;
    rs.z = (int)bytes;
    rs.w = 0x00020000;
    return rs;
}

// The staged kernel, for many tiles with full workgroups (8 waves, each
// owning whole 16-token tiles as in the streaming kernel above): x and
// W_r both pass through LDS in chunks of kSC hidden entries, so every global
// load is a direct-to-LDS load of whole 256-byte row segments (16 rows x 256
// bytes per wave and chunk, four loads) and W_r needs no up-front copy (a
// chunk's kSC rows of it, 256 * EP bytes, come with the chunk).  kSStages
// stages rotate through LDS: while chunk c is multiplied, the loads of chunks
// c+1 .. c+kSStages-1 are in flight; one barrier per chunk (every wave's loads
// of chunk c have landed, and nobody reads chunk c-1's stage any more, which
// then takes chunk c+kSStages-1).  x rows sit in LDS 256 bytes apart with the
// 16-byte piece q of row r at slot q ^ (r % 16), so the A-fragment reads
// (16 rows, one piece each) hit distinct banks.  Products are summed per
// 256 hidden entries in a fresh accumulator, then added to the running
// total, as in the streaming kernel (the blocks in the workgroup's chunk
// order, below).  A tile's Gumbel noise is computed one value per chunk
// step, while the loads are in flight.  Measured at 32768 tokens, 32
// experts, H = 2048: 37 us after an Infinity Cache flush, against 47 us for
// the streaming kernel (whose per-wave register loads read 16 rows x 64
// bytes each); the softmax / top-k epilogue of the single round of tiles is
// about 5 us of it.
constexpr int kSC = 128;      // hidden entries per chunk
constexpr int kSStages = 4;
constexpr int kSWaves = 8;
template <int NTN>
struct StagedGeom {
    static constexpr int EP = 16 * NTN;
    static constexpr int X_BYTES = kSWaves * kTok * kSC * 2;  // 32 KB
    static constexpr int W_BYTES = kSC * EP * 2;              // 4 KB per 16 experts
    static constexpr int STAGE = X_BYTES + W_BYTES;
    static constexpr int W_LOADS = W_BYTES / 256 / kSWaves;   // dword loads per wave
    static constexpr int LOADS = 4 + W_LOADS;                  // per wave and chunk
    static constexpr size_t LDS = (size_t)kSStages * STAGE;
};

template <int NTN>
__global__ __launch_bounds__(kSWaves * kWave, 1) void route_staged_kernel(RouteParams p, int ntiles) {
    using SG = StagedGeom<NTN>;
    constexpr int EP = SG::EP;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int H = p.H, E = p.E;
    const int nch = H / kSC;
    const int per_round = gridDim.x * kSWaves;
    const int nrounds = (ntiles + per_round - 1) / per_round;
    const int nsteps = nrounds * nch;
    const int tile0 = blockIdx.x * kSWaves + wave;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const lds_void_t*)smem;
    const i32x4_t rsX = route_rsrc(p.x, (uint32_t)((size_t)p.T * H * 2));
    const i32x4_t rsW = route_rsrc(p.w_r, (uint32_t)((size_t)H * E * 2));

    // Workgroup b walks the chunks of its tiles starting at chunk rot and
    // wrapping around: the workgroups of odd XCDs (b % 8) start half a row
    // later, so that at any moment the XCDs read two different halves of
    // their x rows instead of all the same 256 bytes of every row (measured
    // at H = 2048: 47 -> 39 us cold for 32768 tokens; offsets of 1 KB by
    // XCD about the same, offsets varying inside an XCD slower).  rot is
    // even: the 256-entry blocks stay whole.
    const int rot = (blockIdx.x & 1u) ? ((nch / 2) & ~1) : 0;
    // loads of step gs (past the end: the last step again, into a stage
    // nobody reads, so every step issues the same loads)
    auto issue = [&](int gs) {
        if (gs > nsteps - 1) gs = nsteps - 1;
        const int r = gs / nch;
        int ch = gs - r * nch + rot;
        if (ch >= nch) ch -= nch;
        const uint32_t st = lds0 + (uint32_t)((gs % kSStages) * SG::STAGE);
        // x: load j covers rows 4j .. 4j+3 of the wave's 16; lane -> row
        // 4j + lane / 16, LDS slot lane % 16 holding piece slot ^ row
        const int64_t trow0 = (int64_t)(tile0 + r * per_round) * kTok;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = 4 * j + lane / 16;
            int64_t t = trow0 + rr;
            if (t >= p.T) t = p.T - 1;  // clamp: rows past T are never written out
            const int piece = (lane % 16) ^ rr;
            const int voff = (int)((t * H + (int64_t)ch * kSC) * 2) + piece * 16;
            w_dma16(rsX, st + wave * (kTok * kSC * 2) + j * 1024, voff);
        }
        // W_r rows ch*kSC .. +kSC as [kSC][EP], 256 bytes per load; experts
        // past E read as zero (offset past the descriptor's range)
#pragma unroll
        for (int u = 0; u < SG::W_LOADS; ++u) {
            const int i = wave * SG::W_LOADS + u;
            const int b = i * 256 + lane * 4;          // byte in the stage's W image
            const int kr = b / (EP * 2), e = (b % (EP * 2)) / 2;
            const int voff = e < E ? ((ch * kSC + kr) * E + e) * 2 : 0x7FFFFFF0;
            w_dma4(rsW, st + SG::X_BYTES + i * 256, voff);
        }
    };

    float bias[NTN];
#pragma unroll
    for (int n = 0; n < NTN; ++n) {
        const int e = 16 * n + lane % 16;
        bias[n] = (p.b_r && e < E) ? p.b_r[e] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < kSStages - 1; ++q) issue(q);
    f32x4_t acc[NTN], tot[NTN];
    float gn[NTN][4];
#pragma unroll
    for (int n = 0; n < NTN; ++n) {
        tot[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int n = 0; n < NTN; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) gn[n][i] = 0.f;
    const int arow = lane % 16, agrp = lane / 16;
    for (int gs = 0; gs < nsteps; ++gs) {
        const int r = gs / nch, ch = gs - r * nch;
        const int tile = tile0 + r * per_round;
        // this step's loads have landed once at most the newer steps' loads
        // (and any stores issued after them) are outstanding: loads and
        // stores retire in issue order
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kSStages - 2) * SG::LOADS) : "memory");
        __syncthreads();
        issue(gs + kSStages - 1);
        // Gumbel noise of this tile's value q = 4 n + i at step q (the rest
        // at the tile's last step when it has fewer steps than values)
        if (p.mode == 1) {
#pragma unroll
            for (int q = 0; q < 4 * NTN; ++q)
                if (q == ch || (ch == nch - 1 && q > ch)) {
                    const int64_t t = (int64_t)tile * kTok + 4 * agrp + q % 4;
                    const int e = 16 * (q / 4) + lane % 16;
                    gn[q / 4][q % 4] =
                        (e < E && t < p.T)
                            ? gumbel_from_word(philox_word0((uint32_t)t, (uint32_t)e, p.key0, p.key1))
                            : 0.f;
                }
        }
        const unsigned char* xs = smem + (gs % kSStages) * SG::STAGE + wave * (kTok * kSC * 2);
        const unsigned char* wb = smem + (gs % kSStages) * SG::STAGE + SG::X_BYTES;
#pragma unroll
        for (int s2 = 0; s2 < kSC / 32; ++s2) {
            const int slot = (4 * s2 + agrp) ^ arow;
            const bf16x8_t av = as_bf16x8(*reinterpret_cast<const uint4*>(xs + arow * (kSC * 2) + slot * 16));
#pragma unroll
            for (int n = 0; n < NTN; ++n) {
                i16x4_t v[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int kr = s2 * 32 + agrp * 8 + hh * 4 + (lane % 16) / 4;
                    v[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4_t*)(wb + (kr * EP + n * 16 + 4 * (lane % 4)) * 2));
                }
                const uint2 lo = __builtin_bit_cast(uint2, v[0]);
                const uint2 hi = __builtin_bit_cast(uint2, v[1]);
                const bf16x8_t bv = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[n], 0, 0, 0);
            }
        }
        // blocks of 256 hidden entries (two chunks; a last odd chunk alone)
        if ((ch & 1) || ch == nch - 1) {
#pragma unroll
            for (int n = 0; n < NTN; ++n) {
                tot[n] += acc[n];
                acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
        if (ch == nch - 1) {
            if (tile < ntiles) route_tile_epilogue<NTN>(tot, gn, bias, (int64_t)tile * kTok, p, lane);
#pragma unroll
            for (int n = 0; n < NTN; ++n) tot[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    // the padding steps' loads still write LDS: let them land before the
    // workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The k-split kernel, for token counts that leave compute units idle with
// one wave per tile: a workgroup of 8 waves copies W_r into LDS once, in its
// own [H, E] layout (16-byte loads), then walks 16-token tiles; each wave owns
// 1/8 of the hidden dimension and streams its x slice straight from HBM into
// A-operand registers (16 rows x 64 contiguous bytes per load), the next
// tile's loads issued before the current tile's reduction and epilogue; the
// 8 partial logit tiles are summed in LDS in a fixed order, then lane groups
// of width G = 2^ceil(log2 E) hold one token each for the softmax and the k
// rounds of arg-max.
template <int NTN>
__global__ __launch_bounds__(kKThreads) void route_ksplit_kernel(RouteParams p, int ntiles, int gw) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int H = p.H;
    const int nks = H / 32;                    // k-steps of 32
    const int ks_per_wave = nks / kKWaves;     // <= kMaxKsPerWave
    uint4* wlds = reinterpret_cast<uint4*>(smem);                          // [H][16*NTN] bf16
    f32x4_t* red = reinterpret_cast<f32x4_t*>(smem + (size_t)nks * NTN * 1024);  // [8][NTN][64]
    float* lg = reinterpret_cast<float*>(red + kKWaves * NTN * kWave);     // [16][16*NTN]
    constexpr int ld = 16 * NTN;

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const uint16_t* xb = static_cast<const uint16_t*>(p.x);

    // wave w takes hidden slice (w + 4 (b & 1)) % 8: the workgroups of odd
    // XCDs start half a row later (see the staged kernel); partials are
    // summed by slice, so the sums do not depend on the assignment
    const int slice = (wave + ((blockIdx.x & 1u) ? kKWaves / 2 : 0)) % kKWaves;
    const int ks0 = slice * ks_per_wave;
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

    // Stage W_r [H, E] in LDS as [H][16*NTN] (experts past E are zero); with
    // E a multiple of 8 by direct-to-LDS loads, all in flight together with
    // the x loads above.
    constexpr int EP = 16 * NTN;
    stage_w<NTN>(p, smem, 0, H);
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
        for (int n = 0; n < NTN; ++n) red[(slice * NTN + n) * kWave + lane] = acc[n];
        __syncthreads();
        // fixed-order sum of the 8 partial tiles -> lg[token][expert]
        for (int q = tid; q < kTok * ld; q += kKThreads) {
            const int tt = q / ld, e = q % ld;
            const int n = e / 16;
            const int l = (tt / 4) * 16 + (e % 16);
            const int r = tt % 4;
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < kKWaves; ++w) s += red[(w * NTN + n) * kWave + l][r];
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

// LDS one workgroup may hold on the current device (0 if unknown)
size_t max_lds() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || n <= 0)
        return 0;
    return (size_t)n;
}

template <int NTN>
moe_status_t launch_ksplit(const RouteParams& p, hipStream_t st) {
    const int nks = p.H / 32;
    const size_t lds = (size_t)nks * NTN * 1024 + (size_t)kKWaves * NTN * kWave * 16 +
                       (size_t)kTok * 16 * NTN * 4;
    if (lds > 160 * 1024) return MOE_ERR_UNSUPPORTED;
    if (hipFuncSetAttribute((const void*)route_ksplit_kernel<NTN>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return MOE_ERR_LAUNCH;
    const int ntiles = (int)((p.T + kTok - 1) / kTok);
    const int per_cu = lds <= 72 * 1024 ? 2 : 1;
    int grid = num_cus() * per_cu;
    if (grid > ntiles) grid = ntiles;
    hipLaunchKernelGGL(route_ksplit_kernel<NTN>, dim3(grid), dim3(kKThreads), lds, st, p, ntiles,
                       group_width(p.E));
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

template <int NTN>
moe_status_t launch_bf16(const RouteParams& p, hipStream_t st) {
    constexpr int EP = 16 * NTN;
    // W_r rows per LDS stage: all of them when they fit, else a multiple of 256
    int hs = p.H;
    if ((size_t)hs * EP * 2 > (size_t)kWStageMax) hs = kWStageMax / (EP * 2) / kKC * kKC;
    const int ntiles = (int)((p.T + kTok - 1) / kTok);
    const int cus = num_cus();
    // fewer tiles than 8 per compute unit: the k-split kernel, which puts 8
    // waves on each tile, when W_r fits its LDS image (H <= 4096)
    if ((int64_t)ntiles < (int64_t)cus * kRMaxWaves && p.H / 32 / kKWaves <= kMaxKsPerWave) {
        const moe_status_t s = launch_ksplit<NTN>(p, st);
        if (s != MOE_ERR_UNSUPPORTED) return s;
    }
    // one workgroup per compute unit, up to 8 waves of one tile each
    int waves = (ntiles + cus - 1) / cus;
    if (waves > kRMaxWaves) waves = kRMaxWaves;
    if (waves < 1) waves = 1;
    int grid = (ntiles + waves - 1) / waves;
    if (grid > cus) grid = cus;
    // full workgroups: x and W_r staged through LDS together (x addressed
    // with 32-bit byte offsets, W_r by 4-byte loads of expert pairs)
    if (waves == kSWaves && p.E % 8 == 0 && (int64_t)p.T * p.H * 2 < ((int64_t)1 << 31) &&
        StagedGeom<NTN>::LDS <= max_lds()) {
        using SG = StagedGeom<NTN>;
        if (hipFuncSetAttribute((const void*)route_staged_kernel<NTN>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)SG::LDS) != hipSuccess)
            return MOE_ERR_LAUNCH;
        hipLaunchKernelGGL(route_staged_kernel<NTN>, dim3(grid), dim3(kSWaves * kWave), SG::LDS, st,
                           p, ntiles);
        MOE_CHECK_LAUNCH();
        return MOE_OK;
    }
    const size_t lds = (size_t)hs * EP * 2;
    if (hipFuncSetAttribute((const void*)route_bf16_kernel<NTN>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return MOE_ERR_LAUNCH;
    hipLaunchKernelGGL(route_bf16_kernel<NTN>, dim3(grid), dim3(waves * kWave), lds, st, p, ntiles,
                       hs);
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
    if (H % kKC) return MOE_ERR_ALIGN;
    if (H * E * 2 >= ((int64_t)1 << 27)) return MOE_ERR_UNSUPPORTED;  // 32-bit LDS-load offsets
    if (((T + kTok - 1) / kTok + 1) * (H / kKC) >= ((int64_t)1 << 30)) return MOE_ERR_UNSUPPORTED;
    if (!moe_aligned16(x) || !moe_aligned16(w_r)) return MOE_ERR_ALIGN;
    const int ntn = (E + 15) / 16;
    switch (ntn) {
        case 1: return launch_bf16<1>(p, st);
        case 2: return launch_bf16<2>(p, st);
        case 3: return launch_bf16<3>(p, st);
        default: return launch_bf16<4>(p, st);
    }
}
