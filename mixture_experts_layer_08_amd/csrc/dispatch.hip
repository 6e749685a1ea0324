// Capacity-bounded dispatch of token copies into per-expert row buffers.
//
// [P2] MoE basics page (dpshk.com/news/6005940) section 2.4: each expert
//      accepts at most C = ceil(tokens / experts * cf) rows; the excess is
//      dropped.
// [P1] LLaMA4-MoE guide (dpshk.com/news/5809432) section 2.4: group the
//      flattened [T, k] assignments by expert id (a stable sort), then run
//      each expert on its contiguous group.
//
// The stable sort is a counting sort with a deterministic order, so every
// integer output is reproducible bit for bit:
//  1. histogram: per block of 256 assignments, LDS integer counts;
//  2. scan: one block turns the per-block counts into per-block starting
//     rows for every expert (exclusive scan in block order; with the aux
//     statistics, 1024 threads over stripes of blocks), and finishes
//     kept[e] = min(count, C) and the dropped total;
//  3. rank: each wave walks 64 assignments at a time in (t, j) order; a
//     ballot per distinct expert in the chunk gives each lane its rank among
//     same-expert lanes; slot and slot_token follow;
//  4. copy: token-major gather of x rows into x_disp, one 16-byte vector per
//     lane, each row read once and written to each of its kept slots
//     (bandwidth-bound; many blocks so all CUs stream).
// moe_dispatch_aux also produces the load-balancing statistics ([P2]
// section 2.3, [P1] section 3.2) in the same launches: the histogram blocks
// sum their tokens' router probabilities per expert as well, and the scan
// block, which already totals each expert's assignments, finishes f, P and
// L_aux from those totals and partial sums (both in block order).
#include "moe_common.h"

#include <mutex>

namespace {

constexpr int kDChunk = 256;           // assignments per histogram / rank block
constexpr int kDThreads = 256;
constexpr int kDWaveSpan = kDChunk / (kDThreads / 64);  // 64 assignments per wave
constexpr int kCopyTok = 8;            // tokens per copy block

__global__ __launch_bounds__(kDThreads) void disp_hist_kernel(const int32_t* __restrict__ idx,
                                                             int64_t A, int E,
                                                             int32_t* __restrict__ hist) {
    __shared__ int cnt[MOE_MAX_EXPERTS];
    if (threadIdx.x < E) cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t a0 = (int64_t)blockIdx.x * kDChunk;
    int64_t a1 = a0 + kDChunk;
    if (a1 > A) a1 = A;
    for (int64_t a = a0 + threadIdx.x; a < a1; a += kDThreads) {
        const unsigned e = (unsigned)idx[a];
        if (e < (unsigned)E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (threadIdx.x < E) hist[(size_t)blockIdx.x * E + threadIdx.x] = cnt[threadIdx.x];
}

// The histogram of disp_hist_kernel plus, per block, the column sums of the
// router probabilities of its tokens (token t belongs to the block holding
// its first assignment t*k), in double.
__global__ __launch_bounds__(kDThreads) void disp_hist_aux_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ probs, int64_t A, int E, int k,
    int32_t* __restrict__ hist, double* __restrict__ psum) {
    __shared__ int cnt[MOE_MAX_EXPERTS];
    __shared__ double colsum[kDThreads];
    const int tid = threadIdx.x;
    if (tid < E) cnt[tid] = 0;
    __syncthreads();
    const int64_t a0 = (int64_t)blockIdx.x * kDChunk;
    int64_t a1 = a0 + kDChunk;
    if (a1 > A) a1 = A;
    for (int64_t a = a0 + tid; a < a1; a += kDThreads) {
        const unsigned e = (unsigned)idx[a];
        if (e < (unsigned)E) atomicAdd(&cnt[e], 1);
    }
    // tokens ceil(a0/k) .. ceil(a1/k)-1; thread (r, e) strides over them
    const int64_t t0 = (a0 + k - 1) / k, t1 = (a1 + k - 1) / k;
    const int rows = kDThreads / E;
    const int r = tid / E, e = tid % E;
    double sacc = 0.0;
    if (r < rows)
        for (int64_t t = t0 + r; t < t1; t += rows) sacc += (double)probs[t * E + e];
    colsum[tid] = sacc;
    __syncthreads();
    if (tid < E) {
        double acc = 0.0;
        for (int rr = 0; rr < rows; ++rr) acc += colsum[rr * E + tid];
        psum[(size_t)blockIdx.x * E + tid] = acc;
        hist[(size_t)blockIdx.x * E + tid] = cnt[tid];
    }
}

// The scan of disp_scan_kernel plus the statistics: counts[e] = the
// expert's assignments before the drop, f = counts/(T k), P = (sum of the
// block partials)/T, L_aux = alpha E sum_e f P.  One workgroup of 1024
// threads: thread (r, e) owns stripe r of consecutive histogram blocks for
// expert e, sums the stripe (its loads all in flight together), the stripe
// totals are scanned in stripe order, and each thread then writes its
// blocks' starting rows.  P adds each stripe's partial sums in block order,
// then the stripes in order (a fixed order: deterministic).
constexpr int kScanThreads = 1024;
constexpr int kScanUnroll = 8;

__global__ __launch_bounds__(kScanThreads) void disp_scan_aux_kernel(
    const int32_t* __restrict__ hist, const double* __restrict__ psum, int nb, int E, int64_t C,
    int64_t T, int k, float alpha, int32_t* __restrict__ off, int32_t* __restrict__ kept,
    int32_t* __restrict__ dropped, int32_t* __restrict__ counts, float* __restrict__ f,
    float* __restrict__ p, float* __restrict__ l_aux) {
    __shared__ int64_t s_cnt[kScanThreads];     // [stripe][expert] counts
    __shared__ double s_ps[kScanThreads];       // [stripe][expert] probability sums
    __shared__ int64_t over[MOE_MAX_EXPERTS];
    __shared__ double fp[MOE_MAX_EXPERTS];
    const int tid = threadIdx.x;
    const int R = kScanThreads / E;             // stripes
    const int S = (nb + R - 1) / R;             // blocks per stripe
    const int r = tid / E, e = tid % E;
    const bool active = r < R;
    const int b0 = r * S, b1 = min(b0 + S, nb);
    int64_t cnt = 0;
    double ps = 0.0;
    if (active) {
        for (int b = b0; b < b1; b += kScanUnroll) {
            int h[kScanUnroll];
            double q[kScanUnroll];
#pragma unroll
            for (int u = 0; u < kScanUnroll; ++u) {
                h[u] = b + u < b1 ? hist[(size_t)(b + u) * E + e] : 0;
                q[u] = b + u < b1 ? psum[(size_t)(b + u) * E + e] : 0.0;
            }
#pragma unroll
            for (int u = 0; u < kScanUnroll; ++u) {
                cnt += h[u];
                if (b + u < b1) ps += q[u];
            }
        }
        s_cnt[tid] = cnt;
        s_ps[tid] = ps;
    }
    __syncthreads();
    if (tid < E) {  // stripe bases in stripe order; totals
        int64_t run = 0;
        double pt = 0.0;
        for (int rr = 0; rr < R; ++rr) {
            const int64_t c = s_cnt[rr * E + tid];
            s_cnt[rr * E + tid] = run;
            run += c;
            pt += s_ps[rr * E + tid];
        }
        kept[tid] = (int32_t)(run < C ? run : C);
        over[tid] = run > C ? run - C : 0;
        const double fe = T > 0 ? (double)run / ((double)T * k) : 0.0;
        const double pe = T > 0 ? pt / (double)T : 0.0;
        counts[tid] = (int32_t)run;
        f[tid] = (float)fe;
        p[tid] = (float)pe;
        fp[tid] = fe * pe;
    }
    __syncthreads();
    if (active) {  // each block's starting row, from the stripe's base
        int64_t run = s_cnt[tid];
        for (int b = b0; b < b1; ++b) {
            off[(size_t)b * E + e] = (int32_t)run;
            run += hist[(size_t)b * E + e];
        }
    }
    if (tid == 0) {
        int64_t d = 0;
        double acc = 0.0;
        for (int i = 0; i < E; ++i) {
            d += over[i];
            acc += fp[i];
        }
        *dropped = (int32_t)d;
        *l_aux = (float)((double)alpha * E * acc);
    }
}

__global__ __launch_bounds__(MOE_MAX_EXPERTS) void disp_scan_kernel(const int32_t* __restrict__ hist,
                                                                   int nb, int E, int64_t C,
                                                                   int32_t* __restrict__ off,
                                                                   int32_t* __restrict__ kept,
                                                                   int32_t* __restrict__ dropped) {
    __shared__ int64_t over[MOE_MAX_EXPERTS];
    const int e = threadIdx.x;
    if (e < E) {
        int64_t run = 0;
        int b = 0;
        for (; b + 8 <= nb; b += 8) {  // eight independent loads in flight
            int h[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) h[u] = hist[(size_t)(b + u) * E + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                off[(size_t)(b + u) * E + e] = (int32_t)run;
                run += h[u];
            }
        }
        for (; b < nb; ++b) {
            off[(size_t)b * E + e] = (int32_t)run;
            run += hist[(size_t)b * E + e];
        }
        kept[e] = (int32_t)(run < C ? run : C);
        over[e] = run > C ? run - C : 0;
    }
    __syncthreads();
    if (e == 0) {
        int64_t d = 0;
        for (int i = 0; i < E; ++i) d += over[i];
        *dropped = (int32_t)d;
    }
}

// Rank of this lane's assignment among the earlier lanes of the wave with the
// same expert, plus the wave's running count of that expert (held by lane e
// of `run`, which is updated).  One uniform iteration per distinct expert in
// the chunk; the leader's expert and the running count are read with
// readlane, so no step waits on LDS.
__device__ __forceinline__ int wave_rank(int e, bool ok, int& run, int lane, uint64_t lt_mask) {
    int r = 0;
    uint64_t rem = __ballot(ok);
    while (rem) {
        const int leader = __builtin_ctzll(rem);
        const int ee = __builtin_amdgcn_readlane(e, leader);
        const uint64_t m = __ballot(ok && e == ee);
        const int base = __builtin_amdgcn_readlane(run, ee);
        if (ok && e == ee) r = base + __popcll(m & lt_mask);
        run += (lane == ee) ? __popcll(m) : 0;
        rem &= ~m;
    }
    return r;
}

__global__ __launch_bounds__(kDThreads) void disp_rank_kernel(
    const int32_t* __restrict__ idx, int64_t A, int E, int k, int64_t C,
    const int32_t* __restrict__ off, const int32_t* __restrict__ kept, int32_t* __restrict__ slot,
    int32_t* __restrict__ slot_token) {
    __shared__ int tot[kDThreads / 64][MOE_MAX_EXPERTS];
    __shared__ int wbase[kDThreads / 64][MOE_MAX_EXPERTS];
    constexpr int kChunks = kDWaveSpan / 64;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int64_t start = (int64_t)blockIdx.x * kDChunk + (int64_t)wave * kDWaveSpan;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    int run = 0;            // lane e: this wave's running count of expert e
    int rank[kChunks];
    int my_e[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        const int64_t a = start + c * 64 + lane;
        const bool valid = a < A;
        const int e = valid ? idx[a] : -1;
        my_e[c] = e;
        rank[c] = wave_rank(e, valid && (unsigned)e < (unsigned)E, run, lane, lt_mask);
    }
    if (lane < E) tot[wave][lane] = run;
    __syncthreads();
    if (threadIdx.x < E) {
        int acc = ((int64_t)blockIdx.x * kDChunk < A) ? off[(size_t)blockIdx.x * E + threadIdx.x] : 0;
        for (int w = 0; w < kDThreads / 64; ++w) {
            wbase[w][threadIdx.x] = acc;
            acc += tot[w][threadIdx.x];
        }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        const int64_t a = start + c * 64 + lane;
        if (a < A) {
            const int e = my_e[c];
            if ((unsigned)e >= (unsigned)E) {  // caller error: treated as dropped
                slot[a] = -1;
                continue;
            }
            const int64_t pos = (int64_t)wbase[wave][e] + rank[c];
            if (pos < C) {
                slot[a] = (int32_t)(e * C + pos);
                slot_token[e * C + pos] = (int32_t)(a / k);
            } else {
                slot[a] = -1;
            }
        }
    }
    // rows past kept[e] carry no token
    const int64_t total = (int64_t)E * C;
    for (int64_t q = (int64_t)blockIdx.x * kDThreads + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * kDThreads) {
        const int64_t e = q / C, pos = q % C;
        if (pos >= kept[e]) slot_token[q] = -1;
    }
}

// Copy rows in 16-byte vectors: row_vecs vectors per row.
__global__ __launch_bounds__(kDThreads) void disp_copy_kernel(const uint4* __restrict__ x,
                                                             const int32_t* __restrict__ slot,
                                                             int64_t T, int k, int row_vecs,
                                                             uint4* __restrict__ x_disp) {
    const int64_t t0 = (int64_t)blockIdx.x * kCopyTok;
    int nt = kCopyTok;
    if (t0 + nt > T) nt = (int)(T - t0);
    for (int v = threadIdx.x; v < row_vecs; v += kDThreads) {
        uint4 buf[kCopyTok];
#pragma unroll
        for (int i = 0; i < kCopyTok; ++i)
            if (i < nt) buf[i] = x[(t0 + i) * row_vecs + v];
#pragma unroll
        for (int i = 0; i < kCopyTok; ++i) {
            if (i < nt) {
                for (int j = 0; j < k; ++j) {
                    const int s = slot[(t0 + i) * k + j];
                    if (s >= 0) x_disp[(int64_t)s * row_vecs + v] = buf[i];
                }
            }
        }
    }
}

int disp_blocks(int64_t A) { return (int)((A + kDChunk - 1) / kDChunk); }

}  // namespace

size_t moe_dispatch_ws_bytes(int64_t T, int E, int k) {
    const int nb = disp_blocks(T * k);
    return (size_t)nb * E * 2 * sizeof(int32_t) + 256;
}

// moe_dispatch_aux: the dispatch workspace, then nb * E double partial sums
size_t moe_dispatch_aux_ws_bytes(int64_t T, int E, int k) {
    const int nb = disp_blocks(T * k);
    return ((size_t)nb * E * 2 * sizeof(int32_t) + 255) / 256 * 256 + (size_t)nb * E * sizeof(double) +
           256;
}

extern "C" moe_status_t moe_dispatch(void* stream, moe_dtype_t dtype, const void* x,
                                     const int32_t* topk_idx, int64_t T, int64_t H, int E, int k,
                                     int64_t C, void* x_disp, int32_t* slot, int32_t* slot_token,
                                     int32_t* kept, int32_t* dropped, void* ws, size_t ws_bytes) {
    if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (T < 0 || H <= 0 || E < 1 || k < 1 || k > E || C < 0) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
    if (T * k >= ((int64_t)1 << 31) || (int64_t)E * C >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    const int esz = dtype == MOE_BF16 ? 2 : 4;
    if ((H * esz) % 16) return MOE_ERR_ALIGN;
    if (!kept || !dropped) return MOE_ERR_NULL;
    if (T > 0 && (!topk_idx || !slot)) return MOE_ERR_NULL;
    if (C > 0 && !slot_token) return MOE_ERR_NULL;
    if (T > 0 && x_disp && !x) return MOE_ERR_NULL;  // x_disp NULL: indices only, no copy
    if ((x && !moe_aligned16(x)) || (x_disp && !moe_aligned16(x_disp))) return MOE_ERR_ALIGN;
    const int64_t A = T * k;
    const int nb = disp_blocks(A);
    if (nb > 0 && (!ws || ws_bytes < moe_dispatch_ws_bytes(T, E, k))) return MOE_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t* hist = static_cast<int32_t*>(ws);
    int32_t* off = hist + (size_t)nb * E;
    if (nb > 0) {
        hipLaunchKernelGGL(disp_hist_kernel, dim3(nb), dim3(kDThreads), 0, st, topk_idx, A, E, hist);
        MOE_CHECK_LAUNCH();
        hipLaunchKernelGGL(disp_scan_kernel, dim3(1), dim3(MOE_MAX_EXPERTS), 0, st, hist, nb, E, C,
                           off, kept, dropped);
        MOE_CHECK_LAUNCH();
        hipLaunchKernelGGL(disp_rank_kernel, dim3(nb), dim3(kDThreads), 0, st, topk_idx, A, E, k, C,
                           off, kept, slot, slot_token);
        MOE_CHECK_LAUNCH();
    } else {
        // no assignments: kept = 0, dropped = 0, every row is empty
        hipLaunchKernelGGL(disp_scan_kernel, dim3(1), dim3(MOE_MAX_EXPERTS), 0, st, hist, 0, E, C,
                           off, kept, dropped);
        MOE_CHECK_LAUNCH();
        if (C > 0) {
            hipLaunchKernelGGL(disp_rank_kernel, dim3(1), dim3(kDThreads), 0, st, topk_idx,
                               (int64_t)0, E, k, C, off, kept, slot, slot_token);
            MOE_CHECK_LAUNCH();
        }
    }
    if (T > 0 && C > 0 && x_disp) {
        const int row_vecs = (int)(H * esz / 16);
        const int64_t grid = (T + kCopyTok - 1) / kCopyTok;
        hipLaunchKernelGGL(disp_copy_kernel, dim3((unsigned)grid), dim3(kDThreads), 0, st,
                           static_cast<const uint4*>(x), slot, T, k, row_vecs,
                           static_cast<uint4*>(x_disp));
        MOE_CHECK_LAUNCH();
    }
    return MOE_OK;
}

namespace {

// Dispatch and the load-balancing statistics in one pass over the routing;
// ws holds the per-block histograms, offsets and partial sums.
moe_status_t dispatch_aux_impl(void* stream, moe_dtype_t dtype, const void* x,
                               const int32_t* topk_idx, const float* probs, int64_t T, int64_t H,
                               int E, int k, int64_t C, float alpha, void* x_disp, int32_t* slot,
                               int32_t* slot_token, int32_t* kept, int32_t* dropped,
                               int32_t* counts, float* f, float* p, float* l_aux, void* ws,
                               size_t ws_bytes) {
    if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (T < 0 || H <= 0 || E < 1 || k < 1 || k > E || C < 0) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
    if (T * k >= ((int64_t)1 << 31) || (int64_t)E * C >= ((int64_t)1 << 31) ||
        T * E >= ((int64_t)1 << 31))
        return MOE_ERR_UNSUPPORTED;
    const int esz = dtype == MOE_BF16 ? 2 : 4;
    if ((H * esz) % 16) return MOE_ERR_ALIGN;
    if (!kept || !dropped || !counts || !f || !p || !l_aux) return MOE_ERR_NULL;
    if (T > 0 && (!topk_idx || !slot || !probs)) return MOE_ERR_NULL;
    if (C > 0 && !slot_token) return MOE_ERR_NULL;
    if (T > 0 && x_disp && !x) return MOE_ERR_NULL;  // x_disp NULL: indices only, no copy
    if ((x && !moe_aligned16(x)) || (x_disp && !moe_aligned16(x_disp))) return MOE_ERR_ALIGN;
    if (!ws || ws_bytes < moe_dispatch_aux_ws_bytes(T, E, k)) return MOE_ERR_WORKSPACE;
    if (!moe_aligned16(ws)) return MOE_ERR_ALIGN;
    const int64_t A = T * k;
    const int nb = disp_blocks(A);
    hipStream_t st = static_cast<hipStream_t>(stream);
    int32_t* hist = static_cast<int32_t*>(ws);
    int32_t* off = hist + (size_t)nb * E;
    double* psum = reinterpret_cast<double*>(static_cast<unsigned char*>(ws) +
                                             ((size_t)nb * E * 2 * sizeof(int32_t) + 255) / 256 * 256);
    if (nb > 0) {
        hipLaunchKernelGGL(disp_hist_aux_kernel, dim3(nb), dim3(kDThreads), 0, st, topk_idx, probs,
                           A, E, k, hist, psum);
        MOE_CHECK_LAUNCH();
    }
    hipLaunchKernelGGL(disp_scan_aux_kernel, dim3(1), dim3(kScanThreads), 0, st, hist, psum, nb, E,
                       C, T, k, alpha, off, kept, dropped, counts, f, p, l_aux);
    MOE_CHECK_LAUNCH();
    if (nb > 0 || C > 0) {
        hipLaunchKernelGGL(disp_rank_kernel, dim3(nb > 0 ? nb : 1), dim3(kDThreads), 0, st,
                           topk_idx, A, E, k, C, off, kept, slot, slot_token);
        MOE_CHECK_LAUNCH();
    }
    if (T > 0 && C > 0 && x_disp) {
        const int row_vecs = (int)(H * esz / 16);
        const int64_t grid = (T + kCopyTok - 1) / kCopyTok;
        hipLaunchKernelGGL(disp_copy_kernel, dim3((unsigned)grid), dim3(kDThreads), 0, st,
                           static_cast<const uint4*>(x), slot, T, k, row_vecs,
                           static_cast<uint4*>(x_disp));
        MOE_CHECK_LAUNCH();
    }
    return MOE_OK;
}

// The workspace of moe_dispatch_aux_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it only stands for the symbol); it
// uses the device address that hipGetSymbolAddress returns for the current
// device, looked up once per device.
constexpr size_t kNoallocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (nullptr if it cannot be had).
void* noalloc_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" moe_status_t moe_dispatch_aux(void* stream, moe_dtype_t dtype, const void* x,
                                         const int32_t* topk_idx, const float* probs, int64_t T,
                                         int64_t H, int E, int k, int64_t C, float alpha,
                                         void* x_disp, int32_t* slot, int32_t* slot_token,
                                         int32_t* kept, int32_t* dropped, int32_t* counts,
                                         float* f, float* p, float* l_aux, void* ws,
                                         size_t ws_bytes) {
    return dispatch_aux_impl(stream, dtype, x, topk_idx, probs, T, H, E, k, C, alpha, x_disp, slot,
                             slot_token, kept, dropped, counts, f, p, l_aux, ws, ws_bytes);
}

extern "C" moe_status_t moe_dispatch_aux_noalloc(void* stream, moe_dtype_t dtype, const void* x,
                                                 const int32_t* topk_idx, const float* probs,
                                                 int64_t T, int64_t H, int E, int k, int64_t C,
                                                 float alpha, void* x_disp, int32_t* slot,
                                                 int32_t* slot_token, int32_t* kept,
                                                 int32_t* dropped, int32_t* counts, float* f,
                                                 float* p, float* l_aux) {
    if (T >= 0 && E >= 1 && E <= MOE_MAX_EXPERTS && k >= 1 && k <= MOE_MAX_TOPK &&
        T * k < ((int64_t)1 << 31) && moe_dispatch_aux_ws_bytes(T, E, k) > kNoallocScratchBytes)
        return MOE_ERR_UNSUPPORTED;  // the static workspace is too small for this call
    void* ws = noalloc_scratch();
    if (!ws) return MOE_ERR_LAUNCH;
    return dispatch_aux_impl(stream, dtype, x, topk_idx, probs, T, H, E, k, C, alpha, x_disp, slot,
                             slot_token, kept, dropped, counts, f, p, l_aux, ws,
                             kNoallocScratchBytes);
}
