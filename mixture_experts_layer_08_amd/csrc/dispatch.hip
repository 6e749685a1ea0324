// Capacity-bounded dispatch of token copies into per-expert row buffers.
//
// [P2] MoE basics page (dpshk.com/news/6005940) section 2.4: each expert
//      accepts at most C = ceil(tokens / experts * cf) rows; the excess is
//      dropped.
// [P1] LLaMA4-MoE guide (dpshk.com/news/5809432) section 2.4: group the
//      flattened [T, k] assignments by expert id (a stable sort), then run
//      each expert on its contiguous group.
// moe_dispatch_aux also produces the load-balancing statistics ([P2]
// section 2.3, [P1] section 3.2): counts, f = counts / (T k), P = the mean
// router probability, L_aux = alpha E sum_e f P.
//
// The stable sort is a counting sort in one launch (plus the row copy, when
// asked for).  Up to 4096 assignments one workgroup does it all
// (disp_small_kernel).  Above that, at most 64 blocks: block b takes a
// ticket from an arrival counter (so every block with a smaller ticket has
// already started) and owns assignments [b m 512, (b + 1) m 512) in (t, j)
// order, m = ceil(T k / 32768):
//  1. each wave walks its 64 m assignments 64 at a time; a ballot per
//     distinct expert gives each lane its rank among earlier same-expert
//     lanes and the wave's running count per expert;
//  2. the block publishes its count per expert (and, for the statistics,
//     its fp64 sum of the router probabilities) as two 64-bit words, each
//     with a flag bit, so a word is read whole or not at all, and adds up
//     the count words of every earlier block, waiting on any not yet
//     published: its first row per expert.  Blocks publish before they
//     read, and wait only on earlier tickets, so every wait ends; there is
//     no chain of inclusive prefixes, so no block waits for more than one
//     round of loads after its predecessors' histograms (at most 64
//     blocks: the reads are at most 64 x E words);
//  3. slot, slot_token follow from first row + in-block offset + rank;
//  4. the last block to arrive (a second counter) totals the counts (and,
//     for the statistics, the blocks' fp64 probability sums in block order:
//     deterministic), writes kept, dropped, counts, f, P, L_aux, marks the
//     rows past kept[e] empty, and clears the counters and the words.
// Every value that crosses blocks travels in a flagged word that its reader
// waits on, so the arrival counter needs no release / acquire ordering (with
// it, and the sums as plain stores: 0.4-1.4 us more per call at 8192-65536
// assignments).  The workspace must be zero before its first use and every
// call leaves it zero again.  The row copy (x_disp) is a separate
// token-major launch with many blocks: bandwidth-bound.
#include "moe_common.h"

#include <mutex>

namespace {

constexpr int kOThreads = 512;               // 8 waves per block
constexpr int kOWaves = kOThreads / 64;
constexpr int kOMaxBlocks = 64;
constexpr int kORegPasses = 8;
constexpr unsigned long long kPublished = 1ull << 63;  // flag of a published word
constexpr int kSpinLimit = 1 << 20;          // ~1 s: only a workspace that was not zero gets there
constexpr int kCopyTok = 8;                  // tokens per copy block
constexpr size_t kHeaderBytes = 256;         // two arrival counters

// One per (block, expert), both words flagged when published: word = the
// block's row count for the expert (bits 32..62) and the low half of its
// fp64 sum of the router probabilities of its tokens for that expert (bits
// 0..31); hi = the high half of that sum (bits 0..31).
struct DispCell {
    unsigned long long word;
    unsigned long long hi;
};
__device__ __forceinline__ int word_count(unsigned long long w) { return (int)((w >> 32) & 0x7fffffffu); }

struct DispGeom {
    int nb;  // blocks
    int m;   // 512-assignment passes per block
};

DispGeom disp_geom(int64_t A) {
    if (A <= 0) return {0, 1};
    const int64_t per = (int64_t)kOThreads * kOMaxBlocks;
    const int64_t m = (A + per - 1) / per;
    const int64_t span = m * kOThreads;
    return {(int)((A + span - 1) / span), (int)m};
}

enum : int { kMaps = 0, kMapsStats = 1, kStats = 2 };

struct OnePassArgs {
    const int32_t* idx;
    const float* probs;
    int64_t A, T, C;
    int E, k, nb, m;
    bool vec4;  // probs rows read as float4 (E a multiple of 4, 16-byte aligned)
    float alpha;
    int32_t *slot, *slot_token, *kept, *dropped, *counts;
    float *f, *p, *l_aux;
    unsigned int* hdr;  // [0] block tickets, [1] arrivals
    DispCell* cell;     // [nb][E]
};

__device__ __forceinline__ unsigned long long ld_word(const unsigned long long* q) {
    return __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_word(unsigned long long* q, unsigned long long v) {
    __hip_atomic_store(q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A published word (spins until its flag is set; gives up after kSpinLimit
// tries, which only a workspace that was not zero reaches, and then returns
// whatever the word holds).
__device__ __forceinline__ unsigned long long published_word(const unsigned long long* q) {
    unsigned long long w = ld_word(q);
    for (int i = 0; !(w & kPublished) && i < kSpinLimit; ++i) {
        __builtin_amdgcn_s_sleep(1);
        w = ld_word(q);
    }
    return w;
}

// Sum over tokens t = t0, t0 + step, ... < t1 of probs[t, e] in token order
// (fp64), eight loads in flight.
__device__ __forceinline__ double column_sum(const float* __restrict__ probs, int64_t t0, int64_t t1,
                                             int step, int E, int e) {
    double s = 0.0;
    for (int64_t t = t0; t < t1; t += (int64_t)8 * step) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t tt = t + (int64_t)u * step;
            v[u] = tt < t1 ? probs[tt * E + e] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (t + (int64_t)u * step < t1) s += (double)v[u];
    }
    return s;
}

// Fixed-order fp64 sums over tokens [t0, t1) of probs[t, e] for every e, by
// NT threads: thread (r, g) takes tokens t0 + r, t0 + r + rows, ... in order,
// for the four columns 4g..4g+3 with 16-byte loads when vec4 (E a multiple
// of 4, probs 16-byte aligned), else for column e alone; part (LDS, 5 NT
// doubles) holds each thread's sums, then NT / E threads per column add runs
// of consecutive rows, and out[e] (LDS) is the sum of those runs in order.
// Every thread must call it; out is ready after a barrier.
template <int NT>
__device__ void block_prob_sums(const float* __restrict__ probs, int64_t t0, int64_t t1, int E,
                                bool vec4, double* part, double* out) {
    const int tid = threadIdx.x;
    int rows;
    if (vec4) {
        const int G = E / 4;
        rows = NT / G;
        const int r = tid / G, g = tid % G;
        if (r < rows) {
            double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
            for (int64_t t = t0 + r; t < t1; t += (int64_t)8 * rows) {
                float4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int64_t tt = t + (int64_t)u * rows;
                    v[u] = tt < t1 ? *reinterpret_cast<const float4*>(probs + tt * E + 4 * g)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (t + (int64_t)u * rows < t1) {
                        s0 += (double)v[u].x;
                        s1 += (double)v[u].y;
                        s2 += (double)v[u].z;
                        s3 += (double)v[u].w;
                    }
            }
            double* q = part + r * E + 4 * g;
            q[0] = s0;
            q[1] = s1;
            q[2] = s2;
            q[3] = s3;
        }
    } else {
        rows = NT / E;
        const int r = tid / E, e = tid % E;
        if (r < rows) part[r * E + e] = column_sum(probs, t0 + r, t1, rows, E, e);
    }
    if (t1 - t0 < rows) rows = t1 > t0 ? (int)(t1 - t0) : 0;  // rows holding a token
    __syncthreads();
    double* run = part + 4 * NT;  // [Q][E]
    const int Q = NT / E, RQ = (rows + Q - 1) / Q;
    {
        const int q = tid / E, e = tid % E;
        if (q < Q) {
            double acc = 0.0;
            for (int rr = q * RQ; rr < rows && rr < (q + 1) * RQ; ++rr) acc += part[rr * E + e];
            run[q * E + e] = acc;
        }
    }
    __syncthreads();
    if (tid < E) {
        double acc = 0.0;
        for (int q = 0; q < Q; ++q) acc += run[q * E + tid];
        out[tid] = acc;
    }
}

// Adds the counts of cells [0, n) into cnt[cell mod E]: eight word loads in
// flight per thread, then a wait only on words not yet published.
constexpr int kLoadBatch = 8;
__device__ __forceinline__ void add_published(const DispCell* cell, int n, int E, int* cnt) {
    for (int q0 = threadIdx.x; q0 < n; q0 += kLoadBatch * kOThreads) {
        unsigned long long w[kLoadBatch];
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
            const int q = q0 + u * kOThreads;
            w[u] = q < n ? ld_word(&cell[q].word) : kPublished;
        }
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
            const int q = q0 + u * kOThreads;
            if (q < n) {
                const int c = word_count((w[u] & kPublished) ? w[u] : published_word(&cell[q].word));
                atomicAdd(&cnt[q % E], c);
            }
        }
    }
}

// Rank of this lane's assignment among the earlier lanes of the wave with the
// same expert, plus `run` (lane e: the running row count of expert e, which
// is updated).  One uniform iteration per distinct expert among the lanes;
// the leader's expert and the running count are read with readlane.
__device__ __forceinline__ int wave_rank(int e, bool ok, int& run, int lane, uint64_t lt_mask) {
    int r = 0;
    uint64_t rem = __ballot(ok);
    while (rem) {
        const int leader = __builtin_ctzll(rem);
        const int ee = __builtin_amdgcn_readlane(e, leader);
        const uint64_t msk = __ballot(ok && e == ee);
        const int base = __builtin_amdgcn_readlane(run, ee);
        if (ok && e == ee) r = base + __popcll(msk & lt_mask);
        run += (lane == ee) ? __popcll(msk) : 0;
        rem &= ~msk;
    }
    return r;
}

__device__ __forceinline__ void put_slot(const OnePassArgs& a, int64_t i, int e, int64_t pos) {
    if (pos >= 0 && pos < a.C) {
        a.slot[i] = (int32_t)(e * a.C + pos);
        a.slot_token[e * a.C + pos] = (int32_t)(i / a.k);
    } else {
        a.slot[i] = -1;
    }
}

template <int MODE>
__global__ __launch_bounds__(kOThreads) void disp_onepass_kernel(OnePassArgs a) {
    __shared__ int s_b, s_last;
    __shared__ int tot[kOWaves][MOE_MAX_EXPERTS];   // per wave, then its in-block offset
    __shared__ int first[MOE_MAX_EXPERTS];          // rows of earlier blocks / totals
    __shared__ int keptL[MOE_MAX_EXPERTS];
    __shared__ double colsum[5 * kOThreads];
    __shared__ double bsum[MOE_MAX_EXPERTS];
    __shared__ double fp[MOE_MAX_EXPERTS];
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int E = a.E;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (tid < E) first[tid] = 0;

    if (a.nb > 0) {
        if (tid == 0)
            s_b = (int)__hip_atomic_fetch_add(&a.hdr[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int b = s_b;
        if (b >= a.nb) return;  // only with a workspace that was not zero
        const int64_t span = (int64_t)a.m * kOThreads;
        const int64_t a0 = (int64_t)b * span;
        const int64_t a1 = a0 + span < a.A ? a0 + span : a.A;
        const int64_t wa0 = a0 + (int64_t)wave * a.m * 64;

        // 1. ranks and per-wave counts, eight 64-assignment passes' loads in
        // flight at a time (up to eight passes the ranks stay in registers)
        int run = 0;
        int ek[kORegPasses], rk[kORegPasses];
        for (int c0 = 0; c0 < a.m; c0 += kORegPasses) {
#pragma unroll
            for (int u = 0; u < kORegPasses; ++u) {
                const int64_t i = wa0 + (int64_t)(c0 + u) * 64 + lane;
                ek[u] = (c0 + u < a.m && i < a1) ? a.idx[i] : -1;
            }
#pragma unroll
            for (int u = 0; u < kORegPasses; ++u)
                if (c0 + u < a.m)
                    rk[u] = wave_rank(ek[u], (unsigned)ek[u] < (unsigned)E, run, lane, lt_mask);
        }
        if (lane < E) tot[wave][lane] = run;
        if (MODE != kMaps)  // probability sums of the block's tokens (a barrier inside)
            block_prob_sums<kOThreads>(a.probs, (a0 + a.k - 1) / a.k, (a1 + a.k - 1) / a.k, E,
                                       a.vec4, colsum, bsum);
        __syncthreads();
        if (tid < E) {  // wave 0: in-block offsets, the block's count, publish
            int acc = 0;
            for (int w = 0; w < kOWaves; ++w) {
                const int c = tot[w][tid];
                tot[w][tid] = acc;
                acc += c;
            }
            // with the statistics, the block's probability sum goes with its
            // count (block_prob_sums' thread tid wrote bsum[tid])
            const unsigned long long ps =
                MODE != kMaps ? (unsigned long long)__double_as_longlong(bsum[tid]) : 0ull;
            st_word(&a.cell[(size_t)b * E + tid].word,
                    kPublished | ((unsigned long long)acc << 32) | (ps & 0xffffffffull));
            if (MODE != kMaps) st_word(&a.cell[(size_t)b * E + tid].hi, kPublished | (ps >> 32));
        }
        // 2. rows taken by earlier blocks: every earlier block's word
        if (MODE != kStats) add_published(a.cell, b * E, E, first);
        __syncthreads();
        // 3. the maps
        if (MODE != kStats) {
            if (a.m <= kORegPasses) {
#pragma unroll
                for (int u = 0; u < kORegPasses; ++u) {
                    const int64_t i = wa0 + (int64_t)u * 64 + lane;
                    if (u < a.m && i < a1) {
                        const int e = ek[u];
                        if ((unsigned)e < (unsigned)E)
                            put_slot(a, i, e, (int64_t)first[e] + tot[wave][e] + rk[u]);
                        else
                            a.slot[i] = -1;  // caller error: treated as dropped
                    }
                }
            } else {  // ranks again, now from the wave's first rows
                int run2 = lane < E ? first[lane] + tot[wave][lane] : 0;
                for (int c = 0; c < a.m; ++c) {
                    const int64_t i = wa0 + (int64_t)c * 64 + lane;
                    const bool valid = i < a1;
                    const int e = valid ? a.idx[i] : -1;
                    const bool ok = valid && (unsigned)e < (unsigned)E;
                    const int pos = wave_rank(e, ok, run2, lane, lt_mask);
                    if (ok)
                        put_slot(a, i, e, pos);
                    else if (valid)
                        a.slot[i] = -1;
                }
            }
        }
        // 4. arrival (relaxed: the last block waits on the flags of the
        // words it reads)
        if (tid == 0) {
            const unsigned old =
                __hip_atomic_fetch_add(&a.hdr[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = old == (unsigned)a.nb - 1;
        }
        __syncthreads();
        if (!s_last) return;
        if (tid < E) first[tid] = 0;
        __syncthreads();
    } else {
        __syncthreads();
    }

    // The last block: totals, statistics, empty rows, clearing.
    const int nb = a.nb;
    add_published(a.cell, nb * E, E, first);
    if (MODE != kMaps) {  // thread (r, e) sums stripe r of the blocks in order
        const int rows = kOThreads / E;
        const int r = tid / E, e = tid % E;
        const int S = (nb + rows - 1) / rows;
        const int j1 = (r + 1) * S < nb ? (r + 1) * S : nb;
        double s = 0.0;
        if (r < rows)
            for (int j0 = r * S; j0 < j1; j0 += kLoadBatch) {
                unsigned long long lo[kLoadBatch], hi[kLoadBatch];
#pragma unroll
                for (int u = 0; u < kLoadBatch; ++u) {
                    const DispCell* c = &a.cell[(size_t)(j0 + u) * E + e];
                    lo[u] = j0 + u < j1 ? ld_word(&c->word) : kPublished;
                    hi[u] = j0 + u < j1 ? ld_word(&c->hi) : kPublished;
                }
#pragma unroll
                for (int u = 0; u < kLoadBatch; ++u)
                    if (j0 + u < j1) {
                        const DispCell* c = &a.cell[(size_t)(j0 + u) * E + e];
                        if (!(lo[u] & kPublished)) lo[u] = published_word(&c->word);
                        if (!(hi[u] & kPublished)) hi[u] = published_word(&c->hi);
                        s += __longlong_as_double((long long)(((hi[u] & 0xffffffffull) << 32) |
                                                              (lo[u] & 0xffffffffull)));
                    }
            }
        colsum[tid] = s;
    }
    __syncthreads();
    if (tid < E) {
        const int64_t run = first[tid];
        const int kp = (int)(run < a.C ? run : a.C);
        keptL[tid] = kp;
        if (MODE != kStats) a.kept[tid] = kp;
        if (MODE != kMaps) {
            const int rows = kOThreads / E;
            double pt = 0.0;
            for (int rr = 0; rr < rows; ++rr) pt += colsum[rr * E + tid];
            const double fe = a.T > 0 ? (double)run / ((double)a.T * a.k) : 0.0;
            const double pe = a.T > 0 ? pt / (double)a.T : 0.0;
            a.counts[tid] = (int32_t)run;
            a.f[tid] = (float)fe;
            a.p[tid] = (float)pe;
            fp[tid] = fe * pe;
        }
    }
    __syncthreads();
    if (tid == 0) {
        if (MODE != kStats) {
            int64_t d = 0;
            for (int e = 0; e < E; ++e) d += first[e] - keptL[e];
            *a.dropped = (int32_t)d;
        }
        if (MODE != kMaps) {
            double acc = 0.0;
            for (int e = 0; e < E; ++e) acc += fp[e];
            *a.l_aux = (float)((double)a.alpha * E * acc);
        }
    }
    if (MODE != kStats)  // rows past kept[e] carry no token
        for (int e = 0; e < E; ++e)
            for (int64_t q = keptL[e] + tid; q < a.C; q += kOThreads) a.slot_token[e * a.C + q] = -1;
    if (nb > 0) {
        for (int q = tid; q < nb * E; q += kOThreads) {
            st_word(&a.cell[q].word, 0ull);
            st_word(&a.cell[q].hi, 0ull);
        }
        if (tid == 0) {
            __hip_atomic_store(&a.hdr[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.hdr[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Up to 4096 assignments one workgroup does the whole sort with no global
// synchronisation: 16 waves each rank a contiguous run of at most 4
// 64-assignment passes (all loads issued first, ranks kept in registers),
// an LDS scan over the waves gives each wave's first rows, then the maps,
// kept, dropped and (MODE kMapsStats) the statistics, as in the one-pass
// kernel's last block.
constexpr int kSThreads = 1024;
constexpr int kSWaves = kSThreads / 64;
constexpr int kSMaxPasses = 4;
constexpr int64_t kSmallMaxA = (int64_t)kSWaves * kSMaxPasses * 64;

template <int MODE>
__global__ __launch_bounds__(kSThreads) void disp_small_kernel(OnePassArgs a) {
    __shared__ int tot[kSWaves][MOE_MAX_EXPERTS];
    __shared__ int cnt[MOE_MAX_EXPERTS];
    __shared__ int keptL[MOE_MAX_EXPERTS];
    __shared__ double colsum[5 * kSThreads];
    __shared__ double psum[MOE_MAX_EXPERTS];
    __shared__ double fp[MOE_MAX_EXPERTS];
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
    const int E = a.E;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int np = (int)((a.A + kSWaves * 64 - 1) / (kSWaves * 64));  // passes per wave
    const int64_t wa0 = (int64_t)wave * np * 64;
    // per pass: the expert id, then (rank << 7) | expert, or -1 for an id
    // outside [0, E) (one register per pass)
    int ek[kSMaxPasses];
#pragma unroll
    for (int u = 0; u < kSMaxPasses; ++u) {
        const int64_t i = wa0 + (int64_t)u * 64 + lane;
        ek[u] = (u < np && i < a.A) ? a.idx[i] : -1;
    }
    if (MODE != kMaps)  // a barrier inside
        block_prob_sums<kSThreads>(a.probs, 0, a.T, E, a.vec4, colsum, psum);
    int run = 0;
#pragma unroll
    for (int u = 0; u < kSMaxPasses; ++u)
        if (u < np) {
            const bool ok = (unsigned)ek[u] < (unsigned)E;
            const int r = wave_rank(ek[u], ok, run, lane, lt_mask);
            ek[u] = ok ? (r << 7) | ek[u] : -1;
        }
    if (lane < E) tot[wave][lane] = run;
    __syncthreads();
    if (tid < E) {
        int acc = 0;
        for (int w = 0; w < kSWaves; ++w) {
            const int c = tot[w][tid];
            tot[w][tid] = acc;
            acc += c;
        }
        const int kp = (int)(acc < a.C ? acc : a.C);
        cnt[tid] = acc;
        keptL[tid] = kp;
        a.kept[tid] = kp;
        if (MODE != kMaps) {
            const double pt = psum[tid];
            const double fe = a.T > 0 ? (double)acc / ((double)a.T * a.k) : 0.0;
            const double pe = a.T > 0 ? pt / (double)a.T : 0.0;
            a.counts[tid] = acc;
            a.f[tid] = (float)fe;
            a.p[tid] = (float)pe;
            fp[tid] = fe * pe;
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kSMaxPasses; ++u) {
        const int64_t i = wa0 + (int64_t)u * 64 + lane;
        if (u < np && i < a.A) {
            if (ek[u] >= 0) {
                const int e = ek[u] & 127;
                put_slot(a, i, e, (int64_t)tot[wave][e] + (ek[u] >> 7));
            } else {
                a.slot[i] = -1;  // caller error: treated as dropped
            }
        }
    }
    if (tid == 0) {
        int64_t d = 0;
        for (int e = 0; e < E; ++e) d += cnt[e] - keptL[e];
        *a.dropped = (int32_t)d;
        if (MODE != kMaps) {
            double acc = 0.0;
            for (int e = 0; e < E; ++e) acc += fp[e];
            *a.l_aux = (float)((double)a.alpha * E * acc);
        }
    }
    for (int e = 0; e < E; ++e)  // rows past kept[e] carry no token
        for (int64_t q = keptL[e] + tid; q < a.C; q += kSThreads) a.slot_token[e * a.C + q] = -1;
}

// Copy rows in 16-byte vectors: row_vecs vectors per row.  Each thread reads
// one vector of each of the block's kCopyTok rows (all loads in flight), then
// writes it to every kept slot of its token; the slots are wave-uniform.
__global__ __launch_bounds__(256) void disp_copy_kernel(const uint4* __restrict__ x,
                                                        const int32_t* __restrict__ slot, int64_t T,
                                                        int k, int row_vecs,
                                                        uint4* __restrict__ x_disp) {
    const int64_t t0 = (int64_t)blockIdx.x * kCopyTok;
    const int nt = t0 + kCopyTok > T ? (int)(T - t0) : kCopyTok;
    for (int v = threadIdx.x; v < row_vecs; v += 256) {
        uint4 buf[kCopyTok];
#pragma unroll
        for (int i = 0; i < kCopyTok; ++i)
            if (i < nt) buf[i] = x[(t0 + i) * row_vecs + v];
#pragma unroll
        for (int i = 0; i < kCopyTok; ++i) {
            if (i < nt) {
                const uint4 val = buf[i];
                for (int j = 0; j < k; ++j) {
                    const int s = slot[(t0 + i) * k + j];
                    if (s >= 0) x_disp[(int64_t)s * row_vecs + v] = val;
                }
            }
        }
    }
}

// Enqueues the one-pass kernel (and the row copy).  Arguments already checked.
moe_status_t onepass_launch(int mode, hipStream_t st, const int32_t* idx, const float* probs,
                            int64_t T, int E, int k, int64_t C, float alpha, int32_t* slot,
                            int32_t* slot_token, int32_t* kept, int32_t* dropped, int32_t* counts,
                            float* f, float* p, float* l_aux, void* ws) {
    OnePassArgs a;
    const int64_t A = T * k;
    const DispGeom g = disp_geom(A);
    a.idx = idx;
    a.probs = probs;
    a.A = A;
    a.T = T;
    a.C = C;
    a.E = E;
    a.k = k;
    a.nb = g.nb;
    a.m = g.m;
    a.vec4 = probs && E % 4 == 0 && moe_aligned16(probs);
    a.alpha = alpha;
    a.slot = slot;
    a.slot_token = slot_token;
    a.kept = kept;
    a.dropped = dropped;
    a.counts = counts;
    a.f = f;
    a.p = p;
    a.l_aux = l_aux;
    a.hdr = static_cast<unsigned int*>(ws);
    a.cell = ws ? reinterpret_cast<DispCell*>(static_cast<unsigned char*>(ws) + kHeaderBytes)
                : nullptr;
    const dim3 grid(g.nb > 0 ? g.nb : 1);
    if (mode != kStats && A <= kSmallMaxA) {
        if (mode == kMaps)
            hipLaunchKernelGGL(disp_small_kernel<kMaps>, dim3(1), dim3(kSThreads), 0, st, a);
        else
            hipLaunchKernelGGL(disp_small_kernel<kMapsStats>, dim3(1), dim3(kSThreads), 0, st, a);
    } else if (mode == kMaps)
        hipLaunchKernelGGL(disp_onepass_kernel<kMaps>, grid, dim3(kOThreads), 0, st, a);
    else if (mode == kMapsStats)
        hipLaunchKernelGGL(disp_onepass_kernel<kMapsStats>, grid, dim3(kOThreads), 0, st, a);
    else
        hipLaunchKernelGGL(disp_onepass_kernel<kStats>, grid, dim3(kOThreads), 0, st, a);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

moe_status_t copy_launch(hipStream_t st, const void* x, const int32_t* slot, int64_t T, int64_t H,
                         int esz, int k, void* x_disp) {
    const int row_vecs = (int)(H * esz / 16);
    const int64_t grid = (T + kCopyTok - 1) / kCopyTok;
    hipLaunchKernelGGL(disp_copy_kernel, dim3((unsigned)grid), dim3(256), 0, st,
                       static_cast<const uint4*>(x), slot, T, k, row_vecs,
                       static_cast<uint4*>(x_disp));
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

}  // namespace

// One workspace serves moe_aux_stats, moe_dispatch and moe_dispatch_aux: a
// header of two counters, then one 16-byte cell per (block, expert).
size_t moe_dispatch_ws_bytes(int64_t T, int E, int k) {
    const DispGeom g = disp_geom(T * k);
    return kHeaderBytes + (size_t)g.nb * E * sizeof(DispCell);
}
size_t moe_dispatch_aux_ws_bytes(int64_t T, int E, int k) { return moe_dispatch_ws_bytes(T, E, k); }

// moe_aux_stats above one workgroup's size: the one-pass kernel without the
// maps (aux_stats.hip).
moe_status_t moe_stats_onepass(void* stream, const int32_t* idx, const float* probs, int64_t T,
                               int E, int k, float alpha, int32_t* counts, float* f, float* p,
                               float* l_aux, void* ws) {
    return onepass_launch(kStats, static_cast<hipStream_t>(stream), idx, probs, T, E, k, 0, alpha,
                          nullptr, nullptr, nullptr, nullptr, counts, f, p, l_aux, ws);
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
    if (T > 0 && (!ws || ws_bytes < moe_dispatch_ws_bytes(T, E, k))) return MOE_ERR_WORKSPACE;
    if (ws && !moe_aligned16(ws)) return MOE_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    moe_status_t s = onepass_launch(kMaps, st, topk_idx, nullptr, T, E, k, C, 0.f, slot, slot_token,
                                    kept, dropped, nullptr, nullptr, nullptr, nullptr, ws);
    if (s != MOE_OK) return s;
    if (T > 0 && C > 0 && x_disp) return copy_launch(st, x, slot, T, H, esz, k, x_disp);
    return MOE_OK;
}

namespace {

// Dispatch and the load-balancing statistics in one pass over the routing.
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
    hipStream_t st = static_cast<hipStream_t>(stream);
    moe_status_t s = onepass_launch(kMapsStats, st, topk_idx, probs, T, E, k, C, alpha, slot,
                                    slot_token, kept, dropped, counts, f, p, l_aux, ws);
    if (s != MOE_OK) return s;
    if (T > 0 && C > 0 && x_disp) return copy_launch(st, x, slot, T, H, esz, k, x_disp);
    return MOE_OK;
}

// The workspace of moe_dispatch_aux_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it only stands for the symbol); it
// uses the device address that hipGetSymbolAddress returns for the current
// device, looked up once per device.  The array starts zeroed (static
// storage) and every call leaves it zero, as the workspace contract asks.
constexpr size_t kNoallocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static_assert(kHeaderBytes + (size_t)kOMaxBlocks * MOE_MAX_EXPERTS * sizeof(DispCell) <=
                  kNoallocScratchBytes,
              "every accepted shape's workspace fits the static array");
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

__global__ __launch_bounds__(256) void disp_zero_kernel(unsigned long long* q, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) q[i] = 0ull;
}

// The current device's address of `scratch` (nullptr if it cannot be had).
// On a device's first call it is also cleared on the caller's stream (unless
// that stream is being captured), in case the loader left it dirty.
void* noalloc_scratch(hipStream_t st) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone) {
            const int n = (int)(kNoallocScratchBytes / 8);
            hipLaunchKernelGGL(disp_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, st,
                               static_cast<unsigned long long*>(ptr), n);
            if (hipGetLastError() != hipSuccess) return nullptr;
        }
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
    void* ws = noalloc_scratch(static_cast<hipStream_t>(stream));
    if (!ws) return MOE_ERR_LAUNCH;
    return dispatch_aux_impl(stream, dtype, x, topk_idx, probs, T, H, E, k, C, alpha, x_disp, slot,
                             slot_token, kept, dropped, counts, f, p, l_aux, ws,
                             kNoallocScratchBytes);
}
