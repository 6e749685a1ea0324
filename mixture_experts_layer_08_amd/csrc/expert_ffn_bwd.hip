// Backward of the expert FFNs as grouped GEMMs on the matrix cores.
//
// [P2] MoE basics page (dpshk.com/news/6005940) sections 2.2 and 3.1 (the
//      expert FFNs), [P5] llama-moe essay (coreui.cn/article/2610641) section
//      2.1 (SwiGLU); [P4] long-context page (2kiu.com/news/5130654) section 2
//      and [P3] Loop-MoE page (discosf.com/news/5228035) section 4 train the
//      layer, which needs these gradients.
//
// For each expert e with rows X (kept[e] of them) and output gradient dY:
//   SwiGLU  g = X W_gate, u = X W_up, h = silu(g) u, Y = h W_down
//     dh = dY W_down^T;  dg = dh u silu'(g);  du = dh silu(g)
//     dX = dg W_gate^T + du W_up^T
//     dW_down = h^T dY;  dW_gate = X^T dg;  dW_up = X^T du
//   GELU    z = X W1 + b1, h = gelu(z), Y = h W2 + b2
//     dz = (dY W2^T) gelu'(z);  dX = dz W1^T
//     dW2 = h^T dY;  dW1 = X^T dz;  db1 = sum_rows dz;  db2 = sum_rows dY
// h and g, u (or z) come from re-running the first product with its
// pre-activations saved (bf16, as the forward keeps h).
//
// Two kernel shapes, both persistent 256 x 256 tiles with 8 waves of 128 x 64
// and v_mfma_f32_32x32x16_bf16, double-buffered LDS filled by direct
// global->LDS loads, as in the forward:
//   DGRAD  rows = the expert's kept rows, K = a weight dimension.  Both
//          operands are k-contiguous (dY or dg rows; the weight read along its
//          rows, which is its transpose), staged as 128-byte LDS rows and read
//          with ds_read_b128.  Two (A, B) pairs may be chained along K
//          (dg W_gate^T + du W_up^T in one accumulation).
//   WGRAD  rows and columns = weight dimensions, K = the expert's kept rows
//          (ragged: k-rows past kept[e] read as zero).  Both operands are
//          token rows read across (h, X, dY, dg, du are m- or n-contiguous),
//          staged as 256-byte k-rows and read with ds_read_b64_tr_b16.
#include "moe_common.h"
#include "gemm_common.h"
#include "internal.h"

#include <type_traits>


namespace {

enum { SCHED_DGRAD = 0, SCHED_WGRAD = 1 };
enum { EPI_F32 = 0, EPI_DH_SWIGLU = 1, EPI_DH_GELU = 2 };

struct BwdArgs {
    const uint16_t* A0;     // DGRAD: [E][C][K] rows; WGRAD: [E][C][M] k-rows
    const uint16_t* B0;     // DGRAD: [E][N][K] (a weight read as its transpose); WGRAD: [E][C][N]
    const uint16_t* A1;     // DGRAD: second (A, B) pair chained along K, or null
    const uint16_t* B1;
    const int32_t* kept;    // [E]
    int E;
    int64_t C;
    int M;                  // WGRAD: output rows
    int N;                  // output columns
    int K;                  // DGRAD: contraction of one pair
    void* out;              // DGRAD: [E][C][N]; WGRAD: [E][M][N]; fp32 (EPI_F32) or bf16
    uint16_t* out1;         // EPI_DH_SWIGLU: du (out holds dg)
    const uint16_t* side0;  // EPI_DH_*: g (SwiGLU) or z (GELU), [E][C][N]
    const uint16_t* side1;  // EPI_DH_SWIGLU: u
    // DGRAD: split-K of the last, partly filled round of tiles (null: off)
    float* part;            // per-piece fp32 partial tiles, kBwdPartBytes each
    int smax;               // at most this many pieces per tile
};

constexpr size_t kBwdPartBytes = (size_t)kBM * kBNMax * 4;  // one fp32 tile
constexpr int kBwdSMax = 8;

// DGRAD tiles fill total / G rounds of a G-workgroup launch; when the last
// round would leave at least half of the workgroups idle, its tiles are cut
// along K into this many pieces (1: no split), each keeping two k-steps.
__device__ __forceinline__ int bwd_tail_splits(const BwdArgs& g, int total, int G, int nk) {
    const int remt = total % G;
    if (!g.part || remt == 0 || 2 * remt > G) return 1;
    int sp = G / remt;
    if (sp > g.smax) sp = g.smax;
    if (sp > kBwdSMax) sp = kBwdSMax;
    if (sp > nk / 2) sp = nk / 2;
    return sp < 1 ? 1 : sp;
}

// The schedule's per-expert row tiles and tile prefixes (one thread).  DGRAD
// (row tiles over kept[e]) puts an expert's last row tile after every other
// tile when it has at most 64 rows (thin: little MFMA work for a whole tile's
// loads), as the forward products do: the main run (s_pref, s_mt row tiles
// per expert), then the thin run (s_tpref, one row tile per expert that has
// one), so the thin tiles fall in the last, split round.
__device__ void bwd_prefix(const BwdArgs& g, bool KC, int NT, int* s_pref, int* s_mt,
                           int* s_tpref) {
    int cum = 0, tcum = 0;
    for (int e = 0; e < g.E; ++e) {
        int kp = g.kept[e];
        if (kp < 0) kp = 0;
        if (kp > g.C) kp = (int)g.C;
        const int mt_all = KC ? (kp + kBM - 1) / kBM : g.M / kBM;
        const int thin = (KC && mt_all > 0 && kp - (mt_all - 1) * kBM <= 64) ? 1 : 0;
        s_mt[e] = mt_all - thin;
        s_pref[e] = cum;
        s_tpref[e] = tcum;
        cum += (mt_all - thin) * NT;
        tcum += thin * NT;
    }
    s_pref[g.E] = cum;
    s_tpref[g.E] = tcum;
}

// Tile `logical` of the schedule above -> expert, row tile and column tile.
__device__ __forceinline__ void bwd_map_tile(int logical, const int* s_pref, const int* s_mt,
                                             const int* s_tpref, int E, int NT, int& e,
                                             int& m_tile, int& n_tile) {
    if (logical < s_pref[E]) {
        map_tile(logical, s_pref, s_mt, E, NT, e, m_tile, n_tile);
        return;
    }
    const int t = logical - s_pref[E];
    e = 0;
    while (e + 1 < E && s_tpref[e + 1] <= t) ++e;
    m_tile = s_mt[e];  // the thin tile follows the expert's main row tiles
    n_tile = t - s_tpref[e];
}

struct BTile {
    bool valid;
    int e, m0, n0, rows;    // rows: valid output rows from m0 (DGRAD: kept - m0)
    int nks, kstep_pair;    // k-steps of the tile (from kb), and of one (A, B) pair
    int kb;                 // first k-step (a piece of a split tail tile starts later)
    int pslot;              // piece of a split tail tile: tile * splits + piece; else -1
    int kept;
    i32x4_t rsA0, rsB0, rsA1, rsB1;
};

template <int SCHED, int EPI>
__global__ __launch_bounds__(kGThreads, 1) void grouped_gemm_bwd_kernel(BwdArgs g) {
    constexpr bool KC = SCHED == SCHED_DGRAD;   // both operands k-contiguous
    constexpr int kStage = 2 * kStageA;         // A 32 KB + B 32 KB
    constexpr int WM_ROWS = kBM / kWMn, WN_COLS = kBNMax / kWN;
    constexpr int TM = WM_ROWS / 32, TN = WN_COLS / 32;
    constexpr int QL = 32 / kNW;                // 1 KB loads per wave per operand per k-step
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_pref[MOE_MAX_EXPERTS + 1];
    __shared__ int s_mt[MOE_MAX_EXPERTS];
    __shared__ int s_tpref[MOE_MAX_EXPERTS + 1];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int wm = wave / kWN, wn = wave % kWN;
    const int NT = g.N / kBNMax;
    if (tid == 0) bwd_prefix(g, KC, NT, s_pref, s_mt, s_tpref);
    __syncthreads();
    const int total = __builtin_amdgcn_readfirstlane(s_pref[g.E] + s_tpref[g.E]);
    const int G = gridDim.x;
    const int xcd = blockIdx.x % 8, slot8 = blockIdx.x / 8;
    const int full = total / G;
    const int remt = total - full * G;
    // DGRAD k-steps of a whole tile (both chained pairs)
    const int nk_tile = (g.A1 ? 2 : 1) * (g.K / kBK);
    const int splits =
        KC ? __builtin_amdgcn_readfirstlane(bwd_tail_splits(g, total, G, nk_tile)) : 1;

    auto tile_at = [&](int round) {
        BTile c;
        const int pos = round == full ? (int)blockIdx.x : xcd * (G / 8) + slot8;
        int logical = round * G + pos;
        c.kb = 0;
        c.pslot = -1;
        int piece = 0;
        if (splits > 1 && round == full) {
            const int t = pos / splits;
            piece = pos - t * splits;
            logical = pos < remt * splits ? full * G + t : total;
            c.pslot = pos;
        }
        c.valid = logical < total;
        if (!c.valid) return c;
        int e, m_tile, n_tile;
        bwd_map_tile(logical, s_pref, s_mt, s_tpref, g.E, NT, e, m_tile, n_tile);
        int kept = g.kept[e];
        if (kept < 0) kept = 0;
        if (kept > g.C) kept = (int)g.C;
        c.e = __builtin_amdgcn_readfirstlane(e);
        c.kept = __builtin_amdgcn_readfirstlane(kept);
        c.m0 = __builtin_amdgcn_readfirstlane(m_tile * kBM);
        c.n0 = __builtin_amdgcn_readfirstlane(n_tile * kBNMax);
        if (KC) {
            c.rows = c.kept - c.m0;
            c.kstep_pair = g.K / kBK;
            c.nks = g.A1 ? 2 * c.kstep_pair : c.kstep_pair;
            if (c.pslot >= 0) {  // a piece: k-steps kb .. kb + nks - 1 of the tile
                c.kb = piece * c.nks / splits;
                c.nks = (piece + 1) * c.nks / splits - c.kb;
            }
            // A: the expert's rows from m0 (rows past kept read as zero);
            // B: weight rows n0.. of length K
            const size_t abytes = (size_t)c.rows * g.K * 2;
            const size_t boff = ((size_t)c.e * g.N + c.n0) * g.K;
            const size_t bbytes = (size_t)(g.N - c.n0) * g.K * 2;
            c.rsA0 = make_rsrc(g.A0 + ((size_t)c.e * g.C + c.m0) * g.K, (uint32_t)abytes);
            c.rsB0 = make_rsrc(g.B0 + boff, (uint32_t)bbytes);
            if (g.A1) {
                c.rsA1 = make_rsrc(g.A1 + ((size_t)c.e * g.C + c.m0) * g.K, (uint32_t)abytes);
                c.rsB1 = make_rsrc(g.B1 + boff, (uint32_t)bbytes);
            } else {
                c.rsA1 = c.rsA0;
                c.rsB1 = c.rsB0;
            }
        } else {
            c.rows = kBM;
            int nks = (c.kept + kBK - 1) / kBK;
            c.nks = nks < 2 ? 2 : nks;  // the k pipeline runs at least two steps
            c.kstep_pair = c.nks;
            // k-rows 0 .. kept-1 of the expert; columns m0.. / n0..; the wave's
            // 128-column half of each operand gets its own descriptor
            const int sub = (wave * QL) / 16;
            const size_t ao = (size_t)c.e * g.C * g.M + c.m0 + sub * 128;
            const size_t bo = (size_t)c.e * g.C * g.N + c.n0 + sub * 128;
            int64_t an = (int64_t)c.kept * g.M - c.m0 - sub * 128;  // elements from the base
            int64_t bn = (int64_t)c.kept * g.N - c.n0 - sub * 128;  // (none when kept = 0)
            c.rsA0 = make_rsrc(g.A0 + ao, (uint32_t)(an > 0 ? an * 2 : 0));
            c.rsB0 = make_rsrc(g.B0 + bo, (uint32_t)(bn > 0 ? bn * 2 : 0));
            c.rsA1 = c.rsA0;
            c.rsB1 = c.rsB0;
        }
        return c;
    };

    // k-contiguous operand tile (256 rows x 64 k, 128-byte rows, chunk XOR
    // swz_a(row)): load q of this wave fills tile row R = (wave*QL + q)*8 + lane/8
    const int voffK0 = (((lane % 8) ^ (lane / 16)) * 8) * 2;
    const int voffK1 = (((lane % 8) ^ (4 + lane / 16)) * 8) * 2;
    const int rowK = wave * QL * 8 + lane / 8;
    // token-row operand tile (64 k-rows x 256 columns as two 128-column
    // sub-tiles of 256-byte rows, chunk XOR swz_b(k)): load q fills k-row
    // ((wave*QL + q) % 16)*4 + lane/16 of sub-tile (wave*QL)/16
    const int chM = ((lane % 16) ^ ((lane / 16) << 2)) * 8 * 2;
    auto issue = [&](const BTile& c, int kt, int stage) {
        unsigned char* st = smem + stage * kStage;
        if (KC) {
            const bool p1 = kt >= c.kstep_pair;
            const int kk = p1 ? kt - c.kstep_pair : kt;
            const i32x4_t ra = p1 ? c.rsA1 : c.rsA0;
            const i32x4_t rb = p1 ? c.rsB1 : c.rsB0;
#pragma unroll
            for (int q = 0; q < QL; ++q) {
                const int vo = (rowK * g.K) * 2 + ((q & 1) ? voffK1 : voffK0);
                lds_dma16(ra, st + (wave * QL + q) * 1024, vo, (q * 8 * g.K + kk * kBK) * 2);
                lds_dma16(rb, st + kStageA + (wave * QL + q) * 1024, vo,
                          (q * 8 * g.K + kk * kBK) * 2);
            }
        } else {
#pragma unroll
            for (int q = 0; q < QL; ++q) {
                const int kr = ((wave * QL + q) % 16) * 4 + kt * kBK;
                lds_dma16(c.rsA0, st + (wave * QL + q) * 1024, (lane / 16) * g.M * 2 + chM,
                          kr * g.M * 2);
                lds_dma16(c.rsB0, st + kStageA + (wave * QL + q) * 1024,
                          (lane / 16) * g.N * 2 + chM, kr * g.N * 2);
            }
        }
    };

    // MFMA operand fragment (lane l: index l % 32 along rows or columns,
    // k values (l / 32)*8 .. +7 of the 16-wide slice k16)
    auto frag_kc = [&](const unsigned char* T, int r0, int k16) {
        const int row = r0 + lane % 32;
        const int phys = (k16 * 2 + lane / 32) ^ swz_a(row);
        return as_bf16x8(*reinterpret_cast<const uint4*>(T + row * 128 + phys * 16));
    };
    auto frag_mc = [&](const unsigned char* T, int c0, int k16) {
        const int sb = c0 / 128;
        const int col = c0 % 128 + ((lane / 16) % 2) * 16 + 4 * (lane % 4);
        i16x4_t v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kr = k16 * 16 + (lane / 32) * 8 + h * 4 + (lane % 16) / 4;
            const int phys = (col >> 3) ^ swz_b(kr);
            v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t*)(T + sb * 16384 + kr * 256 + phys * 16 + (col & 7) * 2));
        }
        const uint2 lo = __builtin_bit_cast(uint2, v[0]);
        const uint2 hi = __builtin_bit_cast(uint2, v[1]);
        return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
    };
    // (only the first NI 32-row blocks of the wave's A rows: the others lie
    // past the valid rows)
    auto load_frags = [&](auto ni, int stage, int kk, bf16x8_t (&af)[2][TM],
                          bf16x8_t (&bfr)[2][TN]) {
        constexpr int NI = decltype(ni)::value;
        const unsigned char* As = smem + stage * kStage;
        const unsigned char* Bs = As + kStageA;
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
            const int k16 = kk * 2 + ss;
#pragma unroll
            for (int i = 0; i < NI; ++i)
                af[ss][i] = KC ? frag_kc(As, wm * WM_ROWS + i * 32, k16)
                               : frag_mc(As, wm * WM_ROWS + i * 32, k16);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bfr[ss][j] = KC ? frag_kc(Bs, wn * WN_COLS + j * 32, k16)
                                : frag_mc(Bs, wn * WN_COLS + j * 32, k16);
        }
    };

    BTile cur = tile_at(0);
    if (!cur.valid) return;
    issue(cur, cur.kb, 0);
    issue(cur, cur.kb + 1, 1);
    int base = 0;
    for (int round = 0;; ++round) {
        const BTile nxt = tile_at(round + 1);
        f32x16_t acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
        auto mma = [&](auto ni, const bf16x8_t (&af)[2][TM], const bf16x8_t (&bfr)[2][TN]) {
            constexpr int NI = decltype(ni)::value;
#pragma unroll
            for (int ss = 0; ss < 2; ++ss)
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ss][i], bfr[ss][j],
                                                                            acc[i][j], 0, 0, 0);
        };
        // The forward's pipeline: one barrier per k-step, the second half of
        // step kt read while the first half's MFMAs run, step kt+2's loads
        // issued into the stage step kt frees; the next tile's first two
        // k-steps load during this tile's last two.  A wave reads fragments
        // and runs MFMAs for its 32-row blocks that hold valid rows only (none
        // when all its rows are past them: thin last row tiles of an expert).
        auto kloop = [&](auto ni) {
            constexpr bool Mth = decltype(ni)::value > 0;
            bf16x8_t a0[2][TM], b0[2][TN], a1[2][TM], b1[2][TN];
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (Mth) load_frags(ni, base, 0, a0, b0);
            const int nks = cur.nks;
            int kt = 0;
            for (; kt + 2 < nks; ++kt) {
                const int s0 = (base + kt) & 1;
                if (Mth) {
                    load_frags(ni, s0, 1, a1, b1);
                    mma(ni, a0, b0);
                }
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                issue(cur, cur.kb + kt + 2, s0);
                if (Mth) {
                    load_frags(ni, s0 ^ 1, 0, a0, b0);
                    mma(ni, a1, b1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            const int s0 = (base + kt) & 1;
            if (Mth) {
                load_frags(ni, s0, 1, a1, b1);
                mma(ni, a0, b0);
            }
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (nxt.valid) issue(nxt, nxt.kb, s0);
            if (Mth) {
                load_frags(ni, s0 ^ 1, 0, a0, b0);
                mma(ni, a1, b1);
                load_frags(ni, s0 ^ 1, 1, a1, b1);
                mma(ni, a0, b0);
                mma(ni, a1, b1);
            }
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            if (nxt.valid) issue(nxt, nxt.kb + 1, s0 ^ 1);
        };
        {
            const int wrows = cur.rows - wm * WM_ROWS;  // WGRAD: every row is valid
            if (wrows > 64)
                kloop(std::integral_constant<int, TM>{});
            else if (wrows > 32)
                kloop(std::integral_constant<int, (TM < 2 ? TM : 2)>{});
            else if (wrows > 0)
                kloop(std::integral_constant<int, 1>{});
            else
                kloop(std::integral_constant<int, 0>{});
        }

        if (cur.pslot >= 0) {
            // a piece of a split tail tile: store the fp32 partial, lane-major
            // (16-byte group gi of thread tid at gi * kGThreads + tid), skipping
            // 32-row blocks wholly past the valid rows; bwd_tail_reduce_kernel
            // finishes the tile.  Pieces are the last round.
            const i32x4_t rsP = make_rsrc(g.part + (size_t)cur.pslot * (kBwdPartBytes / 4),
                                          (uint32_t)kBwdPartBytes);
            constexpr int NG = TM * TN * 4;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const int i = gi / (TN * 4), j = (gi / 4) % TN, q4 = gi % 4;
                if (wm * WM_ROWS + i * 32 >= cur.rows) continue;
                f32x4_t v;
                v.x = acc[i][j][4 * q4];
                v.y = acc[i][j][4 * q4 + 1];
                v.z = acc[i][j][4 * q4 + 2];
                v.w = acc[i][j][4 * q4 + 3];
                buffer_store_f32x4(v, rsP, (gi * kGThreads + tid) * 16, 0, 0);
            }
            break;
        }

        // epilogue.  Element q of a 32 x 32 accumulator in lane l is row
        // 8*(q/4) + 4*(l/32) + q%4, column l%32 of its block; a quad transpose
        // over each four rows leaves lane l with row 8*(q/4) + 4*(l/32) + l%4,
        // columns (l%32 & ~3) .. +3, so fp32 outputs go out as one 16-byte
        // store and the dh epilogues read g, u (or z) and write dg, du (or dz)
        // with one 8-byte access each: every access of a wave covers 8 rows of
        // 64 or 128 contiguous bytes.  Descriptors end at the last valid row,
        // so padding rows are neither read nor written.
        {
            const int R = KC ? (int)g.C : g.M;  // rows of the output per expert
            const size_t obase = ((size_t)cur.e * R + cur.m0) * g.N + cur.n0;
            const uint32_t obytes = (uint32_t)(((size_t)cur.rows * g.N - cur.n0));
            const int row_t = wm * WM_ROWS + (lane / 32) * 4 + (lane & 3);
            if (EPI == EPI_F32) {
                const i32x4_t rsO = make_rsrc(static_cast<float*>(g.out) + obase, obytes * 4);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int voff = (row_t * g.N + wn * WN_COLS + j * 32 + ((lane % 32) & ~3)) * 4;
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const float v[4] = {acc[i][j][4 * q4], acc[i][j][4 * q4 + 1],
                                                acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]};
                            store_rows4_f32(v, rsO, voff, ((i * 32 + q4 * 8) * g.N) * 4, lane);
                        }
                }
            } else {
                const i32x4_t rsO = make_rsrc(static_cast<uint16_t*>(g.out) + obase, obytes * 2);
                const i32x4_t rs0 = make_rsrc(g.side0 + obase, obytes * 2);
                i32x4_t rsO1 = rsO, rs1 = rs0;
                if (EPI == EPI_DH_SWIGLU) {
                    rsO1 = make_rsrc(g.out1 + obase, obytes * 2);
                    rs1 = make_rsrc(g.side1 + obase, obytes * 2);
                }
                // side reads of the next 32 x 32 block are in flight while the
                // current block's math and stores run
                moe_i32x2_t sa[2][4], su[2][4];
                auto side = [&](int blk, moe_i32x2_t (&a)[4], moe_i32x2_t (&u)[4]) {
                    const int i = blk % TM, j = blk / TM;
                    const int voff = (row_t * g.N + wn * WN_COLS + j * 32 + ((lane % 32) & ~3)) * 2;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int so = ((i * 32 + q4 * 8) * g.N) * 2;
                        a[q4] = buffer_load_i32x2(rs0, voff, so, 0);
                        if (EPI == EPI_DH_SWIGLU) u[q4] = buffer_load_i32x2(rs1, voff, so, 0);
                    }
                };
                side(0, sa[0], su[0]);
#pragma unroll
                for (int blk = 0; blk < TM * TN; ++blk) {
                    const int i = blk % TM, j = blk / TM;
                    if (blk + 1 < TM * TN) side(blk + 1, sa[(blk + 1) & 1], su[(blk + 1) & 1]);
                    const int voff = (row_t * g.N + wn * WN_COLS + j * 32 + ((lane % 32) & ~3)) * 2;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int so = ((i * 32 + q4 * 8) * g.N) * 2;
                        float dh[4] = {acc[i][j][4 * q4], acc[i][j][4 * q4 + 1],
                                       acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]};
                        quad_transpose_f32(dh, lane);
                        float r0[4], r1[4];
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const uint32_t wa = (uint32_t)sa[blk & 1][q4][c / 2];
                            const float a = (c & 1) ? bf_hi(wa) : bf_lo(wa);
                            if (EPI == EPI_DH_SWIGLU) {
                                const uint32_t wu = (uint32_t)su[blk & 1][q4][c / 2];
                                const float u = (c & 1) ? bf_hi(wu) : bf_lo(wu);
                                const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-a));
                                const float dsilu = sg * (1.0f + a * (1.0f - sg));
                                r0[c] = dh[c] * u * dsilu;
                                r1[c] = dh[c] * a * sg;
                            } else {
                                const float cdf = 0.5f * (1.0f + erff(a * 0.70710678118654752f));
                                const float pdf = 0.39894228040143268f * __expf(-0.5f * a * a);
                                r0[c] = dh[c] * (cdf + a * pdf);
                            }
                        }
                        moe_i32x2_t o0;
                        o0.x = (int)pack_bf2(r0[0], r0[1]);
                        o0.y = (int)pack_bf2(r0[2], r0[3]);
                        buffer_store_i32x2(o0, rsO, voff, so, 0);
                        if (EPI == EPI_DH_SWIGLU) {
                            moe_i32x2_t o1;
                            o1.x = (int)pack_bf2(r1[0], r1[1]);
                            o1.y = (int)pack_bf2(r1[2], r1[3]);
                            buffer_store_i32x2(o1, rsO1, voff, so, 0);
                        }
                    }
                }
            }
        }
        if (!nxt.valid) break;
        base = (base + cur.nks) & 1;
        cur = nxt;
    }
}

// Finishes the split tail tiles of one DGRAD launch of G workgroups:
// recomputes the schedule from kept[], sums each element's partials in piece
// order (the result does not depend on which piece finished first) and runs
// the product's epilogue.  A work item is one 16-byte group of one product
// thread: rows row0 .. row0+3 of one output column.  The four threads of a
// quad hold four consecutive columns (consecutive product threads), so the
// dh epilogues transpose each quad as the product does and read and write
// four consecutive columns of one row per thread.
template <int EPI>
__global__ __launch_bounds__(256) void bwd_tail_reduce_kernel(BwdArgs g, int G) {
    constexpr int WM_ROWS = kBM / kWMn, WN_COLS = kBNMax / kWN;
    constexpr int TM = WM_ROWS / 32, TN = WN_COLS / 32;
    constexpr int PER_TILE = kGThreads * TM * TN * 4;
    __shared__ int s_pref[MOE_MAX_EXPERTS + 1];
    __shared__ int s_mt[MOE_MAX_EXPERTS];
    __shared__ int s_tpref[MOE_MAX_EXPERTS + 1];
    const int NT = g.N / kBNMax;
    if (threadIdx.x == 0) bwd_prefix(g, true, NT, s_pref, s_mt, s_tpref);
    __syncthreads();
    const int total = s_pref[g.E] + s_tpref[g.E];
    const int splits = bwd_tail_splits(g, total, G, (g.A1 ? 2 : 1) * (g.K / kBK));
    if (splits <= 1) return;
    const int full = total / G, remt = total - full * G;
    const float4* part = reinterpret_cast<const float4*>(g.part);
    constexpr size_t PSTRIDE = kBwdPartBytes / 16;
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < (int64_t)remt * PER_TILE;
         w += (int64_t)gridDim.x * blockDim.x) {
        const int t = (int)(w / PER_TILE);
        int r = (int)(w - (int64_t)t * PER_TILE);
        const int vt = r % kGThreads;  // the product thread that held these values
        const int gi = r / kGThreads;
        const int i = gi / (TN * 4), j = (gi / 4) % TN, q4 = gi % 4;
        int e, m_tile, n_tile;
        bwd_map_tile(full * G + t, s_pref, s_mt, s_tpref, g.E, NT, e, m_tile, n_tile);
        int kept = g.kept[e];
        if (kept > g.C) kept = (int)g.C;
        const int vwave = vt / kWave, vlane = vt % kWave;
        const int wm = vwave / kWN, wn = vwave % kWN;
        const int m0 = m_tile * kBM, n0 = n_tile * kBNMax;
        if (m0 + wm * WM_ROWS + i * 32 >= kept) continue;  // block past kept: no partials stored
        const size_t base = (size_t)t * splits * PSTRIDE + (size_t)gi * kGThreads + vt;
        float4 s = part[base];
        for (int pc = 1; pc < splits; ++pc) {
            const float4 v = part[base + pc * PSTRIDE];
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        // the group holds rows row0 .. row0+3 of one column
        const int row0 = m0 + wm * WM_ROWS + i * 32 + 8 * q4 + 4 * (vlane / 32);
        if (EPI == EPI_F32) {
            const int col = n0 + wn * WN_COLS + j * 32 + vlane % 32;
            const float v4[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (row0 + u >= kept) break;                // not an output row
                static_cast<float*>(g.out)[((size_t)e * g.C + row0 + u) * g.N + col] = v4[u];
            }
            continue;
        }
        // quad transpose (every lane of the wave is here: the skip above is
        // per wave): row row0 + vlane % 4, columns col4 .. col4 + 3
        float dh[4] = {s.x, s.y, s.z, s.w};
        quad_transpose_f32(dh, vlane);
        const int row = row0 + (vlane & 3);
        if (row >= kept) continue;                         // not an output row
        const int col4 = n0 + wn * WN_COLS + j * 32 + ((vlane % 32) & ~3);
        const size_t o = ((size_t)e * g.C + row) * g.N + col4;
        {
            const uint2 wa = *reinterpret_cast<const uint2*>(g.side0 + o);
            uint2 wu = make_uint2(0u, 0u);
            if (EPI == EPI_DH_SWIGLU) wu = *reinterpret_cast<const uint2*>(g.side1 + o);
            float r0[4], r1[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t xa = c < 2 ? wa.x : wa.y;
                const float a = (c & 1) ? bf_hi(xa) : bf_lo(xa);
                if (EPI == EPI_DH_SWIGLU) {
                    const uint32_t xu = c < 2 ? wu.x : wu.y;
                    const float u = (c & 1) ? bf_hi(xu) : bf_lo(xu);
                    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-a));
                    const float dsilu = sg * (1.0f + a * (1.0f - sg));
                    r0[c] = dh[c] * u * dsilu;
                    r1[c] = dh[c] * a * sg;
                } else {
                    const float cdf = 0.5f * (1.0f + erff(a * 0.70710678118654752f));
                    const float pdf = 0.39894228040143268f * __expf(-0.5f * a * a);
                    r0[c] = dh[c] * (cdf + a * pdf);
                }
            }
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.out) + o) =
                make_uint2(pack_bf2(r0[0], r0[1]), pack_bf2(r0[2], r0[3]));
            if (EPI == EPI_DH_SWIGLU)
                *reinterpret_cast<uint2*>(g.out1 + o) =
                    make_uint2(pack_bf2(r1[0], r1[1]), pack_bf2(r1[2], r1[3]));
        }
    }
}

// Column sums over each expert's kept rows (the bias gradients), in row
// order: out[e][n] = sum_{r < kept[e]} src[e][r][n].
__global__ __launch_bounds__(256) void colsum_kernel(const uint16_t* __restrict__ src,
                                                     const int32_t* __restrict__ kept, int E,
                                                     int64_t C, int N, float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)E * N) return;
    const int e = (int)(i / N), n = (int)(i % N);
    int kp = kept[e];
    if (kp > C) kp = (int)C;
    const uint16_t* p = src + (size_t)e * C * N + n;
    float s = 0.f;
    for (int r = 0; r < kp; ++r) s += bf2f(p[(size_t)r * N]);
    out[i] = s;
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

template <int SCHED, int EPI>
moe_status_t launch_bwd(const BwdArgs& a, int64_t max_tiles, hipStream_t st) {
    auto kern = grouped_gemm_bwd_kernel<SCHED, EPI>;
    const int lds = 2 * 2 * kStageA;
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds) !=
        hipSuccess)
        return MOE_ERR_LAUNCH;
    // split tail pieces may use more workgroups than there are tiles
    const int64_t max_units = (SCHED == SCHED_DGRAD && a.part) ? max_tiles * a.smax : max_tiles;
    int64_t grid = num_cus();
    if (grid > max_units) grid = (max_units + 7) / 8 * 8;
    grid = grid / 8 * 8;
    if (grid < 8) grid = 8;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kGThreads), lds, st, a);
    MOE_CHECK_LAUNCH();
    if (SCHED == SCHED_DGRAD && a.part) {  // finishes the split tail tiles, if any were split
        hipLaunchKernelGGL(bwd_tail_reduce_kernel<EPI>, dim3((unsigned)(4 * num_cus())), dim3(256),
                           0, st, a, (int)grid);
        MOE_CHECK_LAUNCH();
    }
    return MOE_OK;
}

// h, g, u, dg, du planes (GELU uses h, z, dz), then the split tails'
// partial tiles (one per workgroup of a full-device launch) and the forward
// down product's tile counters: the forward products' workspace
size_t bwd_planes_bytes(int E, int64_t C, int64_t I) {
    return ((size_t)5 * E * C * I * 2 + 255) / 256 * 256;
}
size_t bwd_ws_bytes(int E, int64_t C, int64_t I) {
    static_assert(kBwdPartBytes == (size_t)kBM * kBNMax * 4, "the forward's partial tile");
    return bwd_planes_bytes(E, C, I) + moe_expert_ffn_ws_bytes();
}

}  // namespace

extern "C" size_t moe_expert_ffn_bwd_ws_bytes(int E, int64_t C, int64_t I) {
    if (E < 1 || C < 0 || I < 0) return 0;
    return bwd_ws_bytes(E, C, I);
}

extern "C" moe_status_t moe_expert_ffn_bwd(void* stream, moe_dtype_t dtype, moe_act_t act,
                                           const void* x_disp, const int32_t* kept, int E,
                                           int64_t C, int64_t H, int64_t I, const void* w1,
                                           const void* w3, const void* w2, const void* b1,
                                           const void* dy_disp, float* dx_disp, float* dw1,
                                           float* dw3, float* dw2, float* db1, float* db2,
                                           void* ws, size_t ws_bytes, int saved) {
    if (dtype != MOE_BF16) return dtype == MOE_F32 ? MOE_ERR_UNSUPPORTED : MOE_ERR_DTYPE;
    if (act != MOE_ACT_SWIGLU && act != MOE_ACT_GELU_BIAS) return MOE_ERR_DTYPE;
    if (E < 1 || C < 0 || H <= 0 || I <= 0) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    if (H % kBNMax || I % kBNMax || H < 2 * kBK || I < 2 * kBK) return MOE_ERR_ALIGN;
    if (C > (1 << 30) / 8 || H > (1 << 16) || I > (1 << 16)) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)E * C * I >= ((int64_t)1 << 31) || (int64_t)E * C * H >= ((int64_t)1 << 31))
        return MOE_ERR_UNSUPPORTED;
    if (!kept || !w1 || !w2 || !dw1 || !dw2) return MOE_ERR_NULL;
    if (act == MOE_ACT_SWIGLU && (!w3 || !dw3)) return MOE_ERR_NULL;
    if (act == MOE_ACT_GELU_BIAS && (!b1 || !db1)) return MOE_ERR_NULL;
    if (C > 0 && (!x_disp || !dy_disp || !dx_disp)) return MOE_ERR_NULL;
    const void* ptrs[] = {x_disp, w1, w3, w2, b1, dy_disp, dx_disp, dw1, dw3, dw2, ws};
    for (const void* q : ptrs)
        if (q && !moe_aligned16(q)) return MOE_ERR_ALIGN;
    if (C > 0 && (!ws || ws_bytes < bwd_ws_bytes(E, C, I))) return MOE_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool sw = act == MOE_ACT_SWIGLU;
    const size_t plane = (size_t)E * C * I;
    uint16_t* wsb = static_cast<uint16_t*>(ws);
    uint16_t* h = wsb;
    uint16_t* s0 = wsb + plane;        // g or z
    uint16_t* s1 = wsb + 2 * plane;    // u
    uint16_t* d0 = wsb + 3 * plane;    // dg or dz
    uint16_t* d1 = wsb + 4 * plane;    // du
    float* part = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) +
                                           bwd_planes_bytes(E, C, I));
    if (C > 0) {
        // 1. the first product again, saving h and its pre-activations
        // (unless moe_expert_ffn_fwd_save left them in the workspace)
        moe_status_t s = MOE_OK;
        if (!saved) {
            s = moe_ffn1_save(st, act, x_disp, kept, E, C, H, I, w1, w3, b1, h, s0,
                              sw ? s1 : nullptr);
            if (s != MOE_OK) return s;
        }
        const int64_t mt_max = (C + kBM - 1) / kBM;
        // 2. dh = dY W2^T, then the activation's derivative in the epilogue
        BwdArgs a{};
        a.A0 = static_cast<const uint16_t*>(dy_disp);
        a.B0 = static_cast<const uint16_t*>(w2);   // [E][I][H]: rows n = i of length K = H
        a.kept = kept;
        a.E = E;
        a.C = C;
        a.N = (int)I;
        a.K = (int)H;
        a.out = d0;
        a.out1 = d1;
        a.side0 = s0;
        a.side1 = s1;
        a.part = part;
        a.smax = kBwdSMax;
        s = sw ? launch_bwd<SCHED_DGRAD, EPI_DH_SWIGLU>(a, E * mt_max * (I / kBNMax), st)
               : launch_bwd<SCHED_DGRAD, EPI_DH_GELU>(a, E * mt_max * (I / kBNMax), st);
        if (s != MOE_OK) return s;
        // 3. dX = dg W_gate^T (+ du W_up^T), fp32
        BwdArgs b{};
        b.A0 = d0;
        b.B0 = static_cast<const uint16_t*>(w1);   // [E][H][I]: rows n = h of length K = I
        b.A1 = sw ? d1 : nullptr;
        b.B1 = sw ? static_cast<const uint16_t*>(w3) : nullptr;
        b.kept = kept;
        b.E = E;
        b.C = C;
        b.N = (int)H;
        b.K = (int)I;
        b.out = dx_disp;
        b.part = part;
        b.smax = kBwdSMax;
        s = launch_bwd<SCHED_DGRAD, EPI_F32>(b, E * mt_max * (H / kBNMax), st);
        if (s != MOE_OK) return s;
    }
    // 4. weight gradients, contraction over each expert's kept rows (zero
    // for an expert without rows); C = 0 leaves every expert empty
    BwdArgs w{};
    w.kept = kept;
    w.E = E;
    w.C = C;
    if (C == 0) {  // no rows: every weight gradient is zero (a fill kernel, not a memset)
        float* zs[] = {dw1, dw2, sw ? dw3 : nullptr, sw ? nullptr : db1, sw ? nullptr : db2};
        const int64_t ns[] = {(int64_t)E * H * I, (int64_t)E * I * H, (int64_t)E * H * I,
                              (int64_t)E * I, (int64_t)E * H};
        for (int q = 0; q < 5; ++q)
            if (zs[q]) {
                hipLaunchKernelGGL(zero_f32_kernel, dim3(1024), dim3(256), 0, st, zs[q], ns[q]);
                MOE_CHECK_LAUNCH();
            }
        return MOE_OK;
    }
    moe_status_t s;
    w.A0 = h;                                       // dW2 = h^T dY: [I][H]
    w.B0 = static_cast<const uint16_t*>(dy_disp);
    w.M = (int)I;
    w.N = (int)H;
    w.out = dw2;
    s = launch_bwd<SCHED_WGRAD, EPI_F32>(w, E * (I / kBM) * (H / kBNMax), st);
    if (s != MOE_OK) return s;
    w.A0 = static_cast<const uint16_t*>(x_disp);    // dW1 = X^T dg: [H][I]
    w.B0 = d0;
    w.M = (int)H;
    w.N = (int)I;
    w.out = dw1;
    s = launch_bwd<SCHED_WGRAD, EPI_F32>(w, E * (H / kBM) * (I / kBNMax), st);
    if (s != MOE_OK) return s;
    if (sw) {
        w.B0 = d1;                                  // dW3 = X^T du
        w.out = dw3;
        s = launch_bwd<SCHED_WGRAD, EPI_F32>(w, E * (H / kBM) * (I / kBNMax), st);
        if (s != MOE_OK) return s;
    } else {
        const int64_t n1 = (int64_t)E * I;
        hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, st, d0,
                           kept, E, C, (int)I, db1);
        MOE_CHECK_LAUNCH();
        if (db2) {
            const int64_t n2 = (int64_t)E * H;
            hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, st,
                               static_cast<const uint16_t*>(dy_disp), kept, E, C, (int)H, db2);
            MOE_CHECK_LAUNCH();
        }
    }
    return MOE_OK;
}

// Training forward: the expert products with the first product's
// pre-activations kept in the backward workspace (h, g, u or h, z planes),
// so moe_expert_ffn_bwd(..., saved = 1) skips its recompute.
extern "C" moe_status_t moe_expert_ffn_fwd_save(void* stream, moe_dtype_t dtype, moe_act_t act,
                                                const void* x_disp, const int32_t* kept, int E,
                                                int64_t C, int64_t H, int64_t I, const void* w1,
                                                const void* w3, const void* w2, const void* b1,
                                                const void* b2, void* y_disp, void* ws,
                                                size_t ws_bytes) {
    if (dtype != MOE_BF16) return dtype == MOE_F32 ? MOE_ERR_UNSUPPORTED : MOE_ERR_DTYPE;
    if (act != MOE_ACT_SWIGLU && act != MOE_ACT_GELU_BIAS) return MOE_ERR_DTYPE;
    if (E < 1 || C < 0 || H <= 0 || I <= 0) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    if (H % kBNMax || I % kBNMax || H < 2 * kBK || I < 2 * kBK) return MOE_ERR_ALIGN;
    if (C > (1 << 30) / 8 || H > (1 << 16) || I > (1 << 16)) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)E * C * I >= ((int64_t)1 << 31) || (int64_t)E * C * H >= ((int64_t)1 << 31))
        return MOE_ERR_UNSUPPORTED;
    if (!kept || !w1 || !w2) return MOE_ERR_NULL;
    if (act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_NULL;
    if (act == MOE_ACT_GELU_BIAS && !b1) return MOE_ERR_NULL;
    if (C == 0) return MOE_OK;
    if (!x_disp || !y_disp) return MOE_ERR_NULL;
    const void* ptrs[] = {x_disp, w1, w3, w2, b1, b2, y_disp, ws};
    for (const void* q : ptrs)
        if (q && !moe_aligned16(q)) return MOE_ERR_ALIGN;
    if (!ws || ws_bytes < bwd_ws_bytes(E, C, I)) return MOE_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool sw = act == MOE_ACT_SWIGLU;
    const size_t plane = (size_t)E * C * I;
    uint16_t* wsb = static_cast<uint16_t*>(ws);
    uint16_t* h = wsb;
    moe_status_t s = moe_ffn1_save(st, act, x_disp, kept, E, C, H, I, w1, w3, b1, h, wsb + plane,
                                   sw ? wsb + 2 * plane : nullptr);
    if (s != MOE_OK) return s;
    void* part = static_cast<unsigned char*>(ws) + bwd_planes_bytes(E, C, I);
    return moe_ffn2(st, h, kept, E, C, H, I, w2, b2, y_disp, part, moe_expert_ffn_ws_bytes());
}
