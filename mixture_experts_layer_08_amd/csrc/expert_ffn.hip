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
// ceil(kept[e] / 256) row tiles times N / BN_OUT column tiles, and last row
// tiles of at most 64 rows are scheduled after all other tiles.  Workgroup b
// sits on XCD b % 8; in full rounds it takes tile r*G + (b % 8)*(G/8) + b/8,
// so each XCD works through a contiguous run of tiles, ordered expert by
// expert in groups that cover every row tile of an expert across a few
// column tiles, and the A rows and B panels a group shares stay in that
// XCD's L2.  The last, partly filled round goes round-robin over the XCDs;
// when it would leave at least half of the workgroups idle its tiles are cut
// along K into pieces, one per workgroup, and the piece that completes a
// tile's count of stored pieces sums them and finishes the tile.
//
// Per tile: 256 x 256 outputs of the B tile (for SwiGLU 128 gate + 128 up
// columns), K in steps of 64, 8 waves in a 2 x 4 grid, each wave 128 rows x
// 64 columns = 4 x 2 v_mfma_f32_32x32x16_bf16 accumulators (128 fp32
// registers).
//   * Global -> LDS: buffer_load_dwordx4 ... lds writes each lane's 16 bytes
//     straight into LDS (no staging registers, no VALU); two LDS stages of
//     64 KB, the next k-step's loads in flight during the current MFMAs,
//     one barrier per k-step; the next tile's first two k-steps load during
//     the current tile's last ones.
//   * A = rows of x_disp or h, k-contiguous: LDS rows of 128 bytes with the
//     16-byte chunk index XOR ((row >> 1) & 7), read with ds_read_b128.  The
//     A descriptor's byte range ends at row kept[e]: padding rows read as
//     zero without touching memory.
//   * B = W[e] in its own [K, N] layout (n-contiguous).  gfx950's
//     ds_read_b64_tr_b16 reads 4 k-values of one column per lane straight
//     from an n-contiguous tile: inside each 16-lane group, lane L points at
//     row k0 + L/4, columns 4*(L%4) .. +3, and receives rows k0..k0+3 of
//     column L.  Two such reads make one MFMA B operand, so the weights
//     need no repacking.  The chunk index of each 256-byte B row is XORed
//     with 4*(k & 3) so the rows one read serves fall in different banks.
//   * 8-bit weights (F8): B = e4m3 codes stored [E, N, K], each output
//     column's K codes contiguous, with one fp32 scale per column.  The B
//     stage is 256 rows x 64 bytes (16-byte chunk index XOR ((row >> 2) & 3),
//     so the 16 rows one ds_read_b64 pass serves hit distinct banks); a lane
//     reads the 8 codes of its column for its k-slice and turns them into
//     the MFMA's 8 bf16 values with four v_cvt_scalef32_pk_bf16_fp8 (exact:
//     every e4m3 value is a bf16 value).  The column scale multiplies the
//     fp32 accumulator in the epilogue (sum_k x_k q_kn s_n = s_n sum_k x_k
//     q_kn), so the products run on the codes' exact values.
// Epilogues run on the fp32 accumulators in registers:
//   SwiGLU:  a tile holds matching gate and up columns, so
//            h = silu(g) * u needs no extra pass;
//   GELU:    h = gelu_erf(acc + b1);   second product: y = acc (+ b2).
// h is rounded to bf16, y stays fp32; a quad transpose gives each lane four
// consecutive columns, stored with one 8- or 16-byte store through a
// descriptor that ends at row kept[e], so the hardware drops the padding
// rows' stores.
//   Fused combine (moe_expert_ffn_gather_combine; [P3] section 2.1 reduces
//   each token's k expert rows inside the expert kernel): the second
//   product's tiles also finish the tokens whose last kept copy they hold,
//   writing the bf16 layer output; see fused_finish.
#include "moe_common.h"
#include "gemm_common.h"
#include "internal.h"

#include <math.h>

#include <type_traits>

#ifndef FFN1_SPLIT_MAX
#define FFN1_SPLIT_MAX 4  // most K pieces of a tail tile, first product
#endif
#ifndef FFN2_SPLIT_MAX
#define FFN2_SPLIT_MAX 8  // and second product
#endif

namespace {

using namespace moe;

// Training variants of the first product: the same epilogue, which also
// stores the pre-activations the backward needs (SwiGLU: g = X W_gate and
// u = X W_up; GELU: z = X W1 + b1), rounded to bf16.
enum { MODE_SWIGLU_SAVE = 3, MODE_GELU_SAVE = 4 };
// The down product with the combine fused into its epilogue (inference):
// each tile's rows are stored as in MODE_DOWN, then the last of a token's
// kept copies to arrive writes the token's output row (see fused_finish).
enum { MODE_DOWN_FUSED = 5 };
constexpr int mode_base(int m) {
    return m == MODE_SWIGLU_SAVE ? MODE_SWIGLU
         : m == MODE_GELU_SAVE   ? MODE_GELU
         : m == MODE_DOWN_FUSED  ? MODE_DOWN
                                 : m;
}
constexpr bool mode_saves(int m) { return m == MODE_SWIGLU_SAVE || m == MODE_GELU_SAVE; }

struct GemmArgs {
    const uint16_t* A;      // [E, C, K], or with slot_token the token rows [a_rows, K]
    const int32_t* slot_token;  // [E, C] token of each row (-1: empty), or null
    int64_t a_rows;
    const uint16_t* B0;     // [E, K, N] gate / W1 / W2
    const uint16_t* B1;     // [E, K, N] up (SwiGLU)
    const uint16_t* bias;   // [E, N] or null
    void* out;              // [E, C, N]: bf16 (first product) or fp32 (second)
    const int32_t* kept;    // [E]
    int E;
    int64_t C;
    int K;
    int N;                  // output columns
    // split-K of the last, partly filled round of tiles (null part: off)
    float* part;            // per-piece fp32 partial tiles, kPartBytes each
    uint32_t* cnt;          // per split tile: pieces stored so far (zero between launches)
    int smax;               // at most this many pieces per tile
    uint16_t* save0;        // *_SAVE modes: [E, C, N_out] g (or z)
    uint16_t* save1;        // SwiGLU: [E, C, N_out] u
    // 8-bit weights: e4m3 codes [E, N, K] (in place of B0 / B1) and the
    // per-column fp32 scales [E, N]; null scales: bf16 weights
    const uint8_t* Q0;
    const uint8_t* Q1;
    const float* scale0;
    const float* scale1;
    // MODE_DOWN_FUSED: the combine's inputs and output
    const int32_t* row_token;  // [E, C] token of each row (moe_dispatch's slot_token)
    const int32_t* slot;       // [T, k] row of each copy (e * C + r), or -1 (dropped)
    const float* topk_w;       // [T, k] combine weights
    const float* yadd;         // [T, N] fp32 addend row (shared expert) or null
    uint16_t* y;               // [T, N] bf16 output
    uint32_t* tcnt;            // [T, N / 128] copies stored so far per token and column
                               // tile (zero between launches)
    int64_t tokens;            // T
    int k;
};

constexpr size_t kPartBytes = (size_t)kBM * kBNMax * 4;  // one fp32 tile
constexpr int kSMax = 8;  // most pieces per split tile
// rows each thread of the fused combine finishes at a time (k <= 2)
#ifndef FUSE_ROWS
#define FUSE_ROWS 2
#endif

// ---------------------------------------------------------- tile schedule --
// Expert e has ceil(kept[e] / BM) row tiles times NT column tiles.  A last
// row tile with at most thin_rows rows (thin) costs nearly a whole tile's
// loads for little MFMA work, so the schedule puts every expert's other tiles
// first (the main run, expert by expert) and the thin tiles after them (the
// thin run, expert by expert, columns in order): the thin tiles then fall in
// the last, partly filled round, which is cut along K.  The schedule is held
// in registers by every wave of a workgroup: lane e < E holds expert e's
// values and the ends of its two runs (inclusive prefix sums over the lanes).
struct WaveSched {
    int kp;          // kept[e], clamped to [0, C]
    int mt;          // row tiles in the main run
    int end;         // end of expert e's main run
    int tend;        // end of expert e's part of the thin run
    int main_total;  // tiles of the main run (wave-uniform)
    int total;       // all tiles (wave-uniform)
};
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}
__device__ __forceinline__ WaveSched wave_sched(const GemmArgs& g, int NT, int BM, int thin_rows,
                                                int lane) {
    WaveSched w;
    int kp = lane < g.E ? g.kept[lane] : 0;
    if (kp < 0) kp = 0;
    if (kp > g.C) kp = (int)g.C;
    w.kp = kp;
    const int mt_all = (kp + BM - 1) / BM;
    const int thin = (mt_all > 0 && kp - (mt_all - 1) * BM <= thin_rows) ? 1 : 0;
    w.mt = mt_all - thin;
    w.end = wave_incl_scan(w.mt * NT, lane);
    w.tend = wave_incl_scan(thin * NT, lane);
    w.main_total = __builtin_amdgcn_readlane(w.end, 63);
    w.total = w.main_total + __builtin_amdgcn_readlane(w.tend, 63);
    return w;
}

// Tile `logical` -> expert and row / column tile.  In the main run, inside
// an expert, tiles run in groups of every row tile times gn column tiles
// (about GEMM_GROUP tiles), column-fastest, so one XCD's run of tiles shares
// A rows and B panels in its L2.  The expert is the number of experts whose
// run ends at or before the tile.  Every lane of the wave must be active.
__device__ __forceinline__ void map_tile_w(int logical, const WaveSched& w, int E, int NT, int lane,
                                           int& e, int& m_tile, int& n_tile) {
    if (logical < w.main_total) {
        e = (int)__popcll(__ballot(lane < E && w.end <= logical));
        if (e > E - 1) e = E - 1;
        e = __builtin_amdgcn_readfirstlane(e);
        const int start = e > 0 ? __builtin_amdgcn_readlane(w.end, e - 1) : 0;
        const int mt = __builtin_amdgcn_readlane(w.mt, e);
        const int local = logical - start;
        int gn = GEMM_GROUP / mt;
        if (gn < 1) gn = 1;
        if (gn > NT) gn = NT;
        const int grp = local / (mt * gn);
        int width = NT - grp * gn;
        if (width > gn) width = gn;
        const int rem = local - grp * mt * gn;
        m_tile = rem / width;
        n_tile = grp * gn + rem % width;
    } else {
        const int t = logical - w.main_total;
        e = (int)__popcll(__ballot(lane < E && w.tend <= t));
        if (e > E - 1) e = E - 1;
        e = __builtin_amdgcn_readfirstlane(e);
        const int start = e > 0 ? __builtin_amdgcn_readlane(w.tend, e - 1) : 0;
        m_tile = __builtin_amdgcn_readlane(w.mt, e);  // the thin tile follows the main ones
        n_tile = t - start;
    }
}

// Whole tiles fill total / G rounds of a G-workgroup launch.  When the last
// round would leave at least half of the workgroups idle, its tiles are cut
// along K into this many pieces (1: no split).
__device__ __forceinline__ int tail_splits(const GemmArgs& g, int total, int G, int nk) {
    const int remt = total % G;
    if (!g.part || remt == 0 || 2 * remt > G) return 1;
    int sp = G / remt;
    if (sp > g.smax) sp = g.smax;
    if (sp > kSMax) sp = kSMax;
    if (sp > nk / 2) sp = nk / 2;  // each piece keeps at least two k-steps
    return sp < 1 ? 1 : sp;
}

// LDS holds NS slots of A k-steps, then NS slots of B k-steps; stream step
// p of a workgroup (its tiles' k-steps one after another) uses slot p % NS.
//   * default: two slots; the loads of step p+2 are issued once every wave
//     is done with step p, so one k-step of loads is in flight while one is
//     read.  (A third B slot that issues the weight loads one step earlier
//     measured no faster: the loads are not waiting on latency alone.)
//   * THIN: 64-row tiles (every expert has at most 64 rows, as in a decode
//     step) with three slots, two k-steps of loads in flight: a thin tile
//     does little MFMA work per k-step, and with two slots each k-step would
//     wait a whole load round trip.
template <int MODE, int BN, bool F8 = false, bool THIN = false>
struct Epi {
    static constexpr int MB = mode_base(MODE);
    static_assert(BN == 256 || (BN == 128 && MB != MODE_SWIGLU), "B tile is 256 or 128 columns");
    static constexpr int BM = THIN ? 64 : kBM;
    // last row tiles of at most this many rows go to the end of the schedule
    static constexpr int THIN_ROWS = THIN ? 0 : 64;
    static constexpr int NS = THIN ? 3 : 2;
    static constexpr int STAGE_A = BM * kBK * 2;            // 32 KB (8 KB thin)
    static constexpr int STAGE_B = kBK * BN * (F8 ? 1 : 2);  // 32 or 16 KB (8 or 16 KB for codes)
    static constexpr int BN_OUT = (MB == MODE_SWIGLU) ? BN / 2 : BN;
    static constexpr int OUT_BYTES = (MB == MODE_DOWN) ? 4 : 2;
    static constexpr size_t SLOTS = (size_t)NS * (STAGE_A + STAGE_B);
    // MODE_DOWN_FUSED: after the split-state word, a count and the tile's
    // finishing rows (token, then the token's k rows and weights)
    static constexpr size_t FUSE_LDS =
        MODE == MODE_DOWN_FUSED ? 16 + (size_t)BM * 4 * (1 + 2 * MOE_MAX_TOPK) : 0;
    // + a word that broadcasts a split tile's state
    static constexpr size_t LDS = SLOTS + 16 + FUSE_LDS;
    static_assert(LDS <= 160 * 1024, "LDS of one compute unit");
};

// One tile of work: expert e, rows m0.., output columns n0.., and the buffer
// descriptors of its A rows and B columns.
struct TileCtx {
    bool valid;
    int e, m0, n0, kept;
    int kb, nks;                // k-steps kb .. kb + nks - 1
    int pslot;                  // piece of a split tail tile: tile * splits + piece; else -1
    i32x4_t rsA, rsB;
    // gathered A: token of each of this lane's (up to 4) A rows, or -1 (a
    // vector, not an array, so element access stays in registers)
    i32x4_t tok;
};

// GATHER: the A rows are read from the token rows x[slot_token[e, r]]
// instead of a dispatched copy (rows with token -1 read as zero).
template <int MODE, int BN, bool GATHER, bool F8, bool THIN>
__global__ __launch_bounds__(kGThreads, 1) void grouped_gemm_kernel(GemmArgs g) {
    using EP = Epi<MODE, BN, F8, THIN>;
    static_assert(!F8 || !mode_saves(MODE), "8-bit weights: inference products only");
    constexpr int MB = mode_base(MODE);
    constexpr bool SAVE = mode_saves(MODE);
    constexpr bool FUSE = MODE == MODE_DOWN_FUSED;
    // y_disp rows of the fused down product are read by other workgroups
    // (a token's copies sit in different experts' tiles, on any XCD), so they
    // are written through to memory
    constexpr int AUX_OUT = FUSE ? kAuxSystem : 0;
    constexpr int WM_ROWS = EP::BM / kWMn;    // rows per wave
    constexpr int WN_COLS = BN / kWN;         // B columns per wave
    constexpr int TM = WM_ROWS / 32, TN = WN_COLS / 32;  // 32 x 32 MFMA tiles per wave
    constexpr int TH = TN / 2 > 0 ? TN / 2 : 1;           // SwiGLU: gate (or up) tiles per wave
    constexpr int QA = EP::STAGE_A / 1024 / kNW;  // 1 KB A loads per wave per k-step
    // 1 KB B loads per wave per k-step (codes: 16 rows of 64 bytes each)
    constexpr int QB = F8 ? BN / 16 / kNW : (BN / 128) * 16 / kNW;
    static_assert(QA == 1 || (QA <= 4 && QA % 2 == 0), "A loads per wave");
    // store instructions of one wave's whole-tile epilogue (one per four
    // rows of a 32 x 32 accumulator and output column block, plus the saved
    // planes), and the waits of the tile that follows it (see kloop)
    constexpr int TNO_E = (MB == MODE_SWIGLU) ? TN / 2 : TN;
    constexpr int NS_EPI = TNO_E * TM * 4 * (1 + (SAVE ? (MB == MODE_SWIGLU ? 2 : 1) : 0));
    constexpr int kWaitFirst = (QA + QB + NS_EPI) < 63 ? (QA + QB + NS_EPI) : 63;
    constexpr int kWaitMid = NS_EPI < 63 ? NS_EPI : 63;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int wm = wave / kWN, wn = wave % kWN;  // wave rows wm*WM_ROWS.., columns per wn
    const int NT = g.N / EP::BN_OUT;
    const WaveSched ws = wave_sched(g, NT, EP::BM, EP::THIN_ROWS, lane);
    const int total = ws.total;
    const int G = gridDim.x;
    const int xcd = blockIdx.x % 8, slot8 = blockIdx.x / 8;
    const int nk = g.K / kBK;
    // Whole tiles fill `full` rounds; the last round's `remt` tiles may be cut
    // along K into `splits` pieces, one per workgroup.  A piece stores its
    // fp32 partial tile and counts itself in the tile's counter; the piece
    // that completes the count sums the pieces in piece order and runs the
    // epilogue.
    const int full = total / G;
    const int remt = total - full * G;
    const int splits = __builtin_amdgcn_readfirstlane(tail_splits(g, total, G, nk));
    // B sub-tiles are 128 columns (16 KB); wave w fills 1 KB blocks w*QB..,
    // all inside sub-tile (w*QB)/16 (codes: 128 rows = 8 blocks per sub-tile)
    const int sub = F8 ? (wave * QB) / 8 : (wave * QB) / 16;

    auto tile_at = [&](int round) {
        TileCtx c;
        // full rounds: each XCD takes a contiguous run of G/8 tiles (shared
        // A rows and B panels stay in its L2); the last, partial round goes
        // round-robin over the XCDs so that every XCD's fabric bandwidth works
        const int pos = round == full ? (int)blockIdx.x : xcd * (G / 8) + slot8;
        int logical = round * G + pos;
        c.pslot = -1;
        c.kb = 0;
        c.nks = nk;
        if (splits > 1 && round == full) {
            const int t = pos / splits, piece = pos - t * splits;
            logical = pos < remt * splits ? full * G + t : total;
            c.pslot = pos;
            c.kb = piece * nk / splits;
            c.nks = (piece + 1) * nk / splits - c.kb;
        }
        c.valid = logical < total;
        if (!c.valid) return c;
        int e, m_tile, n_tile;
        map_tile_w(logical, ws, g.E, NT, lane, e, m_tile, n_tile);
        c.kept = __builtin_amdgcn_readlane(ws.kp, e);
        c.e = __builtin_amdgcn_readfirstlane(e);
        c.m0 = __builtin_amdgcn_readfirstlane(m_tile * EP::BM);
        c.n0 = __builtin_amdgcn_readfirstlane(n_tile * EP::BN_OUT);
        if (GATHER) {
            // A: token rows; a row past kept (or an empty slot) reads as zero.
            // The tokens of the wave's rows come in by scalar buffer loads
            // (eight rows each, wave-uniform): they are counted by lgkmcnt,
            // so using them never waits for the vector memory queue, which
            // at a tile's start holds the next k-steps' loads and the last
            // tile's epilogue stores.
            c.rsA = make_rsrc(g.A, (uint32_t)((size_t)g.a_rows * g.K * 2));
            const i32x4_t rsT = make_rsrc(g.slot_token + (size_t)c.e * g.C, (uint32_t)c.kept * 4);
#pragma unroll
            for (int q = 0; q < QA; ++q) {
                const int r0 = c.m0 + (wave * QA + q) * 8;
                const moe_i32x8_t sv = s_buffer_load_i32x8(rsT, r0 * 4, 0);
                const int j = lane / 8;
                int t = sv[0];
#pragma unroll
                for (int u = 1; u < 8; ++u) t = j == u ? sv[u] : t;
                c.tok[q] = r0 + j < c.kept ? t : -1;
            }
        } else {
            // A: rows m0.. of expert e; rows at or past kept read as zero
            c.rsA = make_rsrc(g.A + ((size_t)c.e * g.C + c.m0) * g.K,
                              (uint32_t)((size_t)(c.kept - c.m0) * g.K * 2));
        }
        if (F8) {
            // codes: tile row r is weight column n0 + r (SwiGLU: gate rows
            // 0..127, up rows 128..255, each from its own tensor)
            const uint8_t* q = (MB == MODE_SWIGLU && sub == 1) ? g.Q1 : g.Q0;
            c.rsB = make_rsrc(q + ((size_t)c.e * g.N + c.n0) * g.K,
                              (uint32_t)(((size_t)g.N - c.n0) * g.K));
            return c;
        }
        const uint16_t* bsrc;
        size_t coloff;
        if (MB == MODE_SWIGLU) {
            bsrc = (sub == 0 ? g.B0 : g.B1) + (size_t)c.e * g.K * g.N + c.n0;
            coloff = (size_t)c.n0;
        } else {
            bsrc = g.B0 + (size_t)c.e * g.K * g.N + c.n0 + sub * 128;
            coloff = (size_t)c.n0 + sub * 128;
        }
        c.rsB = make_rsrc(bsrc, (uint32_t)(((size_t)g.K * g.N - coloff) * 2));
        return c;
    };

    // A load q of this wave: tile row R = (wave*QA + q)*8 + lane/8 holds in
    // its chunk lane % 8 the logical chunk (lane % 8) ^ swz_a(R), and
    // swz_a(R) = 4*((wave*QA + q) & 1) + lane/16
    const int voffA0 = ((wave * QA * 8 + lane / 8) * g.K + (((lane % 8) ^ (lane / 16)) * 8)) * 2;
    const int voffA1 = ((wave * QA * 8 + lane / 8) * g.K + (((lane % 8) ^ (4 + lane / 16)) * 8)) * 2;
    // B load q: sub-tile row kr = ((wave*QB + q) % 16)*4 + lane/16,
    // chunk (lane % 16) ^ swz_b(kr) with swz_b(kr) = 4*(lane/16)
    const int voffB = ((lane / 16) * g.N + (((lane % 16) ^ ((lane / 16) << 2)) * 8)) * 2;
    // gathered A: the same chunk positions, row offset from the token; an
    // empty row gets an offset past the descriptor's range (reads zero)
    const int chA0 = (((lane % 8) ^ (lane / 16)) * 8) * 2;
    const int chA1 = (((lane % 8) ^ (4 + lane / 16)) * 8) * 2;
    // code load q: tile row R = (wave*QB + q)*16 + lane/4 (its weight row
    // is R, less 128 for SwiGLU's up half), chunk (lane % 4) ^ ((R >> 2) & 3)
    // = (lane % 4) ^ (lane / 16)
    const int rowQ = wave * QB * 16 + lane / 4 - ((MB == MODE_SWIGLU) ? sub * 128 : 0);
    const int voffQ = rowQ * g.K + (((lane % 4) ^ (lane / 16)) * 16);
    // LDS slots (A slots first, then B slots) as 32-bit LDS addresses and
    // as pointers for the fragment reads
    const uint32_t lds_base = (uint32_t)(uintptr_t)(const lds_void_t*)smem;
    auto a_at = [&](int slot) { return smem + slot * EP::STAGE_A; };
    auto b_at = [&](int slot) { return smem + EP::NS * EP::STAGE_A + slot * EP::STAGE_B; };
    auto issue_a = [&](const TileCtx& c, int kt, int slot) {
        const uint32_t st = lds_base + slot * EP::STAGE_A;
#pragma unroll
        for (int q = 0; q < QA; ++q) {
            if (GATHER) {
                const int tk = c.tok[q];
                const int vo = tk >= 0 ? tk * g.K * 2 + (((wave * QA + q) & 1) ? chA1 : chA0)
                                       : (int)0x80000000;
                lds_dma16_at(c.rsA, st + (wave * QA + q) * 1024, vo, kt * kBK * 2);
            } else {
                lds_dma16_at(c.rsA, st + (wave * QA + q) * 1024, ((wave * QA + q) & 1) ? voffA1 : voffA0,
                             (q * 8 * g.K + kt * kBK) * 2);
            }
        }
    };
    auto issue_b = [&](const TileCtx& c, int kt, int slot) {
        const uint32_t st = lds_base + EP::NS * EP::STAGE_A + slot * EP::STAGE_B;
#pragma unroll
        for (int q = 0; q < QB; ++q) {
            if (F8)
                lds_dma16_at(c.rsB, st + (wave * QB + q) * 1024, voffQ, q * 16 * g.K + kt * kBK);
            else
                lds_dma16_at(c.rsB, st + (wave * QB + q) * 1024, voffB,
                             ((((wave * QB + q) % 16) * 4 + kt * kBK) * g.N) * 2);
        }
    };

    // Fragments of one 32-wide half of a k-step: two 16-wide MFMA slices,
    // A (TM x 32 rows) and B (TN x 32 columns) per slice.
    // Only the first NI 32-row blocks of the wave's A rows are read (the
    // others lie past kept[e]).
    auto load_frags = [&](auto ni, int aslot, int bslot, int kk, bf16x8_t (&af)[2][TM],
                          bf16x8_t (&bfr)[2][TN]) {
        constexpr int NI = decltype(ni)::value;
        const unsigned char* As = a_at(aslot);
        const unsigned char* Bs = b_at(bslot);
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
            const int k16 = kk * 2 + ss;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int row = wm * WM_ROWS + i * 32 + lane % 32;
                const int phys = (k16 * 2 + lane / 32) ^ swz_a(row);
                af[ss][i] = as_bf16x8(*reinterpret_cast<const uint4*>(As + row * 128 + phys * 16));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if (F8) {
                    // tile row (= weight column) of this lane; 8 codes of k16's
                    // k values (lane / 32)*8 .. +7
                    const int nr = ((MB == MODE_SWIGLU) ? ((j < TN / 2) ? 0 : 128) +
                                                             wn * (WN_COLS / 2) + (j % TH) * 32
                                                       : wn * WN_COLS + j * 32) + lane % 32;
                    const int phys = k16 ^ ((nr >> 2) & 3);
                    const uint2 v = *reinterpret_cast<const uint2*>(Bs + nr * 64 + phys * 16 +
                                                                    (lane / 32) * 8);
                    uint4 w;
                    w.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false));
                    w.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true));
                    w.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false));
                    w.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true));
                    bfr[ss][j] = as_bf16x8(w);
                    continue;
                }
                int sb, col;  // B sub-tile and column inside it
                if (MB == MODE_SWIGLU) {  // first half of the wave's tiles gate, second up
                    sb = (j < TN / 2) ? 0 : 1;
                    col = wn * (WN_COLS / 2) + (j % TH) * 32;
                } else {
                    const int c = wn * WN_COLS + j * 32;
                    sb = c / 128;
                    col = c % 128;
                }
                // lanes 16-31 / 48-63 take the second 16 columns; lanes 32-63 the k rows 8-15
                col += ((lane / 16) % 2) * 16 + 4 * (lane % 4);
                i16x4_t v[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kr = k16 * 16 + (lane / 32) * 8 + h * 4 + (lane % 16) / 4;
                    const int phys = (col >> 3) ^ swz_b(kr);
                    v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(
                        Bs + sb * 16384 + kr * 256 + phys * 16 + (col & 7) * 2));
                }
                const uint2 lo = __builtin_bit_cast(uint2, v[0]);
                const uint2 hi = __builtin_bit_cast(uint2, v[1]);
                bfr[ss][j] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
            }
        }
    };

    // MODE_DOWN_FUSED, after a tile's rows are stored (y_disp, written
    // through to memory): the combine of [P1] section 2.4 / [P2] section 3.1
    // for the tokens this tile completes.  Each token has n kept copies in n
    // different experts' tiles, and a counter per token and column tile
    // counts the copies stored so far; the tile that brings it to n (or a
    // token's only copy) writes that token's output columns: the addend row
    // (or zero), then w_j * y_j added for j = 0 .. k-1 in order by fused
    // multiply-add (a dropped copy adds w_j * 0), rounded once to bf16 --
    // the same operations as moe_combine, so the output is bitwise the same
    // whichever copy arrives last.
    //   1. every wave waits until its stores have completed, then a barrier:
    //      the tile's rows are in memory before any count includes them;
    //   2. one thread per tile row reads its token, the token's k rows and
    //      weights, and counts the copy with a system-scope atomic (the
    //      counter is set back to zero by the copy that completes it); the
    //      completed tokens are listed in LDS;
    //   3. the workgroup reads the listed tokens' rows (system scope: other
    //      XCDs wrote them), eight columns per thread, and writes y.
    // This is the split tail's publication protocol: rows written through to
    // memory and completed before the relaxed count, read at system scope
    // after it.  The wait in step 1 also drains the next tile's first loads,
    // so the next tile's partial waits hold trivially.
    auto fused_finish = [&](const TileCtx& c) {
        if constexpr (FUSE) {
            constexpr int BNO = EP::BN_OUT;
            constexpr int TPR = BNO / 8;            // threads per row
            constexpr int RPP = kGThreads / TPR;    // rows per pass
            constexpr int KM = MOE_MAX_TOPK;
            int* s_cnt = reinterpret_cast<int*>(smem + EP::SLOTS + 16);
            int* s_tok = s_cnt + 4;
            int* s_slot = s_tok + EP::BM;
            float* s_w = reinterpret_cast<float*>(s_slot + EP::BM * KM);
            // the row's token is loaded while the stores drain (a token out of
            // range, from a slot_token that is not this dispatch's, is skipped)
            const bool row = tid < EP::BM && c.m0 + tid < c.kept;
            const int t = row ? g.row_token[(size_t)c.e * g.C + c.m0 + tid] : -1;
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if (tid == 0) *s_cnt = 0;
            __syncthreads();
            const int k = g.k;
            if (row && t >= 0 && t < g.tokens) {
                int sl[KM];
                float wv[KM];
                int n = 0;
#pragma unroll
                for (int j = 0; j < KM; ++j) {
                    if (j < k) {
                        sl[j] = g.slot[(size_t)t * k + j];
                        wv[j] = g.topk_w[(size_t)t * k + j];
                        n += sl[j] >= 0 ? 1 : 0;
                    }
                }
                bool fin = true;
                if (n > 1) {
                    uint32_t* cp = g.tcnt + (size_t)t * (g.N / BNO) + c.n0 / BNO;
                    const uint32_t before =
                        __hip_atomic_fetch_add(cp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                    fin = before == (uint32_t)(n - 1);
                    if (fin) __hip_atomic_store(cp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                }
                if (fin) {
                    const int idx = atomicAdd(s_cnt, 1);
                    s_tok[idx] = t;
#pragma unroll
                    for (int j = 0; j < KM; ++j) {
                        if (j < k) {
                            s_slot[idx * KM + j] = sl[j];
                            s_w[idx * KM + j] = wv[j];
                        }
                    }
                }
            }
            __syncthreads();
            const int nf = *s_cnt;
            const int c8 = tid % TPR, rsub = tid / TPR;
            const int col = c.n0 + c8 * 8;
            const i32x4_t rsY = make_rsrc(g.out, (uint32_t)((size_t)g.E * g.C * g.N * 4));
            // U rows per thread at a time; the loads of JB copies of each are
            // in flight together, then added in j order
            auto finish_rows = [&](auto u_c, auto jb_c) {
                constexpr int U = decltype(u_c)::value;
                constexpr int JB = decltype(jb_c)::value;
                for (int b0 = 0; b0 < nf; b0 += RPP * U) {
                    f32x4_t a0[U], a1[U];
                    int tt[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int idx = b0 + u * RPP + rsub;
                        tt[u] = idx < nf ? s_tok[idx] : -1;
                        a0[u] = a1[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                        if (tt[u] >= 0 && g.yadd) {
                            const f32x4_t* ya =
                                reinterpret_cast<const f32x4_t*>(g.yadd + (size_t)tt[u] * g.N + col);
                            a0[u] = ya[0];
                            a1[u] = ya[1];
                        }
                    }
                    for (int j0 = 0; j0 < k; j0 += JB) {
                        f32x4_t q0[U][JB], q1[U][JB];
                        float wj[U][JB];
#pragma unroll
                        for (int u = 0; u < U; ++u) {
                            const int idx = b0 + u * RPP + rsub;
#pragma unroll
                            for (int jj = 0; jj < JB; ++jj) {
                                const bool on = tt[u] >= 0 && j0 + jj < k;
                                const int sj = on ? s_slot[idx * KM + j0 + jj] : -1;
                                wj[u][jj] = on ? s_w[idx * KM + j0 + jj] : 0.f;
                                if (sj >= 0) {
                                    const uint32_t off =
                                        ((uint32_t)sj * (uint32_t)g.N + (uint32_t)col) * 4u;
                                    q0[u][jj] = buffer_load_f32x4(rsY, (int)off, 0, kAuxSystem);
                                    q1[u][jj] = buffer_load_f32x4(rsY, (int)(off + 16u), 0, kAuxSystem);
                                } else {
                                    q0[u][jj] = q1[u][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                                }
                            }
                        }
#pragma unroll
                        for (int jj = 0; jj < JB; ++jj) {
                            if (j0 + jj >= k) break;
#pragma unroll
                            for (int u = 0; u < U; ++u) {
                                const float w_ = wj[u][jj];
                                a0[u].x = fmaf(w_, q0[u][jj].x, a0[u].x);
                                a0[u].y = fmaf(w_, q0[u][jj].y, a0[u].y);
                                a0[u].z = fmaf(w_, q0[u][jj].z, a0[u].z);
                                a0[u].w = fmaf(w_, q0[u][jj].w, a0[u].w);
                                a1[u].x = fmaf(w_, q1[u][jj].x, a1[u].x);
                                a1[u].y = fmaf(w_, q1[u][jj].y, a1[u].y);
                                a1[u].z = fmaf(w_, q1[u][jj].z, a1[u].z);
                                a1[u].w = fmaf(w_, q1[u][jj].w, a1[u].w);
                            }
                        }
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        if (tt[u] < 0) continue;
                        *reinterpret_cast<uint4*>(g.y + (size_t)tt[u] * g.N + col) =
                            make_uint4(pack_bf2(a0[u].x, a0[u].y), pack_bf2(a0[u].z, a0[u].w),
                                       pack_bf2(a1[u].x, a1[u].y), pack_bf2(a1[u].z, a1[u].w));
                    }
                }
            };
            // FUSE_ROWS tunes the k <= 2 case alone (at 4 rows the 256-column
            // tiles spill registers; at the default 2 both calls are the same)
            if (k <= 2)
                finish_rows(std::integral_constant<int, FUSE_ROWS>{}, std::integral_constant<int, 2>{});
            else
                finish_rows(std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{});
        }
    };

    TileCtx cur = tile_at(0);
    if (!cur.valid) return;
    bool finish = false;  // this workgroup finishes its split tile after the loop
    // the first two steps of the stream, in the order the loop issues them
    // (the partial wait at a tile's start counts on it)
    issue_a(cur, cur.kb, 0);
    issue_b(cur, cur.kb, 0);
    issue_a(cur, cur.kb + 1, 1);
    issue_b(cur, cur.kb + 1, 1);
    int p0 = 0;  // stream index of the current tile's first k-step
    for (int round = 0;; ++round) {
        const TileCtx nxt = tile_at(round + 1);
        // every round after the first follows a whole tile's epilogue (a
        // split piece ends the loop)
        const bool epi_prev = round > 0;
        // loads of stream step p: the current tile or, past its end, the next
        auto stream_a = [&](int p) {
            const int r = p - p0;
            if (r < cur.nks)
                issue_a(cur, cur.kb + r, p % EP::NS);
            else if (nxt.valid)
                issue_a(nxt, nxt.kb + r - cur.nks, p % EP::NS);
        };
        auto stream_b = [&](int p) {
            const int r = p - p0;
            if (r < cur.nks)
                issue_b(cur, cur.kb + r, p % EP::NS);
            else if (nxt.valid)
                issue_b(nxt, nxt.kb + r - cur.nks, p % EP::NS);
        };
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
        // Software pipeline over k-steps of 64 (two 32-wide halves), stream
        // step p = p0 + kt: the second half of step p is read while the first
        // half's MFMAs run; then the barrier (step p+1 has landed, nobody
        // reads step p any more), the loads of step p+2 go into the slot step
        // p freed, and the first half of step p+1 is read while the second
        // half's MFMAs of step p run.  The tile's last step has no mid-step
        // barrier; after its MFMAs a barrier frees its slot for the next
        // tile's loads, so the next tile starts with its first two steps in
        // flight.  At a tile's start only step p0 must have landed: the loads
        // of step p0+1, issued after it, may stay in flight (loads complete in
        // issue order; any newer stores only make the wait longer).  A wave with
        // rows at or past kept[e] (the tail of an expert's last row tile) runs
        // the same loop with fragment reads and MFMAs for its live 32-row
        // blocks only (none when every row is past kept): it issues the same
        // loads and joins the same barriers (a barrier counts arrivals, so
        // the loop variants stay in step).  sched_barrier(0) keeps each MFMA
        // group on its side of a barrier.
        // After a whole tile's epilogue, the vector memory queue of each wave
        // holds, in issue order: the loads of this tile's first step, those of
        // its second step (QA + QB), then the epilogue's NS_EPI stores (vmcnt
        // counts loads and stores and retires them in issue order).  A wait
        // for vmcnt <= N completes everything older than the newest N
        // operations, so the first step waits with N = QA + QB + NS_EPI and
        // its mid-step wait (for the second step's loads) with N = NS_EPI:
        // the stores stay in flight under the first step's MFMAs instead of
        // draining before the tile starts.  NS_EPI counts the epilogue's
        // store instructions, all issued unconditionally, so the waits are
        // exact or stricter; the counter field holds at most 63.
        auto kloop = [&](auto ni) {
            constexpr bool M = decltype(ni)::value > 0;
            bf16x8_t a0[2][TM], b0[2][TN], a1[2][TM], b1[2][TN];
            if (epi_prev)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWaitFirst) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(QA + QB) : "memory");
            __syncthreads();
            if (GATHER) {
                // The row tokens come from scalar loads; using them here makes
                // the compiler's wait for those (lgkmcnt, which also counts
                // LDS reads) happen once, now, instead of before a load issue
                // inside the loop, where fragment reads are in flight.
#pragma unroll
                for (int q = 0; q < QA; ++q) asm volatile("" ::"v"(cur.tok[q]));
            }
            if (M) load_frags(ni, p0 % EP::NS, p0 % EP::NS, 0, a0, b0);
            const int nks = cur.nks;
            int kt = 0;
            for (; kt + 1 < nks; ++kt) {
                const int p = p0 + kt;
                if (M) {
                    load_frags(ni, p % EP::NS, p % EP::NS, 1, a1, b1);
                    mma(ni, a0, b0);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (kt == 0 && epi_prev)
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWaitMid) : "memory");
                else
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                stream_a(p + 2);
                stream_b(p + 2);
                if (M) {
                    load_frags(ni, (p + 1) % EP::NS, (p + 1) % EP::NS, 0, a0, b0);
                    mma(ni, a1, b1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // the tile's last step
            const int p = p0 + kt;
            if (M) {
                load_frags(ni, p % EP::NS, p % EP::NS, 1, a1, b1);
                mma(ni, a0, b0);
                mma(ni, a1, b1);
            }
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();  // every wave is done with step p
            stream_a(p + 2);
            stream_b(p + 2);
        };
        // THIN: three slots, one barrier per k-step.  Step p+2 is loaded
        // into the slots step p-1 used (free once every wave has passed this
        // step's barrier) while step p is read, so two k-steps of loads are in
        // flight; the wait before the barrier lets the newest step's loads (NL
        // buffer loads per wave) stay outstanding, since loads complete in
        // issue order.  The first step of a tile waits for everything (the
        // previous tile's epilogue stores included).  The last two iterations
        // load the next tile's first two steps.
        auto kloop_thin = [&](auto ni) {
            constexpr bool M = decltype(ni)::value > 0;
            constexpr int NL = QA + QB;
            bf16x8_t af[2][TM], bfr[2][TN];
            const int nks = cur.nks;
            for (int kt = 0; kt < nks; ++kt) {
                if (kt == 0) {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                } else if (kt + 1 < nks || nxt.valid) {
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NL) : "memory");
                } else {
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                }
                __syncthreads();
                if (GATHER && kt == 0) {
#pragma unroll
                    for (int q = 0; q < QA; ++q) asm volatile("" ::"v"(cur.tok[q]));
                }
                stream_a(p0 + kt + 2);
                stream_b(p0 + kt + 2);
                if (M) {
                    const int sc = (p0 + kt) % 3;
                    load_frags(ni, sc, sc, 0, af, bfr);
                    mma(ni, af, bfr);
                    load_frags(ni, sc, sc, 1, af, bfr);
                    mma(ni, af, bfr);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // MFMAs only on the wave's 32-row blocks that hold rows below kept[e]
        // (thin last row tiles of an expert, decode steps)
        if constexpr (THIN) {
            if (cur.kept - (cur.m0 + wm * WM_ROWS) > 0)
                kloop_thin(std::integral_constant<int, 1>{});
            else
                kloop_thin(std::integral_constant<int, 0>{});
        } else {
            const int rows = cur.kept - (cur.m0 + wm * WM_ROWS);
            if (rows > 64)
                kloop(std::integral_constant<int, TM>{});
            else if (rows > 32)
                kloop(std::integral_constant<int, (TM < 2 ? TM : 2)>{});
            else if (rows > 0)
                kloop(std::integral_constant<int, 1>{});
            else
                kloop(std::integral_constant<int, 0>{});
        }

        if (cur.pslot >= 0) {
            // A piece of a split tail tile (pieces are the last round): store
            // the fp32 partial, lane-major (16-byte group gi of thread tid at
            // gi * kGThreads + tid), skipping 32-row blocks wholly past
            // kept[e], which nobody reads.  The pieces of a tile sit on
            // different XCDs, each with its own L2, so partials are written
            // and read at system scope (through to memory), and a piece counts
            // itself in the tile's counter (a system-scope atomic) only once
            // every wave's stores have completed.  The piece that brings the
            // count to `splits` finishes the tile after the loop and sets the
            // counter back to zero for the next launch; the others are done.
            // (No L2-wide write-back or invalidate: those cost tens of
            // microseconds when every piece does them.)
            const i32x4_t rsP = make_rsrc(g.part + (size_t)cur.pslot * (kPartBytes / 4),
                                          (uint32_t)kPartBytes);
            constexpr int NG = TM * TN * 4;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const int i = gi / (TN * 4), j = (gi / 4) % TN, q4 = gi % 4;
                if (cur.m0 + wm * WM_ROWS + i * 32 >= cur.kept) continue;
                f32x4_t v;
                v.x = acc[i][j][4 * q4];
                v.y = acc[i][j][4 * q4 + 1];
                v.z = acc[i][j][4 * q4 + 2];
                v.w = acc[i][j][4 * q4 + 3];
                buffer_store_f32x4(v, rsP, (gi * kGThreads + tid) * 16, 0, kAuxSystem);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            uint32_t* last = reinterpret_cast<uint32_t*>(smem + EP::SLOTS);
            if (tid == 0) {
                uint32_t* cnt = g.cnt + cur.pslot / splits;
                const uint32_t before =
                    __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                const bool fin = before == (uint32_t)(splits - 1);
                if (fin) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                *last = fin ? 1u : 0u;
            }
            __syncthreads();
            finish = *last != 0u;
            break;
        }

        // epilogue: activation on the fp32 accumulators, stored straight from
        // registers.  Element q of a 32 x 32 accumulator in lane l is row
        // 8*(q/4) + 4*(l/32) + q%4, column l%32; a quad transpose over each
        // four rows (q%4) and four lanes leaves lane l with row
        // 8*(q/4) + 4*(l/32) + l%4, columns (l%32 & ~3) .. +3, stored with one
        // 8-byte (bf16) or 16-byte (fp32) store.  The output descriptor ends
        // at row kept[e], so rows past it are dropped by the hardware.
        {
            const uint16_t* biasb = g.bias ? g.bias + (size_t)cur.e * g.N + cur.n0 : nullptr;
            constexpr int TNO = (MB == MODE_SWIGLU) ? TN / 2 : TN;
            constexpr int B = EP::OUT_BYTES;
            static_assert(!SAVE || B == 2, "saved planes share h's layout");
            const i32x4_t rsO = make_rsrc(
                static_cast<unsigned char*>(g.out) + (((size_t)cur.e * g.C + cur.m0) * g.N + cur.n0) * B,
                (uint32_t)(((size_t)(cur.kept - cur.m0) * g.N - cur.n0) * B));
            const int row_t = wm * WM_ROWS + (lane / 32) * 4 + (lane & 3);
            i32x4_t rsS0 = rsO, rsS1 = rsO;  // same layout and row bound as h
            if (SAVE) {
                const size_t off = ((size_t)cur.e * g.C + cur.m0) * g.N + cur.n0;
                rsS0 = make_rsrc(g.save0 + off, (uint32_t)(((size_t)(cur.kept - cur.m0) * g.N - cur.n0) * 2));
                if (MB == MODE_SWIGLU)
                    rsS1 = make_rsrc(g.save1 + off,
                                     (uint32_t)(((size_t)(cur.kept - cur.m0) * g.N - cur.n0) * 2));
            }
#pragma unroll
            for (int j = 0; j < TNO; ++j) {
                const int cbase = (MB == MODE_SWIGLU ? wn * (WN_COLS / 2) : wn * WN_COLS) + j * 32;
                const int ocol = cbase + lane % 32;  // this lane's column before the transpose
                const int voff = (row_t * g.N + cbase + ((lane % 32) & ~3)) * B;
                float bv = 0.f;
                if (MB != MODE_SWIGLU && biasb) bv = bf2f(biasb[ocol]);
                // 8-bit weights: the column scales of this lane's column
                float sc0 = 1.f, sc1 = 1.f;
                if (F8) {
                    sc0 = g.scale0[(size_t)cur.e * g.N + cur.n0 + ocol];
                    if (MB == MODE_SWIGLU) sc1 = g.scale1[(size_t)cur.e * g.N + cur.n0 + ocol];
                }
#pragma unroll
                for (int i = 0; i < TM; ++i) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int soff = ((i * 32 + q4 * 8) * g.N) * B;
                        float v[4], s0v[4], s1v[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int q = 4 * q4 + r;
                            if (MB == MODE_SWIGLU)
                                v[r] = F8 ? silu_f(acc[i][j][q] * sc0) * (acc[i][j + TN / 2][q] * sc1)
                                          : silu_f(acc[i][j][q]) * acc[i][j + TN / 2][q];
                            else if (MB == MODE_GELU)
                                v[r] = gelu_f((F8 ? acc[i][j][q] * sc0 : acc[i][j][q]) + bv);
                            else
                                v[r] = (F8 ? acc[i][j][q] * sc0 : acc[i][j][q]) + bv;
                            if (SAVE && MB == MODE_SWIGLU) {
                                s0v[r] = acc[i][j][q];
                                s1v[r] = acc[i][j + TN / 2][q];
                            } else if (SAVE) {
                                s0v[r] = acc[i][j][q] + bv;
                            }
                        }
                        if (MB == MODE_DOWN)
                            store_rows4_f32<AUX_OUT>(v, rsO, voff, soff, lane);
                        else
                            store_rows4_bf16(v, rsO, voff, soff, lane);
                        if (SAVE) {
                            store_rows4_bf16(s0v, rsS0, voff, soff, lane);
                            if (MB == MODE_SWIGLU) store_rows4_bf16(s1v, rsS1, voff, soff, lane);
                        }
                    }
                }
            }
        }
        fused_finish(cur);
        if (!nxt.valid) break;
        p0 += cur.nks;
        // the next tile was computed at the top of this round (the prefetch
        // used it); the 8-bit gathered variant recomputes it, which keeps
        // fewer registers live across its loop
        if constexpr (GATHER && F8)
            cur = tile_at(round + 1);
        else
            cur = nxt;
    }
    if (SAVE || !finish) return;  // (the training variants never split)

    // The last piece of a split tile to arrive finishes it: each element's
    // partials summed in piece order (the same sums whichever piece arrives
    // last), then the epilogue's activation and stores.  Each thread reads
    // the value groups it stored itself (16-byte, coalesced), one 32-row
    // block at a time with the loads of two pieces in flight together
    // (pieces past `splits` lie past the descriptor and read as zero; they
    // are not added).  This runs after the tile loop, apart from its
    // registers.
    {
        constexpr int TNO = (MB == MODE_SWIGLU) ? TN / 2 : TN;
        constexpr int B = EP::OUT_BYTES;
        const int piece = cur.pslot % splits;
        const i32x4_t rsT = make_rsrc(g.part + (size_t)(cur.pslot - piece) * (kPartBytes / 4),
                                      (uint32_t)(kPartBytes * splits));
        const i32x4_t rsO = make_rsrc(
            static_cast<unsigned char*>(g.out) + (((size_t)cur.e * g.C + cur.m0) * g.N + cur.n0) * B,
            (uint32_t)(((size_t)(cur.kept - cur.m0) * g.N - cur.n0) * B));
        const int row_t = wm * WM_ROWS + (lane / 32) * 4 + (lane & 3);
        const uint16_t* biasb = g.bias ? g.bias + (size_t)cur.e * g.N + cur.n0 : nullptr;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if (cur.m0 + wm * WM_ROWS + i * 32 >= cur.kept) break;  // no partials stored
            constexpr int PG = 2;  // pieces loaded together
            f32x4_t sum[TN][4];
#pragma unroll
            for (int pg = 0; pg < kSMax; pg += PG) {
                if (pg >= splits) break;
                f32x4_t part[PG][TN][4];
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int off = (((i * TN + j) * 4 + q4) * kGThreads + tid) * 16;
#pragma unroll
                        for (int u = 0; u < PG; ++u)
                            part[u][j][q4] = buffer_load_f32x4(
                                rsT, (pg + u) * (int)kPartBytes + off, 0, kAuxSystem);
                    }
#pragma unroll
                for (int u = 0; u < PG; ++u) {
                    if (pg + u >= splits) break;
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            if (pg + u == 0) {
                                sum[j][q4] = part[u][j][q4];
                                continue;
                            }
                            sum[j][q4].x += part[u][j][q4].x;
                            sum[j][q4].y += part[u][j][q4].y;
                            sum[j][q4].z += part[u][j][q4].z;
                            sum[j][q4].w += part[u][j][q4].w;
                        }
                }
            }
#pragma unroll
            for (int j = 0; j < TNO; ++j) {
                const int cbase = (MB == MODE_SWIGLU ? wn * (WN_COLS / 2) : wn * WN_COLS) + j * 32;
                const int ocol = cbase + lane % 32;
                const int voff = (row_t * g.N + cbase + ((lane % 32) & ~3)) * B;
                float bv = 0.f;
                if (MB != MODE_SWIGLU && biasb) bv = bf2f(biasb[ocol]);
                float sc0 = 1.f, sc1 = 1.f;
                if (F8) {  // 8-bit weights: the column scales
                    sc0 = g.scale0[(size_t)cur.e * g.N + cur.n0 + ocol];
                    if (MB == MODE_SWIGLU) sc1 = g.scale1[(size_t)cur.e * g.N + cur.n0 + ocol];
                }
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int soff = ((i * 32 + q4 * 8) * g.N) * B;
                    const f32x4_t a = sum[j][q4];
                    const f32x4_t u = sum[(MB == MODE_SWIGLU) ? j + TN / 2 : j][q4];
                    const float av[4] = {a.x, a.y, a.z, a.w};
                    const float uv[4] = {u.x, u.y, u.z, u.w};
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (MB == MODE_SWIGLU)
                            v[r] = F8 ? silu_f(av[r] * sc0) * (uv[r] * sc1) : silu_f(av[r]) * uv[r];
                        else if (MB == MODE_GELU)
                            v[r] = gelu_f((F8 ? av[r] * sc0 : av[r]) + bv);
                        else
                            v[r] = (F8 ? av[r] * sc0 : av[r]) + bv;
                    }
                    if (MB == MODE_DOWN)
                        store_rows4_f32<AUX_OUT>(v, rsO, voff, soff, lane);
                    else
                        store_rows4_bf16(v, rsO, voff, soff, lane);
                }
            }
        }
    }
    fused_finish(cur);
}

// ----------------------------------------------------------- fp32 path ----
// Plain fp32 tiles (16 x 16 outputs per block, K in steps of 16 through LDS);
// meant for small fp32 layers.
template <int MODE>
__global__ __launch_bounds__(256) void ffn_f32_kernel(const float* __restrict__ A,
                                                      const int32_t* __restrict__ slot_token,
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
    const float* Ab = A + (size_t)e * C * K;  // gathered: rows of A via slot_token
    const float* B0b = B0 + (size_t)e * K * N;
    const float* B1b = (MODE == MODE_SWIGLU) ? B1 + (size_t)e * K * N : nullptr;
    float s0 = 0.f, s1 = 0.f;
    for (int k0 = 0; k0 < K; k0 += 16) {
        const int r = m0 + ty, kk = k0 + tx;
        float av = 0.f;
        if (r < kept && kk < K) {
            if (slot_token) {
                const int tok = slot_token[(size_t)e * C + r];
                av = tok >= 0 ? A[(size_t)tok * K + kk] : 0.f;
            } else {
                av = Ab[(size_t)r * K + kk];
            }
        }
        as[ty][tx] = av;
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


template <int MODE, int BN, bool GATHER = false, bool F8 = false, bool THIN = false>
moe_status_t launch_gemm(const GemmArgs& args, hipStream_t st) {
    using EP = Epi<MODE, BN, F8, THIN>;
    const GemmArgs& a = args;
    auto kern = grouped_gemm_kernel<MODE, BN, GATHER, F8, THIN>;
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)EP::LDS) != hipSuccess)
        return MOE_ERR_LAUNCH;
    const int64_t max_tiles = (int64_t)a.E * ((a.C + EP::BM - 1) / EP::BM) * (a.N / EP::BN_OUT);
    const int64_t max_units = a.part ? max_tiles * a.smax : max_tiles;
    int64_t grid = num_cus();
    if (grid > max_units) grid = (max_units + 7) / 8 * 8;
    grid = grid / 8 * 8;
    if (grid < 8) grid = 8;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kGThreads), EP::LDS, st, a);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

// A single-matrix product (GELU first product, down product) can run with
// 128-column B tiles.  They do half the work of a 256-column tile but run
// about 35% less efficiently per FLOP on MI355X, so they are used only when
// they cut the rounds of 256-column tiles (on the largest tile count kept[]
// allows) by more than 40%: small products whose single round is mostly empty.
bool use_narrow_tiles(const GemmArgs& a, int bm) {
    if (a.N % 128) return false;
    const int64_t cus = num_cus();
    const int64_t mt = (int64_t)a.E * ((a.C + bm - 1) / bm);
    const int64_t t256 = (a.N % 256) ? -1 : mt * (a.N / 256);
    if (t256 < 0) return true;
    const int64_t t128 = mt * (a.N / 128);
    const double c256 = (double)((t256 + cus - 1) / cus);
    const double c128 = 0.5 * (double)((t128 + cus - 1) / cus);
    return c128 < 0.6 * c256;
}

template <int MODE, bool GATHER = false, bool F8 = false, bool THIN = false>
moe_status_t launch_single(const GemmArgs& a, hipStream_t st) {
    return use_narrow_tiles(a, THIN ? 64 : kBM) ? launch_gemm<MODE, 128, GATHER, F8, THIN>(a, st)
                                               : launch_gemm<MODE, 256, GATHER, F8, THIN>(a, st);
}

// Every expert has at most kThinRows rows (C <= kThinRows): 64-row tiles with
// a three-stage pipeline (decode steps).
constexpr int64_t kThinRows = 64;

template <bool GATHER, bool F8, bool THIN>
moe_status_t launch_first(moe_act_t act, const GemmArgs& a, hipStream_t st) {
    return act == MOE_ACT_SWIGLU ? launch_gemm<MODE_SWIGLU, 256, GATHER, F8, THIN>(a, st)
                                 : launch_single<MODE_GELU, GATHER, F8, THIN>(a, st);
}

}  // namespace

// Workspace of the split tail round: one fp32 partial tile per workgroup of
// a full-device launch, then one counter per split tile (zero before the
// first launch; every launch leaves them zero).  The two products use it one
// after the other.
static size_t ffn_cnt_bytes() { return ((size_t)num_cus() * 4 + 255) / 256 * 256; }
static size_t ffn_ws_bytes() { return (size_t)num_cus() * kPartBytes + ffn_cnt_bytes(); }
static uint32_t* ffn_cnt(void* ws) {
    return reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(ws) + (size_t)num_cus() * kPartBytes);
}

extern "C" size_t moe_expert_ffn_ws_bytes(void) { return ffn_ws_bytes(); }

namespace {

// The combine's inputs and output when it is fused into the down product.
struct FuseArgs {
    const int32_t* slot;
    const float* topk_w;
    const float* yadd;
    void* y;
    uint32_t* tcnt;
    int64_t tokens;
    int k;
};

// Every entry point: A is x_disp [E, C, H], or with slot_token the token
// rows x [a_rows, H] gathered through slot_token [E, C].  With scales
// (s1 non-null), w1 / w3 / w2 are e4m3 codes [E, N, K] with per-column fp32
// scales s1 / s3 / s2 [E, N] (bf16 activations only).
moe_status_t ffn_impl(void* stream, moe_dtype_t dtype, moe_act_t act, const void* A,
                      const int32_t* slot_token, int64_t a_rows, const int32_t* kept, int E,
                      int64_t C, int64_t H, int64_t I, const void* w1, const void* w3,
                      const void* w2, const void* b1, const void* b2, void* h_ws, void* y_disp,
                      void* ws, size_t ws_bytes, const float* s1 = nullptr,
                      const float* s3 = nullptr, const float* s2 = nullptr,
                      const FuseArgs* fz = nullptr) {
    const bool f8 = s1 != nullptr;
    if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (act != MOE_ACT_SWIGLU && act != MOE_ACT_GELU_BIAS) return MOE_ERR_DTYPE;
    if (E < 1 || C < 0 || H <= 0 || I <= 0 || a_rows < 0) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    if (H > (1 << 20) || I > (1 << 20) || C >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (!kept || !w1 || !w2) return MOE_ERR_NULL;
    if (act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_NULL;
    if (act == MOE_ACT_GELU_BIAS && !b1) return MOE_ERR_NULL;
    if (f8 && (!s2 || (act == MOE_ACT_SWIGLU && !s3))) return MOE_ERR_NULL;
    if (f8 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
    if (C == 0) return MOE_OK;
    if (!A || !h_ws || !y_disp) return MOE_ERR_NULL;
    const int esz = dtype == MOE_BF16 ? 2 : 4;
    // gathered rows are addressed with 32-bit byte offsets
    if (slot_token && a_rows * H * esz >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dtype == MOE_F32) {
        const float* X = static_cast<const float*>(A);
        float* Hh = static_cast<float*>(h_ws);
        float* Y = static_cast<float*>(y_disp);
        dim3 g1((unsigned)((I + 15) / 16), (unsigned)((C + 15) / 16), (unsigned)E);
        dim3 g2((unsigned)((H + 15) / 16), (unsigned)((C + 15) / 16), (unsigned)E);
        if (act == MOE_ACT_SWIGLU)
            hipLaunchKernelGGL(ffn_f32_kernel<MODE_SWIGLU>, g1, dim3(256), 0, st, X, slot_token,
                               static_cast<const float*>(w1), static_cast<const float*>(w3),
                               (const float*)nullptr, Hh, kept, C, (int)H, (int)I);
        else
            hipLaunchKernelGGL(ffn_f32_kernel<MODE_GELU>, g1, dim3(256), 0, st, X, slot_token,
                               static_cast<const float*>(w1), (const float*)nullptr,
                               static_cast<const float*>(b1), Hh, kept, C, (int)H, (int)I);
        MOE_CHECK_LAUNCH();
        hipLaunchKernelGGL(ffn_f32_kernel<MODE_DOWN>, g2, dim3(256), 0, st, (const float*)Hh,
                           (const int32_t*)nullptr, static_cast<const float*>(w2),
                           (const float*)nullptr, static_cast<const float*>(b2), Y, kept, C,
                           (int)I, (int)H);
        MOE_CHECK_LAUNCH();
        return MOE_OK;
    }
    // bf16: K steps of 64; output tiles of 128 (SwiGLU h) or 256 columns
    if (H % kBNMax || I % kBK) return MOE_ERR_ALIGN;
    if (act == MOE_ACT_SWIGLU ? (I % (kBNMax / 2)) : (I % kBNMax)) return MOE_ERR_ALIGN;
    if (C > (1 << 30) / 8) return MOE_ERR_UNSUPPORTED;
    if (H < 2 * kBK || I < 2 * kBK) return MOE_ERR_ALIGN;  // the k pipeline needs two steps
    const void* ptrs[] = {A, w1, w3, w2, b1, b2, h_ws, y_disp, ws, s1, s3, s2};
    for (const void* q : ptrs)
        if (q && !moe_aligned16(q)) return MOE_ERR_ALIGN;
    // code rows are addressed with 32-bit offsets from an expert's column
    if (f8 && (int64_t)H * I >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    // buffer descriptors hold 32-bit byte ranges and offsets: one expert's
    // bf16 weight matrix (k-step offsets reach its end, a signed 32-bit
    // soffset) and one expert's rows of x_disp, h and fp32 y_disp
    if ((int64_t)H * I * 2 >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (C * (H > I ? H : I) * 4 >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
    GemmArgs a1{};
    a1.A = static_cast<const uint16_t*>(A);
    a1.slot_token = slot_token;
    a1.a_rows = a_rows;
    a1.B0 = static_cast<const uint16_t*>(w1);
    a1.B1 = static_cast<const uint16_t*>(w3);
    a1.bias = act == MOE_ACT_GELU_BIAS ? static_cast<const uint16_t*>(b1) : nullptr;
    a1.out = h_ws;
    a1.save0 = a1.save1 = nullptr;
    a1.Q0 = f8 ? static_cast<const uint8_t*>(w1) : nullptr;
    a1.Q1 = f8 ? static_cast<const uint8_t*>(w3) : nullptr;
    a1.scale0 = s1;
    a1.scale1 = f8 ? s3 : nullptr;
    a1.kept = kept;
    a1.E = E;
    a1.C = C;
    a1.K = (int)H;
    a1.N = (int)I;
    // with a workspace, each product may split its last, partly filled round
    const bool split = ws && ws_bytes >= ffn_ws_bytes();
    a1.part = split ? static_cast<float*>(ws) : nullptr;
    a1.cnt = split ? ffn_cnt(ws) : nullptr;
    a1.smax = FFN1_SPLIT_MAX;
    const bool thin = C <= kThinRows;
    const int sel = (slot_token ? 4 : 0) + (f8 ? 2 : 0) + (thin ? 1 : 0);
    moe_status_t s;
    switch (sel) {
        case 0: s = launch_first<false, false, false>(act, a1, st); break;
        case 1: s = launch_first<false, false, true>(act, a1, st); break;
        case 2: s = launch_first<false, true, false>(act, a1, st); break;
        case 3: s = launch_first<false, true, true>(act, a1, st); break;
        case 4: s = launch_first<true, false, false>(act, a1, st); break;
        case 5: s = launch_first<true, false, true>(act, a1, st); break;
        case 6: s = launch_first<true, true, false>(act, a1, st); break;
        default: s = launch_first<true, true, true>(act, a1, st); break;
    }
    if (s != MOE_OK) return s;
    GemmArgs a2 = a1;
    a2.A = static_cast<const uint16_t*>(h_ws);
    a2.slot_token = nullptr;
    a2.a_rows = 0;
    a2.B0 = static_cast<const uint16_t*>(w2);
    a2.B1 = nullptr;
    a2.bias = static_cast<const uint16_t*>(b2);
    a2.out = y_disp;
    a2.K = (int)I;
    a2.N = (int)H;
    a2.part = split ? static_cast<float*>(ws) : nullptr;
    a2.cnt = split ? ffn_cnt(ws) : nullptr;
    a2.smax = FFN2_SPLIT_MAX;
    a2.Q0 = f8 ? static_cast<const uint8_t*>(w2) : nullptr;
    a2.Q1 = nullptr;
    a2.scale0 = f8 ? s2 : nullptr;
    a2.scale1 = nullptr;
    if (fz) {
        a2.row_token = slot_token;
        a2.slot = fz->slot;
        a2.topk_w = fz->topk_w;
        a2.yadd = fz->yadd;
        a2.y = static_cast<uint16_t*>(fz->y);
        a2.tcnt = fz->tcnt;
        a2.tokens = fz->tokens;
        a2.k = fz->k;
        if (thin)
            return f8 ? launch_single<MODE_DOWN_FUSED, false, true, true>(a2, st)
                      : launch_single<MODE_DOWN_FUSED, false, false, true>(a2, st);
        return f8 ? launch_single<MODE_DOWN_FUSED, false, true>(a2, st)
                  : launch_single<MODE_DOWN_FUSED>(a2, st);
    }
    if (thin)
        return f8 ? launch_single<MODE_DOWN, false, true, true>(a2, st)
                  : launch_single<MODE_DOWN, false, false, true>(a2, st);
    return f8 ? launch_single<MODE_DOWN, false, true>(a2, st) : launch_single<MODE_DOWN>(a2, st);
}

}  // namespace

// The first product again with its pre-activations saved (the backward's
// recompute): h [E, C, I] and g, u (SwiGLU) or z (GELU), all bf16.
moe_status_t moe_ffn1_save(hipStream_t st, moe_act_t act, const void* x_disp, const int32_t* kept,
                           int E, int64_t C, int64_t H, int64_t I, const void* w1, const void* w3,
                           const void* b1, void* h, void* save0, void* save1) {
    GemmArgs a{};
    a.A = static_cast<const uint16_t*>(x_disp);
    a.slot_token = nullptr;
    a.a_rows = 0;
    a.B0 = static_cast<const uint16_t*>(w1);
    a.B1 = static_cast<const uint16_t*>(w3);
    a.bias = act == MOE_ACT_GELU_BIAS ? static_cast<const uint16_t*>(b1) : nullptr;
    a.out = h;
    a.save0 = static_cast<uint16_t*>(save0);
    a.save1 = static_cast<uint16_t*>(save1);
    a.Q0 = a.Q1 = nullptr;
    a.scale0 = a.scale1 = nullptr;
    a.kept = kept;
    a.E = E;
    a.C = C;
    a.K = (int)H;
    a.N = (int)I;
    a.part = nullptr;
    a.cnt = nullptr;
    a.smax = 1;
    return act == MOE_ACT_SWIGLU ? launch_gemm<MODE_SWIGLU_SAVE, 256>(a, st)
                                 : launch_gemm<MODE_GELU_SAVE, 256>(a, st);
}

moe_status_t moe_ffn2(hipStream_t st, const void* h, const int32_t* kept, int E, int64_t C,
                      int64_t H, int64_t I, const void* w2, const void* b2, void* y_disp,
                      void* part, size_t part_bytes) {
    GemmArgs a{};
    a.A = static_cast<const uint16_t*>(h);
    a.slot_token = nullptr;
    a.a_rows = 0;
    a.B0 = static_cast<const uint16_t*>(w2);
    a.B1 = nullptr;
    a.bias = static_cast<const uint16_t*>(b2);
    a.out = y_disp;
    a.save0 = a.save1 = nullptr;
    a.Q0 = a.Q1 = nullptr;
    a.scale0 = a.scale1 = nullptr;
    a.kept = kept;
    a.E = E;
    a.C = C;
    a.K = (int)I;
    a.N = (int)H;
    a.part = (part && part_bytes >= ffn_ws_bytes()) ? static_cast<float*>(part) : nullptr;
    a.cnt = a.part ? ffn_cnt(part) : nullptr;
    a.smax = FFN2_SPLIT_MAX;
    return launch_single<MODE_DOWN>(a, st);
}

extern "C" moe_status_t moe_expert_ffn(void* stream, moe_dtype_t dtype, moe_act_t act,
                                       const void* x_disp, const int32_t* kept, int E, int64_t C,
                                       int64_t H, int64_t I, const void* w1, const void* w3,
                                       const void* w2, const void* b1, const void* b2, void* h_ws,
                                       void* y_disp, void* ws, size_t ws_bytes) {
    return ffn_impl(stream, dtype, act, x_disp, nullptr, 0, kept, E, C, H, I, w1, w3, w2, b1, b2,
                    h_ws, y_disp, ws, ws_bytes);
}

extern "C" moe_status_t moe_expert_ffn_gather(void* stream, moe_dtype_t dtype, moe_act_t act,
                                              const void* x, const int32_t* slot_token,
                                              int64_t T, const int32_t* kept, int E, int64_t C,
                                              int64_t H, int64_t I, const void* w1,
                                              const void* w3, const void* w2, const void* b1,
                                              const void* b2, void* h_ws, void* y_disp, void* ws,
                                              size_t ws_bytes) {
    if (C > 0 && !slot_token) return MOE_ERR_NULL;
    if (T < 0) return MOE_ERR_SHAPE;
    return ffn_impl(stream, dtype, act, x, slot_token, T, kept, E, C, H, I, w1, w3, w2, b1, b2,
                    h_ws, y_disp, ws, ws_bytes);
}

// Counters of the fused combine: one per token and 128-column tile (the
// narrowest output tile), after the split-tail workspace.
static size_t fuse_cnt_bytes(int64_t T, int64_t H) {
    return ((size_t)T * (size_t)(H / 128) * 4 + 255) / 256 * 256;
}

extern "C" size_t moe_expert_ffn_combine_ws_bytes(int64_t T, int64_t H) {
    if (T < 0 || H <= 0) return 0;
    return ffn_ws_bytes() + fuse_cnt_bytes(T, H);
}

namespace {

// The fused call's own checks, then ffn_impl (bf16 weights, or 8-bit codes
// with scales s1 / s3 / s2), then the rows of tokens with no kept copy.
moe_status_t gather_combine_impl(void* stream, moe_act_t act, const void* x,
                                 const int32_t* slot_token, const int32_t* slot,
                                 const float* topk_w, int64_t T, int k, const int32_t* kept, int E,
                                 int64_t C, int64_t H, int64_t I, const void* w1, const void* w3,
                                 const void* w2, const void* b1, const void* b2,
                                 const float* y_shared, void* h_ws, void* y_disp, void* ws,
                                 size_t ws_bytes, void* y, const float* s1, const float* s3,
                                 const float* s2) {
    if (T < 0 || k < 1 || E < 1 || H <= 0 || I <= 0 || C < 0) return MOE_ERR_SHAPE;
    if (k > MOE_MAX_TOPK || k > E || T * k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    if (!slot || !topk_w || !y || !kept) return MOE_ERR_NULL;
    if (C > 0 && !slot_token) return MOE_ERR_NULL;
    if (!ws || ws_bytes < moe_expert_ffn_combine_ws_bytes(T, H)) return MOE_ERR_WORKSPACE;
    if (!moe_aligned16(ws) || !moe_aligned16(y) || (y_shared && !moe_aligned16(y_shared)))
        return MOE_ERR_ALIGN;
    if (H % 8) return MOE_ERR_ALIGN;
    // the finishing tiles read y_disp rows through one 32-bit buffer range
    if ((int64_t)E * C * H * 4 >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
    FuseArgs fz;
    fz.slot = slot;
    fz.topk_w = topk_w;
    fz.yadd = y_shared;
    fz.y = y;
    fz.tcnt = reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(ws) + ffn_ws_bytes());
    fz.tokens = T;
    fz.k = k;
    const moe_status_t s = ffn_impl(stream, MOE_BF16, act, x, slot_token, T, kept, E, C, H, I, w1,
                                    w3, w2, b1, b2, h_ws, y_disp, ws, ffn_ws_bytes(), s1, s3, s2,
                                    &fz);
    if (s != MOE_OK) return s;
    return moe_combine_empty(static_cast<hipStream_t>(stream), slot, topk_w, T, H, k, y_shared, y);
}

}  // namespace

extern "C" moe_status_t moe_expert_ffn_gather_combine(
    void* stream, moe_act_t act, const void* x, const int32_t* slot_token, const int32_t* slot,
    const float* topk_w, int64_t T, int k, const int32_t* kept, int E, int64_t C, int64_t H,
    int64_t I, const void* w1, const void* w3, const void* w2, const void* b1, const void* b2,
    const float* y_shared, void* h_ws, void* y_disp, void* ws, size_t ws_bytes, void* y) {
    return gather_combine_impl(stream, act, x, slot_token, slot, topk_w, T, k, kept, E, C, H, I, w1,
                               w3, w2, b1, b2, y_shared, h_ws, y_disp, ws, ws_bytes, y, nullptr,
                               nullptr, nullptr);
}

extern "C" moe_status_t moe_expert_ffn_gather_combine_fp8(
    void* stream, moe_act_t act, const void* x, const int32_t* slot_token, const int32_t* slot,
    const float* topk_w, int64_t T, int k, const int32_t* kept, int E, int64_t C, int64_t H,
    int64_t I, const uint8_t* w1q, const uint8_t* w3q, const uint8_t* w2q, const float* s1,
    const float* s3, const float* s2, const void* b1, const void* b2, const float* y_shared,
    void* h_ws, void* y_disp, void* ws, size_t ws_bytes, void* y) {
    if (!s1) return MOE_ERR_NULL;
    return gather_combine_impl(stream, act, x, slot_token, slot, topk_w, T, k, kept, E, C, H, I, w1q,
                               w3q, w2q, b1, b2, y_shared, h_ws, y_disp, ws, ws_bytes, y, s1, s3,
                               s2);
}

extern "C" moe_status_t moe_expert_ffn_fp8(void* stream, moe_act_t act, const void* x_disp,
                                           const int32_t* kept, int E, int64_t C, int64_t H,
                                           int64_t I, const uint8_t* w1q, const uint8_t* w3q,
                                           const uint8_t* w2q, const float* s1, const float* s3,
                                           const float* s2, const void* b1, const void* b2,
                                           void* h_ws, void* y_disp, void* ws, size_t ws_bytes) {
    if (!s1) return MOE_ERR_NULL;
    return ffn_impl(stream, MOE_BF16, act, x_disp, nullptr, 0, kept, E, C, H, I, w1q, w3q, w2q, b1,
                    b2, h_ws, y_disp, ws, ws_bytes, s1, s3, s2);
}

extern "C" moe_status_t moe_expert_ffn_gather_fp8(void* stream, moe_act_t act, const void* x,
                                                  const int32_t* slot_token, int64_t T,
                                                  const int32_t* kept, int E, int64_t C, int64_t H,
                                                  int64_t I, const uint8_t* w1q,
                                                  const uint8_t* w3q, const uint8_t* w2q,
                                                  const float* s1, const float* s3,
                                                  const float* s2, const void* b1, const void* b2,
                                                  void* h_ws, void* y_disp, void* ws,
                                                  size_t ws_bytes) {
    if (!s1) return MOE_ERR_NULL;
    if (C > 0 && !slot_token) return MOE_ERR_NULL;
    if (T < 0) return MOE_ERR_SHAPE;
    return ffn_impl(stream, MOE_BF16, act, x, slot_token, T, kept, E, C, H, I, w1q, w3q, w2q, b1,
                    b2, h_ws, y_disp, ws, ws_bytes, s1, s3, s2);
}
