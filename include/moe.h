/*
 * moe.h — C ABI of libmoe_mi355x.so: the forward pass of one sparse
 * Mixture-of-Experts FFN layer on one AMD Instinct MI355X (gfx950).
 *
 * The layer is five calls, issued in this order on one HIP stream:
 *
 *   moe_route       router logits x.W_r (+b_r), softmax, top-k with
 *                   renormalised weights (or Gumbel hard top-k);
 *   moe_aux_stats   load-balancing statistics f_i, p_i and
 *                   L_aux = alpha * E * sum_i f_i p_i;
 *   moe_dispatch    capacity-bounded grouping of the token copies by expert;
 *   moe_expert_ffn  every expert's FFN over its rows (grouped GEMM);
 *   moe_combine     weighted sum of each token's expert outputs.
 *
 * Sources (cited by page and section):
 *   [P1] LLaMA4-MoE hand-built guide, dpshk.com/news/5809432
 *   [P2] MoE basics and minimal PyTorch MoELayer, dpshk.com/news/6005940
 *   [P3] How to Loop MoE: Flatten the Experts, Untie the Attention,
 *        discosf.com/news/5228035
 *   [P4] Long-context MoE training on one A100-80G, 2kiu.com/news/5130654
 *   [P5] pjlab-sys4nlp/llama-moe architecture essay, coreui.cn/article/2610641
 *
 * Conventions shared by every call
 *   - Every array argument is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or synchronises, and keeps no state
 *     between calls, so calls on different streams are independent.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; results are valid once the caller synchronises that stream.
 *   - Arrays are dense and row-major with the shapes given.  Element type is
 *     bf16 (stored as its 16-bit pattern) or fp32 as `dtype` says; integer
 *     outputs are int32; probabilities, weights and statistics are fp32.
 *   - Arguments are validated on the host BEFORE anything is enqueued; on
 *     any error nothing is enqueued and a status other than MOE_OK is
 *     returned.  MOE_ERR_LAUNCH reports a failed kernel launch.  Faults that
 *     only the device can see surface at the caller's synchronisation.
 *   - Limits: 1 <= k <= MOE_MAX_TOPK, k <= E <= MOE_MAX_EXPERTS, T >= 0.
 *     For bf16, H and I must be multiples of 256 and 128 (the grouped GEMM's
 *     tile sizes) and pointers 16-byte aligned; fp32 needs H, I multiples
 *     of 4.  T = 0 is a valid empty call.
 *   - The output of a call depends only on its inputs: there are no
 *     floating-point atomics, so two runs are bitwise identical.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MAX_EXPERTS 64
#define MOE_MAX_TOPK 8

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL                 */
    MOE_ERR_SHAPE = 2,       /* a size is negative, zero or inconsistent   */
    MOE_ERR_DTYPE = 3,       /* unknown dtype / mode / activation          */
    MOE_ERR_UNSUPPORTED = 4, /* legal but beyond this library's limits     */
    MOE_ERR_ALIGN = 5,       /* size or pointer alignment not met          */
    MOE_ERR_WORKSPACE = 6,   /* workspace missing or too small             */
    MOE_ERR_LAUNCH = 7       /* the HIP runtime rejected a kernel launch   */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

typedef enum {
    MOE_ROUTE_SOFTMAX_TOPK = 0,  /* [P2] 2.1 / 3.1, [P5] 3.1            */
    MOE_ROUTE_GUMBEL_HARD = 1    /* [P4] 2 and 5.2                      */
} moe_route_mode_t;

typedef enum {
    MOE_ACT_SWIGLU = 0,      /* (silu(x W1) * (x W3)) W2, no biases      */
    MOE_ACT_GELU_BIAS = 1    /* gelu_erf(x W1 + b1) W2 + b2 ([P2] 3.1)   */
} moe_act_t;

/* Expert capacity C = ceil(T * k * cf / E), evaluated in double in that
 * order ([P2] section 2.4 gives ceil(tokens / experts * cf); the tokens here
 * are the T*k router assignments, which agrees for k = 1).  Host-only and
 * pure.  Returns -1 when an argument is out of range (T < 0, k < 1, E < 1,
 * cf <= 0 or not finite). */
int64_t moe_capacity(int64_t T, int k, int E, double cf);

/* Static, NUL-terminated text for a status code (never NULL). */
const char* moe_status_string(int status);

/* Bytes of workspace moe_aux_stats, moe_dispatch and moe_dispatch_aux need
 * for T tokens, E experts and top-k: a 256-byte header of two arrival
 * counters, then 16 bytes per (block, expert) for at most 64 blocks of
 * 512 assignments or more (at most 65792 bytes).  0 if arguments are out
 * of range.  The workspace must be zero-filled before its first use; every
 * call of those three leaves its counters and flag words zero again, whatever
 * the shape, so one workspace is cleared once and may be shared by them. */
size_t moe_workspace_bytes(int64_t T, int E, int k);

/* Router.  [P2] section 2.1 (score = x . W_r, softmax, keep the top-k);
 * [P2] section 3.1 and [P5] section 3.1 (renormalise the selected weights);
 * [P4] sections 2 and 5.2 (Gumbel hard top-k, temperature 1 + 1e-4 seq_len).
 *
 *   x        [T, H]  dtype       token activations
 *   w_r      [H, E]  dtype       router weight (x . w_r gives the logits)
 *   b_r      [E]     fp32|NULL   optional logit bias
 *   mode     SOFTMAX_TOPK: key = l = x.w_r + b_r; probs = softmax(l);
 *            GUMBEL_HARD:  key = s = l + g, g = -log(-log u), u from
 *                          Philox4x32-10 word 0 at counter (t, e, 0, 0) with
 *                          key (seed & 0xffffffff, seed >> 32) mapped to
 *                          (word + 0.5) * 2^-32; probs = softmax(s / tau),
 *                          tau = 1 + 1e-4 * seq_len (seq_len > 0 required).
 *   topk_idx [T, k]  int32 out   the k largest keys, slot 0 = largest, equal
 *                                keys ordered by lower expert index first
 *   topk_w   [T, k]  fp32  out   probs[t, idx] / sum over the k selected
 *   probs    [T, E]  fp32  out   the row probabilities defined above
 *   keys     [T, E]  fp32|NULL   optional output of the selection keys
 * Logits, softmax and weights are computed in fp32 (bf16 products are
 * exact in fp32; accumulation is fp32). */
moe_status_t moe_route(void* stream, moe_dtype_t dtype, const void* x,
                       const void* w_r, const float* b_r, int64_t T, int64_t H,
                       int E, int k, moe_route_mode_t mode, uint64_t seed,
                       int64_t seq_len, int32_t* topk_idx, float* topk_w,
                       float* probs, float* keys);

/* Load-balancing statistics.  [P2] section 2.3 (f_i, p_i and
 * L_aux = alpha * N * sum f_i p_i; worked example f_1 = 7/8), [P1] 3.2.
 *
 *   topk_idx [T, k] int32, probs [T, E] fp32   (outputs of moe_route)
 *   counts   [E] int32 out   router assignments per expert (before capacity)
 *   f        [E] fp32  out   counts / (T * k)
 *   p        [E] fp32  out   mean over tokens of probs[:, e]
 *   l_aux    [1] fp32  out   alpha * E * sum_e f[e] * p[e]
 *   ws       workspace of at least moe_workspace_bytes(T, E, k) bytes,
 *            zero-filled before its first use, 16-byte aligned (may be
 *            NULL when T = 0; unused when T * E <= 65536, where one
 *            workgroup does the whole reduction)
 * Reductions run in a fixed order (fp64 partial sums): deterministic.
 * With T = 0 every output is zero. */
moe_status_t moe_aux_stats(void* stream, const int32_t* topk_idx,
                           const float* probs, int64_t T, int E, int k,
                           float alpha, int32_t* counts, float* f, float* p,
                           float* l_aux, void* ws, size_t ws_bytes);

/* Capacity-bounded dispatch.  [P2] section 2.4 (a per-expert capacity;
 * overflow tokens are dropped), [P1] section 2.4 (group the token copies by
 * expert id).  Assignment (t, j) takes the next free row of expert
 * e = topk_idx[t, j], walking assignments in row-major (t, then j) order;
 * the row index pos is kept when pos < C.
 *
 *   x          [T, H]    dtype         token activations (may be NULL when
 *                                      x_disp is NULL)
 *   topk_idx   [T, k]    int32         expert of each assignment (< E)
 *   C          rows per expert (normally moe_capacity(T, k, E, cf)), >= 0
 *   x_disp     [E, C, H] dtype  out    x_disp[e, pos] = x[t]; rows >= kept[e]
 *                                      are left untouched.  NULL: only the
 *                                      indices below are produced (for
 *                                      moe_expert_ffn_gather)
 *   slot       [T, k]    int32  out    e * C + pos, or -1 when dropped
 *   slot_token [E, C]    int32  out    token in that row, or -1
 *   kept       [E]       int32  out    min(assignments to e, C)
 *   dropped    [1]       int32  out    number of dropped assignments
 *   ws         workspace of at least moe_workspace_bytes(T, E, k) bytes,
 *              zero-filled before its first use, 16-byte aligned (may be
 *              NULL when T = 0)
 * One launch computes the maps (plus one for the row copy): blocks of 512 or
 * more assignments publish their per-expert counts in ws and each adds up
 * those of the blocks before it; the last block to finish writes kept and
 * dropped and clears what it used.
 * Expert ids outside [0, E) are a caller error (not checked on device). */
moe_status_t moe_dispatch(void* stream, moe_dtype_t dtype, const void* x,
                          const int32_t* topk_idx, int64_t T, int64_t H, int E,
                          int k, int64_t C, void* x_disp, int32_t* slot,
                          int32_t* slot_token, int32_t* kept, int32_t* dropped,
                          void* ws, size_t ws_bytes);

/* Dispatch and aux statistics in one pass: the outputs of moe_dispatch and of
 * moe_aux_stats (same arguments, same meanings: probs [T, E] fp32 and alpha
 * as for moe_aux_stats; counts, f, p, l_aux out) from the same launch —
 * each block also sums its tokens' probabilities and the last block to
 * finish adds those sums in block order (fp64) and finishes the statistics.
 * [P2] sections 2.3 and 2.4, [P1] sections 2.4 and 3.2.
 *   ws  workspace of at least moe_workspace_bytes(T, E, k) bytes, 16-byte
 *       aligned, zero-filled before its first use
 * In addition T * E must be below 2^31. */
moe_status_t moe_dispatch_aux(void* stream, moe_dtype_t dtype, const void* x,
                              const int32_t* topk_idx, const float* probs,
                              int64_t T, int64_t H, int E, int k, int64_t C,
                              float alpha, void* x_disp, int32_t* slot,
                              int32_t* slot_token, int32_t* kept, int32_t* dropped,
                              int32_t* counts, float* f, float* p, float* l_aux,
                              void* ws, size_t ws_bytes);

/* moe_dispatch_aux without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs and results as
 * moe_dispatch_aux (the same kernels run); its workspace is instead a static
 * device array of MOE_NOALLOC_SCRATCH_BYTES bytes inside the library, one
 * per GPU, held until the process ends.  It calls no allocating routine.
 *   - The largest workspace any accepted shape needs is 256 + 64 * 64 * 16
 *     = 65792 bytes (E = 64), so every call the other checks accept fits;
 *     MOE_ERR_UNSUPPORTED would report one that did not.
 *   - Every call on one GPU shares that GPU's array: two calls that may
 *     run at the same time on one GPU (different streams, no ordering
 *     between them) race and give wrong results.  Calls ordered on one
 *     stream are safe: each leaves the array's counters and flags zero.
 *   - MOE_ERR_LAUNCH when the array's device address cannot be looked up. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 10)
moe_status_t moe_dispatch_aux_noalloc(void* stream, moe_dtype_t dtype, const void* x,
                                      const int32_t* topk_idx, const float* probs,
                                      int64_t T, int64_t H, int E, int k, int64_t C,
                                      float alpha, void* x_disp, int32_t* slot,
                                      int32_t* slot_token, int32_t* kept,
                                      int32_t* dropped, int32_t* counts, float* f,
                                      float* p, float* l_aux);

/* Expert FFNs as one grouped GEMM over the dispatched rows.
 * [P2] sections 2.2 and 3.1 (each expert is an FFN; GELU expert with two
 * biased Linears), [P5] section 2.1 (SwiGLU), [P2] section 4.4 / [P5] 6.3
 * (merge each expert's tokens into one large matrix product).
 *
 *   x_disp [E, C, H] dtype      rows r < kept[e] are used
 *   kept   [E]       int32      (device) rows per expert, 0 <= kept <= C
 *   w1     [E, H, I] dtype      SwiGLU gate / GELU first matrix
 *   w3     [E, H, I] dtype      SwiGLU up matrix; NULL for GELU
 *   w2     [E, I, H] dtype      down / second matrix
 *   b1     [E, I]    dtype      GELU first bias (required for GELU)
 *   b2     [E, H]    dtype|NULL GELU second bias (optional)
 *   h_ws   [E, C, I] dtype      caller workspace for the hidden activation
 *   y_disp [E, C, H] fp32  out  expert outputs (fp32 for both dtypes, so
 *                               the combine rounds only once); rows >=
 *                               kept[e] untouched
 *   ws     NULL, or a workspace of ws_bytes >= moe_expert_ffn_ws_bytes()
 *          bytes, 16-byte aligned and zero-filled before its first use (its
 *          tile counters must start at zero; every call leaves them zero
 *          again, so a workspace is cleared once, when it is allocated).
 *          With it, each product's last, partly filled round of tiles is
 *          cut along K: every piece stores its fp32 partial tile and the
 *          piece that completes a tile sums the pieces in piece order
 *          (results stay bitwise reproducible); without it, or when it is
 *          too small, that round runs whole.  Two calls that run at the
 *          same time must not share one ws.
 * bf16 runs on the matrix cores with fp32 accumulation; h is rounded to bf16
 * (nearest-even) between the two products.  An expert with kept = 0 is a
 * valid no-op.  bf16 limits: H a multiple of 256, I a multiple of 128
 * (SwiGLU) or 256 (GELU), H and I >= 128; fp32 has no size limit beyond
 * int32 indexing. */
moe_status_t moe_expert_ffn(void* stream, moe_dtype_t dtype, moe_act_t act,
                            const void* x_disp, const int32_t* kept, int E,
                            int64_t C, int64_t H, int64_t I, const void* w1,
                            const void* w3, const void* w2, const void* b1,
                            const void* b2, void* h_ws, void* y_disp, void* ws,
                            size_t ws_bytes);

/* moe_expert_ffn with the row copy fused into the first product's loads:
 * the A rows come straight from the token activations through slot_token,
 * so no x_disp is written or read ([P3] section 2.1 gathers each expert's
 * tokens inside the expert kernel instead of materialising them).
 *
 *   x          [T, H]    dtype   token activations (16-byte aligned)
 *   slot_token [E, C]    int32   moe_dispatch's output: token of each row
 *                                r < kept[e]; entries past kept[e] unused
 * Every other argument, output, workspace use and limit is as for
 * moe_expert_ffn; in addition T * H * sizeof(dtype) must be below 2^31.
 * The result equals moe_expert_ffn on the dispatched copy. */
moe_status_t moe_expert_ffn_gather(void* stream, moe_dtype_t dtype, moe_act_t act,
                                   const void* x, const int32_t* slot_token,
                                   int64_t T, const int32_t* kept, int E,
                                   int64_t C, int64_t H, int64_t I,
                                   const void* w1, const void* w3,
                                   const void* w2, const void* b1,
                                   const void* b2, void* h_ws, void* y_disp,
                                   void* ws, size_t ws_bytes);

/* moe_expert_ffn_gather with moe_combine fused into the down product:
 * [P3] section 2.1 reads each expert's rows by routing index inside the
 * expert kernel, and the weighted sum of [P1] section 2.4 / [P2] section 3.1
 * is done by the down product's tiles instead of a separate pass.  The
 * tile holding the last of a token's kept copies to finish (a token's only
 * copy, at once) computes the token's output columns exactly as
 * moe_combine does (the addend row or zero, then fused multiply-adds of
 * w[t, j] * y_disp row for j = 0 .. k-1 in order, a dropped copy adding
 * w * 0, one bf16 rounding), so y is bitwise moe_combine's whichever copy
 * finishes last; tokens with no kept copy get their row from a small pass.
 *
 *   slot, topk_w [T, k]      moe_dispatch's slot and moe_route's weights
 *   y_shared     [T, H] fp32 optional addend row (shared expert) or NULL
 *   y_disp       [E, C, H] fp32  workspace (holds the expert rows after
 *                                the call, as moe_expert_ffn_gather's)
 *   ws           >= moe_expert_ffn_combine_ws_bytes(T, H) bytes, 16-byte
 *                aligned, zero-filled before its first use; every call
 *                leaves it zero again (per-token counters and the split
 *                tail's workspace).  Required (MOE_ERR_WORKSPACE).  Two
 *                calls that run at the same time must not share one ws.
 *   y            [T, H] bf16 out
 * slot_token, slot and kept must come from one moe_dispatch (or
 * moe_dispatch_aux) call: the kept copies of a token are counted from slot
 * and must each appear in slot_token; with an inconsistent set the output
 * rows are wrong and the counters may stay non-zero (a slot_token entry
 * outside [0, T) is skipped).  bf16 activations and weights only; other
 * arguments and limits as for moe_expert_ffn_gather, and E * C * H * 4
 * below 2^32. */
size_t moe_expert_ffn_combine_ws_bytes(int64_t T, int64_t H);
moe_status_t moe_expert_ffn_gather_combine(void* stream, moe_act_t act, const void* x,
                                           const int32_t* slot_token, const int32_t* slot,
                                           const float* topk_w, int64_t T, int k,
                                           const int32_t* kept, int E, int64_t C, int64_t H,
                                           int64_t I, const void* w1, const void* w3,
                                           const void* w2, const void* b1, const void* b2,
                                           const float* y_shared, void* h_ws, void* y_disp,
                                           void* ws, size_t ws_bytes, void* y);

/* ------------------------------------------------------ 8-bit weights ----
 * [P4] section 3 keeps the expert weights in 8 bits and restores them with
 * a scale computed per expert and per dimension; [P1] section 5.2 and [P5]
 * section 5.1 name low-bit expert weights for inference.  Here the 8-bit
 * code is the OCP float8 e4m3 format (gfx950 turns two codes into two bf16
 * values in one instruction, and every e4m3 value is exactly a bf16 value),
 * with one fp32 scale per expert and output column.
 *
 * Quantisation of W [E, K, N] (bf16, finite):
 *   scale [E, N] fp32 out  max_k |W[e, k, n]| / 448 (correctly rounded;
 *                          1 for an all-zero column)
 *   q     [E, N, K] u8 out the e4m3 code nearest to W[e, k, n] / scale[e, n]
 *                          (fp32 quotient, ties to the even code), stored
 *                          transposed: each column's K codes contiguous
 * K must be a multiple of 16 (q 16-byte aligned); K < 2^22. */
moe_status_t moe_quantize_fp8(void* stream, const void* w, int E, int64_t K,
                              int64_t N, uint8_t* q, float* scale);

/* Dequantisation: w [E, K, N] fp32 out = decode(q[e, n, k]) * scale[e, n],
 * rounded once to fp32 (NaN codes give NaN).  Same layouts and limits as
 * moe_quantize_fp8. */
moe_status_t moe_dequantize_fp8(void* stream, const uint8_t* q, const float* scale,
                                int E, int64_t K, int64_t N, float* w);

/* Expert FFNs on 8-bit weights: moe_expert_ffn (resp. _gather) with
 *   w1q [E, I, H], w3q [E, I, H] (SwiGLU), w2q [E, H, I]  e4m3 codes as
 *       moe_quantize_fp8 writes them (of W1, W3 [E, H, I], W2 [E, I, H])
 *   s1 [E, I], s3 [E, I], s2 [E, H]                        their scales
 * in place of w1, w3, w2; activations, biases, h_ws and y_disp are bf16 /
 * bf16 / bf16 / fp32 as for moe_expert_ffn.  The products run on the codes'
 * exact values in bf16 and each output column is multiplied by its scale
 * on the fp32 accumulator, so the result is the layer with the dequantised
 * weights.  Limits and the optional ws (zero-filled before its first use) as
 * for moe_expert_ffn; in addition H * I < 2^31. */
moe_status_t moe_expert_ffn_fp8(void* stream, moe_act_t act, const void* x_disp,
                                const int32_t* kept, int E, int64_t C, int64_t H,
                                int64_t I, const uint8_t* w1q, const uint8_t* w3q,
                                const uint8_t* w2q, const float* s1, const float* s3,
                                const float* s2, const void* b1, const void* b2,
                                void* h_ws, void* y_disp, void* ws, size_t ws_bytes);
moe_status_t moe_expert_ffn_gather_fp8(void* stream, moe_act_t act, const void* x,
                                       const int32_t* slot_token, int64_t T,
                                       const int32_t* kept, int E, int64_t C,
                                       int64_t H, int64_t I, const uint8_t* w1q,
                                       const uint8_t* w3q, const uint8_t* w2q,
                                       const float* s1, const float* s3,
                                       const float* s2, const void* b1,
                                       const void* b2, void* h_ws, void* y_disp,
                                       void* ws, size_t ws_bytes);

/* moe_expert_ffn_gather_combine on 8-bit weights: the codes and scales as for
 * moe_expert_ffn_gather_fp8 in place of w1, w3, w2; every other argument,
 * the workspace and the bitwise agreement with moe_combine as for
 * moe_expert_ffn_gather_combine. */
moe_status_t moe_expert_ffn_gather_combine_fp8(void* stream, moe_act_t act, const void* x,
                                               const int32_t* slot_token, const int32_t* slot,
                                               const float* topk_w, int64_t T, int k,
                                               const int32_t* kept, int E, int64_t C, int64_t H,
                                               int64_t I, const uint8_t* w1q, const uint8_t* w3q,
                                               const uint8_t* w2q, const float* s1,
                                               const float* s3, const float* s2, const void* b1,
                                               const void* b2, const float* y_shared, void* h_ws,
                                               void* y_disp, void* ws, size_t ws_bytes, void* y);

/* Bytes of the optional moe_expert_ffn workspace on the current device:
 * one 256 KiB fp32 tile per compute unit, then one 4-byte tile counter per
 * compute unit (rounded up to 256 bytes). */
size_t moe_expert_ffn_ws_bytes(void);

/* Weighted combine back to token order.  [P1] section 2.4 and [P2]
 * section 3.1 (each token's output is the weighted sum of its selected
 * experts' outputs).  Dropped assignments (slot < 0) add nothing and the
 * other weights are not renormalised; a token with every copy dropped gets
 * zeros (plus the shared experts' row, if any).
 *
 *   y_disp   [E*C, H] fp32 (moe_expert_ffn's output), slot [T, k] int32,
 *   topk_w   [T, k] fp32
 *   y_shared [T, H]   fp32 or NULL: the shared experts' output, added to
 *            every token's sum with weight 1 ([P1] section 5.2: shared
 *            experts every token passes through; moe_expert_ffn with E = 1,
 *            C = T, kept = {T} and x itself as x_disp computes it)
 *   y        [T, H]   dtype out   (fp32 accumulation, bf16 rounded once)
 * H must be a multiple of 8; y_disp, y_shared and y 16-byte aligned.
 * Every slot must be -1 or a row index below E*C (not checked on device). */
moe_status_t moe_combine(void* stream, moe_dtype_t dtype, const void* y_disp,
                         const int32_t* slot, const float* topk_w, int64_t T,
                         int64_t H, int k, const float* y_shared, void* y);

/* ------------------------------------------------------------ backward ----
 * Gradients of  L = sum(dy * y) + dl_aux * L_aux  for a given output
 * gradient dy.  The top-k choice and the capacity drop are piecewise
 * constant and pass no gradient; f_i is a count and is held constant.
 * One backward step, in order:
 *   moe_combine_bwd     dy_disp, dw (gradient of the combine weights)
 *   moe_expert_ffn_bwd  dx_disp and every expert weight gradient
 *   moe_dispatch_bwd    dx = sum over each token's kept copies of dx_disp
 *   moe_route_bwd       dlogits, dW_r, db_r, and dx += dlogits W_r^T
 * All gradient outputs are fp32; every sum runs in a fixed order
 * (bitwise reproducible). */

/* Combine backward.  [P1] section 2.4 (y_t = sum_j w_tj Y[slot_tj]).
 *   dy      [T, H]   dtype   output gradient
 *   y_disp  [E*C, H] fp32    the forward's expert outputs
 *   slot    [T, k]   int32,  topk_w [T, k] fp32  (the forward's)
 *   dy_disp [E*C, H] dtype out  w_tj * dy_t at row slot_tj for every kept
 *                               copy; other rows untouched
 *   dw      [T, k]   fp32  out  <dy_t, Y[slot_tj]>, 0 for a dropped copy
 * H must be a multiple of 8; pointers 16-byte aligned. */
moe_status_t moe_combine_bwd(void* stream, moe_dtype_t dtype, const void* dy,
                             const void* y_disp, const int32_t* slot,
                             const float* topk_w, int64_t T, int64_t H, int k,
                             void* dy_disp, float* dw);

/* Expert FFN backward.  [P2] sections 2.2 and 3.1, [P5] section 2.1 (the
 * expert FFNs being differentiated).  Re-runs the first product to recover
 * h and its pre-activations (bf16) — or, with saved != 0, takes them from
 * ws, where moe_expert_ffn_fwd_save left them for the same inputs — then
 *   SwiGLU: dh = dY W_down^T, dg = dh u silu'(g), du = dh silu(g),
 *           dX = dg W_gate^T + du W_up^T, dW_down = h^T dY,
 *           dW_gate = X^T dg, dW_up = X^T du
 *   GELU:   dz = (dY W2^T) gelu'(z), dX = dz W1^T, dW2 = h^T dY,
 *           dW1 = X^T dz, db1 = sum_rows dz, db2 = sum_rows dY
 * over each expert's kept rows.
 *   x_disp  [E, C, H] bf16       the forward's dispatched rows
 *   kept    [E]       int32      (device)
 *   w1, w3, w2, b1               as for moe_expert_ffn (w3 SwiGLU only,
 *                                b1 GELU only)
 *   dy_disp [E, C, H] bf16       moe_combine_bwd's output
 *   dx_disp [E, C, H] fp32 out   rows < kept[e] written
 *   dw1 [E, H, I], dw3 [E, H, I] (SwiGLU), dw2 [E, I, H]   fp32 out
 *   db1 [E, I] (GELU, required), db2 [E, H] (GELU, may be NULL)  fp32 out
 *   ws      moe_expert_ffn_bwd_ws_bytes(E, C, I) bytes, 16-byte aligned,
 *           zero-filled before its first use (the tile counters at its end;
 *           every call leaves them zero again)
 *   saved   0: recompute the first product; else ws holds its saved planes
 * bf16 only (MOE_ERR_UNSUPPORTED for fp32); H and I multiples of 256. An
 * expert with no rows gets zero weight gradients. */
moe_status_t moe_expert_ffn_bwd(void* stream, moe_dtype_t dtype, moe_act_t act,
                                const void* x_disp, const int32_t* kept, int E,
                                int64_t C, int64_t H, int64_t I, const void* w1,
                                const void* w3, const void* w2, const void* b1,
                                const void* dy_disp, float* dx_disp, float* dw1,
                                float* dw3, float* dw2, float* db1, float* db2,
                                void* ws, size_t ws_bytes, int saved);

/* Bytes of moe_expert_ffn_bwd's workspace on the current device: five bf16
 * [E, C, I] planes, then moe_expert_ffn_ws_bytes() bytes (the partial tiles
 * of the split tail rounds and the forward products' tile counters). */
size_t moe_expert_ffn_bwd_ws_bytes(int E, int64_t C, int64_t I);

/* Training forward of the expert FFNs: the result of moe_expert_ffn
 * (y_disp [E, C, H] fp32; same products, same bounds), with h and the first
 * product's pre-activations written into ws (moe_expert_ffn_bwd_ws_bytes
 * bytes, zero-filled before its first use as for moe_expert_ffn_bwd) for a
 * later moe_expert_ffn_bwd(..., saved = 1) on the same x_disp,
 * kept and weights, which then skips its recompute (P3 section 3.3 trades
 * that recompute against memory; here the memory is five bf16 [E, C, I]
 * planes).  bf16 only; H and I multiples of 256. */
moe_status_t moe_expert_ffn_fwd_save(void* stream, moe_dtype_t dtype, moe_act_t act,
                                     const void* x_disp, const int32_t* kept, int E,
                                     int64_t C, int64_t H, int64_t I, const void* w1,
                                     const void* w3, const void* w2, const void* b1,
                                     const void* b2, void* y_disp, void* ws,
                                     size_t ws_bytes);

/* Dispatch backward: dx[t] = dx_add[t] + sum over kept j of
 * dx_disp[slot[t, j]] (fp32; dx_add may be NULL, then a token with every
 * copy dropped gets zeros).  [P1] section 2.4 (the copies are gathered back
 * by token); dx_add carries the shared experts' input gradient ([P1]
 * section 5.2).  H a multiple of 8; pointers 16-byte aligned. */
moe_status_t moe_dispatch_bwd(void* stream, const float* dx_disp,
                              const int32_t* slot, int64_t T, int64_t H, int k,
                              const float* dx_add, float* dx);

/* Router backward.  [P5] section 3.1 (renormalised top-k of the softmax),
 * [P2] section 2.3 (L_aux), [P4] section 2 (Gumbel soft path).
 *   x [T, H], w_r [H, E]  dtype;  probs [T, E] fp32 (the forward's p, or q in
 *   Gumbel mode);  topk_idx, topk_w [T, k] (the forward's);  dw [T, k] fp32
 *   (moe_combine_bwd's);  f [E] fp32 (moe_aux_stats');  alpha, dl_aux;
 *   seq_len (the temperature, Gumbel mode)
 *   dlogits [T, E] fp32 out   gradient of the router logits
 *   dx      [T, H] fp32 in/out dx += dlogits W_r^T (NULL: skipped)
 *   dw_r    [H, E] fp32 out;  db_r [E] fp32 out (NULL when there is no bias)
 *   ws      moe_route_bwd_ws_bytes(T, H, E) bytes
 * H a multiple of 8; x, w_r, dx and ws 16-byte aligned (MOE_ERR_ALIGN). */
moe_status_t moe_route_bwd(void* stream, moe_dtype_t dtype, moe_route_mode_t mode,
                           const void* x, const void* w_r, const float* probs,
                           const int32_t* topk_idx, const float* topk_w,
                           const float* dw, const float* f, float alpha,
                           float dl_aux, int64_t T, int64_t H, int E, int k,
                           int64_t seq_len, float* dlogits, float* dx, float* dw_r,
                           float* db_r, void* ws, size_t ws_bytes);

size_t moe_route_bwd_ws_bytes(int64_t T, int64_t H, int E);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
