// Library-internal entry points shared between translation units (not part
// of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/moe.h"

// The first expert product on x_disp with its pre-activations saved for the
// backward: h [E, C, I] and, all bf16 with the same layout, g = X W_gate and
// u = X W_up (SwiGLU) or z = X W1 + b1 in save0 (GELU; save1 unused).
moe_status_t moe_ffn1_save(hipStream_t st, moe_act_t act, const void* x_disp, const int32_t* kept,
                           int E, int64_t C, int64_t H, int64_t I, const void* w1, const void* w3,
                           const void* b1, void* h, void* save0, void* save1);

// The second expert product, y_disp [E, C, H] fp32 = h W2 (+ b2), bf16 h and
// W2; part / part_bytes: the split-tail workspace, laid out and cleared as
// moe_expert_ffn's ws (null or too small: no split).
moe_status_t moe_ffn2(hipStream_t st, const void* h, const int32_t* kept, int E, int64_t C,
                      int64_t H, int64_t I, const void* w2, const void* b2, void* y_disp,
                      void* part, size_t part_bytes);

// The rows of the tokens none of whose copies was kept (slot[t, j] < 0 for
// every j), as moe_combine computes them: bf16 y [T, H] from the optional
// fp32 addend y_shared [T, H] and the weights; other rows are not touched.
// Arguments as moe_combine's (already checked by the caller).
moe_status_t moe_combine_empty(hipStream_t st, const int32_t* slot, const float* topk_w, int64_t T,
                               int64_t H, int k, const float* y_shared, void* y);
