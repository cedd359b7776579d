// The model's other int4 matrix-vector products per decode token: the dense
// SwiGLU MLP of layers 0 and 1 and the output head.
#pragma once
#include "flint_dense.h"
#include "flint_device.h"

namespace flint {

constexpr int DENSE_MAX_TOKENS = FLINT_DENSE_MAX_TOKENS;

// h[t][r] = silu(Wg[r] . a_t) * (Wu[r] . a_t), a_t = bf16(rmsnorm(x_t)), for
// r < inter; then out[t][c] = x[t][c] + Wd[c] . h_t.  out may equal x.
hipError_t launch_dense_mlp(const uint8_t* gate, const uint16_t* gate_s, const uint8_t* up, const uint16_t* up_s,
                            const uint8_t* down, const uint16_t* down_s, int inter, const float* x, int n, float* h,
                            float* out, hipStream_t s);

// logits[t][r] = W[r] . a_t for r < rows.
hipError_t launch_head(const uint8_t* codes, const uint16_t* scales, int rows, const float* x, int n, float* logits,
                       hipStream_t s);

}  // namespace flint
