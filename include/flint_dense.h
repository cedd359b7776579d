/*
 * flint_dense.h - C ABI of the library's other int4 matrix-vector products of
 * one Flint decode step: the dense SwiGLU MLP of model layers 0 and 1 and the
 * output head.
 *
 * The pages give their shapes (How to Run Flint Locally, "The architecture,
 * from config.json": table row "Dense MLP size": width 6,144, used by the first
 * two layers;
 * table row "Vocabulary", 150,144; section "One decode step in bytes": the
 * lm_head is 150,144 x 2,048, every token reads all of it, and the research
 * system quantised it to 4 bits).  Both use the int4 format of flint_moe.h
 * (flint_q4: codes [rows][K/2], bf16 scales [rows][K/FLINT_GROUP], row-major,
 * device pointers) and the block input of the MoE layers:
 *   a = bf16(rmsnorm(x)), epsilon 1e-6, gain 1, fp32 accumulation of exact
 *   code x activation products.
 * Tokens are independent: each token's result is bitwise the same whatever
 * n_tokens is.  All calls are asynchronous on `stream` (a hipStream_t, NULL =
 * the default stream), validate their arguments before enqueuing anything,
 * return FLINT_OK or a negative status (text in flint_moe_last_error()), and
 * allocate nothing: the caller owns every buffer.
 */
#ifndef FLINT_DENSE_H
#define FLINT_DENSE_H

#include "flint_moe.h"

#ifdef __cplusplus
extern "C" {
#endif

#define FLINT_DENSE_MLP_SIZE   6144    /* width of the dense MLP of layers 0 and 1 */
#define FLINT_VOCAB            150144  /* rows of the output head */
#define FLINT_DENSE_MAX_TOKENS 16      /* tokens per call (decode) */

/* Dense SwiGLU MLP of one layer:
 *   a = bf16(rmsnorm(x_t));  h_t = silu(Wg a) * (Wu a);  out_t = x_t + Wd h_t
 * gate, up: [inter][FLINT_HIDDEN] int4; down: [FLINT_HIDDEN][inter] int4.
 * inter is a multiple of 2048 and at most FLINT_DENSE_MLP_SIZE.
 * x, out: fp32 [n_tokens][FLINT_HIDDEN]; out == x is allowed, partial overlap
 * is not.  h: fp32 [n_tokens][inter], written (the SwiGLU output, also a
 * result); it must not overlap x or out.  1 <= n_tokens <= FLINT_DENSE_MAX_TOKENS.
 * Pointers 16-byte aligned. */
int flint_dense_mlp_forward(flint_q4 gate, flint_q4 up, flint_q4 down, int inter, const float* x, int n_tokens,
                            float* h, float* out, void* stream);

/* Output head: logits_t[r] = sum_k W[r][k] a_t[k], a_t = bf16(rmsnorm(x_t)),
 * for r < rows.  head: [rows][FLINT_HIDDEN] int4, rows >= 1 (FLINT_VOCAB for
 * Flint).  x: fp32 [n_tokens][FLINT_HIDDEN]; logits: fp32 [n_tokens][rows],
 * not overlapping x.  1 <= n_tokens <= FLINT_DENSE_MAX_TOKENS.  Pointers
 * 16-byte aligned. */
int flint_head_forward(flint_q4 head, int rows, const float* x, int n_tokens, float* logits, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FLINT_DENSE_H */
