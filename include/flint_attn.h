/*
 * flint_attn.h - C ABI of the library's decode attention: one layer's
 * attention for up to 16 query tokens against a bf16 KV cache, with one
 * learned sink logit per query head.
 *
 * Shapes and rules from the pages (TandemLLM "21 Flint", 21.1 table rows
 * "attention", "sliding layers" and "full layers"; How to Run Flint Locally,
 * "Sinks and the 513-token window"): 32 query heads and 4 KV heads of
 * dimension 128; a window layer's token sees itself and the 512 positions
 * before it, and its cache is a ring of 640 rows; a full layer's token sees
 * every position; a sink is one more softmax slot whose logit is the head's
 * learned offset and which has no value vector.  Readings: query head h reads
 * KV head h / 8; scores are q . k / sqrt(128); q, k and v arrive already
 * RMS-normed and rotated (the projections, the QK norm, RoPE and the cache
 * write are not part of this call).
 *
 * For query token t at position pos[t], with first = max(0, pos[t] - window + 1)
 * (first = 0 when window == 0) and head h, g = h / 8:
 *   s_p   = q[t][h] . k[p % ring_rows][g] / sqrt(128),  p = first .. pos[t]
 *   out[t][h] = sum_p e^(s_p - M) v[p % ring_rows][g] / (e^(o_h - M) + sum_p e^(s_p - M))
 * with o_h = sinks[h] and M the largest of the s_p and o_h.  Scores, weights
 * and sums are fp32, every sum in a fixed order: results are deterministic
 * and each token's result is bitwise independent of n_tokens.
 *
 * All calls are asynchronous on `stream` (a hipStream_t, NULL = the default
 * stream), validate their arguments before enqueuing anything, return
 * FLINT_OK or a negative status (text in flint_moe_last_error()) and allocate
 * nothing: the caller owns every buffer, including the workspace.
 */
#ifndef FLINT_ATTN_H
#define FLINT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include "flint_moe.h"

#ifdef __cplusplus
extern "C" {
#endif

#define FLINT_ATT_Q_HEADS    32
#define FLINT_ATT_KV_HEADS   4
#define FLINT_ATT_HEAD_DIM   128
#define FLINT_ATT_WINDOW     513   /* positions a window layer's token sees */
#define FLINT_ATT_RING       640   /* cache rows of a window layer */
#define FLINT_ATT_MAX_TOKENS 16

/* Bytes of device workspace flint_attn_decode needs for n_tokens query tokens
 * of which none sees more than max_seen positions (0 if an argument is out of
 * range). */
size_t flint_attn_workspace_bytes(int n_tokens, int max_seen);

/* One layer's decode attention.
 *   q         fp32 [n_tokens][32][128], device
 *   k, v      bf16 bit patterns [ring_rows][4][128], device; position p at row
 *             p % ring_rows (its K and V already written)
 *   sinks     fp32 [32], device: the layer's sink logit per query head
 *   pos       int32 [n_tokens], HOST memory: each query token's position
 *   window    positions a token sees, ending at its own (FLINT_ATT_WINDOW on
 *             window layers); 0 = every position 0 .. pos (full layers)
 *   out       fp32 [n_tokens][32][128], device; must not overlap q
 *   workspace device, at least flint_attn_workspace_bytes(n_tokens, max_seen)
 *             bytes where max_seen is the most positions any token sees;
 *             workspace_bytes is its size
 * 1 <= n_tokens <= FLINT_ATT_MAX_TOKENS; pos[t] >= 0; every token's visible
 * positions must fit the ring (pos[t] - first + 1 <= ring_rows); q, k, v, out
 * and workspace 16-byte aligned.  FLINT_ERR_INVALID_ARG otherwise. */
int flint_attn_decode(const float* q, const uint16_t* k, const uint16_t* v, int ring_rows, const float* sinks,
                      const int32_t* pos, int n_tokens, int window, float* out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Size of the library's own scratch for flint_attn_decode_noalloc: 16 MiB of
 * device memory per GPU, held from the first such call on that GPU until the
 * process ends. */
#define FLINT_ATT_SCRATCH_BYTES ((size_t)16 << 20)

/* flint_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory around the call (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  The chunk partials go to
 * a fixed scratch array of FLINT_ATT_SCRATCH_BYTES that the library holds per
 * GPU; the call itself allocates nothing (its first call on a GPU looks up the
 * array's device address).  The same arguments, rules and results as
 * flint_attn_decode, bitwise; in addition flint_attn_workspace_bytes(n_tokens,
 * max_seen) must not exceed FLINT_ATT_SCRATCH_BYTES (FLINT_ERR_INVALID_ARG
 * otherwise: for one token, up to 253,952 visible positions; for 16 tokens,
 * up to 15,872 each).  Every call on one GPU uses that GPU's one scratch
 * array: calls that may run at the same time on one GPU (on different
 * streams, or from different threads) race and must be serialised by the
 * caller. */
int flint_attn_decode_noalloc(const float* q, const uint16_t* k, const uint16_t* v, int ring_rows,
                              const float* sinks, const int32_t* pos, int n_tokens, int window, float* out,
                              void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FLINT_ATTN_H */
