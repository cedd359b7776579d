/*
 * flint_moe.h - C ABI of the MI355X (gfx950) library for the Flint per-token
 * mixture-of-experts FFN block.
 *
 * The block (How to Run Flint Locally, "The architecture, from config.json",
 * table rows "Hidden size", "Routed experts", "Shared expert", and the
 * paragraph on the MoE block after the table; TandemLLM "21 Flint", 21.1 table
 * row "MLP"):
 *   a   = bf16(rmsnorm(x))                               block input (W4A16)
 *   s   = sigmoid(Wr a),  c = s + b                      router, bias for selection
 *   T   = the 6 experts with the largest c (ties: lower index)
 *   w_i = s_i / sum_{j in T} s_j                          normalised top-k weights
 *   y_e = Wd_e (silu(Wg_e a) * (Wu_e a))                  SwiGLU experts, size 512
 *   out = x + sum_{i in T} w_i y_i + y_shared             shared expert, size 1024
 * applied layer after layer over the 47 MoE layers (same section, table row
 * "Layers"), with the residual kept in fp32 between layers.  Every token is
 * independent: its result does not depend on the other tokens of the call
 * (Flint preview, "What is in it": batched requests give the same output as
 * running alone).
 *
 * Weight format (the library's own int4 layout; the pages publish weights in
 * formats not present here): symmetric two's-complement int4 codes in [-8, 7],
 * two per byte along the input dimension K (byte j of a row holds k = 2j in
 * bits 0-3 and k = 2j + 1 in bits 4-7), and one bf16 scale per (row, group of
 * FLINT_GROUP consecutive k): W[r][k] = code[r][k] * scale[r][k / FLINT_GROUP].
 * Weights are read as given and copied losslessly into library-owned memory at
 * create time (vLLM recipe "Flint", guide "Overview": the NVFP4 checkpoint is
 * repacked losslessly at load and run weight-only with bf16 activations).
 *
 * Errors: every call returns FLINT_OK (0) or a negative status; the text of the
 * last failure on the calling thread is flint_moe_last_error().  Arguments are
 * validated before anything is enqueued.  Faults inside kernels surface at the
 * caller's stream synchronisation; flint_moe_status() reports the library's own
 * device-side checks.
 */
#ifndef FLINT_MOE_H
#define FLINT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fixed Flint dimensions (config table of the pages). */
#define FLINT_HIDDEN       2048  /* H */
#define FLINT_EXPERTS      256   /* E, routed experts per layer */
#define FLINT_EXPERT_SIZE  512   /* I */
#define FLINT_SHARED_SIZE  1024  /* I_s */
#define FLINT_TOP_K        6
#define FLINT_GROUP        128   /* K-group of one bf16 scale */
#define FLINT_MAX_LAYERS   64
#define FLINT_MAX_TOKENS   2048

#define FLINT_OK                 0
#define FLINT_ERR_INVALID_ARG   -1  /* null pointer, bad count, range or alignment */
#define FLINT_ERR_OUT_OF_MEMORY -2  /* device allocation failed */
#define FLINT_ERR_HIP           -3  /* HIP runtime or launch error */
#define FLINT_ERR_UNSUPPORTED   -4  /* request outside what this build supports */
#define FLINT_ERR_DEVICE        -5  /* a device-side check fired (see last_error) */

typedef struct flint_moe* flint_moe_t;

/* One int4 matrix: codes [rows][K/2] bytes and scales [rows][K/FLINT_GROUP]
 * bf16 bit patterns, both row-major, device pointers.  For per-expert
 * matrices the experts are stored one after another (expert-major). */
typedef struct {
  const uint8_t* codes;
  const uint16_t* scales;
} flint_q4;

/* One MoE layer, all device pointers (any alignment: create copies them).
 *   router_w    [E][H]   bf16 bits
 *   router_bias [E]      fp32
 *   gate, up    [E][I][H/2] codes,  [E][I][H/G] scales
 *   down        [E][H][I/2] codes,  [E][H][I/G] scales
 *   sh_gate, sh_up  [I_s][H/2] codes, [I_s][H/G] scales
 *   sh_down     [H][I_s/2] codes,   [H][I_s/G] scales                       */
typedef struct {
  const uint16_t* router_w;
  const float* router_bias;
  flint_q4 gate, up, down;
  flint_q4 sh_gate, sh_up, sh_down;
} flint_moe_layer;

/* Create a handle holding n_layers layers (1 <= n_layers <= FLINT_MAX_LAYERS)
 * on the current HIP device.  Synchronous: the weights are copied into memory
 * the library owns, so the caller may free its buffers when the call returns.
 * Besides the copy as given, the library keeps a second copy of every int4
 * matrix and its scales rearranged for the prefill GEMMs (same size), so a
 * handle holds about twice the weight bytes (about 0.84 GB per layer).
 * `weights` is a host array of n_layers descriptors of device pointers.
 * On failure *out is set to NULL and nothing is leaked.  Test hook: with the
 * environment variable FLINT_MOE_FAIL_ALLOC=k (k >= 1), the k-th device
 * allocation of the call fails with FLINT_ERR_OUT_OF_MEMORY. */
int flint_moe_create(const flint_moe_layer* weights, int n_layers, flint_moe_t* out);

/* Create a handle for weights in the fp16-intermediate pack form (TandemLLM
 * "21 Flint", 21.2: the packs divide each routed expert's up projection by a
 * power of two, expert_interm_div, so that the SwiGLU outputs of the top
 * layers fit fp16; the factor is restored on the routing weights at run time).
 * `weights` as for flint_moe_create, with every routed expert's up-projection
 * scales already divided by interm_div (a power of two in [1, 32768]; 128 in
 * the pages' packs); the shared expert is not divided.  forward on such a
 * handle rounds the SwiGLU output of every expert (routed and shared) to fp16,
 * nearest even (overflow gives inf), before its down projection, and scales
 * the routed weights by interm_div in the combine.  It is implemented for
 * decode calls (1 <= n_tokens <= 16) on GPUs that run the persistent decode
 * kernel, each token's result bitwise the same as running it alone; prefill
 * calls (n_tokens > 16) and the per-layer decode mode return
 * FLINT_ERR_UNSUPPORTED.  interm_div = 0 is flint_moe_create. */
int flint_moe_create_fp16_interm(const flint_moe_layer* weights, int n_layers, int interm_div,
                                 flint_moe_t* out);

/* Apply layers [layer_begin, layer_end) to n_tokens independent fp32 residual
 * rows x [n_tokens][H] (device), writing out [n_tokens][H] (device).  out == x
 * is allowed; partial overlap is not.  1 <= n_tokens <= FLINT_MAX_TOKENS and
 * 0 <= layer_begin < layer_end <= n_layers.  Asynchronous on `stream` (a
 * hipStream_t; NULL = the default stream).  One handle serves one stream at a
 * time: calls on a handle must not overlap.  Decode calls (n_tokens <= 16)
 * need the whole GPU at once: a decode call on another stream than the
 * previous decode call on the device (of any handle in this process) waits
 * for that call.  If other work keeps part of the GPU busy for more than a
 * second, the call stops and flint_moe_status reports FLINT_ERR_DEVICE.
 * A call must not be captured into a HIP graph for replay: each call takes
 * per-call state from the host (the tags and slot parity of its exchanges
 * between workgroups).  For n_tokens <= 16 each token's
 * result is bitwise independent of n_tokens (decode path).  Larger calls take
 * the prefill path: tokens sorted by expert, grouped GEMMs on the matrix
 * cores, the SwiGLU output kept as two bf16 parts (about 16 significant bits)
 * for the down projection; deterministic, but not bitwise equal to the decode
 * path.  Each token is still routed and combined independently
 * (How to Run Flint Locally, "What vLLM changed": prefill runs the same
 * block over many tokens). */
int flint_moe_forward(flint_moe_t h, const float* x, int n_tokens, int layer_begin,
                      int layer_end, float* out, void* stream);

/* Record each layer's selection: ids [n_layers][capacity][FLINT_TOP_K] int32
 * and weights [n_layers][capacity][FLINT_TOP_K] fp32 (device buffers, ordered
 * by decreasing selection score), written by forward for the layers it runs.
 * NULL ids disables tracing.  While tracing, forward rejects n_tokens above
 * `capacity`. */
int flint_moe_set_trace(flint_moe_t h, int32_t* ids, float* weights, int capacity);

/* Blocking: wait for the handle's work on `stream` and report FLINT_ERR_DEVICE
 * if a device-side check fired (for example a bounded wait that expired). */
int flint_moe_status(flint_moe_t h, void* stream);

/* Testing hook.  Decode calls tag the words they exchange between workgroups
 * with a per-call counter that advances by 256 each call; when it would wrap,
 * the call clears the exchange buffers first and restarts the counter.  This
 * sets the counter so that a test reaches that branch in a few calls.
 * `epoch` must be a multiple of 256 and not below the current value (a lower
 * one could match tags left by earlier calls): FLINT_ERR_INVALID_ARG
 * otherwise.  Not thread-safe with respect to calls on the same handle. */
int flint_moe_debug_set_epoch(flint_moe_t h, uint32_t epoch);

/* Testing hook.  The number of device allocations that the process's handles
 * hold right now (each create makes 10 and destroy releases them; a failed
 * create releases those it had made before it returns).  Device-level free
 * memory cannot show this exactly, since the HIP runtime may keep freed blocks
 * for reuse and hand them back to the device later.  Never fails. */
int flint_moe_debug_live_allocations(void);

/* Release the handle and its device memory.  NULL is ignored. */
void flint_moe_destroy(flint_moe_t h);

/* Text of the last failure on the calling thread ("" if none). */
const char* flint_moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FLINT_MOE_H */
