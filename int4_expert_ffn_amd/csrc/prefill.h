// Prefill path (DECODE_MAX_TOKENS < n_tokens <= FLINT_MAX_TOKENS): per layer,
// the block input of every token, a router GEMM, top-6 per token, a
// deterministic token -> expert sort, and MFMA grouped GEMMs for the routed
// experts plus dense GEMMs for the shared expert, with a fixed-order combine.
#pragma once
#include "decode.h"

namespace flint {

constexpr int PF_TM = 32;                                   // (token, slot) pairs per routed GEMM tile
constexpr int PF_BW = FLINT_MAX_TOKENS / 32;                // bitmap words per expert
constexpr int PF_MAX_TILES = (FLINT_MAX_TOKENS * TOPK + PF_TM - 1) / PF_TM + E;

// Device workspace, sized for FLINT_MAX_TOKENS tokens.
struct PrefillWS {
  uint16_t* a;         // [n][H] block input, bf16, 8-element chunks in pair order
  float* z;            // [n][E] router logits
  int* ids;            // [n][TOPK] picks (decreasing score)
  float* w;            // [n][TOPK] routing weights
  uint32_t* bitmap;    // [E][PF_BW] bit t: token t picked expert e
  int* offsets;        // [E + 1] first position of expert e's (token, slot) pairs
  int4* tiles;         // [PF_MAX_TILES] (expert, first position, rows, 0), grouped by XCD
  int* tile_start;     // [9] the tiles for XCD x (blockIdx % 8) are [tile_start[x], tile_start[x + 1])
  int* perm;           // [n * TOPK] pair t * TOPK + slot at each position (by expert, then token)
  uint16_t* h_hi;      // [n * TOPK][I] routed SwiGLU output by position: bf16 high part
  uint16_t* h_lo;      // [n * TOPK][I] bf16 of the remainder (h - hi); pair-order chunks
  float* y;            // [n * TOPK][H] routed down output by pair t * TOPK + slot
  uint16_t* hs_hi;     // [n][IS] shared SwiGLU output, high part
  uint16_t* hs_lo;     // [n][IS] remainder
};

typedef int (*alloc_fn)(void** p, size_t bytes, const char* what);

// Allocates the workspace in one block (*mem owns it).
int prefill_workspace_alloc(PrefillWS* ws, char** mem, alloc_fn alloc);

// Tile-major copy of a layer's int4 matrices, the layout the prefill GEMMs
// stream: for rows 32 b .. 32 b + 31 of a matrix with K codes per row
// (K / G groups), the codes of group g are two contiguous 1 KB runs
// [b][g][i][lane][16 bytes], lane = 32 hl + r holding bytes 64 g + 32 hl + 16 i
// of row 32 b + r, so that one 16-byte load per lane gives a wave the MFMA
// operands of 32 rows; the scales are [b][g][r].  Each tensor keeps its
// row-major size.  dst's router and bias are not used.
hipError_t prefill_pack_layer(const LayerW& src, const LayerW& dst, hipStream_t s);

// One layer for n tokens: out = x + moe(rmsnorm(x)).  out may equal xin.
// L: the layer (router and bias are read from it), P: its tile-major copy.
// trace_ids / trace_w (may be null) receive the picks and weights [n][TOPK].
hipError_t launch_prefill_layer(const float* xin, float* out, int n, const LayerW& L, const LayerW& P,
                                const PrefillWS& ws, int* trace_ids, float* trace_w, hipStream_t s);

}  // namespace flint
