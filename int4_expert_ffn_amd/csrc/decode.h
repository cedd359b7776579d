// Internal interfaces between the runtime and the kernels.
#pragma once
#include "flint_device.h"

namespace flint {

// One layer's tensors in library-owned device memory (canonical layout).
struct LayerW {
  const uint16_t* router;    // [E][H] bf16
  const float* bias;         // [E]
  const uint8_t* gate;       // [E][I][H/2]
  const uint16_t* gate_s;    // [E][I][H/G]
  const uint8_t* up;
  const uint16_t* up_s;
  const uint8_t* down;       // [E][H][I/2]
  const uint16_t* down_s;    // [E][H][I/G]
  const uint8_t* sh_gate;    // [IS][H/2]
  const uint16_t* sh_gate_s; // [IS][H/G]
  const uint8_t* sh_up;
  const uint16_t* sh_up_s;
  const uint8_t* sh_down;    // [H][IS/2]
  const uint16_t* sh_down_s; // [H][IS/G]
};

// Decode workspace (device), sized for DECODE_MAX_TOKENS tokens.
struct DecodeWS {
  uint16_t* a;     // [T][H] block input, bf16, pair order
  float* asum;     // [T][64] sums of a over each lane chunk of 32 elements
  double* c;       // [T][E] selection scores sigmoid(z) + b
  double* s;       // [T][E] sigmoid(z)
  int* ids;        // [T][TOPK]
  float* w;        // [T][TOPK]
  float* h;        // [T][TOPK][I]
  float* hsh;      // [T][IS]
};

hipError_t launch_decode_layer(const float* xin, float* out, int n, const LayerW& L, const DecodeWS& ws,
                               int* trace_ids, float* trace_w, hipStream_t s);

}  // namespace flint
