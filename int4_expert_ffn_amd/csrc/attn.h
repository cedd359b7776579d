// Decode attention with learned sinks: launch entry points.
#pragma once
#include "flint_attn.h"
#include "flint_device.h"

namespace flint {

// Workspace bytes for n_tokens tokens of which none sees more than max_seen positions.
size_t attn_workspace_bytes(int n_tokens, int max_seen);

// The allocation-free entry point's scratch: FLINT_ATT_SCRATCH_BYTES of device
// memory per GPU (a file-scope array); its device address on the current
// device (looked up once per device).
constexpr size_t ATTN_SCRATCH_BYTES = FLINT_ATT_SCRATCH_BYTES;
constexpr int ATTN_MAX_DEVICES = 64;
hipError_t attn_scratch(float** p);

// Token t sees positions first[t] .. first[t] + count[t] - 1 (count >= 1),
// held at rows p % ring of k and v; host arrays.
hipError_t launch_attn_decode(const float* q, const uint16_t* k, const uint16_t* v, int ring, const float* sinks,
                              const int* first, const int* count, int n_tokens, float* out, float* ws,
                              hipStream_t s);

}  // namespace flint
