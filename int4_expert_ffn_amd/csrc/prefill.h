// Prefill path (n_tokens > DECODE_MAX_TOKENS): token->expert sort and grouped
// MFMA GEMMs.  Interfaces between the runtime and the prefill kernels.
#pragma once
#include "decode.h"

namespace flint {

struct PrefillWS {
  char* base;
};

typedef int (*alloc_fn)(void** p, size_t bytes, const char* what);

int prefill_workspace_alloc(PrefillWS* ws, char** mem, alloc_fn alloc);

hipError_t launch_prefill_layer(const float* xin, float* out, int n, const LayerW& L, const PrefillWS& ws,
                                int* trace_ids, float* trace_w, hipStream_t s);

}  // namespace flint
