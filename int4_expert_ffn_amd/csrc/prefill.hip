// Prefill path: not built yet; forward() reports FLINT_ERR_UNSUPPORTED.
#include "prefill.h"

namespace flint {

int prefill_workspace_alloc(PrefillWS* ws, char** mem, alloc_fn) {
  ws->base = nullptr;
  *mem = nullptr;
  return FLINT_OK;
}

hipError_t launch_prefill_layer(const float*, float*, int, const LayerW&, const PrefillWS&, int*, float*,
                                hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace flint
