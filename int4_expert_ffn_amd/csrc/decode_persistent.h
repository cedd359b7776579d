// Persistent decode kernel: arguments and launch entry points.
#pragma once
#include "decode.h"

namespace flint {

constexpr int NWG = 256;   // workgroups of the persistent kernel: one per CU of an MI355X

struct PersistArgs {
  const float* x;          // [n][H] input residual (caller)
  float* out;              // [n][H] output residual (caller; may equal x)
  int n, l0, l1;
  LayerW base;             // pointers of layer 0; layer l is at + l * layer_stride bytes
  size_t layer_stride;
  uint64_t* xz;            // [T][2][E][2] scores c then s (fp64 as two words each)
  uint64_t* xh;            // [T][TOPK*I + IS] h of routed slots, then shared
  uint64_t* xx;            // [T][H] residual between layers
  int* trace_ids;          // [layers][cap][TOPK] or NULL
  float* trace_w;
  int trace_cap;
  int* err;                // device error word
  uint32_t epoch;          // tag base of this call (multiple of 256, never 0)
  // Single-token exchanges of x and h: untagged 32-bit values in one slot per
  // layer and call parity, re-armed to EMPTY_WORD by the call of the other parity.
  uint32_t* vx;            // [2][n_layers][H] residual after each layer
  uint32_t* vh;            // [2][n_layers][TOPK*I + IS] h of each layer, workgroup-major
  int n_layers;            // layers of the handle (every one is re-armed)
  int parity;              // half of vx / vh that this call writes
  float interm_mult;       // 0: fp32 SwiGLU outputs; else fp16 ones, routed weights times this
};

// Value of an exchange slot that has not been written in the current call (a
// NaN pattern that published values never carry: NaNs are published as the
// canonical quiet NaN).
constexpr uint32_t EMPTY_WORD = 0xFFFFFFFFu;

__host__ __device__ inline LayerW layer_at(const LayerW& b, size_t stride, int l) {
  const size_t o = stride * (size_t)l;
  auto m = [o](auto* p) { return reinterpret_cast<decltype(p)>(reinterpret_cast<const char*>(p) + o); };
  LayerW r;
  r.router = m(b.router);
  r.bias = m(b.bias);
  r.gate = m(b.gate);
  r.gate_s = m(b.gate_s);
  r.up = m(b.up);
  r.up_s = m(b.up_s);
  r.down = m(b.down);
  r.down_s = m(b.down_s);
  r.sh_gate = m(b.sh_gate);
  r.sh_gate_s = m(b.sh_gate_s);
  r.sh_up = m(b.sh_up);
  r.sh_up_s = m(b.sh_up_s);
  r.sh_down = m(b.sh_down);
  r.sh_down_s = m(b.sh_down_s);
  return r;
}

// words in each exchange buffer
constexpr size_t XZ_WORDS = (size_t)DECODE_MAX_TOKENS * E * 4;
constexpr size_t XH_WORDS = (size_t)DECODE_MAX_TOKENS * (TOPK * I + IS);
constexpr size_t XX_WORDS = (size_t)DECODE_MAX_TOKENS * H;

// 32-bit words in each single-token exchange slot array (both parities)
inline size_t vx_words(int n_layers) { return (size_t)2 * n_layers * H; }
inline size_t vh_words(int n_layers) { return (size_t)2 * n_layers * (TOPK * I + IS); }

hipError_t launch_decode_persistent(const PersistArgs& args, hipStream_t s);
hipError_t clear_exchange(uint64_t* p, size_t n_words, hipStream_t s);

}  // namespace flint
