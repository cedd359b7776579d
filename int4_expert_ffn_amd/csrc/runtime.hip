// C ABI of the Flint MoE library: handle, argument validation, the
// library-owned weight arena, workspaces, tracing and error reporting.
#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "attn.h"
#include "decode.h"
#include "decode_persistent.h"
#include "dense.h"
#include "prefill.h"

using namespace flint;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int fail_hip(hipError_t e, const char* what) {
  return fail(FLINT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t ALIGN = 256;
size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

// byte sizes of one layer's tensors, in arena order
struct LayerSizes {
  size_t router = (size_t)E * H * 2, bias = (size_t)E * 4;
  size_t gate = (size_t)E * I * (H / 2), gate_s = (size_t)E * I * (H / G) * 2;
  size_t down = (size_t)E * H * (I / 2), down_s = (size_t)E * H * (I / G) * 2;
  size_t sh_gu = (size_t)IS * (H / 2), sh_gu_s = (size_t)IS * (H / G) * 2;
  size_t sh_down = (size_t)H * (IS / 2), sh_down_s = (size_t)H * (IS / G) * 2;
  size_t list[14] = {router, bias, gate, gate_s, gate, gate_s, down, down_s,
                     sh_gu, sh_gu_s, sh_gu, sh_gu_s, sh_down, sh_down_s};
  // the row-major tensors, then the tile-major copies of tensors 2..13 (the
  // int4 matrices and their scales) that the prefill path streams
  size_t row_major() const {
    size_t t = 0;
    for (size_t s : list) t += align_up(s);
    return t;
  }
  size_t total() const {
    size_t t = row_major();
    for (int i = 2; i < 14; ++i) t += align_up(list[i]);
    return t;
  }
};

}  // namespace

struct flint_moe {
  int device = -1;
  int n_layers = 0;
  char* arena = nullptr;
  std::vector<LayerW> layers;
  std::vector<LayerW> players;   // tile-major copies of the int4 matrices (prefill)
  DecodeWS dws{};
  char* dws_mem = nullptr;
  PrefillWS pws{};
  char* pws_mem = nullptr;
  int* dev_error = nullptr;  // device-side check word
  int32_t* trace_ids = nullptr;
  float* trace_w = nullptr;
  int trace_capacity = 0;
  // persistent decode
  bool persistent = false;
  LayerW* layers_dev = nullptr;
  size_t layer_stride = 0;
  uint64_t* xz = nullptr;
  uint64_t* xh = nullptr;
  uint64_t* xx = nullptr;
  uint32_t epoch = 0;
  uint32_t* vx = nullptr;   // single-token exchange slots, two call parities
  uint32_t* vh = nullptr;
  int parity = 0;           // parity of the next single-token call
  int interm_div = 0;       // 0: fp32 SwiGLU outputs; else the fp16-intermediate form with this divisor
};

// Device allocations held by all handles of the process (every one is made by
// checked_malloc below and released by dev_free).
static std::atomic<int> g_live_allocs{0};

static void dev_free(void* p) {
  if (!p) return;
  (void)hipFree(p);
  g_live_allocs.fetch_sub(1, std::memory_order_relaxed);
}

static void release(flint_moe* h) {
  if (!h) return;
  if (h->device >= 0) (void)hipSetDevice(h->device);
  dev_free(h->arena);
  dev_free(h->dws_mem);
  dev_free(h->pws_mem);
  dev_free(h->dev_error);
  dev_free(h->layers_dev);
  dev_free(h->xz);
  dev_free(h->xh);
  dev_free(h->xx);
  dev_free(h->vx);
  dev_free(h->vh);
  delete h;
}

// Test hook: FLINT_MOE_FAIL_ALLOC=k (k >= 1) makes the k-th device allocation
// of a create call fail as if the device were out of memory, so that every
// partial-release path of create can be exercised.
static thread_local int g_alloc_count = 0;

static int checked_malloc(void** p, size_t bytes, const char* what) {
  const char* inj = getenv("FLINT_MOE_FAIL_ALLOC");
  if (inj && ++g_alloc_count == atoi(inj)) {
    *p = nullptr;
    return fail(FLINT_ERR_OUT_OF_MEMORY, "allocation %d (%zu bytes for %s) failed (injected)", g_alloc_count,
                bytes, what);
  }
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
      return fail(FLINT_ERR_OUT_OF_MEMORY, "allocation of %zu bytes for %s failed", bytes, what);
    return fail_hip(e, "hipMalloc");
  }
  g_live_allocs.fetch_add(1, std::memory_order_relaxed);
  return FLINT_OK;
}

extern "C" {

const char* flint_moe_last_error(void) { return g_last_error.c_str(); }

int flint_moe_create(const flint_moe_layer* weights, int n_layers, flint_moe_t* out) {
  return flint_moe_create_fp16_interm(weights, n_layers, 0, out);
}

int flint_moe_create_fp16_interm(const flint_moe_layer* weights, int n_layers, int interm_div, flint_moe_t* out) {
  if (!out) return fail(FLINT_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (interm_div != 0 && (interm_div < 1 || interm_div > (1 << 15) || (interm_div & (interm_div - 1)) != 0))
    return fail(FLINT_ERR_INVALID_ARG, "interm_div = %d is not a power of two in [1, 32768]", interm_div);
  if (!weights) return fail(FLINT_ERR_INVALID_ARG, "weights is NULL");
  if (n_layers < 1 || n_layers > FLINT_MAX_LAYERS)
    return fail(FLINT_ERR_INVALID_ARG, "n_layers = %d outside [1, %d]", n_layers, FLINT_MAX_LAYERS);
  for (int l = 0; l < n_layers; ++l) {
    const flint_moe_layer& w = weights[l];
    const void* ptrs[14] = {w.router_w, w.router_bias, w.gate.codes, w.gate.scales, w.up.codes, w.up.scales,
                            w.down.codes, w.down.scales, w.sh_gate.codes, w.sh_gate.scales, w.sh_up.codes,
                            w.sh_up.scales, w.sh_down.codes, w.sh_down.scales};
    for (int i = 0; i < 14; ++i)
      if (!ptrs[i]) return fail(FLINT_ERR_INVALID_ARG, "layer %d: tensor %d is NULL", l, i);
  }
  flint_moe* h = new flint_moe();
  g_alloc_count = 0;
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) { int r = fail_hip(e, "hipGetDevice"); h->device = -1; release(h); return r; }
  h->n_layers = n_layers;
  h->interm_div = interm_div;
  LayerSizes sz;
  const size_t per_layer = sz.total();
  int rc = checked_malloc((void**)&h->arena, per_layer * n_layers, "weights");
  if (rc) { release(h); return rc; }
  h->layers.resize(n_layers);
  h->players.resize(n_layers);
  h->layer_stride = per_layer;
  for (int l = 0; l < n_layers; ++l) {
    const flint_moe_layer& w = weights[l];
    const void* src[14] = {w.router_w, w.router_bias, w.gate.codes, w.gate.scales, w.up.codes, w.up.scales,
                           w.down.codes, w.down.scales, w.sh_gate.codes, w.sh_gate.scales, w.sh_up.codes,
                           w.sh_up.scales, w.sh_down.codes, w.sh_down.scales};
    char* base = h->arena + per_layer * l;
    char* dst[14];
    size_t off = 0;
    for (int i = 0; i < 14; ++i) {
      dst[i] = base + off;
      e = hipMemcpy(dst[i], src[i], sz.list[i], hipMemcpyDefault);
      if (e != hipSuccess) { rc = fail_hip(e, "copying weights"); release(h); return rc; }
      off += align_up(sz.list[i]);
    }
    LayerW& L = h->layers[l];
    L.router = (const uint16_t*)dst[0];
    L.bias = (const float*)dst[1];
    L.gate = (const uint8_t*)dst[2];
    L.gate_s = (const uint16_t*)dst[3];
    L.up = (const uint8_t*)dst[4];
    L.up_s = (const uint16_t*)dst[5];
    L.down = (const uint8_t*)dst[6];
    L.down_s = (const uint16_t*)dst[7];
    L.sh_gate = (const uint8_t*)dst[8];
    L.sh_gate_s = (const uint16_t*)dst[9];
    L.sh_up = (const uint8_t*)dst[10];
    L.sh_up_s = (const uint16_t*)dst[11];
    L.sh_down = (const uint8_t*)dst[12];
    L.sh_down_s = (const uint16_t*)dst[13];
    char* pk[14] = {};
    for (int i = 2; i < 14; ++i) {
      pk[i] = base + off;
      off += align_up(sz.list[i]);
    }
    LayerW& P = h->players[l];
    P = L;
    P.gate = (const uint8_t*)pk[2];
    P.gate_s = (const uint16_t*)pk[3];
    P.up = (const uint8_t*)pk[4];
    P.up_s = (const uint16_t*)pk[5];
    P.down = (const uint8_t*)pk[6];
    P.down_s = (const uint16_t*)pk[7];
    P.sh_gate = (const uint8_t*)pk[8];
    P.sh_gate_s = (const uint16_t*)pk[9];
    P.sh_up = (const uint8_t*)pk[10];
    P.sh_up_s = (const uint16_t*)pk[11];
    P.sh_down = (const uint8_t*)pk[12];
    P.sh_down_s = (const uint16_t*)pk[13];
    e = prefill_pack_layer(L, P, nullptr);
    if (e != hipSuccess) { rc = fail_hip(e, "packing weights"); release(h); return rc; }
  }
  // decode workspace
  {
    const int T = DECODE_MAX_TOKENS;
    size_t sizes[8] = {(size_t)T * H * 2, (size_t)T * 64 * 4, (size_t)T * E * 8, (size_t)T * E * 8,
                       (size_t)T * TOPK * 4, (size_t)T * TOPK * 4, (size_t)T * TOPK * I * 4, (size_t)T * IS * 4};
    size_t tot = 0;
    for (size_t s : sizes) tot += align_up(s);
    rc = checked_malloc((void**)&h->dws_mem, tot, "decode workspace");
    if (rc) { release(h); return rc; }
    char* p = h->dws_mem;
    void** dst[8] = {(void**)&h->dws.a, (void**)&h->dws.asum, (void**)&h->dws.c, (void**)&h->dws.s,
                     (void**)&h->dws.ids, (void**)&h->dws.w, (void**)&h->dws.h, (void**)&h->dws.hsh};
    for (int i = 0; i < 8; ++i) { *dst[i] = p; p += align_up(sizes[i]); }
  }
  rc = prefill_workspace_alloc(&h->pws, &h->pws_mem, checked_malloc);
  if (rc) { release(h); return rc; }
  rc = checked_malloc((void**)&h->dev_error, 256, "error word");
  if (rc) { release(h); return rc; }
  e = hipMemset(h->dev_error, 0, 256);
  if (e != hipSuccess) { rc = fail_hip(e, "create"); release(h); return rc; }
  // persistent decode: needs exactly NWG compute units, all resident at once
  // (the device must support the co-resident launch model)
  {
    int cus = 0, coop = 0;
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device);
    (void)hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, h->device);
    const char* mode = getenv("FLINT_MOE_DECODE");
    const bool layered = mode && strcmp(mode, "layered") == 0;
    h->persistent = !layered && cus == NWG && coop;
    rc = checked_malloc((void**)&h->layers_dev, sizeof(LayerW) * n_layers, "layer table");
    if (!rc) rc = checked_malloc((void**)&h->xz, XZ_WORDS * 8, "exchange z");
    if (!rc) rc = checked_malloc((void**)&h->xh, XH_WORDS * 8, "exchange h");
    if (!rc) rc = checked_malloc((void**)&h->xx, XX_WORDS * 8, "exchange x");
    if (!rc) rc = checked_malloc((void**)&h->vx, vx_words(n_layers) * 4, "exchange slots x");
    if (!rc) rc = checked_malloc((void**)&h->vh, vh_words(n_layers) * 4, "exchange slots h");
    if (rc) { release(h); return rc; }
    e = hipMemcpy(h->layers_dev, h->layers.data(), sizeof(LayerW) * n_layers, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemset(h->xz, 0, XZ_WORDS * 8);
    if (e == hipSuccess) e = hipMemset(h->xh, 0, XH_WORDS * 8);
    if (e == hipSuccess) e = hipMemset(h->xx, 0, XX_WORDS * 8);
    static_assert(EMPTY_WORD == 0xFFFFFFFFu, "slots are armed with 0xFF bytes");
    if (e == hipSuccess) e = hipMemset(h->vx, 0xFF, vx_words(n_layers) * 4);
    if (e == hipSuccess) e = hipMemset(h->vh, 0xFF, vh_words(n_layers) * 4);
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) { rc = fail_hip(e, "create"); release(h); return rc; }
  *out = h;
  return FLINT_OK;
}

int flint_moe_forward(flint_moe_t h, const float* x, int n_tokens, int layer_begin, int layer_end, float* out,
                      void* stream) {
  if (!h) return fail(FLINT_ERR_INVALID_ARG, "handle is NULL");
  if (!x || !out) return fail(FLINT_ERR_INVALID_ARG, "x or out is NULL");
  if (((uintptr_t)x | (uintptr_t)out) & 15) return fail(FLINT_ERR_INVALID_ARG, "x and out must be 16-byte aligned");
  if (n_tokens < 1 || n_tokens > FLINT_MAX_TOKENS)
    return fail(FLINT_ERR_INVALID_ARG, "n_tokens = %d outside [1, %d]", n_tokens, FLINT_MAX_TOKENS);
  if (h->interm_div && !(n_tokens <= DECODE_MAX_TOKENS && h->persistent))
    return fail(FLINT_ERR_UNSUPPORTED, "fp16 intermediates are implemented for calls of up to %d tokens on the "
                                       "persistent decode path (n_tokens = %d)", DECODE_MAX_TOKENS, n_tokens);
  if (layer_begin < 0 || layer_end > h->n_layers || layer_begin >= layer_end)
    return fail(FLINT_ERR_INVALID_ARG, "layer range [%d, %d) invalid for %d layers", layer_begin, layer_end,
                h->n_layers);
  const size_t bytes = (size_t)n_tokens * H * sizeof(float);
  const char *xb = (const char*)x, *ob = (const char*)out;
  if (xb != ob && xb < ob + bytes && ob < xb + bytes)
    return fail(FLINT_ERR_INVALID_ARG, "x and out overlap partially");
  if (h->trace_ids && n_tokens > h->trace_capacity)
    return fail(FLINT_ERR_INVALID_ARG, "n_tokens = %d above the trace capacity %d", n_tokens, h->trace_capacity);
  hipError_t e = hipSetDevice(h->device);
  if (e != hipSuccess) return fail_hip(e, "hipSetDevice");
  hipStream_t s = (hipStream_t)stream;
  if (n_tokens <= DECODE_MAX_TOKENS && h->persistent) {
    h->epoch += 256;
    if (h->epoch == 0 || h->epoch > 0xFFFFFE00u) {   // tags wrapped: start again from clean buffers
      e = clear_exchange(h->xz, XZ_WORDS, s);
      if (e == hipSuccess) e = clear_exchange(h->xh, XH_WORDS, s);
      if (e == hipSuccess) e = clear_exchange(h->xx, XX_WORDS, s);
      if (e != hipSuccess) return fail_hip(e, "clearing exchange buffers");
      h->epoch = 256;
    }
    PersistArgs a;
    a.x = x;
    a.out = out;
    a.n = n_tokens;
    a.l0 = layer_begin;
    a.l1 = layer_end;
    a.base = h->layers[0];
    a.layer_stride = h->layer_stride;
    a.xz = h->xz;
    a.xh = h->xh;
    a.xx = h->xx;
    a.trace_ids = h->trace_ids;
    a.trace_w = h->trace_w;
    a.trace_cap = h->trace_capacity;
    a.err = h->dev_error;
    a.epoch = h->epoch;
    a.vx = h->vx;
    a.vh = h->vh;
    a.n_layers = h->n_layers;
    a.parity = h->parity;
    a.interm_mult = (float)h->interm_div;
    e = launch_decode_persistent(a, s);
    if (e != hipSuccess) return fail_hip(e, "persistent decode launch");
    // a single-token call writes the slots of its parity and re-arms the
    // others, which the next single-token call then uses
    if (n_tokens == 1) h->parity ^= 1;
    return FLINT_OK;
  }
  for (int l = layer_begin; l < layer_end; ++l) {
    const float* xin = (l == layer_begin) ? x : out;
    int32_t* tid = h->trace_ids ? h->trace_ids + (size_t)l * h->trace_capacity * TOPK : nullptr;
    float* tw = h->trace_w ? h->trace_w + (size_t)l * h->trace_capacity * TOPK : nullptr;
    if (n_tokens <= DECODE_MAX_TOKENS)
      e = launch_decode_layer(xin, out, n_tokens, h->layers[l], h->dws, tid, tw, s);
    else
      e = launch_prefill_layer(xin, out, n_tokens, h->layers[l], h->players[l], h->pws, tid, tw, s);
    if (e != hipSuccess) return fail_hip(e, "kernel launch");
  }
  return FLINT_OK;
}

int flint_moe_set_trace(flint_moe_t h, int32_t* ids, float* weights, int capacity) {
  if (!h) return fail(FLINT_ERR_INVALID_ARG, "handle is NULL");
  if (!ids) {
    h->trace_ids = nullptr;
    h->trace_w = nullptr;
    h->trace_capacity = 0;
    return FLINT_OK;
  }
  if (!weights) return fail(FLINT_ERR_INVALID_ARG, "trace weights buffer is NULL");
  if (capacity < 1 || capacity > FLINT_MAX_TOKENS)
    return fail(FLINT_ERR_INVALID_ARG, "trace capacity %d outside [1, %d]", capacity, FLINT_MAX_TOKENS);
  h->trace_ids = ids;
  h->trace_w = weights;
  h->trace_capacity = capacity;
  return FLINT_OK;
}

int flint_moe_status(flint_moe_t h, void* stream) {
  if (!h) return fail(FLINT_ERR_INVALID_ARG, "handle is NULL");
  hipError_t e = hipSetDevice(h->device);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  int word = 0;
  if (e == hipSuccess) e = hipMemcpy(&word, h->dev_error, sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail_hip(e, "status");
  if (word) return fail(FLINT_ERR_DEVICE, "device-side check fired (code %d)", word);
  return FLINT_OK;
}

int flint_moe_debug_set_epoch(flint_moe_t h, uint32_t epoch) {
  if (!h) return fail(FLINT_ERR_INVALID_ARG, "handle is NULL");
  if (epoch & 255u) return fail(FLINT_ERR_INVALID_ARG, "epoch %u is not a multiple of 256", epoch);
  if (epoch < h->epoch) return fail(FLINT_ERR_INVALID_ARG, "epoch %u is below the current %u", epoch, h->epoch);
  h->epoch = epoch;
  return FLINT_OK;
}

int flint_moe_debug_live_allocations(void) { return g_live_allocs.load(std::memory_order_relaxed); }

void flint_moe_destroy(flint_moe_t h) { release(h); }

// ------------------------------------------------------------- dense MLP and head
static bool misaligned16(const void* p) { return ((uintptr_t)p & 15) != 0; }

static bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const char *pa = (const char*)a, *pb = (const char*)b;
  return pa < pb + nb && pb < pa + na;
}

static int check_q4(flint_q4 m, const char* name) {
  if (!m.codes || !m.scales) return fail(FLINT_ERR_INVALID_ARG, "%s: codes or scales is NULL", name);
  if (misaligned16(m.codes)) return fail(FLINT_ERR_INVALID_ARG, "%s: codes must be 16-byte aligned", name);
  if (misaligned16(m.scales)) return fail(FLINT_ERR_INVALID_ARG, "%s: scales must be 16-byte aligned", name);
  return FLINT_OK;
}

int flint_dense_mlp_forward(flint_q4 gate, flint_q4 up, flint_q4 down, int inter, const float* x, int n_tokens,
                            float* h, float* out, void* stream) {
  int rc;
  if ((rc = check_q4(gate, "gate")) || (rc = check_q4(up, "up")) || (rc = check_q4(down, "down"))) return rc;
  if (!x || !h || !out) return fail(FLINT_ERR_INVALID_ARG, "x, h or out is NULL");
  if (misaligned16(x) || misaligned16(h) || misaligned16(out))
    return fail(FLINT_ERR_INVALID_ARG, "x, h and out must be 16-byte aligned");
  if (n_tokens < 1 || n_tokens > FLINT_DENSE_MAX_TOKENS)
    return fail(FLINT_ERR_INVALID_ARG, "n_tokens = %d outside [1, %d]", n_tokens, FLINT_DENSE_MAX_TOKENS);
  if (inter < 2048 || inter > FLINT_DENSE_MLP_SIZE || inter % 2048)
    return fail(FLINT_ERR_INVALID_ARG, "inter = %d: a multiple of 2048 up to %d is required", inter,
                FLINT_DENSE_MLP_SIZE);
  const size_t xb = (size_t)n_tokens * H * sizeof(float), hb = (size_t)n_tokens * inter * sizeof(float);
  if ((const void*)x != (const void*)out && overlap(x, xb, out, xb))
    return fail(FLINT_ERR_INVALID_ARG, "x and out overlap partially");
  if (overlap(h, hb, x, xb) || overlap(h, hb, out, xb)) return fail(FLINT_ERR_INVALID_ARG, "h overlaps x or out");
  const hipError_t e = launch_dense_mlp(gate.codes, gate.scales, up.codes, up.scales, down.codes, down.scales, inter,
                                        x, n_tokens, h, out, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "dense MLP launch");
  return FLINT_OK;
}

int flint_head_forward(flint_q4 head, int rows, const float* x, int n_tokens, float* logits, void* stream) {
  int rc;
  if ((rc = check_q4(head, "head"))) return rc;
  if (!x || !logits) return fail(FLINT_ERR_INVALID_ARG, "x or logits is NULL");
  if (misaligned16(x) || misaligned16(logits)) return fail(FLINT_ERR_INVALID_ARG, "x and logits must be 16-byte aligned");
  if (n_tokens < 1 || n_tokens > FLINT_DENSE_MAX_TOKENS)
    return fail(FLINT_ERR_INVALID_ARG, "n_tokens = %d outside [1, %d]", n_tokens, FLINT_DENSE_MAX_TOKENS);
  if (rows < 1) return fail(FLINT_ERR_INVALID_ARG, "rows = %d must be positive", rows);
  if (overlap(x, (size_t)n_tokens * H * sizeof(float), logits, (size_t)n_tokens * rows * sizeof(float)))
    return fail(FLINT_ERR_INVALID_ARG, "logits overlaps x");
  const hipError_t e = launch_head(head.codes, head.scales, rows, x, n_tokens, logits, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "head launch");
  return FLINT_OK;
}

// ------------------------------------------------------------- decode attention
size_t flint_attn_workspace_bytes(int n_tokens, int max_seen) {
  if (n_tokens < 1 || n_tokens > FLINT_ATT_MAX_TOKENS || max_seen < 1) return 0;
  return attn_workspace_bytes(n_tokens, max_seen);
}

// Checks shared by the two attention entry points: the visible range of every
// token (first[t], count[t]) and the most positions any token sees.
static int attn_check(const float* q, const uint16_t* k, const uint16_t* v, int ring_rows, const float* sinks,
                      const int32_t* pos, int n_tokens, int window, float* out, int* first, int* count,
                      int* max_seen) {
  if (!q || !k || !v || !sinks || !pos || !out)
    return fail(FLINT_ERR_INVALID_ARG, "q, k, v, sinks, pos or out is NULL");
  if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(out))
    return fail(FLINT_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (n_tokens < 1 || n_tokens > FLINT_ATT_MAX_TOKENS)
    return fail(FLINT_ERR_INVALID_ARG, "n_tokens = %d outside [1, %d]", n_tokens, FLINT_ATT_MAX_TOKENS);
  if (ring_rows < 1) return fail(FLINT_ERR_INVALID_ARG, "ring_rows = %d must be positive", ring_rows);
  if (window < 0) return fail(FLINT_ERR_INVALID_ARG, "window = %d must not be negative", window);
  *max_seen = 0;
  for (int t = 0; t < n_tokens; ++t) {
    if (pos[t] < 0) return fail(FLINT_ERR_INVALID_ARG, "pos[%d] = %d is negative", t, pos[t]);
    first[t] = window ? std::max(0, pos[t] - window + 1) : 0;
    count[t] = pos[t] - first[t] + 1;
    if (count[t] > ring_rows)
      return fail(FLINT_ERR_INVALID_ARG, "token %d sees %d positions, more than the %d cache rows", t, count[t],
                  ring_rows);
    *max_seen = std::max(*max_seen, count[t]);
  }
  const size_t qb = (size_t)n_tokens * FLINT_ATT_Q_HEADS * FLINT_ATT_HEAD_DIM * sizeof(float);
  if (overlap(q, qb, out, qb)) return fail(FLINT_ERR_INVALID_ARG, "out overlaps q");
  return FLINT_OK;
}

int flint_attn_decode(const float* q, const uint16_t* k, const uint16_t* v, int ring_rows, const float* sinks,
                      const int32_t* pos, int n_tokens, int window, float* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int first[FLINT_ATT_MAX_TOKENS], count[FLINT_ATT_MAX_TOKENS], max_seen = 0;
  int rc = attn_check(q, k, v, ring_rows, sinks, pos, n_tokens, window, out, first, count, &max_seen);
  if (rc) return rc;
  if (!workspace) return fail(FLINT_ERR_INVALID_ARG, "workspace is NULL");
  if (misaligned16(workspace)) return fail(FLINT_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const size_t need = attn_workspace_bytes(n_tokens, max_seen);
  if (workspace_bytes < need)
    return fail(FLINT_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const size_t qb = (size_t)n_tokens * FLINT_ATT_Q_HEADS * FLINT_ATT_HEAD_DIM * sizeof(float);
  if (overlap(workspace, need, out, qb) || overlap(workspace, need, q, qb))
    return fail(FLINT_ERR_INVALID_ARG, "workspace overlaps q or out");
  const hipError_t e = launch_attn_decode(q, k, v, ring_rows, sinks, first, count, n_tokens, out, (float*)workspace,
                                          (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "attention launch");
  return FLINT_OK;
}

int flint_attn_decode_noalloc(const float* q, const uint16_t* k, const uint16_t* v, int ring_rows,
                              const float* sinks, const int32_t* pos, int n_tokens, int window, float* out,
                              void* stream) {
  int first[FLINT_ATT_MAX_TOKENS], count[FLINT_ATT_MAX_TOKENS], max_seen = 0;
  int rc = attn_check(q, k, v, ring_rows, sinks, pos, n_tokens, window, out, first, count, &max_seen);
  if (rc) return rc;
  const size_t need = attn_workspace_bytes(n_tokens, max_seen);
  if (need > ATTN_SCRATCH_BYTES)
    return fail(FLINT_ERR_INVALID_ARG,
                "%d tokens seeing up to %d positions need %zu bytes of scratch, above the %zu this entry point holds",
                n_tokens, max_seen, need, ATTN_SCRATCH_BYTES);
  float* ws = nullptr;
  hipError_t e = attn_scratch(&ws);
  if (e != hipSuccess) return fail_hip(e, "attention scratch address");
  e = launch_attn_decode(q, k, v, ring_rows, sinks, first, count, n_tokens, out, ws, (hipStream_t)stream);
  if (e != hipSuccess) return fail_hip(e, "attention launch");
  return FLINT_OK;
}

}  // extern "C"
