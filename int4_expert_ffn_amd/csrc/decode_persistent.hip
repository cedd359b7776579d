// Decode path, persistent form: one launch runs every layer of a forward call
// on 256 resident workgroups (one per CU), with no kernel boundaries between
// the dependent stages of a layer.
//
// Work of workgroup w (8 wavefronts) in layer l, for each token:
//   P0  block input a = bf16(rmsnorm(x_l)) (every workgroup, redundantly)
//   P1  router row w over all waves -> (c, s) published first; then shared-
//       expert gate/up row 4 w + wave on waves 0..3 -> h_shared
//   P2  all 256 (c, s) -> top-6 (every workgroup, redundantly); gate/up rows
//       of the distinct picked experts, spread over all waves -> h
//   P3  all h -> output row 8 w + wave (six routed down rows + shared down
//       row, fixed-order combine) -> x_{l+1}
// Values cross workgroups through exchange buffers of 64-bit words that carry
// a 32-bit payload and a 32-bit tag (call epoch, layer, stage).  Writers use
// relaxed agent-scope atomic stores, readers relaxed agent-scope atomic loads
// and wait until the tag matches; one word is read or written as a whole, so
// no fences are needed and no value is read before it is written.  Every wait
// is bounded: after one second a device error word is set and all workgroups
// leave the kernel.
//
// The arithmetic is the same code as the per-layer kernels (decode_common.h),
// so both launch modes give bitwise-identical results.
#include <hip/hip_fp16.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "decode_common.h"
#include "decode_persistent.h"

namespace flint {

constexpr int HW = TOPK * I + IS;                  // h words per token (routed, then shared)
constexpr long long SPIN_TICKS = 100000000LL;      // 1 s of the 100 MHz wall clock

// Phase timestamps for profiling builds only (-DFLINT_PHASE_TS): thread 0 of
// each workgroup records the 100 MHz wall clock at marker k of layer l into
// LDS (a global store would delay that wave's next poll: its memory counter
// retires in order), and copies them out when the kernel ends.
#ifdef FLINT_PHASE_TS
constexpr int TS_LAYERS = 48;
__device__ unsigned long long g_phase_ts[TS_LAYERS][16][NWG];
__device__ unsigned long long g_gather_ts[TS_LAYERS][4][4];
#define PHASE_MARK(k) \
  do { if (threadIdx.x == 0 && l < TS_LAYERS) ts_lds[l][k] = wall_clock64(); } while (0)
#define PUB_MARK(k) \
  do { if (threadIdx.x == 64 * PUB_WAVE && l < TS_LAYERS) ts_lds[l][k] = wall_clock64(); } while (0)
#define GATHER_PROBE(slot, v) \
  do { if (threadIdx.x == 0 && dbg_id >= 0 && dbg_layer < TS_LAYERS) gts_lds[dbg_layer][dbg_id][slot] = (v); } while (0)
extern "C" int flint_moe_debug_phase_ts(unsigned long long* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase_ts), sizeof(g_phase_ts));
}
extern "C" int flint_moe_debug_gather_ts(unsigned long long* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_gather_ts), sizeof(g_gather_ts));
}
#else
#define PHASE_MARK(k) do { } while (0)
#define PUB_MARK(k) do { } while (0)
#define GATHER_PROBE(slot, v) do { } while (0)
#endif

__device__ __forceinline__ void publish(uint64_t* p, uint32_t tag, uint32_t v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t load_word(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until words src[0..nwords) carry `tag`; store the payload of word j
// in dst[pos(j)].  Thread i handles words i + NT k, k < K.  Returns false on
// timeout (the device error word is then set).
#ifdef FLINT_PHASE_TS
typedef unsigned long long (*GtsLds)[4][4];
#else
typedef void* GtsLds;
#endif
template <int K, typename Pos, int NTHR = NT>
__device__ __forceinline__ bool gather(const uint64_t* src, int nwords, uint32_t tag, uint32_t* dst, int* err,
                                       Pos pos, int tid, int dbg_layer, int dbg_id, GtsLds gts_lds) {
  GATHER_PROBE(0, wall_clock64());
  unsigned long long iters = 0;
  uint64_t v[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int j = tid + NTHR * k;
    v[k] = (j < nwords) ? load_word(src + j) : ((uint64_t)tag << 32);
  }
  const long long t0 = wall_clock64();
  while (true) {
    bool all = true;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if ((uint32_t)(v[k] >> 32) != tag) {
        all = false;
        v[k] = load_word(src + tid + NTHR * k);
      }
    }
    if (iters++ == 0) GATHER_PROBE(1, wall_clock64());
    if (all) break;
    if (wall_clock64() - t0 > SPIN_TICKS) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
  GATHER_PROBE(2, wall_clock64());
  GATHER_PROBE(3, iters);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int j = tid + NTHR * k;
    if (j < nwords) dst[pos(j)] = (uint32_t)v[k];
  }
  return true;
}

// Single-token exchanges without tags.  A slot holds EMPTY_WORD until its
// producer stores the value with one 32-bit store, so a reader that sees
// anything else sees the whole value.  Pollers read 16 bytes per load with the
// sc1 cache policy, the policy the compiler gives agent-scope atomic loads on
// this chip: the load is served from the device-coherent level, never from a
// workgroup's or an XCD's stale copy.  Half the bytes of the tagged words, a
// quarter of the load instructions.
__device__ __forceinline__ void publish_value(uint32_t* p, float v) {
  const uint32_t u = (v != v) ? 0x7FC00000u : __float_as_uint(v);   // never EMPTY_WORD
  __hip_atomic_store(p, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint4 load_values16(__amdgpu_buffer_rsrc_t rs, int byte_offset) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  constexpr int SC1 = 16;   // cache-policy bit of the buffer instructions
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, byte_offset, 0, SC1);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bool has_empty(uint4 v) {
  return v.x == EMPTY_WORD || v.y == EMPTY_WORD || v.z == EMPTY_WORD || v.w == EMPTY_WORD;
}

// Wait until values src[0..nvals) (nvals a multiple of 4) are all written;
// hand values j .. j + 3 (j a multiple of 4) to sink(j, values).  Thread i
// polls the 16-byte groups i + NTHR k, k < K.  Returns false on timeout (the
// device error word is then set).
template <int K, typename Sink, int NTHR = NT>
__device__ __forceinline__ bool gather_values(const uint32_t* src, int nvals, int* err, Sink sink, int tid,
                                              int dbg_layer, int dbg_id, GtsLds gts_lds) {
  GATHER_PROBE(0, wall_clock64());
  unsigned long long iters = 0;
  const int ngroups = nvals >> 2;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(src), 0, nvals * 4,
                                                                      0x00020000);
  uint4 v[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int j = tid + NTHR * k;
    v[k] = (j < ngroups) ? load_values16(rs, 16 * j) : make_uint4(0u, 0u, 0u, 0u);
  }
  const long long t0 = wall_clock64();
  while (true) {
    // the buffer loads are plain reads to the compiler: keep each round's
    // loads from being merged with the previous round's
    asm volatile("" ::: "memory");
    bool all = true;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (has_empty(v[k])) {
        all = false;
        v[k] = load_values16(rs, 16 * (tid + NTHR * k));
      }
    }
    if (iters++ == 0) GATHER_PROBE(1, wall_clock64());
    if (all) break;
    if (wall_clock64() - t0 > SPIN_TICKS) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
  GATHER_PROBE(2, wall_clock64());
  GATHER_PROBE(3, iters);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int j = tid + NTHR * k;
    if (j < ngroups) sink(4 * j, v[k]);
  }
  return true;
}

struct Identity {
  __device__ int operator()(int j) const { return j; }
};

// (c, s) word j of a token, published as [c lo, c hi, s lo, s hi] per expert
// (one aligned 32-byte store per expert) -> c[E] then s[E] as fp64 halves
struct ZPos {
  __device__ int operator()(int j) const {
    const int e = j >> 2, p = j & 3;
    return p < 2 ? 2 * e + p : 2 * E + 2 * e + (p - 2);
  }
};

// h word j of a token (routed slots [TOPK][I], then shared [IS]) -> transposed position
struct HPos {
  __device__ int operator()(int j) const {
    return j < TOPK * I ? (j & ~(I - 1)) + transposed_pos(j & (I - 1), I / 32)
                        : TOPK * I + transposed_pos(j - TOPK * I, IS / 32);
  }
};

// Single-token h exchange, workgroup-major: workgroup w's 16 values (4 shared
// rows 4 w .., then 12 routed rows 12 w .. of the six slots) are the 128-byte
// run of words 16 w .. 16 w + 15, written by one store.  Word j -> h index ->
// transposed position.
struct HPosWG {
  __device__ int operator()(int j) const {
    const int w = j >> 4, k = j & 15;
    return HPos()(k < 4 ? TOPK * I + 4 * w + k : 12 * w + (k - 4));
  }
};

// Where the single-token gathers put their values in LDS: four values at a
// time, values j .. j + 3 of a 16-byte group (j a multiple of 4).  The layouts
// map each such group to four consecutive, 16-byte aligned LDS words (for h:
// a workgroup's run of 16 values splits into groups of one kind, shared or
// routed, each 4-aligned, and the transposed position keeps the low two bits
// of the index), so one address and one 16-byte store serve the group.
struct StoreAt {   // values j.. -> dst[j..]
  uint32_t* dst;
  __device__ void operator()(int j, uint4 v) const { *reinterpret_cast<uint4*>(dst + j) = v; }
};
struct StoreH {    // fp32 h words j.. (workgroup-major) -> their transposed positions
  uint32_t* dst;
  __device__ void operator()(int j, uint4 v) const { *reinterpret_cast<uint4*>(dst + HPosWG()(j)) = v; }
};
struct StoreH16 {  // words j.. = fp16 h values 2 j .. 2 j + 7 (low half first) -> fp32 at their positions
  float* dst;
  __device__ static float lo(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w & 0xFFFFu))); }
  __device__ static float hi(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w >> 16))); }
  __device__ void operator()(int j, uint4 v) const {
    *reinterpret_cast<float4*>(dst + HPosWG()(2 * j)) = make_float4(lo(v.x), hi(v.x), lo(v.y), hi(v.y));
    *reinterpret_cast<float4*>(dst + HPosWG()(2 * j + 4)) = make_float4(lo(v.z), hi(v.z), lo(v.w), hi(v.w));
  }
};

// fp16 bits of a value that is already exactly an fp16 value (or inf); NaN
// becomes the canonical quiet NaN, so a packed pair is never EMPTY_WORD.
__device__ __forceinline__ uint32_t fp16_bits(float v) {
  return (v != v) ? 0x7E00u : (uint32_t)__half_as_ushort(__float2half_rn(v));
}

// Role split inside a workgroup: on GFX9 a wavefront's memory counter retires
// loads and stores in issue order, so a poll issued after a store waits for
// that store's acknowledgement.  The last wave publishes each exchange (from
// LDS) and the other waves poll, so pollers never have a store in flight.
constexpr int PUB_WAVE = NWAVES - 1;
constexpr int NPOLL = NT - 64;   // polling threads: waves 0 .. NWAVES-2

// F16H: the fp16-intermediate form (TandemLLM "21 Flint", 21.2).  The up
// matrices of the routed experts arrive scaled down by a power of two, which
// keeps every SwiGLU output inside fp16's range; the combine multiplies the
// routing weights by the same power of two.
// Every expert's SwiGLU output is rounded to fp16; the h exchange carries two
// values per word; routed weights are scaled by A.interm_mult in the combine.
template <bool F16H>
__global__ void __launch_bounds__(NT) k_decode_persistent(PersistArgs A) {
  __shared__ __align__(16) uint4 a_lds[DECODE_MAX_TOKENS][256];
  __shared__ float asum_lds[DECODE_MAX_TOKENS][64];
  __shared__ float xown[DECODE_MAX_TOKENS][8];
  // gather destination, shared by the three exchanges of a layer (their
  // contents are never live together): x of one token [H], (c, s) of 4
  // tokens [4][4 E] as fp64 halves, h of one token [HW] in transposed order
  __shared__ __align__(16) uint32_t stage[HW];
  float* const xstage = reinterpret_cast<float*>(stage);
  uint32_t (*const zbuf)[4 * E] = reinterpret_cast<uint32_t (*)[4 * E]>(stage);
  float* const hbuf = reinterpret_cast<float*>(stage);
  static_assert(H <= HW && 4 * 4 * E <= HW, "gather staging too small");
  // this workgroup's h values before publication: at most 2 D routed rows
  // (D <= 16 * 6 distinct experts) times 16 tokens, plus 4 shared rows x 16
  constexpr int HLOC = 2 * DECODE_MAX_TOKENS * TOPK * DECODE_MAX_TOKENS + 4 * DECODE_MAX_TOKENS;
  __shared__ float hloc[HLOC];
  __shared__ int hloc_idx[HLOC];
  __shared__ float xnew[DECODE_MAX_TOKENS][8];
  __shared__ int ids_l[DECODE_MAX_TOKENS][TOPK];
  __shared__ float w_l[DECODE_MAX_TOKENS][TOPK];
  __shared__ int list[DECODE_MAX_TOKENS * TOPK];
  __shared__ int wave_tot[4];
  __shared__ double red[2][NWAVES];
  __shared__ double zpart[DECODE_MAX_TOKENS][NWAVES];
#ifdef FLINT_PHASE_TS
  __shared__ unsigned long long ts_lds[TS_LAYERS][16];
  __shared__ unsigned long long gts_lds[TS_LAYERS][4][4];
#else
  GtsLds gts_lds = nullptr;
#endif

  __shared__ int bail[2];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int w = blockIdx.x;
  constexpr int n = 1;   // this kernel runs one token; 2..16 run in the token-group kernels
  const bool poller = wave != PUB_WAVE;

  // Barrier that also tells every wave whether any thread timed out.  The
  // flags are sticky and used alternately: the reads after one such barrier
  // all happen before the next one, which is the earliest a thread can set the
  // other flag, so no read can see a later call's failure.
  if (tid < 2) bail[tid] = 0;
  int bail_par = 0;
  auto sync_or = [&](bool fail) {
    if (fail) bail[bail_par] = 1;
    wg_sync();
    const bool r = bail[bail_par] != 0;
    bail_par ^= 1;
    return r;
  };
  // Re-arm this workgroup's slots of the other parity for every layer (its x
  // rows 8 w .. 8 w + 7 and h words 16 w .. 16 w + 15, or 8 w .. 8 w + 7 with
  // two fp16 values per word): the next call writes them.  Runs on every way
  // out of the kernel.
  constexpr int HWORDS_WG = F16H ? 8 : 16;   // h words per workgroup
  constexpr int RQ = 2 + HWORDS_WG / 4;      // 16-byte pieces re-armed per layer
  const int other = A.parity ^ 1;
  auto rearm = [&]() {
    if (wave != PUB_WAVE) return;
    const uint4 empty = make_uint4(EMPTY_WORD, EMPTY_WORD, EMPTY_WORD, EMPTY_WORD);
    for (int i = lane; i < RQ * A.n_layers; i += 64) {
      const int lc = i / RQ, q = i % RQ;
      const size_t slot = (size_t)other * A.n_layers + lc;
      uint32_t* p = q < 2 ? A.vx + slot * H + 8 * w + 4 * q : A.vh + slot * HW + HWORDS_WG * w + 4 * (q - 2);
      *reinterpret_cast<uint4*>(p) = empty;
    }
  };
  wg_sync();

  for (int l = A.l0; l < A.l1; ++l) {
    const LayerW L = layer_at(A.base, A.layer_stride, l);
    const uint32_t tag = A.epoch + ((uint32_t)l << 2);
    uint32_t* const vh_l = A.vh + ((size_t)A.parity * A.n_layers + l) * HW;

    // this workgroup's router row (8 bytes per thread) and bias, requested
    // before the x exchange so that its wait hides them
    const uint2 rw = load_router_part(L.router + (size_t)w * H);
    const float bias_w = L.bias[w];

    // ---------------- P0: block input of every token
    PHASE_MARK(0);
    for (int t = 0; t < n; ++t) {
      bool ok = true;
      if (l == A.l0) {
        if (tid < H / 4) reinterpret_cast<float4*>(xstage)[tid] = reinterpret_cast<const float4*>(A.x + (size_t)t * H)[tid];
      } else if (poller) {
        ok = gather_values<(H / 4 + NPOLL - 1) / NPOLL, StoreAt, NPOLL>(
            A.vx + ((size_t)A.parity * A.n_layers + (l - 1)) * H, H, A.err,
            StoreAt{reinterpret_cast<uint32_t*>(xstage)}, tid, l, 0, gts_lds);
      }
      if (sync_or(!ok)) { rearm(); return; }
      if (t == 0) PHASE_MARK(1);
      const float4 xv = reinterpret_cast<const float4*>(xstage)[tid];
      if ((tid >> 1) == w) {   // this workgroup's 8 output rows, kept for the residual
        float* xo = xown[t] + 4 * (tid & 1);
        xo[0] = xv.x; xo[1] = xv.y; xo[2] = xv.z; xo[3] = xv.w;
      }
      block_input(xv, reinterpret_cast<uint32_t*>(a_lds[t]), asum_lds[t], red[t & 1]);
      wg_sync();   // xstage is rewritten by the next token
    }

    // ---------------- P1: router row w over all waves -> the publisher wave writes (c, s)
    PHASE_MARK(2);
    for (int t = 0; t < n; ++t) {
      const double p = router_part(rw, a_lds[t]);
      if (lane == 0) zpart[t][wave] = p;
    }
    wg_sync();
    PUB_MARK(11);
    if (wave == PUB_WAVE && lane < 4) {   // lane p writes word p of [c lo, c hi, s lo, s hi]: one 32-byte store
      double sv, cv;
      router_scores(zpart[0], bias_w, sv, cv);
      const unsigned long long v = (unsigned long long)__double_as_longlong(lane < 2 ? cv : sv);
      publish(A.xz + 4 * w + lane, tag, (lane & 1) ? (uint32_t)(v >> 32) : (uint32_t)v);
    }

    // shared-expert gate/up row 4 w + wave of waves 0..3, requested before the
    // (c, s) exchange so that its wait hides them
    uint4 shg = make_uint4(0u, 0u, 0u, 0u), shu = shg;
    uint32_t shsg = 0u, shsu = 0u;
    if (wave < 4) {
      const size_t r = (size_t)4 * w + wave;
      shg = reinterpret_cast<const uint4*>(L.sh_gate + r * (H / 2))[lane];
      shu = reinterpret_cast<const uint4*>(L.sh_up + r * (H / 2))[lane];
      shsg = L.sh_gate_s[r * (H / G) + (lane >> 2)];
      shsu = L.sh_up_s[r * (H / G) + (lane >> 2)];
    }
    PUB_MARK(12);
    PHASE_MARK(3);
    PHASE_MARK(4);

    // ---------------- P2: routing, routed gate/up
    for (int t0 = 0; t0 < n; t0 += 4) {
      const int nb = min(4, n - t0);
      for (int i = 0; i < nb; ++i) {
        bool ok = true;
        if (poller)
          ok = gather<(4 * E + NPOLL - 1) / NPOLL, ZPos, NPOLL>(A.xz + (size_t)(t0 + i) * 4 * E, 4 * E, tag,
                                                                zbuf[i], A.err, ZPos(), tid, l,
                                                                    (t0 + i == 0) ? 1 : -1, gts_lds);
        if (sync_or(!ok)) { rearm(); return; }
      }
      PHASE_MARK(5);
      if (wave == 0) {   // the selection; the publisher wave adds the weights below
        int sel[TOPK];
        route_select(reinterpret_cast<const double*>(zbuf[0]), sel);
        write_ids(sel, ids_l[0]);
      }
      wg_sync();
    }
    PHASE_MARK(6);
    // distinct experts of the call (for one token: its six picks, in pick order)
    const int D = (n == 1) ? TOPK : distinct_experts(ids_l, n, list, wave_tot);
    const int* dl = (n == 1) ? ids_l[0] : list;
    PHASE_MARK(7);
    // down codes of the first token for output row 8 w + wave: needed after the
    // h exchange.  Requested once this wave's gate/up rows are computed, so
    // that the gate/up rows do not share the memory's bandwidth with them;
    // they arrive during the h exchange (whose first poll waits for them).
    const int row = NWAVES * w + wave;
    uint4 ca0, cb0;
    uint32_t sa0, sb0;
    {
      // Row-pair tasks of this workgroup: 4 shared-expert rows (4 w .. 4 w + 3,
      // weights prefetched) and R = 2 D routed rows (w R .. w R + R - 1 of the
      // distinct experts' rows), dealt round-robin over the waves: local task j
      // goes to wave j % 8; j < 4 are the shared rows.  Results go to LDS; the
      // publisher wave writes them out after a barrier.
      const int R = 2 * D;
      constexpr int TB = 2;            // routed tasks a wave holds in flight
      uint4 qg[TB], qu[TB];
      uint32_t qsg[TB], qsu[TB];
      auto load_batch = [&](int j0) {
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          const int j = j0 + b * NWAVES;
          if (j < 4 + R) {
            const int q = w * R + (j - 4);
            const size_t rr = (size_t)dl[q / I] * I + (q % I);
            qg[b] = reinterpret_cast<const uint4*>(L.gate + rr * (H / 2))[lane];
            qu[b] = reinterpret_cast<const uint4*>(L.up + rr * (H / 2))[lane];
            qsg[b] = L.gate_s[rr * (H / G) + (lane >> 2)];
            qsu[b] = L.up_s[rr * (H / G) + (lane >> 2)];
          }
        }
      };
      // one h value per task j, kept in task order so that the publisher's
      // lanes write consecutive words (whole 32-byte pieces)
      auto emit = [&](int j, int word, float hv) {
        if (lane == 0) {
          hloc[j] = F16H ? __half2float(__float2half_rn(hv)) : hv;
          hloc_idx[j] = word;
        }
      };
      auto compute_batch = [&](int j0) {
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          const int j = j0 + b * NWAVES;
          if (j >= 4 + R) break;
          const int q = w * R + (j - 4);
          const int e = dl[q / I], r = q % I;
          for (int t = 0; t < n; ++t) {
            const int slot = slot_of(ids_l[t], e);
            if (slot < 0) continue;
            emit(j, t * HW + slot * I + r, gateup_row_token(qg[b], qsg[b], qu[b], qsu[b], a_lds[t], asum_lds[t][lane]));
          }
        }
      };
      int j0 = 4 + ((wave - 4 + NWAVES) % NWAVES);   // first routed task of this wave
      load_batch(j0);
      if (wave == PUB_WAVE) {   // routing weights, while this wave's loads fly (needed after the h exchange)
        int sel[TOPK];
#pragma unroll
        for (int r = 0; r < TOPK; ++r) sel[r] = ids_l[0][r];
        const float wv = route_weights(reinterpret_cast<const double*>(zbuf[0]) + E, sel, w_l[0]);
        if (w == 0 && A.trace_ids && lane < TOPK) {
          const size_t o = (size_t)l * A.trace_cap * TOPK + lane;
          A.trace_ids[o] = ids_l[0][lane];
          A.trace_w[o] = wv;
        }
      }
      if (wave < 4) {   // the shared row (its weights requested earlier) while the routed loads fly
        const int r = w * 4 + wave;
        for (int t = 0; t < n; ++t)
          emit(wave, t * HW + TOPK * I + r,
               gateup_row_token(shg, shsg, shu, shsu, a_lds[t], asum_lds[t][lane]));
      }
      compute_batch(j0);
      for (j0 += TB * NWAVES; j0 < 4 + R; j0 += TB * NWAVES) {
        load_batch(j0);
        compute_batch(j0);
      }
      load_down_row(L, ids_l[0], row, ca0, sa0, cb0, sb0);
    }
    wg_sync();
    PUB_MARK(13);
    if (wave == PUB_WAVE) {
      const int cnt = 4 + 2 * D;   // one value per task (one token): 16
      if constexpr (F16H) {
        // one 32-byte run per workgroup: values 2 k and 2 k + 1 in word k
        if (lane < cnt / 2) {
          const int w0 = hloc_idx[2 * lane], w1 = hloc_idx[2 * lane + 1];
          if (w0 >= 0 && w0 < HW && w1 >= 0 && w1 < HW)
            __hip_atomic_store(vh_l + 8 * w + lane, fp16_bits(hloc[2 * lane]) | (fp16_bits(hloc[2 * lane + 1]) << 16),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else
            __hip_atomic_store(A.err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        for (int k = lane; k < cnt; k += 64) {
          const int word = hloc_idx[k];
          // one 64-byte run per workgroup (the h values of its tasks, in task order)
          if (word >= 0 && word < n * HW) publish_value(vh_l + 16 * w + k, hloc[k]);
          else __hip_atomic_store(A.err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    PUB_MARK(14);
    PHASE_MARK(8);

    // ---------------- P3: down row 8 w + wave and combine, per token
    for (int t = 0; t < n; ++t) {
      uint4 ca = ca0, cb = cb0;
      uint32_t sa = sa0, sb = sb0;
      if (t > 0) load_down_row(L, ids_l[t], row, ca, sa, cb, sb);
      bool ok = true;
      if (poller) {
        if constexpr (F16H)
          ok = gather_values<(HW / 8 + NPOLL - 1) / NPOLL, StoreH16, NPOLL>(vh_l, HW / 2, A.err, StoreH16{hbuf}, tid,
                                                                           l, 2, gts_lds);
        else
          ok = gather_values<(HW / 4 + NPOLL - 1) / NPOLL, StoreH, NPOLL>(
              vh_l, HW, A.err, StoreH{reinterpret_cast<uint32_t*>(hbuf)}, tid, l, 2, gts_lds);
      }
      if (sync_or(!ok)) { rearm(); return; }
      if (t == 0) PHASE_MARK(9);
      const int sub = lane & 15;
      auto load_a = [&] { return load_chunk_transposed(hbuf + (lane >> 4) * I, sub, I / 32); };
      auto load_b = [&] {
        return (lane < 32) ? load_chunk_transposed(hbuf + (4 + (lane >> 4)) * I, sub, I / 32)
                           : load_chunk_transposed(hbuf + TOPK * I, lane - 32, IS / 32);
      };
      float wsc[TOPK];   // routed weights, times the pack's divisor in the fp16 form
#pragma unroll
      for (int i = 0; i < TOPK; ++i) wsc[i] = F16H ? w_l[t][i] * A.interm_mult : w_l[t][i];
      const float v = down_row_token(ca, sa, cb, sb, load_a, load_b, wsc, xown[t][wave]);
      if (lane == 0) xnew[t][wave] = v;
      wg_sync();   // hbuf is rewritten by the next token
    }
    if (wave == PUB_WAVE) {
      for (int i = lane; i < 8 * n; i += 64) {
        const int t = i >> 3, r = NWAVES * w + (i & 7);
        const float v = xnew[t][i & 7];
        if (l + 1 < A.l1) publish_value(A.vx + ((size_t)A.parity * A.n_layers + l) * H + r, v);
        else A.out[(size_t)t * H + r] = v;
      }
    }
    PUB_MARK(15);
    PHASE_MARK(10);
  }
  rearm();
#ifdef FLINT_PHASE_TS
  if (threadIdx.x == 0) {
    for (int l = A.l0; l < A.l1 && l < TS_LAYERS; ++l) {
      for (int k = 0; k < 16; ++k) g_phase_ts[l][k][blockIdx.x] = ts_lds[l][k];
      if (blockIdx.x == 0)
        for (int g = 0; g < 4; ++g)
          for (int k = 0; k < 4; ++k) g_gather_ts[l][g][k] = gts_lds[l][g][k];
    }
  }
#endif
}

// ------------------------------------------------------------- token groups
// Persistent decode for up to K = 2, 4, 8 or 16 tokens: the grid splits into
// one group of P = NWG / K workgroups per token (groups past n exit at once).  A group runs the
// single-token schedule above for its token with every workgroup doing K
// times the rows: router rows
// K u .. K u + K - 1, shared gate/up rows 4 K u .., routed gate/up rows
// 12 K u .. of the token's six experts, and output rows 8 K u ...  Its
// exchanges carry one token and involve only its P workgroups, so their size
// does not grow with n.  Every row is computed by the same device function
// with the same reduction shape as in a single-token call, so each token's
// result is bitwise the same as running it alone.  F16H: the fp16-intermediate
// form, each SwiGLU output rounded to fp16 and the routed weights scaled by
// A.interm_mult, as in the one-token kernel (one value per exchange word).
template <int K, bool F16H>
__global__ void __launch_bounds__(NT) k_decode_groups(PersistArgs A) {
  constexpr int P = NWG / K;
  constexpr int NSH = 4 * K, NRT = 12 * K, NTASK = NSH + NRT;   // gate/up row pairs of a workgroup
  constexpr int NOUT = 8 * K;                                     // output rows of a workgroup
  __shared__ __align__(16) uint4 a_lds[256];
  __shared__ float asum_lds[64];
  __shared__ float xown[NOUT];
  __shared__ __align__(16) uint32_t stage[HW];   // gather destination: x, then (c, s), then h
  float* const xstage = reinterpret_cast<float*>(stage);
  float* const hbuf = reinterpret_cast<float*>(stage);
  __shared__ float hloc[NTASK];
  __shared__ int hloc_idx[NTASK];
  __shared__ float xnew[NOUT];
  __shared__ int ids_l[TOPK];
  __shared__ float w_l[TOPK];
  __shared__ double red[2][NWAVES];
  __shared__ double zpart[K][NWAVES];
  __shared__ int bail[2];
  GtsLds gts_lds = nullptr;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t = blockIdx.x / P, u = blockIdx.x % P;   // token of this group, workgroup in the group
  if (t >= A.n) return;                               // no group waits for this workgroup
  const bool poller = wave != PUB_WAVE;

  if (tid < 2) bail[tid] = 0;
  int bail_par = 0;
  auto sync_or = [&](bool fail) {
    if (fail) bail[bail_par] = 1;
    wg_sync();
    const bool r = bail[bail_par] != 0;
    bail_par ^= 1;
    return r;
  };
  wg_sync();

  for (int l = A.l0; l < A.l1; ++l) {
    // thread indices recomputed from an opaque copy each layer, so that the
    // compiler does not hoist addresses derived from them out of the layer
    // loop (held across it, they would not fit in registers and be spilled)
    int tid_l = threadIdx.x;
    asm volatile("" : "+v"(tid_l));
    const int tid = tid_l, wave = tid_l >> 6, lane = tid_l & 63;
    const LayerW L = layer_at(A.base, A.layer_stride, l);
    const uint32_t tag = A.epoch + ((uint32_t)l << 2);
    // router rows of this workgroup: requested before the x exchange
    uint2 rw[K];
#pragma unroll
    for (int j = 0; j < K; ++j) rw[j] = load_router_part(L.router + (size_t)(K * u + j) * H);

    // ---------------- P0: block input
    bool ok = true;
    if (l == A.l0) {
      if (tid < H / 4) reinterpret_cast<float4*>(xstage)[tid] = reinterpret_cast<const float4*>(A.x + (size_t)t * H)[tid];
    } else if (poller) {
      ok = gather<(H + NPOLL - 1) / NPOLL, Identity, NPOLL>(A.xx + (size_t)t * H, H, tag - 4 + 2,
                                                          reinterpret_cast<uint32_t*>(xstage), A.err, Identity(), tid,
                                                          l, -1, gts_lds);
    }
    if (sync_or(!ok)) return;
    const float4 xv = reinterpret_cast<const float4*>(xstage)[tid];
    if (tid >= (NOUT / 4) * u && tid < (NOUT / 4) * (u + 1)) {   // this workgroup's output rows, kept for the residual
      float* xo = xown + 4 * (tid - (NOUT / 4) * u);
      xo[0] = xv.x; xo[1] = xv.y; xo[2] = xv.z; xo[3] = xv.w;
    }
    block_input(xv, reinterpret_cast<uint32_t*>(a_lds), asum_lds, red[l & 1]);
    wg_sync();

    // ---------------- P1: router rows -> the publisher wave writes (c, s)
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const double p = router_part(rw[j], a_lds);
      if (lane == 0) zpart[j][wave] = p;
    }
    wg_sync();
    if (wave == PUB_WAVE) {   // lane L writes word L % 4 of expert K u + L / 4: one store of 4 K words
      unsigned long long cb = 0, sb = 0;
      if (lane < K) {
        double sv, cv;
        router_scores(zpart[lane], L.bias[K * u + lane], sv, cv);
        cb = (unsigned long long)__double_as_longlong(cv);
        sb = (unsigned long long)__double_as_longlong(sv);
      }
      const int src = lane >> 2, pw = lane & 3;
      const uint32_t c_lo = __shfl((uint32_t)cb, src), c_hi = __shfl((uint32_t)(cb >> 32), src);
      const uint32_t s_lo = __shfl((uint32_t)sb, src), s_hi = __shfl((uint32_t)(sb >> 32), src);
      if (lane < 4 * K)
        publish(A.xz + (size_t)t * 4 * E + 4 * K * u + lane, tag, pw == 0 ? c_lo : pw == 1 ? c_hi : pw == 2 ? s_lo : s_hi);
    }

    // gate/up row pairs come in batches of TB tasks (below).  With K >= 4 the
    // first batch holds shared rows only, which do not depend on the routing:
    // it is requested before the (c, s) exchange, whose wait hides it.
    constexpr int TB = 2;
    struct Batch {
      uint4 qg[TB], qu[TB];
      uint32_t qsg[TB], qsu[TB];
    };
    constexpr bool EARLY = NSH >= TB * NWAVES;
    Batch ba;
    if constexpr (EARLY) {
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        const size_t rr = (size_t)NSH * u + wave + b * NWAVES;
        ba.qg[b] = reinterpret_cast<const uint4*>(L.sh_gate + rr * (H / 2))[lane];
        ba.qu[b] = reinterpret_cast<const uint4*>(L.sh_up + rr * (H / 2))[lane];
        ba.qsg[b] = L.sh_gate_s[rr * (H / G) + (lane >> 2)];
        ba.qsu[b] = L.sh_up_s[rr * (H / G) + (lane >> 2)];
      }
    }

    // ---------------- P2: routing, gate/up
    ok = true;
    if (poller)
      ok = gather<(4 * E + NPOLL - 1) / NPOLL, ZPos, NPOLL>(A.xz + (size_t)t * 4 * E, 4 * E, tag, stage, A.err,
                                                            ZPos(), tid, l, -1, gts_lds);
    if (sync_or(!ok)) return;
    if (wave == 0) {
      const double* zc = reinterpret_cast<const double*>(stage);
      route_token(zc, zc + E, ids_l, w_l);
    }
    wg_sync();
    if (u == 0 && A.trace_ids && wave == PUB_WAVE && lane < TOPK) {
      const size_t o = ((size_t)l * A.trace_cap + t) * TOPK + lane;
      A.trace_ids[o] = ids_l[lane];
      A.trace_w[o] = w_l[lane];
    }
    // down codes of this wave's first output row: needed after the h exchange,
    // requested after the gate/up rows (they then do not share the memory's
    // bandwidth with them)
    const int row0 = NOUT * u + wave;
    uint4 ca0, cb0;
    uint32_t sa0, sb0;
    {
      // task j: j < NSH shared row NSH u + j, else routed row q = NRT u + j - NSH
      // of the token's experts in pick order (slot q / I, row q % I); task j
      // goes to wave j % 8.  Batches of TB tasks in two register sets: the
      // next batch's rows are requested before the current one is computed.
      // Loads are unconditional (tasks past the last re-read it), so each
      // wait counts exactly the loads issued after the ones it needs.
      auto task_row = [&](int j, const uint8_t*& g, const uint16_t*& gs, const uint8_t*& up, const uint16_t*& us,
                          size_t& rr) {
        if (j < NSH) {
          rr = (size_t)NSH * u + j;
          g = L.sh_gate; gs = L.sh_gate_s; up = L.sh_up; us = L.sh_up_s;
        } else {
          const int q = NRT * u + (j - NSH);
          rr = (size_t)ids_l[q / I] * I + (q % I);
          g = L.gate; gs = L.gate_s; up = L.up; us = L.up_s;
        }
      };
      auto load_batch = [&](int j0, Batch& bt) {
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          const int j = min(j0 + b * NWAVES, NTASK - 1);
          const uint8_t *g, *up;
          const uint16_t *gs, *us;
          size_t rr;
          task_row(j, g, gs, up, us, rr);
          bt.qg[b] = reinterpret_cast<const uint4*>(g + rr * (H / 2))[lane];
          bt.qu[b] = reinterpret_cast<const uint4*>(up + rr * (H / 2))[lane];
          bt.qsg[b] = gs[rr * (H / G) + (lane >> 2)];
          bt.qsu[b] = us[rr * (H / G) + (lane >> 2)];
        }
      };
      auto compute_batch = [&](int j0, const Batch& bt) {
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          const int j = j0 + b * NWAVES;
          if (j >= NTASK) break;
          const int word = j < NSH ? TOPK * I + NSH * u + j : NRT * u + (j - NSH);   // slot * I + row
          const float hv = gateup_row_token(bt.qg[b], bt.qsg[b], bt.qu[b], bt.qsu[b], a_lds, asum_lds[lane]);
          if (lane == 0) {   // in task order: the publisher's lanes write consecutive words
            hloc[j] = F16H ? __half2float(__float2half_rn(hv)) : hv;
            hloc_idx[j] = word;
          }
        }
      };
      // NTASK / 8 = 2 K tasks per wave: an even number of batches of 2
      static_assert((NTASK / NWAVES) % (2 * TB) == 0, "batches come in pairs");
      Batch bb;
      if constexpr (!EARLY) load_batch(wave, ba);
      constexpr int NPAIR = NTASK / NWAVES / (2 * TB);
#pragma unroll
      for (int k = 0; k < NPAIR; ++k) {
        const int j0 = wave + k * 2 * TB * NWAVES;
        load_batch(j0 + TB * NWAVES, bb);
        compute_batch(j0, ba);
        if (k + 1 < NPAIR) load_batch(j0 + 2 * TB * NWAVES, ba);   // known at compile time
        compute_batch(j0 + TB * NWAVES, bb);
      }
      load_down_row(L, ids_l, row0, ca0, sa0, cb0, sb0);
    }
    wg_sync();
    if (wave == PUB_WAVE) {
      for (int k = lane; k < NTASK; k += 64) {   // one value per task
        const int word = hloc_idx[k];
        if (word >= 0 && word < HW) publish(A.xh + (size_t)t * HW + word, tag + 1, __float_as_uint(hloc[k]));
        else __hip_atomic_store(A.err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }

    // ---------------- P3: output rows NOUT u + wave + 8 i (i < K), fixed-order combine
    ok = true;
    if (poller)
      ok = gather<(HW + NPOLL - 1) / NPOLL, HPos, NPOLL>(A.xh + (size_t)t * HW, HW, tag + 1,
                                                        reinterpret_cast<uint32_t*>(hbuf), A.err, HPos(), tid, l, -1,
                                                        gts_lds);
    if (sync_or(!ok)) return;
    {
      const int sub = lane & 15;
      // this token's h chunks are the same for every output row of the wave:
      // read and summed once, before the rows
      const HChunk hca = load_chunk_transposed(hbuf + (lane >> 4) * I, sub, I / 32);
      const HChunk hcb = (lane < 32) ? load_chunk_transposed(hbuf + (4 + (lane >> 4)) * I, sub, I / 32)
                                     : load_chunk_transposed(hbuf + TOPK * I, lane - 32, IS / 32);
      auto load_a = [&] { return hca; };
      auto load_b = [&] { return hcb; };
      float wsc[TOPK];   // fp16 form: routed weights times the pack's divisor
#pragma unroll
      for (int i = 0; i < TOPK; ++i) wsc[i] = F16H ? w_l[i] * A.interm_mult : 0.f;
      uint4 ca = ca0, cb = cb0;
      uint32_t sa = sa0, sb = sb0;
      for (int i = 0; i < K; ++i) {
        const int lr = wave + NWAVES * i;   // local output row
        uint4 nca = ca, ncb = cb;
        uint32_t nsa = sa, nsb = sb;
        if (i + 1 < K) load_down_row(L, ids_l, NOUT * u + lr + NWAVES, nca, nsa, ncb, nsb);
        float v;
        if constexpr (F16H) v = down_row_token(ca, sa, cb, sb, load_a, load_b, wsc, xown[lr]);
        else v = down_row_token(ca, sa, cb, sb, load_a, load_b, w_l, xown[lr]);
        if (lane == 0) xnew[lr] = v;
        ca = nca; cb = ncb; sa = nsa; sb = nsb;
      }
    }
    wg_sync();
    if (wave == PUB_WAVE) {
      for (int i = lane; i < NOUT; i += 64) {
        const int r = NOUT * u + i;
        const float v = xnew[i];
        if (l + 1 < A.l1) publish(A.xx + (size_t)t * H + r, tag + 2, __float_as_uint(v));
        else A.out[(size_t)t * H + r] = v;
      }
    }
  }
}

// ------------------------------------------------------------- token groups, any n
// Persistent decode for token counts well below a power of two: the grid
// splits into one group of P = NWG / n workgroups per token (rounded down;
// the workgroups past n P exit at once).  A group runs the single-token
// schedule above for its token, with workgroup u of the group taking the u-th
// of P near-equal ranges of each kind of row: router rows (experts), shared
// gate/up rows, the token's routed gate/up rows and output rows.  A range
// holds at most K times the rows of a single-token workgroup, for K the power
// of two at or above n (then NWG / P <= K).
// Its exchanges carry one token and involve only its P workgroups, so their
// size does not grow with n.  Every row is computed by the same device
// function with the same reduction shape as in a single-token call, so each
// token's result is bitwise the same as running it alone.  F16H as above.
// NPAIR: pairs of gate/up batches every workgroup runs (enough for the
// workgroup of the call with the most tasks; chosen on the host from n).
template <int K, bool F16H, int NPAIR>
__global__ void __launch_bounds__(NT) k_decode_groups_any(PersistArgs A) {
  constexpr int MSH = 4 * K, MRT = 12 * K, MTASK = MSH + MRT;   // most gate/up row pairs of a workgroup
  constexpr int MOUT = 8 * K;                                   // most output rows of a workgroup
  __shared__ __align__(16) uint4 a_lds[256];
  __shared__ float asum_lds[64];
  __shared__ float xown[MOUT];
  __shared__ __align__(16) uint32_t stage[HW];   // gather destination: x, then (c, s), then h
  float* const xstage = reinterpret_cast<float*>(stage);
  float* const hbuf = reinterpret_cast<float*>(stage);
  __shared__ float hloc[MTASK];
  __shared__ int hloc_idx[MTASK];
  __shared__ float xnew[MOUT];
  __shared__ int ids_l[TOPK];
  __shared__ float w_l[TOPK];
  __shared__ double red[2][NWAVES];
  __shared__ double zpart[K][NWAVES];
  __shared__ int bail[2];
  GtsLds gts_lds = nullptr;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int P = NWG / A.n;
  const int t = blockIdx.x / P, u = blockIdx.x % P;   // token of this group, workgroup in the group
  if (t >= A.n) return;                               // no group waits for this workgroup
  const bool poller = wave != PUB_WAVE;
  // this workgroup's ranges: [T u / P, T (u + 1) / P) of T rows
  auto lo = [&](int T) { return T * u / P; };
  auto hi = [&](int T) { return T * (u + 1) / P; };
  const int r0 = lo(E), nr = hi(E) - r0;                       // router rows (experts)
  const int s0 = lo(IS), nsh = hi(IS) - s0;                    // shared gate/up rows
  const int q0 = lo(TOPK * I), nrt = hi(TOPK * I) - q0;        // routed gate/up rows of the token
  const int o0 = lo(H), nout = hi(H) - o0;                     // output rows
  const int ntask = nsh + nrt;

  if (tid < 2) bail[tid] = 0;
  int bail_par = 0;
  auto sync_or = [&](bool fail) {
    if (fail) bail[bail_par] = 1;
    wg_sync();
    const bool r = bail[bail_par] != 0;
    bail_par ^= 1;
    return r;
  };
  wg_sync();

  for (int l = A.l0; l < A.l1; ++l) {
    // thread indices recomputed from an opaque copy each layer, so that the
    // compiler does not hoist addresses derived from them out of the layer
    // loop (held across it, they would not fit in registers and be spilled)
    int tid_l = threadIdx.x;
    asm volatile("" : "+v"(tid_l));
    const int tid = tid_l, wave = tid_l >> 6, lane = tid_l & 63;
    const LayerW L = layer_at(A.base, A.layer_stride, l);
    const uint32_t tag = A.epoch + ((uint32_t)l << 2);
    // router rows of this workgroup: requested before the x exchange
    uint2 rw[K];
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (j < nr) rw[j] = load_router_part(L.router + (size_t)(r0 + j) * H);

    // ---------------- P0: block input
    bool ok = true;
    if (l == A.l0) {
      if (tid < H / 4) reinterpret_cast<float4*>(xstage)[tid] = reinterpret_cast<const float4*>(A.x + (size_t)t * H)[tid];
    } else if (poller) {
      ok = gather<(H + NPOLL - 1) / NPOLL, Identity, NPOLL>(A.xx + (size_t)t * H, H, tag - 4 + 2,
                                                          reinterpret_cast<uint32_t*>(xstage), A.err, Identity(), tid,
                                                          l, -1, gts_lds);
    }
    if (sync_or(!ok)) return;
    for (int i = tid; i < nout; i += NT) xown[i] = xstage[o0 + i];   // this workgroup's rows, for the residual
    const float4 xv = reinterpret_cast<const float4*>(xstage)[tid];
    block_input(xv, reinterpret_cast<uint32_t*>(a_lds), asum_lds, red[l & 1]);
    wg_sync();

    // ---------------- P1: router rows -> the publisher wave writes (c, s)
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if (j < nr) {
        const double p = router_part(rw[j], a_lds);
        if (lane == 0) zpart[j][wave] = p;
      }
    }
    wg_sync();
    if (wave == PUB_WAVE) {   // lane L writes word L % 4 of expert r0 + L / 4: one store of 4 nr words
      unsigned long long cb = 0, sb = 0;
      if (lane < nr) {
        double sv, cv;
        router_scores(zpart[lane], L.bias[r0 + lane], sv, cv);
        cb = (unsigned long long)__double_as_longlong(cv);
        sb = (unsigned long long)__double_as_longlong(sv);
      }
      const int src = lane >> 2, pw = lane & 3;
      const uint32_t c_lo = __shfl((uint32_t)cb, src), c_hi = __shfl((uint32_t)(cb >> 32), src);
      const uint32_t s_lo = __shfl((uint32_t)sb, src), s_hi = __shfl((uint32_t)(sb >> 32), src);
      if (lane < 4 * nr)
        publish(A.xz + (size_t)t * 4 * E + 4 * r0 + lane, tag, pw == 0 ? c_lo : pw == 1 ? c_hi : pw == 2 ? s_lo : s_hi);
    }

    // ---------------- P2: routing, gate/up
    // gate/up row pairs come in batches of TB tasks (below).  The first batch
    // (tasks wave and wave + 8) holds shared rows only, which do not depend on
    // the routing (every workgroup of these calls has nsh >= 20 shared row
    // pairs: at most 51 workgroups per token): it is requested before the
    // (c, s) exchange, whose wait hides it.
    constexpr int TB = 2;
    struct Batch {
      uint4 qg[TB], qu[TB];
      uint32_t qsg[TB], qsu[TB];
    };
    Batch ba;
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const size_t rr = (size_t)(s0 + min(wave + b * NWAVES, nsh - 1));
      ba.qg[b] = reinterpret_cast<const uint4*>(L.sh_gate + rr * (H / 2))[lane];
      ba.qu[b] = reinterpret_cast<const uint4*>(L.sh_up + rr * (H / 2))[lane];
      ba.qsg[b] = L.sh_gate_s[rr * (H / G) + (lane >> 2)];
      ba.qsu[b] = L.sh_up_s[rr * (H / G) + (lane >> 2)];
    }
    ok = true;
    if (poller)
      ok = gather<(4 * E + NPOLL - 1) / NPOLL, ZPos, NPOLL>(A.xz + (size_t)t * 4 * E, 4 * E, tag, stage, A.err,
                                                            ZPos(), tid, l, -1, gts_lds);
    if (sync_or(!ok)) return;
    if (wave == 0) {
      const double* zc = reinterpret_cast<const double*>(stage);
      route_token(zc, zc + E, ids_l, w_l);
    }
    wg_sync();
    if (u == 0 && A.trace_ids && wave == PUB_WAVE && lane < TOPK) {
      const size_t o = ((size_t)l * A.trace_cap + t) * TOPK + lane;
      A.trace_ids[o] = ids_l[lane];
      A.trace_w[o] = w_l[lane];
    }
    // down codes of this wave's first output row: needed after the h exchange
    uint4 ca0 = make_uint4(0u, 0u, 0u, 0u), cb0 = ca0;
    uint32_t sa0 = 0u, sb0 = 0u;
    if (wave < nout) load_down_row(L, ids_l, o0 + wave, ca0, sa0, cb0, sb0);
    {
      // task j: j < nsh shared row s0 + j, else routed row q = q0 + j - nsh of
      // the token's experts in pick order (slot q / I, row q % I); task j goes
      // to wave j % 8.  Batches of TB tasks in two register sets: the next
      // batch's rows are requested before the current one is computed.  The
      // loop runs the most batches any workgroup of the call has (a count
      // fixed at compile time), its loads unconditional (tasks past the last
      // re-read it), so each wait counts exactly the loads issued after the
      // ones it needs.
      auto load_batch = [&](int j0, Batch& bt) {
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          const int j = min(j0 + b * NWAVES, ntask - 1);
          const bool sh = j < nsh;
          const int q = q0 + (j - nsh);
          const size_t rr = sh ? (size_t)(s0 + j) : (size_t)ids_l[q / I] * I + (q % I);
          bt.qg[b] = reinterpret_cast<const uint4*>((sh ? L.sh_gate : L.gate) + rr * (H / 2))[lane];
          bt.qu[b] = reinterpret_cast<const uint4*>((sh ? L.sh_up : L.up) + rr * (H / 2))[lane];
          bt.qsg[b] = (sh ? L.sh_gate_s : L.gate_s)[rr * (H / G) + (lane >> 2)];
          bt.qsu[b] = (sh ? L.sh_up_s : L.up_s)[rr * (H / G) + (lane >> 2)];
        }
      };
      auto compute_batch = [&](int j0, const Batch& bt) {
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          const int j = j0 + b * NWAVES;
          if (j < ntask) {   // wave-uniform
            const int word = j < nsh ? TOPK * I + s0 + j : q0 + (j - nsh);   // slot * I + row
            const float hv = gateup_row_token(bt.qg[b], bt.qsg[b], bt.qu[b], bt.qsu[b], a_lds, asum_lds[lane]);
            if (lane == 0) {   // in task order: the publisher's lanes write consecutive words
              hloc[j] = F16H ? __half2float(__float2half_rn(hv)) : hv;
              hloc_idx[j] = word;
            }
          }
        }
      };
      static_assert((MTASK / NWAVES) % (2 * TB) == 0, "batches come in pairs");
      static_assert(NPAIR >= 1 && NPAIR <= MTASK / NWAVES / (2 * TB), "batch pairs");
      Batch bb;
#pragma unroll
      for (int k = 0; k < NPAIR; ++k) {
        const int j0 = wave + k * 2 * TB * NWAVES;
        load_batch(j0 + TB * NWAVES, bb);
        compute_batch(j0, ba);
        if (k + 1 < NPAIR) load_batch(j0 + 2 * TB * NWAVES, ba);   // known at compile time
        compute_batch(j0 + TB * NWAVES, bb);
      }
    }
    wg_sync();
    if (wave == PUB_WAVE) {
      for (int k = lane; k < ntask; k += 64) {   // one value per task
        const int word = hloc_idx[k];
        if (word >= 0 && word < HW) publish(A.xh + (size_t)t * HW + word, tag + 1, __float_as_uint(hloc[k]));
        else __hip_atomic_store(A.err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }

    // ---------------- P3: output rows o0 + wave + 8 i, fixed-order combine
    ok = true;
    if (poller)
      ok = gather<(HW + NPOLL - 1) / NPOLL, HPos, NPOLL>(A.xh + (size_t)t * HW, HW, tag + 1,
                                                        reinterpret_cast<uint32_t*>(hbuf), A.err, HPos(), tid, l, -1,
                                                        gts_lds);
    if (sync_or(!ok)) return;
    {
      const int sub = lane & 15;
      // this token's h chunks are the same for every output row of the wave:
      // read and summed once, before the rows
      const HChunk hca = load_chunk_transposed(hbuf + (lane >> 4) * I, sub, I / 32);
      const HChunk hcb = (lane < 32) ? load_chunk_transposed(hbuf + (4 + (lane >> 4)) * I, sub, I / 32)
                                     : load_chunk_transposed(hbuf + TOPK * I, lane - 32, IS / 32);
      auto load_a = [&] { return hca; };
      auto load_b = [&] { return hcb; };
      // unrolled with a fixed bound: the prefetched codes are renamed, never
      // copied (a copy would wait for the load in flight)
      float wsc[TOPK];   // fp16 form: routed weights times the pack's divisor
#pragma unroll
      for (int i = 0; i < TOPK; ++i) wsc[i] = F16H ? w_l[i] * A.interm_mult : 0.f;
      uint4 ca = ca0, cb = cb0;
      uint32_t sa = sa0, sb = sb0;
#pragma unroll
      for (int i = 0; i < K; ++i) {   // nout <= 8 K
        const int lr = wave + NWAVES * i;   // local output row
        if (lr < nout) {   // wave-uniform; no break, so the loop unrolls
          uint4 nca = ca, ncb = cb;
          uint32_t nsa = sa, nsb = sb;
          if (lr + NWAVES < nout) load_down_row(L, ids_l, o0 + lr + NWAVES, nca, nsa, ncb, nsb);
          float v;
          if constexpr (F16H) v = down_row_token(ca, sa, cb, sb, load_a, load_b, wsc, xown[lr]);
          else v = down_row_token(ca, sa, cb, sb, load_a, load_b, w_l, xown[lr]);
          if (lane == 0) xnew[lr] = v;
          ca = nca; cb = ncb; sa = nsa; sb = nsb;
        }
      }
    }
    wg_sync();
    if (wave == PUB_WAVE) {
      for (int i = lane; i < nout; i += 64) {
        const int r = o0 + i;
        const float v = xnew[i];
        if (l + 1 < A.l1) publish(A.xx + (size_t)t * H + r, tag + 2, __float_as_uint(v));
        else A.out[(size_t)t * H + r] = v;
      }
    }
  }
}

__global__ void k_clear_words(uint64_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

// Pairs of gate/up batches the exact-range kernel needs for n tokens: the
// most shared + routed row pairs of any workgroup (the same ranges as the
// kernel's), 2 TB NWAVES = 32 tasks per pair.
static int exact_batch_pairs(int n) {
  const int P = NWG / n;
  int most = 0;
  for (int u = 0; u < P; ++u) {
    auto cnt = [&](int T) { return T * (u + 1) / P - T * u / P; };
    most = std::max(most, cnt(IS) + cnt(TOPK * I));
  }
  return (most + 31) / 32;
}

// The kernel for K-token groups (K = 1: the one-token schedule); F16H: the
// fp16-intermediate form.  The exact-range kernels come with the batch-pair
// counts that 5..15 tokens need, rounded up to one that is built.
template <bool F16H>
static const void* decode_kernel(int K, bool exact, int n) {
  if (K == 2) return reinterpret_cast<const void*>(k_decode_groups<2, F16H>);
  if (K == 4) return reinterpret_cast<const void*>(k_decode_groups<4, F16H>);   // 3, 4 tokens: never exact
  if (K == 8) {
    if (!exact) return reinterpret_cast<const void*>(k_decode_groups<8, F16H>);
    return exact_batch_pairs(n) <= 3 ? reinterpret_cast<const void*>(k_decode_groups_any<8, F16H, 3>)
                                     : reinterpret_cast<const void*>(k_decode_groups_any<8, F16H, 4>);
  }
  if (K == 16) {
    if (!exact) return reinterpret_cast<const void*>(k_decode_groups<16, F16H>);
    const int np = exact_batch_pairs(n);
    return np <= 5   ? reinterpret_cast<const void*>(k_decode_groups_any<16, F16H, 5>)
           : np <= 6 ? reinterpret_cast<const void*>(k_decode_groups_any<16, F16H, 6>)
           : np <= 7 ? reinterpret_cast<const void*>(k_decode_groups_any<16, F16H, 7>)
                     : reinterpret_cast<const void*>(k_decode_groups_any<16, F16H, 8>);
  }
  return reinterpret_cast<const void*>(k_decode_persistent<F16H>);
}

// Launch of a persistent kernel: NWG workgroups that must all be resident at
// once (one per CU: their LDS allows no second one).  They are launched as
// ordinary kernels.  A cooperative launch would guarantee co-residency, but
// on this runtime it costs about 20 us per call, against a 590 us kernel.
// What the guarantee prevents is handled here instead:
// - Two persistent launches from different streams could each hold part of
//   the CUs and wait for workgroups that cannot be placed.  So a launch on a
//   stream other than the previous launch's (of any handle on this device)
//   first waits for that launch: an event is recorded behind every launch.
// - Other work on the GPU can only delay the placement of some workgroups.
//   Every wait in the kernels is bounded (1 s), so a launch that cannot get
//   its CUs ends with the device error word set instead of hanging.
// The handle requires a GPU with exactly NWG CUs, and each kernel's LDS and
// register use (checked at compile time) let one workgroup fit a CU.
static hipError_t launch_resident(const void* k, void** kargs, hipStream_t s) {
  constexpr int MAX_DEV = 64;
  static std::mutex mu;
  static hipEvent_t done[MAX_DEV] = {};
  static hipStream_t last[MAX_DEV] = {};
  static bool used[MAX_DEV] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!done[dev]) {
    e = hipEventCreateWithFlags(&done[dev], hipEventDisableTiming);
    if (e != hipSuccess) { done[dev] = nullptr; return e; }
  }
  if (used[dev] && last[dev] != s) {
    e = hipStreamWaitEvent(s, done[dev], 0);
    if (e != hipSuccess) return e;
  }
  e = hipLaunchKernel(k, dim3(NWG), dim3(NT), kargs, 0, s);
  if (e != hipSuccess) return e;
  e = hipEventRecord(done[dev], s);
  if (e != hipSuccess) return e;
  last[dev] = s;
  used[dev] = true;
  return hipSuccess;
}

hipError_t launch_decode_persistent(const PersistArgs& args, hipStream_t s) {
  PersistArgs a = args;
  void* kargs[] = {&a};
  // One token: the schedule above.  Otherwise groups for K tokens, K the
  // power of two at or above n: the statically sized kernel leaves K - n
  // groups idle, the exact-range kernel uses every workgroup; measured, the
  // exact ranges win up to n = 13 K / 16 (5, 6 and 9..13 tokens).
  const int n = a.n;
  const int K = n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : n <= 8 ? 8 : 16;
  // FLINT_MOE_GROUPS=exact or =pow2 forces one form for every n that is not a
  // power of two (for measuring the rule below)
  static const int force = [] {
    const char* v = getenv("FLINT_MOE_GROUPS");
    return !v ? 0 : strcmp(v, "exact") == 0 ? 1 : strcmp(v, "pow2") == 0 ? 2 : 0;
  }();
  // (exact ranges need n >= 5: their first gate/up batch is shared rows only)
  const bool exact = n >= 5 && (force == 1 ? n != K : force == 2 ? false : 16 * n <= 13 * K);
  const void* k = a.interm_mult != 0.f ? decode_kernel<true>(K, exact, n) : decode_kernel<false>(K, exact, n);
  return launch_resident(k, kargs, s);
}

hipError_t clear_exchange(uint64_t* p, size_t n_words, hipStream_t s) {
  hipLaunchKernelGGL(k_clear_words, dim3(256), dim3(256), 0, s, p, n_words);
  return hipGetLastError();
}

}  // namespace flint
