// Decode path, persistent form: one cooperative launch runs every layer of a
// forward call on 256 workgroups (one per CU), with no kernel boundaries
// between the dependent stages of a layer.
//
// Work of workgroup w (4 wavefronts) in layer l, for each token:
//   P0  block input a = bf16(rmsnorm(x_l)) (every workgroup, redundantly)
//   P1  router row w -> z[w]; shared-expert gate/up row 4 w + wave -> h_sh
//   P2  all 256 z -> sigmoid + bias + top-6 (every workgroup, redundantly);
//       gate/up rows of the distinct picked experts, spread over all waves -> h
//   P3  all h -> output rows 8 w .. 8 w + 7 (six routed down rows + shared
//       down row, fixed-order combine) -> x_{l+1}
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
#include "decode_common.h"
#include "decode_persistent.h"

namespace flint {

constexpr int HW = TOPK * I + IS;                  // h words per token (routed, then shared)

// Phase timestamps for profiling builds only (-DFLINT_PHASE_TS): thread 0 of
// each workgroup records the 100 MHz wall clock at marker k of layer l.
#ifdef FLINT_PHASE_TS
__device__ unsigned long long g_phase_ts[64][16][NWG];
#define PHASE_MARK(k) \
  do { if (threadIdx.x == 0) g_phase_ts[l][k][blockIdx.x] = wall_clock64(); } while (0)
extern "C" int flint_moe_debug_phase_ts(unsigned long long* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase_ts), sizeof(g_phase_ts));
}
#else
#define PHASE_MARK(k) do { } while (0)
#endif
constexpr long long SPIN_TICKS = 100000000LL;      // 1 s of the 100 MHz wall clock

__device__ __forceinline__ void publish(uint64_t* p, uint32_t tag, uint32_t v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t load_word(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until words src[0..nwords) carry `tag`; store the payload of word j
// in dst[pos(j)].  Thread i handles words i + 256 k, k < K.  Returns false on
// timeout (the device error word is then set).
template <int K, typename Pos>
__device__ __forceinline__ bool gather(const uint64_t* src, int nwords, uint32_t tag, uint32_t* dst, int* err,
                                       Pos pos) {
  const int tid = threadIdx.x;
  uint64_t v[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int j = tid + 256 * k;
    v[k] = (j < nwords) ? load_word(src + j) : ((uint64_t)tag << 32);
  }
  const long long t0 = wall_clock64();
  while (true) {
    bool all = true;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if ((uint32_t)(v[k] >> 32) != tag) {
        all = false;
        v[k] = load_word(src + tid + 256 * k);
      }
    }
    if (all) break;
    if (wall_clock64() - t0 > SPIN_TICKS) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int j = tid + 256 * k;
    if (j < nwords) dst[pos(j)] = (uint32_t)v[k];
  }
  return true;
}

struct Identity {
  __device__ int operator()(int j) const { return j; }
};

// h word j of a token (routed slots [TOPK][I], then shared [IS]) -> transposed position
struct HPos {
  __device__ int operator()(int j) const {
    return j < TOPK * I ? (j & ~(I - 1)) + transposed_pos(j & (I - 1), I / 32)
                        : TOPK * I + transposed_pos(j - TOPK * I, IS / 32);
  }
};

__global__ void __launch_bounds__(256) k_decode_persistent(PersistArgs A) {
  __shared__ __align__(16) uint4 a_lds[DECODE_MAX_TOKENS][256];
  __shared__ float asum_lds[DECODE_MAX_TOKENS][64];
  __shared__ __align__(16) float xstage[H];
  __shared__ float xown[DECODE_MAX_TOKENS][8];
  __shared__ __align__(16) uint32_t zbuf[4][4 * E];   // per token: c[E] then s[E], fp64
  __shared__ __align__(16) float hbuf[HW];
  __shared__ int ids_l[DECODE_MAX_TOKENS][TOPK];
  __shared__ float w_l[DECODE_MAX_TOKENS][TOPK];
  __shared__ int mark[E];
  __shared__ int list[DECODE_MAX_TOKENS * TOPK];
  __shared__ int wave_tot[4];
  __shared__ signed char slotmap[DECODE_MAX_TOKENS * TOPK][DECODE_MAX_TOKENS];
  __shared__ double red[4];
  __shared__ double zpart[DECODE_MAX_TOKENS][4];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int w = blockIdx.x;
  const int n = A.n;

  // P1 weights of the current layer, loaded one layer ahead
  uint4 wr, cg, cu;
  float sg, su, bw;
  auto load_p1 = [&](const LayerW& L) {
    wr = reinterpret_cast<const uint4*>(L.router + (size_t)w * H)[4 * lane + wave];
    bw = L.bias[w];
    const int r = w * 4 + wave;
    cg = reinterpret_cast<const uint4*>(L.sh_gate + (size_t)r * (H / 2))[lane];
    cu = reinterpret_cast<const uint4*>(L.sh_up + (size_t)r * (H / 2))[lane];
    sg = bf16_bits_to_f32(L.sh_gate_s[r * (H / G) + (lane >> 2)]);
    su = bf16_bits_to_f32(L.sh_up_s[r * (H / G) + (lane >> 2)]);
  };
  load_p1(layer_at(A.base, A.layer_stride, A.l0));
  compiler_fence();

  for (int l = A.l0; l < A.l1; ++l) {
    const LayerW L = layer_at(A.base, A.layer_stride, l);
    const uint32_t tag = A.epoch + ((uint32_t)l << 2);

    PHASE_MARK(0);
    // ---------------- P0: block input of every token
    for (int t = 0; t < n; ++t) {
      bool ok = true;
      if (l == A.l0) {
        const float4* xs = reinterpret_cast<const float4*>(A.x + (size_t)t * H);
        for (int j = tid; j < H / 4; j += 256) reinterpret_cast<float4*>(xstage)[j] = xs[j];
      } else {
        ok = gather<H / 256>(A.xx + (size_t)t * H, H, tag - 4 + 2, reinterpret_cast<uint32_t*>(xstage), A.err,
                         Identity());
      }
      if (__syncthreads_or(!ok)) return;
      if (tid < 8) xown[t][tid] = xstage[8 * w + tid];
      if (t == 0) PHASE_MARK(1);
      block_input_to_lds(xstage, a_lds[t], asum_lds[t], red);
      __syncthreads();
    }

    PHASE_MARK(2);
    // ---------------- P1: router row w (all four waves), then shared gate/up row 4 w + wave
    for (int t = 0; t < n; ++t) {
      const double p = router_part(wr, a_lds[t]);
      if (lane == 0) zpart[t][wave] = p;
    }
    __syncthreads();
    if (tid < n) {
      double sv, cv;
      router_scores(zpart[tid], bw, sv, cv);
      const unsigned long long cb = (unsigned long long)__double_as_longlong(cv);
      const unsigned long long sb = (unsigned long long)__double_as_longlong(sv);
      uint64_t* z = A.xz + (size_t)tid * 4 * E;
      publish(z + 2 * w, tag, (uint32_t)cb);
      publish(z + 2 * w + 1, tag, (uint32_t)(cb >> 32));
      publish(z + 2 * E + 2 * w, tag, (uint32_t)sb);
      publish(z + 2 * E + 2 * w + 1, tag, (uint32_t)(sb >> 32));
    }
    PHASE_MARK(3);
    {
      const int r = w * 4 + wave;
      for (int t = 0; t < n; ++t) {
        const float hv = gateup_row_token(cg, sg, cu, su, a_lds[t], asum_lds[t][lane]);
        if (lane == 0) publish(A.xh + (size_t)t * HW + TOPK * I + r, tag + 1, __float_as_uint(hv));
      }
    }

    PHASE_MARK(4);
    // ---------------- P2: routing, routed gate/up
    mark[tid] = 0;
    for (int t0 = 0; t0 < n; t0 += 4) {
      const int nb = min(4, n - t0);
      for (int i = 0; i < nb; ++i) {
        const bool ok = gather<4 * E / 256>(A.xz + (size_t)(t0 + i) * 4 * E, 4 * E, tag, zbuf[i], A.err, Identity());
        if (__syncthreads_or(!ok)) return;
        if (t0 + i == 0) PHASE_MARK(5);
      }
      if (wave < nb) {
        const double* zc = reinterpret_cast<const double*>(zbuf[wave]);
        route_token(zc, zc + E, ids_l[t0 + wave], w_l[t0 + wave]);
      }
      __syncthreads();
    }
    PHASE_MARK(6);
    if (w == 0 && A.trace_ids && tid < n * TOPK) {
      const size_t o = (size_t)l * A.trace_cap * TOPK + tid;
      A.trace_ids[o] = ids_l[tid / TOPK][tid % TOPK];
      A.trace_w[o] = w_l[tid / TOPK][tid % TOPK];
    }
    if (tid < n * TOPK) mark[ids_l[tid / TOPK][tid % TOPK]] = 1;
    __syncthreads();
    const int D = distinct_experts(mark, list, wave_tot);
    for (int i = tid; i < D * DECODE_MAX_TOKENS; i += 256)
      slotmap[i / DECODE_MAX_TOKENS][i % DECODE_MAX_TOKENS] = -1;
    __syncthreads();
    if (tid < n * TOPK) slotmap[mark[ids_l[tid / TOPK][tid % TOPK]]][tid / TOPK] = (signed char)(tid % TOPK);
    __syncthreads();
    PHASE_MARK(7);
    {
      // this wave's tasks q = w*4 + wave + k*NWG*4 over (distinct expert, row), loaded TB at a time
      constexpr int TB = 4;
      const int q0 = w * 4 + wave, nq = D * I;
      for (int base = q0; base < nq; base += TB * NWG * 4) {
        uint4 qg[TB], qu[TB];
        float qsg[TB], qsu[TB];
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          const int q = base + b * NWG * 4;
          if (q < nq) {
            const size_t row = (size_t)list[q / I] * I + (q % I);
            qg[b] = reinterpret_cast<const uint4*>(L.gate + row * (H / 2))[lane];
            qu[b] = reinterpret_cast<const uint4*>(L.up + row * (H / 2))[lane];
            qsg[b] = bf16_bits_to_f32(L.gate_s[row * (H / G) + (lane >> 2)]);
            qsu[b] = bf16_bits_to_f32(L.up_s[row * (H / G) + (lane >> 2)]);
          }
        }
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          const int q = base + b * NWG * 4;
          if (q >= nq) break;
          const int d = q / I, r = q % I;
          for (int t = 0; t < n; ++t) {
            const int slot = slotmap[d][t];
            if (slot < 0) continue;
            const float hv = gateup_row_token(qg[b], qsg[b], qu[b], qsu[b], a_lds[t], asum_lds[t][lane]);
            if (lane == 0) publish(A.xh + (size_t)t * HW + slot * I + r, tag + 1, __float_as_uint(hv));
          }
        }
      }
    }
    PHASE_MARK(8);
    if (l + 1 < A.l1) load_p1(layer_at(A.base, A.layer_stride, l + 1));
    compiler_fence();   // issue the next layer's loads now, before the waits below

    // ---------------- P3: down rows 8 w + 2 wave + {0, 1} and combine
    for (int t = 0; t < n; ++t) {
      uint4 ca[2], cb[2];
      float sa[2], sb[2];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) load_down_row(L, ids_l[t], 8 * w + 2 * wave + rr, ca[rr], sa[rr], cb[rr], sb[rr]);
      compiler_fence();   // down codes in flight while waiting for h
      const bool ok = gather<HW / 256>(A.xh + (size_t)t * HW, HW, tag + 1, reinterpret_cast<uint32_t*>(hbuf), A.err, HPos());
      if (__syncthreads_or(!ok)) return;
      const int sub = lane & 15;
      if (t == 0) PHASE_MARK(9);
      const HChunk ha = load_chunk_transposed(hbuf + (lane >> 4) * I, sub, I / 32);
      const HChunk hb = (lane < 32) ? load_chunk_transposed(hbuf + (4 + (lane >> 4)) * I, sub, I / 32)
                                    : load_chunk_transposed(hbuf + TOPK * I, lane - 32, IS / 32);
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int row = 8 * w + 2 * wave + rr;
        const float v = down_row_token(ca[rr], sa[rr], cb[rr], sb[rr], ha, hb, w_l[t], xown[t][row - 8 * w]);
        if (lane == 0) {
          if (l + 1 < A.l1) publish(A.xx + (size_t)t * H + row, tag + 2, __float_as_uint(v));
          else A.out[(size_t)t * H + row] = v;
        }
      }
      __syncthreads();
    }
    PHASE_MARK(10);
  }
}

__global__ void k_clear_words(uint64_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0;
}

hipError_t launch_decode_persistent(const PersistArgs& args, hipStream_t s) {
  PersistArgs a = args;
  void* kargs[] = {&a};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_decode_persistent), dim3(NWG), dim3(256), kargs,
                                    0, s);
}

hipError_t clear_exchange(uint64_t* p, size_t n_words, hipStream_t s) {
  hipLaunchKernelGGL(k_clear_words, dim3(256), dim3(256), 0, s, p, n_words);
  return hipGetLastError();
}

}  // namespace flint
