// Decode path, per-layer form (n_tokens <= DECODE_MAX_TOKENS): three kernels
// per layer, ordered by the stream.  The persistent kernel does the same work
// in one launch; both use the same device math with the same wave and lane
// roles, so their results are bitwise identical.
//
//   k_norm_router : block input a = bf16(rmsnorm(x)) per token (fp64 norm);
//                   router row e = blockIdx over all 8 waves (fp64), s and c;
//                   then waves 0..3: shared-expert gate/up row 4 e + wave.
//   k_route_gateup: top-6 per token (fp64 scores), the distinct experts of
//                   the call, their gate/up rows over all waves -> h.
//   k_down_combine: output rows 8 b + wave: six routed down rows and the
//                   shared one, fixed-order combine into the residual.
#include "decode_common.h"

namespace flint {

__global__ void __launch_bounds__(NT) k_norm_router(const float* __restrict__ x, int n, LayerW L, DecodeWS ws) {
  __shared__ __align__(16) uint4 a_lds[DECODE_MAX_TOKENS][256];
  __shared__ float asum_lds[DECODE_MAX_TOKENS][64];
  __shared__ double red[2][NWAVES];
  __shared__ double zpart[DECODE_MAX_TOKENS][NWAVES];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int t = 0; t < n; ++t) {
    const float4 xv = reinterpret_cast<const float4*>(x + (size_t)t * H)[tid];
    block_input(xv, reinterpret_cast<uint32_t*>(a_lds[t]), asum_lds[t], red[t & 1]);
  }
  wg_sync();
  if (blockIdx.x == 0) {
    for (int t = 0; t < n; ++t) {
      if (tid < 256) reinterpret_cast<uint4*>(ws.a)[t * 256 + tid] = a_lds[t][tid];
      if (tid < 64) ws.asum[t * 64 + tid] = asum_lds[t][tid];
    }
  }
  const int e = blockIdx.x;
  {
    const uint2 wr = load_router_part(L.router + (size_t)e * H);
    for (int t = 0; t < n; ++t) {
      const double p = router_part(wr, a_lds[t]);
      if (lane == 0) zpart[t][wave] = p;
    }
  }
  wg_sync();
  if (tid < n) {
    double s, c;
    router_scores(zpart[tid], L.bias[e], s, c);
    ws.s[tid * E + e] = s;
    ws.c[tid * E + e] = c;
  }
  if (wave < 4) {
    const int r = e * 4 + wave;
    const uint4 cg = reinterpret_cast<const uint4*>(L.sh_gate + (size_t)r * (H / 2))[lane];
    const uint4 cu = reinterpret_cast<const uint4*>(L.sh_up + (size_t)r * (H / 2))[lane];
    const uint32_t sg = L.sh_gate_s[r * (H / G) + (lane >> 2)];
    const uint32_t su = L.sh_up_s[r * (H / G) + (lane >> 2)];
    for (int t = 0; t < n; ++t) {
      const float hv = gateup_row_token(cg, sg, cu, su, a_lds[t], asum_lds[t][lane]);
      if (lane == 0) ws.hsh[t * IS + r] = hv;
    }
  }
}

__global__ void __launch_bounds__(NT) k_route_gateup(int n, LayerW L, DecodeWS ws, int* trace_ids, float* trace_w) {
  __shared__ __align__(16) uint4 a_lds[DECODE_MAX_TOKENS][256];
  __shared__ float asum_lds[DECODE_MAX_TOKENS][64];
  __shared__ int ids_l[DECODE_MAX_TOKENS][TOPK];
  __shared__ float w_l[DECODE_MAX_TOKENS][TOPK];
  __shared__ int list[DECODE_MAX_TOKENS * TOPK];
  __shared__ int wave_tot[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int t = 0; t < n; ++t) {
    if (tid < 256) a_lds[t][tid] = reinterpret_cast<const uint4*>(ws.a)[t * 256 + tid];
    if (tid < 64) asum_lds[t][tid] = ws.asum[t * 64 + tid];
  }
  for (int t = wave; t < n; t += NWAVES) route_token(ws.c + t * E, ws.s + t * E, ids_l[t], w_l[t]);
  wg_sync();
  if (blockIdx.x == 0 && tid < n * TOPK) {
    ws.ids[tid] = ids_l[tid / TOPK][tid % TOPK];
    ws.w[tid] = w_l[tid / TOPK][tid % TOPK];
    if (trace_ids) {
      trace_ids[tid] = ids_l[tid / TOPK][tid % TOPK];
      trace_w[tid] = w_l[tid / TOPK][tid % TOPK];
    }
  }
  const int D = (n == 1) ? TOPK : distinct_experts(ids_l, n, list, wave_tot);
  const int* dl = (n == 1) ? ids_l[0] : list;
  const int nw = gridDim.x * NWAVES;
  for (int q = blockIdx.x * NWAVES + wave; q < D * I; q += nw) {
    const int e = dl[q / I], r = q % I;
    const size_t row = (size_t)e * I + r;
    const uint4 cg = reinterpret_cast<const uint4*>(L.gate + row * (H / 2))[lane];
    const uint4 cu = reinterpret_cast<const uint4*>(L.up + row * (H / 2))[lane];
    const uint32_t sg = L.gate_s[row * (H / G) + (lane >> 2)];
    const uint32_t su = L.up_s[row * (H / G) + (lane >> 2)];
    for (int t = 0; t < n; ++t) {
      const int slot = slot_of(ids_l[t], e);
      if (slot < 0) continue;
      const float hv = gateup_row_token(cg, sg, cu, su, a_lds[t], asum_lds[t][lane]);
      if (lane == 0) ws.h[(t * TOPK + slot) * I + r] = hv;
    }
  }
}

__global__ void __launch_bounds__(NT) k_down_combine(const float* xin, float* out, int n, LayerW L, DecodeWS ws) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, sub = lane & 15;
  const int nrow = blockIdx.x * NWAVES + wave;
  for (int t = 0; t < n; ++t) {
    uint4 ca, cb;
    uint32_t sa, sb;
    load_down_row(L, ws.ids + t * TOPK, nrow, ca, sa, cb, sb);
    const float* h = ws.h + (size_t)t * TOPK * I;
    const float* hs = ws.hsh + (size_t)t * IS;
    auto load_a = [&] { return load_chunk_natural(h + (lane >> 4) * I, sub); };
    auto load_b = [&] {
      return (lane < 32) ? load_chunk_natural(h + (4 + (lane >> 4)) * I, sub) : load_chunk_natural(hs, lane - 32);
    };
    const float v = down_row_token(ca, sa, cb, sb, load_a, load_b, ws.w + t * TOPK, xin[(size_t)t * H + nrow]);
    if (lane == 0) out[(size_t)t * H + nrow] = v;
  }
}

hipError_t launch_decode_layer(const float* xin, float* out, int n, const LayerW& L, const DecodeWS& ws,
                               int* trace_ids, float* trace_w, hipStream_t s) {
  hipLaunchKernelGGL(k_norm_router, dim3(E), dim3(NT), 0, s, xin, n, L, ws);
  hipLaunchKernelGGL(k_route_gateup, dim3(256), dim3(NT), 0, s, n, L, ws, trace_ids, trace_w);
  hipLaunchKernelGGL(k_down_combine, dim3(H / NWAVES), dim3(NT), 0, s, xin, out, n, L, ws);
  return hipGetLastError();
}

}  // namespace flint
