// Decode path (n_tokens <= DECODE_MAX_TOKENS): three kernels per layer.
//
//   k_norm_router : block input a = bf16(rmsnorm(x)) per token (fp64 norm),
//                   router logits z = Wr a (fp64 accumulation), shared-expert
//                   gate/up rows -> h_shared.
//   k_route_gateup: sigmoid + bias + top-6 per token (fp64), the distinct
//                   experts of the call, their gate/up rows -> h.
//   k_down_combine: per output row, the 6 routed down rows and the shared
//                   down row, combined in a fixed order into the residual.
//
// Every (token, expert, row) dot product is done by one wavefront with the
// same lane partition and reduction tree whatever the number of tokens, so a
// token's result is bitwise independent of the batch it came in.
#include "decode_common.h"

namespace flint {

// ----------------------------------------------------------------- kernel 1
__global__ void __launch_bounds__(256) k_norm_router(const float* __restrict__ x, int n, LayerW L, DecodeWS ws) {
  __shared__ uint4 a_lds[DECODE_MAX_TOKENS][256];
  __shared__ float asum_lds[DECODE_MAX_TOKENS][64];
  __shared__ double red[4];
  for (int t = 0; t < n; ++t) block_input_to_lds(x + (size_t)t * H, a_lds[t], asum_lds[t], red);
  __syncthreads();
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (blockIdx.x == 0) {
    for (int t = 0; t < n; ++t) {
      reinterpret_cast<uint4*>(ws.a)[t * 256 + tid] = a_lds[t][tid];
      if (tid < 64) ws.asum[t * 64 + tid] = asum_lds[t][tid];
    }
  }
  // router row e = blockIdx.x, split over the four waves
  {
    __shared__ double zpart[DECODE_MAX_TOKENS][4];
    const int e = blockIdx.x;
    const uint4 wr = reinterpret_cast<const uint4*>(L.router + (size_t)e * H)[4 * lane + wave];
    for (int t = 0; t < n; ++t) {
      const double p = router_part(wr, a_lds[t]);
      if (lane == 0) zpart[t][wave] = p;
    }
    __syncthreads();
    if (tid < n) {
      double s, c;
      router_scores(zpart[tid], L.bias[e], s, c);
      ws.s[tid * E + e] = s;
      ws.c[tid * E + e] = c;
    }
  }
  // shared expert gate/up: one row per wave
  const int r = blockIdx.x * 4 + wave;
  const uint4 cg = reinterpret_cast<const uint4*>(L.sh_gate + (size_t)r * (H / 2))[lane];
  const uint4 cu = reinterpret_cast<const uint4*>(L.sh_up + (size_t)r * (H / 2))[lane];
  const float sg = bf16_bits_to_f32(L.sh_gate_s[r * (H / G) + (lane >> 2)]);
  const float su = bf16_bits_to_f32(L.sh_up_s[r * (H / G) + (lane >> 2)]);
  for (int t = 0; t < n; ++t) {
    float hv = gateup_row_token(cg, sg, cu, su, a_lds[t], asum_lds[t][lane]);
    if (lane == 0) ws.hsh[t * IS + r] = hv;
  }
}

__global__ void __launch_bounds__(256) k_route_gateup(int n, LayerW L, DecodeWS ws, int* trace_ids,
                                                      float* trace_w) {
  __shared__ uint4 a_lds[DECODE_MAX_TOKENS][256];
  __shared__ float asum_lds[DECODE_MAX_TOKENS][64];
  __shared__ int ids_l[DECODE_MAX_TOKENS][TOPK];
  __shared__ float w_l[DECODE_MAX_TOKENS][TOPK];
  __shared__ int mark[E];
  __shared__ int list[DECODE_MAX_TOKENS * TOPK];
  __shared__ signed char slotmap[DECODE_MAX_TOKENS * TOPK][DECODE_MAX_TOKENS];
  __shared__ int wave_tot[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int t = 0; t < n; ++t) {
    a_lds[t][tid] = reinterpret_cast<const uint4*>(ws.a)[t * 256 + tid];
    if (tid < 64) asum_lds[t][tid] = ws.asum[t * 64 + tid];
  }
  mark[tid] = 0;
  for (int t = wave; t < n; t += 4) route_token(ws.c + t * E, ws.s + t * E, ids_l[t], w_l[t]);
  __syncthreads();
  if (blockIdx.x == 0 && tid < n * TOPK) {
    ws.ids[tid] = ids_l[tid / TOPK][tid % TOPK];
    ws.w[tid] = w_l[tid / TOPK][tid % TOPK];
    if (trace_ids) {
      trace_ids[tid] = ids_l[tid / TOPK][tid % TOPK];
      trace_w[tid] = w_l[tid / TOPK][tid % TOPK];
    }
  }
  if (tid < n * TOPK) mark[ids_l[tid / TOPK][tid % TOPK]] = 1;
  __syncthreads();
  const int D = distinct_experts(mark, list, wave_tot);

  for (int i = tid; i < D * DECODE_MAX_TOKENS; i += 256) slotmap[i / DECODE_MAX_TOKENS][i % DECODE_MAX_TOKENS] = -1;
  __syncthreads();
  if (tid < n * TOPK) slotmap[mark[ids_l[tid / TOPK][tid % TOPK]]][tid / TOPK] = (signed char)(tid % TOPK);
  __syncthreads();
  // tasks: (distinct expert d, row r), one per wave at a time
  const int nwaves = gridDim.x * 4;
  for (int q = blockIdx.x * 4 + wave; q < D * I; q += nwaves) {
    const int d = q / I, r = q % I, e = list[d];
    const size_t row = (size_t)e * I + r;
    const uint4 cg = reinterpret_cast<const uint4*>(L.gate + row * (H / 2))[lane];
    const uint4 cu = reinterpret_cast<const uint4*>(L.up + row * (H / 2))[lane];
    const float sg = bf16_bits_to_f32(L.gate_s[row * (H / G) + (lane >> 2)]);
    const float su = bf16_bits_to_f32(L.up_s[row * (H / G) + (lane >> 2)]);
    for (int t = 0; t < n; ++t) {
      const int slot = slotmap[d][t];
      if (slot < 0) continue;
      float hv = gateup_row_token(cg, sg, cu, su, a_lds[t], asum_lds[t][lane]);
      if (lane == 0) ws.h[(t * TOPK + slot) * I + r] = hv;
    }
  }
}

__global__ void __launch_bounds__(256) k_down_combine(const float* xin, float* out, int n, LayerW L, DecodeWS ws) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, sub = lane & 15;
  const int nrow = blockIdx.x * 4 + wave;
  for (int t = 0; t < n; ++t) {
    uint4 ca, cb;
    float sa, sb;
    load_down_row(L, ws.ids + t * TOPK, nrow, ca, sa, cb, sb);
    const float* h = ws.h + (size_t)t * TOPK * I;
    const HChunk ha = load_chunk_natural(h + (lane >> 4) * I, sub);
    const HChunk hb = (lane < 32) ? load_chunk_natural(h + (4 + (lane >> 4)) * I, sub)
                                  : load_chunk_natural(ws.hsh + (size_t)t * IS, lane - 32);
    const float v = down_row_token(ca, sa, cb, sb, ha, hb, ws.w + t * TOPK, xin[(size_t)t * H + nrow]);
    if (lane == 0) out[(size_t)t * H + nrow] = v;
  }
}

// ----------------------------------------------------------------- launch
hipError_t launch_decode_layer(const float* xin, float* out, int n, const LayerW& L, const DecodeWS& ws,
                               int* trace_ids, float* trace_w, hipStream_t s) {
  hipLaunchKernelGGL(k_norm_router, dim3(E), dim3(256), 0, s, xin, n, L, ws);
  hipLaunchKernelGGL(k_route_gateup, dim3(256), dim3(256), 0, s, n, L, ws, trace_ids, trace_w);
  hipLaunchKernelGGL(k_down_combine, dim3(H / 4), dim3(256), 0, s, xin, out, n, L, ws);
  return hipGetLastError();
}

}  // namespace flint
