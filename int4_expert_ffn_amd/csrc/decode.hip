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
#include "decode.h"

namespace flint {

// ----------------------------------------------------------------- helpers
// Block input of token t into LDS (pair order) and its 64 lane-chunk sums.
// 256 threads: thread i owns elements [8 i, 8 i + 8), one pair-order uint4.
__device__ void block_input_to_lds(const float* __restrict__ x, uint4* a_lds, float* asum_lds,
                                   double* red) {
  const int tid = threadIdx.x;
  const float4* xp = reinterpret_cast<const float4*>(x) + 2 * tid;
  float4 v0 = xp[0], v1 = xp[1];
  double xs[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += xs[j] * xs[j];     // exact squares of fp32 values
  ss = wave_sum(ss);
  const int wave = tid >> 6, lane = tid & 63;
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  double tot = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  double den = sqrt(tot / (double)H + RMS_EPS);
  uint32_t b[8];
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    b[j] = f64_to_bf16_rne(xs[j] / den);
    part += bf16_bits_to_f32(b[j]);
  }
  // pair order (0,2),(4,6),(1,3),(5,7)
  a_lds[tid] = make_uint4(b[0] | (b[2] << 16), b[4] | (b[6] << 16), b[1] | (b[3] << 16), b[5] | (b[7] << 16));
  part = group_sum<4>(part);          // 4 threads = 32 elements = one lane chunk
  if ((tid & 3) == 0) asum_lds[tid >> 2] = part;
}

// fp64 dot of 8 router weights (natural order) with 8 activations (pair order)
__device__ __forceinline__ double router_dot8(uint4 w, uint4 a) {
  // natural k0..k7 from w; activations: a.x=(k0,k2) a.y=(k4,k6) a.z=(k1,k3) a.w=(k5,k7)
  float wk[8] = {bf16_bits_to_f32(w.x & 0xFFFF), bf16_bits_to_f32(w.x >> 16),
                 bf16_bits_to_f32(w.y & 0xFFFF), bf16_bits_to_f32(w.y >> 16),
                 bf16_bits_to_f32(w.z & 0xFFFF), bf16_bits_to_f32(w.z >> 16),
                 bf16_bits_to_f32(w.w & 0xFFFF), bf16_bits_to_f32(w.w >> 16)};
  float ak[8] = {bf16_bits_to_f32(a.x & 0xFFFF), bf16_bits_to_f32(a.z & 0xFFFF),
                 bf16_bits_to_f32(a.x >> 16), bf16_bits_to_f32(a.z >> 16),
                 bf16_bits_to_f32(a.y & 0xFFFF), bf16_bits_to_f32(a.w & 0xFFFF),
                 bf16_bits_to_f32(a.y >> 16), bf16_bits_to_f32(a.w >> 16)};
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (double)(wk[j] * ak[j]);   // bf16 x bf16 is exact in fp32
  return s;
}

// gate/up of one row for one token: returns h = silu(g) u (same in all lanes)
__device__ __forceinline__ float gateup_row_token(uint4 cg, float sg, uint4 cu, float su,
                                                  const uint4* a_tok, float asum_lane) {
  const int lane = threadIdx.x & 63;
  const uint4* a4 = a_tok + 4 * lane;
  uint4 av[4] = {a4[0], a4[1], a4[2], a4[3]};
  float g = wave_sum(lane_dot_gateup(cg, av, asum_lane, sg));
  float u = wave_sum(lane_dot_gateup(cu, av, asum_lane, su));
  return silu_mul(g, u);
}

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
  // router row e = blockIdx.x, by wave 0: lane owns k in [32 lane, 32 lane + 32)
  if (wave == 0) {
    const int e = blockIdx.x;
    const uint4* wr = reinterpret_cast<const uint4*>(L.router + (size_t)e * H) + 4 * lane;
    uint4 w[4] = {wr[0], wr[1], wr[2], wr[3]};
    for (int t = 0; t < n; ++t) {
      double s = 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j) s += router_dot8(w[j], a_lds[t][4 * lane + j]);
      s = wave_sum(s);
      if (lane == 0) ws.z[t * E + e] = s;
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

// ----------------------------------------------------------------- kernel 2
// Top-6 of token t by one wavefront.  Lane l holds experts l + 64 j.
__device__ void route_token(const double* __restrict__ z, const float* __restrict__ bias, int* ids_out,
                            float* w_out) {
  const int lane = threadIdx.x & 63;
  double s[4], c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    s[j] = sigmoid_f64(z[e]);
    c[j] = s[j] + (double)bias[e];
    if (c[j] != c[j]) c[j] = -INFINITY;   // a NaN score never wins; ids stay in [0, E)
  }
  unsigned removed = 0;
  int ids[TOPK];
  double ss[TOPK];
  for (int r = 0; r < TOPK; ++r) {
    double bc = -INFINITY;
    int be = 1 << 20;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (!((removed >> j) & 1u) && (c[j] > bc || (c[j] == bc && e < be))) { bc = c[j]; be = e; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      double oc = __shfl_xor(bc, off);
      int oe = __shfl_xor(be, off);
      if (oc > bc || (oc == bc && oe < be)) { bc = oc; be = oe; }
    }
    ids[r] = be;
    if ((be & 63) == lane) removed |= 1u << (be >> 6);
    double mine = s[0];
#pragma unroll
    for (int j = 1; j < 4; ++j) if ((be >> 6) == j) mine = s[j];
    ss[r] = __shfl(mine, be & 63);
  }
  double tot = 0.0;
#pragma unroll
  for (int r = 0; r < TOPK; ++r) tot += ss[r];
  if (lane < TOPK) {
    int id = ids[0];
    double sv = ss[0];
#pragma unroll
    for (int r = 1; r < TOPK; ++r) if (lane == r) { id = ids[r]; sv = ss[r]; }
    ids_out[lane] = id;
    w_out[lane] = (float)(sv / tot);
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
  __shared__ int n_distinct;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int t = 0; t < n; ++t) {
    a_lds[t][tid] = reinterpret_cast<const uint4*>(ws.a)[t * 256 + tid];
    if (tid < 64) asum_lds[t][tid] = ws.asum[t * 64 + tid];
  }
  mark[tid] = 0;
  for (int t = wave; t < n; t += 4) route_token(ws.z + t * E, L.bias, ids_l[t], w_l[t]);
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
  // distinct experts in increasing id order
  if (tid == 0) {
    int d = 0;
    for (int e = 0; e < E; ++e) {
      if (mark[e]) { mark[e] = d; list[d++] = e; }
      else mark[e] = -1;
    }
    n_distinct = d;
  }
  __syncthreads();
  const int D = n_distinct;
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

// ----------------------------------------------------------------- kernel 3
__device__ __forceinline__ float lane_down(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                           int K, int row, int sub, const float* __restrict__ h) {
  const uint4 c = reinterpret_cast<const uint4*>(codes + (size_t)row * (K / 2))[sub];
  const float sc = bf16_bits_to_f32(scales[(size_t)row * (K / G) + (sub >> 2)]);
  const float4* h4 = reinterpret_cast<const float4*>(h + 32 * sub);
  float4 hv[8];
  float hs = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    hv[j] = h4[j];
    hs += ((hv[j].x + hv[j].y) + hv[j].z) + hv[j].w;
  }
  return lane_dot_down(c, hv, hs, sc);
}

__global__ void __launch_bounds__(256) k_down_combine(const float* xin, float* out, int n, LayerW L, DecodeWS ws) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nrow = blockIdx.x * 4 + wave;
  const int sub = lane & 15;
  for (int t = 0; t < n; ++t) {
    const int* ids = ws.ids + t * TOPK;
    const float* w = ws.w + t * TOPK;
    // pass A: slots 0..3, 16 lanes each
    const int sa = lane >> 4;
    float ya = lane_down(L.down + (size_t)ids[sa] * H * (I / 2), L.down_s + (size_t)ids[sa] * H * (I / G),
                         I, nrow, sub, ws.h + (t * TOPK + sa) * I);
    ya = group_sum<16>(ya);
    // pass B: slots 4, 5 on lanes 0..31, shared expert on lanes 32..63
    float yb;
    if (lane < 32) {
      const int sb = 4 + (lane >> 4);
      yb = lane_down(L.down + (size_t)ids[sb] * H * (I / 2), L.down_s + (size_t)ids[sb] * H * (I / G),
                     I, nrow, sub, ws.h + (t * TOPK + sb) * I);
    } else {
      yb = lane_down(L.sh_down, L.sh_down_s, IS, nrow, lane - 32, ws.hsh + t * IS);
    }
    const float yb16 = group_sum<16>(yb);
    const float yb32 = yb16 + __shfl_xor(yb16, 16);   // 32-lane sum (used by lanes 32..63)
    const float y0 = __shfl(ya, 0), y1 = __shfl(ya, 16), y2 = __shfl(ya, 32), y3 = __shfl(ya, 48);
    const float y4 = __shfl(yb16, 0), y5 = __shfl(yb16, 16), ysh = __shfl(yb32, 32);
    if (lane == 0) {
      float d = w[0] * y0;
      d = fmaf(w[1], y1, d);
      d = fmaf(w[2], y2, d);
      d = fmaf(w[3], y3, d);
      d = fmaf(w[4], y4, d);
      d = fmaf(w[5], y5, d);
      d += ysh;
      out[(size_t)t * H + nrow] = xin[(size_t)t * H + nrow] + d;
    }
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
