// Device math shared by both decode launch modes (per-layer kernels and the
// persistent kernel): both call these same functions with the same lane
// partitions and reduction trees, so they produce bitwise-identical results.
#pragma once
#include "decode.h"

namespace flint {

// ----------------------------------------------------------------- block input
// Block input of one token into LDS and its 64 lane-chunk sums.
// 256 threads: thread i owns elements [8 i, 8 i + 8), one pair-order uint4.
// Layout: the 8-element chunk c = 4 L + j (lane chunk L, j < 4) sits at uint4
// position j * 64 + L, so lane L reading its four chunks touches consecutive
// 16-byte slots across lanes (no LDS bank conflicts).
// RMSNorm in fp64 (squares of fp32 values are exact), one rounding to bf16.
__device__ __forceinline__ void block_input_to_lds(const float* __restrict__ x, uint4* a_lds, float* asum_lds,
                                                   double* red) {
  const int tid = threadIdx.x;
  const float4* xp = reinterpret_cast<const float4*>(x) + 2 * tid;
  const float4 v0 = xp[0], v1 = xp[1];
  const double xs[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += xs[j] * xs[j];
  ss = wave_sum(ss);
  const int wave = tid >> 6, lane = tid & 63;
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const double tot = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  const double den = sqrt(tot / (double)H + RMS_EPS);
  uint32_t b[8];
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    b[j] = f64_to_bf16_rne(xs[j] / den);
    part += bf16_bits_to_f32(b[j]);
  }
  // pair order (0,2),(4,6),(1,3),(5,7)
  a_lds[(tid & 3) * 64 + (tid >> 2)] =
      make_uint4(b[0] | (b[2] << 16), b[4] | (b[6] << 16), b[1] | (b[3] << 16), b[5] | (b[7] << 16));
  part += dpp_f32<DPP_XOR1>(part);     // 4 threads = 32 elements = one lane chunk
  part += dpp_f32<DPP_XOR2>(part);
  if ((tid & 3) == 0) asum_lds[tid >> 2] = part;
}

// ----------------------------------------------------------------- router
// fp64 dot of 8 router weights (natural order) with 8 activations (pair order)
__device__ __forceinline__ double router_dot8(uint4 w, uint4 a) {
  // natural k0..k7 from w; activations: a.x=(k0,k2) a.y=(k4,k6) a.z=(k1,k3) a.w=(k5,k7)
  const float wk[8] = {bf16_bits_to_f32(w.x & 0xFFFF), bf16_bits_to_f32(w.x >> 16),
                       bf16_bits_to_f32(w.y & 0xFFFF), bf16_bits_to_f32(w.y >> 16),
                       bf16_bits_to_f32(w.z & 0xFFFF), bf16_bits_to_f32(w.z >> 16),
                       bf16_bits_to_f32(w.w & 0xFFFF), bf16_bits_to_f32(w.w >> 16)};
  const float ak[8] = {bf16_bits_to_f32(a.x & 0xFFFF), bf16_bits_to_f32(a.z & 0xFFFF),
                       bf16_bits_to_f32(a.x >> 16), bf16_bits_to_f32(a.z >> 16),
                       bf16_bits_to_f32(a.y & 0xFFFF), bf16_bits_to_f32(a.w & 0xFFFF),
                       bf16_bits_to_f32(a.y >> 16), bf16_bits_to_f32(a.w >> 16)};
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (double)(wk[j] * ak[j]);   // bf16 x bf16 is exact in fp32
  return s;
}

// Part of the router logit of one expert row held by wave v: lane L holds the
// row's weights for chunk 4 L + v (one uint4); summed over the wavefront.
// The four waves' parts are added in order 0..3 by router_scores().
__device__ __forceinline__ double router_part(uint4 wr, const uint4* a_tok) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return wave_sum(router_dot8(wr, a_tok[wave * 64 + lane]));
}

// s = sigmoid(z), c = s + b from the four parts (fp64).  A NaN selection
// score is replaced by -inf so it never wins.
__device__ __forceinline__ void router_scores(const double* part4, float bias, double& s, double& c) {
  const double z = ((part4[0] + part4[1]) + part4[2]) + part4[3];
  s = sigmoid_f64(z);
  c = s + (double)bias;
  if (c != c) c = -INFINITY;
}

// ----------------------------------------------------------------- selection
// Order-preserving 32-bit key of a selection score with the expert index in
// its low byte: the score rounded toward -inf to fp32, mapped so unsigned
// order equals numeric order, with the low 8 bits replaced by 255 - e (ties
// in the kept 24 bits go to the lower index).  key(c1) > key(c2) implies
// c1 > c2 whenever the kept 24 bits differ.
__device__ __forceinline__ uint32_t coarse_key(double c, int e) {
  const uint32_t u = __float_as_uint(__double2float_rd(c));
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (ord & 0xFFFFFF00u) | (uint32_t)(255 - e);
}

// Exact top-k by (c descending, index ascending) with fp64 comparisons;
// used when the coarse keys cannot separate the k-th and (k+1)-th scores.
__device__ __forceinline__ void topk_exact(const double* c, int* ids) {
  const int lane = threadIdx.x & 63;
  double cv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cv[j] = c[lane + 64 * j];
  unsigned removed = 0;
  for (int r = 0; r < TOPK; ++r) {
    double bc = -INFINITY;
    int be = E;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (!((removed >> j) & 1u) && (cv[j] > bc || (cv[j] == bc && e < be))) { bc = cv[j]; be = e; }
    }
    double t = bc;                       // row maxima, then the max of the four rows
    t = fmax(t, dpp_f64<DPP_XOR1>(t));
    t = fmax(t, dpp_f64<DPP_XOR2>(t));
    t = fmax(t, dpp_f64<DPP_HALF_MIRROR>(t));
    t = fmax(t, dpp_f64<DPP_MIRROR>(t));
    const double m = fmax(fmax(lane_bcast(t, 0), lane_bcast(t, 16)), fmax(lane_bcast(t, 32), lane_bcast(t, 48)));
    unsigned long long hit = __ballot(bc == m);   // lanes whose best equals the max
    int best = E;
    while (hit) {
      const int l2 = __ffsll((long long)hit) - 1;
      hit &= hit - 1;
      best = min(best, __builtin_amdgcn_readlane(be, l2));
    }
    ids[r] = best;
    if ((best & 63) == lane) removed |= 1u << (best >> 6);
  }
}

// Top-6 of one token by one wavefront from its 256 scores (LDS), written as
// ids (decreasing c, ties to the lower index) and weights s_i / sum_T s.
__device__ __forceinline__ void route_token(const double* __restrict__ c, const double* __restrict__ s,
                                            int* ids_out, float* w_out) {
  const int lane = threadIdx.x & 63;
  uint32_t k[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) k[j] = coarse_key(c[lane + 64 * j], lane + 64 * j);
  uint32_t picked[TOPK + 1];
#pragma unroll
  for (int r = 0; r <= TOPK; ++r) {
    const uint32_t m = wave_max_u32(max(max(k[0], k[1]), max(k[2], k[3])));
    picked[r] = m;
    const int e = 255 - (int)(m & 0xFFu);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == e) k[j] = 0u;
  }
  int ids[TOPK];
  if ((picked[TOPK - 1] >> 8) != (picked[TOPK] >> 8)) {
    // the k-th and (k+1)-th keys differ in their kept bits: the set is exact;
    // order it by the exact scores (insertion sort, uniform across lanes)
#pragma unroll
    for (int r = 0; r < TOPK; ++r) ids[r] = 255 - (int)(picked[r] & 0xFFu);
#pragma unroll
    for (int i = 1; i < TOPK; ++i) {
#pragma unroll
      for (int j = i; j > 0; --j) {
        const int a = ids[j - 1], b = ids[j];
        const bool swap = c[b] > c[a] || (c[b] == c[a] && b < a);
        if (swap) { ids[j - 1] = b; ids[j] = a; }
      }
    }
  } else {
    topk_exact(c, ids);
  }
  double sv[TOPK], tot = 0.0;
#pragma unroll
  for (int r = 0; r < TOPK; ++r) {
    sv[r] = s[ids[r]];
    tot += sv[r];
  }
  if (lane < TOPK) {
    int id = ids[0];
    double v = sv[0];
#pragma unroll
    for (int r = 1; r < TOPK; ++r)
      if (lane == r) { id = ids[r]; v = sv[r]; }
    ids_out[lane] = id;
    w_out[lane] = (float)(v / tot);
  }
}

// ----------------------------------------------------------------- gate / up
// gate/up of one row for one token: returns h = silu(g) u (same in all lanes)
__device__ __forceinline__ float gateup_row_token(uint4 cg, float sg, uint4 cu, float su, const uint4* a_tok,
                                                  float asum_lane) {
  const int lane = threadIdx.x & 63;
  const uint4 av[4] = {a_tok[lane], a_tok[64 + lane], a_tok[128 + lane], a_tok[192 + lane]};
  const float g = wave_sum(lane_dot_gateup(cg, av, asum_lane, sg));
  const float u = wave_sum(lane_dot_gateup(cu, av, asum_lane, su));
  return silu_mul(g, u);
}

// ----------------------------------------------------------------- down
// h values of one lane chunk (32 consecutive k) as 8 float4, and their sum.
struct HChunk {
  float4 v[8];
  float sum;
};

__device__ __forceinline__ void chunk_finish(HChunk& hc) {
  float hs = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) hs += ((hc.v[j].x + hc.v[j].y) + hc.v[j].z) + hc.v[j].w;
  hc.sum = hs;
}

// chunk `sub` of h in natural order (h[32 sub .. 32 sub + 32))
__device__ __forceinline__ HChunk load_chunk_natural(const float* h, int sub) {
  HChunk hc;
  const float4* p = reinterpret_cast<const float4*>(h + 32 * sub);
#pragma unroll
  for (int j = 0; j < 8; ++j) hc.v[j] = p[j];
  chunk_finish(hc);
  return hc;
}

// chunk `sub` of h stored transposed: float4 j of chunk sub at (j * nsub + sub)
__device__ __forceinline__ HChunk load_chunk_transposed(const float* h, int sub, int nsub) {
  HChunk hc;
  const float4* p = reinterpret_cast<const float4*>(h);
#pragma unroll
  for (int j = 0; j < 8; ++j) hc.v[j] = p[j * nsub + sub];
  chunk_finish(hc);
  return hc;
}

// Position of h word k of a K-wide vector in the transposed layout.
__device__ __forceinline__ int transposed_pos(int k, int nsub) {
  return ((((k & 31) >> 2) * nsub + (k >> 5)) << 2) | (k & 3);
}

// Codes and scale of lane `sub` of down row `row` of a [rows][K] int4 matrix.
__device__ __forceinline__ void load_down_lane(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                               int K, int row, int sub, uint4& c, float& sc) {
  c = reinterpret_cast<const uint4*>(codes + (size_t)row * (K / 2))[sub];
  sc = bf16_bits_to_f32(scales[(size_t)row * (K / G) + (sub >> 2)]);
}

// This lane's down codes for output row `row` of one token:
//   pass A: lanes 16 s .. 16 s + 15 take routed slot s (s = 0..3)
//   pass B: lanes 0..31 take slots 4, 5; lanes 32..63 the shared expert.
__device__ __forceinline__ void load_down_row(const LayerW& L, const int* ids, int row, uint4& ca, float& sa,
                                              uint4& cb, float& sb) {
  const int lane = threadIdx.x & 63, sub = lane & 15;
  const int e_a = ids[lane >> 4];
  load_down_lane(L.down + (size_t)e_a * H * (I / 2), L.down_s + (size_t)e_a * H * (I / G), I, row, sub, ca, sa);
  if (lane < 32) {
    const int e_b = ids[4 + (lane >> 4)];
    load_down_lane(L.down + (size_t)e_b * H * (I / 2), L.down_s + (size_t)e_b * H * (I / G), I, row, sub, cb, sb);
  } else {
    load_down_lane(L.sh_down, L.sh_down_s, IS, row, lane - 32, cb, sb);
  }
}

// One output row of one token by one wavefront: the six routed down rows and
// the shared one, then out = x + ((((w0 y0 + w1 y1) + w2 y2) + ...) + w5 y5)
// + y_shared.  ha: this lane's h chunk for pass A (slot lane / 16); hb: for
// pass B (slot 4 + lane / 16 on lanes 0..31, the shared expert on 32..63).
// The result is the same in every lane.
__device__ __forceinline__ float down_row_token(uint4 ca, float sa, uint4 cb, float sb, const HChunk& ha,
                                                const HChunk& hb, const float* w, float xres) {
  const float ya = row16_sum(lane_dot_down(ca, ha.v, ha.sum, sa));
  const float yb = row16_sum(lane_dot_down(cb, hb.v, hb.sum, sb));
  const float ysh = lane_bcast(yb + dpp_f32<DPP_BCAST15, 0x8>(yb), 63);   // rows 2 + 3: shared row
  const float y0 = lane_bcast(ya, 0), y1 = lane_bcast(ya, 16), y2 = lane_bcast(ya, 32), y3 = lane_bcast(ya, 48);
  const float y4 = lane_bcast(yb, 0), y5 = lane_bcast(yb, 16);
  float d = w[0] * y0;
  d = fmaf(w[1], y1, d);
  d = fmaf(w[2], y2, d);
  d = fmaf(w[3], y3, d);
  d = fmaf(w[4], y4, d);
  d = fmaf(w[5], y5, d);
  d += ysh;
  return xres + d;
}

// Distinct experts among the picks flagged in mark[E] (non-zero = picked), in
// increasing id order: on return mark[e] = rank or -1, list[rank] = e.
// Needs blockDim.x == E; wave_tot is LDS scratch of 4 ints.
__device__ __forceinline__ int distinct_experts(int* mark, int* list, int* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int f = mark[tid] != 0;
  const unsigned long long b = __ballot(f);
  const int pre = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) wave_tot[wave] = __popcll(b);
  __syncthreads();
  int off = 0;
  for (int i = 0; i < wave; ++i) off += wave_tot[i];
  const int D = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
  const int r = f ? off + pre : -1;
  mark[tid] = r;
  if (f) list[r] = tid;
  __syncthreads();
  return D;
}

}  // namespace flint
