// Device math shared by both decode launch modes (per-layer kernels and the
// persistent kernel): both call these same functions with the same lane
// partitions and reduction trees, so they produce bitwise-identical results.
#pragma once
#include "decode.h"

namespace flint {

// ----------------------------------------------------------------- block input
constexpr int NT = 512;          // threads per workgroup of the decode kernels
constexpr int NWAVES = NT / 64;

// Block input of one token: thread i holds elements [4 i, 4 i + 4) of the fp32
// residual.  RMSNorm in fp64 (squares of fp32 values are exact; per-thread
// sums, then a fixed wave tree, then the 8 waves in order), one rounding to
// bf16.  `red` holds NWAVES doubles and must not be reused by the next call
// before a barrier (callers alternate two buffers).  Writes the activation to LDS in pair order and transposed layout:
// the 8-element chunk c = 4 L + j (lane chunk L, j < 4) is the uint4 at
// position j * 64 + L, holding (k0,k2),(k4,k6),(k1,k3),(k5,k7); lane L reading
// its four chunks touches consecutive 16-byte slots (no bank conflicts).
// asum_lds[L] = sum of the 32 bf16 values of lane chunk L.
__device__ __forceinline__ void block_input(float4 xv, uint32_t* a_u32, float* asum_lds, double* red) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const double xs[4] = {xv.x, xv.y, xv.z, xv.w};
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) ss += xs[j] * xs[j];
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  wg_sync();
  double tot = red[0];
#pragma unroll
  for (int i = 1; i < NWAVES; ++i) tot += red[i];
  const double ms = tot / (double)H + RMS_EPS;
  const double rinv = rsqrt(ms);
  double q[4];
  float qf[4];
  bool hard = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    q[j] = xs[j] * rinv;
    qf[j] = (float)q[j];
    hard |= f32_on_bf16_midpoint(qf[j]);
  }
  uint32_t b[4];
  if (__builtin_expect(__ballot(hard) != 0ull, 0)) {   // wave-uniform, rare
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // x * rsqrt(ms) is within a few fp64 ulps of x / sqrt(ms); where that
      // could change the bf16 rounding, use the correctly rounded quotient
      double qq = q[j];
      if (near_bf16_midpoint(qq)) qq = xs[j] / sqrt(ms);
      b[j] = f64_to_bf16_rne(qq);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = f32_to_bf16_rne(qf[j]);
  }
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) part += bf16_bits_to_f32(b[j]);
  const int c = tid >> 1, half = tid & 1;
  const int P = ((c & 3) * 64 + (c >> 2)) * 4;
  a_u32[P + half] = b[0] | (b[2] << 16);       // (k0,k2) or (k4,k6)
  a_u32[P + 2 + half] = b[1] | (b[3] << 16);   // (k1,k3) or (k5,k7)
  part += dpp_f32<DPP_XOR1>(part);             // 8 threads = 32 elements = one lane chunk
  part += dpp_f32<DPP_XOR2>(part);
  part += dpp_f32<DPP_HALF_MIRROR>(part);
  if ((tid & 7) == 0) asum_lds[tid >> 3] = part;
}

// The router row of expert e is split over the 512 threads of a workgroup:
// thread t holds the row's 4 weights (8 bytes) for elements 4 t .. 4 t + 3,
// i.e. half t & 1 of 8-element chunk t >> 1.
__device__ __forceinline__ uint2 load_router_part(const uint16_t* router_row) {
  return reinterpret_cast<const uint2*>(router_row)[threadIdx.x];
}

// This wave's part of the router logit (fp64, same value in every lane).
__device__ __forceinline__ double router_part(uint2 w, const uint4* a_tok) {
  const int c = threadIdx.x >> 1, half = threadIdx.x & 1;
  const uint4 a = a_tok[(c & 3) * 64 + (c >> 2)];
  // weights in natural order k0..k3 of the half; activations in pair order
  const uint32_t alo = half ? a.y : a.x;   // (k0,k2) or (k4,k6)
  const uint32_t ahi = half ? a.w : a.z;   // (k1,k3) or (k5,k7)
  const float wk[4] = {bf16_bits_to_f32(w.x & 0xFFFF), bf16_bits_to_f32(w.x >> 16),
                       bf16_bits_to_f32(w.y & 0xFFFF), bf16_bits_to_f32(w.y >> 16)};
  const float ak[4] = {bf16_bits_to_f32(alo & 0xFFFF), bf16_bits_to_f32(ahi & 0xFFFF),
                       bf16_bits_to_f32(alo >> 16), bf16_bits_to_f32(ahi >> 16)};
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += (double)(wk[j] * ak[j]);   // bf16 x bf16 is exact in fp32
  return wave_sum(s);
}

// s = sigmoid(z), c = s + b from the 8 wave parts (summed in order, fp64).
// A NaN selection score is replaced by -inf so it never wins.
__device__ __forceinline__ void router_scores(const double* part, float bias, double& s, double& c) {
  double z = part[0];
#pragma unroll
  for (int i = 1; i < NWAVES; ++i) z += part[i];
  s = sigmoid_f64(z);
  c = s + (double)bias;
  if (c != c) c = -INFINITY;
}

// ----------------------------------------------------------------- selection
// Order-preserving 32-bit key of a selection score with the expert index in
// its low byte: the top 24 bits of the score's fp64 pattern mapped so that
// unsigned order equals numeric order (sign, exponent, 12 mantissa bits),
// with 255 - e below them (ties in the kept bits go to the lower index).
// key(c1) > key(c2) implies c1 > c2 whenever the kept 24 bits differ.
__device__ __forceinline__ uint32_t coarse_key(double c, int e) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(c);
  const unsigned long long ord = (u >> 63) ? ~u : (u | 0x8000000000000000ull);
  return ((uint32_t)(ord >> 32) & 0xFFFFFF00u) | (uint32_t)(255 - e);
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

// Maximum of a 32-bit unsigned key over the wavefront, in every lane: rows of
// 16 by DPP, then rows 0+1 and 2+3, then the two halves by the lane-swap
// instructions (no read-back through a scalar register).
__device__ __forceinline__ uint32_t wave_max_all_u32(uint32_t v) {
  v = max(v, dpp_u32<DPP_XOR1>(v));
  v = max(v, dpp_u32<DPP_XOR2>(v));
  v = max(v, dpp_u32<DPP_HALF_MIRROR>(v));
  v = max(v, dpp_u32<DPP_MIRROR>(v));
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);   // rows (0,0,2,2) / (1,1,3,3)
  v = max((uint32_t)r[0], (uint32_t)r[1]);
  const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);   // halves (lo,lo) / (hi,hi)
  return max((uint32_t)h[0], (uint32_t)h[1]);
}

// Top-6 of one token by one wavefront from its 256 selection scores c: ids in
// decreasing c, ties to the lower index (the same values in every lane).
__device__ __forceinline__ void route_select(const double* __restrict__ c, int (&ids)[TOPK]) {
  const int lane = threadIdx.x & 63;
  uint32_t k0 = coarse_key(c[lane], lane), k1 = coarse_key(c[lane + 64], lane + 64);
  uint32_t k2 = coarse_key(c[lane + 128], lane + 128), k3 = coarse_key(c[lane + 192], lane + 192);
  // the lane's four keys in decreasing order (five compare-exchanges)
  auto cx = [](uint32_t& hi, uint32_t& lo) {
    const uint32_t a = max(hi, lo), b = min(hi, lo);
    hi = a;
    lo = b;
  };
  cx(k0, k1);
  cx(k2, k3);
  cx(k0, k2);
  cx(k1, k3);
  cx(k1, k2);
  // seven rounds: the largest remaining key (keys are distinct: the index is
  // in their low byte) leaves the head of its lane's list; every real key is
  // above 0
  uint32_t picked[TOPK + 1];
#pragma unroll
  for (int r = 0; r <= TOPK; ++r) {
    const uint32_t m = wave_max_all_u32(k0);
    picked[r] = m;
    const bool hit = k0 == m;
    k0 = hit ? k1 : k0;
    k1 = hit ? k2 : k1;
    k2 = hit ? k3 : k2;
    k3 = hit ? 0u : k3;
  }
#pragma unroll
  for (int r = 0; r <= TOPK; ++r) picked[r] = (uint32_t)__builtin_amdgcn_readfirstlane((int)picked[r]);
  if ((picked[TOPK - 1] >> 8) != (picked[TOPK] >> 8)) {
    // the k-th and (k+1)-th keys differ in their kept bits: the set is exact.
    // The keys order it exactly too, except inside runs of equal kept bits,
    // which are re-ordered by the exact scores (rare).
    bool tie = false;
#pragma unroll
    for (int r = 0; r < TOPK; ++r) {
      ids[r] = 255 - (int)(picked[r] & 0xFFu);
      if (r > 0) tie |= (picked[r - 1] >> 8) == (picked[r] >> 8);
    }
    if (tie) {
#pragma unroll
      for (int i = 1; i < TOPK; ++i) {
#pragma unroll
        for (int j = i; j > 0; --j) {
          const int a = ids[j - 1], b = ids[j];
          const bool swap = c[b] > c[a] || (c[b] == c[a] && b < a);
          if (swap) { ids[j - 1] = b; ids[j] = a; }
        }
      }
    }
  } else {
    topk_exact(c, ids);
  }
}

// ids[0..6) to memory, by lanes 0..5.
__device__ __forceinline__ void write_ids(const int (&ids)[TOPK], int* ids_out) {
  const int lane = threadIdx.x & 63;
  if (lane < TOPK) {
    int id = ids[0];
#pragma unroll
    for (int r = 1; r < TOPK; ++r)
      if (lane == r) id = ids[r];
    ids_out[lane] = id;
  }
}

// Weights of the picks ids[0..6): s_i / sum_T s in fp64, summed in pick
// order; written as fp32 by lanes 0..5, which also return their weight.
__device__ __forceinline__ float route_weights(const double* __restrict__ s, const int (&ids)[TOPK], float* w_out) {
  const int lane = threadIdx.x & 63;
  double sv[TOPK], tot = 0.0;
#pragma unroll
  for (int r = 0; r < TOPK; ++r) {
    sv[r] = s[ids[r]];
    tot += sv[r];
  }
  float wv = 0.f;
  if (lane < TOPK) {
    double v = sv[0];
#pragma unroll
    for (int r = 1; r < TOPK; ++r)
      if (lane == r) v = sv[r];
    wv = (float)(v / tot);
    w_out[lane] = wv;
  }
  return wv;
}

// Top-6 of one token by one wavefront from its 256 scores: ids (decreasing c,
// ties to the lower index) and weights s_i / sum_T s.
__device__ __forceinline__ void route_token(const double* __restrict__ c, const double* __restrict__ s,
                                            int* ids_out, float* w_out) {
  int ids[TOPK];
  route_select(c, ids);
  write_ids(ids, ids_out);
  route_weights(s, ids, w_out);
}

// ----------------------------------------------------------------- gate / up
// Scales are passed as raw bf16 bits and widened where they are used: a
// conversion next to the load would make the wave wait for that load (and,
// the memory counter being in order, for every load issued before it).

// gate/up of one row for one token: returns h = silu(g) u (same in all lanes)
__device__ __forceinline__ float gateup_row_token(uint4 cg, uint32_t sg_bits, uint4 cu, uint32_t su_bits,
                                                  const uint4* a_tok, float asum_lane) {
  const int lane = threadIdx.x & 63;
  const uint4 av[4] = {a_tok[lane], a_tok[64 + lane], a_tok[128 + lane], a_tok[192 + lane]};
  const float g = wave_sum(lane_dot_gateup(cg, av, asum_lane, bf16_bits_to_f32(sg_bits)));
  const float u = wave_sum(lane_dot_gateup(cu, av, asum_lane, bf16_bits_to_f32(su_bits)));
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

// Codes and scale bits of lane `sub` of down row `row` of a [rows][K] int4 matrix.
__device__ __forceinline__ void load_down_lane(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                               int K, int row, int sub, uint4& c, uint32_t& sc) {
  c = reinterpret_cast<const uint4*>(codes + (size_t)row * (K / 2))[sub];
  sc = scales[(size_t)row * (K / G) + (sub >> 2)];
}

// This lane's down codes for output row `row` of one token:
//   pass A: lanes 16 s .. 16 s + 15 take routed slot s (s = 0..3)
//   pass B: lanes 0..31 take slots 4, 5; lanes 32..63 the shared expert.
__device__ __forceinline__ void load_down_row(const LayerW& L, const int* ids, int row, uint4& ca, uint32_t& sa,
                                              uint4& cb, uint32_t& sb) {
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
// + y_shared.  load_a() gives this lane's h chunk for pass A (slot lane / 16),
// load_b() for pass B (slot 4 + lane / 16 on lanes 0..31, the shared expert
// on 32..63); they are called one after the other so only one chunk is live.
// The result is the same in every lane.
template <typename LoadA, typename LoadB>
__device__ __forceinline__ float down_row_token(uint4 ca, uint32_t sa, uint4 cb, uint32_t sb, LoadA load_a,
                                                LoadB load_b, const float* w, float xres) {
  float ya, yb;
  {
    const HChunk ha = load_a();
    ya = row16_sum(lane_dot_down(ca, ha.v, ha.sum, bf16_bits_to_f32(sa)));
  }
  {
    const HChunk hb = load_b();
    yb = row16_sum(lane_dot_down(cb, hb.v, hb.sum, bf16_bits_to_f32(sb)));
  }
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

// Distinct experts among the picks ids[0..n)[0..TOPK), in increasing id order,
// into list[]; returns their number.  Threads 0..E-1 test one expert each.
__device__ __forceinline__ int distinct_experts(const int (*ids)[TOPK], int n, int* list, int* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int f = 0;
  if (tid < E)
    for (int i = 0; i < n * TOPK; ++i) f |= (ids[i / TOPK][i % TOPK] == tid);
  const unsigned long long bal = __ballot(f);
  if (lane == 0 && wave < E / 64) wave_tot[wave] = __popcll(bal);
  wg_sync();
  if (f) {
    int off = __popcll(bal & ((1ull << lane) - 1ull));
    for (int i = 0; i < wave; ++i) off += wave_tot[i];
    list[off] = tid;
  }
  int D = 0;
#pragma unroll
  for (int i = 0; i < E / 64; ++i) D += wave_tot[i];
  wg_sync();
  return D;
}

// Slot of expert e in a token's picks, or -1.
__device__ __forceinline__ int slot_of(const int* ids, int e) {
  int s = -1;
#pragma unroll
  for (int i = TOPK - 1; i >= 0; --i)
    if (ids[i] == e) s = i;
  return s;
}

}  // namespace flint
