// The dense SwiGLU MLP of layers 0 and 1 and the output head: int4 rows of
// K = 2048 against the bf16 block input (gate/up, head), and the dense down
// projection of K = inter against fp32 h.  HBM-bound matrix-vector products
// for up to 16 tokens; each token's arithmetic has a fixed shape, so results
// do not depend on the number of tokens in the call.
#include <algorithm>

#include "dense.h"
#include "decode_common.h"

namespace flint {

// ------------------------------------------------------------- K = 2048 rows
// Block inputs of the call's tokens, in the transposed pair order block_input
// writes (lane L reads uint4 j at j * 64 + L), and their lane-chunk sums.
struct DenseInput {
  uint32_t a[DENSE_MAX_TOKENS][H / 2];
  float asum[DENSE_MAX_TOKENS][64];
  double red[2][NWAVES];
};

// One workgroup (NT threads) normalises every token of the call.
__device__ __forceinline__ void dense_inputs(const float* __restrict__ x, int n, DenseInput& in) {
  float4 xv[DENSE_MAX_TOKENS];
#pragma unroll
  for (int t = 0; t < DENSE_MAX_TOKENS; ++t)
    if (t < n) xv[t] = reinterpret_cast<const float4*>(x + (size_t)t * H)[threadIdx.x];
#pragma unroll
  for (int t = 0; t < DENSE_MAX_TOKENS; ++t)
    if (t < n) block_input(xv[t], in.a[t], in.asum[t], in.red[t & 1]);
  wg_sync();
}

// The 8 nibbles of one code dword as bf16 pairs 128 + n' (n' = code + 8), in
// the pair order of the block input: (k0,k2), (k4,k6), (k1,k3), (k5,k7).
__device__ __forceinline__ void expand8(uint32_t code, uint32_t* p) {
  const uint32_t x = code ^ 0x88888888u;
  const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
  const uint32_t K43 = 0x43434343u;
  p[0] = __builtin_amdgcn_perm(K43, lo, 0x04010400u);
  p[1] = __builtin_amdgcn_perm(K43, lo, 0x04030402u);
  p[2] = __builtin_amdgcn_perm(K43, hi, 0x04010400u);
  p[3] = __builtin_amdgcn_perm(K43, hi, 0x04030402u);
}

typedef __bf16 dn_bf16x8 __attribute__((ext_vector_type(8)));
typedef float dn_f32x4 __attribute__((ext_vector_type(4)));

// D = A B + C for 16 x 32 (A) by 32 x 16 (B): lane l holds row l % 16 of A and
// column l % 16 of B, each for k = 8 (l / 16) .. + 7; D register r of lane l
// is row 4 (l / 16) + r, column l % 16.
__device__ __forceinline__ dn_f32x4 mfma16(uint4 a, uint4 b, dn_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(dn_bf16x8, a), __builtin_bit_cast(dn_bf16x8, b),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ uint4 expand8_u4(uint32_t code) {
  uint32_t p[4];
  expand8(code, p);
  return make_uint4(p[0], p[1], p[2], p[3]);
}

// The tokens' block inputs for the matrix cores: chunk c (8 bf16, pair order)
// of token t at at[c][t], zero for the tokens past n (16 consecutive 16-byte
// slots per chunk: one MFMA operand read has no bank conflicts).
struct DenseTokens {
  uint4 at[H / 8][DENSE_MAX_TOKENS];
};

// Rows of K = 2048 on the matrix cores, all tokens of the call at once (the M
// dimension of v_mfma_f32_16x16x32_bf16 is the 16 tokens, N is 16 weight
// rows).  Wave w of the grid takes 16-row blocks w, w + waves, ...  Lane l
// covers weight row l % 16 and, in each 128-element K-group, the 32 elements
// 32 (l / 16) .. + 31 (16 code bytes): MFMA step s takes their 8-element
// chunk s.  Each K-group is accumulated from zero as sum (code + 136) a and
// added times the row's scale; one more MFMA step subtracts
// 136 sum_g s[r][g] R[t][g], R the sum of a_t over group g split into three
// bf16 parts (exact products).  A block streams as two chunks of 8 K-groups,
// the next chunk in flight while one is used.
// SWIGLU: y[t][r] = silu(W0[r] . a_t) * (W1[r] . a_t), else y[t][r] = W0[r] . a_t.
template <bool SWIGLU>
__global__ void __launch_bounds__(NT, 2) k_rows_mfma(const float* __restrict__ x, int n,
                                                     const uint8_t* __restrict__ c0, const uint16_t* __restrict__ s0,
                                                     const uint8_t* __restrict__ c1, const uint16_t* __restrict__ s1,
                                                     int rows, float* __restrict__ y) {
  constexpr int NM = SWIGLU ? 2 : 1;     // matrices
  constexpr int CG = SWIGLU ? 4 : 8;     // K-groups per streamed chunk
  constexpr int NCH = 16 / CG;           // chunks per matrix of a block
  __shared__ DenseInput in;
  __shared__ DenseTokens tk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, col = lane & 15, q = lane >> 4;
  const int gw = blockIdx.x * NWAVES + wave, nw = gridDim.x * NWAVES;
  const int nblk = (rows + 15) >> 4;
  const int my_blocks = gw < nblk ? (nblk - 1 - gw) / nw + 1 : 0;
  const uint8_t* const C[2] = {c0, c1};
  const uint16_t* const S[2] = {s0, s1};
  // this lane's weight row in block j of the wave; blocks past the last re-read it
  auto row_of = [&](int j) {
    const int b = gw + min(j, max(my_blocks - 1, 0)) * nw;
    return (size_t)min(b * 16 + col, rows - 1);
  };
  // chunk k of a block: K-groups CG h .. CG h + CG - 1 (h = k % NCH) of matrix
  // k / NCH, and the row's scales of the 8 groups that hold them
  auto load = [&](int j, int k, uint4 (&c)[CG], uint4& sc) {
    const size_t r = row_of(j);
    const int m = k / NCH, h = k % NCH;
    const uint4* p = reinterpret_cast<const uint4*>(C[m] + r * (H / 2));
#pragma unroll
    for (int g = 0; g < CG; ++g) c[g] = p[(CG * h + g) * 4 + q];
    sc = reinterpret_cast<const uint4*>(S[m] + r * (H / G))[(CG * h) >> 3];
  };
  dense_inputs(x, n, in);
  uint4 ca[CG], cb[CG], sa, sb;
  load(0, 0, ca, sa);
  load(0, 1, cb, sb);
  // transpose the block inputs to at[c][t] (zeros past n)
  for (int i = threadIdx.x; i < (H / 8) * DENSE_MAX_TOKENS; i += NT) {
    const int c = i >> 4, t = i & 15;
    tk.at[c][t] = t < n ? reinterpret_cast<const uint4*>(in.a[t])[(c & 3) * 64 + (c >> 2)] : make_uint4(0u, 0u, 0u, 0u);
  }
  wg_sync();   // the only other barrier; every wave gets here
  // R[t][g] of this lane's token t = l % 16 and groups 8 q + i (q < 2), in three bf16 parts
  uint4 rp[3];
  {
    uint32_t w3[3][4] = {};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = 8 * q + i;
      float v = 0.f;
      if (q < 2 && col < n)
        v = ((in.asum[col][4 * g] + in.asum[col][4 * g + 1]) + in.asum[col][4 * g + 2]) + in.asum[col][4 * g + 3];
      const uint32_t b0 = f32_to_bf16_rne(v);
      const float r1 = v - bf16_bits_to_f32(b0);
      const uint32_t b1 = f32_to_bf16_rne(r1);
      const uint32_t b2 = f32_to_bf16_rne(r1 - bf16_bits_to_f32(b1));
      const int sh = 16 * (i & 1);
      w3[0][i >> 1] |= b0 << sh;
      w3[1][i >> 1] |= b1 << sh;
      w3[2][i >> 1] |= b2 << sh;
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) rp[k] = make_uint4(w3[k][0], w3[k][1], w3[k][2], w3[k][3]);
  }
  auto chunk = [&](int h, const uint4 (&c)[CG], const uint4& sc, dn_f32x4& acc) {
#pragma unroll
    for (int g = 0; g < CG; ++g) {
      const int gg = CG * h + g;   // K-group
      uint4 a[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) a[st] = tk.at[gg * 16 + 4 * q + st][col];
      const uint32_t cw[4] = {c[g].x, c[g].y, c[g].z, c[g].w};
      dn_f32x4 temp = mfma16(a[0], expand8_u4(cw[0]), dn_f32x4{});
#pragma unroll
      for (int st = 1; st < 4; ++st) temp = mfma16(a[st], expand8_u4(cw[st]), temp);
      const uint32_t sw[4] = {sc.x, sc.y, sc.z, sc.w};
      const int gi = gg & 7;
      const float sg = bf16_bits_to_f32((gi & 1) ? (sw[gi >> 1] >> 16) : (sw[gi >> 1] & 0xFFFFu));
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = gg == 0 ? sg * temp[r] : fmaf(sg, temp[r], acc[r]);
      __builtin_amdgcn_sched_barrier(0);   // one K-group at a time: bounded register use
    }
  };
  // NM x NCH chunks per block through two buffers; the chunk two ahead
  // (possibly of the next block) is requested as soon as a buffer is free
  constexpr int NK = NM * NCH;
  for (int j = 0; j < my_blocks; ++j) {
    dn_f32x4 acc[NM];
    uint4 shalf[NM][2];   // scales of groups 0..7 and 8..15, for the correction
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      uint4(&c)[CG] = (k & 1) ? cb : ca;
      uint4& sc = (k & 1) ? sb : sa;
      chunk(k % NCH, c, sc, acc[k / NCH]);
      shalf[k / NCH][(CG * (k % NCH)) >> 3] = sc;
      const int kn = k + 2;
      load(kn < NK ? j : j + 1, kn % NK, c, sc);
    }
    float v[NM][4];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint4 bs = q == 0 ? shalf[m][0] : q == 1 ? shalf[m][1] : make_uint4(0u, 0u, 0u, 0u);
      dn_f32x4 corr = mfma16(rp[0], bs, dn_f32x4{});
      corr = mfma16(rp[1], bs, corr);
      corr = mfma16(rp[2], bs, corr);
#pragma unroll
      for (int r = 0; r < 4; ++r) v[m][r] = fmaf(-136.f, corr[r], acc[m][r]);
    }
    const int row = (gw + j * nw) * 16 + col;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 4 * q + r;
      if (t < n && row < rows) y[(size_t)t * rows + row] = SWIGLU ? silu_mul(v[0][r], v[NM - 1][r]) : v[0][r];
    }
  }
}

// ------------------------------------------------------------- dense MLP
// Both products of the dense MLP run on the matrix cores with the call's
// tokens as the M dimension of v_mfma_f32_16x16x32_bf16 (zeros past n) and 16
// weight rows as N, so a token's arithmetic never depends on the other tokens.
// The codes become bf16 16 + n' = code + 24 (n' = code + 8 in [0, 15]: low
// byte 0x80 | n' << 3 under the high byte 0x41), in the pair order of the
// activations; each K-group's products sum (code + 24) v over its 128 elements
// exactly, are scaled by the row's scale, and 24 s R is removed, R the group's
// sum of v.  (The smaller offset of 24, against 136 in the head, keeps the
// cancellation at the down projection's 6,144-element rows small.)
__device__ __forceinline__ uint4 expand8_o24(uint32_t code) {
  const uint32_t x = code ^ 0x88888888u;
  const uint32_t lo = ((x & 0x0F0F0F0Fu) << 3) | 0x80808080u;   // bytes: k0, k2, k4, k6
  const uint32_t hi = ((x >> 1) & 0x78787878u) | 0x80808080u;   // bytes: k1, k3, k5, k7
  const uint32_t K41 = 0x41414141u;
  return make_uint4(__builtin_amdgcn_perm(K41, lo, 0x04010400u), __builtin_amdgcn_perm(K41, lo, 0x04030402u),
                    __builtin_amdgcn_perm(K41, hi, 0x04010400u), __builtin_amdgcn_perm(K41, hi, 0x04030402u));
}

// Pair order of 8 bf16 values v0..v7: (v0,v2), (v4,v6), (v1,v3), (v5,v7).
__device__ __forceinline__ uint4 pack_pair_order(const uint32_t (&b)[8]) {
  return make_uint4(b[0] | (b[2] << 16), b[4] | (b[6] << 16), b[1] | (b[3] << 16), b[5] | (b[7] << 16));
}

// Block input of token t by one wave.  Lane L holds the 8-element chunks
// L + 64 j (j < 4), elements 8 (L + 64 j) .. + 7, as float4s 2 j and 2 j + 1
// of xv (xt is the token's row, re-read on the rare exact path).  RMSNorm in
// fp64 (exact squares, a per-lane sum in order, then the fixed wave tree), one
// rounding to bf16.  Writes the chunks as MFMA operands at[t][c] (consecutive
// lanes on consecutive 16-byte slots) and, per K-group g (chunks 16 g .. 16 g
// + 15: lanes 16 (g % 4) .. + 15 of chunk set j = g / 4), the sum of its 128
// bf16 values to R[t][g].
constexpr int DG_ROW = H / 8 + 1;   // LDS row of one token's chunks, padded so rows start on other banks

__device__ __forceinline__ void wave_block_input_store(const uint32_t (&b)[32], int t, uint4 (*at)[DG_ROW],
                                                       float (*R)[H / G]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t cb[8];
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      cb[e] = b[8 * j + e];
      part += bf16_bits_to_f32(cb[e]);
    }
    at[t][lane + 64 * j] = pack_pair_order(cb);
    part = row16_sum(part);
    if ((lane & 15) == 0) R[t][4 * j + (lane >> 4)] = part;
  }
}

// Where some fp32 quotient lands on a bf16 midpoint: every value of the lane
// from the correctly rounded quotient near midpoints (rare; kept out of line
// so that the common path keeps few registers).
__device__ __noinline__ void wave_block_input_exact(const float* __restrict__ xt, double ms, double rinv, int t,
                                                    uint4 (*at)[DG_ROW], float (*R)[H / G]) {
  const int lane = threadIdx.x & 63;
  uint32_t b[32];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double v = xt[8 * (lane + 64 * j) + e];
      double q = v * rinv;
      if (near_bf16_midpoint(q)) q = v / sqrt(ms);
      b[8 * j + e] = f64_to_bf16_rne(q);
    }
  wave_block_input_store(b, t, at, R);
}

__device__ __forceinline__ void load_x_chunks(const float* __restrict__ xt, float4 (&xv)[8]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    xv[2 * j] = reinterpret_cast<const float4*>(xt)[2 * (lane + 64 * j)];
    xv[2 * j + 1] = reinterpret_cast<const float4*>(xt)[2 * (lane + 64 * j) + 1];
  }
}

__device__ __forceinline__ void wave_block_input(const float4 (&xv)[8], const float* __restrict__ xt, int t,
                                                 uint4 (*at)[DG_ROW], float (*R)[H / G]) {
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const double v[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = fma(v[e], v[e], ss);
  }
  ss = wave_sum(ss);
  const double ms = ss / (double)H + RMS_EPS;
  const double rinv = rsqrt(ms);
  uint32_t b[32];
  bool hard = false;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float v[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float qf = (float)((double)v[e] * rinv);
      hard |= f32_on_bf16_midpoint(qf);
      b[4 * j + e] = f32_to_bf16_rne(qf);
    }
  }
  if (__builtin_expect(__ballot(hard) != 0ull, 0))   // wave-uniform
    wave_block_input_exact(xt, ms, rinv, t, at, R);
  else
    wave_block_input_store(b, t, at, R);
}

// Gate/up: h[t][r] = silu(Wg[r] . a_t) * (Wu[r] . a_t).  Workgroup b owns rows
// rpw b .. rpw b + rpw - 1 (rpw <= 16 rows: inter / 512, so that the grid is
// two workgroups per CU); wave w takes K-groups 2 w and 2 w + 1 of both
// matrices (lane l: row min(l % 16, rpw - 1), the 32 elements 32 (l / 16) .. + 31
// of each group; the MFMA columns past rpw repeat the last row and are not stored).
// Its codes are requested before the block inputs are formed (wave w forms
// tokens w and w + 8); the 8 waves' partial sums are added in wave order.
struct DenseGateUpLds {
  union {
    uint4 at[DENSE_MAX_TOKENS][DG_ROW];  // block inputs: chunk c of token t
    float4 red[NWAVES][2][64];           // partial results of each wave (gate, up)
  };
  float R[DENSE_MAX_TOKENS][H / G];
};

__global__ void __launch_bounds__(NT, 4) k_dense_gateup(const float* __restrict__ x, int n,
                                                        const uint8_t* __restrict__ gate,
                                                        const uint16_t* __restrict__ gate_s,
                                                        const uint8_t* __restrict__ up,
                                                        const uint16_t* __restrict__ up_s, int rows, int rpw,
                                                        float* __restrict__ h) {
  __shared__ DenseGateUpLds L;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 15, q = lane >> 4;
  const size_t row = (size_t)blockIdx.x * rpw + min(col, rpw - 1);
  // this wave's first token (w, or n - 1 when w >= n) before the codes: the
  // norm then waits for its own loads only (loads complete in issue order)
  float4 xv[8];
  load_x_chunks(x + (size_t)min(w, n - 1) * H, xv);
  uint4 cg[2], cu[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    cg[i] = reinterpret_cast<const uint4*>(gate + row * (H / 2))[(2 * w + i) * 4 + q];
    cu[i] = reinterpret_cast<const uint4*>(up + row * (H / 2))[(2 * w + i) * 4 + q];
  }
  const uint32_t sg = reinterpret_cast<const uint32_t*>(gate_s + row * (H / G))[w];   // groups 2w, 2w+1
  const uint32_t su = reinterpret_cast<const uint32_t*>(up_s + row * (H / G))[w];
  if (w < n) {   // wave-uniform
    wave_block_input(xv, x + (size_t)w * H, w, L.at, L.R);
  } else {
    // a use on this path too, so the loads above stay ahead of the codes'
    // instead of moving into the branch that normalises
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(xv[j].x), "v"(xv[j].y), "v"(xv[j].z), "v"(xv[j].w));
  }
  if (w + 8 < n) {   // wave-uniform
    load_x_chunks(x + (size_t)(w + 8) * H, xv);
    wave_block_input(xv, x + (size_t)(w + 8) * H, w + 8, L.at, L.R);
  }
  wg_sync();
  // operands first (reads are unconditional; lanes of tokens past n take zeros)
  const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
  uint4 a[2][4];
  float Rg[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint4 v = L.at[col][16 * (2 * w + i) + 4 * q + st];
      a[i][st] = col < n ? v : zero4;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = L.R[4 * q + r][2 * w + i];
      Rg[i][r] = 4 * q + r < n ? v : 0.f;
    }
  }
  // four independent accumulation chains: (group, matrix)
  dn_f32x4 tg[2], tu[2];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t wg = st == 0 ? cg[i].x : st == 1 ? cg[i].y : st == 2 ? cg[i].z : cg[i].w;
      const uint32_t wu = st == 0 ? cu[i].x : st == 1 ? cu[i].y : st == 2 ? cu[i].z : cu[i].w;
      tg[i] = mfma16(a[i][st], expand8_o24(wg), st == 0 ? dn_f32x4{} : tg[i]);
      tu[i] = mfma16(a[i][st], expand8_o24(wu), st == 0 ? dn_f32x4{} : tu[i]);
    }
  }
  dn_f32x4 acc[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint32_t s2 = m ? su : sg;
    const float s0 = bf16_bits_to_f32(s2 & 0xFFFFu), s1 = bf16_bits_to_f32(s2 >> 16);
    const dn_f32x4& t0 = m ? tu[0] : tg[0];
    const dn_f32x4& t1 = m ? tu[1] : tg[1];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      acc[m][r] = fmaf(s0, t0[r], -24.f * s0 * Rg[0][r]) + fmaf(s1, t1[r], -24.f * s1 * Rg[1][r]);
  }
  wg_sync();   // every wave is done with the block inputs
#pragma unroll
  for (int m = 0; m < 2; ++m) L.red[w][m][lane] = make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
  wg_sync();
  if (threadIdx.x < 256) {
    const int c = threadIdx.x & 15, t = threadIdx.x >> 4;
    if (t < n && c < rpw) {
      const int l = 16 * (t >> 2) + c, r = t & 3;
      float gsum = 0.f, usum = 0.f;
#pragma unroll
      for (int v = 0; v < NWAVES; ++v) {
        gsum += reinterpret_cast<const float*>(&L.red[v][0][l])[r];
        usum += reinterpret_cast<const float*>(&L.red[v][1][l])[r];
      }
      h[(size_t)t * rows + (size_t)blockIdx.x * rpw + c] = silu_mul(gsum, usum);
    }
  }
}

// Down: out[t][c] = x[t][c] + Wd[c] . h_t, K = inter = 128 NG.  Workgroup b
// owns rows 8 b .. 8 b + 7 (256 workgroups, one per CU; the MFMA's columns
// 8 .. 15 repeat rows 0 .. 7 and are not stored); wave w takes the K-groups w, w + 8, w + 16, ...
// in that order, whatever the call's size, so every token's arithmetic is the
// same for any n.  h is fp32: the workgroup splits the h values of the call's
// tokens into three bf16 parts (v = p0 + p1 + p2 exactly: each part takes the
// next 8 significant bits) and stages them in LDS, a slice of 8 GW K-groups at
// a time (GW groups per wave; fewer, larger slices when fewer tokens need
// room); the 16 threads that stage one group of one token also form its sum R
// with a row tree.  In the MFMA each token takes four rows of A (its three
// parts and a zero row), so one instruction serves four tokens and a token's
// three part sums come out in one lane, where they are added in part order;
// the 8 waves' partial sums are added in wave order.  Thread i
// stages the (token, chunk) pairs i + 512 m, tokens 0 .. 4 NI - 1 (NI =
// ceil(n / 4)), and requests the h of DEPTH slices ahead; its loads are
// unconditional (tokens past n re-read token n - 1), so each wait counts
// exactly the loads issued after the ones it needs.
constexpr int dd_gw(int ng, int ni) {   // K-groups per wave per slice
  const int cand[5] = {6, 4, 3, 2, 1};
  for (int g : cand)
    if (ng % (8 * g) == 0 && 3 * (4 * ni) * (128 * g + 1) * 16 <= 100 * 1024) return g;
  return 1;
}

template <int TC, int CH>   // staged tokens, 8-element chunks per token per slice
struct DenseDownLds {
  union {
    uint4 hp[3][TC][CH + 1];   // chunk c of token t, part p (rows padded onto other banks)
    float red[NWAVES][TC / 4][64];
  };
  float R[TC][CH / 16];         // per K-group of the slice: sum of the token's h
};

constexpr int DD_RPW = 8;   // output rows per down workgroup
template <int NG, int NI>   // K-groups (inter / 128); (token, chunk) pairs per thread and group-slice column
__global__ void __launch_bounds__(NT, 1) k_dense_down(const float* __restrict__ h, int n,
                                                      const uint8_t* __restrict__ down,
                                                      const uint16_t* __restrict__ down_s, const float* x,
                                                      float* out) {
  constexpr int inter = NG * G;
  constexpr int GW = dd_gw(NG, NI);               // groups per wave per slice
  constexpr int NSL = NG / (8 * GW);              // slices
  constexpr int TC = 4 * NI;                      // tokens with room in LDS
  constexpr int CH = 128 * GW;                    // chunks per token per slice
  constexpr int IT = NI * GW;                     // (token, chunk) pairs per thread per slice
  constexpr int DEPTH = NSL < 16 / IT ? NSL : (16 / IT > 0 ? 16 / IT : 1);   // slices in flight
  static_assert(TC * CH == NT * IT, "pairs per slice");
  __shared__ DenseDownLds<TC, CH> L;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 15, q = lane >> 4;
  const size_t row = (size_t)blockIdx.x * DD_RPW + (col & (DD_RPW - 1));
  // codes and scale of this wave's K-groups w + 8 k, k < NG / 8
  constexpr int KW = NG / 8;
  uint4 code[KW];
  float sc[KW];
#pragma unroll
  for (int k = 0; k < KW; ++k) {
    const int g = 8 * k + w;
    code[k] = reinterpret_cast<const uint4*>(down + row * (inter / 2))[g * 4 + q];
    sc[k] = bf16_bits_to_f32(down_s[row * (inter / G) + g]);
  }
  float4 hv[DEPTH][IT][2];
  auto load_h = [&](int s, float4 (&buf)[IT][2]) {
#pragma unroll
    for (int m = 0; m < IT; ++m) {
      const int j = threadIdx.x + NT * m, t = min(j / CH, n - 1), c = j % CH;
      const float4* p = reinterpret_cast<const float4*>(h + (size_t)t * inter + (size_t)CH * 8 * s + 8 * c);
      buf[m][0] = p[0];
      buf[m][1] = p[1];
    }
  };
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) load_h(s, hv[s]);
  const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
  float acc[NI] = {};   // token 4 tg + q, column col
#pragma unroll
  for (int s = 0; s < NSL; ++s) {
    float4 (&buf)[IT][2] = hv[s % DEPTH];
#pragma unroll
    for (int m = 0; m < IT; ++m) {
      const int j = threadIdx.x + NT * m, t = j / CH, c = j % CH;
      float csum = 0.f;
      if (t < n) {
        const float e[8] = {buf[m][0].x, buf[m][0].y, buf[m][0].z, buf[m][0].w,
                            buf[m][1].x, buf[m][1].y, buf[m][1].z, buf[m][1].w};
        uint32_t b0[8], b1[8], b2[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          b0[k] = f32_to_bf16_rne(e[k]);
          const float r1 = e[k] - bf16_bits_to_f32(b0[k]);
          b1[k] = f32_to_bf16_rne(r1);
          b2[k] = f32_to_bf16_rne(r1 - bf16_bits_to_f32(b1[k]));
        }
        L.hp[0][t][c] = pack_pair_order(b0);
        L.hp[1][t][c] = pack_pair_order(b1);
        L.hp[2][t][c] = pack_pair_order(b2);
        csum = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      }
      csum = row16_sum(csum);   // the 16 threads of a row: one K-group of one token
      if ((c & 15) == 0 && t < n) L.R[t][c >> 4] = csum;
    }
    if (s + DEPTH < NSL) load_h(s + DEPTH, buf);
    wg_sync();
#pragma unroll
    for (int gi = 0; gi < GW; ++gi) {
      const int gl = 8 * gi + w;   // K-group of the slice
      const int k = s * GW + gi;   // this wave's k-th K-group: w + 8 k
      const uint32_t cw[4] = {code[k].x, code[k].y, code[k].z, code[k].w};
      uint4 bw[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) bw[st] = expand8_o24(cw[st]);
#pragma unroll
      for (int tg = 0; tg < NI; ++tg) {
        // rows of the MFMA's A: 4 per token (parts 0, 1, 2 and a zero row);
        // lane l holds row l % 16 = 4 (token % 4) + part
        const int t = 4 * tg + (col >> 2), part = col & 3;
        uint4 a[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const uint4 v = L.hp[part < 3 ? part : 0][t][16 * gl + 4 * q + st];
          a[st] = (t < n && part < 3) ? v : zero4;
        }
        dn_f32x4 d = mfma16(a[0], bw[0], dn_f32x4{});
#pragma unroll
        for (int st = 1; st < 4; ++st) d = mfma16(a[st], bw[st], d);
        // D rows 4 q + r: token 4 tg + q, part r
        const int tq = 4 * tg + q;
        const float Rt = tq < n ? L.R[tq][gl] : 0.f;
        acc[tg] += fmaf(sc[k], (d[0] + d[1]) + d[2], -24.f * sc[k] * Rt);
      }
    }
    wg_sync();   // the next slice's staging (or the partial sums) must not overtake these reads
  }
  float xo = 0.f;
  const int oc = threadIdx.x & 15, ot = threadIdx.x >> 4;
  const bool writer = threadIdx.x < 256 && ot < n && oc < DD_RPW;
  const size_t o = (size_t)ot * H + (size_t)blockIdx.x * DD_RPW + oc;
  if (writer) xo = x[o];
#pragma unroll
  for (int tg = 0; tg < NI; ++tg) L.red[w][tg][lane] = acc[tg];
  wg_sync();
  if (writer) {
    const int tg = ot >> 2, l = 16 * (ot & 3) + oc;
    float y = 0.f;
#pragma unroll
    for (int v = 0; v < NWAVES; ++v) y += L.red[v][tg][l];
    out[o] = xo + y;
  }
}

template <int NG>
static void launch_dense_down(int n, const float* h, const uint8_t* down, const uint16_t* down_s, const float* x,
                              float* out, hipStream_t s) {
  const dim3 grid(H / DD_RPW), block(NT);
  switch ((n + 3) / 4) {
    case 1: hipLaunchKernelGGL((k_dense_down<NG, 1>), grid, block, 0, s, h, n, down, down_s, x, out); break;
    case 2: hipLaunchKernelGGL((k_dense_down<NG, 2>), grid, block, 0, s, h, n, down, down_s, x, out); break;
    case 3: hipLaunchKernelGGL((k_dense_down<NG, 3>), grid, block, 0, s, h, n, down, down_s, x, out); break;
    default: hipLaunchKernelGGL((k_dense_down<NG, 4>), grid, block, 0, s, h, n, down, down_s, x, out); break;
  }
}

// ------------------------------------------------------------- host side
constexpr int DN_GRID = 256;   // one workgroup per CU (132 KB of LDS)

hipError_t launch_dense_mlp(const uint8_t* gate, const uint16_t* gate_s, const uint8_t* up, const uint16_t* up_s,
                            const uint8_t* down, const uint16_t* down_s, int inter, const float* x, int n, float* h,
                            float* out, hipStream_t s) {
  if (n < 1 || n > DENSE_MAX_TOKENS || inter < 2048 || inter > FLINT_DENSE_MLP_SIZE || inter % 2048)
    return hipErrorInvalidValue;
  const int rpw = inter / 512;   // 4, 8 or 12 rows: 512 workgroups, two per CU
  hipLaunchKernelGGL(k_dense_gateup, dim3(inter / rpw), dim3(NT), 0, s, x, n, gate, gate_s, up, up_s, inter, rpw, h);
  if (inter == 2048)
    launch_dense_down<16>(n, h, down, down_s, x, out, s);
  else if (inter == 4096)
    launch_dense_down<32>(n, h, down, down_s, x, out, s);
  else
    launch_dense_down<48>(n, h, down, down_s, x, out, s);
  return hipGetLastError();
}

hipError_t launch_head(const uint8_t* codes, const uint16_t* scales, int rows, const float* x, int n, float* logits,
                       hipStream_t s) {
  if (n < 1 || n > DENSE_MAX_TOKENS || rows < 1) return hipErrorInvalidValue;
  const int grid = std::min(DN_GRID, ((rows + 15) / 16 + NWAVES - 1) / NWAVES);
  hipLaunchKernelGGL(k_rows_mfma<false>, dim3(grid), dim3(NT), 0, s, x, n, codes, scales, codes, scales, rows,
                     logits);
  return hipGetLastError();
}

}  // namespace flint
