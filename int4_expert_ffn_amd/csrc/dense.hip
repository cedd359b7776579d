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

// Lane part of one K = 2048 row for one token from expanded codes: the 32
// products summed in fp32 in a fixed order, minus 136 * (sum of the lane's
// activations), times the row's scale.
__device__ __forceinline__ float lane_dot_expanded(const uint32_t (&p)[16], const uint4 (&a)[4], float asum,
                                                   float scale) {
  float acc = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t av[4] = {a[d].x, a[d].y, a[d].z, a[d].w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p[4 * d + q]),
                                            __builtin_bit_cast(bf16x2_t, av[q]), acc, false);
  }
  return fmaf(-136.f, asum, acc) * scale;
}

// Wave w of the grid takes rows w, w + waves, ...; U rows per batch and three
// batches in a ring, two in flight while one is used (loads are never
// conditional, so waiting for one batch never waits for a younger one: rows
// past the wave's last one re-read it).  The first two batches are requested
// before the block inputs are computed.  Each row's codes are expanded once
// and used for every token.
// SWIGLU: y[t][r] = silu(W0[r] . a_t) * (W1[r] . a_t), else y[t][r] = W0[r] . a_t.
template <bool SWIGLU, int U>
__global__ void __launch_bounds__(NT, 2) k_rows_k2048(const float* __restrict__ x, int n,
                                                      const uint8_t* __restrict__ c0, const uint16_t* __restrict__ s0,
                                                      const uint8_t* __restrict__ c1, const uint16_t* __restrict__ s1,
                                                      int rows, float* __restrict__ y) {
  __shared__ DenseInput in;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gw = blockIdx.x * NWAVES + wave, nw = gridDim.x * NWAVES;
  const int my_rows = gw < rows ? (rows - 1 - gw) / nw + 1 : 1;   // waves past the last row re-read row 0..
  const int nb = gw < rows ? (my_rows + U - 1) / U : 0;
  auto row_of = [&](int j) { return (size_t)min(gw, rows - 1) + (size_t)min(j, my_rows - 1) * nw; };
  auto load = [&](int b, uint4 (&c)[U], uint32_t (&sc)[U], uint4 (&cu)[U], uint32_t (&su)[U]) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const size_t r = row_of(b * U + i);
      c[i] = reinterpret_cast<const uint4*>(c0 + r * (H / 2))[lane];
      sc[i] = s0[r * (H / G) + (lane >> 2)];
      if (SWIGLU) {
        cu[i] = reinterpret_cast<const uint4*>(c1 + r * (H / 2))[lane];
        su[i] = s1[r * (H / G) + (lane >> 2)];
      }
    }
  };
  auto compute = [&](int b, const uint4 (&c)[U], const uint32_t (&sc)[U], const uint4 (&cu)[U],
                     const uint32_t (&su)[U]) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int j = b * U + i;
      if (j >= my_rows) break;   // wave-uniform
      const size_t r = row_of(j);
      uint32_t pg[16], pu[16];
      expand8(c[i].x, pg);
      expand8(c[i].y, pg + 4);
      expand8(c[i].z, pg + 8);
      expand8(c[i].w, pg + 12);
      if (SWIGLU) {
        expand8(cu[i].x, pu);
        expand8(cu[i].y, pu + 4);
        expand8(cu[i].z, pu + 8);
        expand8(cu[i].w, pu + 12);
      }
      const float sg = bf16_bits_to_f32(sc[i]), su_f = SWIGLU ? bf16_bits_to_f32(su[i]) : 0.f;
      for (int t = 0; t < n; ++t) {
        const uint4* at = reinterpret_cast<const uint4*>(in.a[t]);
        const uint4 av[4] = {at[lane], at[64 + lane], at[128 + lane], at[192 + lane]};
        const float asum = in.asum[t][lane];
        float v = wave_sum(lane_dot_expanded(pg, av, asum, sg));
        if (SWIGLU) v = silu_mul(v, wave_sum(lane_dot_expanded(pu, av, asum, su_f)));
        if (lane == 0) y[(size_t)t * rows + r] = v;
      }
    }
  };
  uint4 ca[U], cb[U], cc[U], ua[U], ub[U], uc[U];
  uint32_t sa[U], sb[U], sc_[U], ta[U], tb[U], tc[U];
  load(0, ca, sa, ua, ta);
  load(1, cb, sb, ub, tb);
  dense_inputs(x, n, in);   // the only barrier; every wave gets here
  for (int b = 0; b < nb; b += 3) {
    load(b + 2, cc, sc_, uc, tc);
    compute(b, ca, sa, ua, ta);
    load(b + 3, ca, sa, ua, ta);
    compute(b + 1, cb, sb, ub, tb);
    load(b + 4, cb, sb, ub, tb);
    compute(b + 2, cc, sc_, uc, tc);
  }
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
// The head runs here; the dense MLP's gate/up run in k_rows_k2048 (6,144 rows
// make only 384 blocks of 16, too few to fill the chip).
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

// ------------------------------------------------------------- dense down
// out[t][c] = x[t][c] + Wd[c] . h_t, K = inter = P x 2048.  Wave w of
// workgroup b owns rows 16 b + 4 w .. + 3; lane L covers k = 2048 p + 32 L ..
// + 31 of pass p.  h of up to DD_TC tokens is staged in LDS, float4 j of lane
// chunk (p, L) at (8 p + j) * 64 + L, with the chunk sums beside it.
constexpr int DD_TC = 4;
constexpr int DD_ROWS = 2;                    // rows per wave
constexpr int DD_NT = 256;
constexpr int DD_PMAX = FLINT_DENSE_MLP_SIZE / 2048;
constexpr int DD_GRID = H / (DD_ROWS * DD_NT / 64);

__global__ void __launch_bounds__(DD_NT) k_dense_down(const float* __restrict__ h, int n, int inter,
                                                      const uint8_t* __restrict__ dc, const uint16_t* __restrict__ ds,
                                                      const float* x, float* out) {
  __shared__ float4 hb[DD_TC][FLINT_DENSE_MLP_SIZE / 4];
  __shared__ float hsum[DD_TC][DD_PMAX * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int P = inter / 2048, q4 = inter / 4;
  const int r0 = (blockIdx.x * (DD_NT / 64) + wave) * DD_ROWS;
  uint4 code[DD_ROWS][DD_PMAX];
  uint32_t sc[DD_ROWS][DD_PMAX];
#pragma unroll
  for (int i = 0; i < DD_ROWS; ++i)
#pragma unroll
    for (int p = 0; p < DD_PMAX; ++p) {
      const int pp = p < P ? p : 0;
      code[i][p] = reinterpret_cast<const uint4*>(dc + (size_t)(r0 + i) * (inter / 2))[pp * 64 + lane];
      sc[i][p] = ds[(size_t)(r0 + i) * (inter / G) + pp * 16 + (lane >> 2)];
    }
  for (int t0 = 0; t0 < n; t0 += DD_TC) {
    const int tc = min(DD_TC, n - t0);
    wg_sync();   // the previous chunk's readers are done
    for (int i = threadIdx.x; i < tc * q4; i += DD_NT) {
      const int tt = i / q4, q = i - tt * q4;   // float4 q of token tt: k = 4 q
      const int p = q >> 9, L = (q >> 3) & 63, j = q & 7;
      hb[tt][(p * 8 + j) * 64 + L] = reinterpret_cast<const float4*>(h + (size_t)(t0 + tt) * inter)[q];
    }
    wg_sync();
    for (int i = threadIdx.x; i < tc * P * 64; i += DD_NT) {
      const int tt = i / (P * 64), pl = i - tt * (P * 64), p = pl >> 6, L = pl & 63;
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 v = hb[tt][(p * 8 + j) * 64 + L];
        s += ((v.x + v.y) + v.z) + v.w;
      }
      hsum[tt][pl] = s;
    }
    wg_sync();
    for (int tt = 0; tt < tc; ++tt) {
      // keep the codes' conversions inside the token loop (hoisted, the
      // converted values of all rows and passes would not fit in registers)
#pragma unroll
      for (int i = 0; i < DD_ROWS; ++i)
#pragma unroll
        for (int p = 0; p < DD_PMAX; ++p)
          asm volatile("" : "+v"(code[i][p].x), "+v"(code[i][p].y), "+v"(code[i][p].z), "+v"(code[i][p].w));
      float acc[DD_ROWS] = {};
#pragma unroll
      for (int p = 0; p < DD_PMAX; ++p) {
        if (p < P) {
          float4 h4[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) h4[j] = hb[tt][(p * 8 + j) * 64 + lane];
          const float hs = hsum[tt][p * 64 + lane];
#pragma unroll
          for (int i = 0; i < DD_ROWS; ++i) acc[i] += lane_dot_down(code[i][p], h4, hs, bf16_bits_to_f32(sc[i][p]));
        }
      }
#pragma unroll
      for (int i = 0; i < DD_ROWS; ++i) {
        const float v = wave_sum(acc[i]);
        if (lane == 0) {
          const size_t o = (size_t)(t0 + tt) * H + r0 + i;
          out[o] = x[o] + v;
        }
      }
    }
  }
}

// ------------------------------------------------------------- host side
constexpr int DN_GRID = 256;   // one workgroup per CU (132 KB of LDS)

hipError_t launch_dense_mlp(const uint8_t* gate, const uint16_t* gate_s, const uint8_t* up, const uint16_t* up_s,
                            const uint8_t* down, const uint16_t* down_s, int inter, const float* x, int n, float* h,
                            float* out, hipStream_t s) {
  if (n < 1 || n > DENSE_MAX_TOKENS || inter < 2048 || inter > FLINT_DENSE_MLP_SIZE || inter % 2048)
    return hipErrorInvalidValue;
  const int grid = std::min(DN_GRID, (inter + NWAVES - 1) / NWAVES);
  hipLaunchKernelGGL((k_rows_k2048<true, 4>), dim3(grid), dim3(NT), 0, s, x, n, gate, gate_s, up, up_s, inter, h);
  hipLaunchKernelGGL(k_dense_down, dim3(DD_GRID), dim3(DD_NT), 0, s, h, n, inter, down, down_s, x, out);
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
