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

// ------------------------------------------------------------- dense down
// out[t][c] = x[t][c] + Wd[c] . h_t, K = inter = P x 2048.  Wave w of
// workgroup b owns rows 16 b + 4 w .. + 3; lane L covers k = 2048 p + 32 L ..
// + 31 of pass p.  h of up to DD_TC tokens is staged in LDS, float4 j of lane
// chunk (p, L) at (8 p + j) * 64 + L, with the chunk sums beside it.
constexpr int DD_TC = 4;
constexpr int DD_ROWS = 4;                    // rows per wave
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
constexpr int DN_GRID = 256;   // one workgroup per CU: 8 waves, 16 rows in flight each

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
  const int grid = std::min(DN_GRID, (rows + NWAVES - 1) / NWAVES);
  hipLaunchKernelGGL((k_rows_k2048<false, 4>), dim3(grid), dim3(NT), 0, s, x, n, codes, scales, codes, scales, rows,
                     logits);
  return hipGetLastError();
}

}  // namespace flint
