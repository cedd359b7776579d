// Prefill path: a block of n tokens (DECODE_MAX_TOKENS < n <= FLINT_MAX_TOKENS)
// through one layer, where the block becomes a dense contraction: ~48 tokens
// per expert on average at n = 2048, so each expert's weights are read once
// per 64-token tile and multiplied on the matrix cores.
//
//   k_pf_input    block input a = bf16(rmsnorm(x)) per token (the decode's
//                 rounding rule), 8-element chunks in pair order
//   k_pf_router   z = a Wr^T, bf16 MFMA with fp32 accumulation
//   k_pf_route    per token (one wave): s = sigmoid(z), c = s + b in fp64,
//                 top-6 and weights; marks the token in each pick's bitmap
//   k_pf_offsets  per-expert counts, their exclusive scan, the 64-token tiles
//   k_pf_scatter  (token, slot) pairs in expert order, tokens increasing
//                 within an expert (popcounts of the bitmap prefix)
//   k_pf_gateup   routed gate/up + SwiGLU per tile (grouped GEMM)
//   k_pf_sh_gateup  shared gate/up + SwiGLU (dense GEMM)
//   k_pf_down     routed down projection per tile -> y by (token, slot)
//   k_pf_sh_down  shared down projection and the fixed-order combine
//                 out = x + ((w0 y0 + w1 y1) + ... + w5 y5) + y_shared
//
// Numerics: int4 codes enter the MFMA as bf16 128 + n' (n' = code + 8, exact)
// against bf16 activations, fp32 accumulation.  Each 128-element K-group is
// accumulated from zero, giving sum (code + 136) a, and added to the result
// times the row's scale; one last MFMA step subtracts 136 sum_g s_g R_g
// (R_g: sum of the activations over group g, split into three bf16 parts so
// that the products are exact).  The SwiGLU output h is kept as two bf16
// parts (hi + lo, about 16 significant bits) for the down projection.
// Nothing depends on the order of atomic operations, so results are
// deterministic.
#include <algorithm>

#include "prefill.h"
#include "decode_common.h"

namespace flint {

constexpr int PF_NT = 256;   // threads of the prefill kernels (4 waves)

typedef __bf16 pf_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pf_f32x16 __attribute__((ext_vector_type(16)));

// D = A B + C for 32 x 16 (A) by 16 x 32 (B).  Lane l holds row l % 32 of A
// and column l % 32 of B, each for k = 8 (l / 32) .. + 7; D register r of lane
// l is row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
__device__ __forceinline__ pf_f32x16 mfma_bf16(uint4 a, uint4 b, pf_f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(pf_bf16x8, a), __builtin_bit_cast(pf_bf16x8, b),
                                                 c, 0, 0, 0);
}

// 8 int4 codes of one dword (k0 in bits 0-3) -> bf16 128 + n' in pair order
// (k0, k2, k4, k6, k1, k3, k5, k7), n' = code + 8.
__device__ __forceinline__ uint4 expand_codes(uint32_t code) {
  const uint32_t x = code ^ 0x88888888u;
  const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
  const uint32_t K43 = 0x43434343u;
  return make_uint4(__builtin_amdgcn_perm(K43, lo, 0x04010400u), __builtin_amdgcn_perm(K43, lo, 0x04030402u),
                    __builtin_amdgcn_perm(K43, hi, 0x04010400u), __builtin_amdgcn_perm(K43, hi, 0x04030402u));
}

// 8 bf16 in natural order (4 dwords) -> pair order
__device__ __forceinline__ uint4 to_pair_order(uint4 v) {
  return make_uint4(__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.w, v.z, 0x05040100u),
                    __builtin_amdgcn_perm(v.y, v.x, 0x07060302u), __builtin_amdgcn_perm(v.w, v.z, 0x07060302u));
}

__device__ __forceinline__ float bf16x8_sum(uint4 v) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += bf16_bits_to_f32(d[i] & 0xFFFFu) + bf16_bits_to_f32(d[i] >> 16);
  return s;
}

// ------------------------------------------------------------- block input
__global__ void __launch_bounds__(PF_NT) k_pf_input(const float* __restrict__ x, int n, uint16_t* __restrict__ a,
                                                     uint32_t* __restrict__ bitmap) {
  __shared__ double red[PF_NT / 64];
  const int t = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = t * PF_NT + tid; i < E * PF_BW; i += gridDim.x * PF_NT) bitmap[i] = 0u;
  const float4* xr = reinterpret_cast<const float4*>(x + (size_t)t * H) + 2 * tid;
  const float4 v0 = xr[0], v1 = xr[1];
  const double xs[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += xs[j] * xs[j];
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  wg_sync();
  const double tot = ((red[0] + red[1]) + red[2]) + red[3];
  const double ms = tot / (double)H + RMS_EPS;
  const double rinv = rsqrt(ms);
  double q[8];
  float qf[8];
  bool hard = false;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    q[j] = xs[j] * rinv;
    qf[j] = (float)q[j];
    hard |= f32_on_bf16_midpoint(qf[j]);
  }
  uint32_t b[8];
  if (__builtin_expect(__ballot(hard) != 0ull, 0)) {   // wave-uniform, rare: the exact rule
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      double qq = q[j];
      if (near_bf16_midpoint(qq)) qq = xs[j] / sqrt(ms);
      b[j] = f64_to_bf16_rne(qq);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = f32_to_bf16_rne(qf[j]);
  }
  reinterpret_cast<uint4*>(a + (size_t)t * H)[tid] =
      make_uint4(b[0] | (b[2] << 16), b[4] | (b[6] << 16), b[1] | (b[3] << 16), b[5] | (b[7] << 16));
}

// ------------------------------------------------------------- router GEMM
// 32 tokens x 32 experts per workgroup.  Wave w sums K in [512 w, 512 w + 512)
// with two interleaved accumulators (short dependency chains), and the four
// partial sums are added in wave order.
__global__ void __launch_bounds__(PF_NT) k_pf_router(const uint16_t* __restrict__ a, int n,
                                                      const uint16_t* __restrict__ router, float* __restrict__ z) {
  __shared__ float part[3][16][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lrow = lane & 31, hl = lane >> 5;
  const int m0 = blockIdx.x * 32, e = blockIdx.y * 32 + lrow;
  const int m = min(m0 + lrow, n - 1);   // rows past n repeat the last token and are not stored
  const uint4* ar = reinterpret_cast<const uint4*>(a + (size_t)m * H) + wave * 64 + hl;
  const uint4* wr = reinterpret_cast<const uint4*>(router + (size_t)e * H) + wave * 64 + hl;
  pf_f32x16 acc0 = {}, acc1 = {};
#pragma unroll 4
  for (int j = 0; j < 32; j += 2) {   // MFMA step j: chunks 2 j (lanes 0..31) and 2 j + 1 (lanes 32..63)
    acc0 = mfma_bf16(ar[2 * j], to_pair_order(wr[2 * j]), acc0);
    acc1 = mfma_bf16(ar[2 * j + 2], to_pair_order(wr[2 * j + 2]), acc1);
  }
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) part[wave - 1][r][lane] = acc0[r] + acc1[r];
  }
  wg_sync();
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = (((acc0[r] + acc1[r]) + part[0][r][lane]) + part[1][r][lane]) + part[2][r][lane];
      const int mm = m0 + 8 * (r >> 2) + 4 * hl + (r & 3);
      if (mm < n) z[(size_t)mm * E + e] = v;
    }
  }
}

// ------------------------------------------------------------- routing
__global__ void __launch_bounds__(PF_NT) k_pf_route(const float* __restrict__ z, int n, const float* __restrict__ bias,
                                                     int* __restrict__ ids, float* __restrict__ w,
                                                     uint32_t* __restrict__ bitmap, int* trace_ids, float* trace_w) {
  __shared__ double cs[PF_NT / 64][2 * E];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * (PF_NT / 64) + wave;
  if (t >= n) return;   // the whole wave; nothing below waits for other waves
  double* c = cs[wave];
#pragma unroll
  for (int j = 0; j < E / 64; ++j) {
    const int e = lane + 64 * j;
    const double s = sigmoid_f64((double)z[(size_t)t * E + e]);
    double cv = s + (double)bias[e];
    if (cv != cv) cv = -INFINITY;
    c[e] = cv;
    c[E + e] = s;
  }
  route_token(c, c + E, ids + (size_t)t * TOPK, w + (size_t)t * TOPK);
  if (lane < TOPK) {
    const int id = ids[(size_t)t * TOPK + lane];   // written by this lane above
    atomicOr(&bitmap[id * PF_BW + (t >> 5)], 1u << (t & 31));
    if (trace_ids) {
      trace_ids[(size_t)t * TOPK + lane] = id;
      trace_w[(size_t)t * TOPK + lane] = w[(size_t)t * TOPK + lane];
    }
  }
}

// ------------------------------------------------------------- sort
// One workgroup, thread e = expert.  Besides the offsets, the 64-row tiles are
// listed grouped by XCD: experts are ranked by tile count (then index) and
// dealt to the 8 XCDs in snake order (0..7, 7..0, ...), so that all tiles of
// one expert run on one XCD, whose L2 then holds the expert's weights, and
// the XCDs get similar amounts of work.  Workgroup b of the GEMM kernels runs
// on XCD b % 8 (round-robin dispatch); only speed depends on that.
__device__ __forceinline__ int snake_rank(int x, int j) { return 16 * (j >> 1) + ((j & 1) ? 15 - x : x); }

constexpr int PF_NT_BINS = FLINT_MAX_TOKENS / PF_TM + 1;   // tile counts 0..32 of one expert

__global__ void __launch_bounds__(E) k_pf_offsets(const uint32_t* __restrict__ bitmap, int n, int* __restrict__ offsets,
                                                   int4* __restrict__ tiles, int* __restrict__ tile_start) {
  __shared__ int sc[2][E];
  __shared__ int nt_hist[PF_NT_BINS];
  __shared__ uint32_t nt_mask[PF_NT_BINS][E / 32];   // experts with a given tile count
  __shared__ int nt_by_rank[E], xcd_tiles[8];
  const int e = threadIdx.x;
  for (int i = e; i < PF_NT_BINS * (E / 32); i += E) (&nt_mask[0][0])[i] = 0u;
  if (e < PF_NT_BINS) nt_hist[e] = 0;
  // the bitmap is cleared in full for every layer, so all words are read
  const uint4* bm = reinterpret_cast<const uint4*>(bitmap + e * PF_BW);
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < PF_BW / 4; ++i) {
    const uint4 v = bm[i];
    cnt += __popc(v.x) + __popc(v.y) + __popc(v.z) + __popc(v.w);
  }
  const int nt = (cnt + PF_TM - 1) / PF_TM;
  wg_sync();
  atomicAdd(&nt_hist[nt], 1);
  atomicOr(&nt_mask[nt][e >> 5], 1u << (e & 31));
  int vc = cnt, b = 0;
  for (int d = 1; d < E; d <<= 1) {   // inclusive scan (fixed shape); its barriers also order the atomics
    sc[b][e] = vc;
    wg_sync();
    if (e >= d) vc += sc[b][e - d];
    b ^= 1;
  }
  const int oc = vc - cnt;
  offsets[e] = oc;
  if (e == E - 1) offsets[E] = vc;
  // rank: experts with more tiles first, equal counts by index
  int r = 0;
  for (int v = nt + 1; v < PF_NT_BINS; ++v) r += nt_hist[v];
  for (int w = 0; w < (e >> 5); ++w) r += __popc(nt_mask[nt][w]);
  r += __popc(nt_mask[nt][e >> 5] & ((1u << (e & 31)) - 1u));
  nt_by_rank[r] = nt;
  wg_sync();
  const int u = r & 15, x = u < 8 ? u : 15 - u, j = r >> 3;
  int before = 0;   // tiles of the experts dealt to XCD x ahead of this one
  for (int jj = 0; jj < j; ++jj) before += nt_by_rank[snake_rank(x, jj)];
  if (e < 8) {
    int tot = 0;
    for (int jj = 0; jj < E / 8; ++jj) tot += nt_by_rank[snake_rank(e, jj)];
    xcd_tiles[e] = tot;
  }
  wg_sync();
  int base = 0;
  for (int xx = 0; xx < x; ++xx) base += xcd_tiles[xx];
  if (e <= 8) {
    int s0 = 0;
    for (int xx = 0; xx < e; ++xx) s0 += xcd_tiles[xx];
    tile_start[e] = s0;
  }
  for (int i = 0; i < nt; ++i)
    tiles[base + before + i] = make_int4(e, oc + i * PF_TM, min(PF_TM, cnt - i * PF_TM), 0);
}

__global__ void __launch_bounds__(PF_NT) k_pf_scatter(const int* __restrict__ ids, int n,
                                                       const uint32_t* __restrict__ bitmap,
                                                       const int* __restrict__ offsets, int* __restrict__ perm) {
  const int p = blockIdx.x * PF_NT + threadIdx.x;
  if (p >= n * TOPK) return;
  const int t = p / TOPK, e = ids[p], wt = t >> 5;
  // the tokens before t in expert e's bitmap: whole words below word wt, all
  // requested at once (16-byte loads, none waits for another), then the low
  // bits of word wt
  const uint4* bm4 = reinterpret_cast<const uint4*>(bitmap + e * PF_BW);
  int pos = offsets[e];
#pragma unroll
  for (int i = 0; i < PF_BW / 4; ++i) {
    const uint4 v = bm4[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int word = 4 * i + j;
      pos += word < wt ? __popc(w[j]) : word == wt ? __popc(w[j] & ((1u << (t & 31)) - 1u)) : 0;
    }
  }
  perm[pos] = p;
}

// ------------------------------------------------------------- GEMM tile
// One workgroup computes 64 tile rows (rows of A given by rows_lds[m]; -1 is
// padding: computed from tile row 0, never stored) against NB x 32 weight rows
// per wave starting at wrow0, for NMAT weight matrices that share A.
// A: bf16 rows of lda elements in pair-order 8-element chunks, NSPLIT parts
// whose sum is the operand.  W: int4 codes [rows][KG x 64 bytes], S: bf16
// scales [rows][KG].  acc[mat][nb][mb] receives row block mb (tile rows
// 32 mb ..) for columns nb x 32 + lane % 32 of this wave's rows.
//
// Per K-group g the MFMAs accumulate sum_k (code_k + 136) a_k from zero, and
// that is added to acc times the scale s[n][g].  The remaining
// -136 sum_g s[n][g] R[m][g] (R: sums of A over each group) is one more MFMA
// step at the end, with R split into three bf16 parts so its products are
// exact.
// LDS: a_lds [2][NSPLIT][2][16][32] uint4 (chunk c of tile row r at row
// position r ^ (c & 14)), rsum_lds [64][KG] floats.
template <int NB, int NMAT, int KG, int NSPLIT>
__device__ __forceinline__ void gemm_tile(const uint16_t* const (&A)[NSPLIT], int lda, const int* rows_lds,
                                          const uint8_t* const (&W)[NMAT], const uint16_t* const (&S)[NMAT],
                                          int wrow0, pf_f32x16 (&acc)[NMAT][NB][2], uint4* a_lds, float* rsum_lds) {
  const int tid = threadIdx.x, lane = tid & 63, lrow = lane & 31, hl = lane >> 5;
  const int srow = tid >> 3, scp = tid & 7;   // staging: row, chunk pair
  constexpr int KB = KG * 64;                 // code bytes per weight row

  // codes and scale bits of this lane's weight rows for one K-group
  struct Codes {
    uint4 c[NMAT][NB][2];
    uint32_t s[NMAT][NB];
  };
  auto load_codes = [&](int g, Codes& d) {
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const size_t wr = (size_t)(wrow0 + nb * 32 + lrow);
        const uint4* p = reinterpret_cast<const uint4*>(W[mat] + wr * KB + g * 64 + hl * 32);
        d.c[mat][nb][0] = p[0];
        d.c[mat][nb][1] = p[1];
        d.s[mat][nb] = S[mat][wr * KG + g];
      }
  };
  // Loads are issued unconditionally so that the wave's memory counter can
  // wait for the A tile without waiting for the younger code loads: padding
  // rows read tile row 0, and the last group is re-read.
  uint4 stg[NSPLIT][2][2];
  auto stage_load = [&](int g) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int r = rows_lds[mb * 32 + srow];
      const int rr = r < 0 ? rows_lds[0] : r;
#pragma unroll
      for (int sp = 0; sp < NSPLIT; ++sp) {
        const uint4* p = reinterpret_cast<const uint4*>(A[sp] + (size_t)rr * lda + g * 128) + 2 * scp;
        stg[sp][mb][0] = p[0];
        stg[sp][mb][1] = p[1];
      }
    }
  };
  auto stage_store = [&](int buf, int g, bool sums) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float part = 0.f;
#pragma unroll
      for (int sp = 0; sp < NSPLIT; ++sp) {
        const uint4 v0 = stg[sp][mb][0], v1 = stg[sp][mb][1];
        uint4* d = a_lds + ((size_t)((buf * NSPLIT + sp) * 2 + mb) * 16) * 32;
        d[(2 * scp) * 32 + (srow ^ (2 * scp))] = v0;   // rows swizzled by chunk pair: the 16
        d[(2 * scp + 1) * 32 + (srow ^ (2 * scp))] = v1;   // lanes of one store cycle hit 16 bank groups
        part += bf16x8_sum(v0) + bf16x8_sum(v1);
      }
      part += dpp_f32<DPP_XOR1>(part);   // the 8 threads of one row
      part += dpp_f32<DPP_XOR2>(part);
      part += dpp_f32<DPP_HALF_MIRROR>(part);
      if (sums && scp == 0) rsum_lds[(mb * 32 + srow) * KG + g] = part;
    }
  };

  // One K-group: codes of group g in `cur`; the codes of group g + 2 are
  // loaded into `nxt2` and the A tile of g + 1 into registers, then stored
  // to the other LDS buffer after the MFMAs.
  auto group = [&](int g, Codes& cur, Codes& nxt2) {
    const int buf = g & 1;
    stage_load(min(g + 1, KG - 1));
    load_codes(min(g + 2, KG - 1), nxt2);
    // keep the loads ahead of the MFMAs, and their first uses (the stores of
    // the next A tile) after them
    __builtin_amdgcn_sched_barrier(0);
    pf_f32x16 temp[NMAT][NB][2];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = 8 * hl + j;   // chunk of the group
      uint4 af[NSPLIT][2];
#pragma unroll
      for (int sp = 0; sp < NSPLIT; ++sp)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          af[sp][mb] = a_lds[((size_t)((buf * NSPLIT + sp) * 2 + mb) * 16 + c) * 32 + (lrow ^ (c & 14))];
#pragma unroll
      for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint4 cw = cur.c[mat][nb][j >> 2];
          const uint32_t dw = (j & 3) == 0 ? cw.x : (j & 3) == 1 ? cw.y : (j & 3) == 2 ? cw.z : cw.w;
          const uint4 bx = expand_codes(dw);
#pragma unroll
          for (int sp = 0; sp < NSPLIT; ++sp)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
              temp[mat][nb][mb] = mfma_bf16(af[sp][mb], bx, (j == 0 && sp == 0) ? pf_f32x16{} : temp[mat][nb][mb]);
        }
    }
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float sc = bf16_bits_to_f32(cur.s[mat][nb]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mat][nb][mb][r] = fmaf(sc, temp[mat][nb][mb][r], acc[mat][nb][mb][r]);
      }
    __builtin_amdgcn_sched_barrier(0);
    stage_store(buf ^ 1, g + 1, g + 1 < KG);   // after the last group: unused
    wg_sync();
  };

  // Codes run two groups ahead of the MFMAs (three register sets, rotated
  // after each group), the A tile one group ahead.
  Codes c0, c1, c2;
  load_codes(0, c0);
  load_codes(min(1, KG - 1), c1);
  stage_load(0);
  stage_store(0, 0, true);
  wg_sync();
#pragma unroll 1
  for (int g = 0; g < KG; ++g) {
    group(g, c0, c2);
    c0 = c1;
    c1 = c2;
  }

  // -136 sum_g s[n][g] R[m][g]: K = the KG groups (zero-padded to 16)
  uint4 rp[3][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    uint32_t h2[4], m2[4], l2[4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      float v[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int g = 8 * hl + i + u;
        v[u] = g < KG ? rsum_lds[(mb * 32 + lrow) * KG + g] : 0.f;
      }
      uint32_t hb[2], mbits[2], lb[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        hb[u] = f32_to_bf16_rne(v[u]);
        const float r1 = v[u] - bf16_bits_to_f32(hb[u]);
        mbits[u] = f32_to_bf16_rne(r1);
        lb[u] = f32_to_bf16_rne(r1 - bf16_bits_to_f32(mbits[u]));
      }
      h2[i / 2] = hb[0] | (hb[1] << 16);
      m2[i / 2] = mbits[0] | (mbits[1] << 16);
      l2[i / 2] = lb[0] | (lb[1] << 16);
    }
    rp[0][mb] = make_uint4(h2[0], h2[1], h2[2], h2[3]);
    rp[1][mb] = make_uint4(m2[0], m2[1], m2[2], m2[3]);
    rp[2][mb] = make_uint4(l2[0], l2[1], l2[2], l2[3]);
  }
#pragma unroll
  for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint16_t* sp = S[mat] + (size_t)(wrow0 + nb * 32 + lrow) * KG;
      uint32_t sw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const int g = 8 * hl + i;
        if (g + 1 < KG) sw[i / 2] = (uint32_t)sp[g] | ((uint32_t)sp[g + 1] << 16);
      }
      const uint4 sb = make_uint4(sw[0], sw[1], sw[2], sw[3]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        pf_f32x16 corr = mfma_bf16(rp[0][mb], sb, pf_f32x16{});
        corr = mfma_bf16(rp[1][mb], sb, corr);
        corr = mfma_bf16(rp[2][mb], sb, corr);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mat][nb][mb][r] = fmaf(-136.f, corr[r], acc[mat][nb][mb][r]);
      }
    }
}

// tile row of accumulator register r of row block mb
__device__ __forceinline__ int tile_row(int mb, int r) {
  return mb * 32 + 8 * (r >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (r & 3);
}

// h = silu(g) u as bf16 hi + lo at pair-order position of feature col
__device__ __forceinline__ void store_h(uint16_t* hi_row, uint16_t* lo_row, int col, float g, float u) {
  const float hv = silu_mul(g, u);
  const uint32_t hi = f32_to_bf16_rne(hv);
  const uint32_t lo = f32_to_bf16_rne(hv - bf16_bits_to_f32(hi));
  const int p = perm_order(col);
  hi_row[p] = (uint16_t)hi;
  lo_row[p] = (uint16_t)lo;
}

constexpr int LDS_A1 = 2 * 1 * 2 * 16 * 32;   // uint4, NSPLIT = 1
constexpr int LDS_A2 = 2 * 2 * 2 * 16 * 32;   // uint4, NSPLIT = 2

// Work items of the persistent GEMM kernels: (tile, N-slice) pairs, numbered
// so that the NT slices of one tile are 8 apart (one XCD, whose L2 then holds
// the tile's A rows) and come up in the same round of the grid.
__device__ __forceinline__ void pf_item(int q, int nt_count, int& tile, int& nt) {
  tile = 8 * (q / (8 * nt_count)) + (q & 7);
  nt = (q >> 3) % nt_count;
}
__host__ __device__ constexpr int pf_items(int tiles, int nt_count) { return (tiles + 7) / 8 * 8 * nt_count; }

// ------------------------------------------------------------- routed gate/up
__global__ void __launch_bounds__(PF_NT, 2) k_pf_gateup(const uint16_t* __restrict__ a, const int4* __restrict__ tiles,
                                                      const int* __restrict__ tile_start, const int* __restrict__ perm,
                                                      LayerW L, uint16_t* __restrict__ h_hi, uint16_t* __restrict__ h_lo) {
  __shared__ __align__(16) uint4 a_lds[LDS_A1];
  __shared__ __align__(16) float rsum[PF_TM * (H / G)];
  __shared__ int rows[PF_TM];
  constexpr int NT = I / 128;
  const int tid = threadIdx.x, wave = tid >> 6, lrow = tid & 31;
  // this XCD's tiles, the NT column slices of a tile on consecutive workgroups
  const int x = blockIdx.x & 7, t0 = tile_start[x], items = (tile_start[x + 1] - t0) * NT;
  for (int q = blockIdx.x >> 3; q < items; q += gridDim.x >> 3) {
    const int nt = q % NT;
    const int4 tl = tiles[t0 + q / NT];
    const int e = tl.x, pos0 = tl.y, cnt = tl.z;
    wg_sync();   // the previous item is done with the LDS
    if (tid < PF_TM) rows[tid] = tid < cnt ? perm[pos0 + tid] / TOPK : -1;
    wg_sync();
    const int wrow0 = nt * 128 + wave * 32;
    const uint8_t* const W[2] = {L.gate + (size_t)e * I * (H / 2), L.up + (size_t)e * I * (H / 2)};
    const uint16_t* const S[2] = {L.gate_s + (size_t)e * I * (H / G), L.up_s + (size_t)e * I * (H / G)};
    const uint16_t* const Ap[1] = {a};
    pf_f32x16 acc[2][1][2] = {};
    gemm_tile<1, 2, H / G, 1>(Ap, H, rows, W, S, wrow0, acc, a_lds, rsum);
    const int col = wrow0 + lrow;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = tile_row(mb, r);
        if (m < cnt) store_h(h_hi + (size_t)(pos0 + m) * I, h_lo + (size_t)(pos0 + m) * I, col, acc[0][0][mb][r],
                             acc[1][0][mb][r]);
      }
  }
}

// ------------------------------------------------------------- shared gate/up
__global__ void __launch_bounds__(PF_NT, 2) k_pf_sh_gateup(const uint16_t* __restrict__ a, int n, LayerW L,
                                                         uint16_t* __restrict__ hs_hi, uint16_t* __restrict__ hs_lo) {
  __shared__ __align__(16) uint4 a_lds[LDS_A1];
  __shared__ __align__(16) float rsum[PF_TM * (H / G)];
  __shared__ int rows[PF_TM];
  constexpr int NT = IS / 128;
  const int T = (n + PF_TM - 1) / PF_TM;
  const int tid = threadIdx.x, wave = tid >> 6, lrow = tid & 31;
  for (int q = blockIdx.x; q < pf_items(T, NT); q += gridDim.x) {
    int ti, nt;
    pf_item(q, NT, ti, nt);
    if (ti >= T) continue;
    const int m0 = ti * PF_TM;
    wg_sync();
    if (tid < PF_TM) rows[tid] = m0 + tid < n ? m0 + tid : -1;
    wg_sync();
    const int wrow0 = nt * 128 + wave * 32;
    const uint8_t* const W[2] = {L.sh_gate, L.sh_up};
    const uint16_t* const S[2] = {L.sh_gate_s, L.sh_up_s};
    const uint16_t* const Ap[1] = {a};
    pf_f32x16 acc[2][1][2] = {};
    gemm_tile<1, 2, H / G, 1>(Ap, H, rows, W, S, wrow0, acc, a_lds, rsum);
    const int col = wrow0 + lrow;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + tile_row(mb, r);
        if (m < n) store_h(hs_hi + (size_t)m * IS, hs_lo + (size_t)m * IS, col, acc[0][0][mb][r], acc[1][0][mb][r]);
      }
  }
}

// ------------------------------------------------------------- routed down
// Work item: 32 rows of a tile (a half tile) x a quarter of the H output
// columns.  The half tile's h rows (both bf16 parts, all of K = 512: 64 KB)
// are staged into LDS once; each wave then streams the int4 rows of its 128
// columns in blocks of 32, the codes of the next block in flight during the
// MFMAs of the current one.  Output: y[pair][col] for each (token, slot) pair.
constexpr int PD_TM = 32;              // rows of a half tile
constexpr int PD_NQ = 4;               // column quarters of H per half tile
constexpr int PD_NB = H / PD_NQ / 128; // 32-column blocks per wave (4 waves)
constexpr int PD_KC = I / 8;           // 8-element chunks of a row (64)
constexpr int PD_KG = I / G;           // K-groups (4)
static_assert(PD_KC == 64 && PD_KG == 4 && PD_NB == 4, "routed down layout");

// codes and scales of one lane's weight row: group g, bytes 32 hl + [0, 32)
struct DownCodes {
  uint4 c[PD_KG][2];
  uint2 s;   // the row's 4 bf16 scales
};

__device__ __forceinline__ void down_load(const uint8_t* W, const uint16_t* S, int row, int hl, DownCodes& d) {
  const uint4* p = reinterpret_cast<const uint4*>(W + (size_t)row * (I / 2)) + 2 * hl;
#pragma unroll
  for (int g = 0; g < PD_KG; ++g) {
    d.c[g][0] = p[4 * g];
    d.c[g][1] = p[4 * g + 1];
  }
  d.s = *reinterpret_cast<const uint2*>(S + (size_t)row * PD_KG);
}

// One 32 x 32 output block: rows of the half tile, columns of code block d.
// a_lds[part][chunk][slot]: chunk c of tile row r at slot r ^ (c & 15).
__device__ __forceinline__ pf_f32x16 down_block(const uint4 (*a_lds)[PD_KC][PD_TM], const DownCodes& d,
                                                const uint4 (&rp)[3], int lrow, int hl) {
  pf_f32x16 acc;
#pragma unroll
  for (int g = 0; g < PD_KG; ++g) {
    pf_f32x16 temp;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = 16 * g + 8 * hl + j;
      const uint4 a0 = a_lds[0][c][lrow ^ (8 * hl + j)];
      const uint4 a1 = a_lds[1][c][lrow ^ (8 * hl + j)];
      const uint4 cw = d.c[g][j >> 2];
      const uint32_t dw = (j & 3) == 0 ? cw.x : (j & 3) == 1 ? cw.y : (j & 3) == 2 ? cw.z : cw.w;
      const uint4 bx = expand_codes(dw);
      temp = mfma_bf16(a0, bx, j == 0 ? pf_f32x16{} : temp);
      temp = mfma_bf16(a1, bx, temp);
    }
    const uint32_t sbits = (g & 1) ? ((g < 2 ? d.s.x : d.s.y) >> 16) : ((g < 2 ? d.s.x : d.s.y) & 0xFFFFu);
    const float sc = bf16_bits_to_f32(sbits);
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = g == 0 ? sc * temp[r] : fmaf(sc, temp[r], acc[r]);
  }
  // -136 sum_g s[n][g] R[m][g]: K = the 4 groups in lanes 0..31, zero-padded
  const uint4 sb = hl == 0 ? make_uint4(d.s.x, d.s.y, 0u, 0u) : make_uint4(0u, 0u, 0u, 0u);
  pf_f32x16 corr = mfma_bf16(rp[0], sb, pf_f32x16{});
  corr = mfma_bf16(rp[1], sb, corr);
  corr = mfma_bf16(rp[2], sb, corr);
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = fmaf(-136.f, corr[r], acc[r]);
  return acc;
}

__global__ void __launch_bounds__(PF_NT, 2) k_pf_down(const uint16_t* __restrict__ h_hi,
                                                       const uint16_t* __restrict__ h_lo,
                                                       const int4* __restrict__ tiles, const int* __restrict__ tile_start,
                                                       const int* __restrict__ perm, LayerW L, float* __restrict__ y) {
  __shared__ __align__(16) uint4 a_lds[2][PD_KC][PD_TM];
  __shared__ float rsum[PD_TM][PD_KG];
  __shared__ int pairs[PD_TM];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lrow = lane & 31, hl = lane >> 5;
  // this XCD's half tiles, the column quarters of one on consecutive workgroups
  const int x = blockIdx.x & 7, t0 = tile_start[x], items = (tile_start[x + 1] - t0) * 2 * PD_NQ;
  for (int q = blockIdx.x >> 3; q < items; q += gridDim.x >> 3) {
    const int ht = q / PD_NQ, nq = q % PD_NQ;
    const int4 tl = tiles[t0 + (ht >> 1)];
    const int e = tl.x, pos = tl.y + PD_TM * (ht & 1), rows = min(tl.z - PD_TM * (ht & 1), PD_TM);
    if (rows <= 0) continue;
    const uint8_t* W = L.down + (size_t)e * H * (I / 2);
    const uint16_t* S = L.down_s + (size_t)e * H * PD_KG;
    const int n0 = nq * (H / PD_NQ) + wave * (PD_NB * 32);
    wg_sync();   // the previous item is done with the LDS
    // stage the half tile: thread = (chunk lane, rows wave + 4 i); padding rows
    // read the first row
    uint4 st[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wave + 4 * i;
      const size_t src = (size_t)(pos + (r < rows ? r : 0)) * I;
      st[i][0] = reinterpret_cast<const uint4*>(h_hi + src)[lane];
      st[i][1] = reinterpret_cast<const uint4*>(h_lo + src)[lane];
    }
    const int pr = tid < rows ? perm[pos + tid] : 0;
    DownCodes c0, c1;
    down_load(W, S, n0 + lrow, hl, c0);
    __builtin_amdgcn_sched_barrier(0);
    if (tid < PD_TM) pairs[tid] = pr;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wave + 4 * i;
      a_lds[0][lane][r ^ (lane & 15)] = st[i][0];
      a_lds[1][lane][r ^ (lane & 15)] = st[i][1];
      float part = bf16x8_sum(st[i][0]) + bf16x8_sum(st[i][1]);
      part += dpp_f32<DPP_XOR1>(part);   // the 16 chunks of one group
      part += dpp_f32<DPP_XOR2>(part);
      part += dpp_f32<DPP_HALF_MIRROR>(part);
      part += dpp_f32<DPP_MIRROR>(part);
      if ((lane & 15) == 0) rsum[r][lane >> 4] = part;
    }
    wg_sync();
    // R of this lane's row split into three bf16 parts (exact products)
    uint4 rp[3];
    {
      uint32_t w3[3][2] = {};
#pragma unroll
      for (int g = 0; g < PD_KG; ++g) {
        const float v = hl == 0 ? rsum[lrow][g] : 0.f;
        const uint32_t b0 = f32_to_bf16_rne(v);
        const float r1 = v - bf16_bits_to_f32(b0);
        const uint32_t b1 = f32_to_bf16_rne(r1);
        const uint32_t b2 = f32_to_bf16_rne(r1 - bf16_bits_to_f32(b1));
        const int sh = 16 * (g & 1);
        w3[0][g >> 1] |= b0 << sh;
        w3[1][g >> 1] |= b1 << sh;
        w3[2][g >> 1] |= b2 << sh;
      }
#pragma unroll
      for (int k = 0; k < 3; ++k) rp[k] = make_uint4(w3[k][0], w3[k][1], 0u, 0u);
    }
    auto store = [&](int nb, const pf_f32x16& acc) {
      const int col = n0 + nb * 32 + lrow;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = tile_row(0, r);
        if (m < rows) y[(size_t)pairs[m] * H + col] = acc[r];
      }
    };
    // four column blocks, two code sets in turn (no register copies while a
    // load is in flight)
    down_load(W, S, n0 + 32 + lrow, hl, c1);
    __builtin_amdgcn_sched_barrier(0);
    store(0, down_block(a_lds, c0, rp, lrow, hl));
    __builtin_amdgcn_sched_barrier(0);
    down_load(W, S, n0 + 64 + lrow, hl, c0);
    __builtin_amdgcn_sched_barrier(0);
    store(1, down_block(a_lds, c1, rp, lrow, hl));
    __builtin_amdgcn_sched_barrier(0);
    down_load(W, S, n0 + 96 + lrow, hl, c1);
    __builtin_amdgcn_sched_barrier(0);
    store(2, down_block(a_lds, c0, rp, lrow, hl));
    __builtin_amdgcn_sched_barrier(0);
    store(3, down_block(a_lds, c1, rp, lrow, hl));
  }
}

// ------------------------------------------------------------- shared down + combine
__global__ void __launch_bounds__(PF_NT) k_pf_sh_down(const float* xin, float* out, int n,
                                                       const uint16_t* __restrict__ hs_hi,
                                                       const uint16_t* __restrict__ hs_lo, LayerW L,
                                                       const float* __restrict__ w, const float* __restrict__ y) {
  __shared__ __align__(16) uint4 a_lds[LDS_A2];
  __shared__ __align__(16) float rsum[PF_TM * (IS / G)];
  __shared__ int rows[PF_TM];
  constexpr int NT = H / 256;
  const int T = (n + PF_TM - 1) / PF_TM;
  const int tid = threadIdx.x, wave = tid >> 6, lrow = tid & 31;
  for (int q = blockIdx.x; q < pf_items(T, NT); q += gridDim.x) {
    int ti, nt;
    pf_item(q, NT, ti, nt);
    if (ti >= T) continue;
    const int m0 = ti * PF_TM;
    wg_sync();
    if (tid < PF_TM) rows[tid] = m0 + tid < n ? m0 + tid : -1;
    wg_sync();
    const int wrow0 = nt * 256 + wave * 64;
    const uint8_t* const W[1] = {L.sh_down};
    const uint16_t* const S[1] = {L.sh_down_s};
    const uint16_t* const Ap[2] = {hs_hi, hs_lo};
    pf_f32x16 acc[1][2][2] = {};
    gemm_tile<2, 1, IS / G, 2>(Ap, IS, rows, W, S, wrow0, acc, a_lds, rsum);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int col = wrow0 + nb * 32 + lrow;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = m0 + tile_row(mb, r);
          if (t < n) {
            const float* wt = w + (size_t)t * TOPK;
            const float* yt = y + (size_t)t * TOPK * H + col;
            float d = wt[0] * yt[0];
#pragma unroll
            for (int s = 1; s < TOPK; ++s) d = fmaf(wt[s], yt[(size_t)s * H], d);
            d += acc[0][nb][mb][r];
            out[(size_t)t * H + col] = xin[(size_t)t * H + col] + d;
          }
        }
    }
  }
}

// ------------------------------------------------------------- host side
int prefill_workspace_alloc(PrefillWS* ws, char** mem, alloc_fn alloc) {
  const size_t T = FLINT_MAX_TOKENS, P = T * TOPK;
  const size_t sizes[14] = {T * H * 2,      T * E * 4,  T * TOPK * 4, T * TOPK * 4, (size_t)E * PF_BW * 4,
                            (size_t)(E + 1) * 4, (size_t)PF_MAX_TILES * 16, 9 * 4, P * 4, P * I * 2,
                            P * I * 2,      P * H * 4,  T * IS * 2,   T * IS * 2};
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t tot = 0;
  for (size_t s : sizes) tot += up(s);
  char* p = nullptr;
  const int rc = alloc((void**)&p, tot, "prefill workspace");
  if (rc) return rc;
  *mem = p;
  void** dst[14] = {(void**)&ws->a,     (void**)&ws->z,       (void**)&ws->ids,   (void**)&ws->w,
                    (void**)&ws->bitmap, (void**)&ws->offsets, (void**)&ws->tiles, (void**)&ws->tile_start,
                    (void**)&ws->perm,  (void**)&ws->h_hi,    (void**)&ws->h_lo,  (void**)&ws->y,
                    (void**)&ws->hs_hi, (void**)&ws->hs_lo};
  for (int i = 0; i < 14; ++i) {
    *dst[i] = p;
    p += up(sizes[i]);
  }
  return FLINT_OK;
}

hipError_t launch_prefill_layer(const float* xin, float* out, int n, const LayerW& L, const PrefillWS& ws,
                                int* trace_ids, float* trace_w, hipStream_t s) {
  if (n <= DECODE_MAX_TOKENS || n > FLINT_MAX_TOKENS) return hipErrorInvalidValue;
  const int mt = (n + PF_TM - 1) / PF_TM;
  hipLaunchKernelGGL(k_pf_input, dim3(n), dim3(PF_NT), 0, s, xin, n, ws.a, ws.bitmap);
  hipLaunchKernelGGL(k_pf_router, dim3((n + 31) / 32, E / 32), dim3(PF_NT), 0, s, ws.a, n, L.router, ws.z);
  hipLaunchKernelGGL(k_pf_route, dim3((n + 3) / 4), dim3(PF_NT), 0, s, ws.z, n, L.bias, ws.ids, ws.w, ws.bitmap,
                     trace_ids, trace_w);
  hipLaunchKernelGGL(k_pf_offsets, dim3(1), dim3(E), 0, s, ws.bitmap, n, ws.offsets, ws.tiles, ws.tile_start);
  hipLaunchKernelGGL(k_pf_scatter, dim3((n * TOPK + PF_NT - 1) / PF_NT), dim3(PF_NT), 0, s, ws.ids, n, ws.bitmap,
                     ws.offsets, ws.perm);
  // persistent grids: about one round of resident workgroups, at most one per item
  auto grid = [](int items, int resident) { return dim3(std::max(1, std::min(items, resident))); };
  // routed GEMMs: two resident workgroups per CU, 64 per XCD (a multiple of 8)
  hipLaunchKernelGGL(k_pf_gateup, dim3(2 * 256), dim3(PF_NT), 0, s, ws.a, ws.tiles, ws.tile_start, ws.perm, L,
                     ws.h_hi, ws.h_lo);
  hipLaunchKernelGGL(k_pf_sh_gateup, grid(pf_items(mt, IS / 128), 2 * 256), dim3(PF_NT), 0, s, ws.a, n, L, ws.hs_hi,
                     ws.hs_lo);
  hipLaunchKernelGGL(k_pf_down, dim3(2 * 256), dim3(PF_NT), 0, s, ws.h_hi, ws.h_lo, ws.tiles, ws.tile_start, ws.perm,
                     L, ws.y);
  hipLaunchKernelGGL(k_pf_sh_down, grid(pf_items(mt, H / 256), 256), dim3(PF_NT), 0, s, xin, out, n, ws.hs_hi,
                     ws.hs_lo, L, ws.w, ws.y);
  return hipGetLastError();
}

}  // namespace flint
