// Prefill path: a block of n tokens (DECODE_MAX_TOKENS < n <= FLINT_MAX_TOKENS)
// through one layer, where the block becomes a dense contraction: ~48 tokens
// per expert on average at n = 2048, so each expert's weights are read once
// per 32-row tile and multiplied on the matrix cores.
//
//   k_pf_input    block input a = bf16(rmsnorm(x)) per token (the decode's
//                 rounding rule), 8-element chunks in pair order
//   k_pf_router   z = a Wr^T, bf16 MFMA with fp32 accumulation
//   k_pf_route    per token (one wave): s = sigmoid(z), c = s + b in fp64,
//                 top-6 and weights; marks the token in each pick's bitmap
//   k_pf_offsets  per-expert counts, their exclusive scan, the 32-row tiles
//   k_pf_scatter  (token, slot) pairs in expert order, tokens increasing
//                 within an expert (popcounts of the bitmap prefix)
//   k_pf_gateup   routed gate/up + SwiGLU per (tile, half of the rows)
//   k_pf_sh_gateup  shared gate/up + SwiGLU (32 tokens, a quarter of the rows)
//   k_pf_down     routed down projection per (tile, quarter of H) -> y by
//                 (token, slot)
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
  // (nibble ^ 8) of the low and the high nibbles: one and-xor each
  const uint32_t lo = (code & 0x0F0F0F0Fu) ^ 0x08080808u, hi = ((code >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
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
// (a and router are not marked __restrict__: the compiler fence below must
// order their loads, which it does not for memory known to be read-only)
__global__ void __launch_bounds__(PF_NT) k_pf_router(const uint16_t* a, int n, const uint16_t* router,
                                                      float* __restrict__ z) {
  __shared__ float part[3][16][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lrow = lane & 31, hl = lane >> 5;
  const int m0 = blockIdx.x * 32, e = blockIdx.y * 32 + lrow;
  const int m = min(m0 + lrow, n - 1);   // rows past n repeat the last token and are not stored
  const uint4* ar = reinterpret_cast<const uint4*>(a + (size_t)m * H) + wave * 64 + hl;
  const uint4* wr = reinterpret_cast<const uint4*>(router + (size_t)e * H) + wave * 64 + hl;
  pf_f32x16 acc0 = {}, acc1 = {};
  // MFMA step j: chunks 2 j (lanes 0..31) and 2 j + 1 (lanes 32..63).  The
  // operands of eight steps are requested as one batch, the next batch before
  // the current one is used (left to itself the compiler interleaves each
  // load with its use, about four in flight per wave).
  constexpr int RB = 8;
  uint4 av[2][RB], wv[2][RB];
  auto load = [&](int buf, int j0) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      av[buf][i] = ar[2 * (j0 + i)];
      wv[buf][i] = wr[2 * (j0 + i)];
    }
  };
  load(0, 0);
#pragma unroll
  for (int b = 0; b < 32 / RB; ++b) {
    if (b + 1 < 32 / RB) load((b + 1) & 1, RB * (b + 1));
    compiler_fence();
    // the current batch's operands pass through an empty asm statement after
    // the fence, so its MFMAs cannot be hoisted above the next batch's loads
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      uint4& x = av[b & 1][i];
      uint4& y = wv[b & 1][i];
      asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w), "+v"(y.x), "+v"(y.y), "+v"(y.z), "+v"(y.w));
    }
#pragma unroll
    for (int i = 0; i < RB; i += 2) {
      acc0 = mfma_bf16(av[b & 1][i], to_pair_order(wv[b & 1][i]), acc0);
      acc1 = mfma_bf16(av[b & 1][i + 1], to_pair_order(wv[b & 1][i + 1]), acc1);
    }
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

constexpr int PF_NT_BINS = FLINT_MAX_TOKENS / PF_TM + 1;   // tile counts 0..64 of one expert

// Inclusive sum over the lanes of each aligned group of W lanes (W = 32 or 64).
template <int W>
__device__ __forceinline__ int group_inclusive_sum(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < W; d <<= 1) {
    const int o = __shfl_up(v, d, W);
    if ((lane & (W - 1)) >= d) v += o;
  }
  return v;
}

__global__ void __launch_bounds__(E) k_pf_offsets(const uint32_t* __restrict__ bitmap, int n, int* __restrict__ offsets,
                                                   int4* __restrict__ tiles, int* __restrict__ tile_start) {
  __shared__ int wsum[E / 64];
  __shared__ int nt_hist[PF_NT_BINS], nt_above[PF_NT_BINS];
  __shared__ uint32_t nt_mask[PF_NT_BINS][E / 32];   // experts with a given tile count
  __shared__ int nt_by_rank[E], dealt_before[E], xcd_tiles[8];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
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
  // inclusive scan of the counts: within each wave, then the waves' totals
  const int vw = group_inclusive_sum<64>(cnt);
  if (lane == 63) wsum[wave] = vw;
  wg_sync();   // also orders the atomics above
  int vc = vw;
  for (int w = 0; w < wave; ++w) vc += wsum[w];
  const int oc = vc - cnt;
  offsets[e] = oc;
  if (e == E - 1) offsets[E] = vc;
  // experts with more tiles than each count (bins above it), by one wave
  if (wave == 0) {
    // lane l takes bin PF_NT_BINS - 1 - l (bins 64 .. 1); bin 0 has nothing above
    // bin 1 but is never needed above anything: nt_above[v] = sum of bins > v
    const int bin = PF_NT_BINS - 1 - lane;   // 64 .. 1
    const int incl = group_inclusive_sum<64>(nt_hist[bin]);
    nt_above[bin - 1] = incl;                // bins >= bin, i.e. > bin - 1
    if (lane == 0) nt_above[PF_NT_BINS - 1] = 0;
  }
  wg_sync();
  // rank: experts with more tiles first, equal counts by index
  int r = nt_above[nt];
  for (int w = 0; w < (e >> 5); ++w) r += __popc(nt_mask[nt][w]);
  r += __popc(nt_mask[nt][e >> 5] & ((1u << (e & 31)) - 1u));
  nt_by_rank[r] = nt;
  wg_sync();
  // dealing: thread (x, j) = (e / 32, e % 32) holds the tiles of the j-th
  // expert dealt to XCD x; exclusive sums over j give each one's place
  {
    const int x = e >> 5, jj = e & 31;
    const int v = nt_by_rank[snake_rank(x, jj)];
    const int incl = group_inclusive_sum<32>(v);
    dealt_before[e] = incl - v;
    if (jj == 31) xcd_tiles[x] = incl;
  }
  wg_sync();
  const int u = r & 15, x = u < 8 ? u : 15 - u, j = r >> 3;
  const int before = dealt_before[32 * x + j];   // tiles of the experts dealt to XCD x ahead of this one
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

// ------------------------------------------------------------- resident-tile GEMM
// One workgroup of PR_NT threads (8 waves) computes a tile of 32 A rows against
// weight rows.  The whole tile, all of K, sits in LDS for the item, so the K
// loop needs no barrier: each wave streams the int4 codes and scales of its
// own weight rows through a ring of RD register sets (step = one K-group of
// 32 rows of each weight matrix), the loads of step s + RD in flight while
// step s runs on the matrix cores.
//
// A: bf16 rows of K elements in pair-order 8-element chunks, NSPLIT parts
// whose sum is the operand (the block input; or h as hi + lo).  W, S: int4
// codes and bf16 scales in the tile-major layout (prefill.h).  The MFMA is 32 x 32 x 16
// with the tile rows as M and 32 weight rows as N; in K-group g, step j, lane
// half hl multiplies chunk 16 g + 8 hl + j (the lane's code dword j of its 32
// bytes g * 64 + 32 hl of the row).
//
// Per K-group the MFMAs accumulate sum_k (code_k + 136) a_k from zero (exact
// products, fp32), and that is added to acc times the scale s[n][g].  The
// remaining -136 sum_g s[n][g] R[m][g] (R: the sums of A over each group) is
// one more MFMA step per 32 x 32 block, with R split into three bf16 parts so
// that its products are exact.
constexpr int PR_TM = 32;    // A rows of a tile
constexpr int PR_NT = 512;   // threads of the resident-tile kernels (8 waves)
constexpr int PR_D = 2;      // steps of weight loads in flight per wave (4 measured slower: more requests
                             // in flight congest the memory system rather than hide its latency)

// chunk c of tile row r of part sp at a[sp][c][r]: the 32 rows of one chunk
// are one contiguous 512-byte run (a conflict-free fragment read, at a fixed
// offset from the lane's base address), and the one-slot pad per chunk puts
// the 16 chunks of a row that one staging store writes in distinct banks
template <int K, int NSPLIT>
struct PrTile {
  uint4 a[NSPLIT][K / 8][PR_TM + 1];
  float rsum[PR_TM][K / G];
  int rows[PR_TM];   // source row of each tile row; -1: padding (reads row 0, never stored)
};

// Stage the tile whose source rows are in T.rows: thread (row tid / 16, chunk
// lane tid % 16) loads chunks 16 g + lane of every group g and part; the 16
// lanes of a row then sum each group (R) with DPP.
template <int K, int NSPLIT>
__device__ __forceinline__ void pr_stage_load(const uint16_t* const (&A)[NSPLIT], const PrTile<K, NSPLIT>& T,
                                              uint4 (&v)[NSPLIT][K / G]) {
  constexpr int KG = K / G;
  static_assert(NSPLIT * KG <= 16 && PR_NT == PR_TM * 16, "at most 16 loads per thread");
  const int r = threadIdx.x >> 4, cl = threadIdx.x & 15;
  const int src = T.rows[r] < 0 ? T.rows[0] : T.rows[r];
#pragma unroll
  for (int sp = 0; sp < NSPLIT; ++sp)
#pragma unroll
    for (int g = 0; g < KG; ++g) v[sp][g] = reinterpret_cast<const uint4*>(A[sp] + (size_t)src * K)[16 * g + cl];
}

template <int K, int NSPLIT>
__device__ __forceinline__ void pr_stage_store(PrTile<K, NSPLIT>& T, const uint4 (&v)[NSPLIT][K / G]) {
  constexpr int KG = K / G;
  const int r = threadIdx.x >> 4, cl = threadIdx.x & 15;
#pragma unroll
  for (int g = 0; g < KG; ++g) {
    float part = 0.f;
#pragma unroll
    for (int sp = 0; sp < NSPLIT; ++sp) {
      const int c = 16 * g + cl;
      T.a[sp][c][r] = v[sp][g];
      part += bf16x8_sum(v[sp][g]);
    }
    part += dpp_f32<DPP_XOR1>(part);   // the 16 chunks of the group
    part += dpp_f32<DPP_XOR2>(part);
    part += dpp_f32<DPP_HALF_MIRROR>(part);
    part += dpp_f32<DPP_MIRROR>(part);
    if (cl == 0) T.rsum[r][g] = part;
  }
}

// codes and scale bits of one step (K-group) for this lane's row of each matrix
template <int NMAT>
struct PrStep {
  uint4 c[NMAT][2];
  uint32_t s[NMAT];
};

// W and S in the tile-major layout (one contiguous 1 KB load per half step
// and matrix, one 64-byte run of scales)
template <int K, int NMAT>
__device__ __forceinline__ void pr_load(const uint8_t* const (&W)[NMAT], const uint16_t* const (&S)[NMAT], int row,
                                        int g, PrStep<NMAT>& d) {
  constexpr int KG = K / G;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int mat = 0; mat < NMAT; ++mat) {
    const uint4* p = reinterpret_cast<const uint4*>(W[mat] + (size_t)(row >> 5) * (32 * K / 2)) + g * 128 + lane;
    d.c[mat][0] = p[0];
    d.c[mat][1] = p[64];
    d.s[mat] = S[mat][(size_t)(row >> 5) * (32 * KG) + g * 32 + (row & 31)];
  }
}

// The first RD steps of a wave's stream (issued before the tile is staged).
template <int K, int NMAT, int RD>
__device__ __forceinline__ void pr_prologue(const uint8_t* const (&W)[NMAT], const uint16_t* const (&S)[NMAT],
                                            int wrow0, PrStep<NMAT> (&ring)[RD]) {
#pragma unroll
  for (int u = 0; u < RD; ++u) pr_load<K, NMAT>(W, S, wrow0 + (threadIdx.x & 31), u, ring[u]);
}

// The wave's NB blocks of 32 weight rows (wrow0 + 32 nb + lane % 32) against
// the staged tile; epi(nb, acc) receives each block's results: register r of
// acc[mat] is tile row 8 (r / 4) + 4 hl + r % 4, weight row wrow0 + 32 nb + lane % 32.
template <int K, int NSPLIT, int NMAT, int NB, int RD, class Epi>
__device__ __forceinline__ void pr_compute(const PrTile<K, NSPLIT>& T, const uint8_t* const (&W)[NMAT],
                                           const uint16_t* const (&S)[NMAT], int wrow0, PrStep<NMAT> (&ring)[RD],
                                           Epi epi) {
  constexpr int KG = K / G;
  static_assert(KG % RD == 0 && KG <= 16, "ring steps per group count");
  const int lane = threadIdx.x & 63, lrow = lane & 31, hl = lane >> 5;
  // R of this lane's tile row, groups 8 hl .. 8 hl + 7, in three bf16 parts
  uint4 rp[3];
  {
    uint32_t w3[3][4] = {};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int g = 8 * hl + i;
      const float v = g < KG ? T.rsum[lrow][g] : 0.f;
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
  // A fragments of MFMA step q = 8 g + j, read PR_FA steps before their use
  constexpr int PR_FA = 2;
  auto frag = [&](int q, uint4 (&d)[NSPLIT]) {
    const int c = 16 * (q >> 3) + 8 * hl + (q & 7);
#pragma unroll
    for (int sp = 0; sp < NSPLIT; ++sp) d[sp] = T.a[sp][c][lrow];
  };
#pragma unroll 1
  for (int nb = 0; nb < NB; ++nb) {
    pf_f32x16 acc[NMAT];
    uint32_t sw[NMAT][4] = {};   // scales of groups 8 hl .. 8 hl + 7 for the correction
    const int row_next = wrow0 + 32 * min(nb + 1, NB - 1) + lrow;
    uint4 fr[PR_FA + 1][NSPLIT];
#pragma unroll
    for (int q = 0; q < PR_FA; ++q) frag(q, fr[q]);
#pragma unroll
    for (int g = 0; g < KG; ++g) {
      PrStep<NMAT>& cur = ring[g % RD];
      pf_f32x16 tmp[NMAT];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = 8 * g + j;
        if (q + PR_FA < 8 * KG) frag(q + PR_FA, fr[(q + PR_FA) % (PR_FA + 1)]);
        const uint4 (&af)[NSPLIT] = fr[q % (PR_FA + 1)];
#pragma unroll
        for (int mat = 0; mat < NMAT; ++mat) {
          const uint4 cw = cur.c[mat][j >> 2];
          const uint32_t dw = (j & 3) == 0 ? cw.x : (j & 3) == 1 ? cw.y : (j & 3) == 2 ? cw.z : cw.w;
          const uint4 bx = expand_codes(dw);
#pragma unroll
          for (int sp = 0; sp < NSPLIT; ++sp)
            tmp[mat] = mfma_bf16(af[sp], bx, (j == 0 && sp == 0) ? pf_f32x16{} : tmp[mat]);
        }
      }
#pragma unroll
      for (int mat = 0; mat < NMAT; ++mat) {
        const uint32_t sb = cur.s[mat] & 0xFFFFu;
        const float sc = bf16_bits_to_f32(sb);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          acc[mat][r] = g == 0 ? sc * tmp[mat][r] : fmaf(sc, tmp[mat][r], acc[mat][r]);
          // computed here: sunk into the epilogue's stores, it would keep
          // every group's partial sums alive until then
          asm volatile("" : "+v"(acc[mat][r]));
        }
        if ((g >> 3) == hl) sw[mat][(g & 7) >> 1] |= sb << (16 * (g & 1));
      }
      // refill this ring slot with the step RD ahead (the next block's
      // first groups; past the last block, its last rows again, unused)
      if (g + RD < KG)
        pr_load<K, NMAT>(W, S, wrow0 + 32 * nb + lrow, g + RD, cur);
      else
        pr_load<K, NMAT>(W, S, row_next, g + RD - KG, cur);
      // one step at a time: nothing of the next step is hoisted into this one
      // (its fragment reads and expansions would hold registers the ring needs)
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat) {
      const uint4 sb = make_uint4(sw[mat][0], sw[mat][1], sw[mat][2], sw[mat][3]);
      pf_f32x16 corr = mfma_bf16(rp[0], sb, pf_f32x16{});
      corr = mfma_bf16(rp[1], sb, corr);
      corr = mfma_bf16(rp[2], sb, corr);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mat][r] = fmaf(-136.f, corr[r], acc[mat][r]);
    }
    epi(nb, acc);
  }
}

// tile row of accumulator register r
__device__ __forceinline__ int pr_row(int r) { return 8 * (r >> 2) + 4 * ((threadIdx.x >> 5) & 1) + (r & 3); }

// silu(g) u with the hardware exponential and reciprocal (each within a few
// fp32 ulps; the prefill bound on the block output is 2e-5)
__device__ __forceinline__ float pf_silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}

// h = silu(g) u as bf16 hi + lo at pair-order position of feature col
__device__ __forceinline__ void store_h(uint16_t* hi_row, uint16_t* lo_row, int col, float g, float u) {
  const float hv = pf_silu_mul(g, u);
  const uint32_t hi = f32_to_bf16_rne(hv);
  const uint32_t lo = f32_to_bf16_rne(hv - bf16_bits_to_f32(hi));
  const int p = perm_order(col);
  hi_row[p] = (uint16_t)hi;
  lo_row[p] = (uint16_t)lo;
}

// Work items of the dense (shared-expert) kernels: (tile, N-slice) pairs,
// numbered so that the NT slices of one tile are 8 apart (one XCD, whose L2
// then holds the tile's A rows) and come up in the same round of the grid.
__device__ __forceinline__ void pf_item(int q, int nt_count, int& tile, int& nt) {
  tile = 8 * (q / (8 * nt_count)) + (q & 7);
  nt = (q >> 3) % nt_count;
}
__host__ __device__ constexpr int pf_items(int tiles, int nt_count) { return (tiles + 7) / 8 * 8 * nt_count; }

// ------------------------------------------------------------- routed gate/up
// Item: one tile (<= 32 (token, slot) pairs of one expert) against half of the
// gate and up rows (256 each); wave w takes rows 32 w .. 32 w + 31 of the
// half.  The workgroups of XCD x (blockIdx % 8) walk the items of the tiles
// dealt to x; both halves of a tile run there, so its A rows and the expert's
// weights are shared through that XCD's L2.  (Whole tiles per item would
// leave some CUs a third round: about 520 tiles for 256 CUs at 2,048 tokens.)
__global__ void __launch_bounds__(PR_NT) k_pf_gateup(const uint16_t* __restrict__ a, const int4* __restrict__ tiles,
                                                     const int* __restrict__ tile_start, const int* __restrict__ perm,
                                                     LayerW P, uint16_t* __restrict__ h_hi,
                                                     uint16_t* __restrict__ h_lo) {
  __shared__ PrTile<H, 1> T;
  const int tid = threadIdx.x, wave = tid >> 6, lrow = tid & 31;
  const int x = blockIdx.x & 7, t0 = tile_start[x], ntl = tile_start[x + 1] - t0;
  const uint16_t* const Ap[1] = {a};
  for (int q = blockIdx.x >> 3; q < 2 * ntl; q += gridDim.x >> 3) {
    const int4 tl = tiles[t0 + (q >> 1)];
    const int wrow0 = (q & 1) * (I / 2) + wave * 32;
    const int e = tl.x, pos0 = tl.y, cnt = tl.z;
    const uint8_t* const W[2] = {P.gate + (size_t)e * I * (H / 2), P.up + (size_t)e * I * (H / 2)};
    const uint16_t* const S[2] = {P.gate_s + (size_t)e * I * (H / G), P.up_s + (size_t)e * I * (H / G)};
    const int pr = tid < cnt ? perm[pos0 + tid] / TOPK : -1;
    wg_sync();   // the previous item is done with the tile
    if (tid < PR_TM) T.rows[tid] = pr;
    wg_sync();
    uint4 v[1][H / G];
    pr_stage_load<H, 1>(Ap, T, v);
    PrStep<2> ring[PR_D];
    pr_prologue<H, 2, PR_D>(W, S, wrow0, ring);
    pr_stage_store<H, 1>(T, v);
    wg_sync();
    pr_compute<H, 1, 2, 1, PR_D>(T, W, S, wrow0, ring, [&](int nb, const pf_f32x16 (&acc)[2]) {
      const int col = wrow0 + lrow;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = pr_row(r);
        if (m < cnt) store_h(h_hi + (size_t)(pos0 + m) * I, h_lo + (size_t)(pos0 + m) * I, col, acc[0][r], acc[1][r]);
      }
    });
  }
}

// ------------------------------------------------------------- shared gate/up
// Item: 32 consecutive tokens against a quarter of the shared gate and up rows
// (256 each); wave w takes rows 32 w .. 32 w + 31 of the quarter.
constexpr int PS_NQ = IS / 256;
__global__ void __launch_bounds__(PR_NT) k_pf_sh_gateup(const uint16_t* __restrict__ a, int n, LayerW P,
                                                        uint16_t* __restrict__ hs_hi, uint16_t* __restrict__ hs_lo) {
  __shared__ PrTile<H, 1> T;
  const int tid = threadIdx.x, wave = tid >> 6, lrow = tid & 31;
  const int nt = (n + PR_TM - 1) / PR_TM;
  const uint8_t* const W[2] = {P.sh_gate, P.sh_up};
  const uint16_t* const S[2] = {P.sh_gate_s, P.sh_up_s};
  const uint16_t* const Ap[1] = {a};
  for (int q = blockIdx.x; q < pf_items(nt, PS_NQ); q += gridDim.x) {
    int ti, nq;
    pf_item(q, PS_NQ, ti, nq);
    if (ti >= nt) continue;
    const int m0 = ti * PR_TM, wrow0 = nq * 256 + wave * 32;
    wg_sync();
    if (tid < PR_TM) T.rows[tid] = m0 + tid < n ? m0 + tid : -1;
    wg_sync();
    uint4 v[1][H / G];
    pr_stage_load<H, 1>(Ap, T, v);
    PrStep<2> ring[PR_D];
    pr_prologue<H, 2, PR_D>(W, S, wrow0, ring);
    pr_stage_store<H, 1>(T, v);
    wg_sync();
    pr_compute<H, 1, 2, 1, PR_D>(T, W, S, wrow0, ring, [&](int nb, const pf_f32x16 (&acc)[2]) {
      const int col = wrow0 + lrow;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = m0 + pr_row(r);
        if (t < n) store_h(hs_hi + (size_t)t * IS, hs_lo + (size_t)t * IS, col, acc[0][r], acc[1][r]);
      }
    });
  }
}

// ------------------------------------------------------------- routed down
// Item: a tile (<= 32 (token, slot) pairs of one expert) x a quarter of the H
// output columns (512); wave w takes columns 64 w .. 64 w + 63 of it.  A is
// the tile's h (both bf16 parts, K = 512: 64 KB of LDS, so two workgroups
// share a CU: four waves per SIMD, 128 registers).  Output: y[pair][col]
// for each (token, slot) pair.
constexpr int PD_NQ = 4;   // column quarters of H per tile
__global__ void __launch_bounds__(PR_NT, 4) k_pf_down(const uint16_t* __restrict__ h_hi,
                                                      const uint16_t* __restrict__ h_lo,
                                                      const int4* __restrict__ tiles, const int* __restrict__ tile_start,
                                                      const int* __restrict__ perm, LayerW P, float* __restrict__ y) {
  __shared__ PrTile<I, 2> T;
  __shared__ int pairs[PR_TM];
  const int tid = threadIdx.x, wave = tid >> 6, lrow = tid & 31;
  // this XCD's tiles, the column quarters of one on consecutive items
  const int x = blockIdx.x & 7, t0 = tile_start[x], items = (tile_start[x + 1] - t0) * PD_NQ;
  const uint16_t* const Ap[2] = {h_hi, h_lo};
  for (int q = blockIdx.x >> 3; q < items; q += gridDim.x >> 3) {
    const int4 tl = tiles[t0 + q / PD_NQ];
    const int e = tl.x, pos0 = tl.y, cnt = tl.z;
    const int wrow0 = (q % PD_NQ) * (H / PD_NQ) + wave * 64;
    const uint8_t* const W[1] = {P.down + (size_t)e * H * (I / 2)};
    const uint16_t* const S[1] = {P.down_s + (size_t)e * H * (I / G)};
    const int pr = tid < cnt ? perm[pos0 + tid] : 0;
    wg_sync();   // the previous item is done with the tile
    if (tid < PR_TM) {
      T.rows[tid] = tid < cnt ? pos0 + tid : -1;
      pairs[tid] = pr;
    }
    wg_sync();
    uint4 v[2][I / G];
    pr_stage_load<I, 2>(Ap, T, v);
    PrStep<1> ring[2];   // depth 2: four waves per SIMD leave 128 registers
    pr_prologue<I, 1, 2>(W, S, wrow0, ring);
    pr_stage_store<I, 2>(T, v);
    wg_sync();
    pr_compute<I, 2, 1, 2, 2>(T, W, S, wrow0, ring, [&](int nb, const pf_f32x16 (&acc)[1]) {
      const int col = wrow0 + 32 * nb + lrow;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = pr_row(r);
        if (m < cnt) y[(size_t)pairs[m] * H + col] = acc[0][r];
      }
    });
  }
}

// ------------------------------------------------------------- shared down + combine
// Item: 32 consecutive tokens against an eighth of the output columns (256);
// wave w takes columns 32 w .. 32 w + 31 of it.  The epilogue adds the routed
// outputs in slot order and the residual: out = x + ((w0 y0 + w1 y1) + ... + w5 y5) + y_shared.
constexpr int PS_NS = H / 256;
__global__ void __launch_bounds__(PR_NT) k_pf_sh_down(const float* xin, float* out, int n,
                                                      const uint16_t* __restrict__ hs_hi,
                                                      const uint16_t* __restrict__ hs_lo, LayerW P,
                                                      const float* __restrict__ w, const float* __restrict__ y) {
  __shared__ PrTile<IS, 2> T;
  const int tid = threadIdx.x, wave = tid >> 6, lrow = tid & 31;
  const int nt = (n + PR_TM - 1) / PR_TM;
  const uint8_t* const W[1] = {P.sh_down};
  const uint16_t* const S[1] = {P.sh_down_s};
  const uint16_t* const Ap[2] = {hs_hi, hs_lo};
  for (int q = blockIdx.x; q < pf_items(nt, PS_NS); q += gridDim.x) {
    int ti, ns;
    pf_item(q, PS_NS, ti, ns);
    if (ti >= nt) continue;
    const int m0 = ti * PR_TM, wrow0 = ns * 256 + wave * 32;
    wg_sync();
    if (tid < PR_TM) T.rows[tid] = m0 + tid < n ? m0 + tid : -1;
    wg_sync();
    uint4 v[2][IS / G];
    pr_stage_load<IS, 2>(Ap, T, v);
    PrStep<1> ring[PR_D];
    pr_prologue<IS, 1, PR_D>(W, S, wrow0, ring);
    pr_stage_store<IS, 2>(T, v);
    wg_sync();
    // the epilogue's routed outputs and residual, requested after the tile's
    // stores (a wait for those would otherwise cover these loads too: the
    // memory counter retires in order) so that they arrive during the K loop;
    // rows past n repeat the last token and are not used
    const int col = wrow0 + lrow;
    float yv[16][TOPK], xv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = min(m0 + pr_row(r), n - 1);
      const float* yt = y + (size_t)t * TOPK * H + col;
#pragma unroll
      for (int s = 0; s < TOPK; ++s) yv[r][s] = yt[(size_t)s * H];
      xv[r] = xin[(size_t)t * H + col];
    }
    pr_compute<IS, 2, 1, 1, PR_D>(T, W, S, wrow0, ring, [&](int nb, const pf_f32x16 (&acc)[1]) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = m0 + pr_row(r);
        if (t < n) {
          const float* wt = w + (size_t)t * TOPK;
          float d = wt[0] * yv[r][0];
#pragma unroll
          for (int s = 1; s < TOPK; ++s) d = fmaf(wt[s], yv[r][s], d);
          d += acc[0][r];
          out[(size_t)t * H + col] = xv[r] + d;
        }
      }
    });
  }
}

// ------------------------------------------------------------- tile-major copy
// Codes: one thread per 16-byte piece of the destination; rows of kb bytes.
__global__ void k_pf_pack_codes(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, size_t rows, int kb) {
  const int kg = kb / 64;
  const size_t total = rows * kb / 16;
  for (size_t o = blockIdx.x * (size_t)blockDim.x + threadIdx.x; o < total; o += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(o & 63), i = (int)((o >> 6) & 1);
    const size_t bg = o >> 7;   // (row block, group)
    const int g = (int)(bg % kg);
    const size_t row = 32 * (bg / kg) + (lane & 31);
    reinterpret_cast<uint4*>(dst)[o] =
        *reinterpret_cast<const uint4*>(src + row * kb + 64 * g + 32 * (lane >> 5) + 16 * i);
  }
}

// Scales: [rows][kg] -> [rows / 32][kg][32].
__global__ void k_pf_pack_scales(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, size_t rows, int kg) {
  const size_t total = rows * kg;
  for (size_t o = blockIdx.x * (size_t)blockDim.x + threadIdx.x; o < total; o += (size_t)gridDim.x * blockDim.x) {
    const size_t r = o & 31, bg = o >> 5;
    dst[o] = src[(32 * (bg / kg) + r) * kg + bg % kg];
  }
}

hipError_t prefill_pack_layer(const LayerW& src, const LayerW& dst, hipStream_t s) {
  struct M {
    const uint8_t* c;
    const uint16_t* sc;
    const uint8_t* pc;
    const uint16_t* ps;
    size_t rows;
    int k;
  };
  const M ms[6] = {{src.gate, src.gate_s, dst.gate, dst.gate_s, (size_t)E * I, H},
                   {src.up, src.up_s, dst.up, dst.up_s, (size_t)E * I, H},
                   {src.down, src.down_s, dst.down, dst.down_s, (size_t)E * H, I},
                   {src.sh_gate, src.sh_gate_s, dst.sh_gate, dst.sh_gate_s, (size_t)IS, H},
                   {src.sh_up, src.sh_up_s, dst.sh_up, dst.sh_up_s, (size_t)IS, H},
                   {src.sh_down, src.sh_down_s, dst.sh_down, dst.sh_down_s, (size_t)H, IS}};
  for (const M& m : ms) {
    hipLaunchKernelGGL(k_pf_pack_codes, dim3(4096), dim3(256), 0, s, m.c, const_cast<uint8_t*>(m.pc), m.rows,
                       m.k / 2);
    hipLaunchKernelGGL(k_pf_pack_scales, dim3(1024), dim3(256), 0, s, m.sc, const_cast<uint16_t*>(m.ps), m.rows,
                       m.k / G);
  }
  return hipGetLastError();
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

hipError_t launch_prefill_layer(const float* xin, float* out, int n, const LayerW& L, const LayerW& P,
                                const PrefillWS& ws, int* trace_ids, float* trace_w, hipStream_t s) {
  if (n <= DECODE_MAX_TOKENS || n > FLINT_MAX_TOKENS) return hipErrorInvalidValue;
  const int mt = (n + PR_TM - 1) / PR_TM;
  hipLaunchKernelGGL(k_pf_input, dim3(n), dim3(PF_NT), 0, s, xin, n, ws.a, ws.bitmap);
  hipLaunchKernelGGL(k_pf_router, dim3((n + 31) / 32, E / 32), dim3(PF_NT), 0, s, ws.a, n, L.router, ws.z);
  hipLaunchKernelGGL(k_pf_route, dim3((n + 3) / 4), dim3(PF_NT), 0, s, ws.z, n, L.bias, ws.ids, ws.w, ws.bitmap,
                     trace_ids, trace_w);
  hipLaunchKernelGGL(k_pf_offsets, dim3(1), dim3(E), 0, s, ws.bitmap, n, ws.offsets, ws.tiles, ws.tile_start);
  hipLaunchKernelGGL(k_pf_scatter, dim3((n * TOPK + PF_NT - 1) / PF_NT), dim3(PF_NT), 0, s, ws.ids, n, ws.bitmap,
                     ws.offsets, ws.perm);
  // persistent grids: at most one round of resident workgroups (one per CU
  // for the resident-tile kernels, whose tile fills most of the LDS), at most
  // one per item; the routed kernels' grids are multiples of 8 (one XCD's
  // workgroups walk that XCD's tiles)
  auto grid = [](int items, int resident) { return dim3(std::max(1, std::min(items, resident))); };
  hipLaunchKernelGGL(k_pf_gateup, dim3(256), dim3(PR_NT), 0, s, ws.a, ws.tiles, ws.tile_start, ws.perm, P, ws.h_hi,
                     ws.h_lo);
  hipLaunchKernelGGL(k_pf_sh_gateup, grid(pf_items(mt, PS_NQ), 256), dim3(PR_NT), 0, s, ws.a, n, P, ws.hs_hi,
                     ws.hs_lo);
  hipLaunchKernelGGL(k_pf_down, dim3(2 * 256), dim3(PR_NT), 0, s, ws.h_hi, ws.h_lo, ws.tiles, ws.tile_start, ws.perm,
                     P, ws.y);
  hipLaunchKernelGGL(k_pf_sh_down, grid(pf_items(mt, PS_NS), 256), dim3(PR_NT), 0, s, xin, out, n, ws.hs_hi,
                     ws.hs_lo, P, ws.w, ws.y);
  return hipGetLastError();
}

}  // namespace flint
