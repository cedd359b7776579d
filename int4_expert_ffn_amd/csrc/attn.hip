// Decode attention with learned sinks: one layer, up to 16 query tokens,
// split over the positions a token sees (TandemLLM "21 Flint", 21.1 table rows
// "attention", "sliding layers", "full layers"; How to Run Flint Locally,
// "Sinks and the 513-token window").
//
//   k_attn_chunk    one workgroup per (chunk of 256 positions, or of 64 for a
//                   token that sees at most 768, KV head, token):
//                   scores of the KV head's 8 query heads on the matrix cores
//                   (keys bf16, the query split into three bf16 parts so that
//                   every product is exact and the scores carry fp32
//                   precision), the chunk's maximum, e^(s - m), their sum and
//                   the weighted sum of the values, also on the matrix cores
//                   (the weights as two bf16 parts) -> one partial per head
//   k_attn_combine  per (query head, 16 dimensions, token): the partials and
//                   the sink in a fixed order (16 interleaved subsets of the
//                   chunks, each in chunk order, then the subsets in order)
//                   -> out
// Each token's chunks are computed the same way whatever the other tokens
// are, and every sum has a fixed order, so results are deterministic and
// bitwise independent of the token count.
#include <mutex>

#include "attn.h"

namespace flint {

namespace {

constexpr int AQ = FLINT_ATT_Q_HEADS, AKV = FLINT_ATT_KV_HEADS, AD = FLINT_ATT_HEAD_DIM;
constexpr int AG = AQ / AKV;   // query heads per KV head
constexpr int ACH = 256;       // positions per chunk: 4 waves x 4 blocks of 16
constexpr int APART = AD + 4;  // floats per partial: m, l, 2 unused, acc[AD]
constexpr int ANT = 256;
constexpr int AVP = AD + 4;    // padded value row (u16)

typedef __bf16 at_bf16x8 __attribute__((ext_vector_type(8)));
typedef float at_f32x4 __attribute__((ext_vector_type(4)));

// D = A B + C, 16 x 32 by 32 x 16: lane l holds row l % 16 of A and column
// l % 16 of B for k = 8 (l / 16) .. + 7 (natural order on both); D register r
// of lane l is row 4 (l / 16) + r, column l % 16.
__device__ __forceinline__ at_f32x4 mfma16(uint4 a, uint4 b, at_f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(at_bf16x8, a), __builtin_bit_cast(at_bf16x8, b),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

}  // namespace

// Per token: the first position it sees, how many, its chunks, and the chunk
// size (ACH, or ACH_S for a token that sees at most ACH_SMAX positions: more
// workgroups for short ranges such as the 513-position window).
struct AttnTokens {
  int first[FLINT_ATT_MAX_TOKENS];
  int count[FLINT_ATT_MAX_TOKENS];
  int nch[FLINT_ATT_MAX_TOKENS];
  int chunk[FLINT_ATT_MAX_TOKENS];
};
constexpr int ACH_S = 64, ACH_SMAX = 768;

// CH positions per chunk (a multiple of 64): wave w scores positions
// CH / 4 w + 16 b of the chunk for its CH / 64 blocks.  Workgroup (c, g, t)
// takes chunk c of token t and KV head g; tokens whose chunk size is not CH
// are left to the other instance.
template <int CH>
__global__ void __launch_bounds__(ANT) k_attn_chunk(const float* __restrict__ q, const uint16_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v, int ring, AttnTokens T, int nch_max,
                                                    float* __restrict__ ws) {
  constexpr int BW = CH / 64;   // blocks of 16 positions per wave
  constexpr int NV = CH / 32;   // value loads per thread and half row
  // scores [position][head]; once they are in registers the same memory holds
  // e^(s - m) as two bf16 parts [2 h + part][position]
  __shared__ __align__(16) float sp_lds[CH * AG];
  float (*const s_lds)[AG] = reinterpret_cast<float (*)[AG]>(sp_lds);
  uint16_t (*const p16)[CH] = reinterpret_cast<uint16_t (*)[CH]>(sp_lds);
  static_assert(2 * AG * CH * 2 == CH * AG * 4, "weights reuse the score memory");
  __shared__ float red[4][AG];
  // the chunk's value rows of this KV head, rows padded to 264 bytes so that
  // the matrix-core operand reads (16 dimensions x rows 8 apart) hit distinct banks
  __shared__ __align__(16) uint16_t v_lds[CH][AVP];
  const int t = blockIdx.z, g = blockIdx.y;
  if (T.chunk[t] != CH) return;
  const int nch = T.nch[t], first = T.first[t], last = T.first[t] + T.count[t];
  const int c = blockIdx.x;
  if (c >= nch) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  // ---- the chunk's keys and values into registers.  Keys: the A operand, row =
  // position CH / 4 wave + 16 b + lane % 16 of the chunk, 256 contiguous bytes
  // (rows past the chunk's end read an in-ring row and are masked below).
  // Values: 8 threads per 256-byte row, 32 bytes each (rows past the chunk's
  // end repeat its first row), written to LDS after the scores.
  const int p0 = first + c * CH, cnt = min(CH, last - p0);
  uint4 ka[BW][4], vst[NV], vst2[NV];
  auto load_keys = [&]() {
#pragma unroll
    for (int b = 0; b < BW; ++b) {
      const int j = 16 * BW * wave + 16 * b + (lane & 15);
      const uint4* kr = reinterpret_cast<const uint4*>(k + ((size_t)((p0 + j) % ring) * AKV + g) * AD);
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[b][s] = kr[4 * s + (lane >> 4)];
    }
  };
  auto load_values = [&]() {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = 32 * i + (tid >> 3), piece = tid & 7;   // rows 32 i .. 32 i + 31
      const int jj = j < cnt ? j : 0;
      vst[i] = reinterpret_cast<const uint4*>(v + ((size_t)((p0 + jj) % ring) * AKV + g) * AD)[2 * piece];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = 32 * i + (tid >> 3), piece = tid & 7;
      const int jj = j < cnt ? j : 0;
      vst2[i] = reinterpret_cast<const uint4*>(v + ((size_t)((p0 + jj) % ring) * AKV + g) * AD)[2 * piece + 1];
    }
  };
  // ---- B operands of the scores.  Column n = lane % 16 is query head
  // 8 g + n / 2 (n even: the query's high bf16 part, odd: the middle part); a
  // second B carries the low part in the even columns.  q = hi + mid + lo exactly.
  // The keys are requested before the query and the values after it (loads
  // return in order: the query's wait covers the keys only).
  load_keys();
  float4 qv[8];
  {
    const float* qh = q + ((size_t)t * AQ + AG * g + ((lane & 15) >> 1)) * AD + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qv[2 * s] = *reinterpret_cast<const float4*>(qh + 32 * s);
      qv[2 * s + 1] = *reinterpret_cast<const float4*>(qh + 32 * s + 4);
    }
  }
  load_values();
  // keep the conversion below every load: the values must not wait for the keys
  compiler_fence();
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(qv[i].x), "+v"(qv[i].y), "+v"(qv[i].z), "+v"(qv[i].w));
  uint4 bq[4], bl[4];
  {
    const int odd = lane & 1;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float4 x0 = qv[2 * s], x1 = qv[2 * s + 1];
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      uint32_t w[8], wl[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t hi = f32_to_bf16_rne(xs[i]);
        const float r1 = xs[i] - bf16_bits_to_f32(hi);
        const uint32_t mid = f32_to_bf16_rne(r1);
        const uint32_t lo = f32_to_bf16_rne(r1 - bf16_bits_to_f32(mid));
        w[i] = odd ? mid : hi;
        wl[i] = odd ? 0u : lo;
      }
      bq[s] = make_uint4(pack2(w[0], w[1]), pack2(w[2], w[3]), pack2(w[4], w[5]), pack2(w[6], w[7]));
      bl[s] = make_uint4(pack2(wl[0], wl[1]), pack2(wl[2], wl[3]), pack2(wl[4], wl[5]), pack2(wl[6], wl[7]));
    }
  }
  const float scale = 0.08838834764831845f;   // 1 / sqrt(128), exact to fp32 rounding
  // ---- scores
#pragma unroll
  for (int b = 0; b < BW; ++b) {
    at_f32x4 d = {0.f, 0.f, 0.f, 0.f}, e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      d = mfma16(ka[b][s], bq[s], d);
      e = mfma16(ka[b][s], bl[s], e);
    }
    // lanes n, n ^ 1 hold the two parts of one head: (hi + mid) + lo
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float other = dpp_f32<DPP_XOR1>(d[r]);
      const float sum = ((lane & 1) ? other + d[r] : d[r] + other) + e[r];   // hi + mid, then + lo
      const int j = 16 * BW * wave + 16 * b + 4 * (lane >> 4) + r;
      if ((lane & 1) == 0) s_lds[j][(lane & 15) >> 1] = j < cnt ? sum * scale : -INFINITY;
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = 32 * i + (tid >> 3), piece = tid & 7;
    uint2* row = reinterpret_cast<uint2*>(&v_lds[j][0]) + 4 * piece;
    row[0] = make_uint2(vst[i].x, vst[i].y);
    row[1] = make_uint2(vst[i].z, vst[i].w);
    row[2] = make_uint2(vst2[i].x, vst2[i].y);
    row[3] = make_uint2(vst2[i].z, vst2[i].w);
  }
  wg_sync();

  // ---- per head: chunk maximum, e^(s - m) and their sum (thread = position)
  float sv[AG], m[AG];
  if (tid < CH) {
    const float4 s0 = *reinterpret_cast<const float4*>(&s_lds[tid][0]);
    const float4 s1 = *reinterpret_cast<const float4*>(&s_lds[tid][4]);
    sv[0] = s0.x; sv[1] = s0.y; sv[2] = s0.z; sv[3] = s0.w;
    sv[4] = s1.x; sv[5] = s1.y; sv[6] = s1.z; sv[7] = s1.w;
  } else {
#pragma unroll
    for (int h = 0; h < AG; ++h) sv[h] = -INFINITY;   // threads past the chunk
  }
#pragma unroll
  for (int h = 0; h < AG; ++h) {
    float x = sv[h];
    x = fmaxf(x, dpp_f32<DPP_XOR1>(x));
    x = fmaxf(x, dpp_f32<DPP_XOR2>(x));
    x = fmaxf(x, dpp_f32<DPP_HALF_MIRROR>(x));
    x = fmaxf(x, dpp_f32<DPP_MIRROR>(x));
    x = fmaxf(fmaxf(lane_bcast(x, 0), lane_bcast(x, 16)), fmaxf(lane_bcast(x, 32), lane_bcast(x, 48)));
    if (lane == 0) red[wave][h] = x;
  }
  wg_sync();
#pragma unroll
  for (int h = 0; h < AG; ++h) m[h] = fmaxf(fmaxf(red[0][h], red[1][h]), fmaxf(red[2][h], red[3][h]));
  float ev[AG];
#pragma unroll
  for (int h = 0; h < AG; ++h) {
    ev[h] = tid < cnt ? expf(sv[h] - m[h]) : 0.f;
    const uint32_t hi = f32_to_bf16_rne(ev[h]);
    if (tid < CH) {
      p16[2 * h][tid] = (uint16_t)hi;
      p16[2 * h + 1][tid] = (uint16_t)f32_to_bf16_rne(ev[h] - bf16_bits_to_f32(hi));
    }
  }
  wg_sync();   // red is reused below; p16 holds the weights (the scores were read before the last barrier)
  float lsum[AG];
#pragma unroll
  for (int h = 0; h < AG; ++h) {
    const float x = wave_sum(ev[h]);   // fixed tree
    if (lane == 0) red[wave][h] = x;
  }
  wg_sync();
#pragma unroll
  for (int h = 0; h < AG; ++h) lsum[h] = ((red[0][h] + red[1][h]) + red[2][h]) + red[3][h];

  // ---- weighted values on the matrix cores: O^T[d][2 h + part] =
  // sum_p V[p][d] P16[2 h + part][p] (A: 16 dimensions x 32 positions, the
  // value column gathered from LDS; B: 32 positions x 16 weight rows), all
  // CH positions in CH / 32 steps; O[h][d] = part 0 + part 1.  Wave w takes
  // the dimensions 32 w .. 32 w + 31 (two blocks of 16).
  at_f32x4 o[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int st = 0; st < CH / 32; ++st) {
    const int kb = 32 * st + 8 * (lane >> 4);
    const uint4 bp = *reinterpret_cast<const uint4*>(&p16[lane & 15][kb]);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int dd = 32 * wave + 16 * db + (lane & 15);
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)v_lds[kb + 2 * i][dd] | ((uint32_t)v_lds[kb + 2 * i + 1][dd] << 16);
      o[db] = mfma16(make_uint4(w[0], w[1], w[2], w[3]), bp, o[db]);
    }
  }
  // ---- partials: lanes 2 n and 2 n + 1 hold the two weight parts of head
  // n for the dimensions 32 wave + 16 db + 4 (lane / 16) .. + 3; both form
  // the sum (the same value), the even lane stores block db = 0 and the odd
  // lane db = 1, 16 bytes each
  {
    float4 res;
    const int db = lane & 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s0 = o[0][r] + dpp_f32<DPP_XOR1>(o[0][r]);
      const float s1 = o[1][r] + dpp_f32<DPP_XOR1>(o[1][r]);
      (&res.x)[r] = db ? s1 : s0;
    }
    const int h = (lane & 15) >> 1, dd = 32 * wave + 16 * db + 4 * (lane >> 4);
    *reinterpret_cast<float4*>(ws + (((size_t)t * AQ + AG * g + h) * nch_max + c) * APART + 4 + dd) = res;
  }
#pragma unroll
  for (int h = 0; h < AG; ++h)
    if (tid == h) {
      float* part = ws + (((size_t)t * AQ + AG * g + h) * nch_max + c) * APART;
      part[0] = m[h];
      part[1] = lsum[h];
    }
}

// One workgroup per (query head, 16 dimensions, token): 16 dimensions x 16
// chunk subsets.  M = max(o, m_c) over the chunks (exact);
// f_c = e^(m_c - M); L = e^(o - M) + sum_c l_c f_c and O = sum_c acc_c f_c,
// each subset summing its chunks c = sub, sub + 16, ... in order, then the 16
// subsets in order.
constexpr int ACS = 16;         // chunk subsets
constexpr int ACD = AD / 8;     // dimensions per workgroup
__global__ void __launch_bounds__(ACD * ACS) k_attn_combine(const float* __restrict__ sinks, AttnTokens T,
                                                            int nch_max, const float* __restrict__ ws,
                                                            float* __restrict__ out) {
  __shared__ float mred[ACD * ACS / 64];
  __shared__ float lsub[ACS], osub[ACS][ACD];
  const int h = blockIdx.x, dq = blockIdx.y, t = blockIdx.z, tid = threadIdx.x;
  const int dl = tid % ACD, sub = tid / ACD, d = ACD * dq + dl;
  const int lane = tid & 63, wave = tid >> 6;
  const int nch = T.nch[t];
  const float* part = ws + ((size_t)t * AQ + h) * nch_max * APART;
  const float o = sinks[h];
  float mx = o;
  for (int c = tid; c < nch; c += ACD * ACS) mx = fmaxf(mx, part[(size_t)c * APART]);
  mx = fmaxf(mx, dpp_f32<DPP_XOR1>(mx));
  mx = fmaxf(mx, dpp_f32<DPP_XOR2>(mx));
  mx = fmaxf(mx, dpp_f32<DPP_HALF_MIRROR>(mx));
  mx = fmaxf(mx, dpp_f32<DPP_MIRROR>(mx));
  mx = fmaxf(fmaxf(lane_bcast(mx, 0), lane_bcast(mx, 16)), fmaxf(lane_bcast(mx, 32), lane_bcast(mx, 48)));
  if (lane == 0) mred[wave] = mx;
  __syncthreads();
  float M = mred[0];
#pragma unroll
  for (int i = 1; i < ACD * ACS / 64; ++i) M = fmaxf(M, mred[i]);
  float L = 0.f, acc = 0.f;
  int c = sub;
  constexpr int AU = 8;   // chunks of this subset in flight
  for (; c + (AU - 1) * ACS < nch; c += AU * ACS) {
    float mc[AU], lc[AU], ac[AU];
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const float* pc = part + (size_t)(c + u * ACS) * APART;
      mc[u] = pc[0];
      lc[u] = pc[1];
      ac[u] = pc[4 + d];
    }
#pragma unroll
    for (int u = 0; u < AU; ++u) {
      const float f = expf(mc[u] - M);
      L = fmaf(lc[u], f, L);
      acc = fmaf(ac[u], f, acc);
    }
  }
  for (; c < nch; c += ACS) {
    const float* pc = part + (size_t)c * APART;
    const float f = expf(pc[0] - M);
    L = fmaf(pc[1], f, L);
    acc = fmaf(pc[4 + d], f, acc);
  }
  osub[sub][dl] = acc;
  if (dl == 0) lsub[sub] = L;
  __syncthreads();
  if (sub == 0) {
    float Lt = expf(o - M), At = 0.f;
#pragma unroll
    for (int i = 0; i < ACS; ++i) {
      Lt += lsub[i];
      At += osub[i][dl];
    }
    out[((size_t)t * AQ + h) * AD + d] = At / Lt;
  }
}

// Scratch of the allocation-free entry point (flint_attn_decode_noalloc): the
// chunk partials live in this file-scope device array, which every GPU the
// library runs on holds until the process ends.  In host code `scratch` only
// names the symbol; its device address, per device, comes from
// hipGetSymbolAddress on the first call on that device (attn_scratch).  Each
// call writes every partial it reads, so nothing needs clearing between calls.
__device__ __align__(256) float scratch[ATTN_SCRATCH_BYTES / sizeof(float)];

namespace {
std::mutex g_scratch_mu;
float* g_scratch_dev[ATTN_MAX_DEVICES] = {};
}  // namespace

hipError_t attn_scratch(float** p) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= ATTN_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = static_cast<float*>(a);
  }
  *p = g_scratch_dev[dev];
  return hipSuccess;
}

size_t attn_workspace_bytes(int n_tokens, int max_seen) {
  // chunks of the longer of: ACH positions, or ACH_S positions up to ACH_SMAX seen
  const size_t nch = std::max<size_t>((size_t)(max_seen + ACH - 1) / ACH,
                                      (size_t)(std::min(max_seen, ACH_SMAX) + ACH_S - 1) / ACH_S);
  return (size_t)n_tokens * AQ * nch * APART * sizeof(float);
}

hipError_t launch_attn_decode(const float* q, const uint16_t* k, const uint16_t* v, int ring, const float* sinks,
                              const int* first, const int* count, int n_tokens, float* out, float* ws,
                              hipStream_t s) {
  AttnTokens T = {};
  int nch_max = 0, nch_big = 0, nch_small = 0;
  for (int t = 0; t < n_tokens; ++t) {
    T.first[t] = first[t];
    T.count[t] = count[t];
    T.chunk[t] = count[t] <= ACH_SMAX ? ACH_S : ACH;   // by the token's own range only
    T.nch[t] = (count[t] + T.chunk[t] - 1) / T.chunk[t];
    nch_max = max(nch_max, T.nch[t]);
    if (T.chunk[t] == ACH) nch_big = max(nch_big, T.nch[t]);
    else nch_small = max(nch_small, T.nch[t]);
  }
  if (nch_big)
    hipLaunchKernelGGL(k_attn_chunk<ACH>, dim3(nch_big, AKV, n_tokens), dim3(ANT), 0, s, q, k, v, ring, T, nch_max, ws);
  if (nch_small)
    hipLaunchKernelGGL(k_attn_chunk<ACH_S>, dim3(nch_small, AKV, n_tokens), dim3(ANT), 0, s, q, k, v, ring, T, nch_max,
                       ws);
  hipLaunchKernelGGL(k_attn_combine, dim3(AQ, AD / ACD, n_tokens), dim3(ACD * ACS), 0, s, sinks, T, nch_max, ws, out);
  return hipGetLastError();
}

}  // namespace flint
