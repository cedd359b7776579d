// Device-side building blocks of the Flint MoE block for gfx950 (CDNA4).
//
// Conventions (one wavefront = 64 lanes):
//  * gate/up rows have K = 2048: 1024 code bytes = 64 lanes x 16 bytes, so
//    lane l owns k in [32 l, 32 l + 32), all inside scale group l / 4.
//  * down rows have K = 512 (routed) or 1024 (shared): 16 or 32 lanes x 16 B.
//  * block inputs a are bf16 (W4A16, bf16 activations), kept per token in a
//    "pair order" so one 16-byte read gives the bf16 pairs that match the
//    nibble pairs extracted from one code dword (see perm_order()).
//  * every reduction has a fixed shape, so a (token, expert, row) result does
//    not depend on how many tokens share the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/flint_moe.h"

namespace flint {

constexpr int H = FLINT_HIDDEN;
constexpr int E = FLINT_EXPERTS;
constexpr int I = FLINT_EXPERT_SIZE;
constexpr int IS = FLINT_SHARED_SIZE;
constexpr int TOPK = FLINT_TOP_K;
constexpr int G = FLINT_GROUP;
constexpr int DECODE_MAX_TOKENS = 16;   // forward() uses the decode kernels up to this n
constexpr double RMS_EPS = 1e-6;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits) {
  return __uint_as_float(bits << 16);
}

// Round a double to bf16 with a single round-to-nearest-even: round to fp32
// toward zero and make the result's last bit sticky ("round to odd"), then
// round that fp32 to bf16 to nearest even.  fp32 carries 16 more significand
// bits than bf16, so the two steps equal one direct rounding.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
  float f = __double2float_rz(x);
  uint32_t b = __float_as_uint(f);
  if ((double)f != x) b |= 1u;
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}

// Position of element k of a 2048-wide activation in pair order.  Within each
// 8-element chunk the order is (0, 2, 4, 6, 1, 3, 5, 7): the even elements are
// the low nibbles of a code dword, the odd ones the high nibbles.
__device__ __forceinline__ int perm_order(int k) {
  int j = k & 7;
  return (k & ~7) | ((j & 1) ? 4 + (j >> 1) : (j >> 1));
}

// ------------------------------------------------------------------ reductions
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;  // identical in every lane (each step adds the same two values)
}

// sum over aligned groups of `width` lanes (width a power of two <= 64)
template <int width, typename T>
__device__ __forceinline__ T group_sum(T v) {
#pragma unroll
  for (int off = width / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// ------------------------------------------------------------------ int4 dots
// One code dword holds 8 nibbles (k0..k7).  After xor 0x88888888 each nibble
// n' = code + 8 is in [0, 15].  bf16 bits 0x4300 | n' encode 128 + n' exactly,
// so a bf16 dot of these values with a gives sum (code + 136) a; the caller
// removes 136 * sum(a) afterwards.  Products are exact in fp32.
__device__ __forceinline__ float dot8_bf16(uint32_t code, uint4 a, float acc) {
  uint32_t x = code ^ 0x88888888u;
  uint32_t lo = x & 0x0F0F0F0Fu;          // bytes: k0, k2, k4, k6
  uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;   // bytes: k1, k3, k5, k7
  const uint32_t K43 = 0x43434343u;
  // __builtin_amdgcn_perm(s0, s1, sel): selector bytes 0..3 pick s1's bytes,
  // 4..7 pick s0's bytes.
  uint32_t p0 = __builtin_amdgcn_perm(K43, lo, 0x04010400u);   // (k0, k2)
  uint32_t p1 = __builtin_amdgcn_perm(K43, lo, 0x04030402u);   // (k4, k6)
  uint32_t p2 = __builtin_amdgcn_perm(K43, hi, 0x04010400u);   // (k1, k3)
  uint32_t p3 = __builtin_amdgcn_perm(K43, hi, 0x04030402u);   // (k5, k7)
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p0), __builtin_bit_cast(bf16x2_t, a.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p1), __builtin_bit_cast(bf16x2_t, a.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p2), __builtin_bit_cast(bf16x2_t, a.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p3), __builtin_bit_cast(bf16x2_t, a.w), acc, false);
  return acc;
}

// Lane part of a K=2048 row: 16 code bytes against the lane's 32 activations
// (pair order, 4 x uint4), minus 136 * asum, times the row's scale.
__device__ __forceinline__ float lane_dot_gateup(uint4 code, const uint4* a4, float asum, float scale) {
  float acc = 0.f;
  acc = dot8_bf16(code.x, a4[0], acc);
  acc = dot8_bf16(code.y, a4[1], acc);
  acc = dot8_bf16(code.z, a4[2], acc);
  acc = dot8_bf16(code.w, a4[3], acc);
  return fmaf(-136.f, asum, acc) * scale;
}

// Lane part of a down row: 16 code bytes (32 nibbles, k in natural order)
// against 32 fp32 h values.  Codes are converted exactly to floats n' =
// code + 8, summed as n' h in fp32, and 8 * sum(h) is removed afterwards.
__device__ __forceinline__ float lane_dot_down(uint4 code, const float4* h4, float hsum, float scale) {
  uint32_t c[4] = {code.x, code.y, code.z, code.w};
  float acc = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t x = c[d] ^ 0x88888888u;
    uint32_t lo = x & 0x0F0F0F0Fu;          // k = 8d + 0, 2, 4, 6
    uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;   // k = 8d + 1, 3, 5, 7
    float4 ha = h4[2 * d], hb = h4[2 * d + 1];
    acc = fmaf((float)(lo & 0xFF), ha.x, acc);
    acc = fmaf((float)(hi & 0xFF), ha.y, acc);
    acc = fmaf((float)((lo >> 8) & 0xFF), ha.z, acc);
    acc = fmaf((float)((hi >> 8) & 0xFF), ha.w, acc);
    acc = fmaf((float)((lo >> 16) & 0xFF), hb.x, acc);
    acc = fmaf((float)((hi >> 16) & 0xFF), hb.y, acc);
    acc = fmaf((float)(lo >> 24), hb.z, acc);
    acc = fmaf((float)(hi >> 24), hb.w, acc);
  }
  return fmaf(-8.f, hsum, acc) * scale;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.f + expf(-g)) * u;
}

__device__ __forceinline__ double sigmoid_f64(double z) {
  if (z >= 0.0) return 1.0 / (1.0 + exp(-z));
  double ez = exp(z);
  return ez / (1.0 + ez);
}

}  // namespace flint
