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

#include "flint_moe.h"

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

// Round a double to bf16 with one round-to-nearest-even, with integer
// operations on its bits (no rounding-mode changes).  Finite inputs only.
// bf16 keeps 8 significant bits and fp32's exponent range; below 2^-126 the
// spacing is 2^-133 (subnormals), handled with an exact power-of-two scaling.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(u >> 63) << 15;
  const int e11 = (int)((u >> 52) & 0x7FF);
  if (e11 > 1023 - 127) {   // |x| >= 2^-126: normal bf16 (or rounds up into one)
    const unsigned long long m = u & 0x7FFFFFFFFFFFFFFFull;
    const unsigned long long r = m + 0xFFFFFFFFFFFull + ((m >> 45) & 1ull);   // RNE at bit 45
    const uint32_t hi = (uint32_t)(r >> 45);            // exp11 (11 bits) | mant7
    return sign | (uint32_t)(((hi >> 7) - (1023 - 127)) << 7) | (hi & 0x7F);
  }
  // |x| < 2^-126: multiple of 2^-133 nearest to |x|, ties to even (exact scaling)
  const double q = rint(fabs(x) * 0x1p133);
  return sign | (uint32_t)q;   // q <= 128; 128 is the smallest normal 0x0080
}

// True when x is within 8 fp64 units in the last place of a bf16 rounding
// midpoint (or in the subnormal range), i.e. when a value known to within
// 8 ulps of x might round differently from x.
__device__ __forceinline__ bool near_bf16_midpoint(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const int e11 = (int)((u >> 52) & 0x7FF);
  const long long d = (long long)(u & 0x1FFFFFFFFFFFull) - (long long)0x100000000000ull;   // low 45 bits - half
  return e11 <= 1023 - 127 || (d >= -8 && d <= 8);
}

// bf16 bits of an fp32 value, rounded to nearest even (hardware conversion).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Rounding fp64 -> fp32 -> bf16 (both to nearest even) gives the bf16 nearest
// to x except when the fp32 value is itself a bf16 midpoint (low 16 bits
// 0x8000).  That test also holds whenever x lies within 8 fp64 ulps of a
// midpoint (the fp32 rounding of such an x is the midpoint), so a false
// result here implies a false near_bf16_midpoint(x) outside the subnormal
// range, and there the two roundings agree as well.
__device__ __forceinline__ bool f32_on_bf16_midpoint(float f) {
  return (__float_as_uint(f) & 0xFFFFu) == 0x8000u;
}

// Position of element k of a 2048-wide activation in pair order.  Within each
// 8-element chunk the order is (0, 2, 4, 6, 1, 3, 5, 7): the even elements are
// the low nibbles of a code dword, the odd ones the high nibbles.
__device__ __forceinline__ int perm_order(int k) {
  int j = k & 7;
  return (k & ~7) | ((j & 1) ? 4 + (j >> 1) : (j >> 1));
}

// ------------------------------------------------------------------ reductions
// Cross-lane moves use DPP (data-parallel primitives: operand routing inside
// the VALU, a few cycles) rather than LDS permutes.  Controls (GFX9 family):
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <- lane 7-i within 8
constexpr int DPP_MIRROR = 0x140;       // lane i <- lane 15-i within 16
constexpr int DPP_BCAST15 = 0x142;      // row r <- lane 15 of row r-1
constexpr int DPP_BCAST31 = 0x143;      // rows 2,3 <- lane 31

// Value of `v` moved by a DPP control; lanes outside row_mask receive 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL, ROW_MASK>(__float_as_uint(v)));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)b), hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

__device__ __forceinline__ float lane_bcast(float v, int lane) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), lane));
}
__device__ __forceinline__ double lane_bcast(double v, int lane) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Sum over each row of 16 lanes; every lane of the row gets the row's sum.
template <typename T>
__device__ __forceinline__ T row16_sum(T v) {
  if constexpr (sizeof(T) == 8) {
    v += dpp_f64<DPP_XOR1>(v);
    v += dpp_f64<DPP_XOR2>(v);
    v += dpp_f64<DPP_HALF_MIRROR>(v);
    v += dpp_f64<DPP_MIRROR>(v);
  } else {
    v += dpp_f32<DPP_XOR1>(v);
    v += dpp_f32<DPP_XOR2>(v);
    v += dpp_f32<DPP_HALF_MIRROR>(v);
    v += dpp_f32<DPP_MIRROR>(v);
  }
  return v;
}

// Sum over the wavefront with a fixed tree (rows of 16, then rows 0+1 and
// 2+3, then all); the total is taken from lane 63 and is the same in every lane.
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  v = row16_sum(v);
  if constexpr (sizeof(T) == 8) {
    v += dpp_f64<DPP_BCAST15, 0xA>(v);
    v += dpp_f64<DPP_BCAST31, 0xC>(v);
  } else {
    v += dpp_f32<DPP_BCAST15, 0xA>(v);
    v += dpp_f32<DPP_BCAST31, 0xC>(v);
  }
  return lane_bcast(v, 63);
}

// Maximum of a 32-bit unsigned key over the wavefront (same in every lane).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<DPP_XOR1>(v));
  v = max(v, dpp_u32<DPP_XOR2>(v));
  v = max(v, dpp_u32<DPP_HALF_MIRROR>(v));
  v = max(v, dpp_u32<DPP_MIRROR>(v));
  v = max(v, dpp_u32<DPP_BCAST15, 0xA>(v));
  v = max(v, dpp_u32<DPP_BCAST31, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Keep the compiler from moving memory operations across this point (used to
// issue prefetch loads before a wait loop).  Emits no instruction.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Workgroup barrier that orders LDS only.  __syncthreads() also orders global
// memory, so each wave first waits for the acknowledgement of every store it
// has in flight; stores that are written through to device memory take
// microseconds to acknowledge.  No kernel here passes data between waves of
// one workgroup through global memory, so the LDS fences suffice.
__device__ __forceinline__ void wg_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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
