// Shared device-side types and helpers of the gfx950 kernels (internal header).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Softcaps up to this value use a fixed log-sum-exp shift: with |s| <= c every term
// exp2((s - c) * log2 e) lies in [2^(-2 c log2 e), 1], which stays a normal float for c <= 40.
constexpr float kFixedShiftMaxCap = 40.0f;

// Rows of the token tile one workgroup owns (4 waves x 64 rows) and vocabulary rows per tile.
constexpr int kRowsPerWG = 256;
constexpr int kVocabTile = 64;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even float -> bf16 bit pattern (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Softcap constants in base 2. With a = z * alpha, e = 2^a, r = 1 / (1 + e):
//   tanh(z / c) = 1 - 2 r,  s * log2 e = M + K r  with M = c log2 e and K = -2 M.
// K r is evaluated as rcp(e / K + 1 / K), i.e. one fma and one reciprocal.
//
// Small logits (|z| <= c / 8) use the tanh series instead, truncated after x^7:
//   tanh(x) = x - x^3/3 + 2 x^5/15 - 17 x^7/315 + O(x^9)   (coefficients from the Bernoulli
// numbers); at |x| <= 1/8 the first omitted term, 62 x^9/2835, is below 1.4e-9 |x|, far under float
// rounding. In base 2: s * log2 e = z * Q(z^2), Q(u) = q0 + q1 u + q2 u^2 + q3 u^3 with
// q0 = log2 e, q1 = -log2 e / (3 c^2), q2 = 2 log2 e / (15 c^4), q3 = -17 log2 e / (315 c^6):
// three fma and two multiplies, no transcendental.
struct Softcap {
  float c;        // cap (0 = none)
  float alpha;    // 2 log2 e / c
  float M;        // c log2 e
  float K;        // -2 M
  float invK;     // 1 / K
  float invM;     // 1 / M
  float q0, q1, q2, q3;  // series coefficients of s * log2 e in powers of z^2
  float thr;      // series used when every |z| of a block is <= thr (c / 8; 0 = never)
  bool fixed;     // fixed log-sum-exp shift M (0 < c <= kFixedShiftMaxCap)
  __host__ static Softcap make(float cap) {
    Softcap s;
    s.c = cap;
    if (cap > 0.f) {
      const double c = cap, l2e = 1.4426950408889634;
      s.alpha = (float)(2.0 * l2e / c);
      s.M = (float)(c * l2e);
      s.K = -2.0f * s.M;
      s.invK = 1.0f / s.K;
      s.invM = 1.0f / s.M;
      s.q0 = (float)l2e;
      s.q1 = (float)(-l2e / (3.0 * c * c));
      s.q2 = (float)(2.0 * l2e / (15.0 * c * c * c * c));
      s.q3 = (float)(-17.0 * l2e / (315.0 * c * c * c * c * c * c));
      s.thr = (cap >= 0.01f) ? cap / 8.0f : 0.0f;
      s.fixed = cap <= kFixedShiftMaxCap;
    } else {
      s.alpha = 0.f; s.M = 0.f; s.K = 0.f; s.invK = 0.f; s.invM = 0.f;
      s.q0 = s.q1 = s.q2 = s.q3 = 0.f; s.thr = 0.f; s.fixed = false;
    }
    return s;
  }
};

// s * log2 e by the series (valid for |z| <= c / 8).
__device__ __forceinline__ float capped_log2_series(float z, const Softcap& sc) {
  const float u = z * z;
  const float q = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(sc.q3, u, sc.q2), u, sc.q1), u, sc.q0);
  return z * q;
}

// (s - M) * log2 e for c > 0, i.e. K * r; overflow-safe: e -> inf gives 0 (s = c), e -> 0 gives K.
__device__ __forceinline__ float capped_shifted(float z, float alpha, float invK) {
  float e = fexp2(z * alpha);
  return frcp(__builtin_fmaf(e, invK, invK));
}

// Capped logit in base 2 (s * log2 e).
__device__ __forceinline__ float capped_log2(float z, const Softcap& sc) {
  if (sc.c > 0.f) return sc.M + capped_shifted(z, sc.alpha, sc.invK);
  return z * kLog2e;
}

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Merge two (max, sum) pairs of a base-2 log-sum-exp.
__device__ __forceinline__ void lse_merge(float& m, float& l, float m2, float l2) {
  float mn = fmaxf(m, m2);
  if (mn == -INFINITY) { l = l + l2; return; }
  l = l * fexp2(m - mn) + l2 * fexp2(m2 - mn);
  m = mn;
}

}  // namespace pg
