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
// log2(l) - ly for a sum l of non-negative terms one of which is 2^ly: l >= 2^ly exactly, so the
// difference is >= 0 wherever the hardware log2 is monotone; a negative rounding artefact is
// returned as 0 (NaN, the poison of an unmatched target, passes through).
__device__ __forceinline__ float log2_ratio(float l, float ly) {
  const float d = flog2(l) - ly;
  return d < 0.f ? 0.f : d;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ float load_value(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_value(const uint16_t* p, int64_t i) { return __uint_as_float(((uint32_t)p[i]) << 16); }

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
// Small logits (|z| <= c / 8) use the tanh series instead, truncated after x^5:
//   tanh(x) = x - x^3/3 + 2 x^5/15 - 17 x^7/315 + ...   (coefficients from the Bernoulli numbers;
// the series alternates with decreasing terms for |x| < pi/2, so the truncation error is below the
// first omitted term). At |x| <= 1/8 that term is at most 17/(315 * 8^6) |x| < 2.1e-7 |x|, i.e.
// |error of s| < 2.6e-8 c: a few float ulps of s at the edge of the range, far below them inside.
// In base 2: s * log2 e = z * Q(z^2), Q(u) = q0 + q1 u + q2 u^2 with q0 = log2 e,
// q1 = -log2 e / (3 c^2), q2 = 2 log2 e / (15 c^4): two fma and two multiplies, no transcendental.
//
// Asymmetric caps: c (the fields above) applies to z >= 0 and cn to z < 0, each side with its own
// constants (series coefficients included); 0 leaves that side uncapped. The series then needs
// both sides capped and is taken below the smaller cap / 8 (thr); the fixed log-sum-exp shift is
// M = c log2 e.
struct Softcap {
  float c;        // cap (0 = none); the cap of z >= 0 when asym
  float alpha;    // 2 log2 e / c
  float M;        // c log2 e
  float K;        // -2 M
  float invK;     // 1 / K
  float invM;     // 1 / M
  float q0, q1, q2;  // series coefficients of s * log2 e in powers of z^2
  float thr;      // series used when every |z| of a block is <= thr (c / 8; 0 = never)
  bool fixed;     // fixed log-sum-exp shift M (every side capped, caps <= kFixedShiftMaxCap)
  bool asym;      // separate cap cn for z < 0
  float cn, alpha_n, M_n, invK_n;   // the z < 0 side (asym only)
  float q1n, q2n;                    // series coefficients of the z < 0 side (asym only; q0 is shared)
  // z < 0 side of the stored training gradient (asym only): with t = s log2 e - M, the slope
  // 1 - (s / cn)^2 is -(t + dza_n)(t + dzb_n) dzw_n / M^2 (dza_n = M - M_n, dzb_n = M + M_n,
  // dzw_n = M^2 / M_n^2), the form of the z >= 0 side, -t (t - K) / M^2, with other constants
  float dza_n, dzb_n, dzw_n, invM_n;
  __host__ static Softcap make(float cap) { return make(cap, cap); }
  __host__ static Softcap make(float cap, float cap_neg) {
    Softcap s{};
    const double l2e = 1.4426950408889634;
    s.c = cap;
    s.asym = cap != cap_neg;
    if (cap > 0.f) {
      const double c = cap;
      s.alpha = (float)(2.0 * l2e / c);
      s.M = (float)(c * l2e);
      s.K = -2.0f * s.M;
      s.invK = 1.0f / s.K;
      s.invM = 1.0f / s.M;
      s.q0 = (float)l2e;
      s.q1 = (float)(-l2e / (3.0 * c * c));
      s.q2 = (float)(2.0 * l2e / (15.0 * c * c * c * c));
      s.thr = cap >= 0.01f ? cap / 8.0f : 0.0f;
    }
    if (s.asym && cap_neg > 0.f) {
      const double cn = cap_neg;
      s.cn = cap_neg;
      s.alpha_n = (float)(2.0 * l2e / cn);
      s.M_n = (float)(cn * l2e);
      s.invK_n = 1.0f / (-2.0f * s.M_n);
      s.q1n = (float)(-l2e / (3.0 * cn * cn));
      s.q2n = (float)(2.0 * l2e / (15.0 * cn * cn * cn * cn));
      const double Mp = cap > 0.f ? (double)cap * l2e : 0.0, Mn = cn * l2e;
      s.dza_n = (float)(Mp - Mn);
      s.dzb_n = (float)(Mp + Mn);
      s.dzw_n = (float)((Mp * Mp) / (Mn * Mn));
      s.invM_n = (float)(1.0 / Mn);
    }
    // asymmetric caps: the series on both sides needs both capped, below the smaller cap / 8
    if (s.asym) s.thr = (cap >= 0.01f && cap_neg >= 0.01f) ? (cap < cap_neg ? cap : cap_neg) / 8.0f : 0.0f;
    s.fixed = cap > 0.f && cap <= kFixedShiftMaxCap &&
              (!s.asym || (cap_neg > 0.f && cap_neg <= kFixedShiftMaxCap));
    return s;
  }
  // some side of the cap is active
  __host__ __device__ bool capped() const { return c > 0.f || (asym && cn > 0.f); }
};

// s * log2 e by the series (valid for |z| <= c / 8).
__device__ __forceinline__ float capped_log2_series(float z, const Softcap& sc) {
  const float u = z * z;
  const float q = __builtin_fmaf(__builtin_fmaf(sc.q2, u, sc.q1), u, sc.q0);
  return z * q;
}

// (s - M) * log2 e for c > 0, i.e. K * r; overflow-safe: e -> inf gives 0 (s = c), e -> 0 gives K.
__device__ __forceinline__ float capped_shifted(float z, float alpha, float invK) {
  float e = fexp2(z * alpha);
  return frcp(__builtin_fmaf(e, invK, invK));
}

// s * log2 e and ds/dz = 1 - (s / c_side)^2 for either cap form (exact, no series).
__device__ __forceinline__ void capped_log2_slope(float z, const Softcap& sc, float& s2, float& slope) {
  const bool neg = sc.asym && z < 0.f;
  const float c = neg ? sc.cn : sc.c;
  if (c > 0.f) {
    const float invK = neg ? sc.invK_n : sc.invK;
    const float rk = capped_shifted(z, neg ? sc.alpha_n : sc.alpha, invK);   // K r
    s2 = (neg ? sc.M_n : sc.M) + rk;
    const float rr = rk * invK;
    slope = rr * __builtin_fmaf(-4.0f, rr, 4.0f);                            // 4 r (1 - r)
  } else {
    s2 = z * kLog2e;
    slope = 1.0f;
  }
}

// Capped logit in base 2 (s * log2 e).
__device__ __forceinline__ float capped_log2(float z, const Softcap& sc) {
  if (!sc.asym) {
    if (sc.c > 0.f) return sc.M + capped_shifted(z, sc.alpha, sc.invK);
    return z * kLog2e;
  }
  float s2, slope;
  capped_log2_slope(z, sc, s2, slope);
  return s2;
}

// (s * log2 e) - M for the fixed-shift log-sum-exp (sc.fixed: every side capped).
__device__ __forceinline__ float capped_shifted_sc(float z, const Softcap& sc) {
  if (!sc.asym) return capped_shifted(z, sc.alpha, sc.invK);
  return z < 0.f ? (sc.M_n - sc.M) + capped_shifted(z, sc.alpha_n, sc.invK_n)
                 : capped_shifted(z, sc.alpha, sc.invK);
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
