// Backward of the fused tied LM head + logit softcap + cross-entropy for gfx950.
//
// L = g * sum over scored rows of nats (repo-explainer, "The Baseline Is a Map": loss.backward()).
// With p = softmax(s) per row and s = c tanh(z / c):
//   dZ[t, v] = (p[t, v] - [v == y[t]]) * (1 - (s / c)^2)   (g is applied later, in float32)
//   dH = g * dZ . E          dE = g * dZ^T . H   (LM-head part of the tied embedding's gradient)
// The logits are recomputed from H and E with the lse of the forward; dZ is written once to the
// workspace in bf16 and read by the two products.
#include "pg_common.h"
#include "pg_internal.h"

namespace pg {

template <typename TIn>
__device__ __forceinline__ float bload(const TIn* p, int64_t i);
template <>
__device__ __forceinline__ float bload<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float bload<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

// dZ of one row per wave (plain vector code; any dtype and width).
template <typename TIn>
__global__ __launch_bounds__(256) void dz_generic_kernel(const TIn* H, const TIn* E, const int32_t* target,
                                                         const float* lse, const int32_t* rows,
                                                         const int32_t* n_dev, int64_t n_host, int D, int V,
                                                         Softcap sc, uint16_t* dz) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t n = n_dev ? (int64_t)(*n_dev) : n_host;
  if (i >= n) return;
  const int64_t r = rows ? (int64_t)rows[i] : i;
  const TIn* hrow = H + r * D;
  const int y = target[r];
  const float lse2 = lse[r] * kLog2e;
  for (int v = lane; v < V; v += 64) {
    const TIn* erow = E + (int64_t)v * D;
    float z = 0.f;
    for (int d = 0; d < D; ++d) z = __builtin_fmaf(bload(hrow, d), bload(erow, d), z);
    float p, slope;
    if (sc.c > 0.f) {
      const float rk = capped_shifted(z, sc.alpha, sc.invK);   // K r
      p = fexp2(sc.M + rk - lse2);
      const float rr = rk * sc.invK;                            // r = 1 / (1 + e^(2z/c))
      slope = 4.0f * rr * (1.0f - rr);                          // 1 - tanh^2 = 4 r (1 - r)
    } else {
      p = fexp2(z * kLog2e - lse2);
      slope = 1.0f;
    }
    const float g = (v == y) ? p - 1.0f : p;
    dz[i * V + v] = f32_to_bf16(g * slope);
  }
}

// dH[rows[i], d] = g * sum_v dZ[i, v] E[v, d]: one thread per output (plain vector code).
template <typename TIn>
__global__ __launch_bounds__(256) void dh_generic_kernel(const uint16_t* dz, const TIn* E, const int32_t* rows,
                                                         const int32_t* n_dev, int64_t n_host, int D, int V,
                                                         float g, float* dH) {
  const int64_t n = n_dev ? (int64_t)(*n_dev) : n_host;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = idx / D;
  const int d = (int)(idx % D);
  if (i >= n) return;
  float acc = 0.f;
  for (int v = 0; v < V; ++v) acc = __builtin_fmaf(bf16_to_f32(dz[i * V + v]), bload(E, (int64_t)v * D + d), acc);
  const int64_t r = rows ? (int64_t)rows[i] : i;
  dH[r * D + d] = g * acc;
}

// dE[v, d] = g * sum_i dZ[i, v] H[rows[i], d]: one thread per output (plain vector code).
template <typename TIn>
__global__ __launch_bounds__(256) void de_generic_kernel(const uint16_t* dz, const TIn* H, const int32_t* rows,
                                                         const int32_t* n_dev, int64_t n_host, int D, int V,
                                                         float g, float* dE) {
  const int64_t n = n_dev ? (int64_t)(*n_dev) : n_host;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t v = idx / D;
  const int d = (int)(idx % D);
  if (v >= V) return;
  float acc = 0.f;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t r = rows ? (int64_t)rows[i] : i;
    acc = __builtin_fmaf(bf16_to_f32(dz[i * V + v]), bload(H, r * D + d), acc);
  }
  dE[v * D + d] = g * acc;
}

// Zero the dH rows of unscored positions.
__global__ __launch_bounds__(256) void zero_unscored_kernel(const uint8_t* mask, int64_t T, int D, float* dH) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * D) return;
  if (!mask[idx / D]) dH[idx] = 0.f;
}

// ------------------------------------------------------------------------------------ host side

constexpr int kDeSplit = 4;

BwdWorkspace bwd_workspace(int64_t T, int32_t D, int32_t V) {
  BwdWorkspace L;
  size_t o = 0;
  L.n_rows = o; o += 256;
  L.rows = o; o += align256((size_t)T * 4);
  L.dz = o; o += align256((size_t)T * (size_t)V * 2);
  L.de_part = o; o += align256((size_t)kDeSplit * (size_t)V * (size_t)D * 4);
  L.total = o;
  return L;
}

hipError_t launch_bwd(const void* H, const void* E, int32_t dtype, const int32_t* target,
                      const uint8_t* mask, const float* lse, int64_t T, int32_t D, int32_t V,
                      float softcap, float grad_scale, float* dH, float* dE, char* ws,
                      const DeviceInfo& dev, hipStream_t st) {
  (void)dev;
  const BwdWorkspace L = bwd_workspace(T, D, V);
  const Softcap sc = Softcap::make(softcap);
  const int32_t* rows = nullptr;
  const int32_t* n_dev = nullptr;
  if (mask && T > 0) {
    FwdWorkspace F{};
    F.rows = L.rows;
    F.n_rows = L.n_rows;
    hipError_t e = launch_compact_rows(mask, T, ws, F, nullptr, nullptr, st);
    if (e != hipSuccess) return e;
    rows = reinterpret_cast<const int32_t*>(ws + L.rows);
    n_dev = reinterpret_cast<const int32_t*>(ws + L.n_rows);
    const int64_t tot = T * D;
    hipLaunchKernelGGL(zero_unscored_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, mask, T, D, dH);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  uint16_t* dz = reinterpret_cast<uint16_t*>(ws + L.dz);
  const unsigned rblocks = (unsigned)((T + 3) / 4);
  const unsigned hblocks = (unsigned)((T * D + 255) / 256);
  const unsigned eblocks = (unsigned)(((int64_t)V * D + 255) / 256);
  if (T > 0) {
    if (dtype == 0) {
      hipLaunchKernelGGL(dz_generic_kernel<uint16_t>, dim3(rblocks), dim3(256), 0, st, (const uint16_t*)H,
                         (const uint16_t*)E, target, lse, rows, n_dev, T, D, V, sc, dz);
      hipLaunchKernelGGL(dh_generic_kernel<uint16_t>, dim3(hblocks), dim3(256), 0, st, dz, (const uint16_t*)E,
                         rows, n_dev, T, D, V, grad_scale, dH);
    } else {
      hipLaunchKernelGGL(dz_generic_kernel<float>, dim3(rblocks), dim3(256), 0, st, (const float*)H,
                         (const float*)E, target, lse, rows, n_dev, T, D, V, sc, dz);
      hipLaunchKernelGGL(dh_generic_kernel<float>, dim3(hblocks), dim3(256), 0, st, dz, (const float*)E,
                         rows, n_dev, T, D, V, grad_scale, dH);
    }
  }
  if (dtype == 0)
    hipLaunchKernelGGL(de_generic_kernel<uint16_t>, dim3(eblocks), dim3(256), 0, st, dz, (const uint16_t*)H,
                       rows, n_dev, T, D, V, grad_scale, dE);
  else
    hipLaunchKernelGGL(de_generic_kernel<float>, dim3(eblocks), dim3(256), 0, st, dz, (const float*)H,
                       rows, n_dev, T, D, V, grad_scale, dE);
  return hipGetLastError();
}

}  // namespace pg
