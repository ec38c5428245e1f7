// Per-row symmetric int8 form of the tied embedding, for scoring a quantised head: the model is
// quantised to fit the artifact (trios issue #19, approach table, "Квантование": INT4/INT8; README
// leaderboard, GPTQ and LQER rows), and the tied embedding is then both the input lookup and the
// output head. The pages give no format; the one used here is
//   scale[v] = max_d |E[v, d]| / 127                       (float32, correctly rounded division)
//   q[v, d]  = round_half_even(E[v, d] / scale[v])          (int8 in [-127, 127]; 0 when scale = 0)
//   E'[v, d] = bf16_round_half_even(float32(q[v, d]) * scale[v])   (the dequantised embedding)
// so that the head computes on exactly E' and a float64 reference can reproduce it bit for bit.
// Both kernels are HBM-bound elementwise passes (one wave per row for the quantiser).
#include "pg_common.h"
#include "pg_internal.h"

namespace pg {

// One wave per row: lanes stride over the row, reduce max |E| across the wave, then write q.
template <typename TIn>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const TIn* E, int V, int D, int8_t* q, float* scale) {
  const int lane = threadIdx.x & 63;
  const int64_t v = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (v >= V) return;
  const TIn* row = E + v * D;
  float m = 0.f;
  for (int d = lane; d < D; d += 64) m = fmaxf(m, fabsf(load_value(row, d)));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const float s = __fdiv_rn(m, 127.0f);
  for (int d = lane; d < D; d += 64) {
    float r = 0.f;
    if (s > 0.f) r = __builtin_rintf(__fdiv_rn(load_value(row, d), s));
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    q[v * D + d] = (int8_t)r;
  }
  if (lane == 0) scale[v] = s;
}

// E'[v, d] = bf16(float(q[v, d]) * scale[v]), 8 elements per thread.
__global__ __launch_bounds__(256) void dequantize_rows_kernel(const int8_t* q, const float* scale, int64_t n8, int D,
                                                              uint16_t* E) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e0 = i * 8;
    const float s = scale[e0 / D];
    const uint2 raw = reinterpret_cast<const uint2*>(q)[i];
    const uint32_t w[2] = {raw.x, raw.y};
    uint16_t out[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int8_t qi = (int8_t)((w[k >> 2] >> (8 * (k & 3))) & 0xff);
      out[k] = f32_to_bf16((float)qi * s);
    }
    uint4 o;
    o.x = out[0] | ((uint32_t)out[1] << 16);
    o.y = out[2] | ((uint32_t)out[3] << 16);
    o.z = out[4] | ((uint32_t)out[5] << 16);
    o.w = out[6] | ((uint32_t)out[7] << 16);
    reinterpret_cast<uint4*>(E)[i] = o;
  }
}

hipError_t launch_quantize(const void* E, int32_t dtype, int32_t V, int32_t D, int8_t* q, float* scale,
                           hipStream_t st) {
  const unsigned blocks = (unsigned)((V + 3) / 4);
  if (dtype == 0)
    hipLaunchKernelGGL(quantize_rows_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st, (const uint16_t*)E, V, D, q,
                       scale);
  else
    hipLaunchKernelGGL(quantize_rows_kernel<float>, dim3(blocks), dim3(256), 0, st, (const float*)E, V, D, q, scale);
  return hipGetLastError();
}

hipError_t launch_dequantize(const int8_t* q, const float* scale, int32_t V, int32_t D, uint16_t* E, hipStream_t st) {
  const int64_t n8 = (int64_t)V * D / 8;
  hipLaunchKernelGGL(dequantize_rows_kernel, dim3(stride_blocks(n8, 256)), dim3(256), 0, st, q, scale, n8, D, E);
  return hipGetLastError();
}

}  // namespace pg
