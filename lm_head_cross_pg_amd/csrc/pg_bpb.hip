// Bits per byte over the scored rows: sum of nats (float64), sum of UTF-8 bytes of the targets
// (int64) and the number of scored rows, then bpb = sum_nats / (ln 2 * sum_bytes).
// (README introduction: the score is compression in bits per byte, independent of the tokenizer; tproger
// article, "Правила и метрика"; byte counts per position as in the README leaderboard's PR #1736
// row: byte counts carried per position beside the tokens.)
//
// Two launches, no atomics: every workgroup reduces a fixed contiguous range of rows in a fixed
// order into one partial, then a single workgroup adds the partials in index order. The result is
// bitwise reproducible from run to run.
#include "pg_common.h"
#include "pg_internal.h"

namespace pg {

constexpr int kBpbThreads = 256;
constexpr int kBpbMaxBlocks = 1024;
constexpr int64_t kBpbRowsPerBlockMin = kBpbThreads;   // one row per thread up to 256 Ki rows

struct BpbPartial {
  double nats;
  long long bytes;
  long long count;
};

// Workgroup sum in a fixed order: a butterfly within each wave, then the four wave sums in wave
// order. Thread 0 returns the result.
__device__ BpbPartial block_reduce(BpbPartial v) {
  __shared__ BpbPartial sh[kBpbThreads / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    v.nats += __shfl_xor(v.nats, off);
    v.bytes += __shfl_xor(v.bytes, off);
    v.count += __shfl_xor(v.count, off);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    v = sh[0];
#pragma unroll
    for (int w = 1; w < kBpbThreads / 64; ++w) {
      v.nats += sh[w].nats;
      v.bytes += sh[w].bytes;
      v.count += sh[w].count;
    }
  }
  return v;
}

__global__ __launch_bounds__(kBpbThreads) void bpb_partial_kernel(const float* nats, const int32_t* target,
                                                                  const uint8_t* mask, const int32_t* byte_len,
                                                                  const int32_t* byte_per_pos, int64_t T, int V,
                                                                  int64_t rows_per_block, BpbPartial* part) {
  const int64_t b = (int64_t)blockIdx.x * rows_per_block;
  const int64_t e = (b + rows_per_block < T) ? b + rows_per_block : T;
  BpbPartial acc{0.0, 0, 0};
  for (int64_t t = b + threadIdx.x; t < e; t += kBpbThreads) {
    if (mask && !mask[t]) continue;
    acc.nats += (double)nats[t];
    acc.count += 1;
    if (byte_per_pos) {
      acc.bytes += byte_per_pos[t];
    } else {
      const int y = target[t];
      if (y >= 0 && y < V) acc.bytes += byte_len[y];   // out of range: no bytes (its nats are NaN)
    }
  }
  acc = block_reduce(acc);
  if (threadIdx.x == 0) part[blockIdx.x] = acc;
}

// accumulate: out[0..2] already hold running sums (of earlier calls in stream order); this call's
// sums are added to them and out[3] is the bits per byte of the running sums.
__global__ __launch_bounds__(kBpbThreads) void bpb_final_kernel(const BpbPartial* part, int nblocks, double* out,
                                                                int accumulate) {
  BpbPartial acc{0.0, 0, 0};
  for (int i = threadIdx.x; i < nblocks; i += kBpbThreads) {
    acc.nats += part[i].nats;
    acc.bytes += part[i].bytes;
    acc.count += part[i].count;
  }
  acc = block_reduce(acc);
  if (threadIdx.x == 0) {
    double sum_nats = acc.nats;
    double sum_bytes = (double)acc.bytes;   // exact below 2^53 bytes
    double count = (double)acc.count;
    if (accumulate) {
      sum_nats += out[0];
      sum_bytes += out[1];
      count += out[2];
    }
    out[0] = sum_nats;
    out[1] = sum_bytes;
    out[2] = count;
    out[3] = sum_nats / (0.6931471805599453 * sum_bytes);
  }
}

static void bpb_grid(int64_t T, int& blocks, int64_t& rows_per_block) {
  int64_t b = (T + kBpbRowsPerBlockMin - 1) / kBpbRowsPerBlockMin;
  if (b > kBpbMaxBlocks) b = kBpbMaxBlocks;
  if (b < 1) b = 1;
  rows_per_block = (T + b - 1) / b;
  if (rows_per_block < 1) rows_per_block = 1;
  blocks = (int)b;
}

BpbWorkspace bpb_workspace(int64_t T) {
  (void)T;
  BpbWorkspace L;
  L.part = 0;
  L.total = align256(sizeof(BpbPartial) * kBpbMaxBlocks);
  return L;
}

hipError_t launch_bpb(const float* nats, const int32_t* target, const uint8_t* mask,
                      const int32_t* byte_len, const int32_t* byte_per_pos, int64_t T, int32_t V,
                      double* out, char* ws, hipStream_t st, bool accumulate) {
  int blocks;
  int64_t rpb;
  bpb_grid(T, blocks, rpb);
  BpbPartial* part = reinterpret_cast<BpbPartial*>(ws + bpb_workspace(T).part);
  hipLaunchKernelGGL(bpb_partial_kernel, dim3(blocks), dim3(kBpbThreads), 0, st, nats, target, mask, byte_len,
                     byte_per_pos, T, V, rpb, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bpb_final_kernel, dim3(1), dim3(kBpbThreads), 0, st, part, blocks, out, (int)accumulate);
  return hipGetLastError();
}

}  // namespace pg
