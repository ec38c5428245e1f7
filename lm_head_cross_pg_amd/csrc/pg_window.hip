// Sliding-window evaluation of a token stream with score-first test-time training, on gfx950.
//
// Sliding-window evaluation scores each next-token prediction with a long context: windows of
// `window` tokens advance by `stride` tokens, and each window scores only the predictions no earlier
// window has scored (parameter-golf README leaderboard, "Sliding Window Eval" row: stride 64,
// each scored token with a long context). Score-first test-time training adapts the model only on
// validation chunks that have already been scored (README leaderboard, "Legal Score-First TTT"
// rows, and the row whose test-time training runs in phases over validation chunks already scored; HYDRA Golf site, leaderboard entry
// #2, "Score-First TTT").
//
// Schedule (predictions p = 0 .. n_tokens - 2, prediction p being token p + 1 after tokens 0..p):
//   window w covers input positions w stride .. w stride + window - 1;
//   window 0 scores p in [0, window); window w >= 1 scores p in [w stride + window - stride,
//   w stride + window), the predictions it adds, each with at least window - stride tokens of
//   context. Every prediction is scored exactly once, and the last window is the first whose range
//   reaches n_tokens - 2.
// A batch of n_windows consecutive windows is laid out as n_windows x window rows: row (b, r) is
// input position (first_window + b) stride + r. The kernels below build its targets and score mask,
// accumulate bits per byte across batches, and apply a plain SGD step to the tied embedding.
#include "pg_common.h"
#include "pg_internal.h"

namespace pg {

// Targets and score mask of a batch of windows, one row per thread, grid-stride.
__global__ __launch_bounds__(256) void window_rows_kernel(const int32_t* tokens, int64_t n_tokens, int32_t window,
                                                          int32_t stride, int64_t first_window, int64_t rows,
                                                          int32_t* target, uint8_t* mask) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t w = first_window + i / window;
    const int32_t r = (int32_t)(i % window);
    const int64_t p = w * stride + r;                 // input position; it predicts token p + 1
    const bool in_stream = p + 1 < n_tokens;
    target[i] = in_stream ? tokens[p + 1] : 0;
    mask[i] = (in_stream && (w == 0 || r >= window - stride)) ? 1 : 0;
  }
}

// SGD on float32 master weights and their bf16 copy: u = lr g and w = w - u, each rounded once to
// float32, then the bf16 copy by round-to-nearest-even. Contraction is switched off so that the
// compiler keeps the two roundings (it fuses them into one fma otherwise) and the step is
// reproducible operation by operation.
__global__ __launch_bounds__(256) void sgd_step_kernel(float* master, const float* grad, float lr, int64_t n,
                                                       uint16_t* out) {
#pragma clang fp contract(off)
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const float u = lr * grad[i];
    const float w = master[i] - u;
    master[i] = w;
    out[i] = f32_to_bf16(w);
  }
}

int64_t window_count(int64_t n_tokens, int32_t window, int32_t stride) {
  const int64_t n_pred = n_tokens - 1;
  if (n_pred <= 0) return 0;
  if (n_pred <= window) return 1;
  return 1 + (n_pred - window + stride - 1) / stride;
}

// Predictions scored by windows 0 .. k - 1: the frontier after window k - 1, min(n_pred,
// (k - 1) stride + window) (each window scores the run from the previous frontier to its end).
static int64_t window_frontier(int64_t n_pred, int32_t window, int32_t stride, int64_t k) {
  if (k <= 0 || n_pred <= 0) return 0;
  const int64_t end = (k - 1) * stride + window;
  return end < n_pred ? end : n_pred;
}

int64_t window_scored(int64_t n_tokens, int32_t window, int32_t stride, int64_t first_window, int64_t n_windows) {
  const int64_t n_pred = n_tokens - 1;
  const int64_t count = window_count(n_tokens, window, stride);
  const int64_t a = first_window < count ? first_window : count;
  const int64_t b = n_windows < count - a ? a + n_windows : count;
  return window_frontier(n_pred, window, stride, b) - window_frontier(n_pred, window, stride, a);
}

hipError_t launch_window_rows(const int32_t* tokens, int64_t n_tokens, int32_t window, int32_t stride,
                              int64_t first_window, int64_t n_windows, int32_t* target, uint8_t* mask,
                              hipStream_t st) {
  const int64_t rows = n_windows * window;
  hipLaunchKernelGGL(window_rows_kernel, dim3(stride_blocks(rows, 256)), dim3(256), 0, st, tokens, n_tokens, window,
                     stride, first_window, rows, target, mask);
  return hipGetLastError();
}

hipError_t launch_sgd_step(float* master, const float* grad, float lr, int64_t n, uint16_t* out, hipStream_t st) {
  hipLaunchKernelGGL(sgd_step_kernel, dim3(stride_blocks(n, 256)), dim3(256), 0, st, master, grad, lr, n, out);
  return hipGetLastError();
}

}  // namespace pg
