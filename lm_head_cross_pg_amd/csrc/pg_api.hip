// C ABI of the library: host-side validation, workspace sizing, device check and dispatch.
// Validation happens before anything is enqueued and has no side effects.
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/pg_lmhead.h"
#include "pg_internal.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, -1 = not usable; the CU count is cached beside it.
std::atomic<int> g_dev_state[kMaxDevices];
std::atomic<int> g_dev_cus[kMaxDevices];

pg_status device_check(pg::DeviceInfo& info) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return PG_ERR_DEVICE;
  }
  if (dev >= kMaxDevices) return PG_ERR_DEVICE;
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return PG_ERR_DEVICE;
    }
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    st = ok ? 1 : -1;
    g_dev_state[dev].store(st, std::memory_order_release);
  }
  if (st != 1) return PG_ERR_DEVICE;
  info.cu_count = g_dev_cus[dev].load(std::memory_order_relaxed);
  return PG_OK;
}

inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Scratch of pg_lmhead_ce_fwd_noalloc: a file-scope device array that every GPU the library runs
// on holds until the process ends. Its size covers the forward's workspace for T <= 2^20 rows
// (scored-row list, target terms and per-split partial sums: 16 MiB + 256 B there), whatever D and
// V are. In host code `scratch` is only a stand-in for the symbol: its device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and only that address is
// handed to kernels.
constexpr size_t kScratchBytes = ((size_t)16 << 20) + 256;
__device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of this device's scratch array (the caller has run device_check).
pg_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return PG_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return PG_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PG_OK;
}

// Rows up to 2^31 - 256: every row index fits an int32, and the MFMA kernels' grids of one
// 512-thread workgroup per 256 rows stay within the 2^32 - 1 work items of a launch.
constexpr int64_t kMaxRows = 2147483648LL - 256;
constexpr int32_t kMaxWidth = 1 << 20;

pg_status check_shape(int64_t T, int32_t D, int32_t V) {
  if (T < 0 || T > kMaxRows || D < 1 || D > kMaxWidth || V < 1 || V > kMaxWidth) return PG_ERR_SHAPE;
  return PG_OK;
}

// The backward's products on the MFMA path: the dH grid grows with T D (256 x 256 output tiles).
pg_status check_bwd_shape(int64_t T, int32_t D, int32_t V) {
  if (!pg::mfma_width(D)) return PG_OK;   // vector kernels: grid-stride loops
  if (pg::gemm_grid_x(T, D, false) > pg::kMaxGrid512 || pg::gemm_grid_x(V, D, true) > pg::kMaxGrid512)
    return PG_ERR_SHAPE;
  return PG_OK;
}

pg_status check_softcap(float c) {
  if (!std::isfinite(c) || c < 0.f) return PG_ERR_SOFTCAP;
  return PG_OK;
}

}  // namespace

extern "C" {

int32_t pg_abi_version(void) { return PG_ABI_VERSION; }

const char* pg_status_str(pg_status s) {
  switch (s) {
    case PG_OK: return "ok";
    case PG_ERR_NULL: return "a required pointer is NULL";
    case PG_ERR_SHAPE: return "invalid shape (T < 0, D < 1, V < 1 or beyond the supported range)";
    case PG_ERR_DTYPE: return "unknown dtype";
    case PG_ERR_SOFTCAP: return "softcap negative or not finite, or grad_scale or learning rate not finite";
    case PG_ERR_WORKSPACE: return "workspace smaller than pg_workspace_bytes()";
    case PG_ERR_ALIGN: return "pointer not 16-byte aligned";
    case PG_ERR_DEVICE: return "no HIP device, or the current device is not gfx950";
    case PG_ERR_HIP: return "HIP runtime or kernel launch failure";
    case PG_ERR_SCRATCH: return "the shape needs more scratch than the static buffer of the allocation-free entry holds";
    default: return "unknown status";
  }
}

size_t pg_workspace_bytes(int32_t op, int64_t T, int32_t D, int32_t V) {
  if (check_shape(T, D, V) != PG_OK) return 0;
  switch (op) {
    case PG_OP_FWD: return pg::fwd_workspace(T, D, V).total;
    case PG_OP_BWD:
      if (check_bwd_shape(T, D, V) != PG_OK) return 0;
      return pg::bwd_workspace(T, D, V).total;
    case PG_OP_BPB: return pg::bpb_workspace(T).total;
    case PG_OP_FWD_BWD:
      if (check_bwd_shape(T, D, V) != PG_OK) return 0;
      return pg::train_workspace(T, D, V).total;
    case PG_OP_FWD_Q8:
      if (D % 8 != 0) return 0;
      return pg::align256((size_t)V * (size_t)D * 2) + pg::fwd_workspace(T, D, V).total;
    default: return 0;
  }
}

// The forward's arguments other than the workspace (host only, in the order of the status codes).
static pg_status fwd_args(const void* hidden, const void* embed, int32_t dtype, const int32_t* target,
                          const uint8_t* score_mask, int64_t T, int32_t D, int32_t V, float cap_pos, float cap_neg,
                          const float* nats, const float* lse) {
  pg_status s;
  if ((s = check_shape(T, D, V)) != PG_OK) return s;
  if (T > 0 && (!hidden || !target || !nats)) return PG_ERR_NULL;
  if (!embed) return PG_ERR_NULL;
  if (dtype != PG_DTYPE_BF16 && dtype != PG_DTYPE_F32) return PG_ERR_DTYPE;
  if ((s = check_softcap(cap_pos)) != PG_OK || (s = check_softcap(cap_neg)) != PG_OK) return s;
  if (misaligned(hidden) || misaligned(embed) || misaligned(target) || misaligned(score_mask) ||
      misaligned(nats) || misaligned(lse))
    return PG_ERR_ALIGN;
  return PG_OK;
}

static pg_status fwd_impl(const void* hidden, const void* embed, int32_t dtype, const int32_t* target,
                          const uint8_t* score_mask, int64_t T, int32_t D, int32_t V, float cap_pos, float cap_neg,
                          float* nats, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  pg_status s;
  if ((s = fwd_args(hidden, embed, dtype, target, score_mask, T, D, V, cap_pos, cap_neg, nats, lse)) != PG_OK)
    return s;
  if (!workspace) return PG_ERR_NULL;
  if (misaligned(workspace)) return PG_ERR_ALIGN;
  if (workspace_bytes < pg_workspace_bytes(PG_OP_FWD, T, D, V)) return PG_ERR_WORKSPACE;
  pg::DeviceInfo dev{};
  if ((s = device_check(dev)) != PG_OK) return s;
  hipError_t e = pg::launch_fwd(hidden, embed, dtype, target, score_mask, T, D, V, cap_pos, cap_neg, nats, lse,
                                static_cast<char*>(workspace), dev, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PG_OK : PG_ERR_HIP;
}

static pg_status bwd_impl(const void* hidden, const void* embed, int32_t dtype, const int32_t* target,
                          const uint8_t* score_mask, const float* lse, int64_t T, int32_t D, int32_t V,
                          float cap_pos, float cap_neg, float grad_scale, float* dhidden, float* dembed,
                          void* workspace, size_t workspace_bytes, void* stream) {
  pg_status s;
  if ((s = check_shape(T, D, V)) != PG_OK || (s = check_bwd_shape(T, D, V)) != PG_OK) return s;
  if (T > 0 && (!hidden || !target || !lse)) return PG_ERR_NULL;   // dhidden may be NULL: no dH
  if (!embed || !dembed || !workspace) return PG_ERR_NULL;
  if (dtype != PG_DTYPE_BF16 && dtype != PG_DTYPE_F32) return PG_ERR_DTYPE;
  if ((s = check_softcap(cap_pos)) != PG_OK || (s = check_softcap(cap_neg)) != PG_OK) return s;
  if (!std::isfinite(grad_scale)) return PG_ERR_SOFTCAP;
  if (misaligned(hidden) || misaligned(embed) || misaligned(target) || misaligned(score_mask) ||
      misaligned(lse) || misaligned(dhidden) || misaligned(dembed) || misaligned(workspace))
    return PG_ERR_ALIGN;
  if (workspace_bytes < pg_workspace_bytes(PG_OP_BWD, T, D, V)) return PG_ERR_WORKSPACE;
  pg::DeviceInfo dev{};
  if ((s = device_check(dev)) != PG_OK) return s;
  hipError_t e = pg::launch_bwd(hidden, embed, dtype, target, score_mask, lse, T, D, V, cap_pos, cap_neg,
                                grad_scale, dhidden, dembed, static_cast<char*>(workspace), dev,
                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PG_OK : PG_ERR_HIP;
}

pg_status pg_lmhead_ce_fwd(const void* hidden, const void* embed, int32_t dtype,
                           const int32_t* target, const uint8_t* score_mask,
                           int64_t T, int32_t D, int32_t V, float softcap,
                           float* nats, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(hidden, embed, dtype, target, score_mask, T, D, V, softcap, softcap, nats, lse, workspace,
                  workspace_bytes, stream);
}

pg_status pg_lmhead_ce_fwd_noalloc(const void* hidden, const void* embed, int32_t dtype,
                                   const int32_t* target, const uint8_t* score_mask,
                                   int64_t T, int32_t D, int32_t V, float softcap,
                                   float* nats, float* lse, void* stream) {
  pg_status s;
  if ((s = fwd_args(hidden, embed, dtype, target, score_mask, T, D, V, softcap, softcap, nats, lse)) != PG_OK)
    return s;
  if (pg::fwd_workspace(T, D, V).total > kScratchBytes) return PG_ERR_SCRATCH;
  pg::DeviceInfo dev{};
  if ((s = device_check(dev)) != PG_OK) return s;
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != PG_OK) return s;
  // the forward writes every scratch entry it reads (row count, scored rows, partial sums) in the
  // same stream first, so nothing has to be cleared between calls
  hipError_t e = pg::launch_fwd(hidden, embed, dtype, target, score_mask, T, D, V, softcap, softcap, nats, lse,
                                static_cast<char*>(ws), dev, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PG_OK : PG_ERR_HIP;
}

pg_status pg_lmhead_ce_bwd(const void* hidden, const void* embed, int32_t dtype,
                           const int32_t* target, const uint8_t* score_mask, const float* lse,
                           int64_t T, int32_t D, int32_t V, float softcap, float grad_scale,
                           float* dhidden, float* dembed,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(hidden, embed, dtype, target, score_mask, lse, T, D, V, softcap, softcap, grad_scale, dhidden,
                  dembed, workspace, workspace_bytes, stream);
}

static pg_status train_impl(const void* hidden, const void* embed, int32_t dtype, const int32_t* target,
                            const uint8_t* score_mask, int64_t T, int32_t D, int32_t V, float cap_pos,
                            float cap_neg, float grad_scale, float* nats, float* lse, float* dhidden,
                            float* dembed, void* workspace, size_t workspace_bytes, void* stream) {
  pg_status s;
  if ((s = check_shape(T, D, V)) != PG_OK || (s = check_bwd_shape(T, D, V)) != PG_OK) return s;
  if (T > 0 && (!hidden || !target || !nats || !lse)) return PG_ERR_NULL;   // dhidden may be NULL: no dH
  if (!embed || !dembed || !workspace) return PG_ERR_NULL;
  if (dtype != PG_DTYPE_BF16 && dtype != PG_DTYPE_F32) return PG_ERR_DTYPE;
  if ((s = check_softcap(cap_pos)) != PG_OK || (s = check_softcap(cap_neg)) != PG_OK) return s;
  if (!std::isfinite(grad_scale)) return PG_ERR_SOFTCAP;
  if (misaligned(hidden) || misaligned(embed) || misaligned(target) || misaligned(score_mask) ||
      misaligned(nats) || misaligned(lse) || misaligned(dhidden) || misaligned(dembed) || misaligned(workspace))
    return PG_ERR_ALIGN;
  if (workspace_bytes < pg_workspace_bytes(PG_OP_FWD_BWD, T, D, V)) return PG_ERR_WORKSPACE;
  pg::DeviceInfo dev{};
  if ((s = device_check(dev)) != PG_OK) return s;
  hipError_t e = pg::launch_train(hidden, embed, dtype, target, score_mask, T, D, V, cap_pos, cap_neg, grad_scale,
                                  nats, lse, dhidden, dembed, static_cast<char*>(workspace), dev,
                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PG_OK : PG_ERR_HIP;
}

pg_status pg_lmhead_ce_fwd_bwd(const void* hidden, const void* embed, int32_t dtype,
                               const int32_t* target, const uint8_t* score_mask,
                               int64_t T, int32_t D, int32_t V, float softcap, float grad_scale,
                               float* nats, float* lse, float* dhidden, float* dembed,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return train_impl(hidden, embed, dtype, target, score_mask, T, D, V, softcap, softcap, grad_scale, nats, lse,
                    dhidden, dembed, workspace, workspace_bytes, stream);
}

pg_status pg_lmhead_ce_fwd_bwd_asym(const void* hidden, const void* embed, int32_t dtype,
                                    const int32_t* target, const uint8_t* score_mask,
                                    int64_t T, int32_t D, int32_t V, float cap_pos, float cap_neg,
                                    float grad_scale, float* nats, float* lse, float* dhidden, float* dembed,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return train_impl(hidden, embed, dtype, target, score_mask, T, D, V, cap_pos, cap_neg, grad_scale, nats, lse,
                    dhidden, dembed, workspace, workspace_bytes, stream);
}

pg_status pg_lmhead_ce_fwd_asym(const void* hidden, const void* embed, int32_t dtype,
                                const int32_t* target, const uint8_t* score_mask,
                                int64_t T, int32_t D, int32_t V, float cap_pos, float cap_neg,
                                float* nats, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_impl(hidden, embed, dtype, target, score_mask, T, D, V, cap_pos, cap_neg, nats, lse, workspace,
                  workspace_bytes, stream);
}

pg_status pg_lmhead_ce_bwd_asym(const void* hidden, const void* embed, int32_t dtype,
                                const int32_t* target, const uint8_t* score_mask, const float* lse,
                                int64_t T, int32_t D, int32_t V, float cap_pos, float cap_neg, float grad_scale,
                                float* dhidden, float* dembed,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(hidden, embed, dtype, target, score_mask, lse, T, D, V, cap_pos, cap_neg, grad_scale, dhidden,
                  dembed, workspace, workspace_bytes, stream);
}

pg_status pg_quantize_q8(const void* embed, int32_t dtype, int32_t V, int32_t D, int8_t* embed_q8,
                         float* embed_scale, void* stream) {
  pg_status s;
  if ((s = check_shape(0, D, V)) != PG_OK) return s;
  if (D % 8 != 0) return PG_ERR_SHAPE;
  if (!embed || !embed_q8 || !embed_scale) return PG_ERR_NULL;
  if (dtype != PG_DTYPE_BF16 && dtype != PG_DTYPE_F32) return PG_ERR_DTYPE;
  if (misaligned(embed) || misaligned(embed_q8) || misaligned(embed_scale)) return PG_ERR_ALIGN;
  pg::DeviceInfo dev{};
  if ((s = device_check(dev)) != PG_OK) return s;
  hipError_t e = pg::launch_quantize(embed, dtype, V, D, embed_q8, embed_scale, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PG_OK : PG_ERR_HIP;
}

pg_status pg_lmhead_ce_fwd_q8(const void* hidden, const int8_t* embed_q8, const float* embed_scale,
                              const int32_t* target, const uint8_t* score_mask,
                              int64_t T, int32_t D, int32_t V, float softcap,
                              float* nats, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream) {
  pg_status s;
  if ((s = check_shape(T, D, V)) != PG_OK) return s;
  if (D % 8 != 0) return PG_ERR_SHAPE;
  if (T > 0 && (!hidden || !target || !nats)) return PG_ERR_NULL;
  if (!embed_q8 || !embed_scale || !workspace) return PG_ERR_NULL;
  if ((s = check_softcap(softcap)) != PG_OK) return s;
  if (misaligned(hidden) || misaligned(embed_q8) || misaligned(embed_scale) || misaligned(target) ||
      misaligned(score_mask) || misaligned(nats) || misaligned(lse) || misaligned(workspace))
    return PG_ERR_ALIGN;
  if (workspace_bytes < pg_workspace_bytes(PG_OP_FWD_Q8, T, D, V)) return PG_ERR_WORKSPACE;
  pg::DeviceInfo dev{};
  if ((s = device_check(dev)) != PG_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  char* fws = ws + pg::align256((size_t)V * (size_t)D * 2);
  hipError_t e;
  // Converting on chip costs every workgroup the conversion of every tile it visits (about 13 % of
  // a full-size forward, which runs at the power limit); the bf16 head written first costs one fixed
  // pass (about 7 us at V = 8192). So the forward converts on chip when few row tiles are scored:
  // calls with a mask (sliding-window evaluation scores one row in 32) and calls of up to
  // kQ8OnChipMaxRows rows.
  constexpr int64_t kQ8OnChipMaxRows = 8192;
  if (pg::fwd_reads_q8(D, softcap) && (score_mask || T <= kQ8OnChipMaxRows)) {
    // the forward reads the int8 rows and converts each tile in LDS (the workspace's first
    // V * D * 2 bytes stay unused)
    e = pg::launch_fwd(hidden, nullptr, PG_DTYPE_BF16, target, score_mask, T, D, V, softcap, softcap, nats, lse, fws,
                       dev, st, nullptr, embed_q8, embed_scale);
  } else {
    // other widths and caps: the bf16 rows into the workspace, then the bf16 forward on them
    uint16_t* deq = reinterpret_cast<uint16_t*>(ws);
    e = pg::launch_dequantize(embed_q8, embed_scale, V, D, deq, st);
    if (e == hipSuccess)
      e = pg::launch_fwd(hidden, deq, PG_DTYPE_BF16, target, score_mask, T, D, V, softcap, softcap, nats, lse, fws,
                         dev, st);
  }
  return e == hipSuccess ? PG_OK : PG_ERR_HIP;
}

static pg_status bpb_impl(const float* nats, const int32_t* target, const uint8_t* score_mask,
                          const int32_t* byte_len, const int32_t* byte_per_pos, int64_t T, int32_t V, double* out,
                          void* workspace, size_t workspace_bytes, void* stream, bool accumulate) {
  pg_status s;
  if ((s = check_shape(T, 1, V)) != PG_OK) return s;
  if (T > 0 && (!nats || (!byte_per_pos && !target))) return PG_ERR_NULL;
  if (!byte_per_pos && !byte_len) return PG_ERR_NULL;
  if (!out || !workspace) return PG_ERR_NULL;
  if (misaligned(nats) || misaligned(target) || misaligned(score_mask) || misaligned(byte_len) ||
      misaligned(byte_per_pos) || misaligned(out) || misaligned(workspace))
    return PG_ERR_ALIGN;
  if (workspace_bytes < pg_workspace_bytes(PG_OP_BPB, T, 1, V)) return PG_ERR_WORKSPACE;
  pg::DeviceInfo dev{};
  if ((s = device_check(dev)) != PG_OK) return s;
  hipError_t e = pg::launch_bpb(nats, target, score_mask, byte_len, byte_per_pos, T, V, out,
                                static_cast<char*>(workspace), static_cast<hipStream_t>(stream), accumulate);
  return e == hipSuccess ? PG_OK : PG_ERR_HIP;
}

pg_status pg_bpb_reduce(const float* nats, const int32_t* target, const uint8_t* score_mask,
                        const int32_t* byte_len, const int32_t* byte_per_pos,
                        int64_t T, int32_t V, double* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return bpb_impl(nats, target, score_mask, byte_len, byte_per_pos, T, V, out, workspace, workspace_bytes, stream,
                  false);
}

pg_status pg_bpb_accumulate(const float* nats, const int32_t* target, const uint8_t* score_mask,
                            const int32_t* byte_len, const int32_t* byte_per_pos,
                            int64_t T, int32_t V, double* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return bpb_impl(nats, target, score_mask, byte_len, byte_per_pos, T, V, out, workspace, workspace_bytes, stream,
                  true);
}

// ------------------------------------------------------------------ sliding-window evaluation

// A stream longer than 2^40 tokens (4 TiB of ids) cannot be in device memory; the bound keeps
// every position w stride + r of a window that starts in the stream far inside int64.
constexpr int64_t kMaxStreamTokens = (int64_t)1 << 40;

static bool window_args_ok(int64_t n_tokens, int32_t window, int32_t stride) {
  return n_tokens >= 0 && n_tokens <= kMaxStreamTokens && window >= 1 && stride >= 1 && stride <= window;
}

// first_window may name the window just past the last one (an empty run) but nothing beyond it.
static bool first_window_ok(int64_t n_tokens, int32_t window, int32_t stride, int64_t first_window) {
  return first_window >= 0 && first_window <= pg::window_count(n_tokens, window, stride);
}

int64_t pg_window_count(int64_t n_tokens, int32_t window, int32_t stride) {
  if (!window_args_ok(n_tokens, window, stride)) return PG_ERR_SHAPE;
  return pg::window_count(n_tokens, window, stride);
}

int64_t pg_window_scored(int64_t n_tokens, int32_t window, int32_t stride, int64_t first_window, int32_t n_windows) {
  if (!window_args_ok(n_tokens, window, stride) || !first_window_ok(n_tokens, window, stride, first_window) ||
      n_windows < 0)
    return PG_ERR_SHAPE;
  return pg::window_scored(n_tokens, window, stride, first_window, n_windows);
}

pg_status pg_window_rows(const int32_t* tokens, int64_t n_tokens, int32_t window, int32_t stride,
                         int64_t first_window, int32_t n_windows, int32_t* target, uint8_t* score_mask,
                         void* stream) {
  if (!window_args_ok(n_tokens, window, stride) || !first_window_ok(n_tokens, window, stride, first_window) ||
      n_windows < 1 || (int64_t)n_windows * window > kMaxRows)
    return PG_ERR_SHAPE;
  if ((n_tokens > 0 && !tokens) || !target || !score_mask) return PG_ERR_NULL;
  if (misaligned(tokens) || misaligned(target) || misaligned(score_mask)) return PG_ERR_ALIGN;
  pg::DeviceInfo dev{};
  pg_status s;
  if ((s = device_check(dev)) != PG_OK) return s;
  hipError_t e = pg::launch_window_rows(tokens, n_tokens, window, stride, first_window, n_windows, target,
                                        score_mask, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PG_OK : PG_ERR_HIP;
}

pg_status pg_sgd_step_bf16(float* master, const float* grad, float lr, int64_t n, void* embed_bf16, void* stream) {
  if (n < 0) return PG_ERR_SHAPE;
  if (!std::isfinite(lr)) return PG_ERR_SOFTCAP;
  if (n == 0) return PG_OK;
  if (!master || !grad || !embed_bf16) return PG_ERR_NULL;
  if (misaligned(master) || misaligned(grad) || misaligned(embed_bf16)) return PG_ERR_ALIGN;
  pg::DeviceInfo dev{};
  pg_status s;
  if ((s = device_check(dev)) != PG_OK) return s;
  hipError_t e = pg::launch_sgd_step(master, grad, lr, n, static_cast<uint16_t*>(embed_bf16),
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PG_OK : PG_ERR_HIP;
}

}  // extern "C"
