// C ABI of the library: host-side validation, workspace sizing, device check and dispatch.
// Validation happens before anything is enqueued and has no side effects.
#include <atomic>
#include <cmath>
#include <cstring>

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

constexpr int64_t kMaxRows = 2147483647LL;
constexpr int32_t kMaxWidth = 1 << 20;

pg_status check_shape(int64_t T, int32_t D, int32_t V) {
  if (T < 0 || T > kMaxRows || D < 1 || D > kMaxWidth || V < 1 || V > kMaxWidth) return PG_ERR_SHAPE;
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
    case PG_ERR_SOFTCAP: return "softcap or grad_scale is negative or not finite";
    case PG_ERR_WORKSPACE: return "workspace smaller than pg_workspace_bytes()";
    case PG_ERR_ALIGN: return "pointer not 16-byte aligned";
    case PG_ERR_DEVICE: return "no HIP device, or the current device is not gfx950";
    case PG_ERR_HIP: return "HIP runtime or kernel launch failure";
    default: return "unknown status";
  }
}

size_t pg_workspace_bytes(int32_t op, int64_t T, int32_t D, int32_t V) {
  if (check_shape(T, D, V) != PG_OK) return 0;
  switch (op) {
    case PG_OP_FWD: return pg::fwd_workspace(T, D, V).total;
    case PG_OP_BWD: return pg::bwd_workspace(T, D, V).total;
    case PG_OP_BPB: return pg::bpb_workspace(T).total;
    case PG_OP_FWD_BWD: return pg::train_workspace(T, D, V).total;
    case PG_OP_FWD_Q8:
      if (D % 8 != 0) return 0;
      return pg::align256((size_t)V * (size_t)D * 2) + pg::fwd_workspace(T, D, V).total;
    default: return 0;
  }
}

static pg_status fwd_impl(const void* hidden, const void* embed, int32_t dtype, const int32_t* target,
                          const uint8_t* score_mask, int64_t T, int32_t D, int32_t V, float cap_pos, float cap_neg,
                          float* nats, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  pg_status s;
  if ((s = check_shape(T, D, V)) != PG_OK) return s;
  if (T > 0 && (!hidden || !target || !nats)) return PG_ERR_NULL;
  if (!embed || !workspace) return PG_ERR_NULL;
  if (dtype != PG_DTYPE_BF16 && dtype != PG_DTYPE_F32) return PG_ERR_DTYPE;
  if ((s = check_softcap(cap_pos)) != PG_OK || (s = check_softcap(cap_neg)) != PG_OK) return s;
  if (misaligned(hidden) || misaligned(embed) || misaligned(target) || misaligned(score_mask) ||
      misaligned(nats) || misaligned(lse) || misaligned(workspace))
    return PG_ERR_ALIGN;
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
  if ((s = check_shape(T, D, V)) != PG_OK) return s;
  if (T > 0 && (!hidden || !target || !lse || !dhidden)) return PG_ERR_NULL;
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
  if ((s = check_shape(T, D, V)) != PG_OK) return s;
  if (T > 0 && (!hidden || !target || !nats || !lse || !dhidden)) return PG_ERR_NULL;
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
  uint16_t* deq = reinterpret_cast<uint16_t*>(ws);
  hipError_t e = pg::launch_dequantize(embed_q8, embed_scale, V, D, deq, st);
  if (e == hipSuccess)
    e = pg::launch_fwd(hidden, deq, PG_DTYPE_BF16, target, score_mask, T, D, V, softcap, softcap, nats, lse,
                       ws + pg::align256((size_t)V * (size_t)D * 2), dev, st);
  return e == hipSuccess ? PG_OK : PG_ERR_HIP;
}

pg_status pg_bpb_reduce(const float* nats, const int32_t* target, const uint8_t* score_mask,
                        const int32_t* byte_len, const int32_t* byte_per_pos,
                        int64_t T, int32_t V, double* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
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
                                static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PG_OK : PG_ERR_HIP;
}

}  // extern "C"
