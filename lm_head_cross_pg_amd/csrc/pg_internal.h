// Host-side launchers shared between the translation units of the library (internal header).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pg {

// Byte offsets of the pieces of a workspace, all 256-byte aligned.
struct FwdWorkspace {
  size_t n_rows;    // int32: number of scored rows (device-side count)
  size_t rows;      // int32[T]: scored row indices in ascending order
  size_t s_target;  // f32[T]: capped target logit (base 2) per compacted row
  size_t part_l;    // f32[P]: partial exp-sums per (split, compacted row)
  size_t part_m;    // f32[P]: partial maxima per (split, compacted row) (uncapped / large caps)
  size_t total;
};
FwdWorkspace fwd_workspace(int64_t T, int32_t D, int32_t V);
int64_t fwd_partial_entries(int64_t T);

struct BwdWorkspace {
  size_t n_rows;   // int32
  size_t rows;     // int32[T]
  size_t dz;       // bf16[T, V]: dZ without the grad_scale factor
  size_t de_part;  // f32[KSPLIT, V, D]: split-K partials of dE
  size_t total;
};
BwdWorkspace bwd_workspace(int64_t T, int32_t D, int32_t V);

struct BpbWorkspace {
  size_t part;     // per-block partials
  size_t total;
};
BpbWorkspace bpb_workspace(int64_t T);

// Device facts needed to size launches (cached per device by the API layer).
struct DeviceInfo {
  int cu_count;
};

// Forward launchers (pg_fwd.hip). `ws` is the workspace base.
hipError_t launch_compact_rows(const uint8_t* mask, int64_t T, char* ws, const FwdWorkspace& L,
                               float* nats, float* lse, hipStream_t st);
hipError_t launch_fwd(const void* H, const void* E, int32_t dtype, const int32_t* target,
                      const uint8_t* mask, int64_t T, int32_t D, int32_t V, float softcap,
                      float* nats, float* lse, char* ws, const DeviceInfo& dev, hipStream_t st);

// Backward launcher (pg_bwd.hip).
hipError_t launch_bwd(const void* H, const void* E, int32_t dtype, const int32_t* target,
                      const uint8_t* mask, const float* lse, int64_t T, int32_t D, int32_t V,
                      float softcap, float grad_scale, float* dH, float* dE, char* ws,
                      const DeviceInfo& dev, hipStream_t st);

// Bits-per-byte launcher (pg_bpb.hip).
hipError_t launch_bpb(const float* nats, const int32_t* target, const uint8_t* mask,
                      const int32_t* byte_len, const int32_t* byte_per_pos, int64_t T, int32_t V,
                      double* out, char* ws, hipStream_t st);

// True when the bf16 MFMA kernels cover this hidden width.
inline bool mfma_width(int32_t D) {
  return D == 32 || D == 64 || D == 128 || D == 256 || D == 512;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace pg
