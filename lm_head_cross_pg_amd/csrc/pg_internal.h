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
  size_t dz;       // bf16 dZ without the grad_scale factor, block layout, T rounded up to 256, V to 64
  size_t hc;       // bf16[T, D]: hidden rows of the scored positions, compacted (masked calls)
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

// Forward launchers (pg_fwd.hip). `ws` is the workspace base. Caps: z >= 0 uses cap_pos, z < 0
// cap_neg (equal for the symmetric softcap); 0 = uncapped side.
hipError_t launch_compact_rows(const uint8_t* mask, int64_t T, char* ws, const FwdWorkspace& L,
                               float* nats, float* lse, hipStream_t st);
// dz (nullable): when given, the forward also writes the unnormalised dZ blocks (only where
// fwd_writes_dz holds; rows padded to 256, vocabulary rows to the tile).
hipError_t launch_fwd(const void* H, const void* E, int32_t dtype, const int32_t* target,
                      const uint8_t* mask, int64_t T, int32_t D, int32_t V, float cap_pos, float cap_neg,
                      float* nats, float* lse, char* ws, const DeviceInfo& dev, hipStream_t st,
                      uint16_t* dz = nullptr, const int8_t* eq = nullptr, const float* qscale = nullptr);
// eq, qscale (nullable): the head is the per-row int8 embedding (q[V, D], scales[V]) read by the
// forward itself (E is then unused); only where fwd_reads_q8 holds, without dz.
bool fwd_reads_q8(int32_t D, float cap);
// The forward can write the unnormalised dZ: bf16 MFMA widths, every side capped within the
// fixed-shift range (one cap, or two).
bool fwd_writes_dz(int32_t dtype, int32_t D, float cap_pos, float cap_neg);

// Forward + backward in one call (pg_bwd.hip). Where fwd_writes_dz holds, the forward writes the
// unnormalised dZ and no logit is computed twice; otherwise it is launch_fwd then launch_bwd.
struct TrainWorkspace {
  size_t fwd;        // FwdWorkspace
  size_t bwd;        // BwdWorkspace (dz, scaled compacted hidden rows, dE partials)
  size_t row_scale;  // f32[T]: per compacted row, g 2^(M - lse log2 e) (-1 / M^2)
  size_t total;
};
TrainWorkspace train_workspace(int64_t T, int32_t D, int32_t V);
hipError_t launch_train(const void* H, const void* E, int32_t dtype, const int32_t* target,
                        const uint8_t* mask, int64_t T, int32_t D, int32_t V, float cap_pos, float cap_neg,
                        float grad_scale, float* nats, float* lse, float* dH, float* dE, char* ws,
                        const DeviceInfo& dev, hipStream_t st);

// Backward launcher (pg_bwd.hip).
hipError_t launch_bwd(const void* H, const void* E, int32_t dtype, const int32_t* target,
                      const uint8_t* mask, const float* lse, int64_t T, int32_t D, int32_t V,
                      float cap_pos, float cap_neg, float grad_scale, float* dH, float* dE, char* ws,
                      const DeviceInfo& dev, hipStream_t st);

// Per-row int8 embedding (pg_quant.hip): quantiser and dequantiser to bf16.
hipError_t launch_quantize(const void* E, int32_t dtype, int32_t V, int32_t D, int8_t* q, float* scale,
                           hipStream_t st);
hipError_t launch_dequantize(const int8_t* q, const float* scale, int32_t V, int32_t D, uint16_t* E, hipStream_t st);

// Bits-per-byte launcher (pg_bpb.hip); accumulate adds to the running sums already in out.
hipError_t launch_bpb(const float* nats, const int32_t* target, const uint8_t* mask,
                      const int32_t* byte_len, const int32_t* byte_per_pos, int64_t T, int32_t V,
                      double* out, char* ws, hipStream_t st, bool accumulate = false);

// Sliding-window evaluation (pg_window.hip): the schedule's arithmetic on the host, the targets and
// score mask of a batch of windows, and the SGD step of score-first test-time training.
int64_t window_count(int64_t n_tokens, int32_t window, int32_t stride);
int64_t window_scored(int64_t n_tokens, int32_t window, int32_t stride, int64_t first_window, int64_t n_windows);
hipError_t launch_window_rows(const int32_t* tokens, int64_t n_tokens, int32_t window, int32_t stride,
                              int64_t first_window, int64_t n_windows, int32_t* target, uint8_t* mask,
                              hipStream_t st);
hipError_t launch_sgd_step(float* master, const float* grad, float lr, int64_t n, uint16_t* out, hipStream_t st);

// dZ block layout (the backward's workspace). dZ[t][v] is stored in 32 x 32 blocks laid out like
// the accumulator of v_mfma_f32_32x32x16_bf16: block (bt, bv) holds tokens 32 bt .. 32 bt + 31 and
// vocabulary rows 32 bv .. 32 bv + 31 as 1024 bf16 at offset (bt * nvb + bv) * 1024, nvb = number
// of vocabulary blocks; inside a block, element (t, v) sits at 512 (r >> 3) + 8 L + (r & 7) with
//   L = t + 32 ((v >> 2) & 1)   (the lane that computed it),  r = 4 (v >> 3) + (v & 3).
// The writers store a lane's accumulator registers 8 j .. 8 j + 7 as 16 bytes at 512 j + 8 L, so
// each 16-byte store instruction of a wave fills one contiguous KiB (the first half of the block,
// then the second), and each block is one 2 KiB run.

// C = alpha * A B in bf16 with float32 accumulation (pg_gemm.hip), k in 32-deep chunks.
constexpr int kGemmBK = 32;
struct GemmParams {
  const uint16_t* A;      // dZ blocks; element (m, k) = dZ[m][k], or dZ[k][m] when A_TRANS
  int64_t lda;            // vocabulary blocks per token block (nvb)
  int64_t a_mblocks;      // 32-blocks of A along m that exist in memory (reads past them are clamped)
  int64_t k_blocks;       // A_TRANS: 32-blocks of A along k (token blocks) that exist in memory
  const uint16_t* B;      // element (k, n): B[k * ldb + n]
  int64_t ldb;
  const int32_t* n_dev;   // device count that replaces M (m_dev) or K (k_dev)
  int m_dev, k_dev;
  int64_t M, N, K;        // sizes (upper bounds when taken from n_dev)
  int64_t kvalid;         // rows of B that exist (host bound; clamped below the device count)
  float alpha;
  float* C;
  int64_t ldc;
  const int32_t* crows;   // output row of m when given
  int64_t split_stride;   // elements between the partial outputs of k splits
  const float* row_scale; // when given: C row m = alpha * row_scale[m] * (A B)[m]
};
// a_trans: A's element (m, k) is dZ[k][m] (else dZ[m][k]). k is split over ksplit workgroups per
// output tile; with several splits, C receives one partial output per split at split_stride.
// M and N are the host bounds that size the grid.
hipError_t launch_gemm(const GemmParams& g, bool a_trans, int ksplit, hipStream_t st);
// dH (a, not transposed, one split) and dE (b, transposed, ksb splits) in one launch; the same
// results as the two launch_gemm calls.
hipError_t launch_gemm_pair(const GemmParams& a, const GemmParams& b, int ksb, hipStream_t st);
// Output tile of each product (rows x columns).
int gemm_tile_m(bool a_trans);
int gemm_tile_n(bool a_trans);
// Workgroups along x of the launch of an M x N product (256 threads each; the shape checks hold
// them to kMaxGrid512, which is stricter than the launch limit).
int64_t gemm_grid_x(int64_t M, int64_t N, bool a_trans);
// Most workgroups of 512 threads one launch can hold (2^32 - 1 work items).
constexpr int64_t kMaxGrid512 = ((int64_t)1 << 23) - 1;
// out[i] = sum over s < nsplit of part[s * stride + i], in split order (nsplit = 0 writes zeros).
hipError_t launch_sum_splits(const float* part, int nsplit, int64_t stride, int64_t count, float* out,
                             hipStream_t st);

// True when the bf16 MFMA kernels cover this hidden width.
inline bool mfma_width(int32_t D) {
  return D == 32 || D == 64 || D == 128 || D == 256 || D == 512;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workgroups of a grid-stride launch over `count` items at `per_block` items per workgroup and
// pass. A launch may hold at most 2^32 - 1 work items, so element-wise and row-wise kernels loop
// over their range with a grid capped at kMaxStrideBlocks workgroups (16 Mi threads at 256).
constexpr int64_t kMaxStrideBlocks = (int64_t)1 << 16;
inline unsigned stride_blocks(int64_t count, int64_t per_block) {
  const int64_t b = (count + per_block - 1) / per_block;
  return (unsigned)(b < 1 ? 1 : (b > kMaxStrideBlocks ? kMaxStrideBlocks : b));
}

}  // namespace pg
