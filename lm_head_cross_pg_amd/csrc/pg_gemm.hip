// bf16 GEMM with float32 accumulation for the two products of the backward, dH = g dZ E and
// dE = g dZ^T H, on gfx950 (v_mfma_f32_32x32x16_bf16).
//
// 128 x 512 output tiles per workgroup (4 waves of 128 x 128, sixteen 32 x 32 accumulators each,
// held in AGPRs), 32-deep k-chunks in a 3-stage LDS ring filled by global_load_lds_dwordx4.
// A is dZ in its 32 x 32 block layout (described in pg_internal.h); each stage's A tile is four
// whole blocks, i.e. four contiguous 2 KiB runs. The other operand (E for dH, H for dE) is k x n
// row-major and is fed to the MFMA with ds_read_b64_tr_b16, which gives each lane 4 consecutive k
// of one column, so no transpose pass over memory is needed; for dE the A operand is read the same
// way from the blocks.
#include "pg_common.h"
#include "pg_internal.h"
#include "pg_tile.h"

namespace pg {

// LDS tile layouts (bytes), 16-byte chunk indices permuted so that the 16 lanes of an LDS read
// phase hit 16 different 16-byte bank groups:
//   A: four dZ blocks of 2 KiB; chunk c of a block stored at chunk a_swz(c)
//   B: [32 k][512 n], 1 KiB rows; chunk c of row k stored at c ^ (4 (k & 3))
// a_swz flips chunk bit 0 when bit 4 is set (the plain 16-byte reads of dH, which stride two
// chunks per lane) and bit 3 when bit 6 is set (the transposed reads of dE, which pair chunks 64
// apart); it is its own inverse.
__device__ __forceinline__ int a_swz(int c) { return c ^ ((c >> 4) & 1) ^ (((c >> 6) & 1) << 3); }

// A workgroup owns a 128 x 512 output tile (the whole hidden width), so dZ is read from memory once.
template <bool A_TRANS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(GemmParams g) {
  constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
  constexpr int ABYTES = BM * BK * 2, BBYTES = BN * BK * 2, SBYTES = ABYTES + BBYTES;
  constexpr int A_LOADS = ABYTES / 1024, B_LOADS = BBYTES / 1024;   // 1 KiB load instructions
  constexpr int LOADS_PER_WAVE = (A_LOADS + B_LOADS) / 4;
  static_assert(BM == 128 && BN == 512 && BK == 32, "tile shape assumed by the layouts below");
  __shared__ __attribute__((aligned(1024))) char smem[kGemmStages * SBYTES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5;

  const int64_t ndev = g.n_dev ? (int64_t)(*g.n_dev) : 0;
  const int64_t M = g.m_dev ? ndev : g.M;
  const int64_t K = g.k_dev ? ndev : g.K;
  const int64_t m0 = (int64_t)blockIdx.x * BM;
  const int64_t n0 = (int64_t)blockIdx.y * BN;
  if (m0 >= M) return;
  const int64_t kchunks = (K + BK - 1) / BK;
  const int nsplit = gridDim.z;
  const int64_t cps = (kchunks + nsplit - 1) / nsplit;
  const int64_t kc_begin = (int64_t)blockIdx.z * cps;
  const int64_t kc_end = kc_begin + cps < kchunks ? kc_begin + cps : kchunks;
  const int64_t nk = kc_end > kc_begin ? kc_end - kc_begin : 0;
  const int64_t kvalid = g.k_dev ? ndev : g.kvalid;

  // ---- stage loader: each wave issues LOADS_PER_WAVE global_load_lds_dwordx4; load_one(kc, st, i)
  //      issues this wave's i-th, so that the loads of a stage can be spread over the MFMAs of the
  //      previous one (issued in a burst they stall the wave for longer than the MFMAs take)
  static_assert(A_LOADS % 4 == 0 && B_LOADS % 4 == 0, "loads split evenly over the 4 waves");
  auto load_one = [&](int64_t kc, int st, int i) {
    char* sA = smem + st * SBYTES;
    char* sB = sA + ABYTES;
    const int64_t k0 = kc * BK;
    if (i < A_LOADS / 4) {
      const int j = wave + 4 * i;       // half (j & 1) of block bm = j / 2 of the stage
      const int bm = j >> 1;
      int64_t bt, bv;
      if (!A_TRANS) {                   // dH: m = token, k = vocabulary
        bt = (m0 >> 5) + bm;
        bv = k0 >> 5;
      } else {                          // dE: m = vocabulary, k = token
        bt = k0 >> 5;
        bv = (m0 >> 5) + bm;
        bv = bv < g.lda ? bv : g.lda - 1;
      }
      const int chunk = a_swz(64 * (j & 1) + lane);
      const uint16_t* src = g.A + (bt * g.lda + bv) * 1024 + chunk * 8;
      lds_dma16(src, (const lds_char*)(sA + j * 1024));
    } else {
      const int j = wave + 4 * (i - A_LOADS / 4);   // row j of the B tile
      const int lc = lane ^ (4 * (j & 3));
      int64_t k = k0 + j;
      k = k < kvalid ? k : kvalid - 1;
      int64_t col = n0 + 8 * lc;
      col = col <= g.ldb - 8 ? col : g.ldb - 8;
      lds_dma16(g.B + k * g.ldb + col, (const lds_char*)(sB + j * 1024));
    }
  };
  auto load_stage = [&](int64_t kc, int st) {
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) load_one(kc, st, i);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int grp = lane >> 4, li = lane & 15;
  // transposed read: lanes of group grp take rows k0 + li / 4 and columns cbase + 16 (grp & 1) +
  // 4 (li & 3) .. + 3, for k0 = 16 ks + 8 (grp >> 1) + 4 half; lane i of the group receives 4
  // consecutive k of column cbase + 16 (grp & 1) + i
  // With INTERLEAVED k order, half `half` of lane l's eight values covers rows 16 ks + 8 half +
  // 4 (l / 32) .. + 3 instead of 16 ks + 8 (l / 32) + 4 half .. + 3 (the order the dZ blocks hold).
  auto read_tr = [&](const char* tile, int pitch, int ks, int cbase, bool interleaved) -> bf16x8 {
    i16x4 part[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k = 16 * ks + (interleaved ? 8 * half + 4 * (grp >> 1) : 8 * (grp >> 1) + 4 * half) + (li >> 2);
      const int c = cbase + 16 * (grp & 1) + 4 * (li & 3);
      const int addr = k * pitch + 16 * ((c >> 3) ^ (4 * (k & 3))) + 2 * (c & 7);
      part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + addr));
    }
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 v = {part[0][0], part[0][1], part[0][2], part[0][3], part[1][0], part[1][1], part[1][2], part[1][3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  // Fragments of one 16-deep k step: the 4 A blocks of this wave and its 4 B blocks.
  auto load_frags = [&](const char* sA, const char* sB, int ks, bf16x8 (&af)[4], bf16x8 (&bfr)[4]) {
#pragma unroll
    for (int bm = 0; bm < 4; ++bm) {
      const char* blk = sA + bm * 2048;
      if (!A_TRANS) {
        // lane l holds row l % 32 of the block in its own 32 bytes: the 16 at chunk 2 l + ks are
        // vocabulary rows 16 ks + 8 (j / 4) + 4 (l / 32) + j % 4, j = 0..7
        af[bm] = *(const __attribute__((address_space(3))) bf16x8*)((const lds_char*)blk + a_swz(2 * lane + ks) * 16);
      } else {
        // transposed read: lane l receives vocabulary row l % 32 at tokens 16 ks + 8 (l / 32) + j;
        // the lanes of a 16-lane group address 4 tokens x 4 runs of 4 vocabulary rows
        i16x4 part[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int t = 16 * ks + 8 * (grp >> 1) + 4 * half + (li >> 2);
          const int cg = li & 3;
          const int c = 2 * (t + 32 * (cg & 1)) + (grp & 1);
          part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(blk + a_swz(c) * 16 + 8 * (cg >> 1)));
        }
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        i16x8 v = {part[0][0], part[0][1], part[0][2], part[0][3], part[1][0], part[1][1], part[1][2], part[1][3]};
        af[bm] = __builtin_bit_cast(bf16x8, v);
      }
    }
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) bfr[bn] = read_tr(sB, BN * 2, ks, wave * 128 + bn * 32, !A_TRANS);
  };

  if (nk > 0) load_stage(kc_begin, 0);
  if (nk > 1) load_stage(kc_begin + 1, 1);
  for (int64_t it = 0; it < nk; ++it) {
    // this wave's loads of stage `it` are done when at most one stage (the next) is in flight
    if (it + 1 < nk) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS_PER_WAVE) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();   // every wave's loads of stage `it` landed; stage it-1 is free
    const int st = (int)(it % kGemmStages);
    const char* sA = smem + st * SBYTES;
    const char* sB = sA + ABYTES;
    // every fragment of the stage is requested before the first MFMA; the compiler's waits then
    // release each MFMA as soon as its own two fragments have arrived
    bf16x8 af[BK / 16][4], bfr[BK / 16][4];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) load_frags(sA, sB, ks, af[ks], bfr[ks]);
    __builtin_amdgcn_sched_barrier(0);
    // the MFMAs of this stage with the loads of stage it + 2 (into the buffer stage it - 1 used)
    // issued between them, one every MFMA_PER_LOAD MFMAs
    constexpr int NMFMA = (BK / 16) * 16;
    constexpr int MFMA_PER_LOAD = NMFMA / LOADS_PER_WAVE;
    const bool prefetch = it + 2 < nk;
    const int64_t kc_pf = kc_begin + it + 2;
    const int st_pf = (int)((it + 2) % kGemmStages);
#pragma unroll
    for (int mi = 0; mi < NMFMA; ++mi) {
      const int ks = mi >> 4, bm = (mi >> 2) & 3, bn = mi & 3;
      acc[bm][bn] = mfma32x32x16(af[ks][bm], bfr[ks][bn], acc[bm][bn]);
      if (mi % MFMA_PER_LOAD == 0 && mi / MFMA_PER_LOAD < LOADS_PER_WAVE && prefetch)
        load_one(kc_pf, st_pf, mi / MFMA_PER_LOAD);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue: alpha * acc to C (row-scattered) or to this split's partial tile
  float* C = g.C + (int64_t)blockIdx.z * g.split_stride;
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const int64_t n = n0 + wave * 128 + bn * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + bm * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M && n < g.N) {
          const int64_t crow = g.crows ? (int64_t)g.crows[m] : m;
          C[crow * g.ldc + n] = g.alpha * acc[bm][bn][r];
        }
      }
    }
}

// out[i] = sum over s of part[s * stride + i], in split order.
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* part, int nsplit, int64_t stride, int64_t count,
                                                         float* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float s = 0.f;
  for (int k = 0; k < nsplit; ++k) s += part[(int64_t)k * stride + i];
  out[i] = s;
}


hipError_t launch_gemm(const GemmParams& g, bool a_trans, dim3 grid, hipStream_t st) {
  if (a_trans) hipLaunchKernelGGL(gemm_bf16_kernel<true>, grid, dim3(256), 0, st, g);
  else hipLaunchKernelGGL(gemm_bf16_kernel<false>, grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_sum_splits(const float* part, int nsplit, int64_t stride, int64_t count, float* out,
                             hipStream_t st) {
  hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, part, nsplit,
                     stride, count, out);
  return hipGetLastError();
}

}  // namespace pg
