// bf16 GEMM with float32 accumulation for the two products of the backward, dH = g dZ E and
// dE = g dZ^T H, on gfx950 (v_mfma_f32_32x32x16_bf16).
//
// A workgroup owns a 128 x 512 output tile (BM = 64 MB, MB = 2) and runs 8 waves, two per SIMD,
// in a 2 x 4 grid; each wave accumulates 64 x 128 of the tile in eight 32 x 32 accumulators. k
// advances in 32-deep chunks; B and A are filled by global_load_lds_dwordx4 into LDS rings of 3 and
// 4 slots.
//
// Why this shape: the operand streams mix a unique stream from HBM (dZ) with a stream that every
// workgroup shares from L2 (E or H). A CU returns vector-memory data in issue order, so the HBM
// latency paces the shared stream too, and the CU sustains about 28 B/clk of this mix. Each stage
// therefore issues the B loads of stage s + 2 first and the A load of stage s + 3 after them: a B
// load waits only for A loads issued a stage or more before it, and every load has three stage
// periods to land (A needs the extra ring slot). A 128 x 512 tile needs 40 KiB per 4.2 MFLOP
// chunk; a 192 x 512 one would need less per MFLOP, but at T = 65536 its 342 tiles do not fill
// 256 CUs evenly. Two waves per SIMD keep the matrix pipe busy while the other wave of the SIMD is
// held up issuing a load.
//
// A is dZ in its 32 x 32 block layout (described in pg_internal.h); each stage's A tile is BM / 32
// whole blocks, i.e. contiguous 2 KiB runs. The other operand (E for dH, H for dE) is k x n
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

// The tile covers the whole hidden width (512), so dZ is read from memory once.
template <bool A_TRANS, int MB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_kernel(GemmParams g) {
  constexpr int BM = 64 * MB, BN = kGemmBN, BK = kGemmBK;
  constexpr int NW = 8;
  constexpr int ABYTES = BM * BK * 2, BBYTES = BN * BK * 2;
  constexpr int A_LOADS = ABYTES / 1024, B_LOADS = BBYTES / 1024;   // 1 KiB load instructions
  constexpr int NL = A_LOADS + B_LOADS;
  constexpr int LPW = (NL + NW - 1) / NW;                           // loads per wave (the first NL % NW waves)
  static_assert(BN == 512 && BK == 32 && MB == 2, "tile shape assumed by the layouts below (one A load per wave)");
  // B: ring of kGemmStages slots; A: ring of AST slots, one stage deeper, so that each stage's A
  // load can be issued after its B loads and a stage earlier
  constexpr int AST = kGemmStages + 1;
  static_assert(kGemmStages * BBYTES + AST * ABYTES <= 160 * 1024, "LDS rings");
  __shared__ __attribute__((aligned(1024))) char smem[kGemmStages * BBYTES + AST * ABYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar branches
  const int h = lane >> 5;
  const int wm = wave >> 2, wn = wave & 3;   // this wave's rows wm * 32 MB .., columns wn * 128 ..

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

  // ---- the load group of stage kc: this wave's B rows of stage kc (i < B_LOADS / NW: rows
  //      wave + NW i), then its A chunk of stage kc + 1 (i = B_LOADS / NW: half (wave & 1) of A
  //      block wave / 2). load_one(kc, i) issues the i-th, so that a group can be spread over the
  //      MFMAs of the stage two before it.
  auto load_one = [&](int64_t kc, int i) {
    const int bpw = B_LOADS / NW;
    const int64_t rel = kc - kc_begin;
    int q;
    if (i < bpw) { q = A_LOADS + wave + NW * i; }
    else { q = wave; kc = kc + 1; }
    char* sA = smem + kGemmStages * BBYTES + (int)((rel + (i < bpw ? 0 : 1)) % AST) * ABYTES;
    char* sB = smem + (int)(rel % kGemmStages) * BBYTES;
    const int64_t k0 = kc * BK;
    if (q < A_LOADS) {
      const int bm = q >> 1;             // half (q & 1) of block bm of the stage
      int64_t bt, bv;
      if (!A_TRANS) {                    // dH: m = token, k = vocabulary
        bt = (m0 >> 5) + bm;
        bt = bt < g.a_mblocks ? bt : g.a_mblocks - 1;
        bv = k0 >> 5;
        bv = bv < g.lda ? bv : g.lda - 1;
      } else {                           // dE: m = vocabulary, k = token
        bt = k0 >> 5;
        bt = bt < g.k_blocks ? bt : g.k_blocks - 1;
        bv = (m0 >> 5) + bm;
        bv = bv < g.a_mblocks ? bv : g.a_mblocks - 1;
      }
      const int chunk = a_swz(64 * (q & 1) + lane);
      const uint16_t* src = g.A + (bt * g.lda + bv) * 1024 + chunk * 8;
      lds_dma16(src, (const lds_char*)(sA + q * 1024));
    } else {
      const int j = q - A_LOADS;         // row j of the B tile
      const int lc = lane ^ (4 * (j & 3));
      int64_t k = k0 + j;
      k = k < kvalid ? k : kvalid - 1;
      int64_t col = n0 + 8 * lc;
      col = col <= g.ldb - 8 ? col : g.ldb - 8;
      lds_dma16(g.B + k * g.ldb + col, (const lds_char*)(sB + j * 1024));
    }
  };
  auto load_stage = [&](int64_t kc) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) load_one(kc, i);
  };

  f32x16 acc[MB][4];
#pragma unroll
  for (int i = 0; i < MB; ++i)
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

  // Fragments of one 16-deep k step: this wave's MB A blocks (all at once) and its 4 B blocks
  // (one at a time).
  auto load_afrags = [&](const char* sA, int ks, bf16x8 (&af)[MB]) {
#pragma unroll
    for (int bm = 0; bm < MB; ++bm) {
      const char* blk = sA + (wm * MB + bm) * 2048;
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
  };
  auto load_bfrag = [&](const char* sB, int ks, int bn) -> bf16x8 {
    return read_tr(sB, BN * 2, ks, wn * 128 + bn * 32, !A_TRANS);
  };

  // A chunk of stage 0, then the groups of stages 0 and 1; every stage's group is issued (with
  // clamped addresses past the end), so the waits below are constant
  if (nk > 0) {
    load_one(kc_begin - 1, B_LOADS / NW);
    load_stage(kc_begin);
    load_stage(kc_begin + 1);
  }
  for (int64_t it = 0; it < nk; ++it) {
    // B(it) and A(it) landed: issued after B(it)'s last load are A(it + 1) and the group of it + 1
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPW + 1) : "memory");
    __builtin_amdgcn_s_barrier();
    const char* sA = smem + kGemmStages * BBYTES + (int)(it % AST) * ABYTES;
    const char* sB = smem + (int)(it % kGemmStages) * BBYTES;
    // The MFMAs of this stage, one 16-deep step at a time and one B block at a time (the next B
    // fragment is read while the MB MFMAs of the current one run), with the loads of stage it + 2
    // (into the buffer stage it - 1 used) issued between them. Wave priority drops from 3 to 1 halfway
    // through the stage: the two waves of a SIMD share one matrix pipe, and at equal priority the
    // older one would run ahead and leave the other to finish the stage alone.
    constexpr int NMFMA = (BK / 16) * MB * 4;
    constexpr int MFMA_PER_LOAD = NMFMA / LPW;
    const int64_t kc_pf = kc_begin + it + 2;
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[MB], bcur, bnext;
      load_afrags(sA, ks, af);
      bcur = load_bfrag(sB, ks, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) {
        if (bn + 1 < 4) bnext = load_bfrag(sB, ks, bn + 1);
#pragma unroll
        for (int bm = 0; bm < MB; ++bm) {
          const int mi = (ks * 4 + bn) * MB + bm;
          acc[bm][bn] = mfma32x32x16(af[bm], bcur, acc[bm][bn]);
          if (mi % MFMA_PER_LOAD == 0 && mi / MFMA_PER_LOAD < LPW) load_one(kc_pf, mi / MFMA_PER_LOAD);
          if (mi == NMFMA / 2) __builtin_amdgcn_s_setprio(1);
          __builtin_amdgcn_sched_barrier(0);
        }
        bcur = bnext;
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the clamped loads past the end landed

  // ---- epilogue: alpha * acc to C (row-scattered) or to this split's partial tile
  float* C = g.C + (int64_t)blockIdx.z * g.split_stride;
#pragma unroll
  for (int bm = 0; bm < MB; ++bm)
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const int64_t n = n0 + wn * 128 + bn * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + (wm * MB + bm) * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
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
  if (a_trans) hipLaunchKernelGGL((gemm_bf16_kernel<true, kGemmMBdE>), grid, dim3(512), 0, st, g);
  else hipLaunchKernelGGL((gemm_bf16_kernel<false, kGemmMBdH>), grid, dim3(512), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_sum_splits(const float* part, int nsplit, int64_t stride, int64_t count, float* out,
                             hipStream_t st) {
  hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, part, nsplit,
                     stride, count, out);
  return hipGetLastError();
}

}  // namespace pg
