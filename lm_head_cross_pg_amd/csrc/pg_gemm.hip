// bf16 GEMM with float32 accumulation for the two products of the backward, dH = g dZ E and
// dE = g dZ^T H, on gfx950 (v_mfma_f32_32x32x16_bf16).
//
// A workgroup owns a 256 x 256 output tile and runs 8 waves, two per SIMD, in a 2 x 4 grid; each
// wave accumulates 128 x 64 of the tile in eight 32 x 32 accumulators. k advances in 32-deep
// chunks; B and A are filled by global_load_lds_dwordx4 into LDS rings of NS and NS + 1 slots.
//
// Why this shape: the operand streams mix a unique stream from HBM (dZ) with a stream that every
// workgroup shares from L2 (E or H). A CU returns vector-memory data in issue order, so the HBM
// latency paces the shared stream too. Each stage therefore issues the B loads of stage
// s + NS - 1 first and the A loads of stage s + NS after them: a B load waits only for A loads
// issued a stage or more before it, and every load has NS stage periods to land (A needs the extra
// ring slot). A 256 x 256 tile moves 32 KiB per 4.2 MFLOP chunk, against 40 KiB for 128 x 512, and
// at T = 65536 it still gives 512 tiles (two full rounds on 256 CUs). The two column tiles of a row
// tile are launched 8 workgroup ids apart: workgroups are dealt to the 8 XCDs in turn, so the pair
// runs on one XCD at the same time and its L2 serves the second read of their dZ rows (the HBM
// fetch stays at one pass over dZ). Two waves per SIMD keep the matrix pipe busy while the other
// wave of the SIMD is held up issuing a load.
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
//   A: BM / 32 dZ blocks of 2 KiB; chunk c of a block stored at chunk a_swz(c)
//   B: [32 k][BN n], rows of 2 BN bytes; chunk c of row k stored at c ^ (4 (k & 3))
// a_swz flips chunk bit 0 when bit 4 is set (the plain 16-byte reads of dH, which stride two
// chunks per lane) and bit 3 when bit 6 is set (the transposed reads of dE, which pair chunks 64
// apart); it is its own inverse.
__device__ __forceinline__ int a_swz(int c) { return c ^ ((c >> 4) & 1) ^ (((c >> 6) & 1) << 3); }

// Tile shape: each wave accumulates WM x WN blocks of 32 x 32; the 8 waves form a WGM x (8 / WGM)
// grid, so the workgroup tile is BM x BN = (32 WM WGM) x (32 WN (8 / WGM)).
template <int WM, int WN, int WGM>
struct GemmShape {
  static constexpr int NW = 8, WGN = NW / WGM;
  static constexpr int BM = 32 * WM * WGM, BN = 32 * WN * WGN, BK = kGemmBK;
};

template <bool A_TRANS, int WM, int WN, int WGM, int NS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_kernel(GemmParams g) {
  using S = GemmShape<WM, WN, WGM>;
  constexpr int BM = S::BM, BN = S::BN, BK = S::BK, NW = S::NW;
  constexpr int ABYTES = BM * BK * 2, BBYTES = BN * BK * 2;
  constexpr int A_LOADS = ABYTES / 1024, B_LOADS = BBYTES / 1024;   // 1 KiB load instructions
  constexpr int APW = A_LOADS / NW, BPW = B_LOADS / NW, LPW = APW + BPW;   // per wave and stage
  constexpr int RPL = 1024 / (BN * 2);                              // B rows per load (1 or 2)
  static_assert(BK == 32 && A_LOADS % NW == 0 && B_LOADS % NW == 0 && (RPL == 1 || RPL == 2),
                "tile shape assumed by the layouts below");
  // B: ring of NS slots; A: ring of AST slots, one stage deeper, so that each stage's A
  // loads can be issued after its B loads and a stage earlier
  constexpr int AST = NS + 1;
  static_assert(NS * BBYTES + AST * ABYTES <= 160 * 1024, "LDS rings");
  __shared__ __attribute__((aligned(1024))) char smem[NS * BBYTES + AST * ABYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar branches
  const int h = lane >> 5;
  const int wm = wave / S::WGN, wn = wave % S::WGN;   // this wave's rows wm * 32 WM .., columns wn * 32 WN ..

  const int64_t ndev = g.n_dev ? (int64_t)(*g.n_dev) : 0;
  const int64_t M = g.m_dev ? ndev : g.M;
  const int64_t K = g.k_dev ? ndev : g.K;
  // Workgroups are dealt to the 8 XCDs in turn; the NT column tiles of one row tile get ids 8 apart,
  // so they run on the same XCD at the same time and share its L2 copy of their dZ rows.
  const int NT = (int)((g.N + BN - 1) / BN);
  const int64_t wid = blockIdx.x;
  const int64_t mt = (wid / (8 * NT)) * 8 + (wid % 8);
  const int nt = (int)((wid / 8) % NT);
  const int64_t m0 = mt * BM;
  const int64_t n0 = (int64_t)nt * BN;
  if (m0 >= M) return;
  const int64_t kchunks = (K + BK - 1) / BK;
  const int nsplit = gridDim.z;
  const int64_t cps = (kchunks + nsplit - 1) / nsplit;
  const int64_t kc_begin = (int64_t)blockIdx.z * cps;
  const int64_t kc_end = kc_begin + cps < kchunks ? kc_begin + cps : kchunks;
  const int64_t nk = kc_end > kc_begin ? kc_end - kc_begin : 0;
  const int64_t kvalid = g.k_dev ? ndev : g.kvalid;

  // ---- the load group of stage kc: this wave's B loads of stage kc (i < BPW: load wave + NW i,
  //      rows RPL (wave + NW i) ..), then its A loads of stage kc + 1 (i >= BPW: load
  //      wave + NW (i - BPW), half of an A block). load_one(kc, i) issues the i-th, so that a group
  //      can be spread over the MFMAs of stage kc - (NS - 1).
  auto load_one = [&](int64_t kc, int i) {
    const int64_t rel = kc - kc_begin;
    if (i >= BPW) {
      const int q = wave + NW * (i - BPW);
      char* sA = smem + NS * BBYTES + (int)((rel + 1) % AST) * ABYTES;
      const int64_t k0 = (kc + 1) * BK;
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
      const int q = wave + NW * i;
      char* sB = smem + (int)(rel % NS) * BBYTES;
      const int j = q * RPL + lane / (64 / RPL);    // row of the B tile
      const int lc = (lane % (64 / RPL)) ^ (4 * (j & 3));
      int64_t k = kc * BK + j;
      k = k < kvalid ? k : kvalid - 1;
      int64_t col = n0 + 8 * lc;
      col = col <= g.ldb - 8 ? col : g.ldb - 8;
      lds_dma16(g.B + k * g.ldb + col, (const lds_char*)(sB + q * 1024));
    }
  };
  auto load_stage = [&](int64_t kc) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) load_one(kc, i);
  };

  f32x16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
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

  // Fragments of one 16-deep k step: this wave's WM A blocks (all at once) and its WN B blocks
  // (one at a time).
  auto load_afrags = [&](const char* sA, int ks, bf16x8 (&af)[WM]) {
#pragma unroll
    for (int bm = 0; bm < WM; ++bm) {
      const char* blk = sA + (wm * WM + bm) * 2048;
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
    return read_tr(sB, BN * 2, ks, wn * (32 * WN) + bn * 32, !A_TRANS);
  };

  // A loads of stage 0, then the groups of stages 0 .. NS - 2; every stage's group is issued (with
  // clamped addresses past the end), so the waits below are constant
  if (nk > 0) {
#pragma unroll
    for (int i = BPW; i < LPW; ++i) load_one(kc_begin - 1, i);
#pragma unroll
    for (int d = 0; d < NS - 1; ++d) load_stage(kc_begin + d);
  }
  for (int64_t it = 0; it < nk; ++it) {
    // B(it) and A(it) landed: issued after B(it)'s last load are A(it + 1) and the groups of
    // it + 1 .. it + NS - 2
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(APW + (NS - 2) * LPW) : "memory");
    __builtin_amdgcn_s_barrier();
    const char* sA = smem + NS * BBYTES + (int)(it % AST) * ABYTES;
    const char* sB = smem + (int)(it % NS) * BBYTES;
    // The MFMAs of this stage, one 16-deep step at a time and one B block at a time (the next B
    // fragment is read while the WM MFMAs of the current one run), with the loads of the group of
    // it + NS - 1 (into the slots that stage it - 1 used) issued between them. Wave priority drops from 3
    // to 1 halfway through the stage: the two waves of a SIMD share one matrix pipe, and at equal
    // priority the older one would run ahead and leave the other to finish the stage alone.
    constexpr int NMFMA = (BK / 16) * WM * WN;
    constexpr int MFMA_PER_LOAD = NMFMA / LPW;
    const int64_t kc_pf = kc_begin + it + (NS - 1);
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[WM], bcur, bnext;
      load_afrags(sA, ks, af);
      bcur = load_bfrag(sB, ks, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int bn = 0; bn < WN; ++bn) {
        if (bn + 1 < WN) bnext = load_bfrag(sB, ks, bn + 1);
#pragma unroll
        for (int bm = 0; bm < WM; ++bm) {
          const int mi = (ks * WN + bn) * WM + bm;
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

  // ---- epilogue: alpha (times the row's scale when given) * acc to C (row-scattered) or to this
  //      split's partial tile
  float* C = g.C + (int64_t)blockIdx.z * g.split_stride;
#pragma unroll
  for (int bm = 0; bm < WM; ++bm)
#pragma unroll
    for (int bn = 0; bn < WN; ++bn) {
      const int64_t n = n0 + wn * (32 * WN) + bn * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + (wm * WM + bm) * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M && n < g.N) {
          const int64_t crow = g.crows ? (int64_t)g.crows[m] : m;
          const float f = g.row_scale ? g.alpha * g.row_scale[m] : g.alpha;
          C[crow * g.ldc + n] = f * acc[bm][bn][r];
        }
      }
    }
}

// out[i] = sum over s of part[s * stride + i], in split order, starting from 0. Four elements per
// thread when the layout allows 16-byte accesses, with the loads of up to 8 splits issued before
// the sum.
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* part, int nsplit, int64_t stride, int64_t count,
                                                         float* out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t gstride = (int64_t)gridDim.x * blockDim.x;
  const bool vec = nsplit <= 8 && stride % 4 == 0 && ((uintptr_t)part & 15) == 0 && ((uintptr_t)out & 15) == 0;
  const int64_t n4 = vec ? count / 4 : 0;
  for (int64_t i = gid; i < n4; i += gstride) {
    f32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < nsplit) v[k] = reinterpret_cast<const f32x4*>(part + (int64_t)k * stride)[i];
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < nsplit) s += v[k];
    reinterpret_cast<f32x4*>(out)[i] = s;
  }
  for (int64_t i = 4 * n4 + gid; i < count; i += gstride) {
    float s = 0.f;
    for (int k = 0; k < nsplit; ++k) s += part[(int64_t)k * stride + i];
    out[i] = s;
  }
}

// dH: 256 x 256 tiles, 4-slot B ring; dE: 256 x 256 tiles, 3-slot B ring (measured best for each).
using DhShape = GemmShape<4, 2, 2>;
using DeShape = GemmShape<4, 2, 2>;
int gemm_tile_m(bool a_trans) { return a_trans ? DeShape::BM : DhShape::BM; }
int gemm_tile_n(bool a_trans) { return a_trans ? DeShape::BN : DhShape::BN; }

int64_t gemm_grid_x(int64_t M, int64_t N, bool a_trans) {
  const int64_t bm = gemm_tile_m(a_trans), bn = gemm_tile_n(a_trans);
  const int64_t mt = (M + bm - 1) / bm, nt = (N + bn - 1) / bn;
  return nt > 1 ? 8 * nt * ((mt + 7) / 8) : mt;   // the id mapping of the kernel
}

hipError_t launch_gemm(const GemmParams& g, bool a_trans, int ksplit, hipStream_t st) {
  const int64_t gx = gemm_grid_x(g.M, g.N, a_trans);
  if (gx == 0 || ksplit < 1) return hipSuccess;
  if (gx > kMaxGrid512) return hipErrorInvalidConfiguration;   // the API layer rejects such shapes first
  const dim3 grid((unsigned)gx, 1, (unsigned)ksplit);
  if (a_trans) hipLaunchKernelGGL((gemm_bf16_kernel<true, 4, 2, 2, 3>), grid, dim3(512), 0, st, g);
  else hipLaunchKernelGGL((gemm_bf16_kernel<false, 4, 2, 2, 4>), grid, dim3(512), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_sum_splits(const float* part, int nsplit, int64_t stride, int64_t count, float* out,
                             hipStream_t st) {
  hipLaunchKernelGGL(sum_splits_kernel, dim3(stride_blocks((count + 3) / 4, 256)), dim3(256), 0, st, part, nsplit,
                     stride, count, out);
  return hipGetLastError();
}

}  // namespace pg
