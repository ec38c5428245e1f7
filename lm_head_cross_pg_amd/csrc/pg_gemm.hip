// bf16 GEMM with float32 accumulation for the two products of the backward, dH = g dZ E and
// dE = g dZ^T H, on gfx950 (v_mfma_f32_32x32x16_bf16).
//
// A workgroup owns a 256 x 256 output tile and runs 4 waves, one per SIMD, in a 2 x 2 grid; each
// wave accumulates 128 x 128 of the tile in sixteen 32 x 32 accumulators, which fill its AGPRs. k
// advances in stages of SPS 32-deep sub-stages (one 32 x 32 dZ block along k each); B and A are
// filled by global_load_lds_dwordx4 into LDS rings of NS and NS + AL stages.
//
// Why this shape: the operand streams mix a unique stream from HBM (dZ) with a stream that every
// workgroup shares from L2 (E or H). A 256 x 256 tile moves 32 KiB per 4.2 MFLOP chunk, against
// 40 KiB for 128 x 512, and at T = 65536 it still gives 512 tiles (two full rounds on 256 CUs);
// larger tiles do not fit the register file. The two column tiles of a row tile are launched 8
// workgroup ids apart: workgroups are dealt to the 8 XCDs in turn, so the pair runs on one XCD at
// the same time and its L2 serves the second read of their dZ rows (the HBM fetch stays at one
// pass over dZ). With 128 x 128 per wave, a wave reads 8 KiB of LDS fragments per 16-deep step
// for 16 MFMAs; two waves of 128 x 64 per SIMD read 6 KiB for 8 MFMAs each, so that fragment reads
// and DMA writes together needed 128 bytes of LDS bandwidth per clock at the full matrix rate,
// against 96 here. The lone wave has no partner on its SIMD to cover a wait, so it reads the
// fragments of the next 16-deep step during the MFMAs of the current one, and the barrier of stage
// s + 1 sits before the last step of stage s (all of stage s's fragments are in registers by
// then): that step's MFMAs run while the first fragments of stage s + 1 are read. The loop issues
// about 5 other instructions per MFMA, near what a lone wave can issue in an MFMA's 32 cycles, so
// every instruction in it counts: the per-lane load addresses are formed before the loop, and
// 64-deep stages (SPS = 2) halve the per-stage work of waits, barrier and ring counters.
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
// In the dZ block layout, chunk 64 j + L holds registers 8 j .. 8 j + 7 of lane L. The plain
// 16-byte reads of dH take chunks 64 ks + lane, 16 consecutive ones per read phase. A 32-lane
// phase of the transposed 8-byte reads of dE takes four runs of 4 chunks at offsets 0, 32, 64
// and 96, which fall on the same banks, so a_swz XORs chunk bits 2-3 with bits 5-6: the four runs
// land on four different quarters of the 64 banks. Within an aligned run of 16 chunks this only
// permutes, so the dH reads stay conflict-free; it is its own inverse.
__device__ __forceinline__ int a_swz(int c) { return c ^ (((c >> 5) & 3) << 2); }

// The loads of each stage are split around the barrier: A of stage s + NS + AL - 1 before barrier
// s + 1 (into the slot of stage s - 1), B of stage s + NS after it (into the slot stage s has
// finished reading). A thus runs AL stages further ahead than B. With 32-deep stages, rings of
// 3 + 1, 4 + 1, 4 + 2 and 3 + 3 stages measured the same: the feed's latency does not pace the
// product, so the 64-deep stages take the smallest rings, 2 + 1 (160 KiB).
// The product of one workgroup: wid is its index along x (the output tile), zsplit its k split
// of nsplit; smem is the kernel's LDS (NS stages of B and NS + AL of A).
template <bool A_TRANS, int NS, int AL, int SPS>
__device__ __forceinline__ void gemm_body(const GemmParams& g, int64_t wid, int zsplit, int nsplit, lds_char* smem) {
  constexpr int WM = 4, WN = 4, NW = 4, WGN = 2;
  // a stage is SPS sub-stages of 32 k (one 32 x 32 dZ block along k each), i.e. 2 SPS 16-deep
  // steps; each sub-stage's A and B tiles take 16 KiB of their stage's ring slot
  constexpr int BM = 256, BN = 256, BK = kGemmBK * SPS, KS = 2 * SPS;
  constexpr int SUBA = BM * kGemmBK * 2, SUBB = BN * kGemmBK * 2;
  constexpr int ABYTES = SUBA * SPS, BBYTES = SUBB * SPS;
  constexpr int APS = SUBA / 1024 / NW, BPS = SUBB / 1024 / NW;   // loads per wave and sub-stage
  constexpr int APW = APS * SPS, BPW = BPS * SPS, LPW = APW + BPW;
  constexpr int RPL = 1024 / (BN * 2);
  static_assert(kGemmBK == 32 && APS == 4 && BPS == 4 && RPL == 2 && (SPS == 1 || SPS == 2),
                "tile shape assumed below");
  constexpr int AST = NS + AL;   // A is issued AL stages ahead of B
  static_assert(AL >= 1 && NS * BBYTES + AST * ABYTES <= 160 * 1024, "LDS rings");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int wm = wave / WGN, wn = wave % WGN;

  const int64_t ndev = g.n_dev ? (int64_t)(*g.n_dev) : 0;
  const int64_t M = g.m_dev ? ndev : g.M;
  const int64_t K = g.k_dev ? ndev : g.K;
  const int NT = (int)((g.N + BN - 1) / BN);
  const int64_t mt = (wid / (8 * NT)) * 8 + (wid % 8);
  const int nt = (int)((wid / 8) % NT);
  const int64_t m0 = mt * BM;
  const int64_t n0 = (int64_t)nt * BN;
  if (m0 >= M) return;
  const int64_t kchunks = (K + BK - 1) / BK;
  const int64_t cps = (kchunks + nsplit - 1) / nsplit;
  const int64_t kc_begin = (int64_t)zsplit * cps;
  const int64_t kc_end = kc_begin + cps < kchunks ? kc_begin + cps : kchunks;
  const int64_t nk = kc_end > kc_begin ? kc_end - kc_begin : 0;
  const int64_t kvalid = g.k_dev ? ndev : g.kvalid;

  // A load i of a sub-stage: half q & 1 of its A block q / 2, q = wave + NW i; B load i: its rows
  // RPL q .. RPL q + RPL - 1. load_a / load_b issue load i of stage kc into ring slot `slot`. The per-lane part of each
  // address is fixed for the whole k loop; a stage adds a uniform offset (and, for B, clamps the
  // lane's row to the last one that exists, which only bites in a partial last chunk and in the
  // stages past the end that the ring issues anyway).
  const uint16_t* pa[APS];
  const uint16_t* pb[BPS];
  int jbo[BPS];   // B load i: element offset of this lane's row within a sub-stage, j ldb
#pragma unroll
  for (int i = 0; i < APS; ++i) {
    const int q = wave + NW * i;
    int64_t blk = (m0 >> 5) + (q >> 1);            // dH: token block; dE: vocabulary block
    blk = blk < g.a_mblocks ? blk : g.a_mblocks - 1;
    pa[i] = g.A + (A_TRANS ? blk : blk * g.lda) * 1024 + a_swz(64 * (q & 1) + lane) * 8;
  }
#pragma unroll
  for (int i = 0; i < BPS; ++i) {
    const int q = wave + NW * i;
    const int j = q * RPL + lane / (64 / RPL);
    const int lc = (lane % (64 / RPL)) ^ (4 * (j & 3));
    int64_t col = n0 + 8 * lc;
    col = col <= g.ldb - 8 ? col : g.ldb - 8;
    pb[i] = g.B + col;
    jbo[i] = j * (int)g.ldb;
  }
  // load i of a stage: sub-stage i / APS (resp. BPS), load i % APS of the sub-stage
  auto load_a = [&](int64_t kc, int slot, int i) {
    // dH: vocabulary block SPS kc + sub; dE: token block SPS kc + sub (clamped to the last block)
    const int64_t kb = SPS * kc + i / APS;
    const int64_t off = A_TRANS ? (kb < g.k_blocks ? kb : g.k_blocks - 1) * g.lda * 1024
                                : (kb < g.lda ? kb : g.lda - 1) * 1024;
    lds_dma16(pa[i % APS] + off, (smem + NS * BBYTES + slot * ABYTES + (i / APS) * SUBA +
                                                   (wave + NW * (i % APS)) * 1024));
  };
  auto load_b = [&](int64_t kc, int slot, int ib) {
    const int i = ib % BPS;
    const int64_t kcb = kc * BK + (ib / BPS) * kGemmBK;
    int64_t rl = kvalid - 1 - kcb;                  // last row that exists, relative to the stage
    rl = rl < BK ? rl : BK;
    const int lim = (int)rl * (int)g.ldb;          // |rl| <= BK (NS + AL + 1) and ldb <= 512
    const int r = jbo[i] < lim ? jbo[i] : lim;
    lds_dma16(pb[i] + kcb * g.ldb + r, (smem + slot * BBYTES + (ib / BPS) * SUBB + (wave + NW * i) * 1024));
  };

  const int grp = lane >> 4, li = lane & 15;
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  // fragment f of 16-deep step ks of a stage: f < WM is A block f of this wave, f >= WM is B block f - WM
  auto read_frag = [&](const lds_char* sA0, const lds_char* sB0, int kss, int f) -> bf16x8 {
    const lds_char* sA = sA0 + (kss >> 1) * SUBA;
    const lds_char* sB = sB0 + (kss >> 1) * SUBB;
    const int ks = kss & 1;
    if (f < WM) {
      const lds_char* blk = sA + (wm * WM + f) * 2048;
      // dH: lane l takes row l % 32 of the block, registers 8 ks .. 8 ks + 7 of lane l: vocabulary
      // rows 16 ks + 8 (j / 4) + 4 (l / 32) + j % 4, j = 0..7
      if (!A_TRANS)
        return *(const __attribute__((address_space(3))) bf16x8*)(blk + a_swz(64 * ks + lane) * 16);
      i16x4 part[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int t = 16 * ks + 8 * (grp >> 1) + 4 * half + (li >> 2);
        const int cg = li & 3;
        const int c = 64 * (grp & 1) + t + 32 * (cg & 1);   // registers 8 (grp & 1) .. of lane t + 32 (cg & 1)
        part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(blk + a_swz(c) * 16 + 8 * (cg >> 1)));
      }
      i16x8 v = {part[0][0], part[0][1], part[0][2], part[0][3], part[1][0], part[1][1], part[1][2], part[1][3]};
      return __builtin_bit_cast(bf16x8, v);
    }
    const int cbase = wn * (32 * WN) + (f - WM) * 32;
    const bool interleaved = !A_TRANS;
    i16x4 part[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k = 16 * ks + (interleaved ? 8 * half + 4 * (grp >> 1) : 8 * (grp >> 1) + 4 * half) + (li >> 2);
      const int c = cbase + 16 * (grp & 1) + 4 * (li & 3);
      const int addr = k * (BN * 2) + 16 * ((c >> 3) ^ (4 * (k & 3))) + 2 * (c & 7);
      part[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sB + addr));
    }
    i16x8 v = {part[0][0], part[0][1], part[0][2], part[0][3], part[1][0], part[1][1], part[1][2], part[1][3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  f32x16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  constexpr int NF = WM + WN;
  bf16x8 fa[NF], fb[NF];   // fragments of the even and of the odd 16-deep steps of a stage
  if (nk > 0) {
    // A of stages 0 .. AL - 1, then B of stage d and A of stage d + AL for d < NS, A only while
    // d + AL < NS + AL - 1 (stage d in slot d): the steady state issues A of stage s + NS + AL - 1
    // before barrier s + 1 and B of stage s + NS after it
#pragma unroll
    for (int d = 0; d < AL; ++d)
#pragma unroll
      for (int i = 0; i < APW; ++i) load_a(kc_begin + d, d, i);
#pragma unroll
    for (int d = 0; d < NS; ++d) {
#pragma unroll
      for (int i = 0; i < BPW; ++i) load_b(kc_begin + d, d, i);
      if (d + AL < NS + AL - 1)
#pragma unroll
        for (int i = 0; i < APW; ++i) load_a(kc_begin + d + AL, d + AL, i);
    }
    // issued after B of stage 0: the A loads of stages AL .. NS + AL - 2, the B loads of 1 .. NS - 1
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 1) * LPW) : "memory");
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int f = 0; f < NF; ++f) fa[f] = read_frag(smem + NS * BBYTES, smem, 0, f);
  }
  // One 16-deep step: the MFMAs on cur, with the fragments of the step after it read into nxt
  // (from the ring slots rA / rB, step rks) and loads of this stage's group interleaved: counting
  // MFMAs from gbase (the MFMAs of earlier steps in the same run of loads), load n is issued at
  // MFMA off + n every (A loads when a_loads, else B loads).
  auto mstep = [&](const bf16x8 (&cur)[NF], bf16x8 (&nxt)[NF], const lds_char* rA, const lds_char* rB, int rks,
                   bool a_loads, int gbase, int every, int off, int64_t kc_l, int slot_l) {
#pragma unroll
    for (int bn = 0; bn < WN; ++bn)
#pragma unroll
      for (int bm = 0; bm < WM; ++bm) {
        const int mi = bn * WM + bm;
        acc[bm][bn] = mfma32x32x16(cur[WM + bn], cur[bm], acc[bm][bn]);   // transposed block (epilogue)
        if (mi % 2 == 0) nxt[mi / 2] = read_frag(rA, rB, rks, mi / 2);
        const int g = gbase + mi - off;
        if (g >= 0 && g % every == 0 && g / every < (a_loads ? APW : BPW)) {
          if (a_loads) load_a(kc_l, slot_l, g / every);
          else load_b(kc_l, slot_l, g / every);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  // A loads spread over the MFMAs of steps 0 .. KS - 2, B loads over step KS - 1
  constexpr int AEVERY = (KS - 1) * WM * WN / APW, BEVERY = WM * WN / BPW;
  // ring slots of stage it (A and B) and of stage it - 1 (A), kept as counters
  int sa = 0, sb = 0, sa_prev = AST - 1;
  for (int64_t it = 0; it < nk; ++it) {
    const int sa1 = sa + 1 < AST ? sa + 1 : 0, sb1 = sb + 1 < NS ? sb + 1 : 0;
    const lds_char* sA = smem + NS * BBYTES + sa * ABYTES;
    const lds_char* sB = smem + sb * BBYTES;
    const lds_char* sA1 = smem + NS * BBYTES + sa1 * ABYTES;
    const lds_char* sB1 = smem + sb1 * BBYTES;
    const int64_t kc_n = kc_begin + it + NS;   // B of this stage and A of stage kc_n + AL - 1 are issued here
    // steps 0 .. KS - 2 (even steps on fa, odd on fb), with the A loads of stage it + NS + AL - 1
    // into the slot of stage it - 1
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      if (ks % 2 == 0) mstep(fa, fb, sA, sB, ks + 1, true, ks * WM * WN, AEVERY, 1, kc_n + AL - 1, sa_prev);
      else mstep(fb, fa, sA, sB, ks + 1, true, ks * WM * WN, AEVERY, 1, kc_n + AL - 1, sa_prev);
    }
    // every fragment of stage it is in registers; stage it + 1 landed: issued after B of stage
    // it + 1 (A of a stage goes out before its B) are NS - 2 groups of B and A loads and the A loads
    // above, in the prologue as in the loop. After the last stage the barrier and the reads below
    // are harmless: nothing is read from what they fetch.
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(APW + (NS - 2) * LPW) : "memory");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // last step: MFMAs on fb, the next stage's first fragments into fa, B loads of stage it + NS
    // into the slot of stage it
    mstep(fb, fa, sA1, sB1, 0, false, 0, BEVERY, BEVERY > 1 ? 1 : 0, kc_n, sb);
    sa_prev = sa;
    sa = sa1;
    sb = sb1;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: alpha (times the row's scale when given) * acc to C (row-scattered) or to this
  //      split's partial tile. The MFMAs take the B fragment as their first operand, so each
  //      accumulator holds its 32 x 32 block transposed: lane l has row l % 32 of the block and,
  //      in elements 4 k .. 4 k + 3, the four consecutive columns 8 k + 4 (l / 32) .. + 3, i.e. one
  //      16-byte store each (the untransposed layout took 4-byte stores, 71 us more per dH launch
  //      at the training shape).
  float* C = g.C + (int64_t)zsplit * g.split_stride;
#pragma unroll
  for (int bm = 0; bm < WM; ++bm) {
    const int64_t m = m0 + (wm * WM + bm) * 32 + (lane & 31);
    if (m < M) {
      const int64_t crow = g.crows ? (int64_t)g.crows[m] : m;
      const float f = g.row_scale ? g.alpha * g.row_scale[m] : g.alpha;
      float* crow_p = C + crow * g.ldc;
#pragma unroll
      for (int bn = 0; bn < WN; ++bn)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int64_t n = n0 + wn * (32 * WN) + bn * 32 + 8 * k + 4 * h;
          const f32x4 v = {f * acc[bm][bn][4 * k], f * acc[bm][bn][4 * k + 1], f * acc[bm][bn][4 * k + 2],
                           f * acc[bm][bn][4 * k + 3]};
          if (n + 4 <= g.N) {
            *reinterpret_cast<f32x4*>(crow_p + n) = v;   // ldc and n are multiples of 4, C 16-byte aligned
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < g.N) crow_p[n + e] = v[e];
          }
        }
    }
  }
}

// Both products' tiles are 256 x 256, with 64-deep stages, a 2-stage B ring and A one stage ahead.
constexpr int kGemmNS = 2, kGemmAL = 1, kGemmSPS = 2;
constexpr size_t kGemmLds = (size_t)(kGemmNS + kGemmNS + kGemmAL) * 256 * kGemmBK * kGemmSPS * 2;

template <bool A_TRANS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(GemmParams g) {
  __shared__ __attribute__((aligned(1024))) char smem[kGemmLds];
  gemm_body<A_TRANS, kGemmNS, kGemmAL, kGemmSPS>(g, blockIdx.x, blockIdx.z, gridDim.z, (lds_char*)smem);
}

// dH and dE in one launch: workgroups 0 .. gxa - 1 take dH's tiles, the rest dE's (ksb k splits of
// gxb tiles each). A CU that finishes its last dH tile picks up dE work at once, instead of idling
// until the slowest dH tile ends. gxa and gxb are multiples of 8, so every workgroup keeps the XCD
// its own product's id mapping gives it.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_pair_kernel(GemmParams a, GemmParams b, int64_t gxa, int64_t gxb, int ksb) {
  __shared__ __attribute__((aligned(1024))) char smem[kGemmLds];
  const int64_t w = blockIdx.x;
  if (w < gxa) gemm_body<false, kGemmNS, kGemmAL, kGemmSPS>(a, w, 0, 1, (lds_char*)smem);
  else gemm_body<true, kGemmNS, kGemmAL, kGemmSPS>(b, (w - gxa) % gxb, (int)((w - gxa) / gxb), ksb, (lds_char*)smem);
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

constexpr int kGemmBM = 256, kGemmBN = 256;
int gemm_tile_m(bool) { return kGemmBM; }
int gemm_tile_n(bool) { return kGemmBN; }

int64_t gemm_grid_x(int64_t M, int64_t N, bool) {
  const int64_t mt = (M + kGemmBM - 1) / kGemmBM, nt = (N + kGemmBN - 1) / kGemmBN;
  return nt > 1 ? 8 * nt * ((mt + 7) / 8) : mt;   // the id mapping of the kernel
}

hipError_t launch_gemm(const GemmParams& g, bool a_trans, int ksplit, hipStream_t st) {
  const int64_t gx = gemm_grid_x(g.M, g.N, a_trans);
  if (gx == 0 || ksplit < 1) return hipSuccess;
  if (gx > kMaxGrid512) return hipErrorInvalidConfiguration;   // the API layer rejects such shapes first
  const dim3 grid((unsigned)gx, 1, (unsigned)ksplit);
  if (a_trans) hipLaunchKernelGGL(gemm_bf16_kernel<true>, grid, dim3(256), 0, st, g);
  else hipLaunchKernelGGL(gemm_bf16_kernel<false>, grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_gemm_pair(const GemmParams& a, const GemmParams& b, int ksb, hipStream_t st) {
  const int64_t gxa = gemm_grid_x(a.M, a.N, false), gxb = gemm_grid_x(b.M, b.N, true);
  if (ksb < 1 || gxa % 8 != 0 || gxb % 8 != 0) {   // the id mapping needs whole groups of 8
    hipError_t e = launch_gemm(a, false, 1, st);
    return e != hipSuccess ? e : launch_gemm(b, true, ksb, st);
  }
  const int64_t n = gxa + gxb * ksb;
  if (n > kMaxGrid512) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(gemm_pair_kernel, dim3((unsigned)n), dim3(256), 0, st, a, b, gxa, gxb, ksb);
  return hipGetLastError();
}

hipError_t launch_sum_splits(const float* part, int nsplit, int64_t stride, int64_t count, float* out,
                             hipStream_t st) {
  hipLaunchKernelGGL(sum_splits_kernel, dim3(stride_blocks((count + 3) / 4, 256)), dim3(256), 0, st, part, nsplit,
                     stride, count, out);
  return hipGetLastError();
}

}  // namespace pg
