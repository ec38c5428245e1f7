// Pieces shared by the forward and backward kernels that stream the tied embedding through LDS
// against register-resident hidden rows (internal header).
#pragma once
#include "pg_common.h"

namespace pg {

// Shape of the token tile: NB 32-token MFMA column blocks per wave, 256 rows per workgroup.
//   NB = 1: 8 waves (two per SIMD), hidden rows of 32 tokens in VGPRs; every embedding fragment
//           read from LDS feeds one MFMA.
//   NB = 2: 4 waves (one per SIMD), hidden rows of 64 tokens in AGPRs; every fragment feeds two.
template <int NB>
struct WaveShape {
  static constexpr int kWaves = 8 / NB;
  static constexpr int kTok = 32 * NB;
  static constexpr int kThreads = 64 * kWaves;
};

// LDS layout of one embedding tile (kVocabTile rows). D = 512: one 1 KiB row per load
// instruction, rows padded to 1040 bytes so that 16 lanes reading 16 consecutive rows at the same
// column hit 16 different bank groups. Smaller D: dense rows with the 16-byte chunk index XORed by
// a function of the row (global_load_lds writes each instruction's 1 KiB contiguously, so there is
// no room for padding inside it).
template <int D>
struct TileLayout {
  static constexpr int ROWB = 2 * D;
  static constexpr bool PAD = (ROWB == 1024);
  static constexpr int PITCH = PAD ? ROWB + 16 : ROWB;
  static constexpr int TILEB = kVocabTile * PITCH;
  static constexpr int RPB = (256 / ROWB) > 1 ? (256 / ROWB) : 1;
  static constexpr int CPR = D / 8;
  static constexpr int SWZ = CPR < 16 ? CPR : 16;
  __device__ static int swz(int row) { return PAD ? 0 : (row / RPB) % SWZ; }
};

// One 16-byte-per-lane LDS DMA (global_load_lds_dwordx4: lane i's 16 bytes land at lds_base + 16 i)
// issued as assembly. Issued through the builtin, a DMA still in flight makes the compiler wait for
// every outstanding LDS read (lgkmcnt(0)) before each MFMA operand is used, which cancels the read
// prefetch of the MFMA chains; here the compiler does not see it, so completion is the caller's
// business: an explicit s_waitcnt vmcnt before the barrier that publishes the tile. M0 (the LDS base
// of the DMA) is saved and restored around it.
__device__ __forceinline__ void lds_dma16(const void* gptr, const lds_char* lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base))
      : "memory");
}

// The same DMA with the LDS address given as a 32-bit value (an SGPR).
__device__ __forceinline__ void lds_dma16_m0(const void* gptr, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(lds_addr)
      : "memory");
}

// One embedding tile from global memory into LDS buffer `buf` (LDS pointers throughout: a generic
// pointer cast back to LDS in the loop costs a null check per cast) with global_load_lds_dwordx4
// (1 KiB per instruction, no VGPR round trip), spread over `nwaves` waves. Rows past the end of
// the vocabulary repeat the last row (valid memory; their logits are masked by the caller).
template <int D, int NWAVES>
__device__ __forceinline__ void load_embed_tile(const lds_char* lds, const uint16_t* E, int V, int tile, int buf,
                                                int wave, int lane) {
  using TL = TileLayout<D>;
  constexpr int NI = kVocabTile * TL::ROWB / 1024;
  const int v0 = tile * kVocabTile;
#pragma unroll
  for (int j = wave; j < NI; j += NWAVES) {
    const int byte = j * 1024 + lane * 16;
    const int row = byte / TL::ROWB;
    const int pchunk = (byte % TL::ROWB) / 16;
    const int lchunk = pchunk ^ TL::swz(row);
    const int v = min(v0 + row, V - 1);
    const char* g = reinterpret_cast<const char*>(E + (int64_t)v * D) + lchunk * 16;
    lds_dma16(g, lds + buf * TL::TILEB + (TL::PAD ? j * TL::PITCH : j * 1024));
  }
}

// The same tile load split into per-wave pieces, so that the loads can be spread over the MFMA
// chain that runs meanwhile (a burst of 1 KiB LDS DMAs right after a barrier stalls every wave on
// issue, and with it the MFMAs): embed_loads_per_wave<D, NWAVES>() pieces, piece i issued by
// load_embed_piece.
template <int D, int NWAVES>
__host__ __device__ constexpr int embed_loads_per_wave() {
  return (kVocabTile * TileLayout<D>::ROWB / 1024 + NWAVES - 1) / NWAVES;
}
// Per-tile bases of the pieces of padded (D = 512) tiles, where piece i of wave w is the whole row
// w + NWAVES i: the LDS address of the wave's first row in the buffer and its vocabulary row. Both
// are made opaque to the compiler, so that each piece's address is one scalar add from them: left
// to itself, the compiler hoists every piece's offsets out of the loop as invariants, which do not
// fit the SGPRs and come back as VALU lane reads in every chain.
struct PieceBase {
  uint32_t lds;   // LDS address of row `wave` of the buffer
  int row;        // vocabulary row of that row
};
template <int D>
__device__ __forceinline__ PieceBase piece_base(const lds_char* lds, int tile, int buf, int wave) {
  using TL = TileLayout<D>;
  PieceBase b;
  b.lds = (uint32_t)(uintptr_t)(lds + buf * TL::TILEB + wave * TL::PITCH);
  b.row = tile * kVocabTile + wave;
  asm volatile("" : "+s"(b.lds), "+s"(b.row));
  return b;
}
template <int D, int NWAVES>
__device__ __forceinline__ void load_embed_piece_padded(const PieceBase& b, const uint16_t* E, int V, int lane, int i) {
  using TL = TileLayout<D>;
  static_assert(TL::PAD, "rows of 1 KiB");
  const int v = min(b.row + i * NWAVES, V - 1);
  lds_dma16_m0(reinterpret_cast<const char*>(E + (int64_t)v * D) + lane * 16, b.lds + i * NWAVES * TL::PITCH);
}

template <int D, int NWAVES>
__device__ __forceinline__ void load_embed_piece(const lds_char* lds, const uint16_t* E, int V, int tile, int buf, int wave,
                                                 int lane, int i) {
  using TL = TileLayout<D>;
  constexpr int NI = kVocabTile * TL::ROWB / 1024;
  const int j = wave + i * NWAVES;
  if (NI % NWAVES != 0 && j >= NI) return;
  const int v0 = tile * kVocabTile;
  const int byte = j * 1024 + lane * 16;
  const int row = byte / TL::ROWB;
  const int pchunk = (byte % TL::ROWB) / 16;
  const int lchunk = pchunk ^ TL::swz(row);
  const int v = min(v0 + row, V - 1);
  const char* g = reinterpret_cast<const char*>(E + (int64_t)v * D) + lchunk * 16;
  lds_dma16(g, lds + buf * TL::TILEB + (TL::PAD ? j * TL::PITCH : j * 1024));
}

// v_mfma_f32_32x32x16_bf16 with the B operand (hidden rows) read straight from AGPRs and the
// accumulator in VGPRs. Written as inline assembly because the compiler otherwise copies AGPR
// operands back into VGPRs before every MFMA. Hazards the compiler cannot see here are covered
// by hand: the first MFMA of a chain takes an inline-constant zero accumulator (no VALU write
// before an MFMA read), a chain of MFMAs on one accumulator is a same-size srcC/vdst overlap
// (no wait states), and mfma_drain() keeps VALU readers of the result 24 wait states away.
// One embedding fragment against both token blocks: the two MFMAs stay adjacent so that the
// two accumulation chains alternate in the matrix pipeline.
__device__ __forceinline__ void mfma_pair_b_agpr(f32x16& c0, f32x16& c1, const bf16x8& a, const bf16x8& b0,
                                                 const bf16x8& b1) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\tv_mfma_f32_32x32x16_bf16 %1, %2, %4, %1"
      : "+v"(c0), "+v"(c1) : "v"(a), "a"(b0), "a"(b1));
}
__device__ __forceinline__ void mfma_pair_b_agpr_first(f32x16& c0, f32x16& c1, const bf16x8& a, const bf16x8& b0,
                                                       const bf16x8& b1) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %2, %3, 0\n\tv_mfma_f32_32x32x16_bf16 %1, %2, %4, 0"
      : "=&v"(c0), "=&v"(c1) : "v"(a), "a"(b0), "a"(b1));
}
__device__ __forceinline__ void mfma_drain(f32x16& a0, f32x16& a1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a0), "+v"(a1));
}

// Wave priority for the chains of a two-block vocabulary tile. When two waves of a SIMD share one
// matrix pipe the arbiter favours the older wave at equal priority, so over any stretch where the
// two run at the same level the older one issues first and the younger one finishes that stretch
// alone. Priority therefore falls with progress (the wave that is behind wins), and the stretches
// shrink towards the end of the tile, because the last one is what the younger wave runs alone
// before the barrier: 3 over block 0, then 2, 1 and 0 from chain steps 0, P1 and P0 of block 1.
// Measured on the D = 512 forward: 6110 shader cycles per tile against 6165 with four equal
// stretches (the older wave's wait at the barrier falls from about 640 to 540 cycles).
template <int KS>
__device__ __forceinline__ void tile_step_priority(int vb, int k) {
  constexpr int P1 = KS * 5 / 8, P0 = KS - (KS / 8 > 0 ? KS / 8 : 1);
  if (vb == 0) {
    if (k == 0) __builtin_amdgcn_s_setprio(3);
  } else {
    if (k == 0) __builtin_amdgcn_s_setprio(2);
    else if (k == P1) __builtin_amdgcn_s_setprio(1);
    else if (k == P0) __builtin_amdgcn_s_setprio(0);
  }
}
// The same levels for a chain issued as a whole: before (second_half = false) and after it.
__device__ __forceinline__ void tile_stage_priority(int vb, bool second_half) {
  if (vb == 0) {
    if (second_half) __builtin_amdgcn_s_setprio(2); else __builtin_amdgcn_s_setprio(3);
  } else {
    if (second_half) __builtin_amdgcn_s_setprio(0); else __builtin_amdgcn_s_setprio(1);
  }
}

// Wait until at most n LDS operations of this wave are outstanding (n <= 4). LDS reads return
// in order, so with n younger reads in flight the oldest one has landed.
__device__ __forceinline__ void lds_wait_upto(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt lgkmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt lgkmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt lgkmcnt(3)" ::: "memory"); break;
    default: asm volatile("s_waitcnt lgkmcnt(4)" ::: "memory"); break;
  }
}

// One MFMA step of the chain: the embedding fragment `a` against every token block.
template <int NB, int KS>
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[NB], const bf16x8& a, const bf16x8 (&hf)[NB][KS], int ks) {
  if constexpr (NB == 2) {
    if (ks == 0) mfma_pair_b_agpr_first(acc[0], acc[1], a, hf[0][ks], hf[1][ks]);
    else mfma_pair_b_agpr(acc[0], acc[1], a, hf[0][ks], hf[1][ks]);
  } else {
    if (ks == 0) {
      const f32x16 zero = {};
      acc[0] = mfma32x32x16(a, hf[0][ks], zero);
    } else {
      acc[0] = mfma32x32x16(a, hf[0][ks], acc[0]);
    }
  }
}

// End of a chain: the assembly form needs its wait states before VALU readers by hand.
template <int NB>
__device__ __forceinline__ void mfma_finish(f32x16 (&acc)[NB]) {
  if constexpr (NB == 2) mfma_drain(acc[0], acc[1]);
}

// Z^T blocks: 32 vocabulary rows (vb*32 ... of LDS buffer `buf`) against this lane's NB tokens.
// Accumulator register r holds vocabulary row 8 (r/4) + 4 h + r%4 of the block.
template <int D, int NB>
__device__ __forceinline__ void logit_blocks(const lds_char* lds, int buf, int vb, int h, int col,
                                             const bf16x8 (&hf)[NB][D / 16], f32x16 (&acc)[NB]) {
  using TL = TileLayout<D>;
  constexpr int KS = D / 16;
  const int row = vb * 32 + col;
  const lds_char* rbase = lds + buf * TL::TILEB + row * TL::PITCH;
  const int sw = TL::swz(row);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int chunk = (h * KS + ks) ^ sw;
    const bf16x8 a = *(const __attribute__((address_space(3))) bf16x8*)(rbase + chunk * 16);
    mfma_step<NB, KS>(acc, a, hf, ks);
  }
  mfma_finish<NB>(acc);
}

}  // namespace pg
