// Forward of the fused tied LM head + logit softcap + cross-entropy for gfx950.
//
// What is computed (per scored row t): z = H[t] . E^T (tied head: trios issue #19, approach
// table, "Tied embeddings"), s = c tanh(z / c) (the fused softcapped cross-entropy of the HYDRA Golf stack list),
// nats = logsumexp(s) - s[y[t]] (trios issue, "Контекст": cross-entropy). The T x V logits never
// reach memory.
//
// Kernel layout (bf16, D in {32..512}):
//   * one workgroup = 8 waves (two per SIMD) = 256 token rows; each wave keeps the bf16 hidden
//     rows of its 32 tokens in registers as the B operand of v_mfma_f32_32x32x16_bf16 (lane l:
//     token l % 32, half l / 32 of the hidden width);
//   * the embedding streams through LDS in tiles of 64 vocabulary rows, double-buffered, loaded
//     with global_load_lds_dwordx4 (no VGPR round trip) into a padded or XOR-swizzled layout;
//   * each 32 x 32 accumulator holds 16 vocabulary rows of one token per lane, so the softcap and
//     the log-sum-exp run per lane with no cross-lane traffic until the very end;
//   * for 0 < c <= 40 the log-sum-exp uses the fixed shift c (|s| <= c): no running maximum, no
//     rescaling. A block whose logits all satisfy |z| <= c/8 evaluates the cap by the tanh series
//     (one exp2 per logit); otherwise by exp2, fma, rcp (three transcendentals per logit);
//   * the epilogue of one vocabulary block is interleaved with the MFMA chain of the next block;
//   * a variant also writes, for training, the gradient of every logit up to a per-row factor
//     (see FwdCore, DZ);
//   * a grid smaller than the chip (few scored rows) splits the vocabulary across workgroups and
//     merges the partial sums in a second kernel, in a fixed order.
#include "pg_common.h"
#include "pg_internal.h"
#include "pg_tile.h"

namespace pg {

struct FwdParams {
  const uint16_t* H;
  const uint16_t* E;
  const int32_t* target;
  const int32_t* rows;    // compacted scored rows, or nullptr (row i = i)
  const int32_t* n_dev;   // device row count, or nullptr (use n_host)
  int64_t n_host;
  int V;
  int n_vtiles;
  int splits_host;        // > 0: number of vocabulary splits; 0: derived on the device
  Softcap sc;
  int direct;             // 1: one split, write nats / lse directly
  float* nats;
  float* lse;
  float* part_l;
  float* part_m;
  float* s_target;
  uint16_t* dz;           // unnormalised dZ blocks (the kernels that write them), else unused
  int64_t ldz;            // vocabulary rows of dz (V rounded up to the tile)
  const int8_t* Eq;       // int8 head (the kernel that reads it; E is then unused): q[V, D]
  const float* qscale;    // and its per-row scales [V]
};

__device__ __forceinline__ int device_splits(int64_t n, int n_vtiles, int grid) {
  int rt = (int)((n + kRowsPerWG - 1) / kRowsPerWG);
  if (rt <= 0) return 1;
  int s = grid / rt;
  return s < 1 ? 1 : (s > n_vtiles ? n_vtiles : s);
}

// LDS fragment reads issued this many MFMA steps ahead of their use. Two steps cover the LDS
// latency under the epilogue work between MFMAs; four keep 16 more VGPRs live and make the D = 512
// kernels spill. Two take 5460 instead of 6005 shader cycles per tile, but the launch time is the
// same: the kernel is power-limited and its clock falls by as much.
constexpr int kPrefetch = 2;

#ifndef PG_FWD_TOK_BLOCKS
#define PG_FWD_TOK_BLOCKS 1
#endif
// 32-token MFMA column blocks per wave in the forward (see WaveShape).
constexpr int kFwdTokBlocks = PG_FWD_TOK_BLOCKS;

// ASYM: separate caps for z >= 0 and z < 0, each side with its own constants in both epilogue
// forms; a template parameter so that it compiles to a kernel of its own.
// DZ (fixed shift, one cap): the epilogue also stores, for every logit, the unnormalised gradient
//   d = 2^t t (t - K),  t = s log2 e - M  (the exponent it sums),  K = -2 M,
// in the dZ block layout. Since s / c = 1 + t / M, the softcap's slope is 1 - (s / c)^2 =
// -t (t - K) / M^2, so the normalised dZ of a row is d 2^(M - lse log2 e) (-1 / M^2) - [v = y] slope,
// a per-row factor applied after this kernel, where lse is known (the target element is rewritten
// then as well).
// Q8 (D = 512, fixed shift, one cap): the head is the per-row int8 embedding q with scales s. Wave
// w owns rows 8 w .. 8 w + 7 of each tile. During the first MFMA chain of a tile it copies the
// int8 bytes of its rows of the next tile (4 KiB) by DMA into the tail of its own rows' region of
// the next tile buffer (from byte kQ8StageOff of the 8 padded rows, 8320 bytes), and during the
// second chain it turns them, row by row from the front, into the bf16 rows bf16(float(q) s) of
// that region; the tile's barrier then publishes them. bf16 row p ends before int8 row p + 1
// begins, so no byte is overwritten before it is read, and no wave touches another's region: the
// staging needs no LDS of its own and no barrier. The bytes are biased (q ^ 0x80 = q + 128 as an
// unsigned byte, which converts in one instruction), and fma(q + 128, s, -128 s) is float(q) s
// rounded once, as the product is; the bf16 rounding is the hardware's round-to-nearest-even.
template <int D, bool FIXED, int NB, bool ASYM, bool DZ = false, bool Q8 = false>
struct FwdCore {
  static_assert(!DZ || FIXED, "unnormalised dZ needs the fixed shift");
  static_assert(!Q8 || (D == 512 && NB == 1 && FIXED && !ASYM && !DZ), "int8 tiles: the D = 512 fixed-shift forward");
  using TL = TileLayout<D>;
  static constexpr int kQ8RowsPerWave = kVocabTile / 8;       // rows of a tile each wave stages
  static constexpr int kQ8WaveBytes = kQ8RowsPerWave * D;    // int8 bytes each wave stages (4 KiB)
  // where those bytes land in the wave's region of kQ8RowsPerWave padded rows: its last 4 KiB
  static constexpr int kQ8StageOff = kQ8RowsPerWave * TL::PITCH - kQ8WaveBytes;
  static_assert(!Q8 || (TL::PAD && kQ8StageOff % 16 == 0 &&
                        (kQ8RowsPerWave - 2) * TL::PITCH + 2 * D <= kQ8StageOff + (kQ8RowsPerWave - 1) * D),
                "bf16 row p must end before int8 row p + 1 begins");
  static constexpr int KS = D / 16;
  static constexpr int kWaves = WaveShape<NB>::kWaves;
  static constexpr int kLoads = embed_loads_per_wave<D, kWaves>();
  const lds_char* lds;
  const uint16_t* E;
  const int8_t* Eq;      // Q8
  const float* qscale;   // Q8
  float qs;              // Q8: scale of tile row kQ8RowsPerWave * wave + (lane % 8) of the staged tile
  int wave, lane;
  int h, col, V;
  Softcap sc;
  bf16x8 hf[NB][KS];
  float lsum[NB];
  float mrun[NB];
  int exact_left;   // blocks still to take the exact form before the series is tried again (uniform)
  uint16_t* dzblk[NB];   // DZ: block (its token block, vocabulary block 0); wave-uniform
  int dzlane;            // DZ: this lane's elements in a block (offsets lane * 8 and 512 + lane * 8)
  // The target logit is taken from the accumulators the log-sum-exp sums, so that the two share
  // every rounding: ykey is the target id when this lane holds its logit (lane half h holds rows
  // with ((v >> 2) & 1) == h of every 32-row block), else -1. ty is, with the fixed shift, the very
  // term 2^t that the exp-sum added for the target (-1 until found); with a running maximum, the
  // target's s log2 e (-inf until found).
  int ykey[NB];
  float ty[NB];

  // (s log2 e) - M (fixed shift) and s log2 e (running maximum) of logit z. The cap form is chosen
  // by the template parameter, so a symmetric kernel carries no code or constants of the other side.
  __device__ __forceinline__ float shifted(float z) const {
    return ASYM ? capped_shifted_sc(z, sc) : capped_shifted(z, sc.alpha, sc.invK);
  }
  __device__ __forceinline__ float log2cap(float z) const {
    if (ASYM) return capped_log2(z, sc);
    return sc.c > 0.f ? sc.M + capped_shifted(z, sc.alpha, sc.invK) : z * kLog2e;
  }

  // The term 2^t the exp-sum adds for logit z in each form: the operations of the pipelined stages
  // below (and of part_exact), in the same order, so the value is the one that was summed.
  __device__ __forceinline__ float term_exact(float z) const { return fexp2(shifted(z)); }
  __device__ __forceinline__ float term_series(float z) const {
    const bool neg = ASYM && z < 0.f;
    const float u = z * z;
    float q = __builtin_fmaf(neg ? sc.q2n : sc.q2, u, neg ? sc.q1n : sc.q1);
    q = __builtin_fmaf(q, u, sc.q0);
    return fexp2(__builtin_fmaf(z, q, -sc.M));
  }

  // After the epilogue of the block at vbase: a lane holding its target's logit there keeps the
  // target's term (FIXED; `series` says which form the sum took) or s log2 e (running maximum).
  // Wave-uniform branch: only blocks that hold some lane's target pay for the select.
  __device__ __forceinline__ void take_target(const f32x16 (&acc)[NB], int vbase, bool series) {
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      const bool hit = (ykey[tb] >> 5) == (vbase >> 5);
      if (__any(hit)) {
        const int y = ykey[tb] & 31;
        const int ri = 4 * (y >> 3) + (y & 3);     // accumulator register of row y of the block
        float z = acc[tb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) z = ri == r ? acc[tb][r] : z;
        if (hit) {
          if (!FIXED) ty[tb] = log2cap(z);
          else ty[tb] = series ? term_series(z) : term_exact(z);
        }
      }
    }
  }

  // DZ: eight values of this lane (accumulator registers 8 j8 .. 8 j8 + 7 of the block whose
  // vocabulary rows start at vbase) as one 16-byte store into the block layout.
  __device__ __forceinline__ void store8(const float* vals, int vbase, int tb, int j8) const {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)vals[e];
    *reinterpret_cast<bf16x8*>(dzblk[tb] + (int64_t)(vbase >> 5) * 1024 + dzlane + 512 * j8) = o;
  }

  // DZ: the slope factor of the stored gradient from the exponent t = s log2 e - M: t (t - K) for
  // z >= 0; with asymmetric caps, (t + dza_n)(t + dzb_n) dzw_n for z < 0 (the same row factor
  // -2^(M - lse log2 e) / M^2 then turns either into the gradient).
  __device__ __forceinline__ float dz_slope(float t, bool neg) const {
    if (!ASYM) return t * (t - sc.K);
    return neg ? (t + sc.dza_n) * (t + sc.dzb_n) * sc.dzw_n : t * (t - sc.K);
  }

  // DZ, not pipelined: the exact exponent t of each logit, d = 2^t times its slope factor; MASKED
  // stores 0 for rows >= V.
  template <bool MASKED>
  __device__ __forceinline__ void dz_exact(const f32x16& acc, int vbase, int tb) const {
    float d[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float t = shifted(acc[r]);
      d[r] = fexp2(t) * dz_slope(t, ASYM && acc[r] < 0.f);
      if (MASKED) d[r] = (vbase + 8 * (r >> 2) + 4 * h + (r & 3)) < V ? d[r] : 0.f;
    }
    store8(d, vbase, tb, 0);
    store8(d + 8, vbase, tb, 1);
  }

  __device__ __forceinline__ void chain(int buf, int vb, f32x16 (&acc)[NB]) const {
    logit_blocks<D, NB>(lds, buf, vb, h, col, hf, acc);
  }

  // Q8: this wave's staged bytes in buffer buf.
  __device__ __forceinline__ const lds_char* q8_stage(int buf) const {
    return lds + buf * TL::TILEB + kQ8RowsPerWave * wave * TL::PITCH + kQ8StageOff;
  }
  // Q8: the scale load of this wave's staged rows (lane l: row l % 8), issued with the DMA.
  __device__ __forceinline__ void q8_scale(int tile) {
    const int v = min(tile * kVocabTile + kQ8RowsPerWave * wave + (lane & 7), V - 1);
    qs = qscale[v];
  }
  // Q8: DMA piece j of this wave's staged rows (1 KiB: two rows of D int8), rows past the end of
  // the vocabulary repeating the last row (their logits are masked).
  __device__ __forceinline__ void q8_dma(int tile, int buf, int j) const {
    const int r = kQ8RowsPerWave * wave + 2 * j + (lane >> 5);
    const int v = min(tile * kVocabTile + r, V - 1);
    lds_dma16(Eq + (int64_t)v * D + 16 * (lane & 31), q8_stage(buf) + j * 1024);
  }
  // Q8: staged row p of this wave in buffer buf, lane l's 8 bytes (elements 8 l .. 8 l + 7).
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __device__ __forceinline__ u32x2 q8_read(int buf, int p) const {
    return *(const __attribute__((address_space(3))) u32x2*)(q8_stage(buf) + p * D + 8 * lane);
  }
  // Q8: those 8 elements as bf16(float(q) s) into the row's logical chunk `lane` of buffer buf.
  __device__ __forceinline__ void q8_write(int buf, int p, u32x2 raw) const {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const int r = kQ8RowsPerWave * wave + p;
    const float sc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qs), p));
    const float nb = -128.0f * sc;
    const uint32_t w[2] = {raw[0] ^ 0x80808080u, raw[1] ^ 0x80808080u};
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f32x2 f;
      f[0] = __builtin_fmaf((float)((w[e >> 1] >> (16 * (e & 1))) & 0xffu), sc, nb);
      f[1] = __builtin_fmaf((float)((w[e >> 1] >> (16 * (e & 1) + 8)) & 0xffu), sc, nb);
      o[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
    }
    *(__attribute__((address_space(3))) u32x4*)(lds + buf * TL::TILEB + r * TL::PITCH + lane * 16) = o;
  }
  // Q8: a whole tile into buffer buf, not overlapped (first tile, and tiles after a partial one).
  __device__ __forceinline__ void q8_load_tile(int tile, int buf) {
    q8_scale(tile);
#pragma unroll
    for (int j = 0; j < kQ8WaveBytes / 1024; ++j) q8_dma(tile, buf, j);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int p = 0; p < kQ8RowsPerWave; ++p) q8_write(buf, p, q8_read(buf, p));
  }

  // Exp-sum with the fixed shift M, exact softcap. Register r holds vocabulary row
  // vbase + 8 (r/4) + 4 h + r%4; MASKED drops rows >= V.
  template <bool MASKED>
  __device__ __forceinline__ float part_exact(const f32x16& acc, int vbase) const {
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float w = fexp2(shifted(acc[r]));
      if (MASKED) {
        const int v = vbase + 8 * (r >> 2) + 4 * h + (r & 3);
        part += v < V ? w : 0.f;
      } else {
        part += w;
      }
    }
    return part;
  }

  // Running-maximum variant for c = 0 and caps above the fixed-shift range.
  template <bool MASKED>
  __device__ __forceinline__ void online(const f32x16& acc, int vbase, int tb) {
    float s2[16];
    float bm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = vbase + 8 * (r >> 2) + 4 * h + (r & 3);
      s2[r] = (!MASKED || v < V) ? log2cap(acc[r]) : -INFINITY;
      bm = fmaxf(bm, s2[r]);
    }
    const float mn = fmaxf(mrun[tb], bm);
    if (mn != -INFINITY) {
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) part += fexp2(s2[r] - mn);
      lsum[tb] = lsum[tb] * fexp2(mrun[tb] - mn) + part;
      mrun[tb] = mn;
    }
  }

  // Epilogue outside the interleaved steady state (first, last and partial blocks).
  template <bool MASKED>
  __device__ __forceinline__ void epilogue(const f32x16 (&acc)[NB], int vbase) {
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      if (FIXED) lsum[tb] += part_exact<MASKED>(acc[tb], vbase);
      else online<MASKED>(acc[tb], vbase, tb);
      if (DZ) dz_exact<MASKED>(acc[tb], vbase, tb);
    }
  }

  // MFMA chain of block (buf, vb) with NST-stage per-logit work on the pending full block `prev`,
  // software pipelined by hand: k-step k issues the LDS read of step k + kPrefetch, the MFMA of
  // step k and stage s of the element group that started s steps earlier (stage(s, e, z) for the
  // logits z = prev[e / 16][e % 16] of the group), so that dependent VALU operations sit one MFMA
  // step apart. The group starts are spread over all the steps that let a group finish within the
  // chain, which evens out the VALU work per MFMA (6110 -> 5990 shader cycles per D = 512 tile
  // against starting one group per step from step 0). Scheduling barriers
  // keep each step's instructions together. With LOAD the chain also issues this wave's pieces of
  // the load of embedding tile load_tile into LDS buffer load_buf, spread over its steps. Wave
  // priority is staged over the tile by tile_step_priority.
  // Q8: LOAD issues the int8 DMA of load_tile into buffer load_buf instead (pieces on steps 0, 4, 8,
  // 12, the scale load with the first), and CONVERT turns the staged bytes there into bf16 rows
  // (row p read on step 4 p, converted and stored on step 4 p + 2, after a wait for the DMA).
  template <bool LOAD, int NST, bool CONVERT = false, typename Stage>
  __device__ __forceinline__ void pipelined(int buf, int vb, f32x16 (&a)[NB], const f32x16 (&prev)[NB], int load_tile,
                                            int load_buf, Stage&& stage) {
    constexpr int NE = NB * 16;                     // logits of `prev` per lane
    constexpr int EPC = (NE + KS - 1) / KS;         // elements per group
    constexpr int NG = (NE + EPC - 1) / EPC;        // element groups
    constexpr int SPAN = KS - NST + 1 > NG ? KS - NST + 1 : NG;   // steps on which a group can start
    constexpr int NSTEP = (SPAN + NST - 1) > KS ? (SPAN + NST - 1) : KS;
    constexpr int PF = kPrefetch < KS ? kPrefetch : KS;
    const int row = vb * 32 + col;
    const lds_char* rbase = lds + buf * TL::TILEB + row * TL::PITCH;
    const int sw = TL::swz(row);
    auto frag = [&](int ks) -> bf16x8 {
      return *(const __attribute__((address_space(3))) bf16x8*)(rbase + ((h * KS + ks) ^ sw) * 16);
    };
    bf16x8 fr[KS];
#pragma unroll
    for (int k = 0; k < PF; ++k) fr[k] = frag(k);
    constexpr int LOAD_EVERY = (KS / kLoads) < 4 ? ((KS / kLoads) < 1 ? 1 : KS / kLoads) : 4;
    PieceBase pb{};
    if (LOAD && !Q8 && TL::PAD) pb = piece_base<D>(lds, load_tile, load_buf, wave);
    u32x2 qraw{};
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
      if (k < KS) tile_step_priority<KS>(vb, k);
      if (k + PF < KS) fr[k + PF] = frag(k + PF);
      if constexpr (Q8) {
        constexpr int kPieces = kQ8WaveBytes / 1024;
        if (LOAD && k == 0) q8_scale(load_tile);
        if (LOAD && k % 4 == 0 && k / 4 < kPieces) q8_dma(load_tile, load_buf, k / 4);
        if (CONVERT && k == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (CONVERT && k % 4 == 0 && k / 4 < kQ8RowsPerWave) qraw = q8_read(load_buf, k / 4);
        if (CONVERT && k % 4 == 2 && k / 4 < kQ8RowsPerWave) q8_write(load_buf, k / 4, qraw);
      } else if (LOAD && k % LOAD_EVERY == 0 && k / LOAD_EVERY < kLoads) {
        if constexpr (TL::PAD) load_embed_piece_padded<D, kWaves>(pb, E, V, lane, k / LOAD_EVERY);
        else load_embed_piece<D, kWaves>(lds, E, V, load_tile, load_buf, wave, lane, k / LOAD_EVERY);
      }
      if (k < KS) {
        if (NB == 2) lds_wait_upto((k + PF < KS ? k + PF : KS - 1) - k);
        mfma_step<NB, KS>(a, fr[k], hf, k);
      }
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        // group g starts at step (g SPAN) / NG: the starts spread over every step that still lets
        // its last stage finish within the chain, one group per step at most
        const int s0 = k - st;
        if (s0 < 0 || s0 >= SPAN) continue;
        const int g = (s0 * NG + SPAN - 1) / SPAN;
        if (g >= NG || (g * SPAN) / NG != s0) continue;
#pragma unroll
        for (int e = g * EPC; e < (g + 1) * EPC && e < NE; ++e) stage(st, e, prev[e / 16][e % 16]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_finish<NB>(a);
  }

  // MFMA chain of block (buf, vb) with the exp-sum of the pending full block `prev` (fixed shift).
  // Two forms, both pipelined into the chain:
  //   series (|z| <= c/8): u = z^2, q = Q(u), 2^(z q - M), sum: five VALU and one exp2 per logit. It
  //     is speculative: when some |z| of `prev` exceeds c/8 (a wave-uniform branch) the exact sum
  //     replaces it after the chain, and the next blocks take the exact form directly;
  //   exact: 2^(z alpha), fma, rcp, 2^(K r), sum: three transcendentals per logit, any z.
  // With asymmetric caps both forms take each side's constants, and the series needs both sides
  // capped (below the smaller cap / 8); otherwise they take the exact form.
  // After a series miss the exact form runs for kExactRun blocks, then the series is tried again, so
  // inputs whose logits are mostly large pay the speculation once per kExactRun blocks.
  static constexpr int kExactRun = 16;
  // Returns true when the sums of `prev` came from the series (take_target needs the form).
  template <bool LOAD, bool CONVERT = false>
  __device__ __forceinline__ bool chain_with_epilogue(int buf, int vb, f32x16 (&a)[NB], const f32x16 (&prev)[NB],
                                                      int vprev, int load_tile = 0, int load_buf = 0) {
    constexpr int NE = NB * 16;
    static_assert(!CONVERT || Q8, "conversion of staged rows: int8 tiles only");
    if (!FIXED) {   // running maximum (c = 0 or caps above the fixed-shift range)
      if (LOAD)
        for (int i = 0; i < kLoads; ++i) load_embed_piece<D, kWaves>(lds, E, V, load_tile, load_buf, wave, lane, i);
      tile_stage_priority(vb, false);
      chain(buf, vb, a);
      tile_stage_priority(vb, true);
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) online<false>(prev[tb], vprev, tb);
      return false;
    }
    float part[NB] = {};
    float q[NE];
    float w[DZ ? NE : 1];   // DZ: the slope factor of t, then the stored value
    // DZ adds a stage: 4 also forms the slope factor, 5 multiplies it by 2^t, 6 stores eight at a time
    constexpr int NST = DZ ? 7 : 6;
    if (exact_left > 0 || (ASYM && !(sc.thr > 0.f))) {
      pipelined<LOAD, NST, CONVERT>(buf, vb, a, prev, load_tile, load_buf, [&](int st, int e, float z) {
        const bool neg = ASYM && z < 0.f;
        switch (st) {
          case 0: q[e] = z * (neg ? sc.alpha_n : sc.alpha); break;
          case 1: q[e] = fexp2(q[e]); break;
          case 2: { const float ik = neg ? sc.invK_n : sc.invK; q[e] = __builtin_fmaf(q[e], ik, ik); break; }
          case 3: q[e] = frcp(q[e]); break;                                  // K r = (s - c) log2 e
          case 4:
            if (ASYM) q[e] += neg ? sc.M_n - sc.M : 0.f;
            if (DZ) w[e] = dz_slope(q[e], neg);
            q[e] = fexp2(q[e]);
            break;
          case 5:
            part[e / 16] += q[e];
            if (DZ) w[e] = w[e] * q[e];
            break;
          default:
            if (DZ && (e & 7) == 7) store8(&w[e - 7], vprev, e / 16, (e & 15) >> 3);
            break;
        }
      });
      // as for the series below: a use of the sums right here keeps the compiler from sinking the
      // whole epilogue past the chain to where lsum is next read (it would then run after the
      // MFMAs instead of between them)
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) asm volatile("" ::"v"(part[tb]));
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) lsum[tb] += part[tb];
      if (exact_left > 0) --exact_left;
      return false;
    }
    float u[NE];
    float amax = 0.f;
    pipelined<LOAD, NST, CONVERT>(buf, vb, a, prev, load_tile, load_buf, [&](int st, int e, float z) {
      switch (st) {
        case 0: u[e] = z * z; amax = fmaxf(amax, fabsf(z)); break;
        case 1: {   // asymmetric caps: each side's own coefficients (q0 = log2 e is shared)
          const bool neg = ASYM && z < 0.f;
          q[e] = __builtin_fmaf(neg ? sc.q2n : sc.q2, u[e], neg ? sc.q1n : sc.q1);
          break;
        }
        case 2: q[e] = __builtin_fmaf(q[e], u[e], sc.q0); break;
        case 3:
          if (ASYM && DZ) w[e] = z * q[e];                       // s log2 e
          q[e] = __builtin_fmaf(z, q[e], -sc.M);                 // t (the form term_series repeats)
          break;
        case 4:
          if (ASYM && DZ) {
            // w = s log2 e here; |s| <= min(caps) / 8, so the slope factor can be formed as
            // (s log2 e)^2 M^2 / M_side^2 - M^2 without cancellation: one select instead of three
            const float tp = w[e];
            w[e] = __builtin_fmaf(tp * (z < 0.f ? sc.dzw_n : 1.f), tp, -sc.M * sc.M);
          } else if (DZ) {
            w[e] = dz_slope(q[e], false);
          }
          q[e] = fexp2(q[e]);
          break;
        case 5:
          part[e / 16] += q[e];
          if (DZ) w[e] = w[e] * q[e];
          break;
        default:
          if (DZ && (e & 7) == 7) store8(&w[e - 7], vprev, e / 16, (e & 15) >> 3);
          break;
      }
    });
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) asm volatile("" ::"v"(part[tb]));   // keep the speculation in the pipeline
    const bool series = __all(amax <= sc.thr);
    if (!series) {   // the exact sums replace the series; DZ stores again
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) {
        part[tb] = part_exact<false>(prev[tb], vprev);
        if (DZ) dz_exact<false>(prev[tb], vprev, tb);
      }
      exact_left = kExactRun;
    }
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) lsum[tb] += part[tb];
    return series;
  }
};

template <int D, bool FIXED, int NB, bool ASYM, bool DZ = false, bool Q8 = false>
__global__ __launch_bounds__(WaveShape<NB>::kThreads) __attribute__((amdgpu_waves_per_eu(3 - NB, 3 - NB)))
void fwd_mfma_kernel(FwdParams p) {
  using TL = TileLayout<D>;
  constexpr int KS = D / 16;
  constexpr int kTokPerWave = WaveShape<NB>::kTok;
  constexpr int kFwdWaves = WaveShape<NB>::kWaves;
  __shared__ __attribute__((aligned(1024))) char smem[2 * TL::TILEB];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar addressing
  const int h = lane >> 5, col = lane & 31;

  const int64_t n = p.n_dev ? (int64_t)(*p.n_dev) : p.n_host;
  const int rt_count = (int)((n + kRowsPerWG - 1) / kRowsPerWG);
  const int S = p.splits_host > 0 ? p.splits_host : device_splits(n, p.n_vtiles, gridDim.x);
  const int id = blockIdx.x;
  if (id >= rt_count * S) return;
  const int rt = id / S, split = id % S;
  const int tps = (p.n_vtiles + S - 1) / S;
  const int t_begin = split * tps;
  const int t_end = min(t_begin + tps, p.n_vtiles);
  const int V = p.V;
  const int64_t tok0 = (int64_t)rt * kRowsPerWG + wave * kTokPerWave;   // first token of this wave

  FwdCore<D, FIXED, NB, ASYM, DZ, Q8> core;
  const lds_char* lds = (const lds_char*)smem;
  core.lds = lds;
  core.E = p.E;
  core.Eq = p.Eq;
  core.qscale = p.qscale;
  core.wave = wave;
  core.lane = lane;
  core.h = h;
  core.col = col;
  core.V = V;
  core.sc = p.sc;
  core.exact_left = 0;

  // ---- the first embedding tile goes out first, so that its latency overlaps the prologue
  const int ntiles = t_end - t_begin;
  if (ntiles > 0) {
    if constexpr (Q8) {   // its DMA and scale load now, the conversion after the hidden rows' loads
      core.q8_scale(t_begin);
#pragma unroll
      for (int j = 0; j < core.kQ8WaveBytes / 1024; ++j) core.q8_dma(t_begin, 0, j);
    } else {
      load_embed_tile<D, kFwdWaves>(lds, p.E, V, t_begin, 0, wave, lane);
    }
  }

  // ---- this lane's tokens: hidden row halves into registers (B operands of the MFMA)
  // (token and row indices are recomputed after the main loop, so that they hold no registers)
  auto token = [&](int tb) -> int64_t { return tok0 + tb * 32 + col; };
  auto row_of = [&](int64_t t) -> int64_t {
    const int64_t ic = t < n ? t : n - 1;
    return p.rows ? (int64_t)p.rows[ic] : ic;
  };
  core.dzlane = lane * 8;
#pragma unroll
  for (int tb = 0; tb < NB; ++tb) {
    core.lsum[tb] = 0.f;
    core.mrun[tb] = -INFINITY;
    const int64_t grow = row_of(token(tb));
    const bf16x8* src = reinterpret_cast<const bf16x8*>(p.H + grow * D + h * (D / 2));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) core.hf[tb][ks] = src[ks];
    // the wave's 32 tokens form one token block of dZ
    if (DZ) core.dzblk[tb] = p.dz + ((tok0 >> 5) + tb) * (p.ldz >> 5) * 1024;
    const int y = p.target[grow];

    // the target: its logit is picked from the accumulators in the main loop (take_target), by the
    // one lane and split that compute it
    const bool ok = (y >= 0) && (y < V);
    core.ykey[tb] = (ok && ((y >> 2) & 1) == h) ? y : -1;
    core.ty[tb] = FIXED ? -1.0f : -INFINITY;
  }
  if constexpr (Q8) {
    if (ntiles > 0) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int p8 = 0; p8 < core.kQ8RowsPerWave; ++p8) core.q8_write(0, p8, core.q8_read(0, p8));
    }
  }

  // ---- main loop. Only the last tile of the vocabulary can be partial; it runs the masked
  //      epilogue. Elsewhere the epilogue of the previous 32-row block is interleaved with the
  //      MFMA chain of the current one.
  const bool last_partial = (t_end == p.n_vtiles) && (V % kVocabTile != 0);
  f32x16 accp[NB];
  int vprev = -1;
  for (int i = 0; i < ntiles; ++i) {
    const int tile = t_begin + i;
    const int buf = i & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const bool next = i + 1 < ntiles;
    const int vb0 = tile * kVocabTile;
    f32x16 a0[NB];
    // the steady state spreads the next tile's load over the first chain; elsewhere it goes first
    const bool steady = !(last_partial && i + 1 == ntiles) && vprev >= 0;
    if (next && !steady) {
      if constexpr (Q8) core.q8_load_tile(tile + 1, buf ^ 1);
      else load_embed_tile<D, kFwdWaves>(lds, p.E, V, tile + 1, buf ^ 1, wave, lane);
    }
    if (last_partial && i + 1 == ntiles) {
      core.chain(buf, 0, a0);
      if (vprev >= 0) {
        core.template epilogue<false>(accp, vprev);
        core.take_target(accp, vprev, false);
      }
      f32x16 a1[NB];
      core.chain(buf, 1, a1);
      core.template epilogue<true>(a0, vb0);
      core.take_target(a0, vb0, false);
      core.template epilogue<true>(a1, vb0 + 32);
      core.take_target(a1, vb0 + 32, false);
      vprev = -1;
    } else if (vprev < 0) {
      core.chain(buf, 0, a0);
      const bool ser = core.template chain_with_epilogue<false>(buf, 1, accp, a0, vb0);
      core.take_target(a0, vb0, ser);
      vprev = vb0 + 32;
    } else {
      bool ser;
      if (next) ser = core.template chain_with_epilogue<true>(buf, 0, a0, accp, vprev, tile + 1, buf ^ 1);
      else ser = core.template chain_with_epilogue<false>(buf, 0, a0, accp, vprev);
      core.take_target(accp, vprev, ser);
      // the int8 head: the second chain turns the staged rows into the next tile's buffer
      if (Q8 && next) ser = core.template chain_with_epilogue<false, Q8>(buf, 1, accp, a0, vb0, tile + 1, buf ^ 1);
      else ser = core.template chain_with_epilogue<false>(buf, 1, accp, a0, vb0);
      core.take_target(a0, vb0, ser);
      vprev = vb0 + 32;
    }
  }
  if (vprev >= 0) {
    core.template epilogue<false>(accp, vprev);
    core.take_target(accp, vprev, false);
  }

  // ---- combine the two lane halves (each holds 16 of every 32 vocabulary rows) and write out.
  //      With the fixed shift nats = ln 2 (log2 l - log2 e_y), where e_y is the target's own term of
  //      the sum l: since l >= e_y, nats >= 0 (log2_ratio floors a rounding of the hardware log2
  //      below 0 at 0), and nats = 0 exactly when e_y is all of l (V = 1).
  //      With a running maximum m, nats = ln 2 (m + log2 l - s_y log2 e), where l >= 1 (the maximum's
  //      own term) and m >= s_y log2 e.
#pragma unroll
  for (int tb = 0; tb < NB; ++tb) {
    float l = core.lsum[tb], m = core.mrun[tb];
    const float l2 = __shfl_xor(l, 32);
    if (FIXED) {
      l += l2;
    } else {
      const float m2 = __shfl_xor(m, 32);
      lse_merge(m, l, m2, l2);
    }
    const float ty = fmaxf(core.ty[tb], __shfl_xor(core.ty[tb], 32));   // the half that found it
    const bool found = FIXED ? ty >= 0.f : ty > -INFINITY;
    // log2 of the target's term (fixed shift) or its s log2 e; NaN when the target is not in [0, V)
    const float sy = found ? (FIXED ? flog2(ty) : ty) : __builtin_nanf("");
    const int64_t tok = token(tb);
    if (h == 0 && tok < n) {
      const int64_t grow = row_of(tok);
      if (p.direct) {
        const float lse2 = (FIXED ? p.sc.M : m) + flog2(l);
        p.nats[grow] = kLn2 * (FIXED ? log2_ratio(l, sy) : lse2 - sy);
        if (p.lse) p.lse[grow] = kLn2 * lse2;
      } else {
        p.part_l[(int64_t)split * n + tok] = l;
        if (!FIXED) p.part_m[(int64_t)split * n + tok] = m;
        // the split whose tiles hold the target writes it; split 0 marks a target outside [0, V)
        const int y = p.target[grow];
        if (found || (split == 0 && !(y >= 0 && y < V))) p.s_target[tok] = sy;
      }
    }
  }
}

// Merge the per-split partial sums of each compacted row, in split order.
__global__ __launch_bounds__(256) void fwd_finalize_kernel(FwdParams p, int main_grid, int fixed) {
  const int64_t n = p.n_dev ? (int64_t)(*p.n_dev) : p.n_host;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int S = p.splits_host > 0 ? p.splits_host : device_splits(n, p.n_vtiles, main_grid);
  // partials in split order; the loads go out eight at a time so that their latencies overlap
  constexpr int kBatch = 8;
  float lse2;
  if (fixed) {
    float l = 0.f;
    int s = 0;
    for (; s + kBatch <= S; s += kBatch) {
      float v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) v[j] = p.part_l[(int64_t)(s + j) * n + i];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) l += v[j];
    }
    for (; s < S; ++s) l += p.part_l[(int64_t)s * n + i];
    // s_target holds log2 of the target's own term of l (see fwd_mfma_kernel)
    const int64_t r = p.rows ? (int64_t)p.rows[i] : i;
    p.nats[r] = kLn2 * log2_ratio(l, p.s_target[i]);
    if (p.lse) p.lse[r] = kLn2 * (p.sc.M + flog2(l));
    return;
  } else {
    float m = -INFINITY, l = 0.f;
    int s = 0;
    for (; s + kBatch <= S; s += kBatch) {
      float vm[kBatch], vl[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        vm[j] = p.part_m[(int64_t)(s + j) * n + i];
        vl[j] = p.part_l[(int64_t)(s + j) * n + i];
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) lse_merge(m, l, vm[j], vl[j]);
    }
    for (; s < S; ++s) lse_merge(m, l, p.part_m[(int64_t)s * n + i], p.part_l[(int64_t)s * n + i]);
    lse2 = m + flog2(l);
  }
  const int64_t r = p.rows ? (int64_t)p.rows[i] : i;
  p.nats[r] = kLn2 * (lse2 - p.s_target[i]);
  if (p.lse) p.lse[r] = kLn2 * lse2;
}

// Plain vector kernel for f32 inputs and hidden widths without an MFMA instantiation: one wave
// per row, lanes stride over the vocabulary with a running (max, sum) each, merged at the end.
template <typename TIn>
__device__ __forceinline__ float load_in(const TIn* p, int64_t i);
template <>
__device__ __forceinline__ float load_in<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_in<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename TIn>
__global__ __launch_bounds__(256) void fwd_generic_kernel(const TIn* H, const TIn* E, const int32_t* target,
                                                          const int32_t* rows, const int32_t* n_dev,
                                                          int64_t n_host, int D, int V, Softcap sc,
                                                          float* nats, float* lse) {
  const int lane = threadIdx.x & 63;
  const int64_t n = n_dev ? (int64_t)(*n_dev) : n_host;
  // one row per wave, grid-stride over the rows
  for (int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); i < n; i += (int64_t)gridDim.x * 4) {
    const int64_t r = rows ? (int64_t)rows[i] : i;
    const TIn* hrow = H + r * D;
    float m = -INFINITY, l = 0.f;
    for (int v = lane; v < V; v += 64) {
      const TIn* erow = E + (int64_t)v * D;
      float z = 0.f;
      for (int d = 0; d < D; ++d) z = __builtin_fmaf(load_in(hrow, d), load_in(erow, d), z);
      lse_merge(m, l, capped_log2(z, sc), 1.0f);
    }
    for (int off = 32; off >= 1; off >>= 1) {
      float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
      lse_merge(m, l, m2, l2);
    }
    if (lane == 0) {
      // the target's logit by the same loop as the lane that summed it: the same value, so
      // m >= s_y and l >= 1 (the maximum's own term) give nats >= 0
      const int y = target[r];
      float sy = __builtin_nanf("");
      if (y >= 0 && y < V) {
        const TIn* erow = E + (int64_t)y * D;
        float z = 0.f;
        for (int d = 0; d < D; ++d) z = __builtin_fmaf(load_in(hrow, d), load_in(erow, d), z);
        sy = capped_log2(z, sc);
      }
      const float lse2 = m + flog2(l);
      nats[r] = kLn2 * (lse2 - sy);
      if (lse) lse[r] = kLn2 * lse2;
    }
  }
}

// Scored-row selection: one workgroup walks the mask in chunks of 16 KiB, each thread taking 16
// consecutive rows with one aligned 16-byte load (the next chunk's load is issued before the
// current chunk is processed). Each thread counts its scored rows; a scan within each wave and the
// wave totals in wave order give its offset in the ascending list of scored rows, which it then
// writes. It also writes 0 to nats and lse of all its 16 rows with 16-byte stores: the forward
// overwrites the scored ones afterwards, in stream order. The count goes to n_out at the end.
constexpr int kCompactThreads = 1024;
__global__ __launch_bounds__(kCompactThreads) void compact_rows_kernel(const uint8_t* mask, int64_t T, int32_t* rows,
                                                                       int32_t* n_out, float* nats, float* lse) {
  constexpr int kWaves = kCompactThreads / 64;
  constexpr int64_t kChunk = (int64_t)kCompactThreads * 16;
  __shared__ int wsum[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // this thread's 16 mask bytes of the chunk at c0 (zero past T)
  auto load16 = [&](int64_t c0) -> uint4 {
    const int64_t t0 = c0 + (int64_t)tid * 16;
    if (t0 + 16 <= T) return *reinterpret_cast<const uint4*>(mask + t0);   // mask and t0 16-byte aligned
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int j = 0; j < 16; ++j)
      if (t0 + j < T) w[j >> 2] |= (uint32_t)mask[t0 + j] << (8 * (j & 3));
    return make_uint4(w[0], w[1], w[2], w[3]);
  };
  int64_t base = 0;   // scored rows before the current chunk (the same in every thread)
  uint4 cur = T > 0 ? load16(0) : make_uint4(0u, 0u, 0u, 0u);
  for (int64_t c0 = 0; c0 < T; c0 += kChunk) {
    const uint4 nxt = c0 + kChunk < T ? load16(c0 + kChunk) : make_uint4(0u, 0u, 0u, 0u);
    const int64_t t0 = c0 + (int64_t)tid * 16;
    if (t0 < T && (nats || lse)) {
      if (t0 + 16 <= T) {
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (nats) reinterpret_cast<float4*>(nats + t0)[q] = z;
          if (lse) reinterpret_cast<float4*>(lse + t0)[q] = z;
        }
      } else {
        for (int64_t t = t0; t < T; ++t) {
          if (nats) nats[t] = 0.f;
          if (lse) lse[t] = 0.f;
        }
      }
    }
    const uint32_t w[4] = {cur.x, cur.y, cur.z, cur.w};
    uint8_t m[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) m[j] = (uint8_t)(w[j >> 2] >> (8 * (j & 3)));
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) cnt += m[j] != 0;
    int x = cnt;   // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
      before += w2 < wave ? wsum[w2] : 0;
      total += wsum[w2];
    }
    int64_t pos = base + before + (x - cnt);
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (m[j]) rows[pos++] = (int32_t)(t0 + j);   // m[j] is 0 past T
    base += total;
    cur = nxt;
    __syncthreads();   // wsum is rewritten by the next chunk
  }
  if (tid == 0) *n_out = (int32_t)base;
}

// Scored-row selection for up to kCompactMultiMaxRows rows, in one launch of one workgroup per
// 4096-row chunk. Workgroup b writes 0 to nats and lse of its rows (the forward overwrites the
// scored ones afterwards), counts the scored rows of all chunks before it (rereading the mask
// there: at most 1 MiB per workgroup, with every load issued at once), then places its own rows
// with a scan over its threads; the last workgroup writes the count. Each workgroup's sum is
// exact in integers, so the list is the same as the single-workgroup kernel's.
constexpr int kCompactMultiThreads = 256;
constexpr int64_t kCompactMultiChunk = (int64_t)kCompactMultiThreads * 16;
constexpr int64_t kCompactMultiMaxRows = (int64_t)1 << 20;

// Scored (nonzero) bytes among the four of w.
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
  uint32_t t = w | (w >> 4);
  t |= t >> 2;
  t |= t >> 1;
  return __builtin_popcount(t & 0x01010101u);
}

__global__ __launch_bounds__(kCompactMultiThreads) void compact_rows_multi_kernel(const uint8_t* mask, int64_t T,
                                                                                  int32_t* rows, int32_t* n_out,
                                                                                  float* nats, float* lse) {
  constexpr int kWaves = kCompactMultiThreads / 64;
  __shared__ int wsum[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kCompactMultiChunk;
  const int64_t t0 = c0 + (int64_t)tid * 16;
  // this thread's 16 rows: mask bytes (0 past T), and zeros for nats and lse
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (t0 + 16 <= T) {   // the mask is 16-byte aligned and t0 a multiple of 16
    const uint4 v = *reinterpret_cast<const uint4*>(mask + t0);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
    for (int j = 0; j < 16; ++j)
      if (t0 + j < T) w[j >> 2] |= (uint32_t)mask[t0 + j] << (8 * (j & 3));
  }
  if (t0 < T && (nats || lse)) {
    if (t0 + 16 <= T) {
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (nats) reinterpret_cast<float4*>(nats + t0)[q] = z;
        if (lse) reinterpret_cast<float4*>(lse + t0)[q] = z;
      }
    } else {
      for (int64_t t = t0; t < T; ++t) {
        if (nats) nats[t] = 0.f;
        if (lse) lse[t] = 0.f;
      }
    }
  }
  // scored rows before this chunk: the mask bytes of [0, c0), whole 16-byte pieces
  int before_chunk = 0;
  for (int64_t o = (int64_t)tid * 16; o < c0; o += kCompactMultiChunk) {
    const uint4 v = *reinterpret_cast<const uint4*>(mask + o);
    before_chunk += nonzero_bytes(v.x) + nonzero_bytes(v.y) + nonzero_bytes(v.z) + nonzero_bytes(v.w);
  }
  const int cnt = nonzero_bytes(w[0]) + nonzero_bytes(w[1]) + nonzero_bytes(w[2]) + nonzero_bytes(w[3]);
  // inclusive scan of cnt over the wave; the wave sum of before_chunk rides along
  int x = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) before_chunk += __shfl_xor(before_chunk, off);
  __shared__ int bsum[kWaves];
  if (lane == 63) wsum[wave] = x;
  if (lane == 0) bsum[wave] = before_chunk;
  __syncthreads();
  int base = 0, before = 0, total = 0;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    base += bsum[v];
    before += v < wave ? wsum[v] : 0;
    total += wsum[v];
  }
  int64_t pos = (int64_t)base + before + (x - cnt);
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if ((w[j >> 2] >> (8 * (j & 3))) & 0xffu) rows[pos++] = (int32_t)(t0 + j);
  if (blockIdx.x == gridDim.x - 1 && tid == 0) *n_out = base + total;
}

// ------------------------------------------------------------------------------------ host side

int64_t fwd_partial_entries(int64_t T) {
  // Launch grids never exceed max(ceil(T / 256), 1024) workgroups, and splits x compacted rows
  // never exceed grid x 256.
  int64_t rt = (T + kRowsPerWG - 1) / kRowsPerWG;
  int64_t g = rt > 1024 ? rt : 1024;
  return g * kRowsPerWG;
}

FwdWorkspace fwd_workspace(int64_t T, int32_t D, int32_t V) {
  (void)D; (void)V;
  FwdWorkspace L;
  size_t o = 0;
  L.n_rows = o; o += 256;
  L.rows = o; o += align256((size_t)T * 4);
  L.s_target = o; o += align256((size_t)T * 4);
  const size_t P = (size_t)fwd_partial_entries(T);
  L.part_l = o; o += align256(P * 4);
  L.part_m = o; o += align256(P * 4);
  L.total = o;
  return L;
}

hipError_t launch_compact_rows(const uint8_t* mask, int64_t T, char* ws, const FwdWorkspace& L,
                               float* nats, float* lse, hipStream_t st) {
  int32_t* rows = reinterpret_cast<int32_t*>(ws + L.rows);
  int32_t* n_out = reinterpret_cast<int32_t*>(ws + L.n_rows);
  if (T > 0 && T <= kCompactMultiMaxRows) {
    const unsigned blocks = (unsigned)((T + kCompactMultiChunk - 1) / kCompactMultiChunk);
    hipLaunchKernelGGL(compact_rows_multi_kernel, dim3(blocks), dim3(kCompactMultiThreads), 0, st, mask, T, rows,
                       n_out, nats, lse);
  } else {
    hipLaunchKernelGGL(compact_rows_kernel, dim3(1), dim3(kCompactThreads), 0, st, mask, T, rows, n_out, nats, lse);
  }
  return hipGetLastError();
}

template <int D, bool FIXED, bool ASYM, bool DZ = false, bool Q8 = false>
static void launch_mfma(const FwdParams& p, int grid, hipStream_t st) {
  hipLaunchKernelGGL((fwd_mfma_kernel<D, FIXED, kFwdTokBlocks, ASYM, DZ, Q8>), dim3(grid),
                     dim3(WaveShape<kFwdTokBlocks>::kThreads), 0, st, p);
}

template <int D>
static void launch_mfma_d(const FwdParams& p, int grid, hipStream_t st) {
  if constexpr (D == 512 && kFwdTokBlocks == 1) {
    if (p.Eq) {   // the caller checked fwd_reads_q8
      launch_mfma<D, true, false, false, true>(p, grid, st);
      return;
    }
  }
  if (p.dz) {   // the caller checked fwd_writes_dz
    if (p.sc.asym) launch_mfma<D, true, true, true>(p, grid, st);
    else launch_mfma<D, true, false, true>(p, grid, st);
  } else if (p.sc.asym) {
    if (p.sc.fixed) launch_mfma<D, true, true>(p, grid, st);
    else launch_mfma<D, false, true>(p, grid, st);
  } else {
    if (p.sc.fixed) launch_mfma<D, true, false>(p, grid, st);
    else launch_mfma<D, false, false>(p, grid, st);
  }
}

bool fwd_writes_dz(int32_t dtype, int32_t D, float cap_pos, float cap_neg) {
  const Softcap sc = Softcap::make(cap_pos, cap_neg);
  return dtype == 0 && mfma_width(D) && sc.fixed;
}

bool fwd_reads_q8(int32_t D, float cap) {
  const Softcap sc = Softcap::make(cap, cap);
  return D == 512 && kFwdTokBlocks == 1 && sc.fixed && !sc.asym;
}

hipError_t launch_fwd(const void* H, const void* E, int32_t dtype, const int32_t* target,
                      const uint8_t* mask, int64_t T, int32_t D, int32_t V, float cap_pos, float cap_neg,
                      float* nats, float* lse, char* ws, const DeviceInfo& dev, hipStream_t st, uint16_t* dz,
                      const int8_t* eq, const float* qscale) {
  if (T == 0) return hipSuccess;
  if (dz && !fwd_writes_dz(dtype, D, cap_pos, cap_neg)) return hipErrorInvalidValue;
  if (eq && (dz || dtype != 0 || cap_pos != cap_neg || !qscale || !fwd_reads_q8(D, cap_pos)))
    return hipErrorInvalidValue;
  const FwdWorkspace L = fwd_workspace(T, D, V);
  const Softcap sc = Softcap::make(cap_pos, cap_neg);
  const int32_t* rows = nullptr;
  const int32_t* n_dev = nullptr;
  if (mask) {
    hipError_t e = launch_compact_rows(mask, T, ws, L, nats, lse, st);
    if (e != hipSuccess) return e;
    rows = reinterpret_cast<const int32_t*>(ws + L.rows);
    n_dev = reinterpret_cast<const int32_t*>(ws + L.n_rows);
  }

  if (dtype != 0 || !mfma_width(D)) {
    const unsigned blocks = stride_blocks(T, 4);
    if (dtype == 0)
      hipLaunchKernelGGL(fwd_generic_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st,
                         (const uint16_t*)H, (const uint16_t*)E, target, rows, n_dev, T, D, V, sc, nats, lse);
    else
      hipLaunchKernelGGL(fwd_generic_kernel<float>, dim3(blocks), dim3(256), 0, st,
                         (const float*)H, (const float*)E, target, rows, n_dev, T, D, V, sc, nats, lse);
    return hipGetLastError();
  }

  FwdParams p{};
  p.H = (const uint16_t*)H;
  p.E = (const uint16_t*)E;
  p.target = target;
  p.rows = rows;
  p.n_dev = n_dev;
  p.n_host = T;
  p.V = V;
  p.n_vtiles = (V + kVocabTile - 1) / kVocabTile;
  p.sc = sc;
  p.nats = nats;
  p.lse = lse;
  p.part_l = reinterpret_cast<float*>(ws + L.part_l);
  p.part_m = reinterpret_cast<float*>(ws + L.part_m);
  p.s_target = reinterpret_cast<float*>(ws + L.s_target);
  p.dz = dz;
  p.ldz = (int64_t)p.n_vtiles * kVocabTile;
  p.Eq = eq;
  p.qscale = qscale;

  const int64_t rt = (T + kRowsPerWG - 1) / kRowsPerWG;
  const int ncu = dev.cu_count > 0 ? (dev.cu_count < 1024 ? dev.cu_count : 1024) : 256;
  int grid;
  if (!mask) {
    int64_t s = ncu / rt;
    s = s < 1 ? 1 : (s > p.n_vtiles ? p.n_vtiles : s);
    p.splits_host = (int)s;
    p.direct = (s == 1);
    grid = (int)(rt * s);
  } else {
    p.splits_host = 0;
    p.direct = 0;
    grid = (int)(rt > ncu ? rt : ncu);
  }

  switch (D) {
    case 32: launch_mfma_d<32>(p, grid, st); break;
    case 64: launch_mfma_d<64>(p, grid, st); break;
    case 128: launch_mfma_d<128>(p, grid, st); break;
    case 256: launch_mfma_d<256>(p, grid, st); break;
    default: launch_mfma_d<512>(p, grid, st); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.direct) return e;
  const int64_t fin_blocks = (T + 255) / 256;
  hipLaunchKernelGGL(fwd_finalize_kernel, dim3((unsigned)fin_blocks), dim3(256), 0, st, p, grid, (int)sc.fixed);
  return hipGetLastError();
}

}  // namespace pg
