// Backward of the fused tied LM head + logit softcap + cross-entropy for gfx950.
//
// L = g * sum over scored rows of nats (repo-explainer, "The Baseline Is a Map": the backward pass of the baseline's loss).
// With p = softmax(s) per row and s = c tanh(z / c):
//   dZ[t, v] = (p[t, v] - [v == y[t]]) * (1 - (s / c)^2)   (g is applied later, in float32)
//   dH = g * dZ . E          dE = g * dZ^T . H   (LM-head part of the tied embedding's gradient)
// The logits are recomputed from H and E with the lse of the forward; dZ is written once to the
// workspace in bf16 and read by the two products.
#include "pg_common.h"
#include "pg_internal.h"
#include "pg_tile.h"

namespace pg {

template <typename TIn>
__device__ __forceinline__ float bload(const TIn* p, int64_t i);
template <>
__device__ __forceinline__ float bload<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float bload<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

// dZ of one row per wave (plain vector code; any dtype and width).
template <typename TIn>
__global__ __launch_bounds__(256) void dz_generic_kernel(const TIn* H, const TIn* E, const int32_t* target,
                                                         const float* lse, const int32_t* rows,
                                                         const int32_t* n_dev, int64_t n_host, int D, int V,
                                                         Softcap sc, uint16_t* dz) {
  const int lane = threadIdx.x & 63;
  const int64_t n = n_dev ? (int64_t)(*n_dev) : n_host;
  // one row per wave, grid-stride over the rows
  for (int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); i < n; i += (int64_t)gridDim.x * 4) {
    const int64_t r = rows ? (int64_t)rows[i] : i;
    const TIn* hrow = H + r * D;
    const int y = target[r];
    // a target outside [0, V) poisons the row (NaN nats in the forward): NaN dZ, so NaN dH and dE
    const float lse2 = (y >= 0 && y < V) ? lse[r] * kLog2e : __builtin_nanf("");
    for (int v = lane; v < V; v += 64) {
      const TIn* erow = E + (int64_t)v * D;
      float z = 0.f;
      for (int d = 0; d < D; ++d) z = __builtin_fmaf(bload(hrow, d), bload(erow, d), z);
      float s2, slope;
      capped_log2_slope(z, sc, s2, slope);                        // s log2 e, 1 - (s / c)^2
      const float p = fexp2(s2 - lse2);
      const float g = (v == y) ? p - 1.0f : p;
      dz[i * V + v] = f32_to_bf16(g * slope);
    }
  }
}

// dH[rows[i], d] = g * sum_v dZ[i, v] E[v, d]: one thread per output (plain vector code).
template <typename TIn>
__global__ __launch_bounds__(256) void dh_generic_kernel(const uint16_t* dz, const TIn* E, const int32_t* rows,
                                                         const int32_t* n_dev, int64_t n_host, int D, int V,
                                                         float g, float* dH) {
  const int64_t n = n_dev ? (int64_t)(*n_dev) : n_host;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n * D;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = idx / D;
    const int d = (int)(idx % D);
    float acc = 0.f;
    for (int v = 0; v < V; ++v) acc = __builtin_fmaf(bf16_to_f32(dz[i * V + v]), bload(E, (int64_t)v * D + d), acc);
    const int64_t r = rows ? (int64_t)rows[i] : i;
    dH[r * D + d] = g * acc;
  }
}

// dE[v, d] = g * sum_i dZ[i, v] H[rows[i], d]: one thread per output (plain vector code).
template <typename TIn>
__global__ __launch_bounds__(256) void de_generic_kernel(const uint16_t* dz, const TIn* H, const int32_t* rows,
                                                         const int32_t* n_dev, int64_t n_host, int D, int V,
                                                         float g, float* dE) {
  const int64_t n = n_dev ? (int64_t)(*n_dev) : n_host;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < (int64_t)V * D;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t v = idx / D;
    const int d = (int)(idx % D);
    float acc = 0.f;
    for (int64_t i = 0; i < n; ++i) {
      const int64_t r = rows ? (int64_t)rows[i] : i;
      acc = __builtin_fmaf(bf16_to_f32(dz[i * V + v]), bload(H, r * D + d), acc);
    }
    dE[v * D + d] = g * acc;
  }
}

// Hc[i] = H[rows[i]] for the compacted scored rows (16 bytes per thread).
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* H, const int32_t* rows, const int32_t* n_dev,
                                                          int64_t T, int D, uint16_t* Hc) {
  const int64_t cpr = D / 8;
  const int64_t n = (int64_t)(*n_dev) < T ? (int64_t)(*n_dev) : T;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n * cpr;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = idx / cpr, c = idx % cpr;
    reinterpret_cast<uint4*>(Hc + i * D)[c] = reinterpret_cast<const uint4*>(H + (int64_t)rows[i] * D)[c];
  }
}

// Zero the dH rows of unscored positions.
__global__ __launch_bounds__(256) void zero_unscored_kernel(const uint8_t* mask, int64_t T, int D, float* dH) {
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < T * D;
       idx += (int64_t)gridDim.x * blockDim.x)
    if (!mask[idx / D]) dH[idx] = 0.f;
}

// =============================================================================== MFMA path
//
// 1. bwd_dz_kernel: the forward's structure (8 waves x 32 tokens per workgroup, hidden rows in
//    registers, the embedding streamed through LDS) recomputes each 32 x 32 logit block with
//    v_mfma_f32_32x32x16_bf16 and turns it into dZ = (p - onehot) * (1 - (s/c)^2) in the epilogue,
//    which is interleaved with the next block's MFMA chain. The epilogue always takes the exact
//    softcap (three transcendentals per logit): unlike the forward's speculative series, its cost
//    does not depend on the size of the logits (at D = 512, V = 8192, T = 65536: 680 us at the
//    initialisation scale, 675 us at a trained model's, against 634 and 1005 us for the series
//    with an exact redo of the blocks it cannot take). dZ goes to the workspace as bf16 in
//    32 x 32 blocks laid out like the MFMA accumulator (described in pg_internal.h), so that
//    each 16-byte store instruction of a wave fills one contiguous KiB and each block is one
//    contiguous 2 KiB run; zero in the padding rows and columns.
// 2. The bf16 GEMM of pg_gemm.hip forms the two products from those blocks:
//      dH = g dZ E      A = dZ blocks, B = E [V][D]
//      dE = g dZ^T H    A = dZ blocks read transposed, B = H rows (compacted when masked)
//    dE splits k over several workgroups; a final kernel adds the partial tiles in a fixed order.

struct DzParams {
  const uint16_t* H;
  const uint16_t* E;
  const int32_t* target;
  const float* lse;
  const int32_t* rows;
  const int32_t* n_dev;
  int64_t n_host;
  int V;
  int n_vtiles;
  int64_t ldz;            // vocabulary extent of dZ (V rounded up to 64)
  Softcap sc;
  uint16_t* dz;
};

// ASYM: separate caps for z >= 0 and z < 0 (exact form only), compiled as a kernel of its own.
template <int D, bool CAPPED, int NB, bool ASYM>
struct DzCore {
  static constexpr int KS = D / 16;
  static constexpr int kWaves = WaveShape<NB>::kWaves;
  static constexpr int kLoads = embed_loads_per_wave<D, kWaves>();
  const lds_char* lds;
  const uint16_t* E;
  int wave, lane;
  int h, col, V;
  Softcap sc;
  bf16x8 hf[NB][KS];
  float bias[NB];      // -lse * log2 e of this lane's rows (-inf for padding rows, NaN for a
                       // target outside [0, V): the row's dZ, and with it dH and dE, become NaN)
  int ytok[NB];        // targets of this lane's rows (never matching for padding rows)
  uint16_t* dzblk[NB]; // this lane's first 8 elements of block (token block, vocabulary block 0)

  __device__ __forceinline__ void chain(int buf, int vb, f32x16 (&acc)[NB]) const {
    logit_blocks<D, NB>(lds, buf, vb, h, col, hf, acc);
  }

  // Eight dZ values of this lane (accumulator registers 8 j8 .. 8 j8 + 7 of the block whose
  // vocabulary rows start at vbase) as one 16-byte store into the block layout.
  __device__ __forceinline__ void store8(const float* vals, int vbase, int tb, int j8) const {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)vals[e];
    *reinterpret_cast<bf16x8*>(dzblk[tb] + (int64_t)(vbase >> 5) * 1024 + 512 * j8) = o;
  }

  // dZ of one block, not pipelined. MODE 1: exact softcap (either cap form), 2: no cap.
  template <int MODE, bool MASKED>
  __device__ __forceinline__ void store_block(const f32x16& acc, int vbase, int tb) const {
    const int dy = ytok[tb] - vbase;
    float vals[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int off = 8 * (r >> 2) + 4 * h + (r & 3);
      const float z = acc[r];
      float p, slope;
      if (MODE == 1) {
        float s2;
        capped_log2_slope(z, sc, s2, slope);                     // either cap form, exact
        p = fexp2(s2 + bias[tb]);
      } else {
        p = fexp2(__builtin_fmaf(z, kLog2e, bias[tb]));
        slope = 1.0f;
      }
      const float g = (off == dy) ? p - 1.0f : p;
      float val = g * slope;
      if (MASKED) val = (vbase + off < V) ? val : 0.0f;
      vals[r] = val;
    }
    store8(vals, vbase, tb, 0);
    store8(vals + 8, vbase, tb, 1);
  }

  template <bool MASKED>
  __device__ __forceinline__ void store_exact(const f32x16 (&acc)[NB], int vbase) const {
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
      if (CAPPED) store_block<1, MASKED>(acc[tb], vbase, tb);
      else store_block<2, MASKED>(acc[tb], vbase, tb);
    }
  }

  // MFMA chain of (buf, vb) with NST-stage per-logit work on the pending full block `prev`, software
  // pipelined by hand: k-step k issues the LDS read of a later step, the MFMA of step k and stage s
  // of the element group that started s steps earlier (stage(s, e, z) for the logits
  // z = prev[e / 16][e % 16] of the group; group starts spread over every step that lets a group
  // finish within the chain), so that the dependent operations of one logit sit an MFMA step apart
  // and independent logits fill the gaps. With LOAD the chain also issues this wave's pieces of the load of embedding tile
  // load_tile into LDS buffer load_buf, spread over its steps (a burst of them would stall the
  // MFMAs). Wave priority is staged over the tile by tile_step_priority.
  static constexpr int kNST = 9;   // epilogue stages
  template <bool LOAD, typename Stage>
  __device__ __forceinline__ void pipelined(int buf, int vb, f32x16 (&a)[NB], const f32x16 (&prev)[NB], int load_tile,
                                            int load_buf, Stage&& stage) {
    using TL = TileLayout<D>;
    constexpr int NST = kNST;
    constexpr int NE = NB * 16;                              // logits of `prev` per lane
    // elements per group (a power of two, so a group of eight stored together is never split), small
    // enough that every group finishes its last stage by step KS - 1 where possible
    constexpr int SPAN = KS - NST + 1 > 0 ? KS - NST + 1 : 1;   // (short chains do not come here)
    constexpr int EPC0 = (NE + SPAN - 1) / SPAN;
    constexpr int EPC = EPC0 <= 1 ? 1 : EPC0 <= 2 ? 2 : EPC0 <= 4 ? 4 : EPC0 <= 8 ? 8 : 16;
    constexpr int NG = (NE + EPC - 1) / EPC;
    constexpr int SPAN_G = KS - NST + 1 > NG ? KS - NST + 1 : NG;   // steps on which a group can start
    constexpr int NSTEP = (SPAN_G + NST - 1) > KS ? (SPAN_G + NST - 1) : KS;
    constexpr int PF = 4 < KS ? 4 : KS;
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
    if (LOAD && TL::PAD) pb = piece_base<D>(lds, load_tile, load_buf, wave);
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
      if (k < KS) tile_step_priority<KS>(vb, k);
      if (k + PF < KS) fr[k + PF] = frag(k + PF);
      if (LOAD && k % LOAD_EVERY == 0 && k / LOAD_EVERY < kLoads) {
        if constexpr (TL::PAD) load_embed_piece_padded<D, kWaves>(pb, E, V, lane, k / LOAD_EVERY);
        else load_embed_piece<D, kWaves>(lds, E, V, load_tile, load_buf, wave, lane, k / LOAD_EVERY);
      }
      if (k < KS) mfma_step<NB, KS>(a, fr[k], hf, k);
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        // group g starts at step (g SPAN_G) / NG: the starts spread over every step that still lets
        // its last stage finish within the chain, one group per step at most
        const int s0 = k - st;
        if (s0 < 0 || s0 >= SPAN_G) continue;
        const int g = (s0 * NG + SPAN_G - 1) / SPAN_G;
        if (g >= NG || (g * SPAN_G) / NG != s0) continue;
#pragma unroll
        for (int e = g * EPC; e < (g + 1) * EPC && e < NE; ++e) stage(st, e, prev[e / 16][e % 16]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_finish<NB>(a);
  }

  // MFMA chain of (buf, vb) with dZ of the pending full block `prev` formed and stored, pipelined
  // into the chain: K r = rcp(2^(z alpha) / K + 1 / K), log2 p = M + K r - lse log2 e,
  // slope 4 r (1 - r) (each side of asymmetric caps with its own constants). Short chains, no cap,
  // and asymmetric caps with one side uncapped form dZ after the chain instead.
  template <bool LOAD>
  __device__ __forceinline__ void chain_with_store(int buf, int vb, f32x16 (&a)[NB], const f32x16 (&prev)[NB],
                                                   int vprev, int load_tile = 0, int load_buf = 0) {
    if (!CAPPED || KS < 2 * kNST || (ASYM && !(sc.c > 0.f && sc.cn > 0.f))) {   // not pipelined
      if (LOAD)
        for (int i = 0; i < kLoads; ++i) load_embed_piece<D, kWaves>(lds, E, V, load_tile, load_buf, wave, lane, i);
      tile_stage_priority(vb, false);
      chain(buf, vb, a);
      tile_stage_priority(vb, true);
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) {
        if (CAPPED) store_block<1, false>(prev[tb], vprev, tb);
        else store_block<2, false>(prev[tb], vprev, tb);
      }
      return;
    }
    constexpr int NE = NB * 16;
    float q[NE], t[NE], v[NE];
    int dy[NB];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) dy[tb] = ytok[tb] - vprev;
    pipelined<LOAD>(buf, vb, a, prev, load_tile, load_buf, [&](int st, int e, float z) {
      const int tb = e / 16, r = e % 16;
      const int off = 8 * (r >> 2) + 4 * h + (r & 3);
      const bool neg = ASYM && z < 0.f;
      switch (st) {
        case 0: q[e] = z * (neg ? sc.alpha_n : sc.alpha); break;
        case 1: q[e] = fexp2(q[e]); break;
        case 2: { const float ik = neg ? sc.invK_n : sc.invK; q[e] = __builtin_fmaf(q[e], ik, ik); break; }
        case 3: q[e] = frcp(q[e]); break;                                               // K r
        case 4: t[e] = q[e] * (neg ? sc.invK_n : sc.invK);                              // r
                q[e] = q[e] + ((neg ? sc.M_n : sc.M) + bias[tb]); break;                // log2 p
        case 5: q[e] = fexp2(q[e]); t[e] = t[e] * __builtin_fmaf(-4.0f, t[e], 4.0f); break;   // p; 4 r (1 - r)
        case 6: v[e] = (off == dy[tb]) ? q[e] - 1.0f : q[e]; break;
        case 7: v[e] = v[e] * t[e]; break;
        default:
          if ((r & 7) == 7) store8(&v[e - 7], vprev, tb, r >> 3);   // eight values: one 16-byte store
          break;
      }
    });
  }
};

template <int D, bool CAPPED, int NB, bool ASYM>
__global__ __launch_bounds__(WaveShape<NB>::kThreads) __attribute__((amdgpu_waves_per_eu(3 - NB, 3 - NB)))
void bwd_dz_kernel(DzParams p) {
  using TL = TileLayout<D>;
  constexpr int KS = D / 16;
  constexpr int kTokPerWave = WaveShape<NB>::kTok;
  constexpr int kFwdWaves = WaveShape<NB>::kWaves;
  __shared__ __attribute__((aligned(1024))) char smem[2 * TL::TILEB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar addressing
  const int h = lane >> 5, col = lane & 31;
  const int64_t n = p.n_dev ? (int64_t)(*p.n_dev) : p.n_host;
  const int rt = blockIdx.x;
  if ((int64_t)rt * kRowsPerWG >= n) return;
  const int V = p.V;

  DzCore<D, CAPPED, NB, ASYM> core;
  const lds_char* lds = (const lds_char*)smem;
  core.lds = lds;
  core.E = p.E;
  core.wave = wave;
  core.lane = lane;
  core.h = h;
  core.col = col;
  core.V = V;
  core.sc = p.sc;
#pragma unroll
  for (int tb = 0; tb < NB; ++tb) {
    const int64_t tok = (int64_t)rt * kRowsPerWG + wave * kTokPerWave + tb * 32 + col;
    const bool valid = tok < n;
    const int64_t ic = valid ? tok : n - 1;
    const int64_t grow = p.rows ? (int64_t)p.rows[ic] : ic;
    const bf16x8* src = reinterpret_cast<const bf16x8*>(p.H + grow * D + h * (D / 2));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) core.hf[tb][ks] = src[ks];
    const int y = p.target[grow];
    core.bias[tb] = !valid ? -INFINITY : (y >= 0 && y < V) ? -p.lse[grow] * kLog2e : __builtin_nanf("");
    core.ytok[tb] = valid ? y : -(1 << 30);
    core.dzblk[tb] = p.dz + ((tok >> 5) * (p.ldz >> 5)) * 1024 + lane * 8;
  }

  const int ntiles = p.n_vtiles;
  const bool last_partial = (V % kVocabTile) != 0;
  f32x16 accp[NB];
  int vprev = -1;
  load_embed_tile<D, kFwdWaves>(lds, p.E, V, 0, 0, wave, lane);
  for (int i = 0; i < ntiles; ++i) {
    const int buf = i & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const bool next = i + 1 < ntiles;
    // the steady state spreads the next tile's load over its first chain; elsewhere it goes first
    const bool steady = !(last_partial && i + 1 == ntiles) && vprev >= 0;
    if (next && !steady) load_embed_tile<D, kFwdWaves>(lds, p.E, V, i + 1, buf ^ 1, wave, lane);
    const int vb0 = i * kVocabTile;
    f32x16 a0[NB];
    if (last_partial && i + 1 == ntiles) {
      core.chain(buf, 0, a0);
      if (vprev >= 0) core.template store_exact<false>(accp, vprev);
      f32x16 a1[NB];
      core.chain(buf, 1, a1);
      core.template store_exact<true>(a0, vb0);
      if (vb0 + 32 < p.ldz) core.template store_exact<true>(a1, vb0 + 32);
      vprev = -1;
    } else if (vprev < 0) {
      core.chain(buf, 0, a0);
      core.template chain_with_store<false>(buf, 1, accp, a0, vb0);
      vprev = vb0 + 32;
    } else {
      if (next) core.template chain_with_store<true>(buf, 0, a0, accp, vprev, i + 1, buf ^ 1);
      else core.template chain_with_store<false>(buf, 0, a0, accp, vprev);
      core.template chain_with_store<false>(buf, 1, accp, a0, vb0);
      vprev = vb0 + 32;
    }
  }
  if (vprev >= 0) core.template store_exact<false>(accp, vprev);
}

// The step from the forward's unnormalised dZ to what the two GEMMs read, one wave per compacted
// row i. The forward stored d = 2^t t (t - K) for every logit (t = s log2 e - M; with asymmetric
// caps, z < 0 logits carry that side's slope in the same scale), and g dZ of a non-target element
// is f d with the row's factor f = g 2^(M - lse log2 e) (-1 / M^2). This kernel
// writes the target element as (p_y - 1) slope_y / (f / g), from the row's nats and lse
// (p_y = e^-nats; s_y log2 e = (lse - nats) log2 e), then f (the dH product scales its output rows
// by it) and the hidden row times f in bf16 (the B operand of dE, whose sum runs over rows). Rows from the last
// scored row to the end of its 256-row tile are cleared: the forward wrote them from duplicated
// hidden rows, and the dE sum runs over them.
__device__ __forceinline__ void train_prep_row(int64_t i, int lane, const uint16_t* H, const int32_t* target,
                                               const float* nats, const float* lse, const int32_t* rows, int64_t n,
                                               int D, int V, int64_t nvb, const Softcap& sc, float g, uint16_t* dz,
                                               uint16_t* hs, float* row_scale) {
  uint16_t* zblk = dz + (i >> 5) * nvb * 1024;   // vocabulary block 0 of the row's token block
  const int l0 = (int)(i & 31);                  // the row's elements: those of lanes l0 and l0 + 32
  if (i >= n) {
    bf16x8 zero;
#pragma unroll
    for (int e = 0; e < 8; ++e) zero[e] = (__bf16)0.f;
    for (int64_t bv = lane; bv < nvb; bv += 64) {
      uint16_t* blk = zblk + bv * 1024;
      *reinterpret_cast<bf16x8*>(blk + 8 * l0) = zero;
      *reinterpret_cast<bf16x8*>(blk + 512 + 8 * l0) = zero;
      *reinterpret_cast<bf16x8*>(blk + 8 * (l0 + 32)) = zero;
      *reinterpret_cast<bf16x8*>(blk + 512 + 8 * (l0 + 32)) = zero;
    }
    return;
  }
  const int64_t r = rows ? (int64_t)rows[i] : i;
  // the row's hidden values go out first, so that their latency overlaps the row factor's loads
  constexpr int kMaxChunks = 1;   // D <= 512 (the MFMA widths): one 8-element chunk per lane
  bf16x8 xh[kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c)
    if (lane * 8 + c * 512 < D) xh[c] = *reinterpret_cast<const bf16x8*>(H + r * D + lane * 8 + c * 512);
  const float lse2 = lse[r] * kLog2e;
  float f = g * fexp2(sc.M - lse2) * (-sc.invM * sc.invM);
  // The target element: (p_y - 1) slope_y / (f / g), rounded to bf16. It outweighs the rest of the
  // row about V / sqrt(V) times in dH, so the row factor is then taken from the rounded value
  // (f = g val / stored): the target term becomes exact, and the other elements of the row move by
  // the same relative amount, at most 2^-9.
  const int y = target[r];
  if (y >= 0 && y < V) {
    const float nl2 = nats[r] * kLog2e;
    const float sy2 = lse2 - nl2;                                // s_y log2 e
    const float w = sy2 * (sc.asym && sy2 < 0.f ? sc.invM_n : sc.invM);   // s_y / (its side's cap)
    const float val = (fexp2(-nl2) - 1.f) * (1.f - w * w);       // (p_y - 1) slope_y
    const __bf16 stored = (__bf16)(val * (-sc.M * sc.M) * fexp2(lse2 - sc.M));
    if ((float)stored != 0.f) f = g * val / (float)stored;
    if (lane == 0) {
      const int L = l0 + 32 * ((y >> 2) & 1);
      const int r = 4 * ((y & 31) >> 3) + (y & 3);   // the accumulator register that holds row y
      zblk[(int64_t)(y >> 5) * 1024 + 512 * (r >> 3) + 8 * L + (r & 7)] = __builtin_bit_cast(uint16_t, stored);
    }
  } else {
    f = __builtin_nanf("");   // a target outside [0, V) poisons the row: NaN dH row, NaN dE
  }
  if (lane == 0) row_scale[i] = f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int d0 = lane * 8 + c * 512;
    if (d0 >= D) break;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)(f * (float)xh[c][e]);
    *reinterpret_cast<bf16x8*>(hs + i * D + d0) = o;
  }
}

__global__ __launch_bounds__(256) void train_prep_kernel(const uint16_t* H, const int32_t* target, const float* nats,
                                                         const float* lse, const int32_t* rows, const int32_t* n_dev,
                                                         int64_t n_host, int D, int V, int64_t nvb, Softcap sc,
                                                         float g, uint16_t* dz, uint16_t* hs, float* row_scale) {
  const int lane = threadIdx.x & 63;
  const int64_t n = n_dev ? (int64_t)(*n_dev) : n_host;
  const int64_t npad = (n + kRowsPerWG - 1) / kRowsPerWG * kRowsPerWG;
  // one row per wave, grid-stride over the rows up to the end of the last 256-row tile
  for (int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); i < npad; i += (int64_t)gridDim.x * 4)
    train_prep_row(i, lane, H, target, nats, lse, rows, n, D, V, nvb, sc, g, dz, hs, row_scale);
}

// ------------------------------------------------------------------------------------ host side

constexpr int kDeSplit = 4;
// 32-token MFMA column blocks per wave in the dZ kernel (see WaveShape): one (two waves per SIMD,
// which keep the matrix pipe busier than one wave with two blocks: 605 vs 750 us at D = 512,
// V = 8192, T = 65536), except at D = 256, where that shape runs out of registers.
template <int D>
constexpr int dz_tok_blocks() { return D == 256 ? 2 : 1; }

template <int D>
static void launch_dz(const DzParams& q, unsigned blocks, hipStream_t st) {
  constexpr int NB = dz_tok_blocks<D>();
  if (q.sc.asym)
    hipLaunchKernelGGL((bwd_dz_kernel<D, true, NB, true>), dim3(blocks), dim3(WaveShape<NB>::kThreads), 0, st, q);
  else if (q.sc.capped())
    hipLaunchKernelGGL((bwd_dz_kernel<D, true, NB, false>), dim3(blocks), dim3(WaveShape<NB>::kThreads), 0, st, q);
  else
    hipLaunchKernelGGL((bwd_dz_kernel<D, false, NB, false>), dim3(blocks), dim3(WaveShape<NB>::kThreads), 0, st, q);
}

BwdWorkspace bwd_workspace(int64_t T, int32_t D, int32_t V) {
  BwdWorkspace L;
  size_t o = 0;
  L.n_rows = o; o += 256;
  L.rows = o; o += align256((size_t)T * 4);
  const size_t rows_pad = (size_t)((T + kRowsPerWG - 1) / kRowsPerWG) * kRowsPerWG;
  const size_t ldz = (size_t)((V + kVocabTile - 1) / kVocabTile) * kVocabTile;
  L.dz = o; o += align256(rows_pad * ldz * 2);
  L.de_part = o; o += align256((size_t)kDeSplit * (size_t)V * (size_t)D * 4);
  L.hc = o; o += align256((size_t)T * (size_t)D * 2);
  L.total = o;
  return L;
}

hipError_t launch_bwd(const void* H, const void* E, int32_t dtype, const int32_t* target,
                      const uint8_t* mask, const float* lse, int64_t T, int32_t D, int32_t V,
                      float cap_pos, float cap_neg, float grad_scale, float* dH, float* dE, char* ws,
                      const DeviceInfo& dev, hipStream_t st) {
  const BwdWorkspace L = bwd_workspace(T, D, V);
  const Softcap sc = Softcap::make(cap_pos, cap_neg);
  const int32_t* rows = nullptr;
  const int32_t* n_dev = nullptr;
  if (mask && T > 0) {
    FwdWorkspace F{};
    F.rows = L.rows;
    F.n_rows = L.n_rows;
    hipError_t e = launch_compact_rows(mask, T, ws, F, nullptr, nullptr, st);
    if (e != hipSuccess) return e;
    rows = reinterpret_cast<const int32_t*>(ws + L.rows);
    n_dev = reinterpret_cast<const int32_t*>(ws + L.n_rows);
    if (dH) {
      hipLaunchKernelGGL(zero_unscored_kernel, dim3(stride_blocks(T * D, 256)), dim3(256), 0, st, mask, T, D, dH);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  uint16_t* dz = reinterpret_cast<uint16_t*>(ws + L.dz);
  if (dtype == 0 && mfma_width(D)) {
    GemmParams a{};
    if (T > 0) {
      DzParams q{};
      q.H = (const uint16_t*)H;
      q.E = (const uint16_t*)E;
      q.target = target;
      q.lse = lse;
      q.rows = rows;
      q.n_dev = n_dev;
      q.n_host = T;
      q.V = V;
      q.n_vtiles = (V + kVocabTile - 1) / kVocabTile;
      q.ldz = (int64_t)q.n_vtiles * kVocabTile;
      q.sc = sc;
      q.dz = dz;
      const unsigned rblk = (unsigned)((T + kRowsPerWG - 1) / kRowsPerWG);
      switch (D) {
        case 32: launch_dz<32>(q, rblk, st); break;
        case 64: launch_dz<64>(q, rblk, st); break;
        case 128: launch_dz<128>(q, rblk, st); break;
        case 256: launch_dz<256>(q, rblk, st); break;
        default: launch_dz<512>(q, rblk, st); break;
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;

      // dH = g dZ E (left out when the caller takes no dH), launched with dE below
      if (dH) {
        a.A = dz; a.lda = q.ldz / 32;
        a.a_mblocks = (int64_t)rblk * (kRowsPerWG / 32);   // token blocks of the padded dZ rows
        a.B = (const uint16_t*)E; a.ldb = D;
        a.n_dev = n_dev; a.m_dev = n_dev != nullptr; a.k_dev = 0;
        a.M = T; a.N = D; a.K = V; a.kvalid = V;
        a.alpha = grad_scale;
        a.C = dH; a.ldc = D; a.crows = rows; a.split_stride = 0;
      }
    }
    // dE = g dZ^T H, k split over workgroups when the output has few tiles
    const int64_t tiles = ((int64_t)(V + gemm_tile_m(true) - 1) / gemm_tile_m(true)) *
                          ((D + gemm_tile_n(true) - 1) / gemm_tile_n(true));
    const int ncu = dev.cu_count > 0 ? dev.cu_count : 256;
    int64_t ks = ncu / (tiles > 0 ? tiles : 1);
    ks = ks < 1 ? 1 : (ks > kDeSplit ? kDeSplit : ks);
    if (T == 0) return launch_sum_splits(nullptr, 0, (int64_t)V * D, (int64_t)V * D, dE, st);
    float* part = reinterpret_cast<float*>(ws + L.de_part);
    GemmParams b{};
    b.A = dz; b.lda = ((V + kVocabTile - 1) / kVocabTile) * (int64_t)kVocabTile / 32;
    b.a_mblocks = b.lda;                                 // vocabulary blocks of the padded dZ columns
    b.k_blocks = (int64_t)((T + kRowsPerWG - 1) / kRowsPerWG) * (kRowsPerWG / 32);   // token blocks of dZ
    b.B = (const uint16_t*)H; b.ldb = D;
    if (rows) {   // masked: the scored hidden rows, compacted, so that k runs over them directly
      uint16_t* hc = reinterpret_cast<uint16_t*>(ws + L.hc);
      hipLaunchKernelGGL(gather_rows_kernel, dim3(stride_blocks(T * (D / 8), 256)), dim3(256), 0, st, (const uint16_t*)H,
                         rows, n_dev, T, D, hc);
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
      b.B = hc;
    }
    b.n_dev = n_dev; b.m_dev = 0; b.k_dev = n_dev != nullptr;
    b.M = V; b.N = D; b.K = T; b.kvalid = T;
    b.alpha = grad_scale;
    b.C = ks > 1 ? part : dE; b.ldc = D; b.crows = nullptr; b.split_stride = (int64_t)V * D;
    // both products in one launch when dH is taken (T > 0 here)
    hipError_t e = dH ? launch_gemm_pair(a, b, (int)ks, st) : launch_gemm(b, true, (int)ks, st);
    if (e != hipSuccess || ks == 1) return e;
    return launch_sum_splits(part, (int)ks, (int64_t)V * D, (int64_t)V * D, dE, st);
  }
  const unsigned rblocks = stride_blocks(T, 4);
  const unsigned hblocks = stride_blocks(T * D, 256);
  const unsigned eblocks = stride_blocks((int64_t)V * D, 256);
  if (T > 0) {
    if (dtype == 0) {
      hipLaunchKernelGGL(dz_generic_kernel<uint16_t>, dim3(rblocks), dim3(256), 0, st, (const uint16_t*)H,
                         (const uint16_t*)E, target, lse, rows, n_dev, T, D, V, sc, dz);
      if (dH)
        hipLaunchKernelGGL(dh_generic_kernel<uint16_t>, dim3(hblocks), dim3(256), 0, st, dz, (const uint16_t*)E,
                           rows, n_dev, T, D, V, grad_scale, dH);
    } else {
      hipLaunchKernelGGL(dz_generic_kernel<float>, dim3(rblocks), dim3(256), 0, st, (const float*)H,
                         (const float*)E, target, lse, rows, n_dev, T, D, V, sc, dz);
      if (dH)
        hipLaunchKernelGGL(dh_generic_kernel<float>, dim3(hblocks), dim3(256), 0, st, dz, (const float*)E,
                           rows, n_dev, T, D, V, grad_scale, dH);
    }
  }
  if (dtype == 0)
    hipLaunchKernelGGL(de_generic_kernel<uint16_t>, dim3(eblocks), dim3(256), 0, st, dz, (const uint16_t*)H,
                       rows, n_dev, T, D, V, grad_scale, dE);
  else
    hipLaunchKernelGGL(de_generic_kernel<float>, dim3(eblocks), dim3(256), 0, st, dz, (const float*)H,
                       rows, n_dev, T, D, V, grad_scale, dE);
  return hipGetLastError();
}

TrainWorkspace train_workspace(int64_t T, int32_t D, int32_t V) {
  TrainWorkspace W;
  size_t o = 0;
  W.fwd = o; o += align256(fwd_workspace(T, D, V).total);
  W.bwd = o; o += align256(bwd_workspace(T, D, V).total);
  W.row_scale = o; o += align256((size_t)T * 4);
  W.total = o;
  return W;
}

hipError_t launch_train(const void* H, const void* E, int32_t dtype, const int32_t* target,
                        const uint8_t* mask, int64_t T, int32_t D, int32_t V, float cap_pos, float cap_neg,
                        float grad_scale, float* nats, float* lse, float* dH, float* dE, char* ws,
                        const DeviceInfo& dev, hipStream_t st) {
  const TrainWorkspace W = train_workspace(T, D, V);
  const bool fused = T > 0 && fwd_writes_dz(dtype, D, cap_pos, cap_neg);
  const BwdWorkspace L = bwd_workspace(T, D, V);
  uint16_t* dz = reinterpret_cast<uint16_t*>(ws + W.bwd + L.dz);
  hipError_t e = launch_fwd(H, E, dtype, target, mask, T, D, V, cap_pos, cap_neg, nats, lse, ws + W.fwd, dev, st,
                            fused ? dz : nullptr);
  if (e != hipSuccess) return e;
  if (!fused)
    return launch_bwd(H, E, dtype, target, mask, lse, T, D, V, cap_pos, cap_neg, grad_scale, dH, dE, ws + W.bwd,
                      dev, st);

  const Softcap sc = Softcap::make(cap_pos, cap_neg);
  const FwdWorkspace F = fwd_workspace(T, D, V);
  const int32_t* rows = mask ? reinterpret_cast<const int32_t*>(ws + W.fwd + F.rows) : nullptr;
  const int32_t* n_dev = mask ? reinterpret_cast<const int32_t*>(ws + W.fwd + F.n_rows) : nullptr;
  if (mask && dH) {
    hipLaunchKernelGGL(zero_unscored_kernel, dim3(stride_blocks(T * D, 256)), dim3(256), 0, st, mask, T, D, dH);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t ldz = (int64_t)((V + kVocabTile - 1) / kVocabTile) * kVocabTile;
  const int64_t rblk = (T + kRowsPerWG - 1) / kRowsPerWG;
  uint16_t* hs = reinterpret_cast<uint16_t*>(ws + W.bwd + L.hc);
  float* row_scale = reinterpret_cast<float*>(ws + W.row_scale);
  hipLaunchKernelGGL(train_prep_kernel, dim3(stride_blocks(rblk * kRowsPerWG, 4)), dim3(256), 0, st,
                     (const uint16_t*)H, target, nats, lse, rows, n_dev, T, D, V, ldz / 32, sc, grad_scale, dz, hs,
                     row_scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // dH = f dZ' E, row by row (left out when the caller takes no dH)
  GemmParams a{};
  if (dH) {
    a.A = dz; a.lda = ldz / 32;
    a.a_mblocks = rblk * (kRowsPerWG / 32);
    a.B = (const uint16_t*)E; a.ldb = D;
    a.n_dev = n_dev; a.m_dev = n_dev != nullptr; a.k_dev = 0;
    a.M = T; a.N = D; a.K = V; a.kvalid = V;
    a.alpha = 1.f;
    a.C = dH; a.ldc = D; a.crows = rows; a.split_stride = 0; a.row_scale = row_scale;
  }

  // dE = dZ'^T (f H): the row factors sit in the scaled hidden rows
  const int64_t tiles = ((int64_t)(V + gemm_tile_m(true) - 1) / gemm_tile_m(true)) *
                        ((D + gemm_tile_n(true) - 1) / gemm_tile_n(true));
  const int ncu = dev.cu_count > 0 ? dev.cu_count : 256;
  int64_t ks = ncu / (tiles > 0 ? tiles : 1);
  ks = ks < 1 ? 1 : (ks > kDeSplit ? kDeSplit : ks);
  float* part = reinterpret_cast<float*>(ws + W.bwd + L.de_part);
  GemmParams b{};
  b.A = dz; b.lda = ldz / 32;
  b.a_mblocks = b.lda;
  b.k_blocks = rblk * (kRowsPerWG / 32);
  b.B = hs; b.ldb = D;
  b.n_dev = n_dev; b.m_dev = 0; b.k_dev = n_dev != nullptr;
  b.M = V; b.N = D; b.K = T; b.kvalid = T;
  b.alpha = 1.f;
  b.C = ks > 1 ? part : dE; b.ldc = D; b.crows = nullptr; b.split_stride = (int64_t)V * D;
  // both products in one launch when dH is taken (dE's workgroups fill the CUs dH's last ones leave)
  e = dH ? launch_gemm_pair(a, b, (int)ks, st) : launch_gemm(b, true, (int)ks, st);
  if (e != hipSuccess || ks == 1) return e;
  return launch_sum_splits(part, (int)ks, (int64_t)V * D, (int64_t)V * D, dE, st);
}

}  // namespace pg
