// Backward of the fused tied LM head + logit softcap + cross-entropy for gfx950.
//
// L = g * sum over scored rows of nats (repo-explainer, "The Baseline Is a Map": loss.backward()).
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
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t n = n_dev ? (int64_t)(*n_dev) : n_host;
  if (i >= n) return;
  const int64_t r = rows ? (int64_t)rows[i] : i;
  const TIn* hrow = H + r * D;
  const int y = target[r];
  const float lse2 = lse[r] * kLog2e;
  for (int v = lane; v < V; v += 64) {
    const TIn* erow = E + (int64_t)v * D;
    float z = 0.f;
    for (int d = 0; d < D; ++d) z = __builtin_fmaf(bload(hrow, d), bload(erow, d), z);
    float p, slope;
    if (sc.c > 0.f) {
      const float rk = capped_shifted(z, sc.alpha, sc.invK);   // K r
      p = fexp2(sc.M + rk - lse2);
      const float rr = rk * sc.invK;                            // r = 1 / (1 + e^(2z/c))
      slope = 4.0f * rr * (1.0f - rr);                          // 1 - tanh^2 = 4 r (1 - r)
    } else {
      p = fexp2(z * kLog2e - lse2);
      slope = 1.0f;
    }
    const float g = (v == y) ? p - 1.0f : p;
    dz[i * V + v] = f32_to_bf16(g * slope);
  }
}

// dH[rows[i], d] = g * sum_v dZ[i, v] E[v, d]: one thread per output (plain vector code).
template <typename TIn>
__global__ __launch_bounds__(256) void dh_generic_kernel(const uint16_t* dz, const TIn* E, const int32_t* rows,
                                                         const int32_t* n_dev, int64_t n_host, int D, int V,
                                                         float g, float* dH) {
  const int64_t n = n_dev ? (int64_t)(*n_dev) : n_host;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = idx / D;
  const int d = (int)(idx % D);
  if (i >= n) return;
  float acc = 0.f;
  for (int v = 0; v < V; ++v) acc = __builtin_fmaf(bf16_to_f32(dz[i * V + v]), bload(E, (int64_t)v * D + d), acc);
  const int64_t r = rows ? (int64_t)rows[i] : i;
  dH[r * D + d] = g * acc;
}

// dE[v, d] = g * sum_i dZ[i, v] H[rows[i], d]: one thread per output (plain vector code).
template <typename TIn>
__global__ __launch_bounds__(256) void de_generic_kernel(const uint16_t* dz, const TIn* H, const int32_t* rows,
                                                         const int32_t* n_dev, int64_t n_host, int D, int V,
                                                         float g, float* dE) {
  const int64_t n = n_dev ? (int64_t)(*n_dev) : n_host;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t v = idx / D;
  const int d = (int)(idx % D);
  if (v >= V) return;
  float acc = 0.f;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t r = rows ? (int64_t)rows[i] : i;
    acc = __builtin_fmaf(bf16_to_f32(dz[i * V + v]), bload(H, r * D + d), acc);
  }
  dE[v * D + d] = g * acc;
}

// Zero the dH rows of unscored positions.
__global__ __launch_bounds__(256) void zero_unscored_kernel(const uint8_t* mask, int64_t T, int D, float* dH) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * D) return;
  if (!mask[idx / D]) dH[idx] = 0.f;
}

// =============================================================================== MFMA path
//
// 1. bwd_dz_kernel: the forward's structure (8 waves x 32 tokens per workgroup, hidden rows in
//    registers, the embedding streamed through LDS) recomputes each 32 x 32 logit block with
//    v_mfma_f32_32x32x16_bf16 and turns it into dZ = (p - onehot) * (1 - (s/c)^2) in the epilogue,
//    which is interleaved with the next block's MFMA chain. dZ goes to the workspace as bf16,
//    [rows rounded up to 256][V rounded up to 64], zero in the padding.
// 2. gemm_bf16_kernel: C = alpha * A B on 256 x 256 tiles (4 waves of 128 x 128, 16 MFMA
//    accumulators each), 32-deep k-chunks in a 3-stage LDS ring filled by global_load_lds. An
//    operand stored with its k index slow (dZ^T for dE, E and H for both products) is read with
//    ds_read_b64_tr_b16, which hands each lane 4 consecutive k of one column: no transpose pass.
//      dH = g dZ E      A = dZ [rows][V] (k = v contiguous), B = E [V][D]
//      dE = g dZ^T H    A = dZ read transposed, B = H rows (gathered through the scored-row list)
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
  int64_t ldz;
  Softcap sc;
  uint16_t* dz;
};

template <int D, bool CAPPED>
struct DzCore {
  static constexpr int KS = D / 16;
  const lds_char* lds;
  int h, col, V;
  Softcap sc;
  bf16x8 hf[KS];
  float bias;      // -lse * log2 e of this lane's row (-inf for padding rows)
  int ytok;        // target of this lane's row (never matches for padding rows)
  uint16_t* dzrow;

  __device__ __forceinline__ f32x16 chain(int buf, int vb) const { return logit_block<D>(lds, buf, vb, h, col, hf); }

  // mode 0: series softcap (|z| <= c/8), 1: exact softcap, 2: no cap
  template <int MODE, bool MASKED>
  __device__ __forceinline__ void store_block(const f32x16& acc, int vbase) const {
    const int dy = ytok - vbase;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float vals[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * q + e;
        const int off = 8 * q + 4 * h + e;
        const float z = acc[r];
        float p, slope;
        if (MODE == 0) {
          const float u = z * z;
          const float s2 = z * __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(sc.q3, u, sc.q2), u, sc.q1), u, sc.q0);
          p = fexp2(s2 + bias);
          const float t = s2 * sc.invM;              // s / c = tanh(z / c)
          slope = __builtin_fmaf(-t, t, 1.0f);
        } else if (MODE == 1) {
          const float rk = capped_shifted(z, sc.alpha, sc.invK);   // K r, r = 1 / (1 + e^(2z/c))
          p = fexp2(rk + (sc.M + bias));
          const float rr = rk * sc.invK;
          slope = rr * __builtin_fmaf(-4.0f, rr, 4.0f);             // 4 r (1 - r) = 1 - tanh^2
        } else {
          p = fexp2(__builtin_fmaf(z, kLog2e, bias));
          slope = 1.0f;
        }
        float g = (off == dy) ? p - 1.0f : p;
        float val = g * slope;
        if (MASKED) val = (vbase + off < V) ? val : 0.0f;
        vals[e] = val;
      }
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (__bf16)vals[e];
      *reinterpret_cast<bf16x4*>(dzrow + vbase + 8 * q + 4 * h) = o;
    }
  }

  template <bool MASKED>
  __device__ __forceinline__ void store_exact(const f32x16& acc, int vbase) const {
    if (CAPPED) store_block<1, MASKED>(acc, vbase);
    else store_block<2, MASKED>(acc, vbase);
  }

  __device__ __forceinline__ f32x16 chain_with_store(int buf, int vb, const f32x16& prev, int vprev) const {
    f32x16 a;
    if (CAPPED) {
      a = chain(buf, vb);
      store_block<0, false>(prev, vprev);
      const float amax = wave_absmax16(prev);
      interleave_hint<KS, (16 * 13 + KS - 1) / KS>();
      if (!__all(amax <= sc.thr)) store_block<1, false>(prev, vprev);
    } else {
      a = chain(buf, vb);
      store_block<2, false>(prev, vprev);
    }
    return a;
  }
};

template <int D, bool CAPPED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dz_kernel(DzParams p) {
  using TL = TileLayout<D>;
  constexpr int KS = D / 16;
  __shared__ __attribute__((aligned(1024))) char smem[2 * TL::TILEB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int64_t n = p.n_dev ? (int64_t)(*p.n_dev) : p.n_host;
  const int rt = blockIdx.x;
  if ((int64_t)rt * kRowsPerWG >= n) return;
  const int V = p.V;

  DzCore<D, CAPPED> core;
  core.lds = (const lds_char*)smem;
  core.h = h;
  core.col = col;
  core.V = V;
  core.sc = p.sc;
  const int64_t tok = (int64_t)rt * kRowsPerWG + wave * kTokPerWave + col;
  const bool valid = tok < n;
  const int64_t ic = valid ? tok : n - 1;
  const int64_t grow = p.rows ? (int64_t)p.rows[ic] : ic;
  {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(p.H + grow * D + h * (D / 2));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) core.hf[ks] = src[ks];
  }
  core.bias = valid ? -p.lse[grow] * kLog2e : -INFINITY;
  core.ytok = valid ? p.target[grow] : -(1 << 30);
  core.dzrow = p.dz + tok * p.ldz;

  const int ntiles = p.n_vtiles;
  const bool last_partial = (V % kVocabTile) != 0;
  f32x16 accp;
  int vprev = -1;
  load_embed_tile<D, kFwdWaves>(smem, p.E, V, 0, 0, wave, lane);
  for (int i = 0; i < ntiles; ++i) {
    const int buf = i & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (i + 1 < ntiles) load_embed_tile<D, kFwdWaves>(smem, p.E, V, i + 1, buf ^ 1, wave, lane);
    const int vb0 = i * kVocabTile;
    if (last_partial && i + 1 == ntiles) {
      const f32x16 a0 = core.chain(buf, 0);
      if (vprev >= 0) core.template store_exact<false>(accp, vprev);
      const f32x16 a1 = core.chain(buf, 1);
      core.template store_exact<true>(a0, vb0);
      if (vb0 + 32 < p.ldz) core.template store_exact<true>(a1, vb0 + 32);
      vprev = -1;
    } else if (vprev < 0) {
      const f32x16 a0 = core.chain(buf, 0);
      accp = core.chain_with_store(buf, 1, a0, vb0);
      vprev = vb0 + 32;
    } else {
      const f32x16 a0 = core.chain_with_store(buf, 0, accp, vprev);
      accp = core.chain_with_store(buf, 1, a0, vb0);
      vprev = vb0 + 32;
    }
  }
  if (vprev >= 0) core.template store_exact<false>(accp, vprev);
}

// ------------------------------------------------------------------------------- bf16 GEMM
constexpr int kGemmBM = 256, kGemmBN = 256, kGemmBK = 32, kGemmStages = 3;

struct GemmParams {
  const uint16_t* A;      // element (m, k): A_TRANS ? A[k * lda + m] : A[m * lda + k]
  int64_t lda;
  const uint16_t* B;      // element (k, n): B[krow(k) * ldb + n]
  int64_t ldb;
  const int32_t* brows;   // krow(k) = brows[k] when given, else k
  const int32_t* n_dev;   // device count that replaces M (m_dev) or K (k_dev)
  int m_dev, k_dev;
  int64_t M, N, K;        // sizes (upper bounds when taken from n_dev)
  int64_t kvalid;         // rows of B that exist (host bound; clamped below the device count)
  float alpha;
  float* C;
  int64_t ldc;
  const int32_t* crows;   // output row of m when given
  int64_t split_stride;   // elements between the partial outputs of k splits
};

// LDS tile layouts (bytes):
//   k-contiguous A: [256 m][32 k], 64 B rows; 16-byte chunk c of row m stored at c ^ ((m >> 2) & 3)
//   k-slow A or B: [32 k][256 m|n], 512 B rows; chunk c of row k stored at c ^ (4 (k & 3))
// Both keep the 16 lanes of an LDS read phase on 16 different 16-byte bank groups.
template <bool A_TRANS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(GemmParams g) {
  constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
  constexpr int ABYTES = BM * BK * 2, BBYTES = BN * BK * 2, SBYTES = ABYTES + BBYTES;
  __shared__ __attribute__((aligned(1024))) char smem[kGemmStages * SBYTES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;

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

  // ---- stage loader: 32 global_load_lds_dwordx4 per stage, 8 per wave
  auto load_stage = [&](int64_t kc, int st) {
    char* sA = smem + st * SBYTES;
    char* sB = sA + ABYTES;
    const int64_t k0 = kc * BK;
#pragma unroll
    for (int j = wave; j < 16; j += 4) {
      const uint16_t* src;
      if (!A_TRANS) {
        const int row = 16 * j + (lane >> 2);
        const int lc = (lane & 3) ^ ((row >> 2) & 3);
        int64_t m = m0 + row;
        m = m < M ? m : M - 1;
        src = g.A + m * g.lda + k0 + 8 * lc;
      } else {
        const int row = 2 * j + (lane >> 5);
        const int lc = (lane & 31) ^ (4 * (row & 3));
        int64_t col = m0 + 8 * lc;
        col = col <= g.lda - 8 ? col : g.lda - 8;
        src = g.A + (k0 + row) * g.lda + col;
      }
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(sA + j * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int j = wave; j < 16; j += 4) {
      const int row = 2 * j + (lane >> 5);
      const int lc = (lane & 31) ^ (4 * (row & 3));
      int64_t k = k0 + row;
      k = k < kvalid ? k : kvalid - 1;
      const int64_t krow = g.brows ? (int64_t)g.brows[k] : k;
      int64_t col = n0 + 8 * lc;
      col = col <= g.ldb - 8 ? col : g.ldb - 8;
      __builtin_amdgcn_global_load_lds(g.B + krow * g.ldb + col, (lds_void*)(sB + j * 1024), 16, 0, 0);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int grp = lane >> 4, li = lane & 15;
  // transposed-read lane address inside a [32 k][256] tile: row k0 + li / 4, columns
  // cbase + 16 (grp & 1) + 4 (li & 3) .. + 3, for k0 = 16 ks + 8 (grp >> 1) + 4 half
  auto tr_addr = [&](int ks, int half, int cbase) -> int {
    const int k = 16 * ks + 8 * (grp >> 1) + 4 * half + (li >> 2);
    const int c = cbase + 16 * (grp & 1) + 4 * (li & 3);
    return k * 512 + 16 * ((c >> 3) ^ (4 * (k & 3))) + 2 * (c & 7);
  };
  auto read_tr = [&](const char* tile, int ks, int cbase) -> bf16x8 {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + tr_addr(ks, 0, cbase)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + tr_addr(ks, 1, cbase)));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  if (nk > 0) load_stage(kc_begin, 0);
  if (nk > 1) load_stage(kc_begin + 1, 1);
  for (int64_t it = 0; it < nk; ++it) {
    if (it + 1 < nk) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 2 < nk) load_stage(kc_begin + it + 2, (int)((it + 2) % kGemmStages));
    const int st = (int)(it % kGemmStages);
    const char* sA = smem + st * SBYTES;
    const char* sB = sA + ABYTES;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int bm = 0; bm < 4; ++bm) {
        const int mb = wm * 128 + bm * 32;
        if (!A_TRANS) {
          const int row = mb + (lane & 31);
          const int chunk = (2 * ks + h) ^ ((row >> 2) & 3);
          af[bm] = *(const __attribute__((address_space(3))) bf16x8*)((const lds_char*)sA + row * 64 + chunk * 16);
        } else {
          af[bm] = read_tr(sA, ks, mb);
        }
      }
#pragma unroll
      for (int bn = 0; bn < 4; ++bn) bfr[bn] = read_tr(sB, ks, wn * 128 + bn * 32);
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
#pragma unroll
        for (int bn = 0; bn < 4; ++bn) acc[bm][bn] = mfma32x32x16(af[bm], bfr[bn], acc[bm][bn]);
    }
  }

  // ---- epilogue: alpha * acc to C (row-scattered) or to this split's partial tile
  float* C = g.C + (int64_t)blockIdx.z * g.split_stride;
#pragma unroll
  for (int bm = 0; bm < 4; ++bm)
#pragma unroll
    for (int bn = 0; bn < 4; ++bn) {
      const int64_t n = n0 + wn * 128 + bn * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 128 + bm * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
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

// ------------------------------------------------------------------------------------ host side

constexpr int kDeSplit = 4;

template <int D>
static void launch_dz(const DzParams& q, unsigned blocks, hipStream_t st) {
  if (q.sc.c > 0.f)
    hipLaunchKernelGGL((bwd_dz_kernel<D, true>), dim3(blocks), dim3(kFwdWaves * 64), 0, st, q);
  else
    hipLaunchKernelGGL((bwd_dz_kernel<D, false>), dim3(blocks), dim3(kFwdWaves * 64), 0, st, q);
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
  L.total = o;
  return L;
}

hipError_t launch_bwd(const void* H, const void* E, int32_t dtype, const int32_t* target,
                      const uint8_t* mask, const float* lse, int64_t T, int32_t D, int32_t V,
                      float softcap, float grad_scale, float* dH, float* dE, char* ws,
                      const DeviceInfo& dev, hipStream_t st) {
  const BwdWorkspace L = bwd_workspace(T, D, V);
  const Softcap sc = Softcap::make(softcap);
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
    const int64_t tot = T * D;
    hipLaunchKernelGGL(zero_unscored_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, mask, T, D, dH);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  uint16_t* dz = reinterpret_cast<uint16_t*>(ws + L.dz);
  if (dtype == 0 && mfma_width(D)) {
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

      // dH = g dZ E
      GemmParams a{};
      a.A = dz; a.lda = q.ldz;
      a.B = (const uint16_t*)E; a.ldb = D;
      a.brows = nullptr;
      a.n_dev = n_dev; a.m_dev = n_dev != nullptr; a.k_dev = 0;
      a.M = T; a.N = D; a.K = V; a.kvalid = V;
      a.alpha = grad_scale;
      a.C = dH; a.ldc = D; a.crows = rows; a.split_stride = 0;
      hipLaunchKernelGGL(gemm_bf16_kernel<false>, dim3(rblk, (unsigned)((D + kGemmBN - 1) / kGemmBN), 1), dim3(256),
                         0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // dE = g dZ^T H, k split over workgroups when the output has few tiles
    const int64_t tiles = ((int64_t)(V + kGemmBM - 1) / kGemmBM) * ((D + kGemmBN - 1) / kGemmBN);
    const int ncu = dev.cu_count > 0 ? dev.cu_count : 256;
    int64_t ks = ncu / (tiles > 0 ? tiles : 1);
    ks = ks < 1 ? 1 : (ks > kDeSplit ? kDeSplit : ks);
    if (T == 0) {
      const int64_t cnt = (int64_t)V * D;
      hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st,
                         (const float*)nullptr, 0, cnt, cnt, dE);
      return hipGetLastError();
    }
    float* part = reinterpret_cast<float*>(ws + L.de_part);
    GemmParams b{};
    b.A = dz; b.lda = ((V + kVocabTile - 1) / kVocabTile) * (int64_t)kVocabTile;
    b.B = (const uint16_t*)H; b.ldb = D;
    b.brows = rows;
    b.n_dev = n_dev; b.m_dev = 0; b.k_dev = n_dev != nullptr;
    b.M = V; b.N = D; b.K = T; b.kvalid = T;
    b.alpha = grad_scale;
    b.C = ks > 1 ? part : dE; b.ldc = D; b.crows = nullptr; b.split_stride = (int64_t)V * D;
    hipLaunchKernelGGL(gemm_bf16_kernel<true>, dim3((unsigned)((V + kGemmBM - 1) / kGemmBM),
                       (unsigned)((D + kGemmBN - 1) / kGemmBN), (unsigned)ks), dim3(256), 0, st, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ks == 1) return e;
    const int64_t cnt = (int64_t)V * D;
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, st, part, (int)ks,
                       cnt, cnt, dE);
    return hipGetLastError();
  }
  const unsigned rblocks = (unsigned)((T + 3) / 4);
  const unsigned hblocks = (unsigned)((T * D + 255) / 256);
  const unsigned eblocks = (unsigned)(((int64_t)V * D + 255) / 256);
  if (T > 0) {
    if (dtype == 0) {
      hipLaunchKernelGGL(dz_generic_kernel<uint16_t>, dim3(rblocks), dim3(256), 0, st, (const uint16_t*)H,
                         (const uint16_t*)E, target, lse, rows, n_dev, T, D, V, sc, dz);
      hipLaunchKernelGGL(dh_generic_kernel<uint16_t>, dim3(hblocks), dim3(256), 0, st, dz, (const uint16_t*)E,
                         rows, n_dev, T, D, V, grad_scale, dH);
    } else {
      hipLaunchKernelGGL(dz_generic_kernel<float>, dim3(rblocks), dim3(256), 0, st, (const float*)H,
                         (const float*)E, target, lse, rows, n_dev, T, D, V, sc, dz);
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

}  // namespace pg
