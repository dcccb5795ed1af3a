// Tiled MFMA GEMM core for gfx950: C[M x N] = X[M x K] * Y[N x K]^T, fp32 accumulation.
//
// Both operands are K-contiguous ("row-major X, row-major Y"). Every contraction of the
// inner loop is arranged into this one form by keeping the operands it needs in the
// matching layout (weights in both orientations, transposed activations written by the
// producing kernels), so a single tile engine serves the whole path.
//
// Tile engine:
//   * 256 threads = 4 waves in a 2 x 2 grid; a wave owns a (BM/2) x (BN/2) sub-tile made of
//     16 x 16 MFMA blocks (v_mfma_f32_16x16x32_bf16 for bf16, 4 x v_mfma_f32_16x16x4_f32
//     for fp32);
//   * one K-iteration moves a 128-byte slice of every tile row (64 bf16 / 32 fp32) through
//     LDS; two stages, the next slice's global loads are in flight during the MFMAs;
//   * LDS rows are 128 B with the 16-B chunk index XOR-swizzled by (row & 7), so both the
//     row-wise stores and the column-of-rows MFMA operand reads are bank-conflict free;
//   * workgroups are renumbered so that each XCD (dispatch is round-robin over the 8 XCDs)
//     receives a contiguous run of tiles: neighbouring tiles share operand slabs in the
//     same L2;
//   * optional split-K over gridDim.y; each split hands its partial tile to the epilogue.
// The epilogue receives the wave's accumulators and their coordinates:
//   acc[i][j][e] holds C[row0 + 16 i + 4 (lane / 16) + e][col0 + 16 j + lane % 16].
#pragma once

#include "common.h"

// A GEMM may carry a second K-segment: C = X Y^T + X2 Y2^T (same M, N). The kernel walks
// the concatenated K range, so the two products share accumulators, tiles and splits.
struct GemmArgs {
  const void* X;
  const void* Y;
  const void* X2;
  const void* Y2;
  int64_t ldx, ldy, ldx2, ldy2;  // row strides in elements
  int M, N, K, K2;
  int tiles_m, tiles_n;
  int kit_a;   // K-iterations (of 128 bytes) of the first segment
  int kiters;  // K-iterations of both segments
  int kps;     // K-iterations per split
};

struct EpiPos {
  int row0, col0;  // global coordinates of this wave's sub-tile
  int lane, wave, wm, wn;
  int tm, tn, tile;  // tile coordinates; tile = tn * tiles_m + tm (a stable slot id)
  int split;
  int M, N;
  char* smem;  // the kernel's LDS, free for the epilogue
};

__device__ __forceinline__ int epi_row(const EpiPos& p, int i, int e) { return p.row0 + 16 * i + 4 * (p.lane >> 4) + e; }
__device__ __forceinline__ int epi_col(const EpiPos& p, int j) { return p.col0 + 16 * j + (p.lane & 15); }

template <class T, int BM, int BN, class Epi>
__global__ void __launch_bounds__(256) gemm_nt_kernel(GemmArgs g, Epi epi) {
  constexpr int ROWB = 128;
  constexpr int KE = ROWB / (int)sizeof(T);
  constexpr int KC = 16 / (int)sizeof(T);
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int STAGE = (BM + BN) * ROWB;
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile sizes must be multiples of 32");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware renumbering (a bijection of [0, nblk); correctness never depends on it).
  const int nblk = gridDim.x * gridDim.y;
  const int lin = blockIdx.y * gridDim.x + blockIdx.x;
  const int per = nblk >> 3, rem = nblk & 7;
  const int xcd = lin & 7;
  const int id = xcd * per + min(xcd, rem) + (lin >> 3);
  const int ntiles = g.tiles_m * g.tiles_n;
  const int split = id / ntiles;
  const int tile = id - split * ntiles;
  const int tm = tile % g.tiles_m, tn = tile / g.tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kit0 = split * g.kps;
  const int kit1 = min(g.kiters, kit0 + g.kps);

  const int lrow = tid >> 3, lch = tid & 7;
  const char* __restrict__ Xp = (const char*)g.X;
  const char* __restrict__ Yp = (const char*)g.Y;
  const char* __restrict__ X2p = (const char*)g.X2;
  const char* __restrict__ Y2p = (const char*)g.Y2;
  uint4 ra[BM / 32], rb[BN / 32];

  auto gload = [&](int kit) {
    const bool seg2 = kit >= g.kit_a;
    const int kk = (seg2 ? kit - g.kit_a : kit) * KE + lch * KC;
    const bool kok = kk < (seg2 ? g.K2 : g.K);
    const char* xb = seg2 ? X2p : Xp;
    const char* yb = seg2 ? Y2p : Yp;
    const int64_t lx = seg2 ? g.ldx2 : g.ldx, ly = seg2 ? g.ldy2 : g.ldy;
#pragma unroll
    for (int p = 0; p < BM / 32; ++p) {
      const int r = m0 + p * 32 + lrow;
      ra[p] = (kok && r < g.M) ? *(const uint4*)(xb + ((int64_t)r * lx + kk) * (int64_t)sizeof(T))
                               : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < BN / 32; ++p) {
      const int r = n0 + p * 32 + lrow;
      rb[p] = (kok && r < g.N) ? *(const uint4*)(yb + ((int64_t)r * ly + kk) * (int64_t)sizeof(T))
                               : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int stage) {
    char* sa = smem + stage * STAGE;
    char* sb = sa + BM * ROWB;
    const int sw = (lch ^ (lrow & 7)) << 4;
#pragma unroll
    for (int p = 0; p < BM / 32; ++p) *(uint4*)(sa + (p * 32 + lrow) * ROWB + sw) = ra[p];
#pragma unroll
    for (int p = 0; p < BN / 32; ++p) *(uint4*)(sb + (p * 32 + lrow) * ROWB + sw) = rb[p];
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (kit0 < kit1) {
    gload(kit0);
    sstore(0);
    __syncthreads();
    for (int it = kit0; it < kit1; ++it) {
      const int cur = (it - kit0) & 1;
      const bool more = it + 1 < kit1;
      if (more) gload(it + 1);
      const char* sa = smem + cur * STAGE;
      const char* sb = sa + BM * ROWB;
#pragma unroll
      for (int kg = 0; kg < 2; ++kg) {
        const int ch = kg * 4 + (lane >> 4);
        uint4 af[FM], bfr[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm * WTM + i * 16 + (lane & 15);
          af[i] = *(const uint4*)(sa + r * ROWB + ((ch ^ (r & 7)) << 4));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = wn * WTN + j * 16 + (lane & 15);
          bfr[j] = *(const uint4*)(sb + r * ROWB + ((ch ^ (r & 7)) << 4));
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) mfma_chunk(acc[i][j], af[i], bfr[j], T());
      }
      if (more) sstore(cur ^ 1);
      __syncthreads();
    }
  }

  EpiPos pos;
  pos.row0 = m0 + wm * WTM;
  pos.col0 = n0 + wn * WTN;
  pos.lane = lane;
  pos.wave = wave;
  pos.wm = wm;
  pos.wn = wn;
  pos.tm = tm;
  pos.tn = tn;
  pos.tile = tile;
  pos.split = split;
  pos.M = g.M;
  pos.N = g.N;
  pos.smem = smem;
  epi.template apply<FM, FN>(pos, acc);
}

// ------------------------------------------------------------------------- epilogues
// Store 4 vertically adjacent outputs (rows r..r+3 of one column) into a transposed
// matrix, i.e. 4 consecutive elements of one row of C^T. Packs the store when possible.
template <class T>
__device__ __forceinline__ void store4_t(T* dst, float v0, float v1, float v2, float v3, int nvalid);
template <>
__device__ __forceinline__ void store4_t<bf16_t>(bf16_t* dst, float v0, float v1, float v2, float v3, int nvalid) {
  if (nvalid >= 4) {
    uint2 u;
    u.x = (uint32_t)f2bf(v0) | ((uint32_t)f2bf(v1) << 16);
    u.y = (uint32_t)f2bf(v2) | ((uint32_t)f2bf(v3) << 16);
    *(uint2*)dst = u;
  } else {
    if (nvalid > 0) dst[0] = f2bf(v0);
    if (nvalid > 1) dst[1] = f2bf(v1);
    if (nvalid > 2) dst[2] = f2bf(v2);
  }
}
template <>
__device__ __forceinline__ void store4_t<float>(float* dst, float v0, float v1, float v2, float v3, int nvalid) {
  if (nvalid >= 4) {
    *(float4*)dst = make_float4(v0, v1, v2, v3);
  } else {
    if (nvalid > 0) dst[0] = v0;
    if (nvalid > 1) dst[1] = v1;
    if (nvalid > 2) dst[2] = v2;
  }
}

// Plain fp32 store, optionally accumulating, with one output slab per split.
struct EpiStoreF32 {
  float* C;
  int64_t ldc;
  int64_t split_stride;
  int accumulate;
  template <int FM, int FN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
    float* Cs = C + (int64_t)p.split * split_stride;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = epi_row(p, i, e);
        if (row >= p.M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = epi_col(p, j);
          if (col >= p.N) continue;
          float* d = Cs + (int64_t)row * ldc + col;
          *d = accumulate ? *d + acc[i][j][e] : acc[i][j][e];
        }
      }
  }
};

// Per-row sum over the tile's columns of a per-element value v[i][e] (already summed over
// the wave's j blocks by the caller): 16-lane butterfly, then the two column-half waves are
// combined through LDS and written to out[tn * ldo + row]. Fixed order, so deterministic.
// Uses 2 * BM floats of LDS; all threads of the block must call it.
template <int FM>
__device__ __forceinline__ void row_partial_store(const EpiPos& p, float (&v)[FM][4], float* out, int64_t ldo) {
  constexpr int WTM = 16 * FM;
  float* l1 = (float*)p.smem;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[i][e] = xor16_sum(v[i][e]);
      if (p.wn == 1 && (p.lane & 15) == 0) l1[p.wm * WTM + 16 * i + 4 * (p.lane >> 4) + e] = v[i][e];
    }
  __syncthreads();
  if (p.wn == 0 && (p.lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = epi_row(p, i, e);
        if (row < p.M) out[(int64_t)p.tn * ldo + row] = v[i][e] + l1[p.wm * WTM + 16 * i + 4 * (p.lane >> 4) + e];
      }
  }
}

// Up-projection of a GELU block: U = Hn W1 -> A = GELU(U) (row-major and transposed) and
// GELU'(U) for the backward pass. RES (optional) keeps A - rn(A), the rounding residual of
// the stored operand, for the first-order loss compensation.
template <class T>
struct EpiGelu {
  T* A;     // [M x lda]
  T* AT;    // [N x ldat]
  T* GP;    // [M x lda]
  T* RES;   // [M x lda] or null
  int64_t lda, ldat;
  template <int FM, int FN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r0 = epi_row(p, i, 0);
      const int nv = min(4, p.M - r0);
      if (nv <= 0) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = epi_col(p, j);
        if (col >= p.N) continue;
        float a[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float u = acc[i][j][e];
          a[e] = gelu_f(u);
          if (e < nv) {
            const int64_t o = (int64_t)(r0 + e) * lda + col;
            const T q = from_f<T>(a[e]);
            A[o] = q;
            GP[o] = from_f<T>(gelu_prime_f(u));
            if (RES) RES[o] = from_f<T>(a[e] - to_f<T>(q));
          }
        }
        store4_t<T>(AT + (int64_t)col * ldat + r0, a[0], a[1], a[2], a[3], nv);
      }
    }
  }
};

// Up-projection of a SwiGLU block (gate result already in UG): V = Hn Wu is kept (fp32) for
// the backward pass, A = SiLU(UG) * V is stored row-major and transposed, RES as above.
template <class T>
struct EpiSwiglu {
  const float* UG;  // [M x lda] fp32 gate pre-activation
  float* VU;        // [M x lda] fp32 up-projection (may be null)
  T* A;
  T* AT;
  T* RES;           // may be null
  int64_t lda, ldat;
  template <int FM, int FN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r0 = epi_row(p, i, 0);
      const int nv = min(4, p.M - r0);
      if (nv <= 0) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = epi_col(p, j);
        if (col >= p.N) continue;
        float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (e < nv) {
            const int64_t o = (int64_t)(r0 + e) * lda + col;
            a[e] = silu_f(UG[o]) * acc[i][j][e];
            const T q = from_f<T>(a[e]);
            A[o] = q;
            if (VU) VU[o] = acc[i][j][e];
            if (RES) RES[o] = from_f<T>(a[e] - to_f<T>(q));
          }
        }
        store4_t<T>(AT + (int64_t)col * ldat + r0, a[0], a[1], a[2], a[3], nv);
      }
    }
  }
};

// Backward through GELU: dA = dY W2^T (the accumulator); dU = dA * GELU'(U), row-major and
// transposed. With RES, also the per-token partial dot <dA_t, A_t - rn(A_t)> of this tile's
// columns into cdot[tn * M + row].
template <class T>
struct EpiDU {
  const T* GP;   // [M x ld]
  T* DU;         // [M x ld]
  T* DUT;        // [N x ldt]
  const T* RES;  // [M x ld] or null
  float* cdot;   // [tiles_n x M] or null
  int64_t ld, ldt;
  template <int FM, int FN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
    float dots[FM][4];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) dots[i][e] = 0.f;
      const int r0 = epi_row(p, i, 0);
      const int nv = min(4, p.M - r0);
      if (nv <= 0) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = epi_col(p, j);
        if (col >= p.N) continue;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (e < nv) {
            const int64_t o = (int64_t)(r0 + e) * ld + col;
            v[e] = acc[i][j][e] * to_f<T>(GP[o]);
            DU[o] = from_f<T>(v[e]);
            if (RES) dots[i][e] += acc[i][j][e] * to_f<T>(RES[o]);
          }
        }
        store4_t<T>(DUT + (int64_t)col * ldt + r0, v[0], v[1], v[2], v[3], nv);
      }
    }
    if (cdot) row_partial_store<FM>(p, dots, cdot, p.M);
  }
};

// Backward into a SwiGLU block whose gate/up are frozen (only needed to carry the loss
// compensation below the block): dA = dY W2^T (accumulator); dG = dA * V * SiLU'(UG),
// dV = dA * SiLU(UG); plus the per-token partial dot <dA_t, RES_t> as in EpiDU.
template <class T>
struct EpiSwigluBwd {
  const float* UG;
  const float* VU;
  T* DG;
  T* DV;
  const T* RES;
  float* cdot;
  int64_t ld;
  template <int FM, int FN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
    float dots[FM][4];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dots[i][e] = 0.f;
        const int row = epi_row(p, i, e);
        if (row >= p.M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = epi_col(p, j);
          if (col >= p.N) continue;
          const int64_t o = (int64_t)row * ld + col;
          const float da = acc[i][j][e];
          const float g = UG[o];
          const float sg = 1.0f / (1.0f + expf(-g));
          DG[o] = from_f<T>(da * VU[o] * sg * (1.0f + g * (1.0f - sg)));
          DV[o] = from_f<T>(da * g * sg);
          dots[i][e] += da * to_f<T>(RES[o]);
        }
      }
    row_partial_store<FM>(p, dots, cdot, p.M);
  }
};

// Weight gradient: store G (fp32) and this tile's sum of squares into slot[tile].
struct EpiGrad {
  float* G;
  int64_t ldg;
  float* slot;
  template <int FM, int FN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = epi_row(p, i, e);
        if (row >= p.M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = epi_col(p, j);
          if (col >= p.N) continue;
          const float v = acc[i][j][e];
          G[(int64_t)row * ldg + col] = v;
          ss += v * v;
        }
      }
    ss = wave_sum(ss);
    float* red = (float*)p.smem;
    if (p.lane == 0) red[p.wave] = ss;
    __syncthreads();
    if (p.wave == 0 && p.lane == 0) slot[p.tile] = (red[0] + red[1]) + (red[2] + red[3]);
  }
};

// Online-softmax partials of one vocab tile of the LM head: per row, the tile's max
// logit, sum of exp(z - max) and first argmax; the target logit is stored by the one
// lane whose column is the row's target.
__device__ __forceinline__ void ce_combine(float& mx, float& sm, int& ix, float omx, float osm, int oix) {
  const float nm = fmaxf(mx, omx);
  const float a = (mx == -INFINITY) ? 0.f : sm * expf(mx - nm);
  const float b = (omx == -INFINITY) ? 0.f : osm * expf(omx - nm);
  if (omx > mx || (omx == mx && oix < ix)) ix = oix;
  mx = nm;
  sm = a + b;
}

struct EpiCEPartial {
  const int* tgt;    // [M] target ids
  float* pmax;       // [tiles_n x ldp]
  float* psum;
  int* pidx;
  float* tgt_logit;  // [M]
  int ldp;
  template <int FM, int FN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
    constexpr int WTM = 16 * FM, BM = 2 * WTM;
    float* lmax = (float*)p.smem;
    float* lsum = lmax + BM;
    int* lidx = (int*)(lsum + BM);
    float rm[FM][4], rs[FM][4];
    int ri[FM][4];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = epi_row(p, i, e);
        const int tg = row < p.M ? tgt[row] : -1;
        float mx = -INFINITY;
        int ix = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = epi_col(p, j);
          if (col < p.N) {
            const float v = acc[i][j][e];
            if (v > mx) { mx = v; ix = col; }
            if (col == tg) tgt_logit[row] = v;
          }
        }
        float sm = 0.f;
        if (mx != -INFINITY) {
#pragma unroll
          for (int j = 0; j < FN; ++j)
            if (epi_col(p, j) < p.N) sm += expf(acc[i][j][e] - mx);
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          const float omx = __shfl_xor(mx, off, TTT_WAVE);
          const float osm = __shfl_xor(sm, off, TTT_WAVE);
          const int oix = __shfl_xor(ix, off, TTT_WAVE);
          ce_combine(mx, sm, ix, omx, osm, oix);
        }
        rm[i][e] = mx;
        rs[i][e] = sm;
        ri[i][e] = ix;
        const int lr = p.wm * WTM + 16 * i + 4 * (p.lane >> 4) + e;
        if (p.wn == 1 && (p.lane & 15) == 0) {
          lmax[lr] = mx;
          lsum[lr] = sm;
          lidx[lr] = ix;
        }
      }
    __syncthreads();
    if (p.wn == 0 && (p.lane & 15) == 0) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = epi_row(p, i, e);
          if (row >= p.M) continue;
          const int lr = p.wm * WTM + 16 * i + 4 * (p.lane >> 4) + e;
          float mx = rm[i][e], sm = rs[i][e];
          int ix = ri[i][e];
          ce_combine(mx, sm, ix, lmax[lr], lsum[lr], lidx[lr]);
          const int64_t o = (int64_t)p.tn * ldp + row;
          pmax[o] = mx;
          psum[o] = sm;
          pidx[o] = ix;
        }
    }
  }
};

// dlogits of one vocab super-tile, recomputed from the logits tile in registers:
// P[t, v] = (exp(z - lse_t) - [v == x_t]) / b, stored in the GEMM operand precision.
template <class T>
struct EpiCEProb {
  const int* tgt;
  const float* lse;
  T* P;
  int64_t ldp;
  int col_base;  // vocab id of column 0
  float inv_b;
  template <int FM, int FN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = epi_row(p, i, e);
        if (row >= p.M) continue;
        const int tg = tgt[row] - col_base;
        const float ls = lse[row];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = epi_col(p, j);
          if (col >= p.N) continue;
          const float v = (expf(acc[i][j][e] - ls) - (col == tg ? 1.f : 0.f)) * inv_b;
          P[(int64_t)row * ldp + col] = from_f<T>(v);
        }
      }
  }
};

// ------------------------------------------------------------------------- launcher
// Second K-segment of a GEMM (absent when K2 == 0).
struct Seg2 {
  const void* X = nullptr;
  int64_t ldx = 0;
  const void* Y = nullptr;
  int64_t ldy = 0;
  int K = 0;
};

template <class T, int BM, int BN, class Epi>
inline hipError_t launch_gemm(hipStream_t st, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M,
                              int N, int K, int splits, const Epi& epi, const Seg2& s2 = Seg2()) {
  if (M <= 0 || N <= 0) return hipSuccess;
  constexpr int KE = 128 / (int)sizeof(T);
  GemmArgs g;
  g.X = X;
  g.Y = Y;
  g.ldx = ldx;
  g.ldy = ldy;
  g.X2 = s2.X;
  g.Y2 = s2.Y;
  g.ldx2 = s2.ldx;
  g.ldy2 = s2.ldy;
  g.M = M;
  g.N = N;
  g.K = K;
  g.K2 = s2.K;
  g.tiles_m = (M + BM - 1) / BM;
  g.tiles_n = (N + BN - 1) / BN;
  g.kit_a = (K + KE - 1) / KE;
  g.kiters = g.kit_a + (s2.K + KE - 1) / KE;
  if (splits < 1) splits = 1;
  g.kps = (g.kiters + splits - 1) / splits;
  dim3 grid(g.tiles_m * g.tiles_n, splits);
  hipLaunchKernelGGL((gemm_nt_kernel<T, BM, BN, Epi>), grid, dim3(256), 0, st, g, epi);
  return hipGetLastError();
}
