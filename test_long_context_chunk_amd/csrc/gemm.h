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
//   * optional split-K over gridDim.y; each split hands its partial tile to the epilogue;
//   * optional grouping over gridDim.z: independent products of one shape whose operands
//     sit at fixed strides, with their outputs stacked row-wise (see GemmArgs).
// The epilogue receives the wave's accumulators and their coordinates:
//   acc[i][j][e] holds C[row0 + 16 i + 4 (lane / 16) + e][col0 + 16 j + lane % 16].
#pragma once

#include "common.h"

#include <type_traits>

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
  // Grouped launch: gridDim.z independent products of this shape. Product z reads its
  // operands at z * (gx, gy, gx2, gy2) elements past X, Y, X2, Y2 (0: shared by every
  // product), and its epilogue sees stacked coordinates: rows z * M + i (bound (z + 1) * M)
  // and tile ids z * gtile + t.
  int64_t gx, gy, gx2, gy2;
  int gtile;
};

// Which product, split and output tile a workgroup computes. The linear workgroup index is
// renumbered so that consecutive ids share an XCD (a bijection of [0, nblk); correctness
// never depends on it); products vary slowest, then splits, then tiles.
struct GemmWork {
  int z, split, tile;
};
__device__ __forceinline__ GemmWork gemm_work(const GemmArgs& g) {
  const int nblk = gridDim.x * gridDim.y * gridDim.z;
  const int lin = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
  const int per = nblk >> 3, rem = nblk & 7;
  const int xcd = lin & 7;
  int id = xcd * per + min(xcd, rem) + (lin >> 3);
  const int ntiles = g.tiles_m * g.tiles_n;
  const int pz = ntiles * gridDim.y;
  GemmWork w;
  w.z = id / pz;
  id -= w.z * pz;
  w.split = id / ntiles;
  w.tile = id - w.split * ntiles;
  return w;
}

// Operand bases of product z.
template <class T>
__device__ __forceinline__ void gemm_group_bases(const GemmArgs& g, int z, const char*& X, const char*& Y,
                                                 const char*& X2, const char*& Y2) {
  X = (const char*)g.X + (int64_t)z * g.gx * (int64_t)sizeof(T);
  Y = (const char*)g.Y + (int64_t)z * g.gy * (int64_t)sizeof(T);
  X2 = (const char*)g.X2 + (int64_t)z * g.gx2 * (int64_t)sizeof(T);
  Y2 = (const char*)g.Y2 + (int64_t)z * g.gy2 * (int64_t)sizeof(T);
}

struct EpiPos {
  int row0, col0;  // global coordinates of this wave's sub-tile
  int lane, wave, wm, wn;
  int wgm, wgn;      // wave grid of the workgroup (rows x columns of waves)
  int bm, bn;        // tile rows and columns
  int tid, nthr;     // thread index and count of the workgroup
  int smem_bytes;    // LDS the epilogue may use
  int tm, tn, tile;  // tile coordinates; tile = tn * tiles_m + tm (a stable slot id)
  int split;
  int M, N;
  char* smem;  // the kernel's LDS, free for the epilogue (at least 16 KB)
};

__device__ __forceinline__ int epi_row(const EpiPos& p, int i, int e) { return p.row0 + 16 * i + 4 * (p.lane >> 4) + e; }
__device__ __forceinline__ int epi_col(const EpiPos& p, int j) { return p.col0 + 16 * j + (p.lane & 15); }

// Register-staged variant (any K that is a multiple of the 16-byte chunk): global loads go
// through VGPRs into two LDS stages, with zero fill outside the operands.
template <class T, int BM, int BN, class Epi>
__global__ void __launch_bounds__(256) gemm_reg_kernel(GemmArgs g, Epi epi) {
  constexpr int WGM_ = 2, WGN_ = 2;
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

  const GemmWork w = gemm_work(g);
  const int split = w.split, tile = w.tile;
  const int tm = tile % g.tiles_m, tn = tile / g.tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kit0 = split * g.kps;
  const int kit1 = min(g.kiters, kit0 + g.kps);

  const int lrow = tid >> 3, lch = tid & 7;
  const char *Xb, *Yb, *X2b, *Y2b;
  gemm_group_bases<T>(g, w.z, Xb, Yb, X2b, Y2b);
  const char* __restrict__ Xp = Xb;
  const char* __restrict__ Yp = Yb;
  const char* __restrict__ X2p = X2b;
  const char* __restrict__ Y2p = Y2b;
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
  pos.row0 = w.z * g.M + m0 + wm * WTM;
  pos.col0 = n0 + wn * WTN;
  pos.lane = lane;
  pos.wave = wave;
  pos.wm = wm;
  pos.wn = wn;
  pos.wgm = 2;
  pos.wgn = 2;
  pos.bm = BM;
  pos.bn = BN;
  pos.tid = tid;
  pos.nthr = 256;
  pos.smem_bytes = 2 * STAGE;
  pos.tm = tm;
  pos.tn = tn;
  pos.tile = w.z * g.gtile + tile;
  pos.split = split;
  pos.M = (w.z + 1) * g.M;
  pos.N = g.N;
  pos.smem = smem;
  epi.template apply<FM, FN, WGM_, WGN_>(pos, acc);
}

// LDS stages of the direct-load pipeline for an output tile shape: three when three fit the
// 160 KB of a CU (one workgroup per CU), else two; the 128 x 128 tile keeps two so that two
// workgroups share a CU.
constexpr int gemm_stages(int BM, int BN) {
  return ((BM + BN) * 128 * 3 <= 160 * 1024 && !(BM == 128 && BN == 128)) ? 3 : 2;
}
// Stages of the shared-X form (NB = 2 B regions per stage): two at 256 x 128, three at 256 x 64.
constexpr int gemm_stages_nb(int BM, int BN, int NB) {
  return NB == 1 ? gemm_stages(BM, BN) : (((BM + NB * BN) * 128 * 3 <= 160 * 1024) ? 3 : 2);
}
// LDS of a launch: its stages, and never less than the one-segment form's, whose size the
// epilogues' staging areas are planned for (TileGeo).
constexpr int gemm_lds_bytes(int BM, int BN, int NB) {
  const int a = gemm_stages_nb(BM, BN, NB) * (BM + NB * BN) * 128;
  const int b = gemm_stages(BM, BN) * (BM + BN) * 128;
  return a > b ? a : b;
}

// XOR swizzle of the 16-byte chunks of a 128-byte LDS tile row (tile-local row index t;
// the A rows come first, then the B rows, both regions a multiple of 16 rows). 16 x 16
// fragments: 8 consecutive rows share a chunk, swizzled by t mod 8. 32 x 32 fragments: 16
// consecutive lanes read 16 consecutive rows of one chunk; with t / 2 mod 8 the even rows
// fall in one half of the 256-byte bank window and the odd rows in the other, eight
// distinct chunks each, so no two lanes share a bank.
template <bool M32>
__device__ __forceinline__ int lds_swz(int t) {
  if constexpr (M32) return (t >> 1) & 7;
  else return t & 7;
}
// Tile shapes whose bf16 K loop runs on 32 x 32 MFMA blocks with gemm_stages(BM, BN) stages
// (the wave tiles must be multiples of 32).
constexpr bool tile_m32(int BM, int BN) { return !(BM == 128 && BN == 128) && !(BM == 256 && BN == 256); }
template <class T, int BM, int BN, int WGM, int WGN>
constexpr bool use_mfma32() {
  return sizeof(T) == 2 && tile_m32(BM, BN) && (BM / WGM) % 32 == 0 && (BN / WGN) % 32 == 0;
}

// Direct-to-LDS variant (K of both segments a multiple of the 128-byte slice): every wave
// streams whole 8-row blocks of the tile with global_load_lds_dwordx4 (64 lanes x 16 B =
// one 1 KB block), choosing each lane's source chunk so that the block lands in the same
// XOR-swizzled layout the MFMA operand reads expect. No VGPR staging, no zero fill: rows
// past M or N re-read the last valid row and only feed outputs the epilogue never stores.
// Two LDS stages: the next slice is requested right after the barrier that retires the
// stage it overwrites.
//
// One K-iteration: request the next slice into stage `nxt` and multiply the slice held in
// stage `cur`. The two stage pointers are restrict-qualified: they never overlap, and
// saying so lets the compiler read `cur` while the direct loads into `nxt` are still in
// flight (without it, every LDS read would first wait for those loads to land).
template <class T, int BM, int BN, int WGM, int WGN, int PW>
__device__ __forceinline__ void dma_iteration(const char* __restrict__ cur, char* __restrict__ nxt, bool issue,
                                              const char* const (&src)[PW], int64_t kb, int wm, int wn, int lane,
                                              f32x4_t (&acc)[BM / WGM / 16][BN / WGN / 16]) {
  constexpr int ROWB = 128;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  if (issue) {
#pragma unroll
    for (int q = 0; q < PW; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(src[q] + kb),
                                       (__attribute__((address_space(3))) void*)(nxt + q * 1024), 16, 0, 0);
  }
  const char* sb = cur + BM * ROWB;
#pragma unroll
  for (int kg = 0; kg < 2; ++kg) {
    const int ch = kg * 4 + (lane >> 4);
    uint4 af[FM], bfr[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WTM + i * 16 + (lane & 15);
      af[i] = *(const uint4*)(cur + r * ROWB + ((ch ^ (r & 7)) << 4));
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
}

// bf16 K-iteration on 32 x 32 output blocks (see mfma32): four 16-k steps per 128-byte slice;
// in step ks, lanes 0..31 read 16-byte chunk 2 ks of their row, lanes 32..63 chunk 2 ks + 1.
template <int BM, int BN, int WGM, int WGN, int PW>
__device__ __forceinline__ void dma_iteration32(const char* __restrict__ cur, char* __restrict__ nxt, bool issue,
                                                const char* const (&src)[PW], int64_t kb, int wm, int wn, int lane,
                                                f32x16_t (&acc)[BM / WGM / 32][BN / WGN / 32]) {
  constexpr int ROWB = 128;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  if (issue) {
#pragma unroll
    for (int q = 0; q < PW; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(src[q] + kb),
                                       (__attribute__((address_space(3))) void*)(nxt + q * 1024), 16, 0, 0);
  }
  const char* sb = cur + BM * ROWB;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ch = 2 * ks + (lane >> 5);
    uint4 af[FM], bfr[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WTM + i * 32 + (lane & 31);
      af[i] = *(const uint4*)(cur + r * ROWB + ((ch ^ lds_swz<true>(r)) << 4));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = wn * WTN + j * 32 + (lane & 31);
      bfr[j] = *(const uint4*)(sb + r * ROWB + ((ch ^ lds_swz<true>(r)) << 4));
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) mfma32(acc[i][j], af[i], bfr[j]);
  }
}

// Re-deal a wave's 32 x 32 accumulator blocks into the 16 x 16 register layout the
// epilogues are written for (lane l, value e of sub-tile (i, j): row 16 i + 4 (l / 16) + e,
// column 16 j + l % 16). Each block goes through a wave-private column-major LDS scratch
// (column stride 36 floats: the 16-byte writes and reads of 16 lanes hit distinct banks).
// Only this wave touches its scratch, and its LDS accesses complete in order.
template <int FM32, int FN32>
__device__ __forceinline__ void acc32_to_16(char* smem, int wave, int lane, const f32x16_t (&a32)[FM32][FN32],
                                            f32x4_t (&a16)[2 * FM32][2 * FN32]) {
  constexpr int LD = 36;
  float* buf = (float*)smem + wave * (32 * LD);
#pragma unroll
  for (int i = 0; i < FM32; ++i)
#pragma unroll
    for (int j = 0; j < FN32; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(f32x4_t*)(buf + (lane & 31) * LD + 8 * q + 4 * (lane >> 5)) =
            f32x4_t{a32[i][j][4 * q], a32[i][j][4 * q + 1], a32[i][j][4 * q + 2], a32[i][j][4 * q + 3]};
      __asm__ __volatile__("" ::: "memory");
#pragma unroll
      for (int sr = 0; sr < 2; ++sr)
#pragma unroll
        for (int sc = 0; sc < 2; ++sc)
          a16[2 * i + sr][2 * j + sc] = *(const f32x4_t*)(buf + (16 * sc + (lane & 15)) * LD + 16 * sr + 4 * (lane >> 4));
      __asm__ __volatile__("" ::: "memory");
    }
}

// ---- bf16 S-stage pipeline (S = gemm_stages): slice it + S - 1 is requested while slice it
// is multiplied. Every iteration issues the same number of direct loads (the tail re-reads
// the last slice into a stage that is never read), so "this stage has landed" is always
// "at most (S - 2) * PW of this wave's loads outstanding".
template <int PW>
__device__ __forceinline__ void dma_slice(const char* const (&p1)[PW], const char* const (&p2)[PW], int kit_a, int kit,
                                          char* dst) {
  const bool seg2 = kit >= kit_a;
  const int64_t kb = (int64_t)(seg2 ? kit - kit_a : kit) * 128;
#pragma unroll
  for (int q = 0; q < PW; ++q)
    __builtin_amdgcn_global_load_lds((const void*)((seg2 ? p2[q] : p1[q]) + kb),
                                     (__attribute__((address_space(3))) void*)(dst + q * 1024), 16, 0, 0);
}

// The four 16-k steps of one 128-byte slice held in `cur`, on 32 x 32 output blocks.
// With NB = 2 the stage holds two B regions of BN rows each (the same output columns of two
// weight operands, Y then Y2): each A fragment read from LDS feeds both, and both products
// accumulate into the same blocks (independent blocks first, so no MFMA waits on the one
// just issued).
template <int BM, int BN, int WGM, int WGN, int NB = 1>
__device__ __forceinline__ void mma_slice32(const char* cur, int wm, int wn, int lane,
                                            f32x16_t (&acc)[BM / WGM / 32][BN / WGN / 32]) {
  __builtin_amdgcn_iglp_opt(0);  // let the scheduler interleave the LDS reads with the MFMAs
  constexpr int ROWB = 128;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  const char* sb = cur + BM * ROWB;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ch = 2 * ks + (lane >> 5);
    uint4 af[FM], bfr[NB][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WTM + i * 32 + (lane & 31);
      af[i] = *(const uint4*)(cur + r * ROWB + ((ch ^ lds_swz<true>(r)) << 4));
    }
#pragma unroll
    for (int s = 0; s < NB; ++s)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WTN + j * 32 + (lane & 31);
        bfr[s][j] = *(const uint4*)(sb + s * BN * ROWB + r * ROWB + ((ch ^ lds_swz<true>(r)) << 4));
      }
#pragma unroll
    for (int s = 0; s < NB; ++s)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mfma32(acc[i][j], af[i], bfr[s][j]);
  }
}

template <int J, int S>
__device__ __forceinline__ char* stage_ptr(char* s0, char* s1, char* s2) {
  constexpr int j = J % S;
  if constexpr (j == 0) return s0;
  else if constexpr (j == 1) return s1;
  else return s2;
}

// One K-iteration on stage J: wait until this wave's loads of the stage have landed (newer
// stages may stay in flight) and its LDS reads are done, barrier (everyone's loads landed,
// everyone finished reading the stage refilled next), request slice it + S - 1 into the
// stage read last iteration, multiply stage J. The barrier is written out because a
// fence-based barrier would also wait for the newer loads.
template <int BM, int BN, int WGM, int WGN, int PW, int S, int J, int NB>
__device__ __forceinline__ void step_slice32(char* s0, char* s1, char* s2, const char* const (&p1)[PW],
                                             const char* const (&p2)[PW], int kit_a, int kit0, int it, int n, int dmaoff,
                                             int wm, int wn, int lane,
                                             f32x16_t (&acc)[BM / WGM / 32][BN / WGN / 32]) {
  constexpr int NOUT = (S - 2) * PW;
  static_assert(NOUT < 64, "vmcnt holds at most 63");
  __asm__ __volatile__("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NOUT) : "memory");
  dma_slice<PW>(p1, p2, kit_a, kit0 + min(it + S - 1, n - 1), stage_ptr<J + S - 1, S>(s0, s1, s2) + dmaoff);
  mma_slice32<BM, BN, WGM, WGN, NB>(stage_ptr<J, S>(s0, s1, s2), wm, wn, lane, acc);
}

// The K loop. The stage pointers are restrict-qualified (they never overlap) and reach here
// through an opaque offset, so every LDS read and direct load carries an alias scope: the
// compiler then never waits for loads into one stage before reading another.
template <int BM, int BN, int WGM, int WGN, int PW, int S, int NB>
__device__ __forceinline__ void kloop32(char* __restrict__ s0, char* __restrict__ s1, char* __restrict__ s2,
                                        const char* const (&p1)[PW], const char* const (&p2)[PW], int kit_a, int kit0,
                                        int n, int dmaoff, int wm, int wn, int lane,
                                        f32x16_t (&acc)[BM / WGM / 32][BN / WGN / 32]) {
  static_assert(S == 2 || S == 3, "two or three stages");
  dma_slice<PW>(p1, p2, kit_a, kit0, s0 + dmaoff);
  if constexpr (S > 2) dma_slice<PW>(p1, p2, kit_a, kit0 + min(1, n - 1), s1 + dmaoff);
  for (int it = 0; it < n; it += S) {
    step_slice32<BM, BN, WGM, WGN, PW, S, 0, NB>(s0, s1, s2, p1, p2, kit_a, kit0, it, n, dmaoff, wm, wn, lane, acc);
    if (it + 1 < n)
      step_slice32<BM, BN, WGM, WGN, PW, S, 1, NB>(s0, s1, s2, p1, p2, kit_a, kit0, it + 1, n, dmaoff, wm, wn, lane, acc);
    if constexpr (S > 2)
      if (it + 2 < n)
        step_slice32<BM, BN, WGM, WGN, PW, S, 2, NB>(s0, s1, s2, p1, p2, kit_a, kit0, it + 2, n, dmaoff, wm, wn, lane, acc);
  }
  __syncthreads();  // every request has landed and every read is done: the LDS is free
}

// NB = 2 (bf16, 32 x 32 blocks only): C = X (Y + Y2)^T for a second K-segment that reads the
// same X rows (X2 = X): each stage holds the A rows once and the B rows of both weights, so a
// K-slice moves (BM + 2 BN) rows for the work of two slices of the concatenated walk, which
// would move 2 (BM + BN). kiters then counts one segment's slices.
template <class T, int BM, int BN, int WGM, int WGN, class Epi, int NB = 1>
__global__ void __launch_bounds__(WGM * WGN * 64) gemm_dma_kernel(GemmArgs g, Epi epi) {
  constexpr int WGM_ = WGM, WGN_ = WGN;
  constexpr int NW = WGM * WGN;
  constexpr int ROWB = 128;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int STAGE = (BM + NB * BN) * ROWB;
  constexpr int PW = (BM + NB * BN) / 8 / NW;  // 8-row blocks per wave
  static_assert(((BM + NB * BN) / 8) % NW == 0, "whole 8-row blocks per wave");
  static_assert(NB == 1 || (sizeof(T) == 2 && use_mfma32<T, BM, BN, WGM, WGN>()), "shared-X form: bf16, 32 x 32 blocks");
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  const GemmWork w = gemm_work(g);
  const int split = w.split, tile = w.tile;
  const int tm = tile % g.tiles_m, tn = tile / g.tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kit0 = split * g.kps;
  const int kit1 = min(g.kiters, kit0 + g.kps);

  // per 8-row block of this wave (A rows first, then B rows): source pointers of both
  // K-segments, formed once outside the K loop
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int rsub = lane >> 3;
  const bool has2 = g.kiters > g.kit_a;
  const char *gX, *gY, *gX2, *gY2;
  gemm_group_bases<T>(g, w.z, gX, gY, gX2, gY2);
  const char* p1[PW];
  const char* p2[PW];
#pragma unroll
  for (int q = 0; q < PW; ++q) {
    const int blk = wave_s * PW + q;
    const bool xs = blk * 8 < BM;  // whole 8-row blocks: BM % 8 == 0
    const int t = blk * 8 + rsub;  // tile-local row
    // lane L writes physical chunk L & 7 of row t; it loads logical chunk (L & 7) ^ swz(t)
    const int cbyte = ((lane & 7) ^ lds_swz<use_mfma32<T, BM, BN, WGM, WGN>()>(t)) << 4;
    if constexpr (NB == 2) {
      // A rows, then the B rows of Y, then those of Y2 (regions of 16k rows: the swizzle of
      // a row is the same counted from its region's start)
      const bool ys2 = t >= BM + BN;
      const int r = xs ? min(m0 + t, g.M - 1) : min(n0 + t - BM - (ys2 ? BN : 0), g.N - 1);
      const char* const b = xs ? gX : (ys2 ? gY2 : gY);
      const int64_t l = (xs ? g.ldx : (ys2 ? g.ldy2 : g.ldy)) * (int64_t)sizeof(T);
      p1[q] = b + (int64_t)r * l + cbyte;
      p2[q] = p1[q];
    } else {
      const int r = xs ? min(m0 + t, g.M - 1) : min(n0 + t - BM, g.N - 1);
      const char* const b1 = xs ? gX : gY;
      const char* const b2 = xs ? gX2 : gY2;
      const int64_t l1 = (xs ? g.ldx : g.ldy) * (int64_t)sizeof(T);
      const int64_t l2 = (xs ? g.ldx2 : g.ldy2) * (int64_t)sizeof(T);
      p1[q] = b1 + (int64_t)r * l1 + cbyte;
      p2[q] = has2 ? b2 + (int64_t)r * l2 + cbyte : p1[q];
    }
  }
  char* const sdst = smem + (wave_s * PW) * 1024;
  const int kit_a = g.kit_a;

  auto issue = [&](int kit, int stage) {
    const bool seg2 = kit >= kit_a;
    const int64_t kb = (int64_t)(seg2 ? kit - kit_a : kit) * ROWB;
    char* const d = sdst + stage * STAGE;
#pragma unroll
    for (int q = 0; q < PW; ++q)
      __builtin_amdgcn_global_load_lds((const void*)((seg2 ? p2[q] : p1[q]) + kb),
                                       (__attribute__((address_space(3))) void*)(d + q * 1024), 16, 0, 0);
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if constexpr (use_mfma32<T, BM, BN, WGM, WGN>()) {
    // 32 x 32 MFMA blocks, S-stage pipeline; re-dealt into the 16 x 16 layout after
    constexpr int S = gemm_stages_nb(BM, BN, NB);
    f32x16_t acc32[WTM / 32][WTN / 32];
#pragma unroll
    for (int i = 0; i < WTM / 32; ++i)
#pragma unroll
      for (int j = 0; j < WTN / 32; ++j) acc32[i][j] = f32x16_t{};
    int zero;
    __asm__ __volatile__("s_mov_b32 %0, 0" : "=s"(zero));
    char* const sm = smem + zero;
    if (kit0 < kit1)
      kloop32<BM, BN, WGM, WGN, PW, S, NB>(sm, sm + STAGE, S > 2 ? sm + 2 * STAGE : sm + STAGE, p1, p2, kit_a,
                                           kit0, kit1 - kit0, (wave_s * PW) * 1024, wm, wn, lane, acc32);
    acc32_to_16<WTM / 32, WTN / 32>(smem, wave, lane, acc32, acc);
    __syncthreads();  // the epilogue may reuse the LDS
  } else if constexpr (NB == 1) {
    if (kit0 < kit1) issue(kit0, 0);
    for (int it = kit0; it < kit1; ++it) {
      const int cur = (it - kit0) & 1;
      __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
      __syncthreads();
      const int nit = it + 1;
      const bool seg2 = nit >= kit_a;
      const int64_t kb = (int64_t)(seg2 ? nit - kit_a : nit) * ROWB;
      const char* src[PW];
#pragma unroll
      for (int q = 0; q < PW; ++q) src[q] = seg2 ? p2[q] : p1[q];
      dma_iteration<T, BM, BN, WGM, WGN, PW>(smem + cur * STAGE, sdst + (cur ^ 1) * STAGE, nit < kit1, src, kb, wm,
                                             wn, lane, acc);
    }
    __syncthreads();  // the epilogue may reuse the LDS
  }

  EpiPos pos;
  pos.row0 = w.z * g.M + m0 + wm * WTM;
  pos.col0 = n0 + wn * WTN;
  pos.lane = lane;
  pos.wave = wave;
  pos.wm = wm;
  pos.wn = wn;
  pos.wgm = WGM;
  pos.wgn = WGN;
  pos.bm = BM;
  pos.bn = BN;
  pos.tid = tid;
  pos.nthr = NW * 64;
  pos.smem_bytes = gemm_lds_bytes(BM, BN, NB);
  pos.tm = tm;
  pos.tn = tn;
  pos.tile = w.z * g.gtile + tile;
  pos.split = split;
  pos.M = (w.z + 1) * g.M;
  pos.N = g.N;
  pos.smem = smem;
  epi.template apply<FM, FN, WGM_, WGN_>(pos, acc);
}

// ---- token-major operands (bf16): C[M x N] = sum over k of X[k][i] Y[k][j], with X [K x M]
// and Y [K x N] stored row by row (the K index slowest), as the activations and their
// gradients come out of the chunk's row-major products: the weight gradients read them as
// they are, with no transposed copy. A K-slice of 64 rows of each operand goes to LDS by
// direct loads (each 1 KB load fills 64 consecutive 16-byte chunks of the row-major slice
// tile); the 16-byte chunks of a tile row are XOR-swizzled by km_swz, and the MFMA
// operands come out of LDS through gfx950's transposing read ds_read_b64_tr_b16: within
// each 16-lane group, lane 4q + w addresses row q, columns 4w .. 4w + 3 of a 4 x 16 block,
// and lane p receives column p, rows 0 .. 3. Two such reads give a lane the 8 consecutive
// k of its row that a 32 x 32 x 16 MFMA takes. Needs K a multiple of 64 and M, N multiples
// of 8.
// Swizzle of a slice-tile row's 16-byte chunks (cpr chunks per row). Half a wave's
// transposing read covers 4 consecutive rows x 4 aligned chunks; these 16 chunks take
// distinct 16-byte slots of the 256-byte bank window when every row's 4 chunks land in a
// quarter of their own. Rows of a multiple of 16 chunks all start at the same slot: XOR the
// chunk index with 4 (k mod 4). Rows of 24 chunks (192 columns): odd rows already start
// half a window away, so 4 ((k / 2) mod 2) suffices (and keeps the XOR within the row).
__device__ __forceinline__ int km_swz(int k, int cpr) {
  return (cpr & 15) == 0 ? (k & 3) << 2 : ((k >> 1) & 1) << 2;
}

typedef short km_v4s __attribute__((ext_vector_type(4)));
// One lane's 8 consecutive k (rows 16 ks + 8 (lane / 32) ..) of tile column c0 + lane % 32,
// from the slice tile at `tile` (RB bytes per row), as an MFMA operand.
template <int RB>
__device__ __forceinline__ uint4 km_operand(const char* tile, int c0, int ks, int lane) {
  const int g = lane >> 4, rl = lane & 15;
  const int col = c0 + 16 * (g & 1) + 4 * (rl & 3);
  const int k = 16 * ks + 8 * (g >> 1) + (rl >> 2);
  const int jl = col >> 3, within = (col & 7) * 2;
  const int o0 = k * RB + ((jl ^ km_swz(k, RB / 16)) << 4) + within;
  const int o1 = (k + 4) * RB + ((jl ^ km_swz(k + 4, RB / 16)) << 4) + within;
  const km_v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) km_v4s*)(tile + o0));
  const km_v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) km_v4s*)(tile + o1));
  const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  return make_uint4(ua.x, ua.y, ub.x, ub.y);
}

// One K-slice of the token-major loop on stage J (as step_slice32): wait until this wave's
// loads of the stage have landed and its LDS reads are done, barrier, request slice
// it + S - 1 into the stage read last iteration, multiply stage J.
template <int RBX, int RBY, int WTM, int WTN, int PW, int S, int J>
__device__ __forceinline__ void km_step(char* s0, char* s1, char* s2, const char* const (&src)[PW],
                                        const int64_t (&step)[PW], int it, int n, int dmaoff, int wm, int wn,
                                        int lane, f32x16_t (&acc)[WTM / 32][WTN / 32]) {
  constexpr int XB = 64 * RBX;
  constexpr int NOUT = (S - 2) * PW;
  __asm__ __volatile__("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NOUT) : "memory");
  {
    char* dst = stage_ptr<J + S - 1, S>(s0, s1, s2) + dmaoff;
    const int64_t kit = min(it + S - 1, n - 1);
#pragma unroll
    for (int q = 0; q < PW; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(src[q] + kit * step[q]),
                                       (__attribute__((address_space(3))) void*)(dst + q * 1024), 16, 0, 0);
  }
  const char* tx = stage_ptr<J, S>(s0, s1, s2);
  const char* ty = tx + XB;
  __builtin_amdgcn_iglp_opt(0);  // let the scheduler interleave the LDS reads with the MFMAs
  // the operands of k-step ks + 1 are read while the MFMAs of k-step ks run
  uint4 af[2][WTM / 32], bfr[2][WTN / 32];
#pragma unroll
  for (int i = 0; i < WTM / 32; ++i) af[0][i] = km_operand<RBX>(tx, wm * WTM + 32 * i, 0, lane);
#pragma unroll
  for (int j = 0; j < WTN / 32; ++j) bfr[0][j] = km_operand<RBY>(ty, wn * WTN + 32 * j, 0, lane);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int c = ks & 1;
    if (ks < 3) {
#pragma unroll
      for (int i = 0; i < WTM / 32; ++i) af[c ^ 1][i] = km_operand<RBX>(tx, wm * WTM + 32 * i, ks + 1, lane);
#pragma unroll
      for (int j = 0; j < WTN / 32; ++j) bfr[c ^ 1][j] = km_operand<RBY>(ty, wn * WTN + 32 * j, ks + 1, lane);
    }
#pragma unroll
    for (int i = 0; i < WTM / 32; ++i)
#pragma unroll
      for (int j = 0; j < WTN / 32; ++j) mfma32(acc[i][j], af[c][i], bfr[c][j]);
  }
}
// The K loop: restrict-qualified stage pointers reached through an opaque offset (as in
// kloop32), so that LDS reads of one stage never wait for the direct loads into another.
template <int RBX, int RBY, int WTM, int WTN, int PW, int S>
__device__ __forceinline__ void km_loop(char* __restrict__ s0, char* __restrict__ s1, char* __restrict__ s2,
                                        const char* const (&src)[PW], const int64_t (&step)[PW], int n, int dmaoff,
                                        int wm, int wn, int lane, f32x16_t (&acc)[WTM / 32][WTN / 32]) {
  static_assert(S == 2 || S == 3, "two or three stages");
#pragma unroll
  for (int q = 0; q < PW; ++q)
    __builtin_amdgcn_global_load_lds((const void*)src[q], (__attribute__((address_space(3))) void*)(s0 + dmaoff + q * 1024),
                                     16, 0, 0);
  if constexpr (S > 2) {
    const int64_t k1 = min(1, n - 1);
#pragma unroll
    for (int q = 0; q < PW; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(src[q] + k1 * step[q]),
                                       (__attribute__((address_space(3))) void*)(s1 + dmaoff + q * 1024), 16, 0, 0);
  }
  for (int it = 0; it < n; it += S) {
    km_step<RBX, RBY, WTM, WTN, PW, S, 0>(s0, s1, s2, src, step, it, n, dmaoff, wm, wn, lane, acc);
    if (it + 1 < n) km_step<RBX, RBY, WTM, WTN, PW, S, 1>(s0, s1, s2, src, step, it + 1, n, dmaoff, wm, wn, lane, acc);
    if constexpr (S > 2)
      if (it + 2 < n) km_step<RBX, RBY, WTM, WTN, PW, S, 2>(s0, s1, s2, src, step, it + 2, n, dmaoff, wm, wn, lane, acc);
  }
  __syncthreads();  // every request has landed and every read is done: the LDS is free
}

template <int BM, int BN, int WGM, int WGN, class Epi>
__global__ void __launch_bounds__(WGM * WGN * 64) gemm_km_kernel(GemmArgs g, Epi epi) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM32 = WTM / 32, FN32 = WTN / 32;
  constexpr int RBX = 2 * BM, RBY = 2 * BN;          // bytes per slice-tile row
  constexpr int XB = 64 * RBX, YB = 64 * RBY;        // bytes per slice tile
  constexpr int STAGE = XB + YB;
  constexpr int S = gemm_stages(BM, BN);  // 128 x 128: two stages, two workgroups per CU
  constexpr int NL = STAGE / 1024;                   // 1 KB direct loads per slice
  constexpr int PW = NL / NW;
  static_assert(XB % 1024 == 0 && YB % 1024 == 0 && NL % NW == 0, "whole 1 KB loads per wave");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0 && BM % 64 == 0 && BN % 64 == 0, "32 x 32 blocks, 8-chunk rows");
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const GemmWork w = gemm_work(g);
  const int tile = w.tile;
  const int tm = tile % g.tiles_m, tn = tile / g.tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const char *gX, *gY, *gX2, *gY2;
  gemm_group_bases<bf16_t>(g, w.z, gX, gY, gX2, gY2);
  // this lane's source of each of the wave's loads (slice 0), and the step to the next slice
  const char* src[PW];
  int64_t step[PW];
#pragma unroll
  for (int q = 0; q < PW; ++q) {
    const int t = wave_s * PW + q;           // load index within the stage
    const bool xs = t < XB / 1024;
    const int tl = xs ? t : t - XB / 1024;   // within the operand's tile
    const int cpr = (xs ? RBX : RBY) / 16;   // chunks per tile row
    const int c = 64 * tl + lane;
    const int k = c / cpr, jp = c - k * cpr;
    const int jl = jp ^ km_swz(k, cpr);
    const int lim = xs ? g.M : g.N, base = xs ? m0 : n0;
    int col = base + 8 * jl;
    if (col > lim - 8) col = lim - 8;        // columns past the edge: a valid chunk, masked later
    const int64_t ld = xs ? g.ldx : g.ldy;
    src[q] = (xs ? gX : gY) + ((int64_t)k * ld + col) * 2;
    step[q] = 64 * ld * 2;
  }
  f32x16_t acc32[FM32][FN32];
#pragma unroll
  for (int i = 0; i < FM32; ++i)
#pragma unroll
    for (int j = 0; j < FN32; ++j) acc32[i][j] = f32x16_t{};
  int zero;
  __asm__ __volatile__("s_mov_b32 %0, 0" : "=s"(zero));
  char* const sm = smem + zero;
  km_loop<RBX, RBY, WTM, WTN, PW, S>(sm, sm + STAGE, S > 2 ? sm + 2 * STAGE : sm + STAGE, src, step, g.kiters,
                                     (wave_s * PW) * 1024, wm, wn, lane, acc32);
  f32x4_t acc[WTM / 16][WTN / 16];
  acc32_to_16<FM32, FN32>(smem, wave, lane, acc32, acc);
  __syncthreads();
  EpiPos pos;
  pos.row0 = w.z * g.M + m0 + wm * WTM;
  pos.col0 = n0 + wn * WTN;
  pos.lane = lane;
  pos.wave = wave;
  pos.wm = wm;
  pos.wn = wn;
  pos.wgm = WGM;
  pos.wgn = WGN;
  pos.bm = BM;
  pos.bn = BN;
  pos.tid = tid;
  pos.nthr = NW * 64;
  pos.smem_bytes = S * STAGE;
  pos.tm = tm;
  pos.tn = tn;
  pos.tile = w.z * g.gtile + tile;
  pos.split = 0;
  pos.M = (w.z + 1) * g.M;
  pos.N = g.N;
  pos.smem = smem;
  epi.template apply<WTM / 16, WTN / 16, WGM, WGN>(pos, acc);
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

// ---- LDS staging of bf16 tiles, so that global traffic is 16-byte and row-contiguous.
// A lane's 4 vertically adjacent values (rows r0..r0+3 of one column) travel packed in two
// dwords: lo half = row r0 (or r0+2), hi half = row r0+1 (or r0+3).
template <int FM, int FN>
using Packed = uint32_t[FM][FN][2];

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) { return pack_bf16x2(lo, hi); }

// Copy the LDS tile (R rows of L elements, row stride ldl) to dst rows [g0, g0 + R) and
// columns [c0, c0 + L), clipped to rows < gr_lim and columns < gc_lim.
__device__ __forceinline__ void lds_to_global_bf16(const EpiPos& p, const bf16_t* lds, int ldl, int R, int L,
                                                   bf16_t* dst, int64_t ld, int g0, int c0, int gr_lim, int gc_lim) {
  const int cpr = L / 8;
  const bool vec_ok = (ld % 8) == 0;
  for (int idx = p.tid; idx < R * cpr; idx += p.nthr) {
    const int r = idx / cpr, c = (idx - r * cpr) * 8;
    const int gr = g0 + r, gc = c0 + c;
    if (gr >= gr_lim || gc >= gc_lim) continue;
    const bf16_t* s = lds + r * ldl + c;
    bf16_t* d = dst + (int64_t)gr * ld + gc;
    if (vec_ok && gc + 8 <= gc_lim) {
      *(uint4*)d = *(const uint4*)s;
    } else {
      for (int k = 0; k < 8 && gc + k < gc_lim; ++k) d[k] = s[k];
    }
  }
}

// Row-major store of the tile's values into dst [M x ld]. Returns false (nothing written)
// when the tile does not fit the LDS; the caller then stores directly.
// Compile-time tile geometry of an epilogue: BM x BN tile, LDS of the two K stages.
template <int FM, int FN, int WGM, int WGN>
struct TileGeo {
  static constexpr int WTM = 16 * FM, WTN = 16 * FN;
  static constexpr int BM = WGM * WTM, BN = WGN * WTN;
  static constexpr int SMEM = gemm_stages(BM, BN) * (BM + BN) * 128;
  static constexpr bool ROWS_PAD = BM * (BN + 8) * 2 <= SMEM;
  static constexpr int LDR = ROWS_PAD ? BN + 8 : BN;         // row-major staging stride
  static constexpr bool ROWS_FIT = BM * LDR * 2 <= SMEM;
  static constexpr int LDC = BM + 8;                          // transposed staging stride
  static constexpr bool COLS_FIT = BN * LDC * 2 <= SMEM;
};

template <int FM, int FN, int WGM, int WGN>
__device__ __forceinline__ bool stage_rows_bf16(const EpiPos& p, const Packed<FM, FN>& v, bf16_t* dst, int64_t ld) {
  using G = TileGeo<FM, FN, WGM, WGN>;
  if constexpr (!G::ROWS_FIT) return false;
  constexpr int ldl = G::LDR, WTM = G::WTM, WTN = G::WTN;
  bf16_t* lds = (bf16_t*)p.smem;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int rl = p.wm * WTM + 16 * i + 4 * (p.lane >> 4);
      const int cl = p.wn * WTN + 16 * j + (p.lane & 15);
      lds[(rl + 0) * ldl + cl] = (bf16_t)(v[i][j][0] & 0xffff);
      lds[(rl + 1) * ldl + cl] = (bf16_t)(v[i][j][0] >> 16);
      lds[(rl + 2) * ldl + cl] = (bf16_t)(v[i][j][1] & 0xffff);
      lds[(rl + 3) * ldl + cl] = (bf16_t)(v[i][j][1] >> 16);
    }
  __syncthreads();
  lds_to_global_bf16(p, lds, ldl, G::BM, G::BN, dst, ld, p.row0 - p.wm * WTM, p.col0 - p.wn * WTN, p.M, p.N);
  return true;
}

// Transposed store: dstT [N x ldt] receives the tile's columns as rows.
template <int FM, int FN, int WGM, int WGN>
__device__ __forceinline__ bool stage_cols_bf16(const EpiPos& p, const Packed<FM, FN>& v, bf16_t* dstT, int64_t ldt) {
  using G = TileGeo<FM, FN, WGM, WGN>;
  if constexpr (!G::COLS_FIT) return false;
  constexpr int ldl = G::LDC, WTM = G::WTM, WTN = G::WTN;
  bf16_t* lds = (bf16_t*)p.smem;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int rl = p.wm * WTM + 16 * i + 4 * (p.lane >> 4);
      const int cl = p.wn * WTN + 16 * j + (p.lane & 15);
      *(uint2*)(lds + cl * ldl + rl) = make_uint2(v[i][j][0], v[i][j][1]);
    }
  __syncthreads();
  lds_to_global_bf16(p, lds, ldl, G::BN, G::BM, dstT, ldt, p.col0 - p.wn * WTN, p.row0 - p.wm * WTM, p.N, p.M);
  return true;
}

// Load the tile region [rows of the tile] x [columns of the tile] of a row-major bf16
// matrix into LDS (row stride bn + 8; values outside M x N read as 0). Returns false when
// it does not fit; afterwards lane values are read with staged_at().
template <int FM, int FN, int WGM, int WGN>
__device__ __forceinline__ bool stage_load_bf16(const EpiPos& p, const bf16_t* src, int64_t ld) {
  using G = TileGeo<FM, FN, WGM, WGN>;
  if constexpr (!(G::ROWS_PAD && G::ROWS_FIT)) return false;
  constexpr int ldl = G::BN + 8;
  bf16_t* lds = (bf16_t*)p.smem;
  const int g0 = p.row0 - p.wm * G::WTM, c0 = p.col0 - p.wn * G::WTN;
  constexpr int cpr = G::BN / 8;
  const bool vec_ok = (ld % 8) == 0;
  __syncthreads();
  for (int idx = p.tid; idx < G::BM * cpr; idx += WGM * WGN * 64) {
    const int r = idx / cpr, c = (idx - r * cpr) * 8;
    const int gr = g0 + r, gc = c0 + c;
    bf16_t* dl = lds + r * ldl + c;
    const bf16_t* s = src + (int64_t)gr * ld + gc;
    if (gr < p.M && vec_ok && gc + 8 <= p.N) {
      *(uint4*)dl = *(const uint4*)s;
    } else {
      for (int k = 0; k < 8; ++k) dl[k] = (gr < p.M && gc + k < p.N) ? s[k] : (bf16_t)0;
    }
  }
  __syncthreads();
  return true;
}
template <int FM, int FN, int WGM, int WGN>
__device__ __forceinline__ float staged_at(const EpiPos& p, int rl, int cl) {
  return bf2f(((const bf16_t*)p.smem)[rl * (TileGeo<FM, FN, WGM, WGN>::BN + 8) + cl]);
}

// ---- fp32 accumulator tile in LDS, processed by rolled loops (small register footprint,
// row-contiguous global traffic). Needs BM * BN * 4 bytes of LDS (the 128 x 128 tiles).
template <int FM, int FN, int WGM, int WGN>
struct AccTile {
  using G = TileGeo<FM, FN, WGM, WGN>;
  static constexpr bool FITS = G::BM * G::BN * 4 <= G::SMEM;
  static constexpr int NT = WGM * WGN * 64;
};

// Write the accumulators into LDS as a row-major [BM][BN] fp32 tile.
template <int FM, int FN, int WGM, int WGN>
__device__ __forceinline__ void acc_to_lds(const EpiPos& p, const f32x4_t (&acc)[FM][FN]) {
  using G = TileGeo<FM, FN, WGM, WGN>;
  float* U = (float*)p.smem;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int rl = p.wm * G::WTM + 16 * i + 4 * (p.lane >> 4);
      const int cl = p.wn * G::WTN + 16 * j + (p.lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) U[(rl + e) * G::BN + cl] = acc[i][j][e];
    }
  __syncthreads();
}

__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
// Store 4 consecutive values of a row (8 bytes when aligned and whole).
__device__ __forceinline__ void store_row4_bf16(bf16_t* d, float a, float b, float c, float e, int nvalid) {
  if (nvalid >= 4) {
    *(uint2*)d = pack4_bf16(a, b, c, e);
  } else {
    if (nvalid > 0) d[0] = f2bf(a);
    if (nvalid > 1) d[1] = f2bf(b);
    if (nvalid > 2) d[2] = f2bf(c);
  }
}
__device__ __forceinline__ float4 load_row4_bf16(const bf16_t* s, int nvalid) {
  if (nvalid >= 4) {
    const uint2 u = *(const uint2*)s;
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                       __uint_as_float(u.y & 0xffff0000u));
  }
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (nvalid > 0) v[0] = bf2f(s[0]);
  if (nvalid > 1) v[1] = bf2f(s[1]);
  if (nvalid > 2) v[2] = bf2f(s[2]);
  return make_float4(v[0], v[1], v[2], v[3]);
}

// Store 8 consecutive values of a row: one 16-byte store when whole and aligned.
__device__ __forceinline__ void store_row8_bf16(bf16_t* d, const float (&v)[8], int nvalid, bool aligned) {
  if (nvalid >= 8 && aligned) {
    *(uint4*)d = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                            pack_bf16x2(v[6], v[7]));
  } else {
    store_row4_bf16(d, v[0], v[1], v[2], v[3], nvalid);
    if (nvalid > 4) store_row4_bf16(d + 4, v[4], v[5], v[6], v[7], nvalid - 4);
  }
}

// Transposed store of the LDS fp32 tile: dstT row (n0 + c) gets tile column c, 8 rows per
// thread (16-byte stores); lanes walk consecutive columns (bank-conflict-free LDS reads).
template <int FM, int FN, int WGM, int WGN>
__device__ __forceinline__ void lds_cols_to_global_bf16(const EpiPos& p, bf16_t* dstT, int64_t ldt) {
  using G = TileGeo<FM, FN, WGM, WGN>;
  const float* U = (const float*)p.smem;
  const int m0 = p.row0 - p.wm * G::WTM, n0 = p.col0 - p.wn * G::WTN;
  const bool vec_ok = (ldt % 8) == 0;
#pragma unroll 1
  for (int idx = p.tid; idx < G::BN * (G::BM / 8); idx += AccTile<FM, FN, WGM, WGN>::NT) {
    const int c = idx % G::BN, r = (idx / G::BN) * 8;
    const int gc = n0 + c, gr = m0 + r;
    if (gc >= p.N || gr >= p.M) continue;
    bf16_t* d = dstT + (int64_t)gc * ldt + gr;
    if (vec_ok && gr + 8 <= p.M) {
      uint4 v;
      v.x = pack_bf2(U[(r + 0) * G::BN + c], U[(r + 1) * G::BN + c]);
      v.y = pack_bf2(U[(r + 2) * G::BN + c], U[(r + 3) * G::BN + c]);
      v.z = pack_bf2(U[(r + 4) * G::BN + c], U[(r + 5) * G::BN + c]);
      v.w = pack_bf2(U[(r + 6) * G::BN + c], U[(r + 7) * G::BN + c]);
      *(uint4*)d = v;
    } else {
      for (int k = 0; k < 8 && gr + k < p.M; ++k) d[k] = f2bf(U[(r + k) * G::BN + c]);
    }
  }
}

// Plain fp32 store, optionally accumulating, with one output slab per split.
struct EpiStoreF32 {
  float* C;
  int64_t ldc;
  int64_t split_stride;
  int accumulate;
  template <int FM, int FN, int WGM, int WGN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
    float* Cs = C + (int64_t)p.split * split_stride;
    if (accumulate) {
      // every old value is requested before any is used (clamped addresses, masked below)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = min(epi_row(p, i, e), p.M - 1);
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j][e] += Cs[(int64_t)row * ldc + min(epi_col(p, j), p.N - 1)];
        }
    }
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
          Cs[(int64_t)row * ldc + col] = acc[i][j][e];
        }
      }
  }
};

// Per-row sum over the tile's columns of a per-element value v[i][e] (already summed over
// the wave's j blocks by the caller): 16-lane butterfly, then the column waves' partials
// are combined through LDS in column order and written to out[tn * ldo + row]. Fixed
// order, so deterministic. Uses wgn * bm floats of LDS; all threads must call it.
template <int FM>
__device__ __forceinline__ void row_partial_store(const EpiPos& p, float (&v)[FM][4], float* out, int64_t ldo) {
  constexpr int WTM = 16 * FM;
  float* l1 = (float*)p.smem;
  __syncthreads();  // the LDS may still be read by a preceding staged copy
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[i][e] = xor16_sum(v[i][e]);
      if ((p.lane & 15) == 0) l1[p.wn * p.bm + p.wm * WTM + 16 * i + 4 * (p.lane >> 4) + e] = v[i][e];
    }
  __syncthreads();
  if (p.wn == 0 && (p.lane & 15) == 0) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = epi_row(p, i, e);
        const int lr = p.wm * WTM + 16 * i + 4 * (p.lane >> 4) + e;
        float sum = l1[lr];
        for (int c = 1; c < p.wgn; ++c) sum += l1[c * p.bm + lr];
        if (row < p.M) out[(int64_t)p.tn * ldo + row] = sum;
      }
  }
}

// Up-projection of a GELU block: U = Hn W1 -> A = GELU(U) (row-major and transposed) and
// GELU'(U) for the backward pass. RES (optional) keeps A - rn(A), the rounding residual of
// the stored operand, for the first-order loss compensation.
template <class T>
struct EpiGelu {
  T* A;     // [M x lda]
  T* AT;    // [N x ldat] or null
  T* GP;    // [M x lda]
  T* RES;   // [M x lda] or null
  int64_t lda, ldat;
  const float* ADD = nullptr;  // [M x lda] fp32 added to U before the GELU, or null
  template <int FM, int FN, int WGM, int WGN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
    if constexpr (sizeof(T) == 2 && AccTile<FM, FN, WGM, WGN>::FITS) {
      using G = TileGeo<FM, FN, WGM, WGN>;
      acc_to_lds<FM, FN, WGM, WGN>(p, acc);
      float* U = (float*)p.smem;
      const int m0 = p.row0 - p.wm * G::WTM, n0 = p.col0 - p.wn * G::WTN;
      const bool aligned = (lda & 7) == 0;
      // rows of 8: A, GELU'(U), rounding residual; A written back in place for the transposed pass
#pragma unroll 1
      for (int idx = p.tid; idx < G::BM * (G::BN / 8); idx += AccTile<FM, FN, WGM, WGN>::NT) {
        const int r = idx / (G::BN / 8), c = (idx % (G::BN / 8)) * 8;
        const int gr = m0 + r, gc = n0 + c;
        float4* up = (float4*)(U + r * G::BN + c);
        const float4 u0 = up[0], u1 = up[1];
        float uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        if (ADD && gr < p.M) {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (gc + q < p.N) uu[q] += ADD[(int64_t)gr * lda + gc + q];
        }
        float a[8], gp[8], rs[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          gelu_pair(uu[q], a[q], gp[q]);
          rs[q] = a[q] - bf2f(f2bf(a[q]));
        }
        up[0] = make_float4(a[0], a[1], a[2], a[3]);
        up[1] = make_float4(a[4], a[5], a[6], a[7]);
        if (gr < p.M && gc < p.N) {
          const int nv = min(8, p.N - gc);
          const int64_t o = (int64_t)gr * lda + gc;
          store_row8_bf16((bf16_t*)A + o, a, nv, aligned);
          store_row8_bf16((bf16_t*)GP + o, gp, nv, aligned);
          if (RES) store_row8_bf16((bf16_t*)RES + o, rs, nv, aligned);
        }
      }
      __syncthreads();
      if (AT) lds_cols_to_global_bf16<FM, FN, WGM, WGN>(p, (bf16_t*)AT, ldat);
      return;
    }
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
          float gp;
          const float add = (ADD && e < nv) ? ADD[(int64_t)(r0 + e) * lda + col] : 0.f;
          gelu_pair(acc[i][j][e] + add, a[e], gp);
          if (e < nv) {
            const int64_t o = (int64_t)(r0 + e) * lda + col;
            const T q = from_f<T>(a[e]);
            A[o] = q;
            GP[o] = from_f<T>(gp);
            if (RES) RES[o] = from_f<T>(a[e] - to_f<T>(q));
          }
        }
        if (AT) store4_t<T>(AT + (int64_t)col * ldat + r0, a[0], a[1], a[2], a[3], nv);
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
  template <int FM, int FN, int WGM, int WGN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
    if constexpr (sizeof(T) == 2 && AccTile<FM, FN, WGM, WGN>::FITS && TileGeo<FM, FN, WGM, WGN>::BN == 128) {
      // interior tiles: the fp32 tile in LDS, rows of 8 columns per thread with 16-byte
      // accesses (every gate piece requested before any is used); A written back to LDS for
      // the transposed pass
      using G = TileGeo<FM, FN, WGM, WGN>;
      constexpr int NT = AccTile<FM, FN, WGM, WGN>::NT;
      constexpr int TPR = G::BN / 8, RPP = NT / TPR, NP = G::BM / RPP;
      const int m0 = p.row0 - p.wm * G::WTM, n0 = p.col0 - p.wn * G::WTN;
      if (m0 + G::BM <= p.M && n0 + G::BN <= p.N && (lda & 7) == 0 && (NT % TPR) == 0 && (G::BM % RPP) == 0) {
        acc_to_lds<FM, FN, WGM, WGN>(p, acc);
        float* U = (float*)p.smem;
        const int c = (p.tid % TPR) * 8;
        float4 g0[NP], g1[NP];
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          const int64_t o = (int64_t)(m0 + k * RPP + p.tid / TPR) * lda + n0 + c;
          g0[k] = *(const float4*)(UG + o);
          g1[k] = *(const float4*)(UG + o + 4);
        }
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          const int r = k * RPP + p.tid / TPR;
          const int64_t o = (int64_t)(m0 + r) * lda + n0 + c;
          float4* up = (float4*)(U + r * G::BN + c);
          const float4 v0 = up[0], v1 = up[1];
          const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
          const float g[8] = {g0[k].x, g0[k].y, g0[k].z, g0[k].w, g1[k].x, g1[k].y, g1[k].z, g1[k].w};
          float a[8], rs[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            a[q] = silu_f(g[q]) * v[q];
            rs[q] = a[q] - bf2f(f2bf(a[q]));
          }
          store_row8_bf16((bf16_t*)A + o, a, 8, true);
          if (VU) {
            *(float4*)(VU + o) = v0;
            *(float4*)(VU + o + 4) = v1;
          }
          if (RES) store_row8_bf16((bf16_t*)RES + o, rs, 8, true);
          up[0] = make_float4(a[0], a[1], a[2], a[3]);
          up[1] = make_float4(a[4], a[5], a[6], a[7]);
        }
        __syncthreads();
        if (AT) lds_cols_to_global_bf16<FM, FN, WGM, WGN>(p, (bf16_t*)AT, ldat);
        return;
      }
    }
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
        if (AT) store4_t<T>(AT + (int64_t)col * ldat + r0, a[0], a[1], a[2], a[3], nv);
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
  T* DUT;        // [N x ldt] or null
  const T* RES;  // [M x ld] or null
  float* cdot;   // [tiles_n x ldc] or null (ldc >= rows of the stacked output)
  int64_t ld, ldt, ldc;
  template <int FM, int FN, int WGM, int WGN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
    float dots[FM][4];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) dots[i][e] = 0.f;
    if constexpr (sizeof(T) == 2 && AccTile<FM, FN, WGM, WGN>::FITS && TileGeo<FM, FN, WGM, WGN>::BN == 128) {
      // rows are covered by 32 consecutive threads (4 columns each): their partial dots
      // combine with a 32-lane butterfly in a fixed order
      using G = TileGeo<FM, FN, WGM, WGN>;
      acc_to_lds<FM, FN, WGM, WGN>(p, acc);
      float* U = (float*)p.smem;
      const int m0 = p.row0 - p.wm * G::WTM, n0 = p.col0 - p.wn * G::WTN;
      constexpr int NT = AccTile<FM, FN, WGM, WGN>::NT;
      constexpr int TPR = G::BN / 8, RPP = NT / TPR, NP = G::BM / RPP;  // rows of 8 per thread
      if (m0 + G::BM <= p.M && n0 + G::BN <= p.N && (ld & 7) == 0 && (NT % TPR) == 0 && (G::BM % RPP) == 0) {
        // interior tile: every GP / RES row piece is requested before any is used
        const int c = (p.tid % TPR) * 8;
        uint4 gq[NP], rq[NP];
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          const int64_t o = (int64_t)(m0 + k * RPP + p.tid / TPR) * ld + n0 + c;
          gq[k] = *(const uint4*)((const bf16_t*)GP + o);
          rq[k] = RES ? *(const uint4*)((const bf16_t*)RES + o) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < NP; ++k) {
          const int r = k * RPP + p.tid / TPR;
          float4* up = (float4*)(U + r * G::BN + c);
          const float4 a0 = up[0], a1 = up[1];
          const float da[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
          const uint32_t gw[4] = {gq[k].x, gq[k].y, gq[k].z, gq[k].w};
          const uint32_t rw[4] = {rq[k].x, rq[k].y, rq[k].z, rq[k].w};
          float du[8];
          float dot = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            du[2 * q] = da[2 * q] * __uint_as_float(gw[q] << 16);
            du[2 * q + 1] = da[2 * q + 1] * __uint_as_float(gw[q] & 0xffff0000u);
            dot = fmaf(da[2 * q], __uint_as_float(rw[q] << 16), dot);
            dot = fmaf(da[2 * q + 1], __uint_as_float(rw[q] & 0xffff0000u), dot);
          }
          *(uint4*)((bf16_t*)DU + (int64_t)(m0 + r) * ld + n0 + c) =
              make_uint4(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]), pack_bf16x2(du[4], du[5]),
                         pack_bf16x2(du[6], du[7]));
          up[0] = make_float4(du[0], du[1], du[2], du[3]);
          up[1] = make_float4(du[4], du[5], du[6], du[7]);
          if (cdot) {
            if constexpr (TPR == 16) {
              dot = row16_sum(dot);
            } else {
#pragma unroll
              for (int off = 1; off < TPR; off <<= 1) dot += __shfl_xor(dot, off, TTT_WAVE);
            }
            if ((p.tid % TPR) == 0) cdot[(int64_t)p.tn * ldc + m0 + r] = dot;
          }
        }
        __syncthreads();
        if (DUT) lds_cols_to_global_bf16<FM, FN, WGM, WGN>(p, (bf16_t*)DUT, ldt);
        return;
      }
#pragma unroll 1
      for (int base = 0; base < G::BM * 32; base += AccTile<FM, FN, WGM, WGN>::NT) {
        const int idx = base + p.tid;
        const int r = idx >> 5, c = (idx & 31) * 4;
        const int gr = m0 + r, gc = n0 + c;
        float4* up = (float4*)(U + r * G::BN + c);
        const float4 da = *up;
        float4 du = make_float4(0.f, 0.f, 0.f, 0.f);
        float dot = 0.f;
        if (gr < p.M && gc < p.N) {
          const int nv = min(4, p.N - gc);
          const int64_t o = (int64_t)gr * ld + gc;
          const float4 g = load_row4_bf16((const bf16_t*)GP + o, nv);
          du = make_float4(da.x * g.x, da.y * g.y, da.z * g.z, da.w * g.w);
          store_row4_bf16((bf16_t*)DU + o, du.x, du.y, du.z, du.w, nv);
          if (RES) {
            const float4 rr = load_row4_bf16((const bf16_t*)RES + o, nv);
            dot = (da.x * rr.x + da.y * rr.y) + (da.z * rr.z + da.w * rr.w);
          }
        }
        *up = du;
        if (cdot) {
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) dot += __shfl_xor(dot, off, TTT_WAVE);
          if ((p.lane & 31) == 0 && gr < p.M) cdot[(int64_t)p.tn * ldc + gr] = dot;
        }
      }
      __syncthreads();
      if (DUT) lds_cols_to_global_bf16<FM, FN, WGM, WGN>(p, (bf16_t*)DUT, ldt);
      return;
    }
    if constexpr (sizeof(T) == 2 && TileGeo<FM, FN, WGM, WGN>::BN != 128 &&
                  (TileGeo<FM, FN, WGM, WGN>::BM * TileGeo<FM, FN, WGM, WGN>::BN * 4 +
                   TileGeo<FM, FN, WGM, WGN>::BM * (TileGeo<FM, FN, WGM, WGN>::BN / 8) * 4) <=
                      TileGeo<FM, FN, WGM, WGN>::SMEM) {
      // other tile widths: the fp32 tile in LDS, rows of 8 columns per thread (16-byte
      // accesses), each piece's partial dot kept in LDS and summed per row in column order
      using G = TileGeo<FM, FN, WGM, WGN>;
      constexpr int CH = G::BN / 8, NT = WGM * WGN * 64;
      acc_to_lds<FM, FN, WGM, WGN>(p, acc);
      float* U = (float*)p.smem;
      float* red = U + G::BM * G::BN;
      const int m0 = p.row0 - p.wm * G::WTM, n0 = p.col0 - p.wn * G::WTN;
      const bool vec = (ld & 7) == 0;
#pragma unroll 1
      for (int idx = p.tid; idx < G::BM * CH; idx += NT) {
        const int r = idx / CH, c = (idx - r * CH) * 8;
        const int gr = m0 + r, gc = n0 + c;
        float* up = U + r * G::BN + c;
        float du[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float dot = 0.f;
        if (gr < p.M && gc < p.N) {
          const int64_t o = (int64_t)gr * ld + gc;
          const int nv = min(8, p.N - gc);
          if (vec && nv == 8) {
            const uint4 gq = *(const uint4*)((const bf16_t*)GP + o);
            const uint4 rq = RES ? *(const uint4*)((const bf16_t*)RES + o) : make_uint4(0, 0, 0, 0);
            const uint32_t gw[4] = {gq.x, gq.y, gq.z, gq.w}, rw[4] = {rq.x, rq.y, rq.z, rq.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float a0 = up[2 * q], a1 = up[2 * q + 1];
              du[2 * q] = a0 * __uint_as_float(gw[q] << 16);
              du[2 * q + 1] = a1 * __uint_as_float(gw[q] & 0xffff0000u);
              dot = fmaf(a0, __uint_as_float(rw[q] << 16), dot);
              dot = fmaf(a1, __uint_as_float(rw[q] & 0xffff0000u), dot);
            }
            *(uint4*)((bf16_t*)DU + o) = make_uint4(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]),
                                                    pack_bf16x2(du[4], du[5]), pack_bf16x2(du[6], du[7]));
          } else {
            for (int k = 0; k < nv; ++k) {
              du[k] = up[k] * to_f<T>(GP[o + k]);
              DU[o + k] = from_f<T>(du[k]);
              if (RES) dot = fmaf(up[k], to_f<T>(RES[o + k]), dot);
            }
          }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) up[k] = du[k];
        red[idx] = dot;
      }
      __syncthreads();
      if (cdot) {
        for (int r = p.tid; r < G::BM; r += NT) {
          float sum = red[r * CH];
          for (int k = 1; k < CH; ++k) sum += red[r * CH + k];
          if (m0 + r < p.M) cdot[(int64_t)p.tn * ldc + m0 + r] = sum;
        }
      }
      if (DUT) lds_cols_to_global_bf16<FM, FN, WGM, WGN>(p, (bf16_t*)DUT, ldt);
      return;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
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
        if (DUT) store4_t<T>(DUT + (int64_t)col * ldt + r0, v[0], v[1], v[2], v[3], nv);
      }
    }
    if (cdot) row_partial_store<FM>(p, dots, cdot, ldc);
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
  float* cdot;  // [tiles_n x ldc]
  int64_t ld, ldc;
  template <int FM, int FN, int WGM, int WGN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
    if constexpr (sizeof(T) == 2 && AccTile<FM, FN, WGM, WGN>::FITS && TileGeo<FM, FN, WGM, WGN>::BN == 128) {
      // interior tiles: the fp32 tile in LDS, rows of 8 columns per thread with 16-byte
      // accesses, in two halves of a thread's rows (each half's operand pieces requested
      // before any is used); each row's partial dot sums its 16 pieces in a fixed order
      using G = TileGeo<FM, FN, WGM, WGN>;
      constexpr int NT = AccTile<FM, FN, WGM, WGN>::NT;
      constexpr int TPR = G::BN / 8, RPP = NT / TPR, NP = G::BM / RPP, NH = NP / 2;
      const int m0 = p.row0 - p.wm * G::WTM, n0 = p.col0 - p.wn * G::WTN;
      if (m0 + G::BM <= p.M && n0 + G::BN <= p.N && (ld & 7) == 0 && (NT % TPR) == 0 && (G::BM % RPP) == 0 &&
          NP % 2 == 0 && TPR == 16) {
        acc_to_lds<FM, FN, WGM, WGN>(p, acc);
        const float* U = (const float*)p.smem;
        const int c = (p.tid % TPR) * 8;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float4 g0[NH], g1[NH], v0[NH], v1[NH];
          uint4 rq[NH];
#pragma unroll
          for (int k = 0; k < NH; ++k) {
            const int64_t o = (int64_t)(m0 + (h * NH + k) * RPP + p.tid / TPR) * ld + n0 + c;
            g0[k] = *(const float4*)(UG + o);
            g1[k] = *(const float4*)(UG + o + 4);
            v0[k] = *(const float4*)(VU + o);
            v1[k] = *(const float4*)(VU + o + 4);
            rq[k] = RES ? *(const uint4*)((const bf16_t*)RES + o) : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int k = 0; k < NH; ++k) {
            const int r = (h * NH + k) * RPP + p.tid / TPR;
            const int64_t o = (int64_t)(m0 + r) * ld + n0 + c;
            const float4 a0 = *(const float4*)(U + r * G::BN + c), a1 = *(const float4*)(U + r * G::BN + c + 4);
            const float da[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float g[8] = {g0[k].x, g0[k].y, g0[k].z, g0[k].w, g1[k].x, g1[k].y, g1[k].z, g1[k].w};
            const float vu[8] = {v0[k].x, v0[k].y, v0[k].z, v0[k].w, v1[k].x, v1[k].y, v1[k].z, v1[k].w};
            const uint32_t rw[4] = {rq[k].x, rq[k].y, rq[k].z, rq[k].w};
            float dg[8], dv[8];
            float dot = 0.f;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const float sg = 1.0f / (1.0f + expf(-g[q]));
              dg[q] = da[q] * vu[q] * sg * (1.0f + g[q] * (1.0f - sg));
              dv[q] = da[q] * g[q] * sg;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              dot += da[2 * q] * __uint_as_float(rw[q] << 16);
              dot += da[2 * q + 1] * __uint_as_float(rw[q] & 0xffff0000u);
            }
            store_row8_bf16((bf16_t*)DG + o, dg, 8, true);
            store_row8_bf16((bf16_t*)DV + o, dv, 8, true);
            dot = row16_sum(dot);
            if (cdot && (p.tid % TPR) == 0) cdot[(int64_t)p.tn * ldc + m0 + r] = dot;
          }
        }
        return;
      }
    }
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
    row_partial_store<FM>(p, dots, cdot, ldc);
  }
};

// Weight gradient: store G in the GEMM operand precision (bf16 tiles through LDS, 16-byte
// row stores; fp32 directly) and this tile's sum of squares of the fp32 accumulators into
// slot[tile] (the clip norm never sees the rounding of the stored G).
template <class T>
struct EpiGrad {
  T* G;
  int64_t ldg;
  float* slot;
  template <int FM, int FN, int WGM, int WGN>
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
          if (epi_col(p, j) >= p.N) continue;
          const float v = acc[i][j][e];
          ss += v * v;
        }
      }
    ss = wave_sum(ss);
    float* red = (float*)p.smem;
    if (p.lane == 0) red[p.wave] = ss;
    __syncthreads();
    if (p.wave == 0 && p.lane == 0) {
      float t = red[0];
      for (int w = 1; w < p.wgm * p.wgn; ++w) t += red[w];
      slot[p.tile] = t;
    }
    if constexpr (sizeof(T) == 2 && TileGeo<FM, FN, WGM, WGN>::ROWS_FIT) {
      Packed<FM, FN> pg;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          pg[i][j][0] = pack_bf2(acc[i][j][0], acc[i][j][1]);
          pg[i][j][1] = pack_bf2(acc[i][j][2], acc[i][j][3]);
        }
      stage_rows_bf16<FM, FN, WGM, WGN>(p, pg, (bf16_t*)G, ldg);  // begins with a barrier
      return;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = epi_row(p, i, e);
        if (row >= p.M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = epi_col(p, j);
          if (col < p.N) G[(int64_t)row * ldg + col] = from_f<T>(acc[i][j][e]);
        }
      }
  }
};

// Plain store in the GEMM operand precision (bf16 tiles through LDS as 16-byte row pieces).
template <class T>
struct EpiStoreT {
  T* C;
  int64_t ldc;
  template <int FM, int FN, int WGM, int WGN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
    if constexpr (sizeof(T) == 2 && TileGeo<FM, FN, WGM, WGN>::ROWS_FIT) {
      Packed<FM, FN> pc;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          pc[i][j][0] = pack_bf2(acc[i][j][0], acc[i][j][1]);
          pc[i][j][1] = pack_bf2(acc[i][j][2], acc[i][j][3]);
        }
      stage_rows_bf16<FM, FN, WGM, WGN>(p, pc, (bf16_t*)C, ldc);
      return;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = epi_row(p, i, e);
        if (row >= p.M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = epi_col(p, j);
          if (col < p.N) C[(int64_t)row * ldc + col] = from_f<T>(acc[i][j][e]);
        }
      }
  }
};

// The product in two 16-bit forms: Ch = rn_bf16(C) for products that take bf16 operands, and
// Cf = rn_f16(C) (11 significant bits) for products that read it in half precision.
struct EpiStoreBf16F16 {
  bf16_t* Ch;
  f16_t* Cf;
  int64_t ldc;
  template <int FM, int FN, int WGM, int WGN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
    // each form staged through LDS as whole rows (16-byte stores); direct stores otherwise
    Packed<FM, FN> h, f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        h[i][j][0] = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        h[i][j][1] = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        f[i][j][0] = pack_f16x2(acc[i][j][0], acc[i][j][1]);
        f[i][j][1] = pack_f16x2(acc[i][j][2], acc[i][j][3]);
      }
    if (stage_rows_bf16<FM, FN, WGM, WGN>(p, h, Ch, ldc) && stage_rows_bf16<FM, FN, WGM, WGN>(p, f, Cf, ldc)) return;
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
          Ch[(int64_t)row * ldc + col] = f2bf(v);
          Cf[(int64_t)row * ldc + col] = f2h(v);
        }
      }
  }
};

// Merge two online-softmax partials (max logit, sum of exp(z - max), first argmax) of
// disjoint column sets; an empty partial is (-inf, 0, any index).
__device__ __forceinline__ void ce_combine(float& mx, float& sm, int& ix, float omx, float osm, int oix) {
  const float nm = fmaxf(mx, omx);
  const float a = (mx == -INFINITY) ? 0.f : sm * __builtin_amdgcn_exp2f((mx - nm) * 1.4426950408889634f);
  const float b = (omx == -INFINITY) ? 0.f : osm * __builtin_amdgcn_exp2f((omx - nm) * 1.4426950408889634f);
  if (omx > mx || (omx == mx && oix < ix)) ix = oix;
  mx = nm;
  sm = a + b;
}

// LM head + online-softmax partials over the full vocabulary, one record per row and per
// column wave (the wave's WTN consecutive vocabulary entries, record index = column / WTN):
// max logit, sum of exp(z - max) and first argmax; the target logit is stored by the one
// lane whose column is the row's target. With Q, also every softmax numerator relative to
// its record's max, Q[t, v] = exp(z - max), in the GEMM operand precision (missing columns
// contribute nothing).
template <class T>
struct EpiCEPartial {
  // 256 x 256 tiles (2 x 4 waves of 128 x 64, the same 64-column records): measured 132.4
  // against 151.6 us at 1024 x 32000 x 1536 and 469 against 535 us at 512 x 151936 x 2560
  static constexpr bool kSquareTiles = true;
  const int* tgt;    // [M] target ids
  float* pmax;       // [M x nrec]
  float* psum;
  int* pidx;
  float* tgt_logit;  // [M]
  int nrec;
  T* Q;              // [M x ldq] or null
  int64_t ldq;
  template <int FM, int FN, int WGM, int WGN>
  __device__ __forceinline__ void apply(const EpiPos& p, f32x4_t (&acc)[FM][FN]) const {
    constexpr float L2E = 1.4426950408889634f;
    const int lc = p.col0 + (p.lane & 15);      // this lane's columns: lc + 16 j
    const bool full = p.col0 + 16 * FN <= p.N;  // wave-uniform: every column of the wave exists
    const int rec = p.col0 / (16 * FN);
    // all target ids first: independent loads in flight together
    int tgs[FM][4];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) tgs[i][e] = tgt[min(epi_row(p, i, e), p.M - 1)];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = epi_row(p, i, e);
        const int tg = row < p.M ? tgs[i][e] : -1;
        // this lane's values (missing columns as -inf), max and first argmax
        float v[FN];
        float mx = -INFINITY;
        int jx = 0;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          v[j] = (full || lc + 16 * j < p.N) ? acc[i][j][e] : -INFINITY;
          jx = v[j] > mx ? j : jx;
          mx = fmaxf(mx, v[j]);
        }
        int ix = mx == -INFINITY ? 0x7fffffff : lc + 16 * jx;
        // the target logit, if one of this lane's columns is the target
        const int jt = tg - lc;
        const bool hit = jt >= 0 && jt < 16 * FN && (jt & 15) == 0;
        float tv = v[0];
#pragma unroll
        for (int j = 1; j < FN; ++j) tv = (jt >> 4) == j ? v[j] : tv;
        // row max and first argmax over the 16 lanes of the row, then one exp per element
        row16_max_argmax(mx, ix);
        const float nm = mx == -INFINITY ? 0.f : -mx * L2E;
        float sm = 0.f;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const float q = __builtin_amdgcn_exp2f(fmaf(v[j], L2E, nm));
          sm += q;
          acc[i][j][e] = q;
        }
        sm = row16_sum(sm);
        if (hit) tgt_logit[row] = tv;
        if ((p.lane & 15) == 0 && row < p.M && p.col0 < p.N) {
          const int64_t o = (int64_t)row * nrec + rec;
          pmax[o] = mx;
          psum[o] = sm;
          pidx[o] = ix;
        }
      }
    if (!Q) return;
    if constexpr (sizeof(T) == 2) {
      Packed<FM, FN> qq;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          qq[i][j][0] = pack_bf2(acc[i][j][0], acc[i][j][1]);
          qq[i][j][1] = pack_bf2(acc[i][j][2], acc[i][j][3]);
        }
      if (stage_rows_bf16<FM, FN, WGM, WGN>(p, qq, (bf16_t*)Q, ldq)) return;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = epi_row(p, i, e);
        if (row >= p.M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = epi_col(p, j);
          if (col < p.N) Q[(int64_t)row * ldq + col] = from_f<T>(acc[i][j][e]);
        }
      }
  }
};

// Epilogues that handle 256 x 256 tiles well (their per-wave work does not depend on the
// tile fitting an fp32 LDS staging area) declare kSquareTiles = true.
template <class E, class = void>
struct SquareTiles : std::false_type {};
template <class E>
struct SquareTiles<E, std::void_t<decltype(E::kSquareTiles)>> : std::bool_constant<E::kSquareTiles> {};

// ------------------------------------------------------------------------- launcher
// Second K-segment of a GEMM (absent when K2 == 0).
struct Seg2 {
  const void* X = nullptr;
  int64_t ldx = 0;
  const void* Y = nullptr;
  int64_t ldy = 0;
  int K = 0;
  int share = -1;  // shared-X form over the same X rows: -1 by the plan's rule, 0 never, 1 where the tile allows
};

// n products of one shape in one launch (see GemmArgs): per-product operand offsets in
// elements, and the tile-id stride of their epilogues.
struct Group {
  int n = 1;
  int64_t x = 0, y = 0, x2 = 0, y2 = 0;
  int tile = 0;
};

template <class T, int BM, int BN, int WGM, int WGN, class Epi, int NB = 1>
inline hipError_t launch_dma(hipStream_t st, const GemmArgs& g, int splits, int groups, const Epi& epi) {
  constexpr size_t lds = (size_t)gemm_lds_bytes(BM, BN, NB);
  auto kern = gemm_dma_kernel<T, BM, BN, WGM, WGN, Epi, NB>;
  static bool lds_attr = false;  // per instantiation
  if (!lds_attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_attr = true;
  }
  dim3 grid(g.tiles_m * g.tiles_n, splits, groups);
  hipLaunchKernelGGL(kern, grid, dim3(WGM * WGN * 64), lds, st, g, epi);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, class Epi>
inline hipError_t launch_km(hipStream_t st, const GemmArgs& g, int groups, const Epi& epi) {
  constexpr int STAGE = 64 * 2 * (BM + BN);
  constexpr size_t lds = (size_t)gemm_stages(BM, BN) * STAGE;
  auto kern = gemm_km_kernel<BM, BN, WGM, WGN, Epi>;
  static bool lds_attr = false;  // per instantiation
  if (!lds_attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_attr = true;
  }
  dim3 grid(g.tiles_m * g.tiles_n, 1, groups);
  hipLaunchKernelGGL(kern, grid, dim3(WGM * WGN * 64), lds, st, g, epi);
  return hipGetLastError();
}

// Tile plan of a GEMM launch (shared with the host code that sizes per-tile buffers and
// picks split-K factors). slots = workgroups the chip runs at once for that tile.
struct TilePlan {
  int bm, bn;
  bool dma;
  int slots;
  int wtn;  // columns of one wave's sub-tile
};
inline TilePlan gemm_plan(int M, int N, int K, int K2, int es, int splits, int groups = 1) {
  const int ke = 128 / es;
  const bool dma = (K % ke == 0) && (K2 % ke == 0);
  const int tiles256 = ((M + 255) / 256) * ((N + 255) / 256);
  if (dma && es == 2) {
    // measured per shape at b = 1024: split-K, the wide-N up / dA GEMMs and the LM head
    // run best on 256 x 128 tiles (32 x 32 blocks, 3 stages). Short-K GEMMs (the weight
    // gradients) take 128 x 128 tiles (two per CU) or 192 x 192 (one per CU, 32 x 32 blocks),
    // whichever leaves fewer outputs per CU over its rounds of workgroups.
    if (splits <= 1 && K + K2 <= 1024) {
      const int64_t t128 = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
      const int64_t t192 = (int64_t)((M + 191) / 192) * ((N + 191) / 192);
      const int64_t load128 = (t128 + 511) / 512 * (2 * 128 * 128), load192 = (t192 + 255) / 256 * (192 * 192);
      if (load192 < load128) return TilePlan{192, 192, true, 256, 96};
      return TilePlan{128, 128, true, 512, 64};
    }
    if (splits <= 1) {
      // A long-K product whose 256 x 64 tiles (all groups) still fit one round of one
      // workgroup per CU, i.e. whose 256 x 128 tiles would leave at least half the CUs idle,
      // takes them: measured 35.4 against 41.7 us alone at 1024 x 3072 x 3072, and the 760M
      // fuller-block step 87.8 against 91.9 ms. (128 x 192 tiles for the 760M up and dA
      // products, 256 tiles each, measured faster alone, 44.5 against 47.1 us, but 0.5%
      // slower over the step.)
      const int64_t g = groups < 1 ? 1 : groups;
      if ((int64_t)((M + 255) / 256) * ((N + 63) / 64) * g <= 256) return TilePlan{256, 64, true, 256, 32};
    }
    return TilePlan{256, 128, true, 256, 64};
  }
  TilePlan t{128, 128, dma, 512, 64};  // 4 waves, 2 stages, 2 per CU
  if (t.dma && splits <= 1 && tiles256 >= 256) t = TilePlan{256, 256, true, 256, 64};
  return t;
}

// A second segment over the same X rows (same pointer, stride, K and per-product offset):
// the product is X (Y + Y2)^T and the shared-X form applies.
inline bool shared_x(const void* X, int64_t ldx, int K, const Seg2& s2, const Group& gr) {
  return s2.share != 0 && s2.K == K && s2.X == X && s2.ldx == ldx && gr.x2 == gr.x && K > 0;
}

// C = X Y^T (+ X2 Y2^T) with a fused epilogue. K-slices of 128 bytes go through LDS by
// direct loads when both K extents are whole slices, else through registers. Wide outputs
// (at least one 256 x 256 tile per CU) use 256 x 256 tiles with 8 waves; the rest 128 x 128.
template <class T, class Epi>
inline hipError_t launch_gemm(hipStream_t st, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                              int K, int splits, const Epi& epi, const Seg2& s2 = Seg2(),
                              const Group& gr = Group()) {
  if (M <= 0 || N <= 0 || gr.n <= 0) return hipSuccess;
  if (gr.n > 65535) return hipErrorInvalidValue;
  constexpr int KE = 128 / (int)sizeof(T);
  if (splits < 1) splits = 1;
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
  g.kit_a = (K + KE - 1) / KE;
  g.kiters = g.kit_a + (s2.K + KE - 1) / KE;
  g.gx = gr.x;
  g.gy = gr.y;
  g.gx2 = s2.K > 0 ? gr.x2 : 0;
  g.gy2 = s2.K > 0 ? gr.y2 : 0;
  g.gtile = gr.tile;
  const TilePlan plan = gemm_plan(M, N, K, s2.K, (int)sizeof(T), splits, gr.n);
  if (plan.dma) {
    if constexpr (sizeof(T) == 2) {
      if constexpr (SquareTiles<Epi>::value) {
        // a long-K product with at least one full round of 256 x 256 tiles: half the operand
        // bytes per flop of the 256 x 128 tile (2 stages of 64 KB, 16 x 16 MFMA blocks)
        const int64_t t256 = (int64_t)((M + 255) / 256) * ((N + 255) / 256) * gr.n;
        if (plan.bm == 256 && plan.bn == 128 && splits <= 1 && t256 >= 256) {
          g.tiles_m = (M + 255) / 256;
          g.tiles_n = (N + 255) / 256;
          g.kps = g.kiters;
          return launch_dma<T, 256, 256, 2, 4>(st, g, 1, gr.n, epi);
        }
      }
      if (plan.bm == 256 && plan.bn == 128) {
        g.tiles_m = (M + 255) / 256;
        g.tiles_n = (N + 127) / 128;
        // the shared-X form of this tile has two stages only; measured alone it is slower than the
        // concatenated walk at every split-K and wide-N product of the workloads (1024 x 6144 x
        // 1536 x 2: 56.7 against 47.3 us; 1024 x 1536 x 6144 x 2 in 5 slabs: 50.6 against 43.3)
        // and faster only over a long single slab, so it is used here only when asked for
        if (s2.share == 1 && shared_x(X, ldx, K, s2, gr)) {
          g.kiters = g.kit_a;
          g.kps = (g.kiters + splits - 1) / splits;
          return launch_dma<T, 256, 128, 4, 2, Epi, 2>(st, g, splits, gr.n, epi);
        }
        g.kps = (g.kiters + splits - 1) / splits;
        return launch_dma<T, 256, 128, 4, 2>(st, g, splits, gr.n, epi);
      }
      if (plan.bm == 192) {
        g.tiles_m = (M + 191) / 192;
        g.tiles_n = (N + 191) / 192;
        g.kps = (g.kiters + splits - 1) / splits;
        return launch_dma<T, 192, 192, 2, 2>(st, g, splits, gr.n, epi);
      }
      if (plan.bm == 256 && plan.bn == 64) {
        g.tiles_m = (M + 255) / 256;
        g.tiles_n = (N + 63) / 64;
        if (shared_x(X, ldx, K, s2, gr)) {
          // the second segment reads the same X rows: one X slice per pair of weight slices,
          // three stages (measured 18.1 against 20.5 us at 1024 x 3072 x 768 x 2, 28.7 against
          // 34.0 at 1024 x 3072 x 1536 x 2)
          g.kiters = g.kit_a;
          g.kps = g.kiters;
          return launch_dma<T, 256, 64, 4, 2, Epi, 2>(st, g, 1, gr.n, epi);
        }
        g.kps = g.kiters;
        return launch_dma<T, 256, 64, 4, 2>(st, g, 1, gr.n, epi);
      }
    }
    if constexpr (sizeof(T) == 4) {
      if (plan.bm == 256) {
        g.tiles_m = (M + 255) / 256;
        g.tiles_n = (N + 255) / 256;
        g.kps = g.kiters;
        return launch_dma<T, 256, 256, 2, 4>(st, g, 1, gr.n, epi);
      }
    }
    {
      g.tiles_m = (M + 127) / 128;
      g.tiles_n = (N + 127) / 128;
      g.kps = (g.kiters + splits - 1) / splits;
      return launch_dma<T, 128, 128, 2, 2>(st, g, splits, gr.n, epi);
    }
  }
  g.tiles_m = (M + 127) / 128;
  g.tiles_n = (N + 127) / 128;
  g.kps = (g.kiters + splits - 1) / splits;
  dim3 grid(g.tiles_m * g.tiles_n, splits, gr.n);
  hipLaunchKernelGGL((gemm_reg_kernel<T, 128, 128, Epi>), grid, dim3(256), 0, st, g, epi);
  return hipGetLastError();
}
