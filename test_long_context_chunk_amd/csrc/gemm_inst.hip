// Instantiations of the MFMA GEMM core with the inner loop's fused epilogues.
#include "launchers.h"
#include "gemm.h"


#define DISPATCH_T(prec, ...)  \
  do {                         \
    if ((prec) == PREC_BF16) { \
      using T = bf16_t;        \
      __VA_ARGS__;             \
    } else {                   \
      using T = float;         \
      __VA_ARGS__;             \
    }                          \
  } while (0)

namespace {
inline Group grp(const GemmGroup& g) {
  Group r;
  r.n = g.n;
  r.x = g.x;
  r.y = g.y;
  r.x2 = g.x2;
  r.y2 = g.y2;
  r.tile = g.tile;
  return r;
}
inline Seg2 seg(const GemmSeg2& s) {
  Seg2 r;
  r.X = s.X;
  r.ldx = s.ldx;
  r.Y = s.Y;
  r.ldy = s.ldy;
  r.K = s.K;
  r.share = s.share;
  return r;
}
}  // namespace

hipError_t gemm_f32(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                    int K, int splits, float* C, int64_t ldc, int64_t split_stride, int accumulate,
                    const GemmSeg2& s2, const GemmGroup& gg) {
  EpiStoreF32 e{C, ldc, split_stride, accumulate};
  DISPATCH_T(prec, return (launch_gemm<T>(st, X, ldx, Y, ldy, M, N, K, splits, e, seg(s2), grp(gg))));
}

hipError_t gemm_gelu(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                     int K, void* A, void* AT, void* GP, void* RES, int64_t lda, int64_t ldat, const GemmSeg2& s2,
                     const GemmGroup& gg, const float* add) {
  DISPATCH_T(prec, {
    EpiGelu<T> e{(T*)A, (T*)AT, (T*)GP, (T*)RES, lda, ldat, add};
    return launch_gemm<T>(st, X, ldx, Y, ldy, M, N, K, 1, e, seg(s2), grp(gg));
  });
}

hipError_t gemm_swiglu(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                       int K, const float* UG, float* VU, void* A, void* AT, void* RES, int64_t lda, int64_t ldat) {
  DISPATCH_T(prec, {
    EpiSwiglu<T> e{UG, VU, (T*)A, (T*)AT, (T*)RES, lda, ldat};
    return launch_gemm<T>(st, X, ldx, Y, ldy, M, N, K, 1, e);
  });
}

hipError_t gemm_du(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                   int K, const void* GP, void* DU, void* DUT, const void* RES, float* cdot, int64_t ld, int64_t ldt,
                   int64_t ldc, const GemmGroup& gg) {
  DISPATCH_T(prec, {
    EpiDU<T> e{(const T*)GP, (T*)DU, (T*)DUT, (const T*)RES, cdot, ld, ldt, ldc};
    return launch_gemm<T>(st, X, ldx, Y, ldy, M, N, K, 1, e, Seg2(), grp(gg));
  });
}

hipError_t gemm_swiglu_bwd(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M,
                           int N, int K, const float* UG, const float* VU, void* DG, void* DV, const void* RES,
                           float* cdot, int64_t ld, int64_t ldc, const GemmGroup& gg) {
  DISPATCH_T(prec, {
    EpiSwigluBwd<T> e{UG, VU, (T*)DG, (T*)DV, (const T*)RES, cdot, ld, ldc};
    return launch_gemm<T>(st, X, ldx, Y, ldy, M, N, K, 1, e, Seg2(), grp(gg));
  });
}

hipError_t gemm_store(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                      int K, void* C, int64_t ldc) {
  DISPATCH_T(prec, {
    EpiStoreT<T> e{(T*)C, ldc};
    return launch_gemm<T>(st, X, ldx, Y, ldy, M, N, K, 1, e);
  });
}

hipError_t gemm_store_bf16_f16(hipStream_t st, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                              int K, void* Ch, void* Cf, int64_t ldc, const GemmSeg2& s2) {
  EpiStoreBf16F16 e{(bf16_t*)Ch, (f16_t*)Cf, ldc};
  return launch_gemm<bf16_t>(st, X, ldx, Y, ldy, M, N, K, 1, e, seg(s2));
}

int gemm_split_k(int prec, int M, int N, int K, int K2, int max_splits) {
  const int es = prec == PREC_BF16 ? 2 : 4;
  const TilePlan t = gemm_plan(M, N, K, K2, es, 2);
  const int tiles = ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
  const int kiters = (K + K2) / (128 / es);
  int s = t.slots / tiles;
  if (s > kiters / 4) s = kiters / 4;
  if (s > max_splits) s = max_splits;
  return s < 1 ? 1 : s;
}

void gemm_tile_shape(int prec, int M, int N, int K, int K2, int splits, int* tile_m, int* tile_n, int groups) {
  const TilePlan t = gemm_plan(M, N, K, K2, prec == PREC_BF16 ? 2 : 4, splits, groups);
  *tile_m = t.bm;
  *tile_n = t.bn;
}

int gemm_wave_cols(int prec, int M, int N, int K, int K2, int splits, int groups) {
  const TilePlan t = gemm_plan(M, N, K, K2, prec == PREC_BF16 ? 2 : 4, splits, groups);
  return t.dma ? t.wtn : 64;  // the register-staged kernel: 2 x 2 waves of a 128 x 128 tile
}

hipError_t gemm_grad(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                     int K, void* G, int64_t ldg, float* slot, const GemmGroup& gg) {
  DISPATCH_T(prec, {
    EpiGrad<T> e{(T*)G, ldg, slot};
    return launch_gemm<T>(st, X, ldx, Y, ldy, M, N, K, 1, e, Seg2(), grp(gg));
  });
}

hipError_t gemm_grad_km(hipStream_t st, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N, int K,
                        void* G, int64_t ldg, float* slot, const GemmGroup& gg) {
  if (M <= 0 || N <= 0 || gg.n <= 0) return hipSuccess;
  if (K <= 0 || K % 64 || M % 8 || N % 8 || gg.n > 65535) return hipErrorInvalidValue;
  EpiGrad<bf16_t> e{(bf16_t*)G, ldg, slot};
  GemmArgs g{};
  g.X = X;
  g.Y = Y;
  g.ldx = ldx;
  g.ldy = ldy;
  g.M = M;
  g.N = N;
  g.K = K;
  g.kit_a = g.kiters = g.kps = K / 64;
  g.gx = gg.x;
  g.gy = gg.y;
  g.gtile = gg.tile;
  // the same output tiles as the row-major path (per-tile slots are sized from them)
  const TilePlan t = gemm_plan(M, N, K, 0, 2, 1);
  if (t.bm == 192 && t.bn == 192) {
    g.tiles_m = (M + 191) / 192;
    g.tiles_n = (N + 191) / 192;
    return launch_km<192, 192, 2, 2>(st, g, gg.n, e);
  }
  if (t.bm == 128 && t.bn == 128) {
    g.tiles_m = (M + 127) / 128;
    g.tiles_n = (N + 127) / 128;
    return launch_km<128, 128, 2, 2>(st, g, gg.n, e);
  }
  return hipErrorInvalidValue;
}

hipError_t gemm_ce_partial(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M,
                           int N, int K, const int* tgt, float* pmax, float* psum, int* pidx, float* tgt_logit,
                           int nrec, void* Q, int64_t ldq, const GemmSeg2& s2) {
  DISPATCH_T(prec, {
    EpiCEPartial<T> e{tgt, pmax, psum, pidx, tgt_logit, nrec, (T*)Q, ldq};
    return launch_gemm<T>(st, X, ldx, Y, ldy, M, N, K, 1, e, seg(s2));
  });
}
