// Instantiations of the MFMA GEMM core with the inner loop's fused epilogues.
#include "launchers.h"
#include "gemm.h"

namespace {
constexpr int BM = 128, BN = 128;
}

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

hipError_t gemm_f32(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                    int K, int splits, float* C, int64_t ldc, int64_t split_stride, int accumulate) {
  EpiStoreF32 e{C, ldc, split_stride, accumulate};
  DISPATCH_T(prec, return (launch_gemm<T, BM, BN>(st, X, ldx, Y, ldy, M, N, K, splits, e)));
}

hipError_t gemm_gelu(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                     int K, void* A, void* AT, void* GP, int64_t lda, int64_t ldat) {
  DISPATCH_T(prec, {
    EpiGelu<T> e{(T*)A, (T*)AT, (T*)GP, lda, ldat};
    return launch_gemm<T, BM, BN>(st, X, ldx, Y, ldy, M, N, K, 1, e);
  });
}

hipError_t gemm_swiglu(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                       int K, const float* UG, void* A, void* AT, int64_t lda, int64_t ldat) {
  DISPATCH_T(prec, {
    EpiSwiglu<T> e{UG, (T*)A, (T*)AT, lda, ldat};
    return launch_gemm<T, BM, BN>(st, X, ldx, Y, ldy, M, N, K, 1, e);
  });
}

hipError_t gemm_du(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                   int K, const void* GP, void* DU, void* DUT, int64_t ld, int64_t ldt) {
  DISPATCH_T(prec, {
    EpiDU<T> e{(const T*)GP, (T*)DU, (T*)DUT, ld, ldt};
    return launch_gemm<T, BM, BN>(st, X, ldx, Y, ldy, M, N, K, 1, e);
  });
}

int gemm_grad_slots(int M, int N) { return ((M + BM - 1) / BM) * ((N + BN - 1) / BN); }

hipError_t gemm_grad(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                     int K, float* G, int64_t ldg, float* slot) {
  EpiGrad e{G, ldg, slot};
  DISPATCH_T(prec, return (launch_gemm<T, BM, BN>(st, X, ldx, Y, ldy, M, N, K, 1, e)));
}

hipError_t gemm_ce_partial(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M,
                           int N, int K, const int* tgt, float* pmax, float* psum, int* pidx, float* tgt_logit) {
  static_assert(BN == GEMM_CE_BN, "CE partial tiles must match the merge");
  EpiCEPartial e{tgt, pmax, psum, pidx, tgt_logit, M};
  DISPATCH_T(prec, return (launch_gemm<T, BM, BN>(st, X, ldx, Y, ldy, M, N, K, 1, e)));
}

hipError_t gemm_ce_prob(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M,
                        int N, int K, const int* tgt, const float* lse, void* P, int64_t ldp, int col_base,
                        float inv_b) {
  DISPATCH_T(prec, {
    EpiCEProb<T> e{tgt, lse, (T*)P, ldp, col_base, inv_b};
    return launch_gemm<T, BM, BN>(st, X, ldx, Y, ldy, M, N, K, 1, e);
  });
}
