// Host-side launchers of the TTT inner-loop kernels. Every launcher enqueues on `st` and
// returns the launch status; `prec` is PREC_FP32 or PREC_BF16 and selects the element type
// of the GEMM-operand buffers (void* below). fp32 buffers are typed float*.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

enum { PREC_FP32 = 0, PREC_BF16 = 1 };

// Rows of a chunk step that stacks several independent streams: row t is position t % bs of
// stream t / bs; that stream's per-token records (token ids, losses, argmax) start at
// (t / bs) * ld. One stream: bs = rows, ld unused.
struct StreamRows {
  int bs;
  int64_t ld;
};

// ---- row / elementwise kernels (kernels.hip)
// The residual stream entering a block (gather of the embeddings when tokens is non-null,
// else H + the split-K slabs part) and, when Hn is non-null, its pre-norm (see k_row_in).
// Yl (with Yb): the rounding residual rn(h - rn(h)) of the LM head's operand.
hipError_t run_row_in(hipStream_t st, int prec, const int* tokens, StreamRows sr, int V, const void* E, int* tok_prev,
                      int* tok_tgt, int* err, const float* part, int S, int64_t pstride, float* H, int b, int d, void* Yb,
                      float eps, int rms, void* Hn, float* r, void* RES, void* Yl = nullptr);
hipError_t run_transpose(hipStream_t st, int prec, const void* src, int64_t lds, int R, int C, void* dst, int64_t ldd);
hipError_t run_dy_finish(hipStream_t st, int prec, const float* part, int S, int64_t pstride, int b, int d,
                         float* dH, void* dHb, const float* Hres, const void* Yb, float* cdot);
hipError_t run_loss_correct(hipStream_t st, const float* cpart, int nslot, int b, StreamRows sr, float scale,
                            float* loss);
hipError_t run_ce_merge(hipStream_t st, const float* pmax, const float* psum, const int* pidx, int nrec, int b,
                        StreamRows sr, const float* tgt_logit, float* lse, float* loss, int* amax);
// dlogits in place: Q [b x V] (numerators relative to record max pmax[t][v / W]) becomes
// P = (Q exp(pmax - lse) - onehot(target)) / b.
hipError_t run_ce_dlogits(hipStream_t st, int prec, void* Q, int b, int V, int W, const float* pmax, int nrec,
                          const float* lse, const int* tgt, float inv_b);
hipError_t run_norm_bwd(hipStream_t st, int prec, const float* part, int S, int64_t pstride, const void* Hn,
                        const float* r, int b, int d, int rms, float* dH, void* dHb, const void* RES, float* cdot,
                        int update_dh);
// One clip scale per stream: stream z reads slot[z nslot ..], writes sc[4 z ..], stat[z stat_ld ..].
hipError_t run_gradnorm(hipStream_t st, const float* slot, int nslot, float clip, float* sc, float* stat,
                        int64_t stat_ld, int streams, int* err);
// One fast tensor of every stream: G, D, Wop, WtT of stream z lie R C elements apart, W0 is shared.
hipError_t run_update(hipStream_t st, int prec, const void* G, float* D, const void* W0, void* Wop, void* WtT, int R,
                      int C, float lr, const float* sc, int delta_t, int streams);
hipError_t run_export(hipStream_t st, int prec, const float* D, const void* W0, int64_t n, int kind, float* dst);
hipError_t run_fill_u32(hipStream_t st, void* p, int64_t n, uint32_t v);

// ---- decode (kernels.hip): one activation row, fp32 activations
enum { GEMV_STORE = 0, GEMV_GELU = 1, GEMV_RESIDUAL = 2, GEMV_SWIGLU = 3 };
// How a decode product builds its activation row x (see k_gemv): from xin, or by the gather
// of tok[0] from E (then H, pend and err are written as the gather's side effects); then the
// pre-norm when norm is set.
struct GemvIn {
  const float* xin = nullptr;
  const int* tok = nullptr;
  int first = 0;
  int* pend = nullptr;
  const void* E = nullptr;
  int V = 0;
  float* H = nullptr;
  int* err = nullptr;
  int norm = 0;
  float eps = 0.f;
  // STORE only: one online-softmax record per block of gemv_rec_rows(N) outputs
  float* rmax = nullptr;
  float* rsum = nullptr;
  int* ridx = nullptr;
};
// Outputs per record of a STORE product with records (the records number ceil(N / that)).
inline int gemv_rec_rows(int N) { return N >= 16384 ? 16 : 4; }
// out[n] (mode) x . Y[n] (+ x . Y2[n]); Y [N x K] row stride ldy in the operand precision.
hipError_t run_gemv(hipStream_t st, int prec, int mode, const GemvIn& in, int K, const void* Y, const void* Y2,
                    int64_t ldy, int N, float* out);
// lse, first argmax and loss = lse - z[*tgt] of one logits row from the product's records;
// records loss[0], amax[0] (and argmax_out[0] when non-null).
hipError_t run_dec_ce(hipStream_t st, const float* z, int V, const float* rmax, const float* rsum, const int* ridx,
                      int nrec, const int* tgt, float* loss, int* amax, int* argmax_out);

// ---- evaluation and Settlement (kernels.hip)
// acc[0] (fp64) += sum of n losses (zeroed first when first); out <- losses when non-null; when
// last, mean[0] = acc[0] / count (when mean is non-null).
hipError_t run_eval_accum(hipStream_t st, const float* loss, int n, double* acc, float* out, int first, int last,
                          int64_t count, float* mean);
// A = (sums[0] - sums[1]) / count, commit = A >= 0; also into A_out / commit_out when non-null.
hipError_t run_settle_decide(hipStream_t st, const double* sums, int64_t count, float* A, int* commit, float* A_out,
                             int* commit_out);
// dst <- src (bytes, a multiple of 16) unless *commit.
hipError_t run_restore_unless(hipStream_t st, const int* commit, const void* src, void* dst, int64_t bytes);

// ---- sliding-window attention (attention.hip), bf16, heads of 128
// One chunk step of `streams` streams: qkv [streams b x 3d] holds the chunk's q | k | v
// (stream z: rows z b ..); kc, vc [streams][cr x d] the ring of earlier keys and values
// (position p at slot p % cr, cr >= window - 1); pos the position of the chunk's first row.
// Each of q, k, v is held twice: bf16 (qkv, kc, vc), read by the backward, and half precision
// (qkv16, kc16, vc16: 11 significant bits), read by the forward and by decode.
struct SwaShape {
  const void* qkv = nullptr;
  const void* qkv16 = nullptr;
  void* kc = nullptr;
  void* vc = nullptr;
  void* kc16 = nullptr;
  void* vc16 = nullptr;
  int cr = 0, b = 0, d = 0, window = 0, streams = 1;
  int64_t pos = 0;
};
// O (fp32 Of, bf16 Ob and its rounding residual Ol, [streams b x d]) and lse2
// [streams][d / 128][b]. When swa_fwd_splits(s) > 1 the key range of each query block is
// shared by that many workgroups, whose partial states (part [n][streams b x d], pm and pl
// [n][streams][d / 128][b], scratch) a merge combines.
int swa_fwd_splits(const SwaShape& s);
// Workgroups per query block of the dQ pass (its partial dQ take part [splits][R x d]).
int swa_dq_splits(const SwaShape& s);
// Workgroups per key block of the dK, dV pass (partials take part [2 splits][R x d]).
int swa_dkdv_splits(const SwaShape& s);
hipError_t run_swa_fwd(hipStream_t st, const SwaShape& s, float* Of, void* Ob, void* Ol, float* lse2, float* part,
                       float* pm, float* pl);
// From dO (fp32 dOf for the row term D, bf16 dOb for the products): dQ, dK, dV of the
// chunk's rows (bf16) into dQKV [streams b x 3d], in three parts: the row term Dq
// [streams][d / 128][b] from dOf and Of; then dQ (part: its split partials,
// [swa_dq_splits(s)][streams b x d] fp32) and dK, dV (part: theirs, [2 swa_dkdv_splits(s)]
// [streams b x d]). The last two read only dOb, lse2, Dq and the forward's q, k, v, write
// disjoint columns of dQKV, and may run at once (two streams) when their part buffers differ.
hipError_t run_swa_dsum(hipStream_t st, const SwaShape& s, const float* dOf, const float* Of, float* Dq);
hipError_t run_swa_bwd_dq(hipStream_t st, const SwaShape& s, const void* dOb, const float* lse2, const float* Dq,
                          void* dQKV, float* part);
hipError_t run_swa_bwd_dkdv(hipStream_t st, const SwaShape& s, const void* dOb, const float* lse2, const float* Dq,
                            void* dQKV, float* part);
// Decode of one row at position s.pos (single stream): its key and value (fp32 qkv [3d]) join
// the ring, and o [d] (fp32) = its attention over the window; part is scratch of
// d / 128 * swa_dec_splits(window) * 130 floats.
int swa_dec_splits(int window);
hipError_t run_swa_decode(hipStream_t st, const SwaShape& s, const float* qkv, float* part, float* o);
// The chunk's keys and values (its last min(b, cr), cr being at least b) into the ring.
hipError_t run_kv_append(hipStream_t st, const SwaShape& s);

// ---- GEMMs, C = X Y^T with X [M x K], Y [N x K] (gemm_inst.hip)
// Optional second K-segment of a GEMM: C = X Y^T + X2 Y2^T (K2 = 0: absent).
struct GemmSeg2 {
  const void* X = nullptr;
  int64_t ldx = 0;
  const void* Y = nullptr;
  int64_t ldy = 0;
  int K = 0;
  int share = -1;  // over the same X rows: -1 the plan's choice of form, 0 the concatenated walk, 1 shared-X
};

// n independent products of one shape in one launch. Product z reads X, Y, X2, Y2 at
// z * (x, y, x2, y2) elements past the given pointers (0: one operand shared by all), and
// writes its outputs as rows z * M .. z * M + M - 1 of outputs stacked over the products
// (so every output pointer and leading dimension below describes the stacked [n M x ...]
// array, and transposed outputs hold product z in columns z * M ..); per-tile slots of
// product z start at z * tile.
struct GemmGroup {
  int n = 1;
  int64_t x = 0, y = 0, x2 = 0, y2 = 0;
  int tile = 0;
};

// Plain fp32 output; split-K partial slab s lands at C + s * split_stride; accumulate adds
// to the existing values instead of overwriting them.
hipError_t gemm_f32(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                    int K, int splits, float* C, int64_t ldc, int64_t split_stride, int accumulate,
                    const GemmSeg2& s2 = GemmSeg2(), const GemmGroup& gg = GemmGroup());
// GELU up-projection epilogue: A = GELU(U) [M x lda], A^T [N x ldat] (AT may be null),
// GELU'(U) [M x lda], and (RES non-null) the rounding residual A - rn(A) [M x lda]; with add
// (fp32 [M x lda]), U = X Y^T + add.
hipError_t gemm_gelu(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                     int K, void* A, void* AT, void* GP, void* RES, int64_t lda, int64_t ldat,
                     const GemmSeg2& s2 = GemmSeg2(), const GemmGroup& gg = GemmGroup(), const float* add = nullptr);
// SwiGLU up epilogue: V = X Y^T kept in VU (fp32, may be null), A = SiLU(UG) * V stored as
// A [M x lda] and A^T [N x ldat], RES as above.
hipError_t gemm_swiglu(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                       int K, const float* UG, float* VU, void* A, void* AT, void* RES, int64_t lda, int64_t ldat);
// GELU backward epilogue: dU = (X Y^T) * GP, dU [M x ld], dU^T [N x ldt]; with RES, per-token
// partial dots <X Y^T, RES> of each column tile into cdot [tiles x ldc].
hipError_t gemm_du(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                   int K, const void* GP, void* DU, void* DUT, const void* RES, float* cdot, int64_t ld, int64_t ldt,
                   int64_t ldc, const GemmGroup& gg = GemmGroup());
// SwiGLU backward through frozen gate/up: dA = X Y^T; dG, dV [M x ld]; partial dots with RES.
hipError_t gemm_swiglu_bwd(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M,
                           int N, int K, const float* UG, const float* VU, void* DG, void* DV, const void* RES,
                           float* cdot, int64_t ld, int64_t ldc, const GemmGroup& gg = GemmGroup());
// C [M x ldc] in the GEMM operand precision.
hipError_t gemm_store(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                      int K, void* C, int64_t ldc);
// bf16 operands: C stored twice, Ch = rn_bf16(C) and Cf = rn_f16(C), both [M x ldc].
hipError_t gemm_store_bf16_f16(hipStream_t st, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                              int K, void* Ch, void* Cf, int64_t ldc, const GemmSeg2& s2 = GemmSeg2());
// Output tile shape the launcher uses for a GEMM of this shape (M, N, K, K2, splits, and the
// number of products of a grouped launch): per-tile buffers (CE partials, sums of squares,
// partial dots) are sized from it.
void gemm_tile_shape(int prec, int M, int N, int K, int K2, int splits, int* tile_m, int* tile_n, int groups = 1);
// Split-K slabs for a GEMM with a small output and a long K (K + K2): as many as fit in one
// round of the workgroups the chip runs at once for its tile shape, at least 4 K-iterations
// per slab, at most max_splits.
int gemm_split_k(int prec, int M, int N, int K, int K2, int max_splits);
// Weight-gradient epilogue: G [M x ldg] in the GEMM precision and one sum of squares of the
// fp32 accumulators per output tile in slot[tile].
hipError_t gemm_grad(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N,
                     int K, void* G, int64_t ldg, float* slot, const GemmGroup& gg = GemmGroup());
// The same weight gradient from token-major operands (bf16): G [M x ldg] = sum over k < K
// of X[k][i] Y[k][j], X [K x ldx], Y [K x ldy] row-major (the activations as the forward
// and backward products write them); K a multiple of 64, M and N multiples of 8. Same tiles
// and slots as gemm_grad with K token columns; hipErrorInvalidValue for other shapes.
hipError_t gemm_grad_km(hipStream_t st, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M, int N, int K,
                        void* G, int64_t ldg, float* slot, const GemmGroup& gg = GemmGroup());
// LM head + online-softmax partials over the full vocabulary (N = V): one record per row and
// per wave column block of gemm_wave_cols() vocabulary entries (records [M x nrec]), and,
// when Q is non-null, the numerators exp(z - record max) [M x ldq] in the GEMM precision.
hipError_t gemm_ce_partial(hipStream_t st, int prec, const void* X, int64_t ldx, const void* Y, int64_t ldy, int M,
                           int N, int K, const int* tgt, float* pmax, float* psum, int* pidx, float* tgt_logit,
                           int nrec, void* Q, int64_t ldq, const GemmSeg2& s2 = GemmSeg2());
// Columns of one wave's sub-tile for a GEMM of this shape (the CE record width).
int gemm_wave_cols(int prec, int M, int N, int K, int K2, int splits, int groups = 1);
