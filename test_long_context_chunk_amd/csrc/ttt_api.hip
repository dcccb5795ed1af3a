// Host side of the C ABI declared in include/ttt.h: configuration checks, the device
// memory plan, weight ingestion, and the chunk loop that enqueues the kernels.
#include <mutex>
#include <new>
#include <vector>

#include "common.h"
#include "launchers.h"
#include "ttt.h"

namespace {

constexpr int SPLIT_MAX = 8;       // split-K slabs for the small-M, long-K GEMMs
constexpr int PAD = 64;             // token dimension of transposed activations is padded to this

// One fast tensor, natural layout [rows x cols] (W1 [d x m], W2 [m x d]), one copy of its
// state per stream (D, Wop, WtT, G: stream z at z rows cols elements) over a shared W0. The
// forward GEMMs read it transposed, the backward GEMMs row-major:
//   fp32: forward X (W0 + D)^T via WtT; backward X (W0 + D) via Wop.
//   bf16: forward X W0^T + X rn(D)^T via W0T and WtT (two K-segments, so updates far below
//         the rounding step of W0 still reach the forward pass); backward X rn(W0 + D) via Wop.
struct FastTensor {
  int rows = 0, cols = 0;
  void* W0 = nullptr;      // initial weights (GEMM precision) [rows x cols]
  void* W0T = nullptr;     // bf16 only: W0^T [cols x rows]
  float* D = nullptr;      // accumulated update, fp32 [streams][rows x cols]
  void* Wop = nullptr;     // rn(W0 + D) [streams][rows x cols]
  void* WtT = nullptr;     // bf16: rn(D)^T, fp32: (W0 + D)^T  [streams][cols x rows]
  void* G = nullptr;       // chunk gradient in the GEMM precision [streams][rows x cols]
  int slot0 = 0;           // first grad-norm slot (within a stream's slots)
  hipEvent_t ev_upd = nullptr;  // recorded on the aux stream after this tensor's last update
  // snapshot of the state a step changes (D, Wop, WtT), allocated at the first snapshot
  void* snapD = nullptr;
  void* snapWop = nullptr;
  void* snapWtT = nullptr;
};

struct Block {
  FastTensor w1, w2;        // w1 unused for SwiGLU
  void* WgT = nullptr;      // SwiGLU frozen gate, [m x d]
  void* WuT = nullptr;      // SwiGLU frozen up, [m x d]
  void* Wg = nullptr;       // SwiGLU frozen gate/up, natural [d x m] (loss compensation only)
  void* Wu = nullptr;
  // per-token buffers hold the R = streams x b rows of one step (stream z: rows z b ..);
  // transposed ones [.. x Rp] hold stream z in columns z bp ..
  void* Hn = nullptr;       // normed block input [R x d]
  void* HnT = nullptr;      // its transpose [d x Rp]
  float* r = nullptr;       // RMSNorm scale per token [R]
  void* AT = nullptr;       // activation transpose [m x Rp] (weight gradients from transposed operands)
  void* A = nullptr;        // activation [R x m] (weight gradients from token-major operands)
  void* GP = nullptr;       // GELU'(U) [R x m]
  void* ResN = nullptr;     // bf16 only: n - rn(n) [R x d]
  void* ResA = nullptr;     // bf16 only: A - rn(A) [R x m]
  float* VU = nullptr;      // SwiGLU + bf16: up projection n Wu [R x m] fp32
  int cslot = 0;            // first loss-compensation slot of this block
  // frozen static MLP before the fast one (m_s > 0): its weights in both orientations, and
  // what its backward reads
  void* SW1T = nullptr;     // Ws1^T [m_s x d] (forward)
  void* SW2T = nullptr;     // Ws2^T [d x m_s] (forward)
  void* SW1 = nullptr;      // Ws1 [d x m_s] (backward)
  void* SW2 = nullptr;      // Ws2 [m_s x d] (backward)
  void* Sn = nullptr;       // its normed input [R x d]
  float* Sr = nullptr;      // its RMSNorm scale [R]
  void* SGP = nullptr;      // GELU'(U_s) [R x m_s]
  void* SResN = nullptr;    // bf16 only: n_s - rn(n_s) [R x d]
  void* SResA = nullptr;    // bf16 only: A_s - rn(A_s) [R x m_s]
  int scslot = 0;           // first loss-compensation slot of the static MLP
  // frozen sliding-window attention first in the block (window > 0)
  void* WqkvT = nullptr;    // [Wq Wk Wv]^T [3d x d] (forward)
  void* Wqkv = nullptr;     // [Wq Wk Wv] [d x 3d] (backward)
  void* WoT = nullptr;      // Wo^T [d x d] (forward)
  void* Wo = nullptr;       // Wo [d x d] (backward)
  void* Na = nullptr;       // its normed input [R x d]
  float* ra = nullptr;      // its RMSNorm scale [R]
  void* ResNa = nullptr;    // bf16 only: n_a - rn(n_a)
  void* QKV = nullptr;      // the chunk's q | k | v [R x 3d]
  void* QKV16 = nullptr;    // the same in half precision (the attention forward's operands)
  float* Of = nullptr;      // attention output, fp32 [R x d]
  void* Ob = nullptr;       // and its GEMM operand copy
  void* Obl = nullptr;      // and that copy's rounding residual
  float* lse2 = nullptr;    // log2 softmax denominators [streams][heads][b]
  void* Kc = nullptr;       // ring of earlier keys / values [streams][cr x d], bf16
  void* Vc = nullptr;
  void* Kc16 = nullptr;     // and in half precision
  void* Vc16 = nullptr;
  void* Ke = nullptr;       // the same for a passage being scored (single stream) [cr x d]
  void* Ve = nullptr;
  void* Ke16 = nullptr;
  void* Ve16 = nullptr;
  int acslot = 0;           // loss-compensation slots of the attention: O, n_a
};

}  // namespace

struct ttt_ctx {
  ttt_config cfg{};
  hipStream_t st = nullptr;
  int prec = 0, es = 4;
  int b = 0, bp = 0, V = 0, d = 0, m = 0, L = 0;
  // independent token streams advanced together (each with its own fast state, records and
  // clip); a step covers R = nb b token rows, Rp = nb bp columns of the transposed buffers
  int nb = 1, R = 0, Rp = 0;
  // bf16 training with whole 64-token slices: the weight gradients read the activations and
  // their gradients token-major (no transposed copies)
  bool km = false;
  int ms = 0;          // hidden size of the static MLP of every block (0: none)
  int window = 0;      // keys per query of the attention of every block (0: none)
  int cr = 0;          // ring positions per stream and block (window + chunk)
  bool eval_ring = false;  // the attention reads and fills the passage rings (evaluation)
  float *dOf = nullptr, *Dq = nullptr;  // attention backward scratch: dO fp32, row terms
  float *swa_part = nullptr, *swa_m = nullptr, *swa_l = nullptr;  // forward split partials
  float* swa_part2 = nullptr;  // the dK, dV pass's split partials (it runs beside the dQ pass)
  void *dOb = nullptr, *dQKV = nullptr;
  int dot_tiles_s = 0;  // column tiles of the static dA GEMM
  std::vector<void*> allocs;

  void *E_in = nullptr, *E_out = nullptr, *E_outT = nullptr;
  std::vector<Block> blocks;
  std::vector<FastTensor*> fast;

  float* H = nullptr;
  void* Yb = nullptr;
  int *tok_prev = nullptr, *tok_tgt = nullptr;
  float *pmax = nullptr, *psum = nullptr, *tgt_logit = nullptr, *lse = nullptr;
  int* pidx = nullptr;
  int ce_w = 0;     // vocabulary entries per CE record (one wave's columns of the LM-head GEMM)
  int ce_nrec = 0;  // CE records per row: ceil(V / ce_w)
  int dot_tiles = 0;  // column tiles of the dA GEMM (one partial dot per tile and row)
  void* P = nullptr;
  // decode: ids of the pending (not yet stepped) chunk [b + 1], how many of its pairs are
  // filled, and the one-row fp32 activations
  int* dec_tok = nullptr;
  int npend = 0;
  // evaluation and Settlement: one chunk's losses and argmax, fp64 loss sums, A and the decision
  float* eval_loss = nullptr;
  int* eval_amax = nullptr;
  double* eval_acc = nullptr;  // [3]: ttt_evaluate, L(q, W), L(q, W + delta)
  float* settle_A = nullptr;
  int* settle_commit = nullptr;
  bool has_snap = false;
  int dev = 0;  // the device current at creation (the stream's device)
  float *dec_h = nullptr, *dec_a = nullptr, *dec_z = nullptr, *dec_rmax = nullptr, *dec_rsum = nullptr;
  int* dec_ridx = nullptr;
  // decode with attention: the row's q | k | v [3d], the attention output [d] and the
  // attention's per-share states
  float *dec_qkv = nullptr, *dec_o = nullptr, *dec_part = nullptr;
  float* part = nullptr;
  float* dH = nullptr;
  void *dHb = nullptr, *dHT = nullptr, *A = nullptr, *dU = nullptr, *dUT = nullptr;
  float* UG = nullptr;
  void *DG = nullptr, *DV = nullptr;  // SwiGLU + bf16: gradients at the gate / up outputs
  bool foc = false;                   // first-order loss compensation (bf16 with blocks)
  // bf16 with attention: every forward product reads its activation operand as two bf16
  // terms (the value and its rounding residual), instead of the loss compensation
  bool split = false;
  float* Ul = nullptr;                // split: the residual term of the fast up-projection [R x m]
  void* Yl = nullptr;                 // split: the residual of the LM head's operand [R x d]
  float* cpart = nullptr;             // compensation slots [ncslot x R]
  int ncslot = 0;
  float* slots = nullptr;  // grad-norm slots [nb x nslots]
  int nslots = 0;          // per stream
  float* sc = nullptr;     // clip scale and skip flag, 4 floats per stream
  float* losses = nullptr;  // [nb x max_tokens]
  int* amax = nullptr;      // [nb x max_tokens]
  float* stats = nullptr;   // [nb x max_chunks x 2]
  int* err = nullptr;
  int64_t max_chunks = 0;

  int64_t pos = 0;
  ttt_status sticky = TTT_OK;

  // off-critical-path work (the weight gradients of GELU blocks on the token-major path, and
  // the SGD step) runs on a second stream (default priority): it starts after an event on the
  // main stream, and the main stream waits for its event right before the consumer
  hipStream_t aux = nullptr;
  hipEvent_t ev_to_aux = nullptr, ev_from_aux = nullptr;
  // GELU blocks, token-major gradients: each block's two weight gradients run on the aux
  // stream beside the main stream's dHn, norm backward, frozen layers and the next block's dA.
  // Each block then has backward row buffers of its own (dHl[l] holds the gradient at block
  // l's output, dUl[l] its fast dU; blocks 0 and 1 use dHb / dU and dHb2 / dU2), so nothing
  // the main stream writes in a chunk is read by a gradient still running on the aux stream:
  // a block's buffers are rewritten only in the next chunk, whose forward pass waits for the
  // SGD steps queued behind every gradient. The gradients between a block's sublayers go to
  // dHm and the static MLP's dU to dUs; ev_grad[0] marks the lowest block's gradients done.
  bool agrad = false;
  bool grads_inflight = false;  // the last step's gradients may still read the lowest block's Hn
  void *dHb2 = nullptr, *dU2 = nullptr, *dHm = nullptr, *dUs = nullptr;
  std::vector<void*> dHl, dUl;
  hipEvent_t ev_gin = nullptr, ev_grad[2] = {nullptr, nullptr};
  // attention backward: the dK, dV pass on the aux stream beside the dQ pass
  hipEvent_t ev_ain = nullptr, ev_aout = nullptr;
  // recorded on the main stream after the backward's last product that reads rn(W0 + D) (the
  // lowest block's dHn, else its dA): the SGD steps on the aux stream wait for it
  hipEvent_t ev_wread = nullptr;

  // tracing: event pairs around launches of the kinds set in prof_mask
  uint32_t prof_mask = 0;
  int prof_period = 1;      // trace every prof_period-th chunk
  int64_t prof_chunks = 0;  // chunks run since tracing was configured
  bool prof_on = false;     // the current chunk is traced
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
  std::vector<int> ev_kind;
};

namespace {

struct HipFail {
  ttt_status s;
};

// Events that only order work between this library's streams on one device: no timing and a
// device-scope release (the default system-scope release writes back and invalidates the
// caches at every record, for a host that never reads this memory).
constexpr unsigned kSyncEvent = hipEventDisableTiming | hipEventReleaseToDevice;

inline void check(hipError_t e) {
  if (e == hipSuccess) return;
  // clear the runtime's last-error state, so that a refused allocation is reported here
  // only and not again by the caller's next unrelated HIP call
  (void)hipGetLastError();
  if (e == hipErrorOutOfMemory) throw HipFail{TTT_ENOMEM};
  throw HipFail{TTT_EDEVICE};
}

template <class P>
P* dalloc(ttt_ctx* c, int64_t bytes) {
  void* p = nullptr;
  if (bytes <= 0) bytes = 16;
  check(hipMalloc(&p, (size_t)bytes));
  c->allocs.push_back(p);
  return (P*)p;
}

void free_all(ttt_ctx* c) {
  for (void* p : c->allocs) (void)hipFree(p);
  c->allocs.clear();
}

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Enqueue on the aux stream after everything enqueued so far on the main stream.
void aux_fork(ttt_ctx* c) {
  check(hipEventRecord(c->ev_to_aux, c->st));
  check(hipStreamWaitEvent(c->aux, c->ev_to_aux, 0));
}
// Mark the aux work enqueued so far; aux_join makes the main stream wait for it.
void aux_mark(ttt_ctx* c) { check(hipEventRecord(c->ev_from_aux, c->aux)); }
void aux_join(ttt_ctx* c) { check(hipStreamWaitEvent(c->st, c->ev_from_aux, 0)); }

ttt_status validate(const ttt_config* c, const ttt_weights* w) {
  if (!c || !w) return TTT_EINVAL;
  if (c->abi_version != TTT_ABI_VERSION || c->reserved != 0 || c->reserved_f != 0.f) return TTT_EINVAL;
  if (c->vocab < 2 || c->vocab % 8 || c->d_model < 8 || c->d_model % 8 || c->d_hidden < 8 || c->d_hidden % 8)
    return TTT_EINVAL;
  if (c->n_blocks < 0 || c->n_blocks > 64) return TTT_EINVAL;
  if (c->mlp != TTT_MLP_GELU && c->mlp != TTT_MLP_SWIGLU_W2) return TTT_EINVAL;
  if (c->mlp == TTT_MLP_SWIGLU_W2 && c->n_blocks != 1) return TTT_EINVAL;
  if (c->norm != TTT_NORM_NONE && c->norm != TTT_NORM_RMS) return TTT_EINVAL;
  if (c->precision != TTT_FP32 && c->precision != TTT_BF16) return TTT_EINVAL;
  if (c->chunk < 1 || c->chunk > (1 << 20)) return TTT_EINVAL;
  if (c->max_tokens < c->chunk || c->max_tokens % c->chunk) return TTT_EINVAL;
  if (!(c->lr >= 0.f) || !(c->rms_eps >= 0.f) || c->clip != c->clip) return TTT_EINVAL;
  if (c->norm == TTT_NORM_RMS && !(c->rms_eps > 0.f)) return TTT_EINVAL;
  if ((int64_t)c->vocab * c->d_model > (int64_t)1 << 31) return TTT_EINVAL;
  if (!w->embed || !w->lm_head) return TTT_EINVAL;
  if (c->n_blocks > 0) {
    if (!w->w1 || !w->w2) return TTT_EINVAL;
    if (c->mlp == TTT_MLP_SWIGLU_W2 && !w->w_up) return TTT_EINVAL;
    for (int l = 0; l < c->n_blocks; ++l) {
      if (!w->w1[l] || !w->w2[l]) return TTT_EINVAL;
      if (c->mlp == TTT_MLP_SWIGLU_W2 && !w->w_up[l]) return TTT_EINVAL;
    }
  }
  return TTT_OK;
}

ttt_status validate_ext(const ttt_config* c, const ttt_block_ext* e) {
  if (!e) return TTT_OK;
  if (e->reserved) return TTT_EINVAL;
  if (e->static_hidden < 0 || e->swa_window < 0) return TTT_EINVAL;
  if (e->static_hidden > 0) {
    if (e->static_hidden < 8 || e->static_hidden % 8 || c->mlp != TTT_MLP_GELU) return TTT_EINVAL;
    if (c->n_blocks > 0) {
      if (!e->ws1 || !e->ws2) return TTT_EINVAL;
      for (int l = 0; l < c->n_blocks; ++l)
        if (!e->ws1[l] || !e->ws2[l]) return TTT_EINVAL;
    }
  }
  if (e->swa_window > 0) {
    // bf16 heads of 128 over the GELU block
    if (c->precision != TTT_BF16 || c->mlp != TTT_MLP_GELU || e->swa_window > (1 << 24)) return TTT_EINVAL;
    if (e->swa_heads < 1 || c->d_model != e->swa_heads * 128) return TTT_EINVAL;
    if (c->n_blocks > 0) {
      if (!e->wq || !e->wk || !e->wv || !e->wo) return TTT_EINVAL;
      for (int l = 0; l < c->n_blocks; ++l)
        if (!e->wq[l] || !e->wk[l] || !e->wv[l] || !e->wo[l]) return TTT_EINVAL;
    }
  }
  return TTT_OK;
}

// A frozen weight [rows x cols] copied into the library in natural and transposed layout.
void frozen_pair(ttt_ctx* c, const void* src, int rows, int cols, void** nat, void** tr) {
  const int64_t bytes = (int64_t)rows * cols * c->es;
  *nat = dalloc<char>(c, bytes);
  *tr = dalloc<char>(c, bytes);
  check(hipMemcpyAsync(*nat, src, bytes, hipMemcpyDeviceToDevice, c->st));
  check(run_transpose(c->st, c->prec, src, cols, rows, cols, *tr, rows));
}

// The attention's problem description for block B's chunk starting at position pos.
SwaShape swa_shape(ttt_ctx* c, Block& B, int64_t pos) {
  SwaShape s;
  s.qkv = B.QKV;
  s.qkv16 = B.QKV16;
  const bool e = c->eval_ring;
  s.kc = e ? B.Ke : B.Kc;
  s.vc = e ? B.Ve : B.Vc;
  s.kc16 = e ? B.Ke16 : B.Kc16;
  s.vc16 = e ? B.Ve16 : B.Vc16;
  s.cr = c->cr;
  s.b = c->b;
  s.d = c->d;
  s.window = c->window;
  s.streams = c->nb;
  s.pos = pos;
  return s;
}

void init_fast(ttt_ctx* c, FastTensor& f, int rows, int cols, const void* src) {
  const int64_t n = (int64_t)rows * cols;
  f.rows = rows;
  f.cols = cols;
  const int64_t nz = n * c->nb;
  f.W0 = dalloc<char>(c, n * c->es);
  f.D = dalloc<float>(c, nz * 4);
  f.Wop = dalloc<char>(c, nz * c->es);
  f.WtT = dalloc<char>(c, nz * c->es);
  f.G = dalloc<char>(c, nz * c->es);
  check(hipMemcpyAsync(f.W0, src, n * c->es, hipMemcpyDeviceToDevice, c->st));
  if (c->prec == PREC_BF16) {
    f.W0T = dalloc<char>(c, n * c->es);
    check(run_transpose(c->st, c->prec, f.W0, cols, rows, cols, f.W0T, rows));
  }
  f.slot0 = c->nslots;
  int tm = 0, tn = 0;
  gemm_tile_shape(c->prec, rows, cols, c->bp, 0, 1, &tm, &tn);
  c->nslots += cdiv(rows, tm) * cdiv(cols, tn);
  check(hipEventCreateWithFlags(&f.ev_upd, kSyncEvent));
  c->fast.push_back(&f);
}

void reset_fast(ttt_ctx* c, FastTensor& f) {
  const int64_t n = (int64_t)f.rows * f.cols;
  check(run_fill_u32(c->st, f.D, n * c->nb, 0u));
  if (c->prec == PREC_BF16) check(run_fill_u32(c->st, f.WtT, n * c->nb * c->es / 4, 0u));  // rn(D)^T with D = 0
  for (int z = 0; z < c->nb; ++z) {
    check(hipMemcpyAsync((char*)f.Wop + z * n * c->es, f.W0, n * c->es, hipMemcpyDeviceToDevice, c->st));
    if (c->prec != PREC_BF16)
      check(run_transpose(c->st, c->prec, f.W0, f.cols, f.rows, f.cols, (char*)f.WtT + z * n * c->es, f.rows));
  }
}

void build(ttt_ctx* c, const ttt_weights* w, const ttt_block_ext* ext) {
  const int b = c->b, V = c->V, d = c->d, m = c->m, L = c->L, es = c->es;
  const int Rr = c->R, Rp = c->Rp, nb = c->nb, ms = c->ms;
  const int mx = m > ms ? m : ms;  // widest hidden activation
  const int64_t Vd = (int64_t)V * d;
  c->E_in = dalloc<char>(c, Vd * es);
  c->E_out = dalloc<char>(c, Vd * es);
  c->E_outT = dalloc<char>(c, Vd * es);
  check(hipMemcpyAsync(c->E_in, w->embed, Vd * es, hipMemcpyDeviceToDevice, c->st));
  check(hipMemcpyAsync(c->E_out, w->lm_head, Vd * es, hipMemcpyDeviceToDevice, c->st));
  check(run_transpose(c->st, c->prec, c->E_out, d, V, d, c->E_outT, V));

  c->foc = c->prec == PREC_BF16 && L > 0 && c->window == 0;
  c->split = c->prec == PREC_BF16 && L > 0 && c->window > 0;
  const bool res = c->foc || c->split;  // rounding residuals of the forward operands are kept
  int tmm = 0, tnm_w = 0;
  gemm_tile_shape(c->prec, b, m, d, 0, 1, &tmm, &tnm_w, nb);  // the dA GEMM (M = b, N = m, K = d, per stream)
  const int tnm = cdiv(m, tnm_w);
  c->dot_tiles = tnm;
  int tns = 0;
  if (ms > 0) {
    int tsm = 0, tsn = 0;
    gemm_tile_shape(c->prec, Rr, ms, d, 0, 1, &tsm, &tsn);  // the static dA GEMM
    tns = cdiv(ms, tsn);
  }
  c->dot_tiles_s = tns;
  c->ncslot = 1;  // slot 0: the LM-head input Y
  c->blocks.resize(L);
  for (int l = 0; l < L; ++l) {
    Block& B = c->blocks[l];
    if (c->cfg.mlp == TTT_MLP_GELU) {
      init_fast(c, B.w1, d, m, w->w1[l]);
      B.GP = dalloc<char>(c, (int64_t)Rr * m * es);
      if (!c->km) {
        B.HnT = dalloc<char>(c, (int64_t)d * Rp * es);
        check(hipMemsetAsync(B.HnT, 0, (int64_t)d * Rp * es, c->st));
      }
    } else {
      B.WgT = dalloc<char>(c, (int64_t)m * d * es);
      B.WuT = dalloc<char>(c, (int64_t)m * d * es);
      check(run_transpose(c->st, c->prec, w->w1[l], m, d, m, B.WgT, d));
      check(run_transpose(c->st, c->prec, w->w_up[l], m, d, m, B.WuT, d));
      if (c->foc) {
        B.Wg = dalloc<char>(c, (int64_t)m * d * es);
        B.Wu = dalloc<char>(c, (int64_t)m * d * es);
        check(hipMemcpyAsync(B.Wg, w->w1[l], (int64_t)m * d * es, hipMemcpyDeviceToDevice, c->st));
        check(hipMemcpyAsync(B.Wu, w->w_up[l], (int64_t)m * d * es, hipMemcpyDeviceToDevice, c->st));
        B.VU = dalloc<float>(c, (int64_t)Rr * m * 4);
      }
    }
    init_fast(c, B.w2, m, d, w->w2[l]);
    if (c->window > 0) {
      const int64_t dd = (int64_t)d * d * es;
      B.WqkvT = dalloc<char>(c, 3 * dd);
      B.Wqkv = dalloc<char>(c, 3 * dd);
      const void* const* src[3] = {ext->wq, ext->wk, ext->wv};
      for (int j = 0; j < 3; ++j) {
        check(run_transpose(c->st, c->prec, src[j][l], d, d, d, (char*)B.WqkvT + j * dd, d));
        check(hipMemcpy2DAsync((char*)B.Wqkv + (int64_t)j * d * es, (size_t)3 * d * es, src[j][l], (size_t)d * es,
                               (size_t)d * es, d, hipMemcpyDeviceToDevice, c->st));
      }
      frozen_pair(c, ext->wo[l], d, d, &B.Wo, &B.WoT);
      B.Na = dalloc<char>(c, (int64_t)Rr * d * es);
      B.ra = dalloc<float>(c, (int64_t)Rr * 4);
      B.QKV = dalloc<char>(c, (int64_t)Rr * 3 * d * es);
      B.QKV16 = dalloc<char>(c, (int64_t)Rr * 3 * d * 2);
      B.Of = dalloc<float>(c, (int64_t)Rr * d * 4);
      B.Ob = dalloc<char>(c, (int64_t)Rr * d * es);
      B.Obl = dalloc<char>(c, (int64_t)Rr * d * es);
      B.lse2 = dalloc<float>(c, (int64_t)Rr * (d / 128) * 4);
      B.Kc = dalloc<char>(c, (int64_t)nb * c->cr * d * es);
      B.Vc = dalloc<char>(c, (int64_t)nb * c->cr * d * es);
      B.Kc16 = dalloc<char>(c, (int64_t)nb * c->cr * d * 2);
      B.Vc16 = dalloc<char>(c, (int64_t)nb * c->cr * d * 2);
      if (nb == 1) {  // evaluation (single-stream contexts only)
        B.Ke = dalloc<char>(c, (int64_t)c->cr * d * es);
        B.Ve = dalloc<char>(c, (int64_t)c->cr * d * es);
        B.Ke16 = dalloc<char>(c, (int64_t)c->cr * d * 2);
        B.Ve16 = dalloc<char>(c, (int64_t)c->cr * d * 2);
      }
      if (res) B.ResNa = dalloc<char>(c, (int64_t)Rr * d * es);
      if (c->foc) {
        B.acslot = c->ncslot;
        c->ncslot += 2;  // O, n_a
      }
    }
    if (ms > 0) {
      frozen_pair(c, ext->ws1[l], d, ms, &B.SW1, &B.SW1T);
      frozen_pair(c, ext->ws2[l], ms, d, &B.SW2, &B.SW2T);
      B.Sn = dalloc<char>(c, (int64_t)Rr * d * es);
      B.Sr = dalloc<float>(c, (int64_t)Rr * 4);
      B.SGP = dalloc<char>(c, (int64_t)Rr * ms * es);
      if (res) {
        B.SResN = dalloc<char>(c, (int64_t)Rr * d * es);
        B.SResA = dalloc<char>(c, (int64_t)Rr * ms * es);
      }
      if (c->foc) {
        B.scslot = c->ncslot;
        c->ncslot += tns + 1;  // tns partial dots for A_s, one for n_s
      }
    }
    B.Hn = dalloc<char>(c, (int64_t)Rr * d * es);
    B.r = dalloc<float>(c, (int64_t)Rr * 4);
    if (c->km) {
      B.A = dalloc<char>(c, (int64_t)Rr * m * es);
    } else {
      B.AT = dalloc<char>(c, (int64_t)m * Rp * es);
      check(hipMemsetAsync(B.AT, 0, (int64_t)m * Rp * es, c->st));
    }
    if (res) {
      B.ResN = dalloc<char>(c, (int64_t)Rr * d * es);
      B.ResA = dalloc<char>(c, (int64_t)Rr * m * es);
    }
    if (c->foc) {
      B.cslot = c->ncslot;
      c->ncslot += tnm + 1;  // tnm partial dots for A, one for n
    }
  }
  for (FastTensor* f : c->fast) reset_fast(c, *f);

  c->H = dalloc<float>(c, (int64_t)Rr * d * 4);
  c->Yb = dalloc<char>(c, (int64_t)Rr * d * es);
  c->tok_prev = dalloc<int>(c, (int64_t)Rr * 4);
  c->tok_tgt = dalloc<int>(c, (int64_t)Rr * 4);
  c->ce_w = gemm_wave_cols(c->prec, Rr, V, d, c->split ? d : 0, 1);  // the LM-head GEMM (all streams' rows)
  c->ce_nrec = cdiv(V, c->ce_w);
  c->pmax = dalloc<float>(c, (int64_t)c->ce_nrec * Rr * 4);
  c->psum = dalloc<float>(c, (int64_t)c->ce_nrec * Rr * 4);
  c->pidx = dalloc<int>(c, (int64_t)c->ce_nrec * Rr * 4);
  c->tgt_logit = dalloc<float>(c, (int64_t)Rr * 4);
  c->lse = dalloc<float>(c, (int64_t)Rr * 4);
  if (L > 0) c->P = dalloc<char>(c, (int64_t)Rr * V * es);  // softmax numerators, then dlogits
  // split-K slabs; the split forward adds the residual terms' slabs after the main ones
  c->part = dalloc<float>(c, (int64_t)(c->split ? 2 : 1) * SPLIT_MAX * Rr * d * 4);
  if (c->split) {
    c->Ul = dalloc<float>(c, (int64_t)Rr * m * 4);
    c->Yl = dalloc<char>(c, (int64_t)Rr * d * es);
  }
  c->dec_tok = dalloc<int>(c, (int64_t)(b + 1) * 4);
  c->eval_loss = dalloc<float>(c, (int64_t)b * 4);
  c->eval_amax = dalloc<int>(c, (int64_t)b * 4);
  c->eval_acc = dalloc<double>(c, 3 * 8);
  c->settle_A = dalloc<float>(c, 4);
  c->settle_commit = dalloc<int>(c, 4);
  c->dec_h = dalloc<float>(c, (int64_t)d * 4);
  c->dec_a = dalloc<float>(c, (int64_t)mx * 4);
  c->dec_z = dalloc<float>(c, (int64_t)V * 4);
  c->dec_rmax = dalloc<float>(c, (int64_t)cdiv(V, gemv_rec_rows(V)) * 4);
  c->dec_rsum = dalloc<float>(c, (int64_t)cdiv(V, gemv_rec_rows(V)) * 4);
  c->dec_ridx = dalloc<int>(c, (int64_t)cdiv(V, gemv_rec_rows(V)) * 4);
  c->dH = dalloc<float>(c, (int64_t)Rr * d * 4);
  c->dHb = dalloc<char>(c, (int64_t)Rr * d * es);
  if (!c->km) {
    c->dHT = dalloc<char>(c, (int64_t)d * Rp * es);
    check(hipMemsetAsync(c->dHT, 0, (int64_t)d * Rp * es, c->st));
  }
  c->A = dalloc<char>(c, (int64_t)Rr * mx * es);
  c->dU = dalloc<char>(c, (int64_t)Rr * mx * es);
  if (c->agrad) {
    c->dHb2 = dalloc<char>(c, (int64_t)Rr * d * es);
    c->dU2 = dalloc<char>(c, (int64_t)Rr * mx * es);
    for (int l = 0; l < L; ++l) {
      c->dHl.push_back(l == 0 ? c->dHb : l == 1 ? c->dHb2 : dalloc<char>(c, (int64_t)Rr * d * es));
      c->dUl.push_back(l == 0 ? c->dU : l == 1 ? c->dU2 : dalloc<char>(c, (int64_t)Rr * mx * es));
    }
    if (c->ms > 0 || c->window > 0) c->dHm = dalloc<char>(c, (int64_t)Rr * d * es);
    if (c->ms > 0) c->dUs = dalloc<char>(c, (int64_t)Rr * c->ms * es);
  }
  if (!c->km) {
    c->dUT = dalloc<char>(c, (int64_t)m * Rp * es);
    check(hipMemsetAsync(c->dUT, 0, (int64_t)m * Rp * es, c->st));
  }
  if (c->cfg.mlp == TTT_MLP_SWIGLU_W2) c->UG = dalloc<float>(c, (int64_t)Rr * m * 4);
  if (c->window > 0 && L > 0) {
    c->dec_qkv = dalloc<float>(c, (int64_t)3 * d * 4);
    c->dec_o = dalloc<float>(c, (int64_t)d * 4);
    c->dec_part = dalloc<float>(c, (int64_t)(d / 128) * swa_dec_splits(c->window) * 130 * 4);
    c->dOf = dalloc<float>(c, (int64_t)Rr * d * 4);
    c->dOb = dalloc<char>(c, (int64_t)Rr * d * es);
    c->Dq = dalloc<float>(c, (int64_t)Rr * (d / 128) * 4);
    c->dQKV = dalloc<char>(c, (int64_t)Rr * 3 * d * es);
    const SwaShape sh = swa_shape(c, c->blocks[0], 0);
    const int ns = std::max({swa_fwd_splits(sh), swa_dq_splits(sh), 2 * swa_dkdv_splits(sh)});
    if (ns > 1) {
      c->swa_part = dalloc<float>(c, (int64_t)ns * Rr * d * 4);
      c->swa_m = dalloc<float>(c, (int64_t)ns * Rr * (d / 128) * 4);
      c->swa_l = dalloc<float>(c, (int64_t)ns * Rr * (d / 128) * 4);
    }
    if (swa_dkdv_splits(sh) > 1) c->swa_part2 = dalloc<float>(c, (int64_t)2 * swa_dkdv_splits(sh) * Rr * d * 4);
  }
  if (c->foc && c->cfg.mlp == TTT_MLP_SWIGLU_W2) {
    c->DG = dalloc<char>(c, (int64_t)Rr * m * es);
    c->DV = dalloc<char>(c, (int64_t)Rr * m * es);
  }
  if (c->foc) {
    c->cpart = dalloc<float>(c, (int64_t)c->ncslot * Rr * 4);
    check(hipMemsetAsync(c->cpart, 0, (int64_t)c->ncslot * Rr * 4, c->st));
  }
  const int64_t nsl = (int64_t)nb * (c->nslots > 0 ? c->nslots : 1);
  c->slots = dalloc<float>(c, nsl * 4);
  check(hipMemsetAsync(c->slots, 0, nsl * 4, c->st));
  c->sc = dalloc<float>(c, (int64_t)nb * 4 * 4);
  const int64_t ntok = (int64_t)nb * c->cfg.max_tokens;
  c->losses = dalloc<float>(c, ntok * 4);
  c->amax = dalloc<int>(c, ntok * 4);
  c->max_chunks = c->cfg.max_tokens / b;
  c->stats = dalloc<float>(c, nb * c->max_chunks * 2 * 4);
  c->err = dalloc<int>(c, 4);
  check(hipMemsetAsync(c->err, 0, 4, c->st));
  check(hipMemsetAsync(c->losses, 0, ntok * 4, c->st));
  check(hipMemsetAsync(c->amax, 0, ntok * 4, c->st));
  check(hipMemsetAsync(c->stats, 0, nb * c->max_chunks * 2 * 4, c->st));
  check(hipStreamCreateWithFlags(&c->aux, hipStreamNonBlocking));
  check(hipEventCreateWithFlags(&c->ev_to_aux, kSyncEvent));
  check(hipEventCreateWithFlags(&c->ev_from_aux, kSyncEvent));
  if (c->agrad)
    for (hipEvent_t* e : {&c->ev_gin, &c->ev_grad[0], &c->ev_grad[1], &c->ev_wread})
      check(hipEventCreateWithFlags(e, kSyncEvent));
  if (c->window > 0)
    for (hipEvent_t* e : {&c->ev_ain, &c->ev_aout}) check(hipEventCreateWithFlags(e, kSyncEvent));
}

// Wait for the aux stream, then release it (before any buffer it may read is freed).
void release_aux_stream(ttt_ctx* c) {
  if (c->aux) {
    (void)hipStreamSynchronize(c->aux);
    (void)hipStreamDestroy(c->aux);
    c->aux = nullptr;
  }
  for (hipEvent_t* e : {&c->ev_to_aux, &c->ev_from_aux, &c->ev_gin, &c->ev_grad[0], &c->ev_grad[1], &c->ev_ain,
                        &c->ev_aout, &c->ev_wread})
    if (*e) {
      (void)hipEventDestroy(*e);
      *e = nullptr;
    }
  for (FastTensor* f : c->fast)
    if (f->ev_upd) {
      (void)hipEventDestroy(f->ev_upd);
      f->ev_upd = nullptr;
    }
}

void prof_mark(ttt_ctx* c, hipStream_t st) {
  if (c->ev_used == c->ev_pool.size()) {
    hipEvent_t e;
    check(hipEventCreateWithFlags(&e, hipEventReleaseToDevice));
    c->ev_pool.push_back(e);
  }
  check(hipEventRecord(c->ev_pool[c->ev_used++], st));
}

// Enqueue one launch on stream `st`; bracket it with events on that stream when its kind is
// traced.
#define RUN_ON(kind, st_, expr)                 \
  do {                                          \
    const bool traced_ = c->prof_on && ((c->prof_mask >> (kind)) & 1u); \
    if (traced_) prof_mark(c, (st_));           \
    check(expr);                                \
    if (traced_) {                              \
      prof_mark(c, (st_));                      \
      c->ev_kind.push_back(kind);               \
    }                                           \
  } while (0)
#define RUN(kind, expr) RUN_ON(kind, c->st, expr)

// One chunk of [E2E] eq. (5): forward at W_{i-1}, record l_t(W_{i-1}) (eq. 6) into loss_out
// and the argmax into amax_out, backward to every fast tensor, global-norm clip ([SGF]), SGD
// step (chunk statistics at chunk_idx). With train = false, an evaluation at the current
// weights: the same losses, with the backward run only as far as the loss compensation needs
// it (no weight gradients, no step).
//
// bf16 only, first-order loss compensation: the forward rounds three kinds of GEMM operands
// to bf16 (block inputs n, activations A, the LM-head input Y). Each recorded loss is
// corrected by b * sum <dL/dX_t, X_t - rn(X_t)> over those operands, with dL/dX the
// chunk-mean-loss gradients the backward pass computes anyway, so l_t matches the loss of
// the unrounded forward to first order in the rounding error.
void run_chunk(ttt_ctx* c, const int32_t* tok, int64_t ldtok, float* loss_out, int* amax_out, int64_t ldl, bool train,
               int64_t chunk_idx) {
  hipStream_t st = c->st;
  c->prof_on = c->prof_mask != 0 && (c->prof_chunks++ % c->prof_period) == 0;
  const int prec = c->prec;
  const int b = c->b, bp = c->bp, V = c->V, d = c->d, m = c->m, L = c->L;
  // all streams' rows at once: R rows, transposed buffers Rp wide
  const int nb = c->nb, Rr = c->R, Rp = c->Rp;
  const int rms = c->cfg.norm == TTT_NORM_RMS;
  const bool gelu = c->cfg.mlp == TTT_MLP_GELU;
  const bool bf = prec == PREC_BF16;
  const bool foc = c->foc;
  const int64_t Rd = (int64_t)Rr * d;
  const int64_t n1 = (int64_t)d * m, n2 = (int64_t)m * d;  // elements of one stream's W1, W2
  const int tnm = c->dot_tiles;
  const StreamRows srt{b, ldtok}, srl{b, ldl};
  const int64_t chunk_pos = chunk_idx * b;  // position of the chunk's first row in each stream
  // Products with a stream's own fast weights run as one grouped launch over the streams
  // (stream z: token rows z b .., its weights z n .. past the first stream's); products
  // with frozen weights run once over all R rows.
  auto fw = [&](int64_t rows_x, int64_t ldx, int64_t nw, bool w_shared) {
    GemmGroup g;
    g.n = nb;
    g.x = rows_x * ldx;
    g.y = w_shared ? 0 : nw;
    g.x2 = rows_x * ldx;
    g.y2 = nw;
    return g;
  };
  auto gradg = [&](int64_t slot_stride) {  // weight gradients: K = a stream's token columns
    GemmGroup g;
    g.n = nb;
    g.x = bp;
    g.y = bp;
    g.tile = (int)slot_stride;
    return g;
  };
  auto gradkm = [&](int64_t ldx, int64_t ldy, int64_t slot_stride) {  // the same, token-major: a stream's rows
    GemmGroup g;
    g.n = nb;
    g.x = (int64_t)b * ldx;
    g.y = (int64_t)b * ldy;
    g.tile = (int)slot_stride;
    return g;
  };

  const int ms = c->ms;
  // where a row kernel leaves the pre-norm of the next MLP: block l's static MLP (when the
  // blocks have one) comes before its fast MLP
  struct NormOut {
    void* n = nullptr;
    float* r = nullptr;
    void* res = nullptr;
  };
  const bool split = c->split, keep_res = foc || split;
  auto mlp_norm = [&](Block& B) {  // the first MLP of the block
    NormOut o;
    o.n = ms > 0 ? B.Sn : B.Hn;
    o.r = ms > 0 ? B.Sr : B.r;
    o.res = keep_res ? (ms > 0 ? B.SResN : B.ResN) : nullptr;
    return o;
  };
  auto first_norm = [&](int l) {
    NormOut o;
    if (l >= L) return o;
    Block& B = c->blocks[l];
    if (c->window > 0) {
      o.n = B.Na;
      o.r = B.ra;
      o.res = keep_res ? B.ResNa : nullptr;
      return o;
    }
    return mlp_norm(B);
  };

  // The previous step's gradients on the aux stream read the lowest block's normed input
  // Hn: the row kernel that rewrites it waits for them first.
  auto guard_hn0 = [&](const void* n) {
    if (c->grads_inflight && L > 0 && n == c->blocks[0].Hn) {
      check(hipStreamWaitEvent(st, c->ev_grad[0], 0));
      c->grads_inflight = false;
    }
  };

  // a1 gather, and a2 the lowest block's pre-norm
  {
    const NormOut o = first_norm(0);
    guard_hn0(o.n);
    RUN(TTT_K_GATHER, run_row_in(st, prec, tok, srt, V, c->E_in, c->tok_prev, c->tok_tgt, c->err, nullptr, 0, 0, c->H,
                                 Rr, d, L == 0 ? c->Yb : nullptr, c->cfg.rms_eps, rms, o.n, o.r, o.res,
                                 L == 0 && split ? c->Yl : nullptr));
  }

  // a2-a4 forward through the blocks
  for (int l = 0; l < L; ++l) {
    Block& B = c->blocks[l];
    if (c->window > 0) {
      // the frozen sliding-window attention ([E2E] section 3), once over all streams' rows:
      // q | k | v, attention against the ring and the chunk's own keys, output projection
      RUN(TTT_K_UP, gemm_store_bf16_f16(st, B.Na, d, B.WqkvT, d, Rr, 3 * d, d, B.QKV, B.QKV16, 3 * d,
                                          split ? GemmSeg2{B.ResNa, d, B.WqkvT, d, d} : GemmSeg2()));
      RUN(TTT_K_ATTN, run_swa_fwd(st, swa_shape(c, B, chunk_pos), B.Of, B.Ob, B.Obl, B.lse2, c->swa_part, c->swa_m,
                                  c->swa_l));
      const int So = gemm_split_k(prec, Rr, d, d, split ? d : 0, SPLIT_MAX);
      RUN(TTT_K_DOWN, gemm_f32(st, prec, B.Ob, d, B.WoT, d, Rr, d, d, So, c->part, d, Rd, 0,
                               split ? GemmSeg2{B.Obl, d, B.WoT, d, d} : GemmSeg2()));
      const NormOut o = mlp_norm(B);
      guard_hn0(o.n);
      RUN(TTT_K_RESIDUAL, run_row_in(st, prec, nullptr, srt, V, nullptr, nullptr, nullptr, nullptr, c->part, So, Rd,
                                     c->H, Rr, d, nullptr, c->cfg.rms_eps, rms, o.n, o.r, o.res));
    }
    if (ms > 0) {
      // the frozen static MLP ([E2E] section 3.1), once over all streams' rows; its
      // transposed activation is never needed
      RUN(TTT_K_UP, gemm_gelu(st, prec, B.Sn, d, B.SW1T, d, Rr, ms, d, c->A, nullptr, B.SGP,
                              keep_res ? B.SResA : nullptr, ms, 0,
                              split ? GemmSeg2{B.SResN, d, B.SW1T, d, d} : GemmSeg2()));
      const int Ss = gemm_split_k(prec, Rr, d, ms, split ? ms : 0, SPLIT_MAX);
      RUN(TTT_K_DOWN, gemm_f32(st, prec, c->A, ms, B.SW2T, ms, Rr, d, ms, Ss, c->part, d, Rd, 0,
                               split ? GemmSeg2{B.SResA, ms, B.SW2T, ms, ms} : GemmSeg2()));
      guard_hn0(B.Hn);
      RUN(TTT_K_RESIDUAL, run_row_in(st, prec, nullptr, srt, V, nullptr, nullptr, nullptr, nullptr, c->part, Ss, Rd,
                                     c->H, Rr, d, nullptr, c->cfg.rms_eps, rms, B.Hn, B.r,
                                     keep_res ? B.ResN : nullptr));
    }
    if (gelu) {
      // Hn^T is read only by the W1 gradient of the backward pass
      if (train && !c->km) check(run_transpose(st, prec, B.Hn, d, Rr, d, B.HnT, Rp));
      // the previous chunk's steps: the lowest block waits for W1's here and for W2's before its
      // down-projection; a higher block's steps finish long before its forward pass, so one
      // wait for W2's (queued after W1's on the aux stream) covers both (each wait costs
      // queue time on the main stream even when it is satisfied)
      check(hipStreamWaitEvent(st, (l > 0 ? B.w2 : B.w1).ev_upd, 0));
      GemmSeg2 s2;
      if (bf) s2 = GemmSeg2{B.Hn, d, B.w1.WtT, d, d};
      // split: the input's residual term against W0 as its own product, added before the GELU
      if (split)
        RUN(TTT_K_UP, gemm_f32(st, prec, B.ResN, d, B.w1.W0T, d, b, m, d, 1, c->Ul, m, 0, 0, GemmSeg2(),
                               fw(b, d, n1, true)));
      RUN(TTT_K_UP, gemm_gelu(st, prec, B.Hn, d, bf ? B.w1.W0T : B.w1.WtT, d, b, m, d, c->km ? B.A : c->A, B.AT, B.GP,
                              keep_res ? B.ResA : nullptr, m, Rp, s2, fw(b, d, n1, bf), split ? c->Ul : nullptr));
    } else {
      RUN(TTT_K_UP, gemm_f32(st, prec, B.Hn, d, B.WgT, d, Rr, m, d, 1, c->UG, m, 0, 0));
      RUN(TTT_K_UP, gemm_swiglu(st, prec, B.Hn, d, B.WuT, d, Rr, m, d, c->UG, foc ? B.VU : nullptr, c->km ? B.A : c->A, B.AT,
                                foc ? B.ResA : nullptr, m, Rp));
    }
    const int S = gemm_split_k(prec, Rr, d, m, bf ? m : 0, SPLIT_MAX);
    if (!gelu || l == 0) check(hipStreamWaitEvent(st, B.w2.ev_upd, 0));  // the previous chunk's step of W2
    GemmSeg2 s2;
    void* const Ablk = c->km ? B.A : c->A;  // this block's activation
    if (bf) s2 = GemmSeg2{Ablk, m, B.w2.WtT, m, m};
    RUN(TTT_K_DOWN, gemm_f32(st, prec, Ablk, m, bf ? B.w2.W0T : B.w2.WtT, m, b, d, m, S, c->part, d, Rd, 0, s2,
                             fw(b, m, n2, bf)));
    int St = S;  // slabs the residual sums
    if (split) {
      // the activation's residual term against W0, as more slabs after the main ones
      const int Sx = gemm_split_k(prec, Rr, d, m, 0, SPLIT_MAX);
      RUN(TTT_K_DOWN, gemm_f32(st, prec, B.ResA, m, B.w2.W0T, m, b, d, m, Sx, c->part + (int64_t)S * Rd, d, Rd, 0,
                               GemmSeg2(), fw(b, m, n2, true)));
      St += Sx;
    }
    // a4 residual, and a2 the next block's pre-norm
    const NormOut o = first_norm(l + 1);
    RUN(TTT_K_RESIDUAL, run_row_in(st, prec, nullptr, srt, V, nullptr, nullptr, nullptr, nullptr, c->part, St, Rd, c->H,
                                   Rr, d, l == L - 1 ? c->Yb : nullptr, c->cfg.rms_eps, rms, o.n, o.r, o.res,
                                   l == L - 1 && split ? c->Yl : nullptr));
  }

  // a5 LM head + CE forward: online softmax over vocabulary records; the numerators are kept
  // for the backward pass (no logits are recomputed)
  RUN(TTT_K_CE_FWD, gemm_ce_partial(st, prec, c->Yb, d, c->E_out, d, Rr, V, d, c->tok_tgt, c->pmax, c->psum, c->pidx,
                                    c->tgt_logit, c->ce_nrec, c->P, V,
                                    c->split ? GemmSeg2{c->Yl, d, c->E_out, d, d} : GemmSeg2()));
  RUN(TTT_K_CE_MERGE, run_ce_merge(st, c->pmax, c->psum, c->pidx, c->ce_nrec, Rr, srl, c->tgt_logit, c->lse,
                                   loss_out, amax_out));

  // an evaluation (no step) runs the backward only for the loss compensation
  if (L > 0 && (train || foc)) {
    // a6 CE backward: dlogits in place from the stored numerators, then dY = P E_out over the
    // whole vocabulary (split-K slabs)
    RUN(TTT_K_CE_PROB, run_ce_dlogits(st, prec, c->P, Rr, V, c->ce_w, c->pmax, c->ce_nrec, c->lse, c->tok_tgt,
                                      1.0f / (float)b));
    const int S2 = gemm_split_k(prec, Rr, d, V, 0, SPLIT_MAX);
    // the backward row buffers of block l (one pair per block with gradients on the aux
    // stream): the gradient at its output, and its dU
    const bool ag = c->agrad && train;
    auto dHbuf = [&](int l) { return ag ? c->dHl[l] : c->dHb; };
    auto dUbuf = [&](int l) { return ag ? c->dUl[l] : c->dU; };
    RUN(TTT_K_CE_DY, gemm_f32(st, prec, c->P, V, c->E_outT, V, Rr, d, V, S2, c->part, d, Rd, 0));
    RUN(TTT_K_DY_SUM, run_dy_finish(st, prec, c->part, S2, Rd, Rr, d, c->dH, dHbuf(L - 1), c->H, c->Yb,
                                    foc ? c->cpart : nullptr));
    // dH^T, read by the W2 gradient
    if (train && !c->km) check(run_transpose(st, prec, c->dHb, d, Rr, d, c->dHT, Rp));

    // a7 block backward, top to bottom
    for (int l = L - 1; l >= 0; --l) {
      Block& B = c->blocks[l];
      float* cA = foc ? c->cpart + (int64_t)B.cslot * Rr : nullptr;        // tnm slots
      float* cN = foc ? c->cpart + (int64_t)(B.cslot + tnm) * Rr : nullptr;  // one slot
      if (gelu) {
        if (ag) {
          // G2 = A^T dH on the aux stream as soon as the gradient at the block's output is in
          check(hipEventRecord(c->ev_gin, st));
          check(hipStreamWaitEvent(c->aux, c->ev_gin, 0));
          RUN_ON(TTT_K_DW, c->aux, gemm_grad_km(c->aux, B.A, m, dHbuf(l), d, m, d, b, B.w2.G, d,
                                                c->slots + B.w2.slot0, gradkm(m, d, c->nslots)));
        }
        RUN(TTT_K_DU, gemm_du(st, prec, dHbuf(l), d, B.w2.Wop, d, b, m, d, B.GP, dUbuf(l), c->km ? nullptr : c->dUT,
                              foc ? B.ResA : nullptr, cA, m, Rp, Rr, fw(b, d, n2, false)));
        if (train) {
          if (ag) {
            // G1 = Hn^T dU on the aux stream once this block's dU is in
            check(hipEventRecord(c->ev_gin, st));
            check(hipStreamWaitEvent(c->aux, c->ev_gin, 0));
            RUN_ON(TTT_K_DW, c->aux, gemm_grad_km(c->aux, B.Hn, d, dUbuf(l), m, d, m, b, B.w1.G, m,
                                                  c->slots + B.w1.slot0, gradkm(d, m, c->nslots)));
            if (l == 0) check(hipEventRecord(c->ev_grad[0], c->aux));
          } else if (c->km) {
            RUN(TTT_K_DW, gemm_grad_km(st, B.A, m, c->dHb, d, m, d, b, B.w2.G, d, c->slots + B.w2.slot0,
                                       gradkm(m, d, c->nslots)));
            RUN(TTT_K_DW, gemm_grad_km(st, B.Hn, d, c->dU, m, d, m, b, B.w1.G, m, c->slots + B.w1.slot0,
                                       gradkm(d, m, c->nslots)));
          } else {
            RUN(TTT_K_DW, gemm_grad(st, prec, B.AT, Rp, c->dHT, Rp, m, d, bp, B.w2.G, d, c->slots + B.w2.slot0,
                                    gradg(c->nslots)));
            RUN(TTT_K_DW, gemm_grad(st, prec, B.HnT, Rp, c->dUT, Rp, d, m, bp, B.w1.G, m, c->slots + B.w1.slot0,
                                    gradg(c->nslots)));
          }
        }
        // Which input gradients this block needs, going down (fast MLP, static MLP,
        // attention): a sublayer's input gradient is needed when a fast block lies below, or
        // a frozen sublayer below it in this block has rounded operands to compensate (bf16);
        // its pre-norm's backward also runs for the compensation of a rounded n (every n but
        // the lowest block's first, E_in[x], when there is no norm).
        const bool has_s = ms > 0, has_a = c->window > 0;
        const bool below_f = l > 0 || (foc && (has_s || has_a));
        const bool first_f = !has_s && !has_a;
        // where the gradients between this block's sublayers go, and the buffer of the one at
        // its input (block l - 1's output; the lowest block's is not written)
        void* const mid = ag ? c->dHm : c->dHb;
        auto to_below = [&]() { return dHbuf(l > 0 ? l - 1 : 0); };
        if (below_f || (foc && (rms || !first_f))) {
          const int S = gemm_split_k(prec, Rr, d, m, 0, SPLIT_MAX);
          RUN(TTT_K_DHN, gemm_f32(st, prec, dUbuf(l), m, B.w1.Wop, m, b, d, m, S, c->part, d, Rd, 0, GemmSeg2(),
                                  fw(b, m, n1, false)));
          if (ag && l == 0) check(hipEventRecord(c->ev_wread, st));
          RUN(TTT_K_NORM_BWD, run_norm_bwd(st, prec, c->part, S, Rd, B.Hn, B.r, Rr, d, rms, c->dH,
                                           first_f ? to_below() : mid, foc ? B.ResN : nullptr, cN, below_f));
        }
        if (ag && l == 0 && !(below_f || (foc && (rms || !first_f)))) check(hipEventRecord(c->ev_wread, st));
        const bool below_s = l > 0 || (foc && has_a);
        if (has_s && below_f) {
          // back through the static MLP (frozen: no weight gradient), once over all rows
          float* cAs = foc ? c->cpart + (int64_t)B.scslot * Rr : nullptr;
          float* cNs = foc ? c->cpart + (int64_t)(B.scslot + c->dot_tiles_s) * Rr : nullptr;
          void* const dUs = ag ? c->dUs : c->dU;  // the fast dU may still be read on the aux stream
          RUN(TTT_K_DU, gemm_du(st, prec, mid, d, B.SW2, d, Rr, ms, d, B.SGP, dUs, nullptr,
                                foc ? B.SResA : nullptr, cAs, ms, 0, Rr));
          if (below_s || (foc && (rms || has_a))) {
            const int Ss = gemm_split_k(prec, Rr, d, ms, 0, SPLIT_MAX);
            RUN(TTT_K_DHN, gemm_f32(st, prec, dUs, ms, B.SW1, ms, Rr, d, ms, Ss, c->part, d, Rd, 0));
            RUN(TTT_K_NORM_BWD, run_norm_bwd(st, prec, c->part, Ss, Rd, B.Sn, B.Sr, Rr, d, rms, c->dH,
                                             has_a ? mid : to_below(), foc ? B.SResN : nullptr, cNs, below_s));
          }
        }
        if (has_a && (has_s ? below_s : below_f)) {
          // back through the attention (frozen): dO = dH Wo^T, with the compensation of the
          // rounded O; then dQ, dK, dV of the chunk's rows and dn = [dQ dK dV] [Wq Wk Wv]^T
          float* cO = foc ? c->cpart + (int64_t)B.acslot * Rr : nullptr;
          float* cNa = foc ? c->cpart + (int64_t)(B.acslot + 1) * Rr : nullptr;
          const int So = gemm_split_k(prec, Rr, d, d, 0, SPLIT_MAX);
          RUN(TTT_K_DHN, gemm_f32(st, prec, mid, d, B.Wo, d, Rr, d, d, So, c->part, d, Rd, 0));
          RUN(TTT_K_NORM_BWD, run_dy_finish(st, prec, c->part, So, Rd, Rr, d, c->dOf, c->dOb, foc ? B.Of : nullptr,
                                            foc ? B.Ob : nullptr, cO));
          if (l > 0 || (foc && rms)) {
            // dK, dV on the aux stream beside dQ: both read only dO, D and the chunk's q, k, v
            const SwaShape sh = swa_shape(c, B, chunk_pos);
            RUN(TTT_K_ATTN_BWD, run_swa_dsum(st, sh, c->dOf, B.Of, c->Dq));
            check(hipEventRecord(c->ev_ain, st));
            check(hipStreamWaitEvent(c->aux, c->ev_ain, 0));
            RUN_ON(TTT_K_ATTN_BWD, c->aux, run_swa_bwd_dkdv(c->aux, sh, c->dOb, B.lse2, c->Dq, c->dQKV, c->swa_part2));
            check(hipEventRecord(c->ev_aout, c->aux));
            RUN(TTT_K_ATTN_BWD, run_swa_bwd_dq(st, sh, c->dOb, B.lse2, c->Dq, c->dQKV, c->swa_part));
            check(hipStreamWaitEvent(st, c->ev_aout, 0));
            const int Sq = gemm_split_k(prec, Rr, d, 3 * d, 0, SPLIT_MAX);
            RUN(TTT_K_DHN, gemm_f32(st, prec, c->dQKV, 3 * d, B.Wqkv, 3 * d, Rr, d, 3 * d, Sq, c->part, d, Rd, 0));
            RUN(TTT_K_NORM_BWD, run_norm_bwd(st, prec, c->part, Sq, Rd, B.Na, B.ra, Rr, d, rms, c->dH, to_below(),
                                             foc ? B.ResNa : nullptr, cNa, l > 0));
          }
        }
        // dH^T at this block's input, read by the W2 gradient of the block below
        if (l > 0 && train && !c->km) check(run_transpose(st, prec, c->dHb, d, Rr, d, c->dHT, Rp));
      } else if (train) {
        if (c->km)
          RUN(TTT_K_DW, gemm_grad_km(st, B.A, m, c->dHb, d, m, d, b, B.w2.G, d, c->slots + B.w2.slot0,
                                     gradkm(m, d, c->nslots)));
        else
          RUN(TTT_K_DW, gemm_grad(st, prec, B.AT, Rp, c->dHT, Rp, m, d, bp, B.w2.G, d, c->slots + B.w2.slot0,
                                  gradg(c->nslots)));
      }
      if (!gelu && foc) {
        // SwiGLU (one block, W2 only fast): dA, then dn = dG Wg^T + dV Wu^T, only to carry
        // the loss compensation of A and n.
        RUN(TTT_K_DU, gemm_swiglu_bwd(st, prec, c->dHb, d, B.w2.Wop, d, b, m, d, c->UG, B.VU, c->DG, c->DV, B.ResA,
                                      cA, m, Rr, fw(b, d, n2, false)));
        if (rms) {
          const int S = gemm_split_k(prec, Rr, d, m, m, SPLIT_MAX);
          GemmSeg2 s2{c->DV, m, B.Wu, m, m};
          RUN(TTT_K_DHN, gemm_f32(st, prec, c->DG, m, B.Wg, m, Rr, d, m, S, c->part, d, Rd, 0, s2));
          RUN(TTT_K_NORM_BWD, run_norm_bwd(st, prec, c->part, S, Rd, B.Hn, B.r, Rr, d, rms, c->dH, c->dHb, B.ResN,
                                           cN, 0));
        }
      }
    }
    if (foc) RUN(TTT_K_CE_MERGE, run_loss_correct(st, c->cpart, c->ncslot, Rr, srl, (float)b, loss_out));
  }
  if (!train) {
    // an evaluated passage's keys and values join its own ring for its next chunk
    for (int l = 0; l < L && c->window > 0; ++l) check(run_kv_append(st, swa_shape(c, c->blocks[l], chunk_pos)));
    return;
  }

  // the chunk's keys and values join each attention ring once nothing reads the old slots
  for (int l = 0; l < L && c->window > 0; ++l) check(run_kv_append(st, swa_shape(c, c->blocks[l], chunk_pos)));

  // a8 global grad norm and clip scale, one per stream, once every gradient is in; a9 update.
  // The step runs on the aux stream, in the order the next chunk's forward pass needs the
  // tensors; each GEMM that reads a fast tensor waits for that tensor's event. (A context
  // with no blocks has no fast tensors.) With the gradients on the aux stream the norm runs
  // there too, right behind them, so no stream hop separates it from the step; the step
  // waits only for the backward's last product on the main stream that reads rn(W0 + D).
  if (c->agrad && !c->fast.empty()) {
    RUN_ON(TTT_K_GRADNORM, c->aux, run_gradnorm(c->aux, c->slots, c->nslots, c->cfg.clip, c->sc,
                                                c->stats + 2 * chunk_idx, 2 * c->max_chunks, nb, c->err));
    check(hipStreamWaitEvent(c->aux, c->ev_wread, 0));
    // the lowest block's W1 gradient reads its normed input, which the next forward pass
    // rewrites: that pass waits for the gradients right before (guard_hn0)
    c->grads_inflight = true;
  } else {
    RUN(TTT_K_GRADNORM, run_gradnorm(st, c->slots, c->nslots, c->cfg.clip, c->sc, c->stats + 2 * chunk_idx,
                                     2 * c->max_chunks, nb, c->err));
    if (!c->fast.empty()) aux_fork(c);
  }
  if (!c->fast.empty()) {
    for (FastTensor* f : c->fast) {
      RUN_ON(TTT_K_UPDATE, c->aux, run_update(c->aux, prec, f->G, f->D, f->W0, f->Wop, f->WtT, f->rows, f->cols,
                                              c->cfg.lr, c->sc, bf ? 1 : 0, nb));
      check(hipEventRecord(f->ev_upd, c->aux));
    }
    aux_mark(c);
  }
}

// Decode of one token ([E2E] Method, decoding; section 3.2): the pair (tok[0], tok[1]) joins
// the pending chunk, and f(tok[0]; W) at the current weights gives the logits of tok[1]'s
// position, its loss and argmax (recorded at c->pos, like a prefilled token's). The fast
// weights are read exactly as the forward GEMMs read them (bf16: W0 and rn(D) as two
// segments); activations stay in fp32.
void decode_token(ttt_ctx* c, const int32_t* tok, int32_t* am_out, float* z_out) {
  hipStream_t st = c->st;
  const int prec = c->prec;
  const int V = c->V, d = c->d, m = c->m, L = c->L;
  const int rms = c->cfg.norm == TTT_NORM_RMS;
  const bool gelu = c->cfg.mlp == TTT_MLP_GELU;
  const bool bf = prec == PREC_BF16;
  const float eps = c->cfg.rms_eps;
  float* z = z_out ? z_out : c->dec_z;
  c->prof_on = c->prof_mask != 0 && (c->prof_chunks++ % c->prof_period) == 0;
  // the first product gathers the token's embedding (and files the pair in the pending chunk)
  GemvIn g0;
  g0.tok = tok;
  g0.first = c->npend == 0;
  g0.pend = c->dec_tok + c->npend;
  g0.E = c->E_in;
  g0.V = V;
  g0.H = c->dec_h;
  g0.err = c->err;
  g0.eps = eps;
  GemvIn gh;  // the residual stream as the activation row
  gh.xin = c->dec_h;
  gh.eps = eps;
  GemvIn ga;  // the block's activation row
  ga.xin = c->dec_a;
  bool gathered = false;  // the first product of the token gathers its embedding
  auto next_in = [&]() {
    GemvIn in = gathered ? gh : g0;
    in.norm = rms;
    gathered = true;
    return in;
  };
  for (int l = 0; l < L; ++l) {
    Block& B = c->blocks[l];
    if (c->window > 0) {
      // the frozen sliding-window attention first: q | k | v of the row, its key and value
      // join the ring at position pos, the attention over the window, the output projection
      RUN(TTT_K_DEC_GEMV, run_gemv(st, prec, GEMV_STORE, next_in(), d, B.WqkvT, nullptr, d, 3 * d, c->dec_qkv));
      RUN(TTT_K_ATTN, run_swa_decode(st, swa_shape(c, B, c->pos), c->dec_qkv, c->dec_part, c->dec_o));
      GemvIn go;
      go.xin = c->dec_o;
      RUN(TTT_K_DEC_GEMV, run_gemv(st, prec, GEMV_RESIDUAL, go, d, B.WoT, nullptr, d, d, c->dec_h));
    }
    if (c->ms > 0) {  // the frozen static MLP first
      RUN(TTT_K_DEC_GEMV, run_gemv(st, prec, GEMV_GELU, next_in(), d, B.SW1T, nullptr, d, c->ms, c->dec_a));
      RUN(TTT_K_DEC_GEMV, run_gemv(st, prec, GEMV_RESIDUAL, ga, c->ms, B.SW2T, nullptr, c->ms, d, c->dec_h));
    }
    GemvIn in = next_in();
    if (gelu)
      RUN(TTT_K_DEC_GEMV, run_gemv(st, prec, GEMV_GELU, in, d, bf ? B.w1.W0T : B.w1.WtT, bf ? B.w1.WtT : nullptr, d, m,
                                   c->dec_a));
    else
      RUN(TTT_K_DEC_GEMV, run_gemv(st, prec, GEMV_SWIGLU, in, d, B.WgT, B.WuT, d, m, c->dec_a));
    RUN(TTT_K_DEC_GEMV, run_gemv(st, prec, GEMV_RESIDUAL, ga, m, bf ? B.w2.W0T : B.w2.WtT, bf ? B.w2.WtT : nullptr, m,
                                 d, c->dec_h));
  }
  GemvIn gz = L == 0 ? g0 : gh;
  gz.rmax = c->dec_rmax;
  gz.rsum = c->dec_rsum;
  gz.ridx = c->dec_ridx;
  RUN(TTT_K_DEC_GEMV, run_gemv(st, prec, GEMV_STORE, gz, d, c->E_out, nullptr, d, V, z));
  check(run_dec_ce(st, z, V, c->dec_rmax, c->dec_rsum, c->dec_ridx, cdiv(V, gemv_rec_rows(V)),
                   c->dec_tok + c->npend + 1, c->losses + c->pos, c->amax + c->pos, am_out));
}

// Losses of a passage q (nq + 1 ids, nq a multiple of b) at the current weights, chunk by
// chunk, without any step; their fp64 sum lands in acc[0], and the losses / their mean in the
// caller's buffers when given.
//
// With attention the passage is a sequence of its own ([SGF], Settlement: the two scores
// leave the attention as it is): its chunks sit at positions 0, b, .. of the passage rings,
// which start empty, and the stream's rings are neither read nor changed.
void evaluate(ttt_ctx* c, const int32_t* q, int64_t nq, double* acc, float* losses, float* mean) {
  const int b = c->b;
  struct PassageRings {
    ttt_ctx* c;
    explicit PassageRings(ttt_ctx* x) : c(x) { c->eval_ring = c->window > 0; }
    ~PassageRings() { c->eval_ring = false; }
  } rings(c);
  for (int64_t i = 0; i < nq; i += b) {
    run_chunk(c, q + i, 0, c->eval_loss, c->eval_amax, b, false, i / b);
    check(run_eval_accum(c->st, c->eval_loss, b, acc, losses ? losses + i : nullptr, i == 0, i + b >= nq, nq,
                         mean));
  }
}

// Where a snapshot of the state a step changes (D, Wop, WtT of every fast tensor) lives.
struct SnapSlots {
  std::vector<char*> D, Wop, WtT;
};

// The context's own snapshot slot (allocated on first use).
SnapSlots ctx_slots(ttt_ctx* c) {
  SnapSlots s;
  for (FastTensor* f : c->fast) {
    const int64_t n = (int64_t)f->rows * f->cols;
    if (!f->snapD) {
      f->snapD = dalloc<char>(c, n * 4);
      f->snapWop = dalloc<char>(c, n * c->es);
      f->snapWtT = dalloc<char>(c, n * c->es);
    }
    s.D.push_back((char*)f->snapD);
    s.Wop.push_back((char*)f->snapWop);
    s.WtT.push_back((char*)f->snapWtT);
  }
  return s;
}

// Copy the state into the slots, or back.
void copy_state(ttt_ctx* c, const SnapSlots& s, bool to_snapshot) {
  aux_join(c);  // no step may still be writing the state
  for (size_t i = 0; i < c->fast.size(); ++i) {
    FastTensor* f = c->fast[i];
    const int64_t n = (int64_t)f->rows * f->cols;
    const hipMemcpyKind k = hipMemcpyDeviceToDevice;
    if (to_snapshot) {
      check(hipMemcpyAsync(s.D[i], f->D, n * 4, k, c->st));
      check(hipMemcpyAsync(s.Wop[i], f->Wop, n * c->es, k, c->st));
      check(hipMemcpyAsync(s.WtT[i], f->WtT, n * c->es, k, c->st));
    } else {
      check(hipMemcpyAsync(f->D, s.D[i], n * 4, k, c->st));
      check(hipMemcpyAsync(f->Wop, s.Wop[i], n * c->es, k, c->st));
      check(hipMemcpyAsync(f->WtT, s.WtT[i], n * c->es, k, c->st));
    }
  }
}

// The Settlement rule ([SGF], Settlement) for one candidate chunk, with the pre-candidate
// state kept in the given slots: L(q, W); snapshot; the candidate chunk scored at W and
// stepped to W + delta as in prefill; L(q, W + delta); A and the decision on the device; the
// slots copied back unless the candidate is kept.
void settle(ttt_ctx* c, const int32_t* tokens, const int32_t* q, int64_t nq, float* A, int32_t* committed,
            const SnapSlots& s) {
  evaluate(c, q, nq, c->eval_acc + 1, nullptr, nullptr);  // L(q, W)
  copy_state(c, s, true);
  run_chunk(c, tokens, 0, c->losses + c->pos, c->amax + c->pos, c->b, true, c->pos / c->b);
  evaluate(c, q, nq, c->eval_acc + 2, nullptr, nullptr);  // L(q, W + delta)
  check(run_settle_decide(c->st, c->eval_acc + 1, nq, c->settle_A, c->settle_commit, A, committed));
  aux_join(c);
  for (size_t i = 0; i < c->fast.size(); ++i) {
    FastTensor* f = c->fast[i];
    const int64_t n = (int64_t)f->rows * f->cols;
    check(run_restore_unless(c->st, c->settle_commit, s.D[i], f->D, n * 4));
    check(run_restore_unless(c->st, c->settle_commit, s.Wop[i], f->Wop, n * c->es));
    check(run_restore_unless(c->st, c->settle_commit, s.WtT[i], f->WtT, n * c->es));
  }
}

// ---- the library's static scratch, for callers that cannot allocate device memory.
// One copy per GPU, alive until the process ends. Host code never uses the array's name
// as an address (on the host it is only a stand-in): the device address comes from
// hipGetSymbolAddress, once per device with that device current, and is kept here.
static __device__ __align__(256) char scratch[TTT_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

ttt_status scratch_address(int dev, char** out) {
  if (dev < 0 || dev >= kMaxDevices) return TTT_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) {
      (void)hipGetLastError();
      return TTT_EDEVICE;
    }
    if (cur != dev && hipSetDevice(dev) != hipSuccess) {
      (void)hipGetLastError();
      return TTT_EDEVICE;
    }
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return TTT_EDEVICE;
    }
    g_scratch_ptr[dev] = (char*)p;
  }
  *out = g_scratch_ptr[dev];
  return TTT_OK;
}

inline int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Bytes of the static scratch a context's Settlement snapshot needs.
int64_t static_settle_bytes(const ttt_ctx* c) {
  int64_t total = 0;
  for (const FastTensor* f : c->fast) {
    const int64_t n = (int64_t)f->rows * f->cols;
    total += align256(n * 4) + 2 * align256(n * c->es);
  }
  return total;
}

ttt_status read_sticky(ttt_ctx* c) {
  int e = 0;
  aux_join(c);  // the grad norm, which may raise the non-finite bit, can run on the aux stream
  check(hipMemcpyAsync(&e, c->err, 4, hipMemcpyDeviceToHost, c->st));
  check(hipStreamSynchronize(c->st));
  if (c->sticky == TTT_OK) {
    if (e & ERRBIT_RANGE) c->sticky = TTT_ERANGE;
    else if (e & ERRBIT_NONFINITE) c->sticky = TTT_ENONFINITE;
  }
  return c->sticky;
}

}  // namespace

extern "C" {

ttt_status ttt_create_ext(const ttt_config* cfg, const ttt_weights* w, const ttt_block_ext* ext, int32_t streams,
                          void* stream, ttt_ctx** out) {
  if (!out) return TTT_EINVAL;
  *out = nullptr;
  ttt_status v = validate(cfg, w);
  if (v != TTT_OK) return v;
  v = validate_ext(cfg, ext);
  if (v != TTT_OK) return v;
  if (streams < 1 || streams > TTT_MAX_STREAMS) return TTT_EINVAL;
  // several streams stack their rows: whole PAD-wide column groups per stream in the
  // transposed buffers, and a bounded row count per step
  if (streams > 1 && (cfg->chunk % PAD || (int64_t)streams * cfg->chunk > ((int64_t)1 << 21))) return TTT_EINVAL;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return TTT_EDEVICE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return TTT_EDEVICE;
  }
  ttt_ctx* c = new (std::nothrow) ttt_ctx();
  if (!c) return TTT_ENOMEM;
  c->cfg = *cfg;
  c->dev = dev;
  c->st = (hipStream_t)stream;
  c->prec = cfg->precision == TTT_BF16 ? PREC_BF16 : PREC_FP32;
  c->es = c->prec == PREC_BF16 ? 2 : 4;
  c->b = cfg->chunk;
  c->bp = (cfg->chunk + PAD - 1) / PAD * PAD;
  c->nb = streams;
  c->R = streams * c->b;
  c->Rp = streams * c->bp;
  c->km = c->prec == PREC_BF16 && c->b % 64 == 0 && c->b <= 1024;
  c->ms = ext ? ext->static_hidden : 0;
  c->window = ext ? ext->swa_window : 0;
  c->agrad = c->km && cfg->mlp == TTT_MLP_GELU;
  // ring positions: the window, plus the b positions a pending decoded chunk writes before
  // its step reads the window in front of it
  c->cr = c->window > 0 ? c->window + c->b : 0;
  c->V = cfg->vocab;
  c->d = cfg->d_model;
  c->m = cfg->d_hidden;
  c->L = cfg->n_blocks;
  // set-up of the static scratch on this device (its address is looked up once per device;
  // the runtime may back the array with memory at that point, so it happens here and not in
  // the entry point that must not allocate); a failure here only resurfaces in that entry point
  {
    char* unused = nullptr;
    (void)scratch_address(dev, &unused);
  }
  try {
    build(c, w, ext);
    check(hipStreamSynchronize(c->st));
  } catch (const HipFail& f) {
    (void)hipStreamSynchronize(c->st);
    release_aux_stream(c);
    free_all(c);
    delete c;
    return f.s;
  } catch (const std::bad_alloc&) {
    (void)hipStreamSynchronize(c->st);
    release_aux_stream(c);
    free_all(c);
    delete c;
    return TTT_ENOMEM;
  }
  *out = c;
  return TTT_OK;
}

ttt_status ttt_create(const ttt_config* cfg, const ttt_weights* w, void* stream, ttt_ctx** out) {
  return ttt_create_ext(cfg, w, nullptr, 1, stream, out);
}

ttt_status ttt_create_batch(const ttt_config* cfg, const ttt_weights* w, int32_t streams, void* stream,
                            ttt_ctx** out) {
  return ttt_create_ext(cfg, w, nullptr, streams, stream, out);
}

int32_t ttt_streams(const ttt_ctx* c) { return c ? c->nb : -1; }

ttt_status ttt_prefill_chunks(ttt_ctx* c, const int32_t* tokens, int64_t n_tokens) {
  if (!c || c->nb != 1) return TTT_EINVAL;
  return ttt_prefill_batch(c, tokens, n_tokens + 1, n_tokens);
}

ttt_status ttt_prefill_batch(ttt_ctx* c, const int32_t* tokens, int64_t ld_tokens, int64_t n_tokens) {
  if (!c || !tokens) return TTT_EINVAL;
  if (c->sticky != TTT_OK) return TTT_ESTATE;
  if (n_tokens <= 0 || n_tokens % c->b || c->npend != 0) return TTT_EINVAL;
  if (c->nb > 1 && ld_tokens < n_tokens + 1) return TTT_EINVAL;
  const int64_t ldtok = c->nb > 1 ? ld_tokens : 0;
  if (c->pos + n_tokens > c->cfg.max_tokens) return TTT_EINVAL;
  try {
    for (int64_t i = 0; i < n_tokens; i += c->b)
      run_chunk(c, tokens + i, ldtok, c->losses + c->pos + i, c->amax + c->pos + i, c->cfg.max_tokens, true,
                (c->pos + i) / c->b);
  } catch (const HipFail& f) {
    c->sticky = f.s;
    return f.s;
  }
  c->pos += n_tokens;
  return TTT_OK;
}

ttt_status ttt_decode(ttt_ctx* c, const int32_t* tokens, int64_t n, int32_t* argmax, float* logits) {
  if (!c || !tokens || n < 0 || c->nb != 1) return TTT_EINVAL;
  if (c->sticky != TTT_OK) return TTT_ESTATE;
  if (c->pos + n > c->cfg.max_tokens) return TTT_EINVAL;
  if (n == 0) return TTT_OK;
  try {
    aux_join(c);  // a step still in flight on the aux stream lands before these predictions
    for (int64_t i = 0; i < n; ++i) {
      decode_token(c, tokens + i, argmax ? argmax + i : nullptr, logits ? logits + i * (int64_t)c->V : nullptr);
      c->pos += 1;
      if (++c->npend == c->b) {
        // the decoded tokens fill a mini-batch: its step, as in prefill ([E2E] section 3.2)
        run_chunk(c, c->dec_tok, 0, c->losses + c->pos - c->b, c->amax + c->pos - c->b, c->b, true,
                  (c->pos - c->b) / c->b);
        c->npend = 0;
        aux_join(c);
      }
    }
  } catch (const HipFail& f) {
    c->sticky = f.s;
    return f.s;
  }
  return TTT_OK;
}

int64_t ttt_decode_pending(const ttt_ctx* c) { return c ? c->npend : -1; }

ttt_status ttt_evaluate(ttt_ctx* c, const int32_t* q, int64_t nq, float* losses, float* mean) {
  if (!c || !q || nq <= 0 || nq % c->b || c->nb != 1) return TTT_EINVAL;
  if (c->sticky != TTT_OK) return TTT_ESTATE;
  try {
    evaluate(c, q, nq, c->eval_acc, losses, mean);
  } catch (const HipFail& f) {
    c->sticky = f.s;
    return f.s;
  }
  return TTT_OK;
}

ttt_status ttt_snapshot(ttt_ctx* c) {
  if (!c || c->nb != 1) return TTT_EINVAL;
  if (c->sticky != TTT_OK) return TTT_ESTATE;
  try {
    copy_state(c, ctx_slots(c), true);
  } catch (const HipFail& f) {
    c->sticky = f.s;
    return f.s;
  }
  c->has_snap = true;
  return TTT_OK;
}

ttt_status ttt_restore(ttt_ctx* c) {
  if (!c || c->nb != 1) return TTT_EINVAL;
  if (c->sticky != TTT_OK || !c->has_snap) return TTT_ESTATE;
  try {
    copy_state(c, ctx_slots(c), false);
  } catch (const HipFail& f) {
    c->sticky = f.s;
    return f.s;
  }
  return TTT_OK;
}

ttt_status ttt_settle_chunk(ttt_ctx* c, const int32_t* tokens, const int32_t* q, int64_t nq, float* A,
                            int32_t* committed) {
  if (!c || !tokens || !q || nq <= 0 || nq % c->b || c->npend != 0 || c->nb != 1) return TTT_EINVAL;
  if (c->sticky != TTT_OK) return TTT_ESTATE;
  if (c->pos + c->b > c->cfg.max_tokens) return TTT_EINVAL;
  try {
    const SnapSlots slots = ctx_slots(c);
    c->has_snap = true;  // the slot holds W from here on (ttt_restore returns to it)
    settle(c, tokens, q, nq, A, committed, slots);
  } catch (const HipFail& f) {
    c->sticky = f.s;
    return f.s;
  }
  c->pos += c->b;
  return TTT_OK;
}

ttt_status ttt_settle_chunk_noalloc(ttt_ctx* c, const int32_t* tokens, const int32_t* q, int64_t nq, float* A,
                                    int32_t* committed) {
  if (!c || !tokens || !q || nq <= 0 || nq % c->b || c->npend != 0 || c->nb != 1) return TTT_EINVAL;
  if (c->sticky != TTT_OK) return TTT_ESTATE;
  if (c->pos + c->b > c->cfg.max_tokens) return TTT_EINVAL;
  if (static_settle_bytes(c) > (int64_t)TTT_STATIC_SCRATCH_BYTES) return TTT_EINVAL;
  char* base = nullptr;
  const ttt_status st = scratch_address(c->dev, &base);
  if (st != TTT_OK) return st;
  SnapSlots slots;
  int64_t off = 0;
  for (const FastTensor* f : c->fast) {
    const int64_t n = (int64_t)f->rows * f->cols;
    slots.D.push_back(base + off);
    off += align256(n * 4);
    slots.Wop.push_back(base + off);
    off += align256(n * c->es);
    slots.WtT.push_back(base + off);
    off += align256(n * c->es);
  }
  try {
    settle(c, tokens, q, nq, A, committed, slots);
  } catch (const HipFail& f) {
    c->sticky = f.s;
    return f.s;
  }
  c->pos += c->b;
  return TTT_OK;
}

ttt_status ttt_sync(ttt_ctx* c) {
  if (!c) return TTT_EINVAL;
  try {
    if (c->aux) check(hipStreamSynchronize(c->aux));
    return read_sticky(c);
  } catch (const HipFail& f) {
    return f.s;
  }
}

static ttt_status copy_record(ttt_ctx* c, void* dst, const void* src, int64_t offset, int64_t n, int64_t limit,
                              int64_t elem) {
  if (!c || (!dst && n > 0) || offset < 0 || n < 0 || offset + n > limit) return TTT_EINVAL;
  try {
    if (n > 0)
      check(hipMemcpyAsync(dst, (const char*)src + offset * elem, n * elem, hipMemcpyDeviceToDevice, c->st));
    return read_sticky(c);
  } catch (const HipFail& f) {
    return f.s;
  }
}

ttt_status ttt_stream_token_losses(ttt_ctx* c, int32_t s, float* dst, int64_t offset, int64_t n) {
  if (!c || s < 0 || s >= c->nb) return TTT_EINVAL;
  return copy_record(c, dst, c->losses + (int64_t)s * c->cfg.max_tokens, offset, n, c->pos, 4);
}

ttt_status ttt_stream_token_argmax(ttt_ctx* c, int32_t s, int32_t* dst, int64_t offset, int64_t n) {
  if (!c || s < 0 || s >= c->nb) return TTT_EINVAL;
  return copy_record(c, dst, c->amax + (int64_t)s * c->cfg.max_tokens, offset, n, c->pos, 4);
}

ttt_status ttt_stream_chunk_stats(ttt_ctx* c, int32_t s, float* dst, int64_t offset, int64_t n) {
  if (!c || s < 0 || s >= c->nb) return TTT_EINVAL;
  if (!dst && n > 0) return TTT_EINVAL;
  if (offset < 0 || n < 0 || offset + n > c->pos / c->b) return TTT_EINVAL;
  try {
    const float* src = c->stats + (int64_t)s * 2 * c->max_chunks + 2 * offset;
    aux_join(c);  // the grad norm that writes them can run on the aux stream
    if (n > 0) check(hipMemcpyAsync(dst, src, n * 8, hipMemcpyDeviceToDevice, c->st));
    return read_sticky(c);
  } catch (const HipFail& f) {
    return f.s;
  }
}

ttt_status ttt_stream_fast_weights(ttt_ctx* c, int32_t s, int32_t block, int32_t which, int32_t kind, float* dst) {
  if (!c || !dst || s < 0 || s >= c->nb || block < 0 || block >= c->L || (kind != 0 && kind != 1))
    return TTT_EINVAL;
  if (which != 1 && which != 2) return TTT_EINVAL;
  if (which == 1 && c->cfg.mlp != TTT_MLP_GELU) return TTT_EINVAL;
  FastTensor& f = which == 1 ? c->blocks[block].w1 : c->blocks[block].w2;
  const int64_t n = (int64_t)f.rows * f.cols;
  try {
    aux_join(c);  // a pending step of the last chunk
    check(run_export(c->st, c->prec, f.D + s * n, f.W0, n, kind, dst));
    return read_sticky(c);
  } catch (const HipFail& e) {
    return e.s;
  }
}

ttt_status ttt_token_losses(ttt_ctx* c, float* dst, int64_t offset, int64_t n) {
  return ttt_stream_token_losses(c, 0, dst, offset, n);
}

ttt_status ttt_token_argmax(ttt_ctx* c, int32_t* dst, int64_t offset, int64_t n) {
  return ttt_stream_token_argmax(c, 0, dst, offset, n);
}

ttt_status ttt_chunk_stats(ttt_ctx* c, float* dst, int64_t offset, int64_t n) {
  return ttt_stream_chunk_stats(c, 0, dst, offset, n);
}

ttt_status ttt_fast_weights(ttt_ctx* c, int32_t block, int32_t which, int32_t kind, float* dst) {
  return ttt_stream_fast_weights(c, 0, block, which, kind, dst);
}

ttt_status ttt_reset(ttt_ctx* c) {
  if (!c) return TTT_EINVAL;
  try {
    aux_join(c);  // no pending step may land after the reset
    for (FastTensor* f : c->fast) reset_fast(c, *f);
    check(run_fill_u32(c->st, c->err, 1, 0u));
  } catch (const HipFail& f) {
    return f.s;
  }
  c->pos = 0;
  c->npend = 0;
  c->sticky = TTT_OK;
  return TTT_OK;
}

int64_t ttt_tokens_consumed(const ttt_ctx* c) { return c ? c->pos : -1; }

ttt_status ttt_profile_enable(ttt_ctx* c, uint32_t mask) {
  if (!c || (mask >> TTT_K_COUNT) != 0) return TTT_EINVAL;
  c->prof_mask = mask;
  c->prof_chunks = 0;
  return TTT_OK;
}

ttt_status ttt_profile_period(ttt_ctx* c, int32_t period) {
  if (!c || period < 1) return TTT_EINVAL;
  c->prof_period = period;
  c->prof_chunks = 0;
  return TTT_OK;
}

ttt_status ttt_profile_read(ttt_ctx* c, double* total_ms, int64_t* launches) {
  if (!c || !total_ms || !launches) return TTT_EINVAL;
  for (int k = 0; k < TTT_K_COUNT; ++k) {
    total_ms[k] = 0.0;
    launches[k] = 0;
  }
  try {
    check(hipStreamSynchronize(c->st));
    if (c->aux) check(hipStreamSynchronize(c->aux));  // the SGD steps are traced on the aux stream
    for (size_t p = 0; p < c->ev_kind.size(); ++p) {
      float ms = 0.f;
      check(hipEventElapsedTime(&ms, c->ev_pool[2 * p], c->ev_pool[2 * p + 1]));
      total_ms[c->ev_kind[p]] += ms;
      launches[c->ev_kind[p]] += 1;
    }
  } catch (const HipFail& f) {
    return f.s;
  }
  c->ev_used = 0;
  c->ev_kind.clear();
  return TTT_OK;
}

ttt_status ttt_destroy(ttt_ctx* c) {
  if (!c) return TTT_OK;
  (void)hipStreamSynchronize(c->st);
  release_aux_stream(c);
  for (hipEvent_t e : c->ev_pool) (void)hipEventDestroy(e);
  free_all(c);
  delete c;
  return TTT_OK;
}

const char* ttt_status_string(ttt_status s) {
  switch (s) {
    case TTT_OK: return "ok";
    case TTT_EINVAL: return "invalid argument or configuration";
    case TTT_ENOMEM: return "device out of memory";
    case TTT_EDEVICE: return "HIP device or runtime error";
    case TTT_ERANGE: return "token id out of range";
    case TTT_ENONFINITE: return "non-finite gradient norm (update skipped)";
    case TTT_ESTATE: return "context holds a sticky error";
  }
  return "unknown status";
}

ttt_status ttt_test_gemm(int32_t precision, const void* X, int64_t ldx, const void* Y, int64_t ldy, float* C,
                         int64_t ldc, int32_t M, int32_t N, int32_t K, void* stream) {
  if (precision != TTT_FP32 && precision != TTT_BF16) return TTT_EINVAL;
  if (!X || !Y || !C || M < 0 || N < 0 || K < 0) return TTT_EINVAL;
  const int kc = precision == TTT_BF16 ? 8 : 4;
  if (K % kc || ldx % kc || ldy % kc || ldx < K || ldy < K || ldc < N) return TTT_EINVAL;
  const int prec = precision == TTT_BF16 ? PREC_BF16 : PREC_FP32;
  hipError_t e = gemm_f32((hipStream_t)stream, prec, X, ldx, Y, ldy, M, N, K, 1, C, ldc, 0, 0);
  return e == hipSuccess ? TTT_OK : TTT_EDEVICE;
}

ttt_status ttt_test_gemm_pair(const void* X, int64_t ldx, const void* Y, int64_t ldy, const void* Y2, int64_t ldy2,
                              float* C, int64_t ldc, int32_t M, int32_t N, int32_t K, int32_t splits, int32_t form,
                              void* stream) {
  if (!X || !Y || !Y2 || !C || M < 0 || N < 0 || K < 0 || splits < 1 || splits > SPLIT_MAX) return TTT_EINVAL;
  if (K % 8 || ldx % 8 || ldy % 8 || ldy2 % 8 || ldx < K || ldy < K || ldy2 < K || ldc < N) return TTT_EINVAL;
  if (form < 0 || form > 2) return TTT_EINVAL;
  const hipError_t e = gemm_f32((hipStream_t)stream, PREC_BF16, X, ldx, Y, ldy, M, N, K, splits, C, ldc,
                                (int64_t)M * ldc, 0, GemmSeg2{X, ldx, Y2, ldy2, K, form - 1});
  return e == hipSuccess ? TTT_OK : TTT_EDEVICE;
}

ttt_status ttt_test_grad(const void* X, int64_t ldx, const void* Y, int64_t ldy, void* G, int64_t ldg, float* slots,
                         int32_t M, int32_t N, int32_t K, int32_t token_major, void* stream) {
  if (!X || !Y || !G || !slots || M <= 0 || N <= 0 || K <= 0 || K % 64 || ldg < N || ldg % 8) return TTT_EINVAL;
  if (token_major != 0 && token_major != 1) return TTT_EINVAL;
  if (token_major) {
    if (M % 8 || N % 8 || ldx < M || ldy < N || ldx % 8 || ldy % 8) return TTT_EINVAL;
  } else if (ldx < K || ldy < K || ldx % 8 || ldy % 8) {
    return TTT_EINVAL;
  }
  hipStream_t st = (hipStream_t)stream;
  const hipError_t e = token_major ? gemm_grad_km(st, X, ldx, Y, ldy, M, N, K, G, ldg, slots)
                                   : gemm_grad(st, PREC_BF16, X, ldx, Y, ldy, M, N, K, G, ldg, slots);
  return e == hipSuccess ? TTT_OK : e == hipErrorInvalidValue ? TTT_EINVAL : TTT_EDEVICE;
}

}  // extern "C"
