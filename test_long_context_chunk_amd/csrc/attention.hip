// Frozen sliding-window attention of a TTT'd block ([E2E] section 3): per head of 128,
// softmax(q.k / sqrt(128)) over the keys of the last `window` positions up to the query's
// own, o = sum p v. The keys and values of positions before the chunk come from a ring of
// `cr` positions per stream (written by k_kv_append after the chunk's step); the chunk's own
// come from the QKV product of this chunk. q, k and v are held in two 16-bit forms: half
// precision (11 significant bits) for the forward and decode, bf16 for the backward. Three
// MFMA kernels:
//   k_swa_fwd      online-softmax forward in half precision: O (fp32 and bf16) and the
//                  log-sum-exp per query;
//   k_swa_bwd_dq   dQ over every key a query sees (cached keys included), bf16;
//   k_swa_bwd_dkdv dK, dV of the chunk's own keys (cached keys are constants), bf16.
// Each lane of a wave owns one query (forward, dQ) or one key (dK/dV) as the column of
// 16 x 16 x 32 MFMA blocks; the probabilities never leave registers: the products that
// contract over them take them as the B operand in the k-slot order they already have, and
// read the other operand from LDS in that same order. Each pass can divide its range among
// several workgroups (k_swa_merge, k_swa_dq_sum and k_swa_dkdv_sum combine the partials in
// a fixed order). Decoding one row: k_swa_dec files its key and value and attends over the
// window in fp32 (keys and values read in half precision), k_swa_dec_merge combines its shares.
#include "launchers.h"
#include "common.h"

namespace {

constexpr int DH = 128;      // head size
constexpr int BLK = 64;      // queries or keys per workgroup and per staged block
constexpr int SPLIT_CAP = 16;  // most workgroups one query block's key range is divided among
constexpr int NT_A = 256;    // 4 waves x 16 rows
constexpr int LDR = DH + 8;  // row stride (elements) of a [row][dim] tile: 272 B
constexpr int LDT = BLK + 8; // row stride of a [dim][row] tile: 144 B (conflict-free pair stores)

struct SwaGeo {
  const bf16_t* qkv;  // [R x 3d] q | k | v of the chunk's rows (stream z: rows z b ..), bf16
  const bf16_t* kc;   // key ring [nb][cr x d]: position p at slot p % cr, bf16
  const bf16_t* vc;
  const f16_t* qkv16;  // the same three in half precision (the forward's operands)
  const f16_t* kc16;
  const f16_t* vc16;
  int cr, b, d, window;
  int64_t pos;        // position of the chunk's first row
};

// Where the rows of one key block [kb, kb + BLK) come from, with 32-bit per-row arithmetic:
// the first nr rows from the ring (slot s0 + r, wrapping at cr), the others from the chunk's
// own rows (chunk row c0 + r - nr); rows past `last` (block-relative) lie beyond the range.
struct KeySrc {
  int nr, s0, c0, last;
};
__device__ __forceinline__ KeySrc key_src(const SwaGeo& g, int64_t kb, int64_t khi) {
  KeySrc k;
  const int64_t before = g.pos - kb;
  k.nr = before <= 0 ? 0 : (before >= BLK ? BLK : (int)before);
  k.s0 = k.nr > 0 ? (int)(kb % g.cr) : 0;
  k.c0 = (int)(kb + k.nr - g.pos);
  const int64_t l = khi - kb;
  k.last = l >= BLK ? BLK - 1 : (int)l;
  return k;
}

// Staging through registers: a block of BLK rows is 1024 16-byte chunks, four per thread.
// All four are requested before any is stored, and a loop requests the next block's chunks
// before computing on the current one, so global latency overlaps the MFMAs.
constexpr int CPT = BLK * (DH / 8) / NT_A;  // chunks per thread per tile
struct Chunks {
  uint4 v[CPT];
};
// Blocks that also go into a [dim][row] tile are fetched as row pairs: chunk i of a thread is
// row 2 p + (i % 2), p = lane-in-32, at 16-byte column (t / 32) + 8 (i / 2). A pair gives one
// 4-byte word per dim, and the 64 lanes of a wave store to 64 distinct banks (row stride 72).
template <class Src>
__device__ __forceinline__ void fetch_p(Chunks& R, Src src) {
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int p = threadIdx.x & 31, c = ((threadIdx.x >> 5) + 8 * (i >> 1)) * 8;
    const bf16_t* s = src(2 * p + (i & 1));
    R.v[i] = s ? *(const uint4*)(s + c) : make_uint4(0, 0, 0, 0);
  }
}
__device__ __forceinline__ void put_p(const Chunks& R, bf16_t* tile, bf16_t* T) {
#pragma unroll
  for (int ip = 0; ip < CPT / 2; ++ip) {
    const int p = threadIdx.x & 31, c = ((threadIdx.x >> 5) + 8 * ip) * 8;
    const uint4 a = R.v[2 * ip], b = R.v[2 * ip + 1];
    if (tile) {
      *(uint4*)(tile + (2 * p) * LDR + c) = a;
      *(uint4*)(tile + (2 * p + 1) * LDR + c) = b;
    }
    if (!T) continue;
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // dims c + 2q (low halves) and c + 2q + 1 (high halves) of rows 2p, 2p + 1
      *(uint32_t*)(T + (c + 2 * q) * LDT + 2 * p) = __builtin_amdgcn_perm(wb[q], wa[q], 0x05040100u);
      *(uint32_t*)(T + (c + 2 * q + 1) * LDT + 2 * p) = __builtin_amdgcn_perm(wb[q], wa[q], 0x07060302u);
    }
  }
}

// Key-block fetch in the row-pair layout of fetch_p for several tiles at once (keys or
// values, bf16 or half). Each tile's base pointers for the workgroup's stream and head are
// set up once (uniform over the workgroup); per block a thread resolves its two rows (ring
// slot or chunk row, plus its 16-byte column) once and reads every tile from them. Rows past the block's last
// key repeat that key: its scores are masked and its probabilities are zero, so the values
// only have to be finite.
struct KvBase {
  const uint16_t* ring;   // slot 0 of the stream's ring
  const uint16_t* chunk;  // row 0 of the stream's chunk rows (q | k | v)
};
__device__ __forceinline__ KvBase kv_base(const SwaGeo& g, int z, int h, int which, bool half) {
  const uint16_t* ring = which == 1 ? (half ? g.kc16 : g.kc) : (half ? g.vc16 : g.vc);
  KvBase b;
  b.ring = ring + (int64_t)z * g.cr * g.d + h * DH;
  b.chunk = (half ? g.qkv16 : g.qkv) + (int64_t)z * g.b * (3 * (int64_t)g.d) + (int64_t)which * g.d + h * DH;
  return b;
}
template <int NTL>
__device__ __forceinline__ void fetch_rows(Chunks (&R)[NTL], const KvBase (&B)[NTL], const SwaGeo& g,
                                           const KeySrc& ks) {
  const int p = threadIdx.x & 31, col = (threadIdx.x >> 5) * 8;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int r = min(2 * p + a, ks.last);
    const bool ring = r < ks.nr;
    int slot = ks.s0 + r;  // used for ring rows only: then below 2 cr
    if (slot >= g.cr) slot -= g.cr;
    const int64_t ro = (int64_t)slot * g.d + col;
    const int64_t co = (int64_t)(ks.c0 + r - ks.nr) * (3 * (int64_t)g.d) + col;
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
      const uint16_t* src = ring ? B[t].ring + ro : B[t].chunk + co;
      R[t].v[a] = *(const uint4*)src;
      R[t].v[2 + a] = *(const uint4*)(src + 64);
    }
  }
}

// A operand chunk from a [dim][row] tile: row dim, rows {32t + 4g .. +3, 32t + 16 + 4g .. +3}
// (the k-slot order of an accumulator pair held by lane group g).
__device__ __forceinline__ uint4 tchunk(const bf16_t* T, int dim, int t, int g) {
  const uint2 lo = *(const uint2*)(T + dim * LDT + 32 * t + 4 * g);
  const uint2 hi = *(const uint2*)(T + dim * LDT + 32 * t + 16 + 4 * g);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// B operand chunk from two accumulator blocks (4 values each) in that same slot order.
__device__ __forceinline__ uint4 pchunk(const f32x4_t& a, const f32x4_t& b) {
  return make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]));
}
__device__ __forceinline__ uint4 pchunk_f16(const f32x4_t& a, const f32x4_t& b) {
  return make_uint4(pack_f16x2(a[0], a[1]), pack_f16x2(a[2], a[3]), pack_f16x2(b[0], b[1]), pack_f16x2(b[2], b[3]));
}

constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------------------- forward
// grid (ceil(b / 64), H, streams). Outputs O fp32 and bf16 [R x d] (head h in columns
// 128 h ..), lse2 [streams][H][b] = log2 of the softmax denominator in units of the scaled
// logits s log2(e) / sqrt(128). q, k, v and p enter in half precision (relative rounding
// 2^-12, an eighth of bf16's), one MFMA per 32-k step of each product, fp32 accumulation.
// With nsplit > 1 the key blocks of each query block are divided among nsplit workgroups
// (blockIdx.x = query block * nsplit + split), each leaving its unnormalised partial O and its
// (max, sum) in part / pm / pl for k_swa_merge.
struct SwaSplit {
  int n;        // workgroups per query block
  float* part;  // [n][R x d] partial O (scaled by 2^-max)
  float* pm;    // [n][streams][H][b] running max (scaled base-2 units)
  float* pl;    // [n][streams][H][b] sum of 2^(s - max)
};

// QG query groups of 16 per wave (a workgroup covers 64 QG queries): every K and V operand
// read from LDS feeds QG products, so a larger QG moves fewer tile bytes per query.
template <int QG>
__global__ void __launch_bounds__(NT_A, 2) k_swa_fwd(SwaGeo g, SwaSplit sp, float* __restrict__ Of,
                                                                   bf16_t* __restrict__ Ob, bf16_t* __restrict__ Ol,
                                                                   float* __restrict__ lse2) {
  __shared__ __attribute__((aligned(16))) f16_t sK[BLK * LDR];
  __shared__ __attribute__((aligned(16))) f16_t sVt[DH * LDT];
  constexpr int QB = BLK * QG;  // queries per workgroup
  const int z = blockIdx.z, h = blockIdx.y, H = gridDim.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int split = blockIdx.x % sp.n;
  const int q0 = (blockIdx.x / sp.n) * QB;
  const float sc = LOG2E * 0.08838834764831845f;  // log2(e) / sqrt(128)

  // this lane's queries (chunk rows q0 + 16 (QG wave + gq) + lr) as B-operand chunks (dims
  // 32 s + 8 lg ..), and their running O, max and sum
  int q[QG];
  bool qok[QG];
  uint4 qf[QG][4];
  f32x4_t ot[QG][8];
  float m[QG], lsum[QG];
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    q[gq] = q0 + 16 * (QG * wave + gq) + lr;
    qok[gq] = q[gq] < g.b;
    const int64_t o = ((int64_t)z * g.b + (qok[gq] ? q[gq] : 0)) * (3 * (int64_t)g.d) + h * DH;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qf[gq][s] = qok[gq] ? *(const uint4*)(g.qkv16 + o + 32 * s + 8 * lg) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) ot[gq][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m[gq] = -INFINITY;
    lsum[gq] = 0.f;
  }

  const int64_t qlo = g.pos + q0, qhi = g.pos + min(q0 + QB, g.b) - 1;
  int64_t klo = qlo - g.window + 1;
  if (klo < 0) klo = 0;
  // this workgroup's share of the key blocks [klo, qhi]
  int64_t kend = qhi;
  if (sp.n > 1) {
    const int64_t nblk = (qhi - klo) / BLK + 1;
    const int64_t b0 = nblk * split / sp.n, b1 = nblk * (split + 1) / sp.n;
    kend = min(qhi, klo + b1 * BLK - 1);
    klo += b0 * BLK;
  }
  Chunks cb[2];  // K, V (half precision)
  const KvBase kvb[2] = {kv_base(g, z, h, 1, true), kv_base(g, z, h, 2, true)};
  auto fetch_block = [&](int64_t kb) { fetch_rows<2>(cb, kvb, g, key_src(g, kb, qhi)); };
  // the wave's first query position (its 16 QG queries follow)
  const int64_t qw0 = g.pos + q0 + 16 * QG * wave;
  if (klo <= kend) fetch_block(klo);
  for (int64_t kb = klo; kb <= kend; kb += BLK) {
    __syncthreads();  // the previous block's tiles are no longer read
    put_p(cb[0], sK, nullptr);
    put_p(cb[1], nullptr, sVt);
    __syncthreads();
    if (kb + BLK <= kend) fetch_block(kb + BLK);  // in flight during this block's MFMAs

    // S^T = K Q^T: st[gq][j][e] = s(key kb + 16 j + 4 lg + e, query q[gq])
    f32x4_t st[QG][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int gq = 0; gq < QG; ++gq) st[gq][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 a = *(const uint4*)(sK + (16 * j + lr) * LDR + 32 * s + 8 * lg);
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) mfma_chunk_f16(st[gq][j], a, qf[gq][s]);
      }
    }
    // mask (distance query - key in [0, window), 32-bit) and block max (scaled units); a
    // block that every query of the wave sees whole needs no mask
    const bool whole = qw0 - (kb + BLK - 1) >= 0 && qw0 + 16 * QG - 1 - kb < g.window;
    uint4 pb[QG][2];
#pragma unroll
    for (int gq = 0; gq < QG; ++gq) {
      float bm = -INFINITY;
      if (whole) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            st[gq][j][e] *= sc;
            bm = fmaxf(bm, st[gq][j][e]);
          }
      } else {
        const int dq0 = qok[gq] ? (int)(g.pos + q[gq] - kb) - 4 * lg : -(1 << 30);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int dist = dq0 - 16 * j - e;
            const bool ok = dist >= 0 && dist < g.window;
            st[gq][j][e] = ok ? st[gq][j][e] * sc : -INFINITY;
            bm = fmaxf(bm, st[gq][j][e]);
          }
      }
      bm = fmaxf(bm, __shfl_xor(bm, 16, TTT_WAVE));
      bm = fmaxf(bm, __shfl_xor(bm, 32, TTT_WAVE));
      // online softmax; a query with no visible key yet keeps m = -inf and adds zeros (no
      // branch: the MFMAs below run for the whole wave)
      const float mn = fmaxf(m[gq], bm);
      const float alpha =
          (m[gq] == -INFINITY || mn == -INFINITY) ? (m[gq] == mn ? 1.f : 0.f) : __builtin_amdgcn_exp2f(m[gq] - mn);
      m[gq] = mn;
      lsum[gq] *= alpha;
      if (__any(alpha != 1.f)) {  // once the maxima settle, most blocks leave O as it is
#pragma unroll
        for (int c = 0; c < 8; ++c) ot[gq][c] *= alpha;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = st[gq][j][e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st[gq][j][e] - mn);
          st[gq][j][e] = p;
          lsum[gq] += p;
        }
      // p (at most 1) as half-precision B operands, in the k-slot order of tchunk
#pragma unroll
      for (int t = 0; t < 2; ++t) pb[gq][t] = pchunk_f16(st[gq][2 * t], st[gq][2 * t + 1]);
    }
    // O^T += V^T P^T: ot[gq][c][e] = o(dim 16 c + 4 lg + e, query q[gq])
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 vh = tchunk(sVt, 16 * c + lr, t, lg);
#pragma unroll
        for (int gq = 0; gq < QG; ++gq) mfma_chunk_f16(ot[gq][c], vh, pb[gq][t]);
      }
    }
  }
#pragma unroll
  for (int gq = 0; gq < QG; ++gq) {
    float ls = lsum[gq];
    ls += __shfl_xor(ls, 16, TTT_WAVE);
    ls += __shfl_xor(ls, 32, TTT_WAVE);
    if (!qok[gq]) continue;
    const int64_t row = (int64_t)z * g.b + q[gq];
    if (sp.n > 1) {
      // partial state: O unnormalised, its max and sum
      float* P = sp.part + (int64_t)split * ((int64_t)gridDim.z * g.b) * g.d;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *(float4*)(P + row * g.d + h * DH + 16 * c + 4 * lg) =
            make_float4(ot[gq][c][0], ot[gq][c][1], ot[gq][c][2], ot[gq][c][3]);
      if (lg == 0) {
        const int64_t o = ((int64_t)split * gridDim.z * H + (int64_t)z * H + h) * g.b + q[gq];
        sp.pm[o] = m[gq];
        sp.pl[o] = ls;
      }
      continue;
    }
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int col = h * DH + 16 * c + 4 * lg;
      const float4 o = make_float4(ot[gq][c][0] * inv, ot[gq][c][1] * inv, ot[gq][c][2] * inv, ot[gq][c][3] * inv);
      *(float4*)(Of + row * g.d + col) = o;
      const uint2 hb = make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
      *(uint2*)(Ob + row * g.d + col) = hb;
      const bf16_t* hv = (const bf16_t*)&hb;
      *(uint2*)(Ol + row * g.d + col) = make_uint2(pack_bf16x2(o.x - bf2f(hv[0]), o.y - bf2f(hv[1])),
                                                   pack_bf16x2(o.z - bf2f(hv[2]), o.w - bf2f(hv[3])));
    }
    if (lg == 0) lse2[((int64_t)z * H + h) * g.b + q[gq]] = m[gq] + log2f(ls);
  }
}

// Merge of the split partial states: grid (streams b rows, H), 64 threads x 2 dims.
__global__ void __launch_bounds__(64) k_swa_merge(SwaSplit sp, int b, int d, float* __restrict__ Of,
                                                  bf16_t* __restrict__ Ob, bf16_t* __restrict__ Ol,
                                                  float* __restrict__ lse2) {
  const int64_t row = blockIdx.x;
  const int h = blockIdx.y, H = gridDim.y;
  const int64_t R = (int64_t)gridDim.x;
  const int z = (int)(row / b), q = (int)(row - (int64_t)z * b);
  const int64_t nz = R / b;
  float M = -INFINITY;
  for (int s = 0; s < sp.n; ++s) M = fmaxf(M, sp.pm[((int64_t)s * nz * H + (int64_t)z * H + h) * b + q]);
  float L = 0.f, o0 = 0.f, o1 = 0.f;
  const int64_t col = (int64_t)h * DH + 2 * threadIdx.x;
  for (int s = 0; s < sp.n; ++s) {
    const int64_t i = ((int64_t)s * nz * H + (int64_t)z * H + h) * b + q;
    const float ms = sp.pm[i];
    const float w = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    L += w * sp.pl[i];
    const float2 pv = *(const float2*)(sp.part + (int64_t)s * R * d + row * d + col);
    o0 += w * pv.x;
    o1 += w * pv.y;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  o0 *= inv;
  o1 *= inv;
  *(float2*)(Of + row * d + col) = make_float2(o0, o1);
  const uint32_t hb = pack_bf16x2(o0, o1);
  *(uint32_t*)(Ob + row * d + col) = hb;
  const bf16_t* hv = (const bf16_t*)&hb;
  *(uint32_t*)(Ol + row * d + col) = pack_bf16x2(o0 - bf2f(hv[0]), o1 - bf2f(hv[1]));
  if (threadIdx.x == 0) lse2[((int64_t)z * H + h) * b + q] = M + log2f(L);
}

// ---------------------------------------------------------------------------- backward
// Dq[z][h][q] = sum over the head's dims of dO * O (the row term of the softmax backward).
__global__ void __launch_bounds__(64) k_swa_dsum(const float* __restrict__ dO, const float* __restrict__ O, int d,
                                                 int b, float* __restrict__ Dq) {
  const int row = blockIdx.x, h = blockIdx.y, H = gridDim.y;
  const int64_t o = (int64_t)row * d + h * DH + 2 * threadIdx.x;
  float v = dO[o] * O[o] + dO[o + 1] * O[o + 1];
  v = wave_sum(v);
  if (threadIdx.x == 0) {
    const int z = row / b, q = row - z * b;
    Dq[((int64_t)z * H + h) * b + q] = v;
  }
}

// dQ: grid (ceil(b / 64), H, streams). dQ = (1 / sqrt(128)) sum_key dS K with
// dS = P (dP - D), P recomputed from the stored lse2; written (bf16) into columns 128 h ..
// of dQKV [R x 3d].
// With nsplit > 1 (blockIdx.x = query block * nsplit + split) each workgroup takes a share of
// the key blocks and writes its fp32 partial dQ into part[split]; k_swa_dq_sum adds them in
// split order.
__global__ void __launch_bounds__(NT_A) k_swa_bwd_dq(SwaGeo g, int nsplit, float* __restrict__ part,
                                                     const bf16_t* __restrict__ dOb, const float* __restrict__ lse2,
                                                     const float* __restrict__ Dq, bf16_t* __restrict__ dQKV) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[BLK * LDR];
  __shared__ __attribute__((aligned(16))) bf16_t sV[BLK * LDR];
  __shared__ __attribute__((aligned(16))) bf16_t sKt[DH * LDT];
  const int z = blockIdx.z, h = blockIdx.y, H = gridDim.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int split = blockIdx.x % nsplit;
  const int q0 = (blockIdx.x / nsplit) * BLK;
  const int q = q0 + wave * 16 + lr;
  const bool qok = q < g.b;
  const int64_t qp = g.pos + q;
  const float sc = LOG2E * 0.08838834764831845f;
  const int64_t row = (int64_t)z * g.b + (qok ? q : 0);

  uint4 qf[4], df[4];
  {
    const bf16_t* qr = g.qkv + row * (3 * (int64_t)g.d) + h * DH;
    const bf16_t* dr = dOb + row * g.d + h * DH;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qf[s] = qok ? *(const uint4*)(qr + 32 * s + 8 * lg) : make_uint4(0, 0, 0, 0);
      df[s] = qok ? *(const uint4*)(dr + 32 * s + 8 * lg) : make_uint4(0, 0, 0, 0);
    }
  }
  const float L2 = qok ? lse2[((int64_t)z * H + h) * g.b + q] : 0.f;
  const float Dv = qok ? Dq[((int64_t)z * H + h) * g.b + q] : 0.f;
  f32x4_t dq[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) dq[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t qlo = g.pos + q0, qhi = g.pos + min(q0 + BLK, g.b) - 1;
  int64_t klo = qlo - g.window + 1;
  if (klo < 0) klo = 0;
  int64_t kend = qhi;
  if (nsplit > 1) {
    const int64_t nblk = (qhi - klo) / BLK + 1;
    const int64_t b0 = nblk * split / nsplit, b1 = nblk * (split + 1) / nsplit;
    kend = min(qhi, klo + b1 * BLK - 1);
    klo += b0 * BLK;
  }
  Chunks cb[2];  // K, V
  const KvBase kvb[2] = {kv_base(g, z, h, 1, false), kv_base(g, z, h, 2, false)};
  auto fetch_block = [&](int64_t kb) { fetch_rows<2>(cb, kvb, g, key_src(g, kb, qhi)); };
  const int64_t qw0 = g.pos + q0 + wave * 16;
  if (klo <= kend) fetch_block(klo);
  for (int64_t kb = klo; kb <= kend; kb += BLK) {
    __syncthreads();
    put_p(cb[0], sK, sKt);
    put_p(cb[1], sV, nullptr);
    __syncthreads();
    if (kb + BLK <= kend) fetch_block(kb + BLK);
    f32x4_t st[4], dp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      st[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      dp[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        mfma_chunk(st[j], *(const uint4*)(sK + (16 * j + lr) * LDR + 32 * s + 8 * lg), qf[s], bf16_t());
        mfma_chunk(dp[j], *(const uint4*)(sV + (16 * j + lr) * LDR + 32 * s + 8 * lg), df[s], bf16_t());
      }
    }
    // dS = P (dP - D), P = exp2(s sc - lse2) on the window, 0 elsewhere (no mask for a
    // block every query of the wave sees whole)
    if (qw0 - (kb + BLK - 1) >= 0 && qw0 + 15 - kb < g.window) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) st[j][e] = __builtin_amdgcn_exp2f(st[j][e] * sc - L2) * (dp[j][e] - Dv);
    } else {
      const int dq0 = qok ? (int)(qp - kb) - 4 * lg : -(1 << 30);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dist = dq0 - 16 * j - e;
          const bool ok = dist >= 0 && dist < g.window;
          const float p = ok ? __builtin_amdgcn_exp2f(st[j][e] * sc - L2) : 0.f;
          st[j][e] = p * (dp[j][e] - Dv);
        }
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint4 sb = pchunk(st[2 * t], st[2 * t + 1]);
#pragma unroll
      for (int c = 0; c < 8; ++c) mfma_chunk(dq[c], tchunk(sKt, 16 * c + lr, t, lg), sb, bf16_t());
    }
  }
  if (!qok) return;
  const float rs = 0.08838834764831845f;
  if (nsplit > 1) {
    float* P = part + ((int64_t)split * gridDim.z * g.b + (int64_t)z * g.b + q) * g.d + h * DH;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      *(float4*)(P + 16 * c + 4 * lg) = make_float4(dq[c][0] * rs, dq[c][1] * rs, dq[c][2] * rs, dq[c][3] * rs);
    return;
  }
  bf16_t* out = dQKV + ((int64_t)z * g.b + q) * (3 * (int64_t)g.d) + h * DH;
#pragma unroll
  for (int c = 0; c < 8; ++c)
    *(uint2*)(out + 16 * c + 4 * lg) =
        make_uint2(pack_bf16x2(dq[c][0] * rs, dq[c][1] * rs), pack_bf16x2(dq[c][2] * rs, dq[c][3] * rs));
}

// dQ = sum of the split partials in split order, into columns 0 .. d of dQKV (bf16):
// grid (streams b rows), 256 threads x 8 columns.
__global__ void __launch_bounds__(NT_A) k_swa_dq_sum(const float* __restrict__ part, int nsplit, int d,
                                                     bf16_t* __restrict__ dQKV) {
  const int64_t row = blockIdx.x, R = gridDim.x;
  for (int c = threadIdx.x * 8; c < d; c += NT_A * 8) {
    float acc[8];
    const float4 a0 = *(const float4*)(part + row * d + c), a1 = *(const float4*)(part + row * d + c + 4);
    acc[0] = a0.x; acc[1] = a0.y; acc[2] = a0.z; acc[3] = a0.w;
    acc[4] = a1.x; acc[5] = a1.y; acc[6] = a1.z; acc[7] = a1.w;
    for (int s = 1; s < nsplit; ++s) {
      const float* p = part + ((int64_t)s * R + row) * d + c;
      const float4 b0 = *(const float4*)p, b1 = *(const float4*)(p + 4);
      acc[0] += b0.x; acc[1] += b0.y; acc[2] += b0.z; acc[3] += b0.w;
      acc[4] += b1.x; acc[5] += b1.y; acc[6] += b1.z; acc[7] += b1.w;
    }
    *(uint4*)(dQKV + row * (3 * (int64_t)d) + c) = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                               pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

// dK, dV of the chunk's own keys: grid (ceil(b / 64), H, streams); each lane owns one key.
// dV = sum_q P dO, dK = (1 / sqrt(128)) sum_q dS Q over the chunk's queries that see the key;
// written (bf16) into columns d + 128 h .. and 2 d + 128 h .. of dQKV.
// With nsplit > 1 (blockIdx.x = key block * nsplit + split) each workgroup takes a share of
// the query blocks that see its keys and writes fp32 partial dK | dV into part[split] ([R x
// 2d]); k_swa_dkdv_sum adds them in split order. The share is what balances the launch: the
// first key block of a chunk is seen by every query block, the last by one.
__global__ void __launch_bounds__(NT_A, 2) k_swa_bwd_dkdv(SwaGeo g, int nsplit, float* __restrict__ part,
                                                       const bf16_t* __restrict__ dOb,
                                                       const float* __restrict__ lse2, const float* __restrict__ Dq,
                                                       bf16_t* __restrict__ dQKV) {
  __shared__ __attribute__((aligned(16))) bf16_t sQ[BLK * LDR];
  __shared__ __attribute__((aligned(16))) bf16_t sD[BLK * LDR];
  __shared__ __attribute__((aligned(16))) bf16_t sQt[DH * LDT];
  __shared__ __attribute__((aligned(16))) bf16_t sDt[DH * LDT];
  __shared__ float sL[BLK], sDq[BLK];
  const int z = blockIdx.z, h = blockIdx.y, H = gridDim.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int split = blockIdx.x % nsplit;
  const int k0 = (blockIdx.x / nsplit) * BLK;
  const int kq = k0 + wave * 16 + lr;  // this lane's key (chunk row)
  const bool kok = kq < g.b;
  const float sc = LOG2E * 0.08838834764831845f;

  uint4 kf[4], vf[4];
  {
    const int64_t row = (int64_t)z * g.b + (kok ? kq : 0);
    const bf16_t* kr = g.qkv + row * (3 * (int64_t)g.d) + g.d + h * DH;
    const bf16_t* vr = kr + g.d;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kf[s] = kok ? *(const uint4*)(kr + 32 * s + 8 * lg) : make_uint4(0, 0, 0, 0);
      vf[s] = kok ? *(const uint4*)(vr + 32 * s + 8 * lg) : make_uint4(0, 0, 0, 0);
    }
  }
  f32x4_t dk[8], dv[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    dk[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    dv[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // chunk queries that see a key of this block: from its first key to the window's end
  const int kmax = min(k0 + BLK, g.b) - 1;
  int qend = (int)min((int64_t)g.b - 1, (int64_t)kmax + g.window - 1);
  int qfirst = k0;  // this workgroup's share of the query blocks [k0, qend]
  if (nsplit > 1) {
    const int nq = (qend - k0) / BLK + 1;
    const int b0 = nq * split / nsplit, b1 = nq * (split + 1) / nsplit;
    qend = min(qend, k0 + b1 * BLK - 1);
    qfirst = k0 + b0 * BLK;
  }
  const int64_t base = (int64_t)z * g.b;
  Chunks cq, cd;
  float fl = 0.f, fd = 0.f;
  auto fetch_block = [&](int qb) {
    fetch_p(cq, [&](int r) -> const bf16_t* {
      return qb + r <= qend ? g.qkv + (base + qb + r) * (3 * (int64_t)g.d) + h * DH : nullptr;
    });
    fetch_p(cd, [&](int r) -> const bf16_t* {
      return qb + r <= qend ? dOb + (base + qb + r) * g.d + h * DH : nullptr;
    });
    if (threadIdx.x < BLK) {
      const int qq = qb + threadIdx.x;
      const int64_t o = ((int64_t)z * H + h) * g.b + qq;
      fl = qq <= qend ? lse2[o] : 0.f;
      fd = qq <= qend ? Dq[o] : 0.f;
    }
  };
  if (qfirst <= qend) fetch_block(qfirst);
  for (int qb = qfirst; qb <= qend; qb += BLK) {
    __syncthreads();
    put_p(cq, sQ, sQt);
    put_p(cd, sD, sDt);
    if (threadIdx.x < BLK) {
      sL[threadIdx.x] = fl;
      sDq[threadIdx.x] = fd;
    }
    __syncthreads();
    if (qb + BLK <= qend) fetch_block(qb + BLK);
    // S[q][key] and dP[q][key]: sa[i][e], pa[i][e] for query qb + 16 i + 4 lg + e
    f32x4_t sa[4], pa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      pa[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        mfma_chunk(sa[i], *(const uint4*)(sQ + (16 * i + lr) * LDR + 32 * s + 8 * lg), kf[s], bf16_t());
        mfma_chunk(pa[i], *(const uint4*)(sD + (16 * i + lr) * LDR + 32 * s + 8 * lg), vf[s], bf16_t());
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ql = 16 * i + 4 * lg + e;
        const int dist = qb + ql - kq;  // query - key, both chunk rows
        const bool ok = kok && qb + ql <= qend && dist >= 0 && dist < g.window;
        const float p = ok ? __builtin_amdgcn_exp2f(sa[i][e] * sc - sL[ql]) : 0.f;
        sa[i][e] = p;
        pa[i][e] = p * (pa[i][e] - sDq[ql]);
      }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint4 pb = pchunk(sa[2 * t], sa[2 * t + 1]);
      const uint4 db = pchunk(pa[2 * t], pa[2 * t + 1]);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        mfma_chunk(dv[c], tchunk(sDt, 16 * c + lr, t, lg), pb, bf16_t());
        mfma_chunk(dk[c], tchunk(sQt, 16 * c + lr, t, lg), db, bf16_t());
      }
    }
  }
  if (!kok) return;
  const float rs = 0.08838834764831845f;
  if (nsplit > 1) {
    float* P = part + ((int64_t)split * gridDim.z * g.b + (int64_t)z * g.b + kq) * (2 * (int64_t)g.d) + h * DH;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int col = 16 * c + 4 * lg;
      *(float4*)(P + col) = make_float4(dk[c][0] * rs, dk[c][1] * rs, dk[c][2] * rs, dk[c][3] * rs);
      *(float4*)(P + g.d + col) = make_float4(dv[c][0], dv[c][1], dv[c][2], dv[c][3]);
    }
    return;
  }
  bf16_t* out = dQKV + ((int64_t)z * g.b + kq) * (3 * (int64_t)g.d) + h * DH;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int col = 16 * c + 4 * lg;
    *(uint2*)(out + g.d + col) =
        make_uint2(pack_bf16x2(dk[c][0] * rs, dk[c][1] * rs), pack_bf16x2(dk[c][2] * rs, dk[c][3] * rs));
    *(uint2*)(out + 2 * g.d + col) =
        make_uint2(pack_bf16x2(dv[c][0], dv[c][1]), pack_bf16x2(dv[c][2], dv[c][3]));
  }
}

// The last min(b, cr) keys and values of the chunk into the ring (both forms): grid (rows,
// streams).
__global__ void __launch_bounds__(64) k_kv_append(const bf16_t* __restrict__ qkv, const f16_t* __restrict__ qkv16,
                                                  int b, int d, int64_t pos, int cr, bf16_t* __restrict__ kc,
                                                  bf16_t* __restrict__ vc, f16_t* __restrict__ kc16,
                                                  f16_t* __restrict__ vc16) {
  const int n = min(b, cr);
  const int r = b - n + blockIdx.x, z = blockIdx.y;
  const int64_t so = ((int64_t)z * b + r) * (3 * (int64_t)d);
  const int64_t dst = ((int64_t)z * cr + (pos + r) % cr) * d;
  for (int c = threadIdx.x * 8; c < d; c += 64 * 8) {
    *(uint4*)(kc + dst + c) = *(const uint4*)(qkv + so + d + c);
    *(uint4*)(vc + dst + c) = *(const uint4*)(qkv + so + 2 * d + c);
    *(uint4*)(kc16 + dst + c) = *(const uint4*)(qkv16 + so + d + c);
    *(uint4*)(vc16 + dst + c) = *(const uint4*)(qkv16 + so + 2 * d + c);
  }
}

// ---------------------------------------------------------------------------- decode
// One decoded row (position p, its q | k | v in fp32, qkv [3d]), grid (H, nsplit): the first
// share of each head files the head's part of the row's key and value in
// the ring (bf16 and half, as the chunk path stores them); every share attends over its
// contiguous run of the keys max(0, p - window + 1) .. p in blocks of 64 (half-precision
// keys and values, fp32 arithmetic), taking the key and value at p from the row itself (its
// half-precision values, the ones filed), so that no share reads the slot being written.
// Per block, four lanes score a key (32 dims each, 16-byte loads, two shuffles), one wave
// turns the 64 scores into probabilities, and each lane accumulates 8 dims of o over a
// sixteenth of the keys (16-byte loads of consecutive dims); the sixteenths are summed in
// LDS at the end. k_swa_dec_merge combines the shares per head. (Combining them in the
// share that finishes last, through a per-head counter, needs a device-scope release per
// share: on this chip that writes the L2 back, and decoding measured 502 against 214 us per
// token at the 760M fuller block.)
constexpr int DEC_KB = 64;       // keys per block of the decode kernel
constexpr int DEC_SPLIT_MAX = 64;

__global__ void __launch_bounds__(NT_A) k_swa_dec(const float* __restrict__ qkv, bf16_t* __restrict__ kc,
                                                  f16_t* __restrict__ kc16, bf16_t* __restrict__ vc,
                                                  f16_t* __restrict__ vc16, int d, int64_t p, int cr, int window,
                                                  float* __restrict__ part) {
  __shared__ float sp[DEC_KB];      // the block's probabilities
  __shared__ float sacc[16][DH];    // per key subset, the partial o
  __shared__ float sml[2];          // the block's (max, sum)
  const int h = blockIdx.x, split = blockIdx.y, nsplit = gridDim.y;
  const int t = threadIdx.x;
  if (split == 0 && t < DH) {
    const int64_t o = (p % cr) * d + h * DH + t;
    const float k = qkv[d + h * DH + t], v = qkv[2 * d + h * DH + t];
    kc[o] = f2bf(k);
    kc16[o] = f2h(k);
    vc[o] = f2bf(v);
    vc16[o] = f2h(v);
  }
  // scores: four lanes per key, 32 dims each
  const int kj = t >> 2, kq = (t & 3) * 32;
  float q[32], kown[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    q[i] = qkv[h * DH + kq + i] * 0.08838834764831845f;  // q / sqrt(128)
    kown[i] = h2f(f2h(qkv[d + h * DH + kq + i]));
  }
  // values: lane group g of 8 dims, key subset ks (keys ks, ks + 16, ..)
  const int g = (t & 15) * 8, ks = t >> 4;
  float vown[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) vown[x] = h2f(f2h(qkv[2 * d + h * DH + g + x]));
  int64_t k0 = p - window + 1;
  if (k0 < 0) k0 = 0;
  const int64_t nk = p - k0 + 1;
  const int64_t nblk = (nk + DEC_KB - 1) / DEC_KB;
  const int64_t b0 = nblk * split / nsplit, b1 = nblk * (split + 1) / nsplit;
  float m = -INFINITY, l = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // a block's operands, requested one block ahead: this lane's key (32 dims) and its four
  // value rows (8 dims); ring slots are in range for any position, and keys past p are
  // neither scored nor accumulated
  struct Ops {
    uint4 k[4], v[4];
  };
  auto load = [&](Ops& o, int64_t kb) {
    const int64_t rk = ((kb + kj) % cr) * d + h * DH + kq;
#pragma unroll
    for (int c = 0; c < 4; ++c) o.k[c] = *(const uint4*)(kc16 + rk + 8 * c);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) o.v[jj] = *(const uint4*)(vc16 + ((kb + ks + 16 * jj) % cr) * d + h * DH + g);
  };
  Ops cur, nxt;
  if (b0 < b1) load(cur, k0 + b0 * DEC_KB);
  for (int64_t blk = b0; blk < b1; ++blk) {
    const int64_t kb = k0 + blk * DEC_KB;
    if (blk + 1 < b1) load(nxt, kb + DEC_KB);
    {
      const int64_t kp = kb + kj;
      float a = 0.f;
      if (kp == p) {
#pragma unroll
        for (int i = 0; i < 32; ++i) a = fmaf(kown[i], q[i], a);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f16_t* e = (const f16_t*)&cur.k[c];
#pragma unroll
          for (int x = 0; x < 8; ++x) a = fmaf(h2f(e[x]), q[8 * c + x], a);
        }
      }
      a += __shfl_xor(a, 1, TTT_WAVE);
      a += __shfl_xor(a, 2, TTT_WAVE);
      if ((t & 3) == 0) sp[kj] = kp <= p ? a * LOG2E : -INFINITY;
    }
    __syncthreads();
    if (t < 64) {  // the block's max, probabilities and sum (one wave)
      const float sv = sp[t];
      float bm = sv;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) bm = fmaxf(bm, __shfl_xor(bm, off, TTT_WAVE));
      const float mn = fmaxf(m, bm);
      const float pk = sv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv - mn);
      sp[t] = pk;
      float ps = pk;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) ps += __shfl_xor(ps, off, TTT_WAVE);
      if (t == 0) {
        sml[0] = mn;
        sml[1] = ps;
      }
    }
    __syncthreads();
    const float mn = sml[0];
    const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
    l = l * alpha + sml[1];
    m = mn;
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] *= alpha;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = ks + 16 * jj;
      if (kb + j > p) break;
      const f16_t* e = (const f16_t*)&cur.v[jj];
      const float pj = sp[j];
      if (kb + j == p) {
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[x] = fmaf(pj, vown[x], acc[x]);
      } else {
#pragma unroll
        for (int x = 0; x < 8; ++x) acc[x] = fmaf(pj, h2f(e[x]), acc[x]);
      }
    }
    __syncthreads();  // sp and sml are rewritten by the next block
    cur = nxt;
  }
  // the 16 key subsets' sums per dim, then this share's (max, sum, o[128])
#pragma unroll
  for (int x = 0; x < 8; ++x) sacc[ks][g + x] = acc[x];
  __syncthreads();
  float* P = part + ((int64_t)h * nsplit + split) * (DH + 2);
  if (t < DH) {
    float o = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) o += sacc[k][t];
    P[t] = o;
  }
  if (t == 0) {
    P[DH] = m;
    P[DH + 1] = l;
  }
}

// o [d] = per head, the shares' states combined: grid (H), 128 threads. The shares' maxima
// and sums go through LDS first (one wave reduces them), so the per-dim sums then issue all
// their loads independently.
__global__ void __launch_bounds__(DH) k_swa_dec_merge(const float* __restrict__ part, int nsplit,
                                                      float* __restrict__ o) {
  __shared__ float wts[DEC_SPLIT_MAX];
  __shared__ float sL;
  const int h = blockIdx.x, t = threadIdx.x;
  const float* P = part + (int64_t)h * nsplit * (DH + 2);
  if (t < 64) {
    const float ms = t < nsplit ? P[t * (DH + 2) + DH] : -INFINITY;
    float M = ms;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, TTT_WAVE));
    const float w = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    float L = t < nsplit ? w * P[t * (DH + 2) + DH + 1] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) L += __shfl_xor(L, off, TTT_WAVE);
    wts[t] = w;
    if (t == 0) sL = L;
  }
  __syncthreads();
  float a = 0.f;
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) a += wts[s] * P[s * (DH + 2) + t];
  const float L = sL;
  o[h * DH + t] = L > 0.f ? a / L : 0.f;
}

SwaGeo geo(const SwaShape& s) {
  SwaGeo g;
  g.qkv = (const bf16_t*)s.qkv;
  g.kc = (const bf16_t*)s.kc;
  g.vc = (const bf16_t*)s.vc;
  g.qkv16 = (const f16_t*)s.qkv16;
  g.kc16 = (const f16_t*)s.kc16;
  g.vc16 = (const f16_t*)s.vc16;
  g.cr = s.cr;
  g.b = s.b;
  g.d = s.d;
  g.window = s.window;
  g.pos = s.pos;
  return g;
}

bool shape_ok(const SwaShape& s) {
  return s.d % DH == 0 && s.d >= DH && s.b >= 1 && s.streams >= 1 && s.streams <= 65535 && s.window >= 1 &&
         s.cr >= 1 && s.pos >= 0 && s.qkv && s.kc && s.vc && s.qkv16 && s.kc16 && s.vc16;
}

}  // namespace

// dK | dV = the sum of the split partials in split order, into columns d .. 3d of dQKV
// (bf16): grid (streams b rows), 256 threads x 8 columns.
__global__ void __launch_bounds__(NT_A) k_swa_dkdv_sum(const float* __restrict__ part, int nsplit, int d,
                                                       bf16_t* __restrict__ dQKV) {
  const int64_t row = blockIdx.x, R = gridDim.x;
  for (int c = threadIdx.x * 8; c < 2 * d; c += NT_A * 8) {
    float acc[8];
    const float* p0 = part + row * (2 * (int64_t)d) + c;
    const float4 a0 = *(const float4*)p0, a1 = *(const float4*)(p0 + 4);
    acc[0] = a0.x; acc[1] = a0.y; acc[2] = a0.z; acc[3] = a0.w;
    acc[4] = a1.x; acc[5] = a1.y; acc[6] = a1.z; acc[7] = a1.w;
    for (int s = 1; s < nsplit; ++s) {
      const float* p = part + ((int64_t)s * R + row) * (2 * (int64_t)d) + c;
      const float4 b0 = *(const float4*)p, b1 = *(const float4*)(p + 4);
      acc[0] += b0.x; acc[1] += b0.y; acc[2] += b0.z; acc[3] += b0.w;
      acc[4] += b1.x; acc[5] += b1.y; acc[6] += b1.z; acc[7] += b1.w;
    }
    *(uint4*)(dQKV + row * (3 * (int64_t)d) + d + c) =
        make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                   pack_bf16x2(acc[6], acc[7]));
  }
}

// Query groups of 16 per wave in the forward kernel. Two halve the LDS reads per query.
constexpr int FWD_QG = 1;

// Workgroups of one launch take about equal time, so a launch of wg query blocks split n
// ways costs about ceil(wg n / slots) rounds of 1/n of the key range (slots: workgroups
// resident at once on 256 CUs): the n (at most SPLIT_CAP, whole key blocks per split)
// minimising rounds / n, the smallest on ties.
static int split_count(int64_t wg, const SwaShape& s, int slots) {
  const int64_t kblocks = ((int64_t)(s.window < s.b ? s.b : s.window) + BLK - 1) / BLK;
  int best = 1;
  double cost = 1e30;
  for (int n = 1; n <= SPLIT_CAP && n <= kblocks; ++n) {
    const double c = (double)((wg * n + slots - 1) / slots) / n;
    if (c < cost - 1e-12) {
      cost = c;
      best = n;
    }
  }
  return best;
}

int swa_fwd_splits(const SwaShape& s) {
  // 64 FWD_QG queries per workgroup, two workgroups per CU (about 160 registers at one query
  // group a wave, 230 at two). Three per CU at one group, or two groups a wave, measured no
  // faster at the 760M fuller block: 169 and 165 against 165 us per launch.
  const int qb = BLK * FWD_QG;
  const int64_t wg = (int64_t)((s.b + qb - 1) / qb) * (s.d / DH) * s.streams;
  return split_count(wg, s, 512);
}

int swa_dkdv_splits(const SwaShape& s) {
  // the first key block is seen by the most query blocks: shares of about four of them
  const int64_t first = (int64_t)(s.window + BLK - 2 < s.b - 1 ? s.window + BLK - 2 : s.b - 1) / BLK + 1;
  const int n = (int)((first + 3) / 4);
  return n < 1 ? 1 : (n > 4 ? 4 : n);
}

int swa_dq_splits(const SwaShape& s) {
  // 64 queries per workgroup, two workgroups per CU; at a 1024-token chunk of 12 heads, 8
  const int64_t wg = (int64_t)((s.b + BLK - 1) / BLK) * (s.d / DH) * s.streams;
  return split_count(wg, s, 512);
}

hipError_t run_swa_fwd(hipStream_t st, const SwaShape& s, float* Of, void* Ob, void* Ol, float* lse2, float* part,
                       float* pm, float* pl) {
  if (!shape_ok(s) || !Ol) return hipErrorInvalidValue;
  SwaSplit sp{swa_fwd_splits(s), part, pm, pl};
  if (sp.n > 1 && (!part || !pm || !pl)) return hipErrorInvalidValue;
  const int H = s.d / DH, qb = BLK * FWD_QG;
  dim3 grid((s.b + qb - 1) / qb * sp.n, H, s.streams);
  hipLaunchKernelGGL(k_swa_fwd<FWD_QG>, grid, dim3(NT_A), 0, st, geo(s), sp, Of, (bf16_t*)Ob, (bf16_t*)Ol, lse2);
  if (sp.n > 1)
    hipLaunchKernelGGL(k_swa_merge, dim3((unsigned)((int64_t)s.streams * s.b), H), dim3(64), 0, st, sp, s.b, s.d, Of,
                       (bf16_t*)Ob, (bf16_t*)Ol, lse2);
  return hipGetLastError();
}

hipError_t run_swa_dsum(hipStream_t st, const SwaShape& s, const float* dOf, const float* Of, float* Dq) {
  if (!shape_ok(s)) return hipErrorInvalidValue;
  const unsigned R = (unsigned)((int64_t)s.streams * s.b);
  hipLaunchKernelGGL(k_swa_dsum, dim3(R, s.d / DH), dim3(64), 0, st, dOf, Of, s.d, s.b, Dq);
  return hipGetLastError();
}

hipError_t run_swa_bwd_dq(hipStream_t st, const SwaShape& s, const void* dOb, const float* lse2, const float* Dq,
                          void* dQKV, float* part) {
  if (!shape_ok(s)) return hipErrorInvalidValue;
  const int H = s.d / DH;
  const int ns = swa_dq_splits(s);
  if (ns > 1 && !part) return hipErrorInvalidValue;
  const unsigned R = (unsigned)((int64_t)s.streams * s.b);
  dim3 gq((s.b + BLK - 1) / BLK * ns, H, s.streams);
  hipLaunchKernelGGL(k_swa_bwd_dq, gq, dim3(NT_A), 0, st, geo(s), ns, part, (const bf16_t*)dOb, lse2, Dq,
                     (bf16_t*)dQKV);
  if (ns > 1) hipLaunchKernelGGL(k_swa_dq_sum, dim3(R), dim3(NT_A), 0, st, part, ns, s.d, (bf16_t*)dQKV);
  return hipGetLastError();
}

hipError_t run_swa_bwd_dkdv(hipStream_t st, const SwaShape& s, const void* dOb, const float* lse2, const float* Dq,
                            void* dQKV, float* part) {
  if (!shape_ok(s)) return hipErrorInvalidValue;
  const int H = s.d / DH;
  const int nk = swa_dkdv_splits(s);
  if (nk > 1 && !part) return hipErrorInvalidValue;
  const unsigned R = (unsigned)((int64_t)s.streams * s.b);
  dim3 grid((s.b + BLK - 1) / BLK * nk, H, s.streams);
  hipLaunchKernelGGL(k_swa_bwd_dkdv, grid, dim3(NT_A), 0, st, geo(s), nk, part, (const bf16_t*)dOb, lse2, Dq,
                     (bf16_t*)dQKV);
  if (nk > 1) hipLaunchKernelGGL(k_swa_dkdv_sum, dim3(R), dim3(NT_A), 0, st, part, nk, s.d, (bf16_t*)dQKV);
  return hipGetLastError();
}

int swa_dec_splits(int window) {
  // about two blocks of keys per workgroup, at most 64 workgroups per head
  const int blocks = (window + DEC_KB - 1) / DEC_KB;
  const int n = (blocks + 1) / 2;
  return n < 1 ? 1 : (n > DEC_SPLIT_MAX ? DEC_SPLIT_MAX : n);
}

hipError_t run_swa_decode(hipStream_t st, const SwaShape& s, const float* qkv, float* part, float* o) {
  if (!qkv || !part || !o || s.d % DH || s.cr < 1 || s.window < 1 || s.pos < 0 || !s.kc || !s.vc || !s.kc16 || !s.vc16)
    return hipErrorInvalidValue;
  const int H = s.d / DH, ns = swa_dec_splits(s.window);
  hipLaunchKernelGGL(k_swa_dec, dim3(H, ns), dim3(NT_A), 0, st, qkv, (bf16_t*)s.kc, (f16_t*)s.kc16, (bf16_t*)s.vc,
                     (f16_t*)s.vc16, s.d, s.pos, s.cr, s.window, part);
  hipLaunchKernelGGL(k_swa_dec_merge, dim3(H), dim3(DH), 0, st, part, ns, o);
  return hipGetLastError();
}

hipError_t run_kv_append(hipStream_t st, const SwaShape& s) {
  if (!shape_ok(s)) return hipErrorInvalidValue;
  const int n = s.b < s.cr ? s.b : s.cr;
  hipLaunchKernelGGL(k_kv_append, dim3(n, s.streams), dim3(64), 0, st, (const bf16_t*)s.qkv, (const f16_t*)s.qkv16,
                     s.b, s.d, s.pos, s.cr, (bf16_t*)s.kc, (bf16_t*)s.vc, (f16_t*)s.kc16, (f16_t*)s.vc16);
  return hipGetLastError();
}
