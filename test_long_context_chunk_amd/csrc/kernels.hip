// Row-wise and elementwise kernels of the TTT inner loop (everything that is not a GEMM).
#include "launchers.h"
#include "gemm.h"

namespace {

constexpr int NT = 256;  // threads per block for the row/elementwise kernels

// Block-wide sum in a fixed order (wave butterflies, then waves 0..3 in order).
__device__ __forceinline__ float block_sum_256(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <class T>
__device__ __forceinline__ float4 load4(const T* p);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p) { return *(const float4*)p; }
template <>
__device__ __forceinline__ float4 load4<bf16_t>(const bf16_t* p) {
  const uint2 u = *(const uint2*)p;
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}
template <class T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *(float4*)p = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  *(uint2*)p = make_uint2((uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16), (uint32_t)f2bf(c) | ((uint32_t)f2bf(d) << 16));
}


// ---- row kernels: one block per token row; d is a multiple of 8, so every row moves in
// groups of 4 consecutive elements (16-byte fp32, 8- or 16-byte operand-precision accesses).
// A thread keeps up to ROW_CACHE of its groups in registers between the two passes over a
// row (d <= 4 * NT * ROW_CACHE); further groups are read again (the row is L2-resident).
constexpr int ROW_CACHE = 2;

// The values of v after rounding to the operand precision T.
template <class T>
__device__ __forceinline__ float4 rounded4(const float4 v) {
  return make_float4(to_f<T>(from_f<T>(v.x)), to_f<T>(from_f<T>(v.y)), to_f<T>(from_f<T>(v.z)), to_f<T>(from_f<T>(v.w)));
}

// Sum of the S split-K slabs of 4 consecutive elements, in split order. For the slab counts
// the planner uses (1 .. 8) every slab's load is issued before the first add, so a thread has
// all of them in flight at once; the sum order is the same either way.
template <int S>
__device__ __forceinline__ float4 slab_sum4_n(const float* __restrict__ part, int64_t pstride, int64_t i) {
  float4 p[S];
#pragma unroll
  for (int s = 0; s < S; ++s) p[s] = *(const float4*)(part + (int64_t)s * pstride + i);
  float4 acc = p[0];
#pragma unroll
  for (int s = 1; s < S; ++s) {
    acc.x += p[s].x;
    acc.y += p[s].y;
    acc.z += p[s].z;
    acc.w += p[s].w;
  }
  return acc;
}
__device__ __forceinline__ float4 slab_sum4(const float* __restrict__ part, int S, int64_t pstride, int64_t i) {
  switch (S) {
    case 1: return slab_sum4_n<1>(part, pstride, i);
    case 2: return slab_sum4_n<2>(part, pstride, i);
    case 3: return slab_sum4_n<3>(part, pstride, i);
    case 4: return slab_sum4_n<4>(part, pstride, i);
    case 5: return slab_sum4_n<5>(part, pstride, i);
    case 6: return slab_sum4_n<6>(part, pstride, i);
    case 7: return slab_sum4_n<7>(part, pstride, i);
    case 8: return slab_sum4_n<8>(part, pstride, i);
    default: break;
  }
  float4 acc = *(const float4*)(part + i);
  for (int s = 1; s < S; ++s) {
    const float4 p = *(const float4*)(part + (int64_t)s * pstride + i);
    acc.x += p.x;
    acc.y += p.y;
    acc.z += p.z;
    acc.w += p.w;
  }
  return acc;
}

// a1 + a2, a4 + a2: the residual stream entering block l and its pre-norm.
//   gather (tokens non-null, [E2E] eq. 1: f reads x_{t-1}): h = E_in[x_{t-1}]; ids outside
//     [0, V) raise the sticky range bit and read row 0; the clamped conditioning and target
//     ids are recorded;
//   residual (tokens null): h = H + sum_s part[s] (the down-projection's split-K slabs,
//     summed in split order first).
// Stores H = h (fp32) and, when given, Yb = rn(h) (the LM head's operand). When Hn is given,
// also block l's pre-norm n = h (mean h^2 + eps)^(-1/2) (rms; none: n = h) as rn(n), its
// scale r, and when RES is given the rounding residual n - rn(n).
template <class T>
__global__ void __launch_bounds__(NT) k_row_in(const int* __restrict__ tokens, StreamRows sr, int V,
                                               const T* __restrict__ E,
                                               int* __restrict__ tok_prev, int* __restrict__ tok_tgt,
                                               int* __restrict__ err, const float* __restrict__ part, int S,
                                               int64_t pstride, float* __restrict__ H, int d, T* __restrict__ Yb,
                                               float eps, int rms, T* __restrict__ Hn, float* __restrict__ r,
                                               T* __restrict__ RES, T* __restrict__ Yl) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int64_t base = (int64_t)t * d;
  const T* src = nullptr;
  if (tokens) {
    const int z = t / sr.bs;
    const int* tk = tokens + z * sr.ld + (t - z * sr.bs);
    int xp = tk[0], xt = tk[1];
    const bool bad = (xp < 0 || xp >= V || xt < 0 || xt >= V);
    if (xp < 0 || xp >= V) xp = 0;
    if (xt < 0 || xt >= V) xt = 0;
    if (threadIdx.x == 0) {
      tok_prev[t] = xp;
      tok_tgt[t] = xt;
      if (bad) atomicOr(err, ERRBIT_RANGE);
    }
    src = E + (int64_t)xp * d;
  }
  const int ng = d >> 2;
  float4 hc[ROW_CACHE];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < ROW_CACHE; ++k) hc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int g = threadIdx.x, k = 0; g < ng; g += NT, ++k) {
    const int64_t i = base + (g << 2);
    float4 h;
    if (src) {
      h = load4<T>(src + (g << 2));
    } else {
      const float4 acc = slab_sum4(part, S, pstride, i);
      h = *(const float4*)(H + i);
      h.x += acc.x;
      h.y += acc.y;
      h.z += acc.z;
      h.w += acc.w;
    }
    *(float4*)(H + i) = h;
    if (Yb) store4<T>(Yb + i, h.x, h.y, h.z, h.w);
    if (Yl) {
      const float4 q = rounded4<T>(h);
      store4<T>(Yl + i, h.x - q.x, h.y - q.y, h.z - q.z, h.w - q.w);
    }
    ss += h.x * h.x + h.y * h.y + h.z * h.z + h.w * h.w;
#pragma unroll
    for (int q = 0; q < ROW_CACHE; ++q)
      if (q == k) hc[q] = h;
  }
  if (!Hn) return;
  float rr = 1.0f;
  if (rms) {
    ss = block_sum_256(ss, red);
    rr = 1.0f / sqrtf(ss / (float)d + eps);
  }
  if (threadIdx.x == 0) r[t] = rr;
  for (int g = threadIdx.x, k = 0; g < ng; g += NT, ++k) {
    const int64_t i = base + (g << 2);
    float4 h = hc[0];
    if (k < ROW_CACHE) {
#pragma unroll
      for (int q = 1; q < ROW_CACHE; ++q)
        if (q == k) h = hc[q];
    } else {
      h = *(const float4*)(H + i);  // this thread's own store above
    }
    const float4 n = make_float4(h.x * rr, h.y * rr, h.z * rr, h.w * rr);
    store4<T>(Hn + i, n.x, n.y, n.z, n.w);
    if (RES) {
      const float4 q = rounded4<T>(n);
      store4<T>(RES + i, n.x - q.x, n.y - q.y, n.z - q.z, n.w - q.w);
    }
  }
}


// a6 finish: dY = sum_s part[s] (fixed order) into dH and its GEMM-precision copy. With
// Hres (the fp32 hidden state whose rounded copy Yb fed the LM head), also
// cdot[t] = <dY_t, H_t - rn(H_t)> for the first-order loss compensation.
template <class T>
__global__ void __launch_bounds__(NT) k_dy_finish(const float* __restrict__ part, int S, int64_t pstride, int d,
                                                  float* __restrict__ dH, T* __restrict__ dHb,
                                                  const float* __restrict__ Hres, const T* __restrict__ Yb,
                                                  float* __restrict__ cdot) {
  __shared__ float red[4];
  const int64_t base = (int64_t)blockIdx.x * d;
  float dot = 0.f;
  for (int g = threadIdx.x; g < (d >> 2); g += NT) {
    const int64_t i = base + (g << 2);
    const float4 a = slab_sum4(part, S, pstride, i);
    *(float4*)(dH + i) = a;
    store4<T>(dHb + i, a.x, a.y, a.z, a.w);
    if (cdot) {
      const float4 h = *(const float4*)(Hres + i), y = load4<T>(Yb + i);
      dot += a.x * (h.x - y.x) + a.y * (h.y - y.y) + a.z * (h.z - y.z) + a.w * (h.w - y.w);
    }
  }
  if (cdot) {
    dot = block_sum_256(dot, red);
    if (threadIdx.x == 0) cdot[blockIdx.x] = dot;
  }
}

// a7 norm backward (pre-norm block, through the frozen norm into the residual stream):
//   dn = sum_s part[s] (= dU W1^T);  rms: dH += r (dn - n mean_j(dn_j n_j));  none: dH += dn.
// With RES, also cdot[t] = <dn_t, RES_t> (first-order loss compensation of the rounded n);
// update_dh = 0 computes only that dot (the lowest block, whose input gradient is not needed).
template <class T>
__global__ void __launch_bounds__(NT) k_norm_bwd(const float* __restrict__ part, int S, int64_t pstride,
                                                 const T* __restrict__ Hn, const float* __restrict__ r, int d,
                                                 int rms, float* __restrict__ dH, T* __restrict__ dHb,
                                                 const T* __restrict__ RES, float* __restrict__ cdot, int update_dh) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  const int64_t base = (int64_t)t * d;
  const int ng = d >> 2;
  float4 dc[ROW_CACHE];
#pragma unroll
  for (int k = 0; k < ROW_CACHE; ++k) dc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  float mean = 0.f, rr = 1.f;
  if (rms || cdot) {
    float dot = 0.f, cd = 0.f;
    for (int g = threadIdx.x, k = 0; g < ng; g += NT, ++k) {
      const int64_t i = base + (g << 2);
      const float4 dn = slab_sum4(part, S, pstride, i);
#pragma unroll
      for (int q = 0; q < ROW_CACHE; ++q)
        if (q == k) dc[q] = dn;
      const float4 n = load4<T>(Hn + i);
      dot += dn.x * n.x + dn.y * n.y + dn.z * n.z + dn.w * n.w;
      if (cdot) {
        const float4 e = load4<T>(RES + i);
        cd += dn.x * e.x + dn.y * e.y + dn.z * e.z + dn.w * e.w;
      }
    }
    if (rms) {
      dot = block_sum_256(dot, red);
      mean = dot / (float)d;
      rr = r[t];
    }
    if (cdot) {
      cd = block_sum_256(cd, red);
      if (threadIdx.x == 0) cdot[t] = cd;
    }
  }
  if (!update_dh) return;
  const bool cached = rms || cdot;
  for (int g = threadIdx.x, k = 0; g < ng; g += NT, ++k) {
    const int64_t i = base + (g << 2);
    float4 dn = dc[0];
    if (cached && k < ROW_CACHE) {
#pragma unroll
      for (int q = 1; q < ROW_CACHE; ++q)
        if (q == k) dn = dc[q];
    } else {
      dn = slab_sum4(part, S, pstride, i);
    }
    float4 gv = dn;
    if (rms) {
      const float4 n = load4<T>(Hn + i);
      gv = make_float4(rr * (dn.x - n.x * mean), rr * (dn.y - n.y * mean), rr * (dn.z - n.z * mean),
                       rr * (dn.w - n.w * mean));
    }
    float4 v = *(const float4*)(dH + i);
    v.x += gv.x;
    v.y += gv.y;
    v.z += gv.z;
    v.w += gv.w;
    *(float4*)(dH + i) = v;
    store4<T>(dHb + i, v.x, v.y, v.z, v.w);
  }
}


// dst[c, r] = src[r, c] for r < R, c < C through a 64 x 64 LDS tile. Interior tiles move
// 16-byte pieces both ways (8 bf16 or 4 fp32 consecutive elements of a source row in, of a
// destination row out); edge tiles go element by element.
template <class T>
__global__ void __launch_bounds__(NT) k_transpose(const T* __restrict__ src, int64_t lds, int R, int C,
                                                  T* __restrict__ dst, int64_t ldd) {
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte piece
  __shared__ T tile[64][64 + V];     // [source column][source row]
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const bool full = r0 + 64 <= R && c0 + 64 <= C && (lds % V) == 0 && (ldd % V) == 0;
  if (full) {
    for (int idx = threadIdx.x; idx < 64 * (64 / V); idx += NT) {
      const int r = idx / (64 / V), c = (idx % (64 / V)) * V;
      const uint4 v = *(const uint4*)(src + (int64_t)(r0 + r) * lds + c0 + c);
      const T* e = (const T*)&v;
#pragma unroll
      for (int q = 0; q < V; ++q) tile[c + q][r] = e[q];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * (64 / V); idx += NT) {
      const int c = idx / (64 / V), r = (idx % (64 / V)) * V;
      *(uint4*)(dst + (int64_t)(c0 + c) * ldd + r0 + r) = *(const uint4*)&tile[c][r];
    }
    return;
  }
  for (int idx = threadIdx.x; idx < 64 * 64; idx += NT) {
    const int r = idx / 64, c = idx % 64;
    if (r0 + r < R && c0 + c < C) tile[c][r] = src[(int64_t)(r0 + r) * lds + c0 + c];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 64 * 64; idx += NT) {
    const int c = idx / 64, r = idx % 64;
    if (r0 + r < R && c0 + c < C) dst[(int64_t)(c0 + c) * ldd + r0 + r] = tile[c][r];
  }
}

// Add the first-order rounding compensation to the recorded losses:
//   l_t += scale * sum_s cpart[s * b + t]   (fixed order; b rows of all streams, the loss of
// row t at its stream's record).
// 16 tokens per block; the 16 threads of a token sum interleaved slots, then combine in a
// fixed butterfly order.
__global__ void __launch_bounds__(NT) k_loss_correct(const float* __restrict__ cpart, int nslot, int b, StreamRows sr,
                                                     float scale, float* __restrict__ loss) {
  const int t = blockIdx.x * 16 + (threadIdx.x & 15);
  const int part = threadIdx.x >> 4;  // 0..15
  float acc = 0.f;
  if (t < b)
    for (int s = part; s < nslot; s += 16) acc += cpart[(int64_t)s * b + t];
  // lanes t, t+16, t+32, t+48 of a wave hold the same token: sum across lane groups, then waves
  acc += __shfl_xor(acc, 16, TTT_WAVE);
  acc += __shfl_xor(acc, 32, TTT_WAVE);
  __shared__ float red[4][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane < 16) red[wave][lane] = acc;
  __syncthreads();
  if (threadIdx.x < 16 && t < b) loss[sr.ld * (t / sr.bs) + t % sr.bs] += scale * ((red[0][threadIdx.x] + red[1][threadIdx.x]) + (red[2][threadIdx.x] + red[3][threadIdx.x]));
}

// a5 merge: combine the (max, sum exp, argmax) records of each row in a fixed order:
// lse = M + ln S, l_t = lse - z_t[x_t] ([E2E] eq. 1), argmax (lowest index).
__global__ void __launch_bounds__(NT) k_ce_merge(const float* __restrict__ pmax, const float* __restrict__ psum,
                                                 const int* __restrict__ pidx, int nrec, int b, StreamRows sr,
                                                 const float* __restrict__ tgt_logit, float* __restrict__ lse,
                                                 float* __restrict__ loss, int* __restrict__ amax) {
  // one row per block (a large vocabulary has thousands of records per row): thread t takes
  // records t, t + NT, ..; then a butterfly within each wave and the waves in order
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  float mx = -INFINITY, sm = 0.f;
  int ix = 0x7fffffff;
  for (int j = tid; j < nrec; j += NT) {
    const int64_t o = (int64_t)row * nrec + j;
    ce_combine(mx, sm, ix, pmax[o], psum[o], pidx[o]);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float omx = __shfl_xor(mx, off, TTT_WAVE);
    const float osm = __shfl_xor(sm, off, TTT_WAVE);
    const int oix = __shfl_xor(ix, off, TTT_WAVE);
    ce_combine(mx, sm, ix, omx, osm, oix);
  }
  __shared__ float wmx[NT / 64], wsm[NT / 64];
  __shared__ int wix[NT / 64];
  if (lane == 0) {
    wmx[wave] = mx;
    wsm[wave] = sm;
    wix[wave] = ix;
  }
  __syncthreads();
  if (tid == 0) {
    mx = wmx[0];
    sm = wsm[0];
    ix = wix[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) ce_combine(mx, sm, ix, wmx[w], wsm[w], wix[w]);
    const float l = mx + logf(sm);
    lse[row] = l;
    const int64_t o = sr.ld * (row / sr.bs) + row % sr.bs;
    loss[o] = l - tgt_logit[row];
    amax[o] = ix;
  }
}

// a8: g = sqrt(sum of the per-tile sums of squares of every fast gradient), in fp64 and a
// fixed order; s = min(1, clip / g) (clip <= 0: 1); a non-finite g skips the step. One block
// per stream: stream z's slots, scale pair and statistics pair start at z * nslot, 4 z and
// z * stat_ld.
__global__ void __launch_bounds__(NT) k_gradnorm(const float* __restrict__ slot, int nslot, float clip,
                                                 float* __restrict__ sc, float* __restrict__ stat, int64_t stat_ld,
                                                 int* __restrict__ err) {
  __shared__ double red[4];
  slot += (int64_t)blockIdx.x * nslot;
  sc += 4 * blockIdx.x;
  stat += stat_ld * blockIdx.x;
  double acc = 0.0;
  for (int i = threadIdx.x; i < nslot; i += NT) acc += (double)slot[i];
  acc = wave_sum_d(acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double g = sqrt((red[0] + red[1]) + (red[2] + red[3]));
    const bool finite = isfinite(g);
    double s = 1.0;
    if (!finite) s = 0.0;
    else if (clip > 0.f && g > (double)clip) s = (double)clip / g;
    sc[0] = (float)s;
    sc[1] = finite ? 0.f : 1.f;
    stat[0] = (float)g;
    stat[1] = (float)s;
    if (!finite) atomicOr(err, ERRBIT_NONFINITE);
  }
}

// a6 dlogits of the whole vocabulary, in place ([E2E] eq. 5 through the softmax
// cross-entropy): Q holds exp(z - m) with m the max of the record (W consecutive vocabulary
// entries) the column belongs to, so softmax = Q exp(m - lse) and
//   P[t, v] = (Q[t, v] exp(m - lse_t) - [v == x_t]) / b.
// Eight consecutive columns per thread (W and V are multiples of 8).
template <class T>
__global__ void __launch_bounds__(NT) k_ce_dlogits(T* __restrict__ Q, int b, int V, int W,
                                                   const float* __restrict__ pmax, int nrec,
                                                   const float* __restrict__ lse, const int* __restrict__ tgt,
                                                   float inv_b) {
  const int per_row = V >> 3;
  const int64_t n = (int64_t)b * per_row;
  for (int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * NT) {
    const int row = (int)(idx / per_row);
    const int c0 = (int)(idx - (int64_t)row * per_row) << 3;
    const float s = exp_fast(pmax[(int64_t)row * nrec + c0 / W] - lse[row]) * inv_b;
    const int tc = tgt[row] - c0;
    T* q = Q + (int64_t)row * V + c0;
    const float4 lo = load4<T>(q), hi = load4<T>(q + 4);
    float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = v[k] * s - (k == tc ? inv_b : 0.f);
    store4<T>(q, v[0], v[1], v[2], v[3]);
    store4<T>(q + 4, v[4], v[5], v[6], v[7]);
  }
}

// ---- decode ([E2E] Method: decoding predicts p^_{t+1} = f(x_t; W); section 3.2: a step only
// when the decoded tokens fill a mini-batch). One activation row per launch; activations stay
// in fp32 (the fast weights are the stored bf16 segments), so no operand rounding enters.

// 8 consecutive weights in the operand precision, as loaded (16 bytes bf16, 32 bytes fp32).
struct F8 {
  float4 a, b;
};
template <class T>
using W8 = typename std::conditional<sizeof(T) == 2, uint4, F8>::type;
__device__ __forceinline__ uint4 load_w8(const bf16_t* w) { return *(const uint4*)w; }
__device__ __forceinline__ F8 load_w8(const float* w) { return F8{*(const float4*)w, *(const float4*)(w + 4)}; }
__device__ __forceinline__ float dot8v(const uint4 u, const float* x) {
  const float4 x0 = *(const float4*)x, x1 = *(const float4*)(x + 4);
  float s = __uint_as_float(u.x << 16) * x0.x;
  s = fmaf(__uint_as_float(u.x & 0xffff0000u), x0.y, s);
  s = fmaf(__uint_as_float(u.y << 16), x0.z, s);
  s = fmaf(__uint_as_float(u.y & 0xffff0000u), x0.w, s);
  s = fmaf(__uint_as_float(u.z << 16), x1.x, s);
  s = fmaf(__uint_as_float(u.z & 0xffff0000u), x1.y, s);
  s = fmaf(__uint_as_float(u.w << 16), x1.z, s);
  return fmaf(__uint_as_float(u.w & 0xffff0000u), x1.w, s);
}
__device__ __forceinline__ float dot8v(const F8 w, const float* x) {
  const float4 x0 = *(const float4*)x, x1 = *(const float4*)(x + 4);
  float s = w.a.x * x0.x;
  s = fmaf(w.a.y, x0.y, s);
  s = fmaf(w.a.z, x0.z, s);
  s = fmaf(w.a.w, x0.w, s);
  s = fmaf(w.b.x, x1.x, s);
  s = fmaf(w.b.y, x1.y, s);
  s = fmaf(w.b.z, x1.z, s);
  return fmaf(w.b.w, x1.w, s);
}

// Dot of 8 consecutive operand-precision weights with 8 fp32 activations.
__device__ __forceinline__ float dot8(const bf16_t* w, const float* x) {
  const uint4 u = *(const uint4*)w;
  const float4 x0 = *(const float4*)x, x1 = *(const float4*)(x + 4);
  float s = __uint_as_float(u.x << 16) * x0.x;
  s = fmaf(__uint_as_float(u.x & 0xffff0000u), x0.y, s);
  s = fmaf(__uint_as_float(u.y << 16), x0.z, s);
  s = fmaf(__uint_as_float(u.y & 0xffff0000u), x0.w, s);
  s = fmaf(__uint_as_float(u.z << 16), x1.x, s);
  s = fmaf(__uint_as_float(u.z & 0xffff0000u), x1.y, s);
  s = fmaf(__uint_as_float(u.w << 16), x1.z, s);
  return fmaf(__uint_as_float(u.w & 0xffff0000u), x1.w, s);
}
__device__ __forceinline__ float dot8(const float* w, const float* x) {
  const float4 w0 = *(const float4*)w, w1 = *(const float4*)(w + 4);
  const float4 x0 = *(const float4*)x, x1 = *(const float4*)(x + 4);
  float s = w0.x * x0.x;
  s = fmaf(w0.y, x0.y, s);
  s = fmaf(w0.z, x0.z, s);
  s = fmaf(w0.w, x0.w, s);
  s = fmaf(w1.x, x1.x, s);
  s = fmaf(w1.y, x1.y, s);
  s = fmaf(w1.z, x1.z, s);
  return fmaf(w1.w, x1.w, s);
}

// Decode product of one activation row with the rows of Y [N x K] (row stride ldy, operand
// precision), fp32 throughout. The block first builds x [K] in LDS:
//   xin given:  x = xin (the residual stream H or the activation A);
//   tok given:  x = E_in[tok[0]] (the gather, [E2E] eq. 1: f reads x_{t-1}); block 0 also
//               writes it to H and copies the pair (tok[0], tok[1]) into the pending-chunk
//               ids pend (pend[0] only when first), raising the range bit for ids outside
//               [0, V) (read as id 0);
//   norm:       then x *= (mean x^2 + eps)^(-1/2) (the block's pre-norm, no gain).
// Then, with WPR waves per output row splitting K and RPW rows per wave group:
//   STORE:    out[n] = x.Y[n] (+ x.Y2[n], the second K-segment when Y2 is given)
//   GELU:     out[n] = GELU(x.Y[n] (+ x.Y2[n]))
//   RESIDUAL: out[n] += x.Y[n] (+ x.Y2[n])
//   SWIGLU:   out[n] = SiLU(x.Y[n]) * x.Y2[n] (Y the gate, Y2 the up projection)
template <class T, int MODE, int WPR, int RPW>
__global__ void __launch_bounds__(NT) k_gemv(const float* __restrict__ xin, const int* __restrict__ tok, int first,
                                             int* __restrict__ pend, const T* __restrict__ E, int V,
                                             float* __restrict__ H, int* __restrict__ err, int norm, float eps,
                                             int K, const T* __restrict__ Y, const T* __restrict__ Y2, int64_t ldy,
                                             int N, float* __restrict__ out, float* __restrict__ rmax,
                                             float* __restrict__ rsum, int* __restrict__ ridx) {
  extern __shared__ __attribute__((aligned(16))) float xs[];
  __shared__ float red[4];
  __shared__ float part[2][4][RPW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int GROUPS = (NT / 64) / WPR;  // row groups per block
  const int grp = wave / WPR, kp = wave % WPR;
  const int n0 = (blockIdx.x * GROUPS + grp) * RPW;
  const int kw = K / WPR;  // K per wave (K / WPR is a multiple of 8)
  const int k_lo = kp * kw, k_hi = k_lo + kw;
  const bool two = Y2 != nullptr;
  // the first KP slices of this lane's weights are requested before the activation row is
  // built: they do not depend on it
  constexpr int KP = 3;
  W8<T> w1[KP][RPW], w2[KP][RPW];
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int k = min(k_lo + lane * 8 + i * 512, k_hi - 8);
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int n = min(n0 + r, N - 1);
      w1[i][r] = load_w8(Y + (int64_t)n * ldy + k);
      if (two) w2[i][r] = load_w8(Y2 + (int64_t)n * ldy + k);
    }
  }
  const T* src = nullptr;
  if (tok) {
    int xp = tok[0];
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      const int xt = tok[1];
      if (first) pend[0] = xp;
      pend[1] = xt;
      if (xp < 0 || xp >= V || xt < 0 || xt >= V) atomicOr(err, ERRBIT_RANGE);
    }
    if (xp < 0 || xp >= V) xp = 0;
    src = E + (int64_t)xp * K;
  }
  float ss = 0.f;
  for (int g = threadIdx.x; g < (K >> 2); g += NT) {
    const float4 v = src ? load4<T>(src + 4 * g) : *(const float4*)(xin + 4 * g);
    if (src && blockIdx.x == 0) *(float4*)(H + 4 * g) = v;
    *(float4*)(xs + 4 * g) = v;
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  if (norm) {
    ss = block_sum_256(ss, red);  // includes the barrier that publishes xs
    const float rr = 1.0f / sqrtf(ss / (float)K + eps);
    for (int g = threadIdx.x; g < (K >> 2); g += NT) {
      float4 v = *(float4*)(xs + 4 * g);
      v.x *= rr;
      v.y *= rr;
      v.z *= rr;
      v.w *= rr;
      *(float4*)(xs + 4 * g) = v;
    }
  }
  __syncthreads();
  float s1[RPW], s2[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) s1[r] = s2[r] = 0.f;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int k = k_lo + lane * 8 + i * 512;
    if (k >= k_hi) break;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      s1[r] += dot8v(w1[i][r], xs + k);
      if (two) s2[r] += dot8v(w2[i][r], xs + k);
    }
  }
#pragma unroll 2
  for (int k = k_lo + lane * 8 + KP * 512; k < k_hi; k += 512) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int n = min(n0 + r, N - 1);
      s1[r] += dot8(Y + (int64_t)n * ldy + k, xs + k);
      if (two) s2[r] += dot8(Y2 + (int64_t)n * ldy + k, xs + k);
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    s1[r] = wave_sum(s1[r]);
    s2[r] = wave_sum(s2[r]);
  }
  if constexpr (WPR > 1) {
    if (lane == 0)
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        part[0][wave][r] = s1[r];
        part[1][wave][r] = s2[r];
      }
    __syncthreads();
    if (kp != 0) return;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      float a = part[0][grp * WPR][r], b = part[1][grp * WPR][r];
      for (int q = 1; q < WPR; ++q) {
        a += part[0][grp * WPR + q][r];
        b += part[1][grp * WPR + q][r];
      }
      s1[r] = a;
      s2[r] = b;
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int n = n0 + r;
    if (lane != 0 || n >= N) continue;
    const float a = s1[r], b = s2[r];
    if constexpr (MODE == GEMV_STORE) out[n] = a + b;
    if constexpr (MODE == GEMV_GELU) out[n] = gelu_f(a + b);
    if constexpr (MODE == GEMV_RESIDUAL) out[n] += a + b;
    if constexpr (MODE == GEMV_SWIGLU) out[n] = silu_f(a) * b;
  }
  if constexpr (MODE == GEMV_STORE && WPR == 1) {
    // with records: this block's online-softmax record over its rows (max, sum of
    // exp(z - max), first argmax), for the decode CE merge
    if (rmax) {
      __shared__ float zb[(NT / 64) * RPW];
      if (lane == 0)
#pragma unroll
        for (int r = 0; r < RPW; ++r) zb[wave * RPW + r] = s1[r] + s2[r];
      __syncthreads();
      if (threadIdx.x == 0) {
        const int base = blockIdx.x * (NT / 64) * RPW;
        float mx = -INFINITY;
        int ix = 0x7fffffff;
        for (int q = 0; q < (NT / 64) * RPW && base + q < N; ++q)
          if (zb[q] > mx) {
            mx = zb[q];
            ix = base + q;
          }
        float sm = 0.f;
        for (int q = 0; q < (NT / 64) * RPW && base + q < N; ++q) sm += expf(zb[q] - mx);
        rmax[blockIdx.x] = mx;
        rsum[blockIdx.x] = sm;
        ridx[blockIdx.x] = ix;
      }
    }
  }
}

// Decode CE of one logits row z [V] (fp32) from the LM-head product's per-block records
// (max, sum of exp(z - max), first argmax), merged in a fixed order: lse, first argmax and
// loss = lse - z[target] (target = tgt[0], clamped like the gather). Writes the token's loss
// and argmax records and, when given, argmax_out. One block.
__global__ void __launch_bounds__(NT) k_dec_ce(const float* __restrict__ z, int V, const float* __restrict__ rmax,
                                               const float* __restrict__ rsum, const int* __restrict__ ridx, int nrec,
                                               const int* __restrict__ tgt, float* __restrict__ loss,
                                               int* __restrict__ amax, int* __restrict__ argmax_out) {
  __shared__ float smx[NT], ssm[NT];
  __shared__ int six[NT];
  float mx = -INFINITY, sm = 0.f;
  int ix = 0x7fffffff;
  for (int j = threadIdx.x; j < nrec; j += NT) ce_combine(mx, sm, ix, rmax[j], rsum[j], ridx[j]);
  smx[threadIdx.x] = mx;
  ssm[threadIdx.x] = sm;
  six[threadIdx.x] = ix;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) {
      float m0 = smx[threadIdx.x], s0 = ssm[threadIdx.x];
      int i0 = six[threadIdx.x];
      ce_combine(m0, s0, i0, smx[threadIdx.x + s], ssm[threadIdx.x + s], six[threadIdx.x + s]);
      smx[threadIdx.x] = m0;
      ssm[threadIdx.x] = s0;
      six[threadIdx.x] = i0;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int tg = tgt[0];
    if (tg < 0 || tg >= V) tg = 0;
    const float lse = smx[0] + logf(ssm[0]);
    loss[0] = lse - z[tg];
    amax[0] = six[0];
    if (argmax_out) argmax_out[0] = six[0];
  }
}

// ---- evaluation and Settlement ([SGF], Settlement: a candidate step is committed only if
// it does not raise the loss of a held-out passage).

// Add the n losses of one evaluated chunk to acc[0] (fp64, fixed order; zeroed first when
// first is set), copy them to out when given, and when last is set write acc[0] / count into
// mean (when given). One block.
__global__ void __launch_bounds__(NT) k_eval_accum(const float* __restrict__ loss, int n, double* __restrict__ acc,
                                                   float* __restrict__ out, int first, int last, int64_t count,
                                                   float* __restrict__ mean) {
  __shared__ double red[NT];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += NT) {
    const float v = loss[i];
    s += (double)v;
    if (out) out[i] = v;
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = NT / 2; k > 0; k >>= 1) {
    if (threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double t = (first ? 0.0 : acc[0]) + red[0];
    acc[0] = t;
    if (last && mean) mean[0] = (float)(t / (double)count);
  }
}

// A = (sum0 - sum1) / count = L(q, W) - L(q, W + delta); commit = A >= 0 (a non-finite A
// rejects). Writes A and the decision to the context's words and, when given, the caller's.
__global__ void k_settle_decide(const double* __restrict__ sums, int64_t count, float* __restrict__ A,
                                int* __restrict__ commit, float* __restrict__ A_out, int* __restrict__ commit_out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const double a = (sums[0] - sums[1]) / (double)count;
  const int ok = (a >= 0.0) ? 1 : 0;  // false for NaN
  A[0] = (float)a;
  commit[0] = ok;
  if (A_out) A_out[0] = (float)a;
  if (commit_out) commit_out[0] = ok;
}

// dst <- src (n bytes, 16-byte aligned, n a multiple of 16) unless *commit is set.
__global__ void __launch_bounds__(NT) k_restore_unless(const int* __restrict__ commit, const uint4* __restrict__ src,
                                                       uint4* __restrict__ dst, int64_t n16) {
  if (commit[0]) return;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n16; i += (int64_t)gridDim.x * NT) dst[i] = src[i];
}

// a9: in-place clipped SGD step of one fast tensor [R x C]:
//   D <- D - lr * s * G;  Wop = rn(W0 + D) row-major (the backward GEMMs' operand);
//   WtT = transposed copy of rn(D) when delta_t (bf16: the forward GEMMs add X rn(D)^T to
//   X W0^T, so updates far below W0's rounding step still reach them), else of rn(W0 + D).
// A block owns a 64 x 64 tile: each thread updates 4 consecutive columns of 4 rows with
// vector accesses, and the transposed copy leaves through LDS as 16-byte row pieces.
template <class T>
__global__ void __launch_bounds__(NT) k_update(const T* __restrict__ G, float* __restrict__ D,
                                               const T* __restrict__ W0, T* __restrict__ Wop,
                                               T* __restrict__ WtT, int R, int C, float lr,
                                               const float* __restrict__ sc, int delta_t) {
  // stream blockIdx.z: its own G, D, Wop, WtT (R x C apart) and scale pair; W0 is shared
  {
    const int64_t zo = (int64_t)blockIdx.z * R * C;
    G += zo;
    D += zo;
    Wop += zo;
    WtT += zo;
    sc += 4 * blockIdx.z;
  }
  if (sc[1] != 0.f) return;  // non-finite gradient norm: no step for this chunk
  const float step = lr * sc[0];
  __shared__ T tile[64][64 + 16 / sizeof(T)];  // [col][row] of the transposed output
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int cq = (threadIdx.x & 15) * 4, rq = threadIdx.x >> 4;  // 16 column quads x 16 rows
  const bool vec = (C % 4) == 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rl = rq + 16 * k, r = r0 + rl, c = c0 + cq;
    if (r >= R || c >= C) continue;
    const int64_t i = (int64_t)r * C + c;
    float w[4];
    if (vec) {
      const float4 g = load4<T>(G + i), d = load4<float>(D + i), w0 = load4<T>(W0 + i);
      const float dn[4] = {d.x - step * g.x, d.y - step * g.y, d.z - step * g.z, d.w - step * g.w};
      *(float4*)(D + i) = make_float4(dn[0], dn[1], dn[2], dn[3]);
      const float wv[4] = {w0.x + dn[0], w0.y + dn[1], w0.z + dn[2], w0.w + dn[3]};
      store4<T>(Wop + i, wv[0], wv[1], wv[2], wv[3]);
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = delta_t ? dn[q] : wv[q];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[q] = 0.f;
        if (c + q >= C) continue;
        const float dn = D[i + q] - step * to_f<T>(G[i + q]);
        D[i + q] = dn;
        const float wv = to_f<T>(W0[i + q]) + dn;
        Wop[i + q] = from_f<T>(wv);
        w[q] = delta_t ? dn : wv;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) tile[cq + q][rl] = from_f<T>(w[q]);
  }
  __syncthreads();
  // transposed rows: WtT[c][r0 .. r0 + 63], 16-byte pieces
  constexpr int PER = 16 / sizeof(T);  // elements per piece
  for (int idx = threadIdx.x; idx < 64 * (64 / PER); idx += NT) {
    const int cl = idx / (64 / PER), rl = (idx % (64 / PER)) * PER;
    const int c = c0 + cl, r = r0 + rl;
    if (c >= C || r >= R) continue;
    T* dst = WtT + (int64_t)c * R + r;
    if ((R % PER) == 0 && r + PER <= R) {
      *(uint4*)dst = *(const uint4*)&tile[cl][rl];
    } else {
      for (int q = 0; q < PER && r + q < R; ++q) dst[q] = tile[cl][rl + q];
    }
  }
}

// a9 for bf16 tensors with C a multiple of 8: the same step with 16-byte accesses throughout.
// A block owns a 64 x 64 tile; thread t updates rows 2p, 2p + 1 (p = t / 8) at columns
// 8 (t % 8) .. + 7. The transposed copy goes through LDS as row pairs packed into dwords,
// [column][row pair] with a row stride of 33 dwords: for each column offset q the 64 lanes of
// a wave write 64 distinct banks (8 (t % 8) + t / 8 + 33 q mod 64), and each transposed
// row piece leaves as 16 bytes.
__device__ __forceinline__ void unpack8_bf16(const uint4& u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ uint4 pack8_bf16(const float (&f)[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

__global__ void __launch_bounds__(NT) k_update_bf16x8(const bf16_t* __restrict__ G, float* __restrict__ D,
                                                      const bf16_t* __restrict__ W0, bf16_t* __restrict__ Wop,
                                                      bf16_t* __restrict__ WtT, int R, int C, float lr,
                                                      const float* __restrict__ sc, int delta_t) {
  {
    const int64_t zo = (int64_t)blockIdx.z * R * C;
    G += zo;
    D += zo;
    Wop += zo;
    WtT += zo;
    sc += 4 * blockIdx.z;
  }
  if (sc[1] != 0.f) return;  // non-finite gradient norm: no step for this chunk
  const float step = lr * sc[0];
  constexpr int LDT = 33;                 // dwords per transposed row (32 row pairs + 1)
  __shared__ uint32_t tile[64 * LDT];     // [column][row pair]
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int cg = threadIdx.x & 7, p = threadIdx.x >> 3;  // p in 0..31
  const int c = c0 + 8 * cg;
  float wt[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = r0 + 2 * p + h;
#pragma unroll
    for (int q = 0; q < 8; ++q) wt[h][q] = 0.f;
    if (r >= R || c >= C) continue;
    const int64_t i = (int64_t)r * C + c;
    float g[8], w0[8];
    unpack8_bf16(*(const uint4*)(G + i), g);
    unpack8_bf16(*(const uint4*)(W0 + i), w0);
    const float4 da = *(const float4*)(D + i), db = *(const float4*)(D + i + 4);
    const float d8[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
    float dn[8], wv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      dn[q] = d8[q] - step * g[q];
      wv[q] = w0[q] + dn[q];
      wt[h][q] = delta_t ? dn[q] : wv[q];
    }
    *(float4*)(D + i) = make_float4(dn[0], dn[1], dn[2], dn[3]);
    *(float4*)(D + i + 4) = make_float4(dn[4], dn[5], dn[6], dn[7]);
    *(uint4*)(Wop + i) = pack8_bf16(wv);
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) tile[(8 * cg + q) * LDT + p] = pack_bf16x2(wt[0][q], wt[1][q]);
  __syncthreads();
  // transposed rows WtT[c][r0 .. r0 + 63]: 64 columns x 8 pieces of 16 bytes (4 row pairs)
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = threadIdx.x + k * NT;
    const int cl = idx >> 3, j = idx & 7;
    const int cc = c0 + cl, r = r0 + 8 * j;
    if (cc >= C || r >= R) continue;
    const uint32_t* src = tile + cl * LDT + 4 * j;
    bf16_t* dst = WtT + (int64_t)cc * R + r;
    if ((R % 8) == 0) {
      *(uint4*)dst = make_uint4(src[0], src[1], src[2], src[3]);
    } else {
      for (int q = 0; q < 8 && r + q < R; ++q) dst[q] = (bf16_t)((src[q >> 1] >> (16 * (q & 1))) & 0xffffu);
    }
  }
}

template <class T>
__global__ void __launch_bounds__(NT) k_export(const float* __restrict__ D, const T* __restrict__ W0, int64_t n,
                                               int kind, float* __restrict__ dst) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT)
    dst[i] = kind ? D[i] : to_f<T>(W0[i]) + D[i];
}

__global__ void __launch_bounds__(NT) k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT) p[i] = v;
}

inline int grid_for(int64_t n) {
  int64_t g = (n + NT - 1) / NT;
  if (g > 4096) g = 4096;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

#define DISPATCH_T(prec, ...)                 \
  do {                                        \
    if ((prec) == PREC_BF16) {                \
      using T = bf16_t;                       \
      __VA_ARGS__;                            \
    } else {                                  \
      using T = float;                        \
      __VA_ARGS__;                            \
    }                                         \
  } while (0)

hipError_t run_row_in(hipStream_t st, int prec, const int* tokens, StreamRows sr, int V, const void* E, int* tok_prev,
                      int* tok_tgt, int* err, const float* part, int S, int64_t pstride, float* H, int b, int d, void* Yb,
                      float eps, int rms, void* Hn, float* r, void* RES, void* Yl) {
  if (d % 8 || sr.bs < 1) return hipErrorInvalidValue;
  DISPATCH_T(prec, hipLaunchKernelGGL(k_row_in<T>, dim3(b), dim3(NT), 0, st, tokens, sr, V, (const T*)E, tok_prev, tok_tgt,
                                      err, part, S, pstride, H, d, (T*)Yb, eps, rms, (T*)Hn, r, (T*)RES, (T*)Yl));
  return hipGetLastError();
}

hipError_t run_transpose(hipStream_t st, int prec, const void* src, int64_t lds, int R, int C, void* dst, int64_t ldd) {
  if (R <= 0 || C <= 0) return hipSuccess;
  dim3 grid((C + 63) / 64, (R + 63) / 64);
  DISPATCH_T(prec, hipLaunchKernelGGL(k_transpose<T>, grid, dim3(NT), 0, st, (const T*)src, lds, R, C, (T*)dst, ldd));
  return hipGetLastError();
}

hipError_t run_dy_finish(hipStream_t st, int prec, const float* part, int S, int64_t pstride, int b, int d,
                         float* dH, void* dHb, const float* Hres, const void* Yb, float* cdot) {
  DISPATCH_T(prec, hipLaunchKernelGGL(k_dy_finish<T>, dim3(b), dim3(NT), 0, st, part, S, pstride, d, dH, (T*)dHb, Hres,
                                      (const T*)Yb, cdot));
  return hipGetLastError();
}

hipError_t run_loss_correct(hipStream_t st, const float* cpart, int nslot, int b, StreamRows sr, float scale,
                            float* loss) {
  if (sr.bs < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_loss_correct, dim3((b + 15) / 16), dim3(NT), 0, st, cpart, nslot, b, sr, scale, loss);
  return hipGetLastError();
}

hipError_t run_ce_merge(hipStream_t st, const float* pmax, const float* psum, const int* pidx, int nrec, int b,
                        StreamRows sr, const float* tgt_logit, float* lse, float* loss, int* amax) {
  if (sr.bs < 1) return hipErrorInvalidValue;
  if (b <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_ce_merge, dim3(b), dim3(NT), 0, st, pmax, psum, pidx, nrec, b, sr, tgt_logit, lse, loss, amax);
  return hipGetLastError();
}

hipError_t run_ce_dlogits(hipStream_t st, int prec, void* Q, int b, int V, int W, const float* pmax, int nrec,
                          const float* lse, const int* tgt, float inv_b) {
  if (V % 8 || W % 8 || W <= 0) return hipErrorInvalidValue;
  DISPATCH_T(prec, hipLaunchKernelGGL(k_ce_dlogits<T>, dim3(grid_for((int64_t)b * (V / 8))), dim3(NT), 0, st, (T*)Q, b,
                                      V, W, pmax, nrec, lse, tgt, inv_b));
  return hipGetLastError();
}

hipError_t run_norm_bwd(hipStream_t st, int prec, const float* part, int S, int64_t pstride, const void* Hn,
                        const float* r, int b, int d, int rms, float* dH, void* dHb, const void* RES, float* cdot,
                        int update_dh) {
  DISPATCH_T(prec, hipLaunchKernelGGL(k_norm_bwd<T>, dim3(b), dim3(NT), 0, st, part, S, pstride, (const T*)Hn, r, d,
                                      rms, dH, (T*)dHb, (const T*)RES, cdot, update_dh));
  return hipGetLastError();
}

hipError_t run_gradnorm(hipStream_t st, const float* slot, int nslot, float clip, float* sc, float* stat,
                        int64_t stat_ld, int streams, int* err) {
  if (streams < 1 || streams > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gradnorm, dim3(streams), dim3(NT), 0, st, slot, nslot, clip, sc, stat, stat_ld, err);
  return hipGetLastError();
}

hipError_t run_update(hipStream_t st, int prec, const void* G, float* D, const void* W0, void* Wop, void* WtT, int R,
                      int C, float lr, const float* sc, int delta_t, int streams) {
  if (streams < 1 || streams > 65535) return hipErrorInvalidValue;
  dim3 grid((C + 63) / 64, (R + 63) / 64, streams);
  if (prec == PREC_BF16 && C % 8 == 0 && R % 2 == 0) {
    hipLaunchKernelGGL(k_update_bf16x8, grid, dim3(NT), 0, st, (const bf16_t*)G, D, (const bf16_t*)W0, (bf16_t*)Wop,
                       (bf16_t*)WtT, R, C, lr, sc, delta_t);
    return hipGetLastError();
  }
  DISPATCH_T(prec, hipLaunchKernelGGL(k_update<T>, grid, dim3(NT), 0, st, (const T*)G, D, (const T*)W0, (T*)Wop,
                                      (T*)WtT, R, C, lr, sc, delta_t));
  return hipGetLastError();
}

hipError_t run_export(hipStream_t st, int prec, const float* D, const void* W0, int64_t n, int kind, float* dst) {
  DISPATCH_T(prec, hipLaunchKernelGGL(k_export<T>, dim3(grid_for(n)), dim3(NT), 0, st, D, (const T*)W0, n, kind, dst));
  return hipGetLastError();
}

template <class T, int MODE>
static hipError_t launch_gemv(hipStream_t st, const GemvIn& in, int K, const T* Y, const T* Y2, int64_t ldy, int N,
                              float* out) {
  const size_t lds = (size_t)K * sizeof(float);
  const T* E = (const T*)in.E;
#define TTT_GEMV_ARGS in.xin, in.tok, in.first, in.pend, E, in.V, in.H, in.err, in.norm, in.eps, K, Y, Y2, ldy, N, out, \
    in.rmax, in.rsum, in.ridx
  if (K >= 4096 && K % (4 * 8) == 0 && !in.rmax) {  // long rows: four waves share each row
    hipLaunchKernelGGL((k_gemv<T, MODE, 4, 1>), dim3(N), dim3(NT), lds, st, TTT_GEMV_ARGS);
  } else if (N >= 16384) {
    hipLaunchKernelGGL((k_gemv<T, MODE, 1, 4>), dim3((N + 15) / 16), dim3(NT), lds, st, TTT_GEMV_ARGS);
  } else {
    hipLaunchKernelGGL((k_gemv<T, MODE, 1, 1>), dim3((N + 3) / 4), dim3(NT), lds, st, TTT_GEMV_ARGS);
  }
#undef TTT_GEMV_ARGS
  return hipGetLastError();
}

hipError_t run_gemv(hipStream_t st, int prec, int mode, const GemvIn& in, int K, const void* Y, const void* Y2,
                    int64_t ldy, int N, float* out) {
  if (K % 8 || ldy % 8 || N <= 0 || (size_t)K * sizeof(float) > 64 * 1024) return hipErrorInvalidValue;
  if ((in.xin == nullptr) == (in.tok == nullptr)) return hipErrorInvalidValue;
  DISPATCH_T(prec, {
    switch (mode) {
      case GEMV_STORE: return launch_gemv<T, GEMV_STORE>(st, in, K, (const T*)Y, (const T*)Y2, ldy, N, out);
      case GEMV_GELU: return launch_gemv<T, GEMV_GELU>(st, in, K, (const T*)Y, (const T*)Y2, ldy, N, out);
      case GEMV_RESIDUAL: return launch_gemv<T, GEMV_RESIDUAL>(st, in, K, (const T*)Y, (const T*)Y2, ldy, N, out);
      case GEMV_SWIGLU: return launch_gemv<T, GEMV_SWIGLU>(st, in, K, (const T*)Y, (const T*)Y2, ldy, N, out);
      default: return hipErrorInvalidValue;
    }
  });
}

hipError_t run_dec_ce(hipStream_t st, const float* z, int V, const float* rmax, const float* rsum, const int* ridx,
                      int nrec, const int* tgt, float* loss, int* amax, int* argmax_out) {
  hipLaunchKernelGGL(k_dec_ce, dim3(1), dim3(NT), 0, st, z, V, rmax, rsum, ridx, nrec, tgt, loss, amax, argmax_out);
  return hipGetLastError();
}

hipError_t run_eval_accum(hipStream_t st, const float* loss, int n, double* acc, float* out, int first, int last,
                          int64_t count, float* mean) {
  hipLaunchKernelGGL(k_eval_accum, dim3(1), dim3(NT), 0, st, loss, n, acc, out, first, last, count, mean);
  return hipGetLastError();
}

hipError_t run_settle_decide(hipStream_t st, const double* sums, int64_t count, float* A, int* commit, float* A_out,
                             int* commit_out) {
  hipLaunchKernelGGL(k_settle_decide, dim3(1), dim3(64), 0, st, sums, count, A, commit, A_out, commit_out);
  return hipGetLastError();
}

hipError_t run_restore_unless(hipStream_t st, const int* commit, const void* src, void* dst, int64_t bytes) {
  if (bytes % 16) return hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(k_restore_unless, dim3(grid_for(n16)), dim3(NT), 0, st, commit, (const uint4*)src, (uint4*)dst,
                     n16);
  return hipGetLastError();
}

hipError_t run_fill_u32(hipStream_t st, void* p, int64_t n, uint32_t v) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(n)), dim3(NT), 0, st, (uint32_t*)p, n, v);
  return hipGetLastError();
}
