// Device code of the estimator's steps (2)-(4) (Prism review on
// paper.rainbus.top, pipeline paragraph), shared by the multi-kernel path
// (pool_rms.hip) and the single-launch estimator (score_select.hip): the
// block sums of one work item of the pooling pass, and the temperature
// reduction of one query head. Both kernels run exactly this arithmetic in
// this order, so their pooled vectors, energies and temperatures agree bit
// for bit.
#pragma once

#include "prism_kernels.h"

namespace prism {
namespace {

constexpr int kPoolThreads = 256;  // threads that pool one work item

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <bool FP32>
struct Elem;
template <>
struct Elem<false> {  // bf16: 8 dims per 16-byte load
  static constexpr int E = 8;
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ void add(float *acc, const uint4 v) {
    acc[0] += bf16lo(v.x); acc[1] += bf16hi(v.x);
    acc[2] += bf16lo(v.y); acc[3] += bf16hi(v.y);
    acc[4] += bf16lo(v.z); acc[5] += bf16hi(v.z);
    acc[6] += bf16lo(v.w); acc[7] += bf16hi(v.w);
  }
};
template <>
struct Elem<true> {  // fp32: 4 dims per 16-byte load
  static constexpr int E = 4;
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ void add(float *acc, const uint4 v) {
    acc[0] += __uint_as_float(v.x); acc[1] += __uint_as_float(v.y);
    acc[2] += __uint_as_float(v.z); acc[3] += __uint_as_float(v.w);
  }
};

// streaming 16-byte load that does not allocate in the caches (Q and K are
// read exactly once here)
__device__ __forceinline__ uint4 ld_stream(const char *p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// Work items per batch entry: (tensor, chunk of heads, block), blocks fastest.
__host__ __device__ inline int pool_items(const PoolArgs &a) { return (a.chunks[0] + a.chunks[1]) * a.nb; }

// One work item = (tensor, block of B tokens, chunk of heads); the place in
// it of thread `tid` of the kPoolThreads that pool it. Lanes of a token row:
// TPH per head, heads of the chunk adjacent; tokp token rows are read side
// by side.
template <bool FP32>
struct PoolItem {
  static constexpr int E = Elem<FP32>::E;
  static constexpr int TPH = kHeadDim / E;  // threads per head row
  int ts, i, lanes_per_tok, tokp, tp, hh, dg, h;
  bool active;
  __device__ PoolItem(const PoolArgs &a, int item, int tid) {
    int rem = item;
    ts = 0;
    const int nq = a.chunks[0] * a.nb;
    if (rem >= nq) { ts = 1; rem -= nq; }
    i = rem % a.nb;
    const int chunk = rem / a.nb;
    const int HC = a.heads_per_chunk[ts];
    lanes_per_tok = TPH * HC;
    tokp = kPoolThreads / lanes_per_tok;
    tp = tid / lanes_per_tok;
    hh = (tid % lanes_per_tok) / TPH;
    dg = tid % TPH;
    h = a.h0[ts] + chunk * HC + hh;
    active = tp < tokp && h < a.h0[ts] + a.nheads[ts];
  }
};

// This thread's block sums of one work item (its tokens, in token order).
template <bool FP32>
__device__ __forceinline__ void pool_accum(const PoolArgs &a, int batch, const PoolItem<FP32> &w,
                                           float (&acc)[Elem<FP32>::E]) {
  using El = Elem<FP32>;
  constexpr int E = El::E;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  if (!w.active) return;
  const TensorArg &x = a.x[w.ts];
  const int t0 = w.i * a.block;
  const int n = min(a.block, a.seq - t0);
  const char *base = static_cast<const char *>(x.data) +
                     ((int64_t)batch * x.sb + (int64_t)w.h * x.sh + (int64_t)t0 * x.ss + w.dg * E) * El::kBytes;
  const int64_t rs = x.ss * El::kBytes;
  const int tokp = w.tokp;
  int t = w.tp;
  for (; t + 7 * tokp < n; t += 8 * tokp) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ld_stream(base + (int64_t)(t + u * tokp) * rs);
#pragma unroll
    for (int u = 0; u < 8; ++u) El::add(acc, v[u]);
  }
  for (; t < n; t += tokp) El::add(acc, ld_stream(base + (int64_t)t * rs));
}

// Token-parallel partial sums of an item with tokp > 1: every token row but
// the first leaves its sums in `red` ...
template <bool FP32>
__device__ __forceinline__ void pool_red_put(const PoolItem<FP32> &w, int tid, const float (&acc)[Elem<FP32>::E],
                                             float *red) {
  constexpr int E = Elem<FP32>::E;
  if (w.tokp > 1 && w.tp < w.tokp) {
#pragma unroll
    for (int e = 0; e < E; ++e) red[tid * E + e] = acc[e];
  }
}

// ... and, after a barrier, the first token row adds them in a fixed order;
// then the block mean of this lane's dims and the squares of the mean
// summed per segment (high-only, middle, low-only) over the head row: st
// gets E means, then the three segment energies.
template <bool FP32>
__device__ __forceinline__ void pool_finish(const PoolArgs &a, const PoolItem<FP32> &w, int tid,
                                            float (&acc)[Elem<FP32>::E], const float *red, float *st) {
  constexpr int E = Elem<FP32>::E;
  constexpr int TPH = kHeadDim / E;
  if (w.tokp > 1 && w.tp == 0) {
    for (int k = 1; k < w.tokp; ++k) {
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += red[(tid + k * w.lanes_per_tok) * E + e];
    }
  }
  const int n = min(a.block, a.seq - w.i * a.block);
  const float inv_n = 1.0f / (float)n;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    st[e] = acc[e] * inv_n;
    const int c = w.dg * E + e;  // physical dim
    const int cc = a.half_layout ? (c < kHeadDim / 2 ? 2 * c : 2 * (c - kHeadDim / 2) + 1) : c;
    const float sq = st[e] * st[e];
    if (cc < a.seg_lo) s0 += sq;
    else if (cc < a.seg_hi) s1 += sq;
    else s2 += sq;
  }
  // sum over the TPH lanes of this head row (adjacent lanes, one wave)
#pragma unroll
  for (int off = TPH / 2; off >= 1; off >>= 1) {
    s0 += __shfl_xor(s0, off, TPH);
    s1 += __shfl_xor(s1, off, TPH);
    s2 += __shfl_xor(s2, off, TPH);
  }
  st[E] = s0;
  st[E + 1] = s1;
  st[E + 2] = s2;
}

// Writes one work item's pooled row (canonical order) and energies: `m` holds
// this lane's E means, `en` the head row's three segment energies.
template <bool FP32>
__device__ __forceinline__ void pool_write(const PoolArgs &a, int batch, const PoolItem<FP32> &w, const float *m,
                                           const float *en) {
  constexpr int E = Elem<FP32>::E;
  if (!w.active || w.tp != 0) return;
  const int64_t row = ((int64_t)batch * a.x[w.ts].heads + w.h) * a.nb + w.i;
  float *xb = a.xbar[w.ts] + row * kHeadDim;
  if (!a.half_layout) {
#pragma unroll
    for (int e = 0; e < E; e += 4)
      *reinterpret_cast<float4 *>(xb + w.dg * E + e) = make_float4(m[e], m[e + 1], m[e + 2], m[e + 3]);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int c = w.dg * E + e;
      const int cc = c < kHeadDim / 2 ? 2 * c : 2 * (c - kHeadDim / 2) + 1;
      xb[cc] = m[e];
    }
  }
  if (w.dg == 0) *reinterpret_cast<float4 *>(a.sq[w.ts] + row * 4) = make_float4(en[0], en[1], en[2], 0.f);
}

// Temperatures of query head h of batch entry b from the per-block segment
// energies: fixed-order fp64 sums over all blocks (thread t < kPoolThreads
// takes blocks t, t + kPoolThreads, ...; then a pairwise tree), R = sqrt(energy
// / (nb |D|)) per band and tensor, and tau_z by the mode (FULLSPEC: band
// energy relative to the full spectrum; UNIT: band energy alone; NONE and
// PERVEC: 1, PERVEC scaling per pooled vector in the score kernel instead).
// Every thread of the workgroup calls it (it holds barriers); threads at or
// past kPoolThreads only wait. Thread 0 returns the 8 values (tau_high,
// tau_low, Rq_high, Rq_low, Rq_full, Rk_high, Rk_low, Rk_full) in `out`.
__device__ __forceinline__ void tau_reduce(const TauArgs &a, int b, int h, double (*red)[kPoolThreads],
                                           float *out) {
  const int tid = threadIdx.x;
  const int g = h / (a.hq / a.hkv);
  if (tid < kPoolThreads) {
    const float4 *qs = reinterpret_cast<const float4 *>(a.qsq) + ((int64_t)b * a.hq + h) * a.nb;
    const float4 *ks = reinterpret_cast<const float4 *>(a.ksq) + ((int64_t)b * a.hkv + g) * a.nb;
    double s[6] = {0, 0, 0, 0, 0, 0};
    for (int i = tid; i < a.nb; i += kPoolThreads) {
      const float4 x = qs[i];
      const float4 y = ks[i];
      s[0] += x.x; s[1] += x.y; s[2] += x.z;
      s[3] += y.x; s[4] += y.y; s[5] += y.z;
    }
#pragma unroll
    for (int k = 0; k < 6; ++k) red[k][tid] = s[k];
  }
  __syncthreads();
  for (int w = kPoolThreads / 2; w >= 1; w >>= 1) {
    if (tid < w) {
#pragma unroll
      for (int k = 0; k < 6; ++k) red[k][tid] += red[k][tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double ov = a.overlap ? 1.0 : 0.0;
    const double nb = (double)a.nb;
    double r[6];
    for (int t = 0; t < 2; ++t) {
      const double e0 = red[3 * t][0], e1 = red[3 * t + 1][0], e2 = red[3 * t + 2][0];
      r[3 * t + 0] = sqrt((e0 + ov * e1) / (nb * a.d_high));
      r[3 * t + 1] = sqrt((e2 + ov * e1) / (nb * a.d_low));
      r[3 * t + 2] = sqrt((e0 + e1 + e2) / (nb * kHeadDim));
    }
    double th = 1.0, tl = 1.0;
    const bool okh = r[0] > 0 && r[3] > 0 && r[2] > 0 && r[5] > 0;
    const bool okl = r[1] > 0 && r[4] > 0 && r[2] > 0 && r[5] > 0;
    if (a.tau_mode == PRISM_TAU_FULLSPEC) {
      if (okh) th = (r[0] * r[3]) / (r[2] * r[5]);
      if (okl) tl = (r[1] * r[4]) / (r[2] * r[5]);
    } else if (a.tau_mode == PRISM_TAU_UNIT) {
      if (okh) th = r[0] * r[3];
      if (okl) tl = r[1] * r[4];
    }
    out[0] = (float)th; out[1] = (float)tl;
    out[2] = (float)r[0]; out[3] = (float)r[1]; out[4] = (float)r[2];
    out[5] = (float)r[3]; out[6] = (float)r[4]; out[7] = (float)r[5];
  }
}

}  // namespace
}  // namespace prism
