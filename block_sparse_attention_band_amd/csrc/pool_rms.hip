// Prism estimator, steps (1)-(4) (Prism review on paper.rainbus.top,
// pipeline paragraph): block mean pooling of post-RoPE Q and K, the pooled
// vectors' energy per band segment, and the per-head branch temperatures.
//
// pool_kernel: one streaming pass over Q and K. A work item is one block of
//   B tokens for a chunk of heads of one tensor; each thread reads 16 bytes
//   per token (8 bf16 or 4 fp32 dims), so the workgroup's loads for a token
//   are one contiguous run when heads are adjacent in memory (BSHD); the
//   loads are non-temporal since every byte is read once. The
//   block sum is accumulated in fp32 in token order, divided by the number
//   of tokens present, and written in canonical frequency order (dims 2j,
//   2j+1 = RoPE pair j). The squares of the pooled values are summed per
//   segment (high-only, middle, low-only) for the RMS energies. Two
//   persistent workgroups per CU take the work items in turn and hold their
//   results in LDS until their reads are done.
// tau_kernel: per query head, fixed-order fp64 sums of those segment
//   energies over all blocks give R = sqrt(energy / (nb * |D|)) for the
//   high band, the low band and the full spectrum of Qbar and Kbar, and
//   tau_z = R(Qbar,D_z) R(Kbar,D_z) / (R(Qbar,D_full) R(Kbar,D_full)) (the
//   adopted reading), or R(Qbar,D_z) R(Kbar,D_z) (unit-energy reading), or 1
//   (no temperature, and the per-vector reading, which scales per pooled
//   vector in the score kernel instead).
#include "prism_kernels.h"

namespace prism {
namespace {

constexpr int kThreads = 256;

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

// One work item = (tensor, block of B tokens, chunk of heads); this thread's
// place in it. Lanes of a token row: TPH per head, heads of the chunk
// adjacent; tokp token rows are read side by side.
template <bool FP32>
struct PoolItem {
  static constexpr int E = Elem<FP32>::E;
  static constexpr int TPH = kHeadDim / E;  // threads per head row
  int ts, i, lanes_per_tok, tokp, tp, hh, dg, h;
  bool active;
  __device__ PoolItem(const PoolArgs &a, int item) {
    int rem = item;
    ts = 0;
    const int nq = a.chunks[0] * a.nb;
    if (rem >= nq) { ts = 1; rem -= nq; }
    i = rem % a.nb;
    const int chunk = rem / a.nb;
    const int HC = a.heads_per_chunk[ts];
    lanes_per_tok = TPH * HC;
    tokp = kThreads / lanes_per_tok;
    const int tid = threadIdx.x;
    tp = tid / lanes_per_tok;
    hh = (tid % lanes_per_tok) / TPH;
    dg = tid % TPH;
    h = a.h0[ts] + chunk * HC + hh;
    active = tp < tokp && h < a.h0[ts] + a.nheads[ts];
  }
};

// Block sums of one work item, then the mean and the segment energies of
// this lane's dims, left in `st` (E means, then the three segment energies
// of the head row).
template <bool FP32>
__device__ __forceinline__ void pool_item(const PoolArgs &a, int batch, int item, float *red, float *st) {
  using El = Elem<FP32>;
  constexpr int E = El::E;
  constexpr int TPH = kHeadDim / E;
  const PoolItem<FP32> w(a, item);
  const TensorArg &x = a.x[w.ts];
  const int tid = threadIdx.x;
  const int t0 = w.i * a.block;
  const int n = min(a.block, a.seq - t0);

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;

  if (w.active) {
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

  // combine the token-parallel partial sums in a fixed order
  if (w.tokp > 1) {
    if (w.tp < w.tokp) {
#pragma unroll
      for (int e = 0; e < E; ++e) red[tid * E + e] = acc[e];
    }
    __syncthreads();
    if (w.tp == 0) {
      for (int k = 1; k < w.tokp; ++k) {
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += red[(tid + k * w.lanes_per_tok) * E + e];
      }
    }
  }

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

// Writes one work item's pooled row and energies from `st` (canonical order).
template <bool FP32>
__device__ __forceinline__ void pool_store(const PoolArgs &a, int batch, int item, const float *st) {
  constexpr int E = Elem<FP32>::E;
  const PoolItem<FP32> w(a, item);
  if (!w.active || w.tp != 0) return;
  const int64_t row = ((int64_t)batch * a.x[w.ts].heads + w.h) * a.nb + w.i;
  float *xb = a.xbar[w.ts] + row * kHeadDim;
  if (!a.half_layout) {
#pragma unroll
    for (int e = 0; e < E; e += 4)
      *reinterpret_cast<float4 *>(xb + w.dg * E + e) = make_float4(st[e], st[e + 1], st[e + 2], st[e + 3]);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int c = w.dg * E + e;
      const int cc = c < kHeadDim / 2 ? 2 * c : 2 * (c - kHeadDim / 2) + 1;
      xb[cc] = st[e];
    }
  }
  if (w.dg == 0) *reinterpret_cast<float4 *>(a.sq[w.ts] + row * 4) = make_float4(st[E], st[E + 1], st[E + 2], 0.f);
}

// Persistent: workgroup g takes work items g, g + G, ... (G = gridDim.x,
// two workgroups per CU). The results of up to kPoolSlots items wait in LDS
// and are written after those items' reads: stores issued in the middle of
// the read stream slow it (6.4 vs 5.9 TB/s at 128K when every workgroup's
// items fit the slots).
constexpr int kPoolSlots = 6;
template <bool FP32>
__global__ __launch_bounds__(kThreads) void pool_kernel(PoolArgs a) {
  constexpr int E = Elem<FP32>::E;
  __shared__ float red[kThreads * E];
  __shared__ float stash[kPoolSlots][kThreads * (E + 3)];
  const int total = (a.chunks[0] + a.chunks[1]) * a.nb;
  for (int first = blockIdx.x; first < total; first += kPoolSlots * gridDim.x) {
    int nst = 0;
    for (int item = first; item < total && nst < kPoolSlots; item += gridDim.x, ++nst) {
      pool_item<FP32>(a, blockIdx.y, item, red, stash[nst] + threadIdx.x * (E + 3));
      __syncthreads();  // `red` is reused by the next item
    }
    for (int k = 0; k < nst; ++k)
      pool_store<FP32>(a, blockIdx.y, first + k * (int)gridDim.x, stash[k] + threadIdx.x * (E + 3));
  }
}

__global__ __launch_bounds__(kThreads) void tau_kernel(TauArgs a) {
  __shared__ double red[6][kThreads];
  const int h = a.h0 + blockIdx.x;
  const int b = blockIdx.y;
  const int g = h / (a.hq / a.hkv);
  const float4 *qs = reinterpret_cast<const float4 *>(a.qsq) + ((int64_t)b * a.hq + h) * a.nb;
  const float4 *ks = reinterpret_cast<const float4 *>(a.ksq) + ((int64_t)b * a.hkv + g) * a.nb;
  double s[6] = {0, 0, 0, 0, 0, 0};
  for (int i = threadIdx.x; i < a.nb; i += kThreads) {
    const float4 x = qs[i];
    const float4 y = ks[i];
    s[0] += x.x; s[1] += x.y; s[2] += x.z;
    s[3] += y.x; s[4] += y.y; s[5] += y.z;
  }
#pragma unroll
  for (int k = 0; k < 6; ++k) red[k][threadIdx.x] = s[k];
  __syncthreads();
  for (int w = kThreads / 2; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) {
#pragma unroll
      for (int k = 0; k < 6; ++k) red[k][threadIdx.x] += red[k][threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double ov = a.overlap ? 1.0 : 0.0;
    const double nb = (double)a.nb;
    double r[6];
    for (int t = 0; t < 2; ++t) {
      const double e0 = red[3 * t][0], e1 = red[3 * t + 1][0], e2 = red[3 * t + 2][0];
      r[3 * t + 0] = sqrt((e0 + ov * e1) / (nb * a.d_high));
      r[3 * t + 1] = sqrt((e2 + ov * e1) / (nb * a.d_low));
      r[3 * t + 2] = sqrt((e0 + e1 + e2) / (nb * kHeadDim));
    }
    // FULLSPEC: band energy relative to the full spectrum; UNIT: band
    // energy alone; NONE and PERVEC: 1 (PERVEC scales per pooled vector)
    double th = 1.0, tl = 1.0;
    const bool okh = r[0] > 0 && r[3] > 0 && r[2] > 0 && r[5] > 0;
    const bool okl = r[1] > 0 && r[4] > 0 && r[2] > 0 && r[5] > 0;
    if (a.tau_mode == 0) {
      if (okh) th = (r[0] * r[3]) / (r[2] * r[5]);
      if (okl) tl = (r[1] * r[4]) / (r[2] * r[5]);
    } else if (a.tau_mode == 2) {
      if (okh) th = r[0] * r[3];
      if (okl) tl = r[1] * r[4];
    }
    float *out = a.tau + ((int64_t)b * a.hq + h) * 8;
    out[0] = (float)th; out[1] = (float)tl;
    out[2] = (float)r[0]; out[3] = (float)r[1]; out[4] = (float)r[2];
    out[5] = (float)r[3]; out[6] = (float)r[4]; out[7] = (float)r[5];
  }
}

// Adaptive bands, step 1: the pooled spectrum of one head of one tensor, the
// mean over blocks of each RoPE pair's energy (canonical dims 2j, 2j + 1), in
// fp64 with a fixed summation order (deterministic). Thread t sums pair
// t % 64 over blocks t / 64, t / 64 + 4, ...; the four partial sums are added
// in order.
__global__ __launch_bounds__(kThreads) void spectrum_kernel(SpectrumArgs a) {
  __shared__ double red[kThreads / 64][64];
  const int hh = blockIdx.x, b = blockIdx.y;
  const int t = hh < a.hq ? 0 : 1;
  const int H = t ? a.hkv : a.hq;
  const int h = t ? hh - a.hq : hh;
  const float *x = a.xbar[t] + ((int64_t)b * H + h) * a.nb * kHeadDim;
  const int pr = threadIdx.x & 63, grp = threadIdx.x >> 6;
  double acc = 0.0;
  for (int i = grp; i < a.nb; i += kThreads / 64) {
    const float2 v = *reinterpret_cast<const float2 *>(x + (int64_t)i * kHeadDim + 2 * pr);
    acc += (double)v.x * v.x + (double)v.y * v.y;
  }
  red[grp][pr] = acc;
  __syncthreads();
  if (threadIdx.x < 64) {
    double sum = 0.0;
#pragma unroll
    for (int g = 0; g < kThreads / 64; ++g) sum += red[g][pr];
    a.spec[((int64_t)b * (a.hq + a.hkv) + hh) * 64 + pr] = sum / a.nb;
  }
}

// Adaptive bands, step 2 (one workgroup per batch entry): P_j(h) = spectrum of
// query head h times that of its KV head; the reference share is the share of
// the static high band's d_high / 2 pairs in the mean of P over the query
// heads; head h's high band is [0, j_h) with j_h the smallest multiple of 8
// pairs whose cumulative share of P(h) reaches the reference (relative
// tolerance 1e-9), each band keeping at least 8 pairs, and its low band
// [j_h - o, 64) with o = (d_high + d_low - 128) / 2. Sums run in pair order
// in fp64. Then each head's temperatures from its bands' energies, as the
// tau kernel computes them (the energies of a band are the sum of its pairs').
__global__ __launch_bounds__(kThreads) void split_kernel(SplitArgs a) {
  __shared__ double mean_s[64];
  __shared__ double ref_share;
  const int b = blockIdx.x;
  const int G = a.hq / a.hkv;
  const double *sq = a.spec + (int64_t)b * (a.hq + a.hkv) * 64;
  const double *sk = sq + (int64_t)a.hq * 64;
  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    double m = 0.0;
    for (int h = 0; h < a.hq; ++h) m += sq[h * 64 + j] * sk[(h / G) * 64 + j];
    mean_s[j] = m / a.hq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double c = 0.0, cj0 = 0.0;
    for (int j = 0; j < 64; ++j) {
      c += mean_s[j];
      if (j == a.d_high / 2 - 1) cj0 = c;
    }
    ref_share = c > 0.0 ? cj0 / c : -1.0;
  }
  __syncthreads();
  const int o = (a.d_high + a.d_low - kHeadDim) / 2;
  const int lo_j = max(8, o), hi_j = min(56, 64 + o - 8);
  for (int h = threadIdx.x; h < a.hq; h += blockDim.x) {
    const double *pq = sq + h * 64, *pk = sk + (h / G) * 64;
    double tot = 0.0;
    for (int j = 0; j < 64; ++j) tot += pq[j] * pk[j];
    int jh = a.d_high / 2;
    if (tot > 0.0 && ref_share >= 0.0) {
      jh = hi_j;
      double c = 0.0;
      for (int j = 0; j < 64; ++j) {
        c += pq[j] * pk[j];
        if ((j + 1) % 8 == 0 && j + 1 >= lo_j && j + 1 <= hi_j && c / tot >= ref_share * (1.0 - 1e-9)) {
          jh = j + 1;
          break;
        }
      }
    }
    const int dh = 2 * jh, dl = kHeadDim - 2 * (jh - o), lstart = 2 * (jh - o);
    int32_t *sp = a.split + ((int64_t)b * a.hq + h) * 4;
    sp[0] = min(dh, lstart);
    sp[1] = max(dh, lstart);
    sp[2] = dh;
    sp[3] = dl;
    // band energies (sums of pair energies) and RMS
    double e[2][3] = {{0.0, 0.0, 0.0}, {0.0, 0.0, 0.0}};
    for (int j = 0; j < 64; ++j) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const double v = t ? pk[j] : pq[j];
        if (j < jh) e[t][0] += v;
        if (j >= jh - o) e[t][1] += v;
        e[t][2] += v;
      }
    }
    double r[6];
    for (int t = 0; t < 2; ++t) {
      r[3 * t + 0] = sqrt(e[t][0] / dh);
      r[3 * t + 1] = sqrt(e[t][1] / dl);
      r[3 * t + 2] = sqrt(e[t][2] / kHeadDim);
    }
    double th = 1.0, tl = 1.0;
    const bool okh = r[0] > 0 && r[3] > 0 && r[2] > 0 && r[5] > 0;
    const bool okl = r[1] > 0 && r[4] > 0 && r[2] > 0 && r[5] > 0;
    if (a.tau_mode == 0) {
      if (okh) th = (r[0] * r[3]) / (r[2] * r[5]);
      if (okl) tl = (r[1] * r[4]) / (r[2] * r[5]);
    } else if (a.tau_mode == 2) {
      if (okh) th = r[0] * r[3];
      if (okl) tl = r[1] * r[4];
    }
    float *out = a.tau + ((int64_t)b * a.hq + h) * 8;
    out[0] = (float)th; out[1] = (float)tl;
    out[2] = (float)r[0]; out[3] = (float)r[1]; out[4] = (float)r[2];
    out[5] = (float)r[3]; out[6] = (float)r[4]; out[7] = (float)r[5];
  }
}

}  // namespace

hipError_t launch_spectrum(const SpectrumArgs &a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(spectrum_kernel, dim3(a.hq + a.hkv, batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_split(const SplitArgs &a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(split_kernel, dim3(batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pool(const PoolArgs &a, int batch, int fp32, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = stream_device(s, &dev);
  if (e == hipSuccess) e = device_cu_count(dev, &cus);
  if (e != hipSuccess) return e;
  const int total = (a.chunks[0] + a.chunks[1]) * a.nb;
  const int wgs = 2 * (cus > 0 ? cus : 1);  // two resident workgroups per CU (LDS: 75 KB each)
  const dim3 grid(total < wgs ? total : wgs, batch);
  if (fp32) hipLaunchKernelGGL(pool_kernel<true>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(pool_kernel<false>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_tau(const TauArgs &a, int batch, hipStream_t s) {
  hipLaunchKernelGGL(tau_kernel, dim3(a.nh, batch), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace prism
