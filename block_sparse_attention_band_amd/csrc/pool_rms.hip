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
#include "pool_device.h"

namespace prism {
namespace {

constexpr int kThreads = kPoolThreads;

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
  const int total = pool_items(a);
  const int tid = threadIdx.x;
  for (int first = blockIdx.x; first < total; first += kPoolSlots * gridDim.x) {
    int nst = 0;
    for (int item = first; item < total && nst < kPoolSlots; item += gridDim.x, ++nst) {
      const PoolItem<FP32> w(a, item, tid);
      float acc[E];
      pool_accum<FP32>(a, blockIdx.y, w, acc);
      if (w.tokp > 1) {
        pool_red_put<FP32>(w, tid, acc, red);
        __syncthreads();
      }
      pool_finish<FP32>(a, w, tid, acc, red, stash[nst] + tid * (E + 3));
      __syncthreads();  // `red` is reused by the next item
    }
    for (int k = 0; k < nst; ++k) {
      const float *st = stash[k] + tid * (E + 3);
      pool_write<FP32>(a, blockIdx.y, PoolItem<FP32>(a, first + k * (int)gridDim.x, tid), st, st + E);
    }
  }
}

__global__ __launch_bounds__(kThreads) void tau_kernel(TauArgs a) {
  __shared__ double red[6][kThreads];
  const int h = a.h0 + blockIdx.x;
  const int b = blockIdx.y;
  float t[8];
  tau_reduce(a, b, h, red, t);
  if (threadIdx.x == 0) {
    float *out = a.tau + ((int64_t)b * a.hq + h) * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) out[k] = t[k];
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
  const int total = pool_items(a);
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
