// Prism estimator, steps (5)-(7) (Prism review on paper.rainbus.top,
// pipeline paragraph): per query block i and branch z in {high, low}
//   L_z[i, j] = Qbar_z[i] . Kbar_z[j] / (tau_z sqrt(d_z)),  j in J(i)
//   S_z[i, :] = softmax over J(i) (j <= i when causal),
//   M_z[i, :] = Top-P of S_z[i, :] at mass p, and M = M_high OR M_low.
//
// One workgroup (8 waves) owns RT consecutive query blocks of one head.
// Phase 1: the score tile. Both band dot products come from one pass over
//   the 128 pooled dims split into three segments (high-only, middle,
//   low-only), on fp32 MFMA 16x16x4 (A = 16 key blocks, B = 16 query
//   blocks). Logits (already in log2 units) go to LDS as [branch][row][j].
// Phase 2: selection. One wave per (row, branch): max, exp2, the sum Z, then
//   the largest threshold T (fp32 bit pattern bisection) with
//   mass{e >= T} >= p * Z. Entries above T are kept, entries equal to T
//   are kept in ascending block order until the mass reaches p * Z. This is
//   the sorted-prefix definition (descending scores, equal scores by lower
//   index, shortest prefix with mass >= p) without a sort. The union of the
//   two branches is written as the mask row, zeros included.
#include "prism_kernels.h"

namespace prism {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ int wave_excl_scan_i(int v, int lane) {
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x - v;
}

// Top-P selection of one row held by the wave: element k of lane l is block
// j = 4*l + 256*(k/4) + k%4; x[k] are log2-unit logits (-inf when j is not
// admissible). Returns the selection bits (bit k) of this lane.
template <int EPL>
__device__ uint32_t select_row(const float (&x)[EPL], float p, int lane) {
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < EPL; ++k) mx = fmaxf(mx, x[k]);
  mx = wave_max(mx);
  float ex[EPL];
  float zl = 0.f;
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    ex[k] = (x[k] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x[k] - mx);
    zl += ex[k];
  }
  uint32_t valid = 0;
#pragma unroll
  for (int k = 0; k < EPL; ++k) valid |= (x[k] != -INFINITY ? 1u : 0u) << k;
  if (p >= 1.0f) return valid;
  const float Z = wave_sum(zl);
  const float target = p * Z;

  // invariant: mass(ex >= lo) >= target > mass(ex >= hi)
  uint32_t lo = 0u, hi = 0x3F800001u;  // every ex is <= 1.0f
  while (hi - lo > 1u) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    const float tm = __uint_as_float(mid);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < EPL; ++k) s += (ex[k] >= tm) ? ex[k] : 0.f;
    s = wave_sum(s);
    if (s >= target) lo = mid; else hi = mid;
  }
  const float T = __uint_as_float(lo);

  float above = 0.f;
  int ties = 0;
  uint32_t sel = 0, tie = 0;
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    if (ex[k] > T) { above += ex[k]; sel |= 1u << k; }
    if (ex[k] == T && ((valid >> k) & 1u)) { tie |= 1u << k; ++ties; }
  }
  above = wave_sum(above);
  ties = wave_sum_i(ties);
  // how many of the tied entries, in ascending block order, reach the target
  int need = 0;
  float acc = above;
  while (need < ties && acc < target) { acc += T; ++need; }
  if (need >= ties) return sel | tie;
  // rank the tied entries by block index: order is (k/4, lane, k%4)
  int base = 0;
#pragma unroll
  for (int e4 = 0; e4 < EPL / 4; ++e4) {
    const uint32_t tb = (tie >> (4 * e4)) & 0xFu;
    const int cnt = __popc(tb);
    int rank = base + wave_excl_scan_i(cnt, lane);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if ((tb >> m) & 1u) {
        if (rank < need) sel |= 1u << (4 * e4 + m);
        ++rank;
      }
    }
    base += wave_sum_i(cnt);
  }
  return sel;
}

template <int RT, int EPL>
__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a) {
  constexpr int NBP = 64 * EPL + 4;  // LDS row length in floats (padded)
  __shared__ __attribute__((aligned(16))) float lds[2 * RT * NBP];

  const int nb = a.nb;
  const int ntiles = (nb + RT - 1) / RT;
  const int nbh = a.hq * a.batch;
  const int bid = blockIdx.x;
  const int tile = a.causal ? (ntiles - 1 - bid / nbh) : (bid / nbh);  // longest rows first
  const int bh = bid % nbh;
  const int b = bh / a.hq;
  const int h = bh % a.hq;
  const int g = h / (a.hq / a.hkv);
  const int i0 = tile * RT;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kq = lane >> 4;   // k slot of the MFMA operands
  const int c16 = lane & 15;  // row of A / column of B

  const float *tau = a.tau + ((int64_t)b * a.hq + h) * 8;
  const float kLog2e = 1.4426950408889634f;
  const float ah = kLog2e / (tau[0] * sqrtf((float)a.d_high));
  const float al = kLog2e / (tau[1] * sqrtf((float)a.d_low));
  const float ov = a.overlap ? 1.f : 0.f;

  // ---- phase 1: logits of rows i0..i0+RT-1 against key blocks 0..ncols-1
  const int ncols = a.causal ? min(nb, i0 + RT) : nb;
  {
    const float *qb = a.qbar + ((int64_t)b * a.hq + h) * nb * kHeadDim;
    const float *kb = a.kbar + ((int64_t)b * a.hkv + g) * nb * kHeadDim;
    const int iq = i0 + c16;
    f32x4 qv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (iq < nb && c16 < RT) {
        const float4 t = *reinterpret_cast<const float4 *>(qb + (int64_t)iq * kHeadDim + 16 * q + 4 * kq);
        qv[q] = f32x4{t.x, t.y, t.z, t.w};
      } else {
        qv[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    const int seg_lo[3] = {0, a.seg_lo, a.seg_hi};
    const int seg_hi[3] = {a.seg_lo, a.seg_hi, kHeadDim};
    const int nct = (ncols + 15) / 16;
    for (int jt = wave; jt < nct; jt += kWaves) {
      const int j0 = jt * 16;
      const int jk = j0 + c16;
      f32x4 kv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (jk < nb) {
          const float4 t = *reinterpret_cast<const float4 *>(kb + (int64_t)jk * kHeadDim + 16 * q + 4 * kq);
          kv[q] = f32x4{t.x, t.y, t.z, t.w};
        } else {
          kv[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      f32x4 acc[3];
#pragma unroll
      for (int s = 0; s < 3; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
#pragma unroll
        for (int s = 0; s < 3; ++s) {
          const int lo = seg_lo[s], hi = seg_hi[s];
          if (16 * q >= hi || 16 * q + 16 <= lo) continue;
          const bool whole = 16 * q >= lo && 16 * q + 16 <= hi;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int dim = 16 * q + 4 * kq + e;
            const float av = (whole || (dim >= lo && dim < hi)) ? kv[q][e] : 0.f;
            acc[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, qv[q][e], acc[s], 0, 0, 0);
          }
        }
      }
      // acc[s][r] = segment-s dot of key block j0 + 4*kq + r with query block i0 + c16
      if (c16 < RT) {
        const int i = i0 + c16;
        float lh[4], ll[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + 4 * kq + r;
          const bool ok = j < nb && (!a.causal || j <= i);
          lh[r] = ok ? (acc[0][r] + ov * acc[1][r]) * ah : -INFINITY;
          ll[r] = ok ? (acc[2][r] + ov * acc[1][r]) * al : -INFINITY;
        }
        *reinterpret_cast<float4 *>(&lds[(0 * RT + c16) * NBP + j0 + 4 * kq]) = make_float4(lh[0], lh[1], lh[2], lh[3]);
        *reinterpret_cast<float4 *>(&lds[(1 * RT + c16) * NBP + j0 + 4 * kq]) = make_float4(ll[0], ll[1], ll[2], ll[3]);
      }
    }
  }
  __syncthreads();

  // ---- phase 2: softmax + Top-P per branch, union, mask row
  for (int r = wave; r < RT; r += kWaves) {
    const int i = i0 + r;
    if (i >= nb) continue;
    const int nc = a.causal ? i + 1 : nb;
    uint32_t bits = 0;
#pragma unroll
    for (int z = 0; z < 2; ++z) {
      const float *row = &lds[(z * RT + r) * NBP];
      float x[EPL];
#pragma unroll
      for (int e4 = 0; e4 < EPL / 4; ++e4) {
        const int j = 4 * lane + 256 * e4;
        float4 t = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        if (j < nc) t = *reinterpret_cast<const float4 *>(row + j);
        x[4 * e4 + 0] = t.x;
        x[4 * e4 + 1] = (j + 1 < nc) ? t.y : -INFINITY;
        x[4 * e4 + 2] = (j + 2 < nc) ? t.z : -INFINITY;
        x[4 * e4 + 3] = (j + 3 < nc) ? t.w : -INFINITY;
      }
      bits |= select_row<EPL>(x, a.p, lane);
    }
    uint8_t *mrow = a.mask + (((int64_t)b * a.hq + h) * nb + i) * nb;
#pragma unroll
    for (int e4 = 0; e4 < EPL / 4; ++e4) {
      const int j = 4 * lane + 256 * e4;
      const uint32_t nib = (bits >> (4 * e4)) & 0xFu;
      if ((nb & 3) == 0) {
        if (j < nb) {
          const uint32_t word = (nib & 1u) | ((nib >> 1) & 1u) << 8 | ((nib >> 2) & 1u) << 16 | ((nib >> 3) & 1u) << 24;
          *reinterpret_cast<uint32_t *>(mrow + j) = word;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (j + m < nb) mrow[j + m] = (uint8_t)((nib >> m) & 1u);
      }
    }
  }
}

}  // namespace

hipError_t launch_select(const SelectArgs &a, hipStream_t s) {
  if (a.nb <= 1024) {
    constexpr int RT = 16;
    const int ntiles = (a.nb + RT - 1) / RT;
    hipLaunchKernelGGL((select_kernel<RT, 16>), dim3(ntiles * a.hq * a.batch), dim3(kThreads), 0, s, a);
  } else {
    constexpr int RT = 8;
    const int ntiles = (a.nb + RT - 1) / RT;
    hipLaunchKernelGGL((select_kernel<RT, 32>), dim3(ntiles * a.hq * a.batch), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace prism
