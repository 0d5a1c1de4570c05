// Prism estimator, steps (5)-(7) (Prism review on paper.rainbus.top,
// pipeline paragraph): per query block i and branch z in {high, low}
//   L_z[i, j] = Qbar_z[i] . Kbar_z[j] / (tau_z sqrt(d_z)),  j in J(i)
//   S_z[i, :] = softmax over J(i) (j <= i when causal),
//   M_z[i, :] = Top-P of S_z[i, :] at mass p, and M = M_high OR M_low.
//
// One workgroup (8 waves) owns RT consecutive query blocks of one head and
// runs the two branches one after the other (each band is one contiguous
// range of canonical dims), so one branch's logits fit in ~66 KB of LDS and
// two workgroups share a CU.
// Phase 1: the score tile on fp32 MFMA 16x16x4 (A = 16 key blocks, B = 16
//   query blocks) over the band's dims; 4 waves per SIMD keep key-tile loads
//   in flight. Logits (in log2 units) go to LDS.
// Phase 2: selection, one wave per (row, branch), exact and sort-free:
//   * max, e_j = exp2(L_j - max), and integer masses m_j = e_j * 2^31
//     (fixed point, so every sum is exact and independent of order);
//   * a 64-bin histogram of the masses over e's exponent and top two
//     mantissa bits (quarter octaves, monotone in e) by LDS atomics;
//   * a wave scan over the bins from the top finds the bin b* where the
//     cumulative mass first reaches p * Z: bins above b* are kept, bins below
//     are dropped;
//   * the (usually few) entries of b* are ranked exactly by (value
//     descending, block index ascending); an entry is kept when the mass
//     ranked before it is still short of p * Z.
//   This is the sorted-prefix definition (shortest prefix of the descending
//   order with mass >= p, equal scores by lower index) without a sort. A bin
//   holding more than 64 entries falls back to a bisection over the fp32 bit
//   pattern of the threshold. The first branch's selection stays in
//   registers; the union of both is written as the mask row, zeros included.
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

// per-wave LDS scratch of the histogram selection
struct WaveHist {
  unsigned long long bin[64];  // (count << 52) | fixed-point mass
  uint32_t cand_key[64];       // the threshold bin's entries: value bits
  uint32_t cand_j[64];         //   and block index
};

__device__ __forceinline__ unsigned long long shfl_up_u64(unsigned long long v, int off) {
  const int lo = __shfl_up((int)(uint32_t)v, off);
  const int hi = __shfl_up((int)(uint32_t)(v >> 32), off);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int off) {
  const int lo = __shfl_xor((int)(uint32_t)v, off);
  const int hi = __shfl_xor((int)(uint32_t)(v >> 32), off);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}

// histogram bin of a positive e (bit pattern): quarter octaves from e = 1
__device__ __forceinline__ int bin_of(uint32_t ebits) { return min(max(508 - (int)(ebits >> 21), 0), 63); }

constexpr float kMassScale = 2147483648.0f;  // fixed point: mass = e * 2^31, e <= 1
__device__ __forceinline__ uint32_t fixed_mass(uint32_t ebits) {
  return (uint32_t)(__uint_as_float(ebits) * kMassScale);
}

// Top-P of one row held by the wave (element k of lane l is block
// j = 4*l + 256*(k/4) + k%4; x[k] are log2-unit logits, -inf when j is not
// admissible; ne4 = number of 4-element slots that hold admissible blocks).
// Radix select on the bit pattern of e = exp2(x - max) (monotone in e):
// each level histograms the still-undecided entries into 64 bins with exact
// fixed-point masses, keeps every bin above the one where the cumulative
// mass reaches p * Z, drops every bin below, and refines that bin (next 6
// key bits, or the next 64 quarter octaves of the tail) until at most 64
// entries remain, which are ranked exactly by (value desc, index asc).
// Returns this lane's selection bits, or sets *fallback if eight levels did
// not resolve the row.
template <int EPL>
__device__ uint32_t select_row_hist(const float (&x)[EPL], int ne4, float p, int lane, WaveHist &H,
                                    bool *fallback) {
  *fallback = false;
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < EPL; ++k) mx = fmaxf(mx, x[k]);
  mx = wave_max(mx);
  uint32_t valid = 0;
#pragma unroll
  for (int k = 0; k < EPL; ++k) valid |= (x[k] != -INFINITY ? 1u : 0u) << k;
  if (p >= 1.0f) return valid;

  // key = bit pattern of e; 0 marks an entry that is not admissible or whose
  // e underflowed to 0 (never needed, since p * Z <= Z)
  uint32_t key[EPL];
  uint32_t act = 0;  // entries still undecided
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    key[k] = 0u;
    if (k / 4 < ne4 && ((valid >> k) & 1u)) key[k] = __float_as_uint(__builtin_amdgcn_exp2f(x[k] - mx));
    act |= (key[k] ? 1u : 0u) << k;
  }
  unsigned long long Z = 0, target = 0, before = 0;
  uint32_t sel = 0;
  int shift = 21, base = 508;  // level 0: quarter octaves below e = 1 ...
  bool tail = true;            // ... with everything smaller in bin 63
  for (int level = 0; level < 8; ++level) {
    H.bin[lane] = 0ull;
#pragma unroll
    for (int k = 0; k < EPL; ++k)
      if ((act >> k) & 1u)
        atomicAdd(&H.bin[min(max(base - (int)(key[k] >> shift), 0), 63)], (1ull << 52) | fixed_mass(key[k]));
    const unsigned long long hv = H.bin[lane];
    const unsigned long long mass = hv & ((1ull << 52) - 1ull);
    unsigned long long cum = mass;  // inclusive scan, largest values first
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned long long y = shfl_up_u64(cum, off);
      if (lane >= off) cum += y;
    }
    if (level == 0) {
      Z = readlane_u64(cum, 63);
      target = (unsigned long long)ceil((double)Z * (double)p);
    }
    const unsigned long long need = target - before;  // > 0 at every level
    const int bstar = __ffsll((long long)__ballot(cum >= need)) - 1;
    before += readlane_u64(cum, bstar) - readlane_u64(mass, bstar);
    const uint32_t c = (uint32_t)(readlane_u64(hv, bstar) >> 52);
    uint32_t nact = 0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      if ((act >> k) & 1u) {
        const int bk = min(max(base - (int)(key[k] >> shift), 0), 63);
        if (bk < bstar) sel |= 1u << k;
        if (bk == bstar) nact |= 1u << k;
      }
    }
    act = nact;
    if (c <= 64u) break;
    if (tail && bstar == 63) {
      base -= 64;  // the next 64 quarter octaves
      if (base < 63) break;  // only vanishing masses left; ranked below
    } else if (shift > 0) {
      const int bits = shift >= 6 ? 6 : shift;
      shift -= bits;
      base = ((base - bstar) << bits) + (1 << bits) - 1;
      tail = false;
    } else {
      break;  // all undecided entries share one value; ranked by index below
    }
    if (level == 7) {
      *fallback = true;
      return 0;
    }
  }
  // rank the undecided entries by (value desc, index asc); keep each entry
  // whose ranked-before mass is still short of the target
  int pos = 0;
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    if (k / 4 < ne4) {
      const bool is = (act >> k) & 1u;
      const uint64_t bal = __ballot(is);
      const int at = pos + __popcll(bal & ((1ull << lane) - 1ull));
      if (is && at < 64) {
        H.cand_key[at] = key[k];
        H.cand_j[at] = 4 * lane + 256 * (k / 4) + (k & 3);
      }
      pos += __popcll(bal);
    }
  }
  if (pos > 64) {
    // many undecided entries: exact by count when they share one value
    // (equal masses; index order is (k/4, lane, k%4)), else the fallback
    uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
    for (int k = 0; k < EPL; ++k)
      if ((act >> k) & 1u) { kmin = min(kmin, key[k]); kmax = max(kmax, key[k]); }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
    }
    if (kmin != kmax) {
      *fallback = true;
      return 0;
    }
    const unsigned long long m = fixed_mass(kmin);
    const unsigned long long take = (target - before + m - 1) / m;  // entries needed, >= 1
    unsigned long long rank0 = 0;
#pragma unroll
    for (int e4 = 0; e4 < EPL / 4; ++e4) {
      const uint32_t nib = (act >> (4 * e4)) & 0xFu;
      const int cnt = __popc(nib);
      int r = (int)rank0 + wave_excl_scan_i(cnt, lane);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if ((nib >> q) & 1u) {
          if ((unsigned long long)r < take) sel |= 1u << (4 * e4 + q);
          ++r;
        }
      rank0 += (unsigned long long)wave_sum_i(cnt);
    }
    return sel;
  }
  const int cn = pos;
  const uint32_t mk = lane < cn ? H.cand_key[lane] : 0u;
  const uint32_t mj = lane < cn ? H.cand_j[lane] : 0u;
  unsigned long long ahead = 0;  // mass ranked before this entry
  for (int q = 0; q < cn; q += 4) {
    uint32_t kk[4], jj[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kk[u] = q + u < cn ? H.cand_key[q + u] : 0u;
      jj[u] = q + u < cn ? H.cand_j[q + u] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (kk[u] > mk || (kk[u] == mk && jj[u] < mj)) ahead += fixed_mass(kk[u]);
  }
  const bool chosen = lane < cn && before + ahead < target;
  // the last chosen entry in rank order: smallest value, then largest index
  unsigned long long cut = chosen ? (((unsigned long long)mk << 11) | (unsigned long long)(2047u - mj)) : ~0ull;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long y = shfl_xor_u64(cut, off);
    cut = y < cut ? y : cut;
  }
  const uint32_t cut_key = (uint32_t)(cut >> 11);
  const uint32_t cut_j = 2047u - (uint32_t)(cut & 2047ull);
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    if ((act >> k) & 1u) {
      const uint32_t j = 4 * lane + 256 * (k / 4) + (k & 3);
      if (key[k] > cut_key || (key[k] == cut_key && j <= cut_j)) sel |= 1u << k;
    }
  }
  return sel;
}

template <int RT, int EPL>
__global__ __launch_bounds__(kThreads, EPL <= 16 ? 4 : 2) void select_kernel(SelectArgs a) {
  constexpr int NBP = 64 * EPL + 4;  // LDS row length in floats (padded)
  __shared__ __attribute__((aligned(16))) float lds[RT * NBP];  // one branch's logits
  __shared__ WaveHist whist[kWaves];

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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kq = lane >> 4;   // k slot of the MFMA operands
  const int c16 = lane & 15;  // row of A / column of B

  const float *tau = a.tau + ((int64_t)b * a.hq + h) * 8;
  const float kLog2e = 1.4426950408889634f;
  const float *qb = a.qbar + ((int64_t)b * a.hq + h) * nb * kHeadDim;
  const float *kb = a.kbar + ((int64_t)b * a.hkv + g) * nb * kHeadDim;
  const int ncols = a.causal ? min(nb, i0 + RT) : nb;
  const int nct = (ncols + 15) / 16;
  const int iq = i0 + c16;

  // selection bits of this wave's rows (r = wave + kWaves * x), per branch
  constexpr int RPW = (RT + kWaves - 1) / kWaves;
  uint32_t bits[RPW];
#pragma unroll
  for (int x = 0; x < RPW; ++x) bits[x] = 0;

#pragma unroll 1
  for (int z = 0; z < 2; ++z) {
    // the branch's band is the canonical dim range [dlo, dhi)
    const int dlo = z == 0 ? 0 : kHeadDim - a.d_low;
    const int dhi = z == 0 ? a.d_high : kHeadDim;
    const float scale = kLog2e / (tau[z] * sqrtf((float)(dhi - dlo)));
    const int g0 = dlo >> 4, g1 = (dhi + 15) >> 4;  // 16-dim groups the band touches

    // ---- phase 1: logits of rows i0..i0+RT-1 against key blocks 0..ncols-1
    f32x4 qv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      qv[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (q >= g0 && q < g1 && iq < nb && c16 < RT) {
        const float4 t = *reinterpret_cast<const float4 *>(qb + (int64_t)iq * kHeadDim + 16 * q + 4 * kq);
        qv[q] = f32x4{t.x, t.y, t.z, t.w};
      }
    }
    auto load_k = [&](int jt, f32x4 (&kv)[8]) {
      const int jk = jt * 16 + c16;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        kv[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (q >= g0 && q < g1 && jk < nb) {
          const float4 t = *reinterpret_cast<const float4 *>(kb + (int64_t)jk * kHeadDim + 16 * q + 4 * kq);
          kv[q] = f32x4{t.x, t.y, t.z, t.w};
        }
      }
    };
    for (int jt = wave; jt < nct; jt += kWaves) {
      f32x4 kv[8];
      load_k(jt, kv);
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (q < g0 || q >= g1) continue;
        const bool whole = 16 * q >= dlo && 16 * q + 16 <= dhi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dim = 16 * q + 4 * kq + e;
          const float av = (whole || (dim >= dlo && dim < dhi)) ? kv[q][e] : 0.f;
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, qv[q][e], acc, 0, 0, 0);
        }
      }
      // acc[r] = band dot of key block j0 + 4*kq + r with query block i0 + c16
      if (c16 < RT) {
        const int j0 = jt * 16;
        const int i = i0 + c16;
        float l4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + 4 * kq + r;
          l4[r] = (j < nb && (!a.causal || j <= i)) ? acc[r] * scale : -INFINITY;
        }
        *reinterpret_cast<float4 *>(&lds[c16 * NBP + j0 + 4 * kq]) = make_float4(l4[0], l4[1], l4[2], l4[3]);
      }
    }
    __syncthreads();

    // ---- phase 2: softmax + Top-P of this branch for the wave's rows
#pragma unroll
    for (int x = 0; x < RPW; ++x) {
      const int r = wave + kWaves * x;
      const int i = i0 + r;
      if (r >= RT || i >= nb) continue;
      const int nc = a.causal ? i + 1 : nb;
      auto load_row = [&](float (&xr)[EPL]) {
        const float *row = &lds[r * NBP];
#pragma unroll
        for (int e4 = 0; e4 < EPL / 4; ++e4) {
          const int j = 4 * lane + 256 * e4;
          float4 t = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
          if (j < nc) t = *reinterpret_cast<const float4 *>(row + j);
          xr[4 * e4 + 0] = t.x;
          xr[4 * e4 + 1] = (j + 1 < nc) ? t.y : -INFINITY;
          xr[4 * e4 + 2] = (j + 2 < nc) ? t.z : -INFINITY;
          xr[4 * e4 + 3] = (j + 3 < nc) ? t.w : -INFINITY;
        }
      };
      bool fallback;
      uint32_t bz;
      {
        float xr[EPL];
        load_row(xr);
        bz = select_row_hist<EPL>(xr, (nc + 255) / 256, a.p, lane, whist[wave], &fallback);
      }
      if (fallback) {
        float xr[EPL];
        load_row(xr);
        bz = select_row<EPL>(xr, a.p, lane);
      }
      bits[x] |= bz;
    }
    __syncthreads();  // the next branch overwrites the logits
  }

  // ---- union of the branches -> mask rows, zeros included
#pragma unroll
  for (int x = 0; x < RPW; ++x) {
    const int r = wave + kWaves * x;
    const int i = i0 + r;
    if (r >= RT || i >= nb) continue;
    uint8_t *mrow = a.mask + (((int64_t)b * a.hq + h) * nb + i) * nb;
#pragma unroll
    for (int e4 = 0; e4 < EPL / 4; ++e4) {
      const int j = 4 * lane + 256 * e4;
      const uint32_t nib = (bits[x] >> (4 * e4)) & 0xFu;
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
