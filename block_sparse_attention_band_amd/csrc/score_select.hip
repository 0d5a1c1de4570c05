// Prism estimator, steps (5)-(7) (Prism review on paper.rainbus.top,
// pipeline paragraph): per query block i and branch z in {high, low}
//   L_z[i, j] = Qbar_z[i] . Kbar_z[j] / (tau_z sqrt(d_z)),  j in J(i)
//   S_z[i, :] = softmax over J(i) (j <= i when causal),
//   M_z[i, :] = Top-P of S_z[i, :] at mass p, and M = M_high OR M_low.
//
// score_kernel: both branches' logits in one pass. The canonical dims split
//   into three segments, high-only / middle / low-only; each 64 x 64 tile of
//   (query block, key block) pairs accumulates the three segment dot products
//   on fp32 MFMA 32x32x2 (every dim enters once), then
//   L_high = (s0 + s1) * c_high and L_low = (s1 + s2) * c_low (the middle
//   segment only when the bands overlap), in log2 units, go to the logit
//   planes of the workspace.
// topp_kernel: one wave per (row, both branches); exact and sort-free:
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
//   holding more than 64 entries is refined on the next key bits; rows that
//   stay unresolved fall back to a bisection over the fp32 bit pattern of
//   the threshold. The first branch's selection stays in registers; the
//   union of both is written as the mask row (bytes or bits), zeros
//   included.
// topp_long_kernel: rows of more than 2048 blocks (up to 8192), which do not
//   fit in registers: the same rule by a five-pass radix select on the key
//   over the same fixed-point masses, the row re-read from the logit plane at
//   every pass.
#include "prism_kernels.h"

namespace prism {
namespace {


// ---- wave-wide scans and reductions on DPP: Hillis-Steele shifts within
// each 16-lane row, then the row broadcasts (lane 15 -> rows 1 and 3, lane
// 31 -> rows 2 and 3). Lane 63 ends with the whole wave's result. No LDS
// round trips, unlike lane shuffles.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint64_t dpp64(uint64_t old, uint64_t x) {
  const uint32_t lo = dpp<CTRL, ROWS>((uint32_t)old, (uint32_t)x);
  const uint32_t hi = dpp<CTRL, ROWS>((uint32_t)(old >> 32), (uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118;
constexpr int kBcast15 = 0x142, kBcast31 = 0x143;

// inclusive prefix sum over lanes 0..l (lanes shifted in from outside a
// row, and rows a broadcast skips, add 0)
__device__ __forceinline__ uint32_t scan_add(uint32_t x) {
  x += dpp<kShr1>(0u, x);
  x += dpp<kShr2>(0u, x);
  x += dpp<kShr4>(0u, x);
  x += dpp<kShr8>(0u, x);
  x += dpp<kBcast15, 0xA>(0u, x);
  x += dpp<kBcast31, 0xC>(0u, x);
  return x;
}
__device__ __forceinline__ unsigned long long scan_add(unsigned long long x) {
  x += dpp64<kShr1>(0ull, x);
  x += dpp64<kShr2>(0ull, x);
  x += dpp64<kShr4>(0ull, x);
  x += dpp64<kShr8>(0ull, x);
  x += dpp64<kBcast15, 0xA>(0ull, x);
  x += dpp64<kBcast31, 0xC>(0ull, x);
  return x;
}
__device__ __forceinline__ float scan_add(float x) {
  x += __uint_as_float(dpp<kShr1>(0u, __float_as_uint(x)));
  x += __uint_as_float(dpp<kShr2>(0u, __float_as_uint(x)));
  x += __uint_as_float(dpp<kShr4>(0u, __float_as_uint(x)));
  x += __uint_as_float(dpp<kShr8>(0u, __float_as_uint(x)));
  x += __uint_as_float(dpp<kBcast15, 0xA>(0u, __float_as_uint(x)));
  x += __uint_as_float(dpp<kBcast31, 0xC>(0u, __float_as_uint(x)));
  return x;
}
// running min / max: lanes without a source keep their own value, which
// min and max leave unchanged, so no identity element is needed
template <typename Op>
__device__ __forceinline__ uint32_t scan_keep(uint32_t x, Op op) {
  x = op(x, dpp<kShr1>(x, x));
  x = op(x, dpp<kShr2>(x, x));
  x = op(x, dpp<kShr4>(x, x));
  x = op(x, dpp<kShr8>(x, x));
  x = op(x, dpp<kBcast15, 0xA>(x, x));
  x = op(x, dpp<kBcast31, 0xC>(x, x));
  return x;
}

__device__ __forceinline__ uint32_t lane63(uint32_t v) { return __builtin_amdgcn_readlane(v, 63); }
__device__ __forceinline__ unsigned long long lane63(unsigned long long v) {
  // readlane returns int: widen each half as unsigned (no sign extension)
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ float wave_max(float v) {
  const uint32_t r = scan_keep(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  });
  return __uint_as_float(lane63(r));
}
__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
  return lane63(scan_keep(v, [](uint32_t a, uint32_t b) { return b < a ? b : a; }));
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
  return lane63(scan_keep(v, [](uint32_t a, uint32_t b) { return b > a ? b : a; }));
}
__device__ __forceinline__ float wave_sum(float v) { return __uint_as_float(lane63(__float_as_uint(scan_add(v)))); }
__device__ __forceinline__ int wave_sum_i(int v) { return (int)lane63(scan_add((uint32_t)v)); }
__device__ __forceinline__ int wave_excl_scan_i(int v, int) { return (int)scan_add((uint32_t)v) - v; }

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
  uint32_t cand_key[64];       // the threshold bin's entries (value bits), ascending block order
  uint32_t cand_keep[64];      // their selection flags
};

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

// The lanes of one wave exchange data through LDS (histogram bins,
// candidate lists). The hardware runs a wave's LDS instructions in order; this
// fence keeps the compiler from reordering accesses across the exchange point
// or forwarding a lane's own earlier store to its later load.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Radix state: the bin of key y is clamp(base - (y >> shift), 0, 63). Level 0
// bins quarter octaves of e below 1 (base 508 = 4 * 127, shift 21) with every
// smaller e in bin 63 (tail). Refining bin b* either moves the tail window
// down so that its bin 0 is the old bin 63's top quarter octave (every bin
// then holds exactly one value of y >> shift, except the new tail), or splits
// b* on the next (up to) 6 key bits. Returns false when the keys of b* cannot
// be split further (all equal) or only masses that round to 0 remain.
struct Radix {
  int shift = 21, base = 508;
  bool tail = true;
  __device__ int bin(uint32_t y) const { return min(max(base - (int)(y >> shift), 0), 63); }
  __device__ bool refine(int bstar) {
    if (tail && bstar == 63) {
      base -= 63;
      return base >= 63;
    }
    if (shift == 0) return false;
    const int bits = shift >= 6 ? 6 : shift;
    shift -= bits;
    base = ((base - bstar) << bits) + (1 << bits) - 1;
    tail = false;
    return true;
  }
};

// One histogram pass: entries with `in` set add (1 << 52 | mass) to their
// bin; returns the threshold bin b* (cumulative mass from the top reaches the
// target there), adds the mass of the bins above it to `before` and returns
// b*'s entry count in *count. At the first pass (*Z == 0) it also sets Z and
// the target ceil(p * Z).
struct Hist {
  __device__ static int pass_done(WaveHist &H, int lane, float p, unsigned long long &Z, unsigned long long &target,
                                  unsigned long long &before, uint32_t *count) {
    wave_lds_sync();
    const unsigned long long hv = H.bin[lane];
    const unsigned long long mass = hv & ((1ull << 52) - 1ull);
    const unsigned long long cum = scan_add((unsigned long long)mass);  // largest values first
    if (Z == 0) {
      Z = readlane_u64(cum, 63);
      target = (unsigned long long)ceil((double)Z * (double)p);
    }
    const unsigned long long need = target - before;  // > 0 at every pass
    const int bstar = __ffsll((long long)__ballot(cum >= need)) - 1;
    before += readlane_u64(cum, bstar) - readlane_u64(mass, bstar);
    *count = (uint32_t)(readlane_u64(hv, bstar) >> 52);
    return bstar;
  }
};

// Top-P of one row held by the wave (element k of lane l is block
// j = 4*l + 256*(k/4) + k%4; x[k] are log2-unit logits, -inf when j is not
// admissible; slots k/4 >= ne4 hold no admissible block).
// Radix select on the bit pattern of e = exp2(x - max) (monotone in e) with
// exact fixed-point masses: each pass histograms the undecided entries into
// 64 bins, keeps every bin above the one where the cumulative mass reaches
// p * Z, drops every bin below, and goes on with that bin. Passes run over
// all entries while the bin holds more than 64 of them; then its entries are
// compacted in ascending block order (one per lane) and refined there until
// one entry decides or the rest share one value, which are taken by block
// index. This is the shortest prefix of the (value desc, index asc) order
// whose mass reaches p * Z. Returns this lane's selection bits, or sets
// *fallback when the passes cannot resolve the row.
template <int EPL>
__device__ uint32_t select_row_hist(const float (&x)[EPL], int ne4, float p, int lane, WaveHist &H,
                                    bool *fallback) {
  *fallback = false;
  float mx = -INFINITY;
#pragma unroll
  for (int e4 = 0; e4 < EPL / 4; ++e4) {
    if (e4 >= ne4) break;
#pragma unroll
    for (int m = 0; m < 4; ++m) mx = fmaxf(mx, x[4 * e4 + m]);
  }
  mx = wave_max(mx);
  if (p >= 1.0f) {
    uint32_t valid = 0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) valid |= (x[k] != -INFINITY ? 1u : 0u) << k;
    return valid;
  }

  // key = bit pattern of e (exp2(-inf) = 0 marks an entry that is not
  // admissible; an e that underflows to 0 is never needed since p * Z <= Z).
  // The first histogram pass runs while the keys are made.
  uint32_t key[EPL];
#pragma unroll
  for (int k = 0; k < EPL; ++k) key[k] = 0u;
  Radix R;
  H.bin[lane] = 0ull;
  wave_lds_sync();
#pragma unroll
  for (int e4 = 0; e4 < EPL / 4; ++e4) {
    if (e4 >= ne4) break;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int k = 4 * e4 + m;
      key[k] = __float_as_uint(__builtin_amdgcn_exp2f(x[k] - mx));
      if (key[k]) atomicAdd(&H.bin[R.bin(key[k])], (1ull << 52) | fixed_mass(key[k]));
    }
  }
  unsigned long long Z = 0, target = 0, before = 0;
  uint32_t sel = 0, c = 0, act = 0;
  int bstar = 0;
  for (int level = 0;; ++level) {
    if (level > 0) {
      H.bin[lane] = 0ull;
      wave_lds_sync();
#pragma unroll
      for (int e4 = 0; e4 < EPL / 4; ++e4) {
        if (e4 >= ne4) break;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int k = 4 * e4 + m;
          if ((act >> k) & 1u) atomicAdd(&H.bin[R.bin(key[k])], (1ull << 52) | fixed_mass(key[k]));
        }
      }
    }
    bstar = Hist::pass_done(H, lane, p, Z, target, before, &c);
    wave_lds_sync();
    // bins above b* hold keys >= hi_key, b* holds [lo_key, hi_key) (the tail
    // bin everything below hi_key); at level 0 every nonzero key is undecided
    const uint32_t hi_key = (uint32_t)(R.base - bstar + 1) << R.shift;
    const uint32_t lo_key = (R.tail && bstar == 63) ? 1u : (uint32_t)(R.base - bstar) << R.shift;
    uint32_t nact = 0;
#pragma unroll
    for (int e4 = 0; e4 < EPL / 4; ++e4) {
      if (e4 >= ne4) break;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int k = 4 * e4 + m;
        const bool undecided = level == 0 ? key[k] != 0u : ((act >> k) & 1u) != 0u;
        if (undecided && key[k] >= hi_key) sel |= 1u << k;
        if (undecided && key[k] >= lo_key && key[k] < hi_key) nact |= 1u << k;
      }
    }
    act = nact;
    if (c <= 64u) break;
    if (!R.refine(bstar)) {
      // more than 64 undecided entries of one value: equal masses, taken
      // by count in ascending block order (k/4, lane, k%4)
      uint32_t kmin = ~0u, kmax = 0u;
#pragma unroll
      for (int k = 0; k < EPL; ++k)
        if ((act >> k) & 1u) { kmin = min(kmin, key[k]); kmax = max(kmax, key[k]); }
      kmin = wave_min_u(kmin);
      kmax = wave_max_u(kmax);
      const unsigned long long mq = fixed_mass(kmin);
      if (kmin != kmax || mq == 0) {
        *fallback = true;
        return 0;
      }
      const unsigned long long take = (target - before + mq - 1) / mq;  // entries needed, >= 1
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
    if (level == 7) {
      *fallback = true;
      return 0;
    }
  }

  // compact b*'s entries in ascending block order: slot group e4, then lane,
  // then k % 4
  int off[EPL / 4];
  int total = 0;
#pragma unroll
  for (int e4 = 0; e4 < EPL / 4; ++e4) {
    off[e4] = 0;
    if (e4 >= ne4) continue;
    const uint32_t nib = (act >> (4 * e4)) & 0xFu;
    const uint32_t cnt = __popc(nib);
    const uint32_t incl = scan_add(cnt);
    off[e4] = total + (int)(incl - cnt);
    total += (int)lane63(incl);
    int o = off[e4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if ((nib >> m) & 1u) H.cand_key[o++] = key[4 * e4 + m];
  }

  // refine on the compacted entries, one per lane
  wave_lds_sync();
  const uint32_t ck = lane < (int)c ? H.cand_key[lane] : 0u;
  bool rem = lane < (int)c;  // still undecided
  bool keep = false;
  bool split = R.refine(bstar);
  for (int level = 0; split && level < 8; ++level) {
    H.bin[lane] = 0ull;
    wave_lds_sync();
    if (rem) atomicAdd(&H.bin[R.bin(ck)], (1ull << 52) | fixed_mass(ck));
    uint32_t c2;
    const int b2 = Hist::pass_done(H, lane, p, Z, target, before, &c2);
    wave_lds_sync();
    if (rem) {
      const int bk = R.bin(ck);
      keep = keep || bk < b2;
      rem = bk == b2;
    }
    if (c2 == 1u) {  // that entry completes the mass
      keep = keep || rem;
      rem = false;
      break;
    }
    split = R.refine(b2);
  }
  const uint64_t rb = __ballot(rem);
  if (rb) {
    // the undecided entries share one value: the first `take` in list order
    const uint32_t kv = __builtin_amdgcn_readlane(ck, __ffsll((long long)rb) - 1);
    const unsigned long long mq = fixed_mass(kv);
    if (mq == 0) {
      *fallback = true;
      return 0;
    }
    const unsigned long long take = (target - before + mq - 1) / mq;
    const unsigned long long r = __popcll(rb & ((1ull << lane) - 1ull));
    keep = keep || (rem && r < take);
  }
  H.cand_keep[lane] = keep ? 1u : 0u;
  wave_lds_sync();
#pragma unroll
  for (int e4 = 0; e4 < EPL / 4; ++e4) {
    if (e4 >= ne4) continue;
    const uint32_t nib = (act >> (4 * e4)) & 0xFu;
    int o = off[e4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if ((nib >> m) & 1u) {
        if (H.cand_keep[o]) sel |= 1u << (4 * e4 + m);
        ++o;
      }
  }
  return sel;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// segment of canonical dim d: 0 high-only, 1 middle, 2 low-only
__device__ __forceinline__ int seg_of(int d, int lo, int hi) { return d < lo ? 0 : (d < hi ? 1 : 2); }

constexpr int kScoreTilesPerWg = 4;  // key tiles one workgroup sweeps along its strip

// Accumulates the 16 dim chunks of one tile into the segment accumulators.
// Chunk c holds canonical dims 8c..8c+7; lane half hf supplies dims
// 8c + 4hf + e for MFMA e (A and B agree, so each dim enters once).
// LO8, HI8 >= 0: both segment boundaries are multiples of 8 (lo = 8 LO8,
// hi = 8 HI8), every chunk lies in one segment known at compile time.
// LO8 == kRuntime8: both boundaries are multiples of 8 given at run time;
// the segment of each chunk is a wave-uniform branch.
// Otherwise (LO8 < 0) each chunk feeds all three accumulators with the dims
// of the other segments zeroed (three times the MFMAs, for band widths that
// are not multiples of 8).
constexpr int kRuntime8 = 100;

template <int LO8, int HI8>
__device__ __forceinline__ void score_tile(const float4 (&qa)[16], const float4 *kr, int krow, int hf, int lo, int hi,
                                           int overlap, f32x16 &acc0, f32x16 &acc1, f32x16 &acc2) {
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const float4 k4 = kr[(2 * c + hf) ^ (krow & 15)];
    const float qv[4] = {qa[c].x, qa[c].y, qa[c].z, qa[c].w};
    const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
    if constexpr (LO8 >= 0) {
      const int lo8 = LO8 == kRuntime8 ? lo >> 3 : LO8;
      const int hi8 = LO8 == kRuntime8 ? hi >> 3 : HI8;
      if (c < lo8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(qv[e], kv[e], acc0, 0, 0, 0);
      } else if (c < hi8) {
        if (overlap) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(qv[e], kv[e], acc1, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc2 = __builtin_amdgcn_mfma_f32_32x32x2f32(qv[e], kv[e], acc2, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int sd = seg_of(8 * c + 4 * hf + e, lo, hi);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(sd == 0 ? qv[e] : 0.f, kv[e], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(sd == 1 && overlap ? qv[e] : 0.f, kv[e], acc1, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_32x32x2f32(sd == 2 ? qv[e] : 0.f, kv[e], acc2, 0, 0, 0);
      }
    }
  }
}

// One workgroup = query blocks I*64..I*64+63 of one head against up to
// kScoreTilesPerWg consecutive 64-key-block tiles of its strip. Wave w owns
// the 32 x 32 quadrant (w / 2, w % 2) of each tile. The wave's 32 Qbar rows
// stay in registers (lane l: row l % 32, dims 8c + 4(l / 32)..+3 of chunk c);
// Kbar tiles (64 x 128 fp32) stream through two LDS buffers, the next tile's
// global loads in flight while the current one is computed. LDS rows are 512
// bytes; 16-byte slot s of row r sits at s ^ (r % 16), so the 16 rows one
// ds_read_b128 pass touches fall in 16 different bank groups.
// Per-vector temperature factor r_z(v) = R(v, D_full) / R(v, D_z) of one
// pooled vector from its segment energies e = (high-only, middle, low-only);
// 1 when the band holds no energy.
__device__ __forceinline__ float pervec_factor(const float4 &e, int z, int overlap, int dz) {
  const float mid = overlap ? e.y : 0.f;
  const float ez = (z == 0 ? e.x : e.z) + mid;
  const float ef = e.x + e.y + e.z;
  return ez > 0.f ? sqrtf(ef * (float)dz / ((float)kHeadDim * ez)) : 1.f;
}

template <int LO8, int HI8, bool PV>
__global__ __launch_bounds__(256, 2) void score_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) float4 kt[2][64 * 32];
  const int nI = (a.nb + 63) / 64;
  constexpr int T = kScoreTilesPerWg;
  // Work item -> (head, strip I, tile chunk). Per head, the chunks of T tiles
  // come first (longest strips first), then the shorter remainders; the heads
  // of one chunk rank are adjacent in the grid, so the long work starts first.
  const int nbh = a.batch * a.nh;
  const int lbh = blockIdx.x % nbh;
  const int bh = (lbh / a.nh) * a.hq + a.h0 + lbh % a.nh;
  int w = blockIdx.x / nbh, I = nI - 1, J0 = 0, J1 = 0;
  int nfull = 0;
  for (int t = 0; t < nI; ++t) nfull += (a.causal ? t + 1 : nI) / T;
  if (w < nfull) {
    for (;; --I) {
      const int nf = (a.causal ? I + 1 : nI) / T;
      if (w < nf) break;
      w -= nf;
    }
    J0 = w * T;
    J1 = J0 + T;
  } else {
    w -= nfull;
    for (;; --I) {
      const int nJ = a.causal ? I + 1 : nI;
      if (nJ % T == 0) continue;
      if (w == 0) {
        J0 = nJ - nJ % T;
        J1 = nJ;
        break;
      }
      --w;
    }
  }

  const int b = bh / a.hq, h = bh % a.hq, g = h / (a.hq / a.hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31, hf = lane >> 5;
  const int i0 = I * 64 + 32 * (wave >> 1);
  const int lo = a.seg_lo, hi = a.seg_hi;

  // the wave's Qbar rows
  float4 qa[16];
  {
    const float *qp = a.qbar + ((int64_t)bh * a.nb + min(i0 + r32, a.nb - 1)) * kHeadDim + 4 * hf;
#pragma unroll
    for (int c = 0; c < 16; ++c) qa[c] = *reinterpret_cast<const float4 *>(qp + 8 * c);
  }
  // tile staging: thread t moves float4 u = t + 256 x of the tile (row u / 32,
  // 16-byte slot u % 32); the row index is clamped at the sequence end
  const float *kbase = a.kbar + ((int64_t)b * a.hkv + g) * a.nb * kHeadDim;
  const int srow = tid >> 5, sslot = tid & 31;  // x adds 8 rows
#define PRISM_LOAD_TILE(J)                                                                                   \
  _Pragma("unroll") for (int x = 0; x < 8; ++x) pre[x] = *reinterpret_cast<const f32x4v *>(                \
      kbase + (int64_t)min((J) * 64 + srow + 8 * x, a.nb - 1) * kHeadDim + 4 * sslot);
#define PRISM_STORE_TILE(buf)                                                                                \
  _Pragma("unroll") for (int x = 0; x < 8; ++x)                                                              \
      *reinterpret_cast<f32x4v *>(&(buf)[(srow + 8 * x) * 32 + (sslot ^ ((srow + 8 * x) & 15))]) = pre[x];

  const float kLog2e = 1.4426950408889634f;
  const float *tau = a.tau + (int64_t)bh * 8;
  const float ch = kLog2e / (tau[0] * sqrtf((float)a.d_high));
  const float cl = kLog2e / (tau[1] * sqrtf((float)a.d_low));
  float *ph = a.logits + (int64_t)bh * 2 * a.plane;
  float *pl = ph + a.plane;
  const int nb4 = (a.nb + 3) & ~3;
  const int krow = 32 * (wave & 1) + r32;  // this lane's key row within a tile

  {
    f32x4v pre[8];
    PRISM_LOAD_TILE(J0)
    PRISM_STORE_TILE(kt[0])
  }
  // Qbar and the first tile have landed: s_waitcnt vmcnt(0), so that the
  // loop's waits only ever cover its own prefetch
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int J = J0; J < J1; ++J) {
    const int cur = (J - J0) & 1;
    const bool more = J + 1 < J1;
    f32x4v pre[8];
    if (more) { PRISM_LOAD_TILE(J + 1) }
    // keep the next tile's loads here, ahead of this tile's MFMAs
    __builtin_amdgcn_sched_barrier(0);
    const int j0 = J * 64 + 32 * (wave & 1);
    if (i0 < a.nb && j0 < a.nb && !(a.causal && j0 > i0 + 31)) {
      f32x16 acc0, acc1, acc2;
#pragma unroll
      for (int r = 0; r < 16; ++r) { acc0[r] = 0.f; acc1[r] = 0.f; acc2[r] = 0.f; }
      score_tile<LO8, HI8>(qa, kt[cur] + krow * 32, krow, hf, lo, hi, a.overlap, acc0, acc1, acc2);
      const int j = j0 + r32;
      float kfh = 1.f, kfl = 1.f;  // per-vector factors of key block j
      if constexpr (PV) {
        const float4 e = *reinterpret_cast<const float4 *>(a.ksq + (((int64_t)b * a.hkv + g) * a.nb +
                                                                    min(j, a.nb - 1)) * 4);
        kfh = pervec_factor(e, 0, a.overlap, a.d_high);
        kfl = pervec_factor(e, 1, a.overlap, a.d_low);
      }
      // acc[r] = segment dot of query block i0 + 8(r/4) + 4*hf + r%4 with
      // key block j; each group of 4 rows starts at a multiple of 4, so the
      // 4 row starts are base + rr * step (32-bit offsets within the plane)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int ib = i0 + 8 * gq + 4 * hf;
        const int q4 = ib >> 2;
        const int base = a.causal ? 8 * q4 * (q4 + 1) : ib * nb4;
        const int step = a.causal ? 4 * (q4 + 1) : nb4;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int i = ib + rr, r = 4 * gq + rr;
          if (i < a.nb && j < a.nb && (!a.causal || j <= i)) {
            const float mid = a.overlap ? acc1[r] : 0.f;
            const int o = base + rr * step + j;
            if constexpr (PV) {
              const float4 e = *reinterpret_cast<const float4 *>(a.qsq + ((int64_t)bh * a.nb + i) * 4);
              ph[o] = (acc0[r] + mid) * ch * (pervec_factor(e, 0, a.overlap, a.d_high) * kfh);
              pl[o] = (acc2[r] + mid) * cl * (pervec_factor(e, 1, a.overlap, a.d_low) * kfl);
            } else {
              ph[o] = (acc0[r] + mid) * ch;
              pl[o] = (acc2[r] + mid) * cl;
            }
          }
        }
      }
    }
    if (more) { PRISM_STORE_TILE(kt[cur ^ 1]) }
    __syncthreads();
  }
#undef PRISM_LOAD_TILE
#undef PRISM_STORE_TILE
}

// Writes one chunk of a mask row from the wave's selection bits: bit
// 4 e4 + m of lane l is block jbase + 4 l + 256 e4 + m, for e4 < ne4 (every
// block of the chunk below nb is written, zeros included). U8 rows get one
// byte per block; bit-packed rows one u32 per 32 blocks, which are the
// nibbles of 8 adjacent lanes (gathered by lane exchanges, all lanes taking
// part).
__device__ void write_mask_chunk(const TopPArgs &a, int64_t row_index, int jbase, int ne4, uint32_t bits, int lane) {
  if (a.bits) {
    uint32_t *wrow = static_cast<uint32_t *>(a.mask) + row_index * a.words;
    for (int e4 = 0; e4 < ne4; ++e4) {
      uint32_t v = ((bits >> (4 * e4)) & 0xFu) << (4 * (lane & 7));
      v |= __shfl_xor(v, 1);
      v |= __shfl_xor(v, 2);
      v |= __shfl_xor(v, 4);
      const int j = jbase + 256 * e4 + 32 * (lane >> 3);  // first block of the word
      if ((lane & 7) == 0 && j < a.nb) wrow[j >> 5] = v;
    }
    return;
  }
  uint8_t *mrow = static_cast<uint8_t *>(a.mask) + row_index * a.nb;
  for (int e4 = 0; e4 < ne4; ++e4) {
    const int j = jbase + 4 * lane + 256 * e4;
    const uint32_t nib = (bits >> (4 * e4)) & 0xFu;
    if ((a.nb & 3) == 0) {
      if (j < a.nb) {
        const uint32_t word = (nib & 1u) | ((nib >> 1) & 1u) << 8 | ((nib >> 2) & 1u) << 16 | ((nib >> 3) & 1u) << 24;
        *reinterpret_cast<uint32_t *>(mrow + j) = word;
      }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (j + m < a.nb) mrow[j + m] = (uint8_t)((nib >> m) & 1u);
    }
  }
}

// One workgroup = two rows (batch, head, query block) x two branches: wave w
// selects branch w % 2 of row w / 2; the branch pairs meet in LDS and the
// even wave writes the union as the mask row. Rows are taken longest first.
template <int EPL>
__global__ __launch_bounds__(256) void topp_kernel(TopPArgs a) {
  __shared__ WaveHist whist[4];
  __shared__ uint32_t sel_s[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int z = wave & 1;
  const int nbh = a.batch * a.nh;
  const int rid = blockIdx.x * 2 + (wave >> 1);
  const bool live = rid < nbh * a.nb;
  const int rr = live ? rid : 0;
  const int i = a.causal ? a.nb - 1 - rr / nbh : rr / nbh;
  const int lbh = rr % nbh;
  const int bh = (lbh / a.nh) * a.hq + a.h0 + lbh % a.nh;
  const int nc = a.causal ? i + 1 : a.nb;
  const float *row = a.logits + ((int64_t)bh * 2 + z) * a.plane + logit_row(i, a.nb, a.causal);

  auto load_row = [&](float (&xr)[EPL]) {
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

  uint32_t bits = 0;
  if (live) {
    bool fallback;
    {
      float xr[EPL];
      load_row(xr);
      bits = select_row_hist<EPL>(xr, (nc + 255) / 256, a.p, lane, whist[wave], &fallback);
    }
    if (fallback) {
      float xr[EPL];
      load_row(xr);
      bits = select_row<EPL>(xr, a.p, lane);
    }
  }
  sel_s[wave][lane] = bits;
  __syncthreads();
  if (!live || z != 0) return;
  bits |= sel_s[wave + 1][lane];
  // union of the branches -> mask row, zeros included
  write_mask_chunk(a, (int64_t)bh * a.nb + i, 0, EPL / 4, bits, lane);
}

// Top-P of a row of more than kShortRow blocks, one wave, the row read from
// the logit plane in chunks of 2048 blocks (element k of lane l in chunk c
// is block 2048 c + 4 l + 256 (k / 4) + k % 4). The selection rule is
// select_row_hist's: masses m = floor(e 2^31) of e = exp2(L - max), target
// ceil(p Z), the shortest prefix of (e descending, block ascending) whose
// mass reaches the target. It is found by a radix select on the key (the
// bit pattern of e, monotone in e): five passes over the row, the first
// binning the keys by octave (exponent 64..127, all smaller e in the lowest
// bin: their masses are 0), the others by the next 6, 6, 6 and 5 mantissa
// bits of the keys that share the prefix found so far (fixed-point masses,
// exact in any order), each keeping the bin where the mass from the top
// reaches the target. That gives the key T with
// mass(key >= T) >= target > mass(key > T); every key above T is kept, and
// of the entries with key T the first ceil((target - mass(key > T)) / m(T))
// in block order. Keys are recomputed from the logits at every pass (the
// row stays in L2). sel[c] receives this lane's bits of chunk c; bins is
// the wave's 64-entry LDS histogram.
constexpr int kLongChunks = kMaxBlocks / 2048;

__device__ void select_row_long(const float *row, int nc, float p, int lane, unsigned long long *bins,
                                uint32_t (&sel)[kLongChunks]) {
  const int nch = (nc + 2047) / 2048;
  // logits of elements 4 e4 .. 4 e4 + 3 of chunk c (-inf past the row)
  auto logits4 = [&](int c, int e4, float (&x)[4]) {
    const int j = 2048 * c + 4 * lane + 256 * e4;
    float4 t = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    if (j < nc) t = *reinterpret_cast<const float4 *>(row + j);
    x[0] = t.x;
    x[1] = (j + 1 < nc) ? t.y : -INFINITY;
    x[2] = (j + 2 < nc) ? t.z : -INFINITY;
    x[3] = (j + 3 < nc) ? t.w : -INFINITY;
  };
  float mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < kLongChunks; ++c) {
    if (c >= nch) break;
#pragma unroll
    for (int e4 = 0; e4 < 8; ++e4) {
      float x[4];
      logits4(c, e4, x);
      mx = fmaxf(fmaxf(mx, fmaxf(x[0], x[1])), fmaxf(x[2], x[3]));
    }
  }
  mx = wave_max(mx);
#pragma unroll
  for (int c = 0; c < kLongChunks; ++c) sel[c] = 0u;
  if (p >= 1.0f) {
#pragma unroll
    for (int c = 0; c < kLongChunks; ++c) {
      if (c >= nch) break;
#pragma unroll
      for (int e4 = 0; e4 < 8; ++e4) {
        float x[4];
        logits4(c, e4, x);
#pragma unroll
        for (int m = 0; m < 4; ++m) sel[c] |= (x[m] != -INFINITY ? 1u : 0u) << (4 * e4 + m);
      }
    }
    return;
  }
  // radix levels: the exponent (octaves), then mantissa bits 22..17, 16..11,
  // 10..5 and 4..0; exp2(-inf) = 0 marks the inadmissible entries (never
  // counted)
  unsigned long long target = 0, above = 0;  // above: mass of the keys above the prefix's range
  uint32_t prefix = 0;
#pragma unroll 1
  for (int level = 0; level < 5; ++level) {
    const int shift = level == 0 ? 23 : 23 - 6 * level + (level == 4 ? 1 : 0);  // 23, 17, 11, 5, 0
    const int width = level == 0 ? 0 : (level == 4 ? 5 : 6);                    // prefix bits kept per level
    bins[lane] = 0ull;
    wave_lds_sync();
#pragma unroll
    for (int c = 0; c < kLongChunks; ++c) {
      if (c >= nch) break;
#pragma unroll
      for (int e4 = 0; e4 < 8; ++e4) {
        float x[4];
        logits4(c, e4, x);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t k = __float_as_uint(__builtin_amdgcn_exp2f(x[m] - mx));
          if (k != 0u && (level == 0 || (k >> (shift + width)) == prefix)) {
            const uint32_t bin = level == 0 ? (uint32_t)max((int)(k >> 23) - 64, 0)
                                            : (k >> shift) & ((1u << width) - 1u);
            atomicAdd(&bins[bin], (unsigned long long)fixed_mass(k));
          }
        }
      }
    }
    wave_lds_sync();
    const unsigned long long mass = bins[63 - lane];  // lane 0 holds the largest keys
    const unsigned long long cum = scan_add(mass);     // mass of this bin and every bin above it
    if (level == 0) target = (unsigned long long)ceil((double)lane63(cum) * (double)p);
    const unsigned long long need = target - above;    // > 0 at every level
    int t = __ffsll((long long)__ballot(cum >= need)) - 1;
    t = t < 0 ? 63 : t;  // unreachable: the range always holds at least `need`
    above += readlane_u64(cum, t) - readlane_u64(mass, t);
    prefix = level == 0 ? (uint32_t)(63 - t + 64) : (prefix << width) | (uint32_t)(63 - t);
    wave_lds_sync();  // every lane has read the bins before the next level clears them
  }
  const uint32_t T = prefix;                    // the threshold key itself
  const unsigned long long mT = fixed_mass(T);  // > 0: the keys equal to T carry mass
  const unsigned long long take = (target - above + mT - 1) / mT;
  // keep key > T, and the first `take` entries with key T in block order
  // (chunk, then e4, then lane, then element)
  unsigned long long rank0 = 0;
#pragma unroll
  for (int c = 0; c < kLongChunks; ++c) {
    if (c >= nch) break;
#pragma unroll
    for (int e4 = 0; e4 < 8; ++e4) {
      float x[4];
      logits4(c, e4, x);
      uint32_t tie = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t k = __float_as_uint(__builtin_amdgcn_exp2f(x[m] - mx));
        if (k > T) sel[c] |= 1u << (4 * e4 + m);
        if (k == T) tie |= 1u << m;
      }
      const int cnt = __popc(tie);
      unsigned long long r = rank0 + (unsigned long long)wave_excl_scan_i(cnt, lane);
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if ((tie >> m) & 1u) {
          if (r < take) sel[c] |= 1u << (4 * e4 + m);
          ++r;
        }
      rank0 += (unsigned long long)wave_sum_i(cnt);
    }
  }
}

// Rows of more than kShortRow blocks: one workgroup = two rows x two
// branches as in topp_kernel, each wave running select_row_long.
__global__ __launch_bounds__(256) void topp_long_kernel(TopPArgs a) {
  __shared__ uint32_t sel_s[4][kLongChunks][64];
  __shared__ unsigned long long bins_s[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int z = wave & 1;
  const int nbh = a.batch * a.nh;
  const int rid = blockIdx.x * 2 + (wave >> 1);
  const bool live = rid < nbh * a.nb;
  const int rr = live ? rid : 0;
  const int i = a.causal ? a.nb - 1 - rr / nbh : rr / nbh;
  const int lbh = rr % nbh;
  const int bh = (lbh / a.nh) * a.hq + a.h0 + lbh % a.nh;
  const int nc = a.causal ? i + 1 : a.nb;
  const float *row = a.logits + ((int64_t)bh * 2 + z) * a.plane + logit_row(i, a.nb, a.causal);
  uint32_t sel[kLongChunks];
#pragma unroll
  for (int c = 0; c < kLongChunks; ++c) sel[c] = 0u;
  if (live) select_row_long(row, nc, a.p, lane, bins_s[wave], sel);
#pragma unroll
  for (int c = 0; c < kLongChunks; ++c) sel_s[wave][c][lane] = sel[c];
  __syncthreads();
  if (!live || z != 0) return;
  const int nchunks = (a.nb + 2047) / 2048;  // the whole row, zeros included
#pragma unroll
  for (int c = 0; c < kLongChunks; ++c)
    if (c < nchunks) write_mask_chunk(a, (int64_t)bh * a.nb + i, 2048 * c, 8, sel[c] | sel_s[wave + 1][c][lane], lane);
}

}  // namespace

hipError_t launch_score(const ScoreArgs &a, hipStream_t s) {
  const int nI = (a.nb + 63) / 64;
  int per_head = 0;
  for (int I = 0; I < nI; ++I) per_head += ((a.causal ? I + 1 : nI) + kScoreTilesPerWg - 1) / kScoreTilesPerWg;
  const dim3 grid(per_head * a.nh * a.batch);  // heads x (full chunks, then remainders)
  const bool def = a.seg_lo == 32 && a.seg_hi == 64, equal = a.seg_lo == 0 && a.seg_hi == 128;
  const bool by8 = a.seg_lo % 8 == 0 && a.seg_hi % 8 == 0;
  if (a.pervec) {
    if (def) hipLaunchKernelGGL((score_kernel<4, 8, true>), grid, dim3(256), 0, s, a);
    else if (by8) hipLaunchKernelGGL((score_kernel<kRuntime8, 0, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((score_kernel<-1, -1, true>), grid, dim3(256), 0, s, a);
  } else if (def) {
    hipLaunchKernelGGL((score_kernel<4, 8, false>), grid, dim3(256), 0, s, a);
  } else if (equal) {
    hipLaunchKernelGGL((score_kernel<0, 16, false>), grid, dim3(256), 0, s, a);
  } else if (by8) {
    hipLaunchKernelGGL((score_kernel<kRuntime8, 0, false>), grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((score_kernel<-1, -1, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_topp(const TopPArgs &a, hipStream_t s) {
  const int rows = a.batch * a.nh * a.nb;
  const dim3 grid((rows + 1) / 2);
  if (a.nb <= 1024) hipLaunchKernelGGL((topp_kernel<16>), grid, dim3(256), 0, s, a);
  else if (a.nb <= kShortRow) hipLaunchKernelGGL((topp_kernel<32>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(topp_long_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace prism
