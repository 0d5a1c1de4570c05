// Prism estimator, steps (5)-(7) (Prism review on paper.rainbus.top,
// pipeline paragraph): per query block i and branch z in {high, low}
//   L_z[i, j] = Qbar_z[i] . Kbar_z[j] / (tau_z sqrt(d_z)),  j in J(i)
//   S_z[i, :] = softmax over J(i) (j <= i when causal),
//   M_z[i, :] = Top-P of S_z[i, :] at mass p, and M = M_high OR M_low.
//
// Selection rule (every kernel below): e_j = exp2(L_j - max), integer masses
//   m_j = floor(e_j 2^31) (fixed point, so every sum is exact and independent
//   of order), target ceil(p Z); the kept set is the shortest prefix of the
//   order (e descending, block index ascending) whose mass reaches the
//   target -- the sorted-prefix Top-P, found without a sort by a radix select
//   on the key (the bit pattern of e, monotone in e) over 64-bin LDS
//   histograms. The union of both branches is written as the mask row (bytes
//   or bits), zeros included.
//
// score_topp_kernel (rows of at most 1024 blocks): both branches' logits of a
//   strip of 16 query blocks on fp32 MFMA 16x16x4, kept on chip (LDS, then
//   registers), and the selection of each row (select_row_radix).
// score_kernel + topp_kernel (rows of 1025..8192 blocks): the logits of both
//   branches go through the workspace's logit planes (64 x 64 tiles on fp32
//   MFMA 32x32x2), then one wave per row and branch reads its row once into
//   registers (32, 64 or 128 logits per lane) and selects.
// estimate_single_kernel (rows of at most 1024 blocks, static bands): the
//   whole estimator in one persistent launch -- the pooling pass, a grid-wide
//   barrier, then per strip the head's temperatures and score_topp's work --
//   with the multi-kernel path's arithmetic, so both give the same bits.
// In every score kernel the canonical dims split into three segments,
//   high-only / middle / low-only, each dim entering one segment's dot
//   product once; L_high = (s0 + s1) c_high and L_low = (s1 + s2) c_low (the
//   middle segment only when the bands overlap), in log2 units.
#include "pool_device.h"

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

__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}

constexpr float kMassScale = 2147483648.0f;  // fixed point: mass = e * 2^31, e <= 1
__device__ __forceinline__ uint32_t fixed_mass(uint32_t ebits) {
  return (uint32_t)(__uint_as_float(ebits) * kMassScale);
}

// The lanes of one wave exchange data through LDS (histogram bins). The
// hardware runs a wave's LDS instructions in order; this fence keeps the
// compiler from reordering accesses across the exchange point or forwarding
// a lane's own earlier store to its later load.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Radix state: the bin of key y is clamp(base - (y >> shift), 0, 63), so
// larger keys fall in lower bins. Level 0 bins quarter octaves of e below 1
// (base 508 = 4 * 127, shift 21) with every smaller e in bin 63 (tail).
// Refining bin b* either moves the tail window down so that its bin 0 is the
// old bin 63's top quarter octave (every bin then holds exactly one value of
// y >> shift, except the new tail), or splits b* on the next (up to) 6 key
// bits. Returns false when b* holds a single key value (shift 0) or, in the
// tail, only keys whose masses are 0.
struct Radix {
  int shift = 21, base = 508;
  bool tail = true;
  __device__ int bin(uint32_t y) const { return min(max(base - (int)(y >> shift), 0), 63); }
  // keys of bin b: [lo(b), hi(b))
  __device__ uint32_t hi(int b) const { return (uint32_t)(base - b + 1) << shift; }
  __device__ uint32_t lo(int b) const { return (tail && b == 63) ? 1u : (uint32_t)(base - b) << shift; }
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

// Histogram of one wave in LDS: 64 bins, then one spare slot per lane that
// takes the adds of entries outside the level's range (adds without a
// branch). A bin word is (count << CS) | fixed-point mass: CS = 52 for rows
// of up to 2048 entries (counts below 2^12), 50 beyond (counts up to 8192
// below 2^14, masses up to 8192 * 2^31 = 2^44 below 2^50).
constexpr int kBinSlots = 128;
template <int EPL>
constexpr int count_shift() { return EPL <= 32 ? 52 : 50; }
__device__ __forceinline__ void clear_bins(unsigned long long *bins, int lane) { bins[lane] = 0ull; }

// Reads the wave's 64-bin histogram ((count << CS) | fixed-point mass per bin,
// bin 0 = largest keys) and returns the threshold bin b*: the first bin,
// from the top, where the cumulative mass reaches target - before. Adds the
// mass of the bins above b* to `before` and returns b*'s entry count in
// *count. At the first level (*Z == 0) it also sets Z and the target
// ceil(p * Z).
template <int CS>
__device__ __forceinline__ int threshold_bin(const unsigned long long *bins, int lane, float p, unsigned long long &Z,
                                             unsigned long long &target, unsigned long long &before, uint32_t *count) {
  wave_lds_sync();
  const unsigned long long hv = bins[lane];
  const unsigned long long mass = hv & ((1ull << CS) - 1ull);
  const unsigned long long cum = scan_add((unsigned long long)mass);  // largest values first
  if (Z == 0) {
    Z = readlane_u64(cum, 63);
    target = (unsigned long long)ceil((double)Z * (double)p);
  }
  const unsigned long long need = target - before;  // > 0 at every level
  const int bstar = __ffsll((long long)__ballot(cum >= need)) - 1;
  before += readlane_u64(cum, bstar) - readlane_u64(mass, bstar);
  *count = (uint32_t)(readlane_u64(hv, bstar) >> CS);
  wave_lds_sync();  // every lane has read the bins before they are cleared again
  return bstar;
}

// One histogram level: the keys in [lo, hi) of the admissible slots add
// (1 << CS) | mass to their bin, the others to the lane's spare slot.
template <int EPL>
__device__ __forceinline__ void hist_range(const uint32_t (&key)[EPL], int ne4, uint32_t lo, uint32_t hi,
                                           const Radix &R, unsigned long long *bins, int lane) {
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    if (k / 4 >= ne4) continue;
    const bool in = key[k] - lo < hi - lo;  // unsigned: lo <= key < hi
    atomicAdd(&bins[in ? R.bin(key[k]) : 64 + lane], (1ull << count_shift<EPL>()) | fixed_mass(key[k]));
  }
}

// Top-P of one row held by the wave: element k of lane l is block
// j = 4 l + 256 (k / 4) + k % 4; x[k] are log2-unit logits, -inf where j is
// not admissible; slots k / 4 >= ne4 hold no admissible block. `bins` is the
// wave's LDS histogram (kBinSlots entries). Leaves this lane's selection bits
// in sel: bit k % 32 of word k / 32 for slot k (word c covers blocks
// 2048 c .. 2048 c + 2047).
//
// The rule: e_j = exp2(x_j - max), integer masses m_j = floor(e_j 2^31)
// (fixed point: every sum exact and independent of order), target
// ceil(p Z) with Z the sum of the masses; the selection is the shortest
// prefix of the order (e descending, block ascending) whose mass reaches the
// target. It is found by a radix select on the key (the bit pattern of e,
// monotone in e): each level histograms the undecided keys into 64 bins and
// keeps the bin b* where the mass from the top reaches the target; keys
// above b* are kept, keys below dropped, and the next level splits b*. It
// ends when b* holds one entry (which the target needs: every key down to
// it is kept) or one key value (the first ceil(still needed / its mass)
// entries with that key are kept, in block order). No sort, no fallback.
template <int EPL, int W>
__device__ void select_row_radix_w(const float (&x)[EPL], int ne4, float p, int lane, unsigned long long *bins,
                                   uint32_t (&sel)[W]) {
  static_assert(W == (EPL + 31) / 32, "one selection word per 32 slots");
  constexpr int CS = count_shift<EPL>();
#pragma unroll
  for (int w = 0; w < W; ++w) sel[w] = 0u;
  float mx = -INFINITY;
#pragma unroll
  for (int e4 = 0; e4 < EPL / 4; ++e4) {
    if (e4 >= ne4) {
      if constexpr (EPL <= 32) break;
      else continue;  // a compile-time trip count keeps the wide loops unrolled
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) mx = fmaxf(mx, x[4 * e4 + m]);
  }
  mx = wave_max(mx);
  if (p >= 1.0f) {
#pragma unroll
    for (int k = 0; k < EPL; ++k) sel[k >> 5] |= (x[k] != -INFINITY ? 1u : 0u) << (k & 31);
    return;
  }

  // keys (exp2(-inf) = 0 marks an entry that is not admissible; an e that
  // underflows to 0 is never needed since p * Z <= Z); the first level's
  // histogram is made with them, keys 0 going to the lane's spare slot.
  uint32_t key[EPL];
#pragma unroll
  for (int k = 0; k < EPL; ++k) key[k] = 0u;
  Radix R;
  clear_bins(bins, lane);
  wave_lds_sync();
#pragma unroll
  for (int e4 = 0; e4 < EPL / 4; ++e4) {
    if (e4 >= ne4) {
      if constexpr (EPL <= 32) break;
      else continue;  // a compile-time trip count keeps the wide loops unrolled
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int k = 4 * e4 + m;
      key[k] = __float_as_uint(__builtin_amdgcn_exp2f(x[k] - mx));
      atomicAdd(&bins[key[k] ? R.bin(key[k]) : 64 + lane], (1ull << CS) | fixed_mass(key[k]));
    }
  }
  unsigned long long Z = 0, target = 0, before = 0;
  uint32_t c, lo, hi;
  for (;;) {
    const int bstar = threshold_bin<CS>(bins, lane, p, Z, target, before, &c);
    lo = R.lo(bstar);
    hi = R.hi(bstar);
    if (c <= 1u || !R.refine(bstar)) break;
    clear_bins(bins, lane);
    wave_lds_sync();
    hist_range<EPL>(key, ne4, lo, hi, R, bins, lane);
  }
  if (c <= 1u) {  // b*'s one entry completes the mass: every key down to it is kept
#pragma unroll
    for (int k = 0; k < EPL; ++k) sel[k >> 5] |= (key[k] >= lo ? 1u : 0u) << (k & 31);
    return;
  }
  // b* holds c > 1 entries of one key value lo: keys above it are kept, and
  // of those equal to it the first `take` in block order (k / 4, lane, k % 4)
  const unsigned long long mq = fixed_mass(lo);  // > 0: b* carries mass
  const unsigned long long take = (target - before + mq - 1) / mq;
  unsigned long long rank0 = 0;
#pragma unroll
  for (int e4 = 0; e4 < EPL / 4; ++e4) {
    uint32_t nib = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int k = 4 * e4 + m;
      if (key[k] >= hi) sel[k >> 5] |= 1u << (k & 31);
      if (key[k] == lo) nib |= 1u << m;
    }
    if (e4 >= ne4) continue;
    const int cnt = __popc(nib);
    unsigned long long r = rank0 + (unsigned long long)wave_excl_scan_i(cnt, lane);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if ((nib >> m) & 1u) {
        if (r < take) sel[(4 * e4 + m) >> 5] |= 1u << ((4 * e4 + m) & 31);
        ++r;
      }
    rank0 += (unsigned long long)wave_sum_i(cnt);
  }
}
// rows of at most 2048 entries: the selection bits as one word
template <int EPL>
__device__ __forceinline__ uint32_t select_row_radix(const float (&x)[EPL], int ne4, float p, int lane,
                                                     unsigned long long *bins) {
  uint32_t sel[1];
  select_row_radix_w<EPL, 1>(x, ne4, p, lane, bins, sel);
  return sel[0];
}

// Weighted merge (prism_merge_t MIX): one Top-P on the equal-weight mixture
// of the two branches' block distributions, v_j = e_high,j / Z_high +
// e_low,j / Z_low (the weights 1/2 cancel), selected by the same radix rule
// on log2 v. fp32 throughout; slots past the row hold -inf.
template <int EPL>
__device__ uint32_t select_row_mix(const float (&xh)[EPL], const float (&xl)[EPL], int ne4, float p, int lane,
                                  unsigned long long *bins) {
  float mh = -INFINITY, ml = -INFINITY;
#pragma unroll
  for (int k = 0; k < EPL; ++k)
    if (k / 4 < ne4) {
      mh = fmaxf(mh, xh[k]);
      ml = fmaxf(ml, xl[k]);
    }
  mh = wave_max(mh);
  ml = wave_max(ml);
  float eh[EPL], el[EPL];
  float zh = 0.f, zl = 0.f;
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    eh[k] = k / 4 < ne4 ? __builtin_amdgcn_exp2f(xh[k] - mh) : 0.f;
    el[k] = k / 4 < ne4 ? __builtin_amdgcn_exp2f(xl[k] - ml) : 0.f;
    zh += eh[k];
    zl += el[k];
  }
  const float ih = 1.0f / wave_sum(zh), il = 1.0f / wave_sum(zl);
  float xm[EPL];
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    const float v = eh[k] * ih + el[k] * il;
    xm[k] = v > 0.f ? __builtin_amdgcn_logf(v) : -INFINITY;  // v_log_f32: log2
  }
  return select_row_radix<EPL>(xm, ne4, p, lane, bins);
}

// The bands of one head: those of the launch (static split), or the head's
// own from the split section (adaptive split).
__device__ __forceinline__ void head_bands(ScoreArgs &a, int64_t bh) {
  if (a.split) {
    const int4 v = *reinterpret_cast<const int4 *>(a.split + bh * 4);
    a.seg_lo = v.x;
    a.seg_hi = v.y;
    a.d_high = v.z;
    a.d_low = v.w;
  }
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

  head_bands(a, bh);
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
  constexpr int W = EPL / 32;  // selection words per lane (2048 blocks each)
  __shared__ unsigned long long bins_s[4][kBinSlots];
  __shared__ uint32_t sel_s[4][W][64];
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

  uint32_t bits[W];
#pragma unroll
  for (int w = 0; w < W; ++w) bits[w] = 0u;
  if (live) {
    float xr[EPL];
    load_row(xr);
    select_row_radix_w<EPL, W>(xr, (nc + 255) / 256, a.p, lane, bins_s[wave], bits);
  }
#pragma unroll
  for (int w = 0; w < W; ++w) sel_s[wave][w][lane] = bits[w];
  __syncthreads();
  if (!live || z != 0) return;
  // union (or intersection) of the branches -> mask row, zeros included
#pragma unroll
  for (int w = 0; w < W; ++w)
    if (2048 * w < a.nb) {
      const uint32_t other = sel_s[wave + 1][w][lane];
      write_mask_chunk(a, (int64_t)bh * a.nb + i, 2048 * w, 8,
                       a.merge == PRISM_MERGE_INTERSECT ? (bits[w] & other) : (bits[w] | other), lane);
    }
}

// ---- scores and Top-P in one kernel (rows of at most 1024 blocks)
//
// One workgroup (8 waves) = 16 consecutive query blocks of one head; wave w
// owns query blocks 16 I + w and 16 I + w + 8. Two workgroups share a CU
// (registers and LDS are sized for it), so that one's MFMA phase runs
// beside the other's selection phase. The strip's logits are made 256 key
// blocks at a time: wave w computes the 16 x 16 tiles w and w + 8 (key
// blocks 256 c + 16 t .. + 15) x (the strip's 16 query blocks) on fp32 MFMA
// 16x16x4, with A = Kbar rows (lane l: key l % 16, dims 16 m + 4 (l / 16) + e
// of dim group m, loaded from global memory as one float4 per group) and
// B = Qbar (the same dims of query l % 16, from LDS), so every canonical dim
// enters once and each group of 16 dims lies in one segment (high-only,
// middle, low-only) when the segment boundaries are multiples of 16. The
// lane's outputs are four consecutive key blocks of one query block; both
// branches' logits go to an LDS chunk buffer (rows padded to 260 floats, so
// the 16 query rows of one store fall in distinct banks), and after the
// barrier every wave reads its two rows in the selection layout (element k
// of lane l = block 4 l + 256 (k / 4) + k % 4). The logits never leave the
// chip. Then each wave selects its rows' branches in turn
// (select_row_radix) and writes each row's union as its mask row.
constexpr int kStrip = 16;             // query blocks per workgroup
constexpr int kFusedWaves = 8;
constexpr int kFusedChunk = 256;       // key blocks per score chunk
constexpr int kFusedPitch = kFusedChunk + 4;
constexpr int kRuntime16 = 100;

// LDS of one strip: both branches' logits of a 256-block chunk, the strip's
// Qbar rows, and each wave's selection histogram.
struct FusedLds {
  float lt[2][kStrip][kFusedPitch];                // [branch][row][key]
  float4 qs[kStrip * 32];                          // Qbar rows, 16-byte slots swizzled
  unsigned long long bins_s[kFusedWaves][kBinSlots];
};

// Strip I (query blocks 16 I .. 16 I + 15) of head bh = b * Hq + h, with the
// head's branch temperatures tau_h, tau_l; every thread of the 8-wave
// workgroup calls it (it holds barriers).
template <int LO16, int HI16, bool PV, bool MIX, typename AfterScores>
__device__ __forceinline__ void score_topp_strip(ScoreArgs a, const TopPArgs &t, int I, int bh, float tau_h,
                                                 float tau_l, FusedLds &L, int tid, AfterScores &&after_scores) {
  auto &lt = L.lt;
  auto &qs = L.qs;
  auto &bins_s = L.bins_s;
  head_bands(a, bh);
  const int b = bh / a.hq, h = bh % a.hq, gk = h / (a.hq / a.hkv);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q0 = I * kStrip;
  const int ncol = a.causal ? min(a.nb, q0 + kStrip) : a.nb;  // key blocks any row of the strip admits
  const int nchunk = (ncol + kFusedChunk - 1) / kFusedChunk;
  const int r16 = lane & 15, g4 = lane >> 4;

  // the strip's Qbar rows -> LDS: row r, slot s (dims 4s..4s+3) at s ^ r
  {
    const int r = tid >> 5, s = tid & 31;  // 512 threads, one slot each
    qs[r * 32 + (s ^ r)] = *reinterpret_cast<const float4 *>(
        a.qbar + ((int64_t)bh * a.nb + min(q0 + r, a.nb - 1)) * kHeadDim + 4 * s);
  }

  const float kLog2e = 1.4426950408889634f;
  const float ch = kLog2e / (tau_h * sqrtf((float)a.d_high));
  const float cl = kLog2e / (tau_l * sqrtf((float)a.d_low));
  float fqh = 1.f, fql = 1.f;  // per-vector factors of this lane's query block
  if constexpr (PV) {
    const float4 e = *reinterpret_cast<const float4 *>(a.qsq + ((int64_t)bh * a.nb + min(q0 + r16, a.nb - 1)) * 4);
    fqh = pervec_factor(e, 0, a.overlap, a.d_high);
    fql = pervec_factor(e, 1, a.overlap, a.d_low);
  }
  const float *kbase = a.kbar + ((int64_t)b * a.hkv + gk) * a.nb * kHeadDim;
  const float *ksq = a.ksq + ((int64_t)b * a.hkv + gk) * a.nb * 4;

  // this wave's two query blocks: r = 0 -> 16 I + w, r = 1 -> 16 I + w + 8
  int iq[2], nc[2];
  bool live[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    iq[r] = q0 + wave + kFusedWaves * r;
    live[r] = iq[r] < a.nb;
    nc[r] = a.causal ? iq[r] + 1 : a.nb;
  }
  float xh[2][16], xl[2][16];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int k = 0; k < 16; ++k) { xh[r][k] = -INFINITY; xl[r][k] = -INFINITY; }

  // Kbar operands stream in half tiles (dim groups 4 hf .. 4 hf + 3, one
  // float4 each) through two register buffers: the next half tile's loads
  // are issued before the current one's MFMAs (across tiles and chunks too),
  // so the load latency overlaps the MFMAs, the barriers and the row reads.
  // Valid (chunk, tile) pairs form a prefix of the sequence.
  auto tile_valid = [&](int c, int tt) { return c < nchunk && kFusedChunk * c + 16 * (wave + kFusedWaves * tt) < ncol; };
  auto load_half = [&](int c, int tt, int hf, float4 (&dst)[4]) {
    const int j = min(kFusedChunk * c + 16 * (wave + kFusedWaves * tt) + r16, a.nb - 1);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      dst[m] = *reinterpret_cast<const float4 *>(kbase + (int64_t)j * kHeadDim + 16 * (4 * hf + m) + 4 * g4);
  };
  float4 kb[2][4];
  if (tile_valid(0, 0)) load_half(0, 0, 0, kb[0]);

  __syncthreads();  // Qbar in LDS
#pragma unroll
  for (int c = 0; c < kFusedMaxBlocks / kFusedChunk; ++c) {
    if (c >= nchunk) break;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tile = wave + kFusedWaves * tt;
      const int jt = kFusedChunk * c + 16 * tile;  // first key block of the tile
      if (!tile_valid(c, tt)) continue;
      f32x4v acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, acc2 = acc0;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int st = 4 * c + 2 * tt + hf;  // step of the sequence; buffer st % 2
        // prefetch the next step's half tile
        if (hf == 0) {
          load_half(c, tt, 1, kb[(st + 1) & 1]);
        } else if (tt == 0) {
          if (tile_valid(c, 1)) load_half(c, 1, 0, kb[(st + 1) & 1]);
        } else {
          if (tile_valid(c + 1, 0)) load_half(c + 1, 0, 0, kb[(st + 1) & 1]);
        }
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          const int m = 4 * hf + mm;
          const float4 qv4 = qs[r16 * 32 + ((4 * m + g4) ^ r16)];
          const float qv[4] = {qv4.x, qv4.y, qv4.z, qv4.w};
          const float4 k4 = kb[st & 1][mm];
          const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
          if constexpr (LO16 >= 0) {
            const int lo16 = LO16 == kRuntime16 ? a.seg_lo >> 4 : LO16;
            const int hi16 = LO16 == kRuntime16 ? a.seg_hi >> 4 : HI16;
            if (m < lo16) {
#pragma unroll
              for (int e = 0; e < 4; ++e) acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[e], qv[e], acc0, 0, 0, 0);
            } else if (m < hi16) {
              if (a.overlap) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[e], qv[e], acc1, 0, 0, 0);
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[e], qv[e], acc2, 0, 0, 0);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int sd = seg_of(16 * m + 4 * g4 + e, a.seg_lo, a.seg_hi);
              acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(sd == 0 ? kv[e] : 0.f, qv[e], acc0, 0, 0, 0);
              acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(sd == 1 && a.overlap ? kv[e] : 0.f, qv[e], acc1, 0, 0, 0);
              acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(sd == 2 ? kv[e] : 0.f, qv[e], acc2, 0, 0, 0);
            }
          }
        }
      }
      // acc[r]: key block jt + 4 g4 + r against query block q0 + r16
      f32x4v lh, ll;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mid = a.overlap ? acc1[r] : 0.f;
        lh[r] = (acc0[r] + mid) * ch;
        ll[r] = (acc2[r] + mid) * cl;
      }
      if constexpr (PV) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float4 e = *reinterpret_cast<const float4 *>(ksq + (int64_t)min(jt + 4 * g4 + r, a.nb - 1) * 4);
          lh[r] *= fqh * pervec_factor(e, 0, a.overlap, a.d_high);
          ll[r] *= fql * pervec_factor(e, 1, a.overlap, a.d_low);
        }
      }
      *reinterpret_cast<f32x4v *>(&lt[0][r16][16 * tile + 4 * g4]) = lh;
      *reinterpret_cast<f32x4v *>(&lt[1][r16][16 * tile + 4 * g4]) = ll;
    }
    __syncthreads();
    // this wave's rows, chunk c: elements 4c..4c+3 of lane l are key blocks
    // 256 c + 4 l + e (-inf where the row does not admit them)
    {
      const int j = kFusedChunk * c + 4 * lane;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = wave + kFusedWaves * r;
        const f32x4v vh = *reinterpret_cast<const f32x4v *>(&lt[0][row][4 * lane]);
        const f32x4v vl = *reinterpret_cast<const f32x4v *>(&lt[1][row][4 * lane]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xh[r][4 * c + e] = j + e < nc[r] ? vh[e] : -INFINITY;
          xl[r][4 * c + e] = j + e < nc[r] ? vl[e] : -INFINITY;
        }
        if (a.keep_logits && live[r]) {  // inspection copy in the plane layout
          float *ph = a.logits + (int64_t)bh * 2 * a.plane + logit_row(iq[r], a.nb, a.causal);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j + e < nc[r]) {
              ph[j + e] = vh[e];
              ph[a.plane + j + e] = vl[e];
            }
        }
      }
    }
    __syncthreads();  // every wave has read the chunk before the next one is stored
  }
  after_scores();

#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (!live[r]) continue;
    const int ne4 = (nc[r] + 255) / 256;
    uint32_t bits;
    if constexpr (MIX) {  // the mixture's selection is its own instance (registers)
      bits = select_row_mix<16>(xh[r], xl[r], ne4, t.p, lane, bins_s[wave]);
    } else {
      const uint32_t bh_ = select_row_radix<16>(xh[r], ne4, t.p, lane, bins_s[wave]);
      const uint32_t bl_ = select_row_radix<16>(xl[r], ne4, t.p, lane, bins_s[wave]);
      bits = t.merge == PRISM_MERGE_INTERSECT ? (bh_ & bl_) : (bh_ | bl_);
    }
    write_mask_chunk(t, (int64_t)bh * a.nb + iq[r], 0, 4, bits, lane);
  }
}

// One workgroup per (strip, head), longest strips first.
template <int LO16, int HI16, bool PV, bool MIX>
__global__ __launch_bounds__(kFusedWaves * 64) __attribute__((amdgpu_waves_per_eu(4)))
void score_topp_kernel(ScoreArgs a, TopPArgs t) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[sizeof(FusedLds)];
  const int nI = (a.nb + kStrip - 1) / kStrip;
  const int nbh = a.batch * a.nh;
  const int lbh = blockIdx.x % nbh;
  const int rank = blockIdx.x / nbh;
  const int I = a.causal ? nI - 1 - rank : rank;
  const int bh = (lbh / a.nh) * a.hq + a.h0 + lbh % a.nh;
  const float *tau = a.tau + (int64_t)bh * 8;
  score_topp_strip<LO16, HI16, PV, MIX>(a, t, I, bh, tau[0], tau[1], *reinterpret_cast<FusedLds *>(smem), threadIdx.x,
                                        [] {});
}


// ---- the whole estimator in one launch (rows of at most 1024 blocks)
//
// A persistent grid of 8-wave workgroups, all resident at once (cooperative
// launch), runs the work of the multi-kernel path with one grid-wide barrier
// in place of the kernel boundaries:
//  (1)-(3) pooling: the first 256 threads of each workgroup pool work items
//    exactly as pool_kernel does (pool_device.h), the results of up to
//    kSingleSlots items waiting in LDS until their reads are done (the other
//    waves only join the barriers: eight streaming waves per CU read faster
//    than sixteen);
//  barrier: every workgroup publishes its writes (release at device scope,
//    then its own barrier word := this call's tag) and waits until every
//    word holds the tag (acquire at device scope);
//  (4) temperatures: workgroup w computes those of head w, w + G, ...
//    (tau_reduce, the tau kernel's arithmetic), writes them to the workspace
//    and publishes tau_high and tau_low each in a 64-bit word beside the low
//    32 bits of the tag (one atomic store each, so a reader that sees the
//    tag sees the value: no fence and no cache invalidation on either side);
//  (5)-(7) strips: taken from a ticket counter in the order the fused kernel's
//    grid has (longest strips first, heads fastest), so that a workgroup
//    that finishes early takes the next strip; per strip the head's two
//    temperatures are read from their words, then score_topp_strip.
// No word has to start at zero (the counter is set by workgroup 0 before the
// barrier; the other words are recognised by the tag), so the call needs no
// clearing launch. Every wait gives up after g.wait_ticks of the 100 MHz
// real-time counter (then `status` := 1 and the call's outputs are not
// valid); the host sizes it far above the pooling pass's duration.
constexpr int kSingleSlots = 6;

template <bool FP32>
struct SinglePoolLds {
  static constexpr int E = Elem<FP32>::E;
  float red[kPoolThreads * E];                                  // token-parallel partial sums
  float4 means[kSingleSlots][kPoolThreads * E / 4];            // E means per thread, per item
  float4 energy[kSingleSlots][kPoolThreads / (kHeadDim / E)];  // three segment energies per head row
};
struct TauLds {
  double red[6][kPoolThreads];
  float out[8];
};
constexpr size_t kSingleLdsBytes = sizeof(SinglePoolLds<false>) > sizeof(FusedLds)
                                       ? (sizeof(SinglePoolLds<false>) > sizeof(TauLds) ? sizeof(SinglePoolLds<false>)
                                                                                         : sizeof(TauLds))
                                       : (sizeof(FusedLds) > sizeof(TauLds) ? sizeof(FusedLds) : sizeof(TauLds));
static_assert(sizeof(SinglePoolLds<true>) <= kSingleLdsBytes, "fp32 pooling LDS");
static_assert(kSingleLdsBytes <= 80 * 1024 - 64, "two workgroups per CU");

template <bool FP32>
__device__ __forceinline__ void single_pool(const PoolArgs &a, int batch, unsigned char *smem) {
  constexpr int E = Elem<FP32>::E;
  constexpr int TPH = kHeadDim / E;
  auto &L = *reinterpret_cast<SinglePoolLds<FP32> *>(smem);
  const int tid = threadIdx.x;
  const bool worker = tid < kPoolThreads;
  const int per = pool_items(a);
  const int all = batch * per, G = gridDim.x;  // < 2^31: at most 1024 blocks and 2^20 heads in all
  for (int first = blockIdx.x; first < all; first += kSingleSlots * G) {
    int nst = 0;
    for (int gi = first; gi < all && nst < kSingleSlots; gi += G, ++nst) {
      // batch entry and item, uniform (scalar registers: the addresses below stay scalar + lane offset)
      const int b = __builtin_amdgcn_readfirstlane(gi / per), item = __builtin_amdgcn_readfirstlane(gi % per);
      const PoolItem<FP32> w(a, item, worker ? tid : 0);
      float acc[E];
      if (worker) {
        pool_accum<FP32>(a, b, w, acc);
        pool_red_put<FP32>(w, tid, acc, L.red);
      }
      if (w.tokp > 1) __syncthreads();
      if (worker) {
        float st[E + 3];
        pool_finish<FP32>(a, w, tid, acc, L.red, st);
#pragma unroll
        for (int e = 0; e < E; e += 4) L.means[nst][(tid * E + e) / 4] = make_float4(st[e], st[e + 1], st[e + 2], st[e + 3]);
        if (w.tp == 0 && w.dg == 0) L.energy[nst][tid / TPH] = make_float4(st[E], st[E + 1], st[E + 2], 0.f);
      }
      __syncthreads();  // `red` is reused by the next item
    }
    if (worker) {
      for (int k = 0; k < nst; ++k) {
        const int gi = first + k * G;
        const int b = __builtin_amdgcn_readfirstlane(gi / per), item = __builtin_amdgcn_readfirstlane(gi % per);
        const PoolItem<FP32> w(a, item, tid);
        const float4 en = L.energy[k][tid / TPH];
        const float e3[3] = {en.x, en.y, en.z};
        pool_write<FP32>(a, b, w, reinterpret_cast<const float *>(&L.means[k][tid * E / 4]), e3);
      }
    }
    __syncthreads();  // the slots are reused by the next round
  }
}

__device__ __forceinline__ bool waited_too_long(const SingleArgs &g, uint64_t t0) {
  return __builtin_amdgcn_s_memrealtime() - t0 > g.wait_ticks;
}

// One pass of the grid barrier: every workgroup sets its barrier word to
// `v`; workgroup 0 waits until every word holds v, then sets the go words to
// v; each of the others waits on one go word (one thread polling, about once
// a microsecond; kGoCopies copies on separate lines, so no one memory channel
// takes every poll). `before_go` runs in workgroup 0 between the two.
template <typename BeforeGo>
__device__ __forceinline__ void barrier_pass(const SingleArgs &g, uint64_t v, uint64_t t0, BeforeGo &&before_go) {
  if (threadIdx.x == 0) __hip_atomic_store(g.slots + blockIdx.x, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (blockIdx.x == 0) {
    for (;;) {
      int ok = 1;
      for (int w = threadIdx.x; w < (int)gridDim.x; w += blockDim.x)
        ok &= __hip_atomic_load(g.slots + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == v;
      if (__syncthreads_and(ok)) break;
      if (__syncthreads_or(threadIdx.x == 0 && waited_too_long(g, t0))) {
        if (threadIdx.x == 0) __hip_atomic_store(g.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(32);
    }
    before_go();
    if (threadIdx.x < kGoCopies)
      __hip_atomic_store(g.go + threadIdx.x * kGoStride, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (threadIdx.x == 0) {
    const uint64_t *go = g.go + (blockIdx.x % kGoCopies) * kGoStride;
    while (__hip_atomic_load(go, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != v) {
      if (waited_too_long(g, t0)) {
        __hip_atomic_store(g.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(32);
    }
  }
  __syncthreads();
}

// The grid barrier after the pooling, in two passes. Publishing to the other
// XCDs takes a write-back of this XCD's L2 (the release at device scope);
// issued by a workgroup while others still stream their pooling reads, those
// write-backs slowed the reads by 13% (measured). So the first pass only
// says that this workgroup's stores have reached its L2 (tag); once every
// workgroup is there, each writes its L2 back and says so (tag + 1), and
// after the second pass every workgroup invalidates its caches (the acquire
// at device scope).
__device__ __forceinline__ void grid_barrier(const SingleArgs &g) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have reached the L2
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  barrier_pass(g, g.tag, t0, [] {});
  if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  barrier_pass(g, g.tag + 1, t0, [] { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "agent"); });
  if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
}

// a temperature published with the tag: (tag32 << 32) | float bits
__device__ __forceinline__ uint64_t tagged(uint32_t tag32, float v) {
  return ((uint64_t)tag32 << 32) | __float_as_uint(v);
}

// word i of the published temperatures, once it carries the tag (1 after
// the wait limit without it, and status := 1)
__device__ __forceinline__ float wait_tau(const SingleArgs &g, int i, uint32_t tag32) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  uint64_t v;
  while (((v = __hip_atomic_load(g.tau_words + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) >> 32) != tag32) {
    if (waited_too_long(g, t0)) {
      __hip_atomic_store(g.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return 1.f;
    }
    __builtin_amdgcn_s_sleep(4);
  }
  return __uint_as_float((uint32_t)v);
}
constexpr int kTauCache = 512;  // heads whose temperatures a workgroup keeps in LDS

typedef const SingleParams __attribute__((address_space(4))) *ParamPtr;  // kernel-argument segment
template <typename T>
__device__ __forceinline__ T load_param(const T __attribute__((address_space(4))) *p) {
  T v;
  __builtin_memcpy(&v, (const T *)p, sizeof(T));
  return v;
}

template <int LO16, int HI16, bool PV, bool MIX, bool FP32>
__global__ __launch_bounds__(kFusedWaves * 64) __attribute__((amdgpu_waves_per_eu(4)))
void estimate_single_kernel(SingleParams P) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSingleLdsBytes];
  __shared__ int64_t ticket_s;
  __shared__ float tau_s[2];
  __shared__ float tau_cache[2 * kTauCache];
  const uint32_t tag32 = (uint32_t)P.g.tag;
  if (blockIdx.x == 0 && threadIdx.x == 0)  // tickets 0 .. G - 1 are taken implicitly (workgroup w: w)
    __hip_atomic_store(P.g.ticket, ((uint64_t)tag32 << 32) | gridDim.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  single_pool<FP32>(P.pa, P.batch, smem);
  grid_barrier(P.g);

  auto &T = *reinterpret_cast<TauLds *>(smem);
  auto &F = *reinterpret_cast<FusedLds *>(smem);
  const int nbh = P.sa.batch * P.sa.nh;
  for (int lbh = blockIdx.x; lbh < nbh; lbh += gridDim.x) {
    const int bh = (lbh / P.sa.nh) * P.sa.hq + P.sa.h0 + lbh % P.sa.nh;
    tau_reduce(P.ta, bh / P.sa.hq, bh % P.sa.hq, T.red, T.out);
    __syncthreads();
    if (threadIdx.x < 8) P.ta.tau[(int64_t)bh * 8 + threadIdx.x] = T.out[threadIdx.x];
    if (threadIdx.x < 2)
      __hip_atomic_store(P.g.tau_words + 2 * bh + threadIdx.x, tagged(tag32, T.out[threadIdx.x]), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }

  // every head's temperatures into LDS (when they fit), once they are published
  const bool cached = nbh <= kTauCache;
  if (cached) {
    for (int i = threadIdx.x; i < 2 * nbh; i += blockDim.x) {
      const int lbh = i >> 1;
      const int bh = (lbh / P.sa.nh) * P.sa.hq + P.sa.h0 + lbh % P.sa.nh;
      tau_cache[i] = wait_tau(P.g, 2 * bh + (i & 1), tag32);
    }
    __syncthreads();
  }

  const int nI = (P.sa.nb + kStrip - 1) / kStrip;
  const int64_t ntask = (int64_t)nI * nbh;
  int64_t ticket = blockIdx.x;
  int cur = -1;
  float th = 1.f, tl = 1.f;
  while (ticket < ntask) {
    // The arguments (the kernel's only one, at the start of its argument
    // segment) and the thread index are read through values opaque to the
    // compiler in every strip, so it re-reads them there instead of holding
    // them, and everything derived from them, in registers across the loop.
    ParamPtr pp = (ParamPtr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(pp));
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const ScoreArgs sa = load_param(&pp->sa);
    const TopPArgs tp = load_param(&pp->tp);
    const SingleArgs g = load_param(&pp->g);
    const int lbh = (int)(ticket % nbh), rank = (int)(ticket / nbh);
    const int I = sa.causal ? nI - 1 - rank : rank;
    const int bh = (lbh / sa.nh) * sa.hq + sa.h0 + lbh % sa.nh;
    __syncthreads();  // the previous strip is done with the LDS and tau_s
    if (cached) {
      th = tau_cache[2 * lbh];
      tl = tau_cache[2 * lbh + 1];
    } else if (bh != cur) {  // this head's temperatures, once they are published
      if (tid < 2) tau_s[tid] = wait_tau(g, 2 * bh + tid, tag32);
      __syncthreads();
      th = tau_s[0];
      tl = tau_s[1];
      cur = bh;
    }
    // the next ticket, taken once the strip's loads are done (a returning
    // atomic in flight would hold up every wait for them)
    uint64_t next = 0;
    score_topp_strip<LO16, HI16, PV, MIX>(sa, tp, I, bh, th, tl, F, tid, [&] {
      if (tid == 0) next = __hip_atomic_fetch_add(g.ticket, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    });
    if (tid == 0) {
      // a counter without this call's tag was not set by this call: stop
      ticket_s = (next >> 32) == tag32 ? (int64_t)(uint32_t)next : ntask;
      if ((next >> 32) != tag32) __hip_atomic_store(g.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    ticket = ticket_s;
  }
}

template <int LO16, int HI16, bool PV, bool MIX>
hipError_t launch_single_as(const SingleParams &P, int fp32, int grid_cap, hipStream_t s) {
  const void *f = fp32 ? reinterpret_cast<const void *>(&estimate_single_kernel<LO16, HI16, PV, MIX, true>)
                       : reinterpret_cast<const void *>(&estimate_single_kernel<LO16, HI16, PV, MIX, false>);
  int per_cu = 0, cus = 0, dev = 0;
  hipError_t e = stream_device(s, &dev);
  if (e == hipSuccess) e = device_cu_count(dev, &cus);
  if (e == hipSuccess) e = kernel_occupancy(f, kFusedWaves * 64, &per_cu);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const int G = min(per_cu * cus, grid_cap);
  SingleParams p = P;
  void *args[] = {&p};
  return hipLaunchCooperativeKernel(f, dim3(G), dim3(kFusedWaves * 64), args, 0, s);
}

}  // namespace

hipError_t launch_score(const ScoreArgs &a, hipStream_t s) {
  const int nI = (a.nb + 63) / 64;
  int per_head = 0;
  for (int I = 0; I < nI; ++I) per_head += ((a.causal ? I + 1 : nI) + kScoreTilesPerWg - 1) / kScoreTilesPerWg;
  const dim3 grid(per_head * a.nh * a.batch);  // heads x (full chunks, then remainders)
  // per-head bands (multiples of 16) take the run-time segment variant
  const bool def = !a.split && a.seg_lo == 32 && a.seg_hi == 64;
  const bool equal = !a.split && a.seg_lo == 0 && a.seg_hi == 128;
  const bool by8 = a.split || (a.seg_lo % 8 == 0 && a.seg_hi % 8 == 0);
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

hipError_t launch_score_topp(const ScoreArgs &a, const TopPArgs &t, hipStream_t s) {
  const dim3 grid(((a.nb + kStrip - 1) / kStrip) * a.nh * a.batch), block(kFusedWaves * 64);
  const bool def = !a.split && a.seg_lo == 32 && a.seg_hi == 64;
  const bool by16 = a.split || (a.seg_lo % 16 == 0 && a.seg_hi % 16 == 0);
  if (t.merge == PRISM_MERGE_MIX) {
    if (a.pervec) {
      if (by16) hipLaunchKernelGGL((score_topp_kernel<kRuntime16, 0, true, true>), grid, block, 0, s, a, t);
      else hipLaunchKernelGGL((score_topp_kernel<-1, -1, true, true>), grid, block, 0, s, a, t);
    } else if (by16) {
      hipLaunchKernelGGL((score_topp_kernel<kRuntime16, 0, false, true>), grid, block, 0, s, a, t);
    } else {
      hipLaunchKernelGGL((score_topp_kernel<-1, -1, false, true>), grid, block, 0, s, a, t);
    }
  } else if (a.pervec) {
    if (def) hipLaunchKernelGGL((score_topp_kernel<2, 4, true, false>), grid, block, 0, s, a, t);
    else if (by16) hipLaunchKernelGGL((score_topp_kernel<kRuntime16, 0, true, false>), grid, block, 0, s, a, t);
    else hipLaunchKernelGGL((score_topp_kernel<-1, -1, true, false>), grid, block, 0, s, a, t);
  } else if (def) {
    hipLaunchKernelGGL((score_topp_kernel<2, 4, false, false>), grid, block, 0, s, a, t);
  } else if (by16) {
    hipLaunchKernelGGL((score_topp_kernel<kRuntime16, 0, false, false>), grid, block, 0, s, a, t);
  } else {
    hipLaunchKernelGGL((score_topp_kernel<-1, -1, false, false>), grid, block, 0, s, a, t);
  }
  return hipGetLastError();
}

hipError_t launch_estimate_single(const SingleParams &P, int fp32, int grid_cap, hipStream_t s) {
  const bool def = P.sa.seg_lo == 32 && P.sa.seg_hi == 64;
  const bool by16 = P.sa.seg_lo % 16 == 0 && P.sa.seg_hi % 16 == 0;
  if (P.tp.merge == PRISM_MERGE_MIX) {
    if (P.sa.pervec) {
      if (by16) return launch_single_as<kRuntime16, 0, true, true>(P, fp32, grid_cap, s);
      return launch_single_as<-1, -1, true, true>(P, fp32, grid_cap, s);
    }
    if (by16) return launch_single_as<kRuntime16, 0, false, true>(P, fp32, grid_cap, s);
    return launch_single_as<-1, -1, false, true>(P, fp32, grid_cap, s);
  }
  if (P.sa.pervec) {
    if (def) return launch_single_as<2, 4, true, false>(P, fp32, grid_cap, s);
    if (by16) return launch_single_as<kRuntime16, 0, true, false>(P, fp32, grid_cap, s);
    return launch_single_as<-1, -1, true, false>(P, fp32, grid_cap, s);
  }
  if (def) return launch_single_as<2, 4, false, false>(P, fp32, grid_cap, s);
  if (by16) return launch_single_as<kRuntime16, 0, false, false>(P, fp32, grid_cap, s);
  return launch_single_as<-1, -1, false, false>(P, fp32, grid_cap, s);
}

hipError_t launch_topp(const TopPArgs &a, hipStream_t s) {
  const int rows = a.batch * a.nh * a.nb;
  const dim3 grid((rows + 1) / 2);
  // the row in registers: 32, 64 or 128 logits per lane
  if (a.nb <= 2048) hipLaunchKernelGGL((topp_kernel<32>), grid, dim3(256), 0, s, a);
  else if (a.nb <= 4096) hipLaunchKernelGGL((topp_kernel<64>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((topp_kernel<128>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace prism
