// Block-sparse causal attention prefill (Prism abstract; gist.science
// Technical Summary section 1: attention is computed only on the selected
// blocks). For query t of query block i, head h (KV head h / G):
//   out[t] = sum_{s in A(t)} softmax_s(q_t . k_s / sqrt(d)) v_s,
//   A(t) = { s < N : mask[i][s / 128] == 1, s <= t when causal },
// and out[t] = 0 when A(t) is empty.
//
// bf16 kernel (gfx950 MFMA), one workgroup of 4 waves per (batch, head,
// query block of 128 tokens); each wave owns 32 query rows.
//   * The workgroup compacts its mask row (bytes or bits) into an ascending
//     list of key blocks in LDS, 2048 blocks of the row at a time; only those
//     blocks are loaded and computed.
//   * Keys and values stream in sub-tiles of 64 tokens through two LDS
//     buffers by direct global-to-LDS loads (buffer_load ... lds, no staging
//     registers): the next sub-tile's loads are in flight while the current
//     one is computed, issued between its S MFMAs. Rows sit in LDS with
//     XOR-swizzled 16-byte chunks so every operand read is free of bank
//     conflicts; rows past the sequence end lie outside the buffer range and
//     read as zeros.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with Q held in registers. Key
//     rows are fed to the MFMA in a permuted order chosen so that each lane's
//     16 accumulator registers per 32-key tile hold, for k-step v, eight
//     consecutive keys 16v + 8*(lane/32) + 0..7 of one query column. The
//     softmax'd values are therefore already the B operand (P^T) of
//     O^T += V^T P^T. V^T operands come from V's row-major LDS tile through
//     gfx950's transposing LDS read (two ds_read_b64_tr_b16 per operand).
//     All K fragments of a sub-tile are read before its first MFMA and all
//     V^T fragments right after its last S MFMA, and the wave raises its
//     issue priority over the P.V MFMAs.
//   * Online softmax in fp32 registers (base 2, scale folded into one FMA).
//     The exponent reference only moves, and O and the row sum are only
//     rescaled, when some query's running max has grown by more than 8 in
//     log2 units (a wave-wide vote), so most sub-tiles skip the rescale. Row
//     sums accumulate the bf16-rounded probabilities (the values P.V uses)
//     with a bf16 dot2. The two lanes sharing a query column combine with a
//     cross-half lane swap. The causal mask is applied only on the diagonal
//     block, the sequence end only on the ragged last block.
//   * Work order: longest rows first; when the KV groups divide evenly over
//     the 8 XCDs, every XCD owns whole KV groups so a group's K/V tiles are
//     shared through that XCD's L2.
//   * Past 3072 blocks a KV group's K and V no longer stay in the caches
//     between query blocks and the K/V stream bounds the kernel: there one
//     workgroup of 8 waves serves two query heads of a group on the same
//     query block and loads each K/V sub-tile once for both.
// fp32 kernel: same contract in plain fp32 arithmetic (4 threads per query),
// for fp32 inputs.
#include "prism_kernels.h"

namespace prism {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
// Sequences longer than this many blocks take the head-pair kernel. Measured
// (Llama-3-8B-shaped layer, density 0.95, alternating launches on one box):
// the pair kernel is 1.3% slower at 1024 blocks and 2.1% at 2048 and 3072;
// on another box 1.7% faster at 3073, 6.2% at 3584 and 7.5% at 4096; ~1.3x
// faster at 8192, where the one-head kernel is bound by the K/V stream.
constexpr int kPairMinBlocks = 3072;
constexpr int kSub = 64;                 // keys per sub-tile
constexpr int kXcds = 8;

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// pack two fp32 to bf16 (round to nearest even) in one dword: lo | hi << 16
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
constexpr float kLazy = 8.0f;  // log2-domain slack before O and l are rescaled

// max / sum of lane l and lane l^32 (the two lanes holding one query column)
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// (batch, head, query block) of this workgroup
__device__ __forceinline__ void work_item(const AttnArgs &a, int &b, int &h, int &i) {
  const int bid = blockIdx.x;
  const int G = a.hq / a.hkv;
  const int ngroups = a.batch * a.hkv;
  if (ngroups % kXcds == 0 && (int)gridDim.x % kXcds == 0) {
    const int xcd = bid % kXcds;
    const int local = bid / kXcds;
    const int per_group = G * a.nb;
    const int slot = local / per_group;
    const int rem = local % per_group;
    const int group = xcd + kXcds * slot;
    b = group / a.hkv;
    const int g = group % a.hkv;
    i = a.nb - 1 - rem / G;
    h = g * G + rem % G;
  } else {
    const int nbh = a.batch * a.hq;
    i = a.nb - 1 - bid / nbh;
    b = (bid % nbh) / a.hq;
    h = (bid % nbh) % a.hq;
  }
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

// direct global -> LDS load: each lane's 16 bytes land at lds + 16 * lane
extern "C" __device__ void llvm_amdgcn_raw_buffer_load_lds(i32x4 rsrc, LDS_AS uint32_t *lds, int size, int voffset,
                                                           int soffset, int offset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");

// raw buffer resource over [base, base + nbytes) (wave-uniform)
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t nbytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r[1] = __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int)nbytes);
  r[3] = 0x00020000;
  return r;
}

__device__ __forceinline__ void dma16(const i32x4 &rs, uint8_t *lds, int voff, int soff) {
  llvm_amdgcn_raw_buffer_load_lds(rs, (LDS_AS uint32_t *)(LDS_AS void *)lds, 16, voff, soff, 0, 0);
}

// LDS tiles of 64 keys x 128 dims (256-byte rows, 16 chunks of 8 dims).
// K: chunk c of row r sits in slot c ^ (r & 15): the 16 rows one
//    ds_read_b128 pass touches land in 16 different bank groups.
// V: chunk c of row r sits in slot c ^ (4 * (r & 3)): the 4 rows x 4 chunks
//    a transposing read touches per half-wave land in 16 different groups.
// Block-list entries: key block j (13 bits, j < 8192) | 1 << 13 when the
// first head of the workgroup selected it | 1 << 14 for the second head.
constexpr uint32_t kBlockBits = 0x1FFFu;

__device__ __forceinline__ bool mask_bit(const AttnArgs &a, int64_t row_index, int j) {
  if (a.bits) return ((static_cast<const uint32_t *>(a.mask)[row_index * a.words + (j >> 5)] >> (j & 31)) & 1u) != 0u;
  return static_cast<const uint8_t *>(a.mask)[row_index * a.nb + j] != 0;
}

// Compacts the key blocks jlo..jhi (at most kListCap) selected by mask row
// row0 or (row1 >= 0) row1 into blist in ascending order with the per-head
// flags; one wave, lane 0 stores the count.
__device__ __forceinline__ void compact_row(const AttnArgs &a, int64_t row0, int64_t row1, int jlo, int jhi,
                                            int lane, uint16_t *blist, int *nsel) {
  int cnt = 0;
  for (int j0 = jlo; j0 <= jhi; j0 += 64) {
    const int j = j0 + lane;
    bool s0 = false, s1 = false;
    if (j <= jhi) {
      s0 = mask_bit(a, row0, j);
      s1 = row1 >= 0 && mask_bit(a, row1, j);
    }
    const bool sel = s0 || s1;
    const uint64_t bal = __ballot(sel);
    if (sel)
      blist[cnt + __popcll(bal & ((1ull << lane) - 1ull))] = (uint16_t)(j | (s0 ? 1u << 13 : 0u) | (s1 ? 1u << 14 : 0u));
    cnt += __popcll(bal);
  }
  if (lane == 0) *nsel = cnt;
}

__device__ __forceinline__ int kslot(int c, int r) { return c ^ (r & 15); }
__device__ __forceinline__ int vslot(int c, int r) { return c ^ ((r & 3) << 2); }

// PAIR: one workgroup of 8 waves serves two query heads of one KV group
// (waves 0-3 the first, 4-7 the second) on the same query block, over the
// union of their selected key blocks: every K/V sub-tile is loaded once for
// both, and a wave skips the blocks its own head did not select. It halves
// the K/V traffic per FLOP, which is what bounds very long sequences, where
// a KV group's K and V no longer stay in the caches between query blocks.
template <bool PAIR>
__global__ __launch_bounds__(PAIR ? 512 : 256, PAIR ? 1 : 2) void attn_bf16_kernel(AttnArgs a) {
  constexpr int NW = PAIR ? 8 : 4;  // waves
  constexpr int DPW = 16 / NW;      // DMA instructions per wave, per tensor and sub-tile
  __shared__ __attribute__((aligned(1024))) uint8_t K0[kSub * 256];
  __shared__ __attribute__((aligned(1024))) uint8_t K1[kSub * 256];
  __shared__ __attribute__((aligned(1024))) uint8_t V0[kSub * 256];
  __shared__ __attribute__((aligned(1024))) uint8_t V1[kSub * 256];
  __shared__ uint16_t blist[kListCap];
  __shared__ int nsel_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave & 3;   // the wave's 32-row slice of the query block
  const int l32 = lane & 31;
  const int hf = lane >> 5;  // lane half
  int b, h, i;
  if constexpr (PAIR) {
    AttnArgs ap = a;  // work items over head pairs
    ap.hq = a.hq / 2;
    int hp;
    work_item(ap, b, hp, i);
    h = 2 * hp + (wave >> 2);
  } else {
    work_item(a, b, h, i);
  }
  const int h0 = PAIR ? (h & ~1) : h;  // the workgroup's first head
  const int g = h / (a.hq / a.hkv);
  const int N = a.seq;
  const int64_t row0 = ((int64_t)b * a.hq + h0) * a.nb + i;
  const int64_t row1 = PAIR ? row0 + a.nb : -1;
  const uint32_t myflag = 1u << (13 + (PAIR ? (wave >> 2) : 0));
  const int jmax = a.causal ? i : a.nb - 1;

  // ---- compact the mask row(s) (the first kListCap blocks; the rest pass by
  // pass below): selected key blocks in ascending order
  if (wave == 0) compact_row(a, row0, row1, 0, min(jmax, kListCap - 1), lane, blist, &nsel_s);

  // ---- Q rows of this wave as MFMA B operands (registers for the whole loop)
  const int qrow = i * kBlock + wq * 32 + l32;
  const bool qvalid = qrow < N;
  bf16x8 qf[8];
  {
    // rows past the sequence end read the last row (never stored)
    const char *qp = static_cast<const char *>(a.q.data) +
                     ((int64_t)b * a.q.sb + (int64_t)min(qrow, N - 1) * a.q.ss + (int64_t)h * a.q.sh) * 2;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(ld16(qp + (16 * s + 8 * hf) * 2));
  }
  // Q must have landed before the loop on every path: s_waitcnt vmcnt(0)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  // ---- K/V of this (batch, KV head); row strides in bytes. The raw buffer
  // resource of a sub-tile starts at its first key row (64-bit address
  // arithmetic), so every buffer offset stays below 64 row strides whatever
  // the sequence length and layout (row strides up to 16 MiB, checked by the
  // host).
  const int64_t kss = a.k.ss * 2, vss = a.v.ss * 2;
  const char *kbase = static_cast<const char *>(a.k.data) + ((int64_t)b * a.k.sb + (int64_t)g * a.k.sh) * 2;
  const char *vbase = static_cast<const char *>(a.v.data) + ((int64_t)b * a.v.sb + (int64_t)g * a.v.sh) * 2;

  // DMA instruction u of wave w fills LDS bytes [(NW u + w) * 1024, +1024):
  // tile rows 4(NW u + w) .. +3, lane -> (row + lane/16, slot lane%16)
  int kdma[DPW], vdma[DPW];
#pragma unroll
  for (int u = 0; u < DPW; ++u) {
    const int row = 4 * (NW * u + wave) + (lane >> 4), slot = lane & 15;
    kdma[u] = row * (int)kss + (kslot(slot, row) << 4);
    vdma[u] = row * (int)vss + (vslot(slot, row) << 4);
  }
  // The loads of one sub-tile: dma_prep sets their buffer resources (scalar
  // work only), dma_one(u) issues load u (K for u < DPW, then V). A
  // sub-tile's record range ends with the sequence's last row, so rows past
  // the sequence end read as zeros: their scores are masked and their
  // probabilities are exactly 0. A sub-tile that is not needed (live false:
  // none follows the last) gets an empty range and only zero-fills the idle
  // buffer.
  i32x4 pk = {0, 0, 0, 0}, pv = {0, 0, 0, 0};
  uint8_t *pK = K0, *pV = V0;
  auto dma_prep = [&](int n, uint32_t ent, uint8_t *Kd, uint8_t *Vd, bool live) {
    const int kv0 = (int)(ent & kBlockBits) * kBlock + (n & 1) * kSub;
    const int rows = live ? min(kSub, N - kv0) : 0;  // <= 0 past the sequence end
    const int kv = live ? kv0 : 0;
    pk = make_rsrc(kbase + kv * kss, rows > 0 ? (uint32_t)((rows - 1) * kss + 256) : 0u);
    pv = make_rsrc(vbase + kv * vss, rows > 0 ? (uint32_t)((rows - 1) * vss + 256) : 0u);
    pK = Kd;
    pV = Vd;
  };
  auto dma_one = [&](int u) {
    if (u < DPW) dma16(pk, pK + (NW * u + wave) * 1024, kdma[u], 0);
    else dma16(pv, pV + (NW * (u - DPW) + wave) * 1024, vdma[u - DPW], 0);
  };
  auto dma_all = [&]() {
#pragma unroll
    for (int u = 0; u < 2 * DPW; ++u) dma_one(u);
  };

  // LDS read offsets. K (A operand of S^T): lane feeds key row 32t + pm,
  // chunk 2s + hf. V^T (A operand of O^T) by transposing reads: lane group
  // gr = lane/16 reads rows 16u + 8(gr/2) + (lane%16)/4 (+4 for the upper
  // half of the k-step) and dims 32d + 16(gr%2) + 4(lane%4); each lane then
  // holds 4 consecutive keys of dim 32d + lane%32.
  const int pm = 16 * (l32 >> 4) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);
  int kaddr[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) kaddr[s] = pm * 256 + (kslot(2 * s + hf, pm) << 4);
  int vaddr[4];
  {
    const int gr = (lane >> 4) & 3, s16 = lane & 15;
    const int row = 8 * (gr >> 1) + (s16 >> 2);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int c = 4 * d + 2 * (gr & 1) + ((s16 & 3) >> 1);
      vaddr[d] = row * 256 + (vslot(c, row) << 4) + 8 * (s16 & 1);
    }
  }

  f32x16 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[d][r] = 0.f;
  float m_ref = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;

  auto compute = [&](int n, uint32_t ent, const uint8_t *Kb, const uint8_t *Vb) {
    const int j = (int)(ent & kBlockBits);
    const int kv0 = j * kBlock + (n & 1) * kSub;
    const bool diag = a.causal && j == i;
    // The head-pair kernel skips a block this wave's head did not select
    // (the other head's), a whole sub-tile after every query of this wave
    // and one past the sequence end. The single-head kernel computes the
    // last two as fully masked sub-tiles (probabilities exactly 0; two waves
    // on the diagonal block, once per row): its compute carries the next
    // sub-tile's loads, which every wave must issue.
    if constexpr (PAIR) {
      if (!(ent & myflag) || (diag && kv0 > i * kBlock + wq * 32 + 31) || kv0 >= N) return;
    }
    // All 16 K fragments of the sub-tile are requested before the first
    // MFMA, and all 16 V^T fragments right after the last S MFMA (they are in
    // flight during the softmax): each MFMA then waits for at most one LDS
    // round trip per sub-tile instead of one per MFMA. The scheduling
    // barriers keep the compiler from interleaving the reads back into the
    // MFMA chain.
    bf16x8 kf[2][8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) kf[t][s] = as_bf16x8(*reinterpret_cast<const uint4 *>(Kb + t * 8192 + kaddr[s]));
    __builtin_amdgcn_sched_barrier(0);
    f32x16 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int t = 0; t < 2; ++t) sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t][s], qf[s], sacc[t], 0, 0, 0);
      if constexpr (!PAIR) dma_one(s);
    }
    if constexpr (!PAIR) {
      // Single-head kernel: the next sub-tile's eight loads go out one after
      // every two S MFMAs, so the wave waits for the load path (which the
      // workgroup's 32 loads keep busy for ~500 cycles) while its own MFMAs
      // run, instead of all at once after the barrier; all V^T reads follow
      // the last S MFMA (0.8% faster than letting the compiler spread them
      // over the last few).
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        if (s == 7) __builtin_amdgcn_sched_group_barrier(0x100, 32, 0);  // DS read
      }
    }
    bf16x8 vf[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4 *)(LDS_AS void *)(Vb + u * 4096 + vaddr[d]));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4 *)(LDS_AS void *)(Vb + u * 4096 + 1024 + vaddr[d]));
        vf[d][u] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    __builtin_amdgcn_sched_barrier(0);
    // sacc[t][r] = q_row . k_s with s = kv0 + 32t + 16(r/8) + 8*hf + r%8
    if (diag || kv0 + kSub > N) {
      const int lim = a.causal ? min(qrow, N - 1) : N - 1;  // last admissible key
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int s = kv0 + 32 * t + 16 * (r >> 3) + 8 * hf + (r & 7);
          sacc[t][r] = s > lim ? -INFINITY : sacc[t][r];
        }
    }
    // row max as two chains of three-input maxes (one v_max3 per two scores)
    float ma = fmaxf(sacc[0][0], sacc[0][1]), mb = fmaxf(sacc[1][0], sacc[1][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
      ma = __builtin_fmaxf(__builtin_fmaxf(ma, sacc[0][r]), sacc[0][r + 1]);
      mb = __builtin_fmaxf(__builtin_fmaxf(mb, sacc[1][r]), sacc[1][r + 1]);
    }
    const float mloc = xhalf_max(fmaxf(ma, mb));
    // Lazy rescaling: the exponent reference m_ref only moves (and O, l are
    // rescaled) when some query's running max exceeds it by more than
    // kLazy in log2 units; until then p <= 2^kLazy, exact in fp32/bf16 range.
    const float m_new = fmaxf(m_ref, mloc);
    if (__any((m_new - m_ref) * c > kLazy)) {
      const float alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_ref - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[d][r] *= alpha;
      m_ref = m_new;
    }
    const float mc = (m_ref == -INFINITY ? 0.f : m_ref) * c;
    bf16x8 pf[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[t][8 * v + e], c, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[t][8 * v + e + 1], c, -mc));
          w[e >> 1] = pack_bf16(p0, p1);
          // row sum of the rounded probabilities, the values P.V uses
          l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e >> 1]), kOnes2, l_run, false);
        }
        pf[2 * t + v] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
      }
    // O^T[dv][q] += V^T[dv][kv] P^T[kv][q]. The wave raises its issue
    // priority for this block: the other wave on the SIMD (another
    // workgroup) then fills the gaps with its own softmax VALU work instead
    // of competing with these MFMAs (about 2% over equal priority).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int u = 0; u < 4; ++u) oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[d][u], pf[u], oacc[d], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  for (int cb = 0;;) {
    const int nsel = nsel_s;
    const int nsub = 2 * nsel;
    // Block list entries (uniform): e_cur is the block of sub-tiles n and
    // n + 1; the next block's entry is read from LDS a whole sub-tile ahead,
    // so its latency hides behind the fragment reads instead of stalling the
    // wave twice per sub-tile between the barrier and its next MFMA (a
    // per-wave timeline measured ~300 cycles per round trip there).
    uint32_t e_cur = nsel > 0 ? (uint32_t)__builtin_amdgcn_readfirstlane((int)blist[0]) : 0u;
    if (nsub > 0) {
      dma_prep(0, e_cur, K0, V0, true);
      dma_all();
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    __syncthreads();
    // The next sub-tile's loads are prepared before the barrier that
    // precedes their issue, so the fragment reads follow a barrier at once.
    // The single-head kernel issues them inside compute (between its S
    // MFMAs), the head-pair kernel before it.
    if (nsub > 0) dma_prep(1, e_cur, K1, V1, 1 < nsub);
    for (int n = 0; n < nsub; n += 2) {
      const int e_raw = (n >> 1) + 1 < nsel ? (int)blist[(n >> 1) + 1] : 0;
      if constexpr (PAIR) dma_all();
      compute(n, e_cur, K0, V0);
      const uint32_t e_nxt = (uint32_t)__builtin_amdgcn_readfirstlane(e_raw);
      dma_prep(n + 2, e_nxt, K0, V0, n + 2 < nsub);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      if (n + 1 >= nsub) break;
      if constexpr (PAIR) dma_all();
      compute(n + 1, e_cur, K1, V1);
      dma_prep(n + 3, e_nxt, K1, V1, n + 3 < nsub);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      e_cur = e_nxt;
    }
    // rows longer than kListCap blocks: the next part of the mask row (every
    // wave has passed the last barrier, so blist is free)
    cb += kListCap;
    if (cb > jmax) break;
    if (wave == 0) compact_row(a, row0, row1, cb, min(jmax, cb + kListCap - 1), lane, blist, &nsel_s);
    __syncthreads();
  }

  // ---- normalise and store: oacc[d][r] = O[qrow][32d + 8(r/4) + 4*hf + r%4]
  const float l_tot = xhalf_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (qvalid) {
    char *op = static_cast<char *>(const_cast<void *>(a.o.data)) +
               ((int64_t)b * a.o.sb + (int64_t)qrow * a.o.ss + (int64_t)h * a.o.sh) * 2;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        uint2 w;
        w.x = pack_bf16(oacc[d][4 * r4 + 0] * inv, oacc[d][4 * r4 + 1] * inv);
        w.y = pack_bf16(oacc[d][4 * r4 + 2] * inv, oacc[d][4 * r4 + 3] * inv);
        *reinterpret_cast<uint2 *>(op + (32 * d + 8 * r4 + 4 * hf) * 2) = w;
      }
  }
}

// ------------------------------------------------------------------ fp32
constexpr int kF32Threads = 512;  // 128 queries x 4 threads
constexpr int kF32Tile = 32;      // keys per LDS tile

__global__ __launch_bounds__(kF32Threads) void attn_fp32_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) float Kt[kF32Tile * kHeadDim];
  __shared__ __attribute__((aligned(16))) float Vs[kF32Tile * kHeadDim];
  __shared__ uint16_t blist[kListCap];
  __shared__ int nsel_s;

  int b, h, i;
  work_item(a, b, h, i);
  const int g = h / (a.hq / a.hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int qi = tid >> 2;   // query within the block
  const int part = tid & 3;  // 32-dim slice
  const int N = a.seq;
  const int qrow = i * kBlock + qi;
  const bool qvalid = qrow < N;
  const int64_t mrow_index = ((int64_t)b * a.hq + h) * a.nb + i;
  const int jmax = a.causal ? i : a.nb - 1;

  if (tid < 64) compact_row(a, mrow_index, -1, 0, min(jmax, kListCap - 1), lane, blist, &nsel_s);

  float qv[32], ov[32];
  {
    const float *qp = static_cast<const float *>(a.q.data) + (int64_t)b * a.q.sb + (int64_t)qrow * a.q.ss +
                      (int64_t)h * a.q.sh + 32 * part;
#pragma unroll
    for (int e = 0; e < 32; ++e) { qv[e] = qvalid ? qp[e] : 0.f; ov[e] = 0.f; }
  }
  __syncthreads();
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;
  const float *kb = static_cast<const float *>(a.k.data) + (int64_t)b * a.k.sb + (int64_t)g * a.k.sh;
  const float *vb = static_cast<const float *>(a.v.data) + (int64_t)b * a.v.sb + (int64_t)g * a.v.sh;

  for (int cb = 0;;) {
  const int nsel = nsel_s;
  for (int n = 0; n < nsel * (kBlock / kF32Tile); ++n) {
    const int j = (int)(blist[n / (kBlock / kF32Tile)] & kBlockBits);
    const int kv0 = j * kBlock + (n % (kBlock / kF32Tile)) * kF32Tile;
    for (int c4 = tid; c4 < kF32Tile * kHeadDim / 4; c4 += kF32Threads) {
      const int row = c4 / (kHeadDim / 4), col = (c4 % (kHeadDim / 4)) * 4;
      const int s = kv0 + row;
      float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
      if (s < N) {
        kx = *reinterpret_cast<const float4 *>(kb + (int64_t)s * a.k.ss + col);
        vx = *reinterpret_cast<const float4 *>(vb + (int64_t)s * a.v.ss + col);
      }
      *reinterpret_cast<float4 *>(&Kt[row * kHeadDim + col]) = kx;
      *reinterpret_cast<float4 *>(&Vs[row * kHeadDim + col]) = vx;
    }
    __syncthreads();
    for (int kk = 0; kk < kF32Tile; ++kk) {
      const int s = kv0 + kk;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) dot = fmaf(qv[e], Kt[kk * kHeadDim + 32 * part + e], dot);
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      const bool ok = s < N && (!a.causal || s <= qrow);
      if (ok) {
        const float m_new = fmaxf(m_run, dot);
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
        const float p = __builtin_amdgcn_exp2f((dot - m_new) * c);
        l_run = l_run * alpha + p;
#pragma unroll
        for (int e = 0; e < 32; ++e) ov[e] = fmaf(p, Vs[kk * kHeadDim + 32 * part + e], ov[e] * alpha);
        m_run = m_new;
      }
    }
    __syncthreads();
  }
  // rows longer than kListCap blocks: the next part of the mask row, once
  // every thread has read this part's count and list
  cb += kListCap;
  if (cb > jmax) break;
  __syncthreads();
  if (tid < 64) compact_row(a, mrow_index, -1, cb, min(jmax, cb + kListCap - 1), lane, blist, &nsel_s);
  __syncthreads();
  }
  if (qvalid) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float *op = static_cast<float *>(const_cast<void *>(a.o.data)) + (int64_t)b * a.o.sb + (int64_t)qrow * a.o.ss +
                (int64_t)h * a.o.sh + 32 * part;
#pragma unroll
    for (int e = 0; e < 32; e += 4)
      *reinterpret_cast<float4 *>(op + e) = make_float4(ov[e] * inv, ov[e + 1] * inv, ov[e + 2] * inv, ov[e + 3] * inv);
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t s) {
  // head pairs share K/V tiles on long sequences (an even group size needed)
  if ((a.hq / a.hkv) % 2 == 0 && a.nb > kPairMinBlocks)
    hipLaunchKernelGGL(attn_bf16_kernel<true>, dim3(a.batch * (a.hq / 2) * a.nb), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<false>, dim3(a.batch * a.hq * a.nb), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_fp32(const AttnArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(attn_fp32_kernel, dim3(a.batch * a.hq * a.nb), dim3(kF32Threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace prism
