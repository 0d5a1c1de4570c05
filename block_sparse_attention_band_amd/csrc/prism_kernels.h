// Internal interface between the C ABI layer (prism_abi.cpp) and the HIP
// kernels. Arguments reaching these launchers have been validated already.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "prism.h"

namespace prism {

constexpr int kHeadDim = 128;
constexpr int kBlock = 128;
constexpr int kMaxBlocks = 8192;   // blocks per sequence (1,048,576 tokens)
constexpr int kFusedMaxBlocks = 1024;  // rows up to this many blocks: scores and selection in one kernel
constexpr int kListCap = 2048;     // attention: key blocks compacted per pass over a mask row

// One tensor [batch, seq, heads, 128], strides in elements.
struct TensorArg {
  const void *data;
  int64_t sb, ss, sh;
  int32_t heads;
};

// ---------------------------------------------------------------- estimator
struct PoolArgs {
  TensorArg x[2];        // 0 = Q, 1 = K
  float *xbar[2];        // [batch][heads][nb][128], canonical frequency order
  float *sq[2];          // [batch][heads][nb][4]
  int32_t h0[2];         // first head of the range pooled, per tensor
  int32_t nheads[2];     // heads in the range
  int32_t chunks[2];     // head chunks per tensor
  int32_t heads_per_chunk[2];
  int32_t seq, nb, block;
  int32_t half_layout;   // 1: RoPE pair j = dims (j, j + 64)
  int32_t seg_lo, seg_hi;
};

// Adaptive bands: per-pair pooled spectra, then each head's split and
// temperatures from them.
struct SpectrumArgs {
  const float *xbar[2];    // Qbar [batch][Hq][nb][128], Kbar [batch][Hkv][nb][128] (canonical order)
  double *spec;            // [batch][Hq + Hkv][64]: mean over blocks of each pair's energy
  int32_t hq, hkv, nb;
};
struct SplitArgs {
  const double *spec;      // as written by the spectrum kernel
  float *tau;              // [batch][Hq][8], as the tau kernel's
  int32_t *split;          // [batch][Hq][4]: seg_lo, seg_hi, d_high, d_low
  int32_t hq, hkv;
  int32_t d_high, d_low;   // the static split the rule starts from
  int32_t tau_mode;        // FULLSPEC, NONE or UNIT
};

struct TauArgs {
  const float *qsq, *ksq;  // [batch][H][nb][4]
  float *tau;              // [batch][Hq][8]
  int32_t hq, hkv, nb;
  int32_t h0, nh;          // query heads h0 .. h0 + nh - 1
  int32_t d_high, d_low, overlap;
  int32_t tau_mode;        // prism_tau_mode_t
};

// Band logits in the workspace: one fp32 plane per (batch, query head,
// branch), planes `plane` floats apart. Row i of a plane starts at
// logit_row(i): packed lower triangle (rows padded to 4 floats) when causal,
// rows of round_up(nb, 4) floats otherwise.
__host__ __device__ inline int64_t logit_row(int64_t i, int64_t nb, int causal) {
  if (!causal) return i * ((nb + 3) & ~int64_t(3));
  const int64_t q = i >> 2, r = i & 3;  // sum over rows < i of 4 * ceil((row + 1) / 4)
  return 8 * q * (q + 1) + 4 * r * (q + 1);
}
__host__ __device__ inline int64_t logit_plane(int64_t nb, int causal) {
  return (logit_row(nb, nb, causal) + 63) & ~int64_t(63);  // 256-byte aligned planes
}

struct ScoreArgs {
  const float *qbar, *kbar, *tau;
  float *logits;           // [batch][Hq][2][plane]
  int64_t plane;
  int32_t hq, hkv, nb, batch;
  int32_t h0, nh;          // query heads h0 .. h0 + nh - 1
  int32_t seg_lo, seg_hi, overlap;
  int32_t d_high, d_low;
  int32_t causal;
  const float *qsq, *ksq;  // per-block segment energies (per-vector temperature)
  int32_t pervec;          // 1: scale logits by the per-vector band factors
  int32_t keep_logits;     // fused kernel: also store the logits in the planes
  const int32_t *split;    // adaptive bands: [batch][Hq][4] per head (seg_lo, seg_hi, d_high, d_low); else null
};

struct TopPArgs {
  const float *logits;
  void *mask;              // [batch][Hq][nb][row]: nb bytes, or `words` u32 of bits
  int32_t bits;            // 1: bit-packed rows
  int32_t words;           // u32 words per bit-packed row, ceil(nb / 32)
  int64_t plane;
  int32_t hq, nb, batch;
  int32_t h0, nh;          // query heads h0 .. h0 + nh - 1
  int32_t causal;
  float p;
  int32_t merge;           // prism_merge_t
};

hipError_t launch_pool(const PoolArgs &a, int batch, int fp32, hipStream_t s);
hipError_t launch_tau(const TauArgs &a, int batch, hipStream_t s);
hipError_t launch_spectrum(const SpectrumArgs &a, int batch, hipStream_t s);
hipError_t launch_split(const SplitArgs &a, int batch, hipStream_t s);
hipError_t launch_score(const ScoreArgs &a, hipStream_t s);
hipError_t launch_topp(const TopPArgs &a, hipStream_t s);
// both at once, logits kept on chip (nb <= kFusedMaxBlocks)
hipError_t launch_score_topp(const ScoreArgs &sc, const TopPArgs &tp, hipStream_t s);

// The estimator in one persistent launch (nb <= kFusedMaxBlocks, static
// bands): its grid-wide barrier words and status.
struct SingleArgs {
  uint64_t *slots;         // one barrier word per workgroup (any prior contents)
  int32_t *status;         // set to 1 when a workgroup gave up waiting
  uint64_t *ticket;        // the strips' ticket counter: (tag low 32 bits << 32) | next strip
  uint64_t *go;            // kGoCopies words kGoStride apart, := tag once every workgroup has reached the barrier
  uint64_t *tau_words;     // [batch * Hq][2]: tau_high, tau_low as (tag low 32 bits << 32) | float bits
  uint64_t tag;            // this call's value, unlike any earlier call's (odd)
  uint64_t wait_ticks;     // longest wait, in ticks of the 100 MHz real-time counter
};
constexpr int kSingleMaxWgs = 4096;  // barrier words in the workspace
constexpr int kGoCopies = 16, kGoStride = 32;  // go words: 16 copies, 256 bytes apart
// the barrier section: kSingleMaxWgs barrier words, the status word (8 bytes
// with padding), the ticket counter, the go words (from a 256-byte boundary),
// then two words per query head
constexpr size_t kSingleStatusOffset = kSingleMaxWgs * 8;
constexpr size_t kSingleTicketOffset = kSingleStatusOffset + 8;
constexpr size_t kSingleGoOffset = kSingleStatusOffset + 256;
constexpr size_t kSingleTauOffset = kSingleGoOffset + kGoCopies * kGoStride * 8;

struct SingleParams {
  PoolArgs pa;
  TauArgs ta;
  ScoreArgs sa;
  TopPArgs tp;
  SingleArgs g;
  int32_t batch;
};
hipError_t launch_estimate_single(const SingleParams &p, int fp32, int grid_cap, hipStream_t s);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  TensorArg q, k, v, o;
  const void *mask;        // [batch][Hq][nb][row]: nb bytes, or `words` u32 of bits
  int32_t bits;            // 1: bit-packed rows
  int32_t words;
  int32_t batch, seq, nb, hq, hkv;
  int32_t causal;
  float scale_log2;        // log2(e) / sqrt(head_dim)
};

hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_fp32(const AttnArgs &a, hipStream_t s);

// ---------------------------------------------------------- host helpers
// The estimator's host side, shared by the entry points that take a caller
// workspace and the one that uses the library's own scratch: every check but
// the workspace's (fills *L; PRISM_OK or the status), then the launches.
int check_estimate_call(const prism_tensor_t *q, const prism_tensor_t *k, const prism_cfg_t *cfg,
                        const prism_mask_t *mask_out, prism_workspace_layout_t *L);
int enqueue_estimate(const prism_tensor_t *q, const prism_tensor_t *k, const prism_cfg_t *cfg,
                     const prism_mask_t *mask_out, const prism_workspace_layout_t &L, void *workspace,
                     hipStream_t s);

// The device a stream belongs to (the current device for the null stream).
hipError_t stream_device(hipStream_t s, int *dev);
// Whether work enqueued on the stream now is being captured into a graph.
hipError_t stream_capturing(hipStream_t s, bool *capturing);
// Compute units of a device, queried once per device and cached.
hipError_t device_cu_count(int dev, int *cus);
// Workgroups of `threads` threads of kernel f resident per CU (on the current
// device; every device this library runs on is a gfx950), cached per kernel.
hipError_t kernel_occupancy(const void *f, int threads, int *per_cu);

}  // namespace prism
