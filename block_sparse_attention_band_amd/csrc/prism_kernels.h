// Internal interface between the C ABI layer (prism_abi.cpp) and the HIP
// kernels. Arguments reaching these launchers have been validated already.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
};

hipError_t launch_pool(const PoolArgs &a, int batch, int fp32, hipStream_t s);
hipError_t launch_tau(const TauArgs &a, int batch, hipStream_t s);
hipError_t launch_score(const ScoreArgs &a, hipStream_t s);
hipError_t launch_topp(const TopPArgs &a, hipStream_t s);
// both at once, logits kept on chip (nb <= kFusedMaxBlocks)
hipError_t launch_score_topp(const ScoreArgs &sc, const TopPArgs &tp, hipStream_t s);

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

}  // namespace prism
