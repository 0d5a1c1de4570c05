// C ABI of libprism: argument validation, workspace layout and launch order.
// Every check below runs on the host before the first HIP call of an entry
// point; a failed check returns its status with nothing enqueued.
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>

#include "prism.h"
#include "prism_kernels.h"

namespace {

using prism::kBlock;
using prism::kHeadDim;
using prism::kMaxBlocks;

constexpr int64_t kMaxKvRowStrideBytes = int64_t(1) << 24;
constexpr int64_t kMaxBatch = 65535;                                   // a grid dimension of the estimator
constexpr int64_t kMaxExtent = int64_t(kMaxBlocks) * kBlock;           // 2^20 tokens, heads or batch x heads
constexpr int64_t kMaxStride = int64_t(1) << 40;                      // elements

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int64_t esize(int32_t dtype) { return dtype == PRISM_BF16 ? 2 : 4; }

// one [batch, seq, heads, head_dim] operand
int check_tensor(const prism_tensor_t *t) {
  if (!t || !t->data) return PRISM_ERR_NULL;
  if (t->dtype != PRISM_BF16 && t->dtype != PRISM_FP32) return PRISM_ERR_DTYPE;
  if (t->batch < 1 || t->seq < 1 || t->heads < 1 || t->head_dim < 1) return PRISM_ERR_SHAPE;
  // Every extent and stride is bounded before any product is formed, so no
  // size arithmetic below (or in the layout) can overflow: batch < 2^16,
  // heads and seq <= 2^20, strides <= 2^40 elements.
  if (t->batch > kMaxBatch || t->heads > kMaxExtent || t->seq > kMaxExtent || t->head_dim != kHeadDim)
    return PRISM_ERR_UNSUPPORTED;
  if (t->heads * t->batch > kMaxExtent) return PRISM_ERR_UNSUPPORTED;  // grid size limit
  if (t->stride_b < 1 || t->stride_s < 1 || t->stride_h < 1) return PRISM_ERR_STRIDE;
  if (t->stride_b > kMaxStride || t->stride_s > kMaxStride || t->stride_h > kMaxStride) return PRISM_ERR_UNSUPPORTED;
  const int64_t es = esize(t->dtype);
  if (reinterpret_cast<uintptr_t>(t->data) % 16) return PRISM_ERR_ALIGN;
  if ((t->stride_b * es) % 16 || (t->stride_s * es) % 16 || (t->stride_h * es) % 16) return PRISM_ERR_ALIGN;
  return PRISM_OK;
}

// rows (b, s, h) of an output tensor must not overlap
bool non_overlapping(const prism_tensor_t *t) {
  struct D { int64_t stride, extent; } d[3] = {{t->stride_b, t->batch}, {t->stride_s, t->seq}, {t->stride_h, t->heads}};
  for (int x = 0; x < 3; ++x)
    for (int y = x + 1; y < 3; ++y)
      if (d[y].stride < d[x].stride) { D tmp = d[x]; d[x] = d[y]; d[y] = tmp; }
  int64_t span = t->head_dim;  // elements covered by one row
  for (int x = 0; x < 3; ++x) {
    if (d[x].extent == 1) continue;
    if (d[x].stride < span) return false;
    span = d[x].stride * d[x].extent;
  }
  return true;
}

int check_qk(const prism_tensor_t *q, const prism_tensor_t *k) {
  int st = check_tensor(q);
  if (st) return st;
  st = check_tensor(k);
  if (st) return st;
  if (q->dtype != k->dtype) return PRISM_ERR_DTYPE;
  if (q->batch != k->batch || q->seq != k->seq || q->head_dim != k->head_dim) return PRISM_ERR_SHAPE;
  if (q->heads % k->heads) return PRISM_ERR_SHAPE;
  return PRISM_OK;
}

// Launch geometry: the largest grid (one 512-thread workgroup per batch,
// query head and query block) stays below 2^32 work-items, and the batch,
// a second grid dimension of the estimator, below 65536.
int check_launch(int64_t batch, int64_t heads, int64_t nb) {
  if (batch > 65535) return PRISM_ERR_UNSUPPORTED;
  if (batch * heads * nb * 512 > (int64_t)0xFFFFFFFF) return PRISM_ERR_UNSUPPORTED;
  return PRISM_OK;
}

int check_cfg(const prism_cfg_t *cfg, int64_t seq) {
  if (!cfg) return PRISM_ERR_NULL;
  if (cfg->block_size < 1) return PRISM_ERR_CONFIG;
  if (cfg->d_high < 2 || cfg->d_high > kHeadDim || cfg->d_high % 2) return PRISM_ERR_CONFIG;
  if (cfg->d_low < 2 || cfg->d_low > kHeadDim || cfg->d_low % 2) return PRISM_ERR_CONFIG;
  if (!(cfg->p > 0.0f && cfg->p <= 1.0f)) return PRISM_ERR_CONFIG;
  if (cfg->causal != 0 && cfg->causal != 1) return PRISM_ERR_CONFIG;
  if (cfg->rope_layout != PRISM_ROPE_INTERLEAVED && cfg->rope_layout != PRISM_ROPE_HALF) return PRISM_ERR_CONFIG;
  if (cfg->tau_mode < PRISM_TAU_FULLSPEC || cfg->tau_mode > PRISM_TAU_PERVEC) return PRISM_ERR_CONFIG;
  if (cfg->flags & ~(PRISM_EST_KEEP_LOGITS | PRISM_EST_SINGLE_LAUNCH)) return PRISM_ERR_CONFIG;
  if (cfg->merge < PRISM_MERGE_UNION || cfg->merge > PRISM_MERGE_MIX) return PRISM_ERR_CONFIG;
  if (cfg->band_mode != PRISM_BANDS_STATIC && cfg->band_mode != PRISM_BANDS_ADAPTIVE) return PRISM_ERR_CONFIG;
  if (cfg->band_mode == PRISM_BANDS_ADAPTIVE &&
      (cfg->d_high % 16 || cfg->d_low % 16 || cfg->tau_mode == PRISM_TAU_PERVEC))
    return PRISM_ERR_CONFIG;
  if (cfg->block_size != kBlock) return PRISM_ERR_UNSUPPORTED;
  if ((seq + kBlock - 1) / kBlock > kMaxBlocks) return PRISM_ERR_UNSUPPORTED;
  // the mixture merge selects both branches' rows in one wave: fused path only
  if (cfg->merge == PRISM_MERGE_MIX && (seq + kBlock - 1) / kBlock > prism::kFusedMaxBlocks)
    return PRISM_ERR_UNSUPPORTED;
  // one launch: the fused scores and selection, and one grid barrier (no
  // spectrum and split phases)
  if ((cfg->flags & PRISM_EST_SINGLE_LAUNCH) &&
      ((seq + kBlock - 1) / kBlock > prism::kFusedMaxBlocks || cfg->band_mode != PRISM_BANDS_STATIC))
    return PRISM_ERR_UNSUPPORTED;
  return PRISM_OK;
}

int check_estimate_args(const prism_tensor_t *q, const prism_tensor_t *k, const prism_cfg_t *cfg) {
  int st = check_qk(q, k);
  if (st) return st;
  st = check_cfg(cfg, q->seq);
  if (st) return st;
  return check_launch(q->batch, q->heads, (q->seq + cfg->block_size - 1) / cfg->block_size);
}

void make_layout(const prism_tensor_t *q, const prism_tensor_t *k, const prism_cfg_t *cfg,
                 prism_workspace_layout_t *L) {
  const int64_t nb = (q->seq + cfg->block_size - 1) / cfg->block_size;
  const size_t b = (size_t)q->batch;
  size_t off = 0;
  L->qbar_offset = off; off = round_up(off + b * q->heads * nb * kHeadDim * 4, 256);
  L->kbar_offset = off; off = round_up(off + b * k->heads * nb * kHeadDim * 4, 256);
  L->qsq_offset = off;  off = round_up(off + b * q->heads * nb * 16, 256);
  L->ksq_offset = off;  off = round_up(off + b * k->heads * nb * 16, 256);
  L->tau_offset = off;  off = round_up(off + b * q->heads * 32, 256);
  const bool logits = nb > prism::kFusedMaxBlocks || (cfg->flags & PRISM_EST_KEEP_LOGITS);
  L->logits_plane = logits ? prism::logit_plane(nb, cfg->causal) : 0;
  L->logits_offset = off; off = round_up(off + b * q->heads * 2 * (size_t)L->logits_plane * 4, 256);
  const bool adaptive = cfg->band_mode == PRISM_BANDS_ADAPTIVE;
  L->spectrum_offset = off; off = round_up(off + (adaptive ? b * (q->heads + k->heads) * (kHeadDim / 2) * 8 : 0), 256);
  L->split_offset = off;    off = round_up(off + (adaptive ? b * q->heads * 16 : 0), 256);
  const bool single = cfg->flags & PRISM_EST_SINGLE_LAUNCH;
  L->barrier_offset = off;  off = round_up(off + (single ? prism::kSingleTauOffset + b * q->heads * 16 : 0), 256);
  L->total_bytes = off;
  L->nb = nb;
  const int lo_start = kHeadDim - cfg->d_low;
  L->seg_lo = cfg->d_high < lo_start ? cfg->d_high : lo_start;
  L->seg_hi = cfg->d_high < lo_start ? lo_start : cfg->d_high;
  L->overlap = (cfg->d_high + cfg->d_low > kHeadDim) ? 1 : 0;
  L->reserved = 0;
}

// format and alignment of a mask descriptor; 0 or a status
int check_mask_format(const prism_mask_t *m) {
  if (m->format != PRISM_MASK_U8 && m->format != PRISM_MASK_BITS) return PRISM_ERR_CONFIG;
  if (reinterpret_cast<uintptr_t>(m->data) % (m->format == PRISM_MASK_U8 ? 16 : 4)) return PRISM_ERR_ALIGN;
  return PRISM_OK;
}

// A value for the single-launch estimator's barrier words that no earlier
// call of this process wrote (and, seeded from the clock, that a stale
// workspace is unlikely to hold): odd, distinct per call.
uint64_t barrier_tag() {
  static const uint64_t seed =
      (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() * 0x9E3779B97F4A7C15ull;
  static std::atomic<uint64_t> calls{0};
  return (seed + 2 * calls.fetch_add(1, std::memory_order_relaxed)) | 1u;
}

prism::TensorArg targ(const prism_tensor_t *t) {
  prism::TensorArg a;
  a.data = t->data;
  a.sb = t->stride_b;
  a.ss = t->stride_s;
  a.sh = t->stride_h;
  a.heads = (int32_t)t->heads;
  return a;
}

}  // namespace

extern "C" {

int prism_abi_version(void) { return PRISM_ABI_VERSION; }

const char *prism_status_str(int status) {
  switch (status) {
    case PRISM_OK: return "ok";
    case PRISM_ERR_NULL: return "null pointer";
    case PRISM_ERR_DTYPE: return "unsupported or mismatched dtype";
    case PRISM_ERR_SHAPE: return "inconsistent shape";
    case PRISM_ERR_STRIDE: return "invalid stride";
    case PRISM_ERR_ALIGN: return "misaligned pointer or stride";
    case PRISM_ERR_CONFIG: return "invalid configuration";
    case PRISM_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case PRISM_ERR_UNSUPPORTED: return "unsupported size or setting";
    case PRISM_ERR_LAUNCH: return "kernel launch failed";
    case PRISM_ERR_SCRATCH: return "problem needs more workspace than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

int prism_estimate_workspace_layout(const prism_tensor_t *q, const prism_tensor_t *k, const prism_cfg_t *cfg,
                                    prism_workspace_layout_t *layout) {
  const int st = check_estimate_args(q, k, cfg);
  if (st) return st;
  if (!layout) return PRISM_ERR_NULL;
  make_layout(q, k, cfg, layout);
  return PRISM_OK;
}

size_t prism_estimate_workspace_bytes(const prism_tensor_t *q, const prism_tensor_t *k, const prism_cfg_t *cfg) {
  prism_workspace_layout_t L;
  if (prism_estimate_workspace_layout(q, k, cfg, &L) != PRISM_OK) return 0;
  return L.total_bytes;
}

}  // extern "C"

namespace prism {

int check_estimate_call(const prism_tensor_t *q, const prism_tensor_t *k, const prism_cfg_t *cfg,
                        const prism_mask_t *mask_out, prism_workspace_layout_t *L) {
  int st = check_estimate_args(q, k, cfg);
  if (st) return st;
  make_layout(q, k, cfg, L);
  if (!mask_out || !mask_out->data) return PRISM_ERR_NULL;
  if (mask_out->batch != q->batch || mask_out->heads != q->heads || mask_out->nq_blocks != L->nb ||
      mask_out->nk_blocks != L->nb || mask_out->block_size != cfg->block_size)
    return PRISM_ERR_SHAPE;
  return check_mask_format(mask_out);
}

int enqueue_estimate(const prism_tensor_t *q, const prism_tensor_t *k, const prism_cfg_t *cfg,
                     const prism_mask_t *mask_out, const prism_workspace_layout_t &L, void *workspace,
                     hipStream_t s) {
  char *ws = static_cast<char *>(workspace);
  const int fp32 = q->dtype == PRISM_FP32;
  const int nb = (int)L.nb;

  prism::PoolArgs pa;
  const prism_tensor_t *xs[2] = {q, k};
  for (int t = 0; t < 2; ++t) pa.x[t] = targ(xs[t]);
  pa.xbar[0] = reinterpret_cast<float *>(ws + L.qbar_offset);
  pa.xbar[1] = reinterpret_cast<float *>(ws + L.kbar_offset);
  pa.sq[0] = reinterpret_cast<float *>(ws + L.qsq_offset);
  pa.sq[1] = reinterpret_cast<float *>(ws + L.ksq_offset);
  pa.seq = (int)q->seq;
  pa.nb = nb;
  pa.block = cfg->block_size;
  pa.half_layout = cfg->rope_layout == PRISM_ROPE_HALF;
  pa.seg_lo = L.seg_lo;
  pa.seg_hi = L.seg_hi;

  prism::TauArgs ta;
  ta.qsq = pa.sq[0];
  ta.ksq = pa.sq[1];
  ta.tau = reinterpret_cast<float *>(ws + L.tau_offset);
  ta.hq = (int)q->heads;
  ta.hkv = (int)k->heads;
  ta.nb = nb;
  ta.d_high = cfg->d_high;
  ta.d_low = cfg->d_low;
  ta.overlap = L.overlap;
  ta.tau_mode = cfg->tau_mode;

  prism::ScoreArgs sc;
  sc.qbar = pa.xbar[0];
  sc.kbar = pa.xbar[1];
  sc.tau = ta.tau;
  sc.logits = reinterpret_cast<float *>(ws + L.logits_offset);
  sc.plane = L.logits_plane;
  sc.hq = ta.hq;
  sc.hkv = ta.hkv;
  sc.nb = nb;
  sc.batch = (int)q->batch;
  sc.seg_lo = L.seg_lo;
  sc.seg_hi = L.seg_hi;
  sc.overlap = L.overlap;
  sc.d_high = cfg->d_high;
  sc.d_low = cfg->d_low;
  sc.causal = cfg->causal;
  sc.qsq = pa.sq[0];
  sc.ksq = pa.sq[1];
  sc.pervec = cfg->tau_mode == PRISM_TAU_PERVEC;
  sc.keep_logits = L.logits_plane > 0;
  const bool adaptive = cfg->band_mode == PRISM_BANDS_ADAPTIVE;
  sc.split = adaptive ? reinterpret_cast<const int32_t *>(ws + L.split_offset) : nullptr;

  prism::TopPArgs tp;
  tp.logits = sc.logits;
  tp.mask = mask_out->data;
  tp.bits = mask_out->format == PRISM_MASK_BITS;
  tp.words = (int)((L.nb + 31) / 32);
  tp.plane = L.logits_plane;
  tp.hq = ta.hq;
  tp.nb = nb;
  tp.batch = (int)q->batch;
  tp.causal = cfg->causal;
  tp.p = cfg->p;
  tp.merge = cfg->merge;

  const int per_chunk_max = fp32 ? 8 : 16;  // heads one 256-thread workgroup covers per token
  const int nh[2] = {ta.hq, ta.hkv};
  for (int t = 0; t < 2; ++t) {
    const int hc = nh[t] < per_chunk_max ? nh[t] : per_chunk_max;
    pa.h0[t] = 0;
    pa.nheads[t] = nh[t];
    pa.heads_per_chunk[t] = hc;
    pa.chunks[t] = (nh[t] + hc - 1) / hc;
  }
  ta.h0 = 0;
  ta.nh = ta.hq;
  sc.h0 = tp.h0 = 0;
  sc.nh = tp.nh = ta.hq;
  if (cfg->flags & PRISM_EST_SINGLE_LAUNCH) {
    // One launch's tag baked into a captured graph would be replayed: the
    // barrier words would already hold it. Graph capture takes the default.
    bool capturing = true;
    if (prism::stream_capturing(s, &capturing) != hipSuccess || capturing) return PRISM_ERR_UNSUPPORTED;
    prism::SingleParams P;
    P.pa = pa;
    P.ta = ta;
    P.sa = sc;
    P.tp = tp;
    P.g.slots = reinterpret_cast<uint64_t *>(ws + L.barrier_offset);
    P.g.status = reinterpret_cast<int32_t *>(ws + L.barrier_offset + prism::kSingleStatusOffset);
    P.g.ticket = reinterpret_cast<uint64_t *>(ws + L.barrier_offset + prism::kSingleTicketOffset);
    P.g.go = reinterpret_cast<uint64_t *>(ws + L.barrier_offset + prism::kSingleGoOffset);
    P.g.tau_words = reinterpret_cast<uint64_t *>(ws + L.barrier_offset + prism::kSingleTauOffset);
    P.g.tag = barrier_tag();
    // Longest device-side wait: 10 s plus the pooling pass at 0.5 TB/s (a
    // twelfth of the part's read rate), so only a broken protocol reaches it.
    const double pooled = (double)q->batch * (double)q->seq * (double)(q->heads + k->heads) * kHeadDim *
                          (double)(fp32 ? 4 : 2);
    P.g.wait_ticks = (uint64_t)(1e8 * (10.0 + pooled / 5e11));
    P.batch = (int)q->batch;
    const hipError_t e = prism::launch_estimate_single(P, fp32, prism::kSingleMaxWgs, s);
    return e == hipSuccess ? PRISM_OK : PRISM_ERR_LAUNCH;
  }
  if (prism::launch_pool(pa, (int)q->batch, fp32, s) != hipSuccess) return PRISM_ERR_LAUNCH;
  if (adaptive) {
    prism::SpectrumArgs sa;
    sa.xbar[0] = pa.xbar[0];
    sa.xbar[1] = pa.xbar[1];
    sa.spec = reinterpret_cast<double *>(ws + L.spectrum_offset);
    sa.hq = ta.hq;
    sa.hkv = ta.hkv;
    sa.nb = nb;
    prism::SplitArgs sp;
    sp.spec = sa.spec;
    sp.tau = ta.tau;
    sp.split = reinterpret_cast<int32_t *>(ws + L.split_offset);
    sp.hq = ta.hq;
    sp.hkv = ta.hkv;
    sp.d_high = cfg->d_high;
    sp.d_low = cfg->d_low;
    sp.tau_mode = cfg->tau_mode;
    if (prism::launch_spectrum(sa, (int)q->batch, s) != hipSuccess) return PRISM_ERR_LAUNCH;
    if (prism::launch_split(sp, (int)q->batch, s) != hipSuccess) return PRISM_ERR_LAUNCH;
  } else if (prism::launch_tau(ta, (int)q->batch, s) != hipSuccess) {
    return PRISM_ERR_LAUNCH;
  }
  if (nb <= prism::kFusedMaxBlocks) {
    if (prism::launch_score_topp(sc, tp, s) != hipSuccess) return PRISM_ERR_LAUNCH;
  } else {
    if (prism::launch_score(sc, s) != hipSuccess) return PRISM_ERR_LAUNCH;
    if (prism::launch_topp(tp, s) != hipSuccess) return PRISM_ERR_LAUNCH;
  }
  return PRISM_OK;
}

}  // namespace prism

extern "C" {

int prism_estimate(const prism_tensor_t *q, const prism_tensor_t *k, const prism_cfg_t *cfg,
                   prism_mask_t *mask_out, void *stream) {
  prism_workspace_layout_t L;
  const int st = prism::check_estimate_call(q, k, cfg, mask_out, &L);
  if (st) return st;
  if (!cfg->workspace || reinterpret_cast<uintptr_t>(cfg->workspace) % 256 || cfg->workspace_bytes < L.total_bytes)
    return PRISM_ERR_WORKSPACE;
  return prism::enqueue_estimate(q, k, cfg, mask_out, L, cfg->workspace, static_cast<hipStream_t>(stream));
}

int prism_block_sparse_attn(const prism_tensor_t *q, const prism_tensor_t *k, const prism_tensor_t *v,
                            const prism_mask_t *mask, prism_tensor_t *out, void *stream) {
  int st = check_qk(q, k);
  if (st) return st;
  if ((st = check_tensor(v))) return st;
  if ((st = check_tensor(out))) return st;
  if (v->dtype != q->dtype || out->dtype != q->dtype) return PRISM_ERR_DTYPE;
  if (v->batch != q->batch || v->seq != q->seq || v->heads != k->heads || v->head_dim != q->head_dim)
    return PRISM_ERR_SHAPE;
  if (out->batch != q->batch || out->seq != q->seq || out->heads != q->heads || out->head_dim != q->head_dim)
    return PRISM_ERR_SHAPE;
  if (!non_overlapping(out)) return PRISM_ERR_STRIDE;
  // the bf16 kernel addresses K and V rows relative to each 64-key sub-tile
  // in 32 bits: row strides up to 16 MiB (sequence length and batch/head
  // strides are unrestricted)
  if (k->stride_s * esize(k->dtype) > kMaxKvRowStrideBytes || v->stride_s * esize(v->dtype) > kMaxKvRowStrideBytes)
    return PRISM_ERR_UNSUPPORTED;
  if (!mask || !mask->data) return PRISM_ERR_NULL;
  if (mask->causal != 0 && mask->causal != 1) return PRISM_ERR_CONFIG;
  if (mask->block_size < 1) return PRISM_ERR_SHAPE;
  if (mask->block_size != kBlock) return PRISM_ERR_UNSUPPORTED;
  const int64_t nb = (q->seq + kBlock - 1) / kBlock;
  if (nb > kMaxBlocks) return PRISM_ERR_UNSUPPORTED;
  if ((st = check_launch(q->batch, q->heads, nb))) return st;
  if (mask->batch != q->batch || mask->heads != q->heads || mask->nq_blocks != nb || mask->nk_blocks != nb)
    return PRISM_ERR_SHAPE;
  if ((st = check_mask_format(mask))) return st;

  prism::AttnArgs a;
  a.q = targ(q);
  a.k = targ(k);
  a.v = targ(v);
  a.o = targ(out);
  a.mask = mask->data;
  a.bits = mask->format == PRISM_MASK_BITS;
  a.words = (int)((nb + 31) / 32);
  a.batch = (int)q->batch;
  a.seq = (int)q->seq;
  a.nb = (int)nb;
  a.hq = (int)q->heads;
  a.hkv = (int)k->heads;
  a.causal = mask->causal;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)kHeadDim));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = q->dtype == PRISM_BF16 ? prism::launch_attn_bf16(a, s) : prism::launch_attn_fp32(a, s);
  return e == hipSuccess ? PRISM_OK : PRISM_ERR_LAUNCH;
}

}  // extern "C"
