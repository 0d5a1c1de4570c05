/*
 * prism.h -- C ABI of libprism: Prism's spectral-aware block-importance
 * estimator and the causal block-sparse attention prefill that consumes its
 * block mask, on AMD Instinct MI355X (gfx950).
 *
 * Method: "Prism: Spectral-Aware Block-Sparse Attention" (arXiv 2602.08426).
 * The pipeline (Prism review, paper.rainbus.top, pipeline paragraph):
 *   (1) slice post-RoPE Q, K into a high band (first d_high dims) and a low
 *       band (last d_low dims); (2) mean-pool each band over blocks of B
 *       tokens; (3) RMS energy of each pooled band; (4) a per-branch
 *       temperature tau_z that aligns the branch's logits with the full
 *       spectrum; (5) S_z = softmax(Qbar_z Kbar_z^T / (tau_z sqrt(d_z)));
 *       (6) Top-P per branch; (7) M = M_high OR M_low.
 * Block-sparse prefill (abstract; gist.science Technical Summary section 1)
 * then computes attention only on the selected (query block, key block) tiles.
 *
 * Conventions shared by every entry point
 *   - Every pointer in a descriptor is device memory owned by the caller.
 *     The library allocates nothing, frees nothing, never synchronises, and
 *     only enqueues work on `stream` (a hipStream_t; NULL = default stream).
 *   - Every argument check runs on the host before any HIP call. When a
 *     check fails the call returns its status, nothing is enqueued and no
 *     output is touched. PRISM_ERR_LAUNCH reports a failed launch; faults
 *     inside a kernel surface at the caller's next synchronisation.
 *   - Calls are reentrant and thread-safe; the library keeps no state
 *     between calls. Two calls that share an output or a workspace and run
 *     concurrently on different streams race.
 *   - Tensors are [batch, seq, heads, head_dim] with arbitrary element
 *     strides for batch, seq and heads (BSHD, BHSD, ...); the head_dim
 *     stride is 1. Grouped-query attention: query head h reads KV head
 *     h / (Hq / Hkv); Hq must be a multiple of Hkv.
 *   - Supported: head_dim 128, block size 128, bf16 throughout or fp32
 *     throughout, any seq >= 1 (a partial last block is handled), any
 *     batch >= 1, up to 8192 blocks per sequence (seq <= 1048576; scaling
 *     to a million tokens is the pages' stated future work, Prism review,
 *     limitations paragraph). Launch limits: batch <= 65535 and
 *     batch * query heads * blocks * 512 < 2^32; larger problems return
 *     PRISM_ERR_UNSUPPORTED (split them by batch or head); so do strides
 *     above 2^40 elements. Attention: the seq strides of k and v may span at
 *     most 16 MiB (16,777,216 bytes) per token; the tensors themselves may
 *     span any size (64-bit addressing).
 */
#ifndef PRISM_H
#define PRISM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PRISM_ABI_VERSION 7

typedef enum {
  PRISM_OK = 0,
  PRISM_ERR_NULL = 1,        /* a required pointer is NULL */
  PRISM_ERR_DTYPE = 2,       /* unknown dtype, or the tensors' dtypes differ */
  PRISM_ERR_SHAPE = 3,       /* sizes inconsistent with each other or non-positive */
  PRISM_ERR_STRIDE = 4,      /* a stride is non-positive or rows would overlap */
  PRISM_ERR_ALIGN = 5,       /* data pointer or row start not 16-byte aligned */
  PRISM_ERR_CONFIG = 6,      /* d_high, d_low, p, rope_layout, tau_mode, merge or band_mode out of
                                range, or a band mode the other settings exclude */
  PRISM_ERR_WORKSPACE = 7,   /* workspace NULL, not 256-byte aligned, or too small */
  PRISM_ERR_UNSUPPORTED = 8, /* valid but not built: head_dim != 128, block != 128, too many blocks */
  PRISM_ERR_LAUNCH = 9,      /* a kernel launch failed */
  PRISM_ERR_SCRATCH = 10     /* prism_estimate_noalloc: the problem needs more workspace than
                                PRISM_NOALLOC_SCRATCH_BYTES */
} prism_status_t;

typedef enum { PRISM_BF16 = 0, PRISM_FP32 = 1 } prism_dtype_t;

/* Where RoPE puts the two coordinates of frequency pair j (frequency falls
 * with j). INTERLEAVED: dims (2j, 2j+1) -- "first d_high dims" is then the
 * d_high/2 fastest pairs. HALF (rotate-half): dims (j, j + head_dim/2); the
 * bands are taken over the same frequency pairs. */
typedef enum { PRISM_ROPE_INTERLEAVED = 0, PRISM_ROPE_HALF = 1 } prism_rope_layout_t;

/* FULLSPEC: tau_z = R(Qbar,D_z) R(Kbar,D_z) / (R(Qbar,D_full) R(Kbar,D_full)),
 *           R = RMS over all pooled blocks of the head and the band's dims;
 *           tau_z = 1 when any R is 0.
 * NONE:     tau_z = 1 (plain pooled scores per band).
 * UNIT:     tau_z = R(Qbar,D_z) R(Kbar,D_z) (unit-energy reading; 1 when any R is 0).
 * PERVEC:   tau_z = 1, and the logit of query block i and key block j is scaled by
 *           r_z(Qbar_i) r_z(Kbar_j) with r_z(v) = R(v,D_full) / R(v,D_z) taken over
 *           that one pooled vector (1 when R(v,D_z) is 0).
 * UNIT and PERVEC are the two readings of the (unprinted) temperature formula
 * that FULLSPEC was chosen over; they exist for comparison. */
typedef enum {
  PRISM_TAU_FULLSPEC = 0,
  PRISM_TAU_NONE = 1,
  PRISM_TAU_UNIT = 2,
  PRISM_TAU_PERVEC = 3
} prism_tau_mode_t;

typedef struct {
  void *data;        /* device address of element [0, 0, 0, 0] */
  int32_t dtype;     /* prism_dtype_t */
  int32_t reserved;  /* set to 0 */
  int64_t batch, seq, heads, head_dim;
  int64_t stride_b, stride_s, stride_h; /* in elements; the head_dim stride is 1 */
} prism_tensor_t;

/* Storage of a block mask row (query block i of one batch and head).
 * U8:   nk_blocks bytes, byte j = 1 when key block j is selected, 0 otherwise
 *       (prism_block_sparse_attn treats any nonzero byte as selected).
 * BITS: ceil(nk_blocks / 32) 32-bit words, bit (j % 32) of word j / 32 set when
 *       key block j is selected; bits past nk_blocks are 0 (prism_estimate) or
 *       ignored (prism_block_sparse_attn). At a million tokens a U8 mask row is
 *       8 KB and a head's mask 64 MiB; BITS is 8 times smaller. */
typedef enum { PRISM_MASK_U8 = 0, PRISM_MASK_BITS = 1 } prism_mask_format_t;

typedef struct {
  void *data;        /* device, row-major [batch][heads][nq_blocks][row], row as `format` says;
                        4-byte aligned (BITS) or 16-byte aligned (U8) */
  int64_t batch, heads, nq_blocks, nk_blocks;
  int32_t block_size;
  int32_t causal;    /* prism_block_sparse_attn: 1 = blocks above the diagonal are ignored
                        even when set, and key s is masked for query t when s > t */
  int32_t format;    /* prism_mask_format_t */
  int32_t reserved;  /* set to 0 */
} prism_mask_t;

/* How the two branches' masks become the final mask. The pages' step (7) is
 * the union; the other two answer the weakness the Prism review lists (the
 * union may over-select) and exist for comparison.
 * UNION:     M = M_high OR M_low.
 * INTERSECT: M = M_high AND M_low.
 * MIX:       one Top-P at p on the equal-weight mixture (S_high + S_low) / 2 of
 *            the branches' block distributions (up to 1024 blocks). */
typedef enum { PRISM_MERGE_UNION = 0, PRISM_MERGE_INTERSECT = 1, PRISM_MERGE_MIX = 2 } prism_merge_t;

/* Band split. STATIC: d_high / d_low for every head (the pages' design).
 * ADAPTIVE (the review's other listed weakness, a static split for heads of
 * different spectra): per query head, the high band ends at the smallest
 * multiple of 8 RoPE pairs whose share of the head's pooled spectrum (per
 * pair: mean pooled energy of Qbar times that of Kbar, fastest pair first)
 * reaches the share that the static high band's d_high / 2 pairs hold in the
 * mean spectrum of all query heads (of that batch entry); the low band keeps
 * the static overlap d_high + d_low - head_dim, and each band keeps at least
 * 8 pairs. Heads that share one spectrum get the static split. Needs d_high
 * and d_low multiples of 16 and a tau_mode other than PERVEC. */
typedef enum { PRISM_BANDS_STATIC = 0, PRISM_BANDS_ADAPTIVE = 1 } prism_band_mode_t;

/* Estimator flags (prism_cfg_t.flags). KEEP_LOGITS: also store both branches'
 * logits in the workspace (see logits_offset) for inspection. Sequences of at
 * most 1024 blocks otherwise keep them on chip: their scores and selection
 * run in one kernel, and the workspace has no logit planes.
 * SINGLE_LAUNCH: run the whole estimator as one persistent kernel (a
 * cooperative launch, every workgroup resident) with a grid-wide barrier
 * between the pooling pass and the per-head temperatures, scores and
 * selection, instead of three launches; same results, bit for bit. Needs at
 * most 1024 blocks and PRISM_BANDS_STATIC (else PRISM_ERR_UNSUPPORTED). Its
 * device-side words live in the workspace's barrier section (see
 * barrier_offset); they are tagged with a value new to each call, so any
 * prior contents are fine (a stale word matching that tag by chance, odds
 * 2^-32 per word, would corrupt the call). The status word becomes 1 if a
 * workgroup waited longer than 10 s plus the time to read Q and K at
 * 0.5 TB/s (the call's outputs are then not valid); the library never clears
 * it. Not for HIP graph capture (a captured call would replay one tag):
 * PRISM_ERR_UNSUPPORTED on a capturing stream. */
#define PRISM_EST_KEEP_LOGITS 1
#define PRISM_EST_SINGLE_LAUNCH 2

typedef struct {
  int32_t block_size; /* B, tokens per block: 128 */
  int32_t d_high;     /* high-band width, even, 2..head_dim */
  int32_t d_low;      /* low-band width, even, 2..head_dim */
  float p;            /* Top-P mass threshold, 0 < p <= 1 (p = 1 keeps every admissible block) */
  int32_t causal;     /* 1: query block i scores key blocks j <= i only */
  int32_t rope_layout;/* prism_rope_layout_t */
  int32_t tau_mode;   /* prism_tau_mode_t */
  int32_t flags;      /* 0, or PRISM_EST_KEEP_LOGITS and/or PRISM_EST_SINGLE_LAUNCH */
  int32_t merge;      /* prism_merge_t (PRISM_MERGE_UNION: the pages' step (7)) */
  int32_t band_mode;  /* prism_band_mode_t (PRISM_BANDS_STATIC: the pages' split) */
  void *workspace;    /* device scratch, 256-byte aligned, >= prism_estimate_workspace_bytes() */
  size_t workspace_bytes;
} prism_cfg_t;

/* Byte offsets of the estimator's intermediates inside the workspace, valid
 * after prism_estimate's work has completed on its stream. Pooled vectors are
 * stored in canonical frequency order: canonical dim 2j and 2j+1 hold RoPE
 * pair j (for INTERLEAVED this is the physical order). The three segments
 * [0, seg_lo), [seg_lo, seg_hi), [seg_hi, head_dim) of canonical dims are
 * high-only, middle and low-only; the middle one belongs to both bands when
 * `overlap` is 1 (d_high + d_low > head_dim) and to neither when 0. With
 * PRISM_BANDS_ADAPTIVE the per-block energies and seg_lo / seg_hi are those of
 * the static split and each head's own segments are in the split section. */
typedef struct {
  size_t qbar_offset; /* fp32 [batch][Hq][nb][head_dim]: block means of Q */
  size_t kbar_offset; /* fp32 [batch][Hkv][nb][head_dim]: block means of K */
  size_t qsq_offset;  /* fp32 [batch][Hq][nb][4]: per-block sums of qbar^2 over the 3 segments, 0 */
  size_t ksq_offset;  /* fp32 [batch][Hkv][nb][4] */
  size_t tau_offset;  /* fp32 [batch][Hq][8]: tau_high, tau_low, Rq_high, Rq_low, Rq_full,
                         Rk_high, Rk_low, Rk_full */
  size_t logits_offset; /* present when logits_plane > 0 (nb > 1024, or PRISM_EST_KEEP_LOGITS):
                         fp32 [batch][Hq][2][logits_plane]: branch z's (0 high, 1 low) logits
                         L_z[i][j] in log2 units, log2(e) Qbar_z[i].Kbar_z[j] / (tau_z sqrt(d_z)).
                         causal: packed lower triangle, row i holds j = 0..i and starts at
                         8 Q (Q + 1) + 4 R (Q + 1) floats (Q = i / 4, R = i % 4; rows padded to
                         4 floats); otherwise row i holds all nb blocks and starts at
                         i * round_up(nb, 4). */
  int64_t logits_plane; /* floats between consecutive logit planes (a multiple of 64); 0 when
                           the logits are not stored */
  size_t spectrum_offset; /* PRISM_BANDS_ADAPTIVE: fp64 [batch][Hq + Hkv][head_dim / 2], the mean
                           pooled energy of each RoPE pair (query heads, then KV heads) */
  size_t split_offset;  /* PRISM_BANDS_ADAPTIVE: int32 [batch][Hq][4], each head's seg_lo,
                           seg_hi, d_high, d_low (the bands in canonical dims as above) */
  size_t total_bytes; /* == prism_estimate_workspace_bytes() */
  int64_t nb;         /* blocks per sequence, ceil(seq / block_size) */
  int32_t seg_lo, seg_hi, overlap, reserved;
  size_t barrier_offset; /* PRISM_EST_SINGLE_LAUNCH: 4096 uint64 barrier words (one per
                           workgroup), the int32 status word (padded to 8 bytes), a uint64
                           counter of score tasks, at byte 33024 16 go words 256 bytes apart,
                           then at byte 37120 two uint64 words per query head (batch * Hq)
                           that publish its temperatures */
} prism_workspace_layout_t;

/* Version of this ABI (PRISM_ABI_VERSION). */
int prism_abi_version(void);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char *prism_status_str(int status);

/* Workspace bytes prism_estimate needs for these shapes and settings, or 0
 * when the arguments are invalid (the same checks as prism_estimate, except
 * the workspace and mask). Host-only; no HIP call. */
size_t prism_estimate_workspace_bytes(const prism_tensor_t *q, const prism_tensor_t *k,
                                      const prism_cfg_t *cfg);

/* Fills *layout for these shapes and settings. Host-only; no HIP call.
 * Returns PRISM_OK or the status prism_estimate would return for the same
 * q, k and cfg (workspace and mask not checked). */
int prism_estimate_workspace_layout(const prism_tensor_t *q, const prism_tensor_t *k,
                                    const prism_cfg_t *cfg, prism_workspace_layout_t *layout);

/* Prism's block-importance estimator, steps (1)-(7) above.
 *   q: post-RoPE queries [batch, seq, Hq, head_dim]; k: post-RoPE keys
 *      [batch, seq, Hkv, head_dim]; same dtype, batch, seq, head_dim.
 *   cfg: band widths, p, causal flag, RoPE layout, temperature mode, workspace.
 *   mask_out: written in full, [batch][Hq][nb][row] in mask_out->format with
 *      nb = ceil(seq / block_size), block_size == cfg->block_size; every byte
 *      of the mask is written (0 above the diagonal when causal).
 * Work: one streaming read of Q and K (block means and segment energies),
 * a per-head temperature reduction, and per query block the two band score
 * rows, their softmax, Top-P and the union. Scores and selection run in fp32.
 * Three kernels in order on `stream` for up to 1024 blocks (scores and
 * selection fused, logits on chip), or one with PRISM_EST_SINGLE_LAUNCH;
 * four beyond (the logits pass through the workspace). Every row, up to 8192 blocks, is selected from registers
 * by the same radix select over fixed-point masses.
 * Deterministic: the same inputs give bit-identical masks and workspace. */
int prism_estimate(const prism_tensor_t *q, const prism_tensor_t *k, const prism_cfg_t *cfg,
                   prism_mask_t *mask_out, void *stream);

/* Bytes of the device array prism_estimate_noalloc uses as its workspace
 * (40 MiB: the 131,072-token Llama-3-8B layer needs 22 MB, the 64-query-head
 * share of a Llama-3-70B layer at the same length 37 MiB). */
#define PRISM_NOALLOC_SCRATCH_BYTES (40u << 20)

/* prism_estimate for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, checks, kernels and results as prism_estimate, except that
 * cfg->workspace and cfg->workspace_bytes are ignored: the workspace is a
 * device array of PRISM_NOALLOC_SCRATCH_BYTES inside the library, one per
 * device (held from the library's first use on that device until the process
 * ends; the stream's device is used). The call allocates nothing. Problems
 * whose workspace (prism_estimate_workspace_bytes) exceeds that size return
 * PRISM_ERR_SCRATCH with nothing enqueued. Every call on a device shares that
 * device's array, so calls that overlap on one device race (one stream, or
 * calls ordered by the caller, per device); the workspace intermediates are
 * not readable by the caller. */
int prism_estimate_noalloc(const prism_tensor_t *q, const prism_tensor_t *k, const prism_cfg_t *cfg,
                           prism_mask_t *mask_out, void *stream);

/* Causal block-sparse attention prefill (abstract; gist.science Technical
 * Summary section 1): for query t of query block i and head h,
 *   out[t] = sum_{s in A(t)} softmax_s(q_t . k_s / sqrt(head_dim)) v_s,
 *   A(t) = { s < seq : mask[i][s / B] == 1, and s <= t when mask->causal },
 * keys and values from KV head h / (Hq / Hkv); out[t] = 0 when A(t) is empty.
 *   q, out: [batch, seq, Hq, 128]; k, v: [batch, seq, Hkv, 128]; all one dtype.
 *   mask: [batch][Hq][nb][row] with block_size 128 in either format, e.g. from
 *      prism_estimate.
 * bf16: MFMA products with fp32 accumulation, fp32 online softmax, the
 * probabilities rounded to bf16 for the P.V product; out rounded to bf16.
 * fp32: fp32 throughout. Skipped blocks are neither read nor computed.
 * Deterministic: the same inputs give bit-identical outputs. */
int prism_block_sparse_attn(const prism_tensor_t *q, const prism_tensor_t *k, const prism_tensor_t *v,
                            const prism_mask_t *mask, prism_tensor_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PRISM_H */
