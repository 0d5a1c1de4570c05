// Host-only check of the C ABI layer (prism_abi.cpp) under AddressSanitizer
// and UndefinedBehaviorSanitizer. The kernel launchers are replaced by stubs
// that only count what would be enqueued, so every entry point runs its full
// host logic -- argument checks, workspace layout, launch arguments -- with
// valid, invalid and extreme arguments (sizes near the int64 range), and the
// checks below confirm that a rejected call enqueues nothing and an accepted
// one enqueues the documented kernels. Device pointers are fake and never
// dereferenced. Built and run by tests/test_abi_sanitized.py.
#include <climits>
#include <cstdio>
#include <cstring>

#include "prism.h"
#include "prism_kernels.h"

namespace prism {
int g_launches = 0;
hipError_t launch_pool(const PoolArgs &, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_tau(const TauArgs &, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_spectrum(const SpectrumArgs &, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_split(const SplitArgs &, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_score(const ScoreArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_topp(const TopPArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_score_topp(const ScoreArgs &, const TopPArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
SingleParams g_single;  // the last single-launch parameters
hipError_t launch_estimate_single(const SingleParams &p, int, int grid_cap, hipStream_t) {
  ++g_launches;
  g_single = p;
  return grid_cap >= 1 ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_attn_bf16(const AttnArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_attn_fp32(const AttnArgs &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t stream_device(hipStream_t, int *dev) { *dev = 0; return hipSuccess; }
bool g_capturing = false;  // what the capture query reports
hipError_t stream_capturing(hipStream_t, bool *capturing) { *capturing = g_capturing; return hipSuccess; }
hipError_t device_cu_count(int, int *cus) { *cus = 256; return hipSuccess; }
}  // namespace prism

namespace {
int g_fail = 0;
void* const FAKE = reinterpret_cast<void *>(0x7F0000000000ull);

#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);    \
      ++g_fail;                                                         \
    }                                                                   \
  } while (0)

prism_tensor_t tensor(int64_t seq, int64_t heads, int32_t dtype = PRISM_BF16, int64_t batch = 1) {
  prism_tensor_t t;
  std::memset(&t, 0, sizeof t);
  t.data = FAKE; t.dtype = dtype; t.batch = batch; t.seq = seq; t.heads = heads; t.head_dim = 128;
  t.stride_h = 128; t.stride_s = heads * 128; t.stride_b = seq * heads * 128;
  return t;
}
prism_mask_t mask(int64_t seq, int64_t heads, int64_t batch = 1, int32_t format = PRISM_MASK_U8) {
  prism_mask_t m;
  std::memset(&m, 0, sizeof m);
  const int64_t nb = (seq + 127) / 128;
  m.data = FAKE; m.batch = batch; m.heads = heads; m.nq_blocks = nb; m.nk_blocks = nb; m.block_size = 128;
  m.causal = 1; m.format = format;
  return m;
}
prism_cfg_t cfg() {
  prism_cfg_t c;
  std::memset(&c, 0, sizeof c);
  c.block_size = 128; c.d_high = 64; c.d_low = 96; c.p = 0.95f; c.causal = 1;
  c.workspace = FAKE; c.workspace_bytes = (size_t)1 << 40;
  return c;
}

// one estimator call; returns the status and checks the launch count rule
int est(prism_tensor_t q, prism_tensor_t k, prism_cfg_t c, prism_mask_t m, int expect_launches_if_ok) {
  prism::g_launches = 0;
  const int st = prism_estimate(&q, &k, &c, &m, nullptr);
  CHECK(st != PRISM_OK ? prism::g_launches == 0 : prism::g_launches == expect_launches_if_ok);
  prism::g_launches = 0;
  prism_workspace_layout_t L;
  const int st2 = prism_estimate_workspace_layout(&q, &k, &c, &L);
  CHECK(prism::g_launches == 0);
  if (st2 == PRISM_OK) CHECK(L.total_bytes == prism_estimate_workspace_bytes(&q, &k, &c) && L.total_bytes % 256 == 0);
  return st;
}
int attn(prism_tensor_t q, prism_tensor_t k, prism_tensor_t v, prism_mask_t m, prism_tensor_t o) {
  prism::g_launches = 0;
  const int st = prism_block_sparse_attn(&q, &k, &v, &m, &o, nullptr);
  CHECK(st != PRISM_OK ? prism::g_launches == 0 : prism::g_launches == 1);
  return st;
}
}  // namespace

int main() {
  CHECK(prism_abi_version() == PRISM_ABI_VERSION);
  for (int s = -3; s < 20; ++s) CHECK(prism_status_str(s) != nullptr);

  // accepted: three kernels up to 1024 blocks, four beyond
  CHECK(est(tensor(131072, 32), tensor(131072, 8), cfg(), mask(131072, 32), 3) == PRISM_OK);
  CHECK(est(tensor(131073, 32), tensor(131073, 8), cfg(), mask(131073, 32), 4) == PRISM_OK);
  CHECK(est(tensor(1 << 20, 32), tensor(1 << 20, 8), cfg(), mask(1 << 20, 32, 1, PRISM_MASK_BITS), 4) == PRISM_OK);
  CHECK(est(tensor(1, 1), tensor(1, 1), cfg(), mask(1, 1), 3) == PRISM_OK);
  {  // adaptive bands: pool, spectrum, split, scores + selection
    prism_cfg_t c = cfg();
    c.band_mode = PRISM_BANDS_ADAPTIVE;
    CHECK(est(tensor(131072, 32), tensor(131072, 8), c, mask(131072, 32), 4) == PRISM_OK);
    c.merge = PRISM_MERGE_MIX;
    CHECK(est(tensor(4096, 32), tensor(4096, 8), c, mask(4096, 32), 4) == PRISM_OK);
    CHECK(est(tensor(131073, 32), tensor(131073, 8), c, mask(131073, 32), 4) == PRISM_ERR_UNSUPPORTED);
  }
  {  // one persistent launch: up to 1024 blocks, static bands; its barrier words in the workspace
    prism_cfg_t c = cfg();
    c.flags = PRISM_EST_SINGLE_LAUNCH;
    prism_tensor_t q = tensor(131072, 32), k = tensor(131072, 8);
    CHECK(est(q, k, c, mask(131072, 32), 1) == PRISM_OK);
    prism_workspace_layout_t L;
    CHECK(prism_estimate_workspace_layout(&q, &k, &c, &L) == PRISM_OK);
    CHECK(L.barrier_offset % 256 == 0 && L.total_bytes >= L.barrier_offset + 4096 * 8 + 4);
    const char *ws = static_cast<const char *>(c.workspace);
    CHECK(reinterpret_cast<const char *>(prism::g_single.g.slots) == ws + L.barrier_offset);
    CHECK(reinterpret_cast<const char *>(prism::g_single.g.status) == ws + L.barrier_offset + 4096 * 8);
    CHECK(reinterpret_cast<const char *>(prism::g_single.g.ticket) == ws + L.barrier_offset + 4096 * 8 + 8);
    CHECK(reinterpret_cast<const char *>(prism::g_single.g.go) == ws + L.barrier_offset + 33024);
    CHECK(reinterpret_cast<const char *>(prism::g_single.g.tau_words) == ws + L.barrier_offset + 37120);
    CHECK(L.total_bytes >= L.barrier_offset + 37120 + 32 * 16);
    const uint64_t tag1 = prism::g_single.g.tag;
    CHECK(est(q, k, c, mask(131072, 32), 1) == PRISM_OK);
    CHECK(prism::g_single.g.tag != tag1 && (prism::g_single.g.tag & 1));  // a new value per call
    c.flags = PRISM_EST_SINGLE_LAUNCH | PRISM_EST_KEEP_LOGITS;
    CHECK(est(q, k, c, mask(131072, 32), 1) == PRISM_OK);
    c.flags = PRISM_EST_SINGLE_LAUNCH;
    CHECK(est(tensor(131073, 32), tensor(131073, 8), c, mask(131073, 32), 1) == PRISM_ERR_UNSUPPORTED);
    c.band_mode = PRISM_BANDS_ADAPTIVE;
    CHECK(est(q, k, c, mask(131072, 32), 1) == PRISM_ERR_UNSUPPORTED);
    c.band_mode = PRISM_BANDS_STATIC;
    c.flags = 4;
    CHECK(est(q, k, c, mask(131072, 32), 1) == PRISM_ERR_CONFIG);
    // the longest device wait: 10 s plus Q and K (2.7 GB here) at 0.5 TB/s, in 100 MHz ticks
    c.flags = PRISM_EST_SINGLE_LAUNCH;
    CHECK(est(q, k, c, mask(131072, 32), 1) == PRISM_OK);
    CHECK(prism::g_single.g.wait_ticks > 1000000000ull && prism::g_single.g.wait_ticks < 1100000000ull);
    // a capturing stream: refused, nothing enqueued (the default path is capturable)
    prism::g_capturing = true;
    CHECK(est(q, k, c, mask(131072, 32), 1) == PRISM_ERR_UNSUPPORTED);
    c.flags = 0;
    CHECK(est(q, k, c, mask(131072, 32), 3) == PRISM_OK);
    prism::g_capturing = false;
  }
  CHECK(attn(tensor(131072, 32), tensor(131072, 8), tensor(131072, 8), mask(131072, 32), tensor(131072, 32)) == PRISM_OK);

  // NULLs everywhere
  {
    prism_tensor_t q = tensor(4096, 32), k = tensor(4096, 8);
    prism_cfg_t c = cfg();
    prism_mask_t m = mask(4096, 32);
    prism::g_launches = 0;
    CHECK(prism_estimate(nullptr, &k, &c, &m, nullptr) == PRISM_ERR_NULL);
    CHECK(prism_estimate(&q, nullptr, &c, &m, nullptr) == PRISM_ERR_NULL);
    CHECK(prism_estimate(&q, &k, nullptr, &m, nullptr) == PRISM_ERR_NULL);
    CHECK(prism_estimate(&q, &k, &c, nullptr, nullptr) == PRISM_ERR_NULL);
    CHECK(prism_estimate_workspace_bytes(nullptr, &k, &c) == 0);
    CHECK(prism_estimate_workspace_layout(&q, &k, &c, nullptr) == PRISM_ERR_NULL);
    CHECK(prism_block_sparse_attn(&q, &k, &k, nullptr, &q, nullptr) == PRISM_ERR_NULL);
    CHECK(prism_block_sparse_attn(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == PRISM_ERR_NULL);
    CHECK(prism::g_launches == 0);
  }

  // extreme sizes and strides: every one must be refused (or accepted) without
  // signed overflow anywhere in the checks or the layout arithmetic
  const int64_t huge[] = {INT64_MAX, INT64_MAX / 2, INT64_MAX / 128, (int64_t)1 << 62, (int64_t)1 << 40,
                          (int64_t)1 << 32, (int64_t)1 << 31, 65536, 0, -1, INT64_MIN};
  for (int64_t x : huge) {
    prism_tensor_t q = tensor(4096, 32), k = tensor(4096, 8);
    prism_mask_t m = mask(4096, 32);
    prism_tensor_t t;
    t = q; t.seq = x; CHECK(est(t, k, cfg(), m, 3) != PRISM_OK);
    t = q; t.batch = x; CHECK(est(t, k, cfg(), m, 3) != PRISM_OK);
    t = q; t.heads = x; CHECK(est(t, k, cfg(), m, 3) != PRISM_OK);
    t = q; t.stride_s = x; est(t, k, cfg(), m, 3);
    t = q; t.stride_b = x; est(t, k, cfg(), m, 3);
    t = q; t.stride_h = x; est(t, k, cfg(), m, 3);
    prism_mask_t mm = m; mm.nq_blocks = x; CHECK(est(q, k, cfg(), mm, 3) != PRISM_OK);
    mm = m; mm.batch = x; CHECK(est(q, k, cfg(), mm, 3) != PRISM_OK);
    prism_tensor_t v = tensor(4096, 8), o = tensor(4096, 32);
    t = k; t.stride_s = x; attn(q, t, v, m, o);
    t = o; t.stride_s = x; attn(q, k, v, m, t);
    t = o; t.stride_b = x; attn(q, k, v, m, t);
    t = q; t.seq = x; CHECK(attn(t, k, v, m, o) != PRISM_OK);
    t = q; t.heads = x; CHECK(attn(t, k, v, m, o) != PRISM_OK);
    t = q; t.batch = x; CHECK(attn(t, k, v, m, o) != PRISM_OK);
  }
  // configuration extremes
  {
    prism_tensor_t q = tensor(4096, 32), k = tensor(4096, 8);
    prism_mask_t m = mask(4096, 32);
    prism_cfg_t c;
    const int32_t ints[] = {INT32_MIN, -1, 0, 1, 2, 63, 64, 128, 130, INT32_MAX};
    for (int32_t x : ints) {
      c = cfg(); c.d_high = x; est(q, k, c, m, 3);
      c = cfg(); c.d_low = x; est(q, k, c, m, 3);
      c = cfg(); c.block_size = x; est(q, k, c, m, 3);
      c = cfg(); c.tau_mode = x; est(q, k, c, m, 3);
      c = cfg(); c.rope_layout = x; est(q, k, c, m, 3);
      c = cfg(); c.flags = x; est(q, k, c, m, (x & PRISM_EST_SINGLE_LAUNCH) ? 1 : 3);
      c = cfg(); c.merge = x; est(q, k, c, m, 3);
      c = cfg(); c.band_mode = x; est(q, k, c, m, x == PRISM_BANDS_ADAPTIVE ? 4 : 3);
      prism_mask_t mm = m; mm.format = x; est(q, k, cfg(), mm, 3);
      mm = m; mm.block_size = x; est(q, k, cfg(), mm, 3);
    }
    const float ps[] = {-1.f, 0.f, 1e-30f, 0.5f, 1.f, 1.0000001f, 1e30f, __builtin_inff(), __builtin_nanf("")};
    for (float p : ps) { c = cfg(); c.p = p; est(q, k, c, m, 3); }
    c = cfg(); c.workspace_bytes = 0; CHECK(est(q, k, c, m, 3) == PRISM_ERR_WORKSPACE);
  }
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("abi host check: ok\n");
  return 0;
}
