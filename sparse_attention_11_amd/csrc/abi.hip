// C ABI of libdsa (declared in include/dsa.h): argument validation, per-launch segment
// tables, workspace layout and kernel launches on the caller's stream.  Nothing here
// allocates device memory or synchronises the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "dsa.h"
#include "dsa_device.h"

namespace dsa {
hipError_t launch_indexer(const IndexerArgs& a, int h_idx, int d_idx, bool fp8, hipStream_t s);
hipError_t launch_fill_outside(const FillArgs& a, hipStream_t s);
int indexer_rows_per_block();
hipError_t launch_topk(const TopkArgs& a, int max_window, hipStream_t s);
hipError_t launch_sparse_attn(const AttnArgs& a, int h, int d_qk, int d_v, int nblocks,
                              hipStream_t s);
hipError_t launch_sparse_attn_bwd(const AttnBwdArgs& a, int h, int d_qk, int d_v, hipStream_t s);
hipError_t launch_quant_fp8_rows(const QuantArgs& a, hipStream_t s);
hipError_t launch_indexer_kl(const IdxKlArgs& a, const KeyListArgs& kl, hipStream_t s, bool lists);
hipError_t launch_loss_total(const float* loss, int n, float* out, hipStream_t s);
hipError_t launch_dense_attn(const DenseArgs& a, int nqblk, hipStream_t s);
int dense_rows_per_block();
}  // namespace dsa

namespace {

thread_local std::string g_err;

dsa_status fail(dsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

dsa_status ok() {
  g_err.clear();
  return DSA_OK;
}

dsa_status hip_fail(hipError_t e, const char* what) {
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxTopk = 4096;
constexpr int64_t kMaxWindow = 65536;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool indexer_dims_ok(int h_idx, int d_idx) {
  return (h_idx == 64 && d_idx == 128) || (h_idx == 4 && d_idx == 32);
}
bool attn_dims_ok(int h, int d_qk, int d_v) {
  return (h == 128 && d_qk == 576 && d_v == 512) || (h == 8 && d_qk == 80 && d_v == 64);
}

struct Plan {
  std::vector<dsa_segment> segs;  // non-empty segments, longest windows first
  int64_t max_window = 0;         // longest window over all rows
  int64_t covered_rows = 0;
};

enum Need { kNeedIndexer = 1, kNeedTopk = 2, kNeedAttn = 4, kNeedSegs = 8 };

dsa_status check_shape(const dsa_shape* s, int need, Plan& p) {
  if (!s) return fail(DSA_ERR_INVALID_ARG, "shape is NULL");
  if (s->n_q < 0 || s->n_k < 0) return fail(DSA_ERR_INVALID_ARG, "negative n_q or n_k");
  if ((need & (kNeedTopk | kNeedAttn)) && (s->topk < 1))
    return fail(DSA_ERR_INVALID_ARG, "topk must be >= 1 (got %d)", s->topk);
  if ((need & (kNeedTopk | kNeedAttn)) && s->topk > kMaxTopk)
    return fail(DSA_ERR_UNSUPPORTED, "topk %d > %d", s->topk, kMaxTopk);
  if (need & kNeedIndexer) {
    if (s->idx_dtype != DSA_IDX_BF16 && s->idx_dtype != DSA_IDX_FP8_E4M3)
      return fail(DSA_ERR_INVALID_ARG, "unknown idx_dtype %d", s->idx_dtype);
    if (!indexer_dims_ok(s->h_idx, s->d_idx))
      return fail(DSA_ERR_UNSUPPORTED, "indexer dims (h_idx=%d, d_idx=%d) not built",
                  s->h_idx, s->d_idx);
  }
  if (need & kNeedAttn) {
    if (!attn_dims_ok(s->h, s->d_qk, s->d_v))
      return fail(DSA_ERR_UNSUPPORTED, "attention dims (h=%d, d_qk=%d, d_v=%d) not built",
                  s->h, s->d_qk, s->d_v);
    if (!std::isfinite(s->softmax_scale))
      return fail(DSA_ERR_INVALID_ARG, "softmax_scale is not finite");
    // the gather addresses latent rows with 32-bit byte offsets
    if ((int64_t)s->n_k * s->d_qk * 2 > (int64_t)UINT32_MAX)
      return fail(DSA_ERR_UNSUPPORTED, "latent KV of %d rows exceeds 4 GiB", s->n_k);
  }
  p = Plan();
  if (!(need & kNeedSegs)) return DSA_OK;
  if (s->n_segs < 0) return fail(DSA_ERR_INVALID_ARG, "negative n_segs");
  if (s->n_segs > 0 && !s->segs) return fail(DSA_ERR_INVALID_ARG, "segs is NULL");
  std::vector<std::pair<int64_t, int64_t>> spans;
  for (int i = 0; i < s->n_segs; ++i) {
    const dsa_segment& g = s->segs[i];
    if (g.q_start < 0 || g.q_len < 0 || g.k_start < 0 || g.k_len < 0 || g.pos0 < 0)
      return fail(DSA_ERR_INVALID_ARG, "segment %d has a negative field", i);
    if ((int64_t)g.q_start + g.q_len > s->n_q)
      return fail(DSA_ERR_INVALID_ARG, "segment %d: query rows past n_q", i);
    if ((int64_t)g.k_start + g.k_len > s->n_k)
      return fail(DSA_ERR_INVALID_ARG, "segment %d: key rows past n_k", i);
    if (g.q_len == 0) continue;
    if ((int64_t)g.pos0 + g.q_len > g.k_len)
      return fail(DSA_ERR_INVALID_ARG,
                  "segment %d: last position %lld is beyond its %d keys", i,
                  (long long)g.pos0 + g.q_len - 1, g.k_len);
    const int64_t w = (int64_t)g.pos0 + g.q_len;
    if (w > kMaxWindow)
      return fail(DSA_ERR_UNSUPPORTED, "segment %d: window of %lld keys > %lld", i,
                  (long long)w, (long long)kMaxWindow);
    p.max_window = std::max(p.max_window, w);
    p.covered_rows += g.q_len;
    spans.push_back({g.q_start, (int64_t)g.q_start + g.q_len});
    p.segs.push_back(g);
  }
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].first < spans[i - 1].second)
      return fail(DSA_ERR_INVALID_ARG, "segments overlap in query rows");
  std::stable_sort(p.segs.begin(), p.segs.end(), [](const dsa_segment& a, const dsa_segment& b) {
    return (int64_t)a.pos0 + a.q_len > (int64_t)b.pos0 + b.q_len;
  });
  return DSA_OK;
}

// Split the plan into launch-sized tables; rows_per_block rows of a segment share a block.
std::vector<dsa::SegTable> make_tables(const Plan& p, int rows_per_block) {
  std::vector<dsa::SegTable> out;
  for (size_t i = 0; i < p.segs.size(); i += dsa::kMaxSegs) {
    dsa::SegTable t = {};
    const size_t n = std::min(p.segs.size() - i, (size_t)dsa::kMaxSegs);
    t.n = (int)n;
    int blk = 0;
    for (size_t j = 0; j < n; ++j) {
      const dsa_segment& g = p.segs[i + j];
      t.q_start[j] = g.q_start;
      t.q_len[j] = g.q_len;
      t.k_start[j] = g.k_start;
      t.pos0[j] = g.pos0;
      t.blk_off[j] = blk;
      blk += (g.q_len + rows_per_block - 1) / rows_per_block;
    }
    t.blk_off[n] = blk;
    out.push_back(t);
  }
  return out;
}

// Forward workspace: the candidate count of every row, the indices (used when the caller
// does not keep them), then for every row `cap` candidate slots: fp32 scores, and in a second
// region their keys as 16-bit window offsets.  The expected number of candidates a row's
// running bound lets through is about topk (1 + ln(window / topk)); the default gives a row
// 4.5 topk slots (at most the longest window rounded up to 64), enough for windows to about
// 30 topk without a compaction; a smaller workspace gives fewer slots, down to topk + 192
// (the indexer's room check between stages keeps 192 free), and rows compact more often.
constexpr int64_t kCandRoom = 192;
int64_t round64(int64_t x) { return (x + 63) / 64 * 64; }
int64_t cand_cap_max(const dsa_shape* s, const Plan& p) {
  const int64_t k = s->topk;
  return std::min(round64(p.max_window), std::max(round64(k) + kCandRoom, round64((9 * k + 1) / 2)));
}
int64_t cand_cap_min(const dsa_shape* s, const Plan& p) {
  return std::min(round64(p.max_window), round64(s->topk) + kCandRoom);
}

struct WsLayout {
  size_t ccnt_off = 0, idx_off = 0, scores_off = 0, ckey_off = 0, total = 0;
  int64_t cap = 0;
};

WsLayout ws_layout_cap(const dsa_shape* s, int64_t cap) {
  WsLayout w;
  const size_t n = (size_t)s->n_q;
  w.cap = cap;
  w.ccnt_off = 0;
  w.idx_off = align_up(n * sizeof(int32_t));
  w.scores_off = w.idx_off + align_up(n * (size_t)s->topk * sizeof(int32_t));
  w.ckey_off = w.scores_off + align_up(n * (size_t)cap * sizeof(float));
  w.total = w.ckey_off + align_up(n * (size_t)cap * sizeof(uint16_t));
  return w;
}

WsLayout ws_layout(const dsa_shape* s, const Plan& p) { return ws_layout_cap(s, cand_cap_max(s, p)); }

// The layout with the most candidate slots per row that `bytes` holds (cap 0: not even
// cap_min fits).
WsLayout ws_layout_for(const dsa_shape* s, const Plan& p, size_t bytes) {
  const int64_t hi = cand_cap_max(s, p), lo = cand_cap_min(s, p);
  WsLayout w = ws_layout_cap(s, hi);
  if (w.total <= bytes) return w;
  const WsLayout base = ws_layout_cap(s, 0);
  const size_t per = (size_t)s->n_q * (sizeof(float) + sizeof(uint16_t));
  int64_t cap = bytes > base.total && per > 0 ? (int64_t)((bytes - base.total) / per) / 64 * 64 : 0;
  cap = std::min(cap, hi);
  while (cap >= lo && ws_layout_cap(s, cap).total > bytes) cap -= 64;   // region rounding
  if (cap < lo) {
    WsLayout none = ws_layout_cap(s, lo);
    none.cap = 0;
    return none;
  }
  return ws_layout_cap(s, cap);
}

dsa_status run_indexer(const dsa_shape* s, const Plan& p, const void* q_idx,
                       const float* q_scale, const void* k_idx, const float* k_scale,
                       const float* w_idx, float* scores, long long ld, int dense,
                       hipStream_t st, uint16_t* cand_key = nullptr, int* cand_cnt = nullptr) {
  const bool fp8 = s->idx_dtype == DSA_IDX_FP8_E4M3;
  for (const dsa::SegTable& t : make_tables(p, dsa::indexer_rows_per_block())) {
    dsa::IndexerArgs a = {};
    a.segs = t;
    a.q_idx = q_idx;
    a.k_idx = k_idx;
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    a.w_idx = w_idx;
    a.scores = scores;
    a.ld = ld;
    a.dense = dense;
    a.cand_key = cand_key;
    a.cand_cnt = cand_cnt;
    a.topk = s->topk;
    hipError_t e = dsa::launch_indexer(a, s->h_idx, s->d_idx, fp8, st);
    if (e != hipSuccess) return hip_fail(e, "indexer launch");
  }
  return DSA_OK;
}

dsa_status run_topk(const dsa_shape* s, const Plan& p, const float* scores, long long ld,
                    int dense, int32_t* idx, hipStream_t st, const uint16_t* cand_key = nullptr,
                    const int* cand_cnt = nullptr) {
  for (const dsa::SegTable& t : make_tables(p, 1)) {
    dsa::TopkArgs a = {};
    a.segs = t;
    a.scores = scores;
    a.ld = ld;
    a.dense = dense;
    a.topk = s->topk;
    a.idx = idx;
    a.cand_key = cand_key;
    a.cand_cnt = cand_cnt;
    hipError_t e = dsa::launch_topk(a, (int)p.max_window, st);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
  }
  return DSA_OK;
}

dsa_status run_attn(const dsa_shape* s, const Plan* p, const void* q, const void* kv,
                    const int32_t* idx, void* out, float* smax, float* ssum, hipStream_t st) {
  dsa::AttnArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(kv);
  a.idx = idx;
  a.out = static_cast<uint16_t*>(out);
  a.smax = smax;
  a.ssum = ssum;
  a.n_q = s->n_q;
  a.n_k = s->n_k;
  a.topk = s->topk;
  a.scale_log2 = s->softmax_scale * 1.4426950408889634f;
  if (!p) {
    a.use_segs = 0;
    a.xcd_remap = (s->n_q % 8) == 0;
    hipError_t e = dsa::launch_sparse_attn(a, s->h, s->d_qk, s->d_v, s->n_q, st);
    if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
    return DSA_OK;
  }
  for (const dsa::SegTable& t : make_tables(*p, 1)) {
    a.segs = t;
    a.use_segs = 1;
    const int nb = t.blk_off[t.n];
    a.xcd_remap = (nb % 8) == 0;
    hipError_t e = dsa::launch_sparse_attn(a, s->h, s->d_qk, s->d_v, nb, st);
    if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
  }
  return DSA_OK;
}

dsa_status check_idx_ptrs(const dsa_shape* s, const void* q_idx, const float* q_scale,
                          const void* k_idx, const float* k_scale, const float* w_idx) {
  if (!q_idx || !k_idx || !w_idx) return fail(DSA_ERR_INVALID_ARG, "indexer input is NULL");
  if (s->idx_dtype == DSA_IDX_FP8_E4M3) {
    if (!q_scale || !k_scale) return fail(DSA_ERR_INVALID_ARG, "fp8 indexer needs q_scale and k_scale");
  } else if (q_scale || k_scale) {
    return fail(DSA_ERR_INVALID_ARG, "q_scale / k_scale must be NULL for bf16 indexer inputs");
  }
  return DSA_OK;
}

// Backward workspace.  Per call: per-key counters, offsets and cursors (3 n_k + 1 ints).  Per
// row of a chunk: bf16 P and softmax_scale * dS for every (slot, head) and the bf16 dKV
// contribution of every slot, with the slots padded to a multiple of 96 (the tile rings
// process tiles in threes), and one list entry per slot.
size_t bwd_topkp(const dsa_shape* s) { return ((size_t)s->topk + 95) / 96 * 96; }
size_t bwd_row_bytes(const dsa_shape* s) {
  return 2 * bwd_topkp(s) * (size_t)s->h * 2 + bwd_topkp(s) * s->d_qk * 2 + (size_t)s->topk * 4;
}
size_t bwd_fixed_bytes(const dsa_shape* s) {
  return align_up(((size_t)3 * s->n_k + 1) * 4) + 8 * kAlign;   // + slack for region alignment
}
constexpr int kBwdChunkRows = 2048;

dsa_status check_bwd_dims(const dsa_shape* s) {
  if (!(s->h == 128 && s->d_qk == 576 && s->d_v == 512))
    return fail(DSA_ERR_UNSUPPORTED, "attention backward built for (h, d_qk, d_v) = "
                "(128, 576, 512) only (got %d, %d, %d)", s->h, s->d_qk, s->d_v);
  return DSA_OK;
}

// The fused indexer + top-k: candidate scores, keys and counts in the workspace, then the
// selection over each row's candidates.
dsa_status run_indexer_topk(const dsa_shape* s, const Plan& p, const void* q_idx,
                            const float* q_scale, const void* k_idx, const float* k_scale,
                            const float* w_idx, char* ws, const WsLayout& w, int32_t* idx,
                            hipStream_t st) {
  float* scores = reinterpret_cast<float*>(ws + w.scores_off);
  uint16_t* ckey = reinterpret_cast<uint16_t*>(ws + w.ckey_off);
  int* ccnt = reinterpret_cast<int*>(ws + w.ccnt_off);
  const long long ld = w.cap;
  dsa_status e = run_indexer(s, p, q_idx, q_scale, k_idx, k_scale, w_idx, scores, ld, 0, st,
                             ckey, ccnt);
  if (e != DSA_OK) return e;
  return run_topk(s, p, scores, ld, 0, idx, st, ckey, ccnt);
}

// Indexer-loss workspace.  Per call: the per-key counters (as for the attention backward).
// Per row of a chunk: the bf16 index-key gradient and the fp32 dI of every slot (slots padded
// to a multiple of 96; the dI array has 1 KB of slack for whole-piece LDS DMA reads) and one
// list entry per slot.
constexpr int kKlMaxTopk = 2048;   // the per-row target / indexer arrays live in LDS
size_t kl_topkp(const dsa_shape* s) { return ((size_t)s->topk + 95) / 96 * 96; }
size_t kl_row_bytes(const dsa_shape* s) {
  return kl_topkp(s) * (128 * 2 + 4) + (size_t)s->topk * 4;
}
size_t kl_fixed_bytes(const dsa_shape* s) {
  return align_up(((size_t)3 * s->n_k + 1) * 4) + 1024 + 8 * kAlign;
}

dsa_status check_kl_dims(const dsa_shape* s) {
  if (s->idx_dtype != DSA_IDX_BF16)
    return fail(DSA_ERR_UNSUPPORTED, "indexer loss is built for bf16 index tensors only");
  if (!(s->h_idx == 64 && s->d_idx == 128 && s->h == 128 && s->d_qk == 576))
    return fail(DSA_ERR_UNSUPPORTED, "indexer loss built for (h_idx, d_idx, h, d_qk) = "
                "(64, 128, 128, 576) only (got %d, %d, %d, %d)", s->h_idx, s->d_idx, s->h, s->d_qk);
  if (s->topk < 1 || s->topk > kKlMaxTopk)
    return fail(s->topk < 1 ? DSA_ERR_INVALID_ARG : DSA_ERR_UNSUPPORTED,
                "indexer loss needs 1 <= topk <= %d (got %d)", kKlMaxTopk, s->topk);
  if (!std::isfinite(s->softmax_scale))
    return fail(DSA_ERR_INVALID_ARG, "softmax_scale is not finite");
  if ((int64_t)s->n_k * s->d_qk * 2 > (int64_t)UINT32_MAX)
    return fail(DSA_ERR_UNSUPPORTED, "latent KV of %d rows exceeds 4 GiB", s->n_k);
  return DSA_OK;
}

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// Pointer alignment the kernels' vector loads and stores need: {pointer, bytes, name}; NULL
// pointers (optional outputs) pass.
struct AlignReq {
  const void* p;
  size_t a;
  const char* name;
};

dsa_status check_align(std::initializer_list<AlignReq> reqs) {
  for (const AlignReq& r : reqs)
    if (r.p && !aligned(r.p, r.a))
      return fail(DSA_ERR_INVALID_ARG, "%s must be %zu-byte aligned", r.name, r.a);
  return DSA_OK;
}

// Index-side tensors: q_idx / k_idx rows are read in 16-byte pieces.
dsa_status check_idx_align(const void* q_idx, const float* q_scale, const void* k_idx,
                           const float* k_scale, const float* w_idx) {
  return check_align({{q_idx, 16, "q_idx"}, {k_idx, 16, "k_idx"}, {w_idx, 4, "w_idx"},
                      {q_scale, 4, "q_scale"}, {k_scale, 4, "k_scale"}});
}

// Attention-side tensors: q and kv rows are gathered / staged in 16-byte pieces and output
// rows leave in 16-byte pieces.
dsa_status check_attn_align(const void* q, const void* kv, const int32_t* idx, const void* out,
                            const float* smax, const float* ssum) {
  return check_align({{q, 16, "q"}, {kv, 16, "kv"}, {idx, 4, "topk_idx"}, {out, 16, "out"},
                      {smax, 4, "softmax_max"}, {ssum, 4, "softmax_sum"}});
}

// ---- the allocation-free forward ---------------------------------------------------------
// For callers that cannot allocate device memory: the forward's workspace is this fixed array
// (each GPU the library runs on holds its own copy until the process ends).  Host code never
// passes the array's name to a kernel or copy (in host code it is a stand-in, not a device
// address): the device address comes from hipGetSymbolAddress, looked up once per device.
constexpr size_t kNoallocScratchBytes = (size_t)DSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the current device (the stream's device must be the
// current one).
dsa_status scratch_address(hipStream_t st, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (st) {
    hipDevice_t sd = -1;
    e = hipStreamGetDevice(st, &sd);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    if (sd != dev)
      return fail(DSA_ERR_INVALID_ARG, "the stream belongs to device %d, device %d is current",
                  (int)sd, dev);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DSA_ERR_UNSUPPORTED, "device %d beyond the %d this library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

// The segments of local rows [r0, r1), renumbered from r0 (empty pieces dropped).
std::vector<dsa_segment> clip_segments(const Plan& p, int r0, int r1) {
  std::vector<dsa_segment> out;
  for (const dsa_segment& g : p.segs) {
    const int a = std::max(g.q_start, r0), b = std::min(g.q_start + g.q_len, r1);
    if (a >= b) continue;
    dsa_segment c = g;
    c.q_start = a - r0;
    c.q_len = b - a;
    c.pos0 = g.pos0 + (a - g.q_start);
    out.push_back(c);
  }
  return out;
}

}  // namespace

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_last_error(void) { return g_err.c_str(); }

dsa_status dsa_workspace_bytes(const dsa_shape* shape, size_t* bytes) {
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is NULL");
  Plan p;
  dsa_status st = check_shape(shape, kNeedSegs | kNeedTopk, p);
  if (st != DSA_OK) return st;
  *bytes = ws_layout(shape, p).total;
  return ok();
}

dsa_status dsa_indexer_scores(const dsa_shape* shape, const void* q_idx, const float* q_scale,
                              const void* k_idx, const float* k_scale, const float* w_idx,
                              float* scores, void* stream) {
  Plan p;
  dsa_status st = check_shape(shape, kNeedSegs | kNeedIndexer, p);
  if (st != DSA_OK) return st;
  if (p.covered_rows == 0) return ok();
  if ((st = check_idx_ptrs(shape, q_idx, q_scale, k_idx, k_scale, w_idx)) != DSA_OK) return st;
  if (!scores) return fail(DSA_ERR_INVALID_ARG, "scores is NULL");
  if ((st = check_idx_align(q_idx, q_scale, k_idx, k_scale, w_idx)) != DSA_OK) return st;
  if ((st = check_align({{scores, 4, "scores"}})) != DSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  for (const dsa::SegTable& t : make_tables(p, 1)) {
    dsa::FillArgs f = {};
    f.segs = t;
    f.scores = scores;
    f.ld = shape->n_k;
    f.n_k = shape->n_k;
    hipError_t e = dsa::launch_fill_outside(f, hs);
    if (e != hipSuccess) return hip_fail(e, "fill launch");
  }
  st = run_indexer(shape, p, q_idx, q_scale, k_idx, k_scale, w_idx, scores, shape->n_k, 1, hs);
  return st == DSA_OK ? ok() : st;
}

dsa_status dsa_topk_select(const dsa_shape* shape, const float* scores, int32_t* topk_idx,
                           void* stream) {
  Plan p;
  dsa_status st = check_shape(shape, kNeedSegs | kNeedTopk, p);
  if (st != DSA_OK) return st;
  if (p.covered_rows == 0) return ok();
  if (!scores || !topk_idx) return fail(DSA_ERR_INVALID_ARG, "scores or topk_idx is NULL");
  if ((st = check_align({{scores, 4, "scores"}, {topk_idx, 4, "topk_idx"}})) != DSA_OK) return st;
  st = run_topk(shape, p, scores, shape->n_k, 1, topk_idx, static_cast<hipStream_t>(stream));
  return st == DSA_OK ? ok() : st;
}

dsa_status dsa_sparse_attn(const dsa_shape* shape, const void* q, const void* kv,
                           const int32_t* topk_idx, void* out, float* softmax_max,
                           float* softmax_sum, void* stream) {
  Plan p;
  dsa_status st = check_shape(shape, kNeedAttn, p);
  if (st != DSA_OK) return st;
  if (shape->n_q == 0) return ok();
  if (!q || !kv || !topk_idx || !out) return fail(DSA_ERR_INVALID_ARG, "attention tensor is NULL");
  if ((st = check_attn_align(q, kv, topk_idx, out, softmax_max, softmax_sum)) != DSA_OK) return st;
  st = run_attn(shape, nullptr, q, kv, topk_idx, out, softmax_max, softmax_sum,
                static_cast<hipStream_t>(stream));
  return st == DSA_OK ? ok() : st;
}

dsa_status dsa_dense_attn(const dsa_shape* shape, const void* q, const void* k, const void* v,
                          void* out, float* lse, void* stream) {
  Plan p;
  dsa_status st = check_shape(shape, kNeedSegs, p);
  if (st != DSA_OK) return st;
  if (shape->h < 1) return fail(DSA_ERR_INVALID_ARG, "h must be >= 1 (got %d)", shape->h);
  if (shape->d_qk != 192 || shape->d_v != 128)
    return fail(DSA_ERR_UNSUPPORTED, "dense attention dims (d_qk=%d, d_v=%d) not built",
                shape->d_qk, shape->d_v);
  if (!std::isfinite(shape->softmax_scale) || !(shape->softmax_scale > 0.f))
    return fail(DSA_ERR_INVALID_ARG, "softmax_scale must be finite and positive");
  // the tile DMA addresses key rows with 32-bit byte offsets
  if ((int64_t)shape->n_k * shape->h * shape->d_qk * 2 > (int64_t)UINT32_MAX)
    return fail(DSA_ERR_UNSUPPORTED, "K of %d rows x %d heads exceeds 4 GiB", shape->n_k,
                shape->h);
  if (p.covered_rows == 0) return ok();
  if (!q || !k || !v || !out) return fail(DSA_ERR_INVALID_ARG, "dense attention tensor is NULL");
  if ((st = check_align({{q, 16, "q"}, {k, 16, "k"}, {v, 16, "v"}, {out, 16, "out"},
                         {lse, 4, "lse"}})) != DSA_OK)
    return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  for (const dsa::SegTable& t : make_tables(p, dsa::dense_rows_per_block())) {
    dsa::DenseArgs a = {};
    a.segs = t;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.h = shape->h;
    a.scale_log2 = shape->softmax_scale * 1.4426950408889634f;
    hipError_t e = dsa::launch_dense_attn(a, t.blk_off[t.n], hs);
    if (e != hipSuccess) return hip_fail(e, "dense attention launch");
  }
  return ok();
}

dsa_status dsa_forward(const dsa_shape* shape, const void* q_idx, const float* q_scale,
                       const void* k_idx, const float* k_scale, const float* w_idx,
                       const void* q, const void* kv, void* out, int32_t* topk_idx,
                       float* softmax_max, float* softmax_sum, void* workspace,
                       size_t workspace_bytes, void* stream) {
  Plan p;
  dsa_status st = check_shape(shape, kNeedSegs | kNeedIndexer | kNeedTopk | kNeedAttn, p);
  if (st != DSA_OK) return st;
  if (p.covered_rows == 0) return ok();   // nothing to do: no pointer is read
  if ((st = check_idx_ptrs(shape, q_idx, q_scale, k_idx, k_scale, w_idx)) != DSA_OK) return st;
  if (!q || !kv || !out) return fail(DSA_ERR_INVALID_ARG, "attention tensor is NULL");
  if ((st = check_idx_align(q_idx, q_scale, k_idx, k_scale, w_idx)) != DSA_OK) return st;
  if ((st = check_attn_align(q, kv, topk_idx, out, softmax_max, softmax_sum)) != DSA_OK) return st;
  const WsLayout w = ws_layout_for(shape, p, workspace ? workspace_bytes : 0);
  if (!workspace || w.cap == 0)
    return fail(DSA_ERR_WORKSPACE, "workspace of at least %zu bytes needed, %zu given", w.total,
                workspace ? workspace_bytes : (size_t)0);
  if ((st = check_align({{workspace, 16, "workspace"}})) != DSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(ws + w.idx_off);
  if ((st = run_indexer_topk(shape, p, q_idx, q_scale, k_idx, k_scale, w_idx, ws, w, idx, hs)) != DSA_OK)
    return st;
  if ((st = run_attn(shape, &p, q, kv, idx, out, softmax_max, softmax_sum, hs)) != DSA_OK) return st;
  return ok();
}

dsa_status dsa_indexer_topk(const dsa_shape* shape, const void* q_idx, const float* q_scale,
                            const void* k_idx, const float* k_scale, const float* w_idx,
                            int32_t* topk_idx, void* workspace, size_t workspace_bytes,
                            void* stream) {
  Plan p;
  dsa_status st = check_shape(shape, kNeedSegs | kNeedIndexer | kNeedTopk, p);
  if (st != DSA_OK) return st;
  if (p.covered_rows == 0) return ok();
  if ((st = check_idx_ptrs(shape, q_idx, q_scale, k_idx, k_scale, w_idx)) != DSA_OK) return st;
  if (!topk_idx) return fail(DSA_ERR_INVALID_ARG, "topk_idx is NULL");
  if ((st = check_idx_align(q_idx, q_scale, k_idx, k_scale, w_idx)) != DSA_OK) return st;
  if ((st = check_align({{topk_idx, 4, "topk_idx"}})) != DSA_OK) return st;
  const WsLayout w = ws_layout_for(shape, p, workspace ? workspace_bytes : 0);
  if (!workspace || w.cap == 0)
    return fail(DSA_ERR_WORKSPACE, "workspace of at least %zu bytes needed, %zu given", w.total,
                workspace ? workspace_bytes : (size_t)0);
  if ((st = check_align({{workspace, 16, "workspace"}})) != DSA_OK) return st;
  st = run_indexer_topk(shape, p, q_idx, q_scale, k_idx, k_scale, w_idx,
                        static_cast<char*>(workspace), w, topk_idx,
                        static_cast<hipStream_t>(stream));
  return st == DSA_OK ? ok() : st;
}

dsa_status dsa_quantize_fp8_rows(const void* x_bf16, int64_t rows, int32_t cols, void* x_fp8,
                                 float* scale, void* stream) {
  if (rows < 0 || cols < 0) return fail(DSA_ERR_INVALID_ARG, "negative rows or cols");
  if (rows > 0x7fffffff) return fail(DSA_ERR_UNSUPPORTED, "more than 2^31-1 rows");
  if (rows == 0) return ok();
  if (!x_bf16 || !x_fp8 || !scale) return fail(DSA_ERR_INVALID_ARG, "quantize tensor is NULL");
  dsa_status st = check_align({{x_bf16, 2, "x_bf16"}, {scale, 4, "scale"}});
  if (st != DSA_OK) return st;
  dsa::QuantArgs a = {};
  a.x = static_cast<const uint16_t*>(x_bf16);
  a.y = static_cast<uint8_t*>(x_fp8);
  a.scale = scale;
  a.rows = rows;
  a.cols = cols;
  hipError_t e = dsa::launch_quant_fp8_rows(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quantize launch");
  return ok();
}

dsa_status dsa_sparse_attn_bwd_workspace_bytes(const dsa_shape* shape, size_t* bytes) {
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is NULL");
  Plan p;
  dsa_status st = check_shape(shape, kNeedAttn, p);
  if (st != DSA_OK) return st;
  if ((st = check_bwd_dims(shape)) != DSA_OK) return st;
  *bytes = bwd_fixed_bytes(shape) + bwd_row_bytes(shape) * (size_t)std::min(shape->n_q, kBwdChunkRows);
  return ok();
}

// ---- attention backward and indexer loss: validation, argument set-up and the chunk loops

namespace {

dsa_status bwd_validate(const dsa_shape* shape, const void* q, const void* kv,
                        const int32_t* topk_idx, const void* out, const void* dout,
                        const float* softmax_max, const float* softmax_sum, const void* dq,
                        const float* dkv, const void* workspace) {
  if (!q || !kv || !topk_idx || !out || !dout || !softmax_max || !softmax_sum || !dq || !dkv)
    return fail(DSA_ERR_INVALID_ARG, "attention backward tensor is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0 || reinterpret_cast<uintptr_t>(dkv) % 16 != 0)
    return fail(DSA_ERR_INVALID_ARG, "workspace and dkv must be 16-byte aligned");
  dsa_status st = check_attn_align(q, kv, topk_idx, out, softmax_max, softmax_sum);
  if (st != DSA_OK) return st;
  (void)shape;
  return check_align({{dout, 16, "dout"}, {dq, 16, "dq"}});
}

dsa_status kl_validate(const void* q_idx, const void* k_idx, const float* w_idx, const void* q,
                       const void* kv, const int32_t* topk_idx, const float* softmax_max,
                       const float* softmax_sum, const float* loss_rows, const void* dq_idx,
                       const float* dw_idx, const float* dk_idx, const void* workspace) {
  if (!q_idx || !k_idx || !w_idx || !q || !kv || !topk_idx || !softmax_max || !softmax_sum ||
      !loss_rows || !dq_idx || !dw_idx || !dk_idx)
    return fail(DSA_ERR_INVALID_ARG, "indexer loss tensor is NULL");
  if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(w_idx, 16) || !aligned(q, 16) ||
      !aligned(kv, 16) || !aligned(softmax_max, 16) || !aligned(softmax_sum, 16) ||
      !aligned(dk_idx, 16) || !aligned(workspace, 16) || !aligned(dq_idx, 8) ||
      !aligned(topk_idx, 4) || !aligned(loss_rows, 4) || !aligned(dw_idx, 4))
    return fail(DSA_ERR_INVALID_ARG, "indexer loss tensors, dk_idx and workspace must be "
                "16-byte aligned (dq_idx 8-byte)");
  return DSA_OK;
}

// Rows per chunk that `workspace_bytes` holds at `per_row` bytes a row over `fixed`; 0 (with
// the error set) if not even one.  List entries are row * topkp + slot within a chunk: the
// chunk keeps them below 2^31.
int chunk_rows(const dsa_shape* shape, const void* workspace, size_t workspace_bytes,
               size_t fixed, size_t per_row, size_t topkp) {
  const size_t fit = workspace && workspace_bytes > fixed ? (workspace_bytes - fixed) / per_row : 0;
  if (fit == 0) {
    fail(DSA_ERR_WORKSPACE, "workspace of at least %zu bytes (one row) needed, %zu given",
         fixed + per_row, workspace ? workspace_bytes : (size_t)0);
    return 0;
  }
  const size_t max_rows = (size_t)INT32_MAX / topkp;
  return (int)std::min({fit, (size_t)shape->n_q, max_rows});
}

// Bump allocator over the workspace (regions 256-byte aligned).
struct WsTake {
  char* w;
  size_t at = 0;
  char* operator()(size_t bytes) {
    char* p = w + at;
    at = align_up(at + bytes);
    return p;
  }
};

// The call-wide fields of the attention backward's arguments.
dsa::AttnBwdArgs bwd_args(const dsa_shape* shape, const void* kv, float* dkv, size_t topkp) {
  dsa::AttnBwdArgs a = {};
  a.kv = static_cast<const uint16_t*>(kv);
  a.dkv = dkv;
  a.n_k = shape->n_k;
  a.topk = shape->topk;
  a.topkp = (int)topkp;
  a.scale = shape->softmax_scale;
  a.scale_log2 = shape->softmax_scale * 1.4426950408889634f;
  return a;
}

// The chunk [r0, r0 + rows) of the attention backward.
void bwd_chunk(dsa::AttnBwdArgs& a, const dsa_shape* shape, int r0, int rows, const void* q,
               const int32_t* topk_idx, const void* out, const void* dout,
               const float* softmax_max, const float* softmax_sum, void* dq) {
  const int h = shape->h, dqk = shape->d_qk, dv = shape->d_v, topk = shape->topk;
  a.rows = rows;
  a.q = static_cast<const uint16_t*>(q) + (size_t)r0 * h * dqk;
  a.idx = topk_idx + (size_t)r0 * topk;
  a.out = static_cast<const uint16_t*>(out) + (size_t)r0 * h * dv;
  a.dout = static_cast<const uint16_t*>(dout) + (size_t)r0 * h * dv;
  a.smax = softmax_max + (size_t)r0 * h;
  a.ssum = softmax_sum + (size_t)r0 * h;
  a.dq = static_cast<uint16_t*>(dq) + (size_t)r0 * h * dqk;
  a.xcd_remap = rows % 8 == 0;
}

// The call-wide fields of the indexer loss's arguments.
dsa::IdxKlArgs kl_args(const dsa_shape* shape, const void* k_idx, const void* kv, float* dk_idx,
                       float loss_grad, size_t topkp) {
  dsa::IdxKlArgs a = {};
  a.k_idx = static_cast<const uint16_t*>(k_idx);
  a.kv = static_cast<const uint16_t*>(kv);
  a.dk = dk_idx;
  a.n_k = shape->n_k;
  a.topk = shape->topk;
  a.topkp = (int)topkp;
  a.scale_log2 = shape->softmax_scale * 1.4426950408889634f;
  a.loss_grad = loss_grad;
  return a;
}

// The chunk [r0, r0 + rows) of the indexer loss.
void kl_chunk(dsa::IdxKlArgs& a, const dsa_shape* shape, int r0, int rows, const void* q_idx,
              const float* w_idx, const void* q, const int32_t* topk_idx,
              const float* softmax_max, const float* softmax_sum, float* loss_rows, void* dq_idx,
              float* dw_idx) {
  const int topk = shape->topk;
  a.rows = rows;
  a.q_idx = static_cast<const uint16_t*>(q_idx) + (size_t)r0 * 64 * 128;
  a.w = w_idx + (size_t)r0 * 64;
  a.q = static_cast<const uint16_t*>(q) + (size_t)r0 * 128 * 576;
  a.idx = topk_idx + (size_t)r0 * topk;
  a.smax = softmax_max + (size_t)r0 * 128;
  a.ssum = softmax_sum + (size_t)r0 * 128;
  a.loss = loss_rows + r0;
  a.dq_idx = static_cast<uint16_t*>(dq_idx) + (size_t)r0 * 64 * 128;
  a.dw = dw_idx + (size_t)r0 * 64;
  a.xcd_remap = rows % 8 == 0;
}

// Combined backward workspace per row: the attention backward's, plus the fp32 per-slot head
// sums of P handed to the indexer loss (whose per-slot arrays reuse the attention backward's
// regions once they are consumed, and whose key lists are the attention backward's).
size_t bwdkl_row_bytes(const dsa_shape* s) { return bwd_row_bytes(s) + bwd_topkp(s) * 4; }

}  // namespace

dsa_status dsa_sparse_attn_bwd(const dsa_shape* shape, const void* q, const void* kv,
                               const int32_t* topk_idx, const void* out, const void* dout,
                               const float* softmax_max, const float* softmax_sum, void* dq,
                               float* dkv, void* workspace, size_t workspace_bytes,
                               void* stream) {
  Plan p;
  dsa_status st = check_shape(shape, kNeedAttn, p);
  if (st != DSA_OK) return st;
  if ((st = check_bwd_dims(shape)) != DSA_OK) return st;
  if (shape->n_q == 0) return ok();
  if ((st = bwd_validate(shape, q, kv, topk_idx, out, dout, softmax_max, softmax_sum, dq, dkv,
                         workspace)) != DSA_OK)
    return st;
  const size_t topkp = bwd_topkp(shape);
  const int chunk = chunk_rows(shape, workspace, workspace_bytes, bwd_fixed_bytes(shape),
                               bwd_row_bytes(shape), topkp);
  if (chunk == 0) return DSA_ERR_WORKSPACE;
  const int h = shape->h, dqk = shape->d_qk, dv = shape->d_v, topk = shape->topk;
  WsTake take{static_cast<char*>(workspace)};
  dsa::AttnBwdArgs a = bwd_args(shape, kv, dkv, topkp);
  a.cnt = reinterpret_cast<int*>(take((size_t)shape->n_k * 4));
  a.off = reinterpret_cast<int*>(take(((size_t)shape->n_k + 1) * 4));
  a.cur = reinterpret_cast<int*>(take((size_t)shape->n_k * 4));
  a.ws_p = reinterpret_cast<uint16_t*>(take((size_t)chunk * topkp * h * 2));
  a.ws_ds = reinterpret_cast<uint16_t*>(take((size_t)chunk * topkp * h * 2));
  a.ws_c = reinterpret_cast<uint16_t*>(take((size_t)chunk * topkp * dqk * 2));
  a.list = reinterpret_cast<int*>(take((size_t)chunk * topk * 4));
  if (take.at > workspace_bytes)
    return fail(DSA_ERR_WORKSPACE, "internal workspace layout exceeds %zu bytes", workspace_bytes);
  for (int r0 = 0; r0 < shape->n_q; r0 += chunk) {
    bwd_chunk(a, shape, r0, std::min(chunk, shape->n_q - r0), q, topk_idx, out, dout,
              softmax_max, softmax_sum, dq);
    hipError_t e = dsa::launch_sparse_attn_bwd(a, h, dqk, dv, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "attention backward launch");
  }
  return ok();
}

dsa_status dsa_indexer_kl_workspace_bytes(const dsa_shape* shape, size_t* bytes) {
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is NULL");
  if (!shape) return fail(DSA_ERR_INVALID_ARG, "shape is NULL");
  if (shape->n_q < 0 || shape->n_k < 0) return fail(DSA_ERR_INVALID_ARG, "negative n_q or n_k");
  dsa_status st = check_kl_dims(shape);
  if (st != DSA_OK) return st;
  *bytes = kl_fixed_bytes(shape) + kl_row_bytes(shape) * (size_t)std::min(shape->n_q, kBwdChunkRows);
  return ok();
}

dsa_status dsa_indexer_kl_loss_grad(const dsa_shape* shape, const void* q_idx, const void* k_idx,
                                    const float* w_idx, const void* q, const void* kv,
                                    const int32_t* topk_idx, const float* softmax_max,
                                    const float* softmax_sum, float loss_grad, float* loss_rows,
                                    float* loss, void* dq_idx, float* dw_idx, float* dk_idx,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape) return fail(DSA_ERR_INVALID_ARG, "shape is NULL");
  if (shape->n_q < 0 || shape->n_k < 0) return fail(DSA_ERR_INVALID_ARG, "negative n_q or n_k");
  dsa_status st = check_kl_dims(shape);
  if (st != DSA_OK) return st;
  if (!std::isfinite(loss_grad)) return fail(DSA_ERR_INVALID_ARG, "loss_grad is not finite");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (shape->n_q == 0) {
    if (loss) {   // an empty sum (a kernel, so the call stays capturable in a graph)
      hipError_t e = dsa::launch_loss_total(loss_rows, 0, loss, hs);
      if (e != hipSuccess) return hip_fail(e, "loss sum launch");
    }
    return ok();
  }
  if ((st = kl_validate(q_idx, k_idx, w_idx, q, kv, topk_idx, softmax_max, softmax_sum,
                        loss_rows, dq_idx, dw_idx, dk_idx, workspace)) != DSA_OK)
    return st;
  const size_t topkp = kl_topkp(shape);
  const int chunk = chunk_rows(shape, workspace, workspace_bytes, kl_fixed_bytes(shape),
                               kl_row_bytes(shape), topkp);
  if (chunk == 0) return DSA_ERR_WORKSPACE;
  const int topk = shape->topk;
  WsTake take{static_cast<char*>(workspace)};
  dsa::KeyListArgs kl = {};
  kl.cnt = reinterpret_cast<int*>(take((size_t)shape->n_k * 4));
  kl.off = reinterpret_cast<int*>(take(((size_t)shape->n_k + 1) * 4));
  kl.cur = reinterpret_cast<int*>(take((size_t)shape->n_k * 4));
  uint16_t* ws_c = reinterpret_cast<uint16_t*>(take((size_t)chunk * topkp * 128 * 2));
  float* ws_di = reinterpret_cast<float*>(take((size_t)chunk * topkp * 4 + 1024));
  kl.list = reinterpret_cast<int*>(take((size_t)chunk * topk * 4));
  if (take.at > workspace_bytes)
    return fail(DSA_ERR_WORKSPACE, "internal workspace layout exceeds %zu bytes", workspace_bytes);
  kl.n_k = shape->n_k;
  kl.topk = topk;
  kl.topkp = (int)topkp;
  dsa::IdxKlArgs a = kl_args(shape, k_idx, kv, dk_idx, loss_grad, topkp);
  a.ws_c = ws_c;
  a.ws_di = ws_di;
  a.list = kl.list;
  a.off = kl.off;
  for (int r0 = 0; r0 < shape->n_q; r0 += chunk) {
    const int rows = std::min(chunk, shape->n_q - r0);
    kl_chunk(a, shape, r0, rows, q_idx, w_idx, q, topk_idx, softmax_max, softmax_sum, loss_rows,
             dq_idx, dw_idx);
    kl.rows = rows;
    kl.idx = a.idx;
    hipError_t e = dsa::launch_indexer_kl(a, kl, hs, true);
    if (e != hipSuccess) return hip_fail(e, "indexer loss launch");
  }
  if (loss) {
    hipError_t e = dsa::launch_loss_total(loss_rows, shape->n_q, loss, hs);
    if (e != hipSuccess) return hip_fail(e, "loss sum launch");
  }
  return ok();
}

dsa_status dsa_sparse_attn_bwd_indexer_kl_workspace_bytes(const dsa_shape* shape, size_t* bytes) {
  if (!bytes) return fail(DSA_ERR_INVALID_ARG, "bytes is NULL");
  Plan p;
  dsa_status st = check_shape(shape, kNeedAttn, p);
  if (st != DSA_OK) return st;
  if ((st = check_bwd_dims(shape)) != DSA_OK) return st;
  if ((st = check_kl_dims(shape)) != DSA_OK) return st;
  *bytes = bwd_fixed_bytes(shape) + bwdkl_row_bytes(shape) * (size_t)std::min(shape->n_q, kBwdChunkRows);
  return ok();
}

dsa_status dsa_sparse_attn_bwd_indexer_kl(
    const dsa_shape* shape, const void* q, const void* kv, const int32_t* topk_idx,
    const void* out, const void* dout, const float* softmax_max, const float* softmax_sum,
    void* dq, float* dkv, const void* q_idx, const void* k_idx, const float* w_idx,
    float loss_grad, float* loss_rows, float* loss, void* dq_idx, float* dw_idx, float* dk_idx,
    void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  dsa_status st = check_shape(shape, kNeedAttn, p);
  if (st != DSA_OK) return st;
  if ((st = check_bwd_dims(shape)) != DSA_OK) return st;
  if ((st = check_kl_dims(shape)) != DSA_OK) return st;
  if (!std::isfinite(loss_grad)) return fail(DSA_ERR_INVALID_ARG, "loss_grad is not finite");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (shape->n_q == 0) {
    if (loss) {
      hipError_t e = dsa::launch_loss_total(loss_rows, 0, loss, hs);
      if (e != hipSuccess) return hip_fail(e, "loss sum launch");
    }
    return ok();
  }
  if ((st = bwd_validate(shape, q, kv, topk_idx, out, dout, softmax_max, softmax_sum, dq, dkv,
                         workspace)) != DSA_OK)
    return st;
  if ((st = kl_validate(q_idx, k_idx, w_idx, q, kv, topk_idx, softmax_max, softmax_sum,
                        loss_rows, dq_idx, dw_idx, dk_idx, workspace)) != DSA_OK)
    return st;
  const size_t topkp = bwd_topkp(shape);
  const int chunk = chunk_rows(shape, workspace, workspace_bytes, bwd_fixed_bytes(shape),
                               bwdkl_row_bytes(shape), topkp);
  if (chunk == 0) return DSA_ERR_WORKSPACE;
  const int h = shape->h, dqk = shape->d_qk, dv = shape->d_v, topk = shape->topk;
  WsTake take{static_cast<char*>(workspace)};
  dsa::AttnBwdArgs a = bwd_args(shape, kv, dkv, topkp);
  a.cnt = reinterpret_cast<int*>(take((size_t)shape->n_k * 4));
  a.off = reinterpret_cast<int*>(take(((size_t)shape->n_k + 1) * 4));
  a.cur = reinterpret_cast<int*>(take((size_t)shape->n_k * 4));
  a.ws_p = reinterpret_cast<uint16_t*>(take((size_t)chunk * topkp * h * 2));
  a.ws_ds = reinterpret_cast<uint16_t*>(take((size_t)chunk * topkp * h * 2));
  a.ws_c = reinterpret_cast<uint16_t*>(take((size_t)chunk * topkp * dqk * 2));
  a.list = reinterpret_cast<int*>(take((size_t)chunk * topk * 4));
  a.psum = reinterpret_cast<float*>(take((size_t)chunk * topkp * 4));
  if (take.at > workspace_bytes)
    return fail(DSA_ERR_WORKSPACE, "internal workspace layout exceeds %zu bytes", workspace_bytes);
  dsa::IdxKlArgs b = kl_args(shape, k_idx, kv, dk_idx, loss_grad, topkp);
  // per slot of the chunk: the key gradient over the attention backward's contributions and
  // dI over its probabilities, both read by then (stream order)
  b.ws_c = a.ws_c;
  b.ws_di = reinterpret_cast<float*>(a.ws_p);
  static_assert(128 * 2 <= 576 * 2, "key gradients fit the contribution region");
  b.list = a.list;
  b.off = a.off;
  b.psum = a.psum;
  const dsa::KeyListArgs none = {};
  for (int r0 = 0; r0 < shape->n_q; r0 += chunk) {
    const int rows = std::min(chunk, shape->n_q - r0);
    bwd_chunk(a, shape, r0, rows, q, topk_idx, out, dout, softmax_max, softmax_sum, dq);
    hipError_t e = dsa::launch_sparse_attn_bwd(a, h, dqk, dv, hs);
    if (e != hipSuccess) return hip_fail(e, "attention backward launch");
    kl_chunk(b, shape, r0, rows, q_idx, w_idx, q, topk_idx, softmax_max, softmax_sum, loss_rows,
             dq_idx, dw_idx);
    e = dsa::launch_indexer_kl(b, none, hs, false);
    if (e != hipSuccess) return hip_fail(e, "indexer loss launch");
  }
  if (loss) {
    hipError_t e = dsa::launch_loss_total(loss_rows, shape->n_q, loss, hs);
    if (e != hipSuccess) return hip_fail(e, "loss sum launch");
  }
  return ok();
}

dsa_status dsa_forward_noalloc(const dsa_shape* shape, const void* q_idx, const float* q_scale,
                               const void* k_idx, const float* k_scale, const float* w_idx,
                               const void* q, const void* kv, void* out, int32_t* topk_idx,
                               float* softmax_max, float* softmax_sum, void* stream) {
  Plan p;
  dsa_status st = check_shape(shape, kNeedSegs | kNeedIndexer | kNeedTopk | kNeedAttn, p);
  if (st != DSA_OK) return st;
  if (p.covered_rows == 0) return ok();
  if ((st = check_idx_ptrs(shape, q_idx, q_scale, k_idx, k_scale, w_idx)) != DSA_OK) return st;
  if (!q || !kv || !out) return fail(DSA_ERR_INVALID_ARG, "attention tensor is NULL");
  if ((st = check_idx_align(q_idx, q_scale, k_idx, k_scale, w_idx)) != DSA_OK) return st;
  if ((st = check_attn_align(q, kv, topk_idx, out, softmax_max, softmax_sum)) != DSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  void* base = nullptr;
  if ((st = scratch_address(hs, &base)) != DSA_OK) return st;
  // rows per pass: as many as the scratch holds with the default candidate slots of the
  // whole share (a pass's own windows are no longer)
  const int64_t cap = cand_cap_max(shape, p);
  dsa_shape one = *shape;
  one.n_q = 1;
  const size_t per_row = ws_layout_cap(&one, cap).total;
  int64_t rows = (int64_t)(kNoallocScratchBytes / per_row);
  dsa_shape sub = *shape;
  for (; rows > 1; --rows) {   // region rounding: at most a few steps
    sub.n_q = (int32_t)std::min<int64_t>(rows, shape->n_q);
    if (ws_layout_cap(&sub, cap).total <= kNoallocScratchBytes) break;
  }
  rows = std::max<int64_t>(1, std::min<int64_t>(rows, shape->n_q));
  for (int64_t r0 = 0; r0 < shape->n_q; r0 += rows) {
    const int r1 = (int)std::min<int64_t>(r0 + rows, shape->n_q);
    std::vector<dsa_segment> segs = clip_segments(p, (int)r0, r1);
    if (segs.empty()) continue;
    sub = *shape;
    sub.n_q = r1 - (int)r0;
    sub.segs = segs.data();
    sub.n_segs = (int32_t)segs.size();
    Plan sp;
    if ((st = check_shape(&sub, kNeedSegs | kNeedIndexer | kNeedTopk | kNeedAttn, sp)) != DSA_OK)
      return st;
    const WsLayout w = ws_layout_for(&sub, sp, kNoallocScratchBytes);
    if (w.cap == 0)
      return fail(DSA_ERR_UNSUPPORTED, "one row's workspace (%zu bytes) exceeds the %zu-byte "
                  "scratch of the allocation-free forward", w.total, kNoallocScratchBytes);
    char* ws = static_cast<char*>(base);
    const size_t qi_row = (size_t)shape->h_idx * shape->d_idx *
                          (shape->idx_dtype == DSA_IDX_FP8_E4M3 ? 1 : 2);
    const char* qi = static_cast<const char*>(q_idx) + (size_t)r0 * qi_row;
    const float* qs = q_scale ? q_scale + r0 : nullptr;
    const float* wi = w_idx + (size_t)r0 * shape->h_idx;
    const char* qq = static_cast<const char*>(q) + (size_t)r0 * shape->h * shape->d_qk * 2;
    char* oo = static_cast<char*>(out) + (size_t)r0 * shape->h * shape->d_v * 2;
    int32_t* idx = topk_idx ? topk_idx + (size_t)r0 * shape->topk
                            : reinterpret_cast<int32_t*>(ws + w.idx_off);
    float* sm = softmax_max ? softmax_max + (size_t)r0 * shape->h : nullptr;
    float* ss = softmax_sum ? softmax_sum + (size_t)r0 * shape->h : nullptr;
    if ((st = run_indexer_topk(&sub, sp, qi, qs, k_idx, k_scale, wi, ws, w, idx, hs)) != DSA_OK)
      return st;
    if ((st = run_attn(&sub, &sp, qq, kv, idx, oo, sm, ss, hs)) != DSA_OK) return st;
  }
  return ok();
}

}  // extern "C"
