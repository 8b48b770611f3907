// Device-side building blocks shared by the gfx950 kernels of libdsa: bf16 / MFMA vector
// types, the launch-argument structs (segment tables are passed by value in kernel
// arguments, so no device metadata buffer is needed) and small wave/block primitives.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

// Segments handed to one launch.  A launch covers at most kMaxSegs segments; the host splits
// larger tables over several launches.
constexpr int kMaxSegs = 64;

struct SegTable {
  int n;                       // segments in this launch
  int q_start[kMaxSegs];
  int q_len[kMaxSegs];
  int k_start[kMaxSegs];
  int pos0[kMaxSegs];
  int blk_off[kMaxSegs + 1];   // first block of each segment; blk_off[n] = grid size
};

// Find the segment owning block `blk` (linear scan: at most kMaxSegs entries).
__device__ __forceinline__ int seg_of_block(const SegTable& t, int blk) {
  int g = 0;
  while (g + 1 < t.n && blk >= t.blk_off[g + 1]) ++g;
  return g;
}

struct IndexerArgs {
  SegTable segs;
  const void* q_idx;      // [n_q, h_idx, d_idx] bf16 or e4m3fn codes
  const void* k_idx;      // [n_k, d_idx]
  const float* q_scale;   // fp8 only
  const float* k_scale;   // fp8 only
  const float* w_idx;     // [n_q, h_idx]
  float* scores;          // row i at scores + i * ld (+ k_start when dense)
  long long ld;           // row stride of scores in elements
  int dense;              // 1: column = absolute key row; 0: column = key - k_start
  // candidate mode (fused with the top-k): only scores that can still be in the row's top-k
  // are written, compacted in key order to scores + i * ld (ld = the row's candidate slots),
  // with their keys as offsets in the row's window (a window holds at most 65536 keys) at
  // cand_key + i * ld and their number at cand_cnt[i]; a row whose candidates would outgrow
  // its ld slots is compacted in place
  uint16_t* cand_key;
  int* cand_cnt;
  int topk;
};

struct FillArgs {
  SegTable segs;
  float* scores;
  long long ld;
  int n_k;
};

struct TopkArgs {
  SegTable segs;
  const float* scores;
  long long ld;
  int dense;
  int topk;
  int32_t* idx;           // [n_q, topk]
  const uint16_t* cand_key;  // candidate mode: the rows' candidate keys (window offsets), counts
  const int* cand_cnt;
  int cand_min;              // candidate mode: rows with at most this many are served elsewhere
};

// fp32 -> uint32 whose unsigned order is the float order; -0.0 is mapped like +0.0
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct AttnArgs {
  SegTable segs;          // rows to compute when use_segs (else rows 0 .. grid-1)
  int use_segs;
  int xcd_remap;          // 1: give each XCD a contiguous run of rows (grid % 8 == 0)
  const uint16_t* q;      // [n_q, H, DQK] bf16
  const uint16_t* kv;     // [n_k, DQK] bf16
  const int32_t* idx;     // [n_q, topk]
  uint16_t* out;          // [n_q, H, DV] bf16
  float* smax;            // [n_q, H] or null
  float* ssum;            // [n_q, H] or null
  int n_q, n_k, topk;
  int nrows;              // rows (blocks) of this launch
  float scale_log2;       // softmax_scale * log2(e)
};

// Dense causal attention of a head shard: per-head K and V (not a shared latent row).
struct DenseArgs {
  SegTable segs;          // query blocks of 256 rows per segment (blk_off), times the heads
  const uint16_t* q;      // [n_q, H, 192] bf16
  const uint16_t* k;      // [n_k, H, 192] bf16
  const uint16_t* v;      // [n_k, H, 128] bf16
  uint16_t* out;          // [n_q, H, 128] bf16
  float* lse;             // [n_q, H] natural-log logsumexp of the scaled logits, or null
  int h;
  float scale_log2;       // softmax_scale * log2(e)
};

// Sparse-attention backward over one chunk of query rows (pointers offset to the chunk).
struct AttnBwdArgs {
  const uint16_t* q;      // [rows, H, DQK] bf16
  const uint16_t* kv;     // [n_k, DQK] bf16
  const int32_t* idx;     // [rows, topk]
  const uint16_t* out;    // [rows, H, DV] bf16 forward output
  const uint16_t* dout;   // [rows, H, DV] bf16
  const float* smax;      // [rows, H] forward softmax_max
  const float* ssum;      // [rows, H] forward softmax_sum
  uint16_t* ws_p;         // [rows, topkp, H] bf16 probabilities
  uint16_t* ws_ds;        // [rows, topkp, H] bf16 softmax_scale * dS
  uint16_t* dq;           // [rows, H, DQK] bf16
  float* dkv;             // [n_k, DQK] fp32, accumulated
  uint16_t* ws_c;         // [rows, topkp, DQK] bf16 per-(row, slot) dKV contributions
  int* list;              // [rows * topk] (row * topkp + slot) entries grouped by key
  int* cnt;               // [n_k] entries per key
  int* off;               // [n_k + 1] first entry of each key in `list`
  int* cur;               // [n_k] fill cursor
  float* psum;            // [rows, topkp] fp32 sum over heads of P per slot, or null
  int rows, n_k, topk;
  int topkp;              // workspace slots per row: topk rounded up to 96
  int xcd_remap;
  float scale, scale_log2;
};

// Indexer KL loss and its gradients over one chunk of query rows (pointers offset to the chunk).
struct IdxKlArgs {
  const uint16_t* q_idx;  // [rows, 64, 128] bf16 index queries
  const uint16_t* k_idx;  // [n_k, 128] bf16 index keys
  const float* w;         // [rows, 64] index weights
  const uint16_t* q;      // [rows, 128, 576] bf16 attention queries
  const uint16_t* kv;     // [n_k, 576] bf16 latent rows
  const int32_t* idx;     // [rows, topk]
  const float* smax;      // [rows, 128] forward softmax_max
  const float* ssum;      // [rows, 128] forward softmax_sum
  float* loss;            // [rows] per-row KL terms
  uint16_t* dq_idx;       // [rows, 64, 128] bf16
  float* dw;              // [rows, 64]
  uint16_t* ws_c;         // [rows, topkp, 128] bf16 per-(row, slot) index-key gradients
  float* ws_di;           // [rows, topkp] fp32 dI per slot (+ 1 KB slack at the end)
  float* dk;              // [n_k, 128] fp32, accumulated
  const int* list;        // key lists of the chunk (see KeyListArgs)
  const int* off;
  const float* psum;      // [rows, topkp] sum over heads of P per slot (from the attention
                          // backward), or null: the target is recomputed from q and kv
  int rows, n_k, topk;
  int topkp;              // workspace slots per row: topk rounded up to 96
  int xcd_remap;
  float scale_log2;       // softmax_scale * log2(e)
  float loss_grad;        // gradient arriving at each row's loss term
};

// Per-key entry lists of a chunk of top-k rows: every valid (row, slot) entry, as
// row * topkp + slot, grouped by key (off[k] .. off[k + 1] in list).
struct KeyListArgs {
  const int32_t* idx;     // [rows, topk]
  int* list;              // [rows * topk]
  int* cnt;               // [n_k]
  int* off;               // [n_k + 1]
  int* cur;               // [n_k]
  int rows, n_k, topk;
  int topkp;              // slot stride of the per-(row, slot) workspaces the lists index
};

// Builds the lists on stream s (counting sort; integer atomics on the counters only).
hipError_t launch_key_lists(const KeyListArgs& a, hipStream_t s);

struct QuantArgs {
  const uint16_t* x;
  uint8_t* y;
  float* scale;
  long long rows;
  int cols;
};

// ----------------------------------------------------------------------------------------
// small helpers

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// number of set bits of `mask` below the calling lane
__device__ __forceinline__ unsigned lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0u));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((unsigned)b) << 16);
}

// round-to-nearest-even float -> bf16 bits (inputs here are finite)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// Inclusive prefix sum over the 64 lanes of a wave by DPP, with no LDS round trip: row shifts
// by 1, 2, 4 and 8 within each 16-lane row, then the last lane of each row broadcast into the
// rows above it (lanes a shift or broadcast does not reach add 0).
__device__ __forceinline__ unsigned wave_incl_scan(unsigned x) {
  x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);   // row_shr:8
  x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);   // row_bcast:15
  x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return x;
}

// Minimum and maximum over the 64 lanes of a wave (the same DPP pattern; lanes it does not
// reach take the identity), returned to every lane.
__device__ __forceinline__ unsigned wave_min_u32(unsigned x) {
  const int I = -1;
  x = min(x, (unsigned)__builtin_amdgcn_update_dpp(I, (int)x, 0x111, 0xF, 0xF, false));
  x = min(x, (unsigned)__builtin_amdgcn_update_dpp(I, (int)x, 0x112, 0xF, 0xF, false));
  x = min(x, (unsigned)__builtin_amdgcn_update_dpp(I, (int)x, 0x114, 0xF, 0xF, false));
  x = min(x, (unsigned)__builtin_amdgcn_update_dpp(I, (int)x, 0x118, 0xF, 0xF, false));
  x = min(x, (unsigned)__builtin_amdgcn_update_dpp(I, (int)x, 0x142, 0xA, 0xF, false));
  x = min(x, (unsigned)__builtin_amdgcn_update_dpp(I, (int)x, 0x143, 0xC, 0xF, false));
  return (unsigned)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ unsigned wave_max_u32(unsigned x) {
  x = max(x, (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false));
  x = max(x, (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false));
  x = max(x, (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false));
  x = max(x, (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false));
  x = max(x, (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false));
  x = max(x, (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false));
  return (unsigned)__builtin_amdgcn_readlane((int)x, 63);
}

// Block-wide exclusive prefix sum of one value per thread; `scratch` holds NW words of LDS.
// Returns the exclusive prefix; `total` receives the block sum.  Contains two barriers.
template <int NW>
__device__ __forceinline__ unsigned block_excl_scan(unsigned v, unsigned* scratch,
                                                    unsigned& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const unsigned x = wave_incl_scan(v);
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  unsigned before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    unsigned s = scratch[w];
    before += (w < wave) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

}  // namespace dsa
