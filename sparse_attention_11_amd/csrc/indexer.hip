// Lightning Indexer scores on gfx950 MFMA.
//
// Page "CANNTorchTitan: DeepSeek-V3.2 32k长序列预训练昇腾优化实践", section
// "SparseLightningIndexerGradKLLoss": the score of query token t against key s is the
// per-token weighted sum over the token's index heads of ReLU(q_head . k_s); the heads are
// merged into one matrix so one index key row serves all of them (MQA).
//
// Mapping: a workgroup of 8 waves owns 8 consecutive query rows of one segment (one row per
// wave) and sweeps the union of their causal windows in 64-key stages staged through LDS
// (double-buffered, one barrier per stage).  Per wave and 32-key sub-tile the contraction is
//     C[head, key] = sum_d q[row, head, d] * k[key, d]        (M = heads, N = keys, K = d_idx)
// on v_mfma_f32_32x32x16_bf16 (bf16 path) or v_mfma_scale_f32_32x32x64_f8f6f4 with e4m3
// operands (fp8 path).  The query fragments stay in VGPRs for the whole sweep; each key
// fragment read from LDS is reused by every 32-head M tile.  The epilogue runs in registers:
// each lane holds 16 heads of one key column per M tile, so ReLU * w and the head sum are
// per-lane FMAs plus one exchange with the lane 32 apart (which holds the other 16 heads).
// Causal work is uneven, so blocks of later (longer-window) rows are launched first.
//
// Candidate mode (the indexer fused with the top-k, page "CANN/torchtitan-npu融合算子适配",
// section "DSA": the indexer operator hands out indices, not scores): each wave keeps, for its
// row, a running lower bound tau of the row's k-th largest score and writes only the scores
// >= tau (with their keys, compacted in key order); a score below tau is below the final k-th
// largest, so the top-k of the candidates is the top-k of the window, ties included.  tau
// comes from a 256-bin LDS histogram of the candidates' order-preserving keys (bins over a
// range set by the row's first 32 scores, clamped at both ends): the lower edge of the highest
// bin with at least k candidates at or above it.  Only candidates are counted, which keeps the
// counts exact for every bin at or above tau's bin, the only ones the search reads.  A row has
// a fixed number of candidate slots; when the next group might not fit, the wave finds the
// k-th largest candidate exactly and compacts its list in place to what can still be selected.
#include "dsa_device.h"

namespace dsa {

namespace {

constexpr int kIdxWaves = 8;    // query rows (waves) per workgroup
constexpr int kIdxKeys = 64;    // keys per LDS stage
// Candidate slots a bf16 row keeps free after its room check between stages: the late
// waves' pending 64-key group plus the next stage's two (the fp8 kernel offers one group per
// stage and keeps kIdxKeys free).  A row's slots must number at least topk + this many, or
// hold the row's whole window.
constexpr int kRoomBf16 = 3 * kIdxKeys;

// ReLU(x) * w + s with ReLU as one integer max on the fp32 bits: a set sign bit (negative
// values and -0.0) makes the integer negative, so the result is +0 exactly as max(x, 0).
__device__ __forceinline__ float relu_fma(float x, float w, float s) {
  return fmaf(__int_as_float(max(__float_as_int(x), 0)), w, s);
}

// sum of v over the lane pair (l, l ^ 32)
__device__ __forceinline__ float pair_sum(float v) {
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(pr[0]) + __int_as_float(pr[1]);
}

struct RowInfo {
  int row, r, q_len, k_lo, pos, L_blk;
  bool ok;
};

// Per-row state of the candidate filter (one wave per row; all fields wave-uniform).
struct CandRow {
  uint32_t* hist;     // this wave's 256 LDS bins
  float* cs;          // candidate scores of the row
  uint16_t* ck;       // candidate keys (offsets in the row's window)
  int n;              // candidates written so far
  int cap;            // candidate slots of the row
  uint32_t base;      // order key of bin 0's upper part
  int shift;          // bin width (log2) in order-key units
  bool init;
  uint32_t tau;       // order-key threshold (0: keep everything)
};

__device__ __forceinline__ void cand_begin(CandRow& c, uint32_t* hist_wave, float* cs,
                                           uint16_t* ck, int cap) {
  c.hist = hist_wave;
  c.cs = cs;
  c.ck = ck;
  c.n = 0;
  c.cap = cap;
  c.base = 0u;
  c.shift = 0;
  c.init = false;
  c.tau = 0u;
  *reinterpret_cast<uint4*>(hist_wave + 4 * (threadIdx.x & 63)) = make_uint4(0, 0, 0, 0);
}

// The highest of the wave's 256 bins b with at least `need` entries in bins >= b (the lane
// holds bins 4 lane .. 4 lane + 3; the bins must hold at least `need` in total): returns b,
// with the count in the bins above b in `above` and b's own count in `cnt`.
__device__ __forceinline__ int hist_crossing(const uint32_t* hist, uint32_t need, uint32_t& above,
                                             uint32_t& cnt) {
  const int lane = threadIdx.x & 63;
  const uint4 h = *reinterpret_cast<const uint4*>(hist + 4 * lane);
  const uint32_t s4 = h.x + h.y + h.z + h.w;
  // entries in bins >= 4 lane: the total minus an inclusive prefix sum over the lanes
  const uint32_t pre = wave_incl_scan(s4);
  const uint32_t suf = (uint32_t)__builtin_amdgcn_readlane((int)pre, 63) - pre + s4;
  const uint32_t s3 = suf - s4 + h.w, s2 = s3 + h.z, s1 = s2 + h.y, s0 = s1 + h.x;
  const unsigned long long ball = __ballot(s0 >= need);   // lanes 0 .. L*
  const int lstar = 63 - __clzll(ball);
  const int j = s3 >= need ? 3 : s2 >= need ? 2 : s1 >= need ? 1 : 0;
  const uint32_t ab = j == 3 ? suf - s4 : j == 2 ? s3 : j == 1 ? s2 : s1;
  const uint32_t cn = j == 3 ? h.w : j == 2 ? h.z : j == 1 ? h.y : h.x;
  above = (uint32_t)__builtin_amdgcn_readlane((int)ab, lstar);
  cnt = (uint32_t)__builtin_amdgcn_readlane((int)cn, lstar);
  return 4 * lstar + __builtin_amdgcn_readlane(j, lstar);
}

constexpr int kCB = 2;   // candidate groups of 64 loaded together by the compaction (more
                         // would push the indexer's main loop past its registers)

// Order keys of candidates j0 + 64 u + lane, u < kCB (0 past n), loaded together.
__device__ __forceinline__ void cand_keys(const CandRow& c, int j0, int n, uint32_t* ok) {
  const int lane = threadIdx.x & 63;
  float v[kCB];
#pragma unroll
  for (int u = 0; u < kCB; ++u) v[u] = c.cs[min(j0 + 64 * u + lane, n - 1)];
#pragma unroll
  for (int u = 0; u < kCB; ++u) ok[u] = j0 + 64 * u + lane < n ? order_key(v[u]) : 0u;
}

// Room for the next stage when the row's slots are nearly full.  The k-th largest candidate
// key T lies in the histogram's crossing bin; when that bin is a bounded one (neither the
// clamped bottom nor top bin) its range is exact, otherwise the search starts from the
// candidates' min and max.  Radix passes over the stored candidates (the wave's 256 bins,
// 8-bit digits of the offset into the current range) narrow the range until it is small
// enough to keep whole, or down to T itself.  The list is then rewritten in place, in key
// order, keeping every key at or above the range (when narrowed to T: every key above T, then
// the first keys equal to T up to k in all; later equal keys lose the tie to lower ones), and
// the histogram is rebuilt over what is kept.  Only keys that can no longer be in the row's
// top-k are dropped: k kept keys lie at or above the new bound and each precedes every later
// key.  n >= k on entry; the list ends with at most k + (cap - margin - k) / 2 entries.
__device__ __forceinline__ void cand_compact(CandRow& c, int k, int margin) {
  const int lane = threadIdx.x & 63;
  const int n = c.n;
  // this wave's candidate stores complete before its lanes read each other's entries
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  // keeping a whole range is enough once the list then holds at most this many
  const uint32_t limit = (uint32_t)k + (uint32_t)max(0, c.cap - margin - k) / 2u;
  uint32_t above, cnt;
  const int b = hist_crossing(c.hist, (uint32_t)k, above, cnt);
  const uint4 h4 = *reinterpret_cast<const uint4*>(c.hist + 4 * lane);
  const unsigned long long nz = __ballot((h4.x | h4.y | h4.z | h4.w) != 0u);
  const int hl_ = 63 - __clzll(nz);   // highest lane with a nonempty bin (n >= k > 0)
  const uint4 ht = *reinterpret_cast<const uint4*>(c.hist + 4 * hl_);
  const int hb = 4 * hl_ + (ht.w ? 3 : ht.z ? 2 : ht.y ? 1 : 0);   // highest nonempty bin
  uint32_t lo, mxk;   // the range [lo, lo + 2^w) holds T; mxk >= every key
  int w;
  uint32_t krem;      // keys still to take from inside the range
  if (b >= 1 && hb <= 254) {
    lo = c.base + ((uint32_t)b << c.shift);   // (bin b holds keys, so its edge is below 2^32)
    w = c.shift;
    krem = (uint32_t)k - above;
    const unsigned long long top =
        (unsigned long long)c.base + ((unsigned long long)(hb + 1) << c.shift) - 1ull;
    mxk = top > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)top;
  } else {
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int j0 = 0; j0 < n; j0 += 64 * kCB) {
      uint32_t ok[kCB];
      cand_keys(c, j0, n, ok);
#pragma unroll
      for (int u = 0; u < kCB; ++u) {
        if (j0 + 64 * u + lane < n) {
          mn = min(mn, ok[u]);
          mx = max(mx, ok[u]);
        }
      }
    }
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    lo = mn;
    mxk = mx;
    w = mn == mx ? 0 : 32 - __clz((int)(mx - mn));   // 2^w > mx - mn
    krem = (uint32_t)k;
    cnt = (uint32_t)n;
  }
  uint4* hq = reinterpret_cast<uint4*>(c.hist + 4 * lane);
  while (w > 0 && (uint32_t)k - krem + cnt > limit) {
    const int width = min(8, w);
    const int shift = w - width;
    __builtin_amdgcn_wave_barrier();
    *hq = make_uint4(0, 0, 0, 0);
    __builtin_amdgcn_wave_barrier();
    for (int j0 = 0; j0 < n; j0 += 64 * kCB) {
      uint32_t ok[kCB];
      cand_keys(c, j0, n, ok);
#pragma unroll
      for (int u = 0; u < kCB; ++u) {
        const uint32_t off = ok[u] - lo;
        if (j0 + 64 * u + lane < n && ok[u] >= lo && (w >= 32 || (off >> w) == 0u))
          atomicAdd(&c.hist[off >> shift], 1u);
      }
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    uint32_t ab;
    const int d = hist_crossing(c.hist, krem, ab, cnt);
    lo += (uint32_t)d << shift;
    krem -= ab;
    w = shift;
  }
  const bool exact = w == 0 && (uint32_t)k - krem + cnt > limit;   // keep only k
  const uint32_t lo32 = lo;
  // the new histogram: the kept keys span [lo, mxk] over bins 0 .. 127 (bins above are
  // headroom for larger later scores; both ends clamp)
  const uint32_t span = mxk - lo;
  const int nshift = span == 0u ? 0 : max(0, 32 - __clz((int)span) - 7);
  __builtin_amdgcn_wave_barrier();
  *hq = make_uint4(0, 0, 0, 0);
  __builtin_amdgcn_wave_barrier();
  int m = 0;
  uint32_t eqseen = 0;
  for (int j0 = 0; j0 < n; j0 += 64 * kCB) {
    float v[kCB];
    uint16_t kk[kCB];
#pragma unroll
    for (int u = 0; u < kCB; ++u) {
      const int j = min(j0 + 64 * u + lane, n - 1);
      v[u] = c.cs[j];
      kk[u] = c.ck[j];
    }
    // both groups are loaded before the first store: the stores go to positions at or
    // below these, and below every later load
#pragma unroll
    for (int u = 0; u < kCB; ++u) {
      const bool in = j0 + 64 * u + lane < n;
      const uint32_t ok = order_key(v[u]);
      bool keep;
      if (exact) {
        const bool eq = in && ok == lo32;
        const unsigned long long me = __ballot(eq);
        keep = (in && ok > lo32) || (eq && eqseen + lanes_below(me) < krem);
        eqseen += (uint32_t)__popcll(me);
      } else {
        keep = in && ok >= lo32;
      }
      const unsigned long long mk = __ballot(keep);
      if (keep) {
        const int p = m + (int)lanes_below(mk);
        c.cs[p] = v[u];
        c.ck[p] = kk[u];
        atomicAdd(&c.hist[min(255u, (ok - lo32) >> nshift)], 1u);
      }
      m += __popcll(mk);
    }
  }
  // the rewrite's stores complete here: the stage loop around this rarely taken path then
  // carries no pending stores whose registers the next operand reads would have to wait for
  __builtin_amdgcn_s_waitcnt(0);
  c.n = m;
  c.base = lo32;
  c.shift = nshift;
  c.init = true;
  // exact: a later key equal to T loses the tie to the k kept keys
  c.tau = exact ? (lo32 == 0xFFFFFFFFu ? lo32 : lo32 + 1u) : max(c.tau, lo32);
}

// A 64-lane group marked as candidates (bookkeeping and histogram done) whose list writes are
// still to be issued: writing them at the end of the stage, after the key stage's loads have
// landed, keeps the stage loop's waits on those loads from also waiting on fresh stores.
// Only the score is per lane: lane l of the group holds key kb + l, and its list slot is the
// row's count before the group plus the kept lanes below it.
struct CandPend {
  float s;
  int kb;                   // the group's first key
  int nb;                   // the row's candidates before the group
  unsigned long long m;     // kept lanes
  bool valid;
};

// Lane l offers score s of key kb + l (valid v).
__device__ __forceinline__ void cand_mark(CandRow& c, float s, int kb, bool v, CandPend& pd) {
  const uint32_t ok = order_key(s);
  if (!c.init) {   // bin range from the row's first group: its span over 64 of the 256 bins
    const uint32_t mn = wave_min_u32(v ? ok : 0xFFFFFFFFu), mx = wave_max_u32(v ? ok : 0u);
    const uint32_t span = mx - mn;
    c.base = mn;
    c.shift = span == 0u ? 0 : max(0, 32 - __clz((int)span) - 6);
    c.init = true;
  }
  const bool keep = v && ok >= c.tau;
  const unsigned long long m = __ballot(keep);
  // the previous group's registers stay reserved until now, so no asynchronous load ever
  // lands in a register a pending store still reads
  asm volatile("" :: "v"(pd.s));
  pd.s = s;
  pd.kb = kb;
  pd.nb = c.n;
  pd.m = m;
  pd.valid = true;
  if (keep) {
    const uint32_t d = ok < c.base ? 0u : min(255u, (ok - c.base) >> c.shift);
    atomicAdd(&c.hist[d], 1u);
  }
  c.n += __popcll(m);
}

__device__ __forceinline__ void cand_flush(const CandRow& c, CandPend& pd) {
  if (pd.valid) {
    const int lane = threadIdx.x & 63;
    if (__builtin_amdgcn_inverse_ballot_w64(pd.m)) {
      // 32-bit byte offsets from the row's (scalar) list bases
      const unsigned p = (unsigned)pd.nb + (unsigned)lanes_below(pd.m);
      *reinterpret_cast<float*>(reinterpret_cast<char*>(c.cs) + p * 4u) = pd.s;
      *reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(c.ck) + p * 2u) = (uint16_t)(pd.kb + lane);
    }
    pd.valid = false;
  }
}

// Whether the row must compact before offering up to `margin` more keys (slots fewer than
// k + margin hold the row's whole window, so everything fits).  Wave-uniform.
__device__ __forceinline__ bool cand_full(const CandRow& c, int k, int margin) {
  return c.n > c.cap - margin && c.n >= k && c.cap >= k + margin;
}

// Raise tau from the histogram (once k candidates exist).
__device__ __forceinline__ void cand_update(CandRow& c, int k) {
  if (c.n < k) return;
  __builtin_amdgcn_wave_barrier();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's histogram atomics landed
  uint32_t above, cnt;
  const int b = hist_crossing(c.hist, (uint32_t)k, above, cnt);
  if (b > 0) {
    const unsigned long long e = (unsigned long long)c.base + ((unsigned long long)b << c.shift);
    // (a bin holding k candidates starts below 2^32)
    c.tau = max(c.tau, (uint32_t)min(e, 0xFFFFFFFFull));
  }
}

__device__ __forceinline__ RowInfo indexer_row(const SegTable& segs) {
  RowInfo ri;
  const int blk = blockIdx.x;
  const int g = seg_of_block(segs, blk);
  const int nb = segs.blk_off[g + 1] - segs.blk_off[g];
  const int lb = nb - 1 - (blk - segs.blk_off[g]);  // later rows (longer windows) first
  // (wave-uniform, and known so: the row's pointers and window bounds stay scalar)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  ri.q_len = segs.q_len[g];
  const int r0 = lb * kIdxWaves;
  ri.r = r0 + wave;
  ri.ok = ri.r < ri.q_len;
  ri.row = segs.q_start[g] + ri.r;
  ri.k_lo = segs.k_start[g];
  ri.pos = segs.pos0[g] + ri.r;  // window = k_lo + [0, pos]
  ri.L_blk = segs.pos0[g] + min(r0 + kIdxWaves, ri.q_len);
  return ri;
}

}  // namespace

// ------------------------------------------------------------------------------- bf16 ----

template <int HI, int DI, bool CAND>
__global__ __launch_bounds__(kIdxWaves * 64) void k_indexer_bf16(IndexerArgs a) {
  constexpr int MT = (HI + 31) / 32;     // 32-head M tiles
  constexpr int KS = DI / 16;            // K steps of the 32x32x16 MFMA
  constexpr int CPR = DI / 8;            // 16-byte chunks per key row
  constexpr int SWM = CPR - 1;           // chunk swizzle mask (by row)
  constexpr int KST = 2 * kIdxKeys;      // keys per LDS stage (two 64-key halves per barrier)
  constexpr int TILE = KST * DI;         // elements per stage buffer
  constexpr int NPC = TILE * 2 / 1024;   // 1 KB LDS-DMA pieces per stage
  constexpr int PPW = NPC / kIdxWaves;   // pieces per wave
  constexpr int RPP = 1024 / (DI * 2);   // key rows per piece
  static_assert(DI % 16 == 0 && NPC % kIdxWaves == 0 && CPR * RPP == 64, "stage layout");
  // key rows unpadded; physical chunk c of row r holds logical chunk c ^ (r & SWM): the 16
  // rows a 128-bit fragment read serves together then fall in 16 distinct bank groups
  __shared__ __attribute__((aligned(16))) uint16_t sk[2][TILE];
  __shared__ __attribute__((aligned(16))) uint32_t chist[CAND ? kIdxWaves * 256 : 4];

  const RowInfo ri = indexer_row(a.segs);
  const int tid = threadIdx.x, lane = tid & 63, hl = lane & 31, g = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint16_t* qsrc = reinterpret_cast<const uint16_t*>(a.q_idx);
  const uint16_t* ksrc = reinterpret_cast<const uint16_t*>(a.k_idx);

  // query fragments (A operand: row = head, 8 consecutive d per lane) and head weights of the
  // 16 heads this lane's accumulators hold per M tile
  bf16x8 qf[MT][KS];
  float wv[MT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = mt * 32 + hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ri.ok && h < HI)
        v = *reinterpret_cast<const uint4*>(qsrc + ((size_t)ri.row * HI + h) * DI + ks * 16 + g * 8);
      qf[mt][ks] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hh = mt * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
      wv[mt][r] = (ri.ok && hh < HI) ? a.w_idx[(size_t)ri.row * HI + hh] : 0.f;
    }
  }

  float* out = a.scores + (size_t)ri.row * a.ld + (a.dense ? ri.k_lo : 0);
  const int ntiles = (ri.L_blk + KST - 1) / KST;
  CandRow cr;
  if constexpr (CAND)
    cand_begin(cr, chist + (tid >> 6) * 256, out, a.cand_key + (size_t)ri.row * a.ld, (int)a.ld);

  // Stage t's key rows go HBM -> LDS by LDS DMA (no registers held; the compiler never waits
  // on these loads, the stage loop does): piece i of a stage is rows i RPP .. i RPP + RPP - 1,
  // lane L fills physical chunk L % CPR of row i RPP + L / CPR.  Rows past the block's
  // windows copy the union's last key: finite values whose scores the epilogue masks.
  typedef __attribute__((address_space(3))) uint16_t* lds_u16_t;
  const unsigned sk_lds = (unsigned)(size_t)(lds_u16_t)&sk[0][0];
  auto fetch_piece = [&](int t, int buf, int j) {
    const int i = wave_u + kIdxWaves * j;
    const int r = i * RPP + lane / CPR;
    const int c = (lane % CPR) ^ (r & SWM);
    const int kr = min(t * KST + r, ri.L_blk - 1);
    const unsigned voff = (unsigned)(ri.k_lo + kr) * (unsigned)(DI * 2) + (unsigned)c * 16u;
    // (wave-uniform; readfirstlane makes it a scalar, as M0 requires)
    const unsigned m0v = (unsigned)__builtin_amdgcn_readfirstlane(
        (int)(sk_lds + (unsigned)(buf * TILE * 2 + i * 1024)));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(m0v), "v"(voff), "s"(ksrc) : "memory", "m0");
  };
  auto fetch = [&](int t, int buf) {
#pragma unroll
    for (int j = 0; j < PPW; ++j) fetch_piece(t, buf, j);
  };
  static_assert(PPW <= KS, "one DMA piece per K step at most");

  // Per 64-key half: the contraction (32 MFMAs into acc), then the epilogue.  The two waves of
  // a SIMD (w and w + 4) would otherwise reach their epilogues together and leave the matrix
  // pipe idle meanwhile; the upper four waves run each epilogue one half late (after the
  // barrier, at the start of the next half), so one wave's MFMAs overlap the other's
  // epilogue.  The late epilogue needs no more registers: it finishes with acc before the
  // next contraction starts.
  constexpr int NTK = kIdxKeys / 32;
  f32x16 acc[NTK][MT];
  // rows nt * 32 + hl of a half keep hl's swizzle; per K step one lane offset, the rest
  // (buffer, half, sub-tile) are immediate offsets of the read
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = hl * DI + (((2 * ks + g) ^ (hl & SWM)) * 8);
  auto bfrag = [&](int buf, int hh, int ks, int nt) {
    return *reinterpret_cast<const bf16x8*>(&sk[buf][(hh * kIdxKeys + nt * 32) * DI + koff[ks]]);
  };
  // b0: the first PF K steps' key fragments, read by the caller ahead of an epilogue so
  // their LDS latency is hidden behind it
  constexpr int PF = CAND ? 1 : 2;
  // ft >= 0: this wave's DMA pieces of stage ft go out between the K steps (into the other
  // buffer), so that the stage's DMA instructions do not all queue at the stage start
  auto mma = [&](int buf, int hh, const bf16x8 (*b0)[NTK], int ft) {
    // both 32-key sub-tiles are computed unconditionally (keys past the row's window are
    // only masked at the store); K steps outer, so the MT x 2 accumulators form independent
    // chains and consecutive MFMAs never wait for each other
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 b[NTK];
#pragma unroll
      for (int nt = 0; nt < NTK; ++nt) b[nt] = ks < PF ? b0[ks < PF ? ks : 0][nt] : bfrag(buf, hh, ks, nt);
#pragma unroll
      for (int nt = 0; nt < NTK; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[mt][ks], b[nt], acc[nt][mt], 0, 0, 0);
      if (ft >= 0 && ks % (KS / PPW) == 0) fetch_piece(ft, buf ^ 1, ks / (KS / PPW));
    }
  };
  // The epilogue's output (candidate marks, or the dense scores) is written at the end of the
  // stage, after the stage's DMA has landed: no wait of the stage loop then covers a fresh store
  CandPend pend[KST / kIdxKeys];   // per half of a stage
#pragma unroll
  for (int i = 0; i < KST / kIdxKeys; ++i) pend[i] = CandPend{0.f, 0, 0, 0ull, false};
  auto epi = [&](int kb, int slot) {   // kb: first key of the half
    float sv[NTK];
#pragma unroll
    for (int nt = 0; nt < NTK; ++nt) {
      float s = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s = relu_fma(acc[nt][mt][r], wv[mt][r], s);
      sv[nt] = pair_sum(s);   // (both lanes of the pair hold the sum)
    }
    // lane (hl, g) takes key kb + 32 g + hl: 64 keys over the 64 lanes, in key order
    static_assert(kIdxKeys == 64, "two 32-key groups per half-stage");
    const int key = kb + 32 * g + hl;   // = kb + lane
    const float sk_ = g ? sv[1] : sv[0];
    if constexpr (CAND) {
      cand_mark(cr, sk_, kb, key <= ri.pos, pend[slot]);
    } else {
      CandPend& pd = pend[slot];
      asm volatile("" :: "v"(pd.s));   // (see cand_mark)
      pd.s = sk_;
      pd.kb = kb;
      pd.valid = true;
    }
  };
  auto flush = [&]() {
#pragma unroll
    for (int i = 0; i < KST / kIdxKeys; ++i) {
      if constexpr (CAND) {
        cand_flush(cr, pend[i]);
      } else if (pend[i].valid) {
        const int key = pend[i].kb + lane;
        if (key <= ri.pos) out[key] = pend[i].s;
        pend[i].valid = false;
      }
    }
  };
  const bool lag = (tid >> 6) >= kIdxWaves / 2;   // wave-uniform
  int pkb = -1;                                   // half whose epilogue is pending (lag waves)

  fetch(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): stage 0 and the query loads landed
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    // The next stage's DMA.  In candidate mode the non-lag waves issue their pieces inside
    // their first contraction of the stage: issued by all eight waves at the stage start, the
    // DMA instructions queue for hundreds of cycles while the matrix pipe idles.  The lag
    // waves start with their pending epilogue and issue theirs first (from inside their
    // epilogue or contraction, or all by the non-lag waves, the kernel ran slower); so does
    // the plain scores kernel, which ran slower with the spread.
    const int ft = t + 1 < ntiles ? t + 1 : -1;
    const bool fin = CAND && !lag && ri.ok && t * KST <= ri.pos;   // first contraction runs
    if (ft >= 0 && !fin) fetch(ft, buf ^ 1);
    bf16x8 bn[PF][NTK];   // non-lag waves: the second half's first fragments
#pragma unroll
    for (int hh = 0; hh < KST / kIdxKeys; ++hh) {
      const int kb = t * KST + hh * kIdxKeys;   // first key of this 64-key half
      const bool act = ri.ok && kb <= ri.pos;
      if (lag) {
        bf16x8 b0[PF][NTK];
        if (act)
#pragma unroll
          for (int k = 0; k < PF; ++k)
#pragma unroll
            for (int nt = 0; nt < NTK; ++nt) b0[k][nt] = bfrag(buf, hh, k, nt);
        if (pkb >= 0) epi(pkb, hh);
        pkb = -1;
        if (act) {
          mma(buf, hh, b0, -1);
          pkb = kb;
        }
      } else if (act) {
        bf16x8 b0[PF][NTK];
#pragma unroll
        for (int k = 0; k < PF; ++k)
#pragma unroll
          for (int nt = 0; nt < NTK; ++nt) b0[k][nt] = hh == 0 ? bfrag(buf, hh, k, nt) : bn[k][nt];
        mma(buf, hh, b0, CAND && hh == 0 ? ft : -1);
        if (hh + 1 < KST / kIdxKeys && kb + kIdxKeys <= ri.pos)
#pragma unroll
          for (int k = 0; k < PF; ++k)
#pragma unroll
            for (int nt = 0; nt < NTK; ++nt) bn[k][nt] = bfrag(buf, hh + 1, k, nt);
        epi(kb, hh);
      }
    }
    if constexpr (CAND) {   // every second stage: the bound only needs to rise now and then
      if (ri.ok && t * KST <= ri.pos && (t & 1) == 1) cand_update(cr, a.topk);
    }
    // this wave's pieces of the next stage have landed (the stage issued no other memory
    // operation: its writes follow), then every wave's, at the barrier
    __builtin_amdgcn_s_waitcnt(0x0F70);
    flush();
    __syncthreads();
    // Room for what comes before the next check: the late waves' pending group, flushed here
    // when the row compacts (then nothing but the query fragments and weights is live, so
    // the compaction's registers cost the loop nothing), and the next stage's two groups.
    if constexpr (CAND) {
      if (ri.ok && cand_full(cr, a.topk, kRoomBf16)) {
        if (pkb >= 0) epi(pkb, 0);
        pkb = -1;
        flush();
        cand_compact(cr, a.topk, kRoomBf16);
      }
    }
  }
  if (pkb >= 0) epi(pkb, 0);
  flush();
  if constexpr (CAND) {
    if (ri.ok && lane == 0) a.cand_cnt[ri.row] = cr.n;
  }
}

// -------------------------------------------------------------------------------- fp8 ----

template <int HI, int DI, bool CAND>
__global__ __launch_bounds__(kIdxWaves * 64) void k_indexer_fp8(IndexerArgs a) {
  constexpr int MT = (HI + 31) / 32;
  constexpr int KS = (DI + 63) / 64;     // K steps of the 32x32x64 f8f6f4 MFMA (zero padded)
  constexpr int DP = KS * 64;            // padded width in bytes
  constexpr int CPR = DP / 16;           // 16-byte chunks per LDS row
  constexpr int RPW = 256 / DP;          // rows per 256-byte bank window
  constexpr int TILE = kIdxKeys * DP;    // bytes per stage buffer
  constexpr int NPC = TILE / 1024;       // 1 KB LDS-DMA pieces per stage
  constexpr int RPP = 1024 / DP;         // key rows per piece
  static_assert(DI % 16 == 0 && NPC <= kIdxWaves && CPR * RPP == 64, "stage layout");
  // key rows unpadded, physical chunk c of row r holds logical chunk c ^ ((r / RPW) % CPR): the
  // 16 rows a 128-bit fragment read serves together fall in 16 distinct bank groups.  Logical
  // chunks past d_idx (zero padding of the K dimension) repeat the row's first chunks: finite
  // values the zero query chunks multiply away.
  __shared__ __attribute__((aligned(16))) uint8_t sk[2][TILE];
  // key scales of three stages: a late epilogue reads its stage's while other waves already
  // write the scales of the stage after next
  __shared__ float sks[3][kIdxKeys];
  __shared__ __attribute__((aligned(16))) uint32_t chist[CAND ? kIdxWaves * 256 : 4];

  const RowInfo ri = indexer_row(a.segs);
  const int tid = threadIdx.x, lane = tid & 63, hl = lane & 31, g = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q_idx);
  const uint8_t* ksrc = reinterpret_cast<const uint8_t*>(a.k_idx);

  i32x8 qf[MT][KS];
  float wv[MT][16];
  const float qs = ri.ok ? a.q_scale[ri.row] : 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = mt * 32 + hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i32x8 v = {};
      const int d0 = ks * 64 + g * 32;
      if (ri.ok && h < HI) {
        const uint8_t* p = qsrc + ((size_t)ri.row * HI + h) * DI + d0;
        if (d0 + 32 <= DI) {
          const uint4 x0 = *reinterpret_cast<const uint4*>(p);
          const uint4 x1 = *reinterpret_cast<const uint4*>(p + 16);
          v = (i32x8){(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                      (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        } else if (d0 < DI) {
          // partial chunk (d_idx not a multiple of 64): 16-byte granules
#pragma unroll
          for (int c = 0; c < 2; ++c)
            if (d0 + c * 16 < DI) {
              const uint4 x = *reinterpret_cast<const uint4*>(p + c * 16);
              v[c * 4 + 0] = (int)x.x; v[c * 4 + 1] = (int)x.y;
              v[c * 4 + 2] = (int)x.z; v[c * 4 + 3] = (int)x.w;
            }
        }
      }
      qf[mt][ks] = v;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hh = mt * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
      // the query's per-token scale is folded into the head weights
      wv[mt][r] = (ri.ok && hh < HI) ? a.w_idx[(size_t)ri.row * HI + hh] * qs : 0.f;
    }
  }

  float* out = a.scores + (size_t)ri.row * a.ld + (a.dense ? ri.k_lo : 0);
  const int ntiles = (ri.L_blk + kIdxKeys - 1) / kIdxKeys;
  CandRow cr;
  if constexpr (CAND)
    cand_begin(cr, chist + (tid >> 6) * 256, out, a.cand_key + (size_t)ri.row * a.ld, (int)a.ld);

  // Stage t's key rows by LDS DMA (piece i = rows i RPP .., lane L fills physical chunk L % CPR
  // of row i RPP + L / CPR; rows past the block's windows copy the union's last key), and the
  // stage's key scales through a register (one per thread of the first 64, index clamped the
  // same way), written to LDS at the end of the stage.
  typedef __attribute__((address_space(3))) uint8_t* lds_u8_t;
  const unsigned sk_lds = (unsigned)(size_t)(lds_u8_t)&sk[0][0];
  float pres = 0.f;
  auto fetch = [&](int t, int buf) {
    if (wave_u < NPC) {
      const int i = wave_u;
      const int r = i * RPP + lane / CPR;
      const int lc = (lane % CPR) ^ ((r / RPW) % CPR);
      const int kr = min(t * kIdxKeys + r, ri.L_blk - 1);
      const unsigned voff = (unsigned)(ri.k_lo + kr) * (unsigned)DI + (unsigned)(lc % (DI / 16)) * 16u;
      const unsigned m0v = (unsigned)__builtin_amdgcn_readfirstlane(
          (int)(sk_lds + (unsigned)(buf * TILE + i * 1024)));
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(m0v), "v"(voff), "s"(ksrc) : "memory", "m0");
    }
    if (tid < kIdxKeys) pres = a.k_scale[ri.k_lo + min(t * kIdxKeys + tid, ri.L_blk - 1)];
  };
  auto stash_scale = [&](int sbuf) {
    if (tid < kIdxKeys) sks[sbuf][tid] = pres;
  };
  CandPend pend = CandPend{0.f, 0, 0, 0ull, false};
  auto flush = [&]() {
    if constexpr (CAND) {
      cand_flush(cr, pend);
    } else if (pend.valid) {
      const int key = pend.kb + lane;
      if (key <= ri.pos) out[key] = pend.s;
      pend.valid = false;
    }
  };

  // Per stage: the contraction (both 32-key sub-tiles, 8 MFMAs), then one epilogue for the
  // 64 keys (lane (hl, g) takes key kb + 32 g + hl, so the filter and the writes run once per
  // 64 keys on every lane).  The two waves of a SIMD (w and w + 4) would reach their
  // epilogues together and leave the matrix pipe idle; the upper four waves run each
  // epilogue one stage late (after the barrier, before their next contraction), so one wave's
  // MFMAs overlap the other's epilogue.  Stage t's key scales are in sks[t % 3].
  f32x16 acc[2][MT];
  auto mma = [&](int buf) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int row = nt * 32 + hl;
        const int sw = (row / RPW) % CPR;
        const uint8_t* rp = &sk[buf][row * DP];
        const uint4 b0 = *reinterpret_cast<const uint4*>(rp + (((ks * 4 + 2 * g) ^ sw) * 16));
        const uint4 b1 = *reinterpret_cast<const uint4*>(rp + (((ks * 4 + 2 * g + 1) ^ sw) * 16));
        const i32x8 b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                         (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          // formats: A and B e4m3 (0); block scales 127 = 2^0
          acc[nt][mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              qf[mt][ks], b, acc[nt][mt], 0, 0, 0, 127, 0, 127);
      }
    }
  };
  auto epi = [&](int kb, int sbuf) {
    float sv[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float s = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s = relu_fma(acc[nt][mt][r], wv[mt][r], s);
      sv[nt] = pair_sum(s);   // (both lanes of the pair hold the sum)
    }
    static_assert(kIdxKeys == 64, "two 32-key sub-tiles per stage");
    const int key = kb + 32 * g + hl;   // = kb + lane
    const float sc = (g ? sv[1] : sv[0]) * sks[sbuf][32 * g + hl];
    if constexpr (CAND) {
      cand_mark(cr, sc, kb, key <= ri.pos, pend);
    } else {
      asm volatile("" :: "v"(pend.s));   // (see cand_mark)
      pend.s = sc;
      pend.kb = kb;
      pend.valid = true;
    }
  };
  const bool lag = (tid >> 6) >= kIdxWaves / 2;   // wave-uniform
  int pkb = -1;                                   // stage whose epilogue is pending (lag waves)

  fetch(0, 0);
  stash_scale(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): stage 0 landed
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) fetch(t + 1, buf ^ 1);
    const int kb = t * kIdxKeys;   // first key of the stage
    const bool act = ri.ok && kb <= ri.pos;
    if (lag) {
      if (pkb >= 0) epi(pkb, (t + 2) % 3);   // stage t - 1
      pkb = -1;
      if (act) {
        mma(buf);
        pkb = kb;
      }
    } else if (act) {
      mma(buf);
      epi(kb, t % 3);
    }
    if (ri.ok) {
      if constexpr (CAND) {   // every fourth 64-key stage
        if (t * kIdxKeys <= ri.pos && (t & 3) == 3) cand_update(cr, a.topk);
      }
    }
    // the next stage's rows and scales landed (the stage's own writes follow), then every
    // wave's, at the barrier
    stash_scale((t + 1) % 3);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    flush();
    __syncthreads();
    // the next check comes after the late waves' pending group and the next stage's group
    if constexpr (CAND) {
      if (ri.ok && cand_full(cr, a.topk, 2 * kIdxKeys)) {
        if (pkb >= 0) epi(pkb, t % 3);
        pkb = -1;
        flush();
        cand_compact(cr, a.topk, 2 * kIdxKeys);
      }
    }
  }
  if (pkb >= 0) epi(pkb, (ntiles - 1) % 3);
  flush();
  if constexpr (CAND) {
    if (ri.ok && lane == 0) a.cand_cnt[ri.row] = cr.n;
  }
}

// ------------------------------------------------------------- -inf outside the windows ----

// One block per covered row (grid from the segment table, 1 block per row).
__global__ __launch_bounds__(256) void k_fill_outside(FillArgs a) {
  const int blk = blockIdx.x;
  const int g = seg_of_block(a.segs, blk);
  const int r = blk - a.segs.blk_off[g];
  const int row = a.segs.q_start[g] + r;
  const int lo = a.segs.k_start[g];
  const int hi = lo + a.segs.pos0[g] + r + 1;   // exclusive end of the window
  float* p = a.scores + (size_t)row * a.ld;
  const float ninf = -__builtin_huge_valf();
  for (int c = threadIdx.x; c < a.n_k; c += 256)
    if (c < lo || c >= hi) p[c] = ninf;
}

// ------------------------------------------------------------------------------ launch ----

hipError_t launch_indexer(const IndexerArgs& a, int h_idx, int d_idx, bool fp8,
                          hipStream_t s) {
  const dim3 grid(a.segs.blk_off[a.segs.n]), block(kIdxWaves * 64);
  if (grid.x == 0) return hipSuccess;
  const bool cand = a.cand_cnt != nullptr;
  if (!fp8) {
    if (h_idx == 64 && d_idx == 128) {
      if (cand) k_indexer_bf16<64, 128, true><<<grid, block, 0, s>>>(a);
      else k_indexer_bf16<64, 128, false><<<grid, block, 0, s>>>(a);
    } else if (h_idx == 4 && d_idx == 32) {
      if (cand) k_indexer_bf16<4, 32, true><<<grid, block, 0, s>>>(a);
      else k_indexer_bf16<4, 32, false><<<grid, block, 0, s>>>(a);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    if (h_idx == 64 && d_idx == 128) {
      if (cand) k_indexer_fp8<64, 128, true><<<grid, block, 0, s>>>(a);
      else k_indexer_fp8<64, 128, false><<<grid, block, 0, s>>>(a);
    } else if (h_idx == 4 && d_idx == 32) {
      if (cand) k_indexer_fp8<4, 32, true><<<grid, block, 0, s>>>(a);
      else k_indexer_fp8<4, 32, false><<<grid, block, 0, s>>>(a);
    } else {
      return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_fill_outside(const FillArgs& a, hipStream_t s) {
  const dim3 grid(a.segs.blk_off[a.segs.n]), block(256);
  if (grid.x == 0) return hipSuccess;
  k_fill_outside<<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

int indexer_rows_per_block() { return kIdxWaves; }

}  // namespace dsa
