// Per-row causal top-k over indexer scores: LDS radix select with a deterministic tie-break.
//
// Page "CANNTorchTitan: DeepSeek-V3.2 32k长序列预训练昇腾优化实践", section
// "SparseLightningIndexerGradKLLoss": K_topk holds the keys of each token's top-k indexer
// scores; the selection here keeps n = min(topk, window) keys, gives equal scores to the
// lower key index (-0.0 counts as +0.0) and emits the kept keys in ascending order.
//
// One workgroup per row.  The row's window (at most THREADS * ITEMS scores) is read once from
// HBM, coalesced, into registers as order-preserving 32-bit keys.  Radix passes over digits
// of up to 12 bits (LDS histograms, one LDS atomic per candidate, candidates narrowing to
// those matching the prefix found so far) find the exact k-th largest key T and how many
// keys equal to T are needed; once the threshold bin holds at most 256 keys, they are
// gathered in LDS and T is found by counting, for each of them, the keys above it.  The digits cover only the bits below the common prefix of the
// row's smallest and largest key: a row's scores share their leading bits, and digits taken
// from those bits would send every key of the first pass to a handful of bins.  A single ballot / mbcnt compaction in key-index order
// then writes every key > T and the first `need` keys == T straight to their output slot, so
// the output comes out sorted by key index with no sort.  Rows whose window is not longer
// than topk skip the selection and write the window plus -1 padding.
#include "dsa_device.h"

namespace dsa {

// CAND: the row's input is the candidate list the fused indexer wrote (scores compacted in
// key order, their keys as window offsets, their count) instead of the whole window.  The list holds every key
// that can be in the top-k, in key order, so the same selection applies with the list
// position standing in for the key index.
template <int THREADS, int ITEMS, bool CAND>
__global__ __launch_bounds__(THREADS) void k_topk(TopkArgs a) {
  constexpr int NW = THREADS / 64;
  constexpr int NE = ITEMS * NW;          // (item, wave) compaction groups
  static_assert(NE <= THREADS, "compaction scan needs one group per thread");
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t grp_gt[NE];
  __shared__ uint32_t grp_eq[NE];
  __shared__ uint32_t scan_tmp[NW];
  __shared__ uint32_t found[2];
  constexpr int CAP = 256;                // candidate set small enough for a direct rank count
  __shared__ uint32_t cand[CAP];
  __shared__ uint32_t ncand;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int blk = blockIdx.x;
  const int g = seg_of_block(a.segs, blk);
  const int r = a.segs.q_len[g] - 1 - (blk - a.segs.blk_off[g]);  // longer windows first
  const int row = a.segs.q_start[g] + r;
  const int k_lo = a.segs.k_start[g];
  const int L = CAND ? a.cand_cnt[row] : a.segs.pos0[g] + r + 1;
  // candidate mode with two launches: this configuration serves the rows whose candidates
  // fit in it and that the smaller configuration before it could not hold
  if (CAND && (L > THREADS * ITEMS || L <= a.cand_min)) return;
  const int topk = a.topk;
  const float* src = a.scores + (size_t)row * a.ld + (a.dense ? k_lo : 0);
  const uint16_t* ckey = CAND ? a.cand_key + (size_t)row * a.ld : nullptr;
  int32_t* dst = a.idx + (size_t)row * topk;
  auto key_of = [&](int e) { return CAND ? k_lo + (int)ckey[e] : k_lo + e; };

  if (L <= topk) {
    for (int t = tid; t < topk; t += THREADS) dst[t] = t < L ? key_of(t) : -1;
    return;
  }

  // unconditional loads (clamped index), so all of them are in flight at once; in candidate
  // mode the candidates' key indices come with them (read here, not at the output writes,
  // where each would be a dependent memory round trip) where the registers allow: at most 16
  // items per thread (with 32 the extra registers cost the 512-thread tier its second
  // workgroup per CU, and the 1024-thread tiers have only 128 VGPRs per lane)
  constexpr bool PRE = CAND && THREADS <= 512 && ITEMS <= 16;
  uint32_t key[ITEMS];
  int32_t ckv[PRE ? ITEMS : 1];
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) key[j] = __float_as_uint(src[min(j * THREADS + tid, L - 1)]);
  if constexpr (PRE) {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) ckv[j] = k_lo + (int)ckey[min(j * THREADS + tid, L - 1)];
  }
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) key[j] = j * THREADS + tid < L ? order_key(__uint_as_float(key[j])) : 0u;

  // The keys of one row usually share their leading bits (scores of a row lie in a narrow
  // band): digits start below the common prefix of the row's min and max key, so the first
  // histogram spreads over its bins instead of piling into a few.
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    if (j * THREADS + tid < L) {
      kmin = min(kmin, key[j]);
      kmax = max(kmax, key[j]);
    }
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    grp_gt[wave] = kmin;
    grp_eq[wave] = kmax;
  }
  __syncthreads();
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kmin = min(kmin, grp_gt[w]);
    kmax = max(kmax, grp_eq[w]);
  }
  __syncthreads();
  const int nbits = kmin == kmax ? 0 : 32 - __clz((int)(kmin ^ kmax));   // differing low bits
  uint32_t pmask = nbits == 32 ? 0u : ~((1u << nbits) - 1u);
  uint32_t prefix = kmin & pmask, krem = (uint32_t)topk;
  for (int done = 0; done < nbits;) {   // block-uniform trip count (at most 3 passes)
    const int width = min(12, nbits - done);
    const int shift = nbits - done - width;
    const int nbins = 1 << width;
    const uint32_t dmask = (uint32_t)(nbins - 1);
    for (int b = tid; b < nbins; b += THREADS) hist[b] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int e = j * THREADS + tid;
      if (e < L && (key[j] & pmask) == prefix) atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread t owns chunk (nchunks-1-t) of consecutive bins, so the exclusive scan in thread
    // order counts the keys in all higher bins
    const int cpt = nbins >= THREADS ? nbins / THREADS : 1;
    const int nchunks = nbins / cpt;
    const int chunk = nchunks - 1 - tid;
    uint32_t csum = 0;
    if (chunk >= 0)
      for (int i = 0; i < cpt; ++i) csum += hist[chunk * cpt + i];
    uint32_t tot;
    uint32_t above = block_excl_scan<NW>(csum, scan_tmp, tot);
    if (chunk >= 0 && above < krem && krem <= above + csum) {
      for (int i = cpt - 1; i >= 0; --i) {
        const uint32_t h = hist[chunk * cpt + i];
        if (above + h >= krem) {
          found[0] = (uint32_t)(chunk * cpt + i);
          found[1] = above;
          break;
        }
        above += h;
      }
    }
    __syncthreads();
    prefix |= found[0] << shift;
    pmask |= dmask << shift;
    krem -= found[1];
    done += width;
    const uint32_t nb = hist[found[0]];   // keys left in the threshold bin (block-uniform)
    __syncthreads();
    if (done < nbits && nb <= (uint32_t)CAP) {
      // few candidates left: gather them and find the krem-th largest by counting, for each
      // candidate, the candidates above it and equal to it (instead of further passes)
      if (tid == 0) ncand = 0u;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < ITEMS; ++j) {
        const int e = j * THREADS + tid;
        if (e < L && (key[j] & pmask) == prefix) cand[atomicAdd(&ncand, 1u)] = key[j];
      }
      __syncthreads();
      for (int i = tid; i < (int)nb; i += THREADS) {
        const uint32_t ki = cand[i];
        uint32_t gt = 0, eq = 0;
        for (int j = 0; j < (int)nb; ++j) {
          const uint32_t kj = cand[j];
          gt += kj > ki;
          eq += kj == ki;
        }
        if (gt < krem && krem <= gt + eq) {   // tied candidates all write the same values
          found[0] = ki;
          found[1] = gt;
        }
      }
      __syncthreads();
      prefix = found[0];
      krem -= found[1];
      break;
    }
  }
  const uint32_t T = prefix;   // the topk-th largest key
  const uint32_t need = krem;  // how many keys equal to T are kept (lowest indices first)

#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int e = j * THREADS + tid;
    const bool v = e < L;
    const unsigned long long mg = __ballot(v && key[j] > T);
    const unsigned long long me = __ballot(v && key[j] == T);
    if (lane == 0) {
      grp_gt[j * NW + wave] = (uint32_t)__popcll(mg);
      grp_eq[j * NW + wave] = (uint32_t)__popcll(me);
    }
  }
  __syncthreads();
  {
    const uint32_t vg = tid < NE ? grp_gt[tid] : 0u;
    const uint32_t ve = tid < NE ? grp_eq[tid] : 0u;
    uint32_t tg, te;
    const uint32_t eg = block_excl_scan<NW>(vg, scan_tmp, tg);
    const uint32_t ee = block_excl_scan<NW>(ve, scan_tmp, te);
    if (tid < NE) {
      grp_gt[tid] = eg;
      grp_eq[tid] = ee;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int e = j * THREADS + tid;
    const bool v = e < L;
    const bool gt = v && key[j] > T;
    const bool eq = v && key[j] == T;
    const unsigned long long mg = __ballot(gt);
    const unsigned long long me = __ballot(eq);
    const uint32_t n_gt = grp_gt[j * NW + wave] + lanes_below(mg);
    const uint32_t n_eq = grp_eq[j * NW + wave] + lanes_below(me);
    const uint32_t pos = n_gt + min(n_eq, need);
    if ((gt || (eq && n_eq < need)) && pos < (uint32_t)topk)
      dst[pos] = PRE ? ckv[PRE ? j : 0] : key_of(e);
  }
}

template <bool CAND>
hipError_t launch_topk_t(const TopkArgs& a, int max_window, hipStream_t s) {
  const dim3 grid(a.segs.blk_off[a.segs.n]);
  if (grid.x == 0) return hipSuccess;
  if (max_window <= 2048) k_topk<256, 8, CAND><<<grid, 256, 0, s>>>(a);
  else if (max_window <= 8192) k_topk<512, 16, CAND><<<grid, 512, 0, s>>>(a);
  else if (max_window <= 32768) k_topk<1024, 32, CAND><<<grid, 1024, 0, s>>>(a);
  else if (max_window <= 65536) k_topk<1024, 64, CAND><<<grid, 1024, 0, s>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, int max_window, hipStream_t s) {
  if (!a.cand_cnt) return launch_topk_t<false>(a, max_window, s);
  // candidates (at most a.ld per row): rows with at most 8192 go to a small configuration
  // (several workgroups per CU), rows with up to 16384 to a middle one, the rest (up to
  // 32768) to a large one; each launch skips the rows another one serves
  const dim3 grid(a.segs.blk_off[a.segs.n]);
  if (grid.x == 0) return hipSuccess;
  const long long cap = a.ld;
  if (cap > 32768) return hipErrorInvalidValue;
  TopkArgs t = a;
  t.cand_min = 0;
  if (cap <= 2048) {
    k_topk<256, 8, true><<<grid, 256, 0, s>>>(t);
    return hipGetLastError();
  }
  k_topk<512, 16, true><<<grid, 512, 0, s>>>(t);
  if (cap > 8192) {
    t.cand_min = 8192;
    k_topk<512, 32, true><<<grid, 512, 0, s>>>(t);
  }
  if (cap > 16384) {
    t.cand_min = 16384;
    k_topk<1024, 32, true><<<grid, 1024, 0, s>>>(t);
  }
  return hipGetLastError();
}

}  // namespace dsa
