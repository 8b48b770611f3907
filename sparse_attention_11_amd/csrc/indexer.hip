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
#include "dsa_device.h"

namespace dsa {

namespace {

constexpr int kIdxWaves = 8;    // query rows (waves) per workgroup
constexpr int kIdxKeys = 64;    // keys per LDS stage

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

__device__ __forceinline__ RowInfo indexer_row(const SegTable& segs) {
  RowInfo ri;
  const int blk = blockIdx.x;
  const int g = seg_of_block(segs, blk);
  const int nb = segs.blk_off[g + 1] - segs.blk_off[g];
  const int lb = nb - 1 - (blk - segs.blk_off[g]);  // later rows (longer windows) first
  const int wave = threadIdx.x >> 6;
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

template <int HI, int DI>
__global__ __launch_bounds__(kIdxWaves * 64) void k_indexer_bf16(IndexerArgs a) {
  constexpr int MT = (HI + 31) / 32;     // 32-head M tiles
  constexpr int KS = DI / 16;            // K steps of the 32x32x16 MFMA
  constexpr int ROW = DI + 8;            // LDS row in bf16 elements (16-byte pad)
  constexpr int CPR = DI / 8;            // 16-byte chunks per key row
  constexpr int KST = 2 * kIdxKeys;      // keys per LDS stage (two 64-key halves per barrier)
  constexpr int CH = KST * CPR;          // chunks per stage
  constexpr int NT = kIdxWaves * 64;
  constexpr int PER = (CH + NT - 1) / NT;
  static_assert(DI % 16 == 0, "d_idx must be a multiple of 16");
  __shared__ __attribute__((aligned(16))) uint16_t sk[2][KST * ROW];

  const RowInfo ri = indexer_row(a.segs);
  const int tid = threadIdx.x, lane = tid & 63, hl = lane & 31, g = lane >> 5;
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

  uint4 pre[PER];
  auto fetch = [&](int t) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = tid + p * NT;
      const int key = c / CPR, col = c % CPR;
      const int kr = t * KST + key;
      pre[p] = make_uint4(0, 0, 0, 0);
      if (c < CH && kr < ri.L_blk)
        pre[p] = *reinterpret_cast<const uint4*>(ksrc + (size_t)(ri.k_lo + kr) * DI + col * 8);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = tid + p * NT;
      if (c < CH) {
        const int key = c / CPR, col = c % CPR;
        *reinterpret_cast<uint4*>(&sk[buf][key * ROW + col * 8]) = pre[p];
      }
    }
  };

  fetch(0);
  stash(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) fetch(t + 1);
#pragma unroll
    for (int hh = 0; hh < KST / kIdxKeys; ++hh) {
    const int kb = t * KST + hh * kIdxKeys;   // first key of this 64-key half
    if (ri.ok && kb <= ri.pos) {
      // both 32-key sub-tiles are computed unconditionally (keys past the row's window are
      // only masked at the store); K steps outer, so the MT x 2 accumulators form independent
      // chains and consecutive MFMAs never wait for each other
      constexpr int NT = kIdxKeys / 32;
      f32x16 acc[NT][MT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = (f32x16){};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 b[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          b[nt] = *reinterpret_cast<const bf16x8*>(&sk[buf][(hh * kIdxKeys + nt * 32 + hl) * ROW + ks * 16 + g * 8]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[mt][ks], b[nt], acc[nt][mt], 0, 0, 0);
      }
#pragma unroll
      for (int nt = 0; nt < kIdxKeys / 32; ++nt) {
        float s = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) s = relu_fma(acc[nt][mt][r], wv[mt][r], s);
        s = pair_sum(s);
        const int key = kb + nt * 32 + hl;
        if (g == 0 && key <= ri.pos) out[key] = s;
      }
    }
    }
    if (t + 1 < ntiles) stash(buf ^ 1);
    __syncthreads();
  }
}

// -------------------------------------------------------------------------------- fp8 ----

template <int HI, int DI>
__global__ __launch_bounds__(kIdxWaves * 64) void k_indexer_fp8(IndexerArgs a) {
  constexpr int MT = (HI + 31) / 32;
  constexpr int KS = (DI + 63) / 64;     // K steps of the 32x32x64 f8f6f4 MFMA (zero padded)
  constexpr int DP = KS * 64;            // padded width in bytes
  constexpr int ROW = DP + 16;           // LDS row in bytes (16-byte pad)
  constexpr int CPR = DP / 16;
  constexpr int CH = kIdxKeys * CPR;
  constexpr int NT = kIdxWaves * 64;
  constexpr int PER = (CH + NT - 1) / NT;
  static_assert(DI % 16 == 0, "d_idx must be a multiple of 16");
  __shared__ __attribute__((aligned(16))) uint8_t sk[2][kIdxKeys * ROW];
  __shared__ float sks[2][kIdxKeys];

  const RowInfo ri = indexer_row(a.segs);
  const int tid = threadIdx.x, lane = tid & 63, hl = lane & 31, g = lane >> 5;
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

  uint4 pre[PER];
  float pres = 0.f;
  auto fetch = [&](int t) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = tid + p * NT;
      const int key = c / CPR, col = c % CPR;
      const int kr = t * kIdxKeys + key;
      pre[p] = make_uint4(0, 0, 0, 0);
      if (c < CH && kr < ri.L_blk && col * 16 < DI)
        pre[p] = *reinterpret_cast<const uint4*>(ksrc + (size_t)(ri.k_lo + kr) * DI + col * 16);
    }
    if (tid < kIdxKeys) {
      const int kr = t * kIdxKeys + tid;
      pres = kr < ri.L_blk ? a.k_scale[ri.k_lo + kr] : 0.f;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = tid + p * NT;
      if (c < CH) {
        const int key = c / CPR, col = c % CPR;
        *reinterpret_cast<uint4*>(&sk[buf][key * ROW + col * 16]) = pre[p];
      }
    }
    if (tid < kIdxKeys) sks[buf][tid] = pres;
  };

  fetch(0);
  stash(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) fetch(t + 1);
    if (ri.ok) {
#pragma unroll
      for (int nt = 0; nt < kIdxKeys / 32; ++nt) {
        const int kbase = t * kIdxKeys + nt * 32;
        if (kbase <= ri.pos) {
          f32x16 acc[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x16){};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const uint8_t* bp = &sk[buf][(nt * 32 + hl) * ROW + ks * 64 + g * 32];
            const uint4 b0 = *reinterpret_cast<const uint4*>(bp);
            const uint4 b1 = *reinterpret_cast<const uint4*>(bp + 16);
            const i32x8 b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                             (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              // formats: A and B e4m3 (0); block scales 127 = 2^0
              acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qf[mt][ks], b, acc[mt],
                                                                        0, 0, 0, 127, 0, 127);
          }
          float s = 0.f;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) s = relu_fma(acc[mt][r], wv[mt][r], s);
          s = pair_sum(s);
          const int key = kbase + hl;
          if (g == 0 && key <= ri.pos) out[key] = s * sks[buf][nt * 32 + hl];
        }
      }
    }
    if (t + 1 < ntiles) stash(buf ^ 1);
    __syncthreads();
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
  if (!fp8) {
    if (h_idx == 64 && d_idx == 128) k_indexer_bf16<64, 128><<<grid, block, 0, s>>>(a);
    else if (h_idx == 4 && d_idx == 32) k_indexer_bf16<4, 32><<<grid, block, 0, s>>>(a);
    else return hipErrorInvalidValue;
  } else {
    if (h_idx == 64 && d_idx == 128) k_indexer_fp8<64, 128><<<grid, block, 0, s>>>(a);
    else if (h_idx == 4 && d_idx == 32) k_indexer_fp8<4, 32><<<grid, block, 0, s>>>(a);
    else return hipErrorInvalidValue;
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
