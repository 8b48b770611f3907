// Indexer KL loss and its gradients on gfx950 MFMA.
//
// Page "CANNTorchTitan: DeepSeek-V3.2 32k长序列预训练昇腾优化实践", section
// "SparseLightningIndexerGradKLLoss": for each query token the target distribution over its
// selected keys is the Sparse Flash Attention probability summed over the query heads and
// normalised to unit L1 norm; the indexer's distribution is the softmax of its top-k values
// I = sum_j w_j ReLU(q_idx_j . k_idx); the loss is the KL divergence of the indexer's
// distribution from the target, dI = softmax(I) - p, and the gradients of the index weights,
// queries and keys follow through the ReLU, the key gradients being scatter-added into the
// selected rows.  The attention probabilities are recomputed from the forward's softmax
// statistics rather than stored.
//
// One workgroup per query row, four waves, 32 selected keys per tile, two passes over the
// row's tiles:
//   * Pass 1 gathers each tile's latent rows (576 wide) and index-key rows (128 wide) into
//     LDS rings by LDS DMA.  The logits C[head, key] = Q K^T run on 32x32x16 MFMA with the
//     wave's 32 heads x 576 dims of Q held in VGPRs (nothing else of that size is live, so Q
//     needs no LDS staging here) in two accumulator chains; each lane owns one key and 16
//     heads, so the head sum of the probabilities is lane-local up to one lane swap.  The
//     same tile gives S[index head, key] on 16x16x32 MFMA (16 index heads per wave) and the
//     weighted ReLU head sum.  Per-wave partial sums meet in LDS and are added in a fixed
//     order into two per-row arrays (target mass, I), so the result is deterministic.
//   * Between the passes the block forms softmax(I), the normalised target, the row's KL term
//     and dI (stored over the target array).
//   * Pass 2 gathers the index-key tiles again and recomputes S^T[key, index head].  dS, dW
//     and dq_idx^T += K^T dS^T stay in registers (K^T read with the transposing LDS read; the
//     MFMA's K order is the accumulator's key order, so dS feeds it without a shuffle).  dS
//     is shared through LDS and each slot's key gradient dS^T q_idx is formed by the wave
//     that owns 32 of its 128 dims and written as bf16 per (row, slot).
//   * The per-slot key gradients are then summed per key (the chunk's entries grouped by key,
//     16 lanes per key) and added to dk_idx: no float atomics.
// When the attention backward runs in the same call it hands over each slot's sum over heads
// of P, and pass 1 (k_idx_kl_p1t) gathers only the index keys and forms I; the target mass is
// read, not recomputed.
#include <algorithm>

#include "attn_common.h"

namespace dsa {

namespace {

constexpr int kH = 128, kDQK = 576, kDV = 512;   // attention heads, latent row, value width
constexpr int kG = 64, kDI = 128;                 // index heads, index head width
using AC = AttnCfg<kH, kDQK, kDV>;
constexpr int NK = AC::NK;             // keys per tile (32)
constexpr int kKs = kDQK / 16;         // K steps of the logits product
constexpr int kMaxSlots = 2112;        // 66 tiles: topk <= 2048, rounded up to rings of 3 tiles
constexpr int KT = NK * kDI;           // elements of an index-key tile (8 KB)
constexpr int DSR = NK + 4;            // LDS row stride (elements) of the shared dS tile
constexpr int GK = 2;                  // index-key gather instructions per wave and tile
constexpr int kDiLds = 2304;           // dI floats in LDS: 66 tiles x 32 rounded up to 1 KB pieces
constexpr float kLog2e = 1.44269504088896340736f;
static_assert(AC::RPW == 8 && AC::FLAT, "tile split of the gathers");

typedef __attribute__((address_space(3))) const bf16x8* lds_cb8_t;
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x + x of the lane 16 (32) apart, in every lane (one lane swap between row pairs).
__device__ __forceinline__ float pair16_sum(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(p[0]) + __int_as_float(p[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(p[0]) + __int_as_float(p[1]);
}

// two floats -> two round-to-nearest-even bf16 in one dword (one packed conversion)
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Block-wide sum / max over the 4 waves (two barriers).
__device__ __forceinline__ float block_sum(float x, float* sb) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) sb[threadIdx.x >> 6] = x;
  __syncthreads();
  const float r = (sb[0] + sb[1]) + (sb[2] + sb[3]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_max(float x, float* sb) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  if ((threadIdx.x & 63) == 0) sb[threadIdx.x >> 6] = x;
  __syncthreads();
  const float r = fmaxf(fmaxf(sb[0], sb[1]), fmaxf(sb[2], sb[3]));
  __syncthreads();
  return r;
}

// The wave's 8 index-key rows of a tile (tile rows 8 w .. 8 w + 7) into an LDS tile of 256-B
// rows by LDS DMA.  Instruction i copies rows 8 w + 4 i .. +3: lane L fills physical chunk
// L % 16 of row 8 w + 4 i + L / 16, which holds logical chunk (L % 16) ^ (row % 16).  The XOR
// makes 16 rows x one logical chunk (the MFMA operand reads) hit 16 different bank groups.
// Empty slots copy row 0 (masked later).  sk: byte offsets in k_idx of the wave's 8 rows,
// scalars (0 for empty slots).
__device__ __forceinline__ void gather_ktile_piece(const IdxKlArgs& a, const RowCtx& c,
                                                   const unsigned* sk, unsigned lds_tile, int i) {
  const int sub = c.lane >> 4, ch = c.lane & 15;
  const bool b0 = c.lane & 16, b1 = c.lane & 32;
  // (opaque to the optimiser: selects between loads of sk[] would otherwise become one load
  // at a lane-dependent index, through scratch memory)
  unsigned s0 = sk[4 * i], s1 = sk[4 * i + 1], s2 = sk[4 * i + 2], s3 = sk[4 * i + 3];
  asm("" : "+s"(s0), "+s"(s1), "+s"(s2), "+s"(s3));
  const unsigned lo = b0 ? s1 : s0;
  const unsigned hi = b0 ? s3 : s2;
  const unsigned ro = b1 ? hi : lo;
  const int r = c.wave * 8 + 4 * i + sub;
  const unsigned voff = ro + (unsigned)((ch ^ (r & 15)) * 16);
  const unsigned m0v = lds_tile + (unsigned)((c.wave_u * 8 + 4 * i) * kDI * 2);
  const uint16_t* base = a.k_idx;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m0v), "v"(voff), "s"(base) : "memory", "m0");
}

__device__ __forceinline__ void gather_ktile_so(const IdxKlArgs& a, const RowCtx& c,
                                                const unsigned* sk, unsigned lds_tile) {
#pragma unroll
  for (int i = 0; i < GK; ++i) gather_ktile_piece(a, c, sk, lds_tile, i);
}

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(__attribute__((address_space(3))) const void*)p;
}

// The row's distributions, KL term and dI (block-wide), from the target mass s_p and the
// indexer values s_i of its ntiles * 32 slots; dI replaces the target in s_p and goes to the
// workspace for pass 2.
__device__ __forceinline__ void kl_row_tail(const IdxKlArgs& a, const RowCtx& c, int ntiles,
                                            float* s_p, const float* s_i, float* s_blk) {
  const int row = c.row;
  {
    const int nsl = ntiles * NK;
    float m = kNegInf;
    for (int s = c.tid; s < nsl; s += 256) m = fmaxf(m, s_i[s]);
    m = block_max(m, s_blk);
    float se = 0.f, pt = 0.f;
    for (int s = c.tid; s < nsl; s += 256) {
      se += expf(s_i[s] - m);
      pt += s_p[s];
    }
    se = block_sum(se, s_blk);
    pt = block_sum(pt, s_blk);
    const float lse = m + logf(se);
    const float ipt = pt > 0.f ? 1.f / pt : 0.f;
    float kl = 0.f;
    for (int s = c.tid; s < nsl; s += 256) {
      const float p = s_p[s] * ipt;
      const float lr = s_i[s] - lse;       // log softmax(I); -inf at empty slots
      if (p > 0.f) kl += p * (logf(p) - lr);
      s_p[s] = a.loss_grad * (expf(lr) - p);
    }
    kl = block_sum(kl, s_blk);             // (its barriers also publish dI)
    if (c.tid == 0) a.loss[row] = kl;
  }
  // dI of the row's slots -> workspace, for the pass-2 kernel
  {
    float* dst = a.ws_di + (size_t)row * a.topkp;
    for (int sl = c.tid * 4; sl < ntiles * NK; sl += 256 * 4)
      *reinterpret_cast<float4*>(dst + sl) = *reinterpret_cast<const float4*>(s_p + sl);
  }
}

__global__ __launch_bounds__(256) void k_idx_kl_p1(IdxKlArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t kv0[AC::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t kv1[AC::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t kv2[AC::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t kt0[KT];
  __shared__ __attribute__((aligned(16))) uint16_t kt1[KT];
  __shared__ __attribute__((aligned(16))) uint16_t kt2[KT];
  __shared__ __attribute__((aligned(16))) float s_p[kMaxSlots];   // target mass, then dI
  __shared__ __attribute__((aligned(16))) float s_i[kMaxSlots];   // indexer values I
  __shared__ float s_red[2][2][4][NK];   // [tile parity][mass, I][wave][key]
  __shared__ __attribute__((aligned(16))) int32_t idxr[2 * kIdxChunk];   // index ring
  __shared__ int s_last[4];
  __shared__ float s_blk[4];

  RowCtx c = make_ctx(a, block_row(a));
  c.buf[0] = kv0;
  c.buf[1] = kv1;
  c.buf[2] = kv2;
  c.ntiles = row_tiles<kH, kDQK, kDV>(a, c, s_last);
  const int row = c.row;
  if (c.ntiles == 0) {   // nothing selected: loss 0 (the pass-2 kernel zeroes the gradients)
    if (c.tid == 0) a.loss[row] = 0.f;
    return;
  }
  // the row's slot indices reach LDS in chunks of eight tiles (no per-tile index loads,
  // whose wait would also stall the first LDS read of every step); issued after the early
  // exit, so no LDS DMA can outlive the block
  const unsigned idxr_lds = lds_addr(idxr);
  idx_chunk_dma<kH, kDQK, kDV>(a, c, 0, idxr_lds);
  idx_chunk_dma<kH, kDQK, kDV>(a, c, 1, idxr_lds);
  const uint16_t* kts[3] = {kt0, kt1, kt2};
  const int i16 = c.lane & 15, G = c.lane >> 4;

  // ---- row operands
  bf16x8 qf[kKs];   // Q of head wave*32 + hl, dims 16 ks + 8 g .. +7 (A of the logits)
  {
    const uint16_t* qp = a.q + ((size_t)row * kH + c.head) * kDQK + c.g * 8;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + ks * 16));
  }
  // softmax statistics of the lane's 16 heads (accumulator register r holds head
  // wave*32 + (r/4)*8 + 4 g + r%4), folded into one exponent bias per head:
  // P = exp(z - max) / sum = exp2(z log2(e) - (max log2(e) + log2(sum)))
  float bias[16];
  {
    const size_t hb = (size_t)row * kH + c.wave * 32 + 4 * c.g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 mx = *reinterpret_cast<const float4*>(a.smax + hb + 8 * j);
      const float4 sm = *reinterpret_cast<const float4*>(a.ssum + hb + 8 * j);
      const float mv[4] = {mx.x, mx.y, mx.z, mx.w}, sv[4] = {sm.x, sm.y, sm.z, sm.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)   // (a head without keys: bias +inf, P = 0)
        bias[4 * j + u] = (sv[u] > 0.f && mv[u] != kNegInf) ? fmaf(mv[u], kLog2e, __log2f(sv[u]))
                                                            : __builtin_huge_valf();
    }
  }
  bf16x8 qi[4];   // index query of head 16 wave + i16, dims 32 s + 8 G .. +7
  {
    const uint16_t* p = a.q_idx + ((size_t)row * kG + 16 * c.wave + i16) * kDI + 8 * G;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qi[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p + 32 * s));
  }
  // weights of index heads 16 wave + 4 G + r (the S accumulator rows of this lane)
  const float4 wq = *reinterpret_cast<const float4*>(a.w + (size_t)row * kG + 16 * c.wave + 4 * G);
  // index-key tile: row i16 (and i16 + 16), logical chunk 4 s + G
  int koff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = i16 * kDI + (((4 * s + G) ^ i16) * 8);

  unsigned loff[AC::NI], wb[3], kb[3];
#pragma unroll
  for (int i = 0; i < AC::NI; ++i) loff[i] = flat_lane_offset<kH, kDQK, kDV>(c, i);
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    wb[k] = lds_addr(c.buf[k]) + c.wave_u * (AC::RPW * AC::ROWE * 2);
    kb[k] = lds_addr(kts[k]);
  }
  // gather of the tile whose slots sit in lanes lane0 .. lane0 + 31 of the decoded offsets
  // (kvo: byte offset in kv, kio: in k_idx; 0 for empty slots)
  auto gather = [&](unsigned kvo, unsigned kio, int lane0, int k) {
    unsigned so[AC::RPW], sk[AC::RPW];
#pragma unroll
    for (int j = 0; j < AC::RPW; ++j) {
      so[j] = __builtin_amdgcn_readlane(kvo, lane0 + c.wave_u * AC::RPW + j);
      sk[j] = __builtin_amdgcn_readlane(kio, lane0 + c.wave_u * AC::RPW + j);
    }
    gather_tile_flat_so<kH, kDQK, kDV>(a, c, so, loff, wb[k]);
    gather_ktile_so(a, c, sk, kb[k]);
  };
  // a slot as the gathers use it: validity ballot, byte offsets of its rows
  auto decode = [&](int v, int slot, unsigned& kvo, unsigned& kio) {
    const bool ok = slot < a.topk && (unsigned)v < (unsigned)a.n_k;
    kvo = ok ? (unsigned)v * (AC::CPR * 16u) : 0u;
    kio = ok ? (unsigned)v * (kDI * 2u) : 0u;
    return (unsigned)__ballot(ok);
  };
  const lds_ci32_t ir = (lds_ci32_t)idxr;
  // slot read by this lane for step t: lanes 0..31 the tile the step computes (t), lanes
  // 32..63 the tile it gathers (t+2)
  auto step_slot = [&](int t) { return (t + 2 * (c.lane >> 5)) * NK + (c.lane & 31); };
  // row loads and index chunks done (a wait the compiler sees, so it adds none inside the
  // ring, where the counter also holds the in-flight gathers); the chunks are every wave's
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  // ---- pass 1: target mass and indexer values per slot
  // Pipelined by one tile: while the matrix cores run tile t's logits, the wave issues the
  // VALU epilogue of tile t-1 (probabilities, head sums, the indexer's ReLU head sums) between
  // the MFMAs, so the epilogue does not serialise behind the product.  Q moves to AGPRs and
  // the logits MFMAs (inline asm) read their A operand from there, which leaves the VGPRs to
  // the LDS prefetch and the carried state of the previous tile.
  const int ntiles = (c.ntiles + 2) / 3 * 3;
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks) asm volatile("" : "+a"(qf[ks]));
  {
    {   // tiles 0 and 1 from chunk 0
      unsigned kvo, kio;
      (void)decode(ir[c.lane], c.lane, kvo, kio);
      gather(kvo, kio, 0, 0);
      gather(kvo, kio, 32, 1);
    }
    int iv = ir[step_slot(0)];
    wait_vm_barrier<0>();

    f32x16 sp0 = (f32x16){}, sp1 = (f32x16){};   // previous tile: logits (two chains)
    f32x4 xp0 = (f32x4){}, xp1 = (f32x4){};      // previous tile: index scores
    unsigned vmp = 0;                             // previous tile: validity bits
    float pm = 0.f, v0 = 0.f, v1 = 0.f;
    // unit u of the previous tile's epilogue (units 0 .. 23); the results land in
    // s_red[(t-1) & 1] (at t = 0 a harmless all-empty tile -1)
    auto epi = [&](int u, int t) {
      if (u < 16) {
        pm += __builtin_amdgcn_exp2f(fmaf(sp0[u] + sp1[u], a.scale_log2, -bias[u]));
      } else if (u == 16) {
        pm = pair32_sum(pm);
      } else if (u == 17) {
        v0 = wq.x * fmaxf(xp0[0], 0.f) + wq.y * fmaxf(xp0[1], 0.f) +
             wq.z * fmaxf(xp0[2], 0.f) + wq.w * fmaxf(xp0[3], 0.f);
      } else if (u == 18) {
        v1 = wq.x * fmaxf(xp1[0], 0.f) + wq.y * fmaxf(xp1[1], 0.f) +
             wq.z * fmaxf(xp1[2], 0.f) + wq.w * fmaxf(xp1[3], 0.f);
      } else if (u == 19) {
        v0 = pair16_sum(v0);
      } else if (u == 20) {
        v1 = pair16_sum(v1);
      } else if (u == 21) {
        v0 = pair32_sum(v0);
      } else if (u == 22) {
        v1 = pair32_sum(v1);
      } else if (u == 23) {
        // lane = key (lanes 32..63 repeat lanes 0..31 with equal values)
        const int pb = (t - 1) & 1, key = c.lane & 31;
        s_red[pb][0][c.wave][key] = ((vmp >> key) & 1u) ? pm : 0.f;
        s_red[pb][1][c.wave][key] = ((vmp >> key) & 1u) ? ((c.lane & 16) ? v1 : v0) : kNegInf;
        pm = 0.f;
      }
    };
    auto lazy_sum = [&](int tt) {   // tile tt's per-wave partials -> row arrays
      const int pb = tt & 1;
      s_p[tt * NK + c.lane] = (s_red[pb][0][0][c.lane] + s_red[pb][0][1][c.lane]) +
                              (s_red[pb][0][2][c.lane] + s_red[pb][0][3][c.lane]);
      s_i[tt * NK + c.lane] = (s_red[pb][1][0][c.lane] + s_red[pb][1][1][c.lane]) +
                              (s_red[pb][1][2][c.lane] + s_red[pb][1][3][c.lane]);
    };

    auto step = [&](int t, int slot, int ahead2) {
      unsigned kvo, kio;
      // validity of tile t (lanes 0..31: bit k = key k), rows of tile t+2 (lanes 32..63)
      const unsigned vmask = decode(iv, step_slot(t), kvo, kio);
      // chunk t/8 + 1 (first read at the end of step t + 5, for the gather of tile t + 8)
      // into the ring half chunk t/8 - 1 left; a load ahead of this step's gather, so
      // complete once tile t+2 has landed
      if ((t & 7) == 0 && t > 0) idx_chunk_dma<kH, kDQK, kDV>(a, c, t / 8 + 1, idxr_lds);
      // tile t+2's gather, one LDS DMA piece every third K step of the logits (issued together
      // at the step start, the four waves' 44 DMA instructions queued for about a thousand
      // cycles ahead of the first MFMA); each piece reads its rows' offsets from the decoded
      // slots (lanes 32 + 8 wave ..) as it goes out
      const int l0 = 32 + c.wave_u * AC::RPW;
      auto piece = [&](int p) {
        if (p < AC::NI) {   // latent rows: 1 KB of the wave's eight rows
          const int j0 = p * 64 / AC::CPR;
          const int b = (j0 + 1) * AC::CPR - 64 * p;
          unsigned ro = __builtin_amdgcn_readlane(kvo, l0 + j0);
          if (b < 64) {
            const unsigned r1 = __builtin_amdgcn_readlane(kvo, l0 + j0 + 1);
            ro = c.lane >= b ? r1 : ro;
          }
          const unsigned voff = loff[p] + ro;
          const unsigned m0v = wb[ahead2] + (unsigned)p * 1024u;
          const uint16_t* base = a.kv;
          asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                       :: "s"(m0v), "v"(voff), "s"(base) : "memory", "m0");
        } else {            // index-key rows
          const int i = p - AC::NI;   // (< GK)
          unsigned sk[AC::RPW];
#pragma unroll
          for (int j = 0; j < AC::RPW; ++j)
            sk[j] = j / 4 == i ? __builtin_amdgcn_readlane(kio, l0 + j) : 0u;
          gather_ktile_piece(a, c, sk, kb[ahead2], i);
        }
      };
      static_assert(3 * (AC::NI + GK) <= kKs, "gather pieces placement");
      if (t >= 2 && c.wave_u == (t & 3) && c.lane < NK) lazy_sum(t - 2);

      // logits C[head, key]: A = Q (AGPRs), B = latent row hl of the tile, chunk 2 ks + g
      // (physical chunk (2 ks + g) ^ swz(hl)); even / odd K steps in two chains, PD
      // fragments read ahead
      const lds_cptr_t lt = (lds_cptr_t)c.buf[slot];
      const int sw = swz(c.hl);
      lds_cptr_t bb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = lt + c.hl * AC::ROWE + (((2 * j + c.g) ^ sw) - 2 * j) * 8;
      auto at = [&](int ks) { return bb[ks & 3] + ks * 16; };
      const lds_cptr_t kt = (lds_cptr_t)kts[slot];
      constexpr int PD = 6;
      bf16x8 f[PD], kf[8];
      f32x16 s0, s1;
#pragma unroll
      for (int i = 0; i < PD; ++i) f[i] = *(lds_cb8_t)(at(i));
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
        const bf16x8 cur = f[ks % PD];
        if (ks + PD < kKs) f[ks % PD] = *(lds_cb8_t)(at(ks + PD));
        if (ks >= kKs - 8) {   // this tile's index-key fragments, ahead of the index product
          const int j = ks - (kKs - 8);
          kf[j] = *(lds_cb8_t)(kt + koff[j >> 1] + (j & 1) * 16 * kDI);
        }
        const bf16x8 qa = qf[ks];
        if (ks == 0) {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&a"(s0) : "a"(qa), "v"(cur));
        } else if (ks == 1) {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&a"(s1) : "a"(qa), "v"(cur));
        } else if (ks % 2 == 0) {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(s0) : "a"(qa), "v"(cur));
        } else if (ks == kKs - 1) {
          // the results are read by VALU next: wait out the MFMA write-to-read distance
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                       : "+a"(s1) : "a"(qa), "v"(cur));
        } else {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(s1) : "a"(qa), "v"(cur));
        }
        if (ks < 24) epi(ks, t);
        if (ks % 3 == 1 && ks / 3 < AC::NI + GK) piece(ks / 3);
        __builtin_amdgcn_sched_barrier(0);
      }
      // indexer S[index head, key]: A = index-query rows, B = index-key rows i16, 16 + i16
      f32x4 x0 = (f32x4){}, x1 = (f32x4){};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        x0 = mfma16(qi[s], kf[2 * s], x0);
        x1 = mfma16(qi[s], kf[2 * s + 1], x1);
      }
      sp0 = s0;
      sp1 = s1;
      xp0 = x0;
      xp1 = x1;
      vmp = vmask;
      iv = ir[step_slot(t + 1) & (2 * kIdxChunk - 1)];
      // tile t+1 landed for every wave (only tile t+2's gathers, and maybe an index chunk
      // ahead of them, may still be in flight)
      wait_vm_barrier<AC::GOPS + GK>();
    };
    for (int t = 0; t < ntiles; t += 3) {
      step(t, 0, 2);
      step(t + 1, 1, 0);
      step(t + 2, 2, 1);
    }
#pragma unroll
    for (int u = 0; u < 24; ++u) epi(u, ntiles);   // the last tile's epilogue
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // gathers past the last tile
    __syncthreads();
    if (c.wave_u == 0 && c.lane < NK) lazy_sum(ntiles - 2);
    if (c.wave_u == 1 && c.lane < NK) lazy_sum(ntiles - 1);
  }
  __syncthreads();

  kl_row_tail(a, c, ntiles, s_p, s_i, s_blk);
}

// Pass 1 with the target given: each slot's sum over heads of the attention probabilities
// comes from the attention backward (its probability kernel forms them anyway), so the tiles
// need neither the latent rows nor the logits; only the index keys are gathered (a three-tile
// ring, tile t+2 during step t) and I formed.  44 KB of LDS: three workgroups per CU.
__global__ __launch_bounds__(256, 3) void k_idx_kl_p1t(IdxKlArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t kt0[KT];
  __shared__ __attribute__((aligned(16))) uint16_t kt1[KT];
  __shared__ __attribute__((aligned(16))) uint16_t kt2[KT];
  __shared__ __attribute__((aligned(16))) float s_p[kMaxSlots];   // target mass, then dI
  __shared__ __attribute__((aligned(16))) float s_i[kMaxSlots];   // indexer values I
  __shared__ float s_red[2][4][NK];   // [tile parity][wave][key] partial I
  __shared__ __attribute__((aligned(16))) int32_t idxr[2 * kIdxChunk];   // index ring
  __shared__ int s_last[4];
  __shared__ float s_blk[4];

  RowCtx c = make_ctx(a, block_row(a));
  c.ntiles = row_tiles<kH, kDQK, kDV>(a, c, s_last);
  const int row = c.row;
  if (c.ntiles == 0) {
    if (c.tid == 0) a.loss[row] = 0.f;
    return;
  }
  const unsigned idxr_lds = lds_addr(idxr);
  idx_chunk_dma<kH, kDQK, kDV>(a, c, 0, idxr_lds);
  idx_chunk_dma<kH, kDQK, kDV>(a, c, 1, idxr_lds);
  const int ntiles = (c.ntiles + 2) / 3 * 3;
  // the target mass of the row's slots (zero past its last tile)
  for (int sl = c.tid; sl < ntiles * NK; sl += 256)
    s_p[sl] = sl < c.ntiles * NK ? a.psum[(size_t)row * a.topkp + sl] : 0.f;
  const uint16_t* kts[3] = {kt0, kt1, kt2};
  const int i16 = c.lane & 15, G = c.lane >> 4;
  bf16x8 qi[4];   // index query of head 16 wave + i16, dims 32 s + 8 G .. +7
  {
    const uint16_t* p = a.q_idx + ((size_t)row * kG + 16 * c.wave + i16) * kDI + 8 * G;
#pragma unroll
    for (int sx = 0; sx < 4; ++sx)
      qi[sx] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p + 32 * sx));
  }
  const float4 wq = *reinterpret_cast<const float4*>(a.w + (size_t)row * kG + 16 * c.wave + 4 * G);
  int koff[4];
#pragma unroll
  for (int sx = 0; sx < 4; ++sx) koff[sx] = i16 * kDI + (((4 * sx + G) ^ i16) * 8);
  unsigned kb[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) kb[k] = lds_addr(kts[k]);
  auto decode = [&](int v, int slot, unsigned& kio) {
    const bool ok = slot < a.topk && (unsigned)v < (unsigned)a.n_k;
    kio = ok ? (unsigned)v * (kDI * 2u) : 0u;
    return (unsigned)__ballot(ok);
  };
  auto gather = [&](unsigned kio, int lane0, int k) {
    unsigned sk[AC::RPW];
#pragma unroll
    for (int j = 0; j < AC::RPW; ++j)
      sk[j] = __builtin_amdgcn_readlane(kio, lane0 + c.wave_u * AC::RPW + j);
    gather_ktile_so(a, c, sk, kb[k]);
  };
  const lds_ci32_t ir = (lds_ci32_t)idxr;
  auto step_slot = [&](int t) { return (t + 2 * (c.lane >> 5)) * NK + (c.lane & 31); };
  auto lazy_sum = [&](int tt) {   // tile tt's per-wave partials -> I
    const int pb = tt & 1;
    s_i[tt * NK + c.lane] = (s_red[pb][0][c.lane] + s_red[pb][1][c.lane]) +
                            (s_red[pb][2][c.lane] + s_red[pb][3][c.lane]);
  };
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  {
    unsigned kio;
    (void)decode(ir[c.lane], c.lane, kio);
    gather(kio, 0, 0);
    gather(kio, 32, 1);
  }
  int iv = ir[step_slot(0)];
  wait_vm_barrier<0>();
  auto step = [&](int t, int slot, int ahead2) {
    unsigned kio;
    // validity of tile t (lanes 0..31), rows of tile t+2 (lanes 32..63)
    const unsigned vmask = decode(iv, step_slot(t), kio);
    if ((t & 7) == 0 && t > 0) idx_chunk_dma<kH, kDQK, kDV>(a, c, t / 8 + 1, idxr_lds);
    gather(kio, 32, ahead2);
    if (t >= 1 && c.wave_u == (t & 3) && c.lane < NK) lazy_sum(t - 1);
    const lds_cptr_t kt = (lds_cptr_t)kts[slot];
    bf16x8 kf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kf[j] = *(lds_cb8_t)(kt + koff[j >> 1] + (j & 1) * 16 * kDI);
    f32x4 x0 = (f32x4){}, x1 = (f32x4){};
#pragma unroll
    for (int sx = 0; sx < 4; ++sx) {
      x0 = mfma16(qi[sx], kf[2 * sx], x0);
      x1 = mfma16(qi[sx], kf[2 * sx + 1], x1);
    }
    float v0 = wq.x * fmaxf(x0[0], 0.f) + wq.y * fmaxf(x0[1], 0.f) +
               wq.z * fmaxf(x0[2], 0.f) + wq.w * fmaxf(x0[3], 0.f);
    float v1 = wq.x * fmaxf(x1[0], 0.f) + wq.y * fmaxf(x1[1], 0.f) +
               wq.z * fmaxf(x1[2], 0.f) + wq.w * fmaxf(x1[3], 0.f);
    v0 = pair32_sum(pair16_sum(v0));
    v1 = pair32_sum(pair16_sum(v1));
    if (c.lane < NK) {   // lane = key
      const int key = c.lane;
      s_red[t & 1][c.wave][key] = ((vmask >> key) & 1u) ? ((c.lane & 16) ? v1 : v0) : kNegInf;
    }
    iv = ir[step_slot(t + 1) & (2 * kIdxChunk - 1)];
    wait_vm_barrier<GK>();   // tile t+1 landed (only tile t+2's gathers may be in flight)
  };
  for (int t = 0; t < ntiles; t += 3) {
    step(t, 0, 2);
    step(t + 1, 1, 0);
    step(t + 2, 2, 1);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // gathers past the last tile
  if (c.wave_u == 0 && c.lane < NK) lazy_sum(ntiles - 1);
  __syncthreads();
  kl_row_tail(a, c, ntiles, s_p, s_i, s_blk);
}

// Pass 2 (a kernel of its own: it needs 51 KB of LDS, so three workgroups share a CU and
// one workgroup's waits overlap another's work).  One workgroup per row, four waves.  The
// index-key tiles are gathered again and S^T[key, index head] recomputed; dS, dW and
// dq_idx^T += K^T dS^T stay in registers (K^T from the transposing LDS read; the MFMA's K order
// is the accumulator's key order, so dS is the B operand as it stands); dS is shared through
// LDS and each wave forms the key gradient dS^T q_idx of its 32 of the 128 dims for every
// slot, written as bf16 per (row, slot).
__global__ __launch_bounds__(256, 3) void k_idx_kl_p2(IdxKlArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t kt0[KT];
  __shared__ __attribute__((aligned(16))) uint16_t kt1[KT];
  __shared__ __attribute__((aligned(16))) uint16_t kt2[KT];
  __shared__ __attribute__((aligned(16))) uint16_t stage[kG * kDI];   // q_idx, then dS tiles
  __shared__ __attribute__((aligned(16))) float s_di[kDiLds];        // dI of the row's slots
  __shared__ __attribute__((aligned(16))) int32_t idxr[2 * kIdxChunk];   // index ring
  __shared__ int s_last[4];
  static_assert(2 * kG * DSR <= kG * kDI, "two dS tiles fit in the staging area");

  RowCtx c = make_ctx(a, block_row(a));
  c.ntiles = row_tiles<kH, kDQK, kDV>(a, c, s_last);
  const int row = c.row;
  if (c.ntiles == 0) {   // nothing selected: no gradient
    uint4* dq = reinterpret_cast<uint4*>(a.dq_idx + (size_t)row * kG * kDI);
    for (int j = c.tid; j < kG * kDI / 8; j += 256) dq[j] = make_uint4(0, 0, 0, 0);
    if (c.tid < kG) a.dw[(size_t)row * kG + c.tid] = 0.f;
    return;
  }
  const int ntiles = (c.ntiles + 2) / 3 * 3;
  // the row's slot indices by LDS DMA (after the early exit: no DMA outlives the block)
  const unsigned idxr_lds = lds_addr(idxr);
  idx_chunk_dma<kH, kDQK, kDV>(a, c, 0, idxr_lds);
  idx_chunk_dma<kH, kDQK, kDV>(a, c, 1, idxr_lds);
  const uint16_t* kts[3] = {kt0, kt1, kt2};
  unsigned kb[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) kb[k] = lds_addr(kts[k]);
  const int i16 = c.lane & 15, G = c.lane >> 4;
  bf16x8 qi[4];   // index query of head 16 wave + i16, dims 32 s + 8 G .. +7
  {
    const uint16_t* p = a.q_idx + ((size_t)row * kG + 16 * c.wave + i16) * kDI + 8 * G;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qi[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p + 32 * s));
  }
  const float wn = a.w[(size_t)row * kG + 16 * c.wave + i16];
  int koff[4];   // index-key tile: row i16 (and i16 + 16), logical chunk 4 s + G
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = i16 * kDI + (((4 * s + G) ^ i16) * 8);
  // the row's index queries (64 x 128 bf16) and its dI (rounded up to whole 1 KB pieces; the
  // workspace has the slack) by LDS DMA
  dma_copy_flat<4>(lds_addr(stage), a.q_idx + (size_t)row * kG * kDI, kG * kDI * 2, c.wave_u, c.lane);
  dma_copy_flat<4>(lds_addr(s_di), a.ws_di + (size_t)row * a.topkp, (ntiles * NK * 4 + 1023) & ~1023,
                   c.wave_u, c.lane);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  // A of the key gradient (q_idx^T): dims 32 wave + 16 mb + i16, index heads 32 ks + 8 G .. +7
  bf16x8 qt[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qt[mb][ks] = tr_frag(stage, kDI, 32 * ks + 8 * G, 32 * c.wave + 16 * mb, i16);
  __syncthreads();   // the staging area now holds the dS tiles
  // dS[index head][key] of a tile, two buffers
  auto dsb = [&](int par) { return stage + (par & 1) * (kG * DSR); };
  // transposing reads of an index-key tile: rows (keys) 4 G + i16/4 (+16), columns 16 Mb + 4 (i16 % 4)
  int toff[8];
  {
    const int r = 4 * G + (i16 >> 2), q4 = i16 & 3;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
      toff[mb] = r * kDI + (((2 * mb + (q4 >> 1)) ^ (r & 15)) * 8) + (q4 & 1) * 4;
  }
  float dwacc = 0.f;
  f32x4 dqa[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) dqa[mb] = (f32x4){};
  const uint16_t* cbase = a.ws_c + (size_t)row * a.topkp * kDI;   // the row's slot gradients

  // key gradients of tile u for this wave's 32 dims: C[dim, key] = q_idx^T dS over 64 heads
  auto key_grad = [&](int u) {
    const uint16_t* dsu = dsb(u);
    f32x4 z[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) z[mb][0] = z[mb][1] = (f32x4){};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const bf16x8 b = tr_frag(dsu, DSR, 32 * ks + 8 * G, 16 * nb, i16);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) z[mb][nb] = mfma16(qt[mb][ks], b, z[mb][nb]);
      }
    // lane: key 16 nb + i16, dims 32 wave + 16 mb + 4 G .. +3 -> one 8-byte store each
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const u32x2 v = {pack_bf16(z[mb][nb][0], z[mb][nb][1]), pack_bf16(z[mb][nb][2], z[mb][nb][3])};
        const unsigned off = (unsigned)((((u * NK + 16 * nb + i16) * kDI) + 32 * c.wave + 16 * mb + 4 * G) * 2);
        const uint16_t* b0 = cbase;
        asm volatile("global_store_dwordx2 %0, %1, %2" :: "v"(off), "v"(v), "s"(b0) : "memory");
      }
  };

  {
    const lds_ci32_t ir = (lds_ci32_t)idxr;
    // byte offset in k_idx of a slot's row (0 for an empty slot), and the gather of the tile
    // whose slots sit in lanes lane0 .. lane0 + 31
    auto kio_of = [&](int v, int slot) {
      return (slot < a.topk && (unsigned)v < (unsigned)a.n_k) ? (unsigned)v * (kDI * 2u) : 0u;
    };
    auto gather = [&](unsigned kio, int lane0, int k) {
      unsigned sk[AC::RPW];
#pragma unroll
      for (int j = 0; j < AC::RPW; ++j)
        sk[j] = __builtin_amdgcn_readlane(kio, lane0 + c.wave_u * AC::RPW + j);
      gather_ktile_so(a, c, sk, kb[k]);
    };
    // slot read by every lane for step t: the tile it gathers (t+2)
    auto step_slot = [&](int t) { return (t + 2) * NK + (c.lane & 31); };
    {   // tiles 0 and 1 from chunk 0
      const unsigned kio = kio_of(ir[c.lane], c.lane);
      gather(kio, 0, 0);
      gather(kio, 32, 1);
    }
    int iv = ir[step_slot(0)];
    wait_vm_barrier<0>();

    auto step = [&](int t, int slot, int ahead2) {
      // chunk t/8 + 1 (first read at the end of step t + 5, for the gather of tile t + 8)
      // into the ring half chunk t/8 - 1 left; a load ahead of this step's gather, so
      // complete once tile t+2 has landed
      if ((t & 7) == 0 && t > 0) idx_chunk_dma<kH, kDQK, kDV>(a, c, t / 8 + 1, idxr_lds);
      gather(kio_of(iv, step_slot(t)), 0, ahead2);
      if (t > 0) key_grad(t - 1);
      const lds_cptr_t kt = (lds_cptr_t)kts[slot];
      // S^T[key, index head]: A = index-key rows i16 / 16 + i16, B = index-query rows
      f32x4 y0 = (f32x4){}, y1 = (f32x4){};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 a0 = *(lds_cb8_t)(kt + koff[s]);
        const bf16x8 a1 = *(lds_cb8_t)(kt + koff[s] + 16 * kDI);
        y0 = mfma16(a0, qi[s], y0);
        y1 = mfma16(a1, qi[s], y1);
      }
      // lane: index head 16 wave + i16; keys 4 G + r (y0) and 16 + 4 G + r (y1)
      const float4 e0 = *reinterpret_cast<const float4*>(s_di + t * NK + 4 * G);
      const float4 e1 = *reinterpret_cast<const float4*>(s_di + t * NK + 16 + 4 * G);
      const float d0[4] = {e0.x, e0.y, e0.z, e0.w}, d1[4] = {e1.x, e1.y, e1.z, e1.w};
      float g0[4], g1[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dwacc += d0[r] * fmaxf(y0[r], 0.f) + d1[r] * fmaxf(y1[r], 0.f);
        g0[r] = y0[r] > 0.f ? wn * d0[r] : 0.f;
        g1[r] = y1[r] > 0.f ? wn * d1[r] : 0.f;
      }
      const unsigned p0 = pack_bf16(g0[0], g0[1]), p1 = pack_bf16(g0[2], g0[3]);
      const unsigned p2 = pack_bf16(g1[0], g1[1]), p3 = pack_bf16(g1[2], g1[3]);
      uint16_t* dst = dsb(t) + (16 * c.wave + i16) * DSR + 4 * G;
      *reinterpret_cast<uint2*>(dst) = make_uint2(p0, p1);
      *reinterpret_cast<uint2*>(dst + 16) = make_uint2(p2, p3);
      // dq_idx^T[dim, head] += K^T dS^T: the K order (keys 4 G .. +3, 16 + 4 G .. +3 in lane
      // group G) is the accumulator order of dS, so dS is the B fragment as it stands
      const bf16x8 bds = __builtin_bit_cast(bf16x8, make_uint4(p0, p1, p2, p3));
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const lds_cptr_t pa = kt + toff[mb];
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)pa);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(pa + 16 * kDI));
        const bf16x8 ka = __builtin_bit_cast(bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        dqa[mb] = mfma16(ka, bds, dqa[mb]);
      }
      // tile t+1 landed; the dS tile is complete for every wave.  Counted: tile t+2's gathers
      // only, so the key-gradient stores issued at the step's start are waited for too (they
      // are done by then).
      iv = ir[step_slot(t + 1) & (2 * kIdxChunk - 1)];
      wait_vm_barrier<GK>();
    };
    for (int t = 0; t < ntiles; t += 3) {
      step(t, 0, 2);
      step(t + 1, 1, 0);
      step(t + 2, 2, 1);
    }
    key_grad(ntiles - 1);
  }
  // dq_idx: lane holds head 16 wave + i16, dims 16 mb + 4 G .. +3
  {
    uint16_t* dqp = a.dq_idx + ((size_t)row * kG + 16 * c.wave + i16) * kDI + 4 * G;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
      *reinterpret_cast<uint2*>(dqp + 16 * mb) =
          make_uint2(pack_bf16(dqa[mb][0], dqa[mb][1]), pack_bf16(dqa[mb][2], dqa[mb][3]));
  }
  dwacc = pair32_sum(pair16_sum(dwacc));
  if (c.lane < 16) a.dw[(size_t)row * kG + 16 * c.wave + c.lane] = dwacc;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no gather or store may outlive the block
}

// dk[k] += sum of the key's slot gradients: 16 lanes per key, 8 dims (16 B) per lane, eight
// entries in flight (the slot gradients are read once: non-temporal loads); each key's sum is
// formed by one lane group, so the update is a plain read-modify-write.
__global__ __launch_bounds__(256) void k_idx_kl_reduce(IdxKlArgs a) {
  const int k = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  if (k >= a.n_k) return;
  const int beg = a.off[k], end = a.off[k + 1];
  if (beg == end) return;
  float s[8] = {};
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  auto src = [&](int e) {   // e: the slot's row in the workspace (row * topkp + slot)
    return reinterpret_cast<const u32x4*>(a.ws_c + (size_t)e * kDI + 8 * l);
  };
  auto add = [&](const u32x4& v) {
    const uint32_t vv[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[2 * j] += __uint_as_float(vv[j] << 16);
      s[2 * j + 1] += __uint_as_float(vv[j] & 0xFFFF0000u);
    }
  };
  // 16 entries in flight per lane group: a chunk's lists belong to few keys (one document's),
  // so about one workgroup per CU has work and the sum is bound by loads in flight
  constexpr int F = 16;
  int p = beg;
  for (; p + F <= end; p += F) {
    u32x4 v[F];
#pragma unroll
    for (int j = 0; j < F; ++j) v[j] = __builtin_nontemporal_load(src(a.list[p + j]));
#pragma unroll
    for (int j = 0; j < F; ++j) add(v[j]);
  }
  for (; p + 4 <= end; p += 4) {
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load(src(a.list[p + j]));
#pragma unroll
    for (int j = 0; j < 4; ++j) add(v[j]);
  }
  for (; p < end; ++p) add(__builtin_nontemporal_load(src(a.list[p])));
  float4* d = reinterpret_cast<float4*>(a.dk + (size_t)k * kDI + 8 * l);
  float4 x0 = d[0], x1 = d[1];
  x0.x += s[0]; x0.y += s[1]; x0.z += s[2]; x0.w += s[3];
  x1.x += s[4]; x1.y += s[5]; x1.z += s[6]; x1.w += s[7];
  d[0] = x0;
  d[1] = x1;
}

// out[0] = sum of loss[0 .. n) in a fixed order (fp64 partials), one workgroup.
__global__ __launch_bounds__(1024) void k_loss_total(const float* loss, int n, float* out) {
  __shared__ double part[16];
  double acc = 0.0;
  for (int i = threadIdx.x; i < n; i += 1024) acc += (double)loss[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < 16; ++w) t += part[w];
    out[0] = (float)t;
  }
}

}  // namespace

// lists: build the chunk's key lists first (false: the caller's are already in a.list / a.off).
// a.psum set: pass 1 takes the target from it (k_idx_kl_p1t).
hipError_t launch_indexer_kl(const IdxKlArgs& a, const KeyListArgs& kl, hipStream_t s, bool lists) {
  if (a.rows == 0) return hipSuccess;
  if (lists) {
    hipError_t e = launch_key_lists(kl, s);
    if (e != hipSuccess) return e;
  }
  if (a.psum)
    k_idx_kl_p1t<<<a.rows, 256, 0, s>>>(a);
  else
    k_idx_kl_p1<<<a.rows, 256, 0, s>>>(a);
  k_idx_kl_p2<<<a.rows, 256, 0, s>>>(a);
  k_idx_kl_reduce<<<(a.n_k + 15) / 16, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_loss_total(const float* loss, int n, float* out, hipStream_t s) {
  k_loss_total<<<1, 1024, 0, s>>>(loss, n, out);
  return hipGetLastError();
}

}  // namespace dsa
