// Sparse multi-query attention over gathered latent rows on gfx950 MFMA.
//
// Page "CANNTorchTitan: DeepSeek-V3.2 32k长序列预训练昇腾优化实践", section
// "SparseLightningIndexerGradKLLoss" (Sparse Flash Attention formula): per query token and
// head, softmax(q K_topk^T / sqrt(d)) over the token's selected keys, applied to the same
// selected rows; under weight absorption key and value are one shared latent row whose first
// d_v columns are the value and whose tail is the rope part.  softmax_max / softmax_sum are
// exported for the indexer-loss boundary (page "context_parallel.md", section "DSA CP").
//
// Mapping: one workgroup per query row, one wave per 32 query heads (4 waves for 128 heads,
// one per SIMD), 32 selected keys per tile.
//   * Gather: the tile's 32 latent rows are copied HBM -> LDS with global_load_lds (16 B per
//     lane, no VGPR staging).  Each wave copies whole rows, so the row base is a scalar.  Rows
//     are stored unpadded with their 16-byte chunks XOR-swizzled by row, which keeps both the
//     16-row logits reads and the 4-row transposing value reads free of bank conflicts.  Empty
//     slots gather row 0 and are masked.
//   * Logits: S^T[key, head] = K_tile (A, from LDS) x Q^T (B) on v_mfma_f32_32x32x16_bf16.  A
//     rows are fed in a fixed key permutation so that each lane's 16 accumulators come out as
//     two runs of 8 consecutive keys of one head -- the B-operand layout of the next product.
//   * Softmax per lane (a lane pair holds one head), exp2 with the scale folded in.  The
//     scaling max is the first valid tile's max; p = exp2(z - m) may exceed 1 (fp32 / bf16
//     keep their relative precision), and only growth past 2^64 is treated as overflow: the
//     row is then marked (a NaN-payload sentinel in its first output element) and a second,
//     normally idle launch recomputes marked rows exactly (row max first).  The accumulator
//     is never rescaled and never carried through a branch.
//   * Output: O^T[col, head] += V^T (A: read straight from the row-major LDS tile with the
//     transposing ds_read_b64_tr_b16) x P^T (B: the lane's bf16 probabilities, no shuffle).
//     O^T is DV/32 M-tiles of 32 value columns; each lane owns one head's columns, so the
//     final 1/l is lane-local.
//   * 128 heads (k_sparse_attn_ring): the 128 x 512 fp32 accumulator of a row fills the AGPRs
//     and all of Q the VGPRs, one wave per SIMD, so nothing hides a wave's own latencies: each
//     step interleaves two independent MFMA streams -- the logits of tile t+1 and the output
//     product of tile t -- with the LDS operand reads, the gather of tile t+3 and the step's
//     bookkeeping in their shadow; the softmax of tile t+1 runs under the second half of the
//     output product.  Four tile buffers (a gather has two steps to land), the slot indices
//     in an LDS ring filled by LDS DMA, one barrier per step.  The output accumulator is
//     pinned to AGPRs and the logits accumulator to VGPRs (asm MFMAs), so no accumulator
//     moves between the files.
//   * Other shapes and the exact pass: three tile buffers, the Q dims past the first 416 staged
//     once in LDS, indices read with scalar loads.
#include "attn_common.h"

namespace dsa {

namespace {

// S^T for one tile (32 keys x the wave's 32 heads), unscaled, -inf at empty slots; `mx`
// receives the lane pair's (= one head's) tile max in scaled log2 units.  The first KQR K
// steps of Q come from qf, the rest from the staged rows in c.qlds.
template <int H, int DQK, int DV, int KQR = AttnCfg<H, DQK, DV>::KSR>
__device__ __forceinline__ f32x16 tile_logits(const AttnArgs& a, const RowCtx& c,
                                              const bf16x8* qf, const uint16_t* tile,
                                              unsigned vmask, float& mx) {
  using C = AttnCfg<H, DQK, DV>;
  static_assert(KQR == C::KSR || KQR == C::KS, "Q split");
  f32x16 s = (f32x16){};
  // row key_perm(hl), logical chunk 2*ks + g at physical chunk (2*ks + g) ^ swz(row): the
  // XOR only touches the low 3 bits, so four per-lane bases (ks mod 4) plus the immediate
  // offset 128 B * (ks / 4) address every step
  const int arow_i = key_perm(c.hl);
  const int asw = C::SWZ ? swz(arow_i) : 0;
  const lds_cptr_t ltile = (lds_cptr_t)tile;
  lds_cptr_t abase[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    abase[j] = ltile + arow_i * C::ROWE + (((2 * j + c.g) ^ asw) - 2 * j) * 8;
  auto arow_at = [&](int ks) { return abase[ks & 3] + ks * 16; };
  const uint16_t* qlrow = KQR < C::KS ? c.qlds + (C::DQL > 0 ? c.head % H : 0) * C::QROWE + c.g * 8
                                       : nullptr;
  // A fragments (and, past the register part of Q, the staged Q fragments) are read one
  // group of K steps ahead of their MFMAs; sched_barrier bounds the live fragments
  constexpr int QG = 3;                 // K steps per prefetch group (36 = 12 x 3)
  constexpr int NG = (C::KS + QG - 1) / QG;
  typedef __attribute__((address_space(3))) const bf16x8* lds_cb8_t;
  bf16x8 af[2][QG], bt[2][QG];
  auto fetch = [&](int gi, int buf) {
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      const int ks = gi * QG + u;
      if (ks < C::KS) {
        af[buf][u] = *(lds_cb8_t)(arow_at(ks));
        if (ks >= KQR) bt[buf][u] = *reinterpret_cast<const bf16x8*>(qlrow + (ks - KQR) * 16);
      }
    }
  };
  fetch(0, 0);
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int cur = gi & 1;
    if (gi + 1 < NG) fetch(gi + 1, cur ^ 1);
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      const int ks = gi * QG + u;
      if (ks < C::KS) {
        const bf16x8 bq = ks < KQR ? qf[ks < KQR ? ks : 0] : bt[cur][u];
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][u], bq, s, 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (vmask != 0xFFFFFFFFu) {   // uniform: only tiles with empty slots pay for the mask
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (!((vmask >> acc_key(r, c.g)) & 1u)) s[r] = kNegInf;
  }
  float m = kNegInf;
#pragma unroll
  for (int r = 0; r < 16; ++r) m = fmaxf(m, s[r]);
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_int(m), __float_as_int(m), false, false);
  // the scale is positive, so scaling after the max keeps the order
  mx = fmaxf(__int_as_float(pr[0]), __int_as_float(pr[1])) * a.scale_log2;
  return s;
}

// O^T += V^T P^T for one tile
template <int H, int DQK, int DV>
__device__ __forceinline__ void tile_pv(const RowCtx& c, const uint16_t* tile, const bf16x8* pf,
                                        f32x16* o) {
  using C = AttnCfg<H, DQK, DV>;
  // transposing read: lane (G = lane/16, i = lane%16) supplies row kbase + i/4, columns
  // cbase + (i%4)*4 .. +3 and receives column cbase + i of rows kbase .. kbase+3
  const int G = c.lane >> 4, i = c.lane & 15;
  // Lane reads row r = kk*16 + (G/2)*8 + i/4 (+4 for the second half), logical chunk
  // 4*mt + low with low = 2*(G&1) + (i&3)/2, at physical chunk 4*(mt ^ s2) + (low ^ s01)
  // where s2 = swz(r) >> 2, s01 = swz(r) & 3.  For even / odd mt that is
  // 4*mt + 4*s2 / 4*mt - 4*s2: two per-lane bases per (kk, half) plus an immediate 64 B * mt.
  // swz ignores row bit 4, so the kk = 1 rows (16 further) share the kk = 0 bases plus an
  // immediate 16-row offset.
  const int low = 2 * (G & 1) + ((i & 3) >> 1);
  const lds_cptr_t ltile = (lds_cptr_t)tile;
  lds_cptr_t vb[2][2];   // [half][mt parity]
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int r = (G >> 1) * 8 + (i >> 2) + hf * 4;
    const int sw = C::SWZ ? swz(r) : 0;
    const lds_cptr_t b = ltile + r * C::ROWE + ((low ^ (sw & 3)) * 8) + (i & 1) * 4;
    vb[hf][0] = b + (sw >> 2) * 32;
    vb[hf][1] = b - (sw >> 2) * 32;
  }
  auto vfrag = [&](int kk, int mt) {
    const int off = kk * 16 * C::ROWE + mt * 32;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(vb[0][mt & 1] + off));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(vb[1][mt & 1] + off));
    return __builtin_bit_cast(bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };
  // K-step outer, M tiles inner: consecutive MFMAs go to different accumulators (two
  // back-to-back MFMAs into one accumulator would wait for each other)
  constexpr int PD = 2;            // fragments read ahead of their MFMA
  constexpr int NIT = 2 * C::MTV;
  bf16x8 vf[PD + 1];
#pragma unroll
  for (int it = 0; it < PD; ++it) vf[it] = vfrag(it / C::MTV, it % C::MTV);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int kk = it / C::MTV, mt = it % C::MTV;
    if (it + PD < NIT) vf[(it + PD) % (PD + 1)] = vfrag((it + PD) / C::MTV, (it + PD) % C::MTV);
    o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[it % (PD + 1)], pf[kk], o[mt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int H, int DQK, int DV>
__device__ __forceinline__ void write_row(const AttnArgs& a, const RowCtx& c, const f32x16* o,
                                          float lsum, float m_used, float m_true) {
  using C = AttnCfg<H, DQK, DV>;
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_int(lsum), __float_as_int(lsum),
                                                   false, false);
  lsum = __int_as_float(pr[0]) + __int_as_float(pr[1]);
  if (c.head >= H) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t* op = a.out + ((size_t)c.row * H + c.head) * DV;
#pragma unroll
  for (int mt = 0; mt < C::MTV; ++mt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int col = mt * 32 + q4 * 8 + c.g * 4;
      const uint32_t lo = (uint32_t)f32_to_bf16(o[mt][q4 * 4 + 0] * inv) |
                          ((uint32_t)f32_to_bf16(o[mt][q4 * 4 + 1] * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(o[mt][q4 * 4 + 2] * inv) |
                          ((uint32_t)f32_to_bf16(o[mt][q4 * 4 + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(op + col) = make_uint2(lo, hi);
    }
  }
  if (c.g == 0) {
    const size_t si = (size_t)c.row * H + c.head;
    const bool any = m_true != kNegInf;
    if (a.smax) a.smax[si] = any ? m_true * kLn2 : kNegInf;
    if (a.ssum) a.ssum[si] = any ? lsum * exp2f(m_used - m_true) : 0.f;
  }
}

// write_row through LDS: the wave's 32 output rows (bf16, 1 KB each) are assembled in `stage`
// (32 KB of LDS no other wave uses any more), then each row leaves as one fully coalesced
// 1 KB store, instead of 64 stores per wave that each touch 32 rows 16 bytes at a time.  In
// `stage` the 16-byte chunk ch of head row hl sits at chunk ch ^ hl: the 8-byte writes of the
// 32 heads of one column block then spread over the banks.
template <int H, int DQK, int DV>
__device__ __forceinline__ void write_row_staged(const AttnArgs& a, const RowCtx& c,
                                                 const f32x16* o, float lsum, float m_used,
                                                 float m_true, uint16_t* stage) {
  using C = AttnCfg<H, DQK, DV>;
  static_assert(H % 32 == 0 && DV == 512, "staged rows are 1 KB, 64 chunks");
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_int(lsum), __float_as_int(lsum),
                                                   false, false);
  lsum = __int_as_float(pr[0]) + __int_as_float(pr[1]);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) u32x2* lds_u2_t;
  typedef __attribute__((address_space(3))) const u32x4* lds_cu4_t;
  const lds_u16_ptr_t srow = (lds_u16_ptr_t)stage + c.hl * DV;
#pragma unroll
  for (int mt = 0; mt < C::MTV; ++mt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int ch = mt * 4 + q4;                       // logical 16-byte chunk (8 columns)
      const uint32_t lo = (uint32_t)f32_to_bf16(o[mt][q4 * 4 + 0] * inv) |
                          ((uint32_t)f32_to_bf16(o[mt][q4 * 4 + 1] * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(o[mt][q4 * 4 + 2] * inv) |
                          ((uint32_t)f32_to_bf16(o[mt][q4 * 4 + 3] * inv) << 16);
      *(lds_u2_t)(srow + (ch ^ c.hl) * 8 + c.g * 4) = (u32x2){lo, hi};
    }
  }
  // each instruction: one head row, lane L carries logical chunk L (own wave's writes only,
  // so the LDS counter orders them).  Non-temporal: the output (2.1 GB at the 32K CP shard) is
  // not read again here, and streamed past the caches it leaves them to the latent rows the
  // other rows gather (8.52 -> 8.40 ms on one box).
  uint16_t* obase = a.out + ((size_t)c.row * H + c.wave * 32) * DV;
#pragma unroll 4
  for (int h = 0; h < 32; ++h) {
    const u32x4 v = *(lds_cu4_t)((lds_u16_ptr_t)stage + h * DV + (c.lane ^ h) * 8);
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(obase + (size_t)h * DV + c.lane * 8));
  }
  if (c.g == 0) {
    const size_t si = (size_t)c.row * H + c.head;
    const bool any = m_true != kNegInf;
    if (a.smax) a.smax[si] = any ? m_true * kLn2 : kNegInf;
    if (a.ssum) a.ssum[si] = any ? lsum * exp2f(m_used - m_true) : 0.f;
  }
}

// Logits and probabilities of one tile for the wave's heads (pf: the lane's 16 keys as the
// B operand of the value product).  Returns whether some head's max exceeded the scaling max
// by more than the fast path's range.
template <int H, int DQK, int DV, int KQR = AttnCfg<H, DQK, DV>::KSR>
__device__ __forceinline__ bool tile_probs(const AttnArgs& a, const RowCtx& c, const bf16x8* qf,
                                           const uint16_t* tile, unsigned vmask, float& m_used,
                                           float& m_true, float& lsum, bf16x8* pf) {
  float mx;
  f32x16 s = tile_logits<H, DQK, DV, KQR>(a, c, qf, tile, vmask, mx);
  m_true = fmaxf(m_true, mx);
  if (m_used == kNegInf) m_used = mx;  // first tile with a valid key
  const bool over = mx > m_used + kOverflowLog2;
  // m_used is still -inf only while every key so far is empty; all logits are then -inf
  const float msub = m_used == kNegInf ? 0.f : m_used;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float ls = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    // p = 2^(z * scale - m) (0 at -inf); the sum uses the same bf16-rounded probabilities
    // that enter the value product, so the output is an exact convex combination of them
    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[r], a.scale_log2, -msub));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], a.scale_log2, -msub));
    const bf16x2 pk = {(__bf16)p0, (__bf16)p1};
    ls = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, ls, false);
    pf[r >> 3][r & 7] = pk[0];
    pf[r >> 3][(r & 7) + 1] = pk[1];
  }
  lsum += ls;
  return over;
}

// Logits, probabilities and the output product of one tile (each wave: its own heads, all
// value columns).
template <int H, int DQK, int DV>
__device__ __forceinline__ bool tile_step(const AttnArgs& a, const RowCtx& c, const bf16x8* qf,
                                          const uint16_t* tile, unsigned vmask, float& m_used,
                                          float& m_true, float& lsum, f32x16* o) {
  bf16x8 pf[2];
  const bool over = tile_probs<H, DQK, DV>(a, c, qf, tile, vmask, m_used, m_true, lsum, pf);
  tile_pv<H, DQK, DV>(c, tile, pf, o);
  return over;
}

// Fast path: tiles in a 3-deep LDS ring (gathers of tiles t+1 and t+2 in flight while tile t
// is computed).  The loop is unrolled by three so every buffer is a distinct LDS object with
// a static role: the compiler then only waits for the gather of the buffer it reads, and
// the explicit vmcnt before each barrier retires exactly this wave's gather of the next
// tile.  The tile count is padded to a multiple of three with empty tiles (p = 0).
// Returns false -- outputs not written -- when some head's max outgrows the scaling range
// (the loop still runs to the end: a second loop exit would keep the accumulator from
// staying in registers).
template <int H, int DQK, int DV, bool AL8>
__device__ __forceinline__ bool accumulate_fast(const AttnArgs& a, const RowCtx& c,
                                                const bf16x8* qf) {
  using C = AttnCfg<H, DQK, DV>;
  f32x16 o[C::MTV];
#pragma unroll
  for (int mt = 0; mt < C::MTV; ++mt) o[mt] = (f32x16){};
  float m_used = kNegInf, m_true = kNegInf, lsum = 0.f;
  bool overflow = false;
  const int ntiles = (c.ntiles + 2) / 3 * 3;
  constexpr int RPW = C::NK / C::NW;
  using TI = TileIdx<H, DQK, DV>;
  unsigned loff[C::NI];
  unsigned wb[3];
  if constexpr (C::FLAT) {
#pragma unroll
    for (int i = 0; i < C::NI; ++i) loff[i] = flat_lane_offset<H, DQK, DV>(c, i);
#pragma unroll
    for (int k = 0; k < 3; ++k)
      wb[k] = (unsigned)(size_t)(lds_u16_ptr_t)(c.buf[k]) + c.wave_u * (RPW * C::ROWE * 2);
  }
  auto gather = [&](const TI& ti, int k) {
    if constexpr (C::FLAT) gather_tile_flat<H, DQK, DV>(a, c, ti, loff, wb[k]);
    else gather_tile_s<H, DQK, DV>(a, c, ti, c.buf[k]);
  };
  const TI i0 = load_tile_idx_s<H, DQK, DV, AL8>(a, c, 0);
  const TI i1 = load_tile_idx_s<H, DQK, DV, AL8>(a, c, 1);
  TI i2 = load_tile_idx_s<H, DQK, DV, AL8>(a, c, 2);
  gather(i0, 0);
  gather(i1, 1);
  if (c.lane == 0) {
    c.vm[0 * C::NW + c.wave] = tile_bits<H, DQK, DV>(a, i0);
    c.vm[1 * C::NW + c.wave] = tile_bits<H, DQK, DV>(a, i1);
  }
  wait_vm_barrier<C::GOPS>();          // tile 0 landed; tile 1 may be in flight

  // step t: fetch the indices of t+3, gather t+2, compute t, then retire this wave's gather
  // of t+1 and meet at the barrier.  `nxt2` holds the indices of t+2 on entry, t+3 on exit.
  auto step = [&](int t, int slot, uint16_t* cur, int ahead2, TI& nxt2) {
    const TI i3 = load_tile_idx_s<H, DQK, DV, AL8>(a, c, t + 3);
    gather(nxt2, ahead2);
    if (c.lane == 0) c.vm[((slot + 2) % 3) * C::NW + c.wave] = tile_bits<H, DQK, DV>(a, nxt2);
    unsigned vmask = 0;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) vmask |= c.vm[slot * C::NW + w] << (w * RPW);
    const bool over = tile_step<H, DQK, DV>(a, c, qf, cur, vmask, m_used, m_true, lsum, o);
    if (c.lane == 0) c.flags[(t & 1) * C::NW + c.wave] = __ballot(over) != 0ull;
    wait_vm_barrier<C::GOPS>();        // tile t+1 landed for every wave; t+2 may be in flight
#pragma unroll
    for (int w = 0; w < C::NW; ++w) overflow |= c.flags[(t & 1) * C::NW + w] != 0;
    nxt2 = i3;
  };
  for (int t = 0; t < ntiles; t += 3) {
    step(t, 0, c.buf[0], 2, i2);
    step(t + 1, 1, c.buf[1], 0, i2);
    step(t + 2, 2, c.buf[2], 1, i2);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no gather may outlive the block
  if (overflow) return false;
  write_row<H, DQK, DV>(a, c, o, lsum, m_used, m_true);
  return true;
}

// ---- four-buffer ring fast path (128 heads) ------------------------------------------------
// Q lives in VGPRs whole (36 fragments), which frees the LDS the staged Q tail took: the tile
// ring is four buffers deep, so a gather has two steps to land instead of one.  Step t forms
// the output product of tile t and the logits of tile t+1 while tile t+2 lands and the gather of
// tile t+3 goes out, then meets the other waves at its only barrier.
// The row's slot indices reach LDS in chunks of eight tiles by LDS DMA (idx_chunk_dma); each
// step reads its two tiles' slots from there: the validity of the tile whose logits it forms
// and the rows of the tile it gathers.
constexpr int kStepFull = 0, kStepNoGather = 1, kStepPvOnly = 2;

// Lane offsets (elements, from a tile's base) of the first two value fragments of a tile,
// [fragment][half]: the addressing of ring_tile's vfrag for fragments 0 and 1, computed once
// per row; those two fragments of each tile are read ahead, across the step's barrier.
template <int H, int DQK, int DV>
__device__ __forceinline__ void vcarry_offsets(const RowCtx& c, unsigned (*vo)[2]) {
  using C = AttnCfg<H, DQK, DV>;
  const int G = c.lane >> 4, i = c.lane & 15;
  const int low = 2 * (G & 1) + ((i & 3) >> 1);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int r = (G >> 1) * 8 + (i >> 2) + hf * 4;
    const int sw = C::SWZ ? swz(r) : 0;
    const int b = r * C::ROWE + ((low ^ (sw & 3)) * 8) + (i & 1) * 4;
    vo[0][hf] = (unsigned)(b + (sw >> 2) * 32);        // fragment 0: mt 0
    vo[1][hf] = (unsigned)(b - (sw >> 2) * 32 + 32);   // fragment 1: mt 1
  }
}

template <int H, int DQK, int DV>
__device__ __forceinline__ bf16x8 vfrag_at(lds_cptr_t tile, const unsigned* vo) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(tile + vo[0]));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(tile + vo[1]));
  return __builtin_bit_cast(bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// One step.  The logits of tile kt (32 keys x the wave's 32 heads, validity bits vmask) are
// interleaved with the output product of the previous tile vt, whose probabilities arrive in
// pf; then the probabilities of kt are formed (returned in pf) while the second half of that
// output product runs.  The gather of a later tile goes out piece by piece between the MFMAs
// (so: byte offsets in kv of this wave's rows of it, wbg: LDS address of the wave's first row
// in the destination buffer).  Each lane owns one head's value columns, as in tile_pv.
// vcarry: the first two value fragments of vt on entry (read before the barrier), those of kt
// on return.  Returns whether some head's max outgrew the scaling range.
// MODE: kStepFull as above; kStepNoGather when no later tile is left to gather; kStepPvOnly
// for the row's last step: the output product of vt alone.
template <int H, int DQK, int DV, int MODE>
__device__ __forceinline__ bool ring_tile(const AttnArgs& a, const RowCtx& c, const bf16x8* qf,
                                          lds_cptr_t ktile, unsigned vmask, lds_cptr_t vtile,
                                          bf16x8* pf, f32x16* o, float& m_used, float& m_true,
                                          float& lsum, const unsigned* so, const unsigned* loff,
                                          unsigned wbg, bf16x8* vcarry, const unsigned (*vco)[2]) {
  using C = AttnCfg<H, DQK, DV>;
  typedef __attribute__((address_space(3))) const bf16x8* lds_cb8_t;
  // logits operands: addressing as in tile_logits
  const int arow_i = key_perm(c.hl);
  const int asw = C::SWZ ? swz(arow_i) : 0;
  lds_cptr_t abase[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    abase[j] = ktile + arow_i * C::ROWE + (((2 * j + c.g) ^ asw) - 2 * j) * 8;
  constexpr int QG = 2;                    // K steps per prefetch group
  constexpr int NG = C::KS / QG;
  static_assert(C::KS % QG == 0, "logits K steps");
  bf16x8 af[2][QG];
  auto fetch = [&](int gi, int buf) {
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      const int ks = gi * QG + u;
      af[buf][u] = *(lds_cb8_t)(abase[ks & 3] + ks * 16);
    }
  };
  // value operands: addressing as in tile_pv
  const int G = c.lane >> 4, i = c.lane & 15;
  const int low = 2 * (G & 1) + ((i & 3) >> 1);
  lds_cptr_t vb[2][2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int r = (G >> 1) * 8 + (i >> 2) + hf * 4;
    const int sw = C::SWZ ? swz(r) : 0;
    const lds_cptr_t b = vtile + r * C::ROWE + ((low ^ (sw & 3)) * 8) + (i & 1) * 4;
    vb[hf][0] = b + (sw >> 2) * 32;
    vb[hf][1] = b - (sw >> 2) * 32;
  }
  auto vfrag = [&](int j) {
    const int kk = j / C::MTV, mt = j % C::MTV;
    const int off = kk * 16 * C::ROWE + mt * 32;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(vb[0][mt & 1] + off));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(vb[1][mt & 1] + off));
    return __builtin_bit_cast(bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };
  constexpr int NP = 2 * C::MTV;           // output-product MFMAs per tile
  constexpr int NPA = 20;                  // of which interleaved with the logits
  constexpr int NPQ = (NP - NPA - 4) / 4;  // per quarter of the softmax
  constexpr int PD = 2;                    // value fragments read ahead of their MFMA
  bf16x8 vf[PD + 1];
  // the accumulator stays in AGPRs (the logits accumulator and every operand in VGPRs): an
  // asm MFMA pins it there, so the register allocator never swaps accumulators between the
  // two files.  Only MFMAs read it until the row ends.
  auto pv = [&](int j) {
    if (j + PD < NP) vf[(j + PD) % (PD + 1)] = vfrag(j + PD);
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                 : "+a"(o[j % C::MTV]) : "v"(vf[j % (PD + 1)]), "v"(pf[j / C::MTV]));
  };
  // one piece (1 KB) of the wave's share of the next gather
  auto gather_piece = [&](int gi) {
    const int j0 = gi * 64 / C::CPR;
    const int b = (j0 + 1) * C::CPR - 64 * gi;
    unsigned ro = so[j0];
    if (b < 64) ro = c.lane >= b ? so[j0 + 1] : ro;
    const unsigned voff = loff[gi] + ro;
    const unsigned m0v = wbg + (unsigned)gi * 1024u;
    const uint16_t* base = a.kv;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(m0v), "v"(voff), "s"(base) : "memory", "m0");
  };

  constexpr bool LOGITS = MODE != kStepPvOnly;
  constexpr bool GATHER = MODE == kStepFull;
  f32x16 s;
  if constexpr (LOGITS) fetch(0, 0);
  // the tile's first two value fragments were read before the step's barrier
  static_assert(PD == 2, "two carried value fragments");
  vf[0] = vcarry[0];
  vf[1] = vcarry[1];
  // the first two output-product MFMAs go ahead of the logits: their operands are in
  // registers, so they cover the LDS latency of the first key fragments
  constexpr int NPRE = LOGITS ? 2 : 0;
  if constexpr (LOGITS) {
    pv(0);
    pv(1);
  }
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int cur = gi & 1;
    if (LOGITS && gi + 1 < NG) fetch(gi + 1, cur ^ 1);
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      const int ks = gi * QG + u;
      if constexpr (!LOGITS) {
#pragma unroll
        for (int j = ks * NPA / C::KS; j < (ks + 1) * NPA / C::KS; ++j) pv(j);
        continue;
      }
      // the logits accumulator is pinned to VGPRs (the AGPRs hold the output accumulator);
      // VALU reads it after the last step: wait out the MFMA write-to-read distance there
      if (ks == 0)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(af[cur][u]), "v"(qf[ks]));
      else if (ks == C::KS - 1)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+v"(s) : "v"(af[cur][u]), "v"(qf[ks]));
      else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(af[cur][u]), "v"(qf[ks]));
      if (GATHER && ks >= 2 && ks < 2 + C::NI) gather_piece(ks - 2);
#pragma unroll
      for (int j = ks * NPA / C::KS; j < (ks + 1) * NPA / C::KS; ++j)
        if (j >= NPRE) pv(j);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!LOGITS) {
#pragma unroll
    for (int j = NPA; j < NP; ++j) pv(j);
    return false;
  }

  // probabilities of kt (as in tile_logits / tile_probs), interleaved with the second half
  // of the output product of vt
  if (vmask != 0xFFFFFFFFu) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (!((vmask >> acc_key(r, c.g)) & 1u)) s[r] = kNegInf;
  }
  float m = kNegInf;
#pragma unroll
  for (int r = 0; r < 16; ++r) m = fmaxf(m, s[r]);
  const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_int(m), __float_as_int(m), false, false);
  const float mx = fmaxf(__int_as_float(pr[0]), __int_as_float(pr[1])) * a.scale_log2;
  pv(NPA + 0);
  pv(NPA + 1);
  pv(NPA + 2);
  pv(NPA + 3);
  __builtin_amdgcn_sched_barrier(0);
  m_true = fmaxf(m_true, mx);
  if (m_used == kNegInf) m_used = mx;
  const bool over = mx > m_used + kOverflowLog2;
  const float msub = m_used == kNegInf ? 0.f : m_used;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float ls = 0.f;
  bf16x8 pn[2];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int r = 4 * q; r < 4 * q + 4; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[r], a.scale_log2, -msub));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[r + 1], a.scale_log2, -msub));
      const bf16x2 pk = {(__bf16)p0, (__bf16)p1};
      // pinned here, between the output-product MFMAs (pure arithmetic would otherwise sink
      // past them to its use at the end of the step)
      asm volatile("" :: "v"(pk));
      ls = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, ls, false);
      pn[r >> 3][r & 7] = pk[0];
      pn[r >> 3][(r & 7) + 1] = pk[1];
    }
#pragma unroll
    for (int j = NPA + 4 + NPQ * q; j < NPA + 4 + NPQ * (q + 1); ++j) pv(j);
    __builtin_amdgcn_sched_barrier(0);
  }
  static_assert(NPA + 4 + NPQ * 4 == NP, "every output-product MFMA issued once");
  lsum += ls;
  pf[0] = pn[0];
  pf[1] = pn[1];
  // the next step's output product is of kt: its first value fragments are read now, ahead
  // of the barrier
  vcarry[0] = vfrag_at<H, DQK, DV>(ktile, vco[0]);
  vcarry[1] = vfrag_at<H, DQK, DV>(ktile, vco[1]);
  return over;
}

// The ring fast path of one row.  bufs: the four tile buffers; idxr: the index ring (chunks 0
// and 1 landed in the row prologue), idxr_lds its LDS byte address; flags: NW ints.
// Tiles past the row's last valid slot are neither gathered nor computed: the last two steps
// with logits gather nothing, and the row's last step is the output product of its last tile
// alone.  Returns false -- outputs not written -- when some head's max outgrew the scaling
// range (the loop still runs to the end: a second loop exit would keep the accumulator from
// staying in registers).
template <int H, int DQK, int DV>
__device__ __forceinline__ bool accumulate_ring(const AttnArgs& a, const RowCtx& c,
                                                const bf16x8* qf, uint16_t* const* bufs,
                                                const int32_t* idxr, unsigned idxr_lds,
                                                int* flags) {
  using C = AttnCfg<H, DQK, DV>;
  constexpr int RPW = C::RPW;
  static_assert(RPW == 8 && C::NW == 4 && C::NK == 32, "ring slot layout");
  f32x16 o[C::MTV];
#pragma unroll
  for (int mt = 0; mt < C::MTV; ++mt) o[mt] = (f32x16){};
  float m_used = kNegInf, m_true = kNegInf, lsum = 0.f;
  unsigned loff[C::NI];
#pragma unroll
  for (int i = 0; i < C::NI; ++i) loff[i] = flat_lane_offset<H, DQK, DV>(c, i);
  unsigned wb[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    wb[k] = (unsigned)(size_t)(lds_u16_ptr_t)(bufs[k]) + c.wave_u * (RPW * C::ROWE * 2);
  const lds_ci32_t ir = (lds_ci32_t)idxr;
  // slot read by this lane for step t: lanes 0..31 the tile whose logits the step forms (t+1),
  // lanes 32..63 the tile it gathers (t+3)
  auto step_slot = [&](int t) { return (t + 1 + 2 * (c.lane >> 5)) * C::NK + (c.lane & 31); };

  // tiles 0, 1, 2 from chunk 0
  unsigned mask0;
  {
    const int s0 = c.lane, s1 = 2 * C::NK + (c.lane & 31);
    unsigned off0, off1, so[RPW];
    mask0 = (unsigned)decode_slot<H, DQK, DV>(a, ir[s0], s0, off0);
    (void)decode_slot<H, DQK, DV>(a, ir[s1], s1, off1);
    wave_row_offsets<H, DQK, DV>(c, off0, 0, so);
    gather_tile_flat_so<H, DQK, DV>(a, c, so, loff, wb[0]);
    wave_row_offsets<H, DQK, DV>(c, off0, 32, so);
    gather_tile_flat_so<H, DQK, DV>(a, c, so, loff, wb[1]);
    wave_row_offsets<H, DQK, DV>(c, off1, 32, so);
    gather_tile_flat_so<H, DQK, DV>(a, c, so, loff, wb[2]);
  }
  wait_vm_barrier<2 * C::NI>();        // tile 0 landed; tiles 1 and 2 may be in flight
  bf16x8 pf[2];
  // overflow of this wave's heads, combined over the waves once the row is done
  bool over_any = tile_probs<H, DQK, DV, C::KS>(a, c, qf, bufs[0], mask0, m_used, m_true, lsum,
                                                 pf);
  int iv = ir[step_slot(0)];
  wait_vm_barrier<C::NI>();            // tile 1 landed
  unsigned vco[2][2];
  vcarry_offsets<H, DQK, DV>(c, vco);
  bf16x8 vcarry[2] = {vfrag_at<H, DQK, DV>((lds_cptr_t)bufs[0], vco[0]),
                      vfrag_at<H, DQK, DV>((lds_cptr_t)bufs[0], vco[1])};

  // ring slots (LDS addresses, gather bases) rotating in registers: the accumulator keeps its
  // registers across iterations, and no indexed private array (scratch memory) is involved
  lds_cptr_t bv = (lds_cptr_t)bufs[0], bk = (lds_cptr_t)bufs[1], bl = (lds_cptr_t)bufs[2],
             bg = (lds_cptr_t)bufs[3];
  unsigned wv = wb[0], wk = wb[1], wl = wb[2], wg = wb[3];
  auto rotate = [&]() {
    const lds_cptr_t b0 = bv;
    bv = bk;
    bk = bl;
    bl = bg;
    bg = b0;
    const unsigned w0 = wv;
    wv = wk;
    wk = wl;
    wl = wg;
    wg = w0;
  };
  // step t: output product of t, logits of t+1, gather of t+3 into the buffer tile t-1 left;
  // then wait for this wave's gather of t+2 and meet at the barrier
  auto step = [&](auto mode, int t) {
    constexpr int MODE = decltype(mode)::value;
    unsigned vmask = 0u;
    unsigned so[RPW] = {};
    if constexpr (MODE != kStepPvOnly) {
      unsigned off;
      vmask = (unsigned)decode_slot<H, DQK, DV>(a, iv, step_slot(t), off);
      if constexpr (MODE == kStepFull) {
        wave_row_offsets<H, DQK, DV>(c, off, 32, so);
        // chunk t/8 + 1 (first needed by the gather of step t + 5) into the ring half that
        // chunk t/8 - 1 left; issued before the step's gather, so the step's final wait
        // covers it
        if ((t & 7) == 0 && t > 0) idx_chunk_dma<H, DQK, DV>(a, c, t / 8 + 1, idxr_lds);
      }
    }
    over_any |= ring_tile<H, DQK, DV, MODE>(a, c, qf, bk, vmask, bv, pf, o, m_used, m_true, lsum,
                                            so, loff, wg, vcarry, vco);
    if constexpr (MODE != kStepPvOnly) {
      iv = ir[step_slot(t + 1) & (2 * kIdxChunk - 1)];
      if constexpr (MODE == kStepFull) wait_vm_barrier<C::NI>();   // t+2 landed, t+3 in flight
      else wait_vm_barrier<0>();
    }
  };
  const int T = c.ntiles;
  for (int t = 0; t < T - 3; ++t) {
    step(std::integral_constant<int, kStepFull>{}, t);
    rotate();
  }
  for (int t = max(T - 3, 0); t < T - 1; ++t) {
    step(std::integral_constant<int, kStepNoGather>{}, t);
    rotate();
  }
  if (T >= 1) step(std::integral_constant<int, kStepPvOnly>{}, T - 1);
  // no gather may outlive the block; the accumulator's last MFMA writes are read by VALU next
  asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  if (c.lane == 0) flags[c.wave] = __ballot(over_any) != 0ull;
  __syncthreads();
  bool overflow = false;
#pragma unroll
  for (int w = 0; w < C::NW; ++w) overflow |= flags[w] != 0;
  if (overflow) return false;
  // the ring is free (every wave is past the loop): one 36 KB buffer per wave for the staging
  static_assert(C::TILE >= 32 * DV, "staging space");
  uint16_t* const stg = c.wave_u == 0 ? bufs[0]
                      : (c.wave_u == 1 ? bufs[1] : (c.wave_u == 2 ? bufs[2] : bufs[3]));
  write_row_staged<H, DQK, DV>(a, c, o, lsum, m_used, m_true, stg);
  return true;
}

// Exact path: scaling max fixed to the row max (computed beforehand), two buffers, full
// waits; only runs for rows the fast path gave up on.
template <int H, int DQK, int DV>
__device__ __forceinline__ void accumulate_exact(const AttnArgs& a, const RowCtx& c,
                                                 const bf16x8* qf, float m_fix) {
  using C = AttnCfg<H, DQK, DV>;
  f32x16 o[C::MTV];
#pragma unroll
  for (int mt = 0; mt < C::MTV; ++mt) o[mt] = (f32x16){};
  float m_used = m_fix, m_true = kNegInf, lsum = 0.f;
  __syncthreads();
  for (int t = 0; t < c.ntiles; ++t) {
    gather_tile<H, DQK, DV>(a, c, t, c.buf[0]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    (void)tile_step<H, DQK, DV>(a, c, qf, c.buf[0], tile_vmask<H, DQK, DV>(a, c, t), m_used,
                                m_true, lsum, o);
    __syncthreads();
  }
  write_row<H, DQK, DV>(a, c, o, lsum, m_used, m_true);
}

// One row of the fast path or of the exact pass (block index bi of nblk; the LDS arrays are
// the kernel's).
template <int H, int DQK, int DV, bool EXACT, bool AL8>
__device__ __forceinline__ void attn_row(const AttnArgs& a, int bi, int nblk, uint16_t* kv0,
                                         uint16_t* kv1, uint16_t* kv2, uint16_t* qlds, int* flags,
                                         unsigned* vmring, int* s_last) {
  using C = AttnCfg<H, DQK, DV>;
  // XCD-aware row order: consecutive blocks go to different XCDs; give each XCD a contiguous
  // run of rows (neighbouring queries tend to select neighbouring keys).
  int blk = EXACT ? bi : (int)blockIdx.x;
  if (!EXACT && a.xcd_remap) blk = (blk & 7) * (nblk >> 3) + (blk >> 3);
  RowCtx c;
  if (a.use_segs) {
    const int g0 = seg_of_block(a.segs, blk);
    c.row = a.segs.q_start[g0] + (blk - a.segs.blk_off[g0]);
  } else {
    c.row = blk;
  }
  if (EXACT) {
    __syncthreads();   // the previous row's LDS use is over
    if (a.out[(size_t)c.row * H * DV] != kOverflowMark) return;
  }
  c.tid = threadIdx.x;
  c.lane = c.tid & 63;
  c.wave = c.tid >> 6;
  c.wave_u = __builtin_amdgcn_readfirstlane(c.wave);
  c.hl = c.lane & 31;
  c.g = c.lane >> 5;
  c.head = c.wave * 32 + c.hl;
  c.idx_row = a.idx + (size_t)c.row * a.topk;
  c.buf[0] = kv0;
  c.buf[1] = kv1;
  c.buf[2] = kv2;
  c.qlds = qlds;
  c.flags = flags;
  c.vm = vmring;

  // Row prologue in one memory round trip: the staged part of Q goes to LDS by LDS DMA, and
  // the register part of Q and the index scan (tiles past the last valid slot are never
  // gathered or computed) are issued before anything waits.
  static_assert(EXACT || !C::PIPE, "the 128-head fast path is k_sparse_attn_ring");
  stage_q_tail<H, DQK, DV>(a, c, qlds);
  bf16x8 qf[C::KSR];
  load_q<H, DQK, DV>(a, c, qf);
  int last = thread_last_valid<C::NT>(c.idx_row, a.topk, a.n_k, c.tid);
  last = (int)wave_max_u32((unsigned)(last + 1)) - 1;   // (last >= -1)
  if (c.lane == 0) s_last[c.wave] = last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // staged Q landed (DMA is not tracked)
  __syncthreads();
  last = -1;
#pragma unroll
  for (int w = 0; w < C::NW; ++w) last = max(last, s_last[w]);
  c.ntiles = (last + C::NK) / C::NK;

  // compiler-visible vmcnt(0) (exp/lgkm counters left alone): the Q loads are done before the
  // gather ring starts, so the compiler adds no waits for them inside the loop
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if (EXACT) {
    // row max from the logits alone, then the exact accumulation
    float m_fix = kNegInf;
    __syncthreads();
    for (int t = 0; t < c.ntiles; ++t) {
      gather_tile<H, DQK, DV>(a, c, t, c.buf[0]);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      float mx;
      (void)tile_logits<H, DQK, DV>(a, c, qf, c.buf[0], tile_vmask<H, DQK, DV>(a, c, t), mx);
      m_fix = fmaxf(m_fix, mx);
      __syncthreads();
    }
    accumulate_exact<H, DQK, DV>(a, c, qf, m_fix);
  } else {
    const bool done = accumulate_fast<H, DQK, DV, AL8>(a, c, qf);
    if (!done && c.tid == 0) a.out[(size_t)c.row * H * DV] = kOverflowMark;
  }
}

}  // namespace

// The fast path of the 128-head shape: a block per row, the four-buffer tile ring, the index
// ring and all of Q in registers (no staged Q).
template <int H, int DQK, int DV>
__global__ __launch_bounds__(64 * ((H + 31) / 32)) void k_sparse_attn_ring(AttnArgs a) {
  using C = AttnCfg<H, DQK, DV>;
  static_assert(C::PIPE, "ring path shape");
  __shared__ __attribute__((aligned(16))) uint16_t kv0[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t kv1[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t kv2[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t kv3[C::TILE];
  __shared__ __attribute__((aligned(16))) int32_t idxr[2 * kIdxChunk];
  __shared__ int flags[C::NW];
  __shared__ int s_last[C::NW];

  // XCD-aware row order, as in attn_row
  int blk = (int)blockIdx.x;
  if (a.xcd_remap) blk = (blk & 7) * ((int)gridDim.x >> 3) + (blk >> 3);
  RowCtx c;
  if (a.use_segs) {
    const int g0 = seg_of_block(a.segs, blk);
    c.row = a.segs.q_start[g0] + (blk - a.segs.blk_off[g0]);
  } else {
    c.row = blk;
  }
  c.tid = threadIdx.x;
  c.lane = c.tid & 63;
  c.wave = c.tid >> 6;
  c.wave_u = __builtin_amdgcn_readfirstlane(c.wave);
  c.hl = c.lane & 31;
  c.g = c.lane >> 5;
  c.head = c.wave * 32 + c.hl;
  c.idx_row = a.idx + (size_t)c.row * a.topk;
  c.buf[0] = c.buf[1] = c.buf[2] = nullptr;
  c.qlds = nullptr;
  c.flags = flags;
  c.vm = nullptr;
  uint16_t* const bufs[4] = {kv0, kv1, kv2, kv3};
  const unsigned idxr_lds = (unsigned)(size_t)(__attribute__((address_space(3))) int32_t*)idxr;

  // Row prologue in one memory round trip: the first two index chunks go to LDS by LDS DMA,
  // and so do the wave's 32 Q rows (36 KB, into the ring buffer numbered like the wave), while
  // the index scan loads.  Q travels through LDS because the register layout wants, per load
  // instruction, 32 bytes of each of 32 head rows: fetched directly that is 32 cache lines per
  // instruction, against 9 for the coalesced 1 KB pieces of the DMA.  The Q rows are stored
  // like tile rows (chunks swizzled by swz), so the fragment reads below are free of bank
  // conflicts.
  idx_chunk_dma<H, DQK, DV>(a, c, 0, idxr_lds);
  idx_chunk_dma<H, DQK, DV>(a, c, 1, idxr_lds);
  static_assert(C::TILE == 32 * DQK && C::SWZ, "a wave's Q rows fill one ring buffer");
  uint16_t* const qbuf = c.wave_u == 0 ? kv0 : (c.wave_u == 1 ? kv1 : (c.wave_u == 2 ? kv2 : kv3));
  {
    const uint16_t* qsrc = a.q + ((size_t)c.row * H + c.wave_u * 32) * DQK;
    const unsigned qdst = (unsigned)(size_t)(lds_u16_ptr_t)qbuf;
#pragma unroll 4
    for (int i = 0; i < C::TILE * 2 / 1024; ++i) {
      const int f = i * 64 + c.lane;            // physical chunk f % CPR of row f / CPR
      const int r = f / C::CPR, ch = f - r * C::CPR;
      const unsigned voff = (unsigned)(r * C::CPR + (ch ^ swz(r))) * 16u;
      const unsigned m0v = qdst + (unsigned)i * 1024u;
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(m0v), "v"(voff), "s"(qsrc) : "memory", "m0");
    }
  }
  int last = thread_last_valid<C::NT>(c.idx_row, a.topk, a.n_k, c.tid);
  last = (int)wave_max_u32((unsigned)(last + 1)) - 1;   // (last >= -1)
  if (c.lane == 0) s_last[c.wave] = last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // index chunks landed (DMA is not tracked)
  __syncthreads();
  last = -1;
#pragma unroll
  for (int w = 0; w < C::NW; ++w) last = max(last, s_last[w]);
  c.ntiles = (last + C::NK) / C::NK;
  // compiler-visible vmcnt(0): the index scan loads are done before the gather ring starts,
  // so the compiler adds no waits for them inside the loop
  __builtin_amdgcn_s_waitcnt(0x0F70);
  // the wave's Q fragments: head row hl, logical chunk 2 ks + g
  bf16x8 qf[C::KS];
  {
    typedef __attribute__((address_space(3))) const bf16x8* lds_cb8_t;
    const int sw = swz(c.hl);
    const lds_cptr_t qrow = (lds_cptr_t)qbuf + c.hl * C::ROWE;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = *(lds_cb8_t)(qrow + ((2 * ks + c.g) ^ sw) * 8);
  }
  __syncthreads();   // every wave holds its Q: the ring buffers take tiles from here on
  const bool done = accumulate_ring<H, DQK, DV>(a, c, qf, bufs, idxr, idxr_lds, flags);
  if (!done && c.tid == 0) a.out[(size_t)c.row * H * DV] = kOverflowMark;
}

// EXACT = false: the fast path over blocks = rows (a block per row).
// EXACT = true: a grid-stride pass that recomputes only rows the fast path marked, with the
// row max found first so nothing can overflow.
template <int H, int DQK, int DV, bool EXACT, bool AL8>
__global__ __launch_bounds__(64 * ((H + 31) / 32)) void k_sparse_attn(AttnArgs a) {
  using C = AttnCfg<H, DQK, DV>;
  __shared__ __attribute__((aligned(16))) uint16_t kv0[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t kv1[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t kv2[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t qlds[C::QLDS];
  __shared__ int flags[2 * C::NW];
  __shared__ unsigned vmring[3 * C::NW];
  __shared__ int s_last[C::NW];

  const int nblk = EXACT ? a.nrows : (int)gridDim.x;
  // one row per block on the fast path (no loop around it: per-lane values would be hoisted
  // out of a loop and spilled, and their reloads would add memory round trips to the row
  // prologue); the exact pass walks the rows in a grid-stride loop
  if constexpr (EXACT) {
    // block b owns rows b, b + G, b + 2G, ... (G = gridDim.x); their marks are checked C::NT
    // at a time, one per thread, so a group with no marked row (the normal case) costs one
    // load per thread
    const int G = (int)gridDim.x;
    for (int j0 = 0; (int)blockIdx.x + j0 * G < nblk; j0 += C::NT) {
      const int bi = (int)blockIdx.x + (j0 + (int)threadIdx.x) * G;
      bool marked = false;
      if (bi < nblk) {
        int row = bi;
        if (a.use_segs) {
          const int g = seg_of_block(a.segs, bi);
          row = a.segs.q_start[g] + (bi - a.segs.blk_off[g]);
        }
        marked = a.out[(size_t)row * H * DV] == kOverflowMark;
      }
      if (!__syncthreads_or(marked)) continue;
      for (int k = 0; k < C::NT && (int)blockIdx.x + (j0 + k) * G < nblk; ++k)
        attn_row<H, DQK, DV, EXACT, AL8>(a, (int)blockIdx.x + (j0 + k) * G, nblk, kv0, kv1, kv2,
                                         qlds, flags, vmring, s_last);
    }
  } else {
    attn_row<H, DQK, DV, EXACT, AL8>(a, (int)blockIdx.x, nblk, kv0, kv1, kv2, qlds, flags, vmring,
                                     s_last);
  }
}

hipError_t launch_sparse_attn(const AttnArgs& a, int h, int d_qk, int d_v, int nblocks,
                              hipStream_t s) {
  if (nblocks == 0) return hipSuccess;
  AttnArgs ax = a;
  ax.nrows = nblocks;
  const int exact_grid = nblocks < 1024 ? nblocks : 1024;
  if (h == 128 && d_qk == 576 && d_v == 512) {
    k_sparse_attn_ring<128, 576, 512><<<nblocks, 256, 0, s>>>(ax);
    k_sparse_attn<128, 576, 512, true, false><<<exact_grid, 256, 0, s>>>(ax);
  } else if (h == 8 && d_qk == 80 && d_v == 64) {
    k_sparse_attn<8, 80, 64, false, false><<<nblocks, 64, 0, s>>>(ax);
    k_sparse_attn<8, 80, 64, true, false><<<exact_grid, 64, 0, s>>>(ax);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dsa
