// Sparse multi-query attention backward on gfx950 MFMA.
//
// Page "CANNTorchTitan: DeepSeek-V3.2 32k长序列预训练昇腾优化实践", section
// "SparseFlashAttentionGrad": the selected latent rows are gathered again, the probabilities
// P are recomputed from the forward's softmax statistics, dP = dY V_sel^T,
// dS = P * (dP - D) with D = rowsum(dY * out) (the FlashSoftmaxGrad step),
// dQ = dS K_sel / sqrt(d), and the key / value gradients dS^T Q / sqrt(d) and P^T dY are
// scatter-added into the selected rows.  Under weight absorption key and value share one
// latent row, so both land in one fp32 dKV row (the value part in its first d_v columns).
//
// Three kernels over a chunk of query rows, one workgroup per row and four waves:
//   * k_attn_bwd_p_ring: the forward's ring design (index ring, four tile buffers); every
//     16-dim A fragment of the key tile feeds both S^T = K Q^T and (first d_v dims)
//     dP^T = V dY^T, so the tile is read from LDS once for both.  Each wave owns 32 heads.
//     It writes P and softmax_scale * dS as bf16 to a [row][slot][head] workspace (zero at
//     empty slots), the element work of one tile interleaved with the products of the next.
//     For the combined backward + indexer-loss call it also writes each slot's fp32 sum of P
//     over the heads (the indexer loss's target, page section
//     "SparseLightningIndexerGradKLLoss"), from the fp32 probabilities before rounding.
//   * k_attn_bwd_dq_ring: gathers the key tiles again (index ring) together with the
//     tile's dS block (both by LDS DMA) and accumulates dQ^T[dim, head] += K^T dS^T, each
//     wave over 144 latent dims and all 128 heads (K^T and dS^T read with the transposing
//     LDS read).
//   * k_attn_bwd_dkv_part: no gather.  Each wave owns 144 of the 576 latent dims and holds
//     Q[:, dims] and dY[:, dims] for all 128 heads as MFMA fragments (staged through LDS once
//     per row); per tile it forms C[slot, dims] = dS^T Q + P^T dY on 16x16x32 MFMA with the
//     P / dS tile streamed through an LDS ring by LDS DMA, and writes every slot's 576-wide
//     contribution as bf16 with plain stores.
//   * The contributions are then summed per key: the chunk's (row, slot) entries are counted
//     per key, prefix-summed and scattered into per-key lists (integer atomics on counters
//     only), and k_bwd_reduce gives each key one wave that sums its list in fp32 and adds the
//     result to dKV.  Float atomics on dKV would cost one atomic per element (576 per
//     selected key), and the L2 retires those about five times slower than plain stores.
#include <algorithm>

#include "attn_common.h"

namespace dsa {

namespace {

constexpr float kLog2e = 1.44269504088896340736f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------------
// k_attn_bwd_p_ring: the same outputs for the 128-head shape, on the forward's ring design
// ---------------------------------------------------------------------------------------
//
// Step t of a row forms P and softmax_scale * dS of tile t from its S^T / dP^T accumulators
// (computed in step t-1) and stores them, interleaved with the S^T / dP^T products of tile
// t+1, while the gather of tile t+4 goes out between the first MFMAs; then tile t+2 is waited
// for and the block meets at one barrier.  Four tile buffers (the wave's Q rows pass through
// them first; in step t they hold tiles t+1 .. t+3 and take t+4 into tile t's), the slot
// indices in the LDS index ring, all of Q in AGPRs (read by the MFMAs from there) and dY in
// VGPRs, the two tiles' accumulators alternating between two AGPR sets (about 200 registers
// in each file).  Every step has the
// same memory instructions: near the row's end the gathers fetch row 0 for slots past the
// list, and the last step's products run on whatever the buffer holds (their accumulators
// are never read).
//
// The wait for a tile counts only the loads issued after its gather (the next two gathers and
// any index chunk), so the P / dS stores issued in between are waited for too; they go out
// spread over the step, and by its end they are done.

constexpr int kBwdGatherKs0 = 1;       // K step of the first gather piece (one per K step)
constexpr int kBwdParts = 16;          // element parts per tile: one accumulator register each
constexpr int kBwdPartKs0 = 2, kBwdPartKsStride = 2;   // K step after which part r runs

// Per-row constants of the element step.
struct BwdRowK {
  float msub, invl, D;
  unsigned vo0, vo4;   // store byte offsets (from the tile's row base) of parts 0-3 and 4-7
  unsigned sel;        // byte selector assembling a head pair's dword (differs for odd heads)
};

// DPP source modes of the 16-lane sums: lane l reads lane l ^ 1, l ^ 2, (l & ~7) | (7 - l % 8)
// and l ^ 8 of its 16-lane row; row_shr:1 moves every lane's value one lane up the row.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRor8 = 0x128, kDppShl4 = 0x104,
              kDppShr4 = 0x114;
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// x of lane L ^ 4 within each row of 16: banks 1 and 3 (lanes 4-7, 12-15) take lane L - 4,
// banks 0 and 2 lane L + 4
__device__ __forceinline__ float dpp_xor4(float x) {
  const int lo = __builtin_amdgcn_update_dpp(0, __float_as_int(x), kDppShr4, 0xF, 0xA, false);
  return __int_as_float(__builtin_amdgcn_update_dpp(lo, __float_as_int(x), kDppShl4, 0xF, 0x5, false));
}

// One ring step (PARTS) or the row prologue's products of tile 0 alone (no parts, no gather).
// PSUM: also the sum over the 16 heads of each 16-lane row of P for every part, by a
// transposing butterfly over the parts as they come (partners lane ^ 1, ^ 2, ^ 4, ^ 8: at
// each level a lane keeps the half of the pending sums its lane bit names and adds the
// partner's copy of it), so after the tile row position i holds part i's sum in hsum.
template <int H, int DQK, int DV, bool PARTS, bool PSUM = false>
__device__ __forceinline__ void bwd_ring_tile(const AttnBwdArgs& a, const RowCtx& c,
                                              const bf16x8* qf, const bf16x8* dof,
                                              lds_cptr_t ktile, f32x16& s_nx, f32x16& d_nx,
                                              const f32x16& s_cu, const f32x16& d_cu,
                                              unsigned vmask, bool store,
                                              const uint16_t* pt, const uint16_t* dt,
                                              const BwdRowK& k,
                                              const unsigned* so, const unsigned* loff,
                                              unsigned wbg, float& hsum) {
  using C = AttnCfg<H, DQK, DV>;
  constexpr int KSV = DV / 16;
  typedef __attribute__((address_space(3))) const bf16x8* lds_cb8_t;
  static_assert(kBwdPartKs0 + kBwdPartKsStride * (kBwdParts - 1) < C::KS, "parts placement");
  static_assert(kBwdGatherKs0 + C::NI <= C::KS, "gather placement");
  const int arow_i = key_perm(c.hl);
  const int asw = C::SWZ ? swz(arow_i) : 0;
  lds_cptr_t abase[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    abase[j] = ktile + arow_i * C::ROWE + (((2 * j + c.g) ^ asw) - 2 * j) * 8;
  constexpr int QG = 2;                    // K steps per group (one sched region)
  constexpr int NG = C::KS / QG;
  constexpr int PF = 2;                    // groups of key fragments read ahead
  static_assert(C::KS % QG == 0, "K steps");
  bf16x8 af[PF + 1][QG];
  auto fetch = [&](int gi, int buf) {
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      const int ks = gi * QG + u;
      af[buf][u] = *(lds_cb8_t)(abase[ks & 3] + ks * 16);
    }
  };
  auto gather_piece = [&](int gi) {
    const int j0 = gi * 64 / C::CPR;
    const int b = (j0 + 1) * C::CPR - 64 * gi;
    unsigned ro = so[j0];
    if (b < 64) {
      // (opaque to the optimiser: a select between two loads of so[] would otherwise become
      // one load at a lane-dependent index, a chain of compares over all of so[])
      unsigned r1 = so[j0 + 1];
      asm("" : "+s"(r1));
      ro = c.lane >= b ? r1 : ro;
    }
    const unsigned voff = loff[gi] + ro;
    const unsigned m0v = wbg + (unsigned)gi * 1024u;
    const uint16_t* base = a.kv;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(m0v), "v"(voff), "s"(base) : "memory", "m0");
  };
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  // part r: accumulator register r of tile t (key acc_key(r, g)): P and dS of the lane's
  // head; after an odd r the pair (r-1, r) is stored: the head pair's dword assembled across
  // the lane pair, one store per tensor
  float p0 = 0.f, g0 = 0.f;
  float hx1 = 0.f, hx2 = 0.f, hx3 = 0.f;   // pending butterfly sums (PSUM)
  auto part = [&](int r) {
    // validity of the key per lane half, as a lane mask (the list's validity bits are
    // wave-uniform): lanes 0-31 hold key acc_key(r, 0), lanes 32-63 acc_key(r, 1)
    const uint64_t m = ((vmask >> acc_key(r, 0)) & 1u ? 0xFFFFFFFFull : 0ull) |
                       ((vmask >> acc_key(r, 1)) & 1u ? 0xFFFFFFFF00000000ull : 0ull);
    // the accumulators are read here, not all at the step's start (32 more live VGPRs)
    float x, y;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(s_cu[r]));
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(y) : "a"(d_cu[r]));
    float p = __builtin_amdgcn_exp2f(fmaf(x, a.scale_log2, -k.msub)) * k.invl;
    p = __builtin_amdgcn_inverse_ballot_w64(m) ? p : 0.f;
    const float g = a.scale * p * (y - k.D);
    if constexpr (PSUM) {
      static_assert(kBwdParts == 16, "one butterfly level per bit of the part index");
      // lane-bit masks as SGPR pairs: lanes with bit 0 / 1 / 2 / 3 set
      const bool b0 = __builtin_amdgcn_inverse_ballot_w64(0xAAAAAAAAAAAAAAAAull);
      const bool b1 = __builtin_amdgcn_inverse_ballot_w64(0xCCCCCCCCCCCCCCCCull);
      const bool b2 = __builtin_amdgcn_inverse_ballot_w64(0xF0F0F0F0F0F0F0F0ull);
      const bool b3 = __builtin_amdgcn_inverse_ballot_w64(0xFF00FF00FF00FF00ull);
      if (r & 1) {   // parts r-1 (p0) and r over lane pairs
        const float x1 = (b0 ? p : p0) + dpp_mov<kDppXor1>(b0 ? p0 : p);
        if ((r & 2) == 0) {
          hx1 = x1;
        } else {     // parts r-3 .. r over lane quads
          const float x2 = (b1 ? x1 : hx1) + dpp_mov<kDppXor2>(b1 ? hx1 : x1);
          if ((r & 4) == 0) {
            hx2 = x2;
          } else {   // parts r-7 .. r over lane octets
            const float x3 = (b2 ? x2 : hx2) + dpp_xor4(b2 ? hx2 : x2);
            if ((r & 8) == 0) hx3 = x3;
            else hsum = (b3 ? x3 : hx3) + dpp_mov<kDppRor8>(b3 ? hx3 : x3);
          }
        }
      }
    }
    if ((r & 1) == 0) {
      p0 = p;
      g0 = g;
      return;
    }
    const int j = r >> 1;
    const float p1 = p, g1 = g;
    const bf16x2v pk = {(__bf16)p0, (__bf16)p1};
    const bf16x2v gk = {(__bf16)g0, (__bf16)g1};
    const unsigned pu = __builtin_bit_cast(unsigned, pk), gu = __builtin_bit_cast(unsigned, gk);
    const unsigned py = (unsigned)__builtin_amdgcn_mov_dpp((int)pu, 0xB1, 0xF, 0xF, false);
    const unsigned gy = (unsigned)__builtin_amdgcn_mov_dpp((int)gu, 0xB1, 0xF, 0xF, false);
    const unsigned vp = __builtin_amdgcn_perm(py, pu, k.sel);
    const unsigned vd = __builtin_amdgcn_perm(gy, gu, k.sel);
    const unsigned vo = j < 4 ? k.vo0 : k.vo4;
    const uint16_t* b0 = pt;
    const uint16_t* b1 = dt;
    // non-temporal: P and dS (34 GB at the 32K varlen shape) stream past the caches that
    // hold the gathered latent rows and the next rows' Q / dY
    if (store) {
      asm volatile("global_store_dword %0, %1, %2 offset:%3 nt"
                   :: "v"(vo), "v"(vp), "s"(b0), "n"((j & 3) * 4 * H) : "memory");
      asm volatile("global_store_dword %0, %1, %2 offset:%3 nt"
                   :: "v"(vo), "v"(vd), "s"(b1), "n"((j & 3) * 4 * H) : "memory");
    }
  };

#pragma unroll
  for (int gi = 0; gi < PF; ++gi) fetch(gi, gi);
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int cur = gi % (PF + 1);
    if (gi + PF < NG) fetch(gi + PF, (gi + PF) % (PF + 1));
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      const int ks = gi * QG + u;
      if (ks == 0)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                     : "=&a"(s_nx) : "v"(af[cur][u]), "a"(qf[ks]));
      else if (ks == C::KS - 1)   // VALU reads the accumulators next step: wait out the MFMA
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(s_nx) : "v"(af[cur][u]), "a"(qf[ks]));
      else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+a"(s_nx) : "v"(af[cur][u]), "a"(qf[ks]));
      if (ks == 0)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
                     : "=&a"(d_nx) : "v"(af[cur][u]), "v"(dof[0]));
      else if (ks < KSV)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+a"(d_nx) : "v"(af[cur][u]), "v"(dof[ks < KSV ? ks : 0]));
      if constexpr (PARTS) {
        if (ks >= kBwdGatherKs0 && ks < kBwdGatherKs0 + C::NI) gather_piece(ks - kBwdGatherKs0);
        if (ks >= kBwdPartKs0 && (ks - kBwdPartKs0) % kBwdPartKsStride == 0 &&
            (ks - kBwdPartKs0) / kBwdPartKsStride < kBwdParts)
          part((ks - kBwdPartKs0) / kBwdPartKsStride);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// PSUM: also each slot's sum over all heads of P (a.psum), for the indexer loss's target.  A
// wave's 16-lane rows sum their heads inside the element parts; after the tile one lane
// swap adds the two rows of each half, the waves' sums meet in LDS, and in the next step one
// wave adds the four and stores the tile's 32 sums.
template <int H, int DQK, int DV, bool PSUM>
__global__ __launch_bounds__(64 * (H / 32)) void k_attn_bwd_p_ring(AttnBwdArgs a) {
  using C = AttnCfg<H, DQK, DV>;
  static_assert(C::PIPE && C::RPW == 8 && C::NK == 32, "ring shape");
  static_assert(C::TILE == 32 * DQK && C::SWZ, "a wave's Q rows fill one ring buffer");
  constexpr int RPW = C::RPW;
  constexpr int KSV = DV / 16;
  __shared__ __attribute__((aligned(16))) uint16_t kv0[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t kv1[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t kv2[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t kv3[C::TILE];
  __shared__ __attribute__((aligned(16))) int32_t idxr[2 * kIdxChunk];
  __shared__ int s_last[C::NW];
  __shared__ float s_hs[PSUM ? 2 : 1][C::NW][C::NK];   // per tile parity, wave and key

  RowCtx c = make_ctx(a, block_row(a));
  uint16_t* const bufs[4] = {kv0, kv1, kv2, kv3};
  const unsigned idxr_lds = (unsigned)(size_t)(__attribute__((address_space(3))) int32_t*)idxr;

  // Row prologue in one memory round trip: index chunks 0 and 1 and the wave's 32 Q rows go
  // to LDS by LDS DMA (Q rows stored like tile rows, chunks swizzled), dY and the forward
  // output load into registers, the index scan finds the row's tile count.
  idx_chunk_dma<H, DQK, DV>(a, c, 0, idxr_lds);
  idx_chunk_dma<H, DQK, DV>(a, c, 1, idxr_lds);
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
  // dY fragments (B operand of dP^T, the lane layout of Q) and D = rowsum(dY * out)
  bf16x8 dof[KSV];
  const size_t hrow = (size_t)c.row * H + c.head;
  float dpart = 0.f;
  {
    const uint16_t* dop = a.dout + hrow * DV + c.g * 8;
    const uint16_t* op = a.out + hrow * DV + c.g * 8;
#pragma unroll
    for (int ks = 0; ks < KSV; ++ks) {
      dof[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(dop + ks * 16));
      const bf16x8 ov = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(op + ks * 16));
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 x = {dof[ks][e], dof[ks][e + 1]};
        const bf16x2 y = {ov[e], ov[e + 1]};
        dpart = __builtin_amdgcn_fdot2_f32_bf16(x, y, dpart, false);
      }
    }
  }
  const float mrow = a.smax[hrow];
  const float lrow = a.ssum[hrow];
  int last = thread_last_valid<C::NT>(c.idx_row, a.topk, a.n_k, c.tid);
  last = (int)wave_max_u32((unsigned)(last + 1)) - 1;   // (last >= -1)
  if (c.lane == 0) s_last[c.wave] = last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // index chunks and Q landed (DMA untracked)
  __syncthreads();
  last = -1;
#pragma unroll
  for (int w = 0; w < C::NW; ++w) last = max(last, s_last[w]);
  const int T = (last + C::NK) / C::NK;
  // compiler-visible vmcnt(0): the row loads are done before the ring starts, so the compiler
  // adds no waits for them inside the loop
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if (T == 0) return;   // nothing selected: the row has no P / dS and no dKV share

  BwdRowK k;
  {
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_int(dpart), __float_as_int(dpart),
                                                     false, false);
    k.D = __int_as_float(pr[0]) + __int_as_float(pr[1]);
    k.msub = mrow == kNegInf ? 0.f : mrow * kLog2e;   // scaled log2 units
    k.invl = lrow > 0.f ? 1.f / lrow : 0.f;
    const bool odd = c.hl & 1;
    const int hpair = c.wave * 32 + (c.hl & ~1);
    k.vo0 = (unsigned)(((c.g * 8 + (odd ? 1 : 0)) * H + hpair) * 2);
    k.vo4 = k.vo0 + 16u * H * 2u;
    k.sel = odd ? 0x03020706u : 0x05040100u;
  }
  bf16x8 qf[C::KS];
  {
    typedef __attribute__((address_space(3))) const bf16x8* lds_cb8_t;
    const int sw = swz(c.hl);
    const lds_cptr_t qrow = (lds_cptr_t)qbuf + c.hl * C::ROWE;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = *(lds_cb8_t)(qrow + ((2 * ks + c.g) ^ sw) * 8);
  }
  __syncthreads();   // every wave holds its Q: the ring buffers take tiles from here on

  unsigned loff[C::NI];
#pragma unroll
  for (int i = 0; i < C::NI; ++i) loff[i] = flat_lane_offset<H, DQK, DV>(c, i);
  unsigned wb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    wb[q] = (unsigned)(size_t)(lds_u16_ptr_t)(bufs[q]) + c.wave_u * (RPW * C::ROWE * 2);
  const lds_ci32_t ir = (lds_ci32_t)idxr;
  // slot read by this lane for step t: lanes 0..31 the tile whose P / dS the step forms (t),
  // lanes 32..63 the tile it gathers (t+4)
  auto step_slot = [&](int t) { return (t + 4 * (c.lane >> 5)) * C::NK + (c.lane & 31); };

  // tiles 0 .. 3 from chunk 0
  {
    const int s0 = c.lane, s1 = 2 * C::NK + c.lane;
    unsigned off0, off1, so[RPW];
    (void)decode_slot<H, DQK, DV>(a, ir[s0], s0, off0);
    (void)decode_slot<H, DQK, DV>(a, ir[s1], s1, off1);
    wave_row_offsets<H, DQK, DV>(c, off0, 0, so);
    gather_tile_flat_so<H, DQK, DV>(a, c, so, loff, wb[0]);
    wave_row_offsets<H, DQK, DV>(c, off0, 32, so);
    gather_tile_flat_so<H, DQK, DV>(a, c, so, loff, wb[1]);
    wave_row_offsets<H, DQK, DV>(c, off1, 0, so);
    gather_tile_flat_so<H, DQK, DV>(a, c, so, loff, wb[2]);
    wave_row_offsets<H, DQK, DV>(c, off1, 32, so);
    gather_tile_flat_so<H, DQK, DV>(a, c, so, loff, wb[3]);
  }
  wait_vm_barrier<3 * C::NI>();   // tile 0 landed; tiles 1 .. 3 may be in flight
  f32x16 sa, da, sb, db;
  float hsum = 0.f;
  {
    const unsigned so0[RPW] = {};
    bwd_ring_tile<H, DQK, DV, false>(a, c, qf, dof, (lds_cptr_t)bufs[0], sa, da, sb, db, 0u,
                                     false, nullptr, nullptr, k, so0, loff, 0u, hsum);
  }
  int iv = ir[step_slot(0)];
  wait_vm_barrier<2 * C::NI>();   // tile 1 landed

  // ring slots rotating in registers: tile t+1 (read by step t), t+2, t+3 (landing), t (its
  // buffer takes the gather of t+4): LDS pointers of the read side, the wave's LDS DMA
  // address of the gather side
  lds_cptr_t b1 = (lds_cptr_t)bufs[1], b2 = (lds_cptr_t)bufs[2], b3 = (lds_cptr_t)bufs[3],
             b0 = (lds_cptr_t)bufs[0];
  unsigned w0 = wb[0], w1 = wb[1], w2 = wb[2], w3 = wb[3];
  const uint16_t* const prow = a.ws_p + (size_t)c.row * a.topkp * H;
  const uint16_t* const drow = a.ws_ds + (size_t)c.row * a.topkp * H;
  // tile tt's head sums: the four waves' parts added (lanes 0..31 = keys), stored by the wave
  // whose turn it is (its LDS reads follow the barrier that ended tile tt's step)
  auto psum_flush = [&](int tt) {
    if (c.wave_u == (tt & 3) && c.lane < C::NK) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < C::NW; ++w) v += s_hs[PSUM ? tt & 1 : 0][w][c.lane];
      const float* base = a.psum + (size_t)c.row * a.topkp + (size_t)tt * C::NK;
      const unsigned voff = (unsigned)c.lane * 4u;
      asm volatile("global_store_dword %0, %1, %2 nt" :: "v"(voff), "v"(v), "s"(base) : "memory");
    }
  };
  auto step = [&](int t, f32x16& s_nx, f32x16& d_nx, const f32x16& s_cu, const f32x16& d_cu) {
    if constexpr (PSUM) {
      if (t > 0 && t - 1 < T) psum_flush(t - 1);
    }
    unsigned off, so[RPW];
    const unsigned vmask = (unsigned)decode_slot<H, DQK, DV>(a, iv, step_slot(t), off);
    wave_row_offsets<H, DQK, DV>(c, off, 32, so);
    // chunk t/8 + 1 (first read at the end of step t + 3, for the gather of tile t + 8) into
    // the ring half chunk t/8 - 1 left; a load ahead of this step's gather, so complete once
    // the wait of step t + 2 has seen that gather land
    if ((t & 7) == 0 && t > 0) idx_chunk_dma<H, DQK, DV>(a, c, t / 8 + 1, idxr_lds);
    const size_t toff = (size_t)t * C::NK * H;
    bwd_ring_tile<H, DQK, DV, true, PSUM>(a, c, qf, dof, b1, s_nx, d_nx, s_cu, d_cu, vmask,
                                          t < T, prow + toff, drow + toff, k, so, loff, w0, hsum);
    if constexpr (PSUM) {
      // rows 0 + 1 and 2 + 3: the sum over the wave's 32 heads of key acc_key(lane % 16, g)
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(hsum), __float_as_uint(hsum),
                                                       false, false);
      const float hw = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      if ((c.lane & 16) == 0) s_hs[t & 1][c.wave_u][acc_key(c.lane & 15, c.g)] = hw;
    }
    iv = ir[step_slot(t + 1) & (2 * kIdxChunk - 1)];
    // tile t+2 landed: its gather is followed by at least the gathers of t+3 and t+4
    wait_vm_barrier<2 * C::NI>();
    const lds_cptr_t bt = b0;
    b0 = b1;
    b1 = b2;
    b2 = b3;
    b3 = bt;
    const unsigned wt = w0;
    w0 = w1;
    w1 = w2;
    w2 = w3;
    w3 = wt;
  };
  // steps in pairs (the accumulator sets alternate); for odd T the pair's second step is
  // past the row's last tile and stores nothing (the waits count loads only, so skipped
  // stores change no count)
  for (int t = 0; t < T; t += 2) {
    step(t, sb, db, sa, da);
    step(t + 1, sa, da, sb, db);
  }
  if constexpr (PSUM) {
    if ((T & 1) == 0) psum_flush(T - 1);   // (odd T: step T flushed it)
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no gather or store may outlive the block
}

// ---------------------------------------------------------------------------------------
// k_attn_bwd_dq_ring: dQ = (softmax_scale * dS) K_sel, split by latent dims
// ---------------------------------------------------------------------------------------
//
// Each wave owns 144 of the 576 latent dims for all 128 heads: dQ^T[dim, head] += K^T dS^T
// on 16x16x32 MFMA, one K step (the tile's 32 keys) per tile, 9 dim tiles x 8 head tiles of
// accumulators.  A wave reads only its quarter of the gathered key tile (transposing LDS
// reads) and the tile's whole dS block, half the LDS traffic of a split by heads, where every
// wave reads the whole key tile.  Slot indices come from the LDS index ring; three tile
// buffers, the gather of tile t+2 during step t.  Empty slots carry dS = 0, so their key
// rows (gathered from row 0) add nothing and no validity mask is needed; the row runs its
// tiles exactly (no padding tiles).

template <int H, int DQK, int DV>
__global__ __launch_bounds__(256) void k_attn_bwd_dq_ring(AttnBwdArgs a) {
  using C = AttnCfg<H, DQK, DV>;
  static_assert(H == 128 && C::NW == 4 && C::FLAT && C::RPW == 8 && C::NK == 32 && C::SWZ,
                "ring shape");
  constexpr int NW = C::NW;
  constexpr int DW = DQK / NW;           // latent dims per wave (144)
  constexpr int MT = DW / 16;            // 16-dim tiles per wave (9)
  constexpr int NB = H / 16;             // 16-head tiles (8)
  constexpr int DST = C::NK * H;         // dS tile elements: [32 slots][128 heads]
  constexpr int GOPS2 = C::NI + 2;       // loads per wave and tile: the key rows and two dS pieces
  static_assert(DQK % (16 * NW) == 0 && DST * 2 == NW * 2 * 1024, "tiling");
  __shared__ __attribute__((aligned(16))) uint16_t kv0[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t kv1[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t kv2[C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t ds0[DST];
  __shared__ __attribute__((aligned(16))) uint16_t ds1[DST];
  __shared__ __attribute__((aligned(16))) uint16_t ds2[DST];
  __shared__ __attribute__((aligned(16))) int32_t idxr[2 * kIdxChunk];
  __shared__ int s_last[NW];

  RowCtx c = make_ctx(a, block_row(a));
  const unsigned idxr_lds = (unsigned)(size_t)(__attribute__((address_space(3))) int32_t*)idxr;
  idx_chunk_dma<H, DQK, DV>(a, c, 0, idxr_lds);
  idx_chunk_dma<H, DQK, DV>(a, c, 1, idxr_lds);
  int last = thread_last_valid<C::NT>(c.idx_row, a.topk, a.n_k, c.tid);
  last = (int)wave_max_u32((unsigned)(last + 1)) - 1;   // (last >= -1)
  if (c.lane == 0) s_last[c.wave] = last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // index chunks landed (DMA is not tracked)
  __syncthreads();
  last = -1;
#pragma unroll
  for (int w = 0; w < NW; ++w) last = max(last, s_last[w]);
  const int T = (last + C::NK) / C::NK;
  __builtin_amdgcn_s_waitcnt(0x0F70);   // compiler-visible: the scan loads are done

  const int i16 = c.lane & 15, G = c.lane >> 4;
  const int d0 = c.wave_u * DW;
  f32x4 acc[MT][NB];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[m][nb] = (f32x4){};

  if (T > 0) {
    unsigned loff[C::NI];
#pragma unroll
    for (int i = 0; i < C::NI; ++i) loff[i] = flat_lane_offset<H, DQK, DV>(c, i);
    // ring slots rotating in registers (tile t's buffers, t+1's, t+2's): LDS pointers for the
    // reads, the wave's LDS DMA addresses for the gathers
    lds_cptr_t k0 = (lds_cptr_t)kv0, k1 = (lds_cptr_t)kv1, k2 = (lds_cptr_t)kv2;
    lds_cptr_t e0 = (lds_cptr_t)ds0, e1 = (lds_cptr_t)ds1, e2 = (lds_cptr_t)ds2;
    const unsigned kwo = c.wave_u * (C::RPW * C::ROWE * 2), dwo = c.wave_u * 2048u;
    auto lds_addr = [](lds_cptr_t p) { return (unsigned)(size_t)p; };
    // dS tile in LDS: slot rows of 256 bytes, 16-byte chunk c of slot s at physical chunk
    // c ^ 2 (s % 4), which makes the transposing reads (4 slots x 2 chunks per 16 lanes)
    // conflict-free.  The wave copies slots 8 wave .. +7 with two 1 KB DMA pieces; lane L of
    // piece i fills physical chunk L % 16 of slot 8 wave + 4 i + L / 16.
    unsigned dsoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int s = 8 * c.wave + 4 * i + (c.lane >> 4), p = c.lane & 15;
      dsoff[i] = (unsigned)((s * H + 8 * (p ^ (2 * (s & 3)))) * 2);
    }
    const uint16_t* dsrow = a.ws_ds + (size_t)c.row * a.topkp * H;
    auto gather = [&](int u, const unsigned* so, lds_cptr_t kd, lds_cptr_t dd) {
      gather_tile_flat_so<H, DQK, DV>(a, c, so, loff, lds_addr(kd) + kwo);
      const uint16_t* src = dsrow + (size_t)min(u, T - 1) * DST;
      const unsigned dm0 = lds_addr(dd) + dwo;
      static_for<2>([&](auto I) {
        constexpr int i = decltype(I)::value;
        const unsigned voff = dsoff[i];
        const unsigned m0 = dm0;
        const uint16_t* base = src;
        asm volatile("s_add_u32 m0, %0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3"
                     :: "s"(m0), "n"(i * 1024), "v"(voff), "s"(base) : "memory", "m0", "scc");
      });
    };
    // transposing-read addresses (elements from the buffer base): lane i16 of group G
    // supplies row 8 G + i16 / 4 (and + 4), columns c0 + 4 (i16 % 4) .. +3
    const int tr_row = 8 * G + (i16 >> 2);
    const int cq = i16 & 3;
    // key tile: columns d0 + 16 m + 4 cq, chunk (2 (d0 / 16 + m) + cq / 2) ^ swz(row)
    int ka[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int r = tr_row + 4 * hf;
      ka[hf] = r * C::ROWE + (cq & 1) * 4;
    }
    const int ksw0 = swz(tr_row), ksw1 = swz(tr_row + 4);
    auto kfrag = [&](lds_cptr_t tb, int m) {
      const int ch = d0 / 8 + 2 * m + (cq >> 1);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_ptr_t)(tb + ka[0] + (ch ^ ksw0) * 8));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_ptr_t)(tb + ka[1] + (ch ^ ksw1) * 8));
      return __builtin_bit_cast(bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };
    // dS tile: columns (heads) 16 nb + 4 cq, chunk (2 nb + cq / 2) ^ 2 (row % 4)
    const int da0 = tr_row * H + (cq & 1) * 4, da1 = (tr_row + 4) * H + (cq & 1) * 4;
    const int dsw0 = 2 * (tr_row & 3), dsw1 = 2 * ((tr_row + 4) & 3);
    auto dfrag = [&](lds_cptr_t db, int nb) {
      const int ch = 2 * nb + (cq >> 1);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(db + da0 + (ch ^ dsw0) * 8));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(db + da1 + (ch ^ dsw1) * 8));
      return __builtin_bit_cast(bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };

    const lds_ci32_t ir = (lds_ci32_t)idxr;
    // slot read by this lane for step t: the tile it gathers (t+2); both lane halves read it
    auto step_slot = [&](int t) { return (t + 2) * C::NK + (c.lane & 31); };
    {
      unsigned off, so[C::RPW];
      (void)decode_slot<H, DQK, DV>(a, ir[c.lane], c.lane, off);   // tiles 0 and 1
      wave_row_offsets<H, DQK, DV>(c, off, 0, so);
      gather(0, so, k0, e0);
      wave_row_offsets<H, DQK, DV>(c, off, 32, so);
      gather(1, so, k1, e1);
    }
    int iv = ir[step_slot(0)];
    wait_vm_barrier<GOPS2>();   // tile 0 landed; tile 1 may be in flight
    for (int t = 0; t < T; ++t) {
      unsigned off, so[C::RPW];
      (void)decode_slot<H, DQK, DV>(a, iv, step_slot(t), off);
      wave_row_offsets<H, DQK, DV>(c, off, 0, so);
      // chunk t/8 + 1 (first read at the end of step t + 5) into the ring half chunk t/8 - 1
      // left; a load ahead of this step's gather, so complete once tile t+2 has landed
      if ((t & 7) == 0 && t > 0) idx_chunk_dma<H, DQK, DV>(a, c, t / 8 + 1, idxr_lds);
      gather(t + 2, so, k2, e2);   // (past the row's last tile: row 0 and a clamped dS)
      const lds_cptr_t tb = k0;
      const lds_cptr_t db = e0;
      bf16x8 bq[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) bq[nb] = dfrag(db, nb);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const bf16x8 af = kfrag(tb, m);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          // 288 accumulator registers: the first 256 fill the AGPRs; the last dim tile's are
          // pinned to VGPRs (an asm MFMA with VGPR C / D), else the compiler cycles them
          // through the AGPRs with copies every step
          if (m < MT - 1)
            acc[m][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bq[nb], acc[m][nb], 0, 0, 0);
          else
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                         : "+v"(acc[m][nb]) : "v"(af), "v"(bq[nb]));
        }
      }
      iv = ir[step_slot(t + 1) & (2 * kIdxChunk - 1)];
      // tile t+1 landed: its loads are followed by tile t+2's (and maybe an index chunk)
      wait_vm_barrier<GOPS2>();
      const lds_cptr_t kt = k0, et = e0;
      k0 = k1;
      k1 = k2;
      k2 = kt;
      e0 = e1;
      e1 = e2;
      e2 = et;
    }
    // no gather may outlive the block; VALU reads the asm MFMAs' VGPR results next
    asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  }

  // dQ^T C layout: lane (head 16 nb + i16, group G) holds dims d0 + 16 m + 4 G .. +3
  uint16_t* qrow = a.dq + (size_t)c.row * H * DQK;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t lo = (uint32_t)f32_to_bf16(acc[m][nb][0]) |
                          ((uint32_t)f32_to_bf16(acc[m][nb][1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(acc[m][nb][2]) |
                          ((uint32_t)f32_to_bf16(acc[m][nb][3]) << 16);
      // (non-temporal: dQ is not read again by the backward)
      __builtin_nontemporal_store(
          (u32x2){lo, hi},
          reinterpret_cast<u32x2*>(qrow + (size_t)(16 * nb + i16) * DQK + d0 + 16 * m + 4 * G));
    }
  }
}

// ---------------------------------------------------------------------------------------
// dKV: per-(row, slot) contributions, then a per-key reduction (no float atomics)
// ---------------------------------------------------------------------------------------

// k_attn_bwd_dkv_part: C[row, slot, :] = (scale dS)^T Q + P^T dY for every slot of the
// row's tiles (empty slots have P = dS = 0), bf16, [row][slot padded to topkp][DQK].
// Each wave owns DQK / 4 latent dims and holds Q[:, dims] and dY[:, dims] for all heads as
// A fragments (staged through LDS once per row).  Per tile C^T[dim, slot] comes out of
// 16x16x32 MFMA with lane (slot n, group G) holding dims 4G .. 4G+3 of each 16-dim tile,
// stored as one 8-byte write.
template <int H, int DQK, int DV>
__global__ __launch_bounds__(256) void k_attn_bwd_dkv_part(AttnBwdArgs a) {
  constexpr int NW = 4;
  constexpr int DW = DQK / NW;         // latent dims per wave (144)
  constexpr int NT = DW / 16;          // 16-dim tiles per wave
  constexpr int KH = H / 32;           // 32-head K steps
  constexpr int NK = 32;               // slots per tile
  static_assert(DQK % (16 * NW) == 0 && H % 32 == 0, "tiling");
  __shared__ __attribute__((aligned(16))) uint16_t stage[H * DQK];
  __shared__ int s_last[NW];

  const int row = block_row(a);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, G = lane >> 4;
  const int32_t* idx_row = a.idx + (size_t)row * a.topk;
  int last = thread_last_valid<256>(idx_row, a.topk, a.n_k, tid);
  last = (int)wave_max_u32((unsigned)(last + 1)) - 1;   // (last >= -1)
  if (lane == 0) s_last[wave] = last;
  __syncthreads();
  last = max(max(s_last[0], s_last[1]), max(s_last[2], s_last[3]));
  const int ntiles = (last + NK) / NK;
  if (ntiles == 0) return;

  const int d0 = wave * DW;
  // fragments of Q^T[dim d0 + 16 nt + n, heads 32 kk + 8 G .. +7] and the same of dY
  bf16x8 qa[NT][KH], da[NT][KH];
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // uniform: DMA bases are scalars
  const unsigned stage_lds = (unsigned)(size_t)(lds_u16_ptr_t)stage;
  {
    static_assert((H * DQK * 2) % 1024 == 0 && (H * DV * 2) % 1024 == 0, "whole DMA pieces");
    dma_copy_flat<NW>(stage_lds, a.q + (size_t)row * H * DQK, H * DQK * 2, wave_u, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int kk = 0; kk < KH; ++kk)
        qa[nt][kk] = tr_frag(stage, DQK, 32 * kk + 8 * G, d0 + 16 * nt, n);
    __syncthreads();
    dma_copy_flat<NW>(stage_lds, a.dout + (size_t)row * H * DV, H * DV * 2, wave_u, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int kk = 0; kk < KH; ++kk)
        da[nt][kk] = (d0 + 16 * nt < DV) ? tr_frag(stage, DV, 32 * kk + 8 * G, d0 + 16 * nt, n)
                                         : (bf16x8){};
  }

  __syncthreads();   // the staging area becomes the tile ring

  // Ring of three tiles in the staging area: tile = [P | dS] x [32 slots][16 chunks of 8
  // heads], chunk c of slot s stored at physical chunk c ^ (s & 15) (conflict-free reads of
  // 16 slots x one chunk).  Each wave copies a quarter of a tile (4 x 1 KB LDS DMA pieces:
  // tensor wave / 2, slots 16 (wave % 2) .. +15), so every tile needs the barrier.
  constexpr int TILE_E = 2 * NK * H;   // bf16 elements per ring tile
  static_assert(3 * TILE_E <= H * DQK && H == 128, "ring fits the staging area");
  const uint16_t* tsrc0 = (wave_u >> 1) ? a.ws_ds : a.ws_p;
  const uint16_t* tsrc = tsrc0 + (size_t)row * a.topkp * H;
  unsigned doff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = 16 * (wave & 1) + 4 * i + (lane >> 4);
    const int c = (lane & 15) ^ (slot & 15);
    doff[i] = (unsigned)(slot * H * 2 + c * 16);
  }
  const unsigned ring_lds = stage_lds;
  const unsigned wdst = (unsigned)((wave_u >> 1) * NK * H * 2 + (wave_u & 1) * 16 * H * 2);
  auto dma_tile = [&](int t, int k) {
    const uint16_t* src = tsrc + (size_t)min(t, ntiles - 1) * NK * H;
    const unsigned m0v = ring_lds + (unsigned)(k * TILE_E * 2) + wdst;
    static_for<4>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const unsigned voff = doff[i];
      const unsigned m0 = m0v;
      const uint16_t* base = src;
      asm volatile("s_add_u32 m0, %0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3"
                   :: "s"(m0), "n"(i * 1024), "v"(voff), "s"(base) : "memory", "m0", "scc");
    });
  };

  f32x4 acc[2][NT];
  const uint16_t* cbase = a.ws_c + (size_t)row * a.topkp * DQK;   // scalar base of the row
  // lane's byte offset of (slot n of the 16-slot group, dims d0 + 4 G ..): + slot / dim terms
  const unsigned coff = (unsigned)((n * DQK + d0 + 4 * G) * 2);
  constexpr int NST = 2 * NT;   // 8-byte stores per lane and tile (exact: issued from asm)
  static_assert(2 * NST + 4 < 64, "vmcnt range");
  constexpr int NMF = KH * 4 * NT;   // MFMAs per tile
  constexpr int SGAP = 8;            // MFMAs between two stores of the previous tile
  static_assert(SGAP / 2 + SGAP * (NST - 1) < NMF, "store placement");
  // The stores are software-pipelined: tile t's contributions (bf16, packed after its
  // products) go out during step t+1, one after every SGAP of that step's MFMAs, so the write
  // path drains while the matrix cores run (issued as a burst after the products, the stores
  // and the products took turns and each left the other's unit idle).
  u32x2 cst[2][NT];
  auto store_prev = [&](int tp, int j) {
    const int mt = j / NT, nt = j % NT;
    const unsigned off = coff + (unsigned)(((tp * NK + 16 * mt) * DQK + 16 * nt) * 2);
    const u32x2 d = cst[mt][nt];
    const uint16_t* base = cbase;
    asm volatile("global_store_dwordx2 %0, %1, %2" :: "v"(off), "v"(d), "s"(base) : "memory");
  };
  auto step = [&](int t, int k) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (f32x4){};
    dma_tile(t + 2, (k + 2) % 3);
    const lds_cptr_t tb = (lds_cptr_t)stage + k * TILE_E;
    const bool sp = t > 0;   // the previous tile's stores (none before the first tile)
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
      // B fragments: slot 16 mt + n, heads 32 kk + 8 G .. +7 (logical chunk 4 kk + G)
      bf16x8 bp[2], bd[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int e = (16 * mt + n) * H + (((4 * kk + G) ^ n) * 8);
        bp[mt] = *(__attribute__((address_space(3))) const bf16x8*)(tb + e);
        bd[mt] = *(__attribute__((address_space(3))) const bf16x8*)(tb + NK * H + e);
      }
      // (dims past DV have zero dY fragments: the product is issued anyway -- the wave
      // owning them would otherwise only finish early, which buys nothing)
#pragma unroll
      for (int i = 0; i < 4 * NT; ++i) {
        const int mt = (i / NT) & 1, nt = i % NT;
        if (i < 2 * NT)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[nt][kk], bd[mt], acc[mt][nt], 0, 0, 0);
        else
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da[nt][kk], bp[mt], acc[mt][nt], 0, 0, 0);
        const int g = kk * 4 * NT + i;   // MFMA index within the tile
        if (g >= SGAP / 2 && (g - SGAP / 2) % SGAP == 0 && (g - SGAP / 2) / SGAP < NST) {
          if (sp) store_prev(t - 1, (g - SGAP / 2) / SGAP);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // every slot of the tile is stored (empty and padding slots too: they lie inside the
    // row's padded area and are never listed), so the store count per step is fixed
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint32_t lo = (uint32_t)f32_to_bf16(acc[mt][nt][0]) |
                            ((uint32_t)f32_to_bf16(acc[mt][nt][1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(acc[mt][nt][2]) |
                            ((uint32_t)f32_to_bf16(acc[mt][nt][3]) << 16);
        cst[mt][nt] = (u32x2){lo, hi};
      }
    }
    // tile t+1 landed for every wave.  After its DMA (step t-1's start) come the previous
    // tile's stores of step t-1, tile t+2's DMA and this step's stores: 2 NST + 4 memory
    // instructions from step 2 on; at step 1, NST + 4 (step 0 stores nothing); at step 0 tile
    // 1 landed in the prologue.  (Vector memory instructions of a wave complete in issue order,
    // loads and stores alike.)
    if (t >= 2) wait_vm_barrier<2 * NST + 4>();
    else wait_vm_barrier<NST + 4>();
  };
  dma_tile(0, 0);
  dma_tile(1, 1);
  wait_vm_barrier<0>();    // both first tiles
  const int npad = (ntiles + 2) / 3 * 3;
  for (int t = 0; t < npad; t += 3) {
    step(t, 0);
    step(t + 1, 1);
    step(t + 2, 2);
  }
#pragma unroll
  for (int j = 0; j < NST; ++j) store_prev(npad - 1, j);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no DMA or store may outlive the block
}

// Zero the per-key counters.
__global__ __launch_bounds__(256) void k_keys_zero(KeyListArgs a) {
  for (int k = blockIdx.x * 256 + threadIdx.x; k < a.n_k; k += gridDim.x * 256) a.cnt[k] = 0;
}

// Count the valid (row, slot) entries of the chunk per key.
__global__ __launch_bounds__(256) void k_keys_count(KeyListArgs a) {
  const long long total = (long long)a.rows * a.topk;
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (long long)gridDim.x * 256) {
    const int k = a.idx[e];
    if ((unsigned)k < (unsigned)a.n_k) atomicAdd(&a.cnt[k], 1);
  }
}

// off = exclusive prefix sum of cnt (off[n_k] = total), cur = off.  One workgroup of 16 waves,
// in passes of 16 x 1024 counters: each wave scans its 1024 as 16 coalesced groups of 64 (all
// loaded together, DPP scans carried in registers), one block scan places the waves' runs.
// (One block scan per 1024 counters, each a barrier pair, took 27 us for 32768 keys.)
__global__ __launch_bounds__(1024) void k_keys_scan(KeyListArgs a) {
  __shared__ unsigned scratch[16];
  constexpr int CH = 16;                       // groups of 64 per wave and pass
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned base = 0;
  for (int p0 = 0; p0 < a.n_k; p0 += 16 * CH * 64) {
    const int w0 = p0 + wave * CH * 64;
    unsigned v[CH];   // counts, then the exclusive prefix within the wave's run
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int k = w0 + c * 64 + lane;
      v[c] = k < a.n_k ? (unsigned)a.cnt[k] : 0u;
    }
    unsigned carry = 0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const unsigned x = wave_incl_scan(v[c]) + carry;
      carry = (unsigned)__builtin_amdgcn_readlane((int)x, 63);
      v[c] = x - v[c];
    }
    unsigned total;
    const unsigned wbase = base + block_excl_scan<16>(lane == 63 ? carry : 0u, scratch, total);
    // (block_excl_scan's value for lane 63 of each wave is the sum of the earlier waves' runs)
    const unsigned woff = (unsigned)__builtin_amdgcn_readlane((int)wbase, 63);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int k = w0 + c * 64 + lane;
      if (k < a.n_k) {
        a.off[k] = (int)(woff + v[c]);
        a.cur[k] = (int)(woff + v[c]);
      }
    }
    base += total;
  }
  if (threadIdx.x == 0) a.off[a.n_k] = (int)base;
}

// list[cur[k]++] = row * topkp + slot for every valid entry: the entry's row in the
// per-(row, slot) workspaces, so the reductions read it with no division.
__global__ __launch_bounds__(256) void k_keys_scatter(KeyListArgs a) {
  const long long total = (long long)a.rows * a.topk;
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (long long)gridDim.x * 256) {
    const int k = a.idx[e];
    if ((unsigned)k < (unsigned)a.n_k) {
      const int r = (int)(e / a.topk), sl = (int)(e - (long long)r * a.topk);
      a.list[atomicAdd(&a.cur[k], 1)] = r * a.topkp + sl;
    }
  }
}

// dkv[k] += sum of the key's contributions; one wave per key, so the row is owned and the
// update is a plain read-modify-write.  Lane l sums dims 8 l .. 8 l + 7 (and, for l < 8,
// the 64 dims past 512), sixteen entries in flight.
template <int DQK>
__global__ __launch_bounds__(256) void k_bwd_reduce(AttnBwdArgs a) {
  static_assert(DQK == 576, "lane split of the latent row");
  const int k = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (k >= a.n_k) return;
  const int beg = a.off[k], end = a.off[k + 1];
  if (beg == end) return;
  float s0[8] = {}, s1[8] = {};
  const bool tail = lane < 8;
  auto add = [&](int e) {
    const uint16_t* src = a.ws_c + (size_t)e * DQK;
    const uint4 v = *reinterpret_cast<const uint4*>(src + 8 * lane);
    uint4 w = make_uint4(0, 0, 0, 0);
    if (tail) w = *reinterpret_cast<const uint4*>(src + 512 + 8 * lane);
    const uint32_t vv[4] = {v.x, v.y, v.z, v.w}, ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s0[2 * j] += __uint_as_float(vv[j] << 16);
      s0[2 * j + 1] += __uint_as_float(vv[j] & 0xFFFF0000u);
      s1[2 * j] += __uint_as_float(ww[j] << 16);
      s1[2 * j + 1] += __uint_as_float(ww[j] & 0xFFFF0000u);
    }
  };
  int p = beg;
  for (; p + 16 <= end; p += 16) {
    int e[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) e[j] = a.list[p + j];
#pragma unroll
    for (int j = 0; j < 16; ++j) add(e[j]);
  }
  for (; p + 8 <= end; p += 8) {
    int e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = a.list[p + j];
#pragma unroll
    for (int j = 0; j < 8; ++j) add(e[j]);
  }
  for (; p + 4 <= end; p += 4) {
    const int e0 = a.list[p], e1 = a.list[p + 1], e2 = a.list[p + 2], e3 = a.list[p + 3];
    add(e0);
    add(e1);
    add(e2);
    add(e3);
  }
  for (; p < end; ++p) add(a.list[p]);
  float* dst = a.dkv + (size_t)k * DQK;
  float4* d0 = reinterpret_cast<float4*>(dst + 8 * lane);
  float4 x0 = d0[0], x1 = d0[1];
  x0.x += s0[0]; x0.y += s0[1]; x0.z += s0[2]; x0.w += s0[3];
  x1.x += s0[4]; x1.y += s0[5]; x1.z += s0[6]; x1.w += s0[7];
  d0[0] = x0;
  d0[1] = x1;
  if (tail) {
    float4* d1 = reinterpret_cast<float4*>(dst + 512 + 8 * lane);
    float4 y0 = d1[0], y1 = d1[1];
    y0.x += s1[0]; y0.y += s1[1]; y0.z += s1[2]; y0.w += s1[3];
    y1.x += s1[4]; y1.y += s1[5]; y1.z += s1[6]; y1.w += s1[7];
    d1[0] = y0;
    d1[1] = y1;
  }
}

}  // namespace

hipError_t launch_key_lists(const KeyListArgs& a, hipStream_t s) {
  const long long entries = (long long)a.rows * a.topk;
  if (entries == 0) return hipSuccess;
  const int eg = (int)std::min<long long>((entries + 255) / 256, 8192);
  k_keys_zero<<<std::min((a.n_k + 255) / 256, 1024), 256, 0, s>>>(a);
  k_keys_count<<<eg, 256, 0, s>>>(a);
  k_keys_scan<<<1, 1024, 0, s>>>(a);
  k_keys_scatter<<<eg, 256, 0, s>>>(a);
  return hipGetLastError();
}

// The chunk's key lists first, then the four kernels (the lists stay in a.list / a.off for a
// caller that runs the indexer loss over the same chunk next).
hipError_t launch_sparse_attn_bwd(const AttnBwdArgs& a, int h, int d_qk, int d_v, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (!(h == 128 && d_qk == 576 && d_v == 512)) return hipErrorInvalidValue;
  KeyListArgs kl = {a.idx, a.list, a.cnt, a.off, a.cur, a.rows, a.n_k, a.topk, a.topkp};
  hipError_t e = launch_key_lists(kl, s);
  if (e != hipSuccess) return e;
  if (a.psum)
    k_attn_bwd_p_ring<128, 576, 512, true><<<a.rows, 256, 0, s>>>(a);
  else
    k_attn_bwd_p_ring<128, 576, 512, false><<<a.rows, 256, 0, s>>>(a);
  k_attn_bwd_dq_ring<128, 576, 512><<<a.rows, 256, 0, s>>>(a);
  k_attn_bwd_dkv_part<128, 576, 512><<<a.rows, 256, 0, s>>>(a);
  k_bwd_reduce<576><<<(a.n_k + 3) / 4, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dsa
