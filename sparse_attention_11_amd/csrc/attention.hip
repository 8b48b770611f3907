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
//     lane, no VGPR staging) into a ring of three tile buffers, so the gathers of the next two
//     tiles overlap this tile's math.  Each wave copies whole rows, so the row base is a
//     scalar (its index is read ahead through the scalar cache).  Rows are stored unpadded
//     with their 16-byte chunks XOR-swizzled by row, which keeps both the 16-row logits reads
//     and the 4-row transposing value reads free of bank conflicts.  Empty slots gather row 0
//     and are masked.
//   * Logits: S^T[key, head] = K_tile (A, from LDS) x Q^T (B) on v_mfma_f32_32x32x16_bf16.
//     The first 416 Q dims stay in VGPRs for the whole row, the rest are staged once in LDS
//     (Q and the 512-wide accumulator do not both fit in registers otherwise).  A rows
//     are fed in a fixed key permutation so that each lane's 16 accumulators come out as two
//     runs of 8 consecutive keys of one head -- the B-operand layout of the next product.
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
#include <utility>

#include "dsa_device.h"

namespace dsa {

namespace {

typedef __attribute__((address_space(3))) uint16_t* lds_u16_ptr_t;
typedef __attribute__((address_space(3))) const uint16_t* lds_cptr_t;   // 32-bit LDS address
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_ptr_t;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;

// LDS row (within a 32-key tile) that feeds A-operand row m of the logits product
__device__ __forceinline__ int key_perm(int m) {
  const int q = m >> 3, gg = (m >> 2) & 1, rr = m & 3;
  return (q >> 1) * 16 + gg * 8 + (q & 1) * 4 + rr;
}

// key within the tile held by accumulator register r of a lane in half g (0/1)
__device__ __forceinline__ int acc_key(int r, int g) {
  return r < 8 ? g * 8 + r : 16 + g * 8 + (r - 8);
}

constexpr float kOverflowLog2 = 64.0f;  // p may reach 2^64 before the row is recomputed
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();
// bf16 quiet NaN with a payload arithmetic does not produce: marks a row for the exact pass
constexpr uint16_t kOverflowMark = 0x7FD5;

template <int H, int DQK, int DV>
struct AttnCfg {
  static constexpr int NW = (H + 31) / 32;   // waves, 32 heads each
  static constexpr int NT = NW * 64;
  static constexpr int KS = DQK / 16;        // K steps of the logits product
  static constexpr int DQR = DQK > 416 ? 416 : DQK;  // Q dims held in VGPRs
  static constexpr int KSR = DQR / 16;
  static constexpr int DQL = DQK - DQR;      // Q dims staged in LDS
  static constexpr int QROWE = DQL + 8;      // LDS row stride (elements) of staged Q
  static constexpr int MTV = DV / 32;        // 32-column M tiles of the output product
  static constexpr int NK = 32;              // keys per tile
  static constexpr int CPR = DQK / 8;        // 16-byte chunks per latent row
  // Rows are stored unpadded; when a row is a whole number of 8-chunk groups the 16-byte
  // chunks of row r are XOR-swizzled by swz(r) (< 8, so a chunk never leaves its group).  With
  // 64 four-byte banks this makes both LDS read patterns conflict-free: 16 rows x one chunk
  // (logits operand) and 4 consecutive rows x 4 consecutive chunks (transposed value reads).
  static constexpr bool SWZ = CPR % 8 == 0;
  static constexpr int ROWE = CPR * 8;       // LDS row stride (elements)
  static constexpr int TILE = NK * ROWE;     // elements per KV tile buffer
  static constexpr int QLDS = DQL > 0 ? H * QROWE : 8;
  static constexpr int NBUF = 3;             // gather ring depth (tiles t+1, t+2 in flight)
  static constexpr int RPW = NK / NW;        // tile rows gathered by each wave
  // Flat gather: a wave's RPW rows are RPW*CPR consecutive 16-byte chunks of the tile buffer,
  // copied by NI full-wave instructions; each instruction then spans at most two rows.
  static constexpr bool FLAT = CPR >= 64 && (RPW * CPR) % 64 == 0;
  static constexpr int NI = FLAT ? RPW * CPR / 64 : 1;
  // vector-memory instructions one wave issues per tile gather
  static constexpr int GOPS = FLAT ? NI : RPW * ((CPR + 63) / 64);
  static_assert(GOPS < 64, "vmcnt range");
  static_assert(DQK % 16 == 0 && DV % 32 == 0 && DV <= DQK && DQR % 16 == 0, "head dims");
};

__device__ __forceinline__ int swz(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }

// Per-row state shared by the fast and exact paths.
struct RowCtx {
  int row, tid, lane, wave, wave_u, hl, g, head, ntiles;
  const int32_t* idx_row;
  uint16_t* buf[3];  // KV tile buffers (separate LDS objects)
  uint16_t* qlds;    // staged Q dims
  int* flags;        // [2][NW] per-tile overflow flags
  unsigned* vm;      // [3][NW] per-tile validity bits of each wave's gathered rows
};

// Copy one latent row into LDS row `key` of `dst`: the LDS DMA, issued from inline asm so
// the compiler neither sees the LDS write nor adds waits for it (completion is tracked by
// hand with vmcnt before each barrier).  M0 holds the wave's LDS destination and lane L
// writes 16 bytes at M0 + 16 L; the source is the row base (SGPRs) plus a 32-bit per-lane
// offset that applies the chunk swizzle: physical chunk c0 + L holds logical chunk
// c0 + (L ^ swz(key)) (c0 is a multiple of 64, swz < 8).
template <int H, int DQK, int DV>
__device__ __forceinline__ void gather_row(const AttnArgs& a, const RowCtx& c, int id, int key,
                                           uint16_t* dst) {
  using C = AttnCfg<H, DQK, DV>;
  id = (id < 0 || id >= a.n_k) ? 0 : id;   // empty slot: any in-bounds row, masked later
  const uint16_t* src = a.kv + (size_t)id * DQK;
  const unsigned sw16 = C::SWZ ? (unsigned)swz(key) * 16u : 0u;
  const unsigned voff = ((unsigned)c.lane * 16u) ^ sw16;
#pragma unroll
  for (int c0 = 0; c0 < C::CPR; c0 += 64) {
    const unsigned lds_addr = (unsigned)(size_t)(lds_u16_ptr_t)(dst + key * C::ROWE + c0 * 8);
    // the chunk-group offset goes into the scalar base: an immediate instruction offset would
    // also move the LDS destination
    if (c0 + c.lane < C::CPR)
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(lds_addr), "v"(voff), "s"(src + c0 * 8) : "memory", "m0");
  }
}

// Gather of tile t with the indices read by scalar loads (exact path)
template <int H, int DQK, int DV>
__device__ __forceinline__ void gather_tile(const AttnArgs& a, const RowCtx& c, int t,
                                            uint16_t* dst) {
  using C = AttnCfg<H, DQK, DV>;
#pragma unroll
  for (int rr = 0; rr < C::NK / C::NW; ++rr) {
    const int key = rr * C::NW + c.wave_u;
    const int slot = t * C::NK + key;
    const int id = slot < a.topk ? c.idx_row[slot] : -1;
    gather_row<H, DQK, DV>(a, c, __builtin_amdgcn_readfirstlane(id), key, dst);
  }
}

// The slot indices one wave gathers for tile t (rows wave*RPW .. +RPW-1 of the tile), read
// with scalar loads: they count against lgkmcnt, so waiting for them never drains the
// in-flight gathers (which count against vmcnt).  Slots past topk read as -1.
template <int H, int DQK, int DV>
struct TileIdx {
  int v[AttnCfg<H, DQK, DV>::NK / AttnCfg<H, DQK, DV>::NW];
};

// AL8: topk is a multiple of 8 and the index rows are 32-byte aligned, so a wave's 8 slots of
// a tile are one aligned 8-dword block, read by one scalar load (the block of the last slots
// stands in for blocks past topk, whose slots read as -1).
template <int H, int DQK, int DV, bool AL8>
__device__ __forceinline__ TileIdx<H, DQK, DV> load_tile_idx_s(const AttnArgs& a,
                                                               const RowCtx& c, int t) {
  using C = AttnCfg<H, DQK, DV>;
  constexpr int RPW = C::NK / C::NW;
  // the index list is read-only while the kernel runs: reading it through the constant
  // address space lets uniform loads go to the scalar unit
  typedef __attribute__((address_space(4))) const int32_t* cidx_t;
  typedef __attribute__((address_space(4))) const i32x8* cidx8_t;
  const cidx_t ip = (cidx_t)c.idx_row;
  TileIdx<H, DQK, DV> r;
  if constexpr (AL8 && RPW == 8) {
    const int s0 = t * C::NK + c.wave_u * RPW;
    const i32x8 v = *(cidx8_t)(ip + min(s0, a.topk - RPW));
#pragma unroll
    for (int j = 0; j < RPW; ++j) r.v[j] = s0 < a.topk ? v[j] : -1;
  } else {
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int slot = t * C::NK + c.wave_u * RPW + j;
      const int v = ip[min(slot, a.topk - 1)];
      r.v[j] = slot < a.topk ? v : -1;
    }
  }
  return r;
}

// Validity bits of this wave's slots of a tile (bit j: row wave*RPW + j).
template <int H, int DQK, int DV>
__device__ __forceinline__ unsigned tile_bits(const AttnArgs& a, const TileIdx<H, DQK, DV>& ti) {
  constexpr int RPW = AttnCfg<H, DQK, DV>::NK / AttnCfg<H, DQK, DV>::NW;
  unsigned m = 0;
#pragma unroll
  for (int j = 0; j < RPW; ++j) m |= (ti.v[j] >= 0 && ti.v[j] < a.n_k) ? (1u << j) : 0u;
  return m;
}

template <int H, int DQK, int DV>
__device__ __forceinline__ void gather_tile_s(const AttnArgs& a, const RowCtx& c,
                                              const TileIdx<H, DQK, DV>& ti, uint16_t* dst) {
  constexpr int RPW = AttnCfg<H, DQK, DV>::NK / AttnCfg<H, DQK, DV>::NW;
#pragma unroll
  for (int j = 0; j < RPW; ++j) gather_row<H, DQK, DV>(a, c, ti.v[j], c.wave_u * RPW + j, dst);
}

template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Byte offset, within its latent row, of the chunk this lane copies in flat instruction i:
// the lane fills physical chunk f = 64 i + lane of the wave's rows, i.e. chunk f mod CPR of
// row f / CPR, which holds logical chunk (f mod CPR) ^ swz(row).
template <int H, int DQK, int DV>
__device__ __forceinline__ unsigned flat_lane_offset(const RowCtx& c, int i) {
  using C = AttnCfg<H, DQK, DV>;
  const int f = i * 64 + c.lane;
  const int j = f / C::CPR, ch = f - j * C::CPR;
  const int sw = C::SWZ ? swz(c.wave * C::RPW + j) : 0;
  return (unsigned)(ch ^ sw) * 16u;
}

// Flat gather of this wave's rows of a tile.  wb: LDS byte address of the wave's first row.
// The row offsets are scalars; each lane picks the one of the (at most two) rows its chunk
// falls in.  Empty slots copy row 0 (masked later).
template <int H, int DQK, int DV>
__device__ __forceinline__ void gather_tile_flat(const AttnArgs& a, const RowCtx& c,
                                                 const TileIdx<H, DQK, DV>& ti,
                                                 const unsigned* loff, unsigned wb) {
  using C = AttnCfg<H, DQK, DV>;
  unsigned so[C::RPW];
#pragma unroll
  for (int j = 0; j < C::RPW; ++j)
    so[j] = (unsigned)ti.v[j] < (unsigned)a.n_k ? (unsigned)ti.v[j] * (C::CPR * 16u) : 0u;
  static_for<C::NI>([&](auto I) {
    constexpr int i = decltype(I)::value;
    constexpr int j0 = i * 64 / C::CPR;              // row of lane 0
    constexpr int b = (j0 + 1) * C::CPR - 64 * i;    // first lane in row j0 + 1
    unsigned ro = so[j0];
    if constexpr (b < 64) ro = c.lane >= b ? so[j0 + 1] : ro;
    const unsigned voff = loff[i] + ro;
    const unsigned m0v = wb;       // (named locals: asm operands alone do not capture)
    const uint16_t* base = a.kv;
    // M0 = LDS destination of lane 0; one wait state between writing M0 and the DMA
    asm volatile("s_add_u32 m0, %0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3"
                 :: "s"(m0v), "n"(i * 1024), "v"(voff), "s"(base) : "memory", "m0", "scc");
  });
}

// Wait until at most N of this wave's vector-memory instructions are outstanding, then meet
// the other waves at a barrier (one asm block, so no memory access moves across it).
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// S^T for one tile (32 keys x the wave's 32 heads), unscaled, -inf at empty slots; `mx`
// receives the lane pair's (= one head's) tile max in scaled log2 units.
template <int H, int DQK, int DV>
__device__ __forceinline__ f32x16 tile_logits(const AttnArgs& a, const RowCtx& c,
                                              const bf16x8* qf, const uint16_t* tile,
                                              unsigned vmask, float& mx) {
  using C = AttnCfg<H, DQK, DV>;
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
  const uint16_t* qlrow = c.qlds + (C::DQL > 0 ? c.head % H : 0) * C::QROWE + c.g * 8;
  // A fragments one group ahead of their MFMAs; sched_barrier bounds the live fragments
  constexpr int QG = 3;                 // K steps per prefetch group (36 = 12 x 3)
  constexpr int NG = (C::KS + QG - 1) / QG;
  bf16x8 af[2][QG];
#pragma unroll
  for (int u = 0; u < QG; ++u)
    if (u < C::KS) af[0][u] = *(__attribute__((address_space(3))) const bf16x8*)(arow_at(u));
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int cur = gi & 1;
    if (gi + 1 < NG) {
#pragma unroll
      for (int u = 0; u < QG; ++u) {
        const int ks = (gi + 1) * QG + u;
        if (ks < C::KS) af[cur ^ 1][u] = *(__attribute__((address_space(3))) const bf16x8*)(arow_at(ks));
      }
    }
#pragma unroll
    for (int u = 0; u < QG; ++u) {
      const int ks = gi * QG + u;
      if (ks < C::KS) {
        bf16x8 bq;
        if (ks < C::KSR) bq = qf[ks < C::KSR ? ks : 0];
        else bq = *reinterpret_cast<const bf16x8*>(qlrow + (ks - C::KSR) * 16);
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
  bf16x8 vf[2][2];
  vf[0][0] = vfrag(0, 0);
  vf[0][1] = vfrag(1, 0);
#pragma unroll
  for (int mt = 0; mt < C::MTV; ++mt) {
    const int cur = mt & 1;
    if (mt + 1 < C::MTV) {
      vf[cur ^ 1][0] = vfrag(0, mt + 1);
      vf[cur ^ 1][1] = vfrag(1, mt + 1);
    }
    o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[cur][0], pf[0], o[mt], 0, 0, 0);
    o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[cur][1], pf[1], o[mt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int H, int DQK, int DV>
__device__ __forceinline__ unsigned tile_vmask(const AttnArgs& a, const RowCtx& c, int t) {
  const int slot = t * AttnCfg<H, DQK, DV>::NK + c.hl;
  const int id = slot < a.topk ? c.idx_row[slot] : -1;
  return (unsigned)__ballot(id >= 0 && id < a.n_k);
}



template <int H, int DQK, int DV>
__device__ __forceinline__ void load_q(const AttnArgs& a, const RowCtx& c, bf16x8* qf) {
  using C = AttnCfg<H, DQK, DV>;
  const bool hv = (H % 32 == 0) || c.head < H;
  const uint16_t* qp = a.q + ((size_t)c.row * H + (hv ? c.head : 0)) * DQK + c.g * 8;
#pragma unroll
  for (int ks = 0; ks < C::KSR; ++ks) {
    const uint4 v = *reinterpret_cast<const uint4*>(qp + ks * 16);
    qf[ks] = hv ? __builtin_bit_cast(bf16x8, v) : (bf16x8){};
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

// Logits, probabilities and the output product of one tile.  Returns whether some head's
// max exceeded the scaling max by more than the fast path's range.
template <int H, int DQK, int DV>
__device__ __forceinline__ bool tile_step(const AttnArgs& a, const RowCtx& c, const bf16x8* qf,
                                          const uint16_t* tile, unsigned vmask, float& m_used,
                                          float& m_true, float& lsum, f32x16* o) {
  float mx;
  f32x16 s = tile_logits<H, DQK, DV>(a, c, qf, tile, vmask, mx);
  m_true = fmaxf(m_true, mx);
  if (m_used == kNegInf) m_used = mx;  // first tile with a valid key
  const bool over = mx > m_used + kOverflowLog2;
  // m_used is still -inf only while every key so far is empty; all logits are then -inf
  const float msub = m_used == kNegInf ? 0.f : m_used;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x8 pf[2];
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

}  // namespace

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
  for (int bi = EXACT ? (int)blockIdx.x : 0; bi < (EXACT ? nblk : 1); bi += (int)gridDim.x) {
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
    if (a.out[(size_t)c.row * H * DV] != kOverflowMark) continue;
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

  // tiles past the last valid slot are never gathered or computed
  int last = -1;
  for (int sl = c.tid; sl < a.topk; sl += C::NT) {
    const int id = c.idx_row[sl];
    if (id >= 0 && id < a.n_k) last = sl;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
  if (c.lane == 0) s_last[c.wave] = last;

  // stage q[row, :, DQR:] in LDS
  if constexpr (C::DQL > 0) {
    constexpr int CH = C::DQL / 8;
    const uint16_t* qrow = a.q + (size_t)c.row * H * DQK + C::DQR;
    for (int i = c.tid; i < H * CH; i += C::NT) {
      const int hh = i / CH, cc = i % CH;
      *reinterpret_cast<uint4*>(&qlds[hh * C::QROWE + cc * 8]) =
          *reinterpret_cast<const uint4*>(qrow + (size_t)hh * DQK + cc * 8);
    }
  }
  __syncthreads();
  last = -1;
#pragma unroll
  for (int w = 0; w < C::NW; ++w) last = max(last, s_last[w]);
  c.ntiles = (last + C::NK) / C::NK;

  bf16x8 qf[C::KSR];
  load_q<H, DQK, DV>(a, c, qf);
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
  } else if (!accumulate_fast<H, DQK, DV, AL8>(a, c, qf) && c.tid == 0) {
    a.out[(size_t)c.row * H * DV] = kOverflowMark;
  }
  }
}

hipError_t launch_sparse_attn(const AttnArgs& a, int h, int d_qk, int d_v, int nblocks,
                              hipStream_t s) {
  if (nblocks == 0) return hipSuccess;
  AttnArgs ax = a;
  ax.nrows = nblocks;
  const int exact_grid = nblocks < 1024 ? nblocks : 1024;
  // 8-slot index blocks: topk a multiple of 8 and 32-byte aligned index rows
  const bool al8 = a.topk >= 8 && a.topk % 8 == 0 && (reinterpret_cast<uintptr_t>(a.idx) & 31) == 0;
  if (h == 128 && d_qk == 576 && d_v == 512) {
    if (al8) k_sparse_attn<128, 576, 512, false, true><<<nblocks, 256, 0, s>>>(ax);
    else k_sparse_attn<128, 576, 512, false, false><<<nblocks, 256, 0, s>>>(ax);
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
