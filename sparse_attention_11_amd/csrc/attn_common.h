// Tile machinery shared by the sparse-attention forward and backward kernels: the latent-row
// gather into LDS (per-row and flat LDS-DMA forms, scalar index reads), the LDS row swizzle,
// the MFMA key permutation and the per-row context.  Kernel argument structs only need the
// fields kv, n_k, topk and q used here.
#ifndef DSA_ATTN_COMMON_H
#define DSA_ATTN_COMMON_H

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
  // Shape of the ring fast path (four tile buffers, all of Q in VGPRs): the logits of tile
  // t+1 are interleaved with the output product of tile t (each wave: its own heads, all value
  // columns), one barrier per tile.
  static constexpr bool PIPE = H == 128 && DV == 512 && NW == 4 && FLAT && NI <= KS;
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
template <int H, int DQK, int DV, class Args>
__device__ __forceinline__ void gather_row(const Args& a, const RowCtx& c, int id, int key,
                                           uint16_t* dst) {
  using C = AttnCfg<H, DQK, DV>;
  // empty slot: any in-bounds row, masked later; the id is wave-uniform (one row per call),
  // made explicit so the row base is an SGPR pair as the DMA's address operand requires
  id = __builtin_amdgcn_readfirstlane((id < 0 || id >= a.n_k) ? 0 : id);
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
template <int H, int DQK, int DV, class Args>
__device__ __forceinline__ void gather_tile(const Args& a, const RowCtx& c, int t,
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
template <int H, int DQK, int DV, bool AL8, class Args>
__device__ __forceinline__ TileIdx<H, DQK, DV> load_tile_idx_s(const Args& a,
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
template <int H, int DQK, int DV, class Args>
__device__ __forceinline__ unsigned tile_bits(const Args& a, const TileIdx<H, DQK, DV>& ti) {
  constexpr int RPW = AttnCfg<H, DQK, DV>::NK / AttnCfg<H, DQK, DV>::NW;
  unsigned m = 0;
#pragma unroll
  for (int j = 0; j < RPW; ++j) m |= (ti.v[j] >= 0 && ti.v[j] < a.n_k) ? (1u << j) : 0u;
  return m;
}

template <int H, int DQK, int DV, class Args>
__device__ __forceinline__ void gather_tile_s(const Args& a, const RowCtx& c,
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

// Flat gather of this wave's rows of a tile.  wb: LDS byte address of the wave's first row;
// so: byte offsets of the rows in kv, scalars (0 for empty slots: row 0 is copied and masked
// later).  Each lane picks the one of the (at most two) rows its chunk falls in.
template <int H, int DQK, int DV, class Args>
__device__ __forceinline__ void gather_tile_flat_so(const Args& a, const RowCtx& c,
                                                    const unsigned* so, const unsigned* loff,
                                                    unsigned wb) {
  using C = AttnCfg<H, DQK, DV>;
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

// The same from the tile's slot indices (-1 or out of range: empty).
template <int H, int DQK, int DV, class Args>
__device__ __forceinline__ void gather_tile_flat(const Args& a, const RowCtx& c,
                                                 const TileIdx<H, DQK, DV>& ti,
                                                 const unsigned* loff, unsigned wb) {
  using C = AttnCfg<H, DQK, DV>;
  unsigned so[C::RPW];
#pragma unroll
  for (int j = 0; j < C::RPW; ++j)
    so[j] = (unsigned)ti.v[j] < (unsigned)a.n_k ? (unsigned)ti.v[j] * (C::CPR * 16u) : 0u;
  gather_tile_flat_so<H, DQK, DV>(a, c, so, loff, wb);
}

// Wait until at most N of this wave's vector-memory instructions are outstanding, then meet
// the other waves at a barrier (one asm block, so no memory access moves across it).
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int H, int DQK, int DV, class Args>
__device__ __forceinline__ unsigned tile_vmask(const Args& a, const RowCtx& c, int t) {
  const int slot = t * AttnCfg<H, DQK, DV>::NK + c.hl;
  const int id = slot < a.topk ? c.idx_row[slot] : -1;
  return (unsigned)__ballot(id >= 0 && id < a.n_k);
}

template <int H, int DQK, int DV, class Args>
__device__ __forceinline__ void load_q(const Args& a, const RowCtx& c, bf16x8* qf) {
  using C = AttnCfg<H, DQK, DV>;
  const bool hv = (H % 32 == 0) || c.head < H;
  const uint16_t* qp = a.q + ((size_t)c.row * H + (hv ? c.head : 0)) * DQK + c.g * 8;
#pragma unroll
  for (int ks = 0; ks < C::KSR; ++ks) {
    const uint4 v = *reinterpret_cast<const uint4*>(qp + ks * 16);
    qf[ks] = hv ? __builtin_bit_cast(bf16x8, v) : (bf16x8){};
  }
}

// The last slot index (slots tid, tid + NT, ...) of a row's index list that holds a valid
// key, as seen by this thread (-1 if none).  The loads go out eight at a time with clamped
// addresses, so a list of up to 8 * NT slots costs one memory round trip, not one per slot.
template <int NT>
__device__ __forceinline__ int thread_last_valid(const int32_t* idx_row, int topk, int n_k,
                                                 int tid) {
  int last = -1;
  for (int base = 0; base * NT < topk; base += 8) {
    int v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = idx_row[min((base + j) * NT + tid, topk - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sl = (base + j) * NT + tid;
      if (sl < topk && v[j] >= 0 && v[j] < n_k) last = sl;
    }
  }
  return last;
}

// Per-row context of a backward-style kernel (one workgroup per row of a chunk; the argument
// struct has idx, topk and n_k).
template <class Args>
__device__ __forceinline__ RowCtx make_ctx(const Args& a, int row) {
  RowCtx c;
  c.row = row;
  c.tid = threadIdx.x;
  c.lane = c.tid & 63;
  c.wave = c.tid >> 6;
  c.wave_u = __builtin_amdgcn_readfirstlane(c.wave);
  c.hl = c.lane & 31;
  c.g = c.lane >> 5;
  c.head = c.wave * 32 + c.hl;
  c.idx_row = a.idx + (size_t)row * a.topk;
  c.flags = nullptr;
  c.vm = nullptr;
  c.qlds = nullptr;
  return c;
}

// Row of this workgroup; with xcd_remap (grid a multiple of 8) consecutive rows go to one
// XCD (workgroups are dealt to the 8 XCDs round-robin), so rows that share keys share an L2.
template <class Args>
__device__ __forceinline__ int block_row(const Args& a) {
  int blk = blockIdx.x;
  if (a.xcd_remap) blk = (blk & 7) * ((int)gridDim.x >> 3) + (blk >> 3);
  return blk;
}

// Number of 32-slot tiles up to the row's last valid index (block-wide; one barrier).
template <int H, int DQK, int DV, class Args>
__device__ __forceinline__ int row_tiles(const Args& a, const RowCtx& c, int* s_last) {
  using C = AttnCfg<H, DQK, DV>;
  int last = thread_last_valid<C::NT>(c.idx_row, a.topk, a.n_k, c.tid);
  last = (int)wave_max_u32((unsigned)(last + 1)) - 1;   // (last >= -1)
  if (c.lane == 0) s_last[c.wave] = last;
  __syncthreads();
  last = -1;
#pragma unroll
  for (int w = 0; w < C::NW; ++w) last = max(last, s_last[w]);
  return (last + C::NK) / C::NK;
}

// Transposed fragment of a row-major LDS matrix with `cols` columns: within each 16-lane
// group, lane i supplies row r0 + i/4 (r0 + 4 + i/4 for the second half), columns
// c0 + 4 (i % 4) .. +3, and receives column c0 + i of rows r0 .. r0 + 7.
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* m, int cols, int r0, int c0, int i) {
  const lds_cptr_t b = (lds_cptr_t)m + (r0 + (i >> 2)) * cols + c0 + (i & 3) * 4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)b);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(b + 4 * cols));
  return __builtin_bit_cast(bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// Copy `bytes` (a multiple of 1024) from global `src` to LDS byte address `lds` by LDS DMA,
// one 1 KB piece per wave instruction, pieces spread over the block's NW waves.  Completion
// is not tracked by the compiler: wait with vmcnt before reading.
template <int NW>
__device__ __forceinline__ void dma_copy_flat(unsigned lds, const void* src, int bytes, int wave_u,
                                              int lane) {
  for (int i = wave_u; i < bytes / 1024; i += NW) {
    const unsigned voff = (unsigned)i * 1024u + (unsigned)lane * 16u;
    const unsigned m0v = lds + (unsigned)i * 1024u;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(m0v), "v"(voff), "s"(src) : "memory", "m0");
  }
}

// Q[row, :, DQR:] into the padded LDS rows of `qlds` by LDS DMA (no registers held).  The
// padding chunk at the end of each LDS row copies a harmless chunk of the same Q row.
template <int H, int DQK, int DV, class Args>
__device__ __forceinline__ void stage_q_tail(const Args& a, const RowCtx& c, uint16_t* qlds) {
  using C = AttnCfg<H, DQK, DV>;
  if constexpr (C::DQL > 0) {
    constexpr int RC = C::QROWE / 8;                   // 16-byte chunks per padded LDS row
    constexpr int NQI = (H * RC * 16 + 1023) / 1024;   // full-wave DMA pieces
    static_assert(H * RC * 16 == NQI * 1024, "padded Q rows fill whole DMA pieces");
    const uint16_t* qrow = a.q + (size_t)c.row * H * DQK;
    const unsigned qlds_lds = (unsigned)(size_t)(lds_u16_ptr_t)qlds;
    for (int i = c.wave_u; i < NQI; i += C::NW) {
      const int f = i * 64 + c.lane;
      const int hh = f / RC, ch = f - hh * RC;
      const unsigned voff = (unsigned)((hh * DQK + C::DQR + (ch < RC - 1 ? ch * 8 : 0)) * 2);
      const unsigned m0v = qlds_lds + (unsigned)i * 1024u;
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(m0v), "v"(voff), "s"(qrow) : "memory", "m0");
    }
  }
}

// Index ring: a row's slot indices reach LDS in chunks of eight tiles by LDS DMA, so a tile
// loop needs no compiler-tracked vector load (the compiler does not see the tile gathers, and
// its wait for such a load would also drain every gather in flight) and no scalar load (whose
// wait, shared with LDS reads, would stall the first LDS read after it).
constexpr int kIdxChunk = 256;   // index slots per chunk (eight tiles); the LDS ring holds two

typedef __attribute__((address_space(3))) const int32_t* lds_ci32_t;

// Index chunk ch (slots 256 ch .. 256 ch + 255 of the row, reads clamped to the row's last
// slot) into ring half ch % 2 at LDS byte address idxr: each wave copies 64 slots with one
// dword LDS DMA.  Completion is tracked by hand (vmcnt before a barrier).
template <int H, int DQK, int DV, class Args>
__device__ __forceinline__ void idx_chunk_dma(const Args& a, const RowCtx& c, int ch,
                                              unsigned idxr) {
  const int slot = min(ch * kIdxChunk + c.wave_u * 64 + c.lane, a.topk - 1);
  const unsigned voff = (unsigned)slot * 4u;
  const unsigned m0v = idxr + (unsigned)((ch & 1) * kIdxChunk * 4) + (unsigned)c.wave_u * 256u;
  const int32_t* base = c.idx_row;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(m0v), "v"(voff), "s"(base) : "memory", "m0");
}

// A slot index as the gather uses it: byte offset of its latent row in kv (0 for a slot past
// topk or an index outside [0, n_k): such rows are gathered from row 0 and masked); returns
// the validity ballot.
template <int H, int DQK, int DV, class Args>
__device__ __forceinline__ uint64_t decode_slot(const Args& a, int v, int slot, unsigned& off) {
  using C = AttnCfg<H, DQK, DV>;
  const bool ok = slot < a.topk && (unsigned)v < (unsigned)a.n_k;
  off = ok ? (unsigned)v * (C::CPR * 16u) : 0u;
  return __ballot(ok);
}

// Row offsets (scalars) of this wave's eight rows of a tile whose slots sit in lanes
// lane0 .. lane0 + 31 of `off`.
template <int H, int DQK, int DV>
__device__ __forceinline__ void wave_row_offsets(const RowCtx& c, unsigned off, int lane0,
                                                 unsigned* so) {
#pragma unroll
  for (int j = 0; j < AttnCfg<H, DQK, DV>::RPW; ++j)
    so[j] = __builtin_amdgcn_readlane(off, lane0 + c.wave_u * AttnCfg<H, DQK, DV>::RPW + j);
}

}  // namespace

}  // namespace dsa

#endif  // DSA_ATTN_COMMON_H
