// Dense causal attention of an Ulysses head shard on gfx950 MFMA.
//
// Page "自定义Context Parallel特性", section "SDPA Ulysses CP": the dense model's attention is
// wrapped in an all-to-all that turns sequence-sharded Q/K/V into head-sharded ones, so each
// device runs ordinary causal softmax attention over the whole sequence for its own heads.
// Page "context_parallel.md", section "ContextParallel 模式": Pure Ulysses (every rank holds
// the whole sequence of H / cp heads) and Hybrid (a query shard of the sequence against K/V
// gathered over the Colossal group).  Segments carry both placements, and packed documents:
// row r of a segment attends keys k_start .. k_start + pos0 + r.
//
// Mapping: a block owns 256 query rows of one head (8 waves x 32 rows, two waves per SIMD);
// keys stream in tiles of 64 (K rows 384 B, V rows 256 B) through a 3-deep LDS ring filled by
// LDS DMA (global_load_lds, 16 B per lane, no VGPR staging), two tiles in flight while one is
// computed.
//   * Logits: S^T[key, q] = K (A, LDS) x Q^T (B: the wave's 32 query rows, in VGPRs for the
//     whole block), 12 MFMAs 32x32x16 per 32-key half tile.  K rows are chunk-swizzled by
//     swz() (the 16-row fragment reads are conflict-free) and fed in the key permutation of
//     key_perm(), so each lane's accumulators come out as two runs of 8 consecutive keys of
//     its query: the B operand of the value product.
//   * Softmax: a lane pair per query, scaled log2 units.  The running max moves only when a
//     tile's max exceeds it by more than 8 (then the accumulator and the sum are rescaled), so
//     p = 2^(z - m) stays below 2^8 and bf16 / fp32 keep their relative precision.
//   * Output: O^T[col, q] += V^T (A: transposing ds_read_b64_tr_b16 from the row-major V tile,
//     16-byte chunks XOR-swizzled by 4 (row & 3), conflict-free) x P^T (B: the lane's bf16
//     probabilities).  The final 1/l is lane-local.
//   * Causality: a wave skips the tiles after its last row and masks only tiles that cross
//     its diagonal.  Blocks go out latest rows first (longest windows first), heads fastest,
//     so with a multiple of 8 heads each head's blocks share one XCD and its L2.
#include "attn_common.h"

namespace dsa {

namespace {

constexpr int kDq = 192, kDv = 128;
constexpr int kNWd = 8;                     // waves per block
constexpr int kRowsW = 32;                  // query rows per wave
constexpr int kRowsB = kNWd * kRowsW;       // query rows per block
constexpr int kKeysT = 64;                  // keys per tile
constexpr int kKsD = kDq / 16;              // K steps of the logits product
constexpr int kMtD = kDv / 32;              // 32-column M tiles of the value product
constexpr int kKCh = kDq / 8;               // 16-byte chunks per K row
constexpr int kVCh = kDv / 8;               // per V row
constexpr int kKTileE = kKeysT * kDq;       // elements per K tile
constexpr int kVTileE = kKeysT * kDv;       // per V tile
constexpr int kKPc = kKeysT * kKCh / 64;    // 1 KB DMA pieces of a K tile
constexpr int kVPc = kKeysT * kVCh / 64;    // of a V tile
constexpr int kPcW = (kKPc + kVPc) / kNWd;  // pieces per wave and tile
constexpr int kRing = 3;
constexpr float kLazy = 8.f;                // max growth (log2 units) absorbed without rescale
static_assert((kKPc + kVPc) % kNWd == 0, "pieces per wave");
static_assert(kNWd * kRowsW * kDv <= kRing * kKTileE, "output staging fits the K ring");

__device__ __forceinline__ int vswz(int row) { return 4 * (row & 3); }

// One DMA piece (1 KB: 64 lanes x 16 B) of a tile: LDS byte address m0v, per-lane source
// offset voff (bytes) from base.
__device__ __forceinline__ void dma_piece(unsigned m0v, unsigned voff, const uint16_t* base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m0v), "v"(voff), "s"(base) : "memory", "m0");
}

}  // namespace

__global__ __launch_bounds__(kNWd * 64) void k_dense_attn(DenseArgs a) {
  // ring slot s: K tile at ring + s kKTileE, V tile at ring + kRing kKTileE + s kVTileE
  __shared__ __attribute__((aligned(16))) uint16_t ring[kRing * (kKTileE + kVTileE)];

  const int H = a.h;
  const int head = (int)blockIdx.x % H;
  const int qblk = (int)blockIdx.x / H;
  const int sg = seg_of_block(a.segs, qblk);
  const int nb = a.segs.blk_off[sg + 1] - a.segs.blk_off[sg];
  const int r0 = (nb - 1 - (qblk - a.segs.blk_off[sg])) * kRowsB;   // latest rows first
  const int nrows = min(kRowsB, a.segs.q_len[sg] - r0);
  const int qrow0 = a.segs.q_start[sg] + r0;       // first local query row of the block
  const int p0 = a.segs.pos0[sg] + r0;             // its position in the key sequence
  const int kst = a.segs.k_start[sg];
  const int plast = p0 + nrows - 1;                // last position of the block
  const int T = plast / kKeysT + 1;                // key tiles the block needs

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int hl = lane & 31, g = lane >> 5;
  // this wave's rows: 32 wave + hl of the block; rows past nrows compute on the block's last
  // row and are not written, and a wave with no row left computes nothing
  const bool wactive = kRowsW * wave_u < nrows;
  const int wrow = min(kRowsW * wave + hl, nrows - 1);
  const int qpos = p0 + kRowsW * wave + hl;
  const int wpos_lo = p0 + kRowsW * wave_u;
  const int t_last = min(wpos_lo + kRowsW - 1, plast) / kKeysT;   // last tile of this wave

  const unsigned ring_lds = (unsigned)(size_t)(lds_u16_ptr_t)ring;
  // DMA of tile t into ring slot s: wave w copies pieces w kPcW .. + kPcW - 1 of the 40 (K
  // pieces first); key rows past the block's last position are clamped to it (in bounds,
  // masked by causality)
  auto issue_piece = [&](int t, int s, int i) {
    const int kbase = kst + t * kKeysT;
    const int klast = kst + plast;
    {
      const int pc = wave_u * kPcW + i;
      if (pc < kKPc) {
        const int f = pc * 64 + lane;
        const int row = f / kKCh, ch = f - row * kKCh;
        const int key = min(kbase + row, klast);
        const unsigned voff = ((unsigned)(key * H + head) * kDq + (unsigned)((ch ^ swz(row)) * 8)) * 2u;
        dma_piece(ring_lds + (unsigned)(s * kKTileE * 2 + pc * 1024), voff, a.k);
      } else {
        const int f = (pc - kKPc) * 64 + lane;
        const int row = f / kVCh, ch = f - row * kVCh;
        const int key = min(kbase + row, klast);
        const unsigned voff = ((unsigned)(key * H + head) * kDv + (unsigned)((ch ^ vswz(row)) * 8)) * 2u;
        dma_piece(ring_lds + (unsigned)(kRing * kKTileE * 2 + s * kVTileE * 2 + (pc - kKPc) * 1024),
                  voff, a.v);
      }
    }
  };
  auto issue_tile = [&](int t, int s) {
#pragma unroll
    for (int i = 0; i < kPcW; ++i) issue_piece(t, s, i);
  };
  static_assert(2 * kPcW <= kKsD, "one DMA piece every second K step of the logits");

  // prologue: tiles 0 and 1 in flight with the wave's Q rows (B operand: lane (hl, g) holds
  // dims 16 ks + 8 g .. + 7 of row hl)
  issue_tile(0, 0);
  if (T > 1) issue_tile(1, 1);
  bf16x8 qf[kKsD];
  {
    const uint16_t* qp = a.q + ((size_t)(qrow0 + wrow) * H + head) * kDq + g * 8;
#pragma unroll
    for (int ks = 0; ks < kKsD; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + ks * 16));
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // DMA is not tracked by the compiler
  __builtin_amdgcn_s_waitcnt(0x0F70);                // compiler-visible: Q landed
  __syncthreads();

  f32x16 o[kMtD];
#pragma unroll
  for (int mt = 0; mt < kMtD; ++mt) o[mt] = (f32x16){};
  float m = kNegInf, lsum = 0.f;
  const float sl2 = a.scale_log2;
  // per-lane LDS offsets (elements): the logits A rows (key_perm; +32 rows for the second
  // half tile, same swizzle) and the transposing value reads
  const int arow = key_perm(hl);
  const int asw = swz(arow);
  const int G = lane >> 4, i16 = lane & 15;
  const int vlow = 2 * (G & 1) + ((i16 & 3) >> 1);
  const int vrow = (G >> 1) * 8 + (i16 >> 2);

  typedef __attribute__((address_space(3))) const bf16x8* lds_cb8_t;
  for (int t = 0, s = 0; t < T; ++t, s = (s == kRing - 1 ? 0 : s + 1)) {
    const int s2 = s == 0 ? 2 : s - 1;             // slot of tile t + 2 (= slot of t - 1)
    // tile t + 2's DMA: between the logits' K steps when the wave computes this tile (issued
    // by all eight waves together at the step start, the 40 DMA instructions queue while the
    // matrix pipe idles), else here
    const bool busy = wactive && t <= t_last;
    if (t + 2 < T && !busy) issue_tile(t + 2, s2);
    if (busy) {
      const lds_cptr_t kt = (lds_cptr_t)ring + s * kKTileE;
      const lds_cptr_t vt = (lds_cptr_t)ring + kRing * kKTileE + s * kVTileE;
      f32x16 sc[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
      for (int ks = 0; ks < kKsD; ++ks) {
        const int ch = ((2 * ks + g) ^ asw) * 8;
        const bf16x8 a0 = *(lds_cb8_t)(kt + arow * kDq + ch);
        const bf16x8 a1 = *(lds_cb8_t)(kt + (arow + 32) * kDq + ch);
        sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], sc[0], 0, 0, 0);
        sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], sc[1], 0, 0, 0);
        if (t + 2 < T && ks % 2 == 0 && ks / 2 < kPcW) issue_piece(t + 2, s2, ks / 2);
      }
      const int kt0 = t * kKeysT;
      if (kt0 + kKeysT - 1 > wpos_lo) {            // the tile crosses this wave's diagonal
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kt0 + 32 * j + acc_key(r, g) > qpos) sc[j][r] = kNegInf;
      }
      float mx = kNegInf;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[j][r]);
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_int(mx), __float_as_int(mx),
                                                       false, false);
      mx = fmaxf(__int_as_float(pr[0]), __int_as_float(pr[1])) * sl2;
      if (mx > m + kLazy) {                        // first tile, or a large growth of the max
        const float alpha = __builtin_amdgcn_exp2f(m - mx);   // 0 while m = -inf
#pragma unroll
        for (int mt = 0; mt < kMtD; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[mt][r] *= alpha;
        lsum *= alpha;
        m = mx;
      }
      const float msub = m == kNegInf ? 0.f : m;
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      bf16x8 pf[4];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float e0 = __builtin_amdgcn_exp2f(fmaf(sc[j][r], sl2, -msub));
          const float e1 = __builtin_amdgcn_exp2f(fmaf(sc[j][r + 1], sl2, -msub));
          const bf16x2 pk = {(__bf16)e0, (__bf16)e1};
          // the sum takes the same bf16-rounded probabilities the value product uses
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, lsum, false);
          pf[2 * j + (r >> 3)][r & 7] = pk[0];
          pf[2 * j + (r >> 3)][(r & 7) + 1] = pk[1];
        }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int mt = 0; mt < kMtD; ++mt) {
          // V^T fragment: rows 16 kk + vrow (+4), logical chunk 4 mt + vlow at physical
          // 4 (mt ^ (row & 3)) + vlow
          const int r = 16 * kk + vrow;
          const lds_cptr_t b = vt + r * kDv + (4 * (mt ^ (i16 >> 2)) + vlow) * 8 + (i16 & 1) * 4;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)b);
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr_t)(b + 4 * kDv));
          const bf16x8 vf = __builtin_bit_cast(
              bf16x8, (i16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], o[mt], 0, 0, 0);
        }
      }
    }
    // tile t + 1 landed for every wave (t + 2 may be in flight); slot s is free
    if (t + 2 < T) wait_vm_barrier<kPcW>();
    else wait_vm_barrier<0>();
  }

  // epilogue: the lane pair's sums, 1/l, rows staged in LDS (the ring is free: the loop's
  // last barrier is behind every wave) and written as whole 256-byte rows
  {
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_int(lsum), __float_as_int(lsum),
                                                     false, false);
    lsum = __int_as_float(pr[0]) + __int_as_float(pr[1]);
  }
  if (!wactive) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) u32x2* lds_u2_t;
  typedef __attribute__((address_space(3))) const u32x4* lds_cu4_t;
  // row hl of the wave's staging area: 8-byte unit u (4 columns) at unit u ^ hl
  const lds_u16_ptr_t stg = (lds_u16_ptr_t)ring + wave * (kRowsW * kDv);
#pragma unroll
  for (int mt = 0; mt < kMtD; ++mt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int u = mt * 8 + q4 * 2 + g;
      const uint32_t lo = (uint32_t)f32_to_bf16(o[mt][q4 * 4 + 0] * inv) |
                          ((uint32_t)f32_to_bf16(o[mt][q4 * 4 + 1] * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(o[mt][q4 * 4 + 2] * inv) |
                          ((uint32_t)f32_to_bf16(o[mt][q4 * 4 + 3] * inv) << 16);
      *(lds_u2_t)(stg + hl * kDv + (u ^ hl) * 4) = (u32x2){lo, hi};
    }
  if (a.lse && g == 0 && kRowsW * wave + hl < nrows)
    a.lse[(size_t)(qrow0 + kRowsW * wave + hl) * H + head] =
        (m + __log2f(lsum)) * kLn2;
  // each instruction: 4 rows x 256 B; lane L carries 16-byte chunk L % 16 of row 4 it + L / 16,
  // whose two units sit in chunk c ^ (row >> 1), swapped when the row is odd (the own wave's
  // LDS writes are ordered before these reads)
#pragma unroll
  for (int it = 0; it < kRowsW / 4; ++it) {
    const int row = it * 4 + (lane >> 4), c = lane & 15;
    u32x4 v = *(lds_cu4_t)(stg + row * kDv + (c ^ (row >> 1)) * 8);
    if (row & 1) v = (u32x4){v[2], v[3], v[0], v[1]};
    if (kRowsW * wave + row < nrows)
      *reinterpret_cast<u32x4*>(a.out + ((size_t)(qrow0 + kRowsW * wave + row) * H + head) * kDv +
                                c * 8) = v;
  }
}

int dense_rows_per_block() { return kRowsB; }

hipError_t launch_dense_attn(const DenseArgs& a, int nqblk, hipStream_t s) {
  if (nqblk == 0 || a.h == 0) return hipSuccess;
  k_dense_attn<<<nqblk * a.h, kNWd * 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dsa
