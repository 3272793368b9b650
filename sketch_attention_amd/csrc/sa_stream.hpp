// Streamed, software-pipelined fused pass for bf16 inputs on gfx950.
//
// Same operation and work split across groups as the lockstep pass in
// sa_fused.hpp (SequenceO1 close-reading page, section 2.1 for the affinity,
// the prototype-axis softmax and the aggregation; section 2.4 for the fused,
// on-chip shape): s'_ji = M_j . x_i with the folded M, a_ji = 2^s'_ji /
// sum_j' 2^s'_j'i, X~_j += a_ji x_i, float32 partial sketches per (group,
// user) piece reduced by a second kernel.
//
// What changes is the schedule inside a group.  WJ waves split the
// prototypes (KW each) and WI split the rows; a wave owns RW = 16 * RB rows
// of every tile of NT = RW * WI rows.  The group walks one list of tiles
// (never crossing a user boundary) over all the pieces it owns, and each
// wave keeps two affinity tiles in flight:
//
//   iteration t  (one barrier at its end)
//     issue the LDS DMA of tile t+NS-1 into the slot tile t-1 left
//     S(t+1) = X(t+1) . M^T          matrix cores (M held in registers)
//     factors of tile t               row sums of all waves from LDS, 1/sum,
//                                     spread to the lanes by DPP broadcasts
//     A(t) = S(t) * factors -> bf16   VALU
//     acc += A(t) . X(t)              matrix cores
//     S(t+1) <- 2^S(t+1), row sums    VALU + DPP, this wave's sums to LDS
//     flush acc when tile t ends a piece
//
// so the affinity product of one tile overlaps the normalisation of the
// previous one and the aggregation product overlaps the exponentials of the
// next one.
//
// X goes from HBM straight into a ring of NS LDS tiles by LDS DMA
// (global_load_lds_dwordx4: 64 lanes x 16 bytes land at consecutive LDS
// addresses), issued NS - 1 tiles ahead and awaited with explicit vmcnt waits
// before the barrier that publishes a tile, so no register or LDS store
// instruction touches X on its way in.  Rows are stored unpadded with their
// 16-byte chunks XOR-swizzled (chunk c of row r at c ^ sw(r)); each DMA lane
// reads the global chunk that belongs at its LDS position.  The swizzle keeps
// both read patterns free of bank conflicts: the affinity's 16-byte fragment
// reads (16 rows, one chunk) and the aggregation's transposing reads.
// The aggregation needs X with the row index along each lane's reduction
// slots; gfx950's transposing LDS read (ds_read_b64_tr_b16) delivers exactly
// that from the row-major tile: within a 16-lane group, output lane o gets
// element o % 4 of the 8-byte words read by lanes o / 4 + 4e, e = 0..3.  Lane
// s of group g therefore reads row 4g + s / 4, columns 4 (s % 4) .. +3 of a
// 16-column block, and receives one column of four consecutive rows.
//
// Rows past the end of a piece are loaded as copies of its last row (loads
// never leave the piece) and get factor 0, so they add nothing to the sketch.
// The softmax takes 2^s' without a shift; when the total of a row leaves
// [2^-100, 2^100] the wave holding it recomputes its rows with the
// max-shifted softmax on its own (an online max/sum pass over all
// prototypes, M read from global
// memory), so no other wave waits for it.
#pragma once

#include <type_traits>

#include "sa_fused.hpp"

namespace sa {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;


// Integer sum over the 16 lanes of a DPP row (every lane gets the total).
__device__ __forceinline__ int row16_sum_i(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);  // row_mirror
  return x;
}

// Value of lane n of this lane's 16-lane row (DPP row_newbcast).
template <int n>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + n, 0xF, 0xF,
                                                                false));
}

typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// LDS reads at 32-bit LDS byte addresses (constant offsets fold into the
// instructions' offset fields); lds_tr16 returns four consecutive rows of one
// column, see the header comment.
__device__ __forceinline__ bf16x8 lds_b128(uint32_t byte) { return *(const lds_bf16x8*)(size_t)byte; }
__device__ __forceinline__ u32x2 lds_tr16(uint32_t byte) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(size_t)byte);
  return __builtin_bit_cast(u32x2, v);
}

// LDS DMA of one 1 KB block: lane i reads 16 bytes at sbase + voff and they
// land at LDS byte lds_byte + 16 i.  In assembly so that the compiler does
// not track it (it would wait for every outstanding DMA before any LDS read
// it cannot prove disjoint); the kernel orders it with wait_vm before the
// barrier that publishes the tile.  M0 is written one instruction ahead of
// its use by the DMA, as the hazard rules require.  No output registers.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_byte)
               : "memory", "m0");
}
// LDS DMA of 64 dwords: lane i reads 4 bytes at sbase + voff and they land
// at LDS byte lds_byte + 4 i (same ordering rules as dma16).
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds_byte)
               : "memory", "m0");
}
// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt and
// lgkmcnt left at their maxima).  Vector-memory loads complete in order, so
// this waits for every load but the N most recent.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Chunk swizzle of LDS row r (16-byte chunks, D / 8 per row), a function of
// r % 16.  Measured on gfx950: 16-byte reads are served 32 lanes at a time
// over 128 four-byte banks, the 8-byte transposing reads 32 lanes at a time
// over 64 banks.  The affinity's reads (32 lanes: rows l16 of one parity
// class per 512 bytes, chunks c, c + 1) and the transposing reads (32 lanes:
// rows 0..7 or 8..15, chunks 2 cb, 2 cb + 1) are then conflict-free when
// sw / 2 takes distinct values over each of those row sets:
//   d = 128: sw / 2 = 4 ((r ^ r / 8) % 2) + (r / 2) % 4
//   d = 64:  sw / 2 = 2 ((r / 4) % 2) + ((r / 2 ^ r / 8) % 2)
template <int D>
__device__ __forceinline__ constexpr int chunk_sw(int r) {
  return D == 128 ? 8 * ((r ^ (r >> 3)) & 1) + 2 * ((r >> 1) & 3) : 4 * ((r >> 2) & 1) + 2 * (((r >> 1) ^ (r >> 3)) & 1);
}

// The tile list of one work group: pieces (user segments) of [r_begin,
// r_end), each cut into tiles of nt rows.  Every lane examines up to four
// users at once (no chain of dependent loads): u_first is the last user
// starting at or before r_begin (a prefix, offsets being non-decreasing; it is
// the user holding row r_begin, so first_end = offsets[u_first + 1] >
// r_begin, read from the lane that loaded it), ntot the sum of the pieces'
// tile counts.  The kernels issue the loads (tile_list_loads) before their
// folded-matrix loads and first tile DMA and finish the scan after those:
// vector-memory loads complete in order, so waiting for the offsets then does
// not wait for the larger transfers issued after them.
struct TileList {
  int u_first, ntot;
  int64_t first_end;
};
struct OffsetLoads {
  int64_t a[4], b[4];  // offsets[lane + 64 q] and offsets[lane + 64 q + 1] (0 past the users)
};
__device__ __forceinline__ OffsetLoads tile_list_loads(const FusedArgs& args, int lane) {
  OffsetLoads o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int uu = lane + 64 * q;
    o.a[q] = 0;
    o.b[q] = 0;
    if (uu < args.users) {
      o.a[q] = args.offsets[uu];
      o.b[q] = args.offsets[uu + 1];
    }
  }
  return o;
}
__device__ __forceinline__ TileList tile_list(const FusedArgs& args, const OffsetLoads& o, int64_t r_begin,
                                              int64_t r_end, int nt, int lane) {
  int cnt = 0, tiles = 0;
  int64_t first_end = r_end;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int uu = lane + 64 * q;
    const int64_t a = o.a[q], b = o.b[q];
    if (uu < args.users) {
      cnt += a <= r_begin ? 1 : 0;
      const int64_t lo = a > r_begin ? a : r_begin, hi = b < r_end ? b : r_end;
      if (hi > lo) tiles += (int)((hi - lo + nt - 1) / nt);
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(uu < args.users && a <= r_begin && b > r_begin);
    if (hit != 0) {
      const int src = __builtin_ctzll(hit);
      first_end = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(b >> 32), src) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane((int)b, src));
    }
  }
  cnt = row16_sum_i(cnt);
  tiles = row16_sum_i(tiles);
  TileList t;
  t.u_first = __builtin_amdgcn_readlane(cnt, 0) + __builtin_amdgcn_readlane(cnt, 16) +
              __builtin_amdgcn_readlane(cnt, 32) + __builtin_amdgcn_readlane(cnt, 48) - 1;
  t.ntot = __builtin_amdgcn_readlane(tiles, 0) + __builtin_amdgcn_readlane(tiles, 16) +
           __builtin_amdgcn_readlane(tiles, 32) + __builtin_amdgcn_readlane(tiles, 48);
  t.first_end = first_end;
  return t;
}

template <int D, int KW, int WJ, int WI, int RB, int PF, int SB>
struct StreamGeom {
  static_assert(KW % 16 == 0 && (D == 64 || D == 128) && PF >= 1 && PF <= 3 && (RB == 2 || RB == 4) &&
                    (SB == 1 || SB == 2),
                "tile shape");
  static constexpr int NW = WJ * WI;
  static constexpr int THREADS = 64 * NW;
  static constexpr int RW = 16 * RB;           // rows per wave and tile
  static constexpr int NT = RW * WI;           // rows per tile
  static constexpr int JB = KW / 16;
  static constexpr int CB = D / 16;
  static constexpr int CS = D / 32;
  static constexpr int KPAD = KW * WJ;
  static constexpr int CH = D / 8;             // 16-byte chunks per row
  // ring of X tiles: the tiles read by a step, the ones the affinity runs
  // ahead of the aggregation, and PF - 1 more in flight
  static constexpr int NS = (SB == 2 ? 4 : 3) + PF - 1;
  static constexpr int SLOT_BYTES = NT * D * 2;
  static constexpr int XR_BYTES = NS * SLOT_BYTES;
  static constexpr int NI = SLOT_BYTES / 1024;  // DMA blocks per tile
  static_assert(SLOT_BYTES % 1024 == 0, "tile of whole DMA blocks");
  static constexpr int NIW = (NI + NW - 1) / NW;  // DMA blocks per wave and tile (some waves may have one fewer)
  static constexpr int RPI = 1024 / (2 * D);      // rows per DMA block
  // row sums of every wave, two parities.  WJ % 4 == 0: [2][WJ / 4][NTP][4]
  // floats, row R at padded position R + 8 (R / 32), so the 16-byte reads of
  // the combine (32 lanes, rows 16 ib + 4 g + r) hit distinct banks; else
  // [2][NT][WJ].
  static constexpr int NTP = NT + 8 * ((NT + 31) / 32);
  static constexpr int XL_BYTES = WJ % 4 == 0 ? 2 * (WJ / 4) * NTP * 16 : 2 * NT * WJ * 4;
  // waves that split the rows add their accumulators through LDS when a
  // piece ends: one prototype block of every wave at a time.  When that fits
  // in a tile it uses the ring slot of the tile just aggregated (free until
  // the next step's DMA), else a buffer of its own.
  static constexpr int STAGE_NEED = WI > 1 ? WJ * CB * 64 * 16 : 0;
  static constexpr bool STAGE_IN_RING = STAGE_NEED <= SLOT_BYTES;
  static constexpr int STAGE_BYTES = STAGE_IN_RING ? 0 : STAGE_NEED;
  static constexpr int OFF_XL = XR_BYTES;
  static constexpr int OFF_STAGE = OFF_XL + XL_BYTES;
  // one score buffer: the folded matrix lives in LDS, rows of D bf16 with
  // their 16-byte chunks XOR-swizzled (chunk c of row r at c ^ ((r / P) % CH),
  // P rows per 256 bytes), so fragment reads are conflict-free without padding
  static constexpr int M_BYTES = SB == 1 ? KPAD * D * 2 : 0;
  static constexpr int OFF_M = OFF_STAGE + STAGE_BYTES;
  static constexpr int LDS_BYTES = OFF_M + M_BYTES;
  // vector-memory operations (X blocks) of one wave per tile
  static constexpr int DMA_LO = NI / NW;
  static constexpr int DMA_HI = DMA_LO + 1;  // waves w < NI % NW issue one block more
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CDNA4 compute unit");
};

// PU: one folded matrix per user (args.m_stride apart) instead of one shared
// matrix; a separate instantiation so the shared case carries none of its
// bookkeeping.  HS: the comparator of section 3.1, the softmax taken over the
// history axis instead of the prototype axis (see the main loop below).  The
// two phases of the pass for more prototypes than one work group holds run on
// sa_stream32.hpp.
template <int D, int KW, int WJ, int WI, int RB, int PF, int SB, bool PAD, bool PU, bool HS = false>
__global__ __launch_bounds__(64 * WJ * WI) void sa_stream_kernel(FusedArgs args) {
  using G = StreamGeom<D, KW, WJ, WI, RB, PF, SB>;
  using MF = Mfma<bf16>;
  constexpr int JB = G::JB, CB = G::CB, CS = G::CS, NT = G::NT, RW = G::RW, THREADS = G::THREADS;

  __shared__ __attribute__((aligned(1024))) unsigned char lds[G::LDS_BYTES];
  const uint32_t xr0 = (uint32_t)(size_t)(__attribute__((address_space(3))) unsigned char*)lds;  // LDS byte address
  auto slot_of = [&](int q) { return xr0 + (uint32_t)(q * G::SLOT_BYTES); };
  float* const xl = reinterpret_cast<float*>(lds + G::OFF_XL);
  // index of the row sum of tile row `row` from prototype wave w, parity par
  auto xl_at = [&](int par, int row, int w) {
    if constexpr (WJ % 4 == 0)
      return ((par * (WJ / 4) + w / 4) * G::NTP + row + 8 * (row >> 5)) * 4 + (w & 3);
    else
      return (par * NT + row) * WJ + w;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wj = wave % WJ;
  const int wi = wave / WJ;
  const int rw = wi * RW;     // first tile row of this wave
  const int jbase = wj * KW;  // first prototype of this wave
  // the comparator beyond one block of prototypes (its softmax is per
  // prototype, so blocks need no merge): the blocks of a row range run on one
  // XCD (group_block)
  const int nblk = HS ? args.blocks : 1;
  const GroupBlock gb = group_block(blockIdx.x, gridDim.x, nblk);
  const int blk = HS ? gb.blk : 0;
  const bf16* const X = static_cast<const bf16*>(args.X);
  const bf16* const Mg = static_cast<const bf16*>(args.M) + (int64_t)blk * G::KPAD * D;
  const int k = args.k - blk * G::KPAD;  // real prototypes of this block (may exceed KPAD)

  const int64_t rows = args.rows;
  const int64_t ngroups = gridDim.x / nblk;
  const int64_t grp = gb.grp;
  const int64_t r_begin = grp * rows / ngroups;
  const int64_t r_end = (grp + 1) * rows / ngroups;
  if (r_begin >= r_end) return;
  const OffsetLoads offs = tile_list_loads(args, lane);  // first: see tile_list

  int u_first = 0, ntot = 0;
  int64_t first_end = 0;  // end of the piece holding r_begin
  // A cursor walks the tile list: first row of the tile, end of its piece
  // (both relative to r_begin: a group's range fits in 32 bits, so the
  // per-step bookkeeping stays in 32-bit scalar arithmetic), user.
  const int nrel = (int)(r_end - r_begin);
  struct Cursor {
    int row, end, u;
  };
  auto user_end = [&](int u) {
    const int64_t e = args.offsets[u + 1] - r_begin;
    return e < (int64_t)nrel ? (int)e : nrel;
  };
  auto cursor_begin = [&]() {
    const int64_t e = first_end - r_begin;
    return Cursor{0, e < (int64_t)nrel ? (int)e : nrel, u_first};
  };
  auto cursor_next = [&](Cursor& c) {
    c.row += NT;
    if (c.row >= c.end) {
      c.row = c.end;
      if (c.row < nrel) {
        ++c.u;
        while (c.u < args.users && args.offsets[c.u + 1] - r_begin <= (int64_t)c.row) ++c.u;
        c.end = user_end(c.u);
      }
    }
  };

  // ---- folded matrix: this wave's KW rows as B fragments, in registers
  // (two score buffers) or in the swizzled LDS copy (one score buffer).  One
  // matrix for all users (m_stride 0, loaded at once) or one per user,
  // loaded when the tile whose affinity comes next belongs to another user
  // (ensure_m below).
  constexpr int MP = 256 / (2 * D);  // rows of M per 256 bytes
  bf16x8 mreg[SB == 2 ? JB : 1][SB == 2 ? CS : 1];
  bf16* const Ms = reinterpret_cast<bf16*>(lds + G::OFF_M);
  int moff[CS];  // element offset of chunk 4 cs + g of this lane's rows (the swizzle depends on l16 only)
  auto load_m = [&](int u) {
    const bf16* const Mu = PU ? Mg + (int64_t)u * args.m_stride : Mg;
    if constexpr (SB == 2) {
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        const bf16* mrow = Mu + (int64_t)(jbase + 16 * jb + l16) * D;
#pragma unroll
        for (int cs = 0; cs < CS; ++cs) mreg[jb][cs] = frag_c<D>(mrow, cs, g);
      }
    } else {
      for (int idx = tid; idx < G::KPAD * G::CH; idx += THREADS) {
        const int r = idx / G::CH, c = idx % G::CH;
        *reinterpret_cast<u32x4*>(Ms + r * D + 8 * (c ^ ((r / MP) % G::CH))) =
            *reinterpret_cast<const u32x4*>(Mu + (int64_t)r * D + 8 * c);
      }
    }
  };
  int m_user = -1;  // user whose matrix is loaded
  if constexpr (!PU) {
    load_m(0);  // LDS copy ordered before the first read by the prologue's barrier
    m_user = 0;
  }
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) moff[cs] = 8 * ((4 * cs + g) ^ ((l16 / MP) % G::CH));

  // ---- LDS DMA of one tile into ring slot q: block j = wave + s NW of the
  // tile (RPI rows) lands at slot + 1024 j; lane i of a block holds row
  // j RPI + i / CH, LDS chunk i % CH, i.e. global chunk (i % CH) ^ sw(row).
  // Rows past the piece read its last row (offsets stay non-negative: past
  // the list every lane reads row c.end - 1), so every load is in bounds.
  int dma_row[G::NIW], dma_col[G::NIW];
#pragma unroll
  for (int s = 0; s < G::NIW; ++s) {
    const int j = wave + s * G::NW;
    dma_row[s] = j * G::RPI + lane / G::CH;
    dma_col[s] = 8 * ((lane % G::CH) ^ chunk_sw<D>(dma_row[s]));
  }
  auto issue_tile = [&](const Cursor& c, int q) {
    const int last = c.end - 1 - c.row;  // -1 past the list
    const int64_t b0 = r_begin + (last < 0 ? c.end - 1 : c.row);
    const int lim = last < 0 ? 0 : (last < G::NT ? last : G::NT - 1);
    const bf16* const base = X + b0 * D;
    const uint32_t slot = slot_of(q);
#pragma unroll
    for (int s = 0; s < G::NIW; ++s) {
      const int j = wave + s * G::NW;
      if (G::NI % G::NW == 0 || j < G::NI) {
        const int rr = dma_row[s] < lim ? dma_row[s] : lim;
        dma16(base, (uint32_t)(rr * D + dma_col[s]) * 2u, slot + 1024u * (uint32_t)j);
      }
    }
  };
  // wait until every DMA block of this wave is done but those of the n most
  // recently issued tiles
  auto wait_tiles = [&](auto n_) {
    constexpr int n = decltype(n_)::value;
    if constexpr (G::NI % G::NW == 0) {
      wait_vm<G::DMA_LO * n>();
    } else {
      if (wave < G::NI % G::NW) wait_vm<G::DMA_HI * n>();
      else wait_vm<G::DMA_LO * n>();
    }
  };

  // tile 0 starts at r_begin whatever the users: its DMA goes out before the
  // tile list is known (rows clamped to the group's range; rows of the next
  // user get factor 0)
  issue_tile(Cursor{0, nrel, 0}, 0);

  // ---- the group's tile list
  {
    const TileList tl = tile_list(args, offs, r_begin, r_end, NT, lane);
    u_first = tl.u_first;
    ntot = tl.ntot;
    first_end = tl.first_end;
  }
  // ---- affinity of rows 16 ib + .. with prototypes 16 jb + .. of block `mf`:
  // s[ib][jb][r] = S'^T[rw + 16 ib + 4 g + r][16 jb + l16]
  auto pad_protos = [&](f32x4 (&s)[RB][JB], int j0) {
    if constexpr (PAD) {
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        const bool ok = j0 + 16 * jb + l16 < k;
#pragma unroll
        for (int ib = 0; ib < RB; ++ib)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[ib][jb][r] = ok ? s[ib][jb][r] : -INFINITY;
      }
    }
  };
  // one reduction step (32 columns of d) of the affinity; cs = 0 starts the sums
  // byte offset of chunk 4 cs + g of this lane's row l16 (the swizzle of rows
  // 16 ib + l16 is that of l16)
  uint32_t aoff[CS];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) aoff[cs] = (uint32_t)(2 * (l16 * D + 8 * ((4 * cs + g) ^ chunk_sw<D>(l16))));
  auto xfrag = [&](uint32_t xs, int ib, int cs) { return lds_b128(xs + aoff[cs] + (uint32_t)(2 * (rw + 16 * ib) * D)); };
  auto affinity_cs = [&](f32x4 (&s)[RB][JB], uint32_t xs, int cs) {
    bf16x8 xa[RB];
#pragma unroll
    for (int ib = 0; ib < RB; ++ib) xa[ib] = xfrag(xs, ib, cs);
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int ib = 0; ib < RB; ++ib) {
        bf16x8 mf;
        if constexpr (SB == 2) {
          mf = mreg[jb][cs];
        } else {
          mf = *reinterpret_cast<const bf16x8*>(Ms + (jbase + 16 * jb + l16) * D + moff[cs]);
        }
        s[ib][jb] = MF::run(xa[ib], mf, cs == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[ib][jb]);
      }
  };
  auto affinity = [&](f32x4 (&s)[RB][JB], uint32_t xs) {
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) affinity_cs(s, xs, cs);
    pad_protos(s, jbase);
  };

  // ---- e = 2^s' in place; this wave's row sums to xl[par].  After the
  // transposing butterfly the four lanes of a quad hold the same total and
  // store it to the same word (no branch).
  auto softmax_ib = [&](f32x4 (&s)[RB][JB], int par, int ib) {
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // the first term starts the sum (0 + e is not foldable for -0)
      float acc = fast_exp2(s[ib][0][r]);
      s[ib][0][r] = acc;
#pragma unroll
      for (int jb = 1; jb < JB; ++jb) {
        const float e = fast_exp2(s[ib][jb][r]);
        s[ib][jb][r] = e;
        acc += e;
      }
      p[r] = acc;
    }
    const float z = rows4_sum_scatter(p, l16);
    const int trow = rw + 16 * ib + 4 * g + ((l16 >> 3) << 1) + ((l16 >> 2) & 1);
    xl[xl_at(par, trow, wj)] = z;
  };
  auto softmax_fast = [&](f32x4 (&s)[RB][JB], int par) {
#pragma unroll
    for (int ib = 0; ib < RB; ++ib) softmax_ib(s, par, ib);
  };

  // ---- factors 1 / sum_w l_w.  Lane (g, l16) finishes row
  // rw + 16 ib + 4 g + r with ib = (l16 / 4) % RB, r = l16 % 4, so each row
  // of the wave lives in the 16-lane DPP row g of the lanes that need it; the
  // aggregation takes the factors of its rows by row broadcasts (fac_of).
  // `bad` is set when a row total left the range of the unshifted softmax.
  const int my_ib = (l16 >> 2) % RB, my_r = l16 & 3;
  const int my_row = rw + 16 * my_ib + 4 * g + my_r;  // tile row whose factor this lane finishes
  auto combine_fast = [&](float& f, float& l, bool& bad, int par) {
    if constexpr (WJ % 4 == 0) {
      f32x4 v = *reinterpret_cast<const f32x4*>(xl + xl_at(par, my_row, 0));
#pragma unroll
      for (int w = 4; w < WJ; w += 4) v += *reinterpret_cast<const f32x4*>(xl + xl_at(par, my_row, w));
      l = (v[0] + v[1]) + (v[2] + v[3]);
    } else {
      const float* p = xl + xl_at(par, my_row, 0);
      l = p[0];
#pragma unroll
      for (int w = 1; w < WJ; ++w) l += p[w];
    }
    bad = __builtin_amdgcn_ballot_w64(!(l >= 0x1p-100f && l <= 0x1p100f)) != 0;
    f = __builtin_amdgcn_rcpf(l);
  };
  // factor of row rw + 16 ib + 4 g + r from the lane that holds it
  auto fac_of = [&](float f, int ib, int r) {
    switch (4 * ib + r) {
      case 0: return row_bcast<0>(f);
      case 1: return row_bcast<1>(f);
      case 2: return row_bcast<2>(f);
      case 3: return row_bcast<3>(f);
      case 4: return row_bcast<4>(f);
      case 5: return row_bcast<5>(f);
      case 6: return row_bcast<6>(f);
      case 7: return row_bcast<7>(f);
      case 8: return row_bcast<8>(f);
      case 9: return row_bcast<9>(f);
      case 10: return row_bcast<10>(f);
      case 11: return row_bcast<11>(f);
      case 12: return row_bcast<12>(f);
      case 13: return row_bcast<13>(f);
      case 14: return row_bcast<14>(f);
      default: return row_bcast<15>(f);
    }
  };

  // ---- exact path of one wave (rare): for each of its row blocks, an online
  // max / shifted-sum pass over all prototypes (M fragments from global
  // memory), then its own prototypes' weights 2^(s' - m) with factor 1 / l.
  auto exact_wave = [&](f32x4 (&s)[RB][JB], float& f, uint32_t xs, int u) {
    const bf16* const Mu = PU ? Mg + (int64_t)u * args.m_stride : Mg;
#pragma unroll  // s[ib] must be indexed by constants to stay in registers
    for (int ib = 0; ib < RB; ++ib) {
      bf16x8 xa[CS];
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) xa[cs] = xfrag(xs, ib, cs);
      float m[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      float l[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
      for (int w = 0; w < WJ; ++w) {
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {  // one 16-prototype block at a time (few live registers)
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
          const int j0 = w * KW + 16 * jb;
          const bf16* mrow = Mu + (int64_t)(j0 + l16) * D;
#pragma unroll
          for (int cs = 0; cs < CS; ++cs) a = MF::run(xa[cs], frag_c<D>(mrow, cs, g), a);
          if constexpr (PAD) {
            const bool ok = j0 + l16 < k;
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = ok ? a[r] : -INFINITY;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float mn = fmaxf(m[r], row16_max(a[r]));
            if (mn != -INFINITY) {  // a block of padding only leaves the state as it is
              l[r] = l[r] * fast_exp2(m[r] - mn) + row16_sum(fast_exp2(a[r] - mn));
              m[r] = mn;
            }
          }
          if (w == wj) s[ib][jb] = a;  // this wave's own scores, kept where its fast-path values were
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) s[ib][jb][r] = fast_exp2(s[ib][jb][r] - m[r]);
        if (ib == my_ib && r == my_r) f = 1.f / l[r];
      }
    }
  };

  // ---- aggregation: acc[jb][cb][r] += sum_i a[jbase+16jb+4g+r][i] X[i][16cb+l16].
  // Reduction slot (g, e) of k-step h is tile row rw + 32 h + 16 (e / 4) +
  // 4 g + e % 4, the rows the affinity layout left in that lane.  This lane
  // reads row 4 g + l16 / 4 (+ rw + 32 h + 16 e/4), columns 16 cb + 4 (l16 % 4):
  // chunk 2 cb + (l16 / 2) % 2 at (2 cb + q) ^ sw, i.e. element offset
  // 16 cb ^ (8 (q ^ sw) + 4 (l16 % 2)) in the row, one XOR per column block.
  const uint32_t trb = (uint32_t)(2 * ((4 * g + (l16 >> 2)) * D + 8 * (((l16 >> 1) & 1) ^ chunk_sw<D>(4 * g + (l16 >> 2))) +
                                       4 * (l16 & 1)));
  auto weights_h = [&](bf16x8 (&a)[RB / 2][JB], const f32x4 (&s)[RB][JB], float f, int h) {
    float fac[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) fac[e] = fac_of(f, 2 * h + (e >> 2), e & 3);
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int e = 0; e < 8; ++e) a[h][jb][e] = (bf16)(s[2 * h + (e >> 2)][jb][e & 3] * fac[e]);
  };
  auto weights = [&](bf16x8 (&a)[RB / 2][JB], const f32x4 (&s)[RB][JB], float f) {
#pragma unroll
    for (int h = 0; h < RB / 2; ++h) weights_h(a, s, f, h);
  };
  auto aggregate_h = [&](f32x4 (&acc)[JB][CB], const bf16x8 (&a)[RB / 2][JB], uint32_t xs, int h) {
    const uint32_t xp = xs + (uint32_t)(2 * rw * D) + trb;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const uint32_t xc = xp ^ (uint32_t)(32 * cb);  // the slot and row parts are multiples of 2 D bytes
      const u32x2 lo = lds_tr16(xc + (uint32_t)(2 * 32 * h * D));
      const u32x2 hi = lds_tr16(xc + (uint32_t)(2 * (32 * h + 16) * D));
      const bf16x8 xb = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) acc[jb][cb] = MF::run(a[h][jb], xb, acc[jb][cb]);
    }
  };
  auto aggregate = [&](f32x4 (&acc)[JB][CB], const bf16x8 (&a)[RB / 2][JB], uint32_t xs) {
#pragma unroll
    for (int h = 0; h < RB / 2; ++h) aggregate_h(acc, a, xs, h);
  };

  // ---- flush one (group, user) piece: waves that split the rows add their
  // accumulators through LDS in a fixed order, then one wave per prototype
  // slice writes the slot in the lane layout [wj][jb][cb][lane][4].
  auto flush = [&](f32x4 (&acc)[JB][CB], int u, int q) {
    if constexpr (WI > 1) {
      float* stage = reinterpret_cast<float*>(lds + (G::STAGE_IN_RING ? q * G::SLOT_BYTES : G::OFF_STAGE));
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        for (int st = WI - 1; st >= 1; --st) {
          __syncthreads();
          if (wi == st) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
              *reinterpret_cast<f32x4*>(stage + ((wj * CB + cb) * 64 + lane) * 4) = acc[jb][cb];
          }
          __syncthreads();
          if (wi == st - 1) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
              acc[jb][cb] += *reinterpret_cast<const f32x4*>(stage + ((wj * CB + cb) * 64 + lane) * 4);
          }
        }
      }
    }
    if (wi == 0) {
      // block b's slots follow the (groups + users) slots of block b - 1 (one block in the one-pass kernel)
      float* dst = args.partial + ((int64_t)blk * (ngroups + args.users) + grp + u) * (int64_t)(G::KPAD * D);
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          *reinterpret_cast<f32x4*>(dst + (((wj * JB + jb) * CB + cb) * 64 + lane) * 4) = acc[jb][cb];
    }
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[jb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  f32x4 acc[JB][CB];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[jb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  Cursor cc = cursor_begin();  // tile t (aggregation, flush)
  Cursor cl = cc;              // next tile to load from HBM
  constexpr int NS = G::NS;

  // ---- prologue: DMA of tiles 1 .. NS-2 (tile 0 is on its way); the ring
  // position of tile t is t % NS
  cursor_next(cl);
#pragma unroll
  for (int p = 1; p < NS - 1; ++p) {
    issue_tile(cl, p);
    cursor_next(cl);
  }
  // factor of this lane's row of the tile at cursor c (0 for rows past its piece)
  auto row_ok = [&](const Cursor& c) { return my_row < c.end - c.row; };
  // per-user matrices: the matrix of user u before an affinity of its tile.
  // With the LDS copy, the caller's last barrier ended the reads of the old
  // matrix (the affinity runs once per step) and the copy is published by
  // the barrier that follows it here or in the prologue.
  Cursor ca = cc;  // tile whose affinity comes next (per-user matrices only)
  auto ensure_m = [&](bool barrier_after) {
    if constexpr (PU) {
      if (ca.u != m_user) {
        load_m(ca.u);
        m_user = ca.u;
        if constexpr (SB == 1) {
          if (barrier_after) __syncthreads();
        }
      }
    }
  };
  auto next_affinity_tile = [&]() {
    if constexpr (PU) cursor_next(ca);
  };

  if constexpr (HS) {
    // ---- comparator: A_ji = 2^(s'_ji) / sum_i' 2^(s'_ji') over the rows of
    // the user, i.e. a softmax over the history for each prototype.  Each
    // wave owns its prototypes for every row of a tile (no row split), so the
    // normalisation needs no exchange between waves: per prototype a running
    // maximum hm (raised lazily, only when a tile exceeds it by more than
    // 2^8, which bounds every weight by 256) and per lane a partial sum hl of
    // 2^(s' - hm) over the rows it holds; the accumulator is kept in the
    // scale of hm.  A piece's partial carries (acc, hm, sum hl); the
    // reduction merges the pieces of a user with their maxima.
    static_assert(WI == 1, "the history softmax keeps whole tile columns in one wave");
    float hm[JB], hl[JB];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      hm[jb] = -INFINITY;
      hl[jb] = 0.f;
    }
    f32x4 S[RB][JB];
    bf16x8 a[RB / 2][JB];
    // weights of the tile at cursor c from its scores in S (rows past the piece excluded)
    auto hs_weights = [&](const Cursor& c) {
      const int nv = c.end - c.row;
      if (nv < NT) {
#pragma unroll
        for (int ib = 0; ib < RB; ++ib)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool ok = rw + 16 * ib + 4 * g + r < nv;
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) S[ib][jb][r] = ok ? S[ib][jb][r] : -INFINITY;
          }
      }
      float mnew[JB];
      bool grow = false;
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        float tm = S[0][jb][0];
#pragma unroll
        for (int ib = 0; ib < RB; ++ib)
#pragma unroll
          for (int r = 0; r < 4; ++r) tm = fmaxf(tm, S[ib][jb][r]);
        tm = fmaxf(tm, __shfl_xor(tm, 16));
        tm = fmaxf(tm, __shfl_xor(tm, 32));
        mnew[jb] = fmaxf(hm[jb], tm);
        grow |= mnew[jb] > hm[jb] + 8.f;
      }
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // a piece's first tile, or a jump of the maximum
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const float alpha = hm[jb] == -INFINITY ? 0.f : fast_exp2(hm[jb] - mnew[jb]);
          hl[jb] *= alpha;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float ar = __shfl(alpha, 4 * g + r);  // factor of prototype 16 jb + 4 g + r
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) acc[jb][cb][r] *= ar;
          }
          hm[jb] = mnew[jb];
        }
      }
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        const float mu = hm[jb] == -INFINITY ? 0.f : hm[jb];  // all-padding prototypes: weights 0
#pragma unroll
        for (int ib = 0; ib < RB; ++ib)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = fast_exp2(S[ib][jb][r] - mu);
            S[ib][jb][r] = e;
            hl[jb] += e;
          }
      }
#pragma unroll
      for (int h = 0; h < RB / 2; ++h)
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
          for (int e = 0; e < 8; ++e) a[h][jb][e] = (bf16)S[2 * h + (e >> 2)][jb][e & 3];
    };
    // partial of one piece: acc in the lane layout, then the maxima and the
    // sums of every prototype of the slot
    auto hs_flush = [&](int u) {
      float* dst = args.partial + ((int64_t)blk * (ngroups + args.users) + grp + u) * (int64_t)(G::KPAD * (D + 2));
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          *reinterpret_cast<f32x4*>(dst + (((wj * JB + jb) * CB + cb) * 64 + lane) * 4) = acc[jb][cb];
          acc[jb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        float lt = hl[jb] + __shfl_xor(hl[jb], 16);
        lt += __shfl_xor(lt, 32);
        if (g == 0) {
          dst[G::KPAD * D + jbase + 16 * jb + l16] = hm[jb];
          dst[G::KPAD * D + G::KPAD + jbase + 16 * jb + l16] = lt;
        }
        hm[jb] = -INFINITY;
        hl[jb] = 0.f;
      }
    };
    wait_tiles(std::integral_constant<int, NS - 2>{});
    __syncthreads();
    affinity(S, slot_of(0));
    hs_weights(ca);
    cursor_next(ca);
    wait_tiles(std::integral_constant<int, NS - 3>{});
    __syncthreads();
    // Step t: DMA of tile t+NS-1, aggregation of tile t with the weights made
    // in the step before, the piece's partial when tile t ends it (before the
    // next tile starts a new piece's maxima), affinity and weights of tile
    // t+1, wait for tile t+2, one barrier (the ring only).
    int q0 = 0;
    for (int t = 0; t < ntot; ++t) {
      const int q1 = q0 + 1 < NS ? q0 + 1 : 0;
      const int qn = q0 == 0 ? NS - 1 : q0 - 1;
      issue_tile(cl, qn);
      aggregate(acc, a, slot_of(q0));
      if (cc.row + NT >= cc.end) hs_flush(cc.u);
      if (t + 1 < ntot) {
        affinity(S, slot_of(q1));
        hs_weights(ca);
      }
      cursor_next(ca);
      cursor_next(cc);
      cursor_next(cl);
      q0 = q1;
      wait_tiles(std::integral_constant<int, NS - 3>{});  // tile t+2
      __syncthreads();
    }
  } else if constexpr (SB == 2) {
    f32x4 S0[RB][JB], S1[RB][JB];
    ensure_m(false);
    wait_tiles(std::integral_constant<int, NS - 2>{});
    __syncthreads();
    affinity(S0, slot_of(0));
    next_affinity_tile();
    ensure_m(false);
    wait_tiles(std::integral_constant<int, NS - 3>{});
    __syncthreads();
    affinity(S1, slot_of(1));
    next_affinity_tile();
    softmax_fast(S0, 0);
    wait_tiles(std::integral_constant<int, NS - 4>{});
    __syncthreads();

    // ---- main loop.  Step t: DMA of tile t+NS-1, factors and weights of
    // tile t, aggregation of tile t, affinity of tile t+2 (into the registers
    // tile t's scores just left), exponentials of tile t+1 (its affinity came
    // from the step before), wait for tile t+3, one barrier.  The
    // exponentials depend on no product of the same step, so matrix-core and
    // VALU work of a step overlap freely.  Unrolled by two so the two score
    // tiles swap roles without copies.  Past the end of the list the tiles
    // are copies of a row and the scores computed for them are unused, so
    // the hot path has no data-dependent branch but the rare exact one.
    // `full` (compile-time): tiles t+1 and t+2 exist, so the step has no
    // branch but the exact one; the last two steps of a list skip the
    // affinity and exponentials of tiles past its end.
    int q0 = 0;  // ring slot of tile t
    auto step = [&](int t, f32x4 (&Sa)[RB][JB], f32x4 (&Sb)[RB][JB], auto full) {
      const int q2 = q0 + 2 < NS ? q0 + 2 : q0 + 2 - NS;
      const int qn = q0 == 0 ? NS - 1 : q0 - 1;
      issue_tile(cl, qn);
      {
        bf16x8 a[RB / 2][JB];
        float f, l;
        bool bad;
        combine_fast(f, l, bad, t & 1);
        if (bad) exact_wave(Sa, f, slot_of(q0), cc.u);
        f = row_ok(cc) ? f : 0.f;
        weights(a, Sa, f);
        aggregate(acc, a, slot_of(q0));
      }
      ensure_m(false);
      if (decltype(full)::value || t + 2 < ntot) affinity(Sa, slot_of(q2));
      next_affinity_tile();
      if (decltype(full)::value || t + 1 < ntot) softmax_fast(Sb, (t + 1) & 1);
      if (cc.row + NT >= cc.end) flush(acc, cc.u, q0);  // its first barrier ends every read of slot q0
      cursor_next(cc);
      cursor_next(cl);
      q0 = q0 + 1 < NS ? q0 + 1 : 0;
      wait_tiles(std::integral_constant<int, NS - 4>{});  // tile t+3
      __syncthreads();
    };
    using Full = std::integral_constant<bool, true>;
    using Tail = std::integral_constant<bool, false>;
    int t = 0;
    for (; t + 3 < ntot; t += 2) {
      step(t, S0, S1, Full{});
      step(t + 1, S1, S0, Full{});
    }
    // 0..3 steps remain; S0 holds tile t's scores
    if (t < ntot) step(t, S0, S1, Tail{});
    if (t + 1 < ntot) step(t + 1, S1, S0, Tail{});
    if (t + 2 < ntot) step(t + 2, S0, S1, Tail{});
  } else {
    f32x4 S[RB][JB];
    ensure_m(false);
    wait_tiles(std::integral_constant<int, NS - 2>{});
    __syncthreads();  // also publishes the folded matrix
    affinity(S, slot_of(0));
    next_affinity_tile();
    softmax_fast(S, 0);
    wait_tiles(std::integral_constant<int, NS - 3>{});
    __syncthreads();  // tile 1; row sums of tile 0

    // ---- main loop, one score buffer.  Step t: DMA of tile t+NS-1, factors
    // and weights of tile t (the scores become bf16 operands, freeing S),
    // aggregation of tile t, affinity and exponentials of tile t+1 into S,
    // wait for tile t+2, one barrier.
    int q0 = 0;
    auto step = [&](int t) {
      const int q1 = q0 + 1 < NS ? q0 + 1 : 0;
      const int qn = q0 == 0 ? NS - 1 : q0 - 1;
      issue_tile(cl, qn);
      ensure_m(true);  // matrix of tile t+1's user
      float f, l;
      bool bad;
      combine_fast(f, l, bad, t & 1);
      if (bad) exact_wave(S, f, slot_of(q0), cc.u);
      f = row_ok(cc) ? f : 0.f;
      bf16x8 a[RB / 2][JB];
      weights(a, S, f);
      aggregate(acc, a, slot_of(q0));
      affinity(S, slot_of(q1));
      next_affinity_tile();
      softmax_fast(S, (t + 1) & 1);
      if (cc.row + NT >= cc.end) flush(acc, cc.u, q0);  // its first barrier ends every read of slot q0
      cursor_next(cc);
      cursor_next(cl);
      q0 = q1;
      wait_tiles(std::integral_constant<int, NS - 3>{});  // tile t+2
      __syncthreads();
    };
    for (int t = 0; t < ntot; ++t) step(t);
  }
  wait_vm<0>();  // no DMA outlives the work group
}

template <int D, int KW, int WJ, int WI, int RB, int PF, int SB, bool PAD, bool PU, bool HS>
hipError_t launch_stream_pu(const FusedArgs& a, const Launch& l) {
  constexpr int threads = 64 * WJ * WI;
  if (l.start || l.stop) {
    hipExtLaunchKernelGGL((sa_stream_kernel<D, KW, WJ, WI, RB, PF, SB, PAD, PU, HS>), dim3(l.groups), dim3(threads), 0,
                          l.stream, l.start, l.stop, 0, a);
  } else {
    hipLaunchKernelGGL((sa_stream_kernel<D, KW, WJ, WI, RB, PF, SB, PAD, PU, HS>), dim3(l.groups), dim3(threads), 0,
                       l.stream, a);
  }
  return hipGetLastError();
}

template <int D, int KW, int WJ, int WI, int RB, int PF, int SB, bool PAD>
hipError_t launch_stream_t(const FusedArgs& a, const Launch& l) {
  if (a.lse_mode != 0) return hipErrorInvalidValue;  // the two phases run on sa_stream32.hpp
  if constexpr (WI == 1) {
    if (a.history_softmax) return launch_stream_pu<D, KW, WJ, WI, RB, PF, SB, PAD, false, true>(a, l);
  } else {
    if (a.history_softmax) return hipErrorInvalidValue;
  }
  return a.m_stride != 0 ? launch_stream_pu<D, KW, WJ, WI, RB, PF, SB, PAD, true, false>(a, l)
                         : launch_stream_pu<D, KW, WJ, WI, RB, PF, SB, PAD, false, false>(a, l);
}

template <int D, int KW, int WJ, int WI, int RB, int PF, int SB>
hipError_t run_stream_plan(const Plan& p, const FusedArgs& a, const Launch& l, int* occ) {
  constexpr int threads = 64 * WJ * WI;
  if (p.k == p.k_pad) {
    if (occ)
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, sa_stream_kernel<D, KW, WJ, WI, RB, PF, SB, false, false, false>,
                                                          threads, 0);
    return launch_stream_t<D, KW, WJ, WI, RB, PF, SB, false>(a, l);
  }
  if (occ)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, sa_stream_kernel<D, KW, WJ, WI, RB, PF, SB, true, false, false>,
                                                        threads, 0);
  return launch_stream_t<D, KW, WJ, WI, RB, PF, SB, true>(a, l);
}

#define SA_STREAM_PLAN(D_, KW_, WJ_, WI_, RB_, PF_, SB_)                                           \
  if (p.kind == 1 && p.kw == KW_ && p.waves_k == WJ_ && p.waves_rows == WI_ && p.row_blocks == RB_ && \
      p.prefetch == PF_ && p.score_buffers == SB_)                                                  \
    return run_stream_plan<D_, KW_, WJ_, WI_, RB_, PF_, SB_>(p, a, l, occ);

}  // namespace sa
