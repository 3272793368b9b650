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
//     stage tile t+2 from registers into the LDS ring, issue the HBM loads
//       of tile t+2+PF
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
// X is staged once, row-major, in a ring of three LDS tiles (tile t is read
// by the aggregation while t+1 is read by the affinity and t+2 is written).
// The aggregation needs X with the row index along each lane's reduction
// slots; gfx950's transposing LDS read (ds_read_b64_tr_b16) delivers exactly
// that from the row-major tile: within a 16-lane group, output lane o gets
// element o % 4 of the 8-byte words read by lanes o / 4 + 4e, e = 0..3.  Lane
// s of group g therefore reads row 4g + s / 4, columns 4 (s % 4) .. +3 of a
// 16-column block, and receives one column of four consecutive rows.
//
// Rows past the end of a piece are staged as zeros: their affinity is 0,
// their weights are finite and they add nothing to the sketch.  The softmax
// takes 2^s' without a shift; when the total of a row leaves [2^-100, 2^100]
// the wave holding it recomputes its rows with the max-shifted softmax on
// its own (an online max/sum pass over all prototypes, M read from global
// memory), so no other wave waits for it.
#pragma once

#include <type_traits>

#include "sa_fused.hpp"

namespace sa {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Four consecutive rows of one column, see the header comment.
__device__ __forceinline__ u32x2 lds_read_tr16(const bf16* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

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

template <int D, int KW, int WJ, int WI, int RB, int PF, int SB>
struct StreamGeom {
  static_assert(KW % 16 == 0 && D % 32 == 0 && (PF == 1 || PF == 2) && (RB == 2 || RB == 4) && (SB == 1 || SB == 2),
                "tile shape");
  static constexpr int NW = WJ * WI;
  static constexpr int THREADS = 64 * NW;
  static constexpr int RW = 16 * RB;           // rows per wave and tile
  static constexpr int NT = RW * WI;           // rows per tile
  static constexpr int JB = KW / 16;
  static constexpr int CB = D / 16;
  static constexpr int CS = D / 32;
  static constexpr int KPAD = KW * WJ;
  static constexpr int XRS = D + 16;           // row stride (elements): +32 bytes, conflict-free fragment reads
  static constexpr int XR_ELEMS = NT * XRS;
  static constexpr int NXR = SB == 2 ? 4 : 3;   // X tiles in the LDS ring
  static constexpr int CH = D / 8;             // 16-byte chunks per row
  static constexpr int NCH = NT * CH;
  static constexpr int CPT = (NCH + THREADS - 1) / THREADS;  // chunks per thread
  static constexpr int XR_BYTES = NXR * XR_ELEMS * 2;
  static constexpr int XL_BYTES = 2 * NT * WJ * 4;  // row sums of every wave, two parities
  static constexpr int STAGE_BYTES = WI > 1 ? WJ * CB * 64 * 16 : 0;
  static constexpr int OFF_XL = XR_BYTES;
  static constexpr int OFF_STAGE = OFF_XL + XL_BYTES;
  // one score buffer: the folded matrix lives in LDS, rows of D bf16 with
  // their 16-byte chunks XOR-swizzled (chunk c of row r at c ^ ((r / P) % CH),
  // P rows per 256 bytes), so fragment reads are conflict-free without padding
  static constexpr int M_BYTES = SB == 1 ? KPAD * D * 2 : 0;
  static constexpr int OFF_M = OFF_STAGE + STAGE_BYTES;
  static constexpr int LDS_BYTES = OFF_M + M_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CDNA4 compute unit");
};

template <int D, int KW, int WJ, int WI, int RB, int PF, int SB, bool PAD>
__global__ __launch_bounds__(64 * WJ * WI) void sa_stream_kernel(FusedArgs args) {
  using G = StreamGeom<D, KW, WJ, WI, RB, PF, SB>;
  using MF = Mfma<bf16>;
  constexpr int JB = G::JB, CB = G::CB, CS = G::CS, NT = G::NT, RW = G::RW, THREADS = G::THREADS;
  constexpr int XRS = G::XRS;

  __shared__ __attribute__((aligned(16))) unsigned char lds[G::LDS_BYTES];
  bf16* const Xr = reinterpret_cast<bf16*>(lds);
  float* const xl = reinterpret_cast<float*>(lds + G::OFF_XL);  // [2][NT][WJ]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wj = wave % WJ;
  const int wi = wave / WJ;
  const int rw = wi * RW;     // first tile row of this wave
  const int jbase = wj * KW;  // first prototype of this wave
  const bf16* const X = static_cast<const bf16*>(args.X);
  const bf16* const Mg = static_cast<const bf16*>(args.M);
  const int k = args.k;

  const int64_t rows = args.rows;
  const int64_t ngroups = gridDim.x;
  const int64_t grp = blockIdx.x;
  const int64_t r_begin = grp * rows / ngroups;
  const int64_t r_end = (grp + 1) * rows / ngroups;
  if (r_begin >= r_end) return;

  int u_first = 0, ntot = 0;
  // A cursor walks the tile list: first row of the tile, end of its piece, user.
  struct Cursor {
    int64_t row, end;
    int u;
  };
  auto cursor_begin = [&]() { return Cursor{r_begin, min(r_end, args.offsets[u_first + 1]), u_first}; };
  auto cursor_next = [&](Cursor& c) {
    c.row += NT;
    if (c.row >= c.end) {
      c.row = c.end;
      if (c.row < r_end) {
        ++c.u;
        while (c.u < args.users && args.offsets[c.u + 1] <= c.row) ++c.u;
        c.end = min(r_end, args.offsets[c.u + 1]);
      }
    }
  };

  // ---- folded matrix: this wave's KW rows as B fragments, in registers
  // (two score buffers) or in the swizzled LDS copy (one score buffer)
  constexpr int MP = 256 / (2 * D);  // rows of M per 256 bytes
  bf16x8 mreg[SB == 2 ? JB : 1][SB == 2 ? CS : 1];
  bf16* const Ms = reinterpret_cast<bf16*>(lds + G::OFF_M);
  int moff[CS];  // element offset of chunk 4 cs + g of this lane's rows (the swizzle depends on l16 only)
  if constexpr (SB == 2) {
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      const bf16* mrow = Mg + (int64_t)(jbase + 16 * jb + l16) * D;
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) mreg[jb][cs] = frag_c<D>(mrow, cs, g);
    }
  } else {
    for (int idx = tid; idx < G::KPAD * G::CH; idx += THREADS) {
      const int r = idx / G::CH, c = idx % G::CH;
      *reinterpret_cast<u32x4*>(Ms + r * D + 8 * (c ^ ((r / MP) % G::CH))) =
          *reinterpret_cast<const u32x4*>(Mg + (int64_t)r * D + 8 * c);
    }
    // ordered before the first read by the prologue's barrier
  }
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) moff[cs] = 8 * ((4 * cs + g) ^ ((l16 / MP) % G::CH));

  // ---- staging: thread chunk s covers row (tid + s*THREADS) / CH, 16 bytes.
  // A tile's loads read rows clamped to its piece (always in bounds, offsets
  // 32-bit from the tile's first row); rows past the piece are replaced by
  // zeros when the tile is staged, which only a piece's last tile needs.
  u32x4 pre[PF][G::CPT];
  int pre_rows[PF];  // valid rows of the tile held in each register slot (0 past the list)
  auto load_tile = [&](u32x4 (&dst)[G::CPT], int& dst_rows, const Cursor& c, bool valid) {
    const int64_t left = c.end - c.row;
    dst_rows = !valid ? 0 : (left < NT ? (int)left : NT);
    const int last = (int)(c.end - 1 - c.row);  // -1 past the list: c.row + last = c.end - 1 >= 0
    const u32x4* tile = reinterpret_cast<const u32x4*>(X + c.row * D);
#pragma unroll
    for (int s = 0; s < G::CPT; ++s) {
      const int ci = tid + s * THREADS;
      const int r = ci / G::CH, ch = ci % G::CH;
      if (G::NCH % THREADS == 0 || ci < G::NCH) {
        const int rr = r < last ? r : last;
        dst[s] = __builtin_nontemporal_load(tile + (rr * G::CH + ch));
      }
    }
  };
  auto store_tile = [&](const u32x4 (&src)[G::CPT], int rows_valid, bf16* xr) {
    if (rows_valid == NT) {  // uniform: every tile but a piece's last
#pragma unroll
      for (int s = 0; s < G::CPT; ++s) {
        const int ci = tid + s * THREADS;
        const int r = ci / G::CH, ch = ci % G::CH;
        if (G::NCH % THREADS == 0 || ci < G::NCH) *reinterpret_cast<u32x4*>(xr + r * XRS + 8 * ch) = src[s];
      }
    } else {
#pragma unroll
      for (int s = 0; s < G::CPT; ++s) {
        const int ci = tid + s * THREADS;
        const int r = ci / G::CH, ch = ci % G::CH;
        if (G::NCH % THREADS == 0 || ci < G::NCH)
          *reinterpret_cast<u32x4*>(xr + r * XRS + 8 * ch) = r < rows_valid ? src[s] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  // tile 0 starts at r_begin whatever the users: its loads go out before the
  // tile list is known (rows clamped to the group's range, masked at staging)
  u32x4 tile0[G::CPT];
  {
    int unused_rows;
    load_tile(tile0, unused_rows, Cursor{r_begin, r_end, 0}, true);
  }

  // ---- the group's tile list: pieces (user segments) of [r_begin, r_end),
  // each cut into tiles of NT rows.  Every lane examines up to four users at
  // once (no chain of dependent loads): u_first is the last user starting at
  // or before r_begin (a prefix, offsets being non-decreasing; it is
  // non-empty because offsets[u_first + 1] > r_begin), ntot the sum of the
  // pieces' tile counts.
  {
    int cnt = 0, tiles = 0;
    const int nq = (args.users + 63) / 64;
    for (int q = 0; q < nq; ++q) {
      const int uu = lane + 64 * q;
      if (uu < args.users) {
        const int64_t a = args.offsets[uu], b = args.offsets[uu + 1];
        cnt += a <= r_begin ? 1 : 0;
        const int64_t lo = a > r_begin ? a : r_begin, hi = b < r_end ? b : r_end;
        if (hi > lo) tiles += (int)((hi - lo + NT - 1) / NT);
      }
    }
    cnt = row16_sum_i(cnt);
    tiles = row16_sum_i(tiles);
    u_first = __builtin_amdgcn_readlane(cnt, 0) + __builtin_amdgcn_readlane(cnt, 16) +
              __builtin_amdgcn_readlane(cnt, 32) + __builtin_amdgcn_readlane(cnt, 48) - 1;
    ntot = __builtin_amdgcn_readlane(tiles, 0) + __builtin_amdgcn_readlane(tiles, 16) +
           __builtin_amdgcn_readlane(tiles, 32) + __builtin_amdgcn_readlane(tiles, 48);
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
  auto affinity = [&](f32x4 (&s)[RB][JB], const bf16* xr) {
#pragma unroll
    for (int ib = 0; ib < RB; ++ib)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) s[ib][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
      bf16x8 xa[RB];
#pragma unroll
      for (int ib = 0; ib < RB; ++ib) xa[ib] = frag_c<D>(xr + (rw + 16 * ib + l16) * XRS, cs, g);
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
          s[ib][jb] = MF::run(xa[ib], mf, s[ib][jb]);
        }
    }
    pad_protos(s, jbase);
  };

  // ---- e = 2^s' in place; this wave's row sums to xl[par].  After the
  // transposing butterfly the four lanes of a quad hold the same total and
  // store it to the same word (no branch).
  auto softmax_fast = [&](f32x4 (&s)[RB][JB], int par) {
    float* const xlp = xl + par * (NT * WJ);
#pragma unroll
    for (int ib = 0; ib < RB; ++ib) {
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
      xlp[trow * WJ + wj] = z;
    }
  };

  // ---- factors 1 / sum_w l_w.  Lane (g, l16) finishes row
  // rw + 16 ib + 4 g + r with ib = (l16 / 4) % RB, r = l16 % 4, so each row
  // of the wave lives in the 16-lane DPP row g of the lanes that need it; the
  // aggregation takes the factors of its rows by row broadcasts (fac_of).
  // `bad` is set when a row total left the range of the unshifted softmax.
  const int my_ib = (l16 >> 2) % RB, my_r = l16 & 3;
  auto combine_fast = [&](float& f, bool& bad, int par) {
    const float* p = xl + par * (NT * WJ) + (rw + 16 * my_ib + 4 * g + my_r) * WJ;
    float l;
    if constexpr (WJ % 4 == 0) {
      f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
      for (int w = 4; w < WJ; w += 4) v += *reinterpret_cast<const f32x4*>(p + w);
      l = (v[0] + v[1]) + (v[2] + v[3]);
    } else {
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
  auto exact_wave = [&](f32x4 (&s)[RB][JB], float& f, const bf16* xr) {
#pragma unroll  // s[ib] must be indexed by constants to stay in registers
    for (int ib = 0; ib < RB; ++ib) {
      bf16x8 xa[CS];
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) xa[cs] = frag_c<D>(xr + (rw + 16 * ib + l16) * XRS, cs, g);
      float m[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      float l[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
      for (int w = 0; w < WJ; ++w) {
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {  // one 16-prototype block at a time (few live registers)
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
          const int j0 = w * KW + 16 * jb;
          const bf16* mrow = Mg + (int64_t)(j0 + l16) * D;
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
  // 4 g + e % 4, the rows the affinity layout left in that lane.
  const int tr_off = (rw + 4 * g + (l16 >> 2)) * XRS + 4 * (l16 & 3);
  auto weights = [&](bf16x8 (&a)[RB / 2][JB], const f32x4 (&s)[RB][JB], float f) {
#pragma unroll
    for (int h = 0; h < RB / 2; ++h) {
      float fac[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) fac[e] = fac_of(f, 2 * h + (e >> 2), e & 3);
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int e = 0; e < 8; ++e) a[h][jb][e] = (bf16)(s[2 * h + (e >> 2)][jb][e & 3] * fac[e]);
    }
  };
  auto aggregate = [&](f32x4 (&acc)[JB][CB], const bf16x8 (&a)[RB / 2][JB], const bf16* xr) {
#pragma unroll
    for (int h = 0; h < RB / 2; ++h) {
      const bf16* const xp = xr + tr_off + 32 * h * XRS;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const u32x2 lo = lds_read_tr16(xp + 16 * cb);
        const u32x2 hi = lds_read_tr16(xp + 16 * XRS + 16 * cb);
        const bf16x8 xb = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) acc[jb][cb] = MF::run(a[h][jb], xb, acc[jb][cb]);
      }
    }
  };

  // ---- flush one (group, user) piece: waves that split the rows add their
  // accumulators through LDS in a fixed order, then one wave per prototype
  // slice writes the slot in the lane layout [wj][jb][cb][lane][4].
  auto flush = [&](f32x4 (&acc)[JB][CB], int u) {
    if constexpr (WI > 1) {
      float* stage = reinterpret_cast<float*>(lds + G::OFF_STAGE);
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
      float* dst = args.partial + (grp + u) * (int64_t)(G::KPAD * D);
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
  constexpr int NPRE = SB == 2 ? 3 : 2;  // tiles staged by the prologue

  // ---- prologue: tiles 0 .. NPRE-1 into the ring, the next PF into
  // registers (every HBM load issued before the first one is used).  Tile 0
  // is staged alone first, so its affinity runs while the other tiles arrive.
  u32x4 tmp[NPRE - 1][G::CPT];
  int tmp_rows[NPRE];
  tmp_rows[0] = ntot > 0 ? (int)min((int64_t)NT, cl.end - cl.row) : 0;
  cursor_next(cl);
#pragma unroll
  for (int p = 1; p < NPRE; ++p) {
    load_tile(tmp[p - 1], tmp_rows[p], cl, p < ntot);
    cursor_next(cl);
  }
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    load_tile(pre[(NPRE + p) % PF], pre_rows[(NPRE + p) % PF], cl, NPRE + p < ntot);
    cursor_next(cl);
  }
  store_tile(tile0, tmp_rows[0], Xr);
  __syncthreads();
  auto stage_rest = [&]() {
#pragma unroll
    for (int p = 1; p < NPRE; ++p) store_tile(tmp[p - 1], tmp_rows[p], Xr + p * G::XR_ELEMS);
    __syncthreads();
  };

  if constexpr (SB == 2) {
    f32x4 S0[RB][JB], S1[RB][JB];
    affinity(S0, Xr);
    stage_rest();
    affinity(S1, Xr + G::XR_ELEMS);
    softmax_fast(S0, 0);
    __syncthreads();

    // ---- main loop.  Step t: stage tile t+3, factors and weights of tile
    // t, aggregation of tile t, affinity of tile t+2 (into the registers
    // tile t's scores just left), exponentials of tile t+1 (its affinity came
    // from the step before), one barrier.  The exponentials depend on no
    // product of the same step, so matrix-core and VALU work of a step
    // overlap freely.  Unrolled by two so the two score tiles swap roles
    // without copies.  Ring slot of tile t: t % 4.  Past the end of the list
    // the staged tiles are zeros and the scores computed for them are unused,
    // so the hot path has no data-dependent branch but the rare exact one.
    // `full` (compile-time): tiles t+1 and t+2 exist, so the step has no
    // branch but the exact one; the last two steps of a list skip the
    // affinity and exponentials of tiles past its end.
    auto step = [&](int t, f32x4 (&Sa)[RB][JB], f32x4 (&Sb)[RB][JB], u32x4 (&pslot)[G::CPT], int& prow,
                    auto full) {
      bf16* const xr_t = Xr + (t & 3) * G::XR_ELEMS;
      bf16* const xr_t2 = Xr + ((t + 2) & 3) * G::XR_ELEMS;
      bf16* const xr_t3 = Xr + ((t + 3) & 3) * G::XR_ELEMS;
      store_tile(pslot, prow, xr_t3);
      load_tile(pslot, prow, cl, t + 3 + PF < ntot);
      float f;
      bool bad;
      combine_fast(f, bad, t & 1);
      if (bad) exact_wave(Sa, f, xr_t);
      bf16x8 a[RB / 2][JB];
      weights(a, Sa, f);
      aggregate(acc, a, xr_t);
      if (decltype(full)::value || t + 2 < ntot) affinity(Sa, xr_t2);
      if (decltype(full)::value || t + 1 < ntot) softmax_fast(Sb, (t + 1) & 1);
      if (cc.row + NT >= cc.end) flush(acc, cc.u);
      cursor_next(cc);
      cursor_next(cl);
      __syncthreads();
    };
    using Full = std::integral_constant<bool, true>;
    using Tail = std::integral_constant<bool, false>;
    int t = 0;
    for (; t + 3 < ntot; t += 2) {
      step(t, S0, S1, pre[3 % PF], pre_rows[3 % PF], Full{});
      step(t + 1, S1, S0, pre[0], pre_rows[0], Full{});
    }
    // 0..3 steps remain; S0 holds tile t's scores
    if (t < ntot) step(t, S0, S1, pre[3 % PF], pre_rows[3 % PF], Tail{});
    if (t + 1 < ntot) step(t + 1, S1, S0, pre[0], pre_rows[0], Tail{});
    if (t + 2 < ntot) step(t + 2, S0, S1, pre[3 % PF], pre_rows[3 % PF], Tail{});
  } else {
    f32x4 S[RB][JB];
    affinity(S, Xr);
    softmax_fast(S, 0);
    stage_rest();  // its barrier also publishes the row sums of tile 0

    // ---- main loop, one score buffer.  Step t: stage tile t+2, factors and
    // weights of tile t (the scores become bf16 operands, freeing S),
    // aggregation of tile t, affinity and exponentials of tile t+1 into S,
    // one barrier.  Ring slot of tile t: t % 3.
    int q0 = 0;
    auto step = [&](int t, u32x4 (&pslot)[G::CPT], int& prow) {
      const int q1 = q0 == 2 ? 0 : q0 + 1;
      const int q2 = q1 == 2 ? 0 : q1 + 1;
      bf16* const xr_t = Xr + q0 * G::XR_ELEMS;
      bf16* const xr_t1 = Xr + q1 * G::XR_ELEMS;
      bf16* const xr_t2 = Xr + q2 * G::XR_ELEMS;
      store_tile(pslot, prow, xr_t2);
      load_tile(pslot, prow, cl, t + 2 + PF < ntot);
      float f;
      bool bad;
      combine_fast(f, bad, t & 1);
      if (bad) exact_wave(S, f, xr_t);
      bf16x8 a[RB / 2][JB];
      weights(a, S, f);
      aggregate(acc, a, xr_t);
      affinity(S, xr_t1);
      softmax_fast(S, (t + 1) & 1);
      if (cc.row + NT >= cc.end) flush(acc, cc.u);
      cursor_next(cc);
      cursor_next(cl);
      q0 = q1;
      __syncthreads();
    };
    for (int t = 0; t < ntot; t += 2) {
      step(t, pre[2 % PF], pre_rows[2 % PF]);
      if (t + 1 < ntot) step(t + 1, pre[3 % PF], pre_rows[3 % PF]);
    }
  }
}

template <int D, int KW, int WJ, int WI, int RB, int PF, int SB, bool PAD>
hipError_t launch_stream_t(const FusedArgs& a, const Launch& l) {
  constexpr int threads = 64 * WJ * WI;
  if (l.start || l.stop) {
    hipExtLaunchKernelGGL((sa_stream_kernel<D, KW, WJ, WI, RB, PF, SB, PAD>), dim3(l.groups), dim3(threads), 0,
                          l.stream, l.start, l.stop, 0, a);
  } else {
    hipLaunchKernelGGL((sa_stream_kernel<D, KW, WJ, WI, RB, PF, SB, PAD>), dim3(l.groups), dim3(threads), 0, l.stream,
                       a);
  }
  return hipGetLastError();
}

template <int D, int KW, int WJ, int WI, int RB, int PF, int SB>
hipError_t run_stream_plan(const Plan& p, const FusedArgs& a, const Launch& l, int* occ) {
  constexpr int threads = 64 * WJ * WI;
  if (p.k == p.k_pad) {
    if (occ)
      return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, sa_stream_kernel<D, KW, WJ, WI, RB, PF, SB, false>,
                                                          threads, 0);
    return launch_stream_t<D, KW, WJ, WI, RB, PF, SB, false>(a, l);
  }
  if (occ)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, sa_stream_kernel<D, KW, WJ, WI, RB, PF, SB, true>,
                                                        threads, 0);
  return launch_stream_t<D, KW, WJ, WI, RB, PF, SB, true>(a, l);
}

#define SA_STREAM_PLAN(D_, KW_, WJ_, WI_, RB_, PF_, SB_)                                           \
  if (p.kind == 1 && p.kw == KW_ && p.waves_k == WJ_ && p.waves_rows == WI_ && p.row_blocks == RB_ && \
      p.prefetch == PF_ && p.score_buffers == SB_)                                                  \
    return run_stream_plan<D_, KW_, WJ_, WI_, RB_, PF_, SB_>(p, a, l, occ);

}  // namespace sa
