// Streamed fused pass on 32x32x16 matrix-core products with the prototypes
// along the lanes (bf16, d = 128, eight waves of 32 prototypes), gfx950.
//
// The operation is that of sa_stream.hpp (SequenceO1 close-reading page,
// section 2.1: s'_ji = M_j . x_i with the folded M, a_ji = 2^s'_ji / sum_j'
// 2^s'_j'i, X~_j += a_ji x_i; section 2.4: one fused, tiled pass that never
// writes the k x n matrices to memory and accepts ragged batches), with the
// work split, tile list, LDS-DMA ring, X swizzle (chunk_sw32) and partial
// slots of sa_stream32.hpp.  What differs from that pass is the orientation
// of the affinity product:
//
//   affinity    S (32 i x 32 j) = X (32 i x 16 d) . M^T (16 d x 32 j), eight
//               products over d per block of 32 rows.  A lane holds one
//               prototype j (lane % 32) and, in registers, 16 rows of each
//               of the tile's two row blocks: register v of block f is row
//               32 f + 8 (v / 4) + 4 h + v % 4 (h the half-wave).
//   aggregation X~ (32 j x 32 c) += A (32 j x 16 i) . X (16 i x 32 c): the A
//               operand wants one prototype per lane and eight rows per lane
//               in the reduction slots (g, e) -> row 16 q + 8 (e / 4) + 4 g
//               + e % 4, which is where the affinity left them, so the
//               weights go from the scores to the products without leaving
//               the registers (no LDS round trip, no wait on one).
//
// The cost moves to the row sums over the prototypes, which now run across
// the 32 lanes of a half-wave.  A reduce-scatter halves the values a lane
// holds at each lane bit: bits 3 and 2 by DPP adds confined to the lanes of
// two DPP banks (two instructions per result, each half of the lanes keeping
// its own half of the values, no selects), bit 4 by v_permlane16_swap (one
// swap and one add per result), bits 1 and 0 by quad DPP adds with selects.
// Each lane ends with the partial sum of one row of the tile; the partials of
// all waves meet in LDS as in the other passes.  Each lane then finishes two
// rows, chosen so that every 16-lane DPP row holds the 32 factors of its
// half-wave, and the weights take their factors by DPP row broadcasts folded
// into the multiplies.
//
// Each step (one barrier): DMA of tile t+3; the row sums of tile t from LDS;
// the affinity of tile t+1, and in the shadow of its products the factors and
// weights of tile t; the aggregation of tile t, and in the shadow of its
// products the exponentials and row sums of tile t+1.  A row whose total
// leaves [2^-100, 2^100] sends its wave through an exact pass (a running
// maximum over all prototypes, M from global memory).  One pass only: the
// two phases of the pass for more prototypes run on sa_stream32.hpp.
//
// HS: the comparator (the page's section 3.1 baseline), softmax over the
// user's rows per prototype.  This layout suits it: a prototype's 64 scores
// of a tile sit in one lane and its half-wave partner, so the tile maximum
// and the sum over rows are in-lane work plus one half-wave exchange, with no
// exchange between waves.  Per piece each prototype keeps a running maximum m
// (raised only when a tile exceeds it by more than 8 in log2 units, so every
// weight stays below 2^8), the sum l of 2^(s' - m) and the accumulator in the
// scale of m; the weights 2^(s' - m) go to the products as they are.  The
// piece's partial is (acc, m, l), merged by reduce_history_kernel.
#pragma once

#include "sa_stream32.hpp"

namespace sa {

// o[i] = x[i] + x[i] of lane ^ 8 on the lanes whose bit 3 is clear, y[i] +
// y[i] of lane ^ 8 on the others (row_ror:8 within a 16-lane row; bank_mask
// 0x3 writes lanes 0..7 of each row, 0xC lanes 8..15).  The nop covers the
// wait states a DPP read needs after a vector write of its operand.
__device__ __forceinline__ void fold_bit3(float (&o)[4], const float (&x)[4], const float (&y)[4]) {
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %4, %4 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %8, %8 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %1, %5, %5 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %1, %9, %9 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %2, %6, %6 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %2, %10, %10 row_ror:8 row_mask:0xf bank_mask:0xc\n\t"
      "v_add_f32_dpp %3, %7, %7 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %3, %11, %11 row_ror:8 row_mask:0xf bank_mask:0xc"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3]));
}
// the same for lane bit 2: lanes with bit 2 clear (banks 0 and 2, mask 0x5)
// add x of lane + 4 (row_shl:4), the others (mask 0xA) y of lane - 4 (row_shr:4)
__device__ __forceinline__ void fold_bit2(float (&o)[4], const float (&x)[4], const float (&y)[4]) {
  asm("s_nop 1\n\t"
      "v_add_f32_dpp %0, %4, %4 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %0, %8, %8 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %1, %5, %5 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %1, %9, %9 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %2, %6, %6 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %2, %10, %10 row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
      "v_add_f32_dpp %3, %7, %7 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %3, %11, %11 row_shr:4 row_mask:0xf bank_mask:0xa"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3]));
}
// x + y after v_permlane16_swap(x, y): on the lanes of even 16-lane rows the
// sum of x over the row and the next one, on odd rows the sum of y over the
// row and the one before
__device__ __forceinline__ float fold_bit4(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                  false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// value of x in lane n of this lane's 16-lane row (n a constant after unrolling)
__device__ __forceinline__ float bcast16(float x, int n) {
  switch (n) {
    case 0: return row_bcast<0>(x);
    case 1: return row_bcast<1>(x);
    case 2: return row_bcast<2>(x);
    case 3: return row_bcast<3>(x);
    case 4: return row_bcast<4>(x);
    case 5: return row_bcast<5>(x);
    case 6: return row_bcast<6>(x);
    case 7: return row_bcast<7>(x);
    case 8: return row_bcast<8>(x);
    case 9: return row_bcast<9>(x);
    case 10: return row_bcast<10>(x);
    case 11: return row_bcast<11>(x);
    case 12: return row_bcast<12>(x);
    case 13: return row_bcast<13>(x);
    case 14: return row_bcast<14>(x);
    default: return row_bcast<15>(x);
  }
}

template <bool PAD, bool PU, bool HS = false>
__global__ __launch_bounds__(512) void sa_wide_kernel(FusedArgs args) {
  static_assert(!(HS && PU), "the comparator shares one folded matrix");
  constexpr int D = 128, KW = 32, WJ = 8, NW = 8, NT = 64, KC = D / 16, CBK = D / 32, NS = 4;
  constexpr int CH = D / 8;                       // 16-byte chunks per row
  constexpr int SLOT_BYTES = NT * D * 2;          // one X tile
  constexpr int NI = SLOT_BYTES / 1024;           // 1 KB DMA blocks per tile
  constexpr int NIW = NI / NW;                    // per wave
  constexpr int RPI = 1024 / (2 * D);             // rows per DMA block
  constexpr int KPAD = KW * WJ;
  constexpr int kFactorsAt = 2;                   // affinity product after which tile t's factors are formed
  // row partial sums [2 parities][WJ / 4][NTP][4 waves]: row R at R + 8 (R / 32), so the
  // combine's 16-byte reads (rows r, r + 16, r + 32, r + 48 for r in a group of four) reach distinct banks
  constexpr int NTP = NT + 16;
  constexpr int OFF_XL = NS * SLOT_BYTES;
  constexpr int XL_BYTES = 2 * (WJ / 4) * NTP * 16;
  constexpr int LDS_BYTES = OFF_XL + XL_BYTES;
  constexpr int DMA_PER_TILE = NIW;
  static_assert(NI % NW == 0 && LDS_BYTES <= 160 * 1024, "tile geometry");

  __shared__ __attribute__((aligned(1024))) unsigned char lds[LDS_BYTES];
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) unsigned char*)lds;
  auto slot_of = [&](int q) { return lds0 + (uint32_t)(q * SLOT_BYTES); };
  float* const xl = reinterpret_cast<float*>(lds + OFF_XL);
  auto xl_at = [&](int par, int row, int w) { return ((par * (WJ / 4) + w / 4) * NTP + row + 8 * (row >> 5)) * 4 + (w & 3); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;  // half-wave
  const int g16 = lane >> 4;
  const int s16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wj = wave;
  const int jbase = wj * KW;
  // row whose partial sum this lane ends with after the reduce-scatter (lane bits b5..b0:
  // 32 b3 + 16 b2 + 8 b4 + 4 b5 + 2 b1 + b0), and the two rows whose factors it finishes
  // (the same with b4 = 0 and 1: both DPP rows of a half-wave hold all 32 of its factors)
  const int row_a = 32 * ((lane >> 3) & 1) + 16 * ((lane >> 2) & 1) + 4 * h + (lane & 3);
  const int my_row = row_a + 8 * ((lane >> 4) & 1);

  const bf16* const X = static_cast<const bf16*>(args.X);
  const bf16* const Mg = static_cast<const bf16*>(args.M);
  const int k = args.k;

  const int64_t rows = args.rows;
  const int64_t ngroups = gridDim.x;
  const int64_t grp = blockIdx.x;
  const int64_t r_begin = grp * rows / ngroups;
  const int64_t r_end = (grp + 1) * rows / ngroups;
  if (r_begin >= r_end) return;
  const OffsetLoads offs = tile_list_loads(args, lane);  // first: see tile_list

  // ---- tile list: pieces (user segments) of [r_begin, r_end) cut into tiles
  // of NT rows.  Cursor rows are relative to r_begin (a group's range fits in
  // 32 bits), so the per-step bookkeeping stays in 32-bit scalar arithmetic.
  const int nrel = (int)(r_end - r_begin);
  struct Cursor {
    int row, end, u;
  };
  int u_first = 0, ntot = 0;
  auto user_end = [&](int u) {
    const int64_t e = args.offsets[u + 1] - r_begin;
    return e < (int64_t)nrel ? (int)e : nrel;
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

  // ---- folded matrix: lane l holds M[jbase + l % 32][16 kc + 8 h .. + 7] (B operand of the affinity)
  bf16x8 mreg[KC];
  auto load_m = [&](int u) {
    const bf16* const Mu = PU ? Mg + (int64_t)u * args.m_stride : Mg;
    const bf16* const mrow = Mu + (int64_t)(jbase + l32) * D + 8 * h;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) mreg[kc] = *reinterpret_cast<const bf16x8*>(mrow + 16 * kc);
  };
  int m_user = -1;
  if constexpr (!PU) {
    load_m(0);
    m_user = 0;
  }

  // ---- LDS DMA of a tile: block j = wave + s NW lands at slot + 1024 j; lane i
  // holds row j RPI + i / CH, LDS chunk i % CH = global chunk (i % CH) ^ sw(row).
  // Rows past the piece read its last row, so every load stays in bounds.
  int dma_row[NIW], dma_col[NIW];
#pragma unroll
  for (int s = 0; s < NIW; ++s) {
    const int j = wave + s * NW;
    dma_row[s] = j * RPI + lane / CH;
    dma_col[s] = 8 * ((lane % CH) ^ chunk_sw32(dma_row[s]));
  }
  auto issue_tile = [&](const Cursor& c, int q) {
    const int last = c.end - 1 - c.row;  // -1 past the list
    const int64_t b0 = r_begin + (last < 0 ? c.end - 1 : c.row);
    const int lim = last < 0 ? 0 : (last < NT ? last : NT - 1);
    const bf16* const base = X + b0 * D;
    const uint32_t slot = slot_of(q);
#pragma unroll
    for (int s = 0; s < NIW; ++s) {
      const int j = wave + s * NW;
      const int rr = dma_row[s] < lim ? dma_row[s] : lim;
      dma16(base, (uint32_t)(rr * D + dma_col[s]) * 2u, slot + 1024u * (uint32_t)j);
    }
  };
  auto wait_tiles = [&](auto n_) {
    constexpr int n = decltype(n_)::value;
    wait_vm<DMA_PER_TILE * n>();
  };

  issue_tile(Cursor{0, nrel, 0}, 0);
  int64_t first_end;  // end of the piece holding r_begin
  {
    const TileList tl = tile_list(args, offs, r_begin, r_end, NT, lane);
    u_first = tl.u_first;
    ntot = tl.ntot;
    first_end = tl.first_end;
  }

  // ---- affinity: s[f][v] = S'[jbase + l32][row 32 f + 8 (v / 4) + 4 h + v % 4 of the tile]
  uint32_t aoff[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) aoff[kc] = (uint32_t)(2 * (l32 * D + 8 * ((2 * kc + h) ^ chunk_sw32(l32))));
  // fragments are read one d-chunk ahead of their products
  auto affinity = [&](f32x16 (&s)[2], uint32_t xs, auto hook) {
    bf16x8 x[2][2];
    x[0][0] = lds_b128(aoff[0] + xs);
    x[0][1] = lds_b128(aoff[0] + xs + (uint32_t)(2 * 32 * D));
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if (kc + 1 < KC) {
        x[(kc + 1) & 1][0] = lds_b128(aoff[kc + 1] + xs);
        x[(kc + 1) & 1][1] = lds_b128(aoff[kc + 1] + xs + (uint32_t)(2 * 32 * D));
      }
      const f32x16 z = {};
      s[0] = mfma32(x[kc & 1][0], mreg[kc], kc == 0 ? z : s[0]);
      s[1] = mfma32(x[kc & 1][1], mreg[kc], kc == 0 ? z : s[1]);
      hook(kc);  // independent vector work issued in the products' shadow
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (PAD) {
      if (jbase + l32 >= k) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          s[0][v] = -INFINITY;
          s[1][v] = -INFINITY;
        }
      }
    }
  };
  auto no_hook = [](int) {};

  // ---- exponentials and row sums, in four pieces (issued between the
  // aggregation's products).  Piece 2 sl (sl = 0, 1): 2^s' of the registers
  // v = 4 sl + p and 8 + 4 sl + p of both row blocks; piece 2 sl + 1: their
  // sums over lane bits 3 and 2 (rows of q = 2 b2 + sl, p = 0..3 left per
  // lane); after piece 3, bit 4 joins the two slices (q = 2 b2 + b4) and bits
  // 1, 0 pick p, and the lane's partial of row my_row goes to LDS.
  float part[2][4];
  auto softmax_piece = [&](f32x16 (&s)[2], int i, int par) {
    const int sl = i >> 1;
    if ((i & 1) == 0) {
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          s[f][4 * sl + p] = fast_exp2(s[f][4 * sl + p]);
          s[f][8 + 4 * sl + p] = fast_exp2(s[f][8 + 4 * sl + p]);
        }
    } else {
      float x0[4], x1[4], y0[4], y1[4], o0[4], o1[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        x0[p] = s[0][4 * sl + p];
        y0[p] = s[1][4 * sl + p];
        x1[p] = s[0][8 + 4 * sl + p];
        y1[p] = s[1][8 + 4 * sl + p];
      }
      fold_bit3(o0, x0, y0);  // q = sl: rows of block b3
      fold_bit3(o1, x1, y1);  // q = 2 + sl
      fold_bit2(part[sl], o0, o1);
      if (i == 3) {
        float r3[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) r3[p] = fold_bit4(part[0][p], part[1][p]);
        const bool c1 = (lane & 2) != 0, c0 = (lane & 1) != 0;
        float r4[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float keep = c1 ? r3[2 + e] : r3[e], send = c1 ? r3[e] : r3[2 + e];
          r4[e] = keep + dpp_f32<0x4E>(send);  // quad_perm [2,3,0,1]: lane ^ 2
        }
        const float keep = c0 ? r4[1] : r4[0], send = c0 ? r4[0] : r4[1];
        xl[xl_at(par, my_row, wj)] = keep + dpp_f32<0xB1>(send);  // quad_perm [1,0,3,2]: lane ^ 1
      }
    }
  };
  auto softmax_all = [&](f32x16 (&s)[2], int par) {
#pragma unroll
    for (int i = 0; i < 4; ++i) softmax_piece(s, i, par);
  };

  // ---- factors 1 / sum_w l_w of rows row_a and row_a + 8 (reads issued
  // first, summed later); `bad` when a total left the range of the
  // unshifted softmax
  auto combine_issue = [&](f32x4 (&v)[2][WJ / 4], int par) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int w = 0; w < WJ; w += 4) v[r][w / 4] = *reinterpret_cast<const f32x4*>(xl + xl_at(par, row_a + 8 * r, w));
  };
  auto combine_finish = [&](const f32x4 (&v)[2][WJ / 4], float (&fr)[2], float (&lr)[2], bool& bad) {
    bool out = false;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      f32x4 a = v[r][0];
#pragma unroll
      for (int w = 1; w < WJ / 4; ++w) a += v[r][w];
      lr[r] = (a[0] + a[1]) + (a[2] + a[3]);
      out |= !(lr[r] >= 0x1p-100f && lr[r] <= 0x1p100f);
      fr[r] = __builtin_amdgcn_rcpf(lr[r]);
    }
    bad = __builtin_amdgcn_ballot_w64(out) != 0;
  };

  // ---- exact pass of one wave (rare).  The running maximum and shifted sum
  // of every row over all prototypes of the block are taken in the
  // orientation of sa_stream32.hpp (M as the A operand from global memory,
  // one row per lane, so a row's reduction is in-lane plus one half-wave
  // swap); then the wave's own scores, recomputed in this pass's
  // orientation, become 2^(s' - lse) of their rows (lse by lane shuffles),
  // with factors 1.
  auto exact_wave = [&](f32x16 (&s)[2], float (&fr)[2], uint32_t xs, int u) {
    const bf16* const Mu = PU ? Mg + (int64_t)u * args.m_stride : Mg;
    float lse[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      float m = -INFINITY, ls = 0.f;
#pragma unroll 1
      for (int w = 0; w < WJ; ++w) {
        const bf16* const mrow = Mu + (int64_t)(w * KW + l32) * D + 8 * h;
        f32x16 a = {};
#pragma unroll 1
        for (int kc = 0; kc < KC; ++kc)
          a = mfma32(*reinterpret_cast<const bf16x8*>(mrow + 16 * kc), lds_b128(xs + (uint32_t)(2 * 32 * f * D) + aoff[kc]),
                     a);
        if constexpr (PAD) {
#pragma unroll
          for (int v = 0; v < 16; ++v) a[v] = w * KW + 8 * (v >> 2) + 4 * h + (v & 3) < k ? a[v] : -INFINITY;
        }
        float bm = a[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) bm = fmaxf(bm, a[v]);
        const float mn = fmaxf(m, pair32_max(bm));
        if (mn != -INFINITY) {  // a block of padding only leaves the state as it is
          float t = 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) t += fast_exp2(a[v] - mn);
          ls = ls * fast_exp2(m - mn) + pair32_sum(t);
          m = mn;
        }
      }
      lse[f] = m + __log2f(ls);  // row 32 f + l32 (both half-waves)
    }
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      f32x16 a = {};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) a = mfma32(lds_b128(xs + (uint32_t)(2 * 32 * f * D) + aoff[kc]), mreg[kc], a);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float L = __shfl(lse[f], 8 * (v >> 2) + 4 * h + (v & 3));
        s[f][v] = (PAD && jbase + l32 >= k) ? 0.f : fast_exp2(a[v] - L);
      }
    }
    fr[0] = 1.f;
    fr[1] = 1.f;
  };

  // ---- weights of row step rs (rows 16 rs + 8 (e / 4) + 4 h + e % 4, register
  // 8 (rs % 2) + e of block rs / 2): the factor of that row sits in lane
  // 8 (rs / 2) + 4 (rs % 2) + e % 4 of the DPP row, register fr[e / 4]
  auto weights_rs = [&](bf16x8 (&a)[4], const f32x16 (&s)[2], const float (&fr)[2], int rs) {
    const int f = rs >> 1, o = 8 * (rs & 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[rs][e] = (bf16)(s[f][o + e] * bcast16(fr[e >> 2], 8 * f + 4 * (rs & 1) + (e & 3)));
  };

  // ---- aggregation of tile t: acc[cb][v] += sum over the tile's rows of
  // a[jbase + 8 (v / 4) + 4 h + v % 4][row] X[row][32 cb + l32].  X operand
  // rows r0 = 16 q + 4 h + s16 / 4 and r1 = r0 + 8 by transposing reads
  // (addresses as in sa_stream32.hpp); operands of row step q are read while
  // the products of step q - 1 run.
  uint32_t xb[2][2];
#pragma unroll
  for (int qp = 0; qp < 2; ++qp)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = 16 * qp + 4 * h + (s16 >> 2) + 8 * rr;
      const int c0 = 2 * (g16 & 1) + ((s16 & 3) >> 1);
      xb[qp][rr] = (uint32_t)(row * 256 + 16 * (c0 ^ chunk_sw32(row)) + 8 * (s16 & 1));
    }
  auto agg_load = [&](int q, bf16x8 (&B)[CBK], uint32_t xs) {
    const int qp = q & 1;
    const uint32_t qo = (uint32_t)((q >> 1) * 32 * 256);
#pragma unroll
    for (int cb = 0; cb < CBK; ++cb) {
      const u32x2 b0 = lds_tr16((xb[qp][0] ^ (uint32_t)(64 * cb)) + xs + qo);
      const u32x2 b1 = lds_tr16((xb[qp][1] ^ (uint32_t)(64 * cb)) + xs + qo);
      B[cb] = __builtin_bit_cast(bf16x8, u32x4{b0.x, b0.y, b1.x, b1.y});
    }
  };
  // B[0] holds the operands of row step 0, read ahead by the caller
  auto aggregate = [&](f32x16 (&acc)[CBK], const bf16x8 (&a)[4], bf16x8 (&B)[2][CBK], uint32_t xs, auto hook) {
#pragma unroll
    for (int q = 0; q < NT / 16; ++q) {
      if (q + 1 < NT / 16) agg_load(q + 1, B[(q + 1) & 1], xs);
#pragma unroll
      for (int cb = 0; cb < CBK; ++cb) acc[cb] = mfma32(a[q], B[q & 1][cb], acc[cb]);
      hook(q);  // independent vector work issued in the products' shadow
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- partial of one (group, user) piece: float4 number ((wj CBK + cb) 4 + v / 4) 64 + lane of the slot
  float hm = -INFINITY, hl = 0.f;  // comparator: the piece's maximum and this lane's sum for prototype jbase + l32
  auto flush = [&](f32x16 (&acc)[CBK], int u) {
    float* dst = args.partial + (grp + u) * (int64_t)(HS ? KPAD * (D + 2) : KPAD * D);
    if constexpr (HS) {
      // after the accumulators: the maxima [KPAD], then the sums over the piece's rows [KPAD]
      const float lt = pair32_sum(hl);
      if (h == 0) {
        dst[KPAD * D + jbase + l32] = hm;
        dst[KPAD * D + KPAD + jbase + l32] = lt;
      }
      hm = -INFINITY;
      hl = 0.f;
    }
#pragma unroll
    for (int cb = 0; cb < CBK; ++cb)
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const f32x4 v = {acc[cb][4 * vq], acc[cb][4 * vq + 1], acc[cb][4 * vq + 2], acc[cb][4 * vq + 3]};
        *reinterpret_cast<f32x4*>(dst + ((((wj * CBK + cb) * 4 + vq) * 64) + lane) * 4) = v;
      }
#pragma unroll
    for (int cb = 0; cb < CBK; ++cb) acc[cb] = f32x16{};
  };

  f32x16 acc[CBK];
#pragma unroll
  for (int cb = 0; cb < CBK; ++cb) acc[cb] = f32x16{};

  // ---- comparator: rows past the piece out, the tile maximum of the lane's
  // prototype (in-lane, then the half-wave partner), and when a maximum grows
  // by more than 8 the rescale of its sum and accumulator rows (register v of
  // acc holds prototype 8 (v / 4) + 4 h + v % 4, whose factor lane that is)
  auto hs_max = [&](f32x16 (&sv)[2], int nv) {
    if (nv < NT) {
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          sv[f][v] = 32 * f + 8 * (v >> 2) + 4 * h + (v & 3) < nv ? sv[f][v] : -INFINITY;
    }
    float tm = sv[0][0];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) tm = fmaxf(tm, sv[f][v]);
    const float mnew = fmaxf(hm, pair32_max(tm));
    if (__builtin_amdgcn_ballot_w64(mnew > hm + 8.f) != 0) {  // a piece's first tile, or a jump of a maximum
      const float alpha = hm == -INFINITY ? 0.f : fast_exp2(hm - mnew);
      hl *= alpha;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float av = __shfl(alpha, 8 * (v >> 2) + 4 * h + (v & 3));
#pragma unroll
        for (int cb = 0; cb < CBK; ++cb) acc[cb][v] *= av;
      }
      hm = mnew;
    }
  };
  // weights of row step rs, 2^(s' - m) (a prototype that saw no row, i.e. padding: 0)
  auto hs_weights_rs = [&](bf16x8 (&a)[4], const f32x16 (&sv)[2], int rs) {
    const int f = rs >> 1, o = 8 * (rs & 1);
    const float mu = hm == -INFINITY ? 0.f : hm;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float w = fast_exp2(sv[f][o + e] - mu);
      hl += w;
      a[rs][e] = (bf16)w;
    }
  };

  const int64_t e0 = first_end - r_begin;
  Cursor cc{0, e0 < (int64_t)nrel ? (int)e0 : nrel, u_first};  // tile t
  Cursor cl = cc;  // next tile to load
  Cursor ca = cc;  // tile whose affinity comes next
  cursor_next(cl);
#pragma unroll
  for (int p = 1; p < NS - 1; ++p) {
    issue_tile(cl, p);
    cursor_next(cl);
  }
  auto row_ok = [&](const Cursor& c, int row) { return row < c.end - c.row; };
  auto ensure_m = [&]() {
    if constexpr (PU) {
      if (ca.u != m_user) {
        load_m(ca.u);
        m_user = ca.u;
      }
    }
  };

  // prologue: affinity and exponentials of tile 0
  f32x16 S0[2], S1[2];
  ensure_m();
  wait_tiles(std::integral_constant<int, NS - 2>{});
  __syncthreads();
  affinity(S0, slot_of(0), no_hook);
  cursor_next(ca);
  if constexpr (!HS) softmax_all(S0, 0);
  wait_tiles(std::integral_constant<int, NS - 3>{});  // tile 1
  __syncthreads();

  // Step t (one barrier): DMA of tile t+3; the row sums of tile t from LDS
  // (all waves'); the affinity of tile t+1, and in its shadow the factors and
  // weights of tile t; the aggregation of tile t, and in its shadow the
  // exponentials and row sums of tile t+1.  Sa holds tile t's exponentials,
  // Sb receives tile t+1's scores.
  auto step = [&](int t, f32x16 (&Sa)[2], f32x16 (&Sb)[2], auto full, auto q0_) {
    const int q0 = q0_;  // a compile-time constant in the unrolled loop, t % NS in the tail
    const int q1 = q0 + 1 < NS ? q0 + 1 : q0 + 1 - NS;
    const int qn = q0 > 0 ? q0 - 1 : NS - 1;
    constexpr bool F = decltype(full)::value;
    issue_tile(cl, qn);
    const bool nxt = F || t + 1 < ntot;
    if constexpr (HS) {
      // the comparator: tile t's maximum and rescale, its weights in the shadow
      // of tile t+1's affinity, then tile t's aggregation (no row statistics)
      bf16x8 a[4];
      bf16x8 B[2][CBK];
      hs_max(Sa, cc.end - cc.row);
      auto shadow_h = [&](int kc) {
        if (kc < 4) hs_weights_rs(a, Sa, kc);
        if (kc == KC - 1) agg_load(0, B[0], slot_of(q0));
      };
      if (nxt) {
        affinity(Sb, slot_of(q1), shadow_h);
      } else {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) shadow_h(kc);
      }
      cursor_next(ca);
      aggregate(acc, a, B, slot_of(q0), no_hook);
      if (cc.row + NT >= cc.end) flush(acc, cc.u);
      cursor_next(cc);
      cursor_next(cl);
      wait_tiles(std::integral_constant<int, NS - 3>{});  // tile t+2
      __syncthreads();
      return;
    }
    f32x4 pv[2][WJ / 4];
    combine_issue(pv, t & 1);
    float fr[2] = {1.f, 1.f}, lr[2] = {1.f, 1.f};
    bool bad = false;
    bf16x8 a[4];
    // factors of tile t at product kFactorsAt of the affinity (its reads have
    // had the products before to arrive), then its weights in four parts; a
    // wave with a row out of range takes the exact pass after the products
    // instead.  The aggregation's first operands are read during the last
    // affinity product.
    bf16x8 B[2][CBK];
    auto shadow_a = [&](int kc) {
      if (kc == kFactorsAt) {
        combine_finish(pv, fr, lr, bad);
        fr[0] = row_ok(cc, row_a) ? fr[0] : 0.f;
        fr[1] = row_ok(cc, row_a + 8) ? fr[1] : 0.f;
      }
      if (kc > kFactorsAt && kc <= kFactorsAt + 4 && !bad) weights_rs(a, Sa, fr, kc - kFactorsAt - 1);
      if (kc == KC - 1) agg_load(0, B[0], slot_of(q0));
    };
    ensure_m();
    if (nxt) {
      affinity(Sb, slot_of(q1), shadow_a);
    } else {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) shadow_a(kc);
    }
    cursor_next(ca);
    if (bad) {
      exact_wave(Sa, fr, slot_of(q0), cc.u);
      fr[0] = row_ok(cc, row_a) ? 1.f : 0.f;
      fr[1] = row_ok(cc, row_a + 8) ? 1.f : 0.f;
#pragma unroll
      for (int rs = 0; rs < 4; ++rs) weights_rs(a, Sa, fr, rs);
    }
    auto shadow_g = [&](int q) {
      if (nxt) softmax_piece(Sb, q, (t + 1) & 1);
    };
    aggregate(acc, a, B, slot_of(q0), shadow_g);
    if (cc.row + NT >= cc.end) flush(acc, cc.u);
    cursor_next(cc);
    cursor_next(cl);
    wait_tiles(std::integral_constant<int, NS - 3>{});  // tile t+2
    __syncthreads();
  };
  using Full = std::integral_constant<bool, true>;
  using Tail = std::integral_constant<bool, false>;
  static_assert(NS % 2 == 0, "an unrolled pass over the ring leaves the score buffers where it found them");
  int t = 0;
  for (; t + NS < ntot; t += NS) {
    static_for<0, NS>([&](auto i_) {
      constexpr int i = decltype(i_)::value;
      if constexpr (i % 2 == 0)
        step(t + i, S0, S1, Full{}, i_);
      else
        step(t + i, S1, S0, Full{}, i_);
    });
  }
  int q = 0;  // t % NS here
  while (t < ntot) {
    step(t, S0, S1, Tail{}, q);
    q = q + 1 < NS ? q + 1 : 0;
    if (++t >= ntot) break;
    step(t, S1, S0, Tail{}, q);
    q = q + 1 < NS ? q + 1 : 0;
    ++t;
  }
  wait_vm<0>();  // no DMA outlives the work group
}

template <bool PAD, bool PU, bool HS>
hipError_t launch_wide_t(const FusedArgs& a, const Launch& l) {
  if (l.start || l.stop)
    hipExtLaunchKernelGGL((sa_wide_kernel<PAD, PU, HS>), dim3(l.groups), dim3(512), 0, l.stream, l.start, l.stop, 0, a);
  else
    hipLaunchKernelGGL((sa_wide_kernel<PAD, PU, HS>), dim3(l.groups), dim3(512), 0, l.stream, a);
  return hipGetLastError();
}

template <bool PAD>
hipError_t launch_wide_pad(const FusedArgs& a, const Launch& l) {
  if (a.lse_mode != 0) return hipErrorInvalidValue;  // one pass
  if (a.history_softmax) {
    if (a.m_stride != 0 || a.blocks != 1) return hipErrorInvalidValue;  // one shared matrix, one block
    return launch_wide_t<PAD, false, true>(a, l);
  }
  return a.m_stride != 0 ? launch_wide_t<PAD, true, false>(a, l) : launch_wide_t<PAD, false, false>(a, l);
}

}  // namespace sa
