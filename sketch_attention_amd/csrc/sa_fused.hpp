// Fused Sketch Attention compression pass for gfx950 (MI355X).
//
// Operation (SequenceO1 close-reading page, section 2.1): for every history
// row x_i of a user and every prototype j,
//     s'_ji = M_j . x_i            with M = tau * log2(e) * P W_Q W_K^T (folded once)
//     a_ji  = 2^(s'_ji) / sum_j' 2^(s'_j'i)      (softmax over the prototype axis)
//     X~_j += a_ji x_i                            (aggregation of the raw rows)
// Section 2.4 asks for exactly this shape of kernel: the affinity is tiled,
// the softmax statistics are kept on chip, the aggregation is fused, the
// k x n matrices never reach HBM, and batches of unequal-length histories are
// accepted.
//
// Work split.  A launch covers `rows` packed rows of up to 256 users.  Work
// group b of G owns rows [floor(b*rows/G), floor((b+1)*rows/G)), walking
// across user boundaries; each (group, user) piece produces one float32 k x d
// partial sketch in slot (b + u) (unique: b and u both grow along the rows),
// and a second kernel sums the partials of each user in group order.  The
// split is exact because the softmax of one row does not depend on any other
// row, so the sketch is additive over any partition of a user's rows.
//
// Inside a work group.  NW waves (eight for bf16, two per SIMD; four for
// float32): WJ waves split the k_pad prototypes (KW each) and WI = NW / WJ
// split the rows of a tile (32 rows each).  Per tile of NT = 32 * WI rows:
//   1. the tile is staged from HBM (read once, prefetched two tiles ahead into
//      registers) into LDS twice: row-major Xr for the affinity product and
//      transposed Xt for the aggregation product;
//   2. S'^T (32 rows x KW prototypes per wave) = Xr . M^T on the matrix cores
//      (16x16x32 bf16 or 16x16x4 f32), M fragments from LDS or registers;
//   3. in the output layout of that product each lane holds one prototype and
//      four rows per 16x16 block, so the prototype-axis sums are a 16-lane DPP
//      butterfly plus an LDS exchange across the WJ waves; the exponent is
//      taken without a max shift, and a tile whose row sums leave the safe
//      range is recomputed on an exact, max-shifted path;
//   4. the normalised weights are rounded to the operand type in registers
//      and used directly as the A operand of X~ (KW x D) += A (KW x 32) .
//      X (32 x D): the reduction index of that product is the row index, and
//      the rows each lane holds are exactly the rows its operand slot needs,
//      so no LDS round trip is needed for A;
//   5. accumulators stay in registers (float32) for the whole piece.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa_internal.h"

namespace sa {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------- MFMA ops
template <typename T>
struct Mfma;

template <>
struct Mfma<bf16> {
  static constexpr int kStep = 32;  // reduction length of one instruction
  using Frag = bf16x8;              // 8 reduction elements per lane
  __device__ __forceinline__ static f32x4 run(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  static constexpr int kStep = 4;
  using Frag = float;               // 1 reduction element per lane
  __device__ __forceinline__ static f32x4 run(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// ------------------------------------------------- 16-lane DPP reductions
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror:
// after the four steps every lane of a 16-lane row holds the row's result.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));
  x = fmaxf(x, dpp_f32<0x4E>(x));
  x = fmaxf(x, dpp_f32<0x141>(x));
  x = fmaxf(x, dpp_f32<0x140>(x));
  return x;
}

__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  x += dpp_f32<0x140>(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Transposing butterfly over the 16 lanes of a DPP row: p[r] is this lane's
// partial for row r (r = 0..3); on return every lane of a quad holds the
// 16-lane total of row 2*bit3 + bit2 of its lane index.  11 VALU operations
// instead of 16 for four independent all-reductions.
__device__ __forceinline__ float rows4_sum_scatter(const float (&p)[4], int l16) {
  const bool hi = (l16 & 8) != 0;
  const float keep0 = hi ? p[2] : p[0], send0 = hi ? p[0] : p[2];
  const float keep1 = hi ? p[3] : p[1], send1 = hi ? p[1] : p[3];
  const float q0 = keep0 + dpp_f32<0x128>(send0);  // row_ror:8 = lane ^ 8
  const float q1 = keep1 + dpp_f32<0x128>(send1);
  const bool b2 = (l16 & 4) != 0;
  const float keep = b2 ? q1 : q0, send = b2 ? q0 : q1;
  float z = keep + dpp_f32<0x141>(send);           // row_half_mirror flips bit 2
  z += dpp_f32<0xB1>(z);                           // quad xor 1
  z += dpp_f32<0x4E>(z);                           // quad xor 2
  return z;
}

// ------------------------------------------------- work group -> block
// Passes split over prototype blocks launch nblk work groups per row range.
// Work groups are dealt to the 8 XCDs in turn (XCD = index mod 8), so when
// the row ranges come in multiples of 8 the nblk blocks of one range take
// indices 8 apart: one XCD, dispatched together, and the range's X tiles,
// read once per block, meet in that XCD's L2.  Otherwise block = index mod
// nblk, range = index / nblk.
struct GroupBlock {
  int64_t grp;  // row range
  int blk;      // prototype block
};
__device__ __forceinline__ GroupBlock group_block(unsigned bi, unsigned grid, int nblk) {
  const unsigned nb = (unsigned)nblk;
  if (nb > 1 && (grid / nb) % 8u == 0) return {(int64_t)(8u * (bi / 8u / nb) + bi % 8u), (int)((bi / 8u) % nb)};
  return {(int64_t)(bi / nb), (int)(bi % nb)};
}

// ------------------------------------------------------ static geometry
// NW waves per work group: WJ split the prototypes (KW each), WI = NW / WJ
// split the rows of a tile (32 rows each).  The transposed tile copy Xt is
// double-buffered (two barriers per tile) when LDS allows, else single (three).
template <typename T, int D, int KW, int WJ, int WI, bool MLDS>
struct FusedGeom {
  static_assert(KW % 16 == 0 && D % 32 == 0, "tile shape");
  static constexpr int NW = WJ * WI;
  static constexpr int THREADS = 64 * NW;
  static constexpr int NT = kRowsPerWave * WI;   // tile rows
  static constexpr int JB = KW / 16;             // 16-prototype blocks per wave
  static constexpr int CB = D / 16;              // 16-column blocks of the output
  static constexpr int CS = D / Mfma<T>::kStep;  // affinity reduction steps
  static constexpr int KPAD = KW * WJ;
  static constexpr int XRS = D + 32 / (int)sizeof(T);  // Xr row stride (elements): +32 bytes keeps fragment reads conflict-free
  static constexpr int XTS = NT + 4;                   // Xt row stride (elements): odd multiple of 4 spreads the stores
  static constexpr int MS_WIDE = D + 16, MS_NARROW = D + 8;  // LDS M row stride (bf16 elements)
  static constexpr int XR_BYTES = NT * XRS * (int)sizeof(T);
  static constexpr int XT_BYTES = D * XTS * (int)sizeof(T);
  static constexpr int XL_BYTES = NT * WJ * 4;         // per-wave row sums
  static constexpr int FLAG_BYTES = 4 * NW;
  static constexpr int region0 = NT * XRS * (int)sizeof(T) + D * XTS * (int)sizeof(T) + 3 * NT * WJ * 4 + NT * 4 + 4 * NW;
  static constexpr int MS = (!MLDS || region0 + KPAD * MS_WIDE * 2 <= 160 * 1024) ? MS_WIDE : MS_NARROW;
  static constexpr int M_BYTES = MLDS ? KPAD * MS * 2 : 0;
  static constexpr int stage_bytes = WI > 1 ? WJ * CB * 64 * 16 : 0;  // one prototype block of every wave's accumulators
  static constexpr int XF_BYTES = NT * 4;              // per-row factors
  static constexpr int region(int nxt) { return XR_BYTES + nxt * XT_BYTES + 3 * XL_BYTES + XF_BYTES + FLAG_BYTES; }
  static constexpr int NXT = region(2) + M_BYTES <= 160 * 1024 ? 2 : 1;
  static constexpr int XREG = region(NXT) > stage_bytes ? region(NXT) : stage_bytes;
  static constexpr int OFF_XT = XR_BYTES;
  static constexpr int OFF_XL = XR_BYTES + NXT * XT_BYTES;
  static constexpr int OFF_XSM = OFF_XL + XL_BYTES;     // exact path: per-wave row maxima
  static constexpr int OFF_XSL = OFF_XSM + XL_BYTES;    // exact path: per-wave row sums
  static constexpr int OFF_XF = OFF_XSL + XL_BYTES;
  static constexpr int OFF_FLAG = OFF_XF + XF_BYTES;
  static constexpr int OFF_M = XREG;
  static constexpr int LDS_BYTES = XREG + M_BYTES;
  static constexpr int QC = D / 4;                     // 4-column quads per row
  static constexpr int NBLK = (NT / 4) * QC;           // 4x4 blocks per tile
  static constexpr int BPT = (NBLK + THREADS - 1) / THREADS;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CDNA4 compute unit");
};

// ------------------------------------------------------- X tile staging
// One thread moves a 4x4 block (rows 4rq..4rq+3, columns 4cq..4cq+3 of the
// tile) from HBM into registers, then into both LDS layouts.  Consecutive
// threads take consecutive column quads of the same rows, so each global load
// instruction of a wave reads whole rows.  Rows at or past row_end read the
// last valid row (always in bounds) and are then zeroed, so no branch splits
// the surrounding code.
template <typename T>
struct Quad;
template <>
struct Quad<bf16> {
  u32x2 v[4];  // row r: .x = columns 0 (low half) and 1, .y = columns 2 and 3
};
template <>
struct Quad<float> {
  f32x4 v[4];
};

// tile: first row of the tile (uniform); rows_left: valid rows from there,
// 1..NT; r4 = 4*rq.  Offsets stay 32-bit.
template <int D>
__device__ __forceinline__ void quad_load(Quad<bf16>& q, const bf16* tile, int rows_left, int r4, int col) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rr = r4 + r < rows_left ? r4 + r : rows_left - 1;
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(tile + rr * D + col));
    const bool ok = r4 + r < rows_left;
    q.v[r] = u32x2{ok ? v.x : 0u, ok ? v.y : 0u};
  }
}

template <int D>
__device__ __forceinline__ void quad_load(Quad<float>& q, const float* tile, int rows_left, int r4, int col) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rr = r4 + r < rows_left ? r4 + r : rows_left - 1;
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(tile + rr * D + col));
    const bool ok = r4 + r < rows_left;
    q.v[r] = f32x4{ok ? v[0] : 0.f, ok ? v[1] : 0.f, ok ? v[2] : 0.f, ok ? v[3] : 0.f};
  }
}

template <typename T>
__device__ __forceinline__ void quad_zero(Quad<T>& q) {
#pragma unroll
  for (int r = 0; r < 4; ++r) q.v[r] = {};
}

// xr -> Xr[4rq][4cq] (row stride xrs)
__device__ __forceinline__ void quad_store_r(const Quad<bf16>& q, bf16* xr, int xrs) {
#pragma unroll
  for (int r = 0; r < 4; ++r) *reinterpret_cast<u32x2*>(xr + r * xrs) = q.v[r];
}
__device__ __forceinline__ void quad_store_r(const Quad<float>& q, float* xr, int xrs) {
#pragma unroll
  for (int r = 0; r < 4; ++r) *reinterpret_cast<f32x4*>(xr + r * xrs) = q.v[r];
}
// xt -> Xt[4cq][4rq] (row stride xts): column c of the four rows
__device__ __forceinline__ void quad_store_t(const Quad<bf16>& q, bf16* xt, int xts) {
  const u32x2 c0 = {(q.v[0].x & 0xFFFFu) | (q.v[1].x << 16), (q.v[2].x & 0xFFFFu) | (q.v[3].x << 16)};
  const u32x2 c1 = {(q.v[0].x >> 16) | (q.v[1].x & 0xFFFF0000u), (q.v[2].x >> 16) | (q.v[3].x & 0xFFFF0000u)};
  const u32x2 c2 = {(q.v[0].y & 0xFFFFu) | (q.v[1].y << 16), (q.v[2].y & 0xFFFFu) | (q.v[3].y << 16)};
  const u32x2 c3 = {(q.v[0].y >> 16) | (q.v[1].y & 0xFFFF0000u), (q.v[2].y >> 16) | (q.v[3].y & 0xFFFF0000u)};
  *reinterpret_cast<u32x2*>(xt + 0 * xts) = c0;
  *reinterpret_cast<u32x2*>(xt + 1 * xts) = c1;
  *reinterpret_cast<u32x2*>(xt + 2 * xts) = c2;
  *reinterpret_cast<u32x2*>(xt + 3 * xts) = c3;
}
__device__ __forceinline__ void quad_store_t(const Quad<float>& q, float* xt, int xts) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    *reinterpret_cast<f32x4*>(xt + c * xts) = f32x4{q.v[0][c], q.v[1][c], q.v[2][c], q.v[3][c]};
  }
}

// ---------------------------------------------- operand fragment loads
// Reduction slot (g, e) of the affinity product, g = lane / 16 and e the
// element within the lane, maps to column c of X and M:
//   bf16: c = 32*cs + 8*g + e   (8 consecutive columns per lane)
//   f32:  c = g*(D/4) + cs      (one column per lane and step)
// Both operands use the same map, so the product is the plain sum over c.
template <int D>
__device__ __forceinline__ bf16x8 frag_c(const bf16* base_row, int cs, int g) {
  return *reinterpret_cast<const bf16x8*>(base_row + 32 * cs + 8 * g);
}
template <int D>
__device__ __forceinline__ float frag_c(const float* base_row, int cs, int g) {
  return base_row[g * (D / 4) + cs];
}
// The same fragments gathered from the transposed copy Xt (column-major),
// used only when a tile's affinity must be recomputed.
template <int D>
__device__ __forceinline__ bf16x8 frag_c_t(const bf16* xt, int xts, int row, int cs, int g) {
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = xt[(32 * cs + 8 * g + e) * xts + row];
  return f;
}
template <int D>
__device__ __forceinline__ float frag_c_t(const float* xt, int xts, int row, int cs, int g) {
  return xt[(g * (D / 4) + cs) * xts + row];
}

// -------------------------------------------------------------- kernel
// LM (two-phase modes, FusedArgs::lse_mode): 0 one pass; 1 each row's log2
// sum over this block's prototypes into stats[block][row], no aggregation;
// 2 weights 2^(s' - L) with L the row's log2 sum over every block from
// stats[row] (no row sums, no exact path).  In modes 1, 2 and 3 the work
// groups split over the row ranges and the prototype blocks as group_block
// deals them.
// LM 3 is the comparator (FusedArgs::history_softmax; the SequenceO1 page's
// section 3.1 baseline): the softmax runs over the user's rows, per
// prototype, so no row statistics are exchanged between waves.  Per piece
// each prototype keeps a running maximum m (raised only when a tile exceeds
// it by more than 8 in log2 units, so every weight stays below 2^8), the sum
// l of 2^(s' - m) over its rows and the accumulator in the scale of m; the
// piece's partial is (acc, m, l) and reduce_history_kernel merges a user's
// pieces and divides.  Waves never split a tile's rows in this mode.
template <typename T, int D, int KW, int WJ, int WI, bool MLDS, bool PAD, int LM = 0>
__global__ __launch_bounds__(64 * WJ * WI) void sa_fused_kernel(FusedArgs args) {
  using G = FusedGeom<T, D, KW, WJ, WI, MLDS>;
  using MF = Mfma<T>;
  using Frag = typename MF::Frag;
  constexpr int JB = G::JB, CB = G::CB, CS = G::CS, NT = G::NT, NW = G::NW, THREADS = G::THREADS;
  static_assert(!MLDS || sizeof(T) == 2, "LDS-resident M is bf16 only");
  static_assert(LM != 3 || WI == 1, "the comparator keeps whole tile columns per wave");
  constexpr int SLOT = LM == 3 ? G::KPAD * (D + 2) : G::KPAD * D;  // floats per partial slot

  __shared__ __attribute__((aligned(16))) unsigned char lds[G::LDS_BYTES];
  T* const Xr = reinterpret_cast<T*>(lds);
  T* const Xt0 = reinterpret_cast<T*>(lds + G::OFF_XT);
  T* const Xt1 = reinterpret_cast<T*>(lds + G::OFF_XT + (G::NXT - 1) * G::XT_BYTES);
  float* const xl = reinterpret_cast<float*>(lds + G::OFF_XL);    // [NT][WJ]
  float* const xsm = reinterpret_cast<float*>(lds + G::OFF_XSM);  // [NT][WJ]
  float* const xsl = reinterpret_cast<float*>(lds + G::OFF_XSL);  // [NT][WJ]
  float* const xf = reinterpret_cast<float*>(lds + G::OFF_XF);    // [NT]
  int* const flags = reinterpret_cast<int*>(lds + G::OFF_FLAG);   // [NW]
  T* const Ms = reinterpret_cast<T*>(lds + G::OFF_M);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wj = wave % WJ;
  const int wi = wave / WJ;
  const int rw = wi * kRowsPerWave;  // first tile row of this wave
  const int jbase = wj * KW;         // first prototype of this wave (within the block)
  const int nblk = LM ? args.blocks : 1;
  const GroupBlock gb = group_block(blockIdx.x, gridDim.x, nblk);
  const int blk = LM ? gb.blk : 0;
  const T* const X = static_cast<const T*>(args.X);
  const T* const Mg = static_cast<const T*>(args.M) + (int64_t)blk * G::KPAD * D;
  const int k = args.k - blk * G::KPAD;  // real prototypes of this block (may exceed KPAD)
  const bool wave_has_protos = jbase < k;

  const int64_t rows = args.rows;
  const int64_t ngroups = gridDim.x / nblk;
  const int64_t grp = gb.grp;
  const int64_t r_begin = grp * rows / ngroups;
  const int64_t r_end = (grp + 1) * rows / ngroups;
  if (r_begin >= r_end) return;

  // Folded matrix of user u (one shared matrix when m_stride is 0): this
  // wave's KW rows as B fragments of the affinity product.  Called at the
  // start of a piece, before its first barrier, which orders the LDS copy
  // before every read; the barrier before the call (per-user matrices only)
  // ends the reads of the previous piece.
  Frag mreg[MLDS ? 1 : JB][MLDS ? 1 : CS];
  auto load_m = [&](int u) {
    const T* const Mu = Mg + (int64_t)u * args.m_stride;
    if constexpr (MLDS) {
      constexpr int CH = D / 8;  // 16-byte chunks per row
      for (int idx = tid; idx < G::KPAD * CH; idx += THREADS) {
        const int r = idx / CH, ch = idx % CH;
        *reinterpret_cast<u32x4*>(Ms + r * G::MS + ch * 8) = *reinterpret_cast<const u32x4*>(Mu + r * D + ch * 8);
      }
    } else {
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        const T* mrow = Mu + (int64_t)(jbase + 16 * jb + l16) * D;
#pragma unroll
        for (int cs = 0; cs < CS; ++cs) mreg[jb][cs] = frag_c<D>(mrow, cs, g);
      }
    }
  };

  // ---- affinity of one tile: s[ib][jb][r] = S'^T[rw + 16 ib + 4 g + r][jbase + 16 jb + l16],
  // padded prototypes set to -inf.  xfrag(ib, cs) supplies the X fragments.
  auto affinity_from = [&](f32x4 (&s)[2][JB], auto&& xfrag) {
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) s[ib][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
      Frag xa[2];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) xa[ib] = xfrag(ib, cs);
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        Frag mf;
        if constexpr (MLDS) {
          mf = frag_c<D>(Ms + (jbase + 16 * jb + l16) * G::MS, cs, g);
        } else {
          mf = mreg[jb][cs];
        }
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) s[ib][jb] = MF::run(xa[ib], mf, s[ib][jb]);
      }
    }
    if constexpr (PAD) {
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        const bool ok = jbase + 16 * jb + l16 < k;
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[ib][jb][r] = ok ? s[ib][jb][r] : -INFINITY;
      }
    }
  };

  auto affinity = [&](f32x4 (&s)[2][JB]) {
    affinity_from(s, [&](int ib, int cs) { return frag_c<D>(Xr + (rw + 16 * ib + l16) * G::XRS, cs, g); });
  };

  // ---- softmax, fast half: e = 2^s' in place (no shift), this wave's row
  // sums to xl, and a per-wave flag when a sum leaves [2^-100, 2^100] (then
  // the exact shifted path recomputes the tile).
  auto softmax_fast = [&](f32x4 (&s)[2][JB]) {
    bool bad = false;
    if constexpr (LM >= 2) return;  // exponentials are taken against the stored log-sum-exp (2) or the prototype's maximum (3) in finish_tile
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const float e = fast_exp2(s[ib][jb][r]);
          s[ib][jb][r] = e;
          acc += e;
        }
        p[r] = acc;
      }
      const float z = rows4_sum_scatter(p, l16);
      bad |= !(z >= 0x1p-100f && z <= 0x1p100f);
      if ((l16 & 3) == 0) {
        const int trow = rw + 16 * ib + 4 * g + ((l16 >> 3) << 1) + ((l16 >> 2) & 1);
        xl[trow * WJ + wj] = z;
      }
    }
    const bool wave_bad = __builtin_amdgcn_ballot_w64(bad && wave_has_protos) != 0;
    if (lane == 0) flags[wave] = wave_bad ? 1 : 0;  // one flag per wave: waves that split rows share wj
  };

  // ---- after the exchange barrier: per-row factors 1 / sum_w l_w.  Lane
  // L < 32 finishes row rw + L and leaves the factor in xf; each lane then
  // reads the factors of its own eight rows (same wave, LDS in order).
  auto combine_fast = [&](float (&fac)[2][4]) {
    if (lane < kRowsPerWave) {
      const float* p = xl + (rw + lane) * WJ;
      float l = p[0];
#pragma unroll
      for (int w = 1; w < WJ; ++w) l += p[w];
      xf[rw + lane] = __builtin_amdgcn_rcpf(l);
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      const f32x4 f = *reinterpret_cast<const f32x4*>(xf + rw + 16 * ib + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) fac[ib][r] = f[r];
    }
  };

  auto any_flag = [&]() {
    if constexpr (LM >= 2) return false;
    int f = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) f |= flags[w];
    return __builtin_amdgcn_readfirstlane(f) != 0;
  };

  // ---- aggregation: acc[jb][cb][r] += sum_i a[jbase+16jb+4g+r][i] X[i][16cb+l16]
  auto aggregate = [&](f32x4 (&acc)[JB][CB], const f32x4 (&s)[2][JB], const float (&fac)[2][4], const T* xt) {
    if constexpr (sizeof(T) == 2) {
      auto weights = [&](int jb) {
        bf16x8 a;
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = (bf16)(s[e >> 2][jb][e & 3] * fac[e >> 2][e & 3]);
        return a;
      };
      auto xcol = [&](int cb) {
        const T* p = xt + (16 * cb + l16) * G::XTS + rw + 4 * g;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 16);
        return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      };
      // keep the smaller operand set live: all weight fragments (cb outer) or
      // all X fragments (jb outer)
      if constexpr (JB <= CB) {
        bf16x8 a[JB];
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) a[jb] = weights(jb);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const bf16x8 xb = xcol(cb);
#pragma unroll
          for (int jb = 0; jb < JB; ++jb) acc[jb][cb] = MF::run(a[jb], xb, acc[jb][cb]);
        }
      } else {
        bf16x8 xb[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) xb[cb] = xcol(cb);
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const bf16x8 a = weights(jb);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) acc[jb][cb] = MF::run(a, xb[cb], acc[jb][cb]);
        }
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
          const f32x4 xv = *reinterpret_cast<const f32x4*>(xt + (16 * cb + l16) * G::XTS + rw + 16 * ib + 4 * g);
#pragma unroll
          for (int jb = 0; jb < JB; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[jb][cb] = MF::run(s[ib][jb][r] * fac[ib][r], xv[r], acc[jb][cb]);
        }
    }
  };

  // ---- exact path for a tile whose unshifted row sums left the safe range:
  // recompute the wave's affinity tile (the fast path overwrote it) with the
  // tile's rows read again from global memory,
  // shift each row by this wave's maximum, and combine the waves with the
  // usual max/sum rescaling.  Every wave takes it together (it has a barrier).
  auto softmax_exact = [&](f32x4 (&s)[2][JB], const T* tile, int rows_left, float (&fac)[2][4], float (&lse)[2][4]) {
    affinity_from(s, [&](int ib, int cs) {
      const int rr = rw + 16 * ib + l16;
      Frag f = frag_c<D>(tile + (int64_t)(rr < rows_left ? rr : rows_left - 1) * D, cs, g);
      if (rr >= rows_left) f = Frag{};
      return f;
    });
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float m = s[ib][0][r];
#pragma unroll
        for (int jb = 1; jb < JB; ++jb) m = fmaxf(m, s[ib][jb][r]);
        m = row16_max(m);
        const float mu = (m == -INFINITY) ? 0.f : m;  // a wave holding only padding
        float l = 0.f;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const float e = fast_exp2(s[ib][jb][r] - mu);
          s[ib][jb][r] = e;
          l += e;
        }
        l = row16_sum(l);
        fac[ib][r] = m;  // this wave's row maximum until the combine below
        if (l16 == 0) {
          const int trow = rw + 16 * ib + 4 * g + r;
          xsm[trow * WJ + wj] = m;
          xsl[trow * WJ + wj] = l;
        }
      }
    __syncthreads();
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int trow = rw + 16 * ib + 4 * g + r;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < WJ; ++w) mx = fmaxf(mx, xsm[trow * WJ + w]);
        float den = 0.f;
#pragma unroll
        for (int w = 0; w < WJ; ++w) den += xsl[trow * WJ + w] * fast_exp2(xsm[trow * WJ + w] - mx);
        fac[ib][r] = fast_exp2(fac[ib][r] - mx) / den;
        lse[ib][r] = mx + __log2f(den);  // the row's log2 sum over the block's prototypes
      }
  };

  // ---- after the exchange barrier: factors for the tile's rows, then the
  // aggregation (exact path in the rare tiles that need it).
  auto finish_tile = [&](f32x4 (&acc)[JB][CB], f32x4 (&sc)[2][JB], const T* xt, int64_t t0, int rows_left,
                         float (&hm)[JB], float (&hl)[JB]) {
    float fac[2][4];
    if constexpr (LM == 3) {
      // rows past the piece take no weight
      if (rows_left < NT) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool ok = rw + 16 * ib + 4 * g + r < rows_left;
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) sc[ib][jb][r] = ok ? sc[ib][jb][r] : -INFINITY;
          }
      }
      // the tile's maximum per prototype: lanes l16, l16 + 16, l16 + 32 and l16 + 48 share one
      float mnew[JB];
      bool grow = false;
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        float tm = sc[0][jb][0];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
          for (int r = 0; r < 4; ++r) tm = fmaxf(tm, sc[ib][jb][r]);
        tm = fmaxf(tm, __shfl_xor(tm, 16));
        tm = fmaxf(tm, __shfl_xor(tm, 32));
        mnew[jb] = fmaxf(hm[jb], tm);
        grow |= mnew[jb] > hm[jb] + 8.f;
      }
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // a piece's first tile, or a jump of a maximum
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const float alpha = hm[jb] == -INFINITY ? 0.f : fast_exp2(hm[jb] - mnew[jb]);
          hl[jb] *= alpha;
          // accumulator register r of this lane holds prototype 16 jb + 4 g + r, whose factor lane 4 g + r has
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float ar = __shfl(alpha, 4 * g + r);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) acc[jb][cb][r] *= ar;
          }
          hm[jb] = mnew[jb];
        }
      }
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        const float mu = hm[jb] == -INFINITY ? 0.f : hm[jb];  // a prototype that saw no row (padding): weights 0
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float w = fast_exp2(sc[ib][jb][r] - mu);
            hl[jb] += w;
            sc[ib][jb][r] = w;
          }
      }
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) fac[ib][r] = 1.f;
      aggregate(acc, sc, fac, xt);
      return;
    }
    if constexpr (LM == 2) {
      // 2^(s' - L) with the row's log-sum-exp over all blocks; rows past the piece weigh 0
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        const int r0 = rw + 16 * ib + 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float Lr = r0 + r < rows_left ? args.stats[t0 + r0 + r] : INFINITY;
#pragma unroll
          for (int jb = 0; jb < JB; ++jb) sc[ib][jb][r] = fast_exp2(sc[ib][jb][r] - Lr);
          fac[ib][r] = 1.f;
        }
      }
      aggregate(acc, sc, fac, xt);
      return;
    }
    if (any_flag()) {
      float lse[2][4];
      softmax_exact(sc, X + t0 * D, rows_left, fac, lse);
      if constexpr (LM == 1) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int trow = rw + 16 * ib + 4 * g + r;
            if (l16 == 0 && wj == 0 && trow < rows_left) args.stats[(int64_t)blk * rows + t0 + trow] = lse[ib][r];
          }
      }
    } else {
      combine_fast(fac);
      if constexpr (LM == 1) {
        // the row's log2 sum over the block (its unshifted sum is within range here)
        if (wj == 0 && lane < kRowsPerWave && rw + lane < rows_left) {
          const float* p = xl + (rw + lane) * WJ;
          float l = p[0];
#pragma unroll
          for (int w = 1; w < WJ; ++w) l += p[w];
          args.stats[(int64_t)blk * rows + t0 + rw + lane] = __log2f(l);
        }
      }
    }
    if constexpr (LM != 1) aggregate(acc, sc, fac, xt);
  };

  // First user touched: the largest u with offsets[u] <= r_begin.  It is
  // non-empty because offsets[u+1] > r_begin.
  int u;
  {
    int lo = 0, hi = args.users - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (args.offsets[mid] <= r_begin) lo = mid; else hi = mid - 1;
    }
    u = lo;
  }

  int64_t row = r_begin;
  int m_user = -1;  // user whose folded matrix is loaded
  while (row < r_end) {
    if (m_user < 0 || (args.m_stride != 0 && m_user != u)) {
      if (m_user >= 0) __syncthreads();  // every wave is done with the previous user's matrix
      load_m(u);
      m_user = u;
    }
    const int64_t seg_end = min(r_end, args.offsets[u + 1]);
    const int ntiles = (int)((seg_end - row + NT - 1) / NT);

    f32x4 acc[JB][CB];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[jb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float hm[JB], hl[JB];  // comparator: the piece's maximum and sum per prototype (this lane's rows)
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      hm[jb] = -INFINITY;
      hl[jb] = 0.f;
    }

    Quad<T> pre[G::BPT];
    auto prefetch = [&](int it) {
      const int64_t t0 = row + (int64_t)it * NT;
      const int64_t left = seg_end - t0;
      const int rows_left = left < NT ? (int)left : NT;
      const T* tile = X + t0 * D;
#pragma unroll
      for (int s = 0; s < G::BPT; ++s) {
        const int blk = tid + s * THREADS;
        if (G::NBLK % THREADS == 0 || blk < G::NBLK) {
          const int rq = blk / G::QC, cq = blk % G::QC;
          if (rows_left > 0) quad_load<D>(pre[s], tile, rows_left, 4 * rq, 4 * cq);
          else quad_zero(pre[s]);
        }
      }
    };
    auto store_r = [&]() {
#pragma unroll
      for (int s = 0; s < G::BPT; ++s) {
        const int blk = tid + s * THREADS;
        if (G::NBLK % THREADS == 0 || blk < G::NBLK) {
          const int rq = blk / G::QC, cq = blk % G::QC;
          quad_store_r(pre[s], Xr + (4 * rq) * G::XRS + 4 * cq, G::XRS);
        }
      }
    };
    auto store_t = [&](T* xt) {
#pragma unroll
      for (int s = 0; s < G::BPT; ++s) {
        const int blk = tid + s * THREADS;
        if (G::NBLK % THREADS == 0 || blk < G::NBLK) {
          const int rq = blk / G::QC, cq = blk % G::QC;
          quad_store_t(pre[s], xt + (4 * cq) * G::XTS + 4 * rq, G::XTS);
        }
      }
    };

    // Per tile it (rows row + it*NT ...):   affinity + fast softmax | B2 |
    // stage tile it+1 into LDS, issue loads of tile it+2, factors +
    // aggregation of tile it | B1.  With a single Xt buffer the staging of
    // Xt waits for the aggregation behind one more barrier.
    __syncthreads();  // LDS from the previous piece (and M staging) is settled
    prefetch(0);
    store_r();
    store_t(Xt0);
    __syncthreads();
    prefetch(1);
    f32x4 S[2][JB];
    for (int it = 0; it < ntiles; ++it) {
      T* const xt_cur = (G::NXT == 2 && (it & 1)) ? Xt1 : Xt0;
      const int64_t t0 = row + (int64_t)it * NT;
      const int rows_left = seg_end - t0 < NT ? (int)(seg_end - t0) : NT;
      affinity(S);
      softmax_fast(S);
      __syncthreads();  // B2: row sums visible; every wave is done reading Xr
      store_r();        // X(it+1)
      if constexpr (G::NXT == 2) {
        store_t((it & 1) ? Xt0 : Xt1);
        prefetch(it + 2);
        finish_tile(acc, S, xt_cur, t0, rows_left, hm, hl);
      } else {
        finish_tile(acc, S, Xt0, t0, rows_left, hm, hl);
        __syncthreads();  // every wave is done reading Xt
        store_t(Xt0);
        prefetch(it + 2);
      }
      __syncthreads();  // B1: tile it+1 staged
    }

    // ---- flush this (group, user) piece.  Partial layout per slot:
    // [wj][jb][cb][lane][4] float32, i.e. each lane's accumulator registers in
    // order; the reduction kernel maps it back to (prototype, column).  Waves
    // that split the rows first add their accumulators through LDS, one
    // prototype block at a time, in a fixed order.
    if constexpr (WI > 1) {
      float* stage = reinterpret_cast<float*>(lds);
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
    if (LM != 1 && wi == 0) {
      float* dst = args.partial + ((int64_t)blk * (ngroups + args.users) + grp + u) * (int64_t)SLOT;
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          *reinterpret_cast<f32x4*>(dst + (((wj * JB + jb) * CB + cb) * 64 + lane) * 4) = acc[jb][cb];
      if constexpr (LM == 3) {
        // after the accumulators: the maxima [KPAD], then the sums over the piece's rows [KPAD]
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          float lt = hl[jb] + __shfl_xor(hl[jb], 16);
          lt += __shfl_xor(lt, 32);
          if (g == 0) {
            dst[G::KPAD * D + jbase + 16 * jb + l16] = hm[jb];
            dst[G::KPAD * D + G::KPAD + jbase + 16 * jb + l16] = lt;
          }
        }
      }
    }

    row = seg_end;
    ++u;
    while (u < args.users && args.offsets[u + 1] <= row) ++u;  // skip empty histories
  }
}

template <typename T, int D, int KW, int WJ, int WI, bool MLDS, bool PAD, int LM = 0>
hipError_t launch_fused_lm(const FusedArgs& args, const Launch& l) {
  if (l.start || l.stop) {
    hipExtLaunchKernelGGL((sa_fused_kernel<T, D, KW, WJ, WI, MLDS, PAD, LM>), dim3(l.groups), dim3(64 * WJ * WI), 0,
                          l.stream, l.start, l.stop, 0, args);
  } else {
    hipLaunchKernelGGL((sa_fused_kernel<T, D, KW, WJ, WI, MLDS, PAD, LM>), dim3(l.groups), dim3(64 * WJ * WI), 0,
                       l.stream, args);
  }
  return hipGetLastError();
}
// The two-phase modes are compiled for the float32 plan of 4 x 64 prototypes
// per block only (float32 beyond 256 prototypes).
// The comparator (history_softmax) is compiled for the float32 plans of four
// waves over the prototypes and none over the rows (at d = 128 with at most
// 32 prototypes per wave: 64 spill registers there).
template <typename T, int D, int KW, int WJ, int WI, bool MLDS, bool PAD>
hipError_t launch_fused_t(const FusedArgs& args, const Launch& l) {
  if constexpr (sizeof(T) == 4 && WJ == 4 && WI == 1 && !MLDS && (D == 64 || KW <= 32)) {
    if (args.history_softmax) {
      if (args.lse_mode != 0) return hipErrorInvalidValue;
      return launch_fused_lm<T, D, KW, WJ, WI, MLDS, PAD, 3>(args, l);
    }
  }
  if (args.history_softmax) return hipErrorInvalidValue;
  if constexpr (sizeof(T) == 4 && KW == 64 && WJ == 4 && WI == 1 && !MLDS) {
    if (args.lse_mode == 1) return launch_fused_lm<T, D, KW, WJ, WI, MLDS, PAD, 1>(args, l);
    if (args.lse_mode == 2) return launch_fused_lm<T, D, KW, WJ, WI, MLDS, PAD, 2>(args, l);
  }
  if (args.lse_mode != 0) return hipErrorInvalidValue;
  return launch_fused_lm<T, D, KW, WJ, WI, MLDS, PAD, 0>(args, l);
}

template <typename T, int D, int KW, int WJ, int WI, bool MLDS, bool PAD>
hipError_t occupancy_t(int* n) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, sa_fused_kernel<T, D, KW, WJ, WI, MLDS, PAD>, 64 * WJ * WI,
                                                      0);
}

// One plan of the fused pass: launch it, or (occ != nullptr) report how
// many of its work groups fit on a compute unit.
template <typename T, int D, int KW, int WJ, int WI, bool MLDS>
hipError_t run_plan(const Plan& p, const FusedArgs& a, const Launch& l, int* occ) {
  if (p.k == p.k_pad)
    return occ ? occupancy_t<T, D, KW, WJ, WI, MLDS, false>(occ) : launch_fused_t<T, D, KW, WJ, WI, MLDS, false>(a, l);
  return occ ? occupancy_t<T, D, KW, WJ, WI, MLDS, true>(occ) : launch_fused_t<T, D, KW, WJ, WI, MLDS, true>(a, l);
}

#define SA_PLAN(T_, D_, KW_, WJ_, WI_, MLDS_)                                                       \
  if (p.kind == 0 && p.kw == KW_ && p.waves_k == WJ_ && p.waves_rows == WI_ && p.m_in_lds == MLDS_) \
    return run_plan<T_, D_, KW_, WJ_, WI_, MLDS_>(p, a, l, occ);

}  // namespace sa
