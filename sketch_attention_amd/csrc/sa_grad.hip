// Backward pass of Sketch Attention compression on gfx950 (bf16 inputs,
// float32 accumulation).  SequenceO1 close-reading page: section 2.1 defines
// the affinity, the prototype-axis softmax and the aggregation; section 2.4
// trains through the fused kernel, which needs their gradients.  With the
// upstream gradient G = dL/dX~ of a user's sketch:
//
//   dA = G X^T,  c_i = sum_j A_ji dA_ji,  dS = A * (dA - c)   (softmax over j)
//   dQ' = dS X                       (Q' = tau P W_Q W_K^T, S = Q' X^T)
//   dX  = A^T G + dS^T Q'
//
// Two streamed passes over X, each keeping its products on the matrix cores:
//
// grad_stats: the forward's layout.  WJ waves split the prototypes (32
//   each) of a 32-row tile staged in LDS; each computes s' = M x (log2
//   units) and dA = G x for its prototypes, and per row a local maximum, the
//   sum of 2^(s' - m_w) and of 2^(s' - m_w) dA.  One exchange through LDS
//   merges the waves (m = max m_w, l = sum l_w 2^(m_w - m), likewise c), the
//   lanes rebuild A and dS of their prototypes and add dS X into float32
//   accumulators (the forward's aggregation with dS as weights).  The row
//   statistics (m, 1/l, c) go to memory; the accumulators are one partial
//   per work group (all users together: the weights are shared), reduced by
//   the forward's split-n reduction.
//
// grad_dx: the roles swap.  Each wave owns 32 rows (X fragments and the
//   row statistics in registers) and walks the prototypes in chunks of 32
//   whose operands (M, G and the transposed G, Q' blocks, packed per user
//   once) arrive in LDS by DMA, double-buffered.  Per chunk it recomputes
//   s' and dA with the rows along the lanes, forms A and dS from its own
//   rows' statistics (no exchange), and accumulates dX^T = G^T A + Q'^T dS
//   on the matrix cores, so no wave ever needs another wave's prototypes.
#include <hip/hip_runtime.h>

#include "sa_grad.h"
#include "sa_stream.hpp"

namespace sa {

namespace {

// ------------------------------------------------------------ pass 1
// X arrives by LDS DMA into a ring of NS = 4 tiles (issued three tiles
// ahead, rows swizzled as in sa_stream.hpp).  Step t (one barrier): DMA of
// tile t+3 into the slot tile t-1 left; merge of tile t's row statistics
// (written by every wave in step t-1), its dS and the aggregation dQ' +=
// dS X; s' and dA of tile t+1 and their per-wave row statistics; wait for
// tile t+2.  So the products of tile t+1 overlap the merge of tile t.
template <int D, int WJ, bool PAD, int PHASE>
__global__ __launch_bounds__(64 * WJ) void grad_stats_kernel(GradStatsArgs args) {
  constexpr int KW = kGradKW, JB = KW / 16, RB = 2, NT = 16 * RB, CS = D / 32, CB = D / 16, CH = D / 8;
  constexpr int KPAD = KW * WJ;
  constexpr int NS = 4;
  constexpr int TILE_BYTES = NT * D * 2;
  constexpr int NI = TILE_BYTES / 1024;     // DMA blocks per tile
  constexpr int NIW = (NI + WJ - 1) / WJ;   // per wave (some waves may have one fewer, or none)
  constexpr int RPI = 1024 / (2 * D);       // rows per DMA block
  using MF = Mfma<bf16>;

  __shared__ __attribute__((aligned(1024))) unsigned char lds[NS * TILE_BYTES];
  __shared__ float xs_m[2][NT][WJ], xs_l[2][NT][WJ], xs_c[2][NT][WJ];
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) unsigned char*)lds;

  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int wj = __builtin_amdgcn_readfirstlane(tid >> 6);
  // prototype block (phases 1 and 2): prototypes KPAD blk .. of M and G
  constexpr int phase = PHASE;  // args.phase, as a template parameter: one block compiles as before
  const int nblk = phase ? args.blocks : 1;
  const GroupBlock gb = group_block(blockIdx.x, gridDim.x, nblk);  // the blocks of a row range on one XCD
  const int blk = phase ? gb.blk : 0;
  const int jbase = wj * KW;                // within the block
  const int jg = blk * KPAD + jbase;        // first global prototype of this wave
  const int k = args.k;
  const bf16* const X = static_cast<const bf16*>(args.X);
  const bf16* const M = static_cast<const bf16*>(args.M) + (int64_t)blk * KPAD * D;

  const int64_t rows = args.rows, ngroups = gridDim.x / nblk, grp = gb.grp;
  const int64_t r_begin = grp * rows / ngroups, r_end = (grp + 1) * rows / ngroups;
  if (r_begin >= r_end) return;  // the host launches at most one group per row

  // ---- tiles: pieces of [r_begin, r_end) per user, NT rows each
  // cursor rows relative to r_begin (a group's range fits in 32 bits: the
  // per-tile bookkeeping stays in 32-bit scalar arithmetic)
  const int nrel = (int)(r_end - r_begin);
  struct Cursor {
    int row, end, u;
  };
  int u0 = 0;
  while (args.offsets[u0 + 1] <= r_begin) ++u0;
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
        while (args.offsets[c.u + 1] - r_begin <= (int64_t)c.row) ++c.u;
        c.end = user_end(c.u);
      }
    }
  };

  // ---- LDS DMA of the tile at cursor c into ring slot q: block j = wj + s WJ
  // (RPI rows) lands at slot + 1024 j; lane i holds row j RPI + i / CH, LDS
  // chunk i % CH = global chunk (i % CH) ^ sw(row).  Rows past the piece read
  // its last row; past the list every lane reads row c.end - 1 (in bounds).
  auto issue_tile = [&](const Cursor& c, int q) {
    const int last = c.end - 1 - c.row;
    const int64_t b0 = r_begin + (last < 0 ? c.end - 1 : c.row);
    const int lim = last < 0 ? 0 : (last < NT ? last : NT - 1);
#pragma unroll
    for (int s = 0; s < NIW; ++s) {
      const int j = wj + s * WJ;
      if (NI % WJ == 0 || j < NI) {
        const int r = j * RPI + lane / CH;
        const int rr = r < lim ? r : lim;
        dma16(X + b0 * D, (uint32_t)(rr * D + 8 * ((lane % CH) ^ chunk_sw<D>(r))) * 2u,
              lds0 + (uint32_t)(q * TILE_BYTES + 1024 * j));
      }
    }
  };
  // wait until this wave's DMA blocks are done but those of the n most recent tiles
  auto wait_tiles = [&](auto n_) {
    constexpr int n = decltype(n_)::value;
    if constexpr (NI % WJ == 0) {
      wait_vm<(NI / WJ) * n>();
    } else {
      if (wj < NI % WJ) wait_vm<(NI / WJ + 1) * n>();
      else wait_vm<(NI / WJ) * n>();
    }
  };

  // ---- this wave's rows of M (shared) and G (per user) as B fragments
  bf16x8 mreg[JB][CS], greg[JB][CS];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) mreg[jb][cs] = frag_c<D>(M + (int64_t)(jbase + 16 * jb + l16) * D, cs, g);
  int g_user = -1;
  auto ensure_g = [&](int u) {
    u = __builtin_amdgcn_readfirstlane(u);  // uniform: a branch, not a masked block in every step
    if (u == g_user) return;
    g_user = u;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      const int j = jg + 16 * jb + l16;
      const float* grow = args.G + ((int64_t)u * k + (j < k ? j : 0)) * D;
      const float keep = j < k ? 1.f : 0.f;  // padding prototypes get zero rows
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(grow + 32 * cs + 8 * g) * keep;
        const f32x4 b = *reinterpret_cast<const f32x4*>(grow + 32 * cs + 8 * g + 4) * keep;
        typedef float f32x8 __attribute__((ext_vector_type(8)));
        const f32x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
        greg[jb][cs] = __builtin_convertvector(ab, bf16x8);
      }
    }
  };

  // affinity-layout fragment reads (rows 16 ib + l16, chunk 4 cs + g)
  uint32_t aoff[CS];
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) aoff[cs] = (uint32_t)(2 * (l16 * D + 8 * ((4 * cs + g) ^ chunk_sw<D>(l16))));
  // transposing reads for the aggregation (see sa_stream.hpp)
  const uint32_t trb = (uint32_t)(2 * ((4 * g + (l16 >> 2)) * D + 8 * (((l16 >> 1) & 1) ^ chunk_sw<D>(4 * g + (l16 >> 2))) +
                                       4 * (l16 & 1)));
  // lane (g, l16) finishes row my_row of a tile; its 16-lane DPP row holds every lane that needs it
  const int my_ib = (l16 >> 2) & 1, my_r = l16 & 3;
  const int my_row = 16 * my_ib + 4 * g + my_r;
  // row whose 16-lane totals rows4_sum_scatter leaves in this lane (per ib)
  const int sc_r = 2 * (l16 >> 3) + ((l16 >> 2) & 1);

  // s' and dA of the tile in ring slot q for this wave's prototypes
  // (s[ib][jb][r]: row 16 ib + 4 g + r, prototype 16 jb + l16)
  f32x4 s[RB][JB], da[RB][JB];
  auto affinity = [&](int q) {
    const uint32_t slot = lds0 + (uint32_t)(q * TILE_BYTES);
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
      bf16x8 xa[RB];
#pragma unroll
      for (int ib = 0; ib < RB; ++ib) xa[ib] = lds_b128(slot + aoff[cs] + (uint32_t)(2 * 16 * ib * D));
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int ib = 0; ib < RB; ++ib) {
          const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
          s[ib][jb] = MF::run(xa[ib], mreg[jb][cs], cs == 0 ? z : s[ib][jb]);
          da[ib][jb] = MF::run(xa[ib], greg[jb][cs], cs == 0 ? z : da[ib][jb]);
        }
    }
    if constexpr (PAD) {
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        const bool ok = jg + 16 * jb + l16 < k;
#pragma unroll
        for (int ib = 0; ib < RB; ++ib)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            s[ib][jb][r] = ok ? s[ib][jb][r] : -INFINITY;
            da[ib][jb][r] = ok ? da[ib][jb][r] : 0.f;
          }
      }
    }
  };
  // per-wave row statistics of the scores in s, da: m_w, sum 2^(s' - m_w),
  // sum 2^(s' - m_w) dA into xs[par]
  // Unshifted first: 2^s' needs no row maximum while a row's sum over the
  // wave's prototypes stays within [2^-100, 2^100]; a wave that sees a row
  // outside it (huge scores, or all of its prototypes far below) redoes that
  // row block with its own row maxima m_w.  The merge takes any mix of shifts.
  const bool real_protos = jg < k;  // wave-uniform: false for a wave of padding prototypes only
  auto row_stats = [&](int par) {
#pragma unroll
    for (int ib = 0; ib < RB; ++ib) {
      float zm = 0.f, zl = 0.f, zc = 0.f;
      if (real_protos) {
        float pl[4], pc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pl[r] = 0.f;
          pc[r] = 0.f;
#pragma unroll
          for (int jb = 0; jb < JB; ++jb) {
            const float e = fast_exp2(s[ib][jb][r]);
            pl[r] += e;
            pc[r] += e * da[ib][jb][r];
          }
        }
        zl = rows4_sum_scatter(pl, l16);
        zc = rows4_sum_scatter(pc, l16);
        if (args.force_shift ||
            __builtin_amdgcn_ballot_w64(!(zl >= 0x1p-100f && zl <= 0x1p100f) || !(fabsf(zc) <= 0x1p120f)) != 0) {
          float mw[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float m = s[ib][0][r];
#pragma unroll
            for (int jb = 1; jb < JB; ++jb) m = fmaxf(m, s[ib][jb][r]);
            mw[r] = row16_max(m);
            pl[r] = 0.f;
            pc[r] = 0.f;
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
              const float e = fast_exp2(s[ib][jb][r] - mw[r]);
              pl[r] += e;
              pc[r] += e * da[ib][jb][r];
            }
          }
          zl = rows4_sum_scatter(pl, l16);
          zc = rows4_sum_scatter(pc, l16);
          zm = sc_r == 0 ? mw[0] : sc_r == 1 ? mw[1] : sc_r == 2 ? mw[2] : mw[3];
        }
      } else {
        zm = -INFINITY;  // contributes nothing to the merge
      }
      const int trow = 16 * ib + 4 * g + sc_r;
      xs_m[par][trow][wj] = zm;
      xs_l[par][trow][wj] = zl;
      xs_c[par][trow][wj] = zc;
    }
  };

  f32x4 acc[JB][CB];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[jb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  Cursor cc{0, user_end(u0), u0};  // tile t (merge, aggregation)
  Cursor ca = cc;                  // tile t + 1 (affinity)
  Cursor cl = cc;                  // next tile to load
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) {
    issue_tile(cl, p);
    cursor_next(cl);
  }
  wait_tiles(std::integral_constant<int, NS - 2>{});  // tile 0
  __syncthreads();
  ensure_g(ca.u);
  affinity(0);
  if (phase != 2) row_stats(0);
  cursor_next(ca);
  wait_tiles(std::integral_constant<int, NS - 3>{});  // tile 1
  __syncthreads();

  int t = 0;
  while (cc.row < nrel) {
    issue_tile(cl, (t + NS - 1) % NS);  // the slot of tile t - 1
    cursor_next(cl);
    const int par = t & 1;
    const bool valid = my_row < cc.end - cc.row;
    const int64_t grow = r_begin + cc.row + my_row;  // global row of my_row
    float lse, c;
    if (phase == 2) {
      // the merged statistics of all blocks (the lanes of a row read the same 8 bytes)
      const float* st = args.stats + (valid ? grow * 4 : 0);
      lse = st[0];
      c = st[1];
    } else {
      // merge the waves for row my_row of tile t
      float m = xs_m[par][my_row][0];
#pragma unroll
      for (int w = 1; w < WJ; ++w) m = fmaxf(m, xs_m[par][my_row][w]);
      float l = 0.f;
      c = 0.f;
#pragma unroll
      for (int w = 0; w < WJ; ++w) {
        const float f = fast_exp2(xs_m[par][my_row][w] - m);  // 0 for a wave without real prototypes
        l += xs_l[par][my_row][w] * f;
        c += xs_c[par][my_row][w] * f;
      }
      if (phase == 1) {
        // this block's share: (m, l, sum over its prototypes of 2^(s' - m) dA)
        if (valid && wj == 0 && l16 < 8)
          *reinterpret_cast<f32x4*>(args.stats + ((int64_t)blk * rows + grow) * 4) = f32x4{m, l, c, 0.f};
      } else {
        c *= 1.f / l;
        // log-sum-exp of the row in log2 units: A = 2^(s' - lse)
        lse = m + __builtin_amdgcn_logf(l);
        if (valid && wj == 0 && l16 < 8)
          *reinterpret_cast<f32x4*>(args.stats + grow * 4) = f32x4{lse, c, 0.f, 0.f};
      }
    }
    if (phase != 1) {
    if (!valid) lse = INFINITY;  // rows past the piece add nothing

    // dS of this wave's prototypes as bf16 weights of the aggregation
    // (computed in float first and converted in element order, so that
    // consecutive pairs become single packed conversions)
    float dsv[JB][8];
#pragma unroll
    for (int ib = 0; ib < RB; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float mm, cv;
        switch (4 * ib + r) {
          case 0: mm = row_bcast<0>(lse); cv = row_bcast<0>(c); break;
          case 1: mm = row_bcast<1>(lse); cv = row_bcast<1>(c); break;
          case 2: mm = row_bcast<2>(lse); cv = row_bcast<2>(c); break;
          case 3: mm = row_bcast<3>(lse); cv = row_bcast<3>(c); break;
          case 4: mm = row_bcast<4>(lse); cv = row_bcast<4>(c); break;
          case 5: mm = row_bcast<5>(lse); cv = row_bcast<5>(c); break;
          case 6: mm = row_bcast<6>(lse); cv = row_bcast<6>(c); break;
          default: mm = row_bcast<7>(lse); cv = row_bcast<7>(c); break;
        }
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const float A = fast_exp2(s[ib][jb][r] - mm);
          dsv[jb][4 * ib + r] = A * (da[ib][jb][r] - cv);
        }
      }
    bf16x8 a[JB];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int e = 0; e < 8; ++e) a[jb][e] = (bf16)dsv[jb][e];

    // dQ'[j][:] += sum_i dS_ji x_i (reduction slot (g, e) = row 16 (e / 4) + 4 g + e % 4)
    {
      const uint32_t xp = lds0 + (uint32_t)((t % NS) * TILE_BYTES) + trb;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const uint32_t xc = xp ^ (uint32_t)(32 * cb);
        const u32x2 lo = lds_tr16(xc);
        const u32x2 hi = lds_tr16(xc + (uint32_t)(2 * 16 * D));
        const bf16x8 xb = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) acc[jb][cb] = MF::run(a[jb], xb, acc[jb][cb]);
      }
    }
    }  // phase != 1
    // products and row statistics of tile t + 1
    if (ca.row < nrel) {
      ensure_g(ca.u);
      affinity((t + 1) % NS);
      if (phase != 2) row_stats(par ^ 1);
    }
    cursor_next(cc);
    cursor_next(ca);
    ++t;
    wait_tiles(std::integral_constant<int, NS - 3>{});  // tile t + 1 of the new t, read by its affinity
    __syncthreads();
  }
  wait_vm<0>();  // no DMA outlives the work group

  if (phase == 1) return;  // statistics only
  // ---- one partial per group, lane layout [wj][jb][cb][lane][4]; block b's
  // slots follow the ngroups + 1 slots of block b - 1 (the reduction's layout
  // for one user)
  float* dst = args.partial + ((int64_t)blk * (ngroups + 1) + grp) * (int64_t)(KPAD * D);
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      *reinterpret_cast<f32x4*>(dst + (((wj * JB + jb) * CB + cb) * 64 + lane) * 4) = acc[jb][cb];
}

// ------------------------------------------------------------ pass 2
// Packed chunk c of user u (32 prototypes 32 c ..): four blocks of 32 x D
// bf16, laid out as their LDS reads want them:
//   block 0  M rows, row p at p D, 16-byte chunk h at h ^ sw(p)
//   block 1  G rows, same layout
//   block 2  G^T: row t (column t of G) holds the chunk's prototypes in the
//            order pos = 8 g + e <-> prototype 16 (e / 4) + 4 g + e % 4 (the
//            reduction slots of the dX product), 16-byte chunk g stored at
//            g ^ 2 ((t / 8) % 2) so 32 lanes reading 16 rows hit 32 bank groups
//   block 3  Q'^T, same layout
// Prototypes past k are zero.
template <int D>
__global__ __launch_bounds__(256) void grad_pack_kernel(const bf16* M, const bf16* Qp, const float* G, int users, int k,
                                                        int chunks, bf16* packed) {
  constexpr int BLK = kGradKW * D;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)users * chunks * 4 * BLK;
  if (idx >= total) return;
  const int within = (int)(idx % BLK);
  const int part = (int)((idx / BLK) % 4);
  const int64_t uc = idx / (4 * BLK);
  const int c = (int)(uc % chunks);
  const int u = (int)(uc / chunks);
  bf16 v;
  int pos;
  if (part < 2) {
    const int p = within / D, col = within % D;
    const int j = kGradKW * c + p;
    if (part == 0) v = M[(int64_t)j * D + col];
    else v = (bf16)(j < k ? G[((int64_t)u * k + j) * D + col] : 0.f);
    pos = p * D + 8 * ((col >> 3) ^ chunk_sw<D>(p)) + (col & 7);
  } else {
    const int t = within / kGradKW, pp = within % kGradKW;
    const int gg = pp >> 3, e = pp & 7;
    const int j = kGradKW * c + 16 * (e >> 2) + 4 * gg + (e & 3);
    if (part == 2) v = (bf16)(j < k ? G[((int64_t)u * k + j) * D + t] : 0.f);
    else v = j < k ? Qp[(int64_t)j * D + t] : (bf16)0.f;
    pos = t * kGradKW + 8 * (gg ^ (2 * ((t >> 3) & 1))) + e;
  }
  packed[(uc * 4 + part) * BLK + pos] = v;
}

template <int D, int W2, bool PAD>
__global__ __launch_bounds__(64 * W2) void grad_dx_kernel(GradDxArgs args) {
  constexpr int KW = kGradKW, NT = 32 * W2, CS = D / 32, DB = D / 16;
  constexpr int BLK = KW * D * 2;        // bytes of one block of a chunk
  constexpr int CHUNK = 4 * BLK;
  constexpr int CPS = 2;                 // chunks per step (the prototype count is a multiple of 64)
  constexpr int NBLK = CPS * CHUNK / 1024;  // DMA blocks per step
  static_assert(NBLK % W2 == 0, "DMA blocks split evenly over the waves");
  constexpr int BPW = NBLK / W2;
  using MF = Mfma<bf16>;

  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * CPS * CHUNK];
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) unsigned char*)lds;

  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rw = 32 * wave;
  const int k = args.k, chunks = args.chunks;
  const bf16* const X = static_cast<const bf16*>(args.X);
  const unsigned char* const packed = static_cast<const unsigned char*>(args.packed);

  const int64_t rows = args.rows, ngroups = gridDim.x, grp = blockIdx.x;
  const int64_t r_begin = grp * rows / ngroups, r_end = (grp + 1) * rows / ngroups;
  if (r_begin >= r_end) return;

  struct Cursor {
    int64_t row, end;
    int u;
  };
  int u0 = 0;
  while (args.offsets[u0 + 1] <= r_begin) ++u0;
  auto cursor_next = [&](Cursor& c) {
    c.row += NT;
    if (c.row >= c.end) {
      c.row = c.end;
      if (c.row < r_end) {
        ++c.u;
        while (args.offsets[c.u + 1] <= c.row) ++c.u;
        c.end = min(r_end, args.offsets[c.u + 1]);
      }
    }
  };

  // LDS DMA of chunks c .. c + CPS - 1 of user u (adjacent in the packed
  // layout) into buffer b: block j = wave + W2 s lands at 1024 j
  auto issue_chunks = [&](int u, int c, int b) {
    const unsigned char* src = packed + ((int64_t)u * chunks + c) * CHUNK;
#pragma unroll
    for (int s = 0; s < BPW; ++s) {
      const int j = wave + W2 * s;
      dma16(src, (uint32_t)(1024 * j + 16 * lane), lds0 + (uint32_t)(b * CPS * CHUNK + 1024 * j));
    }
  };

  // fragment offsets inside a buffer
  uint32_t moff[CS];  // M / G block: row 16 jb + l16, chunk 4 cs + g
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) moff[cs] = (uint32_t)(2 * (l16 * D + 8 * ((4 * cs + g) ^ chunk_sw<D>(l16))));
  // transposed blocks: row 16 db + l16, chunk g (swizzle by bit 3 of the row)
  const uint32_t toff = (uint32_t)(2 * (l16 * KW + 8 * (g ^ (2 * ((l16 >> 3) & 1)))));

  Cursor cur{r_begin, min(r_end, args.offsets[u0 + 1]), u0};
  issue_chunks(cur.u, 0, 0);
  wait_vm<0>();
  __syncthreads();
  int q = 0;
  while (cur.row < r_end) {
    Cursor nxt = cur;
    cursor_next(nxt);
    const bool has_next = nxt.row < r_end;
    // this wave's rows: X fragments (B operand of s' = M x, rows along the
    // lanes) and the statistics of rows 16 ib + l16
    const int64_t lim = cur.end - 1 - cur.row;
    const bool busy = rw <= lim;  // the wave has rows in this tile (wave-uniform)
    bf16x8 xr[2][CS];
    float sl[2], sc[2];  // log-sum-exp (log2 units, +inf past the piece) and c of rows 16 ib + l16
    bool valid[2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      const int r = rw + 16 * ib + l16;
      valid[ib] = r <= lim;
      const int64_t row = cur.row + (r <= lim ? r : lim);
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) xr[ib][cs] = frag_c<D>(X + row * D, cs, g);
      const f32x4 st = *reinterpret_cast<const f32x4*>(args.stats + row * 4);
      sl[ib] = valid[ib] ? st[0] : INFINITY;
      sc[ib] = st[1];
    }
    f32x4 acc[2][DB];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[ib][db] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c0 = 0; c0 < chunks; c0 += CPS) {
      if (c0 + CPS < chunks) issue_chunks(cur.u, c0 + CPS, q ^ 1);
      else if (has_next) issue_chunks(nxt.u, 0, q ^ 1);
      if (busy) {
#pragma unroll
      for (int h = 0; h < CPS; ++h) {
      const int c = c0 + h;
      const uint32_t buf = lds0 + (uint32_t)((q * CPS + h) * CHUNK);

      // s'[jb][ib][r] and dA for prototype 16 jb + 4 g + r of the chunk, row 16 ib + l16
      f32x4 s[2][2], da[2][2];
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          const bf16x8 mf = lds_b128(buf + moff[cs] + (uint32_t)(2 * 16 * jb * D));
          const bf16x8 gf = lds_b128(buf + (uint32_t)BLK + moff[cs] + (uint32_t)(2 * 16 * jb * D));
#pragma unroll
          for (int ib = 0; ib < 2; ++ib) {
            const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
            s[jb][ib] = MF::run(mf, xr[ib][cs], cs == 0 ? z : s[jb][ib]);
            da[jb][ib] = MF::run(gf, xr[ib][cs], cs == 0 ? z : da[jb][ib]);
          }
        }
      }
      // A and dS as bf16 B operands of the dX product: slot (g, e) <-> prototype 16 (e / 4) + 4 g + e % 4
      bf16x8 wa[2], wd[2];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int jb = e >> 2, r = e & 3;
          const bool ok = !PAD || KW * c + 16 * jb + 4 * g + r < k;
          const float A = ok ? fast_exp2(s[jb][ib][r] - sl[ib]) : 0.f;
          wa[ib][e] = (bf16)A;
          wd[ib][e] = (bf16)(A * (da[jb][ib][r] - sc[ib]));
        }
      // dX^T[16 db + 4 g + r][row 16 ib + l16] += sum over the chunk of G^T A + Q'^T dS
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 gt = lds_b128(buf + (uint32_t)(2 * BLK) + toff + (uint32_t)(2 * 16 * db * KW));
        const bf16x8 qt = lds_b128(buf + (uint32_t)(3 * BLK) + toff + (uint32_t)(2 * 16 * db * KW));
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
          acc[ib][db] = MF::run(gt, wa[ib], acc[ib][db]);
          acc[ib][db] = MF::run(qt, wd[ib], acc[ib][db]);
        }
      }
      }
      }
      wait_vm<0>();  // the next step's DMA (and this tile's loads) are done
      __syncthreads();
      q ^= 1;
    }
    // this lane holds dX[row 16 ib + l16][16 db + 4 g .. + 3]
    bf16* const dX = static_cast<bf16*>(args.dX);
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      if (!valid[ib]) continue;
      bf16* const orow = dX + (cur.row + rw + 16 * ib + l16) * D + 4 * g;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (bf16)acc[ib][db][r];
        *reinterpret_cast<bf16x4*>(orow + 16 * db) = v;
      }
    }
    cur = nxt;
  }
  wait_vm<0>();
}

// ------------------------------------------------------------ block merge
// Row i's statistics over all prototype blocks from the blocks' (m_b, l_b,
// c_b): m = max m_b, l = sum l_b 2^(m_b - m), c = sum c_b 2^(m_b - m) / l,
// written as (m + log2 l, c).
__global__ __launch_bounds__(256) void grad_merge_kernel(const f32x4* bstats, int64_t rows, int blocks, f32x4* stats) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows) return;
  float m = -INFINITY;
  for (int b = 0; b < blocks; ++b) m = fmaxf(m, bstats[(int64_t)b * rows + i][0]);
  float l = 0.f, c = 0.f;
  for (int b = 0; b < blocks; ++b) {
    const f32x4 v = bstats[(int64_t)b * rows + i];
    const float f = exp2f(v[0] - m);  // 0 for a block of padding prototypes only (m_b = -inf)
    l += v[1] * f;
    c += v[2] * f;
  }
  stats[i] = f32x4{m + log2f(l), c / l, 0.f, 0.f};
}

// ------------------------------------------------------------ small products
// Two independent small products per launch (blockIdx.z picks one), one
// 16 x 16 tile of C per work group.  The inner dimension is staged in LDS 256
// at a time with all loads of a stage in flight at once, so a stage costs one
// memory latency; operands are read with arbitrary strides, so transposed
// views need no copy.
template <bool STAGES>  // false: the inner dimension fits one stage (<= 256)
__global__ __launch_bounds__(256) void small_matmul_kernel(MatmulPair pr) {
  __shared__ float As[16][kInnerStage + 1], Bs[kInnerStage][17];
  const Matmul& p = pr.p[blockIdx.z];
  const int m0 = blockIdx.y * 16, n0 = blockIdx.x * 16;
  if (m0 >= p.rows || n0 >= p.cols) return;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float s0 = 0.f, s1 = 0.f;
  for (int t0 = 0; t0 < (STAGES ? p.inner : 1); t0 += kInnerStage) {
    const int n = STAGES ? (p.inner - t0 < kInnerStage ? p.inner - t0 : kInnerStage) : p.inner;
    // all loads in flight before any store; index arithmetic by shifts only
    // (a runtime division per element costs more than the loads)
    float av[16], bv[kInnerStage / 16];
#pragma unroll
    for (int mm = 0; mm < 16; ++mm) {
      const int tt = threadIdx.x;
      av[mm] = tt < n && m0 + mm < p.rows ? p.A[(m0 + mm) * p.a_rs + (t0 + tt) * p.a_cs] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kInnerStage / 16; ++i) {
      const int e = threadIdx.x + 256 * i, tb = e >> 4, nn = e & 15;
      bv[i] = tb < n && n0 + nn < p.cols ? p.B[(t0 + tb) * p.b_rs + (n0 + nn) * p.b_cs] : 0.f;
    }
    if (STAGES && t0 > 0) __syncthreads();  // the previous stage's reads are done
#pragma unroll
    for (int mm = 0; mm < 16; ++mm)
      if (threadIdx.x < n) As[mm][threadIdx.x] = av[mm];
#pragma unroll
    for (int i = 0; i < kInnerStage / 16; ++i) {
      const int e = threadIdx.x + 256 * i;
      if ((e >> 4) < n) Bs[e >> 4][e & 15] = bv[i];
    }
    __syncthreads();
    int t = 0;
    for (; t + 2 <= n; t += 2) {
      s0 = fmaf(As[ty][t], Bs[t][tx], s0);
      s1 = fmaf(As[ty][t + 1], Bs[t + 1][tx], s1);
    }
    if (t < n) s0 = fmaf(As[ty][t], Bs[t][tx], s0);
  }
  if (m0 + ty < p.rows && n0 + tx < p.cols) p.C[(int64_t)(m0 + ty) * p.cols + n0 + tx] = p.alpha * (s0 + s1);
}

__global__ __launch_bounds__(256) void add_kernel(float* dst, const float* src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] += src[i];
}

// dst[i] = 0 for n floats (a kernel rather than a memset node, so that the call can be captured in a graph)
__global__ __launch_bounds__(256) void zero_kernel(float* dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = 0.f;
}

template <int D, int WJ, bool PAD, int PHASE>
hipError_t stats_ph(const GradStatsArgs& a, int groups, hipStream_t s, hipEvent_t e0, hipEvent_t e1, int* occ) {
  if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, grad_stats_kernel<D, WJ, PAD, PHASE>, 64 * WJ, 0);
  if (e0 || e1)
    hipExtLaunchKernelGGL((grad_stats_kernel<D, WJ, PAD, PHASE>), dim3(groups), dim3(64 * WJ), 0, s, e0, e1, 0, a);
  else
    hipLaunchKernelGGL((grad_stats_kernel<D, WJ, PAD, PHASE>), dim3(groups), dim3(64 * WJ), 0, s, a);
  return hipGetLastError();
}
// the two phases over blocks exist for the eight-wave plan only (k > 256)
template <int D, int WJ, bool PAD>
hipError_t stats_p(const GradStatsArgs& a, int groups, hipStream_t s, hipEvent_t e0, hipEvent_t e1, int* occ) {
  if (occ || a.phase == 0) return stats_ph<D, WJ, PAD, 0>(a, groups, s, e0, e1, occ);
  if constexpr (WJ == 8) {
    if (a.phase == 1) return stats_ph<D, WJ, PAD, 1>(a, groups, s, e0, e1, occ);
    if (a.phase == 2) return stats_ph<D, WJ, PAD, 2>(a, groups, s, e0, e1, occ);
  }
  return hipErrorInvalidValue;
}
// padding prototypes (k below 32 WJ) need their scores masked; the occupancy is that of the padded form
template <int D, int WJ>
hipError_t stats_t(const GradStatsArgs& a, int groups, hipStream_t s, hipEvent_t e0, hipEvent_t e1, int* occ) {
  if (occ || a.k != kGradKW * WJ * (a.phase ? a.blocks : 1)) return stats_p<D, WJ, true>(a, groups, s, e0, e1, occ);
  return stats_p<D, WJ, false>(a, groups, s, e0, e1, occ);
}

template <int D>
hipError_t stats_d(int waves, const GradStatsArgs& a, int groups, hipStream_t s, hipEvent_t e0, hipEvent_t e1,
                   int* occ) {
  switch (waves) {
    case 2: return stats_t<D, 2>(a, groups, s, e0, e1, occ);
    case 4: return stats_t<D, 4>(a, groups, s, e0, e1, occ);
    case 8: return stats_t<D, 8>(a, groups, s, e0, e1, occ);
    default: return hipErrorInvalidValue;
  }
}

constexpr int kDxWaves = 8;

template <int D, bool PAD>
hipError_t dx_p(const GradDxArgs& a, int groups, hipStream_t s, hipEvent_t e0, hipEvent_t e1, int* occ) {
  if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, grad_dx_kernel<D, kDxWaves, PAD>, 64 * kDxWaves, 0);
  if (e0 || e1)
    hipExtLaunchKernelGGL((grad_dx_kernel<D, kDxWaves, PAD>), dim3(groups), dim3(64 * kDxWaves), 0, s, e0, e1, 0, a);
  else
    hipLaunchKernelGGL((grad_dx_kernel<D, kDxWaves, PAD>), dim3(groups), dim3(64 * kDxWaves), 0, s, a);
  return hipGetLastError();
}
// padding prototypes (k below 32 chunks) need their weights masked; the occupancy is that of the padded form
template <int D>
hipError_t dx_t(const GradDxArgs& a, int groups, hipStream_t s, hipEvent_t e0, hipEvent_t e1, int* occ) {
  if (occ || a.k != kGradKW * a.chunks) return dx_p<D, true>(a, groups, s, e0, e1, occ);
  return dx_p<D, false>(a, groups, s, e0, e1, occ);
}

}  // namespace

int grad_stats_waves(int k) {
  if (k < 1) return 0;
  if (k <= 2 * kGradKW) return 2;
  if (k <= 4 * kGradKW) return 4;
  if (k <= 4 * kGradBlock) return 8;  // one block of 256, or up to four walked in two phases
  return 0;
}

hipError_t launch_grad_merge(const float* bstats, int64_t rows, int blocks, float* stats, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(grad_merge_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const f32x4*>(bstats), rows, blocks, reinterpret_cast<f32x4*>(stats));
  return hipGetLastError();
}

hipError_t launch_grad_stats(int d, int waves, const GradStatsArgs& a, int groups, hipStream_t s, hipEvent_t start,
                             hipEvent_t stop) {
  if (d == 128) return stats_d<128>(waves, a, groups, s, start, stop, nullptr);
  if (d == 64) return stats_d<64>(waves, a, groups, s, start, stop, nullptr);
  return hipErrorInvalidValue;
}

hipError_t launch_grad_dx(int d, const GradDxArgs& a, int groups, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  if (d == 128) return dx_t<128>(a, groups, s, start, stop, nullptr);
  if (d == 64) return dx_t<64>(a, groups, s, start, stop, nullptr);
  return hipErrorInvalidValue;
}

hipError_t grad_occupancy(int d, int waves, int* stats_groups, int* dx_groups) {
  static const GradStatsArgs sa_unused{};
  static const GradDxArgs dx_unused{};
  hipError_t e;
  if (d == 128) {
    e = stats_d<128>(waves, sa_unused, 0, nullptr, nullptr, nullptr, stats_groups);
    if (e == hipSuccess) e = dx_t<128>(dx_unused, 0, nullptr, nullptr, nullptr, dx_groups);
  } else if (d == 64) {
    e = stats_d<64>(waves, sa_unused, 0, nullptr, nullptr, nullptr, stats_groups);
    if (e == hipSuccess) e = dx_t<64>(dx_unused, 0, nullptr, nullptr, nullptr, dx_groups);
  } else {
    e = hipErrorInvalidValue;
  }
  return e;
}

hipError_t launch_grad_pack(const void* M, const void* Qp, const float* G, int users, int k, int chunks, int d,
                            void* packed, hipStream_t s) {
  const int64_t total = (int64_t)users * chunks * 4 * kGradKW * d;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (d == 128)
    hipLaunchKernelGGL(grad_pack_kernel<128>, grid, dim3(256), 0, s, (const bf16*)M, (const bf16*)Qp, G, users, k,
                       chunks, (bf16*)packed);
  else if (d == 64)
    hipLaunchKernelGGL(grad_pack_kernel<64>, grid, dim3(256), 0, s, (const bf16*)M, (const bf16*)Qp, G, users, k,
                       chunks, (bf16*)packed);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_small_matmuls(const Matmul& a, const Matmul& b, hipStream_t s) {
  for (const Matmul* p : {&a, &b})
    if (p->inner < 1 || p->rows < 1 || p->cols < 1) return hipErrorInvalidValue;
  const int rows = a.rows > b.rows ? a.rows : b.rows, cols = a.cols > b.cols ? a.cols : b.cols;
  const dim3 grid((unsigned)((cols + 15) / 16), (unsigned)((rows + 15) / 16), 2);
  if (a.inner > kInnerStage || b.inner > kInnerStage)
    hipLaunchKernelGGL(small_matmul_kernel<true>, grid, dim3(256), 0, s, MatmulPair{{a, b}});
  else
    hipLaunchKernelGGL(small_matmul_kernel<false>, grid, dim3(256), 0, s, MatmulPair{{a, b}});
  return hipGetLastError();
}

hipError_t launch_add(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(add_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

hipError_t launch_zero(float* dst, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst, n);
  return hipGetLastError();
}

}  // namespace sa
