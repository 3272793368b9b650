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
template <int D, int WJ>
__global__ __launch_bounds__(64 * WJ) void grad_stats_kernel(GradStatsArgs args) {
  constexpr int KW = kGradKW, JB = KW / 16, RB = 2, NT = 16 * RB, CS = D / 32, CB = D / 16, CH = D / 8;
  constexpr int THREADS = 64 * WJ, KPAD = KW * WJ;
  constexpr int TILE_BYTES = NT * D * 2;
  constexpr int NCH = NT * CH;                          // 16-byte chunks per tile
  constexpr int CPT = (NCH + THREADS - 1) / THREADS;    // per thread
  using MF = Mfma<bf16>;

  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * TILE_BYTES];
  __shared__ float xs_m[NT][WJ], xs_l[NT][WJ], xs_c[NT][WJ];
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) unsigned char*)lds;

  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int wj = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jbase = wj * KW;
  const int k = args.k;
  const bf16* const X = static_cast<const bf16*>(args.X);
  const bf16* const M = static_cast<const bf16*>(args.M);

  const int64_t rows = args.rows, ngroups = gridDim.x, grp = blockIdx.x;
  const int64_t r_begin = grp * rows / ngroups, r_end = (grp + 1) * rows / ngroups;
  if (r_begin >= r_end) return;  // the host launches at most one group per row

  // ---- tiles: pieces of [r_begin, r_end) per user, NT rows each
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

  // ---- X tile staging: chunk i of the tile = row i / CH, chunk i % CH, stored
  // at chunk (i % CH) ^ sw(row) of that LDS row; rows past the piece repeat its last row
  u32x4 pre[CPT];
  auto load_tile = [&](const Cursor& c) {
    const int64_t lim = c.end - 1 - c.row;
#pragma unroll
    for (int s = 0; s < CPT; ++s) {
      const int i = tid + s * THREADS;
      if (NCH % THREADS == 0 || i < NCH) {
        const int r = i / CH;
        const int64_t rr = r < lim ? r : lim;
        pre[s] = *reinterpret_cast<const u32x4*>(X + (c.row + rr) * D + 8 * (i % CH));
      }
    }
  };
  auto store_tile = [&](int q) {
#pragma unroll
    for (int s = 0; s < CPT; ++s) {
      const int i = tid + s * THREADS;
      if (NCH % THREADS == 0 || i < NCH) {
        const int r = i / CH;
        *reinterpret_cast<u32x4*>(lds + q * TILE_BYTES + r * D * 2 + 16 * ((i % CH) ^ chunk_sw<D>(r))) = pre[s];
      }
    }
  };

  // ---- this wave's rows of M (shared) and G (per user) as B fragments
  bf16x8 mreg[JB][CS], greg[JB][CS];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) mreg[jb][cs] = frag_c<D>(M + (int64_t)(jbase + 16 * jb + l16) * D, cs, g);
  int g_user = -1;
  auto load_g = [&](int u) {
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      const int j = jbase + 16 * jb + l16;
      const float* grow = args.G + ((int64_t)u * k + (j < k ? j : 0)) * D;
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(grow + 32 * cs + 8 * g);
        const f32x4 b = *reinterpret_cast<const f32x4*>(grow + 32 * cs + 8 * g + 4);
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = (bf16)(j < k ? a[e] : 0.f);
          v[4 + e] = (bf16)(j < k ? b[e] : 0.f);
        }
        greg[jb][cs] = v;
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

  f32x4 acc[JB][CB];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[jb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // lane (g, l16) finishes row my_row of a tile; its 16-lane DPP row holds every lane that needs it
  const int my_ib = (l16 >> 2) & 1, my_r = l16 & 3;
  const int my_row = 16 * my_ib + 4 * g + my_r;
  // row whose 16-lane totals rows4_sum_scatter leaves in this lane (per ib)
  const int sc_r = 2 * (l16 >> 3) + ((l16 >> 2) & 1);

  Cursor cur{r_begin, min(r_end, args.offsets[u0 + 1]), u0};
  load_tile(cur);
  store_tile(0);
  __syncthreads();
  int q = 0;
  while (cur.row < r_end) {
    Cursor nxt = cur;
    cursor_next(nxt);
    const bool has_next = nxt.row < r_end;
    if (has_next) load_tile(nxt);
    if (cur.u != g_user) {
      load_g(cur.u);
      g_user = cur.u;
    }
    const uint32_t slot = lds0 + (uint32_t)(q * TILE_BYTES);

    // s' and dA of this wave's prototypes: s[ib][jb][r] for row 16 ib + 4 g + r, prototype 16 jb + l16
    f32x4 s[RB][JB], da[RB][JB];
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
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      const bool ok = jbase + 16 * jb + l16 < k;
#pragma unroll
      for (int ib = 0; ib < RB; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[ib][jb][r] = ok ? s[ib][jb][r] : -INFINITY;
          da[ib][jb][r] = ok ? da[ib][jb][r] : 0.f;
        }
    }

    // per row and wave: m_w, sum 2^(s' - m_w), sum 2^(s' - m_w) dA
#pragma unroll
    for (int ib = 0; ib < RB; ++ib) {
      float mw[4], pl[4], pc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float m = s[ib][0][r];
#pragma unroll
        for (int jb = 1; jb < JB; ++jb) m = fmaxf(m, s[ib][jb][r]);
        mw[r] = row16_max(m);
        const float ms = mw[r] == -INFINITY ? 0.f : mw[r];  // a wave of padding prototypes only
        pl[r] = 0.f;
        pc[r] = 0.f;
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const float e = fast_exp2(s[ib][jb][r] - ms);
          pl[r] += e;
          pc[r] += e * da[ib][jb][r];
        }
      }
      const float zl = rows4_sum_scatter(pl, l16);
      const float zc = rows4_sum_scatter(pc, l16);
      const float zm = sc_r == 0 ? mw[0] : sc_r == 1 ? mw[1] : sc_r == 2 ? mw[2] : mw[3];
      const int trow = 16 * ib + 4 * g + sc_r;
      xs_m[trow][wj] = zm;
      xs_l[trow][wj] = zl;
      xs_c[trow][wj] = zc;
    }
    __syncthreads();

    // merge the waves for row my_row
    float m = xs_m[my_row][0];
#pragma unroll
    for (int w = 1; w < WJ; ++w) m = fmaxf(m, xs_m[my_row][w]);
    float l = 0.f, c = 0.f;
#pragma unroll
    for (int w = 0; w < WJ; ++w) {
      const float f = fast_exp2(xs_m[my_row][w] - m);  // 0 for a wave without real prototypes
      l += xs_l[my_row][w] * f;
      c += xs_c[my_row][w] * f;
    }
    float inv = 1.f / l;
    c *= inv;
    const bool valid = (int64_t)my_row < cur.end - cur.row;
    if (!valid) inv = 0.f;  // rows past the piece add nothing
    if (valid && wj == 0 && l16 < 8)
      *reinterpret_cast<f32x4*>(args.stats + (cur.row + my_row) * 4) = f32x4{m, inv, c, 0.f};

    // dS of this wave's prototypes as bf16 weights of the aggregation
    bf16x8 a[JB];
#pragma unroll
    for (int ib = 0; ib < RB; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float mm, ii, cc;
        switch (4 * ib + r) {
          case 0: mm = row_bcast<0>(m); ii = row_bcast<0>(inv); cc = row_bcast<0>(c); break;
          case 1: mm = row_bcast<1>(m); ii = row_bcast<1>(inv); cc = row_bcast<1>(c); break;
          case 2: mm = row_bcast<2>(m); ii = row_bcast<2>(inv); cc = row_bcast<2>(c); break;
          case 3: mm = row_bcast<3>(m); ii = row_bcast<3>(inv); cc = row_bcast<3>(c); break;
          case 4: mm = row_bcast<4>(m); ii = row_bcast<4>(inv); cc = row_bcast<4>(c); break;
          case 5: mm = row_bcast<5>(m); ii = row_bcast<5>(inv); cc = row_bcast<5>(c); break;
          case 6: mm = row_bcast<6>(m); ii = row_bcast<6>(inv); cc = row_bcast<6>(c); break;
          default: mm = row_bcast<7>(m); ii = row_bcast<7>(inv); cc = row_bcast<7>(c); break;
        }
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const float A = fast_exp2(s[ib][jb][r] - mm) * ii;
          a[jb][4 * ib + r] = (bf16)(A * (da[ib][jb][r] - cc));
        }
      }

    // dQ'[j][:] += sum_i dS_ji x_i (reduction slot (g, e) = row 16 (e / 4) + 4 g + e % 4)
    {
      const uint32_t xp = slot + trb;
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
    if (has_next) store_tile(q ^ 1);  // that slot was last read before the exchange barrier
    __syncthreads();
    cur = nxt;
    q ^= 1;
  }

  // ---- one partial per group, lane layout [wj][jb][cb][lane][4]
  float* dst = args.partial + grp * (int64_t)(KPAD * D);
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

template <int D, int W2>
__global__ __launch_bounds__(64 * W2) void grad_dx_kernel(GradDxArgs args) {
  constexpr int KW = kGradKW, NT = 32 * W2, CS = D / 32, DB = D / 16;
  constexpr int BLK = KW * D * 2;        // bytes of one block of a chunk
  constexpr int CHUNK = 4 * BLK;
  constexpr int NBLK = CHUNK / 1024;     // DMA blocks per chunk
  static_assert(NBLK % W2 == 0, "DMA blocks split evenly over the waves");
  constexpr int BPW = NBLK / W2;
  using MF = Mfma<bf16>;

  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * CHUNK];
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

  // LDS DMA of chunk c of user u into buffer b: block j = wave + W2 s lands at 1024 j
  auto issue_chunk = [&](int u, int c, int b) {
    const unsigned char* src = packed + ((int64_t)u * chunks + c) * CHUNK;
#pragma unroll
    for (int s = 0; s < BPW; ++s) {
      const int j = wave + W2 * s;
      dma16(src, (uint32_t)(1024 * j + 16 * lane), lds0 + (uint32_t)(b * CHUNK + 1024 * j));
    }
  };

  // fragment offsets inside a buffer
  uint32_t moff[CS];  // M / G block: row 16 jb + l16, chunk 4 cs + g
#pragma unroll
  for (int cs = 0; cs < CS; ++cs) moff[cs] = (uint32_t)(2 * (l16 * D + 8 * ((4 * cs + g) ^ chunk_sw<D>(l16))));
  // transposed blocks: row 16 db + l16, chunk g (swizzle by bit 3 of the row)
  const uint32_t toff = (uint32_t)(2 * (l16 * KW + 8 * (g ^ (2 * ((l16 >> 3) & 1)))));

  Cursor cur{r_begin, min(r_end, args.offsets[u0 + 1]), u0};
  issue_chunk(cur.u, 0, 0);
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
    bf16x8 xr[2][CS];
    float sm[2], si[2], sc[2];
    bool valid[2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      const int r = rw + 16 * ib + l16;
      valid[ib] = r <= lim;
      const int64_t row = cur.row + (r <= lim ? r : lim);
#pragma unroll
      for (int cs = 0; cs < CS; ++cs) xr[ib][cs] = frag_c<D>(X + row * D, cs, g);
      const f32x4 st = *reinterpret_cast<const f32x4*>(args.stats + row * 4);
      sm[ib] = st[0];
      si[ib] = valid[ib] ? st[1] : 0.f;
      sc[ib] = st[2];
    }
    f32x4 acc[2][DB];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[ib][db] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c = 0; c < chunks; ++c) {
      if (c + 1 < chunks) issue_chunk(cur.u, c + 1, q ^ 1);
      else if (has_next) issue_chunk(nxt.u, 0, q ^ 1);
      const uint32_t buf = lds0 + (uint32_t)(q * CHUNK);

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
          const bool ok = KW * c + 16 * jb + 4 * g + r < k;
          const float A = ok ? fast_exp2(s[jb][ib][r] - sm[ib]) * si[ib] : 0.f;
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
      wait_vm<0>();  // the next chunk's DMA (and this tile's loads) are done
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

// ------------------------------------------------------------ small products
template <typename T>
__device__ __forceinline__ float ld_f32(const T* p, int64_t i) {
  return (float)p[i];
}

template <typename T>
__global__ __launch_bounds__(256) void small_matmul_kernel(const T* A, int64_t a_rs, int64_t a_cs, const T* B,
                                                           int64_t b_rs, int64_t b_cs, int rows, int cols, int inner,
                                                           float alpha, float* C) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)rows * cols) return;
  const int m = (int)(idx / cols), n = (int)(idx % cols);
  float s = 0.f;
  for (int t = 0; t < inner; ++t) s = fmaf(ld_f32(A, m * a_rs + t * a_cs), ld_f32(B, t * b_rs + n * b_cs), s);
  C[idx] = alpha * s;
}

__global__ __launch_bounds__(256) void add_kernel(float* dst, const float* src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] += src[i];
}

template <int D, int WJ>
hipError_t stats_t(const GradStatsArgs& a, int groups, hipStream_t s, hipEvent_t e0, hipEvent_t e1, int* occ) {
  if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, grad_stats_kernel<D, WJ>, 64 * WJ, 0);
  if (e0 || e1)
    hipExtLaunchKernelGGL((grad_stats_kernel<D, WJ>), dim3(groups), dim3(64 * WJ), 0, s, e0, e1, 0, a);
  else
    hipLaunchKernelGGL((grad_stats_kernel<D, WJ>), dim3(groups), dim3(64 * WJ), 0, s, a);
  return hipGetLastError();
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

template <int D>
hipError_t dx_t(const GradDxArgs& a, int groups, hipStream_t s, hipEvent_t e0, hipEvent_t e1, int* occ) {
  if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, grad_dx_kernel<D, kDxWaves>, 64 * kDxWaves, 0);
  if (e0 || e1)
    hipExtLaunchKernelGGL((grad_dx_kernel<D, kDxWaves>), dim3(groups), dim3(64 * kDxWaves), 0, s, e0, e1, 0, a);
  else
    hipLaunchKernelGGL((grad_dx_kernel<D, kDxWaves>), dim3(groups), dim3(64 * kDxWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int grad_stats_waves(int k) {
  if (k < 1) return 0;
  if (k <= 2 * kGradKW) return 2;
  if (k <= 4 * kGradKW) return 4;
  if (k <= 8 * kGradKW) return 8;
  return 0;
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

hipError_t launch_small_matmul(int dtype, const void* A, int64_t a_rs, int64_t a_cs, const void* B, int64_t b_rs,
                               int64_t b_cs, int rows, int cols, int inner, float alpha, float* C, hipStream_t s) {
  const dim3 grid((unsigned)(((int64_t)rows * cols + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(small_matmul_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)A, a_rs, a_cs, (const bf16*)B,
                       b_rs, b_cs, rows, cols, inner, alpha, C);
  else
    hipLaunchKernelGGL(small_matmul_kernel<float>, grid, dim3(256), 0, s, (const float*)A, a_rs, a_cs,
                       (const float*)B, b_rs, b_cs, rows, cols, inner, alpha, C);
  return hipGetLastError();
}

hipError_t launch_add(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(add_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

}  // namespace sa
