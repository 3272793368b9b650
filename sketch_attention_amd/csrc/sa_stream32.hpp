// Streamed fused pass on 32x32x16 matrix-core products (bf16, d = 128, eight
// waves of 32 prototypes), gfx950.
//
// The operation is that of sa_stream.hpp (SequenceO1 close-reading page,
// section 2.1: s'_ji = M_j . x_i with the folded M, a_ji = 2^s'_ji / sum_j'
// 2^s'_j'i, X~_j += a_ji x_i; section 2.4: one fused, tiled pass that never
// writes the k x n matrices to memory and accepts ragged batches), with the
// same work split across groups, the same LDS-DMA ring of X tiles, the same
// tile list and the same partial-sketch slots.  What differs is the shape of
// the products, chosen from the measured rates of this chip: a 32x32x16 bf16
// product runs at about twice the throughput of a 16x16x32 one.
//
// Layouts (one wave: 32 prototypes j of M, all 64 rows i of a tile, in two
// blocks of 32 rows):
//   affinity   S (32 j x 32 i) = M (32 j x 16 d) . X^T (16 d x 32 i), eight
//              products over d: each lane ends up with one row i (lane % 32)
//              and 16 prototypes (registers), so a row's sum over the wave's
//              prototypes is 15 in-lane additions and one swap of the two
//              half-waves (v_permlane32_swap), and the row factor is a scalar
//              of the lane;
//   weights    a_ji = 2^s'_ji / l_i, rounded to bf16 and written to a
//              per-wave LDS buffer [64 i][32 j] (8-byte units XOR-swizzled
//              by the row), read back transposed (ds_read_b64_tr_b16) as
//              the A operand of the aggregation: lane = prototype, registers
//              = eight rows;
//   aggregation X~ (32 j x 32 c) += A (32 j x 16 i) . X (16 i x 32 c), four
//              column blocks, four row steps; X comes from the tile by the
//              same transposing read with the same row order.
// The reduction slot of a product maps lane half h and element e to row
// 16 q + 8 (e / 4) + 4 h + e % 4 of the tile; both operands use that order.
//
// LDS rows of X are 256 bytes with 16-byte chunks XOR-swizzled by
// chunk_sw32: the affinity's reads (32 rows, one chunk) and the
// aggregation's transposing reads (4 rows, 4 chunks) are then conflict-free
// under the bank model measured on this chip (16-byte reads: 32 lanes over
// 128 banks; 8-byte transposing reads: 32 lanes over 64 banks; stores: 32
// banks, 16 lanes at a time for 8 bytes, 32 for 4 bytes).
//
// Each step (one barrier): DMA of tile t+3; the row sums of tile t from LDS
// (all waves'); the affinity of tile t+1, and in the shadow of its products
// the factors and weights of tile t (to LDS); the aggregation of tile t, and
// in the shadow of its products the exponentials and row sums of tile t+1.
// The operands of each product are read ahead of it (one d-chunk for the
// affinity, one row step for the aggregation).  A row whose sum leaves
// [2^-100, 2^100] sends the wave through an exact pass (a running maximum
// over all prototypes, M from global memory).  Modes (FusedArgs::lse_mode):
// 0 one pass; 1 and 2 the two phases of the pass for more prototypes than
// one work group holds -- phase 1 writes every row's log-sum-exp over one
// block of prototypes, phase 2 takes the row's log-sum-exp over all
// prototypes (merged between the phases) as given, so its weights are
// 2^(s' - L) with no exchange between waves, and aggregates one block.
#pragma once

#include "sa_stream.hpp"

#ifndef SA32_FENCES
#define SA32_FENCES 1
#endif

namespace sa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Chunk swizzle of an LDS row of 128 bf16 (16 chunks of 16 bytes), a function
// of r % 32: 4 ((r % 4) ^ ((r / 4) % 2)) + (r / 8) % 4.  Over 32 consecutive
// rows each parity class takes all 16 values (the affinity's 16-byte reads),
// and over any 4 rows 4m..4m+3 the upper two bits take all four values (the
// transposing reads of 4 rows x 4 chunks).
__device__ __forceinline__ constexpr int chunk_sw32(int r) {
  return 4 * ((r & 3) ^ ((r >> 2) & 1)) + ((r >> 3) & 3);
}

// The two half-waves' values of x, exchanged by v_permlane32_swap: afterwards
// a holds lanes 0..31 of x in both halves and b lanes 32..63, so a + b (or
// max(a, b)) combines every lane with its partner 32 lanes away.  Written as
// assembly with both operands read and written: the compiler's builtin folds
// the two results of a swap of a value with itself into one.  The nop covers
// the wait state the swap needs after a vector write of its operands.
__device__ __forceinline__ void halves_of(float x, float& a, float& b) {
  a = x;
  b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float pair32_sum(float x) {
  float a, b;
  halves_of(x, a, b);
  return a + b;
}
__device__ __forceinline__ float pair32_max(float x) {
  float a, b;
  halves_of(x, a, b);
  return fmaxf(a, b);
}

// f(integral_constant<int, I>) for I = B .. E - 1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <bool PAD, bool PU, int LM>
__global__ __launch_bounds__(512) void sa_stream32_kernel(FusedArgs args) {
  constexpr int D = 128, KW = 32, WJ = 8, NW = 8, NT = 64, KC = D / 16, CBK = D / 32, NS = 4;
  constexpr int CH = D / 8;                       // 16-byte chunks per row
  constexpr int SLOT_BYTES = NT * D * 2;          // one X tile
  constexpr int NI = SLOT_BYTES / 1024;           // 1 KB DMA blocks per tile
  constexpr int NIW = NI / NW;                    // per wave
  constexpr int RPI = 1024 / (2 * D);             // rows per DMA block
  constexpr int KPAD = KW * WJ;
  constexpr int OFF_XL = NS * SLOT_BYTES;         // row partial sums [2 parities][WJ / 4][NT][4]
  constexpr int XL_BYTES = 2 * (WJ / 4) * NT * 16;
  constexpr int OFF_EB = OFF_XL + XL_BYTES;       // per-wave weight buffers [NT][KW] bf16
  constexpr int EB_BYTES = NT * KW * 2;
  constexpr int OFF_L = OFF_EB + NW * EB_BYTES;   // second phase: log-sum-exp ring [NS][NT]
  constexpr int LDS_BYTES = OFF_L + (LM == 2 ? NS * NT * 4 : 0);
  constexpr int DMA_PER_TILE = NIW + (LM == 2 ? 1 : 0);
  static_assert(NI % NW == 0 && LDS_BYTES <= 160 * 1024, "tile geometry");

  __shared__ __attribute__((aligned(1024))) unsigned char lds[LDS_BYTES];
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) unsigned char*)lds;
  auto slot_of = [&](int q) { return lds0 + (uint32_t)(q * SLOT_BYTES); };
  float* const xl = reinterpret_cast<float*>(lds + OFF_XL);
  // the four waves of a quad share a row's 16 bytes; wave w sits at (w % 4) ^ ((row / 8) % 4), so the 32
  // lanes of a 4-byte store (rows r..r+31) reach distinct banks; the reader only adds the four
  auto xl_at = [&](int par, int w, int row) {
    return ((par * (WJ / 4) + w / 4) * NT + row) * 4 + ((w & 3) ^ ((row >> 3) & 3));
  };
  auto xl_quad = [&](int par, int w, int row) { return ((par * (WJ / 4) + w / 4) * NT + row) * 4; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;       // half-wave
  const int g16 = lane >> 4;     // 16-lane group
  const int s16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wj = wave;
  const int jbase = wj * KW;

  const int nblk = LM ? args.blocks : 1;
  const int64_t ngroups = gridDim.x / nblk;
  const GroupBlock gb = group_block(blockIdx.x, gridDim.x, nblk);  // the nblk blocks of a row range on one XCD
  const int blk = LM ? gb.blk : 0;
  const int64_t grp = gb.grp;
  const bf16* const X = static_cast<const bf16*>(args.X);
  const bf16* const Mg = static_cast<const bf16*>(args.M) + (int64_t)blk * KPAD * D;
  const int k = args.k - blk * KPAD;  // real prototypes of this block (may exceed KPAD)

  const int64_t rows = args.rows;
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

  // ---- folded matrix: lane l holds M[jbase + l % 32][16 kc + 8 h .. + 7] (A operand of the affinity)
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
    if constexpr (LM == 2) {
      const int rr = lane < lim ? lane : lim;
      dma4(args.stats + b0, (uint32_t)rr * 4u, lds0 + (uint32_t)(OFF_L + q * NT * 4));
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

  // ---- affinity: s[rb][v] = S'[jbase + 8 (v / 4) + 4 h + v % 4][row 32 rb + l32 of the tile]
  uint32_t aoff[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) aoff[kc] = (uint32_t)(2 * (l32 * D + 8 * ((2 * kc + h) ^ chunk_sw32(l32))));
  auto pad_protos = [&](f32x16 (&s)[2], int j0) {
    if constexpr (PAD) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const bool ok = j0 + 8 * (v >> 2) + 4 * h + (v & 3) < k;
        s[0][v] = ok ? s[0][v] : -INFINITY;
        s[1][v] = ok ? s[1][v] : -INFINITY;
      }
    }
  };
  // fragments are read one d-chunk ahead of their products (scheduling fences
  // keep the compiler from hoisting all sixteen reads at once)
  auto affinity_with = [&](f32x16 (&s)[2], uint32_t xs, auto mfrag, auto hook) {
    bf16x8 x[2][2];
    x[0][0] = lds_b128(aoff[0] + xs);
    x[0][1] = lds_b128(aoff[0] + xs + (uint32_t)(2 * 32 * D));
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if (kc + 1 < KC) {
        x[(kc + 1) & 1][0] = lds_b128(aoff[kc + 1] + xs);
        x[(kc + 1) & 1][1] = lds_b128(aoff[kc + 1] + xs + (uint32_t)(2 * 32 * D));
      }
      const bf16x8 mf = mfrag(kc);
      const f32x16 z = {};
      s[0] = mfma32(mf, x[kc & 1][0], kc == 0 ? z : s[0]);
      s[1] = mfma32(mf, x[kc & 1][1], kc == 0 ? z : s[1]);
      hook(kc);  // independent vector work issued in the products' shadow
      if (SA32_FENCES) __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto no_hook = [](int) {};
  auto affinity = [&](f32x16 (&s)[2], uint32_t xs, auto hook) {
    affinity_with(s, xs, [&](int kc) { return mreg[kc]; }, hook);
    pad_protos(s, jbase);
  };

  // ---- exponentials of a tile in place and this wave's row sums to LDS (or,
  // in the second phase, 2^(s' - L) with L from the tile's LDS slot)
  Cursor cx{};  // tile whose exponentials come next (second phase)
  auto softmax_next = [&](f32x16 (&s)[2], int par, int q) {
    if constexpr (LM == 2) {
      const float* Lq = reinterpret_cast<const float*>(lds + OFF_L) + q * NT;
      const int nv = cx.end - cx.row;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float L = Lq[32 * rb + l32];
        L = 32 * rb + l32 < nv ? L : INFINITY;  // rows past the piece: weight 0
#pragma unroll
        for (int v = 0; v < 16; ++v) s[rb][v] = fast_exp2(s[rb][v] - L);
      }
      cursor_next(cx);
    } else {
      float sum[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float a0 = fast_exp2(s[rb][0]), a1 = fast_exp2(s[rb][1]);
        s[rb][0] = a0;
        s[rb][1] = a1;
#pragma unroll
        for (int v = 2; v < 16; v += 2) {
          const float e0 = fast_exp2(s[rb][v]), e1 = fast_exp2(s[rb][v + 1]);
          s[rb][v] = e0;
          s[rb][v + 1] = e1;
          a0 += e0;
          a1 += e1;
        }
        sum[rb] = pair32_sum(a0 + a1);
      }
      // lane l writes the partial of row 32 h + l32 (the half-waves hold both rows' sums)
      xl[xl_at(par, wj, 32 * h + l32)] = h ? sum[1] : sum[0];
    }
  };

  // the same in eight slices of four products (slice i: row block i / 4,
  // products 4 (i % 4) .. + 3, summed in the order above), so that the
  // pieces can be issued between the products of another tile
  float sm_a[2], sm_sum[2], sm_L = 0.f;
  auto softmax_slice = [&](f32x16 (&s)[2], int i, int par, int q) {
    const int rb = i >> 2, v0 = 4 * (i & 3);
    if constexpr (LM == 2) {
      if ((i & 3) == 0) {
        const float* Lq = reinterpret_cast<const float*>(lds + OFF_L) + q * NT;
        const float L = Lq[32 * rb + l32];
        sm_L = 32 * rb + l32 < cx.end - cx.row ? L : INFINITY;
      }
#pragma unroll
      for (int v = v0; v < v0 + 4; ++v) s[rb][v] = fast_exp2(s[rb][v] - sm_L);
      if (i == 7) cursor_next(cx);
    } else {
      const float e0 = fast_exp2(s[rb][v0]), e1 = fast_exp2(s[rb][v0 + 1]);
      const float e2 = fast_exp2(s[rb][v0 + 2]), e3 = fast_exp2(s[rb][v0 + 3]);
      s[rb][v0] = e0;
      s[rb][v0 + 1] = e1;
      s[rb][v0 + 2] = e2;
      s[rb][v0 + 3] = e3;
      if ((i & 3) == 0) {
        sm_a[0] = e0;
        sm_a[1] = e1;
      } else {
        sm_a[0] += e0;
        sm_a[1] += e1;
      }
      sm_a[0] += e2;
      sm_a[1] += e3;
      if ((i & 3) == 3) sm_sum[rb] = pair32_sum(sm_a[0] + sm_a[1]);
      if (i == 7) xl[xl_at(par, wj, 32 * h + l32)] = h ? sm_sum[1] : sm_sum[0];
    }
  };

  // ---- factors 1 / sum_w l_w of rows 32 rb + l32; `bad` when a total left the range of the unshifted softmax
  // (the reads are issued first and summed later, so other work can cover their latency)
  auto combine_issue = [&](f32x4 (&v)[2][WJ / 4], int par) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int w = 0; w < WJ; w += 4) v[rb][w / 4] = *reinterpret_cast<const f32x4*>(xl + xl_quad(par, w, 32 * rb + l32));
  };
  auto combine_finish = [&](const f32x4 (&v)[2][WJ / 4], float (&f)[2], float (&l)[2], bool& bad) {
    bool out = false;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      f32x4 a = v[rb][0];
#pragma unroll
      for (int q = 1; q < WJ / 4; ++q) a += v[rb][q];
      l[rb] = (a[0] + a[1]) + (a[2] + a[3]);
      out |= !(l[rb] >= 0x1p-100f && l[rb] <= 0x1p100f);
      f[rb] = __builtin_amdgcn_rcpf(l[rb]);
    }
    bad = __builtin_amdgcn_ballot_w64(out) != 0;
  };

  // ---- exact pass of one wave (rare): running maximum and shifted sum of
  // every row over all prototypes of the block, M from global memory; the
  // wave's own scores become 2^(s' - m), f = 1 / l, lse = m + log2 l.  One
  // row block, one prototype block and one d-chunk at a time (not unrolled),
  // so it needs few registers beyond those live in the main loop.
  auto exact_wave = [&](f32x16 (&s)[2], float (&f)[2], float (&lse)[2], uint32_t xs, int u) {
    const bf16* const Mu = PU ? Mg + (int64_t)u * args.m_stride : Mg;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float m = -INFINITY, ls = 0.f;
#pragma unroll 1
      for (int w = 0; w < WJ; ++w) {
        const bf16* const mrow = Mu + (int64_t)(w * KW + l32) * D + 8 * h;
        f32x16 a = {};
#pragma unroll 1
        for (int kc = 0; kc < KC; ++kc) {
          const uint32_t off = (uint32_t)(2 * (l32 * D + 8 * ((2 * kc + h) ^ chunk_sw32(l32))));
          a = mfma32(*reinterpret_cast<const bf16x8*>(mrow + 16 * kc), lds_b128(xs + (uint32_t)(2 * 32 * rb * D) + off),
                     a);
        }
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
        if (w == wj) s[rb] = a;
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) s[rb][v] = fast_exp2(s[rb][v] - m);
      f[rb] = 1.f / ls;
      lse[rb] = m + __log2f(ls);
    }
  };

  // ---- weights of tile t to this wave's LDS buffer: row r, prototypes 8 b + 4 h .. + 3
  // (8-byte unit 2 b + h, swizzled with fz(r) = (r / 2) % 8: the 16 lanes of an 8-byte
  // store, rows of both parities, reach distinct banks, and the transposing reads of 4
  // rows x 8 units stay conflict-free)
  const uint32_t eb = lds0 + (uint32_t)(OFF_EB + wave * EB_BYTES);
  // unit 2 b + h of row r sits at r * 64 + 8 ((2 b + h) ^ fz(r)) = (r * 64 + 8 (h ^ fz(r))) ^ 16 b
  uint32_t wst[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = 32 * rb + l32;
    wst[rb] = eb + (uint32_t)(row * 64 + 8 * (h ^ ((row >> 1) & 7)));
  }
  // part p of four: row block p / 2, prototypes 16 (p % 2) .. + 15
  auto weights_part = [&](const f32x16 (&s)[2], const float (&f)[2], int p) {
    const int rb = p >> 1;
#pragma unroll
    for (int b = 2 * (p & 1); b < 2 * (p & 1) + 2; ++b) {
      bf16x4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = (bf16)(s[rb][4 * b + r] * f[rb]);
      *(lds_u32x2*)(size_t)(wst[rb] ^ (uint32_t)(16 * b)) = __builtin_bit_cast(u32x2, w);
    }
  };
  auto weights_store = [&](const f32x16 (&s)[2], const float (&f)[2]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) weights_part(s, f, p);
  };

  // ---- aggregation of tile t: acc[cb][v] += sum over the tile's rows of
  // a[jbase + 8 (v / 4) + 4 h + v % 4][row] X[row][32 cb + l32]
  // Rows r0 = 16 q + 4 h + s16 / 4 and r1 = r0 + 8 of the product's reduction
  // slots.  Swizzles depend on the row modulo 32 (X) and modulo 16
  // (weights), i.e. on q mod 2 only: rows of q + 2 are 32 rows further, an
  // immediate offset.  X column block cb: chunk 4 cb + c0 at (4 cb + c0) ^
  // sw(row), i.e. the address of block 0 XOR 64 cb.
  uint32_t ea[2][2], xb[2][2];
#pragma unroll
  for (int qp = 0; qp < 2; ++qp)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = 16 * qp + 4 * h + (s16 >> 2) + 8 * rr;
      ea[qp][rr] = eb + (uint32_t)(row * 64 + 8 * ((4 * (g16 & 1) + (s16 & 3)) ^ ((row >> 1) & 7)));
      const int c0 = 2 * (g16 & 1) + ((s16 & 3) >> 1);
      xb[qp][rr] = (uint32_t)(row * 256 + 16 * (c0 ^ chunk_sw32(row)) + 8 * (s16 & 1));
    }
  // operands of row step q are read while the products of step q - 1 run
  auto aggregate = [&](f32x16 (&acc)[CBK], uint32_t xs, auto hook) {
    auto load = [&](int q, bf16x8& A, bf16x8 (&B)[CBK]) {
      const int qp = q & 1;
      const uint32_t qo_e = (uint32_t)((q >> 1) * 32 * 64), qo_x = (uint32_t)((q >> 1) * 32 * 256);
      const u32x2 a0 = lds_tr16(ea[qp][0] + qo_e), a1 = lds_tr16(ea[qp][1] + qo_e);
      A = __builtin_bit_cast(bf16x8, u32x4{a0.x, a0.y, a1.x, a1.y});
#pragma unroll
      for (int cb = 0; cb < CBK; ++cb) {
        const u32x2 b0 = lds_tr16((xb[qp][0] ^ (uint32_t)(64 * cb)) + xs + qo_x);
        const u32x2 b1 = lds_tr16((xb[qp][1] ^ (uint32_t)(64 * cb)) + xs + qo_x);
        B[cb] = __builtin_bit_cast(bf16x8, u32x4{b0.x, b0.y, b1.x, b1.y});
      }
    };
    bf16x8 A[2], B[2][CBK];
    load(0, A[0], B[0]);
#pragma unroll
    for (int q = 0; q < NT / 16; ++q) {
      if (q + 1 < NT / 16) load(q + 1, A[(q + 1) & 1], B[(q + 1) & 1]);
#pragma unroll
      for (int cb = 0; cb < CBK; ++cb) acc[cb] = mfma32(A[q & 1], B[q & 1][cb], acc[cb]);
      hook(q);  // independent vector work issued in the products' shadow
      if (SA32_FENCES) __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- partial of one (group, user) piece: float4 number ((wj CBK + cb) 4 + v / 4) 64 + lane of the slot
  auto flush = [&](f32x16 (&acc)[CBK], int u) {
    float* dst = args.partial + ((int64_t)blk * (ngroups + args.users) + grp + u) * (int64_t)(KPAD * D);
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

  const int64_t e0 = first_end - r_begin;
  Cursor cc{0, e0 < (int64_t)nrel ? (int)e0 : nrel, u_first};  // tile t
  Cursor cl = cc;  // next tile to load
  Cursor ca = cc;  // tile whose affinity comes next
  cx = cc;
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
  softmax_next(S0, 0, 0);
  wait_tiles(std::integral_constant<int, NS - 3>{});  // tile 1
  __syncthreads();

  // Step t (one barrier): DMA of tile t+3; the row sums of tile t from LDS
  // (all waves'); the affinity of tile t+1, and in its shadow the factors and
  // weights of tile t to LDS; the aggregation of tile t, and in its shadow the
  // exponentials and row sums of tile t+1.  Sa holds tile t's exponentials,
  // Sb receives tile t+1's scores.
  auto step = [&](int t, f32x16 (&Sa)[2], f32x16 (&Sb)[2], auto full, auto q0_) {
    const int q0 = q0_;  // a compile-time constant in the unrolled loop, t % NS in the tail
    const int q1 = q0 + 1 < NS ? q0 + 1 : q0 + 1 - NS;
    const int qn = q0 > 0 ? q0 - 1 : NS - 1;
    constexpr bool F = decltype(full)::value;
    issue_tile(cl, qn);
    const bool nxt = F || t + 1 < ntot;
    f32x4 pv[2][WJ / 4];
    if constexpr (LM != 2) combine_issue(pv, t & 1);
    float f[2] = {1.f, 1.f}, l[2], lse[2];
    bool bad = false;
    // factors of tile t once their reads are in (two products later), then
    // its weights in four parts; a wave with a row out of range takes the
    // exact pass after the products instead
    auto factors = [&]() {
      if constexpr (LM != 2) {
        combine_finish(pv, f, l, bad);
        if constexpr (LM == 1) {
          lse[0] = __log2f(l[0]);
          lse[1] = __log2f(l[1]);
        } else {
          f[0] = row_ok(cc, l32) ? f[0] : 0.f;
          f[1] = row_ok(cc, 32 + l32) ? f[1] : 0.f;
        }
      }
      // in the second phase the exponentials already carry the normalisation
    };
    auto shadow_a = [&](int kc) {
      if (kc == 1) factors();
      if constexpr (LM != 1) {
        if (kc >= 2 && kc < 6 && !bad) weights_part(Sa, f, kc - 2);
      }
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
      exact_wave(Sa, f, lse, slot_of(q0), cc.u);
      if constexpr (LM == 0) {
        f[0] = row_ok(cc, l32) ? f[0] : 0.f;
        f[1] = row_ok(cc, 32 + l32) ? f[1] : 0.f;
      }
      if constexpr (LM != 1) weights_store(Sa, f);
    }
    if constexpr (LM == 1) {
      const int row = 32 * h + l32;
      if (wj == 0 && row_ok(cc, row)) args.stats[(int64_t)blk * rows + r_begin + cc.row + row] = h ? lse[1] : lse[0];
      if (nxt) softmax_next(Sb, (t + 1) & 1, q1);
    } else {
      auto shadow_g = [&](int q) {
        if (nxt) {
          softmax_slice(Sb, 2 * q, (t + 1) & 1, q1);
          softmax_slice(Sb, 2 * q + 1, (t + 1) & 1, q1);
        }
      };
      aggregate(acc, slot_of(q0), shadow_g);
      if (cc.row + NT >= cc.end) flush(acc, cc.u);
    }
    cursor_next(cc);
    cursor_next(cl);
    wait_tiles(std::integral_constant<int, NS - 3>{});  // tile t+2
    __syncthreads();
  };
  using Full = std::integral_constant<bool, true>;
  using Tail = std::integral_constant<bool, false>;
  static_assert(NS % 2 == 0, "an unrolled pass over the ring leaves the score buffers where it found them");
  // ring slot of tile t is t % NS: the main loop is unrolled by NS so every
  // slot offset is a compile-time constant; the tail (at most NS steps, which
  // check at run time whether tile t+1 exists) computes it
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

template <bool PAD, bool PU, int LM>
hipError_t launch_stream32_t(const FusedArgs& a, const Launch& l) {
  if (l.start || l.stop)
    hipExtLaunchKernelGGL((sa_stream32_kernel<PAD, PU, LM>), dim3(l.groups), dim3(512), 0, l.stream, l.start, l.stop, 0,
                          a);
  else
    hipLaunchKernelGGL((sa_stream32_kernel<PAD, PU, LM>), dim3(l.groups), dim3(512), 0, l.stream, a);
  return hipGetLastError();
}

template <bool PAD>
hipError_t launch_stream32_pad(const FusedArgs& a, const Launch& l) {
  const bool pu = a.m_stride != 0;
  switch (a.lse_mode) {
    case 0: return pu ? launch_stream32_t<PAD, true, 0>(a, l) : launch_stream32_t<PAD, false, 0>(a, l);
    case 1: return pu ? launch_stream32_t<PAD, true, 1>(a, l) : launch_stream32_t<PAD, false, 1>(a, l);
    case 2: return pu ? launch_stream32_t<PAD, true, 2>(a, l) : launch_stream32_t<PAD, false, 2>(a, l);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
