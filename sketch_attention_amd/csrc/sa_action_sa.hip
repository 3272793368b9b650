// Action fusion as the prologue of the compression pass (bf16, d = 128, one
// pass over eight waves of 32 prototypes), gfx950.
//
// SequenceO1 close-reading page, section 2.2: the row that enters the
// history matrix is x_i = e_i + FFN([e_i; a_i]); section 2.1: the sketch of
// those rows; section 2.4: one fused pass that writes neither the k x n
// matrices nor, here, X.  Each work group walks the tile list of its rows (the
// pieces of sa_wide.hpp, 64-row tiles cut at user ends) two tiles at a time:
//
//   1. E of the block's two tiles is already in a pair of LDS slots (DMA,
//      issued one block ahead, rows past a piece repeating its last row).
//   2. The FFN (sa_action_ffn.hpp) runs on the slots' rows, a wave per 16
//      rows, z's e part read from the slot and its a part from the action
//      table; the weight chunks stream through two LDS buffers.  x = e + FFN,
//      rounded to bf16, replaces e in the slot.
//   3. The sketch pass of sa_wide.hpp runs on the two tiles: affinity
//      (prototypes along the lanes), max-free exponentials and their row sums
//      through LDS, factors, weights, aggregation into the accumulators that
//      stay in registers across blocks, the partial of a piece written when
//      its last tile is done.  Rows whose totals leave [2^-100, 2^100] send
//      their wave through the exact pass.
//
// Every step forms its values by the same instructions in the same order as
// the standalone action pass followed by the sketch pass (same work split),
// so the two paths agree bit for bit.  The phases do not overlap within a
// work group: the FFN's registers and the sketch's scores are never live
// together, which is what lets both fit beside the accumulators and the
// folded matrix (two waves per SIMD).
#include <hip/hip_runtime.h>

#include "sa_action.h"
#include "sa_action_ffn.hpp"
#include "sa_wide.hpp"

namespace sa {

namespace {

template <int KP, bool PAD>
__global__ __launch_bounds__(512) void action_sa_kernel(ActSaArgs aa) {
  constexpr int D = 128, KW = 32, WJ = 8, NW = 8, NT = 64, KC = D / 16, CBK = D / 32;
  constexpr int CH = D / 8;                       // 16-byte chunks per row
  constexpr int SLOT_BYTES = NT * D * 2;          // one tile
  constexpr int NI = SLOT_BYTES / 1024;           // 1 KB DMA blocks per tile
  constexpr int NIW = NI / NW;                    // per wave
  constexpr int RPI = 1024 / (2 * D);             // rows per DMA block
  constexpr int KPAD = KW * WJ;
  constexpr int KS = KP / 32, KE = D / 32, CB = D / 16;
  using C = ActChunk<D, KP>;
  static_assert(C::CHUNK % 1024 == 0, "whole DMA blocks");
  constexpr int WNBLK = C::CHUNK / 1024;          // DMA blocks per weight chunk
  constexpr int WBPW = (WNBLK + NW - 1) / NW;
  constexpr int NTP = NT + 16;                    // row partial sums as in sa_wide.hpp
  constexpr int OFF_W = 4 * SLOT_BYTES;           // two pairs of tile slots, then two weight buffers
  constexpr int OFF_XL = OFF_W + 2 * C::CHUNK;
  constexpr int XL_BYTES = 2 * (WJ / 4) * NTP * 16;
  constexpr int LDS_BYTES = OFF_XL + XL_BYTES;
  static_assert(NI % NW == 0 && LDS_BYTES <= 160 * 1024, "tile geometry");

  const FusedArgs& args = aa.sa;
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
  const int row_a = 32 * ((lane >> 3) & 1) + 16 * ((lane >> 2) & 1) + 4 * h + (lane & 3);
  const int my_row = row_a + 8 * ((lane >> 4) & 1);

  const bf16* const E = static_cast<const bf16*>(aa.E);
  const bf16* const T = static_cast<const bf16*>(aa.table);
  const unsigned char* const packed = static_cast<const unsigned char*>(aa.packed);
  const bf16* const Mg = static_cast<const bf16*>(args.M);
  const int k = args.k;
  const int chunks = aa.chunks;

  const int64_t rows = args.rows;
  const int64_t ngroups = gridDim.x;
  const int64_t grp = blockIdx.x;
  const int64_t r_begin = grp * rows / ngroups;
  const int64_t r_end = (grp + 1) * rows / ngroups;
  if (r_begin >= r_end) return;
  const OffsetLoads offs = tile_list_loads(args, lane);

  // ---- tile list (cursor rows relative to r_begin), as in sa_wide.hpp
  const int nrel = (int)(r_end - r_begin);
  struct Cursor {
    int row, end, u;
  };
  auto user_end = [&](int u) {
    const int64_t e = args.offsets[u + 1] - r_begin;
    return e < (int64_t)nrel ? (int)e : nrel;
  };
  auto cursor_next = [&](Cursor c) {
    c.row += NT;
    if (c.row >= c.end) {
      c.row = c.end;
      if (c.row < nrel) {
        ++c.u;
        while (c.u < args.users && args.offsets[c.u + 1] - r_begin <= (int64_t)c.row) ++c.u;
        c.end = user_end(c.u);
      }
    }
    return c;
  };
  auto tile_rows = [&](const Cursor& c) {
    const int n = c.end - c.row;
    return n < NT ? n : NT;  // 0 past the list
  };

  // ---- folded matrix: lane l holds M[jbase + l % 32][16 kc + 8 h .. + 7]
  bf16x8 mreg[KC];
  {
    const bf16* const mrow = Mg + (int64_t)(jbase + l32) * D + 8 * h;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) mreg[kc] = *reinterpret_cast<const bf16x8*>(mrow + 16 * kc);
  }

  // ---- LDS DMA of a tile's E rows (layout and clamping of sa_wide.hpp)
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
    const bf16* const base = E + b0 * D;
    const uint32_t slot = slot_of(q);
#pragma unroll
    for (int s = 0; s < NIW; ++s) {
      const int j = wave + s * NW;
      const int rr = dma_row[s] < lim ? dma_row[s] : lim;
      dma16(base, (uint32_t)(rr * D + dma_col[s]) * 2u, slot + 1024u * (uint32_t)j);
    }
  };
  // ---- LDS DMA of weight chunk c into buffer b
  auto issue_w = [&](int c, int b) {
    const unsigned char* const src = packed + (int64_t)c * C::CHUNK;
#pragma unroll
    for (int i = 0; i < WBPW; ++i) {
      const int j = wave + NW * i;
      if (WNBLK % NW == 0 || j < WNBLK)
        dma16(src, (uint32_t)(1024 * j + 16 * lane), lds0 + (uint32_t)(OFF_W + b * C::CHUNK + 1024 * j));
    }
  };

  Cursor c0;
  int ntot;
  {
    const TileList tl = tile_list(args, offs, r_begin, r_end, NT, lane);
    ntot = tl.ntot;
    const int64_t e0 = tl.first_end - r_begin;
    c0 = Cursor{0, e0 < (int64_t)nrel ? (int)e0 : nrel, tl.u_first};
  }
  Cursor c1 = cursor_next(c0);

  // ---- FFN rows of this wave: tile ft = wave / 4 of the block, rows 16 (wave % 4) + l16 of it
  const int ft = wave >> 2;
  const int frow = 16 * (wave & 3) + s16;
  const FfnOffsets<D, KP> fo = ffn_offsets<D, KP>(s16, g16);
  // action id of this lane's FFN row (clamped into the tile like the E rows)
  auto load_id = [&](const Cursor& c) {
    const int n = tile_rows(c);
    if (n <= 0) return 0;
    const int r = frow < n ? frow : n - 1;
    return aa.actions[r_begin + c.row + r];
  };
  int id_next = load_id(ft ? c1 : c0);

  issue_tile(c0, 0);
  issue_tile(c1, 1);
  issue_w(0, 0);

  // ---- sketch-pass pieces, as in sa_wide.hpp (see there for the layouts)
  uint32_t aoff[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) aoff[kc] = (uint32_t)(2 * (l32 * D + 8 * ((2 * kc + h) ^ chunk_sw32(l32))));
  auto affinity = [&](f32x16 (&s)[2], uint32_t xs) {
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
  // exponentials and the reduce-scatter of their row sums; the lane's partial of row my_row goes to LDS
  auto softmax_all = [&](f32x16 (&s)[2], int par) {
    float part[2][4];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          s[f][4 * sl + p] = fast_exp2(s[f][4 * sl + p]);
          s[f][8 + 4 * sl + p] = fast_exp2(s[f][8 + 4 * sl + p]);
        }
      float x0[4], x1[4], y0[4], y1[4], o0[4], o1[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        x0[p] = s[0][4 * sl + p];
        y0[p] = s[1][4 * sl + p];
        x1[p] = s[0][8 + 4 * sl + p];
        y1[p] = s[1][8 + 4 * sl + p];
      }
      fold_bit3(o0, x0, y0);
      fold_bit3(o1, x1, y1);
      fold_bit2(part[sl], o0, o1);
    }
    float r3[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) r3[p] = fold_bit4(part[0][p], part[1][p]);
    const bool c1b = (lane & 2) != 0, c0b = (lane & 1) != 0;
    float r4[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float keep = c1b ? r3[2 + e] : r3[e], send = c1b ? r3[e] : r3[2 + e];
      r4[e] = keep + dpp_f32<0x4E>(send);
    }
    const float keep = c0b ? r4[1] : r4[0], send = c0b ? r4[0] : r4[1];
    xl[xl_at(par, my_row, wj)] = keep + dpp_f32<0xB1>(send);
  };
  // factors 1 / sum_w l_w of rows row_a and row_a + 8; `bad` when a total left the unshifted range
  auto combine = [&](int par, float (&fr)[2], bool& bad) {
    bool out = false;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      f32x4 v[WJ / 4];
#pragma unroll
      for (int w = 0; w < WJ; w += 4) v[w / 4] = *reinterpret_cast<const f32x4*>(xl + xl_at(par, row_a + 8 * r, w));
      f32x4 a = v[0];
#pragma unroll
      for (int w = 1; w < WJ / 4; ++w) a += v[w];
      const float lr = (a[0] + a[1]) + (a[2] + a[3]);
      out |= !(lr >= 0x1p-100f && lr <= 0x1p100f);
      fr[r] = __builtin_amdgcn_rcpf(lr);
    }
    bad = __builtin_amdgcn_ballot_w64(out) != 0;
  };
  // exact pass of one wave: running maximum and shifted sum over all prototypes, then 2^(s' - lse)
  auto exact_wave = [&](f32x16 (&s)[2], float (&fr)[2], uint32_t xs) {
    float lse[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      float m = -INFINITY, ls = 0.f;
#pragma unroll 1
      for (int w = 0; w < WJ; ++w) {
        const bf16* const mrow = Mg + (int64_t)(w * KW + l32) * D + 8 * h;
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
        if (mn != -INFINITY) {
          float t = 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) t += fast_exp2(a[v] - mn);
          ls = ls * fast_exp2(m - mn) + pair32_sum(t);
          m = mn;
        }
      }
      lse[f] = m + __log2f(ls);
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
  auto weights_rs = [&](bf16x8 (&a)[4], const f32x16 (&s)[2], const float (&fr)[2], int rs) {
    const int f = rs >> 1, o = 8 * (rs & 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[rs][e] = (bf16)(s[f][o + e] * bcast16(fr[e >> 2], 8 * f + 4 * (rs & 1) + (e & 3)));
  };
  uint32_t xb[2][2];
#pragma unroll
  for (int qp = 0; qp < 2; ++qp)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = 16 * qp + 4 * h + (s16 >> 2) + 8 * rr;
      const int cc = 2 * (g16 & 1) + ((s16 & 3) >> 1);
      xb[qp][rr] = (uint32_t)(row * 256 + 16 * (cc ^ chunk_sw32(row)) + 8 * (s16 & 1));
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
  auto aggregate = [&](f32x16 (&acc)[CBK], const bf16x8 (&a)[4], uint32_t xs) {
    bf16x8 B[2][CBK];
    agg_load(0, B[0], xs);
#pragma unroll
    for (int q = 0; q < NT / 16; ++q) {
      if (q + 1 < NT / 16) agg_load(q + 1, B[(q + 1) & 1], xs);
#pragma unroll
      for (int cb = 0; cb < CBK; ++cb) acc[cb] = mfma32(a[q], B[q & 1][cb], acc[cb]);
    }
  };
  auto flush = [&](f32x16 (&acc)[CBK], int u) {
    float* dst = args.partial + (grp + u) * (int64_t)(KPAD * D);
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
  // factors, weights, aggregation and (at a piece's end) the flush of one tile
  auto finish_tile = [&](f32x16 (&acc)[CBK], f32x16 (&s)[2], int par, const Cursor& c, uint32_t xs) {
    auto row_ok = [&](int row) { return row < c.end - c.row; };
    float fr[2];
    bool bad;
    combine(par, fr, bad);
    fr[0] = row_ok(row_a) ? fr[0] : 0.f;
    fr[1] = row_ok(row_a + 8) ? fr[1] : 0.f;
    if (bad) {
      exact_wave(s, fr, xs);
      fr[0] = row_ok(row_a) ? 1.f : 0.f;
      fr[1] = row_ok(row_a + 8) ? 1.f : 0.f;
    }
    bf16x8 a[4];
#pragma unroll
    for (int rs = 0; rs < 4; ++rs) weights_rs(a, s, fr, rs);
    aggregate(acc, a, xs);
    if (c.row + NT >= c.end) flush(acc, c.u);
  };

  f32x16 acc[CBK];
#pragma unroll
  for (int cb = 0; cb < CBK; ++cb) acc[cb] = f32x16{};

  wait_vm<0>();
  __syncthreads();
  int wb = 0;  // weight buffer of the next chunk
  for (int t = 0; t < ntot; t += 2) {
    const int pr = 2 * ((t >> 1) & 1);  // the block's slot pair
    const bool have1 = t + 1 < ntot;
    const Cursor c2 = cursor_next(c1), c3 = cursor_next(c2);
    const bool more = t + 2 < ntot;
    if (more) {
      issue_tile(c2, 2 - pr);
      issue_tile(c3, 3 - pr);
    }

    // ---- 2. FFN of the block's rows; x = e + FFN replaces e in the slot
    const bool busy = ft == 0 || have1;  // wave-uniform
    const uint32_t fslot = slot_of(pr + ft);
    uint32_t zaddr[KE];
#pragma unroll
    for (int ks = 0; ks < KE; ++ks)
      zaddr[ks] = fslot + (uint32_t)(frow * 256 + 16 * ((4 * ks + g16) ^ chunk_sw32(frow)));
    bf16x8 zf[1][KS];
    {
      int act = id_next;
      act = act < 0 ? 0 : (act >= aa.n_actions ? aa.n_actions - 1 : act);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int k0 = 32 * ks + 8 * g16;
        if (ks < KE) {
          zf[0][ks] = lds_b128(zaddr[ks]);
        } else if (k0 < D + aa.d_a) {
          zf[0][ks] = *reinterpret_cast<const bf16x8*>(T + (int64_t)act * aa.d_a + (k0 - D));
        } else {
          zf[0][ks] = bf16x8{};
        }
      }
    }
    if (more) id_next = load_id(ft ? c3 : c2);
    f32x4 facc[1][CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) facc[0][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < chunks; ++c) {
      if (c + 1 < chunks) issue_w(c + 1, wb ^ 1);
      else if (more) issue_w(0, wb ^ 1);
      if (busy) ffn_chunk<D, KP, 1>(lds0 + (uint32_t)(OFF_W + wb * C::CHUNK), fo, zf, facc);
      wait_vm<0>();
      __syncthreads();
      wb ^= 1;
    }
    if (busy) {
#pragma unroll
      for (int ks = 0; ks < KE; ++ks)
        *(__attribute__((address_space(3))) bf16x8*)(size_t)zaddr[ks] = ffn_residual<D, KP, 1>(zf, facc, 0, ks);
    }
    __syncthreads();

    // ---- 3. the sketch pass on the block's tiles, one at a time (one tile's
    // scores live at once)
#pragma unroll 1
    for (int i = 0; i < (have1 ? 2 : 1); ++i) {
      f32x16 S[2];
      const uint32_t xs = slot_of(pr + i);
      affinity(S, xs);
      softmax_all(S, i);
      __syncthreads();
      finish_tile(acc, S, i, i ? c1 : c0, xs);
    }
    __syncthreads();  // the slot pair and the row sums are free again
    c0 = c2;
    c1 = c3;
  }
  wait_vm<0>();  // no DMA outlives the work group
}

template <int KP, bool PAD>
hipError_t launch_t(const ActSaArgs& a, const Launch& l, int* occ) {
  if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, action_sa_kernel<KP, PAD>, 512, 0);
  if (l.start || l.stop)
    hipExtLaunchKernelGGL((action_sa_kernel<KP, PAD>), dim3(l.groups), dim3(512), 0, l.stream, l.start, l.stop, 0, a);
  else
    hipLaunchKernelGGL((action_sa_kernel<KP, PAD>), dim3(l.groups), dim3(512), 0, l.stream, a);
  return hipGetLastError();
}

template <int KP>
hipError_t launch_kp(bool pad, const ActSaArgs& a, const Launch& l, int* occ) {
  return pad ? launch_t<KP, true>(a, l, occ) : launch_t<KP, false>(a, l, occ);
}

}  // namespace

hipError_t launch_action_sa(int kp, const ActSaArgs& a, const Launch& l, int* occ) {
  const bool pad = a.sa.k < 256;
  if (kp == 128) return launch_kp<128>(pad, a, l, occ);
  if (kp == 192) return launch_kp<192>(pad, a, l, occ);
  if (kp == 256) return launch_kp<256>(pad, a, l, occ);
  return hipErrorInvalidValue;
}

}  // namespace sa
