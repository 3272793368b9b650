// Streamed, software-pipelined fused pass for bf16 inputs on gfx950.
//
// Same operation and work split across groups as the lockstep pass in
// sa_fused.hpp (SequenceO1 close-reading page, section 2.1 for the affinity,
// the prototype-axis softmax and the aggregation; section 2.4 for the fused,
// on-chip shape): s'_ji = M_j . x_i with the folded M, a_ji = 2^s'_ji /
// sum_j' 2^s'_j'i, X~_j += a_ji x_i, float32 partial sketches per (group,
// user) piece reduced by a second kernel.
//
// What changes is the schedule inside a group.  The group walks one list of
// tiles (NT = 32 * WI rows, never crossing a user boundary) over all the
// pieces it owns, and each wave keeps two affinity tiles in flight:
//
//   iteration t  (one barrier at its end)
//     stage tile t+2 from registers into the LDS ring, issue the HBM loads
//       of tile t+2+PF
//     S(t+1) = X(t+1) . M^T          matrix cores (M held in registers)
//     factors of tile t               LDS exchange of row sums, 1/sum
//     A(t) = S(t) * factors -> bf16   VALU
//     acc += A(t) . X(t)              matrix cores
//     S(t+1) <- 2^S(t+1), row sums    VALU + DPP, partial sums to LDS
//     flush acc when tile t ends a piece
//
// so the affinity product of one tile overlaps the normalisation of the
// previous one and the aggregation product overlaps the exponentials of the
// next one, inside one basic block the compiler can interleave.
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
// their weights are finite and they add nothing to the sketch.  A tile whose
// unshifted row sums leave [2^-100, 2^100] in any wave is recomputed with
// the max-shifted softmax (all waves take that branch together).
#pragma once

#include "sa_fused.hpp"

namespace sa {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Four consecutive rows of one column, see the header comment.
__device__ __forceinline__ u32x2 lds_read_tr16(const bf16* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

template <int D, int KW, int WJ, int WI, int PF>
struct StreamGeom {
  static_assert(KW % 16 == 0 && D % 32 == 0 && (PF == 1 || PF == 2), "tile shape");
  static constexpr int NW = WJ * WI;
  static constexpr int THREADS = 64 * NW;
  static constexpr int NT = kRowsPerWave * WI;  // rows per tile
  static constexpr int JB = KW / 16;
  static constexpr int CB = D / 16;
  static constexpr int CS = D / 32;
  static constexpr int KPAD = KW * WJ;
  static constexpr int XRS = D + 16;           // row stride (elements): +32 bytes, conflict-free fragment reads
  static constexpr int XR_ELEMS = NT * XRS;
  static constexpr int NXR = 3;
  static constexpr int CH = D / 8;             // 16-byte chunks per row
  static constexpr int NCH = NT * CH;
  static constexpr int CPT = (NCH + THREADS - 1) / THREADS;  // chunks per thread
  static constexpr int XR_BYTES = NXR * XR_ELEMS * 2;
  static constexpr int XL_BYTES = 2 * NT * WJ * 4;  // row sums, two parities
  static constexpr int XS_BYTES = NT * WJ * 4;      // exact path: maxima / sums
  static constexpr int XF_BYTES = NW * kRowsPerWave * 4;
  static constexpr int FLAG_BYTES = 2 * NW * 4;
  static constexpr int STAGE_BYTES = WI > 1 ? WJ * CB * 64 * 16 : 0;
  static constexpr int OFF_XL = XR_BYTES;
  static constexpr int OFF_XSM = OFF_XL + XL_BYTES;
  static constexpr int OFF_XSL = OFF_XSM + XS_BYTES;
  static constexpr int OFF_XF = OFF_XSL + XS_BYTES;
  static constexpr int OFF_FLAG = OFF_XF + XF_BYTES;
  static constexpr int OFF_STAGE = (OFF_FLAG + FLAG_BYTES + 15) / 16 * 16;
  static constexpr int LDS_BYTES = OFF_STAGE + STAGE_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CDNA4 compute unit");
};

template <int D, int KW, int WJ, int WI, int PF, bool PAD>
__global__ __launch_bounds__(64 * WJ * WI) void sa_stream_kernel(FusedArgs args) {
  using G = StreamGeom<D, KW, WJ, WI, PF>;
  using MF = Mfma<bf16>;
  constexpr int JB = G::JB, CB = G::CB, CS = G::CS, NT = G::NT, NW = G::NW, THREADS = G::THREADS;
  constexpr int XRS = G::XRS;

  __shared__ __attribute__((aligned(16))) unsigned char lds[G::LDS_BYTES];
  bf16* const Xr = reinterpret_cast<bf16*>(lds);
  float* const xl = reinterpret_cast<float*>(lds + G::OFF_XL);    // [2][NT][WJ]
  float* const xsm = reinterpret_cast<float*>(lds + G::OFF_XSM);  // [NT][WJ]
  float* const xsl = reinterpret_cast<float*>(lds + G::OFF_XSL);  // [NT][WJ]
  int* const flags = reinterpret_cast<int*>(lds + G::OFF_FLAG);   // [2][NW]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wj = wave % WJ;
  const int wi = wave / WJ;
  const int rw = wi * kRowsPerWave;
  const int jbase = wj * KW;
  float* const xf = reinterpret_cast<float*>(lds + G::OFF_XF) + wave * kRowsPerWave;  // this wave's row factors
  const bf16* const X = static_cast<const bf16*>(args.X);
  const bf16* const Mg = static_cast<const bf16*>(args.M);
  const int k = args.k;
  const bool wave_has_protos = jbase < k;

  const int64_t rows = args.rows;
  const int64_t ngroups = gridDim.x;
  const int64_t grp = blockIdx.x;
  const int64_t r_begin = grp * rows / ngroups;
  const int64_t r_end = (grp + 1) * rows / ngroups;
  if (r_begin >= r_end) return;

  // ---- the group's tile list: pieces (user segments) of [r_begin, r_end),
  // each cut into tiles of NT rows.
  int u_first;
  {
    int lo = 0, hi = args.users - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (args.offsets[mid] <= r_begin) lo = mid; else hi = mid - 1;
    }
    u_first = lo;
  }
  int ntot = 0;
  {
    int64_t r = r_begin;
    int u = u_first;
    while (r < r_end) {
      const int64_t e = min(r_end, args.offsets[u + 1]);
      ntot += (int)((e - r + NT - 1) / NT);
      r = e;
      ++u;
      while (u < args.users && args.offsets[u + 1] <= r) ++u;
    }
  }
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
  bf16x8 mreg[JB][CS];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) {
    const bf16* mrow = Mg + (int64_t)(jbase + 16 * jb + l16) * D;
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) mreg[jb][cs] = frag_c<D>(mrow, cs, g);
  }

  // ---- staging: thread chunk s covers row (tid + s*THREADS) / CH, 16 bytes
  u32x4 pre[PF][G::CPT];
  auto load_tile = [&](u32x4 (&dst)[G::CPT], const Cursor& c, bool valid) {
    const int64_t left = c.end - c.row;
    const int rows_left = !valid ? 0 : (left < NT ? (int)left : NT);
    const bf16* tile = X + c.row * D;
#pragma unroll
    for (int s = 0; s < G::CPT; ++s) {
      const int ci = tid + s * THREADS;
      const int r = ci / G::CH, ch = ci % G::CH;
      if (G::NCH % THREADS == 0 || ci < G::NCH) {
        if (r < rows_left) {
          dst[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tile + r * D + 8 * ch));
        } else {
          dst[s] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  auto store_tile = [&](const u32x4 (&src)[G::CPT], bf16* xr) {
#pragma unroll
    for (int s = 0; s < G::CPT; ++s) {
      const int ci = tid + s * THREADS;
      const int r = ci / G::CH, ch = ci % G::CH;
      if (G::NCH % THREADS == 0 || ci < G::NCH) *reinterpret_cast<u32x4*>(xr + r * XRS + 8 * ch) = src[s];
    }
  };

  // ---- affinity: s[ib][jb][r] = S'^T[rw + 16 ib + 4 g + r][jbase + 16 jb + l16]
  auto affinity = [&](f32x4 (&s)[2][JB], const bf16* xr) {
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) s[ib][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cs = 0; cs < CS; ++cs) {
      bf16x8 xa[2];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) xa[ib] = frag_c<D>(xr + (rw + 16 * ib + l16) * XRS, cs, g);
#pragma unroll
      for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) s[ib][jb] = MF::run(xa[ib], mreg[jb][cs], s[ib][jb]);
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

  // ---- e = 2^s' in place, this wave's row sums to xl[par], flag to flags[par]
  auto softmax_fast = [&](f32x4 (&s)[2][JB], int par) {
    bool bad = false;
    float* const xlp = xl + par * (NT * WJ);
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
        xlp[trow * WJ + wj] = z;
      }
    }
    const bool wave_bad = __builtin_amdgcn_ballot_w64(bad && wave_has_protos) != 0;
    if (lane == 0) flags[par * NW + wave] = wave_bad ? 1 : 0;
  };

  auto any_flag = [&](int par) {
    int f = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) f |= flags[par * NW + w];
    return __builtin_amdgcn_readfirstlane(f) != 0;
  };

  // ---- factors 1 / sum_w l_w of this wave's 32 rows (lane L < 32 finishes row rw + L)
  auto combine_fast = [&](float (&fac)[2][4], int par) {
    if (lane < kRowsPerWave) {
      const float* p = xl + par * (NT * WJ) + (rw + lane) * WJ;
      float l = p[0];
#pragma unroll
      for (int w = 1; w < WJ; ++w) l += p[w];
      xf[lane] = __builtin_amdgcn_rcpf(l);
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      const f32x4 f = *reinterpret_cast<const f32x4*>(xf + 16 * ib + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) fac[ib][r] = f[r];
    }
  };

  // ---- exact path: recompute the tile's affinity from LDS, shift each row
  // by its maximum over all prototypes, combine the waves' shifted sums.
  auto softmax_exact = [&](f32x4 (&s)[2][JB], const bf16* xr, float (&fac)[2][4]) {
    affinity(s, xr);
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
        fac[ib][r] = m;
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
      }
  };

  // ---- aggregation: acc[jb][cb][r] += sum_i a[jbase+16jb+4g+r][i] X[i][16cb+l16].
  // Reduction slot (g, e) of a lane is tile row rw + 16 (e / 4) + 4 g + e % 4,
  // the rows the affinity layout left in that lane.
  const int tr_off = (rw + 4 * g + (l16 >> 2)) * XRS + 4 * (l16 & 3);
  auto aggregate = [&](f32x4 (&acc)[JB][CB], const f32x4 (&s)[2][JB], const float (&fac)[2][4], const bf16* xr) {
    bf16x8 a[JB];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
      for (int e = 0; e < 8; ++e) a[jb][e] = (bf16)(s[e >> 2][jb][e & 3] * fac[e >> 2][e & 3]);
    const bf16* const xp = xr + tr_off;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const u32x2 lo = lds_read_tr16(xp + 16 * cb);
      const u32x2 hi = lds_read_tr16(xp + 16 * XRS + 16 * cb);
      const bf16x8 xb = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) acc[jb][cb] = MF::run(a[jb], xb, acc[jb][cb]);
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

  // ---- prologue: tiles 0 and 1 into the ring, tiles 2 .. 1+PF into registers,
  // affinity and exponentials of tile 0.
  Cursor cc = cursor_begin();  // tile t (aggregation, flush)
  Cursor cl = cc;              // next tile to load from HBM
  {
    u32x4 tmp[G::CPT];
    load_tile(tmp, cl, 0 < ntot);
    store_tile(tmp, Xr);
    cursor_next(cl);
    load_tile(tmp, cl, 1 < ntot);
    store_tile(tmp, Xr + G::XR_ELEMS);
    cursor_next(cl);
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      load_tile(pre[(2 + p) % PF], cl, 2 + p < ntot);
      cursor_next(cl);
    }
  }
  __syncthreads();
  f32x4 S0[2][JB], S1[2][JB];
  affinity(S0, Xr);
  softmax_fast(S0, 0);
  __syncthreads();

  // ---- main loop, unrolled by two so the two affinity tiles swap roles
  // without register copies.  ring index of tile t: t % 3.
  int q0 = 0;  // t % 3
  auto step = [&](int t, f32x4 (&Sa)[2][JB], f32x4 (&Sb)[2][JB], u32x4 (&pslot)[G::CPT]) {
    const int q1 = q0 == 2 ? 0 : q0 + 1;
    const int q2 = q1 == 2 ? 0 : q1 + 1;
    bf16* const xr_t = Xr + q0 * G::XR_ELEMS;
    bf16* const xr_t1 = Xr + q1 * G::XR_ELEMS;
    bf16* const xr_t2 = Xr + q2 * G::XR_ELEMS;
    const bool has1 = t + 1 < ntot;
    if (t + 2 < ntot) {
      store_tile(pslot, xr_t2);
      load_tile(pslot, cl, t + 2 + PF < ntot);
      cursor_next(cl);
    }
    if (has1) affinity(Sb, xr_t1);
    float fac[2][4];
    combine_fast(fac, t & 1);
    if (any_flag(t & 1)) softmax_exact(Sa, xr_t, fac);
    aggregate(acc, Sa, fac, xr_t);
    if (has1) softmax_fast(Sb, (t + 1) & 1);
    if (cc.row + NT >= cc.end) flush(acc, cc.u);
    cursor_next(cc);
    q0 = q1;
    __syncthreads();
  };
  for (int t = 0; t < ntot; t += 2) {
    step(t, S0, S1, pre[0]);
    if (t + 1 < ntot) step(t + 1, S1, S0, pre[PF - 1]);
  }
}

template <int D, int KW, int WJ, int WI, int PF>
hipError_t run_stream_plan(const Plan& p, const FusedArgs& a, int groups, hipStream_t st, int* occ) {
  constexpr int threads = 64 * WJ * WI;
  if (p.k == p.k_pad) {
    if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, sa_stream_kernel<D, KW, WJ, WI, PF, false>,
                                                                 threads, 0);
    hipLaunchKernelGGL((sa_stream_kernel<D, KW, WJ, WI, PF, false>), dim3(groups), dim3(threads), 0, st, a);
  } else {
    if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, sa_stream_kernel<D, KW, WJ, WI, PF, true>,
                                                                 threads, 0);
    hipLaunchKernelGGL((sa_stream_kernel<D, KW, WJ, WI, PF, true>), dim3(groups), dim3(threads), 0, st, a);
  }
  return hipGetLastError();
}

#define SA_STREAM_PLAN(D_, KW_, WJ_, WI_, PF_)                                                     \
  if (p.kind == 1 && p.kw == KW_ && p.waves_k == WJ_ && p.waves_rows == WI_ && p.prefetch == PF_) \
    return run_stream_plan<D_, KW_, WJ_, WI_, PF_>(p, a, groups, st, occ);

}  // namespace sa
