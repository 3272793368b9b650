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
// Inside a work group.  Four waves; WJ waves split the k_pad prototypes
// (KW each) and WI = 4 / WJ waves split the rows of a tile (32 rows each).
// Per tile of NT = 32 * WI rows:
//   1. the tile is staged from HBM (read once, prefetched one tile ahead into
//      registers) into LDS twice: row-major Xr for the affinity product and
//      transposed Xt for the aggregation product;
//   2. S^T (32 rows x KW prototypes per wave) = Xr . M^T on the matrix cores
//      (16x16x32 bf16 or 16x16x4 f32), M fragments in registers or LDS;
//   3. in the output layout of that product each lane holds one prototype and
//      four rows per 16x16 block, so the prototype-axis max and sum are a
//      16-lane DPP reduction (plus an LDS exchange across the WJ waves);
//   4. the normalised weights are rounded to the operand type in registers
//      and used directly as the A operand of X~ (KW x D) += A (KW x 32) .
//      X (32 x D): the reduction index of that product is the row index, and
//      the rows each lane holds are exactly the rows its operand slot needs,
//      so no LDS round trip is needed for A;
//   5. accumulators stay in registers (float32) for the whole piece.
#pragma once

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

// ------------------------------------------------------ static geometry
template <typename T, int D, int KW, int WJ, int WI, bool MLDS>
struct FusedGeom {
  static_assert(WJ * WI == kWaves, "four waves per work group");
  static_assert(KW % 16 == 0 && D % 32 == 0, "tile shape");
  static_assert(!(MLDS && WI > 1), "LDS-resident M is used only when all waves split the prototypes");
  static constexpr int NT = kRowsPerWave * WI;   // tile rows
  static constexpr int JB = KW / 16;             // 16-prototype blocks per wave
  static constexpr int CB = D / 16;              // 16-column blocks of the output
  static constexpr int CS = D / Mfma<T>::kStep;  // affinity reduction steps
  static constexpr int KPAD = KW * WJ;
  static constexpr int XRS = D + 16 / (int)sizeof(T);  // Xr row stride (elements), +16 bytes
  static constexpr int XTS = NT + 4;                   // Xt row stride (elements)
  static constexpr int MS = D + 8;                     // LDS M row stride (bf16 elements)
  static constexpr int XR_BYTES = NT * XRS * (int)sizeof(T);
  static constexpr int XT_BYTES = D * XTS * (int)sizeof(T);
  static constexpr int RED_BYTES = WJ > 1 ? 2 * WJ * NT * 4 : 0;
  static constexpr int M_BYTES = MLDS ? KPAD * MS * 2 : 0;
  static constexpr int MAIN_BYTES = XR_BYTES + XT_BYTES + RED_BYTES + M_BYTES;
  static constexpr int ACC_BYTES = WI > 1 ? KPAD * D * 4 : 0;
  static constexpr int LDS_BYTES = MAIN_BYTES > ACC_BYTES ? MAIN_BYTES : ACC_BYTES;
  static constexpr int QC = D / 4;                     // 4-column quads per row
  static constexpr int NBLK = (NT / 4) * QC;           // 4x4 blocks per tile
  static constexpr int BPT = (NBLK + kThreads - 1) / kThreads;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CDNA4 compute unit");
};


// ------------------------------------------------------- X tile staging
// One thread moves a 4x4 block (rows 4rq..4rq+3, columns 4cq..4cq+3 of the
// tile) from HBM into registers, then into both LDS layouts.  Consecutive
// threads take consecutive column quads of the same rows, so each global load
// instruction of a wave reads whole rows.
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

template <int D>
__device__ __forceinline__ void quad_load(Quad<bf16>& q, const bf16* X, int64_t row, int64_t row_end, int col) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    q.v[r] = (row + r < row_end) ? *reinterpret_cast<const u32x2*>(X + (row + r) * D + col) : u32x2{0u, 0u};
  }
}

template <int D>
__device__ __forceinline__ void quad_load(Quad<float>& q, const float* X, int64_t row, int64_t row_end, int col) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    q.v[r] = (row + r < row_end) ? *reinterpret_cast<const f32x4*>(X + (row + r) * D + col)
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// xr -> Xr[4rq][4cq] (row stride xrs), xt -> Xt[4cq][4rq] (row stride xts)
__device__ __forceinline__ void quad_store(const Quad<bf16>& q, bf16* xr, int xrs, bf16* xt, int xts) {
#pragma unroll
  for (int r = 0; r < 4; ++r) *reinterpret_cast<u32x2*>(xr + r * xrs) = q.v[r];
  const u32x2 c0 = {(q.v[0].x & 0xFFFFu) | (q.v[1].x << 16), (q.v[2].x & 0xFFFFu) | (q.v[3].x << 16)};
  const u32x2 c1 = {(q.v[0].x >> 16) | (q.v[1].x & 0xFFFF0000u), (q.v[2].x >> 16) | (q.v[3].x & 0xFFFF0000u)};
  const u32x2 c2 = {(q.v[0].y & 0xFFFFu) | (q.v[1].y << 16), (q.v[2].y & 0xFFFFu) | (q.v[3].y << 16)};
  const u32x2 c3 = {(q.v[0].y >> 16) | (q.v[1].y & 0xFFFF0000u), (q.v[2].y >> 16) | (q.v[3].y & 0xFFFF0000u)};
  *reinterpret_cast<u32x2*>(xt + 0 * xts) = c0;
  *reinterpret_cast<u32x2*>(xt + 1 * xts) = c1;
  *reinterpret_cast<u32x2*>(xt + 2 * xts) = c2;
  *reinterpret_cast<u32x2*>(xt + 3 * xts) = c3;
}

__device__ __forceinline__ void quad_store(const Quad<float>& q, float* xr, int xrs, float* xt, int xts) {
#pragma unroll
  for (int r = 0; r < 4; ++r) *reinterpret_cast<f32x4*>(xr + r * xrs) = q.v[r];
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

// -------------------------------------------------------------- kernel
template <typename T, int D, int KW, int WJ, int WI, bool MLDS>
__global__ __launch_bounds__(kThreads) void sa_fused_kernel(FusedArgs args) {
  using G = FusedGeom<T, D, KW, WJ, WI, MLDS>;
  using MF = Mfma<T>;
  using Frag = typename MF::Frag;
  static_assert(!MLDS || sizeof(T) == 2, "LDS-resident M is bf16 only");

  __shared__ __attribute__((aligned(16))) unsigned char lds[G::LDS_BYTES];
  T* Xr = reinterpret_cast<T*>(lds);
  T* Xt = reinterpret_cast<T*>(lds + G::XR_BYTES);
  float* red_m = reinterpret_cast<float*>(lds + G::XR_BYTES + G::XT_BYTES);
  float* red_l = red_m + WJ * G::NT;
  T* Ms = reinterpret_cast<T*>(lds + G::XR_BYTES + G::XT_BYTES + G::RED_BYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wj = wave % WJ;
  const int wi = wave / WJ;
  const int rw = wi * kRowsPerWave;  // first tile row of this wave
  const int jbase = wj * KW;         // first prototype of this wave
  const T* X = static_cast<const T*>(args.X);
  const T* Mg = static_cast<const T*>(args.M);

  const int64_t rows = args.rows;
  const int64_t ngroups = gridDim.x;
  const int64_t grp = blockIdx.x;
  const int64_t r_begin = grp * rows / ngroups;
  const int64_t r_end = (grp + 1) * rows / ngroups;
  if (r_begin >= r_end) return;

  // Folded matrix: this wave's KW rows as B fragments of the affinity product.
  Frag mreg[MLDS ? 1 : G::JB][MLDS ? 1 : G::CS];
  if constexpr (MLDS) {
    constexpr int CH = D / 8;  // 16-byte chunks per row
    for (int idx = tid; idx < G::KPAD * CH; idx += kThreads) {
      const int r = idx / CH, ch = idx % CH;
      *reinterpret_cast<u32x4*>(Ms + r * G::MS + ch * 8) = *reinterpret_cast<const u32x4*>(Mg + r * D + ch * 8);
    }
    // ordered before the first read by the first tile's barriers
  } else {
#pragma unroll
    for (int jb = 0; jb < G::JB; ++jb) {
      const T* mrow = Mg + (int64_t)(jbase + 16 * jb + l16) * D;
#pragma unroll
      for (int cs = 0; cs < G::CS; ++cs) mreg[jb][cs] = frag_c<D>(mrow, cs, g);
    }
  }

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

  const int k = args.k;
  int64_t row = r_begin;
  while (row < r_end) {
    const int64_t seg_end = min(r_end, args.offsets[u + 1]);

    f32x4 acc[G::JB][G::CB];
#pragma unroll
    for (int jb = 0; jb < G::JB; ++jb)
#pragma unroll
      for (int cb = 0; cb < G::CB; ++cb) acc[jb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    Quad<T> pre[G::BPT];
    auto prefetch = [&](int64_t t0) {
#pragma unroll
      for (int s = 0; s < G::BPT; ++s) {
        const int blk = tid + s * kThreads;
        if (G::NBLK % kThreads == 0 || blk < G::NBLK) {
          const int rq = blk / G::QC, cq = blk % G::QC;
          quad_load<D>(pre[s], X, t0 + 4 * rq, seg_end, 4 * cq);
        }
      }
    };
    prefetch(row);

    for (int64_t t0 = row; t0 < seg_end; t0 += G::NT) {
      __syncthreads();  // every wave is done with the previous tile
#pragma unroll
      for (int s = 0; s < G::BPT; ++s) {
        const int blk = tid + s * kThreads;
        if (G::NBLK % kThreads == 0 || blk < G::NBLK) {
          const int rq = blk / G::QC, cq = blk % G::QC;
          quad_store(pre[s], Xr + (4 * rq) * G::XRS + 4 * cq, G::XRS, Xt + (4 * cq) * G::XTS + 4 * rq, G::XTS);
        }
      }
      __syncthreads();
      if (t0 + G::NT < seg_end) prefetch(t0 + G::NT);

      // ---- affinity: s[ib][jb][r] = S'^T[rw + 16 ib + 4 g + r][jbase + 16 jb + l16]
      f32x4 s[2][G::JB];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < G::JB; ++jb) s[ib][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cs = 0; cs < G::CS; ++cs) {
        Frag xa[2];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) xa[ib] = frag_c<D>(Xr + (rw + 16 * ib + l16) * G::XRS, cs, g);
#pragma unroll
        for (int jb = 0; jb < G::JB; ++jb) {
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

      // padded prototypes take no mass
#pragma unroll
      for (int jb = 0; jb < G::JB; ++jb) {
        if (jbase + 16 * jb + 16 > k) {
          const bool ok = jbase + 16 * jb + l16 < k;
#pragma unroll
          for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) s[ib][jb][r] = ok ? s[ib][jb][r] : -INFINITY;
        }
      }

      // ---- softmax over the prototype axis (base 2; M carries log2(e))
      float fac[2][4];
      float mloc[2][4];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float m = s[ib][0][r];
#pragma unroll
          for (int jb = 1; jb < G::JB; ++jb) m = fmaxf(m, s[ib][jb][r]);
          m = row16_max(m);
          const float mu = (m == -INFINITY) ? 0.f : m;  // a wave holding only padding
          float l = 0.f;
#pragma unroll
          for (int jb = 0; jb < G::JB; ++jb) {
            const float e = fast_exp2(s[ib][jb][r] - mu);
            s[ib][jb][r] = e;
            l += e;
          }
          l = row16_sum(l);
          mloc[ib][r] = m;
          fac[ib][r] = l;
        }
      }
      if constexpr (WJ == 1) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
          for (int r = 0; r < 4; ++r) fac[ib][r] = 1.f / fac[ib][r];
      } else {
        if (l16 == 0) {
#pragma unroll
          for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int trow = rw + 16 * ib + 4 * g + r;
              red_m[wj * G::NT + trow] = mloc[ib][r];
              red_l[wj * G::NT + trow] = fac[ib][r];
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
            for (int w = 0; w < WJ; ++w) mx = fmaxf(mx, red_m[w * G::NT + trow]);
            float den = 0.f;
#pragma unroll
            for (int w = 0; w < WJ; ++w) den += red_l[w * G::NT + trow] * fast_exp2(red_m[w * G::NT + trow] - mx);
            fac[ib][r] = fast_exp2(mloc[ib][r] - mx) / den;
          }
      }

      // ---- aggregation: acc[jb][cb][r] += sum_i a[jbase+16jb+4g+r][i] X[i][16cb+l16]
      if constexpr (sizeof(T) == 2) {
        bf16x8 xb[G::CB];
#pragma unroll
        for (int cb = 0; cb < G::CB; ++cb) {
          const T* xt = Xt + (16 * cb + l16) * G::XTS + rw + 4 * g;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(xt);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(xt + 16);
          xb[cb] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
        }
#pragma unroll
        for (int jb = 0; jb < G::JB; ++jb) {
          bf16x8 a;
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = (bf16)(s[e >> 2][jb][e & 3] * fac[e >> 2][e & 3]);
#pragma unroll
          for (int cb = 0; cb < G::CB; ++cb) acc[jb][cb] = MF::run(a, xb[cb], acc[jb][cb]);
        }
      } else {
        f32x4 xb[G::CB][2];
#pragma unroll
        for (int cb = 0; cb < G::CB; ++cb)
#pragma unroll
          for (int ib = 0; ib < 2; ++ib)
            xb[cb][ib] = *reinterpret_cast<const f32x4*>(Xt + (16 * cb + l16) * G::XTS + rw + 16 * ib + 4 * g);
#pragma unroll
        for (int jb = 0; jb < G::JB; ++jb)
#pragma unroll
          for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float a = s[ib][jb][r] * fac[ib][r];
#pragma unroll
              for (int cb = 0; cb < G::CB; ++cb) acc[jb][cb] = MF::run(a, xb[cb][ib][r], acc[jb][cb]);
            }
      }
    }

    // ---- flush this (group, user) piece.  Partial layout per slot:
    // [wj][jb][cb][lane][4] float32, i.e. each lane's accumulator registers in
    // order; the reduction kernel maps it back to (prototype, column).
    if constexpr (WI > 1) {
      float* accbuf = reinterpret_cast<float*>(lds);
      for (int st = WI - 1; st >= 1; --st) {
        __syncthreads();
        if (wi == st) {
#pragma unroll
          for (int jb = 0; jb < G::JB; ++jb)
#pragma unroll
            for (int cb = 0; cb < G::CB; ++cb)
              *reinterpret_cast<f32x4*>(accbuf + (((wj * G::JB + jb) * G::CB + cb) * 64 + lane) * 4) = acc[jb][cb];
        }
        __syncthreads();
        if (wi == st - 1) {
#pragma unroll
          for (int jb = 0; jb < G::JB; ++jb)
#pragma unroll
            for (int cb = 0; cb < G::CB; ++cb)
              acc[jb][cb] += *reinterpret_cast<const f32x4*>(accbuf + (((wj * G::JB + jb) * G::CB + cb) * 64 + lane) * 4);
        }
      }
    }
    if (wi == 0) {
      float* dst = args.partial + (grp + u) * (int64_t)(G::KPAD * D);
#pragma unroll
      for (int jb = 0; jb < G::JB; ++jb)
#pragma unroll
        for (int cb = 0; cb < G::CB; ++cb)
          *reinterpret_cast<f32x4*>(dst + (((wj * G::JB + jb) * G::CB + cb) * 64 + lane) * 4) = acc[jb][cb];
    }

    row = seg_end;
    ++u;
    while (u < args.users && args.offsets[u + 1] <= row) ++u;  // skip empty histories
  }
}

template <typename T, int D, int KW, int WJ, int WI, bool MLDS>
hipError_t launch_fused_t(const FusedArgs& args, int groups, hipStream_t stream) {
  hipLaunchKernelGGL((sa_fused_kernel<T, D, KW, WJ, WI, MLDS>), dim3(groups), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

template <typename T, int D, int KW, int WJ, int WI, bool MLDS>
hipError_t occupancy_t(int* n) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, sa_fused_kernel<T, D, KW, WJ, WI, MLDS>, kThreads, 0);
}

// Plans compiled for one (dtype, d).  occ != nullptr turns the call into an
// occupancy query for that plan.
template <typename T, int D>
hipError_t dispatch_fused(const Plan& p, const FusedArgs& a, int groups, hipStream_t st, int* occ) {
#define SA_PLAN(KW_, WJ_, MLDS_)                                                          \
  if (p.kw == KW_ && p.waves_k == WJ_ && p.m_in_lds == MLDS_)                             \
    return occ ? occupancy_t<T, D, KW_, WJ_, kWaves / WJ_, MLDS_>(occ)                    \
               : launch_fused_t<T, D, KW_, WJ_, kWaves / WJ_, MLDS_>(a, groups, st);
  SA_PLAN(16, 1, 0)
  SA_PLAN(32, 1, 0)
  SA_PLAN(64, 1, 0)
  SA_PLAN(64, 2, 0)
  SA_PLAN(64, 4, 0)
  if constexpr (sizeof(T) == 2) {
    SA_PLAN(128, 4, 1)
    if constexpr (D == 64) {
      SA_PLAN(256, 4, 1)
    }
  }
#undef SA_PLAN
  return hipErrorInvalidValue;
}

}  // namespace sa
