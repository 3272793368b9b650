// The SwiGLU FFN of the action fusion on 16x16x32 bf16 matrix-core products
// (SequenceO1 close-reading page, section 2.2: x_i = e_i + FFN([e_i; a_i])
// with the gated FFN silu(z W_gate) * (z W_up), then W_down).  Shared by the
// standalone pass (sa_action.hip, which writes X) and the pass that feeds the
// compression directly (sa_action_sa.hip), so both form x_i by the same
// instructions in the same order.
//
// A wave handles NB blocks of 16 rows.  z = [e ; a ; 0] for row 16 ib + l16
// sits in registers as B operands: fragment ks holds K slots 32 ks + 8 g ..
// + 7 (g = lane / 16).  The FFN width is walked in chunks of 32 columns whose
// weights arrive packed in LDS (layout below).  Per chunk:
//   gate^T, up^T = W^T z^T      (A = weight rows, B = z)
//   H = silu(gate) * up         in registers, already in the B-operand layout
//                               of the next product: the 16x16 output puts
//                               chunk column 16 (e / 4) + 4 g + e % 4 in slot
//                               (g, e) of row l16
//   x^T += W_down^T H^T         (A = W_down^T rows permuted to match)
#pragma once

#include "sa_stream.hpp"

namespace sa {

// Byte layout of one packed chunk (32 FFN columns): W_gate^T block [32][KP],
// W_up^T block [32][KP] (16-byte chunk h of row f at h ^ (f % 8)), then the
// W_down^T block [D][32]: row 16 cb + i holds output column
// oc = 32 (cb / 2) + 4 (cb % 2) + 8 (i / 4) + i % 4, W_down[32 c0 + perm(pos)][oc]
// at position pos = 8 g + e, perm = 16 (e / 4) + 4 g + e % 4; chunk g stored
// at g ^ 2 ((row / 8) % 2).  The row order puts output column 32 ks + 8 g + e
// in accumulator (cb = 2 ks + e / 4, register e % 4) of lane group g: the
// lane's z fragment for K slots 32 ks + 8 g .. + 7, so the residual e_i is
// added from registers and stored as 16-byte pieces.
template <int D, int KP>
struct ActChunk {
  static constexpr int W_BYTES = 32 * KP * 2;
  static constexpr int D_BYTES = D * 32 * 2;
  static constexpr int CHUNK = 2 * W_BYTES + D_BYTES;
};

// LDS byte offsets of a lane's weight fragments within a chunk: weight row
// 16 fb + l16, 16-byte chunk 4 ks + g (swizzled by the row's low bits); W_down^T
// row 16 cb + l16, chunk g
template <int D, int KP>
struct FfnOffsets {
  uint32_t woff[KP / 32];
  uint32_t doff;
};
template <int D, int KP>
__device__ __forceinline__ FfnOffsets<D, KP> ffn_offsets(int l16, int g) {
  FfnOffsets<D, KP> o;
#pragma unroll
  for (int ks = 0; ks < KP / 32; ++ks) o.woff[ks] = (uint32_t)(2 * (l16 * KP + 8 * ((4 * ks + g) ^ (l16 & 7))));
  o.doff = (uint32_t)(2 * 2 * 32 * KP + 2 * (l16 * 32 + 8 * (g ^ (2 * ((l16 >> 3) & 1)))));
  return o;
}

// One chunk at LDS byte `buf`: acc[ib][cb] (x^T rows 16 cb + 4 g + r, column
// = row 16 ib + l16 of the wave) += the chunk's share of W_down^T H^T.
template <int D, int KP, int NB>
__device__ __forceinline__ void ffn_chunk(uint32_t buf, const FfnOffsets<D, KP>& o, const bf16x8 (&zf)[NB][KP / 32],
                                          f32x4 (&acc)[NB][D / 16]) {
  using MF = Mfma<bf16>;
  constexpr int KS = KP / 32, CB = D / 16;
  constexpr uint32_t W_BYTES = ActChunk<D, KP>::W_BYTES;
  // gate^T and up^T: [fb][ib] holds column 16 fb + 4 g + r of the chunk for row 16 ib + l16.
  // Unit p = 2 ks + fb (its W_gate^T and W_up^T fragments, 4 NB products),
  // fragments loaded PD units ahead behind scheduling fences, so the LDS
  // latency hides under the products of the units in between.
  constexpr int NU = 2 * KS, PD = 3;
  f32x4 ga[2][NB], ua[2][NB];
  bf16x8 wg[NU], wu[NU];
  auto load = [&](int p) {
    const uint32_t off = o.woff[p >> 1] + (uint32_t)(2 * 16 * (p & 1) * KP);
    wg[p] = lds_b128(buf + off);
    wu[p] = lds_b128(buf + W_BYTES + off);
  };
#pragma unroll
  for (int p = 0; p < PD; ++p) load(p);
#pragma unroll
  for (int p = 0; p < NU; ++p) {
    if (p + PD < NU) load(p + PD);
    __builtin_amdgcn_sched_barrier(0);
    const int ks = p >> 1, fb = p & 1;
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) {
      const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
      ga[fb][ib] = MF::run(wg[p], zf[ib][ks], ks == 0 ? z : ga[fb][ib]);
      ua[fb][ib] = MF::run(wu[p], zf[ib][ks], ks == 0 ? z : ua[fb][ib]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // the W_down^T fragments of this chunk, issued before the H arithmetic
  bf16x8 wd[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) wd[cb] = lds_b128(buf + o.doff + (uint32_t)(2 * 16 * cb * 32));
  // H = silu(gate) * up, slot (g, e) <-> column 16 (e / 4) + 4 g + e % 4
  bf16x8 hf[NB];
#pragma unroll
  for (int ib = 0; ib < NB; ++ib) {
    float hv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float gv = ga[e >> 2][ib][e & 3];
      hv[e] = gv * __builtin_amdgcn_rcpf(1.f + fast_exp2(-1.4426950408889634f * gv)) * ua[e >> 2][ib][e & 3];
    }
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    hf[ib] = __builtin_convertvector((f32x8{hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]}), bf16x8);
  }
  // x^T[16 cb + 4 g + r][row 16 ib + l16] += W_down^T H^T over the chunk
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) acc[ib][cb] = MF::run(wd[cb], hf[ib], acc[ib][cb]);
}

// x = e + FFN for columns 32 ks + 8 g .. + 7 of row 16 ib + l16: the FFN part
// in accumulators 2 ks and 2 ks + 1, e_i in z fragment ks; rounded to bf16
template <int D, int KP, int NB>
__device__ __forceinline__ bf16x8 ffn_residual(const bf16x8 (&zf)[NB][KP / 32], const f32x4 (&acc)[NB][D / 16], int ib,
                                               int ks) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)((float)zf[ib][ks][e] + acc[ib][2 * ks + (e >> 2)][e & 3]);
  return v;
}

}  // namespace sa
