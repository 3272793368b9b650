// Action fusion on gfx950 (bf16 operands, float32 accumulation):
// SequenceO1 close-reading page, section 2.2 -- each history row is
//
//   x_i = e_i + (silu(z_i W_gate) * (z_i W_up)) W_down,   z_i = [e_i ; a_i],
//
// e_i the item embedding, a_i = table[action_i] the action-type embedding.
// One pass over the rows, writing X; waves own rows, the weights stream
// through LDS.  8 waves x 32 rows per 256-row tile; z for the wave's rows is
// built in registers (fragments of e_i from HBM, of a_i from the
// cache-resident table, zero past d + d_a, K padded to a multiple of 64) and
// the FFN runs chunk by chunk as sa_action_ffn.hpp describes, the chunks
// arriving by LDS DMA, double-buffered.  x = e + (x^T)^T is stored in bf16,
// eight columns per lane.  A tile's action ids and, where the registers
// allow, its E fragments are loaded while the previous tile runs.
#include <hip/hip_runtime.h>

#include "sa_action.h"
#include "sa_action_ffn.hpp"

namespace sa {

namespace {

constexpr int kActWaves = 8;

// The packed chunk layout is that of ActChunk (sa_action_ffn.hpp); two steps'
// buffers of CPS chunks each fit in LDS.
template <int D, int KP>
struct ActGeom : ActChunk<D, KP> {
  using ActChunk<D, KP>::CHUNK;
  static constexpr int CPS = 4 * CHUNK <= 144 * 1024 ? 2 : 1;  // chunks per step (two steps' buffers in LDS)
  static constexpr int STEP = CPS * CHUNK;
  static_assert(STEP % 1024 == 0, "whole DMA blocks");
  static constexpr int NBLK = STEP / 1024;
  static constexpr int BPW = (NBLK + kActWaves - 1) / kActWaves;
};

template <int D, int KP>
__global__ __launch_bounds__(256) void action_pack_kernel(const bf16* Wg, const bf16* Wu, const bf16* Wd, int kin,
                                                          int d_ff, bf16* packed) {
  using G = ActGeom<D, KP>;
  constexpr int CH_ELEMS = G::CHUNK / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int chunks = d_ff / 32;
  if (idx >= (int64_t)chunks * CH_ELEMS) return;
  const int c = (int)(idx / CH_ELEMS), w = (int)(idx % CH_ELEMS);
  bf16 v;
  int pos;
  if (w < 2 * 32 * KP) {
    const bf16* W = w < 32 * KP ? Wg : Wu;
    const int ww = w % (32 * KP), f = ww / KP, kk = ww % KP;
    v = kk < kin ? W[(int64_t)kk * d_ff + 32 * c + f] : (bf16)0.f;
    pos = (w / (32 * KP)) * 32 * KP + f * KP + 8 * ((kk >> 3) ^ (f & 7)) + (kk & 7);
  } else {
    const int ww = w - 2 * 32 * KP, col = ww / 32, p = ww % 32, gg = p >> 3, e = p & 7;
    const int f = 32 * c + 16 * (e >> 2) + 4 * gg + (e & 3);
    // packed row col = 16 cb + i holds output column 32 (cb / 2) + 4 (cb % 2) + 8 (i / 4) + i % 4
    const int cb = col >> 4, i = col & 15;
    const int oc = 32 * (cb >> 1) + 4 * (cb & 1) + 8 * (i >> 2) + (i & 3);
    v = Wd[(int64_t)f * D + oc];
    pos = 2 * 32 * KP + col * 32 + 8 * (gg ^ (2 * ((col >> 3) & 1))) + e;
  }
  packed[(int64_t)c * CH_ELEMS + pos] = v;
}

template <int D, int KP>
__global__ __launch_bounds__(64 * kActWaves) void action_fuse_kernel(ActionArgs args) {
  using G = ActGeom<D, KP>;
  constexpr int NT = 32 * kActWaves, KS = KP / 32, CB = D / 16, CPS = G::CPS;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * G::STEP];
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) unsigned char*)lds;

  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rw = 32 * wave;
  const bf16* const E = static_cast<const bf16*>(args.E);
  const bf16* const T = static_cast<const bf16*>(args.table);
  const unsigned char* const packed = static_cast<const unsigned char*>(args.packed);
  bf16* const X = static_cast<bf16*>(args.X);
  const int chunks = args.chunks, steps = chunks / CPS;

  const int64_t rows = args.rows, ngroups = gridDim.x, grp = blockIdx.x;
  const int64_t r_begin = grp * rows / ngroups, r_end = (grp + 1) * rows / ngroups;
  if (r_begin >= r_end) return;

  auto issue_step = [&](int s, int b) {
    const unsigned char* src = packed + (int64_t)s * G::STEP;
#pragma unroll
    for (int i = 0; i < G::BPW; ++i) {
      const int j = wave + kActWaves * i;
      if (G::NBLK % kActWaves == 0 || j < G::NBLK)
        dma16(src, (uint32_t)(1024 * j + 16 * lane), lds0 + (uint32_t)(b * G::STEP + 1024 * j));
    }
  };
  const FfnOffsets<D, KP> fo = ffn_offsets<D, KP>(l16, g);

  // action ids of a tile's rows (this lane's rows 16 ib + l16 of the wave), loaded a tile ahead so that the
  // table rows they select do not wait for them
  auto load_actions = [&](int64_t t, int (&ids)[2]) {
    const int64_t lm = r_end - 1 - t;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      const int r = rw + 16 * ib + l16;
      ids[ib] = args.actions[t + (r <= lm ? r : lm)];
    }
  };
  int act_next[2];
  load_actions(r_begin, act_next);
  // the E fragments (K slots below D) of the next tile too, where the registers allow (all but d = 128 with
  // K padded to 256)
  constexpr int KE = D / 32;
  constexpr bool PF = !(D == 128 && KP == 256);
  bf16x8 ze[2][KE];
  auto load_e = [&](int64_t t) {
    const int64_t lm = r_end - 1 - t;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      const int r = rw + 16 * ib + l16;
      const int64_t row = t + (r <= lm ? r : lm);
#pragma unroll
      for (int ks = 0; ks < KE; ++ks) ze[ib][ks] = *reinterpret_cast<const bf16x8*>(E + row * D + 32 * ks + 8 * g);
    }
  };
  if constexpr (PF) load_e(r_begin);

  int q = 0;
  issue_step(0, 0);
  wait_vm<0>();
  __syncthreads();
  for (int64_t t0 = r_begin; t0 < r_end; t0 += NT) {
    const int64_t lim = r_end - 1 - t0;
    const bool busy = rw <= lim;  // wave-uniform
    int acts[2] = {act_next[0], act_next[1]};
    // z = [e ; a ; 0] for rows 16 ib + l16 of this wave, K slots 32 ks + 8 g ..
    bf16x8 zf[2][KS];
    bool valid[2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      const int r = rw + 16 * ib + l16;
      valid[ib] = r <= lim;
      const int64_t row = t0 + (r <= lim ? r : lim);
      int act = acts[ib];
      act = act < 0 ? 0 : (act >= args.n_actions ? args.n_actions - 1 : act);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int k0 = 32 * ks + 8 * g;
        if (ks < KE) {
          zf[ib][ks] = PF ? ze[ib][ks] : *reinterpret_cast<const bf16x8*>(E + row * D + k0);
        } else if (k0 < D + args.d_a) {
          zf[ib][ks] = *reinterpret_cast<const bf16x8*>(T + (int64_t)act * args.d_a + (k0 - D));
        } else {
          zf[ib][ks] = bf16x8{};
        }
      }
    }
    if (t0 + NT < r_end) {
      load_actions(t0 + NT, act_next);
      if constexpr (PF) load_e(t0 + NT);
    }
    f32x4 acc[2][CB];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[ib][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s = 0; s < steps; ++s) {
      const bool last_tile = t0 + NT >= r_end;
      if (s + 1 < steps) issue_step(s + 1, q ^ 1);
      else if (!last_tile) issue_step(0, q ^ 1);
      if (busy) {
#pragma unroll
        for (int h = 0; h < CPS; ++h) ffn_chunk<D, KP, 2>(lds0 + (uint32_t)(q * G::STEP + h * G::CHUNK), fo, zf, acc);
      }
      wait_vm<0>();
      __syncthreads();
      q ^= 1;
    }
    // x = e + FFN: this lane holds columns 32 ks + 8 g .. + 7 of row 16 ib + l16
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      if (!valid[ib]) continue;
      const int64_t row = t0 + rw + 16 * ib + l16;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        *reinterpret_cast<bf16x8*>(X + row * D + 32 * ks + 8 * g) = ffn_residual<D, KP, 2>(zf, acc, ib, ks);
    }
  }
  wait_vm<0>();
}

template <int D, int KP>
hipError_t fuse_t(const ActionArgs& a, int groups, hipStream_t s, hipEvent_t e0, hipEvent_t e1, int* occ) {
  if (occ) return hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, action_fuse_kernel<D, KP>, 64 * kActWaves, 0);
  if (e0 || e1)
    hipExtLaunchKernelGGL((action_fuse_kernel<D, KP>), dim3(groups), dim3(64 * kActWaves), 0, s, e0, e1, 0, a);
  else
    hipLaunchKernelGGL((action_fuse_kernel<D, KP>), dim3(groups), dim3(64 * kActWaves), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t fuse_d(int kp, const ActionArgs& a, int groups, hipStream_t s, hipEvent_t e0, hipEvent_t e1, int* occ) {
  switch (kp) {
    case 64: return D == 64 ? fuse_t<64, 64>(a, groups, s, e0, e1, occ) : hipErrorInvalidValue;
    case 128: return fuse_t<D, 128>(a, groups, s, e0, e1, occ);
    case 192: return fuse_t<D, 192>(a, groups, s, e0, e1, occ);
    case 256: return fuse_t<D, 256>(a, groups, s, e0, e1, occ);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int KP>
hipError_t pack_t(const void* Wg, const void* Wu, const void* Wd, int kin, int d_ff, void* packed, hipStream_t s) {
  const int64_t total = (int64_t)(d_ff / 32) * (ActGeom<D, KP>::CHUNK / 2);
  hipLaunchKernelGGL((action_pack_kernel<D, KP>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     (const bf16*)Wg, (const bf16*)Wu, (const bf16*)Wd, kin, d_ff, (bf16*)packed);
  return hipGetLastError();
}

}  // namespace

int action_kpad(int d, int d_a) { return 64 * ((d + d_a + 63) / 64); }

size_t action_packed_bytes(int d, int kp, int d_ff) {
  return (size_t)(d_ff / 32) * (size_t)(2 * 32 * kp * 2 + d * 32 * 2);
}

hipError_t launch_action_pack(int d, int kp, const void* Wg, const void* Wu, const void* Wd, int d_a, int d_ff,
                              void* packed, hipStream_t s) {
  const int kin = d + d_a;
  if (d == 128) {
    if (kp == 128) return pack_t<128, 128>(Wg, Wu, Wd, kin, d_ff, packed, s);
    if (kp == 192) return pack_t<128, 192>(Wg, Wu, Wd, kin, d_ff, packed, s);
    if (kp == 256) return pack_t<128, 256>(Wg, Wu, Wd, kin, d_ff, packed, s);
  } else if (d == 64) {
    if (kp == 64) return pack_t<64, 64>(Wg, Wu, Wd, kin, d_ff, packed, s);
    if (kp == 128) return pack_t<64, 128>(Wg, Wu, Wd, kin, d_ff, packed, s);
    if (kp == 192) return pack_t<64, 192>(Wg, Wu, Wd, kin, d_ff, packed, s);
    if (kp == 256) return pack_t<64, 256>(Wg, Wu, Wd, kin, d_ff, packed, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_action_fuse(int d, int kp, const ActionArgs& a, int groups, hipStream_t s, hipEvent_t start,
                              hipEvent_t stop) {
  if (d == 128) return fuse_d<128>(kp, a, groups, s, start, stop, nullptr);
  if (d == 64) return fuse_d<64>(kp, a, groups, s, start, stop, nullptr);
  return hipErrorInvalidValue;
}

hipError_t action_occupancy(int d, int kp, int* groups_per_cu) {
  static const ActionArgs unused{};
  if (d == 128) return fuse_d<128>(kp, unused, 0, nullptr, nullptr, nullptr, groups_per_cu);
  if (d == 64) return fuse_d<64>(kp, unused, 0, nullptr, nullptr, nullptr, groups_per_cu);
  return hipErrorInvalidValue;
}

// ---- float32 path: the rows z = [e; a; 0] gathered into a staging buffer,
// then the FFN as float32 matrix-core products (launch_plain_ffn) with the
// residual e added on output.
namespace {

// dst[c][r] = r < rows_in ? src[r][c] : 0 for c < cols, r < rows_pad
__global__ __launch_bounds__(256) void transpose_pad_kernel(const float* __restrict__ src, int64_t rows_in, int cols,
                                                            int64_t rows_pad, float* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)cols * rows_pad) return;
  const int64_t c = i / rows_pad, r = i % rows_pad;
  dst[i] = r < rows_in ? src[r * cols + c] : 0.f;
}

// Z[r] = [E[r]; table[clamp(actions[r])]; 0 ...] (k_pad floats), one float4 per thread
__global__ __launch_bounds__(256) void gather_f32_kernel(const float* __restrict__ E, const int32_t* __restrict__ actions,
                                                         const float* __restrict__ table, int64_t rows, int d, int d_a,
                                                         int k_pad, int n_actions, float* __restrict__ Z) {
  const int q = k_pad / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * q) return;
  const int64_t r = i / q;
  const int c = 4 * (int)(i % q);
  float4 v = {0.f, 0.f, 0.f, 0.f};
  if (c < d) {
    v = *reinterpret_cast<const float4*>(E + r * d + c);
  } else if (c < d + d_a) {
    int a = actions[r];
    a = a < 0 ? 0 : (a >= n_actions ? n_actions - 1 : a);
    v = *reinterpret_cast<const float4*>(table + (int64_t)a * d_a + (c - d));
  }
  *reinterpret_cast<float4*>(Z + r * k_pad + c) = v;
}

}  // namespace

hipError_t launch_transpose_pad(const float* src, int64_t rows_in, int cols, int64_t rows_pad, float* dst,
                                hipStream_t s) {
  const int64_t n = (int64_t)cols * rows_pad;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_pad_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, rows_in, cols,
                     rows_pad, dst);
  return hipGetLastError();
}

hipError_t launch_action_gather_f32(const float* E, const int32_t* actions, const float* table, int64_t rows, int d,
                                    int d_a, int k_pad, int n_actions, float* Z, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t n = rows * (k_pad / 4);
  hipLaunchKernelGGL(gather_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, E, actions, table, rows,
                     d, d_a, k_pad, n_actions, Z);
  return hipGetLastError();
}

int action_chunks_per_step(int d, int kp) {
  const int chunk = 2 * 32 * kp * 2 + d * 32 * 2;
  return 4 * chunk <= 144 * 1024 ? 2 : 1;
}

}  // namespace sa
