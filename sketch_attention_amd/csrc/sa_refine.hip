// Kernels of stacked refinement (SequenceO1 close-reading page, section 2.2):
// after the first SA pass the k x d state of each user queries its raw
// history again.  The heavy part of a layer is the same fused pass as the
// first (sa_stream.hpp / sa_fused.hpp) with one folded matrix per user; the
// kernels here are the small per-user pieces around it:
//
//   fold_users   M_u = scale * state_u W_QK, W_QK = W_Q W_K^T (per layer)
//   add_ln       out = LN(a + b) over the width d (residual + layer norm)
//   ffn_gate_up  H = silu(Z W_gate) * (Z W_up)      float32 matrix cores
//   ffn_down     F = H W_down                       float32 matrix cores
//
// The residual + layer norm that forms the A rows of the fold or of the gated
// product can run as that kernel's prologue, so a layer's small work is three
// launches (fold, gate/up, down) besides the fused pass and its reduction.
// All in float32; the folded matrices are rounded once to the pass's dtype.
#include <hip/hip_runtime.h>

#include "sa_internal.h"

namespace sa {

typedef __bf16 bf16;

namespace {

// ------------------------------------------------------------ weight prep
// W_QK[a][c] = sum_b W_Q[a][b] W_K[c][b]: the affinity (Q W_Q)(x W_K)^T of a
// query row Q and a history row x equals (Q W_QK) x^T.  Stored transposed,
// out[c][a] = W_QK[a][c], the B layout of the fold product.
template <typename T>
__global__ __launch_bounds__(256) void wqk_t_kernel(const T* WQ, const T* WK, int d, float* out) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= d * d) return;
  const int c = idx / d, a = idx % d;
  float s = 0.f;
  for (int b = 0; b < d; ++b) s += (float)WQ[a * d + b] * (float)WK[c * d + b];
  out[idx] = s;
}

// dst[c][r] = src[r][c] for a rows x cols float32 matrix
__global__ __launch_bounds__(256) void transpose_kernel(const float* src, int rows, int cols, float* dst) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * cols) return;
  const int r = idx / cols, c = idx % cols;
  dst[(int64_t)c * rows + r] = src[idx];
}

// ------------------------------------------------------------ residual + LN
// out[r] = (v - mean) / sqrt(var + eps) * gain + bias with v = a[ra] + b[r],
// ra = r % a_period (a broadcast over users when a_period = k, else r).  One
// wave per row of d = 64 or 128 values; population variance over d.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void add_ln_kernel(const float* a, int64_t a_period, const float* b,
                                                     const float* gain, const float* bias, float eps, int64_t rows,
                                                     float* out) {
  constexpr int PER = D / 64;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t ra = a_period > 0 ? r % a_period : r;
  float v[PER];
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = lane + 64 * e;
    v[e] = a[ra * D + c] + b[r * D + c];
    s += v[e];
  }
  const float mean = wave_sum(s) * (1.f / D);
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    v[e] -= mean;
    q += v[e] * v[e];
  }
  const float inv = 1.f / sqrtf(wave_sum(q) * (1.f / D) + eps);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = lane + 64 * e;
    out[r * D + c] = v[e] * inv * gain[c] + bias[c];
  }
}

// ------------------------------------------------------------ small products
// C = A B for row-major A [M][K] and B given transposed, Bt [N][K], float32
// matrix cores (16x16x4).  A work group owns a 16 x 16 NB tile of C with KS
// waves that split the reduction (wave w takes K chunks w, w + KS, ...), so
// a long reduction is not one serial chain of loads; the waves' sums are
// added through LDS in wave order (deterministic).  Reduction slot (g, s) of
// a 16-column chunk k0 is column k0 + 4 g + s of both operands, so each lane
// reads four consecutive floats of a row.  Rows of A past M read zeros and
// are not stored.  Epilogues:
//   EPI_STORE  C[r][c] = acc
//   EPI_GATED  C[r][c] = silu(A Bt0^T) * (A Bt1^T)      (SwiGLU hidden layer)
//   EPI_RESID  C[r][c] = A Bt0^T + A2[r][c]  (a residual added on output)
//   EPI_FOLD   row r = u k + j of the per-user states -> M[u][j][c] =
//              scale * acc rounded to T (rows k..k_pad-1 of each user are
//              left as they are: zero from allocation)
// With LN = K (64 or 128) the A rows are formed in the kernel as the
// residual + layer norm of the block that precedes the product,
//   A[r] = LN(A[r % a_period (r when 0)] + A2[r]) * gain + bias,
// by all waves of the group into LDS; the work groups of the first column
// block also store them to ln_out (the block's output, needed again later).
typedef float f32x4_t __attribute__((ext_vector_type(4)));
enum { EPI_STORE = 0, EPI_GATED = 1, EPI_FOLD = 2, EPI_RESID = 3 };

struct GemmArgs {
  const float* A;
  int64_t M;
  int K;
  const float* Bt0;
  const float* Bt1;
  int N;
  void* C;
  float scale;
  int k, k_pad;
  // layer-norm prologue (LN > 0 only)
  int64_t a_period;
  const float* A2;
  const float* gain;
  const float* bias;
  float eps;
  float* ln_out;
};

template <int EPI, typename T, int NB, int KS, int LN>
__global__ __launch_bounds__(64 * KS) void small_gemm_kernel(const GemmArgs args) {
  constexpr int NO = EPI == EPI_GATED ? 2 : 1;  // products per tile
  constexpr int LDA = LN + 4;                    // LDS row stride of the normalised A rows (floats)
  __shared__ f32x4_t red[KS > 1 ? KS - 1 : 1][NO][NB][64];
  __shared__ float lnA[LN > 0 ? 16 * LDA : 1];
  const float* A = args.A;
  const int64_t M = args.M;
  const int K = LN > 0 ? LN : args.K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.y * 16;
  const int col0 = blockIdx.x * 16 * NB;
  const int64_t arow = row0 + l16;
  // four partial sums per block (slot s of each chunk), added at the end:
  // four independent chains instead of one long dependent one
  f32x4_t acc0[NB][4], acc1[NB][4];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc0[j][s] = acc1[j][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (LN > 0) {
    constexpr int IT = LN / (16 * KS);  // chunks per wave
    static_assert(IT * 16 * KS == LN, "the reduction must split evenly over the waves");
    // the wave's B operands are loaded before the layer norm so that their latency overlaps it
    f32x4_t pb0[IT][NB], pb1[IT][NB];
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int64_t off = (int64_t)(col0 + 16 * j + l16) * LN + 16 * (i * KS + wave) + 4 * g;
        pb0[i][j] = *reinterpret_cast<const f32x4_t*>(args.Bt0 + off);
        if constexpr (EPI == EPI_GATED) pb1[i][j] = *reinterpret_cast<const f32x4_t*>(args.Bt1 + off);
      }
    {
      // every wave normalises 16 / KS of the rows: LPR lanes per row, lane cl of a row takes the float4s
      // cl, cl + LPR, ... (consecutive lanes read consecutive float4s)
      constexpr int RPW = 16 / KS, LPR = 64 / RPW, NF = LN / (4 * LPR);
      static_assert(RPW * KS == 16 && NF * 4 * LPR == LN, "the layer norm must split evenly over the lanes");
      const int rr = lane / LPR, cl = lane % LPR;
      const int lrow = wave * RPW + rr;
      const int64_t row = row0 + lrow;
      const int64_t ra = args.a_period > 0 ? (int64_t)((uint32_t)row % (uint32_t)args.a_period) : row;  // < 2^31 rows
      f32x4_t v[NF], gn[NF], bs[NF];
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int c = 4 * (cl + LPR * i);
        gn[i] = *reinterpret_cast<const f32x4_t*>(args.gain + c);
        bs[i] = *reinterpret_cast<const f32x4_t*>(args.bias + c);
        v[i] = row < M ? *reinterpret_cast<const f32x4_t*>(A + ra * LN + c) +
                             *reinterpret_cast<const f32x4_t*>(args.A2 + row * LN + c)
                       : f32x4_t{0.f, 0.f, 0.f, 0.f};
        sum += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
      }
#pragma unroll
      for (int o = LPR / 2; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
      const float mean = sum * (1.f / LN);
      float q = 0.f;
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        v[i] -= mean;
        q += (v[i][0] * v[i][0] + v[i][1] * v[i][1]) + (v[i][2] * v[i][2] + v[i][3] * v[i][3]);
      }
#pragma unroll
      for (int o = LPR / 2; o >= 1; o >>= 1) q += __shfl_xor(q, o);
      const float inv = 1.f / sqrtf(q * (1.f / LN) + args.eps);
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const int c = 4 * (cl + LPR * i);
        const f32x4_t out = row < M ? v[i] * inv * gn[i] + bs[i] : f32x4_t{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4_t*>(&lnA[lrow * LDA + c]) = out;
        if (blockIdx.x == 0 && row < M) *reinterpret_cast<f32x4_t*>(args.ln_out + row * LN + c) = out;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&lnA[l16 * LDA + 16 * (i * KS + wave) + 4 * g]);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          acc0[j][s] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], pb0[i][j][s], acc0[j][s], 0, 0, 0);
          if constexpr (EPI == EPI_GATED)
            acc1[j][s] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], pb1[i][j][s], acc1[j][s], 0, 0, 0);
        }
    }
  } else {
#pragma unroll 4  // loads of several chunks in flight
    for (int k0 = 16 * wave; k0 < K; k0 += 16 * KS) {
      const f32x4_t a =
          arow < M ? *reinterpret_cast<const f32x4_t*>(A + arow * K + k0 + 4 * g) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      f32x4_t b0[NB], b1[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        b0[j] = *reinterpret_cast<const f32x4_t*>(args.Bt0 + (int64_t)(col0 + 16 * j + l16) * K + k0 + 4 * g);
        if constexpr (EPI == EPI_GATED)
          b1[j] = *reinterpret_cast<const f32x4_t*>(args.Bt1 + (int64_t)(col0 + 16 * j + l16) * K + k0 + 4 * g);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          acc0[j][s] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b0[j][s], acc0[j][s], 0, 0, 0);
          if constexpr (EPI == EPI_GATED)
            acc1[j][s] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b1[j][s], acc1[j][s], 0, 0, 0);
        }
    }
  }
  f32x4_t sum0[NB], sum1[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    sum0[j] = (acc0[j][0] + acc0[j][1]) + (acc0[j][2] + acc0[j][3]);
    sum1[j] = (acc1[j][0] + acc1[j][1]) + (acc1[j][2] + acc1[j][3]);
  }
  if constexpr (KS > 1) {
    if (wave > 0) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        red[wave - 1][0][j][lane] = sum0[j];
        if constexpr (EPI == EPI_GATED) red[wave - 1][NO - 1][j][lane] = sum1[j];
      }
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < KS - 1; ++w)
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        sum0[j] += red[w][0][j][lane];
        if constexpr (EPI == EPI_GATED) sum1[j] += red[w][NO - 1][j][lane];
      }
  }
  // lane holds C[row0 + 4 g + r][col0 + 16 j + l16]
  T* C = static_cast<T*>(args.C);
  const int N = args.N;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t row = row0 + 4 * g + r;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int col = col0 + 16 * j + l16;
      float v = sum0[j][r];
      if constexpr (EPI == EPI_GATED) {
        // silu(gate) * up, with the hardware exp2 and reciprocal (about 1 ulp each)
        v = v * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * v)) * sum1[j][r];
        C[row * N + col] = (T)v;
      } else if constexpr (EPI == EPI_RESID) {
        C[row * N + col] = (T)(v + args.A2[row * N + col]);
      } else if constexpr (EPI == EPI_FOLD) {
        const int64_t u = row / args.k, jj = row % args.k;
        C[(u * args.k_pad + jj) * N + col] = (T)(args.scale * v);
      } else {
        C[row * N + col] = (T)v;
      }
    }
  }
}

// ln = the layer-norm width (64 or 128), or 0 for plain A rows.
template <int EPI, typename T, int NB, int KS, bool WITH_LN>
hipError_t launch_gemm(const GemmArgs& a, int ln, hipStream_t s) {
  const dim3 grid((unsigned)(a.N / (16 * NB)), (unsigned)((a.M + 15) / 16)), block(64 * KS);
  if constexpr (WITH_LN) {
    if (ln == 128)
      hipLaunchKernelGGL((small_gemm_kernel<EPI, T, NB, KS, 128>), grid, block, 0, s, a);
    else if (ln == 64)
      hipLaunchKernelGGL((small_gemm_kernel<EPI, T, NB, KS, 64>), grid, block, 0, s, a);
    else if (ln == 0)
      hipLaunchKernelGGL((small_gemm_kernel<EPI, T, NB, KS, 0>), grid, block, 0, s, a);
    else
      return hipErrorInvalidValue;
  } else {
    if (ln != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((small_gemm_kernel<EPI, T, NB, KS, 0>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_wqk_t(int dtype, const void* WQ, const void* WK, int d, float* out, hipStream_t s) {
  const int blocks = (d * d + 255) / 256;
  if (dtype == 1)
    hipLaunchKernelGGL(wqk_t_kernel<bf16>, dim3(blocks), dim3(256), 0, s, (const bf16*)WQ, (const bf16*)WK, d, out);
  else
    hipLaunchKernelGGL(wqk_t_kernel<float>, dim3(blocks), dim3(256), 0, s, (const float*)WQ, (const float*)WK, d, out);
  return hipGetLastError();
}

hipError_t launch_transpose(const float* src, int rows, int cols, float* dst, hipStream_t s) {
  hipLaunchKernelGGL(transpose_kernel, dim3((rows * cols + 255) / 256), dim3(256), 0, s, src, rows, cols, dst);
  return hipGetLastError();
}

hipError_t launch_fold_users(int dtype, const LnPrologue* ln, const float* state, const float* wqk_t, float scale,
                             int users, int k, int k_pad, int d, void* M, hipStream_t s) {
  if (d % 32 != 0) return hipErrorInvalidValue;
  GemmArgs a{};
  a.A = ln != nullptr ? ln->a : state;
  a.M = (int64_t)users * k;
  a.K = d;
  a.Bt0 = wqk_t;
  a.N = d;
  a.C = M;
  a.scale = scale;
  a.k = k;
  a.k_pad = k_pad;
  if (ln != nullptr) {
    a.a_period = ln->a_period;
    a.A2 = ln->b;
    a.gain = ln->gain;
    a.bias = ln->bias;
    a.eps = ln->eps;
    a.ln_out = ln->out;
  }
  return dtype == 1 ? launch_gemm<EPI_FOLD, bf16, 2, 2, true>(a, ln ? d : 0, s)
                    : launch_gemm<EPI_FOLD, float, 2, 2, true>(a, ln ? d : 0, s);
}

hipError_t launch_add_ln(const float* a, int64_t a_period, const float* b, const float* gain, const float* bias,
                         float eps, int64_t rows, int d, float* out, hipStream_t s) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (d == 128)
    hipLaunchKernelGGL(add_ln_kernel<128>, grid, dim3(256), 0, s, a, a_period, b, gain, bias, eps, rows, out);
  else if (d == 64)
    hipLaunchKernelGGL(add_ln_kernel<64>, grid, dim3(256), 0, s, a, a_period, b, gain, bias, eps, rows, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_ffn(const LnPrologue* ln, const float* Z, int64_t rows, int d, int d_ff, const float* gate_t,
                      const float* up_t, const float* down_t, float* H, float* F, hipStream_t s) {
  if (d % 32 != 0 || d_ff % 32 != 0) return hipErrorInvalidValue;
  GemmArgs g{};
  g.A = ln != nullptr ? ln->a : Z;
  g.M = rows;
  g.K = d;
  g.Bt0 = gate_t;
  g.Bt1 = up_t;
  g.N = d_ff;
  g.C = H;
  if (ln != nullptr) {
    g.a_period = ln->a_period;
    g.A2 = ln->b;
    g.gain = ln->gain;
    g.bias = ln->bias;
    g.eps = ln->eps;
    g.ln_out = ln->out;
  }
  hipError_t e = launch_gemm<EPI_GATED, float, 2, 2, true>(g, ln ? d : 0, s);
  if (e != hipSuccess) return e;
  // the down projection has few output columns and a long reduction: the reduction is split over eight waves
  GemmArgs dn{};
  dn.A = H;
  dn.M = rows;
  dn.K = d_ff;
  dn.Bt0 = down_t;
  dn.N = d;
  dn.C = F;
  return launch_gemm<EPI_STORE, float, 2, 8, false>(dn, 0, s);
}

hipError_t launch_f32_gemm(const float* A, int64_t M, int K, const float* Bt, int N, float* C, const float* resid,
                           bool long_k, hipStream_t s) {
  if (K % 16 != 0 || N % 32 != 0 || M < 0) return hipErrorInvalidValue;
  if (M == 0) return hipSuccess;
  GemmArgs g{};
  g.A = A;
  g.M = M;
  g.K = K;
  g.Bt0 = Bt;
  g.N = N;
  g.C = C;
  g.A2 = resid;
  if (resid != nullptr)
    return long_k ? launch_gemm<EPI_RESID, float, 2, 8, false>(g, 0, s) : launch_gemm<EPI_RESID, float, 2, 2, false>(g, 0, s);
  return long_k ? launch_gemm<EPI_STORE, float, 2, 8, false>(g, 0, s) : launch_gemm<EPI_STORE, float, 2, 2, false>(g, 0, s);
}

hipError_t launch_plain_ffn(const float* Z, int64_t rows, int k_in, int d_out, int d_ff, const float* gate_t,
                            const float* up_t, const float* down_t, float* H, const float* resid, float* X,
                            hipStream_t s) {
  if (k_in % 16 != 0 || d_out % 32 != 0 || d_ff % 32 != 0 || rows < 0) return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  GemmArgs g{};
  g.A = Z;
  g.M = rows;
  g.K = k_in;
  g.Bt0 = gate_t;
  g.Bt1 = up_t;
  g.N = d_ff;
  g.C = H;
  hipError_t e = launch_gemm<EPI_GATED, float, 2, 2, false>(g, 0, s);
  if (e != hipSuccess) return e;
  GemmArgs dn{};
  dn.A = H;
  dn.M = rows;
  dn.K = d_ff;
  dn.Bt0 = down_t;
  dn.N = d_out;
  dn.C = X;
  dn.A2 = resid;
  return launch_gemm<EPI_RESID, float, 2, 8, false>(dn, 0, s);
}

}  // namespace sa
