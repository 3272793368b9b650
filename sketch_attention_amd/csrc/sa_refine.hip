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
// matrix cores (16x16x4), one wave per work group owning a 16 x 16 NB tile so
// that these small products still spread over the compute units.  Reduction
// slot (g, s) of a 16-column chunk k0 is column k0 + 4 g + s of both
// operands, so each lane reads four consecutive floats of a row.  Rows of A
// past M read zeros and are not stored.  Epilogues:
//   EPI_STORE  C[r][c] = acc
//   EPI_GATED  C[r][c] = silu(A Bt0^T) * (A Bt1^T)      (SwiGLU hidden layer)
//   EPI_FOLD   row r = u k + j of the per-user states -> M[u][j][c] =
//              scale * acc rounded to T (rows k..k_pad-1 of each user are
//              left as they are: zero from allocation)
typedef float f32x4_t __attribute__((ext_vector_type(4)));
enum { EPI_STORE = 0, EPI_GATED = 1, EPI_FOLD = 2 };

template <int EPI, typename T, int NB = 2>
__global__ __launch_bounds__(64) void small_gemm_kernel(const float* A, int64_t M, int K, const float* Bt0,
                                                        const float* Bt1, int N, T* C, float scale, int k, int k_pad) {
  const int lane = threadIdx.x;
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
#pragma unroll 4  // loads of several chunks in flight
  for (int k0 = 0; k0 < K; k0 += 16) {
    const f32x4_t a = arow < M ? *reinterpret_cast<const f32x4_t*>(A + arow * K + k0 + 4 * g)
                               : f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t b0[NB], b1[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      b0[j] = *reinterpret_cast<const f32x4_t*>(Bt0 + (int64_t)(col0 + 16 * j + l16) * K + k0 + 4 * g);
      if constexpr (EPI == EPI_GATED)
        b1[j] = *reinterpret_cast<const f32x4_t*>(Bt1 + (int64_t)(col0 + 16 * j + l16) * K + k0 + 4 * g);
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
  f32x4_t sum0[NB], sum1[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    sum0[j] = (acc0[j][0] + acc0[j][1]) + (acc0[j][2] + acc0[j][3]);
    sum1[j] = (acc1[j][0] + acc1[j][1]) + (acc1[j][2] + acc1[j][3]);
  }
  // lane holds C[row0 + 4 g + r][col0 + 16 j + l16]
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t row = row0 + 4 * g + r;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int col = col0 + 16 * j + l16;
      float v = sum0[j][r];
      if constexpr (EPI == EPI_GATED) {
        v = v / (1.f + expf(-v)) * sum1[j][r];  // silu(gate) * up
        C[row * N + col] = (T)v;
      } else if constexpr (EPI == EPI_FOLD) {
        const int64_t u = row / k, jj = row % k;
        C[(u * k_pad + jj) * N + col] = (T)(scale * v);
      } else {
        C[row * N + col] = (T)v;
      }
    }
  }
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

hipError_t launch_fold_users(int dtype, const float* state, const float* wqk_t, float scale, int users, int k, int k_pad,
                             int d, void* M, hipStream_t s) {
  if (d % 32 != 0) return hipErrorInvalidValue;
  const int64_t rows = (int64_t)users * k;
  const dim3 grid(d / 32, (unsigned)((rows + 15) / 16));
  if (dtype == 1)
    hipLaunchKernelGGL((small_gemm_kernel<EPI_FOLD, bf16>), grid, dim3(64), 0, s, state, rows, d, wqk_t, nullptr, d,
                       (bf16*)M, scale, k, k_pad);
  else
    hipLaunchKernelGGL((small_gemm_kernel<EPI_FOLD, float>), grid, dim3(64), 0, s, state, rows, d, wqk_t, nullptr, d,
                       (float*)M, scale, k, k_pad);
  return hipGetLastError();
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

hipError_t launch_ffn(const float* Z, int64_t rows, int d, int d_ff, const float* gate_t, const float* up_t,
                      const float* down_t, float* H, float* F, hipStream_t s) {
  if (d % 32 != 0 || d_ff % 32 != 0) return hipErrorInvalidValue;
  const unsigned gy = (unsigned)((rows + 15) / 16);
  hipLaunchKernelGGL((small_gemm_kernel<EPI_GATED, float>), dim3(d_ff / 32, gy), dim3(64), 0, s, Z, rows, d, gate_t,
                     up_t, d_ff, H, 1.f, 0, 0);
  // the down projection has few output columns and a long reduction: one 16 x 16 block per wave
  hipLaunchKernelGGL((small_gemm_kernel<EPI_STORE, float, 1>), dim3(d / 16, gy), dim3(64), 0, s, H, rows, d_ff, down_t,
                     nullptr, d, F, 1.f, 0, 0);
  return hipGetLastError();
}

}  // namespace sa
