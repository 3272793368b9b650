// Backward of the prototype-axis softmax for the float32 backward pass: one
// row of the k-wide score and upstream matrices per wave.
//
// For behaviour i with scores s_ij = tau (P W_Q)_j . (x_i W_K) over the
// prototypes j (natural-log units) and upstream values da_ij = G_j . x_i, the
// softmax of section 2.1 (SequenceO1 close-reading page: weights over the
// prototypes sum to one) gives a_ij = exp(s_ij - m_i) / l_i, and its
// Jacobian-vector product ds_ij = a_ij (da_ij - c_i) with c_i = sum_j a_ij
// da_ij (chain rule; the page prints no backward equations).
#include <hip/hip_runtime.h>

#include "sa_internal.h"

namespace sa {
namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// VPL values per lane: column j = lane + 64 v of the row
template <int VPL>
__global__ __launch_bounds__(256) void softmax_grad_rows_kernel(float* __restrict__ S, float* __restrict__ DA,
                                                                int64_t rows, int k, int ld) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float* const srow = S + row * ld;
  float* const drow = DA + row * ld;
  float s[VPL], da[VPL];
  float m = -INFINITY;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int j = lane + 64 * v;
    s[v] = j < k ? srow[j] : -INFINITY;
    da[v] = j < k ? drow[j] : 0.f;
    m = fmaxf(m, s[v]);
  }
  m = wave_max(m);
  float l = 0.f;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    s[v] = lane + 64 * v < k ? expf(s[v] - m) : 0.f;
    l += s[v];
  }
  const float inv = 1.f / wave_sum(l);
  float c = 0.f;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    s[v] *= inv;
    c += s[v] * da[v];
  }
  c = wave_sum(c);
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int j = lane + 64 * v;
    if (j < ld) {
      srow[j] = s[v];
      drow[j] = s[v] * (da[v] - c);
    }
  }
}

}  // namespace

hipError_t launch_softmax_grad_rows(float* S, float* DA, int64_t rows, int k, int ld, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (k < 1 || ld < k || ld > 1024) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  const int vpl = (ld + 63) / 64;
  if (vpl <= 1)
    hipLaunchKernelGGL(softmax_grad_rows_kernel<1>, grid, block, 0, stream, S, DA, rows, k, ld);
  else if (vpl <= 2)
    hipLaunchKernelGGL(softmax_grad_rows_kernel<2>, grid, block, 0, stream, S, DA, rows, k, ld);
  else if (vpl <= 4)
    hipLaunchKernelGGL(softmax_grad_rows_kernel<4>, grid, block, 0, stream, S, DA, rows, k, ld);
  else if (vpl <= 8)
    hipLaunchKernelGGL(softmax_grad_rows_kernel<8>, grid, block, 0, stream, S, DA, rows, k, ld);
  else
    hipLaunchKernelGGL(softmax_grad_rows_kernel<16>, grid, block, 0, stream, S, DA, rows, k, ld);
  return hipGetLastError();
}

}  // namespace sa
