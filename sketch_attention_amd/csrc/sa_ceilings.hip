// On-device ceilings that the roofline fractions are read against: a matrix-
// core loop (bf16 16x16x32 products, independent accumulators, every compute
// unit busy), float32 FMA and exp2 loops on the vector ALUs, and a streaming
// copy through HBM.  Each is timed with HIP events on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sa.h"

#define SA_API extern "C" __attribute__((visibility("default")))

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMfmaChains = 8;   // independent accumulators per wave
constexpr int kValuChains = 8;

// Every wave issues `iters` x kMfmaChains independent bf16 products; the
// operands come from the thread index so nothing folds away, and one lane
// stores a checksum so the products are live.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* sink) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((threadIdx.x + e) & 7);
    b[e] = (__bf16)(float)((threadIdx.x * 3 + e) & 5);
  }
  f32x4 c[kMfmaChains];
  for (int i = 0; i < kMfmaChains; ++i) c[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kMfmaChains; ++i) c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[i], 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < kMfmaChains; ++i) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
  if (s == 1234.5f) sink[blockIdx.x] = s;  // never true for these operands; keeps the loop live
}

// The same with 32x32x16 products (16 accumulator registers each).
__global__ __launch_bounds__(256) void mfma32_loop_kernel(int iters, float* sink) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((threadIdx.x + e) & 7);
    b[e] = (__bf16)(float)((threadIdx.x * 3 + e) & 5);
  }
  f32x16 c[kMfmaChains / 2];
  for (int i = 0; i < kMfmaChains / 2; ++i)
    for (int j = 0; j < 16; ++j) c[i][j] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kMfmaChains / 2; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[i], 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < kMfmaChains / 2; ++i) s += c[i][0] + c[i][15];
  if (s == 1234.5f) sink[blockIdx.x] = s;
}

// kind 0: fma chains; kind 1: exp2 chains (the hardware exp2, as the softmax
// uses it; x = 2^-x converges, the negation is a free input modifier)
__global__ __launch_bounds__(256) void valu_loop_kernel(int iters, int kind, float* sink) {
  float x[kValuChains];
  for (int i = 0; i < kValuChains; ++i) x[i] = 0.001f * (float)(threadIdx.x + i);
  if (kind == 0) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < kValuChains; ++i) x[i] = __builtin_fmaf(x[i], 0.999f, 0.0001f);
  } else {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int i = 0; i < kValuChains; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
  }
  float s = 0.f;
  for (int i = 0; i < kValuChains; ++i) s += x[i];
  if (s == 1234.5f) sink[blockIdx.x] = s;
}

// dst = src over n 16-byte vectors, grid-stride
__global__ __launch_bounds__(256) void copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) dst[i] = src[i];
}

// Read-only stream: each thread XORs the bits of U independent 16-byte
// loads per iteration (grid-stride), so the loads stay in flight together;
// one lane stores only if the result hits a value the zeroed buffer never
// gives.
template <int U>
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ src, int64_t n, unsigned* sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint4 acc = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * stride < n; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc.x ^= v[u].x;
      acc.y ^= v[u].y;
      acc.z ^= v[u].z;
      acc.w ^= v[u].w;
    }
  }
  for (; i < n; i += stride) {
    const uint4 a = src[i];
    acc.x ^= a.x;
    acc.y ^= a.y;
    acc.z ^= a.z;
    acc.w ^= a.w;
  }
  if ((acc.x | acc.y | acc.z | acc.w) == 0x5a5a5a5au) sink[blockIdx.x] = acc.x;
}

}  // namespace

SA_API sa_status sa_measure_hbm_read(double* read_gbs, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return SA_ERR_DEVICE;
  const int cus = prop.multiProcessorCount;
  const int64_t bytes = int64_t(1) << 30;  // four times the Infinity Cache
  const int64_t n = bytes / 16;
  void* buf = nullptr;
  unsigned* sink = nullptr;
  if (hipMalloc(&buf, bytes) != hipSuccess) return SA_ERR_OUT_OF_MEMORY;
  if (hipMalloc(&sink, (size_t)cus * 32 * sizeof(unsigned)) != hipSuccess) {
    (void)hipFree(buf);
    return SA_ERR_OUT_OF_MEMORY;
  }
  hipEvent_t e0 = nullptr, e1 = nullptr;
  sa_status st = SA_OK;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) st = SA_ERR_DEVICE;
  if (st == SA_OK && hipMemsetAsync(buf, 0, bytes, s) != hipSuccess) st = SA_ERR_DEVICE;
  double best = 0.0;
  // the best over four or eight loads in flight per thread and 4 to 32 work
  // groups of four waves per compute unit
  for (int cfg = 0; st == SA_OK && cfg < 8; ++cfg) {
    const dim3 grid(cus * (4 << (cfg % 4)));
    const bool eight = cfg >= 4;
    const uint4* src = static_cast<const uint4*>(buf);
    auto launch = [&] {
      if (eight)
        hipLaunchKernelGGL(read_kernel<8>, grid, dim3(256), 0, s, src, n, sink);
      else
        hipLaunchKernelGGL(read_kernel<4>, grid, dim3(256), 0, s, src, n, sink);
    };
    launch();  // warm-up
    const int reps = 10;
    if (hipEventRecord(e0, s) != hipSuccess) { st = SA_ERR_DEVICE; break; }
    for (int r = 0; r < reps; ++r) launch();
    float ms = 0.f;
    if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0.f) {
      st = SA_ERR_DEVICE;
      break;
    }
    const double gbs = (double)bytes * reps / (ms * 1e-3) / 1e9;
    if (gbs > best) best = gbs;
  }
  if (hipGetLastError() != hipSuccess) st = SA_ERR_DEVICE;
  if (st == SA_OK && read_gbs) *read_gbs = best;
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipStreamSynchronize(s);
  (void)hipFree(sink);
  (void)hipFree(buf);
  return st;
}

SA_API sa_status sa_measure_ceilings(double* mfma_bf16_tflops, double* mfma_bf16_32x32_tflops, double* valu_fma_tflops,
                                     double* exp2_per_sec, double* copy_gbs, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return SA_ERR_DEVICE;
  const int cus = prop.multiProcessorCount;
  const int groups = cus * 8;  // 4 waves each: 8 waves per SIMD on every CU
  const int iters = 4096;
  float* sink = nullptr;
  void* buf = nullptr;
  const int64_t copy_bytes = int64_t(1) << 30;  // read 1 GiB, write 1 GiB (four times the Infinity Cache)
  hipEvent_t e0 = nullptr, e1 = nullptr;
  sa_status st = SA_OK;
  auto timed = [&](auto launch, int reps) -> double {
    launch();  // warm-up
    if (hipEventRecord(e0, s) != hipSuccess) return -1.0;
    for (int r = 0; r < reps; ++r) launch();
    if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return -1.0;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return -1.0;
    return ms * 1e-3 / reps;
  };
  if (hipMalloc(&sink, groups * sizeof(float)) != hipSuccess) return SA_ERR_OUT_OF_MEMORY;
  if (hipMalloc(&buf, 2 * copy_bytes) != hipSuccess) {
    (void)hipFree(sink);
    return SA_ERR_OUT_OF_MEMORY;
  }
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) st = SA_ERR_DEVICE;
  if (st == SA_OK && hipMemsetAsync(buf, 0, 2 * copy_bytes, s) != hipSuccess) st = SA_ERR_DEVICE;
  if (st == SA_OK) {
    const double t = timed([&] { hipLaunchKernelGGL(mfma_loop_kernel, dim3(groups), dim3(256), 0, s, iters, sink); }, 5);
    const double flops = (double)groups * 4 * iters * kMfmaChains * 16.0 * 16 * 32 * 2;
    if (t <= 0) st = SA_ERR_DEVICE;
    else if (mfma_bf16_tflops) *mfma_bf16_tflops = flops / t / 1e12;
  }
  if (st == SA_OK) {
    const double t =
        timed([&] { hipLaunchKernelGGL(mfma32_loop_kernel, dim3(groups), dim3(256), 0, s, iters, sink); }, 5);
    const double flops = (double)groups * 4 * iters * (kMfmaChains / 2) * 32.0 * 32 * 16 * 2;
    if (t <= 0) st = SA_ERR_DEVICE;
    else if (mfma_bf16_32x32_tflops) *mfma_bf16_32x32_tflops = flops / t / 1e12;
  }
  if (st == SA_OK) {
    const double t =
        timed([&] { hipLaunchKernelGGL(valu_loop_kernel, dim3(groups), dim3(256), 0, s, iters, 0, sink); }, 5);
    const double flops = (double)groups * 256 * iters * kValuChains * 2.0;
    if (t <= 0) st = SA_ERR_DEVICE;
    else if (valu_fma_tflops) *valu_fma_tflops = flops / t / 1e12;
  }
  if (st == SA_OK) {
    const double t =
        timed([&] { hipLaunchKernelGGL(valu_loop_kernel, dim3(groups), dim3(256), 0, s, iters, 1, sink); }, 5);
    const double n = (double)groups * 256 * iters * kValuChains;
    if (t <= 0) st = SA_ERR_DEVICE;
    else if (exp2_per_sec) *exp2_per_sec = n / t;
  }
  if (st == SA_OK) {
    const int64_t n = copy_bytes / 16;
    const f32x4* src = static_cast<const f32x4*>(buf);
    f32x4* dst = reinterpret_cast<f32x4*>(static_cast<char*>(buf) + copy_bytes);
    const double t = timed([&] { hipLaunchKernelGGL(copy_kernel, dim3(cus * 16), dim3(256), 0, s, src, dst, n); }, 10);
    if (t <= 0) st = SA_ERR_DEVICE;
    else if (copy_gbs) *copy_gbs = 2.0 * copy_bytes / t / 1e9;
  }
  if (hipGetLastError() != hipSuccess) st = SA_ERR_DEVICE;
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  (void)hipStreamSynchronize(s);
  (void)hipFree(buf);
  (void)hipFree(sink);
  return st;
}
