// Support kernels: weight fold, split-n partial reduction, and the launch
// dispatchers of the fused pass.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "sa_internal.h"

namespace sa {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

// ------------------------------------------------------------------ fold
// Q = P W_Q (k x d, float32): the prototype queries of the affinity
// (SequenceO1 page, section 2.1).
template <typename T>
__global__ __launch_bounds__(256) void fold_q_kernel(const T* P, const T* WQ, int k, int d, float* Q) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= k * d) return;
  const int j = idx / d, b = idx % d;
  float s = 0.f;
  for (int a = 0; a < d; ++a) s = fmaf(to_f32(P[j * d + a]), to_f32(WQ[a * d + b]), s);
  Q[idx] = s;
}

// M[j][c] = scale * sum_b Q[j][b] W_K[c][b]  (= scale * (P W_Q W_K^T)[j][c]),
// rounded once to T; padded rows k..k_pad-1 are zero.
template <typename T>
__global__ __launch_bounds__(256) void fold_m_kernel(const float* Q, const T* WK, float scale, int k, int k_pad, int d,
                                                     T* M) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= k_pad * d) return;
  const int j = idx / d, c = idx % d;
  float s = 0.f;
  if (j < k) {
    for (int b = 0; b < d; ++b) s = fmaf(Q[j * d + b], to_f32(WK[c * d + b]), s);
    s *= scale;
  }
  M[idx] = (T)s;
}

template <typename T>
__global__ __launch_bounds__(256) void unfold_kernel(const T* M, int k, int d, float* dst) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= k * d) return;
  dst[idx] = to_f32(M[idx]);
}

hipError_t launch_fold(int dtype, const void* P, const void* WQ, const void* WK, float scale, int k, int k_pad, int d,
                       float* tmp, void* M, hipStream_t stream) {
  const int gq = (k * d + 255) / 256, gm = (k_pad * d + 255) / 256;
  if (dtype == 1) {
    hipLaunchKernelGGL(fold_q_kernel<bf16>, dim3(gq), dim3(256), 0, stream, (const bf16*)P, (const bf16*)WQ, k, d, tmp);
    hipLaunchKernelGGL(fold_m_kernel<bf16>, dim3(gm), dim3(256), 0, stream, tmp, (const bf16*)WK, scale, k, k_pad, d,
                       (bf16*)M);
  } else {
    hipLaunchKernelGGL(fold_q_kernel<float>, dim3(gq), dim3(256), 0, stream, (const float*)P, (const float*)WQ, k, d,
                       tmp);
    hipLaunchKernelGGL(fold_m_kernel<float>, dim3(gm), dim3(256), 0, stream, tmp, (const float*)WK, scale, k, k_pad,
                       d, (float*)M);
  }
  return hipGetLastError();
}

hipError_t launch_unfold(int dtype, const void* M, int k, int d, float* dst, hipStream_t stream) {
  const int gr = (k * d + 255) / 256;
  if (dtype == 1)
    hipLaunchKernelGGL(unfold_kernel<bf16>, dim3(gr), dim3(256), 0, stream, (const bf16*)M, k, d, dst);
  else
    hipLaunchKernelGGL(unfold_kernel<float>, dim3(gr), dim3(256), 0, stream, (const float*)M, k, d, dst);
  return hipGetLastError();
}

// Zero fill of a device buffer (a kernel rather than a memset node, so a
// stream capture of the calling code records only kernels).
__global__ __launch_bounds__(256) void zero_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
  const int64_t words = (int64_t)(bytes / 4);
  if (words == 0) return hipSuccess;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

// --------------------------------------------------------------- reduce
// out[u] = sum over the work groups b that touched user u of partial[b + u],
// in a fixed order (so results are bitwise reproducible).  Work
// group b of G covers rows [floor(b*R/G), floor((b+1)*R/G)), so the group
// holding row r is floor(((r+1)*G - 1) / R).  A user with no rows gets zeros.
//
// Partial slots hold each lane's accumulator registers in order,
// [wj][jb][cb][lane][4]; float4 number p of a slot holds prototypes
// wj*kw + 16*jb + 4*(lane/16) + 0..3 at column 16*cb + lane%16.
//
// One thread per float4 of a slot and per share of the user's groups: a
// work group of `shares` waves (1..8, chosen from the slots per user) covers
// 64 float4s; wave q sums its contiguous share of the slots b0..b1 (four
// running sums, four loads in flight), and the shares are added through LDS
// in a fixed order, so many waves stream the partials of a user with many
// groups while users with few groups do not pay for idle waves.
constexpr int kReduceLanes = 64;
constexpr int kReduceShares = 8;

__global__ __launch_bounds__(kReduceLanes * kReduceShares) void reduce_kernel(ReduceArgs a) {
  __shared__ f32x4 part_sum[kReduceShares][kReduceLanes];
  const int shares = blockDim.x / kReduceLanes;
  const int u = blockIdx.y;
  const int blk = blockIdx.z;  // prototype block (two-phase pass; 0 otherwise)
  const int slot_f4 = a.k_pad * a.d / 4;
  const int lane = threadIdx.x % kReduceLanes;
  const int q = threadIdx.x / kReduceLanes;
  const int p = blockIdx.x * kReduceLanes + lane;
  const int64_t r0 = a.offsets[u], r1 = a.offsets[u + 1];
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if (r1 > r0 && p < slot_f4) {
    const int64_t G = a.groups, R = a.rows;
    const int64_t b0 = ((r0 + 1) * G - 1) / R;
    const int64_t b1 = (r1 * G - 1) / R;
    const int64_t n = b1 - b0 + 1;
    const int64_t q0 = n * q / shares, q1 = n * (q + 1) / shares;
    const f32x4* part =
        reinterpret_cast<const f32x4*>(a.partial) + ((int64_t)blk * (G + a.users) + b0 + u) * slot_f4 + p;
    f32x4 t0 = s, t1 = s, t2 = s, t3 = s;
    int64_t i = q0;
    for (; i + 4 <= q1; i += 4) {
      t0 += __builtin_nontemporal_load(part + (i + 0) * slot_f4);
      t1 += __builtin_nontemporal_load(part + (i + 1) * slot_f4);
      t2 += __builtin_nontemporal_load(part + (i + 2) * slot_f4);
      t3 += __builtin_nontemporal_load(part + (i + 3) * slot_f4);
    }
    if (i + 0 < q1) t0 += __builtin_nontemporal_load(part + (i + 0) * slot_f4);
    if (i + 1 < q1) t1 += __builtin_nontemporal_load(part + (i + 1) * slot_f4);
    if (i + 2 < q1) t2 += __builtin_nontemporal_load(part + (i + 2) * slot_f4);
    s = (t0 + t1) + (t2 + t3);
  }
  part_sum[q][lane] = s;
  __syncthreads();
  if (q != 0 || p >= slot_f4) return;
#pragma unroll
  for (int w = 1; w < kReduceShares; ++w)
    if (w < shares) s += part_sum[w][lane];
  int j0, c;
  const int l = p & 63;
  if (a.layout == 1) {
    // 32x32 products: float4 ((jb CB + cb) 4 + vq) 64 + lane holds prototypes
    // 32 jb + 8 vq + 4 (lane / 32) + 0..3 at column 32 cb + lane % 32
    int t = p >> 6;
    const int cbs = a.d / 32;
    const int vq = t & 3;
    t >>= 2;
    const int cb = t % cbs;
    const int jb = t / cbs;
    j0 = blk * a.k_pad + 32 * jb + 8 * vq + 4 * (l >> 5);
    c = 32 * cb + (l & 31);
  } else {
    int t = p >> 6;
    const int cbs = a.d / 16, jbs = a.kw / 16;
    const int cb = t % cbs;
    t /= cbs;
    const int jb = t % jbs;
    const int wj = t / jbs;
    j0 = blk * a.k_pad + wj * a.kw + 16 * jb + 4 * (l >> 4);
    c = 16 * cb + (l & 15);
  }
  float* o = a.out + (int64_t)u * a.k * a.d;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (j0 + r < a.k) o[(int64_t)(j0 + r) * a.d + c] = s[r];
}

// Merge of the two-phase pass's per-block statistics: L[i] = log2 sum_b
// 2^Lb[b][i] (a log-sum-exp over the blocks, shifted by their maximum).
__global__ __launch_bounds__(256) void lse_merge_kernel(const float* Lb, int64_t rows, int blocks, float* L) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows) return;
  float m = -INFINITY;
  for (int b = 0; b < blocks; ++b) m = fmaxf(m, Lb[(int64_t)b * rows + i]);
  float s = 0.f;
  for (int b = 0; b < blocks; ++b) s += exp2f(Lb[(int64_t)b * rows + i] - m);
  L[i] = m + log2f(s);
}

hipError_t launch_lse_merge(const float* Lb, int64_t rows, int blocks, float* L, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, Lb, rows, blocks, L);
  return hipGetLastError();
}

// Comparator (softmax over the history axis): slot s of user u holds, for
// every prototype j, acc_s = sum_i 2^(s'_ji - m_s) x_i over its rows (lane
// layout as above), the maximum m_s[j] it used and l_s[j] = sum_i 2^(s'_ji -
// m_s).  The user's summary is sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M)
// l_s with M the largest m_s; zero when no slot saw a row.  One thread per
// float4 of the slot layout (four prototypes, one column) and per share of
// the user's slots; each share merges its slots in order with a running
// maximum, then share 0 merges the shares in order (fixed order throughout).
struct HistPart {
  float m, l, a;
};
__device__ __forceinline__ void hist_merge(HistPart& x, float m, float l, float a) {
  if (m == -INFINITY) return;  // nothing seen
  if (m <= x.m) {
    const float sb = __builtin_amdgcn_exp2f(m - x.m);
    x.a += a * sb;
    x.l += l * sb;
  } else {
    const float sa = __builtin_amdgcn_exp2f(x.m - m);  // 0 when x saw nothing (x.m = -inf)
    x.a = x.a * sa + a;
    x.l = x.l * sa + l;
    x.m = m;
  }
}

__global__ __launch_bounds__(kReduceLanes * kReduceShares) void reduce_history_kernel(ReduceArgs a) {
  __shared__ HistPart part[kReduceShares][kReduceLanes][4];
  const int shares = blockDim.x / kReduceLanes;
  const int u = blockIdx.y;
  const int blk = blockIdx.z;  // prototype block (its slots follow the groups + users slots of block blk - 1)
  const int slot_f4 = a.k_pad * a.d / 4;
  const int64_t slot_floats = (int64_t)a.k_pad * (a.d + 2);
  const int lane = threadIdx.x % kReduceLanes;
  const int q = threadIdx.x / kReduceLanes;
  const int p = blockIdx.x * kReduceLanes + lane;
  const int l = p & 63;
  int j0, c;  // first of the float4's four prototypes (within the block), its column
  if (a.layout == 1) {
    // 32x32 products: float4 ((jb CB + cb) 4 + vq) 64 + lane holds prototypes
    // 32 jb + 8 vq + 4 (lane / 32) + 0..3 at column 32 cb + lane % 32
    int t = p >> 6;
    const int cbs = a.d / 32;
    const int vq = t & 3;
    t >>= 2;
    const int cb = t % cbs;
    const int jb = t / cbs;
    j0 = 32 * jb + 8 * vq + 4 * (l >> 5);
    c = 32 * cb + (l & 31);
  } else {
    int t = p >> 6;
    const int cbs = a.d / 16, jbs = a.kw / 16;
    const int cb = t % cbs;
    t /= cbs;
    const int jb = t % jbs;
    const int wj = t / jbs;
    j0 = wj * a.kw + 16 * jb + 4 * (l >> 4);
    c = 16 * cb + (l & 15);
  }
  HistPart x[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = HistPart{-INFINITY, 0.f, 0.f};
  const int64_t r0 = a.offsets[u], r1 = a.offsets[u + 1];
  if (r1 > r0 && p < slot_f4) {
    const int64_t G = a.groups, R = a.rows;
    const int64_t b0 = ((r0 + 1) * G - 1) / R;
    const int64_t b1 = (r1 * G - 1) / R;
    const int64_t n = b1 - b0 + 1;
    const int64_t q0 = n * q / shares, q1 = n * (q + 1) / shares;
    for (int64_t i = q0; i < q1; ++i) {
      const float* slot = a.partial + ((int64_t)blk * (G + a.users) + b0 + i + u) * slot_floats;
      const f32x4 v = reinterpret_cast<const f32x4*>(slot)[p];
      const float* stats = slot + (int64_t)a.k_pad * a.d;
      const f32x4 ms = *reinterpret_cast<const f32x4*>(stats + j0);
      const f32x4 ls = *reinterpret_cast<const f32x4*>(stats + a.k_pad + j0);
#pragma unroll
      for (int r = 0; r < 4; ++r) hist_merge(x[r], ms[r], ls[r], v[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) part[q][lane][r] = x[r];
  __syncthreads();
  if (q != 0 || p >= slot_f4) return;
  for (int w = 1; w < shares; ++w)
#pragma unroll
    for (int r = 0; r < 4; ++r) hist_merge(x[r], part[w][lane][r].m, part[w][lane][r].l, part[w][lane][r].a);
  float* o = a.out + (int64_t)u * a.k * a.d;
  const int jg = blk * a.k_pad + j0;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (jg + r < a.k) o[(int64_t)(jg + r) * a.d + c] = x[r].l > 0.f ? x[r].a / x[r].l : 0.f;
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  const int64_t per_user = (a.groups + a.users) / (a.users > 0 ? a.users : 1);
  if (a.history_softmax) {
    int shares = 1;
    while (shares < kReduceShares && 8 * shares < per_user) shares *= 2;
    const dim3 grid((a.k_pad * a.d / 4 + kReduceLanes - 1) / kReduceLanes, a.users, a.blocks > 1 ? a.blocks : 1),
        block(kReduceLanes * shares);
    if (start || stop)
      hipExtLaunchKernelGGL(reduce_history_kernel, grid, block, 0, stream, start, stop, 0, a);
    else
      hipLaunchKernelGGL(reduce_history_kernel, grid, block, 0, stream, a);
    return hipGetLastError();
  }
  const int slot_f4 = a.k_pad * a.d / 4;
  int shares = 1;
  while (shares < kReduceShares && 8 * shares <= per_user) shares *= 2;
  const dim3 grid((slot_f4 + kReduceLanes - 1) / kReduceLanes, a.users, a.blocks > 1 ? a.blocks : 1),
      block(kReduceLanes * shares);
  if (start || stop)
    hipExtLaunchKernelGGL(reduce_kernel, grid, block, 0, stream, start, stop, 0, a);
  else
    hipLaunchKernelGGL(reduce_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ dispatch
static DispatchFn plan_group(const Plan& p) {
  if (p.kind == 2 || p.kind == 3) return p.dtype == 1 && p.d == 128 ? dispatch_stream_d128 : nullptr;
  if (p.kind == 1) {
    if (p.dtype != 1) return nullptr;
    if (p.d == 64) return dispatch_stream_d64;
    if (p.d == 128) return dispatch_stream_d128;
    return nullptr;
  }
  if (p.dtype == 1) {
    if (p.d == 64) return dispatch_bf16_d64;
    if (p.d == 128) return dispatch_bf16_d128;
  } else {
    if (p.d == 64) return dispatch_f32_d64;
    if (p.d == 128) return dispatch_f32_d128;
  }
  return nullptr;
}

hipError_t launch_fused(const Plan& plan, const FusedArgs& args, int groups, hipStream_t stream, hipEvent_t start,
                        hipEvent_t stop) {
  DispatchFn f = plan_group(plan);
  const Launch l{groups, stream, start, stop};
  return f ? f(plan, args, l, nullptr) : hipErrorInvalidValue;
}

// ------------------------------------------------- allocation-free workspace
// Partial sketches of sa_compress_batch_noalloc: a fixed device array that
// the code object brings with it, so that call never allocates.  Every GPU
// the library runs on holds its own copy at its own address until the
// process ends; all calls on one GPU share it.  In host code `scratch` names
// a host-side stand-in, never the device memory: its device address is taken
// once per device with hipGetSymbolAddress (that device current) and only
// that address is handed to kernels.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

hipError_t noalloc_scratch(int device, float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[device] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;  // the caller makes `device` current first
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[device] = static_cast<float*>(p);
  }
  *ptr = addr[device];
  return hipSuccess;
}

hipError_t fused_occupancy(const Plan& plan, int* n) {
  DispatchFn f = plan_group(plan);
  static const FusedArgs unused{};
  const Launch l{0, nullptr, nullptr, nullptr};
  return f ? f(plan, unused, l, n) : hipErrorInvalidValue;
}

}  // namespace sa
