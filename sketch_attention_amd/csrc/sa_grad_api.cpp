// Host side of the backward-pass entry points declared in include/sa.h
// (sa_grad_*): argument validation, the weight preparation done once per
// handle, the workspace, and the launch sequence per batch (pack, row
// statistics + dQ', split-n reduction, dX, then the small weight products).
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <new>
#include <vector>

#include "sa.h"
#include "sa_grad.h"
#include "sa_internal.h"

#define SA_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr double kLog2e = 1.4426950408889634073599246810019;
constexpr int64_t kF32ChunkRows = 65536;  // float32 path: rows per pass of one user

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

struct EventPair {
  hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};  // stats start/stop, dx start/stop
};

}  // namespace

struct sa_grad_s {
  int device = 0;
  int cu_count = 0;
  int d = 0, k = 0, k_pad = 0, waves = 0;
  int blocks = 1;  // prototype blocks of pass 1 (k_pad = blocks * waves * 32)
  int stats_per_cu = 1, dx_per_cu = 1;
  float tau = 0.f;
  void* M = nullptr;     // bf16 [k_pad][d], tau log2(e) P W_Q W_K^T
  void* Qp = nullptr;    // bf16 [k_pad][d], tau P W_Q W_K^T
  float* Q = nullptr;    // float32 [k][d], P W_Q
  float* P32 = nullptr;  // float32 copies of the weights
  float* WQ32 = nullptr;
  float* WK32 = nullptr;
  float* dq = nullptr;   // float32 [3][k][d]: dQ' sum, one launch's dQ', dQ
  // workspace, grown on demand
  float* stats = nullptr;
  size_t stats_rows = 0;
  float* bstats = nullptr;  // per-block statistics of pass 1 (more than one block)
  size_t bstats_floats = 0;
  float* partial = nullptr;
  size_t partial_floats = 0;
  void* packed = nullptr;
  size_t packed_bytes = 0;
  // float32 path: prototypes padded to k32 (a multiple of 32); Qp32 [k32][d] = tau P W_Q W_K^T with zero
  // rows past k, QpT = Qp32^T [d][k32]; per call GT [d][k32], G32 [k32][d] (one user's upstream gradient,
  // zero-padded); per pass of at most kF32ChunkRows rows S, DA [rows][k32], DST [k32][rows16], XT [d][rows16]
  sa_dtype dtype = SA_BF16;
  int k32 = 0;
  float* Qp32 = nullptr;
  float* QpT = nullptr;
  float* f32ws = nullptr;  // GT, G32, D1 [k32][d], S, DA, DST, XT
  size_t f32ws_floats = 0;
  bool timing = false;
  std::vector<EventPair> pending, spare;
};

namespace {

template <typename T>
bool grow(T*& p, size_t& have, size_t need, size_t elem) {
  if (need <= have) return true;
  if (p) (void)hipFree(p);
  p = nullptr;
  have = 0;
  if (hipMalloc(reinterpret_cast<void**>(&p), need * elem) != hipSuccess) return false;
  have = need;
  return true;
}

void free_handle(sa_grad_s* h) {
  for (void* p : {(void*)h->M, (void*)h->Qp, (void*)h->Q, (void*)h->P32, (void*)h->WQ32, (void*)h->WK32,
                  (void*)h->dq, (void*)h->stats, (void*)h->bstats, (void*)h->partial, h->packed, (void*)h->Qp32,
                  (void*)h->QpT, (void*)h->f32ws})
    if (p) (void)hipFree(p);
  for (auto* v : {&h->pending, &h->spare})
    for (auto& e : *v)
      for (auto& x : e.ev)
        if (x) (void)hipEventDestroy(x);
  delete h;
}

}  // namespace

SA_API sa_status sa_grad_check_config(int32_t d, int32_t k, float tau, sa_dtype dtype) {
  sa_status st = sa_check_config(d, k, tau, dtype);
  if (st != SA_OK) return st;
  if (dtype == SA_F32) return SA_OK;  // any k of sa_check_config
  if (sa::grad_stats_waves(k) == 0) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

SA_API sa_status sa_grad_create(sa_grad* out, int32_t d, int32_t k, float tau, sa_dtype dtype, const void* P,
                                const void* W_Q, const void* W_K, void* stream) {
  if (out == nullptr) return SA_ERR_INVALID_ARG;
  *out = nullptr;
  sa_status st = sa_grad_check_config(d, k, tau, dtype);
  if (st != SA_OK) return st;
  if (P == nullptr || W_Q == nullptr || W_K == nullptr) return SA_ERR_INVALID_ARG;
  if (!aligned16(P) || !aligned16(W_Q) || !aligned16(W_K)) return SA_ERR_INVALID_ARG;
  sa_grad_s* h = new (std::nothrow) sa_grad_s();
  if (h == nullptr) return SA_ERR_OUT_OF_MEMORY;
  hipStream_t s = static_cast<hipStream_t>(stream);
  h->d = d;
  h->k = k;
  h->tau = tau;
  h->dtype = dtype;
  if (dtype == SA_F32) {
    h->k32 = 32 * ((k + 31) / 32);
    const size_t kd = (size_t)k * d, k32d = (size_t)h->k32 * d, dd = (size_t)d * d;
    if (hipGetDevice(&h->device) != hipSuccess || hipMalloc(&h->Q, kd * 4) != hipSuccess ||
        hipMalloc(&h->P32, kd * 4) != hipSuccess || hipMalloc(&h->WQ32, dd * 4) != hipSuccess ||
        hipMalloc(&h->WK32, dd * 4) != hipSuccess || hipMalloc(&h->dq, 3 * kd * 4) != hipSuccess ||
        hipMalloc(&h->Qp32, k32d * 4) != hipSuccess || hipMalloc(&h->QpT, k32d * 4) != hipSuccess) {
      free_handle(h);
      return SA_ERR_OUT_OF_MEMORY;
    }
    hipError_t e = sa::launch_fold(0, P, W_Q, W_K, tau, k, h->k32, d, h->Q, h->Qp32, s);
    if (e == hipSuccess) e = sa::launch_transpose_pad(h->Qp32, h->k32, d, h->k32, h->QpT, s);
    if (e == hipSuccess) e = sa::launch_unfold(0, P, k, d, h->P32, s);
    if (e == hipSuccess) e = sa::launch_unfold(0, W_Q, d, d, h->WQ32, s);
    if (e == hipSuccess) e = sa::launch_unfold(0, W_K, d, d, h->WK32, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      free_handle(h);
      return SA_ERR_DEVICE;
    }
    *out = h;
    return SA_OK;
  }
  h->waves = sa::grad_stats_waves(k);
  h->blocks = sa::grad_stats_blocks(k);
  h->k_pad = sa::kGradKW * h->waves * h->blocks;
  hipDeviceProp_t prop;
  if (hipGetDevice(&h->device) != hipSuccess || hipGetDeviceProperties(&prop, h->device) != hipSuccess ||
      sa::grad_occupancy(d, h->waves, &h->stats_per_cu, &h->dx_per_cu) != hipSuccess || h->stats_per_cu < 1 ||
      h->dx_per_cu < 1) {
    free_handle(h);
    return SA_ERR_DEVICE;
  }
  h->cu_count = prop.multiProcessorCount;
  const size_t kd = (size_t)k * d, kpd = (size_t)h->k_pad * d, dd = (size_t)d * d;
  if (hipMalloc(&h->M, kpd * 2) != hipSuccess || hipMalloc(&h->Qp, kpd * 2) != hipSuccess ||
      hipMalloc(&h->Q, kd * 4) != hipSuccess || hipMalloc(&h->P32, kd * 4) != hipSuccess ||
      hipMalloc(&h->WQ32, dd * 4) != hipSuccess || hipMalloc(&h->WK32, dd * 4) != hipSuccess ||
      hipMalloc(&h->dq, 3 * kd * 4) != hipSuccess) {
    free_handle(h);
    return SA_ERR_OUT_OF_MEMORY;
  }
  hipError_t e = sa::launch_fold(1, P, W_Q, W_K, (float)((double)tau * kLog2e), k, h->k_pad, d, h->Q, h->M, s);
  if (e == hipSuccess) e = sa::launch_fold(1, P, W_Q, W_K, tau, k, h->k_pad, d, h->Q, h->Qp, s);
  if (e == hipSuccess) e = sa::launch_unfold(1, P, k, d, h->P32, s);
  if (e == hipSuccess) e = sa::launch_unfold(1, W_Q, d, d, h->WQ32, s);
  if (e == hipSuccess) e = sa::launch_unfold(1, W_K, d, d, h->WK32, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    free_handle(h);
    return SA_ERR_DEVICE;
  }
  *out = h;
  return SA_OK;
}

SA_API void sa_grad_destroy(sa_grad h) {
  if (h == nullptr) return;
  DeviceGuard guard(h->device);
  free_handle(h);
}

namespace {

// float32 backward, per user and per pass of at most kF32ChunkRows rows (additive over rows), with
// float32 matrix-core products (chain rule of section 2.1, as in include/sa.h):
//   S = X Qp^T, DA = X G^T                [rows][k32]
//   A = softmax_j(S), DS = A (DA - c)      (launch_softmax_grad_rows, in place)
//   dX = A G + DS Qp                       [rows][d]
//   D1 += DS^T X                           [k32][d], summed over every user and pass
// then dQ = tau D1 W_K, dW_K = tau D1^T (P W_Q), dP = dQ W_Q^T, dW_Q = P^T dQ.
sa_status compute_f32(sa_grad_s* h, const float* X, const int64_t* offsets, int32_t num_users, const float* G,
                      float* dX, float* grad_P, float* grad_W_Q, float* grad_W_K, hipStream_t s) {
  const int d = h->d, k = h->k, k32 = h->k32;
  const size_t kd = (size_t)k * d, k32d = (size_t)k32 * d;
  int64_t max_rows = 0;
  for (int32_t u = 0; u < num_users; ++u) {
    const int64_t n = offsets[u + 1] - offsets[u];
    max_rows = n > max_rows ? n : max_rows;
  }
  const int64_t rc = max_rows < kF32ChunkRows ? max_rows : kF32ChunkRows;  // rows per pass
  const int64_t rc16 = 16 * ((rc + 15) / 16);
  const size_t need = 3 * k32d + 3 * (size_t)rc16 * k32 + (size_t)d * rc16;
  if (!grow(h->f32ws, h->f32ws_floats, need, sizeof(float))) return SA_ERR_OUT_OF_MEMORY;
  float* const GT = h->f32ws;
  float* const G32 = GT + k32d;
  float* const D1 = G32 + k32d;
  float* const Sb = D1 + k32d;
  float* const DA = Sb + (size_t)rc16 * k32;
  float* const DST = DA + (size_t)rc16 * k32;
  float* const XT = DST + (size_t)rc16 * k32;
  hipError_t e = sa::launch_zero(D1, (int64_t)k32d, s);
  for (int32_t u = 0; e == hipSuccess && u < num_users; ++u) {
    const int64_t r0 = offsets[u], r1 = offsets[u + 1];
    if (r1 == r0) continue;
    // the user's upstream gradient, zero-padded to k32 rows: G^T [d][k32], then G [k32][d]
    e = sa::launch_transpose_pad(G + (size_t)u * kd, k, d, k32, GT, s);
    if (e == hipSuccess) e = sa::launch_transpose_pad(GT, d, k32, d, G32, s);
    for (int64_t a = r0; e == hipSuccess && a < r1; a += rc) {
      const int64_t n = r1 - a < rc ? r1 - a : rc;
      const int64_t n16 = 16 * ((n + 15) / 16);
      const float* Xa = X + a * d;
      float* dXa = dX + a * d;
      e = sa::launch_f32_gemm(Xa, n, d, h->Qp32, k32, Sb, nullptr, false, s);
      if (e == hipSuccess) e = sa::launch_f32_gemm(Xa, n, d, G32, k32, DA, nullptr, false, s);
      if (e == hipSuccess) e = sa::launch_softmax_grad_rows(Sb, DA, n, k, k32, s);
      if (e == hipSuccess) e = sa::launch_f32_gemm(Sb, n, k32, GT, d, dXa, nullptr, false, s);
      if (e == hipSuccess) e = sa::launch_f32_gemm(DA, n, k32, h->QpT, d, dXa, dXa, false, s);
      if (e == hipSuccess) e = sa::launch_transpose_pad(DA, n, k32, n16, DST, s);
      if (e == hipSuccess) e = sa::launch_transpose_pad(Xa, n, d, n16, XT, s);
      if (e == hipSuccess) e = sa::launch_f32_gemm(DST, k32, (int)n16, XT, d, D1, D1, true, s);
    }
  }
  float* const dQ = h->dq + 2 * kd;
  // dQ = tau D1 W_K, dW_K = tau D1^T Q, dP = dQ W_Q^T, dW_Q = P^T dQ (D1's first k rows)
  if (e == hipSuccess)
    e = sa::launch_small_matmuls({D1, d, 1, h->WK32, d, 1, k, d, d, h->tau, dQ},
                                 {D1, 1, d, h->Q, d, 1, d, d, k, h->tau, grad_W_K}, s);
  if (e == hipSuccess)
    e = sa::launch_small_matmuls({dQ, d, 1, h->WQ32, 1, d, k, d, d, 1.f, grad_P},
                                 {h->P32, 1, d, dQ, d, 1, d, d, k, 1.f, grad_W_Q}, s);
  return e == hipSuccess ? SA_OK : SA_ERR_DEVICE;
}

}  // namespace

SA_API sa_status sa_grad_compute(sa_grad h, const void* X, const int64_t* offsets, int32_t num_users,
                                 const float* grad_sketch, void* grad_X, float* grad_P, float* grad_W_Q,
                                 float* grad_W_K, void* stream) {
  if (h == nullptr) return SA_ERR_INVALID_ARG;
  sa_status st = sa_check_batch(h->k, offsets, num_users);
  if (st != SA_OK) return st;
  if (grad_P == nullptr || grad_W_Q == nullptr || grad_W_K == nullptr) return SA_ERR_INVALID_ARG;
  if (!aligned16(grad_P) || !aligned16(grad_W_Q) || !aligned16(grad_W_K)) return SA_ERR_INVALID_ARG;
  const int64_t N = num_users > 0 ? offsets[num_users] : 0;
  if (num_users > 0 && (grad_sketch == nullptr || !aligned16(grad_sketch))) return SA_ERR_INVALID_ARG;
  if (N > 0 && (X == nullptr || grad_X == nullptr || !aligned16(X) || !aligned16(grad_X))) return SA_ERR_INVALID_ARG;

  DeviceGuard guard(h->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (h->dtype == SA_F32) return compute_f32(h, static_cast<const float*>(X), offsets, num_users, grad_sketch,
                                             static_cast<float*>(grad_X), grad_P, grad_W_Q, grad_W_K, s);
  const int d = h->d, k = h->k, k_pad = h->k_pad, chunks = k_pad / sa::kGradKW;
  const int nb = h->blocks, kb = sa::kGradKW * h->waves;  // blocks of pass 1 and prototypes per block
  const size_t kd = (size_t)k * d;
  float* const dq_sum = h->dq;
  float* const dq_one = h->dq + kd;
  float* const dQ = h->dq + 2 * kd;

  // workspace for the largest launch
  int64_t max_rows = 0;
  for (int32_t u0 = 0; u0 < num_users; u0 += sa::kMaxUsersPerLaunch) {
    const int32_t u1 = u0 + sa::kMaxUsersPerLaunch < num_users ? u0 + sa::kMaxUsersPerLaunch : num_users;
    const int64_t r = offsets[u1] - offsets[u0];
    if (r > max_rows) max_rows = r;
  }
  const int64_t stats_groups_max = (int64_t)h->cu_count * h->stats_per_cu;
  const int max_users = num_users < sa::kMaxUsersPerLaunch ? num_users : sa::kMaxUsersPerLaunch;
  if (max_rows > 0) {
    const int64_t g1 = max_rows < stats_groups_max ? max_rows : stats_groups_max;
    if (!grow(h->stats, h->stats_rows, (size_t)max_rows * 4, sizeof(float)) ||
        !grow(h->partial, h->partial_floats, (size_t)nb * (g1 + 1) * kb * d, sizeof(float)) ||
        (nb > 1 && !grow(h->bstats, h->bstats_floats, (size_t)nb * max_rows * 4, sizeof(float))) ||
        !grow(reinterpret_cast<unsigned char*&>(h->packed), h->packed_bytes,
              (size_t)max_users * chunks * sa::grad_chunk_bytes(d), 1))
      return SA_ERR_OUT_OF_MEMORY;
  }

  EventPair ev;
  if (h->timing && max_rows > 0) {
    if (!h->spare.empty()) {
      ev = h->spare.back();
      h->spare.pop_back();
    } else {
      for (auto& x : ev.ev)
        if (hipEventCreateWithFlags(&x, hipEventDisableSystemFence) != hipSuccess) return SA_ERR_DEVICE;
    }
  }
  bool timed = false;

  hipError_t e = hipSuccess;
  bool have_dq = false;  // dq_sum written by a launch
  for (int32_t u0 = 0; e == hipSuccess && u0 < num_users; u0 += sa::kMaxUsersPerLaunch) {
    const int32_t u1 = u0 + sa::kMaxUsersPerLaunch < num_users ? u0 + sa::kMaxUsersPerLaunch : num_users;
    const int32_t users = u1 - u0;
    const int64_t base = offsets[u0];
    const int64_t rows = offsets[u1] - base;
    if (rows == 0) continue;
    const float* G = grad_sketch + (size_t)u0 * kd;
    e = sa::launch_grad_pack(h->M, h->Qp, G, users, k, chunks, d, h->packed, s);
    if (e != hipSuccess) break;

    sa::GradStatsArgs a1{};
    a1.X = static_cast<const unsigned char*>(X) + base * d * 2;
    a1.M = h->M;
    a1.G = G;
    a1.stats = h->stats;
    a1.partial = h->partial;
    a1.rows = rows;
    a1.users = users;
    a1.k = k;
    // SA_GRAD_FORCE_SHIFT=1 routes every row block through the shifted path
    // of the statistics pass (that path otherwise runs only for extreme scores)
    const char* fs = std::getenv("SA_GRAD_FORCE_SHIFT");
    a1.force_shift = fs != nullptr && fs[0] == '1';
    for (int32_t u = 0; u <= users; ++u) a1.offsets[u] = offsets[u0 + u] - base;
    const int g1 = (int)(rows < stats_groups_max ? rows : stats_groups_max);
    const bool last = u1 == num_users;
    const bool time_it = h->timing && last;
    if (nb == 1) {
      e = sa::launch_grad_stats(d, h->waves, a1, g1, s, time_it ? ev.ev[0] : nullptr, time_it ? ev.ev[1] : nullptr);
    } else {
      // blocks of 256 prototypes: their statistics, the merge, then the aggregation with the merged values
      a1.blocks = nb;
      a1.phase = 1;
      a1.stats = h->bstats;
      e = sa::launch_grad_stats(d, h->waves, a1, g1 * nb, s, time_it ? ev.ev[0] : nullptr, nullptr);
      if (e == hipSuccess) e = sa::launch_grad_merge(h->bstats, rows, nb, h->stats, s);
      a1.phase = 2;
      a1.stats = h->stats;
      if (e == hipSuccess)
        e = sa::launch_grad_stats(d, h->waves, a1, g1 * nb, s, nullptr, time_it ? ev.ev[1] : nullptr);
    }
    if (e != hipSuccess) break;

    sa::ReduceArgs r{};
    r.partial = h->partial;
    r.history_softmax = 0;
    r.out = have_dq ? dq_one : dq_sum;
    r.rows = rows;
    r.users = 1;  // one slot per group covering every user: the weights are shared
    r.groups = g1;
    r.k = k;
    r.d = d;
    r.kw = sa::kGradKW;
    r.k_pad = kb;
    r.blocks = nb;
    r.offsets[0] = 0;
    r.offsets[1] = rows;
    e = sa::launch_reduce(r, s);
    if (e == hipSuccess && have_dq) e = sa::launch_add(dq_sum, dq_one, (int64_t)kd, s);
    if (e != hipSuccess) break;
    have_dq = true;

    sa::GradDxArgs a2{};
    a2.X = a1.X;
    a2.stats = h->stats;
    a2.packed = h->packed;
    a2.dX = static_cast<unsigned char*>(grad_X) + base * d * 2;
    a2.rows = rows;
    a2.users = users;
    a2.k = k;
    a2.chunks = chunks;
    for (int32_t u = 0; u <= users; ++u) a2.offsets[u] = a1.offsets[u];
    const int64_t dx_groups_max = (int64_t)h->cu_count * h->dx_per_cu;
    const int64_t want = (rows + 31) / 32;
    const int g2 = (int)(want < dx_groups_max ? want : dx_groups_max);
    e = sa::launch_grad_dx(d, a2, g2, s, time_it ? ev.ev[2] : nullptr, time_it ? ev.ev[3] : nullptr);
    timed = timed || (time_it && e == hipSuccess);
  }
  if (e == hipSuccess && !have_dq) e = sa::launch_zero(dq_sum, (int64_t)kd, s);  // no rows: zero gradients
  // dQ = tau dQ' W_K, dW_K = tau dQ'^T Q, dP = dQ W_Q^T, dW_Q = P^T dQ
  if (e == hipSuccess)
    e = sa::launch_small_matmuls({dq_sum, d, 1, h->WK32, d, 1, k, d, d, h->tau, dQ},
                                 {dq_sum, 1, d, h->Q, d, 1, d, d, k, h->tau, grad_W_K}, s);
  if (e == hipSuccess)
    e = sa::launch_small_matmuls({dQ, d, 1, h->WQ32, 1, d, k, d, d, 1.f, grad_P},
                                 {h->P32, 1, d, dQ, d, 1, d, d, k, 1.f, grad_W_Q}, s);
  if (h->timing && max_rows > 0) (timed ? h->pending : h->spare).push_back(ev);
  return e == hipSuccess ? SA_OK : SA_ERR_DEVICE;
}

SA_API sa_status sa_grad_set_kernel_timing(sa_grad h, int32_t enable) {
  if (h == nullptr) return SA_ERR_INVALID_ARG;
  h->timing = enable != 0;
  return SA_OK;
}

SA_API sa_status sa_grad_read_kernel_timing(sa_grad h, double* stats_ms, double* dx_ms, int64_t* calls) {
  if (h == nullptr || stats_ms == nullptr || dx_ms == nullptr || calls == nullptr) return SA_ERR_INVALID_ARG;
  DeviceGuard guard(h->device);
  double a = 0.0, b = 0.0;
  int64_t n = 0;
  for (auto& p : h->pending) {
    float t0 = 0.f, t1 = 0.f;
    if (hipEventSynchronize(p.ev[3]) != hipSuccess || hipEventElapsedTime(&t0, p.ev[0], p.ev[1]) != hipSuccess ||
        hipEventElapsedTime(&t1, p.ev[2], p.ev[3]) != hipSuccess)
      return SA_ERR_DEVICE;
    a += t0;
    b += t1;
    ++n;
    h->spare.push_back(p);
  }
  h->pending.clear();
  *stats_ms = a;
  *dx_ms = b;
  *calls = n;
  return SA_OK;
}
