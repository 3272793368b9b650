// Host side of the action-fusion entry points declared in include/sa.h
// (sa_action_*): validation, packing the weights once, launching the pass.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <new>
#include <vector>

#include "sa.h"
#include "sa_action.h"

#define SA_API extern "C" __attribute__((visibility("default")))

namespace {

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

constexpr int kMaxActionTypes = 1 << 20;
constexpr int64_t kF32ChunkRows = 32768;  // float32 path: rows per staging pass

}  // namespace

struct sa_action_s {
  int device = 0;
  int cu_count = 0;
  int groups_per_cu = 1;
  int d = 0, d_a = 0, d_ff = 0, n_actions = 0, kp = 0;
  sa_dtype dtype = SA_BF16;
  void* table = nullptr;   // [n_actions][d_a] in the dtype, a copy
  void* packed = nullptr;  // bf16: packed weight chunks
  // float32: transposed weights (gate_t, up_t [d_ff][k_pad] with zero columns past d + d_a;
  // down_t [d][d_ff]) and the staging buffers of one pass of kF32ChunkRows rows (Z [rows][k_pad],
  // H [rows][d_ff]), owned by the handle
  int k_pad = 0;
  float* gate_t = nullptr;
  float* up_t = nullptr;
  float* down_t = nullptr;
  float* stage_z = nullptr;
  float* stage_h = nullptr;
  bool timing = false;
  std::vector<hipEvent_t> pending, spare;  // start/stop pairs
};

namespace {

void free_action(sa_action_s* h) {
  if (h->table) (void)hipFree(h->table);
  if (h->packed) (void)hipFree(h->packed);
  for (float* p : {h->gate_t, h->up_t, h->down_t, h->stage_z, h->stage_h})
    if (p) (void)hipFree(p);
  for (auto* v : {&h->pending, &h->spare})
    for (hipEvent_t e : *v)
      if (e) (void)hipEventDestroy(e);
  delete h;
}

}  // namespace

SA_API sa_status sa_action_check_config(int32_t d, int32_t d_a, int32_t d_ff, int32_t n_actions, sa_dtype dtype) {
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_INVALID_ARG;
  if (d < 1 || d_a < 0 || d_ff < 1 || n_actions < 1 || n_actions > kMaxActionTypes) return SA_ERR_INVALID_ARG;
  if ((d != 64 && d != 128) || d_a % 8 != 0 || d + d_a > 256) return SA_ERR_UNSUPPORTED;
  if (dtype == SA_F32) return d_ff % 32 == 0 && d_ff <= 4096 ? SA_OK : SA_ERR_UNSUPPORTED;
  const int kp = sa::action_kpad(d, d_a);
  if (d_ff % (32 * sa::action_chunks_per_step(d, kp)) != 0 || d_ff > 4096) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

SA_API sa_status sa_action_create(sa_action* out, int32_t d, int32_t d_a, int32_t d_ff, int32_t n_actions,
                                  sa_dtype dtype, const void* action_table, const void* W_gate, const void* W_up,
                                  const void* W_down, void* stream) {
  if (out == nullptr) return SA_ERR_INVALID_ARG;
  *out = nullptr;
  sa_status st = sa_action_check_config(d, d_a, d_ff, n_actions, dtype);
  if (st != SA_OK) return st;
  if ((d_a > 0 && action_table == nullptr) || W_gate == nullptr || W_up == nullptr || W_down == nullptr)
    return SA_ERR_INVALID_ARG;
  if ((d_a > 0 && !aligned16(action_table)) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_down))
    return SA_ERR_INVALID_ARG;
  sa_action_s* h = new (std::nothrow) sa_action_s();
  if (h == nullptr) return SA_ERR_OUT_OF_MEMORY;
  hipStream_t s = static_cast<hipStream_t>(stream);
  h->d = d;
  h->d_a = d_a;
  h->d_ff = d_ff;
  h->n_actions = n_actions;
  h->kp = sa::action_kpad(d, d_a);
  hipDeviceProp_t prop;
  if (hipGetDevice(&h->device) != hipSuccess || hipGetDeviceProperties(&prop, h->device) != hipSuccess ||
      sa::action_occupancy(d, h->kp, &h->groups_per_cu) != hipSuccess || h->groups_per_cu < 1) {
    free_action(h);
    return SA_ERR_DEVICE;
  }
  h->cu_count = prop.multiProcessorCount;
  h->dtype = dtype;
  if (dtype == SA_F32) {
    const int kin = d + d_a;
    h->k_pad = 16 * ((kin + 15) / 16);
    const size_t fb = sizeof(float);
    if (hipMalloc(&h->table, (size_t)n_actions * (d_a > 0 ? d_a : 4) * fb) != hipSuccess ||
        hipMalloc(&h->gate_t, (size_t)d_ff * h->k_pad * fb) != hipSuccess ||
        hipMalloc(&h->up_t, (size_t)d_ff * h->k_pad * fb) != hipSuccess ||
        hipMalloc(&h->down_t, (size_t)d * d_ff * fb) != hipSuccess ||
        hipMalloc(&h->stage_z, (size_t)kF32ChunkRows * h->k_pad * fb) != hipSuccess ||
        hipMalloc(&h->stage_h, (size_t)kF32ChunkRows * d_ff * fb) != hipSuccess) {
      free_action(h);
      return SA_ERR_OUT_OF_MEMORY;
    }
    hipError_t e = hipSuccess;
    if (d_a > 0)
      e = hipMemcpyAsync(h->table, action_table, (size_t)n_actions * d_a * fb, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
      e = sa::launch_transpose_pad(static_cast<const float*>(W_gate), kin, d_ff, h->k_pad, h->gate_t, s);
    if (e == hipSuccess)
      e = sa::launch_transpose_pad(static_cast<const float*>(W_up), kin, d_ff, h->k_pad, h->up_t, s);
    if (e == hipSuccess)
      e = sa::launch_transpose_pad(static_cast<const float*>(W_down), d_ff, d, d_ff, h->down_t, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      free_action(h);
      return SA_ERR_DEVICE;
    }
    *out = h;
    return SA_OK;
  }
  const size_t table_bytes = (size_t)n_actions * (d_a > 0 ? d_a : 8) * 2;
  if (hipMalloc(&h->table, table_bytes) != hipSuccess ||
      hipMalloc(&h->packed, sa::action_packed_bytes(d, h->kp, d_ff)) != hipSuccess) {
    free_action(h);
    return SA_ERR_OUT_OF_MEMORY;
  }
  hipError_t e = hipSuccess;
  if (d_a > 0) e = hipMemcpyAsync(h->table, action_table, (size_t)n_actions * d_a * 2, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = sa::launch_action_pack(d, h->kp, W_gate, W_up, W_down, d_a, d_ff, h->packed, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    free_action(h);
    return SA_ERR_DEVICE;
  }
  *out = h;
  return SA_OK;
}

SA_API void sa_action_destroy(sa_action h) {
  if (h == nullptr) return;
  DeviceGuard guard(h->device);
  free_action(h);
}

SA_API sa_status sa_action_fuse(sa_action h, const void* E, const int32_t* actions, int64_t rows, void* X,
                                void* stream) {
  if (h == nullptr || rows < 0) return SA_ERR_INVALID_ARG;
  if (rows == 0) return SA_OK;
  if (E == nullptr || actions == nullptr || X == nullptr || !aligned16(E) || !aligned16(X) ||
      (reinterpret_cast<uintptr_t>(actions) & 3u) != 0)
    return SA_ERR_INVALID_ARG;
  DeviceGuard guard(h->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (h->dtype == SA_F32) {
    // passes of kF32ChunkRows rows through the handle's staging buffers, in stream order
    const float* Ef = static_cast<const float*>(E);
    float* Xf = static_cast<float*>(X);
    for (int64_t r0 = 0; r0 < rows; r0 += kF32ChunkRows) {
      const int64_t n = rows - r0 < kF32ChunkRows ? rows - r0 : kF32ChunkRows;
      hipError_t e = sa::launch_action_gather_f32(Ef + r0 * h->d, actions + r0, static_cast<const float*>(h->table),
                                                  n, h->d, h->d_a, h->k_pad, h->n_actions, h->stage_z, s);
      if (e == hipSuccess)
        e = sa::launch_plain_ffn(h->stage_z, n, h->k_pad, h->d, h->d_ff, h->gate_t, h->up_t, h->down_t, h->stage_h,
                                 Ef + r0 * h->d, Xf + r0 * h->d, s);
      if (e != hipSuccess) return SA_ERR_DEVICE;
    }
    return SA_OK;
  }
  sa::ActionArgs a{};
  a.E = E;
  a.actions = actions;
  a.table = h->table;
  a.packed = h->packed;
  a.X = X;
  a.rows = rows;
  a.n_actions = h->n_actions;
  a.d_a = h->d_a;
  a.chunks = h->d_ff / 32;
  const int64_t gmax = (int64_t)h->cu_count * h->groups_per_cu;
  const int64_t want = (rows + 31) / 32;
  const int groups = (int)(want < gmax ? want : gmax);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (h->timing) {
    if (h->spare.size() >= 2) {
      e1 = h->spare.back();
      h->spare.pop_back();
      e0 = h->spare.back();
      h->spare.pop_back();
    } else if (hipEventCreateWithFlags(&e0, hipEventDisableSystemFence) != hipSuccess) {
      return SA_ERR_DEVICE;
    } else if (hipEventCreateWithFlags(&e1, hipEventDisableSystemFence) != hipSuccess) {
      h->spare.push_back(e0);  // kept for the next timed call rather than leaked
      return SA_ERR_DEVICE;
    }
  }
  const hipError_t e = sa::launch_action_fuse(h->d, h->kp, a, groups, s, e0, e1);
  if (h->timing) {
    h->pending.push_back(e0);
    h->pending.push_back(e1);
  }
  return e == hipSuccess ? SA_OK : SA_ERR_DEVICE;
}

SA_API sa_status sa_action_compress_batch(sa_action a, sa_handle h, const void* E, const int32_t* actions,
                                          const int64_t* offsets, int32_t num_users, float* out, void* stream) {
  if (a == nullptr || h == nullptr) return SA_ERR_INVALID_ARG;
  if (a->d != 128 || a->dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  DeviceGuard guard(a->device);
  sa::ActionSource src{E, actions, a->table, a->packed, a->n_actions, a->d_a, a->d_ff, a->kp, a->device};
  return sa::compress_actions(h, src, offsets, num_users, out, stream);
}

SA_API sa_status sa_action_set_kernel_timing(sa_action h, int32_t enable) {
  if (h == nullptr) return SA_ERR_INVALID_ARG;
  h->timing = enable != 0;
  return SA_OK;
}

SA_API sa_status sa_action_read_kernel_timing(sa_action h, double* ms, int64_t* launches) {
  if (h == nullptr || ms == nullptr || launches == nullptr) return SA_ERR_INVALID_ARG;
  DeviceGuard guard(h->device);
  double total = 0.0;
  int64_t n = 0;
  for (size_t i = 0; i + 1 < h->pending.size(); i += 2) {
    float t = 0.f;
    if (hipEventSynchronize(h->pending[i + 1]) != hipSuccess ||
        hipEventElapsedTime(&t, h->pending[i], h->pending[i + 1]) != hipSuccess)
      return SA_ERR_DEVICE;
    total += t;
    ++n;
  }
  for (hipEvent_t e : h->pending) h->spare.push_back(e);
  h->pending.clear();
  *ms = total;
  *launches = n;
  return SA_OK;
}
