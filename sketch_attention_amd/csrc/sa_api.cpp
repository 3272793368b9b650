// Host side of the C ABI declared in include/sa.h: argument validation, plan
// selection, the handle (folded weights + workspace), batching of users into
// launches, and optional kernel timing.
#include "sa.h"

#include <hip/hip_runtime_api.h>

#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstdint>
#include <cstring>
#include <new>
#include <vector>

#include "sa_action.h"
#include "sa_internal.h"

#define SA_API extern "C" __attribute__((visibility("default")))

namespace {

using sa::Plan;

struct TimingSlot {
  // fused kernel start/stop, reduction kernel start/stop, first phase start/stop of a two-phase pass
  // (recorded by the dispatches)
  hipEvent_t ev[6];
  bool fused;      // false when the launch had no rows (reduce only)
  bool two_phase;  // ev[4], ev[5] were recorded too
};

}  // namespace

struct sa_handle_s {
  int device = 0;
  int cu_count = 0;
  int groups_per_cu = 1;
  float tau = 0.f;
  int norm = SA_NORM_PROTOTYPES;  // softmax axis
  Plan plan{};
  void* M = nullptr;           // folded matrix [k_pad][d], dtype
  float* workspace = nullptr;  // partial sketches
  size_t workspace_bytes = 0;
  bool frozen = false;         // sa_reserve: the workspace never moves; launches are sized to fit it
  bool timing = false;
  std::vector<TimingSlot> slots;  // recorded since the last read
  std::vector<TimingSlot> spare;  // event triples ready for reuse
};

namespace {

constexpr double kLog2e = 1.4426950408889634073599246810019;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Plan of the fused pass for a supported (dtype, d, k).
// bf16 with k > 32: the streamed pass (sa_stream.hpp), eight waves per group
// (four for d = 128, k <= 128).  Up to k = 256 (d = 128) or 512 (d = 64) each
// wave holds 32 prototypes (64 for d = 64 above k = 256), the folded matrix
// in registers and two affinity tiles in flight; above that (k <= 512 for
// d = 128, k <= 1024 for d = 64) each wave holds k_pad / 8 prototypes, one
// affinity tile, and the folded matrix sits in LDS; d = 128 with 128 < k <=
// 256 runs the 32x32x16 pass of sa_wide.hpp instead.  bf16 with k <= 32: the
// lockstep pass (sa_fused.hpp), eight waves.  float32: lockstep, four waves,
// folded matrix in registers.
// SA_PLAN="kw,waves_k,waves_rows,m_in_lds[,kind[,prefetch[,row_blocks[,score_buffers]]]]"
// in the environment overrides the choice when that plan is compiled.
// The comparator (softmax over the history axis) runs, for bf16, the
// streamed pass with waves that never split a tile's rows: four waves of 32
// prototypes for k <= 128, else eight waves of 32 (k <= 256; at d = 128 on
// the 32x32x16 pass with the prototypes along the lanes), 64 (k <= 512) or
// 128 (d = 64, k <= 1024) prototypes each; for float32 the lockstep pass
// (below).
Plan make_history_plan(int dtype, int d, int k) {
  Plan p{};
  if (dtype == SA_F32) {
    // float32: the lockstep pass, four waves over 16, 32 or (d = 64) 64
    // prototypes each and none over the rows, in independent blocks of 128
    // (d = 128) or 256 (d = 64) prototypes beyond that
    p.dtype = SA_F32;
    p.d = d;
    p.k = k;
    p.kind = 0;
    p.prefetch = 1;
    p.row_blocks = 2;
    p.score_buffers = 2;
    p.waves_k = 4;
    p.waves_rows = 1;
    p.kw = k <= 64 ? 16 : (k <= 128 || d == 128 ? 32 : 64);
    p.m_in_lds = 0;
    p.blocks = (k + 4 * p.kw - 1) / (4 * p.kw);
    p.k_pad = 4 * p.kw * p.blocks;
    p.tile_rows = sa::kRowsPerWave;
    return p;
  }
  p.dtype = SA_BF16;
  p.d = d;
  p.k = k;
  p.kind = 1;
  p.prefetch = 1;
  p.waves_k = 8;
  p.waves_rows = 1;
  if (k <= 128) {
    p.kw = 32; p.waves_k = 4; p.row_blocks = 4; p.score_buffers = 2;  // four-wave groups, two per CU
  } else if (k <= 256) {
    p.kw = 32; p.row_blocks = 4; p.score_buffers = 2;
    if (d == 128) p.kind = 3;  // the 32x32x16 pass with the prototypes along the lanes (sa_wide.hpp)
  } else if (k <= 512 || d == 128) {
    p.kw = 64; p.row_blocks = 2; p.score_buffers = d == 128 ? 1 : 2;
  } else {
    p.kw = 128; p.row_blocks = 2; p.score_buffers = 1;
  }
  p.m_in_lds = 0;
  p.tile_rows = 16 * p.row_blocks;
  // d = 128 beyond 512 prototypes: blocks of 8 x 64 prototypes, each its own
  // work groups (the softmax over rows is per prototype, so the blocks are
  // independent and need no second phase)
  p.blocks = (k + p.kw * p.waves_k - 1) / (p.kw * p.waves_k);
  p.k_pad = p.kw * p.waves_k * p.blocks;
  return p;
}

Plan make_plan(int dtype, int d, int k) {
  Plan p{};
  p.dtype = dtype;
  p.d = d;
  p.k = k;
  p.kind = 0;
  p.prefetch = 1;
  p.row_blocks = 2;
  p.score_buffers = 2;
  const int waves = dtype == SA_BF16 ? 8 : 4;
  const int k16 = (k + 15) / 16 * 16;
  const bool stream = dtype == SA_BF16 && k > 32;
  p.blocks = 1;
  if (dtype == SA_BF16 && d == 128 && k > 512) {
    // two-phase pass over blocks of 8 x 32 prototypes (the folded matrix of
    // more prototypes fits neither one group's registers nor its LDS), on
    // 32x32x16 products
    p.kind = 2;
    p.kw = 32;
    p.waves_k = 8;
    p.waves_rows = 1;
    p.row_blocks = 4;
    p.blocks = (k + 255) / 256;
    p.k_pad = p.blocks * 256;
    p.tile_rows = 64;
    p.m_in_lds = 0;
    return p;
  }
  if (dtype == SA_F32 && k > 256) {
    // float32 beyond 256 prototypes: the four-wave plan of 4 x 64 prototypes in
    // two phases over blocks of 256 (its folded matrix lives in registers)
    p.kw = 64;
    p.waves_k = 4;
    p.waves_rows = 1;
    p.m_in_lds = 0;
    p.blocks = (k + 255) / 256;
    p.k_pad = p.blocks * 256;
    p.tile_rows = sa::kRowsPerWave;
    return p;
  }
  if (stream) {
    p.kind = 1;
    const bool wide = d == 128 ? k > 256 : k > 512;  // folded matrix too large for registers
    if (wide) {
      p.kw = d == 128 ? 64 : 128;
      p.waves_k = 8;
      p.score_buffers = 1;
    } else {
      p.kw = (d == 64 && k > 256) ? 64 : 32;
      p.waves_k = k <= 64 ? 2 : (k <= 128 ? 4 : 8);
      p.row_blocks = (p.kw == 32 && (p.waves_k == 8 || p.waves_k == 4)) ? 4 : 2;
    }
    // d = 128, k <= 64: two row waves (four waves per group) keep the four
    // 64-row LDS tiles of the ring within budget; d = 128, k <= 128: four
    // waves over the prototypes and none over the rows, two groups per CU
    // (measured faster than eight waves split 4 x 2: 248 against 273 us on
    // the ragged workload)
    p.waves_rows = (d == 128 && p.waves_k == 2) ? 2 : (d == 128 && p.waves_k == 4) ? 1 : waves / p.waves_k;
    // d = 128, 128 < k <= 256: eight waves of 32 prototypes on 32x32x16
    // products with the prototypes along the lanes (measured 2-3 % faster on
    // the long workload than the 16x16x32 plan of the same shape)
    if (d == 128 && p.kw == 32 && p.waves_k == 8 && p.waves_rows == 1) p.kind = 3;
  } else if (k16 <= 16) {
    p.kw = 16; p.waves_k = 1;
  } else if (k16 <= 32) {
    p.kw = 32; p.waves_k = 1;
  } else if (k16 <= 64) {
    p.kw = 64; p.waves_k = 1;
  } else if (k <= 128) {
    p.kw = 64; p.waves_k = 2;
  } else if (k <= 256) {
    p.kw = 64; p.waves_k = 4;
  } else if (k <= 512) {
    p.kw = 64; p.waves_k = 8;
  } else {
    p.kw = 128; p.waves_k = 8;
  }
  if (!stream && p.kind == 0) p.waves_rows = waves / p.waves_k;
  p.m_in_lds = (dtype == SA_BF16 && !stream) ? 1 : 0;
  if (const char* env = std::getenv("SA_PLAN")) {
    int kw = 0, wk = 0, wr = 0, ml = 0, kind = 0, pf = 1, rb = 2, sb = 2;
    const int n = std::sscanf(env, "%d,%d,%d,%d,%d,%d,%d,%d", &kw, &wk, &wr, &ml, &kind, &pf, &rb, &sb);
    if (n >= 4 && kw % 16 == 0 && kw > 0 && wk > 0 && wr > 0 && kw * wk >= k && kind >= 0 && kind <= 3 &&
        (pf == 1 || pf == 2) && (rb == 2 || rb == 4) && (sb == 1 || sb == 2)) {
      p.kw = kw; p.waves_k = wk; p.waves_rows = wr; p.m_in_lds = ml ? 1 : 0; p.kind = kind; p.prefetch = pf;
      p.row_blocks = rb; p.score_buffers = sb;
    }
  }
  p.k_pad = p.kw * p.waves_k;
  p.tile_rows = p.kind >= 1 ? 16 * p.row_blocks * p.waves_rows : sa::kRowsPerWave * p.waves_rows;
  return p;
}

sa_status check_config(int32_t d, int32_t k, float tau, sa_dtype dtype) {
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_INVALID_ARG;
  if (!std::isfinite(tau)) return SA_ERR_INVALID_ARG;
  if (k < 1 || d < 1) return SA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SA_ERR_UNSUPPORTED;
  if (dtype == SA_BF16 && k > 1024) return SA_ERR_UNSUPPORTED;
  if (dtype == SA_F32 && k > 1024) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

sa_status check_batch(const int64_t* offsets, int32_t num_users) {
  if (num_users < 0) return SA_ERR_INVALID_ARG;
  if (num_users == 0) return SA_OK;
  if (offsets == nullptr) return SA_ERR_INVALID_ARG;
  if (offsets[0] != 0) return SA_ERR_INVALID_ARG;
  for (int32_t u = 0; u < num_users; ++u)
    if (offsets[u + 1] < offsets[u]) return SA_ERR_INVALID_ARG;
  // the streamed kernels keep a work group's rows in 32-bit offsets from its first row
  if (offsets[num_users] > INT32_MAX) return SA_ERR_INVALID_ARG;
  return SA_OK;
}

// Work groups of the fused grid for a launch of `rows` rows: at most one full
// wave of resident groups and no more groups than tiles.  Beyond one group
// per compute unit, extra resident groups are used only when each still gets
// at least kMinTilesPerGroup tiles: a short group is mostly prologue and its
// partial sketch costs as much to write and reduce as a long one's.
constexpr int64_t kMinTilesPerGroup = 8;
int groups_for(const sa_handle_s* h, int64_t rows) {
  const int64_t cap = (int64_t)h->cu_count * h->groups_per_cu;
  const int64_t tiles = (rows + h->plan.tile_rows - 1) / h->plan.tile_rows;
  int64_t g = (tiles + kMinTilesPerGroup - 1) / kMinTilesPerGroup;
  if (g < h->cu_count) g = h->cu_count;
  if (g > cap) g = cap;
  if (g > tiles) g = tiles;
  return g < 1 ? 1 : (int)g;
}

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    int cur = 0;
    if (hipGetDevice(&cur) == hipSuccess && cur != dev) {
      if (hipSetDevice(dev) == hipSuccess) prev = cur;
    }
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

TimingSlot take_slot(sa_handle_s* h) {
  if (!h->spare.empty()) {
    TimingSlot s = h->spare.back();
    h->spare.pop_back();
    return s;
  }
  TimingSlot s{};
  for (auto& e : s.ev) {
    // timing only: no system-scope fence (a cache writeback and invalidation) when it is recorded
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) e = nullptr;
  }
  return s;
}

}  // namespace

SA_API const char* sa_status_string(sa_status s) {
  switch (s) {
    case SA_OK: return "success";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SA_ERR_OUT_OF_MEMORY: return "out of device memory";
    case SA_ERR_DEVICE: return "HIP device error";
  }
  return "unknown status";
}

SA_API sa_status sa_check_config(int32_t d, int32_t k, float tau, sa_dtype dtype) {
  return check_config(d, k, tau, dtype);
}

SA_API sa_status sa_check_batch(int32_t k, const int64_t* offsets, int32_t num_users) {
  if (k < 1) return SA_ERR_INVALID_ARG;
  return check_batch(offsets, num_users);
}

SA_API sa_status sa_create_ex(sa_handle* out, int32_t d, int32_t k, float tau, sa_dtype dtype, const void* P,
                              const void* W_Q, const void* W_K, sa_norm norm, void* stream) {
  if (out == nullptr) return SA_ERR_INVALID_ARG;
  *out = nullptr;
  sa_status st = check_config(d, k, tau, dtype);
  if (st != SA_OK) return st;
  if (norm != SA_NORM_PROTOTYPES && norm != SA_NORM_HISTORY) return SA_ERR_INVALID_ARG;
  if (P == nullptr || W_Q == nullptr || W_K == nullptr) return SA_ERR_INVALID_ARG;
  if (!aligned16(P) || !aligned16(W_Q) || !aligned16(W_K)) return SA_ERR_INVALID_ARG;

  sa_handle_s* h = new (std::nothrow) sa_handle_s();
  if (h == nullptr) return SA_ERR_OUT_OF_MEMORY;
  hipStream_t s = static_cast<hipStream_t>(stream);
  h->tau = tau;
  h->norm = norm;
  h->plan = norm == SA_NORM_HISTORY ? make_history_plan((int)dtype, d, k) : make_plan((int)dtype, d, k);
  const size_t elem = dtype == SA_BF16 ? 2 : 4;
  float* tmp = nullptr;
  hipDeviceProp_t prop;
  if (hipGetDevice(&h->device) != hipSuccess || hipGetDeviceProperties(&prop, h->device) != hipSuccess) {
    delete h;
    return SA_ERR_DEVICE;
  }
  h->cu_count = prop.multiProcessorCount;
  int occ = 0;
  if (sa::fused_occupancy(h->plan, &occ) != hipSuccess || occ < 1) {
    delete h;
    return std::getenv("SA_PLAN") ? SA_ERR_UNSUPPORTED : SA_ERR_DEVICE;
  }
  h->groups_per_cu = occ;
  if (hipMalloc(&h->M, (size_t)h->plan.k_pad * d * elem) != hipSuccess) {
    delete h;
    return SA_ERR_OUT_OF_MEMORY;
  }
  if (hipMalloc(&tmp, (size_t)k * d * sizeof(float)) != hipSuccess) {
    (void)hipFree(h->M);
    delete h;
    return SA_ERR_OUT_OF_MEMORY;
  }
  const float scale = (float)((double)tau * kLog2e);
  hipError_t e = sa::launch_fold((int)dtype, P, W_Q, W_K, scale, k, h->plan.k_pad, d, tmp, h->M, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(tmp);
  if (e != hipSuccess) {
    (void)hipFree(h->M);
    delete h;
    return SA_ERR_DEVICE;
  }
  *out = h;
  return SA_OK;
}

SA_API sa_status sa_create(sa_handle* out, int32_t d, int32_t k, float tau, sa_dtype dtype, const void* P,
                           const void* W_Q, const void* W_K, void* stream) {
  return sa_create_ex(out, d, k, tau, dtype, P, W_Q, W_K, SA_NORM_PROTOTYPES, stream);
}

SA_API void sa_destroy(sa_handle h) {
  if (h == nullptr) return;
  DeviceGuard guard(h->device);
  for (auto* v : {&h->slots, &h->spare})
    for (auto& s : *v)
      for (auto& e : s.ev)
        if (e) (void)hipEventDestroy(e);
  if (h->workspace) (void)hipFree(h->workspace);
  if (h->M) (void)hipFree(h->M);
  delete h;
}

namespace {

// One SA pass over a packed batch into out [U][k][d].  M: the folded matrix
// shared by all users (m_stride 0) or one per user, m_stride elements apart.
// Users go to launches of at most kMaxUsersPerLaunch; a launch is the fused
// pass plus the reduction of its partial sketches, or, for a two-phase plan
// (plan.blocks > 1), the statistics phase, their merge, the aggregation
// phase and the reduction.
// fixed_ws (fixed_bytes long): a workspace that must not grow.  Launches are
// then formed greedily so that each fits (at least one work group per
// prototype block and launch); if one user alone does not fit, nothing is
// enqueued and SA_ERR_UNSUPPORTED is returned.  No event is recorded.
// Workspace sizing of one launch of `rows` rows and `nu` users: a partial
// slot is the block's k x d accumulator (plus per-prototype maxima and sums
// for the comparator) per work group and user piece and prototype block; the
// two-phase pass adds per-block and merged log-sum-exps of every row.
struct Sizing {
  int nb;             // prototype blocks
  size_t slot_bytes;  // one partial slot
  bool two_phase;
};
Sizing sizing_of(const sa_handle_s* h) {
  const Plan& plan = h->plan;
  const bool hist = h->norm == SA_NORM_HISTORY;
  Sizing z;
  z.nb = plan.blocks > 1 ? plan.blocks : 1;
  z.slot_bytes = (size_t)(plan.kw * plan.waves_k) * (plan.d + (hist ? 2 : 0)) * sizeof(float);
  z.two_phase = z.nb > 1 && !hist;
  return z;
}
// work groups per prototype block for a launch of `rows` rows (the grid is nb times that)
int launch_groups(const sa_handle_s* h, const Sizing& z, int64_t rows) {
  if (rows <= 0) return 0;
  const int g = groups_for(h, rows);
  return z.nb > 1 ? (g + z.nb - 1) / z.nb : g;
}
size_t stats_bytes(const Sizing& z, int64_t rows) { return z.two_phase ? (size_t)(z.nb + 1) * (size_t)rows * sizeof(float) : 0; }
size_t launch_bytes(const Sizing& z, int groups, int32_t nu, int64_t rows) {
  return (size_t)z.nb * (groups + nu) * z.slot_bytes + stats_bytes(z, rows);
}

// act: the rows are formed by the action fusion from act->E and act->actions
// inside the sketch kernel (X unused); the handle's plan must be the one-pass
// plan of eight waves of 32 prototypes.
sa_status compress(sa_handle_s* h, const void* X, const int64_t* offsets, int32_t num_users, float* out, void* stream,
                   const void* M, int64_t m_stride, float* fixed_ws = nullptr, size_t fixed_bytes = 0,
                   bool allow_timing = false, const sa::ActionSource* act = nullptr) {
  if (h == nullptr) return SA_ERR_INVALID_ARG;
  sa_status st = check_batch(offsets, num_users);
  if (st != SA_OK) return st;
  if (num_users == 0) return SA_OK;
  const int64_t total = offsets[num_users];
  if (out == nullptr || !aligned16(out)) return SA_ERR_INVALID_ARG;
  if (act != nullptr) {
    X = act->E;
    if (total > 0 && (act->actions == nullptr || (reinterpret_cast<uintptr_t>(act->actions) & 3u) != 0))
      return SA_ERR_INVALID_ARG;
  }
  if (total > 0 && (X == nullptr || !aligned16(X))) return SA_ERR_INVALID_ARG;

  const Plan& plan = h->plan;
  const size_t elem = plan.dtype == SA_BF16 ? 2 : 4;
  const bool hist = h->norm == SA_NORM_HISTORY;
  const Sizing z = sizing_of(h);
  const int nb = z.nb;
  const int block_k = plan.kw * plan.waves_k;  // prototypes per block (one partial slot)
  const size_t slot_bytes = z.slot_bytes;
  // a frozen handle's workspace is fixed: launches are sized to fit it
  if (fixed_ws == nullptr && h->frozen) {
    fixed_ws = h->workspace;
    fixed_bytes = h->workspace_bytes;
    allow_timing = true;
  } else if (fixed_ws == nullptr) {
    allow_timing = true;
  }

  struct LaunchPlan {
    int32_t u0, nu;
    int groups;
    size_t bytes;  // partials + statistics
  };
  std::vector<LaunchPlan> launches;
  for (int32_t u0 = 0; u0 < num_users;) {
    int32_t nu = num_users - u0 < sa::kMaxUsersPerLaunch ? num_users - u0 : sa::kMaxUsersPerLaunch;
    int64_t rows = offsets[u0 + nu] - offsets[u0];
    int g = launch_groups(h, z, rows);
    auto bytes_of = [&](int gg, int32_t n, int64_t r) { return launch_bytes(z, gg, n, r); };
    if (fixed_ws != nullptr) {
      // the most users (up to the launch limit) that fit with at least one group each
      while (nu > 1 && bytes_of(1, nu, rows) > fixed_bytes) {
        nu = nu / 2;
        rows = offsets[u0 + nu] - offsets[u0];
      }
      if (bytes_of(rows > 0 ? 1 : 0, nu, rows) > fixed_bytes) return SA_ERR_UNSUPPORTED;
      g = launch_groups(h, z, rows);
      const int64_t room = (int64_t)((fixed_bytes - stats_bytes(z, rows)) / slot_bytes) / nb - nu;
      if (g > room) g = (int)room;
    }
    launches.push_back({u0, nu, g, bytes_of(g, nu, rows)});
    u0 += nu;
  }

  DeviceGuard guard(h->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Workspace for the largest launch of this call.
  size_t need = 0;
  for (const auto& L : launches) need = L.bytes > need ? L.bytes : need;
  if (fixed_ws == nullptr && need > h->workspace_bytes) {
    // Earlier launches on this stream may still read the old workspace.
    if (h->workspace) {
      if (hipStreamSynchronize(s) != hipSuccess) return SA_ERR_DEVICE;
      (void)hipFree(h->workspace);
      h->workspace = nullptr;
      h->workspace_bytes = 0;
    }
    if (hipMalloc(&h->workspace, need) != hipSuccess) {
      h->workspace = nullptr;
      return SA_ERR_OUT_OF_MEMORY;
    }
    h->workspace_bytes = need;
  }

  float* const partial = fixed_ws != nullptr ? fixed_ws : h->workspace;
  for (const auto& L : launches) {
    const int32_t u0 = L.u0, nu = L.nu;
    const int64_t base = offsets[u0];
    const int64_t rows = offsets[u0 + nu] - base;
    const int groups = L.groups;
    // statistics after this launch's partial slots
    float* const stats_b = partial + (size_t)nb * (groups + nu) * (slot_bytes / sizeof(float));
    float* const stats_m = stats_b + (size_t)nb * rows;

    sa::FusedArgs fa;
    std::memset(&fa, 0, sizeof(fa));
    fa.X = static_cast<const char*>(X) + (size_t)base * plan.d * elem;
    fa.M = static_cast<const char*>(M) + (size_t)u0 * (size_t)m_stride * elem;
    fa.m_stride = m_stride;
    fa.history_softmax = hist ? 1 : 0;
    fa.partial = partial;
    fa.rows = rows;
    fa.users = nu;
    fa.k = plan.k;
    fa.blocks = nb;
    sa::ReduceArgs ra;
    std::memset(&ra, 0, sizeof(ra));
    ra.partial = partial;
    ra.history_softmax = hist ? 1 : 0;
    ra.out = out + (size_t)u0 * plan.k * plan.d;
    ra.rows = rows;
    ra.users = nu;
    ra.groups = groups;
    ra.k = plan.k;
    ra.d = plan.d;
    ra.kw = plan.kw;
    ra.k_pad = block_k;
    ra.blocks = nb;
    ra.layout = plan.kind >= 2 ? 1 : 0;
    for (int32_t i = 0; i <= nu; ++i) {
      fa.offsets[i] = offsets[u0 + i] - base;
      ra.offsets[i] = fa.offsets[i];
    }

    TimingSlot ts{};
    const bool timed = h->timing && allow_timing;
    if (timed) {
      ts = take_slot(h);
      ts.fused = rows > 0;
      ts.two_phase = nb > 1 && !hist;
    }
    if (rows > 0) {
      if (nb > 1 && !hist) {
        // statistics phase, merge, aggregation phase (the aggregation carries events ev[0], ev[1])
        fa.lse_mode = 1;
        fa.stats = stats_b;
        if (sa::launch_fused(plan, fa, nb * groups, s, ts.ev[4], ts.ev[5]) != hipSuccess) return SA_ERR_DEVICE;
        if (sa::launch_lse_merge(stats_b, rows, nb, stats_m, s) != hipSuccess) return SA_ERR_DEVICE;
        fa.lse_mode = 2;
        fa.stats = stats_m;
      }
      if (act != nullptr) {
        sa::ActSaArgs aa;
        aa.sa = fa;
        aa.sa.X = nullptr;
        aa.E = fa.X;
        aa.actions = act->actions + base;
        aa.table = act->table;
        aa.packed = act->packed;
        aa.n_actions = act->n_actions;
        aa.d_a = act->d_a;
        aa.chunks = act->d_ff / 32;
        if (sa::launch_action_sa(act->kp, aa, sa::Launch{groups, s, ts.ev[0], ts.ev[1]}) != hipSuccess)
          return SA_ERR_DEVICE;
      } else if (sa::launch_fused(plan, fa, nb * groups, s, ts.ev[0], ts.ev[1]) != hipSuccess) {
        return SA_ERR_DEVICE;
      }
    }
    if (sa::launch_reduce(ra, s, ts.ev[2], ts.ev[3]) != hipSuccess) return SA_ERR_DEVICE;
    if (timed) h->slots.push_back(ts);
  }
  return SA_OK;
}

}  // namespace

namespace sa {

sa_status compress_actions(sa_handle h, const ActionSource& src, const int64_t* offsets, int32_t num_users,
                           float* out, void* stream) {
  if (h == nullptr) return SA_ERR_INVALID_ARG;
  const Plan& p = h->plan;
  if (p.kind != 3 || p.blocks != 1 || h->norm != SA_NORM_PROTOTYPES || p.d != 128 || p.dtype != SA_BF16 ||
      (src.kp != 128 && src.kp != 192 && src.kp != 256) || src.d_ff % 32 != 0 || src.device != h->device)
    return SA_ERR_UNSUPPORTED;
  return compress(h, nullptr, offsets, num_users, out, stream, h->M, 0, nullptr, 0, false, &src);
}

}  // namespace sa

SA_API sa_status sa_compress_batch(sa_handle h, const void* X, const int64_t* offsets, int32_t num_users, float* out,
                                   void* stream) {
  if (h == nullptr) return SA_ERR_INVALID_ARG;
  return compress(h, X, offsets, num_users, out, stream, h->M, 0);
}

SA_API sa_status sa_compress_batch_noalloc(sa_handle h, const void* X, const int64_t* offsets, int32_t num_users,
                                           float* out, void* stream) {
  if (h == nullptr) return SA_ERR_INVALID_ARG;
  sa_status st = check_batch(offsets, num_users);
  if (st != SA_OK) return st;
  if (num_users == 0) return SA_OK;
  DeviceGuard guard(h->device);
  float* ws = nullptr;
  if (sa::noalloc_scratch(h->device, &ws) != hipSuccess) return SA_ERR_DEVICE;
  return compress(h, X, offsets, num_users, out, stream, h->M, 0, ws, sa::kNoAllocScratchBytes);
}

SA_API sa_status sa_reserve(sa_handle h, int64_t max_rows, int32_t max_users, int32_t freeze, void* stream) {
  if (h == nullptr || max_rows < 0 || max_rows > INT32_MAX || max_users < 0) return SA_ERR_INVALID_ARG;
  DeviceGuard guard(h->device);
  // the largest launch a call within the bounds forms: all its rows (groups grow with rows) and up to the
  // launch limit of users
  const Sizing z = sizing_of(h);
  const int32_t nu = max_users < sa::kMaxUsersPerLaunch ? max_users : sa::kMaxUsersPerLaunch;
  const size_t need = launch_bytes(z, launch_groups(h, z, max_rows), nu, max_rows);
  if (need > h->workspace_bytes) {
    if (h->workspace) {
      if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return SA_ERR_DEVICE;
      (void)hipFree(h->workspace);
      h->workspace = nullptr;
      h->workspace_bytes = 0;
    }
    if (hipMalloc(&h->workspace, need) != hipSuccess) {
      h->workspace = nullptr;
      h->frozen = false;
      return SA_ERR_OUT_OF_MEMORY;
    }
    h->workspace_bytes = need;
  }
  // a frozen handle with no workspace yet (both bounds 0) keeps growing on demand
  h->frozen = freeze != 0 && h->workspace != nullptr;
  return SA_OK;
}

SA_API sa_status sa_get_folded(sa_handle h, float* dst, void* stream) {
  if (h == nullptr || dst == nullptr) return SA_ERR_INVALID_ARG;
  DeviceGuard guard(h->device);
  if (sa::launch_unfold(h->plan.dtype, h->M, h->plan.k, h->plan.d, dst, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return SA_ERR_DEVICE;
  return SA_OK;
}

SA_API sa_status sa_set_kernel_timing(sa_handle h, int32_t enable) {
  if (h == nullptr) return SA_ERR_INVALID_ARG;
  h->timing = enable != 0;
  return SA_OK;
}

SA_API sa_status sa_read_kernel_timing(sa_handle h, double* fused_ms, double* reduce_ms, int64_t* fused_launches) {
  if (h == nullptr) return SA_ERR_INVALID_ARG;
  DeviceGuard guard(h->device);
  double f = 0.0, r = 0.0;
  int64_t n = 0;
  sa_status st = SA_OK;
  for (auto& s : h->slots) {
    if (!s.ev[0] || !s.ev[1] || !s.ev[2] || !s.ev[3] || hipEventSynchronize(s.ev[3]) != hipSuccess) {
      st = SA_ERR_DEVICE;
      continue;
    }
    float a = 0.f, b = 0.f, c = 0.f;
    if ((s.fused && hipEventElapsedTime(&a, s.ev[0], s.ev[1]) != hipSuccess) ||
        (s.fused && s.two_phase && (!s.ev[4] || !s.ev[5] || hipEventElapsedTime(&c, s.ev[4], s.ev[5]) != hipSuccess)) ||
        hipEventElapsedTime(&b, s.ev[2], s.ev[3]) != hipSuccess) {
      st = SA_ERR_DEVICE;
      continue;
    }
    if (s.fused) {
      f += a + c;  // both phases of a two-phase pass
      ++n;
    }
    r += b;
  }
  for (auto& s : h->slots) h->spare.push_back(s);
  h->slots.clear();
  if (fused_ms) *fused_ms = f;
  if (reduce_ms) *reduce_ms = r;
  if (fused_launches) *fused_launches = n;
  return st;
}

SA_API sa_status sa_describe_plan(sa_handle h, int64_t total_rows, int32_t* groups, int32_t* waves_k,
                                  int32_t* waves_rows, int32_t* tile_rows, int32_t* k_padded) {
  if (h == nullptr || total_rows < 0) return SA_ERR_INVALID_ARG;
  if (groups) *groups = total_rows > 0 ? groups_for(h, total_rows) : 0;
  if (waves_k) *waves_k = h->plan.waves_k;
  if (waves_rows) *waves_rows = h->plan.waves_rows;
  if (tile_rows) *tile_rows = h->plan.tile_rows;
  if (k_padded) *k_padded = h->plan.k_pad;
  return SA_OK;
}

// ---------------------------------------------------------------- stacked refinement
// Section 2.2 of the SequenceO1 close-reading page: layer l queries the raw
// history with the previous state (X~(0) = P), adds the aggregate and
// normalises, then applies a residual feed-forward block and a second
// normalisation.  Layer 1 runs the plain SA pass with the shared fold of P;
// layers 2.. fold each user's state into its own matrix and run the same
// pass with per-user matrices.

struct sa_stack_s {
  struct Layer {
    float* wqk_t = nullptr;   // [d][d] (W_Q W_K^T)^T (layers 2..)
    float* ln1_g = nullptr;   // [d] each
    float* ln1_b = nullptr;
    float* ln2_g = nullptr;
    float* ln2_b = nullptr;
    float* gate_t = nullptr;  // [d_ff][d]
    float* up_t = nullptr;    // [d_ff][d]
    float* down_t = nullptr;  // [d][d_ff]
  };
  int device = 0;
  int d = 0, k = 0, d_ff = 0;
  sa_handle_s* base = nullptr;  // plan, fold of P with layer 1's weights, workspace
  float* P = nullptr;           // [k][d] float32 copy of the prototypes
  std::vector<Layer> layers;
  // per-call buffers, grown on demand
  int64_t cap_users = 0;
  void* Mu = nullptr;       // [U][k_pad][d] per-user folded matrices, dtype
  float* y = nullptr;       // [U][k][d] aggregate of the current layer
  float* xbar = nullptr;    // [U][k][d] first normalisation
  float* state = nullptr;   // [U][k][d] X~(l)
  float* ffn_out = nullptr; // [U][k][d]
  float* hidden = nullptr;  // [U][k][d_ff]
};

namespace {

constexpr float kLayerNormEps = 1e-5f;
constexpr int32_t kMaxStackLayers = 16;

void free_stack_buffers(sa_stack_s* h) {
  for (void* p : {h->Mu, (void*)h->y, (void*)h->xbar, (void*)h->state, (void*)h->ffn_out, (void*)h->hidden})
    if (p) (void)hipFree(p);
  h->Mu = nullptr;
  h->y = h->xbar = h->state = h->ffn_out = h->hidden = nullptr;
  h->cap_users = 0;
}

void free_stack(sa_stack_s* h) {
  free_stack_buffers(h);
  for (auto& l : h->layers)
    for (float* p : {l.wqk_t, l.ln1_g, l.ln1_b, l.ln2_g, l.ln2_b, l.gate_t, l.up_t, l.down_t})
      if (p) (void)hipFree(p);
  if (h->P) (void)hipFree(h->P);
  if (h->base) sa_destroy(h->base);
  delete h;
}

template <typename T>
bool dev_alloc(T** p, size_t count) {
  return hipMalloc(reinterpret_cast<void**>(p), count * sizeof(T)) == hipSuccess;
}

}  // namespace

SA_API sa_status sa_stack_create(sa_stack* out, int32_t d, int32_t k, int32_t d_ff, int32_t num_layers, float tau,
                                 sa_dtype dtype, const void* P, const sa_layer_params* params, void* stream) {
  if (out == nullptr) return SA_ERR_INVALID_ARG;
  *out = nullptr;
  sa_status st = check_config(d, k, tau, dtype);
  if (st != SA_OK) return st;
  if (num_layers < 1 || num_layers > kMaxStackLayers || params == nullptr || P == nullptr) return SA_ERR_INVALID_ARG;
  if (d_ff < 64 || d_ff > 8192 || d_ff % 64 != 0) return SA_ERR_UNSUPPORTED;
  for (int32_t l = 0; l < num_layers; ++l) {
    const sa_layer_params& p = params[l];
    for (const void* q : {p.W_Q, p.W_K, (const void*)p.ln1_gain, (const void*)p.ln1_bias, (const void*)p.ffn_gate,
                          (const void*)p.ffn_up, (const void*)p.ffn_down, (const void*)p.ln2_gain,
                          (const void*)p.ln2_bias})
      if (q == nullptr || !aligned16(q)) return SA_ERR_INVALID_ARG;
  }

  sa_stack_s* h = new (std::nothrow) sa_stack_s();
  if (h == nullptr) return SA_ERR_OUT_OF_MEMORY;
  h->d = d;
  h->k = k;
  h->d_ff = d_ff;
  st = sa_create(&h->base, d, k, tau, dtype, P, params[0].W_Q, params[0].W_K, stream);
  if (st != SA_OK) {
    delete h;
    return st;
  }
  h->device = h->base->device;
  hipStream_t s = static_cast<hipStream_t>(stream);
  h->layers.resize(num_layers);
  bool ok = dev_alloc(&h->P, (size_t)k * d) &&
            sa::launch_unfold((int)dtype, P, k, d, h->P, s) == hipSuccess;  // a plain copy to float32
  const size_t dd = (size_t)d * d, dv = (size_t)d, df = (size_t)d * d_ff;
  for (int32_t l = 0; ok && l < num_layers; ++l) {
    const sa_layer_params& p = params[l];
    auto& L = h->layers[l];
    ok = dev_alloc(&L.ln1_g, dv) && dev_alloc(&L.ln1_b, dv) && dev_alloc(&L.ln2_g, dv) && dev_alloc(&L.ln2_b, dv) &&
         dev_alloc(&L.gate_t, df) && dev_alloc(&L.up_t, df) && dev_alloc(&L.down_t, df);
    if (ok && l > 0)
      ok = dev_alloc(&L.wqk_t, dd) && sa::launch_wqk_t((int)dtype, p.W_Q, p.W_K, d, L.wqk_t, s) == hipSuccess;
    ok = ok && hipMemcpyAsync(L.ln1_g, p.ln1_gain, dv * 4, hipMemcpyDeviceToDevice, s) == hipSuccess &&
         hipMemcpyAsync(L.ln1_b, p.ln1_bias, dv * 4, hipMemcpyDeviceToDevice, s) == hipSuccess &&
         hipMemcpyAsync(L.ln2_g, p.ln2_gain, dv * 4, hipMemcpyDeviceToDevice, s) == hipSuccess &&
         hipMemcpyAsync(L.ln2_b, p.ln2_bias, dv * 4, hipMemcpyDeviceToDevice, s) == hipSuccess &&
         sa::launch_transpose(p.ffn_gate, d, d_ff, L.gate_t, s) == hipSuccess &&
         sa::launch_transpose(p.ffn_up, d, d_ff, L.up_t, s) == hipSuccess &&
         sa::launch_transpose(p.ffn_down, d_ff, d, L.down_t, s) == hipSuccess;
  }
  if (ok) ok = hipStreamSynchronize(s) == hipSuccess;  // the caller may free its weights on return
  if (!ok) {
    free_stack(h);
    return SA_ERR_DEVICE;
  }
  *out = h;
  return SA_OK;
}

SA_API void sa_stack_destroy(sa_stack h) {
  if (h == nullptr) return;
  DeviceGuard guard(h->device);
  free_stack(h);
}

SA_API sa_status sa_stack_compress_batch(sa_stack h, const void* X, const int64_t* offsets, int32_t num_users,
                                         float* out, void* stream) {
  if (h == nullptr) return SA_ERR_INVALID_ARG;
  sa_status st = check_batch(offsets, num_users);
  if (st != SA_OK) return st;
  if (num_users == 0) return SA_OK;
  if (out == nullptr || !aligned16(out)) return SA_ERR_INVALID_ARG;
  if (offsets[num_users] > 0 && (X == nullptr || !aligned16(X))) return SA_ERR_INVALID_ARG;

  DeviceGuard guard(h->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Plan& plan = h->base->plan;
  const int d = h->d, k = h->k, d_ff = h->d_ff;
  const size_t elem = plan.dtype == SA_BF16 ? 2 : 4;
  if (num_users > h->cap_users) {
    if (h->cap_users > 0 && hipStreamSynchronize(s) != hipSuccess) return SA_ERR_DEVICE;  // earlier calls may use them
    free_stack_buffers(h);
    const size_t rk = (size_t)num_users * k;
    const size_t mu_bytes = (size_t)num_users * plan.k_pad * d * elem;
    // the folds never write the padding rows k..k_pad-1: zero them once
    const bool ok = hipMalloc(&h->Mu, mu_bytes) == hipSuccess && sa::launch_zero(h->Mu, mu_bytes, s) == hipSuccess &&
                    dev_alloc(&h->y, rk * d) && dev_alloc(&h->xbar, rk * d) && dev_alloc(&h->state, rk * d) &&
                    dev_alloc(&h->ffn_out, rk * d) && dev_alloc(&h->hidden, rk * d_ff);
    if (!ok) {
      free_stack_buffers(h);
      return SA_ERR_OUT_OF_MEMORY;
    }
    h->cap_users = num_users;
  }
  const int64_t rows = (int64_t)num_users * k;
  const float scale = (float)((double)h->base->tau * kLog2e);
  const int nl = (int)h->layers.size();
  // Xbar = LN1(X~(l-1) + Y); X~(l) = LN2(Xbar + FFN(Xbar)); X~(0) = P for every user.  Each residual + layer
  // norm runs as the prologue of the product that reads it (LN1 before the FFN, LN2 of layer l before the
  // fold of layer l + 1), except the last layer's LN2, which writes the output.
  for (int l = 0; l < nl; ++l) {
    const auto& L = h->layers[l];
    if (l == 0) {
      st = compress(h->base, X, offsets, num_users, h->y, stream, h->base->M, 0);
    } else {
      const auto& Lp = h->layers[l - 1];
      const sa::LnPrologue ln2{h->xbar, 0, h->ffn_out, Lp.ln2_g, Lp.ln2_b, kLayerNormEps, h->state};
      if (sa::launch_fold_users(plan.dtype, &ln2, nullptr, L.wqk_t, scale, num_users, k, plan.k_pad, d, h->Mu, s) !=
          hipSuccess)
        return SA_ERR_DEVICE;
      st = compress(h->base, X, offsets, num_users, h->y, stream, h->Mu, (int64_t)plan.k_pad * d);
    }
    if (st != SA_OK) return st;
    const sa::LnPrologue ln1{l == 0 ? h->P : h->state, l == 0 ? k : 0, h->y, L.ln1_g, L.ln1_b, kLayerNormEps,
                             h->xbar};
    if (sa::launch_ffn(&ln1, nullptr, rows, d, d_ff, L.gate_t, L.up_t, L.down_t, h->hidden, h->ffn_out, s) !=
        hipSuccess)
      return SA_ERR_DEVICE;
  }
  if (sa::launch_add_ln(h->xbar, 0, h->ffn_out, h->layers[nl - 1].ln2_g, h->layers[nl - 1].ln2_b, kLayerNormEps, rows,
                        d, out, s) != hipSuccess)
    return SA_ERR_DEVICE;
  return SA_OK;
}

SA_API sa_status sa_stack_set_kernel_timing(sa_stack h, int32_t enable) {
  if (h == nullptr) return SA_ERR_INVALID_ARG;
  return sa_set_kernel_timing(h->base, enable);
}

SA_API sa_status sa_stack_read_kernel_timing(sa_stack h, double* fused_ms, double* reduce_ms,
                                             int64_t* fused_launches) {
  if (h == nullptr) return SA_ERR_INVALID_ARG;
  return sa_read_kernel_timing(h->base, fused_ms, reduce_ms, fused_launches);
}
