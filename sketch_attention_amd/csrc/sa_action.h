// Internal interface of the action-fusion passes (sa_action.hip,
// sa_action_sa.hip, sa_action_api.cpp).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "sa.h"
#include "sa_internal.h"

namespace sa {

struct ActionArgs {
  const void* E;         // bf16 [rows][d] item embeddings
  const int32_t* actions;  // [rows] action-type ids (clamped to [0, n_actions))
  const void* table;     // bf16 [n_actions][d_a] action-type embeddings
  const void* packed;    // packed weight chunks (launch_action_pack)
  void* X;               // bf16 [rows][d] output rows
  int64_t rows;
  int32_t n_actions;
  int32_t d_a;           // multiple of 8
  int32_t chunks;        // d_ff / 32, a multiple of the chunks per step
};

// K of the gate and up products: d + d_a rounded up to a multiple of 64.
int action_kpad(int d, int d_a);
// Chunks of 32 FFN columns per step of the pass (1 or 2): d_ff must be a multiple of 32 times this.
int action_chunks_per_step(int d, int kp);
size_t action_packed_bytes(int d, int kp, int d_ff);
// W_gate, W_up bf16 [d + d_a][d_ff], W_down bf16 [d_ff][d] -> packed chunks.
hipError_t launch_action_pack(int d, int kp, const void* Wg, const void* Wu, const void* Wd, int d_a, int d_ff,
                              void* packed, hipStream_t stream);
hipError_t launch_action_fuse(int d, int kp, const ActionArgs& a, int groups, hipStream_t stream,
                              hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
hipError_t action_occupancy(int d, int kp, int* groups_per_cu);
// float32 path (with launch_transpose_pad of sa_internal.h): the gathered rows
// Z [rows][k_pad] = [E; table[clamp(action)]; 0].
hipError_t launch_action_gather_f32(const float* E, const int32_t* actions, const float* table, int64_t rows, int d,
                                    int d_a, int k_pad, int n_actions, float* Z, hipStream_t stream);

// The action fusion as the prologue of the one-pass sketch kernel of eight
// waves of 32 prototypes (sa_action_sa.hip): sa as for that kernel with
// sa.X unused; E and actions start at the launch's first row.
struct ActSaArgs {
  FusedArgs sa;
  const void* E;           // bf16 [rows][128]
  const int32_t* actions;  // [rows]
  const void* table;       // bf16 [n_actions][d_a]
  const void* packed;      // packed weight chunks (launch_action_pack)
  int32_t n_actions;
  int32_t d_a;
  int32_t chunks;          // d_ff / 32
};
// kp: 128, 192 or 256 (action_kpad(128, d_a)).  occ != nullptr: report the work
// groups that fit on a compute unit instead of launching.
hipError_t launch_action_sa(int kp, const ActSaArgs& a, const Launch& l, int* occ = nullptr);

// Where the fused variant takes its rows from, for the sketch handle's batch
// loop (sa_api.cpp).
struct ActionSource {
  const void* E;
  const int32_t* actions;
  const void* table;
  const void* packed;
  int32_t n_actions, d_a, d_ff, kp;
  int device;  // of the action handle
};
// The sketch of the fused rows of a packed batch into out [U][k][d]: the
// batch loop of sa_compress_batch with the fused kernel in place of the
// sketch kernel.  SA_ERR_UNSUPPORTED unless the handle's plan is the one-pass
// plan of eight waves of 32 prototypes (bf16, d = 128, 128 < k <= 256,
// softmax over the prototypes) on src.device.
sa_status compress_actions(sa_handle h, const ActionSource& src, const int64_t* offsets, int32_t num_users,
                           float* out, void* stream);

}  // namespace sa
