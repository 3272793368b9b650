// Internal interface of the action-fusion pass (sa_action.hip,
// sa_action_api.cpp).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

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

}  // namespace sa
