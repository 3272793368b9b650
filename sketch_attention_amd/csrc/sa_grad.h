// Internal interface of the backward pass (sa_grad.hip, sa_grad_api.cpp).
// Not part of the public ABI.
//
// For one user, with the folded M = tau log2(e) P W_Q W_K^T (bf16), the
// natural-units fold Q' = tau P W_Q W_K^T (bf16), the upstream gradient
// G = dL/dX~ (k x d) and A the prototype-axis softmax of S = Q' X^T:
//   pass 1 (grad_stats)  per row i: lse_i = log2 sum_j 2^s'_ji (s' in log2
//                        units), c_i = sum_j A_ji (G X^T)_ji, written out;
//                        dQ' += dS X with dS = A * (G X^T - c), split over
//                        groups like the forward partial sketches
//   pass 2 (grad_dx)     dX = A^T G + dS^T Q' per row, with A and dS
//                        recomputed from the row statistics
//   then dQ = tau dQ' W_K, dW_K = tau dQ'^T Q, dP = dQ W_Q^T, dW_Q = P^T dQ.
// For k > 256 pass 1 walks blocks of 256 prototypes twice: a statistics
// phase writes each block's row statistics, a merge combines them into
// (lse_i, c_i), and an aggregation phase forms dS from the merged values and
// adds dS X into per-block partials.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "sa_internal.h"

namespace sa {

// Prototypes per wave in pass 1 and per chunk in pass 2.
constexpr int kGradKW = 32;

// Prototypes per block of pass 1 (eight waves of 32).
constexpr int kGradBlock = 256;

struct GradStatsArgs {
  const void* X;      // bf16 rows of this launch [rows][d]
  const void* M;      // bf16 [blocks * waves * 32][d], tau log2(e) P W_Q W_K^T (padding rows zero)
  const float* G;     // float32 [users][k][d], upstream gradient of this launch's users
  float* stats;       // float32 [rows][4]: lse_i = m_i + log2 l_i (log2 units), c_i, 0, 0
                      // (phase 2 reads it; phases 0 and 1 write it, phase 1 per block)
  float* partial;     // float32 [blocks][groups + 1][waves * 32 * d] in the lane layout of the
                      // forward partials (slot groups of a block, one spare, as the reduction reads them)
  int64_t rows;
  int32_t users;
  int32_t k;
  int32_t force_shift;  // 1: every row block takes the shifted (row maximum) path
  int32_t phase;        // 0: one block; 1: block statistics [blocks][rows][4] = (m, l, sum 2^(s'-m) dA, 0)
                        // into stats; 2: aggregation from the merged (lse, c) in stats
  int32_t blocks;       // prototype blocks (work group b % blocks takes block b % blocks)
  int64_t offsets[kMaxUsersPerLaunch + 1];
};

struct GradDxArgs {
  const void* X;        // bf16 [rows][d]
  const float* stats;   // as written by pass 1
  const void* packed;   // per user and 32-prototype chunk: M, G, G^T, Q'^T blocks (pack kernel)
  void* dX;             // bf16 [rows][d]
  int64_t rows;
  int32_t users;
  int32_t k;
  int32_t chunks;       // k_pad / 32
  int64_t offsets[kMaxUsersPerLaunch + 1];
};

// Bytes of one packed chunk: four 32 x d bf16 blocks.
constexpr int grad_chunk_bytes(int d) { return 4 * kGradKW * d * 2; }

// Waves per group of pass 1 for k prototypes (blocks of 32 * waves prototypes), 0 when unsupported.
int grad_stats_waves(int k);
// Blocks of pass 1 for k prototypes.
inline int grad_stats_blocks(int k) { return k > kGradBlock ? (k + kGradBlock - 1) / kGradBlock : 1; }
// Merge of phase 1's block statistics into (lse, c) per row.
hipError_t launch_grad_merge(const float* bstats, int64_t rows, int blocks, float* stats, hipStream_t s);

hipError_t launch_grad_stats(int d, int waves, const GradStatsArgs& a, int groups, hipStream_t s,
                             hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
hipError_t launch_grad_dx(int d, const GradDxArgs& a, int groups, hipStream_t s, hipEvent_t start = nullptr,
                          hipEvent_t stop = nullptr);
hipError_t grad_occupancy(int d, int waves, int* stats_groups_per_cu, int* dx_groups_per_cu);
// packed[u][c] for users 0..users-1 of G (float32 [users][k][d]) and the shared bf16 M and Q' [k_pad][d].
hipError_t launch_grad_pack(const void* M, const void* Qp, const float* G, int users, int k, int chunks, int d,
                            void* packed, hipStream_t s);
// C[m][n] = alpha sum_t A[m * a_rs + t * a_cs] B[t * b_rs + n * b_cs], float32, C [rows][cols].
constexpr int kInnerStage = 256;  // inner elements staged in LDS at a time
struct Matmul {
  const float* A;
  int64_t a_rs, a_cs;
  const float* B;
  int64_t b_rs, b_cs;
  int rows, cols, inner;
  float alpha;
  float* C;
};
struct MatmulPair {
  Matmul p[2];
};
// Both products in one launch (independent of each other).
hipError_t launch_small_matmuls(const Matmul& a, const Matmul& b, hipStream_t stream);
// dst[i] += src[i] for n floats.
hipError_t launch_add(float* dst, const float* src, int64_t n, hipStream_t s);
// dst[i] = 0 for n floats (a kernel, not a memset).
hipError_t launch_zero(float* dst, int64_t n, hipStream_t s);

}  // namespace sa
