// Internal interface between the host library (sa_api.cpp) and the HIP
// kernels (sa_kernels.hip, sa_fused_*.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace sa {

// Users whose offsets travel inline in one launch's kernel arguments.  A
// batch with more users is processed in consecutive launches of at most this
// many users each.
constexpr int kMaxUsersPerLaunch = 256;

// Rows of the history tile that one wave handles per step.
constexpr int kRowsPerWave = 32;

// Launch configuration of the fused pass for one (dtype, d, k).
struct Plan {
  int dtype;        // 0 = f32, 1 = bf16 (sa_dtype)
  int d;            // 64 or 128
  int k;            // prototypes
  int k_pad;        // waves_k * kw
  int kw;           // prototypes per wave (multiple of 16)
  int waves_k;      // waves splitting the prototype axis
  int waves_rows;   // waves splitting the rows of a tile (waves_k * waves_rows waves per group)
  int m_in_lds;     // folded matrix staged in LDS (1) or held in registers (0)
  int tile_rows;    // rows per tile: kRowsPerWave * waves_rows (lockstep), 16 * row_blocks * waves_rows (streamed)
  int kind;         // 0 = lockstep pass (sa_fused.hpp), 1 = streamed pass (sa_stream.hpp, bf16),
                    // 2 = streamed pass on 32x32x16 products (sa_stream32.hpp: bf16, d = 128, 8 x 32 prototypes),
                    // 3 = the same products with the prototypes along the lanes (sa_wide.hpp)
  int prefetch;     // streamed pass: LDS ring slots beyond the minimum, plus one (ring of 3 or 4 + prefetch - 1 tiles)
  int row_blocks;   // streamed pass: 16-row blocks per wave and tile (2 or 4)
  int score_buffers;  // streamed pass: affinity tiles in flight per wave (2: M in registers; 1: M in LDS)
  int blocks;       // prototype blocks of kw * waves_k each (k_pad = blocks * kw * waves_k); > 1: two-phase pass
};

// Arguments of the fused kernel (passed by value in the dispatch packet).
struct FusedArgs {
  const void* X;        // rows of this launch, [rows][d]
  const void* M;        // folded matrix [k_pad][d] in the dtype, or one per user (m_stride apart)
  int64_t m_stride;     // elements between the folded matrices of consecutive users; 0: one shared matrix
  int32_t history_softmax;  // 1: the comparator (softmax over the history axis); partial slots of k_pad (d + 2) floats
  float* partial;       // [slots][k_pad * d] float32, slot = group + user
  int64_t rows;         // rows in this launch (offsets[users])
  int32_t users;        // users in this launch (<= kMaxUsersPerLaunch)
  int32_t k;            // real prototype count (rows k..k_pad-1 of M are padding)
  // Two-phase pass (prototypes in `blocks` blocks of the plan's kw * waves_k
  // rows of M): lse_mode 1 writes each row's log2 sum_j 2^s'_ji over every
  // block into stats [blocks][rows]; lse_mode 2 reads the row's log2 sum over
  // all prototypes from stats [rows] and aggregates 2^(s' - that); 0: the
  // one-pass kernel.  The grid is row ranges x blocks (the blocks of one row
  // range on one XCD when the ranges come in multiples of 8).
  int32_t lse_mode;
  int32_t blocks;
  float* stats;
  int64_t offsets[kMaxUsersPerLaunch + 1];  // relative to this launch's first row
};

struct ReduceArgs {
  const float* partial;  // as above
  int32_t history_softmax;  // partial slots carry (acc, max, sum) per prototype: merge and divide
  float* out;            // [users][k][d] float32
  int64_t rows;
  int32_t users;
  int32_t groups;        // workgroups of the fused launch
  int32_t k;
  int32_t d;
  int32_t kw;
  int32_t k_pad;      // prototypes of one block (one partial slot)
  int32_t blocks;     // prototype blocks; block b's slots follow the (groups + users) slots of block b - 1
  int32_t layout;     // slot layout: 0 as written by sa_fused.hpp / sa_stream.hpp, 1 by sa_stream32.hpp / sa_wide.hpp
  int64_t offsets[kMaxUsersPerLaunch + 1];
};

// Launchers (defined in the .hip translation units).  Non-null start/stop
// events are recorded by the kernel's own dispatch (hipExtLaunchKernelGGL):
// they time the kernel itself and add no packets to the stream.
hipError_t launch_fused(const Plan& plan, const FusedArgs& args, int groups, hipStream_t stream,
                        hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
hipError_t launch_reduce(const ReduceArgs& args, hipStream_t stream, hipEvent_t start = nullptr,
                         hipEvent_t stop = nullptr);
hipError_t launch_fold(int dtype, const void* P, const void* WQ, const void* WK, float scale, int k, int k_pad,
                       int d, float* tmp, void* M, hipStream_t stream);
hipError_t launch_unfold(int dtype, const void* M, int k, int d, float* dst, hipStream_t stream);
// L[i] = log2 sum_b 2^Lb[b][i] for i < rows (the two-phase pass's merge of its per-block statistics).
hipError_t launch_lse_merge(const float* Lb, int64_t rows, int blocks, float* L, hipStream_t stream);
// Zero bytes / 4 words at p (a kernel, never a memset node).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);
// Workgroups of the fused kernel that fit on one compute unit at once.
hipError_t fused_occupancy(const Plan& plan, int* groups_per_cu);

// Bytes of the fixed per-device workspace of sa_compress_batch_noalloc.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
// Device address of that workspace on `device`, which must be the current
// device (looked up on the first call per device, then cached).
hipError_t noalloc_scratch(int device, float** ptr);

// Stacked refinement (sa_refine.hip), all float32 unless noted.
// (W_Q W_K^T)^T (d x d) from weights in the dtype.
hipError_t launch_wqk_t(int dtype, const void* WQ, const void* WK, int d, float* out, hipStream_t stream);
// dst = src^T for a rows x cols matrix.
hipError_t launch_transpose(const float* src, int rows, int cols, float* dst, hipStream_t stream);
// Residual + layer norm computed as the prologue of a product whose A operand it forms:
// A[r] = LN(a[r % a_period (or r when 0)] + b[r]) * gain + bias over d, also stored to out.
struct LnPrologue {
  const float* a;
  int64_t a_period;
  const float* b;
  const float* gain;
  const float* bias;
  float eps;
  float* out;
};
// M[u] = scale * state[u] W_QK in the dtype, [users][k_pad][d], from wqk_t = W_QK^T; padding rows
// k..k_pad-1 are not written (the caller keeps them zero).  With ln, state is ln->a and the rows are
// formed (and stored to ln->out) by the layer norm first.
hipError_t launch_fold_users(int dtype, const LnPrologue* ln, const float* state, const float* wqk_t, float scale,
                             int users, int k, int k_pad, int d, void* M, hipStream_t stream);
// out[r] = LN(a[r % a_period (or r when 0)] + b[r]) * gain + bias over d in {64, 128}.
hipError_t launch_add_ln(const float* a, int64_t a_period, const float* b, const float* gain, const float* bias,
                         float eps, int64_t rows, int d, float* out, hipStream_t stream);
// H = silu(Z W_gate) * (Z W_up) [rows][d_ff], F = H W_down [rows][d]; weights given transposed
// (gate_t, up_t: [d_ff][d]; down_t: [d][d_ff]); d and d_ff multiples of 32.  With ln, Z is ln->a
// and its rows are formed (and stored to ln->out) by the layer norm first.
hipError_t launch_ffn(const LnPrologue* ln, const float* Z, int64_t rows, int d, int d_ff, const float* gate_t,
                      const float* up_t, const float* down_t, float* H, float* F, hipStream_t stream);
// H = silu(Z W_gate) * (Z W_up) [rows][d_ff], X = resid + H W_down [rows][d_out] (float32), with the
// weights given transposed (gate_t, up_t: [d_ff][k_in]; down_t: [d_out][d_ff]); k_in a multiple of 16,
// d_out and d_ff multiples of 32.
// C = A Bt^T ([M][N] float32; A [M][K], Bt [N][K] row-major), plus resid[M][N] when resid is not null
// (resid may be C itself); K a multiple of 16, N a multiple of 32.  long_k splits the reduction over
// eight waves (for K in the thousands), else two.
hipError_t launch_f32_gemm(const float* A, int64_t M, int K, const float* Bt, int N, float* C, const float* resid,
                           bool long_k, hipStream_t stream);
// dst = src^T with the rows of src (rows_in of them, cols wide) padded by zeros to rows_pad: [cols][rows_pad].
hipError_t launch_transpose_pad(const float* src, int64_t rows_in, int cols, int64_t rows_pad, float* dst,
                                hipStream_t stream);
// Backward of the prototype-axis softmax, one row per wave (float32): for each of `rows` rows of S and DA
// ([rows][ld], the first k columns real), A = softmax(S_i) over j < k, c_i = sum_j A_ij DA_ij, and
// DS_ij = A_ij (DA_ij - c_i); A overwrites S and DS overwrites DA (columns k..ld-1 become 0).
hipError_t launch_softmax_grad_rows(float* S, float* DA, int64_t rows, int k, int ld, hipStream_t stream);
hipError_t launch_plain_ffn(const float* Z, int64_t rows, int k_in, int d_out, int d_ff, const float* gate_t,
                            const float* up_t, const float* down_t, float* H, const float* resid, float* X,
                            hipStream_t stream);

// Plan groups, one translation unit each (see sa_fused_*.hip).  With
// occ != nullptr they report occupancy instead of launching.
// Launch description handed to the per-plan dispatchers.
struct Launch {
  int groups;
  hipStream_t stream;
  hipEvent_t start, stop;  // optional, recorded by the dispatch
};
// occ != nullptr: report how many work groups of the plan fit on a CU instead of launching.
using DispatchFn = hipError_t (*)(const Plan&, const FusedArgs&, const Launch&, int*);
hipError_t dispatch_bf16_d64(const Plan&, const FusedArgs&, const Launch&, int*);
hipError_t dispatch_bf16_d128(const Plan&, const FusedArgs&, const Launch&, int*);
hipError_t dispatch_f32_d64(const Plan&, const FusedArgs&, const Launch&, int*);
hipError_t dispatch_f32_d128(const Plan&, const FusedArgs&, const Launch&, int*);
hipError_t dispatch_stream_d64(const Plan&, const FusedArgs&, const Launch&, int*);
hipError_t dispatch_stream_d128(const Plan&, const FusedArgs&, const Launch&, int*);

}  // namespace sa
