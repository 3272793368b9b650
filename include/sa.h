/*
 * sa.h -- C ABI of the MI355X (gfx950) Sketch Attention compression library.
 *
 * The operation (SequenceO1 close-reading page, "SequenceO1: End-to-End
 * Ultra-Long (100K) Sequence Modeling in Recommendation with Low-Rank
 * Caching", section 2.1 "Sketch Attention"): for one user with history
 * X (n x d) and the k shared prototypes P (k x d),
 *
 *     S  = tau * (P W_Q)(X W_K)^T               (k x n affinity)
 *     A  = softmax of S over the prototype axis  (each column sums to one)
 *     X~ = A X                                   (k x d sketch, no value projection)
 *
 * Section 2.4 asks for a fused kernel that never writes the k x n matrices
 * to high-bandwidth memory and that accepts batches of unequal-length
 * histories; that is sa_compress_batch below.  sa_create folds the weights
 * once, M = tau * log2(e) * P W_Q W_K^T (k x d), so the history's key
 * projection X W_K is never formed (section 1 cites the same reordering for
 * single-query cross-attention); exp is then evaluated as exp2.
 *
 * Conventions
 *   - Matrices are dense, row-major, with no padding between rows.
 *   - Row-vector convention: x W, so W[a][b] maps input coordinate a to
 *     output coordinate b.
 *   - "device" pointers are HIP device allocations on the device that is
 *     current when sa_create is called; "host" pointers are ordinary memory.
 *   - Streams are hipStream_t values passed as void* (NULL = null stream).
 *   - Every entry point validates its arguments on the host before any HIP
 *     call or enqueue; on error nothing is enqueued and outputs are not
 *     touched.  Nothing throws across this boundary.
 *   - A handle must not be used from two host threads at once, nor by two
 *     streams whose work can overlap (its workspace is shared).
 *   - The compute entry points (sa_compress_batch, sa_stack_compress_batch,
 *     sa_grad_compute, sa_action_fuse) allocate and synchronise only when a
 *     call needs more workspace than the handle holds (more work groups plus
 *     users in one launch, more rows, or more users for the stack); the
 *     buffers then grow by freeing the old ones.  Otherwise a call enqueues
 *     kernel launches only, no memset or copy nodes, so it can be recorded
 *     by stream capture into a HIP graph and replayed -- but a graph captured
 *     before a later growth still points at the freed buffers and must not be
 *     replayed after it: make the call with the largest workspace need first,
 *     freeze the workspace with sa_reserve, or capture
 *     sa_compress_batch_noalloc, whose workspace never moves.
 *     Kernel timing (the *_set_kernel_timing calls) records events and is for
 *     eager use.
 */
#ifndef SA_H
#define SA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sa_handle_s* sa_handle;

typedef enum sa_status {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = 1,   /* null pointer, bad offsets, non-finite tau, misaligned buffer */
  SA_ERR_UNSUPPORTED = 2,   /* valid request outside what the kernels implement (see sa_create) */
  SA_ERR_OUT_OF_MEMORY = 3, /* device allocation failed */
  SA_ERR_DEVICE = 4         /* a HIP call or kernel launch failed */
} sa_status;

/* Softmax axis of the assignment: SA_NORM_PROTOTYPES is Sketch Attention
 * (section 2.1: each behaviour's weights over the k prototypes sum to one);
 * SA_NORM_HISTORY is the comparator of section 3.1 (Figure 3, Table 1): the
 * usual latent cross-attention, each prototype's weights over the user's n
 * behaviours sum to one, everything else unchanged. */
typedef enum sa_norm {
  SA_NORM_PROTOTYPES = 0,
  SA_NORM_HISTORY = 1
} sa_norm;

typedef enum sa_dtype {
  SA_F32 = 0,   /* float32 inputs, float32 matrix-core products */
  SA_BF16 = 1   /* bfloat16 inputs, float32 accumulation */
} sa_dtype;

/*
 * sa_create -- validate the configuration, copy and fold the weights.
 *
 *   out    host pointer receiving the new handle (set to NULL on error)
 *   d      history / prototype width; supported: 64 or 128
 *   k      number of prototypes; supported: 1..1024 (beyond 512 at d = 128
 *          for SA_BF16, and beyond 256 for SA_F32, the pass runs in two
 *          phases over blocks of 256 prototypes)
 *   tau    affinity scale, finite (any sign, zero allowed)
 *   dtype  element type of P, W_Q, W_K and of every X passed later
 *   P      device, [k][d] prototypes (section 2.1: P^(0), shared by all users)
 *   W_Q    device, [d][d] query projection
 *   W_K    device, [d][d] key projection
 *   stream stream on which the fold runs; sa_create waits for it before
 *          returning, so the caller may free P, W_Q, W_K afterwards
 *
 * The handle owns the folded matrix (computed in float32, rounded once to
 * dtype) and a workspace that grows on demand.  Returns SA_ERR_UNSUPPORTED
 * for a d, k or dtype outside the supported set, SA_ERR_INVALID_ARG for null
 * pointers, non-finite tau or pointers not aligned to 16 bytes.
 */
sa_status sa_create(sa_handle* out, int32_t d, int32_t k, float tau, sa_dtype dtype,
                    const void* P, const void* W_Q, const void* W_K, void* stream);

/*
 * sa_create_ex -- sa_create with a choice of softmax axis.  SA_NORM_HISTORY
 * (the comparator) computes, per user, X~_j = sum_i a_ji x_i with
 * a_ji = exp(S_ji) / sum_i' exp(S_ji') over the user's rows (an empty history
 * gives zeros), for both dtypes over the same d and k range.
 * sa_compress_batch then computes that summary for the handle; all other
 * behaviour is as for sa_create.
 */
sa_status sa_create_ex(sa_handle* out, int32_t d, int32_t k, float tau, sa_dtype dtype,
                       const void* P, const void* W_Q, const void* W_K, sa_norm norm, void* stream);

/*
 * sa_compress_batch -- sketches of a ragged batch of users (section 2.4).
 *
 *   h          handle from sa_create
 *   X          device, [offsets[num_users]][d] packed history rows in the
 *              handle's dtype, 16-byte aligned; user u owns rows
 *              offsets[u] .. offsets[u+1]-1 (section 2.1: X in R^{n x d})
 *   offsets    host, int64 [num_users + 1], offsets[0] == 0, non-decreasing,
 *              offsets[num_users] <= 2^31 - 1 (else SA_ERR_INVALID_ARG)
 *   num_users  U >= 0; U == 0 is a no-op returning SA_OK
 *   out        device, float32 [num_users][k][d], 16-byte aligned, fully
 *              overwritten; a user with no rows gets a zero sketch (empty sum)
 *   stream     the work is only enqueued on this stream (asynchronous):
 *              X and out must stay valid until the stream has passed it
 *
 * X is read from memory once; the k x n affinity and assignment matrices
 * exist only tile by tile in registers.  Results are deterministic: the same
 * inputs give bitwise identical outputs.
 */
sa_status sa_compress_batch(sa_handle h, const void* X, const int64_t* offsets, int32_t num_users,
                            float* out, void* stream);

/*
 * sa_compress_batch_noalloc -- sa_compress_batch for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, result (bitwise, for the
 * same launch split) and errors as sa_compress_batch, but the call never
 * allocates, frees or synchronises: its partial sketches live in a fixed
 * device array of 64 MiB built into the library, one per GPU, held until the
 * process ends.  A launch needs (groups + users) partial slots per prototype
 * block (k_pad * d floats for up to 512 prototypes at d = 128, blocks of 256
 * prototypes above; plus 2 k_pad for SA_NORM_HISTORY) and, for more than 512
 * prototypes at d = 128, 4 (blocks + 1) bytes per row of statistics; users
 * go to launches greedily (at most 256, halved until the launch fits with
 * one work group per block) and the groups are capped to what fits.  If one
 * user alone does not fit (more than about 3 million rows at k = 1024,
 * d = 128), nothing is enqueued and SA_ERR_UNSUPPORTED is returned; every
 * other supported case runs.  Kernel timing is not recorded for it.  All
 * calls on one GPU share the array: calls that can overlap on one GPU (other
 * streams, other handles, other host threads) race and must be serialised by
 * the caller.  The array's device address is looked up on the first call on
 * each GPU (SA_ERR_DEVICE if that fails).
 */
sa_status sa_compress_batch_noalloc(sa_handle h, const void* X, const int64_t* offsets, int32_t num_users,
                                    float* out, void* stream);

/*
 * sa_reserve -- sizes, and optionally freezes, a handle's workspace for
 * callers that record sa_compress_batch into HIP graphs (a graph keeps the
 * workspace's address, which a later growing call would otherwise free).
 *
 *   h          handle from sa_create
 *   max_rows   0 .. 2^31 - 1: the most rows (offsets[num_users]) of a later call
 *   max_users  >= 0: the most users of a later call
 *   freeze     1: later sa_compress_batch calls never free or allocate the
 *              workspace -- a call within the bounds runs exactly as it
 *              would unfrozen, a larger one in more launches sized to the
 *              workspace (as sa_compress_batch_noalloc does), or returns
 *              SA_ERR_UNSUPPORTED if one user alone does not fit; with both
 *              bounds 0 and no workspace yet the handle stays unfrozen.
 *              0: the workspace grows on demand again.
 *   stream     synchronised before an old, smaller workspace is freed
 *
 * Grows the workspace (it never shrinks) to what any call within the bounds
 * needs; call it outside capture.  Errors: SA_ERR_INVALID_ARG (null handle,
 * bounds out of range), SA_ERR_OUT_OF_MEMORY (the handle is then unfrozen),
 * SA_ERR_DEVICE.
 */
sa_status sa_reserve(sa_handle h, int64_t max_rows, int32_t max_users, int32_t freeze, void* stream);

/*
 * sa_destroy -- free the handle and its device memory.  NULL is allowed.
 * The caller must have synchronised every stream that used the handle.
 */
void sa_destroy(sa_handle h);

/* sa_status_string -- static, NUL-terminated description of a status code. */
const char* sa_status_string(sa_status s);

/*
 * Host-only checks with no HIP call, the same ones sa_create and
 * sa_compress_batch run first.  sa_check_config returns what sa_create
 * would return for these scalar arguments with valid pointers;
 * sa_check_batch returns what sa_compress_batch would return for these
 * offsets with valid buffers.
 */
sa_status sa_check_config(int32_t d, int32_t k, float tau, sa_dtype dtype);
sa_status sa_check_batch(int32_t k, const int64_t* offsets, int32_t num_users);

/*
 * sa_get_folded -- write the folded matrix M = tau*log2(e)*P W_Q W_K^T as
 * float32 [k][d] into the device buffer dst (enqueued on stream).  This is
 * the matrix the compression kernels use, after rounding to the dtype.
 */
sa_status sa_get_folded(sa_handle h, float* dst, void* stream);

/*
 * Kernel timing for measurement.  While enabled, each launch of the fused
 * compression kernel and of the partial-sum reduction made by
 * sa_compress_batch carries a start and a stop HIP event that the kernel's
 * own dispatch records on the caller's stream (so the durations are those of
 * the kernels, and no extra work is queued); such launches cost the host more
 * than plain ones.  sa_read_kernel_timing waits for
 * the recorded events, returns the summed durations in milliseconds and the
 * number of fused launches since the previous read, and starts a new count.
 * Any output pointer may be NULL.
 */
sa_status sa_set_kernel_timing(sa_handle h, int32_t enable);
sa_status sa_read_kernel_timing(sa_handle h, double* fused_ms, double* reduce_ms, int64_t* fused_launches);

/*
 * sa_describe_plan -- the launch configuration sa_compress_batch would use
 * for a batch of total_rows rows: workgroups in the fused grid, waves per
 * workgroup that split the prototypes and the rows, rows per tile and the
 * padded prototype count.  Host only; any output pointer may be NULL.
 */
sa_status sa_describe_plan(sa_handle h, int64_t total_rows, int32_t* groups, int32_t* waves_k,
                           int32_t* waves_rows, int32_t* tile_rows, int32_t* k_padded);

/*
 * sa_measure_ceilings -- measured ceilings of the current device, against
 * which the kernels' roofline fractions can be read beside the published
 * peaks: bf16 matrix-core TFLOP/s for loops of independent 16x16x32 and of
 * independent 32x32x16 products on every compute unit (the two instruction
 * shapes do not reach the same rate), float32 FMA TFLOP/s and hardware exp2 evaluations
 * per second on the vector ALUs (loops of independent chains), and the GB/s
 * of a streaming copy (1 GiB read plus 1 GiB written per pass, larger than
 * every cache).  Allocates 2 GiB and a few bytes of scratch, runs on stream
 * and synchronises it; any output pointer may be NULL.  Returns
 * SA_ERR_OUT_OF_MEMORY or SA_ERR_DEVICE on failure.
 */
sa_status sa_measure_ceilings(double* mfma_bf16_tflops, double* mfma_bf16_32x32_tflops, double* valu_fma_tflops,
                              double* exp2_per_sec, double* copy_gbs, void* stream);

/*
 * sa_measure_hbm_read -- GB/s of a read-only stream over 1 GiB (four times
 * the Infinity Cache): 16-byte loads, four or eight in flight per thread,
 * the best over 4 to 32 work groups of 256 threads per compute unit.  The ceiling for kernels that read far more than they
 * write, such as the compression at small k.  Allocates 1 GiB and a few
 * bytes, runs on stream and synchronises it; read_gbs may be NULL.  Returns
 * SA_ERR_OUT_OF_MEMORY or SA_ERR_DEVICE on failure.
 */
sa_status sa_measure_hbm_read(double* read_gbs, void* stream);

/*
 * Stacked refinement (SequenceO1 close-reading page, section 2.2 "Stacked
 * Refinement and action-side fusion").  After one assignment and aggregation
 * the k x d state carries the user's information, so it queries the same raw
 * history again.  Starting from X~(0) = P, layer l = 1..L computes, per user,
 *
 *     Y      = A(l) X     with A(l) the section 2.1 assignment for the query
 *                         X~(l-1): S = tau (X~(l-1) W_Q(l))(X W_K(l))^T,
 *                         softmax over the prototype axis
 *     Xbar   = LN1(X~(l-1) + Y)
 *     X~(l)  = LN2(Xbar + FFN(Xbar)),   FFN(z) = (silu(z W_gate) * (z W_up)) W_down
 *
 * LN normalises each row over its d entries with the population variance and
 * epsilon 1e-5, then applies a per-column gain and bias; silu(x) = x / (1 +
 * e^-x).  The page lost the equations of this update: the post-norm residual
 * form, the SwiGLU FFN (the gated form the page gives for the action fusion)
 * and epsilon are the readings this library takes.  Every layer reads the
 * original history; layer 1 runs the plain SA pass with the shared fold of P,
 * later layers fold each user's state into its own k x d matrix and run the
 * same fused pass with per-user matrices.  The aggregation is in float32
 * from the dtype inputs; LN, FFN and the per-user folds are float32 (the
 * folded matrices are rounded once to the dtype, as in sa_create).
 */
typedef struct sa_stack_s* sa_stack;

/* Weights of one refinement layer: device pointers, row-major, 16-byte aligned. */
typedef struct sa_layer_params {
  const void* W_Q;          /* [d][d], dtype of the stack */
  const void* W_K;          /* [d][d], dtype of the stack */
  const float* ln1_gain;    /* [d] */
  const float* ln1_bias;    /* [d] */
  const float* ffn_gate;    /* [d][d_ff] */
  const float* ffn_up;      /* [d][d_ff] */
  const float* ffn_down;    /* [d_ff][d] */
  const float* ln2_gain;    /* [d] */
  const float* ln2_bias;    /* [d] */
} sa_layer_params;

/*
 * sa_stack_create -- validate, copy every weight (the caller may free them
 * when this returns) and fold layer 1's matrix.
 *
 *   out         host pointer receiving the new handle (NULL on error)
 *   d, k, tau, dtype, P   as for sa_create (P is X~(0), shared by all users)
 *   d_ff        FFN hidden width, a multiple of 64 in 64..8192
 *   num_layers  1..16
 *   params      host array of num_layers layer descriptions
 *   stream      stream for the copies; waited for before returning
 *
 * Errors as sa_create; SA_ERR_UNSUPPORTED also for an unsupported d_ff,
 * SA_ERR_INVALID_ARG for a bad layer count or a null or misaligned pointer.
 */
sa_status sa_stack_create(sa_stack* out, int32_t d, int32_t k, int32_t d_ff, int32_t num_layers, float tau,
                          sa_dtype dtype, const void* P, const sa_layer_params* params, void* stream);

/*
 * sa_stack_compress_batch -- X~(L) for every user of a packed batch.
 * Arguments, ownership, asynchrony and errors as sa_compress_batch; out is
 * float32 [num_users][k][d].  An empty history gives Y = 0 in every layer.
 * The handle holds per-call buffers sized for the largest batch seen (grown
 * on demand, after waiting for the stream); the same concurrency rules as
 * for sa_handle apply.
 */
sa_status sa_stack_compress_batch(sa_stack h, const void* X, const int64_t* offsets, int32_t num_users, float* out,
                                  void* stream);

/* sa_stack_destroy -- release everything the handle owns; NULL is ignored.
 * The caller must have synchronised the streams that used it. */
void sa_stack_destroy(sa_stack h);

/* sa_stack_set_kernel_timing / sa_stack_read_kernel_timing -- as the sa_handle
 * versions, for the fused passes and reductions of every layer (one fused
 * launch per layer and launch of at most 256 users). */
sa_status sa_stack_set_kernel_timing(sa_stack h, int32_t enable);
sa_status sa_stack_read_kernel_timing(sa_stack h, double* fused_ms, double* reduce_ms, int64_t* fused_launches);

/*
 * Backward pass (training miss path).  The close-reading page trains the
 * compression end to end through the fused kernel (sections 2.2 and 2.4);
 * the gradients follow from the definitions of section 2.1 by the chain
 * rule.  For user u with sketch X~_u = A_u X_u and upstream gradient
 * G_u = dL/dX~_u (k x d):
 *   dA = G_u X_u^T, c_i = sum_j A_ji dA_ji, dS = A * (dA - c)
 *   dX_u = A^T G_u + tau dS^T (P W_Q) W_K^T
 *   dP = dQ W_Q^T, dW_Q = P^T dQ, dW_K = tau X^T dS^T (P W_Q), dQ = tau dS X W_K
 * with the weight gradients summed over the users of the batch.
 *
 * sa_grad_check_config -- what sa_grad_create returns for these scalars:
 * d in {64, 128}, 1 <= k <= 1024, SA_BF16 or SA_F32 (else
 * SA_ERR_UNSUPPORTED or SA_ERR_INVALID_ARG as for sa_check_config).  SA_BF16
 * runs two streamed passes; beyond 256 prototypes the row statistics are
 * gathered over blocks of 256 in a first pass, merged, and the gradient of
 * the folded matrix formed in a second pass per block.  SA_F32 works per
 * user on passes of at most 65536 rows with the n x k score, weight and
 * upstream matrices of a pass in the handle's workspace (float32
 * matrix-core products; about 12 (65536 + d) k bytes at most), for callers
 * that need float32 gradients rather than speed.
 *
 * sa_grad_create -- prepare the weights once (device pointers in the dtype,
 * as for sa_create; they are not used after the call returns).  The work is
 * enqueued on stream and synchronised before returning.
 */
typedef struct sa_grad_s* sa_grad;
sa_status sa_grad_check_config(int32_t d, int32_t k, float tau, sa_dtype dtype);
sa_status sa_grad_create(sa_grad* out, int32_t d, int32_t k, float tau, sa_dtype dtype, const void* P,
                         const void* W_Q, const void* W_K, void* stream);

/*
 * sa_grad_compute -- gradients of L for one ragged batch.
 *
 *   X            device, [offsets[num_users]][d] in the dtype, as for sa_compress_batch
 *   offsets      host, int64 [num_users + 1], as for sa_compress_batch
 *   grad_sketch  device, float32 [num_users][k][d], dL/dX~ per user
 *   grad_X       device, [offsets[num_users]][d] in the dtype, fully overwritten
 *   grad_P       device, float32 [k][d]; grad_W_Q, grad_W_K float32 [d][d];
 *                fully overwritten (zero for a batch without rows)
 * All device buffers 16-byte aligned; X and grad_X may be NULL when the
 * batch has no rows.  The work is only enqueued on stream.  Calls on one
 * handle share its workspace and must not overlap (one stream at a time).
 * Errors: SA_ERR_INVALID_ARG for bad arguments (nothing enqueued),
 * SA_ERR_OUT_OF_MEMORY when the workspace cannot grow, SA_ERR_DEVICE for a
 * failed launch.
 */
sa_status sa_grad_compute(sa_grad h, const void* X, const int64_t* offsets, int32_t num_users,
                          const float* grad_sketch, void* grad_X, float* grad_P, float* grad_W_Q, float* grad_W_K,
                          void* stream);

/* sa_grad_set_kernel_timing / sa_grad_read_kernel_timing -- HIP events on the
 * dispatches of the two streamed passes of the last launch of each call
 * (read synchronises them): milliseconds summed over the calls since the
 * last read, and the number of such calls. */
sa_status sa_grad_set_kernel_timing(sa_grad h, int32_t enable);
sa_status sa_grad_read_kernel_timing(sa_grad h, double* stats_ms, double* dx_ms, int64_t* calls);

/* sa_grad_destroy -- free the handle (NULL allowed) after its streams are synchronised. */
void sa_grad_destroy(sa_grad h);

/*
 * Action fusion (section 2.2): the history row of behaviour i is built from
 * the item embedding e_i and the embedding a_i of its action type,
 *   x_i = e_i + (silu(z_i W_gate) * (z_i W_up)) W_down,  z_i = [e_i ; a_i],
 * silu(v) = v / (1 + exp(-v)), no biases.  The page gives neither the action
 * embedding width nor the FFN width: here a_i = action_table[action_i] with
 * d_a columns and the gated layer has d_ff columns (parameters).
 *
 * sa_action_check_config -- d in {64, 128}, d_a a multiple of 8 with
 * d + d_a <= 256, d_ff at most 4096 and, for SA_BF16, a multiple of 64 (of 32
 * when d + d_a > 192 for d = 128), for SA_F32 a multiple of 32;
 * 1 <= n_actions <= 2^20; else SA_ERR_UNSUPPORTED or SA_ERR_INVALID_ARG.
 * SA_BF16 runs one fused pass (bf16 matrix-core products, float32
 * accumulation, x rounded to bf16 once); SA_F32 gathers z into a staging
 * buffer of the handle and runs the FFN as float32 matrix-core products, in
 * passes of 32768 rows.
 *
 * sa_action_create -- device pointers in the dtype, row-major, 16-byte
 * aligned: action_table [n_actions][d_a] (may be NULL when d_a == 0),
 * W_gate and W_up [d + d_a][d_ff], W_down [d_ff][d].  Copied and packed
 * (the caller's buffers are not used after the call); synchronises stream.
 */
typedef struct sa_action_s* sa_action;
sa_status sa_action_check_config(int32_t d, int32_t d_a, int32_t d_ff, int32_t n_actions, sa_dtype dtype);
sa_status sa_action_create(sa_action* out, int32_t d, int32_t d_a, int32_t d_ff, int32_t n_actions, sa_dtype dtype,
                           const void* action_table, const void* W_gate, const void* W_up, const void* W_down,
                           void* stream);

/*
 * sa_action_fuse -- X[i] = x_i for rows i < rows (enqueued on stream).
 *   E        device, [rows][d] in the handle's dtype, 16-byte aligned
 *   actions  device, int32 [rows], 4-byte aligned; ids outside
 *            [0, n_actions) are clamped into it (the device cannot report them)
 *   X        device, [rows][d] in the dtype, 16-byte aligned, fully
 *            overwritten; it is the history input of sa_compress_batch
 * rows == 0 is a no-op.  SA_BF16: calls on one handle may overlap (no
 * workspace).  SA_F32: the handle's staging buffers are reused, so calls on
 * one handle must be ordered (one stream, or synchronised streams).
 */
sa_status sa_action_fuse(sa_action h, const void* E, const int32_t* actions, int64_t rows, void* X, void* stream);

/*
 * sa_action_compress_batch -- out[u] = the sketch (as sa_compress_batch on h)
 * of the rows x_i of user u, formed from E and actions inside the sketch
 * kernel: X is never written to memory (section 2.2 builds the rows the
 * compression of section 2.1 reads; section 2.4 fuses the pass).  E and
 * actions are as for sa_action_fuse, with offsets[num_users] rows, packed as
 * the rows of sa_compress_batch; offsets, out, num_users and the workspace,
 * timing and stream rules are those of sa_compress_batch on h, whose kernel
 * timing covers the fused kernel.  The result equals sa_action_fuse followed
 * by sa_compress_batch bit for bit.
 * SA_ERR_UNSUPPORTED (nothing enqueued) unless a is SA_BF16 with d = 128, h and a are on the
 * same device and h uses the one-pass plan of eight waves of 32 prototypes:
 * SA_BF16, d = 128, 128 < k <= 256, softmax over the prototypes.
 */
sa_status sa_action_compress_batch(sa_action a, sa_handle h, const void* E, const int32_t* actions,
                                   const int64_t* offsets, int32_t num_users, float* out, void* stream);

/* HIP events on the pass's dispatch (as for sa_set_kernel_timing): total
 * milliseconds and launches since the last read. */
sa_status sa_action_set_kernel_timing(sa_action h, int32_t enable);
sa_status sa_action_read_kernel_timing(sa_action h, double* ms, int64_t* launches);

/* sa_action_destroy -- free the handle (NULL allowed) after its streams are synchronised. */
void sa_action_destroy(sa_action h);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
