/*
 * lopt.h - C ABI of the small_fc_lopt learned-optimizer step on MI355X (gfx950).
 *
 * The operation (PyLO page, "PyLO: Towards Accessible Learned Optimizers in
 * PyTorch", sections "Library design" and "CUDA kernel design: two-pass
 * fusion"): an optimizer keeps per-parameter accumulators, and each step
 * builds a feature vector for every parameter element, normalises each
 * feature with a statistic of its squares over the whole tensor (kernel 1),
 * then rebuilds the features, runs a small MLP per element and applies the
 * resulting update (kernel 2).
 *
 * Per element (i, j) of a tensor viewed as rows x cols (a 1-D tensor of length
 * n is 1 x n), at step t = 1, 2, ...:
 *   m_a <- b_a m_a + (1-b_a) g   (a = 1..3),   v <- b_v v + (1-b_v) g^2
 *   r_k <- f_k r_k + (1-f_k)(mean_j g^2 + eps_f),  c_k likewise over i (k = 1..3)
 *   28 features: g, p, m_a, v, m_a/sqrt(v+eps_v), 1/sqrt(v+eps_v), g rho_k,
 *     1/sqrt(r_k[i]), 1/sqrt(c_k[j]), m_a rho_k with
 *     rho_k = (r_k[i] c_k[j] / mean_i r_k)^(-1/2)
 *   each feature divided by sqrt(mean over the tensor of its square + eps_norm)
 *   x = [28 normalised features, tanh(t / tau_q) for q < n_time]
 *   (the VeLO-shaped variant, n_feat = 19, feeds only the first 19 features:
 *   the same page gives VeLO a feature width of about 30 and the same two
 *   kernels; which features is this library's reading)
 *   (dir, mag) = W3 relu(W2 relu(W1 x + b1) + b2) + b3
 *   u = dir exp(mag exp_mult) step_mult;  p <- p - lr u - lr wd p
 *
 * All arithmetic on the device is fp32.  Every call returns an lopt_status;
 * no C++ exception crosses this boundary.  lopt_last_error() gives a
 * thread-local message for the last failing call on the calling thread.
 * A handle is not thread-safe, and the calls on one handle must be ordered on
 * the device: each step reads and writes the handle's workspace, so issue them
 * on one stream (or order the streams yourself).
 */
#ifndef LOPT_H
#define LOPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOPT_N_FEATURES 28    /* per-element features, each normalised per tensor */
#define LOPT_VELO_FEATURES 19 /* per-element features of the VeLO-shaped variant */
#define LOPT_HIDDEN 32     /* width of both hidden layers */
#define LOPT_MAX_TIME 11   /* maximum number of step (time) features */

typedef enum lopt_status {
  LOPT_OK = 0,
  LOPT_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad shape, aliasing, bad config */
  LOPT_ERR_UNSUPPORTED = 2,      /* a tensor with 2^31 or more elements, misalignment */
  LOPT_ERR_WORKSPACE = 3,        /* workspace too small or not 256-byte aligned */
  LOPT_ERR_HIP = 4,              /* a HIP runtime call or kernel launch failed */
  LOPT_ERR_STATE = 5             /* tensor list differs from the one given to init_state */
} lopt_status;

/* Implementation of the per-element MLP in the apply kernel. */
typedef enum lopt_mlp_impl {
  LOPT_MLP_AUTO = 0, /* LOPT_MLP_BF16X8: the fastest of the paths with
                        fp32 arithmetic (each product within one fp32
                        rounding, accumulation in fp32: LOPT_MLP_BF16X8,
                        LOPT_MLP_BF16X9, LOPT_MLP_MFMA, LOPT_MLP_VALU);
                        lopt_get_mlp_impl tells which path runs */
  LOPT_MLP_VALU = 1, /* vector FMA, weights broadcast from scalar registers */
  LOPT_MLP_MFMA = 2, /* fp32 matrix-core path (v_mfma_f32_32x32x1_2b_f32 and
                        v_mfma_f32_32x32x2_f32) */
  LOPT_MLP_BF16X6 = 3, /* bf16 matrix-core path with every fp32 operand split
                          exactly into three bf16 pieces and the six largest
                          piece products accumulated in fp32
                          (v_mfma_f32_32x32x16_bf16); the dropped products are
                          below 2^-21 of each product (median below one fp32
                          rounding) */
  LOPT_MLP_FP16X3 = 4, /* fp16 matrix-core path (v_mfma_f32_32x32x16_f16): the
                          features normalised first, W1 and W2 scaled by powers
                          of two that put their largest weights in [4, 8),
                          every operand split into two fp16 pieces (22
                          significant bits) and the three largest piece
                          products accumulated in fp32; a wave whose layer-2
                          inputs leave fp16's range is rescaled by a power of
                          two.  Faster than LOPT_MLP_BF16X6 and as accurate;
                          a normalised input far below 1 keeps an absolute
                          floor of 2^-25.  lopt_create / lopt_set_config refuse it
                          (LOPT_ERR_UNSUPPORTED) for weights of magnitude
                          2^15 or more, or whose first-layer row-feature
                          weights are too large for its constant term.
                          Narrower than fp32 (22-bit operands). */
  LOPT_MLP_BF16X9 = 5, /* bf16 matrix-core path with every fp32 operand split
                          exactly into three bf16 pieces and all nine piece
                          products (each exact in fp32) accumulated in fp32
                          (v_mfma_f32_32x32x16_bf16): the products of an fp32
                          GEMM, exactly, with fp32 accumulation */
  LOPT_MLP_BF16X8 = 6  /* as LOPT_MLP_BF16X9 without the product of the two
                          low pieces, which is below 2^-30 of the product:
                          every product within 1/64 of one fp32 rounding,
                          accumulated in fp32 */
} lopt_mlp_impl;

/* How lopt_step launches a step.  The PyLO page counts kernel launches as a
 * cost of the step ("Naive implementation bottleneck": 74-252 per step; "Use
 * of the memory hierarchy": 30-114 once fused into its two passes). */
typedef enum lopt_launch {
  LOPT_LAUNCH_AUTO = 0,   /* LOPT_LAUNCH_SPLIT, the faster of the two at every
                             list size measured (65,536 to 4.2 M elements) */
  LOPT_LAUNCH_SPLIT = 1,  /* five kernels: row/column sums of g^2, row/column
                             moving averages, statistics pass, per-tensor
                             finalize, apply pass */
  LOPT_LAUNCH_SINGLE = 2  /* one kernel that runs the same five passes in turn,
                             separated by grid-wide barriers, with a grid no
                             larger than the device keeps resident at once.
                             Results are bit for bit those of
                             LOPT_LAUNCH_SPLIT; slower (each barrier, which
                             writes back and invalidates the caches of every
                             block across the device's eight XCDs, costs more
                             than a kernel boundary).  Each barrier wait is
                             bounded (~2 s): if the blocks of the grid cannot
                             all become resident (a persistent kernel of
                             another stream holds the device), the step ends
                             with invalid results and lopt_get_step reports
                             LOPT_ERR_HIP */
} lopt_launch;

/* Hyperparameters.  lopt_default_config() fills the defaults shown. */
typedef struct lopt_config {
  float beta_m[3];    /* momentum decays, default 0.1, 0.5, 0.9 */
  float beta_v;       /* second-moment decay, default 0.999 */
  float beta_f[3];    /* row/column second-moment decays, default 0.9, 0.99, 0.999 */
  float eps_v;        /* inside 1/sqrt(v + eps_v), default 1e-8; with 0, an element whose v is
                         exactly 0 (a zero gradient from zero state) has infinite features and
                         makes its tensor's update unspecified for that step */
  float eps_f;        /* added to the row/column means of g^2, default 1e-20 */
  float eps_norm;     /* inside the feature normaliser's root, default 1e-30 */
  float exp_mult;     /* default 1e-3 */
  float step_mult;    /* default 1e-3 */
  float lr;           /* multiplies the whole update, default 1 */
  float weight_decay; /* decoupled: p <- p - lr u - lr wd p, default 0 */
  int32_t n_time;     /* number of tanh(t/tau) step features, 0..11, default 11 */
  float timescales[LOPT_MAX_TIME]; /* tau_q, default 1,3,10,30,100,300,1e3,3e3,1e4,3e4,1e5 */
  int32_t mlp_impl;   /* lopt_mlp_impl */
  int32_t n_feat;     /* per-element MLP inputs: LOPT_N_FEATURES (small_fc_lopt,
                         default) or LOPT_VELO_FEATURES (features 0..18 only) */
  int32_t launch;     /* lopt_launch, default LOPT_LAUNCH_AUTO */
} lopt_config;

/* One parameter tensor.  All pointers are device pointers (hipMalloc / torch),
 * fp32, contiguous, 4-byte aligned.
 *   param: rows*cols values, row-major; updated in place by lopt_step.
 *   grad:  rows*cols values; read only.  Its address may change between steps.
 *          NULL: in lopt_step, the tensor is skipped for that step (its
 *          parameters and state stay as they are, as torch optimizers skip a
 *          parameter without a gradient; t still advances).  lopt_workspace_bytes
 *          and lopt_init_state ignore it.
 *   state: lopt_state_floats(rows, cols) values, owned by the caller and
 *          updated in place.  Layout (each block contiguous):
 *            m1 | m2 | m3 | v      (rows*cols each, row-major)
 *            r1 | r2 | r3          (rows each)
 *            c1 | c2 | c3          (cols each)
 *   rows, cols: >= 1, rows*cols < 2^31, and cols < 2^28 when rows > 1
 *          (UNSUPPORTED otherwise).  A 1-D tensor of length n is
 *          passed as rows = 1, cols = n; then c_k is per element and r_k is a
 *          single value.
 * grad must not overlap param or state; no two tensors may overlap. */
typedef struct lopt_tensor {
  float* param;
  const float* grad;
  float* state;
  int64_t rows;
  int64_t cols;
} lopt_tensor;

typedef struct lopt_handle lopt_handle;

/* Fills *out with the default hyperparameters.  Errors: out == NULL. */
lopt_status lopt_default_config(lopt_config* out);

/* Number of floats in the packed MLP weights for n_feat per-element features
 * and n_time step features: W1[32][n_feat+n_time], b1[32], W2[32][32],
 * b2[32], W3[2][32], b3[2] (row-major, out x in).  2402 for (28, 11), 2114
 * for (19, 11).  Returns 0 if n_feat or n_time is out of range. */
size_t lopt_mlp_floats(int32_t n_feat, int32_t n_time);

/* Creates the optimizer object: the PyLO page's "Library design" section
 * describes the learned optimizer as an object that holds the meta-learned
 * MLP's weights and is then stepped over a model's parameters; the handle is
 * that object (the weights and hyperparameters; the per-parameter state stays
 * in the caller's buffers, bound by lopt_init_state).
 * Creates a handle on the current HIP device.  cfg: hyperparameters (copied);
 * mlp_host: host pointer to lopt_mlp_floats(cfg->n_feat, cfg->n_time) floats (copied to
 * device memory that the handle owns).  The call is synchronous.
 * Errors: null pointers or out-of-range config -> INVALID_ARGUMENT;
 * allocation/copy failure -> HIP.  *out is set only on success. */
lopt_status lopt_create(const lopt_config* cfg, const float* mlp_host, lopt_handle** out);

/* Frees the handle, its device memory and its pinned host buffer (not the
 * caller's buffers).  The caller must make sure no step using the handle is
 * still running. */
void lopt_destroy(lopt_handle* h);

/* Floats in one tensor's state buffer: 4*rows*cols + 3*(rows + cols);
 * 0 for an invalid shape. */
size_t lopt_state_floats(int64_t rows, int64_t cols);

/* Bytes of device workspace that lopt_init_state/lopt_step need for this
 * tensor list (n tensors).  h may be NULL (the size depends only on the list);
 * no device call is made.  Errors: as lopt_init_state's validation. */
lopt_status lopt_workspace_bytes(const lopt_handle* h, const lopt_tensor* ts, int32_t n,
                                 size_t* bytes);

/* The per-parameter accumulators of "Library design" (momentum and
 * second-moment moving averages, and the factored row/column averages of the
 * feature families the page names) start at zero for a new optimizer; this
 * call binds them.
 * Binds the tensor list to the handle: validates it, lays out the plan (per-
 * tensor descriptors, work lists and reduction buffers) inside `workspace`,
 * zero-fills every state buffer and sets the step counter to 0.  workspace:
 * device pointer, 256-byte aligned, >= lopt_workspace_bytes(); owned by the
 * caller, which must keep it alive and untouched until the last lopt_step.
 * stream: a hipStream_t (NULL = default stream); the call returns after the
 * plan upload and the zero fill have been queued and the upload has finished.
 * The first binding (and one with more tensors than any before) allocates a
 * pinned host buffer of 32 bytes per tensor, owned by the handle, through which
 * lopt_step passes changed gradient pointers and per-tensor values.
 * To start from pre-warmed accumulators, write the state buffers after this
 * call.  Errors: validation -> INVALID_ARGUMENT / UNSUPPORTED / WORKSPACE
 * (nothing is modified); a current device other than the handle's ->
 * INVALID_ARGUMENT; HIP failure -> HIP. */
lopt_status lopt_init_state(lopt_handle* h, const lopt_tensor* ts, int32_t n, void* workspace,
                            size_t ws_bytes, void* stream);

/* Row shards.  The PyLO page ("Benchmark results" > "Distributed optimization
 * step") distributes the step across GPUs, and lists as future work
 * ("Limitations and outlook" > "Future directions") a sharded step whose
 * exchange is only the d_feat feature statistics.  Here each rank binds its
 * share of every tensor (a 2-D tensor: some of its rows, all of its columns;
 * a 1-D tensor: some of its elements), and a step runs in three phases with
 * two sums exchanged (summed over the ranks, e.g. by an all-reduce) between
 * them: after phase 0, the column sums of g^2 of each 2-D tensor and the sum
 * of g^2 of each 1-D tensor (the column means and a 1-D tensor's r_k need
 * every row); after phase 1, per tensor, the sums of the squares of the 28
 * features and of r_k over the rows (the normalisers and the mean of r_k).
 * The step's result on every shard is then the whole tensor's step restricted
 * to the shard's rows or elements.
 *
 * global_dims: 2 n values, the (rows, cols) of the whole tensor each list
 * entry is a shard of.  A whole tensor with rows > 1 is a matrix: its shard
 * must have cols columns and at most rows rows (one row stays a matrix); a
 * whole tensor with rows == 1 is 1-D: its shard is 1 x (at most cols).
 * Rows and cols lie in [1, 2^40]; a matrix has fewer than 2^28 columns.
 * Errors: as lopt_workspace_bytes / lopt_init_state, and shards that do not
 * fit global_dims -> INVALID_ARGUMENT. */
lopt_status lopt_workspace_bytes_sharded(const lopt_handle* h, const lopt_tensor* ts, int32_t n,
                                         const int64_t* global_dims, size_t* bytes);

/* Binds a list of row shards as lopt_init_state binds a list (state zeroed,
 * t = 0, the same workspace, stream and error rules), with the exchange
 * buffers in the workspace.  Such a binding steps with lopt_step_shard only
 * (lopt_step returns LOPT_ERR_STATE). */
lopt_status lopt_init_state_sharded(lopt_handle* h, const lopt_tensor* ts, int32_t n, const int64_t* global_dims,
                                    void* workspace, size_t ws_bytes, void* stream);

/* The exchange buffers of a row-shard binding, device pointers into its
 * workspace: sums1 (n1 floats: per list entry in order, cols floats for a
 * matrix shard, 1 for a 1-D shard) and sums2 (n2 = 32 n floats: per entry,
 * 28 feature sums, 3 sums of r_k, 1 unused).  Every rank's buffers have the
 * same layout when the ranks bind shards of the same tensors in the same
 * order.  Errors: NULL argument -> INVALID_ARGUMENT; no row-shard binding ->
 * STATE. */
lopt_status lopt_get_shard_sums(const lopt_handle* h, float** sums1, size_t* n1, float** sums2, size_t* n2);

/* One phase of a row-shard step, queued on `stream` (asynchronous):
 *   phase 0: row and column sums of g^2; writes sums1 (this shard's sums);
 *   -- the caller replaces sums1 by its sum over the ranks, on the stream --
 *   phase 1: moving averages (from the summed sums1), statistics pass;
 *            writes sums2 (this shard's sums);
 *   -- the caller replaces sums2 by its sum over the ranks --
 *   phase 2: normalisers from the summed sums2, apply pass; advances t.
 * Phases run in the order 0, 1, 2, 0, ...; ts as for lopt_step, gradient
 * pointers read at phase 0 (a change in a later phase is refused).  With one
 * rank (no exchange) the three phases give lopt_step's result for the whole
 * tensors, bit for bit.  The phases always run as separate kernels
 * (lopt_config.launch does not apply).  Errors: no row-shard binding, a phase
 * out of order, or a different list -> STATE; as lopt_step otherwise.  On
 * error nothing is queued and the expected phase does not change. */
lopt_status lopt_step_shard(lopt_handle* h, const lopt_tensor* ts, int32_t n, int32_t phase, void* stream);

/* Bytes of the device array behind lopt_init_state_static, per GPU. */
#define LOPT_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate memory: code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid allocation.  Binds the
 * tensor list as lopt_init_state does, but lays the plan out in a device
 * array of LOPT_STATIC_SCRATCH_BYTES that the library holds on each GPU (from
 * the first such call on it until the process ends) instead of in a caller
 * workspace, and allocates no memory, device or pinned (lopt_create has
 * allocated the handle's weights before).  A list whose lopt_workspace_bytes
 * exceeds LOPT_STATIC_SCRATCH_BYTES is refused with LOPT_ERR_WORKSPACE, and
 * nothing changes.  The array is shared by every call on that GPU and keeps
 * the last binding's contents: a binding made here (from any handle) replaces
 * the previous static binding on that device, whose handle then gets
 * LOPT_ERR_STATE from lopt_step, lopt_get_step, lopt_set_step and
 * lopt_get_tensor_stats until it is bound again; calls on one GPU that
 * overlap in time (from two threads, or steps of two static bindings queued
 * on different streams) race on the array.  With such a binding, gradient
 * pointers and per-tensor values that change between steps are copied from
 * the handle's host memory and lopt_step then waits for `stream`.  Otherwise
 * as lopt_init_state: state zero-filled, t = 0, the same stream semantics and
 * errors. */
lopt_status lopt_init_state_static(lopt_handle* h, const lopt_tensor* ts, int32_t n, void* stream);

/* The optimizer's step ("Library design": one call per training iteration
 * updates every parameter), computed as "CUDA kernel design: two-pass fusion"
 * > "Fused kernel strategy" lays it out: a statistics pass that sums each
 * feature's squares over every tensor (kernel 1), then a pass that rebuilds
 * the features, normalises them with those sums, evaluates the MLP per
 * element and writes the update (kernel 2); the row/column averages the
 * features need come first, from a pass over the gradients.
 * One optimizer step over the bound tensor list: queues the five kernels of
 * the step, or the one kernel that runs them in turn (lopt_config.launch), on
 * `stream` and returns (asynchronous); the step's finalize pass advances t.  An empty list queues nothing and leaves t unchanged.  ts must
 * list the same tensors (param, state, rows, cols) in the same order as
 * lopt_init_state; grad pointers may differ from the previous call's: the new
 * pointers are copied to the device on `stream` from the handle's pinned
 * buffer (two slots used in turn; the host waits only for the copy queued two
 * changes earlier, which has normally finished), as are per-tensor values set
 * since the last step.  Such a change cannot be captured into a graph
 * (INVALID_ARGUMENT while `stream` is capturing): call lopt_step once with
 * the new gradients before capturing.  Errors: a
 * different list -> STATE; bad pointers, or a current device other than the
 * handle's -> INVALID_ARGUMENT;
 * launch failure -> HIP.  On a validation
 * error nothing is queued.  Non-finite inputs are not checked (they propagate
 * into the accumulators). */
lopt_status lopt_step(lopt_handle* h, const lopt_tensor* ts, int32_t n, void* stream);

/* Step counter: the number of steps taken (t of the last step).  The counter
 * lives in the workspace and the step's finalize kernel advances it, so steps
 * replayed from a captured HIP graph see t = 1, 2, 3, ...  Waits for the
 * device (hipDeviceSynchronize); 0 before lopt_init_state.  Errors: a
 * one-launch step since the binding whose grid barrier timed out
 * (LOPT_LAUNCH_SINGLE) -> HIP (*t is still set); copy failure -> HIP. */
lopt_status lopt_get_step(const lopt_handle* h, int64_t* t);

/* Sets the step counter (to resume from saved state); t >= 0.  Waits for the
 * device, then writes the counter.  Errors: t < 0 -> INVALID_ARGUMENT; no
 * bound list -> STATE. */
lopt_status lopt_set_step(lopt_handle* h, int64_t t);

/* Replaces the hyperparameters for the following lopt_step calls, e.g. a
 * learning-rate schedule or a new weight decay (the PyLO page, "Library
 * design" and "Effect of learning-rate schedules and weight decay": the
 * optimizer composes with torch LR schedulers and decoupled weight decay).
 * Host-side only: steps already queued keep the values they were launched
 * with; a step captured in a HIP graph keeps the values of its capture.
 * Errors: invalid config, or n_feat or n_time different from lopt_create's
 * -> INVALID_ARGUMENT (the handle keeps its previous config). */
lopt_status lopt_set_config(lopt_handle* h, const lopt_config* cfg);

/* The MLP path that the handle's steps run: the config's mlp_impl, with
 * LOPT_MLP_AUTO resolved (LOPT_MLP_BF16X8).  Host-side only.  Errors: NULL argument ->
 * INVALID_ARGUMENT. */
lopt_status lopt_get_mlp_impl(const lopt_handle* h, int32_t* impl);

/* How the handle's steps over the bound list are launched: the config's
 * launch mode, with LOPT_LAUNCH_AUTO resolved for the bound list's size
 * (LOPT_LAUNCH_SINGLE or LOPT_LAUNCH_SPLIT; before a binding, as for an empty
 * list).  Host-side only.  Errors: NULL argument -> INVALID_ARGUMENT. */
lopt_status lopt_get_launch(const lopt_handle* h, int32_t* launch);

/* Per-tensor learning rate and weight decay, as torch's parameter groups give
 * them (the PyLO page, "Library design": the optimizer is a torch optimizer;
 * decoupled weight decay as in lopt_config).  lr[i] and weight_decay[i]
 * replace the config's lr and weight_decay for tensor i of the bound list in
 * the following lopt_step calls; tensor i then gets
 *   p <- p - lr[i] u - lr[i] weight_decay[i] p.
 * Both NULL: back to the config's values for every tensor.  n: the bound
 * list's length.  The arrays are copied on the host; the next lopt_step queues
 * the device copy on its stream through the handle's pinned buffer (no wait),
 * so such a step cannot be captured into a graph (INVALID_ARGUMENT while its
 * stream is capturing).  lopt_init_state forgets the values.  Errors: no bound
 * list or n different from its length -> STATE; exactly one NULL array or a
 * non-finite value -> INVALID_ARGUMENT (nothing changes). */
lopt_status lopt_set_tensor_hyper(lopt_handle* h, const float* lr, const float* weight_decay, int32_t n);

/* Floats per tensor in lopt_get_tensor_stats' output. */
#define LOPT_STAT_FLOATS 32

/* The per-tensor statistics of the step: what the PyLO page's kernel 1
 * collects ("CUDA kernel design: two-pass fusion" > "Fused kernel strategy":
 * one statistic of the squares of each feature over the whole tensor), as the
 * normalisers the apply pass used.  For tensor i of the bound list (n: its
 * length) and d < n_feat:
 *   out[i * LOPT_STAT_FLOATS + d] = s_d = (mean over the tensor of F_d^2 + eps_norm)^(-1/2),
 * 0 for n_feat <= d < 28, then
 *   out[i * LOPT_STAT_FLOATS + 28 + k] = sqrt(mean_i r_k) (k = 0, 1, 2; r_k
 *   after the step's update), and entry 31 = 0.
 * The values are those of the last step that gave tensor i a gradient
 * (unspecified before it has had one).  out: host memory, n *
 * LOPT_STAT_FLOATS floats.  Waits for the device (hipDeviceSynchronize).
 * Errors: NULL handle or out -> INVALID_ARGUMENT; no bound list or n
 * different from its length -> STATE; copy failure -> HIP. */
lopt_status lopt_get_tensor_stats(const lopt_handle* h, float* out, int32_t n);

/* Kernels of one step, in launch order. */
#define LOPT_N_KERNELS 5 /* row/col sums, moving averages, statistics, finalize, apply */

/* Measurement hook (the PyLO page reports step times, "Benchmark results" >
 * "Step-time reduction"; this lets a caller time each kernel of the step on
 * the step's own stream).  events: n caller-owned hipEvent_t handles; with
 * n == LOPT_N_KERNELS + 1 every following lopt_step records events[k] on its
 * stream just before kernel k and events[LOPT_N_KERNELS] after the last one
 * (a one-launch step records events[0..LOPT_N_KERNELS-1] before its kernel
 * and events[LOPT_N_KERNELS] after it, so the whole step counts as the apply
 * kernel's time; a row-shard step records events[0] in phase 0, events[1],
 * [2], [3] in phase 1 before the moving averages, the statistics pass and the
 * second export, events[4], [5] around the apply pass in phase 2, so the
 * exchanges count with the row/column sums and the finalize); n == 0
 * switches recording off.  The array is copied; the events must stay
 * valid while steps that record them are queued.  Errors: NULL handle, NULL
 * events with n > 0, other n -> INVALID_ARGUMENT. */
lopt_status lopt_set_timing_events(lopt_handle* h, void* const* events, int32_t n);

/* Message of the last failing call on this thread ("" if none). */
const char* lopt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LOPT_H */
