// Internal definitions shared by the host planner (lopt_api.cpp) and the
// gfx950 kernels (lopt_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace lopt {

constexpr int kBlock = 256;        // threads per workgroup in every kernel (4 wave64s)
constexpr int kNF = 28;            // per-element features of small_fc_lopt
constexpr int kVeloNF = 19;        // the VeLO-shaped variant feeds features 0..18
constexpr int kH = 32;             // hidden width
constexpr int kMaxTime = 11;
constexpr int kStatStride = 32;    // floats per stats partial / per-tensor scale record

// Work sizes.
constexpr int kTile0Elems = 16384;   // elements per row/column-sum tile
constexpr int kTile0Iters = 64;      // row iterations per 2-D tile (bounds the LDS buffer)
constexpr int kSeg1 = 256;           // rows per moving-average row segment
constexpr int kSegCols1 = 64;        // columns per moving-average column segment ...
constexpr int kColGroups = 4;        // ... each summed by 4 thread groups (64 x 4 = 256 threads)
// Statistics / apply chunks: the plan picks one chunk size for the whole
// tensor list, aiming at kTargetChunks chunks (several rounds of the ~768
// workgroups the apply kernel keeps resident, so the last round is nearly
// full), between kMinChunkElems and kChunkElems elements, a multiple of 256.
constexpr int kChunkElems = 16384;
constexpr int kMinChunkElems = 256;
constexpr int kTargetChunks = 4096;

// Packed MLP in the workspace, written once per step by the finalize kernel:
// W1 feature columns [32][28] (columns >= n_feat zero), b1 with the step
// features folded in [32],
// W2 [32][32], b2 [32], W3 [2][32], b3 [2].
constexpr int kPkW1 = 0;
constexpr int kPkB1 = kPkW1 + kH * kNF;
constexpr int kPkW2 = kPkB1 + kH;
constexpr int kPkB2 = kPkW2 + kH * kH;
constexpr int kPkW3 = kPkB2 + kH;
constexpr int kPkB3 = kPkW3 + 2 * kH;
constexpr int kPkFloats = kPkB3 + 2;

// Per-tensor descriptor (device resident, in the workspace).
struct TensorDesc {
  float* p;
  float* st;                 // state: m1 m2 m3 v (n each) | r1 r2 r3 (R) | c1 c2 c3 (C)
  int32_t R, C;
  uint32_t n;
  uint32_t cmagic;           // e / C == (umulhi(e, cmagic) + e) >> cshift for e < 2^31
  uint32_t cshift;
  int32_t vec;               // R == 1: c_k per element, r_k a single value
  int32_t ncw;               // row partials per row (column windows; flat tiles for vec)
  int32_t nrb;               // column partials per column (row blocks)
  int32_t rseg0, nrseg;      // moving-average row segments (sum of r_k partials)
  int32_t chunk0, nchunk;    // statistics / apply chunks
  int64_t off_rowpart;       // floats: [ncw][R]
  int64_t off_colpart;       // floats: [nrb][C]       (2-D only)
  int64_t off_rq;            // floats: [R][4]  (r_1, r_2, r_3)^(-1/2), 4th unused
  int64_t off_cq;            // floats: [C][4]  (c_1, c_2, c_3)^(-1/2) (2-D only)
  // The whole tensor this one is a row shard of (lopt_init_state_sharded;
  // otherwise Rg = R, ng = n): the divisors of the column means, the mean of
  // r_k and the feature normalisers.
  int64_t Rg;                // rows (1 for a 1-D tensor)
  int64_t ng;                // elements
  int64_t off_sum1;          // first exported sum in StepCtx::sums1 (C of them, 1 for 1-D)
};

// Row/column sum-of-squares tile.
struct Tile0 {
  int32_t tensor;
  int32_t flat;              // 1: flat element range of a 1-D tensor
  int32_t r0, r1;            // 2-D rows [r0, r1)
  int32_t c0, c1;            // 2-D columns [c0, c1); flat: elements [c0, c1)
  int32_t cw_log2;           // 2-D: log2(threads per row slot)
  int32_t rb;                // 2-D: row-block index (column partial slot)
  int32_t win;               // row partial slot (column window, or flat tile index)
  int32_t pad[3];
};

// Moving-average segment.
enum : int32_t { kSegRows = 0, kSegCols = 1, kSegVec = 2 };
struct Seg1 {
  int32_t tensor;
  int32_t kind;
  int32_t a, b;              // rows or columns [a, b)
  int32_t slot;              // rows / vec: index of the r_k partial-sum record
  int32_t pad[3];
};

// Statistics / apply chunk: elements [e0, e1) of one tensor; row0 = e0 / cols.
struct Chunk {
  int32_t tensor;
  uint32_t e0, e1;
  uint32_t row0;
};

// Hyperparameters as the kernels see them.
struct StepParams {
  float beta_m[3];
  float beta_v;
  float beta_f[3];
  float omb_m[3], omb_v, omb_f[3];   // 1 - beta, rounded to fp32 once on the host
  float eps_v, eps_f, eps_norm;
  float exp_mult, step_mult, lr, weight_decay;
  // Update constants folded once on the host:
  //   p <- p * decay - lr_step * dir * exp2(mag * exp2_mult)
  float decay;               // 1 - lr * weight_decay
  float lr_step;             // lr * step_mult
  float exp2_mult;           // exp_mult * log2(e)
  // 1 when every argument of a per-element 1/sqrt is >= FLT_MIN, 0, inf or NaN
  // (eps_v and (1 - beta_f) eps_f are at least 2 FLT_MIN): the kernels then use
  // the bare hardware reciprocal square root, which only differs from rsqrtf
  // on subnormal arguments.
  int32_t rsq_normal;
  // 1: decay and lr_step come per tensor from StepCtx::tensor_hyper (the
  // caller's per-tensor learning rates and weight decays) instead of above
  int32_t per_tensor;
  int32_t n_feat;            // kNF or kVeloNF
  int32_t n_time;
  // fp16x3 path: W1 and W2 enter the A operands times 2^x3_w1 and 2^x3_w2;
  // the constant layer-1 entries carry (b1 + row term) / 2 times
  // 2^(x3_w1 - x3_shift) against a B value of 2^x3_shift, which keeps them
  // inside fp16's range for every input (the shift is bounded from the weights)
  int32_t x3_shift;
  int32_t x3_w1;
  int32_t x3_w2;
  float timescales[kMaxTime];
};

// Where everything lives: the workspace base and the per-step buffers.
struct StepCtx {
  float* ws;                         // workspace base (floats)
  const TensorDesc* desc;
  const float* const* grads;         // per-tensor gradient pointers
  const Tile0* tiles0;
  const Seg1* segs1;
  const Chunk* chunks;
  float* rbar_part;                  // [n_rows_segs][4]
  float* stats_part;                 // [n_chunks][32]
  float* scales;                     // [n_tensors][32]: s_0..s_27, sqrt(rbar_k) at 28..30
  float* packed;                     // kPkFloats
  int64_t* step;                     // steps taken; advanced by k_finalize (graph-replay safe)
  uint32_t* sync;                    // kSyncWords: the one-launch step's barrier words (lopt_single.hip)
  const float* tensor_hyper;         // [n_tensors][2]: decay, lr_step (StepParams::per_tensor)
  const float* mlp;                  // raw weights (handle-owned)
  int32_t n_tensors, n_tiles0, n_segs1, n_chunks;
  int32_t mlp_impl;                  // lopt_mlp_impl, AUTO resolved: 1 VALU, 2 MFMA, 3 BF16X6, 4 FP16X3, 5 BF16X9, 6 BF16X8
  // Row shards: 1 when the list's tensors are shards of larger ones whose sums
  // are exchanged across ranks between the step's phases (sums1: column sums
  // of g^2, sums2: [n_tensors][32] feature sums and sums of r_k).
  int32_t sharded;
  float* sums1;
  float* sums2;
};

hipError_t launch_zero_state(const StepCtx& c, hipStream_t s);

// lopt_init_state_static's workspace: a device array of kScratchBytes per GPU
// (LOPT_STATIC_SCRATCH_BYTES), 256-byte aligned.  scratch_address gives its
// device address on `device`, which must be the current device (the address
// is taken once per device and kept).
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
hipError_t scratch_address(int device, void** out);
constexpr int kNumKernels = 5;
// events: nullptr, or kNumKernels + 1 events recorded around the launches.
hipError_t launch_step(const StepCtx& c, const StepParams& p, hipStream_t s, const hipEvent_t* events);
hipError_t launch_apply(const StepCtx& c, const StepParams& p, hipStream_t s);
// The step of a row-shard binding in three phases, with the exchanges between
// them: row/column sums and the first export; moving averages, statistics
// pass and the second export; finalize and apply.  events as launch_step's:
// [0] before phase 0, [1] [2] [3] before the moving averages, the statistics
// pass and the second export, [4] [5] around the apply pass.
hipError_t launch_shard_phase(const StepCtx& c, const StepParams& p, int phase, hipStream_t s, const hipEvent_t* events);

// The one-launch step (lopt_single.hip).  Barrier words in the workspace,
// zero at binding: [0] launch count, [1] release word, [2] fault (a barrier
// wait ran out: the grid was not resident at once), [kSyncArrive + b] the
// arrival word of block b (at most kSingleMaxBlocks blocks).
constexpr int kSingleMaxBlocks = 2048;
constexpr int kSyncArrive = 16;
constexpr int kSyncWords = kSyncArrive + kSingleMaxBlocks;
constexpr int kSyncFault = 2;
// Blocks of the one-launch kernel for MLP path `impl` that `device` keeps
// resident at once (compute units x blocks per compute unit); cached.
hipError_t single_grid_cap(int device, int impl, int* blocks);
// events as launch_step's: the first kNumKernels are recorded before the
// launch, the last after it.
hipError_t launch_single(const StepCtx& c, const StepParams& p, int blocks, hipStream_t s, const hipEvent_t* events);

// k for the features that carry rho_k (g rho_k, m_a rho_k), else -1.
__host__ __device__ constexpr int rho_feature(int f) {
  return (f >= 10 && f < 13) ? f - 10 : (f >= 19 && f < 28) ? (f - 19) % 3 : -1;
}

// Fast division by a 32-bit divisor for numerators below 2^31
// (round-up multiplier method, Granlund & Montgomery 1994).
inline void fastdiv_magic(uint32_t d, uint32_t* magic, uint32_t* shift) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
  *magic = uint32_t(m);
  *shift = l;
}

}  // namespace lopt
