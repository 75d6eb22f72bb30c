// gfx950 kernels of the small_fc_lopt optimizer step.
//
// The PyLO page ("CUDA kernel design: two-pass fusion" > "Fused kernel
// strategy") splits the step into a statistics pass (features built in
// registers, per-feature sums of squares reduced across the tensor) and an
// apply pass (features rebuilt, normalised, MLP evaluated inline, parameter
// written).  This file keeps that two-pass core and adds what the factored
// row/column accumulators need, as five launches per step over all tensors:
//
//   k_rowcol_sumsq  row and column sums of g^2 per tile (HBM: reads g)
//   k_moving_avg    row/column moving averages, r_k^(-1/2), c_k^(-1/2)
//   k_stats         per-chunk sums of the 28 squared features (reads p, g, m, v)
//   k_finalize      per-tensor feature scales; packs the MLP with the step
//                   features folded into the first bias
//   k_apply_*       features -> MLP -> update; writes p, m, v (and c for 1-D)
//                   (lopt_apply.hip)
//
// Every reduction uses a fixed order (butterfly within a wave, then LDS in
// wave order, then per-chunk partials summed in chunk order), so a step is
// bitwise reproducible run to run.
#include <hip/hip_runtime.h>

#include <mutex>

#include "lopt_passes.h"

namespace lopt {


// ---------------------------------------------------------------------------
// The four streaming passes, one kernel each (bodies in lopt_passes.h).
__global__ __launch_bounds__(kBlock) void k_rowcol_sumsq(StepCtx c) { rowcol_block(c, blockIdx.x); }

__global__ __launch_bounds__(kBlock) void k_moving_avg(StepCtx c, StepParams hp) { moving_avg_block(c, hp, blockIdx.x); }

// Six waves per SIMD (80 VGPRs, a few spilled): 0.370 against 0.372 ms at
// five on ViT-B/16.
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(6))) void k_stats(StepCtx c, StepParams hp) {
  stats_block(c, hp, blockIdx.x);
}

__global__ __launch_bounds__(kBlock) void k_finalize(StepCtx c, StepParams hp) { finalize_block(c, hp, blockIdx.x); }

__global__ __launch_bounds__(kBlock) void k_shard_colsum(StepCtx c) { shard_colsum_block(c, blockIdx.x); }

__global__ __launch_bounds__(kBlock) void k_shard_reduce(StepCtx c) { shard_reduce_block(c, blockIdx.x); }

// ---------------------------------------------------------------------------
// k_zero_state: zero-fills the state over the chunk list (per-element blocks
// of each chunk; the first chunk of a tensor also clears r_k and c_k).
__global__ __launch_bounds__(kBlock) void k_zero_state(StepCtx c) {
  const Chunk ch = c.chunks[blockIdx.x];
  const TensorDesc d = c.desc[ch.tensor];
  const size_t n = d.n;
  float* st = d.st;
  for (uint32_t e = ch.e0 + threadIdx.x; e < ch.e1; e += kBlock) {
    st[e] = 0.f; st[n + e] = 0.f; st[2 * n + e] = 0.f; st[3 * n + e] = 0.f;
    if (d.vec) {
      float* cs = st + 4 * n + 3;
      cs[e] = 0.f; cs[n + e] = 0.f; cs[2 * n + e] = 0.f;
    }
  }
  if (ch.e0 == 0) {
    const size_t rc = d.vec ? 3 : 3 * (size_t(d.R) + size_t(d.C));
    for (size_t q = threadIdx.x; q < rc; q += kBlock) st[4 * n + q] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// The workspace of lopt_init_state_static: a file-scope device array that each
// GPU the library runs on holds until the process ends.  In host code its name
// is only a host-side stand-in, so its device address is taken once per device
// with hipGetSymbolAddress (with that device current) and used from then on:
// kernel arguments and copies receive that address, never the name.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_address(int device, void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *out = addr[device];
  return hipSuccess;
}

hipError_t launch_zero_state(const StepCtx& c, hipStream_t s) {
  if (c.n_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_state, dim3(c.n_chunks), dim3(kBlock), 0, s, c);
  return hipGetLastError();
}

hipError_t launch_step(const StepCtx& c, const StepParams& p, hipStream_t s, const hipEvent_t* ev) {
  if (c.n_tensors == 0) return hipSuccess;
  auto mark = [&](int k) -> hipError_t { return ev ? hipEventRecord(ev[k], s) : hipSuccess; };
  hipError_t e;
  if ((e = mark(0)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_rowcol_sumsq, dim3(c.n_tiles0), dim3(kBlock), 0, s, c);
  if ((e = mark(1)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_moving_avg, dim3(c.n_segs1), dim3(kBlock), 0, s, c, p);
  if ((e = mark(2)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_stats, dim3(c.n_chunks), dim3(kBlock), 0, s, c, p);
  if ((e = mark(3)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_finalize, dim3(c.n_tensors + 1), dim3(kBlock), 0, s, c, p);
  if ((e = mark(4)) != hipSuccess) return e;
  if ((e = launch_apply(c, p, s)) != hipSuccess) return e;
  if ((e = mark(5)) != hipSuccess) return e;
  return hipGetLastError();
}

hipError_t launch_shard_phase(const StepCtx& c, const StepParams& p, int phase, hipStream_t s, const hipEvent_t* ev) {
  if (c.n_tensors == 0) return hipSuccess;
  auto mark = [&](int k) -> hipError_t { return ev ? hipEventRecord(ev[k], s) : hipSuccess; };
  hipError_t e;
  if (phase == 0) {
    if ((e = mark(0)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_rowcol_sumsq, dim3(c.n_tiles0), dim3(kBlock), 0, s, c);
    hipLaunchKernelGGL(k_shard_colsum, dim3(c.n_segs1), dim3(kBlock), 0, s, c);
  } else if (phase == 1) {
    if ((e = mark(1)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_moving_avg, dim3(c.n_segs1), dim3(kBlock), 0, s, c, p);
    if ((e = mark(2)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_stats, dim3(c.n_chunks), dim3(kBlock), 0, s, c, p);
    if ((e = mark(3)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_shard_reduce, dim3(c.n_tensors), dim3(kBlock), 0, s, c);
  } else {
    hipLaunchKernelGGL(k_finalize, dim3(c.n_tensors + 1), dim3(kBlock), 0, s, c, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(4)) != hipSuccess) return e;
    if ((e = launch_apply(c, p, s)) != hipSuccess) return e;
    if ((e = mark(5)) != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace lopt
