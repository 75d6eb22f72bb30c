// The optimizer step in one launch (LOPT_LAUNCH_SINGLE).
//
// The PyLO page counts launches as the cost that fusion removes ("Naive
// implementation bottleneck": 74-252 launches per step; "Use of the memory
// hierarchy": 30-114 after fusing into two passes).  The five-kernel step
// needs five; for a small tensor list each costs more than its work, so this
// kernel runs the five passes in turn inside one grid: every block takes the
// work items of a pass in a block-stride loop (the same per-item bodies as the
// five kernels, hence the same results bit for bit), and a grid-wide barrier
// separates the passes.
//
// The barrier needs every block of the grid resident at once: the host sizes
// the grid to at most (compute units) x (blocks per compute unit that the
// kernel's registers and LDS allow).  Each wait is bounded: a block that waits
// longer than ~2 s (which only a grid that could not become resident, e.g. on
// a device shared with a persistent kernel, can cause) raises the fault word
// and goes on, so every wave still reaches the end of the kernel;
// lopt_get_step reports the fault.
//
// Barrier words (workspace sync record, zero at binding): [0] launch count
// (epoch), [1] release word, [2] fault, [16 + b] arrival word of block b.
// Barrier k (0..3) of the launch with epoch e has the id 4e + k + 1 (mod
// 2^32), unique among the values those words held before.  A block arrives by
// storing the id into its own word; block 0 waits until every arrival word
// holds it, then stores it into the release word, which every block waits
// for.  No two blocks write one word, so the barrier needs no
// read-modify-write on a shared address (those are serialised across the
// eight XCDs).  After the last barrier block 0 advances the epoch; every
// block has read it before its first arrival.
//
// Compiled with -fno-honor-nans, like the apply kernels (lopt_apply_body.h).
#include <hip/hip_runtime.h>

#include <mutex>

#include "lopt_apply_body.h"
#include "lopt_passes.h"

namespace lopt {

constexpr uint32_t kSpinLimit = 1u << 21;  // polls of ~1 us each

// Polls *word until it holds id (relaxed loads at device scope, which read
// past the XCD's L2); on running out of polls raises the fault word and
// returns.
__device__ __forceinline__ void wait_for(const uint32_t* word, uint32_t id, uint32_t* fault) {
  uint32_t polls = 0;
  while (__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != id) {
    __builtin_amdgcn_s_sleep(2);
    if (++polls == kSpinLimit) {
      __hip_atomic_store(fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }
}

// Grid-wide barrier `id`.  The stores of a pass live in the L2 of the XCD
// that made them (the eight XCDs' L2 caches are not coherent for ordinary
// stores), so before a block arrives each of its waves waits until its stores
// have reached the L2, and then one thread writes that L2 back (a device-scope
// release fence) and stores the arrival word; after the release word is seen
// one thread invalidates the block's caches (a device-scope acquire fence).
// One writeback and one invalidation per block and barrier: a fence in every
// wave (four per block) made each barrier cost tens of microseconds.
__device__ __forceinline__ void grid_sync(uint32_t* sync, uint32_t id, uint32_t blocks) {
  uint32_t* release = sync + 1;
  uint32_t* fault = sync + kSyncFault;
  uint32_t* arrive = sync + kSyncArrive;
  __builtin_amdgcn_s_waitcnt(0);   // every counter of this wave at zero: its stores are in the L2
  __syncthreads();
  if (blockIdx.x == 0) {
    for (uint32_t b = 1 + threadIdx.x; b < blocks; b += kBlock) wait_for(arrive + b, id, fault);
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_store(release, id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
  } else if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(arrive + blockIdx.x, id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_for(release, id, fault);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

template <int IMPL>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_step_single(StepCtx c, StepParams hp) {
  const uint32_t G = gridDim.x;
  uint32_t* sync = c.sync;
  const uint32_t epoch = uni(__hip_atomic_load(sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const uint32_t id0 = 4u * epoch + 1u;

  for (uint32_t b = blockIdx.x; b < uint32_t(c.n_tiles0); b += G) {
    rowcol_block(c, b);
    __syncthreads();  // LDS reuse by the next item
  }
  grid_sync(sync, id0, G);
  for (uint32_t b = blockIdx.x; b < uint32_t(c.n_segs1); b += G) {
    moving_avg_block(c, hp, b);
    __syncthreads();
  }
  grid_sync(sync, id0 + 1u, G);
  for (uint32_t b = blockIdx.x; b < uint32_t(c.n_chunks); b += G) {
    stats_block(c, hp, b);
    __syncthreads();
  }
  grid_sync(sync, id0 + 2u, G);
  for (uint32_t b = blockIdx.x; b < uint32_t(c.n_tensors) + 1; b += G) {
    finalize_block(c, hp, b);
    __syncthreads();
  }
  grid_sync(sync, id0 + 3u, G);
  if (blockIdx.x == 0 && threadIdx.x == 0) __hip_atomic_store(sync, epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (uint32_t b = blockIdx.x; b < uint32_t(c.n_chunks); b += G) {
    apply_block<IMPL, false>(c, hp, b);
    __syncthreads();
  }
}

namespace {

typedef void (*SingleKernel)(StepCtx, StepParams);

SingleKernel single_kernel(int impl) {
  switch (impl) {
    case 1: return k_step_single<1>;
    case 2: return k_step_single<2>;
    case 3: return k_step_single<3>;
    case 4: return k_step_single<4>;
    case 5: return k_step_single<5>;
    default: return k_step_single<6>;
  }
}

}  // namespace

hipError_t single_grid_cap(int device, int impl, int* blocks) {
  static std::mutex mu;
  static int cap[kMaxDevices][8] = {};
  if (device < 0 || device >= kMaxDevices || impl < 1 || impl > 6) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lock(mu);
  if (!cap[device][impl]) {
    int cus = 0, occ = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(single_kernel(impl)),
                                                     kBlock, 0);
    if (e != hipSuccess) return e;
    if (cus < 1 || occ < 1) return hipErrorInvalidConfiguration;
    cap[device][impl] = cus * occ;
  }
  *blocks = cap[device][impl];
  return hipSuccess;
}

hipError_t launch_single(const StepCtx& c, const StepParams& p, int blocks, hipStream_t s, const hipEvent_t* ev) {
  if (c.n_tensors == 0) return hipSuccess;
  hipError_t e;
  if (ev)
    for (int k = 0; k < kNumKernels; ++k)
      if ((e = hipEventRecord(ev[k], s)) != hipSuccess) return e;
  hipLaunchKernelGGL(single_kernel(c.mlp_impl), dim3(blocks), dim3(kBlock), 0, s, c, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev && (e = hipEventRecord(ev[kNumKernels], s)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace lopt
