// Apply kernels of the optimizer step, one per MLP path (the PyLO page's
// kernel 2; bodies in lopt_apply_body.h).  Compiled with -fno-honor-nans.
#include <hip/hip_runtime.h>

#include "lopt_apply_body.h"

namespace lopt {

__global__ __launch_bounds__(kBlock) void k_apply_valu(StepCtx c, StepParams hp) { apply_block<1>(c, hp, blockIdx.x); }

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_apply_mfma(StepCtx c, StepParams hp) {
  apply_block<2>(c, hp, blockIdx.x);
}

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_apply_bf16x6(StepCtx c, StepParams hp) {
  apply_block<3>(c, hp, blockIdx.x);
}

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_apply_fp16x3(StepCtx c, StepParams hp) {
  apply_block<4>(c, hp, blockIdx.x);
}

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_apply_bf16x9(StepCtx c, StepParams hp) {
  apply_block<5>(c, hp, blockIdx.x);
}

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_apply_bf16x8(StepCtx c, StepParams hp) {
  apply_block<6>(c, hp, blockIdx.x);
}

hipError_t launch_apply(const StepCtx& c, const StepParams& p, hipStream_t s) {
  if (c.mlp_impl == 1)
    hipLaunchKernelGGL(k_apply_valu, dim3(c.n_chunks), dim3(kBlock), 0, s, c, p);
  else if (c.mlp_impl == 3)
    hipLaunchKernelGGL(k_apply_bf16x6, dim3(c.n_chunks), dim3(kBlock), 0, s, c, p);
  else if (c.mlp_impl == 4)
    hipLaunchKernelGGL(k_apply_fp16x3, dim3(c.n_chunks), dim3(kBlock), 0, s, c, p);
  else if (c.mlp_impl == 5)
    hipLaunchKernelGGL(k_apply_bf16x9, dim3(c.n_chunks), dim3(kBlock), 0, s, c, p);
  else if (c.mlp_impl == 6)
    hipLaunchKernelGGL(k_apply_bf16x8, dim3(c.n_chunks), dim3(kBlock), 0, s, c, p);
  else
    hipLaunchKernelGGL(k_apply_mfma, dim3(c.n_chunks), dim3(kBlock), 0, s, c, p);
  return hipGetLastError();
}

}  // namespace lopt
