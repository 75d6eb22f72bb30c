// Device helpers shared by the gfx950 kernels of the optimizer step
// (feature construction, reductions, index arithmetic).
#pragma once

#include <hip/hip_runtime.h>

#include "lopt_internal.h"

namespace lopt {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Sum over the 256 threads of the block; every thread gets the result.
// `red` must hold 4 floats; the call contains two barriers.
__device__ __forceinline__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// k for the features that carry rho_k (g rho_k, m_a rho_k), else -1.
__host__ __device__ constexpr int rho_feature(int f) {
  return (f >= 10 && f < 13) ? f - 10 : (f >= 19 && f < 28) ? (f - 19) % 3 : -1;
}

__device__ __forceinline__ uint32_t div_c(uint32_t e, uint32_t magic, uint32_t shift) {
  return (__umulhi(e, magic) + e) >> shift;
}

// Global-address-space views of device pointers read from descriptors (the
// compiler then emits global_* instead of flat_* memory instructions).
typedef __attribute__((address_space(1))) float gfloat;
__device__ __forceinline__ const gfloat* gptr(const float* p) { return (const gfloat*)p; }
__device__ __forceinline__ gfloat* gptr(float* p) { return (gfloat*)p; }

// Per-element inputs of the feature construction.
struct Elem {
  float g, p, m[3], v;
  float rq[3];   // r_k[i]^(-1/2)
  float cq[3];   // 2-D: c_k[j]^(-1/2) (already updated); 1-D: old c_k[j] on input
};

// Updated accumulators and the 28 features of one element, with the
// per-tensor factor sqrt(rbar_k) left out of rho_k:
//   2-D:  rho'_k = r_k[i]^(-1/2) c_k[j]^(-1/2)  (rho_k = sqrt(rbar_k) rho'_k; the
//         factored form also avoids the fp32 underflow of r_k c_k)
//   1-D (rows = 1): c_k is per element and rbar_k = r_k, so rho_k = c_k^(-1/2).
// Features 10..12 and 19..27 are linear in rho_k, so the finalize kernel moves
// sqrt(rbar_k) into their normalisation scales (rho_feature below).
template <bool VEC>
__device__ __forceinline__ void build_features(const StepParams& hp, Elem& x, float F[kNF], float cn[3]) {
  const float g = x.g;
  const float g2 = g * g;
#pragma unroll
  for (int a = 0; a < 3; ++a) x.m[a] = fmaf(hp.beta_m[a], x.m[a], (1.0f - hp.beta_m[a]) * g);
  x.v = fmaf(hp.beta_v, x.v, (1.0f - hp.beta_v) * g2);
  float cq[3], rho[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    if (VEC) {
      cn[k] = fmaf(hp.beta_f[k], x.cq[k], (1.0f - hp.beta_f[k]) * (g2 + hp.eps_f));
      cq[k] = rsqrtf(cn[k]);
      rho[k] = cq[k];
    } else {
      cq[k] = x.cq[k];
      rho[k] = x.rq[k] * cq[k];
    }
  }
  const float q = rsqrtf(x.v + hp.eps_v);
  F[0] = g;
  F[1] = x.p;
  F[2] = x.m[0]; F[3] = x.m[1]; F[4] = x.m[2];
  F[5] = x.v;
  F[6] = x.m[0] * q; F[7] = x.m[1] * q; F[8] = x.m[2] * q;
  F[9] = q;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    F[10 + k] = g * rho[k];
    F[13 + k] = x.rq[k];
    F[16 + k] = cq[k];
  }
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int k = 0; k < 3; ++k) F[19 + 3 * a + k] = x.m[a] * rho[k];
}

// Loads the inputs of element e of tensor d.
template <bool VEC>
__device__ __forceinline__ void load_elem(const TensorDesc& d, const float* __restrict__ g_,
                                          const float* __restrict__ ws_, uint32_t e, Elem& x) {
  const size_t n = d.n;
  const gfloat* st = gptr(d.st);
  const gfloat* g = gptr(g_);
  const gfloat* ws = gptr(ws_);
  x.g = g[e];
  x.p = gptr(d.p)[e];
  x.m[0] = st[e];
  x.m[1] = st[n + e];
  x.m[2] = st[2 * n + e];
  x.v = st[3 * n + e];
  if (VEC) {
    const gfloat* c = st + 4 * n + 3;  // R = 1
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      x.cq[k] = c[k * n + e];
      x.rq[k] = ws[d.off_rq + k];
    }
  } else {
    const uint32_t i = div_c(e, d.cmagic, d.cshift);
    const uint32_t j = e - i * uint32_t(d.C);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      x.rq[k] = ws[d.off_rq + size_t(k) * d.R + i];
      x.cq[k] = ws[d.off_cq + size_t(k) * d.C + j];
    }
  }
}

// sqrt(mean_i r_k[i]) from the per-segment partial sums of r_k, summed by the
// whole block in a fixed order (every caller gets bitwise the same value).
// All threads must call it (it contains barriers); 1-D tensors get 1.
__device__ __forceinline__ void block_sr(const StepCtx& c, const TensorDesc& d, float sr[3], float* red) {
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    float s = 0.f;
    for (int q = threadIdx.x; q < d.nrseg; q += kBlock) s += c.rbar_part[(d.rseg0 + q) * 4 + k];
    s = block_sum(s, red);
    sr[k] = d.vec ? 1.0f : sqrtf(s / float(d.R));
  }
}


}  // namespace lopt
