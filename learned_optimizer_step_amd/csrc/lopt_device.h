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

__device__ __forceinline__ uint32_t div_c(uint32_t e, uint32_t magic, uint32_t shift) {
  return (__umulhi(e, magic) + e) >> shift;
}

// Global-address-space views of device pointers read from descriptors (the
// compiler then emits global_* instead of flat_* memory instructions).
typedef __attribute__((address_space(1))) float gfloat;
__device__ __forceinline__ const gfloat* gptr(const float* p) { return (const gfloat*)p; }
__device__ __forceinline__ gfloat* gptr(float* p) { return (gfloat*)p; }

// Wave-uniform copies (scalar registers) of values loaded from the work lists.
// The compiler reads the lists with vector loads (it cannot prove that the
// kernel's own stores leave them untouched); readfirstlane keeps the result
// in scalar registers instead of per-lane copies.
__device__ __forceinline__ uint32_t uni(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int32_t uni(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }
template <class T>
__device__ __forceinline__ T* uni(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<T*>((uint64_t(hi) << 32) | lo);
}
__device__ __forceinline__ int64_t uni(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

// The chunk record, its tensor's descriptor and gradient pointer, as
// wave-uniform values.
__device__ __forceinline__ void load_chunk(const StepCtx& c, uint32_t idx, Chunk& ch, TensorDesc& d,
                                           const float*& g) {
  const Chunk cr = c.chunks[idx];
  ch.tensor = uni(cr.tensor);
  ch.e0 = uni(cr.e0);
  ch.e1 = uni(cr.e1);
  ch.row0 = uni(cr.row0);
  const TensorDesc dr = c.desc[ch.tensor];
  d.p = uni(dr.p);
  d.st = uni(dr.st);
  d.R = uni(dr.R);
  d.C = uni(dr.C);
  d.n = uni(dr.n);
  d.cmagic = uni(dr.cmagic);
  d.cshift = uni(dr.cshift);
  d.vec = uni(dr.vec);
  d.ncw = uni(dr.ncw);
  d.nrb = uni(dr.nrb);
  d.rseg0 = uni(dr.rseg0);
  d.nrseg = uni(dr.nrseg);
  d.chunk0 = uni(dr.chunk0);
  d.nchunk = uni(dr.nchunk);
  d.off_rowpart = uni(dr.off_rowpart);
  d.off_colpart = uni(dr.off_colpart);
  d.off_rq = uni(dr.off_rq);
  d.off_cq = uni(dr.off_cq);
  g = uni(c.grads[ch.tensor]);
}

// Uniform base pointers of one chunk's per-element streams and of its
// row/column vectors.  Every stream is rebased at the chunk's first element
// (and the row vectors at its first row), so a lane's access is a uniform
// 64-bit base plus a small 32-bit byte offset (global_load v, voff, s[base]).
struct Streams {
  const gfloat* g;
  gfloat* p;
  gfloat* m[3];
  gfloat* v;
  gfloat* c[3];          // 1-D tensors: per-element c_k
  const gfloat* rq;      // [row][4] r_k^(-1/2) from the chunk's first row (1-D: one record)
  const gfloat* cq;      // [col][4] c_k^(-1/2) (2-D)
  uint32_t e0, i0, C, cmagic, cshift;
};

__device__ __forceinline__ Streams make_streams(const TensorDesc& d, const float* g, const float* ws,
                                                const Chunk& ch) {
  Streams s;
  const size_t n = d.n;
  const uint32_t e0 = ch.e0;
  gfloat* st = (gfloat*)d.st;
  s.e0 = e0;
  s.i0 = ch.row0;
  s.g = gptr(g) + e0;
  s.p = gptr(d.p) + e0;
#pragma unroll
  for (int a = 0; a < 3; ++a) s.m[a] = st + a * n + e0;
  s.v = st + 3 * n + e0;
#pragma unroll
  for (int k = 0; k < 3; ++k) s.c[k] = st + 4 * n + 3 + k * n + e0;   // 1-D tensors only (R = 1)
  s.rq = gptr(ws) + d.off_rq + 4 * size_t(d.vec ? 0 : s.i0);
  s.cq = gptr(ws) + d.off_cq;
  s.C = uint32_t(d.C);
  s.cmagic = d.cmagic;
  s.cshift = d.cshift;
  return s;
}

// base[byte_off / 4] with a 32-bit byte offset.
typedef __attribute__((address_space(1))) char gchar;
__device__ __forceinline__ float ldb(const gfloat* base, uint32_t byte_off) {
  return *(const gfloat*)((const gchar*)base + byte_off);
}
// Streaming load: each per-element value is read once per kernel, so it is
// fetched with the non-temporal hint (measured: +10 % read bandwidth).
__device__ __forceinline__ float ldb_stream(const gfloat* base, uint32_t byte_off) {
  return __builtin_nontemporal_load((const gfloat*)((const gchar*)base + byte_off));
}
__device__ __forceinline__ void stb(gfloat* base, uint32_t byte_off, float v) {
  *(gfloat*)((gchar*)base + byte_off) = v;
}
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) f32x4 gf32x4;
__device__ __forceinline__ f32x4 ldb4(const gfloat* base, uint32_t byte_off) {
  return *(const gf32x4*)((const gchar*)base + byte_off);
}

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
// 1/sqrt(x).  NORMAL: x is known to be >= FLT_MIN, 0, inf or NaN, where the
// hardware instruction alone is exact to its spec; rsqrtf adds a rescaling of
// subnormal arguments (five more vector instructions per call).
template <bool NORMAL>
__device__ __forceinline__ float rsq(float x) {
  return NORMAL ? __builtin_amdgcn_rsqf(x) : rsqrtf(x);
}

// Compile-time variant of a chunk's per-element code: tensor kind (1-D or
// factored 2-D), 1/sqrt mode, number of per-element features (kNF for
// small_fc_lopt, kVeloNF for the VeLO-shaped variant, which stops at F18), and
// whether the row features are constant over every 64-element wave iteration:
// 1-D tensors (one r_k per tensor) and 2-D tensors whose column count is a
// multiple of 64 (the chunks start at multiples of 256 elements, so a wave
// iteration lies inside one row).
template <bool V, bool N, int F, bool RU = false>
struct Variant {
  static constexpr bool vec = V;
  static constexpr bool normal = N;
  static constexpr int nf = F;
  static constexpr bool rowuni = RU;
};

__device__ __forceinline__ bool rows_uniform(const TensorDesc& d) { return !d.vec && (d.C & 63) == 0; }

// Calls body(Variant<...>{}) for the chunk's tensor kind and the step's 1/sqrt
// mode and feature count (all uniform over the workgroup).  ROWS: also mark
// the row-uniform kinds (only the matrix-core apply kernel uses it).
template <bool ROWS, class Body>
__device__ __forceinline__ void dispatch_variant(const TensorDesc& d, const StepParams& hp, Body&& body) {
  auto by_nf = [&](auto kind) {
    using K = decltype(kind);
    if (hp.n_feat == kNF) {
      if (hp.rsq_normal) body(Variant<K::vec, true, kNF, K::rowuni>{});
      else body(Variant<K::vec, false, kNF, K::rowuni>{});
    } else {
      if (hp.rsq_normal) body(Variant<K::vec, true, kVeloNF, K::rowuni>{});
      else body(Variant<K::vec, false, kVeloNF, K::rowuni>{});
    }
  };
  if (d.vec) by_nf(Variant<true, true, kNF, ROWS>{});
  else if (ROWS && rows_uniform(d)) by_nf(Variant<false, true, kNF, true>{});
  else by_nf(Variant<false, true, kNF, false>{});
}

// Builds F[0..NF) (NF = kNF or kVeloNF; F[NF..kNF) are left unset).
template <bool VEC, bool NORMAL, int NF>
__device__ __forceinline__ void build_features(const StepParams& hp, Elem& x, float F[kNF], float cn[3]) {
  const float g = x.g;
  const float g2 = g * g;
#pragma unroll
  for (int a = 0; a < 3; ++a) x.m[a] = fmaf(hp.beta_m[a], x.m[a], hp.omb_m[a] * g);
  x.v = fmaf(hp.beta_v, x.v, hp.omb_v * g2);
  float cq[3], rho[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    if (VEC) {
      cn[k] = fmaf(hp.beta_f[k], x.cq[k], hp.omb_f[k] * (g2 + hp.eps_f));
      cq[k] = rsq<NORMAL>(cn[k]);
      rho[k] = cq[k];
    } else {
      cq[k] = x.cq[k];
      rho[k] = x.rq[k] * cq[k];
    }
  }
  const float q = rsq<NORMAL>(x.v + hp.eps_v);
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
  if (NF == kNF) {
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
      for (int k = 0; k < 3; ++k) F[19 + 3 * a + k] = x.m[a] * rho[k];
  }
}

// Loads the inputs of element e of tensor d.
// Loads the inputs of element e of the chunk.  All byte offsets fit in 32
// bits: a chunk spans at most kChunkElems elements (and rows), and the host
// rejects 2-D tensors with 2^28 or more columns (16-byte column records).
// ROW (2-D only): the caller guarantees that e lies in the same row as the
// wave-uniform element `row_elem`; the row index is then divided once for the
// wave (scalar unit) and the row record read with one uniform load.
template <bool VEC, bool ROW = false>
__device__ __forceinline__ void load_elem(const Streams& s, uint32_t e, Elem& x, uint32_t row_elem = 0) {
  const uint32_t off = (e - s.e0) * 4u;
  x.g = ldb_stream(s.g, off);
  x.p = ldb_stream(s.p, off);
#pragma unroll
  for (int a = 0; a < 3; ++a) x.m[a] = ldb_stream(s.m[a], off);
  x.v = ldb_stream(s.v, off);
  if (VEC) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      x.cq[k] = ldb_stream(s.c[k], off);
      x.rq[k] = s.rq[k];
    }
  } else {
    const uint32_t i = ROW ? div_c(row_elem, s.cmagic, s.cshift) : div_c(e, s.cmagic, s.cshift);
    const uint32_t j = e - i * s.C;
    const f32x4 r4 = ldb4(s.rq, (i - s.i0) * 16u);
    const f32x4 c4 = ldb4(s.cq, j * 16u);
    x.rq[0] = r4.x; x.rq[1] = r4.y; x.rq[2] = r4.z;
    x.cq[0] = c4.x; x.cq[1] = c4.y; x.cq[2] = c4.z;
  }
}

// Stores the updated per-element accumulators of element e (m, v; 1-D: c).
template <bool VEC>
__device__ __forceinline__ void store_state(const Streams& s, uint32_t e, const Elem& x, const float cn[3]) {
  const uint32_t off = (e - s.e0) * 4u;
#pragma unroll
  for (int a = 0; a < 3; ++a) stb(s.m[a], off, x.m[a]);
  stb(s.v, off, x.v);
  if (VEC) {
#pragma unroll
    for (int k = 0; k < 3; ++k) stb(s.c[k], off, cn[k]);
  }
}

// The update constants of the chunk's tensor: (decay, lr_step) = (1 - lr wd,
// lr step_mult) from the step, or the tensor's own pair (wave-uniform).
__device__ __forceinline__ void update_constants(const StepCtx& c, const StepParams& hp, const Chunk& ch,
                                                 float& decay, float& lr_step) {
  decay = hp.decay;
  lr_step = hp.lr_step;
  if (hp.per_tensor) {
    decay = __int_as_float(uni(__float_as_int(c.tensor_hyper[2 * ch.tensor])));
    lr_step = __int_as_float(uni(__float_as_int(c.tensor_hyper[2 * ch.tensor + 1])));
  }
}

// Stores the updated parameter of element e.
__device__ __forceinline__ void store_param(const Streams& s, uint32_t e, float p_new) {
  stb(s.p, (e - s.e0) * 4u, p_new);
}

}  // namespace lopt
