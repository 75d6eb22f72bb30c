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
//
// Every reduction uses a fixed order (butterfly within a wave, then LDS in
// wave order, then per-chunk partials summed in chunk order), so a step is
// bitwise reproducible run to run.
#include <hip/hip_runtime.h>

#include "lopt_internal.h"

namespace lopt {

namespace {

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

// Per-element inputs of the feature construction.
struct Elem {
  float g, p, m[3], v;
  float rq[3];   // r_k[i]^(-1/2)
  float cq[3];   // 2-D: c_k[j]^(-1/2) (already updated); 1-D: old c_k[j] on input
};

// Updated accumulators and the 28 raw features of one element.
// 2-D: rho_k = sqrt(rbar_k) r_k^(-1/2) c_k^(-1/2) (the factored form avoids the
// fp32 underflow of r_k c_k).  1-D (rows = 1): c_k is per element and rbar_k =
// r_k, so rho_k = c_k^(-1/2).
template <bool VEC>
__device__ __forceinline__ void build_features(const StepParams& hp, Elem& x, const float sr[3],
                                               float F[kNF], float cn[3]) {
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
      rho[k] = sr[k] * x.rq[k] * cq[k];
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
__device__ __forceinline__ void load_elem(const TensorDesc& d, const float* __restrict__ g,
                                          const float* __restrict__ ws, uint32_t e, Elem& x) {
  const size_t n = d.n;
  const float* st = d.st;
  x.g = g[e];
  x.p = d.p[e];
  x.m[0] = st[e];
  x.m[1] = st[n + e];
  x.m[2] = st[2 * n + e];
  x.v = st[3 * n + e];
  if (VEC) {
    const float* c = st + 4 * n + 3;  // R = 1
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

}  // namespace

// ---------------------------------------------------------------------------
// k_rowcol_sumsq: per-tile row sums and column sums of g^2.
//   2-D tile: rows [r0, r1) x a window of CW <= 256 columns.  Thread t handles
//   column c0 + (t mod CW) for rows r0 + (t / CW) + RS q, RS = 256 / CW.
//   Row sums: butterfly over the CW lanes of a row slot (CW <= 64), or over
//   the wave and then the CW/64 waves of the slot through LDS.
//   Column sums: per-thread over its rows, then over the RS row slots in LDS.
//   Flat tile (1-D tensors): one partial of sum g^2 over [c0, c1).
__global__ __launch_bounds__(kBlock) void k_rowcol_sumsq(StepCtx c) {
  const Tile0 tl = c.tiles0[blockIdx.x];
  const TensorDesc d = c.desc[tl.tensor];
  const float* __restrict__ g = c.grads[tl.tensor];
  float* __restrict__ ws = c.ws;
  const int tid = threadIdx.x;
  __shared__ float lds_rows[4 * kTile0Iters];
  __shared__ float lds_cols[kBlock];
  __shared__ float red[4];

  if (tl.flat) {
    float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
    uint32_t e = tl.c0 + tid;
    for (; e + 3 * kBlock < uint32_t(tl.c1); e += 4 * kBlock) {
      const float a = g[e], b = g[e + kBlock], cc = g[e + 2 * kBlock], dd = g[e + 3 * kBlock];
      acc0 = fmaf(a, a, acc0); acc1 = fmaf(b, b, acc1);
      acc2 = fmaf(cc, cc, acc2); acc3 = fmaf(dd, dd, acc3);
    }
    for (; e < uint32_t(tl.c1); e += kBlock) { const float a = g[e]; acc0 = fmaf(a, a, acc0); }
    const float s = block_sum((acc0 + acc1) + (acc2 + acc3), red);
    if (tid == 0) ws[d.off_rowpart + tl.win] = s;
    return;
  }

  const int cwl = tl.cw_log2;
  const int CW = 1 << cwl;
  const int RS = kBlock >> cwl;
  const int slot = tid >> cwl;
  const int lc = tid & (CW - 1);
  const int j = tl.c0 + lc;
  const bool colok = j < tl.c1;
  const int R = d.R, C = d.C;
  const int iters = (tl.r1 - tl.r0 + RS - 1) / RS;
  const int wave = tid >> 6;
  float colacc = 0.f;
  for (int q0 = 0; q0 < iters; q0 += 4) {
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tl.r0 + slot + RS * (q0 + u);
      x[u] = (colok && q0 + u < iters && i < tl.r1) ? g[size_t(i) * C + j] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + u;
      if (q >= iters) break;  // uniform across the block
      const int i = tl.r0 + slot + RS * q;
      const float x2 = x[u] * x[u];
      colacc += x2;
      float rs = x2;
      if (CW <= 64) {
        for (int o = CW >> 1; o > 0; o >>= 1) rs += __shfl_xor(rs, o);
        if (lc == 0 && i < tl.r1) ws[d.off_rowpart + size_t(tl.win) * R + i] = rs;
      } else {
        rs = wave_sum(rs);
        if ((tid & 63) == 0) lds_rows[wave * kTile0Iters + q] = rs;
      }
    }
  }
  lds_cols[tid] = colacc;
  __syncthreads();
  if (CW > 64) {
    const int wps = CW >> 6;  // waves per row slot
    if (tid < RS * iters) {
      const int s = tid / iters, q = tid - s * iters;
      const int i = tl.r0 + s + RS * q;
      if (i < tl.r1) {
        float v = 0.f;
        for (int w = 0; w < wps; ++w) v += lds_rows[(s * wps + w) * kTile0Iters + q];
        ws[d.off_rowpart + size_t(tl.win) * R + i] = v;
      }
    }
  }
  if (tid < CW && colok) {
    float v = 0.f;
    for (int s = 0; s < RS; ++s) v += lds_cols[s * CW + lc];
    ws[d.off_colpart + size_t(tl.rb) * C + j] = v;
  }
}

// ---------------------------------------------------------------------------
// k_moving_avg: r_k and c_k moving averages (written to the state), their
// inverse square roots (workspace) and per-segment partial sums of r_k.
__global__ __launch_bounds__(kBlock) void k_moving_avg(StepCtx c, StepParams hp) {
  const Seg1 sg = c.segs1[blockIdx.x];
  const TensorDesc d = c.desc[sg.tensor];
  float* __restrict__ ws = c.ws;
  const int tid = threadIdx.x;
  __shared__ float red[4];
  const size_t n = d.n;
  float* r = d.st + 4 * n;
  float* cst = r + 3 * size_t(d.R);

  if (sg.kind == kSegRows) {
    const int i = sg.a + tid;
    float loc[3] = {0.f, 0.f, 0.f};
    if (i < sg.b) {
      float s = 0.f;
      for (int w = 0; w < d.ncw; ++w) s += ws[d.off_rowpart + size_t(w) * d.R + i];
      const float mean = s / float(d.C);
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const float rk = fmaf(hp.beta_f[k], r[size_t(k) * d.R + i], (1.0f - hp.beta_f[k]) * (mean + hp.eps_f));
        r[size_t(k) * d.R + i] = rk;
        ws[d.off_rq + size_t(k) * d.R + i] = rsqrtf(rk);
        loc[k] = rk;
      }
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const float s = block_sum(loc[k], red);
      if (tid == 0) c.rbar_part[sg.slot * 4 + k] = s;
    }
  } else if (sg.kind == kSegCols) {
    const int j = sg.a + tid;
    if (j < sg.b) {
      float s = 0.f;
      for (int b = 0; b < d.nrb; ++b) s += ws[d.off_colpart + size_t(b) * d.C + j];
      const float mean = s / float(d.R);
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const float ck = fmaf(hp.beta_f[k], cst[size_t(k) * d.C + j], (1.0f - hp.beta_f[k]) * (mean + hp.eps_f));
        cst[size_t(k) * d.C + j] = ck;
        ws[d.off_cq + size_t(k) * d.C + j] = rsqrtf(ck);
      }
    }
  } else {  // 1-D tensor: r_k is one value per tensor
    float s = 0.f;
    for (int w = tid; w < d.ncw; w += kBlock) s += ws[d.off_rowpart + w];
    s = block_sum(s, red);
    if (tid == 0) {
      const float mean = s / float(d.C);
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const float rk = fmaf(hp.beta_f[k], r[k], (1.0f - hp.beta_f[k]) * (mean + hp.eps_f));
        r[k] = rk;
        ws[d.off_rq + k] = rsqrtf(rk);
        c.rbar_part[sg.slot * 4 + k] = rk;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_stats: per-chunk sums of the squares of the 28 features (the page's
// kernel 1).  Accumulators are updated in registers only; the apply kernel
// recomputes them from the same inputs.
template <bool VEC>
__device__ __forceinline__ void stats_body(const StepCtx& c, const StepParams& hp, const Chunk& ch,
                                           const TensorDesc& d, const float sr[3], float acc[kNF]) {
  const float* __restrict__ g = c.grads[ch.tensor];
  for (uint32_t e = ch.e0 + threadIdx.x; e < ch.e1; e += kBlock) {
    Elem x;
    load_elem<VEC>(d, g, c.ws, e, x);
    float F[kNF], cn[3];
    build_features<VEC>(hp, x, sr, F, cn);
#pragma unroll
    for (int f = 0; f < kNF; ++f) acc[f] = fmaf(F[f], F[f], acc[f]);
  }
}

__global__ __launch_bounds__(kBlock) void k_stats(StepCtx c, StepParams hp) {
  const Chunk ch = c.chunks[blockIdx.x];
  const TensorDesc d = c.desc[ch.tensor];
  __shared__ float lds[4][kNF];
  __shared__ float red[4];
  float sr[3];
  block_sr(c, d, sr, red);
  float acc[kNF];
#pragma unroll
  for (int f = 0; f < kNF; ++f) acc[f] = 0.f;
  if (d.vec) stats_body<true>(c, hp, ch, d, sr, acc);
  else stats_body<false>(c, hp, ch, d, sr, acc);
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int f = 0; f < kNF; ++f) {
    const float s = wave_sum(acc[f]);
    if ((threadIdx.x & 63) == 0) lds[w][f] = s;
  }
  __syncthreads();
  if (threadIdx.x < kNF) {
    const int f = threadIdx.x;
    c.stats_part[size_t(blockIdx.x) * kStatStride + f] = (lds[0][f] + lds[1][f]) + (lds[2][f] + lds[3][f]);
  }
}

// ---------------------------------------------------------------------------
// k_finalize: per tensor, S_d = sum of the chunk partials (chunk order), then
// s_d = (S_d / n + eps_norm)^(-1/2); also sqrt(rbar_k).  Block 0 packs the MLP
// for the apply kernel, folding the step features into the first bias:
// b1' = b1 + W1[:, 28:28+n_time] tanh(t / tau).
__global__ __launch_bounds__(kBlock) void k_finalize(StepCtx c, StepParams hp) {
  const int t = blockIdx.x;
  const TensorDesc d = c.desc[t];
  __shared__ float lds[4][kNF];
  __shared__ float red[4];
  float sr[3];
  block_sr(c, d, sr, red);
  float acc[kNF];
#pragma unroll
  for (int f = 0; f < kNF; ++f) acc[f] = 0.f;
  for (int q = threadIdx.x; q < d.nchunk; q += kBlock) {
    const float* sp = c.stats_part + size_t(d.chunk0 + q) * kStatStride;
#pragma unroll
    for (int f = 0; f < kNF; ++f) acc[f] += sp[f];
  }
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int f = 0; f < kNF; ++f) {
    const float s = wave_sum(acc[f]);
    if ((threadIdx.x & 63) == 0) lds[w][f] = s;
  }
  __syncthreads();
  float* sc = c.scales + size_t(t) * kStatStride;
  if (threadIdx.x < kNF) {
    const int f = threadIdx.x;
    const float S = (lds[0][f] + lds[1][f]) + (lds[2][f] + lds[3][f]);
    sc[f] = 1.0f / sqrtf(S / float(d.n) + hp.eps_norm);
  } else if (threadIdx.x < kNF + 3) {
    const int k = threadIdx.x - kNF;
    sc[kNF + k] = sr[k];
  }

  if (t == 0) {
    const int din = kNF + hp.n_time;
    const float* W1 = c.mlp;
    const float* b1 = W1 + kH * din;
    const float* W2 = b1 + kH;
    const float* b2 = W2 + kH * kH;
    const float* W3 = b2 + kH;
    const float* b3 = W3 + 2 * kH;
    float* pk = c.packed;
    for (int q = threadIdx.x; q < kH * kNF; q += kBlock) {
      const int o = q / kNF, f = q - o * kNF;
      pk[kPkW1 + q] = W1[o * din + f];
    }
    if (threadIdx.x < kH) {
      const int o = threadIdx.x;
      float b = b1[o];
      for (int s = 0; s < hp.n_time; ++s) b = fmaf(W1[o * din + kNF + s], tanhf(hp.t / hp.timescales[s]), b);
      pk[kPkB1 + o] = b;
      pk[kPkB2 + o] = b2[o];
      pk[kPkW3 + o] = W3[o];
      pk[kPkW3 + kH + o] = W3[kH + o];
    }
    for (int q = threadIdx.x; q < kH * kH; q += kBlock) pk[kPkW2 + q] = W2[q];
    if (threadIdx.x < 2) pk[kPkB3 + threadIdx.x] = b3[threadIdx.x];
  }
}

// ---------------------------------------------------------------------------
// k_apply_valu: the page's kernel 2 with the MLP on the vector ALU.  Weights
// are read through uniform (scalar) loads from the packed copy, so every FMA
// takes its weight from a scalar register.
template <bool VEC>
__device__ __forceinline__ void apply_valu_body(const StepCtx& c, const StepParams& hp, const Chunk& ch,
                                                const TensorDesc& d) {
  const float* __restrict__ g = c.grads[ch.tensor];
  const float* __restrict__ pk = c.packed;
  const float* __restrict__ sc = c.scales + size_t(ch.tensor) * kStatStride;
  float sr[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) sr[k] = sc[kNF + k];
  const size_t n = d.n;
  for (uint32_t e = ch.e0 + threadIdx.x; e < ch.e1; e += kBlock) {
    Elem x;
    load_elem<VEC>(d, g, c.ws, e, x);
    const float p_old = x.p;
    float F[kNF], cn[3];
    build_features<VEC>(hp, x, sr, F, cn);
#pragma unroll
    for (int f = 0; f < kNF; ++f) F[f] *= sc[f];
    float h1[kH];
#pragma unroll
    for (int o = 0; o < kH; ++o) {
      float a = pk[kPkB1 + o];
#pragma unroll
      for (int f = 0; f < kNF; ++f) a = fmaf(pk[kPkW1 + o * kNF + f], F[f], a);
      h1[o] = fmaxf(a, 0.f);
    }
    float dir = pk[kPkB3], mag = pk[kPkB3 + 1];
#pragma unroll
    for (int o = 0; o < kH; ++o) {
      float a = pk[kPkB2 + o];
#pragma unroll
      for (int f = 0; f < kH; ++f) a = fmaf(pk[kPkW2 + o * kH + f], h1[f], a);
      a = fmaxf(a, 0.f);
      dir = fmaf(pk[kPkW3 + o], a, dir);
      mag = fmaf(pk[kPkW3 + kH + o], a, mag);
    }
    const float u = dir * expf(mag * hp.exp_mult) * hp.step_mult;
    d.p[e] = p_old - hp.lr * fmaf(hp.weight_decay, p_old, u);
    float* st = d.st;
    st[e] = x.m[0];
    st[n + e] = x.m[1];
    st[2 * n + e] = x.m[2];
    st[3 * n + e] = x.v;
    if (VEC) {
      float* cs = st + 4 * n + 3;
#pragma unroll
      for (int k = 0; k < 3; ++k) cs[k * n + e] = cn[k];
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_apply_valu(StepCtx c, StepParams hp) {
  const Chunk ch = c.chunks[blockIdx.x];
  const TensorDesc d = c.desc[ch.tensor];
  if (d.vec) apply_valu_body<true>(c, hp, ch, d);
  else apply_valu_body<false>(c, hp, ch, d);
}

// ---------------------------------------------------------------------------
// k_apply_mfma: the page's kernel 2 with layers 1 and 2 of the MLP on the fp32
// matrix cores.  A wave owns 64 elements per iteration, one per lane, for all
// per-element work (loads, features, update, stores).  The MLP is a pair of
// 32-element GEMM chains per wave, v_mfma_f32_32x32x2_f32 with the hidden
// units as M (weights = A operand, register resident), the elements as N and
// the features as K:
//   layer 1: 14 K-steps of two features.  v_permlane32_swap of the feature
//     pair (2s, 2s+1) gives, in one instruction, the B operands of both
//     halves: [F_2s of elements 0..31 | F_2s+1 of elements 0..31] and
//     [F_2s of elements 32..63 | F_2s+1 of elements 32..63].
//   layer 2: the layer-1 accumulator register r of a lane holds hidden unit
//     8(r/4) + 4(lane/32) + r%4 of element lane%32, which is exactly a K-step
//     B operand if W2's columns are visited in that order (no data movement).
//   layer 3 (32 -> 2) on the vector ALU: per-lane partial dot products over
//     the lane's 16 hidden units, completed with one more swap.
// Biases enter as the C operand of the first MFMA of each chain; the feature
// scales s_d are folded into W1's columns once per chunk.
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

__device__ __forceinline__ void swap_halves(float x, float y, float& lo, float& hi) {
  // lo = [x lanes 0..31 | y lanes 0..31], hi = [x lanes 32..63 | y lanes 32..63]
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

template <bool VEC>
__device__ __forceinline__ void apply_mfma_body(const StepCtx& c, const StepParams& hp, const Chunk& ch,
                                                const TensorDesc& d) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int row = lane & 31;
  const float* __restrict__ g = c.grads[ch.tensor];
  const float* __restrict__ pk = c.packed;
  const float* __restrict__ sc = c.scales + size_t(ch.tensor) * kStatStride;

  float a1[kNF / 2];   // W1[row][2s + half] * s_(2s + half)
  float a2[kH / 2];    // W2[row][acc_row(s, half)]
  f32x16 bias1, bias2;
  float w3d[16], w3m[16];
#pragma unroll
  for (int q = 0; q < kNF / 2; ++q) a1[q] = pk[kPkW1 + row * kNF + 2 * q + half] * sc[2 * q + half];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int hr = acc_row(q, half);
    a2[q] = pk[kPkW2 + row * kH + hr];
    bias1[q] = pk[kPkB1 + hr];
    bias2[q] = pk[kPkB2 + hr];
    w3d[q] = pk[kPkW3 + hr];
    w3m[q] = pk[kPkW3 + kH + hr];
  }
  const float b3d = pk[kPkB3], b3m = pk[kPkB3 + 1];
  float sr[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) sr[k] = sc[kNF + k];
  const size_t n = d.n;

  for (uint32_t base = ch.e0 + wave * 64; base < ch.e1; base += kBlock) {
    const uint32_t e = base + lane;
    const bool valid = e < ch.e1;
    Elem x;
    load_elem<VEC>(d, g, c.ws, valid ? e : ch.e0, x);
    const float p_old = x.p;
    float F[kNF], cn[3];
    build_features<VEC>(hp, x, sr, F, cn);

    f32x16 accA = bias1, accB = bias1;
#pragma unroll
    for (int q = 0; q < kNF / 2; ++q) {
      float bA, bB;
      swap_halves(F[2 * q], F[2 * q + 1], bA, bB);
      accA = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[q], bA, accA, 0, 0, 0);
      accB = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[q], bB, accB, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      accA[q] = fmaxf(accA[q], 0.f);
      accB[q] = fmaxf(accB[q], 0.f);
    }
    f32x16 acc2A = bias2, acc2B = bias2;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      acc2A = __builtin_amdgcn_mfma_f32_32x32x2f32(a2[q], accA[q], acc2A, 0, 0, 0);
      acc2B = __builtin_amdgcn_mfma_f32_32x32x2f32(a2[q], accB[q], acc2B, 0, 0, 0);
    }
    float dA = 0.f, mA = 0.f, dB = 0.f, mB = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float hA = fmaxf(acc2A[q], 0.f), hB = fmaxf(acc2B[q], 0.f);
      dA = fmaf(w3d[q], hA, dA);
      mA = fmaf(w3m[q], hA, mA);
      dB = fmaf(w3d[q], hB, dB);
      mB = fmaf(w3m[q], hB, mB);
    }
    // lane l < 32 holds chain A's partials of element l (its half) and lane
    // l + 32 the other half; chain B likewise for element 32 + l.
    float d0, d1, m0, m1;
    swap_halves(dA, dB, d0, d1);
    swap_halves(mA, mB, m0, m1);
    const float dir = (d0 + d1) + b3d;
    const float mag = (m0 + m1) + b3m;
    if (valid) {
      const float u = dir * expf(mag * hp.exp_mult) * hp.step_mult;
      d.p[e] = p_old - hp.lr * fmaf(hp.weight_decay, p_old, u);
      float* st = d.st;
      st[e] = x.m[0];
      st[n + e] = x.m[1];
      st[2 * n + e] = x.m[2];
      st[3 * n + e] = x.v;
      if (VEC) {
        float* cs = st + 4 * n + 3;
#pragma unroll
        for (int k = 0; k < 3; ++k) cs[k * n + e] = cn[k];
      }
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_apply_mfma(StepCtx c, StepParams hp) {
  const Chunk ch = c.chunks[blockIdx.x];
  const TensorDesc d = c.desc[ch.tensor];
  if (d.vec) apply_mfma_body<true>(c, hp, ch, d);
  else apply_mfma_body<false>(c, hp, ch, d);
}

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
  hipLaunchKernelGGL(k_finalize, dim3(c.n_tensors), dim3(kBlock), 0, s, c, p);
  if ((e = mark(4)) != hipSuccess) return e;
  if (c.mlp_impl == 1)
    hipLaunchKernelGGL(k_apply_valu, dim3(c.n_chunks), dim3(kBlock), 0, s, c, p);
  else
    hipLaunchKernelGGL(k_apply_mfma, dim3(c.n_chunks), dim3(kBlock), 0, s, c, p);
  if ((e = mark(5)) != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace lopt
