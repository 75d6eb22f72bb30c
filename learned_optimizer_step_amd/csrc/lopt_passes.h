// Bodies of the four streaming passes of the optimizer step, one workgroup's
// share each, indexed by a work-list position: the row/column sums of g^2,
// the row/column moving averages, the statistics pass (the PyLO page's
// kernel 1, "CUDA kernel design: two-pass fusion" > "Fused kernel strategy")
// and the per-tensor finalize.  lopt_kernels.hip launches each as a kernel of
// its own; lopt_single.hip runs all of them, and the apply pass, in one launch.
#pragma once

#include <hip/hip_runtime.h>

#include "lopt_device.h"

namespace lopt {

// ---------------------------------------------------------------------------
// Row/column pass (k_rowcol_sumsq), one tile: row sums and column sums of g^2.
//   2-D tile: rows [r0, r1) x a window of CW <= 256 columns.  Thread t handles
//   column c0 + (t mod CW) for rows r0 + (t / CW) + RS q, RS = 256 / CW.
//   Row sums: butterfly over the CW lanes of a row slot (CW <= 64), or over
//   the wave and then the CW/64 waves of the slot through LDS.
//   Column sums: per-thread over its rows, then over the RS row slots in LDS.
//   Flat tile (1-D tensors): one partial of sum g^2 over [c0, c1).
__device__ __forceinline__ void rowcol_block(const StepCtx& c, uint32_t bid) {
  const Tile0 tl = c.tiles0[bid];
  const float* __restrict__ g = uni(c.grads[tl.tensor]);
  if (!g) return;  // no gradient this step: the tensor is skipped
  const TensorDesc d = c.desc[tl.tensor];
  float* __restrict__ ws = c.ws;
  const int tid = threadIdx.x;
  __shared__ float lds_rows[4 * kTile0Iters];
  __shared__ float lds_cols[kBlock];
  __shared__ float red[4];

  if (tl.flat) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    uint32_t e = tl.c0 + tid;
    for (; e + 7 * kBlock < uint32_t(tl.c1); e += 8 * kBlock) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = __builtin_nontemporal_load(g + e + u * kBlock);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] = fmaf(x[u], x[u], acc[u]);
    }
    for (; e < uint32_t(tl.c1); e += kBlock) {
      const float a = __builtin_nontemporal_load(g + e);
      acc[0] = fmaf(a, a, acc[0]);
    }
    const float s = block_sum(((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7])), red);
    if (tid == 0) ws[d.off_rowpart + tl.win] = s;
    return;
  }

  if (tl.cw_log2 == 8 && (d.C & 3) == 0 && (reinterpret_cast<uintptr_t>(g) & 15) == 0) {
    // 256-column window, rows 16-byte aligned: each wave reads whole row
    // segments with 16-byte loads (lane = 4 columns), waves take rows
    // r0 + wave + 4u; a row's window sum completes inside one wave.
    constexpr int kB = 8;  // rows per wave per batch
    const int lane = tid & 63, wave = tid >> 6;
    const int cb = tl.c0 + 4 * lane;
    const bool act = cb < tl.c1;  // cols % 4 == 0: all four columns valid
    const f32x4* __restrict__ g4 = reinterpret_cast<const f32x4*>(g);
    const int C4 = d.C >> 2;
    float4 ca = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int r = tl.r0 + wave; r < tl.r1; r += 4 * kB) {
      f32x4 x[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int i = r + 4 * u;
        x[u] = (act && i < tl.r1) ? __builtin_nontemporal_load(g4 + size_t(i) * C4 + (cb >> 2)) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const float4 v = make_float4(x[u].x * x[u].x, x[u].y * x[u].y, x[u].z * x[u].z, x[u].w * x[u].w);
        ca.x += v.x; ca.y += v.y; ca.z += v.z; ca.w += v.w;
        const float rs = wave_sum((v.x + v.y) + (v.z + v.w));
        const int i = r + 4 * u;
        if (lane == 0 && i < tl.r1) ws[d.off_rowpart + size_t(tl.win) * d.R + i] = rs;
      }
    }
    __shared__ float lds_c4[4][kBlock];
    lds_c4[wave][4 * lane] = ca.x;
    lds_c4[wave][4 * lane + 1] = ca.y;
    lds_c4[wave][4 * lane + 2] = ca.z;
    lds_c4[wave][4 * lane + 3] = ca.w;
    __syncthreads();
    const int j = tl.c0 + tid;
    if (j < tl.c1)
      ws[d.off_colpart + size_t(tl.rb) * d.C + j] = (lds_c4[0][tid] + lds_c4[1][tid]) + (lds_c4[2][tid] + lds_c4[3][tid]);
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
  constexpr int kRowBatch = 16;  // rows loaded per thread before reducing (bytes in flight)
  for (int q0 = 0; q0 < iters; q0 += kRowBatch) {
    float x[kRowBatch];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) {
      const int i = tl.r0 + slot + RS * (q0 + u);
      x[u] = (colok && q0 + u < iters && i < tl.r1) ? __builtin_nontemporal_load(g + size_t(i) * C + j) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) {
      const int q = q0 + u;
      if (q < iters) {  // uniform across the block
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
// Compensated (Kahan) running sum: the moving-average kernel adds up to
// thousands of similar positive partials per row or column in sequence (a
// 2^31-element matrix has ~11,000 row blocks), where a plain fp32 sum would
// drift by ~sqrt(count) roundings.  The device code is compiled without
// reassociation, so the compensation is kept as written.  Once the sum is
// infinite the compensation stays 0, so an infinite partial gives an
// infinite sum (as a plain sum would), not inf - inf = NaN.
struct KahanSum {
  float s = 0.f, comp = 0.f;
  __device__ __forceinline__ void add(float x) {
    const float y = x - comp;
    const float t = s + y;
    comp = __builtin_isfinite(t) ? (t - s) - y : 0.f;
    s = t;
  }
};

// Sum of g^2 down column j of a 2-D tensor from its row-block partials: 64
// columns per segment, 4 thread groups per column over the partials (b =
// group, group + 4, ...), combined in LDS in group order.  Every thread of the
// block calls it; the result is valid in group 0 for j < end.
__device__ __forceinline__ float column_sumsq(const StepCtx& c, const TensorDesc& d, int j, int end,
                                              float (&part)[kColGroups][kSegCols1]) {
  const int jl = threadIdx.x % kSegCols1, grp = threadIdx.x / kSegCols1;
  KahanSum ks;
  if (j < end)
    for (int b = grp; b < d.nrb; b += kColGroups) ks.add(c.ws[d.off_colpart + size_t(b) * d.C + j]);
  part[grp][jl] = ks.s;
  __syncthreads();
  return (part[0][jl] + part[1][jl]) + (part[2][jl] + part[3][jl]);
}

// Sum of g^2 over a 1-D tensor from its flat-tile partials (every thread gets it).
__device__ __forceinline__ float vector_sumsq(const StepCtx& c, const TensorDesc& d, float* red) {
  KahanSum ks;
  for (int w = threadIdx.x; w < d.ncw; w += kBlock) ks.add(c.ws[d.off_rowpart + w]);
  return block_sum(ks.s, red);
}

// Moving-average pass (k_moving_avg), one segment: r_k and c_k moving averages (written to the state), their
// inverse square roots (workspace) and per-segment partial sums of r_k.
__device__ __forceinline__ void moving_avg_block(const StepCtx& c, const StepParams& hp, uint32_t bid) {
  const Seg1 sg = c.segs1[bid];
  if (!uni(c.grads[sg.tensor])) return;  // no gradient this step: the tensor is skipped
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
      KahanSum ks;
      for (int w = 0; w < d.ncw; ++w) ks.add(ws[d.off_rowpart + size_t(w) * d.R + i]);
      const float mean = ks.s / float(d.C);
      float q[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const float rk = fmaf(hp.beta_f[k], r[size_t(k) * d.R + i], hp.omb_f[k] * (mean + hp.eps_f));
        r[size_t(k) * d.R + i] = rk;
        q[k] = rsqrtf(rk);
        loc[k] = rk;
      }
      reinterpret_cast<float4*>(ws + d.off_rq)[i] = make_float4(q[0], q[1], q[2], 0.f);
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const float s = block_sum(loc[k], red);
      if (tid == 0) c.rbar_part[sg.slot * 4 + k] = s;
    }
  } else if (sg.kind == kSegCols) {
    // the column's sum of g^2: from this list's row-block partials, or, for a
    // row shard (c.sharded), over every shard's rows (the exchanged sums)
    __shared__ float part[kColGroups][kSegCols1];
    const int jl = tid % kSegCols1, grp = tid / kSegCols1;
    const int j = sg.a + jl;
    float s;
    if (c.sharded) s = (grp == 0 && j < sg.b) ? c.sums1[d.off_sum1 + j] : 0.f;
    else s = column_sumsq(c, d, j, sg.b, part);
    if (grp == 0 && j < sg.b) {
      const float mean = s / float(d.Rg);
      float q[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const float ck = fmaf(hp.beta_f[k], cst[size_t(k) * d.C + j], hp.omb_f[k] * (mean + hp.eps_f));
        cst[size_t(k) * d.C + j] = ck;
        q[k] = rsqrtf(ck);
      }
      reinterpret_cast<float4*>(ws + d.off_cq)[j] = make_float4(q[0], q[1], q[2], 0.f);
    }
  } else {  // 1-D tensor: r_k is one value per tensor (over every shard's elements)
    const float s = c.sharded ? c.sums1[d.off_sum1] : vector_sumsq(c, d, red);
    if (tid == 0) {
      const float mean = s / float(d.ng);
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const float rk = fmaf(hp.beta_f[k], r[k], hp.omb_f[k] * (mean + hp.eps_f));
        r[k] = rk;
        ws[d.off_rq + k] = rsqrtf(rk);
        c.rbar_part[sg.slot * 4 + k] = rk;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Statistics pass (k_stats): per-chunk sums of the squares of the 28 features (the page's
// kernel 1).  Accumulators are updated in registers only; the apply kernel
// recomputes them from the same inputs.
template <bool VEC, bool NORMAL, int NF>
__device__ __forceinline__ void stats_accumulate(const StepParams& hp, Elem& x, float acc[kNF]) {
  float F[kNF], cn[3];
  build_features<VEC, NORMAL, NF>(hp, x, F, cn);
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = fmaf(F[f], F[f], acc[f]);
}

// Four elements per thread per iteration, their loads issued together, so
// each thread keeps ~100 bytes of HBM reads in flight.  RU (2-D tensors whose
// column count is a multiple of 64): a wave's 64 consecutive elements lie in
// one row (chunks start at multiples of 256 and end at multiples of 64), so
// the row index is divided once per wave and the row record read once, and
// every loop condition is the same for all lanes of a wave.
template <bool VEC, bool NORMAL, int NF, bool RU>
__device__ __forceinline__ void stats_body(const StepCtx& c, const StepParams& hp, const Chunk& ch,
                                           const TensorDesc& d, const float* g, float acc[kNF]) {
  constexpr bool ROW = RU && !VEC;
  const Streams st = make_streams(d, g, c.ws, ch);
  const uint32_t lane = threadIdx.x & 63;
  uint32_t e = ch.e0 + threadIdx.x;
  for (; e + 3 * kBlock < ch.e1; e += 4 * kBlock) {
    Elem x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t eu = e + u * kBlock;
      load_elem<VEC, ROW>(st, eu, x[u], ROW ? uni(eu - lane) : 0u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) stats_accumulate<VEC, NORMAL, NF>(hp, x[u], acc);
  }
  for (; e < ch.e1; e += kBlock) {
    Elem x;
    load_elem<VEC, ROW>(st, e, x, ROW ? uni(e - lane) : 0u);
    stats_accumulate<VEC, NORMAL, NF>(hp, x, acc);
  }
}

__device__ __forceinline__ void stats_block(const StepCtx& c, const StepParams& hp, uint32_t bid) {
  Chunk ch;
  TensorDesc d;
  const float* g;
  load_chunk(c, bid, ch, d, g);
  if (!g) return;  // no gradient this step: the tensor is skipped
  __shared__ float lds[4][kNF];
  float acc[kNF];
#pragma unroll
  for (int f = 0; f < kNF; ++f) acc[f] = 0.f;
  dispatch_variant<true>(d, hp, [&](auto v) {
    using V = decltype(v);
    stats_body<V::vec, V::normal, V::nf, V::rowuni>(c, hp, ch, d, g, acc);
  });
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int f = 0; f < kNF; ++f) {
    const float s = wave_sum(acc[f]);
    if ((threadIdx.x & 63) == 0) lds[w][f] = s;
  }
  __syncthreads();
  if (threadIdx.x < kNF) {
    const int f = threadIdx.x;
    c.stats_part[size_t(bid) * kStatStride + f] = (lds[0][f] + lds[1][f]) + (lds[2][f] + lds[3][f]);
  }
}

// sqrt(mean_i r_k[i]) from the per-segment partial sums of r_k, summed by the
// whole block in a fixed order (every caller gets bitwise the same value).
// All threads must call it (it contains barriers); a 1-D tensor gets sqrt(r_k).
__device__ __forceinline__ void block_sr(const StepCtx& c, const TensorDesc& d, float sr[3], float* red) {
  // every thread's loads first (one round trip), then the three block sums
  float s[3] = {0.f, 0.f, 0.f};
  for (int q = threadIdx.x; q < d.nrseg; q += kBlock) {
#pragma unroll
    for (int k = 0; k < 3; ++k) s[k] += c.rbar_part[(d.rseg0 + q) * 4 + k];
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) sr[k] = sqrtf(block_sum(s[k], red) / float(d.Rg));
}

// Per-tensor sums of the statistics pass's chunk partials, in two parts so
// that a caller can issue other loads between them: each thread adds its
// chunks in order (chunk_partials), then the wave butterfly and the 4 waves
// in LDS order (feature_wave_sums: lds[w][f] holds wave w's sum of feature f
// after its barrier).
__device__ __forceinline__ void chunk_partials(const StepCtx& c, const TensorDesc& d, float (&acc)[kNF]) {
#pragma unroll
  for (int f = 0; f < kNF; ++f) acc[f] = 0.f;
  for (int q = threadIdx.x; q < d.nchunk; q += kBlock) {
    const float* sp = c.stats_part + size_t(d.chunk0 + q) * kStatStride;
#pragma unroll
    for (int f = 0; f < kNF; ++f) acc[f] += sp[f];
  }
}

__device__ __forceinline__ void feature_wave_sums(const float (&acc)[kNF], float (&lds)[4][kNF]) {
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int f = 0; f < kNF; ++f) {
    const float s = wave_sum(acc[f]);
    if ((threadIdx.x & 63) == 0) lds[w][f] = s;
  }
  __syncthreads();
}

// Packs the MLP for the apply kernel (one block): W1's feature columns, b1
// with the step features folded in, W2, b2, W3, b3; advances the step counter.
__device__ __forceinline__ void pack_mlp(const StepCtx& c, const StepParams& hp) {
  // The step counter lives in device memory so that a captured step, replayed
  // from a graph, still sees t = 1, 2, 3, ...  Every thread reads it, then
  // thread 0 advances it after the barrier below.
  const int64_t step = *c.step + 1;
  const float tf = float(step);
  const int nf = hp.n_feat;
  const int din = nf + hp.n_time;
  const float* W1 = c.mlp;
  const float* b1 = W1 + kH * din;
  const float* W2 = b1 + kH;
  const float* b2 = W2 + kH * kH;
  const float* W3 = b2 + kH;
  const float* b3 = W3 + 2 * kH;
  float* pk = c.packed;
  // the step features tanh(t / tau_s), one per thread, shared through LDS
  __shared__ float tfeat[kMaxTime];
  if (threadIdx.x < hp.n_time) tfeat[threadIdx.x] = tanhf(tf / hp.timescales[threadIdx.x]);
  for (int q = threadIdx.x; q < kH * kNF; q += kBlock) {
    const int o = q / kNF, f = q - o * kNF;
    pk[kPkW1 + q] = f < nf ? W1[o * din + f] : 0.f;
  }
  __syncthreads();
  if (threadIdx.x < kH) {
    const int o = threadIdx.x;
    float b = b1[o];
    for (int s = 0; s < hp.n_time; ++s) b = fmaf(W1[o * din + nf + s], tfeat[s], b);
    pk[kPkB1 + o] = b;
    pk[kPkB2 + o] = b2[o];
    pk[kPkW3 + o] = W3[o];
    pk[kPkW3 + kH + o] = W3[kH + o];
  }
  for (int q = threadIdx.x; q < kH * kH; q += kBlock) pk[kPkW2 + q] = W2[q];
  if (threadIdx.x < 2) pk[kPkB3 + threadIdx.x] = b3[threadIdx.x];
  __syncthreads();
  if (threadIdx.x == 0) *c.step = step;
}

// ---------------------------------------------------------------------------
// Finalize pass (k_finalize), one block per tensor: S'_d = sum of the chunk partials (chunk order).  The
// statistics pass leaves sqrt(rbar_k) out of rho_k, so for the rho features
// S_d = S'_d rbar_k.  Then s_d = (S_d / n + eps_norm)^(-1/2), and the scale
// stored for the apply kernel (which also leaves sqrt(rbar_k) out) is s_d, or
// s_d sqrt(rbar_k) for the rho features.  The last block (index n_tensors)
// packs the MLP for the apply kernel, folding the step features into the first
// bias: b1' = b1 + W1[:, 28:28+n_time] tanh(t / tau); it runs beside the
// per-tensor blocks instead of after tensor 0's.
__device__ __forceinline__ void finalize_block(const StepCtx& c, const StepParams& hp, uint32_t bid) {
  const int t = int(bid);
  if (t == c.n_tensors) {
    pack_mlp(c, hp);
    return;
  }
  if (!uni(c.grads[t])) return;  // no gradient this step: the tensor is skipped
  const TensorDesc d = c.desc[t];
  __shared__ float lds[4][kNF];
  __shared__ float red[4];
  // For a row shard (c.sharded) the sums of r_k over rows and of the squared
  // features come from the exchange buffer, summed over every shard; a 1-D
  // tensor's r_k is the same on every shard already.
  const float* gsum = c.sharded ? c.sums2 + size_t(t) * kStatStride : nullptr;
  float sr[3];
  float acc[kNF];
  if (!gsum) chunk_partials(c, d, acc);   // its loads go out with block_sr's
  if (gsum && !d.vec) {
#pragma unroll
    for (int k = 0; k < 3; ++k) sr[k] = sqrtf(gsum[kNF + k] / float(d.Rg));
  } else {
    block_sr(c, d, sr, red);
  }
  if (!gsum) feature_wave_sums(acc, lds);
  float* sc = c.scales + size_t(t) * kStatStride;
  if (threadIdx.x < kNF) {
    const int f = threadIdx.x;
    const int k = rho_feature(f);
    // a 1-D tensor's rho_k is c_k^(-1/2) itself (its r_k over their mean is 1)
    const float rb = (k < 0 || d.vec) ? 1.0f : sr[k];
    const float Sp = gsum ? gsum[f] : (lds[0][f] + lds[1][f]) + (lds[2][f] + lds[3][f]);
    const float S = Sp * (rb * rb);
    // features the variant does not feed get scale 0 (their weights are 0 too)
    sc[f] = f < hp.n_feat ? rb / sqrtf(S / float(d.ng) + hp.eps_norm) : 0.f;
  } else if (threadIdx.x < kNF + 3) {
    const int k = threadIdx.x - kNF;
    sc[kNF + k] = sr[k];
  }
}

// ---------------------------------------------------------------------------
// Row shards (lopt_init_state_sharded): the two sums a shard exports for the
// exchange across ranks (summed there, then read back by the passes above).
//
// First export, after the row/column pass, one moving-average segment: the
// column sums of g^2 of a 2-D tensor (sums1[off_sum1 + j]) and the sum of g^2
// of a 1-D tensor (sums1[off_sum1]); a row segment exports nothing (its rows'
// sums are complete on the shard).
__device__ __forceinline__ void shard_colsum_block(const StepCtx& c, uint32_t bid) {
  const Seg1 sg = c.segs1[bid];
  if (!uni(c.grads[sg.tensor])) return;  // no gradient this step: the tensor is skipped
  const TensorDesc d = c.desc[sg.tensor];
  __shared__ float red[4];
  if (sg.kind == kSegCols) {
    __shared__ float part[kColGroups][kSegCols1];
    const int jl = threadIdx.x % kSegCols1, grp = threadIdx.x / kSegCols1;
    const int j = sg.a + jl;
    const float s = column_sumsq(c, d, j, sg.b, part);
    if (grp == 0 && j < sg.b) c.sums1[d.off_sum1 + j] = s;
  } else if (sg.kind == kSegVec) {
    const float s = vector_sumsq(c, d, red);
    if (threadIdx.x == 0) c.sums1[d.off_sum1] = s;
  }
}

// Second export, after the statistics pass, one tensor: the sums of the
// squared features over the shard's chunks (sums2[32 t + d], d < 28) and of
// r_k over the shard's rows (sums2[32 t + 28 + k]; 0 for a 1-D tensor, whose
// r_k is not summed across shards), in the finalize pass's order.
__device__ __forceinline__ void shard_reduce_block(const StepCtx& c, uint32_t bid) {
  const int t = int(bid);
  if (!uni(c.grads[t])) return;  // no gradient this step: the tensor is skipped
  const TensorDesc d = c.desc[t];
  __shared__ float lds[4][kNF];
  __shared__ float red[4];
  float* out = c.sums2 + size_t(t) * kStatStride;
  float acc[kNF];
  chunk_partials(c, d, acc);
  float s[3] = {0.f, 0.f, 0.f};   // block_sr's sums, without the root
  for (int q = threadIdx.x; q < d.nrseg; q += kBlock) {
#pragma unroll
    for (int k = 0; k < 3; ++k) s[k] += c.rbar_part[(d.rseg0 + q) * 4 + k];
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const float v = block_sum(s[k], red);
    if (threadIdx.x == 0) out[kNF + k] = d.vec ? 0.f : v;
  }
  feature_wave_sums(acc, lds);
  if (threadIdx.x < kNF) {
    const int f = threadIdx.x;
    out[f] = (lds[0][f] + lds[1][f]) + (lds[2][f] + lds[3][f]);
  } else if (threadIdx.x == kNF + 3) {
    out[kNF + 3] = 0.f;
  }
}

}  // namespace lopt
