// The apply pass of the optimizer step (the PyLO page's kernel 2, "CUDA
// kernel design: two-pass fusion" > "Fused kernel strategy": features rebuilt
// in registers, normalised, MLP evaluated inline, parameter written), one
// chunk per workgroup, on each MLP path.  lopt_apply.hip launches it as a
// kernel per path; lopt_single.hip runs it after the streaming passes in one
// launch.
//
// Translation units that include this file are compiled with -fno-honor-nans:
// the ReLUs then map to one v_max_f32 each instead of a quieting v_max
// followed by the max.  Non-finite inputs are not checked by the library (they
// propagate into the accumulators; a NaN pre-activation leaves the ReLU as 0
// either way).
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "lopt_device.h"

namespace lopt {

// ---------------------------------------------------------------------------
// k_apply_valu: the page's kernel 2 with the MLP on the vector ALU.  Weights
// are read through uniform (scalar) loads from the packed copy, so every FMA
// takes its weight from a scalar register.
template <bool VEC, bool NORMAL, int NF>
__device__ __forceinline__ void apply_valu_body(const StepCtx& c, const StepParams& hp, const Chunk& ch,
                                                const TensorDesc& d, const float* g) {
  const Streams s = make_streams(d, g, c.ws, ch);
  const float* __restrict__ pk = c.packed;
  const float* __restrict__ sc = c.scales + size_t(ch.tensor) * kStatStride;
  float decay, lr_step;
  update_constants(c, hp, ch, decay, lr_step);
  for (uint32_t e = ch.e0 + threadIdx.x; e < ch.e1; e += kBlock) {
    Elem x;
    load_elem<VEC>(s, e, x);
    const float p_old = x.p;
    float F[kNF], cn[3];
    build_features<VEC, NORMAL, NF>(hp, x, F, cn);
    store_state<VEC>(s, e, x, cn);
#pragma unroll
    for (int f = 0; f < NF; ++f) F[f] *= sc[f];
    float h1[kH];
#pragma unroll
    for (int o = 0; o < kH; ++o) {
      float a = pk[kPkB1 + o];
#pragma unroll
      for (int f = 0; f < NF; ++f) a = fmaf(pk[kPkW1 + o * kNF + f], F[f], a);
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
    store_param(s, e, fmaf(-lr_step, dir * __builtin_amdgcn_exp2f(mag * hp.exp2_mult), p_old * decay));
  }
}

__device__ __forceinline__ void apply_valu_block(const StepCtx& c, const StepParams& hp, uint32_t bid) {
  Chunk ch;
  TensorDesc d;
  const float* g;
  load_chunk(c, bid, ch, d, g);
  if (!g) return;  // no gradient this step: the tensor is skipped
  dispatch_variant<false>(d, hp, [&](auto v) {
    using V = decltype(v);
    apply_valu_body<V::vec, V::normal, V::nf>(c, hp, ch, d, g);
  });
}

// ---------------------------------------------------------------------------
// k_apply_mfma: the page's kernel 2 with layers 1 and 2 of the MLP on the fp32
// matrix cores.  A wave owns 64 elements per iteration, one per lane, for all
// per-element work (loads, features, update, stores).  The hidden units are M
// (weights = A operand, register resident), the elements N, the inputs K:
//   layer 1: v_mfma_f32_32x32x1_2b_f32, one instruction per feature (28, or
//     19 for the 19-feature variant; two fewer with the row-term slot below).
//     Its two blocks take their A and B operands from the two lane halves, so
//     block b multiplies W1's column (held by both halves) with the feature of
//     elements 32b..32b+31, each lane feeding its own element: no lane
//     movement.  Block b's 32x32 result lands in accumulator registers
//     16b..16b+15 in the usual 32x32 layout.
//   layer 2: v_mfma_f32_32x32x2_f32, one chain per block.  Layer-1 register r
//     of a lane holds hidden unit 8(r/4) + 4(lane/32) + r%4 of element
//     lane%32 (+32 for the second block), which is exactly a K-step B operand
//     if W2's columns are visited in that order (no data movement).
//   layer 3 (32 -> 2) on the vector ALU: per-lane partial dot products over
//     the lane's 16 hidden units, completed with one lane swap per output.
// b1 rides in the row-term slot where there is one (the layer-1 chain then
// starts from zero); otherwise, and for b2, a bias is the C operand of the
// first MFMA of its chain.  Biases and W3 are read from LDS each iteration,
// which keeps the kernel within 128 VGPRs; the feature scales s_d are folded
// into W1's columns once per chunk.
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x32 __attribute__((ext_vector_type(32)));

__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

__device__ __forceinline__ void swap_halves(float x, float y, float& lo, float& hi) {
  // lo = [x lanes 0..31 | y lanes 0..31], hi = [x lanes 32..63 | y lanes 32..63]
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// Layer-1 slots, one per instruction.  Normally slot s holds feature s.
// With RU (a 1-D tensor, or a wave iteration inside one row) the row features
// F13..F15 are constant over the iteration: their weighted sum, the row term,
// plus b1 becomes the A operand of slot 0 (whose B value is 1), and slots 1,
// 2, ... hold the other features in order.  -1: the constant slot.
__device__ constexpr int slot_feature(int s, bool ru) {
  return !ru ? s : s == 0 ? -1 : (s - 1 < 13 ? s - 1 : s + 2);
}

template <bool VEC, bool NORMAL, int NF, bool RU>
__device__ __forceinline__ void apply_mfma_body(const StepCtx& c, const StepParams& hp, const Chunk& ch,
                                                const TensorDesc& d, const float* g) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform loop control
  const int half = lane >> 5;
  const int row = lane & 31;
  const Streams s = make_streams(d, g, c.ws, ch);
  const float* __restrict__ pk = c.packed;
  const float* __restrict__ sc = c.scales + size_t(ch.tensor) * kStatStride;

  constexpr int NS = RU ? NF - 2 : NF;  // layer-1 slots (RU: NF - 3 features + the constant)
  float a1[NS];        // W1[row][f] * s_f for the feature f of slot j (the constant slot: unused)
  float a2[kH / 2];    // W2[row][acc_row(s, half)]
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int f = slot_feature(j, RU);
    a1[j] = f >= 0 ? pk[kPkW1 + row * kNF + f] * sc[f] : 0.f;
  }
  float arow[3];       // RU: W1[row][13 + k] * s_(13 + k), the row term's weights
#pragma unroll
  for (int k = 0; k < 3; ++k) arow[k] = RU ? pk[kPkW1 + row * kNF + 13 + k] * sc[13 + k] : 0.f;
  const float b1row = RU ? pk[kPkB1 + row] : 0.f;  // RU: b1 rides in the row-term slot
#pragma unroll
  for (int q = 0; q < 16; ++q) a2[q] = pk[kPkW2 + row * kH + acc_row(q, half)];

  // Biases and W3 in accumulator-row order per lane half; read with
  // ds_read_b128 when needed instead of holding 64 registers.  b1 is stored
  // twice so that each layer-1 block loads its own copy (no register moves).
  __shared__ float4 tab[5][2][4];   // {b1, b2, W3 dir, W3 mag, b1} x half x 16 floats
  if (threadIdx.x < 160) {
    const int which = threadIdx.x >> 5, h = (threadIdx.x >> 4) & 1, q = threadIdx.x & 15;
    const int hr = acc_row(q, h);
    const float v = which == 0 || which == 4 ? pk[kPkB1 + hr] : which == 1 ? pk[kPkB2 + hr]
                    : which == 2 ? pk[kPkW3 + hr] : pk[kPkW3 + kH + hr];
    reinterpret_cast<float*>(&tab[which][h][0])[q] = v;
  }
  __syncthreads();
  const float b3d = pk[kPkB3], b3m = pk[kPkB3 + 1];
  float decay, lr_step;
  update_constants(c, hp, ch, decay, lr_step);
  uint32_t base = ch.e0 + wave * 64;
  if (base >= ch.e1) return;  // this wave has no elements in the chunk
  for (; base < ch.e1; base += kBlock) {
    const uint32_t e = base + lane;
    const bool valid = e < ch.e1;
    Elem x;
    // an invalid lane loads the wave's first element instead (inside the
    // chunk, and in the same row when the iteration lies in one row)
    load_elem<VEC, RU && !VEC>(s, valid ? e : base, x, base);
    const float p_decayed = x.p * decay;
    float F[kNF], cn[3];
    build_features<VEC, NORMAL, NF>(hp, x, F, cn);
    // the accumulators are final here: storing them now frees their registers
    // during the MLP
    if (valid) store_state<VEC>(s, e, x, cn);

    f32x32 acc;  // registers 0..15: elements 0..31, 16..31: elements 32..63
    float a_first = a1[0];
    if (RU) {
      // The constant slot (B = 1) adds its A value to every element's hidden
      // unit, as a bias does: it carries b1 plus the row term of hidden unit
      // `row` for this iteration's row (lane 0's element is always inside the
      // chunk), and the chain starts from zero.
      const float r0 = __int_as_float(uni(__float_as_int(x.rq[0])));
      const float r1 = __int_as_float(uni(__float_as_int(x.rq[1])));
      const float r2 = __int_as_float(uni(__float_as_int(x.rq[2])));
      a_first = fmaf(arow[2], r2, fmaf(arow[1], r1, fmaf(arow[0], r0, b1row)));
#pragma unroll
      for (int q = 0; q < 32; ++q) acc[q] = 0.f;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = tab[0][half][q], u = tab[4][half][q];
        acc[4 * q] = v.x; acc[4 * q + 1] = v.y; acc[4 * q + 2] = v.z; acc[4 * q + 3] = v.w;
        acc[16 + 4 * q] = u.x; acc[16 + 4 * q + 1] = u.y; acc[16 + 4 * q + 2] = u.z; acc[16 + 4 * q + 3] = u.w;
      }
    }
    // Higher issue priority while this wave runs its matrix-core chains: the
    // chains then issue back to back ahead of the other waves' vector work
    // (measured: 5 % fewer cycles than without).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int f = slot_feature(j, RU);
      acc = __builtin_amdgcn_mfma_f32_32x32x1f32(j == 0 ? a_first : a1[j], f < 0 ? 1.f : F[f], acc, 0, 0, 0);
    }
    f32x16 accA, accB;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      accA[q] = acc[q];
      accB[q] = acc[16 + q];
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      accA[q] = fmaxf(accA[q], 0.f);
      accB[q] = fmaxf(accB[q], 0.f);
    }
    f32x16 bias2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = tab[1][half][q];
      bias2[4 * q] = v.x; bias2[4 * q + 1] = v.y; bias2[4 * q + 2] = v.z; bias2[4 * q + 3] = v.w;
    }
    f32x16 acc2A = bias2, acc2B = bias2;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float aq = a2[q];
      acc2A = __builtin_amdgcn_mfma_f32_32x32x2f32(aq, accA[q], acc2A, 0, 0, 0);
      acc2B = __builtin_amdgcn_mfma_f32_32x32x2f32(aq, accB[q], acc2B, 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    // half 0's partial sums start at b3, so the sum of the two halves holds it once
    const float d_init = half ? 0.f : b3d, m_init = half ? 0.f : b3m;
    float dA = d_init, mA = m_init, dB = d_init, mB = m_init;
    float w3d[16], w3m[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = tab[2][half][q], u = tab[3][half][q];
      w3d[4 * q] = v.x; w3d[4 * q + 1] = v.y; w3d[4 * q + 2] = v.z; w3d[4 * q + 3] = v.w;
      w3m[4 * q] = u.x; w3m[4 * q + 1] = u.y; w3m[4 * q + 2] = u.z; w3m[4 * q + 3] = u.w;
    }
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
    const float dir = d0 + d1;
    const float mag = m0 + m1;
    if (valid) store_param(s, e, fmaf(-lr_step, dir * __builtin_amdgcn_exp2f(mag * hp.exp2_mult), p_decayed));
  }
}

__device__ __forceinline__ void apply_mfma_block(const StepCtx& c, const StepParams& hp, uint32_t bid) {
  Chunk ch;
  TensorDesc d;
  const float* g;
  load_chunk(c, bid, ch, d, g);
  if (!g) return;  // no gradient this step: the tensor is skipped
  dispatch_variant<true>(d, hp, [&](auto v) {
    using V = decltype(v);
    apply_mfma_body<V::vec, V::normal, V::nf, V::rowuni>(c, hp, ch, d, g);
  });
}

// ---------------------------------------------------------------------------
// k_apply_bf16x9 / k_apply_bf16x6: layers 1 and 2 on the bf16 matrix cores.
// Every fp32 operand x is split into three bf16 pieces, x = h + m + l
// exactly: h is x with its low 16 bits cleared, m the same of r = x - h
// (exact), and l = r - m, which has at most 8 significant bits (truncation
// split of the 24-bit significand into 8-bit parts; |m| < 2^-7 |x|,
// |l| < 2^-15 |x|).  Every piece product (8 x 8 significant bits) is exact
// in the fp32 accumulator, so
//   bf16x9: the nine piece products sum to a.b exactly; the dot product is
//     that of an fp32 GEMM with exact products and fp32 accumulation (the
//     piece-wise emulation of an fp32 GEMM on reduced-precision matrix units
//     known as bf16x9: Henry, Tang & Heinecke, 2019);
//   bf16x8: all but ll, which is below 2^-30 |a b|: each product within
//     1/64 of one fp32 rounding (2^-24 |a b|), accumulated in fp32;
//   bf16x6: the six products whose orders add up to at most 2 (hh, hm, mh,
//     hl, lh, mm); the three dropped ones (ml, lm, ll) stay below
//     2^-21 |a b|, with a median below one fp32 rounding (narrower than
//     fp32).
// (Rounding the pieces to nearest with v_cvt_pk_bf16_f32 bounds bf16x6's
// dropped products by 2^-23 at the same instruction count but measured 4.6 %
// slower.)  Products are issued smallest first.
// On gfx950 a v_mfma_f32_32x32x16_bf16 does 16x the FLOP of the fp32 form in
// half its cycles, and vector instructions of the other waves issue beside
// it (the fp32 form shares their issue cycles), so the six products cost
// less than one fp32 product and the split's vector work overlaps the matrix
// work.
//
// Layout (one wave, 64 elements, lane l owns element l; M = hidden unit
// l%32, K = inputs, N = elements, two 32-element blocks):
//   layer 1: 32 K entries in two K-steps of 16; entry q < NL holds the q-th
//     feature of the variant's list (RU: without the row features), the
//     entries of position (1, 7) in both lane halves hold half of the
//     constant term (b1, plus the row term with RU) against a B value of 1,
//     the rest are zero.  A K-step's B operand takes entries 0..7 from lane
//     half 0 and 8..15 from half 1 for the block's 32 elements, so each pair
//     of entries (one per half, same position) is exchanged between the lane
//     halves once in fp32 (v_permlane32_swap) before the split.
//   layer 2: the layer-1 accumulator register r of lane half h holds hidden
//     unit 8(r/4) + 4h + r%4, which is a B operand entry as it stands (W2's
//     columns are visited in that order, as in the fp32 matrix path).
//   layer 3 on the vector ALU, as in the fp32 matrix path.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The values whose upper halves are the pieces h, m, l of x.
struct Pieces {
  float h, m, l;
};
__device__ __forceinline__ Pieces split3(float x) {
  const float r = x - __uint_as_float(__float_as_uint(x) & 0xffff0000u);
  return {x, r, r - __uint_as_float(__float_as_uint(r) & 0xffff0000u)};
}
__device__ __forceinline__ float piece(const Pieces& p, int k) { return k == 0 ? p.h : k == 1 ? p.m : p.l; }
// bf16 pair: the upper half of a (low) and of b (high).
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight values x[0..7] (the four bf16 pairs of one B operand) to their three
// pieces, as bf16 pairs.  (Taking the remainders x - h and r - m with
// v_dot2c_f32_bf16 against the pair (-1, 0) gives the same pieces bit for bit
// in 7 instead of 11 instructions per pair, but measured 21 % more cycles per
// element: that instruction does not issue beside the bf16 matrix
// instructions as the masks and subtractions do.)
__device__ __forceinline__ void split3_x8(const float (&x)[8], u32x4 (&bt)[3]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const Pieces u0 = split3(x[2 * j]), u1 = split3(x[2 * j + 1]);
#pragma unroll
    for (int p = 0; p < 3; ++p)   // a zero low value: the high value's upper half, the split's own mask
      bt[p][j] = (__builtin_constant_p(x[2 * j]) && x[2 * j] == 0.f) ? __float_as_uint(piece(u1, p)) & 0xffff0000u
                                                                     : pack2(piece(u0, p), piece(u1, p));
  }
}

// Layer-1 entries: feature of entry q (q < 30), -1 = zero.  Entry q sits at
// K-step (q/2)/8, position (q/2)%8, lane half q%2, so a lane's bf16 pair j
// holds entries 4j + h (low) and 4j + 2 + h (high) for lane half h.  The
// features fill the entries in order, except that a last group of one or two
// features moves up by two entries, into the high halves of its pairs: a pair
// whose low entry is zero packs its value's pieces with the masks the split
// already takes (split3_x8).
__device__ constexpr int x6_feature(int q, int nf, bool ru) {
  const int n = ru ? nf - 3 : nf;   // entries that carry a feature
  const int g = n & ~3, r = n & 3;
  if (r == 1 || r == 2) {
    if (q >= g && q < g + 2) return -1;
    if (q >= g + 2 && q < g + 2 + r)
      q -= 2;
    else if (q >= g + 2 + r)
      return -1;
  }
  for (int f = 0; f < nf; ++f) {
    if (ru && f >= 13 && f < 16) continue;
    if (q == 0) return f;
    --q;
  }
  return -1;
}
static_assert(x6_feature(23, kNF, true) == 26 && x6_feature(24, kNF, true) == -1 && x6_feature(25, kNF, true) == -1 &&
                  x6_feature(26, kNF, true) == 27 && x6_feature(27, kNF, true) == -1 &&
                  x6_feature(29, kNF, true) == -1 && x6_feature(27, kNF, false) == 27 &&
                  x6_feature(13, kNF, true) == 16 && x6_feature(16, kVeloNF, true) == -1 &&
                  x6_feature(18, kVeloNF, false) == 18 &&
                  // K-step 1, position 6 (entries 28, 29) is zero on every variant (apply_x6_body's kc1)
                  x6_feature(28, kNF, true) == -1 && x6_feature(29, kNF, false) == -1 &&
                  x6_feature(28, kVeloNF, true) == -1 && x6_feature(29, kVeloNF, false) == -1,
              "bf16x6 layer-1 entries");
// Every fed feature (all n_feat but the folded row features 13..15 with RU) in
// exactly one of the entries 0..29 (30 and 31 hold the constant term).
__device__ constexpr bool x6_layout_ok(int nf, bool ru) {
  for (int f = 0; f < nf; ++f) {
    int hits = 0;
    for (int q = 0; q < 30; ++q) hits += x6_feature(q, nf, ru) == f;
    if (hits != ((ru && f >= 13 && f < 16) ? 0 : 1)) return false;
  }
  for (int q = 0; q < 30; ++q)
    if (x6_feature(q, nf, ru) >= nf) return false;
  return true;
}
static_assert(x6_layout_ok(kNF, false) && x6_layout_ok(kNF, true) && x6_layout_ok(kVeloNF, false) &&
                  x6_layout_ok(kVeloNF, true),
              "bf16x6 layer-1 entries: each fed feature once");

// (A piece, B piece) of product t of NP (9, 8 or 6), smallest terms first:
// bf16x9: ll, then bf16x8's lm, ml, then bf16x6's hl, lh, mm, hm, mh, hh.
__device__ constexpr int xp_a(int np, int t) {
  constexpr int a9[9] = {2, 2, 1, 0, 2, 1, 0, 1, 0};
  return a9[t + 9 - np];
}
__device__ constexpr int xp_b(int np, int t) {
  constexpr int b9[9] = {2, 1, 2, 2, 0, 1, 1, 0, 0};
  return b9[t + 9 - np];
}
static_assert(xp_a(6, 0) == 0 && xp_b(6, 0) == 2 && xp_a(6, 1) == 2 && xp_b(6, 1) == 0 && xp_a(6, 2) == 1 &&
                  xp_b(6, 2) == 1 && xp_a(6, 5) == 0 && xp_b(6, 5) == 0 && xp_a(9, 0) == 2 && xp_b(9, 0) == 2 &&
                  xp_a(8, 0) == 2 && xp_b(8, 0) == 1 && xp_a(8, 1) == 1 && xp_b(8, 1) == 2 && xp_a(8, 7) == 0,
              "piece-product order");

// LDS of the kernel (one copy for every variant the body is instantiated for).
struct X6Lds {
  u32x4 a1[2][3][64];   // layer-1 A operands: K-step, piece, lane
  u32x4 a2[2][3][64];   // layer-2 A operands
  float4 tab[3][2][4];  // {b2, W3 dir, W3 mag} x half x 16 floats
};

template <int NP, bool VEC, bool NORMAL, int NF, bool RU, bool KREG>
__device__ __forceinline__ void apply_x6_body(const StepCtx& c, const StepParams& hp, const Chunk& ch,
                                              const TensorDesc& d, const float* g, X6Lds& L) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int row = lane & 31;
  const Streams s = make_streams(d, g, c.ws, ch);
  const float* __restrict__ pk = c.packed;
  const float* __restrict__ sc = c.scales + size_t(ch.tensor) * kStatStride;

  // A operands, built once per chunk by the first wave and read from LDS
  // (16 bytes per lane per K-step and piece) where needed.  Layer 1: K-step
  // k, piece p: entries of positions 0..7 of the lane's half.  The constant
  // entries (1, 7) are set per iteration with RU; otherwise they hold b1 / 2
  // (two entries, one per half, against B = 1).  Layer 2: W2's columns in
  // accumulator-row order.
  if (threadIdx.x < 64) {
    const float b1half = 0.5f * pk[kPkB1 + row];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = 2 * (8 * k + i);
        const int f0 = x6_feature(q, NF, RU), f1 = x6_feature(q + 1, NF, RU);
        const float w0 = f0 >= 0 ? pk[kPkW1 + row * kNF + f0] * sc[f0] : 0.f;
        const float w1 = f1 >= 0 ? pk[kPkW1 + row * kNF + f1] * sc[f1] : 0.f;
        v[i] = (k == 1 && i == 7) ? (RU ? 0.f : b1half) : half ? w1 : w0;
      }
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        u32x4 t;
#pragma unroll
        for (int j = 0; j < 4; ++j) t[j] = pack2(piece(split3(v[2 * j]), p), piece(split3(v[2 * j + 1]), p));
        L.a1[k][p][lane] = t;
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        u32x4 t;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float w0 = pk[kPkW2 + row * kH + acc_row(8 * k + 2 * j, half)];
          const float w1 = pk[kPkW2 + row * kH + acc_row(8 * k + 2 * j + 1, half)];
          t[j] = pack2(piece(split3(w0), p), piece(split3(w1), p));
        }
        L.a2[k][p][lane] = t;
      }
  }
  float arow[3];       // RU: W1[row][13 + k] * s_(13 + k), the row term's weights
#pragma unroll
  for (int k = 0; k < 3; ++k) arow[k] = RU ? pk[kPkW1 + row * kNF + 13 + k] * sc[13 + k] : 0.f;
  const float b1row = RU ? pk[kPkB1 + row] : 0.f;

  if (threadIdx.x < 96) {
    const int which = threadIdx.x >> 5, h = (threadIdx.x >> 4) & 1, q = threadIdx.x & 15;
    const int hr = acc_row(q, h);
    const float v = which == 0 ? pk[kPkB2 + hr] : which == 1 ? pk[kPkW3 + hr] : pk[kPkW3 + kH + hr];
    reinterpret_cast<float*>(&L.tab[which][h][0])[q] = v;
  }
  __syncthreads();
  const float b3d = pk[kPkB3], b3m = pk[kPkB3 + 1];
  float decay, lr_step;
  update_constants(c, hp, ch, decay, lr_step);
  uint32_t base = ch.e0 + wave * 64;
  if (base >= ch.e1) return;
  // K-step 1's last pair (positions 6 and 7) is always (0, 1): pieces
  // (1.0's upper half in the high half, 0, 0).  KREG holds it in a register
  // the compiler cannot see through: as a constant, each B operand holding it
  // was built by copying a four-register constant and overwriting three of
  // them (10 vector instructions per 64 elements).  The one-launch kernel,
  // whose other passes share the register budget, keeps the constant.
  uint32_t kc1[3] = {0x3f800000u, 0u, 0u};
  if constexpr (KREG) asm volatile("" : "+v"(kc1[0]));
  for (; base < ch.e1; base += kBlock) {
    const uint32_t e = base + lane;
    const bool valid = e < ch.e1;
    Elem x;
    load_elem<VEC, RU && !VEC>(s, valid ? e : base, x, base);
    const float p_decayed = x.p * decay;
    float F[kNF], cn[3];
    build_features<VEC, NORMAL, NF>(hp, x, F, cn);
    if (valid) store_state<VEC>(s, e, x, cn);

    Pieces ct = {0.f, 0.f, 0.f};
    if (RU) {
      // constant entries: (b1 + row term) / 2 in both lane halves
      const float r0 = __int_as_float(uni(__float_as_int(x.rq[0])));
      const float r1 = __int_as_float(uni(__float_as_int(x.rq[1])));
      const float r2 = __int_as_float(uni(__float_as_int(x.rq[2])));
      ct = split3(0.5f * fmaf(arow[2], r2, fmaf(arow[1], r1, fmaf(arow[0], r0, b1row))));
    }
    // The A operands are read from LDS where they are used: an offset the
    // compiler cannot see through keeps the reads in the loop (hoisted, the
    // 48 registers they need would be spilled to scratch).
    int li = lane;
    asm volatile("" : "+v"(li));
    // Layer-1 B values: entry pairs exchanged between the lane halves, so
    // that v[b][k][i] holds position i of K-step k for block b's element.
    float v[2][2][8];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = 2 * (8 * k + i);
        const int f0 = x6_feature(q, NF, RU), f1 = x6_feature(q + 1, NF, RU);
        if (k == 1 && i == 7) {
          v[0][k][i] = v[1][k][i] = 1.f;
        } else if (f0 < 0 && f1 < 0) {
          v[0][k][i] = v[1][k][i] = 0.f;
        } else {
          swap_halves(f0 >= 0 ? F[f0] : 0.f, f1 >= 0 ? F[f1] : 0.f, v[0][k][i], v[1][k][i]);
        }
      }
    f32x16 acc1s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc1s[b][q] = 0.f;
    // Raised issue priority over the MLP: this wave's matrix instructions
    // (and the splits that feed them) go ahead of other waves' feature work
    // (measured: apply 1.2 % faster on ViT-B/16).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      u32x4 a[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        a[p] = L.a1[k][p][li];
        if (RU && k == 1) a[p][3] = __builtin_amdgcn_perm(__float_as_uint(piece(ct, p)), a[p][3], 0x07060100u);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        u32x4 bt[3];
        split3_x8(v[b][k], bt);
        if (k == 1) {
#pragma unroll
          for (int p = 0; p < 3; ++p) bt[p][3] = kc1[p];
        }
#pragma unroll
        for (int t = 0; t < NP; ++t)
          acc1s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[xp_a(NP, t)]), as_bf16x8(bt[xp_b(NP, t)]),
                                                             acc1s[b], 0, 0, 0);
      }
    }
    float dpart[2], mpart[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const f32x16 acc1 = acc1s[b];
      f32x16 acc2;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 w = L.tab[0][half][q];
        acc2[4 * q] = w.x; acc2[4 * q + 1] = w.y; acc2[4 * q + 2] = w.z; acc2[4 * q + 3] = w.w;
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        u32x4 a[3], bt[3];
#pragma unroll
        for (int p = 0; p < 3; ++p) a[p] = L.a2[k][p][li];
        float hx[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) hx[i] = fmaxf(acc1[8 * k + i], 0.f);
        split3_x8(hx, bt);
#pragma unroll
        for (int t = 0; t < NP; ++t)
          acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[xp_a(NP, t)]), as_bf16x8(bt[xp_b(NP, t)]), acc2, 0,
                                                         0, 0);
      }
      float dsum = half ? 0.f : b3d, msum = half ? 0.f : b3m;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 wd = L.tab[1][half][q], wm = L.tab[2][half][q];
        const float hq[4] = {fmaxf(acc2[4 * q], 0.f), fmaxf(acc2[4 * q + 1], 0.f), fmaxf(acc2[4 * q + 2], 0.f),
                             fmaxf(acc2[4 * q + 3], 0.f)};
        dsum = fmaf(wd.x, hq[0], dsum); msum = fmaf(wm.x, hq[0], msum);
        dsum = fmaf(wd.y, hq[1], dsum); msum = fmaf(wm.y, hq[1], msum);
        dsum = fmaf(wd.z, hq[2], dsum); msum = fmaf(wm.z, hq[2], msum);
        dsum = fmaf(wd.w, hq[3], dsum); msum = fmaf(wm.w, hq[3], msum);
      }
      dpart[b] = dsum;
      mpart[b] = msum;
    }
    __builtin_amdgcn_s_setprio(0);
    const float dA = dpart[0], dB = dpart[1], mA = mpart[0], mB = mpart[1];
    float d0, d1, m0, m1;
    swap_halves(dA, dB, d0, d1);
    swap_halves(mA, mB, m0, m1);
    const float dir = d0 + d1;
    const float mag = m0 + m1;
    if (valid) store_param(s, e, fmaf(-lr_step, dir * __builtin_amdgcn_exp2f(mag * hp.exp2_mult), p_decayed));
  }
}

template <int NP, bool KREG>
__device__ __forceinline__ void apply_bf16_block(const StepCtx& c, const StepParams& hp, uint32_t bid) {
  Chunk ch;
  TensorDesc d;
  const float* g;
  load_chunk(c, bid, ch, d, g);
  if (!g) return;  // no gradient this step: the tensor is skipped
  __shared__ X6Lds lds;
  dispatch_variant<true>(d, hp, [&](auto v) {
    using V = decltype(v);
    apply_x6_body<NP, V::vec, V::normal, V::nf, V::rowuni, KREG>(c, hp, ch, d, g, lds);
  });
}


// ---------------------------------------------------------------------------
// k_apply_fp16x3: the same layout on the fp16 matrix cores
// (v_mfma_f32_32x32x16_f16) with two pieces and three products.  An operand x
// is split as h = fp16(x) (nearest) and l = fp16(x - h), 22 significant bits;
// a.b is taken as hh + hl + lh (the dropped ll is below 2^-22 |a b|).  fp16's
// range is the constraint, so the features are normalised on the vector ALU
// first (x = F s, with |x| <= sqrt(n) < 46341 for every element), and the
// rest is rescaled by powers of two, all exact in fp32:
//   * W1 and W2 enter the A operands times 2^a1 and 2^a2 (x3_w1, x3_w2), which
//     put each matrix's largest weight in [4, 8) and keep the low pieces of the
//     small weights out of fp16's subnormal range; as ReLU commutes with the
//     factor, layer 2 starts from b2 2^(a1 + a2) and layer 3 reads
//     W3 2^-(a1 + a2);
//   * the constant entries (b1 plus the row term) carry value * 2^(a1 - k)
//     against a B value of 2^k, k = x3_shift from a bound on the weights;
//   * a wave whose layer-2 inputs (layer-1 outputs) reach 2^15 scales them by
//     2^-j, starts layer 2 from b2 2^(a1 + a2 - j), and multiplies its layer-3
//     sums by 2^j (a ballot over the lanes; the scaling runs only there).
// A normalised feature or hidden value far below 1 keeps fp16's absolute
// floor (2^-25 for its low piece), small beside the sum it enters.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// The two fp16 pieces of x0 and x1 as fp16 pairs: h, l (index 0, 1).
struct Pieces2h {
  uint32_t p[2];
};
__device__ __forceinline__ Pieces2h split2x2(float x0, float x1) {
  Pieces2h s;
  const f16x2 h = __builtin_convertvector(f32x2{x0, x1}, f16x2);
  s.p[0] = __builtin_bit_cast(uint32_t, h);
  const float r0 = x0 - (float)h.x, r1 = x1 - (float)h.y;
  s.p[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, f16x2));
  return s;
}
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
// (A piece, B piece) of product t of the three, smallest first: hl, lh, hh.
__device__ constexpr int x3_a(int t) { return t == 1 ? 1 : 0; }
__device__ constexpr int x3_b(int t) { return t == 0 ? 1 : 0; }

template <bool VEC, bool NORMAL, int NF, bool RU>
__device__ __forceinline__ void apply_x3_body(const StepCtx& c, const StepParams& hp, const Chunk& ch,
                                              const TensorDesc& d, const float* g, X6Lds& L) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int row = lane & 31;
  const Streams s = make_streams(d, g, c.ws, ch);
  const float* __restrict__ pk = c.packed;
  const float* __restrict__ sc = c.scales + size_t(ch.tensor) * kStatStride;
  const float cscale = __builtin_ldexpf(1.0f, hp.x3_w1 - hp.x3_shift);  // exact powers of two
  const float bconst = __builtin_ldexpf(1.0f, hp.x3_shift);

  // A operands (two pieces), built once per chunk by the first wave: layer 1
  // from W1 2^a1 (the features carry their scales), its constant entries
  // (1, 7) as for k_apply_bf16x6 but times 2^(a1 - k); layer 2 from W2 2^a2.
  if (threadIdx.x < 64) {
    const float b1half = 0.5f * pk[kPkB1 + row] * cscale;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = 2 * (8 * k + i);
        const int f0 = x6_feature(q, NF, RU), f1 = x6_feature(q + 1, NF, RU);
        const float w0 = f0 >= 0 ? __builtin_ldexpf(pk[kPkW1 + row * kNF + f0], hp.x3_w1) : 0.f;
        const float w1 = f1 >= 0 ? __builtin_ldexpf(pk[kPkW1 + row * kNF + f1], hp.x3_w1) : 0.f;
        v[i] = (k == 1 && i == 7) ? (RU ? 0.f : b1half) : half ? w1 : w0;
      }
      Pieces2h pc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pc[j] = split2x2(v[2 * j], v[2 * j + 1]);
#pragma unroll
      for (int p = 0; p < 2; ++p) L.a1[k][p][lane] = u32x4{pc[0].p[p], pc[1].p[p], pc[2].p[p], pc[3].p[p]};
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      Pieces2h pc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pc[j] = split2x2(__builtin_ldexpf(pk[kPkW2 + row * kH + acc_row(8 * k + 2 * j, half)], hp.x3_w2),
                         __builtin_ldexpf(pk[kPkW2 + row * kH + acc_row(8 * k + 2 * j + 1, half)], hp.x3_w2));
#pragma unroll
      for (int p = 0; p < 2; ++p) L.a2[k][p][lane] = u32x4{pc[0].p[p], pc[1].p[p], pc[2].p[p], pc[3].p[p]};
    }
  }
  float arow[3];       // RU: W1[row][13 + k] * s_(13 + k), the row term's weights
#pragma unroll
  for (int k = 0; k < 3; ++k) arow[k] = RU ? pk[kPkW1 + row * kNF + 13 + k] * sc[13 + k] : 0.f;
  const float b1row = RU ? pk[kPkB1 + row] : 0.f;
  float scl[kNF];      // the tensor's feature scales (wave-uniform)
#pragma unroll
  for (int f = 0; f < kNF; ++f) scl[f] = f < NF ? __int_as_float(uni(__float_as_int(sc[f]))) : 0.f;

  if (threadIdx.x < 96) {
    const int which = threadIdx.x >> 5, h = (threadIdx.x >> 4) & 1, q = threadIdx.x & 15;
    const int hr = acc_row(q, h);
    // b2 2^(a1 + a2) and W3 2^-(a1 + a2): layer 2's output carries 2^(a1 + a2)
    const int a12 = hp.x3_w1 + hp.x3_w2;
    const float v = which == 0 ? __builtin_ldexpf(pk[kPkB2 + hr], a12)
                    : __builtin_ldexpf(which == 1 ? pk[kPkW3 + hr] : pk[kPkW3 + kH + hr], -a12);
    reinterpret_cast<float*>(&L.tab[which][h][0])[q] = v;
  }
  __syncthreads();
  const float b3d = pk[kPkB3], b3m = pk[kPkB3 + 1];
  float decay, lr_step;
  update_constants(c, hp, ch, decay, lr_step);
  uint32_t base = ch.e0 + wave * 64;
  if (base >= ch.e1) return;
  for (; base < ch.e1; base += kBlock) {
    const uint32_t e = base + lane;
    const bool valid = e < ch.e1;
    Elem x;
    load_elem<VEC, RU && !VEC>(s, valid ? e : base, x, base);
    const float p_decayed = x.p * decay;
    float F[kNF], cn[3];
    build_features<VEC, NORMAL, NF>(hp, x, F, cn);
    if (valid) store_state<VEC>(s, e, x, cn);

    Pieces2h ct = {{0u, 0u}};
    if (RU) {
      // constant entries: (b1 + row term) / 2 * 2^-k in both lane halves
      const float r0 = __int_as_float(uni(__float_as_int(x.rq[0])));
      const float r1 = __int_as_float(uni(__float_as_int(x.rq[1])));
      const float r2 = __int_as_float(uni(__float_as_int(x.rq[2])));
      const float cv = 0.5f * cscale * fmaf(arow[2], r2, fmaf(arow[1], r1, fmaf(arow[0], r0, b1row)));
      ct = split2x2(cv, cv);  // the upper halves are used
    }
    int li = lane;
    asm volatile("" : "+v"(li));
    // normalised layer-1 B values, exchanged between the lane halves
    float v[2][2][8];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = 2 * (8 * k + i);
        const int f0 = x6_feature(q, NF, RU), f1 = x6_feature(q + 1, NF, RU);
        if (k == 1 && i == 7) {
          v[0][k][i] = v[1][k][i] = bconst;
        } else if (f0 < 0 && f1 < 0) {
          v[0][k][i] = v[1][k][i] = 0.f;
        } else {
          swap_halves(f0 >= 0 ? F[f0] * scl[f0] : 0.f, f1 >= 0 ? F[f1] * scl[f1] : 0.f, v[0][k][i], v[1][k][i]);
        }
      }
    f32x16 acc1s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc1s[b][q] = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      u32x4 a[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        a[p] = L.a1[k][p][li];
        if (RU && k == 1) a[p][3] = __builtin_amdgcn_perm(ct.p[p], a[p][3], 0x07060100u);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        u32x4 bt[2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const Pieces2h u = split2x2(v[b][k][2 * j], v[b][k][2 * j + 1]);
          bt[0][j] = u.p[0];
          bt[1][j] = u.p[1];
        }
#pragma unroll
        for (int t = 0; t < 3; ++t)
          acc1s[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(a[x3_a(t)]), as_f16x8(bt[x3_b(t)]), acc1s[b], 0, 0, 0);
      }
    }
    // ReLU in place, and the range guard of the layer-2 inputs
    float top = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        acc1s[b][q] = fmaxf(acc1s[b][q], 0.f);
        top = fmaxf(top, acc1s[b][q]);
      }
    // Layers 2 and 3 for both blocks; SCALED: the wave's layer-2 inputs are
    // multiplied by s2 = 2^-j (b2 and b3 too) and the layer-3 sums by 2^j.
    float dpart[2], mpart[2];
    auto layers23 = [&](auto scaled_tag, float s2, float s2inv) {
      constexpr bool SCALED = decltype(scaled_tag)::value;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        f32x16 acc2;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 w = L.tab[0][half][q];
          acc2[4 * q] = w.x; acc2[4 * q + 1] = w.y; acc2[4 * q + 2] = w.z; acc2[4 * q + 3] = w.w;
        }
        if (SCALED) {
#pragma unroll
          for (int q = 0; q < 16; ++q) acc2[q] *= s2;
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          u32x4 a[2], bt[2];
#pragma unroll
          for (int p = 0; p < 2; ++p) a[p] = L.a2[k][p][li];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float x0 = acc1s[b][8 * k + 2 * j], x1 = acc1s[b][8 * k + 2 * j + 1];
            if (SCALED) {
              x0 *= s2;
              x1 *= s2;
            }
            const Pieces2h u = split2x2(x0, x1);
            bt[0][j] = u.p[0];
            bt[1][j] = u.p[1];
          }
#pragma unroll
          for (int t = 0; t < 3; ++t)
            acc2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(a[x3_a(t)]), as_f16x8(bt[x3_b(t)]), acc2, 0, 0, 0);
        }
        // half 0's partial sums start at b3, so the sum of the two halves holds it once
        float dsum = half ? 0.f : b3d, msum = half ? 0.f : b3m;
        if (SCALED) {
          dsum *= s2;
          msum *= s2;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 wd = L.tab[1][half][q], wm = L.tab[2][half][q];
          const float hq[4] = {fmaxf(acc2[4 * q], 0.f), fmaxf(acc2[4 * q + 1], 0.f), fmaxf(acc2[4 * q + 2], 0.f),
                               fmaxf(acc2[4 * q + 3], 0.f)};
          dsum = fmaf(wd.x, hq[0], dsum); msum = fmaf(wm.x, hq[0], msum);
          dsum = fmaf(wd.y, hq[1], dsum); msum = fmaf(wm.y, hq[1], msum);
          dsum = fmaf(wd.z, hq[2], dsum); msum = fmaf(wm.z, hq[2], msum);
          dsum = fmaf(wd.w, hq[3], dsum); msum = fmaf(wm.w, hq[3], msum);
        }
        if (SCALED) {
          dsum *= s2inv;
          msum *= s2inv;
        }
        dpart[b] = dsum;
        mpart[b] = msum;
      }
    };
    if (__builtin_amdgcn_ballot_w64(!(top < 32768.f)) == 0) {
      layers23(std::false_type{}, 1.f, 1.f);
    } else {
      // rare: scale the wave by 2^-j so that its largest input is below 2^15
      float m = top;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      int ex;
      (void)__builtin_frexpf(m, &ex);  // m < 2^ex
      const int j = ex > 15 ? ex - 15 : 1;
      layers23(std::true_type{}, __builtin_ldexpf(1.0f, -j), __builtin_ldexpf(1.0f, j));
    }
    float d0, d1, m0, m1;
    swap_halves(dpart[0], dpart[1], d0, d1);
    swap_halves(mpart[0], mpart[1], m0, m1);
    const float dir = d0 + d1;
    const float mag = m0 + m1;
    if (valid) store_param(s, e, fmaf(-lr_step, dir * __builtin_amdgcn_exp2f(mag * hp.exp2_mult), p_decayed));
  }
}

__device__ __forceinline__ void apply_fp16x3_block(const StepCtx& c, const StepParams& hp, uint32_t bid) {
  Chunk ch;
  TensorDesc d;
  const float* g;
  load_chunk(c, bid, ch, d, g);
  if (!g) return;  // no gradient this step: the tensor is skipped
  __shared__ X6Lds lds;
  dispatch_variant<true>(d, hp, [&](auto v) {
    using V = decltype(v);
    apply_x3_body<V::vec, V::normal, V::nf, V::rowuni>(c, hp, ch, d, g, lds);
  });
}


// ---------------------------------------------------------------------------
// One chunk of the apply pass on MLP path IMPL (lopt_mlp_impl numbering:
// 1 VALU, 2 fp32 matrix cores, 3 bf16x6, 4 fp16x3, 5 bf16x9, 6 bf16x8).
// KREG: see apply_x6_body (false in the one-launch kernel).
template <int IMPL, bool KREG = true>
__device__ __forceinline__ void apply_block(const StepCtx& c, const StepParams& hp, uint32_t bid) {
  if constexpr (IMPL == 1) apply_valu_block(c, hp, bid);
  else if constexpr (IMPL == 2) apply_mfma_block(c, hp, bid);
  else if constexpr (IMPL == 3) apply_bf16_block<6, KREG>(c, hp, bid);
  else if constexpr (IMPL == 4) apply_fp16x3_block(c, hp, bid);
  else if constexpr (IMPL == 5) apply_bf16_block<9, KREG>(c, hp, bid);
  else apply_bf16_block<8, KREG>(c, hp, bid);
}

}  // namespace lopt
