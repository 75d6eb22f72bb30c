// Measured machine figures behind the roofline of the optimizer step:
//   1. streaming read bandwidth of HBM (the bound of the statistics pass),
//      with plain and with non-temporal loads;
//   2. sustained fp32 matrix throughput (v_mfma_f32_32x32x2_f32) for 1, 2 and
//      4 waves per SIMD and 1, 2 or 4 independent accumulator chains per wave
//      (the apply kernel runs 4 waves with 2 chains each);
//   3. what one vector instruction of a given kind adds to a stream of
//      matrix instructions (4 waves x 2 chains): on gfx950 the fp32 matrix
//      instructions and the vector ALU share the SIMD's issue, so vector work
//      adds to the matrix time instead of hiding under it;
//   4. the same two figures for the bf16 matrix instruction
//      v_mfma_f32_32x32x16_bf16 (the bf16x8, bf16x9 and bf16x6 apply paths),
//      beside which vector instructions of the other waves do issue, and the
//      time of 4 of them with 16, 32, 48 or 64 independent v_fma_f32 beside
//      them (the apply kernels issue about one vector cycle per matrix
//      cycle): how much vector work the matrix instructions hide;
//   5. the throughput of the fp16 matrix instruction v_mfma_f32_32x32x16_f16
//      (the fp16x3 apply path).
// Prints one JSON object.  Every kernel writes only out[block * 64 + lane],
// and out is sized for the largest grid launched.
#include <hip/hip_runtime.h>

#include <cstdio>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void read_stream(const float4* __restrict__ a, size_t n4, float* __restrict__ out) {
  float acc = 0.f;
  size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  const size_t stride = size_t(gridDim.x) * 256;
  for (; i + 3 * stride < n4; i += 4 * stride) {
    const float4 x0 = a[i], x1 = a[i + stride], x2 = a[i + 2 * stride], x3 = a[i + 3 * stride];
    acc += ((x0.x + x0.y) + (x0.z + x0.w)) + ((x1.x + x1.y) + (x1.z + x1.w)) +
           ((x2.x + x2.y) + (x2.z + x2.w)) + ((x3.x + x3.y) + (x3.z + x3.w));
  }
  for (; i < n4; i += stride) acc += (a[i].x + a[i].y) + (a[i].z + a[i].w);
  out[size_t(blockIdx.x) * 256 + threadIdx.x] = acc;
}

// The same read with the non-temporal hint (how the optimizer's kernels read
// their per-element streams).
__global__ __launch_bounds__(256) void read_stream_nt(const f32x4* __restrict__ a, size_t n4, float* __restrict__ out) {
  float acc = 0.f;
  size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  const size_t stride = size_t(gridDim.x) * 256;
  for (; i + 3 * stride < n4; i += 4 * stride) {
    const f32x4 x0 = __builtin_nontemporal_load(a + i), x1 = __builtin_nontemporal_load(a + i + stride);
    const f32x4 x2 = __builtin_nontemporal_load(a + i + 2 * stride), x3 = __builtin_nontemporal_load(a + i + 3 * stride);
    acc += ((x0.x + x0.y) + (x0.z + x0.w)) + ((x1.x + x1.y) + (x1.z + x1.w)) +
           ((x2.x + x2.y) + (x2.z + x2.w)) + ((x3.x + x3.y) + (x3.z + x3.w));
  }
  for (; i < n4; i += stride) {
    const f32x4 x = __builtin_nontemporal_load(a + i);
    acc += (x.x + x.y) + (x.z + x.w);
  }
  out[size_t(blockIdx.x) * 256 + threadIdx.x] = acc;
}

// 16 matrix instructions per iteration over NACC independent accumulators.
template <int NACC>
__global__ __launch_bounds__(64) void mfma_chains(float* out, int iters, float s) {
  f32x16 a[NACC];
#pragma unroll
  for (int k = 0; k < NACC; ++k) a[k] = f32x16{0};
  const float x = s * threadIdx.x, y = s + threadIdx.x;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 16 / NACC; ++r)
#pragma unroll
      for (int k = 0; k < NACC; ++k) a[k] = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, a[k], 0, 0, 0);
  }
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < NACC; ++k)
    for (int i = 0; i < 16; ++i) acc += a[k][i];
  out[size_t(blockIdx.x) * 64 + threadIdx.x] = acc;
}

// 4 matrix instructions (2 chains) plus 16 independent vector instructions of
// one kind per iteration.  OP 0: none, 1: v_fma_f32, 2: v_max_f32 (ReLU form),
// 3: v_permlane32_swap (8 instructions, each swapping a pair), 4: v_add_u32.
template <int OP>
__global__ __launch_bounds__(64) void mfma_plus(float* out, int iters, float s) {
  f32x16 a0 = {0}, a1 = {0};
  float v[16];
  unsigned u[16];
  for (int i = 0; i < 16; ++i) {
    v[i] = threadIdx.x * 0.001f + i;
    u[i] = threadIdx.x * 7u + i;
  }
  const float x = s * threadIdx.x, y = s + threadIdx.x;
  for (int it = 0; it < iters; ++it) {
    a0 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, a1, 0, 0, 0);
    a0 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, a1, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (OP == 1) v[i] = fmaf(v[i], s, x);
      if (OP == 2) v[i] = __builtin_fmaxf(-v[i], 0.f);
      if (OP == 3 && (i & 1) == 0) {
        const auto p = __builtin_amdgcn_permlane32_swap(u[i], u[i + 1], false, false);
        u[i] = p[0];
        u[i + 1] = p[1];
      }
      if (OP == 4) u[i] = u[i] + u[(i + 1) & 15];
    }
  }
  float acc = 0.f;
  for (int i = 0; i < 16; ++i) acc += a0[i] + a1[i] + v[i] + float(u[i]);
  out[size_t(blockIdx.x) * 64 + threadIdx.x] = acc;
}

// bf16 operands (8 per lane) from two floats.
__device__ __forceinline__ bf16x8 bf16_operand(float a, float b) {
  bf16x8 v;
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)(i & 1 ? b : a);
  return v;
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// 16 fp16 matrix instructions per iteration over 2 independent accumulators.
__global__ __launch_bounds__(64) void mfma_f16_chains(float* out, int iters, float s) {
  f32x16 a0 = {0}, a1 = {0};
  f16x8 x, y;
  for (int i = 0; i < 8; ++i) {
    x[i] = (_Float16)(i & 1 ? s : s * threadIdx.x * 1e-3f);
    y[i] = (_Float16)(i & 1 ? s * 0.5f : s + 1e-3f);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(x, y, a1, 0, 0, 0);
    }
  }
  float acc = 0.f;
  for (int i = 0; i < 16; ++i) acc += a0[i] + a1[i];
  out[size_t(blockIdx.x) * 64 + threadIdx.x] = acc;
}

// 16 bf16 matrix instructions per iteration over NACC independent accumulators.
template <int NACC>
__global__ __launch_bounds__(64) void mfma_bf16_chains(float* out, int iters, float s) {
  f32x16 a[NACC];
#pragma unroll
  for (int k = 0; k < NACC; ++k) a[k] = f32x16{0};
  const bf16x8 x = bf16_operand(s * threadIdx.x * 1e-3f, s), y = bf16_operand(s + 1e-3f, s * 0.5f);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 16 / NACC; ++r)
#pragma unroll
      for (int k = 0; k < NACC; ++k) a[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, a[k], 0, 0, 0);
  }
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < NACC; ++k)
    for (int i = 0; i < 16; ++i) acc += a[k][i];
  out[size_t(blockIdx.x) * 64 + threadIdx.x] = acc;
}

// 4 bf16 matrix instructions (2 chains) plus 16 * OP independent v_fma_f32
// per iteration (OP = 0: none).
template <int OP>
__global__ __launch_bounds__(64) void mfma_bf16_plus(float* out, int iters, float s) {
  f32x16 a0 = {0}, a1 = {0};
  float v[16];
  for (int i = 0; i < 16; ++i) v[i] = threadIdx.x * 0.001f + i;
  const bf16x8 x = bf16_operand(s * threadIdx.x * 1e-3f, s), y = bf16_operand(s + 1e-3f, s * 0.5f);
  const float xf = s * threadIdx.x;
  for (int it = 0; it < iters; ++it) {
    a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, a1, 0, 0, 0);
    a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, a1, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < OP; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = fmaf(v[i], s, xf);
  }
  float acc = 0.f;
  for (int i = 0; i < 16; ++i) acc += a0[i] + a1[i] + v[i];
  out[size_t(blockIdx.x) * 64 + threadIdx.x] = acc;
}

#define CHECK(x)                                                      \
  do {                                                                \
    if ((x) != hipSuccess) {                                          \
      fprintf(stderr, "HIP error %s at %s:%d\n", #x, __FILE__, __LINE__); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

static hipEvent_t e0, e1;

// Best of 3 timed launches (the first of 4 warms up), in ms; < 0 on error.
template <class F>
static float time_ms(F launch) {
  float best = 1e30f;
  for (int rep = 0; rep < 4; ++rep) {
    if (hipEventRecord(e0) != hipSuccess) return -1.f;
    launch();
    if (hipEventRecord(e1) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return -1.f;
    float ms;
    if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return -1.f;
    if (rep > 0 && ms < best) best = ms;
  }
  return hipGetLastError() == hipSuccess ? best : -1.f;
}

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));

  // 1. read bandwidth, 2 GiB, best per grid size
  const size_t bytes = size_t(2) << 30;
  const int max_grid = 65536;
  float *buf, *out;
  CHECK(hipMalloc(&buf, bytes));
  CHECK(hipMalloc(&out, size_t(max_grid) * 256 * sizeof(float)));  // also >= cus * 16 * 64 floats
  if (size_t(max_grid) * 256 < size_t(cus) * 16 * 64) return 1;
  CHECK(hipMemset(buf, 0, bytes));
  double best_bw = 0.0;
  int best_grid = 0;
  for (int grid : {2048, 4096, 8192, 16384, 65536}) {
    const float ms = time_ms([&] {
      hipLaunchKernelGGL(read_stream, dim3(grid), dim3(256), 0, 0, reinterpret_cast<const float4*>(buf), bytes / 16,
                         out);
    });
    if (ms <= 0.f) return 1;
    const double bw = bytes / (ms * 1e-3) / 1e12;
    if (bw > best_bw) {
      best_bw = bw;
      best_grid = grid;
    }
  }
  double best_nt = 0.0;
  int best_nt_grid = 0;
  for (int grid : {2048, 4096, 8192, 16384, 65536}) {
    const float ms = time_ms([&] {
      hipLaunchKernelGGL(read_stream_nt, dim3(grid), dim3(256), 0, 0, reinterpret_cast<const f32x4*>(buf), bytes / 16,
                         out);
    });
    if (ms <= 0.f) return 1;
    const double bw = bytes / (ms * 1e-3) / 1e12;
    if (bw > best_nt) {
      best_nt = bw;
      best_nt_grid = grid;
    }
  }
  CHECK(hipFree(buf));
  printf("{\"device\": \"%s\", \"cus\": %d, \"read_bw_TBps\": %.3f, \"read_bw_grid\": %d, "
         "\"read_bw_nontemporal_TBps\": %.3f, \"read_bw_nontemporal_grid\": %d",
         prop.gcnArchName, cus, best_bw, best_grid, best_nt, best_nt_grid);

  // 2. matrix throughput: waves per SIMD x accumulator chains per wave
  const int iters = 4000;
  printf(", \"mfma_tflops\": {");
  double w4c2 = 0.0;
  bool first = true;
  for (int w : {1, 2, 4}) {
    const int blocks = cus * 4 * w;
    for (int nacc : {1, 2, 4}) {
      const float ms = time_ms([&] {
        if (nacc == 1) hipLaunchKernelGGL(mfma_chains<1>, dim3(blocks), dim3(64), 0, 0, out, iters, 1.0001f);
        if (nacc == 2) hipLaunchKernelGGL(mfma_chains<2>, dim3(blocks), dim3(64), 0, 0, out, iters, 1.0001f);
        if (nacc == 4) hipLaunchKernelGGL(mfma_chains<4>, dim3(blocks), dim3(64), 0, 0, out, iters, 1.0001f);
      });
      if (ms <= 0.f) return 1;
      const double tf = double(blocks) * iters * 16 * 4096 / (ms * 1e-3) / 1e12;  // 4096 FLOP per instruction
      if (w == 4 && nacc == 2) w4c2 = tf;
      printf("%s\"waves%d_chains%d\": %.1f", first ? "" : ", ", w, nacc, tf);
      first = false;
    }
  }
  printf("}, \"mfma_4waves_2chains_tflops\": %.1f", w4c2);

  // 3. added cycles per vector instruction, 4 waves x 2 chains: alone, the 4
  // matrix instructions of an iteration take 4 x 64 = 256 SIMD cycles
  {
    const int blocks = cus * 4 * 4, it2 = 8000;
    float ms[5];
    for (int op = 0; op < 5; ++op) {
      ms[op] = time_ms([&] {
        if (op == 0) hipLaunchKernelGGL(mfma_plus<0>, dim3(blocks), dim3(64), 0, 0, out, it2, 1.0001f);
        if (op == 1) hipLaunchKernelGGL(mfma_plus<1>, dim3(blocks), dim3(64), 0, 0, out, it2, 1.0001f);
        if (op == 2) hipLaunchKernelGGL(mfma_plus<2>, dim3(blocks), dim3(64), 0, 0, out, it2, 1.0001f);
        if (op == 3) hipLaunchKernelGGL(mfma_plus<3>, dim3(blocks), dim3(64), 0, 0, out, it2, 1.0001f);
        if (op == 4) hipLaunchKernelGGL(mfma_plus<4>, dim3(blocks), dim3(64), 0, 0, out, it2, 1.0001f);
      });
      if (ms[op] <= 0.f) return 1;
    }
    const char* names[5] = {"", "v_fma_f32", "v_max_f32", "v_permlane32_swap", "v_add_u32"};
    const int count[5] = {0, 16, 16, 8, 16};  // instructions per iteration
    printf(", \"added_cycles_per_vector_op\": {");
    for (int op = 1; op < 5; ++op)
      printf("%s\"%s\": %.2f", op == 1 ? "" : ", ", names[op], (ms[op] - ms[0]) / ms[0] * 256.0 / count[op]);
    printf("}");
  }
  // 4. bf16 matrix instruction: throughput (4 waves x 2 chains; 32768 FLOP
  // each) and the added cycles per v_fma_f32 beside it (alone, the 4 matrix
  // instructions of an iteration take 4 x 32 = 128 SIMD cycles)
  {
    const int blocks = cus * 4 * 4;
    const float ms = time_ms([&] {
      hipLaunchKernelGGL(mfma_bf16_chains<2>, dim3(blocks), dim3(64), 0, 0, out, iters, 1.0001f);
    });
    if (ms <= 0.f) return 1;
    printf(", \"bf16_mfma_4waves_2chains_tflops\": %.1f", double(blocks) * iters * 16 * 32768 / (ms * 1e-3) / 1e12);
    const int it2 = 8000;
    const float m0 = time_ms([&] {
      hipLaunchKernelGGL(mfma_bf16_plus<0>, dim3(blocks), dim3(64), 0, 0, out, it2, 1.0001f);
    });
    const float m1 = time_ms([&] {
      hipLaunchKernelGGL(mfma_bf16_plus<1>, dim3(blocks), dim3(64), 0, 0, out, it2, 1.0001f);
    });
    if (m0 <= 0.f || m1 <= 0.f) return 1;
    printf(", \"added_cycles_per_v_fma_f32_beside_bf16_mfma\": %.2f", (m1 - m0) / m0 * 128.0 / 16);
    // SIMD cycles per iteration (4 matrix instructions = 128 alone) with
    // 16 k vector FMAs beside them (alone: 4 cycles each)
    const float m2 = time_ms([&] {
      hipLaunchKernelGGL(mfma_bf16_plus<2>, dim3(blocks), dim3(64), 0, 0, out, it2, 1.0001f);
    });
    const float m3 = time_ms([&] {
      hipLaunchKernelGGL(mfma_bf16_plus<3>, dim3(blocks), dim3(64), 0, 0, out, it2, 1.0001f);
    });
    const float m4 = time_ms([&] {
      hipLaunchKernelGGL(mfma_bf16_plus<4>, dim3(blocks), dim3(64), 0, 0, out, it2, 1.0001f);
    });
    if (m2 <= 0.f || m3 <= 0.f || m4 <= 0.f) return 1;
    printf(", \"bf16_mfma_cycles_with_vector_fmas\": {\"0\": 128.0, \"16\": %.1f, \"32\": %.1f, \"48\": %.1f, \"64\": %.1f}",
           128.0 * m1 / m0, 128.0 * m2 / m0, 128.0 * m3 / m0, 128.0 * m4 / m0);
  }
  // 5. fp16 matrix instruction throughput (4 waves x 2 chains)
  {
    const int blocks = cus * 4 * 4;
    const float ms = time_ms([&] {
      hipLaunchKernelGGL(mfma_f16_chains, dim3(blocks), dim3(64), 0, 0, out, iters, 1.0001f);
    });
    if (ms <= 0.f) return 1;
    printf(", \"f16_mfma_4waves_2chains_tflops\": %.1f", double(blocks) * iters * 16 * 32768 / (ms * 1e-3) / 1e12);
  }
  printf("}\n");
  CHECK(hipFree(out));
  return 0;
}
