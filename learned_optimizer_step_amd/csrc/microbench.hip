// Measured machine figures behind the roofline of the optimizer step:
//   1. streaming read bandwidth of HBM (the bound of the statistics pass),
//   2. fp32 matrix-core vs vector-ALU issue: the time of a loop of
//      independent v_mfma_f32_32x32x2_f32, of a loop of independent v_fma_f32,
//      and of both interleaved (if the two co-execute, "both" ~ max; if they
//      share the SIMD's issue, "both" ~ sum).
// Prints one JSON object.  Every kernel stays inside its buffers.
#include <hip/hip_runtime.h>

#include <cstdio>

typedef float f32x16 __attribute__((ext_vector_type(16)));

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

// MODE 1: 4 MFMAs per iteration; 2: 64 FMAs per iteration; 3: both.
template <int MODE>
__global__ __launch_bounds__(64) void issue_mix(float* out, int iters, float s) {
  f32x16 a0 = {0}, a1 = {0}, a2 = {0}, a3 = {0};
  float v[16];
  for (int i = 0; i < 16; ++i) v[i] = threadIdx.x * 0.001f + i;
  const float x = s * threadIdx.x, y = s + threadIdx.x;
  for (int it = 0; it < iters; ++it) {
    if (MODE & 1) {
      a0 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, a1, 0, 0, 0);
      a2 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, a2, 0, 0, 0);
      a3 = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, a3, 0, 0, 0);
    }
    if (MODE & 2) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = fmaf(v[i], s, x);
    }
  }
  float acc = 0.f;
  for (int i = 0; i < 16; ++i) acc += a0[i] + a1[i] + a2[i] + a3[i] + v[i];
  out[size_t(blockIdx.x) * 64 + threadIdx.x] = acc;
}

#define CHECK(x)                                                      \
  do {                                                                \
    if ((x) != hipSuccess) {                                          \
      fprintf(stderr, "HIP error %s at %s:%d\n", #x, __FILE__, __LINE__); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));

  // 1. read bandwidth, 2 GiB, best of 5 per grid size
  const size_t bytes = size_t(2) << 30;
  float *buf, *out;
  const int max_grid = 65536;
  CHECK(hipMalloc(&buf, bytes));
  CHECK(hipMalloc(&out, size_t(max_grid) * 256 * sizeof(float)));
  CHECK(hipMemset(buf, 0, bytes));
  double best_bw = 0.0;
  int best_grid = 0;
  for (int grid : {2048, 4096, 8192, 16384, 65536}) {
    for (int r = 0; r < 5; ++r) {
      CHECK(hipEventRecord(e0));
      hipLaunchKernelGGL(read_stream, dim3(grid), dim3(256), 0, 0, reinterpret_cast<const float4*>(buf),
                         bytes / 16, out);
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      const double bw = bytes / (ms * 1e-3) / 1e12;
      if (bw > best_bw) { best_bw = bw; best_grid = grid; }
    }
  }
  CHECK(hipFree(buf));

  // 2. matrix vs vector issue, one and four waves per SIMD
  const int iters = 20000;
  printf("{\"device\": \"%s\", \"cus\": %d, \"read_bw_TBps\": %.3f, \"read_bw_grid\": %d", prop.gcnArchName, cus,
         best_bw, best_grid);
  for (int wps : {1, 4}) {
    const int blocks = cus * 4 * wps;
    float ms[3];
    for (int m = 0; m < 3; ++m) {
      for (int rep = 0; rep < 2; ++rep) {  // first launch warms up
        CHECK(hipEventRecord(e0));
        if (m == 0) hipLaunchKernelGGL(issue_mix<1>, dim3(blocks), dim3(64), 0, 0, out, iters, 1.0001f);
        if (m == 1) hipLaunchKernelGGL(issue_mix<2>, dim3(blocks), dim3(64), 0, 0, out, iters, 1.0001f);
        if (m == 2) hipLaunchKernelGGL(issue_mix<3>, dim3(blocks), dim3(64), 0, 0, out, iters, 1.0001f);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        CHECK(hipEventElapsedTime(&ms[m], e0, e1));
      }
    }
    const double mx = ms[0] > ms[1] ? ms[0] : ms[1];
    printf(", \"waves_per_simd_%d\": {\"mfma_ms\": %.3f, \"valu_ms\": %.3f, \"both_ms\": %.3f, "
           "\"both_over_max\": %.3f, \"both_over_sum\": %.3f}",
           wps, ms[0], ms[1], ms[2], ms[2] / mx, ms[2] / (ms[0] + ms[1]));
  }
  printf("}\n");
  CHECK(hipFree(out));
  return 0;
}
