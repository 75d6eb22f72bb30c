// Host stand-ins for the HIP runtime calls and the kernel launches of the
// library's host planner (lopt_api.cpp), for a CPU-only build of the planner
// under AddressSanitizer and UndefinedBehaviorSanitizer.  Device memory is
// host memory (so every copy the planner makes into its workspace is checked
// by the sanitizer against the buffer's real size), copies are memcpy,
// streams and events do nothing.  The two launch functions do not run
// kernels: they check the plan that the planner wrote into the workspace
// (check_plan) -- every index the kernels would use stays inside its tensor,
// its partial-sum array and the workspace -- and write every workspace range
// the kernels write (touch_workspace).
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "../../learned_optimizer_step_amd/csrc/lopt_internal.h"

// Size of the workspace the test program handed to lopt_init_state (set by
// planner_main.cpp; check_plan keeps every offset below it).
size_t g_stub_ws_bytes = 0;
long g_stub_plan_checks = 0;

extern "C" {
hipError_t hipMalloc(void** p, size_t n) {
  *p = std::malloc(n ? n : 1);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* p) {
  std::free(p);
  return hipSuccess;
}
hipError_t hipHostMalloc(void** p, size_t n, unsigned int) { return hipMalloc(p, n); }
hipError_t hipHostFree(void* p) { return hipFree(p); }
hipError_t hipMemcpy(void* d, const void* s, size_t n, hipMemcpyKind) {
  std::memcpy(d, s, n);
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* d, const void* s, size_t n, hipMemcpyKind k, hipStream_t) { return hipMemcpy(d, s, n, k); }
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceSynchronize() { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* s) {
  *s = hipStreamCaptureStatusNone;
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
  *e = reinterpret_cast<hipEvent_t>(new char[16]);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventDestroy(hipEvent_t e) {
  delete[] reinterpret_cast<char*>(e);
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "host stub"; }
}

namespace {

[[noreturn]] void bad(const char* what, long a, long b) {
  std::fprintf(stderr, "plan check failed: %s (%ld, %ld)\n", what, a, b);
  std::abort();
}
#define REQUIRE(cond, a, b) \
  do {                      \
    if (!(cond)) bad(#cond, long(a), long(b)); \
  } while (0)

void check_plan(const lopt::StepCtx& c) {
  using namespace lopt;
  ++g_stub_plan_checks;
  const char* ws = reinterpret_cast<const char*>(c.ws);
  const size_t wsf = g_stub_ws_bytes / sizeof(float);
  auto inside = [&](const void* p, size_t bytes) {
    const char* q = static_cast<const char*>(p);
    return q >= ws && q + bytes <= ws + g_stub_ws_bytes;
  };
  REQUIRE(c.n_tensors >= 0 && c.n_chunks >= 0 && c.n_tiles0 >= 0 && c.n_segs1 >= 0, c.n_tensors, c.n_chunks);
  REQUIRE(inside(c.desc, sizeof(TensorDesc) * c.n_tensors), c.n_tensors, 0);
  REQUIRE(inside(c.grads, sizeof(float*) * c.n_tensors), c.n_tensors, 0);
  REQUIRE(inside(c.tiles0, sizeof(Tile0) * c.n_tiles0), c.n_tiles0, 0);
  REQUIRE(inside(c.segs1, sizeof(Seg1) * c.n_segs1), c.n_segs1, 0);
  REQUIRE(inside(c.chunks, sizeof(Chunk) * c.n_chunks), c.n_chunks, 0);
  REQUIRE(inside(c.stats_part, sizeof(float) * kStatStride * c.n_chunks), c.n_chunks, 0);
  REQUIRE(inside(c.scales, sizeof(float) * kStatStride * c.n_tensors), c.n_tensors, 0);
  REQUIRE(inside(c.packed, sizeof(float) * kPkFloats), 0, 0);
  REQUIRE(inside(c.step, sizeof(int64_t)), 0, 0);
  REQUIRE(inside(c.tensor_hyper, 2 * sizeof(float) * c.n_tensors), c.n_tensors, 0);
  int32_t n_rseg = 0;
  int64_t next_chunk = 0;
  for (int32_t t = 0; t < c.n_tensors; ++t) {
    const TensorDesc& d = c.desc[t];
    REQUIRE(d.R >= 1 && d.C >= 1 && uint64_t(d.R) * uint64_t(d.C) == d.n && d.n < (1u << 31), d.R, d.C);
    REQUIRE(d.vec == (d.R == 1), d.vec, d.R);
    // the division constants: e / C for e at the edges and a sweep of the index range
    for (uint64_t e = 0; e < d.n; e += 1 + d.n / 4099) {
      for (uint64_t q : {e, uint64_t(d.n) - 1 - e}) {
        const uint32_t got = uint32_t(((q * d.cmagic >> 32) + q) >> d.cshift);
        REQUIRE(got == q / uint64_t(d.C), q, d.C);
      }
    }
    // per-tensor arrays inside the workspace's float region
    REQUIRE(d.off_rowpart >= 0 && uint64_t(d.off_rowpart) + uint64_t(d.ncw) * d.R <= wsf, d.off_rowpart, d.ncw);
    if (!d.vec) REQUIRE(d.off_colpart >= 0 && uint64_t(d.off_colpart) + uint64_t(d.nrb) * d.C <= wsf, d.off_colpart, d.nrb);
    REQUIRE(d.off_rq % 4 == 0 && uint64_t(d.off_rq) + 4ull * d.R <= wsf, d.off_rq, d.R);
    if (!d.vec) REQUIRE(d.off_cq % 4 == 0 && uint64_t(d.off_cq) + 4ull * d.C <= wsf, d.off_cq, d.C);
    // chunks: consecutive, covering [0, n) of the tensor in order
    REQUIRE(d.chunk0 == next_chunk && d.nchunk >= 1, d.chunk0, next_chunk);
    uint32_t e = 0;
    for (int32_t k = 0; k < d.nchunk; ++k) {
      const Chunk& ch = c.chunks[d.chunk0 + k];
      REQUIRE(ch.tensor == t && ch.e0 == e && ch.e1 > ch.e0 && ch.e1 <= d.n, ch.e0, ch.e1);
      REQUIRE(ch.e0 % 256 == 0 && ch.row0 == ch.e0 / uint32_t(d.C), ch.e0, ch.row0);
      REQUIRE(ch.e1 - ch.e0 <= uint32_t(kChunkElems), ch.e1 - ch.e0, 0);
      e = ch.e1;
    }
    REQUIRE(e == d.n, e, d.n);
    next_chunk += d.nchunk;
    REQUIRE(d.rseg0 == n_rseg && d.nrseg >= 1, d.rseg0, n_rseg);
    n_rseg += d.nrseg;
  }
  REQUIRE(next_chunk == c.n_chunks, next_chunk, c.n_chunks);
  REQUIRE(inside(c.rbar_part, 4 * sizeof(float) * size_t(n_rseg)), n_rseg, 0);
  // row/column tiles: every element of every tensor covered exactly once
  std::vector<uint64_t> covered(size_t(c.n_tensors), 0);
  for (int32_t q = 0; q < c.n_tiles0; ++q) {
    const Tile0& tl = c.tiles0[q];
    REQUIRE(tl.tensor >= 0 && tl.tensor < c.n_tensors, tl.tensor, q);
    const TensorDesc& d = c.desc[tl.tensor];
    REQUIRE(tl.flat == d.vec, tl.flat, d.vec);
    REQUIRE(tl.win >= 0 && tl.win < d.ncw, tl.win, d.ncw);
    if (tl.flat) {
      REQUIRE(tl.c0 >= 0 && tl.c0 < tl.c1 && uint32_t(tl.c1) <= d.n, tl.c0, tl.c1);
      covered[tl.tensor] += uint64_t(tl.c1 - tl.c0);
    } else {
      REQUIRE(tl.r0 >= 0 && tl.r0 < tl.r1 && tl.r1 <= d.R, tl.r0, tl.r1);
      REQUIRE(tl.c0 >= 0 && tl.c0 < tl.c1 && tl.c1 <= d.C, tl.c0, tl.c1);
      REQUIRE(tl.rb >= 0 && tl.rb < d.nrb, tl.rb, d.nrb);
      REQUIRE(tl.cw_log2 >= 0 && tl.cw_log2 <= 8 && (tl.c1 - tl.c0) <= (1 << tl.cw_log2), tl.cw_log2, tl.c1 - tl.c0);
      REQUIRE((tl.r1 - tl.r0) <= (kBlock >> tl.cw_log2) * kTile0Iters, tl.r1 - tl.r0, tl.cw_log2);
      covered[tl.tensor] += uint64_t(tl.r1 - tl.r0) * uint64_t(tl.c1 - tl.c0);
    }
  }
  for (int32_t t = 0; t < c.n_tensors; ++t) REQUIRE(covered[t] == c.desc[t].n, covered[t], c.desc[t].n);
  // moving-average segments: rows and columns of every tensor exactly once
  std::vector<uint64_t> rows(size_t(c.n_tensors), 0), cols(size_t(c.n_tensors), 0);
  for (int32_t q = 0; q < c.n_segs1; ++q) {
    const Seg1& sg = c.segs1[q];
    REQUIRE(sg.tensor >= 0 && sg.tensor < c.n_tensors, sg.tensor, q);
    const TensorDesc& d = c.desc[sg.tensor];
    REQUIRE(sg.a >= 0 && sg.a < sg.b, sg.a, sg.b);
    if (sg.kind == kSegVec) {
      REQUIRE(d.vec && sg.slot == d.rseg0, sg.slot, d.rseg0);
      rows[sg.tensor] += 1;
      cols[sg.tensor] += d.C;
    } else if (sg.kind == kSegRows) {
      REQUIRE(!d.vec && sg.b <= d.R && sg.b - sg.a <= kSeg1, sg.b, d.R);
      REQUIRE(sg.slot >= d.rseg0 && sg.slot < d.rseg0 + d.nrseg, sg.slot, d.rseg0);
      rows[sg.tensor] += uint64_t(sg.b - sg.a);
    } else {
      REQUIRE(sg.kind == kSegCols && !d.vec && sg.b <= d.C && sg.b - sg.a <= kSegCols1, sg.kind, sg.b);
      cols[sg.tensor] += uint64_t(sg.b - sg.a);
    }
  }
  for (int32_t t = 0; t < c.n_tensors; ++t)
    REQUIRE(rows[t] == uint64_t(c.desc[t].R) && cols[t] == uint64_t(c.desc[t].C), rows[t], cols[t]);
}

// Writes every workspace range the step's kernels write (the row/column
// partials and records of each tensor, the r-bar partials, the statistics
// partials, the scales, the packed MLP, the step counter) and reads the ones
// they only read, through memset/memcpy, which the sanitizer checks against
// the workspace's real allocation.
void touch_workspace(const lopt::StepCtx& c) {
  using namespace lopt;
  float* ws = c.ws;
  for (int32_t t = 0; t < c.n_tensors; ++t) {
    const TensorDesc& d = c.desc[t];
    std::memset(ws + d.off_rowpart, 0, sizeof(float) * size_t(d.ncw) * d.R);
    if (!d.vec) std::memset(ws + d.off_colpart, 0, sizeof(float) * size_t(d.nrb) * d.C);
    std::memset(ws + d.off_rq, 0, sizeof(float) * 4 * size_t(d.R));
    if (!d.vec) std::memset(ws + d.off_cq, 0, sizeof(float) * 4 * size_t(d.C));
    const float* g = nullptr;
    std::memcpy(&g, &c.grads[t], sizeof(g));
    (void)g;
  }
  int32_t n_rseg = 0;
  for (int32_t t = 0; t < c.n_tensors; ++t) n_rseg += c.desc[t].nrseg;
  std::memset(c.rbar_part, 0, sizeof(float) * 4 * size_t(n_rseg));
  std::memset(c.stats_part, 0, sizeof(float) * kStatStride * size_t(c.n_chunks));
  std::memset(c.scales, 0, sizeof(float) * kStatStride * size_t(c.n_tensors));
  std::memset(c.packed, 0, sizeof(float) * kPkFloats);
  std::vector<float> th(2 * size_t(c.n_tensors) + 1);
  std::memcpy(th.data(), c.tensor_hyper, sizeof(float) * 2 * size_t(c.n_tensors));
  int64_t step = 0;
  std::memcpy(&step, c.step, sizeof(step));
  ++step;
  std::memcpy(c.step, &step, sizeof(step));
}

}  // namespace

namespace lopt {
// lopt_init_state_static's array: host memory of the same size here
alignas(256) static unsigned char g_scratch[kScratchBytes];
hipError_t scratch_address(int device, void** out) {
  if (device != 0) return hipErrorInvalidDevice;
  *out = g_scratch;
  return hipSuccess;
}
hipError_t launch_zero_state(const StepCtx& c, hipStream_t) {
  check_plan(c);
  return hipSuccess;
}
hipError_t launch_step(const StepCtx& c, const StepParams& p, hipStream_t, const hipEvent_t*) {
  check_plan(c);
  touch_workspace(c);
  if (p.n_feat != kNF && p.n_feat != kVeloNF) return hipErrorInvalidValue;
  return hipSuccess;
}
// a row-shard phase: the plan, the exchange buffers inside the workspace
// (phase 0 writes sums1, phase 1 sums2, phase 2 reads both), then the step's
// own workspace ranges
hipError_t launch_shard_phase(const StepCtx& c, const StepParams& p, int phase, hipStream_t s, const hipEvent_t*) {
  REQUIRE(c.sharded == 1 && phase >= 0 && phase <= 2, c.sharded, phase);
  size_t n1 = 0;
  for (int32_t t = 0; t < c.n_tensors; ++t) {
    const TensorDesc& d = c.desc[t];
    REQUIRE(d.off_sum1 == int64_t(n1), d.off_sum1, n1);
    REQUIRE(d.Rg >= d.R && d.ng >= d.n, d.Rg, d.ng);
    n1 += d.vec ? 1 : size_t(d.C);
  }
  const char* ws = reinterpret_cast<const char*>(c.ws);
  const char* a1 = reinterpret_cast<const char*>(c.sums1);
  const char* a2 = reinterpret_cast<const char*>(c.sums2);
  REQUIRE(c.n_tensors == 0 || (a1 >= ws && a1 + 4 * n1 <= ws + g_stub_ws_bytes), a1 - ws, n1);
  REQUIRE(c.n_tensors == 0 || (a2 >= ws && a2 + 4 * size_t(kStatStride) * c.n_tensors <= ws + g_stub_ws_bytes), a2 - ws,
          c.n_tensors);
  if (phase == 0) std::memset(c.sums1, 0, 4 * n1);
  if (phase == 1) std::memset(c.sums2, 0, 4 * size_t(kStatStride) * c.n_tensors);
  if (phase == 2) return launch_step(c, p, s, nullptr);
  check_plan(c);
  return hipSuccess;
}
// the one-launch step: 1024 resident blocks, as a 256-CU device at four per CU
hipError_t single_grid_cap(int device, int impl, int* blocks) {
  if (device != 0 || impl < 1 || impl > 6) return hipErrorInvalidValue;
  *blocks = 1024;
  return hipSuccess;
}
hipError_t launch_single(const StepCtx& c, const StepParams& p, int blocks, hipStream_t s, const hipEvent_t* ev) {
  const int work = std::max(std::max(c.n_tiles0, c.n_segs1), std::max(c.n_chunks, c.n_tensors + 1));
  if (c.n_tensors > 0) REQUIRE(blocks >= 1 && blocks <= 1024 && blocks <= work, blocks, work);
  const char* ws = reinterpret_cast<const char*>(c.ws);
  const char* q = reinterpret_cast<const char*>(c.sync);
  REQUIRE(q >= ws && q + sizeof(uint32_t) * kSyncWords <= ws + g_stub_ws_bytes, q - ws, g_stub_ws_bytes);
  REQUIRE(blocks <= kSingleMaxBlocks, blocks, kSingleMaxBlocks);
  std::vector<uint32_t> words(kSyncWords);
  std::memcpy(words.data(), c.sync, sizeof(uint32_t) * kSyncWords);
  ++words[0];
  for (int b = 0; b < blocks; ++b) words[kSyncArrive + b] = 4 * words[0];
  std::memcpy(c.sync, words.data(), sizeof(uint32_t) * kSyncWords);
  return launch_step(c, p, s, ev);
}
}  // namespace lopt
