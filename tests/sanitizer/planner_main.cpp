// Drives the library's host planner (lopt_api.cpp, linked with the host
// stand-ins of hip_host_stub.cpp) through its C ABI on the CPU, built with
// AddressSanitizer and UndefinedBehaviorSanitizer: argument validation,
// workspace sizing and planning for a seeded sweep of tensor lists and for the
// lists named on the command line (a file of "rows cols" lines each), the
// uploads between steps (changed gradient pointers, per-tensor learning rates
// and weight decays), the step counter and the statistics read-back.  Every
// workspace is allocated with exactly the size lopt_workspace_bytes reports,
// so a write past it is a sanitizer error; the launch stand-ins check the
// plan itself.  Tensor addresses are fake: the planner never dereferences them.
//
//   planner_sanitized [LIST_FILE ...]     exit status 0: every case passed
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <random>
#include <string>
#include <utility>
#include <vector>

#include "lopt.h"

extern size_t g_stub_ws_bytes;
extern long g_stub_plan_checks;

namespace {

int g_failures = 0;

void expect(bool ok, const std::string& what) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s (last error: %s)\n", what.c_str(), lopt_last_error());
    ++g_failures;
  }
}

using Shape = std::pair<int64_t, int64_t>;

// Disjoint fake device ranges, 256-byte aligned, far from any real mapping.
struct FakeSpace {
  uint64_t next = uint64_t(1) << 44;
  float* take(uint64_t bytes) {
    const uint64_t a = next;
    next += (bytes + 4095) / 4096 * 4096 + 4096;
    return reinterpret_cast<float*>(a);
  }
};

std::vector<lopt_tensor> make_list(const std::vector<Shape>& shapes, FakeSpace& fs) {
  std::vector<lopt_tensor> ts(shapes.size());
  for (size_t i = 0; i < shapes.size(); ++i) {
    const int64_t r = shapes[i].first, c = shapes[i].second;
    ts[i].rows = r;
    ts[i].cols = c;
    ts[i].param = fs.take(4 * uint64_t(r) * uint64_t(c));
    ts[i].grad = fs.take(4 * uint64_t(r) * uint64_t(c));
    ts[i].state = fs.take(4 * uint64_t(lopt_state_floats(r, c)));
  }
  return ts;
}

void run_list(const std::vector<Shape>& shapes, const std::string& name, int n_feat) {
  FakeSpace fs;
  std::vector<lopt_tensor> ts = make_list(shapes, fs);
  const int32_t n = int32_t(ts.size());
  size_t bytes = 0;
  expect(lopt_workspace_bytes(nullptr, ts.data(), n, &bytes) == LOPT_OK, name + ": workspace_bytes");
  if (g_failures) return;
  void* ws = nullptr;
  if (posix_memalign(&ws, 256, bytes ? bytes : 1) != 0) {
    expect(false, name + ": host allocation");
    return;
  }
  g_stub_ws_bytes = bytes;
  lopt_config cfg;
  lopt_default_config(&cfg);
  cfg.n_feat = n_feat;
  std::vector<float> mlp(lopt_mlp_floats(n_feat, cfg.n_time), 0.01f);
  lopt_handle* h = nullptr;
  expect(lopt_create(&cfg, mlp.data(), &h) == LOPT_OK, name + ": create");
  if (!h) {
    std::free(ws);
    return;
  }
  if (bytes > 0) {
    expect(lopt_init_state(h, ts.data(), n, ws, bytes - 1, nullptr) == LOPT_ERR_WORKSPACE, name + ": short workspace");
    expect(lopt_init_state(h, ts.data(), n, static_cast<char*>(ws) + 16, bytes, nullptr) == LOPT_ERR_WORKSPACE,
           name + ": unaligned workspace");
  }
  expect(lopt_init_state(h, ts.data(), n, ws, bytes, nullptr) == LOPT_OK, name + ": init_state");
  expect(lopt_step(h, ts.data(), n, nullptr) == LOPT_OK, name + ": step");
  // new gradient buffers (torch's zero_grad(set_to_none=True) gives new addresses), some without one
  for (int round = 0; round < 3; ++round) {
    for (int32_t i = 0; i < n; ++i)
      ts[i].grad = (i + round) % 5 == 0 ? nullptr : fs.take(4 * uint64_t(ts[i].rows) * uint64_t(ts[i].cols));
    expect(lopt_step(h, ts.data(), n, nullptr) == LOPT_OK, name + ": step with new gradients");
  }
  std::vector<float> lr(size_t(n) + 1, 0.5f), wd(size_t(n) + 1, 0.01f);
  expect(lopt_set_tensor_hyper(h, lr.data(), wd.data(), n) == LOPT_OK, name + ": set_tensor_hyper");
  expect(lopt_step(h, ts.data(), n, nullptr) == LOPT_OK, name + ": step with per-tensor values");
  expect(lopt_set_tensor_hyper(h, lr.data(), wd.data(), n + 1) == LOPT_ERR_STATE, name + ": hyper count");
  expect(lopt_set_tensor_hyper(h, nullptr, nullptr, n) == LOPT_OK, name + ": clear per-tensor values");
  for (int32_t mode : {LOPT_LAUNCH_SINGLE, LOPT_LAUNCH_SPLIT, LOPT_LAUNCH_AUTO}) {
    cfg.launch = mode;
    expect(lopt_set_config(h, &cfg) == LOPT_OK && lopt_step(h, ts.data(), n, nullptr) == LOPT_OK,
           name + ": step with launch mode " + std::to_string(mode));
  }
  int64_t t = -1;
  expect(lopt_set_step(h, 41) == LOPT_OK && lopt_get_step(h, &t) == LOPT_OK && t == 41, name + ": step counter");
  std::vector<float> stats(size_t(n) * LOPT_STAT_FLOATS + 1);
  expect(lopt_get_tensor_stats(h, stats.data(), n) == LOPT_OK, name + ": tensor stats");
  expect(lopt_get_tensor_stats(h, stats.data(), n + 1) == LOPT_ERR_STATE, name + ": stats count");
  if (n > 0) {
    std::vector<lopt_tensor> other = ts;
    other[n - 1].rows += 0;
    other[n - 1].state = fs.take(4 * uint64_t(lopt_state_floats(other[n - 1].rows, other[n - 1].cols)));
    expect(lopt_step(h, other.data(), n, nullptr) == LOPT_ERR_STATE, name + ": a different list");
  }
  lopt_destroy(h);
  std::free(ws);
}

// A row-shard binding of `shapes`, each the shard of a whole tensor with
// `factor` times its rows (a 1-D shard: times its length): sizing, binding,
// two steps of three phases, the exchange buffers, the phase order and the
// refusal of lopt_step.
void run_sharded(const std::vector<Shape>& shapes, int64_t factor, const std::string& name) {
  if (g_failures) return;
  FakeSpace fs;
  std::vector<lopt_tensor> ts = make_list(shapes, fs);
  const int32_t n = int32_t(ts.size());
  std::vector<int64_t> dims;
  for (const Shape& sh : shapes) {
    dims.push_back(sh.first == 1 ? 1 : sh.first * factor);
    dims.push_back(sh.first == 1 ? sh.second * factor : sh.second);
  }
  size_t bytes = 0;
  expect(lopt_workspace_bytes_sharded(nullptr, ts.data(), n, dims.data(), &bytes) == LOPT_OK, name + ": bytes");
  void* ws = nullptr;
  if (posix_memalign(&ws, 256, bytes ? bytes : 1) != 0) {
    expect(false, name + ": host allocation");
    return;
  }
  g_stub_ws_bytes = bytes;
  lopt_config cfg;
  lopt_default_config(&cfg);
  std::vector<float> mlp(lopt_mlp_floats(cfg.n_feat, cfg.n_time), 0.01f);
  lopt_handle* h = nullptr;
  expect(lopt_create(&cfg, mlp.data(), &h) == LOPT_OK, name + ": create");
  if (!h) {
    std::free(ws);
    return;
  }
  expect(lopt_init_state_sharded(h, ts.data(), n, dims.data(), ws, bytes, nullptr) == LOPT_OK, name + ": init");
  float* s1 = nullptr;
  float* s2 = nullptr;
  size_t n1 = 0, n2 = 0;
  expect(lopt_get_shard_sums(h, &s1, &n1, &s2, &n2) == LOPT_OK, name + ": shard sums");
  size_t want1 = 0;
  for (const Shape& sh : shapes) want1 += sh.first == 1 ? 1 : size_t(sh.second);
  expect(n1 == want1 && n2 == 32 * size_t(n), name + ": exchange sizes");
  expect(lopt_step(h, ts.data(), n, nullptr) == LOPT_ERR_STATE, name + ": lopt_step refused");
  expect(lopt_step_shard(h, ts.data(), n, 1, nullptr) == LOPT_ERR_STATE, name + ": phase out of order");
  for (int step = 0; step < 2; ++step)
    for (int32_t phase = 0; phase < 3; ++phase) {
      expect(lopt_step_shard(h, ts.data(), n, phase, nullptr) == LOPT_OK, name + ": phase " + std::to_string(phase));
      if (phase < 2 && n1 + n2 > 0) {  // the exchange: the caller adds the other ranks' sums in place
        for (size_t q = 0; q < n1; ++q) s1[q] *= float(factor);
        for (size_t q = 0; q < n2; ++q) s2[q] *= float(factor);
      }
    }
  if (n > 0) {
    std::vector<lopt_tensor> moved = ts;
    moved[0].grad = fs.take(4 * uint64_t(ts[0].rows) * uint64_t(ts[0].cols));
    expect(lopt_step_shard(h, ts.data(), n, 0, nullptr) == LOPT_OK, name + ": phase 0 again");
    expect(lopt_step_shard(h, moved.data(), n, 1, nullptr) == LOPT_ERR_STATE, name + ": gradients moved mid-step");
  }
  int64_t t = -1;
  expect(lopt_get_step(h, &t) == LOPT_OK && t >= 0, name + ": step counter");
  lopt_destroy(h);
  std::free(ws);
}

// lopt_init_state_static: the same checks on the library's static array (the
// stand-in holds LOPT_STATIC_SCRATCH_BYTES of host memory), a list too large
// for it, and a second static binding that takes the array over.
void static_cases() {
  FakeSpace fs;
  lopt_config cfg;
  lopt_default_config(&cfg);
  std::vector<float> mlp(lopt_mlp_floats(28, 11), 0.01f);
  lopt_handle *a = nullptr, *b = nullptr;
  expect(lopt_create(&cfg, mlp.data(), &a) == LOPT_OK && lopt_create(&cfg, mlp.data(), &b) == LOPT_OK, "create");
  std::vector<lopt_tensor> big = make_list(std::vector<Shape>(12, Shape{32000, 2048}), fs);
  size_t bytes = 0;
  expect(lopt_workspace_bytes(nullptr, big.data(), int32_t(big.size()), &bytes) == LOPT_OK &&
             bytes > LOPT_STATIC_SCRATCH_BYTES, "a list larger than the static array");
  g_stub_ws_bytes = LOPT_STATIC_SCRATCH_BYTES;
  expect(lopt_init_state_static(a, big.data(), int32_t(big.size()), nullptr) == LOPT_ERR_WORKSPACE,
         "static binding refuses a list larger than the array");
  expect(lopt_step(a, big.data(), int32_t(big.size()), nullptr) == LOPT_ERR_STATE, "still unbound");
  g_stub_ws_bytes = LOPT_STATIC_SCRATCH_BYTES;
  std::vector<lopt_tensor> l1 = make_list({{300, 512}, {1, 7000}, {64, 64}, {33, 65}}, fs);
  std::vector<lopt_tensor> l2 = make_list({{40, 64}, {1, 100}}, fs);
  expect(lopt_init_state_static(a, l1.data(), 4, nullptr) == LOPT_OK, "static binding");
  for (int k = 0; k < 3; ++k) {
    for (auto& t : l1) t.grad = fs.take(4 * uint64_t(t.rows) * uint64_t(t.cols));   // new gradients each step
    expect(lopt_step(a, l1.data(), 4, nullptr) == LOPT_OK, "static step");
  }
  std::vector<float> lr(4, 0.5f), wd(4, 0.01f);
  expect(lopt_set_tensor_hyper(a, lr.data(), wd.data(), 4) == LOPT_OK && lopt_step(a, l1.data(), 4, nullptr) == LOPT_OK,
         "static step with per-tensor values");
  expect(lopt_init_state_static(b, l2.data(), 2, nullptr) == LOPT_OK, "second static binding, smaller list");
  expect(lopt_step(b, l2.data(), 2, nullptr) == LOPT_OK, "step of the second binding");
  int64_t t = 0;
  expect(lopt_step(a, l1.data(), 4, nullptr) == LOPT_ERR_STATE, "the replaced binding's step is refused");
  expect(lopt_get_step(a, &t) == LOPT_ERR_STATE, "the replaced binding's counter is refused");
  expect(lopt_init_state_static(a, l1.data(), 4, nullptr) == LOPT_OK && lopt_step(a, l1.data(), 4, nullptr) == LOPT_OK,
         "binding again");
  lopt_destroy(b);
  lopt_destroy(a);
}

void validation_cases() {
  FakeSpace fs;
  auto status = [](const std::vector<lopt_tensor>& ts) {
    size_t b = 0;
    return lopt_workspace_bytes(nullptr, ts.data(), int32_t(ts.size()), &b);
  };
  auto base = [&] { return make_list({{16, 16}, {1, 9}, {3, 5}}, fs); };
  std::vector<lopt_tensor> ts;
  ts = base(); ts[0].rows = 0; expect(status(ts) == LOPT_ERR_INVALID_ARGUMENT, "rows 0");
  ts = base(); ts[1].cols = -3; expect(status(ts) == LOPT_ERR_INVALID_ARGUMENT, "negative cols");
  ts = base(); ts[2].param = nullptr; expect(status(ts) == LOPT_ERR_INVALID_ARGUMENT, "NULL param");
  ts = base(); ts[2].state = nullptr; expect(status(ts) == LOPT_ERR_INVALID_ARGUMENT, "NULL state");
  ts = base(); ts[0].param = reinterpret_cast<float*>(reinterpret_cast<char*>(ts[0].param) + 2);
  expect(status(ts) == LOPT_ERR_UNSUPPORTED, "misaligned param");
  ts = base(); ts[0].rows = int64_t(1) << 16; ts[0].cols = int64_t(1) << 15;
  expect(status(ts) == LOPT_ERR_UNSUPPORTED, "2^31 elements");
  ts = base(); ts[0].rows = 2; ts[0].cols = int64_t(1) << 28; expect(status(ts) == LOPT_ERR_UNSUPPORTED, "2^28 columns");
  ts = base(); ts[0].rows = int64_t(1) << 40; ts[0].cols = int64_t(1) << 40;
  expect(status(ts) == LOPT_ERR_UNSUPPORTED, "rows * cols overflowing 64 bits");
  ts = base(); ts[0].grad = ts[0].param; expect(status(ts) == LOPT_ERR_INVALID_ARGUMENT, "grad aliasing param");
  ts = base(); ts[1].grad = ts[0].state + 7; expect(status(ts) == LOPT_ERR_INVALID_ARGUMENT, "grad inside a state");
  ts = base(); ts[2].state = ts[0].param + 3; expect(status(ts) == LOPT_ERR_INVALID_ARGUMENT, "state overlapping a param");
  ts = base(); ts[1].param = ts[1].state; expect(status(ts) == LOPT_ERR_INVALID_ARGUMENT, "param aliasing own state");
  ts = base(); ts[2].grad = ts[1].grad; expect(status(ts) == LOPT_OK, "shared gradient buffers are allowed");
  ts = base(); ts[1].grad = nullptr; expect(status(ts) == LOPT_OK, "NULL gradient is allowed");
  size_t b = 0;
  expect(lopt_workspace_bytes(nullptr, nullptr, 2, &b) == LOPT_ERR_INVALID_ARGUMENT, "NULL list");
  expect(lopt_workspace_bytes(nullptr, ts.data(), -1, &b) == LOPT_ERR_INVALID_ARGUMENT, "negative count");
  expect(lopt_workspace_bytes(nullptr, ts.data(), 3, nullptr) == LOPT_ERR_INVALID_ARGUMENT, "NULL output");
  lopt_config cfg;
  lopt_default_config(&cfg);
  std::vector<float> mlp(lopt_mlp_floats(28, 11), 0.f);
  lopt_handle* h = nullptr;
  cfg.mlp_impl = 99;
  expect(lopt_create(&cfg, mlp.data(), &h) == LOPT_ERR_INVALID_ARGUMENT && !h, "unknown mlp_impl");
  lopt_default_config(&cfg);
  cfg.launch = 3;
  expect(lopt_create(&cfg, mlp.data(), &h) == LOPT_ERR_INVALID_ARGUMENT && !h, "unknown launch mode");
  lopt_default_config(&cfg);
  mlp[7] = std::nanf("");
  expect(lopt_create(&cfg, mlp.data(), &h) == LOPT_ERR_INVALID_ARGUMENT && !h, "NaN weight");
  mlp[7] = 0.f;
  expect(lopt_create(&cfg, mlp.data(), &h) == LOPT_OK && h, "create");
  expect(lopt_step(h, ts.data(), 3, nullptr) == LOPT_ERR_STATE, "step before init_state");
  expect(lopt_get_tensor_stats(h, nullptr, 0) == LOPT_ERR_INVALID_ARGUMENT, "stats NULL output");
  lopt_destroy(h);
}

std::vector<Shape> random_list(std::mt19937_64& rng) {
  std::vector<Shape> out;
  const int n = 1 + int(rng() % 24);
  for (int i = 0; i < n; ++i) {
    const int kind = int(rng() % 5);
    const int64_t a = 1 + int64_t(rng() % 3000), b = 1 + int64_t(rng() % 3000);
    if (kind == 0) out.push_back({1, 1 + int64_t(rng() % (1 << 20))});    // 1-D
    else if (kind == 1) out.push_back({a, 64 * (1 + int64_t(rng() % 40))});  // columns a multiple of 64
    else if (kind == 2) out.push_back({a, 1 + int64_t(rng() % 7)});         // thin
    else if (kind == 3) out.push_back({1 + int64_t(rng() % 5), b * 37});    // wide
    else out.push_back({a, b});
  }
  return out;
}

std::vector<Shape> read_list(const char* path) {
  std::vector<Shape> out;
  std::ifstream f(path);
  int64_t r, c;
  while (f >> r >> c) out.push_back({r, c});
  return out;
}

}  // namespace

int main(int argc, char** argv) {
  validation_cases();
  static_cases();
  // the edges of the size range
  run_list({{1, 1}}, "1x1", 28);
  run_list({{1, (int64_t(1) << 31) - 1}}, "1 x (2^31 - 1)", 28);
  run_list({{2, (int64_t(1) << 28) - 1}}, "2 x (2^28 - 1)", 19);
  run_list({{int64_t(1) << 16, (int64_t(1) << 15) - 1}}, "2^16 x (2^15 - 1)", 28);
  run_list({{716064, 2999}, {1, 1}, {2999, 1}}, "716064 x 2999 and small ones", 28);
  run_list({}, "empty list", 28);
  run_sharded({{16, 64}, {1, 100}, {1, 7}, {300, 5}}, 8, "row shards, one eighth");
  run_sharded({{1, 2048}, {2, 3}}, 1, "row shards, one rank");
  run_sharded({}, 4, "row shards, empty list");
  std::mt19937_64 rng(20261202);
  int lists = 6;
  for (int k = 0; k < 150; ++k, ++lists) run_list(random_list(rng), "random list " + std::to_string(k), k % 3 ? 28 : 19);
  for (int a = 1; a < argc; ++a, ++lists) run_list(read_list(argv[a]), argv[a], 28);
  std::printf("planner checks: %d lists, %ld plan checks, %d failures\n", lists, g_stub_plan_checks, g_failures);
  return g_failures ? 1 : 0;
}
