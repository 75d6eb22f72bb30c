// C ABI of the small_fc_lopt optimizer step: validation, planning of the
// per-step work lists inside the caller's workspace, and the launch sequence.
//
// The interface follows the PyLO page's "Library design" section: an
// optimizer object holds the learned-optimizer weights and the per-parameter
// accumulators and exposes a step over the parameter list.  Here the caller
// owns all tensors (allocated by PyTorch); the library owns a device copy of
// the MLP weights and nothing else.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <stdexcept>
#include <string>
#include <vector>

#include "../../include/lopt.h"
#include "lopt_internal.h"

using namespace lopt;

namespace {

thread_local std::string g_last_error;

struct ApiError {
  lopt_status code;
  std::string msg;
};

[[noreturn]] void fail(lopt_status code, const std::string& msg) { throw ApiError{code, msg}; }

void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) fail(LOPT_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

template <class F>
lopt_status guarded(F&& f) {
  try {
    f();
    g_last_error.clear();
    return LOPT_OK;
  } catch (const ApiError& e) {
    g_last_error = e.msg;
    return e.code;
  } catch (const std::bad_alloc&) {
    g_last_error = "host allocation failed";
    return LOPT_ERR_HIP;
  } catch (const std::exception& e) {
    g_last_error = e.what();
    return LOPT_ERR_HIP;
  } catch (...) {
    g_last_error = "unknown error";
    return LOPT_ERR_HIP;
  }
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int pow2_log2_ceil(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

// Work lists and workspace layout for one tensor list.
struct Plan {
  std::vector<TensorDesc> desc;
  std::vector<const float*> grads;
  std::vector<Tile0> tiles0;
  std::vector<Seg1> segs1;
  std::vector<Chunk> chunks;
  int32_t n_rseg = 0;
  uint32_t chunk_elems = 0;
  // byte offsets inside the workspace
  size_t off_desc = 0, off_grads = 0, off_tiles0 = 0, off_segs1 = 0, off_chunks = 0;
  size_t off_rbar = 0, off_stats = 0, off_scales = 0, off_packed = 0, off_step = 0, off_sync = 0, off_th = 0;
  size_t off_floats = 0;
  // row shards (lopt_init_state_sharded): the two exchanged buffers
  bool sharded = false;
  size_t off_sums1 = 0, n_sums1 = 0, off_sums2 = 0;
  size_t floats = 0;  // per-tensor float arrays (row/col partials, rq, cq)
  size_t total = 0;
  std::vector<lopt_tensor> bound;
};

void validate_config(const lopt_config* c) {
  if (!c) fail(LOPT_ERR_INVALID_ARGUMENT, "config is NULL");
  auto finite = [](float x) { return std::isfinite(x); };
  for (int a = 0; a < 3; ++a)
    if (!(c->beta_m[a] >= 0.f && c->beta_m[a] <= 1.f) || !(c->beta_f[a] >= 0.f && c->beta_f[a] <= 1.f))
      fail(LOPT_ERR_INVALID_ARGUMENT, "decays must lie in [0, 1]");
  if (!(c->beta_v >= 0.f && c->beta_v <= 1.f)) fail(LOPT_ERR_INVALID_ARGUMENT, "beta_v must lie in [0, 1]");
  if (!(c->eps_v >= 0.f) || !(c->eps_f >= 0.f) || !(c->eps_norm >= 0.f) || !finite(c->eps_v) ||
      !finite(c->eps_f) || !finite(c->eps_norm))
    fail(LOPT_ERR_INVALID_ARGUMENT, "epsilons must be finite and >= 0");
  if (!finite(c->exp_mult) || !finite(c->step_mult) || !finite(c->lr) || !finite(c->weight_decay))
    fail(LOPT_ERR_INVALID_ARGUMENT, "exp_mult, step_mult, lr and weight_decay must be finite");
  if (c->n_time < 0 || c->n_time > LOPT_MAX_TIME) fail(LOPT_ERR_INVALID_ARGUMENT, "n_time must be in 0..11");
  for (int q = 0; q < c->n_time; ++q)
    if (!(c->timescales[q] > 0.f) || !finite(c->timescales[q]))
      fail(LOPT_ERR_INVALID_ARGUMENT, "timescales must be finite and > 0");
  if (c->mlp_impl < LOPT_MLP_AUTO || c->mlp_impl > LOPT_MLP_BF16X8)
    fail(LOPT_ERR_INVALID_ARGUMENT, "unknown mlp_impl");
  if (c->n_feat != LOPT_N_FEATURES && c->n_feat != LOPT_VELO_FEATURES)
    fail(LOPT_ERR_INVALID_ARGUMENT, "n_feat must be 28 or 19");
  if (c->launch < LOPT_LAUNCH_AUTO || c->launch > LOPT_LAUNCH_SINGLE)
    fail(LOPT_ERR_INVALID_ARGUMENT, "unknown launch mode");
}

struct Range {
  uintptr_t a, b;  // [a, b)
  int tensor;
};

// Gradient pointers may be NULL everywhere: lopt_step skips such a tensor.
void validate_tensors(const lopt_tensor* ts, int32_t n) {
  if (n < 0) fail(LOPT_ERR_INVALID_ARGUMENT, "negative tensor count");
  if (n > 0 && !ts) fail(LOPT_ERR_INVALID_ARGUMENT, "tensor list is NULL");
  std::vector<Range> written;
  written.reserve(2 * size_t(n));
  for (int32_t i = 0; i < n; ++i) {
    const lopt_tensor& t = ts[i];
    const std::string at = "tensor " + std::to_string(i) + ": ";
    if (!t.param || !t.state) fail(LOPT_ERR_INVALID_ARGUMENT, at + "NULL param or state");
    if (t.rows < 1 || t.cols < 1) fail(LOPT_ERR_INVALID_ARGUMENT, at + "rows and cols must be >= 1");
    if (t.rows > INT32_MAX || t.cols > INT32_MAX || t.rows * t.cols >= (int64_t(1) << 31))
      fail(LOPT_ERR_UNSUPPORTED, at + "tensors must have fewer than 2^31 elements");
    if (t.rows > 1 && t.cols >= (int64_t(1) << 28))
      fail(LOPT_ERR_UNSUPPORTED, at + "matrices must have fewer than 2^28 columns");
    if ((reinterpret_cast<uintptr_t>(t.param) | reinterpret_cast<uintptr_t>(t.grad) |
         reinterpret_cast<uintptr_t>(t.state)) & 3u)
      fail(LOPT_ERR_UNSUPPORTED, at + "pointers must be 4-byte aligned");
    const size_t ne = size_t(t.rows * t.cols);
    const size_t ns = lopt_state_floats(t.rows, t.cols);
    const uintptr_t p = reinterpret_cast<uintptr_t>(t.param);
    const uintptr_t s = reinterpret_cast<uintptr_t>(t.state);
    written.push_back({p, p + 4 * ne, i});
    written.push_back({s, s + 4 * ns, i});
  }
  std::sort(written.begin(), written.end(), [](const Range& x, const Range& y) { return x.a < y.a; });
  for (size_t k = 1; k < written.size(); ++k)
    if (written[k].a < written[k - 1].b)
      fail(LOPT_ERR_INVALID_ARGUMENT, "param/state buffers of tensors " + std::to_string(written[k - 1].tensor) +
                                          " and " + std::to_string(written[k].tensor) + " overlap");
  for (int32_t i = 0; i < n; ++i) {
    if (!ts[i].grad) continue;
    const uintptr_t g = reinterpret_cast<uintptr_t>(ts[i].grad);
    const uintptr_t ge = g + 4 * size_t(ts[i].rows * ts[i].cols);
    // first written range that ends after g
    auto it = std::upper_bound(written.begin(), written.end(), g,
                               [](uintptr_t v, const Range& r) { return v < r.a; });
    if (it != written.begin()) {
      auto prev = std::prev(it);
      if (prev->b > g) fail(LOPT_ERR_INVALID_ARGUMENT, "grad of tensor " + std::to_string(i) + " overlaps a written buffer");
    }
    if (it != written.end() && it->a < ge)
      fail(LOPT_ERR_INVALID_ARGUMENT, "grad of tensor " + std::to_string(i) + " overlaps a written buffer");
  }
}

// sharded: a row-shard binding, with global_dims the (rows, cols) of the
// whole tensor each list entry is a shard of (validated by the caller).
Plan build_plan(const lopt_tensor* ts, int32_t n, bool sharded = false, const int64_t* global_dims = nullptr) {
  validate_tensors(ts, n);
  Plan pl;
  pl.sharded = sharded;
  if (!sharded) global_dims = nullptr;
  pl.bound.assign(ts, ts + n);
  pl.desc.resize(n);
  pl.grads.resize(n);
  size_t fl = 0;  // floats of per-tensor arrays
  int32_t rseg = 0;
  uint64_t total = 0;
  for (int32_t ti = 0; ti < n; ++ti) total += uint64_t(ts[ti].rows * ts[ti].cols);
  const uint64_t chunk = std::min<uint64_t>(
      kChunkElems, std::max<uint64_t>(kMinChunkElems, align_up((total + kTargetChunks - 1) / kTargetChunks, 256)));
  pl.chunk_elems = uint32_t(chunk);
  for (int32_t ti = 0; ti < n; ++ti) {
    const lopt_tensor& t = ts[ti];
    TensorDesc& d = pl.desc[ti];
    std::memset(&d, 0, sizeof(d));
    d.p = t.param;
    d.st = t.state;
    d.R = int32_t(t.rows);
    d.C = int32_t(t.cols);
    d.n = uint32_t(t.rows * t.cols);
    // a shard of a matrix stays a matrix even when it holds one row
    d.vec = global_dims ? global_dims[2 * ti] == 1 : t.rows == 1;
    d.Rg = global_dims ? global_dims[2 * ti] : int64_t(d.R);
    d.ng = global_dims ? global_dims[2 * ti] * global_dims[2 * ti + 1] : int64_t(d.n);
    d.off_sum1 = int64_t(pl.n_sums1);
    pl.n_sums1 += d.vec ? 1 : size_t(d.C);
    fastdiv_magic(uint32_t(d.C), &d.cmagic, &d.cshift);
    // host check of the divisor constants at the edges of the index range
    for (uint64_t e : {uint64_t(0), uint64_t(d.C) - 1, uint64_t(d.C), uint64_t(d.n) - 1,
                       uint64_t(d.n) - uint64_t(d.C), uint64_t(d.n) / 2}) {
      if (e >= d.n) continue;
      const uint32_t q = uint32_t(((uint64_t(e) * d.cmagic >> 32) + e) >> d.cshift);
      if (q != e / uint64_t(d.C)) fail(LOPT_ERR_UNSUPPORTED, "internal: division constants failed check");
    }
    pl.grads[ti] = t.grad;

    // row/column sum tiles
    if (d.vec) {
      const int32_t nt = int32_t((int64_t(d.n) + kTile0Elems - 1) / kTile0Elems);
      d.ncw = nt;
      d.nrb = 0;
      for (int32_t q = 0; q < nt; ++q) {
        Tile0 tl{};
        tl.tensor = ti;
        tl.flat = 1;
        tl.c0 = q * kTile0Elems;
        tl.c1 = int32_t(std::min<int64_t>(int64_t(q + 1) * kTile0Elems, d.n));
        tl.win = q;
        pl.tiles0.push_back(tl);
      }
    } else {
      const int cwl = std::min(8, pow2_log2_ceil(d.C));
      const int CW = 1 << cwl;
      const int RS = kBlock / CW;
      const int ncw = (d.C + CW - 1) / CW;
      int TR = RS * kTile0Iters;  // rows per tile
      while (TR > RS && int64_t(TR / 2) * CW >= kTile0Elems) TR /= 2;
      const int nrb = (d.R + TR - 1) / TR;
      d.ncw = ncw;
      d.nrb = nrb;
      for (int b = 0; b < nrb; ++b)
        for (int w = 0; w < ncw; ++w) {
          Tile0 tl{};
          tl.tensor = ti;
          tl.flat = 0;
          tl.r0 = b * TR;
          tl.r1 = std::min(d.R, (b + 1) * TR);
          tl.c0 = w * CW;
          tl.c1 = std::min(d.C, (w + 1) * CW);
          tl.cw_log2 = cwl;
          tl.rb = b;
          tl.win = w;
          pl.tiles0.push_back(tl);
        }
    }
    // per-tensor float arrays
    d.off_rowpart = int64_t(fl);
    fl += size_t(d.ncw) * d.R;
    d.off_colpart = int64_t(fl);
    fl += size_t(d.nrb) * d.C;
    fl = align_up(fl, 4);
    d.off_rq = int64_t(fl);
    fl += 4 * size_t(d.R);
    d.off_cq = int64_t(fl);
    fl += d.vec ? 0 : 4 * size_t(d.C);

    // moving-average segments
    d.rseg0 = rseg;
    if (d.vec) {
      pl.segs1.push_back(Seg1{ti, kSegVec, 0, 1, rseg, {0, 0, 0}});
      d.nrseg = 1;
      ++rseg;
    } else {
      d.nrseg = (d.R + kSeg1 - 1) / kSeg1;
      for (int a = 0; a < d.R; a += kSeg1)
        pl.segs1.push_back(Seg1{ti, kSegRows, a, std::min(d.R, a + kSeg1), rseg++, {0, 0, 0}});
      for (int a = 0; a < d.C; a += kSegCols1)
        pl.segs1.push_back(Seg1{ti, kSegCols, a, std::min(d.C, a + kSegCols1), -1, {0, 0, 0}});
    }

    // statistics / apply chunks
    d.chunk0 = int32_t(pl.chunks.size());
    for (uint64_t e = 0; e < d.n; e += chunk)
      pl.chunks.push_back(Chunk{ti, uint32_t(e), uint32_t(std::min<uint64_t>(e + chunk, d.n)),
                                uint32_t(e / uint64_t(d.C))});
    d.nchunk = int32_t(pl.chunks.size()) - d.chunk0;
  }
  pl.n_rseg = rseg;
  pl.floats = fl;

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  pl.off_desc = take(sizeof(TensorDesc) * pl.desc.size());
  pl.off_grads = take(sizeof(const float*) * pl.grads.size());
  pl.off_tiles0 = take(sizeof(Tile0) * pl.tiles0.size());
  pl.off_segs1 = take(sizeof(Seg1) * pl.segs1.size());
  pl.off_chunks = take(sizeof(Chunk) * pl.chunks.size());
  pl.off_rbar = take(sizeof(float) * 4 * size_t(pl.n_rseg));
  pl.off_stats = take(sizeof(float) * kStatStride * pl.chunks.size());
  pl.off_scales = take(sizeof(float) * kStatStride * pl.desc.size());
  pl.off_packed = take(sizeof(float) * kPkFloats);
  pl.off_step = take(sizeof(int64_t));
  pl.off_sync = take(sizeof(uint32_t) * kSyncWords);
  pl.off_th = take(sizeof(float) * 2 * pl.desc.size());
  pl.off_floats = take(sizeof(float) * pl.floats);
  if (pl.sharded) {
    pl.off_sums1 = take(sizeof(float) * pl.n_sums1);
    pl.off_sums2 = take(sizeof(float) * kStatStride * pl.desc.size());
  }
  pl.total = off;
  // per-tensor float offsets are relative to the workspace base
  const int64_t base = int64_t(pl.off_floats / sizeof(float));
  for (auto& d : pl.desc) {
    d.off_rowpart += base;
    d.off_colpart += base;
    d.off_rq += base;
    d.off_cq += base;
  }
  return pl;
}

// The fp16x3 path's power-of-two exponents (computed by fp16x3_scales)
struct X3Scales {
  int32_t shift = -1;  // constant layer-1 entries: 2^-shift against a B value of 2^shift
  int32_t w1 = 0;      // W1 enters the A operand times 2^w1
  int32_t w2 = 0;      // W2 enters the A operand times 2^w2
};

}  // namespace

struct lopt_handle {
  lopt_config cfg{};
  int device = 0;
  float* d_mlp = nullptr;
  // fp16x3 path: its scalings (shift -1 when the weights do not fit)
  X3Scales x3;
  bool bound = false;
  Plan plan;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  std::vector<hipEvent_t> events;  // optional timing events (kNumKernels + 1)
  // Per-tensor learning rates and weight decays (lopt_set_tensor_hyper).
  bool th_active = false;          // the step uses them instead of cfg.lr / cfg.weight_decay
  bool th_dirty = false;           // the device copy is out of date
  std::vector<float> th_lr, th_wd;
  // Uploads between steps (gradient pointers, per-tensor pairs): two slots of
  // pinned host memory used in turn, each [cap pointers][cap x 2 floats];
  // slot_done[k] is recorded after the copies that last read slot k.
  char* staging = nullptr;
  size_t staging_cap = 0;          // tensors per slot
  hipEvent_t slot_done[2] = {nullptr, nullptr};
  int next_slot = 0;
  // Bound with lopt_init_state_static: the plan lives in the device's static
  // scratch array (shared by every handle on that device) and changes between
  // steps are copied from host memory without pinned slots.
  bool static_ws = false;
  // Row-shard binding: the phase lopt_step_shard runs next (0, 1, 2).
  int32_t shard_next = 0;
};

namespace {

// The handle whose list the static scratch array of each device holds.
std::mutex g_scratch_mu;
const lopt_handle* g_scratch_owner[kMaxDevices] = {};

bool owns_scratch(const lopt_handle* h) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return h->device >= 0 && h->device < kMaxDevices && g_scratch_owner[h->device] == h;
}

void set_scratch_owner(const lopt_handle* h, bool own) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (h->device < 0 || h->device >= kMaxDevices) return;
  if (own) g_scratch_owner[h->device] = h;
  else if (g_scratch_owner[h->device] == h) g_scratch_owner[h->device] = nullptr;
}

// A static binding's data is in the shared scratch only while no later static
// binding on its device has replaced it.
void check_static_owner(const lopt_handle* h) {
  if (h->bound && h->static_ws && !owns_scratch(h))
    fail(LOPT_ERR_STATE, "the device's static scratch now holds another binding (lopt_init_state_static was "
                         "called again on this device); bind this list again");
}

// AUTO: bf16x8, measured the fastest of the paths with fp32 arithmetic
// (bf16x8, bf16x9, the fp32 matrix cores, the vector ALU) for any weights
int32_t resolved_mlp_impl(const lopt_handle* h) {
  if (h->cfg.mlp_impl != LOPT_MLP_AUTO) return h->cfg.mlp_impl;
  return LOPT_MLP_BF16X8;
}

// AUTO: the five kernels, measured faster than the one-launch step at every
// list size (its grid-wide barriers each cost more than a kernel boundary)
int32_t resolved_launch(const lopt_handle* h) {
  if (h->cfg.launch != LOPT_LAUNCH_AUTO) return h->cfg.launch;
  return LOPT_LAUNCH_SPLIT;
}

StepCtx make_ctx(const lopt_handle* h) {
  const Plan& pl = h->plan;
  StepCtx c{};
  c.ws = reinterpret_cast<float*>(h->ws);
  c.desc = reinterpret_cast<const TensorDesc*>(h->ws + pl.off_desc);
  c.grads = reinterpret_cast<const float* const*>(h->ws + pl.off_grads);
  c.tiles0 = reinterpret_cast<const Tile0*>(h->ws + pl.off_tiles0);
  c.segs1 = reinterpret_cast<const Seg1*>(h->ws + pl.off_segs1);
  c.chunks = reinterpret_cast<const Chunk*>(h->ws + pl.off_chunks);
  c.rbar_part = reinterpret_cast<float*>(h->ws + pl.off_rbar);
  c.stats_part = reinterpret_cast<float*>(h->ws + pl.off_stats);
  c.scales = reinterpret_cast<float*>(h->ws + pl.off_scales);
  c.packed = reinterpret_cast<float*>(h->ws + pl.off_packed);
  c.step = reinterpret_cast<int64_t*>(h->ws + pl.off_step);
  c.sync = reinterpret_cast<uint32_t*>(h->ws + pl.off_sync);
  c.sharded = pl.sharded ? 1 : 0;
  c.sums1 = pl.sharded ? reinterpret_cast<float*>(h->ws + pl.off_sums1) : nullptr;
  c.sums2 = pl.sharded ? reinterpret_cast<float*>(h->ws + pl.off_sums2) : nullptr;
  c.tensor_hyper = reinterpret_cast<const float*>(h->ws + pl.off_th);
  c.mlp = h->d_mlp;
  c.n_tensors = int32_t(pl.desc.size());
  c.n_tiles0 = int32_t(pl.tiles0.size());
  c.n_segs1 = int32_t(pl.segs1.size());
  c.n_chunks = int32_t(pl.chunks.size());
  c.mlp_impl = resolved_mlp_impl(h);
  return c;
}

StepParams make_params(const lopt_handle* h) {
  const lopt_config& c = h->cfg;
  StepParams p{};
  for (int a = 0; a < 3; ++a) {
    p.beta_m[a] = c.beta_m[a];
    p.beta_f[a] = c.beta_f[a];
    p.omb_m[a] = 1.0f - c.beta_m[a];
    p.omb_f[a] = 1.0f - c.beta_f[a];
  }
  p.beta_v = c.beta_v;
  p.omb_v = 1.0f - c.beta_v;
  p.eps_v = c.eps_v;
  p.eps_f = c.eps_f;
  p.eps_norm = c.eps_norm;
  p.exp_mult = c.exp_mult;
  p.step_mult = c.step_mult;
  p.lr = c.lr;
  p.weight_decay = c.weight_decay;
  p.decay = 1.0f - c.lr * c.weight_decay;
  p.lr_step = c.lr * c.step_mult;
  p.exp2_mult = float(double(c.exp_mult) * 1.4426950408889634);  // log2(e)
  // Arguments of the per-element 1/sqrt: v + eps_v >= eps_v, and (1-D tensors)
  // beta_f c + (1 - beta_f)(g^2 + eps_f) >= fl((1 - beta_f) eps_f) for c >= 0.
  bool normal = c.eps_v >= 2.0f * FLT_MIN;
  for (int k = 0; k < 3; ++k) normal = normal && p.omb_f[k] * c.eps_f >= 2.0f * FLT_MIN;
  p.rsq_normal = normal ? 1 : 0;
  p.per_tensor = h->th_active ? 1 : 0;
  p.n_time = c.n_time;
  p.n_feat = c.n_feat;
  p.x3_shift = h->x3.shift > 0 ? h->x3.shift : 0;
  p.x3_w1 = h->x3.w1;
  p.x3_w2 = h->x3.w2;
  for (int q = 0; q < kMaxTime; ++q) p.timescales[q] = q < c.n_time ? c.timescales[q] : 1.f;
  return p;
}

template <class T>
void upload(char* ws, size_t off, const std::vector<T>& v, hipStream_t s) {
  if (v.empty()) return;
  hip_check(hipMemcpyAsync(ws + off, v.data(), sizeof(T) * v.size(), hipMemcpyHostToDevice, s),
            "hipMemcpyAsync(plan)");
}

// The handle's weights and workspace live on the device that was current at
// lopt_create; launching from another device would hand its kernels foreign
// pointers.
void check_device(const lopt_handle* h) {
  int dev = -1;
  hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (dev != h->device)
    fail(LOPT_ERR_INVALID_ARGUMENT, "current device " + std::to_string(dev) + " is not the handle's device " +
                                        std::to_string(h->device));
}

// Waits until no queued copy reads the pinned staging slots.
void drain_slots(lopt_handle* h) {
  for (hipEvent_t e : h->slot_done)
    if (e) hip_check(hipEventSynchronize(e), "hipEventSynchronize(staging slot)");
}

size_t slot_bytes(size_t cap) { return cap * (sizeof(const float*) + 2 * sizeof(float)); }

// Pinned staging slots for n tensors, and their events (created once).
void reserve_slots(lopt_handle* h, size_t n) {
  for (hipEvent_t& e : h->slot_done)
    if (!e) hip_check(hipEventCreateWithFlags(&e, hipEventDisableTiming), "hipEventCreate");
  if (n <= h->staging_cap && h->staging) return;
  // allocate first: on failure the handle keeps its old slots
  const size_t cap = std::max<size_t>(n, 1);
  void* p = nullptr;
  hip_check(hipHostMalloc(&p, 2 * slot_bytes(cap), hipHostMallocDefault), "hipHostMalloc(staging slots)");
  drain_slots(h);
  if (h->staging) (void)hipHostFree(h->staging);
  h->staging = static_cast<char*>(p);
  h->staging_cap = cap;
}

// Queues, on s, the copies of whatever changed since the last step into the
// plan's tables: the gradient pointers of ts and/or the per-tensor (decay,
// lr_step) pairs.  The source is a pinned slot that no queued copy still
// reads, so the host does not wait for the stream.
void upload_changes(lopt_handle* h, const lopt_tensor* ts, int32_t n, bool grads, bool pairs, hipStream_t s) {
  if (!h->staging) {
    // no pinned slots (a static binding): copy from the handle's host memory
    // and wait for the stream, so the host copy can change afterwards
    std::vector<float> th;
    if (grads)
      for (int32_t i = 0; i < n; ++i) {
        h->plan.grads[i] = ts[i].grad;
        h->plan.bound[i].grad = ts[i].grad;
      }
    if (grads && n > 0)
      hip_check(hipMemcpyAsync(h->ws + h->plan.off_grads, h->plan.grads.data(), sizeof(const float*) * size_t(n),
                               hipMemcpyHostToDevice, s),
                "hipMemcpyAsync(gradient pointers)");
    if (pairs && n > 0) {
      th.resize(2 * size_t(n));
      for (int32_t i = 0; i < n; ++i) {
        th[2 * i] = 1.0f - h->th_lr[i] * h->th_wd[i];
        th[2 * i + 1] = h->th_lr[i] * h->cfg.step_mult;
      }
      hip_check(hipMemcpyAsync(h->ws + h->plan.off_th, th.data(), th.size() * sizeof(float), hipMemcpyHostToDevice, s),
                "hipMemcpyAsync(per-tensor hyperparameters)");
    }
    hip_check(hipStreamSynchronize(s), "hipStreamSynchronize(upload)");
    if (pairs) h->th_dirty = false;
    return;
  }
  const int k = h->next_slot;
  hip_check(hipEventSynchronize(h->slot_done[k]), "hipEventSynchronize(staging slot)");
  char* slot = h->staging + size_t(k) * slot_bytes(h->staging_cap);
  if (grads) {
    const float** gp = reinterpret_cast<const float**>(slot);
    for (int32_t i = 0; i < n; ++i) gp[i] = ts[i].grad;
    hip_check(hipMemcpyAsync(h->ws + h->plan.off_grads, gp, sizeof(const float*) * size_t(n), hipMemcpyHostToDevice, s),
              "hipMemcpyAsync(gradient pointers)");
  }
  if (pairs) {
    float* th = reinterpret_cast<float*>(slot + sizeof(const float*) * h->staging_cap);
    for (int32_t i = 0; i < n; ++i) {
      // the same fp32 expressions as the whole-list values in make_params
      th[2 * i] = 1.0f - h->th_lr[i] * h->th_wd[i];
      th[2 * i + 1] = h->th_lr[i] * h->cfg.step_mult;
    }
    hip_check(hipMemcpyAsync(h->ws + h->plan.off_th, th, 2 * sizeof(float) * size_t(n), hipMemcpyHostToDevice, s),
              "hipMemcpyAsync(per-tensor hyperparameters)");
  }
  hip_check(hipEventRecord(h->slot_done[k], s), "hipEventRecord(staging slot)");
  h->next_slot = k ^ 1;
  if (grads)
    for (int32_t i = 0; i < n; ++i) {
      h->plan.grads[i] = ts[i].grad;
      h->plan.bound[i].grad = ts[i].grad;
    }
  if (pairs) h->th_dirty = false;
}

void check_same_list(const lopt_handle* h, const lopt_tensor* ts, int32_t n, bool* grads_changed) {
  if (!h->bound) fail(LOPT_ERR_STATE, "lopt_init_state has not been called");
  const auto& b = h->plan.bound;
  if (n != int32_t(b.size())) fail(LOPT_ERR_STATE, "tensor count differs from lopt_init_state");
  if (n > 0 && !ts) fail(LOPT_ERR_INVALID_ARGUMENT, "tensor list is NULL");
  *grads_changed = false;
  for (int32_t i = 0; i < n; ++i) {
    if (ts[i].param != b[i].param || ts[i].state != b[i].state || ts[i].rows != b[i].rows ||
        ts[i].cols != b[i].cols)
      fail(LOPT_ERR_STATE, "tensor " + std::to_string(i) + " differs from lopt_init_state");
    if (ts[i].grad != b[i].grad) *grads_changed = true;
  }
  if (*grads_changed) validate_tensors(ts, n);
}

// The fp16x3 path's power-of-two scalings.  Each weight matrix W1, W2 enters
// the A operand times 2^a, a in [0, 24], with a as large as puts its largest
// magnitude in [4, 8) (never scaled down): the fp16 low pieces of its smaller
// weights then stay out of fp16's subnormal range.  ReLU commutes with the
// positive factor, so layer 2 starts from b2 2^(a1 + a2) and layer 3 reads
// W3 2^-(a1 + a2) (exact in fp32).  The constant layer-1 entries,
// (b1' + row term) / 2 with b1' = b1 plus the step features (|tanh| <= 1) and
// the row term the three normalised row features (each at most
// sqrt(n) < 46341 for n < 2^31) times their weights, carry 2^a1 too (a1 is
// lowered while their bound would need k > 14); shift is the smallest k with
// that bound * 2^(a1 - k) < 2^15, or -1 when k would exceed 14 or a weight
// has magnitude 2^15 or more.
X3Scales fp16x3_scales(const float* mlp, int32_t n_feat, int32_t n_time) {
  X3Scales x;
  const int din = n_feat + n_time;
  const size_t nw = lopt_mlp_floats(n_feat, n_time);
  for (size_t i = 0; i < nw; ++i)
    if (!(std::fabs(mlp[i]) < 32768.f)) return x;
  const float* W1 = mlp;
  const float* b1 = W1 + kH * din;
  const float* W2 = b1 + kH;
  // 3 - e for the largest magnitude m = f 2^e, f in [0.5, 1): m 2^(3 - e) in [4, 8)
  auto to_four = [](float m) {
    int e = 0;
    (void)std::frexp(m, &e);
    return m > 0.f ? std::min(std::max(3 - e, 0), 24) : 0;
  };
  float m1 = 0.f, m2 = 0.f;
  for (int u = 0; u < kH; ++u)
    for (int f = 0; f < n_feat; ++f) m1 = std::max(m1, std::fabs(W1[u * din + f]));
  for (int i = 0; i < kH * kH; ++i) m2 = std::max(m2, std::fabs(W2[i]));
  x.w1 = to_four(m1);
  x.w2 = to_four(m2);
  double bound = 0.0;
  for (int u = 0; u < kH; ++u) {
    double c = std::fabs(double(b1[u]));
    for (int s = 0; s < n_time; ++s) c += std::fabs(double(W1[u * din + n_feat + s]));
    for (int k = 0; k < 3; ++k) c += 46341.0 * std::fabs(double(W1[u * din + 13 + k]));
    bound = std::max(bound, 0.5 * c * 1.001);
  }
  while (x.w1 > 0 && std::ldexp(bound, x.w1) >= std::ldexp(32768.0, 14)) --x.w1;
  bound = std::ldexp(bound, x.w1);
  int32_t k = 0;
  while (bound * std::ldexp(1.0, -k) >= 32768.0) ++k;
  x.shift = k <= 14 ? k : -1;
  return x;
}

void check_fp16x3(const lopt_handle* h, const lopt_config* cfg) {
  if (cfg->mlp_impl == LOPT_MLP_FP16X3 && h->x3.shift < 0)
    fail(LOPT_ERR_UNSUPPORTED, "the MLP weights are too large for mlp_impl = LOPT_MLP_FP16X3");
}

}  // namespace

extern "C" {

lopt_status lopt_default_config(lopt_config* out) {
  return guarded([&] {
    if (!out) fail(LOPT_ERR_INVALID_ARGUMENT, "out is NULL");
    lopt_config c{};
    c.beta_m[0] = 0.1f; c.beta_m[1] = 0.5f; c.beta_m[2] = 0.9f;
    c.beta_v = 0.999f;
    c.beta_f[0] = 0.9f; c.beta_f[1] = 0.99f; c.beta_f[2] = 0.999f;
    c.eps_v = 1e-8f;
    c.eps_f = 1e-20f;
    c.eps_norm = 1e-30f;
    c.exp_mult = 1e-3f;
    c.step_mult = 1e-3f;
    c.lr = 1.f;
    c.weight_decay = 0.f;
    c.n_time = 11;
    const float ts[LOPT_MAX_TIME] = {1.f, 3.f, 10.f, 30.f, 100.f, 300.f, 1e3f, 3e3f, 1e4f, 3e4f, 1e5f};
    std::memcpy(c.timescales, ts, sizeof(ts));
    c.mlp_impl = LOPT_MLP_AUTO;
    c.n_feat = LOPT_N_FEATURES;
    c.launch = LOPT_LAUNCH_AUTO;
    *out = c;
  });
}

size_t lopt_mlp_floats(int32_t n_feat, int32_t n_time) {
  if (n_time < 0 || n_time > LOPT_MAX_TIME) return 0;
  if (n_feat != LOPT_N_FEATURES && n_feat != LOPT_VELO_FEATURES) return 0;
  const size_t din = size_t(n_feat + n_time);
  return size_t(kH) * din + kH + size_t(kH) * kH + kH + 2 * kH + 2;
}

size_t lopt_state_floats(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 1 || rows > INT32_MAX || cols > INT32_MAX) return 0;
  return size_t(4 * rows * cols + 3 * (rows + cols));
}

lopt_status lopt_create(const lopt_config* cfg, const float* mlp_host, lopt_handle** out) {
  return guarded([&] {
    if (!out) fail(LOPT_ERR_INVALID_ARGUMENT, "out is NULL");
    if (!mlp_host) fail(LOPT_ERR_INVALID_ARGUMENT, "mlp_host is NULL");
    validate_config(cfg);
    const size_t nw = lopt_mlp_floats(cfg->n_feat, cfg->n_time);
    for (size_t i = 0; i < nw; ++i)
      if (!std::isfinite(mlp_host[i])) fail(LOPT_ERR_INVALID_ARGUMENT, "MLP weights must be finite");
    auto* h = new lopt_handle();
    h->cfg = *cfg;
    h->x3 = fp16x3_scales(mlp_host, cfg->n_feat, cfg->n_time);
    try {
      check_fp16x3(h, cfg);
      hip_check(hipGetDevice(&h->device), "hipGetDevice");
      hip_check(hipMalloc(reinterpret_cast<void**>(&h->d_mlp), nw * sizeof(float)), "hipMalloc(weights)");
      hip_check(hipMemcpy(h->d_mlp, mlp_host, nw * sizeof(float), hipMemcpyHostToDevice), "hipMemcpy(weights)");
    } catch (...) {
      if (h->d_mlp) (void)hipFree(h->d_mlp);
      delete h;
      throw;
    }
    *out = h;
  });
}

void lopt_destroy(lopt_handle* h) {
  if (!h) return;
  set_scratch_owner(h, false);
  for (hipEvent_t e : h->slot_done)
    if (e) {
      (void)hipEventSynchronize(e);
      (void)hipEventDestroy(e);
    }
  if (h->staging) (void)hipHostFree(h->staging);
  if (h->d_mlp) (void)hipFree(h->d_mlp);
  delete h;
}

lopt_status lopt_workspace_bytes(const lopt_handle* h, const lopt_tensor* ts, int32_t n, size_t* bytes) {
  return guarded([&] {
    (void)h;  // the plan depends only on the tensor list
    if (!bytes) fail(LOPT_ERR_INVALID_ARGUMENT, "NULL output");
    Plan pl = build_plan(ts, n);
    *bytes = pl.total;
  });
}

namespace {

// The whole tensors of a row-shard binding: (rows, cols) per list entry; a
// 2-D shard holds all columns and some rows, a 1-D shard some elements.
void validate_global_dims(const lopt_tensor* ts, int32_t n, const int64_t* dims) {
  if (n > 0 && !dims) fail(LOPT_ERR_INVALID_ARGUMENT, "global_dims is NULL");
  for (int32_t i = 0; i < n; ++i) {
    const int64_t R = dims[2 * i], C = dims[2 * i + 1];
    const std::string at = "tensor " + std::to_string(i) + ": ";
    if (R < 1 || C < 1 || R > (int64_t(1) << 40) || C > (int64_t(1) << 40))
      fail(LOPT_ERR_INVALID_ARGUMENT, at + "global dims must lie in [1, 2^40]");
    if (R == 1) {
      if (ts[i].rows != 1 || ts[i].cols > C)
        fail(LOPT_ERR_INVALID_ARGUMENT, at + "a shard of a 1-D tensor is 1 x (at most its length)");
    } else {
      if (ts[i].cols != C || ts[i].rows > R)
        fail(LOPT_ERR_INVALID_ARGUMENT, at + "a shard of a matrix holds all of its columns and at most its rows");
      if (C >= (int64_t(1) << 28)) fail(LOPT_ERR_UNSUPPORTED, at + "matrices must have fewer than 2^28 columns");
    }
  }
}

// Binds a planned list to a workspace (a caller's, or the static scratch):
// uploads the plan, zeroes the state, resets the step counter.
void bind_plan(lopt_handle* h, Plan&& pl, char* ws, size_t ws_bytes, bool static_ws, hipStream_t s) {
  if (!static_ws) reserve_slots(h, pl.bound.size());
  drain_slots(h);  // a queued copy of the previous binding may still target its workspace
  const std::vector<int64_t> step0{0};
  const std::vector<uint32_t> sync0(kSyncWords, 0u);
  upload(ws, pl.off_desc, pl.desc, s);
  upload(ws, pl.off_grads, pl.grads, s);
  upload(ws, pl.off_tiles0, pl.tiles0, s);
  upload(ws, pl.off_segs1, pl.segs1, s);
  upload(ws, pl.off_chunks, pl.chunks, s);
  upload(ws, pl.off_step, step0, s);
  upload(ws, pl.off_sync, sync0, s);
  hip_check(hipStreamSynchronize(s), "hipStreamSynchronize(plan upload)");
  h->plan = std::move(pl);
  h->ws = ws;
  h->ws_bytes = ws_bytes;
  h->bound = true;
  h->static_ws = static_ws;
  h->shard_next = 0;
  set_scratch_owner(h, static_ws);
  h->th_active = h->th_dirty = false;  // per-tensor values belong to the previous list
  h->th_lr.clear();
  h->th_wd.clear();
  hip_check(launch_zero_state(make_ctx(h), s), "launch(zero state)");
}

void bind_workspace(lopt_handle* h, Plan&& pl, void* workspace, size_t ws_bytes, void* stream) {
  if (pl.total > 0 && !workspace) fail(LOPT_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) fail(LOPT_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < pl.total)
    fail(LOPT_ERR_WORKSPACE, "workspace too small: need " + std::to_string(pl.total) + " bytes");
  bind_plan(h, std::move(pl), static_cast<char*>(workspace), ws_bytes, false, static_cast<hipStream_t>(stream));
}

}  // namespace

lopt_status lopt_init_state(lopt_handle* h, const lopt_tensor* ts, int32_t n, void* workspace, size_t ws_bytes,
                            void* stream) {
  return guarded([&] {
    if (!h) fail(LOPT_ERR_INVALID_ARGUMENT, "handle is NULL");
    check_device(h);
    bind_workspace(h, build_plan(ts, n), workspace, ws_bytes, stream);
  });
}

lopt_status lopt_workspace_bytes_sharded(const lopt_handle* h, const lopt_tensor* ts, int32_t n,
                                         const int64_t* global_dims, size_t* bytes) {
  return guarded([&] {
    (void)h;
    if (!bytes) fail(LOPT_ERR_INVALID_ARGUMENT, "NULL output");
    validate_tensors(ts, n);
    validate_global_dims(ts, n, global_dims);
    *bytes = build_plan(ts, n, true, global_dims).total;
  });
}

lopt_status lopt_init_state_sharded(lopt_handle* h, const lopt_tensor* ts, int32_t n, const int64_t* global_dims,
                                    void* workspace, size_t ws_bytes, void* stream) {
  return guarded([&] {
    if (!h) fail(LOPT_ERR_INVALID_ARGUMENT, "handle is NULL");
    check_device(h);
    validate_tensors(ts, n);
    validate_global_dims(ts, n, global_dims);
    bind_workspace(h, build_plan(ts, n, true, global_dims), workspace, ws_bytes, stream);
  });
}

lopt_status lopt_get_shard_sums(const lopt_handle* h, float** sums1, size_t* n1, float** sums2, size_t* n2) {
  return guarded([&] {
    if (!h || !sums1 || !n1 || !sums2 || !n2) fail(LOPT_ERR_INVALID_ARGUMENT, "NULL argument");
    if (!h->bound || !h->plan.sharded) fail(LOPT_ERR_STATE, "no row-shard binding (lopt_init_state_sharded)");
    check_static_owner(h);
    *sums1 = reinterpret_cast<float*>(h->ws + h->plan.off_sums1);
    *n1 = h->plan.n_sums1;
    *sums2 = reinterpret_cast<float*>(h->ws + h->plan.off_sums2);
    *n2 = size_t(kStatStride) * h->plan.desc.size();
  });
}

lopt_status lopt_step_shard(lopt_handle* h, const lopt_tensor* ts, int32_t n, int32_t phase, void* stream) {
  return guarded([&] {
    if (!h) fail(LOPT_ERR_INVALID_ARGUMENT, "handle is NULL");
    if (!h->bound || !h->plan.sharded) fail(LOPT_ERR_STATE, "no row-shard binding (lopt_init_state_sharded)");
    if (phase != h->shard_next)
      fail(LOPT_ERR_STATE, "shard phase " + std::to_string(phase) + " called where phase " +
                               std::to_string(h->shard_next) + " comes next");
    bool grads_changed = false;
    check_same_list(h, ts, n, &grads_changed);
    check_device(h);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool pairs_changed = h->th_active && h->th_dirty;
    if (phase == 0 && (grads_changed || pairs_changed)) {
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      hip_check(hipStreamIsCapturing(s, &cs), "hipStreamIsCapturing");
      if (cs != hipStreamCaptureStatusNone)
        fail(LOPT_ERR_INVALID_ARGUMENT,
             "gradient pointers or per-tensor hyperparameters changed while the stream is being captured: "
             "step once with them before capturing");
      upload_changes(h, ts, n, grads_changed, pairs_changed, s);
    } else if (phase != 0 && grads_changed) {
      fail(LOPT_ERR_STATE, "gradient pointers changed between the phases of a step");
    }
    hip_check(launch_shard_phase(make_ctx(h), make_params(h), phase, s, h->events.empty() ? nullptr : h->events.data()),
              "launch(shard phase)");
    h->shard_next = (phase + 1) % 3;
  });
}

lopt_status lopt_init_state_static(lopt_handle* h, const lopt_tensor* ts, int32_t n, void* stream) {
  return guarded([&] {
    if (!h) fail(LOPT_ERR_INVALID_ARGUMENT, "handle is NULL");
    check_device(h);
    Plan pl = build_plan(ts, n);
    if (pl.total > kScratchBytes)
      fail(LOPT_ERR_WORKSPACE, "the tensor list needs " + std::to_string(pl.total) +
                                   " bytes of workspace; the static scratch holds " + std::to_string(kScratchBytes) +
                                   ": use lopt_init_state with a workspace");
    void* scratch = nullptr;
    hip_check(scratch_address(h->device, &scratch), "hipGetSymbolAddress(scratch)");
    bind_plan(h, std::move(pl), static_cast<char*>(scratch), kScratchBytes, true, static_cast<hipStream_t>(stream));
  });
}

lopt_status lopt_step(lopt_handle* h, const lopt_tensor* ts, int32_t n, void* stream) {
  return guarded([&] {
    if (!h) fail(LOPT_ERR_INVALID_ARGUMENT, "handle is NULL");
    bool grads_changed = false;
    check_same_list(h, ts, n, &grads_changed);
    check_static_owner(h);
    check_device(h);
    if (h->plan.sharded)
      fail(LOPT_ERR_STATE, "a row-shard binding steps with lopt_step_shard (phases 0, 1, 2 with the exchanges "
                           "between them)");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool pairs_changed = h->th_active && h->th_dirty;
    if (grads_changed || pairs_changed) {
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      hip_check(hipStreamIsCapturing(s, &cs), "hipStreamIsCapturing");
      if (cs != hipStreamCaptureStatusNone)
        fail(LOPT_ERR_INVALID_ARGUMENT,
             "gradient pointers or per-tensor hyperparameters changed while the stream is being captured: "
             "step once with them before capturing");
      upload_changes(h, ts, n, grads_changed, pairs_changed, s);
    }
    const StepParams p = make_params(h);
    const StepCtx c = make_ctx(h);
    const hipEvent_t* ev = h->events.empty() ? nullptr : h->events.data();
    if (resolved_launch(h) == LOPT_LAUNCH_SINGLE) {
      int cap = 0;
      hip_check(single_grid_cap(h->device, c.mlp_impl, &cap), "occupancy query (one-launch step)");
      const int work = std::max(std::max(c.n_tiles0, c.n_segs1), std::max(c.n_chunks, c.n_tensors + 1));
      hip_check(launch_single(c, p, std::min(std::min(cap, work), kSingleMaxBlocks), s, ev),
                "launch(one-launch step)");
    } else {
      hip_check(launch_step(c, p, s, ev), "launch(step)");
    }
  });
}

lopt_status lopt_get_step(const lopt_handle* h, int64_t* t) {
  return guarded([&] {
    if (!h || !t) fail(LOPT_ERR_INVALID_ARGUMENT, "NULL handle or output");
    if (!h->bound) {
      *t = 0;
      return;
    }
    check_static_owner(h);
    hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize");
    hip_check(hipMemcpy(t, h->ws + h->plan.off_step, sizeof(int64_t), hipMemcpyDeviceToHost), "hipMemcpy(step)");
    uint32_t fault = 0;
    hip_check(hipMemcpy(&fault, h->ws + h->plan.off_sync + sizeof(uint32_t) * kSyncFault, sizeof(fault),
                        hipMemcpyDeviceToHost), "hipMemcpy(sync)");
    if (fault)
      fail(LOPT_ERR_HIP, "a one-launch step's grid barrier timed out: its blocks were not all resident at once "
                         "(another kernel held the device); the results of that step are not valid");
  });
}

lopt_status lopt_set_step(lopt_handle* h, int64_t t) {
  return guarded([&] {
    if (!h) fail(LOPT_ERR_INVALID_ARGUMENT, "handle is NULL");
    if (t < 0) fail(LOPT_ERR_INVALID_ARGUMENT, "step must be >= 0");
    if (!h->bound) fail(LOPT_ERR_STATE, "lopt_init_state has not been called");
    check_static_owner(h);
    hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize");
    hip_check(hipMemcpy(h->ws + h->plan.off_step, &t, sizeof(int64_t), hipMemcpyHostToDevice), "hipMemcpy(step)");
  });
}

lopt_status lopt_set_config(lopt_handle* h, const lopt_config* cfg) {
  return guarded([&] {
    if (!h) fail(LOPT_ERR_INVALID_ARGUMENT, "handle is NULL");
    validate_config(cfg);
    if (cfg->n_time != h->cfg.n_time || cfg->n_feat != h->cfg.n_feat)
      fail(LOPT_ERR_INVALID_ARGUMENT, "n_feat and n_time are fixed by the MLP weights given to lopt_create");
    check_fp16x3(h, cfg);
    h->cfg = *cfg;
    if (h->th_active) h->th_dirty = true;  // lr_step depends on step_mult
  });
}

lopt_status lopt_get_mlp_impl(const lopt_handle* h, int32_t* impl) {
  return guarded([&] {
    if (!h || !impl) fail(LOPT_ERR_INVALID_ARGUMENT, "NULL argument");
    *impl = resolved_mlp_impl(h);
  });
}

lopt_status lopt_get_launch(const lopt_handle* h, int32_t* launch) {
  return guarded([&] {
    if (!h || !launch) fail(LOPT_ERR_INVALID_ARGUMENT, "NULL argument");
    *launch = resolved_launch(h);
  });
}

lopt_status lopt_set_tensor_hyper(lopt_handle* h, const float* lr, const float* weight_decay, int32_t n) {
  return guarded([&] {
    if (!h) fail(LOPT_ERR_INVALID_ARGUMENT, "handle is NULL");
    if (!h->bound) fail(LOPT_ERR_STATE, "lopt_init_state has not been called");
    if (n != int32_t(h->plan.bound.size())) fail(LOPT_ERR_STATE, "n differs from the bound tensor count");
    if (!lr && !weight_decay) {
      h->th_active = h->th_dirty = false;
      h->th_lr.clear();
      h->th_wd.clear();
      return;
    }
    if (!lr || !weight_decay) fail(LOPT_ERR_INVALID_ARGUMENT, "lr and weight_decay must both be given or both be NULL");
    for (int32_t i = 0; i < n; ++i)
      if (!std::isfinite(lr[i]) || !std::isfinite(weight_decay[i]))
        fail(LOPT_ERR_INVALID_ARGUMENT, "tensor " + std::to_string(i) + ": lr and weight_decay must be finite");
    h->th_lr.assign(lr, lr + n);
    h->th_wd.assign(weight_decay, weight_decay + n);
    h->th_active = n > 0;
    h->th_dirty = h->th_active;
  });
}

lopt_status lopt_get_tensor_stats(const lopt_handle* h, float* out, int32_t n) {
  return guarded([&] {
    if (!h || !out) fail(LOPT_ERR_INVALID_ARGUMENT, "NULL handle or output");
    if (!h->bound) fail(LOPT_ERR_STATE, "lopt_init_state has not been called");
    if (n != int32_t(h->plan.bound.size())) fail(LOPT_ERR_STATE, "n differs from the bound tensor count");
    check_static_owner(h);
    if (n == 0) return;
    // the workspace records: s_d, except s_d sqrt(mean r_k) for the features
    // that carry rho_k in a matrix (the apply pass folds that factor in; a 1-D
    // tensor's rho_k has none), sqrt(mean r_k) at 28..30
    std::vector<float> rec(size_t(n) * kStatStride);
    hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize");
    hip_check(hipMemcpy(rec.data(), h->ws + h->plan.off_scales, rec.size() * sizeof(float), hipMemcpyDeviceToHost),
              "hipMemcpy(tensor statistics)");
    for (int32_t i = 0; i < n; ++i) {
      const float* r = rec.data() + size_t(i) * kStatStride;
      float* o = out + size_t(i) * LOPT_STAT_FLOATS;
      const bool matrix = !h->plan.desc[size_t(i)].vec;   // a one-row shard of a matrix is a matrix
      for (int f = 0; f < kNF; ++f) {
        const int k = rho_feature(f);
        o[f] = (k < 0 || !matrix) ? r[f] : float(double(r[f]) / double(r[kNF + k]));
      }
      for (int k = 0; k < 3; ++k) o[kNF + k] = r[kNF + k];
      o[kNF + 3] = 0.f;
    }
  });
}

lopt_status lopt_set_timing_events(lopt_handle* h, void* const* events, int32_t n) {
  return guarded([&] {
    if (!h) fail(LOPT_ERR_INVALID_ARGUMENT, "handle is NULL");
    if (n == 0) {
      h->events.clear();
      return;
    }
    if (n != kNumKernels + 1 || !events) fail(LOPT_ERR_INVALID_ARGUMENT, "expected LOPT_N_KERNELS + 1 events");
    std::vector<hipEvent_t> ev(n);
    for (int32_t k = 0; k < n; ++k) {
      if (!events[k]) fail(LOPT_ERR_INVALID_ARGUMENT, "NULL event");
      ev[k] = static_cast<hipEvent_t>(events[k]);
    }
    h->events = std::move(ev);
  });
}

const char* lopt_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
