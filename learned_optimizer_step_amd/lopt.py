"""ctypes binding of liblopt (include/lopt.h).  Argument marshalling only.

Every function has the C name and raises ``LoptError`` on a non-OK status.
The library must be built (``python -m learned_optimizer_step_amd.build``);
loading fails loudly when it is missing -- there is no fallback path.

``LOpt`` is a small convenience around the C calls for PyTorch tensors: it
allocates the state buffers and the workspace with torch (device memory is
all torch is used for) and passes raw pointers and the current stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblopt.so")

LOPT_OK = 0
LOPT_ERR_INVALID_ARGUMENT = 1
LOPT_ERR_UNSUPPORTED = 2
LOPT_ERR_WORKSPACE = 3
LOPT_ERR_HIP = 4
LOPT_ERR_STATE = 5
STATUS_NAMES = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP", 5: "STATE"}

LOPT_MLP_AUTO = 0
LOPT_MLP_VALU = 1
LOPT_MLP_MFMA = 2
LOPT_MLP_BF16X6 = 3
LOPT_MLP_FP16X3 = 4
LOPT_MLP_BF16X9 = 5
LOPT_MLP_BF16X8 = 6
LOPT_LAUNCH_AUTO = 0     # LOPT_LAUNCH_SPLIT (measured faster at every size)
LOPT_LAUNCH_SPLIT = 1    # five kernels per step
LOPT_LAUNCH_SINGLE = 2   # one kernel per step (the five passes behind grid-wide barriers)
LOPT_MAX_TIME = 11
LOPT_N_FEATURES = 28     # small_fc_lopt's per-element features
LOPT_VELO_FEATURES = 19  # the VeLO-shaped variant's (features 0..18)


class LoptError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class lopt_config(ctypes.Structure):
    _fields_ = [("beta_m", ctypes.c_float * 3), ("beta_v", ctypes.c_float),
                ("beta_f", ctypes.c_float * 3), ("eps_v", ctypes.c_float),
                ("eps_f", ctypes.c_float), ("eps_norm", ctypes.c_float),
                ("exp_mult", ctypes.c_float), ("step_mult", ctypes.c_float),
                ("lr", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("n_time", ctypes.c_int32), ("timescales", ctypes.c_float * LOPT_MAX_TIME),
                ("mlp_impl", ctypes.c_int32), ("n_feat", ctypes.c_int32), ("launch", ctypes.c_int32)]


class lopt_tensor(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("state", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Loads liblopt.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("LOPT_LIBRARY") or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m learned_optimizer_step_amd.build`")
    try:
        import torch  # noqa: F401  (binds libamdhip64 to torch's copy first)
    except ImportError:
        pass
    lib = ctypes.CDLL(p)
    st = ctypes.c_int
    sig = {
        "lopt_default_config": (st, [ctypes.POINTER(lopt_config)]),
        "lopt_mlp_floats": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32]),
        "lopt_create": (st, [ctypes.POINTER(lopt_config), ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]),
        "lopt_destroy": (None, [ctypes.c_void_p]),
        "lopt_state_floats": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
        "lopt_workspace_bytes": (st, [ctypes.c_void_p, ctypes.POINTER(lopt_tensor), ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_size_t)]),
        "lopt_init_state": (st, [ctypes.c_void_p, ctypes.POINTER(lopt_tensor), ctypes.c_int32,
                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
        "lopt_init_state_static": (st, [ctypes.c_void_p, ctypes.POINTER(lopt_tensor), ctypes.c_int32, ctypes.c_void_p]),
        "lopt_step": (st, [ctypes.c_void_p, ctypes.POINTER(lopt_tensor), ctypes.c_int32, ctypes.c_void_p]),
        "lopt_workspace_bytes_sharded": (st, [ctypes.c_void_p, ctypes.POINTER(lopt_tensor), ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]),
        "lopt_init_state_sharded": (st, [ctypes.c_void_p, ctypes.POINTER(lopt_tensor), ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
        "lopt_get_shard_sums": (st, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_size_t),
                                     ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_size_t)]),
        "lopt_step_shard": (st, [ctypes.c_void_p, ctypes.POINTER(lopt_tensor), ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_void_p]),
        "lopt_get_step": (st, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)]),
        "lopt_set_step": (st, [ctypes.c_void_p, ctypes.c_int64]),
        "lopt_set_timing_events": (st, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]),
        "lopt_set_config": (st, [ctypes.c_void_p, ctypes.POINTER(lopt_config)]),
        "lopt_get_mlp_impl": (st, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)]),
        "lopt_get_launch": (st, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)]),
        "lopt_set_tensor_hyper": (st, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]),
        "lopt_get_tensor_stats": (st, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32]),
        "lopt_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != LOPT_OK:
        raise LoptError(status, lopt_last_error())


def lopt_last_error() -> str:
    return load_library().lopt_last_error().decode()


def lopt_default_config() -> lopt_config:
    c = lopt_config()
    _check(load_library().lopt_default_config(ctypes.byref(c)))
    return c


def lopt_mlp_floats(n_feat: int, n_time: int) -> int:
    return int(load_library().lopt_mlp_floats(n_feat, n_time))


def lopt_state_floats(rows: int, cols: int) -> int:
    return int(load_library().lopt_state_floats(rows, cols))


def lopt_create(cfg: lopt_config, mlp_host: np.ndarray) -> ctypes.c_void_p:
    w = np.ascontiguousarray(mlp_host, dtype=np.float32)
    nw = lopt_mlp_floats(cfg.n_feat, cfg.n_time)
    if w.size != nw:
        raise ValueError(f"expected {nw} MLP floats, got {w.size}")
    h = ctypes.c_void_p()
    _check(load_library().lopt_create(ctypes.byref(cfg), w.ctypes.data_as(ctypes.c_void_p), ctypes.byref(h)))
    return h


def lopt_destroy(h) -> None:
    load_library().lopt_destroy(h)


def tensor_array(ts: Sequence[lopt_tensor]):
    arr = (lopt_tensor * max(1, len(ts)))()
    for i, t in enumerate(ts):
        arr[i] = t
    return arr


def lopt_workspace_bytes(h, ts: Sequence[lopt_tensor]) -> int:
    out = ctypes.c_size_t()
    _check(load_library().lopt_workspace_bytes(h, tensor_array(ts), len(ts), ctypes.byref(out)))
    return int(out.value)


def lopt_init_state(h, ts: Sequence[lopt_tensor], workspace: int, ws_bytes: int, stream: int) -> None:
    _check(load_library().lopt_init_state(h, tensor_array(ts), len(ts), ctypes.c_void_p(workspace),
                                          ws_bytes, ctypes.c_void_p(stream)))


LOPT_STATIC_SCRATCH_BYTES = 64 << 20


def lopt_init_state_static(h, ts: Sequence[lopt_tensor], stream: int) -> None:
    _check(load_library().lopt_init_state_static(h, tensor_array(ts), len(ts), ctypes.c_void_p(stream)))


def lopt_step(h, ts: Sequence[lopt_tensor], stream: int) -> None:
    _check(load_library().lopt_step(h, tensor_array(ts), len(ts), ctypes.c_void_p(stream)))


def _dims_array(global_dims) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(global_dims, dtype=np.int64).reshape(-1))


def lopt_workspace_bytes_sharded(h, ts: Sequence[lopt_tensor], global_dims) -> int:
    """global_dims: (rows, cols) of the whole tensor of each shard."""
    out = ctypes.c_size_t()
    dims = _dims_array(global_dims)
    _check(load_library().lopt_workspace_bytes_sharded(h, tensor_array(ts), len(ts), dims.ctypes.data_as(ctypes.c_void_p),
                                                       ctypes.byref(out)))
    return int(out.value)


def lopt_init_state_sharded(h, ts: Sequence[lopt_tensor], global_dims, workspace: int, ws_bytes: int,
                            stream: int) -> None:
    dims = _dims_array(global_dims)
    _check(load_library().lopt_init_state_sharded(h, tensor_array(ts), len(ts), dims.ctypes.data_as(ctypes.c_void_p),
                                                  ctypes.c_void_p(workspace), ws_bytes, ctypes.c_void_p(stream)))


def lopt_get_shard_sums(h):
    """(sums1 device address, floats, sums2 device address, floats)."""
    p1, p2 = ctypes.c_void_p(), ctypes.c_void_p()
    n1, n2 = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().lopt_get_shard_sums(h, ctypes.byref(p1), ctypes.byref(n1), ctypes.byref(p2), ctypes.byref(n2)))
    return int(p1.value or 0), int(n1.value), int(p2.value or 0), int(n2.value)


def lopt_step_shard(h, ts: Sequence[lopt_tensor], phase: int, stream: int) -> None:
    _check(load_library().lopt_step_shard(h, tensor_array(ts), len(ts), phase, ctypes.c_void_p(stream)))


def lopt_get_step(h) -> int:
    t = ctypes.c_int64()
    _check(load_library().lopt_get_step(h, ctypes.byref(t)))
    return int(t.value)


def lopt_set_step(h, t: int) -> None:
    _check(load_library().lopt_set_step(h, t))


def lopt_set_config(h, cfg: lopt_config) -> None:
    _check(load_library().lopt_set_config(h, ctypes.byref(cfg)))


def lopt_get_mlp_impl(h) -> int:
    """The MLP path the handle's steps run (LOPT_MLP_AUTO resolved)."""
    impl = ctypes.c_int32()
    _check(load_library().lopt_get_mlp_impl(h, ctypes.byref(impl)))
    return int(impl.value)


def lopt_get_launch(h) -> int:
    """How the handle's steps over the bound list are launched (LOPT_LAUNCH_AUTO resolved)."""
    mode = ctypes.c_int32()
    _check(load_library().lopt_get_launch(h, ctypes.byref(mode)))
    return int(mode.value)


def lopt_set_tensor_hyper(h, lr: Optional[Sequence[float]], weight_decay: Optional[Sequence[float]],
                          n: Optional[int] = None) -> None:
    """Per-tensor lr and weight decay for the bound list; (None, None) goes back to the config's."""
    if lr is None and weight_decay is None:
        _check(load_library().lopt_set_tensor_hyper(h, None, None, 0 if n is None else n))
        return
    if lr is None or weight_decay is None:
        raise ValueError("give both lr and weight_decay, or neither")
    a = np.ascontiguousarray(lr, dtype=np.float32)
    b = np.ascontiguousarray(weight_decay, dtype=np.float32)
    if a.shape != b.shape or a.ndim != 1:
        raise ValueError("lr and weight_decay must be 1-D sequences of the same length")
    if n is not None and a.size != n:
        raise ValueError(f"expected {n} values, got {a.size}")
    _check(load_library().lopt_set_tensor_hyper(h, a.ctypes.data_as(ctypes.c_void_p), b.ctypes.data_as(ctypes.c_void_p),
                                                 a.size if n is None else n))


LOPT_STAT_FLOATS = 32


def lopt_get_tensor_stats(h, n: int) -> np.ndarray:
    """(n, LOPT_STAT_FLOATS) float32: per tensor, the feature normalisers s_d of
    its last step (entries 0..27) and sqrt(mean r_k) (28..30)."""
    out = np.zeros((max(n, 0), LOPT_STAT_FLOATS), np.float32)
    _check(load_library().lopt_get_tensor_stats(h, out.ctypes.data_as(ctypes.c_void_p), n))
    return out


LOPT_N_KERNELS = 5
KERNEL_NAMES = ("k_rowcol_sumsq", "k_moving_avg", "k_stats", "k_finalize", "k_apply")


def lopt_set_timing_events(h, events: Sequence[int]) -> None:
    """events: LOPT_N_KERNELS + 1 raw hipEvent_t handles (ints), or [] to stop."""
    arr = (ctypes.c_void_p * max(1, len(events)))(*events)
    _check(load_library().lopt_set_timing_events(h, arr, len(events)))


def config_from(**overrides) -> lopt_config:
    """Default config with fields replaced (lists for the array fields)."""
    c = lopt_default_config()
    for k, v in overrides.items():
        if k in ("beta_m", "beta_f", "timescales"):
            arr = getattr(c, k)
            for i, x in enumerate(v):
                arr[i] = x
        else:
            setattr(c, k, v)
    return c


def matrix_shape(shape) -> tuple:
    """(rows, cols) view of a contiguous tensor: a scalar is 1 x 1, length n is
    1 x n, a matrix stays as given, and a tensor of more dimensions is its first
    dimension by the product of the others (a convolution weight: output
    channels x fan-in)."""
    dims = [int(d) for d in shape]
    if len(dims) == 0:
        return 1, 1
    if len(dims) == 1:
        return 1, dims[0]
    cols = 1
    for d in dims[1:]:
        cols *= d
    return dims[0], cols


# numpy view of an array of lopt_tensor (three pointers and two int64 per entry)
_TENSOR_DTYPE = np.dtype([("param", "<u8"), ("grad", "<u8"), ("state", "<u8"), ("rows", "<i8"), ("cols", "<i8")])


class LOpt:
    """The optimizer over a list of fp32 CUDA (HIP) tensors.

    params: torch tensors (contiguous, float32, all on one device; viewed as
    matrices by ``matrix_shape``).
    mlp: packed fp32 MLP weights (numpy).  cfg: lopt_config.
    The tensor table handed to lopt_step is kept between steps; each step only
    writes the gradient addresses into it.
    """

    def __init__(self, params, mlp: np.ndarray, cfg: Optional[lopt_config] = None, global_dims=None):
        """global_dims: None, or the (rows, cols) of the whole tensor that each
        parameter is a row shard of (lopt_init_state_sharded); such an
        optimizer steps with ``step_sharded``."""
        import torch
        self.torch = torch
        self.params = list(params)
        dev = self.params[0].device if self.params else torch.device("cuda")
        for p in self.params:
            if p.dtype != torch.float32 or not p.is_cuda or not p.is_contiguous() or p.device != dev:
                raise ValueError("parameters must be contiguous float32 tensors on one device")
        self.device = dev
        self.cfg = cfg if cfg is not None else lopt_default_config()
        self.shapes = [matrix_shape(p.shape) for p in self.params]
        self.states = [torch.empty(lopt_state_floats(r, c), dtype=torch.float32, device=dev)
                       for r, c in self.shapes]
        n = len(self.params)
        assert _TENSOR_DTYPE.itemsize == ctypes.sizeof(lopt_tensor)
        self._table = np.zeros(max(1, n), _TENSOR_DTYPE)
        if n:
            self._table["param"][:n] = [p.data_ptr() for p in self.params]
            self._table["state"][:n] = [s.data_ptr() for s in self.states]
            self._table["rows"][:n] = [r for r, _ in self.shapes]
            self._table["cols"][:n] = [c for _, c in self.shapes]
        self._table_ptr = self._table.ctypes.data_as(ctypes.POINTER(lopt_tensor))
        lib = load_library()
        # the handle belongs to the device that is current at lopt_create: the parameters'
        with torch.cuda.device(dev):
            self.handle = lopt_create(self.cfg, mlp)
            ws = ctypes.c_size_t()
            stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
            # gradients are first needed by lopt_step: NULL grad pointers here
            self.global_dims = None if global_dims is None else _dims_array(global_dims)
            if self.global_dims is None:
                _check(lib.lopt_workspace_bytes(self.handle, self._table_ptr, n, ctypes.byref(ws)))
            else:
                if len(self.global_dims) != 2 * n:
                    raise ValueError("global_dims needs (rows, cols) for every parameter")
                dims = self.global_dims.ctypes.data_as(ctypes.c_void_p)
                _check(lib.lopt_workspace_bytes_sharded(self.handle, self._table_ptr, n, dims, ctypes.byref(ws)))
            self.ws_bytes = int(ws.value)
            self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
            wsp = ctypes.c_void_p(self.workspace.data_ptr())
            if self.global_dims is None:
                _check(lib.lopt_init_state(self.handle, self._table_ptr, n, wsp, self.ws_bytes, stream))
            else:
                _check(lib.lopt_init_state_sharded(self.handle, self._table_ptr, n, dims, wsp, self.ws_bytes, stream))

    def _set_grads(self, grads) -> int:
        """Checks the gradients and writes their addresses into the table."""
        grads = list(grads)
        n = len(self.params)
        if len(grads) != n:
            raise ValueError(f"expected {n} gradients, got {len(grads)}")
        f32, dev = self.torch.float32, self.device
        for g, p in zip(grads, self.params):
            if g is not None and (g.dtype != f32 or not g.is_contiguous() or g.numel() != p.numel()
                                  or g.device != dev):
                raise ValueError("gradients must be contiguous float32 tensors shaped like the parameters, "
                                 "on the parameters' device (or None)")
        if n:
            self._table["grad"][:n] = [0 if g is None else g.data_ptr() for g in grads]
        return n

    def step(self, grads) -> None:
        """One step; grads[i] None skips parameter i (it and its state stay as they are)."""
        n = self._set_grads(grads)
        dev = self.device
        with self.torch.cuda.device(dev):
            _check(load_library().lopt_step(self.handle, self._table_ptr, n,
                                            ctypes.c_void_p(self.torch.cuda.current_stream(dev).cuda_stream)))

    def shard_sums(self):
        """The two exchange buffers of a row-shard binding as float32 views of
        the workspace: (column sums of g^2, per-tensor feature sums and sums
        of r_k)."""
        p1, n1, p2, n2 = lopt_get_shard_sums(self.handle)
        base = self.workspace.data_ptr()
        f = self.workspace.view(self.torch.float32)
        return f[(p1 - base) // 4:(p1 - base) // 4 + n1], f[(p2 - base) // 4:(p2 - base) // 4 + n2]

    def step_shard_phase(self, phase: int, grads=None) -> None:
        """Phase 0, 1 or 2 of a row-shard step (lopt_step_shard); the
        gradients are given with phase 0."""
        n = self._set_grads(grads) if phase == 0 else len(self.params)
        with self.torch.cuda.device(self.device):
            stream = ctypes.c_void_p(self.torch.cuda.current_stream(self.device).cuda_stream)
            _check(load_library().lopt_step_shard(self.handle, self._table_ptr, n, phase, stream))

    def step_sharded(self, grads, allreduce) -> None:
        """One step of a row-shard binding: the three phases of lopt_step_shard
        with allreduce(buf) summing each exchange buffer over the ranks in
        place (e.g. torch.distributed.all_reduce) between them.  With one
        rank, allreduce may do nothing."""
        s1, s2 = self.shard_sums()
        self.step_shard_phase(0, grads)
        allreduce(s1)
        self.step_shard_phase(1)
        allreduce(s2)
        self.step_shard_phase(2)

    @property
    def t(self) -> int:
        return lopt_get_step(self.handle)

    @t.setter
    def t(self, value: int) -> None:
        lopt_set_step(self.handle, value)

    def set_tensor_hyper(self, lr: Optional[Sequence[float]], weight_decay: Optional[Sequence[float]]) -> None:
        """Per-parameter lr and weight decay (None, None: the config's for all)."""
        lopt_set_tensor_hyper(self.handle, lr, weight_decay, len(self.params))

    def tensor_stats(self) -> np.ndarray:
        """Per tensor, the feature normalisers of its last step and sqrt(mean r_k)
        (lopt_get_tensor_stats)."""
        return lopt_get_tensor_stats(self.handle, len(self.params))

    def state_views(self, i: int) -> dict:
        """Views of tensor i's state: m (3,R,C), v (R,C), r (3,R), c (3,C)."""
        R, C = self.shapes[i]
        s = self.states[i]
        n = R * C
        return {"m": s[:3 * n].view(3, R, C), "v": s[3 * n:4 * n].view(R, C),
                "r": s[4 * n:4 * n + 3 * R].view(3, R), "c": s[4 * n + 3 * R:].view(3, C)}

    def close(self) -> None:
        if getattr(self, "handle", None) is not None:
            self.torch.cuda.synchronize()
            lopt_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def allreduce_through_host(group=None):
    """An in-place sum over the ranks of torch.distributed's default (or given)
    process group for device buffers, through a host copy: for backends that
    take host tensors only (gloo).  With RCCL, torch.distributed.all_reduce
    takes the device buffer directly."""
    import torch.distributed as dist

    def allreduce(buf):
        host = buf.cpu()
        dist.all_reduce(host, group=group)
        buf.copy_(host)
    return allreduce


def _torch_optimizer_base():
    import torch
    return torch.optim.Optimizer


class LearnedOptimizer(_torch_optimizer_base()):
    """small_fc_lopt as a ``torch.optim.Optimizer`` over fp32 device parameters.

    Each ``step()`` is one ``lopt_step`` over every parameter, with the
    gradients in ``p.grad``; a parameter whose ``grad`` is None is skipped.  ``lr`` and ``weight_decay`` are read from the
    parameter groups at every step, so ``torch.optim.lr_scheduler`` schedules
    drive them; groups may differ (say, no weight decay on biases and norms).
    One setting for all groups goes to the library with ``lopt_set_config``,
    several with ``lopt_set_tensor_hyper``.  The accumulators live in
    ``self.lopt.states`` (layout of ``include/lopt.h``).
    """

    def __init__(self, params, mlp: np.ndarray, lr: float = 1.0, weight_decay: float = 0.0,
                 config: Optional[lopt_config] = None):
        super().__init__(params, dict(lr=lr, weight_decay=weight_decay))
        plist = [p for g in self.param_groups for p in g["params"]]
        cfg = config if config is not None else lopt_default_config()
        cfg.lr, cfg.weight_decay = lr, weight_decay
        self.lopt = LOpt(plist, mlp, cfg)
        self._applied = (float(cfg.lr), float(cfg.weight_decay))
        self._applied_per_tensor = None

    def _sync_hyper(self):
        """Hands the groups' lr / weight_decay to the library when they changed."""
        pairs = [(float(g["lr"]), float(g["weight_decay"])) for g in self.param_groups for _ in g["params"]]
        distinct = set(pairs)
        if len(distinct) <= 1:
            lr, wd = distinct.pop() if distinct else self._applied
            if self._applied_per_tensor is not None:
                self.lopt.set_tensor_hyper(None, None)
                self._applied_per_tensor = None
            if (lr, wd) != self._applied:
                cfg = self.lopt.cfg
                cfg.lr, cfg.weight_decay = lr, wd
                lopt_set_config(self.lopt.handle, cfg)
                self._applied = (float(cfg.lr), float(cfg.weight_decay))
        elif pairs != self._applied_per_tensor:
            self.lopt.set_tensor_hyper([a for a, _ in pairs], [b for _, b in pairs])
            self._applied_per_tensor = pairs

    def step(self, closure=None):
        import torch
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        self._sync_hyper()
        # a parameter without a gradient is skipped, as torch optimizers do
        self.lopt.step([p.grad for p in self.lopt.params])
        return loss

    def state_dict(self):
        """torch's optimizer state (parameter groups) plus what the library keeps:
        each parameter's accumulator buffer (layout of include/lopt.h) and the
        step count."""
        sd = super().state_dict()
        sd["lopt"] = {"t": self.lopt.t, "n_feat": int(self.lopt.cfg.n_feat),
                      "states": [s.detach().clone() for s in self.lopt.states]}
        return sd

    def load_state_dict(self, state_dict):
        sd = dict(state_dict)
        lo = sd.pop("lopt", None)
        if lo is None:
            raise ValueError("the state dict holds no learned-optimizer state")
        if int(lo["n_feat"]) != int(self.lopt.cfg.n_feat) or len(lo["states"]) != len(self.lopt.states):
            raise ValueError("the state dict belongs to another parameter list or learned optimizer")
        for dst, src in zip(self.lopt.states, lo["states"]):
            if src.numel() != dst.numel():
                raise ValueError("accumulator buffer size differs from the parameter's")
        super().load_state_dict(sd)   # parameter groups: lr and weight decay reach the library at the next step
        for dst, src in zip(self.lopt.states, lo["states"]):
            dst.copy_(src.to(device=dst.device, dtype=dst.dtype))
        self.lopt.t = int(lo["t"])
