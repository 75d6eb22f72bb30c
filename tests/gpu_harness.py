"""Test-side glue: runs a workload through the HIP library (via the C-ABI
binding) and through the CPU oracle on identical seeded inputs, and compares
them element by element."""
from __future__ import annotations

import dataclasses
import hashlib
import sys
from collections import OrderedDict
from typing import Dict, List, Optional, Sequence

import numpy as np

import oracle
from learned_optimizer_step_amd import lopt as L
from learned_optimizer_step_amd import workloads as W

RTOL = 1e-5   # parity bar on p, m1..m3, v, r1..r3, c1..c3
ATOL = 1e-7

# Every MLP path, the default first: bf16x8 and bf16x9 (fp32 arithmetic from
# bf16 pieces), the fp32 matrix cores, the vector ALU, and the two narrower
# split paths (bf16x6, fp16x3).
IMPLS = [L.LOPT_MLP_BF16X8, L.LOPT_MLP_BF16X9, L.LOPT_MLP_MFMA, L.LOPT_MLP_VALU, L.LOPT_MLP_BF16X6, L.LOPT_MLP_FP16X3]


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def hyper_from_cfg(cfg) -> oracle.Hyper:
    return oracle.Hyper(beta_m=tuple(cfg.beta_m), beta_v=cfg.beta_v, beta_f=tuple(cfg.beta_f),
                        eps_v=cfg.eps_v, eps_f=cfg.eps_f, eps_norm=cfg.eps_norm,
                        exp_mult=cfg.exp_mult, step_mult=cfg.step_mult, lr=cfg.lr,
                        weight_decay=cfg.weight_decay, n_time=cfg.n_time,
                        timescales=tuple(cfg.timescales)[: cfg.n_time], n_feat=cfg.n_feat)


def to_matrix_state(st: dict) -> dict:
    return {k: np.asarray(v, dtype=np.float32) for k, v in st.items()}


class DeviceRun:
    """A workload on the GPU through LOpt; inputs from the seeded generator."""

    def __init__(self, w: W.Workload, mlp: np.ndarray, cfg, torch):
        self.w, self.torch = w, torch
        self.params = []
        for i, t in enumerate(w.tensors):
            p = W.param_init(w, i).reshape(t.shape)
            self.params.append(torch.from_numpy(p).cuda())
        self.opt = L.LOpt(self.params, mlp, cfg)
        if w.prewarm_std is not None:
            for i in range(len(w.tensors)):
                st = W.state_init(w, i)
                v = self.opt.state_views(i)
                for k in ("m", "v", "r", "c"):
                    v[k].copy_(torch.from_numpy(st[k]))
        self.grads = None

    def step(self, t: int, reuse_grads: bool = False):
        if not reuse_grads or self.grads is None:
            self.grads = [self.torch.from_numpy(W.grad_at(self.w, i, t).reshape(tt.shape)).cuda()
                          for i, tt in enumerate(self.w.tensors)]
        self.opt.step(self.grads)

    def fetch(self, i: int) -> dict:
        self.torch.cuda.synchronize()
        v = self.opt.state_views(i)
        out = {k: v[k].cpu().numpy().copy() for k in ("m", "v", "r", "c")}
        out["p"] = self.params[i].cpu().numpy().reshape(self.w.tensors[i].rows, self.w.tensors[i].cols).copy()
        return out

    def close(self):
        self.opt.close()


_ORACLE_CACHE: "OrderedDict[tuple, Dict[int, dict]]" = OrderedDict()


def oracle_run(w: W.Workload, mlp: np.ndarray, hp: oracle.Hyper, steps: int,
               subset: Optional[Sequence[int]] = None, tensor_hyper=None) -> Dict[int, dict]:
    """Oracle trajectory of the tensors in ``subset`` (tensors are independent);
    tensor_hyper: optional (lr, weight_decay) for every tensor of the workload.
    Per tensor: p, m, v, r, c after the last step, and that step's feature
    normalisers (scales) and sqrt(mean r_k) (sqrt_rbar).  The result does not
    depend on the GPU's MLP path, so it is kept for the next call with the same
    inputs (a few recent ones)."""
    idx = list(range(len(w.tensors))) if subset is None else list(subset)
    th = None if tensor_hyper is None else tuple(tuple(float(x) for x in tensor_hyper[i]) for i in idx)
    key = (w, steps, hp, hashlib.sha1(np.ascontiguousarray(mlp, np.float32).tobytes()).hexdigest(), tuple(idx), th)
    if key in _ORACLE_CACHE:
        _ORACLE_CACHE.move_to_end(key)
        return _ORACLE_CACHE[key]
    hp32 = hp.as_f32()
    m = oracle.unpack_mlp(mlp, hp32.n_time, hp32.n_feat)
    out = {}
    for j, i in enumerate(idx):
        # the per-tensor (lr, weight decay), fp32 numbers as the library takes them
        hpi = hp32 if th is None else dataclasses.replace(hp32, lr=float(np.float32(th[j][0])),
                                                          weight_decay=float(np.float32(th[j][1])))
        p, st = W.param_init(w, i), W.state_init(w, i)
        for t in range(1, steps + 1):
            p, st, info = oracle.step_tensor(p, W.grad_at(w, i, t), st, t, m, hpi)
        out[i] = dict(p=p, **st, scales=np.asarray(info.scales, np.float64),
                      sqrt_rbar=np.sqrt(np.asarray(st["r"], np.float64).mean(axis=1)))
    _ORACLE_CACHE[key] = out
    while len(_ORACLE_CACHE) > 4:
        _ORACLE_CACHE.popitem(last=False)
    return out


def compare_stats(got: np.ndarray, want: dict, n_feat: int, label: str, rtol=RTOL, atol=ATOL) -> List[str]:
    """The GPU's per-tensor statistics (a lopt_get_tensor_stats row) against the
    oracle's: the feature normalisers s_d (relative) and sqrt(mean r_k)."""
    errs = []
    s_got = np.asarray(got[:n_feat], np.float64)
    s_want = np.asarray(want["scales"], np.float64)
    bad = ~(np.abs(s_got - s_want) <= rtol * np.abs(s_want))
    if bad.any():
        d = int(np.argmax(bad))
        errs.append(f"{label}.s_{d}: gpu={s_got[d]!r} oracle={s_want[d]!r} ({int(bad.sum())} features off)")
    if np.any(np.asarray(got[n_feat:28]) != 0):
        errs.append(f"{label}: normalisers of the features the variant does not feed are not 0")
    r_got = np.asarray(got[28:31], np.float64)
    if not np.all(np.abs(r_got - want["sqrt_rbar"]) <= atol + rtol * want["sqrt_rbar"]):
        errs.append(f"{label}.sqrt_rbar: gpu={r_got!r} oracle={want['sqrt_rbar']!r}")
    return errs


def compare(got: dict, want: dict, label: str, rtol=RTOL, atol=ATOL) -> List[str]:
    """Element-wise |got - want| <= atol + rtol |want| on every array; returns failures."""
    errs = []
    for k in ("p", "m", "v", "r", "c"):
        a = np.asarray(got[k], np.float64)
        b = np.asarray(want[k], np.float64).reshape(a.shape)
        err = np.abs(a - b)
        bound = atol + rtol * np.abs(b)
        bad = ~(err <= bound)
        if bad.any():
            j = np.unravel_index(np.argmax(np.where(bad, err / bound, 0)), a.shape)
            errs.append(f"{label}.{k}: {int(bad.sum())}/{a.size} out of tolerance; worst at {j}: "
                        f"gpu={a[j]!r} oracle={b[j]!r}")
    return errs


def parity(w: W.Workload, mlp: np.ndarray, cfg, torch, steps: Optional[int] = None,
           subset: Optional[Sequence[int]] = None, tensor_hyper=None) -> List[str]:
    """GPU steps through the C ABI against the oracle, element by element;
    tensor_hyper: optional (lr, weight_decay) per tensor (lopt_set_tensor_hyper)."""
    steps = w.steps if steps is None else steps
    say(f"[parity] {w.key}: {len(w.tensors)} tensors, {w.n_params} params, {steps} steps, impl={cfg.mlp_impl}"
        + (", per-tensor lr/wd" if tensor_hyper is not None else ""))
    run = DeviceRun(w, mlp, cfg, torch)
    if tensor_hyper is not None:
        run.opt.set_tensor_hyper([a for a, _ in tensor_hyper], [b for _, b in tensor_hyper])
    for t in range(1, steps + 1):
        run.step(t)
    idx = list(range(len(w.tensors))) if subset is None else list(subset)
    got = {i: run.fetch(i) for i in idx}
    stats = run.opt.tensor_stats()
    run.close()
    want = oracle_run(w, mlp, hyper_from_cfg(cfg), steps, idx, tensor_hyper)
    errs = []
    for i in idx:
        label = f"{w.key}[{i}:{w.tensors[i].name} {w.tensors[i].rows}x{w.tensors[i].cols}]"
        errs += compare(got[i], want[i], label)
        errs += compare_stats(stats[i], want[i], int(cfg.n_feat), label)
    return errs


def parity_one_step_rows(w: W.Workload, mlp: np.ndarray, cfg, torch, picks) -> List[str]:
    """One full-size GPU step over the whole workload; the oracle then checks
    the tensors in ``picks`` = {tensor index: rows or None (all rows)}: the
    per-tensor sums always cover the whole tensor, the update is compared on
    the listed rows."""
    say(f"[parity-rows] {w.key}: {len(w.tensors)} tensors, {w.n_params} params, 1 step, impl={cfg.mlp_impl}")
    run = DeviceRun(w, mlp, cfg, torch)
    run.step(1)
    got = {i: run.fetch(i) for i in picks}
    run.close()
    hp = hyper_from_cfg(cfg).as_f32()
    m = oracle.unpack_mlp(mlp, hp.n_time, hp.n_feat)
    errs = []
    for i, rows in picks.items():
        t = w.tensors[i]
        p0, g, st = W.param_init(w, i), W.grad_at(w, i, 1), W.state_init(w, i)
        label = f"{w.key}[{i}:{t.name} {t.rows}x{t.cols}]"
        if rows is None:
            pn, sn, _ = oracle.step_tensor(p0, g, st, 1, m, hp)
            want = dict(p=pn, **sn)
            gsel = got[i]
        else:
            pn, sn = oracle.step_tensor_rows(p0, g, st, 1, m, hp, rows)
            want = dict(p=pn, **sn)
            gg = got[i]
            gsel = {"p": gg["p"][rows], "m": gg["m"][:, rows], "v": gg["v"][rows], "r": gg["r"], "c": gg["c"]}
            label += f" rows {list(rows)[:4]}..."
        errs += compare(gsel, want, label)
    return errs
