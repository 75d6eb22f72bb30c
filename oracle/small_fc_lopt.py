"""CPU oracle for one small_fc_lopt learned-optimizer step (fp64, NumPy).

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its binding) never calls it and shares no code with it.

Source: the PyLO page ("PyLO: Towards Accessible Learned Optimizers in
PyTorch", MLSys 2026 talk notes):
  * "Background": a small meta-learned MLP predicts a per-parameter update.
  * "Library design": the optimizer keeps per-parameter accumulators, builds
    features and applies the update.
  * "CUDA kernel design: two-pass fusion" > "Naive implementation bottleneck":
    the per-element feature tensor is mn x d_feat.
  * "Fused kernel strategy", kernel 1: every feature's sum of squares over the
    tensor is collected (one scalar per feature); kernel 2: features are
    rebuilt, normalised with those statistics and fed through the MLP, whose
    output updates the parameter.
  * "Use of the memory hierarchy": d_feat is about 39 for small_fc_lopt, the
    hidden width about 32, the MLP has four layers; g, p, m, v are read.

The page does not print the feature list, the decay constants, the epsilons,
the activation, the sign of the update or the step counter.  This oracle fixes
them as follows (each choice is one "reading"):

  R1  28 per-element features (below) + 11 step features = 39 inputs.
  R2  beta_m = (0.1, 0.5, 0.9), beta_v = 0.999, beta_f = (0.9, 0.99, 0.999).
  R3  eps_v = 1e-8 inside the root of v; eps_f = 1e-20 added to row/column means.
  R4  eps_norm = 1e-30 inside the root of each feature's mean square.
  R5  each feature is divided by its root-mean-square over the whole tensor.
  R6  descent: p <- p - u.
  R7  accumulators are updated with the current g first; features use the new
      accumulators and the old p.
  R8  the step counter t is 1 on the first call.
  R9  step features tanh(t / tau_q) for 11 timescales, not normalised.
  R10 population mean (divide by n).
  R11 a 1-D tensor of length n is viewed as 1 x n.
  R12 a matrix is viewed as given: first dimension = rows, row-major (a
      tensor of more dimensions: first dimension x the product of the others).
  R13 ReLU on both hidden layers, linear output.
  R14 three weight matrices d_in -> 32 -> 32 -> 2.
  R16 learning-rate multiplier lr (default 1) and decoupled weight decay wd
      (default 0): p <- p - lr*u - lr*wd*p.
  R28 a tensor without a gradient in a step is left as it is (parameters and
      accumulators), as torch optimizers skip such parameters; t is the
      optimizer's and advances with every step.
  R18 hyperparameters are fp32 numbers (they are passed as fp32).
  R24 no bias correction of the moving averages.
  R26 the VeLO-shaped variant (n_feat = 19): the same page gives VeLO's feature
      width as about 30 and runs it through the same two fused kernels, but
      lists no feature; here it keeps F0..F18 (every family: parameter,
      gradient, momentum and RMS averages, factored row/column terms) and the
      11 step features, 30 inputs, with the same MLP shape and update rule.

Per element (i, j) of a tensor viewed as R x C, with a = 1..3 and k = 1..3:
  m_a <- b_a m_a + (1 - b_a) g            v <- b_v v + (1 - b_v) g^2
  gr[i] = mean_j g^2, gc[j] = mean_i g^2
  r_k <- f_k r_k + (1 - f_k)(gr + eps_f)  c_k <- f_k c_k + (1 - f_k)(gc + eps_f)
  rbar_k = mean_i r_k[i];  rho_k = (r_k[i] c_k[j] / rbar_k)^(-1/2)
  F0 = g, F1 = p, F2..4 = m_a, F5 = v, F6..8 = m_a (v + eps_v)^(-1/2),
  F9 = (v + eps_v)^(-1/2), F10..12 = g rho_k, F13..15 = r_k[i]^(-1/2),
  F16..18 = c_k[j]^(-1/2), F19 + 3(a-1) + (k-1) = m_a rho_k.
  s_d = (sum F_d^2 / n + eps_norm)^(-1/2);  x = [F s, tanh(t / tau)]
  (dir, mag) = W3 relu(W2 relu(W1 x + b1) + b2) + b3
  u = dir exp(mag exp_mult) step_mult;    p <- p - lr u - lr wd p

Numerics: state and parameters are stored in fp32; each step reads them,
computes in fp64 and rounds the returned state and parameters to fp32 once.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Sequence, Tuple

import numpy as np

N_FEATURES = 28          # per-element features of small_fc_lopt (R1)
VELO_FEATURES = 19       # per-element features of the VeLO-shaped variant (R26)
FEATURE_SETS = (N_FEATURES, VELO_FEATURES)
HIDDEN = 32
DEFAULT_TIMESCALES = (1.0, 3.0, 10.0, 30.0, 100.0, 300.0, 1e3, 3e3, 1e4, 3e4, 1e5)

# Index of the feature m_a * rho_k (a, k = 0-based)
def cross_index(a: int, k: int) -> int:
    return 19 + 3 * a + k


def _f32(x):
    """Value of x as an fp32 number, returned as a Python float (fp64)."""
    return float(np.float32(x))


@dataclass(frozen=True)
class Hyper:
    beta_m: Tuple[float, float, float] = (0.1, 0.5, 0.9)
    beta_v: float = 0.999
    beta_f: Tuple[float, float, float] = (0.9, 0.99, 0.999)
    eps_v: float = 1e-8
    eps_f: float = 1e-20
    eps_norm: float = 1e-30
    exp_mult: float = 1e-3
    step_mult: float = 1e-3
    lr: float = 1.0
    weight_decay: float = 0.0
    n_time: int = 11
    timescales: Tuple[float, ...] = DEFAULT_TIMESCALES
    n_feat: int = N_FEATURES   # per-element MLP inputs: the first n_feat of F0..F27

    def as_f32(self) -> "Hyper":
        """The same hyperparameters rounded to fp32 (what the fp32 config holds)."""
        return Hyper(tuple(_f32(b) for b in self.beta_m), _f32(self.beta_v),
                     tuple(_f32(b) for b in self.beta_f), _f32(self.eps_v), _f32(self.eps_f),
                     _f32(self.eps_norm), _f32(self.exp_mult), _f32(self.step_mult),
                     _f32(self.lr), _f32(self.weight_decay), int(self.n_time),
                     tuple(_f32(x) for x in self.timescales[: self.n_time]), int(self.n_feat))


@dataclass
class Mlp:
    W1: np.ndarray  # (32, n_feat + n_time)
    b1: np.ndarray  # (32,)
    W2: np.ndarray  # (32, 32)
    b2: np.ndarray
    W3: np.ndarray  # (2, 32)
    b3: np.ndarray  # (2,)


def mlp_size(n_time: int, n_feat: int = N_FEATURES) -> int:
    d_in = n_feat + n_time
    return HIDDEN * d_in + HIDDEN + HIDDEN * HIDDEN + HIDDEN + 2 * HIDDEN + 2


def unpack_mlp(flat: np.ndarray, n_time: int, n_feat: int = N_FEATURES) -> Mlp:
    """Packed row-major (out x in) layout: W1, b1, W2, b2, W3, b3."""
    flat = np.asarray(flat, dtype=np.float64)
    d_in = n_feat + n_time
    if flat.size != mlp_size(n_time, n_feat):
        raise ValueError(f"expected {mlp_size(n_time, n_feat)} MLP floats, got {flat.size}")
    sizes = [(HIDDEN, d_in), (HIDDEN,), (HIDDEN, HIDDEN), (HIDDEN,), (2, HIDDEN), (2,)]
    out, o = [], 0
    for s in sizes:
        cnt = int(np.prod(s))
        out.append(flat[o:o + cnt].reshape(s))
        o += cnt
    return Mlp(*out)


def pack_mlp(m: Mlp) -> np.ndarray:
    return np.concatenate([m.W1.ravel(), m.b1, m.W2.ravel(), m.b2, m.W3.ravel(), m.b3]).astype(np.float32)


def zero_state(rows: int, cols: int) -> dict:
    return {"m": np.zeros((3, rows, cols), np.float32), "v": np.zeros((rows, cols), np.float32),
            "r": np.zeros((3, rows), np.float32), "c": np.zeros((3, cols), np.float32)}


def as_matrix(x: np.ndarray) -> np.ndarray:
    """R11/R12: 1-D of length n -> 1 x n; a matrix stays as given."""
    x = np.asarray(x)
    if x.ndim == 1:
        return x.reshape(1, -1)
    if x.ndim != 2:
        raise ValueError("tensors are 1-D or 2-D")
    return x


# ---------------------------------------------------------------- accumulators
@dataclass
class Accumulators:
    m: np.ndarray      # (3, R, C) fp64
    v: np.ndarray      # (R, C)
    r: np.ndarray      # (3, R)
    c: np.ndarray      # (3, C)
    rbar: np.ndarray   # (3,)


def accumulate(g: np.ndarray, state: dict, hp: Hyper) -> Accumulators:
    """Moving averages of g (per element) and of the row/column means of g^2."""
    g = as_matrix(g).astype(np.float64)
    R, C = g.shape
    m = np.empty((3, R, C))
    for a in range(3):
        b = hp.beta_m[a]
        m[a] = b * state["m"][a].astype(np.float64) + (1.0 - b) * g
    v = hp.beta_v * state["v"].astype(np.float64) + (1.0 - hp.beta_v) * (g * g)
    g2 = g * g
    row_mean = g2.sum(axis=1) / C    # mean over the columns of row i
    col_mean = g2.sum(axis=0) / R    # mean over the rows of column j
    r = np.empty((3, R))
    c = np.empty((3, C))
    for k in range(3):
        f = hp.beta_f[k]
        r[k] = f * state["r"][k].astype(np.float64) + (1.0 - f) * (row_mean + hp.eps_f)
        c[k] = f * state["c"][k].astype(np.float64) + (1.0 - f) * (col_mean + hp.eps_f)
    rbar = r.mean(axis=1)
    return Accumulators(m, v, r, c, rbar)


# ------------------------------------------------------------------- features
def features(p: np.ndarray, g: np.ndarray, acc: Accumulators, hp: Hyper,
             rows: slice = slice(None)) -> np.ndarray:
    """The first ``hp.n_feat`` of the 28 per-element features of the rows ``rows``;
    shape (rows, C, n_feat)."""
    p = as_matrix(p)[rows].astype(np.float64)
    g = as_matrix(g)[rows].astype(np.float64)
    m = acc.m[:, rows]
    v = acc.v[rows]
    r = acc.r[:, rows]
    c = acc.c
    nr, C = g.shape
    F = np.empty((nr, C, N_FEATURES))
    F[..., 0] = g
    F[..., 1] = p
    for a in range(3):
        F[..., 2 + a] = m[a]
    F[..., 5] = v
    inv_rms_v = 1.0 / np.sqrt(v + hp.eps_v)
    for a in range(3):
        F[..., 6 + a] = m[a] * inv_rms_v
    F[..., 9] = inv_rms_v
    for k in range(3):
        vhat = r[k][:, None] * c[k][None, :] / acc.rbar[k]   # factored estimate of g^2
        rho = 1.0 / np.sqrt(vhat)
        F[..., 10 + k] = g * rho
        F[..., 13 + k] = (1.0 / np.sqrt(r[k]))[:, None]
        F[..., 16 + k] = (1.0 / np.sqrt(c[k]))[None, :]
        for a in range(3):
            F[..., cross_index(a, k)] = m[a] * rho
    return F[..., : hp.n_feat]


def time_features(t: int, hp: Hyper) -> np.ndarray:
    return np.array([np.tanh(t / tau) for tau in hp.timescales[: hp.n_time]], dtype=np.float64)


def feature_scales(sum_sq: np.ndarray, n: int, hp: Hyper) -> np.ndarray:
    """s_d = (mean over the tensor of F_d^2 + eps_norm)^(-1/2)."""
    return 1.0 / np.sqrt(sum_sq / n + hp.eps_norm)


def mlp_forward(x: np.ndarray, w: Mlp) -> Tuple[np.ndarray, np.ndarray]:
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    h1 = np.maximum(x2 @ w.W1.T + w.b1, 0.0)
    h2 = np.maximum(h1 @ w.W2.T + w.b2, 0.0)
    out = h2 @ w.W3.T + w.b3
    return out[:, 0].reshape(lead), out[:, 1].reshape(lead)


def update_from_output(direction, magnitude, hp: Hyper):
    return direction * np.exp(magnitude * hp.exp_mult) * hp.step_mult


# ------------------------------------------------------------------ one tensor
@dataclass
class StepInfo:
    sum_sq: np.ndarray          # (n_feat,) sum of F_d^2 over the tensor
    scales: np.ndarray          # (n_feat,) s_d
    u: Optional[np.ndarray] = None
    F: Optional[np.ndarray] = None       # (R, C, n_feat) raw features
    x: Optional[np.ndarray] = None       # (R, C, n_feat + n_time) MLP input
    acc: Optional[Accumulators] = None


def step_tensor(p, g, state: dict, t: int, mlp: Mlp, hp: Hyper,
                block_rows: Optional[int] = None, keep: bool = False,
                store_dtype=np.float32):
    """One optimizer step of one tensor.

    p, g: fp32 arrays, 1-D or 2-D.  state: dict of fp32 accumulators.
    Returns (p_new in p's shape, new state, StepInfo); both are rounded to
    ``store_dtype`` (fp32 storage; tests of closed forms pass np.float64 to
    keep the exact fp64 trajectory).
    ``block_rows`` splits the sums over the tensor and the MLP evaluation into
    groups of rows to bound memory; it changes only the fp64 summation order.
    """
    shape = np.shape(p)
    P = as_matrix(p)
    G = as_matrix(g)
    R, C = G.shape
    n = R * C
    acc = accumulate(G, state, hp)
    if block_rows is None:
        block_rows = max(1, (1 << 14) // max(C, 1)) if not keep else R
    blocks = [slice(i, min(i + block_rows, R)) for i in range(0, R, block_rows)]

    # pass 1: sum of squares of each feature over the tensor
    nf = hp.n_feat
    sum_sq = np.zeros(nf)
    for rs in blocks:
        F = features(P, G, acc, hp, rs)
        sum_sq += (F * F).reshape(-1, nf).sum(axis=0)
    scales = feature_scales(sum_sq, n, hp)
    T = time_features(t, hp)

    # pass 2: normalised features -> MLP -> update
    p_new = np.empty((R, C))
    u_all = np.empty((R, C)) if keep else None
    F_all = np.empty((R, C, nf)) if keep else None
    x_all = np.empty((R, C, nf + hp.n_time)) if keep else None
    for rs in blocks:
        F = features(P, G, acc, hp, rs)
        nr = F.shape[0]
        x = np.concatenate([F * scales, np.broadcast_to(T, (nr, C, hp.n_time))], axis=-1)
        d, mg = mlp_forward(x, mlp)
        u = update_from_output(d, mg, hp)
        p_old = P[rs].astype(np.float64)
        p_new[rs] = p_old - hp.lr * u - hp.lr * hp.weight_decay * p_old
        if keep:
            u_all[rs] = u
            F_all[rs] = F
            x_all[rs] = x
    sd = store_dtype
    new_state = {"m": acc.m.astype(sd), "v": acc.v.astype(sd),
                 "r": acc.r.astype(sd), "c": acc.c.astype(sd)}
    info = StepInfo(sum_sq, scales, u_all, F_all, x_all, acc if keep else None)
    return p_new.astype(sd).reshape(shape), new_state, info


def step_tensor_rows(p, g, state: dict, t: int, mlp: Mlp, hp: Hyper, rows: Sequence[int],
                     block_rows: Optional[int] = None):
    """One step of one tensor, with the update evaluated only on ``rows``.

    The per-tensor quantities (row/column moving averages and every feature's
    sum of squares) are computed over the whole tensor exactly as in
    ``step_tensor``; the MLP and the update are evaluated for the listed rows
    only.  Returns (p_new[rows], {"m": m[:, rows], "v": v[rows], "r", "c"}),
    rounded to fp32.
    """
    P = as_matrix(p)
    G = as_matrix(g)
    R, C = G.shape
    n = R * C
    rows = np.asarray(rows, dtype=np.int64)
    acc = accumulate(G, state, hp)
    if block_rows is None:
        block_rows = max(1, (1 << 14) // max(C, 1))
    nf = hp.n_feat
    sum_sq = np.zeros(nf)
    for r0 in range(0, R, block_rows):
        F = features(P, G, acc, hp, slice(r0, min(r0 + block_rows, R)))
        sum_sq += (F * F).reshape(-1, nf).sum(axis=0)
    scales = feature_scales(sum_sq, n, hp)
    T = time_features(t, hp)
    sub = Accumulators(acc.m[:, rows], acc.v[rows], acc.r[:, rows], acc.c, acc.rbar)
    F = features(P[rows], G[rows], sub, hp)
    x = np.concatenate([F * scales, np.broadcast_to(T, (len(rows), C, hp.n_time))], axis=-1)
    d, mg = mlp_forward(x, mlp)
    u = update_from_output(d, mg, hp)
    p_old = P[rows].astype(np.float64)
    p_new = p_old - hp.lr * u - hp.lr * hp.weight_decay * p_old
    st = {"m": sub.m.astype(np.float32), "v": sub.v.astype(np.float32),
          "r": acc.r.astype(np.float32), "c": acc.c.astype(np.float32)}
    return p_new.astype(np.float32), st


def step_tensor_sub(p, g, state: dict, t: int, mlp: Mlp, hp: Hyper,
                    rows: Optional[Sequence[int]] = None, cols: Optional[Sequence[int]] = None,
                    block_rows: Optional[int] = None):
    """One step of one tensor, with the update evaluated on a sub-block only.

    Everything per tensor -- the row/column moving averages r, c, their means
    rbar and every feature's sum of squares -- is computed over the whole
    tensor, as in ``step_tensor``; the features, the MLP and the update are
    then evaluated on the elements of the listed ``rows`` x ``cols`` (all of
    them when None).  Returns (p_new[rows][:, cols], {"m": (3, nr, nc), "v":
    (nr, nc), "r": (3, R), "c": (3, C)}, StepInfo(sum_sq, scales, acc)) with
    the arrays rounded to fp32 (r and c in full)."""
    P = as_matrix(p)
    G = as_matrix(g)
    R, C = G.shape
    n = R * C
    ri = np.arange(R) if rows is None else np.asarray(rows, dtype=np.int64)
    ci = np.arange(C) if cols is None else np.asarray(cols, dtype=np.int64)
    acc = accumulate(G, state, hp)
    if block_rows is None:
        block_rows = max(1, (1 << 14) // max(C, 1))
    nf = hp.n_feat
    sum_sq = np.zeros(nf)
    for r0 in range(0, R, block_rows):
        F = features(P, G, acc, hp, slice(r0, min(r0 + block_rows, R)))
        sum_sq += (F * F).reshape(-1, nf).sum(axis=0)
    scales = feature_scales(sum_sq, n, hp)
    T = time_features(t, hp)
    sub = Accumulators(acc.m[:, ri][:, :, ci], acc.v[ri][:, ci], acc.r[:, ri], acc.c[:, ci], acc.rbar)
    Psub = P[ri][:, ci]
    F = features(Psub, G[ri][:, ci], sub, hp)
    x = np.concatenate([F * scales, np.broadcast_to(T, F.shape[:2] + (hp.n_time,))], axis=-1)
    d, mg = mlp_forward(x, mlp)
    u = update_from_output(d, mg, hp)
    p_old = Psub.astype(np.float64)
    p_new = p_old - hp.lr * u - hp.lr * hp.weight_decay * p_old
    st = {"m": sub.m.astype(np.float32), "v": sub.v.astype(np.float32),
          "r": acc.r.astype(np.float32), "c": acc.c.astype(np.float32)}
    return p_new.astype(np.float32), st, StepInfo(sum_sq, scales, acc=acc)


def step(params: Sequence[np.ndarray], grads: Sequence[np.ndarray], states: Sequence[dict],
         t: int, mlp_flat: np.ndarray, hp: Hyper = Hyper(),
         tensor_hyper: Optional[Sequence[Tuple[float, float]]] = None, **kw):
    """One optimizer step over a list of tensors (tensors are independent; t is shared).

    ``t`` is the 1-based index of this step.  ``tensor_hyper``: optional
    (lr, weight_decay) per tensor, replacing hp's for that tensor (R16; torch's
    parameter groups).  A gradient of None leaves its tensor and state as they
    are (R28).  Returns (new params, new states).
    """
    hp32 = hp.as_f32()
    if hp32.n_feat not in FEATURE_SETS:
        raise ValueError(f"n_feat must be one of {FEATURE_SETS}")
    if tensor_hyper is not None and len(tensor_hyper) != len(params):
        raise ValueError("tensor_hyper needs one (lr, weight_decay) pair per tensor")
    mlp = unpack_mlp(mlp_flat, hp32.n_time, hp32.n_feat)
    outs_p, outs_s = [], []
    for i, (p, g, s) in enumerate(zip(params, grads, states)):
        if g is None:
            outs_p.append(p)
            outs_s.append(s)
            continue
        hpi = hp32
        if tensor_hyper is not None:
            lr, wd = tensor_hyper[i]
            hpi = replace(hp32, lr=_f32(lr), weight_decay=_f32(wd))
        pn, sn, _ = step_tensor(p, g, s, t, mlp, hpi, **kw)
        outs_p.append(pn)
        outs_s.append(sn)
    return outs_p, outs_s
