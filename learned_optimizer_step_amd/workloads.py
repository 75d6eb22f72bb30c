"""Seeded synthetic inputs for the small_fc_lopt optimizer step.

This module holds shapes, value distributions and random-number recipes only;
it contains none of the optimizer's arithmetic.  Both the HIP path (through the
tests and the benchmark) and the CPU oracle are fed from here, so the two sides
see bit-identical fp32 inputs.

Workloads (parameter-set shapes stand in for the models the PyLO page times,
"Benchmark results / step-time reduction" table: ViT-B/16 and GPT-2-class
transformers; for an optimizer step only the parameter shapes matter):

* ``single256``   one 256x256 weight, 10 steps, fresh gradients per step
* ``single4096``  one 4096x4096 weight, accumulators pre-warmed, 1 step
* ``vit_b16``     the ViT-B/16 parameter set (86,563,584 params, 147 tensors)
* ``llama1b``     a Llama-style 1.26 G-parameter set (200 tensors)
* ``ragged10k``   10,000 tensors with log-uniform sizes 16..1e6
* ``gpt2_355m``   the GPT-2 355M parameter set (354,823,168 params, 292 tensors)

Random numbers: numpy ``Generator(PCG64(SeedSequence([...])))`` keyed by
(workload id, tensor index, step, stream) so any tensor can be regenerated on
its own.  Normal draws are made in float32 and scaled in float32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np

HIDDEN = 32
N_FEATURES = 28        # small_fc_lopt's per-element features
VELO_FEATURES = 19     # the d_feat = 30 VeLO-shaped variant's per-element features
N_TIME = 11

# RNG stream ids inside a (workload, tensor, step) key
STREAM_PARAM = 0
STREAM_GRAD = 1
STREAM_STATE0 = 2  # m1, m2, m3, v, r1, r2, r3, c1, c2, c3 -> 2..11

MLP_SEED = (0, 9999)


@dataclass(frozen=True)
class TensorSpec:
    name: str
    rows: int
    cols: int
    vector: bool  # 1-D parameter (viewed as 1 x n)

    @property
    def n(self) -> int:
        return self.rows * self.cols

    @property
    def shape(self) -> Tuple[int, ...]:
        return (self.cols,) if self.vector else (self.rows, self.cols)


@dataclass(frozen=True)
class Workload:
    key: str
    wid: int
    tensors: Tuple[TensorSpec, ...]
    param_std: float
    grad_std: float
    steps: int
    prewarm_std: Optional[float] = None  # |N(0, s)| for every accumulator
    description: str = ""

    @property
    def n_params(self) -> int:
        return sum(t.n for t in self.tensors)


def _mat(name, r, c):
    return TensorSpec(name, int(r), int(c), False)


def _vec(name, n):
    return TensorSpec(name, 1, int(n), True)


def vit_b16_tensors() -> Tuple[TensorSpec, ...]:
    d = 768
    ts = [_mat("patch_embed", d, d), _mat("pos_embed", 197, d)]
    for b in range(12):
        p = f"blocks.{b}."
        ts += [
            _mat(p + "qkv.weight", d, 3 * d), _vec(p + "qkv.bias", 3 * d),
            _mat(p + "proj.weight", d, d), _vec(p + "proj.bias", d),
            _mat(p + "fc1.weight", d, 4 * d), _vec(p + "fc1.bias", 4 * d),
            _mat(p + "fc2.weight", 4 * d, d), _vec(p + "fc2.bias", d),
            _vec(p + "norm1.weight", d), _vec(p + "norm1.bias", d),
            _vec(p + "norm2.weight", d), _vec(p + "norm2.bias", d),
        ]
    ts.append(_mat("head", 1000, d))
    return tuple(ts)


def llama1b_tensors() -> Tuple[TensorSpec, ...]:
    d, f, v = 2048, 5632, 32000
    ts = [_mat("embed", v, d)]
    for layer in range(22):
        p = f"layers.{layer}."
        ts += [_mat(p + n, d, d) for n in ("q", "k", "v", "o")]
        ts += [_mat(p + "gate", d, f), _mat(p + "up", d, f), _mat(p + "down", f, d)]
        ts += [_vec(p + "attn_norm", d), _vec(p + "mlp_norm", d)]
    ts.append(_mat("unembed", v, d))
    return tuple(ts)


def gpt2_355m_tensors() -> Tuple[TensorSpec, ...]:
    """GPT-2 medium (24 layers, d_model 1024, vocab 50257, 1024 positions), the
    page's second step-time workload.  Weights are stored (in, out) as GPT-2's
    Conv1D layers do; the output head is tied to the token embedding."""
    d, f, v, ctx = 1024, 4096, 50257, 1024
    ts = [_mat("wte", v, d), _mat("wpe", ctx, d)]
    for layer in range(24):
        p = f"h.{layer}."
        ts += [_vec(p + "ln_1.weight", d), _vec(p + "ln_1.bias", d),
               _mat(p + "attn.c_attn.weight", d, 3 * d), _vec(p + "attn.c_attn.bias", 3 * d),
               _mat(p + "attn.c_proj.weight", d, d), _vec(p + "attn.c_proj.bias", d),
               _vec(p + "ln_2.weight", d), _vec(p + "ln_2.bias", d),
               _mat(p + "mlp.c_fc.weight", d, f), _vec(p + "mlp.c_fc.bias", f),
               _mat(p + "mlp.c_proj.weight", f, d), _vec(p + "mlp.c_proj.bias", d)]
    ts += [_vec("ln_f.weight", d), _vec("ln_f.bias", d)]
    return tuple(ts)


def ragged_tensors(count: int = 10000, lo: int = 16, hi: int = 1_000_000,
                   seed: int = 5) -> Tuple[TensorSpec, ...]:
    """Log-uniform sizes; half 1-D, half 2-D with log-uniform aspect in [1/64, 64]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 77, 0, 99])))
    ts = []
    for i in range(count):
        n = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        if rng.uniform() < 0.5:
            ts.append(_vec(f"t{i}", n))
        else:
            a = math.exp(rng.uniform(math.log(1 / 64), math.log(64)))
            r = min(max(int(round(math.sqrt(n * a))), 1), n)
            c = max(1, int(round(n / r)))
            ts.append(_mat(f"t{i}", r, c))
    return tuple(ts)


def get_workload(key: str) -> Workload:
    if key == "single256":
        return Workload(key, 1, (_mat("w", 256, 256),), 0.02, 1e-2, 10,
                        description="one fp32 256x256 weight, 10 steps")
    if key == "single4096":
        return Workload(key, 2, (_mat("w", 4096, 4096),), 0.02, 1e-3, 1, prewarm_std=1e-3,
                        description="one fp32 4096x4096 weight, pre-warmed accumulators, 1 step")
    if key == "vit_b16":
        return Workload(key, 3, vit_b16_tensors(), 0.02, 1e-3, 5,
                        description="ViT-B/16 parameter set, 86,563,584 fp32 params in 147 tensors")
    if key == "llama1b":
        return Workload(key, 4, llama1b_tensors(), 0.02, 1e-4, 1,
                        description="Llama-style parameter set, 1,261,527,040 fp32 params in 200 tensors")
    if key == "gpt2_355m":
        return Workload(key, 6, gpt2_355m_tensors(), 0.02, 1e-3, 1,
                        description="GPT-2 355M parameter set, 354,823,168 fp32 params in 292 tensors")
    if key == "ragged10k":
        return Workload(key, 5, ragged_tensors(), 0.02, 1e-3, 1,
                        description="10,000 ragged tensors, sizes log-uniform 16..1e6")
    raise KeyError(key)


WORKLOADS = ("single256", "single4096", "vit_b16", "llama1b", "ragged10k", "gpt2_355m")


def custom_workload(key: str, shapes: Sequence[Tuple[int, ...]], param_std=0.02,
                    grad_std=1e-2, steps=10, prewarm_std=None, wid=100) -> Workload:
    """A workload from explicit shapes: (n,) is a 1-D tensor, (r, c) a matrix."""
    ts = []
    for i, s in enumerate(shapes):
        if len(s) == 1:
            ts.append(_vec(f"t{i}", s[0]))
        else:
            ts.append(_mat(f"t{i}", s[0], s[1]))
    return Workload(key, wid, tuple(ts), param_std, grad_std, steps, prewarm_std)


def _rng(wid, tidx, step, stream) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wid, tidx, step, stream])))


def _normal(rng, n, std) -> np.ndarray:
    x = rng.standard_normal(n, dtype=np.float32)
    x *= np.float32(std)
    return x


def param_init(w: Workload, tidx: int) -> np.ndarray:
    """fp32 parameter values of tensor ``tidx`` in its (rows, cols) view."""
    t = w.tensors[tidx]
    return _normal(_rng(w.wid, tidx, 0, STREAM_PARAM), t.n, w.param_std).reshape(t.rows, t.cols)


def grad_at(w: Workload, tidx: int, step: int) -> np.ndarray:
    """fp32 gradient of tensor ``tidx`` for 1-based ``step``, (rows, cols) view."""
    t = w.tensors[tidx]
    return _normal(_rng(w.wid, tidx, step, STREAM_GRAD), t.n, w.grad_std).reshape(t.rows, t.cols)


def state_init(w: Workload, tidx: int) -> dict:
    """Initial accumulators of tensor ``tidx``: zeros, or |N(0, s)| when pre-warmed.

    Keys: m (3, R, C), v (R, C), r (3, R), c (3, C); all fp32.
    """
    t = w.tensors[tidx]
    R, C = t.rows, t.cols
    if w.prewarm_std is None:
        return {"m": np.zeros((3, R, C), np.float32), "v": np.zeros((R, C), np.float32),
                "r": np.zeros((3, R), np.float32), "c": np.zeros((3, C), np.float32)}

    def draw(stream, n):
        return np.abs(_normal(_rng(w.wid, tidx, 0, STREAM_STATE0 + stream), n, w.prewarm_std))

    m = np.stack([draw(a, R * C).reshape(R, C) for a in range(3)])
    v = draw(3, R * C).reshape(R, C)
    r = np.stack([draw(4 + k, R) for k in range(3)])
    c = np.stack([draw(7 + k, C) for k in range(3)])
    return {"m": m, "v": v, "r": r, "c": c}


def mlp_weights(n_time: int = N_TIME, seed=MLP_SEED, bias_std: float = 0.0,
                n_feat: int = N_FEATURES) -> np.ndarray:
    """Packed fp32 MLP weights W1[32][n_feat+n_time], b1[32], W2[32][32], b2[32], W3[2][32], b3[2].

    Weights ~ N(0, 1/fan_in) (variance 1/fan_in); biases zero unless ``bias_std`` > 0.
    """
    d_in = n_feat + n_time
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed))))
    parts = []
    for fan_out, fan_in in ((HIDDEN, d_in), (HIDDEN, HIDDEN), (2, HIDDEN)):
        w = rng.standard_normal(fan_out * fan_in) / math.sqrt(fan_in)
        b = rng.standard_normal(fan_out) * bias_std if bias_std > 0 else np.zeros(fan_out)
        parts += [w, b]
    return np.concatenate(parts).astype(np.float32)


def mlp_floats(n_time: int = N_TIME, n_feat: int = N_FEATURES) -> int:
    d_in = n_feat + n_time
    return HIDDEN * d_in + HIDDEN + HIDDEN * HIDDEN + HIDDEN + 2 * HIDDEN + 2
