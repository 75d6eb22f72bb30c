"""Scalar-loop twin of the oracle for tiny tensors (pure Python, ``math`` only).

TEST INFRASTRUCTURE.  Written independently of ``small_fc_lopt.py`` (no NumPy,
no vectorisation, one element at a time) so that an indexing, broadcasting or
axis mistake in the vectorised oracle shows up as a disagreement.  It follows
the same statement of the step (PyLO page, "Fused kernel strategy": per-element
features, per-tensor sums of squares, normalisation, MLP, update) and the same
readings listed in ``small_fc_lopt.py``'s header.

Tensors are nested lists ``x[i][j]`` (rows x cols).  fp32 storage is modelled
with ``struct`` round trips.
"""
from __future__ import annotations

import math
import struct


def f32(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


def relu(z: float) -> float:
    return z if z > 0.0 else 0.0


def twin_step(p, g, st, t, w, hp):
    """One step on one tensor.

    p, g: lists of rows.  st: dict with m[a][i][j], v[i][j], r[k][i], c[k][j].
    w: dict with W1 (list of 32 rows), b1, W2, b2, W3, b3 (plain floats).
    hp: object with the oracle's hyperparameter fields (fp32 values).
    Returns (p_new, st_new, raw): p_new and st_new rounded to fp32, raw holds
    the unrounded fp64 update ``u`` and accumulators ``m, v, r, c``.
    """
    R = len(g)
    C = len(g[0])
    n = R * C

    # accumulators, element by element
    m = [[[0.0] * C for _ in range(R)] for _ in range(3)]
    v = [[0.0] * C for _ in range(R)]
    for i in range(R):
        for j in range(C):
            gij = g[i][j]
            for a in range(3):
                b = hp.beta_m[a]
                m[a][i][j] = b * st["m"][a][i][j] + (1.0 - b) * gij
            v[i][j] = hp.beta_v * st["v"][i][j] + (1.0 - hp.beta_v) * gij * gij

    r = [[0.0] * R for _ in range(3)]
    c = [[0.0] * C for _ in range(3)]
    for i in range(R):
        s = 0.0
        for j in range(C):
            s += g[i][j] * g[i][j]
        for k in range(3):
            f = hp.beta_f[k]
            r[k][i] = f * st["r"][k][i] + (1.0 - f) * (s / C + hp.eps_f)
    for j in range(C):
        s = 0.0
        for i in range(R):
            s += g[i][j] * g[i][j]
        for k in range(3):
            f = hp.beta_f[k]
            c[k][j] = f * st["c"][k][j] + (1.0 - f) * (s / R + hp.eps_f)
    rbar = [sum(r[k]) / R for k in range(3)]

    def feats(i, j):
        gij, pij, vij = g[i][j], p[i][j], v[i][j]
        ma = [m[a][i][j] for a in range(3)]
        q = 1.0 / math.sqrt(vij + hp.eps_v)
        rho = [1.0 / math.sqrt(r[k][i] * c[k][j] / rbar[k]) for k in range(3)]
        out = [gij, pij, ma[0], ma[1], ma[2], vij,
               ma[0] * q, ma[1] * q, ma[2] * q, q,
               gij * rho[0], gij * rho[1], gij * rho[2],
               1.0 / math.sqrt(r[0][i]), 1.0 / math.sqrt(r[1][i]), 1.0 / math.sqrt(r[2][i]),
               1.0 / math.sqrt(c[0][j]), 1.0 / math.sqrt(c[1][j]), 1.0 / math.sqrt(c[2][j])]
        for a in range(3):
            for k in range(3):
                out.append(ma[a] * rho[k])
        return out

    nf = getattr(hp, "n_feat", 28)   # the VeLO-shaped variant uses the first 19
    sums = [0.0] * nf
    for i in range(R):
        for j in range(C):
            fe = feats(i, j)
            for d in range(nf):
                sums[d] += fe[d] * fe[d]
    scale = [1.0 / math.sqrt(sums[d] / n + hp.eps_norm) for d in range(nf)]
    tfeat = [math.tanh(t / hp.timescales[q]) for q in range(hp.n_time)]

    p_new = [[0.0] * C for _ in range(R)]
    u_all = [[0.0] * C for _ in range(R)]
    for i in range(R):
        for j in range(C):
            fe = feats(i, j)
            x = [fe[d] * scale[d] for d in range(nf)] + tfeat
            h1 = [relu(w["b1"][o] + sum(w["W1"][o][k] * x[k] for k in range(len(x)))) for o in range(32)]
            h2 = [relu(w["b2"][o] + sum(w["W2"][o][k] * h1[k] for k in range(32))) for o in range(32)]
            d_out = w["b3"][0] + sum(w["W3"][0][k] * h2[k] for k in range(32))
            m_out = w["b3"][1] + sum(w["W3"][1][k] * h2[k] for k in range(32))
            u = d_out * math.exp(m_out * hp.exp_mult) * hp.step_mult
            u_all[i][j] = u
            p_new[i][j] = f32(p[i][j] - hp.lr * u - hp.lr * hp.weight_decay * p[i][j])

    st_new = {
        "m": [[[f32(m[a][i][j]) for j in range(C)] for i in range(R)] for a in range(3)],
        "v": [[f32(v[i][j]) for j in range(C)] for i in range(R)],
        "r": [[f32(r[k][i]) for i in range(R)] for k in range(3)],
        "c": [[f32(c[k][j]) for j in range(C)] for k in range(3)],
    }
    raw = {"u": u_all, "m": m, "v": v, "r": r, "c": c}
    return p_new, st_new, raw


def unpack(flat, n_time, n_feat=28):
    """Packed layout W1[32][n_feat+n_time], b1, W2[32][32], b2, W3[2][32], b3 -> dict of lists."""
    d_in = n_feat + n_time
    flat = [float(x) for x in flat]
    o = 0

    def take(rows, cols):
        nonlocal o
        if cols is None:
            out = flat[o:o + rows]
            o += rows
            return out
        out = [flat[o + r * cols:o + (r + 1) * cols] for r in range(rows)]
        o += rows * cols
        return out

    W1 = take(32, d_in); b1 = take(32, None)
    W2 = take(32, 32); b2 = take(32, None)
    W3 = take(2, 32); b3 = take(2, None)
    assert o == len(flat)
    return {"W1": W1, "b1": b1, "W2": W2, "b2": b2, "W3": W3, "b3": b3}
