"""GPU parity at the largest tensor the boundary accepts (rows * cols < 2^31).

The oracle cannot step a 2^31-element tensor in a test's time, so these cases
use a property that holds at any size: a tensor made of K exact copies of one
seeded tile (a 1-D tile repeated end to end; a 2-D tile repeated down the
rows) has the tile's row means, column means, mean of r_k and per-feature mean
squares, so after one step from zero state every copy must equal the oracle's
step of the tile alone (to the parity bar; the GPU's sums over 2^31 elements
round differently from the tile's).  Sampled copies are compared, first and
last included.  This exercises the 32-bit offsets, the magic-number division
and the multi-level reductions at the top of their ranges.

Each case needs ~60 GB of device memory (parameters, gradients, state) and
releases it before the next test; it steps every MLP path on the same buffers.
"""
import gc

import numpy as np
import pytest

import oracle
from gpu_harness import IMPLS, compare, hyper_from_cfg, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from learned_optimizer_step_amd import lopt as L  # noqa: E402
from learned_optimizer_step_amd import workloads as W  # noqa: E402

# 1-D: n = 64 * 31 * 601 * 1801 = 2^31 - 64, a tile of 38,464 elements repeated 55,831 times
VEC_TILE, VEC_REPS = 64 * 601, 31 * 1801
# 2-D: 716,064 x 2999 = 2,147,475,936 elements (odd column count: unaligned rows),
# a tile of 8 x 2999 repeated 89,508 times down the rows
MAT_TILE, MAT_REPS = (8, 2999), 89_508


def need_bytes(n, rows, cols):
    return 4 * (2 * n + L.lopt_state_floats(rows, cols)) + (2 << 30)


@pytest.mark.parametrize("kind", ["vector", "matrix"])
@pytest.mark.parametrize("n_feat", [L.LOPT_N_FEATURES, L.LOPT_VELO_FEATURES])
def test_maximum_size_tensor_equals_its_tile(kind, n_feat):
    """One step on every MLP path (the buffers are allocated once; parameters,
    state and step counter are reset between the paths)."""
    if kind == "vector":
        tile_shape, reps = (VEC_TILE,), VEC_REPS
        rows, cols = 1, VEC_TILE * VEC_REPS
    else:
        tile_shape, reps = MAT_TILE, MAT_REPS
        rows, cols = MAT_TILE[0] * MAT_REPS, MAT_TILE[1]
    n = rows * cols
    assert n < 2 ** 31
    free, _ = torch.cuda.mem_get_info()
    if free < need_bytes(n, rows, cols):
        pytest.skip(f"needs {need_bytes(n, rows, cols) / 2**30:.0f} GiB of free device memory")
    say(f"[maxsize] {kind} {rows}x{cols} ({n} elements), n_feat={n_feat}")

    w = W.custom_workload("tile", [tile_shape], grad_std=1e-3, steps=1, wid=120)
    p_tile = W.param_init(w, 0).reshape(tile_shape)
    g_tile = W.grad_at(w, 0, 1).reshape(tile_shape)
    mlp = W.mlp_weights(bias_std=0.1, n_feat=n_feat)
    cfg = L.config_from(n_feat=n_feat)

    rep = (reps,) if kind == "vector" else (reps, 1)
    p_dev_tile = torch.from_numpy(p_tile).cuda()
    p = p_dev_tile.repeat(*rep)
    g = torch.from_numpy(g_tile).cuda().repeat(*rep)
    opt = L.LOpt([p], mlp, cfg)

    hp = hyper_from_cfg(cfg).as_f32()
    st0 = oracle.zero_state(*((1, VEC_TILE) if kind == "vector" else MAT_TILE))
    p_want, st_want, _ = oracle.step_tensor(p_tile, g_tile, st0, 1,
                                            oracle.unpack_mlp(mlp, hp.n_time, hp.n_feat), hp)
    want = dict(p=oracle.as_matrix(p_want), **st_want)

    rng = np.random.default_rng(7)
    picks = sorted(set([0, 1, reps // 2, reps - 1] + rng.choice(reps, 6, replace=False).tolist()))
    views = opt.state_views(0)
    errs = []
    for impl in IMPLS:
        say(f"[maxsize] {kind} n_feat={n_feat} impl={impl}")
        if kind == "vector":
            p.view(reps, -1).copy_(p_dev_tile.view(1, -1).expand(reps, -1))
        else:
            p.view(reps, *MAT_TILE).copy_(p_dev_tile.view(1, *MAT_TILE).expand(reps, *MAT_TILE))
        opt.states[0].zero_()
        opt.t = 0
        L.lopt_set_config(opt.handle, L.config_from(n_feat=n_feat, mlp_impl=impl))
        opt.step([g])
        torch.cuda.synchronize()
        assert opt.t == 1
        for k in picks:
            if kind == "vector":
                sl = slice(k * VEC_TILE, (k + 1) * VEC_TILE)
                got = {"p": p[sl].reshape(1, -1), "m": views["m"][:, :, sl], "v": views["v"][:, sl],
                       "r": views["r"], "c": views["c"][:, sl]}
            else:
                sl = slice(k * MAT_TILE[0], (k + 1) * MAT_TILE[0])
                got = {"p": p[sl], "m": views["m"][:, sl], "v": views["v"][sl], "r": views["r"][:, sl],
                       "c": views["c"]}
            got = {key: t.cpu().numpy() for key, t in got.items()}
            errs += compare(got, want, f"{kind}[impl {impl}, copy {k}]")
    opt.close()
    del opt, p, g, views, p_dev_tile
    gc.collect()
    torch.cuda.empty_cache()
    assert not errs, "\n".join(errs[:20])
