"""GPU parity on the full-size workloads, every tensor, every MLP path.

The 4096 x 4096 weight with pre-warmed accumulators (1 step), the ViT-B/16
parameter set (147 tensors, 5 steps), the GPT-2 355M set (292 tensors, 1 step),
the Llama-style set (200 tensors, 1.26 G parameters, 1 step) and the ragged
set (10,000 tensors, 1 step), each at its own step count (reading R20), with
the default configuration and the seeded MLP; the comparison is described in
tests/full_parity.py.  (File name: collected after the other GPU tests, so the
oracle worker has their run time to finish.)
"""
import gc
import os

import pytest

import full_parity as FP
from gpu_harness import IMPLS

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu, pytest.mark.timeout(1200)]

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from learned_optimizer_step_amd import lopt as L  # noqa: E402
from learned_optimizer_step_amd import workloads as W  # noqa: E402

_cache = {}


def prepared(key, steps):
    """The reference and the device inputs of one workload (the previous
    workload's are released first)."""
    if _cache.get("key") != key:
        _cache.clear()
        gc.collect()
        torch.cuda.empty_cache()
        want = FP.load_reference(os.environ.get("LOPT_FULL_PARITY_DIR"), key, steps)
        dev = FP.DeviceInputs(W.get_workload(key), steps, torch)
        _cache.update(key=key, want=want, dev=dev)
    return _cache["want"], _cache["dev"]


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("key,steps", FP.WORKLOADS)
def test_every_tensor_of_the_full_workload(key, steps, impl):
    want, dev = prepared(key, steps)
    errs = FP.gpu_compare(W.get_workload(key), steps, want, dev, W.mlp_weights(), L.config_from(mlp_impl=impl), torch)
    assert not errs, "\n".join(errs[:20])
