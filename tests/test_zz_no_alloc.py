"""lopt_init_state_static, the binding that allocates nothing, against lopt_init_state.

Two calls in a row, the second with a smaller tensor list: each list is bound
with lopt_init_state_static (the plan in the library's static device array)
and stepped three times with fresh gradient buffers (their addresses change
every step, so the copies from host memory are exercised) and then once with
per-tensor learning rates and weight decays; the parameters and every
accumulator must equal, bit for bit, the same steps of the same list bound with
lopt_init_state and a caller workspace (the kernels and the plan are the same).
Then: the first handle's binding was replaced by the second's, so its step is
refused with LOPT_ERR_STATE until it binds again, and a list whose workspace
exceeds LOPT_STATIC_SCRATCH_BYTES is refused with LOPT_ERR_WORKSPACE.
"""

import numpy as np
import pytest

from gpu_harness import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from learned_optimizer_step_amd import lopt as L  # noqa: E402
from learned_optimizer_step_amd import workloads as W  # noqa: E402

STEPS = 3
LR, WD = [0.5, 1.5, 0.8, 1.0, 0.3], [0.01, 0.0, 0.2, 0.05, 0.1]


class Run:
    """A tensor list on the GPU with its own parameters, state buffers and handle."""

    def __init__(self, w, mlp, static):
        self.w = w
        self.params = [torch.from_numpy(W.param_init(w, i).reshape(t.rows, t.cols)).cuda() for i, t in enumerate(w.tensors)]
        self.states = [torch.zeros(L.lopt_state_floats(t.rows, t.cols), dtype=torch.float32, device="cuda")
                       for t in w.tensors]
        self.handle = L.lopt_create(L.lopt_default_config(), mlp)
        self.stream = torch.cuda.current_stream().cuda_stream
        ts = self.table([None] * len(w.tensors))
        if static:
            L.lopt_init_state_static(self.handle, ts, self.stream)
            self.ws = None
        else:
            nb = L.lopt_workspace_bytes(self.handle, ts)
            self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
            L.lopt_init_state(self.handle, ts, self.ws.data_ptr(), nb, self.stream)

    def table(self, grads):
        return [L.lopt_tensor(p.data_ptr(), None if g is None else g.data_ptr(), s.data_ptr(), t.rows, t.cols)
                for p, g, s, t in zip(self.params, grads, self.states, self.w.tensors)]

    def step(self, t):
        grads = [torch.from_numpy(W.grad_at(self.w, i, t).reshape(tt.rows, tt.cols)).cuda()
                 for i, tt in enumerate(self.w.tensors)]
        L.lopt_step(self.handle, self.table(grads), self.stream)
        self._grads = grads       # alive until the step has run

    def result(self):
        torch.cuda.synchronize()
        return [(p.cpu().numpy(), s.cpu().numpy()) for p, s in zip(self.params, self.states)]

    def close(self):
        torch.cuda.synchronize()
        L.lopt_destroy(self.handle)


def run_both(w, mlp):
    """The static binding and the workspace binding of w, stepped alike."""
    static, regular = Run(w, mlp, True), Run(w, mlp, False)
    n = len(w.tensors)
    for r in (static, regular):
        for t in range(1, STEPS + 1):
            r.step(t)
        L.lopt_set_tensor_hyper(r.handle, LR[:n], WD[:n], n)
        r.step(STEPS + 1)
    return static, regular


def assert_same(a, b, label):
    for i, ((pa, sa), (pb, sb)) in enumerate(zip(a, b)):
        assert np.array_equal(pa, pb), f"{label}: tensor {i} parameters differ"
        assert np.array_equal(sa, sb), f"{label}: tensor {i} state differs"


def test_static_binding_equals_the_workspace_binding_on_two_lists():
    mlp = W.mlp_weights(bias_std=0.1)
    big = W.custom_workload("noalloc1", [(300, 512), (7000,), (64, 64), (33, 65), (1000, 3)], grad_std=1e-2,
                            steps=STEPS, wid=190)
    small = W.custom_workload("noalloc2", [(40, 64), (100,)], grad_std=1e-2, steps=STEPS, wid=191)

    say("[no-alloc] first call: 5 tensors")
    s1, r1 = run_both(big, mlp)
    assert L.lopt_get_step(s1.handle) == STEPS + 1
    assert_same(s1.result(), r1.result(), "first list")
    stats_s = L.lopt_get_tensor_stats(s1.handle, 5)
    stats_r = L.lopt_get_tensor_stats(r1.handle, 5)
    assert np.array_equal(stats_s, stats_r)
    r1.close()

    say("[no-alloc] second call: 2 tensors")
    s2, r2 = run_both(small, mlp)
    assert_same(s2.result(), r2.result(), "second list")
    r2.close()

    # the second static binding took the array over from the first handle
    with pytest.raises(L.LoptError) as e:
        s1.step(STEPS + 2)
    assert e.value.status == L.LOPT_ERR_STATE
    with pytest.raises(L.LoptError) as e:
        L.lopt_get_step(s1.handle)
    assert e.value.status == L.LOPT_ERR_STATE
    # binding again works (and takes the array back from the second handle)
    L.lopt_init_state_static(s1.handle, s1.table([None] * 5), s1.stream)
    s1.step(1)
    assert L.lopt_get_step(s1.handle) == 1
    with pytest.raises(L.LoptError) as e:
        s2.step(STEPS + 2)
    assert e.value.status == L.LOPT_ERR_STATE
    s1.close()
    s2.close()


def test_static_binding_refuses_a_list_beyond_its_size():
    # twelve 32000 x 2048 tensors need more workspace than the static array;
    # the library refuses them on the host before any device work (the tensor
    # addresses are never used)
    h = L.lopt_create(L.lopt_default_config(), W.mlp_weights())
    base = 1 << 44
    ts = []
    for k in range(12):
        ts.append(L.lopt_tensor(base, base + (1 << 36), base + (2 << 36), 32000, 2048))
        base += 3 << 36
    assert L.lopt_workspace_bytes(h, ts) > L.LOPT_STATIC_SCRATCH_BYTES
    with pytest.raises(L.LoptError) as e:
        L.lopt_init_state_static(h, ts, torch.cuda.current_stream().cuda_stream)
    assert e.value.status == L.LOPT_ERR_WORKSPACE
    assert "static scratch" in str(e.value)
    L.lopt_destroy(h)
