"""Host-side tests of the C ABI: the library loads, exports every function the
header declares, and validates arguments before any device work.  No kernel is
launched; pointers passed here are fake device addresses that are never
dereferenced (validation and planning are host-only)."""
import ctypes
import os
import re

import pytest

from learned_optimizer_step_amd import lopt as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lopt.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lopt_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("liblopt.so not built")
    return L.load_library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n


def test_default_config_values(lib):
    c = L.lopt_default_config()
    assert list(c.beta_m) == pytest.approx([0.1, 0.5, 0.9])
    assert c.beta_v == pytest.approx(0.999)
    assert list(c.beta_f) == pytest.approx([0.9, 0.99, 0.999])
    assert c.eps_v == pytest.approx(1e-8) and c.eps_f == pytest.approx(1e-20)
    assert c.eps_norm == pytest.approx(1e-30)
    assert c.exp_mult == pytest.approx(1e-3) and c.step_mult == pytest.approx(1e-3)
    assert c.lr == 1.0 and c.weight_decay == 0.0 and c.n_time == 11
    assert c.n_feat == 28 and c.mlp_impl == L.LOPT_MLP_AUTO
    assert c.launch == L.LOPT_LAUNCH_AUTO   # last field: the struct layouts agree
    assert list(c.timescales) == pytest.approx([1, 3, 10, 30, 100, 300, 1e3, 3e3, 1e4, 3e4, 1e5])
    assert lib.lopt_default_config(None) == L.LOPT_ERR_INVALID_ARGUMENT
    assert "NULL" in L.lopt_last_error()


def test_sizes(lib):
    assert L.lopt_mlp_floats(28, 11) == 2402
    assert L.lopt_mlp_floats(28, 0) == 32 * 28 + 32 + 1024 + 32 + 64 + 2
    assert L.lopt_mlp_floats(19, 11) == 32 * 30 + 32 + 1024 + 32 + 64 + 2 == 2114
    assert L.lopt_mlp_floats(28, 12) == 0 and L.lopt_mlp_floats(28, -1) == 0
    assert L.lopt_mlp_floats(20, 11) == 0 and L.lopt_mlp_floats(0, 11) == 0
    assert L.lopt_state_floats(4, 5) == 4 * 20 + 3 * 9
    assert L.lopt_state_floats(1, 7) == 4 * 7 + 3 * 8
    assert L.lopt_state_floats(0, 3) == 0


BASE = 1 << 40  # fake, 256-byte aligned device addresses


def fake_list(shapes, gap=1 << 30, with_grads=True):
    ts, a = [], BASE
    for r, c in shapes:
        n = r * c
        p, a = a, a + gap
        g, a = a, a + gap
        s, a = a, a + gap
        ts.append(L.lopt_tensor(p, g if with_grads else None, s, r, c))
    return ts


def ws_status(ts):
    out = ctypes.c_size_t()
    st = L.load_library().lopt_workspace_bytes(None, L.tensor_array(ts), len(ts), ctypes.byref(out))
    return st, out.value


def test_workspace_bytes_grows_with_list(lib):
    st1, b1 = ws_status(fake_list([(256, 256)]))
    st2, b2 = ws_status(fake_list([(256, 256), (1, 1000), (3, 7)]))
    assert st1 == L.LOPT_OK and st2 == L.LOPT_OK and b2 > b1 > 0 and b1 % 256 == 0
    st0, b0 = ws_status([])
    assert st0 == L.LOPT_OK


def test_workspace_bytes_accepts_null_grads(lib):
    st, b = ws_status(fake_list([(8, 8), (1, 5)], with_grads=False))
    assert st == L.LOPT_OK and b > 0


@pytest.mark.parametrize("mutate,code", [
    (lambda t: setattr(t, "rows", 0), L.LOPT_ERR_INVALID_ARGUMENT),
    (lambda t: setattr(t, "cols", -3), L.LOPT_ERR_INVALID_ARGUMENT),
    (lambda t: setattr(t, "param", None), L.LOPT_ERR_INVALID_ARGUMENT),
    (lambda t: setattr(t, "state", None), L.LOPT_ERR_INVALID_ARGUMENT),
    (lambda t: setattr(t, "param", t.param + 2), L.LOPT_ERR_UNSUPPORTED),
    (lambda t: (setattr(t, "rows", 1 << 16), setattr(t, "cols", 1 << 15)), L.LOPT_ERR_UNSUPPORTED),
    (lambda t: (setattr(t, "rows", 2), setattr(t, "cols", 1 << 28)), L.LOPT_ERR_UNSUPPORTED),
    (lambda t: setattr(t, "grad", t.param), L.LOPT_ERR_INVALID_ARGUMENT),
    (lambda t: setattr(t, "grad", t.state + 64), L.LOPT_ERR_INVALID_ARGUMENT),
    (lambda t: setattr(t, "state", t.param + 4), L.LOPT_ERR_INVALID_ARGUMENT),
])
def test_validation_codes(lib, mutate, code):
    ts = fake_list([(16, 16), (1, 9)])
    mutate(ts[0])
    st, _ = ws_status(ts)
    assert st == code, L.lopt_last_error()
    assert L.lopt_last_error() != ""


def test_overlap_between_tensors_is_rejected(lib):
    ts = fake_list([(16, 16), (16, 16)])
    ts[1].param = ts[0].state + 8  # inside tensor 0's state
    st, _ = ws_status(ts)
    assert st == L.LOPT_ERR_INVALID_ARGUMENT and "overlap" in L.lopt_last_error()


def test_shared_gradient_buffer_is_allowed(lib):
    ts = fake_list([(16, 16), (16, 16)])
    ts[1].grad = ts[0].grad  # read-only aliasing between gradients is harmless
    st, _ = ws_status(ts)
    assert st == L.LOPT_OK


def test_create_rejects_bad_config_without_device(lib):
    w = (ctypes.c_float * 2402)()
    h = ctypes.c_void_p()
    c = L.lopt_default_config()
    c.n_time = 12
    assert lib.lopt_create(ctypes.byref(c), w, ctypes.byref(h)) == L.LOPT_ERR_INVALID_ARGUMENT
    c = L.config_from(beta_m=[0.1, 1.5, 0.9])
    assert lib.lopt_create(ctypes.byref(c), w, ctypes.byref(h)) == L.LOPT_ERR_INVALID_ARGUMENT
    c = L.config_from(eps_v=-1.0)
    assert lib.lopt_create(ctypes.byref(c), w, ctypes.byref(h)) == L.LOPT_ERR_INVALID_ARGUMENT
    c = L.config_from(timescales=[1.0, 0.0])
    assert lib.lopt_create(ctypes.byref(c), w, ctypes.byref(h)) == L.LOPT_ERR_INVALID_ARGUMENT
    c = L.config_from(n_feat=20)
    assert lib.lopt_create(ctypes.byref(c), w, ctypes.byref(h)) == L.LOPT_ERR_INVALID_ARGUMENT
    assert "n_feat" in L.lopt_last_error()
    c = L.config_from(mlp_impl=L.LOPT_MLP_BF16X8 + 1)
    assert lib.lopt_create(ctypes.byref(c), w, ctypes.byref(h)) == L.LOPT_ERR_INVALID_ARGUMENT
    assert "mlp_impl" in L.lopt_last_error()
    for bad in (-1, L.LOPT_LAUNCH_SINGLE + 1):
        c = L.config_from(launch=bad)
        assert lib.lopt_create(ctypes.byref(c), w, ctypes.byref(h)) == L.LOPT_ERR_INVALID_ARGUMENT
        assert "launch" in L.lopt_last_error()
    c = L.lopt_default_config()
    assert lib.lopt_create(ctypes.byref(c), None, ctypes.byref(h)) == L.LOPT_ERR_INVALID_ARGUMENT
    assert lib.lopt_create(None, w, ctypes.byref(h)) == L.LOPT_ERR_INVALID_ARGUMENT
    assert h.value is None


def test_create_refuses_fp16x3_for_weights_outside_its_range_without_device(lib):
    """LOPT_MLP_FP16X3 needs weights below 2^15 and a constant-term shift of at
    most 14 (first-layer row-feature weights times sqrt(2^31)); otherwise
    lopt_create refuses it before touching the device."""
    h = ctypes.c_void_p()
    c = L.config_from(mlp_impl=L.LOPT_MLP_FP16X3)
    big = (ctypes.c_float * 2402)()
    big[5] = 40000.0                      # a W1 entry beyond fp16's piece range
    assert lib.lopt_create(ctypes.byref(c), big, ctypes.byref(h)) == L.LOPT_ERR_UNSUPPORTED
    assert "LOPT_MLP_FP16X3" in L.lopt_last_error()
    rowf = (ctypes.c_float * 2402)()
    rowf[13] = 30000.0                    # W1[0][13]: row term up to ~7e8, shift 15
    assert lib.lopt_create(ctypes.byref(c), rowf, ctypes.byref(h)) == L.LOPT_ERR_UNSUPPORTED
    assert h.value is None


def test_null_handle_calls(lib):
    t = ctypes.c_int64()
    assert lib.lopt_get_step(None, ctypes.byref(t)) == L.LOPT_ERR_INVALID_ARGUMENT
    assert lib.lopt_set_step(None, 3) == L.LOPT_ERR_INVALID_ARGUMENT
    assert lib.lopt_step(None, None, 0, None) == L.LOPT_ERR_INVALID_ARGUMENT
    assert lib.lopt_init_state(None, None, 0, None, 0, None) == L.LOPT_ERR_INVALID_ARGUMENT
    assert lib.lopt_set_tensor_hyper(None, None, None, 0) == L.LOPT_ERR_INVALID_ARGUMENT
    impl = ctypes.c_int32()
    assert lib.lopt_get_mlp_impl(None, ctypes.byref(impl)) == L.LOPT_ERR_INVALID_ARGUMENT
    assert lib.lopt_get_launch(None, ctypes.byref(impl)) == L.LOPT_ERR_INVALID_ARGUMENT
    out = (ctypes.c_float * L.LOPT_STAT_FLOATS)()
    assert lib.lopt_get_tensor_stats(None, out, 1) == L.LOPT_ERR_INVALID_ARGUMENT
    lib.lopt_destroy(None)  # no-op


def test_binding_has_the_c_names():
    for n in declared_functions():
        assert hasattr(L, n), n


def test_numpy_tensor_table_matches_the_struct_layout(lib):
    # LOpt hands lopt_step a persistent numpy table instead of ctypes structs
    import numpy as np
    assert L._TENSOR_DTYPE.itemsize == ctypes.sizeof(L.lopt_tensor)
    ts = fake_list([(16, 16), (1, 9), (300, 7)])
    tab = np.zeros(3, L._TENSOR_DTYPE)
    for i, t in enumerate(ts):
        tab[i] = (t.param, t.grad, t.state, t.rows, t.cols)
    out = ctypes.c_size_t()
    st = lib.lopt_workspace_bytes(None, tab.ctypes.data_as(ctypes.POINTER(L.lopt_tensor)), 3, ctypes.byref(out))
    assert st == L.LOPT_OK
    assert (st, out.value) == ws_status(ts)
    tab[1]["rows"] = 0    # the library reads the rows field where the struct has it
    st = lib.lopt_workspace_bytes(None, tab.ctypes.data_as(ctypes.POINTER(L.lopt_tensor)), 3, ctypes.byref(out))
    assert st == L.LOPT_ERR_INVALID_ARGUMENT


def test_matrix_view_of_parameter_shapes():
    # scalar 1 x 1, vector 1 x n, matrix as given, more dimensions: first x product of the rest
    assert L.matrix_shape(()) == (1, 1)
    assert L.matrix_shape((5,)) == (1, 5)
    assert L.matrix_shape((3, 4)) == (3, 4)
    assert L.matrix_shape((8, 3, 5, 5)) == (8, 75)
    assert L.matrix_shape((2, 1, 1)) == (2, 1)


def test_sharded_planning_and_validation_without_device(lib):
    """Row-shard bindings: workspace size (host-only planning), the global
    shapes the shards must fit, and the calls that need a binding."""
    ts = fake_list([(16, 16), (1, 9), (300, 7)])
    arr = (L.lopt_tensor * 3)(*ts)
    out = ctypes.c_size_t()
    assert lib.lopt_workspace_bytes(None, arr, 3, ctypes.byref(out)) == L.LOPT_OK
    plain = out.value
    import numpy as np
    good = np.array([64, 16, 1, 20, 900, 7], dtype=np.int64)       # matrix rows 16 of 64, 9 of 20 elements, ...
    assert lib.lopt_workspace_bytes_sharded(None, arr, 3, good.ctypes.data_as(ctypes.c_void_p),
                                            ctypes.byref(out)) == L.LOPT_OK
    # the exchange buffers: 16 + 1 + 7 column sums, 32 floats per tensor (each 256-byte aligned)
    assert out.value >= plain + 4 * (16 + 1 + 7) + 4 * 32 * 3
    bad = [np.array([64, 17, 1, 20, 900, 7], dtype=np.int64),    # other column count
           np.array([8, 16, 1, 20, 900, 7], dtype=np.int64),     # fewer rows than the shard
           np.array([64, 16, 1, 5, 900, 7], dtype=np.int64),     # shorter than the 1-D shard
           np.array([64, 16, 2, 9, 900, 7], dtype=np.int64),     # a 1 x 9 shard of a matrix with 9 columns? rows 2
           np.array([0, 16, 1, 20, 900, 7], dtype=np.int64)]
    expect = [L.LOPT_ERR_INVALID_ARGUMENT] * 3 + [L.LOPT_OK, L.LOPT_ERR_INVALID_ARGUMENT]
    for dims, want in zip(bad, expect):
        got = lib.lopt_workspace_bytes_sharded(None, arr, 3, dims.ctypes.data_as(ctypes.c_void_p), ctypes.byref(out))
        assert got == want, (dims, got, L.lopt_last_error())
    assert lib.lopt_workspace_bytes_sharded(None, arr, 3, None, ctypes.byref(out)) == L.LOPT_ERR_INVALID_ARGUMENT
    p1, p2 = ctypes.c_void_p(), ctypes.c_void_p()
    n1, n2 = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.lopt_get_shard_sums(None, ctypes.byref(p1), ctypes.byref(n1), ctypes.byref(p2),
                                   ctypes.byref(n2)) == L.LOPT_ERR_INVALID_ARGUMENT
    assert lib.lopt_step_shard(None, arr, 3, 0, None) == L.LOPT_ERR_INVALID_ARGUMENT
    assert lib.lopt_init_state_sharded(None, arr, 3, good.ctypes.data_as(ctypes.c_void_p), None, 0,
                                       None) == L.LOPT_ERR_INVALID_ARGUMENT


def test_binding_classes_have_their_methods():
    """The GPU tests use these; a CPU run checks that they exist."""
    for m in ("step", "t", "set_tensor_hyper", "tensor_stats", "state_views", "close", "shard_sums",
              "step_shard_phase", "step_sharded"):
        assert hasattr(L.LOpt, m), m
    for m in ("step", "state_dict", "load_state_dict", "zero_grad"):
        assert hasattr(L.LearnedOptimizer, m), m
    assert callable(L.allreduce_through_host)
