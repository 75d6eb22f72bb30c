"""The oracle's network shape against the sizes the PyLO page states."""
import json
import os

import numpy as np

from oracle import HIDDEN, N_FEATURES, Hyper, mlp_size, unpack_mlp

HERE = os.path.dirname(os.path.abspath(__file__))


def test_network_shape_matches_page():
    with open(os.path.join(HERE, "golden", "pylo_page_structure.json")) as f:
        page = json.load(f)
    hp = Hyper()
    assert N_FEATURES + hp.n_time == page["d_feat_small_fc_lopt"]["value"]
    assert HIDDEN == page["d_hidden"]["value"]
    m = unpack_mlp(np.zeros(mlp_size(hp.n_time)), hp.n_time)
    assert m.W1.shape == (HIDDEN, 39) and m.W3.shape == (page["outputs"]["value"], HIDDEN)
    # input, two hidden and output layers: three weight matrices
    assert page["mlp_layers"]["value"] - 1 == 3
    # per-tensor statistics: one per normalised feature.  The page's 30..39
    # counts the step features too; here they bypass normalisation (a tensor-
    # constant feature normalised over its own tensor would become +-1).
    lo, hi = page["stats_scalars_range"]["value"]
    assert N_FEATURES < lo <= N_FEATURES + hp.n_time <= hi
