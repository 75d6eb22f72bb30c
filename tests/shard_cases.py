"""The tensor list and the cut into shards shared by test_gpu_sharded.py and
its per-rank process script sharded_rank.py."""
import numpy as np

# every tensor has at least 3 rows (2-D) or elements (1-D): one per shard for 3 shards
SHAPES = [(64, 96), (1, 5000), (300, 7), (129, 257), (33, 64), (3, 3), (1, 3), (7, 4096), (9, 65), (1, 40000)]


def shard_range(t, k, ranks):
    """Rows (2-D) or elements (1-D) [a, b) of shard k of tensor t."""
    N = t.rows if t.rows > 1 else t.cols
    return N * k // ranks, N * (k + 1) // ranks


def take(x, t, a, b):
    """Shard [a, b) of x, the whole tensor t's values."""
    x = np.asarray(x).reshape(t.rows, t.cols)
    return np.ascontiguousarray(x[a:b] if t.rows > 1 else x[:, a:b])
