"""Pins of the oracle's recursive principal-component split
("ClusterAttention: training-free acceleration of bidirectional attention":
abstract, power-of-two cluster sizes; end of section 2, recursive splits
along principal components into clusters of a preset size).  CPU only."""
import numpy as np
import pytest

from oracle import pcasplit as ops
from oracle import stats as ost


def _rng(s):
    return np.random.default_rng(s)


@pytest.mark.parametrize("n,b", [(1, 4), (4, 4), (5, 4), (64, 8), (100, 8), (1000, 64), (4096, 256), (777, 32)])
def test_exact_power_of_two_sizes(n, b):
    """Every cluster holds exactly b points except at most one (the last),
    ceil(n / b) clusters in all, and n = b 2^k gives only full clusters."""
    X = _rng(n).standard_normal((n, 6))
    out = ops.pca_split(X, b, 128)
    sizes = out["sizes"]
    assert sizes.sum() == n and len(sizes) == ops.n_clusters(n, b) == -(-n // b)
    assert np.all(sizes[:-1] == b) and 1 <= sizes[-1] <= b
    assert sizes.tolist() == ops.leaf_sizes(n, b)
    if n % b == 0:
        assert np.all(sizes == b)


def test_power_of_two_only():
    with pytest.raises(ValueError):
        ops.pca_split(np.zeros((10, 2)), 6, 16)


def test_perm_is_the_stable_sort_of_labels():
    X = _rng(2).standard_normal((500, 5))
    out = ops.pca_split(X, 16, 64)
    perm, seg = ost.counting_sort(out["labels"], out["nclusters"])
    assert np.array_equal(perm, out["perm"]) and np.array_equal(seg, out["seg"])
    for c in range(out["nclusters"]):
        mem = out["perm"][out["seg"][c]:out["seg"][c + 1]]
        assert np.all(np.diff(mem) > 0)
        assert np.allclose(out["cent"][c], X[mem].mean(axis=0))


def test_every_split_is_a_plane_cut_along_the_leading_eigenvector():
    """For every internal node: the direction is a unit eigenvector of the
    subsample's covariance with its largest eigenvalue (checked with a
    symmetric eigensolver, not the SVD the oracle uses), oriented so its
    largest component is positive, and the left child holds the smallest
    projections (a plane separates the children, ties by token index)."""
    r = _rng(3)
    X = np.concatenate([r.standard_normal((300, 7)) * [5, 3, 2, 1, 1, 0.5, 0.2] + 4,
                        r.standard_normal((212, 7)) - 3])
    out = ops.pca_split(X, 16, 64, trace=True)
    assert len(out["nodes"]) == out["nclusters"] - 1
    for level, idx, v in out["nodes"]:
        sub = idx[ops.subsample(idx.size, 64)]
        Y = X[sub] - X[sub].mean(axis=0)
        C = Y.T @ Y
        w = np.linalg.eigvalsh(C)
        assert abs(np.linalg.norm(v) - 1) < 1e-12
        assert np.allclose(C @ v, w[-1] * v, atol=1e-9 * max(1.0, w[-1]))
        assert v[np.argmax(np.abs(v))] > 0
        lo, hi = ops.split_node(X, idx, 16, v)
        assert lo.size == ops.split_sizes(idx.size, 16)[0]
        assert np.max(X[lo] @ v) <= np.min(X[hi] @ v)


def test_points_on_a_line_split_into_runs():
    """Points t * u + c on a line: the principal direction is u, so every
    cluster is a run of consecutive t, in increasing t."""
    r = _rng(4)
    u = r.standard_normal(9)
    u /= np.linalg.norm(u)
    t = r.permutation(np.arange(200, dtype=np.float64))
    X = t[:, None] * u[None, :] + 2.0
    out = ops.pca_split(X, 8, 1000)
    sign = 1 if ops.orient(u)[0] * u[0] > 0 else -1
    for c in range(out["nclusters"]):
        ts = np.sort(t[out["perm"][out["seg"][c]:out["seg"][c + 1]]])
        assert np.all(np.diff(ts) == 1)
    first = t[out["perm"][:8]]
    assert (first.max() < 8) if sign > 0 else (first.min() > 191)


def test_two_separated_blobs_split_first():
    """Two far blobs of b 2^k points each: the first cut separates them."""
    r = _rng(5)
    A = r.standard_normal((128, 4))
    B = r.standard_normal((128, 4)) + [30, 0, 0, 0]
    X = np.concatenate([A, B])[r.permutation(256)]
    out = ops.pca_split(X, 32, 256)
    far = X[:, 0] > 15
    half = out["perm"][:128]
    assert np.all(far[half]) or not np.any(far[half])


def test_anisotropic_cloud_direction_is_its_long_axis():
    r = _rng(6)
    X = r.standard_normal((2000, 5)) * [1, 1, 10, 1, 1]
    v = ops.principal_direction(X[ops.subsample(2000, 512)])
    assert abs(v[2]) > 0.99 and v[2] > 0


def test_subsample_is_strided_and_whole_below_the_cap():
    assert np.array_equal(ops.subsample(10, 16), np.arange(10))
    s = ops.subsample(1000, 100)
    assert s.size == 100 and s[0] == 0 and np.all(np.diff(s) == 10)


def test_degenerate_identical_points():
    X = np.ones((40, 3))
    out = ops.pca_split(X, 8, 16)
    assert out["sizes"].tolist() == [8] * 5
    assert np.array_equal(out["perm"], np.arange(40))
