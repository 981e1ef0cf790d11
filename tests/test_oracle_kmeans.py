"""Pins for the oracle's k-means (Semantic-Aware Smoothing steps a-b).

note.zhuruihan.top, "Semantic-Aware Smoothing": k-means over tokens along the
sequence axis; each group's centroid is its mean value.  paper.rainbus.top,
method paragraph, SAS (a)-(b).

Pinned against: SciPy's kmeans2 (an independent library Lloyd's k-means whose
empty clusters also keep their previous centroid), run one iteration at a time
with the centroids rounded to fp32 between iterations; exhaustive search over
all partitions of tiny inputs; the page's sky-vector example; and invariants
(objective never rises, group residual means vanish).
"""
import itertools
import json
import os
import warnings

import numpy as np
import pytest
import torch
from scipy.cluster.vq import kmeans2

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _blobs(rng, n, d, k, spread=0.3):
    centers = rng.standard_normal((k, d)) * 3
    lab = rng.integers(0, k, n)
    return (centers[lab] + spread * rng.standard_normal((n, d))).astype(np.float32)


@pytest.mark.parametrize("seed,n,d,k,iters", [(0, 300, 8, 5, 6), (1, 1000, 64, 16, 10),
                                              (2, 257, 3, 7, 4), (3, 500, 128, 32, 3)])
def test_kmeans_matches_scipy_lloyd(oracle, seed, n, d, k, iters):
    rng = np.random.default_rng(seed)
    X = _blobs(rng, n, d, k)
    C0 = X[rng.choice(n, k, replace=False)].copy()
    C_or, pi_or = oracle.kmeans(X, C0, iters)
    C = C0.astype(np.float64)
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        for _ in range(iters):
            C, lab = kmeans2(X.astype(np.float64), C, iter=1, minit="matrix")
            C = C.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(pi_or, lab)
    np.testing.assert_array_equal(C_or, C.astype(np.float32))


def test_empty_cluster_keeps_centroid(oracle):
    X = np.array([[0.0], [0.1], [10.0]], np.float32)
    C0 = np.array([[0.0], [10.0], [1000.0]], np.float32)  # cluster 2 gets nobody
    C, pi = oracle.kmeans(X, C0, 2)
    assert pi.tolist() == [0, 0, 1]
    assert C[2, 0] == 1000.0 and C[1, 0] == 10.0
    assert C[0, 0] == np.float32(np.float64(np.float32(0.1)) / 2)


def test_assign_tie_goes_to_smallest_index(oracle):
    X = np.array([[1.0, 0.0]], np.float32)
    C = np.array([[2.0, 0.0], [0.0, 0.0], [1.0, 1.0], [1.0, -1.0]], np.float32)
    assert oracle.assign(X, C).tolist() == [0]  # all four at distance 1
    assert oracle.assign(X, C[1:]).tolist() == [0]


def _objective(X, C, pi):
    diff = X.astype(np.float64) - C.astype(np.float64)[pi]
    return float((diff * diff).sum())


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_tiny(oracle, seed):
    """All C^N partitions of N<=8 points: Lloyd started from the optimal
    partition's means stays there, and Lloyd from any start is never better
    than the exhaustive optimum."""
    rng = np.random.default_rng(100 + seed)
    N, d, k = 7, 2, 3
    X = (rng.standard_normal((N, d)) * 2).astype(np.float32)
    X64 = X.astype(np.float64)
    best, best_lab = np.inf, None
    for lab in itertools.product(range(k), repeat=N):
        lab = np.array(lab)
        if len(set(lab.tolist())) < k:
            continue
        cost = sum(((X64[lab == j] - X64[lab == j].mean(0)) ** 2).sum() for j in range(k))
        if cost < best:
            best, best_lab = cost, lab
    # brute-force argmin check of the assign step on a dense grid of centroids
    C = (rng.standard_normal((k, d)) * 2).astype(np.float32)
    D = ((X64[:, None, :] - C.astype(np.float64)[None]) ** 2).sum(-1)
    assert oracle.assign(X, C).tolist() == D.argmin(1).tolist()
    # optimum is a fixed point
    Copt = np.stack([X64[best_lab == j].mean(0) for j in range(k)]).astype(np.float32)
    C1, pi1 = oracle.kmeans(X, Copt, 3)
    assert pi1.tolist() == best_lab.tolist()
    assert abs(_objective(X, C1, pi1) - best) <= 1e-6 * max(best, 1)
    # any start is no better than the optimum
    for s in range(5):
        C0 = X[np.random.default_rng(s).choice(N, k, replace=False)]
        C2, pi2 = oracle.kmeans(X, C0, 10)
        assert _objective(X, C2, oracle.assign(X, C2)) >= best * (1 - 1e-9)


def test_sky_example_centroid(oracle):
    g = json.load(open(os.path.join(GOLD, "sky_centroid.json")))
    X = np.array(g["tokens"], np.float32)
    C, cnt = oracle.update(X, np.zeros(3, np.int32), np.zeros((1, 4), np.float32))
    assert cnt.tolist() == [3]
    np.testing.assert_allclose(C[0], g["centroid_4dp"], atol=5e-5)
    np.testing.assert_array_equal(C[0], (X.astype(np.float64).sum(0) / 3).astype(np.float32))


def test_objective_non_increasing_and_zero_mean_groups(oracle):
    from means_residual_compression_amd import synth
    X = synth.video_cache(0, 0, 1, 8, 8, 8, 32, 50.0, torch.float32)[0].numpy()
    rng = np.random.default_rng(9)
    C = X[rng.choice(len(X), 16, replace=False)].copy()
    prev = np.inf
    for _ in range(8):
        pi = oracle.assign(X, C)
        obj = _objective(X, C, pi)
        assert obj <= prev * (1 + 1e-12)
        prev = obj
        C, cnt = oracle.update(X, pi, C)
        # after the update, the members' residuals average to ~0 per group
        for j in np.nonzero(cnt)[0]:
            m = X[pi == j].astype(np.float64) - C[j].astype(np.float64)
            scale = np.abs(X[pi == j]).max() + 1e-30
            assert np.all(np.abs(m.mean(0)) <= 4 * np.finfo(np.float32).eps * scale)
