"""Pins for the oracle's stage plumbing: the centroid subtraction, the stage
inputs of later stages, and the seeded cold-start draw.

paper.rainbus.top, method paragraph: SAS (c) subtracts each token's centroid;
PRQ runs stage t on the residual R(t-1) of the previous stage, so a cold stage
starts from rows of R(t-1).  The draw of those rows is a pinned reading
(splitmix64 seeding a partial Fisher-Yates shuffle); its generator is checked
against the published splitmix64 output sequence.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_round(x32):
    """fp32 array -> nearest bf16 values (ties to even), as fp32."""
    u = np.ascontiguousarray(x32, np.float32).view(np.uint32).astype(np.uint64)
    b = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return b.astype(np.uint32).view(np.float32)


def test_subtract_hand_rows(oracle):
    g = json.load(open(os.path.join(GOLDEN, "subtract.json")))
    R = np.array(g["tokens"], np.float32)
    C = np.array(g["centroids"], np.float32)
    out = oracle.subtract(R, np.array(g["assign"], np.int32), C)
    np.testing.assert_array_equal(out, np.array(g["residuals"], np.float32))


def test_path_subtracts_the_stored_bf16_centroid(oracle):
    """Two tokens of one cluster: 1.0 and 1 + 2^-7 in every channel.  Their mean
    1 + 2^-8 is a bf16 tie and rounds to 1.0 (even mantissa), so the stored
    centroid is 1.0 and token 0's residual is exactly zero: its scales are 0
    and it reconstructs exactly.  Subtracting the unrounded mean would leave
    -2^-8 in token 0 and a nonzero scale."""
    d = 8
    X = np.array([[1.0] * d, [1.0078125] * d], np.float32)
    Xb = (X.view(np.uint32) >> 16).astype(np.uint16)[None]
    rec = oracle.compress(Xb, C=1, T=1, iters=1, bits=2, G=8, init_idx=np.zeros((1, 1, 1), np.int32))
    assert rec["cent"][0, 0, 0, 0] == 0x3F80          # bf16 1.0
    np.testing.assert_array_equal(rec["cache"][0, 0, 0], np.float32(1.00390625))
    assert rec["scales"][0, 0, 0] == 0 and rec["scales"][0, 1, 0] != 0
    out = oracle.decompress(rec["codes"], rec["scales"], rec["assign"], rec["cent"], 2, 8)
    np.testing.assert_array_equal(out[0, 0], Xb[0, 0])


def test_stage_two_starts_from_rows_of_the_first_residual(oracle):
    """T = 2, one iteration per stage.  Brute force in numpy: R(1) = X -
    bf16(C1)[pi1] from the stage-1 record, stage-2 start = R(1)[idx2], stage-2
    assignment = argmin of fp64 distances to those rows (first index on
    ties), stage-2 centroid = bf16 of the fp64 group mean.  Two well
    separated clumps make R(1) rows and X rows lead to different stage-2
    assignments, which the test also checks, so the two readings cannot
    agree by accident."""
    rng = np.random.default_rng(5)
    N, d, C = 64, 16, 4
    X = rng.normal(0.0, 1.0, (N, d)) + np.where(np.arange(N)[:, None] < N // 2, 30.0, -30.0)
    X = _bf16_round(X.astype(np.float32))
    Xb = (X.view(np.uint32) >> 16).astype(np.uint16)[None]
    idx = np.array([[[0, 40, 1, 41], [3, 50, 10, 60]]], np.int32)
    rec = oracle.compress(Xb, C=C, T=2, iters=1, bits=2, G=16, init_idx=idx)
    c1 = (rec["cent"][0, 0].astype(np.uint32) << 16).view(np.float32)
    pi1 = rec["assign"][0, 0].astype(np.int64)
    R1 = (X - c1[pi1]).astype(np.float32)                # fp32 subtraction
    start = R1[idx[0, 1]].astype(np.float64)
    D = ((R1.astype(np.float64)[:, None, :] - start[None]) ** 2).sum(-1)
    pi2 = D.argmin(1)
    np.testing.assert_array_equal(rec["assign"][0, 1], pi2)
    c2 = np.stack([R1[pi2 == j].astype(np.float64).mean(0) if np.any(pi2 == j) else start[j]
                   for j in range(C)]).astype(np.float32)
    np.testing.assert_array_equal((rec["cent"][0, 1].astype(np.uint32) << 16).view(np.float32),
                                  _bf16_round(c2))
    # the other reading (rows of X) assigns differently here
    Dx = ((R1.astype(np.float64)[:, None, :] - X[idx[0, 1]].astype(np.float64)[None]) ** 2).sum(-1)
    assert not np.array_equal(Dx.argmin(1), pi2)


def test_splitmix64_published_sequence(oracle):
    """The first outputs of splitmix64 from state 0, as listed with the
    published reference implementation."""
    assert oracle.splitmix64(0, 4) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                       0x06C45D188009454F, 0xF88BB8A8724C81EC]


@pytest.mark.parametrize("N,C", [(1, 1), (7, 7), (10, 3), (1000, 256), (32760, 256)])
def test_sample_rows_distinct_and_in_range(oracle, N, C):
    for h, t in ((0, 1), (5, 2), (11, 4)):
        r = oracle.sample_rows(N, C, 1234, h, t)
        assert r.min() >= 0 and r.max() < N and len(np.unique(r)) == C
    if C == N:  # a full draw is a permutation
        assert sorted(oracle.sample_rows(N, C, 9, 0, 1).tolist()) == list(range(N))


def test_sample_rows_hand_steps(oracle):
    """Partial Fisher-Yates written out for N = 5, C = 3 from the generator's
    own outputs: swap position j with j + (z_j mod (5 - j))."""
    seed, h, t = 77, 2, 3
    st = seed ^ ((0x9E3779B97F4A7C15 * (h + 1)) % 2**64) ^ ((0xD1B54A32D192ED03 * t) % 2**64)
    z = oracle.splitmix64(st, 3)
    perm = [0, 1, 2, 3, 4]
    for j in range(3):
        k = j + z[j] % (5 - j)
        perm[j], perm[k] = perm[k], perm[j]
    assert oracle.sample_rows(5, 3, seed, h, t).tolist() == perm[:3]


def test_sample_rows_uniform_over_orderings(oracle):
    """N = 3, C = 3 over many seeds: each of the 6 orderings about 1/6 of the
    time (modulo bias is below 2^-60 here)."""
    counts = {}
    for seed in range(3000):
        key = tuple(oracle.sample_rows(3, 3, seed, 0, 1).tolist())
        counts[key] = counts.get(key, 0) + 1
    assert len(counts) == 6
    assert all(abs(c - 500) < 100 for c in counts.values())


def test_seeded_compress_uses_the_drawn_rows(oracle):
    """compress(seed=s) equals compress(init_idx=the rows sample_rows draws for
    each head and stage)."""
    rng = np.random.default_rng(3)
    H, N, d, C, T = 2, 200, 16, 8, 2
    X = rng.normal(0, 1, (H, N, d)).astype(np.float32)
    idx = np.array([[oracle.sample_rows(N, C, 42, h, t + 1) for t in range(T)] for h in range(H)],
                   np.int32)
    a = oracle.compress(X, C=C, T=T, iters=3, bits=2, G=16, seed=42)
    b = oracle.compress(X, C=C, T=T, iters=3, bits=2, G=16, init_idx=idx)
    for k in ("codes", "scales", "assign", "cent", "cache"):
        np.testing.assert_array_equal(a[k], b[k])


def test_threaded_assignment_changes_nothing(oracle):
    """The oracle splits one head's assignment over threads when the call has
    fewer heads than threads; every token's argmin is its own, so the record
    is the same as with one thread."""
    rng = np.random.default_rng(8)
    X = rng.normal(0, 1, (1, 3001, 32)).astype(np.float32)
    a = oracle.compress(X, C=24, T=2, iters=3, bits=2, G=32, seed=5, threads=1)
    b = oracle.compress(X, C=24, T=2, iters=3, bits=2, G=32, seed=5, threads=7)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
