"""Pins for the NABLA mask oracle (CPU only).

Each test checks the oracle against something other than itself: closed forms,
brute force over all subsets, a library softmax, or invariants the method fixes.
"""
import itertools
import os

import numpy as np
import pytest
import scipy.special

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pool_identical_tokens_is_exact():
    # bf16-representable values: sums of 64 copies are exact in fp64
    rng = np.random.default_rng(0)
    tok = rng.integers(-255, 256, size=16) / 64.0
    x = np.tile(tok, (64 * 3, 1))
    out = oracle.block_pool(x, 64)
    assert out.shape == (3, 16)
    assert np.array_equal(out, np.tile(tok, (3, 1)))


def test_pool_arithmetic_series_closed_form():
    # tokens r = 0..S-1 with value r in every channel: block i averages to i*n + (n-1)/2
    n, nb = 64, 5
    x = np.repeat(np.arange(n * nb, dtype=np.float64)[:, None], 3, axis=1)
    out = oracle.block_pool(x, n)
    assert np.array_equal(out[:, 0], np.arange(nb) * n + (n - 1) / 2)


def test_pool_permutation_inside_block_invariant():
    rng = np.random.default_rng(1)
    x = rng.integers(-50, 50, size=(128, 8)).astype(np.float64) / 8   # exact sums
    perm = np.concatenate([rng.permutation(64), 64 + rng.permutation(64)])
    assert np.array_equal(oracle.block_pool(x, 64), oracle.block_pool(x[perm], 64))


def test_softmax_matches_scipy_and_normalises():
    rng = np.random.default_rng(2)
    qb, kb = rng.standard_normal((7, 32)), rng.standard_normal((7, 32))
    L = oracle.reduced_map(qb, kb, 0.3)
    P = oracle.row_softmax(L)
    ref = scipy.special.softmax(0.3 * np.einsum("id,jd->ij", qb, kb), axis=1)
    assert np.max(np.abs(P - ref)) < 1e-15
    assert np.max(np.abs(P.sum(axis=1) - 1)) < 1e-14


def _brute_min_cardinality(p, target):
    nb = len(p)
    for size in range(1, nb + 1):
        best = max(sum(p[list(c)]) for c in itertools.combinations(range(nb), size))
        if best >= target:
            return size
    return nb


@pytest.mark.parametrize("seed", range(12))
def test_cdf_select_brute_force_small_rows(seed):
    rng = np.random.default_rng(100 + seed)
    nb = int(rng.integers(2, 10))
    P = rng.dirichlet(np.full(nb, 0.7), size=3)
    thr = float(rng.uniform(0.02, 0.9))
    keep, E = oracle.cdf_select(P, thr)
    for r in range(3):
        p = P[r]
        k_star = _brute_min_cardinality(p, 1 - thr)
        assert keep[r].sum() == k_star
        # the kept set is the k_star largest entries
        top = set(np.argsort(-p, kind="stable")[:k_star])
        assert set(np.nonzero(keep[r])[0]) == top
        # E is the mass strictly before each entry in descending order
        for j in range(nb):
            before = sum(p[i] for i in range(nb) if (p[i], -i) > (p[j], -j))
            assert abs(E[r, j] - before) < 1e-15


def test_cdf_ties_broken_by_ascending_index():
    P = np.array([[0.3, 0.2, 0.3, 0.2]])
    keep, E = oracle.cdf_select(P, 0.5)          # needs mass 0.5: the first 0.3 then the second 0.3
    assert keep.tolist() == [[True, False, True, False]]
    keep, _ = oracle.cdf_select(P, 0.25)         # 0.75 needed: 0.3+0.3+0.2 (index 1 before 3)
    assert keep.tolist() == [[True, True, True, False]]


def _geometric_inputs(nb, perm, D=64):
    """Token-level Q, K whose reduced logits are L[i, j] = -perm_inv(j)/16 for every row i."""
    q = np.zeros((nb * 64, D))
    q[:, 0] = 1.0
    k = np.zeros((nb * 64, D))
    for j in range(nb):
        # key block at position perm[j] carries rank j
        k[perm[j] * 64:(perm[j] + 1) * 64, 0] = -j / 2.0
    return q, k


def _golden_geometric():
    rows = []
    with open(os.path.join(GOLDEN, "geometric_rows.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                nb, thr, k = line.split()
                rows.append((int(nb), float(thr), int(k)))
    return rows


@pytest.mark.parametrize("scale", [1.0 / 8.0, None], ids=["explicit", "default"])
@pytest.mark.parametrize("nb,thr,k_star", _golden_geometric())
def test_geometric_rows_closed_form(nb, thr, k_star, scale):
    # scale None: the default temperature 1/sqrt(D) (D = 64 -> 1/8) must give the same rows
    rng = np.random.default_rng(nb)
    perm = rng.permutation(nb)
    q, k = _geometric_inputs(nb, perm)
    keep, E, P = oracle.nabla_mask(q, k, 64, thr, scale=scale)
    rho = np.exp(-1.0 / 16.0)
    expect_p = rho ** np.arange(nb) * (1 - rho) / (1 - rho ** nb)
    assert np.max(np.abs(P[0, perm] - expect_p)) < 1e-13
    for i in range(nb):
        assert keep[i].sum() == k_star
        assert set(np.nonzero(keep[i])[0]) == set(perm[:k_star])


def _rand_qk(seed, nb=24, D=32):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((nb * 64, D)) + np.repeat(rng.standard_normal((nb, D)) * 2, 64, 0)
    k = rng.standard_normal((nb * 64, D)) + np.repeat(rng.standard_normal((nb, D)) * 2, 64, 0)
    return q, k


@pytest.mark.parametrize("thr", [0.05, 0.2, 0.5, 0.9])
def test_invariants_random(thr):
    q, k = _rand_qk(7)
    keep, E, P = oracle.nabla_mask(q, k, 64, thr)
    band = 1e-6
    for i in range(keep.shape[0]):
        kept, dropped = P[i][keep[i]], P[i][~keep[i]]
        assert len(kept) >= 1
        assert kept.sum() >= (1 - thr) - band                    # covers 1 - thr
        assert kept.sum() - kept.min() < (1 - thr) + band        # smallest such prefix
        if len(dropped):
            assert kept.min() >= dropped.max()                   # it is a top set
    assert np.all(keep[np.arange(len(keep)), np.argmax(P, axis=1)])


def test_monotone_in_thr():
    q, k = _rand_qk(8)
    prev = None
    for thr in [0.0, 0.05, 0.1, 0.2, 0.4, 0.7, 0.95]:
        keep, _, _ = oracle.nabla_mask(q, k, 64, thr)
        if prev is not None:
            assert np.all(prev >= keep)        # larger thr keeps a subset
        prev = keep


def test_thr_zero_keeps_every_block_with_mass():
    q, k = _rand_qk(9, nb=8, D=16)
    keep, E, P = oracle.nabla_mask(q * 0.1, k * 0.1, 64, 0.0)
    assert keep.all()


def test_block_permutation_equivariance():
    q, k = _rand_qk(10)
    nb = q.shape[0] // 64
    rng = np.random.default_rng(11)
    pq, pk = rng.permutation(nb), rng.permutation(nb)
    keep, _, _ = oracle.nabla_mask(q, k, 64, 0.3)
    qp = q.reshape(nb, 64, -1)[pq].reshape(q.shape)
    kp = k.reshape(nb, 64, -1)[pk].reshape(k.shape)
    keep_p, _, _ = oracle.nabla_mask(qp, kp, 64, 0.3)
    assert np.array_equal(keep_p, keep[pq][:, pk])


def test_multi_head_matches_single_head():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, 3, 256, 16))
    k = rng.standard_normal((2, 3, 256, 16))
    keep, E = oracle.nabla_masks(q, k, 64, 0.2)
    for b in range(2):
        for h in range(3):
            kk, ee, _ = oracle.nabla_mask(q[b, h], k[b, h], 64, 0.2)
            assert np.array_equal(kk, keep[b, h]) and np.array_equal(ee, E[b, h])


# ----------------------------------------------------------------------------- Top-k
def test_topk_brute_force_and_count():
    rng = np.random.default_rng(11)
    for _ in range(200):
        nb = int(rng.integers(1, 10))
        P = rng.dirichlet(np.ones(nb), size=3)
        P[0, : nb // 2] = P[0, 0]                     # a tie group
        P /= P.sum(1, keepdims=True)
        for kk in range(0, nb + 2):
            keep = oracle.topk_select(P, kk)
            assert np.all(keep.sum(1) == min(kk, nb))
            for r in range(3):
                if keep[r].any() and (~keep[r]).any():
                    assert P[r][keep[r]].min() >= P[r][~keep[r]].max()
                # among equal values the lower indices are kept first
                for j in range(nb):
                    for j2 in range(j + 1, nb):
                        if P[r, j] == P[r, j2]:
                            assert not (keep[r, j2] and not keep[r, j])


@pytest.mark.parametrize("nb,thr,k_star", _golden_geometric()[:3])
def test_topk_default_temperature_on_geometric_rows(nb, thr, k_star):
    # the default temperature of topk_mask (1/sqrt(D), D = 64) on the geometric rows: the k*
    # largest entries are the blocks of rank 0 .. k*-1, wherever the permutation put them
    perm = np.random.default_rng(nb + 1).permutation(nb)
    q, k = _geometric_inputs(nb, perm)
    keep, P = oracle.topk_mask(q, k, 64, k_star)
    rho = np.exp(-1.0 / 16.0)
    assert np.max(np.abs(P[0, perm] - rho ** np.arange(nb) * (1 - rho) / (1 - rho ** nb))) < 1e-13
    for i in range(nb):
        assert set(np.nonzero(keep[i])[0]) == set(perm[:k_star])


def test_topk_equals_cdf_mask_at_the_cdf_count():
    # CDF keeps a prefix of the same descending order, so each row equals Top-k with k = its kept count
    rng = np.random.default_rng(12)
    q = rng.standard_normal((512, 32))
    k = q + 0.5 * rng.standard_normal((512, 32))
    for thr in (0.05, 0.2, 0.6):
        keep, _, P = oracle.nabla_mask(q, k, 64, thr)
        for i in range(P.shape[0]):
            assert np.array_equal(oracle.topk_select(P[i:i + 1], int(keep[i].sum()))[0], keep[i])
