"""Pins for the block-sparse attention oracle and the CSR helpers (CPU only)."""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle


def _qkv(seed, S=256, D=32):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((S, D)), rng.standard_normal((S, D)), rng.standard_normal((S, D)))


def test_full_mask_equals_dense_sdpa():
    q, k, v = _qkv(0)
    O, lse = oracle.block_sparse_attention(q, k, v, np.ones((4, 4), bool), 64, 256)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0].numpy()
    assert np.max(np.abs(O - ref)) < 1e-12
    s = (q @ k.T) / math.sqrt(32)
    assert np.max(np.abs(lse - scipy.special.logsumexp(s, axis=1))) < 1e-12


def test_brute_force_loops_with_mask_and_padding():
    S, D, n, Sv = 32, 4, 8, 29
    q, k, v = _qkv(1, S, D)
    rng = np.random.default_rng(2)
    bm = rng.random((4, 4)) < 0.5
    bm[2] = False                                 # a query block with no kept key block
    O, lse = oracle.block_sparse_attention(q, k, v, bm, n, Sv, scale=0.7)
    for p in range(S):
        allowed = [c for c in range(Sv) if bm[p // n, c // n]]
        if p >= Sv or not allowed:
            assert np.all(O[p] == 0) and lse[p] == -np.inf
            continue
        w = [math.exp(0.7 * sum(q[p, d] * k[c, d] for d in range(D))) for c in allowed]
        z = sum(w)
        for d in range(D):
            assert abs(O[p, d] - sum(wi * v[c, d] for wi, c in zip(w, allowed)) / z) < 1e-12
        assert abs(lse[p] - math.log(z)) < 1e-12


def test_rows_are_convex_combinations_of_allowed_values():
    q, k, v = _qkv(3)
    bm = np.random.default_rng(4).random((4, 4)) < 0.6
    bm[np.arange(4), np.arange(4)] = True
    O, _ = oracle.block_sparse_attention(q * 3, k * 3, v, bm, 64, 256)
    for i in range(4):
        cols = np.concatenate([np.arange(j * 64, j * 64 + 64) for j in np.nonzero(bm[i])[0]])
        lo, hi = v[cols].min(0), v[cols].max(0)
        assert np.all(O[i * 64:(i + 1) * 64] >= lo - 1e-12)
        assert np.all(O[i * 64:(i + 1) * 64] <= hi + 1e-12)


def test_constant_values_reproduced():
    q, k, _ = _qkv(5)
    v = np.tile(np.linspace(-2, 2, 32), (256, 1))
    bm = np.eye(4, dtype=bool) | np.eye(4, k=1, dtype=bool)
    O, _ = oracle.block_sparse_attention(q, k, v, bm, 64, 256)
    assert np.max(np.abs(O - v)) < 1e-12


def test_key_shift_invariance():
    q, k, v = _qkv(6)
    bm = np.random.default_rng(7).random((4, 4)) < 0.5
    bm[:, 0] = True
    c = np.random.default_rng(8).standard_normal(32)
    O1, _ = oracle.block_sparse_attention(q, k, v, bm, 64, 256)
    O2, _ = oracle.block_sparse_attention(q, k + c, v, bm, 64, 256)
    assert np.max(np.abs(O1 - O2)) < 1e-10


def test_dropping_a_block_changes_output():
    q, k, v = _qkv(9)
    full = np.ones((4, 4), bool)
    part = full.copy()
    part[1, 3] = False
    O1, _ = oracle.block_sparse_attention(q, k, v, full, 64, 256)
    O2, _ = oracle.block_sparse_attention(q, k, v, part, 64, 256)
    assert np.array_equal(O1[:64], O2[:64]) and not np.allclose(O1[64:128], O2[64:128])


def test_sampled_blocks_equal_full_run():
    q, k, v = _qkv(10)
    bm = np.random.default_rng(11).random((4, 4)) < 0.5
    Of, lf = oracle.block_sparse_attention(q, k, v, bm, 64, 250)
    Os, ls = oracle.block_sparse_attention(q, k, v, bm, 64, 250, q_blocks=[1, 3])
    assert np.array_equal(Of[64:128], Os[64:128]) and np.array_equal(Of[192:], Os[192:])
    assert np.isnan(Os[0]).all()


def test_mask_or_truth_table():
    a = np.array([0, 0, 1, 1], bool)
    b = np.array([0, 1, 0, 1], bool)
    assert oracle.mask_or(a, b).tolist() == [False, True, True, True]


def test_csr_round_trip():
    rng = np.random.default_rng(12)
    m = rng.random((37, 23)) < 0.3
    m[5] = False
    rp, ci = oracle.mask_to_csr(m)
    assert rp[0] == 0 and rp[-1] == m.sum()
    assert np.array_equal(np.diff(rp), m.sum(1))
    back = np.zeros_like(m)
    for r in range(37):
        cols = ci[rp[r]:rp[r + 1]]
        assert np.all(np.diff(cols) > 0)
        back[r, cols] = True
    assert np.array_equal(back, m)


def test_longest_first_order_worked_example():
    # row counts 2, 0, 3, 2, 3, 1 -> by count descending, equal counts by index:
    # rows 2, 4 (3 kept), 0, 3 (2 kept), 5 (1 kept), 1 (0 kept); worked by hand
    m = np.zeros((6, 4), bool)
    m[0, [0, 3]] = True
    m[2, [0, 1, 2]] = True
    m[3, [1, 2]] = True
    m[4, [1, 2, 3]] = True
    m[5, [3]] = True
    assert oracle.longest_first_order(m).tolist() == [2, 4, 0, 3, 5, 1]


def test_longest_first_order_invariants():
    rng = np.random.default_rng(3)
    m = rng.random((300, 9)) < 0.4           # few distinct counts: many ties
    order = oracle.longest_first_order(m)
    counts = m.sum(1)
    assert sorted(order.tolist()) == list(range(300))          # a permutation
    c = counts[order]
    assert np.all(np.diff(c) <= 0)                              # largest first
    same = np.diff(c) == 0
    assert np.all(np.diff(order)[same] > 0)                     # ties by index
