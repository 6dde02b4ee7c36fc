"""Property tests of the oracle over random small shapes and thresholds (hypothesis).

Each property is one that the pages or the mathematics fix, checked on many random
inputs instead of a few fixed ones:
  * CDF selection (NABLA review, "What carries the argument" and "Core claim"): the kept
    set of a row is a prefix of its descending order, covers mass >= 1 - thr, is the
    smallest such prefix, and grows as thr falls;
  * Top-k (Appendix C's comparison): exactly min(k, nb) entries per row, none smaller
    than a dropped one;
  * kv lists: the CSR of a mask lists exactly its kept blocks, ascending, and the
    longest-first order is a permutation sorted by count (ties by index);
  * attention (FlashAttention abstract, online softmax statement): each output row is a
    convex combination of the allowed V rows, a full mask gives dense attention, the
    result does not depend on the order of the key blocks, and lse is the log of the sum
    of exp over the allowed keys.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def distributions(draw):
    rows = draw(st.integers(1, 6))
    nb = draw(st.integers(1, 40))
    seed = draw(st.integers(0, 2**31 - 1))
    spread = draw(st.sampled_from([0.1, 1.0, 4.0, 12.0]))
    rng = np.random.default_rng(seed)
    L = rng.normal(0.0, spread, (rows, nb))
    if draw(st.booleans()):        # ties: some entries repeated exactly
        L[:, nb // 2:] = L[:, :nb - nb // 2]
    return oracle.row_softmax(L)


thresholds = st.floats(min_value=0.0, max_value=0.999, allow_nan=False)


@SETTINGS
@given(distributions(), thresholds)
def test_cdf_select_is_the_smallest_descending_prefix(P, thr):
    keep, E = oracle.cdf_select(P, thr)
    for p, k, e in zip(P, keep, E):
        order = sorted(range(len(p)), key=lambda j: (-p[j], j))
        flags = [bool(k[j]) for j in order]
        n = sum(flags)
        assert flags == [True] * n + [False] * (len(p) - n)          # a prefix of the order
        mass = float(np.sum(p[order[:n]]))
        assert mass >= (1.0 - thr) - 1e-12                             # covers 1 - thr
        if n > 1:                                                      # one entry fewer does not
            assert float(np.sum(p[order[:n - 1]])) < (1.0 - thr) + 1e-12
        # E is the mass strictly before each entry in that order
        run = 0.0
        for j in order:
            assert abs(e[j] - run) <= 1e-12
            run += p[j]


@SETTINGS
@given(distributions(), thresholds, thresholds)
def test_cdf_select_grows_as_thr_falls(P, t1, t2):
    lo, hi = min(t1, t2), max(t1, t2)
    keep_lo, _ = oracle.cdf_select(P, lo)
    keep_hi, _ = oracle.cdf_select(P, hi)
    assert np.all(keep_lo | ~keep_hi)       # kept at the larger thr => kept at the smaller


@SETTINGS
@given(distributions(), st.integers(0, 50))
def test_topk_keeps_the_k_largest(P, k):
    keep = oracle.topk_select(P, k)
    nb = P.shape[1]
    assert np.all(keep.sum(axis=1) == min(k, nb))
    for p, kr in zip(P, keep):
        if kr.any() and (~kr).any():
            assert p[kr].min() >= p[~kr].max()


@SETTINGS
@given(st.integers(1, 12), st.integers(1, 30), st.integers(0, 2**31 - 1), st.floats(0.0, 1.0))
def test_csr_and_longest_first_order(R, nb, seed, density):
    mask = np.random.default_rng(seed).random((R, nb)) < density
    row_ptr, col_idx = oracle.mask_to_csr(mask)
    assert row_ptr[0] == 0 and len(row_ptr) == R + 1
    back = np.zeros_like(mask)
    for r in range(R):
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        assert np.all(np.diff(cols) > 0)
        back[r, cols] = True
    assert np.array_equal(back, mask)
    order = oracle.longest_first_order(mask)
    assert sorted(order.tolist()) == list(range(R))
    counts = mask.sum(axis=1)
    keys = [(-int(counts[r]), int(r)) for r in order]
    assert keys == sorted(keys)


@st.composite
def attention_cases(draw):
    n = draw(st.sampled_from([1, 2, 4]))
    nb = draw(st.integers(1, 5))
    D = draw(st.sampled_from([1, 3, 8]))
    S = n * nb
    s_valid = draw(st.integers(1, S))
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    q, k, v = (rng.normal(0.0, draw(st.sampled_from([0.5, 2.0])), (S, D)) for _ in range(3))
    mask = rng.random((nb, nb)) < draw(st.floats(0.0, 1.0))
    return q, k, v, mask, n, s_valid


@SETTINGS
@given(attention_cases())
def test_attention_rows_are_convex_combinations(case):
    q, k, v, mask, n, s_valid = case
    O, lse = oracle.block_sparse_attention(q, k, v, mask, n, s_valid)
    scale = 1.0 / np.sqrt(q.shape[1])
    for p in range(q.shape[0]):
        allowed = [j for j in range(s_valid) if mask[p // n, j // n]]
        if p >= s_valid or not allowed:
            assert np.all(O[p] == 0) and lse[p] == -np.inf
            continue
        Va = v[allowed]
        assert np.all(O[p] >= Va.min(axis=0) - 1e-12) and np.all(O[p] <= Va.max(axis=0) + 1e-12)
        logits = scale * (k[allowed] @ q[p])
        m = logits.max()
        assert abs(lse[p] - (m + np.log(np.sum(np.exp(logits - m))))) <= 1e-12 * max(1.0, abs(lse[p]))


@SETTINGS
@given(attention_cases())
def test_full_mask_is_dense_and_block_order_is_irrelevant(case):
    q, k, v, mask, n, s_valid = case
    nb = mask.shape[0]
    full = np.ones_like(mask)
    O, _ = oracle.block_sparse_attention(q, k, v, full, n, s_valid)
    scale = 1.0 / np.sqrt(q.shape[1])
    W = np.exp(scale * q[:s_valid] @ k[:s_valid].T)
    dense = (W / W.sum(axis=1, keepdims=True)) @ v[:s_valid]
    assert np.allclose(O[:s_valid], dense, rtol=1e-10, atol=1e-12)
    # permuting whole key blocks (K, V rows and the mask columns alike) changes nothing,
    # as long as the padded tail stays last
    if s_valid == q.shape[0] and nb > 1:
        perm = np.random.default_rng(nb).permutation(nb)
        rows = np.concatenate([np.arange(j * n, (j + 1) * n) for j in perm])
        O1, L1 = oracle.block_sparse_attention(q, k, v, mask, n, s_valid)
        O2, L2 = oracle.block_sparse_attention(q, k[rows], v[rows], mask[:, perm], n, s_valid)
        assert np.allclose(O1, O2, rtol=1e-10, atol=1e-12)
        assert np.allclose(L1, L2, rtol=1e-12, atol=1e-12, equal_nan=False)
