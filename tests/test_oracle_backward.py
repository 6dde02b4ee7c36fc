"""Pins for the gradient oracle of block-sparse attention (CPU only).

Each pin is independent of the formulas the oracle uses: central finite differences
of the (separately pinned) forward oracle, torch autograd of dense attention in
float64, a per-element loop evaluation of the softmax Jacobian, and exact identities
that follow from the definition (shift invariance of the keys, rows of P summing to
one, padded and empty rows carrying no gradient).
"""
import math

import numpy as np
import torch

import oracle


def _problem(seed, S, D, n, s_valid, p_keep=0.5, empty_row=None):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((S, D)) for _ in range(4))
    nb = S // n
    bm = rng.random((nb, nb)) < p_keep
    bm[np.arange(nb), np.arange(nb)] = True
    if empty_row is not None:
        bm[empty_row] = False
    return q, k, v, do, bm


def _loss(q, k, v, do, bm, n, s_valid, scale):
    O, _ = oracle.block_sparse_attention(q, k, v, bm, n, s_valid, scale=scale)
    return float(np.sum(O * do))


def test_central_finite_differences():
    # L = sum(O * dO); dL/dX must equal the oracle's dX for X in (q, k, v), every element
    S, D, n, Sv, scale = 12, 3, 4, 10, 0.8
    q, k, v, do, bm = _problem(0, S, D, n, Sv, empty_row=1)
    dq, dk, dv = oracle.block_sparse_attention_bwd(q, k, v, do, bm, n, Sv, scale=scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            lp = _loss(**{**args, name: xp}, do=do, bm=bm, n=n, s_valid=Sv, scale=scale)
            lm = _loss(**{**args, name: xm}, do=do, bm=bm, n=n, s_valid=Sv, scale=scale)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[idx]) < 1e-7, (name, idx, fd, g[idx])


def test_full_mask_equals_autograd_of_dense_sdpa():
    S, D = 256, 32
    q, k, v, do, _ = _problem(1, S, D, 64, S)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None])[0]
    out.backward(torch.from_numpy(do))
    dq, dk, dv = oracle.block_sparse_attention_bwd(q, k, v, do, np.ones((4, 4), bool), 64, S)
    for ours, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(ours - ref.numpy())) < 1e-12


def test_element_loops_of_the_softmax_jacobian():
    # dS_pq = sum_r (dO_p . V_r) dP_r/ds_pq with dP_r/ds_pq = P_r (1[r = q] - P_q), by loops
    S, D, n, Sv, scale = 16, 3, 4, 14, 0.6
    q, k, v, do, bm = _problem(2, S, D, n, Sv)
    dq, dk, dv = oracle.block_sparse_attention_bwd(q, k, v, do, bm, n, Sv, scale=scale)
    ref_dq = np.zeros((S, D))
    ref_dk = np.zeros((S, D))
    ref_dv = np.zeros((S, D))
    for p in range(Sv):
        allowed = [c for c in range(Sv) if bm[p // n, c // n]]
        w = [math.exp(scale * sum(q[p, d] * k[c, d] for d in range(D))) for c in allowed]
        z = sum(w)
        P = [wi / z for wi in w]
        g = [sum(do[p, d] * v[c, d] for d in range(D)) for c in allowed]   # dL/dP_pc
        for a, ca in enumerate(allowed):
            ds = sum(g[r] * P[r] * ((1.0 if r == a else 0.0) - P[a]) for r in range(len(allowed)))
            for d in range(D):
                ref_dq[p, d] += scale * ds * k[ca, d]
                ref_dk[ca, d] += scale * ds * q[p, d]
                ref_dv[ca, d] += P[a] * do[p, d]
    assert np.max(np.abs(dq - ref_dq)) < 1e-12
    assert np.max(np.abs(dk - ref_dk)) < 1e-12
    assert np.max(np.abs(dv - ref_dv)) < 1e-12


def test_identities_padding_and_empty_rows():
    S, D, n, Sv = 256, 16, 64, 230
    q, k, v, do, bm = _problem(3, S, D, n, Sv, p_keep=0.4, empty_row=2)
    dq, dk, dv = oracle.block_sparse_attention_bwd(q, k, v, do, bm, n, Sv)
    live = np.array([p < Sv and bm[p // n].any() for p in range(S)])
    # adding one vector to every key shifts a row's logits by a constant: O unchanged
    assert np.max(np.abs(dk.sum(axis=0))) < 1e-12
    # every live row of P sums to one
    assert np.max(np.abs(dv.sum(axis=0) - do[live].sum(axis=0))) < 1e-12
    # padded queries, queries with no allowed key, padded keys carry no gradient
    assert np.all(dq[~live] == 0)
    assert np.all(dk[Sv:] == 0) and np.all(dv[Sv:] == 0)


def test_block_selection_matches_the_full_computation():
    S, D, n, Sv = 512, 8, 64, 500
    q, k, v, do, bm = _problem(4, S, D, n, Sv, p_keep=0.3)
    full = oracle.block_sparse_attention_bwd(q, k, v, do, bm, n, Sv)
    part = oracle.block_sparse_attention_bwd(q, k, v, do, bm, n, Sv, q_blocks=[1, 7], kv_blocks=[0, 5])
    for i in (1, 7):
        assert np.array_equal(part[0][i * n:(i + 1) * n], full[0][i * n:(i + 1) * n])
    for j in (0, 5):
        sl = slice(j * n, (j + 1) * n)
        assert np.max(np.abs(part[1][sl] - full[1][sl])) < 1e-12
        assert np.max(np.abs(part[2][sl] - full[2][sl])) < 1e-12
    assert np.isnan(part[0][0]).all() and np.isnan(part[1][n]).all()
