"""Pins for the content-aware block-mask oracle (CPU only): the pooled logits
against brute force over token pairs, the softmax rows, the Top-tau rule's
limits (tau = 0: sink + diagonal only; tau = 1: every causal block, so SA
equals FA), tie order, the budget cap, nesting in tau, a planted block, and
greedy minimality."""

import numpy as np
import pytest
import scipy.special

import oracle

rng = np.random.default_rng(20261203)


def _qk(S, hq, hkv, d, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((S, hq, d)), r.standard_normal((S, hkv, d))


@pytest.mark.parametrize("S,B", [(10, 4), (16, 4), (7, 8), (1, 4)])
def test_pooled_logits_brute_force(S, B):
    """z[h, i, j] is the mean over the block pair of the token-level scaled
    products (linearity of the mean); a partial last block averages its own
    rows; KV head of query head h is h // (Hq/Hkv)."""
    hq, hkv, d = 4, 2, 6
    q, k = _qk(S, hq, hkv, d, 1 + S)
    scale = 0.37
    z = oracle.coarse_logits(q, k, B, scale)
    nb = (S + B - 1) // B
    assert z.shape == (hq, nb, nb)
    for h in range(hq):
        g = h // (hq // hkv)
        for i in range(nb):
            ti = range(i * B, min(S, (i + 1) * B))
            for j in range(nb):
                if j > i:
                    assert z[h, i, j] == -np.inf
                    continue
                tj = range(j * B, min(S, (j + 1) * B))
                brute = np.mean([scale * sum(q[t, h, c] * k[u, g, c] for c in range(d)) for t in ti for u in tj])
                assert abs(z[h, i, j] - brute) < 1e-12


def test_default_scale_is_inverse_sqrt_d():
    q, k = _qk(8, 2, 1, 9, 3)
    np.testing.assert_allclose(oracle.coarse_logits(q, k, 4), oracle.coarse_logits(q, k, 4, 1.0 / 3.0))


def test_probs_rows():
    """Causal rows of P sum to 1, zero above the diagonal, and equal the mean
    over heads of scipy's softmax of each head's causal logits."""
    q, k = _qk(40, 4, 2, 8, 5)
    B = 8
    P = oracle.block_probs(q, k, B)
    z = oracle.coarse_logits(q, k, B)
    nb = P.shape[0]
    for i in range(nb):
        assert abs(P[i, :i + 1].sum() - 1.0) < 1e-12
        assert np.all(P[i, i + 1:] == 0.0)
        ref = np.mean([scipy.special.softmax(z[h, i, :i + 1]) for h in range(z.shape[0])], axis=0)
        np.testing.assert_allclose(P[i, :i + 1], ref, rtol=1e-12, atol=1e-15)


def test_tau_zero_keeps_sink_and_diagonal_only():
    q, k = _qk(64, 2, 2, 8, 7)
    for s in (0, 1, 3):
        m, _ = oracle.dynamic_block_mask(q, k, 8, 0.0, s)
        nb = m.shape[0]
        ref = np.zeros_like(m)
        for i in range(nb):
            for j in range(i + 1):
                ref[i, j] = 1 if (j < s or j == i) else 0
        np.testing.assert_array_equal(m, ref)


def test_tau_one_selects_every_causal_block_and_sa_equals_fa():
    """With tau = 1 and no cap every causal block is kept (P > 0 everywhere,
    so the mass stays below 1 until the last block); SA with that mask is FA."""
    S, hq, hkv, d, B = 48, 4, 2, 8, 8
    q, k = _qk(S, hq, hkv, d, 9)
    v = np.random.default_rng(10).standard_normal((S, hkv, d))
    m, _ = oracle.dynamic_block_mask(q, k, B, 1.0, 1)
    nb = m.shape[0]
    np.testing.assert_array_equal(m, np.tril(np.ones((nb, nb), dtype=np.uint8)))
    sa = oracle.attention_prefill(q, k, v, False, m, B)
    fa = oracle.attention_prefill(q, k, v, True)
    np.testing.assert_allclose(sa, fa, rtol=1e-12, atol=1e-12)


def test_ties_take_smaller_block_first():
    """Zero queries give equal logits, hence a uniform row: Top-tau then keeps
    the lowest-indexed candidates, as many as the mass needs."""
    S, B = 64, 8
    q = np.zeros((S, 2, 4))
    k = rng.standard_normal((S, 1, 4))
    P = oracle.block_probs(q, k, B)
    m = oracle.select_blocks(P, 0.5, 0)
    nb = m.shape[0]
    for i in range(nb):
        n = i + 1
        # the diagonal is mandatory (mass 1/n), then candidates 0, 1, ... until mass >= 0.5
        need = 0
        mass = 1.0 / n
        while mass < 0.5 - 1e-12 and need < n - 1:
            need += 1
            mass += 1.0 / n
        expect = set(range(need)) | {i}
        assert set(np.nonzero(m[i])[0].tolist()) == expect, (i, need)


def test_budget_cap():
    q, k = _qk(128, 2, 1, 8, 11)
    for cap in (1, 3, 5):
        m, _ = oracle.dynamic_block_mask(q, k, 8, 1.0, 1, max_blocks=cap)
        for i in range(m.shape[0]):
            mandatory = len({0, i})
            assert m[i].sum() == max(min(i + 1, cap), mandatory)


def test_nested_in_tau():
    q, k = _qk(96, 4, 2, 8, 13)
    P = oracle.block_probs(q, k, 8)
    prev = None
    for tau in (0.0, 0.2, 0.5, 0.8, 0.95, 1.0):
        m = oracle.select_blocks(P, tau, 1)
        if prev is not None:
            assert np.all(m >= prev)
        prev = m


def test_planted_block_is_chosen():
    """Every query shares a direction u and key block 2 is aligned with it:
    that block carries most of every later row's mass and is picked first."""
    S, hq, hkv, d, B = 96, 2, 1, 16, 8
    r = np.random.default_rng(17)
    u = r.standard_normal(d)
    u /= np.linalg.norm(u)
    q = r.standard_normal((S, hq, d)) * 0.3 + 3.0 * u
    k = r.standard_normal((S, hkv, d)) * 0.3
    k[2 * B:3 * B] += 6.0 * u
    m, P = oracle.dynamic_block_mask(q, k, B, 0.3, 0)
    for i in range(3, m.shape[0]):
        assert m[i, 2] == 1
        assert int(np.argmax(P[i, :i])) == 2
        assert m[i, :i].sum() == 1  # block 2 alone brings the row past tau


def test_greedy_prefix_and_minimality():
    q, k = _qk(200, 4, 2, 8, 19)
    B, tau, s = 8, 0.6, 2
    m, P = oracle.dynamic_block_mask(q, k, B, tau, s)
    for i in range(m.shape[0]):
        mand = [j for j in range(i + 1) if j < s or j == i]
        cand = sorted([j for j in range(i + 1) if j not in mand], key=lambda j: (-P[i, j], j))
        chosen = [j for j in cand if m[i, j]]
        assert chosen == cand[:len(chosen)]  # a prefix of the sorted order
        base = P[i, mand].sum()
        if chosen:
            assert base + P[i, chosen[:-1]].sum() < tau  # the last one was still needed
        full = base + P[i, chosen].sum()
        assert full >= tau or len(chosen) == len(cand)


def test_block_probs_rows_matches_loops():
    q, k = _qk(70, 4, 2, 8, 23)
    P = oracle.block_probs(q, k, 8)
    rows = [0, 3, 8]
    np.testing.assert_allclose(oracle.block_probs_rows(q, k, 8, rows), P[rows], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(oracle.block_probs_rows(q, k, 8, rows, 0.21),
                               oracle.block_probs(q, k, 8, 0.21)[rows], rtol=1e-12, atol=1e-15)
