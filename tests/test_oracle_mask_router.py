"""Pins for the block-mask and Layer Router oracles (CPU only)."""

import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                yield line


# ---------------------------------------------------------------- mask

def test_mask_tiny_golden():
    rows = list(_golden_lines("mask_tiny.txt"))
    ref = np.array([[int(c) for c in r] for r in rows], dtype=np.uint8)
    np.testing.assert_array_equal(oracle.block_mask(8, 1, 2), ref)


def test_mask_nnz_golden():
    for line in _golden_lines("mask_nnz.txt"):
        nb, s, w, nnz = map(int, line.split())
        assert oracle.mask_nnz(nb, s, w) == nnz
        if nb <= 256:
            assert int(oracle.block_mask(nb, s, w).sum()) == nnz


@pytest.mark.parametrize("nb", [1, 2, 7, 33, 300])
@pytest.mark.parametrize("s,w", [(0, 1), (1, 2), (3, 1), (2, 5), (0, 400), (5, 5)])
def test_mask_row_counts_closed_form(nb, s, w):
    m = oracle.block_mask(nb, s, w)
    for i in range(nb):
        assert int(m[i].sum()) == oracle.mask_row_count(i, s, w)
        assert m[i, i] == 1          # the diagonal block is always active
        assert m[i, i + 1:].sum() == 0  # causal


def test_mask_lower_triangle_special_case():
    for nb in (1, 5, 16):
        np.testing.assert_array_equal(oracle.block_mask(nb, 0, nb),
                                      np.tril(np.ones((nb, nb), dtype=np.uint8)))


def test_mask_prefix_property():
    big = oracle.block_mask(40, 2, 3)
    for nb in (1, 9, 27):
        np.testing.assert_array_equal(oracle.block_mask(nb, 2, 3), big[:nb, :nb])


def test_csr_consistency():
    m = oracle.block_mask(50, 1, 4)
    rp, ci = oracle.mask_to_csr(m)
    assert rp[0] == 0 and rp[-1] == m.sum()
    for i in range(50):
        cols = ci[rp[i]:rp[i + 1]]
        assert (np.diff(cols) > 0).all()
        np.testing.assert_array_equal(cols, np.nonzero(m[i])[0])


def test_num_blocks():
    assert oracle.num_blocks(512, 64) == 8
    assert oracle.num_blocks(513, 64) == 9
    assert oracle.num_blocks(1, 128) == 1
    assert oracle.num_blocks(32768, 128) == 256


def test_mask_rejects_bad_params():
    with pytest.raises(ValueError):
        oracle.block_mask(4, 1, 0)
    with pytest.raises(ValueError):
        oracle.block_mask(4, -1, 1)


# ---------------------------------------------------------------- router: pooling

def test_pool_ramp_golden():
    for line in _golden_lines("pool_ramp.txt"):
        S, mean = line.split()
        S = int(S)
        h = np.tile(np.arange(S, dtype=np.float64)[:, None], (1, 3))
        np.testing.assert_array_equal(oracle.pool_mean(h), np.full(3, float(mean)))


def test_pool_positions_set():
    assert list(oracle.pool_positions(5)) == [0, 1, 2, 3, 4]
    p = oracle.pool_positions(512)
    assert len(p) == 200 and p[0] == 0 and p[99] == 99 and p[100] == 412 and p[-1] == 511
    p = oracle.pool_positions(150)   # overlapping ends count once
    assert list(p) == list(range(150))
    with pytest.raises(ValueError):
        oracle.pool_positions(0)


def test_pool_one_hot_membership():
    h = np.zeros((400, 400))
    h[np.arange(400), np.arange(400)] = 1.0   # row p is the unit vector e_p
    pooled = oracle.pool_mean(h)
    inside = set(oracle.pool_positions(400))
    for p in range(400):
        assert pooled[p] == (1.0 / 200 if p in inside else 0.0)


def test_pool_permutation_invariance_on_integers():
    r = np.random.default_rng(1)
    S = 600
    h = r.integers(-50, 50, size=(S, 8)).astype(np.float64)
    pos = oracle.pool_positions(S)
    h2 = h.copy()
    h2[pos] = h[r.permutation(pos)]
    np.testing.assert_array_equal(oracle.pool_mean(h), oracle.pool_mean(h2))


# ---------------------------------------------------------------- router: MLP + threshold

def test_mlp_equals_torch_linear_float64():
    r = np.random.default_rng(2)
    D, H1, L = 32, 16, 5
    x = r.standard_normal(D)
    w1, b1 = r.standard_normal((H1, D)), r.standard_normal(H1)
    w2, b2 = r.standard_normal((L, H1)), r.standard_normal(L)
    l1 = torch.nn.Linear(D, H1, dtype=torch.float64)
    l2 = torch.nn.Linear(H1, L, dtype=torch.float64)
    with torch.no_grad():
        l1.weight.copy_(torch.from_numpy(w1)); l1.bias.copy_(torch.from_numpy(b1))
        l2.weight.copy_(torch.from_numpy(w2)); l2.bias.copy_(torch.from_numpy(b2))
        ref = l2(torch.relu(l1(torch.from_numpy(x)))).numpy()
    np.testing.assert_allclose(oracle.router_mlp(x, w1, b1, w2, b2), ref, rtol=0, atol=1e-12)


def test_mlp_hand_sized():
    # identity first layer, ReLU clips the negative entry, second layer sums
    x = np.array([2.0, -3.0, 0.5])
    z = oracle.router_mlp(x, np.eye(3), np.zeros(3), np.array([[1.0, 1.0, 1.0], [-1.0, 0.0, 0.0]]),
                          np.array([0.0, 1.0]))
    np.testing.assert_array_equal(z, np.array([2.5, -1.0]))


def test_threshold_matches_sigmoid_half():
    # sigmoid(z) >= 1/2 iff z >= 0.  A computed sigmoid rounds to exactly 0.5
    # for |z| below ~1e-16, so the library check uses |z| >= 1e-12 (and 0).
    z = np.array([-1e-12, -1e-8, -3.0, 0.0, 1e-12, 2.0, -0.0, 40.0, -40.0])
    expect = (scipy.special.expit(z) >= 0.5).astype(np.uint8)
    np.testing.assert_array_equal(oracle.threshold_route(z), expect)
    assert oracle.threshold_route(np.array([-1e-300]))[0] == 0
    assert oracle.threshold_route(np.array([0.0]))[0] == 1  # exact tie -> FA


def test_zero_router_ties_to_fa():
    route, z = oracle.route_requests(np.ones((300, 4)), [0, 300], np.zeros((3, 4)), np.zeros(3),
                                     np.zeros((2, 3)), np.zeros(2))
    np.testing.assert_array_equal(route, [[1, 1]])
    np.testing.assert_array_equal(z, [[0.0, 0.0]])


def test_route_requests_packed_matches_single_and_is_deterministic():
    r = np.random.default_rng(4)
    lens = [250, 120, 512]
    cu = np.cumsum([0] + lens)
    D, H1, L = 16, 8, 6
    h = r.standard_normal((cu[-1], D))
    w1, b1 = r.standard_normal((H1, D)), r.standard_normal(H1)
    w2, b2 = r.standard_normal((L, H1)), r.standard_normal(L)
    route, z = oracle.route_requests(h, cu, w1, b1, w2, b2)
    route2, z2 = oracle.route_requests(h, cu, w1, b1, w2, b2)
    np.testing.assert_array_equal(z, z2)
    for i in range(3):
        zi = oracle.router_mlp(oracle.pool_mean(h[cu[i]:cu[i + 1]]), w1, b1, w2, b2)
        np.testing.assert_array_equal(z[i], zi)
        np.testing.assert_array_equal(route[i], (zi >= 0).astype(np.uint8))
