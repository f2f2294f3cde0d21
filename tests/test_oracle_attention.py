"""Pins for the float64 attention oracle (CPU only).

Each test ties the oracle to something other than itself: hand-worked values
(tests/golden), brute force with math.exp on tiny inputs, torch's
scaled_dot_product_attention in float64 (a library routine), closed forms and
invariants of the masked-softmax definition.  The last tests plant mistakes
in the oracle and check that a pin catches each one.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def rand_qkv(r, S, hq, hkv, d):
    return (r.standard_normal((S, hq, d)), r.standard_normal((S, hkv, d)),
            r.standard_normal((S, hkv, d)))


def sdpa_causal(q, k, v):
    """torch SDPA, float64, causal, KV heads repeated per group."""
    S, hq, d = q.shape
    group = hq // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).repeat_interleave(group, dim=1).permute(1, 0, 2)
    vt = torch.from_numpy(v).repeat_interleave(group, dim=1).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    return o.permute(1, 0, 2).numpy()


def sa_key_set(p, B, s, w):
    """Key positions an SA query at position p may read, enumerated from the
    pattern description (sink tokens, then the window blocks), not from the
    block-mask formula."""
    keys = set()
    for t in range(0, min(s * B, p + 1)):           # sink blocks
        keys.add(t)
    first_win_block = max(0, p // B - (w - 1))      # w blocks ending at p's block
    for t in range(first_win_block * B, p + 1):     # window, causal
        keys.add(t)
    return sorted(keys)


# ---------------------------------------------------------------- golden

def test_golden_three_tokens():
    g = json.load(open(os.path.join(GOLDEN, "attention_3tok.json")))
    q = np.array([[0.0, 0.0], [math.sqrt(2) * math.log(3), 0.0], [0.0, math.sqrt(2) * math.log(2)]])
    k = np.array(g["k"])
    v = np.array(g["v"])
    q, k, v = q[:, None, :], k[:, None, :], v[:, None, :]
    fa = oracle.attention_prefill(q, k, v, True)[:, 0, :]
    np.testing.assert_allclose(fa, np.array(g["fa"]), rtol=0, atol=1e-12)
    m = oracle.block_mask(3, 0, 1)
    sa = oracle.attention_prefill(q, k, v, False, m, 1)[:, 0, :]
    np.testing.assert_allclose(sa, np.array(g["sa_b1_s0_w1"]), rtol=0, atol=1e-12)
    m = oracle.block_mask(3, 1, 1)
    sa = oracle.attention_prefill(q, k, v, False, m, 1)[:, 0, :]
    np.testing.assert_allclose(sa, np.array(g["sa_b1_s1_w1"]), rtol=0, atol=1e-12)
    # decode at N = 3 is prefill row 2
    kc, vc = k.transpose(1, 0, 2)[None], v.transpose(1, 0, 2)[None]
    dec = oracle.attention_decode(q[2:3], kc, vc, [3], True)[0, 0]
    np.testing.assert_allclose(dec, np.array(g["fa"][2]), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- brute force

def brute_force(q, k, v, fa, B, s, w, scale):
    """Triple loop with math.exp over an explicitly enumerated key set."""
    S, hq, d = q.shape
    group = hq // k.shape[1]
    out = np.zeros_like(q)
    for h in range(hq):
        g = h // group
        for p in range(S):
            keys = list(range(p + 1)) if fa else sa_key_set(p, B, s, w)
            sc = [scale * sum(q[p, h, i] * k[t, g, i] for i in range(d)) for t in keys]
            mx = max(sc)
            wts = [math.exp(x - mx) for x in sc]
            tot = sum(wts)
            for i in range(d):
                out[p, h, i] = sum(wt * v[t, g, i] for wt, t in zip(wts, keys)) / tot
    return out


@pytest.mark.parametrize("S,hq,hkv,d,B,s,w", [
    (9, 2, 1, 4, 2, 1, 2), (7, 4, 2, 3, 3, 0, 1), (9, 3, 3, 2, 2, 2, 1), (8, 2, 2, 4, 1, 1, 3)])
def test_brute_force_tiny(S, hq, hkv, d, B, s, w):
    q, k, v = rand_qkv(rng(S * 10 + d), S, hq, hkv, d)
    scale = 1.0 / math.sqrt(d)
    nb = oracle.num_blocks(S, B)
    m = oracle.block_mask(nb, s, w)
    for fa in (True, False):
        ref = brute_force(q, k, v, fa, B, s, w, scale)
        got = oracle.attention_prefill(q, k, v, fa, m, B)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("S,hq,hkv,d", [(64, 4, 2, 16), (37, 8, 8, 8), (130, 4, 1, 32)])
def test_fa_equals_torch_sdpa_float64(S, hq, hkv, d):
    q, k, v = rand_qkv(rng(S + hq), S, hq, hkv, d)
    got = oracle.attention_prefill(q, k, v, True)
    np.testing.assert_allclose(got, sdpa_causal(q, k, v), rtol=0, atol=1e-12)


@pytest.mark.parametrize("S,B,s,w", [(200, 16, 1, 3), (129, 32, 2, 2), (300, 64, 0, 1), (96, 8, 3, 4)])
def test_sa_rows_equal_sdpa_on_gathered_keys(S, B, s, w):
    hq, hkv, d = 4, 2, 8
    q, k, v = rand_qkv(rng(S + B), S, hq, hkv, d)
    m = oracle.block_mask(oracle.num_blocks(S, B), s, w)
    got = oracle.attention_prefill(q, k, v, False, m, B)
    for p in [0, 1, B - 1, B, S // 2, S - 1]:
        keys = sa_key_set(p, B, s, w)
        for h in range(hq):
            g = h // (hq // hkv)
            qt = torch.from_numpy(q[p, h][None, None, :])
            kt = torch.from_numpy(k[keys, g][None])
            vt = torch.from_numpy(v[keys, g][None])
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0].numpy()
            np.testing.assert_allclose(got[p, h], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariants

def test_probability_rows():
    S, B, s, w, d = 150, 16, 1, 3, 8
    r = rng(3)
    q, k = r.standard_normal((S, d)), r.standard_normal((S, d))
    m = oracle.block_mask(oracle.num_blocks(S, B), s, w)
    rows = np.arange(S)
    for fa in (True, False):
        p = oracle.attention_probs(q, k, rows, fa, m, B, 1 / math.sqrt(d))
        ok = oracle.allowed_matrix(rows, S, fa, m, B)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert (p >= 0).all()
        assert (p[~ok] == 0).all()
        assert (p[ok] > 0).all()


def test_sa_all_ones_mask_equals_fa():
    S, hq, hkv, d, B = 100, 4, 2, 8, 16
    q, k, v = rand_qkv(rng(5), S, hq, hkv, d)
    nb = oracle.num_blocks(S, B)
    fa = oracle.attention_prefill(q, k, v, True)
    for s, w in [(0, nb), (nb, 1), (2, nb + 5)]:
        sa = oracle.attention_prefill(q, k, v, False, oracle.block_mask(nb, s, w), B)
        np.testing.assert_array_equal(sa, fa)


def test_sa_equals_fa_when_window_covers_sequence():
    S, B, w = 60, 16, 4  # S <= w * B
    q, k, v = rand_qkv(rng(6), S, 2, 1, 8)
    m = oracle.block_mask(oracle.num_blocks(S, B), 1, w)
    np.testing.assert_array_equal(oracle.attention_prefill(q, k, v, False, m, B),
                                  oracle.attention_prefill(q, k, v, True))


@pytest.mark.parametrize("fa", [True, False])
def test_causality_perturbation(fa):
    S, B = 80, 16
    q, k, v = rand_qkv(rng(7), S, 4, 2, 8)
    m = oracle.block_mask(oracle.num_blocks(S, B), 1, 2)
    base = oracle.attention_prefill(q, k, v, fa, m, B)
    p = 41
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[p + 1:] += 5.0
    k2[p + 1:] *= -3.0
    v2[p + 1:] += 7.0
    pert = oracle.attention_prefill(q2, k2, v2, fa, m, B)
    np.testing.assert_array_equal(pert[:p + 1], base[:p + 1])
    assert not np.array_equal(pert[p + 1:], base[p + 1:])


def test_row_zero_is_v0():
    q, k, v = rand_qkv(rng(8), 10, 4, 2, 8)
    o = oracle.attention_prefill(q, k, v, True)
    for h in range(4):
        np.testing.assert_array_equal(o[0, h], v[0, h // 2])


def test_identical_keys_give_mean_of_allowed_values():
    S, B, s, w, d = 70, 8, 1, 2, 4
    r = rng(9)
    q = r.standard_normal((S, 2, d))
    k = np.tile(r.standard_normal((1, 1, d)), (S, 1, 1))
    v = r.standard_normal((S, 1, d))
    m = oracle.block_mask(oracle.num_blocks(S, B), s, w)
    for fa in (True, False):
        o = oracle.attention_prefill(q, k, v, fa, m, B)
        for p in range(S):
            keys = list(range(p + 1)) if fa else sa_key_set(p, B, s, w)
            np.testing.assert_allclose(o[p, 0], v[keys, 0].mean(axis=0), rtol=0, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    S, hq, hkv, d, B = 90, 8, 2, 8, 16
    q, k, v = rand_qkv(rng(10), S, hq, hkv, d)
    m = oracle.block_mask(oracle.num_blocks(S, B), 1, 2)
    kr, vr = np.repeat(k, hq // hkv, axis=1), np.repeat(v, hq // hkv, axis=1)
    for fa in (True, False):
        np.testing.assert_allclose(oracle.attention_prefill(q, k, v, fa, m, B),
                                   oracle.attention_prefill(q, kr, vr, fa, m, B),
                                   rtol=0, atol=1e-14)


def test_scale_invariance():
    S, d = 50, 8
    q, k, v = rand_qkv(rng(11), S, 2, 2, d)
    c = 3.0
    a = oracle.attention_prefill(q, k, v, True)
    b = oracle.attention_prefill(q * c, k, v, True, scale=1.0 / (c * math.sqrt(d)))
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("fa", [True, False])
def test_decode_equals_last_prefill_row(fa):
    S, hq, hkv, d, B = 150, 4, 2, 8, 16
    max_len = 160
    r = rng(12)
    nseq = 3
    lens = [150, 129, 17]
    q = r.standard_normal((nseq, S, hq, d))
    kc = r.standard_normal((nseq, hkv, max_len, d))
    vc = r.standard_normal((nseq, hkv, max_len, d))
    m = oracle.block_mask(oracle.num_blocks(max_len, B), 1, 3)
    qd = np.stack([q[b, lens[b] - 1] for b in range(nseq)])
    dec = oracle.attention_decode(qd, kc, vc, lens, fa, m, B)
    for b in range(nseq):
        n = lens[b]
        pre = oracle.attention_prefill(q[b, :n], kc[b, :, :n].transpose(1, 0, 2),
                                       vc[b, :, :n].transpose(1, 0, 2), fa, m, B, rows=[n - 1])
        np.testing.assert_array_equal(dec[b], pre[0])


def test_varlen_requests_are_independent():
    lens = [40, 65, 17]
    cu = np.cumsum([0] + lens)
    T = cu[-1]
    q, k, v = rand_qkv(rng(13), T, 4, 2, 8)
    B = 16
    m = oracle.block_mask(oracle.num_blocks(max(lens), B), 1, 2)
    route = np.array([[1, 0], [0, 1], [1, 1]], dtype=np.uint8)
    for layer in (0, 1):
        outs = oracle.attention_prefill_varlen(q, k, v, cu, route, layer, m, B)
        for r, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
            ref = oracle.attention_prefill(q[a:b], k[a:b], v[a:b], bool(route[r, layer]), m, B)
            np.testing.assert_array_equal(outs[r], ref)


# ---------------------------------------------------------------- planted mistakes

def _fa_pin_fails(fn):
    q, k, v = rand_qkv(rng(99), 40, 4, 2, 8)
    try:
        np.testing.assert_allclose(fn(q, k, v), sdpa_causal(q, k, v), rtol=0, atol=1e-9)
    except AssertionError:
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    # correct oracle passes
    assert not _fa_pin_fails(lambda q, k, v: oracle.attention_prefill(q, k, v, True))
    # 1. scale dropped
    assert _fa_pin_fails(lambda q, k, v: oracle.attention_prefill(q, k, v, True, scale=1.0))
    # 2. causal mask off by one (key p excluded -> row 0 empty, so allow t < p+1 shifted)
    orig = oatt.allowed_matrix

    def shifted(rows, n_keys, fa, mask, B):
        ok = orig(np.asarray(rows) + 1, n_keys, fa, mask, B)
        return ok
    monkeypatch.setattr(oatt, "allowed_matrix", shifted)
    assert _fa_pin_fails(lambda q, k, v: oracle.attention_prefill(q, k, v, True))
    monkeypatch.setattr(oatt, "allowed_matrix", orig)
    # 3. wrong GQA map (h % hkv instead of h // group)
    def wrong_gqa(q, k, v):
        out = np.zeros_like(q)
        for h in range(q.shape[1]):
            out[:, h:h + 1] = oracle.attention_prefill(q[:, h:h + 1], k[:, h % k.shape[1]:h % k.shape[1] + 1],
                                                       v[:, h % k.shape[1]:h % k.shape[1] + 1], True)
        return out
    assert _fa_pin_fails(wrong_gqa)
    # 4. transposed operand in P @ V is caught by the identical-keys closed form
    r = rng(5)
    S, d = 12, 12
    kk = np.tile(r.standard_normal((1, 1, d)), (S, 1, 1))
    vv = r.standard_normal((S, 1, d))
    qq = r.standard_normal((S, 1, d))
    p = oracle.attention_probs(qq[:, 0], kk[:, 0], np.arange(S), True, None, None, 1 / math.sqrt(d))
    wrong = p @ vv[:, 0].T  # transposed V
    right = np.stack([vv[:t + 1, 0].mean(axis=0) for t in range(S)])
    assert not np.allclose(wrong, right)
    # 5. window one block too narrow is caught by the gathered-key-set pin
    S, B, s, w = 64, 8, 1, 3
    q, k, v = rand_qkv(rng(21), S, 1, 1, 4)
    narrow = oracle.attention_prefill(q, k, v, False, oracle.block_mask(8, s, w - 1), B)
    keys = sa_key_set(40, B, s, w)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[40, 0][None, None]), torch.from_numpy(k[keys, 0][None]),
        torch.from_numpy(v[keys, 0][None]))[0, 0].numpy()
    assert not np.allclose(narrow[40, 0], ref, atol=1e-9)


def _soft_reference(q, k, v, r, B, s, w, rows):
    """r * causal SDPA + (1 - r) * SDPA over the gathered SA key set, by torch in float64."""
    fa = sdpa_causal(q, k, v)
    out = []
    for p in rows:
        keys = sa_key_set(p, B, s, w)
        sa = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[p][:, None]), torch.from_numpy(k[keys].transpose(1, 0, 2)),
            torch.from_numpy(v[keys].transpose(1, 0, 2)))[:, 0].numpy()
        out.append(r * fa[p] + (1.0 - r) * sa)
    return np.stack(out)


@pytest.mark.parametrize("r", [1.0, 0.0, 0.25])
def test_soft_routing_is_the_convex_combination(r):
    """The soft-routed forward (technical summary, section 2) against torch SDPA:
    r = 1 is FA, r = 0 is SA, and in between the weights apply as r / 1 - r."""
    S, B, s, w = 48, 8, 1, 2
    q, k, v = rand_qkv(rng(31), S, 1, 1, 8)
    rows = [0, 7, 8, 23, 24, 47]
    m = oracle.block_mask(oracle.num_blocks(S, B), s, w)
    got = oracle.attention_prefill_soft(q, k, v, r, m, B, rows=rows)[:, 0]
    np.testing.assert_allclose(got, _soft_reference(q, k, v, r, B, s, w, rows)[:, 0], rtol=0, atol=1e-12)


def test_soft_routing_planted_swap_is_caught():
    S, B, s, w = 48, 8, 1, 2
    q, k, v = rand_qkv(rng(31), S, 1, 1, 8)
    rows = [23, 47]
    m = oracle.block_mask(oracle.num_blocks(S, B), s, w)
    swapped = oracle.attention_prefill_soft(q, k, v, 0.75, m, B, rows=rows)[:, 0]  # r and 1 - r exchanged
    assert not np.allclose(swapped, _soft_reference(q, k, v, 0.25, B, s, w, rows)[:, 0], atol=1e-9)
