"""Content-aware SA block mask through the C ABI binding
(flux_build_block_mask_dynamic), against the float64 oracle.

The selection is integer output decided by floating point (the kernel sums
in fp32, the oracle in fp64), so every row is checked for the defining
properties with the oracle's probabilities and a small tolerance, and rows
whose decision has a clear margin must equal the oracle's row exactly.  SA
prefill on the GPU's mask is then compared with the oracle's attention on the
same mask."""

import numpy as np
import pytest
import torch

import oracle
from tests.flux_testlib import assert_attn_close, ensure_built

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ensure_built()
    import block_sparse_attention_flux_amd as flux
    from synth import inputs as syn
    from tests.test_gpu_parity import f32, say
else:  # collected on CPU only to be deselected
    flux = None

DEV = "cuda"
EPS_MASS = 2e-5   # fp32 accumulation of probabilities that sum to 1
EPS_P = 2e-6      # relative: fp32 exponentials and sums against fp64


def csr_to_dense(row_ptr, col_idx, nb):
    rp = row_ptr.cpu().numpy()
    ci = col_idx.cpu().numpy()
    m = np.zeros((nb, nb), dtype=np.uint8)
    for i in range(nb):
        cols = ci[rp[i]:rp[i + 1]]
        assert np.all(np.diff(cols) > 0), f"row {i} columns not increasing"
        m[i, cols] = 1
    return m


def check_rows(m, P, rows, tau, sink, cap, what):
    """Top-tau properties of the GPU rows ``m[rows]`` under the oracle's
    probabilities (``P[n]`` is row ``rows[n]``); rows whose decision has a
    clear margin must equal the oracle's row.  Returns how many did."""
    exact = 0
    for n, i in enumerate(rows):
        p = P[n]
        row = m[i]
        assert np.all(row[i + 1:] == 0), f"{what}: row {i} not causal"
        mand = [j for j in range(i + 1) if j < sink or j == i]
        assert all(row[j] for j in mand), f"{what}: row {i} lost a mandatory block"
        cand = sorted([j for j in range(i + 1) if j not in mand], key=lambda j: (-p[j], j))
        chosen = [j for j in cand if row[j]]
        if cap > 0:
            assert len(mand) + len(chosen) <= max(cap, len(mand)), f"{what}: row {i} over the cap"
        base = p[mand].sum()
        mass = base + p[chosen].sum()
        full = len(chosen) == len(cand) or (cap > 0 and len(mand) + len(chosen) >= cap)
        assert mass >= tau - EPS_MASS or full, f"{what}: row {i} stops short of tau ({mass} < {tau})"
        if chosen:
            low = min(p[j] for j in chosen)
            assert mass - low < tau + EPS_MASS, f"{what}: row {i} keeps a block it did not need"
            for j in cand:
                if not row[j]:
                    assert p[j] <= low * (1 + EPS_P) + 1e-12, f"{what}: row {i} skipped a heavier block {j}"
        # a clear decision (the cut far from tau and from a tie) must match exactly
        ref = oracle.select_row(p, i, tau, sink, cap)
        kk = len(ref) - len(mand)
        cum = base + np.cumsum([p[j] for j in cand]) if cand else np.array([])
        margins = [abs(base - tau)] + [abs(cum[r] - tau) for r in range(max(kk - 2, 0), min(kk + 1, len(cand)))]
        gaps = [abs(p[cand[r]] - p[cand[r + 1]]) / max(p[cand[r]], 1e-30)
                for r in range(max(kk - 1, 0), min(kk + 1, len(cand) - 1))]
        if min(margins) > 1e-3 and (not gaps or min(gaps) > 1e-4):
            assert sorted(np.nonzero(row)[0].tolist()) == ref, f"{what}: row {i}"
            exact += 1
    return exact


def qk(S, hq, hkv, d, seed, planted=False):
    g = syn.generator(seed, DEV)
    q = syn.normal((S, hq, d), g, DEV)
    k = syn.normal((S, hkv, d), g, DEV)
    if planted:  # every query leans on one direction; a few key blocks align with it
        u = syn.normal((d,), g, DEV, torch.float32)
        u = u / u.norm()
        q = (q.float() * 0.3 + 2.0 * u).to(torch.bfloat16)
        kf = k.float() * 0.3
        B = 64
        for blk in (1, 5, 9):
            if blk * B < S:
                kf[blk * B:(blk + 1) * B] += 4.0 * u
        k = kf.to(torch.bfloat16)
    return q, k


@pytest.mark.parametrize("case", [
    # S, hq, hkv, d, B, tau, sink, cap, planted
    (1000, 8, 2, 128, 64, 0.6, 1, 0, False),
    (777, 4, 4, 64, 64, 0.9, 2, 6, False),
    (2048, 16, 2, 128, 128, 0.5, 0, 0, True),
    (1300, 8, 1, 64, 64, 0.3, 1, 4, True),
    (640, 6, 2, 64, 64, 0.7, 1, 0, False),     # group 3 (padded to 4 in the kernel)
    (900, 16, 1, 128, 64, 0.8, 2, 6, True),    # group 16
])
def test_dynamic_mask_matches_oracle(case):
    S, hq, hkv, d, B, tau, sink, cap, planted = case
    say(f"dynamic mask {case}")
    q, k = qk(S, hq, hkv, d, 500 + S, planted)
    row_ptr, col_idx = flux.build_block_mask_dynamic(q, k, B, sink, tau, cap)
    torch.cuda.synchronize()
    nb = (S + B - 1) // B
    m = csr_to_dense(row_ptr, col_idx, nb)
    P = oracle.block_probs(f32(q), f32(k), B)
    exact = check_rows(m, P, list(range(nb)), tau, sink, cap, f"case {case}")
    assert exact >= nb // 2, f"only {exact} of {nb} rows had a clear decision"


@pytest.mark.parametrize("tau,cap", [(0.0, 0), (1.0, 0), (5.0, 3)])
def test_dynamic_mask_limits(tau, cap):
    """tau = 0: sink + diagonal; tau = 1, no cap: every causal block (exactly,
    P > 0 everywhere); a cap with tau past 1: the first blocks by P, as many as
    the cap allows."""
    S, hq, hkv, d, B, sink = 900, 4, 2, 64, 64, 1
    say(f"dynamic mask limits tau={tau} cap={cap}")
    q, k = qk(S, hq, hkv, d, 31)
    row_ptr, col_idx = flux.build_block_mask_dynamic(q, k, B, sink, tau, cap)
    torch.cuda.synchronize()
    nb = (S + B - 1) // B
    m = csr_to_dense(row_ptr, col_idx, nb)
    if tau == 0.0:
        for i in range(nb):
            assert set(np.nonzero(m[i])[0].tolist()) == ({0, i} if sink else {i})
    elif cap == 0:
        np.testing.assert_array_equal(m, np.tril(np.ones((nb, nb), dtype=np.uint8)))
    else:
        P = oracle.block_probs(f32(q), f32(k), B)
        check_rows(m, P, list(range(nb)), tau, sink, cap, "cap")
        for i in range(nb):
            assert m[i].sum() == max(min(i + 1, cap), len({0, i}))


def test_sa_prefill_on_dynamic_mask():
    """The SA layer reads the GPU's dynamic mask exactly like the static one:
    compare with the oracle's attention on that same mask."""
    S, hq, hkv, d, B = 1500, 8, 2, 128, 128
    say("SA prefill on a dynamic mask")
    q, k = qk(S, hq, hkv, d, 41, planted=True)
    g = syn.generator(42, DEV)
    v = syn.normal((S, hkv, d), g, DEV)
    row_ptr, col_idx = flux.build_block_mask_dynamic(q, k, B, 1, 0.7, 5)
    nb = (S + B - 1) // B
    cu = torch.tensor([0, S], dtype=torch.int32, device=DEV)
    route = torch.tensor([[0]], dtype=torch.uint8, device=DEV)
    sa = flux.SAParams(B, 1, 2)
    out = flux.attn_prefill(q, k, v, cu, S, route, 0, row_ptr, col_idx, sa)
    torch.cuda.synchronize()
    m = csr_to_dense(row_ptr, col_idx, nb)
    ref = oracle.attention_prefill(f32(q), f32(k), f32(v), False, m, B)
    assert_attn_close(f32(out), ref, "SA on dynamic mask")


def test_dynamic_mask_32k_sampled():
    """The 32K layer shape (32 / 8 heads, d 128, blocks of 128) with the
    bench's parameters: every row checked for the Top-tau properties against
    the oracle's probabilities of sampled rows."""
    S, hq, hkv, d, B, tau, sink, cap = 32768, 32, 8, 128, 128, 0.9, 1, 17
    say("dynamic mask 32K")
    q, k = qk(S, hq, hkv, d, 1002)
    row_ptr, col_idx = flux.build_block_mask_dynamic(q, k, B, sink, tau, cap)
    torch.cuda.synchronize()
    nb = S // B
    m = csr_to_dense(row_ptr, col_idx, nb)
    rows = [0, 1, 2, 17, 100, 200, 255]
    P = oracle.block_probs_rows(f32(q), f32(k), B, rows)
    check_rows(m, P, rows, tau, sink, cap, "32K")
    counts = m.sum(axis=1)
    # random data: the rows are nearly uniform, so past row 18 the cap binds before tau
    assert counts.max() <= cap and counts[19:].min() == cap


def test_decode_on_dynamic_mask():
    """SA decode reads any CSR row, scattered blocks included: the dynamic mask
    of a 3000-token prompt drives decode at several cached lengths (the mask
    row is that of each sequence's last block), against the oracle's decode on
    the same mask."""
    from tests.test_gpu_parity import make_decode
    S, hq, hkv, d, B = 3000, 8, 2, 128, 128
    say("decode on a dynamic mask")
    q, k = qk(S, hq, hkv, d, 61, planted=True)
    row_ptr, col_idx = flux.build_block_mask_dynamic(q, k, B, 1, 0.5, 6)
    nb = (S + B - 1) // B
    m = csr_to_dense(row_ptr, col_idx, nb)
    assert not np.array_equal(m, oracle.block_mask(nb, 1, 5))  # not a sink + window pattern
    seqlens = [3000, 1777, 129, 1]
    qd, kc, vc, sl = make_decode(len(seqlens), S, seqlens, hq, hkv, d, 62)
    sa = flux.SAParams(B, 1, 5)
    route = torch.tensor([[0]] * len(seqlens), dtype=torch.uint8, device=DEV)
    out = flux.attn_decode(qd, kc, vc, sl, route, 0, row_ptr, col_idx, sa)
    torch.cuda.synchronize()
    ref = oracle.attention_decode(f32(qd), f32(kc), f32(vc), seqlens, False, m, B)
    assert_attn_close(f32(out), ref, "decode on dynamic mask")
