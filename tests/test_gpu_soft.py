"""Soft-routed forward r * FA + (1 - r) * SA (one kernel pass with one
softmax state: the SA blocks first, the weighted SA output parked in bf16,
then FA's other blocks) through the C ABI binding, against the float64
oracle, including r = 1 and r = 0 (within the attention tolerance of the
routed FA and SA layers: the parked SA part is rounded to bf16 once) and a
mask whose rows leave out their diagonal block."""

import numpy as np
import pytest
import torch

import oracle
from tests.flux_testlib import assert_attn_close, ensure_built

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ensure_built()
    import block_sparse_attention_flux_amd as flux
    from tests.test_gpu_parity import f32, run_prefill_case, say
else:  # collected on CPU only to be deselected
    flux = None

DEV = "cuda"


@pytest.mark.parametrize("case", [
    # lens, hq, hkv, d, B, s, w, r per request
    ([900, 1, 2300, 130], 8, 2, 128, 128, 1, 3, [0.3, 1.0, 0.0, 0.8]),
    ([1024, 515], 4, 4, 64, 64, 2, 2, [0.5, 0.125]),
    ([700, 260], 6, 2, 64, 128, 1, 2, [0.7, 0.2]),    # group 3, d 64 with 128-row blocks
])
def test_soft_prefill(case):
    lens, hq, hkv, d, B, s, w, rs = case
    say(f"soft prefill {case}")
    q, k, v, cu, sa, rp, ci, route = run_prefill_case(lens, hq, hkv, d, B, s, w, [[1, 0]] * len(lens),
                                                      1200 + d)
    r_soft = torch.tensor([[x, 1.0 - x] for x in rs], dtype=torch.float32, device=DEV)
    m = oracle.block_mask(oracle.num_blocks(max(lens), B), s, w)
    cu_h = np.cumsum([0] + lens)
    qf, kf, vf = f32(q), f32(k), f32(v)
    for layer in range(2):
        out = flux.attn_prefill_soft(q, k, v, cu, max(lens), r_soft, layer, rp, ci, sa)
        torch.cuda.synchronize()
        of = f32(out)
        for i, (a, b) in enumerate(zip(cu_h[:-1], cu_h[1:])):
            ref = oracle.attention_prefill_soft(qf[a:b], kf[a:b], vf[a:b], float(r_soft[i, layer]), m, B)
            assert_attn_close(of[a:b], ref, f"req {i} layer {layer} r {float(r_soft[i, layer])}")
    # endpoints: r = 1 is the FA layer, r = 0 the SA layer, against the oracle
    # and against the routed layers
    ones = torch.ones((len(lens), 1), dtype=torch.float32, device=DEV)
    fa = flux.attn_prefill(q, k, v, cu, max(lens), route, 0, rp, ci, sa)
    sa_out = flux.attn_prefill(q, k, v, cu, max(lens), route, 1, rp, ci, sa)
    s1 = flux.attn_prefill_soft(q, k, v, cu, max(lens), ones, 0, rp, ci, sa)
    s0 = flux.attn_prefill_soft(q, k, v, cu, max(lens), ones * 0, 0, rp, ci, sa)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(cu_h[:-1], cu_h[1:])):
        ref1 = oracle.attention_prefill(qf[a:b], kf[a:b], vf[a:b], True, m, B)
        ref0 = oracle.attention_prefill(qf[a:b], kf[a:b], vf[a:b], False, m, B)
        assert_attn_close(f32(s1)[a:b], ref1, f"req {i} r = 1")
        assert_attn_close(f32(s0)[a:b], ref0, f"req {i} r = 0")
        assert_attn_close(f32(s1)[a:b], f32(fa)[a:b], f"req {i} r = 1 vs the FA layer")
        assert_attn_close(f32(s0)[a:b], f32(sa_out)[a:b], f"req {i} r = 0 vs the SA layer")


def test_soft_prefill_rows_without_their_diagonal_block():
    """A hand-made mask: row i keeps block 0 and every block j < i with j % 3
    == 1, and its diagonal block only when i % 2 == 0 (rows 0 and 1 keep block
    0 only).  The soft pass then visits FA's remaining blocks, the diagonal
    among them, after the SA ones."""
    S, hq, hkv, d, B = 1000, 4, 2, 64, 64
    nb = -(-S // B)
    m = np.zeros((nb, nb), dtype=np.uint8)
    for i in range(nb):
        m[i, 0] = 1
        for j in range(1, i):
            if j % 3 == 1:
                m[i, j] = 1
        if i % 2 == 0:
            m[i, i] = 1
    rp_h, ci_h = oracle.mask_to_csr(m)
    say("soft prefill, rows without their diagonal block")
    q, k, v, cu, sa, _, _, _ = run_prefill_case([S], hq, hkv, d, B, 1, 1, [[1, 0]], 1300)
    rp = torch.tensor(rp_h, dtype=torch.int32, device=DEV)
    ci = torch.tensor(ci_h, dtype=torch.int32, device=DEV)
    qf, kf, vf = f32(q), f32(k), f32(v)
    for r in (0.0, 0.35, 1.0):
        r_soft = torch.full((1, 1), r, dtype=torch.float32, device=DEV)
        out = flux.attn_prefill_soft(q, k, v, cu, S, r_soft, 0, rp, ci, sa)
        torch.cuda.synchronize()
        ref = oracle.attention_prefill_soft(qf, kf, vf, r, m, B)
        assert_attn_close(f32(out), ref, f"r {r}")
