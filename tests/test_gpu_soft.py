"""Soft-routed forward r * FA + (1 - r) * SA (one kernel pass, two softmax
states) through the C ABI binding, against the float64 oracle; r = 1 and
r = 0 must reproduce the routed FA and SA layers bit for bit."""

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
    # endpoints: r = 1 is the routed FA layer, r = 0 the routed SA layer, bitwise
    ones = torch.ones((len(lens), 1), dtype=torch.float32, device=DEV)
    fa = flux.attn_prefill(q, k, v, cu, max(lens), route, 0, rp, ci, sa)
    sa_out = flux.attn_prefill(q, k, v, cu, max(lens), route, 1, rp, ci, sa)
    s1 = flux.attn_prefill_soft(q, k, v, cu, max(lens), ones, 0, rp, ci, sa)
    s0 = flux.attn_prefill_soft(q, k, v, cu, max(lens), ones * 0, 0, rp, ci, sa)
    torch.cuda.synchronize()
    assert torch.equal(s1, fa)
    assert torch.equal(s0, sa_out)
