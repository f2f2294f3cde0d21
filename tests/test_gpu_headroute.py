"""Head-level routing (one FA/SA decision per request, layer and kv head)
through the C ABI binding, against the float64 oracle evaluated head group by
head group with that group's decision; a route that is the same for every kv
head must reproduce the per-layer route bit for bit."""

import numpy as np
import pytest
import torch

import oracle
from synth import inputs as syn
from tests.flux_testlib import assert_attn_close, ensure_built

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ensure_built()
    import block_sparse_attention_flux_amd as flux
    from tests.test_gpu_parity import f32, make_decode, run_prefill_case, say
else:  # collected on CPU only to be deselected
    flux = None

DEV = "cuda"


@pytest.mark.parametrize("case", [
    # lens, hq, hkv, d, B, s, w
    ([700, 1, 2100, 129], 8, 4, 128, 128, 1, 3),
    ([1500, 333], 16, 8, 64, 64, 2, 4),
    ([900, 257], 6, 2, 128, 128, 1, 2),    # group 3
])
def test_prefill_head_route(case):
    lens, hq, hkv, d, B, s, w = case
    say(f"prefill head route {case}")
    rng = np.random.default_rng(sum(lens) + hkv)
    route_h = rng.integers(0, 2, size=(len(lens), 2, hkv)).astype(np.uint8)
    route_h[0, 0, :] = 1  # one layer of one request all FA, one all SA
    route_h[0, 1, :] = 0
    q, k, v, cu, sa, rp, ci, _ = run_prefill_case(lens, hq, hkv, d, B, s, w, [[1, 0]] * len(lens),
                                                  900 + d)
    route = torch.from_numpy(route_h).to(DEV)
    m = oracle.block_mask(oracle.num_blocks(max(lens), B), s, w)
    group = hq // hkv
    cu_h = np.cumsum([0] + lens)
    qf, kf, vf = f32(q), f32(k), f32(v)
    for layer in range(2):
        out = flux.attn_prefill(q, k, v, cu, max(lens), route, layer, rp, ci, sa)
        torch.cuda.synchronize()
        of = f32(out)
        for r, (a, b) in enumerate(zip(cu_h[:-1], cu_h[1:])):
            for g in range(hkv):
                heads = list(range(g * group, (g + 1) * group))
                ref = oracle.attention_prefill(qf[a:b], kf[a:b], vf[a:b], bool(route_h[r, layer, g]), m,
                                               B, heads=heads)
                assert_attn_close(of[a:b][:, heads], ref, f"req {r} layer {layer} kv head {g}")
    # uniform per-head decisions == the per-layer route, bitwise
    per_layer = torch.tensor([[1, 0]] * len(lens), dtype=torch.uint8, device=DEV)
    uniform = per_layer[:, :, None].repeat(1, 1, hkv).contiguous()
    for layer in range(2):
        a = flux.attn_prefill(q, k, v, cu, max(lens), per_layer, layer, rp, ci, sa)
        b = flux.attn_prefill(q, k, v, cu, max(lens), uniform, layer, rp, ci, sa)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_decode_head_route():
    n_seq, max_len, seqlens, hq, hkv, d, B, s, w = 4, 3000, [3000, 1, 1290, 2049], 16, 4, 128, 128, 1, 4
    say("decode head route")
    q, kc, vc, sl = make_decode(n_seq, max_len, seqlens, hq, hkv, d, 321)
    sa = flux.SAParams(B, s, w)
    _, rp, ci = flux.build_block_mask(max_len, sa, dense=False)
    m = oracle.block_mask(oracle.num_blocks(max_len, B), s, w)
    rng = np.random.default_rng(5)
    route_h = rng.integers(0, 2, size=(n_seq, 3, hkv)).astype(np.uint8)
    route = torch.from_numpy(route_h).to(DEV)
    group = hq // hkv
    qf, kf, vf = f32(q), f32(kc), f32(vc)
    for layer in range(3):
        out = flux.attn_decode(q, kc, vc, sl, route, layer, rp, ci, sa)
        torch.cuda.synchronize()
        of = f32(out)
        for g in range(hkv):
            heads = list(range(g * group, (g + 1) * group))
            ref = oracle.attention_decode(qf, kf, vf, seqlens, route_h[:, layer, g].astype(bool), m, B,
                                          heads=heads)
            assert_attn_close(of[:, heads], ref, f"decode layer {layer} kv head {g}")
