"""flux_attn_decode_noalloc (the decode entry point that allocates nothing and
keeps its partials in the library's device scratch) against flux_attn_decode
with a caller workspace: bit-identical outputs on two calls in a row, the
second with a smaller input, and within tolerance of the float64 oracle.
"""

import pytest
import torch

import oracle
from synth import inputs as syn
from tests.flux_testlib import assert_attn_close, ensure_built

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    ensure_built()
    import block_sparse_attention_flux_amd as flux
else:  # collected on CPU only to be deselected
    flux = None

DEV = "cuda"


def f32(t):
    return t.detach().float().cpu().numpy()


def case(lens, hq, hkv, d, B, s, w, seed):
    n, max_len = len(lens), max(lens)
    g = syn.generator(seed, DEV)
    q = syn.normal((n, hq, d), g, DEV)
    kc = syn.normal((n, hkv, max_len, d), g, DEV)
    vc = syn.normal((n, hkv, max_len, d), g, DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    sa = flux.SAParams(B, s, w)
    _, rp, ci = flux.build_block_mask(max_len, sa, dense=False)
    m = oracle.block_mask(oracle.num_blocks(max_len, B), s, w)
    return q, kc, vc, sl, sa, rp, ci, m


def test_noalloc_matches_workspace_decode_twice():
    big = ([20000, 3000, 129, 1, 9000, 2176], 32, 8, 128, 128, 1, 16, 8181)
    small = ([700, 65, 2], 8, 2, 64, 64, 1, 3, 8282)
    for lens, hq, hkv, d, B, s, w, seed in (big, small):
        print(f"noalloc decode lens={lens} hq={hq} hkv={hkv} d={d}", flush=True)
        q, kc, vc, sl, sa, rp, ci, m = case(lens, hq, hkv, d, B, s, w, seed)
        n = len(lens)
        route = torch.tensor([[1, 0], [0, 1]] * (n // 2) + [[1, 0]] * (n % 2), dtype=torch.uint8,
                             device=DEV)
        assert 0 < flux.decode_workspace_size(n, hq, hkv, d, max(lens)) <= (16 << 20)
        for layer in (0, 1):
            ref_out = flux.attn_decode(q, kc, vc, sl, route, layer, rp, ci, sa)
            got = flux.attn_decode_noalloc(q, kc, vc, sl, route, layer, rp, ci, sa)
            torch.cuda.synchronize()
            assert torch.equal(got, ref_out), f"layer {layer}: differs from flux_attn_decode"
            fa = [bool(route[b, layer]) for b in range(n)]
            ref = oracle.attention_decode(f32(q), f32(kc), f32(vc), lens, fa, m, B)
            assert_attn_close(f32(got), ref, f"noalloc layer {layer}")
