"""GPU tests of the decode caches through the C ABI binding: the prompt store
and the per-step append are exact byte moves, and SA decode over a compact
cache (sink rows + a ring of the window) is bit-identical to SA decode over
the full cache, step after step, across block boundaries and ring wrap-round;
sampled steps are also checked against the float64 oracle."""

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
    from tests.test_gpu_parity import f32, say
else:  # collected on CPU only to be deselected
    flux = None

DEV = "cuda"


def packed(lens, hkv, d, g):
    T = sum(lens)
    return syn.normal((T, hkv, d), g, DEV), syn.normal((T, hkv, d), g, DEV)


def test_store_and_append_full_cache_exact():
    say("kv store/append full")
    lens, hkv, d, max_len = [5, 130, 1000], 2, 128, 1100
    sa = flux.SAParams(128, 1, 2)
    g = syn.generator(501, DEV)
    k, v = packed(lens, hkv, d, g)
    cu = syn.cu_seqlens(lens, DEV)
    kc, vc = flux.kv_cache(len(lens), hkv, d, max_len, sa)
    flux.kv_store_prefill(k, v, cu, max(lens), kc, vc, max_len, sa)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    new = []
    for t in range(5):
        sl = sl + 1
        kn, vn = syn.normal((len(lens), hkv, d), g, DEV), syn.normal((len(lens), hkv, d), g, DEV)
        flux.kv_append(kn, vn, sl, kc, vc, max_len, sa)
        new.append((kn, vn))
    torch.cuda.synchronize()
    c = [0] + list(np.cumsum(lens))
    for b, S in enumerate(lens):
        assert torch.equal(kc[b, :, :S], k[c[b]:c[b + 1]].transpose(0, 1))
        assert torch.equal(vc[b, :, :S], v[c[b]:c[b + 1]].transpose(0, 1))
        for t, (kn, vn) in enumerate(new):
            assert torch.equal(kc[b, :, S + t], kn[b]) and torch.equal(vc[b, :, S + t], vn[b])
        assert not kc[b, :, S + 5:].any() and not vc[b, :, S + 5:].any()  # untouched rows


@pytest.mark.parametrize("case", [
    # lens, hq, hkv, d, B, s, w, steps
    ([70, 1000, 4100], 8, 2, 128, 64, 1, 3, 300),
    ([129, 2500], 4, 4, 64, 128, 2, 4, 300),
    ([1, 640, 3000], 16, 1, 128, 64, 0, 2, 200),
])
def test_compact_sa_decode_matches_full(case):
    lens, hq, hkv, d, B, s, w, steps = case
    say(f"compact decode {case}")
    n = len(lens)
    max_len = max(lens) + steps
    sa = flux.SAParams(B, s, w)
    g = syn.generator(700 + d + B, DEV)
    k, v = packed(lens, hkv, d, g)
    cu = syn.cu_seqlens(lens, DEV)
    kf, vf = flux.kv_cache(n, hkv, d, max_len, sa)
    kcp, vcp = flux.kv_cache(n, hkv, d, max_len, sa, compact=True)
    assert kcp.shape[2] == (s + w) * B
    flux.kv_store_prefill(k, v, cu, max(lens), kf, vf, max_len, sa)
    flux.kv_store_prefill(k, v, cu, max(lens), kcp, vcp, max_len, sa, compact=True)
    _, rp, ci = flux.build_block_mask(max_len, sa, dense=False)
    route = torch.zeros((n, 1), dtype=torch.uint8, device=DEV)  # every sequence SA
    ws_full = flux.decode_workspace(n, hq, hkv, d, max_len, DEV)
    ws_cmp = flux.decode_workspace(n, hq, hkv, d, max_len, DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    m = oracle.block_mask(oracle.num_blocks(max_len, B), s, w)
    check_at = {0, steps // 2, steps - 1}
    for t in range(steps):
        sl = sl + 1
        kn, vn = syn.normal((n, hkv, d), g, DEV), syn.normal((n, hkv, d), g, DEV)
        flux.kv_append(kn, vn, sl, kf, vf, max_len, sa)
        flux.kv_append(kn, vn, sl, kcp, vcp, max_len, sa, compact=True)
        q = syn.normal((n, hq, d), g, DEV)
        full = flux.attn_decode(q, kf, vf, sl, route, 0, rp, ci, sa, ws_full)
        cmp_ = flux.attn_decode_sa_compact(q, kcp, vcp, sl, max_len, rp, ci, sa, ws_cmp)
        torch.cuda.synchronize()
        assert torch.equal(full, cmp_), f"step {t}: compact and full caches differ"
        if t in check_at:
            ref = oracle.attention_decode(f32(q), f32(kf), f32(vf), sl.cpu().numpy(), False, m, B)
            assert_attn_close(f32(cmp_), ref, f"compact decode step {t}")


@pytest.mark.parametrize("case", [
    # lens, hq, hkv, d, B, s, w, steps
    ([9000, 130, 1, 2000, 4095], 32, 8, 128, 128, 1, 16, 6),
    ([700, 64, 63], 8, 2, 64, 64, 1, 3, 4),
])
def test_fused_append_matches_append_then_decode(case):
    """flux_attn_decode_append equals flux_kv_append + flux_attn_decode bit for
    bit, outputs and caches, step after step, with mixed routes and a sequence
    whose length falls outside [1, max_len] (no row appended, as kv_append);
    one step is also checked against the oracle."""
    lens, hq, hkv, d, B, s, w, steps = case
    n = len(lens)
    max_len = max(lens) + steps
    say(f"fused append {case}")
    sa = flux.SAParams(B, s, w)
    g = syn.generator(8383, DEV)
    kc = syn.normal((n, hkv, max_len, d), g, DEV)
    vc = syn.normal((n, hkv, max_len, d), g, DEV)
    kc2, vc2 = kc.clone(), vc.clone()
    _, rp, ci = flux.build_block_mask(max_len, sa, dense=False)
    route = torch.tensor([[1, 0], [0, 1]] * (n // 2) + [[1, 1]] * (n % 2), dtype=torch.uint8, device=DEV)
    base = torch.tensor(lens, dtype=torch.int32, device=DEV)
    for t in range(steps):
        sl = base + t + 1
        if t == steps - 1:
            sl[1] = max_len + 5   # out of range: no row is appended, the length is clamped
        q = syn.normal((n, hq, d), g, DEV)
        kn, vn = syn.normal((n, hkv, d), g, DEV), syn.normal((n, hkv, d), g, DEV)
        for layer in (0, 1):
            fused = flux.attn_decode_append(q, kn, vn, kc, vc, sl, route, layer, rp, ci, sa)
            flux.kv_append(kn, vn, sl, kc2, vc2, max_len, sa)
            ref_out = flux.attn_decode(q, kc2, vc2, sl, route, layer, rp, ci, sa)
            torch.cuda.synchronize()
            assert torch.equal(fused, ref_out), f"step {t} layer {layer}: output differs"
            assert torch.equal(kc, kc2) and torch.equal(vc, vc2), f"step {t} layer {layer}: caches differ"
        if t == 2:
            m = oracle.block_mask(oracle.num_blocks(max_len, B), s, w)
            lens_t = [int(x) for x in sl.tolist()]
            fa = [bool(route[b, 1]) for b in range(n)]
            ref = oracle.attention_decode(f32(q), f32(kc), f32(vc), lens_t, fa, m, B)
            assert_attn_close(f32(fused), ref, f"fused append step {t}")
