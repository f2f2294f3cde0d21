"""GPU parity on the two long workloads, through the C ABI binding, against
the float64 oracle on the same seeded inputs.

prefill131k -- Qwen3-4B shapes at 131072 tokens: the router (2560 -> 256 -> 36)
    on a 131072 x 2560 bf16 hidden matrix, then FA and SA layers (SA: blocks of
    128, 1 sink block, a 4096-token window) on sampled rows and all heads; the
    layers are routed by the router's own decisions.
varlen8 -- Llama-3-8B shapes: 8 prompts with seeded lengths in [8192, 65536],
    the router (4096 -> 256 -> 32) per request, a packed prefill layer routed by
    it and one routed FA/SA per request in a checkerboard, then 128 decode
    steps that append one seeded K/V row per step to each sequence's cache
    (the append is plain tensor indexing here), checked at three steps.

The router's pooling reads only the first and last 100 rows of a request, so
the oracle is handed exactly the rows that oracle.pool_positions names for
each request, as a request of that many rows (whose pool is all of its rows).
Rows, heads and sequences are sampled where the oracle would otherwise widen
gigabytes per call; the bar is the one of test_gpu_parity.py.
"""

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
    from tests.test_gpu_parity import check_route, f32, sampled_rows, say
else:  # collected on CPU only to be deselected
    flux = None

DEV = "cuda"


def route_and_check(hidden, lens, w1, b1, w2, b2):
    """flux_route on the device, checked against the oracle on the pooled rows."""
    cu = syn.cu_seqlens(lens, DEV)
    L = w2.shape[0]
    logits = torch.empty((len(lens), L), dtype=torch.float32, device=DEV)
    route, _ = flux.route(hidden, cu, w1.to(DEV), b1.to(DEV), w2.to(DEV), b2.to(DEV),
                          logits_out=logits)
    torch.cuda.synchronize()
    starts = np.cumsum([0] + list(lens))[:-1]
    picked = [a + oracle.pool_positions(S) for a, S in zip(starts, lens)]
    rows = torch.from_numpy(np.concatenate(picked)).to(DEV)
    sub = f32(hidden.index_select(0, rows))
    sub_lens = [len(p) for p in picked]
    r_ref, z_ref = oracle.route_requests(sub, np.cumsum([0] + sub_lens), w1.numpy(), b1.numpy(),
                                         w2.numpy(), b2.numpy())
    cs = np.cumsum([0] + sub_lens)
    hs = [np.maximum(w1.numpy().astype(np.float64) @ oracle.pool_mean(sub[a:b]) + b1.numpy(), 0)
          for a, b in zip(cs[:-1], cs[1:])]
    scale = np.stack([np.abs(w2.numpy()) @ np.abs(h) + np.abs(b2.numpy()) for h in hs])
    ties = check_route(route.cpu().numpy(), logits.cpu().numpy(), r_ref, z_ref, w2, scale)
    assert ties == 0
    return route


def test_prefill_131k_routed():
    wl = syn.PREFILL128K
    S, B = wl.seqlens[0], wl.block_size
    say("prefill 131k: router")
    g = syn.generator(wl.seed, DEV)
    hidden = syn.normal((S, wl.hidden_dim), g, DEV)
    w1, b1, w2, b2 = syn.router_weights(wl.hidden_dim, wl.router_h1, wl.n_layers, wl.seed)
    route = route_and_check(hidden, [S], w1, b1, w2, b2)
    del hidden
    r = route.cpu().numpy()[0]
    say(f"prefill 131k: router sends {int(r.sum())} of {wl.n_layers} layers to FA")
    # layers to run: the first FA and the first SA layer the router chose, and
    # a forced FA/SA pair on the same inputs so both modes are always covered
    layers = [int(np.argmax(r == 1))] if (r == 1).any() else []
    layers += [int(np.argmax(r == 0))] if (r == 0).any() else []
    q = syn.normal((S, wl.hq, wl.head_dim), g, DEV)
    k = syn.normal((S, wl.hkv, wl.head_dim), g, DEV)
    v = syn.normal((S, wl.hkv, wl.head_dim), g, DEV)
    cu = syn.cu_seqlens([S], DEV)
    sa = flux.SAParams(B, wl.sink_blocks, wl.local_blocks)
    _, rp, ci = flux.build_block_mask(S, sa, dense=False)
    m = oracle.block_mask(oracle.num_blocks(S, B), wl.sink_blocks, wl.local_blocks)
    rows = sampled_rows(S, B, 6, 41)
    rows = np.array(sorted(set(rows.tolist()) | {4095, 4096, 4097, 65535, 65536}))
    qf, kf, vf = f32(q), f32(k), f32(v)
    forced = torch.tensor([[1, 0]], dtype=torch.uint8, device=DEV)
    runs = [(route, l, bool(r[l])) for l in layers] + [(forced, 0, True), (forced, 1, False)]
    for rt, layer, fa in runs:
        say(f"prefill 131k: layer {layer} fa={fa}")
        out = flux.attn_prefill(q, k, v, cu, S, rt, layer, rp, ci, sa)
        torch.cuda.synchronize()
        ref = oracle.attention_prefill(qf, kf, vf, fa, m, B, rows=rows)
        assert_attn_close(f32(out)[rows], ref, f"131k layer {layer} fa={fa}")


def test_varlen8_routed_prefill_and_decode():
    wl = syn.varlen8()
    lens = list(wl.seqlens)
    B = wl.block_size
    n = len(lens)
    say(f"varlen8: lengths {lens}")
    g = syn.generator(wl.seed, DEV)
    T = sum(lens)
    hidden = syn.normal((T, wl.hidden_dim), g, DEV)
    w1, b1, w2, b2 = syn.router_weights(wl.hidden_dim, wl.router_h1, wl.n_layers, wl.seed)
    route = route_and_check(hidden, lens, w1, b1, w2, b2)
    del hidden
    r = route.cpu().numpy()
    say(f"varlen8: FA decisions per request {r.sum(axis=1).tolist()} of {wl.n_layers}")

    # ---- prefill: the router's route at one layer, and a checkerboard route
    q = syn.normal((T, wl.hq, wl.head_dim), g, DEV)
    k = syn.normal((T, wl.hkv, wl.head_dim), g, DEV)
    v = syn.normal((T, wl.hkv, wl.head_dim), g, DEV)
    cu = syn.cu_seqlens(lens, DEV)
    cu_h = np.cumsum([0] + lens)
    max_s = max(lens)
    sa = flux.SAParams(B, wl.sink_blocks, wl.local_blocks)
    _, rp, ci = flux.build_block_mask(max_s + wl.decode_steps, sa, dense=False)
    m = oracle.block_mask(oracle.num_blocks(max_s + wl.decode_steps, B), wl.sink_blocks,
                          wl.local_blocks)
    heads = [0, 9, 22, 31]
    rows_per_req = [sampled_rows(S, B, 3, 60 + i) for i, S in enumerate(lens)]
    qf, kf, vf = f32(q), f32(k), f32(v)
    checker = torch.tensor([[(i + j) % 2 for j in range(2)] for i in range(n)], dtype=torch.uint8,
                           device=DEV)
    layer_r = 7
    for rt, layer in ((route, layer_r), (checker, 0)):
        rt_h = rt.cpu().numpy()
        say(f"varlen8 prefill: layer {layer} route {rt_h[:, layer].tolist()}")
        out = flux.attn_prefill(q, k, v, cu, max_s, rt, layer, rp, ci, sa)
        torch.cuda.synchronize()
        refs = oracle.attention_prefill_varlen(qf, kf, vf, cu_h, rt_h, layer, m, B,
                                               rows_per_req=rows_per_req, heads=heads)
        of = f32(out)
        for i, (a, rows) in enumerate(zip(cu_h[:-1], rows_per_req)):
            assert_attn_close(of[a + rows][:, heads], refs[i], f"req {i} layer {layer}")
    del qf, q

    # ---- decode: caches hold the prompts' K/V, one seeded row appended per step
    max_len = max_s + wl.decode_steps
    kc = torch.zeros((n, wl.hkv, max_len, wl.head_dim), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    for i, (a, b) in enumerate(zip(cu_h[:-1], cu_h[1:])):
        kc[i, :, :b - a] = k[a:b].transpose(0, 1)
        vc[i, :, :b - a] = v[a:b].transpose(0, 1)
    del k, v, kf, vf
    base = torch.tensor(lens, dtype=torch.int32, device=DEV)
    ws = flux.decode_workspace(n, wl.hq, wl.hkv, wl.head_dim, max_len, DEV)
    checks = {0: None, 64: None, wl.decode_steps - 1: None}
    for t in range(wl.decode_steps):
        pos = base + t  # the new token's row
        knew = syn.normal((n, wl.hkv, wl.head_dim), g, DEV)
        vnew = syn.normal((n, wl.hkv, wl.head_dim), g, DEV)
        idx = torch.arange(n, device=DEV)
        kc[idx, :, pos.long()] = knew
        vc[idx, :, pos.long()] = vnew
        qt = syn.normal((n, wl.hq, wl.head_dim), g, DEV)
        seqlens = (pos + 1).to(torch.int32)
        outs = [flux.attn_decode(qt, kc, vc, seqlens, rt, layer, rp, ci, sa, ws)
                for rt, layer in ((route, layer_r), (checker, 0))]
        if t in checks:
            checks[t] = (qt.clone(), seqlens.clone(), [o.clone() for o in outs])
    torch.cuda.synchronize()
    say("varlen8 decode: checking steps " + ", ".join(str(t) for t in checks))
    kcf, vcf = f32(kc), f32(vc)
    for t, (qt, seqlens, outs) in checks.items():
        sl = seqlens.cpu().numpy()
        for (rt, layer), out in zip(((route, layer_r), (checker, 0)), outs):
            fa = rt.cpu().numpy()[:, layer].astype(bool)
            ref = oracle.attention_decode(f32(qt), kcf, vcf, sl, fa, m, B, heads=heads)
            assert_attn_close(f32(out)[:, heads], ref, f"decode step {t} layer {layer}")
