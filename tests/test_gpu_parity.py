"""GPU parity: libflux kernels (through the C ABI binding) against the float64
oracle on the same seeded inputs.

Bar: route bits and block masks bit-exact; attention within atol 2e-2 /
rtol 1e-2 elementwise AND relative Frobenius error <= 1e-2.  Small cases are
checked in full; the 32K prefill and decode shapes on sampled rows/sequences
(all heads, block boundaries, first/last rows).
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
else:  # collected on CPU only to be deselected
    flux = None

DEV = "cuda"


def f32(t):
    """Exact float32 copy on the host (bf16 widens exactly)."""
    return t.detach().float().cpu().numpy()


def say(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- mask

@pytest.mark.parametrize("seqlen,B,s,w", [
    (512, 64, 1, 2), (32768, 128, 1, 16), (131072, 128, 1, 32), (1000, 128, 3, 2),
    (581, 64, 0, 3), (65536, 64, 2, 5), (64, 64, 1, 1), (300, 128, 0, 8)])
def test_mask_bit_exact(seqlen, B, s, w):
    say(f"mask seqlen={seqlen} B={B} s={s} w={w}")
    sa = flux.SAParams(B, s, w)
    m, rp, ci = flux.build_block_mask(seqlen, sa)
    torch.cuda.synchronize()
    nb = oracle.num_blocks(seqlen, B)
    ref = oracle.block_mask(nb, s, w)
    rp_ref, ci_ref = oracle.mask_to_csr(ref)
    np.testing.assert_array_equal(m.cpu().numpy(), ref)
    np.testing.assert_array_equal(rp.cpu().numpy(), rp_ref)
    np.testing.assert_array_equal(ci.cpu().numpy(), ci_ref)


# ---------------------------------------------------------------- router

def check_route(route_gpu, z_gpu, route_ref, z_ref, w2, h_bound):
    """Bit-exact route wherever the oracle logit clears a forward error bound."""
    z_gpu = z_gpu.astype(np.float64)
    bound = 1e-4 * h_bound + 1e-6
    assert np.all(np.abs(z_gpu - z_ref) <= bound), np.abs(z_gpu - z_ref).max()
    decided = np.abs(z_ref) > bound
    np.testing.assert_array_equal(route_gpu[decided], route_ref[decided])
    return int((~decided).sum())


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_router_tiny_and_varlen(dtype):
    say(f"router dtype={dtype}")
    cases = [((512,), 256, 64, 2), ((150, 200, 201, 3000, 1, 777, 99, 4096), 4096, 256, 32),
             ((131072, 333), 264, 256, 36)]
    for lens, D, H1, L in cases:
        g = syn.generator(7 + D, DEV)
        T = sum(lens)
        hidden = syn.normal((T, D), g, DEV, dtype)
        w1, b1, w2, b2 = syn.router_weights(D, H1, L, 11 + D)
        cu = syn.cu_seqlens(lens, DEV)
        logits = torch.empty((len(lens), L), dtype=torch.float32, device=DEV)
        route, _ = flux.route(hidden, cu, w1.to(DEV), b1.to(DEV), w2.to(DEV), b2.to(DEV),
                              logits_out=logits)
        route2, _ = flux.route(hidden, cu, w1.to(DEV), b1.to(DEV), w2.to(DEV), b2.to(DEV),
                               logits_out=(logits2 := torch.empty_like(logits)))
        torch.cuda.synchronize()
        assert torch.equal(logits, logits2) and torch.equal(route, route2)  # bitwise reproducible
        r_ref, z_ref = oracle.route_requests(f32(hidden), np.cumsum([0] + list(lens)), w1.numpy(),
                                             b1.numpy(), w2.numpy(), b2.numpy())
        # |W2| |h| + |b2| scale of each logit
        hs = [np.maximum(w1.numpy().astype(np.float64) @ oracle.pool_mean(f32(hidden)[a:b]) + b1.numpy(), 0)
              for a, b in zip(np.cumsum([0] + list(lens))[:-1], np.cumsum(lens))]
        scale = np.stack([np.abs(w2.numpy()) @ np.abs(h) + np.abs(b2.numpy()) for h in hs])
        ties = check_route(route.cpu().numpy(), logits.cpu().numpy(), r_ref, z_ref, w2, scale)
        assert ties == 0


def test_router_zero_weights_tie_to_fa():
    say("router zero weights")
    hidden = torch.ones((300, 64), device=DEV)
    z = torch.zeros
    route, _ = flux.route(hidden, syn.cu_seqlens([300], DEV), z((8, 64), device=DEV), z(8, device=DEV),
                          z((3, 8), device=DEV), z(3, device=DEV))
    torch.cuda.synchronize()
    assert route.cpu().tolist() == [[1, 1, 1]]


# ---------------------------------------------------------------- prefill

def run_prefill_case(lens, hq, hkv, d, B, s, w, route_rows, seed, dtype_in=torch.bfloat16):
    g = syn.generator(seed, DEV)
    T = sum(lens)
    q = syn.normal((T, hq, d), g, DEV, dtype_in).to(torch.bfloat16)
    k = syn.normal((T, hkv, d), g, DEV, dtype_in).to(torch.bfloat16)
    v = syn.normal((T, hkv, d), g, DEV, dtype_in).to(torch.bfloat16)
    cu = syn.cu_seqlens(lens, DEV)
    sa = flux.SAParams(B, s, w)
    _, rp, ci = flux.build_block_mask(max(lens), sa, dense=False)
    route = torch.tensor(route_rows, dtype=torch.uint8, device=DEV)
    return q, k, v, cu, sa, rp, ci, route


@pytest.mark.parametrize("layer_route", [[1, 0], [0, 1]])
def test_prefill_tiny_full(layer_route):
    """Tiny routed stack (512 tokens, 2 layers, 4/2 heads, d 64, B 64, 1 sink + 2 local)."""
    say(f"prefill tiny route={layer_route}")
    wl = syn.TINY
    q, k, v, cu, sa, rp, ci, route = run_prefill_case(
        list(wl.seqlens), wl.hq, wl.hkv, wl.head_dim, wl.block_size, wl.sink_blocks,
        wl.local_blocks, [layer_route], wl.seed, torch.float32)
    m = oracle.block_mask(oracle.num_blocks(512, 64), 1, 2)
    for layer in range(2):
        out = flux.attn_prefill(q, k, v, cu, 512, route, layer, rp, ci, sa)
        torch.cuda.synchronize()
        ref = oracle.attention_prefill(f32(q), f32(k), f32(v), bool(layer_route[layer]), m, 64)
        assert_attn_close(f32(out), ref, f"tiny layer {layer}")


VARLEN_CASES = [
    # lens, hq, hkv, d, B, s, w
    ((1, 63, 64, 65, 200, 513, 1000), 4, 2, 128, 128, 1, 2),
    ((1, 63, 64, 65, 200, 513, 1000), 4, 2, 64, 64, 1, 3),
    ((700, 129, 1500), 8, 1, 128, 64, 0, 1),
    ((300, 2049), 16, 16, 64, 128, 2, 3),
    ((4100,), 32, 8, 128, 128, 1, 16),
]


@pytest.mark.parametrize("case", VARLEN_CASES)
def test_prefill_varlen_full(case):
    lens, hq, hkv, d, B, s, w = case
    say(f"prefill varlen lens={lens} hq={hq} hkv={hkv} d={d} B={B} s={s} w={w}")
    rng = np.random.default_rng(sum(lens))
    route_rows = [[int(x) for x in rng.integers(0, 2, size=2)] for _ in lens]
    route_rows[0] = [1, 0]
    q, k, v, cu, sa, rp, ci, route = run_prefill_case(list(lens), hq, hkv, d, B, s, w, route_rows,
                                                      100 + d + B)
    m = oracle.block_mask(oracle.num_blocks(max(lens), B), s, w)
    cu_h = np.cumsum([0] + list(lens))
    qf, kf, vf = f32(q), f32(k), f32(v)
    for layer in range(2):
        out = flux.attn_prefill(q, k, v, cu, max(lens), route, layer, rp, ci, sa)
        torch.cuda.synchronize()
        refs = oracle.attention_prefill_varlen(qf, kf, vf, cu_h, np.array(route_rows), layer, m, B)
        of = f32(out)
        for r, (a, b) in enumerate(zip(cu_h[:-1], cu_h[1:])):
            assert_attn_close(of[a:b], refs[r], f"req {r} layer {layer}")


def sampled_rows(S, B, n_random, seed):
    rows = {0, 1, B - 1, B, B + 1, S // 2, S - B, S - 1, 2047, 2048, 2049}
    rows |= set(int(x) for x in np.random.default_rng(seed).integers(0, S, size=n_random))
    return np.array(sorted(r for r in rows if 0 <= r < S))


def test_prefill_32k_sampled():
    """Qwen3-4B-shaped layer at 32768 tokens: FA and SA on identical inputs."""
    wl = syn.PREFILL32K
    S = wl.seqlens[0]
    say("prefill 32k FA+SA")
    q, k, v, cu, sa, rp, ci, route = run_prefill_case(
        [S], wl.hq, wl.hkv, wl.head_dim, wl.block_size, wl.sink_blocks, wl.local_blocks,
        [[1, 0]], wl.seed)
    m = oracle.block_mask(oracle.num_blocks(S, wl.block_size), wl.sink_blocks, wl.local_blocks)
    rows = sampled_rows(S, wl.block_size, 12, 5)
    qf, kf, vf = f32(q), f32(k), f32(v)
    for layer in (0, 1):
        out = flux.attn_prefill(q, k, v, cu, S, route, layer, rp, ci, sa)
        torch.cuda.synchronize()
        ref = oracle.attention_prefill(qf, kf, vf, layer == 0, m, wl.block_size, rows=rows)
        assert_attn_close(f32(out)[rows], ref, f"32k layer {layer}")
        out2 = flux.attn_prefill(q, k, v, cu, S, route, layer, rp, ci, sa)
        torch.cuda.synchronize()
        assert torch.equal(out, out2), "prefill is not bitwise reproducible"


def test_prefill_causality_on_gpu():
    say("prefill causality")
    lens = [777]
    for fa in (1, 0):
        q, k, v, cu, sa, rp, ci, route = run_prefill_case(lens, 4, 2, 128, 128, 1, 2, [[fa]], 31)
        base = flux.attn_prefill(q, k, v, cu, 777, route, 0, rp, ci, sa)
        p = 300
        k2, v2 = k.clone(), v.clone()
        k2[p + 1:] = -k2[p + 1:] * 3
        v2[p + 1:] += 5
        pert = flux.attn_prefill(q, k2, v2, cu, 777, route, 0, rp, ci, sa)
        torch.cuda.synchronize()
        assert torch.equal(base[:p + 1], pert[:p + 1])
        assert not torch.equal(base[p + 1:], pert[p + 1:])


# ---------------------------------------------------------------- decode

def make_decode(n_seq, max_len, seqlens, hq, hkv, d, seed):
    g = syn.generator(seed, DEV)
    q = syn.normal((n_seq, hq, d), g, DEV)
    kc = syn.normal((n_seq, hkv, max_len, d), g, DEV)
    vc = syn.normal((n_seq, hkv, max_len, d), g, DEV)
    sl = torch.tensor(seqlens, dtype=torch.int32, device=DEV)
    return q, kc, vc, sl


DECODE_CASES = [
    # n_seq, max_len, seqlens, hq, hkv, d, B, s, w
    (5, 1100, [1, 64, 65, 700, 1100], 4, 2, 128, 128, 1, 2),
    (5, 1100, [1, 64, 65, 700, 1100], 8, 8, 64, 64, 1, 3),
    (3, 5000, [5000, 2049, 4097], 32, 8, 128, 128, 1, 16),
    (2, 300, [300, 37], 16, 1, 128, 64, 0, 1),
]


@pytest.mark.parametrize("case", DECODE_CASES)
def test_decode_full(case):
    n_seq, max_len, seqlens, hq, hkv, d, B, s, w = case
    say(f"decode {case}")
    q, kc, vc, sl = make_decode(n_seq, max_len, seqlens, hq, hkv, d, 77 + d)
    sa = flux.SAParams(B, s, w)
    _, rp, ci = flux.build_block_mask(max_len, sa, dense=False)
    m = oracle.block_mask(oracle.num_blocks(max_len, B), s, w)
    route = torch.tensor([[1, 0]] * n_seq, dtype=torch.uint8, device=DEV)
    qf, kf, vf = f32(q), f32(kc), f32(vc)
    for layer in (0, 1):
        out = flux.attn_decode(q, kc, vc, sl, route, layer, rp, ci, sa)
        torch.cuda.synchronize()
        ref = oracle.attention_decode(qf, kf, vf, seqlens, layer == 0, m, B)
        assert_attn_close(f32(out), ref, f"decode layer {layer}")


def test_decode_32k_sampled():
    """Qwen3-4B-shaped decode: 16 sequences x 32768 cached tokens, one FA and one SA layer."""
    wl = syn.DECODE32K
    n_seq, L = len(wl.seqlens), wl.seqlens[0]
    say("decode 32k")
    q, kc, vc, sl = make_decode(n_seq, L, list(wl.seqlens), wl.hq, wl.hkv, wl.head_dim, wl.seed)
    sa = flux.SAParams(wl.block_size, wl.sink_blocks, wl.local_blocks)
    _, rp, ci = flux.build_block_mask(L, sa, dense=False)
    m = oracle.block_mask(oracle.num_blocks(L, wl.block_size), wl.sink_blocks, wl.local_blocks)
    route = torch.tensor([[1, 0]] * n_seq, dtype=torch.uint8, device=DEV)
    seqs = [0, 7, 15]
    qf = f32(q[seqs])
    kf, vf = f32(kc[seqs]), f32(vc[seqs])
    for layer in (0, 1):
        out = flux.attn_decode(q, kc, vc, sl, route, layer, rp, ci, sa)
        out2 = flux.attn_decode(q, kc, vc, sl, route, layer, rp, ci, sa)
        torch.cuda.synchronize()
        assert torch.equal(out, out2), "decode is not bitwise reproducible"
        ref = oracle.attention_decode(qf, kf, vf, [L] * len(seqs), layer == 0, m, wl.block_size)
        assert_attn_close(f32(out)[seqs], ref, f"decode32k layer {layer}")


def test_decode_workspace_reuse():
    """One workspace, sized for the largest call, serves calls of different
    shapes one after another; results equal those of a fresh workspace."""
    say("decode workspace reuse")
    big = (4, 6000, [6000, 4097, 1, 5000], 32, 8, 128)
    small = (2, 3000, [3000, 1500], 16, 4, 64)
    ws = flux.decode_workspace(4, 32, 8, 128, 6000, DEV)
    for case in (big, small, big):
        n_seq, max_len, seqlens, hq, hkv, d = case
        q, kc, vc, sl = make_decode(n_seq, max_len, seqlens, hq, hkv, d, 91 + d)
        sa = flux.SAParams(128, 1, 4)
        _, rp, ci = flux.build_block_mask(max_len, sa, dense=False)
        route = torch.tensor([[1, 0]] * n_seq, dtype=torch.uint8, device=DEV)
        for layer in (0, 1):
            assert flux.decode_workspace_size(n_seq, hq, hkv, d, max_len) <= ws.numel()
            shared = flux.attn_decode(q, kc, vc, sl, route, layer, rp, ci, sa, workspace=ws)
            fresh = flux.attn_decode(q, kc, vc, sl, route, layer, rp, ci, sa)
            torch.cuda.synchronize()
            assert torch.equal(shared, fresh)


def test_decode_matches_prefill_last_row():
    say("decode vs prefill last row")
    S, hq, hkv, d = 1500, 8, 2, 128
    for fa in (1, 0):
        q, k, v, cu, sa, rp, ci, route = run_prefill_case([S], hq, hkv, d, 128, 1, 3, [[fa]], 55)
        pre = flux.attn_prefill(q, k, v, cu, S, route, 0, rp, ci, sa)
        kc = k.permute(1, 0, 2).contiguous()[None]
        vc = v.permute(1, 0, 2).contiguous()[None]
        for n in (S, 1000, 129):
            dec = flux.attn_decode(q[n - 1][None].contiguous(), kc, vc,
                                   torch.tensor([n], dtype=torch.int32, device=DEV), route, 0, rp, ci, sa)
            if n == S:
                torch.cuda.synchronize()
                assert_attn_close(f32(dec)[0], f32(pre)[S - 1], f"fa={fa} n={n}")
            else:
                # a prefix of the same data: compare with the oracle's row n-1
                torch.cuda.synchronize()
                m = oracle.block_mask(oracle.num_blocks(S, 128), 1, 3)
                ref = oracle.attention_prefill(f32(q)[:n], f32(k)[:n], f32(v)[:n], bool(fa), m, 128,
                                               rows=[n - 1])
                assert_attn_close(f32(dec)[0], ref[0], f"fa={fa} n={n}")
