"""GPU decode over its work list: items sized by the keys each (sequence, kv
head) visits, so a long FA sequence beside short SA sequences is split finer
than they are.  Checked against the float64 oracle; the same sequence decoded
alone and inside a batch (different item splits) agrees; nothing is written
outside the workspace and the outputs; calls with more pairs than the plan
holds (one item per pair) are checked too.

Bar: attention within atol 2e-2 / rtol 1e-2 elementwise AND relative
Frobenius error <= 1e-2 against the oracle.
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
    return t.detach().float().cpu().numpy()


def say(msg):
    print(msg, flush=True)


def oracle_rows(q, kc, vc, seqlens, fa_per_seq, mask, B, seqs):
    """Oracle decode output of the listed sequences, each from only its own
    valid cache rows (downloaded one sequence at a time)."""
    out = []
    for b in seqs:
        n = int(seqlens[b])
        ref = oracle.attention_decode(f32(q[b:b + 1]), f32(kc[b:b + 1, :, :n]), f32(vc[b:b + 1, :, :n]),
                                      [n], bool(fa_per_seq[b]), mask, B)
        out.append(ref[0])
    return np.stack(out)


def test_long_fa_sequence_beside_short_sa_sequences():
    """A 65536-key FA sequence in one call with short SA sequences (and a
    second layer where a 40000-key sequence is FA too): Qwen3-4B-shaped heads."""
    lens = [65536, 2176, 3000, 129, 1, 7000, 40000, 2049]
    n, hq, hkv, d, B, s, w = len(lens), 32, 8, 128, 128, 1, 16
    max_len = max(lens)
    say(f"decode long FA beside short SA: lens {lens}")
    g = syn.generator(4242, DEV)
    q = syn.normal((n, hq, d), g, DEV)
    kc = syn.normal((n, hkv, max_len, d), g, DEV)
    vc = syn.normal((n, hkv, max_len, d), g, DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    sa = flux.SAParams(B, s, w)
    _, rp, ci = flux.build_block_mask(max_len, sa, dense=False)
    m = oracle.block_mask(oracle.num_blocks(max_len, B), s, w)
    routes = [[1, 0, 0, 0, 0, 0, 0, 0], [1, 0, 0, 0, 0, 0, 1, 0]]
    route = torch.tensor(routes, dtype=torch.uint8, device=DEV).t().contiguous()  # [n][2]
    for layer in (0, 1):
        out = flux.attn_decode(q, kc, vc, sl, route, layer, rp, ci, sa)
        again = flux.attn_decode(q, kc, vc, sl, route, layer, rp, ci, sa)
        torch.cuda.synchronize()
        assert torch.equal(out, again), "decode is not bitwise reproducible"
        ref = oracle_rows(q, kc, vc, lens, routes[layer], m, B, range(n))
        assert_attn_close(f32(out), ref, f"layer {layer}")


@pytest.mark.parametrize("fa", [1, 0])
def test_same_sequence_alone_and_in_a_batch(fa):
    """Sequence X decoded alone (8 pairs: about 78 items each) and as one of
    16 sequences (about 6 items each): both within tolerance of the oracle
    and of each other."""
    n, hq, hkv, d, B, s, w = 16, 32, 8, 128, 128, 1, 16
    lx, lo, slot = 20000, 30000, 5
    say(f"decode split invariance fa={fa}")
    g = syn.generator(5151, DEV)
    q = syn.normal((n, hq, d), g, DEV)
    kc = syn.normal((n, hkv, lo, d), g, DEV)
    vc = syn.normal((n, hkv, lo, d), g, DEV)
    lens = [lo] * n
    lens[slot] = lx
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    sa = flux.SAParams(B, s, w)
    _, rp, ci = flux.build_block_mask(lo, sa, dense=False)
    route = torch.full((n, 1), fa, dtype=torch.uint8, device=DEV)
    batch = flux.attn_decode(q, kc, vc, sl, route, 0, rp, ci, sa)
    qx = q[slot:slot + 1].contiguous()
    kx = kc[slot:slot + 1, :, :lx].contiguous()
    vx = vc[slot:slot + 1, :, :lx].contiguous()
    _, rpx, cix = flux.build_block_mask(lx, sa, dense=False)
    alone = flux.attn_decode(qx, kx, vx, sl[slot:slot + 1].contiguous(), route[:1].contiguous(), 0, rpx,
                             cix, sa)
    torch.cuda.synchronize()
    assert flux.decode_workspace_size(1, hq, hkv, d, lx) > 0
    m = oracle.block_mask(oracle.num_blocks(lo, B), s, w)
    ref = oracle_rows(q, kc, vc, lens, [fa] * n, m, B, [slot])[0]
    assert_attn_close(f32(batch)[slot], ref, "in a batch of 16")
    assert_attn_close(f32(alone)[0], ref, "alone")
    assert_attn_close(f32(alone)[0], f32(batch)[slot], "alone vs batch")


def test_no_writes_outside_workspace_and_outputs():
    """NaN guard bands before and after the workspace and the output stay
    bit for bit untouched; the output between them matches the oracle."""
    lens = [9000, 1, 300, 4097]
    n, hq, hkv, d, B, s, w = len(lens), 32, 8, 128, 128, 1, 8
    max_len = max(lens)
    say("decode guard bands")
    g = syn.generator(6161, DEV)
    q = syn.normal((n, hq, d), g, DEV)
    kc = syn.normal((n, hkv, max_len, d), g, DEV)
    vc = syn.normal((n, hkv, max_len, d), g, DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    sa = flux.SAParams(B, s, w)
    _, rp, ci = flux.build_block_mask(max_len, sa, dense=False)
    m = oracle.block_mask(oracle.num_blocks(max_len, B), s, w)
    need = flux.decode_workspace_size(n, hq, hkv, d, max_len)
    assert need > 0
    G = 1 << 16  # guard bytes on each side (keeps the workspace 16-byte aligned)
    ws_full = torch.full((need + 2 * G,), 0xFF, dtype=torch.uint8, device=DEV)
    ws = ws_full[G:G + need]
    ne = n * hq * d
    Ge = 4096  # guard elements on each side of the output
    out_full = torch.full((ne + 2 * Ge,), float("nan"), dtype=torch.bfloat16, device=DEV)
    out = out_full[Ge:Ge + ne].view(n, hq, d)
    guard_ws = ws_full.clone()
    guard_out = out_full.clone()
    route = torch.tensor([[1, 0]] * n, dtype=torch.uint8, device=DEV)
    for layer in (0, 1):
        flux.attn_decode(q, kc, vc, sl, route, layer, rp, ci, sa, workspace=ws, out=out)
        torch.cuda.synchronize()
        assert torch.equal(ws_full[:G], guard_ws[:G]) and torch.equal(ws_full[G + need:], guard_ws[G + need:])
        ob = out_full.view(torch.int16)
        gb = guard_out.view(torch.int16)
        assert torch.equal(ob[:Ge], gb[:Ge]) and torch.equal(ob[Ge + ne:], gb[Ge + ne:])
        ref = oracle_rows(q, kc, vc, lens, [layer == 0] * n, m, B, range(n))
        assert_attn_close(f32(out), ref, f"guarded layer {layer}")


def test_more_pairs_than_the_plan_holds():
    """1040 (sequence, kv head) pairs: one item per pair, mixed routes."""
    n, hq, hkv, d, B, s, w = 130, 16, 8, 64, 64, 1, 3
    gen = torch.Generator().manual_seed(7171)
    lens = [int(x) for x in torch.randint(1, 601, (n,), generator=gen)]
    fa = [int(x) for x in torch.randint(0, 2, (n,), generator=gen)]
    max_len = 600
    say("decode one item per pair (1040 pairs)")
    assert flux.decode_workspace_size(n, hq, hkv, d, max_len) == 0
    g = syn.generator(7272, DEV)
    q = syn.normal((n, hq, d), g, DEV)
    kc = syn.normal((n, hkv, max_len, d), g, DEV)
    vc = syn.normal((n, hkv, max_len, d), g, DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    sa = flux.SAParams(B, s, w)
    _, rp, ci = flux.build_block_mask(max_len, sa, dense=False)
    m = oracle.block_mask(oracle.num_blocks(max_len, B), s, w)
    route = torch.tensor(fa, dtype=torch.uint8, device=DEV)[:, None].contiguous()
    out = flux.attn_decode(q, kc, vc, sl, route, 0, rp, ci, sa)
    torch.cuda.synchronize()
    ref = oracle.attention_decode(f32(q), f32(kc), f32(vc), lens, fa, m, B)
    assert_attn_close(f32(out), ref, "1040 pairs")
