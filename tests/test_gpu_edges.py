"""Edge cases through the C ABI binding, against the float64 oracle: an empty
request inside a packed batch, a zero decode length, the largest supported
GQA group, inputs whose scores span a huge range (every row moves its running
max many times and the overflow check of the exponentials fires), and
softmax scales other than 1/sqrt(d)."""

import math

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


def check_varlen(q, k, v, cu_h, lens, route_rows, layer, out, m, B, scale=None, what=""):
    qf, kf, vf, of = f32(q), f32(k), f32(v), f32(out)
    refs = oracle.attention_prefill_varlen(qf, kf, vf, cu_h, np.array(route_rows), layer, m, B, scale)
    for r, (a, b) in enumerate(zip(cu_h[:-1], cu_h[1:])):
        if b > a:
            assert_attn_close(of[a:b], refs[r], f"{what} req {r} layer {layer}")


def test_empty_request_in_batch():
    """A zero-length request contributes no rows and leaves the others alone;
    the router pools nothing for it (a zero vector, as documented)."""
    say("empty request")
    lens, hq, hkv, d, B = [300, 0, 129, 0], 8, 2, 128, 64
    route_rows = [[1, 0]] * len(lens)
    q, k, v, cu, sa, rp, ci, route = run_prefill_case(lens, hq, hkv, d, B, 1, 2, route_rows, 77)
    m = oracle.block_mask(oracle.num_blocks(max(lens), B), 1, 2)
    cu_h = np.cumsum([0] + lens)
    for layer in (0, 1):
        out = torch.full_like(q, float("nan"))
        flux.attn_prefill(q, k, v, cu, max(lens), route, layer, rp, ci, sa, out=out)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any()  # every row of the batch belongs to a non-empty request
        check_varlen(q, k, v, cu_h, lens, route_rows, layer, out, m, B, what="empty-in-batch")
    # router: requests of length 0 pool a zero vector
    D, H1, L = 64, 32, 5
    g = syn.generator(78, DEV)
    hidden = syn.normal((sum(lens), D), g, DEV, torch.float32)
    w1, b1, w2, b2 = syn.router_weights(D, H1, L, 79, std=0.3)
    logits = torch.empty((len(lens), L), dtype=torch.float32, device=DEV)
    rt, _ = flux.route(hidden, cu, w1.to(DEV), b1.to(DEV), w2.to(DEV), b2.to(DEV), logits_out=logits)
    torch.cuda.synchronize()
    z0 = oracle.router_mlp(np.zeros(D), w1.numpy(), b1.numpy(), w2.numpy(), b2.numpy())
    for r in (1, 3):
        np.testing.assert_allclose(logits[r].cpu().numpy(), z0, rtol=1e-5, atol=1e-6)
        decided = np.abs(z0) > 1e-4
        np.testing.assert_array_equal(rt[r].cpu().numpy()[decided], oracle.threshold_route(z0)[decided])


def test_decode_zero_length_is_one():
    say("decode seqlen 0")
    q, kc, vc, sl = make_decode(3, 400, [0, 1, 400], 8, 2, 128, 81)
    sa = flux.SAParams(128, 1, 2)
    _, rp, ci = flux.build_block_mask(400, sa, dense=False)
    route = torch.tensor([[1, 0]] * 3, dtype=torch.uint8, device=DEV)
    for layer in (0, 1):
        a = flux.attn_decode(q, kc, vc, sl, route, layer, rp, ci, sa)
        b = flux.attn_decode(q, kc, vc, torch.tensor([1, 1, 400], dtype=torch.int32, device=DEV), route,
                             layer, rp, ci, sa)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0])  # seqlens 0 reads as 1: the query sees key 0 only
        assert_attn_close(f32(a)[0], f32(vc)[0, :, 0].repeat(4, 0), "decode len 0 = v0")


def test_largest_gqa_group_prefill():
    """16 query heads per KV head, the largest group the kernels take."""
    say("gqa 16")
    lens, hq, hkv, d, B = [700, 257], 16, 1, 128, 128
    route_rows = [[1, 0], [0, 1]]
    q, k, v, cu, sa, rp, ci, route = run_prefill_case(lens, hq, hkv, d, B, 1, 2, route_rows, 83)
    m = oracle.block_mask(oracle.num_blocks(max(lens), B), 1, 2)
    cu_h = np.cumsum([0] + lens)
    for layer in (0, 1):
        out = flux.attn_prefill(q, k, v, cu, max(lens), route, layer, rp, ci, sa)
        torch.cuda.synchronize()
        check_varlen(q, k, v, cu_h, lens, route_rows, layer, out, m, B, what="gqa16")


@pytest.mark.parametrize("gain", [6.0, 14.0])
def test_wide_score_range(gain):
    """q and k scaled so that scores span hundreds of log2 units: rows move
    their running max again and again and the exponentials overflow the
    check, exercising the re-max path against the oracle."""
    say(f"wide scores gain={gain}")
    lens, hq, hkv, d, B = [1000, 333], 8, 2, 128, 64
    route_rows = [[1, 0], [0, 1]]
    q, k, v, cu, sa, rp, ci, route = run_prefill_case(lens, hq, hkv, d, B, 1, 3, route_rows, 85)
    ramp = torch.linspace(0.2, 1.0, q.shape[0], device=DEV)[:, None, None]
    q = (q.float() * gain * ramp).to(torch.bfloat16)
    k = (k.float() * gain * ramp[:, :, :]).to(torch.bfloat16)
    m = oracle.block_mask(oracle.num_blocks(max(lens), B), 1, 3)
    cu_h = np.cumsum([0] + lens)
    for layer in (0, 1):
        out = flux.attn_prefill(q, k, v, cu, max(lens), route, layer, rp, ci, sa)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        check_varlen(q, k, v, cu_h, lens, route_rows, layer, out, m, B, what=f"gain {gain}")
    # decode on the same kind of data
    qd, kc, vc, sl = make_decode(2, 1500, [1500, 700], 8, 2, 128, 86)
    qd = (qd.float() * gain).to(torch.bfloat16)
    kc = (kc.float() * gain).to(torch.bfloat16)
    sa2 = flux.SAParams(128, 1, 3)
    _, rp2, ci2 = flux.build_block_mask(1500, sa2, dense=False)
    m2 = oracle.block_mask(oracle.num_blocks(1500, 128), 1, 3)
    rt = torch.tensor([[1, 0]] * 2, dtype=torch.uint8, device=DEV)
    for layer in (0, 1):
        out = flux.attn_decode(qd, kc, vc, sl, rt, layer, rp2, ci2, sa2)
        torch.cuda.synchronize()
        ref = oracle.attention_decode(f32(qd), f32(kc), f32(vc), [1500, 700], layer == 0, m2, 128)
        assert_attn_close(f32(out), ref, f"decode gain {gain} layer {layer}")


@pytest.mark.parametrize("scale", [0.02, 0.5])
def test_softmax_scales(scale):
    say(f"scale {scale}")
    lens, hq, hkv, d, B = [600, 65], 4, 2, 64, 64
    route_rows = [[1, 0], [0, 1]]
    q, k, v, cu, sa, rp, ci, route = run_prefill_case(lens, hq, hkv, d, B, 0, 2, route_rows, 87)
    m = oracle.block_mask(oracle.num_blocks(max(lens), B), 0, 2)
    cu_h = np.cumsum([0] + lens)
    for layer in (0, 1):
        out = flux.attn_prefill(q, k, v, cu, max(lens), route, layer, rp, ci, sa, softmax_scale=scale)
        torch.cuda.synchronize()
        check_varlen(q, k, v, cu_h, lens, route_rows, layer, out, m, B, scale, what=f"scale {scale}")
    qd, kc, vc, sl = make_decode(2, 600, [600, 65], 4, 2, 64, 88)
    rt = torch.tensor([[1, 0]] * 2, dtype=torch.uint8, device=DEV)
    for layer in (0, 1):
        out = flux.attn_decode(qd, kc, vc, sl, rt, layer, rp, ci, sa, softmax_scale=scale)
        torch.cuda.synchronize()
        ref = oracle.attention_decode(f32(qd), f32(kc), f32(vc), [600, 65], layer == 0, m, B, scale)
        assert_attn_close(f32(out), ref, f"decode scale {scale} layer {layer}")


def test_request_longer_than_max_seqlen_is_cut():
    """A request longer than max_seqlen is cut to max_seqlen rows: those rows
    are exact (a causal row never reads keys past itself) and the rows past
    the cut are left untouched."""
    say("request longer than max_seqlen")
    lens, hq, hkv, d, B, cut = [300], 4, 2, 128, 64, 200
    route_rows = [[1, 0]]
    q, k, v, cu, sa, rp, ci, route = run_prefill_case(lens, hq, hkv, d, B, 1, 2, route_rows, 91)
    m = oracle.block_mask(oracle.num_blocks(max(lens), B), 1, 2)
    for layer in (0, 1):
        out = torch.full_like(q, float("nan"))
        flux.attn_prefill(q, k, v, cu, cut, route, layer, rp, ci, sa, out=out)
        torch.cuda.synchronize()
        assert torch.isnan(out[cut:]).all()
        ref = oracle.attention_prefill(f32(q)[:cut], f32(k)[:cut], f32(v)[:cut], layer == 0, m, B)
        assert_attn_close(f32(out)[:cut], ref, f"cut layer {layer}")


@pytest.mark.parametrize("hq,hkv", [(6, 2), (5, 1), (7, 7)])
def test_odd_gqa_groups(hq, hkv):
    """GQA groups of 3, 5 and 1 query heads per kv head: prefill (both layer
    types, ragged lengths) and decode against the oracle."""
    say(f"odd GQA group hq={hq} hkv={hkv}")
    lens, d, B = [333, 70, 129], 128, 64
    route_rows = [[1, 0], [0, 1], [1, 1]]
    q, k, v, cu, sa, rp, ci, route = run_prefill_case(lens, hq, hkv, d, B, 1, 2, route_rows, 95 + hq)
    m = oracle.block_mask(oracle.num_blocks(max(lens), B), 1, 2)
    cu_h = np.cumsum([0] + lens)
    for layer in (0, 1):
        out = flux.attn_prefill(q, k, v, cu, max(lens), route, layer, rp, ci, sa)
        torch.cuda.synchronize()
        check_varlen(q, k, v, cu_h, lens, route_rows, layer, out, m, B, what=f"group {hq // hkv}")
    seqlens = [333, 64, 1]
    qd, kc, vc, sl = make_decode(3, 333, seqlens, hq, hkv, d, 96 + hq)
    _, rp2, ci2 = flux.build_block_mask(333, sa, dense=False)
    rt = torch.tensor(route_rows, dtype=torch.uint8, device=DEV)
    for layer in (0, 1):
        out = flux.attn_decode(qd, kc, vc, sl, rt, layer, rp2, ci2, sa)
        torch.cuda.synchronize()
        for i, n in enumerate(seqlens):
            ref = oracle.attention_decode(f32(qd[i:i + 1]), f32(kc[i:i + 1]), f32(vc[i:i + 1]), [n],
                                          route_rows[i][layer] == 1, m, B)
            assert_attn_close(f32(out[i:i + 1]), ref, f"decode group {hq // hkv} seq {i} layer {layer}")


def test_sa_rows_without_their_diagonal_block():
    """SA prefill on a hand-made mask whose odd rows leave out their diagonal
    block: those rows are visited in their own order (the diagonal-first
    order applies only to rows that end with the diagonal block), even rows
    start with it; every row against the oracle."""
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
    say("SA prefill, rows without their diagonal block")
    q, k, v, cu, sa, _, _, route = run_prefill_case([S], hq, hkv, d, B, 1, 1, [[0]], 1400)
    rp = torch.tensor(rp_h, dtype=torch.int32, device=DEV)
    ci = torch.tensor(ci_h, dtype=torch.int32, device=DEV)
    out = flux.attn_prefill(q, k, v, cu, S, route, 0, rp, ci, sa)
    torch.cuda.synchronize()
    ref = oracle.attention_prefill(f32(q), f32(k), f32(v), False, m, B)
    assert_attn_close(f32(out), ref, "SA, rows without their diagonal block")
