"""GPU prefill with the balancing workspace.  The tail of every XCD's work
list is handed out at run time, so the workgroup that computes a query block
changes, but nothing else does: outputs must equal the fixed-order launch bit
for bit (the same tiles in the same order per query block), every query
block must be computed, and the workspace must be zero again after every call
(the launch that follows the kernel clears it), so that one workspace serves
calls of different shapes in a row.  Cases: a 32K prompt (FA and SA layers
through the queues), a prompt shorter than max_seqlen (queue items past its
end), the soft pass, 64-wide heads and 64-row blocks, packed batches with
mixed routes and with empty and one-token requests, shapes below one round of workgroups or with a work count that
is not a multiple of 8 (fixed order with a workspace passed), the binding's
per-stream workspace, and a balanced launch replayed from a HIP graph.  The
oracle comparisons of every other prefill test run with the workspace too
(the binding's default)."""

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


def say(msg):
    print(msg, flush=True)


def bits(t):
    return t.view(torch.int16)


def new_workspace():
    return torch.zeros(flux._lib.FLUX_PREFILL_WORKSPACE_BYTES // 4, dtype=torch.int32, device=DEV)


def inputs(lens, hq, hkv, d, B, w, seed):
    T, S = sum(lens), max(lens)
    g = syn.generator(seed, DEV)
    q = syn.normal((T, hq, d), g, DEV)
    k = syn.normal((T, hkv, d), g, DEV)
    v = syn.normal((T, hkv, d), g, DEV)
    sa = flux.SAParams(B, 1, w)
    _, rp, ci = flux.build_block_mask(S, sa, dense=False)
    return q, k, v, syn.cu_seqlens(lens, DEV), sa, rp, ci


def check_pair(q, k, v, cu, max_len, route, layer, rp, ci, sa, ws, what):
    """Fixed order vs balanced with ws, outputs NaN-filled before each call."""
    fixed = torch.full_like(q, float("nan"))
    flux.attn_prefill(q, k, v, cu, max_len, route, layer, rp, ci, sa, out=fixed, workspace=None)
    bal = torch.full_like(q, float("nan"))
    flux.attn_prefill(q, k, v, cu, max_len, route, layer, rp, ci, sa, out=bal, workspace=ws)
    torch.cuda.synchronize()
    assert not torch.isnan(bal).any(), f"{what}: a query block was never computed"
    assert torch.equal(bits(bal), bits(fixed)), f"{what}: differs from the fixed order"
    assert not ws.any(), f"{what}: the workspace is not zero after the call"
    return bal


def test_single_prompt_32k_fa_and_sa():
    S, hq, hkv, d = 32768, 32, 8, 128
    say("balanced prefill 32K FA/SA")
    q, k, v, cu, sa, rp, ci = inputs([S], hq, hkv, d, 128, 16, 8101)
    route = torch.tensor([[1, 0]], dtype=torch.uint8, device=DEV)
    ws = new_workspace()
    for rep in range(3):
        for layer in (0, 1):
            check_pair(q, k, v, cu, S, route, layer, rp, ci, sa, ws, f"32K layer {layer} rep {rep}")


def test_prompt_shorter_than_max_seqlen():
    """Queue items past the prompt's end are taken and end at once."""
    S, max_len, hq, hkv, d = 5000, 8192, 32, 8, 128
    say("balanced prefill, prompt of 5000 under max_seqlen 8192")
    q, k, v, cu, sa, rp, ci = inputs([S], hq, hkv, d, 128, 8, 8202)
    _, rp, ci = flux.build_block_mask(max_len, sa, dense=False)
    route = torch.tensor([[1, 0]], dtype=torch.uint8, device=DEV)
    ws = new_workspace()
    for layer in (0, 1):
        check_pair(q, k, v, cu, max_len, route, layer, rp, ci, sa, ws, f"short prompt layer {layer}")
    # the balanced FA result against the oracle on rows across the prompt
    out = flux.attn_prefill(q, k, v, cu, max_len, route, 0, rp, ci, sa, workspace=ws).float().cpu().numpy()
    rows = sorted(set(range(0, S, 157)) | {S - 1})
    ref = oracle.attention_prefill(q.float().cpu().numpy(), k.float().cpu().numpy(), v.float().cpu().numpy(),
                                   True, rows=rows)
    assert_attn_close(out[rows], ref, "short prompt FA vs oracle")
    assert not ws.any()


def test_soft_pass():
    S, hq, hkv, d = 8192, 32, 8, 128
    say("balanced soft-routed prefill")
    q, k, v, cu, sa, rp, ci = inputs([S], hq, hkv, d, 128, 4, 8303)
    r = torch.tensor([[0.3]], dtype=torch.float32, device=DEV)
    ws = new_workspace()
    fixed = flux.attn_prefill_soft(q, k, v, cu, S, r, 0, rp, ci, sa, workspace=None)
    bal = flux.attn_prefill_soft(q, k, v, cu, S, r, 0, rp, ci, sa, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(bits(bal), bits(fixed))
    assert not ws.any()


@pytest.mark.parametrize("shape", [
    # (lens, hq, hkv, d, B): balanced with 64-wide heads and 64-row blocks;
    # below one round of workgroups, or 131 blocks x 20 heads (not a multiple
    # of 8): the fixed order even with a workspace; a packed batch (balanced)
    ([4096], 16, 4, 64, 64),
    ([4000], 16, 4, 128, 64),
    ([512], 4, 2, 64, 64),
    ([300], 4, 2, 128, 128),
    ([16700], 20, 4, 128, 128),
    ([130, 7000], 8, 8, 64, 64),
])
def test_other_shapes(shape):
    lens, hq, hkv, d, B = shape
    S = max(lens)
    say(f"balanced prefill {shape}")
    q, k, v, cu, sa, rp, ci = inputs(lens, hq, hkv, d, B, 2, 8404)
    route = torch.tensor([[1, 0]] * len(lens), dtype=torch.uint8, device=DEV)
    ws = new_workspace()
    for layer in (0, 1):
        check_pair(q, k, v, cu, S, route, layer, rp, ci, sa, ws, f"{shape} layer {layer}")


def test_packed_batch_with_mixed_routes():
    """Four prompts, FA for two and SA for the other two in one launch, every
    item through the same queues; then all four under each route."""
    lens = [3000, 9000, 20000, 512]
    S, hq, hkv, d = max(lens), 32, 8, 128
    say("balanced prefill, packed batch with mixed routes")
    q, k, v, cu, sa, rp, ci = inputs(lens, hq, hkv, d, 128, 8, 8707)
    route = torch.tensor([[1, 1, 0], [0, 1, 0], [1, 1, 0], [0, 1, 0]], dtype=torch.uint8, device=DEV)
    ws = new_workspace()
    for layer in (0, 1, 2):
        check_pair(q, k, v, cu, S, route, layer, rp, ci, sa, ws, f"packed layer {layer}")


def test_packed_batch_with_empty_and_one_token_requests():
    """Through the queues, a packed batch whose requests include two empty
    ones and a one-token one (its row is V's first row); every other request
    is checked against the oracle on rows across it, under both routes."""
    lens = [3000, 0, 9000, 1, 0, 12000]
    S, hq, hkv, d, B = max(lens), 32, 8, 128, 128
    say("balanced prefill, packed batch with empty and one-token requests")
    q, k, v, cu, sa, rp, ci = inputs(lens, hq, hkv, d, B, 8, 8808)
    route = torch.tensor([[1, 0], [0, 1], [0, 1], [1, 0], [1, 0], [0, 1]], dtype=torch.uint8, device=DEV)
    ws = new_workspace()
    m = oracle.block_mask(oracle.num_blocks(S, B), 1, 8)
    qh, kh, vh = (t.float().cpu().numpy() for t in (q, k, v))
    cu_h = [0]
    for n in lens:
        cu_h.append(cu_h[-1] + n)
    for layer in (0, 1):
        out = check_pair(q, k, v, cu, S, route, layer, rp, ci, sa, ws, f"empty/one-token layer {layer}")
        got = out.float().cpu().numpy()
        for r, n in enumerate(lens):
            if n == 0:
                continue
            a = cu_h[r]
            rows = sorted(set(range(0, n, max(1, n // 9))) | {n - 1})
            heads = [0, 13, 31]
            ref = oracle.attention_prefill(qh[a:a + n], kh[a:a + n], vh[a:a + n], bool(route[r, layer]), m, B,
                                           rows=rows, heads=heads)
            assert_attn_close(got[a:a + n][rows][:, heads], ref, f"request {r} layer {layer}")


def test_stream_workspace_is_reused_and_stays_zero():
    """The binding's per-stream workspace: the same tensor on every call,
    zero after each."""
    S, hq, hkv, d = 8192, 32, 8, 128
    q, k, v, cu, sa, rp, ci = inputs([S], hq, hkv, d, 128, 4, 8505)
    route = torch.tensor([[1, 0]], dtype=torch.uint8, device=DEV)
    ws = flux.prefill_workspace(DEV)
    assert ws is flux.prefill_workspace(DEV)
    first = flux.attn_prefill(q, k, v, cu, S, route, 0, rp, ci, sa)
    for _ in range(4):
        again = flux.attn_prefill(q, k, v, cu, S, route, 0, rp, ci, sa)
        torch.cuda.synchronize()
        assert torch.equal(bits(again), bits(first))
        assert not ws.any()


def test_balanced_prefill_under_graph_capture():
    """A balanced FA launch captured in a HIP graph: every replay (with eager
    work in between) reproduces the eager output and leaves the workspace
    zero, since the kernel itself resets the counters."""
    S, hq, hkv, d = 8192, 32, 8, 128
    say("balanced prefill under graph capture")
    q, k, v, cu, sa, rp, ci = inputs([S], hq, hkv, d, 128, 4, 8606)
    route = torch.tensor([[1, 0]], dtype=torch.uint8, device=DEV)
    ws = new_workspace()
    out = torch.empty_like(q)
    flux.attn_prefill(q, k, v, cu, S, route, 0, rp, ci, sa, out=out, workspace=ws)
    torch.cuda.synchronize()
    eager = bits(out).clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        flux.attn_prefill(q, k, v, cu, S, route, 0, rp, ci, sa, out=out, workspace=ws)
    for rep in range(3):
        out.fill_(float("nan"))
        torch.randn(1 << 20, device=DEV).sum()  # the program's own work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), eager), f"replay {rep}"
        assert not ws.any(), f"replay {rep}: workspace not zero"
