"""The library under HIP graph capture and on concurrent streams.

A whole routed stack (router, mask, FA and SA prefill, FA and SA decode)
is captured once in a HIP graph and replayed several times, with the
program's own eager work and synchronisations between the replays; every
replay must reproduce the eager outputs bit for bit.  The library issues no
memset or copy of its own, so a graph holds only its kernels.

Two calls on two streams at the same time (a prefill on one, a decode with
its own workspace on the other) must give what they give one after the
other: the library keeps no state shared between calls (the decode entry
point without allocation is the documented exception and is not used here).
"""

import pytest
import torch

from synth import inputs as syn
from tests.flux_testlib import ensure_built

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
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


class Stack:
    """Inputs and outputs of one routed stack: 2 layers over 2 packed prompts."""

    def __init__(self, seed, lens=(3000, 1234), hq=16, hkv=4, d=128, B=128, D=512):
        g = syn.generator(seed, DEV)
        self.lens = list(lens)
        T, S = sum(lens), max(lens)
        self.S = S
        self.cu = syn.cu_seqlens(lens, DEV)
        self.hidden = syn.normal((T, D), g, DEV)
        w1, b1, w2, b2 = syn.router_weights(D, 64, 2, seed)
        b2 = torch.tensor([1.0, -1.0])  # layer 0 FA, layer 1 SA
        self.w = [t.to(DEV) for t in (w1, b1, w2, b2)]
        self.q = syn.normal((T, hq, d), g, DEV)
        self.k = syn.normal((T, hkv, d), g, DEV)
        self.v = syn.normal((T, hkv, d), g, DEV)
        self.sa = flux.SAParams(B, 1, 4)
        n = len(lens)
        self.qd = syn.normal((n, hq, d), g, DEV)
        self.kc = syn.normal((n, hkv, S, d), g, DEV)
        self.vc = syn.normal((n, hkv, S, d), g, DEV)
        self.sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
        self.route = torch.empty((n, 2), dtype=torch.uint8, device=DEV)
        self.logits = torch.empty((n, 2), dtype=torch.float32, device=DEV)
        self.rws = torch.empty(flux.route_workspace_size(n, D, 64), dtype=torch.uint8, device=DEV)
        nb = flux.mask_blocks(S, self.sa)
        self.rp = torch.empty(nb + 1, dtype=torch.int32, device=DEV)
        self.ci = torch.empty(flux.mask_nnz(S, self.sa), dtype=torch.int32, device=DEV)
        self.dws = flux.decode_workspace(n, hq, hkv, d, S, DEV)
        self.out = [torch.empty_like(self.q) for _ in range(2)]
        self.dout = [torch.empty_like(self.qd) for _ in range(2)]

    def outputs(self):
        return [self.route, self.logits, self.rp, self.ci] + self.out + self.dout

    def run(self):
        flux.route(self.hidden, self.cu, *self.w, route_out=self.route, logits_out=self.logits,
                   workspace=self.rws)
        flux._check(flux._LIB.flux_build_block_mask(self.S, self.sa.c(), None, flux._ptr(self.rp),
                                                    flux._ptr(self.ci), flux._stream(self.q.device)),
                    "flux_build_block_mask")
        for layer in (0, 1):
            flux.attn_prefill(self.q, self.k, self.v, self.cu, self.S, self.route, layer, self.rp, self.ci,
                              self.sa, out=self.out[layer])
            flux.attn_decode(self.qd, self.kc, self.vc, self.sl, self.route, layer, self.rp, self.ci, self.sa,
                             self.dws, out=self.dout[layer])


def test_routed_stack_graph_replays():
    say("graph capture of a routed stack")
    st = Stack(9101)
    st.run()
    torch.cuda.synchronize()
    assert st.route[:, 0].all() and not st.route[:, 1].any(), "the biases route layer 0 to FA, 1 to SA"
    eager = [bits(t).clone() for t in st.outputs()]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.run()
    for rep in range(3):
        for t in st.outputs():
            t.zero_()
        scratch = torch.randn(1 << 20, device=DEV).sum()  # the program's own work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(st.outputs(), eager)):
            assert torch.equal(bits(a), b), f"replay {rep}: output {i} differs from the eager run"
        del scratch


def test_prefill_and_decode_on_two_streams_at_once():
    say("concurrent prefill and decode on two streams")
    a, b = Stack(9202), Stack(9303, lens=(5000, 4096), hq=32, hkv=8)
    a.run()
    b.run()
    torch.cuda.synchronize()
    ref_a = [bits(t).clone() for t in a.out]
    ref_b = [bits(t).clone() for t in b.dout]
    for t in a.out + b.dout:
        t.zero_()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    for _ in range(2):
        with torch.cuda.stream(s1):
            for layer in (0, 1):
                flux.attn_prefill(a.q, a.k, a.v, a.cu, a.S, a.route, layer, a.rp, a.ci, a.sa, out=a.out[layer])
        with torch.cuda.stream(s2):
            for layer in (0, 1):
                flux.attn_decode(b.qd, b.kc, b.vc, b.sl, b.route, layer, b.rp, b.ci, b.sa, b.dws,
                                 out=b.dout[layer])
        torch.cuda.synchronize()
        for x, y in zip(a.out, ref_a):
            assert torch.equal(bits(x), y), "prefill on a second stream differs"
        for x, y in zip(b.dout, ref_b):
            assert torch.equal(bits(x), y), "decode on a second stream differs"
