"""Host-side logic (CPU only): the seeded input recipes, the workload shapes
they describe, and the parts of bench.py that need no GPU (the one-GPU
refusal, the check that counted HBM traffic still belongs to the current
kernel source)."""

import hashlib
import json
import os
import subprocess
import sys

import pytest
import torch

from synth import inputs as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# ---------------------------------------------------------------- synthetic inputs

def test_normal_is_seeded_and_rounded_once():
    a = syn.normal((64, 4, 32), syn.generator(7))
    b = syn.normal((64, 4, 32), syn.generator(7))
    c = syn.normal((64, 4, 32), syn.generator(8))
    assert a.dtype == torch.bfloat16 and torch.equal(a, b) and not torch.equal(a, c)
    f = syn.normal((64, 4, 32), syn.generator(7), dtype=torch.float32)
    assert torch.equal(f.to(torch.bfloat16), a)  # the bf16 draw is the fp32 draw rounded (RNE)
    assert abs(float(f.mean())) < 0.05 and abs(float(f.std()) - 1.0) < 0.05


def test_router_weights_order_and_scale():
    w1, b1, w2, b2 = syn.router_weights(256, 64, 2, 11)
    assert w1.shape == (64, 256) and b1.shape == (64,) and w2.shape == (2, 64) and b2.shape == (2,)
    assert all(t.dtype == torch.float32 for t in (w1, b1, w2, b2))
    # one stream in the order W1, b1, W2, b2
    g = syn.generator(11)
    ref = [torch.randn(s, generator=g) * 0.02 for s in ((64, 256), (64,), (2, 64), (2,))]
    for t, r in zip((w1, b1, w2, b2), ref):
        assert torch.equal(t, r)
    assert abs(float(w1.std()) - 0.02) < 0.002


@pytest.mark.parametrize("n_layers,n_sa", [(36, 18), (2, 1), (32, 0), (5, 5)])
def test_seeded_route_has_exactly_n_sa(n_layers, n_sa):
    r = syn.seeded_route(n_layers, n_sa, 3)
    assert r.dtype == torch.uint8 and r.shape == (n_layers,)
    assert int((r == 0).sum()) == n_sa and int((r == 1).sum()) == n_layers - n_sa
    assert torch.equal(r, syn.seeded_route(n_layers, n_sa, 3))


def test_varlen_lengths_and_offsets():
    lens = syn.varlen_lengths(8, 8192, 65536, 1005)
    assert len(lens) == 8 and all(8192 <= x <= 65536 for x in lens)
    assert lens == syn.varlen_lengths(8, 8192, 65536, 1005)
    cu = syn.cu_seqlens(lens)
    assert cu.dtype == torch.int32 and int(cu[0]) == 0
    assert [int(cu[i + 1] - cu[i]) for i in range(8)] == list(lens)
    assert syn.varlen8().seqlens == lens


def test_workload_shapes():
    w = syn.PREFILL32K
    assert (w.seqlens, w.hq, w.hkv, w.head_dim, w.block_size, w.sink_blocks, w.local_blocks) == \
        ((32768,), 32, 8, 128, 128, 1, 16)
    assert w.local_blocks * w.block_size == 2048  # the 2048-token window
    d = syn.DECODE32K
    assert d.seqlens == (32768,) * 16 and d.n_layers == 36 and d.n_sa_layers == 18
    assert (d.sink_blocks * d.block_size, d.local_blocks * d.block_size) == (128, 2048)
    p = syn.PREFILL128K
    assert p.seqlens == (131072,) and p.n_layers == 36 and p.local_blocks * p.block_size == 4096
    assert (p.hidden_dim, p.router_h1) == (2560, 256)
    v = syn.varlen8()
    assert v.n_layers == 32 and (v.hidden_dim, v.router_h1) == (4096, 256) and v.decode_steps == 128
    t = syn.TINY
    assert (t.seqlens, t.hq, t.hkv, t.head_dim, t.block_size) == ((512,), 4, 2, 64, 64)
    assert len({w.seed for w in (t, w, d, p, v)}) == 5


# ---------------------------------------------------------------- bench.py host logic

def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_counted_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    src = tmp_path / "k.hip"
    src.write_text("kernel source v1\n")
    (tmp_path / "profiles").mkdir()
    rec = {"source": "k.hip", "source_sha256": hashlib.sha256(b"kernel source v1\n").hexdigest(),
           "build_flags": ["-O9"], "fa_bytes": 123}
    (tmp_path / "profiles" / "hbm_traffic_32k.json").write_text(json.dumps({"k": rec}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "build_flags", lambda source: ["-O9"])
    assert bench.counted_traffic("k")["fa_bytes"] == 123
    assert bench.counted_traffic("other") is None
    monkeypatch.setattr(bench, "build_flags", lambda source: [])  # built differently since
    assert bench.counted_traffic("k") is None
    monkeypatch.setattr(bench, "build_flags", lambda source: ["-O9"])
    src.write_text("kernel source v2\n")  # the kernel changed since the counters were taken
    assert bench.counted_traffic("k") is None


def test_build_flags_of_the_package_sources():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.build_flags("block_sparse_attention_flux_amd/csrc/prefill.hip") == \
        ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
    assert bench.build_flags("block_sparse_attention_flux_amd/csrc/decode.hip") == []


def _bench():
    import bench
    return bench


@pytest.mark.parametrize("S,fa,B,s,w", [(512, True, 64, 1, 2), (512, False, 64, 1, 2), (1000, False, 128, 3, 2),
                                        (581, True, 64, 0, 3), (300, False, 128, 0, 8), (129, False, 64, 1, 1)])
def test_prefill_work_counts_against_brute_force(S, fa, B, s, w):
    """The three work counts of bench.prefill_work, recounted one query row,
    one key and one (wave, tile) pair at a time from the oracle's mask."""
    import numpy as np
    import oracle
    d, hq, bn = 64, 2, 32
    nb = oracle.num_blocks(S, B)
    m = oracle.block_mask(nb, s, w)
    allowed = oracle.allowed_matrix(np.arange(S), S, fa, m, B)
    blocks = int(np.tril(np.ones((nb, nb))).sum()) if fa else int(m.sum())
    tiles = 0
    for t in range(nb):
        cols = range(t + 1) if fa else [j for j in range(nb) if m[t, j]]
        starts = [j * B + k * bn for j in cols for k in range(B // bn)]
        for wi in range(B // bn):
            first_row = t * B + wi * bn
            if first_row < S:
                tiles += sum(1 for st in starts if st <= first_row + bn - 1 and st < min(t * B + B, S))
    got = _bench().prefill_work(S, fa, B, s, w, d, hq, bn)
    assert got["causal"] == allowed.sum() * 4 * d * hq
    assert got["blocks"] == blocks * 4 * B * B * d * hq
    assert got["tiles"] == tiles * 4 * bn * bn * d * hq


def test_prefill_work_at_32k():
    """32768 tokens, 32 q heads, d 128, B 128: FA 32896 blocks, SA 4216 blocks
    (1 sink + 16 window blocks); every diagonal block runs 10 of its 16
    (wave, tile) pairs."""
    b = _bench()
    blk = 4.0 * 128 * 128 * 128 * 32
    fa = b.prefill_work(32768, True, 128, 1, 16, 128, 32)
    sa = b.prefill_work(32768, False, 128, 1, 16, 128, 32)
    assert fa["blocks"] == 32896 * blk and sa["blocks"] == 4216 * blk
    assert fa["tiles"] == (32896 - 256) * blk + 256 * blk * 10 / 16
    assert sa["tiles"] == (4216 - 256) * blk + 256 * blk * 10 / 16
    assert fa["causal"] == 32768 * 32769 // 2 * 4.0 * 128 * 32
