"""libflux C ABI on the host: the library loads, exports every symbol that
include/flux.h declares, and its host-side functions and argument validation
behave as documented.  No GPU work is launched: every validation case below
fails before the library touches the HIP runtime."""

import ctypes
import re

import pytest
import torch

import oracle
from tests.flux_testlib import HEADER, LIB, ensure_built

ensure_built()
from block_sparse_attention_flux_amd import _lib  # noqa: E402

lib = _lib.load()
NULL = None
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation rejects the call first
SA = _lib.SAParamsC


PROBE_HEADER = HEADER.replace("flux.h", "flux_probe.h")


def declared_symbols(header=HEADER):
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(flux_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    syms = declared_symbols()
    assert len(syms) == 21, syms
    raw = ctypes.CDLL(LIB)
    for s in syms:
        assert hasattr(raw, s), s
    assert sorted(n for n, _, _ in _lib.SIGNATURES) == syms
    probes = declared_symbols(PROBE_HEADER)
    assert len(probes) == 3, probes
    for s in probes:
        assert hasattr(raw, s), s
    assert sorted(n for n, _, _ in _lib.PROBE_SIGNATURES) == probes


def test_probe_host_validation():
    assert lib.flux_probe_mfma(NULL, 4, 4, NULL) == -1
    assert lib.flux_probe_mfma(FAKE, 0, 4, NULL) == -1
    assert lib.flux_probe_read(FAKE, 20, FAKE, 4, NULL) == -1  # not a multiple of 16
    assert lib.flux_probe_read(NULL, 4096, FAKE, 4, NULL) == -1
    assert lib.flux_probe_mfma_flops(2, 3) == 4 * 2 * 3 * 4 * 32 * 32 * 16 * 2


def test_status_strings():
    assert lib.flux_status_str(0) == b"ok"
    assert lib.flux_status_str(-1) == b"invalid argument"
    assert lib.flux_status_str(-4) == b"HIP runtime error"
    assert lib.flux_status_str(7) == b"unknown status"


@pytest.mark.parametrize("seqlen,B,s,w", [(512, 64, 1, 2), (32768, 128, 1, 16), (131072, 128, 1, 32),
                                          (1, 64, 0, 1), (1000, 128, 3, 2), (65536, 64, 0, 2000)])
def test_mask_nnz_matches_oracle(seqlen, B, s, w):
    nb = oracle.num_blocks(seqlen, B)
    assert lib.flux_mask_blocks(seqlen, SA(B, s, w)) == nb
    assert lib.flux_mask_nnz(seqlen, SA(B, s, w)) == oracle.mask_nnz(nb, s, w)


def test_mask_host_validation():
    assert lib.flux_mask_nnz(0, SA(64, 1, 2)) == _lib.FLUX_ERR_INVALID_ARG
    assert lib.flux_mask_nnz(10, SA(64, 1, 0)) == _lib.FLUX_ERR_INVALID_ARG
    assert lib.flux_mask_nnz(10, SA(64, -1, 1)) == _lib.FLUX_ERR_INVALID_ARG
    assert lib.flux_mask_blocks(-5, SA(64, 1, 1)) == _lib.FLUX_ERR_INVALID_ARG
    # builder: null outputs, bad params, unsupported block size, too many blocks
    assert lib.flux_build_block_mask(512, SA(64, 1, 2), NULL, NULL, FAKE, NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert lib.flux_build_block_mask(512, SA(64, 1, 0), NULL, FAKE, FAKE, NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert lib.flux_build_block_mask(512, SA(32, 1, 2), NULL, FAKE, FAKE, NULL) == _lib.FLUX_ERR_UNSUPPORTED
    assert lib.flux_build_block_mask(2**31 - 1, SA(64, 1, 2), NULL, FAKE, FAKE, NULL) == _lib.FLUX_ERR_UNSUPPORTED


def test_route_validation():
    ws = lib.flux_route_workspace_size(1, 256, 64)
    assert ws == 1 * (256 + 64) * 4
    assert lib.flux_route_workspace_size(0, 256, 64) == 0
    args = dict(hidden=FAKE, dt=0, cu=FAKE, n_req=1, d_in=256, w1=FAKE, b1=FAKE, h1=64, w2=FAKE,
                b2=FAKE, L=2, route=FAKE, logits=NULL, ws=FAKE, wsb=ws, stream=NULL)

    def call(**kw):
        a = dict(args, **kw)
        return lib.flux_route(a["hidden"], a["dt"], a["cu"], a["n_req"], a["d_in"], a["w1"], a["b1"],
                              a["h1"], a["w2"], a["b2"], a["L"], a["route"], a["logits"], a["ws"],
                              a["wsb"], a["stream"])
    assert call(hidden=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert call(route=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert call(dt=5) == _lib.FLUX_ERR_INVALID_ARG
    assert call(n_req=0) == _lib.FLUX_ERR_INVALID_ARG
    assert call(L=0) == _lib.FLUX_ERR_INVALID_ARG
    assert call(d_in=65537) == _lib.FLUX_ERR_UNSUPPORTED
    assert call(n_req=70000) == _lib.FLUX_ERR_UNSUPPORTED
    assert call(ws=NULL) == _lib.FLUX_ERR_WORKSPACE
    assert call(wsb=ws - 1) == _lib.FLUX_ERR_WORKSPACE


PREFILL_OK = dict(q=FAKE, k=FAKE, v=ctypes.c_void_p(0x2000), out=ctypes.c_void_p(0x3000), cu=FAKE,
                  n_req=1, max_seqlen=512, hq=4, hkv=2, d=64, scale=0.125, route=FAKE, L=2, layer=0,
                  rp=FAKE, ci=FAKE, mb=8, sa=SA(64, 1, 2), ws=NULL, wsb=0, stream=NULL)


def prefill(**kw):
    a = dict(PREFILL_OK, **kw)
    return lib.flux_attn_prefill(a["q"], a["k"], a["v"], a["out"], a["cu"], a["n_req"], a["max_seqlen"],
                                 a["hq"], a["hkv"], a["d"], a["scale"], a["route"], a["L"], a["layer"],
                                 a["rp"], a["ci"], a["mb"], a["sa"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), -1), (dict(route=NULL), -1), (dict(rp=NULL), -1),
    (dict(out=FAKE), -1),                      # out aliases q
    (dict(hq=5, hkv=2), -1), (dict(hkv=0), -1), (dict(n_req=0), -1), (dict(max_seqlen=0), -1),
    (dict(layer=2), -1), (dict(layer=-1), -1), (dict(scale=0.0), -1), (dict(scale=float("nan")), -1),
    (dict(sa=SA(64, 1, 0)), -1), (dict(sa=SA(64, -2, 1)), -1),
    (dict(mb=7), -1),                          # mask too small for max_seqlen
    (dict(d=96), -2), (dict(sa=SA(32, 1, 2)), -2), (dict(hq=34, hkv=2), -2),
    (dict(ws=ctypes.c_void_p(0x4000), wsb=1023), -3),                  # balancing workspace too small
    (dict(ws=ctypes.c_void_p(0x4000), wsb=64), -3),
    (dict(ws=ctypes.c_void_p(0x4008), wsb=1024), -3),                  # ... or not 16-byte aligned
    (dict(ws=ctypes.c_void_p(0x4000), wsb=1024, hq=5, hkv=2), -1),     # other checks still apply
])
def test_prefill_validation(kw, code):
    assert prefill(**kw) == code


def test_prefill_workspace_size():
    """The balancing workspace is a fixed 1024 bytes: 8 queue counters, each
    on a 128-byte line of its own."""
    assert lib.flux_attn_prefill_workspace_size() == _lib.FLUX_PREFILL_WORKSPACE_BYTES == 1024


def test_decode_workspace_size():
    """Workspace = fp32 partials (head_dim values + max + sum) of every work-item
    slot for each query head of a kv group, then one (first slot, count) pair
    per (sequence, kv head).  Slots: at most 1024, and at most the pairs plus
    one per 256 keys a call can visit; 0 when no pair can be split."""
    def size(n, hq, hkv, d, ml):
        return lib.flux_attn_decode_workspace_size(n, hq, hkv, d, ml)
    units = 16 * 8
    assert size(16, 32, 8, 128, 32768) == 1024 * 4 * (128 + 2) * 4 + units * 8
    assert size(2, 4, 2, 64, 300) == (4 + 4 * 427 // 256) * 2 * 66 * 4 + 4 * 8
    assert size(1, 1, 1, 64, 128) == 0          # 255 keys at most: never split
    assert size(1, 1, 1, 64, 129) > 0
    assert size(129, 32, 8, 128, 4096) == 0     # 1032 pairs: one item each
    assert size(128, 32, 8, 128, 4096) == 0     # 1024 pairs fill the 1024 slots
    assert size(127, 32, 8, 128, 4096) > 0
    assert size(0, 32, 8, 128, 32768) == 0
    assert size(16, 30, 8, 128, 32768) == 0     # hq not a multiple of hkv


def test_decode_noalloc_validation():
    """flux_attn_decode_noalloc checks its arguments like flux_attn_decode
    before any HIP call (so these run without a GPU); its device scratch holds
    the largest workspace a valid call can need."""
    assert _lib.FLUX_DECODE_SCRATCH_BYTES == 9 << 20
    worst = max(lib.flux_attn_decode_workspace_size(n, 16 * hkv, hkv, 128, 1 << 20)
                for n, hkv in ((1, 1), (16, 8), (127, 8), (64, 16), (1023, 1)))
    assert 8 << 20 < worst <= _lib.FLUX_DECODE_SCRATCH_BYTES

    def dec(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, out=ctypes.c_void_p(0x3000), sl=FAKE, n=16, ml=32768, hq=32,
                 hkv=8, d=128, scale=0.088, route=FAKE, L=36, layer=0, rp=FAKE, ci=FAKE, mb=256,
                 sa=SA(128, 1, 16), stream=NULL)
        a.update(kw)
        return lib.flux_attn_decode_noalloc(a["q"], a["k"], a["v"], a["out"], a["sl"], a["n"], a["ml"],
                                            a["hq"], a["hkv"], a["d"], a["scale"], a["route"], a["L"],
                                            a["layer"], a["rp"], a["ci"], a["mb"], a["sa"], a["stream"])
    assert dec(q=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(out=FAKE) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(route=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(hq=30) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(mb=255) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(layer=36) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(d=80) == _lib.FLUX_ERR_UNSUPPORTED
    assert dec(hq=64, hkv=2) == _lib.FLUX_ERR_UNSUPPORTED   # 32 query heads per kv head


def test_decode_append_validation():
    """flux_attn_decode_append: flux_attn_decode's checks plus the new rows,
    which must be given and must not alias the caches or the output."""
    ws = lib.flux_attn_decode_workspace_size(16, 32, 8, 128, 32768)
    KC, VC, KN, VN, OUT = (ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000, 0x40000, 0x50000))

    def dec(**kw):
        a = dict(q=FAKE, kn=KN, vn=VN, kc=KC, vc=VC, out=OUT, sl=FAKE, n=16, ml=32768, hq=32, hkv=8,
                 d=128, scale=0.088, route=FAKE, L=36, layer=0, rp=FAKE, ci=FAKE, mb=256,
                 sa=SA(128, 1, 16), ws=FAKE, wsb=ws, stream=NULL)
        a.update(kw)
        return lib.flux_attn_decode_append(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["out"], a["sl"],
                                           a["n"], a["ml"], a["hq"], a["hkv"], a["d"], a["scale"],
                                           a["route"], a["L"], a["layer"], a["rp"], a["ci"], a["mb"],
                                           a["sa"], a["ws"], a["wsb"], a["stream"])
    assert dec(kn=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(vn=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(kc=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(kn=KC) == _lib.FLUX_ERR_INVALID_ARG      # new row aliases a cache
    assert dec(vn=VC) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(out=KC) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(vc=KC) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(q=OUT) == _lib.FLUX_ERR_INVALID_ARG      # out aliases q
    assert dec(mb=255) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(d=80) == _lib.FLUX_ERR_UNSUPPORTED
    assert dec(ws=NULL) == _lib.FLUX_ERR_WORKSPACE


def test_decode_validation():
    ws = lib.flux_attn_decode_workspace_size(16, 32, 8, 128, 32768)
    assert ws > 0 and ws % 4 == 0
    assert lib.flux_attn_decode_workspace_size(0, 32, 8, 128, 32768) == 0

    def dec(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, out=ctypes.c_void_p(0x3000), sl=FAKE, n=16, ml=32768, hq=32,
                 hkv=8, d=128, scale=0.088, route=FAKE, L=36, layer=0, rp=FAKE, ci=FAKE, mb=256,
                 sa=SA(128, 1, 16), ws=FAKE, wsb=ws, stream=NULL)
        a.update(kw)
        return lib.flux_attn_decode(a["q"], a["k"], a["v"], a["out"], a["sl"], a["n"], a["ml"], a["hq"],
                                    a["hkv"], a["d"], a["scale"], a["route"], a["L"], a["layer"], a["rp"],
                                    a["ci"], a["mb"], a["sa"], a["ws"], a["wsb"], a["stream"])
    assert dec(q=NULL) == -1
    assert dec(out=FAKE) == -1
    assert dec(mb=255) == -1
    assert dec(layer=36) == -1
    assert dec(d=80) == -2
    assert dec(ws=NULL) == -3
    assert dec(wsb=ws - 4) == -3
    assert dec(ws=ctypes.c_void_p(0x1008)) == -3   # not 16-byte aligned


def test_binding_rejects_host_tensors():
    import block_sparse_attention_flux_amd as flux
    x = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        flux.attn_prefill(x, x[:, :1].contiguous(), x[:, :1].contiguous(), torch.zeros(2, dtype=torch.int32),
                          4, torch.ones(1, 1, dtype=torch.uint8), 0, torch.zeros(2, dtype=torch.int32),
                          torch.zeros(1, dtype=torch.int32), flux.SAParams(64, 1, 1))
    assert flux.mask_nnz(32768, flux.SAParams(128, 1, 16)) == 4216
    with pytest.raises(ValueError):
        flux.mask_nnz(0, flux.SAParams(128, 1, 16))


def test_kv_rows_and_cache_validation():
    sa = SA(128, 1, 16)
    assert lib.flux_kv_rows(32768, sa, 0) == 32768
    assert lib.flux_kv_rows(32768, sa, 1) == 17 * 128
    assert lib.flux_kv_rows(5000, SA(64, 0, 3), 1) == 3 * 64
    assert lib.flux_kv_rows(0, sa, 0) == _lib.FLUX_ERR_INVALID_ARG
    assert lib.flux_kv_rows(100, sa, 2) == _lib.FLUX_ERR_INVALID_ARG
    assert lib.flux_kv_rows(100, SA(128, 1, 0), 1) == _lib.FLUX_ERR_INVALID_ARG

    def store(k=FAKE, cu=FAKE, n_req=2, max_s=100, hkv=8, d=128, max_len=200, compact=0, p=sa):
        return lib.flux_kv_store_prefill(k, FAKE, cu, n_req, max_s, hkv, d, FAKE, FAKE, max_len,
                                         compact, p, NULL)
    assert store(k=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert store(cu=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert store(max_s=300) == _lib.FLUX_ERR_INVALID_ARG          # prompt longer than the cache
    assert store(d=96) == _lib.FLUX_ERR_UNSUPPORTED
    assert store(compact=3) == _lib.FLUX_ERR_INVALID_ARG
    assert store(compact=1, p=SA(96, 1, 2)) == _lib.FLUX_ERR_UNSUPPORTED
    assert store(compact=1, p=SA(128, -1, 2)) == _lib.FLUX_ERR_INVALID_ARG
    assert store(n_req=70000, max_len=200) == _lib.FLUX_ERR_UNSUPPORTED

    def append(kn=FAKE, sl=FAKE, n=4, hkv=8, d=128, max_len=100, compact=0, p=sa):
        return lib.flux_kv_append(kn, FAKE, sl, n, hkv, d, FAKE, FAKE, max_len, compact, p, NULL)
    assert append(kn=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert append(sl=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert append(n=0) == _lib.FLUX_ERR_INVALID_ARG
    assert append(hkv=0) == _lib.FLUX_ERR_INVALID_ARG
    assert append(d=80) == _lib.FLUX_ERR_UNSUPPORTED
    assert append(compact=1, p=SA(128, 1, 0)) == _lib.FLUX_ERR_INVALID_ARG


def test_compact_decode_validation():
    sa = SA(128, 1, 16)
    ws = lib.flux_attn_decode_workspace_size(16, 32, 8, 128, 32768)

    def dec(q=FAKE, out=FAKE, n=16, max_len=32768, hq=32, hkv=8, d=128, scale=0.088, rp=FAKE,
            mb=256, p=sa, w=FAKE, wsb=ws):
        return lib.flux_attn_decode_sa_compact(q, FAKE, FAKE, out, FAKE, n, max_len, hq, hkv, d,
                                               scale, rp, FAKE, mb, p, w, wsb, NULL)
    assert dec(q=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(out=FAKE, q=FAKE) == _lib.FLUX_ERR_INVALID_ARG    # out aliases q
    assert dec(rp=NULL, out=ctypes.c_void_p(0x2000)) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(hq=30, out=ctypes.c_void_p(0x2000)) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(d=96, out=ctypes.c_void_p(0x2000)) == _lib.FLUX_ERR_UNSUPPORTED
    assert dec(mb=255, out=ctypes.c_void_p(0x2000)) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(p=SA(128, 1, 0), out=ctypes.c_void_p(0x2000)) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(w=NULL, out=ctypes.c_void_p(0x2000)) == _lib.FLUX_ERR_WORKSPACE
    assert dec(wsb=ws - 4, out=ctypes.c_void_p(0x2000)) == _lib.FLUX_ERR_WORKSPACE


def test_head_route_and_soft_validation():
    """The per-kv-head and soft entry points reject bad arguments on the host
    exactly like flux_attn_prefill / flux_attn_decode (nothing is launched)."""
    sa = SA(128, 1, 16)
    OUT = ctypes.c_void_p(0x2000)

    def pre(fn, route=FAKE, hq=32, hkv=8, d=128, mb=256):
        if fn is lib.flux_attn_prefill_soft:  # the soft pass takes the balancing workspace too
            return fn(FAKE, FAKE, FAKE, OUT, FAKE, 1, 32768, hq, hkv, d, 0.088, route, 2, 0, FAKE, FAKE,
                      mb, sa, NULL, 0, NULL)
        return fn(FAKE, FAKE, FAKE, OUT, FAKE, 1, 32768, hq, hkv, d, 0.088, route, 2, 0, FAKE, FAKE,
                  mb, sa, NULL)
    assert lib.flux_attn_prefill_soft(FAKE, FAKE, FAKE, OUT, FAKE, 1, 32768, 32, 8, 128, 0.088, FAKE, 2, 0,
                                      FAKE, FAKE, 256, sa, ctypes.c_void_p(0x4000), 32, NULL) \
        == _lib.FLUX_ERR_WORKSPACE
    for fn in (lib.flux_attn_prefill_heads, lib.flux_attn_prefill_soft):
        assert pre(fn, route=NULL) == _lib.FLUX_ERR_INVALID_ARG   # route / r_soft missing
        assert pre(fn, hq=30) == _lib.FLUX_ERR_INVALID_ARG
        assert pre(fn, d=96) == _lib.FLUX_ERR_UNSUPPORTED
        assert pre(fn, hq=64, hkv=2) == _lib.FLUX_ERR_UNSUPPORTED  # group of 32 > 16
        assert pre(fn, mb=255) == _lib.FLUX_ERR_INVALID_ARG
    ws = lib.flux_attn_decode_workspace_size(16, 32, 8, 128, 32768)

    def dec(route=FAKE, w=FAKE, wsb=ws):
        return lib.flux_attn_decode_heads(FAKE, FAKE, FAKE, OUT, FAKE, 16, 32768, 32, 8, 128, 0.088, route,
                                          2, 0, FAKE, FAKE, 256, sa, w, wsb, NULL)
    assert dec(route=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert dec(w=NULL) == _lib.FLUX_ERR_WORKSPACE
    assert dec(wsb=ws - 1) == _lib.FLUX_ERR_WORKSPACE


def test_dynamic_mask_workspace_size_and_validation():
    """flux_build_block_mask_dynamic: workspace formula (pooled Q and K in fp32,
    per-KV-head probability sums, one count per row, a row-stride column
    buffer) and host-side rejections."""
    S, hq, hkv, d, B = 32768, 32, 8, 128, 128
    nb = S // B
    ws = lib.flux_dynamic_mask_workspace_size(S, hq, hkv, d, B)
    assert ws == (nb * hq * d + nb * hkv * d + nb * hkv * nb) * 4 + nb * 4 + nb * nb * 4
    assert lib.flux_dynamic_mask_workspace_size(0, hq, hkv, d, B) == 0
    DP = _lib.DynParamsC
    W = ctypes.c_void_p(0x2000)
    cap = nb * (nb + 1) // 2

    def call(q=FAKE, k=FAKE, s=S, h=hq, hk=hkv, dd=d, scale=0.088, p=None, rp=FAKE, ci=FAKE, c=cap, w=W, wb=ws):
        p = p or DP(B, 1, 0.9, 17)
        return lib.flux_build_block_mask_dynamic(q, k, s, h, hk, dd, scale, p, rp, ci, c, w, wb, NULL)
    assert call(q=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert call(rp=NULL) == _lib.FLUX_ERR_INVALID_ARG
    assert call(h=30) == _lib.FLUX_ERR_INVALID_ARG
    assert call(s=0) == _lib.FLUX_ERR_INVALID_ARG
    assert call(scale=0.0) == _lib.FLUX_ERR_INVALID_ARG
    assert call(p=DP(B, -1, 0.9, 0)) == _lib.FLUX_ERR_INVALID_ARG
    assert call(p=DP(B, 1, -0.5, 0)) == _lib.FLUX_ERR_INVALID_ARG
    assert call(p=DP(B, 1, float("nan"), 0)) == _lib.FLUX_ERR_INVALID_ARG
    assert call(p=DP(B, 1, 0.9, -3)) == _lib.FLUX_ERR_INVALID_ARG
    assert call(dd=96) == _lib.FLUX_ERR_UNSUPPORTED
    assert call(p=DP(32, 1, 0.9, 0)) == _lib.FLUX_ERR_UNSUPPORTED
    assert call(h=64, hk=2) == _lib.FLUX_ERR_UNSUPPORTED        # GQA group of 32
    assert call(s=1024 * 128 + 1) == _lib.FLUX_ERR_UNSUPPORTED  # 1025 blocks
    assert call(c=cap - 1) == _lib.FLUX_ERR_INVALID_ARG
    assert call(w=NULL) == _lib.FLUX_ERR_WORKSPACE
    assert call(wb=ws - 1) == _lib.FLUX_ERR_WORKSPACE
    assert call(w=ctypes.c_void_p(0x2008)) == _lib.FLUX_ERR_WORKSPACE  # not 16-byte aligned
