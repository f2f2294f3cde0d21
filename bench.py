#!/usr/bin/env python3
"""Throughput of the routed-attention hot path on one MI355X.

Metric: routed-attention prefill tok/s at 32K and decode tok/s at 32K context,
with the fraction of the bf16 MFMA peak (prefill) and of the HBM peak (decode).

Prefill step (the JSON line's `value`), Qwen3-4B-shaped, 32768 tokens, 32 q /
8 kv heads, head_dim 128, bf16 N(0,1) inputs resident in HBM:
  flux_route      hidden [32768][2560] bf16 -> MLP 2560 -> 256 -> 2 -> route;
                  the seeded N(0, 0.02) weights carry output biases (+1, -1)
                  so layer 0 routes to FA and layer 1 to SA: the workload runs
                  FA and SA on identical inputs, and the kernels read the
                  router's output on the device (no host sync);
  flux_build_block_mask  SA mask, blocks of 128, 1 sink block, window 2048;
  flux_attn_prefill x 2  layer 0 (FA) and layer 1 (SA) on the same q/k/v.
  value = 32768 tokens / step time.
Decode phase (the "decode" object): 16 sequences x 32768 cached tokens, 36
layers with distinct caches (72 GiB), a seeded route with exactly 18 SA layers;
one step = 36 flux_attn_decode calls; tok/s = 16 / step time.

Roofline: the dominant kernel is the prefill kernel; achieved = algorithmic
(computed-block) flops of its launches / their summed duration, timed with HIP
events on the launch stream.  Computed-block flops per layer =
active 128x128 blocks * 4 * 128^2 * head_dim * hq (FA: all 32896 causal
blocks; SA: 4216 blocks).  Decode bytes per step = K+V bytes the layers must
read (FA: all 32768 keys, SA: 17 blocks of 128 keys).
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "routed-attention prefill tok/s @32K & decode tok/s @32K ctx; % MFMA / HBM peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=10)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the 131072-token routed prefill and the varlen8 prefill + decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 256 MiB device copy (counter calibration)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard by KV-head group for prefill and by sequence for decode)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import __graft_entry__
    __graft_entry__._build_module().ensure_built()  # rebuilds only if the sources changed
    import block_sparse_attention_flux_amd as flux
    from synth import inputs as syn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ------------------------------------------------------------ prefill inputs
    wl = syn.PREFILL32K
    S, hq, hkv, d = wl.seqlens[0], wl.hq, wl.hkv, wl.head_dim
    sa = flux.SAParams(wl.block_size, wl.sink_blocks, wl.local_blocks)
    g = syn.generator(wl.seed, dev)
    hidden = syn.normal((S, wl.hidden_dim), g, dev)
    q = syn.normal((S, hq, d), g, dev)
    k = syn.normal((S, hkv, d), g, dev)
    v = syn.normal((S, hkv, d), g, dev)
    w1, b1, w2, b2 = syn.router_weights(wl.hidden_dim, wl.router_h1, wl.n_layers, wl.seed)
    b2 = b2 + torch.tensor([1.0, -1.0])  # layer 0 -> FA, layer 1 -> SA
    w1, b1, w2, b2 = (t.to(dev) for t in (w1, b1, w2, b2))
    cu = syn.cu_seqlens([S], dev)
    nb = flux.mask_blocks(S, sa)
    nnz = flux.mask_nnz(S, sa)
    route = torch.empty((1, wl.n_layers), dtype=torch.uint8, device=dev)
    row_ptr = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(nnz, dtype=torch.int32, device=dev)
    out = [torch.empty_like(q) for _ in range(wl.n_layers)]
    L = flux._lib
    F = flux._LIB
    cstream = __import__("ctypes").c_void_p(stream.cuda_stream)

    def P(t):
        return __import__("ctypes").c_void_p(t.data_ptr())

    def check(code, what):
        if code != 0:
            raise RuntimeError(f"{what} failed: {flux.status_str(code)}")

    route_ws = torch.empty(flux.route_workspace_size(1, wl.hidden_dim, wl.router_h1), dtype=torch.uint8,
                           device=dev)

    def route_call():
        check(F.flux_route(P(hidden), L.FLUX_BF16, P(cu), 1, wl.hidden_dim, P(w1), P(b1), wl.router_h1,
                           P(w2), P(b2), wl.n_layers, P(route), None, P(route_ws), route_ws.numel(),
                           cstream), "flux_route")

    def mask_call():
        check(F.flux_build_block_mask(S, sa.c(), None, P(row_ptr), P(col_idx), cstream), "mask")

    def prefill_call(layer):
        check(F.flux_attn_prefill(P(q), P(k), P(v), P(out[layer]), P(cu), 1, S, hq, hkv, d,
                                  1.0 / math.sqrt(d), P(route), wl.n_layers, layer, P(row_ptr),
                                  P(col_idx), nb, sa.c(), cstream), "prefill")

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def prefill_step(timers=None):
        if timers is None:
            route_call(); mask_call(); prefill_call(0); prefill_call(1)
            return
        e = [ev() for _ in range(5)]
        e[0].record(stream); route_call(); mask_call()
        e[1].record(stream); prefill_call(0)
        e[2].record(stream); prefill_call(1)
        e[3].record(stream)
        timers.append(e)

    log(f"prefill warmup x{args.warmup}")
    for _ in range(args.warmup):
        prefill_step()
    torch.cuda.synchronize()
    assert route[0].tolist() == [1, 0], f"router did not produce the FA/SA split: {route.tolist()}"

    log(f"prefill timed x{args.steps}")
    timers = []
    t0, t1 = ev(), ev()
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        prefill_step(timers)
    t1.record(stream)
    torch.cuda.synchronize()
    step_ms = t0.elapsed_time(t1) / args.steps
    rm = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])]
                   for e in timers])
    router_mask_ms, fa_ms, sa_ms = (float(x) for x in rm.mean(axis=0))
    blk_flops = 4.0 * wl.block_size ** 2 * d * hq
    fa_flops = nb * (nb + 1) / 2 * blk_flops
    sa_flops = nnz * blk_flops
    pre_tflops = (fa_flops + sa_flops) / ((fa_ms + sa_ms) * 1e-3) / 1e12
    value = S / (step_ms * 1e-3)
    log(f"prefill step {step_ms:.3f} ms  FA {fa_ms:.3f} ms ({fa_flops / fa_ms / 1e9:.1f} TF/s)  "
        f"SA {sa_ms:.3f} ms ({sa_flops / sa_ms / 1e9:.1f} TF/s)  router+mask {router_mask_ms:.3f} ms")

    if args.copy_probe:
        # plain elementwise kernel with known traffic: reads 256 MiB, writes 256 MiB
        src = torch.zeros(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log("copy probe: add kernel reads 268435456 bytes and writes 268435456 bytes")
        del src, dst

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 q/k/v and hidden states, seeded N(0,0.02) router",
        "config": {
            "workload": "Qwen3-4B-shaped routed prefill, 32768 tokens, 1 FA + 1 SA layer on identical inputs",
            "global_batch": 1, "seq_len": S, "hq": hq, "hkv": hkv, "head_dim": d,
            "sa": {"block": wl.block_size, "sink_blocks": wl.sink_blocks, "local_blocks": wl.local_blocks},
            "router": f"{wl.hidden_dim}->{wl.router_h1}->{wl.n_layers}", "parallelism": "single GPU",
        },
        "prefill": {
            "fa_ms": round(fa_ms, 4), "sa_ms": round(sa_ms, 4), "router_mask_ms": round(router_mask_ms, 4),
            "fa_tflops": round(fa_flops / fa_ms / 1e9, 1), "sa_tflops": round(sa_flops / sa_ms / 1e9, 1),
            "fa_frac_mfma": round(fa_flops / fa_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "sa_frac_mfma": round(sa_flops / sa_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "fa_tok_s": round(S / (fa_ms * 1e-3), 1), "sa_tok_s": round(S / (sa_ms * 1e-3), 1),
        },
        "roofline": {
            "kernel": "prefill_kernel<128,128,32,3> (FA + SA launches)",
            "bound": "mfma", "achieved": round(pre_tflops, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
        },
    }
    result["head_routing"] = head_routing(flux, q, k, v, cu, S, row_ptr, col_idx, sa, fa_ms, sa_ms,
                                          fa_flops + sa_flops, stream, log)
    result["soft_routing"] = soft_routing(flux, q, k, v, cu, S, row_ptr, col_idx, sa, fa_ms, sa_ms,
                                          fa_flops, sa_flops, stream, log)
    result["dynamic_mask"] = dynamic_mask(flux, q, k, v, cu, S, wl, sa, sa_ms, stream, log)
    att = attainable(flux, dev, stream, log)
    result["attainable"] = att
    result["roofline"]["frac_attainable"] = round(pre_tflops / att["mfma_tflops"], 4)
    result["prefill"]["fa_frac_attainable"] = round(fa_flops / fa_ms / 1e9 / att["mfma_tflops"], 4)
    result["prefill"]["sa_frac_attainable"] = round(sa_flops / sa_ms / 1e9 / att["mfma_tflops"], 4)
    tr = counted_traffic("prefill_kernel")
    if tr is not None:
        result["roofline"]["traffic"] = round(tr["per_launch_bytes"])
        result["roofline"]["traffic_note"] = ("bytes per launch (mean of the FA and SA launch) from "
                                              "profiles/hbm_traffic_32k.json")
    del hidden
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ decode phase
    if not args.no_decode:
        result["decode"] = run_decode(args, flux, syn, dev, stream, log)
        result["decode"]["roofline"]["frac_attainable"] = round(
            result["decode"]["roofline"]["achieved"] / att["hbm_read_gbs"], 4)

    # ------------------------------------------------------------ long workloads
    if not args.no_long:
        result["prefill131k"] = run_prefill_131k(flux, syn, dev, stream, log)
        result["varlen8"] = run_varlen8(flux, syn, dev, stream, log)

    # ------------------------------------------------------------ oracle on the host
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, q, k, v, S, wl, log)

    print(json.dumps(result), flush=True)
    return 0


def head_routing(flux, q, k, v, cu, S, row_ptr, col_idx, sa, fa_ms, sa_ms, pair_flops, stream, log):
    """Layer-level against head-level routing on the same 32K inputs and the
    same total work: the layer-routed pair is one FA layer + one SA layer; the
    head-routed pair is two layers that each send half of the kv heads to FA
    and the other half to SA (complementary halves).  The pages' case for
    layer-level routing is that head-level decisions leave the GPU waiting on
    the heaviest heads (load imbalance, long tails)."""
    import torch

    hkv = k.shape[1]
    out = torch.empty_like(q)

    def timed(route, layer, reps=5):
        flux.attn_prefill(q, k, v, cu, S, route, layer, row_ptr, col_idx, sa, out=out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            flux.attn_prefill(q, k, v, cu, S, route, layer, row_ptr, col_idx, sa, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    res = {"layer_level_pair_ms": round(fa_ms + sa_ms, 4)}
    patterns = {"halves": [1 if g < hkv // 2 else 0 for g in range(hkv)],
                "alternate": [1 - g % 2 for g in range(hkv)]}
    for name, pat in patterns.items():
        r = torch.tensor([[pat, [1 - x for x in pat]]], dtype=torch.uint8, device=q.device)
        ms = timed(r, 0) + timed(r, 1)
        res[f"head_level_pair_ms_{name}"] = round(ms, 4)
        res[f"slowdown_{name}"] = round(ms / (fa_ms + sa_ms), 3)
    log(f"head routing: layer-level pair {fa_ms + sa_ms:.3f} ms, head-level pair "
        f"{res['head_level_pair_ms_halves']:.3f} ms (halves) / {res['head_level_pair_ms_alternate']:.3f} ms "
        f"(alternate) for the same {pair_flops / 1e12:.2f} TFLOP")
    res["note"] = ("head-routed launches deal every kv-head group to every XCD (a layer-routed launch "
                   "keeps whole groups on one XCD for L2 locality; the same interleaving costs a "
                   "layer-routed FA layer ~4 % and an SA layer ~15 %)")
    return res


def dynamic_mask(flux, q, k, v, cu, S, wl, sa, sa_ms, stream, log):
    """A content-aware SA mask for the 32K layer (mean-pooled coarse attention,
    Top-tau with tau 0.9, the sink block kept, at most as many blocks per row
    as the static mask), its build time, and the SA layer run on it, beside the
    SA layer on the static sink + window mask."""
    import torch

    B = wl.block_size
    cap = wl.sink_blocks + wl.local_blocks
    build = lambda: flux.build_block_mask_dynamic(q, k, B, wl.sink_blocks, 0.9, cap)
    row_ptr, col_idx = build()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record(stream)
    for _ in range(reps):
        row_ptr, col_idx = build()
    e1.record(stream)
    torch.cuda.synchronize()
    build_ms = e0.elapsed_time(e1) / reps
    nb = (S + B - 1) // B
    nnz = int(row_ptr[nb].item())
    route = torch.tensor([[0]], dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    flux.attn_prefill(q, k, v, cu, S, route, 0, row_ptr, col_idx, sa, out=out)
    torch.cuda.synchronize()
    reps = 20
    e0.record(stream)
    for _ in range(reps):
        flux.attn_prefill(q, k, v, cu, S, route, 0, row_ptr, col_idx, sa, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = nnz * 4.0 * B * B * q.shape[2] * q.shape[1]
    log(f"dynamic mask: build {build_ms:.3f} ms, {nnz} blocks; SA layer on it {ms:.3f} ms "
        f"({flops / ms / 1e9:.0f} TF/s) vs {sa_ms:.3f} ms on the static mask")
    return {"tau": 0.9, "max_blocks_per_row": cap, "build_ms": round(build_ms, 4), "nnz_blocks": nnz,
            "density": round(nnz / (nb * (nb + 1) / 2), 4), "sa_ms": round(ms, 4),
            "sa_tflops": round(flops / ms / 1e9, 1), "static_sa_ms": round(sa_ms, 4),
            "note": "synthetic N(0,1) inputs give nearly uniform block scores, so the cap decides "
                    "most rows; the build is the overhead a content-aware mask adds per layer"}


def soft_routing(flux, q, k, v, cu, S, row_ptr, col_idx, sa, fa_ms, sa_ms, fa_flops, sa_flops, stream,
                 log):
    """The soft-routed forward r FA + (1 - r) SA of one 32K layer in one pass,
    against the FA and SA layers run separately (the soft pass shares S and the
    K/V tiles of the SA blocks with the FA branch)."""
    import torch

    r = torch.tensor([[0.5, 0.5]], dtype=torch.float32, device=q.device)
    out = torch.empty_like(q)
    flux.attn_prefill_soft(q, k, v, cu, S, r, 0, row_ptr, col_idx, sa, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record(stream)
    for _ in range(reps):
        flux.attn_prefill_soft(q, k, v, cu, S, r, 0, row_ptr, col_idx, sa, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    log(f"soft routing: one pass {ms:.3f} ms vs FA + SA layers {fa_ms + sa_ms:.3f} ms")
    return {"soft_pass_ms": round(ms, 4), "fa_plus_sa_ms": round(fa_ms + sa_ms, 4),
            "speedup_vs_two_layers": round((fa_ms + sa_ms) / ms, 3),
            "tflops_fa_plus_sa_work": round((fa_flops + sa_flops) / ms / 1e9, 1)}


def attainable(flux, dev, stream, log):
    """What this GPU reaches on a dense bf16 MFMA loop and on a streaming HBM
    read (the library's probe kernels): the ceilings beside the published peaks."""
    import torch

    def best_ms(fn, reps=3):
        fn()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return min(out)

    n_wg, iters = 256 * 3, 4096  # 12 waves per CU, as the prefill kernel runs
    sink = torch.empty(n_wg, dtype=torch.float32, device=dev)
    flops = flux.probe_mfma(sink, n_wg, iters)
    mfma_tflops = flops / best_ms(lambda: flux.probe_mfma(sink, n_wg, iters)) / 1e9
    src = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    rsink = torch.empty(4096, dtype=torch.int32, device=dev)
    read_gbs = src.numel() / best_ms(lambda: flux.probe_read(src, rsink)) / 1e6
    del src
    log(f"attainable: bf16 MFMA loop {mfma_tflops:.0f} TF/s, HBM streaming read {read_gbs:.0f} GB/s")
    return {"mfma_tflops": round(mfma_tflops, 1), "hbm_read_gbs": round(read_gbs, 1),
            "how": "library probe kernels: 768 workgroups x 4 waves of v_mfma_f32_32x32x16_bf16 chains; "
                   "one read of a 2 GiB buffer with 16-byte streaming loads; best of 3"}


def build_flags(source):
    """The extra hipcc flags the package's build script gives `source`."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_flux_build", os.path.join(ROOT, "block_sparse_attention_flux_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return list(mod.EXTRA_FLAGS.get(os.path.basename(source), []))


def counted_traffic(kernel):
    """HBM bytes measured by rocprofv3 counters for `kernel`, or None once the
    kernel's source or its build flags have changed since the counters were
    taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic_32k.json")
    try:
        rec = json.load(open(path))[kernel]
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
        flags = build_flags(rec["source"])
    except (OSError, KeyError, ValueError):
        return None
    if hashlib.sha256(src).hexdigest() != rec["source_sha256"] or rec.get("build_flags", []) != flags:
        return None
    return rec


def _events(torch, stream, n):
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    return ev


def run_prefill_131k(flux, syn, dev, stream, log):
    """The 131072-token workload: router on 131072 x 2560 bf16 hidden states
    (2560 -> 256 -> 36), mask, then all 36 layers routed by the router's
    decisions.  The 36 layers share one q/k/v set (1.5 GiB; every layer has
    the same shapes and the kernels are compute-bound, so the time is that of
    36 distinct layers).  One untimed pass, then one timed pass with an event
    around every layer."""
    import torch

    wl = syn.PREFILL128K
    S, L, d = wl.seqlens[0], wl.n_layers, wl.head_dim
    g = syn.generator(wl.seed, dev)
    hidden = syn.normal((S, wl.hidden_dim), g, dev)
    w1, b1, w2, b2 = (t.to(dev) for t in syn.router_weights(wl.hidden_dim, wl.router_h1, L, wl.seed))
    q = syn.normal((S, wl.hq, d), g, dev)
    k = syn.normal((S, wl.hkv, d), g, dev)
    v = syn.normal((S, wl.hkv, d), g, dev)
    out = torch.empty_like(q)
    cu = syn.cu_seqlens([S], dev)
    sa = flux.SAParams(wl.block_size, wl.sink_blocks, wl.local_blocks)
    nb = flux.mask_blocks(S, sa)
    nnz = flux.mask_nnz(S, sa)
    rws = torch.empty(flux.route_workspace_size(1, wl.hidden_dim, wl.router_h1), dtype=torch.uint8,
                      device=dev)
    route = torch.empty((1, L), dtype=torch.uint8, device=dev)

    def one_pass(ev=None):
        if ev:
            ev[0].record(stream)
        flux.route(hidden, cu, w1, b1, w2, b2, route_out=route, workspace=rws)
        _, rp, ci = flux.build_block_mask(S, sa, device=dev, dense=False)
        if ev:
            ev[1].record(stream)
        for layer in range(L):
            flux.attn_prefill(q, k, v, cu, S, route, layer, rp, ci, sa, out=out)
            if ev:
                ev[2 + layer].record(stream)

    log("prefill131k: untimed pass")
    one_pass()
    torch.cuda.synchronize()
    ev = _events(torch, stream, L + 2)
    one_pass(ev)
    torch.cuda.synchronize()
    r = route.cpu().numpy()[0]
    lay = [ev[1 + i].elapsed_time(ev[2 + i]) for i in range(L)]
    fa = [t for t, x in zip(lay, r) if x == 1]
    sa_t = [t for t, x in zip(lay, r) if x == 0]
    pass_ms = ev[0].elapsed_time(ev[L + 1])
    blk = 4.0 * wl.block_size ** 2 * d * wl.hq
    fa_fl, sa_fl = nb * (nb + 1) / 2 * blk, nnz * blk
    res = {"workload": "Qwen3-4B-shaped routed prefill, 131072 tokens, 36 layers routed by the "
                       "router (2560->256->36), SA window 4096 (1 sink + 32 blocks of 128)",
           "n_fa_layers": int(r.sum()), "pass_ms": round(pass_ms, 3),
           "tok_s": round(S / (pass_ms * 1e-3), 1),
           "router_mask_ms": round(ev[0].elapsed_time(ev[1]), 4)}
    if fa:
        res["fa_layer_ms"] = round(sum(fa) / len(fa), 3)
        res["fa_tflops"] = round(fa_fl / (sum(fa) / len(fa)) / 1e9, 1)
    if sa_t:
        res["sa_layer_ms"] = round(sum(sa_t) / len(sa_t), 3)
        res["sa_tflops"] = round(sa_fl / (sum(sa_t) / len(sa_t)) / 1e9, 1)
    log(f"prefill131k: {res['n_fa_layers']} FA layers, pass {pass_ms:.1f} ms ({res['tok_s']:.0f} tok/s), "
        f"FA {res.get('fa_tflops')} TF/s, SA {res.get('sa_tflops')} TF/s")
    del hidden, q, k, v, out
    torch.cuda.empty_cache()
    return res


def run_varlen8(flux, syn, dev, stream, log):
    """The varlen workload: 8 prompts (seeded lengths in [8192, 65536]), router
    4096 -> 256 -> 32 per request, all 32 layers of packed prefill routed per
    request (one q/k/v set shared by the layers), then 128 decode steps over 32
    layers whose caches start from the prompts and grow by one seeded K/V row
    per step (the append is tensor indexing, outside the kernels but inside
    the timed step)."""
    import numpy as np
    import torch

    wl = syn.varlen8()
    lens, L, d, n = list(wl.seqlens), wl.n_layers, wl.head_dim, len(wl.seqlens)
    T, max_s = sum(lens), max(lens)
    max_len = max_s + wl.decode_steps
    g = syn.generator(wl.seed, dev)
    hidden = syn.normal((T, wl.hidden_dim), g, dev)
    w1, b1, w2, b2 = (t.to(dev) for t in syn.router_weights(wl.hidden_dim, wl.router_h1, L, wl.seed))
    cu = syn.cu_seqlens(lens, dev)
    sa = flux.SAParams(wl.block_size, wl.sink_blocks, wl.local_blocks)
    _, rp, ci = flux.build_block_mask(max_len, sa, device=dev, dense=False)
    route, _ = flux.route(hidden, cu, w1, b1, w2, b2)
    del hidden
    q = syn.normal((T, wl.hq, d), g, dev)
    k = syn.normal((T, wl.hkv, d), g, dev)
    v = syn.normal((T, wl.hkv, d), g, dev)
    out = torch.empty_like(q)

    def prefill_pass():
        for layer in range(L):
            flux.attn_prefill(q, k, v, cu, max_s, route, layer, rp, ci, sa, out=out)

    prefill_pass()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    prefill_pass()
    e1.record(stream)
    torch.cuda.synchronize()
    pre_ms = e0.elapsed_time(e1)
    r = route.cpu().numpy()
    blk = 4.0 * wl.block_size ** 2 * d * wl.hq
    flops = 0.0
    for i, S in enumerate(lens):
        nb = -(-S // wl.block_size)
        nnz = flux.mask_nnz(S, sa)
        flops += (r[i].sum() * nb * (nb + 1) / 2 + (L - r[i].sum()) * nnz) * blk
    log(f"varlen8 prefill: {T} tokens x {L} layers in {pre_ms:.1f} ms ({T / pre_ms * 1e3:.0f} tok/s, "
        f"{flops / pre_ms / 1e9:.0f} TF/s)")

    # decode caches: per layer [n][hkv][max_len][d], the prompts' K/V first
    # (mixed per-request routes in a layer: full caches for every layer)
    kc, vc = [], []
    for _ in range(L):
        a, b = flux.kv_cache(n, wl.hkv, d, max_len, sa, device=dev)
        flux.kv_store_prefill(k, v, cu, max_s, a, b, max_len, sa)
        kc.append(a)
        vc.append(b)
    del q, k, v, out
    torch.cuda.empty_cache()
    ws = flux.decode_workspace(n, wl.hq, wl.hkv, d, max_len, dev)
    base = torch.tensor(lens, dtype=torch.int32, device=dev)
    knew = syn.normal((wl.decode_steps, L, n, wl.hkv, d), g, dev)
    vnew = syn.normal((wl.decode_steps, L, n, wl.hkv, d), g, dev)
    qd = syn.normal((wl.decode_steps, L, n, wl.hq, d), g, dev)
    dout = torch.empty((n, wl.hq, d), dtype=torch.bfloat16, device=dev)
    seq_t = [(base + t + 1).to(torch.int32) for t in range(wl.decode_steps)]
    e0.record(stream)
    for t in range(wl.decode_steps):
        seqlens = seq_t[t]
        for layer in range(L):
            # the new token's K/V row is appended by the same launch
            flux.attn_decode_append(qd[t, layer], knew[t, layer], vnew[t, layer], kc[layer], vc[layer],
                                    seqlens, route, layer, rp, ci, sa, ws, out=dout)
    e1.record(stream)
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / wl.decode_steps
    # bytes per step, averaged over the steps: every K/V row the step reads,
    # once (FA: the N cached keys; SA: the keys below N of its mask row's blocks)
    byts = decode_bytes_varlen(lens, r, wl, range(1, wl.decode_steps + 1)) / wl.decode_steps
    res = {"workload": "Llama-3-8B-shaped varlen mix: 8 prompts (seeded lengths in [8192, 65536]), "
                       "32 layers routed per request by the router (4096->256->32), then 128 decode steps",
           "lengths": lens, "fa_layers_per_request": r.sum(axis=1).tolist(),
           "prefill_ms": round(pre_ms, 3), "prefill_tok_s": round(T / (pre_ms * 1e-3), 1),
           "prefill_tflops": round(flops / pre_ms / 1e9, 1),
           "decode_ms_per_step": round(dec_ms, 4), "decode_tok_s": round(n / (dec_ms * 1e-3), 1),
           "decode_gbs": round(byts / (dec_ms * 1e-3) / 1e9, 1),
           "decode_note": "each layer's step appends its new K/V row in the same launch (flux_attn_decode_append); bytes are "
                          "the K/V rows each step reads at its own cache length, averaged over the 128 steps"}
    log(f"varlen8 decode: {dec_ms:.3f} ms/step ({res['decode_tok_s']:.0f} tok/s, {res['decode_gbs']:.0f} GB/s)")
    del kc, vc, knew, vnew, qd
    torch.cuda.empty_cache()
    return res


def decode_bytes_varlen(lens, route, wl, grow):
    """K/V bytes that decode steps read: for every step (cache length
    lens[i] + t for t in grow), request and layer, the rows of the keys the
    layer visits (FA: all N keys; SA: the keys below N of mask row (N-1)/B,
    i.e. its sink blocks and window blocks, the last one partial)."""
    B, s, w = wl.block_size, wl.sink_blocks, wl.local_blocks
    row_b = wl.hkv * wl.head_dim * 2 * 2
    total = 0
    for i, S in enumerate(lens):
        n_fa = int(route[i].sum())
        for t in grow:
            N = S + t
            mrow = (N - 1) // B
            blocks = min(mrow + 1, w) + min(s, max(0, mrow + 1 - w))
            sa_keys = (blocks - 1) * B + (N - mrow * B)
            total += (n_fa * N + (len(route[i]) - n_fa) * sa_keys) * row_b
    return total


def run_decode(args, flux, syn, dev, stream, log):
    import numpy as np
    import torch

    wl = syn.DECODE32K
    n_seq, ctx = len(wl.seqlens), wl.seqlens[0]
    hq, hkv, d, nl = wl.hq, wl.hkv, wl.head_dim, wl.n_layers
    sa = flux.SAParams(wl.block_size, wl.sink_blocks, wl.local_blocks)
    g = syn.generator(wl.seed, dev)
    log(f"decode: allocating {nl} layers x 2 x {n_seq * hkv * ctx * d * 2 / 2**30:.1f} GiB caches")
    kc = [syn.normal((n_seq, hkv, ctx, d), g, dev) for _ in range(nl)]
    vc = [syn.normal((n_seq, hkv, ctx, d), g, dev) for _ in range(nl)]
    q = [syn.normal((n_seq, hq, d), g, dev) for _ in range(nl)]
    out = [torch.empty((n_seq, hq, d), dtype=torch.bfloat16, device=dev) for _ in range(nl)]
    route_vec = syn.seeded_route(nl, wl.n_sa_layers, wl.seed)
    route = route_vec[None].repeat(n_seq, 1).to(dev).contiguous()
    seqlens = torch.full((n_seq,), ctx, dtype=torch.int32, device=dev)
    _, rp, ci = flux.build_block_mask(ctx, sa, device=dev, dense=False)
    ws = flux.decode_workspace(n_seq, hq, hkv, d, ctx, dev)

    def step(timers=None):
        for layer in range(nl):
            if timers is not None:
                e = torch.cuda.Event(enable_timing=True)
                e.record(stream)
                timers.append(e)
            flux.attn_decode(q[layer], kc[layer], vc[layer], seqlens, route, layer, rp, ci, sa, ws,
                             out[layer])
        if timers is not None:
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            timers.append(e)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"decode timed x{args.decode_steps}")
    # whole steps back to back, events only around them
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.decode_steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / args.decode_steps
    # the per-layer split (FA vs SA layer times) from separate steps with an
    # event between layers
    lay = np.zeros(nl)
    for _ in range(args.decode_steps):
        tm = []
        step(tm)
        torch.cuda.synchronize()
        lay += np.array([tm[i].elapsed_time(tm[i + 1]) for i in range(nl)])
    lay /= args.decode_steps

    # The same step captured once in a HIP graph and replayed: the host's
    # launch gaps between the 72 kernels disappear.  Every checked replay must
    # reproduce the eager outputs bit for bit.
    eager = [o.clone() for o in out]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(2):
        for o in out:
            o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(out, eager)):
            raise RuntimeError("decode graph replay differs from the eager step")
    e0.record(stream)
    for _ in range(args.decode_steps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1) / args.decode_steps
    del graph

    # The same step with the SA layers on compact caches (sink rows + a ring
    # of the window: 2176 rows per head instead of 32768); FA layers unchanged.
    # The two steps are timed alternately (twice each, the faster kept) so
    # that neither gains from running first.
    sa_set = set(i for i in range(nl) if int(route_vec[i]) == 0)
    cmp_caches = {}
    for layer in sa_set:
        shape = (n_seq, hkv, flux.kv_rows(ctx, sa, compact=True), d)
        cmp_caches[layer] = (syn.normal(shape, g, dev), syn.normal(shape, g, dev))
    ws2 = flux.decode_workspace(n_seq, hq, hkv, d, ctx, dev)

    def step_compact():
        for layer in range(nl):
            if layer in sa_set:
                a, b = cmp_caches[layer]
                flux.attn_decode_sa_compact(q[layer], a, b, seqlens, ctx, rp, ci, sa, ws2, out[layer])
            else:
                flux.attn_decode(q[layer], kc[layer], vc[layer], seqlens, route, layer, rp, ci, sa, ws,
                                 out[layer])

    def timed_steps(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.decode_steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.decode_steps

    compact_ms = timed_steps(step_compact)
    full_again_ms = timed_steps(step)
    compact_ms = min(compact_ms, timed_steps(step_compact))
    full_cache_gib = nl * 2 * n_seq * hkv * ctx * d * 2 / 2**30
    mixed_cache_gib = (len(sa_set) * 2 * n_seq * hkv * flux.kv_rows(ctx, sa, compact=True) * d * 2
                       + (nl - len(sa_set)) * 2 * n_seq * hkv * ctx * d * 2) / 2**30
    log(f"decode step with compact SA caches {compact_ms:.3f} ms (full caches, timed beside it: "
        f"{full_again_ms:.3f} ms); caches {full_cache_gib:.1f} GiB -> "
        f"{mixed_cache_gib:.1f} GiB")
    del cmp_caches
    fa_layers = [i for i in range(nl) if int(route_vec[i]) == 1]
    sa_layers = [i for i in range(nl) if int(route_vec[i]) == 0]
    sa_keys = (wl.sink_blocks + wl.local_blocks) * wl.block_size
    kv_bytes_tok = hkv * d * 2 * 2 * n_seq
    fa_bytes = ctx * kv_bytes_tok
    sa_bytes = sa_keys * kv_bytes_tok
    step_bytes = len(fa_layers) * fa_bytes + len(sa_layers) * sa_bytes
    fa_ms = float(lay[fa_layers].mean())
    sa_ms = float(lay[sa_layers].mean())
    gbs = step_bytes / (step_ms * 1e-3) / 1e9
    fa_gbs = fa_bytes / (fa_ms * 1e-3) / 1e9
    log(f"decode step {step_ms:.3f} ms ({16 / step_ms * 1e3:.0f} tok/s), graph replay {graph_ms:.3f} ms  "
        f"FA layer {fa_ms:.3f} ms ({fa_gbs:.0f} GB/s)  SA layer {sa_ms:.3f} ms "
        f"({sa_bytes / sa_ms / 1e6:.0f} GB/s)")
    res = {
        "workload": "Qwen3-4B-shaped decode, 16 seqs x 32768 ctx, 36 layers (18 FA / 18 SA seeded)",
        "value": round(n_seq / (step_ms * 1e-3), 1), "unit": "tok/s",
        "ms_per_step": round(step_ms, 4), "steps": args.decode_steps,
        "graph_ms_per_step": round(graph_ms, 4),
        "graph_tok_s": round(n_seq / (graph_ms * 1e-3), 1),
        "graph_gbs": round(step_bytes / (graph_ms * 1e-3) / 1e9, 1),
        "compact_sa_ms_per_step": round(compact_ms, 4),
        "full_ms_per_step_beside_compact": round(full_again_ms, 4),
        "cache_gib_full": round(full_cache_gib, 2), "cache_gib_compact_sa": round(mixed_cache_gib, 2),
        "fa_layer_ms": round(fa_ms, 4), "sa_layer_ms": round(sa_ms, 4),
        "bytes_per_step": step_bytes,
        "roofline": {"kernel": "decode_split_kernel<128> + decode_combine_kernel<128>",
                     "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "fa_layer_gbs": round(fa_gbs, 1),
                     "sa_layer_gbs": round(sa_bytes / sa_ms / 1e6, 1)},
    }
    tr = counted_traffic("decode_split_kernel")
    if tr is not None:
        res["roofline"]["traffic"] = round(len(fa_layers) * tr["fa_bytes"] + len(sa_layers) * tr["sa_bytes"])
        res["roofline"]["traffic_note"] = "bytes per decode step from profiles/hbm_traffic_32k.json"
    del kc, vc
    torch.cuda.empty_cache()
    return res


def cpu_baseline(args, q, k, v, S, wl, log):
    """The float64 oracle, as it stands, on a bounded sample of the same
    prefill workload: router + mask in full, then FA and SA layer rows sampled
    uniformly over the prompt (all heads) until the time budget is spent."""
    import numpy as np
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    cores = len(os.sched_getaffinity(0))
    log(f"cpu baseline: oracle on host ({cores} cores visible, BLAS threads {threads})")
    qf = q.float().cpu().numpy()
    kf = k.float().cpu().numpy()
    vf = v.float().cpu().numpy()
    rng = np.random.default_rng(0)
    t_start = time.perf_counter()
    nb = oracle.num_blocks(S, wl.block_size)
    m = oracle.block_mask(nb, wl.sink_blocks, wl.local_blocks)
    t_mask = time.perf_counter() - t_start
    rows_done = 0
    t_rows = 0.0
    while t_rows < args.cpu_seconds:
        rows = np.sort(rng.integers(0, S, size=8))
        t0 = time.perf_counter()
        oracle.attention_prefill(qf, kf, vf, True, m, wl.block_size, rows=rows)
        oracle.attention_prefill(qf, kf, vf, False, m, wl.block_size, rows=rows)
        t_rows += time.perf_counter() - t0
        rows_done += len(rows)
    per_row = t_rows / rows_done
    tok_s = 1.0 / per_row  # mask/router are per prompt: amortised below
    full_prompt_s = per_row * S + t_mask
    log(f"cpu baseline: {rows_done} rows in {t_rows:.1f} s -> {S / full_prompt_s:.2f} tok/s")
    return {"value": round(S / full_prompt_s, 3), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows_done} query rows sampled uniformly from the 32768-token prompt, all 32 heads, "
                      f"FA + SA layer each ({t_rows:.1f} s), plus the mask build; scaled to a full prompt",
            "per_row_ms": round(per_row * 1e3, 3), "rows_per_s": round(tok_s, 2)}


if __name__ == "__main__":
    sys.exit(main())
