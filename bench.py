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
flops of its launches / their summed duration, timed with HIP events on the
launch stream.  Flops per layer = (32-row wave, 32-key tile) pairs the kernel
executes * 4 * 32 * 32 * head_dim * hq (a wave skips the key tiles past its
last row, so a diagonal 128-block runs 10 of its 16 pairs); the active
128x128 block count and the attending (query, key) pair count are reported
beside it.  Decode bytes per step = K+V bytes the layers must read (FA: all
32768 keys, SA: 17 blocks of 128 keys).

Also timed, each in its own JSON object: the 131072-token 36-layer routed
prefill, an 8-prompt packed prefill + decode (varlen8), head- vs layer-level
routing, the soft-routed pass, the content-aware mask, compact SA caches, a
tiny 2-layer stack part by part, the router alone, and the float64 oracle on
the host cores (cpu_baseline).
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


def prefill_work(S, fa, B, s, w, d, hq, bn=32):
    """Work of one prefill layer of one request of S tokens, counted three
    ways, in flops (one multiply-add = 2 flops, QK^T and PV alike):
      blocks -- active B x B mask blocks x 4 B^2 d hq (a ragged last block
                counts whole): the computed-block count;
      tiles  -- (32-row wave, 32-key tile) pairs the prefill kernel executes
                x 4 * 32 * 32 * d * hq: a wave skips the tiles that start past
                its last row, so a diagonal block runs 10 of its 16 pairs at
                B = 128, and waves past the end of the request run none;
      causal -- (query, key) pairs the layer lets attend x 4 d hq.
    fa: every key block up to the diagonal; else the sink + window pattern."""
    nb = -(-S // B)
    tpb = B // bn
    blocks = tiles = causal = 0
    for t in range(nb):
        nbr = t + 1 if fa else min(t + 1, w) + min(s, max(0, t + 1 - w))
        blocks += nbr
        for wi in range(B // bn):
            if t * B + wi * bn < S:
                tiles += (nbr - 1) * tpb + wi + 1
        rows = min(t * B + B, S) - t * B
        causal += rows * (nbr - 1) * B + rows * (rows + 1) // 2
    return {"blocks": blocks * 4.0 * B * B * d * hq, "tiles": tiles * 4.0 * bn * bn * d * hq,
            "causal": causal * 4.0 * d * hq}


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
    ap.add_argument("--no-graph", action="store_true",
                    help="time the decode steps with eager launches only (profiler runs, which serialise every launch)")
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

    pws = flux.prefill_workspace(dev)  # the balancing workspace of this stream (left zero by every call)

    def prefill_call(layer):
        check(F.flux_attn_prefill(P(q), P(k), P(v), P(out[layer]), P(cu), 1, S, hq, hkv, d,
                                  1.0 / math.sqrt(d), P(route), wl.n_layers, layer, P(row_ptr),
                                  P(col_idx), nb, sa.c(), P(pws), pws.numel() * 4, cstream), "prefill")

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
    # work of the two layers: (wave, tile) pairs the kernel executes (the
    # headline), and for reference computed blocks and causal pairs
    fa_w = prefill_work(S, True, wl.block_size, wl.sink_blocks, wl.local_blocks, d, hq)
    sa_w = prefill_work(S, False, wl.block_size, wl.sink_blocks, wl.local_blocks, d, hq)
    fa_flops, sa_flops = fa_w["tiles"], sa_w["tiles"]
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
            "fa_frac_mfma_blocks": round(fa_w["blocks"] / fa_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "sa_frac_mfma_blocks": round(sa_w["blocks"] / sa_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "fa_frac_mfma_causal": round(fa_w["causal"] / fa_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "sa_frac_mfma_causal": round(sa_w["causal"] / sa_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "flops_count": "tflops / frac_mfma: 32x32 (wave, key tile) pairs the kernel executes x 4*32*32*d*hq "
                           "(a diagonal 128-block runs 10 of 16); _blocks: active 128x128 blocks x 4*128^2*d*hq; "
                           "_causal: attending (query, key) pairs x 4*d*hq",
            "fa_tok_s": round(S / (fa_ms * 1e-3), 1), "sa_tok_s": round(S / (sa_ms * 1e-3), 1),
        },
        "roofline": {
            "kernel": "prefill_kernel<128,128,32,3> (FA + SA launches; flops: executed (wave, tile) pairs)",
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
    result["tiny"] = run_tiny(flux, syn, dev, stream, log)
    result["router"] = router_latency(flux, syn, dev, stream, log)

    # ------------------------------------------------------------ decode phase
    if not args.no_decode:
        result["decode"] = run_decode(args, flux, syn, dev, stream, log)
        result["decode"]["roofline"]["frac_attainable"] = round(
            result["decode"]["roofline"]["achieved"] / att["hbm_read_gbs"], 4)

    # ------------------------------------------------------------ long workloads
    if not args.no_long:
        result["prefill131k"] = run_prefill_131k(flux, syn, dev, stream, log)
        result["varlen8"] = run_varlen8(flux, syn, dev, stream, log, graph=not args.no_graph)

    # ------------------------------------------------------------ oracle on the host
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, log)

    print(json.dumps(result), flush=True)
    return 0


def run_tiny(flux, syn, dev, stream, log, reps=200):
    """The tiny routed stack (1 x 512 tokens, 2 layers, 4/2 heads, d 64, router
    256 -> 64 -> 2, blocks of 64 with 1 sink + 2 local blocks), inputs in HBM:
    router, mask, the FA and the SA prefill layer, and one decode step of the
    last token for each layer.  Mean over `reps` back-to-back stacks, each
    part timed with events on the launch stream (a launch-latency workload:
    no roofline claim)."""
    import torch

    wl = syn.TINY
    S = wl.seqlens[0]
    g = syn.generator(wl.seed, dev)
    hidden = syn.normal((S, wl.hidden_dim), g, dev, torch.float32)
    q = syn.normal((S, wl.hq, wl.head_dim), g, dev)
    k = syn.normal((S, wl.hkv, wl.head_dim), g, dev)
    v = syn.normal((S, wl.hkv, wl.head_dim), g, dev)
    w1, b1, w2, b2 = (t.to(dev) for t in syn.router_weights(wl.hidden_dim, wl.router_h1, wl.n_layers, wl.seed))
    cu = syn.cu_seqlens([S], dev)
    sa = flux.SAParams(wl.block_size, wl.sink_blocks, wl.local_blocks)
    route = torch.tensor([[1, 0]], dtype=torch.uint8, device=dev)  # one FA and one SA layer
    r_out = torch.empty((1, wl.n_layers), dtype=torch.uint8, device=dev)
    rws = torch.empty(flux.route_workspace_size(1, wl.hidden_dim, wl.router_h1), dtype=torch.uint8, device=dev)
    kc = k.permute(1, 0, 2).contiguous()[None]
    vc = v.permute(1, 0, 2).contiguous()[None]
    qd = q[S - 1][None].contiguous()
    sl = torch.tensor([S], dtype=torch.int32, device=dev)
    nb = flux.mask_blocks(S, sa)
    rp = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(flux.mask_nnz(S, sa), dtype=torch.int32, device=dev)
    ws = flux.decode_workspace(1, wl.hq, wl.hkv, wl.head_dim, S, dev)
    pws = flux.prefill_workspace(dev)
    outs = [torch.empty_like(q) for _ in range(2)]
    douts = [torch.empty_like(qd) for _ in range(2)]
    L, F = flux._lib, flux._LIB
    cs = __import__("ctypes").c_void_p(stream.cuda_stream)

    def P(t):
        return __import__("ctypes").c_void_p(t.data_ptr())

    parts = [
        ("router", lambda: F.flux_route(P(hidden), L.FLUX_F32, P(cu), 1, wl.hidden_dim, P(w1), P(b1), wl.router_h1,
                                        P(w2), P(b2), wl.n_layers, P(r_out), None, P(rws), rws.numel(), cs)),
        ("mask", lambda: F.flux_build_block_mask(S, sa.c(), None, P(rp), P(ci), cs)),
    ] + [(f"prefill_{n}", (lambda layer: lambda: F.flux_attn_prefill(
            P(q), P(k), P(v), P(outs[layer]), P(cu), 1, S, wl.hq, wl.hkv, wl.head_dim,
            1.0 / math.sqrt(wl.head_dim), P(route), 2, layer, P(rp), P(ci), nb, sa.c(), P(pws),
            pws.numel() * 4, cs))(layer))
         for layer, n in ((0, "fa"), (1, "sa"))
    ] + [(f"decode_{n}", (lambda layer: lambda: F.flux_attn_decode(
            P(qd), P(kc), P(vc), P(douts[layer]), P(sl), 1, S, wl.hq, wl.hkv, wl.head_dim,
            1.0 / math.sqrt(wl.head_dim), P(route), 2, layer, P(rp), P(ci), nb, sa.c(), P(ws), ws.numel(),
            cs))(layer))
         for layer, n in ((0, "fa"), (1, "sa"))]
    for _ in range(5):
        for _, fn in parts:
            if fn() != 0:
                raise RuntimeError("tiny stack: a call failed")
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in range(reps)]
    for e in ev:
        e[0].record(stream)
        for i, (_, fn) in enumerate(parts):
            fn()
            e[i + 1].record(stream)
    torch.cuda.synchronize()
    res = {"workload": "tiny routed stack: 1 x 512 tokens, 2 layers (FA + SA), 4/2 heads, d 64, router "
                       "256->64->2, blocks of 64 (1 sink + 2 local), decode of the last token per layer",
           "reps": reps}
    for i, (name, _) in enumerate(parts):
        res[f"{name}_us"] = round(sum(e[i].elapsed_time(e[i + 1]) for e in ev) / reps * 1e3, 2)
    res["stack_us"] = round(sum(e[0].elapsed_time(e[-1]) for e in ev) / reps * 1e3, 2)
    res["prefill_stack_tok_s"] = round(S / ((res["router_us"] + res["mask_us"] + res["prefill_fa_us"]
                                              + res["prefill_sa_us"]) * 1e-6), 1)
    log(f"tiny stack: {res['stack_us']:.1f} us (router {res['router_us']}, mask {res['mask_us']}, prefill FA "
        f"{res['prefill_fa_us']} / SA {res['prefill_sa_us']}, decode FA {res['decode_fa_us']} / SA "
        f"{res['decode_sa_us']} us)")
    return res


def router_latency(flux, syn, dev, stream, log, reps=50):
    """flux_route alone (pool of the first and last 100 rows, MLP, threshold),
    inputs in HBM, mean of `reps` calls, at the three router shapes: 32768 x
    2560 -> 256 -> 2, 131072 x 2560 -> 256 -> 36, and 8 requests of the
    varlen8 lengths x 4096 -> 256 -> 32; reported per call and per routed
    layer beside the pages' figure (0.20 ms per layer, technical summary
    section 4)."""
    import torch

    v8 = syn.varlen8()
    shapes = [("prefill32k", syn.PREFILL32K.seqlens, 2560, 256, 2),
              ("prefill131k", syn.PREFILL128K.seqlens, 2560, 256, 36),
              ("varlen8", v8.seqlens, 4096, 256, 32)]
    res = {"pages_ms_per_layer": 0.20}
    for name, lens, D, H1, L in shapes:
        g = syn.generator(77, dev)
        hidden = syn.normal((sum(lens), D), g, dev)
        w1, b1, w2, b2 = (t.to(dev) for t in syn.router_weights(D, H1, L, 77))
        cu = syn.cu_seqlens(list(lens), dev)
        n = len(lens)
        r_out = torch.empty((n, L), dtype=torch.uint8, device=dev)
        ws = torch.empty(flux.route_workspace_size(n, D, H1), dtype=torch.uint8, device=dev)
        call = lambda: flux.route(hidden, cu, w1, b1, w2, b2, route_out=r_out, workspace=ws)  # noqa: E731
        call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"requests": n, "tokens": int(sum(lens)), "mlp": f"{D}->{H1}->{L}", "ms": round(ms, 4),
                     "ms_per_layer": round(ms / L, 5)}
        del hidden
    torch.cuda.empty_cache()
    log("router alone: " + ", ".join(f"{k} {v['ms'] * 1e3:.1f} us ({v['ms_per_layer'] * 1e3:.2f} us/layer)"
                                     for k, v in res.items() if isinstance(v, dict)))
    return res


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
    against the FA and SA layers run separately and against the FA layer
    alone (the pass visits the SA blocks first, parks the weighted SA output,
    and completes FA with the same softmax state: FA's work)."""
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
    return {"soft_pass_ms": round(ms, 4), "fa_plus_sa_ms": round(fa_ms + sa_ms, 4), "fa_layer_ms": round(fa_ms, 4),
            "vs_fa_layer": round(ms / fa_ms, 3),
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
    fa_w = prefill_work(S, True, wl.block_size, wl.sink_blocks, wl.local_blocks, d, wl.hq)
    sa_w = prefill_work(S, False, wl.block_size, wl.sink_blocks, wl.local_blocks, d, wl.hq)
    n_fa = int(r.sum())
    layers_ms = sum(lay)
    pass_fl = n_fa * fa_w["tiles"] + (L - n_fa) * sa_w["tiles"]
    res = {"workload": "Qwen3-4B-shaped routed prefill, 131072 tokens, 36 layers routed by the "
                       "router (2560->256->36), SA window 4096 (1 sink + 32 blocks of 128)",
           "n_fa_layers": n_fa, "pass_ms": round(pass_ms, 3),
           "tok_s": round(S / (pass_ms * 1e-3), 1),
           "router_mask_ms": round(ev[0].elapsed_time(ev[1]), 4),
           "layers_tflops": round(pass_fl / layers_ms / 1e9, 1),
           "frac_mfma": round(pass_fl / layers_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
           "flops_count": "executed (wave, tile) pairs, as prefill.flops_count"}
    if fa:
        res["fa_layer_ms"] = round(sum(fa) / len(fa), 3)
        res["fa_tflops"] = round(fa_w["tiles"] / (sum(fa) / len(fa)) / 1e9, 1)
        res["fa_frac_mfma"] = round(res["fa_tflops"] / PEAK_BF16_TFLOPS, 4)
    if sa_t:
        res["sa_layer_ms"] = round(sum(sa_t) / len(sa_t), 3)
        res["sa_tflops"] = round(sa_w["tiles"] / (sum(sa_t) / len(sa_t)) / 1e9, 1)
        res["sa_frac_mfma"] = round(res["sa_tflops"] / PEAK_BF16_TFLOPS, 4)
        res["sa_frac_mfma_blocks"] = round(sa_w["blocks"] / (sum(sa_t) / len(sa_t)) / 1e9 / PEAK_BF16_TFLOPS, 4)
    log(f"prefill131k: {res['n_fa_layers']} FA layers, pass {pass_ms:.1f} ms ({res['tok_s']:.0f} tok/s), "
        f"FA {res.get('fa_tflops')} TF/s, SA {res.get('sa_tflops')} TF/s")
    del hidden, q, k, v, out
    torch.cuda.empty_cache()
    return res


def run_varlen8(flux, syn, dev, stream, log, graph=True):
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
    flops = 0.0  # executed (wave, tile) pairs, as prefill.flops_count
    for i, S in enumerate(lens):
        n_fa = int(r[i].sum())
        flops += n_fa * prefill_work(S, True, wl.block_size, wl.sink_blocks, wl.local_blocks, d, wl.hq)["tiles"]
        flops += (L - n_fa) * prefill_work(S, False, wl.block_size, wl.sink_blocks, wl.local_blocks, d,
                                           wl.hq)["tiles"]
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
        if (t + 1) % 32 == 0:
            log(f"varlen8 decode: {t + 1} eager steps launched")
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / wl.decode_steps
    dec_ms = eager_ms

    # The same 128 steps with one step captured as a HIP graph: the 32
    # decode-append launches on device-resident lengths, then the lengths'
    # increment, replayed once per step (every step reads the rows of its own
    # lengths, as above; its q and new rows are one fixed set).  The first
    # replay is checked bit for bit against the same step launched eagerly.
    if graph:
        sl_dev = seq_t[0].clone()
        douts = [torch.empty_like(dout) for _ in range(L)]

        def gstep():
            for layer in range(L):
                flux.attn_decode_append(qd[0, layer], knew[0, layer], vnew[0, layer], kc[layer], vc[layer],
                                        sl_dev, route, layer, rp, ci, sa, ws, out=douts[layer])
        gstep()
        torch.cuda.synchronize()
        eager_out = [o.clone() for o in douts]
        g_step = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_step):
            gstep()
            sl_dev.add_(1)
        for o in douts:
            o.zero_()
        g_step.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(douts, eager_out)):
            raise RuntimeError("varlen8 decode graph replay differs from the eager step")
        sl_dev.copy_(seq_t[0])
        e0.record(stream)
        for _ in range(wl.decode_steps):
            g_step.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        dec_ms = e0.elapsed_time(e1) / wl.decode_steps
        del g_step, douts, eager_out
    # bytes per step, averaged over the steps: every K/V row the step reads,
    # once (FA: the N cached keys; SA: the keys below N of its mask row's blocks)
    byts = decode_bytes_varlen(lens, r, wl, range(1, wl.decode_steps + 1)) / wl.decode_steps
    res = {"workload": "Llama-3-8B-shaped varlen mix: 8 prompts (seeded lengths in [8192, 65536]), "
                       "32 layers routed per request by the router (4096->256->32), then 128 decode steps",
           "lengths": lens, "fa_layers_per_request": r.sum(axis=1).tolist(),
           "prefill_ms": round(pre_ms, 3), "prefill_tok_s": round(T / (pre_ms * 1e-3), 1),
           "prefill_tflops": round(flops / pre_ms / 1e9, 1),
           "prefill_frac_mfma": round(flops / pre_ms / 1e9 / PEAK_BF16_TFLOPS, 4),
           "decode_ms_per_step": round(dec_ms, 4), "decode_tok_s": round(n / (dec_ms * 1e-3), 1),
           "decode_gbs": round(byts / (dec_ms * 1e-3) / 1e9, 1),
           "decode_frac_hbm": round(byts / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "decode_eager_ms_per_step": round(eager_ms, 4),
           "decode_eager_frac_hbm": round(byts / (eager_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "decode_note": "each layer's step appends its new K/V row in the same launch (flux_attn_decode_append); "
                          + ("decode_* = one step captured as a HIP graph (32 launches + the lengths' increment) "
                             "replayed per step, the first replay bitwise equal to the eager step; decode_eager_* = "
                             "every launch from Python" if graph else "eager launches only (--no-graph)")
                          + "; bytes are the K/V rows each step reads at its own cache length, averaged over the "
                            "128 steps"}
    log(f"varlen8 decode: {dec_ms:.3f} ms/step ({'graph replay' if graph else 'eager'}), {eager_ms:.3f} eager "
        f"({res['decode_tok_s']:.0f} tok/s, {res['decode_gbs']:.0f} GB/s)")
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
    log(f"decode timed x{args.decode_steps} (twice, the faster pass kept)")
    # whole steps back to back, events only around them; two passes (the first
    # pass after the 72 GiB of caches were written has read up to 5 % slower)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    passes = []
    for _ in range(2):
        e0.record(stream)
        for _ in range(args.decode_steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        passes.append(e0.elapsed_time(e1) / args.decode_steps)
    step_ms = min(passes)
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
    graph_ms = step_ms
    if not args.no_graph:
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
    gbs = step_bytes / (graph_ms * 1e-3) / 1e9
    fa_gbs = fa_bytes / (fa_ms * 1e-3) / 1e9
    log(f"decode step {step_ms:.3f} ms ({16 / step_ms * 1e3:.0f} tok/s), graph replay {graph_ms:.3f} ms  "
        f"FA layer {fa_ms:.3f} ms ({fa_gbs:.0f} GB/s)  SA layer {sa_ms:.3f} ms "
        f"({sa_bytes / sa_ms / 1e6:.0f} GB/s)")
    res = {
        "workload": "Qwen3-4B-shaped decode, 16 seqs x 32768 ctx, 36 layers (18 FA / 18 SA seeded)",
        "value": round(n_seq / (graph_ms * 1e-3), 1), "unit": "tok/s",
        "ms_per_step": round(graph_ms, 4), "steps": args.decode_steps,
        "launch": ("the step's 72 launches captured once in a HIP graph and replayed (every checked replay "
                   "bitwise equal to the eager step); eager_* = the same step launched from Python")
        if not args.no_graph else "eager launches only (--no-graph)",
        "eager_ms_per_step": round(step_ms, 4), "eager_tok_s": round(n_seq / (step_ms * 1e-3), 1),
        "pass_ms_per_step": [round(x, 4) for x in passes],
        "eager_gbs": round(step_bytes / (step_ms * 1e-3) / 1e9, 1),
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


def host_info():
    """The host the oracle runs on: cores this process may use, the machine's
    count, the CPU model, and the BLAS threads numpy uses."""
    info = {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(), "cpu_model": None}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        info["blas_threads"] = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        info["blas_threads"] = 1
    return info


def oracle_pairs(S, chunk):
    """(query row, key) pairs the oracle's prefill evaluates for a whole prompt
    of S rows: rows in chunks of `chunk`, each chunk against keys 0 .. its
    last row, whatever the layer's route (it masks, it does not skip)."""
    return sum((min(S, c0 + chunk) - c0) * min(S, c0 + chunk) for c0 in range(0, S, chunk))


def oracle_prefill_rate(oracle, np, S, hq, hkv, d, B, s, w, starts, W, seed):
    """Seconds per (query row, key) pair (all heads) of the oracle's prefill,
    measured on windows of W consecutive rows starting at `starts`, each run
    as an FA and as an SA layer, on seeded N(0, 1) inputs of the shape."""
    import time as _t
    rng = np.random.default_rng(seed)
    n_keys = max(starts) + W
    q = np.empty((n_keys, hq, d), dtype=np.float32)  # only the window rows are touched
    for p0 in starts:
        q[p0:p0 + W] = rng.standard_normal((W, hq, d), dtype=np.float32)
    k = rng.standard_normal((n_keys, hkv, d), dtype=np.float32)
    v = rng.standard_normal((n_keys, hkv, d), dtype=np.float32)
    m = oracle.block_mask(oracle.num_blocks(S, B), s, w)
    spent, pairs = 0.0, 0
    for p0 in starts:
        rows = np.arange(p0, p0 + W)
        for fa in (True, False):
            t0 = _t.perf_counter()
            oracle.attention_prefill(q, k, v, fa, m, B, rows=rows)
            spent += _t.perf_counter() - t0
            pairs += W * (p0 + W)
    return spent / pairs, spent


def oracle_decode_time(oracle, np, N, hq, hkv, d, B, s, w, seed):
    """Seconds of one oracle decode of one sequence with N cached keys (all
    heads), as an FA and as an SA layer, on seeded N(0, 1) inputs."""
    import time as _t
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, hq, d), dtype=np.float32)
    kc = rng.standard_normal((1, hkv, N, d), dtype=np.float32)
    vc = rng.standard_normal((1, hkv, N, d), dtype=np.float32)
    m = oracle.block_mask(oracle.num_blocks(N, B), s, w)
    out = {}
    for name, fa in (("fa", True), ("sa", False)):
        t0 = _t.perf_counter()
        oracle.attention_decode(q, kc, vc, [N], fa, m, B)
        out[name] = _t.perf_counter() - t0
    return out


def cpu_baseline(args, log):
    """The float64 oracle, as it stands, timed on this host for every workload
    (after the GPU runs), with the host's core count.  The tiny stack runs in
    full; the larger workloads run a bounded sample of their own shapes and
    are extrapolated linearly by the work the oracle would do on the whole
    workload (labelled): prefill by (query row, key) pairs, which is what its
    cost follows, decode by cached keys."""
    import time as _t

    import numpy as np
    import oracle
    from oracle.attention import ROW_CHUNK
    from synth import inputs as syn

    host = host_info()
    log(f"cpu baseline: oracle on host ({host['affinity_cores']} cores usable of {host['cpu_count']}, "
        f"BLAS threads {host['blas_threads']}, {host['cpu_model']})")
    t_all = _t.perf_counter()
    res = {}

    # tiny stack, in full: router, mask, FA + SA prefill, FA + SA decode of the last token
    wl = syn.TINY
    S = wl.seqlens[0]
    rng = np.random.default_rng(wl.seed)
    hid = rng.standard_normal((S, wl.hidden_dim), dtype=np.float32)
    q, k, v = (rng.standard_normal((S, h, wl.head_dim), dtype=np.float32) for h in (wl.hq, wl.hkv, wl.hkv))
    w1, b1, w2, b2 = (x.numpy() for x in syn.router_weights(wl.hidden_dim, wl.router_h1, wl.n_layers, wl.seed))
    t0 = _t.perf_counter()
    oracle.route_requests(hid, [0, S], w1, b1, w2, b2)
    m = oracle.block_mask(oracle.num_blocks(S, wl.block_size), wl.sink_blocks, wl.local_blocks)
    for fa in (True, False):
        oracle.attention_prefill(q, k, v, fa, m, wl.block_size)
    t_pre = _t.perf_counter() - t0
    kc, vc = k.transpose(1, 0, 2)[None], v.transpose(1, 0, 2)[None]
    for fa in (True, False):
        oracle.attention_decode(q[S - 1][None], kc, vc, [S], fa, m, wl.block_size)
    t_tiny = _t.perf_counter() - t0
    res["tiny"] = {"stack_us": round(t_tiny * 1e6, 1), "prefill_tok_s": round(S / t_pre, 1),
                   "sample": "the whole stack (router, mask, FA + SA prefill, FA + SA decode)"}

    # router at the 32K shape (pools 200 rows of 32768 x 2560): timed in full
    wl = syn.PREFILL32K
    S, D = wl.seqlens[0], wl.hidden_dim
    hid = np.zeros((S, D), dtype=np.float32)
    hid[:100] = rng.standard_normal((100, D), dtype=np.float32)
    hid[-100:] = rng.standard_normal((100, D), dtype=np.float32)
    w1, b1, w2, b2 = (x.numpy() for x in syn.router_weights(D, wl.router_h1, wl.n_layers, wl.seed))
    t0 = _t.perf_counter()
    oracle.route_requests(hid, [0, S], w1, b1, w2, b2)
    t_router = _t.perf_counter() - t0
    t0 = _t.perf_counter()
    oracle.mask_to_csr(oracle.block_mask(oracle.num_blocks(S, wl.block_size), wl.sink_blocks, wl.local_blocks))
    t_mask = _t.perf_counter() - t0
    del hid

    # 32K layer pair: windows of 128 rows at 1/4 and 3/4 of the prompt
    rate, spent = oracle_prefill_rate(oracle, np, S, wl.hq, wl.hkv, wl.head_dim, wl.block_size,
                                      wl.sink_blocks, wl.local_blocks, [S // 4, 3 * S // 4], 128, 11)
    t_layer = rate * oracle_pairs(S, ROW_CHUNK)
    t_step = t_router + t_mask + 2 * t_layer
    res["prefill32k"] = {"tok_s": round(S / t_step, 3), "step_s": round(t_step, 2),
                         "ns_per_row_key": round(rate * 1e9, 3), "router_ms": round(t_router * 1e3, 2),
                         "extrapolated": True,
                         "sample": f"4 calls (FA, SA x 128-row windows at rows {S // 4}, {3 * S // 4}; {spent:.1f} s), "
                                   "scaled by (row, key) pairs to the router + mask + FA + SA step"}

    # 131K routed prefill: windows of 64 rows at 1/8 and 1/2 of the prompt
    wl4 = syn.PREFILL128K
    S4 = wl4.seqlens[0]
    rate4, spent4 = oracle_prefill_rate(oracle, np, S4, wl4.hq, wl4.hkv, wl4.head_dim, wl4.block_size,
                                        wl4.sink_blocks, wl4.local_blocks, [S4 // 8, S4 // 2], 64, 12)
    t4 = wl4.n_layers * rate4 * oracle_pairs(S4, ROW_CHUNK)
    res["prefill131k"] = {"tok_s": round(S4 / t4, 4), "pass_s": round(t4, 1), "ns_per_row_key": round(rate4 * 1e9, 3),
                          "extrapolated": True,
                          "sample": f"4 calls (FA, SA x 64-row windows at rows {S4 // 8}, {S4 // 2}; {spent4:.1f} s), "
                                    "scaled by (row, key) pairs to 36 layers (the oracle's cost does not depend "
                                    "on the route)"}

    # 32K decode: one FA and one SA layer of one sequence (all heads)
    wl3 = syn.DECODE32K
    N3 = wl3.seqlens[0]
    dt = oracle_decode_time(oracle, np, N3, wl3.hq, wl3.hkv, wl3.head_dim, wl3.block_size, wl3.sink_blocks,
                            wl3.local_blocks, 13)
    n_sa = wl3.n_sa_layers
    t3 = len(wl3.seqlens) * ((wl3.n_layers - n_sa) * dt["fa"] + n_sa * dt["sa"])
    res["decode32k"] = {"tok_s": round(len(wl3.seqlens) / t3, 4), "step_s": round(t3, 2), "extrapolated": True,
                        "sample": f"one sequence's FA and SA layer decode ({dt['fa'] + dt['sa']:.2f} s), scaled to "
                                  "16 sequences x (18 FA + 18 SA) layers"}

    # varlen8: windows of the longest prompt; decode of the longest sequence
    wl5 = syn.varlen8()
    lens = list(wl5.seqlens)
    S5 = max(lens)
    rate5, spent5 = oracle_prefill_rate(oracle, np, S5, wl5.hq, wl5.hkv, wl5.head_dim, wl5.block_size,
                                        wl5.sink_blocks, wl5.local_blocks, [S5 // 4, S5 // 2], 64, 14)
    t5 = wl5.n_layers * rate5 * sum(oracle_pairs(x, ROW_CHUNK) for x in lens)
    d5 = oracle_decode_time(oracle, np, S5, wl5.hq, wl5.hkv, wl5.head_dim, wl5.block_size, wl5.sink_blocks,
                            wl5.local_blocks, 15)
    per_key = (d5["fa"] + d5["sa"]) / 2 / S5
    t5d = per_key * wl5.n_layers * sum(x + wl5.decode_steps // 2 for x in lens)
    res["varlen8"] = {"prefill_tok_s": round(sum(lens) / t5, 4), "prefill_s": round(t5, 1),
                      "decode_tok_s": round(len(lens) / t5d, 3), "decode_step_s": round(t5d, 2), "extrapolated": True,
                      "sample": f"4 prefill calls (FA, SA x 64-row windows of the {S5}-token prompt; {spent5:.1f} s) "
                                f"scaled by (row, key) pairs to 8 prompts x 32 layers; one FA and one SA decode of "
                                f"the {S5}-key sequence scaled by cached keys to a step of 8 sequences x 32 layers"}
    total = _t.perf_counter() - t_all
    log(f"cpu baseline: {total:.1f} s; 32K prefill {res['prefill32k']['tok_s']:.2f} tok/s, decode "
        f"{res['decode32k']['tok_s']:.3f} tok/s, tiny stack {res['tiny']['stack_us'] / 1e3:.1f} ms")
    return {"value": res["prefill32k"]["tok_s"], "unit": "tok/s", "cores": host["blas_threads"], "kind": "oracle",
            "sample": "32K routed prefill step (router + mask + FA + SA layer) extrapolated by (row, key) pairs "
                      "from 128-row windows; every workload in `configs`",
            "host": host, "seconds": round(total, 1), "configs": res}


if __name__ == "__main__":
    sys.exit(main())
