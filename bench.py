"""Benchmark of the routed-expert FFN step on one MI355X.

Default workload: batch-1 decode through 8 routed-MoE layers (hidden 4096, 128
experts + 1 shared, intermediate 1536, top-8, 4-bit 32-column blocks), every
expert resident in HBM.  One step = router + top-k, expert lookup (device
pointer table), fused dequant + gate/up + SwiGLU, dequant + down, weighted
combine, for all 8 layers, on one token: one moe_route_ffn_combine call per
layer (three kernels), launched eagerly (the host stays ahead of the GPU; with
--graph, one HIP graph per step is replayed instead).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode1]

Prints ONE JSON line: tokens/s through all layers, the roofline of the dominant
kernel (dequant + gate/up + SwiGLU GEMV, timed live with HIP events on the
stream it runs on), and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, vendor figure
# the one-token gate/up kernel as launched alone (units per lane, ring depth, no routing)
GATE_UP_KERNEL = "decode1_gate_up_kernel<2, 1, 0, 0>"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="decode1")
    ap.add_argument("--inputs", type=int, default=8, help="distinct resident input steps cycled through")
    ap.add_argument("--graph", action="store_true",
                    help="replay one HIP graph per step instead of launching eagerly (each replay boundary leaves "
                         "the GPU idle ~8 us, more than the eager launches cost)")
    ap.add_argument("--kernel-iters", type=int, default=50, help="iterations of the per-kernel event timing")
    ap.add_argument("--cpu-tokens", type=int, default=16, help="tokens in the oracle CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream", action="store_true", help="skip the streamed-decode (PCIe) leg")
    ap.add_argument("--stream-workload", default="decode1_stream")
    ap.add_argument("--stream-layers", type=int, default=0,
                    help="layers of the streamed leg (0 = the configuration's; fewer when its host pool exceeds what "
                         "the machine lets one process pin)")
    ap.add_argument("--stream-steps", type=int, default=256)
    ap.add_argument("--stream-warmup", type=int, default=64)
    ap.add_argument("--chain-steps", type=int, default=128,
                    help="timed steps of each chained-layer run of the streamed leg (0 skips them)")
    ap.add_argument("--chain-warmup", type=int, default=32)
    ap.add_argument("--cpu-lane-threads", type=int, default=14,
                    help="worker threads of the streamed leg's CPU-lane run (0 skips it; decode workloads only)")
    ap.add_argument("--no-mx", action="store_true",
                    help="skip the MXFP4 and super-block decode legs (resident and streamed)")
    ap.add_argument("--no-layer-legs", action="store_true",
                    help="skip the one-resident-layer measurements of the 32-token decode and 2048-token prefill shapes")
    ap.add_argument("--traffic-calibration", action="store_true",
                    help="also run 4 plain 256 MiB device copies (reference for HBM traffic counters)")
    return ap.parse_args()


def link_peak(torch, slab_bytes: int):
    """Pinned host -> HBM copy rate on a side stream: best of 1 GiB copies, and
    back-to-back slab-sized copies (the cache's copy pattern)."""
    nbytes = 1 << 30
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    host.fill_(1)
    dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    best = 0.0
    with torch.cuda.stream(side):
        for _ in range(6):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(side)
            dev.copy_(host, non_blocking=True)
            b.record(side)
            b.synchronize()
            best = max(best, nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
        n = nbytes // slab_bytes
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(side)
        for i in range(n):
            dev[i * slab_bytes:(i + 1) * slab_bytes].copy_(host[i * slab_bytes:(i + 1) * slab_bytes],
                                                           non_blocking=True)
        b.record(side)
        b.synchronize()
        slabs = n * slab_bytes / (a.elapsed_time(b) * 1e-3) / 1e9
    # the same slabs each split in two halves on two streams (the cache's split copies)
    side2 = torch.cuda.Stream()
    h = (slab_bytes // 2) & ~4095
    split = 0.0
    for _ in range(3):  # the first pass warms the second stream up
        torch.cuda.synchronize()
        a, b, j = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                   torch.cuda.Event())
        a.record(side)
        side2.wait_event(a)
        for i in range(n):
            o = i * slab_bytes
            with torch.cuda.stream(side):
                dev[o:o + h].copy_(host[o:o + h], non_blocking=True)
            with torch.cuda.stream(side2):
                dev[o + h:o + slab_bytes].copy_(host[o + h:o + slab_bytes], non_blocking=True)
        j.record(side2)
        side.wait_event(j)
        b.record(side)
        b.synchronize()
        split = max(split, n * slab_bytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    del host, dev
    return best, slabs, split


def resident_step_ms(torch, cfg, layers: int, steps: int = 8) -> float:
    """Per-step time of a streamed configuration with every expert resident (the
    compute the copies have to hide), on the same synthetic inputs."""
    from routed_expert_streaming_amd.runtime import MoEStack

    st = MoEStack(cfg, cap=1.0, layers=layers)
    xs = [st.make_inputs(s) for s in range(4)]
    out = st.new_output()
    for s in range(2):
        st.forward(xs[s % 4], out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for s in range(steps):
        st.forward(xs[s % 4], out)
    b.record()
    torch.cuda.synchronize()
    st.close()
    del st, xs, out
    torch.cuda.empty_cache()
    return a.elapsed_time(b) / steps


def format_leg(torch, args, name: str, stream_name: str, fmt0_ms_per_step: float, fmt0_streaming):
    """The one-token decode with another expert weight format -- MXFP4 (E2M1
    codes, one E8M0 scale per 32 weights: 17/32 byte per weight against 20/32) or
    super-blocks (18/32) -- resident, one call per layer, then streamed at the
    same cache cap and router bias as the format-0 streamed leg.  Only that
    format's entry points run on these slabs."""
    import synth
    from routed_expert_streaming_amd.runtime import MoEStack

    cfg = synth.get(name)
    st = MoEStack(cfg)
    xs = [st.make_inputs(s) for s in range(args.inputs)]
    out = st.new_output()
    for s in range(args.warmup):
        st.forward(xs[s % len(xs)], out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for s in range(args.steps):
        st.forward(xs[s % len(xs)], out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    nbytes = step_bytes(st)
    res = {"workload": cfg.name, "layers": cfg.layers, "slab_bytes": st.slab, "tokens_per_s": round(1e3 / ms, 2),
           "ms_per_step": round(ms, 4), "speedup_vs_format0": round(fmt0_ms_per_step / ms, 4),
           "step_bytes": nbytes, "step_GBps": round(nbytes / ms / 1e6, 1), "steps": args.steps}
    st.close()
    del st, xs, out
    torch.cuda.empty_cache()
    if not args.no_stream:
        scfg = synth.get(stream_name)
        ss = MoEStack(scfg)
        sx = [ss.make_inputs(s) for s in range(32)]
        so = ss.new_output()
        for s in range(args.stream_warmup):
            ss.forward(sx[s % 32], so)
        torch.cuda.synchronize()
        h0, m0, b0 = ss.stats()
        t0 = time.perf_counter()
        for s in range(args.stream_steps):
            ss.forward(sx[s % 32], so)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        h1, m1, b1 = ss.stats()
        tps = args.stream_steps / wall
        res["streaming"] = {"workload": scfg.name, "tokens_per_s": round(tps, 2),
                            "ms_per_step": round(wall / args.stream_steps * 1e3, 3),
                            "hit_rate": round((h1 - h0) / max(h1 - h0 + m1 - m0, 1), 4),
                            "h2d_bytes_per_step": (b1 - b0) // args.stream_steps,
                            "h2d_GBps": round((b1 - b0) / wall / 1e9, 2),
                            "speedup_vs_format0": (round(tps / fmt0_streaming["tokens_per_s"], 4)
                                                   if fmt0_streaming else None),
                            "steps": args.stream_steps, "warmup": args.stream_warmup}
        ss.close()
    log(f"{name}: {res}")
    return res


def streaming_leg(torch, args, resident_ms_per_step: float):
    """The streamed decode workload: expert cache capped per layer, misses copied
    from pinned host RAM over PCIe on a copy stream while earlier layers compute.
    resident_ms_per_step: the same shapes with every expert resident (measured
    here when the streamed configuration's shapes differ from the timed one's)."""
    import synth
    from routed_expert_streaming_amd.runtime import MoEStack

    cfg = synth.get(args.stream_workload)
    main = synth.get(args.workload)
    layers = args.stream_layers or cfg.layers
    shape = lambda c, n: (n, c.tokens, c.hidden, c.inter, c.experts, c.shared, c.top_k)
    if shape(cfg, layers) != shape(main, main.layers):
        resident_ms_per_step = resident_step_ms(torch, cfg, layers)
        log(f"{cfg.name} ({layers} layers) with every expert resident: {resident_ms_per_step:.3f} ms/step")
    log(f"streaming leg: {cfg.description}" + (f", {layers} of its {cfg.layers} layers" if layers != cfg.layers else ""))
    st = MoEStack(cfg, layers=layers)
    peak, one_rate, split_rate = link_peak(torch, st.slab)
    slab_rate = split_rate if st.copy_stream2 is not None else one_rate
    log(f"pinned H2D: {peak:.1f} GB/s (1 GiB copies), {one_rate:.1f} GB/s (back-to-back {st.slab} B slabs), "
        f"{split_rate:.1f} GB/s (slabs split over two streams)")
    n_in = 32
    xs = [st.make_inputs(s) for s in range(n_in)]
    out = st.new_output()
    for s in range(args.stream_warmup):  # cold start happens here
        st.forward(xs[s % n_in], out)
    torch.cuda.synchronize()
    h0, m0, b0 = st.stats()
    t0 = time.perf_counter()
    for s in range(args.stream_steps):
        st.forward(xs[s % n_in], out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    h1, m1, b1 = st.stats()
    # chained layers with the deepest lookahead need 2*T*k slots per layer
    chained = (chained_runs(torch, st, args, xs)
               if args.chain_steps > 0 and 2 * cfg.tokens * cfg.top_k <= st.C else None)
    lane = (cpu_lane_run(torch, st, args, xs, args.stream_steps * cfg.tokens / wall)
            if args.cpu_lane_threads > 0 and st.T <= 64 and st.fmt == 0 else None)
    st.close()
    hits, misses, nbytes = h1 - h0, m1 - m0, b1 - b0
    ms_step = wall / args.stream_steps * 1e3
    copy_ms = nbytes / args.stream_steps / (slab_rate * 1e9) * 1e3  # copy-stream busy time at the slab copy rate
    h2d = nbytes / wall / 1e9
    res = {"workload": cfg.name, "layers": layers, "cache_slots_per_layer": st.C,
           "tokens_per_s": round(args.stream_steps * cfg.tokens / wall, 2), "ms_per_step": round(ms_step, 3),
           "hit_rate": round(hits / max(hits + misses, 1), 4), "h2d_bytes_per_step": nbytes // args.stream_steps,
           "h2d_GBps": round(h2d, 2), "link_peak_GBps": round(peak, 2), "slab_copy_GBps": round(slab_rate, 2),
           "slab_copy_one_stream_GBps": round(one_rate, 2), "split_copies": st.copy_stream2 is not None,
           "h2d_frac_of_link_peak": round(h2d / peak, 4),
           "copy_busy_ms_per_step": round(copy_ms, 3), "resident_ms_per_step": round(resident_ms_per_step, 3),
           "wall_over_copy_busy": round(ms_step / copy_ms, 4) if copy_ms > 0 else None,
           "exposed_ms_per_step": round(ms_step - copy_ms, 3),
           # share of the shorter of copy and compute hidden under the other
           "overlap_frac": (round((copy_ms + resident_ms_per_step - ms_step) / min(copy_ms, resident_ms_per_step), 4)
                            if copy_ms > 0 and resident_ms_per_step > 0 else None),
           "steps": args.stream_steps, "warmup": args.stream_warmup}
    if chained:
        res["chained"] = chained
    if lane:
        res["cpu_lane"] = lane
    log(f"streaming: {res}")
    return res


def cpu_lane_run(torch, st, args, xs, streamed_tokens_per_s: float):
    """The same streamed steps with a CPU lane: each step's misses split between
    the copy engine and host cores computing them from the pinned pool, by the
    earliest-finish cost model (runtime.assign_lanes)."""
    from routed_expert_streaming_amd import _lib as L
    st.enable_cpu_lane(args.cpu_lane_threads)
    out = st.new_output()
    n_in = len(xs)
    for s in range(args.stream_warmup):
        st.forward(xs[s % n_in], out)
    torch.cuda.synchronize()
    h0, m0, b0 = st.stats()
    cpu_e = cpu_p = 0
    t0 = time.perf_counter()
    for s in range(args.stream_steps):
        r = st.forward(xs[s % n_in], out)
        cpu_e += r.cpu_experts
        cpu_p += r.cpu_pairs
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    h1, m1, b1 = st.stats()
    n = args.stream_steps
    tps = n * st.T / wall
    res = {"threads": st.lane_threads, "isa_bits": L.moe_cpu_lane_isa(),
           "t_cpu_expert_ms": {"1_token": round(st.t_cpu1 * 1e3, 3), "8_tokens": round(st.t_cpu8 * 1e3, 3)},
           "t_copy_expert_ms": round(st.slab / (st.link_GBps * 1e9) * 1e3, 3), "link_GBps_assumed": st.link_GBps,
           "tokens_per_s": round(tps, 2), "ms_per_step": round(wall / n * 1e3, 3),
           "speedup_vs_streaming": round(tps / streamed_tokens_per_s, 4),
           "cpu_experts_per_step": round(cpu_e / n, 3), "cpu_pairs_per_step": round(cpu_p / n, 3),
           "streamed_experts_per_step": round((m1 - m0) / n, 3),
           "hit_rate_of_gpu_requests": round((h1 - h0) / max(h1 - h0 + m1 - m0, 1), 4),
           "h2d_GBps": round((b1 - b0) / wall / 1e9, 2), "steps": n, "warmup": args.stream_warmup}
    if args.chain_steps > 0 and st.T * st.k <= st.C:
        # chained layers (no lookahead): each layer's misses split between the
        # copy engine and the lane as soon as the layer is routed
        resid, hs = st.chain_buffers()
        st.reset_cache()
        for s in range(args.chain_warmup):
            st.forward_chained(xs[s % n_in][0], hs, resid, out)
        torch.cuda.synchronize()
        h0, m0, b0 = st.stats()
        cpu_e = 0
        t0 = time.perf_counter()
        for s in range(args.chain_steps):
            cpu_e += st.forward_chained(xs[s % n_in][0], hs, resid, out).cpu_experts
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        h1, m1, b1 = st.stats()
        n = args.chain_steps
        res["chained_no_lookahead"] = {"tokens_per_s": round(n * st.T / wall, 2), "ms_per_step": round(wall / n * 1e3, 3),
                                       "cpu_experts_per_step": round(cpu_e / n, 3),
                                       "streamed_experts_per_step": round((m1 - m0) / n, 3),
                                       "steps": n, "warmup": args.chain_warmup}
    log(f"cpu lane: {res}")
    return res


def chained_runs(torch, st, args, xs):
    """The streamed workload with chained layers (layer l+1's input computed from
    layer l's output through a residual stream), so each layer is routed only
    when the one before it is done: without lookahead every miss is exposed;
    with lookahead the next layer's router is applied to the current layer's
    input and the experts it ranks highest are prefetched (gating lookahead);
    the bound is an exact predictor of the same routing."""
    cfg = st.cfg
    resid, hs = st.chain_buffers()
    out = st.new_output()
    n_in = len(xs)
    res = {"model": "pre-norm residual stream between layers (moe_residual_norm, eps 1e-6)",
           "steps": args.chain_steps, "warmup": args.chain_warmup}
    k = cfg.top_k
    for name, la in [("no_lookahead", 0)] + [(f"lookahead_{m}", m) for m in sorted({1, 2, k // 2, k}) if 0 < m <= k]:
        st.reset_cache()
        for s in range(args.chain_warmup):
            st.forward_chained(xs[s % n_in][0], hs, resid, out, lookahead=la)
        torch.cuda.synchronize()
        h0, m0, b0 = st.stats()
        tot = None
        t0 = time.perf_counter()
        for s in range(args.chain_steps):
            c = st.forward_chained(xs[s % n_in][0], hs, resid, out, lookahead=la)
            tot = c if tot is None else type(c)(*[a + b for a, b in zip(vars(tot).values(), vars(c).values())])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        h1, m1, b1 = st.stats()
        n = args.chain_steps
        r = {"tokens_per_s": round(n * cfg.tokens / wall, 2), "ms_per_step": round(wall / n * 1e3, 3),
             "hit_rate": round((h1 - h0) / max(h1 - h0 + m1 - m0, 1), 4), "h2d_bytes_per_step": (b1 - b0) // n,
             "exposed_copies_per_step": round(tot.copies / n, 3)}
        if la:
            r.update({"named_recall": round(tot.predicted / max(tot.routed, 1), 4),
                      "ahead_copies_per_step": round(tot.ahead_copies / n, 3),
                      "ahead_unused_per_step": round(tot.ahead_unused / n, 3)})
        res[name] = r
        log(f"chained, {name}: {r}")
    # exact-predictor bound on the same routing: the chained layer inputs of
    # every step input, recorded, then run with every layer routed up front
    rec = []
    for s in range(n_in):
        st.forward_chained(xs[s][0], hs, resid, out, lookahead=0)
        rec.append(hs.clone())
    st.reset_cache()
    for s in range(args.chain_warmup):
        st.forward(rec[s % n_in], out)
    torch.cuda.synchronize()
    h0, m0, b0 = st.stats()
    t0 = time.perf_counter()
    for s in range(args.chain_steps):
        st.forward(rec[s % n_in], out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    h1, m1, b1 = st.stats()
    n = args.chain_steps
    res["exact_predictor"] = {"tokens_per_s": round(n * cfg.tokens / wall, 2), "ms_per_step": round(wall / n * 1e3, 3),
                              "hit_rate": round((h1 - h0) / max(h1 - h0 + m1 - m0, 1), 4),
                              "h2d_bytes_per_step": (b1 - b0) // n}
    log(f"chained, exact predictor: {res['exact_predictor']}")
    return res


def layer_leg(torch, name: str, path: int, iters: int):
    """One resident layer of a multi-token configuration (every expert in HBM, no
    PCIe): each kernel of the layer timed alone with events over `iters` launches.
    Algorithmic bytes = the slabs of the experts the tokens use (+ shared) plus
    activations; flops = 2·3·H·I per (token, expert) pair."""
    import synth
    from routed_expert_streaming_amd import _lib as L
    from routed_expert_streaming_amd.runtime import MoEStack

    cfg = synth.get(name)
    st = MoEStack(cfg, cap=1.0, layers=1)
    T, H, I, E, k = cfg.tokens, cfg.hidden, cfg.inter, cfg.experts, cfg.top_k
    x = st.make_inputs(0)
    out = st.new_output()
    st.route(x, 0)
    P = T * k + (T if st.has_shared else 0)
    h = torch.empty((P, I), dtype=torch.bfloat16, device="cuda")
    cnt = torch.empty(E, dtype=torch.int32, device="cuda")
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    por = torch.empty(T * k, dtype=torch.int32, device="cuda")
    shared = st.shared[0] if st.has_shared else None
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(iters):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    res = {"workload": f"{name}, one resident layer", "tokens": T, "path": {L.MOE_FFN_MFMA: "mfma",
                                                                              L.MOE_FFN_GROUPED: "grouped",
                                                                              L.MOE_FFN_SPLIT: "split"}[path]}
    res["router_ms"] = timed(lambda: st.route(x, 0))
    res["permute_ms"] = timed(lambda: L.moe_permute(st.idx[0], T, k, E, cnt, off, por))
    res["gate_up_ms"] = timed(lambda: L.moe_expert_gate_up(x[0], T, H, I, E, st.idx[0], k, cnt, off, por,
                                                           st.table[0], shared, None, h, path))
    res["down_ms"] = timed(lambda: L.moe_expert_down(h, T, H, I, E, st.idx[0], k, cnt, off, por, st.table[0],
                                                     shared, None, st.y, path))
    res["combine_ms"] = timed(lambda: st.combine(0, out))
    res["layer_ms"] = timed(lambda: (st.route(x, 0), st.ffn_combine(x, 0, out)))
    idx = st.idx[0].cpu().numpy()
    n_exp = len(set(int(e) for e in idx.ravel())) + (1 if st.has_shared else 0)
    w_bytes = n_exp * st.slab
    flops = 2 * 3 * H * I * P
    ffn_ms = res["gate_up_ms"] + res["down_ms"]
    res.update({"experts_used": n_exp, "weight_bytes": w_bytes, "ffn_flops": flops,
                "ffn_weights_GBps": round(w_bytes / (ffn_ms * 1e-3) / 1e9, 1),
                "ffn_TFLOPs": round(flops / (ffn_ms * 1e-3) / 1e12, 2),
                "hbm_frac": round(w_bytes / (ffn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "bf16_mfma_frac": round(flops / (ffn_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)})
    for key in list(res):
        if key.endswith("_ms"):
            res[key] = round(res[key], 4)
    st.close()
    del st, x, out, h
    torch.cuda.empty_cache()
    log(f"layer leg: {res}")
    return res


def counter_traffic(kernel: str):
    """HBM bytes per launch measured with FETCH_SIZE/WRITE_SIZE (scaled by a plain
    copy of known size), from the committed profile summary; None if the kernel's
    sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "decode1_gate_up_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic_json:"):
            info = json.loads(line.split(":", 1)[1])
            if info.get("kernel") != kernel:
                return None
            h = hashlib.sha1()
            for src in info["sources"]:
                h.update(open(os.path.join(ROOT, src), "rb").read())
            return info["traffic_bytes_per_launch"] if h.hexdigest() == info["sources_sha1"] else None
    return None


def bytes_per_32(stack) -> int:
    """Weight bytes per 32 weights: 16 code bytes plus a 4-byte (fp16 scale, fp16
    min) record, plus a 1-byte E8M0 scale for MXFP4, plus 2 bytes (a 16-byte
    header per 256) for super-blocks."""
    return {0: 20, 1: 17, 2: 18}[stack.fmt]


def gate_up_bytes(stack) -> int:
    """Algorithmic bytes of one gate/up launch: W1+W3 of every distinct expert the
    step uses, the activations read and h written."""
    idx = stack.idx.cpu().numpy()
    per_expert = 2 * (stack.I * stack.H * bytes_per_32(stack) // 32)
    experts = [len(set(int(e) for e in idx[l].ravel())) for l in range(stack.L)]
    P = stack.T * stack.k + (stack.T if stack.has_shared else 0)
    n = np.mean(experts) + (1 if stack.has_shared else 0)
    return int(n * per_expert + stack.T * stack.H * 2 + P * stack.I * 2)


def down_bytes(stack) -> int:
    idx = stack.idx.cpu().numpy()
    per_expert = stack.I * stack.H * bytes_per_32(stack) // 32
    experts = [len(set(int(e) for e in idx[l].ravel())) for l in range(stack.L)]
    P = stack.T * stack.k + (stack.T if stack.has_shared else 0)
    n = np.mean(experts) + (1 if stack.has_shared else 0)
    return int(n * per_expert + P * stack.I * 2 + P * stack.H * 4)


def step_bytes(stack) -> int:
    """Algorithmic HBM bytes of one step: expert slabs used, router weights, x, out."""
    idx = stack.idx.cpu().numpy()
    total = 0
    for l in range(stack.L):
        n = len(set(int(e) for e in idx[l].ravel())) + (1 if stack.has_shared else 0)
        total += n * stack.slab + stack.E * stack.H * 4 + stack.T * stack.H * 2 * 2
    return total


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    from routed_expert_streaming_amd.runtime import MoEStack

    cfg = synth.get(args.workload)
    if cfg.streaming:
        raise SystemExit("the timed workload must be resident; streamed configurations run in the tests")
    if cfg.fmt != 0:
        raise SystemExit("MXFP4 and super-block workloads are measured by the run's mx and superblock legs (the "
                         "per-kernel legs use format-0 calls)")
    t0 = time.time()
    log(f"building {cfg.name}: {cfg.description}")
    stack = MoEStack(cfg)
    xs = [stack.make_inputs(s) for s in range(args.inputs)]
    outs = [stack.new_output() for _ in range(args.inputs)]
    log(f"built in {time.time() - t0:.1f}s")
    dev_stream = torch.cuda.current_stream()

    # warm-up (eager); with --graph, capture one graph per resident input
    for i in range(max(args.warmup, 1)):
        stack.forward(xs[i % args.inputs], outs[i % args.inputs])
    torch.cuda.synchronize()
    graphs = None
    if args.graph:
        graphs = []
        for i in range(args.inputs):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                stack.forward(xs[i], outs[i])
            graphs.append(g)
        for i in range(args.inputs):
            graphs[i].replay()
        torch.cuda.synchronize()
    log("warm-up done")

    # ---------------- timed region: K steps
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(dev_stream)
    for s in range(args.steps):
        i = s % args.inputs
        if graphs is not None:
            graphs[i].replay()
        else:
            stack.forward(xs[i], outs[i])
    ev1.record(dev_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gpu_ms = ev0.elapsed_time(ev1)
    elapsed = max(wall, gpu_ms / 1e3)
    tokens = args.steps * cfg.tokens
    value = tokens / elapsed
    ms_per_step = elapsed / args.steps * 1e3
    log(f"{args.steps} steps: {ms_per_step * 1e3:.1f} us/step, {value:.1f} tokens/s (events {gpu_ms:.2f} ms, "
        f"wall {wall * 1e3:.2f} ms)")

    if args.traffic_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(3)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- dominant kernel, timed live with events on its stream
    h = torch.empty((cfg.tokens * cfg.top_k + cfg.tokens * cfg.shared, cfg.inter), dtype=torch.bfloat16,
                    device="cuda")
    stack.forward(xs[0], outs[0])  # routing of input 0 for every layer
    # back-to-back launches of one kernel between two events: the average launch
    # duration on the stream the kernel runs on.  The launches are captured in one
    # HIP graph and replayed on that stream, so host launch cost (which a profiler
    # inflates) does not show up as idle time between them.
    def time_launches(fn, iters):
        for l in range(stack.L):
            fn(l)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(iters):
                for l in range(stack.L):
                    fn(l)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(dev_stream)
        g.replay()
        b.record(dev_stream)
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) * 1e3 / (iters * stack.L)

    gu_us = time_launches(lambda l: stack.gate_up_only(xs[0], l, h), args.kernel_iters)
    dn_us = time_launches(lambda l: stack.down_only(h, l), args.kernel_iters)
    gu_b, dn_b = gate_up_bytes(stack), down_bytes(stack)
    achieved = gu_b / (gu_us * 1e-6) / 1e9
    log(f"gate/up kernel: {gu_us:.2f} us/launch, {gu_b} B -> {achieved:.0f} GB/s; "
        f"down kernel: {dn_us:.2f} us, {dn_b} B -> {dn_b / (dn_us * 1e-6) / 1e9:.0f} GB/s")
    sb = step_bytes(stack)
    ffn_bytes_step = (gu_b + dn_b) * stack.L
    ffn_us_step = (gu_us + dn_us) * stack.L

    result = {
        "metric": "routed-MoE layer tokens/s at 1 GPU (decode, all layers); achieved HBM GB/s vs peak",
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 activations x 4-bit block weights, fp32 accumulation",
        "data": "synthetic (seeded Philox inputs and random 4-bit expert weights)",
        "config": {"workload": cfg.name, "layers": cfg.layers, "tokens_per_step": cfg.tokens,
                   "hidden": cfg.hidden, "inter": cfg.inter, "experts": cfg.experts, "shared": cfg.shared,
                   "top_k": cfg.top_k, "resident": True, "graph": graphs is not None,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm",
                     "kernel": f"{GATE_UP_KERNEL} (dequant + gate/up + SwiGLU, launched alone "
                               "through moe_expert_gate_up; in the step the same kernel, with a two-deep load "
                               "ring, also finishes the top-k)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic(GATE_UP_KERNEL),
                     "bytes_per_launch": gu_b, "us_per_launch": round(gu_us, 3)},
        "ffn": {"bytes_per_step": ffn_bytes_step, "kernel_us_per_step": round(ffn_us_step, 2),
                "achieved_GBps": round(ffn_bytes_step / (ffn_us_step * 1e-6) / 1e9, 1),
                "down_us_per_launch": round(dn_us, 3), "down_bytes_per_launch": dn_b},
        "step_hbm_bytes": sb,
        "step_hbm_GBps": round(sb / (ms_per_step * 1e-3) / 1e9, 1),
    }

    # ---------------- CPU baseline: the oracle on a bounded sample
    if not args.no_cpu_baseline:
        import oracle
        threads = len(os.sched_getaffinity(0))
        n = args.cpu_tokens
        cpu_s = 0.0
        for l in range(stack.L):
            x = np.concatenate([synth.x_bf16(cfg.seed, s, l, cfg.tokens, cfg.hidden) for s in range(n)])
            slabs = stack.host_slabs(l)
            wr = synth.router_w(cfg.seed, l, cfg.experts, cfg.hidden)
            bias, shared = synth.router_bias(cfg, l), stack.host_shared(l)
            t1 = time.perf_counter()  # input generation stays outside the timed calls
            oracle.moe_layer(x, wr, bias, cfg.top_k, slabs, shared, cfg.inter, threads=threads)
            cpu_s += time.perf_counter() - t1
        result["cpu_baseline"] = {"value": round(n * cfg.tokens / cpu_s, 4), "unit": "tokens/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"{n} decode tokens (steps 0..{n - 1}) through all {stack.L} layers, "
                                            f"fp64 plain-C oracle, {cpu_s:.1f} s"}
        log(f"cpu baseline: {result['cpu_baseline']}")
    stack.close()
    del stack, graphs, xs, outs
    torch.cuda.empty_cache()
    if not args.no_stream:
        result["streaming"] = streaming_leg(torch, args, ms_per_step)
    if not args.no_mx:
        result["mx"] = format_leg(torch, args, "decode1_mx", "decode1_mx_stream", ms_per_step, result.get("streaming"))
        result["superblock"] = format_leg(torch, args, "decode1_sb", "decode1_sb_stream", ms_per_step,
                                          result.get("streaming"))
    if not args.no_layer_legs:
        from routed_expert_streaming_amd import _lib as L
        result["layer_decode32"] = layer_leg(torch, "decode32_stream", L.MOE_FFN_SPLIT, 20)
        result["layer_prefill2048"] = layer_leg(torch, "prefill2048_stream", L.MOE_FFN_MFMA, 3)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
