"""Benchmark of the routed-expert FFN step on one MI355X.

Default workload: a 2048-token prefill chunk through 16 streamed routed-MoE
layers (hidden 6144, 256 experts, intermediate 2048, top-8, 4-bit 32-column
blocks, bias-free routing), the expert cache capped at 102 of 256 experts per
layer and the full expert set in pinned host RAM (layers 8-15 reuse the expert
weights of layers 0-7).  One step = the routers of all 16 layers, one D2H of the
top-k ids, the library's per-layer plan (waves of at most half the slots, hits
first, a small first and last wave),
then per wave: its misses streamed over PCIe on two copy streams, the wait, the
MFMA grouped-GEMM FFN of its experts (dequant + gate/up + SwiGLU, dequant +
down), the release; and per layer the weighted combine.  Inputs of every timed
step are resident in HBM before the timed region.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill2048_stream]

Prints ONE JSON line: tokens/s through all layers; `roofline` = the dominant
kernel (the MFMA gate/up grouped GEMM, each launch of the timed steps bracketed
by HIP events on the stream it runs on) against the HBM peak, with its MFMA
fraction and the PCIe link's (H2D bytes over the measured copy-busy time against
the measured pinned link peak); the CPU oracle timed on a bounded sample; and
extra legs: the resident batch-1 decode, the streamed batch-1 decode, the tiny
one-layer case, the other weight formats and single resident layers.
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
METRIC = "routed-MoE layer tokens/s at 1 GPU; achieved HBM GB/s and PCIe H2D GB/s vs peak"
# the one-token gate/up kernel as launched alone (units per lane, ring depth, no routing)
GATE_UP_KERNEL = "decode1_gate_up_kernel<2, 1, 0, 0>"
# the prefill gate/up kernel (matrix cores; W1/W3 rows, SwiGLU epilogue), by weight format
MFMA_GATE_UP_KERNEL = "mfma_ffn_kernel<true, {fmt}, false>"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill2048_stream",
                    help="streamed headline configuration (prefill2048_stream, decode32_stream, decode1_stream)")
    ap.add_argument("--layers", type=int, default=0, help="layers of the headline stack (0 = the configuration's)")
    ap.add_argument("--inputs", type=int, default=0,
                    help="distinct resident input steps cycled through (0: 4 when a step has at least 128 tokens, "
                         "whose every step needs more experts than a layer holds; otherwise one per step, so that "
                         "the cache cannot end up holding a repeating working set)")
    ap.add_argument("--cpu-tokens", type=int, default=1, help="tokens in the oracle CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="only the headline (no extra legs)")
    ap.add_argument("--decode-steps", type=int, default=400, help="timed steps of the resident batch-1 decode leg")
    ap.add_argument("--decode-warmup", type=int, default=40)
    ap.add_argument("--graph", action="store_true",
                    help="resident decode leg: replay one HIP graph per step instead of launching eagerly (the "
                         "capture slows the streamed legs that follow it)")
    ap.add_argument("--kernel-iters", type=int, default=50, help="iterations of the per-kernel event timing")
    ap.add_argument("--no-stream", action="store_true", help="skip the streamed batch-1 decode (PCIe) leg")
    ap.add_argument("--stream-workload", default="decode1_stream")
    ap.add_argument("--stream-steps", type=int, default=256)
    ap.add_argument("--stream-warmup", type=int, default=64)
    ap.add_argument("--no-c4", action="store_true", help="skip the streamed batch-32 decode leg")
    ap.add_argument("--no-lane", action="store_true", help="no CPU-lane runs beside the streamed headline and C4 leg")
    ap.add_argument("--no-stream-half-cap", dest="stream_half_cap", action="store_false",
                    help="skip the streamed batch-1 decode at half the slots")
    ap.add_argument("--c4-steps", type=int, default=16, help="timed steps of the streamed batch-32 decode leg")
    ap.add_argument("--c4-warmup", type=int, default=8)
    ap.add_argument("--chain-steps", type=int, default=128,
                    help="timed steps of each chained-layer run of the streamed decode leg (0 skips them)")
    ap.add_argument("--chain-warmup", type=int, default=32)
    ap.add_argument("--cpu-lane-threads", type=int, default=14,
                    help="worker threads of the streamed decode leg's CPU-lane run (0 skips it)")
    ap.add_argument("--no-mx", action="store_true",
                    help="skip the MXFP4 and super-block decode legs (resident and streamed)")
    ap.add_argument("--no-layer-legs", action="store_true",
                    help="skip the one-resident-layer measurements of the 32-token decode and 2048-token prefill shapes")
    ap.add_argument("--traffic-calibration", action="store_true",
                    help="also run 4 plain 256 MiB device copies (reference for HBM traffic counters)")
    return ap.parse_args()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
    xs = [st.make_inputs(s) for s in range(8)]
    out = st.new_output()
    for s in range(args.decode_warmup):
        st.forward(xs[s % len(xs)], out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for s in range(args.decode_steps):
        st.forward(xs[s % len(xs)], out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.decode_steps
    nbytes = step_bytes(st)
    res = {"workload": cfg.name, "layers": cfg.layers, "slab_bytes": st.slab, "tokens_per_s": round(1e3 / ms, 2),
           "ms_per_step": round(ms, 4), "speedup_vs_format0": round(fmt0_ms_per_step / ms, 4),
           "step_bytes": nbytes, "step_GBps": round(nbytes / ms / 1e6, 1), "steps": args.decode_steps}
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


def copy_timing_summary(torch, st, nbytes: int, steps: int, ms_step: float, link: tuple, compute_ms_step: float,
                        timed_ms_step: float):
    """PCIe figures of a streamed run from the library's copy timing over `steps`
    steps that streamed `nbytes` with every copy bracketed by HIP events: H2D
    bytes over the copy-busy time (the union of the timed copy intervals on both
    copy streams) against the measured link peak; those steps' own time
    (timed_ms_step) over their busy time, and the overlap of copies and compute.
    ms_step is the step time of the run without copy events (the headline): the
    bytes over it, and it over the time the bytes take at the link peak."""
    from routed_expert_streaming_amd import _lib as L
    busy_ms, span_ms, n_timed = L.moe_cache_copy_busy(st.cache)
    peak, one_rate, split_rate = link
    busy_step = busy_ms / steps
    over_busy = nbytes / (busy_ms * 1e-3) / 1e9 if busy_ms > 0 else None
    res = {"h2d_bytes_per_step": nbytes // steps, "h2d_GBps_over_wall": round(nbytes / steps / ms_step / 1e6, 2),
           "copy_busy_ms_per_step": round(busy_step, 3), "copies_timed": n_timed,
           "h2d_GBps_over_copy_busy": round(over_busy, 2) if over_busy else None,
           "link_peak_GBps": round(peak, 2), "slab_copy_one_stream_GBps": round(one_rate, 2),
           "slab_copy_split_GBps": round(split_rate, 2), "split_copies": st.copy_stream2 is not None,
           # hipMemcpyAsync from pinned host memory runs on the SDMA engines unless HSA_ENABLE_SDMA=0 (blit kernels)
           "copy_engine": "blit kernels" if os.environ.get("HSA_ENABLE_SDMA", "1") == "0" else "SDMA",
           "frac_of_link_peak": round(over_busy / peak, 4) if over_busy else None,
           # the copy-timed steps against their own copy-busy time
           "copy_timed_ms_per_step": round(timed_ms_step, 3),
           "wall_over_copy_busy": round(timed_ms_step / busy_step, 4) if busy_step > 0 else None,
           "exposed_ms_per_step": round(timed_ms_step - busy_step, 3),
           # the step without copy events against the time its bytes take at the link peak
           "wall_over_link_time": round(ms_step / (nbytes / steps / (peak * 1e9) * 1e3), 4) if nbytes else None}
    if compute_ms_step is not None and busy_step > 0 and compute_ms_step > 0:
        res["compute_ms_per_step"] = round(compute_ms_step, 3)
        # share of the shorter of copy and compute hidden under the other (copy-timed steps)
        res["overlap_frac"] = round((busy_step + compute_ms_step - timed_ms_step) / min(busy_step, compute_ms_step), 4)
    return res


def streaming_leg(torch, args, resident_ms_per_step: float):
    """The streamed batch-1 decode: expert cache capped per layer, misses copied
    from pinned host RAM over PCIe on two copy streams while earlier layers
    compute.  resident_ms_per_step: the same shapes with every expert resident
    (the compute the copies have to hide)."""
    import synth
    from routed_expert_streaming_amd import _lib as L
    from routed_expert_streaming_amd.runtime import MoEStack

    cfg = synth.get(args.stream_workload)
    log(f"streaming leg: {cfg.description}")
    st = MoEStack(cfg)
    link = link_peak(torch, st.slab)
    log(f"pinned H2D: {link[0]:.1f} GB/s (1 GiB copies), {link[1]:.1f} GB/s (back-to-back {st.slab} B slabs), "
        f"{link[2]:.1f} GB/s (slabs split over two streams)")
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
    # copy-busy time from a second run with the copies timed (timing events
    # between copies of 11 MB slab halves lengthen these short steps, so the
    # step time above comes from the run without them)
    tsteps = min(args.stream_steps, 64)
    L.moe_cache_copy_timing(st.cache, True)
    _, _, c0 = st.stats()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(tsteps):
        st.forward(xs[s % n_in], out)
    torch.cuda.synchronize()
    timed_ms = (time.perf_counter() - t1) / tsteps * 1e3
    _, _, c1 = st.stats()
    pcie = copy_timing_summary(torch, st, c1 - c0, tsteps, wall / args.stream_steps * 1e3, link,
                               resident_ms_per_step, timed_ms)
    L.moe_cache_copy_timing(st.cache, False)
    pcie["copy_timed_steps"] = tsteps
    # chained layers with the deepest lookahead need 2*T*k slots per layer
    chained = (chained_runs(torch, st, args, xs)
               if args.chain_steps > 0 and 2 * cfg.tokens * cfg.top_k <= st.C else None)
    lane = (cpu_lane_run(torch, st, args, xs, args.stream_steps * cfg.tokens / wall)
            if args.cpu_lane_threads > 0 and st.T <= 64 and st.fmt == 0 else None)
    st.close()
    # the same configuration at half the slots (the harder end of the 60-80% hit
    # range of the configuration's description): tokens/s, hit rate, link time
    half = None
    if args.stream_half_cap:
        sh = MoEStack(cfg, cap=cfg.cap / 2)
        for s in range(args.stream_warmup):
            sh.forward(xs[s % n_in], out)
        torch.cuda.synchronize()
        g0, q0, c0 = sh.stats()
        t2 = time.perf_counter()
        for s in range(args.stream_steps):
            sh.forward(xs[s % n_in], out)
        torch.cuda.synchronize()
        w2 = time.perf_counter() - t2
        g1, q1, c1 = sh.stats()
        nb = (c1 - c0) / args.stream_steps
        half = {"cache_slots_per_layer": sh.C, "tokens_per_s": round(args.stream_steps * cfg.tokens / w2, 2),
                "ms_per_step": round(w2 / args.stream_steps * 1e3, 3),
                "hit_rate": round((g1 - g0) / max(g1 - g0 + q1 - q0, 1), 4), "h2d_bytes_per_step": int(nb),
                "wall_over_link_time": round((w2 / args.stream_steps) / (nb / (link[0] * 1e9)), 4) if nb else None}
        sh.close()
        del sh
    hits, misses = h1 - h0, m1 - m0
    res = {"workload": cfg.name, "layers": st.L, "cache_slots_per_layer": st.C,
           "tokens_per_s": round(args.stream_steps * cfg.tokens / wall, 2),
           "ms_per_step": round(wall / args.stream_steps * 1e3, 3),
           "hit_rate": round(hits / max(hits + misses, 1), 4), "resident_ms_per_step": round(resident_ms_per_step, 3),
           "pcie": pcie, "steps": args.stream_steps, "warmup": args.stream_warmup}
    if half:
        res["half_cap"] = half
    if chained:
        res["chained"] = chained
    if lane:
        res["cpu_lane"] = lane
    log(f"streaming: {res}")
    return res


def decode32_stream_leg(torch, args):
    """The streamed batch-32 decode through all 16 layers (hidden 6144, 256
    experts + 1 shared, intermediate 2048, top-8, Zipf(1.1) routing, 102 slots per
    layer): tokens/s and the PCIe figures, measured as the headline measures its
    own configuration (no oracle sample)."""
    import copy
    import synth

    a = copy.copy(args)
    a.steps, a.warmup, a.layers, a.inputs = args.c4_steps, args.c4_warmup, 0, 0
    a.no_cpu_baseline, a.traffic_calibration = True, False
    cfg = synth.get("decode32_stream")
    r = headline(torch, a, cfg)
    res = {"workload": r["config"]["workload"], "layers": r["config"]["layers"], "tokens_per_step": r["config"]["tokens_per_step"],
           "tokens_per_s": r["value"], "ms_per_step": r["ms_per_step"], "steps": a.steps, "warmup": a.warmup,
           **r["streaming"]}
    if "cpu_lane" in r:
        res["cpu_lane"] = r["cpu_lane"]
    log(f"decode32 streamed: {res}")
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

    res = {"workload": f"{name}, one resident layer", "tokens": T, "format": st.fmt, "slab_bytes": st.slab,
           "path": {L.MOE_FFN_MFMA: "mfma",
                                                                              L.MOE_FFN_GROUPED: "grouped",
                                                                              L.MOE_FFN_SPLIT: "split"}[path]}
    res["router_ms"] = timed(lambda: st.route(x, 0))
    res["permute_ms"] = timed(lambda: L.moe_permute(st.idx[0], T, k, E, cnt, off, por))
    res["gate_up_ms"] = timed(lambda: L.moe_expert_gate_up_fmt(x[0], T, H, I, E, st.idx[0], k, cnt, off, por,
                                                               st.table[0], shared, None, h, path, st.fmt))
    res["down_ms"] = timed(lambda: L.moe_expert_down_fmt(h, T, H, I, E, st.idx[0], k, cnt, off, por, st.table[0],
                                                         shared, None, st.y, path, st.fmt))
    # the FFN as one call (permutation included); for MXFP4 on the MFMA path this
    # is the block-scaled matrix-core route (activation digit pairs, no dequant)
    res["ffn_call_ms"] = timed(lambda: L.moe_expert_ffn_fmt(x[0], T, H, I, E, st.idx[0], k, st.table[0], shared,
                                                            None, st.y, st.ffn_ws, st.ffn_ws_bytes, path, st.fmt))
    res["combine_ms"] = timed(lambda: st.combine(0, out))
    res["layer_ms"] = timed(lambda: (st.route(x, 0), st.ffn_combine(x, 0, out)))
    idx = st.idx[0].cpu().numpy()
    n_exp = len(set(int(e) for e in idx.ravel())) + (1 if st.has_shared else 0)
    w_bytes = n_exp * st.slab
    flops = 2 * 3 * H * I * P
    ffn_ms = res["gate_up_ms"] + res["down_ms"]
    if st.fmt == 1 and path == L.MOE_FFN_MFMA:
        ffn_ms = res["ffn_call_ms"]  # the separate calls dequantise to bf16; the one call is the scaled route
        res["scaled_matrix_cores"] = True
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


def counter_traffic(kernel: str, profile: str):
    """HBM bytes per launch measured with FETCH_SIZE/WRITE_SIZE (scaled by a plain
    copy of known size), from a committed profile summary; None if the kernel's
    sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
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


def row_bytes(K: int, fmt: int) -> int:
    """Bytes of a K-column weight row: K/2 code bytes plus the block parameters
    (format 0: 4 bytes per 32 columns, 1: 1 byte per 32, 2: 16 bytes per 256),
    formats 0 and 1 padded to 16 bytes."""
    if fmt == 2:
        return K // 2 + K // 16
    per = 4 if fmt == 0 else 1
    return (K // 2 + K // 32 * per + 15) // 16 * 16


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


def oracle_sample(torch, cfg, layers: int, x_layers, wr, bias, slabs_of, shared_of, rows, threads: int):
    """The oracle on a bounded sample: the tokens `rows` of one step through every
    layer (router, expert FFNs, combine), input fetching outside the timed calls.
    Returns seconds."""
    import oracle
    cpu_s = 0.0
    for l in range(layers):
        x = np.ascontiguousarray(x_layers[l][rows])
        slabs, shared = slabs_of(l), shared_of(l)
        t1 = time.perf_counter()
        oracle.moe_layer(x, wr[l], bias[l], cfg.top_k, slabs, shared, cfg.inter, threads=threads)
        cpu_s += time.perf_counter() - t1
    return cpu_s


def headline(torch, args, cfg):
    """The streamed configuration through all its layers: tokens/s, the MFMA
    gate/up kernel's roofline from the timed steps, the PCIe link's fraction."""
    import synth
    from routed_expert_streaming_amd import _lib as L
    from routed_expert_streaming_amd.runtime import MoEStack

    t0 = time.time()
    layers = args.layers or cfg.layers
    log(f"building {cfg.name} ({layers} layers): {cfg.description}")
    st = MoEStack(cfg, layers=layers)
    log(f"built in {time.time() - t0:.1f}s: {st.C} slots per layer, {len(st.host)} host weight sets of "
        f"{st.E} x {st.slab} B pinned")
    link = link_peak(torch, st.slab)
    log(f"pinned H2D: {link[0]:.1f} GB/s (1 GiB copies), {link[1]:.1f} GB/s (back-to-back slabs), "
        f"{link[2]:.1f} GB/s (slabs split over two streams)")
    want = args.inputs or (4 if cfg.tokens >= 128 else args.steps + args.warmup)
    n_in = max(1, min(want, args.steps + args.warmup))
    xs = [st.make_inputs(s) for s in range(n_in)]
    out = st.new_output()
    dev_stream = torch.cuda.current_stream()
    for s in range(args.warmup):  # the cold start happens here
        st.forward(xs[s % n_in], out)
    torch.cuda.synchronize()
    log("warm-up done")
    mfma = st.T >= 128 and st.H % 128 == 0 and st.I % 128 == 0
    h0, m0, b0 = st.stats()
    st.kernel_log = [] if mfma else None
    idx_steps, marks = [], []

    # ---------------- timed region: K steps
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(dev_stream)
    for s in range(args.steps):
        marks.append(len(st.kernel_log) if mfma else 0)
        st.forward(xs[s % n_in], out)
        idx_steps.append(st.last_routing())
    ev1.record(dev_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gpu_ms = ev0.elapsed_time(ev1)
    elapsed = max(wall, gpu_ms / 1e3)
    value = args.steps * st.T / elapsed
    ms_per_step = elapsed / args.steps * 1e3
    h1, m1, b1 = st.stats()
    log(f"{args.steps} steps: {ms_per_step:.2f} ms/step, {value:.1f} tokens/s (events {gpu_ms:.1f} ms, "
        f"wall {wall * 1e3:.1f} ms)")

    # ---------------- the dominant kernel, from the events around each launch
    kern = None
    compute_ms_step = None
    if mfma:
        marks.append(len(st.kernel_log))
        gu_w = 2 * st.I * row_bytes(st.H, st.fmt)  # W1 and W3 of one expert
        tot_b = tot_f = 0
        tot_gu = tot_ffn = 0.0
        n = 0
        for s in range(args.steps):
            for a, b, c, l, experts, sh in st.kernel_log[marks[s]:marks[s + 1]]:
                sel = np.isin(idx_steps[s][l], experts)
                pairs = int(sel.sum()) + (st.T if sh else 0)
                toks = st.T if sh else int(sel.any(axis=1).sum())
                tot_b += (len(experts) + (1 if sh else 0)) * gu_w + toks * st.H * 2 + pairs * st.I * 2
                tot_f += 4 * st.H * st.I * pairs
                tot_gu += a.elapsed_time(b)
                tot_ffn += a.elapsed_time(c)
                n += 1
        compute_ms_step = tot_ffn / args.steps
        gbps = tot_b / (tot_gu * 1e-3) / 1e9
        tflops = tot_f / (tot_gu * 1e-3) / 1e12
        kern = {"launches": n, "bytes_per_launch": tot_b // n, "us_per_launch": round(tot_gu * 1e3 / n, 2),
                "flops_per_launch": tot_f // n, "GBps": gbps, "TFLOPs": tflops,
                "ffn_ms_per_step": round(compute_ms_step, 3),
                "gate_up_ms_per_step": round(tot_gu / args.steps, 3)}
        log(f"gate/up: {n} launches, {kern['us_per_launch']} us and {tot_b // n} B each -> {gbps:.0f} GB/s, "
            f"{tflops:.1f} TFLOP/s; FFN {compute_ms_step:.2f} ms/step")
    st.kernel_log = None
    if args.traffic_calibration:  # plain device copies of known size, the reference of the HBM counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(3)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # copy-busy time from further steps with every copy bracketed by HIP events on
    # its copy stream (those events lengthen each of the step's ~5000 slab-half
    # copies by a few microseconds, so the step time above comes from steps
    # without them)
    tsteps = min(args.steps, 4)
    L.moe_cache_copy_timing(st.cache, True)
    _, _, c0 = st.stats()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(tsteps):
        st.forward(xs[(args.steps + s) % n_in], out)
    torch.cuda.synchronize()
    timed_ms = (time.perf_counter() - t1) / tsteps * 1e3
    _, _, c1 = st.stats()
    pcie = copy_timing_summary(torch, st, c1 - c0, tsteps, ms_per_step, link, compute_ms_step, timed_ms)
    L.moe_cache_copy_timing(st.cache, False)
    pcie["copy_timed_steps"] = tsteps
    # control: a few steps with neither copy timing nor kernel events
    ctrl = min(3, args.steps)
    if ctrl:
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for s in range(ctrl):
            st.forward(xs[s % n_in], out)
        torch.cuda.synchronize()
        pcie["control_ms_per_step_untimed"] = round((time.perf_counter() - t1) / ctrl * 1e3, 3)
    log(f"pcie: {pcie}")

    # the same stack with the CPU lane (row f2): each step's misses split between
    # the copy engine and host cores computing them from the pinned pool (decode
    # shapes only: on the 2048-token chunk it measured slower, 1797 against 1962
    # tokens/s -- an expert's 64 tokens cost the host ~6.6 ms against 0.43 ms of
    # copy, so the lane can take only ~8% of the misses)
    lane = None
    if args.cpu_lane_threads > 0 and st.fmt == 0 and not args.no_lane and st.T <= 64:
        import copy
        la = copy.copy(args)
        la.stream_steps, la.stream_warmup, la.chain_steps = args.steps, args.warmup, 0
        lane = cpu_lane_run(torch, st, la, xs, value)

    hits, misses = h1 - h0, m1 - m0
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 activations x 4-bit block weights (bf16 on the matrix cores), fp32 accumulation",
        "data": "synthetic (seeded Philox inputs and random 4-bit expert weights)",
        "config": {"workload": cfg.name, "layers": layers, "tokens_per_step": st.T, "hidden": st.H,
                   "inter": st.I, "experts": st.E, "shared": cfg.shared, "top_k": st.k,
                   "cache_slots_per_layer": st.C, "streamed": True, "expert_weight_sets": len(st.host),
                   "host_pool_bytes": len(st.host) * st.E * st.slab, "router_bias": cfg.bias,
                   "parallelism": "single GPU"},
    }
    if kern:
        kname = MFMA_GATE_UP_KERNEL.format(fmt=st.fmt)
        result["roofline"] = {
            "bound": "hbm", "kernel": f"{kname} (dequant + gate/up + SwiGLU grouped GEMM on the "
                                      "matrix cores, one launch per wave of a layer's experts; every launch of the "
                                      "timed steps bracketed by HIP events on its stream)",
            "achieved": round(kern["GBps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kern["GBps"] / HBM_PEAK_GBS, 4),
            "traffic": counter_traffic(kname, "prefill2048_mfma_counters.md"),
            "bytes_per_launch": kern["bytes_per_launch"], "us_per_launch": kern["us_per_launch"],
            "launches": kern["launches"],
            "mfma": {"achieved": round(kern["TFLOPs"], 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kern["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, 4),
                     "flops_per_launch": kern["flops_per_launch"]},
            "pcie": {"bound": "pcie", "achieved": pcie["h2d_GBps_over_copy_busy"], "peak": pcie["link_peak_GBps"],
                     "unit": "GB/s", "frac": pcie["frac_of_link_peak"],
                     "wall_over_copy_busy": pcie["wall_over_copy_busy"]},
        }
        result["ffn"] = {"gate_up_ms_per_step": kern["gate_up_ms_per_step"], "ffn_ms_per_step": kern["ffn_ms_per_step"]}
    result["streaming"] = {"hit_rate": round(hits / max(hits + misses, 1), 4), **pcie}
    if lane:
        result["cpu_lane"] = lane

    # ---------------- CPU baseline: the oracle on a bounded sample
    if not args.no_cpu_baseline:
        threads = len(os.sched_getaffinity(0))
        n = max(1, args.cpu_tokens)
        rows = [int(r) for r in np.linspace(0, st.T - 1, n).round()]
        xb = xs[0].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        wr = [st.wr[l].cpu().numpy() for l in range(layers)]
        bias = [None if st.bias is None else st.bias[l].cpu().numpy() for l in range(layers)]
        cpu_s = oracle_sample(torch, cfg, layers, xb, wr, bias, st.host_pool_slabs, st.host_shared, rows, threads)
        result["cpu_baseline"] = {"value": round(n / cpu_s, 5), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                                  "cpu_model": cpu_model(),
                                  "sample": f"{n} token(s) of step 0 (rows {rows}) through all {layers} layers "
                                            f"(router, 8 expert FFNs, combine), fp64 plain-C oracle, {threads} "
                                            f"OpenMP threads, {cpu_s:.1f} s"}
        log(f"cpu baseline: {result['cpu_baseline']}")
    st.close()
    del st, xs, out
    torch.cuda.empty_cache()
    return result


def decode_leg(torch, args):
    """Batch-1 decode through 8 resident layers (hidden 4096, 128 experts + 1
    shared, intermediate 1536, top-8): one moe_route_ffn_combine call per layer
    (router partials, gate/up finishing the top-k, down + combine)."""
    import synth
    from routed_expert_streaming_amd.runtime import MoEStack

    cfg = synth.get("decode1")
    stack = MoEStack(cfg)
    n_in = 8
    xs = [stack.make_inputs(s) for s in range(n_in)]
    outs = [stack.new_output() for _ in range(n_in)]
    dev_stream = torch.cuda.current_stream()
    for i in range(max(args.decode_warmup, 1)):
        stack.forward(xs[i % n_in], outs[i % n_in])
    torch.cuda.synchronize()
    graphs = None
    if args.graph:
        graphs = []
        for i in range(n_in):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                stack.forward(xs[i], outs[i])
            graphs.append(g)
        for i in range(n_in):
            graphs[i].replay()
        torch.cuda.synchronize()
    steps = args.decode_steps
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(dev_stream)
    for s in range(steps):
        i = s % n_in
        if graphs is not None:
            graphs[i].replay()
        else:
            stack.forward(xs[i], outs[i])
    ev1.record(dev_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gpu_ms = ev0.elapsed_time(ev1)
    elapsed = max(wall, gpu_ms / 1e3)
    ms_per_step = elapsed / steps * 1e3
    log(f"decode leg: {steps} steps, {ms_per_step * 1e3:.1f} us/step, {steps / elapsed:.1f} tokens/s")
    sb = step_bytes(stack)
    res = {"workload": cfg.name, "layers": cfg.layers, "resident": True, "graph": graphs is not None,
           "tokens_per_s": round(steps / elapsed, 2), "ms_per_step": round(ms_per_step, 4), "steps": steps,
           "warmup": args.decode_warmup, "step_hbm_bytes": sb, "step_hbm_GBps": round(sb / (ms_per_step * 1e-3) / 1e9, 1)}
    if not args.no_cpu_baseline:
        threads = len(os.sched_getaffinity(0))
        x_layers = [np.concatenate([synth.x_bf16(cfg.seed, s, l, 1, cfg.hidden) for s in range(8)])
                    for l in range(stack.L)]
        wr = [synth.router_w(cfg.seed, l, cfg.experts, cfg.hidden) for l in range(stack.L)]
        bias = [synth.router_bias(cfg, l) for l in range(stack.L)]
        slabs = {l: stack.host_slabs(l) for l in range(stack.L)}
        shared = {l: stack.host_shared(l) for l in range(stack.L)}
        t_all = oracle_sample(torch, cfg, stack.L, x_layers, wr, bias, slabs.get, shared.get, list(range(8)), threads)
        t_one = oracle_sample(torch, cfg, stack.L, x_layers, wr, bias, slabs.get, shared.get, [0], 1)
        res["cpu_baseline"] = {"tokens_per_s": round(8 / t_all, 4), "threads": threads, "cpu_model": cpu_model(),
                               "sample": f"8 decode tokens (steps 0..7) through all {stack.L} layers, {t_all:.1f} s",
                               "one_thread_tokens_per_s": round(1 / t_one, 4),
                               "one_thread_sample": f"1 decode token through all {stack.L} layers, {t_one:.1f} s"}
    del graphs, outs[1:]
    log(f"decode leg: {res}")
    return res, (stack, xs[0], outs[0])


def decode_kernels_alone(torch, args, res, held):
    """The resident decode's gate/up and down kernels launched alone, timed with
    HIP events around a HIP graph of back-to-back launches (the gate/up kernel's
    roofline).  Run after every streamed leg: once a process has captured a HIP
    graph, its later streamed steps run slower (measured: the batch-1 streamed
    decode 2.84 -> 3.10 ms per step after one graph capture of a single
    elementwise kernel, the copy engine idling longer between copies)."""
    stack, x0, out0 = held
    cfg = stack.cfg
    dev_stream = torch.cuda.current_stream()
    h = torch.empty((cfg.tokens * cfg.top_k + cfg.tokens * cfg.shared, cfg.inter), dtype=torch.bfloat16,
                    device="cuda")
    stack.forward(x0, out0)  # routing of input 0 for every layer

    # back-to-back launches of one kernel between two events, captured in one HIP
    # graph and replayed, so host launch cost does not show up as idle time
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

    gu_us = time_launches(lambda l: stack.gate_up_only(x0, l, h), args.kernel_iters)
    dn_us = time_launches(lambda l: stack.down_only(h, l), args.kernel_iters)
    gu_b, dn_b = gate_up_bytes(stack), down_bytes(stack)
    res["gate_up_alone"] = {"kernel": GATE_UP_KERNEL, "us_per_launch": round(gu_us, 3), "bytes_per_launch": gu_b,
                            "GBps": round(gu_b / (gu_us * 1e-6) / 1e9, 1),
                            "frac": round(gu_b / (gu_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                            "traffic": counter_traffic(GATE_UP_KERNEL, "decode1_gate_up_hbm_traffic.md")}
    res["down_alone"] = {"us_per_launch": round(dn_us, 3), "bytes_per_launch": dn_b,
                         "GBps": round(dn_b / (dn_us * 1e-6) / 1e9, 1)}
    stack.close()
    del stack, x0, out0, h
    log(f"decode kernels alone: gate/up {res['gate_up_alone']}, down {res['down_alone']}")


def tiny_leg(torch, args):
    """The one-layer case (hidden 256, 16 experts, intermediate 128, top-2, 4
    tokens, resident): microseconds per layer forward (one moe_route_ffn_combine
    call), and the oracle on the same layer with one thread."""
    import synth
    from routed_expert_streaming_amd.runtime import MoEStack

    cfg = synth.get("tiny")
    st = MoEStack(cfg)
    xs = [st.make_inputs(s) for s in range(8)]
    out = st.new_output()
    for s in range(50):
        st.forward(xs[s % 8], out)
    torch.cuda.synchronize()
    reps = 1000
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for s in range(reps):
        st.forward(xs[s % 8], out)
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = max(a.elapsed_time(b) * 1e3, wall * 1e6) / reps
    res = {"workload": cfg.name, "us_per_layer": round(us, 2), "tokens_per_s": round(cfg.tokens * 1e6 / us, 1),
           "reps": reps}
    if not args.no_cpu_baseline:
        x = [synth.x_bf16(cfg.seed, 0, 0, cfg.tokens, cfg.hidden)]
        wr = [synth.router_w(cfg.seed, 0, cfg.experts, cfg.hidden)]
        slabs = st.host_slabs(0)
        n = 20
        t = sum(oracle_sample(torch, cfg, 1, x, wr, [None], lambda l: slabs, lambda l: None,
                              list(range(cfg.tokens)), 1) for _ in range(n)) / n
        res["cpu_one_thread_us_per_layer"] = round(t * 1e6, 1)
    st.close()
    log(f"tiny leg: {res}")
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import synth

    cfg = synth.get(args.workload)
    if not cfg.streaming:
        raise SystemExit("the headline workload is a streamed configuration; the resident decode is an extra leg")
    result = headline(torch, args, cfg)
    if not args.no_legs:
        decode, held = decode_leg(torch, args)
        result["decode1"] = decode
        if not args.no_stream:
            result["decode1_stream"] = streaming_leg(torch, args, decode["ms_per_step"])
            if not args.no_c4:
                result["decode32_stream"] = decode32_stream_leg(torch, args)
        result["tiny"] = tiny_leg(torch, args)
        if not args.no_mx:
            result["mx"] = format_leg(torch, args, "decode1_mx", "decode1_mx_stream", decode["ms_per_step"],
                                      result.get("decode1_stream"))
            result["superblock"] = format_leg(torch, args, "decode1_sb", "decode1_sb_stream", decode["ms_per_step"],
                                              result.get("decode1_stream"))
        if not args.no_layer_legs:
            from routed_expert_streaming_amd import _lib as L
            result["layer_decode32"] = layer_leg(torch, "decode32_stream", L.MOE_FFN_SPLIT, 20)
            result["layer_prefill2048"] = layer_leg(torch, "prefill2048_stream", L.MOE_FFN_MFMA, 3)
            if not args.no_mx:  # the same layers with MXFP4 and super-block weights
                for tag in ("mx", "sb"):
                    result[f"layer_decode32_{tag}"] = layer_leg(torch, f"decode32_{tag}_stream", L.MOE_FFN_SPLIT, 20)
                    result[f"layer_prefill2048_{tag}"] = layer_leg(torch, f"prefill2048_{tag}_stream",
                                                                   L.MOE_FFN_MFMA, 3)
        # last: the kernel timing captures a HIP graph, after which streamed steps run slower
        decode_kernels_alone(torch, args, decode, held)
        del held
        torch.cuda.empty_cache()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
