"""Host runtime around the C ABI: a stack of routed-expert MoE layers.

Device memory and streams come from torch; pinned host memory comes from the
HIP runtime torch already loaded.  Every arithmetic step runs in libmoe.so's
kernels; this module only allocates, fills inputs and orders the calls:

  step:  [resident] per layer: router + gate/up + SwiGLU + down + combine
         [streaming] the routers of every layer (one call, compute stream), one
         D2H of the top-k ids + host wait, then
             prefetch_async(l) for every layer -> the copy stream queues the misses
             per layer: wait(l)  -> compute waits for layer l's copies
                        expert_ffn + combine(l)
                        release(l) -> slots may be overwritten after this point

Chained steps (forward_chained): layer l+1's input is computed from layer l's
output (a residual stream, moe_residual_norm), so each layer is routed only when
the one before it is done; optionally the next layer's experts are predicted by
applying its router to the current layer's input and prefetched (gating
lookahead).

In forward, the routing of every layer is known at the start of a step because each
(step, layer) gets its own synthetic hidden states; the copies of later layers
therefore overlap the FFN of earlier ones (LayerStoRm README "TL;DR": streaming
is overlapped with compute).  When a layer needs more distinct experts than it has
slots, it runs in waves of at most half its slots, hits first, with a small first
and last wave: each wave's misses go into slots that the wave before last
released, so they stream while the previous wave computes.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

import synth

from . import _lib as L


class PinnedHost:
    """Page-locked host buffer from hipHostMalloc (freed with hipHostFree)."""

    def __init__(self, nbytes: int):
        self.nbytes = int(nbytes)
        hip = L.hip_runtime()
        p = ctypes.c_void_p()
        rc = hip.hipHostMalloc(ctypes.byref(p), ctypes.c_size_t(max(self.nbytes, 1)), ctypes.c_uint(0))
        if rc != 0 or not p.value:
            raise MemoryError(f"hipHostMalloc({self.nbytes}) failed with {rc}")
        self.ptr = p.value
        self._hip = hip
        self.array = np.frombuffer((ctypes.c_uint8 * max(self.nbytes, 1)).from_address(self.ptr), dtype=np.uint8)

    def free(self):
        if self.ptr:
            self.array = None
            self._hip.hipHostFree(ctypes.c_void_p(self.ptr))
            self.ptr = 0

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def _bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


@dataclass
class StepStats:
    waves: int = 0
    copies: int = 0
    cpu_experts: int = 0  # misses computed by the CPU lane instead of streamed
    cpu_pairs: int = 0    # (token, expert) pairs among them


def assign_lanes(misses, t_copy: float, t_cpu, copy_busy: float = 0.0, cpu_busy: float = 0.0):
    """Cost model of the CPU lane: misses = [(layer, expert, tokens)] in the order
    both lanes work through them (layer by layer).  Each miss goes to the lane
    that would finish it first -- the copy engine (t_copy per expert, then the
    GPU computes it) or the CPU lane (t_cpu(tokens) per expert) -- ties to the
    copy engine, which also leaves the expert cached.  Returns one bool per miss
    (True = CPU lane) and the two lanes' busy times."""
    to_cpu = []
    for _, _, tokens in misses:
        fc, fp = copy_busy + t_copy, cpu_busy + t_cpu(tokens)
        if fp < fc:
            cpu_busy = fp
            to_cpu.append(True)
        else:
            copy_busy = fc
            to_cpu.append(False)
    return to_cpu, copy_busy, cpu_busy


@dataclass
class ChainStats:
    """Expert copies of one chained step (see MoEStack.forward_chained)."""
    copies: int = 0        # streamed for the layers' own routing (exposed: the layer waits for them)
    ahead_copies: int = 0  # streamed ahead from the predictions (overlap the layer before)
    ahead_unused: int = 0  # of those, experts the layer's own routing did not select
    routed: int = 0        # distinct routed experts of the predicted layers (1 .. L-1)
    predicted: int = 0     # of those, experts the prediction had named
    cpu_experts: int = 0   # misses computed by the CPU lane instead of streamed


RMS_EPS = 1e-6  # eps of the residual stream's RMS normalisation between chained layers


class MoEStack:
    """L routed-expert MoE layers of one configuration on one GPU.

    cap: fraction of experts per layer held in HBM (None = the configuration's).
    layers: number of layers to build (None = the configuration's).
    split_copies: streamed stacks copy each slab in two halves on two copy
    streams (moe_cache_split_copies).
    cpu_lane: worker threads of a CPU lane (0 = none): in streamed steps whose
    layers fit their slots, cache misses are split between the copy engine and
    host cores computing them from the pinned pool (assign_lanes; lane_pick, if
    set, overrides the choice: lane_pick(layer, misses) -> experts for the CPU).
    link_GBps: host-to-device rate the cost model assumes for a streamed expert.
    """

    def __init__(self, cfg: synth.Config, *, layers: int | None = None, cap: float | None = None,
                 device: int = 0, threads: int = 0, path: int = L.MOE_FFN_AUTO, split_copies: bool = True,
                 cpu_lane: int = 0, link_GBps: float = 55.0):
        L.lib()
        self.cfg = cfg
        self.L = layers or cfg.layers
        self.T, self.H, self.I, self.E, self.k = cfg.tokens, cfg.hidden, cfg.inter, cfg.experts, cfg.top_k
        self.has_shared = cfg.shared > 0
        self.cap = cfg.cap if cap is None else cap
        self.C = min(self.E, int(self.cap * self.E + 1e-9))
        self.streaming = self.C < self.E
        self.path = path
        self.dev = torch.device("cuda", device)
        torch.cuda.set_device(self.dev)
        self.copy_stream = torch.cuda.Stream(self.dev)  # default priority
        self.copy_stream2 = torch.cuda.Stream(self.dev) if split_copies else None
        # 0: fp16 scale/min blocks; 1: MXFP4; 2: super-blocks
        self.fmt = cfg.fmt
        self.slab = [L.moe_expert_bytes, L.moe_expert_bytes_mx, L.moe_expert_bytes_sb][self.fmt](self.H, self.I)
        assert self.slab == synth.slab_bytes(self.H, self.I, self.fmt)
        Lyr, T, H, I, E, k = self.L, self.T, self.H, self.I, self.E, self.k

        # router weights and bias
        self.wr = torch.empty((Lyr, E, H), dtype=torch.float32, device=self.dev)
        self.bias = None if cfg.bias == "none" else torch.empty((Lyr, E), dtype=torch.float32, device=self.dev)
        for l in range(Lyr):
            self.wr[l].copy_(torch.from_numpy(synth.router_w(cfg.seed, l, E, H, threads)))
            if self.bias is not None:
                self.bias[l].copy_(torch.from_numpy(synth.router_bias(cfg, l)))

        # shared experts: always resident
        self.shared = None
        if self.has_shared:
            stage = PinnedHost(Lyr * self.slab)
            for l in range(Lyr):
                synth.fill_slabs(cfg.seed, cfg.weight_layer(l), [synth.shared_expert_id(cfg)], H, I,
                                 [stage.ptr + l * self.slab], threads, self.fmt)
            self.shared = torch.empty((Lyr, self.slab), dtype=torch.uint8, device=self.dev)
            self.shared.view(-1).copy_(torch.from_numpy(stage.array[:Lyr * self.slab]), non_blocking=False)
            stage.free()

        # routed experts
        self.host = None
        self.cache = None
        if not self.streaming:
            self.pool = torch.empty((Lyr * E, self.slab), dtype=torch.uint8, device=self.dev)
            stage = PinnedHost(E * self.slab)
            for l in range(Lyr):
                wl = cfg.weight_layer(l)
                if wl != l:  # the same weights as an earlier layer: device-to-device copy
                    self.pool[l * E:(l + 1) * E].copy_(self.pool[wl * E:(wl + 1) * E])
                    continue
                synth.fill_slabs(cfg.seed, wl, list(range(E)), H, I,
                                 [stage.ptr + e * self.slab for e in range(E)], threads, self.fmt)
                self.pool[l * E:(l + 1) * E].view(-1).copy_(torch.from_numpy(stage.array[:E * self.slab]))
            stage.free()
            base = self.pool.data_ptr()
            ptrs = np.array([base + i * self.slab for i in range(Lyr * E)], dtype=np.int64).reshape(Lyr, E)
            self.table = torch.from_numpy(ptrs).to(self.dev)
        else:
            # one pinned allocation per weight set (very large single pinned
            # allocations can be refused where the total would still be granted);
            # layers that share a weight set point at the same host slabs
            n_sets = min(cfg.n_weight_sets, Lyr)
            self.host = [PinnedHost(E * self.slab) for _ in range(n_sets)]
            for j in range(n_sets):
                synth.fill_slabs(cfg.seed, j, list(range(E)), H, I,
                                 [self.host[j].ptr + e * self.slab for e in range(E)], threads, self.fmt)
            self.pool = torch.empty((Lyr * self.C, self.slab), dtype=torch.uint8, device=self.dev)
            self.table = torch.zeros((Lyr, E), dtype=torch.int64, device=self.dev)
            self._host_ptrs = (ctypes.c_void_p * (Lyr * E))(
                *[self.host_slab_ptr(l, e) for l in range(Lyr) for e in range(E)])
            desc = L.moe_cache_desc(Lyr, E, H, I, self.C, self.fmt)
            torch.cuda.synchronize(self.dev)
            self.cache = L.moe_cache_create(desc, ctypes.addressof(self._host_ptrs), self.pool, self.table,
                                            self.copy_stream)
            if self.copy_stream2 is not None:
                L.moe_cache_split_copies(self.cache, self.copy_stream2)
        # workspaces and outputs
        self.router_ws_bytes = L.moe_router_layers_workspace_bytes(Lyr, T, E)
        self.router_ws = torch.zeros(self.router_ws_bytes, dtype=torch.uint8, device=self.dev)
        self.ffn_ws_bytes = L.moe_expert_ffn_workspace_bytes(T, H, I, E, k, self.has_shared)
        self.ffn_ws = torch.empty(self.ffn_ws_bytes, dtype=torch.uint8, device=self.dev)
        self.layer_ws_bytes = L.moe_route_ffn_combine_workspace_bytes(T, H, I, E, k, self.has_shared)
        self.layer_ws = torch.empty(self.layer_ws_bytes, dtype=torch.uint8, device=self.dev)
        self.idx = torch.empty((Lyr, T, k), dtype=torch.int32, device=self.dev)
        self.w = torch.empty((Lyr, T, k), dtype=torch.float32, device=self.dev)
        P = T * k + (T if self.has_shared else 0)
        self.y = torch.empty((P, H), dtype=torch.float32, device=self.dev)
        half = max(1, self.C // 2)
        self.max_waves = (E + half - 1) // half + 2  # moe_cache_plan: at most ceil(n / half) + 2 waves
        self.masks = torch.zeros((Lyr, self.max_waves, E), dtype=torch.uint8, device=self.dev)
        # gate/up timing of the MFMA path (see ffn); the expert grouping (permutation)
        # and h buffers of the grouped paths (more than 64 (token, slot) pairs), so
        # that a layer's waves share one permutation
        self.kernel_log = None
        grouped = T * k > 64 and path in (L.MOE_FFN_AUTO, L.MOE_FFN_GROUPED, L.MOE_FFN_MFMA, L.MOE_FFN_SPLIT)
        self._perm = (torch.empty(E, dtype=torch.int32, device=self.dev),
                      torch.empty(E + 1, dtype=torch.int32, device=self.dev),
                      torch.empty(T * k, dtype=torch.int32, device=self.dev)) if grouped else None
        self._h = torch.empty((P, I), dtype=torch.bfloat16, device=self.dev) if grouped else None
        # a second y and permutation for layers that run in waves: the streamed step
        # runs a layer's leading waves before the previous layer's last one, so two
        # adjacent layers are in flight (buffers taken by layer parity)
        overflow = self.streaming and T * k > self.C
        self._y2 = torch.empty_like(self.y) if overflow else None
        self._perm2 = tuple(torch.empty_like(t) for t in self._perm) if (overflow and grouped) else None
        self.pidx = torch.empty((Lyr, T, k), dtype=torch.int32, device=self.dev)  # predicted experts
        self.pw = torch.empty((Lyr, T, k), dtype=torch.float32, device=self.dev)
        self._idx_host = PinnedHost(max(Lyr, 2) * T * k * 4) if self.streaming else None
        self._mask_host = PinnedHost(Lyr * self.max_waves * E) if self.streaming else None
        # host outputs of the library's step plan (moe_cache_plan_step)
        self._plan_experts = np.empty((Lyr, T * k), np.int32)
        self._plan_starts = np.empty((Lyr, self.max_waves + 1), np.int32)
        self._plan_nwaves = np.empty(Lyr, np.int32)
        # CPU lane: host copies of the layer inputs and the rows it returns
        self.lane = None
        self.lane_pick = None
        self.link_GBps = link_GBps
        if cpu_lane and self.streaming:
            self.enable_cpu_lane(cpu_lane)
        torch.cuda.synchronize(self.dev)

    def host_slab_ptr(self, l: int, e: int) -> int:
        """Pinned host address of layer l's routed expert e (streamed stacks)."""
        return self.host[self.cfg.weight_layer(l)].ptr + e * self.slab

    def host_pool_slabs(self, l: int):
        """Layer l's routed slabs as views of the pinned host pool the cache streams from."""
        arr = self.host[self.cfg.weight_layer(l)].array
        return [arr[e * self.slab:(e + 1) * self.slab] for e in range(self.E)]

    # ------------------------------------------------------------------ inputs
    def make_inputs(self, step: int, threads: int = 0) -> torch.Tensor:
        """Hidden states [L, T, H] (bf16) of one step, resident on the device."""
        xs = np.stack([synth.x_bf16(self.cfg.seed, step, l, self.T, self.H, threads) for l in range(self.L)])
        return _bf16_tensor(xs, self.dev)

    def new_output(self) -> torch.Tensor:
        return torch.empty((self.L, self.T, self.H), dtype=torch.bfloat16, device=self.dev)

    def layer_experts(self, l: int):
        return self.pool, self.table[l]

    # ------------------------------------------------------------------ step
    @property
    def stream(self):
        """Kernels go to torch's current stream at call time (so graph capture works)."""
        return torch.cuda.current_stream(self.dev)

    def route(self, x: torch.Tensor, l: int):
        L.moe_router_topk(x[l], self.T, self.H, self.wr[l], None if self.bias is None else self.bias[l], self.E,
                          self.k, self.idx[l], self.w[l], self.router_ws, self.router_ws_bytes, self.stream)

    def route_with(self, x_l: torch.Tensor, l: int, idx: torch.Tensor, w: torch.Tensor):
        """Router of layer l applied to the hidden states x_l [T,H] (any layer's)."""
        L.moe_router_topk(x_l, self.T, self.H, self.wr[l], None if self.bias is None else self.bias[l], self.E,
                          self.k, idx, w, self.router_ws, self.router_ws_bytes, self.stream)

    def route_all(self, x: torch.Tensor):
        """Routers of every layer in one call."""
        L.moe_router_topk_layers(x, self.L, self.T, self.H, self.wr, self.bias, self.E, self.k, self.idx, self.w,
                                 self.router_ws, self.router_ws_bytes, self.stream)

    def ffn(self, x: torch.Tensor, l: int, mask=None, shared=True, experts=None, permuted=False, y=None, perm=None):
        """Gate/up + SwiGLU and down projection of layer l's pairs whose expert the
        mask admits (all when None) into y.  With more than 64 (token, slot) pairs
        the kernels run in expert grouping as three calls -- the permutation,
        gate/up, down -- and permuted=True reuses the permutation of the same
        layer's routing computed by an earlier call (the layer's earlier waves).
        With kernel_log set to a list and many tokens (the MFMA kernels), timing
        events go before gate/up, between the two and after down, and (the three
        events, layer, experts, shared expert included) is appended to the log.
        y / perm: the output rows and the permutation buffers to use (default
        self.y and self._perm)."""
        sh = self.shared[l] if (self.has_shared and shared) else None
        y = self.y if y is None else y
        # MXFP4 prefill runs on the block-scaled matrix cores, whose activation
        # digit pairs live in the one-call FFN's workspace
        scaled = self.fmt == 1 and self.T >= 128 and self.path in (L.MOE_FFN_AUTO, L.MOE_FFN_MFMA)
        if self._perm is None or scaled:
            L.moe_expert_ffn_fmt(x[l], self.T, self.H, self.I, self.E, self.idx[l], self.k, self.table[l], sh, mask,
                                 y, self.ffn_ws, self.ffn_ws_bytes, self.path, self.fmt, self.stream)
            return
        T, H, I, E, k = self.T, self.H, self.I, self.E, self.k
        cnt, off, por = self._perm if perm is None else perm
        if not permuted:
            L.moe_permute(self.idx[l], T, k, E, cnt, off, por, self.stream)
        log = self.kernel_log is not None and T >= 128 and self.path in (L.MOE_FFN_AUTO, L.MOE_FFN_MFMA)
        if log:
            a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            a.record(self.stream)
        L.moe_expert_gate_up_fmt(x[l], T, H, I, E, self.idx[l], k, cnt, off, por, self.table[l], sh, mask,
                                 self._h, self.path, self.fmt, self.stream)
        if log:
            b.record(self.stream)
        L.moe_expert_down_fmt(self._h, T, H, I, E, self.idx[l], k, cnt, off, por, self.table[l], sh, mask, y,
                              self.path, self.fmt, self.stream)
        if log:
            c.record(self.stream)
            self.kernel_log.append((a, b, c, l, list(range(E)) if experts is None else list(experts),
                                    sh is not None))

    def ffn_combine(self, x: torch.Tensor, l: int, out: torch.Tensor):
        """Gate/up, down and the weighted combine of layer l (every needed expert resident)."""
        if self.fmt:
            (L.moe_mx_expert_ffn_combine if self.fmt == 1 else L.moe_sb_expert_ffn_combine)(x[l], self.T, self.H, self.I, self.E, self.idx[l], self.w[l], self.k,
                                        self.table[l], self.shared[l] if self.has_shared else None, out[l],
                                        self.ffn_ws, self.ffn_ws_bytes, self.stream)
            return
        L.moe_expert_ffn_combine(x[l], self.T, self.H, self.I, self.E, self.idx[l], self.w[l], self.k,
                                 self.table[l], self.shared[l] if self.has_shared else None, out[l], self.ffn_ws,
                                 self.ffn_ws_bytes, self.path, self.stream)

    def route_ffn_combine(self, x: torch.Tensor, l: int, out: torch.Tensor):
        """Router, gate/up, down and combine of layer l in one call (every expert resident).
        The call reads the router weights of the layer that runs next (the first
        after the last) into the device caches while it runs: they are static, so
        this does not depend on the next layer's input."""
        nxt = self.wr[(l + 1) % self.L]
        call = [L.moe_route_ffn_combine, L.moe_mx_route_ffn_combine, L.moe_sb_route_ffn_combine][self.fmt]
        call(x[l], self.T, self.H, self.I, self.wr[l], None if self.bias is None else self.bias[l],
                                self.E, self.k, self.table[l], self.shared[l] if self.has_shared else None,
                                self.idx[l], self.w[l], out[l], self.layer_ws, self.layer_ws_bytes, self.stream,
                                prefetch=nxt, prefetch_bytes=nxt.numel() * 4)

    def combine(self, l: int, out: torch.Tensor, y=None):
        L.moe_combine(self.y if y is None else y, self.w[l], self.T, self.k, self.H, self.has_shared, out[l],
                      self.stream)

    def gate_up_only(self, x: torch.Tensor, l: int, h: torch.Tensor):
        """Only the dequant + gate/up + SwiGLU kernel of layer l (pair grouping), for timing it."""
        L.moe_expert_gate_up_fmt(x[l], self.T, self.H, self.I, self.E, self.idx[l], self.k, None, None, None,
                                 self.table[l], self.shared[l] if self.has_shared else None, None, h,
                                 L.MOE_FFN_PAIRS, self.fmt, self.stream)

    def down_only(self, h: torch.Tensor, l: int):
        """Only the dequant + down-projection kernel of layer l (pair grouping), for timing it."""
        L.moe_expert_down_fmt(h, self.T, self.H, self.I, self.E, self.idx[l], self.k, None, None, None,
                              self.table[l], self.shared[l] if self.has_shared else None, None, self.y,
                              L.MOE_FFN_PAIRS, self.fmt, self.stream)

    def plan_waves(self, l: int, ids, masks=None):
        """The library's step plan of layer l (moe_cache_plan): its top-k ids split
        into waves that fit its slots, resident experts first, each wave's expert
        mask written into masks [max_waves, E] (host) when given."""
        return L.moe_cache_plan(self.cache, l, ids, max_waves=self.max_waves, masks=masks)

    # ------------------------------------------------------------------ CPU lane
    def enable_cpu_lane(self, threads: int):
        """Start a CPU lane of `threads` workers (streamed stacks only) and calibrate it."""
        assert self.streaming and self.lane is None and self.fmt == 0
        P = self.T * self.k + (self.T if self.has_shared else 0)
        self.lane = L.moe_cpu_lane_create(threads)
        self.lane_threads = threads
        self._x_host = torch.empty((self.L, self.T, self.H), dtype=torch.bfloat16, pin_memory=True)
        # the lane's rows of layer l, compact (in submission order), their pair rows
        # in y, and the device copies they are uploaded to before moe_scatter_rows
        self._y_host = torch.empty((self.L, P, self.H), dtype=torch.float32, pin_memory=True)
        self._rows_host = torch.empty((self.L, P), dtype=torch.int32, pin_memory=True)
        self._y_stage = torch.empty((P, self.H), dtype=torch.float32, device=self.dev)
        self._rows_dev = torch.empty((self.L, P), dtype=torch.int32, device=self.dev)
        self.t_cpu1, self.t_cpu8 = self.calibrate_lane()
        self.t_cpu_big = None
        if self.T > 8:  # a third point: an expert's average token count at this batch
            m = max(9, min(self.T, (self.T * self.k + self.E - 1) // self.E))
            self.t_cpu_big = (m, self.calibrate_lane(counts=(m,))[0])

    def t_cpu(self, tokens: int) -> float:
        """CPU lane seconds for one expert and `tokens` tokens: linear through the
        calibrated 1 and 8 tokens, and above 8 through 8 and the third calibrated
        count (stacks of more than 8 tokens)."""
        if tokens <= 8 or self.t_cpu_big is None:
            return self.t_cpu1 + (tokens - 1) * (self.t_cpu8 - self.t_cpu1) / 7.0
        m, t_m = self.t_cpu_big
        return self.t_cpu8 + (tokens - 8) * (t_m - self.t_cpu8) / (m - 8)

    def calibrate_lane(self, reps: int = 3, counts=(1, 8)):
        """Time the lane on layer 0's first slabs (for each token count), best of reps."""
        import time
        n = max(counts)
        ys = torch.empty((n, self.H), dtype=torch.float32)
        xs = torch.zeros((n, self.H), dtype=torch.bfloat16)
        out = []
        for M in counts:
            best = float("inf")
            for r in range(reps + 1):
                slab = self.host_slab_ptr(0, r % self.E)
                t0 = time.perf_counter()
                t = L.moe_cpu_lane_submit(self.lane, slab, self.H, self.I, M,
                                          [xs[i].data_ptr() for i in range(M)], [ys[i].data_ptr() for i in range(M)])
                L.moe_cpu_lane_wait(self.lane, t)
                if r:  # the first run warms the threads
                    best = min(best, time.perf_counter() - t0)
            out.append(best)
        return tuple(out)

    def plan_cpu_lane(self, needed_by_layer, idx_host, layers=None, cpu_head: float = 0.0):
        """Experts of each layer that the CPU lane computes (layers: the layer ids
        of the lists, default 0, 1, ...; cpu_head: seconds the lane starts behind
        the copy engine)."""
        layers = list(range(len(needed_by_layer))) if layers is None else list(layers)
        misses = []
        for i, (l, needed) in enumerate(zip(layers, needed_by_layer)):
            slots, _ = L.moe_cache_lookup(self.cache, l, needed)
            tok = np.bincount(idx_host[i].ravel(), minlength=self.E)
            misses += [(i, e, int(tok[e])) for e, s in zip(needed, slots) if s < 0]
        cpu = [set() for _ in needed_by_layer]
        if self.lane_pick is not None:
            for i, l in enumerate(layers):
                cpu[i] = set(self.lane_pick(l, [e for ii, e, _ in misses if ii == i]))
            return cpu
        to_cpu, _, _ = assign_lanes(misses, self.slab / (self.link_GBps * 1e9), self.t_cpu, cpu_busy=cpu_head)
        for (i, e, _), c in zip(misses, to_cpu):
            if c:
                cpu[i].add(e)
        return cpu

    def submit_cpu_lane(self, l: int, experts, idx_l: np.ndarray):
        """Queue layer l's CPU-lane experts, their rows written compactly into
        layer l's host rows in submission order; returns (last ticket, the pair row
        in y of each compact row)."""
        ticket, rows = 0, []
        for e in sorted(experts):
            ts, iis = np.nonzero(idx_l == e)
            pairs = [int(t) * self.k + int(i) for t, i in zip(ts, iis)]
            n0 = len(rows)
            ticket = L.moe_cpu_lane_submit(self.lane, self.host_slab_ptr(l, e), self.H, self.I, len(pairs),
                                           [self._x_host[l, int(t)].data_ptr() for t in ts],
                                           [self._y_host[l, n0 + j].data_ptr() for j in range(len(pairs))])
            rows += pairs
        return ticket, rows

    def upload_cpu_rows(self, l: int, rows, y=None):
        """The CPU lane's rows of layer l into their pair rows of y (default self.y):
        one copy of the compact rows (and one of their row numbers), then
        moe_scatter_rows."""
        n = len(rows)
        if n == 0:
            return
        self._rows_host[l, :n].numpy()[:] = rows
        self._y_stage[:n].copy_(self._y_host[l, :n], non_blocking=True)
        self._rows_dev[l, :n].copy_(self._rows_host[l, :n], non_blocking=True)
        for i in range(0, n, 65535):
            m = min(65535, n - i)
            L.moe_scatter_rows(self._y_stage[i:], self._rows_dev[l, i:], m, self.H, self.y if y is None else y,
                               self.stream)

    # ------------------------------------------------------------------ steps
    def forward(self, x: torch.Tensor, out: torch.Tensor) -> StepStats:
        """One step over all layers: x [L,T,H] bf16 -> out [L,T,H] bf16."""
        st = StepStats()
        if not self.streaming:
            for l in range(self.L):
                self.route_ffn_combine(x, l, out)
            return st
        self.route_all(x)
        # one small D2H per step, then the host plans every layer
        idx_host = np.frombuffer(self._idx_host.array, dtype=np.int32, count=self.L * self.T * self.k)
        torch.from_numpy(idx_host).copy_(self.idx.view(-1), non_blocking=True)
        if self.lane is not None:
            self._x_host.copy_(x, non_blocking=True)
        self.stream.synchronize()  # also: the previous step's mask upload has read the host masks
        idx3 = idx_host.reshape(self.L, self.T, self.k)
        mh = np.frombuffer(self._mask_host.array, dtype=np.uint8,
                           count=self.L * self.max_waves * self.E).reshape(self.L, self.max_waves, self.E)
        # CPU lane: some misses are computed on the host; the rest of the layer's
        # experts run on the GPU in one wave when they fit its slots, else in the
        # library's waves
        if self.lane is None:
            return self._forward_planned(x, out, idx_host, mh, st)
        lane_jobs = {}
        needed_by_layer = [sorted(set(row)) for row in idx_host.reshape(self.L, -1).tolist()]
        cpu_sets = self.plan_cpu_lane(needed_by_layer, idx3)
        plans = []
        for l in range(self.L):
            if cpu_sets[l]:
                gpu_side = [e for e in needed_by_layer[l] if e not in cpu_sets[l]]
                if len(gpu_side) <= self.C:
                    plans.append([gpu_side])
                    mh[l] = 0
                    mh[l, 0, gpu_side] = 1
                else:  # the library's waves over the GPU's experts
                    plans.append(self.plan_waves(l, np.array(gpu_side, dtype=np.int32), masks=mh[l]))
                lane_jobs[l] = self.submit_cpu_lane(l, cpu_sets[l], idx3[l])
                st.cpu_experts += len(cpu_sets[l])
                st.cpu_pairs += len(lane_jobs[l][1])
                continue
            # the library's plan: one wave when the layer's experts fit its slots,
            # else waves of at most half the slots, hits first, small first and last waves
            plans.append(self.plan_waves(l, idx3[l], masks=mh[l]))
        self.last_cpu_sets = cpu_sets
        if any(len(p) > 1 for p in plans) or lane_jobs:
            self._upload_masks(mh)
        # single-wave layers: every copy is queued before the first FFN launch, so
        # the copy engine starts as soon as the plan is known (each layer evicts
        # only its own slots, released in the previous step); the compute stream
        # waits for a layer's copies just before that layer's kernels
        single = [len(waves) == 1 for waves in plans]
        for l, waves in enumerate(plans):
            if single[l]:
                st.copies += L.moe_cache_prefetch_async(self.cache, l, waves[0])
        pending = []  # a layer in waves whose lane rows and combine wait for the next layer's waves

        def flush():
            while pending:
                lp, yp = pending.pop()
                ticket, rows = lane_jobs[lp]
                L.moe_cpu_lane_wait(self.lane, ticket)
                self.upload_cpu_rows(lp, rows, y=yp)
                self.combine(lp, out, y=yp)

        for l, waves in enumerate(plans):
            if single[l]:
                flush()
            if single[l] and l in lane_jobs:
                # GPU lane: the layer's hits and streamed misses (masked call), then
                # the CPU lane's rows, then the combine of all of them
                L.moe_cache_wait(self.cache, l, self.stream)
                self.ffn(x, l, mask=self.masks[l, 0], shared=True)
                L.moe_cache_release(self.cache, l, self.stream)
                ticket, rows = lane_jobs[l]
                L.moe_cpu_lane_wait(self.lane, ticket)
                self.upload_cpu_rows(l, rows)
                self.combine(l, out)
                st.waves += 1
                continue
            if single[l]:
                L.moe_cache_wait(self.cache, l, self.stream)
                self.ffn_combine(x, l, out)
                L.moe_cache_release(self.cache, l, self.stream)
                st.waves += 1
                continue
            # a layer in waves: its y rows by layer parity, so that the lane rows and
            # the combine of the layer before it can wait until this layer's waves
            # are queued (the host's wait for the lane then leaves the copy engine
            # this layer's copies to work on)
            y = self._y2 if (self._y2 is not None and l % 2 == 1) else self.y
            for wv, experts in enumerate(waves):
                st.copies += L.moe_cache_prefetch(self.cache, l, experts, self.stream)
                self.ffn(x, l, mask=self.masks[l, wv], shared=(wv == 0), experts=experts, permuted=wv > 0, y=y)
                L.moe_cache_release(self.cache, l, self.stream)
                st.waves += 1
            flush()
            if l in lane_jobs:
                pending.append((l, y))
            else:
                self.combine(l, out, y=y)
        flush()
        return st

    def _upload_masks(self, mh: np.ndarray):
        """Copy the step's wave masks (pinned host) to the device over the copy
        stream, ahead of the step's slab copies, and make the compute stream wait
        for them.  On the compute stream the upload is a DMA command of its own
        queue, which the DMA engine can leave behind the copy streams' waits for
        slot releases that only later compute-stream work records (measured: the
        first FFN of a step started ~4 ms late)."""
        with torch.cuda.stream(self.copy_stream):
            self.masks.view(-1).copy_(torch.from_numpy(mh.reshape(-1)), non_blocking=True)
        self.stream.wait_stream(self.copy_stream)

    def _forward_planned(self, x, out, idx_host, mh, st: StepStats) -> StepStats:
        """The streamed step after routing, without a CPU lane: one library call
        plans every layer and queues the copies of the layers that fit their slots
        (the copy engine starts right away); then per layer the wait, the FFN
        (wave by wave for layers that need more experts than they have slots) and
        the release.

        Two adjacent layers that both run in waves overlap: the next layer's
        leading waves (its first two at most, and only those whose experts are
        all resident, so they need no copy; resident experts come first) go
        before this layer's last wave.  They compute while this layer's
        last misses stream and free slots of the next layer, so its first misses
        stream right after this layer's last ones instead of after this layer's
        last wave, its combine and the next layer's first waves have computed.
        The step's layers take their own inputs, so the order of their kernels
        does not change any result; the two layers in flight use the y rows and
        permutation buffers of their parity, and every layer still calls the
        cache in its own wave order (its hits, misses and victims do not change)."""
        ne = self._plan_experts
        starts = self._plan_starts
        nw = self._plan_nwaves
        # a layer can need more waves than one only when its top-k ids outnumber its
        # slots; then the masks go up before any copy of the step is queued
        may_overflow = self.T * self.k > self.C
        st.copies += L.moe_cache_plan_step(self.cache, idx_host, self.T * self.k, ne, starts, self.max_waves, mh, nw,
                                           not may_overflow)
        if may_overflow:
            if (nw > 1).any():
                self._upload_masks(mh)
            for l in range(self.L):
                if nw[l] == 1:
                    st.copies += L.moe_cache_prefetch_async(self.cache, l, ne[l, :starts[l, 1]])
        def wave(l: int, wv: int):
            experts = ne[l, starts[l, wv]:starts[l, wv + 1]]
            st.copies += L.moe_cache_prefetch(self.cache, l, experts, self.stream)
            par = self._y2 is not None and l % 2 == 1
            self.ffn(x, l, mask=self.masks[l, wv], shared=(wv == 0), experts=experts, permuted=wv > 0,
                     y=self._y2 if par else None, perm=self._perm2 if par else None)
            L.moe_cache_release(self.cache, l, self.stream)
            st.waves += 1

        overlap = self._y2 is not None and (self._perm is None or self._perm2 is not None)

        def resident_lead(l: int) -> int:
            # leading waves of layer l (all but its last) whose experts are all
            # resident now: they need no copy, so they can run ahead (the layer's
            # slots change only through its own prefetches)
            n = 0
            for wv in range(int(nw[l]) - 1):
                experts = ne[l, starts[l, wv]:starts[l, wv + 1]]
                if L.moe_cache_lookup(self.cache, l, experts)[1] != len(experts):
                    break
                n += 1
            return n

        led = 0  # waves of layer l already run ahead of layer l-1's last wave
        for l in range(self.L):
            if nw[l] == 1:
                L.moe_cache_wait(self.cache, l, self.stream)
                self.ffn_combine(x, l, out)
                L.moe_cache_release(self.cache, l, self.stream)
                st.waves += 1
                led = 0
                continue
            last = int(nw[l]) - 1
            for wv in range(led, last):
                wave(l, wv)
            led = 0
            if overlap and l + 1 < self.L and nw[l + 1] > 1:
                led = min(2, resident_lead(l + 1))
                for wv in range(led):
                    wave(l + 1, wv)
            wave(l, last)
            self.combine(l, out, y=self._y2 if (self._y2 is not None and l % 2 == 1) else None)
        self.last_cpu_sets = [set() for _ in range(self.L)]
        return st

    # ------------------------------------------------------------------ chained layers
    def chain_buffers(self):
        """Device buffers of a chained step: the residual stream [T,H] fp32 and
        the layer inputs [L,T,H] bf16."""
        resid = torch.empty((self.T, self.H), dtype=torch.float32, device=self.dev)
        xs = torch.empty((self.L, self.T, self.H), dtype=torch.bfloat16, device=self.dev)
        return resid, xs

    def forward_chained(self, h0: torch.Tensor, xs: torch.Tensor, resid: torch.Tensor, out: torch.Tensor,
                        lookahead: int = 0) -> ChainStats:
        """One step with chained layers: h0 [T,H] bf16 starts the residual stream,
        layer l's input xs[l] is the stream RMS-normalised after every earlier
        layer's output was added (moe_residual_norm), out[l] is layer l's output.

        Streamed, a layer's routing is known only when the layer before it is
        done, so the copies for its own routing are exposed.  With lookahead = m
        > 0, layer l+1's router is also applied to layer l's input (gating
        lookahead) and, per token, the m experts it ranks highest are prefetched
        while layer l computes (m = k: every predicted expert); they stay held
        until layer l+1 has run.  Needs T*(k+m) <= C: a layer's own experts fit
        beside the predicted ones."""
        st = ChainStats()
        T, H, k = self.T, self.H, self.k
        resid.zero_()
        L.moe_residual_norm(h0, resid, T, H, RMS_EPS, xs[0], self.stream)
        m = max(0, min(int(lookahead), k))
        if self.streaming and T * (k + m) > self.C:
            raise ValueError(f"chained streaming needs {T * (k + m)} <= {self.C} slots")
        pred = {}  # layer -> (predicted set, set copied ahead)
        self.last_cpu_sets = [set() for _ in range(self.L)]
        for l in range(self.L):
            if not self.streaming:
                self.route_ffn_combine(xs, l, out)
            else:
                ahead = m > 0 and l + 1 < self.L
                self.route(xs, l)
                if ahead:
                    self.route_with(xs[l], l + 1, self.pidx[l + 1], self.pw[l + 1])
                # one small D2H of the ids and a host wait per layer, then the host plans
                hv = np.frombuffer(self._idx_host.array, dtype=np.int32, count=2 * T * k)
                torch.from_numpy(hv[:T * k]).copy_(self.idx[l].view(-1), non_blocking=True)
                if ahead:
                    torch.from_numpy(hv[T * k:]).copy_(self.pidx[l + 1].view(-1), non_blocking=True)
                if self.lane is not None:
                    self._x_host[l].copy_(xs[l], non_blocking=True)
                self.stream.synchronize()
                needed = sorted(set(hv[:T * k].tolist()))
                # CPU lane: some of this layer's misses computed on the host while
                # the copy engine streams the others
                cpu, job = set(), None
                if self.lane is not None:
                    idx_l = hv[:T * k].reshape(T, k).copy()
                    # a layer's first miss always streams: it is exposed either way,
                    # and streamed it is cached for the next step (the lane's
                    # experts are not); the lane takes later misses when it
                    # would finish them first
                    cpu = self.plan_cpu_lane([needed], idx_l[None], layers=[l],
                                             cpu_head=self.slab / (self.link_GBps * 1e9))[0]
                    if cpu:
                        job = self.submit_cpu_lane(l, cpu, idx_l)
                        st.cpu_experts += len(cpu)
                        self.last_cpu_sets[l] = cpu
                gpu_side = [e for e in needed if e not in cpu]
                st.copies += L.moe_cache_prefetch_async(self.cache, l, gpu_side)
                if l in pred:
                    named, copied = pred.pop(l)
                    st.routed += len(needed)
                    st.predicted += len(named.intersection(needed))
                    st.ahead_unused += len(copied.difference(needed))
                if ahead:
                    # the predicted ids come per token in order of descending logit
                    nxt = sorted(set(hv[T * k:].reshape(T, k)[:, :m].ravel().tolist()))
                    slots, _ = L.moe_cache_lookup(self.cache, l + 1, nxt)
                    copied = {e for e, s in zip(nxt, slots) if s < 0}
                    st.ahead_copies += L.moe_cache_prefetch_async(self.cache, l + 1, nxt)
                    pred[l + 1] = (set(nxt), copied)
                L.moe_cache_wait(self.cache, l, self.stream)
                if job is None:
                    self.ffn_combine(xs, l, out)
                    L.moe_cache_release(self.cache, l, self.stream)
                else:
                    mh = np.frombuffer(self._mask_host.array, dtype=np.uint8,
                                       count=self.L * self.max_waves * self.E).reshape(self.L, self.max_waves, self.E)
                    mh[l, 0] = 0
                    mh[l, 0, gpu_side] = 1
                    self.masks[l, 0].copy_(torch.from_numpy(mh[l, 0]), non_blocking=True)
                    self.ffn(xs, l, mask=self.masks[l, 0], shared=True)
                    L.moe_cache_release(self.cache, l, self.stream)
                    L.moe_cpu_lane_wait(self.lane, job[0])
                    self.upload_cpu_rows(l, job[1])
                    self.combine(l, out)
            if l + 1 < self.L:
                L.moe_residual_norm(out[l], resid, T, H, RMS_EPS, xs[l + 1], self.stream)
        return st

    def last_routing(self) -> np.ndarray:
        """Host copy [L, T, k] of the expert ids of the last streamed step."""
        hv = np.frombuffer(self._idx_host.array, dtype=np.int32, count=self.L * self.T * self.k)
        return hv.reshape(self.L, self.T, self.k).copy()

    def stats(self):
        return L.moe_cache_stats(self.cache) if self.cache else (0, 0, 0)

    def reset_cache(self):
        if self.cache:
            L.moe_cache_reset(self.cache)

    def close(self):
        if getattr(self, "lane", None):
            L.moe_cpu_lane_destroy(self.lane)
            self.lane = None
        if self.cache:
            torch.cuda.synchronize(self.dev)
            L.moe_cache_destroy(self.cache)
            self.cache = None
        if self.host is not None:
            for buf in self.host:
                buf.free()
            self.host = None
        for attr in ("_idx_host", "_mask_host"):
            buf = getattr(self, attr, None)
            if buf is not None:
                buf.free()
                setattr(self, attr, None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ host copies for checking
    def host_slabs(self, l: int):
        """Routed slabs of layer l as host numpy arrays (regenerated from the seed)."""
        wl = self.cfg.weight_layer(l)
        return [synth.expert_slab(self.cfg.seed, wl, e, self.H, self.I, self.fmt) for e in range(self.E)]

    def host_shared(self, l: int):
        if not self.has_shared:
            return None
        return synth.expert_slab(self.cfg.seed, self.cfg.weight_layer(l), synth.shared_expert_id(self.cfg), self.H,
                                 self.I, self.fmt)
