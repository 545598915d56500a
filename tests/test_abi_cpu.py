"""Host-side tests of libmoe.so: exported symbols, argument validation, and the
expert-cache policy through the recording copy engine (no GPU needed)."""
import os
import random
import re

import numpy as np

import pytest

from routed_expert_streaming_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    names = declared_functions()
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_status_strings_and_format_sizes():
    assert L.moe_status_str(0) == "ok"
    assert "slots" in L.moe_status_str(L.MOE_E_CAPACITY)
    assert L.moe_expert_bytes(256, 128) == 61440
    assert L.moe_expert_bytes(4096, 1536) == 11796480
    assert L.moe_expert_bytes(6144, 2048) == 23592960
    assert L.moe_expert_bytes(100, 128) == 0
    assert L.moe_router_workspace_bytes(1, 128) >= 256 + 512


def _status(fn, *args):
    with pytest.raises(L.MoEError) as ei:
        fn(*args)
    return ei.value.status


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def test_router_validation():
    ws = L.moe_router_workspace_bytes(4, 16)
    assert _status(L.moe_router_topk, None, 4, 256, FAKE, None, 16, 2, FAKE, FAKE, FAKE, ws) == L.MOE_E_ARG
    assert _status(L.moe_router_topk, FAKE, 4, 250, FAKE, None, 16, 2, FAKE, FAKE, FAKE, ws) == L.MOE_E_SHAPE
    assert _status(L.moe_router_topk, FAKE, 4, 256, FAKE, None, 16, 17, FAKE, FAKE, FAKE, ws) == L.MOE_E_SHAPE
    assert _status(L.moe_router_topk, FAKE, 4, 256, FAKE, None, 2000, 2, FAKE, FAKE, FAKE, 10**8) == L.MOE_E_SHAPE
    assert _status(L.moe_router_topk, FAKE, 4, 256, FAKE, None, 16, 2, FAKE, FAKE, FAKE, ws - 1) == L.MOE_E_NOMEM
    L.moe_router_topk(None, 0, 256, None, None, 16, 2, None, None, None, 0)  # T = 0 is a no-op


def test_router_layers_validation():
    one = L.moe_router_workspace_bytes(4, 16)
    ws = L.moe_router_layers_workspace_bytes(3, 4, 16)
    assert L.moe_router_layers_workspace_bytes(1, 4, 16) == one
    assert ws == 2 * ((one + 255) // 256 * 256) + one
    assert L.moe_router_layers_workspace_bytes(0, 4, 16) == 0
    args = (FAKE, 3, 4, 256, FAKE, None, 16, 2, FAKE, FAKE, FAKE)
    assert _status(L.moe_router_topk_layers, *args, ws - 1) == L.MOE_E_NOMEM
    assert _status(L.moe_router_topk_layers, FAKE, -1, 4, 256, FAKE, None, 16, 2, FAKE, FAKE, FAKE, ws) == L.MOE_E_ARG
    assert _status(L.moe_router_topk_layers, FAKE, 3, 4, 256, FAKE, None, 16, 0, FAKE, FAKE, FAKE, ws) == L.MOE_E_SHAPE
    assert _status(L.moe_router_topk_layers, FAKE, 3, 4, 256, None, None, 16, 2, FAKE, FAKE, FAKE, ws) == L.MOE_E_ARG
    L.moe_router_topk_layers(None, 0, 4, 256, None, None, 16, 2, None, None, None, 0)  # no layers: no-op


def test_ffn_combine_permute_validation():
    ws = L.moe_expert_ffn_workspace_bytes(4, 256, 128, 16, 2, 0)
    args = [FAKE, 4, 256, 128, 16, FAKE, 2, FAKE, None, None, FAKE, FAKE, ws]
    assert _status(L.moe_expert_ffn, None, *args[1:]) == L.MOE_E_ARG
    bad = list(args); bad[2] = 250
    assert _status(L.moe_expert_ffn, *bad) == L.MOE_E_SHAPE
    bad = list(args); bad[3] = 100
    assert _status(L.moe_expert_ffn, *bad) == L.MOE_E_SHAPE
    bad = list(args); bad[6] = 17
    assert _status(L.moe_expert_ffn, *bad) == L.MOE_E_SHAPE
    bad = list(args); bad[12] = ws - 1
    assert _status(L.moe_expert_ffn, *bad) == L.MOE_E_NOMEM
    assert _status(L.moe_expert_ffn, *args, 7) == L.MOE_E_ARG
    assert _status(L.moe_expert_ffn, *args, L.MOE_FFN_SPLIT + 1) == L.MOE_E_ARG
    # grouped, MFMA and split kernels need the permutation
    for path in (L.MOE_FFN_GROUPED, L.MOE_FFN_MFMA, L.MOE_FFN_SPLIT):
        assert _status(L.moe_expert_gate_up, FAKE, 4, 256, 128, 16, FAKE, 2, None, None, None, FAKE, None, None,
                       FAKE, path) == L.MOE_E_ARG
    assert _status(L.moe_combine, None, FAKE, 4, 2, 256, 0, FAKE) == L.MOE_E_ARG
    assert _status(L.moe_combine, FAKE, FAKE, 4, 2, 254, 0, FAKE) == L.MOE_E_SHAPE
    assert _status(L.moe_scatter_rows, FAKE, FAKE, -1, 256, FAKE) == L.MOE_E_ARG
    assert _status(L.moe_scatter_rows, None, FAKE, 4, 256, FAKE) == L.MOE_E_ARG
    assert _status(L.moe_scatter_rows, FAKE, None, 4, 256, FAKE) == L.MOE_E_ARG
    assert _status(L.moe_scatter_rows, FAKE, FAKE, 4, 0, FAKE) == L.MOE_E_ARG
    assert _status(L.moe_scatter_rows, FAKE, FAKE, 4, 254, FAKE) == L.MOE_E_SHAPE
    assert _status(L.moe_scatter_rows, FAKE, FAKE, 65536, 256, FAKE) == L.MOE_E_SHAPE
    L.moe_scatter_rows(None, None, 0, 256, None)  # no rows: nothing to do
    assert _status(L.moe_permute, FAKE, 4096, 8, 256, FAKE, FAKE, FAKE) == L.MOE_E_SHAPE
    assert _status(L.moe_permute, FAKE, 4, 8, 4, FAKE, FAKE, FAKE) == L.MOE_E_SHAPE
    assert _status(L.moe_debug_dequant, FAKE, 256, 128, 3, FAKE) == L.MOE_E_ARG


# ----------------------------------------------------------------------------- cache policy
class LRUModel:
    """Brute-force model of the documented cache rule, one layer at a time."""

    def __init__(self, layers, experts, slots):
        self.E, self.C = experts, slots
        self.slot_of = [dict() for _ in range(layers)]
        self.expert_of = [[-1] * slots for _ in range(layers)]
        self.stamp = [[0] * slots for _ in range(layers)]
        self.held = [[False] * slots for _ in range(layers)]
        self.last_rel = [[-1] * slots for _ in range(layers)]
        self.next_rel = [0] * layers
        self.clock = 0
        self.hits = self.misses = 0

    def prefetch(self, l, experts):
        srt = sorted(experts)
        hits = [e for e in srt if e in self.slot_of[l]]
        misses = [e for e in srt if e not in self.slot_of[l]]
        needed = {self.slot_of[l][e] for e in hits}
        free = sum(1 for s in range(self.C) if not self.held[l][s] and s not in needed)
        if len(experts) > self.C or len(misses) > free:
            return "capacity", []
        cmds = []
        for e in hits:
            s = self.slot_of[l][e]
            self.clock += 1
            self.stamp[l][s] = self.clock
            self.held[l][s] = True
        table = []
        last_wait = -2
        for e in misses:
            victim = min((self.stamp[l][s], s) for s in range(self.C) if not self.held[l][s])[1]
            old = self.expert_of[l][victim]
            if old >= 0:
                del self.slot_of[l][old]
                table.append((3, l, old, -1))
            if self.last_rel[l][victim] >= 0 and self.last_rel[l][victim] != last_wait:
                cmds.append((1, victim, self.last_rel[l][victim], -1))
                last_wait = self.last_rel[l][victim]
            cmds.append((2, l, e, victim))
            self.expert_of[l][victim] = e
            self.slot_of[l][e] = victim
            self.clock += 1
            self.stamp[l][victim] = self.clock
            self.held[l][victim] = True
            table.append((3, l, e, victim))
        cmds += table
        if misses:
            cmds.append((4, l, -1, -1))
        self.hits += len(hits)
        self.misses += len(misses)
        return "ok", cmds

    def release(self, l):
        n = sum(self.held[l])
        if n == 0:
            return []
        rid = self.next_rel[l]
        self.next_rel[l] += 1
        for s in range(self.C):
            if self.held[l][s]:
                self.held[l][s] = False
                self.last_rel[l][s] = rid
        return [(5, l, rid, n)]


def _desc(layers, experts, slots, hidden=256, inter=128):
    return L.moe_cache_desc(layers, experts, hidden, inter, slots)


@pytest.mark.parametrize("seed,layers,experts,slots,maxreq", [
    (1, 1, 16, 4, 4), (2, 3, 16, 8, 6), (3, 2, 128, 32, 8), (4, 2, 64, 25, 25), (5, 1, 8, 8, 8)])
def test_cache_policy_matches_bruteforce_lru(seed, layers, experts, slots, maxreq):
    rng = random.Random(seed)
    cache = L.moe_cache_create_recording(_desc(layers, experts, slots), 1 << 40)
    model = LRUModel(layers, experts, slots)
    expected = []
    for step in range(300):
        l = rng.randrange(layers)
        n = rng.randint(1, maxreq)
        # Zipf-like popularity so that hits happen
        pool = sorted(range(experts), key=lambda e: rng.random() * (e + 1) ** 1.1)
        req = pool[:n]
        status, cmds = model.prefetch(l, req)
        if status == "capacity":
            with pytest.raises(L.MoEError) as ei:
                L.moe_cache_prefetch(cache, l, req)
            assert ei.value.status == L.MOE_E_CAPACITY
        else:
            ncopies = L.moe_cache_prefetch(cache, l, req)
            assert ncopies == sum(1 for c in cmds if c[0] == 2)
            expected += cmds
            slots_got, h = L.moe_cache_lookup(cache, l, req)
            assert all(s >= 0 for s in slots_got) and h == len(req)
        if rng.random() < 0.8:
            L.moe_cache_release(cache, l)
            expected += model.release(l)
    assert L.moe_cache_trace(cache) == expected
    hits, misses, nbytes = L.moe_cache_stats(cache)
    assert (hits, misses) == (model.hits, model.misses)
    assert nbytes == misses * L.moe_expert_bytes(256, 128)
    L.moe_cache_destroy(cache)


def test_cache_slot_addresses_and_capacity_rules():
    slab = L.moe_expert_bytes(256, 128)
    cache = L.moe_cache_create_recording(_desc(2, 16, 4), 1 << 40)
    assert L.moe_cache_prefetch(cache, 1, [3, 1, 2]) == 3
    slots, hits = L.moe_cache_lookup(cache, 1, [1, 2, 3, 4])
    assert slots == [0, 1, 2, -1] and hits == 3  # misses fill never-used slots in ascending id order
    # held slots cannot be evicted: 3 held + 2 new misses > 4 slots
    with pytest.raises(L.MoEError) as ei:
        L.moe_cache_prefetch(cache, 1, [5, 6])
    assert ei.value.status == L.MOE_E_CAPACITY
    with pytest.raises(L.MoEError) as ei:
        L.moe_cache_prefetch(cache, 1, [0, 1, 2, 3, 4])
    assert ei.value.status == L.MOE_E_CAPACITY
    L.moe_cache_release(cache, 1)
    assert L.moe_cache_prefetch(cache, 1, [5, 6]) == 2  # evicts LRU slot 3 (empty) then expert 1's slot 0
    slots, _ = L.moe_cache_lookup(cache, 1, [1, 2, 3, 5, 6])
    assert slots == [-1, 1, 2, 3, 0]
    trace = L.moe_cache_trace(cache)
    assert (1, 0, 0, -1) in trace  # copy into slot 0 waits for release 0 of layer 1
    with pytest.raises(L.MoEError) as ei:
        L.moe_cache_prefetch(cache, 1, [7, 7])
    assert ei.value.status == L.MOE_E_ARG
    with pytest.raises(L.MoEError) as ei:
        L.moe_cache_prefetch(cache, 2, [1])
    assert ei.value.status == L.MOE_E_ARG
    L.moe_cache_reset(cache)
    assert L.moe_cache_lookup(cache, 1, [2, 5])[1] == 0
    assert L.moe_cache_stats(cache) == (0, 0, 0)
    L.moe_cache_destroy(cache)
    assert slab == 61440


def test_cache_copy_failure_leaves_slot_empty():
    cache = L.moe_cache_create_recording(_desc(1, 16, 6), 1 << 40, fail_copy_at=3)
    with pytest.raises(L.MoEError) as ei:
        L.moe_cache_prefetch(cache, 0, [4, 7, 9, 11])
    assert ei.value.status == L.MOE_E_HIP
    slots, hits = L.moe_cache_lookup(cache, 0, [4, 7, 9, 11])
    assert slots[:2] == [0, 1] and slots[2:] == [-1, -1] and hits == 2
    # the request was un-held: a full-size request still fits and re-streams the failed ones
    assert L.moe_cache_prefetch(cache, 0, [4, 7, 9, 11, 12, 13]) == 4
    assert L.moe_cache_lookup(cache, 0, [9, 11])[1] == 2
    L.moe_cache_destroy(cache)


def test_cache_async_prefetch_and_wait():
    cache = L.moe_cache_create_recording(_desc(3, 16, 4), 1 << 40)
    # copies of layers 0 and 2 queued before either layer's wait
    assert L.moe_cache_prefetch_async(cache, 0, [5, 1]) == 2
    assert L.moe_cache_prefetch_async(cache, 2, [3]) == 1
    trace = L.moe_cache_trace(cache)
    assert [c[0] for c in trace] == [2, 2, 3, 3, 2, 3]  # copies and table writes only, no wait yet
    assert trace[0] == (2, 0, 1, 0) and trace[1] == (2, 0, 5, 1) and trace[4] == (2, 2, 3, 0)
    # release before the wait is refused; the slots stay held
    with pytest.raises(L.MoEError) as ei:
        L.moe_cache_release(cache, 0)
    assert ei.value.status == L.MOE_E_STATE
    L.moe_cache_wait(cache, 0)
    L.moe_cache_wait(cache, 0)  # nothing pending: no command
    L.moe_cache_wait(cache, 1)  # never prefetched: no command
    L.moe_cache_release(cache, 0)
    L.moe_cache_wait(cache, 2)
    L.moe_cache_release(cache, 2)
    trace = L.moe_cache_trace(cache)
    assert trace[6:] == [(4, 0, -1, -1), (5, 0, 0, 2), (4, 2, -1, -1), (5, 2, 0, 1)]
    # an all-hit request has nothing to wait for
    assert L.moe_cache_prefetch_async(cache, 0, [1]) == 0
    L.moe_cache_release(cache, 0)
    assert len(L.moe_cache_trace(cache)) == 11
    # the combined call equals async + wait
    assert L.moe_cache_prefetch(cache, 1, [7]) == 1
    assert L.moe_cache_trace(cache)[-1] == (4, 1, -1, -1)
    L.moe_cache_release(cache, 1)
    with pytest.raises(L.MoEError):
        L.moe_cache_wait(cache, 3)
    L.moe_cache_destroy(cache)


def test_cache_create_rejects_bad_descriptions():
    for d in (_desc(0, 16, 4), _desc(1, 16, 0), _desc(1, 16, 17), _desc(1, 16, 4, hidden=100)):
        with pytest.raises(L.MoEError):
            L.moe_cache_create_recording(d)


def test_route_ffn_combine_validation():
    ws = L.moe_route_ffn_combine_workspace_bytes(1, 256, 128, 16, 2, 1)
    assert ws >= L.moe_router_workspace_bytes(1, 16) + L.moe_expert_ffn_workspace_bytes(1, 256, 128, 16, 2, 1)
    args = [FAKE, 1, 256, 128, FAKE, None, 16, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws]
    assert _status(L.moe_route_ffn_combine, None, *args[1:]) == L.MOE_E_ARG
    bad = list(args); bad[4] = None  # router weights
    assert _status(L.moe_route_ffn_combine, *bad) == L.MOE_E_ARG
    bad = list(args); bad[2] = 250
    assert _status(L.moe_route_ffn_combine, *bad) == L.MOE_E_SHAPE
    bad = list(args); bad[7] = 17  # k > E
    assert _status(L.moe_route_ffn_combine, *bad) == L.MOE_E_SHAPE
    # a prefetch size without a pointer
    assert _status(L.moe_route_ffn_combine, *args, None, None, 4096) == L.MOE_E_ARG
    bad = list(args); bad[14] = ws - 1
    assert _status(L.moe_route_ffn_combine, *bad) == L.MOE_E_NOMEM
    L.moe_route_ffn_combine(None, 0, 256, 128, None, None, 16, 2, None, None, None, None, None, None, 0)


def test_residual_norm_validation():
    assert _status(L.moe_residual_norm, FAKE, FAKE, -1, 256, 1e-6, FAKE) == L.MOE_E_ARG
    assert _status(L.moe_residual_norm, FAKE, FAKE, 4, 0, 1e-6, FAKE) == L.MOE_E_ARG
    assert _status(L.moe_residual_norm, FAKE, FAKE, 4, 256, -1.0, FAKE) == L.MOE_E_ARG
    assert _status(L.moe_residual_norm, FAKE, FAKE, 4, 256, float("nan"), FAKE) == L.MOE_E_ARG
    assert _status(L.moe_residual_norm, FAKE, None, 4, 256, 1e-6, FAKE) == L.MOE_E_ARG
    assert _status(L.moe_residual_norm, None, FAKE, 4, 256, 1e-6, None) == L.MOE_E_ARG
    L.moe_residual_norm(None, None, 0, 256, 1e-6, None)  # no rows: nothing to do


def test_split_copies_validation_and_state():
    assert _status(L.moe_cache_split_copies, None, FAKE) == L.MOE_E_ARG
    desc = L.moe_cache_desc(2, 8, 256, 128, 4)
    c = L.moe_cache_create_recording(desc, 0x10000)
    try:
        L.moe_cache_split_copies(c, FAKE)  # a recording cache ignores the stream
        L.moe_cache_prefetch_async(c, 0, [1, 2])
        assert _status(L.moe_cache_split_copies, c, None) == L.MOE_E_STATE  # layer 0 not waited for
        L.moe_cache_wait(c, 0)
        L.moe_cache_split_copies(c, None)
    finally:
        L.moe_cache_destroy(c)


def test_mx_sizes_and_validation():
    """MXFP4 slab sizes, and the format entry points' checks (no kernel runs)."""
    assert L.moe_expert_bytes_mx(4096, 1536) == 3 * 4096 * 1536 * 17 // 32
    assert L.moe_expert_bytes_mx(96, 64) == 2 * 64 * 64 + 96 * 48  # rows of 51 -> 64 and 34 -> 48 bytes
    assert L.moe_expert_bytes_mx(100, 64) == 0
    ws = np.zeros(1 << 20, np.uint8)
    x = np.zeros((2, 4096), np.uint16)
    idx = np.zeros((2, 8), np.int32)
    w = np.zeros((2, 8), np.float32)
    out = np.zeros((2, 4096), np.uint16)
    table = np.zeros(128, np.int64)
    # T = 0: no-op
    L.moe_mx_expert_ffn_combine(x, 0, 4096, 1536, 128, idx, w, 8, table, None, out, ws, ws.size)
    with pytest.raises(L.MoEError) as e:  # I not a multiple of 32
        L.moe_mx_expert_ffn_combine(x, 2, 4096, 1000, 128, idx, w, 8, table, None, out, ws, ws.size)
    assert e.value.status == L.MOE_E_SHAPE
    with pytest.raises(L.MoEError) as e:  # several tokens: the grouped paths' workspace is checked first
        L.moe_mx_expert_ffn_combine(x, 2, 4096, 1536, 128, idx, w, 8, table, None, out, ws, 1024)
    assert e.value.status == L.MOE_E_NOMEM
    wr = np.zeros((128, 4096), np.float32)
    with pytest.raises(L.MoEError) as e:
        L.moe_mx_route_ffn_combine(x, 2, 4096, 1536, wr, None, 128, 8, table, None, idx, w, out, ws, 1024)
    assert e.value.status == L.MOE_E_NOMEM
    y = np.zeros((16, 4096), np.float32)
    for fmt in (-1, 3):  # formats 0, 1, 2 only
        with pytest.raises(L.MoEError) as e:
            L.moe_expert_ffn_fmt(x, 2, 4096, 1536, 128, idx, 8, table, None, None, y, ws, ws.size, L.MOE_FFN_AUTO,
                                 fmt)
        assert e.value.status == L.MOE_E_ARG
        with pytest.raises(L.MoEError) as e:
            L.moe_expert_gate_up_fmt(x, 2, 4096, 1536, 128, idx, 8, None, None, None, table, None, None, y,
                                     L.MOE_FFN_PAIRS, fmt)
        assert e.value.status == L.MOE_E_ARG
    d = L.moe_cache_desc(1, 4, 64, 32, 2, 3)
    with pytest.raises(L.MoEError) as e:
        L.moe_cache_create_recording(d)
    assert e.value.status == L.MOE_E_ARG


def test_superblock_sizes_and_validation():
    assert L.moe_expert_bytes_sb(4096, 1536) == 3 * 4096 * 1536 * 9 // 16
    assert L.moe_expert_bytes_sb(4096, 1504) == 0 and L.moe_expert_bytes_sb(96, 256) == 0
    ws = np.zeros(1 << 20, np.uint8)
    x = np.zeros((2, 4096), np.uint16)
    idx = np.zeros((2, 8), np.int32)
    w = np.zeros((2, 8), np.float32)
    out = np.zeros((2, 4096), np.uint16)
    table = np.zeros(128, np.int64)
    for T, H, I in ((2, 4096, 1504), (1, 4096, 1024 + 32), (2, 4000, 1536)):  # H, I multiples of 256 only
        with pytest.raises(L.MoEError) as e:
            L.moe_sb_expert_ffn_combine(x, T, H, I, 128, idx, w, 8, table, None, out, ws, ws.size)
        assert e.value.status == L.MOE_E_SHAPE, (T, H, I)
    y = np.zeros((16, 4096), np.float32)
    with pytest.raises(L.MoEError) as e:
        L.moe_expert_down_fmt(x, 2, 4096, 1504, 128, idx, 8, None, None, None, table, None, None, y,
                              L.MOE_FFN_PAIRS, 2)
    assert e.value.status == L.MOE_E_SHAPE
    with pytest.raises(L.MoEError) as e:
        L.moe_cache_create_recording(L.moe_cache_desc(1, 4, 64, 32, 2, 2))
    assert e.value.status == L.MOE_E_SHAPE
    with pytest.raises(L.MoEError) as e:
        L.moe_cache_create_recording(L.moe_cache_desc(1, 4, 64, 32, 2, 3))
    assert e.value.status == L.MOE_E_ARG


@pytest.mark.parametrize("seed,experts,slots,k,tokens", [(11, 16, 4, 2, 6), (12, 64, 25, 8, 8), (13, 256, 102, 8, 64),
                                                        (14, 32, 1, 2, 3)])
def test_step_plan_drives_overflowing_layers_through_the_abi(seed, experts, slots, k, tokens):
    """The step plan of moe_cache_plan, then every wave through the ABI alone
    (prefetch, wait, release): waves fit the slots, hits come first, every
    request succeeds, and the recorded commands equal the brute-force LRU model
    driven by the documented plan."""
    rng = np.random.default_rng(seed)
    cache = L.moe_cache_create_recording(_desc(2, experts, slots), 1 << 40)
    model = LRUModel(2, experts, slots)
    expected = []
    half = max(1, slots // 2)
    max_waves = (experts + half - 1) // half + 2
    for step in range(40):
        l = step % 2
        ids = np.stack([rng.choice(experts, k, replace=False) for _ in range(tokens)]).astype(np.int32)
        needed = sorted(set(ids.ravel().tolist()))
        masks = np.full((max_waves, experts), 7, np.uint8)
        waves = L.moe_cache_plan(cache, l, ids, masks=masks)
        # the documented plan
        resident = [e for e in needed if e in model.slot_of[l]]
        order = resident + [e for e in needed if e not in model.slot_of[l]]
        if len(order) <= slots:
            assert waves == [sorted(order)]
        else:  # small first and last waves, between them the fewest of at most half the slots, balanced
            edge = max(1, half // 8)
            mid = len(order) - 2 * edge
            nw = -(-mid // half)
            sizes = [edge] + [mid // nw + (1 if v < mid % nw else 0) for v in range(nw)] + [edge]
            assert max(sizes) <= half
            bounds = np.cumsum([0] + sizes)
            assert waves == [sorted(order[bounds[v]:bounds[v + 1]]) for v in range(len(sizes))]
        assert all(len(v) <= slots for v in waves)
        for v in range(max_waves):
            want = np.zeros(experts, np.uint8)
            if v < len(waves):
                want[waves[v]] = 1
            assert np.array_equal(masks[v], want)
        for wave in waves:
            status, cmds = model.prefetch(l, wave)
            assert status == "ok"
            L.moe_cache_prefetch_async(cache, l, wave)
            L.moe_cache_wait(cache, l)
            L.moe_cache_release(cache, l)
            expected += cmds + model.release(l)
    assert L.moe_cache_trace(cache) == expected
    assert L.moe_cache_stats(cache)[:2] == (model.hits, model.misses)
    # validation: too few waves, an id out of range, NULL outputs
    if slots < experts:
        big = np.arange(experts, dtype=np.int32)
        assert _status(L.moe_cache_plan, cache, 0, big, 1) == L.MOE_E_CAPACITY
    assert _status(L.moe_cache_plan, cache, 0, [experts], 4) == L.MOE_E_ARG
    assert _status(L.moe_cache_plan, cache, 2, [0], 4) == L.MOE_E_ARG
    assert L.moe_cache_plan(cache, 0, [], 4) == []
    L.moe_cache_destroy(cache)


def test_step_plan_equals_per_layer_plans_and_issues_single_wave_layers():
    """moe_cache_plan_step plans every layer as moe_cache_plan does and queues
    the copies of the layers that fit their slots, in layer order."""
    rng = np.random.default_rng(5)
    E, C, Ln, n = 64, 20, 4, 24
    a = L.moe_cache_create_recording(_desc(Ln, E, C), 1 << 40)
    b = L.moe_cache_create_recording(_desc(Ln, E, C), 1 << 40)
    half = C // 2
    mw = (E + half - 1) // half + 2
    for step in range(6):
        ids = np.stack([rng.choice(E, n, replace=(l % 2 == 1)) for l in range(Ln)]).astype(np.int32)
        ids[0, :] = rng.integers(0, 5, n)  # a layer with few distinct experts
        ne = np.empty((Ln, n), np.int32)
        st = np.empty((Ln, mw + 1), np.int32)
        nw = np.empty(Ln, np.int32)
        masks = np.empty((Ln, mw, E), np.uint8)
        copies = L.moe_cache_plan_step(a, ids, n, ne, st, mw, masks, nw, True)
        expect_copies = 0
        for l in range(Ln):
            mref = np.empty((mw, E), np.uint8)
            waves = L.moe_cache_plan(b, l, ids[l], masks=mref)
            assert nw[l] == len(waves)
            assert [ne[l, st[l, v]:st[l, v + 1]].tolist() for v in range(nw[l])] == waves
            assert np.array_equal(masks[l], mref)
            if len(waves) == 1:
                expect_copies += L.moe_cache_prefetch_async(b, l, waves[0])
        assert copies == expect_copies
        for l in range(Ln):
            if nw[l] == 1:
                L.moe_cache_wait(a, l)
                L.moe_cache_release(a, l)
                L.moe_cache_wait(b, l)
                L.moe_cache_release(b, l)
            else:
                for v in range(nw[l]):
                    wave = ne[l, st[l, v]:st[l, v + 1]]
                    assert L.moe_cache_prefetch(a, l, wave) == L.moe_cache_prefetch(b, l, wave.tolist())
                    L.moe_cache_release(a, l)
                    L.moe_cache_release(b, l)
        assert L.moe_cache_trace(a) == L.moe_cache_trace(b)
    L.moe_cache_destroy(a)
    L.moe_cache_destroy(b)
