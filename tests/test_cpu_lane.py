"""The CPU lane (experts computed on host cores from host slabs) against the oracle,
on the CPU: no GPU is involved in this lane.

Bars: y within 2e-2 * max|ref| of the fp64 oracle per (token, expert) (fp32 sums
with h rounded once to bf16, like the GPU kernels); bit-identical results for any
thread count and for every instruction-set version this CPU runs; job tickets
complete in order.
"""
import numpy as np
import pytest

import oracle
import synth
from routed_expert_streaming_amd import _lib as L

SEED = 20261209


def run_lane(lane, slab, H, I, xs):
    """xs [M, H] bf16 bits -> y [M, H] fp32 through one job."""
    M = xs.shape[0]
    xs = np.ascontiguousarray(xs)
    y = np.full((M, H), np.nan, np.float32)
    t = L.moe_cpu_lane_submit(lane, slab, H, I, M, [xs[i].ctypes.data for i in range(M)],
                              [y[i].ctypes.data for i in range(M)])
    L.moe_cpu_lane_wait(lane, t)
    return y


@pytest.fixture(scope="module")
def lane():
    h = L.moe_cpu_lane_create(4)
    yield h
    L.moe_cpu_lane_destroy(h)


@pytest.mark.parametrize("H,I,M", [(256, 128, 1), (96, 64, 11), (4096, 1536, 1), (6144, 2048, 2), (128, 96, 8)])
def test_lane_matches_oracle(lane, H, I, M):
    slab = synth.expert_slab(SEED, 0, H + I + M, H, I)
    xs = synth.x_bf16(SEED, 1, M, M, H)
    y = run_lane(lane, slab, H, I, xs)
    assert np.isfinite(y).all()
    for t in range(M):
        xd = np.array([oracle.bf16_to_double(int(b)) for b in xs[t]])
        ref = oracle.expert_ffn(slab, H, I, xd)[3]
        err = np.abs(y[t].astype(np.float64) - ref).max() / np.abs(ref).max()
        assert err <= 2e-2, (H, I, M, t, err)
        print(f"H{H} I{I} token {t}: max err / max|ref| = {err:.2e}")


def test_constant_expert_closed_form(lane):
    """Every weight of W1, W3, W2 equal: g = u = w*sum(x), h = bf16(silu(g)*u),
    y[r] = w * I * h (h is the same for every row)."""
    from tests.slabkit import build_slab, constant_matrix
    H, I = 64, 32
    w = 0.25 * (3 - 8)  # scale 0.25, code 3, min -8 * scale
    m1 = constant_matrix(I, H, 3, 0.25)
    m2 = constant_matrix(H, I, 3, 0.25)
    slab = build_slab(H, I, m1, m1, m2)
    xs = np.array([[synth.double_to_bf16(0.01 * (c % 7) - 0.02) for c in range(H)]], np.uint16)
    y = run_lane(lane, slab, H, I, xs)
    xsum = sum(oracle.bf16_to_double(int(b)) for b in xs[0])
    g = w * xsum
    h = oracle.bf16_to_double(oracle.double_to_bf16(g / (1 + np.exp(-g)) * g))
    np.testing.assert_allclose(y[0], np.full(H, w * I * h), rtol=1e-5)


def test_thread_count_and_isa_do_not_change_bits():
    H, I, M = 256, 192, 9
    slab = synth.expert_slab(SEED, 1, 7, H, I)
    xs = synth.x_bf16(SEED, 2, 0, M, H)
    results = []
    for threads in (1, 3, 8):
        h = L.moe_cpu_lane_create(threads)
        try:
            for isa in (0, 256, 512):
                if isa > L.moe_cpu_lane_isa():
                    continue
                L.moe_cpu_lane_force_isa(h, isa)
                results.append(((threads, isa), run_lane(h, slab, H, I, xs)))
        finally:
            L.moe_cpu_lane_destroy(h)
    base = results[0][1].view(np.uint32)
    for key, y in results[1:]:
        assert (y.view(np.uint32) == base).all(), key


def test_tickets_complete_in_order_and_validation():
    H, I = 128, 64
    lane = L.moe_cpu_lane_create(3)
    try:
        slabs = [synth.expert_slab(SEED, 2, e, H, I) for e in range(5)]
        xs = synth.x_bf16(SEED, 3, 0, 2, H)
        ys = [np.full((2, H), np.nan, np.float32) for _ in slabs]
        tickets = [L.moe_cpu_lane_submit(lane, s, H, I, 2, [xs[0].ctypes.data, xs[1].ctypes.data],
                                         [y[0].ctypes.data, y[1].ctypes.data]) for s, y in zip(slabs, ys)]
        assert tickets == sorted(tickets) and len(set(tickets)) == 5
        L.moe_cpu_lane_wait(lane, tickets[-1])  # covers every earlier job
        for s, y in zip(slabs, ys):
            assert (y.view(np.uint32) == run_lane(lane, s, H, I, xs).view(np.uint32)).all()
        last = L.moe_cpu_lane_submit(lane, slabs[0], H, I, 0, [], [])
        assert last == tickets[-1] + 5  # M = 0: the last job's ticket
        L.moe_cpu_lane_wait(lane, last)
        with pytest.raises(L.MoEError) as e:
            L.moe_cpu_lane_wait(lane, last + 1)
        assert e.value.status == L.MOE_E_ARG
        x0 = [xs[0].ctypes.data]
        y0 = [ys[0][0].ctypes.data]
        for args, status in [((slabs[0], 100, I, 1, x0, y0), L.MOE_E_SHAPE), ((slabs[0], H, 0, 1, x0, y0), L.MOE_E_SHAPE),
                             ((slabs[0], H, I, -1, x0, y0), L.MOE_E_ARG), ((None, H, I, 1, x0, y0), L.MOE_E_ARG),
                             ((slabs[0], H, I, 1, [0], y0), L.MOE_E_ARG)]:
            with pytest.raises(L.MoEError) as e:
                L.moe_cpu_lane_submit(lane, *args)
            assert e.value.status == status, args
        with pytest.raises(L.MoEError) as e:
            L.moe_cpu_lane_force_isa(lane, 128)
        assert e.value.status == L.MOE_E_ARG
    finally:
        L.moe_cpu_lane_destroy(lane)
    for n in (0, 257):
        with pytest.raises(L.MoEError) as e:
            L.moe_cpu_lane_create(n)
        assert e.value.status == L.MOE_E_ARG


def test_assign_lanes_earliest_finish_and_list_scheduling_bound():
    """The cost model's assignment: each miss to the lane that finishes it first
    (ties to the copy engine); its makespan is within one job of the best split
    over every assignment (the bound of greedy list scheduling on two lanes)."""
    import itertools
    from routed_expert_streaming_amd.runtime import assign_lanes
    inf = float("inf")
    misses = [(0, e, 1) for e in range(5)]
    assert assign_lanes(misses, 1.0, lambda m: inf)[0] == [False] * 5
    assert assign_lanes(misses, inf, lambda m: 1.0)[0] == [True] * 5
    # copy 2, cpu 3: finishes 2 | 3 | 4 | 6=6 (tie: copy) | 6 ...
    assert assign_lanes(misses, 2.0, lambda m: 3.0)[0] == [False, True, False, False, True]
    rng = np.random.default_rng(7)
    for _ in range(200):
        n = int(rng.integers(1, 9))
        toks = rng.integers(1, 9, n)
        t_copy = float(rng.uniform(0.5, 2.0))
        a, b = float(rng.uniform(0.2, 2.0)), float(rng.uniform(0.0, 0.3))
        t_cpu = lambda m: a + b * (m - 1)
        ms = [(0, i, int(t)) for i, t in enumerate(toks)]
        lanes, cb, pb = assign_lanes(ms, t_copy, t_cpu)
        assert np.isclose(cb, t_copy * (len(lanes) - sum(lanes)))
        assert np.isclose(pb, sum(t_cpu(int(t)) for t, c in zip(toks, lanes) if c))
        best = min(max(t_copy * sum(1 for c in cs if not c), sum(t_cpu(int(t)) for t, c in zip(toks, cs) if c))
                   for cs in itertools.product([False, True], repeat=n))
        assert max(cb, pb) <= best + max(t_copy, max(t_cpu(int(t)) for t in toks)) + 1e-12
