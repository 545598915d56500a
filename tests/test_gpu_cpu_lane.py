"""GPU parity of streamed steps with a CPU lane: some cache misses computed on
host cores from the pinned pool while the GPU computes the rest.

Bars: expert indices bit-exact against the oracle router; every layer's output
within 2e-2 * max|ref| of the oracle (the CPU lane's rows and the GPU's combined
as usual); the cache's hits and misses equal to a brute-force LRU replay of the
requests the GPU lane made (the CPU lane's experts bypass the cache); with
nothing sent to the CPU lane the step is bit-identical to a stack without one.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from routed_expert_streaming_amd import _lib as L
from routed_expert_streaming_amd.runtime import MoEStack
from tests.test_abi_cpu import LRUModel
from tests.test_gpu_parity import check_close


def pool_slabs(st: MoEStack, l: int):
    """Layer l's routed slabs as views of the pinned host pool the lanes read."""
    return st.host_pool_slabs(l)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name,layers,steps,rows", [
    ("decode1_stream", 3, 4, None),
    ("decode32_stream", 2, 2, list(range(0, 32, 3))),
])
def test_streamed_with_cpu_lane_against_oracle(name, layers, steps, rows):
    cfg = synth.get(name)
    st = MoEStack(cfg, layers=layers, cpu_lane=4)
    k = cfg.top_k
    try:
        assert st.streaming and st.lane
        # every other miss of each layer to the CPU lane, so both lanes always work
        st.lane_pick = lambda l, misses: misses[::2]
        wr = [st.wr[l].cpu().numpy() for l in range(layers)]
        bias = [None if st.bias is None else st.bias[l].cpu().numpy() for l in range(layers)]
        model = LRUModel(layers, 10 ** 6, st.C)
        out = st.new_output()
        n_cpu = 0
        for s in range(steps):
            x = st.make_inputs(s)
            r = st.forward(x, out)
            torch.cuda.synchronize()
            n_cpu += r.cpu_experts
            xb, ob, idx = bits(x), bits(out), st.idx.cpu().numpy()
            for l in range(layers):
                needed = sorted(set(int(e) for e in idx[l].ravel()))
                gpu_side = [e for e in needed if e not in st.last_cpu_sets[l]]
                assert model.prefetch(l, gpu_side)[0] == "ok"
                model.release(l)
                o = oracle.moe_layer(xb[l], wr[l], bias[l], k, pool_slabs(st, l), st.host_shared(l), cfg.inter,
                                     rows=rows)
                sel = slice(None) if rows is None else rows
                assert (o["idx"][sel] == idx[l][sel]).all(), (name, s, l)
                ratio = check_close(ob[l][sel], o["out64"][sel], f"{name} step {s} layer {l}")
                print(f"{name} step {s} layer {l}: CPU lane {sorted(st.last_cpu_sets[l])}, "
                      f"max err / max|ref| = {ratio:.2e}")
        hits, misses, nbytes = st.stats()
        assert (hits, misses) == (model.hits, model.misses)
        assert nbytes == misses * st.slab
        assert n_cpu > 0
    finally:
        st.close()


def test_cpu_lane_cost_model_run_and_empty_pick_is_identical():
    cfg = synth.get("decode1_stream")
    layers, steps = 2, 3
    plain = MoEStack(cfg, layers=layers)
    ref = []
    out = plain.new_output()
    for s in range(steps):
        plain.forward(plain.make_inputs(s), out)
        torch.cuda.synchronize()
        ref.append(bits(out))
    plain.close()
    st = MoEStack(cfg, layers=layers, cpu_lane=4)
    try:
        assert st.t_cpu1 > 0 and st.t_cpu8 >= 0
        st.lane_pick = lambda l, misses: []
        out = st.new_output()
        for s in range(steps):
            r = st.forward(st.make_inputs(s), out)
            torch.cuda.synchronize()
            assert r.cpu_experts == 0
            assert (bits(out) == ref[s]).all()
        # the cost model itself, a few steps: outputs stay within the bar
        st.lane_pick = None
        wr = [st.wr[l].cpu().numpy() for l in range(layers)]
        bias = [st.bias[l].cpu().numpy() for l in range(layers)]
        for s in range(steps, steps + 3):
            x = st.make_inputs(s)
            r = st.forward(x, out)
            torch.cuda.synchronize()
            xb, ob = bits(x), bits(out)
            for l in range(layers):
                o = oracle.moe_layer(xb[l], wr[l], bias[l], cfg.top_k, pool_slabs(st, l), st.host_shared(l), cfg.inter)
                check_close(ob[l], o["out64"], f"cost model step {s} layer {l}")
            print(f"step {s}: {r.cpu_experts} experts on the CPU lane (t_cpu 1 token {st.t_cpu1 * 1e3:.3f} ms)")
    finally:
        st.close()


def test_chained_with_cpu_lane_against_oracle():
    """Chained layers with the lane (every other miss of a layer on the host):
    layer by layer on the GPU's own inputs, indices bit-exact and outputs within
    the bar; the residual step reproduces the next layer's input."""
    from routed_expert_streaming_amd.runtime import RMS_EPS
    from tests.test_gpu_chained import bf16_ulps
    cfg = synth.get("decode1_stream")
    layers, k = 3, cfg.top_k
    st = MoEStack(cfg, layers=layers, cpu_lane=4)
    try:
        st.lane_pick = lambda l, misses: misses[::2]
        resid, xs = st.chain_buffers()
        out = st.new_output()
        wr = [st.wr[l].cpu().numpy() for l in range(layers)]
        bias = [st.bias[l].cpu().numpy() for l in range(layers)]
        n_cpu = 0
        for s in range(3):
            h0 = st.make_inputs(s)[0]
            c = st.forward_chained(h0, xs, resid, out)
            torch.cuda.synchronize()
            n_cpu += c.cpu_experts
            xb, ob, idx = bits(xs), bits(out), st.idx.cpu().numpy()
            ref_resid = np.zeros((cfg.tokens, cfg.hidden), np.float32)
            x_ref = oracle.residual_norm(bits(h0), ref_resid, RMS_EPS)
            assert bf16_ulps(xb[0], x_ref).max() <= 1
            for l in range(layers):
                o = oracle.moe_layer(xb[l], wr[l], bias[l], k, pool_slabs(st, l), st.host_shared(l), cfg.inter)
                assert (o["idx"] == idx[l]).all(), (s, l)
                check_close(ob[l], o["out64"], f"chained lane step {s} layer {l}")
                if l + 1 < layers:
                    x_ref = oracle.residual_norm(ob[l], ref_resid, RMS_EPS)
                    assert bf16_ulps(xb[l + 1], x_ref).max() <= 1
        assert n_cpu > 0
    finally:
        st.close()


def test_cpu_lane_with_layers_in_waves_against_oracle():
    """The lane beside layers whose GPU experts still exceed their slots: the
    32-token decode shape at a cap of 10% (25 slots per layer), every other miss
    of a layer on the host; the rest run in the library's waves (resident first).
    Indices bit-exact, every output within the bar, and the cache's hits and
    misses equal to an LRU replay of the documented waves of the GPU's experts."""
    from tests.test_gpu_parity import documented_waves
    cfg = synth.get("decode32_stream")
    layers, steps, k = 2, 2, cfg.top_k
    rows = list(range(0, 32, 3))
    st = MoEStack(cfg, layers=layers, cap=0.10, cpu_lane=4)
    try:
        assert st.streaming and st.lane and st.C == 25
        st.lane_pick = lambda l, misses: misses[::2]
        wr = [st.wr[l].cpu().numpy() for l in range(layers)]
        bias = [st.bias[l].cpu().numpy() for l in range(layers)]
        model = LRUModel(layers, 10 ** 6, st.C)
        out = st.new_output()
        n_cpu = most_waves = 0
        for s in range(steps):
            x = st.make_inputs(s)
            r = st.forward(x, out)
            torch.cuda.synchronize()
            n_cpu += r.cpu_experts
            xb, ob, idx = bits(x), bits(out), st.idx.cpu().numpy()
            for l in range(layers):
                needed = sorted(set(int(e) for e in idx[l].ravel()))
                gpu_side = [e for e in needed if e not in st.last_cpu_sets[l]]
                resident = [e for e in gpu_side if e in model.slot_of[l]]
                order = resident + [e for e in gpu_side if e not in model.slot_of[l]]
                waves = documented_waves(order, st.C)
                most_waves = max(most_waves, len(waves))
                for wave in waves:
                    assert model.prefetch(l, wave)[0] == "ok"
                    model.release(l)
                o = oracle.moe_layer(xb[l], wr[l], bias[l], k, pool_slabs(st, l), st.host_shared(l), cfg.inter,
                                     rows=rows)
                assert (o["idx"][rows] == idx[l][rows]).all(), (s, l)
                ratio = check_close(ob[l][rows], o["out64"][rows], f"lane + waves step {s} layer {l}")
                print(f"step {s} layer {l}: {len(st.last_cpu_sets[l])} experts on the CPU lane, {len(waves)} GPU "
                      f"waves, max err / max|ref| = {ratio:.2e}")
        hits, misses, nbytes = st.stats()
        assert (hits, misses) == (model.hits, model.misses)
        assert n_cpu > 0 and most_waves > 1  # the lane ran beside layers in waves
    finally:
        st.close()


def test_scatter_rows_places_rows_exactly():
    """moe_scatter_rows: dst[rows[i]] = src[i], bit for bit; other rows untouched."""
    rng = np.random.default_rng(7)
    for n, H, R in [(1, 4, 3), (37, 256, 100), (700, 6144, 2048)]:
        src = torch.from_numpy(rng.standard_normal((n, H)).astype(np.float32)).cuda()
        rows_np = rng.permutation(R)[:n].astype(np.int32)
        rows = torch.from_numpy(rows_np).cuda()
        dst0 = rng.standard_normal((R, H)).astype(np.float32)
        dst = torch.from_numpy(dst0.copy()).cuda()
        L.moe_scatter_rows(src, rows, n, H, dst)
        torch.cuda.synchronize()
        want = dst0.copy()
        want[rows_np] = src.cpu().numpy()
        assert np.array_equal(dst.cpu().numpy().view(np.uint32), want.view(np.uint32)), (n, H, R)
