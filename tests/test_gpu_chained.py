"""GPU parity of chained layers: the residual-stream kernel against the oracle,
and a chained streamed run (with and without gating lookahead) against the
chained resident run and, layer by layer with the GPU's own inputs, the oracle.

Bars: the fp32 residual update bit-exact; the normalised bf16 row within one
bf16 ulp of the fp64 oracle (the kernel's fp32 mean square decides the rounding
of a value within an ulp of a tie); expert indices bit-exact; layer outputs
within 2e-2 * max|ref|; streamed == resident bit for bit; cache hits and misses
equal to a brute-force LRU replay of the recorded requests.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from routed_expert_streaming_amd import _lib as L
from routed_expert_streaming_amd.runtime import RMS_EPS, MoEStack
from tests.test_abi_cpu import LRUModel
from tests.test_gpu_parity import bf16_dev, check_close

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


def bf16_ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps (sign-magnitude bit patterns mapped to a line)."""
    ia = a.astype(np.int64)
    ib = b.astype(np.int64)
    ia = np.where(ia & 0x8000, -(ia & 0x7FFF), ia)
    ib = np.where(ib & 0x8000, -(ib & 0x7FFF), ib)
    return np.abs(ia - ib)


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    return np.array([oracle.double_to_bf16(float(x)) for x in v.ravel()], np.uint16).reshape(v.shape)


@pytest.mark.parametrize("T,H", [(5, 6144), (1, 4096), (3, 96), (2, 32)])
def test_residual_norm_matches_oracle(T, H):
    rng = np.random.default_rng(1000 * T + H)
    resid = (rng.standard_normal((T, H)) * 30.0).astype(np.float32)
    add = to_bf16_bits(rng.standard_normal((T, H)) * 50.0)
    r_d = torch.from_numpy(resid.copy()).cuda()
    x_d = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    L.moe_residual_norm(bf16_dev(add), r_d, T, H, RMS_EPS, x_d)
    torch.cuda.synchronize()
    ref_r = resid.copy()
    ref_x = oracle.residual_norm(add, ref_r, RMS_EPS)
    assert (r_d.cpu().numpy() == ref_r).all()
    d = bf16_ulps(bits(x_d), ref_x)
    assert d.max() <= 1 and (d > 0).mean() < 0.01, (int(d.max()), float((d > 0).mean()))
    # without an addend the residual is only normalised
    x2 = torch.empty_like(x_d)
    L.moe_residual_norm(None, r_d, T, H, 0.0, x2)
    torch.cuda.synchronize()
    assert (r_d.cpu().numpy() == ref_r).all()
    d2 = bf16_ulps(bits(x2), oracle.residual_norm(None, ref_r.copy(), 0.0))
    assert d2.max() <= 1


def run_chain(stack: MoEStack, steps: int, lookahead: bool):
    resid, xs = stack.chain_buffers()
    out = stack.new_output()
    res = []
    for s in range(steps):
        h0 = stack.make_inputs(s)[0]
        st = stack.forward_chained(h0, xs, resid, out, lookahead=lookahead)
        torch.cuda.synchronize()
        res.append({"h0": bits(h0), "xs": bits(xs), "out": bits(out), "idx": stack.idx.cpu().numpy().copy(),
                    "pidx": stack.pidx.cpu().numpy().copy(), "st": st})
    return res


def lru_replay_chained(run, layers, C, m):
    model = LRUModel(layers, 10 ** 6, C)
    for r in run:
        for l in range(layers):
            assert model.prefetch(l, sorted(set(int(e) for e in r["idx"][l].ravel())))[0] == "ok"
            if m and l + 1 < layers:
                assert model.prefetch(l + 1, sorted(set(int(e) for e in r["pidx"][l + 1][:, :m].ravel())))[0] == "ok"
            model.release(l)
    return model.hits, model.misses


def test_chained_streaming_lookahead_equals_resident_and_oracle():
    cfg = synth.get("decode1_stream")
    layers, steps = 3, 4
    streamed = MoEStack(cfg, layers=layers)
    assert streamed.streaming
    runs, stats = {}, {}
    k = cfg.top_k
    for la in (0, 2, k):
        streamed.reset_cache()
        runs[la] = run_chain(streamed, steps, la)
        stats[la] = streamed.stats()
        hits, misses, nbytes = stats[la]
        assert (hits, misses) == lru_replay_chained(runs[la], layers, streamed.C, la)
        assert nbytes == misses * streamed.slab
    wr = [streamed.wr[l].cpu().numpy() for l in range(layers)]
    bias = [streamed.bias[l].cpu().numpy() for l in range(layers)]
    streamed.close()
    resident = MoEStack(cfg, layers=layers, cap=1.0)
    ref = run_chain(resident, steps, 0)
    for la in (0, 2, k):
        for a, b in zip(runs[la], ref):
            assert (a["xs"] == b["xs"]).all() and (a["out"] == b["out"]).all()
            assert (a["idx"] == b["idx"]).all()
    for la in (2, k):
        st = [r["st"] for r in runs[la]]
        routed, predicted = sum(s.routed for s in st), sum(s.predicted for s in st)
        assert routed == sum(len(set(r["idx"][l].ravel())) for r in runs[la] for l in range(1, layers))
        assert 0 <= predicted <= routed
        print(f"lookahead {la}: {predicted}/{routed} routed experts named by the prediction, "
              f"{sum(s.ahead_copies for s in st)} copied ahead ({sum(s.ahead_unused for s in st)} unused); "
              f"hits/misses {stats[la][:2]} (without lookahead {stats[0][:2]})")

    # layer by layer on the GPU's own inputs (step 0): the oracle's layer and
    # residual step reproduce the chain
    r0 = ref[0]
    T, H = cfg.tokens, cfg.hidden
    ref_resid = np.zeros((T, H), np.float32)
    x_ref = oracle.residual_norm(r0["h0"], ref_resid, RMS_EPS)
    assert bf16_ulps(r0["xs"][0], x_ref).max() <= 1
    for l in range(layers):
        o = oracle.moe_layer(r0["xs"][l], wr[l], bias[l], cfg.top_k, resident.host_slabs(l),
                             resident.host_shared(l), cfg.inter)
        assert (o["idx"] == r0["idx"][l]).all()
        check_close(r0["out"][l], o["out64"], f"chained layer {l}")
        if l + 1 < layers:
            x_ref = oracle.residual_norm(r0["out"][l], ref_resid, RMS_EPS)
            assert bf16_ulps(r0["xs"][l + 1], x_ref).max() <= 1
    resident.close()
