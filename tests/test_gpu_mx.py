"""GPU parity of the MXFP4 (format 1) and super-block (format 2) weight formats
(one-token decode: the fused one-token kernels, and the separate gate/up and
down calls) against the oracle.

Bars: expert indices bit-exact; outputs within 2e-2 * max|ref| of the fp64
oracle reading the same MXFP4 slabs; the one-call layer bit-identical to the
router followed by the MXFP4 FFN + combine call; streamed == resident bit for
bit, with the cache's hits and misses equal to a brute-force LRU replay.
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


@pytest.mark.parametrize("name", ["decode1_mx", "decode1_sb"])
@pytest.mark.parametrize("over", [
    {},                                                        # H4096 I1536, 128 experts + shared, top-8
    {"hidden": 2048, "inter": 2048, "experts": 32, "layers": 2},  # routed variant with one block per lane
    {"hidden": 6144, "inter": 2048, "experts": 24, "layers": 2},  # H above the fused router's range
    {"experts": 16, "shared": 0, "top_k": 4, "layers": 2},
])
def test_format_layers_match_oracle_and_split_calls(name, over):
    cfg = synth.get(name, **over)
    layers = min(cfg.layers, 2)
    st = MoEStack(cfg, layers=layers)
    try:
        assert not st.streaming and st.fmt == cfg.fmt
        for s in range(2):
            x = st.make_inputs(s)
            out = st.new_output()
            st.forward(x, out)  # one call per layer
            torch.cuda.synchronize()
            idx1, ob = st.idx.cpu().numpy().copy(), bits(out)
            # router, then the MXFP4 FFN + combine call: the same bits
            out2 = st.new_output()
            for l in range(layers):
                st.route(x, l)
                st.ffn_combine(x, l, out2)
            torch.cuda.synchronize()
            assert (st.idx.cpu().numpy() == idx1).all()
            assert (bits(out2) == ob).all()
            xb = bits(x)
            # the separate gate/up and down calls on these slabs (the dequant-GEMV
            # in pair grouping), then the combine: checked against the oracle too
            out3 = st.new_output()
            h = torch.empty((st.T * st.k + (st.T if st.has_shared else 0), cfg.inter), dtype=torch.bfloat16,
                            device="cuda")
            for l in range(layers):
                st.gate_up_only(x, l, h)
                st.down_only(h, l)
                st.combine(l, out3)
            torch.cuda.synchronize()
            o3 = bits(out3)
            for l in range(layers):
                wr = st.wr[l].cpu().numpy()
                bias = None if st.bias is None else st.bias[l].cpu().numpy()
                o = oracle.moe_layer(xb[l], wr, bias, cfg.top_k, st.host_slabs(l), st.host_shared(l), cfg.inter,
                                     fmt=cfg.fmt)
                assert (o["idx"] == idx1[l]).all()
                ratio = check_close(ob[l], o["out64"], f"{name} {over} step {s} layer {l}")
                ratio3 = check_close(o3[l], o["out64"], f"{name} {over} step {s} layer {l} (two calls)")
                print(f"{name} {over} step {s} layer {l}: max err / max|ref| = {ratio:.2e} (two calls {ratio3:.2e})")
    finally:
        st.close()


@pytest.mark.parametrize("name", ["decode1_mx_stream", "decode1_sb_stream"])
def test_format_streamed_equals_resident_and_lru(name):
    cfg = synth.get(name)
    layers, steps = 3, 4
    streamed = MoEStack(cfg, layers=layers)
    resident = MoEStack(cfg, layers=layers, cap=1.0)
    try:
        assert streamed.streaming and not resident.streaming
        model = LRUModel(layers, 10 ** 6, streamed.C)
        o1, o2 = streamed.new_output(), resident.new_output()
        for s in range(steps):
            x = streamed.make_inputs(s)
            streamed.forward(x, o1)
            resident.forward(x, o2)
            torch.cuda.synchronize()
            assert (bits(o1) == bits(o2)).all(), s
            idx = streamed.idx.cpu().numpy()
            assert (idx == resident.idx.cpu().numpy()).all()
            for l in range(layers):
                assert model.prefetch(l, sorted(set(int(e) for e in idx[l].ravel())))[0] == "ok"
                model.release(l)
        hits, misses, nbytes = streamed.stats()
        assert (hits, misses) == (model.hits, model.misses) and nbytes == misses * streamed.slab
        assert streamed.slab == 4096 * 1536 * 3 * (17 if cfg.fmt == 1 else 18) // 32
    finally:
        streamed.close()
        resident.close()
