"""Parity at full size, in the launch configuration bench.py times: the streamed
32-token decode and 2048-token prefill configurations over all 16 layers,
against the oracle.  The oracle reads the experts from the same pinned host pool
the cache streams from (layers 8-15 hold the expert weights of layers 0-7: the
full 90 GiB pool is more than one process may page-lock on the test machine;
every layer keeps its own router, inputs, cache slots and misses).

Bars: every layer's expert indices bit-exact for every token of every step;
outputs within 2e-2 * max|ref| per layer on the second step (by then the cache
holds hits and misses; the prefill layers run in waves of half their slots,
since every layer needs all 256 experts).  Output coverage: the 32-token decode,
all 32 tokens of layers 0, 7, 8 and 15 and tokens 0, 11, 22, 31 of the others;
the prefill chunk, every 8th token (256 tokens) of layer 0 and tokens 0, 681,
1362, 2047 of the others.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from routed_expert_streaming_amd import _lib as L
from routed_expert_streaming_amd.runtime import MoEStack
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


def decode32_rows(l):
    return None if l in (0, 7, 8, 15) else [0, 11, 22, 31]


def prefill_rows(l):
    return list(range(0, 2048, 8)) if l == 0 else [0, 681, 1362, 2047]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,steps,out_step,rows_of", [
    ("decode32_stream", 2, 1, decode32_rows),
    ("prefill2048_stream", 2, 1, prefill_rows),
])
def test_streamed_full_size_against_oracle(name, steps, out_step, rows_of):
    cfg = synth.get(name)
    k = cfg.top_k
    st = MoEStack(cfg)
    assert st.streaming and st.L == cfg.layers == 16
    layers = st.L
    try:
        wr = [st.wr[l].cpu().numpy() for l in range(layers)]
        bias = [None if st.bias is None else st.bias[l].cpu().numpy() for l in range(layers)]
        out = st.new_output()
        for s in range(steps):
            x = st.make_inputs(s)
            st.forward(x, out)
            torch.cuda.synchronize()
            xb, ob, idx = bits(x), bits(out), st.idx.cpu().numpy()
            print(f"{name} step {s} done on the GPU", flush=True)
            for l in range(layers):
                _, ridx, _ = oracle.router(xb[l], wr[l], bias[l], k)
                assert (ridx == idx[l]).all(), (name, s, l)
                if s != out_step:
                    continue
                rows = rows_of(l)
                ref = oracle.moe_layer(xb[l], wr[l], bias[l], k, st.host_pool_slabs(l), st.host_shared(l),
                                       cfg.inter, rows=rows)
                sel = slice(None) if rows is None else rows
                assert (ref["idx"][sel] == idx[l][sel]).all()
                ratio = check_close(ob[l][sel], ref["out64"][sel], f"{name} step {s} layer {l}")
                n = cfg.tokens if rows is None else len(rows)
                print(f"{name} step {s} layer {l}: {n} tokens, max err / max|ref| = {ratio:.2e}", flush=True)
        hits, misses, _ = st.stats()
        print(f"{name}: hit rate {hits / max(hits + misses, 1):.3f} over {steps} step(s)")
    finally:
        st.close()
