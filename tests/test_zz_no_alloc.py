"""The allocation-free one-call layer (moe_route_ffn_combine_noalloc) against the
entry point it varies (moe_route_ffn_combine with a caller workspace): the same
inputs give bit-identical expert indices, gate weights and outputs, on two calls
in a row, the second with a smaller input (the scratch then holds the first
call's leftovers), and both within 2e-2 * max|ref| of the oracle.  A workspace
beyond the fixed scratch is refused before anything runs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from routed_expert_streaming_amd import _lib as L

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class Case:
    def __init__(self, T, H, I, E, k, shared, seed):
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.x = synth.x_bf16(seed, 0, 0, T, H)
        self.Wr = synth.router_w(seed, 0, E, H)
        slab = synth.slab_bytes(H, I)
        self.slabs = [np.empty(slab, np.uint8) for _ in range(E)]
        synth.fill_slabs(seed, 0, list(range(E)), H, I, [s.ctypes.data for s in self.slabs])
        self.shared = synth.expert_slab(seed, 0, E, H, I) if shared else None
        self.pool = torch.from_numpy(np.stack(self.slabs)).cuda()
        self.table = torch.tensor([self.pool.data_ptr() + e * slab for e in range(E)], dtype=torch.int64,
                                  device="cuda")
        self.shared_dev = torch.from_numpy(self.shared).cuda() if shared else None
        self.xd = torch.from_numpy(self.x.view(np.int16)).view(torch.bfloat16).cuda()
        self.wr = torch.from_numpy(self.Wr).cuda()

    def run(self, noalloc):
        T, H, I, E, k = self.T, self.H, self.I, self.E, self.k
        idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
        w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
        out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        if noalloc:
            L.moe_route_ffn_combine_noalloc(self.xd, T, H, I, self.wr, None, E, k, self.table, self.shared_dev, idx, w,
                                            out)
        else:
            nb = L.moe_route_ffn_combine_workspace_bytes(T, H, I, E, k, self.shared is not None)
            ws = torch.full((nb,), 0x5A, dtype=torch.uint8, device="cuda")
            L.moe_route_ffn_combine(self.xd, T, H, I, self.wr, None, E, k, self.table, self.shared_dev, idx, w, out,
                                    ws, nb)
        torch.cuda.synchronize()
        return idx.cpu().numpy(), w.cpu().numpy(), bits(out)


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    assert L.moe_noalloc_scratch_bytes() == 16 << 20
    # first call: 32 tokens (split path: the MFMA and GEMV parts run in order on
    # the stream), then one token (router finished inside gate/up) with fewer
    # experts, which finds the first call's data in the scratch
    cases = [Case(32, 2048, 1024, 64, 8, True, 901), Case(1, 4096, 1536, 128, 8, True, 902),
             Case(5, 512, 256, 32, 4, False, 903)]
    got = [c.run(True) for c in cases]
    for c, (idx, w, out) in zip(cases, got):
        ridx, rw, rout = c.run(False)
        assert np.array_equal(idx, ridx)
        assert np.array_equal(w.view(np.uint32), rw.view(np.uint32))
        assert np.array_equal(out, rout)
        ref = oracle.moe_layer(c.x, c.Wr, None, c.k, c.slabs, c.shared, c.I)
        assert np.array_equal(idx, ref["idx"])
        val = (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        scale = float(np.max(np.abs(ref["out64"])))
        assert float(np.max(np.abs(val - ref["out64"]))) <= TOL * scale
    # a second round in the other order gives the same bits again
    for c, (idx, w, out) in zip(cases[::-1], got[::-1]):
        i2, w2, o2 = c.run(True)
        assert np.array_equal(i2, idx) and np.array_equal(o2, out)


def test_noalloc_refuses_workspace_beyond_the_scratch():
    T, H, I, E, k = 2048, 6144, 2048, 256, 8
    need = L.moe_route_ffn_combine_workspace_bytes(T, H, I, E, k, False)
    assert need > L.moe_noalloc_scratch_bytes()
    dummy = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.MoEError) as ei:
        # validation fails before any pointer is read
        L.moe_route_ffn_combine_noalloc(dummy, T, H, I, dummy, None, E, k, dummy, None, dummy, dummy, dummy)
    assert ei.value.status == L.MOE_E_NOMEM
    L.moe_route_ffn_combine_noalloc(None, 0, H, I, None, None, E, k, None, None, None, None, None)  # T = 0: no-op
