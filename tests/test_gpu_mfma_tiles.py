"""GPU parity of the prefill grouped-GEMM (MFMA) path on routings built so that
every token-count case of the kernel is checked element by element.

A workgroup of the MFMA kernels covers an expert's tokens in passes of up to 96
rows (six 16-row M tiles), with the K loop specialised on the pass's tile count.
The routings here are built by hand (the FFN entry points take the routing as an
input), so that experts get 1..96 tokens -- every tile count from 1 to 6, full
and ragged last tiles -- and more than 96 -- several passes, ragged last pass.
Every output row of every case is compared with the oracle's FFN + combine for
the same routing (LayerStoRm README, "TL;DR": the selected experts' FFNs run and
their outputs are combined); the shapes also cover every weight-group variant of
the kernels (reduction length a multiple of 256 or only of 128, one or two W2
tiles per workgroup).

Bars: max|err| <= 2e-2 * max|ref| per tensor; the MFMA rows of the split path
equal the MFMA path's bit for bit (same arithmetic, other workgroup mapping).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from routed_expert_streaming_amd import _lib as L
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


def crafted_routing(counts, k, seed):
    """idx [T,k]: expert e in exactly counts[e] token rows, at most once per row
    (T = sum(counts) / k >= max(counts)); tokens and slots in random order.
    w [T,k] fp32 positive weights summing to about 1 per token."""
    counts = np.asarray(counts)
    total = int(counts.sum())
    assert total % k == 0
    T = total // k
    assert counts.max() <= T
    flat = np.repeat(np.arange(len(counts), dtype=np.int32), counts)  # sorted by expert
    idx = flat.reshape(k, T).T.copy()  # slot (t, i) = flat[i*T + t]: a run of <= T repeats never shares a row
    rng = np.random.default_rng(seed)
    idx = idx[rng.permutation(T)]
    for t in range(T):
        rng.shuffle(idx[t])
    assert all(len(set(row)) == k for row in idx.tolist())
    assert np.array_equal(np.bincount(idx.ravel(), minlength=len(counts)), counts)
    w = rng.uniform(0.05, 1.0, (T, k))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(idx), w


CASES = [
    # name, H, I, k, shared, per-expert token counts
    # every tile count 1..6 (full and ragged last tiles), zero-token experts, a
    # 323-token shared expert (four passes); H = 256: record groups of 4 chunks,
    # two W2 tiles per down workgroup, I = 128: down code groups of 2
    ("tiles_1_to_6", 256, 128, 2, True, [2, 16, 17, 33, 48, 49, 64, 65, 80, 81, 95, 96, 0, 0, 0, 0]),
    # several passes per expert (97 .. 290 tokens: 2-4 passes, ragged last pass)
    # and a GEMV-sized one; H = 384: gate/up record groups of 2, one W2 tile
    # per down workgroup with code and record groups of 4 (I = 256)
    ("multi_pass", 384, 256, 2, False, [97, 112, 150, 192, 193, 200, 250, 288, 290, 2]),
    # I = 384 (a multiple of 128, not of 256): down workgroups of two W2 tiles
    # with groups of 2 chunks; k = 4 with a mix of small and large experts
    ("inter_384", 512, 384, 4, True, [5, 20, 40, 60, 70, 90, 100, 130, 7, 3, 1, 2]),
]


@pytest.mark.parametrize("name,H,I,k,shared,counts", CASES, ids=[c[0] for c in CASES])
def test_mfma_every_tile_count_against_oracle(name, H, I, k, shared, counts):
    seed = 300 + H + I + k
    E = len(counts)
    idx, w = crafted_routing(counts, k, seed)
    T = idx.shape[0]
    x = synth.x_bf16(seed, 0, 0, T, H)
    slab = synth.slab_bytes(H, I)
    slabs = [np.empty(slab, np.uint8) for _ in range(E)]
    synth.fill_slabs(seed, 0, list(range(E)), H, I, [s.ctypes.data for s in slabs])
    shared_np = synth.expert_slab(seed, 0, E, H, I) if shared else None
    ref = oracle.moe_ffn_routed(x, idx, w.astype(np.float64), slabs, shared_np, I)

    pool = torch.from_numpy(np.stack(slabs)).cuda()
    table = torch.tensor([pool.data_ptr() + e * slab for e in range(E)], dtype=torch.int64, device="cuda")
    shared_dev = torch.from_numpy(shared_np).cuda() if shared else None
    xd = bf16_dev(x)
    idx_d = torch.from_numpy(idx).cuda()
    w_d = torch.from_numpy(w).cuda()
    P = T * k + (T if shared else 0)
    fb = L.moe_expert_ffn_workspace_bytes(T, H, I, E, k, shared)
    ws = torch.empty(fb, dtype=torch.uint8, device="cuda")
    ys, outs = {}, {}
    for path in (L.MOE_FFN_MFMA, L.MOE_FFN_SPLIT):
        y = torch.full((P, H), float("nan"), dtype=torch.float32, device="cuda")
        L.moe_expert_ffn(xd, T, H, I, E, idx_d, k, table, shared_dev, None, y, ws, fb, path)
        out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        L.moe_combine(y, w_d, T, k, H, shared, out)
        fused = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        L.moe_expert_ffn_combine(xd, T, H, I, E, idx_d, w_d, k, table, shared_dev, fused, ws, fb, path)
        torch.cuda.synchronize()
        ys[path] = y.cpu().numpy()
        outs[path] = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(fused.view(torch.int16).cpu().numpy().view(np.uint16), outs[path])
        assert not np.isnan(ys[path]).any()
        ratio = check_close(outs[path], ref["out64"], f"{name} path {path}")
        print(f"{name} path {path}: every row, max err / max|ref| = {ratio:.2e}")
    # the split path runs the experts with more than 4 tokens on the same MFMA
    # arithmetic (compact workgroup mapping): those rows are bit-identical
    cnt = np.asarray(counts)
    big = (cnt[idx] > 4).ravel()
    assert np.array_equal(ys[L.MOE_FFN_SPLIT][:T * k][big], ys[L.MOE_FFN_MFMA][:T * k][big])
    if shared:
        assert np.array_equal(ys[L.MOE_FFN_SPLIT][T * k:], ys[L.MOE_FFN_MFMA][T * k:])
