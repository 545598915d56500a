"""GPU parity of the MXFP4 (format 1) and super-block (format 2) expert weight
formats on the multi-token paths -- the dequant-GEMV in pair and expert
grouping, the MFMA grouped GEMM and the split path -- against the oracle reading
the same slabs (LayerStoRm README, "License and attributions": MXFP4 decode
paths; "Serve": a 4-bit k-quant weight type).

Routings are built by hand (the FFN entry points take the routing as an input)
so that experts get 1..96 tokens -- every M-tile count of the MFMA kernel, full
and ragged -- and more than 96 (several passes); the shapes cover reduction
lengths whose last 4-group step is full or partial (for super-blocks: one or
two headers in the last step), and one or two W2 tiles per down workgroup.
Every output row of every case is compared with the oracle.  At full size, the
32-token decode and the 2048-token prefill shapes run streamed through the
cache (2 layers, waves of half the slots for the prefill) and are checked on
sampled rows.

Bars: max|err| <= 2e-2 * max|ref| per tensor; expert grouping bit-identical to
pair grouping (same GEMV arithmetic); the split path's MFMA rows equal the MFMA
path's and its GEMV rows the grouped path's, bit for bit; the one-call format
entry point equals the FFN call followed by the combine; expert indices of the
full-size runs bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from routed_expert_streaming_amd import _lib as L
from routed_expert_streaming_amd.runtime import MoEStack
from tests.test_gpu_mfma_tiles import crafted_routing
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


TILES = [2, 16, 17, 33, 48, 49, 64, 65, 80, 81, 95, 96, 0, 0, 1, 1]
PASSES = [97, 112, 150, 193, 200, 290, 2, 4]
MIXED = [5, 20, 40, 60, 70, 90, 100, 130, 7, 3, 1, 2]
CASES = [
    # name, format, H, I, k, shared, per-expert token counts
    # MXFP4: H 256 (one partial record step), I 128; H 384 (3 groups), I 256; H 512, I 384
    ("mx_tiles", 1, 256, 128, 2, True, TILES),
    ("mx_passes", 1, 384, 256, 2, False, PASSES),
    ("mx_k4", 1, 512, 384, 4, True, MIXED),
    # super-blocks: H 256 and I 256 (one header in the only step), H 512 (two
    # headers), H 768 (last step one header), I 512
    ("sb_tiles", 2, 256, 256, 2, True, TILES),
    ("sb_passes", 2, 512, 256, 2, False, PASSES),
    ("sb_k4", 2, 768, 512, 4, True, MIXED),
]


@pytest.mark.parametrize("name,fmt,H,I,k,shared,counts", CASES, ids=[c[0] for c in CASES])
def test_format_paths_against_oracle(name, fmt, H, I, k, shared, counts):
    seed = 700 + 10 * fmt + H + I + k
    E = len(counts)
    idx, w = crafted_routing(counts, k, seed)
    T = idx.shape[0]
    x = synth.x_bf16(seed, 0, 0, T, H)
    slab = synth.slab_bytes(H, I, fmt)
    slabs = [np.empty(slab, np.uint8) for _ in range(E)]
    synth.fill_slabs(seed, 0, list(range(E)), H, I, [s.ctypes.data for s in slabs], fmt=fmt)
    shared_np = synth.expert_slab(seed, 0, E, H, I, fmt) if shared else None
    ref = oracle.moe_ffn_routed(x, idx, w.astype(np.float64), slabs, shared_np, I, fmt=fmt)
    print(f"{name}: T={T} E={E} slab={slab} B", flush=True)

    pool = torch.from_numpy(np.stack(slabs)).cuda()
    table = torch.tensor([pool.data_ptr() + e * slab for e in range(E)], dtype=torch.int64, device="cuda")
    shared_dev = torch.from_numpy(shared_np).cuda() if shared else None
    xd = bf16_dev(x)
    idx_d = torch.from_numpy(idx).cuda()
    w_d = torch.from_numpy(w).cuda()
    P = T * k + (T if shared else 0)
    fb = L.moe_expert_ffn_workspace_bytes(T, H, I, E, k, shared)
    ws = torch.empty(fb, dtype=torch.uint8, device="cuda")
    ys = {}
    for path in (L.MOE_FFN_PAIRS, L.MOE_FFN_GROUPED, L.MOE_FFN_MFMA, L.MOE_FFN_SPLIT):
        y = torch.full((P, H), float("nan"), dtype=torch.float32, device="cuda")
        L.moe_expert_ffn_fmt(xd, T, H, I, E, idx_d, k, table, shared_dev, None, y, ws, fb, path, fmt)
        out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        L.moe_combine(y, w_d, T, k, H, shared, out)
        torch.cuda.synchronize()
        ys[path] = y.cpu().numpy()
        assert not np.isnan(ys[path]).any(), (name, path)
        ratio = check_close(bits(out), ref["out64"], f"{name} path {path}")
        print(f"{name} path {path}: every row, max err / max|ref| = {ratio:.2e}", flush=True)
    # the one-call entry point (automatic path) equals its FFN call + combine
    fused = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    call = L.moe_mx_expert_ffn_combine if fmt == 1 else L.moe_sb_expert_ffn_combine
    call(xd, T, H, I, E, idx_d, w_d, k, table, shared_dev, fused, ws, fb)
    y = torch.empty((P, H), dtype=torch.float32, device="cuda")
    L.moe_expert_ffn_fmt(xd, T, H, I, E, idx_d, k, table, shared_dev, None, y, ws, fb, L.MOE_FFN_AUTO, fmt)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    L.moe_combine(y, w_d, T, k, H, shared, out)
    torch.cuda.synchronize()
    assert np.array_equal(bits(fused), bits(out))
    # GEMV: expert grouping computes each pair as pair grouping does
    assert np.array_equal(ys[L.MOE_FFN_GROUPED], ys[L.MOE_FFN_PAIRS])
    # the MFMA kernels with dequantised bf16 weights (the two-call form, which
    # has no workspace for MXFP4's activation digit pairs): what the split path's
    # MFMA part runs
    cnt_d = torch.empty(E, dtype=torch.int32, device="cuda")
    off_d = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    por_d = torch.empty(T * k, dtype=torch.int32, device="cuda")
    L.moe_permute(idx_d, T, k, E, cnt_d, off_d, por_d)
    h = torch.empty((P, I), dtype=torch.bfloat16, device="cuda")
    y2 = torch.full((P, H), float("nan"), dtype=torch.float32, device="cuda")
    L.moe_expert_gate_up_fmt(xd, T, H, I, E, idx_d, k, cnt_d, off_d, por_d, table, shared_dev, None, h,
                             L.MOE_FFN_MFMA, fmt)
    L.moe_expert_down_fmt(h, T, H, I, E, idx_d, k, cnt_d, off_d, por_d, table, shared_dev, None, y2,
                          L.MOE_FFN_MFMA, fmt)
    out2 = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    L.moe_combine(y2, w_d, T, k, H, shared, out2)
    torch.cuda.synchronize()
    y_dq = y2.cpu().numpy()
    ratio = check_close(bits(out2), ref["out64"], f"{name} MFMA, two calls")
    print(f"{name} MFMA two calls (bf16 weights): every row, max err / max|ref| = {ratio:.2e}", flush=True)
    if fmt != 1:  # MXFP4's one-call MFMA path runs the block-scaled kernels instead
        assert np.array_equal(y_dq, ys[L.MOE_FFN_MFMA])
    # split: experts with more than 4 tokens on the MFMA arithmetic, the others on the GEMV's
    cnt = np.asarray(counts)
    big = (cnt[idx] > 4).ravel()
    assert np.array_equal(ys[L.MOE_FFN_SPLIT][:T * k][big], y_dq[:T * k][big])
    assert np.array_equal(ys[L.MOE_FFN_SPLIT][:T * k][~big], ys[L.MOE_FFN_GROUPED][:T * k][~big])
    if shared:  # the shared expert has T > 4 tokens
        assert np.array_equal(ys[L.MOE_FFN_SPLIT][T * k:], y_dq[T * k:])


@pytest.mark.parametrize("fmt", [1, 2])
def test_format_gate_up_and_down_calls_equal_the_ffn_call(fmt):
    """The two-call form (permutation, gate/up, down) with an expert mask writes
    the masked pairs as the one-call FFN does and leaves the others untouched."""
    H, I, k, E, shared = 512, 256, 2, 8, True
    counts = [40, 3, 0, 25, 60, 1, 9, 22]
    seed = 900 + fmt
    idx, _ = crafted_routing(counts, k, seed)
    T = idx.shape[0]
    x = synth.x_bf16(seed, 0, 0, T, H)
    slab = synth.slab_bytes(H, I, fmt)
    pool_np = np.empty((E, slab), np.uint8)
    synth.fill_slabs(seed, 0, list(range(E)), H, I, [pool_np[e].ctypes.data for e in range(E)], fmt=fmt)
    pool = torch.from_numpy(pool_np).cuda()
    table = torch.tensor([pool.data_ptr() + e * slab for e in range(E)], dtype=torch.int64, device="cuda")
    shared_dev = torch.from_numpy(synth.expert_slab(seed, 0, E, H, I, fmt)).cuda()
    xd, idx_d = bf16_dev(x), torch.from_numpy(idx).cuda()
    P = T * k + T
    mask = torch.tensor([1, 0, 1, 1, 0, 1, 0, 1], dtype=torch.uint8, device="cuda")
    fb = L.moe_expert_ffn_workspace_bytes(T, H, I, E, k, True)
    ws = torch.empty(fb, dtype=torch.uint8, device="cuda")
    for path in (L.MOE_FFN_GROUPED, L.MOE_FFN_MFMA, L.MOE_FFN_SPLIT):
        y1 = torch.full((P, H), 7.0, dtype=torch.float32, device="cuda")
        L.moe_expert_ffn_fmt(xd, T, H, I, E, idx_d, k, table, shared_dev, mask, y1, ws, fb, path, fmt)
        cnt = torch.empty(E, dtype=torch.int32, device="cuda")
        off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        por = torch.empty(T * k, dtype=torch.int32, device="cuda")
        L.moe_permute(idx_d, T, k, E, cnt, off, por)
        h = torch.empty((P, I), dtype=torch.bfloat16, device="cuda")
        y2 = torch.full((P, H), 7.0, dtype=torch.float32, device="cuda")
        L.moe_expert_gate_up_fmt(xd, T, H, I, E, idx_d, k, cnt, off, por, table, shared_dev, mask, h, path, fmt)
        L.moe_expert_down_fmt(h, T, H, I, E, idx_d, k, cnt, off, por, table, shared_dev, mask, y2, path, fmt)
        torch.cuda.synchronize()
        a, b = y1.cpu().numpy(), y2.cpu().numpy()
        admitted = np.concatenate([mask.cpu().numpy()[idx].ravel().astype(bool), np.ones(T, bool)])
        assert (a[~admitted] == 7.0).all() and not (a[admitted] == 7.0).all(axis=1).any()
        if fmt == 1 and path == L.MOE_FFN_MFMA:
            # one call: the block-scaled kernels; two calls: bf16-dequantised weights
            assert (b[~admitted] == 7.0).all()
            err = np.abs(a[admitted] - b[admitted]).max() / np.abs(b[admitted]).max()
            assert err <= 2e-2, (fmt, path, err)
        else:
            assert np.array_equal(a, b), (fmt, path)


def decode32_rows(l):
    return None if l == 0 else [0, 11, 22, 31]


def prefill_rows(l):
    return list(range(0, 2048, 16)) if l == 0 else [0, 681, 1362, 2047]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,rows_of", [
    ("decode32_mx_stream", decode32_rows),
    ("decode32_sb_stream", decode32_rows),
    ("prefill2048_mx_stream", prefill_rows),
    ("prefill2048_sb_stream", prefill_rows),
])
def test_format_streamed_full_size_against_oracle(name, rows_of):
    """Two layers of the full-size configuration, streamed through the cache:
    the second step (hits and misses) against the oracle on sampled rows."""
    cfg = synth.get(name)
    k = cfg.top_k
    st = MoEStack(cfg, layers=2)
    assert st.streaming and st.fmt == cfg.fmt
    try:
        wr = [st.wr[l].cpu().numpy() for l in range(st.L)]
        bias = [None if st.bias is None else st.bias[l].cpu().numpy() for l in range(st.L)]
        out = st.new_output()
        for s in range(2):
            x = st.make_inputs(s)
            st.forward(x, out)
            torch.cuda.synchronize()
            print(f"{name} step {s} done on the GPU", flush=True)
        xb, ob, idx = bits(x), bits(out), st.idx.cpu().numpy()
        for l in range(st.L):
            rows = rows_of(l)
            ref = oracle.moe_layer(xb[l], wr[l], bias[l], k, st.host_pool_slabs(l), st.host_shared(l), cfg.inter,
                                   rows=rows, fmt=cfg.fmt)
            assert (ref["idx"] == idx[l]).all(), (name, l)
            sel = slice(None) if rows is None else rows
            ratio = check_close(ob[l][sel], ref["out64"][sel], f"{name} layer {l}")
            print(f"{name} layer {l}: max err / max|ref| = {ratio:.2e}", flush=True)
    finally:
        st.close()


def e4m3_values():
    """OCP E4M3 value of every byte (NaN at 0x7F / 0xFF)."""
    b = np.arange(256)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e, m = (b >> 3) & 15, b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def test_quant_act_digit_pairs():
    """moe_quant_act_mx: the row scale rule, the operand byte order, hi the
    truncation of x / 2^u to E4M3, and hi + lo == x / 2^u for every element
    within 2^10 of the row's largest (off by at most 2^-10 otherwise); in place
    equals out of place."""
    rng = np.random.default_rng(77)
    rows, K = 9, 384
    xf = rng.standard_normal((rows, K))
    xf[1] = 0.0                                                      # all zero
    xf[2] = rng.choice([-1, 1], K) * 2.0 ** rng.uniform(-24, 12, K)  # wide dynamic range
    xf[3] = 1e-3 * rng.standard_normal(K)
    xf[3, 17] = 3e4                                                  # one large element, the rest tiny
    xf[4, ::3] = -0.0
    xf[5] = 1e-30 * rng.standard_normal(K)                           # near the bottom of bf16's range
    u32 = xf.astype(np.float32).view(np.uint32)  # to bf16, nearest even (all finite)
    x = ((u32 + 0x7FFF + ((u32 >> 16) & 1)) >> 16).astype(np.uint16)
    xd = bf16_dev(x)
    out = torch.empty((rows, 2 * K), dtype=torch.uint8, device="cuda")
    sc = torch.empty(rows, dtype=torch.int32, device="cuda")
    L.moe_quant_act_mx(xd, rows, K, out, sc)
    inplace = xd.clone()
    sc2 = torch.empty(rows, dtype=torch.int32, device="cuda")
    L.moe_quant_act_mx(inplace, rows, K, inplace, sc2)
    torch.cuda.synchronize()
    q = out.cpu().numpy()
    assert np.array_equal(inplace.view(torch.uint8).cpu().numpy().reshape(rows, 2 * K), q)
    assert np.array_equal(sc2.cpu().numpy(), sc.cpu().numpy())
    u = sc.cpu().numpy().astype(np.int64) - 127
    vals = e4m3_values()
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # column of each output byte: group g, chunk c, byte j
    g, c, j = np.meshgrid(np.arange(K // 128), np.arange(4), np.arange(32), indexing="ij")
    col = (128 * g + np.where(j < 16, 16 * c + j, 64 + 16 * c + j - 16)).ravel()
    hi_pos = (256 * g + 32 * c + j).ravel()
    lo_pos = hi_pos + 128
    assert np.array_equal(np.sort(col), np.arange(K))
    for r in range(rows):
        mx = np.abs(xv[r]).max()
        if mx > 0:
            assert 128.0 <= mx / 2.0 ** u[r] < 256.0, (r, mx, u[r])
        y = xv[r, col] / 2.0 ** u[r]
        hi, lo = vals[q[r, hi_pos]], vals[q[r, lo_pos]]
        assert not np.isnan(hi).any() and not np.isnan(lo).any()
        # hi: y truncated to E4M3 (never larger in magnitude; less than one E4M3 step away)
        assert (np.abs(hi) <= np.abs(y)).all() and (hi * y >= 0).all()
        step = np.where(np.abs(hi) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(hi), 1e-300))) - 3), 2.0 ** -9)
        assert (np.abs(y - hi) < step).all(), r
        big = np.abs(xv[r, col]) >= 2.0 ** (u[r] - 2)
        assert np.array_equal(hi[big] + lo[big], y[big]), r
        assert (np.abs(hi + lo - y) <= 2.0 ** -10).all(), r
