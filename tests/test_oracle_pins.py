"""Pins for the CPU oracle: each checks it against something other than itself
(closed forms, brute force, exact rational arithmetic, a library routine, hand-built
data), chosen so that a dropped term, a wrong sign or index, a swapped gate/up or a
transposed operand fails at least one of them."""
from fractions import Fraction
import itertools
import math

import numpy as np
import pytest
import scipy.special

import oracle
import synth
from tests import slabkit as sk

rng = np.random.default_rng(12345)


# ------------------------------------------------------------------ scalar formats
def test_fp_decoders_closed_forms():
    assert oracle.bf16_to_double(0x3F80) == 1.0
    assert oracle.bf16_to_double(0xC040) == -3.0
    assert oracle.bf16_to_double(0x0001) == 2.0 ** -133
    assert math.isinf(oracle.bf16_to_double(0x7F80))
    assert oracle.fp16_to_double(0x3C00) == 1.0
    assert oracle.fp16_to_double(0x0001) == 2.0 ** -24
    assert oracle.fp16_to_double(0x7BFF) == 65504.0
    assert oracle.fp16_to_double(0x8400) == -(2.0 ** -14)
    assert oracle.fp16_to_double(0xC800) == -8.0


def _bf16_value(bits):
    return oracle.bf16_to_double(bits)


def _nearest_bf16_bruteforce(v: float) -> int:
    """Nearest bf16 by exact comparison among the neighbours of the truncation."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    f32 = np.float32(v)  # any nearby float32; the candidates below bracket v
    base = int(np.array(f32).view(np.uint32)) >> 16
    cands = [c & 0xFFFF for c in range(base - 2, base + 3) if 0 <= (c & 0x7FFF) < 0x7F80]
    target = Fraction(v)
    best = None
    for c in cands:
        cv = Fraction(_bf16_value(c))
        d = abs(cv - target)
        key = (d, c & 1)  # ties go to the even significand
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_bf16_rounding_ties_and_bruteforce():
    assert oracle.double_to_bf16(1.0) == 0x3F80
    assert oracle.double_to_bf16(1.0 + 2 ** -8) == 0x3F80          # tie -> even
    assert oracle.double_to_bf16(1.0 + 3 * 2 ** -8) == 0x3F82      # tie -> even (up)
    assert oracle.double_to_bf16(1.0 + 2 ** -8 + 2 ** -30) == 0x3F81
    assert oracle.double_to_bf16(-0.0) == 0x8000
    assert oracle.double_to_bf16(1e39) == 0x7F80
    assert oracle.double_to_bf16(2.0 ** -133) == 0x0001
    assert oracle.double_to_bf16(1.5 * 2.0 ** -133) == 0x0002      # subnormal tie -> even
    vals = rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000))
    for v in vals:
        assert oracle.double_to_bf16(float(v)) == _nearest_bf16_bruteforce(float(v)), v


# ------------------------------------------------------------------ router
def _round_to_f32_exact(q: Fraction) -> np.float32:
    """Nearest fp32 to an exact rational, ties to even, by exact comparison."""
    f = np.float32(float(q))
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    best = None
    for c in cands:
        key = (abs(Fraction(float(c)) - q), int(np.array(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def _bf16_array(T, H):
    return synth.x_bf16(777, 0, 0, T, H)


def test_router_logits_are_exact_sum_rounded_once():
    T, H, E = 3, 96, 12
    x = _bf16_array(T, H)
    Wr = rng.standard_normal((E, H)).astype(np.float32) * np.float32(0.02)
    b = rng.standard_normal(E).astype(np.float32)
    logits, _, _ = oracle.router(x, Wr, b, 2)
    for t in range(T):
        xs = [Fraction(oracle.bf16_to_double(int(v))) for v in x[t]]
        for e in range(E):
            exact = sum(xs[h] * Fraction(float(Wr[e, h])) for h in range(H)) + Fraction(float(b[e]))
            assert logits[t, e] == _round_to_f32_exact(exact)


def _rank_bruteforce_topk(lg, k):
    """Selection by rank counting: rank(e) = #{strictly larger} + #{equal with lower index}."""
    E = len(lg)
    rank = [sum(1 for f in range(E) if lg[f] > lg[e]) + sum(1 for f in range(e) if lg[f] == lg[e])
            for e in range(E)]
    return [rank.index(i) for i in range(k)]


@pytest.mark.parametrize("k", [1, 2, 8, 16])
def test_topk_matches_rank_bruteforce_with_ties(k):
    T, H, E = 6, 64, 16
    x = _bf16_array(T, H)
    Wr = rng.standard_normal((E, H)).astype(np.float32) * np.float32(0.02)
    # exact ties: duplicated router rows (experts 3==9, 5==6==12)
    Wr[9] = Wr[3]
    Wr[6] = Wr[5]
    Wr[12] = Wr[5]
    logits, idx, w = oracle.router(x, Wr, None, k)
    for t in range(T):
        assert list(idx[t]) == _rank_bruteforce_topk(list(logits[t]), k)


def test_topk_all_zero_router_gives_first_k_and_uniform_weights():
    T, H, E = 4, 64, 16
    x = _bf16_array(T, H)
    for k in (1, 3, 8):
        _, idx, w = oracle.router(x, np.zeros((E, H), np.float32), None, k)
        assert (idx == np.arange(k)).all()
        assert (w == 1.0 / k).all()


def test_weights_special_cases():
    T, H, E = 5, 64, 8
    x = _bf16_array(T, H)
    Wr = rng.standard_normal((E, H)).astype(np.float32) * np.float32(0.05)
    b = rng.standard_normal(E).astype(np.float32)
    _, _, w1 = oracle.router(x, Wr, b, 1)
    assert (w1 == 1.0).all()
    logits, idx, wE = oracle.router(x, Wr, b, E)
    for t in range(T):
        ref = scipy.special.softmax(logits[t].astype(np.float64))
        np.testing.assert_allclose(wE[t], ref[idx[t]], rtol=0, atol=1e-15)
    _, _, w8 = oracle.router(x, Wr, b, 4)
    assert np.all(np.abs(w8.sum(axis=1) - 1.0) <= 4 * 2.0 ** -52)
    assert np.all(np.diff(w8, axis=1) <= 0)  # descending logits -> non-increasing weights


def test_bias_enters_logits_and_selection():
    T, H, E = 2, 64, 8
    x = _bf16_array(T, H)
    bias = np.zeros(E, np.float32)
    bias[5] = 3.0
    bias[2] = 2.0
    logits, idx, w = oracle.router(x, np.zeros((E, H), np.float32), bias, 2)
    assert (idx == [5, 2]).all()
    np.testing.assert_allclose(w[0], [1 / (1 + math.exp(-1.0)), 1 / (1 + math.exp(1.0))], rtol=1e-15)
    assert logits[0, 5] == 3.0 and logits[0, 0] == 0.0


# ------------------------------------------------------------------ dequant and layout
def _handbuilt(H=64, I=32):
    r_I = np.arange(I)[:, None]
    c_H = np.arange(H)[None, :]
    q1 = (r_I + 3 * c_H) % 16
    q3 = (5 * r_I + c_H + 7) % 16
    r_H = np.arange(H)[:, None]
    c_I = np.arange(I)[None, :]
    q2 = (2 * r_H + 5 * c_I + 1) % 16
    s1 = sk.f16(2.0 ** -(np.arange(I * H // 32).reshape(I, H // 32) % 5))
    m1 = sk.f16(-8.0 * s1.view(np.float16).astype(np.float64))
    s3 = sk.f16(np.full((I, H // 32), 0.5))
    m3 = sk.f16(np.full((I, H // 32), 0.25))          # general affine block (min != -8*scale)
    s2 = sk.f16(np.full((H, I // 32), 0.125))
    s2[3, 0] = 0x0001                                  # fp16 subnormal scale
    m2 = sk.f16(-8.0 * s2.view(np.float16).astype(np.float64))
    q2[7, :] = 8                                       # all-8 row with min=-8*scale -> zeros
    mats = ((q1, s1, m1), (q3, s3, m3), (q2, s2, m2))
    return sk.build_slab(H, I, *mats), mats


def test_dequant_round_trip_handbuilt():
    H, I = 64, 32
    slab, mats = _handbuilt(H, I)
    assert slab.size == oracle.slab_bytes(H, I)
    for which in range(3):
        got = oracle.dequant(slab, H, I, which)
        exp = sk.dequant_expected(*mats[which])
        assert np.array_equal(got, exp)
    assert np.all(oracle.dequant(slab, H, I, 2)[7] == 0.0)
    assert oracle.dequant(slab, H, I, 2)[3, 0] == 2.0 ** -24 * mats[2][0][3, 0] - 8 * 2.0 ** -24


def test_dequant_unit_scale_codes_give_q_minus_8():
    H, I = 32, 32
    q = np.tile(np.arange(16), (I, H // 16))
    mat = (q, sk.f16(1.0), sk.f16(-8.0))
    slab = sk.build_slab(H, I, mat, mat, (q.T.copy() if H == I else q, sk.f16(1.0), sk.f16(-8.0)))
    got = oracle.dequant(slab, H, I, 0)
    assert np.array_equal(got, q - 8.0)


def test_one_hot_inputs_recover_columns():
    H, I = 64, 32
    slab, mats = _handbuilt(H, I)
    W1 = sk.dequant_expected(*mats[0])
    W3 = sk.dequant_expected(*mats[1])
    W2 = sk.dequant_expected(*mats[2])
    for j in (0, 1, 30, 31, 32, 33, 63):
        x = np.zeros(H)
        x[j] = 1.0
        g, u, h, y = oracle.expert_ffn(slab, H, I, x)
        assert np.array_equal(g, W1[:, j])
        assert np.array_equal(u, W3[:, j])
    for c in (0, 1, 17, 31):
        hv = np.zeros(I)
        hv[c] = 1.0
        assert np.array_equal(oracle.expert_down(slab, H, I, hv), W2[:, c])


# ------------------------------------------------------------------ SwiGLU and FFN
def _swiglu_probe_slab(gate_code, up_code, H=32, I=32):
    """W1[0,0] = gate_code-8, W3[0,0] = up_code-8 (unit scale), all else 0; W2[:,0] = 1."""
    q1 = np.full((I, H), 8); q1[0, 0] = gate_code
    q3 = np.full((I, H), 8); q3[0, 0] = up_code
    q2 = np.full((H, I), 8); q2[:, 0] = 9
    one, m8 = sk.f16(1.0), sk.f16(-8.0)
    return sk.build_slab(H, I, (q1, one, m8), (q3, one, m8), (q2, one, m8))


def test_swiglu_closed_forms():
    H = I = 32
    x = np.zeros(H)
    x[0] = 1.0
    # g = 2, u = 3 -> h0 = 2*sigmoid(2)*3; swapping gate and up would give 3*sigmoid(3)*2
    g, u, h, y = oracle.expert_ffn(_swiglu_probe_slab(10, 11), H, I, x)
    expect = 2.0 / (1.0 + math.exp(-2.0)) * 3.0
    assert g[0] == 2.0 and u[0] == 3.0
    assert h[0] == pytest.approx(expect, rel=1e-15)
    assert np.all(h[1:] == 0.0)
    np.testing.assert_allclose(y, expect, rtol=1e-15)
    # silu(0) = 0 kills the up projection
    _, _, h0, y0 = oracle.expert_ffn(_swiglu_probe_slab(8, 15), H, I, x)
    assert np.all(h0 == 0.0) and np.all(y0 == 0.0)
    # negative gate: g = -8 -> silu(-8) = -8/(1+e^8)
    _, _, hn, _ = oracle.expert_ffn(_swiglu_probe_slab(0, 9), H, I, x)
    assert hn[0] == pytest.approx(-8.0 / (1.0 + math.exp(8.0)) * 1.0, rel=1e-15)


@pytest.mark.parametrize("H,I", [(64, 32), (256, 128), (96, 160)])
def test_constant_expert_closed_form(H, I):
    s1, s2 = 2.0 ** -6, 2.0 ** -5
    slab = sk.build_slab(H, I, sk.constant_matrix(I, H, 9, s1), sk.constant_matrix(I, H, 9, s1),
                         sk.constant_matrix(H, I, 10, s2))
    xb = synth.x_bf16(99, 0, 0, 1, H)[0]
    x = np.array([oracle.bf16_to_double(int(v)) for v in xb])
    S = math.fsum(x)
    g = s1 * S
    h = g / (1.0 + math.exp(-g)) * g
    _, _, hv, y = oracle.expert_ffn(slab, H, I, x)
    np.testing.assert_allclose(hv, h, rtol=1e-12)
    np.testing.assert_allclose(y, 2 * s2 * I * h, rtol=1e-12)


# ------------------------------------------------------------------ combine
def _const_expert(H, I, s1, code2, s2):
    return sk.build_slab(H, I, sk.constant_matrix(I, H, 9, s1), sk.constant_matrix(I, H, 9, s1),
                         sk.constant_matrix(H, I, code2, s2))


def _const_expert_output(x, I, s1, code2, s2):
    g = s1 * math.fsum(x)
    return (code2 - 8) * s2 * I * (g / (1.0 + math.exp(-g)) * g)


def test_combine_closed_form_two_experts_and_shared():
    H, I, E, k, T = 64, 32, 4, 2, 3
    xb = synth.x_bf16(5, 0, 0, T, H)
    # router reads column 0 only: logits = [0.5, 0, -1, 0.25] * x[t,0]
    Wr = np.zeros((E, H), np.float32)
    Wr[:, 0] = [0.5, 0.0, -1.0, 0.25]
    params = [(2.0 ** -6, 10, 2.0 ** -5), (2.0 ** -5, 12, 2.0 ** -6), (2.0 ** -7, 6, 2.0 ** -4),
              (2.0 ** -6, 13, 2.0 ** -5)]
    slabs = [_const_expert(H, I, *p) for p in params]
    shared_p = (2.0 ** -8, 7, 2.0 ** -3)
    shared = _const_expert(H, I, *shared_p)
    res = oracle.moe_layer(xb, Wr, None, k, slabs, shared, I)
    for t in range(T):
        x = np.array([oracle.bf16_to_double(int(v)) for v in xb[t]])
        lg = np.array([0.5, 0.0, -1.0, 0.25]) * x[0]
        lg32 = lg.astype(np.float32).astype(np.float64)
        order = _rank_bruteforce_topk(list(lg32), k)
        assert list(res["idx"][t]) == order
        ww = np.exp(lg32[order] - lg32[order[0]])
        ww /= ww.sum()
        expect = sum(ww[i] * _const_expert_output(x, I, *params[order[i]]) for i in range(k))
        expect += _const_expert_output(x, I, *shared_p)
        np.testing.assert_allclose(res["out64"][t], expect, rtol=1e-12)


def test_ffn_with_given_routing_closed_form():
    """Steps 4-5 with routing taken as given (arbitrary slot order, weights that
    do not sum to 1, an expert used by many tokens): out = sum_i w_i y(idx_i) +
    shared, from the constant-expert closed form; rows restricts the output."""
    H, I, E, k, T = 64, 32, 5, 3, 7
    xb = synth.x_bf16(8, 0, 0, T, H)
    params = [(2.0 ** -6, 9 + e, 2.0 ** -5) for e in range(E)]
    slabs = [_const_expert(H, I, *p) for p in params]
    shared_p = (2.0 ** -7, 5, 2.0 ** -4)
    idx = np.array([[4, 0, 2], [1, 4, 3], [0, 1, 2], [3, 2, 4], [4, 3, 0], [2, 0, 1], [1, 3, 4]], np.int32)
    w = rng.uniform(-0.5, 1.5, (T, k))
    res = oracle.moe_ffn_routed(xb, idx, w, slabs, _const_expert(H, I, *shared_p), I)
    for t in range(T):
        x = np.array([oracle.bf16_to_double(int(v)) for v in xb[t]])
        expect = sum(w[t, i] * _const_expert_output(x, I, *params[idx[t, i]]) for i in range(k))
        expect += _const_expert_output(x, I, *shared_p)
        np.testing.assert_allclose(res["out64"][t], expect, rtol=1e-12)
    sub = oracle.moe_ffn_routed(xb, idx, w, slabs, None, I, rows=[5, 1])
    for t in range(T):
        if t in (1, 5):
            x = np.array([oracle.bf16_to_double(int(v)) for v in xb[t]])
            expect = sum(w[t, i] * _const_expert_output(x, I, *params[idx[t, i]]) for i in range(k))
            np.testing.assert_allclose(sub["out64"][t], expect, rtol=1e-12)
        else:
            assert np.all(sub["out64"][t] == 0.0)


def test_zero_routed_experts_leave_shared_and_k1_gives_expert():
    H, I, E, T = 64, 32, 4, 2
    xb = synth.x_bf16(6, 0, 0, T, H)
    Wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    zero = sk.build_slab(H, I, sk.constant_matrix(I, H, 8, 1.0), sk.constant_matrix(I, H, 8, 1.0),
                         sk.constant_matrix(H, I, 8, 1.0))
    sp = (2.0 ** -7, 11, 2.0 ** -4)
    res = oracle.moe_layer(xb, Wr, None, 2, [zero] * E, _const_expert(H, I, *sp), I)
    for t in range(T):
        x = np.array([oracle.bf16_to_double(int(v)) for v in xb[t]])
        np.testing.assert_allclose(res["out64"][t], _const_expert_output(x, I, *sp), rtol=1e-12)
    params = [(2.0 ** -6, 9 + e, 2.0 ** -5) for e in range(E)]
    res1 = oracle.moe_layer(xb, Wr, None, 1, [_const_expert(H, I, *p) for p in params], None, I)
    for t in range(T):
        x = np.array([oracle.bf16_to_double(int(v)) for v in xb[t]])
        e = int(res1["idx"][t, 0])
        np.testing.assert_allclose(res1["out64"][t], _const_expert_output(x, I, *params[e]), rtol=1e-12)


def test_relabelling_experts_changes_nothing_and_bf16_output_is_rounded_out64():
    cfg = synth.get("tiny")
    H, I, E, k, T = cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, cfg.tokens
    xb = synth.x_bf16(cfg.seed, 0, 0, T, H)
    Wr = synth.router_w(cfg.seed, 0, E, H)
    bias = rng.standard_normal(E).astype(np.float32) * np.float32(0.1)
    slabs = [synth.expert_slab(cfg.seed, 0, e, H, I) for e in range(E)]
    base = oracle.moe_layer(xb, Wr, bias, k, slabs, None, I)
    perm = rng.permutation(E)          # new label j holds old expert perm[j]
    inv = np.argsort(perm)
    res = oracle.moe_layer(xb, Wr[perm].copy(), bias[perm].copy(), k, [slabs[p] for p in perm], None, I)
    assert (perm[res["idx"]] == base["idx"]).all()
    assert np.array_equal(res["out64"], base["out64"])
    assert (inv[base["idx"]] == res["idx"]).all()
    flat = base["out64"].ravel()
    assert all(oracle.double_to_bf16(float(v)) == int(b) for v, b in zip(flat, base["out_bf16"].ravel()))
    sub = oracle.moe_layer(xb, Wr, bias, k, slabs, None, I, rows=[2, 0])
    assert np.array_equal(sub["out64"][[0, 2]], base["out64"][[0, 2]])
    assert np.all(sub["out64"][[1, 3]] == 0.0)


def test_generator_params_are_scale_and_minus_eight_scale():
    cfg = synth.get("tiny")
    H, I = cfg.hidden, cfg.inter
    slab = synth.expert_slab(cfg.seed, 0, 3, H, I)
    for which in range(3):
        rec = sk.records_of(slab, H, I, which).reshape(-1, 2)
        sc = rec[:, 0].view(np.float16).astype(np.float64)
        mn = rec[:, 1].view(np.float16).astype(np.float64)
        assert np.all(np.isfinite(sc)) and np.all(sc >= 0) and np.array_equal(mn, -8 * sc)
        assert 0.012 < np.sqrt(np.mean(sc ** 2)) < 0.028


# ---------------------------------------------------------------- residual stream of chained layers
def test_residual_norm_closed_forms():
    H = 64
    bf = lambda v: oracle.double_to_bf16(v)
    # a constant row c normalises to sign(c) (eps small against c^2); rows of
    # different magnitudes in one call, so each row must use its own mean square
    cs = (3.0, -0.25, 1024.0, -7.5)
    r = np.array([np.full(H, c) for c in cs], np.float32)
    x = oracle.residual_norm(None, r, 1e-6)
    for t, c in enumerate(cs):
        assert (x[t] == bf(math.copysign(1.0, c))).all(), c
    # sqrt(H) * e_j has mean square 1, so it comes back unchanged (one row per j)
    r = np.zeros((3, H), np.float32)
    for t, j in enumerate((0, 17, 63)):
        r[t, j] = 8.0 * (-1) ** t
    x = oracle.residual_norm(None, r, 0.0)
    for t, j in enumerate((0, 17, 63)):
        want = np.zeros(H, np.uint16)
        want[j] = bf(8.0 * (-1) ** t)
        assert (x[t] == want).all()
    # eps inside the square root: a constant row with c^2 = eps gives 1/sqrt(2)
    r = np.full((1, H), 1e-3, np.float32)
    eps = float(np.float32(1e-3)) ** 2
    x = oracle.residual_norm(None, r, eps)
    assert (x == bf(1.0 / math.sqrt(2.0))).all()
    # the input row is left as it is when nothing is added
    assert (r == np.float32(1e-3)).all()


def test_residual_norm_scale_invariance_and_fp32_update():
    rng = np.random.default_rng(7)
    T, H = 4, 96
    r = rng.standard_normal((T, H)).astype(np.float32)
    base = oracle.residual_norm(None, r.copy(), 0.0)
    for m in (-6, 3, 20):  # power-of-two scalings are exact in fp32
        assert (oracle.residual_norm(None, r * np.float32(2.0 ** m), 0.0) == base).all(), m
    # the update is the fp32 sum of the residual and the bf16 output
    add = np.array([[oracle.double_to_bf16(float(v)) for v in row] for row in rng.standard_normal((T, H)) * 30.0],
                   np.uint16)
    upd = r.copy()
    oracle.residual_norm(add, upd, 1e-6)
    add_f = np.array([[oracle.bf16_to_double(int(b)) for b in row] for row in add], np.float32)
    assert (upd == r + add_f).all()


# ---------------------------------------------------------------- weight format 1 (MXFP4)
# OCP Microscaling Formats v1.0: FP4 E2M1 element values by code (sign bit 3),
# E8M0 scale = 2^(v - 127) with v = 255 NaN.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def mx_row(q, v):
    """One MXFP4 row from codes q [K] and scale bytes v [K/32], written from the
    layout description (byte b: column 2b low nibble, 2b+1 high), padded to 16."""
    q = np.asarray(q, np.uint8)
    body = bytes((q[0::2] | (q[1::2] << 4)).astype(np.uint8)) + bytes(np.asarray(v, np.uint8))
    return body + bytes((-len(body)) % 16)


def mx_slab(H, I, q1, v1, q3, v3, q2, v2):
    blob = b"".join(mx_row(q1[r], v1[r]) + mx_row(q3[r], v3[r]) for r in range(I))
    blob += b"".join(mx_row(q2[r], v2[r]) for r in range(H))
    return np.frombuffer(blob, np.uint8).copy()


def test_mx_element_and_scale_values():
    for q, ref in enumerate(E2M1_TABLE):
        got = oracle.e2m1_to_double(q)
        assert got == ref and np.signbit(got) == np.signbit(ref), q
    assert oracle.e8m0_to_double(127) == 1.0
    assert oracle.e8m0_to_double(120) == 2.0 ** -7
    assert oracle.e8m0_to_double(0) == 2.0 ** -127
    assert oracle.e8m0_to_double(254) == 2.0 ** 127
    assert np.isnan(oracle.e8m0_to_double(255))


@pytest.mark.parametrize("H,I", [(64, 32), (96, 64)])
def test_mx_dequant_matches_layout(H, I):
    rng = np.random.default_rng(H + I)
    q1, q3 = rng.integers(0, 16, (I, H)), rng.integers(0, 16, (I, H))
    q2 = rng.integers(0, 16, (H, I))
    v1, v3 = rng.integers(100, 140, (I, H // 32)), rng.integers(100, 140, (I, H // 32))
    v2 = rng.integers(100, 140, (H, I // 32))
    slab = mx_slab(H, I, q1, v1, q3, v3, q2, v2)
    assert slab.size == oracle.slab_bytes(H, I, 1) == synth.slab_bytes(H, I, 1)
    tab = np.array(E2M1_TABLE)
    for which, (q, v) in enumerate([(q1, v1), (q3, v3), (q2, v2)]):
        ref = tab[q] * np.ldexp(1.0, np.repeat(v, 32, axis=1) - 127)
        np.testing.assert_array_equal(oracle.dequant(slab, H, I, which, fmt=1), ref)


def test_mx_expert_ffn_closed_form():
    """All weights 1.5 * 2^-6 (code 3, scale byte 121): g = u = w * sum(x),
    h = silu(g) * u, y = w * I * h in every row."""
    H, I = 64, 32
    w = 1.5 * 2.0 ** -6
    c = lambda R, K: (np.full((R, K), 3), np.full((R, K // 32), 121))
    slab = mx_slab(H, I, *c(I, H), *c(I, H), *c(H, I))
    x = np.linspace(0.1, 1.0, H)
    g, u, h, y = oracle.expert_ffn(slab, H, I, x, fmt=1)
    gs = w * x.sum()
    np.testing.assert_allclose(g, gs, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(h, gs / (1 + np.exp(-gs)) * gs, rtol=1e-13)
    np.testing.assert_allclose(y, w * I * h[0], rtol=1e-13)


def test_mx_synth_slabs_follow_the_recipe():
    H, I = 96, 64
    slab = synth.expert_slab(5, 1, 3, H, I, fmt=1)
    rb = lambda K: (K // 2 + K // 32 + 15) // 16 * 16
    for r in range(I):
        for off, K in ((2 * r * rb(H), H), (2 * r * rb(H) + rb(H), H)):
            row = slab[off:off + rb(K)]
            assert set(row[K // 2:K // 2 + K // 32].tolist()) <= {120, 121, 122}
            assert not row[K // 2 + K // 32:].any()  # padding
    vals = oracle.dequant(slab, H, I, 2, fmt=1)
    assert np.isfinite(vals).all() and np.abs(vals).max() <= 6 * 2.0 ** -5
    assert (synth.expert_slab(5, 1, 3, H, I, fmt=1) == slab).all()
    assert not (synth.expert_slab(5, 1, 4, H, I, fmt=1) == slab).all()


# ---------------------------------------------------------------- weight format 2 (super-blocks)
def sb_row(q, d, dmin, s, m):
    """One super-block row from codes q [K], fp16 d/dmin per super-block and
    6-bit codes s, m [K/256, 8], written from the layout description."""
    q = np.asarray(q, np.uint8)
    out = bytes((q[0::2] | (q[1::2] << 4)).astype(np.uint8))
    for b in range(len(d)):
        fs = sum(int(s[b][j]) << (6 * j) for j in range(8))
        fm = sum(int(m[b][j]) << (6 * j) for j in range(8))
        out += (np.float16(d[b]).tobytes() + np.float16(dmin[b]).tobytes() + fs.to_bytes(6, "little")
                + fm.to_bytes(6, "little"))
    return out


def test_sb_dequant_matches_layout():
    H, I = 512, 256
    rng = np.random.default_rng(11)
    mats = []
    for R, K in ((I, H), (I, H), (H, I)):
        q = rng.integers(0, 16, (R, K))
        d = rng.uniform(1e-4, 1e-3, (R, K // 256)).astype(np.float16)
        dmin = rng.uniform(1e-4, 1e-3, (R, K // 256)).astype(np.float16)
        s, m = rng.integers(0, 64, (R, K // 256, 8)), rng.integers(0, 64, (R, K // 256, 8))
        mats.append((q, d, dmin, s, m))
    rows = [[sb_row(*(a[r] for a in mat)) for r in range(len(mat[0]))] for mat in mats]
    slab = np.frombuffer(b"".join(rows[0][r] + rows[1][r] for r in range(I)) + b"".join(rows[2]), np.uint8).copy()
    assert slab.size == oracle.slab_bytes(H, I, 2) == synth.slab_bytes(H, I, 2) == 3 * H * I * 9 // 16
    for which, (q, d, dmin, s, m) in enumerate(mats):
        R, K = q.shape
        blk = np.arange(K) // 32
        sbk, j = blk // 8, blk % 8
        ref = (d.astype(np.float64)[:, sbk] * s[:, sbk, j] * q - dmin.astype(np.float64)[:, sbk] * m[:, sbk, j])
        np.testing.assert_array_equal(oracle.dequant(slab, H, I, which, fmt=2), ref)
    assert oracle.slab_bytes(96, 256, 2) == 0


def test_sb_synth_slabs_follow_the_recipe():
    H, I = 512, 256
    slab = synth.expert_slab(9, 0, 2, H, I, fmt=2)
    rb = H // 2 + H // 16
    for r in (0, I - 1):
        h = slab[2 * r * rb + H // 2:2 * r * rb + H // 2 + 16]
        d, dmin = h[0:2].view(np.float16)[0], h[2:4].view(np.float16)[0]
        assert np.float16(4 * np.float64(d)) == dmin and 0.0002 <= float(d) < 0.002
        fs = int.from_bytes(bytes(h[4:10]), "little")
        assert all(16 <= (fs >> (6 * j)) & 63 <= 63 for j in range(8))
    w = oracle.dequant(slab, H, I, 2, fmt=2)
    assert np.isfinite(w).all() and 0.01 < np.abs(w).max() < 1.0
    assert (synth.expert_slab(9, 0, 2, H, I, fmt=2) == slab).all()
