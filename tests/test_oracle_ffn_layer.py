"""Pins for the oracle's expert FFN and whole-layer output (CPU only).

"รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2: h'_t = u_t + sum_i FFN^(s)_i(u_t) + sum_i g_{i,t} FFN^(r)_i(u_t).
"""
import math

import numpy as np
import pytest

import oracle


def _sig(x):
    return 1.0 / (1.0 + math.exp(-x))


def test_ffn_against_scalar_loops():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 4))
    wg, wu, wd = rng.standard_normal((5, 4)), rng.standard_normal((5, 4)), rng.standard_normal((4, 5))
    y = oracle.swiglu_ffn(x, wg, wu, wd)
    for t in range(3):
        h = []
        for n in range(5):
            z = sum(x[t, k] * wg[n, k] for k in range(4))
            v = sum(x[t, k] * wu[n, k] for k in range(4))
            h.append(z * _sig(z) * v)
        for m in range(4):
            ref = sum(h[n] * wd[m, n] for n in range(5))
            assert y[t, m] == pytest.approx(ref, rel=1e-12, abs=1e-14)


def test_ffn_special_cases():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 8))
    wu, wd = rng.standard_normal((6, 8)), rng.standard_normal((8, 6))
    assert (oracle.swiglu_ffn(x, np.zeros((6, 8)), wu, wd) == 0).all()     # SiLU(0) = 0
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert oracle.silu(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-16)
    assert oracle.silu(np.array([1.0]))[0] == pytest.approx(_sig(1.0), rel=1e-15)


def test_bf16_bits_decode():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F], np.uint16)
    v = oracle.bf16_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[3] == 0.0 and np.signbit(v[4])
    assert v[2] == 3.140625
    assert v[5] == (2 - 2 ** -7) * 2.0 ** 127


def test_layer_hand_example():
    """T=1, H=2, N_r=3, K=2, I=1; every intermediate in closed form.

    u = (1, -1); centroids give logits (0, 2, -2) -> s = (1/2, sig(2), sig(-2)).
    Routed expert i: W_g = [[1, 0]] (z = 1), W_u = [[0, c_i]] (v = -c_i), W_d = [[1], [0]]
    -> FFN_i(u) = (-c_i * silu(1), 0) with c = (1, 2, 3).
    Shared: W_g = [[0, -1]] (z = 1), W_u = [[1, 0]] (v = 1), W_d = [[0], [1]] -> (0, silu(1)).
    """
    u = np.array([[1.0, -1.0]])
    E = np.array([[1.0, 1.0], [2.0, 0.0], [0.0, 2.0]])
    c = [1.0, 2.0, 3.0]
    routed = [(np.array([[1.0, 0.0]]), np.array([[0.0, ci]]), np.array([[1.0], [0.0]])) for ci in c]
    shared = [(np.array([[0.0, -1.0]]), np.array([[1.0, 0.0]]), np.array([[0.0], [1.0]]))]
    silu1 = _sig(1.0)
    s = [0.5, _sig(2.0), _sig(-2.0)]
    s32 = [float(np.float32(v)) for v in s]

    # no bias: experts 1 then 0 (s = 0.88, 0.5)
    r = oracle.layer_forward(u, E, np.zeros(3, np.float32), 2, routed, shared)
    assert list(r["idx"][0]) == [1, 0]
    g1, g0 = s[1] / (s[1] + s[0]), s[0] / (s[1] + s[0])
    assert r["gates"][0] == pytest.approx([g1, g0], rel=1e-15)
    exp_out = [1.0 - silu1 * (g1 * 2.0 + g0 * 1.0), -1.0 + silu1]
    assert r["out"][0] == pytest.approx(exp_out, rel=1e-14)
    assert list(r["counts"]) == [1, 1, 0] and list(r["offsets"]) == [0, 1, 2, 2]
    assert list(r["row_token"]) == [0, 0] and list(r["slot_row"]) == [1, 0]

    # bias -1 on expert 1 pushes it out: experts 0 then 2; gates use the unbiased s
    r = oracle.layer_forward(u, E, np.array([0.0, -1.0, 0.0], np.float32), 2, routed, shared)
    assert list(r["idx"][0]) == [0, 2]
    g0, g2 = s[0] / (s[0] + s[2]), s[2] / (s[0] + s[2])
    assert r["gates"][0] == pytest.approx([g0, g2], rel=1e-15)
    assert r["out"][0] == pytest.approx([1.0 - silu1 * (g0 * 1.0 + g2 * 3.0), -1.0 + silu1], rel=1e-14)
    # keys are fp32: fl32(s) + fl32(b)
    assert r["keys"][0, 1] == np.float32(s32[1]) + np.float32(-1.0)


def test_dense_mixture_when_K_equals_N_r():
    """K = N_r with zero bias: the layer is u + FFN_sh(u) + sum_i (s_i / sum_j s_j) FFN_i(u)."""
    rng = np.random.default_rng(4)
    T, H, N_r, I = 9, 8, 5, 6
    u = rng.standard_normal((T, H))
    E = rng.standard_normal((N_r, H)) / math.sqrt(H)
    Wg = rng.standard_normal((N_r, I, H)); Wu = rng.standard_normal((N_r, I, H)); Wd = rng.standard_normal((N_r, H, I))
    Sg, Su, Sd = rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I))
    r = oracle.layer_forward(u, E, np.zeros(N_r, np.float32), N_r, list(zip(Wg, Wu, Wd)), [(Sg, Su, Sd)])
    # independent dense formula (einsum over every expert)
    s = 1.0 / (1.0 + np.exp(-np.einsum("th,eh->te", u, E)))
    w = s / s.sum(axis=1, keepdims=True)
    Z = np.einsum("th,eih->tei", u, Wg)
    V = np.einsum("th,eih->tei", u, Wu)
    Y = np.einsum("tei,ehi->teh", Z / (1 + np.exp(-Z)) * V, Wd)
    zs, vs = u @ Sg.T, u @ Su.T
    ysh = (zs / (1 + np.exp(-zs)) * vs) @ Sd.T
    ref = u + ysh + np.einsum("te,teh->th", w, Y)
    assert np.max(np.abs(r["out"] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_token_sample_matches_full_run():
    rng = np.random.default_rng(6)
    T, H, N_r, K, I = 20, 16, 8, 3, 4
    u = rng.standard_normal((T, H)).astype(np.float32)
    E = rng.standard_normal((N_r, H)).astype(np.float32) / 4
    W = [(rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I))) for _ in range(N_r)]
    S = [(rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I)))]
    full = oracle.layer_forward(u, E, np.zeros(N_r, np.float32), K, W, S)
    part = oracle.layer_forward(u, E, np.zeros(N_r, np.float32), K, W, S, tokens=[3, 17, 0])
    # per-row results do not depend on which other tokens are computed (up to BLAS summation order)
    np.testing.assert_allclose(part["out"], full["out"][[3, 17, 0]], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(part["y_routed"], full["y_routed"][[3, 17, 0]], rtol=1e-13, atol=1e-13)


def test_expert_threads_do_not_change_results():
    rng = np.random.default_rng(8)
    T, H, N_r, K, I = 30, 16, 8, 3, 4
    u = rng.standard_normal((T, H)).astype(np.float32)
    E = rng.standard_normal((N_r, H)).astype(np.float32) / 4
    W = [(rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I))) for _ in range(N_r)]
    S = [(rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I)))]
    a = oracle.layer_forward(u, E, np.zeros(N_r, np.float32), K, W, S)
    b = oracle.layer_forward(u, E, np.zeros(N_r, np.float32), K, W, S, workers=4)
    assert np.array_equal(a["out"], b["out"])
