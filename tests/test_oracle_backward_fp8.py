"""Pins for the oracle's FP8 backward (swiglu_ffn_backward_fp8, layer_backward(fp8=True)), CPU only.

What fixes it, other than its own formulas:
* the 128x1 tile quantizer reduces to quantize_tiles on a zero-padded copy, and each column of
  a tile has its own scale: scaling one column by 2^k scales exactly that column's codes' values;
* which axis each GEMM operand is quantized along: a power-of-two scaling of one ROW of dy changes
  only that row of dh, exactly (row-wise 1x128 tiles along H for the dgrad GEMM), and a
  power-of-two scaling of one COLUMN of dy changes only that row of dW_down, exactly (128x1 tiles
  along the tokens for the weight-gradient GEMM); either wrong axis breaks the exactness;
* the whole backward scales exactly with a power-of-two scaling of dy (Q(2^k x) = 2^k Q(x));
* against the exact float64 backward (pinned by finite differences): the FP8 gradients are within
  a few percent, far closer than any dropped term or sign error would leave them;
* against a composition that quantizes with torch's float8_e4m3fn cast (a library encoder):
  equal to rounding, for every gradient of the expert;
* at the layer: with fp8=False the new code path is the old one, and fp8=True equals the
  per-expert FP8 backward assembled by hand from dispatch order.
Readings ("官方揭秘DeepSeek-V3模型训练全流程" §4.3, §4.5): each GEMM operand is quantized
along that GEMM's reduction; the weight-gradient operands in 128x1 tiles over an expert's rows.
"""
import numpy as np
import pytest
import torch

import oracle


def _expert(seed=0, M=200, H=256, I=128):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, H))
    wg = rng.standard_normal((I, H)) / np.sqrt(H)
    wu = rng.standard_normal((I, H)) / np.sqrt(H)
    wd = rng.standard_normal((H, I)) / np.sqrt(I)
    dy = rng.standard_normal((M, H))
    return x, wg, wu, wd, dy


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_row_block_quantizer_reduces_to_quantize_tiles_and_is_per_column():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((300, 8)).astype(np.float32)
    q = oracle.fp8_roundtrip_row_blocks(x)
    xp = np.zeros((384, 8), np.float32)
    xp[:300] = x
    c, s = oracle.quantize_tiles(xp, 128, 1)
    assert np.array_equal(q, oracle.dequantize_tiles(c, s, 128, 1)[:300])
    assert s.shape == (3, 8)
    # the last tile holds rows 256..299 only: its scale is their amax / 448
    assert np.array_equal(s[2], (np.abs(x[256:]).max(axis=0) / np.float32(448)).astype(np.float32))
    # a power-of-two scaling of one column scales exactly that column
    y = x.copy()
    y[:, 3] *= np.float32(2.0 ** 7)
    q2 = oracle.fp8_roundtrip_row_blocks(y)
    assert np.array_equal(q2[:, 3], q[:, 3] * 2.0 ** 7)
    assert np.array_equal(np.delete(q2, 3, axis=1), np.delete(q, 3, axis=1))


def test_dgrad_quantizes_dy_by_rows_along_h():
    x, wg, wu, wd, dy = _expert(2)
    base = oracle.swiglu_ffn_backward_fp8(x, wg, wu, wd, dy)
    r = 37
    dy2 = dy.copy()
    dy2[r] *= 2.0 ** 9
    b2 = oracle.swiglu_ffn_backward_fp8(x, wg, wu, wd, dy2)
    assert np.array_equal(b2["dh"][r], base["dh"][r] * 2.0 ** 9)
    assert np.array_equal(np.delete(b2["dh"], r, axis=0), np.delete(base["dh"], r, axis=0))
    # and dx follows row by row (dz, dv scale with dh; they are quantized by rows along I)
    assert np.array_equal(np.delete(b2["dx"], r, axis=0), np.delete(base["dx"], r, axis=0))
    assert np.allclose(b2["dx"][r], base["dx"][r] * 2.0 ** 9, rtol=0, atol=0)


def test_weight_gradient_quantizes_dy_by_columns_along_tokens():
    x, wg, wu, wd, dy = _expert(3, M=200)        # two tiles over the rows: 128 + 72
    base = oracle.swiglu_ffn_backward_fp8(x, wg, wu, wd, dy)
    c = 11
    dy2 = dy.copy()
    dy2[:, c] *= 2.0 ** 9
    b2 = oracle.swiglu_ffn_backward_fp8(x, wg, wu, wd, dy2)
    assert np.array_equal(b2["dW_down"][c], base["dW_down"][c] * 2.0 ** 9)
    assert np.array_equal(np.delete(b2["dW_down"], c, axis=0), np.delete(base["dW_down"], c, axis=0))


def test_scales_exactly_with_a_power_of_two_dy():
    x, wg, wu, wd, dy = _expert(4)
    a = oracle.swiglu_ffn_backward_fp8(x, wg, wu, wd, dy)
    b = oracle.swiglu_ffn_backward_fp8(x, wg, wu, wd, dy * 2.0 ** -5)
    for k in ("dx", "dh", "dW_gate", "dW_up", "dW_down"):
        assert np.array_equal(b[k], a[k] * 2.0 ** -5), k


def test_close_to_the_exact_backward():
    x, wg, wu, wd, dy = _expert(5, M=300, H=512, I=256)
    e = oracle.swiglu_ffn_backward(x, wg, wu, wd, dy)
    f = oracle.swiglu_ffn_backward_fp8(x, wg, wu, wd, dy)
    errs = {k: _rel(f[k], e[k]) for k in ("dx", "dW_gate", "dW_up", "dW_down")}
    assert all(v < 0.12 for v in errs.values()), errs
    # a planted sign error or a dropped term would be O(1)
    assert _rel(-f["dx"], e["dx"]) > 1.5 and _rel(f["dW_down"] * 0, e["dW_down"]) == 1.0


def _q_torch(x, tile_rows, tile_cols):
    """deq(Q(fl32(x))) with torch's float8_e4m3fn cast as the encoder (scale = fl32(amax/448))."""
    t = torch.from_numpy(np.asarray(x, np.float32))
    R, C = t.shape
    Rp = -(-R // tile_rows) * tile_rows
    tp = torch.zeros((Rp, C), dtype=torch.float32)
    tp[:R] = t
    v = tp.reshape(Rp // tile_rows, tile_rows, C // tile_cols, tile_cols)
    amax = v.abs().amax(dim=(1, 3), keepdim=True)
    scale = amax / 448.0
    q = torch.where(scale == 0, v, v / scale).to(torch.float8_e4m3fn).to(torch.float64) * scale.double()
    return q.reshape(Rp, C)[:R].numpy()


def test_matches_a_composition_on_torchs_fp8_cast():
    x, wg, wu, wd, dy = _expert(6, M=150, H=256, I=128)
    f = oracle.swiglu_ffn_backward_fp8(x, wg, wu, wd, dy)
    wgq, wuq, wdq = (_q_torch(w, 128, 128) for w in (wg, wu, wd))
    xq = _q_torch(x, 1, 128)
    z, v = xq @ wgq.T, xq @ wuq.T
    sig = 1 / (1 + np.exp(-z))
    h = z * sig * v
    dh = _q_torch(dy, 1, 128) @ wdq
    dz = dh * v * sig * (1 + z * (1 - sig))
    dv = dh * z * sig
    ref = {"dx": _q_torch(dz, 1, 128) @ wgq + _q_torch(dv, 1, 128) @ wuq,
           "dW_down": _q_torch(dy, 128, 1).T @ _q_torch(h, 128, 1),
           "dW_gate": _q_torch(dz, 128, 1).T @ _q_torch(x, 128, 1),
           "dW_up": _q_torch(dv, 128, 1).T @ _q_torch(x, 128, 1)}
    for k, r in ref.items():
        assert _rel(f[k], r) < 1e-12, (k, _rel(f[k], r))


def _layer(seed=7, T=40, H=128, N_r=6, K=2, I=128):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((T, H))
    E = rng.standard_normal((N_r, H)) / np.sqrt(H)
    b = np.zeros(N_r, np.float32)
    mk = lambda: tuple(rng.standard_normal(sh) / np.sqrt(sh[1]) for sh in ((I, H), (I, H), (H, I)))
    routed = [mk() for _ in range(N_r)]
    shared = [mk()]
    dout = rng.standard_normal((T, H))
    return u, E, b, K, routed, shared, dout


def test_layer_fp8_backward_assembles_the_expert_backwards():
    u, E, b, K, routed, shared, dout = _layer()
    L = oracle.layer_backward(u, E, b, K, routed, shared, dout, fp8=True)
    idx, g = L["idx"], L["gates"]
    du = dout.copy()
    sh = oracle.swiglu_ffn_backward_fp8(u, *shared[0], dout)
    du += sh["dx"]
    for e in range(len(routed)):
        rt, rk = np.nonzero(idx == e)
        if rt.size == 0:
            continue
        assert np.all(np.diff(rt) > 0)                  # dispatch order: tokens ascending
        be = oracle.swiglu_ffn_backward_fp8(u[rt], *routed[e], g[rt, rk][:, None] * dout[rt])
        np.add.at(du, rt, be["dx"])
        for j, key in enumerate(("dW_gate", "dW_up", "dW_down")):
            assert np.array_equal(L["routed"][e][j], be[key])
    for j, key in enumerate(("dW_gate", "dW_up", "dW_down")):
        assert np.array_equal(L["shared"][0][j], sh[key])
    # the router part is the bf16 rule on the FP8 forward's outputs
    y = np.zeros((u.shape[0], K, u.shape[1]))
    for e in range(len(routed)):
        rt, rk = np.nonzero(idx == e)
        if rt.size:
            y[rt, rk] = oracle.swiglu_ffn(oracle.fp8_roundtrip(u[rt], 1, 128), *routed[e], fp8=True)
    assert np.allclose(L["dgate"], np.einsum("th,tkh->tk", dout, y), rtol=1e-12, atol=1e-12)
    s_sel = np.take_along_axis(L["s"], idx.astype(np.int64), axis=1)
    dlogit = (L["dgate"] - (g * L["dgate"]).sum(1, keepdims=True)) / s_sel.sum(1, keepdims=True) * s_sel * (1 - s_sel)
    du += np.einsum("tk,tkh->th", dlogit, E[idx])
    assert np.allclose(L["du"], du, rtol=1e-12, atol=1e-12)


def test_layer_fp8_flag_off_is_the_bf16_backward():
    u, E, b, K, routed, shared, dout = _layer(8)
    a = oracle.layer_backward(u, E, b, K, routed, shared, dout)
    c = oracle.layer_backward(u, E, b, K, routed, shared, dout, fp8=False)
    assert np.array_equal(a["du"], c["du"]) and np.array_equal(a["dcentroids"], c["dcentroids"])
