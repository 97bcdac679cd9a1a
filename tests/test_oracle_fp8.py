"""Pins for the oracle's E4M3FN codec and tile/block quantizer (CPU only).

The recipe ("官方揭秘DeepSeek-V3模型训练全流程" §4.3; "รายงานเชิงเทคนิคของ DeepSeek-V3" key ideas FP8 bullet): E4M3 operands,
one scale per 1x128 activation tile / 128x128 weight block from the online
max |x|. The codec is checked against the format's defining points, against
torch's float8_e4m3fn conversion (an independent library routine) on every
rounding boundary, and the quantizer against closed forms.
"""
import numpy as np
import pytest
import torch

import oracle


def test_decode_defining_points():
    d = oracle.e4m3fn_decode
    assert d(0x00) == 0.0 and np.signbit(d(0x80)) and d(0x80) == 0.0
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9           # subnormals 2^-6 * m/8
    assert d(0x08) == 2.0 ** -6                                          # smallest normal
    assert d(0x38) == 1.0 and d(0x3C) == 1.5 and d(0x40) == 2.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0                        # largest finite
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    v = d(np.arange(0x7F))
    assert (np.diff(v) > 0).all()                                        # codes order the values


def test_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.e4m3fn_decode(codes)
    finite = ~np.isnan(ref)
    assert (np.isnan(ours) == ~finite).all()
    assert np.array_equal(ours[finite], ref[finite])
    assert np.array_equal(np.signbit(ours[finite]), np.signbit(ref[finite]))


def test_encode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3fn_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3fn_encode(vals), codes)


def _boundary_sweep():
    """Every fp32 whose exponent is in the E4M3 range, with all top-10 mantissa patterns and
    low-13-bit patterns that sit on, just below and just above every possible rounding boundary."""
    exps = np.arange(127 - 12, 127 + 9)                        # 2^-12 .. 2^8
    top = np.arange(1 << 10)
    low = np.array([0, 1, 0xFFF, 0x1000, 0x1001, 0x1FFF])
    bits = (exps[:, None, None] << 23) | (top[None, :, None] << 13) | low[None, None, :]
    bits = bits.reshape(-1).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.abs(v) <= 448.0]
    return np.concatenate([v, -v, np.float32([0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -10, 448.0, 2.0 ** -149])])


def test_encode_matches_torch_on_every_boundary():
    v = _boundary_sweep()
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = oracle.e4m3fn_encode(v)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (v[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_encode_rounding_closed_forms_and_saturation():
    enc = lambda x: int(oracle.e4m3fn_encode(np.float32(x)))
    assert enc(1.0625) == 0x38            # halfway 1.0 / 1.125 -> even mantissa (1.0)
    assert enc(1.1875) == 0x3A            # halfway 1.125 / 1.25 -> 1.25 (even)
    assert enc(2.0 ** -10) == 0x00        # halfway 0 / 2^-9 -> 0
    assert enc(3 * 2.0 ** -10) == 0x02    # halfway 2^-9 / 2^-8 -> 2^-8
    assert enc(-3 * 2.0 ** -10) == 0x82
    assert enc(-0.0) == 0x80 and enc(0.0) == 0x00
    for x in [448.0, 449.0, 463.99, 464.0, 480.0, 1e6, 3.0e38]:
        assert enc(x) == 0x7E and enc(-x) == 0xFE                        # satfinite, never NaN
    with pytest.raises(ValueError):
        oracle.e4m3fn_encode(np.float32([np.nan]))


def test_quantizer_amax_element_and_scale():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((4, 512)) * np.exp(rng.standard_normal((4, 512)))).astype(np.float32)
    codes, scales = oracle.quantize_tiles(x, 1, 128)
    assert codes.shape == (4, 512) and scales.shape == (4, 4) and scales.dtype == np.float32
    for r in range(4):
        for j in range(4):
            tile = x[r, 128 * j:128 * (j + 1)]
            amax = np.max(np.abs(tile))
            assert scales[r, j] == np.float32(amax) / np.float32(448.0)
            i = int(np.argmax(np.abs(tile)))
            # amax / fl32(amax/448) lies within an ulp of 448, which rounds to the 448 code
            assert codes[r, 128 * j + i] == (0xFE if tile[i] < 0 else 0x7E)


def test_quantizer_zero_tile_and_block_shape():
    x = np.zeros((256, 384), np.float32)
    x[0, 0] = -0.0
    x[200:, 300:] = 1.5
    codes, scales = oracle.quantize_tiles(x, 128, 128)
    assert scales.shape == (2, 3)
    assert scales[0, 0] == 0 and codes[0, 0] == 0x80 and codes[1, 1] == 0x00
    assert scales[1, 2] == np.float32(1.5) / np.float32(448)
    assert (codes[200:, 300:] == 0x7E).all()


def test_quantizer_lossless_on_representable_tiles():
    # a tile whose amax is 448 * 2^k and whose values are E4M3 values * 2^k quantizes exactly
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 0x7F, (128, 256)).astype(np.uint8) | (rng.integers(0, 2, (128, 256)) << 7).astype(np.uint8)
    codes[:, 0] = 0x7E
    codes[:, 128] = 0xFE
    k = rng.integers(-8, 8, (128, 2))
    vals = oracle.e4m3fn_decode(codes) * np.repeat(2.0 ** k, 128, axis=1)
    x = vals.astype(np.float32)
    assert np.array_equal(x.astype(np.float64), vals)
    assert np.array_equal(oracle.fp8_roundtrip(x, 1, 128), vals)
    q, s = oracle.quantize_tiles(x, 1, 128)
    assert np.array_equal(s, (2.0 ** k).astype(np.float32))
    assert np.array_equal(q, codes)


def test_fp8_error_bound():
    # Each E4M3 value is within 2^-4 relative (3-bit mantissa, RNE) of fl32(x/scale) for
    # normal codes, and within 2^-10 * scale absolute in the subnormal range.
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((16, 1024)) * np.where(rng.random((16, 1024)) < 1e-3, 50, 1)).astype(np.float32)
    y = oracle.fp8_roundtrip(x, 1, 128)
    _, s = oracle.quantize_tiles(x, 1, 128)
    sc = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(y - x.astype(np.float64))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 2.0 ** -20)
    assert (err <= bound).all()


def test_fp8_layer_close_to_exact_layer():
    """FP8 emulation changes a small layer by about the E4M3 relative error, not more."""
    rng = np.random.default_rng(3)
    T, H, N_r, K, I = 16, 256, 8, 2, 128
    u = rng.standard_normal((T, H)).astype(np.float32)
    E = (rng.standard_normal((N_r, H)) / 16).astype(np.float32)
    W = [(rng.standard_normal((I, H)) / 16, rng.standard_normal((I, H)) / 16, rng.standard_normal((H, I)) / np.sqrt(I))
         for _ in range(N_r)]
    S = [W[0]]
    exact = oracle.layer_forward(u, E, np.zeros(N_r, np.float32), K, W, S)
    q = oracle.layer_forward(u, E, np.zeros(N_r, np.float32), K, W, S, fp8=True)
    assert np.array_equal(exact["idx"], q["idx"])                      # the router is not quantized
    ffn_e = exact["out"] - u
    ffn_q = q["out"] - u
    rel = np.linalg.norm(ffn_q - ffn_e) / np.linalg.norm(ffn_e)
    assert 1e-3 < rel < 0.1


def _torch_fp8_value(x, tile_rows, tile_cols):
    """FP8 value of x built from library pieces: fp32 amax/448 scale, torch's float8_e4m3fn cast."""
    x = torch.from_numpy(np.asarray(x, np.float32))
    R, C = x.shape
    xt = x.reshape(R // tile_rows, tile_rows, C // tile_cols, tile_cols)
    scale = xt.abs().amax(dim=(1, 3), keepdim=True) / torch.tensor(448.0)
    q = torch.where(scale == 0, xt, xt / scale).to(torch.float8_e4m3fn)
    return (q.to(torch.float64) * scale.to(torch.float64)).reshape(R, C).numpy()


def test_fp8_layer_matches_library_composition():
    """The FP8 layer quantizes u, every weight and h, and nothing else (residual, router, gates stay exact)."""
    rng = np.random.default_rng(9)
    T, H, N_r, K, I = 12, 256, 6, 2, 256
    u = (rng.standard_normal((T, H)) * np.where(rng.random((T, H)) < 0.01, 50, 1)).astype(np.float32)
    E = (rng.standard_normal((N_r, H)) / 16).astype(np.float32)
    W = [tuple(rng.standard_normal(s).astype(np.float32) / 16 for s in [(I, H), (I, H), (H, I)]) for _ in range(N_r + 1)]
    b = (rng.random(N_r) * 0.02 - 0.01).astype(np.float32)
    got = oracle.layer_forward(u, E, b, K, W[:N_r], [W[N_r]], fp8=True)
    xq = _torch_fp8_value(u, 1, 128)

    def ffn(wg, wu, wd, rows):
        wg, wu, wd = (_torch_fp8_value(w, 128, 128) for w in (wg, wu, wd))
        z = np.einsum("th,ih->ti", xq[rows], wg)
        v = np.einsum("th,ih->ti", xq[rows], wu)
        h = _torch_fp8_value((z / (1 + np.exp(-z)) * v).astype(np.float32), 1, 128)
        return np.einsum("ti,hi->th", h, wd)

    s = 1 / (1 + np.exp(-(u.astype(np.float64) @ E.T.astype(np.float64))))
    ref = u.astype(np.float64) + ffn(*W[N_r], np.arange(T))
    for t in range(T):
        sel = got["idx"][t]
        g = s[t, sel] / s[t, sel].sum()
        for k in range(K):
            ref[t] += g[k] * ffn(*W[sel[k]], np.array([t]))[0]
    assert np.max(np.abs(got["out"] - ref)) <= 1e-12 * np.max(np.abs(ref))
