"""moe_grouped_ffn (HIP) against the oracle's SwiGLU expert FFN, group by group.

Group sizes include empty groups, single rows and ragged tails around every row-tile
size (16, 32, 64), for the fp32, bf16 and FP8 (E4M3, 1x128 / 128x128 scales) paths.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_transformer_02_amd as moe
from gpu_helpers import f64, host, max_rel, frob_rel, report, row_frob_max

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _problem(counts, H, I, dtype, seed, x_rows=None, gather=True):
    g = torch.Generator(device=DEV).manual_seed(seed)
    G = len(counts)
    total = int(sum(counts))
    x_rows = x_rows or max(total, 1)
    X = torch.randn((x_rows, H), generator=g, device=DEV).to(dtype)
    wdt = dtype
    Wg = (torch.randn((G, I, H), generator=g, device=DEV) / H ** 0.5).to(wdt)
    Wu = (torch.randn((G, I, H), generator=g, device=DEV) / H ** 0.5).to(wdt)
    Wd = (torch.randn((G, H, I), generator=g, device=DEV) / I ** 0.5).to(wdt)
    offsets = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=DEV)
    row_index = torch.randint(0, x_rows, (total,), generator=g, device=DEV, dtype=torch.int32) if gather else None
    return X, Wg, Wu, Wd, offsets, row_index


def _reference(X, Wg, Wu, Wd, offsets, row_index, fp8=False):
    off = host(offsets)
    x = f64(X)
    if fp8:
        x = oracle.fp8_roundtrip(x, 1, 128)
    ri = host(row_index) if row_index is not None else np.arange(off[-1])
    ys = []
    for gi in range(len(off) - 1):
        rows = ri[off[gi]:off[gi + 1]]
        if rows.size == 0:
            continue
        ys.append(oracle.swiglu_ffn(x[rows], host(Wg[gi]), host(Wu[gi]), host(Wd[gi]), fp8=fp8))
    return np.concatenate(ys) if ys else np.zeros((0, X.shape[1]))


@pytest.mark.parametrize("counts", [[0, 1, 17, 40, 6], [64], [3, 0, 0, 130]])
def test_ffn_f32(counts):
    X, Wg, Wu, Wd, off, ri = _problem(counts, 128, 64, torch.float32, 1)
    Y = moe.moe_grouped_ffn(off, int(sum(counts)), X, Wg, Wu, Wd, row_index=ri)
    ref = _reference(X, Wg, Wu, Wd, off, ri)
    err = max_rel(f64(Y), ref)
    report(f"ffn f32 {counts}", max_rel=err)
    assert err <= 1e-5


@pytest.mark.parametrize("counts,gather,H,I", [
    ([1, 2, 0, 5, 16, 3, 0, 9], True, 256, 128),       # decode-like: <= 16 rows per group (RM=1)
    ([17, 31, 32, 33, 0, 1], True, 256, 128),          # RM = 2 around the 32-row tile
    ([0, 1, 63, 64, 65, 127, 129, 200], True, 256, 128),   # 256x256 LDS tiles, ragged groups
    ([300], False, 256, 128),                          # shared-expert form: one group, no gather
    ([600, 3, 257, 0, 512, 513, 256], True, 256, 128), # several 256-row tiles per group
    # H % 512 == 0 and I % 256 == 0: LDS tiles of 256 rows x 256 columns, a tail of <= 128 rows
    # in a 128 x 512 tile
    ([0, 1, 127, 128, 129, 200, 255, 300], True, 512, 256),
    ([150], False, 512, 256),
    ([600, 3, 257, 0, 512, 513, 256], True, 512, 256),
    ([2600, 5, 300], True, 512, 256),                 # more 256-row tiles than one band of 8, then a tail
    # tails of 129..255 rows: one 256-row tile whose rows past the group re-read a valid row
    ([129, 140, 144, 159, 160, 161, 0, 385, 416, 417], True, 512, 256),
    ([2200, 7, 150], True, 512, 256),                 # a band of 8 256-row tiles, then a 152-row tail
    # H % 512 == 0 and I % 512 == 0 with decode-sized groups: the weight-streaming kernel (a 40-row
    # group takes three 16-row tiles that share each weight tile)
    ([1, 2, 0, 5, 16, 3, 40, 0, 7], True, 1024, 512),
    ([4], False, 512, 1024),
    ([0] * 100 + [700] + [0] * 99 + [1], True, 512, 512),   # one group in 44 row tiles among empty ones
    ([16, 17, 0, 32, 33, 1] + [0] * 8, True, 512, 512),    # row-tile edges of the streaming kernel
])
def test_ffn_bf16(counts, gather, H, I):
    X, Wg, Wu, Wd, off, ri = _problem(counts, H, I, torch.bfloat16, 2, gather=gather)
    Y = moe.moe_grouped_ffn(off, int(sum(counts)), X, Wg, Wu, Wd, row_index=ri)
    ref = _reference(X, Wg, Wu, Wd, off, ri)
    err = max_rel(f64(Y), ref)
    report(f"ffn bf16 {counts}", max_rel=err)
    assert err <= 1e-2


@pytest.mark.parametrize("counts,H,I", [
    ([1, 2, 0, 5, 16, 3, 0, 9], 256, 128),           # register-streamed kernel, RM = 1
    ([17, 31, 32, 33, 0, 1], 256, 128),              # RM = 2
    ([0, 1, 63, 64, 65, 127, 129, 200], 256, 128),   # 256 x 256 LDS tiles
    ([0, 1, 127, 128, 129, 200, 255, 300], 512, 256),   # mixed LDS tiles
    ([130, 160, 161, 0, 416], 512, 256),             # mixed, 256-row tiles for 129+ row tails
    ([1, 2, 0, 5, 16, 3, 40, 0, 7], 1024, 512),      # weight-streaming kernel
])
def test_ffn_bf16_saved_preactivations(counts, H, I):
    # the training form gives bitwise the same Y, and z | v equal to the oracle's products
    X, Wg, Wu, Wd, off, ri = _problem(counts, H, I, torch.bfloat16, 4)
    total = int(sum(counts))
    Y0 = moe.moe_grouped_ffn(off, total, X, Wg, Wu, Wd, row_index=ri)
    zv = torch.full((total, 2 * I), float("nan"), device=DEV)
    Y1 = moe.moe_grouped_ffn(off, total, X, Wg, Wu, Wd, row_index=ri, preact=zv)
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1)
    o, rows, x64 = host(off), host(ri), f64(X)
    err = 0.0
    for g in range(len(counts)):
        r0, r1 = o[g], o[g + 1]
        if r1 == r0:
            continue
        xg = x64[rows[r0:r1]]
        ref = np.concatenate([xg @ f64(Wg[g]).T, xg @ f64(Wu[g]).T], axis=1)
        err = max(err, max_rel(f64(zv)[r0:r1], ref))
    report(f"ffn bf16 saved z|v {counts} H={H} I={I}", max_rel=err)
    assert err <= 1e-5                               # exact bf16 products, fp32 sums


@pytest.mark.parametrize("counts,H,I", [([5, 20, 0, 40], 256, 128),
                                         ([5, 130, 0, 160], 512, 256),  # mixed LDS tiles
                                         ([5, 10, 0, 40], 512, 512)])   # weight-streaming kernel
def test_ffn_bf16_fp32_output_and_rows_past_the_end(counts, H, I):
    X, Wg, Wu, Wd, off, ri = _problem(counts, H, I, torch.bfloat16, 3)
    total = int(sum(counts))
    Y = torch.full((total + 7, H), 123.0, device=DEV)            # 7 rows beyond offsets[-1]
    moe.moe_grouped_ffn(off, total + 7, X, Wg, Wu, Wd, row_index=torch.cat(
        [ri, torch.zeros(7, dtype=torch.int32, device=DEV)]), Y=Y)
    ref = _reference(X, Wg, Wu, Wd, off, ri)
    assert max_rel(f64(Y)[:total], ref) <= 1e-2
    assert (host(Y)[total:] == 123.0).all()                      # untouched


def _decode_counts(n_groups, seed, shared=64):
    """A shared-expert group of `shared` rows, then routed groups of 0..16 rows (decode sizes)."""
    rng = np.random.default_rng(seed)
    return [shared] + [int(c) for c in rng.integers(0, 17, n_groups - 1)]


@pytest.mark.parametrize("counts,H,I", [
    # the weight-streaming kernels at decode-sized groups: 5 and 6 stages per item, thousands of
    # items over the workgroups, a shared-expert group whose row tiles share each weight tile
    (_decode_counts(65, 1), 2560, 1536),
    (_decode_counts(9, 2), 4096, 2048),
    ([3, 0, 5], 2560, 1536),          # fewer items than workgroups: most of them take none
    ([3, 5, 2, 0, 1, 7, 9], 2560, 1536),   # a few more gate/up items than workgroups (1-2 each, all pooled)
    (_decode_counts(257, 4, shared=128), 2560, 1536),   # the layer's decode mix: 257 groups, 128 shared rows
    ([0] * 40 + [1], 2560, 1536),     # a single live row, last group
])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_ffn_bf16_streaming_decode_shapes(counts, H, I, out_dtype):
    X, Wg, Wu, Wd, off, ri = _problem(counts, H, I, torch.bfloat16, 21)
    total = int(sum(counts))
    Y = torch.full((total, H), float("nan"), dtype=out_dtype, device=DEV)
    moe.moe_grouped_ffn(off, total, X, Wg, Wu, Wd, row_index=ri, Y=Y)
    Y2 = torch.full_like(Y, float("nan"))
    moe.moe_grouped_ffn(off, total, X, Wg, Wu, Wd, row_index=ri, Y=Y2)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)          # deterministic
    ref = _reference(X, Wg, Wu, Wd, off, ri)
    err, row_err = max_rel(f64(Y), ref), row_frob_max(f64(Y), ref)
    report(f"ffn bf16 streaming {len(counts)} groups H={H} I={I} {out_dtype}", max_rel=err,
           worst_row=row_err)
    assert err <= 1e-2 and row_err <= 2e-2


def _fp8_problem(counts, H, I, seed):
    X, Wg, Wu, Wd, off, ri = _problem(counts, H, I, torch.bfloat16, seed)
    xc, xs = moe.fp8_quant_tiles(X, 1)
    q = []
    for w in (Wg, Wu, Wd):
        G, R, C = w.shape
        c, s = moe.fp8_quant_tiles(w.reshape(G * R, C), 128)
        q.append((c.view(G, R, C), s.view(G, R // 128, C // 128)))
    return X, Wg, Wu, Wd, off, ri, xc, xs, q


@pytest.mark.parametrize("counts", [[1, 2, 0, 5, 16, 3], [17, 33, 40, 31], [0, 64, 65, 130, 1],
                                    [600, 3, 257, 0, 512, 256]])
def test_ffn_fp8(counts):
    X, Wg, Wu, Wd, off, ri, xc, xs, q = _fp8_problem(counts, 256, 256, 5)
    (gc, gs), (uc, us), (dc, ds) = q
    Y = moe.moe_grouped_ffn(off, int(sum(counts)), xc, gc, uc, dc, row_index=ri, X_scales=xs,
                            Wg_scales=gs, Wu_scales=us, Wd_scales=ds)
    ref = _reference(X, Wg, Wu, Wd, off, ri, fp8=True)
    exact = _reference(X, Wg, Wu, Wd, off, ri, fp8=False)
    err = frob_rel(f64(Y), ref)
    row_err = row_frob_max(f64(Y), ref)
    report(f"ffn fp8 {counts}", frob_rel_vs_fp8_oracle=err, worst_row=row_err,
           frob_rel_vs_unquantized=frob_rel(f64(Y), exact))
    assert err <= 3e-2 and row_err <= 3e-2


@pytest.mark.parametrize("counts,H,I", [
    ([1, 2, 0, 5, 16, 3, 40, 0, 7], 1024, 512),   # weight-streaming fp8 kernels; a 40-row group in 3 tiles
    ([3], 512, 1024),
    ([0] * 100 + [700] + [0] * 99 + [1], 512, 512),   # one group in 44 row tiles among empty ones
    ([16, 17, 0, 32, 33, 1] + [0] * 8, 512, 512),      # row-tile edges
    # a first group of several row tiles (the layer's shared expert): its items weigh more in the
    # split of the work over the workgroups, with fewer items than workgroups and with more
    ([40, 3, 0, 9, 1], 512, 512),
    ([17, 1], 512, 512),
    ([128] + [4, 0, 7, 1, 16, 2, 0, 3] * 4, 1024, 512),
])
def test_ffn_fp8_decode_sized(counts, H, I):
    X, Wg, Wu, Wd, off, ri, xc, xs, q = _fp8_problem(counts, H, I, 13)
    (gc, gs), (uc, us), (dc, ds) = q
    Y = moe.moe_grouped_ffn(off, int(sum(counts)), xc, gc, uc, dc, row_index=ri, X_scales=xs,
                            Wg_scales=gs, Wu_scales=us, Wd_scales=ds)
    ref = _reference(X, Wg, Wu, Wd, off, ri, fp8=True)
    err = frob_rel(f64(Y), ref)
    row_err = row_frob_max(f64(Y), ref)   # every row on its own: a dropped or misplaced small group fails
    report(f"ffn fp8 {counts} H={H} I={I}", frob_rel_vs_fp8_oracle=err, worst_row=row_err)
    assert err <= 3e-2 and row_err <= 3e-2


@pytest.mark.parametrize("H,I", [(8448, 256), (256, 8448)])
def test_ffn_fp8_more_than_64_k_blocks(H, I):
    """66 K blocks of 128 in one GEMM (gate/up, then down): the LDS-tiled fp8 kernels keep the
    weight block scales of blocks 64 and up in a second register per lane."""
    counts = [300, 0, 70]
    X, Wg, Wu, Wd, off, ri, xc, xs, q = _fp8_problem(counts, H, I, 11)
    (gc, gs), (uc, us), (dc, ds) = q
    Y = moe.moe_grouped_ffn(off, int(sum(counts)), xc, gc, uc, dc, row_index=ri, X_scales=xs,
                            Wg_scales=gs, Wu_scales=us, Wd_scales=ds)
    ref = _reference(X, Wg, Wu, Wd, off, ri, fp8=True)
    err = frob_rel(f64(Y), ref)
    row_err = row_frob_max(f64(Y), ref)   # every row on its own: a dropped or misplaced small group fails
    report(f"ffn fp8 {counts} H={H} I={I}", frob_rel_vs_fp8_oracle=err, worst_row=row_err)
    assert err <= 3e-2 and row_err <= 3e-2


def _spoil_rows(ri, x_rows, seed):
    """Every 7th row (offset by the seed) gets a source row outside [0, x_rows): -1, x_rows, x_rows + 1000
    or -5 in turn. Returns the new row_index and the host mask of rows that keep a valid source."""
    r = host(ri).copy()
    bad = np.arange(seed % 7, r.size, 7)
    r[bad] = np.array([-1, x_rows, x_rows + 1000, -5])[np.arange(bad.size) % 4]
    return torch.tensor(r, dtype=torch.int32, device=DEV), (r >= 0) & (r < x_rows)


def _reference_rows(X, Wg, Wu, Wd, offsets, row_index, valid, fp8=False):
    """The oracle's output for the rows with a valid source (in row order), group by group."""
    off, ri, x = host(offsets), host(row_index), f64(X)
    if fp8:
        x = oracle.fp8_roundtrip(x, 1, 128)
    ys = []
    for gi in range(len(off) - 1):
        rows = np.arange(off[gi], off[gi + 1])
        rows = rows[valid[rows]]
        if rows.size:
            ys.append(oracle.swiglu_ffn(x[ri[rows]], host(Wg[gi]), host(Wu[gi]), host(Wd[gi]), fp8=fp8))
    return np.concatenate(ys) if ys else np.zeros((0, X.shape[1]))


@pytest.mark.parametrize("dtype,counts,H,I", [
    ("bf16", _decode_counts(33, 3), 2560, 1536),        # weight-streaming kernels
    ("bf16", [1, 2, 0, 5, 16, 3, 0, 9], 256, 128),      # register-streamed kernel
    ("bf16", [0, 1, 127, 128, 129, 200, 255, 300], 512, 256),   # LDS-tiled kernels
    ("f32", [0, 1, 17, 40, 6], 128, 64),
    ("fp8", [1, 2, 0, 5, 16, 3, 40, 0, 7], 1024, 512),  # weight-streaming fp8 kernels
    ("fp8", [600, 3, 257, 0, 512, 256], 256, 256),      # LDS-tiled fp8 kernels
])
def test_ffn_rows_with_a_source_outside_x(dtype, counts, H, I):
    # the contract: such a row is never read out of bounds and its output is unspecified; every
    # other row is computed as usual (a masked row must not disturb its tile's other rows)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    X, Wg, Wu, Wd, off, ri = _problem(counts, H, I, tdt, 31)
    ri, valid = _spoil_rows(ri, X.shape[0], len(counts))
    total = int(sum(counts))
    if dtype == "fp8":
        xc, xs = moe.fp8_quant_tiles(X, 1)
        q = []
        for w in (Wg, Wu, Wd):
            G, R, C = w.shape
            c, sc = moe.fp8_quant_tiles(w.reshape(G * R, C), 128)
            q.append((c.view(G, R, C), sc.view(G, R // 128, C // 128)))
        (gc, gs), (uc, us), (dc, ds) = q
        Y = moe.moe_grouped_ffn(off, total, xc, gc, uc, dc, row_index=ri, X_scales=xs, Wg_scales=gs,
                                Wu_scales=us, Wd_scales=ds)
    else:
        Y = moe.moe_grouped_ffn(off, total, X, Wg, Wu, Wd, row_index=ri)
    torch.cuda.synchronize()
    ref = _reference_rows(X, Wg, Wu, Wd, off, ri, valid, fp8=dtype == "fp8")
    got = f64(Y)[valid]
    if dtype == "fp8":
        err, row_err = frob_rel(got, ref), row_frob_max(got, ref)
        assert err <= 3e-2 and row_err <= 3e-2
    else:
        err, row_err = max_rel(got, ref), row_frob_max(got, ref)
        assert err <= (1e-5 if dtype == "f32" else 1e-2) and row_err <= (1e-4 if dtype == "f32" else 2e-2)
    report(f"ffn {dtype} rows with a source outside X, {len(counts)} groups H={H} I={I}", err=err,
           worst_row=row_err, spoiled=int((~valid).sum()))


def test_ffn_deterministic():
    counts = [0, 1, 63, 64, 65, 127, 129, 200]
    X, Wg, Wu, Wd, off, ri = _problem(counts, 256, 128, torch.bfloat16, 7)
    a = moe.moe_grouped_ffn(off, int(sum(counts)), X, Wg, Wu, Wd, row_index=ri).clone()
    b = moe.moe_grouped_ffn(off, int(sum(counts)), X, Wg, Wu, Wd, row_index=ri)
    assert torch.equal(a, b)
