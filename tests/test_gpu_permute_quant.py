"""moe_permute, moe_bias_update and fp8_quant_tiles (HIP) against the oracle: all bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_transformer_02_amd as moe
from gpu_helpers import host, report
from layouts import dispatch_with_shared

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rand_idx(T, N_r, K, seed, hot=0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    w = torch.ones(N_r, device=DEV)
    if hot:
        w[:hot] = 40.0
    return torch.multinomial(w.expand(T, N_r), K, replacement=False, generator=g).to(torch.int32)


@pytest.mark.parametrize("T,N_r,K,hot", [(1, 4, 1, 0), (67, 16, 2, 0), (64, 16, 2, 0), (128, 256, 8, 0),
                                         (4096, 256, 8, 0), (16384, 256, 8, 8), (100, 1024, 16, 0),
                                         (3000, 33, 5, 2), (65, 1, 1, 0),
                                         # one-workgroup path (T K <= 4096): several rounds, hot
                                         # experts, the largest batch and the first one past it
                                         (300, 64, 8, 4), (512, 256, 8, 8), (256, 1024, 16, 0),
                                         (513, 256, 8, 0),
                                         # chunked path with one thread per expert in the scan,
                                         # and with 1024 threads sharing one expert's chunks
                                         (600, 1024, 16, 0), (5000, 1, 1, 0)])
def test_permute_bit_exact(T, N_r, K, hot):
    idx = _rand_idx(T, N_r, K, T + N_r, hot)
    counts, offsets, row_token, slot_row = moe.moe_permute(idx, N_r)
    torch.cuda.synchronize()
    ref = oracle.dispatch(host(idx), N_r)
    for name, got in [("counts", counts), ("offsets", offsets), ("row_token", row_token), ("slot_row", slot_row)]:
        assert np.array_equal(host(got), ref[name]), name


@pytest.mark.parametrize("T,N_r,K", [(128, 256, 8), (67, 16, 2), (4096, 256, 8), (300, 256, 8)])
def test_permute_with_shared_group_bit_exact(T, N_r, K):
    idx = _rand_idx(T, N_r, K, 7 * T)
    counts, offsets, row_token, slot_row = moe.moe_permute(idx, N_r, shared_rows=T)
    torch.cuda.synchronize()
    ref = dispatch_with_shared(host(idx), N_r, T)
    for name, got in [("counts", counts), ("offsets", offsets), ("row_token", row_token), ("slot_row", slot_row)]:
        assert np.array_equal(host(got), ref[name]), name


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.uint8])
def test_gather_rows_after_the_dispatch(dtype):
    # x_perm[r] = x[row_token[r]] for the n rows the dispatch made (n read on the device), with a
    # shared group in front; rows past n untouched; a row_token outside [0, T) gives a zero row
    T, H, N_r, K = 300, 256, 32, 4
    g = torch.Generator(device=DEV).manual_seed(21)
    idx = _rand_idx(T, N_r, K, 22)
    idx[7, 2] = N_r + 5                                  # no row for this choice
    counts, offsets, row_token, slot_row = moe.moe_permute(idx, N_r, shared_rows=T)
    n = int(offsets[-1].item())
    max_rows = T + T * K
    assert n == max_rows - 1
    if dtype == torch.uint8:
        x = torch.randint(0, 256, (T, H), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
        xs = torch.rand((T, H // 128), generator=g, device=DEV)
        y = torch.full((max_rows, H), 0xAB, dtype=torch.uint8, device=DEV)
        ys = torch.full((max_rows, H // 128), -1.0, device=DEV)
        rt = row_token.clone()
        rt[5] = T + 3                                    # a row whose source lies outside x
        got, gs = moe.moe_gather_rows(x, rt, offsets[-1:], max_rows, x_scales=xs, x_perm=y, x_perm_scales=ys)
    else:
        x = torch.randn((T, H), generator=g, device=DEV).to(dtype)
        y = torch.full((max_rows, H), 7.0, dtype=dtype, device=DEV)
        rt = row_token.clone()
        rt[5] = -2
        got = moe.moe_gather_rows(x, rt, offsets[-1:], max_rows, x_perm=y)
    torch.cuda.synchronize()
    src = host(rt)[:n]
    ok = (src >= 0) & (src < T)
    want = np.zeros((n, H), dtype=host(x).dtype)
    want[ok] = host(x)[src[ok]]
    view = np.uint8 if dtype == torch.uint8 else (np.uint16 if dtype == torch.bfloat16 else np.uint32)
    g_rows = host(got)[:n]
    assert np.array_equal(g_rows.view(view), want.view(view))
    assert not ok[5] and (g_rows[5] == 0).all()
    tail = host(got)[n:]
    assert (tail.view(view) == host(y)[n:].view(view)).all() and tail.shape[0] == 1
    if dtype == torch.uint8:
        ws = np.zeros((n, H // 128), dtype=np.float32)
        ws[ok] = host(xs)[src[ok]]
        assert np.array_equal(host(gs)[:n].view(np.uint32), ws.view(np.uint32))
        assert (host(gs)[n:] == -1.0).all()
    report(f"gather rows {dtype}", rows=n, max_rows=max_rows)


def test_permute_empty_batch():
    idx = torch.empty((0, 4), dtype=torch.int32, device=DEV)
    counts, offsets, _, _ = moe.moe_permute(idx, 32)
    assert (host(counts) == 0).all() and (host(offsets) == 0).all()


def test_permute_skips_out_of_range_ids():
    idx = _rand_idx(50, 16, 3, 1)
    idx[3, 1] = -1
    idx[7, 0] = 16
    counts, offsets, row_token, slot_row = moe.moe_permute(idx, 16)
    sr = host(slot_row)
    assert sr[3 * 3 + 1] == -1 and sr[7 * 3 + 0] == -1
    assert host(offsets)[-1] == 150 - 2
    valid = host(idx).copy()
    ref_counts = np.bincount(valid[(valid >= 0) & (valid < 16)], minlength=16)
    assert np.array_equal(host(counts), ref_counts)


@pytest.mark.parametrize("T", [8192, 128])
def test_permute_is_deterministic(T):
    idx = _rand_idx(T, 256, 8, 5)
    a = [t.clone() for t in moe.moe_permute(idx, 256)]
    b = moe.moe_permute(idx, 256)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_bias_update_bit_exact():
    g = torch.Generator(device=DEV).manual_seed(3)
    counts = torch.randint(0, 40, (256,), generator=g, device=DEV, dtype=torch.int32)
    counts[:5] = 16                                   # T*K/N_r = 16: unchanged
    bias = ((torch.rand(256, generator=g, device=DEV) * 2 - 1) * 0.01).float()
    b0 = host(bias).copy()
    moe.moe_bias_update(counts, bias, 512, 8, 1e-3)
    ref = oracle.bias_update(b0, host(counts), 512, 8, 1e-3)
    assert np.array_equal(host(bias).view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------------------ FP8
def _check_quant(x, tile_rows, label):
    codes, scales = moe.fp8_quant_tiles(x, tile_rows)
    torch.cuda.synchronize()
    xf = x.float().cpu().numpy()
    rc, rs = oracle.quantize_tiles(xf, tile_rows, 128)
    bad = np.count_nonzero(host(codes) != rc)
    report(f"fp8 quant {label}", mismatched_codes=bad, tiles=rs.size)
    assert np.array_equal(host(scales).view(np.uint32), rs.view(np.uint32))
    assert bad == 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quant_activation_tiles(dtype):
    g = torch.Generator(device=DEV).manual_seed(1)
    x = torch.randn((257, 1024), generator=g, device=DEV)
    m = torch.rand((257, 1024), generator=g, device=DEV) < 1e-3
    x = torch.where(m, x * 50, x)
    x[5] = 0.0                                        # zero tiles
    x[6, :128] = -0.0
    x[7] *= 1e-6                                      # small magnitudes
    _check_quant(x.to(dtype), 1, f"1x128 {dtype}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quant_weight_blocks(dtype):
    g = torch.Generator(device=DEV).manual_seed(2)
    x = torch.randn((3 * 256, 384), generator=g, device=DEV) / 16
    x[:128, :128] = 0
    x[300, 200] = 7.0
    _check_quant(x.to(dtype), 128, f"128x128 {dtype}")


def test_quant_v3_activation_and_weight_shapes():
    g = torch.Generator(device=DEV).manual_seed(4)
    u = torch.randn((8192, 7168), generator=g, device=DEV)
    u = torch.where(torch.rand((8192, 7168), generator=g, device=DEV) < 1e-3, u * 50, u).bfloat16()
    _check_quant(u, 1, "u 8192x7168")
    w = (torch.randn((2 * 2048, 7168), generator=g, device=DEV) / 84.66).bfloat16()
    _check_quant(w, 128, "w 2x2048x7168")


def _boundary_values():
    exps = np.arange(127 - 12, 127 + 9)
    top = np.arange(1 << 10)
    low = np.array([0, 1, 0xFFF, 0x1000, 0x1001, 0x1FFF])
    bits = ((exps[:, None, None] << 23) | (top[None, :, None] << 13) | low[None, None, :]).reshape(-1)
    v = bits.astype(np.uint32).view(np.float32)
    v = v[np.abs(v) <= 448.0]
    return np.concatenate([v, -v, np.float32([0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -149])])


def test_encoder_on_every_rounding_boundary_at_unit_scale():
    # each 1x128 tile holds 448 plus 127 sweep values: scale = 448/448 = 1 exactly, so the codes
    # are the encoder applied to the raw values
    v = _boundary_values()
    n = (v.size + 126) // 127
    tiles = np.zeros((n, 128), np.float32)
    tiles[:, 0] = 448.0
    flat = tiles[:, 1:].reshape(-1)
    flat[: v.size] = v
    tiles[:, 1:] = flat.reshape(n, 127)
    x = torch.from_numpy(tiles.reshape(-1, 1024)[: (n * 128) // 1024]).to(DEV) if (n * 128) % 1024 == 0 \
        else torch.from_numpy(np.concatenate([tiles.reshape(-1), np.zeros((-n * 128) % 1024, np.float32)])
                              .reshape(-1, 1024)).to(DEV)
    codes, scales = moe.fp8_quant_tiles(x, 1)
    rc, rs = oracle.quantize_tiles(x.cpu().numpy(), 1, 128)
    assert np.array_equal(host(codes), rc)
    assert np.array_equal(host(scales), rs)
    assert (host(scales).reshape(-1)[:n] == 1.0).all()
