"""moe_pack_fp8_payload / moe_unpack_fp8_payload (HIP) against the oracle, and a loop-back run.

Send plan, codes and scales are bit-exact; the unpacked rows are bit-exact fp32 (bf16: the same
value rounded to nearest even). Loop-back: the packed rows, fed to the FP8 grouped FFN through
slot_send, give the same expert outputs bit for bit as the local FP8 path.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_transformer_02_amd as moe
import workloads as W
from gpu_helpers import host, report

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _idx(T, N_r, K, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.multinomial(torch.ones(N_r, device=DEV).expand(T, N_r), K, replacement=False,
                             generator=g).to(torch.int32)


def _x(T, H, dtype, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.randn((T, H), generator=g, device=DEV)
    x = torch.where(torch.rand((T, H), generator=g, device=DEV) < 1e-3, x * 50, x)
    return x.to(dtype)


@pytest.mark.parametrize("T,H,N_r,K,R,dtype", [
    (128, 7168, 256, 8, 8, torch.bfloat16), (4096, 1024, 256, 8, 8, torch.bfloat16),
    (67, 256, 16, 4, 4, torch.float32), (33, 512, 32, 8, 32, torch.bfloat16), (50, 128, 64, 6, 1, torch.bfloat16),
    (1, 128, 4, 1, 2, torch.float32), (300, 384, 60, 5, 3, torch.bfloat16)])
def test_pack_bit_exact(T, H, N_r, K, R, dtype):
    x, idx = _x(T, H, dtype, T + H), _idx(T, N_r, K, T * 3 + R)
    p = moe.moe_pack_fp8_payload(x, idx, N_r, R)
    torch.cuda.synchronize()
    ref = oracle.pack_fp8_payload(x.float().cpu().numpy(), host(idx), N_r, R)
    n = int(ref["offsets"][-1])
    for key in ("counts", "offsets", "slot_send"):
        assert np.array_equal(host(p[key]), ref[key]), key
    assert np.array_equal(host(p["send_token"])[:n], ref["send_token"])
    assert np.array_equal(host(p["codes"])[:n], ref["codes"])
    assert np.array_equal(host(p["scales"])[:n].view(np.uint32), ref["scales"].view(np.uint32))
    report(f"payload pack T={T} H={H} N_r={N_r} K={K} R={R}", rows=n, max_rows=T * min(K, R))


def test_pack_skips_out_of_range_ids():
    x, idx = _x(40, 256, torch.bfloat16, 1), _idx(40, 16, 3, 2)
    idx[5, 1] = -3
    idx[9, 0] = 16
    p = moe.moe_pack_fp8_payload(x, idx, 16, 4)
    sl = host(p["slot_send"])
    assert sl[5 * 3 + 1] == -1 and sl[9 * 3 + 0] == -1
    valid = host(idx).copy()
    valid[5, 1] = valid[5, 0]          # repeats of an existing choice: same plan as dropping the entry
    valid[9, 0] = valid[9, 1]
    ref = oracle.dispatch_by_rank(valid, 16, 4)
    assert np.array_equal(host(p["offsets"]), ref["offsets"])


def test_pack_empty_batch():
    p = moe.moe_pack_fp8_payload(torch.empty((0, 128), dtype=torch.bfloat16, device=DEV),
                                 torch.empty((0, 4), dtype=torch.int32, device=DEV), 8, 2)
    assert (host(p["counts"]) == 0).all() and (host(p["offsets"]) == 0).all()


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_unpack_bit_exact(out_dtype):
    x, idx = _x(257, 1024, torch.bfloat16, 3), _idx(257, 64, 8, 4)
    p = moe.moe_pack_fp8_payload(x, idx, 64, 8)
    n = int(host(p["offsets"])[-1])
    out = moe.moe_unpack_fp8_payload(p["codes"][:n], p["scales"][:n], out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = oracle.unpack_fp8_payload(host(p["codes"])[:n], host(p["scales"])[:n])
    if out_dtype == torch.float32:
        assert np.array_equal(host(out).view(np.uint32), ref.view(np.uint32))
    else:
        assert torch.equal(out.cpu(), torch.from_numpy(ref).to(torch.bfloat16))
    # decoded rows stay within the FP8 rounding of the token they carry
    tok = host(p["send_token"])[:n]
    xr = x.float().cpu().numpy()[tok]
    rel = np.abs(ref - xr).max() / np.abs(xr).max()
    report(f"payload unpack {out_dtype}", rows=n, max_rel_vs_source=float(rel))
    assert rel <= 2 ** -4


def test_loopback_payload_feeds_the_fp8_expert_gemm():
    # all 8 ranks looped back to this GPU: every routed row reads its activation from the send row
    # that carries it (slot_send) instead of from the locally quantized u
    cfg = W.config("fp8").scaled(T=512)
    inp = W.make_inputs(cfg, device=DEV, with_weights=False)
    u = inp["u"]
    T, H, N_r, K, I = cfg.T, cfg.H, cfg.N_r, cfg.K, 256
    idx = _idx(T, N_r, K, 9)
    g = torch.Generator(device=DEV).manual_seed(10)
    w = [(torch.randn(s, generator=g, device=DEV) / s[-1] ** 0.5).bfloat16() for s in
         ((N_r, I, H), (N_r, I, H), (N_r, H, I))]
    q = []
    for t in w:
        G_, R_, C_ = t.shape
        c, s = moe.fp8_quant_tiles(t.reshape(G_ * R_, C_), 128)
        q.append((c.view(G_, R_, C_), s.view(G_, R_ // 128, C_ // 128)))
    (gc, gs), (uc, us), (dc, ds) = q
    counts, offsets, row_token, slot_row = moe.moe_permute(idx, N_r)
    uq, usc = moe.fp8_quant_tiles(u, 1)
    y_local = moe.moe_grouped_ffn(offsets, T * K, uq, gc, uc, dc, row_index=row_token, X_scales=usc,
                                  Wg_scales=gs, Wu_scales=us, Wd_scales=ds)
    p = moe.moe_pack_fp8_payload(u, idx, N_r, 8)
    recv_index = torch.empty(T * K, dtype=torch.int32, device=DEV)
    recv_index[slot_row.long()] = p["slot_send"]          # routed row -> the send row carrying its token
    n = int(host(p["offsets"])[-1])
    y_recv = moe.moe_grouped_ffn(offsets, T * K, p["codes"][:n], gc, uc, dc, row_index=recv_index,
                                 X_scales=p["scales"][:n], Wg_scales=gs, Wu_scales=us, Wd_scales=ds)
    torch.cuda.synchronize()
    assert torch.equal(y_recv, y_local)
    report("payload loop-back into the FP8 grouped FFN", rows_sent=n, routed_rows=T * K)
