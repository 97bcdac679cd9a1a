"""moe_route (HIP) against the oracle: affinity, biased top-K, gates.

Selection is compared bit-exactly on identical fp32 affinities (passed to both
sides). From-scratch runs compare affinities to the float64 sigmoid and the
selection on every token whose top-(K+1) keys are not within 1e-6 of each other.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_transformer_02_amd as moe
import workloads as W
from gpu_helpers import f64, host, near_ties, report

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("T,N_r,K,levels", [
    (64, 16, 2, 0), (67, 16, 2, 8), (1, 1, 1, 0), (128, 256, 8, 0), (257, 256, 8, 64),
    (33, 100, 7, 4), (16, 1024, 16, 16), (50, 16, 16, 3), (4096, 256, 8, 1000), (129, 65, 1, 2)])
def test_selection_on_identical_affinities(T, N_r, K, levels):
    cfg = W.config("decode_bf16").scaled(T=T, N_r=N_r, K=K, seed=T * 7 + N_r)
    s = W.make_affinities(cfg, device=DEV, tie_levels=levels)
    g = torch.Generator(device=DEV).manual_seed(T)
    bias = ((torch.rand(N_r, generator=g, device=DEV) * 2 - 1) * 0.05).float()
    if levels:
        bias = torch.round(bias * levels) / levels      # keep keys tied as well
    idx, gate = moe.moe_route(None, None, bias, K, affinity_in=s)
    torch.cuda.synchronize()
    ref = oracle.route(None, None, host(bias), K, affinity_in=host(s))
    assert np.array_equal(host(idx), ref["idx"])
    err = np.max(np.abs(host(gate) - ref["gates"]))
    report(f"route identical T={T} N_r={N_r} K={K} ties={levels}", gate_err=float(err))
    assert err <= 1e-6


def test_all_equal_affinities_pick_lowest_indices():
    s = torch.full((40, 64), 0.5, device=DEV)
    idx, gate = moe.moe_route(None, None, torch.zeros(64, device=DEV), 8, affinity_in=s)
    assert (host(idx) == np.arange(8)).all()
    assert np.array_equal(host(gate), np.full((40, 8), np.float32(0.125)))


def test_bias_dominance_on_gpu():
    s = W.make_affinities(W.config("prefill_bf16").scaled(T=300), device=DEV)
    b = torch.zeros(256, device=DEV)
    b[[5, 77, 200]] = 1.0
    b[:4] = -1.0
    idx, _ = moe.moe_route(None, None, b, 8, affinity_in=s)
    idx = host(idx)
    assert all(set(row[:3]) == {5, 77, 200} for row in idx)
    assert not np.isin(idx, [0, 1, 2, 3]).any()


def _from_scratch(cfg, T=None, bias_scale=None):
    inp = W.make_inputs(cfg, device=DEV, with_weights=False)
    u = inp["u"] if T is None else inp["u"][:T].contiguous()
    bias = inp["bias"]
    if bias_scale:
        bias = bias + (torch.rand(cfg.N_r, device=DEV) * 2 - 1) * bias_scale
    T = u.shape[0]
    aff = torch.empty((T, cfg.N_r), dtype=torch.float32, device=DEV)
    idx, gate = moe.moe_route(u, inp["centroids"], bias, cfg.K, logit_offset=inp["logit_offset"],
                              affinity_out=aff)
    torch.cuda.synchronize()
    off = None if inp["logit_offset"] is None else host(inp["logit_offset"])
    ref = oracle.route(host(u), host(inp["centroids"]), host(bias), cfg.K, logit_offset=off)
    aerr = float(np.max(np.abs(f64(aff) - ref["s"])))
    ties = near_ties(ref["s"], host(bias), cfg.K)
    keep = np.setdiff1d(np.arange(T), ties)
    gi, ri = host(idx), ref["idx"]
    mism = np.nonzero((gi != ri).any(axis=1))[0]
    assert set(mism) <= set(ties), f"selection differs on non-tied tokens {sorted(set(mism) - set(ties))[:10]}"
    gerr = float(np.max(np.abs(host(gate)[keep] - ref["gates"][keep]))) if keep.size else 0.0
    # tokens with near-ties: the chosen keys are still within 1e-6 of a true top-K
    key64 = ref["s"] + host(bias).astype(np.float64)[None, :]
    kth = -np.sort(-key64, axis=1)[:, cfg.K - 1]
    chosen = np.take_along_axis(key64, gi.astype(np.int64), axis=1)
    assert (chosen >= kth[:, None] - 1e-6).all()
    report(f"route scratch {cfg.name} T={T}", aff_err=aerr, gate_err=gerr, near_tie_tokens=len(ties),
           differing=len(mism))
    assert aerr <= 1e-5
    assert gerr <= 1e-6
    return inp, idx


def test_route_from_scratch_tiny_f32():
    _from_scratch(W.config("tiny_f32"))


def test_route_from_scratch_ragged_and_small_N():
    _from_scratch(W.config("tiny_f32").scaled(T=67, N_r=13, K=3, H=200, seed=9), bias_scale=0.05)


def test_route_from_scratch_decode():
    _from_scratch(W.config("decode_bf16"))


def test_route_from_scratch_prefill():
    _from_scratch(W.config("prefill_bf16"), bias_scale=0.01)


@pytest.mark.parametrize("T", [100, 1100])
def test_route_from_scratch_largest_expert_count_and_top_k(T):
    # N_r = 1024 experts and K = 16 (the library's limits) at the V3 hidden size, on both logits
    # kernels (fragments from memory below 1024 tokens, LDS-staged tiles from 1024)
    _from_scratch(W.config("decode_bf16").scaled(T=T, N_r=1024, K=16, seed=T + 3), bias_scale=0.01)


@pytest.mark.parametrize("T,N_r,K", [(128, 256, 8), (37, 16, 2), (600, 1024, 16)])
def test_logits_with_in_register_split_equal_the_split_kernel(T, N_r, K):
    # below 1024 tokens the logits kernel splits 16-byte aligned fp32 centroids into their bf16 parts
    # in registers; centroids without that alignment go through the split kernel first. Both must
    # give the same affinities bit for bit.
    cfg = W.config("decode_bf16").scaled(T=T, N_r=N_r, K=K, seed=T + N_r)
    inp = W.make_inputs(cfg, device=DEV, with_weights=False)
    E = inp["centroids"]
    buf = torch.empty(E.numel() + 1, dtype=torch.float32, device=DEV)
    E_off = buf[1:].view(N_r, cfg.H)            # 4 bytes past a 256-byte boundary
    E_off.copy_(E)
    assert E.data_ptr() % 16 == 0 and E_off.data_ptr() % 16 == 4
    out = []
    for c in (E, E_off):
        aff = torch.empty((T, N_r), dtype=torch.float32, device=DEV)
        idx, gate = moe.moe_route(inp["u"], c, inp["bias"], K, affinity_out=aff)
        out.append((aff, idx, gate))
    torch.cuda.synchronize()
    assert np.array_equal(host(out[0][0]).view(np.uint32), host(out[1][0]).view(np.uint32))
    assert np.array_equal(host(out[0][1]), host(out[1][1]))
    assert np.array_equal(host(out[0][2]).view(np.uint32), host(out[1][2]).view(np.uint32))


def test_route_from_scratch_imbalance_hot_experts():
    inp, idx = _from_scratch(W.config("imbalance_bf16"))
    counts = np.bincount(host(idx).reshape(-1), minlength=256)
    assert counts[:8].min() > 4 * counts[8:].mean()          # +2.0 logits make experts 0-7 hot


# ------------------------------------------------------------------ group-limited (node-limited) routing
@pytest.mark.parametrize("T,N_r,K,G,M,levels", [
    (128, 256, 8, 8, 4, 0), (4096, 256, 8, 8, 4, 64), (64, 16, 2, 4, 2, 8), (33, 96, 6, 6, 3, 4),
    (50, 64, 16, 64, 16, 3), (16, 1024, 16, 64, 8, 16), (100, 256, 8, 8, 8, 0), (200, 60, 4, 3, 1, 5),
    (257, 256, 8, 16, 2, 0)])
def test_group_limited_selection_on_identical_affinities(T, N_r, K, G, M, levels):
    cfg = W.config("decode_bf16").scaled(T=T, N_r=N_r, K=K, seed=T * 11 + N_r + G)
    s = W.make_affinities(cfg, device=DEV, tie_levels=levels)
    g = torch.Generator(device=DEV).manual_seed(T + G)
    bias = ((torch.rand(N_r, generator=g, device=DEV) * 2 - 1) * 0.05).float()
    if levels:
        bias = torch.round(bias * levels) / levels
    idx, gate = moe.moe_route_group_limited(None, None, bias, K, G, M, affinity_in=s)
    torch.cuda.synchronize()
    ref = oracle.route(None, None, host(bias), K, affinity_in=host(s), n_groups=G, topk_groups=M)
    got = host(idx)
    assert np.array_equal(got, ref["idx"])
    assert all(len(set((row // (N_r // G)).tolist())) <= M for row in got)
    err = float(np.max(np.abs(host(gate) - ref["gates"])))
    report(f"group-limited identical T={T} N_r={N_r} K={K} G={G} M={M} ties={levels}", gate_err=err)
    assert err <= 1e-6
    if M == G:                                   # every group kept: plain top-K
        idx2, _ = moe.moe_route(None, None, bias, K, affinity_in=s)
        assert torch.equal(idx, idx2)


def test_group_limited_from_scratch_decode():
    # the whole router from u: selection is bit-exact against the oracle on the GPU's own fp32
    # affinities, and those are within 1e-5 of the float64 sigmoid
    cfg = W.config("decode_bf16")
    inp = W.make_inputs(cfg, device=DEV, with_weights=False)
    aff = torch.empty((cfg.T, cfg.N_r), dtype=torch.float32, device=DEV)
    idx, gate = moe.moe_route_group_limited(inp["u"], inp["centroids"], inp["bias"], cfg.K, 8, 4,
                                            affinity_out=aff)
    torch.cuda.synchronize()
    ref = oracle.route(None, None, host(inp["bias"]), cfg.K, affinity_in=host(aff), n_groups=8, topk_groups=4)
    assert np.array_equal(host(idx), ref["idx"])
    s64 = oracle.route(host(inp["u"]), host(inp["centroids"]), host(inp["bias"]), cfg.K)["s"]
    assert float(np.max(np.abs(f64(aff) - s64))) <= 1e-5
    assert float(np.max(np.abs(host(gate) - ref["gates"]))) <= 1e-6


# ------------------------------------------------------------------ sequence-wise balance loss
@pytest.mark.parametrize("T,N_r,K,seq_len,hot", [(4096, 256, 8, 4096, 0), (4096, 256, 8, 1000, 0),
                                                 (16384, 256, 8, 4096, 8), (37, 16, 2, 8, 0)])
def test_seq_balance_loss_against_oracle(T, N_r, K, seq_len, hot):
    # the formula is this library's reading (parity unpinned against the pages); the GPU value is
    # compared with the oracle's float64 value of the same reading on identical inputs
    cfg = W.config("imbalance_bf16").scaled(T=T, N_r=N_r, K=K, hot_experts=hot, seed=T + seq_len)
    s = W.make_affinities(cfg, device=DEV)
    idx, _ = moe.moe_route(None, None, torch.zeros(N_r, device=DEV), K, affinity_in=s)
    loss = moe.moe_seq_balance_loss(s, idx, seq_len, 1e-4)
    torch.cuda.synchronize()
    ref = oracle.seq_balance_loss(host(s), host(idx), K, seq_len, 1e-4)
    err = float(np.max(np.abs(host(loss) - ref) / np.abs(ref)))
    report(f"seq balance loss T={T} L={seq_len} hot={hot}", rel_err=err, loss=float(ref.mean()))
    assert err <= 1e-5
    if hot:
        assert (ref > 1e-4).all()          # hot experts make the loss exceed its uniform value alpha
