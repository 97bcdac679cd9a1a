"""Layer backward (HIP) against the oracle's chain-rule backward (itself pinned by finite differences).

Tolerances: max|gpu - ref| <= 1e-2 max|ref| per gradient tensor (bf16 operands, fp32
accumulation: h, dy, dz and dv are rounded to bf16 on the GPU); combine backward's dY rows
bit-exact (one fp32 product rounded to bf16); gradients bitwise reproducible run to run.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import LazyExperts, f64, host, max_rel, report
import sparse_moe_transformer_02_amd as moe
from sparse_moe_transformer_02_amd.layer import MoeLayer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ffn_problem(counts, H, I, seed, gather=True):
    g = torch.Generator(device=DEV).manual_seed(seed)
    G, total = len(counts), int(sum(counts))
    x_rows = max(total, 1)
    X = torch.randn((x_rows, H), generator=g, device=DEV).bfloat16()
    Wg = (torch.randn((G, I, H), generator=g, device=DEV) / H ** 0.5).bfloat16()
    Wu = (torch.randn((G, I, H), generator=g, device=DEV) / H ** 0.5).bfloat16()
    Wd = (torch.randn((G, H, I), generator=g, device=DEV) / I ** 0.5).bfloat16()
    dY = torch.randn((max(total, 1), H), generator=g, device=DEV).bfloat16()
    off = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=DEV)
    ri = torch.randint(0, x_rows, (max(total, 1),), generator=g, device=DEV, dtype=torch.int32) if gather else None
    return X, Wg, Wu, Wd, dY, off, ri


@pytest.mark.parametrize("counts,gather,H,I", [
    ([0, 1, 17, 130, 5, 0, 256, 300], True, 256, 128),
    ([150], False, 384, 256),
    ([3, 0, 64, 129], True, 128, 384),
    # H % 512 == 0 and I % 512 == 0: weight gradients through transposed, 64-padded operands
    ([0, 1, 17, 130, 64, 0, 300, 65], True, 1024, 512),
    ([150], False, 512, 512),
    ([0, 0, 1], True, 512, 1024),
])
def test_grouped_ffn_backward(counts, gather, H, I):
    X, Wg, Wu, Wd, dY, off, ri = _ffn_problem(counts, H, I, sum(counts) + H, gather)
    total = int(sum(counts))
    dX, dWg, dWu, dWd = moe.moe_grouped_ffn_backward(off, total, X, Wg, Wu, Wd, dY, row_index=ri)
    torch.cuda.synchronize()
    o = host(off)
    rows = host(ri) if ri is not None else np.arange(total)
    x64, dy64 = f64(X), f64(dY)
    errs = {"dX": 0.0, "dW_gate": 0.0, "dW_up": 0.0, "dW_down": 0.0}
    gdX = f64(dX)
    for gi in range(len(counts)):
        r0, r1 = o[gi], o[gi + 1]
        got = (f64(dWg[gi]), f64(dWu[gi]), f64(dWd[gi]))
        if r1 == r0:
            assert all(np.all(a == 0) for a in got)
            continue
        ref = oracle.swiglu_ffn_backward(x64[rows[r0:r1]], f64(Wg[gi]), f64(Wu[gi]), f64(Wd[gi]), dy64[r0:r1])
        errs["dX"] = max(errs["dX"], max_rel(gdX[r0:r1], ref["dx"]))
        for name, a in zip(("dW_gate", "dW_up", "dW_down"), got):
            errs[name] = max(errs[name], max_rel(a, ref[name]))
    report(f"ffn backward {counts} H={H} I={I}", **errs)
    assert max(errs.values()) <= 1e-2


@pytest.mark.parametrize("counts,gather,H,I", [
    ([0, 1, 17, 130, 5, 0, 256, 300], True, 256, 128),   # recompute on the register-transposing kernel
    ([0, 1, 17, 130, 64, 0, 300, 65], True, 1024, 512),  # recompute on the LDS-tiled kernel
    ([1, 3, 0, 2], True, 512, 512),                       # decode-sized groups: saved by the register-streamed forward
])
def test_grouped_ffn_backward_from_saved_preactivations_is_bitwise_the_same(counts, gather, H, I):
    X, Wg, Wu, Wd, dY, off, ri = _ffn_problem(counts, H, I, sum(counts) + 7, gather)
    total = int(sum(counts))
    zv = torch.empty((total, 2 * I), device=DEV)
    moe.moe_grouped_ffn(off, total, X, Wg, Wu, Wd, row_index=ri, preact=zv)
    a = moe.moe_grouped_ffn_backward(off, total, X, Wg, Wu, Wd, dY, row_index=ri)
    b = moe.moe_grouped_ffn_backward(off, total, X, Wg, Wu, Wd, dY, row_index=ri, preact=zv)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_layer_backward_with_kept_preactivations_is_bitwise_the_same():
    cfg = _bf16_tiny(T=37, seed=24)
    inp, layer = _layer(cfg)
    g = torch.Generator(device=DEV).manual_seed(6)
    dout = torch.randn((cfg.T, cfg.H), generator=g, device=DEV).bfloat16()
    out0 = layer.forward(inp["u"]).clone()
    g0 = {k: v.clone() for k, v in layer.backward(dout).items()}
    out1 = layer.forward(inp["u"], keep_preact=True).clone()
    g1 = layer.backward(dout)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1)
    assert all(torch.equal(g0[k], g1[k]) for k in g0)


def test_grouped_ffn_backward_no_rows_gives_zero_weight_grads():
    X, Wg, Wu, Wd, dY, off, ri = _ffn_problem([0, 0, 0], 128, 128, 1)
    dX, dWg, dWu, dWd = moe.moe_grouped_ffn_backward(off, 0, X, Wg, Wu, Wd, dY, row_index=ri)
    torch.cuda.synchronize()
    assert all(float(t.abs().max()) == 0.0 for t in (dWg, dWu, dWd))


def _bf16_tiny(T=64, seed=21, **kw):
    return W.config("tiny_f32").scaled(dtype="bf16", I=128, T=T, seed=seed, **kw)


def _layer(cfg, **kw):
    inp = W.make_inputs(cfg, device=DEV)
    layer = MoeLayer(inp["centroids"], inp["bias"].clone(), inp["w_gate"], inp["w_up"], inp["w_down"],
                     inp["sw_gate"], inp["sw_up"], inp["sw_down"], cfg.K, dtype=cfg.dtype,
                     logit_offset=inp["logit_offset"], gamma=cfg.gamma, **kw)
    return inp, layer


def test_combine_backward_rows_bit_exact():
    cfg = _bf16_tiny()
    inp, layer = _layer(cfg)
    layer.forward(inp["u"])
    g = torch.Generator(device=DEV).manual_seed(3)
    dout = torch.randn((cfg.T, cfg.H), generator=g, device=DEV).bfloat16()
    b = layer.last
    dY, dgate = moe.moe_combine_backward(dout, b["y"], b["slot_row"], b["gate"], cfg.K, shared_rows=cfg.T)
    torch.cuda.synchronize()
    sr = host(b["slot_row"]).reshape(cfg.T, cfg.K)
    d32 = dout.float().cpu().numpy()
    g32 = host(b["gate"])
    want = torch.from_numpy((g32[:, :, None] * d32[:, None, :]).astype(np.float32)).bfloat16()
    got = dY.cpu()
    assert torch.equal(got[:cfg.T], dout.cpu())                         # shared rows: dout itself
    assert torch.equal(got[torch.from_numpy(sr.reshape(-1)).long()], want.reshape(-1, cfg.H))
    y = f64(b["y"])
    ref = np.einsum("th,tkh->tk", f64(dout), y[sr])
    assert np.max(np.abs(host(dgate) - ref)) <= 1e-5 * np.max(np.abs(ref))


def _check_layer_backward(cfg, layer, inp, dout, experts_to_check, label):
    grads = layer.backward(dout)
    torch.cuda.synchronize()
    aff = host(layer.last_affinity)
    shared = [tuple(host(w[0]) for w in (inp["sw_gate"], inp["sw_up"], inp["sw_down"]))]
    ref = oracle.layer_backward(host(inp["u"]), host(inp["centroids"]), host(layer.bias), cfg.K,
                                LazyExperts(inp["w_gate"], inp["w_up"], inp["w_down"]), shared, host(dout),
                                affinity_in=aff, workers=16, weight_grads=experts_to_check,
                                n_groups=layer.groups[0], topk_groups=layer.groups[1])
    assert np.array_equal(host(layer.last["idx"]), ref["idx"])
    errs = {"du": max_rel(f64(grads["du"]), ref["du"]),
            "dcentroids": max_rel(f64(grads["dcentroids"]), ref["dcentroids"]),
            "dgate": max_rel(f64(grads["dgate"]), ref["dgate"])}
    for j, name in enumerate(("dW_gate", "dW_up", "dW_down")):
        e = max_rel(f64(grads[name][0]), ref["shared"][0][j])
        for ex in experts_to_check:
            if ex in ref["routed"]:
                e = max(e, max_rel(f64(grads[name][ex + 1]), ref["routed"][ex][j]))
            else:
                assert float(grads[name][ex + 1].abs().max()) == 0.0
        errs[name] = e
    report(label, **errs)
    assert max(errs.values()) <= 1e-2
    return grads


def test_layer_backward_tiny_bf16():
    cfg = _bf16_tiny()
    inp, layer = _layer(cfg)
    layer.forward(inp["u"])
    g = torch.Generator(device=DEV).manual_seed(5)
    dout = torch.randn((cfg.T, cfg.H), generator=g, device=DEV).bfloat16()
    grads = _check_layer_backward(cfg, layer, inp, dout, list(range(cfg.N_r)), "layer backward tiny bf16")
    again = layer.backward(dout)
    torch.cuda.synchronize()
    assert all(torch.equal(grads[k], again[k]) for k in grads)        # bitwise reproducible


def test_layer_backward_group_limited_ragged():
    cfg = _bf16_tiny(T=37, seed=22, N_r=16, K=4)
    inp, layer = _layer(cfg, n_groups=4, topk_groups=2)
    layer.forward(inp["u"])
    dout = torch.randn((cfg.T, cfg.H), device=DEV).bfloat16()
    _check_layer_backward(cfg, layer, inp, dout, list(range(cfg.N_r)), "layer backward group-limited T=37")


def test_layer_backward_decode_shape():
    # At the V3 decode shape the oracle evaluates a sample: du and dgate of 6 seeded tokens (a
    # token's input gradient depends only on its own experts), and the weight gradients of the
    # shared expert, the busiest routed expert and an unused one (all of their rows)
    cfg = W.config("decode_bf16")
    inp, layer = _layer(cfg)
    layer.forward(inp["u"])
    g = torch.Generator(device=DEV).manual_seed(7)
    dout = torch.randn((cfg.T, cfg.H), generator=g, device=DEV).bfloat16()
    grads = layer.backward(dout)
    torch.cuda.synchronize()
    aff = host(layer.last_affinity)
    u64, d64 = f64(inp["u"]), f64(dout)
    toks = np.sort(np.random.default_rng(cfg.seed).choice(cfg.T, 6, replace=False))
    shared = [tuple(host(w[0]) for w in (inp["sw_gate"], inp["sw_up"], inp["sw_down"]))]
    experts = LazyExperts(inp["w_gate"], inp["w_up"], inp["w_down"])
    ref = oracle.layer_backward(u64[toks], host(inp["centroids"]), host(layer.bias), cfg.K, experts, shared,
                                d64[toks], affinity_in=aff[toks], workers=16, weight_grads=False)
    errs = {"du_sampled": max_rel(f64(grads["du"])[toks], ref["du"]),
            "dgate_sampled": max_rel(f64(grads["dgate"])[toks], ref["dgate"])}
    r = oracle.route(None, None, host(layer.bias), cfg.K, affinity_in=aff)
    assert np.array_equal(host(layer.last["idx"]), r["idx"])
    b = oracle.swiglu_ffn_backward(u64, *shared[0], d64)
    errs["shared_dW"] = max(max_rel(f64(grads[n][0]), b[n]) for n in ("dW_gate", "dW_up", "dW_down"))
    counts = np.bincount(r["idx"].reshape(-1), minlength=cfg.N_r)
    e = int(np.argmax(counts))
    rt, rk = np.nonzero(r["idx"] == e)
    b = oracle.swiglu_ffn_backward(u64[rt], *experts[e], r["gates"][rt, rk][:, None] * d64[rt])
    errs[f"expert{e}_dW"] = max(max_rel(f64(grads[n][e + 1]), b[n]) for n in ("dW_gate", "dW_up", "dW_down"))
    for z in np.nonzero(counts == 0)[0][:1]:
        assert all(float(grads[n][int(z) + 1].abs().max()) == 0.0 for n in ("dW_gate", "dW_up", "dW_down"))
    report("layer backward decode_bf16 (sampled)", rows_of_busiest=int(counts[e]), **errs)
    assert max(errs.values()) <= 1e-2
    del layer, inp, grads
    gc.collect()
    torch.cuda.empty_cache()


def _misaligned(t):
    """The same values in storage that starts 2 bytes past a 16-byte boundary (forces the per-element
    kernel paths, which need no alignment)."""
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    out = flat[1:1 + t.numel()].view(t.shape)
    out.copy_(t)
    return out


def test_combine_and_router_backward_vector_and_scalar_paths_agree():
    # the 16-byte vector paths (H % 8 == 0, aligned rows) and the per-element paths on the same inputs:
    # dY rows and du bit for bit (same per-element arithmetic), dgate within fp32 reordering
    cfg = _bf16_tiny(T=37, seed=23)
    inp, layer = _layer(cfg)
    layer.forward(inp["u"])
    g = torch.Generator(device=DEV).manual_seed(9)
    dout = torch.randn((cfg.T, cfg.H), generator=g, device=DEV).bfloat16()
    b, u, T = layer.last, layer.last_u, cfg.T
    res = []
    for mis in (False, True):
        f = _misaligned if mis else (lambda t: t)
        dY, dgate = moe.moe_combine_backward(f(dout), f(b["y"]), b["slot_row"], b["gate"], cfg.K, shared_rows=T,
                                             dY=f(torch.empty((b["y"].shape[0], cfg.H), dtype=torch.bfloat16,
                                                              device=DEV)))
        dX = torch.randn((b["y"].shape[0], cfg.H), generator=torch.Generator(device=DEV).manual_seed(4), device=DEV)
        du, dE = moe.moe_router_backward(f(dout), f(u), f(dX), b["offsets"], b["row_token"], b["slot_row"],
                                         layer.last_affinity, b["idx"], b["gate"], dgate, f(layer.centroids),
                                         shared_rows=T, du=f(torch.empty((T, cfg.H), dtype=torch.float32, device=DEV)))
        torch.cuda.synchronize()
        res.append((dY.clone(), dgate.clone(), du.clone(), dE.clone()))
    (dY0, g0, du0, dE0), (dY1, g1, du1, dE1) = res
    assert torch.equal(dY0, dY1)
    assert float((g0 - g1).abs().max()) <= 1e-6 * float(g0.abs().max())
    # du depends on dgate through dlogit: compare with the aligned path's dgate fed to both
    du_again, dE_again = moe.moe_router_backward(
        _misaligned(dout), _misaligned(u), _misaligned(dX), b["offsets"], b["row_token"], b["slot_row"],
        layer.last_affinity, b["idx"], b["gate"], g0, _misaligned(layer.centroids), shared_rows=T,
        du=_misaligned(torch.empty((T, cfg.H), dtype=torch.float32, device=DEV)))
    torch.cuda.synchronize()
    assert torch.equal(du0, du_again)
    assert torch.equal(dE0, dE_again)                 # same dlogit: the per-element path is bit for bit
    assert float((dE0 - dE1).abs().max()) <= 1e-5 * float(dE0.abs().max())
