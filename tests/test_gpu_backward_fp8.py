"""FP8 backward of the grouped expert FFN and of the layer (HIP) against the oracle's FP8-emulating
backward (oracle.swiglu_ffn_backward_fp8 / layer_backward(fp8=True)).

Every GEMM operand is E4M3: activations and their gradients in 1x128 tiles along the reduction
dimension for the row GEMMs, in 128x1 tiles over each group's rows for the weight gradients,
weights in 128x128 blocks ("官方揭秘DeepSeek-V3模型训练全流程" §4.3, §4.5). Gate: relative
Frobenius error <= 3e-2 per gradient (per group for the weight gradients); the transposed weight
codes are bit-exact; groups without rows get exactly zero weight gradients.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_transformer_02_amd as moe
import workloads as W
from gpu_helpers import LazyExperts, f64, frob_rel, host, report
from sparse_moe_transformer_02_amd.layer import MoeLayer

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 3e-2


def _problem(counts, H, I, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    G = len(counts)
    total = int(sum(counts))
    x_rows = max(total, 1)
    X = torch.randn((x_rows, H), generator=g, device=DEV).bfloat16()
    Wg = (torch.randn((G, I, H), generator=g, device=DEV) / H ** 0.5).bfloat16()
    Wu = (torch.randn((G, I, H), generator=g, device=DEV) / H ** 0.5).bfloat16()
    Wd = (torch.randn((G, H, I), generator=g, device=DEV) / I ** 0.5).bfloat16()
    dY = torch.randn((total, H), generator=g, device=DEV).bfloat16()
    offsets = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=DEV)
    row_index = torch.randint(0, x_rows, (total,), generator=g, device=DEV, dtype=torch.int32)
    q = []
    for w in (Wg, Wu, Wd):
        G_, R, C = w.shape
        c, s = moe.fp8_quant_tiles(w.reshape(G_ * R, C), 128)
        q.append((c.view(G_, R, C), s.view(G_, R // 128, C // 128)))
    return X, (Wg, Wu, Wd), q, dY, offsets, row_index


def test_transposed_weight_codes_are_exact():
    counts = [3, 5]
    X, ws, q, dY, off, ri = _problem(counts, 384, 256, 1)
    (gc_, gs), (uc, us), (dc, ds) = q
    wdt, wdts, wgut, wguts = moe.moe_fp8_transpose_weights(gc_, gs, uc, us, dc, ds)
    torch.cuda.synchronize()
    assert torch.equal(wdt, dc.transpose(1, 2).contiguous())
    assert torch.equal(wdts, ds.transpose(1, 2).contiguous())
    assert torch.equal(wgut, torch.cat([gc_.transpose(1, 2), uc.transpose(1, 2)], dim=2).contiguous())
    assert torch.equal(wguts, torch.cat([gs.transpose(1, 2), us.transpose(1, 2)], dim=2).contiguous())


@pytest.mark.parametrize("counts,H,I", [
    ([0, 1, 17, 128, 129, 300], 256, 128),              # register-streamed row GEMMs, ragged 128x1 tiles
    ([1, 2, 0, 5, 16, 3, 40, 0, 7], 1024, 512),         # decode-sized groups: weight-streaming row GEMMs
    ([600, 3, 257, 0, 512, 256], 512, 256),             # LDS-tiled row GEMMs, several 128-row blocks per group
])
def test_grouped_ffn_backward_fp8(counts, H, I):
    X, ws, q, dY, off, ri = _problem(counts, H, I, 2)
    (gc_, gs), (uc, us), (dc, ds) = q
    wdt, wdts, wgut, wguts = moe.moe_fp8_transpose_weights(gc_, gs, uc, us, dc, ds)
    total = int(sum(counts))
    print(f"fp8 backward counts={counts} H={H} I={I}", flush=True)
    dX, dWg, dWu, dWd = moe.moe_grouped_ffn_backward_fp8(off, total, X, gc_, gs, uc, us, wdt, wdts, wgut, wguts, dY,
                                                         row_index=ri)
    torch.cuda.synchronize()
    o, rows, x64, dy64 = host(off), host(ri), f64(X), f64(dY)
    dX64 = f64(dX)
    worst = {"dX": 0.0, "dW_gate": 0.0, "dW_up": 0.0, "dW_down": 0.0}
    for gi in range(len(counts)):
        r0, r1 = o[gi], o[gi + 1]
        if r1 == r0:
            for t in (dWg, dWu, dWd):
                assert not t[gi].any(), "a group without rows must get zero weight gradients"
            continue
        ref = oracle.swiglu_ffn_backward_fp8(x64[rows[r0:r1]], *(host(w[gi]) for w in ws), dy64[r0:r1])
        worst["dX"] = max(worst["dX"], frob_rel(dX64[r0:r1], ref["dx"]))
        for key, t in (("dW_gate", dWg), ("dW_up", dWu), ("dW_down", dWd)):
            worst[key] = max(worst[key], frob_rel(f64(t[gi]), ref[key]))
    report(f"ffn backward fp8 {counts} H={H} I={I}", **{k + "_worst_group": v for k, v in worst.items()})
    assert all(v <= TOL for v in worst.values()), worst


def _layer(cfg):
    inp = W.make_inputs(cfg, device=DEV)
    layer = MoeLayer(inp["centroids"], inp["bias"].clone(), inp["w_gate"], inp["w_up"], inp["w_down"],
                     inp["sw_gate"], inp["sw_up"], inp["sw_down"], cfg.K, dtype="fp8",
                     logit_offset=inp["logit_offset"], gamma=cfg.gamma)
    return inp, layer


def _check_layer(cfg, workers=16):
    inp, layer = _layer(cfg)
    u = inp["u"]
    g = torch.Generator(device=DEV).manual_seed(cfg.seed + 77)
    dout = torch.randn((cfg.T, cfg.H), generator=g, device=DEV).bfloat16()
    print(f"fp8 layer backward {cfg.name} T={cfg.T}", flush=True)
    layer.forward(u)
    grads = layer.backward(dout)
    torch.cuda.synchronize()
    aff = host(layer.last["affinity"])
    b0 = host(layer.bias)
    idx = host(layer.last["idx"])
    want = sorted(set(idx.reshape(-1).tolist()))
    shared = [tuple(host(w[0]) for w in (inp["sw_gate"], inp["sw_up"], inp["sw_down"]))]
    ref = oracle.layer_backward(host(u), host(inp["centroids"]), b0, cfg.K,
                                LazyExperts(inp["w_gate"], inp["w_up"], inp["w_down"]), shared, f64(dout),
                                affinity_in=aff, fp8=True, weight_grads=want, workers=workers)
    assert np.array_equal(ref["idx"], idx)
    errs = {"du": frob_rel(f64(grads["du"]), ref["du"]),
            "dcentroids": frob_rel(f64(grads["dcentroids"]), ref["dcentroids"]),
            "dgate": frob_rel(f64(grads["dgate"]), ref["dgate"])}
    sh = ref["shared"][0]
    for j, key in enumerate(("dW_gate", "dW_up", "dW_down")):
        errs["shared_" + key] = frob_rel(f64(grads[key][0]), sh[j])
        errs["routed_" + key] = max(frob_rel(f64(grads[key][e + 1]), ref["routed"][e][j]) for e in want)
    report(f"layer backward fp8 {cfg.name} T={cfg.T}", experts_checked=len(want), **errs)
    assert all(v <= TOL for v in errs.values()), errs
    del layer, inp, grads
    gc.collect()
    torch.cuda.empty_cache()


def test_layer_backward_fp8_small():
    _check_layer(W.config("fp8").scaled(name="fp8_small", T=96, H=256, N_r=8, K=2, I=128, seed=21))


def test_layer_backward_fp8_decode_shape():
    """The FP8 layer at decode size (T = 128 at the V3 shape). The dgrad path is row-local (every
    quantization along H or I stays inside one token's row), so du and dgate of sampled tokens
    need each expert's FP8 backward on those tokens' rows only; weight gradients (128x1 tiles
    over all of an expert's rows) are checked for the shared expert and 4 routed experts."""
    from concurrent.futures import ThreadPoolExecutor
    cfg = W.config("fp8_decode")
    inp, layer = _layer(cfg)
    u = inp["u"]
    g = torch.Generator(device=DEV).manual_seed(cfg.seed + 77)
    dout = torch.randn((cfg.T, cfg.H), generator=g, device=DEV).bfloat16()
    print("fp8 layer backward at the decode shape: GPU", flush=True)
    layer.forward(u)
    grads = layer.backward(dout)
    torch.cuda.synchronize()
    aff = host(layer.last["affinity"])
    r = oracle.route(None, None, host(layer.bias), cfg.K, affinity_in=aff)
    idx, gates, s = r["idx"], r["gates"], r["s"]
    assert np.array_equal(idx, host(layer.last["idx"]))
    u64, d64 = f64(u), f64(dout)
    toks = np.sort(np.random.default_rng(cfg.seed).choice(cfg.T, 8, replace=False))
    experts = sorted(set(idx[toks].reshape(-1).tolist()))
    wgrad_experts = [int(e) for e in np.unique(idx)[::64][:4]]
    lazy = LazyExperts(inp["w_gate"], inp["w_up"], inp["w_down"])
    shared = tuple(host(w[0]) for w in (inp["sw_gate"], inp["sw_up"], inp["sw_down"]))

    def run(e):
        rows_all = np.nonzero((idx == e).any(axis=1))[0]           # tokens of expert e, ascending
        rt = rows_all if e in wgrad_experts else np.intersect1d(rows_all, toks)
        kk = np.array([int(np.nonzero(idx[t] == e)[0][0]) for t in rt])
        w = lazy[e]
        y = oracle.swiglu_ffn(oracle.fp8_roundtrip(u64[rt], 1, 128), *w, fp8=True)
        b = oracle.swiglu_ffn_backward_fp8(u64[rt], *w, gates[rt, kk][:, None] * d64[rt])
        print(f"  oracle expert {e}: {len(rt)} rows", flush=True)
        return e, rt, kk, y, b

    with ThreadPoolExecutor(max_workers=16) as ex:
        res = {e: out for e, *out in ex.map(run, sorted(set(experts) | set(wgrad_experts)))}
    sh = oracle.swiglu_ffn_backward_fp8(u64, *shared, d64)
    print("  oracle shared expert done", flush=True)
    du = d64[toks] + sh["dx"][toks]
    dgate = np.zeros((len(toks), cfg.K))
    pos = {t: i for i, t in enumerate(toks)}
    for e, (rt, kk, y, b) in res.items():
        for j, t in enumerate(rt):
            if t in pos:
                du[pos[t]] += b["dx"][j]
                dgate[pos[t], kk[j]] = d64[t] @ y[j]
    sel = np.take_along_axis(s[toks], idx[toks].astype(np.int64), axis=1)
    gt = gates[toks]
    dlogit = (dgate - (gt * dgate).sum(1, keepdims=True)) / sel.sum(1, keepdims=True) * sel * (1 - sel)
    du += np.einsum("tk,tkh->th", dlogit, f64(inp["centroids"])[idx[toks]])
    errs = {"du": frob_rel(f64(grads["du"])[toks], du), "dgate": frob_rel(f64(grads["dgate"])[toks], dgate)}
    for j, key in enumerate(("dW_gate", "dW_up", "dW_down")):
        errs["shared_" + key] = frob_rel(f64(grads[key][0]), sh[key])
        errs["routed_" + key] = max(frob_rel(f64(grads[key][e + 1]), res[e][3][key]) for e in wgrad_experts)
    report("layer backward fp8 fp8_decode T=128", sampled_tokens=len(toks), wgrad_experts=len(wgrad_experts), **errs)
    assert all(v <= TOL for v in errs.values()), errs
    del layer, inp, grads
    gc.collect()
    torch.cuda.empty_cache()
