"""The whole layer on the GPU (MoeLayer over the C ABI) against the oracle, per workload.

Routing and dispatch are compared on every token; layer outputs on every token for the
tiny workload and on a seeded token sample at the V3 shapes (the float64 oracle
evaluates one expert at a time). Tolerances: max|gpu - ref| <= 1e-2 max|ref| for
fp32/bf16 outputs, relative Frobenius error <= 3e-2 for FP8 (against the
FP8-emulating oracle); bias updates and dispatch bit-exact.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import LazyExperts, f64, frob_rel, host, max_rel, near_ties, report
from layouts import dispatch_with_shared
from sparse_moe_transformer_02_amd.layer import MoeLayer

pytestmark = pytest.mark.gpu
DEV = "cuda"
WORKERS = 16


def _build(cfg):
    inp = W.make_inputs(cfg, device=DEV)
    layer = MoeLayer(inp["centroids"], inp["bias"].clone(), inp["w_gate"], inp["w_up"], inp["w_down"],
                     inp["sw_gate"], inp["sw_up"], inp["sw_down"], cfg.K, dtype=cfg.dtype,
                     logit_offset=inp["logit_offset"], gamma=cfg.gamma)
    return inp, layer


def _oracle(cfg, inp, u, bias, tokens=None):
    shared = [tuple(host(w[0]) for w in (inp["sw_gate"], inp["sw_up"], inp["sw_down"]))]
    off = None if inp["logit_offset"] is None else host(inp["logit_offset"])
    return oracle.layer_forward(host(u), host(inp["centroids"]), bias, cfg.K,
                                LazyExperts(inp["w_gate"], inp["w_up"], inp["w_down"]), shared,
                                fp8=cfg.dtype == "fp8", logit_offset=off, tokens=tokens, workers=WORKERS)


def _compare(cfg, layer, ref, bias, label, n_sample=None, must_include=()):
    """Checks routing/dispatch on all tokens and the output on ref['tokens']."""
    b = layer.last
    T = b["idx"].shape[0]
    aerr = float(np.max(np.abs(f64(b["affinity"]) - ref["s"])))
    ties = near_ties(ref["s"], bias, cfg.K)
    mism = np.nonzero((host(b["idx"]) != ref["idx"]).any(axis=1))[0]
    assert set(mism) <= set(ties)
    keep = np.setdiff1d(np.arange(T), ties)
    gerr = float(np.max(np.abs(host(b["gate"])[keep] - ref["gates"][keep])))
    # dispatch bit-exact against the oracle run on the GPU's own selection (so near-ties do not
    # matter); the layer dispatches the shared expert as group 0 (T identity rows) first
    d = dispatch_with_shared(host(b["idx"]), cfg.N_r, T)
    for name in ("counts", "offsets", "row_token", "slot_row"):
        assert np.array_equal(host(b[name]), d[name]), name
    toks = ref["tokens"]
    out = f64(b["out"])[toks]
    ysh_gpu = f64(b["y_shared"])[toks]
    if cfg.dtype == "fp8":
        err, ysh = frob_rel(out, ref["out"]), frob_rel(ysh_gpu, ref["y_shared"])
    else:
        err, ysh = max_rel(out, ref["out"]), max_rel(ysh_gpu, ref["y_shared"])
    report(label, aff_err=aerr, gate_err=gerr, near_tie_tokens=len(ties), out_err=err, shared_err=ysh,
           sampled=len(toks))
    assert aerr <= 1e-5 and gerr <= 1e-6
    tol = 3e-2 if cfg.dtype == "fp8" else 1e-2
    assert err <= tol and ysh <= tol
    return mism


def _sample(T, n, seed, avoid=(), must=()):
    rng = np.random.default_rng(seed)
    pool = np.setdiff1d(np.arange(T), np.asarray(avoid, dtype=np.int64))
    pick = rng.choice(pool, size=min(n, pool.size), replace=False)
    return np.unique(np.concatenate([pick, np.asarray(must, dtype=np.int64)])).astype(np.int64)


def test_tiny_forward_update_forward():
    cfg = W.config("tiny_f32")
    inp, layer = _build(cfg)
    u = inp["u"]
    b0 = host(layer.bias).copy()
    layer.forward(u)
    torch.cuda.synchronize()
    ref = _oracle(cfg, inp, u, b0)
    _compare(cfg, layer, ref, b0, "layer tiny_f32 forward 1")
    # routed rows one by one: Y[slot_row[t*K+k]] is FFN_{idx[t,k]}(u_t)
    Y = f64(layer.last["y"])[host(layer.last["slot_row"])].reshape(cfg.T, cfg.K, cfg.H)
    assert max_rel(Y, ref["y_routed"]) <= 1e-5
    layer.update_bias(cfg.T)
    b1 = oracle.bias_update(b0, ref["counts"], cfg.T, cfg.K, cfg.gamma)
    assert np.array_equal(host(layer.bias).view(np.uint32), b1.view(np.uint32))
    assert not np.array_equal(b1, b0)
    layer.forward(u)
    torch.cuda.synchronize()
    ref2 = _oracle(cfg, inp, u, b1)
    _compare(cfg, layer, ref2, b1, "layer tiny_f32 forward 2 (updated bias)")


def test_tiny_ragged_and_degenerate():
    # T not a multiple of any tile, K = N_r (every expert), and a single token
    for cfg in (W.config("tiny_f32").scaled(T=37, N_r=8, K=8, seed=11),
                W.config("tiny_f32").scaled(T=1, seed=12)):
        inp, layer = _build(cfg)
        layer.forward(inp["u"])
        torch.cuda.synchronize()
        ref = _oracle(cfg, inp, inp["u"], host(inp["bias"]))
        _compare(cfg, layer, ref, host(inp["bias"]), f"layer {cfg.name} T={cfg.T} K={cfg.K}")


@pytest.mark.parametrize("name", ["decode_bf16", "fp8_decode"])
def test_v3_shape_single_token_then_a_few(name):
    # the V3 layer shape with one token (8 experts with one row, 248 experts with none: only the
    # selected experts' weights are streamed), its bias update, then three tokens on the same layer
    cfg = W.config(name).scaled(T=1, seed=W.config(name).seed + 50)
    inp, layer = _build(cfg)
    u = inp["u"]
    b0 = host(layer.bias).copy()
    print(f"layer {name}: forward T=1", flush=True)
    layer.forward(u)
    torch.cuda.synchronize()
    ref = _oracle(cfg, inp, u, b0)
    _compare(cfg, layer, ref, b0, f"layer {name} T=1")
    assert int(np.count_nonzero(host(layer.last["counts"]))) == cfg.K
    layer.update_bias(1)
    b1 = oracle.bias_update(b0, ref["counts"], 1, cfg.K, cfg.gamma)
    assert np.array_equal(host(layer.bias).view(np.uint32), b1.view(np.uint32))
    cfg3 = cfg.scaled(T=3)
    g = torch.Generator(device=DEV).manual_seed(cfg.seed + 1)
    u3 = torch.randn((3, cfg.H), generator=g, device=DEV).to(u.dtype)
    print(f"layer {name}: forward T=3", flush=True)
    layer.forward(u3)
    torch.cuda.synchronize()
    ref3 = _oracle(cfg3, inp, u3, b1)
    _compare(cfg3, layer, ref3, b1, f"layer {name} T=3 after the bias update")
    del layer, inp
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,G,M,n_sample", [("tiny_f32", 4, 2, None), ("decode_bf16", 8, 4, 12)])
def test_group_limited_layer(name, G, M, n_sample):
    # node-limited routing inside the layer: selection bit-exact against the oracle on the GPU's own
    # fp32 affinities, every token within M groups, outputs within the dtype's tolerance
    cfg = W.config(name)
    inp = W.make_inputs(cfg, device=DEV)
    layer = MoeLayer(inp["centroids"], inp["bias"].clone(), inp["w_gate"], inp["w_up"], inp["w_down"],
                     inp["sw_gate"], inp["sw_up"], inp["sw_down"], cfg.K, dtype=cfg.dtype,
                     logit_offset=inp["logit_offset"], gamma=cfg.gamma, n_groups=G, topk_groups=M)
    u = inp["u"]
    b0 = host(layer.bias).copy()
    layer.forward(u)
    torch.cuda.synchronize()
    aff = host(layer.last["affinity"])
    toks = None if n_sample is None else _sample(cfg.T, n_sample, cfg.seed + 1)
    shared = [tuple(host(w[0]) for w in (inp["sw_gate"], inp["sw_up"], inp["sw_down"]))]
    ref = oracle.layer_forward(host(u), None, b0, cfg.K, LazyExperts(inp["w_gate"], inp["w_up"], inp["w_down"]),
                               shared, affinity_in=aff, tokens=toks, workers=WORKERS, n_groups=G, topk_groups=M)
    idx = host(layer.last["idx"])
    assert np.array_equal(idx, ref["idx"])
    assert all(len(set((row // (cfg.N_r // G)).tolist())) <= M for row in idx)
    d = dispatch_with_shared(ref["idx"], cfg.N_r, cfg.T)
    for key in ("counts", "offsets", "row_token", "slot_row"):
        assert np.array_equal(host(layer.last[key]), d[key]), key
    out = f64(layer.last["out"])[ref["tokens"]]
    err = max_rel(out, ref["out"])
    report(f"layer {name} group-limited G={G} M={M}", out_err=err, sampled=len(ref["tokens"]))
    assert err <= 1e-2
    layer.update_bias(cfg.T)
    b1 = oracle.bias_update(b0, ref["counts"], cfg.T, cfg.K, cfg.gamma)
    assert np.array_equal(host(layer.bias).view(np.uint32), b1.view(np.uint32))
    del layer, inp
    gc.collect()
    torch.cuda.empty_cache()


def _outlier_tokens(u, n):
    """The n tokens holding the largest activation magnitudes (the outliers of the FP8 workload)."""
    peak = np.abs(f64(u)).max(axis=1)
    return np.argsort(-peak, kind="stable")[:n]


def _full_size(name, n_sample, extra_checks=None, n_outlier_tokens=0):
    cfg = W.config(name)
    inp, layer = _build(cfg)
    u = inp["u"]
    b0 = host(layer.bias).copy()
    print(f"layer {name}: forward T={cfg.T}", flush=True)
    layer.forward(u)
    torch.cuda.synchronize()
    route = oracle.route(host(u), host(inp["centroids"]), b0, cfg.K,
                         logit_offset=None if inp["logit_offset"] is None else host(inp["logit_offset"]))
    ties = near_ties(route["s"], b0, cfg.K)
    must = _outlier_tokens(u, n_outlier_tokens) if n_outlier_tokens else []
    toks = _sample(cfg.T, n_sample, cfg.seed, avoid=ties, must=must)
    ref = _oracle(cfg, inp, u, b0, tokens=toks)
    _compare(cfg, layer, ref, b0, f"layer {name}")
    if extra_checks:
        extra_checks(cfg, inp, layer, ref)
    del layer, inp
    gc.collect()
    torch.cuda.empty_cache()


def test_decode_layer():
    _full_size("decode_bf16", 64)


def test_prefill_layer():
    _full_size("prefill_bf16", 64)


def test_fp8_layer():
    def codes(cfg, inp, layer, ref):
        b = layer.last
        rc, rs = oracle.quantize_tiles(f64(inp["u"]).astype(np.float32), 1, 128)
        assert np.array_equal(host(b["u_codes"]), rc)
        assert np.array_equal(host(b["u_scales"]), rs)
        for j, w in enumerate((inp["w_gate"], inp["w_up"], inp["w_down"])):
            for e in (0, 131, 255):      # the layer's weight tensors hold the shared expert at index 0
                c, s = oracle.quantize_tiles(f64(w[e]).astype(np.float32), 128, 128)
                assert np.array_equal(host(layer.w[j][0][e + 1]), c)
                assert np.array_equal(host(layer.w[j][1][e + 1]), s)
            c, s = oracle.quantize_tiles(f64(inp[("sw_gate", "sw_up", "sw_down")[j]][0]).astype(np.float32), 128, 128)
            assert np.array_equal(host(layer.w[j][0][0]), c)
    # 8 seeded tokens plus the 32 tokens holding the largest outlier magnitudes
    _full_size("fp8", 8, codes, n_outlier_tokens=32)


def test_fp8_decode_layer():
    # the FP8 layer at decode size runs the weight-streaming FP8 kernels
    _full_size("fp8_decode", 8)


def test_imbalance_steps_from_scratch():
    """Three training steps at T=16384 with hot experts 0-7: routing, outputs, counts, bias update.

    Each step starts both sides from the oracle's bias. Tokens whose top-(K+1) keys lie within
    1e-6 may legitimately pick differently (fp32 vs float64 affinities); the count differences
    must be exactly those flips, and every expert's new bias must follow the sign rule for the
    side's own count (bit-exact against the oracle where the counts agree).
    """
    cfg = W.config("imbalance_bf16")
    inp, layer = _build(cfg)
    b = host(layer.bias).copy()
    g = np.float32(cfg.gamma)
    for step in range(3):
        layer.bias.copy_(torch.from_numpy(b))
        u = W.make_tokens(cfg, step, device=DEV)
        layer.step(u)
        torch.cuda.synchronize()
        route = oracle.route(host(u), host(inp["centroids"]), b, cfg.K, logit_offset=host(inp["logit_offset"]))
        toks = _sample(cfg.T, 8, step, avoid=near_ties(route["s"], b, cfg.K))
        ref = _oracle(cfg, inp, u, b, tokens=toks)
        mism = _compare(cfg, layer, ref, b, f"layer imbalance step {step}")
        gi = host(layer.last["idx"])
        delta = np.zeros(cfg.N_r, np.int64)
        for t in mism:
            np.add.at(delta, gi[t], 1)
            np.add.at(delta, ref["idx"][t], -1)
        c_gpu = host(layer.last["counts"]).astype(np.int64)
        assert np.array_equal(c_gpu - ref["counts"], delta)
        b_ref = oracle.bias_update(b, ref["counts"], cfg.T, cfg.K, cfg.gamma)
        b_gpu = host(layer.bias)
        same = delta == 0
        assert np.array_equal(b_gpu[same].view(np.uint32), b_ref[same].view(np.uint32))
        load = cfg.N_r * c_gpu - cfg.T * cfg.K
        expect = np.where(load > 0, b - g, np.where(load < 0, b + g, b)).astype(np.float32)
        assert np.array_equal(b_gpu[~same].view(np.uint32), expect[~same].view(np.uint32))
        stats = oracle.load_stats(ref["counts"], cfg.T, cfg.K)
        report(f"imbalance step {step}", max_over_mean=stats["max_over_mean"], flipped_tokens=len(mism),
               experts_with_other_count=int((~same).sum()))
        b = b_ref
    del layer, inp
    gc.collect()
    torch.cuda.empty_cache()


def _hot_sample(idx, hot, per, seed, n_random):
    """Tokens such that each of the experts 0..hot-1 is selected by at least `per` of them
    (as far as the batch allows), plus n_random seeded tokens."""
    rng = np.random.default_rng(seed)
    need = np.full(hot, per)
    chosen = []
    for t in rng.permutation(idx.shape[0]):
        hits = [int(e) for e in idx[t] if e < hot and need[e] > 0]
        if hits:
            chosen.append(int(t))
            need[hits] -= 1
        if not need.any():
            break
    return _sample(idx.shape[0], n_random, seed + 1, must=chosen)


@pytest.mark.timeout(900)
def test_imbalance_100_steps():
    """The load-imbalance workload as configured: 100 forward + bias-update steps at T = 16384 with
    a fresh u every step and experts 0-7 hot (+2.0 on their logits), the bias carried on the GPU.

    Every step, the oracle routes on the GPU's own fp32 affinities (identical keys, so no tie is
    excluded): expert indices, gates, counts, offsets, the permutation and the updated fp32 bias
    must match it bit for bit (gates within 1e-6). The max/mean expert load is logged per step.
    On steps 0, 49 and 99 the affinities are also checked against the float64 sigmoid, and the
    layer output against the oracle on at least 8 tokens per hot expert plus 8 seeded tokens.
    """
    cfg = W.config("imbalance_bf16")
    inp, layer = _build(cfg)
    b = host(layer.bias).copy()
    E, off = host(inp["centroids"]), host(inp["logit_offset"])
    shared = [tuple(host(w[0]) for w in (inp["sw_gate"], inp["sw_up"], inp["sw_down"]))]
    loads = []
    for step in range(cfg.steps):
        print(f"imbalance step {step}: layer step on the GPU", flush=True)
        u = W.make_tokens(cfg, step, device=DEV)
        layer.step(u)
        torch.cuda.synchronize()
        last = layer.last
        aff = host(last["affinity"])
        ref = oracle.route(None, None, b, cfg.K, affinity_in=aff)
        idx = host(last["idx"])
        assert np.array_equal(idx, ref["idx"]), f"step {step}: selection"
        gerr = float(np.max(np.abs(host(last["gate"]) - ref["gates"])))
        assert gerr <= 1e-6, f"step {step}: gates {gerr}"
        d = dispatch_with_shared(ref["idx"], cfg.N_r, cfg.T)
        for name in ("counts", "offsets", "row_token", "slot_row"):
            assert np.array_equal(host(last[name]), d[name]), f"step {step}: {name}"
        b_next = oracle.bias_update(b, d["counts"], cfg.T, cfg.K, cfg.gamma)
        assert np.array_equal(host(layer.bias).view(np.uint32), b_next.view(np.uint32)), f"step {step}: bias"
        loads.append(oracle.load_stats(d["counts"], cfg.T, cfg.K)["max_over_mean"])
        if step in (0, 49, 99):
            toks = _hot_sample(idx, cfg.hot_experts, 8, 100 + step, 8)
            s64 = oracle.affinities(host(u)[toks], E, off)
            aerr = float(np.max(np.abs(aff[toks].astype(np.float64) - s64)))
            out_ref = oracle.layer_forward(host(u), None, b, cfg.K,
                                           LazyExperts(inp["w_gate"], inp["w_up"], inp["w_down"]), shared,
                                           affinity_in=aff, tokens=toks, workers=WORKERS)
            err = max_rel(f64(last["out"])[toks], out_ref["out"])
            ysh = max_rel(f64(last["y_shared"])[toks], out_ref["y_shared"])
            per_hot = [int((idx[toks] == e).any(axis=1).sum()) for e in range(cfg.hot_experts)]
            report(f"imbalance step {step} outputs", aff_err=aerr, out_err=err, shared_err=ysh, sampled=len(toks),
                   min_tokens_per_hot_expert=min(per_hot))
            assert aerr <= 1e-5 and err <= 1e-2 and ysh <= 1e-2
            assert min(per_hot) >= 8
        report(f"imbalance step {step}", max_over_mean=loads[-1],
               hot_bias=float(b_next[: cfg.hot_experts].mean()))
        b = b_next
    report("imbalance 100 steps", first_max_over_mean=loads[0], last_max_over_mean=loads[-1],
           min_max_over_mean=min(loads))
    assert loads[-1] < loads[0]          # the bias has moved load off the hot experts
    del layer, inp
    gc.collect()
    torch.cuda.empty_cache()


def test_bias_trajectory_100_steps_identical_affinities():
    """100 route -> permute -> bias-update steps on identical fp32 affinities: bias bit-exact every step."""
    import sparse_moe_transformer_02_amd as moe
    cfg = W.config("imbalance_bf16")
    bias = torch.zeros(cfg.N_r, device=DEV)
    b = np.zeros(cfg.N_r, np.float32)
    loads = []
    for step in range(cfg.steps):
        s = W.make_affinities(cfg, step, device=DEV)
        idx, _ = moe.moe_route(None, None, bias, cfg.K, affinity_in=s)
        counts, *_ = moe.moe_permute(idx, cfg.N_r)
        moe.moe_bias_update(counts, bias, cfg.T, cfg.K, cfg.gamma)
        ref = oracle.route(None, None, b, cfg.K, affinity_in=host(s))
        d = oracle.dispatch(ref["idx"], cfg.N_r)
        assert np.array_equal(host(counts), d["counts"])
        b = oracle.bias_update(b, d["counts"], cfg.T, cfg.K, cfg.gamma)
        assert np.array_equal(host(bias).view(np.uint32), b.view(np.uint32)), f"step {step}"
        loads.append(oracle.load_stats(d["counts"], cfg.T, cfg.K)["max_over_mean"])
    report("bias trajectory 100 steps", first_max_over_mean=loads[0], last_max_over_mean=loads[-1])
    assert loads[-1] < loads[0]                 # the bias moves load off the hot experts


def test_layer_is_deterministic():
    cfg = W.config("prefill_bf16").scaled(T=1024)
    inp, layer = _build(cfg)
    a = layer.forward(inp["u"]).clone()
    b = layer.forward(inp["u"])
    assert torch.equal(a, b)
    del layer, inp
    gc.collect()
    torch.cuda.empty_cache()
