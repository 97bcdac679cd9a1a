"""A layer training step captured in a HIP graph (torch.cuda.graph) and replayed.

The step issues only the library's kernels on the caller's stream, with no allocation, host
synchronisation or memset inside, so it can be captured once and replayed. Each replay is
checked against an eager step from the same state: the layer output, the selection and the
bias after the update bit-identical, replay after replay, with eager work (the next input's
copy and an eager step of a second layer) between the replays.
"""
import pytest
import torch

import workloads as W
from sparse_moe_transformer_02_amd.layer import MoeLayer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _layer(cfg, inp):
    return MoeLayer(inp["centroids"], inp["bias"].clone(), inp["w_gate"], inp["w_up"], inp["w_down"],
                    inp["sw_gate"], inp["sw_up"], inp["sw_down"], cfg.K, dtype=cfg.dtype,
                    logit_offset=inp["logit_offset"], gamma=cfg.gamma)


@pytest.mark.parametrize("name", ["decode_bf16", "fp8_decode"])
def test_layer_step_graph_replays_match_eager(name):
    cfg = W.config(name)
    inp = W.make_inputs(cfg, device=DEV)
    T, H = cfg.T, cfg.H
    g = torch.Generator(device=DEV).manual_seed(5)
    us = [(torch.randn((T, H), generator=g, device=DEV) * 0.5).to(inp["u"].dtype) for _ in range(4)]

    # eager reference from the initial bias
    ref = _layer(cfg, inp)
    b0 = ref.bias.clone()
    outs, biases, idxs = [], [], []
    for u in us:
        outs.append(ref.step(u).clone())
        idxs.append(ref.last["idx"].clone())
        biases.append(ref.bias.clone())
    torch.cuda.synchronize()

    lay = _layer(cfg, inp)
    u_static = us[0].clone()
    lay.step(u_static)                   # allocates the per-T buffers outside the capture
    torch.cuda.synchronize()
    lay.bias.copy_(b0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = lay.step(u_static)
    other = _layer(cfg, inp)             # eager work between the replays
    for k, u in enumerate(us):
        u_static.copy_(u)
        graph.replay()
        other.step(u)
        torch.cuda.synchronize()
        assert torch.equal(lay.last["idx"], idxs[k]), k
        assert torch.equal(out, outs[k]), k
        assert torch.equal(lay.bias, biases[k]), k
