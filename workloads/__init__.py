"""Seeded synthetic inputs for the DeepSeekMoE feed-forward layer workloads.

This module only draws random tensors and casts them to their storage dtype.
It holds none of the layer's arithmetic (no affinity, selection, gating,
dispatch, quantization or FFN): both the HIP library and the CPU oracle consume
what it produces, so it must stay free of either side's logic.

Shapes follow the DeepSeek-V3 model as the pages state it: hidden size 7168
("官方揭秘DeepSeek-V3模型训练全流程", §3.1 hyperparameters), 1 shared + 256
routed experts with 8 active ("รายงานเชิงเทคนิคของ DeepSeek-V3", key ideas;
"Deepseek V3 国货之光 开源之光", Mixture of Experts section). The expert
intermediate size 2048 and the value distributions are workload choices: the
pages give neither.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

__all__ = ["MoeConfig", "CONFIGS", "config", "make_inputs", "make_tokens",
           "make_affinities", "bf16_bits"]


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    """One synthetic workload of the layer.

    dtype: "f32" (activations, weights and outputs in fp32), "bf16" (bf16
    activations/weights/outputs) or "fp8" (bf16 inputs and outputs, E4M3 GEMM
    operands with 1x128 activation-tile and 128x128 weight-block scales).
    """
    name: str
    T: int
    H: int
    N_r: int
    K: int
    I: int
    dtype: str
    seed: int
    N_s: int = 1
    bias_init: str = "zero"          # "zero" or "uniform" (U(-bias_range, bias_range))
    bias_range: float = 0.01
    hot_experts: int = 0             # experts 0..hot_experts-1 get hot_logit added to their logit
    hot_logit: float = 0.0
    outlier_frac: float = 0.0        # Bernoulli fraction of activation elements scaled by outlier_scale
    outlier_scale: float = 1.0
    steps: int = 1                   # forward + bias-update steps
    gamma: float = 1e-3

    def scaled(self, **kw) -> "MoeConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny_f32": MoeConfig("tiny_f32", T=64, H=128, N_r=16, K=2, I=64, dtype="f32", seed=1, steps=2),
    "decode_bf16": MoeConfig("decode_bf16", T=128, H=7168, N_r=256, K=8, I=2048, dtype="bf16", seed=2,
                             bias_init="uniform", bias_range=0.01),
    "prefill_bf16": MoeConfig("prefill_bf16", T=4096, H=7168, N_r=256, K=8, I=2048, dtype="bf16", seed=3),
    "imbalance_bf16": MoeConfig("imbalance_bf16", T=16384, H=7168, N_r=256, K=8, I=2048, dtype="bf16",
                                seed=4, hot_experts=8, hot_logit=2.0, steps=100),
    "fp8": MoeConfig("fp8", T=8192, H=7168, N_r=256, K=8, I=2048, dtype="fp8", seed=5,
                     outlier_frac=1e-3, outlier_scale=50.0),
    # serving shape beyond the five above: the FP8 layer at decode size (timed, not a parity config)
    "fp8_decode": MoeConfig("fp8_decode", T=128, H=7168, N_r=256, K=8, I=2048, dtype="fp8", seed=6,
                            outlier_frac=1e-3, outlier_scale=50.0),
}


def config(name: str) -> MoeConfig:
    return CONFIGS[name]


# Sub-seed layout: one base seed per workload, fixed offsets per tensor.
_U, _E, _B, _MASK, _SHARED, _EXPERT0, _STEP0, _AFF = 0, 1, 2, 3, 99, 100, 10000, 20000


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _act_dtype(cfg: MoeConfig) -> torch.dtype:
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def _randn(shape, std, seed, device, dtype):
    x = torch.randn(shape, generator=_gen(device, seed), device=device, dtype=torch.float32)
    return (x * std).to(dtype)


def make_tokens(cfg: MoeConfig, step: int = 0, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    """u [T, H]: N(0,1) hidden states (fresh per step), with optional outliers."""
    T = cfg.T if T is None else T
    seed = cfg.seed * 1_000_003 + (_U if step == 0 else _STEP0 + step)
    x = torch.randn((T, cfg.H), generator=_gen(device, seed), device=device, dtype=torch.float32)
    if cfg.outlier_frac > 0:
        m = torch.rand((T, cfg.H), generator=_gen(device, cfg.seed * 1_000_003 + _MASK + step),
                       device=device) < cfg.outlier_frac
        x = torch.where(m, x * cfg.outlier_scale, x)
    return x.to(_act_dtype(cfg))


def make_affinities(cfg: MoeConfig, step: int = 0, device="cpu", T: Optional[int] = None,
                    tie_levels: int = 0) -> torch.Tensor:
    """Synthetic fp32 affinities in (0,1) [T, N_r], for comparing router stages on identical inputs.

    Uniform in (0, 1); with cfg.hot_experts, those experts draw from (0.5, 1) and the
    rest from (0, 0.5) so that they are hot. tie_levels > 0 quantizes the values onto
    that many levels so that exact ties are frequent.
    """
    T = cfg.T if T is None else T
    s = torch.rand((T, cfg.N_r), generator=_gen(device, cfg.seed * 1_000_003 + _AFF + step),
                   device=device, dtype=torch.float32)
    if cfg.hot_experts > 0:
        s = s * 0.5
        s[:, : cfg.hot_experts] += 0.5
    if tie_levels > 0:
        s = (torch.floor(s * tie_levels) + 0.5) / tie_levels
    return s.clamp_(1e-6, 1 - 1e-6)


def make_inputs(cfg: MoeConfig, device="cpu", with_weights: bool = True) -> dict:
    """All layer inputs for step 0.

    Returns a dict of torch tensors on `device`:
      u [T,H] (f32 or bf16), centroids [N_r,H] f32, bias [N_r] f32,
      logit_offset [N_r] f32 or None,
      w_gate/w_up [N_r,I,H], w_down [N_r,H,I], and the shared expert's
      sw_gate/sw_up [N_s,I,H], sw_down [N_s,H,I] (f32 for "f32", bf16 otherwise).
      The shared and routed weights of one projection are views into one
      [N_s + N_r, ...] tensor, shared first.
    Weight std is 1/sqrt(fan_in); centroid std 1/sqrt(H).
    """
    H, I, N_r = cfg.H, cfg.I, cfg.N_r
    base = cfg.seed * 1_000_003
    wdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    out = {
        "u": make_tokens(cfg, 0, device),
        "centroids": _randn((N_r, H), 1.0 / math.sqrt(H), base + _E, device, torch.float32),
    }
    if cfg.bias_init == "uniform":
        b = torch.rand((N_r,), generator=_gen(device, base + _B), device=device, dtype=torch.float32)
        out["bias"] = (b * 2 - 1) * cfg.bias_range
    else:
        out["bias"] = torch.zeros((N_r,), device=device, dtype=torch.float32)
    if cfg.hot_experts > 0:
        o = torch.zeros((N_r,), device=device, dtype=torch.float32)
        o[: cfg.hot_experts] = cfg.hot_logit
        out["logit_offset"] = o
    else:
        out["logit_offset"] = None
    if with_weights:
        # one tensor per projection holds the shared expert(s) first, then the routed experts;
        # w_* / sw_* are views into it (the layer can then run all experts in one launch)
        S = cfg.N_s
        ga = torch.empty((S + N_r, I, H), device=device, dtype=wdt)
        ua = torch.empty((S + N_r, I, H), device=device, dtype=wdt)
        da = torch.empty((S + N_r, H, I), device=device, dtype=wdt)
        for j in range(S):
            s0 = base + _SHARED * 1000 + 3 * j
            ga[j] = _randn((I, H), 1.0 / math.sqrt(H), s0, device, wdt)
            ua[j] = _randn((I, H), 1.0 / math.sqrt(H), s0 + 1, device, wdt)
            da[j] = _randn((H, I), 1.0 / math.sqrt(I), s0 + 2, device, wdt)
        for e in range(N_r):
            s0 = base + _EXPERT0 + 3 * e
            ga[S + e] = _randn((I, H), 1.0 / math.sqrt(H), s0, device, wdt)
            ua[S + e] = _randn((I, H), 1.0 / math.sqrt(H), s0 + 1, device, wdt)
            da[S + e] = _randn((H, I), 1.0 / math.sqrt(I), s0 + 2, device, wdt)
        out.update(w_gate=ga[S:], w_up=ua[S:], w_down=da[S:], sw_gate=ga[:S], sw_up=ua[:S], sw_down=da[:S])
    return out


def bf16_bits(t: torch.Tensor):
    """The raw 16-bit patterns of a bf16 tensor as a host numpy uint16 array (no arithmetic)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")
