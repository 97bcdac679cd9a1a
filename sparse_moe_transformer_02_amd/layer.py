"""One DeepSeekMoE feed-forward layer on one GPU, composed from the library's entry points.

    route -> permute (shared expert as group 0) -> [fp8_quant_tiles(u)]
          -> grouped FFN (shared + routed experts in one launch) -> combine
          and, at the end of a training step, bias update

(xyznot.com "รายงานเชิงเทคนิคของ DeepSeek-V3", Method §2: h'_t = u_t + shared FFN +
sum_i g_{i,t} FFN_i(u_t); the bias b_i selects experts and moves by -/+gamma each step.)

This class only owns device buffers and sequences the C-ABI calls on one stream;
all arithmetic runs in the HIP kernels. Buffers are allocated once per token
count, so repeated forwards allocate nothing.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (moe_bias_update, moe_combine, moe_grouped_ffn, moe_grouped_ffn_workspace_size,
               moe_combine_backward, moe_grouped_ffn_backward, moe_router_backward,
               moe_fp8_transpose_weights, moe_grouped_ffn_backward_fp8,
               moe_permute, moe_permute_workspace_size, moe_route, moe_route_group_limited,
               moe_route_workspace_size,
               fp8_quant_tiles, F32, BF16, FP8_E4M3)


class MoeLayer:
    """Router + N_r routed experts + shared expert(s), resident on one GPU.

    Weights: w_gate/w_up [N_r, I, H], w_down [N_r, H, I]; shared sw_* with a leading
    N_s (= 1) dimension. dtype "f32" and "bf16" use the weights as given; "fp8"
    quantizes them once here (128x128 blocks) and quantizes activations per
    1x128 tile inside every forward.
    """

    def __init__(self, centroids, bias, w_gate, w_up, w_down, sw_gate, sw_up, sw_down, K: int, *,
                 dtype: str = "bf16", logit_offset=None, gamma: float = 1e-3, n_groups: int = 1,
                 topk_groups: int = 1):
        self.dtype = dtype
        self.K = K
        self.groups = (n_groups, topk_groups)   # > 1 groups: group-limited (node-limited) routing
        self.gamma = gamma
        self.centroids = centroids
        self.bias = bias
        self.logit_offset = logit_offset
        self.N_r, self.I, self.H = w_gate.shape
        if sw_gate.shape[0] != 1:
            raise ValueError("one shared expert is supported")
        self.dev = w_gate.device
        # all experts of one projection in one [1 + N_r, ...] tensor, the shared expert first
        full = [self._joined(sw, w) for sw, w in ((sw_gate, w_gate), (sw_up, w_up), (sw_down, w_down))]
        if dtype == "fp8":
            self.w = [self._quant_weight(w) for w in full]
        else:
            self.w = [(w, None) for w in full]
        self.w_t = None
        self._bufs = {}

    @staticmethod
    def _joined(shared, routed):
        """[shared; routed] along the expert axis: a view when they are adjacent in memory, else a copy."""
        n = shared.shape[0] + routed.shape[0]
        if (shared.is_contiguous() and routed.is_contiguous()
                and shared.untyped_storage().data_ptr() == routed.untyped_storage().data_ptr()
                and shared.storage_offset() + shared.numel() == routed.storage_offset()):
            return torch.as_strided(shared, (n,) + tuple(routed.shape[1:]), routed.stride(), shared.storage_offset())
        return torch.cat([shared, routed], dim=0)

    @staticmethod
    def _quant_weight(w):
        G, R, C = w.shape
        codes, scales = fp8_quant_tiles(w.reshape(G * R, C), 128)
        return codes.view(G, R, C), scales.view(G, R // 128, C // 128)

    def _buffers(self, T: int) -> dict:
        b = self._bufs.get(T)
        if b is not None:
            return b
        d, H, I, K, N_r = self.dev, self.H, self.I, self.K, self.N_r
        act = torch.float32 if self.dtype == "f32" else torch.bfloat16
        xt = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3}[self.dtype]
        rows = T + T * K                       # shared expert rows, then routed rows
        ws = max(moe_route_workspace_size(T, H, N_r), moe_permute_workspace_size(T, K, N_r),
                 moe_grouped_ffn_workspace_size(N_r + 1, rows, H, I, xt))
        y = torch.empty((rows, H), dtype=act, device=d)
        b = {
            "affinity": torch.empty((T, N_r), dtype=torch.float32, device=d),
            "idx": torch.empty((T, K), dtype=torch.int32, device=d),
            "gate": torch.empty((T, K), dtype=torch.float32, device=d),
            "counts": torch.empty(N_r, dtype=torch.int32, device=d),
            "offsets": torch.empty(N_r + 2, dtype=torch.int32, device=d),
            "row_token": torch.empty(rows, dtype=torch.int32, device=d),
            "slot_row": torch.empty(T * K, dtype=torch.int32, device=d),
            "y": y,
            "y_shared": y[:T],
            "out": torch.empty((T, H), dtype=act, device=d),
            "ws": torch.empty(max(ws, 1), dtype=torch.uint8, device=d),
        }
        if self.dtype == "fp8":
            b["u_codes"] = torch.empty((T, H), dtype=torch.uint8, device=d)
            b["u_scales"] = torch.empty((T, H // 128), dtype=torch.float32, device=d)
        self._bufs[T] = b
        return b

    def forward(self, u, *, affinity_in=None, stream=None, ffn_events=None, marks=None,
                keep_preact: bool = False) -> torch.Tensor:
        """h' for u [T, H]; intermediates stay in self.last (a dict of device tensors).

        The returned tensor and everything in self.last are the layer's buffers for this token
        count: the next forward (or step) with the same T overwrites them, and backward() uses
        whichever forward ran last. Callers that keep an output across calls clone it.

        keep_preact (bf16 layers): also keep the experts' gate/up pre-activations for backward(),
        which then does not recompute them (fp32, (T + T K) x 2I).
        ffn_events: optional 4 torch.cuda.Event recorded around the expert FFN's kernels.
        marks: optional list of 6 torch.cuda.Event recorded before the route and after route,
        permute, activation quantization, expert FFN (shared + routed) and combine
        (measurement only).
        """
        T = u.shape[0]
        b = self._buffers(T)
        mark = (lambda i: marks[i].record()) if marks is not None else (lambda i: None)
        mark(0)
        kw = dict(logit_offset=self.logit_offset, affinity_in=affinity_in,
                  affinity_out=b["affinity"] if affinity_in is None else None, topk_idx=b["idx"],
                  topk_gate=b["gate"], workspace=b["ws"], stream=stream)
        if self.groups[0] > 1:
            moe_route_group_limited(u, self.centroids, self.bias, self.K, *self.groups, **kw)
        else:
            moe_route(u, self.centroids, self.bias, self.K, **kw)
        mark(1)
        moe_permute(b["idx"], self.N_r, shared_rows=T, counts=b["counts"], offsets=b["offsets"],
                    row_token=b["row_token"], slot_row=b["slot_row"], workspace=b["ws"], stream=stream)
        mark(2)
        if self.dtype == "fp8":
            fp8_quant_tiles(u, 1, codes=b["u_codes"], scales=b["u_scales"], stream=stream)
            x, xs = b["u_codes"], b["u_scales"]
        else:
            x, xs = u, None
        mark(3)
        (wg, wgs), (wu, wus), (wd, wds) = self.w
        preact = None
        if keep_preact:
            if self.dtype != "bf16":
                raise NotImplementedError("saved pre-activations are built for bf16 layers")
            if "preact" not in b:
                b["preact"] = torch.empty((T + T * self.K, 2 * self.I), dtype=torch.float32, device=self.dev)
            preact = b["preact"]
        moe_grouped_ffn(b["offsets"], T + T * self.K, x, wg, wu, wd, row_index=b["row_token"], X_scales=xs,
                        Wg_scales=wgs, Wu_scales=wus, Wd_scales=wds, Y=b["y"], workspace=b["ws"],
                        stream=stream, events=ffn_events, preact=preact)
        mark(4)
        moe_combine(u, b["y_shared"], b["y"], b["slot_row"], b["gate"], out=b["out"], stream=stream)
        mark(5)
        self.last = b
        self.last_preact = preact
        self.last_u = u
        self.last_affinity = b["affinity"] if affinity_in is None else affinity_in
        return b["out"]

    def backward(self, dout, *, stream=None, ffn_events=None) -> dict:
        """Gradients of the last forward's output for an upstream dout [T, H] (bf16 and fp8 layers).

        combine backward -> grouped FFN backward (shared expert as group 0; bf16: it recomputes the
        gate/up pre-activations unless the forward kept them; fp8: every GEMM operand in E4M3,
        moe_grouped_ffn_backward_fp8) -> gate / router / input backward, all on the library's
        kernels. Returns fp32 tensors: du [T, H], dcentroids [N_r, H], dW_gate / dW_up
        [1 + N_r, I, H] and dW_down [1 + N_r, H, I] with the shared expert first, plus dgate
        [T, K]. The bias gets no gradient (it only selects).
        """
        if self.dtype not in ("bf16", "fp8"):
            raise NotImplementedError("the backward pass is built for bf16 and fp8 layers")
        b, u = self.last, self.last_u
        T = u.shape[0]
        rows = T + T * self.K
        dY, dgate = moe_combine_backward(dout, b["y"], b["slot_row"], b["gate"], self.K, shared_rows=T,
                                         stream=stream)
        if self.dtype == "fp8":
            if getattr(self, "w_t", None) is None:   # transposed codes for the dgrad GEMMs, once per weight set
                (wg, wgs), (wu, wus), (wd, wds) = self.w
                self.w_t = moe_fp8_transpose_weights(wg, wgs, wu, wus, wd, wds, stream=stream)
            (wg, wgs), (wu, wus), _ = self.w
            wdt, wdts, wgut, wguts = self.w_t
            dX, dWg, dWu, dWd = moe_grouped_ffn_backward_fp8(b["offsets"], rows, u, wg, wgs, wu, wus, wdt, wdts, wgut,
                                                             wguts, dY, row_index=b["row_token"], stream=stream,
                                                             events=ffn_events)
        else:
            (wg, _), (wu, _), (wd, _) = self.w
            dX, dWg, dWu, dWd = moe_grouped_ffn_backward(b["offsets"], rows, u, wg, wu, wd, dY,
                                                         row_index=b["row_token"], stream=stream, events=ffn_events,
                                                         preact=self.last_preact)
        du, dE = moe_router_backward(dout, u, dX, b["offsets"], b["row_token"], b["slot_row"], self.last_affinity,
                                     b["idx"], b["gate"], dgate, self.centroids, shared_rows=T, stream=stream)
        return {"du": du, "dcentroids": dE, "dW_gate": dWg, "dW_up": dWu, "dW_down": dWd, "dgate": dgate}

    def update_bias(self, T: int, stream=None):
        """End-of-step bias update from the counts of the last forward."""
        moe_bias_update(self._buffers(T)["counts"], self.bias, T, self.K, self.gamma, stream=stream)

    def step(self, u, stream=None, **measure) -> torch.Tensor:
        """One training-step forward: the layer output, then the bias update."""
        out = self.forward(u, stream=stream, **measure)
        self.update_bias(u.shape[0], stream=stream)
        return out
