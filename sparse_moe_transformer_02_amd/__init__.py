"""MI355X (gfx950) DeepSeekMoE feed-forward layer: Python binding of libmoe_mi355x.so.

The functions here have the names of the C entry points declared in
include/moe.h and only marshal arguments: tensors become device pointers, the
current torch stream becomes the HIP stream, and a non-zero status raises
MoeError. Every step of the layer runs in the library's HIP kernels; nothing
here computes. Output tensors that the caller does not pass are allocated with
torch (device memory is all torch is used for).

The library must be built first (``python -m sparse_moe_transformer_02_amd.build``);
importing works without it, but every call then raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["F32", "BF16", "FP8_E4M3", "MoeError", "lib", "library_path", "moe_route", "moe_route_group_limited",
           "moe_route_workspace_size", "moe_permute", "moe_permute_workspace_size", "moe_permute_noalloc",
           "moe_permute_noalloc_max_bytes", "moe_gather_rows",
           "moe_grouped_ffn", "moe_grouped_ffn_workspace_size", "moe_combine", "moe_bias_update",
           "fp8_quant_tiles", "moe_pack_fp8_payload", "moe_pack_fp8_payload_workspace_size",
           "moe_unpack_fp8_payload", "moe_combine_backward", "moe_grouped_ffn_backward",
           "moe_grouped_ffn_backward_workspace_size", "moe_router_backward", "moe_router_backward_workspace_size",
           "moe_seq_balance_loss", "moe_fp8_transpose_weights", "moe_grouped_ffn_backward_fp8",
           "moe_grouped_ffn_backward_fp8_workspace_size", "moe_abi_version", "EXPORTS"]

F32, BF16, FP8_E4M3 = 0, 1, 2
EXPORTS = ("moe_route_workspace_size", "moe_route", "moe_route_group_limited", "moe_permute_workspace_size",
           "moe_permute", "moe_permute_noalloc_max_bytes", "moe_permute_noalloc", "moe_gather_rows",
           "moe_grouped_ffn_workspace_size", "moe_grouped_ffn", "moe_grouped_ffn_profiled",
           "moe_grouped_ffn_train", "moe_combine", "moe_bias_update",
           "fp8_quant_tiles", "moe_pack_fp8_payload_workspace_size", "moe_pack_fp8_payload",
           "moe_unpack_fp8_payload", "moe_combine_backward", "moe_grouped_ffn_backward_workspace_size",
           "moe_grouped_ffn_backward", "moe_grouped_ffn_backward_profiled", "moe_grouped_ffn_backward_saved",
           "moe_router_backward_workspace_size",
           "moe_router_backward", "moe_fp8_transpose_weights", "moe_grouped_ffn_backward_fp8_workspace_size",
           "moe_grouped_ffn_backward_fp8", "moe_seq_balance_loss_workspace_size", "moe_seq_balance_loss",
           "moe_status_string", "moe_last_error",
           "moe_abi_version")

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmoe_mi355x.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_SIGS = {
    "moe_route_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_route": (_I, [_P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_group_limited": (_I, [_P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "moe_seq_balance_loss_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_seq_balance_loss": (_I, [_P, _P, _I, _I, _I, _I, ctypes.c_float, _P, _P, _SZ, _P]),
    "moe_combine_backward": (_I, [_P, _I, _P, _I, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "moe_grouped_ffn_backward_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "moe_grouped_ffn_backward": (_I, [_I, _P, _I, _P, _P, _I, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_grouped_ffn_backward_profiled": (_I, [_I, _P, _I, _P, _P, _I, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P,
                                               _SZ, _P, _P]),
    "moe_grouped_ffn_backward_saved": (_I, [_I, _P, _I, _P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P,
                                            _P, _SZ, _P, _P]),
    "moe_grouped_ffn_train": (_I, [_I, _P, _I, _P, _P, _I, _P, _P, _P, _I, _I, _P, _I, _P, _P, _SZ, _P, _P]),
    "moe_router_backward_workspace_size": (_SZ, [_I]),
    "moe_fp8_transpose_weights": (_I, [_I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_grouped_ffn_backward_fp8_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "moe_grouped_ffn_backward_fp8": (_I, [_I, _P, _I, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P,
                                          _P, _P, _P, _SZ, _P, _P]),
    "moe_router_backward": (_I, [_P, _P, _I, _P, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P,
                                 _P, _SZ, _P]),
    "moe_pack_fp8_payload_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_pack_fp8_payload": (_I, [_P, _I, _I, _I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_unpack_fp8_payload": (_I, [_P, _P, _I, _I, _P, _I, _P]),
    "moe_permute_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_permute": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute_noalloc_max_bytes": (_SZ, []),
    "moe_permute_noalloc": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P]),
    "moe_gather_rows": (_I, [_P, _P, _I, _I, _I, _P, _P, _I, _P, _P, _P]),
    "moe_grouped_ffn_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
    "moe_grouped_ffn": (_I, [_I, _P, _I, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _I,
                             _P, _SZ, _P]),
    "moe_grouped_ffn_profiled": (_I, [_I, _P, _I, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P,
                                      _I, _P, _SZ, _P, _P]),
    "moe_combine": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "moe_bias_update": (_I, [_P, _I, _I, _I, ctypes.c_float, _P, _P]),
    "fp8_quant_tiles": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_abi_version": (_I, []),
}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it with "
                               "`python -m sparse_moe_transformer_02_amd.build`")
        L = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _tag(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status, lib().moe_last_error().decode())


def _device(*ts) -> torch.device:
    for t in ts:
        if isinstance(t, torch.Tensor):
            return t.device
    return torch.device("cuda")


def _ws(nbytes: int, workspace, dev):
    if workspace is not None or nbytes == 0:
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=dev)


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def moe_abi_version() -> int:
    return lib().moe_abi_version()


# ---------------------------------------------------------------------------- router
def moe_route_workspace_size(T: int, H: int, N_r: int) -> int:
    return lib().moe_route_workspace_size(T, H, N_r)


def moe_route(u, centroids, bias, K: int, *, logit_offset=None, affinity_in=None, affinity_out=None,
              topk_idx=None, topk_gate=None, workspace=None, stream=None):
    """Affinity -> biased top-K -> normalised gates. Returns (topk_idx [T,K] int32, topk_gate [T,K] f32)."""
    return _route("moe_route", u, centroids, bias, K, None, logit_offset, affinity_in, affinity_out,
                  topk_idx, topk_gate, workspace, stream)


def moe_route_group_limited(u, centroids, bias, K: int, n_groups: int, topk_groups: int, *, logit_offset=None,
                            affinity_in=None, affinity_out=None, topk_idx=None, topk_gate=None, workspace=None,
                            stream=None):
    """moe_route with each token's K experts drawn from at most topk_groups of n_groups expert groups."""
    return _route("moe_route_group_limited", u, centroids, bias, K, (n_groups, topk_groups), logit_offset,
                  affinity_in, affinity_out, topk_idx, topk_gate, workspace, stream)


def _route(name, u, centroids, bias, K, groups, logit_offset, affinity_in, affinity_out, topk_idx, topk_gate,
           workspace, stream):
    if affinity_in is not None:
        T, N_r = affinity_in.shape
        H = u.shape[1] if u is not None else 1
    else:
        T, H = u.shape
        N_r = centroids.shape[0]
    dev = _device(u, affinity_in, bias)
    if topk_idx is None:
        topk_idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    if topk_gate is None:
        topk_gate = torch.empty((T, K), dtype=torch.float32, device=dev)
    if affinity_in is None:
        workspace = _ws(moe_route_workspace_size(T, H, N_r), workspace, dev)
    head = (_ptr(u), _tag(u) if u is not None else F32, _ptr(centroids), _ptr(bias), _ptr(logit_offset),
            _ptr(affinity_in), T, H, N_r, K)
    tail = (_ptr(affinity_out), _ptr(topk_idx), _ptr(topk_gate), _ptr(workspace), _nbytes(workspace),
            _stream(stream))
    st = getattr(lib(), name)(*head, *(groups or ()), *tail)
    _check(name, st)
    return topk_idx, topk_gate


# ---------------------------------------------------------------------------- dispatch
def moe_permute_workspace_size(T: int, K: int, N_r: int) -> int:
    return lib().moe_permute_workspace_size(T, K, N_r)


def moe_permute(topk_idx, N_r: int, *, shared_rows: int = 0, counts=None, offsets=None, row_token=None,
                slot_row=None, workspace=None, stream=None):
    """Returns (counts [N_r], offsets [N_r+1 (+1 with shared rows)], row_token [S+T*K], slot_row [T*K])."""
    T, K = topk_idx.shape
    dev = topk_idx.device
    S = int(shared_rows)
    counts = torch.empty(N_r, dtype=torch.int32, device=dev) if counts is None else counts
    if offsets is None:
        offsets = torch.empty(N_r + (2 if S else 1), dtype=torch.int32, device=dev)
    row_token = torch.empty(S + T * K, dtype=torch.int32, device=dev) if row_token is None else row_token
    slot_row = torch.empty(T * K, dtype=torch.int32, device=dev) if slot_row is None else slot_row
    workspace = _ws(moe_permute_workspace_size(T, K, N_r), workspace, dev)
    st = lib().moe_permute(_ptr(topk_idx), T, K, N_r, S, _ptr(counts), _ptr(offsets), _ptr(row_token),
                           _ptr(slot_row), _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check("moe_permute", st)
    return counts, offsets, row_token, slot_row


def moe_permute_noalloc_max_bytes() -> int:
    return lib().moe_permute_noalloc_max_bytes()


def moe_permute_noalloc(topk_idx, N_r: int, *, shared_rows: int, counts, offsets, row_token, slot_row,
                        stream=None):
    """moe_permute with the library's static scratch instead of a workspace: every output is
    caller-provided and nothing is allocated. Calls that overlap on one GPU race."""
    T, K = topk_idx.shape
    st = lib().moe_permute_noalloc(_ptr(topk_idx), T, K, N_r, int(shared_rows), _ptr(counts), _ptr(offsets),
                                   _ptr(row_token), _ptr(slot_row), _stream(stream))
    _check("moe_permute_noalloc", st)
    return counts, offsets, row_token, slot_row


def moe_gather_rows(x, row_token, n_rows, max_rows: int, *, x_scales=None, x_perm=None, x_perm_scales=None,
                    stream=None):
    """x_perm[r] = x[row_token[r]] for r < min(*n_rows, max_rows) (n_rows: a one-element device
    int32 tensor or view, e.g. offsets[-1:] of moe_permute). FP8 codes (uint8) also gather their
    1x128 scales. Returns x_perm (and x_perm_scales for FP8)."""
    T, H = x.shape
    fp8 = _tag(x) == FP8_E4M3
    x_perm = torch.empty((max_rows, H), dtype=x.dtype, device=x.device) if x_perm is None else x_perm
    if fp8 and x_perm_scales is None:
        x_perm_scales = torch.empty((max_rows, H // 128), dtype=torch.float32, device=x.device)
    st = lib().moe_gather_rows(_ptr(x), _ptr(x_scales), _tag(x), T, H, _ptr(row_token), _ptr(n_rows),
                               int(max_rows), _ptr(x_perm), _ptr(x_perm_scales), _stream(stream))
    _check("moe_gather_rows", st)
    return (x_perm, x_perm_scales) if fp8 else x_perm


# ---------------------------------------------------------------------------- expert FFNs
def moe_grouped_ffn_workspace_size(n_groups: int, total_rows: int, H: int, I: int, x_dtype: int) -> int:
    return lib().moe_grouped_ffn_workspace_size(n_groups, total_rows, H, I, x_dtype)


def moe_grouped_ffn(offsets, total_rows: int, X, W_gate, W_up, W_down, *, row_index=None, X_scales=None,
                    Wg_scales=None, Wu_scales=None, Wd_scales=None, Y=None, y_dtype=None,
                    workspace=None, stream=None, events=None, preact=None):
    """Grouped SwiGLU FFN over the row groups given by device `offsets` [n_groups+1]. Returns Y.

    events: optional sequence of 4 torch.cuda.Event (or None) recorded by the library around
    its kernels (moe_grouped_ffn_profiled): before/after the gate-up GEMM, before/after the down GEMM.
    preact: optional fp32 [total_rows, 2I] (bf16 only): also receives z | v (moe_grouped_ffn_train).
    """
    n_groups = offsets.numel() - 1
    x_rows, H = X.shape
    I = W_gate.shape[1]
    xt = _tag(X)
    if Y is None:
        ydt = y_dtype if y_dtype is not None else (torch.float32 if X.dtype == torch.float32 else torch.bfloat16)
        Y = torch.empty((total_rows, H), dtype=ydt, device=X.device)
    workspace = _ws(moe_grouped_ffn_workspace_size(n_groups, total_rows, H, I, xt), workspace, X.device)
    args = [n_groups, _ptr(offsets), total_rows, _ptr(row_index), _ptr(X), _ptr(X_scales), x_rows, xt,
            _ptr(W_gate), _ptr(W_up), _ptr(W_down), _ptr(Wg_scales), _ptr(Wu_scales), _ptr(Wd_scales),
            _tag(W_gate), H, I, _ptr(Y), _tag(Y), _ptr(workspace), _nbytes(workspace), _stream(stream)]
    arr = None if events is None else (ctypes.c_void_p * 4)(*[None if e is None else e.cuda_event for e in events])
    if preact is not None:
        st = lib().moe_grouped_ffn_train(n_groups, _ptr(offsets), total_rows, _ptr(row_index), _ptr(X), x_rows,
                                         _ptr(W_gate), _ptr(W_up), _ptr(W_down), H, I, _ptr(Y), _tag(Y), _ptr(preact),
                                         _ptr(workspace), _nbytes(workspace), _stream(stream), arr)
        _check("moe_grouped_ffn_train", st)
        return Y
    if events is None:
        st = lib().moe_grouped_ffn(*args)
    else:
        st = lib().moe_grouped_ffn_profiled(*args, arr)
    _check("moe_grouped_ffn", st)
    return Y


# ---------------------------------------------------------------------------- combine / bias
def moe_combine(u, shared_y, Y, slot_row, topk_gate, *, out=None, stream=None):
    """out = u + shared_y + sum_k gate * Y[slot_row]. Returns out ([T,H], u's dtype)."""
    T, H = u.shape
    K = topk_gate.shape[1]
    out = torch.empty_like(u) if out is None else out
    st = lib().moe_combine(_ptr(u), _ptr(shared_y), _ptr(Y), _ptr(slot_row), _ptr(topk_gate), T, K, H,
                           Y.shape[0], _tag(u), _tag(Y), _ptr(out), _stream(stream))
    _check("moe_combine", st)
    return out


def moe_bias_update(counts, bias, T: int, K: int, gamma: float = 1e-3, *, stream=None):
    """In-place sign-based bias update from this step's per-expert counts."""
    st = lib().moe_bias_update(_ptr(counts), bias.numel(), T, K, float(gamma), _ptr(bias), _stream(stream))
    _check("moe_bias_update", st)
    return bias


# ---------------------------------------------------------------------------- fp8
def fp8_quant_tiles(x, tile_rows: int, *, codes=None, scales=None, stream=None):
    """E4M3FN codes (uint8, x's shape) and fp32 scales per tile_rows x 128 tile of a 2-D tensor."""
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device) if codes is None else codes
    if scales is None:
        scales = torch.empty((rows // tile_rows, cols // 128), dtype=torch.float32, device=x.device)
    st = lib().fp8_quant_tiles(_ptr(x), _tag(x), rows, cols, tile_rows, 128, _ptr(codes), _ptr(scales),
                               _stream(stream))
    _check("fp8_quant_tiles", st)
    return codes, scales


def moe_pack_fp8_payload_workspace_size(T: int, K: int, n_ranks: int) -> int:
    return lib().moe_pack_fp8_payload_workspace_size(T, K, n_ranks)


def moe_pack_fp8_payload(x, topk_idx, N_r: int, n_ranks: int, *, workspace=None, stream=None) -> dict:
    """Expert-parallel send plan + FP8 payload (one row per token and destination rank).

    Returns counts [R], offsets [R+1], send_token / codes / scales sized for T*min(K, R) rows
    (rows past offsets[R] untouched) and slot_send [T*K]."""
    T, H = x.shape
    K = topk_idx.shape[1]
    dev = x.device
    rows = T * min(K, n_ranks)
    out = {"counts": torch.empty(n_ranks, dtype=torch.int32, device=dev),
           "offsets": torch.empty(n_ranks + 1, dtype=torch.int32, device=dev),
           "send_token": torch.empty(rows, dtype=torch.int32, device=dev),
           "slot_send": torch.empty(T * K, dtype=torch.int32, device=dev),
           "codes": torch.empty((rows, H), dtype=torch.uint8, device=dev),
           "scales": torch.empty((rows, H // 128), dtype=torch.float32, device=dev)}
    workspace = _ws(moe_pack_fp8_payload_workspace_size(T, K, n_ranks), workspace, dev)
    st = lib().moe_pack_fp8_payload(_ptr(x), _tag(x), T, H, _ptr(topk_idx), K, N_r, n_ranks, _ptr(out["counts"]),
                                    _ptr(out["offsets"]), _ptr(out["send_token"]), _ptr(out["slot_send"]),
                                    _ptr(out["codes"]), _ptr(out["scales"]), _ptr(workspace), _nbytes(workspace),
                                    _stream(stream))
    _check("moe_pack_fp8_payload", st)
    return out


def moe_unpack_fp8_payload(codes, scales, *, out_dtype=torch.bfloat16, out=None, stream=None):
    """fl32(decode(code) * scale) per 1x128 tile, stored as out_dtype (bf16 or fp32)."""
    rows, H = codes.shape
    if out is None:
        out = torch.empty((rows, H), dtype=out_dtype, device=codes.device)
    st = lib().moe_unpack_fp8_payload(_ptr(codes), _ptr(scales), rows, H, _ptr(out), _tag(out), _stream(stream))
    _check("moe_unpack_fp8_payload", st)
    return out


def moe_combine_backward(dout, Y, slot_row, topk_gate, K: int, *, shared_rows: int = 0, dY=None, dgate=None,
                         stream=None):
    """dY rows (bf16 [total_rows, H]: shared rows get dout, routed rows g * dout) and dgate [T, K]."""
    T, H = dout.shape
    total_rows = Y.shape[0]
    dY = torch.empty((total_rows, H), dtype=torch.bfloat16, device=dout.device) if dY is None else dY
    dgate = torch.empty((T, K), dtype=torch.float32, device=dout.device) if dgate is None else dgate
    st = lib().moe_combine_backward(_ptr(dout), _tag(dout), _ptr(Y), _tag(Y), _ptr(slot_row), _ptr(topk_gate), T, K, H,
                                    shared_rows, total_rows, _ptr(dY), _ptr(dgate), _stream(stream))
    _check("moe_combine_backward", st)
    return dY, dgate


def moe_grouped_ffn_backward_workspace_size(n_groups: int, total_rows: int, H: int, I: int) -> int:
    return lib().moe_grouped_ffn_backward_workspace_size(n_groups, total_rows, H, I)


def moe_grouped_ffn_backward(offsets, total_rows: int, X, W_gate, W_up, W_down, dY, *, row_index=None, dX=None,
                             dW_gate=None, dW_up=None, dW_down=None, workspace=None, stream=None, events=None,
                             preact=None):
    """dX [total_rows, H] and dW_gate / dW_up [G, I, H], dW_down [G, H, I] (fp32) of the grouped SwiGLU FFN.

    preact: the z | v the forward saved (moe_grouped_ffn(..., preact=...)); then they are not
    recomputed (moe_grouped_ffn_backward_saved), with bitwise the same gradients.
    """
    G, I, H = W_gate.shape
    dev = W_gate.device
    f32 = dict(dtype=torch.float32, device=dev)
    dX = torch.empty((total_rows, H), **f32) if dX is None else dX
    dW_gate = torch.empty((G, I, H), **f32) if dW_gate is None else dW_gate
    dW_up = torch.empty((G, I, H), **f32) if dW_up is None else dW_up
    dW_down = torch.empty((G, H, I), **f32) if dW_down is None else dW_down
    workspace = _ws(moe_grouped_ffn_backward_workspace_size(G, total_rows, H, I), workspace, dev)
    args = (G, _ptr(offsets), total_rows, _ptr(row_index), _ptr(X), X.shape[0], _ptr(W_gate), _ptr(W_up),
            _ptr(W_down), _ptr(dY), H, I, _ptr(dX), _ptr(dW_gate), _ptr(dW_up), _ptr(dW_down), _ptr(workspace),
            _nbytes(workspace), _stream(stream))
    if preact is not None:
        handles = None if events is None else (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e.cuda_event) for e in events])
        a = list(args)
        a.insert(10, _ptr(preact))          # zv follows dY
        st = lib().moe_grouped_ffn_backward_saved(*a, handles)
        _check("moe_grouped_ffn_backward_saved", st)
    elif events is None:
        st = lib().moe_grouped_ffn_backward(*args)
        _check("moe_grouped_ffn_backward", st)
    else:
        handles = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e.cuda_event) for e in events])
        st = lib().moe_grouped_ffn_backward_profiled(*args, handles)
        _check("moe_grouped_ffn_backward_profiled", st)
    return dX, dW_gate, dW_up, dW_down


def moe_fp8_transpose_weights(W_gate, Wg_scales, W_up, Wu_scales, W_down, Wd_scales, *, W_down_t=None,
                              Wd_t_scales=None, W_gate_up_t=None, Wgu_t_scales=None, stream=None):
    """The transposed E4M3 weight codes and block scales the FP8 backward's dgrad GEMMs read:
    W_down_t [G, I, H] (+ [G, I/128, H/128]) and W_gate_up_t [G, H, 2I] (+ [G, H/128, 2I/128])."""
    G, I, H = W_gate.shape
    dev = W_gate.device
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    W_down_t = torch.empty((G, I, H), **u8) if W_down_t is None else W_down_t
    Wd_t_scales = torch.empty((G, I // 128, H // 128), **f32) if Wd_t_scales is None else Wd_t_scales
    W_gate_up_t = torch.empty((G, H, 2 * I), **u8) if W_gate_up_t is None else W_gate_up_t
    Wgu_t_scales = torch.empty((G, H // 128, 2 * I // 128), **f32) if Wgu_t_scales is None else Wgu_t_scales
    st = lib().moe_fp8_transpose_weights(G, H, I, _ptr(W_gate), _ptr(Wg_scales), _ptr(W_up), _ptr(Wu_scales),
                                         _ptr(W_down), _ptr(Wd_scales), _ptr(W_down_t), _ptr(Wd_t_scales),
                                         _ptr(W_gate_up_t), _ptr(Wgu_t_scales), _stream(stream))
    _check("moe_fp8_transpose_weights", st)
    return W_down_t, Wd_t_scales, W_gate_up_t, Wgu_t_scales


def moe_grouped_ffn_backward_fp8_workspace_size(n_groups: int, total_rows: int, H: int, I: int) -> int:
    return lib().moe_grouped_ffn_backward_fp8_workspace_size(n_groups, total_rows, H, I)


def moe_grouped_ffn_backward_fp8(offsets, total_rows: int, X, W_gate, Wg_scales, W_up, Wu_scales, W_down_t,
                                 Wd_t_scales, W_gate_up_t, Wgu_t_scales, dY, *, row_index=None, dX=None,
                                 dW_gate=None, dW_up=None, dW_down=None, workspace=None, stream=None, events=None):
    """FP8 backward of the grouped SwiGLU FFN: dX [total_rows, H], dW_gate / dW_up [G, I, H] and
    dW_down [G, H, I] (fp32). X is the bf16 input of the forward; the weights are the forward's
    E4M3 codes and scales plus their transposes (moe_fp8_transpose_weights)."""
    G, I, H = W_gate.shape
    dev = W_gate.device
    f32 = dict(dtype=torch.float32, device=dev)
    dX = torch.empty((total_rows, H), **f32) if dX is None else dX
    dW_gate = torch.empty((G, I, H), **f32) if dW_gate is None else dW_gate
    dW_up = torch.empty((G, I, H), **f32) if dW_up is None else dW_up
    dW_down = torch.empty((G, H, I), **f32) if dW_down is None else dW_down
    workspace = _ws(moe_grouped_ffn_backward_fp8_workspace_size(G, total_rows, H, I), workspace, dev)
    handles = None if events is None else (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e.cuda_event) for e in events])
    st = lib().moe_grouped_ffn_backward_fp8(G, _ptr(offsets), total_rows, _ptr(row_index), _ptr(X), X.shape[0],
                                            _ptr(W_gate), _ptr(Wg_scales), _ptr(W_up), _ptr(Wu_scales),
                                            _ptr(W_down_t), _ptr(Wd_t_scales), _ptr(W_gate_up_t),
                                            _ptr(Wgu_t_scales), _ptr(dY), H, I, _ptr(dX), _ptr(dW_gate),
                                            _ptr(dW_up), _ptr(dW_down), _ptr(workspace), _nbytes(workspace),
                                            _stream(stream), handles)
    _check("moe_grouped_ffn_backward_fp8", st)
    return dX, dW_gate, dW_up, dW_down


def moe_router_backward_workspace_size(total_rows: int) -> int:
    return lib().moe_router_backward_workspace_size(total_rows)


def moe_router_backward(dout, u, dX_rows, offsets, row_token, slot_row, affinity, topk_idx, topk_gate, dgate,
                        centroids, *, shared_rows: int = 0, du=None, dcentroids=None, workspace=None, stream=None):
    """du [T, H] (fp32) and dcentroids [N_r, H] (fp32): gate, sigmoid, router and input gradients."""
    T, H = u.shape
    N_r = centroids.shape[0]
    K = topk_idx.shape[1]
    total_rows = dX_rows.shape[0]
    du = torch.empty((T, H), dtype=torch.float32, device=u.device) if du is None else du
    dcentroids = torch.empty((N_r, H), dtype=torch.float32, device=u.device) if dcentroids is None else dcentroids
    workspace = _ws(moe_router_backward_workspace_size(total_rows), workspace, u.device)
    st = lib().moe_router_backward(_ptr(dout), _ptr(u), _tag(u), _ptr(dX_rows), _ptr(offsets), _ptr(row_token),
                                   _ptr(slot_row), shared_rows, total_rows, _ptr(affinity), _ptr(topk_idx),
                                   _ptr(topk_gate), _ptr(dgate), _ptr(centroids), T, K, H, N_r, _ptr(du),
                                   _ptr(dcentroids), _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check("moe_router_backward", st)
    return du, dcentroids


def moe_seq_balance_loss_workspace_size(T: int, N_r: int, seq_len: int) -> int:
    return lib().moe_seq_balance_loss_workspace_size(T, N_r, seq_len)


def moe_seq_balance_loss(affinity, topk_idx, seq_len: int, alpha: float = 1e-4, *, loss=None, workspace=None,
                         stream=None):
    """Sequence-wise balance loss per sequence of seq_len tokens (fp32 [ceil(T / seq_len)])."""
    T, N_r = affinity.shape
    K = topk_idx.shape[1]
    n = (T + seq_len - 1) // seq_len
    loss = torch.empty(n, dtype=torch.float32, device=affinity.device) if loss is None else loss
    workspace = _ws(moe_seq_balance_loss_workspace_size(T, N_r, seq_len), workspace, affinity.device)
    st = lib().moe_seq_balance_loss(_ptr(affinity), _ptr(topk_idx), T, N_r, K, seq_len, alpha, _ptr(loss),
                                    _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check("moe_seq_balance_loss", st)
    return loss
