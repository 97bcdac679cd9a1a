"""CPU oracle for the DeepSeekMoE feed-forward layer: forward pass and bias update.

TEST INFRASTRUCTURE. This module exists to check the HIP library. Only the
test suite, the package entry point's smoke check and the benchmark's CPU
baseline may import it; the library itself never does, and shares no code,
table or constant with it.

It is a plain, slow, float64 implementation written from the definitions on
the pages:

* "รายงานเชิงเทคนิคของ DeepSeek-V3" (xyznot.com), Method section 2
  "DeepSeekMoE with auxiliary-loss-free balancing": the layer output h'_t, the
  affinity s_{i,t} = Sigmoid(u_t^T e_i), the gate g'_{i,t} kept only when
  s_{i,t}+b_i is among the Top-K_r of {s_{j,t}+b_j}, the normalisation of g'
  into g, and the end-of-step bias rule b_i -/+ gamma with gamma = 0.001.
* "Deepseek V3 国货之光 开源之光" (databean.com.cn), section "Auxiliary-Loss-Free
  Load Balancing": the same steps in words; the bias only chooses experts and
  never enters the computed affinity.
* "官方揭秘DeepSeek-V3模型训练全流程" (youleyou.com) §4.3 "FP8 训练" and the
  "รายงานเชิงเทคนิคของ DeepSeek-V3" key ideas FP8 bullet: E4M3 for the GEMM operands, one scale per
  1x128 activation tile and per 128x128 weight block, taken online from the
  tile's maximum absolute value, FP32 accumulation; §2.2: no token dropping.

Readings where the pages leave a step open (each also listed in the design
notes):
* gates: g = g' / sum_j g'_j over the selected experts, no extra scaling;
* selection key: fl32(s + b) from fp32 s and fp32 b; Top-K ordered by
  (key descending, expert index ascending), so equal keys go to the lower index;
* "overloaded/underloaded": N_r * c_i compared with T * K (the batch mean);
  equal load leaves b_i unchanged; each change is one fp32 add of fl32(gamma);
* expert FFN: SwiGLU without biases, W_d (SiLU(W_g x) * (W_u x));
* FP8: OCP E4M3FN (largest finite 448, no infinities), scale = fl32(amax/448),
  code = round-to-nearest-even of fl32(x/scale), saturated at 448, sign copied;
  an all-zero tile has scale 0 and zero codes. In FP8 mode the oracle computes
  in float64 on dequantized operands, i.e. quantize -> dequantize at exactly
  the points where the recipe quantizes (u before GEMM1, every weight, h before
  GEMM2), and keeps the residual, gates and combine in float64.

All floating point is float64 except where a definition above rounds to fp32.
Every function is pinned by the tests (brute force, closed forms, invariants,
library cross-checks, finite differences) except seq_balance_loss, which is
"parity unpinned": the pages name the loss and its alpha but not its formula,
so its pins check only the reading's own closed forms and invariants.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0   # largest finite E4M3FN magnitude: exponent field 15, mantissa 6


# --------------------------------------------------------------------------- dtypes

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly: a bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_f64(x) -> np.ndarray:
    """Exact float64 value of an input stored as fp32, fp64, or bf16 bits (uint16)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported input dtype {x.dtype}")


# --------------------------------------------------------------------------- routing

def affinities(u, centroids, logit_offset=None) -> np.ndarray:
    """s_{i,t} = Sigmoid(u_t . e_i) in float64, [T, N_r].

    "รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2, the affinity definition; "Deepseek V3 国货之光 开源之光", Auxiliary-Loss-Free Load Balancing section:
    dot product of the hidden state with each routed expert's centroid, then a
    sigmoid. `logit_offset` [N_r] is a workload knob added to the logit before
    the sigmoid (used to make chosen experts hot); None in normal use.
    """
    logit = as_f64(u) @ as_f64(centroids).T
    if logit_offset is not None:
        logit = logit + as_f64(logit_offset)[None, :]
    return 1.0 / (1.0 + np.exp(-logit))


def selection_keys(s32, bias) -> np.ndarray:
    """key_{i,t} = fl32(s_{i,t} + b_i): fp32 affinity plus fp32 bias, one fp32 rounding.

    "รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2, eq. for g': the bias enters only the Top-K argument.
    """
    s32 = np.asarray(s32, dtype=np.float32)
    b32 = np.asarray(bias, dtype=np.float32)
    return s32 + b32[None, :]          # numpy fp32 add: IEEE round-to-nearest-even


def topk_select(keys, K: int) -> np.ndarray:
    """The K experts with the largest keys per token, ordered by (key desc, index asc). [T, K] int32.

    "รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2: Topk({s_j + b_j}, K_r). Ties go to the lower expert index.
    """
    keys = np.asarray(keys)
    T, N = keys.shape
    if not (1 <= K <= N):
        raise ValueError("K must be in [1, N_r]")
    index = np.broadcast_to(np.arange(N), (T, N))
    order = np.lexsort((index, -keys.astype(np.float64)), axis=-1)   # primary: -key, then index
    return order[:, :K].astype(np.int32)


def group_limited_select(keys, K: int, n_groups: int, topk_groups: int) -> np.ndarray:
    """Node-limited (group-limited) Top-K: a token's K experts come from at most topk_groups groups.

    "DeepSeek：AI 領域的重大突破與開源策略" (dev.clsung.tw), innovation table, Node-Limited
    Routing: each token goes to at most M nodes; "官方揭秘DeepSeek-V3模型训练全流程"
    ("官方揭秘DeepSeek-V3模型训练全流程") §2.2: at most 4 nodes. The experts are split into n_groups equal,
    contiguous groups (group g holds experts [g*N/G, (g+1)*N/G)). The pages do not say how
    the groups are chosen; reading taken:
      1. a group's score is the fp32 sum of its K/topk_groups largest keys, added in rank
         order (key desc, index asc), each addition rounded to fp32;
      2. the topk_groups groups with the largest scores are kept, equal scores going to the
         lower group index;
      3. the K experts are the Top-K (key desc, index asc) among the kept groups' experts.
    Returns [T, K] int32 in rank order, like topk_select.
    """
    keys = np.asarray(keys, dtype=np.float32)
    T, N = keys.shape
    G, M = int(n_groups), int(topk_groups)
    if G < 1 or N % G or not (1 <= M <= G) or K % M or K // M > N // G:
        raise ValueError("need N_r % n_groups == 0, 1 <= topk_groups <= n_groups, "
                         "K % topk_groups == 0 and K / topk_groups <= N_r / n_groups")
    gsz, per = N // G, K // M
    grouped = keys.reshape(T, G, gsz)
    ranked = np.sort(grouped, axis=2)[:, :, ::-1]         # values in descending order
    score = ranked[:, :, 0].copy()
    for j in range(1, per):
        score = (score + ranked[:, :, j]).astype(np.float32)
    gidx = np.broadcast_to(np.arange(G), (T, G))
    gorder = np.lexsort((gidx, -score.astype(np.float64)), axis=-1)[:, :M]
    allowed = np.zeros((T, G), dtype=bool)
    np.put_along_axis(allowed, gorder, True, axis=1)
    masked = np.where(np.repeat(allowed, gsz, axis=1), keys.astype(np.float64), -np.inf)
    return topk_select(masked, K)


def gates(s, idx) -> np.ndarray:
    """g_{t,k} = s_{t,idx_k} / sum_k' s_{t,idx_k'} in float64 (unbiased s).

    "รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2: g is g' normalised, g' = s on the selected experts;
    "Deepseek V3 国货之光 开源之光", Auxiliary-Loss-Free Load Balancing section: the bias does not enter the affinity used here.
    """
    s = as_f64(s)
    sel = np.take_along_axis(s, np.asarray(idx, dtype=np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(u, centroids, bias, K: int, logit_offset=None, affinity_in=None, n_groups: int = 1,
          topk_groups: int = 1) -> dict:
    """Affinity -> biased Top-K (optionally group-limited) -> normalised gates.

    From scratch (affinity_in None): s is the float64 sigmoid; the selection key
    uses fl32(s). With affinity_in (fp32 [T, N_r]) those values are s itself, which
    is how router stages are compared on identical affinities. n_groups > 1 selects
    with group_limited_select.
    """
    if affinity_in is None:
        s = affinities(u, centroids, logit_offset)
        s32 = s.astype(np.float32)
    else:
        s32 = np.asarray(affinity_in, dtype=np.float32)
        s = s32.astype(np.float64)
    keys = selection_keys(s32, bias)
    if n_groups > 1:
        idx = group_limited_select(keys, K, n_groups, topk_groups)
    else:
        idx = topk_select(keys, K)
    return {"s": s, "s32": s32, "keys": keys, "idx": idx, "gates": gates(s, idx)}


# --------------------------------------------------------------------------- dispatch

def dispatch(idx, N_r: int) -> dict:
    """Per-expert counts, offsets and the row permutation (expert ascending, token ascending).

    Single-GPU form of the "dispatch" step: every one of the T*K assignments
    gets a row (no dropping, "官方揭秘DeepSeek-V3模型训练全流程" §2.2). row_token[r] is the token of
    row r; slot_row[t*K + k] is the row that holds token t's k-th choice.
    """
    idx = np.asarray(idx)
    T, K = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    if flat.size and (flat.min() < 0 or flat.max() >= N_r):
        raise ValueError("expert index out of range")
    counts = np.bincount(flat, minlength=N_r).astype(np.int64)
    offsets = np.zeros(N_r + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable")          # slot t*K+k, grouped by expert, slots ascending
    row_token = (order // K).astype(np.int32)
    slot_row = np.empty(T * K, dtype=np.int32)
    slot_row[order] = np.arange(T * K, dtype=np.int32)
    return {"counts": counts.astype(np.int32), "offsets": offsets.astype(np.int32),
            "row_token": row_token, "slot_row": slot_row}


def dispatch_by_rank(idx, N_r: int, n_ranks: int) -> dict:
    """The send plan of an expert-parallel dispatch: one row per (token, destination rank).

    Experts are split evenly over n_ranks ranks (rank r owns experts [r*N_r/R, (r+1)*N_r/R)).
    A token whose K experts sit on m distinct ranks is sent m times, once per rank, however
    many of its experts that rank owns (the point of node-limited routing: "官方揭秘DeepSeek-V3
    模型训练全流程" ("官方揭秘DeepSeek-V3模型训练全流程") §2.2 and its communication bullet, at most 4 nodes per token).
    Send rows are ordered by rank, then token. Returns counts [R] (rows per rank), offsets
    [R+1], send_token [rows] and slot_send [T*K] (the row that carries token t to the rank of
    its k-th expert).
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, K = idx.shape
    R = int(n_ranks)
    if R < 1 or N_r % R:
        raise ValueError("n_ranks must divide N_r")
    if idx.size and (idx.min() < 0 or idx.max() >= N_r):
        raise ValueError("expert id out of range")
    rank = idx // (N_r // R)
    pairs = sorted({(int(rank[t, k]), t) for t in range(T) for k in range(K)})   # (rank, token) ascending
    row_of = {p: i for i, p in enumerate(pairs)}
    counts = np.bincount(np.array([p[0] for p in pairs], dtype=np.int64), minlength=R).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    send_token = np.array([p[1] for p in pairs], dtype=np.int32)
    slot_send = np.array([row_of[(int(rank[t, k]), t)] for t in range(T) for k in range(K)], dtype=np.int32)
    return {"counts": counts, "offsets": offsets, "send_token": send_token, "slot_send": slot_send}


def pack_fp8_payload(x, idx, N_r: int, n_ranks: int) -> dict:
    """FP8 dispatch payload: the send plan plus each send row as 1x128-tile E4M3 codes and scales.

    "官方揭秘DeepSeek-V3模型训练全流程" §4.3, low-precision storage and communication bullet: activations are partly
    quantized to FP8 for communication. Row r holds token send_token[r]'s activation quantized
    exactly as the FP8 GEMM input (quantize_tiles with 1x128 tiles).
    """
    plan = dispatch_by_rank(idx, N_r, n_ranks)
    x = np.asarray(x, dtype=np.float32)
    codes, scales = quantize_tiles(x[plan["send_token"]].reshape(-1, x.shape[1]), 1, 128)
    return {**plan, "codes": codes, "scales": scales}


def unpack_fp8_payload(codes, scales) -> np.ndarray:
    """Received rows back to fp32: fl32(decode(code) * scale), one rounding of an exact product."""
    return dequantize_tiles(codes, scales, 1, 128).astype(np.float32)


# --------------------------------------------------------------------------- FP8 E4M3FN

def _e4m3fn_value(c: np.ndarray) -> np.ndarray:
    """Value of E4M3FN codes from the bit fields: sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0; exponent 0 is subnormal, 2^-6 * m/8; 0x7F / 0xFF are NaN."""
    c = np.asarray(c, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where(s == 1, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


_E4M3_TABLE = _e4m3fn_value(np.arange(256))        # value of every code


def e4m3fn_decode(codes) -> np.ndarray:
    """Value of each E4M3FN code (float64); 0x7F / 0xFF are NaN."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.int64) & 0xFF]


def e4m3fn_encode(v) -> np.ndarray:
    """Round fp32 values to E4M3FN codes: nearest value, ties to the even code, saturate at 448.

    In the binade [2^e, 2^(e+1)), e >= -6, the E4M3FN values are k * 2^(e-3) for
    k = 8..15 and their codes are (e+6)*8 + k; below 2^-6 (subnormals, e taken as
    -6) they are k * 2^-9 with code k. So with e = max(floor(log2|v|), -6) and
    k = rint(|v| * 2^(3-e)) (round half to even; an even k is an even mantissa),
    the code is (e+6)*8 + k — k = 16 carries into the next binade by the same
    formula. Codes above 0x7E (448) saturate to 0x7E. The sign bit is copied from
    the input (-0 gives 0x80); NaN is never produced.
    """
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input to the E4M3 encoder")
    a = np.abs(v)
    e = np.where(a < np.float32(2.0 ** -6), -6, np.frexp(a)[1] - 1).astype(np.int64)   # a = f*2^x, f in [.5,1)
    k = np.rint(np.ldexp(a, (3 - e).astype(np.int32))).astype(np.int64)  # exact power-of-two scaling
    code = np.minimum((e + 6) * 8 + k, 0x7E)
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def quantize_tiles(x, tile_rows: int, tile_cols: int):
    """Per-tile online-absmax E4M3 quantization of a 2-D fp32 array.

    "官方揭秘DeepSeek-V3模型训练全流程" §4.3 (fine-grained 1x128 / 128x128 quantization, online max
    absolute value). Returns (codes uint8 [R, C], scales fp32 [R/tile_rows, C/tile_cols]).
    """
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    if R % tile_rows or C % tile_cols:
        raise ValueError("shape not a multiple of the tile")
    xt = x.reshape(R // tile_rows, tile_rows, C // tile_cols, tile_cols)
    amax = np.abs(xt).max(axis=(1, 3))
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)   # one correctly rounded fp32 division
    sc = scale[:, None, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(sc == 0, xt, xt / sc).astype(np.float32)  # fp32 division; zero tile keeps +-0
    return e4m3fn_encode(q).reshape(R, C), scale


def dequantize_tiles(codes, scales, tile_rows: int, tile_cols: int) -> np.ndarray:
    """decode(code) * scale per tile, float64 (exact: 4-bit x 24-bit significands)."""
    codes = np.asarray(codes)
    R, C = codes.shape
    vals = e4m3fn_decode(codes).reshape(R // tile_rows, tile_rows, C // tile_cols, tile_cols)
    sc = np.asarray(scales, np.float64)[:, None, :, None]
    return (vals * sc).reshape(R, C)


def fp8_roundtrip(x, tile_rows: int, tile_cols: int) -> np.ndarray:
    """deq(Q(fl32(x))): the value an FP8 GEMM operand stands for."""
    codes, scales = quantize_tiles(np.asarray(x, dtype=np.float32), tile_rows, tile_cols)
    return dequantize_tiles(codes, scales, tile_rows, tile_cols)


def fp8_roundtrip_row_blocks(x, block: int = 128) -> np.ndarray:
    """deq(Q(fl32(x))) with one scale per `block` consecutive rows of each column (128x1 tiles).

    The operand of a GEMM that reduces over rows (a weight gradient sums over the tokens of an
    expert) is quantized along that reduction; the rows run in the given order and the last tile
    holds the rows that remain (fewer than `block`). Zero rows appended to fill the last tile
    change no amax and are dropped again.
    """
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    Rp = -(-R // block) * block
    xp = np.zeros((Rp, C), dtype=np.float32)
    xp[:R] = x
    codes, scales = quantize_tiles(xp, block, 1)
    return dequantize_tiles(codes, scales, block, 1)[:R]


# --------------------------------------------------------------------------- expert FFN

def silu(z) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(x, w_gate, w_up, w_down, fp8: bool = False) -> np.ndarray:
    """FFN(x) = W_d (SiLU(W_g x) * (W_u x)), rows of x are tokens; float64.

    The pages name the expert FFN only as a symbol in the "รายงานเชิงเทคนิคของ DeepSeek-V3" h'_t
    equation; SwiGLU without biases is the reading taken. With fp8=True the
    weights are replaced by their 128x128-block FP8 values and h by its 1x128
    FP8 value before the down projection (x must already be the FP8 value of
    the GEMM1 input).
    """
    x = as_f64(x)
    wg, wu, wd = as_f64(w_gate), as_f64(w_up), as_f64(w_down)
    if fp8:
        wg, wu, wd = (fp8_roundtrip(w, 128, 128) for w in (wg, wu, wd))
    z = x @ wg.T
    v = x @ wu.T
    h = silu(z) * v
    if fp8:
        h = fp8_roundtrip(h, 1, 128)
    return h @ wd.T


def swiglu_ffn_backward(x, w_gate, w_up, w_down, dy, weight_grads: bool = True) -> dict:
    """Gradients of y = W_d (SiLU(W_g x) * (W_u x)) for the rows x, given dy (float64).

    Chain rule, with z = x W_g^T, v = x W_u^T, a = SiLU(z), h = a v, y = h W_d^T:
      dh = dy W_d,  dW_d = dy^T h,  dz = dh v SiLU'(z),  dv = dh a,
      dx = dz W_g + dv W_u,  dW_g = dz^T x,  dW_u = dv^T x,
    where SiLU'(z) = sigma(z) (1 + z (1 - sigma(z))).
    """
    x, wg, wu, wd, dy = (as_f64(a) for a in (x, w_gate, w_up, w_down, dy))
    z = x @ wg.T
    v = x @ wu.T
    sig = 1.0 / (1.0 + np.exp(-z))
    a = z * sig
    h = a * v
    dh = dy @ wd
    dz = dh * v * sig * (1.0 + z * (1.0 - sig))
    dv = dh * a
    out = {"dx": dz @ wg + dv @ wu, "z": z, "v": v, "h": h, "dh": dh, "dz": dz, "dv": dv}
    if weight_grads:
        out.update({"dW_gate": dz.T @ x, "dW_up": dv.T @ x, "dW_down": dy.T @ h})
    return out


def swiglu_ffn_backward_fp8(x, w_gate, w_up, w_down, dy) -> dict:
    """The SwiGLU FFN backward of swiglu_ffn_backward with every GEMM operand in E4M3 (float64).

    "官方揭秘DeepSeek-V3模型训练全流程" §4.3 trains with FP8 GEMMs: activations (and their
    gradients) in 1x128 tiles, weights in 128x128 blocks, fp32 accumulation; "support for
    transposed GEMM operations" (§4.5) is the pages' note that the backward needs operands
    quantized along another axis. Readings taken: each GEMM operand is quantized from its
    high-precision value along that GEMM's reduction dimension, so
      forward:   z = Q(x) Q(W_g)^T, v = Q(x) Q(W_u)^T      (x in 1x128 tiles along H)
      dgrad:     dh = Q(dy) Q(W_d)                          (dy in 1x128 tiles along H)
                 dx = Q(dz) Q(W_g) + Q(dv) Q(W_u)           (dz, dv in 1x128 tiles along I)
      wgrad:     dW_d = Qr(dy)^T Qr(h),  dW_g = Qr(dz)^T Qr(x),  dW_u = Qr(dv)^T Qr(x)
    with Q(W) the 128x128-block value (the same blocks serve W and W^T), Qr the 128x1 tiles of
    fp8_roundtrip_row_blocks over the rows in the given order, and the SwiGLU derivative taken
    in high precision: h = SiLU(z) v, dz = dh v SiLU'(z), dv = dh SiLU(z).
    Rows of x are the tokens of one expert in dispatch order.
    """
    x, wg, wu, wd, dy = (as_f64(a) for a in (x, w_gate, w_up, w_down, dy))
    wgq, wuq, wdq = (fp8_roundtrip(w, 128, 128) for w in (wg, wu, wd))
    xq = fp8_roundtrip(x, 1, 128)
    z = xq @ wgq.T
    v = xq @ wuq.T
    sig = 1.0 / (1.0 + np.exp(-z))
    a = z * sig
    h = a * v
    dh = fp8_roundtrip(dy, 1, 128) @ wdq
    dz = dh * v * sig * (1.0 + z * (1.0 - sig))
    dv = dh * a
    dx = fp8_roundtrip(dz, 1, 128) @ wgq + fp8_roundtrip(dv, 1, 128) @ wuq
    xr = fp8_roundtrip_row_blocks(x)
    return {"dx": dx, "z": z, "v": v, "h": h, "dh": dh, "dz": dz, "dv": dv,
            "dW_gate": fp8_roundtrip_row_blocks(dz).T @ xr,
            "dW_up": fp8_roundtrip_row_blocks(dv).T @ xr,
            "dW_down": fp8_roundtrip_row_blocks(dy).T @ fp8_roundtrip_row_blocks(h)}


# --------------------------------------------------------------------------- layer

def layer_forward(u, centroids, bias, K: int, routed, shared, *, fp8: bool = False,
                  logit_offset=None, affinity_in=None, tokens=None, workers: int = 1,
                  n_groups: int = 1, topk_groups: int = 1) -> dict:
    """h'_t = u_t + sum_shared FFN(u_t) + sum_i g_{i,t} FFN_i(u_t)  ("รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2).

    routed[e] -> (W_g [I,H], W_u [I,H], W_d [H,I]) for routed expert e; shared is a
    sequence of such triples. Weights may be fp32/fp64 arrays or bf16 bit arrays; a
    lazy `routed` lets callers stream one expert at a time. Routing and dispatch
    are computed for all T tokens; the FFNs and the output only for `tokens`
    (default: all). `workers` > 1 evaluates different experts on that many threads
    (each expert's arithmetic is unchanged). Returns routing, dispatch, per-token shared output,
    per-(token, k) routed outputs and the layer output, all float64. n_groups > 1 routes
    with group_limited_select.
    """
    u64 = as_f64(u)
    T = u64.shape[0]
    r = route(u64, centroids, bias, K, logit_offset, affinity_in, n_groups, topk_groups)
    N_r = np.asarray(centroids).shape[0] if affinity_in is None else np.asarray(affinity_in).shape[1]
    d = dispatch(r["idx"], N_r)
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    x = u64[toks]
    x_in = fp8_roundtrip(x, 1, 128) if fp8 else x
    y_shared = np.zeros_like(x)
    for (wg, wu, wd) in shared:
        y_shared += swiglu_ffn(x_in, wg, wu, wd, fp8=fp8)
    sel = r["idx"][toks]
    y_routed = np.zeros((len(toks), K, x.shape[1]))

    def expert(e):
        rt, rk = np.nonzero(sel == e)
        wg, wu, wd = routed[int(e)]
        return rt, rk, swiglu_ffn(x_in[rt], wg, wu, wd, fp8=fp8)

    experts = [int(e) for e in np.unique(sel)]
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(expert, experts))
    else:
        results = [expert(e) for e in experts]
    for rt, rk, y in results:
        y_routed[rt, rk] = y
    g = r["gates"][toks]
    out = x + y_shared + np.einsum("tk,tkh->th", g, y_routed)
    return {**r, **d, "tokens": toks, "y_shared": y_shared, "y_routed": y_routed, "out": out}


# --------------------------------------------------------------------------- bias update

def layer_backward(u, centroids, bias, K: int, routed, shared, dout, *, logit_offset=None,
                   affinity_in=None, n_groups: int = 1, topk_groups: int = 1, workers: int = 1,
                   weight_grads=True, fp8: bool = False) -> dict:
    """Gradients of the layer output ("รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2, h'_t) for an upstream dout, float64.

    out_t = u_t + sum_shared FFN(u_t) + sum_k g_{t,k} FFN_{idx_k}(u_t). The selection idx is
    piecewise constant in u, e and b, so no gradient flows through it, and b (which only
    selects: "Deepseek V3 国货之光 开源之光", Auxiliary-Loss-Free Load Balancing section) gets none. With S_t = sum_k s_{t,idx_k}:
      dy_{t,k}   = g_{t,k} dout_t                  (into expert idx_k's FFN backward)
      dg_{t,k}   = dout_t . y_{t,k}
      ds_{t,k}   = (dg_{t,k} - sum_j g_{t,j} dg_{t,j}) / S_t
      dlogit_{t,k} = ds_{t,k} s (1 - s)  at s = s_{t,idx_k}   (s = sigmoid(logit))
      du_t      = dout_t + dx_shared + sum_k dx_{t,k} + sum_k dlogit_{t,k} e_{idx_k}
      de_i      = sum over (t, k) with idx_k = i of dlogit_{t,k} u_t.
    s comes from route(): the float64 sigmoid, or affinity_in when given (then the router terms
    use those values of s and still need centroids). Returns du, dcentroids (None without
    centroids), routed gradients {e: (dW_g, dW_u, dW_d)} for experts with rows, shared gradients,
    dgate [T,K], dlogit [T,K], the routing and every expert's per-row output y [T,K,H].
    weight_grads: True (all experts), False (none) or a collection of expert ids whose weight
    gradients are formed (the other quantities never depend on them).
    fp8: the FP8 layer: y from the FP8 forward (swiglu_ffn with fp8=True on the 1x128 value of
    u) and every expert's backward by swiglu_ffn_backward_fp8, its rows in dispatch order
    (token ascending; the shared expert takes all T tokens in order).
    """
    u64 = as_f64(u)
    dout = as_f64(dout)
    T, H = u64.shape
    r = route(u64, centroids, bias, K, logit_offset, affinity_in, n_groups, topk_groups)
    idx, g, s = r["idx"], r["gates"], r["s"]
    du = dout.copy()
    shared_grads = []
    want = (lambda e: True) if weight_grads is True else (
        (lambda e: False) if weight_grads is False else (lambda e, sel=set(int(x) for x in weight_grads): e in sel))
    def ffn_bwd(x, wg, wu, wd, dy, wgrads):
        if fp8:
            return swiglu_ffn_backward_fp8(x, wg, wu, wd, dy)
        return swiglu_ffn_backward(x, wg, wu, wd, dy, weight_grads=wgrads)

    for (wg, wu, wd) in shared:
        b = ffn_bwd(u64, wg, wu, wd, dout, weight_grads is not False)
        du += b["dx"]
        shared_grads.append((b["dW_gate"], b["dW_up"], b["dW_down"])
                            if "dW_gate" in b and weight_grads is not False else None)

    def expert(e):
        rt, rk = np.nonzero(idx == e)       # rows of expert e in dispatch order (token ascending)
        wg, wu, wd = routed[int(e)]
        x = u64[rt]
        y = swiglu_ffn(fp8_roundtrip(x, 1, 128) if fp8 else x, wg, wu, wd, fp8=fp8)
        b = ffn_bwd(x, wg, wu, wd, g[rt, rk][:, None] * dout[rt], want(int(e)))
        if not want(int(e)):
            b.pop("dW_gate", None)
        return int(e), rt, rk, y, b

    experts = [int(e) for e in np.unique(idx)]
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(expert, experts))
    else:
        results = [expert(e) for e in experts]
    y_routed = np.zeros((T, K, H))
    grads = {}
    for e, rt, rk, y, b in results:
        y_routed[rt, rk] = y
        np.add.at(du, rt, b["dx"])
        if "dW_gate" in b:
            grads[e] = (b["dW_gate"], b["dW_up"], b["dW_down"])
    dgate = np.einsum("th,tkh->tk", dout, y_routed)
    s_sel = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    S = s_sel.sum(axis=1, keepdims=True)
    ds = (dgate - (g * dgate).sum(axis=1, keepdims=True)) / S
    dlogit = ds * s_sel * (1.0 - s_sel)
    dE = None
    if centroids is not None:
        E = as_f64(centroids)
        du += np.einsum("tk,tkh->th", dlogit, E[idx])
        dE = np.zeros_like(E)
        np.add.at(dE, idx.reshape(-1), dlogit.reshape(-1, 1) * np.repeat(u64, K, axis=0))
    return {"du": du, "dcentroids": dE, "routed": grads, "shared": shared_grads, "dgate": dgate,
            "dlogit": dlogit, "idx": idx, "gates": g, "s": s, "y_routed": y_routed}


def seq_balance_loss(s, idx, K: int, seq_len: int, alpha: float = 1e-4) -> np.ndarray:
    """Sequence-wise balance loss, one value per sequence of seq_len consecutive tokens (float64).

    PARITY UNPINNED: the pages give only that a very small sequence-wise balance loss with
    alpha = 0.0001 complements the bias rule ("รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2, last sentence) to stop
    extreme imbalance inside one sequence ("官方揭秘DeepSeek-V3模型训练全流程" §2.2); its formula is not on the pages.
    Reading taken, the usual MoE balance loss applied within each sequence of L tokens:
      f_i = N_r / (K L) * #{t in seq : i among the K selected}
      P_i = (1 / L) * sum_{t in seq} s_{i,t} / sum_j s_{j,t}
      L_seq = alpha * sum_i f_i P_i
    The last sequence may be shorter (L is its own length).
    """
    s = as_f64(s)
    idx = np.asarray(idx, dtype=np.int64)
    T, N_r = s.shape
    out = []
    for t0 in range(0, T, seq_len):
        sl = slice(t0, min(T, t0 + seq_len))
        L = sl.stop - sl.start
        f = np.bincount(idx[sl].reshape(-1), minlength=N_r) * (N_r / (K * L))
        P = (s[sl] / s[sl].sum(axis=1, keepdims=True)).mean(axis=0)
        out.append(alpha * float((f * P).sum()))
    return np.array(out)


def bias_update(bias, counts, T: int, K: int, gamma: float = 1e-3) -> np.ndarray:
    """End-of-step update: b_i <- b_i - gamma if expert i is overloaded, + gamma if underloaded.

    "รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2 (gamma = 0.001); "Deepseek V3 国货之光 开源之光", Auxiliary-Loss-Free Load Balancing section. Load is
    compared with the batch mean T*K/N_r as N_r*c_i vs T*K (integers); equal
    load leaves b_i unchanged. fp32 storage and one fp32 add per step.
    """
    b = np.asarray(bias, dtype=np.float32).copy()
    c = np.asarray(counts, dtype=np.int64)
    N_r = b.shape[0]
    g = np.float32(gamma)
    over = N_r * c > T * K
    under = N_r * c < T * K
    b[over] = b[over] - g
    b[under] = b[under] + g
    return b


def load_stats(counts, T: int, K: int) -> dict:
    """max/mean and min/mean expert load of one step."""
    c = np.asarray(counts, dtype=np.float64)
    mean = T * K / c.shape[0]
    return {"max_over_mean": float(c.max() / mean), "min_over_mean": float(c.min() / mean)}
