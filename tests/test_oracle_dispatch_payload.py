"""Pins for the oracle's expert-parallel send plan and FP8 dispatch payload (CPU only).

"官方揭秘DeepSeek-V3模型训练全流程" (youleyou.com) §2.2 / §4.2: a token is sent to a node once
(at most 4 nodes per token); §4.3: activations are partly quantized to FP8 for communication.
"""
import numpy as np
import pytest

import oracle


def _brute_plan(idx, N_r, R):
    T, K = idx.shape
    per = N_r // R
    rows = []
    for r in range(R):                      # rank ascending
        for t in range(T):                  # token ascending
            if any(idx[t, k] // per == r for k in range(K)):
                rows.append((r, t))
    counts = [sum(1 for rr, _ in rows if rr == r) for r in range(R)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    slot = []
    for t in range(T):
        for k in range(K):
            slot.append(rows.index((idx[t, k] // per, t)))
    return counts, offsets, [t for _, t in rows], slot


@pytest.mark.parametrize("T,N_r,K,R", [(1, 4, 1, 2), (9, 16, 4, 4), (33, 32, 8, 8), (20, 12, 3, 3),
                                       (50, 64, 6, 1), (17, 16, 16, 16), (40, 256, 8, 8)])
def test_send_plan_brute_force(T, N_r, K, R):
    rng = np.random.default_rng(T * 3 + R)
    idx = np.stack([rng.permutation(N_r)[:K] for _ in range(T)]).astype(np.int32)
    d = oracle.dispatch_by_rank(idx, N_r, R)
    counts, offsets, send_token, slot = _brute_plan(idx, N_r, R)
    assert d["counts"].tolist() == counts
    assert d["offsets"].tolist() == offsets
    assert d["send_token"].tolist() == send_token
    assert d["slot_send"].tolist() == slot


def test_one_expert_per_rank_is_the_expert_dispatch():
    rng = np.random.default_rng(3)
    idx = np.stack([rng.permutation(32)[:6] for _ in range(70)]).astype(np.int32)
    d = oracle.dispatch_by_rank(idx, 32, 32)
    e = oracle.dispatch(idx, 32)
    assert np.array_equal(d["counts"], e["counts"]) and np.array_equal(d["offsets"], e["offsets"])
    assert np.array_equal(d["send_token"], e["row_token"]) and np.array_equal(d["slot_send"], e["slot_row"])


def test_single_rank_sends_every_token_once():
    idx = np.array([[3, 1], [0, 2], [2, 3]], dtype=np.int32)
    d = oracle.dispatch_by_rank(idx, 4, 1)
    assert d["send_token"].tolist() == [0, 1, 2]
    assert d["slot_send"].tolist() == [0, 0, 1, 1, 2, 2]


def test_hand_example_dedup_per_rank():
    # 8 experts on 4 ranks (2 each); token 0 -> experts 1, 0 (both rank 0): one row;
    # token 1 -> experts 7, 2 (ranks 3, 1): two rows
    idx = np.array([[1, 0], [7, 2]], dtype=np.int32)
    d = oracle.dispatch_by_rank(idx, 8, 4)
    assert d["counts"].tolist() == [1, 1, 0, 1]
    assert d["send_token"].tolist() == [0, 1, 1]          # rank 0: t0; rank 1: t1; rank 3: t1
    assert d["slot_send"].tolist() == [0, 0, 2, 1]


def test_rows_per_token_is_the_number_of_distinct_ranks():
    rng = np.random.default_rng(5)
    T, N_r, K, R = 200, 256, 8, 8
    idx = np.stack([rng.permutation(N_r)[:K] for _ in range(T)]).astype(np.int32)
    d = oracle.dispatch_by_rank(idx, N_r, R)
    per_token = np.bincount(d["send_token"], minlength=T)
    assert np.array_equal(per_token, [len(set(row // (N_r // R))) for row in idx])
    assert d["offsets"][-1] <= T * min(K, R)


def test_payload_codes_are_the_gathered_gemm_input_codes():
    rng = np.random.default_rng(6)
    T, H, N_r, K, R = 24, 512, 32, 4, 4
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[3, :128] *= 80.0
    idx = np.stack([rng.permutation(N_r)[:K] for _ in range(T)]).astype(np.int32)
    p = oracle.pack_fp8_payload(x, idx, N_r, R)
    codes, scales = oracle.quantize_tiles(x, 1, 128)          # 1x128 tiles: rows quantize independently
    assert np.array_equal(p["codes"], codes[p["send_token"]])
    assert np.array_equal(p["scales"], scales[p["send_token"]])


def test_unpack_closed_form_and_lossless_rows():
    codes = np.zeros((1, 128), np.uint8)
    codes[0, :4] = [0x38, 0xB8, 0x7E, 0x01]                   # 1.0, -1.0, 448, 2^-9
    out = oracle.unpack_fp8_payload(codes, np.float32([[0.5]]))
    assert out[0, :4].tolist() == [0.5, -0.5, 224.0, 2.0 ** -10]
    assert out.dtype == np.float32
    # rows on the E4M3 grid times a power of two come back exactly
    grid = oracle.e4m3fn_decode(np.arange(0, 0x7F, dtype=np.uint8))
    row = np.concatenate([grid, -grid[:128 - grid.size]]).astype(np.float32)[None, :128] * np.float32(0.25)
    row[0, 126] = 448 * 0.25                                  # amax -> scale exactly 0.25
    p = oracle.pack_fp8_payload(row, np.array([[0]]), 2, 2)
    assert np.array_equal(oracle.unpack_fp8_payload(p["codes"], p["scales"]), row)
