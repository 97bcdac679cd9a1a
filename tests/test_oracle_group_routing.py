"""Pins for the oracle's group-limited (node-limited) Top-K selection (CPU only).

Node-limited routing: "DeepSeek：AI 領域的重大突破與開源策略" (dev.clsung.tw), innovation table,
and "官方揭秘DeepSeek-V3模型训练全流程" (youleyou.com) §2.2 (at most 4 nodes per token). The group
score (fp32 sum of a group's K/M largest keys) is this library's reading; the pins below check the
oracle against that rule written as plain loops, hand-worked cases, reductions to ungrouped Top-K
and invariants.
"""
import numpy as np
import pytest

import oracle


def _brute(keys, K, G, M):
    """The selection rule spelled out with Python loops and explicit comparisons."""
    T, N = keys.shape
    gsz, per = N // G, K // M
    out = np.zeros((T, K), dtype=np.int32)
    for t in range(T):
        scores = []
        for g in range(G):
            vals = [float(keys[t, e]) for e in range(g * gsz, (g + 1) * gsz)]
            best = []
            for _ in range(per):                      # `per` largest values, largest first
                bi = None
                for i, v in enumerate(vals):
                    if i in best:
                        continue
                    if bi is None or v > vals[bi]:
                        bi = i
                best.append(bi)
            acc = np.float32(vals[best[0]])
            for i in best[1:]:
                acc = np.float32(acc + np.float32(vals[i]))
            scores.append(acc)
        kept = []
        for _ in range(M):                            # best group, equal scores -> lower index
            bg = None
            for g in range(G):
                if g in kept:
                    continue
                if bg is None or scores[g] > scores[bg]:
                    bg = g
            kept.append(bg)
        chosen = []
        for k in range(K):                            # best allowed expert, ties -> lower index
            be = None
            for e in range(N):
                if e // gsz not in kept or e in chosen:
                    continue
                if be is None or keys[t, e] > keys[t, be]:
                    be = e
            chosen.append(be)
        out[t] = chosen
    return out


@pytest.mark.parametrize("N,G,M,K", [(8, 4, 2, 4), (16, 4, 2, 2), (12, 3, 1, 3), (32, 8, 4, 8),
                                     (24, 6, 3, 6), (16, 8, 8, 8), (64, 8, 4, 8)])
def test_group_limited_matches_loops(N, G, M, K):
    rng = np.random.default_rng(N * 31 + G * 7 + M)
    T = 60
    # keys from a small set of fp32 values, so equal keys and equal group scores are frequent
    keys = rng.choice(np.float32([0.125, 0.25, 0.375, 0.5, 0.5625, 0.75, 1.0]), size=(T, N)).astype(np.float32)
    keys[::5] = rng.random((len(keys[::5]), N)).astype(np.float32)   # and some continuous rows
    got = oracle.group_limited_select(keys, K, G, M)
    assert np.array_equal(got, _brute(keys, K, G, M))


def test_group_limit_changes_the_choice_hand_example():
    # groups of two: g0 = {0,1}, g1 = {2,3}, g2 = {4,5}, g3 = {6,7}; M = 2 groups, K = 4 (2 per group)
    keys = np.float32([[0.9, 0.1, 0.8, 0.75, 0.85, 0.05, 0.3, 0.2]])
    # scores: g0 0.9+0.1, g1 0.8+0.75 = 1.55, g2 0.85+0.05 = 0.9, g3 0.5 -> keep g1, g0
    assert oracle.group_limited_select(keys, 4, 4, 2).tolist() == [[0, 2, 3, 1]]
    # without the limit expert 4 (0.85) would be second
    assert oracle.topk_select(keys, 4).tolist() == [[0, 4, 2, 3]]


def test_equal_group_scores_go_to_the_lower_group():
    keys = np.float32([[0.5, 0.25, 0.25, 0.5, 0.7, 0.05]])   # g0 = 0.75, g1 = 0.75, g2 = 0.75
    assert oracle.group_limited_select(keys, 2, 3, 1).tolist() == [[0, 1]]


def test_one_expert_per_group_reduces_to_plain_topk():
    # G = N_r and K = M: each group is one expert and its score is its key
    rng = np.random.default_rng(5)
    keys = rng.choice(np.float32([0.1, 0.2, 0.3, 0.4]), size=(50, 16)).astype(np.float32)
    assert np.array_equal(oracle.group_limited_select(keys, 4, 16, 4), oracle.topk_select(keys, 4))


def test_keeping_every_group_reduces_to_plain_topk():
    rng = np.random.default_rng(6)
    keys = rng.random((40, 32)).astype(np.float32)
    assert np.array_equal(oracle.group_limited_select(keys, 8, 8, 8), oracle.topk_select(keys, 8))


def test_group_limited_invariants_at_v3_shape():
    rng = np.random.default_rng(7)
    T, N, G, M, K = 300, 256, 8, 4, 8
    s = rng.random((T, N)).astype(np.float32)
    b = (rng.random(N).astype(np.float32) - 0.5) * np.float32(0.02)
    keys = oracle.selection_keys(s, b)
    idx = oracle.group_limited_select(keys, K, G, M)
    gsz = N // G
    for t in range(T):
        groups = set(int(e) // gsz for e in idx[t])
        assert len(groups) <= M
        assert len(set(idx[t].tolist())) == K
        # the chosen experts are the K best of the groups they come from, in rank order
        allowed = [e for e in range(N) if e // gsz in groups]
        best = sorted(allowed, key=lambda e: (-float(keys[t, e]), e))[:K]
        assert idx[t].tolist() == best
    # routing through route(): gates still normalise the unbiased s over the chosen experts
    r = oracle.route(None, None, b, K, affinity_in=s, n_groups=G, topk_groups=M)
    assert np.array_equal(r["idx"], idx)
    assert np.allclose(r["gates"].sum(axis=1), 1.0)


@pytest.mark.parametrize("N,G,M,K", [(16, 3, 1, 2), (16, 4, 3, 4), (16, 4, 1, 8), (16, 4, 5, 5)])
def test_group_limited_rejects_bad_shapes(N, G, M, K):
    with pytest.raises(ValueError):
        oracle.group_limited_select(np.zeros((1, N), np.float32), K, G, M)
