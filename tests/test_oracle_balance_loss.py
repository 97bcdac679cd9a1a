"""Pins for the oracle's sequence-wise balance loss (CPU only). PARITY UNPINNED: the pages give the
loss's purpose and alpha = 0.0001 ("รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2; "官方揭秘DeepSeek-V3模型训练全流程" §2.2) but not its formula, so
these pins check the closed forms and invariants of the reading taken, not the pages."""
import numpy as np
import pytest

import oracle


def test_uniform_routing_and_affinities_give_alpha():
    # every expert taken equally often and equal affinities: f_i = 1, P_i = 1/N_r, sum_i f_i P_i = 1
    N_r, K, L = 8, 2, 16
    idx = np.array([[(2 * t) % N_r, (2 * t + 1) % N_r] for t in range(L)])
    s = np.full((L, N_r), 0.3)
    assert oracle.seq_balance_loss(s, idx, K, L, alpha=1e-4) == pytest.approx([1e-4], rel=1e-15)


def test_all_tokens_on_the_same_experts_with_matching_affinity():
    # K experts take every token and hold all the affinity mass: f = N_r / K on them, P = 1/K each
    N_r, K, L = 16, 4, 10
    idx = np.tile(np.arange(K), (L, 1))
    s = np.zeros((L, N_r))
    s[:, :K] = 0.5
    assert oracle.seq_balance_loss(s, idx, K, L, alpha=1.0) == pytest.approx([N_r / K], rel=1e-15)


def test_sequences_are_independent_and_last_may_be_short():
    rng = np.random.default_rng(2)
    T, N_r, K, L = 23, 12, 3, 8
    s = rng.random((T, N_r))
    idx = np.stack([rng.permutation(N_r)[:K] for _ in range(T)])
    full = oracle.seq_balance_loss(s, idx, K, L)
    parts = [oracle.seq_balance_loss(s[a:a + L], idx[a:a + L], K, L)[0] for a in (0, 8, 16)]
    assert np.allclose(full, parts, rtol=1e-14, atol=0)
    assert full.shape == (3,)


def test_invariant_to_scaling_each_tokens_affinities():
    rng = np.random.default_rng(3)
    s = rng.random((20, 10))
    idx = np.stack([rng.permutation(10)[:2] for _ in range(20)])
    scaled = s * rng.uniform(0.5, 2.0, size=(20, 1))
    assert np.allclose(oracle.seq_balance_loss(s, idx, 2, 5), oracle.seq_balance_loss(scaled, idx, 2, 5), rtol=1e-13)
