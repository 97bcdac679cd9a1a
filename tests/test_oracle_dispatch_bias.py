"""Pins for the oracle's dispatch (counts / offsets / permutation) and bias update (CPU only)."""
import numpy as np
import pytest

import oracle
from layouts import dispatch_with_shared


def _brute_dispatch(idx, N_r):
    T, K = idx.shape
    rows = []                                   # (expert ascending, token ascending)
    for e in range(N_r):
        for t in range(T):
            for k in range(K):
                if idx[t, k] == e:
                    rows.append((t, k))
    row_token = [t for t, _ in rows]
    slot_row = [0] * (T * K)
    for r, (t, k) in enumerate(rows):
        slot_row[t * K + k] = r
    counts = [sum(1 for t in range(T) for k in range(K) if idx[t, k] == e) for e in range(N_r)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    return counts, offsets, row_token, slot_row


@pytest.mark.parametrize("T,N_r,K", [(1, 4, 1), (7, 5, 2), (33, 16, 4), (64, 16, 2), (20, 8, 8)])
def test_dispatch_brute_force(T, N_r, K):
    rng = np.random.default_rng(T * 7 + K)
    idx = np.stack([rng.permutation(N_r)[:K] for _ in range(T)]).astype(np.int32)
    d = oracle.dispatch(idx, N_r)
    counts, offsets, row_token, slot_row = _brute_dispatch(idx, N_r)
    assert list(d["counts"]) == counts
    assert list(d["offsets"]) == offsets
    assert list(d["row_token"]) == row_token
    assert list(d["slot_row"]) == slot_row


def test_dispatch_invariants_and_empty_experts():
    rng = np.random.default_rng(1)
    T, N_r, K = 300, 32, 3
    idx = np.stack([rng.choice(N_r // 2, K, replace=False) for _ in range(T)]).astype(np.int32)  # half the experts unused
    d = oracle.dispatch(idx, N_r)
    assert d["counts"].sum() == T * K and d["offsets"][-1] == T * K
    assert (d["counts"][N_r // 2:] == 0).all()
    # slot_row and row_token are mutually consistent bijections
    assert sorted(d["slot_row"]) == list(range(T * K))
    for t in range(T):
        for k in range(K):
            r = d["slot_row"][t * K + k]
            assert d["row_token"][r] == t
            assert d["offsets"][idx[t, k]] <= r < d["offsets"][idx[t, k] + 1]
    # within each expert segment tokens ascend strictly
    for e in range(N_r):
        seg = d["row_token"][d["offsets"][e]:d["offsets"][e + 1]]
        assert (np.diff(seg) > 0).all()


def test_dispatch_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([[0, 4]]), 4)


# ----------------------------------------------------------------------------- bias update

def test_bias_sign_rule_against_load():
    rng = np.random.default_rng(2)
    N_r, T, K = 64, 256, 4                      # mean load 16
    counts = rng.integers(0, 40, N_r)
    counts[:3] = 16                             # exactly mean
    b0 = (rng.random(N_r) * 0.1 - 0.05).astype(np.float32)
    b1 = oracle.bias_update(b0, counts, T, K, 1e-3)
    d = np.sign(b1.astype(np.float64) - b0.astype(np.float64))
    assert (d == -np.sign(counts - 16)).all()   # overloaded down, underloaded up, equal unchanged
    assert (b1[:3] == b0[:3]).all()


def test_bias_first_step_from_zero_is_exactly_gamma():
    g = np.float32(1e-3)
    b = oracle.bias_update(np.zeros(4, np.float32), np.array([0, 10, 1, 2]), 13, 1, 1e-3)
    # mean = 13/4 = 3.25: every expert except #1 is under-loaded
    assert b.dtype == np.float32
    assert list(b) == [g, -g, g, g]


def test_bias_n_steps_fixed_routing_closed_form():
    # With the same counts every step, step n adds +-fl32(gamma) n times in fp32:
    # |b_n - n*gamma| stays within n rounding errors of size ulp(b_n)/2, and b_n is monotone.
    counts = np.array([5, 1, 3, 3])             # mean 3 (T=4, K=3, N_r=4)
    b = np.zeros(4, np.float32)
    hist = [b]
    for n in range(1, 301):
        b = oracle.bias_update(b, counts, 4, 3, 1e-3)
        hist.append(b)
        bound = n * float(np.spacing(np.float32(n * 1e-3)))
        assert abs(float(b[0]) + n * float(np.float32(1e-3))) <= bound
        assert abs(float(b[1]) - n * float(np.float32(1e-3))) <= bound
        assert b[2] == 0 and b[3] == 0
    h = np.array(hist)
    assert (np.diff(h[:, 0]) < 0).all() and (np.diff(h[:, 1]) > 0).all()


def test_load_stats():
    s = oracle.load_stats(np.array([8, 0, 4, 4]), 4, 4)
    assert s["max_over_mean"] == 2.0 and s["min_over_mean"] == 0.0


def test_dispatch_with_shared_group_brute_force():
    rng = np.random.default_rng(4)
    T, N_r, K = 21, 6, 3
    idx = np.stack([rng.permutation(N_r)[:K] for _ in range(T)]).astype(np.int32)
    d = dispatch_with_shared(idx, N_r, T)
    # group 0 = the shared expert with every token, then routed expert e as group e + 1
    groups = [[t for t in range(T)]] + [[t for t in range(T) for k in range(K) if idx[t, k] == e] for e in range(N_r)]
    flat = [t for grp in groups for t in grp]
    assert list(d["row_token"]) == flat
    bounds = [0]
    for grp in groups:
        bounds.append(bounds[-1] + len(grp))
    assert list(d["offsets"]) == bounds
    for t in range(T):
        for k in range(K):
            r = d["slot_row"][t * K + k]
            assert flat[r] == t and bounds[idx[t, k] + 1] <= r < bounds[idx[t, k] + 2]
    assert list(d["counts"]) == [len(g) for g in groups[1:]]
