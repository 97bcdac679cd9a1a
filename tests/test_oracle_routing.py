"""Pins for the oracle's router: affinity, biased Top-K, gates (CPU only).

Each check is tied to something other than the oracle's own code: closed
forms, brute force over all K-subsets, exact rational arithmetic, or the
behaviour the pages state ("รายงานเชิงเทคนิคของ DeepSeek-V3" Method §2; "Deepseek V3 国货之光 开源之光", Auxiliary-Loss-Free Load Balancing section).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_pages_constants_fixture(golden_dir):
    c = json.load(open(os.path.join(golden_dir, "pages_constants.json")))
    assert c["gamma"]["value"] == 1e-3
    assert c["act_tile"]["value"] == [1, 128] and c["weight_block"]["value"] == [128, 128]
    assert oracle.E4M3_MAX == 448.0
    import inspect
    assert inspect.signature(oracle.bias_update).parameters["gamma"].default == c["gamma"]["value"]


def test_affinity_closed_forms():
    # u . e = 0 gives exactly 0.5; u . e = +-2 gives 1/(1+e^-+2), and s(x) + s(-x) = 1.
    u = np.array([[1.0, -1.0]])
    E = np.array([[1.0, 1.0], [2.0, 0.0], [0.0, 2.0]])
    s = oracle.affinities(u, E)
    assert s[0, 0] == 0.5
    assert s[0, 1] == pytest.approx(1 / (1 + math.exp(-2)), rel=1e-15)
    assert s[0, 2] == pytest.approx(1 / (1 + math.exp(2)), rel=1e-15)
    assert s[0, 1] + s[0, 2] == pytest.approx(1.0, abs=1e-15)
    # logit offset is added before the sigmoid
    s2 = oracle.affinities(u, E, logit_offset=np.array([2.0, 0.0, 0.0]))
    assert s2[0, 0] == pytest.approx(1 / (1 + math.exp(-2)), rel=1e-15)


def _fp32_round_exact(q: Fraction) -> np.float32:
    """Round an exact rational to fp32 (nearest, ties to even) without float arithmetic on q."""
    f = np.float32(float(q))                     # a neighbour (within one ulp)
    cands = {f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))}
    best = sorted(cands, key=lambda c: (abs(Fraction(float(c)) - q),
                                        int(np.array(c, np.float32).view(np.uint32)) & 1))
    return best[0]


def test_selection_key_is_one_fp32_rounding():
    rng = np.random.default_rng(7)
    s = rng.random((50, 9)).astype(np.float32)
    b = (rng.random(9) * 0.02 - 0.01).astype(np.float32)
    b[0] = np.float32(1e-30)                     # far below s: rounding dominated
    b[1] = np.float32(2.0 ** -25)                # near half an ulp of s
    keys = oracle.selection_keys(s, b)
    assert keys.dtype == np.float32
    for t in range(s.shape[0]):
        for i in range(s.shape[1]):
            exact = Fraction(float(s[t, i])) + Fraction(float(b[i]))
            assert keys[t, i] == _fp32_round_exact(exact)


def _brute_topk(keys_row, K):
    """The unique K-subset S with key_i > key_j, or equal keys and i < j, for all i in S, j not in S."""
    N = len(keys_row)
    beats = lambda i, j: keys_row[i] > keys_row[j] or (keys_row[i] == keys_row[j] and i < j)
    valid = [S for S in itertools.combinations(range(N), K)
             if all(beats(i, j) for i in S for j in range(N) if j not in S)]
    assert len(valid) == 1
    return sorted(valid[0], key=lambda i: (-float(keys_row[i]), i))


@pytest.mark.parametrize("N,K,levels", [(4, 1, 0), (5, 2, 3), (6, 3, 2), (7, 4, 0), (8, 2, 4), (8, 8, 3)])
def test_topk_brute_force(N, K, levels):
    rng = np.random.default_rng(N * 100 + K)
    keys = rng.random((40, N)).astype(np.float32)
    if levels:
        keys = (np.floor(keys * levels) / levels).astype(np.float32)   # many exact ties
    idx = oracle.topk_select(keys, K)
    for t in range(keys.shape[0]):
        assert list(idx[t]) == _brute_topk(keys[t], K)


def test_topk_all_equal_keys_gives_lowest_indices():
    keys = np.full((5, 16), 0.25, dtype=np.float32)
    idx = oracle.topk_select(keys, 4)
    assert (idx == np.arange(4)).all()


def test_bias_dominance_closed_form():
    # s in (0,1): a bias of +1 puts an expert above every unbiased one; -1 below.
    rng = np.random.default_rng(3)
    s = rng.random((100, 16)).astype(np.float32) * 0.98 + 0.01
    b = np.zeros(16, np.float32)
    J = [3, 11, 14]
    L = [0, 1, 2, 5]
    b[J] = 1.0
    b[L] = -1.0
    r = oracle.route(None, None, b, 6, affinity_in=s)
    for t in range(100):
        assert set(r["idx"][t, :3]) == set(J)
        assert not set(r["idx"][t]) & set(L)


def test_gates_sum_to_one_and_positive():
    rng = np.random.default_rng(5)
    u = rng.standard_normal((64, 32))
    E = rng.standard_normal((16, 32)) / math.sqrt(32)
    b = (rng.random(16) * 0.2 - 0.1).astype(np.float32)
    r = oracle.route(u, E, b, 4)
    assert np.all(r["gates"] > 0)
    assert np.max(np.abs(r["gates"].sum(axis=1) - 1.0)) <= 1e-15


def test_bias_changes_selection_never_gates():
    # Databean ALF section: b only chooses experts; the affinity used downstream is unbiased.
    rng = np.random.default_rng(11)
    s = rng.random((500, 16)).astype(np.float32)
    b0 = np.zeros(16, np.float32)
    b1 = (rng.random(16) * 0.3 - 0.15).astype(np.float32)
    r0 = oracle.route(None, None, b0, 3, affinity_in=s)
    r1 = oracle.route(None, None, b1, 3, affinity_in=s)
    same = np.array([set(a) == set(c) for a, c in zip(r0["idx"], r1["idx"])])
    assert same.any() and (~same).any()          # the bias does change some selections
    for t in np.nonzero(same)[0]:
        g0 = dict(zip(r0["idx"][t], r0["gates"][t]))
        g1 = dict(zip(r1["idx"][t], r1["gates"][t]))
        for e in g0:
            assert g0[e] == g1[e]                # bitwise identical gate values


def test_gates_ignore_bias_closed_form():
    # hand example: s = [0.5, 0.9, 0.2], K = 2, biases flip which pair is chosen
    s = np.array([[0.5, 0.9, 0.2]], np.float32)
    r = oracle.route(None, None, np.zeros(3, np.float32), 2, affinity_in=s)
    assert list(r["idx"][0]) == [1, 0]
    assert r["gates"][0, 0] == pytest.approx(float(np.float32(0.9)) / (float(np.float32(0.9)) + 0.5), rel=1e-15)
    r = oracle.route(None, None, np.array([0, -0.5, 0.5], np.float32), 2, affinity_in=s)
    assert list(r["idx"][0]) == [2, 0]           # keys 0.5, 0.4, 0.7
    s2, s0 = float(np.float32(0.2)), 0.5
    assert r["gates"][0] == pytest.approx([s2 / (s2 + s0), s0 / (s2 + s0)], rel=1e-15)
