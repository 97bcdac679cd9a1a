"""Pins for the oracle's layer backward (CPU only).

The analytic gradients of oracle.layer_backward are checked against central finite differences
of oracle.layer_forward (the forward is pinned elsewhere), the SwiGLU FFN backward against
torch.autograd in float64, and the gate backward against its invariance under a common
scaling of the selected affinities.
"""
import numpy as np
import pytest
import torch

import oracle


def _tiny(seed=0, T=5, H=8, N_r=6, K=2, I=4):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((T, H))
    E = rng.standard_normal((N_r, H)) * 0.7
    b = np.zeros(N_r, np.float32)
    routed = [tuple(rng.standard_normal(sh) / np.sqrt(sh[1]) for sh in ((I, H), (I, H), (H, I))) for _ in range(N_r)]
    shared = [tuple(rng.standard_normal(sh) / np.sqrt(sh[1]) for sh in ((I, H), (I, H), (H, I)))]
    R = rng.standard_normal((T, H))
    return u, E, b, K, routed, shared, R


def _loss(u, E, b, K, routed, shared, R):
    r = oracle.layer_forward(u, E, b, K, routed, shared)
    return float((r["out"] * R).sum()), r["idx"]


def _fd(f, x, idx0, eps=1e-6):
    """Central differences of f over every entry of the array x (modified in place)."""
    g = np.zeros_like(x)
    for i in np.ndindex(x.shape):
        old = x[i]
        x[i] = old + eps
        fp, ip = f()
        x[i] = old - eps
        fm, im = f()
        x[i] = old
        assert np.array_equal(ip, idx0) and np.array_equal(im, idx0), "selection moved under the probe"
        g[i] = (fp - fm) / (2 * eps)
    return g


def _close(a, b, tol=1e-6):
    return np.max(np.abs(a - b)) <= tol * max(1.0, np.max(np.abs(b)))


@pytest.mark.parametrize("seed", [0, 1])
def test_layer_backward_matches_finite_differences(seed):
    u, E, b, K, routed, shared, R = _tiny(seed)
    f = lambda: _loss(u, E, b, K, routed, shared, R)
    _, idx0 = f()
    g = oracle.layer_backward(u, E, b, K, routed, shared, R)
    assert np.array_equal(g["idx"], idx0)
    assert _close(g["du"], _fd(f, u, idx0))
    assert _close(g["dcentroids"], _fd(f, E, idx0))
    for j in range(3):
        assert _close(g["shared"][0][j], _fd(f, shared[0][j], idx0))
    for e in range(len(routed)):
        for j in range(3):
            fd = _fd(f, routed[e][j], idx0)
            if e in g["routed"]:
                assert _close(g["routed"][e][j], fd)
            else:                                   # an expert with no rows gets no gradient
                assert np.max(np.abs(fd)) <= 1e-9


def test_bias_only_selects():
    # a bias step small enough to keep the selection leaves the output unchanged: no gradient into b
    u, E, b, K, routed, shared, R = _tiny(3)
    f0, idx0 = _loss(u, E, b, K, routed, shared, R)
    f1, idx1 = _loss(u, E, b + np.float32(1e-4), K, routed, shared, R)
    assert np.array_equal(idx0, idx1) and f0 == f1


def test_swiglu_backward_matches_autograd():
    rng = np.random.default_rng(4)
    x, wg, wu, wd, dy = (rng.standard_normal(s) for s in ((7, 16), (12, 16), (12, 16), (16, 12), (7, 16)))
    g = oracle.swiglu_ffn_backward(x, wg, wu, wd, dy)
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, wg, wu, wd)]
    y = (torch.nn.functional.silu(t[0] @ t[1].T) * (t[0] @ t[2].T)) @ t[3].T
    y.backward(torch.tensor(dy))
    for name, tt in zip(("dx", "dW_gate", "dW_up", "dW_down"), t):
        assert np.allclose(g[name], tt.grad.numpy(), rtol=1e-12, atol=1e-12), name


def test_gate_backward_is_blind_to_a_common_scale_of_the_selected_affinities():
    # g = s / sum(s) does not change when every selected s is scaled by c, so the affinity
    # gradient is orthogonal to s: sum_k ds_k s_k = 0, i.e. sum_k dlogit_k / (1 - s_k) = 0
    u, E, b, K, routed, shared, R = _tiny(5, K=3, N_r=8)
    g = oracle.layer_backward(u, E, b, K, routed, shared, R)
    s_sel = np.take_along_axis(g["s"], g["idx"].astype(np.int64), axis=1)
    assert np.max(np.abs((g["dlogit"] / (1 - s_sel)).sum(axis=1))) <= 1e-12 * np.max(np.abs(g["dgate"]))


def test_dense_mixture_gradient_with_every_expert_selected():
    # K = N_r, zero bias: every expert is selected and the layer is a smooth dense mixture, so the
    # finite differences probe the gate path with all experts at once
    u, E, b, K, routed, shared, R = _tiny(6, N_r=4, K=4)
    f = lambda: _loss(u, E, b, K, routed, shared, R)
    _, idx0 = f()
    g = oracle.layer_backward(u, E, b, K, routed, shared, R)
    assert _close(g["du"], _fd(f, u, idx0))
    assert _close(g["dcentroids"], _fd(f, E, idx0))
