"""Pins for the gradient oracle (CPU, no GPU needed).

The gradient oracle differentiates a torch restatement of the layer.  These
tests tie it to things other than itself: the numpy oracle's forward (a
separate statement), central finite differences of the numpy oracle for
every parameter group and the input, and closed forms for the gradients of
the parameters that enter linearly after the LayerNorm (beta, gamma, s)."""
import math

import numpy as np
import pytest

from oracle import r2l_oracle as O
from oracle import r2l_oracle_grad as G


def _rng(seed):
    return np.random.default_rng(seed)


def _weights(rng, D=6, E=8, N=3, R=2, K=4):
    return {
        "in_proj_w": rng.standard_normal((2 * E, D)) / math.sqrt(D),
        "conv_w": rng.standard_normal((E, K)) / 2,
        "conv_b": rng.standard_normal(E) / 2,
        "x_proj_w": rng.standard_normal((R + 2 * N, E)) / math.sqrt(E),
        "dt_proj_w": rng.standard_normal((E, R)) / math.sqrt(R),
        "dt_proj_b": rng.uniform(-3, -1, E),
        "A_log": rng.uniform(-1, 1.5, (E, N)),
        "Dskip": rng.uniform(0.5, 1.5, E),
        "out_proj_w": rng.standard_normal((D, E)) / math.sqrt(E),
        "ln_w": rng.uniform(0.8, 1.2, D),
        "ln_b": rng.uniform(-0.1, 0.1, D),
    }


def _case(seed=70, lens=(7, 1, 0, 5)):
    rng = _rng(seed)
    W = _weights(rng)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    h = rng.standard_normal((T, 6))
    g = rng.standard_normal((T, 6))
    return rng, W, h, cu, g, 0.8


@pytest.mark.parametrize("direction", ["r2l", "l2r"])
@pytest.mark.parametrize("use_ln", [True, False])
def test_torch_forward_equals_numpy_oracle(direction, use_ln):
    _, W, h, cu, _, s = _case()
    P = {k: G._t(W[k]) for k in G.PARAMS}
    got = G.layer_forward_t(G._t(h), cu, P, G._t(s), use_ln=use_ln, direction=direction).numpy()
    ref = O.reverse_mamba_layer(h, cu, W, s, use_ln=use_ln, direction=direction)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def _loss(h, cu, W, s, g, use_ln, direction):
    return float(np.sum(g * O.reverse_mamba_layer(h, cu, W, s, use_ln=use_ln, direction=direction)))


@pytest.mark.parametrize("direction", ["r2l", "l2r"])
@pytest.mark.parametrize("use_ln", [True, False])
def test_layer_grads_match_finite_differences(direction, use_ln):
    """Central differences of the numpy oracle (step 1e-6, fp64) on three
    entries of every parameter, three of h, and s."""
    rng, W, h, cu, g, s = _case()
    grads = G.layer_grads(h, cu, W, s, g, use_ln=use_ln, direction=direction)
    eps = 1e-6
    names = [n for n in G.PARAMS if use_ln or n not in ("ln_w", "ln_b")]
    for name in names + ["h"]:
        arr = h if name == "h" else W[name]
        for _ in range(3):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            if name == "h":
                fp = _loss(plus, cu, W, s, g, use_ln, direction)
                fm = _loss(minus, cu, W, s, g, use_ln, direction)
            else:
                fp = _loss(h, cu, {**W, name: plus}, s, g, use_ln, direction)
                fm = _loss(h, cu, {**W, name: minus}, s, g, use_ln, direction)
            fd = (fp - fm) / (2 * eps)
            assert abs(grads[name][idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (name, idx, grads[name][idx], fd)
    fd = (_loss(h, cu, W, s + eps, g, use_ln, direction) - _loss(h, cu, W, s - eps, g, use_ln, direction)) / (2 * eps)
    assert abs(grads["s"] - fd) <= 1e-6 * max(1.0, abs(fd))


def test_post_norm_gradients_have_closed_forms():
    """h+ = h + tanh(s) (gamma * xhat + beta): d/dbeta = tanh(s) sum_t g_t,
    d/dgamma = tanh(s) sum_t g_t * xhat_t, d/ds = (1 - tanh(s)^2) sum g * r,
    d/dh = g + (terms through the branch), with r and xhat from the numpy
    oracle."""
    _, W, h, cu, g, s = _case(71)
    grads = G.layer_grads(h, cu, W, s, g)
    _, r = O.reverse_mamba_layer(h, cu, W, s, return_branch=True)
    xhat = (r - W["ln_b"]) / W["ln_w"]
    th = math.tanh(s)
    np.testing.assert_allclose(grads["ln_b"], th * g.sum(axis=0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(grads["ln_w"], th * (g * xhat).sum(axis=0), rtol=1e-10, atol=1e-12)
    assert abs(grads["s"] - (1 - th * th) * float(np.sum(g * r))) <= 1e-10 * max(1.0, abs(grads["s"]))


def test_zero_gate_passes_the_gradient_straight_through():
    """At s = 0 (the state the pages' training starts from) every branch
    parameter gets zero gradient and d/dh = g exactly; d/ds = sum g * r."""
    _, W, h, cu, g, _ = _case(72)
    grads = G.layer_grads(h, cu, W, 0.0, g)
    for name in G.PARAMS:
        assert np.all(grads[name] == 0.0), name
    assert np.array_equal(grads["h"], g)
    _, r = O.reverse_mamba_layer(h, cu, W, 0.0, return_branch=True)
    assert abs(grads["s"] - float(np.sum(g * r))) <= 1e-10 * max(1.0, abs(grads["s"]))


def _scan_inputs(rng, T, E=4, N=3):
    return (rng.standard_normal((T, E)), rng.uniform(0.01, 0.5, (T, E)), rng.uniform(-1, 1.5, (E, N)),
            rng.standard_normal((T, N)), rng.standard_normal((T, N)), rng.uniform(0.5, 1.5, E),
            rng.standard_normal((T, E)))


@pytest.mark.parametrize("direction", ["r2l", "l2r"])
def test_scan_grads_match_finite_differences(direction):
    rng = _rng(73)
    lens = [6, 0, 1, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    u, dt, A_log, Bm, Cm, Dk, z = _scan_inputs(rng, T)
    dy = rng.standard_normal(u.shape)
    grads = G.scan_grads(u, dt, A_log, Bm, Cm, cu, dy, Dskip=Dk, z=z, direction=direction)
    base = dict(u=u, dt=dt, A_log=A_log, B=Bm, C=Cm, Dskip=Dk, z=z)

    def loss(v):
        y = O.reverse_selective_scan(v["u"], v["dt"], v["A_log"], v["B"], v["C"], cu, Dskip=v["Dskip"], z=v["z"],
                                     direction=direction)
        return float(np.sum(dy * y))

    eps = 1e-6
    for name, arr in base.items():
        for _ in range(4):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            fd = (loss({**base, name: plus}) - loss({**base, name: minus})) / (2 * eps)
            assert abs(grads[name][idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (name, idx, grads[name][idx], fd)


def test_scan_torch_forward_equals_numpy_oracle():
    rng = _rng(74)
    cu = np.array([0, 5, 5, 9])
    u, dt, A_log, Bm, Cm, Dk, z = _scan_inputs(rng, 9)
    for direction in ("r2l", "l2r"):
        got = G.scan_forward_t(G._t(u), G._t(dt), G._t(A_log), G._t(Bm), G._t(Cm), cu, Dskip=G._t(Dk), z=G._t(z),
                               direction=direction).numpy()
        ref = O.reverse_selective_scan(u, dt, A_log, Bm, Cm, cu, Dskip=Dk, z=z, direction=direction)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Cauchy-Schwarz scales of the token-summed gradients (layer_grads(factors=True))
# ---------------------------------------------------------------------------
CS_NAMES = ("in_proj_w", "x_proj_w", "dt_proj_w", "out_proj_w", "conv_w", "conv_b", "dt_proj_b", "Dskip",
            "ln_w", "ln_b")


@pytest.mark.parametrize("direction", ["r2l", "l2r"])
def test_cs_scales_bound_the_exact_gradients(direction):
    """|sum_t a_t b_t| <= ||a|| ||b||: the exact gradient lies within its
    scale elementwise, and somewhere strictly inside (several tokens)."""
    _, W, h, cu, g, s = _case()
    grads = G.layer_grads(h, cu, W, s, g, direction=direction, factors=True)
    assert set(grads["cs"]) == set(CS_NAMES)
    for k in CS_NAMES:
        sc = grads["cs"][k]
        assert sc.shape == np.shape(W[k]), k
        assert np.all(np.abs(grads[k]) <= sc * (1 + 1e-12) + 1e-300), k
        assert np.any(np.abs(grads[k]) < 0.999 * sc), k


def test_cs_scales_are_exact_for_one_token():
    """With a single token every sum over tokens has one term, so the
    Cauchy-Schwarz bound is attained: |dW| equals its scale (for the conv
    only the tap that meets the token itself is non-zero, and it attains
    it).  A factor taken from the wrong tensor fails here."""
    rng = _rng(71)
    W = _weights(rng)
    h = rng.standard_normal((1, 6))
    g = rng.standard_normal((1, 6))
    grads = G.layer_grads(h, [0, 1], W, 0.8, g, factors=True)
    for k in CS_NAMES:
        got, sc = np.abs(grads[k]), grads["cs"][k]
        if k == "conv_w":
            np.testing.assert_allclose(got[:, -1], sc[:, -1], rtol=1e-12, err_msg=k)
            assert not np.any(got[:, :-1]), k
        else:
            np.testing.assert_allclose(got, sc, rtol=1e-12, atol=1e-300, err_msg=k)
