"""Pins for the CPU oracle (no GPU needed).

Each test checks the oracle against something other than itself: a
brute-force closed form, a special case that reduces to a numpy library
routine or to a geometric series, an invariant the pages state, or the
parameter count the pages print.  Together they are meant to catch a
dropped term, a wrong sign, a wrong index or a transposed operand anywhere
in the oracle.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import r2l_oracle as O
from reverse_selective_scan_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _rng(seed):
    return np.random.default_rng(seed)


def _tiny_weights(rng, D=3, E=5, N=2, R=2, K=4):
    return {
        "in_proj_w": rng.standard_normal((2 * E, D)) / math.sqrt(D),
        "conv_w": rng.standard_normal((E, K)) / 2,
        "conv_b": rng.standard_normal(E) / 2,
        "x_proj_w": rng.standard_normal((R + 2 * N, E)) / math.sqrt(E),
        "dt_proj_w": rng.standard_normal((E, R)) / math.sqrt(R),
        "dt_proj_b": rng.uniform(-4, -1, E),
        "A_log": rng.uniform(-1, 1.5, (E, N)),
        "Dskip": rng.uniform(0.5, 1.5, E),
        "out_proj_w": rng.standard_normal((D, E)) / math.sqrt(E),
        "ln_w": rng.uniform(0.8, 1.2, D),
        "ln_b": rng.uniform(-0.1, 0.1, D),
    }


def _scan_inputs(rng, L, E, N):
    u = rng.standard_normal((L, E))
    dt = rng.uniform(0.01, 0.5, (L, E))
    A_log = rng.uniform(-1, 1.5, (E, N))
    Bm = rng.standard_normal((L, N))
    Cm = rng.standard_normal((L, N))
    Dskip = rng.uniform(0.5, 1.5, E)
    return u, dt, A_log, Bm, Cm, Dskip


# ---------------------------------------------------------------------------
# P5: brute-force closed form of the reverse scan for L <= 8
# ---------------------------------------------------------------------------
def _closed_form_reverse_scan(u, dt, A_log, Bm, Cm, Dskip):
    """y_t[e] = sum_{v >= t} sum_n C_t[n] (prod_{t <= k < v} exp(dt_k[e] A[e,n]))
    dt_v[e] B_v[n] u_v[e] + D[e] u_t[e], written with scalar loops."""
    L, E = u.shape
    N = Bm.shape[1]
    y = np.zeros((L, E))
    for t in range(L):
        for e in range(E):
            acc = 0.0
            for v in range(t, L):
                for n in range(N):
                    A = -math.exp(A_log[e][n])
                    prod = 1.0
                    for k in range(t, v):
                        prod *= math.exp(dt[k][e] * A)
                    acc += Cm[t][n] * prod * dt[v][e] * Bm[v][n] * u[v][e]
            y[t][e] = acc + Dskip[e] * u[t][e]
    return y


@pytest.mark.parametrize("L", [1, 2, 3, 5, 8])
def test_scan_matches_brute_force_closed_form(L):
    rng = _rng(100 + L)
    u, dt, A_log, Bm, Cm, Dskip = _scan_inputs(rng, L, 3, 4)
    got = O.reverse_selective_scan(u, dt, A_log, Bm, Cm, [0, L], Dskip=Dskip)
    ref = _closed_form_reverse_scan(u, dt, A_log, Bm, Cm, Dskip)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_printed_product_bounds_differ_from_recurrence():
    """The unrolled recurrence multiplies decays over t <= k < v.  Moving the
    bounds to t < k <= v (a reading some statements of the closed form
    suggest) gives a different result; this records which reading the
    oracle follows."""
    rng = _rng(7)
    L = 6
    u, dt, A_log, Bm, Cm, Dskip = _scan_inputs(rng, L, 2, 3)
    got = O.reverse_selective_scan(u, dt, A_log, Bm, Cm, [0, L], Dskip=Dskip)
    alt = np.zeros_like(got)
    for t in range(L):
        for e in range(2):
            acc = 0.0
            for v in range(t, L):
                for n in range(3):
                    A = -math.exp(A_log[e][n])
                    prod = math.prod(math.exp(dt[k][e] * A) for k in range(t + 1, v + 1))
                    acc += Cm[t][n] * prod * dt[v][e] * Bm[v][n] * u[v][e]
            alt[t][e] = acc + Dskip[e] * u[t][e]
    assert np.max(np.abs(got - alt)) > 1e-3


# ---------------------------------------------------------------------------
# P6: A = 0 reduces the scan to a suffix sum (numpy cumsum on the flip)
# ---------------------------------------------------------------------------
def test_scan_zero_decay_is_suffix_sum():
    rng = _rng(3)
    L, E, N = 37, 4, 5
    u, dt, _, Bm, Cm, Dskip = _scan_inputs(rng, L, E, N)
    A_log = np.full((E, N), -np.inf)             # A = -exp(-inf) = 0
    got = O.reverse_selective_scan(u, dt, A_log, Bm, Cm, [0, L], Dskip=Dskip)
    b = (dt * u)[:, :, None] * Bm[:, None, :]    # [L, E, N]
    suffix = np.cumsum(b[::-1], axis=0)[::-1]
    ref = np.einsum("ten,tn->te", suffix, Cm) + Dskip * u
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------------------
# P7: very strong decay leaves only the token's own term
# ---------------------------------------------------------------------------
def test_scan_infinite_decay_is_pointwise():
    rng = _rng(4)
    L, E, N = 19, 3, 4
    u, dt, _, Bm, Cm, Dskip = _scan_inputs(rng, L, E, N)
    A_log = np.full((E, N), 80.0)                # A ~ -5.5e34: exp(dt A) = 0
    got = O.reverse_selective_scan(u, dt, A_log, Bm, Cm, [0, L], Dskip=Dskip)
    ref = dt * u * (Bm * Cm).sum(axis=1)[:, None] + Dskip * u
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# P8: constant inputs give a geometric series
# ---------------------------------------------------------------------------
def test_scan_constant_inputs_geometric_series():
    L, E, N = 23, 2, 3
    rng = _rng(5)
    A_log = rng.uniform(-2, 1, (E, N))
    dtv = np.array([0.07, 0.3])
    uv = np.array([0.9, -1.3])
    Bv = np.array([0.5, -0.2, 1.1])
    Cv = np.array([1.2, 0.4, -0.7])
    Dskip = np.array([0.3, 1.0])
    u = np.tile(uv, (L, 1))
    dt = np.tile(dtv, (L, 1))
    Bm = np.tile(Bv, (L, 1))
    Cm = np.tile(Cv, (L, 1))
    got = O.reverse_selective_scan(u, dt, A_log, Bm, Cm, [0, L], Dskip=Dskip)
    a = np.exp(dtv[:, None] * -np.exp(A_log))    # [E, N]
    b = (dtv * uv)[:, None] * Bv[None, :]
    ref = np.empty((L, E))
    for t in range(L):
        m = L - t                                # terms v = t .. L-1
        ref[t] = (Cv[None, :] * b * (1 - a ** m) / (1 - a)).sum(axis=1) + Dskip * uv
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# P9: the scan is linear in u for fixed (dt, B, C); gate excluded
# ---------------------------------------------------------------------------
def test_scan_linear_in_input():
    rng = _rng(6)
    L, E, N = 29, 3, 4
    u1, dt, A_log, Bm, Cm, Dskip = _scan_inputs(rng, L, E, N)
    u2 = rng.standard_normal((L, E))
    cu = [0, 11, 11, L]
    f = lambda u: O.reverse_selective_scan(u, dt, A_log, Bm, Cm, cu, Dskip=Dskip)  # noqa: E731
    np.testing.assert_allclose(f(2.5 * u1 - 0.75 * u2), 2.5 * f(u1) - 0.75 * f(u2), rtol=1e-11, atol=1e-11)


def test_scan_gate_multiplies_by_silu_z():
    rng = _rng(16)
    L, E, N = 9, 3, 2
    u, dt, A_log, Bm, Cm, Dskip = _scan_inputs(rng, L, E, N)
    z = rng.standard_normal((L, E))
    y0 = O.reverse_selective_scan(u, dt, A_log, Bm, Cm, [0, L], Dskip=Dskip)
    yz = O.reverse_selective_scan(u, dt, A_log, Bm, Cm, [0, L], Dskip=Dskip, z=z)
    np.testing.assert_allclose(yz, y0 * z * (1 / (1 + np.exp(-z))), rtol=1e-13)


def test_scan_resets_at_sequence_boundaries():
    rng = _rng(8)
    E, N = 3, 2
    lens = [5, 0, 1, 7, 3]
    T = sum(lens)
    u, dt, A_log, Bm, Cm, Dskip = _scan_inputs(rng, T, E, N)
    cu = np.concatenate([[0], np.cumsum(lens)])
    got = O.reverse_selective_scan(u, dt, A_log, Bm, Cm, cu, Dskip=Dskip)
    for t0, t1 in zip(cu[:-1], cu[1:]):
        if t1 > t0:
            ref = _closed_form_reverse_scan(u[t0:t1], dt[t0:t1], A_log, Bm[t0:t1], Cm[t0:t1], Dskip)
            np.testing.assert_allclose(got[t0:t1], ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# P10: conv orientation under the flip (impulse response)
# ---------------------------------------------------------------------------
def test_reverse_conv_impulse_orientation():
    E, K, L, t0 = 3, 4, 10, 6
    rng = _rng(9)
    w = rng.standard_normal((E, K))
    b = rng.standard_normal(E)
    x = np.zeros((L, E))
    x[t0] = 1.0
    u, _ = O.reverse_conv_silu(x, [0, L], w, b)
    c = np.tile(b, (L, 1))
    for j in range(K):                           # token t0-j sees x[t0] through tap K-1-j
        if t0 - j >= 0:
            c[t0 - j] = b + w[:, K - 1 - j]
    np.testing.assert_allclose(u, c / (1 + np.exp(-c)), rtol=1e-14, atol=1e-15)


def test_causal_conv_impulse():
    E, K, L = 2, 4, 8
    rng = _rng(10)
    w = rng.standard_normal((E, K))
    b = np.zeros(E)
    x = np.zeros((L, E))
    x[2] = 1.0
    c = O.causal_depthwise_conv(x, w, b)
    for j in range(L):
        exp = w[:, K - 1 - (j - 2)] if 0 <= j - 2 < K else np.zeros(E)
        np.testing.assert_allclose(c[j], exp, atol=1e-15)


def test_reverse_conv_sequence_end_is_zero_padded():
    E, K = 2, 4
    rng = _rng(11)
    w = rng.standard_normal((E, K))
    b = rng.standard_normal(E)
    x = rng.standard_normal((5, E))
    u, _ = O.reverse_conv_silu(x, [0, 2, 5], w, b)
    # last token of sequence 0 (t=1) only sees itself through tap K-1
    c = b + w[:, K - 1] * x[1]
    np.testing.assert_allclose(u[1], c / (1 + np.exp(-c)), rtol=1e-14)
    # t=0 sees t=0 (tap K-1) and t=1 (tap K-2), not t=2 (other sequence)
    c = b + w[:, K - 1] * x[0] + w[:, K - 2] * x[1]
    np.testing.assert_allclose(u[0], c / (1 + np.exp(-c)), rtol=1e-14)


# ---------------------------------------------------------------------------
# whole layer: brute force with scalar loops for tiny L, no flip, closed form
# ---------------------------------------------------------------------------
def _brute_layer(h, W, s, eps=1e-5, use_ln=True):
    L, D = h.shape
    E, K = W["conv_w"].shape
    N = W["A_log"].shape[1]
    R = W["dt_proj_w"].shape[1]
    sig = lambda v: 1.0 / (1.0 + math.exp(-v))  # noqa: E731
    x = [[sum(W["in_proj_w"][e][d] * h[t][d] for d in range(D)) for e in range(E)] for t in range(L)]
    z = [[sum(W["in_proj_w"][E + e][d] * h[t][d] for d in range(D)) for e in range(E)] for t in range(L)]
    u = [[0.0] * E for _ in range(L)]
    for t in range(L):
        for e in range(E):
            c = W["conv_b"][e]
            for j in range(K):                   # anti-causal: tap K-1-j sees token t+j
                if t + j < L:
                    c += W["conv_w"][e][K - 1 - j] * x[t + j][e]
            u[t][e] = c * sig(c)
    xd = [[sum(W["x_proj_w"][i][e] * u[t][e] for e in range(E)) for i in range(R + 2 * N)] for t in range(L)]
    dt = [[math.log1p(math.exp(sum(W["dt_proj_w"][e][r] * xd[t][r] for r in range(R)) + W["dt_proj_b"][e]))
           for e in range(E)] for t in range(L)]
    y = _closed_form_reverse_scan(np.array(u), np.array(dt), W["A_log"],
                                  np.array([row[R:R + N] for row in xd]),
                                  np.array([row[R + N:] for row in xd]), W["Dskip"])
    m = [[sum(W["out_proj_w"][d][e] * y[t][e] * z[t][e] * sig(z[t][e]) for e in range(E)) for d in range(D)]
         for t in range(L)]
    out = np.zeros((L, D))
    for t in range(L):
        row = m[t]
        if use_ln:
            mu = sum(row) / D
            var = sum((v - mu) ** 2 for v in row) / D
            row = [W["ln_w"][d] * (row[d] - mu) / math.sqrt(var + eps) + W["ln_b"][d] for d in range(D)]
        for d in range(D):
            out[t][d] = h[t][d] + math.tanh(s) * row[d]
    return out


@pytest.mark.parametrize("L", [1, 2, 3, 4, 6])
@pytest.mark.parametrize("use_ln", [True, False])
def test_layer_matches_scalar_brute_force(L, use_ln):
    rng = _rng(20 + L)
    W = _tiny_weights(rng)
    h = rng.standard_normal((L, 3))
    s = 0.37
    got = O.reverse_mamba_layer(h, [0, L], W, s, use_ln=use_ln)
    ref = _brute_layer(h, W, s, use_ln=use_ln)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------------------
# P4: flip form equals the direct reverse form
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("use_ln", [True, False])
def test_flip_form_equals_direct_reverse_form(use_ln):
    rng = _rng(30)
    W = _tiny_weights(rng, D=6, E=12, N=4, R=3)
    lens = [9, 0, 1, 2, 3, 17]
    h = rng.standard_normal((sum(lens), 6))
    cu = np.concatenate([[0], np.cumsum(lens)])
    a = O.reverse_mamba_layer(h, cu, W, -0.8, use_ln=use_ln)
    b = O.reverse_mamba_layer_direct(h, cu, W, -0.8, use_ln=use_ln)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# P1, P2, P3, P12: zero gate, right-context only, isolation, gate linearity
# ---------------------------------------------------------------------------
def _layer_case(seed=40):
    rng = _rng(seed)
    W = _tiny_weights(rng, D=8, E=16, N=4, R=2)
    lens = [13, 6, 10]
    h = rng.standard_normal((sum(lens), 8))
    return rng, W, h, np.concatenate([[0], np.cumsum(lens)])


def test_zero_gate_returns_input_exactly():
    _, W, h, cu = _layer_case()
    out = O.reverse_mamba_layer(h, cu, W, 0.0)
    assert np.array_equal(out, h)


def test_right_context_only():
    rng, W, h, cu = _layer_case()
    base = O.reverse_mamba_layer(h, cu, W, 0.9)
    j = 7                                        # inside sequence 0 = [0, 13)
    h2 = h.copy()
    h2[j] += rng.standard_normal(h.shape[1])
    pert = O.reverse_mamba_layer(h2, cu, W, 0.9)
    assert np.array_equal(pert[j + 1:], base[j + 1:])   # positions right of j untouched
    assert np.all(np.abs(pert[: j + 1] - base[: j + 1]).max(axis=1) > 0)  # left of j sees it


def test_sequence_isolation():
    rng, W, h, cu = _layer_case()
    base = O.reverse_mamba_layer(h, cu, W, 0.9)
    h2 = h.copy()
    h2[cu[1]:cu[2]] += rng.standard_normal((cu[2] - cu[1], h.shape[1]))
    pert = O.reverse_mamba_layer(h2, cu, W, 0.9)
    assert np.array_equal(pert[:cu[1]], base[:cu[1]])
    assert np.array_equal(pert[cu[2]:], base[cu[2]:])


def test_gate_is_linear_in_tanh_s():
    _, W, h, cu = _layer_case()
    o1, r1 = O.reverse_mamba_layer(h, cu, W, 0.3, return_branch=True)
    o2, r2 = O.reverse_mamba_layer(h, cu, W, -1.7, return_branch=True)
    np.testing.assert_allclose((o1 - h) / math.tanh(0.3), (o2 - h) / math.tanh(-1.7), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(r1, r2)


# ---------------------------------------------------------------------------
# P11: LayerNorm invariants
# ---------------------------------------------------------------------------
def test_layer_norm_invariants():
    rng = _rng(50)
    M = 3.0 * rng.standard_normal((7, 33)) + 2.0
    eps = 1e-5
    r = O.layer_norm(M, np.ones(33), np.zeros(33), eps)
    var = M.var(axis=1)
    np.testing.assert_allclose(r.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose(r.var(axis=1), var / (var + eps), rtol=1e-12)
    g = rng.uniform(0.5, 2, 33)
    b = rng.standard_normal(33)
    np.testing.assert_allclose(O.layer_norm(M, g, b, eps), g * r + b, rtol=1e-12, atol=1e-12)


def test_layer_without_ln_returns_raw_branch():
    _, W, h, cu = _layer_case(41)
    _, r_ln = O.reverse_mamba_layer(h, cu, W, 0.5, return_branch=True)
    _, r_raw = O.reverse_mamba_layer(h, cu, W, 0.5, use_ln=False, return_branch=True)
    t0, t1 = cu[0], cu[1]
    np.testing.assert_allclose(r_ln[t0:t1], O.layer_norm(r_raw[t0:t1], W["ln_w"], W["ln_b"]), rtol=1e-12)


# ---------------------------------------------------------------------------
# P15: special values of the pointwise functions
# ---------------------------------------------------------------------------
def test_pointwise_special_values():
    assert O.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    assert O.silu(0.0) == 0.0
    assert O.softplus(800.0) == 800.0
    assert O.softplus(-50.0) == pytest.approx(math.exp(-50.0), rel=1e-12)
    v = np.linspace(-8, 8, 101)
    assert np.all(np.diff(O.softplus(v)) > 0)
    np.testing.assert_allclose(O.silu(v), v * (1 / (1 + np.exp(-v))), rtol=1e-15)


# ---------------------------------------------------------------------------
# P13: parameter count printed on the pages
# ---------------------------------------------------------------------------
def test_parameter_count_matches_pages():
    with open(os.path.join(HERE, "golden", "paper_dims.json")) as f:
        g = json.load(f)
    shapes = O.param_shapes(g["d_model"], g["d_state"], g["d_conv"], g["expand"])
    per_hook = sum(int(np.prod(s)) for s in shapes.values())
    assert g["hooks"] == g["decoder_layers"] // g["hook_every"]
    total = per_hook * g["hooks"]
    assert round(total / 1e6) == g["r2l_params_millions_printed"]
    assert total == 185_106_439


def test_hook_stack_is_sequential_application():
    _, W, h, cu = _layer_case(42)
    rng = _rng(43)
    W2 = _tiny_weights(rng, D=8, E=16, N=4, R=2)
    a = O.hook_stack(h, cu, [(W, 0.4), (W2, -0.6)])
    b = O.reverse_mamba_layer(O.reverse_mamba_layer(h, cu, W, 0.4), cu, W2, -0.6)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------------------
# the synthetic generator's documented recipe (host logic)
# ---------------------------------------------------------------------------
def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.14159], np.float32)
    got = synth.bf16_round(vals)
    exp = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 3.140625], np.float32)
    np.testing.assert_array_equal(got, exp)


def test_synthetic_recipe_statistics():
    wl = synth.custom([300, 200], 64, 128, dt_rank=8, dtype="bf16", seed=5, h_kind="rms")
    W = synth.make_weights(wl)
    h = synth.make_hidden(wl)
    np.testing.assert_allclose(np.sqrt((h.astype(np.float64) ** 2).mean(axis=1)), 1.0, rtol=1e-2)
    assert np.array_equal(synth.bf16_round(W["in_proj_w"]), W["in_proj_w"])
    dt0 = O.softplus(W["dt_proj_b"])
    assert dt0.min() >= 1e-3 * 0.999 and dt0.max() <= 1e-1 * 1.001
    assert np.std(W["in_proj_w"]) == pytest.approx(1 / 8, rel=0.05)
    np.testing.assert_allclose(np.exp(W["A_log"][0]), np.arange(1, 17), rtol=1e-6)
    lens = synth.workloads()["varlen16"].lengths
    assert len(lens) == 16 and min(lens) >= 512 and max(lens) <= 16384


# ---------------------------------------------------------------------------
# L2R control (§4.4, Table 4: the same block run left to right)
# ---------------------------------------------------------------------------
def _closed_form_forward_scan(u, dt, A_log, Bm, Cm, Dskip):
    """y_t[e] = sum_{v <= t} sum_n C_t[n] (prod_{v < k <= t} exp(dt_k[e] A[e,n]))
    dt_v[e] B_v[n] u_v[e] + D[e] u_t[e], written with scalar loops."""
    L, E = u.shape
    N = Bm.shape[1]
    y = np.zeros((L, E))
    for t in range(L):
        for e in range(E):
            acc = 0.0
            for v in range(0, t + 1):
                for n in range(N):
                    A = -math.exp(A_log[e][n])
                    prod = 1.0
                    for k in range(v + 1, t + 1):
                        prod *= math.exp(dt[k][e] * A)
                    acc += Cm[t][n] * prod * dt[v][e] * Bm[v][n] * u[v][e]
            y[t][e] = acc + Dskip[e] * u[t][e]
    return y


@pytest.mark.parametrize("L", [1, 2, 5, 8])
def test_l2r_scan_matches_brute_force_closed_form(L):
    rng = _rng(300 + L)
    u, dt, A_log, Bm, Cm, Dskip = _scan_inputs(rng, L, 3, 4)
    got = O.reverse_selective_scan(u, dt, A_log, Bm, Cm, [0, L], Dskip=Dskip, direction="l2r")
    ref = _closed_form_forward_scan(u, dt, A_log, Bm, Cm, Dskip)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_l2r_conv_impulse_orientation():
    E, K, L, t0 = 3, 4, 10, 3
    rng = _rng(301)
    w = rng.standard_normal((E, K))
    b = rng.standard_normal(E)
    x = np.zeros((L, E))
    x[t0] = 1.0
    u, _ = O.reverse_conv_silu(x, [0, L], w, b, direction="l2r")
    c = np.tile(b, (L, 1))
    for j in range(K):                           # token t0+j sees x[t0] through tap K-1-j
        c[t0 + j] = b + w[:, K - 1 - j]
    np.testing.assert_allclose(u, c / (1 + np.exp(-c)), rtol=1e-14, atol=1e-15)


def test_l2r_conv_sequence_start_is_zero_padded():
    E, K = 2, 4
    rng = _rng(302)
    w = rng.standard_normal((E, K))
    b = rng.standard_normal(E)
    x = rng.standard_normal((5, E))
    u, _ = O.reverse_conv_silu(x, [0, 2, 5], w, b, direction="l2r")
    # first token of sequence 1 (t=2) only sees itself through tap K-1
    c = b + w[:, K - 1] * x[2]
    np.testing.assert_allclose(u[2], c / (1 + np.exp(-c)), rtol=1e-14)
    # t=3 sees t=3 (tap K-1) and t=2 (tap K-2), not t=1 (other sequence)
    c = b + w[:, K - 1] * x[3] + w[:, K - 2] * x[2]
    np.testing.assert_allclose(u[3], c / (1 + np.exp(-c)), rtol=1e-14)


def test_l2r_layer_left_context_only():
    rng, W, h, cu = _layer_case(41)
    base = O.reverse_mamba_layer(h, cu, W, 0.9, direction="l2r")
    j = 5                                        # inside sequence 0 = [0, 13)
    h2 = h.copy()
    h2[j] += rng.standard_normal(h.shape[1])
    pert = O.reverse_mamba_layer(h2, cu, W, 0.9, direction="l2r")
    assert np.array_equal(pert[:j], base[:j])    # positions left of j untouched
    assert np.all(np.abs(pert[j:cu[1]] - base[j:cu[1]]).max(axis=1) > 0)   # right of j sees it
    assert np.array_equal(pert[cu[1]:], base[cu[1]:])


def test_l2r_of_flipped_sequences_is_flipped_r2l():
    """Reversing every sequence turns one direction into the other."""
    _, W, h, cu = _layer_case(42)
    flip = np.concatenate([np.arange(a, b)[::-1] for a, b in zip(cu[:-1], cu[1:])])
    r2l = O.reverse_mamba_layer(h, cu, W, 0.7)
    l2r = O.reverse_mamba_layer(h[flip], cu, W, 0.7, direction="l2r")
    np.testing.assert_allclose(l2r[flip], r2l, rtol=1e-12, atol=1e-12)
    assert np.max(np.abs(O.reverse_mamba_layer(h, cu, W, 0.7, direction="l2r") - r2l)) > 1e-3
