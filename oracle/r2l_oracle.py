"""CPU oracle for the R2LM ReverseMambaLayer forward -- TEST INFRASTRUCTURE ONLY.

This module is the plain, slow, obviously-correct statement of what the
layer computes.  It exists so that tests, the smoke check and the CPU
baseline leg of the benchmark can check the HIP kernels against it.  The
product path (the C-ABI library and its Python binding) never imports, calls
or links anything in this directory.

Source: "Bifocal Diffusion Language Models: Asymmetric Bidirectional Context
for Parallel Generation" (arXiv 2606.27732, HTML full text).

  * §3.4 "R2LM Architecture", the R2LM stream, steps ❶-❹:
      ❶ reverse the sequence axis,
      ❷ run the Mamba-1 selective-scan block over the reversed sequence,
      ❸ reverse back and apply a LayerNorm that belongs to this stream,
      ❹ add the normalised stream to the hidden state scaled by tanh(s),
        with one scalar s per hooked layer.
  * §4.1 "Experimental Setup": d_state = 16, d_conv = 4, expand = 2,
    one hook after every 4th of 28 decoder layers (7 hooks), d = 2048.
  * §3.5 "Training and Inference": gates start at s = 0, at which point the
    augmented model equals the causal baseline bit for bit.

The Mamba-1 block (the pages name it and cite it, but print no formula) is
read as the standard selective-SSM block: in_proj to (x, z); depthwise
causal conv1d with bias over x; SiLU; x_proj to (delta, B, C); dt_proj with
bias followed by softplus; the selective scan with zero-order hold for A
(a = exp(dt * A), A = -exp(A_log)) and an Euler step for B (b = dt * B * u);
the skip term Dskip * u; the SiLU(z) gate; out_proj without bias.

Everything is computed in float64 from the (exactly representable) inputs.
Matrix products use numpy's ``@`` as a library primitive; the recurrence is
a plain loop over time.  No blocking, fusion or reordering beyond the
definition.

Parity pins: every function here is pinned by the CPU tests in
``tests/test_oracle.py`` (brute-force closed forms, special cases that
reduce to numpy library routines, the flip identity, invariants, the
parameter count printed on the pages).  No function is parity-unpinned.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "silu",
    "softplus",
    "causal_depthwise_conv",
    "selective_scan_causal",
    "mamba_block",
    "layer_norm",
    "gated_residual",
    "reverse_mamba_layer",
    "reverse_mamba_layer_direct",
    "reverse_conv_silu",
    "reverse_selective_scan",
    "hook_stack",
    "param_shapes",
]


# --------------------------------------------------------------------------
# pointwise functions (definitions)
# --------------------------------------------------------------------------
def silu(v):
    """SiLU(v) = v * sigmoid(v) = v / (1 + e^-v)  (Mamba-1 activation)."""
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


def softplus(v):
    """softplus(v) = log(1 + e^v), evaluated as log(e^0 + e^v) by numpy's
    ``logaddexp`` so that large |v| does not overflow."""
    return np.logaddexp(0.0, np.asarray(v, dtype=np.float64))


# --------------------------------------------------------------------------
# Mamba-1 block, run left to right over a sequence already in scan order
# --------------------------------------------------------------------------
def causal_depthwise_conv(x, w, b):
    """Causal depthwise conv1d with bias over one sequence.

    x: [L, E], w: [E, K], b: [E].   c[j] = b + sum_k w[:, k] * x[j-(K-1)+k],
    taking x[i] = 0 for i < 0 (zero left padding, width K).
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    b = np.asarray(b, np.float64)
    L, E = x.shape
    K = w.shape[1]
    c = np.empty((L, E))
    for j in range(L):
        acc = b.copy()
        for k in range(K):
            i = j - (K - 1) + k
            if i >= 0:
                acc = acc + w[:, k] * x[i]
        c[j] = acc
    return c


def selective_scan_causal(u, dt, A, Bm, Cm, Dskip):
    """Selective scan over one sequence in scan order (left to right).

    u, dt: [L, E]; A: [E, N]; Bm, Cm: [L, N]; Dskip: [E] or None.
    H_{-1} = 0;  H_j = exp(dt_j * A) (.) H_{j-1} + (dt_j * u_j) (x) B_j;
    y_j = H_j . C_j + Dskip (.) u_j.
    """
    u = np.asarray(u, np.float64)
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    Bm = np.asarray(Bm, np.float64)
    Cm = np.asarray(Cm, np.float64)
    L, E = u.shape
    H = np.zeros_like(A)
    y = np.empty((L, E))
    for j in range(L):
        H = np.exp(dt[j][:, None] * A) * H + (dt[j] * u[j])[:, None] * Bm[j][None, :]
        y[j] = H @ Cm[j]
    if Dskip is not None:
        y = y + np.asarray(Dskip, np.float64)[None, :] * u
    return y


def mamba_block(F, W, return_parts=False):
    """Mamba-1 block over one sequence F [L, D] in scan order.

    W holds (names in nn.Linear [out, in] layout):
      in_proj_w [2E, D], conv_w [E, K], conv_b [E], x_proj_w [R+2N, E],
      dt_proj_w [E, R], dt_proj_b [E], A_log [E, N], Dskip [E],
      out_proj_w [D, E].
    x is the first E columns of in_proj's output, z the last E; x_proj's
    output is [delta (R) | B (N) | C (N)].
    """
    f = lambda k: np.asarray(W[k], np.float64)  # noqa: E731
    F = np.ascontiguousarray(F, np.float64)     # (a flipped view would bypass BLAS)
    E = f("conv_w").shape[0]
    N = f("A_log").shape[1]
    R = f("dt_proj_w").shape[1]
    xz = F @ f("in_proj_w").T
    x, z = xz[:, :E], xz[:, E:]
    c = causal_depthwise_conv(x, f("conv_w"), f("conv_b"))
    u = silu(c)
    xdbl = u @ f("x_proj_w").T
    delta, Bm, Cm = xdbl[:, :R], xdbl[:, R:R + N], xdbl[:, R + N:R + 2 * N]
    dt = softplus(delta @ f("dt_proj_w").T + f("dt_proj_b")[None, :])
    A = -np.exp(f("A_log"))
    y = selective_scan_causal(u, dt, A, Bm, Cm, f("Dskip"))
    g = y * silu(z)
    m = g @ f("out_proj_w").T
    if return_parts:
        return m, dict(xz=xz, c=c, u=u, xdbl=xdbl, dt=dt, y=y, g=g)
    return m


# --------------------------------------------------------------------------
# stream-local LayerNorm and gated residual (§3.4 steps ❸ and ❹)
# --------------------------------------------------------------------------
def layer_norm(M, gamma, beta, eps=1e-5):
    """LayerNorm over the last axis: biased variance, affine gamma/beta."""
    M = np.asarray(M, np.float64)
    mu = M.mean(axis=-1, keepdims=True)
    var = ((M - mu) ** 2).mean(axis=-1, keepdims=True)
    return np.asarray(gamma, np.float64) * (M - mu) / np.sqrt(var + eps) + np.asarray(beta, np.float64)


def gated_residual(h, r, s):
    """h+ = h + r * tanh(s)   (§3.4 step ❹; s is one scalar per hook)."""
    return np.asarray(h, np.float64) + np.asarray(r, np.float64) * np.tanh(np.float64(s))


def _seq_bounds(cu_seqlens, n_tokens):
    cu = [int(v) for v in cu_seqlens]
    assert cu[0] == 0 and cu[-1] == n_tokens, "cu_seqlens must run from 0 to n_tokens"
    assert all(a <= b for a, b in zip(cu, cu[1:])), "cu_seqlens must be non-decreasing"
    return list(zip(cu[:-1], cu[1:]))


# --------------------------------------------------------------------------
# the layer, literally: flip -> Mamba-1 -> flip -> LN -> gated residual
# --------------------------------------------------------------------------
def _check_direction(direction):
    assert direction in ("r2l", "l2r"), "direction is 'r2l' or 'l2r'"
    return direction == "r2l"


def reverse_mamba_layer(h, cu_seqlens, W, s, use_ln=True, eps=1e-5, return_branch=False,
                        direction="r2l"):
    """ReverseMambaLayer forward over packed sequences (§3.4 steps ❶-❹).

    h: [T, D] hidden states, sequences packed back to back; cu_seqlens:
    [nseq+1] offsets.  Each sequence is flipped, run through the Mamba-1
    block, flipped back, layer-normalised (unless use_ln is False) and added
    to h with weight tanh(s).  Returns h+ (and the branch r if asked).

    direction="l2r" is the ablation control of §4.4 (Table 4, "L2R Mamba"):
    the same block run in the original direction, i.e. with no flips.
    """
    flip = _check_direction(direction)
    h = np.asarray(h, np.float64)
    T, D = h.shape
    r = np.zeros((T, D))
    for t0, t1 in _seq_bounds(cu_seqlens, T):
        if t1 == t0:
            continue
        F = h[t0:t1][::-1] if flip else h[t0:t1]        # ❶ flip
        m = mamba_block(F, W)                           # ❷ Mamba-1 over the flipped sequence
        M = m[::-1] if flip else m                      # ❸ unflip ...
        r[t0:t1] = layer_norm(M, W["ln_w"], W["ln_b"], eps) if use_ln else M  # ... and LN
    out = gated_residual(h, r, s)               # ❹ gated residual
    return (out, r) if return_branch else out


def hook_stack(h, cu_seqlens, layers, use_ln=True, eps=1e-5, direction="r2l"):
    """Apply several hooks in sequence (§4.1: a hook after every 4th decoder
    layer; the decoder layers between hooks are taken as identity here).
    layers: list of (W, s)."""
    cur = np.asarray(h, np.float64)
    for W, s in layers:
        cur = reverse_mamba_layer(cur, cu_seqlens, W, s, use_ln=use_ln, eps=eps, direction=direction)
    return cur


# --------------------------------------------------------------------------
# sub-operations exposed by the library, stated the same literal way
# --------------------------------------------------------------------------
def reverse_conv_silu(x, cu_seqlens, conv_w, conv_b, x_proj_w=None, direction="r2l"):
    """Conv + SiLU (+ x_proj) of the flipped Mamba block, returned in the
    original token order: per sequence, u = flip(SiLU(causal_conv(flip(x)))).
    direction="l2r": u = SiLU(causal_conv(x)) (no flips).
    Returns u [T, E] and, if x_proj_w is given, xdbl = u @ x_proj_w.T."""
    flip = _check_direction(direction)
    x = np.asarray(x, np.float64)
    T, E = x.shape
    u = np.zeros((T, E))
    for t0, t1 in _seq_bounds(cu_seqlens, T):
        if t1 == t0:
            continue
        if flip:
            u[t0:t1] = silu(causal_depthwise_conv(x[t0:t1][::-1], conv_w, conv_b))[::-1]
        else:
            u[t0:t1] = silu(causal_depthwise_conv(x[t0:t1], conv_w, conv_b))
    if x_proj_w is None:
        return u, None
    return u, u @ np.asarray(x_proj_w, np.float64).T


def reverse_selective_scan(u, dt, A_log, Bm, Cm, cu_seqlens, Dskip=None, z=None, direction="r2l"):
    """Selective scan run right to left per sequence, stated as
    flip -> causal scan -> flip; optional Dskip term and SiLU(z) gate.
    direction="l2r": the causal scan itself (no flips).
    u, dt, z: [T, E]; Bm, Cm: [T, N]; A_log: [E, N]."""
    flip = _check_direction(direction)
    u = np.asarray(u, np.float64)
    T, E = u.shape
    A = -np.exp(np.asarray(A_log, np.float64))
    y = np.zeros((T, E))
    o = (lambda a: a[::-1]) if flip else (lambda a: a)  # noqa: E731
    for t0, t1 in _seq_bounds(cu_seqlens, T):
        if t1 == t0:
            continue
        sl = slice(t0, t1)
        y[sl] = o(selective_scan_causal(
            o(u[sl]), o(np.asarray(dt, np.float64)[sl]), A,
            o(np.asarray(Bm, np.float64)[sl]), o(np.asarray(Cm, np.float64)[sl]), Dskip,
        ))
    if z is not None:
        y = y * silu(z)
    return y


# --------------------------------------------------------------------------
# an independent second statement, used only to check the first (flip form)
# --------------------------------------------------------------------------
def reverse_mamba_layer_direct(h, cu_seqlens, W, s, use_ln=True, eps=1e-5):
    """Same layer written directly in the original token order, without any
    flip: an anti-causal conv c_t = b + sum_j w[:, K-1-j] * x_{t+j} (x past the
    sequence end is 0) and a backward recurrence h_t = a_t h_{t+1} + b_t with
    h = 0 past the sequence end.  Scalar loops over (e, n) would be too slow,
    so state updates are vectorised over (e, n) but the time loop runs
    from the last token down to the first."""
    f = lambda k: np.asarray(W[k], np.float64)  # noqa: E731
    h = np.asarray(h, np.float64)
    T, D = h.shape
    E, K = f("conv_w").shape
    N = f("A_log").shape[1]
    R = f("dt_proj_w").shape[1]
    A = -np.exp(f("A_log"))
    out = h.copy()
    tg = np.tanh(np.float64(s))
    for t0, t1 in _seq_bounds(cu_seqlens, T):
        L = t1 - t0
        if L == 0:
            continue
        hs = h[t0:t1]
        xz = hs @ f("in_proj_w").T
        x, z = xz[:, :E], xz[:, E:]
        c = np.tile(f("conv_b"), (L, 1))
        for j in range(min(K, L)):              # tap K-1-j looks j tokens to the right
            c[: L - j] += f("conv_w")[:, K - 1 - j] * x[j:]
        u = c / (1.0 + np.exp(-c))
        xdbl = u @ f("x_proj_w").T
        dt = np.logaddexp(0.0, xdbl[:, :R] @ f("dt_proj_w").T + f("dt_proj_b"))
        Bm, Cm = xdbl[:, R:R + N], xdbl[:, R + N:]
        state = np.zeros((E, N))
        y = np.empty((L, E))
        for t in range(L - 1, -1, -1):
            state = np.exp(dt[t][:, None] * A) * state + (dt[t] * u[t])[:, None] * Bm[t]
            y[t] = state @ Cm[t] + f("Dskip") * u[t]
        m = (y * z / (1.0 + np.exp(-z))) @ f("out_proj_w").T
        if use_ln:
            mu = m.mean(axis=1, keepdims=True)
            var = ((m - mu) ** 2).mean(axis=1, keepdims=True)
            m = f("ln_w") * (m - mu) / np.sqrt(var + eps) + f("ln_b")
        out[t0:t1] = hs + tg * m
    return out


# --------------------------------------------------------------------------
# parameter shapes of one hook (for the parameter count the pages print)
# --------------------------------------------------------------------------
def param_shapes(d_model, d_state=16, d_conv=4, expand=2, dt_rank=None):
    """Shapes of one hook's trainable tensors: the Mamba-1 block, the
    stream's LayerNorm and the scalar gate.  dt_rank defaults to
    ceil(d_model / 16), the Mamba-1 convention."""
    E = expand * d_model
    R = dt_rank if dt_rank is not None else -(-d_model // 16)
    N, K, D = d_state, d_conv, d_model
    return {
        "in_proj_w": (2 * E, D),
        "conv_w": (E, K),
        "conv_b": (E,),
        "x_proj_w": (R + 2 * N, E),
        "dt_proj_w": (E, R),
        "dt_proj_b": (E,),
        "A_log": (E, N),
        "Dskip": (E,),
        "out_proj_w": (D, E),
        "ln_w": (D,),
        "ln_b": (D,),
        "s": (),
    }
