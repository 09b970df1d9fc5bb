"""CPU gradient oracle for the ReverseMambaLayer -- TEST INFRASTRUCTURE ONLY.

The backward pass is what plug-in training of the sidecar needs ("Bifocal
Diffusion Language Models", §3.5 and §4.1: R2LM-PI trains the Mamba
blocks, the stream LayerNorms and the gates s with the backbone frozen).
This module states the layer's forward once more, in plain PyTorch CPU
float64 ops, and takes its gradients with torch's reverse-mode autograd: the
derivative of a definition, with no hand-derived adjoint anywhere.  Like the
numpy oracle it is used only by tests; the product path never imports it.

The restatement follows the same definition as ``r2l_oracle`` (steps ❶-❹ of
§3.4, the standard Mamba-1 block, the "l2r" control of §4.4) with plain
loops over time.  Pins (``tests/test_oracle_grad.py``): its forward equals
the numpy oracle's; central finite differences of the numpy oracle agree
with its gradients for every parameter, the input and s, in both
directions, for the layer and for the standalone scan; the gradients of
beta, gamma and s match their closed forms from the numpy oracle's branch;
and at s = 0 the gradient passes straight through.  No function is
parity-unpinned.
"""
from __future__ import annotations

import numpy as np
import torch

__all__ = ["PARAMS", "layer_forward_t", "layer_grads", "scan_forward_t", "scan_grads"]

PARAMS = ("in_proj_w", "conv_w", "conv_b", "x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "Dskip",
          "out_proj_w", "ln_w", "ln_b")


def _t(a, grad=False):
    t = torch.tensor(np.asarray(a, np.float64), dtype=torch.float64)
    return t.requires_grad_(grad)


def _silu(v):
    return v / (1.0 + torch.exp(-v))


def _causal_conv(x, w, b):
    """c[j] = b + sum_k w[:, k] x[j-(K-1)+k], x[i] = 0 for i < 0."""
    L, E = x.shape
    K = w.shape[1]
    xp = torch.cat([torch.zeros(K - 1, E, dtype=x.dtype), x], dim=0)
    c = b.expand(L, E)
    for k in range(K):
        c = c + w[:, k] * xp[k:k + L]
    return c


def _scan_causal(u, dt, A, Bm, Cm):
    """H_j = exp(dt_j A) H_{j-1} + (dt_j u_j) (x) B_j, y_j = H_j . C_j (left to right)."""
    L, E = u.shape
    H = torch.zeros(A.shape, dtype=u.dtype)
    ys = []
    for j in range(L):
        H = torch.exp(dt[j][:, None] * A) * H + (dt[j] * u[j])[:, None] * Bm[j][None, :]
        ys.append(H @ Cm[j])
    return torch.stack(ys) if ys else torch.zeros(0, E, dtype=u.dtype)


def _keep(keep, **tensors):
    """Record intermediate tensors (and keep their gradients) for the
    Cauchy-Schwarz scales of layer_grads(factors=True); arithmetic-free."""
    if keep is None:
        return
    for name, t in tensors.items():
        if t.requires_grad:
            t.retain_grad()
        keep.setdefault(name, []).append(t)


def _mamba_block(F, P, keep=None):
    E = P["conv_w"].shape[0]
    N = P["A_log"].shape[1]
    R = P["dt_proj_w"].shape[1]
    xz = F @ P["in_proj_w"].T
    x, z = xz[:, :E], xz[:, E:]
    c = _causal_conv(x, P["conv_w"], P["conv_b"])
    u = _silu(c)
    xdbl = u @ P["x_proj_w"].T
    delta, Bm, Cm = xdbl[:, :R], xdbl[:, R:R + N], xdbl[:, R + N:R + 2 * N]
    dtpre = delta @ P["dt_proj_w"].T + P["dt_proj_b"]
    dt = torch.nn.functional.softplus(dtpre)
    A = -torch.exp(P["A_log"])
    y = _scan_causal(u, dt, A, Bm, Cm) + P["Dskip"] * u
    yg = y * _silu(z)
    m = yg @ P["out_proj_w"].T
    _keep(keep, F=F, xz=xz, x=x, c=c, u=u, xdbl=xdbl, delta=delta, dtpre=dtpre, y=y, yg=yg, m=m)
    return m


def _bounds(cu, T):
    cu = [int(v) for v in cu]
    assert cu[0] == 0 and cu[-1] == T and all(a <= b for a, b in zip(cu, cu[1:]))
    return list(zip(cu[:-1], cu[1:]))


def layer_forward_t(h, cu, P, s, use_ln=True, eps=1e-5, direction="r2l", keep=None):
    """h+ = h + tanh(s) LN(unflip(Mamba1(flip(h)))) per sequence (§3.4 ❶-❹);
    direction="l2r" drops the flips.  h, P[*], s: float64 tensors.  keep
    (optional dict): collects the intermediate tensors of every sequence."""
    assert direction in ("r2l", "l2r")
    T, D = h.shape
    rows = []
    for t0, t1 in _bounds(cu, T):
        if t1 == t0:
            continue
        F = h[t0:t1]
        if direction == "r2l":
            F = torch.flip(F, [0])
        m = _mamba_block(F, P, keep)
        if direction == "r2l":
            m = torch.flip(m, [0])
        if use_ln:
            mu = m.mean(dim=1, keepdim=True)
            var = ((m - mu) ** 2).mean(dim=1, keepdim=True)
            xhat = (m - mu) / torch.sqrt(var + eps)
            m = P["ln_w"] * xhat + P["ln_b"]
            _keep(keep, xhat=xhat, r=m)
        rows.append(m)
    r = torch.cat(rows) if rows else torch.zeros(0, D, dtype=h.dtype)
    return h + torch.tanh(s) * r


def layer_grads(h, cu, W, s, g_out, use_ln=True, eps=1e-5, direction="r2l", factors=False):
    """Gradients of sum(g_out * h+) with respect to h, every parameter in
    PARAMS and s.  Returns a dict of float64 numpy arrays ("h", names, "s").

    factors=True adds "cs": for each parameter whose gradient is a sum over
    tokens of products, dW[i, j] = sum_t a_t[i] b_t[j], an array of dW's
    shape holding ||a[:, i]|| ||b[:, j]|| (norms over all tokens; a constant
    factor contributes sqrt(T)).  By the Cauchy-Schwarz inequality |dW| is
    at most that scale elementwise, and so is the error of dW caused by
    relative 2-norm errors of the factors, times the sum of those errors.
    (A_log's gradient has no such two-factor form and gets none.)"""
    ht = _t(h, True)
    P = {k: _t(W[k], True) for k in PARAMS}
    st = _t(s, True)
    keep = {} if factors else None
    out = layer_forward_t(ht, cu, P, st, use_ln=use_ln, eps=eps, direction=direction, keep=keep)
    out.backward(_t(g_out))
    # (a parameter that does not enter the output, e.g. the LN's without LN, gets zeros)
    g = {k: (P[k].grad.numpy() if P[k].grad is not None else np.zeros(np.shape(W[k]))) for k in PARAMS}
    g["h"] = ht.grad.numpy()
    g["s"] = float(st.grad)
    if factors:
        g["cs"] = _cs_factors(keep, np.shape(W["conv_w"])[1])
    return g


def _cs_factors(keep, K):
    """Cauchy-Schwarz scales of the token-summed parameter gradients (see
    layer_grads), from the intermediates of every sequence."""
    if not keep:
        return {}

    def val(name):
        return torch.cat([t.detach() for t in keep[name]])

    def grad(name):
        return torch.cat([(t.grad if t.grad is not None else torch.zeros_like(t)) for t in keep[name]])

    def cn(a):
        return a.norm(dim=0).numpy()

    n = float(np.sqrt(val("u").shape[0]))   # a constant factor of 1 per token
    dc = cn(grad("c"))
    cs = {
        "in_proj_w": np.outer(cn(grad("xz")), cn(val("F"))),
        "x_proj_w": np.outer(cn(grad("xdbl")), cn(val("u"))),
        "dt_proj_w": np.outer(cn(grad("dtpre")), cn(val("delta"))),
        "out_proj_w": np.outer(cn(grad("m")), cn(val("yg"))),
        # tap k of channel e multiplies a copy of x[:, e] shifted by K-1-k
        # tokens within each sequence (zeros shifted in): its norm is at
        # most ||x[:, e]||
        "conv_w": np.outer(dc * cn(val("x")), np.ones(K)),
        "conv_b": dc * n,
        "dt_proj_b": cn(grad("dtpre")) * n,
        "Dskip": cn(grad("y")) * cn(val("u")),
    }
    if "xhat" in keep:
        dr = cn(grad("r"))
        cs["ln_w"] = dr * cn(val("xhat"))
        cs["ln_b"] = dr * n
    return cs


def scan_forward_t(u, dt, A_log, Bm, Cm, cu, Dskip=None, z=None, direction="r2l"):
    """The standalone scan of r2l_oracle.reverse_selective_scan, in torch."""
    T, E = u.shape
    A = -torch.exp(A_log)
    ys = []
    for t0, t1 in _bounds(cu, T):
        if t1 == t0:
            continue
        sl = slice(t0, t1)
        o = (lambda a: torch.flip(a, [0])) if direction == "r2l" else (lambda a: a)  # noqa: E731
        ys.append(o(_scan_causal(o(u[sl]), o(dt[sl]), A, o(Bm[sl]), o(Cm[sl]))))
    y = torch.cat(ys) if ys else torch.zeros(0, E, dtype=u.dtype)
    if Dskip is not None:
        y = y + Dskip * u
    if z is not None:
        y = y * _silu(z)
    return y


def scan_grads(u, dt, A_log, Bm, Cm, cu, dy, Dskip=None, z=None, direction="r2l"):
    """Gradients of sum(dy * y) for the standalone scan: a dict with u, dt,
    A_log, B, C and (when given) Dskip and z."""
    T = {"u": _t(u, True), "dt": _t(dt, True), "A_log": _t(A_log, True), "B": _t(Bm, True), "C": _t(Cm, True)}
    if Dskip is not None:
        T["Dskip"] = _t(Dskip, True)
    if z is not None:
        T["z"] = _t(z, True)
    y = scan_forward_t(T["u"], T["dt"], T["A_log"], T["B"], T["C"], cu, Dskip=T.get("Dskip"), z=T.get("z"),
                       direction=direction)
    y.backward(_t(dy))
    return {k: v.grad.numpy() for k, v in T.items()}
