"""The error floor of the bf16 path: the layer computed from the oracle's own
steps, in fp64, with only the roundings to bf16 that the bf16 path stores
(the in_proj output xz, the x_proj input u, the gated scan output y and the
output h+; dt, B, C, the scan state, every accumulation and the out_proj
output stay unrounded, as on the GPU).  Comparing it with the unrounded
oracle gives the part of the GPU's error that any implementation storing
those tensors in bf16 has, whatever its arithmetic: the floor under the bf16
tolerances.  Test infrastructure (CPU only); it composes the oracle's
functions and adds no arithmetic of its own beyond the roundings."""
import numpy as np

from oracle import r2l_oracle as O
from reverse_selective_scan_amd import synth


def _block_rounded(F, W):
    """oracle.mamba_block with the bf16 path's stored roundings."""
    f = lambda k: np.asarray(W[k], np.float64)  # noqa: E731
    E, N, R = f("conv_w").shape[0], f("A_log").shape[1], f("dt_proj_w").shape[1]
    xz = np.ascontiguousarray(F, np.float64) @ f("in_proj_w").T
    xz = synth.bf16_round(xz.astype(np.float32)).astype(np.float64)         # xz stored in bf16
    x, z = xz[:, :E], xz[:, E:]
    u = O.silu(O.causal_depthwise_conv(x, f("conv_w"), f("conv_b")))
    ub = synth.bf16_round(u.astype(np.float32)).astype(np.float64)          # x_proj's operand in bf16
    xdbl = ub @ f("x_proj_w").T
    delta, Bm, Cm = xdbl[:, :R], xdbl[:, R:R + N], xdbl[:, R + N:R + 2 * N]
    dt = O.softplus(delta @ f("dt_proj_w").T + f("dt_proj_b")[None, :])
    y = O.selective_scan_causal(u, dt, -np.exp(f("A_log")), Bm, Cm, f("Dskip"))
    g = synth.bf16_round((y * O.silu(z)).astype(np.float32)).astype(np.float64)  # gated y stored in bf16
    return g @ f("out_proj_w").T


def layer_rounded(h, cu, W, s, eps=1e-5, use_ln=True, direction="r2l"):
    """(h+, r) with the stored roundings, in the order of
    oracle.reverse_mamba_layer; h+ is rounded to bf16 as the output is."""
    h = np.asarray(h, np.float64)
    r = np.zeros_like(h)
    for t0, t1 in zip(cu[:-1], cu[1:]):
        t0, t1 = int(t0), int(t1)
        if t1 > t0:
            if direction == "r2l":
                m = _block_rounded(h[t0:t1][::-1], W)[::-1]
            else:
                m = _block_rounded(h[t0:t1], W)
            r[t0:t1] = O.layer_norm(m, W["ln_w"], W["ln_b"], eps) if use_ln else m
    out = O.gated_residual(h, r, s)
    return synth.bf16_round(out.astype(np.float32)).astype(np.float64), r
