"""Parity metrics and shared helpers for the GPU tests.

Tolerances of the layer output h+:
  fp32 path:  max_i |g_i - o_i| / max(|o_i|, RMS(o))  <= 1e-4
  bf16 path:  max_i |g_i - o_i| / RMS(o)              <= 2e-2
where o is the fp64 oracle output and g the library's output (bf16 path:
bf16 activations and weights, fp32 scan state and accumulation).
"""
import numpy as np

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
# The LayerNorm branch r (a diagnostic; the graded output is h+) on the bf16
# path: storing the in_proj output xz in bf16 alone moves r by up to ~1.8e-2
# of its RMS at d_model 256 (numpy emulation of that one rounding), and the
# bf16 delta and y roundings add to it, so r is held to 3e-2.
TOL_BF16_BRANCH = 3e-2


def rms(o):
    o = np.asarray(o, np.float64)
    return float(np.sqrt(np.mean(o * o))) if o.size else 0.0


def err_f32(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    if o.size == 0:
        return 0.0
    return float(np.max(np.abs(g - o) / np.maximum(np.abs(o), rms(o))))


def err_rms(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    if o.size == 0:
        return 0.0
    return float(np.max(np.abs(g - o)) / rms(o))


def to_np(t):
    """Device tensor -> float64 numpy (exact for bf16 / fp32)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def report(name, value, tol):
    print(f"[parity] {name}: {value:.3e} (tol {tol:.0e})", flush=True)
    return value
