"""Parity metrics and shared helpers for the GPU tests.

Tolerances of the layer output h+:
  fp32 path:  max_i |g_i - o_i| / max(|o_i|, RMS(o))  <= 1e-4
  bf16 path:  max_i |g_i - o_i| / RMS(o)              <= 2e-2
where o is the fp64 oracle output and g the library's output (bf16 path:
bf16 activations and weights, fp32 scan state and accumulation).

The bf16 path stores four tensors in bf16 (the in_proj output xz, the x_proj
input u, the gated scan output y, and h+ itself); everything else is fp32.
Those storage roundings alone put a floor under the error of any
implementation: tests/bf16_floor.py computes it by running the oracle's own
steps with exactly those roundings.  On top of the fixed bounds, every bf16
layer comparison requires the library's error to stay within
FLOOR_FACTOR x floor + FLOOR_SLACK of that case's floor: the kernels'
arithmetic (fp32 against the floor's fp64, different summation orders) may
add at most a tenth of the floor and 1e-3 of the RMS.
"""
import numpy as np

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
# The LayerNorm branch r on the bf16 path (h+ ~ h hides branch errors when
# tanh(s) is small, so r is checked on its own).  The storage floor of r
# reaches 2.85e-2 on the widest-sample case (8.5 M values at d_model 256,
# the left-to-right direction) and 1.5..2.5e-2 on the full-size workloads,
# so the fixed cap is 3e-2 and the per-case floor bound below is the
# binding one.
TOL_BF16_BRANCH = 3e-2
FLOOR_FACTOR = 1.1
FLOOR_SLACK = 1e-3


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


def floor_bound(floor_err):
    return FLOOR_FACTOR * floor_err + FLOOR_SLACK


def to_np(t):
    """Device tensor -> float64 numpy (exact for bf16 / fp32)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def report(name, value, tol):
    print(f"[parity] {name}: {value:.3e} (tol {tol:.0e})", flush=True)
    return value


def check_bf16(tag, g, ref, floor, cap):
    """bf16 comparison of one output against the oracle: within the fixed
    cap and within the storage floor's bound (floor: the same output of
    tests/bf16_floor.py, or None to skip that part)."""
    e = report(tag, err_rms(g, ref), cap)
    assert e <= cap, (tag, e, cap)
    if floor is not None:
        fe = err_rms(floor, ref)
        b = floor_bound(fe)
        print(f"[parity] {tag} storage floor: {fe:.3e} (bound {b:.3e})", flush=True)
        assert e <= b, (tag, e, b)
    return e
