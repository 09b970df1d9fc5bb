"""Seeded synthetic inputs for the ReverseMambaLayer workloads.

This module only draws random numbers and quantises them; it holds none of
the layer's arithmetic.  Tests, the smoke check and the benchmark feed the
same arrays to the HIP library and to the CPU oracle.

Recipe (one ``numpy.random.Generator`` per tensor, seeded by
``SeedSequence([seed, hook, tensor_id])``):

  h            N(0, 1) per element; "rms" workloads divide each token row by
               sqrt(mean(g^2) + 1e-6) (unit-RMS hidden states).
  in_proj_w    [2E, D]    N(0, std = 1/sqrt(D))
  conv_w       [E, K]     N(0, std = 1/sqrt(K))     (depthwise: fan_in = K)
  conv_b       [E]        N(0, std = 1/sqrt(K))
  x_proj_w     [R+2N, E]  N(0, std = 1/sqrt(E))
  dt_proj_w    [E, R]     N(0, std = 1/sqrt(R))
  dt_proj_b    [E]        inverse softplus of dt0, dt0 log-uniform in
                          [1e-3, 1e-1]  (so softplus(bias) = dt0)
  out_proj_w   [D, E]     N(0, std = 1/sqrt(E))
  A_log        [E, N]     log(n + 1)   (the usual Mamba-1 initialisation)
  Dskip        [E]        1
  s            scalar     N(0, std = 0.5)
  ln_w, ln_b   [D]        1 and 0 (or N(1, 0.1) / N(0, 0.1) when affine)
  lengths      varlen workloads: integers uniform in [lo, hi] inclusive

bf16 workloads round every activation and weight tensor to bf16 with
round-to-nearest-even; arrays are returned as float32 holding those exact
values (plus the raw bf16 bit patterns on request).  A_log, Dskip,
dt_proj_b, ln_w, ln_b and s stay float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

TENSOR_IDS = {
    "h": 0, "in_proj_w": 1, "conv_w": 2, "conv_b": 3, "x_proj_w": 4,
    "dt_proj_w": 5, "dt_proj_b": 6, "out_proj_w": 7, "s": 8, "ln_w": 9,
    "ln_b": 10, "lengths": 11, "aux": 12,
}

ACT_WEIGHTS = ("in_proj_w", "conv_w", "conv_b", "x_proj_w", "dt_proj_w", "out_proj_w")
F32_WEIGHTS = ("dt_proj_b", "A_log", "Dskip", "ln_w", "ln_b")


@dataclass
class Workload:
    name: str
    lengths: List[int]
    d_model: int
    d_inner: int
    d_state: int = 16
    dt_rank: int = 128
    d_conv: int = 4
    dtype: str = "bf16"          # "f32" or "bf16"
    seed: int = 0
    h_kind: str = "normal"       # "normal" or "rms"
    n_hooks: int = 1
    varlen: Optional[tuple] = None  # (count, lo, hi): lengths drawn from the seed
    note: str = ""

    @property
    def n_tokens(self) -> int:
        return int(sum(self.lengths))

    @property
    def nseq(self) -> int:
        return len(self.lengths)

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int32)


def _rng(seed: int, hook: int, name: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, hook, TENSOR_IDS[name]]))


def varlen_lengths(seed: int, count: int, lo: int, hi: int) -> List[int]:
    return [int(v) for v in _rng(seed, 0, "lengths").integers(lo, hi + 1, size=count)]


def workloads() -> dict:
    """The five workload shapes (the long-context one split in two) and the
    denoise-step blocks."""
    W = {}
    W["tiny_f32"] = Workload("tiny_f32", [64], 64, 128, 16, 4, 4, "f32", 0, "normal",
                             note="B=1 L=64 D=64 E=128 N=16 R=4 K=4, fp32 throughout")
    W["single_2k"] = Workload("single_2k", [2048], 2048, 4096, 16, 128, 4, "bf16", 1, "normal",
                              note="B=1 L=2048 D=2048 E=4096, bf16 / fp32 state")
    W["serve_b8"] = Workload("serve_b8", [4128] * 8, 2048, 4096, 16, 128, 4, "bf16", 2, "rms",
                             note="B=8 x (4096 prompt + 32 masked) D=2048, bf16 / fp32 state")
    W["stack7"] = Workload("stack7", [4096] * 8, 2048, 4096, 16, 128, 4, "bf16", 3, "rms", n_hooks=7,
                           note="7 hooks in sequence on [8, 4096, 2048], identity between hooks")
    W["varlen16"] = Workload("varlen16", varlen_lengths(4, 16, 512, 16384), 2048, 4096, 16, 128, 4,
                             "bf16", 4, "rms", varlen=(16, 512, 16384),
                             note="16 packed sequences, lengths uniform in [512, 16384]")
    W["long32k"] = Workload("long32k", [32768], 2048, 4096, 16, 128, 4, "bf16", 4, "rms",
                            note="one sequence of L=32768")
    # the cached-decoding inner loop: each denoise step runs the seven hooks on
    # the masked generation block of every sequence alone
    for g in (32, 128):
        W[f"denoise_g{g}"] = Workload(f"denoise_g{g}", [g] * 8, 2048, 4096, 16, 128, 4, "bf16", 5, "rms",
                                      n_hooks=7, note=f"one denoise step: 7 hooks on B=8 blocks of G={g} tokens")
    return W


def custom(lengths, d_model, d_inner, d_state=16, dt_rank=None, d_conv=4, dtype="bf16",
           seed=0, h_kind="normal", n_hooks=1, name="custom") -> Workload:
    if dt_rank is None:
        dt_rank = -(-d_model // 16)
    return Workload(name, list(int(v) for v in lengths), d_model, d_inner, d_state, dt_rank,
                    d_conv, dtype, seed, h_kind, n_hooks)


# --------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even) on float32 bit patterns
# --------------------------------------------------------------------------
def bf16_bits(a) -> np.ndarray:
    a32 = np.ascontiguousarray(a, dtype=np.float32)
    u = a32.view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def bf16_round(a) -> np.ndarray:
    return (bf16_bits(a).astype(np.uint32) << 16).view(np.float32)


def _quant(a, dtype):
    a = np.asarray(a, dtype=np.float32)
    return bf16_round(a) if dtype == "bf16" else a


def _normal(seed, hook, name, shape, std):
    g = _rng(seed, hook, name).standard_normal(size=shape, dtype=np.float32)
    return g * np.float32(std)


def make_hidden(wl: Workload, hook: int = 0) -> np.ndarray:
    T, D = wl.n_tokens, wl.d_model
    g = _rng(wl.seed, hook, "h").standard_normal(size=(T, D), dtype=np.float32)
    if wl.h_kind == "rms":
        g = g / np.sqrt((g.astype(np.float64) ** 2).mean(axis=1, keepdims=True) + 1e-6).astype(np.float32)
    return _quant(g, wl.dtype)


def make_weights(wl: Workload, hook: int = 0, affine_ln: bool = False, s: Optional[float] = None) -> dict:
    D, E, N, R, K = wl.d_model, wl.d_inner, wl.d_state, wl.dt_rank, wl.d_conv
    sd = wl.seed
    W = {
        "in_proj_w": _normal(sd, hook, "in_proj_w", (2 * E, D), 1 / np.sqrt(D)),
        "conv_w": _normal(sd, hook, "conv_w", (E, K), 1 / np.sqrt(K)),
        "conv_b": _normal(sd, hook, "conv_b", (E,), 1 / np.sqrt(K)),
        "x_proj_w": _normal(sd, hook, "x_proj_w", (R + 2 * N, E), 1 / np.sqrt(E)),
        "dt_proj_w": _normal(sd, hook, "dt_proj_w", (E, R), 1 / np.sqrt(R)),
        "out_proj_w": _normal(sd, hook, "out_proj_w", (D, E), 1 / np.sqrt(E)),
    }
    for k in ACT_WEIGHTS:
        W[k] = _quant(W[k], wl.dtype)
    lo, hi = np.log(1e-3), np.log(1e-1)
    dt0 = np.exp(_rng(sd, hook, "dt_proj_b").uniform(lo, hi, size=E))
    W["dt_proj_b"] = (dt0 + np.log(-np.expm1(-dt0))).astype(np.float32)
    W["A_log"] = np.tile(np.log(np.arange(1, N + 1, dtype=np.float64)), (E, 1)).astype(np.float32)
    W["Dskip"] = np.ones(E, dtype=np.float32)
    if affine_ln:
        W["ln_w"] = (1 + 0.1 * _rng(sd, hook, "ln_w").standard_normal(D)).astype(np.float32)
        W["ln_b"] = (0.1 * _rng(sd, hook, "ln_b").standard_normal(D)).astype(np.float32)
    else:
        W["ln_w"] = np.ones(D, dtype=np.float32)
        W["ln_b"] = np.zeros(D, dtype=np.float32)
    if s is None:
        s = float(np.float32(0.5 * _rng(sd, hook, "s").standard_normal()))
    W["s"] = np.float32(s)
    return W


def make_aux(seed: int, shape, kind="normal", scale=1.0, lo=None, hi=None) -> np.ndarray:
    """Extra seeded arrays for operator-level tests (scan/conv inputs)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 999, TENSOR_IDS["aux"], *shape]))
    if kind == "uniform":
        return rng.uniform(lo, hi, size=shape).astype(np.float32)
    return (scale * rng.standard_normal(size=shape)).astype(np.float32)
