"""Benchmark of the ReverseMambaLayer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload serve_b8]

A step is one r2l_layer_fwd call (in_proj, conv + x_proj, reverse scan,
out_proj, LayerNorm + gated residual) over the whole synthetic batch, with
inputs and weights already resident in HBM.  Prints one JSON line.

Per-kernel durations come from HIP events that the library records around
each of its launches on the launch stream (a second timed region, so the
headline number carries no event overhead).  Algorithmic work per kernel:

  in_proj_gemm   2*T*D*2E flops                      (MFMA, bf16 peak)
  out_proj_gemm  2*T*E*D flops                       (MFMA, bf16 peak)
  conv_xproj     T*(2E + 4P) bytes                   x read, xdbl written
  scan_main      T*(2E + 2E + 4P + 2E) bytes         x, z, xdbl read; y written
                 and T*E*N*5 VALU lane-ops           (per state: 2 mul, 2 fma, 1 exp)
  ln_gate        T*D*(4 + 2 + 2) bytes               fp32 o read, h read, h+ written
with P = R + 2N and 2-byte bf16 activations.

cpu_baseline: the fp64 oracle, untuned, timed on this host over a bounded
sample (whole sequences of the same workload).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
# VALU: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane-instructions per second
# (non-packed fp32; transcendentals counted as one lane-op)
VALU_PEAK_GOPS = 256 * 4 * 16 * 2.4


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="serve_b8")
    ap.add_argument("--cpu-sample-seqs", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build runs the layer on a single MI355X "
              "(sequences shard across GPUs with no communication; see DESIGN.md). "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    from reverse_selective_scan_amd import binding as B
    from reverse_selective_scan_amd import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = synth.workloads()[args.workload]
    assert wl.dtype == "bf16"
    T, D, E, N, R = wl.n_tokens, wl.d_model, wl.d_inner, wl.d_state, wl.dt_rank
    P = R + 2 * N
    W = synth.make_weights(wl)
    h_np = synth.make_hidden(wl)
    w = B.to_device_weights(W, torch.bfloat16, dev)
    h = torch.from_numpy(h_np).to(torch.bfloat16).to(dev)
    out = torch.empty_like(h)
    cu, nseq, max_seqlen = B.cu_seqlens_device(wl.cu_seqlens(), T, dev)
    ws_bytes = B.r2l_layer_workspace_bytes(B.dims_of(w), B.R2L_BF16, T, nseq, max_seqlen)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def step():
        B.r2l_layer_fwd(h, w, cu, out=out, workspace=ws, nseq=nseq, max_seqlen=max_seqlen)

    print(f"[bench] workload {wl.name}: T={T} D={D} E={E} N={N} R={R}, warmup {args.warmup}", flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps
    tok_s = T / (ms_step * 1e-3)
    print(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step (wall {t_wall:.2f}s)", flush=True)

    # per-kernel durations (second timed region, events inside the library)
    B.timing_reset()
    B.timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = B.timing_read()
    B.timing_enable(False)

    flops = {"in_proj_gemm": 2.0 * T * D * 2 * E, "out_proj_gemm": 2.0 * T * E * D}
    bytes_ = {"conv_xproj": T * (2.0 * E + 4.0 * P),
              "scan_main": T * (2.0 * E + 2.0 * E + 4.0 * P + 2.0 * E),
              "ln_gate": T * D * 8.0}
    kernels = {}
    for name, (tot_ms, cnt) in kt.items():
        avg = tot_ms / max(cnt, 1)
        k = {"avg_ms": round(avg, 4), "launches": int(cnt)}
        if name in flops:
            tf = flops[name] / (avg * 1e-3) / 1e12
            k.update(bound="mfma", achieved_tflops=round(tf, 1), frac=round(tf / MFMA_BF16_PEAK_TFLOPS, 4))
        if name in bytes_:
            gbs = bytes_[name] / (avg * 1e-3) / 1e9
            k.update(bound="hbm", achieved_gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4))
        if name == "scan_main":
            gops = T * E * N * 5.0 / (avg * 1e-3) / 1e9
            k.update(valu_gops=round(gops, 1), valu_frac=round(gops / VALU_PEAK_GOPS, 4))
        kernels[name] = k
    dom = max(kernels, key=lambda n: kernels[n]["avg_ms"]) if kernels else None
    roofline = None
    if dom is not None:
        k = kernels[dom]
        if dom in flops:
            roofline = {"kernel": dom, "bound": "mfma", "achieved": k["achieved_tflops"],
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": k["frac"], "traffic": None}
        elif dom in bytes_:
            roofline = {"kernel": dom, "bound": "hbm", "achieved": k["achieved_gbs"], "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": k["frac"], "traffic": None}
    scan = kernels.get("scan_main", {})

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, W, h_np, args.cpu_sample_seqs)

    rec = {
        "metric": "R2L layer tokens/sec at B=8,L=4096,D=2048; scan HBM GB/s (% peak)",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random-init weights of the layer's shapes)",
        "config": {"workload": wl.name, "batch": nseq, "seq_len": max_seqlen, "n_tokens": T, "d_model": D,
                   "d_inner": E, "d_state": N, "dt_rank": R, "d_conv": wl.d_conv,
                   "state_dtype": "f32", "note": wl.note},
        "scan_hbm_gbs": scan.get("achieved_gbs"),
        "scan_hbm_frac": scan.get("frac"),
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def cpu_baseline(wl, W, h_np, nseqs):
    """Time the fp64 oracle on whole sequences of the same workload."""
    from threadpoolctl import threadpool_info

    from oracle import r2l_oracle as O

    cu = wl.cu_seqlens()
    nseqs = max(1, min(nseqs, wl.nseq))
    t0, t1 = int(cu[0]), int(cu[nseqs])
    sample_cu = cu[: nseqs + 1] - cu[0]
    print(f"[bench] cpu baseline: oracle on {nseqs} sequence(s), {t1 - t0} tokens", flush=True)
    t = time.perf_counter()
    O.reverse_mamba_layer(h_np[t0:t1], sample_cu, W, float(W["s"]))
    dt = time.perf_counter() - t
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {"value": round((t1 - t0) / dt, 1), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{nseqs} whole sequence(s) of {wl.name} ({t1 - t0} tokens), fp64 numpy oracle, "
                      f"{dt:.1f} s on {os.cpu_count()} visible host cores"}


if __name__ == "__main__":
    main()
