"""Benchmark of the ReverseMambaLayer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload serve_b8]

A step is one r2l_layer_fwd call (in_proj, conv + x_proj, reverse scan,
out_proj, LayerNorm + gated residual) over the whole synthetic batch, with
inputs and weights already resident in HBM.  Prints one JSON line.  For the
multi-hook workloads (stack7, denoise_g32, denoise_g128) a step applies every
hook in order, and `value` counts layer-tokens (tokens x hooks) per second;
the denoise-step workloads replay each step as one captured HIP graph
(--graph on|off|auto) and report us_per_step.

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
    ap.add_argument("--graph", choices=("auto", "on", "off"), default="auto",
                    help="replay each step as one captured HIP graph (auto: for the denoise-step workloads)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time spent on the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time r2l_layer_bwd (forward recompute + gradients) instead of the forward")
    ap.add_argument("--saved", action="store_true",
                    help="with --backward: the forward runs with R2L_FLAG_TRAIN and the backward reads its "
                         "activations instead of recomputing them")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    ap.add_argument("--calib-mib", type=float, default=0.0,
                    help="with --summarize: size of the calibration copy that was profiled")
    ap.add_argument("--summarize", nargs="+", metavar=("OUT_MD", "DIR"),
                    help="write a profile summary from rocprofv3 outputs instead of benchmarking: "
                         "OUT_MD TRACE_DIR [FETCH_DIR WRITE_DIR]")
    ap.add_argument("--summarize-pmc", nargs="+", metavar=("OUT_MD", "DIR"),
                    help="write a markdown summary of rocprofv3 --pmc runs (one DIR per counter pass) and exit")
    ap.add_argument("--summarize-args", default="",
                    help="with --summarize: the bench.py arguments of the profiled runs (for the header)")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.summarize_args)
        return
    if args.summarize:
        summarize_profiles(args.summarize, args.calib_mib * 1024.0, args.summarize_args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library runs the layer on a single MI355X "
              "(sequences would shard across GPUs with no communication). "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    if args.backward:
        bench_backward(args)
        return

    import torch

    from reverse_selective_scan_amd import binding as B
    from reverse_selective_scan_amd import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = synth.workloads()[args.workload]
    assert wl.dtype == "bf16"
    T, D, E, N, R = wl.n_tokens, wl.d_model, wl.d_inner, wl.d_state, wl.dt_rank
    P = R + 2 * N
    # one weight set per hook; a step applies the hooks in order (identity
    # between hooks), ping-ponging between two hidden-state buffers
    Ws = [synth.make_weights(wl, hook=k) for k in range(wl.n_hooks)]
    W = Ws[0]
    h_np = synth.make_hidden(wl)
    wd = [B.to_device_weights(Wk, torch.bfloat16, dev) for Wk in Ws]
    h = torch.from_numpy(h_np).to(torch.bfloat16).to(dev)
    out = torch.empty_like(h)
    cu, nseq, max_seqlen = B.cu_seqlens_device(wl.cu_seqlens(), T, dev)
    ws_bytes = B.r2l_layer_workspace_bytes(B.dims_of(wd[0]), B.R2L_BF16, T, nseq, max_seqlen)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    bufs = (h, out)

    def eager_step():
        for k, w in enumerate(wd):
            B.r2l_layer_fwd(bufs[k % 2], w, cu, out=bufs[(k + 1) % 2], workspace=ws, nseq=nseq,
                            max_seqlen=max_seqlen)

    step = eager_step
    use_graph = args.graph == "on" or (args.graph == "auto" and wl.name.startswith("denoise"))

    if args.copy_calib_mib > 0:
        # a plain copy kernel of known size, for scaling the HBM byte counters
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    print(f"[bench] workload {wl.name}: T={T} D={D} E={E} N={N} R={R}, hooks {wl.n_hooks}, "
          f"warmup {args.warmup}, graph {use_graph}", flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if use_graph:
        # the whole step (every hook) as one HIP graph on a side stream; the
        # library launches on the caller's current stream and allocates nothing
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            eager_step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager_step()
        torch.cuda.synchronize()
        step = graph.replay
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
    tok_s = T * wl.n_hooks / (ms_step * 1e-3)
    print(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step (wall {t_wall:.2f}s)", flush=True)

    # the layer time as a median of single calls with the caches flushed in
    # between (a 512 MiB write, past the 256 MB last-level cache), one event
    # pair per call; reported beside the back-to-back throughput
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    per_call = []
    for _ in range(args.steps):
        flush.fill_(1)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        step()
        c1.record(stream)
        torch.cuda.synchronize()
        per_call.append(c0.elapsed_time(c1))
    del flush
    flushed_ms = float(np.median(per_call))
    # a measured copy peak (device-to-device copy of 1 GiB, read + write
    # bytes over the best of five), beside the published 8 TB/s
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copy_ms = []
    for _ in range(5):
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_ms.append(c0.elapsed_time(c1))
    del src, dst
    copy_gbs = 2.0 * (1 << 30) / (min(copy_ms) * 1e-3) / 1e9
    l4096 = None
    if wl.name == "serve_b8":
        # the same batch at L = 4096 (the prompt alone: B = 8 x 4096 tokens)
        cu4 = np.arange(0, 8 * 4096 + 1, 4096)
        h4 = h[:8 * 4096].clone()
        o4 = torch.empty_like(h4)
        cu4_d, n4, m4 = B.cu_seqlens_device(cu4, 8 * 4096, dev)
        for _ in range(args.warmup):
            B.r2l_layer_fwd(h4, wd[0], cu4_d, out=o4, workspace=ws, nseq=n4, max_seqlen=m4)
        torch.cuda.synchronize()
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q0.record(stream)
        for _ in range(args.steps):
            B.r2l_layer_fwd(h4, wd[0], cu4_d, out=o4, workspace=ws, nseq=n4, max_seqlen=m4)
        q1.record(stream)
        torch.cuda.synchronize()
        l4096 = 8 * 4096 / (q0.elapsed_time(q1) / args.steps * 1e-3)

    # per-kernel durations (second timed region, events inside the library)
    B.timing_reset()
    B.timing_enable(True)
    for _ in range(args.steps):
        eager_step()
    torch.cuda.synchronize()
    kt = B.timing_read()
    B.timing_enable(False)

    Tf = fused_ln_rows(T, D, E)   # rows of the fused out_proj + LayerNorm kernel; the rest run unfused
    flops = {"in_proj_gemm": 2.0 * T * D * 2 * E, "out_proj_gemm": 2.0 * (T - Tf) * E * D,
             "out_proj_ln": 2.0 * Tf * E * D}
    bytes_ = {"conv_xproj": T * (2.0 * E + 4.0 * P),
              "scan_main": T * (2.0 * E + 2.0 * E + 4.0 * P + 2.0 * E),
              "ln_gate": (T - Tf) * D * 8.0}
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
        tr = measured_traffic(dom)
        traffic = None if tr is None else tr["read_bytes"] + tr["write_bytes"]
        if dom in flops:
            roofline = {"kernel": dom, "bound": "mfma", "achieved": k["achieved_tflops"],
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": k["frac"], "traffic": traffic,
                        "traffic_detail": tr}
        elif dom in bytes_:
            roofline = {"kernel": dom, "bound": "hbm", "achieved": k["achieved_gbs"], "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": k["frac"], "traffic": traffic,
                        "traffic_detail": tr}
        if dom == "scan_main":
            # the recurrence is bound by the vector ALU, not by HBM: report that roofline
            roofline = {"kernel": dom, "bound": "alu", "achieved": k["valu_gops"], "peak": round(VALU_PEAK_GOPS, 1),
                        "unit": "Gop/s (state-update lane-ops, 5 per state per token)", "frac": k["valu_frac"],
                        "hbm_gbs": k["achieved_gbs"], "hbm_frac": k["frac"], "traffic": traffic,
                        "traffic_detail": tr}
    scan = kernels.get("scan_main", {})

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, W, h_np, args.cpu_seconds)

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
                   "d_inner": E, "d_state": N, "dt_rank": R, "d_conv": wl.d_conv, "hooks": wl.n_hooks,
                   "graph": use_graph, "state_dtype": "f32", "note": wl.note},
        "us_per_step": round(ms_step * 1e3, 2),
        "flushed_median_ms": round(flushed_ms, 4),
        "tokens_per_s_L4096": None if l4096 is None else round(l4096, 1),
        "scan_hbm_gbs": scan.get("achieved_gbs"),
        "scan_hbm_frac": scan.get("frac"),
        "copy_peak_gbs": round(copy_gbs, 1),
        "scan_frac_of_copy": (None if scan.get("achieved_gbs") is None
                              else round(scan["achieved_gbs"] / copy_gbs, 4)),
        "ln_frac_of_copy": (None if kernels.get("ln_gate", {}).get("achieved_gbs") is None
                            else round(kernels["ln_gate"]["achieved_gbs"] / copy_gbs, 4)),
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def bench_backward(args):
    """One step = one r2l_layer_bwd call over the whole batch: the forward
    recomputed into the workspace, then every gradient (h, the Mamba block's
    weights, the LayerNorm's and s).  GEMM work per step, with TDE = T*D*E:
    recompute 6 TDE (in_proj 4, out_proj 2), backward 12 TDE (out_proj input
    2 and weight 2, in_proj input 4 and weight 4), plus the x_proj/dt_proj
    products, which are small."""
    import torch

    from reverse_selective_scan_amd import binding as B
    from reverse_selective_scan_amd import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = synth.workloads()[args.workload]
    T, D, E, N, R = wl.n_tokens, wl.d_model, wl.d_inner, wl.d_state, wl.dt_rank
    P = R + 2 * N
    W = synth.make_weights(wl, affine_ln=True)
    w = B.to_device_weights(W, torch.bfloat16, dev)
    h = torch.from_numpy(synth.make_hidden(wl)).to(torch.bfloat16).to(dev)
    g = torch.from_numpy(synth.make_hidden(wl, hook=9)).to(torch.bfloat16).to(dev)
    cu, nseq, max_seqlen = B.cu_seqlens_device(wl.cu_seqlens(), T, dev)
    need = B.r2l_layer_bwd_workspace_bytes(B.dims_of(w), B.R2L_BF16, T, nseq, max_seqlen)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    dh = torch.empty_like(h)
    grads = {k: torch.empty(w[k].shape, dtype=torch.float32, device=dev) for k, _ in B.Grads._fields_}
    saved = None
    out = torch.empty_like(h)
    if args.saved:
        saved = torch.empty(B.r2l_layer_train_workspace_bytes(B.dims_of(w), B.R2L_BF16, T, nseq, max_seqlen),
                            dtype=torch.uint8, device=dev)

    def fwd_train():
        B.r2l_layer_fwd(h, w, cu, out=out, flags=B.R2L_FLAG_TRAIN, workspace=saved, nseq=nseq,
                        max_seqlen=max_seqlen)

    def step():
        B.r2l_layer_bwd(h, w, cu, g, dh=dh, workspace=ws, grads=grads, nseq=nseq, max_seqlen=max_seqlen,
                        saved=saved)

    print(f"[bench] backward {wl.name}: T={T} D={D} E={E} N={N} R={R}, workspace {need / 2**30:.2f} GiB, "
          f"saved activations {args.saved}, warmup {args.warmup}", flush=True)
    fwd_ms = None
    if args.saved:
        for _ in range(args.warmup):
            fwd_train()
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record(torch.cuda.current_stream())
        for _ in range(args.steps):
            fwd_train()
        f1.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        fwd_ms = f0.elapsed_time(f1) / args.steps   # (the saved buffer holds the last call's activations)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] timed {args.steps} backward steps: {ms_step:.3f} ms/step", flush=True)

    B.timing_reset()
    B.timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = B.timing_read()
    B.timing_enable(False)
    TDE = float(T) * D * E
    flops = {"bwd_in_proj": 4 * TDE, "bwd_out_proj": 2 * TDE, "bwd_dyg": 2 * TDE, "bwd_dWout": 2 * TDE,
             "bwd_dh_branch": 4 * TDE, "bwd_dWin": 4 * TDE, "bwd_dt_proj": 2.0 * T * R * E,
             "bwd_ddelta": 2.0 * T * R * E, "bwd_dWdt": 2.0 * T * R * E, "bwd_dux": 2.0 * T * P * E,
             "bwd_dWx": 2.0 * T * P * E}
    kernels = {}
    for name, (tot_ms, cnt) in sorted(kt.items(), key=lambda kv: -kv[1][0]):
        avg = tot_ms / max(cnt, 1)
        k = {"avg_ms": round(avg, 4), "launches": int(cnt), "share": round(tot_ms / args.steps / ms_step, 4)}
        if name in flops:
            tf = flops[name] / (avg * 1e-3) / 1e12
            k.update(bound="mfma", achieved_tflops=round(tf, 1), frac=round(tf / MFMA_BF16_PEAK_TFLOPS, 4))
        kernels[name] = k
    gemm_ms = sum(kernels[n]["avg_ms"] for n in flops if n in kernels)
    gemm_tflops = sum(flops.values()) / (gemm_ms * 1e-3) / 1e12 if gemm_ms else None
    what = "saved forward activations" if args.saved else "forward recompute"
    rec = {
        "metric": f"R2L layer backward tokens/sec ({what} + all gradients) at B=8,L=4096,D=2048",
        "value": round(T / (ms_step * 1e-3), 1),
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
        "config": {"workload": wl.name, "pass": "backward", "saved_activations": bool(args.saved), "batch": nseq,
                   "seq_len": max_seqlen, "n_tokens": T, "d_model": D, "d_inner": E, "d_state": N, "dt_rank": R,
                   "d_conv": wl.d_conv},
        "train_forward_ms": None if fwd_ms is None else round(fwd_ms, 4),
        "train_step_ms": None if fwd_ms is None else round(fwd_ms + ms_step, 4),
        "gemm_ms": round(gemm_ms, 4),
        "gemm_tflops": None if gemm_tflops is None else round(gemm_tflops, 1),
        "gemm_frac": None if gemm_tflops is None else round(gemm_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "kernels": kernels,
    }
    print(json.dumps(rec), flush=True)


def fused_ln_rows(T, D, E):
    """Token rows the library gives to its fused out_proj + LayerNorm kernel:
    whole rounds of 256-row blocks over a grid of 8 x NT x c blocks (NT =
    D / 256 column tiles per row block, at most one block per CU)."""
    import torch
    if D % 256 or E % 32:
        return 0
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    nt = D // 256
    grid = 8 * nt * (ncu // (8 * nt))
    if grid <= 0:
        return 0
    rb_round = grid // nt
    return ((T // 256) // rb_round) * rb_round * 256


KERNEL_SOURCES = {  # the source file that defines each timed kernel
    "in_proj_gemm": "gemm.hip", "out_proj_gemm": "gemm.hip", "out_proj_ln": "gemm.hip", "conv_xproj": "conv.hip",
    "conv_sum": "conv.hip",
    "scan_main": "scan.hip", "scan_summary": "scan.hip", "ln_gate": "ln.hip", "plan_chunks": "scan.hip",
}
# The launches behind each timed label of the serving-shape forward, as
# substrings of the demangled names in rocprofv3 output; each launches once
# per step, so a label's time and traffic per step are sums over its parts.
ROCPROF_NAMES = {
    "in_proj_gemm": ["gemm_bf16_pers_kernel<4>", "gemm_bf16_mid_kernel<true>",
                     "gemm_small_reduce4_kernel<128, 128, false>"],
    "out_proj_gemm": ["gemm_bf16_big_kernel<true, 8, false>", "gemm_bf16_mid_kernel<true>",
                      "gemm_small_reduce4_kernel<128, 128, true>"],
    "out_proj_ln": ["gemm_out_ln_kernel"],
    "conv_xproj": ["conv_xproj_sk_kernel<5, false>"], "conv_sum": ["sk_sum_kernel"],
    "scan_main": ["E, false, 4, false, false>(r2l::ScanArgs)"],
    "scan_summary": ["E, true, 4, false, false>(r2l::ScanArgs)"],
    "ln_gate": ["ln_gate_kernel"], "plan_chunks": ["plan_chunks_kernel"],
}
PROFILE_JSON = os.path.join(ROOT, "profiles", "traffic_serve_b8.json")


def _source_hash(kernel):
    """Hash of the code of the file that defines `kernel`, comments and
    whitespace removed: an edited comment keeps the stored counters valid,
    any change to the code makes them stale."""
    import hashlib
    import re
    f = os.path.join(ROOT, "reverse_selective_scan_amd", "csrc", KERNEL_SOURCES[kernel])
    code = open(f, encoding="utf-8").read()
    code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
    code = re.sub(r"//[^\n]*", " ", code)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None if there is none or the kernel source changed since."""
    try:
        rec = json.load(open(PROFILE_JSON))["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != _source_hash(kernel):
        return None
    return {"read_bytes": rec["read_bytes"], "write_bytes": rec["write_bytes"],
            "copy_scale": rec["copy_scale"], "source": os.path.relpath(PROFILE_JSON, ROOT)}


def _rocprof_rows(d, name):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", name), recursive=True)
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def summarize_profiles(argv, size_kib=0.0, bench_args=""):
    """OUT_MD TRACE_DIR [FETCH_DIR WRITE_DIR]: kernel-trace stats and, when
    counter runs are given, HBM bytes per dispatch scaled by the copy kernel
    (written to the traffic JSON only for the default forward workload)."""
    out_md, trace_dir = argv[0], argv[1]
    extra = (" " + bench_args.strip()) if bench_args.strip() else ""
    lines = ["# Kernel profile: " + os.path.basename(out_md), "",
             "Commands (from the repository root, TMPDIR=/tmp):", "",
             f"    rocprofv3 --kernel-trace --stats --output-format csv -d {trace_dir} -o run -- "
             "python -u bench.py --steps 10 --warmup 3 --no-cpu-baseline" + extra]
    if len(argv) >= 4:
        lines += [f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d {argv[2]} -o run -- "
                  "python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline --copy-calib-mib 1024" + extra,
                  f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d {argv[3]} -o run -- "
                  "python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline --copy-calib-mib 1024" + extra]
    lines += ["    python bench.py --summarize " + " ".join(argv) +
              (" --calib-mib 1024" if len(argv) >= 4 else "") +
              (f' --summarize-args="{bench_args.strip()}"' if extra else ""), ""]
    stats = _rocprof_rows(trace_dir, "*kernel_stats.csv")
    if stats:
        lines += ["## rocprofv3 --kernel-trace --stats", "", "| kernel | calls | avg us | total ms | % |",
                  "|---|---|---|---|---|"]
        for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
            lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                         f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.1f} |")
        lines.append("")
        if not extra:
            # the timed labels of bench.py: sums of their launches' averages
            lines += ["Per bench.py label (the sum of its launches' average durations; compare with the",
                      "label's avg_ms in bench.py's `kernels`):", "", "| label | launches | avg us per step |",
                      "|---|---|---|"]
            for label, parts in ROCPROF_NAMES.items():
                rows = [r for r in stats if any(p in r["Name"] for p in parts)]
                if rows:
                    lines.append(f"| {label} | {len(rows)} | {sum(float(r['AverageNs']) for r in rows) / 1e3:.1f} |")
            lines.append("")
    if len(argv) >= 4:
        def per_kernel(d, counter):
            acc = {}
            for r in _rocprof_rows(d, "*counter_collection.csv"):
                if r["Counter_Name"] != counter:
                    continue
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
            return acc
        fetch, write = per_kernel(argv[2], "FETCH_SIZE"), per_kernel(argv[3], "WRITE_SIZE")
        copy_k = [k for k in fetch if "copy" in k.lower() or "elementwise" in k.lower()]
        calib = {}
        for k in copy_k:   # the copy dispatch that reads the most is the calibration copy
            f, wr = max(fetch[k]), max(write.get(k, [0]))
            if not calib or f > calib["fetch_kib"]:
                calib = {"kernel": k, "fetch_kib": f, "write_kib": wr}
        rec = {"copy": calib, "kernels": {}}
        lines += ["## HBM traffic (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE, KiB per dispatch)", ""]
        if calib and size_kib:
            rs, ws = size_kib / calib["fetch_kib"], size_kib / calib["write_kib"]
            lines.append(f"Calibration: plain copy of {size_kib:.0f} KiB read as FETCH {calib['fetch_kib']:.0f} KiB, "
                         f"WRITE {calib['write_kib']:.0f} KiB -> scale read x{rs:.4f}, write x{ws:.4f}.")
            lines += ["", "| kernel | FETCH KiB | WRITE KiB | read MB (scaled) | write MB (scaled) |", "|---|---|---|---|---|"]
            for ours, parts in ROCPROF_NAMES.items():
                ks = [k for k in fetch if any(p in k for p in parts)]
                if not ks:
                    continue
                # per step: the sum over the label's launches of each one's average per dispatch
                f = sum(sum(fetch[k]) / len(fetch[k]) for k in ks)
                wr = sum(sum(write[k]) / len(write[k]) for k in ks if k in write)
                rb, wb = f * 1024 * rs, wr * 1024 * ws
                rec["kernels"][ours] = {"fetch_kib": f, "write_kib": wr, "read_bytes": round(rb),
                                        "write_bytes": round(wb), "copy_scale": [round(rs, 5), round(ws, 5)],
                                        "source_sha256": _source_hash(ours)}
                lines.append(f"| {ours} | {f:.0f} | {wr:.0f} | {rb / 1e6:.1f} | {wb / 1e6:.1f} |")
            if not extra:
                json.dump(rec, open(PROFILE_JSON, "w"), indent=1)
        lines.append("")
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc(argv, bench_args=""):
    """OUT_MD DIR...: per bench.py label, each counter averaged over the
    label's dispatches (summed over its launches per step) from rocprofv3
    --pmc runs, with the derived fractions: MFMA busy and VALU active per
    SIMD against the shader clock (GRBM_GUI_ACTIVE counts cycles on each of
    the 8 XCDs; the SQ counters count per wave, and ACTIVE / BUSY ones in
    units of 4 cycles)."""
    out_md, dirs = argv[0], argv[1:]
    extra = (" " + bench_args.strip()) if bench_args.strip() else ""
    lines = ["# Counter profile: " + os.path.basename(out_md), "",
             "Commands (from the repository root, TMPDIR=/tmp; one counter pass per run):", ""]
    counters = {}
    for d in dirs:
        names = sorted({r["Counter_Name"] for r in _rocprof_rows(d, "*counter_collection.csv")})
        lines.append(f"    rocprofv3 --pmc {' '.join(names)} --output-format csv -d {d} -o run -- "
                     "python -u bench.py --steps 2 --warmup 1 --no-cpu-baseline" + extra)
        for r in _rocprof_rows(d, "*counter_collection.csv"):
            for label, parts in ROCPROF_NAMES.items():
                if any(p in r["Kernel_Name"] for p in parts):
                    counters.setdefault(label, {}).setdefault(r["Counter_Name"], {}).setdefault(
                        r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    lines += ["    python bench.py --summarize-pmc " + " ".join(argv) +
              (f' --summarize-args="{bench_args.strip()}"' if extra else ""), ""]
    names = sorted({c for lab in counters.values() for c in lab})
    lines += ["## Counters per step (averaged over dispatches, summed over a label's launches)", "",
              "| label | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    per = {}
    for label, cs in counters.items():
        per[label] = {c: sum(sum(v) / len(v) for v in ks.values()) for c, ks in cs.items()}
        lines.append(f"| {label} | " + " | ".join(f"{per[label].get(c, float('nan')):.4g}" for c in names) + " |")
    lines += ["", "## Derived (per SIMD; 256 CUs x 4 SIMDs, 8 XCDs)", "",
              "| label | clock cycles per XCD | MFMA busy | VALU active | LDS active | VALU instr per wave | "
              "transcendental share |", "|---|---|---|---|---|---|---|"]
    for label, c in per.items():
        gui = c.get("GRBM_GUI_ACTIVE")
        if not gui:
            continue
        cyc = gui / 8.0
        mfma = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
        valu = c.get("SQ_ACTIVE_INST_VALU")
        lds = c.get("SQ_ACTIVE_INST_LDS")
        waves = c.get("SQ_WAVES")
        vi = c.get("SQ_INSTS_VALU")
        tr = c.get("SQ_INSTS_VALU_TRANS_F32")

        def frac(x, scale):
            return f"{x * scale / 1024.0 / cyc:.3f}" if x is not None else "-"
        lines.append(f"| {label} | {cyc:.4g} | {frac(mfma, 1.0)} | {frac(valu, 4.0)} | {frac(lds, 4.0)} | "
                     f"{(vi / waves) if (vi and waves) else float('nan'):.0f} | "
                     f"{(tr / vi) if (tr and vi) else float('nan'):.3f} |")
    lines.append("")
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_baseline(wl, W, h_np, seconds):
    """Time the fp64 oracle on whole sequences of the same workload, taking
    sequences in order until about `seconds` of CPU work have been done."""
    from threadpoolctl import threadpool_info

    from oracle import r2l_oracle as O

    cu = wl.cu_seqlens()
    done_tok, done_seq, dt = 0, 0, 0.0
    while done_seq < wl.nseq and (dt < seconds or done_seq == 0):
        t0, t1 = int(cu[done_seq]), int(cu[done_seq + 1])
        print(f"[bench] cpu baseline: oracle on sequence {done_seq} ({t1 - t0} tokens)", flush=True)
        t = time.perf_counter()
        O.reverse_mamba_layer(h_np[t0:t1], np.array([0, t1 - t0]), W, float(W["s"]))
        dt += time.perf_counter() - t
        done_tok += t1 - t0
        done_seq += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    return {"value": round(done_tok / dt, 1), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {done_seq} whole sequence(s) of {wl.name} ({done_tok} tokens), fp64 numpy oracle, "
                      f"{dt:.1f} s with a BLAS pool of {threads} thread(s)"}


if __name__ == "__main__":
    main()
