"""GPU parity of r2l_layer_fwd against the fp64 oracle on the workload
shapes, plus the invariants the pages fix (zero-gate identity,
right-context-only, sequence isolation) checked bit for bit on the GPU.

Full-size workloads are checked on whole sequences where the oracle is
fast enough, and otherwise on sequence suffixes: the layer's output at
position i depends only on tokens i.. of its sequence (pinned on the oracle
by test_oracle.test_right_context_only and on the GPU below), so the oracle
run on h[i:end] gives the exact reference for those positions."""
import time

import numpy as np
import pytest
import torch

from oracle import r2l_oracle as O
from parity import TOL_BF16, TOL_BF16_BRANCH, TOL_F32, err_f32, err_rms, report, to_np
from reverse_selective_scan_amd import binding as B
from reverse_selective_scan_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(name):
    print(f"\n[case] {name}", flush=True)


def _dtype(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def _gpu_layer(wl, W, h, cu, flags=0, branch=False, inplace=False, s=None):
    w = B.to_device_weights(W, _dtype(wl), DEV)
    if s is not None:
        w["s"] = B.gate_tensor(s, DEV)
    hd = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(_dtype(wl)).to(DEV)
    br = torch.empty(hd.shape, dtype=torch.float32, device=DEV) if branch else None
    out = B.r2l_layer_fwd(hd, w, cu, flags=flags, branch_out=br, out=hd if inplace else None)
    torch.cuda.synchronize()
    return to_np(out), (to_np(br) if branch else None)


def _tol(wl):
    return (err_f32, TOL_F32) if wl.dtype == "f32" else (err_rms, TOL_BF16)


# ---------------------------------------------------------------------------
# tiny fp32 workload (B=1 L=64 D=64 E=128 N=16 R=4)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("use_ln", [True, False])
def test_tiny_f32_matches_oracle(use_ln):
    wl = synth.workloads()["tiny_f32"]
    _case(f"tiny_f32 ln={use_ln}")
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    ref, rref = O.reverse_mamba_layer(h, cu, W, float(W["s"]), use_ln=use_ln, return_branch=True)
    g, gr = _gpu_layer(wl, W, h, cu, flags=0 if use_ln else B.R2L_FLAG_NO_LN, branch=True)
    f, tol = _tol(wl)
    assert report("tiny out", f(g, ref), tol) <= tol
    assert report("tiny branch", f(gr, rref), tol) <= tol


def test_tiny_f32_zero_gate_is_identity():
    wl = synth.workloads()["tiny_f32"]
    _case("tiny_f32 s=0")
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    g, _ = _gpu_layer(wl, W, h, cu, s=0.0)
    assert np.array_equal(g.astype(np.float32).view(np.uint32), h.view(np.uint32))


# ---------------------------------------------------------------------------
# small bf16 layers: ragged varlen, sequences shorter than the conv, chunk carries
# ---------------------------------------------------------------------------
SMALL = dict(d_model=256, d_inner=512, dt_rank=16)


@pytest.mark.parametrize("lens", [[1], [3], [700], [5, 0, 130, 1, 300, 2], [1000, 64, 333]])
@pytest.mark.parametrize("affine", [False, True])
def test_small_bf16_varlen_matches_oracle(lens, affine):
    _case(f"small bf16 lens={lens} affine={affine}")
    wl = synth.custom(lens, seed=7, h_kind="rms", **SMALL)
    W = synth.make_weights(wl, affine_ln=affine)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    ref, rref = O.reverse_mamba_layer(h, cu, W, float(W["s"]), return_branch=True)
    g, gr = _gpu_layer(wl, W, h, cu, branch=True)
    assert report("out", err_rms(g, ref), TOL_BF16) <= TOL_BF16
    assert report("branch", err_rms(gr, rref), TOL_BF16_BRANCH) <= TOL_BF16_BRANCH


def test_bf16_split_k_conv_path_matches_oracle():
    """More than 256 tiles of 128 tokens: the conv + x_proj step runs split
    along K over one block per CU (tiles cut between two blocks, partial sums
    added afterwards); odd x_proj width (R = 5, P = 37) and sequences of 1
    and 7 tokens inside split tiles.  (At d_model 64 the bf16 roundings alone
    exceed the tolerance on the LayerNorm branch, so the small-model widths
    are used.)"""
    lens = [20000, 7, 13000, 1, 300]
    _case(f"split-K conv path lens={lens}")
    wl = synth.custom(lens, seed=21, h_kind="rms", d_model=256, d_inner=512, dt_rank=5)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    ref, rref = O.reverse_mamba_layer(h, cu, W, float(W["s"]), return_branch=True)
    g, gr = _gpu_layer(wl, W, h, cu, branch=True)
    assert report("out", err_rms(g, ref), TOL_BF16) <= TOL_BF16
    assert report("branch", err_rms(gr, rref), TOL_BF16_BRANCH) <= TOL_BF16_BRANCH


@pytest.mark.parametrize("hint", ["too_small", "too_large"])
def test_max_seqlen_hint_does_not_change_results(hint):
    """max_seqlen only plans the scan's time chunks: a value below the true
    longest length (one chunk per sequence, no summary pass) or far above it
    (chunks and a carry pass) must still give the oracle's result."""
    lens = [900, 5, 300, 1]
    _case(f"max_seqlen {hint} lens={lens}")
    wl = synth.custom(lens, seed=23, h_kind="rms", **SMALL)
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    ref = O.reverse_mamba_layer(h, cu, W, float(W["s"]))
    w = B.to_device_weights(W, torch.bfloat16, DEV)
    hd = torch.from_numpy(h).to(torch.bfloat16).to(DEV)
    cu_d = torch.from_numpy(np.asarray(cu, np.int32)).to(DEV)
    ms = 2 if hint == "too_small" else 100000
    g = to_np(B.r2l_layer_fwd(hd, w, cu_d, nseq=len(lens), max_seqlen=ms))
    assert report(f"out (max_seqlen {ms})", err_rms(g, ref), TOL_BF16) <= TOL_BF16


def test_small_bf16_no_ln_and_in_place():
    _case("small bf16 NO_LN in place")
    wl = synth.custom([200, 57], seed=8, h_kind="rms", **SMALL)
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    ref = O.reverse_mamba_layer(h, cu, W, float(W["s"]), use_ln=False)
    g, _ = _gpu_layer(wl, W, h, cu, flags=B.R2L_FLAG_NO_LN, inplace=True)
    assert report("out no-ln", err_rms(g, ref), TOL_BF16) <= TOL_BF16


def test_small_bf16_right_context_only_bitwise():
    """§3.4: the stream at position i summarises tokens j >= i.  Perturbing
    token j must leave every output right of j (and every other sequence)
    bit-identical, and must change the output at j."""
    _case("right-context-only")
    wl = synth.custom([900, 300], seed=9, h_kind="rms", **SMALL)
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    base, _ = _gpu_layer(wl, W, h, cu)
    for j in (0, 129, 450, 899):
        h2 = h.copy()
        h2[j] = synth.bf16_round(h2[j] + 0.5)
        pert, _ = _gpu_layer(wl, W, h2, cu)
        assert np.array_equal(pert[j + 1:], base[j + 1:]), j
        assert not np.array_equal(pert[j], base[j]), j


def test_small_bf16_sequence_isolation_and_determinism():
    _case("isolation + determinism")
    wl = synth.custom([400, 250, 330], seed=10, h_kind="rms", **SMALL)
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    base, _ = _gpu_layer(wl, W, h, cu)
    again, _ = _gpu_layer(wl, W, h, cu)
    assert np.array_equal(base, again)
    h2 = h.copy()
    h2[cu[1]:cu[2]] = synth.bf16_round(h2[cu[1]:cu[2]] * -1.5)
    pert, _ = _gpu_layer(wl, W, h2, cu)
    assert np.array_equal(pert[:cu[1]], base[:cu[1]])
    assert np.array_equal(pert[cu[2]:], base[cu[2]:])


def test_small_bf16_gate_linearity():
    """§3.4 step 4: the branch does not depend on s; h+ - h = tanh(s) r."""
    _case("gate linearity")
    wl = synth.custom([500], seed=11, h_kind="rms", **SMALL)
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    g1, r1 = _gpu_layer(wl, W, h, cu, branch=True, s=0.3)
    g2, r2 = _gpu_layer(wl, W, h, cu, branch=True, s=-1.2)
    assert np.array_equal(r1, r2)
    for g, s in ((g1, 0.3), (g2, -1.2)):
        ref = synth.bf16_round((h + np.tanh(np.float32(s)) * r1).astype(np.float32))
        assert err_rms(g, ref) <= 8e-3   # only the final rounding may differ


# ---------------------------------------------------------------------------
# workload shapes at full size
# ---------------------------------------------------------------------------
def _suffix_ref(h, W, s, t0, t1, start):
    """Exact oracle outputs for positions [start, t1) of sequence [t0, t1)."""
    return O.reverse_mamba_layer(h[start:t1], [0, t1 - start], W, s)


def test_single_2k_matches_oracle_and_zero_gate():
    wl = synth.workloads()["single_2k"]
    _case("single_2k (B=1 L=2048 D=2048)")
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    t = time.time()
    ref, rref = O.reverse_mamba_layer(h, cu, W, float(W["s"]), return_branch=True)
    print(f"oracle {time.time() - t:.1f}s", flush=True)
    g, gr = _gpu_layer(wl, W, h, cu, branch=True)
    assert report("single_2k out", err_rms(g, ref), TOL_BF16) <= TOL_BF16
    assert report("single_2k branch", err_rms(gr, rref), TOL_BF16_BRANCH) <= TOL_BF16_BRANCH
    g0, _ = _gpu_layer(wl, W, h, cu, s=0.0)
    assert np.array_equal(g0.astype(np.float32).view(np.uint32), h.view(np.uint32))


def test_serve_b8_matches_oracle():
    wl = synth.workloads()["serve_b8"]
    _case("serve_b8 (B=8 L=4128 D=2048)")
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    s = float(W["s"])
    g, _ = _gpu_layer(wl, W, h, cu)
    t = time.time()
    t0, t1 = int(cu[0]), int(cu[1])
    ref = O.reverse_mamba_layer(h[t0:t1], [0, t1 - t0], W, s)
    assert report("serve_b8 seq0 full", err_rms(g[t0:t1], ref), TOL_BF16) <= TOL_BF16
    for q in range(1, wl.nseq):
        t0, t1 = int(cu[q]), int(cu[q + 1])
        ref = _suffix_ref(h, W, s, t0, t1, t1 - 384)
        assert report(f"serve_b8 seq{q} suffix", err_rms(g[t1 - 384:t1], ref), TOL_BF16) <= TOL_BF16
    print(f"oracle {time.time() - t:.1f}s", flush=True)


def test_stack7_matches_oracle():
    """Seven hooks applied in sequence (identity between hooks).  The hidden
    stream between hooks is a bf16 tensor on both sides: the oracle rounds
    each hook's output to bf16 before feeding the next hook, as the stack's
    input itself is bf16.

    Per hook (strict, 2e-2): GPU hook k run on the oracle's bf16 stream at
    position k against the oracle's fp64 output of hook k.
    End to end (GPU output feeding the next GPU hook): each hook's error
    passes the residual path unchanged and the hooks' errors add, so the
    chain is held to the sum of the per-hook bounds, 7 x 2e-2; the measured
    value is printed.  (A single bf16 rounding flip of the stream at
    |h| in [4, 8) already moves an element by 2^-5, about 3e-2 of the
    stream's RMS, so 2e-2 end to end is out of reach for any bf16 stream.)"""
    wl = synth.workloads()["stack7"]
    _case("stack7 (7 hooks, B=8 L=4096 D=2048)")
    h0, cu = synth.make_hidden(wl), wl.cu_seqlens()
    Ws = [synth.make_weights(wl, hook=k) for k in range(wl.n_hooks)]
    wd = [B.to_device_weights(W, torch.bfloat16, DEV) for W in Ws]
    # GPU chain over the whole batch
    hd = torch.from_numpy(h0).to(torch.bfloat16).to(DEV)
    for w in wd:
        B.r2l_layer_fwd(hd, w, cu, out=hd)
    torch.cuda.synchronize()
    g_chain = to_np(hd)

    t = time.time()
    for q, start in ((0, None), (3, 256), (6, 256)):     # sequence 0 whole, suffixes of two others
        t0, t1 = int(cu[q]), int(cu[q + 1])
        a = t0 if start is None else t1 - start
        cur = h0[a:t1].astype(np.float64)
        for k, W in enumerate(Ws):
            ref = O.reverse_mamba_layer(cur, [0, t1 - a], W, float(W["s"]))
            hin = torch.from_numpy(cur.astype(np.float32)).to(torch.bfloat16).to(DEV)
            g = to_np(B.r2l_layer_fwd(hin, wd[k], [0, t1 - a]))
            assert report(f"stack7 seq{q} rows {a - t0}.. hook {k}", err_rms(g, ref), TOL_BF16) <= TOL_BF16
            cur = synth.bf16_round(ref.astype(np.float32)).astype(np.float64)
        e2e = err_rms(g_chain[a:t1], ref)
        assert report(f"stack7 seq{q} end-to-end", e2e, 7 * TOL_BF16) <= 7 * TOL_BF16
    print(f"oracle {time.time() - t:.1f}s", flush=True)


def test_varlen16_matches_oracle():
    wl = synth.workloads()["varlen16"]
    _case(f"varlen16 (T={wl.n_tokens}, lengths {min(wl.lengths)}..{max(wl.lengths)})")
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    s = float(W["s"])
    g, _ = _gpu_layer(wl, W, h, cu)
    t = time.time()
    order = np.argsort(wl.lengths)
    for q in (int(order[0]), int(order[len(order) // 2])):      # shortest and median, in full
        t0, t1 = int(cu[q]), int(cu[q + 1])
        ref = O.reverse_mamba_layer(h[t0:t1], [0, t1 - t0], W, s)
        assert report(f"varlen16 seq{q} (L={t1 - t0}) full", err_rms(g[t0:t1], ref), TOL_BF16) <= TOL_BF16
    for q in range(wl.nseq):
        t0, t1 = int(cu[q]), int(cu[q + 1])
        ref = _suffix_ref(h, W, s, t0, t1, t1 - 300)
        assert report(f"varlen16 seq{q} suffix", err_rms(g[t1 - 300:t1], ref), TOL_BF16) <= TOL_BF16
    print(f"oracle {time.time() - t:.1f}s", flush=True)


def test_long32k_matches_oracle():
    wl = synth.workloads()["long32k"]
    _case("long32k (B=1 L=32768)")
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    g, _ = _gpu_layer(wl, W, h, cu)
    t = time.time()
    L = wl.lengths[0]
    ref = _suffix_ref(h, W, float(W["s"]), 0, L, L - 6144)   # spans several scan chunks
    assert report("long32k suffix 6144", err_rms(g[L - 6144:], ref), TOL_BF16) <= TOL_BF16
    print(f"oracle {time.time() - t:.1f}s", flush=True)


# ---------------------------------------------------------------------------
# denoise step: seven hooks on the B=8 generation blocks alone
# ---------------------------------------------------------------------------
def _denoise_setup(wl):
    h0, cu = synth.make_hidden(wl), wl.cu_seqlens()
    Ws = [synth.make_weights(wl, hook=k) for k in range(wl.n_hooks)]
    wd = [B.to_device_weights(W, torch.bfloat16, DEV) for W in Ws]
    return h0, cu, Ws, wd


@pytest.mark.parametrize("name", ["denoise_g32", "denoise_g128"])
def test_denoise_step_matches_oracle(name):
    """Every hook of one denoise step on the oracle's bf16 stream (strict),
    and the GPU chain end to end (sum of the per-hook bounds, as for the
    seven-hook stack), over all eight blocks."""
    wl = synth.workloads()[name]
    _case(f"{name} (7 hooks, B=8 x G={wl.lengths[0]})")
    h0, cu, Ws, wd = _denoise_setup(wl)
    hd = torch.from_numpy(h0).to(torch.bfloat16).to(DEV)
    for w in wd:
        B.r2l_layer_fwd(hd, w, cu, out=hd)
    torch.cuda.synchronize()
    g_chain = to_np(hd)
    cur = h0.astype(np.float64)
    for k, W in enumerate(Ws):
        ref = O.reverse_mamba_layer(cur, cu, W, float(W["s"]))
        hin = torch.from_numpy(cur.astype(np.float32)).to(torch.bfloat16).to(DEV)
        g = to_np(B.r2l_layer_fwd(hin, wd[k], cu))
        assert report(f"{name} hook {k}", err_rms(g, ref), TOL_BF16) <= TOL_BF16
        cur = synth.bf16_round(ref.astype(np.float32)).astype(np.float64)
    assert report(f"{name} end-to-end", err_rms(g_chain, ref), 7 * TOL_BF16) <= 7 * TOL_BF16


def test_denoise_step_graph_replays_match_eager():
    """The seven hooks captured as one HIP graph: every replay, with eager
    work and synchronisations between replays, equals the eager step bit
    for bit (the library launches on the caller's stream and allocates or
    clears nothing inside the step)."""
    wl = synth.workloads()["denoise_g32"]
    _case("denoise_g32 graph capture, 4 replays")
    h0, cu, Ws, wd = _denoise_setup(wl)
    T = wl.n_tokens
    cud, nseq, ms = B.cu_seqlens_device(cu, T, DEV)
    ws = torch.empty(B.r2l_layer_workspace_bytes(B.dims_of(wd[0]), B.R2L_BF16, T, nseq, ms),
                     dtype=torch.uint8, device=DEV)
    h = torch.from_numpy(h0).to(torch.bfloat16).to(DEV)
    bufs = [torch.empty_like(h), torch.empty_like(h)]

    def step():
        for k, w in enumerate(wd):
            B.r2l_layer_fwd(bufs[k % 2], w, cud, out=bufs[(k + 1) % 2], workspace=ws, nseq=nseq, max_seqlen=ms)
        return bufs[len(wd) % 2]

    bufs[0].copy_(h)
    ref = step().clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bufs[0].copy_(h)
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out_g = step()
    torch.cuda.synchronize()
    other = torch.from_numpy(synth.make_hidden(wl, hook=1)).to(torch.bfloat16).to(DEV)
    for r in range(4):
        bufs[0].copy_(h)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), f"replay {r} differs from the eager step"
        bufs[0].copy_(other)          # eager work on different data between replays
        step()
        torch.cuda.synchronize()
    print("4 replays equal to the eager step", flush=True)
