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
import bf16_floor
from parity import TOL_BF16, TOL_BF16_BRANCH, TOL_F32, check_bf16, err_f32, err_rms, report, to_np
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
    fo, fr = bf16_floor.layer_rounded(h, cu, W, float(W["s"]))
    g, gr = _gpu_layer(wl, W, h, cu, branch=True)
    check_bf16("out", g, ref, fo, TOL_BF16)
    check_bf16("branch", gr, rref, fr, TOL_BF16_BRANCH)


@pytest.mark.parametrize("dt_rank", [5, 192])
def test_bf16_split_k_conv_path_matches_oracle(dt_rank):
    """More than 256 tiles of 128 tokens: the conv + x_proj step runs split
    along K over the CUs (tiles cut between blocks, partial sums added
    afterwards); sequences of 1 and 7 tokens inside split tiles.  R = 5: odd
    x_proj width (P = 37), two blocks per CU with a 3-stage copy ring;
    R = 192 (P = 224, seven 32-column slices): one block per CU with a
    5-stage ring.  (At d_model 64 the bf16 roundings alone exceed the
    tolerance on the LayerNorm branch, so the small-model widths are used.)"""
    lens = [20000, 7, 13000, 1, 300]
    _case(f"split-K conv path dt_rank={dt_rank} lens={lens}")
    wl = synth.custom(lens, seed=21, h_kind="rms", d_model=256, d_inner=512, dt_rank=dt_rank)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    ref, rref = O.reverse_mamba_layer(h, cu, W, float(W["s"]), return_branch=True)
    fo, fr = bf16_floor.layer_rounded(h, cu, W, float(W["s"]))
    g, gr = _gpu_layer(wl, W, h, cu, branch=True)
    check_bf16("out", g, ref, fo, TOL_BF16)
    check_bf16("branch", gr, rref, fr, TOL_BF16_BRANCH)


@pytest.mark.parametrize("dt_rank", [40, 240, 300])
def test_small_bf16_dt_rank_paths_match_oracle(dt_rank):
    """dt_proj inside the scan on each of its paths: 40 (two MFMA k-steps,
    24 zero columns of padding in the delta split), 240 (x_proj width 272:
    u staged, x_proj on the GEMM, the split made by its own kernel, eight
    k-steps) and 300 (past eight k-steps: dt on the VALU from xdbl)."""
    lens = [300, 1, 77]
    _case(f"small bf16 dt_rank={dt_rank} lens={lens}")
    wl = synth.custom(lens, seed=27, h_kind="rms", d_model=256, d_inner=512, dt_rank=dt_rank)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    ref, rref = O.reverse_mamba_layer(h, cu, W, float(W["s"]), return_branch=True)
    fo, fr = bf16_floor.layer_rounded(h, cu, W, float(W["s"]))
    g, gr = _gpu_layer(wl, W, h, cu, branch=True)
    check_bf16("out", g, ref, fo, TOL_BF16)
    check_bf16("branch", gr, rref, fr, TOL_BF16_BRANCH)


def test_fused_out_proj_layernorm_path_matches_oracle():
    """d_model 512: the fused out_proj + LayerNorm + gated residual kernel
    runs with two column tiles per 256-row block (on 256 compute units:
    128 row blocks per round).  33,308 tokens = one fused round of 32,768
    rows plus 540 rows on the unfused path (out_proj, then the LayerNorm
    kernel), across which sequences run.  Affine LayerNorm and the branch r,
    without the LayerNorm, and s = 0 (an exact copy)."""
    lens = [20000, 7, 13000, 1, 300]
    _case(f"fused out_proj + LN path lens={lens}")
    wl = synth.custom(lens, seed=33, h_kind="rms", d_model=512, d_inner=1024, dt_rank=32)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    s = float(W["s"])
    B.timing_reset()
    B.timing_enable(True)
    g, gr = _gpu_layer(wl, W, h, cu, branch=True)
    names = B.timing_read()
    B.timing_enable(False)
    print(f"kernels: {sorted(names)}", flush=True)
    ref, rref = O.reverse_mamba_layer(h, cu, W, s, return_branch=True)
    fo, fr = bf16_floor.layer_rounded(h, cu, W, s)
    check_bf16("fused out", g, ref, fo, TOL_BF16)
    check_bf16("fused branch", gr, rref, fr, TOL_BF16_BRANCH)
    ref, _ = O.reverse_mamba_layer(h, cu, W, s, use_ln=False, return_branch=True)
    fo, _ = bf16_floor.layer_rounded(h, cu, W, s, use_ln=False)
    g2, _ = _gpu_layer(wl, W, h, cu, flags=B.R2L_FLAG_NO_LN)
    check_bf16("fused out no-ln", g2, ref, fo, TOL_BF16)
    g0, _ = _gpu_layer(wl, W, h, cu, s=0.0)
    assert np.array_equal(g0.astype(np.float32).view(np.uint32), h.view(np.uint32))
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert "out_proj_ln" in names and "ln_gate" in names, names


def test_out_proj_with_d_inner_64_mod_128_matches_oracle():
    """d_inner 576 (9 x 64; out_proj's K is 18 steps of 32, not whole groups
    of four): the fused out_proj + LayerNorm kernel, whose K loop walks whole
    groups of four steps, must not run; the layer takes the unfused path and
    still matches the oracle, with a round's worth of rows at d_model 512."""
    lens = [20000, 7, 13000, 1, 300]
    _case(f"d_inner 576 out_proj lens={lens}")
    wl = synth.custom(lens, seed=39, h_kind="rms", d_model=512, d_inner=576, dt_rank=32)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    s = float(W["s"])
    B.timing_reset()
    B.timing_enable(True)
    g, gr = _gpu_layer(wl, W, h, cu, branch=True)
    names = B.timing_read()
    B.timing_enable(False)
    print(f"kernels: {sorted(names)}", flush=True)
    ref, rref = O.reverse_mamba_layer(h, cu, W, s, return_branch=True)
    fo, fr = bf16_floor.layer_rounded(h, cu, W, s)
    check_bf16("d_inner 576 out", g, ref, fo, TOL_BF16)
    check_bf16("d_inner 576 branch", gr, rref, fr, TOL_BF16_BRANCH)
    assert "out_proj_ln" not in names, names


def test_split_out_proj_layernorm_parts_path_matches_oracle():
    """300 tokens at the pages' widths (D = 2048, E = 4096): out_proj runs on
    the mid-size GEMM split four ways along K, and the LayerNorm kernel adds
    the split's partial tiles itself (no separate sum kernel).  The last
    128-row tile is ragged, and sequences of 100, 7 and 193 tokens run across
    tiles.  Affine LayerNorm with the branch r, without the LayerNorm, and
    s = 0 (an exact copy)."""
    lens = [100, 7, 193]
    _case(f"split out_proj + LN parts path lens={lens}")
    wl = synth.custom(lens, seed=35, h_kind="rms", d_model=2048, d_inner=4096, dt_rank=128)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    s = float(W["s"])
    g, gr = _gpu_layer(wl, W, h, cu, branch=True)
    ref, rref = O.reverse_mamba_layer(h, cu, W, s, return_branch=True)
    fo, fr = bf16_floor.layer_rounded(h, cu, W, s)
    check_bf16("parts out", g, ref, fo, TOL_BF16)
    check_bf16("parts branch", gr, rref, fr, TOL_BF16_BRANCH)
    ref, _ = O.reverse_mamba_layer(h, cu, W, s, use_ln=False, return_branch=True)
    fo, _ = bf16_floor.layer_rounded(h, cu, W, s, use_ln=False)
    g2, _ = _gpu_layer(wl, W, h, cu, flags=B.R2L_FLAG_NO_LN)
    check_bf16("parts out no-ln", g2, ref, fo, TOL_BF16)
    g0, _ = _gpu_layer(wl, W, h, cu, s=0.0)
    assert np.array_equal(g0.astype(np.float32).view(np.uint32), h.view(np.uint32))


_WS_CASES = {
    # small-input conv path; dt_rank 192 makes the delta split (256 columns)
    # wider than the x_proj output (224), so its last columns are never written
    "small_dt192": ([100, 7, 193, 1, 60], 256, 512, 192, 0),
    "small_dt192_l2r": ([100, 7, 193, 1, 60], 256, 512, 192, B.R2L_FLAG_L2R),
    # split-K conv path (more than 256 tiles of 128 tokens), same split widths
    "split_k_dt192": ([20000, 7, 13000, 1, 300], 256, 512, 192, 0),
    # the pages' widths at 300 tokens: in_proj on the mid-size GEMM running the
    # chunk planning, out_proj split along K into the LayerNorm kernel
    "pages_widths_300": ([100, 7, 193], 2048, 4096, 128, 0),
    "pages_widths_300_l2r": ([100, 7, 193], 2048, 4096, 128, B.R2L_FLAG_L2R),
}


@pytest.mark.parametrize("case", sorted(_WS_CASES))
def test_layer_output_does_not_depend_on_workspace_contents(case):
    """The workspace's contents on entry are ignored: a workspace filled with
    0xFF bytes (NaN as bf16 and as fp32) and one filled with zeros give the
    same h+ and branch, bit for bit, and every value is finite.  A read of a
    workspace byte that the same call did not write shows up here as a NaN
    or as a difference between the two runs."""
    lens, dm, di, dtr, flags = _WS_CASES[case]
    _case(f"workspace contents ignored: {case} lens={lens}")
    wl = synth.custom(lens, seed=37, h_kind="rms", d_model=dm, d_inner=di, dt_rank=dtr)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    w = B.to_device_weights(W, torch.bfloat16, DEV)
    hd = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(torch.bfloat16).to(DEV)
    need = B.r2l_layer_workspace_bytes(B.dims_of(w), B.R2L_BF16, wl.n_tokens, len(lens), max(lens))
    outs = []
    for fill in (0xFF, 0x00):
        ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
        br = torch.empty(hd.shape, dtype=torch.float32, device=DEV)
        o = B.r2l_layer_fwd(hd, w, cu, flags=flags, branch_out=br, workspace=ws)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).cpu().numpy(), br.cpu().numpy()))
        del ws
    (oa, ba), (ob, bb) = outs
    oa_f = torch.from_numpy(oa).view(torch.bfloat16).float().numpy()
    assert np.isfinite(oa_f).all(), "non-finite h+ with a NaN-filled workspace"
    assert np.isfinite(ba).all(), "non-finite branch with a NaN-filled workspace"
    assert np.array_equal(oa, ob), "h+ depends on the workspace's contents"
    assert np.array_equal(ba.view(np.uint32), bb.view(np.uint32)), "branch depends on the workspace's contents"


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
    fo, _ = bf16_floor.layer_rounded(h, cu, W, float(W["s"]))
    w = B.to_device_weights(W, torch.bfloat16, DEV)
    hd = torch.from_numpy(h).to(torch.bfloat16).to(DEV)
    cu_d = torch.from_numpy(np.asarray(cu, np.int32)).to(DEV)
    ms = 2 if hint == "too_small" else 100000
    g = to_np(B.r2l_layer_fwd(hd, w, cu_d, nseq=len(lens), max_seqlen=ms))
    check_bf16(f"out (max_seqlen {ms})", g, ref, fo, TOL_BF16)


def test_small_bf16_no_ln_and_in_place():
    _case("small bf16 NO_LN in place")
    wl = synth.custom([200, 57], seed=8, h_kind="rms", **SMALL)
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    ref = O.reverse_mamba_layer(h, cu, W, float(W["s"]), use_ln=False)
    fo, _ = bf16_floor.layer_rounded(h, cu, W, float(W["s"]), use_ln=False)
    g, _ = _gpu_layer(wl, W, h, cu, flags=B.R2L_FLAG_NO_LN, inplace=True)
    check_bf16("out no-ln", g, ref, fo, TOL_BF16)


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
    """Exact oracle outputs (h+, branch r) for positions [start, t1) of
    sequence [t0, t1), and the same outputs of the bf16 storage floor."""
    ref = O.reverse_mamba_layer(h[start:t1], [0, t1 - start], W, s, return_branch=True)
    return ref + bf16_floor.layer_rounded(h[start:t1], [0, t1 - start], W, s)


def _check_rows(tag, g, gr, ref, rref, fo=None, fr=None):
    """h+ (the graded output) and the LayerNorm branch r, each against the
    oracle in the bf16 metric and against the storage floor's bound: h+ ~ h
    hides branch errors when tanh(s) is small, so r is held on its own."""
    check_bf16(f"{tag} out", g, ref, fo, TOL_BF16)
    check_bf16(f"{tag} branch", gr, rref, fr, TOL_BF16_BRANCH)


def test_single_2k_matches_oracle_and_zero_gate():
    wl = synth.workloads()["single_2k"]
    _case("single_2k (B=1 L=2048 D=2048)")
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    t = time.time()
    ref, rref, fo, fr = _suffix_ref(h, W, float(W["s"]), 0, 2048, 0)
    print(f"oracle {time.time() - t:.1f}s", flush=True)
    g, gr = _gpu_layer(wl, W, h, cu, branch=True)
    _check_rows("single_2k", g, gr, ref, rref, fo, fr)
    g0, _ = _gpu_layer(wl, W, h, cu, s=0.0)
    assert np.array_equal(g0.astype(np.float32).view(np.uint32), h.view(np.uint32))


def test_serve_b8_matches_oracle():
    """The serving shape in the launch configuration the benchmark times:
    sequence 0 in full, the last 384 tokens of the other seven."""
    wl = synth.workloads()["serve_b8"]
    _case("serve_b8 (B=8 L=4128 D=2048)")
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    s = float(W["s"])
    g, gr = _gpu_layer(wl, W, h, cu, branch=True)
    t = time.time()
    for q in range(wl.nseq):
        t0, t1 = int(cu[q]), int(cu[q + 1])
        a = t0 if q == 0 else t1 - 384
        ref, rref, fo, fr = _suffix_ref(h, W, s, t0, t1, a)
        _check_rows(f"serve_b8 seq{q} rows {a - t0}..", g[a:t1], gr[a:t1], ref, rref, fo, fr)
    print(f"oracle {time.time() - t:.1f}s", flush=True)


def _chain_metrics(tag, g_chain, ref, n_hooks):
    """End-to-end error of a chain of hooks whose hidden stream is bf16 on
    both sides (the reference chain rounds each hook's output to bf16 before
    the next hook, as the GPU chain does).  Two measures:
      * RMS-normalised, ||g - o||_2 / ||o||_2.  The two chains round the
        stream at slightly different values after every hook, so they drift
        apart like a random walk over n_hooks + 1 roundings.  One rounding's
        RMS is measured on the reference itself (||bf16(o) - o|| / ||o||),
        and the chain is held to 2 sqrt(n_hooks + 1) times that (measured:
        about 0.5 to 0.75 of the bound).
      * max-norm (the per-hook metric).  One rounding flip of an element in
        [4, 8) moves it by 2^-5, about 3e-2 of the stream's RMS, and along
        the chain such flips compound (measured 4e-2 .. 6.6e-2); held to
        0.1, about three flips."""
    one = float(np.linalg.norm(synth.bf16_round(ref.astype(np.float32)) - ref) / np.linalg.norm(ref))
    rel = float(np.linalg.norm(g_chain - ref) / np.linalg.norm(ref))
    bound = 2.0 * np.sqrt(n_hooks + 1) * one
    print(f"[parity] {tag} one bf16 rounding (RMS-normalised): {one:.3e}", flush=True)
    assert report(f"{tag} end-to-end RMS-normalised", rel, bound) <= bound
    assert report(f"{tag} end-to-end max-norm", err_rms(g_chain, ref), 0.1) <= 0.1


def test_stack7_matches_oracle():
    """Seven hooks applied in sequence (identity between hooks).  The hidden
    stream between hooks is a bf16 tensor on both sides: the oracle rounds
    each hook's output to bf16 before feeding the next hook, as the stack's
    input itself is bf16.

    Per hook (strict, 2e-2, and the branch r): GPU hook k run on the
    oracle's bf16 stream at position k against the oracle's fp64 output of
    hook k.  End to end (GPU output feeding the next GPU hook): the two
    measures of _chain_metrics."""
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
            ref, rref, fo, fr = _suffix_ref(cur, W, float(W["s"]), 0, t1 - a, 0)
            hin = torch.from_numpy(cur.astype(np.float32)).to(torch.bfloat16).to(DEV)
            br = torch.empty(hin.shape, dtype=torch.float32, device=DEV)
            g = to_np(B.r2l_layer_fwd(hin, wd[k], [0, t1 - a], branch_out=br))
            _check_rows(f"stack7 seq{q} rows {a - t0}.. hook {k}", g, to_np(br), ref, rref, fo, fr)
            cur = synth.bf16_round(ref.astype(np.float32)).astype(np.float64)
        _chain_metrics(f"stack7 seq{q}", g_chain[a:t1], ref, wl.n_hooks)
    print(f"oracle {time.time() - t:.1f}s", flush=True)


def test_varlen16_matches_oracle():
    """16 packed sequences of 512..16384 tokens: the shortest and the median
    one in full, the last 300 tokens of every sequence."""
    wl = synth.workloads()["varlen16"]
    _case(f"varlen16 (T={wl.n_tokens}, lengths {min(wl.lengths)}..{max(wl.lengths)})")
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    s = float(W["s"])
    g, gr = _gpu_layer(wl, W, h, cu, branch=True)
    t = time.time()
    order = np.argsort(wl.lengths)
    full = (int(order[0]), int(order[len(order) // 2]))
    for q in full:
        t0, t1 = int(cu[q]), int(cu[q + 1])
        ref, rref, fo, fr = _suffix_ref(h, W, s, t0, t1, t0)
        _check_rows(f"varlen16 seq{q} (L={t1 - t0}) full", g[t0:t1], gr[t0:t1], ref, rref, fo, fr)
    for q in range(wl.nseq):
        if q in full:
            continue
        t0, t1 = int(cu[q]), int(cu[q + 1])
        ref, rref, fo, fr = _suffix_ref(h, W, s, t0, t1, t1 - 300)
        _check_rows(f"varlen16 seq{q} suffix", g[t1 - 300:t1], gr[t1 - 300:t1], ref, rref, fo, fr)
    print(f"oracle {time.time() - t:.1f}s", flush=True)


def test_long32k_matches_oracle():
    """One 32,768-token sequence, compared in full: the scan cuts it into
    eight time chunks of 4,096 tokens, so every carry (folding up to seven
    chunk summaries) is compared with the oracle."""
    wl = synth.workloads()["long32k"]
    _case("long32k (B=1 L=32768)")
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    g, gr = _gpu_layer(wl, W, h, cu, branch=True)
    t = time.time()
    L = wl.lengths[0]
    ref, rref, fo, fr = _suffix_ref(h, W, float(W["s"]), 0, L, 0)
    _check_rows("long32k full", g, gr, ref, rref, fo, fr)
    for c in range(8):   # per time chunk, rightmost first
        lo, hi = L - 4096 * (c + 1), L - 4096 * c
        print(f"[parity] long32k chunk {c} branch: {err_rms(gr[lo:hi], rref[lo:hi]):.3e}", flush=True)
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
    """Every hook of one denoise step on the oracle's bf16 stream (strict,
    h+ and the branch r), and the GPU chain end to end (the two measures of
    _chain_metrics), over all eight blocks."""
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
        ref, rref = O.reverse_mamba_layer(cur, cu, W, float(W["s"]), return_branch=True)
        fo, fr = bf16_floor.layer_rounded(cur, cu, W, float(W["s"]))
        hin = torch.from_numpy(cur.astype(np.float32)).to(torch.bfloat16).to(DEV)
        br = torch.empty(hin.shape, dtype=torch.float32, device=DEV)
        g = to_np(B.r2l_layer_fwd(hin, wd[k], cu, branch_out=br))
        _check_rows(f"{name} hook {k}", g, to_np(br), ref, rref, fo, fr)
        cur = synth.bf16_round(ref.astype(np.float32)).astype(np.float64)
    _chain_metrics(name, g_chain, ref, wl.n_hooks)


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
