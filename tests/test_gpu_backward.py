"""GPU parity of the backward pass against the gradient oracle (torch CPU
float64 autograd of the layer's and the scan's definitions, pinned by finite
differences in test_oracle_grad.py), on the same exactly representable
inputs.  The standalone scan's gradients come out in fp32 from fp32
arithmetic for both activation types and are held to the fp32 bound; the
layer's bf16 path rounds its GEMM operands to bf16 and has its own bound
(TOL_GRAD_BF16 below)."""
import time

import numpy as np
import pytest
import torch

from oracle import r2l_oracle as O
from oracle import r2l_oracle_grad as G
from parity import err_f32, err_rms, report, to_np
from reverse_selective_scan_amd import binding as B
from reverse_selective_scan_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_GRAD = 2e-4


def _err(g, ref):
    """err_f32, or the largest |g| where the reference is identically zero
    (e.g. dA_log of one-token sequences: no state reaches a later token)."""
    if not np.any(ref):
        return float(np.max(np.abs(g))) if g.size else 0.0
    return err_f32(g, ref)


def _case(name):
    print(f"\n[case] {name}", flush=True)


def _dev(a, act):
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return (t.to(torch.bfloat16) if act == "bf16" else t).to(DEV)


def _q(a, act):
    return synth.bf16_round(a) if act == "bf16" else np.asarray(a, np.float32)


def _scan_case(T, E, act, seed):
    N = 16
    u = _q(synth.make_aux(seed, (T, E)), act)
    dt = synth.make_aux(seed + 1, (T, E), kind="uniform", lo=1e-3, hi=0.2)
    A_log = synth.make_aux(seed + 2, (E, N), kind="uniform", lo=-1.0, hi=2.5)
    bcx = synth.make_aux(seed + 3, (T, 40))          # B at columns 8..23, C at 24..39
    Dskip = synth.make_aux(seed + 4, (E,), kind="uniform", lo=0.5, hi=1.5)
    z = _q(synth.make_aux(seed + 5, (T, E)), act)
    dy = _q(synth.make_aux(seed + 6, (T, E)), act)
    return u, dt, A_log, bcx, Dskip, z, dy


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("lens,E", [([1], 64), ([17], 64), ([5, 0, 130, 1, 300], 128), ([700, 2, 129], 192),
                                    ([2048], 64), ([8192, 3], 64)])
@pytest.mark.parametrize("gated", [True, False])
def test_scan_bwd_matches_oracle(act, lens, E, gated):
    _case(f"scan bwd {act} lens={lens} E={E} gated={gated}")
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    u, dt, A_log, bcx, Dskip, z, dy = _scan_case(T, E, act, 80 + len(lens) + E)
    Dk, zz = (Dskip, z) if gated else (None, None)
    ref = G.scan_grads(u, dt, A_log, bcx[:, 8:24], bcx[:, 24:40], cu, dy, Dskip=Dk, z=zz)
    bc_d = _dev(bcx, "f32")
    got = B.r2l_scan_bwd(_dev(u, act), _dev(dt, "f32"), _dev(A_log, "f32"), bc_d[:, 8:24], bc_d[:, 24:40], cu,
                         _dev(dy, act), Dskip=_dev(Dk, "f32") if gated else None,
                         z=_dev(zz, act) if gated else None)
    pairs = [("du", "u"), ("ddt", "dt"), ("dA_log", "A_log"), ("dB", "B"), ("dC", "C")]
    if gated:
        pairs += [("dDskip", "Dskip"), ("dz", "z")]
    for gk, rk in pairs:
        assert report(f"scan bwd {gk}", _err(to_np(got[gk]), ref[rk]), TOL_GRAD) <= TOL_GRAD


def test_scan_bwd_is_deterministic():
    _case("scan bwd determinism")
    lens, E = [300, 41, 5], 256
    T = sum(lens)
    u, dt, A_log, bcx, Dskip, z, dy = _scan_case(T, E, "bf16", 90)
    bc_d = _dev(bcx, "f32")
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    args = (_dev(u, "bf16"), _dev(dt, "f32"), _dev(A_log, "f32"), bc_d[:, 8:24], bc_d[:, 24:40], cu, _dev(dy, "bf16"))
    g1 = B.r2l_scan_bwd(*args, Dskip=_dev(Dskip, "f32"), z=_dev(z, "bf16"))
    g2 = B.r2l_scan_bwd(*args, Dskip=_dev(Dskip, "f32"), z=_dev(z, "bf16"))
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


# ---------------------------------------------------------------------------
# the layer
# ---------------------------------------------------------------------------
GRAD_NAMES = ("in_proj_w", "conv_w", "conv_b", "x_proj_w", "dt_proj_w", "dt_proj_b", "A_log", "Dskip",
              "out_proj_w", "ln_w", "ln_b")


def _layer_bwd_case(wl, W, h, cu, g, dtype, flags, saved=False):
    """The backward on the GPU; saved: run the forward with R2L_FLAG_TRAIN
    first and hand its workspace to the backward (no recompute), checking
    on the way that the training forward's output equals the plain one."""
    w = B.to_device_weights(W, dtype, DEV)
    hd = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(dtype).to(DEV)
    gd = torch.from_numpy(np.ascontiguousarray(g, np.float32)).to(dtype).to(DEV)
    sv = None
    if saved:
        T = hd.shape[0]
        cu_np = np.asarray(cu)
        need = B.r2l_layer_train_workspace_bytes(B.dims_of(w), B._act(hd), T, len(cu_np) - 1,
                                                 int(np.diff(cu_np).max()))
        sv = torch.empty(need, dtype=torch.uint8, device=DEV)
        out_t = B.r2l_layer_fwd(hd, w, cu, flags=flags | B.R2L_FLAG_TRAIN, workspace=sv)
        out_p = B.r2l_layer_fwd(hd, w, cu, flags=flags)
        assert torch.equal(out_t, out_p), "the training forward changed the output"
    dh, grads = B.r2l_layer_bwd(hd, w, cu, gd, flags=flags, saved=sv)
    torch.cuda.synchronize()
    return to_np(dh), {k: to_np(v) for k, v in grads.items()}


@pytest.mark.parametrize("dt_rank", [16, 192])
@pytest.mark.parametrize("saved", [False, True])
def test_layer_bwd_does_not_depend_on_buffer_contents(dt_rank, saved):
    """The backward's workspace, the training forward's saved workspace before
    that forward writes it, and the gradient and dh buffers handed in: filled
    with 0xFF bytes (NaN as bf16 and as fp32) or with zeros, the gradients are
    the same bit for bit and finite.  (dt_rank 192: the delta split is wider
    than the x_proj output.)"""
    lens = [300, 7, 129, 1, 64]
    _case(f"backward buffer contents ignored: dt_rank={dt_rank} saved={saved}")
    wl = synth.custom(lens, seed=39, h_kind="rms", d_model=256, d_inner=512, dt_rank=dt_rank)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    g = synth.make_hidden(wl, hook=5)
    w = B.to_device_weights(W, torch.bfloat16, DEV)
    hd = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(torch.bfloat16).to(DEV)
    gd = torch.from_numpy(np.ascontiguousarray(g, np.float32)).to(torch.bfloat16).to(DEV)
    dims, T, ns, ms = B.dims_of(w), wl.n_tokens, len(lens), max(lens)
    res = []
    for fill in (0xFF, 0x00):
        sv = None
        if saved:
            need = B.r2l_layer_train_workspace_bytes(dims, B.R2L_BF16, T, ns, ms)
            sv = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
            B.r2l_layer_fwd(hd, w, cu, flags=B.R2L_FLAG_TRAIN, workspace=sv)
        ws = torch.full((B.r2l_layer_bwd_workspace_bytes(dims, B.R2L_BF16, T, ns, ms),), fill, dtype=torch.uint8,
                        device=DEV)
        grads = {k: torch.empty(w[k].shape, dtype=torch.float32, device=DEV).view(torch.uint8).fill_(fill)
                 .view(torch.float32) for k, _ in B.Grads._fields_}
        dh = torch.empty_like(hd).view(torch.uint8).fill_(fill).view(torch.bfloat16)
        dh, grads = B.r2l_layer_bwd(hd, w, cu, gd, dh=dh, workspace=ws, grads=grads, saved=sv)
        torch.cuda.synchronize()
        res.append((dh.view(torch.int16).cpu().numpy(), {k: v.cpu().numpy() for k, v in grads.items()}))
        del ws, sv
    (dha, ga), (dhb, gb) = res
    assert np.isfinite(torch.from_numpy(dha).view(torch.bfloat16).float().numpy()).all(), "non-finite dh"
    assert np.array_equal(dha, dhb), "dh depends on the buffers' contents"
    for k in ga:
        assert np.isfinite(ga[k]).all(), f"non-finite d{k}"
        assert np.array_equal(ga[k].view(np.uint32), gb[k].view(np.uint32)), f"d{k} depends on the buffers' contents"


def _layer_err(f, got, ref, names, tol, tag):
    worst = 0.0
    for k in names:
        e = f(got[k], ref[k]) if np.any(ref[k]) else float(np.max(np.abs(got[k])))
        report(f"{tag} d{k}", e, tol)
        worst = max(worst, e)
    return worst


@pytest.mark.parametrize("saved", [False, True])
@pytest.mark.parametrize("use_ln", [True, False])
def test_tiny_f32_layer_bwd_matches_oracle(use_ln, saved):
    wl = synth.workloads()["tiny_f32"]
    _case(f"tiny_f32 layer bwd ln={use_ln} saved={saved}")
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    g = synth.make_hidden(wl, hook=9)
    ref = G.layer_grads(h, cu, W, float(W["s"]), g, use_ln=use_ln)
    dh, got = _layer_bwd_case(wl, W, h, cu, g, torch.float32, 0 if use_ln else B.R2L_FLAG_NO_LN, saved=saved)
    names = [n for n in GRAD_NAMES if use_ln or n not in ("ln_w", "ln_b")]
    got["h"], got["s"] = dh, got["s"].reshape(())
    ref["s"] = np.array(ref["s"])
    worst = _layer_err(_err, got, ref, names + ["h", "s"], TOL_GRAD, "tiny")
    assert worst <= TOL_GRAD


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_narrow_model_wide_dt_rank_layer_bwd_matches_oracle(act):
    """d_model 64 with dt_rank 128: x_proj's width R + 2N = 160 exceeds
    2 d_model, so W_x^T [E, 160] is the largest of the four transposed
    weights that share one workspace region (W_out^T, W_dt^T, W_x^T,
    W_in^T); the region must be sized for it."""
    lens = [40, 7, 0, 19]
    _case(f"narrow model, wide dt_rank, {act} layer bwd lens={lens}")
    wl = synth.custom(lens, seed=31, h_kind="rms", d_model=64, d_inner=128, dt_rank=128, dtype=act)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    g = synth.make_hidden(wl, hook=9)
    dtype = torch.float32 if act == "f32" else torch.bfloat16
    dh, got = _layer_bwd_case(wl, W, h, cu, g, dtype, 0)
    got["h"] = dh
    if act == "f32":
        ref = G.layer_grads(h, cu, W, float(W["s"]), g)
        got["s"] = got["s"].reshape(())
        ref["s"] = np.array(ref["s"])
        assert _layer_err(_err, got, ref, list(GRAD_NAMES) + ["h", "s"], TOL_GRAD, "narrow f32") <= TOL_GRAD
    else:
        ref = G.layer_grads(h, cu, W, float(W["s"]), g, factors=True)
        _bf16_grad_checks("narrow bf16", got, ref)


# bf16 activations: the gradients pass through bf16 copies of do, dyg, ddt,
# the x_proj and in_proj input gradients and the transposed activations
# (one rounding each, 2^-9 relative), on top of the forward's bf16 xz, u and
# y.  Three measures, each held to 3e-2:
#  * dh, a per-token gradient, element by element (max |g - o| / RMS(o));
#  * every parameter gradient in the relative Frobenius norm (measured
#    3e-3 .. 7e-3);
#  * the token-summed parameter gradients dW[i, j] = sum_t a_t[i] b_t[j] also
#    element by element, each error divided by its Cauchy-Schwarz scale
#    ||a[:, i]|| ||b[:, j]|| (the gradient oracle's factors): relative
#    2-norm errors of the factors bound it by their sum.  (Divided by the
#    RMS of dW instead, an entry whose sum over tokens cancels would carry
#    the factors' whole rounding error against a tiny value.)
# A_log's gradient has no two-factor form and is held in the Frobenius norm.
TOL_GRAD_BF16 = 3e-2


def cs_err(g, o, scale):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    if o.size == 0:
        return 0.0
    return float(np.max(np.abs(g - o) / np.maximum(scale, 1e-300)))


def _bf16_grad_checks(tag, got, ref):
    """The three measures above; got and ref hold "h" and every name in
    GRAD_NAMES, ref also the oracle's Cauchy-Schwarz scales ("cs")."""
    assert report(f"{tag} dh (max / RMS)", err_rms(got["h"], ref["h"]), TOL_GRAD_BF16) <= TOL_GRAD_BF16
    worst = _layer_err(rel_fro, got, ref, list(GRAD_NAMES) + ["h"], TOL_GRAD_BF16, f"{tag} (Frobenius)")
    assert worst <= TOL_GRAD_BF16
    for k, sc in ref["cs"].items():
        assert report(f"{tag} d{k} (max / Cauchy-Schwarz scale)", cs_err(got[k], ref[k], sc),
                      TOL_GRAD_BF16) <= TOL_GRAD_BF16


def ds_err(got_s, ref_s, g, r, s):
    """ds = (1 - tanh(s)^2) <g, r> is one sum over T x D terms that largely
    cancel, so |ds| can be arbitrarily small.  Its error is at most
    (1 - tanh(s)^2) ||g|| ||dr|| (Cauchy-Schwarz, dr the error of the branch
    r), so it is measured against (1 - tanh(s)^2) ||g|| ||r||: the relative
    error of r in the 2-norm bounds it."""
    scale = (1.0 - np.tanh(s) ** 2) * float(np.linalg.norm(np.asarray(g, np.float64))) * \
        float(np.linalg.norm(np.asarray(r, np.float64)))
    return abs(float(got_s) - float(ref_s)) / scale


def rel_fro(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    n = float(np.linalg.norm(o))
    return float(np.linalg.norm(g - o)) / n if n else float(np.linalg.norm(g))


@pytest.mark.parametrize("saved", [False, True])
@pytest.mark.parametrize("lens", [[5, 0, 130, 1, 300], [700, 33]])
def test_small_bf16_layer_bwd_matches_oracle(lens, saved):
    _case(f"small bf16 layer bwd lens={lens} saved={saved}")
    wl = synth.custom(lens, seed=19, h_kind="rms", d_model=256, d_inner=512, dt_rank=16)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    g = synth.make_hidden(wl, hook=9)
    ref = G.layer_grads(h, cu, W, float(W["s"]), g, factors=True)
    dh, got = _layer_bwd_case(wl, W, h, cu, g, torch.bfloat16, 0, saved=saved)
    got["h"] = dh
    _bf16_grad_checks("small bf16", got, ref)
    _, r = O.reverse_mamba_layer(h, cu, W, float(W["s"]), return_branch=True)
    e = ds_err(got["s"].reshape(()), ref["s"], g, r, float(W["s"]))
    assert report("small bf16 ds (against |g| |r|)", e, TOL_GRAD_BF16) <= TOL_GRAD_BF16


@pytest.mark.parametrize("use_ln", [True, False])
@pytest.mark.parametrize("d_model", [512, 1536])
def test_bf16_layer_bwd_wide_rows_matches_oracle(d_model, use_ln):
    """d_model 512 and 1536: the LayerNorm backward's one-wave form, with one
    and three 512-column chunks per lane, with and without the LayerNorm
    (dgamma and dbeta are defined only with it)."""
    lens = [5, 0, 130, 1, 300]
    _case(f"bf16 layer bwd d_model={d_model} ln={use_ln} lens={lens}")
    wl = synth.custom(lens, seed=43, h_kind="rms", d_model=d_model, d_inner=2 * d_model, dt_rank=32)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    g = synth.make_hidden(wl, hook=9)
    ref = G.layer_grads(h, cu, W, float(W["s"]), g, factors=True, use_ln=use_ln)
    dh, got = _layer_bwd_case(wl, W, h, cu, g, torch.bfloat16, 0 if use_ln else B.R2L_FLAG_NO_LN)
    got["h"] = dh
    tag = f"d_model {d_model} ln={use_ln}"
    names = [n for n in GRAD_NAMES if use_ln or n not in ("ln_w", "ln_b")]
    assert report(f"{tag} dh (max / RMS)", err_rms(got["h"], ref["h"]), TOL_GRAD_BF16) <= TOL_GRAD_BF16
    assert _layer_err(rel_fro, got, ref, names + ["h"], TOL_GRAD_BF16, f"{tag} (Frobenius)") <= TOL_GRAD_BF16
    for k, sc in ref["cs"].items():
        if k in names:
            assert report(f"{tag} d{k} (max / Cauchy-Schwarz scale)", cs_err(got[k], ref[k], sc),
                          TOL_GRAD_BF16) <= TOL_GRAD_BF16
    _, r = O.reverse_mamba_layer(h, cu, W, float(W["s"]), use_ln=use_ln, return_branch=True)
    e = ds_err(got["s"].reshape(()), ref["s"], g, r, float(W["s"]))
    assert report(f"{tag} ds (against |g| |r|)", e, TOL_GRAD_BF16) <= TOL_GRAD_BF16


@pytest.mark.parametrize("saved", [False, True])
def test_serve_b8_backward_suffix_matches_oracle(saved):
    """The serving shape (B=8 x 4128 tokens, D=2048, E=4096: the launch
    configuration that bench.py --backward times).  The layer sees only the
    right context, so with g = dL/dh+ zero outside the last S tokens of each
    sequence every gradient depends on those suffixes alone: dh on the suffix
    rows and every parameter gradient equal the oracle's gradients of the
    suffixes taken as sequences of their own, and dh is exactly zero on the
    other rows (no output there carries any gradient)."""
    wl = synth.workloads()["serve_b8"]
    _case(f"serve_b8 backward, g on the last 192 tokens of each sequence, saved={saved}")
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    S = 192
    mask = np.zeros(wl.n_tokens, bool)
    for q in range(wl.nseq):
        mask[int(cu[q + 1]) - S:int(cu[q + 1])] = True
    g = np.where(mask[:, None], synth.make_hidden(wl, hook=9), 0.0).astype(np.float32)
    dh, got = _layer_bwd_case(wl, W, h, cu, g, torch.bfloat16, 0, saved=saved)
    assert not np.any(dh[~mask]), "gradient outside the suffixes"
    idx = np.nonzero(mask)[0]
    t = time.time()
    ref = G.layer_grads(h[idx], np.arange(0, wl.nseq * S + 1, S), W, float(W["s"]), g[idx], factors=True)
    print(f"oracle {time.time() - t:.1f}s", flush=True)
    got["h"] = dh[idx]
    _bf16_grad_checks("serve_b8 suffix", got, ref)
    cu_s = np.arange(0, wl.nseq * S + 1, S)
    _, r = O.reverse_mamba_layer(h[idx], cu_s, W, float(W["s"]), return_branch=True)
    e = ds_err(got["s"].reshape(()), ref["s"], g[idx], r, float(W["s"]))
    assert report("serve_b8 suffix ds (against |g| |r|)", e, TOL_GRAD_BF16) <= TOL_GRAD_BF16


def test_long_sequence_bf16_layer_bwd_matches_oracle():
    """One 4096-token sequence and a short one: the adjoint carried left to
    right across 256 sub-blocks of the first, and reset at the boundary."""
    lens = [4096, 37]
    _case(f"long bf16 layer bwd lens={lens}")
    wl = synth.custom(lens, seed=23, h_kind="rms", d_model=256, d_inner=512, dt_rank=16)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    g = synth.make_hidden(wl, hook=9)
    t = time.time()
    ref = G.layer_grads(h, cu, W, float(W["s"]), g, factors=True)
    print(f"oracle {time.time() - t:.1f}s", flush=True)
    dh, got = _layer_bwd_case(wl, W, h, cu, g, torch.bfloat16, 0)
    got["h"] = dh
    _bf16_grad_checks("long bf16", got, ref)
    _, r = O.reverse_mamba_layer(h, cu, W, float(W["s"]), return_branch=True)
    e = ds_err(got["s"].reshape(()), ref["s"], g, r, float(W["s"]))
    assert report("long bf16 ds (against |g| |r|)", e, TOL_GRAD_BF16) <= TOL_GRAD_BF16


# ---------------------------------------------------------------------------
# the left-to-right direction (the ablation control)
# ---------------------------------------------------------------------------
def _flip_seqs(a, cu):
    out = np.array(a, copy=True)
    for q in range(len(cu) - 1):
        t0, t1 = int(cu[q]), int(cu[q + 1])
        out[t0:t1] = a[t0:t1][::-1]
    return out


@pytest.mark.parametrize("use_ln", [True, False])
def test_tiny_f32_l2r_layer_bwd_matches_oracle(use_ln):
    wl = synth.workloads()["tiny_f32"]
    _case(f"tiny_f32 l2r layer bwd ln={use_ln}")
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    g = synth.make_hidden(wl, hook=9)
    ref = G.layer_grads(h, cu, W, float(W["s"]), g, use_ln=use_ln, direction="l2r")
    flags = B.R2L_FLAG_L2R | (0 if use_ln else B.R2L_FLAG_NO_LN)
    dh, got = _layer_bwd_case(wl, W, h, cu, g, torch.float32, flags)
    names = [n for n in GRAD_NAMES if use_ln or n not in ("ln_w", "ln_b")]
    got["h"], got["s"] = dh, got["s"].reshape(())
    ref["s"] = np.array(ref["s"])
    assert _layer_err(_err, got, ref, names + ["h", "s"], TOL_GRAD, "tiny l2r") <= TOL_GRAD


def test_small_bf16_l2r_layer_bwd_matches_oracle_and_mirror():
    """Against the oracle's l2r gradients, and bit for bit against the
    default direction's gradients of the reversed sequences (dh reversed)."""
    lens = [5, 0, 130, 1, 300]
    _case(f"small bf16 l2r layer bwd lens={lens}")
    wl = synth.custom(lens, seed=29, h_kind="rms", d_model=256, d_inner=512, dt_rank=16)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    g = synth.make_hidden(wl, hook=9)
    ref = G.layer_grads(h, cu, W, float(W["s"]), g, direction="l2r", factors=True)
    dh, got = _layer_bwd_case(wl, W, h, cu, g, torch.bfloat16, B.R2L_FLAG_L2R)
    got["h"] = dh
    _bf16_grad_checks("small bf16 l2r", got, ref)
    dh_m, got_m = _layer_bwd_case(wl, W, _flip_seqs(h, cu), cu, _flip_seqs(g, cu), torch.bfloat16, 0)
    assert np.array_equal(dh, _flip_seqs(dh_m, cu))
    for k in list(GRAD_NAMES) + ["s"]:
        assert np.array_equal(got[k], got_m[k]), k
