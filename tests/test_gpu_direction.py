"""The left-to-right direction (R2L_FLAG_L2R: the "L2R Mamba" control of the
pages' ablation, §4.4 Table 4) on the GPU: parity of the conv, the scan and
the layer against the oracle run with direction="l2r", and the mirror
identity -- the L2R result on every sequence reversed, reversed back, is
the default (R2L) result -- checked bit for bit where both directions do
the same arithmetic in mirrored order."""
import numpy as np
import pytest
import torch

from oracle import r2l_oracle as O
import bf16_floor
from parity import TOL_BF16, TOL_BF16_BRANCH, check_bf16, err_f32, err_rms, report, to_np
from reverse_selective_scan_amd import binding as B
from reverse_selective_scan_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
L2R = B.R2L_FLAG_L2R


def _case(name):
    print(f"\n[case] {name}", flush=True)


def _dev(a, act):
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return (t.to(torch.bfloat16) if act == "bf16" else t).to(DEV)


def _q(a, act):
    return synth.bf16_round(a) if act == "bf16" else np.asarray(a, np.float32)


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _mirror(lens):
    """Row permutation that reverses every sequence (its own inverse)."""
    cu = _cu(lens)
    return np.concatenate([np.arange(a, b)[::-1] for a, b in zip(cu[:-1], cu[1:])] or [np.zeros(0, int)])


def _bits(a):
    return np.ascontiguousarray(a, np.float64).view(np.uint64)


# ---------------------------------------------------------------------------
# conv + SiLU (+ x_proj)
# ---------------------------------------------------------------------------
def _conv_case(lens, E, R, act):
    N = 16
    T = sum(lens)
    xz = _q(synth.make_aux(31, (T, 2 * E)), act)
    cw = _q(synth.make_aux(32, (E, 4), scale=0.5), act)
    cb = _q(synth.make_aux(33, (E,), scale=0.5), act)
    xw = _q(synth.make_aux(34, (R + 2 * N, E), scale=E ** -0.5), act)
    return xz, cw, cb, xw


def _gpu_conv(xz, cw, cb, xw, cu, E, R, act, flags):
    xz_d = _dev(xz, act)
    u, xd = B.r2l_conv_fwd(xz_d[:, :E], _dev(cw, act), _dev(cb, act), cu, x_proj_w=_dev(xw, act), dt_rank=R,
                           flags=flags)
    return to_np(u), to_np(xd)


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("lens,E,R", [([1], 64, 8), ([2, 3, 1, 0, 40], 128, 16), ([300, 41], 4096, 128)])
def test_conv_l2r_matches_oracle(act, lens, E, R):
    _case(f"conv l2r {act} lens={lens} E={E}")
    xz, cw, cb, xw = _conv_case(lens, E, R, act)
    cu = _cu(lens)
    ref_u, ref_x = O.reverse_conv_silu(xz[:, :E], cu, cw, cb, xw, direction="l2r")
    u, xd = _gpu_conv(xz, cw, cb, xw, cu, E, R, act, L2R)
    if act == "f32":
        assert report("conv l2r u", err_f32(u, ref_u), 1e-5) <= 1e-5
        assert report("conv l2r xdbl", err_f32(xd, ref_x), 1e-4) <= 1e-4
    else:
        assert report("conv l2r u", err_f32(u, ref_u), 5e-3) <= 5e-3
        assert report("conv l2r xdbl", err_rms(xd, ref_x), 1e-2) <= 1e-2


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_conv_l2r_is_mirrored_r2l_bitwise(act):
    lens, E, R = [7, 1, 0, 90, 33], 256, 16
    _case(f"conv mirror {act} lens={lens}")
    xz, cw, cb, xw = _conv_case(lens, E, R, act)
    cu, m = _cu(lens), _mirror(lens)
    u_r, x_r = _gpu_conv(xz, cw, cb, xw, cu, E, R, act, 0)
    u_l, x_l = _gpu_conv(xz[m], cw, cb, xw, cu, E, R, act, L2R)
    assert np.array_equal(_bits(u_l[m]), _bits(u_r))
    assert np.array_equal(_bits(x_l[m]), _bits(x_r))


# ---------------------------------------------------------------------------
# selective scan (standalone: dt given)
# ---------------------------------------------------------------------------
def _scan_case(T, E, act, seed):
    N = 16
    u = _q(synth.make_aux(seed, (T, E)), act)
    dt = synth.make_aux(seed + 1, (T, E), kind="uniform", lo=1e-3, hi=0.2)
    A_log = synth.make_aux(seed + 2, (E, N), kind="uniform", lo=-1.0, hi=2.5)
    bcx = synth.make_aux(seed + 3, (T, 40))          # B at columns 8..23, C at 24..39
    Dskip = synth.make_aux(seed + 4, (E,), kind="uniform", lo=0.5, hi=1.5)
    z = _q(synth.make_aux(seed + 5, (T, E)), act)
    return u, dt, A_log, bcx, Dskip, z


def _gpu_scan(u, dt, A_log, bcx, Dskip, z, cu, act, flags):
    bc_d = _dev(bcx, "f32")
    return to_np(B.r2l_scan_fwd(_dev(u, act), _dev(dt, "f32"), _dev(A_log, "f32"), bc_d[:, 8:24], bc_d[:, 24:40],
                                cu, Dskip=_dev(Dskip, "f32"), z=_dev(z, act), flags=flags))


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("lens,E", [([1], 64), ([5, 0, 130, 1, 300], 128), ([2048], 1024)])
def test_scan_l2r_matches_oracle(act, lens, E):
    """([2048], 1024): 16 channel blocks for one sequence, so the scan is
    cut into time chunks joined by the summary pass."""
    _case(f"scan l2r {act} lens={lens} E={E}")
    T = sum(lens)
    cu = _cu(lens)
    u, dt, A_log, bcx, Dskip, z = _scan_case(T, E, act, 40 + len(lens))
    ref = O.reverse_selective_scan(u, dt, A_log, bcx[:, 8:24], bcx[:, 24:40], cu, Dskip=Dskip, z=z,
                                   direction="l2r")
    g = _gpu_scan(u, dt, A_log, bcx, Dskip, z, cu, act, L2R)
    tol = 1e-4 if act == "f32" else 5e-3
    assert report("scan l2r", err_f32(g, ref), tol) <= tol


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("lens,E", [([5, 0, 130, 1, 300], 128), ([2048], 1024)])
def test_scan_l2r_is_mirrored_r2l_bitwise(act, lens, E):
    _case(f"scan mirror {act} lens={lens} E={E}")
    T = sum(lens)
    cu, m = _cu(lens), _mirror(lens)
    u, dt, A_log, bcx, Dskip, z = _scan_case(T, E, act, 50 + len(lens))
    y_r = _gpu_scan(u, dt, A_log, bcx, Dskip, z, cu, act, 0)
    y_l = _gpu_scan(u[m], dt[m], A_log, bcx[m], Dskip, z[m], cu, act, L2R)
    assert np.array_equal(_bits(y_l[m]), _bits(y_r))


# ---------------------------------------------------------------------------
# the layer
# ---------------------------------------------------------------------------
SMALL = dict(d_model=256, d_inner=512, dt_rank=16)


def _gpu_layer(W, h, cu, dtype, flags, branch=False):
    w = B.to_device_weights(W, dtype, DEV)
    hd = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(dtype).to(DEV)
    br = torch.empty(hd.shape, dtype=torch.float32, device=DEV) if branch else None
    out = B.r2l_layer_fwd(hd, w, cu, flags=flags, branch_out=br)
    torch.cuda.synchronize()
    return to_np(out), (to_np(br) if branch else None)


def test_tiny_f32_layer_l2r_matches_oracle():
    wl = synth.workloads()["tiny_f32"]
    _case("tiny_f32 l2r")
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    ref = O.reverse_mamba_layer(h, cu, W, float(W["s"]), direction="l2r")
    g, _ = _gpu_layer(W, h, cu, torch.float32, L2R)
    assert report("tiny l2r", err_f32(g, ref), 1e-4) <= 1e-4


@pytest.mark.parametrize("lens", [[1], [5, 0, 130, 1, 300, 2], [1000, 64, 333]])
def test_small_bf16_layer_l2r_matches_oracle(lens):
    _case(f"small bf16 l2r lens={lens}")
    wl = synth.custom(lens, seed=17, h_kind="rms", **SMALL)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    ref, rref = O.reverse_mamba_layer(h, cu, W, float(W["s"]), return_branch=True, direction="l2r")
    fo, fr = bf16_floor.layer_rounded(h, cu, W, float(W["s"]), direction="l2r")
    g, gr = _gpu_layer(W, h, cu, torch.bfloat16, L2R, branch=True)
    check_bf16("out l2r", g, ref, fo, TOL_BF16)
    check_bf16("branch l2r", gr, rref, fr, TOL_BF16_BRANCH)


def test_bf16_layer_l2r_split_k_conv_path_matches_oracle():
    """More than 256 tiles of 128 tokens (the split-K conv kernel, whose
    first tile reads the three rows before the sequence start as zeros) and
    long sequences over few channel blocks (time chunks)."""
    lens = [20000, 7, 13000, 1, 300]
    _case(f"split-K conv path l2r lens={lens}")
    wl = synth.custom(lens, seed=22, h_kind="rms", d_model=256, d_inner=512, dt_rank=5)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    ref, rref = O.reverse_mamba_layer(h, cu, W, float(W["s"]), return_branch=True, direction="l2r")
    fo, fr = bf16_floor.layer_rounded(h, cu, W, float(W["s"]), direction="l2r")
    g, gr = _gpu_layer(W, h, cu, torch.bfloat16, L2R, branch=True)
    check_bf16("out l2r", g, ref, fo, TOL_BF16)
    check_bf16("branch l2r", gr, rref, fr, TOL_BF16_BRANCH)


def test_bf16_layer_l2r_at_pages_widths_matches_oracle():
    """300 tokens at the pages' widths (D = 2048, E = 4096, dt_rank 128),
    left to right: in_proj on the mid-size GEMM whose extra block plans the
    time chunks, and out_proj split along K with the LayerNorm kernel adding
    the partial tiles.  Sequences of 100, 7 and 193 tokens cross the 128-row
    tiles and the last tile is ragged."""
    lens = [100, 7, 193]
    _case(f"pages widths l2r lens={lens}")
    wl = synth.custom(lens, seed=36, h_kind="rms", d_model=2048, d_inner=4096, dt_rank=128)
    W = synth.make_weights(wl, affine_ln=True)
    h, cu = synth.make_hidden(wl), wl.cu_seqlens()
    ref, rref = O.reverse_mamba_layer(h, cu, W, float(W["s"]), return_branch=True, direction="l2r")
    fo, fr = bf16_floor.layer_rounded(h, cu, W, float(W["s"]), direction="l2r")
    g, gr = _gpu_layer(W, h, cu, torch.bfloat16, L2R, branch=True)
    check_bf16("out l2r", g, ref, fo, TOL_BF16)
    check_bf16("branch l2r", gr, rref, fr, TOL_BF16_BRANCH)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_layer_l2r_is_mirrored_r2l_bitwise(act):
    """Below the split-K conv's size every per-token step is independent of
    the token's position and the conv and scan are mirrored exactly."""
    lens = [300, 1, 0, 77, 4]
    _case(f"layer mirror {act} lens={lens}")
    wl = synth.custom(lens, seed=18, h_kind="rms", dtype=act, **SMALL)
    W, h, cu = synth.make_weights(wl), synth.make_hidden(wl), wl.cu_seqlens()
    m = _mirror(lens)
    dtype = torch.float32 if act == "f32" else torch.bfloat16
    g_r, _ = _gpu_layer(W, h, cu, dtype, 0)
    g_l, _ = _gpu_layer(W, h[m], cu, dtype, L2R)
    assert np.array_equal(_bits(g_l[m]), _bits(g_r))
