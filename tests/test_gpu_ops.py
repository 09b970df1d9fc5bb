"""GPU parity of the library's operators against the fp64 oracle / numpy
fp64 products on the same (exactly representable) inputs."""
import numpy as np
import pytest
import torch

from oracle import r2l_oracle as O
from parity import TOL_BF16, err_f32, err_rms, report, to_np
from reverse_selective_scan_amd import binding as B
from reverse_selective_scan_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dev(a, act):
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return (t.to(torch.bfloat16) if act == "bf16" else t).to(DEV)


def _q(a, act):
    return synth.bf16_round(a) if act == "bf16" else np.asarray(a, np.float32)


def _case(name):
    print(f"\n[case] {name}", flush=True)


# ---------------------------------------------------------------------------
# dense projection (P14: numpy fp64 product of the same operands)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K", [(1, 1, 8), (33, 17, 64), (128, 128, 64), (300, 520, 136),
                                   (1031, 257, 2048), (640, 8192, 2048),
                                   # large-tile kernel: ragged M and N, and an N%4 != 0 fallback
                                   (8200, 2052, 512), (4099, 4096, 256), (8200, 2050, 512),
                                   # 264 tiles of 256 x 256: a round of 256, then the last tile row (8 tiles) on
                                   # the 128 x 128 kernel
                                   (8448, 2048, 1024),
                                   # 272 tiles: 16 past a round, not a whole tile row: split along K
                                   (8704, 2048, 1024),
                                   # few-row kernel (256-row tiles): the denoise-step projections, ragged M
                                   (256, 8192, 2048), (256, 2048, 4096), (100, 1024, 512), (1024, 2048, 4096),
                                   # 9 x 32 tiles of 256 x 256: a whole round, then the last (ragged) tile row
                                   # on the 128 x 128 kernel
                                   (2200, 8192, 512),
                                   # persistent bf16-output kernel: 576 tiles (2 or 3 per block, ragged last
                                   # tile row); 544 tiles (2 or 3 per block; with a workspace 512 tiles plus
                                   # the last tile row on the 128 x 128 kernel)
                                   (9000, 4096, 768), (4352, 8192, 2048),
                                   # few rows (the 128 x 128 kernel split along K): 7 rows; 256 rows with
                                   # K = 768
                                   (7, 2048, 2048), (256, 4096, 768),
                                   # 128 and 192 tiles of 256 x 256 with a short K: the 128 x 128 kernel
                                   # (512 and 768 tiles, ragged rows in the second)
                                   (1024, 8192, 2048), (1500, 8192, 2048)])
def test_gemm_bf16_matches_fp64_product(M, N, K):
    _case(f"gemm bf16 {M}x{N}x{K}")
    A = synth.make_aux(M * 7 + 1, (M, K))
    Bm = synth.make_aux(N * 7 + 2, (N, K))
    A, Bm = synth.bf16_round(A), synth.bf16_round(Bm)
    ref = A.astype(np.float64) @ Bm.astype(np.float64).T
    g32 = to_np(B.r2l_gemm_nt(_dev(A, "bf16"), _dev(Bm, "bf16"), out_f32=True))
    g16 = to_np(B.r2l_gemm_nt(_dev(A, "bf16"), _dev(Bm, "bf16"), out_f32=False))
    torch.cuda.synchronize()
    assert report("gemm f32-out", err_f32(g32, ref), 1e-4) <= 1e-4
    assert report("gemm bf16-out", err_f32(g16, ref), 5e-3) <= 5e-3   # one bf16 rounding (2^-8)
    # with a workspace the tiles past the last whole round are split along K
    ws = torch.empty(256 * 256 * 1024, dtype=torch.uint8, device=DEV)
    w32 = to_np(B.r2l_gemm_nt(_dev(A, "bf16"), _dev(Bm, "bf16"), out_f32=True, workspace=ws))
    w16 = to_np(B.r2l_gemm_nt(_dev(A, "bf16"), _dev(Bm, "bf16"), out_f32=False, workspace=ws))
    torch.cuda.synchronize()
    assert report("gemm f32-out (ws)", err_f32(w32, ref), 1e-4) <= 1e-4
    assert report("gemm bf16-out (ws)", err_f32(w16, ref), 5e-3) <= 5e-3


@pytest.mark.parametrize("M,N,K,pad", [(9000, 4096, 768, 64), (4352, 8192, 2048, 256)])
def test_gemm_bf16_strided_operands_and_output(M, N, K, pad):
    """Row strides past the logical widths (lda = K + pad, ldb = K + pad,
    ldc = N + pad) through the C ABI: the product matches the fp64 one and the
    padding columns of C are left untouched (persistent kernel's row range
    and whole-row stores; one-tile-per-block kernel for the fp32 output)."""
    _case(f"gemm bf16 strided {M}x{N}x{K} pad {pad}")
    A = synth.bf16_round(synth.make_aux(M * 5 + 3, (M, K)))
    Bm = synth.bf16_round(synth.make_aux(N * 5 + 4, (N, K)))
    ref = A.astype(np.float64) @ Bm.astype(np.float64).T
    Ap = torch.zeros(M, K + pad, dtype=torch.bfloat16, device=DEV)
    Bp = torch.zeros(N, K + pad, dtype=torch.bfloat16, device=DEV)
    Ap[:, :K] = _dev(A, "bf16")
    Bp[:, :K] = _dev(Bm, "bf16")
    ws = torch.empty(256 * 256 * 1024, dtype=torch.uint8, device=DEV)
    for out_f32, tol in ((False, 5e-3), (True, 1e-4)):
        C = torch.full((M, N + pad), 7.0, dtype=torch.float32 if out_f32 else torch.bfloat16, device=DEV)
        rc = B.lib().r2l_gemm_nt(B.R2L_BF16, M, N, K, Ap.data_ptr(), K + pad, Bp.data_ptr(), K + pad,
                                 C.data_ptr(), N + pad, 1 if out_f32 else 0, ws.data_ptr(), ws.numel(),
                                 torch.cuda.current_stream().cuda_stream)
        assert rc == 0, B.lib().r2l_status_string(rc)
        torch.cuda.synchronize()
        got = to_np(C)
        assert report(f"gemm strided out_f32={out_f32}", err_f32(got[:, :N], ref), tol) <= tol
        assert np.all(got[:, N:] == 7.0), "padding columns of C were written"


def test_gemm_bf16_repeats_bit_for_bit():
    """Twenty launches of the persistent kernel (its write-out staged through
    LDS while the next tile's loads and MFMAs run) and of the
    one-tile-per-block kernel give bit-identical outputs: no launch-to-launch
    race in either pipeline."""
    _case("gemm bf16 repeat 4352x8192x2048")
    M, N, K = 4352, 8192, 2048
    A = _dev(synth.bf16_round(synth.make_aux(11, (M, K))), "bf16")
    Bm = _dev(synth.bf16_round(synth.make_aux(12, (N, K))), "bf16")
    ws = torch.empty(256 * 256 * 1024, dtype=torch.uint8, device=DEV)
    for out_f32 in (False, True):
        first = B.r2l_gemm_nt(A, Bm, out_f32=out_f32, workspace=ws)
        for _ in range(20):
            again = B.r2l_gemm_nt(A, Bm, out_f32=out_f32, workspace=ws)
            assert torch.equal(again.view(torch.int16 if not out_f32 else torch.int32),
                               first.view(torch.int16 if not out_f32 else torch.int32))
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (65, 130, 33), (256, 96, 128)])
def test_gemm_f32_matches_fp64_product(M, N, K):
    _case(f"gemm f32 {M}x{N}x{K}")
    A = synth.make_aux(M + 11, (M, K))
    Bm = synth.make_aux(N + 13, (N, K))
    ref = A.astype(np.float64) @ Bm.astype(np.float64).T
    g = to_np(B.r2l_gemm_nt(_dev(A, "f32"), _dev(Bm, "f32")))
    assert report("gemm f32", err_f32(g, ref), 1e-5) <= 1e-5


# ---------------------------------------------------------------------------
# conv + SiLU (+ x_proj)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("lens,E,R", [([1], 64, 8), ([2, 3, 1, 0, 40], 128, 16), ([257, 64, 3], 256, 16),
                                      ([300, 41], 4096, 128)])
def test_conv_fwd_matches_oracle(act, lens, E, R):
    _case(f"conv {act} lens={lens} E={E} R={R}")
    N = 16
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    xz = _q(synth.make_aux(1, (T, 2 * E)), act)
    cw = _q(synth.make_aux(2, (E, 4), scale=0.5), act)
    cb = _q(synth.make_aux(3, (E,), scale=0.5), act)
    xw = _q(synth.make_aux(4, (R + 2 * N, E), scale=E ** -0.5), act)
    ref_u, ref_x = O.reverse_conv_silu(xz[:, :E], cu, cw, cb, xw)
    xz_d = _dev(xz, act)
    u, xd = B.r2l_conv_fwd(xz_d[:, :E], _dev(cw, act), _dev(cb, act), cu, x_proj_w=_dev(xw, act), dt_rank=R)
    u, xd = to_np(u), to_np(xd)
    if act == "f32":
        assert report("conv u", err_f32(u, ref_u), 1e-5) <= 1e-5
        assert report("conv xdbl", err_f32(xd, ref_x), 1e-4) <= 1e-4
    else:
        assert report("conv u", err_f32(u, ref_u), 5e-3) <= 5e-3
        assert report("conv xdbl", err_rms(xd, ref_x), 1e-2) <= 1e-2
        # xdbl does not depend on whether u is also written
        _, xd2 = B.r2l_conv_fwd(xz_d[:, :E], _dev(cw, act), _dev(cb, act), cu, x_proj_w=_dev(xw, act),
                                dt_rank=R, want_u=False)
        assert np.array_equal(to_np(xd2), xd)


def test_conv_fwd_bf16_wide_xproj_uses_staged_u():
    _case("conv bf16 wide x_proj (R+2N > 256)")
    E, R, N, T = 128, 240, 16, 70
    cu = np.array([0, 30, 70], np.int32)
    xz = _q(synth.make_aux(5, (T, E)), "bf16")
    cw = _q(synth.make_aux(6, (E, 4), scale=0.5), "bf16")
    cb = _q(synth.make_aux(7, (E,), scale=0.5), "bf16")
    xw = _q(synth.make_aux(8, (R + 2 * N, E), scale=E ** -0.5), "bf16")
    ref_u, ref_x = O.reverse_conv_silu(xz, cu, cw, cb, xw)
    u, xd = B.r2l_conv_fwd(_dev(xz, "bf16"), _dev(cw, "bf16"), _dev(cb, "bf16"), cu, x_proj_w=_dev(xw, "bf16"),
                           dt_rank=R)
    assert report("conv u", err_f32(to_np(u), ref_u), 5e-3) <= 5e-3
    assert report("conv xdbl", err_rms(to_np(xd), ref_x), 1e-2) <= 1e-2


# ---------------------------------------------------------------------------
# reverse selective scan (standalone: dt given)
# ---------------------------------------------------------------------------
def _scan_inputs(T, E, act, seed):
    N = 16
    u = _q(synth.make_aux(seed, (T, E)), act)
    dt = synth.make_aux(seed + 1, (T, E), kind="uniform", lo=1e-3, hi=0.2)
    A_log = synth.make_aux(seed + 2, (E, N), kind="uniform", lo=-1.0, hi=2.5)
    bcx = synth.make_aux(seed + 3, (T, 40))          # B at columns 8..23, C at 24..39
    Dskip = synth.make_aux(seed + 4, (E,), kind="uniform", lo=0.5, hi=1.5)
    z = _q(synth.make_aux(seed + 5, (T, E)), act)
    return u, dt, A_log, bcx, Dskip, z


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("lens,E", [([1], 64), ([37], 128), ([5, 0, 130, 1, 300], 128), ([700, 2, 129], 192),
                                    ([2048], 1024)])
@pytest.mark.parametrize("with_z", [True, False])
def test_scan_fwd_matches_oracle(act, lens, E, with_z):
    _case(f"scan {act} lens={lens} E={E} z={with_z}")
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    u, dt, A_log, bcx, Dskip, z = _scan_inputs(T, E, act, 20 + len(lens))
    zz = z if with_z else None
    Dk = Dskip if with_z else None
    ref = O.reverse_selective_scan(u, dt, A_log, bcx[:, 8:24], bcx[:, 24:40], cu, Dskip=Dk, z=zz)
    bc_d = _dev(bcx, "f32")
    y = B.r2l_scan_fwd(_dev(u, act), _dev(dt, "f32"), _dev(A_log, "f32"), bc_d[:, 8:24], bc_d[:, 24:40], cu,
                       Dskip=_dev(Dk, "f32") if Dk is not None else None,
                       z=_dev(zz, act) if zz is not None else None)
    g = to_np(y)
    tol = 1e-4 if act == "f32" else 5e-3
    assert report("scan", err_f32(g, ref), tol) <= tol


def test_scan_strong_decay_is_pointwise_on_gpu():
    """A -> -inf: only the token's own term survives (closed form, any length)."""
    _case("scan strong decay")
    T, E = 500, 128
    cu = np.array([0, 200, 500], np.int32)
    u, dt, _, bcx, Dskip, _ = _scan_inputs(T, E, "f32", 60)
    A_log = np.full((E, 16), 80.0, np.float32)
    Bm, Cm = bcx[:, 8:24].astype(np.float64), bcx[:, 24:40].astype(np.float64)
    ref = dt * u * (Bm * Cm).sum(axis=1)[:, None] + Dskip * u
    bc_d = _dev(bcx, "f32")
    g = to_np(B.r2l_scan_fwd(_dev(u, "f32"), _dev(dt, "f32"), _dev(A_log, "f32"), bc_d[:, 8:24], bc_d[:, 24:40],
                             cu, Dskip=_dev(Dskip, "f32")))
    assert report("scan strong decay", err_f32(g, ref), 1e-5) <= 1e-5


def test_scan_fwd_many_short_sequences():
    """600 sequences of 0..40 tokens (zero-length ones included): the chunk
    planner then handles several offsets per thread in its block-wide scans.
    The output matches the oracle, and every sequence's rows equal, bit for
    bit, those of the same sequences run in batches of at most 200 (one
    offset per thread).  E = 192 gives 3 channel blocks per sequence, so
    neither run cuts sequences into time chunks."""
    lens = [int(v) for v in np.random.default_rng(np.random.SeedSequence([41, 600])).integers(0, 41, size=600)]
    lens[0], lens[17], lens[599] = 0, 0, 0
    E = 192
    _case(f"scan, 600 sequences of 0..40 tokens (T={sum(lens)}), E={E}")
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    u, dt, A_log, bcx, Dskip, z = _scan_inputs(T, E, "bf16", 70)
    ref = O.reverse_selective_scan(u, dt, A_log, bcx[:, 8:24], bcx[:, 24:40], cu, Dskip=Dskip, z=z)
    ud, dtd, Ad, bcd, Dd, zd = (_dev(u, "bf16"), _dev(dt, "f32"), _dev(A_log, "f32"), _dev(bcx, "f32"),
                                _dev(Dskip, "f32"), _dev(z, "bf16"))
    y = to_np(B.r2l_scan_fwd(ud, dtd, Ad, bcd[:, 8:24], bcd[:, 24:40], cu, Dskip=Dd, z=zd))
    assert report("scan 600 sequences", err_f32(y, ref), 5e-3) <= 5e-3
    for q0 in range(0, 600, 200):
        a, b = int(cu[q0]), int(cu[q0 + 200])
        cu_b = (cu[q0:q0 + 201] - a).astype(np.int32)
        yb = to_np(B.r2l_scan_fwd(ud[a:b], dtd[a:b], Ad, bcd[a:b, 8:24], bcd[a:b, 24:40], cu_b, Dskip=Dd,
                                  z=zd[a:b]))
        assert np.array_equal(yb, y[a:b]), q0
