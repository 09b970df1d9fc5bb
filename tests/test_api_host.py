"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol the header declares, and rejects bad arguments with the
documented status codes before touching a device."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from reverse_selective_scan_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "r2l.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced: every case fails validation first


def _header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(r2l_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    names = _header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(B._SIGS) == set(names)


def test_version_and_status_strings():
    lib = B.lib()
    assert lib.r2l_version() == 100
    for code in (0, -1, -2, -3, -4):
        assert lib.r2l_status_string(code)
    assert lib.r2l_status_string(-99) == b"unknown status"


def _dims(D=2048, E=4096, N=16, R=128, K=4):
    return B.Dims(d_model=D, d_inner=E, d_state=N, dt_rank=R, d_conv=K)


def test_workspace_query():
    lib = B.lib()
    d = _dims()
    T = 33024
    ws = lib.r2l_layer_workspace_bytes(C.byref(d), B.R2L_BF16, T, 8, 4128)
    # at least in_proj's output, x_proj's output and the gated scan output
    assert ws >= T * 2 * 4096 * 2 + T * 160 * 4 + T * 4096 * 2
    assert ws < T * 4096 * 2 * 4  # and nothing like a fp32 copy of everything
    assert lib.r2l_layer_workspace_bytes(C.byref(d), B.R2L_BF16, 2 * T, 16, 4128) > ws
    bad = _dims(N=8)
    assert lib.r2l_layer_workspace_bytes(C.byref(bad), B.R2L_BF16, T, 8, 4128) == 0
    assert lib.r2l_layer_workspace_bytes(None, B.R2L_BF16, T, 8, 4128) == 0
    assert lib.r2l_layer_workspace_bytes(C.byref(d), 7, T, 8, 4128) == 0
    assert lib.r2l_scan_workspace_bytes(C.byref(d), T, 8, 4128) > 0


def test_check_cu_seqlens():
    lib = B.lib()
    ok = np.array([0, 3, 3, 10], np.int32)
    assert lib.r2l_check_cu_seqlens(ok.ctypes.data, 3, 10, 7) == 0
    assert lib.r2l_check_cu_seqlens(ok.ctypes.data, 3, 10, 6) == B.R2L_ERR_INVALID_ARG  # max_seqlen too small
    assert lib.r2l_check_cu_seqlens(ok.ctypes.data, 3, 11, 7) == B.R2L_ERR_INVALID_ARG  # wrong total
    bad = np.array([0, 5, 4, 10], np.int32)
    assert lib.r2l_check_cu_seqlens(bad.ctypes.data, 3, 10, 10) == B.R2L_ERR_INVALID_ARG
    bad0 = np.array([1, 5, 10], np.int32)
    assert lib.r2l_check_cu_seqlens(bad0.ctypes.data, 2, 10, 10) == B.R2L_ERR_INVALID_ARG
    assert lib.r2l_check_cu_seqlens(None, 2, 10, 10) == B.R2L_ERR_INVALID_ARG


def _weights(**over):
    w = B.Weights(**{f[0]: FAKE for f in B.Weights._fields_})
    for k, v in over.items():
        setattr(w, k, v)
    return w


def _layer(d=None, act=B.R2L_BF16, flags=0, w=None, h_in=FAKE, h_out=FAKE, cu=FAKE, nseq=2, T=100,
           maxlen=60, ws=FAKE, wsb=0, branch=None):
    lib = B.lib()
    d = d if d is not None else _dims()
    w = w if w is not None else _weights()
    return lib.r2l_layer_fwd(C.byref(d), act, flags, C.byref(w), h_in, h_out, cu, nseq, T, maxlen, ws, wsb,
                             branch, None)


def test_layer_fwd_rejects_bad_arguments():
    lib = B.lib()
    w = _weights()
    assert lib.r2l_layer_fwd(None, B.R2L_BF16, 0, C.byref(w), FAKE, FAKE, FAKE, 1, 10, 10, FAKE, 1 << 30,
                             None, None) == B.R2L_ERR_INVALID_ARG
    assert _layer(d=_dims(N=8)) == B.R2L_ERR_UNSUPPORTED
    assert _layer(d=_dims(K=3)) == B.R2L_ERR_UNSUPPORTED
    assert _layer(d=_dims(D=100)) == B.R2L_ERR_UNSUPPORTED
    assert _layer(d=_dims(R=0)) == B.R2L_ERR_INVALID_ARG
    assert _layer(act=5) == B.R2L_ERR_UNSUPPORTED
    assert _layer(flags=0x10) == B.R2L_ERR_INVALID_ARG
    assert _layer(h_in=None) == B.R2L_ERR_INVALID_ARG
    assert _layer(h_out=None) == B.R2L_ERR_INVALID_ARG
    assert _layer(cu=None) == B.R2L_ERR_INVALID_ARG
    assert _layer(nseq=0) == B.R2L_ERR_INVALID_ARG
    assert _layer(T=-1) == B.R2L_ERR_INVALID_ARG
    assert _layer(w=_weights(A_log=None)) == B.R2L_ERR_INVALID_ARG
    assert _layer(w=_weights(ln_w=None)) == B.R2L_ERR_INVALID_ARG
    assert _layer(h_in=FAKE + 2) == B.R2L_ERR_INVALID_ARG          # bf16 operands must be 16-byte aligned
    assert _layer(ws=None, wsb=1 << 40) == B.R2L_ERR_WORKSPACE
    assert _layer(wsb=1024) == B.R2L_ERR_WORKSPACE                 # smaller than the query


def test_layer_fwd_accepts_the_direction_flag():
    assert _layer(flags=B.R2L_FLAG_L2R, wsb=16) == B.R2L_ERR_WORKSPACE
    assert _layer(flags=B.R2L_FLAG_L2R | B.R2L_FLAG_NO_LN, wsb=16) == B.R2L_ERR_WORKSPACE
    assert _layer(flags=0x8) == B.R2L_ERR_INVALID_ARG


def test_train_flag_needs_the_train_workspace():
    lib = B.lib()
    d = _dims()
    T = 33024
    ws = lib.r2l_layer_workspace_bytes(C.byref(d), B.R2L_BF16, T, 8, 4128)
    tws = lib.r2l_layer_train_workspace_bytes(C.byref(d), B.R2L_BF16, T, 8, 4128)
    # the out_proj output gets a region of its own instead of reusing the in_proj output's,
    # and the fused out_proj + LayerNorm's row statistics and counters (training keeps o) go
    fused = (T // 256) * (2048 * 8 + 4)
    assert tws >= ws + T * 2048 * 4 - fused - 4096
    assert lib.r2l_layer_train_workspace_bytes(C.byref(_dims(N=8)), B.R2L_BF16, T, 8, 4128) == 0
    assert _layer(flags=B.R2L_FLAG_TRAIN, T=T, nseq=8, maxlen=4128, wsb=ws) == B.R2L_ERR_WORKSPACE
    # with the train workspace the call passes every check (and then launches nothing: T = 0)
    assert _layer(flags=B.R2L_FLAG_TRAIN, T=0, nseq=1, maxlen=0, ws=FAKE * 256,
                  wsb=lib.r2l_layer_train_workspace_bytes(C.byref(d), B.R2L_BF16, 0, 1, 0)) == B.R2L_OK


def _layer_bwd(flags=0, saved=None, T=100, wsb=None, ws=FAKE * 256):
    lib = B.lib()
    d = _dims()
    w = _weights()
    g = B.Grads(**{f[0]: FAKE for f in B.Grads._fields_})
    if wsb is None:
        wsb = lib.r2l_layer_bwd_workspace_bytes(C.byref(d), B.R2L_BF16, T, 2, 60)
    return lib.r2l_layer_bwd(C.byref(d), B.R2L_BF16, flags, C.byref(w), FAKE, FAKE, FAKE, C.byref(g), FAKE, 2, T, 60,
                             saved, ws, wsb, None)


def test_layer_bwd_rejects_bad_arguments():
    # the left-to-right direction is supported when the forward is recomputed, not with saved activations
    assert _layer_bwd(flags=B.R2L_FLAG_L2R, saved=FAKE * 256) == B.R2L_ERR_UNSUPPORTED
    assert _layer_bwd(flags=0x8) == B.R2L_ERR_INVALID_ARG
    assert _layer_bwd(flags=B.R2L_FLAG_TRAIN) == B.R2L_ERR_INVALID_ARG    # a forward-only flag
    assert _layer_bwd(wsb=1024) == B.R2L_ERR_WORKSPACE
    assert _layer_bwd(saved=FAKE * 256 + 16) == B.R2L_ERR_INVALID_ARG     # saved must be 256-byte aligned
    assert _layer_bwd(T=0, saved=FAKE * 256) == B.R2L_OK                  # nothing to do, nothing launched


def test_layer_fwd_no_ln_needs_no_ln_weights():
    # with the flag, missing LN weights are fine: the call then only fails at the workspace check
    assert _layer(flags=B.R2L_FLAG_NO_LN, w=_weights(ln_w=None, ln_b=None), wsb=16) == B.R2L_ERR_WORKSPACE


def test_zero_tokens_is_a_no_op():
    # T = 0: validation passes and nothing is launched (safe without a GPU)
    d = _dims()
    need = B.lib().r2l_layer_workspace_bytes(C.byref(d), B.R2L_BF16, 0, 1, 0)
    assert need > 0
    assert _layer(T=0, nseq=1, maxlen=0, ws=FAKE * 256, wsb=need) == B.R2L_OK


def test_conv_scan_gemm_reject_bad_arguments():
    lib = B.lib()
    d = _dims()
    # conv: no output requested / xdbl without x_proj / ld_x < E
    assert lib.r2l_conv_fwd(C.byref(d), B.R2L_BF16, 0, FAKE, 8192, FAKE, FAKE, None, None, None, FAKE, 1, 10, 10,
                            None) == B.R2L_ERR_INVALID_ARG
    assert lib.r2l_conv_fwd(C.byref(d), B.R2L_BF16, 0, FAKE, 8192, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1, 10, 10,
                            None) == B.R2L_ERR_INVALID_ARG
    assert lib.r2l_conv_fwd(C.byref(d), B.R2L_BF16, 0, FAKE, 100, FAKE, FAKE, None, FAKE, None, FAKE, 1, 10, 10,
                            None) == B.R2L_ERR_INVALID_ARG
    assert lib.r2l_conv_fwd(C.byref(d), B.R2L_BF16, 0, FAKE, 8190, FAKE, FAKE, None, FAKE, None, FAKE, 1, 10, 10,
                            None) == B.R2L_ERR_INVALID_ARG   # bf16 rows must stay 16-byte aligned
    # scan: missing dt / small ld / missing workspace
    assert lib.r2l_scan_fwd(C.byref(d), B.R2L_F32, 0, FAKE, 4096, None, 4096, FAKE, FAKE, FAKE, 16, None, None, 0,
                            FAKE, FAKE, 1, 10, 10, FAKE, 1 << 30, None) == B.R2L_ERR_INVALID_ARG
    assert lib.r2l_scan_fwd(C.byref(d), B.R2L_F32, 0, FAKE, 4000, FAKE, 4096, FAKE, FAKE, FAKE, 16, None, None, 0,
                            FAKE, FAKE, 1, 10, 10, FAKE, 1 << 30, None) == B.R2L_ERR_INVALID_ARG
    assert lib.r2l_scan_fwd(C.byref(d), B.R2L_F32, 0, FAKE, 4096, FAKE, 4096, FAKE, FAKE, FAKE, 16, None, None, 0,
                            FAKE, FAKE, 1, 10, 10, None, 0, None) == B.R2L_ERR_WORKSPACE
    # unknown flag bits (R2L_FLAG_NO_LN means nothing to the conv or the scan)
    assert lib.r2l_conv_fwd(C.byref(d), B.R2L_BF16, B.R2L_FLAG_NO_LN, FAKE, 8192, FAKE, FAKE, None, FAKE, None,
                            FAKE, 1, 10, 10, None) == B.R2L_ERR_INVALID_ARG
    assert lib.r2l_scan_fwd(C.byref(d), B.R2L_F32, 0x8, FAKE, 4096, FAKE, 4096, FAKE, FAKE, FAKE, 16, None, None,
                            0, FAKE, FAKE, 1, 10, 10, FAKE, 1 << 30, None) == B.R2L_ERR_INVALID_ARG
    # the direction flag passes validation (then fails at the workspace check)
    assert lib.r2l_scan_fwd(C.byref(d), B.R2L_F32, B.R2L_FLAG_L2R, FAKE, 4096, FAKE, 4096, FAKE, FAKE, FAKE, 16,
                            None, None, 0, FAKE, FAKE, 1, 10, 10, None, 0, None) == B.R2L_ERR_WORKSPACE
    # gemm
    assert lib.r2l_gemm_nt(B.R2L_BF16, 10, 10, 12, FAKE, 12, FAKE, 12, FAKE, 10, 0, None, 0, None) == B.R2L_ERR_UNSUPPORTED
    assert lib.r2l_gemm_nt(B.R2L_BF16, 10, 10, 16, FAKE, 8, FAKE, 16, FAKE, 10, 0, None, 0, None) == B.R2L_ERR_INVALID_ARG
    assert lib.r2l_gemm_nt(3, 10, 10, 16, FAKE, 16, FAKE, 16, FAKE, 10, 0, None, 0, None) == B.R2L_ERR_UNSUPPORTED
    assert lib.r2l_gemm_nt(B.R2L_F32, -1, 10, 16, FAKE, 16, FAKE, 16, FAKE, 10, 0, None, 0, None) == B.R2L_ERR_INVALID_ARG
    # workspace pointer and size must agree, and the pointer be 16-byte aligned
    assert lib.r2l_gemm_nt(B.R2L_BF16, 10, 10, 16, FAKE, 16, FAKE, 16, FAKE, 10, 0, None, 64, None) == B.R2L_ERR_INVALID_ARG
    assert lib.r2l_gemm_nt(B.R2L_BF16, 10, 10, 16, FAKE, 16, FAKE, 16, FAKE, 10, 0, FAKE, 0, None) == B.R2L_ERR_INVALID_ARG
    assert lib.r2l_gemm_nt(B.R2L_BF16, 10, 10, 16, FAKE, 16, FAKE, 16, FAKE, 10, 0, FAKE + 8, 64, None) == B.R2L_ERR_INVALID_ARG


def test_timing_read_empty():
    B.timing_reset()
    assert B.timing_read() == {}


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(B, "_lib_handle", None)
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/libr2l.so")
    with pytest.raises(RuntimeError, match="not built"):
        B.lib()


def test_scan_bwd_rejects_bad_arguments():
    lib = B.lib()
    d = _dims()
    need = lib.r2l_scan_bwd_workspace_bytes(C.byref(d), 10, 1)
    assert need > 0

    def call(flags=0, dy=FAKE, dD=None, dz=None, Dskip=None, z=None, ws=FAKE * 256, wsb=need, ld_u=4096):
        return lib.r2l_scan_bwd(C.byref(d), B.R2L_F32, flags, FAKE, ld_u, FAKE, 4096, FAKE, FAKE, FAKE, 16, Dskip,
                                z, 4096, dy, 4096, FAKE, FAKE, FAKE, FAKE, FAKE, dD, dz, FAKE, 1, 10, ws, wsb,
                                None)
    assert call(flags=B.R2L_FLAG_L2R) == B.R2L_ERR_UNSUPPORTED
    assert call(flags=0x8) == B.R2L_ERR_INVALID_ARG
    assert call(dy=None) == B.R2L_ERR_INVALID_ARG
    assert call(Dskip=FAKE) == B.R2L_ERR_INVALID_ARG            # dDskip required with Dskip
    assert call(z=FAKE) == B.R2L_ERR_INVALID_ARG                # dz required with z
    assert call(ld_u=4000) == B.R2L_ERR_INVALID_ARG
    assert call(ws=None, wsb=0) == B.R2L_ERR_WORKSPACE
    assert call(wsb=need - 1) == B.R2L_ERR_WORKSPACE


def test_layer_fwd_noalloc_rejects_before_touching_a_device():
    """The allocation-free forward checks its size against the static array
    (and its flags) before resolving the array on a device."""
    lib = B.lib()
    d = _dims()
    W = B.Weights(**{f[0]: FAKE for f in B.Weights._fields_})
    args = (C.byref(W), FAKE, FAKE, FAKE)
    big = 33024
    assert lib.r2l_layer_workspace_bytes(C.byref(d), B.R2L_BF16, big, 8, 4128) > (128 << 20)
    assert lib.r2l_layer_fwd_noalloc(C.byref(d), B.R2L_BF16, 0, *args, 8, big, 4128, None, None) == B.R2L_ERR_WORKSPACE
    assert lib.r2l_layer_fwd_noalloc(C.byref(d), B.R2L_BF16, B.R2L_FLAG_TRAIN, *args, 8, 256, 32, None,
                                     None) == B.R2L_ERR_UNSUPPORTED
    bad = _dims(N=8)
    assert lib.r2l_layer_fwd_noalloc(C.byref(bad), B.R2L_BF16, 0, *args, 8, 256, 32, None, None) == \
        B.R2L_ERR_INVALID_ARG
