"""ctypes binding of libr2l.so (see include/r2l.h).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing or cannot be
loaded, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# R2L_LIB overrides the library file (the host-sanitizer test loads its
# instrumented build this way); the default is the in-tree libr2l.so
LIB_PATH = os.environ.get("R2L_LIB") or os.path.join(_PKG, "libr2l.so")

R2L_OK, R2L_ERR_INVALID_ARG, R2L_ERR_UNSUPPORTED, R2L_ERR_WORKSPACE, R2L_ERR_HIP = 0, -1, -2, -3, -4
R2L_F32, R2L_BF16 = 0, 1
R2L_FLAG_NO_LN = 0x1
R2L_FLAG_L2R = 0x2
R2L_FLAG_TRAIN = 0x4


class R2LError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {code})")
        self.code = code


class Dims(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("d_inner", C.c_int32), ("d_state", C.c_int32),
                ("dt_rank", C.c_int32), ("d_conv", C.c_int32)]


class Grads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "in_proj_w", "conv_w", "conv_b", "x_proj_w", "dt_proj_w", "out_proj_w",
        "dt_proj_b", "A_log", "Dskip", "ln_w", "ln_b", "s")]


class Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "in_proj_w", "conv_w", "conv_b", "x_proj_w", "dt_proj_w", "out_proj_w",
        "dt_proj_b", "A_log", "Dskip", "ln_w", "ln_b", "s")]


_P, _I32, _I64, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
_SIGS = {
    "r2l_version": (C.c_int, []),
    "r2l_status_string": (C.c_char_p, [C.c_int]),
    "r2l_check_cu_seqlens": (C.c_int, [_P, _I32, _I64, _I32]),
    "r2l_layer_workspace_bytes": (_SZ, [C.POINTER(Dims), C.c_int, _I64, _I32, _I32]),
    "r2l_layer_fwd": (C.c_int, [C.POINTER(Dims), C.c_int, C.c_uint32, C.POINTER(Weights), _P, _P, _P,
                                _I32, _I64, _I32, _P, _SZ, _P, _P]),
    "r2l_layer_fwd_noalloc": (C.c_int, [C.POINTER(Dims), C.c_int, C.c_uint32, C.POINTER(Weights), _P, _P, _P,
                                        _I32, _I64, _I32, _P, _P]),
    "r2l_conv_fwd": (C.c_int, [C.POINTER(Dims), C.c_int, C.c_uint32, _P, _I64, _P, _P, _P, _P, _P, _P, _I32,
                               _I64, _I32, _P]),
    "r2l_scan_workspace_bytes": (_SZ, [C.POINTER(Dims), _I64, _I32, _I32]),
    "r2l_scan_fwd": (C.c_int, [C.POINTER(Dims), C.c_int, C.c_uint32, _P, _I64, _P, _I64, _P, _P, _P, _I64, _P,
                               _P, _I64, _P, _P, _I32, _I64, _I32, _P, _SZ, _P]),
    "r2l_scan_bwd_workspace_bytes": (_SZ, [C.POINTER(Dims), _I64, _I32]),
    "r2l_layer_bwd_workspace_bytes": (_SZ, [C.POINTER(Dims), C.c_int, _I64, _I32, _I32]),
    "r2l_layer_train_workspace_bytes": (_SZ, [C.POINTER(Dims), C.c_int, _I64, _I32, _I32]),
    "r2l_layer_bwd": (C.c_int, [C.POINTER(Dims), C.c_int, C.c_uint32, C.POINTER(Weights), _P, _P, _P,
                                C.POINTER(Grads), _P, _I32, _I64, _I32, _P, _P, _SZ, _P]),
    "r2l_scan_bwd": (C.c_int, [C.POINTER(Dims), C.c_int, C.c_uint32, _P, _I64, _P, _I64, _P, _P, _P, _I64, _P,
                               _P, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I64, _P, _SZ, _P]),
    "r2l_gemm_nt": (C.c_int, [C.c_int, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, C.c_int, _P, C.c_size_t, _P]),
    "r2l_timing_enable": (C.c_int, [C.c_int]),
    "r2l_timing_reset": (C.c_int, []),
    "r2l_timing_read": (C.c_int, [C.POINTER(C.c_char_p), C.POINTER(C.c_double), C.POINTER(C.c_int64),
                                  C.c_int]),
}

_lib_handle = None


def lib() -> C.CDLL:
    """Load libr2l.so (once).  Raises if it is not built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m reverse_selective_scan_amd.build`")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib_handle = h
    return _lib_handle


def _check(fn: str, code: int) -> None:
    if code != R2L_OK:
        raise R2LError(fn, code, lib().r2l_status_string(code).decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _act(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return R2L_BF16
    if t.dtype == torch.float32:
        return R2L_F32
    raise TypeError(f"unsupported activation dtype {t.dtype}")


def _need(t: torch.Tensor, name: str, dtype=None, contiguous=True):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def dims_of(w: Dict[str, torch.Tensor]) -> Dims:
    return Dims(d_model=w["in_proj_w"].shape[1], d_inner=w["conv_w"].shape[0],
                d_state=w["A_log"].shape[1], dt_rank=w["dt_proj_w"].shape[1], d_conv=w["conv_w"].shape[1])


def cu_seqlens_device(cu, n_tokens: int, device) -> tuple:
    """(device int32 tensor, nseq, max_seqlen) from host offsets, validated
    on the host by the library's own checker."""
    cu_np = np.ascontiguousarray(np.asarray(cu, dtype=np.int32))
    nseq = int(cu_np.size - 1)
    if nseq < 1:
        raise ValueError("cu_seqlens needs at least two entries")
    lens = np.diff(cu_np.astype(np.int64))
    max_seqlen = int(lens.max()) if lens.size else 0
    _check("r2l_check_cu_seqlens",
           lib().r2l_check_cu_seqlens(cu_np.ctypes.data, nseq, int(n_tokens), max_seqlen))
    return torch.from_numpy(cu_np).to(device), nseq, max_seqlen


# ---------------------------------------------------------------------------
# the three operations of the path (+ the projection GEMM)
# ---------------------------------------------------------------------------
def r2l_layer_workspace_bytes(dims: Dims, act: int, n_tokens: int, nseq: int, max_seqlen: int) -> int:
    return int(lib().r2l_layer_workspace_bytes(C.byref(dims), act, n_tokens, nseq, max_seqlen))


def r2l_layer_bwd_workspace_bytes(dims: Dims, act: int, n_tokens: int, nseq: int, max_seqlen: int) -> int:
    return int(lib().r2l_layer_bwd_workspace_bytes(C.byref(dims), act, n_tokens, nseq, max_seqlen))


def r2l_layer_train_workspace_bytes(dims: Dims, act: int, n_tokens: int, nseq: int, max_seqlen: int) -> int:
    return int(lib().r2l_layer_train_workspace_bytes(C.byref(dims), act, n_tokens, nseq, max_seqlen))


def r2l_layer_fwd(h: torch.Tensor, w: Dict[str, torch.Tensor], cu_seqlens, *, out: Optional[torch.Tensor] = None,
                  flags: int = 0, branch_out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
                  nseq: Optional[int] = None) -> torch.Tensor:
    """One ReverseMambaLayer hook: returns h + tanh(s) * LN(R2L-Mamba(h)).

    h: [T, D] device tensor (bf16 or fp32); w: dict of device tensors named
    as in r2l_weights (s is a 1-element fp32 device tensor); cu_seqlens:
    host offsets (validated, then uploaded) or an int32 device tensor (then
    nseq and max_seqlen must be given).  out may be h (in place)."""
    _need(h, "h")
    act = _act(h)
    T = h.shape[0]
    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        if nseq is None or max_seqlen is None:
            raise ValueError("device cu_seqlens needs nseq and max_seqlen")
        cu_dev = cu_seqlens
    else:
        cu_dev, nseq, max_seqlen = cu_seqlens_device(cu_seqlens, T, h.device)
    d = dims_of(w)
    for k in ("in_proj_w", "conv_w", "conv_b", "x_proj_w", "dt_proj_w", "out_proj_w"):
        _need(w[k], k, h.dtype)
    for k in ("dt_proj_b", "A_log", "Dskip", "ln_w", "ln_b", "s"):
        _need(w[k], k, torch.float32)
    if out is None:
        out = torch.empty_like(h)
    _need(out, "out", h.dtype)
    if branch_out is not None:
        _need(branch_out, "branch_out", torch.float32)
    need = (r2l_layer_train_workspace_bytes if flags & R2L_FLAG_TRAIN else r2l_layer_workspace_bytes)(
        d, act, T, nseq, max_seqlen)
    if workspace is None or workspace.numel() < need:
        if flags & R2L_FLAG_TRAIN:
            raise ValueError("R2L_FLAG_TRAIN needs a caller workspace of r2l_layer_train_workspace_bytes "
                             "(it is the backward's saved buffer)")
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=h.device)
    W = Weights(**{f[0]: _ptr(w[f[0]]) for f in Weights._fields_})
    _check("r2l_layer_fwd", lib().r2l_layer_fwd(
        C.byref(d), act, flags, C.byref(W), _ptr(h), _ptr(out), _ptr(cu_dev), nseq, T, max_seqlen,
        _ptr(workspace), workspace.numel(), _ptr(branch_out), _stream()))
    return out


def r2l_layer_fwd_noalloc(h: torch.Tensor, w: Dict[str, torch.Tensor], cu_seqlens: torch.Tensor, nseq: int,
                          max_seqlen: int, *, out: torch.Tensor, flags: int = 0,
                          branch_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """r2l_layer_fwd on the library's static scratch array: no workspace and
    no allocation here either (out, and branch_out if wanted, are given;
    cu_seqlens is an int32 device tensor)."""
    _need(h, "h")
    _need(out, "out", h.dtype)
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    if branch_out is not None:
        _need(branch_out, "branch_out", torch.float32)
    d = dims_of(w)
    W = Weights(**{f[0]: _ptr(w[f[0]]) for f in Weights._fields_})
    _check("r2l_layer_fwd_noalloc", lib().r2l_layer_fwd_noalloc(
        C.byref(d), _act(h), flags, C.byref(W), _ptr(h), _ptr(out), _ptr(cu_seqlens), nseq, h.shape[0],
        max_seqlen, _ptr(branch_out), _stream()))
    return out


def r2l_layer_bwd(h: torch.Tensor, w: Dict[str, torch.Tensor], cu_seqlens, g_out: torch.Tensor, *,
                  dh: Optional[torch.Tensor] = None, flags: int = 0,
                  workspace: Optional[torch.Tensor] = None,
                  grads: Optional[Dict[str, torch.Tensor]] = None,
                  max_seqlen: Optional[int] = None, nseq: Optional[int] = None,
                  saved: Optional[torch.Tensor] = None):
    """Gradient of r2l_layer_fwd: given g_out = dL/dh+, returns (dh, grads)
    with grads a dict of fp32 device tensors named like the weights (plus
    "s"); pass `grads` (and `dh`, `workspace`) to reuse buffers.  cu_seqlens
    as for r2l_layer_fwd.  saved: the workspace of r2l_layer_fwd(...,
    flags=R2L_FLAG_TRAIN, workspace=saved) on the same h and weights (None:
    the forward is recomputed)."""
    _need(h, "h")
    act = _act(h)
    T = h.shape[0]
    _need(g_out, "g_out", h.dtype)
    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        if nseq is None or max_seqlen is None:
            raise ValueError("device cu_seqlens needs nseq and max_seqlen")
        cu_dev = cu_seqlens
    else:
        cu_dev, nseq, max_seqlen = cu_seqlens_device(cu_seqlens, T, h.device)
    d = dims_of(w)
    if dh is None:
        dh = torch.empty_like(h)
    if grads is None:
        grads = {k: torch.empty(w[k].shape, dtype=torch.float32, device=h.device) for k, _ in Grads._fields_}
    for k, _ in Grads._fields_:
        _need(grads[k], "grads[" + k + "]", torch.float32)
        if grads[k].numel() != w[k].numel():
            raise ValueError(f"grads[{k}] has {grads[k].numel()} elements, the weight {w[k].numel()}")
    need = r2l_layer_bwd_workspace_bytes(d, act, T, nseq, max_seqlen)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=h.device)
    W = Weights(**{f[0]: _ptr(w[f[0]]) for f in Weights._fields_})
    G = Grads(**{f[0]: _ptr(grads[f[0]]) for f in Grads._fields_})
    if saved is not None:
        _need(saved, "saved", torch.uint8)
        if saved.numel() < r2l_layer_train_workspace_bytes(d, act, T, nseq, max_seqlen):
            raise ValueError("saved is smaller than r2l_layer_train_workspace_bytes")
    _check("r2l_layer_bwd", lib().r2l_layer_bwd(
        C.byref(d), act, flags, C.byref(W), _ptr(h), _ptr(g_out), _ptr(dh), C.byref(G), _ptr(cu_dev), nseq, T,
        max_seqlen, _ptr(saved), _ptr(workspace), workspace.numel(), _stream()))
    return dh, grads


def r2l_conv_fwd(x: torch.Tensor, conv_w: torch.Tensor, conv_b: torch.Tensor, cu_seqlens, *,
                 x_proj_w: Optional[torch.Tensor] = None, d_state: int = 16, dt_rank: Optional[int] = None,
                 want_u: bool = True, flags: int = 0):
    """Anti-causal conv + SiLU (+ x_proj); causal with flags=R2L_FLAG_L2R.
    x may be a strided view whose rows are contiguous (e.g. the x half of
    in_proj's output).  Returns (u or None, xdbl or None)."""
    _need(x, "x", contiguous=False)
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    act = _act(x)
    T, E = x.shape
    cu_dev, nseq, max_seqlen = cu_seqlens_device(cu_seqlens, T, x.device)
    R = dt_rank if dt_rank is not None else (x_proj_w.shape[0] - 2 * d_state if x_proj_w is not None else 1)
    d = Dims(d_model=64, d_inner=E, d_state=d_state, dt_rank=R, d_conv=conv_w.shape[1])
    u = torch.empty(T, E, dtype=x.dtype, device=x.device) if want_u else None
    xdbl = torch.empty(T, R + 2 * d_state, dtype=torch.float32, device=x.device) if x_proj_w is not None else None
    _check("r2l_conv_fwd", lib().r2l_conv_fwd(
        C.byref(d), act, flags, _ptr(x), x.stride(0), _ptr(conv_w), _ptr(conv_b), _ptr(x_proj_w), _ptr(u),
        _ptr(xdbl), _ptr(cu_dev), nseq, T, max_seqlen, _stream()))
    return u, xdbl


def r2l_scan_fwd(u: torch.Tensor, dt: torch.Tensor, A_log: torch.Tensor, B: torch.Tensor, C_: torch.Tensor,
                 cu_seqlens, *, Dskip: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                 dt_rank: int = 1, flags: int = 0) -> torch.Tensor:
    """Reverse selective scan with the Dskip term and SiLU(z) gate (left to
    right with flags=R2L_FLAG_L2R).  B and C may be strided column slices
    (row stride shared)."""
    _need(u, "u", contiguous=False)
    act = _act(u)
    T, E = u.shape
    for t, n in ((u, "u"), (dt, "dt"), (B, "B"), (C_, "C")):
        if t.stride(1) != 1:
            raise ValueError(f"{n} rows must be contiguous")
    if B.stride(0) != C_.stride(0):
        raise ValueError("B and C must share a row stride")
    _need(dt, "dt", torch.float32, contiguous=False)
    _need(A_log, "A_log", torch.float32)
    cu_dev, nseq, max_seqlen = cu_seqlens_device(cu_seqlens, T, u.device)
    d = Dims(d_model=64, d_inner=E, d_state=A_log.shape[1], dt_rank=dt_rank, d_conv=4)
    y = torch.empty(T, E, dtype=u.dtype, device=u.device)
    wsb = int(lib().r2l_scan_workspace_bytes(C.byref(d), T, nseq, max_seqlen))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=u.device)
    _check("r2l_scan_fwd", lib().r2l_scan_fwd(
        C.byref(d), act, flags, _ptr(u), u.stride(0), _ptr(dt), dt.stride(0), _ptr(A_log), _ptr(B), _ptr(C_),
        B.stride(0), _ptr(Dskip), _ptr(z), z.stride(0) if z is not None else 0, _ptr(y), _ptr(cu_dev), nseq, T,
        max_seqlen, _ptr(ws), ws.numel(), _stream()))
    return y


def r2l_scan_bwd(u: torch.Tensor, dt: torch.Tensor, A_log: torch.Tensor, B: torch.Tensor, C_: torch.Tensor,
                 cu_seqlens, dy: torch.Tensor, *, Dskip: Optional[torch.Tensor] = None,
                 z: Optional[torch.Tensor] = None, dt_rank: int = 1) -> Dict[str, torch.Tensor]:
    """Gradient of r2l_scan_fwd: given dy = dL/dy_out, returns fp32 tensors
    du, ddt, dA_log, dB, dC (and dDskip, dz when Dskip, z are given)."""
    _need(u, "u", contiguous=False)
    act = _act(u)
    T, E = u.shape
    for t, n in ((u, "u"), (dt, "dt"), (B, "B"), (C_, "C"), (dy, "dy")):
        if t.stride(1) != 1:
            raise ValueError(f"{n} rows must be contiguous")
    if B.stride(0) != C_.stride(0):
        raise ValueError("B and C must share a row stride")
    _need(dt, "dt", torch.float32, contiguous=False)
    _need(dy, "dy", u.dtype, contiguous=False)
    _need(A_log, "A_log", torch.float32)
    N = A_log.shape[1]
    cu_dev, nseq, _ = cu_seqlens_device(cu_seqlens, T, u.device)
    d = Dims(d_model=64, d_inner=E, d_state=N, dt_rank=dt_rank, d_conv=4)
    f32 = dict(dtype=torch.float32, device=u.device)
    out = {"du": torch.empty(T, E, **f32), "ddt": torch.empty(T, E, **f32), "dA_log": torch.empty(E, N, **f32),
           "dB": torch.empty(T, N, **f32), "dC": torch.empty(T, N, **f32)}
    if Dskip is not None:
        out["dDskip"] = torch.empty(E, **f32)
    if z is not None:
        out["dz"] = torch.empty(T, E, **f32)
    wsb = int(lib().r2l_scan_bwd_workspace_bytes(C.byref(d), T, nseq))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=u.device)
    _check("r2l_scan_bwd", lib().r2l_scan_bwd(
        C.byref(d), act, 0, _ptr(u), u.stride(0), _ptr(dt), dt.stride(0), _ptr(A_log), _ptr(B), _ptr(C_),
        B.stride(0), _ptr(Dskip), _ptr(z), z.stride(0) if z is not None else 0, _ptr(dy), dy.stride(0),
        _ptr(out["du"]), _ptr(out["ddt"]), _ptr(out["dA_log"]), _ptr(out["dB"]), _ptr(out["dC"]),
        _ptr(out.get("dDskip")), _ptr(out.get("dz")), _ptr(cu_dev), nseq, T, _ptr(ws), ws.numel(), _stream()))
    return out


def r2l_gemm_nt(A: torch.Tensor, B: torch.Tensor, *, out_f32: bool = False,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = A @ B^T on the library's GEMM (MFMA for bf16).  workspace: optional
    device scratch (uint8) that lets large problems split their last partial
    round of output tiles along K."""
    _need(A, "A")
    _need(B, "B", A.dtype)
    act = _act(A)
    M, K = A.shape
    N = B.shape[0]
    out = torch.empty(M, N, dtype=torch.float32 if (out_f32 or act == R2L_F32) else A.dtype, device=A.device)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())
    _check("r2l_gemm_nt", lib().r2l_gemm_nt(act, M, N, K, _ptr(A), K, _ptr(B), K, _ptr(out), N,
                                            1 if out.dtype == torch.float32 else 0, ws_ptr, ws_bytes, _stream()))
    return out


# ---------------------------------------------------------------------------
# per-kernel timing
# ---------------------------------------------------------------------------
def timing_enable(on: bool = True) -> None:
    _check("r2l_timing_enable", lib().r2l_timing_enable(1 if on else 0))


def timing_reset() -> None:
    lib().r2l_timing_reset()


def timing_read(max_names: Optional[int] = None) -> Dict[str, tuple]:
    """{kernel name: (total ms, launches)} since the last reset (every name
    unless max_names is given)."""
    if max_names is None:
        max_names = int(lib().r2l_timing_read(None, None, None, 0))
        if max_names < 0:
            _check("r2l_timing_read", max_names)
    max_names = max(max_names, 1)
    names = (C.c_char_p * max_names)()
    tot = (C.c_double * max_names)()
    cnt = (C.c_int64 * max_names)()
    n = lib().r2l_timing_read(names, tot, cnt, max_names)
    if n < 0:
        _check("r2l_timing_read", n)
    return {names[i].decode(): (tot[i], cnt[i]) for i in range(min(n, max_names))}


# ---------------------------------------------------------------------------
# weight upload helper (dtype marshalling of host arrays)
# ---------------------------------------------------------------------------
ACT_KEYS = ("in_proj_w", "conv_w", "conv_b", "x_proj_w", "dt_proj_w", "out_proj_w")
F32_KEYS = ("dt_proj_b", "A_log", "Dskip", "ln_w", "ln_b")


def to_device_weights(W: Dict[str, np.ndarray], act_dtype: torch.dtype, device="cuda") -> Dict[str, torch.Tensor]:
    out = {}
    for k in ACT_KEYS:  # values are exactly representable in act_dtype: the cast is exact
        out[k] = torch.from_numpy(np.ascontiguousarray(W[k], dtype=np.float32)).to(act_dtype).to(device)
    for k in F32_KEYS:
        out[k] = torch.from_numpy(np.ascontiguousarray(W[k], dtype=np.float32)).to(device)
    out["s"] = gate_tensor(float(W["s"]), device)
    return out


def gate_tensor(s: float, device="cuda") -> torch.Tensor:
    return torch.tensor([float(s)], dtype=torch.float32).to(device)
