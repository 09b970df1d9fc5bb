"""The allocation-free layer forward (r2l_layer_fwd_noalloc, for callers that
cannot allocate: graph capture, serving loops) against the workspace entry
point r2l_layer_fwd, through the C ABI: two calls in a row on the same
GPU's static array, the second with a smaller input (so the array holds the
first call's leftovers), each bit-identical to the workspace entry point's
output (same kernels, same inputs); and an input beyond the array's size is
refused with R2L_ERR_WORKSPACE, leaving the output untouched."""
import ctypes as C

import numpy as np
import pytest
import torch

from reverse_selective_scan_amd import binding as B
from reverse_selective_scan_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(lens, seed, **dims):
    wl = synth.custom(lens, seed=seed, h_kind="rms", **dims)
    W = synth.make_weights(wl, affine_ln=True)
    w = B.to_device_weights(W, torch.bfloat16, DEV)
    h = torch.from_numpy(synth.make_hidden(wl)).to(torch.bfloat16).to(DEV)
    cu, nseq, ms = B.cu_seqlens_device(wl.cu_seqlens(), wl.n_tokens, DEV)
    return w, h, cu, nseq, ms


def _both(w, h, cu, nseq, ms):
    ref_out = torch.full_like(h, float("nan"))
    ref_br = torch.full(h.shape, float("nan"), dtype=torch.float32, device=DEV)
    B.r2l_layer_fwd(h, w, cu, out=ref_out, branch_out=ref_br, nseq=nseq, max_seqlen=ms)
    out = torch.full_like(h, float("nan"))
    br = torch.full(h.shape, float("nan"), dtype=torch.float32, device=DEV)
    B.r2l_layer_fwd_noalloc(h, w, cu, nseq, ms, out=out, branch_out=br)
    torch.cuda.synchronize()
    return (ref_out, ref_br), (out, br)


def test_noalloc_matches_workspace_entry_point_twice_then_refuses_too_large():
    print("\n[case] noalloc: denoise block shape (8 x 32 tokens, D 2048), then 3 short sequences", flush=True)
    first = _inputs([32] * 8, 5, d_model=2048, d_inner=4096, dt_rank=128)
    (ro, rb), (o, b) = _both(*first)
    assert torch.equal(o, ro) and torch.equal(b, rb), "first call differs from r2l_layer_fwd"
    second = _inputs([5, 0, 13], 6, d_model=2048, d_inner=4096, dt_rank=128)
    (ro, rb), (o, b) = _both(*second)
    assert torch.equal(o, ro) and torch.equal(b, rb), "second (smaller) call differs from r2l_layer_fwd"
    print("[noalloc] both calls bit-identical to r2l_layer_fwd", flush=True)
    # beyond the static array: refused before any launch, output untouched
    w, h, cu, nseq, ms = first
    T = 4096
    hb = torch.zeros(T, 2048, dtype=torch.bfloat16, device=DEV)
    ob = torch.full_like(hb, 7.0)
    cub, nb, mb = B.cu_seqlens_device([0, T], T, DEV)
    d = B.dims_of(w)
    assert B.r2l_layer_workspace_bytes(d, B.R2L_BF16, T, nb, mb) > (128 << 20)
    W = B.Weights(**{f[0]: w[f[0]].data_ptr() for f in B.Weights._fields_})
    rc = B.lib().r2l_layer_fwd_noalloc(C.byref(d), B.R2L_BF16, 0, C.byref(W), hb.data_ptr(), ob.data_ptr(),
                                       cub.data_ptr(), nb, T, mb, None, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == B.R2L_ERR_WORKSPACE
    assert bool((ob == 7.0).all())
