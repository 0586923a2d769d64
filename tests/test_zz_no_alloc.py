"""The forward entry point that allocates nothing (sparse_ffn_forward_noalloc,
its scratch a static per-GPU array inside the library), called through the C
ABI, against sparse_ffn_forward with a caller-owned workspace: the same
kernels on the same inputs, so y, the mask and the logits must agree bit for
bit. Two calls in a row, the second with a smaller input, on every execution
path; a call beyond the scratch is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

MID = wl.LayerShape(d=512, d_i=2048, rank=64)


def dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def make(shape, seed):
    import activation_sparse_ffn_amd as sffn
    L = wl.make_layer(shape, seed=seed, bias_var=0.5)
    return sffn.SparseFFN(dev(L.W_g), dev(L.W_u), dev(L.W_d), dev(L.A), dev(L.B), dev(L.bias))


def raw_noalloc(ffn, x):
    """sparse_ffn_forward_noalloc through ctypes; returns y, mask, logits."""
    lib = ffn._lib
    T = x.shape[0]
    y = torch.empty_like(x)
    mask = torch.empty((T, ffn.d_i // 64), dtype=torch.int64, device="cuda")
    logits = torch.empty((T, ffn.d_i), dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.sparse_ffn_forward_noalloc(ffn._h, ctypes.c_void_p(x.data_ptr()), T, ctypes.c_void_p(y.data_ptr()),
                                        ctypes.c_void_p(mask.data_ptr()), ctypes.c_void_p(logits.data_ptr()),
                                        stream)
    assert st == 0, lib.sparse_ffn_last_error().decode()
    return y, mask, logits


def same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def check_sequence(ffn, shape, Ts, seed):
    """Each T in turn through both entry points (the no-alloc calls back to
    back, so the second finds the first's leftovers in the scratch)."""
    xs = [dev(wl.make_tokens(shape, T, seed=seed + i)) for i, T in enumerate(Ts)]
    refs = []
    for x in xs:
        y, m, lg = ffn(x, return_mask=True, return_logits=True,
                       workspace=torch.empty(ffn.workspace_size(x.shape[0]), dtype=torch.uint8, device="cuda"))
        refs.append((y.clone(), m.clone(), lg.clone()))
    torch.cuda.synchronize()
    outs = [raw_noalloc(ffn, x) for x in xs]
    torch.cuda.synchronize()
    for T, out, ref in zip(Ts, outs, refs):
        for name, a, b in zip(("y", "mask", "logits"), out, ref):
            assert same(a, b), f"T = {T}: {name} differs"


def test_full_layer_batched_then_decode():
    """The skinny MFMA path (T = 32), then the fused token-gather path
    (T = 1) of the full layer."""
    ffn = make(wl.FULL, seed=0)
    check_sequence(ffn, wl.FULL, [32, 1], seed=10)
    check_sequence(ffn, wl.FULL, [4, 2], seed=20)


def test_mid_layer_every_path_shrinking():
    """The 256-wide MFMA path (T = 300), skinny (T = 40), and the generic
    token-gather kernels (T = 3), each call smaller than the one before."""
    ffn = make(MID, seed=3)
    check_sequence(ffn, MID, [300, 40, 3], seed=30)


def test_beyond_the_scratch_is_refused():
    import activation_sparse_ffn_amd as sffn
    ffn = make(wl.FULL, seed=0)
    T = 1024
    assert ffn.workspace_size(T) > 16 << 20
    x = torch.zeros((T, 4096), dtype=torch.bfloat16, device="cuda")
    y = torch.full_like(x, 7.0)
    lib = ffn._lib
    st = lib.sparse_ffn_forward_noalloc(ffn._h, ctypes.c_void_p(x.data_ptr()), T, ctypes.c_void_p(y.data_ptr()),
                                        None, None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == sffn.SFFN_ERR_WORKSPACE
    assert b"scratch" in lib.sparse_ffn_last_error()
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())          # nothing was enqueued
    assert lib.sparse_ffn_forward_noalloc(ffn._h, None, 0, None, None, None, None) == 0   # T = 0: no-op
