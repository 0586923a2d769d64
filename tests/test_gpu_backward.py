"""GPU parity of the backward pass (soft surrogate gradient through the bank
top-k) through the C ABI, against the oracle's backward with the forward's
mask given to both sides. Every gradient is within relative L2 2e-2 (bf16
operands, fp32 accumulation, against float64)."""
import numpy as np
import pytest
import torch

import oracle as o
import workloads as wl
from tests.conftest import gpu_available
from tests.test_gpu_parity import MID, dev, host, make_ffn, rel_l2, words

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

REL = 2e-2
KEYS = [("x", "g_x"), ("A", "g_A"), ("B", "g_B"), ("W_g", "g_Wg"), ("W_u", "g_Wu"), ("W_d", "g_Wd"),
        ("bias", "g_bias")]


def run_and_check(layer, T, gate, keep, tau, seed, bias=True):
    ffn = make_ffn(layer, bias=bias, keep=keep, gate=gate)
    shape = wl.LayerShape(d=layer.W_g.shape[1], d_i=layer.W_g.shape[0], rank=layer.A.shape[0])
    x = wl.make_tokens(shape, T, seed=seed)
    gy = wl.make_tokens(shape, T, seed=seed + 1)
    xd, gyd = dev(x), dev(gy)
    _, mask = ffn(xd, return_mask=True)
    g = ffn.backward(xd, gyd, mask, tau=tau)
    torch.cuda.synchronize()
    r = o.backward(x, layer.A, layer.B, layer.W_g, layer.W_u, layer.W_d, gy,
                   bias=layer.bias if bias else None, keep=keep, gate=gate, tau=tau, mask_in=words(mask))
    for name, key in KEYS:
        if g[name] is None:
            assert r[key] is None
            continue
        e = rel_l2(host(g[name]), r[key])
        assert e <= REL, f"{name}: rel-L2 {e:.3e}"
    return g, r


@pytest.fixture(scope="module")
def mid_layer():
    return wl.make_layer(MID, seed=21, bias_var=0.5)


@pytest.mark.parametrize("T", [1, 5, 64, 300])
@pytest.mark.parametrize("gate", ["pred", "silu"])
def test_backward_mid(mid_layer, T, gate):
    run_and_check(mid_layer, T, gate, 16, 1.0, seed=100 + T)


@pytest.mark.parametrize("tau", [0.25, float("inf")])
def test_backward_temperature(mid_layer, tau):
    """A sharp surrogate and none at all (tau = inf: the predictor only
    feels the gate of the kept channels)."""
    run_and_check(mid_layer, 40, "pred", 16, tau, seed=7)


def test_backward_full_bank(mid_layer):
    run_and_check(mid_layer, 24, "pred", 64, 1.0, seed=3)


def test_backward_no_bias_and_zero_tokens(mid_layer):
    run_and_check(mid_layer, 8, "silu", 16, 1.0, seed=5, bias=False)
    ffn = make_ffn(mid_layer, bias=True)
    x = dev(wl.make_tokens(MID, 1, seed=1))[:0]
    mask = torch.empty((0, MID.d_i // 64), dtype=torch.int64, device="cuda")
    g = ffn.backward(x, x, mask)
    torch.cuda.synchronize()
    for name in ("A", "B", "W_g", "W_u", "W_d", "bias"):
        assert (g[name] == 0).all()


@pytest.fixture(scope="module")
def full_layer():
    return wl.make_layer(wl.FULL, seed=0, bias_var=0.5)


@pytest.mark.parametrize("T,gate", [(64, "pred"), (300, "silu")])
def test_backward_full(full_layer, T, gate):
    run_and_check(full_layer, T, gate, 16, 1.0, seed=900 + T)


@pytest.mark.parametrize("T", [70, 300])
def test_backward_with_packed_weight_transposes(mid_layer, T):
    """A layer created for the backward (W_g^T and W_u^T packed once) gives
    the same gradients bit for bit, from a smaller workspace."""
    import activation_sparse_ffn_amd as sffn
    x = dev(wl.make_tokens(MID, T, seed=41))
    gy = dev(wl.make_tokens(MID, T, seed=42))
    plain = make_ffn(mid_layer, bias=True)
    L = mid_layer
    ready = sffn.SparseFFN(dev(L.W_g), dev(L.W_u), dev(L.W_d), dev(L.A), dev(L.B), dev(L.bias),
                           for_backward=True)
    assert ready.packed.numel() == plain.packed.numel() + 4 * MID.d * MID.d_i
    _, mask = plain(x, return_mask=True)
    g0 = plain.backward(x, gy, mask)
    g1 = ready.backward(x, gy, mask)
    torch.cuda.synchronize()
    for name in ("x", "A", "B", "bias", "W_g", "W_u", "W_d"):
        assert torch.equal(g0[name], g1[name]), name
    lib = sffn.load_library()
    assert lib.sparse_ffn_backward_workspace_size(ready._h, T) \
        == lib.sparse_ffn_backward_workspace_size(plain._h, T) - 4 * MID.d * MID.d_i


# d = 4096, d_i = 1024, rank 64 at T = 2880: the g_x GEMMs (M = T, N = d)
# have 12 x 16 = 192 output tiles of 256 x 256, enough to run on the 256-wide
# kernel; g_z A (K = rank = 64) stores fp32 in a single K step, and g_u W_g,
# g_v W_u then add into g_x in the accumulating epilogue.
WIDE_GX = wl.LayerShape(d=4096, d_i=1024, rank=64)


@pytest.fixture(scope="module")
def wide_gx_layer():
    return wl.make_layer(WIDE_GX, seed=31, bias_var=0.5)


@pytest.mark.parametrize("gate", ["pred", "silu"])
def test_backward_256_wide_gx_gemms(wide_gx_layer, gate):
    run_and_check(wide_gx_layer, 2880, gate, 16, 1.0, seed=2880)


def test_backward_full_layer_biased_256_wide_logits(full_layer):
    """T = 1024 on the full layer with a bias: the recomputed logits
    p = z B^T + b have 4 x 56 = 224 tiles of 256 x 256 and take the biased
    256-wide fp32 GEMM, the one a 4096-token chunk runs."""
    run_and_check(full_layer, 1024, "pred", 16, 1.0, seed=1024)
