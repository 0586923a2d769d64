"""GPU parity of the Dense-4x baseline (gate="amplitude": post-hoc bank top-k
of |SiLU(u) v|, no predictor) through the C ABI, against the oracle's
amplitude_forward. Same bars as the predictor path: the mask is bit-exact
against the GPU's own amplitudes, differs from the oracle's only where the
oracle's keep-th / (keep+1)-th amplitude gap is below 1e-3, and y is within
relative L2 2e-2 (per token with the GPU mask pinned, and end to end)."""
import numpy as np
import pytest
import torch

import oracle as o
import workloads as wl
from tests.conftest import gpu_available
from tests.test_gpu_parity import GAP, MID, REL_L2, dev, host, rel_l2, words

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def make_amp(layer, keep=16):
    import activation_sparse_ffn_amd as sffn
    L = layer
    return sffn.SparseFFN(dev(L.W_g), dev(L.W_u), dev(L.W_d), keep=keep, gate="amplitude")


def check_amplitude(layer, x, y, mask, amp, tokens=None, keep=16):
    L = layer
    T = x.shape[0]
    rows = np.arange(T) if tokens is None else np.asarray(tokens)
    gw = words(mask)
    ga = host(amp).astype(np.float64)
    yg = o.widen(host(y))
    # 1. the GPU's amplitudes give the GPU's mask
    np.testing.assert_array_equal(o.mask_to_words(o.bank_topk_mask(np.abs(ga[rows]), 64, keep)), gw[rows])
    assert (np.bitwise_count(gw[rows]) == keep).all()
    # 2. against the oracle
    r = o.amplitude_forward(x, L.W_g, L.W_u, L.W_d, keep=keep, tokens=rows)
    scale = max(np.abs(r["a"]).max(), 1.0)
    assert np.abs(ga[rows] - r["a"]).max() <= 2e-3 * scale
    gap = o.logit_gap(r["score"], 64, keep)
    diff = gw[rows] != r["words"]
    assert (gap[diff] < GAP).all(), f"mask differs with gap {gap[diff].max()}"
    # 3. y with the GPU mask pinned, per token, and end to end
    rp = o.amplitude_forward(x, L.W_g, L.W_u, L.W_d, keep=keep, mask_in=gw, tokens=rows)
    for n, t in enumerate(rows):
        e = rel_l2(yg[t], rp["y"][n])
        assert e <= REL_L2, f"token {t}: rel-L2 {e:.3e} (mask pinned)"
    assert rel_l2(yg[rows], r["y"]) <= REL_L2
    return int(diff.sum())


@pytest.fixture(scope="module")
def full_layer():
    return wl.make_layer(wl.FULL, seed=0, bias_var=0.5)


@pytest.fixture(scope="module")
def amp_full(full_layer):
    return make_amp(full_layer)


@pytest.mark.parametrize("T", [1, 3, 5, 64, 130, 300])
def test_amplitude_full(full_layer, amp_full, T):
    x = wl.make_tokens(wl.FULL, T, seed=4000 + T)
    xd = dev(x)
    y, mask, amp = amp_full(xd, return_mask=True, return_logits=True)
    y0 = amp_full(xd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(y0), host(y))
    rows = None if T <= 8 else [0, 1, T // 2, T - 1]
    check_amplitude(full_layer, x, y, mask, amp, tokens=rows)
    assert amp_full.stage_names(T)[0] in ("gateup_dense", "gateup_amp_gemm")


@pytest.mark.parametrize("T", [2, 5, 40, 300])
def test_amplitude_mid(T):
    L = wl.make_layer(MID, seed=11)
    ffn = make_amp(L)
    x = wl.make_tokens(MID, T, seed=T)
    y, mask, amp = ffn(dev(x), return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    check_amplitude(L, x, y, mask, amp)


def test_amplitude_tiny_fp32():
    L = wl.make_layer(wl.TINY, seed=3)
    ffn = make_amp(L)
    x = wl.make_tokens(wl.TINY, 8, seed=9)
    y, mask, amp = ffn(dev(x), return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    check_amplitude(L, x, y, mask, amp)


def test_amplitude_decode_reads_kept_down_columns_only(full_layer, amp_full):
    """Decode: down reads only the kept channels' rows of W_d^T, so NaN in
    the W_d columns of dropped channels leaves y bit-identical."""
    x = dev(wl.make_tokens(wl.FULL, 1, seed=77))
    y, mask = amp_full(x, return_mask=True)
    torch.cuda.synchronize()
    kept = o.words_to_mask(words(mask))[0]
    W_d = full_layer.W_d.copy()
    W_d[:, ~kept] = np.uint16(0x7FC0)          # bf16 quiet NaN
    import activation_sparse_ffn_amd as sffn
    bad = sffn.SparseFFN(dev(full_layer.W_g), dev(full_layer.W_u), dev(W_d), keep=16, gate="amplitude")
    y2 = bad(x)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(y2), host(y))
