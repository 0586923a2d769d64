"""Pins of the oracle's Dense-4x baseline (post-hoc amplitude sparsity):
hand-worked selections, the dense special case against a textbook SwiGLU,
and invariants that a dropped absolute value, a wrong operand or a dense
down projection would break."""
import numpy as np
import pytest
import torch

import oracle as o


def _layer(rng, d, d_i, dtype=np.float32):
    W_g = (rng.standard_normal((d_i, d)) / np.sqrt(d)).astype(dtype)
    W_u = (rng.standard_normal((d_i, d)) / np.sqrt(d)).astype(dtype)
    W_d = (rng.standard_normal((d, d_i)) / np.sqrt(d_i)).astype(dtype)
    return W_g, W_u, W_d


def test_hand_example_ranks_by_magnitude():
    # x = e_0, so u_j = W_g[j, 0] and v_j = W_u[j, 0]:
    #   u = [2, -1, 0.5, 3], v = [1, 4, -8, -0.5]
    #   SiLU(u) * v ~ [1.76, -1.08, -2.49, -1.43]
    # The two largest magnitudes are channels 2 and 0 (ranking the signed
    # values would pick 0 and 1).
    x = np.array([[1.0, 0.0]], dtype=np.float32)
    W_g = np.array([[2, 0], [-1, 0], [0.5, 0], [3, 0]], dtype=np.float32)
    W_u = np.array([[1, 0], [4, 0], [-8, 0], [-0.5, 0]], dtype=np.float32)
    W_d = np.array([[1, 0, 0, 0], [0, 0, 1, 0]], dtype=np.float32)
    r = o.amplitude_forward(x, W_g, W_u, W_d, bank=4, keep=2)
    np.testing.assert_array_equal(r["mask"][0], [True, False, True, False])
    # y picks channels 0 and 2 through W_d: SiLU(2) * 1 and SiLU(0.5) * (-8)
    silu = lambda t: t / (1.0 + np.exp(-t))
    np.testing.assert_allclose(r["y"][0], [silu(2.0), -8.0 * silu(0.5)], rtol=1e-7)
    assert r["h"][0, 1] == 0.0 and r["h"][0, 3] == 0.0


def test_keep_all_is_textbook_dense_swiglu():
    rng = np.random.default_rng(0)
    d, d_i = 32, 128
    W_g, W_u, W_d = _layer(rng, d, d_i)
    x = rng.standard_normal((5, d)).astype(np.float32)
    r = o.amplitude_forward(x, W_g, W_u, W_d, bank=64, keep=64)
    assert r["mask"].all()
    X = torch.from_numpy(x).double()
    ref = (torch.nn.functional.silu(X @ torch.from_numpy(W_g).double().T)
           * (X @ torch.from_numpy(W_u).double().T)) @ torch.from_numpy(W_d).double().T
    # the oracle rounds the amplitudes to fp32 (the ranking precision)
    np.testing.assert_allclose(r["y"], ref.numpy(), rtol=1e-6, atol=1e-7)


def test_mask_keeps_the_largest_magnitudes_per_bank():
    rng = np.random.default_rng(1)
    d, d_i, bank, keep = 16, 64, 16, 4
    W_g, W_u, W_d = _layer(rng, d, d_i)
    x = rng.standard_normal((7, d)).astype(np.float32)
    r = o.amplitude_forward(x, W_g, W_u, W_d, bank=bank, keep=keep)
    s = r["score"].reshape(7, d_i // bank, bank)
    m = r["mask"].reshape(7, d_i // bank, bank)
    assert (m.sum(-1) == keep).all()
    # every kept magnitude is at least every dropped one, bank by bank
    kept_min = np.where(m, s, np.inf).min(-1)
    drop_max = np.where(m, -np.inf, s).max(-1)
    assert (kept_min >= drop_max).all()
    # and the signs of the amplitudes are mixed, so magnitude matters
    a = r["a"].reshape(7, d_i // bank, bank)
    assert (np.where(m, a, 0.0) < 0).any()


def test_sign_and_scale_invariants():
    rng = np.random.default_rng(2)
    d, d_i = 32, 128
    W_g, W_u, W_d = _layer(rng, d, d_i)
    x = rng.standard_normal((4, d)).astype(np.float32)
    r = o.amplitude_forward(x, W_g, W_u, W_d)
    # negating W_u negates every amplitude: same mask, y negated exactly
    rn = o.amplitude_forward(x, W_g, -W_u, W_d)
    np.testing.assert_array_equal(rn["words"], r["words"])
    np.testing.assert_array_equal(rn["y"], -r["y"])
    # W_d does not enter the mask; doubling it doubles y exactly
    r2 = o.amplitude_forward(x, W_g, W_u, 2 * W_d)
    np.testing.assert_array_equal(r2["words"], r["words"])
    np.testing.assert_array_equal(r2["y"], 2 * r["y"])


def test_down_reads_kept_columns_only():
    rng = np.random.default_rng(3)
    d, d_i = 32, 128
    W_g, W_u, W_d = _layer(rng, d, d_i)
    x = rng.standard_normal((3, d)).astype(np.float32)
    r = o.amplitude_forward(x, W_g, W_u, W_d)
    dropped = ~r["mask"].any(axis=0)
    assert dropped.any()
    W_bad = W_d.copy()
    W_bad[:, dropped] = np.nan
    rb = o.amplitude_forward(x, W_g, W_u, W_bad)
    np.testing.assert_array_equal(rb["y"], r["y"])


def test_mask_pinned_mode_and_gap():
    rng = np.random.default_rng(4)
    d, d_i = 32, 128
    W_g, W_u, W_d = _layer(rng, d, d_i)
    x = rng.standard_normal((6, d)).astype(np.float32)
    r = o.amplitude_forward(x, W_g, W_u, W_d)
    rp = o.amplitude_forward(x, W_g, W_u, W_d, mask_in=r["words"], tokens=[1, 4])
    np.testing.assert_array_equal(rp["y"], r["y"][[1, 4]])
    gap = o.logit_gap(r["score"], 64, 16)
    assert (gap >= 0).all()
    assert (o.logit_gap(r["score"], 64, 64) == 0).all()
