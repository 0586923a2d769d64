"""Pins for the oracle's predictor and masked SwiGLU.

The layer is the predictor-gated sparse SwiGLU of "Continual LLM Upcycling"
(gist.science technical summary, Methodologie > 1. Architectuur: predictor
R^d -> R^448 -> R^{d_i}, routing signal in place of sigma(u), bank top-k,
inactive channels exactly zero; 2. Trainingsrecept stage 4: gate routed
through the predictor with a sigmoid; 3. Hardware Implicaties: gate, up and
down skipped for inactive channels).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as o
import workloads as wl

SIG = lambda a: 1.0 / (1.0 + math.exp(-a))  # noqa: E731


def _worked_example(bias=None):
    x = np.array([[1.0, 2.0 ** -8]], np.float32)
    A = np.array([[1, 1], [0, 2]], np.float32)
    B = np.array([[1, 0], [-1, 0], [0, 128], [2, -128]], np.float32)
    W_g = np.array([[1, 0], [5, 5], [0, 4], [7, 7]], np.float32)
    W_u = np.array([[3, 0], [5, 5], [2, 256], [7, 7]], np.float32)
    W_d = np.array([[1, 100, 2, 100], [-1, 100, 0.5, 100]], np.float32)
    return x, A, B, W_g, W_u, W_d, bias


def test_worked_example_pred_gate():
    # z0 = 1 + 2^-8 rounds (tie to even) to 1; z1 = 2^-7.
    # p = [1, -1, 1, 1]; bank {2,3} ties -> channel 2. Kept: 0 and 2.
    # u0 = 1, v0 = 3, u2 = 2^-6, v2 = 3.
    x, A, B, W_g, W_u, W_d, _ = _worked_example()
    r = o.forward(x, A, B, W_g, W_u, W_d, bank=2, keep=1, round_z_bf16=True)
    np.testing.assert_array_equal(r["z"], [[1.0, 2.0 ** -7]])
    np.testing.assert_array_equal(r["p"], [[1.0, -1.0, 1.0, 1.0]])
    np.testing.assert_array_equal(r["words"], [[1, 1]])
    s1 = SIG(1.0)
    want = [3 * s1 * (1 + 2.0 ** -5), s1 * (-3 + 3.0 / 128)]
    np.testing.assert_allclose(r["y"][0], want, rtol=1e-15)
    np.testing.assert_allclose(r["h"][0], [3 * s1, 0.0, 3 * s1 / 64, 0.0], rtol=1e-15)
    assert r["h"][0, 1] == 0.0 and r["h"][0, 3] == 0.0


def test_worked_example_silu_gate_and_bias():
    x, A, B, W_g, W_u, W_d, _ = _worked_example()
    r = o.forward(x, A, B, W_g, W_u, W_d, bank=2, keep=1, gate="silu", round_z_bf16=True)
    h0, h2 = SIG(1.0) * 3, SIG(2.0 ** -6) * 2.0 ** -6 * 3
    np.testing.assert_allclose(r["y"][0], [h0 + 2 * h2, -h0 + 0.5 * h2], rtol=1e-15)
    bias = np.array([0, 0, 0.5, 0], np.float32)
    r = o.forward(x, A, B, W_g, W_u, W_d, bias=bias, bank=2, keep=1, round_z_bf16=True)
    np.testing.assert_array_equal(r["p"], [[1.0, -1.0, 1.5, 1.0]])
    h0, h2 = SIG(1.0) * 3, SIG(1.5) * 3 / 64
    np.testing.assert_allclose(r["y"][0], [h0 + 2 * h2, -h0 + 0.5 * h2], rtol=1e-15)


def test_worked_example_without_z_rounding():
    # fp32 layer: z0 stays 1 + 2^-8, so p0 = 1 + 2^-8 and p3 = 1 + 2^-7
    # beats p2 = 1.
    x, A, B, W_g, W_u, W_d, _ = _worked_example()
    r = o.forward(x, A, B, W_g, W_u, W_d, bank=2, keep=1, round_z_bf16=False)
    np.testing.assert_array_equal(r["words"], [[1, 2]])
    p0, p3 = 1.0 + 2.0 ** -8, 1.0 + 2.0 ** -7
    u3 = 7 * (1 + 2.0 ** -8)
    h0, h3 = SIG(p0) * 3, SIG(p3) * u3 * u3
    np.testing.assert_allclose(r["y"][0], [h0 + 100 * h3, -h0 + 100 * h3], rtol=1e-14)


def test_predictor_exact_rational_brute_force():
    rng = np.random.default_rng(5)
    d, r_, d_i = 24, 6, 16
    x = wl.bf16_bits_from_f32(rng.standard_normal((2, d)).astype(np.float32))
    A = wl.bf16_bits_from_f32(rng.standard_normal((r_, d)).astype(np.float32))
    B = wl.bf16_bits_from_f32(rng.standard_normal((d_i, r_)).astype(np.float32))
    z, p = o.predictor_logits(x, A, B, None, round_z_bf16=False)
    X, Aw, Bw = o.widen(x), o.widen(A), o.widen(B)
    for t in range(2):
        for q in range(r_):
            exact = sum(Fraction(float(X[t, i])) * Fraction(float(Aw[q, i])) for i in range(d))
            assert abs(z[t, q] - float(exact)) <= 1e-15 * max(1.0, abs(float(exact)))
        for j in range(d_i):
            exact = sum(Fraction(float(z[t, q])) * Fraction(float(Bw[j, q])) for q in range(r_))
            assert p[t, j] == np.float32(float(exact))


def test_predictor_one_hot_closed_form():
    rng = np.random.default_rng(6)
    d, r_, d_i = 64, 8, 128
    x = wl.bf16_bits_from_f32(rng.standard_normal((3, d)).astype(np.float32))
    perm = rng.permutation(d)[:r_]
    A = np.zeros((r_, d), np.float32)
    A[np.arange(r_), perm] = 1.0
    pi = rng.integers(0, r_, size=d_i)
    B = np.zeros((d_i, r_), np.float32)
    B[np.arange(d_i), pi] = 1.0
    bias = rng.standard_normal(d_i).astype(np.float32)
    z, p = o.predictor_logits(x, A, B, bias)
    np.testing.assert_array_equal(z, o.widen(x)[:, perm])
    np.testing.assert_array_equal(p, (o.widen(x)[:, perm][:, pi] + bias).astype(np.float32))


def test_bf16_layer_rounds_z():
    layer = wl.make_layer(wl.LayerShape(d=512, d_i=256, rank=64), seed=2)
    x = wl.make_tokens(layer.shape, 4, seed=2)
    z, _ = o.predictor_logits(x, layer.A, layer.B)
    np.testing.assert_array_equal(o.round_to_bf16(z), z)
    z_raw, _ = o.predictor_logits(x, layer.A, layer.B, round_z_bf16=False)
    assert (z_raw != z).mean() > 0.9


def _textbook_swiglu(x, W_g, W_u, W_d):
    X = torch.from_numpy(o.widen(x))
    G = torch.from_numpy(o.widen(W_g))
    U = torch.from_numpy(o.widen(W_u))
    D = torch.from_numpy(o.widen(W_d))
    g = X @ G.T
    return (torch.nn.functional.silu(g) * (X @ U.T)) @ D.T, g


@pytest.fixture(scope="module")
def tiny():
    layer = wl.make_layer(wl.TINY, seed=0)
    x = wl.make_tokens(wl.TINY, 8, seed=0)
    return layer, x


def test_dense_special_case_is_textbook_swiglu(tiny):
    layer, x = tiny
    L = layer
    want, g = _textbook_swiglu(x, L.W_g, L.W_u, L.W_d)
    r = o.forward(x, L.A, L.B, L.W_g, L.W_u, L.W_d, keep=64, gate="silu")
    assert r["mask"].all()
    np.testing.assert_allclose(r["y"], want.numpy(), rtol=1e-12, atol=1e-12)
    # pred gate with the logits replaced by u is the same dense SwiGLU
    ones = np.ones((x.shape[0], L.shape.d_i), bool)
    y2, _ = o.sparse_swiglu(x, L.W_g, L.W_u, L.W_d, g.numpy(), ones, gate="pred")
    np.testing.assert_allclose(y2, want.numpy(), rtol=1e-12, atol=1e-12)


def test_exactly_zero_and_poisoned_skipped_weights(tiny):
    layer, x = tiny
    L = layer
    r = o.forward(x, L.A, L.B, L.W_g, L.W_u, L.W_d)
    m = r["mask"]
    assert (m.reshape(8, -1, 64).sum(-1) == 16).all()
    assert (r["h"][~m] == 0).all() and not np.signbit(r["h"][~m]).any()
    dead = ~m.any(axis=0)                  # channels no token keeps
    assert dead.sum() > 0
    Wg, Wu, Wd = L.W_g.copy(), L.W_u.copy(), L.W_d.copy()
    Wg[dead] = np.nan
    Wu[dead] = np.inf
    Wd[:, dead] = np.nan
    r2 = o.forward(x, L.A, L.B, Wg, Wu, Wd)
    np.testing.assert_array_equal(r2["y"], r["y"])
    assert np.isfinite(r2["y"]).all()
    # per token: poison everything that token does not keep
    for t in (0, 5):
        Wg, Wu, Wd = L.W_g.copy(), L.W_u.copy(), L.W_d.copy()
        Wg[~m[t]] = np.nan
        Wu[~m[t]] = np.nan
        Wd[:, ~m[t]] = np.nan
        r3 = o.forward(x, L.A, L.B, Wg, Wu, Wd, tokens=[t])
        np.testing.assert_array_equal(r3["y"][0], r["y"][t])


def test_mask_depends_only_on_predictor_inputs(tiny):
    layer, x = tiny
    L = layer
    other = wl.make_layer(wl.TINY, seed=9)
    r1 = o.forward(x, L.A, L.B, L.W_g, L.W_u, L.W_d)
    r2 = o.forward(x, L.A, L.B, other.W_g, other.W_u, other.W_d)
    np.testing.assert_array_equal(r1["words"], r2["words"])
    r3 = o.forward(x, other.A, L.B, L.W_g, L.W_u, L.W_d)
    assert (r3["words"] != r1["words"]).any()


def test_power_of_two_scaling_is_exact(tiny):
    layer, x = tiny
    L = layer
    y = o.forward(x, L.A, L.B, L.W_g, L.W_u, L.W_d)["y"]
    y_u = o.forward(x, L.A, L.B, L.W_g, 2 * L.W_u, L.W_d)["y"]
    y_d = o.forward(x, L.A, L.B, L.W_g, L.W_u, 0.5 * L.W_d)["y"]
    y_g = o.forward(x, L.A, L.B, 4 * L.W_g, L.W_u, L.W_d)["y"]
    np.testing.assert_array_equal(y_u, 2 * y)
    np.testing.assert_array_equal(y_d, 0.5 * y)
    np.testing.assert_array_equal(y_g, 4 * y)       # pred gate: linear in u


def test_additive_over_banks(tiny):
    layer, x = tiny
    L = layer
    r = o.forward(x, L.A, L.B, L.W_g, L.W_u, L.W_d)
    m = r["mask"]
    total = np.zeros_like(r["y"])
    for b in range(L.shape.n_banks):
        mb = np.zeros_like(m)
        mb[:, 64 * b:64 * b + 64] = m[:, 64 * b:64 * b + 64]
        yb, _ = o.sparse_swiglu(x, L.W_g, L.W_u, L.W_d, r["p"], mb)
        total += yb
    np.testing.assert_allclose(total, r["y"], rtol=1e-12, atol=1e-12)


def test_mask_pinned_mode_and_token_subset(tiny):
    layer, x = tiny
    L = layer
    r = o.forward(x, L.A, L.B, L.W_g, L.W_u, L.W_d)
    words = r["words"].copy()
    words[2, 3] ^= np.uint64(0b11)            # flip two channels of one bank
    rp = o.forward(x, L.A, L.B, L.W_g, L.W_u, L.W_d, mask_in=words)
    np.testing.assert_array_equal(rp["words"], words)
    same = [t for t in range(8) if t != 2]
    np.testing.assert_array_equal(rp["y"][same], r["y"][same])
    assert (rp["y"][2] != r["y"][2]).any()
    rs = o.forward(x, L.A, L.B, L.W_g, L.W_u, L.W_d, tokens=[6, 1])
    np.testing.assert_array_equal(rs["y"], r["y"][[6, 1]])
