"""Pins of the oracle's backward pass.

* torch autograd (float64) of an explicit straight-through formulation of
  the stated reading (forward value: the hard mask and bf16 z; gradient: the
  surrogate sigmoid((p - theta) / tau) and an unrounded z) gives the same
  gradients as the oracle's hand-written chain rule: a dropped term, a wrong
  sign or a transposed operand in one of them shows up here;
* central finite differences of the forward (a different code path) fix the
  gradients of every weight the mask does not depend on, and, with the
  surrogate switched off (tau = inf), every gradient;
* keep = bank has no threshold and no surrogate term.
"""
import numpy as np
import pytest
import torch

import oracle as o


def _layer(seed, d=24, d_i=64, r=8, bias=True):
    rng = np.random.default_rng(seed)
    f = lambda *s, fan: (rng.standard_normal(s) / np.sqrt(fan)).astype(np.float32)
    L = dict(A=f(r, d, fan=d), B=f(d_i, r, fan=r), W_g=f(d_i, d, fan=d), W_u=f(d_i, d, fan=d),
             W_d=f(d, d_i, fan=d_i), bias=(0.3 * rng.standard_normal(d_i)).astype(np.float32) if bias else None)
    return L, rng


def _autograd(L, x, G, bank, keep, gate, tau, round_z):
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    X, A, B, Wg, Wu, Wd = (t(x), t(L["A"]), t(L["B"]), t(L["W_g"]), t(L["W_u"]), t(L["W_d"]))
    b = t(L["bias"]) if L["bias"] is not None else None
    z = X @ A.T
    if round_z:
        zr = torch.from_numpy(o.round_to_bf16(z.detach().numpy()))
        z = z + (zr - z).detach()
    p = z @ B.T + (b if b is not None else 0.0)
    p32 = p.detach().numpy().astype(np.float32)
    m_hard = torch.from_numpy(o.bank_topk_mask(p32, bank, keep).astype(np.float64))
    if keep < bank:
        theta = torch.from_numpy(np.repeat(o.bank_threshold(p32, bank, keep), bank, axis=1))
        ms = torch.sigmoid((p - theta) / tau)
        m = m_hard + ms - ms.detach()
    else:
        m = m_hard
    U, V = X @ Wg.T, X @ Wu.T
    s = torch.sigmoid(p) if gate == "pred" else torch.sigmoid(U)
    y = (m * s * U * V) @ Wd.T
    (y * torch.from_numpy(G)).sum().backward()
    leaves = dict(g_x=X, g_A=A, g_B=B, g_Wg=Wg, g_Wu=Wu, g_Wd=Wd)
    if b is not None:
        leaves["g_bias"] = b
    # no path from a leaf to y (silu gate, full bank: the predictor) -> 0
    return {k: (v.grad.numpy() if v.grad is not None else np.zeros(tuple(v.shape)))
            for k, v in leaves.items()}


@pytest.mark.parametrize("gate", ["pred", "silu"])
@pytest.mark.parametrize("round_z", [False, True])
@pytest.mark.parametrize("keep,tau", [(4, 0.5), (8, 2.0), (16, 1.0)])
def test_matches_autograd_of_straight_through_form(gate, round_z, keep, tau):
    L, rng = _layer(10 + keep)
    x = rng.standard_normal((5, 24)).astype(np.float32)
    G = rng.standard_normal((5, 24))
    r = o.backward(x, L["A"], L["B"], L["W_g"], L["W_u"], L["W_d"], G, bias=L["bias"], bank=16,
                   keep=keep, gate=gate, tau=tau, round_z_bf16=round_z)
    ref = _autograd(L, x, G, 16, keep, gate, tau, round_z)
    for k, v in ref.items():
        np.testing.assert_allclose(r[k], v, rtol=1e-6, atol=1e-7 * max(1.0, np.abs(v).max()), err_msg=k)
    if keep == 16:
        return                      # a full bank: no threshold, no surrogate term
    # the surrogate term is really there: the predictor's gradient differs
    # from the hard-mask derivative
    r_off = o.backward(x, L["A"], L["B"], L["W_g"], L["W_u"], L["W_d"], G, bias=L["bias"], bank=16,
                       keep=keep, gate=gate, tau=np.inf, round_z_bf16=round_z)
    assert np.abs(r["g_A"] - r_off["g_A"]).max() > 1e-6


def _loss(L, x, G, bank, keep, gate, **over):
    W = dict(L, **over)
    f = o.forward(x, W["A"], W["B"], W["W_g"], W["W_u"], W["W_d"], bias=W["bias"], bank=bank, keep=keep,
                  gate=gate, round_z_bf16=False)
    return float((f["y"] * G).sum()), f["words"]


def _fd(L, x, G, bank, keep, gate, name, idx, eps):
    base = L[name] if name != "x" else x
    plus, minus = base.astype(np.float64).copy(), base.astype(np.float64).copy()
    plus[idx] += eps
    minus[idx] -= eps
    if name == "x":
        lp, wp = _loss(L, plus, G, bank, keep, gate)
        lm, wm = _loss(L, minus, G, bank, keep, gate)
    else:
        lp, wp = _loss(L, x, G, bank, keep, gate, **{name: plus})
        lm, wm = _loss(L, x, G, bank, keep, gate, **{name: minus})
    _, w0 = _loss(L, x, G, bank, keep, gate)
    assert (wp == w0).all() and (wm == w0).all(), "mask moved under the perturbation"
    return (lp - lm) / (2 * eps)


KEYS = {"W_g": "g_Wg", "W_u": "g_Wu", "W_d": "g_Wd", "A": "g_A", "B": "g_B", "bias": "g_bias", "x": "g_x"}


@pytest.mark.parametrize("gate", ["pred", "silu"])
def test_weight_gradients_against_finite_differences(gate):
    """W_g, W_u and W_d do not enter the mask: their gradients are the true
    derivatives of the forward, surrogate or not."""
    L, rng = _layer(3)
    x = rng.standard_normal((4, 24)).astype(np.float32)
    G = rng.standard_normal((4, 24))
    r = o.backward(x, L["A"], L["B"], L["W_g"], L["W_u"], L["W_d"], G, bias=L["bias"], bank=16, keep=4,
                   gate=gate, tau=0.7, round_z_bf16=False)
    for name in ("W_g", "W_u", "W_d"):
        for idx in [tuple(rng.integers(0, n) for n in L[name].shape) for _ in range(6)]:
            fd = _fd(L, x, G, 16, 4, gate, name, idx, 1e-3)
            assert abs(r[KEYS[name]][idx] - fd) <= 1e-4 * max(1.0, abs(fd)), (name, idx)


@pytest.mark.parametrize("gate", ["pred", "silu"])
@pytest.mark.parametrize("keep", [4, 16])
def test_all_gradients_without_surrogate_against_finite_differences(gate, keep):
    """With tau = inf (no surrogate), and at keep = bank (no threshold),
    every gradient is the derivative of the forward where the mask is
    locally constant."""
    L, rng = _layer(5)
    x = rng.standard_normal((4, 24)).astype(np.float32)
    G = rng.standard_normal((4, 24))
    tau = np.inf if keep < 16 else 1.0
    r = o.backward(x, L["A"], L["B"], L["W_g"], L["W_u"], L["W_d"], G, bias=L["bias"], bank=16, keep=keep,
                   gate=gate, tau=tau, round_z_bf16=False)
    for name in ("x", "A", "B", "bias"):
        shape = x.shape if name == "x" else L[name].shape
        for idx in [tuple(rng.integers(0, n) for n in shape) for _ in range(5)]:
            fd = _fd(L, x, G, 16, keep, gate, name, idx, 1e-3)
            assert abs(r[KEYS[name]][idx] - fd) <= 1e-4 * max(1.0, abs(fd)), (name, idx)


def test_threshold_and_full_bank():
    p = np.array([[3, 1, 2, 0, -1, 5, 4, -2]], dtype=np.float32)
    # bank of 8, keep 3: sorted 5, 4, 3 | 2 ... -> midpoint of 3 and 2
    assert o.bank_threshold(p, 8, 3)[0, 0] == 2.5
    assert np.isnan(o.bank_threshold(p, 8, 8)).all()
    q = p.copy()
    q[0, 5] = np.nan                     # NaN ranks last: 4, 3, 2 | 1
    assert o.bank_threshold(q, 8, 3)[0, 0] == 1.5


@pytest.mark.parametrize("gate", ["pred", "silu"])
def test_mask_in_with_own_mask_is_identical(gate):
    """Given its own mask, the backward's min-kept / max-dropped threshold
    equals the sorted keep-th / (keep+1)-th midpoint, and every gradient
    is unchanged."""
    L, rng = _layer(8)
    x = rng.standard_normal((6, 24)).astype(np.float32)
    G = rng.standard_normal((6, 24))
    args = (x, L["A"], L["B"], L["W_g"], L["W_u"], L["W_d"], G)
    kw = dict(bias=L["bias"], bank=16, keep=5, gate=gate, tau=0.8, round_z_bf16=False)
    r = o.backward(*args, **kw)
    rp = o.backward(*args, mask_in=o.mask_to_words(r["mask"], 16), **kw)
    np.testing.assert_array_equal(rp["theta"], r["theta"])
    for k in ("g_x", "g_A", "g_B", "g_bias", "g_Wg", "g_Wu", "g_Wd"):
        np.testing.assert_array_equal(rp[k], r[k])
