"""CPU oracle for the predictor-gated bank-wise sparse SwiGLU FFN forward.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module. The
product (the HIP library and its Python binding) never calls it and shares no
code with it: it has its own bf16 rounding, its own sigmoid and its own top-k.

What it computes follows "Continual LLM Upcycling: A Predictor-Gated Bank-Wise
Sparsity Training Recipe for Dense-to-Sparse LLMs":

* the abstract (catalyzex and searcharxiv author pages): per token and layer a
  low-rank predictor produces FFN-channel routing logits, and a bank-wise
  top-k keeps 16 channels in every 64-channel bank (4x sparsity);
* gist.science technical summary, Methodologie > 1. Architectuur: the
  predictor is a two-layer map R^d -> R^448 -> R^{d_i} applied to the token's
  hidden state before the FFN; its routing signal replaces the dense SwiGLU
  gate sigma(u); d_i = 14336 is split into fixed banks of 64 with a hard top-k
  (k = 16) per bank, d_s = 3584; in the forward pass a hard binary mask is
  applied and inactive channels are exactly zero;
* same summary, 2. Trainingsrecept, stage 4: the main gate is routed through
  the predictor with a sigmoid;
* same summary, 3. Hardware Implicaties: inactive channels may skip all three
  projections (gate, up, down).

Readings where the pages are silent:

* predictor: linear low-rank factorisation p = (x A^T) B^T (+ bias), no
  nonlinearity between the two layers;
* precision: every dot product is evaluated in float64; the predictor's hidden
  z is rounded to bf16 (round to nearest even) when the layer is bf16, as a
  bf16 layer stores it; the logits p are rounded to fp32, the precision the
  top-k decision is taken in;
* ranking: signed logits, largest first; -0 equals +0; NaN ranks below -inf;
  equal values are ordered by the lower channel index;
* banks are contiguous: channel j lies in bank floor(j / bank);
* gate: h_j = m_j * sigma(p_j) * u_j * v_j ("pred"), or the plain SwiGLU gate
  h_j = m_j * sigma(u_j) * u_j * v_j ("silu");
* y is returned in float64; callers compare the GPU's y after widening.

The backward pass follows the same summary's Executie > Backward Pass: the
non-differentiable top-k is crossed by a soft, sigmoid-like local gradient
around the selection threshold, so the language-modelling loss reaches the
predictor. Its form is not given; the reading taken here: the forward keeps
the hard mask m; the backward differentiates
m as if it were sigmoid((p - theta) / tau), with theta the midpoint of the
bank's keep-th and (keep+1)-th largest logits (held constant) and tau > 0 the
caller's temperature; the mask's gradient g_h * s * u * v is taken for every
channel (so gate and up are evaluated densely, as the authors' GPU runs do);
the bf16 rounding of z passes gradients unchanged; with keep == bank there
is no threshold and no surrogate term.

It also computes the Dense-4x baseline the pages compare against (same
summary, Resultaten: naive 4x sparsity applied post hoc from activation
amplitude): gate and up run dense, the per-bank top-k ranks the amplitude
|SiLU(u) * v| of every channel (rounded to fp32, the precision the decision is
taken in), and only the kept channels enter the down projection.

Every function here is pinned by a CPU test (tests/test_oracle_*.py) against
closed forms, hand-worked examples, brute force or library routines.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

__all__ = [
    "widen", "round_to_bf16", "bf16_bits_of", "sigmoid", "predictor_logits",
    "bank_topk_mask", "mask_to_words", "words_to_mask", "sparse_swiglu",
    "forward", "logit_gap", "amplitude_forward", "bank_threshold", "backward",
]


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------

def widen(a: np.ndarray) -> np.ndarray:
    """Exact float64 values of an input array.

    uint16 arrays hold bf16 bit patterns: the value is the fp32 whose upper
    16 bits are the pattern and whose lower 16 bits are zero.
    """
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits and the fp32 exponent range. Written from
    that definition: for |a| = m * 2^e with m in [0.5, 1) the spacing of bf16
    values is 2^(e-8), except below the smallest normal (2^-126) where it is
    fixed at 2^-133. numpy's rint rounds halves to even. Results of magnitude
    2^128 or more are infinite. NaN stays NaN, the sign of zero is kept.
    """
    a = np.asarray(a, dtype=np.float64)
    out = np.array(a, copy=True)
    fin = np.isfinite(a) & (a != 0)
    v = a[fin]
    _, e = np.frexp(v)
    e = np.maximum(e, -125)                       # fixed spacing below 2^-126
    q = np.rint(np.ldexp(v, 8 - e))               # exact power-of-two scaling
    r = np.ldexp(q, e - 8)
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, v), r)
    r = np.where(r == 0, np.copysign(0.0, v), r)  # keep the sign of zero
    out[fin] = r
    return out


def bf16_bits_of(a: np.ndarray) -> np.ndarray:
    """Bit patterns of bf16-representable float64 values (after round_to_bf16)."""
    a = np.asarray(a, dtype=np.float64)
    f = a.astype(np.float32)                      # exact for bf16 values
    bits = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[np.isnan(a)] = np.uint16(0x7FC0)
    return bits


def sigmoid(a: np.ndarray) -> np.ndarray:
    """Logistic function 1 / (1 + e^-a) in float64 (0 at -inf, 1 at +inf)."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


# ----------------------------------------------------------------------------
# predictor (Methodologie > 1. Architectuur: R^d -> R^448 -> R^{d_i})
# ----------------------------------------------------------------------------

def predictor_logits(x, A, B, bias=None, round_z_bf16: bool = True):
    """Routing logits of the low-rank predictor.

    z[t, q] = sum_i x[t, i] * A[q, i]          (float64, then bf16 if asked)
    p[t, j] = sum_q z[t, q] * B[j, q] + bias[j]  (float64, then fp32)

    Returns (z, p): z float64 (bf16 values when rounded), p float32.
    """
    xf, Af, Bf = widen(x), widen(A), widen(B)
    z = xf @ Af.T
    if round_z_bf16:
        z = round_to_bf16(z)
    p = z @ Bf.T
    if bias is not None:
        p = p + widen(bias)[None, :]
    return z, p.astype(np.float32)


# ----------------------------------------------------------------------------
# bank-wise hard top-k (Methodologie > 1. Architectuur: banks of 64, k = 16)
# ----------------------------------------------------------------------------

def _beats(v: np.ndarray) -> np.ndarray:
    """beats[..., a, b] is True when channel a precedes channel b in the
    ranking order of one bank: larger value first, -0 == +0, NaN after every
    number, equal values by lower index."""
    with np.errstate(invalid="ignore"):        # signaling NaNs widen to NaN
        v = np.asarray(v, dtype=np.float64)
    nan = np.isnan(v)
    v = np.where(v == 0.0, 0.0, v)
    n = v.shape[-1]
    idx = np.arange(n)
    lower = idx[:, None] < idx[None, :]
    va, vb = v[..., :, None], v[..., None, :]
    na, nb = nan[..., :, None], nan[..., None, :]
    with np.errstate(invalid="ignore"):
        both_num = ~na & ~nb
        return ((~na & nb)
                | (both_num & ((va > vb) | ((va == vb) & lower)))
                | (na & nb & lower))


def bank_topk_mask(p: np.ndarray, bank: int = 64, keep: int = 16,
                   token_chunk: int = 64) -> np.ndarray:
    """Hard bank-wise top-k: bool mask [T, d_i], exactly ``keep`` per bank.

    Channel j of bank beta (channels beta*bank .. beta*bank + bank - 1) is kept
    when fewer than ``keep`` channels of its bank precede it in the ranking
    order, i.e. rank(j) = #{i in bank : i precedes j} < keep.
    """
    p = np.asarray(p)
    T, d_i = p.shape
    if bank < 1 or d_i % bank != 0:
        raise ValueError("bank must divide d_i")
    if not 1 <= keep <= bank:
        raise ValueError("keep must lie in [1, bank]")
    nb = d_i // bank
    out = np.empty((T, d_i), dtype=bool)
    for t0 in range(0, T, token_chunk):
        v = p[t0:t0 + token_chunk].reshape(-1, nb, bank)
        rank = _beats(v).sum(axis=-2)          # rank[b] = #{a : a precedes b}
        out[t0:t0 + token_chunk] = (rank < keep).reshape(-1, d_i)
    return out


def mask_to_words(m: np.ndarray, bank: int = 64) -> np.ndarray:
    """Pack a bool mask [T, d_i] into one uint64 word per (token, bank):
    bit i of word (t, beta) is channel beta*bank + i."""
    T, d_i = m.shape
    nb = d_i // bank
    bits = m.reshape(T, nb, bank).astype(np.uint64)
    weights = np.left_shift(np.uint64(1), np.arange(bank, dtype=np.uint64))
    return (bits * weights).sum(axis=-1, dtype=np.uint64)


def words_to_mask(w: np.ndarray, bank: int = 64) -> np.ndarray:
    """Inverse of mask_to_words."""
    w = np.asarray(w).astype(np.uint64)
    T, nb = w.shape
    sh = np.arange(bank, dtype=np.uint64)
    bits = (w[..., None] >> sh) & np.uint64(1)
    return bits.astype(bool).reshape(T, nb * bank)


# ----------------------------------------------------------------------------
# masked SwiGLU on kept channels (Architectuur: routing replaces sigma(u);
# Executie: inactive channels exactly zero; Hardware Implicaties: gate, up and
# down are skipped for inactive channels)
# ----------------------------------------------------------------------------

def sparse_swiglu(x, W_g, W_u, W_d, p, m, gate: str = "pred",
                  tokens: Optional[Sequence[int]] = None):
    """y[t] = sum over kept j of h[t, j] * W_d[:, j], with
    u = x[t] . W_g[j], v = x[t] . W_u[j], h = s * u * v and
    s = sigma(p[t, j]) ("pred") or sigma(u) ("silu").

    Only the rows of W_g and W_u and the columns of W_d of kept channels are
    read. Returns (y [n, d] float64, h [n, d_i] float64 with exact zeros off
    the mask) for the selected token rows.
    """
    if gate not in ("pred", "silu"):
        raise ValueError("gate must be 'pred' or 'silu'")
    xs = np.asarray(x)
    rows = range(xs.shape[0]) if tokens is None else list(tokens)
    d = xs.shape[1]
    d_i = np.asarray(W_g).shape[0]
    y = np.zeros((len(rows), d), dtype=np.float64)
    h = np.zeros((len(rows), d_i), dtype=np.float64)
    for n, t in enumerate(rows):
        S = np.flatnonzero(m[t])
        xt = widen(xs[t])
        u = widen(W_g[S]) @ xt
        v = widen(W_u[S]) @ xt
        s = sigmoid(widen(p[t, S])) if gate == "pred" else sigmoid(u)
        hs = s * u * v
        h[n, S] = hs
        y[n] = widen(W_d[:, S]) @ hs
    return y, h


def forward(x, A, B, W_g, W_u, W_d, bias=None, bank: int = 64, keep: int = 16,
            gate: str = "pred", round_z_bf16: Optional[bool] = None,
            mask_in: Optional[np.ndarray] = None,
            tokens: Optional[Sequence[int]] = None) -> dict:
    """The whole forward of one layer for the selected tokens.

    round_z_bf16 defaults to True when x holds bf16 bit patterns.
    ``mask_in`` (uint64 words [T, d_i / 64]) skips the predictor and top-k
    and uses the given mask (mask-pinned mode); the logits are still
    computed, since the "pred" gate needs them.
    """
    x = np.asarray(x)
    rows = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    if round_z_bf16 is None:
        round_z_bf16 = x.dtype == np.uint16
    z, p = predictor_logits(x[rows], A, B, bias, round_z_bf16)
    if mask_in is None:
        m = bank_topk_mask(p, bank, keep)
    else:
        m = words_to_mask(np.asarray(mask_in)[rows], bank)
    y, h = sparse_swiglu(x[rows], W_g, W_u, W_d, p, m, gate)
    return dict(z=z, p=p, mask=m, words=mask_to_words(m, bank), h=h, y=y, tokens=rows)


def logit_gap(p: np.ndarray, bank: int = 64, keep: int = 16) -> np.ndarray:
    """Per (token, bank): the keep-th largest logit minus the (keep+1)-th
    largest (0 when keep == bank). Small gaps mark banks whose selection can
    legitimately change under a different summation order."""
    T, d_i = p.shape
    v = np.sort(np.asarray(p, dtype=np.float64).reshape(T, d_i // bank, bank), axis=-1)[..., ::-1]
    if keep >= bank:
        return np.zeros(v.shape[:2])
    return v[..., keep - 1] - v[..., keep]


# ----------------------------------------------------------------------------
# Dense-4x baseline (Resultaten: naive post-hoc 4x sparsity from activation
# amplitude; no predictor)
# ----------------------------------------------------------------------------

def amplitude_forward(x, W_g, W_u, W_d, bank: int = 64, keep: int = 16,
                      mask_in: Optional[np.ndarray] = None,
                      tokens: Optional[Sequence[int]] = None) -> dict:
    """Post-hoc amplitude sparsity for the selected tokens: u = x W_g^T and
    v = x W_u^T over every channel, a = sigma(u) * u * v, the bank top-k of
    |fp32(a)| gives the mask, h = a on kept channels (0 elsewhere) and y sums
    h[j] * W_d[:, j] over the kept channels only.

    ``mask_in`` (uint64 words) replaces the amplitude top-k (mask-pinned
    mode). Returns the amplitudes ``a`` (float64, fp32-rounded), ``score`` =
    |a| as ranked, the mask, its words, h and y.
    """
    xs = np.asarray(x)
    rows = np.arange(xs.shape[0]) if tokens is None else np.asarray(tokens)
    X = widen(xs[rows])
    u = X @ widen(W_g).T
    v = X @ widen(W_u).T
    a = (sigmoid(u) * u * v).astype(np.float32).astype(np.float64)
    score = np.abs(a)
    if mask_in is None:
        m = bank_topk_mask(score, bank, keep)
    else:
        m = words_to_mask(np.asarray(mask_in)[rows], bank)
    Wd = np.asarray(W_d)
    d = Wd.shape[0]
    h = np.where(m, a, 0.0)
    y = np.zeros((len(rows), d), dtype=np.float64)
    for n in range(len(rows)):
        S = np.flatnonzero(m[n])
        y[n] = widen(Wd[:, S]) @ a[n, S]
    return dict(a=a, score=score, mask=m, words=mask_to_words(m, bank), h=h, y=y, tokens=rows)


# ----------------------------------------------------------------------------
# backward pass (Executie > Backward Pass: soft surrogate gradient around the
# bank threshold; the form is the reading stated in the module docstring)
# ----------------------------------------------------------------------------

def bank_threshold(p: np.ndarray, bank: int = 64, keep: int = 16) -> np.ndarray:
    """Per (token, bank): the midpoint of the keep-th and (keep+1)-th largest
    logits, NaN counted below every number (NaN when keep == bank)."""
    T, d_i = p.shape
    v = np.asarray(p, dtype=np.float64).reshape(T, d_i // bank, bank)
    v = np.where(np.isnan(v), -np.inf, v)
    v = -np.sort(-v, axis=-1)
    if keep >= bank:
        return np.full(v.shape[:2], np.nan)
    return 0.5 * (v[..., keep - 1] + v[..., keep])


def _dsigmoid(a: np.ndarray) -> np.ndarray:
    s = sigmoid(a)
    return s * (1.0 - s)


def backward(x, A, B, W_g, W_u, W_d, g_y, bias=None, bank: int = 64, keep: int = 16,
             gate: str = "pred", tau: float = 1.0,
             round_z_bf16: Optional[bool] = None,
             mask_in: Optional[np.ndarray] = None) -> dict:
    """Gradients of L = sum(y * g_y) for every input of the layer.

    Returns g_x [T, d], g_A [rank, d], g_B [d_i, rank], g_bias [d_i] (or
    None), g_Wg, g_Wu [d_i, d], g_Wd [d, d_i], and the intermediates g_h,
    g_p, theta and the mask, all float64. ``tau = inf`` switches the
    surrogate term off (the derivative of the hard-mask forward).
    ``mask_in`` (uint64 words) gives the forward's mask; theta is then the
    midpoint of each bank's smallest kept and largest dropped logit, which is
    the same value when the mask is the bank top-k of p.
    """
    if gate not in ("pred", "silu"):
        raise ValueError("gate must be 'pred' or 'silu'")
    x = np.asarray(x)
    if round_z_bf16 is None:
        round_z_bf16 = x.dtype == np.uint16
    X = widen(x)
    Aw, Bw, Wg, Wu, Wd = widen(A), widen(B), widen(W_g), widen(W_u), widen(W_d)
    G = widen(g_y)
    # forward, as the forward pass computes it
    z, p32 = predictor_logits(x, A, B, bias, round_z_bf16)
    if mask_in is None:
        m = bank_topk_mask(p32, bank, keep).astype(np.float64)
    else:
        m = words_to_mask(np.asarray(mask_in), bank).astype(np.float64)
    p = p32.astype(np.float64)
    U = X @ Wg.T
    V = X @ Wu.T
    s = sigmoid(p) if gate == "pred" else sigmoid(U)
    h = m * s * U * V
    # down
    g_h = G @ Wd                       # dL/dh for every channel
    g_Wd = G.T @ h
    # through h = m * s * u * v
    if gate == "pred":
        g_U = m * g_h * s * V
        g_p = m * g_h * U * V * _dsigmoid(p)
    else:
        g_U = m * g_h * V * (s + U * _dsigmoid(U))
        g_p = np.zeros_like(p)
    g_V = m * g_h * s * U
    # the surrogate gradient of the mask
    T, d_i = p.shape
    if mask_in is None:
        theta = bank_threshold(p, bank, keep)
    else:
        key = np.where(np.isnan(p), -np.inf, p).reshape(T, d_i // bank, bank)
        mb = m.reshape(T, d_i // bank, bank) > 0
        theta = 0.5 * (np.where(mb, key, np.inf).min(-1) + np.where(mb, -np.inf, key).max(-1))
    if keep < bank and np.isfinite(tau):
        th = np.repeat(theta, bank, axis=1)
        g_m = g_h * s * U * V
        g_p = g_p + g_m * _dsigmoid((p - th) / tau) / tau
    # the predictor (z's bf16 rounding passes gradients unchanged)
    g_bias = g_p.sum(axis=0) if bias is not None else None
    g_B = g_p.T @ z
    g_z = g_p @ Bw
    g_A = g_z.T @ X
    g_x = g_z @ Aw + g_U @ Wg + g_V @ Wu
    g_Wg = g_U.T @ X
    g_Wu = g_V.T @ X
    return dict(g_x=g_x, g_A=g_A, g_B=g_B, g_bias=g_bias, g_Wg=g_Wg, g_Wu=g_Wu, g_Wd=g_Wd,
                g_h=g_h, g_p=g_p, theta=theta, mask=m.astype(bool), z=z, p=p)
