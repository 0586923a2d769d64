"""Seeded synthetic inputs for the predictor-gated bank-wise sparse SwiGLU FFN.

This module only draws random numbers. It performs none of the layer's
arithmetic: the CPU oracle and the GPU path both consume exactly the arrays
made here, so the two sides never share code beyond these draws.

Shapes follow the layer described in "Continual LLM Upcycling: A
Predictor-Gated Bank-Wise Sparsity Training Recipe for Dense-to-Sparse LLMs"
(gist.science technical summary, Methodologie > 1. Architectuur): a predictor
d -> 448 -> d_i, d_i = 14336 split into banks of 64 with 16 kept per bank. The
hidden size d is not stated on the pages; d = 4096 is used for the full layer.

Recipe (stated once, used everywhere):

* N(mu, var) is parametrised by the variance; a weight matrix is drawn from
  N(0, 1/fan_in) with fan_in its input dimension (A: d, B: r, W_g and W_u: d,
  W_d: d_i). Token rows are N(0, 1).
* bf16 tensors are drawn in fp32 and rounded to bf16 (round to nearest even)
  by torch's CPU conversion; they are returned as uint16 bit patterns.
* One numpy PCG64 child stream per tensor, spawned from SeedSequence(seed) in
  the fixed order of ``_STREAMS``.
* Outlier tokens (prefill chunks): a seed-chosen set of round(0.01 * d)
  feature columns is multiplied by 20 before rounding, for every token.
* Routing offsets (batched decode): a per-channel predictor output bias
  b_j ~ N(0, 0.5), shared by all tokens.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

__all__ = [
    "LayerShape", "Layer", "TINY", "FULL", "make_layer", "make_tokens",
    "make_stress_logits", "make_tie_logits", "bf16_bits_from_f32",
    "widen_bf16_bits", "CONFIGS",
]

# Order in which child streams are handed out; never reorder.
_STREAMS = ("A", "B", "W_g", "W_u", "W_d", "bias", "x", "outlier_cols", "spare")


@dataclass(frozen=True)
class LayerShape:
    d: int
    d_i: int
    rank: int
    bank: int = 64
    keep: int = 16
    dtype: str = "bf16"  # "bf16" or "f32"

    @property
    def n_banks(self) -> int:
        return self.d_i // self.bank

    @property
    def d_s(self) -> int:
        return self.n_banks * self.keep


TINY = LayerShape(d=256, d_i=1024, rank=32, dtype="f32")
FULL = LayerShape(d=4096, d_i=14336, rank=448, dtype="bf16")


@dataclass
class Layer:
    """Weights in nn.Linear layout ([out, in], row-major).

    For dtype "bf16" every matrix is a uint16 array of bf16 bit patterns; for
    "f32" it is float32. ``bias`` is float32 [d_i] or None.
    """
    shape: LayerShape
    A: np.ndarray      # [rank, d]
    B: np.ndarray      # [d_i, rank]
    W_g: np.ndarray    # [d_i, d]
    W_u: np.ndarray    # [d_i, d]
    W_d: np.ndarray    # [d, d_i]
    bias: Optional[np.ndarray] = None


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 draws to bf16 with torch's CPU conversion; return the bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def widen_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact bf16 -> fp32 widening of stored bit patterns (for consumers that
    want the drawn values as float32, e.g. to upload as a fp32 tensor)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _rngs(seed: int):
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.default_rng(c) for name, c in zip(_STREAMS, children)}


def _normal(rng, shape, var):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if var != 1.0:
        a *= np.float32(np.sqrt(var))
    return a


def _cast(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_from_f32(a) if dtype == "bf16" else np.ascontiguousarray(a, np.float32)


def make_layer(shape: LayerShape, seed: int = 0, bias_var: Optional[float] = None) -> Layer:
    r = _rngs(seed)
    d, d_i, rank = shape.d, shape.d_i, shape.rank
    A = _cast(_normal(r["A"], (rank, d), 1.0 / d), shape.dtype)
    B = _cast(_normal(r["B"], (d_i, rank), 1.0 / rank), shape.dtype)
    W_g = _cast(_normal(r["W_g"], (d_i, d), 1.0 / d), shape.dtype)
    W_u = _cast(_normal(r["W_u"], (d_i, d), 1.0 / d), shape.dtype)
    W_d = _cast(_normal(r["W_d"], (d, d_i), 1.0 / d_i), shape.dtype)
    bias = None
    if bias_var is not None:
        bias = _normal(r["bias"], (d_i,), bias_var).astype(np.float32)
    return Layer(shape, A, B, W_g, W_u, W_d, bias)


def make_tokens(shape: LayerShape, T: int, seed: int = 0, outlier_frac: float = 0.0,
                outlier_scale: float = 20.0) -> np.ndarray:
    """Token rows x [T, d] ~ N(0, 1); optional outlier feature columns."""
    r = _rngs(seed)
    x = _normal(r["x"], (T, shape.d), 1.0)
    if outlier_frac > 0.0:
        n_out = int(round(outlier_frac * shape.d))
        cols = np.sort(r["outlier_cols"].choice(shape.d, size=n_out, replace=False))
        x[:, cols] *= np.float32(outlier_scale)
    return _cast(x, shape.dtype)


def outlier_columns(shape: LayerShape, seed: int = 0, outlier_frac: float = 0.01) -> np.ndarray:
    """The feature columns ``make_tokens`` scales for the same seed."""
    r = _rngs(seed)
    n_out = int(round(outlier_frac * shape.d))
    return np.sort(r["outlier_cols"].choice(shape.d, size=n_out, replace=False))


def make_stress_logits(T: int, d_i: int, seed: int = 0, bank: int = 64,
                       tie_frac: float = 0.05, ties: str = "random", keep: int = 16) -> np.ndarray:
    """fp32 logits [T, d_i] ~ N(0, 1) with exact ties injected per bank.

    ties="random": in every bank, round(tie_frac * bank) positions are
    overwritten, each with the value of a randomly chosen position of the
    same bank that is not overwritten, so every bank holds at least one exact
    tie.

    ties="boundary": in every bank, round(tie_frac * bank) positions drawn
    from those below the bank's keep-th largest value are overwritten with
    that value, so every bank holds an exact tie that straddles the keep
    boundary (keep - 1 values above it, 1 + round(tie_frac * bank) equal to
    it).
    """
    if ties not in ("random", "boundary"):
        raise ValueError("ties must be 'random' or 'boundary'")
    r = _rngs(seed)
    p = r["x"].standard_normal(size=(T, d_i), dtype=np.float32)
    n_tie = int(round(tie_frac * bank))
    if n_tie and ties == "boundary":
        nb = d_i // bank
        g = r["spare"]
        below = bank - keep                # positions under the keep-th largest value
        step = max(1, (1 << 22) // d_i)    # tokens per slice: bounded index arrays
        for t0 in range(0, T, step):
            pv = p[t0:t0 + step].reshape(-1, nb, bank)
            order = np.argpartition(pv, below, axis=-1)
            kth = np.take_along_axis(pv, order[..., below:below + 1], axis=-1)
            # n_tie distinct picks among the `below` smallest positions
            pick = g.integers(0, below, size=pv.shape[:2] + (1,))
            for k in range(1, n_tie):
                nxt = g.integers(0, below - k, size=pv.shape[:2] + (1,))
                for col in np.split(np.sort(pick, axis=-1), pick.shape[-1], axis=-1):
                    nxt += nxt >= col
                pick = np.concatenate([pick, nxt], axis=-1)
            dst = np.take_along_axis(order, pick, axis=-1)
            np.put_along_axis(pv, dst, np.broadcast_to(kth, dst.shape), axis=-1)
        return p
    if n_tie:
        nb = d_i // bank
        pv = p.reshape(T, nb, bank)
        g = r["spare"]
        def skip_taken(pick, taken):
            # map pick in [0, bank - n) to the pick-th position not in `taken`
            for col in np.split(np.sort(taken, axis=-1), taken.shape[-1], axis=-1):
                pick += pick >= col
            return pick

        # destinations: n_tie distinct positions per bank, one at a time
        dst = g.integers(0, bank, size=(T, nb, 1))
        for k in range(1, n_tie):
            dst = np.concatenate([dst, skip_taken(g.integers(0, bank - k, size=(T, nb, 1)), dst)],
                                 axis=-1)
        # sources: positions that are not destinations
        src = skip_taken(g.integers(0, bank - n_tie, size=dst.shape), dst)
        vals = np.take_along_axis(pv, src, axis=-1)
        np.put_along_axis(pv, dst, vals, axis=-1)
    return p


def make_tie_logits(T: int, d_i: int, seed: int = 0, levels: int = 9) -> np.ndarray:
    """fp32 logits drawn from a few small integers (-(levels//2) .. levels//2),
    plus a sprinkling of -0.0, so that nearly every bank has ties at every rank."""
    r = _rngs(seed)
    h = levels // 2
    p = r["x"].integers(-h, h + 1, size=(T, d_i)).astype(np.float32)
    neg0 = r["spare"].random((T, d_i)) < 0.05
    p[neg0 & (p == 0)] = np.float32(-0.0)
    return p


# The five workloads of this layer, by name.
CONFIGS = {
    "tiny": dict(shape=TINY, T=8),
    "decode": dict(shape=FULL, T=1),
    "batched": dict(shape=FULL, T=32, bias_var=0.5),
    "prefill": dict(shape=FULL, T=4096, outlier_frac=0.01),
    "longctx": dict(shape=FULL, T=32768, chunk=4096, outlier_frac=0.01),
    "topk_stress": dict(T=32768, d_i=14336, tie_frac=0.05),
    # the same with the ties planted on each bank's keep boundary
    "topk_stress_boundary": dict(T=32768, d_i=14336, tie_frac=0.05, ties="boundary"),
}
