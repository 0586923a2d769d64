"""Pins for the oracle's bank-wise hard top-k.

Rule: "Continual LLM Upcycling", gist.science technical summary,
Methodologie > 1. Architectuur -- banks of 64 channels, a hard top-k with
k = 16 per bank, a hard binary mask. Tie, signed-zero and NaN handling are
readings (larger first, -0 == +0, NaN last, lower index first on ties).
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle as o
import workloads as wl


def _order_key(v, i):
    # independent statement of the ranking order as a sortable tuple
    if math.isnan(v):
        return (1, 0.0, i)
    return (0, -(v + 0.0), i)   # v + 0.0 turns -0.0 into +0.0


def _brute_force_subset(vals, keep):
    """The unique subset of size keep whose every member precedes every
    non-member. Enumerates all C(n, keep) subsets."""
    n = len(vals)
    keys = [_order_key(v, i) for i, v in enumerate(vals)]
    hits = []
    for S in itertools.combinations(range(n), keep):
        rest = [j for j in range(n) if j not in S]
        if all(keys[a] < keys[b] for a in S for b in rest):
            hits.append(S)
    assert len(hits) == 1, "the ranking order must single out one subset"
    return set(hits[0])


def _load_cases(golden_dir):
    cases = []
    with open(os.path.join(golden_dir, "topk_bank8_cases.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            vals, keep, want = [s.strip() for s in line.split("|")]
            cases.append(([float(v) for v in vals.split(",")], int(keep), int(want, 16)))
    return cases


def test_golden_bank8_cases(golden_dir):
    cases = _load_cases(golden_dir)
    assert len(cases) >= 10
    for vals, keep, want in cases:
        p = np.array([vals], dtype=np.float32)
        m = o.bank_topk_mask(p, bank=8, keep=keep)
        w = int(o.mask_to_words(m, bank=8)[0, 0])
        assert w == want, f"{vals} keep={keep}: got {w:#x}, want {want:#x}"


def test_brute_force_bank8_all_keeps():
    rng = np.random.default_rng(7)
    pool = [-2.0, -1.0, -0.0, 0.0, 1.0, 2.0, math.inf, -math.inf, math.nan]
    for _ in range(150):
        vals = [pool[k] for k in rng.integers(0, len(pool), size=8)]
        p = np.array([vals], dtype=np.float32)
        for keep in range(1, 9):
            m = o.bank_topk_mask(p, bank=8, keep=keep)[0]
            assert set(np.flatnonzero(m)) == _brute_force_subset(vals, keep)


def test_matches_stable_sort_definition():
    # second, independent definition: stable sort by (NaN last, -value, index)
    p = wl.make_stress_logits(T=48, d_i=64 * 12, seed=3)
    p[5, :64] = np.float32(-0.0)
    p[6, 64:80] = np.nan
    T, d_i = p.shape
    keep = 16
    m = o.bank_topk_mask(p, 64, keep)
    for t in range(T):
        for b in range(d_i // 64):
            v = p[t, 64 * b:64 * b + 64].astype(np.float64)
            nan = np.isnan(v)
            canon = np.where(nan, 0.0, v + 0.0)
            order = np.lexsort((np.arange(64), -canon, nan))
            want = np.zeros(64, bool)
            want[order[:keep]] = True
            np.testing.assert_array_equal(m[t, 64 * b:64 * b + 64], want)


def test_exactly_keep_per_bank_and_threshold_property():
    for p in (wl.make_stress_logits(T=64, d_i=14336 // 8, seed=1),
              wl.make_tie_logits(T=64, d_i=1024, seed=2)):
        for keep in (1, 16, 63, 64):
            m = o.bank_topk_mask(p, 64, keep)
            cnt = m.reshape(p.shape[0], -1, 64).sum(-1)
            assert (cnt == keep).all()
            # every kept value >= every dropped value of the same bank
            v = p.reshape(p.shape[0], -1, 64).astype(np.float64)
            mm = m.reshape(v.shape)
            kmin = np.where(mm, v, np.inf).min(-1)
            dmax = np.where(~mm, v, -np.inf).max(-1)
            assert (kmin >= dmax).all()


def test_special_cases_bank64():
    keep = 16
    eq = np.full((1, 64), 0.5, np.float32)
    assert int(o.mask_to_words(o.bank_topk_mask(eq, 64, keep))[0, 0]) == (1 << 16) - 1
    inc = np.arange(64, dtype=np.float32)[None]
    assert int(o.mask_to_words(o.bank_topk_mask(inc, 64, keep))[0, 0]) == ((1 << 64) - 1) ^ ((1 << 48) - 1)
    allk = o.bank_topk_mask(np.random.default_rng(0).standard_normal((3, 128)).astype(np.float32), 64, 64)
    assert allk.all()
    zeros = np.where(np.arange(64) % 2 == 0, 0.0, -0.0).astype(np.float32)[None]
    assert int(o.mask_to_words(o.bank_topk_mask(zeros, 64, 3))[0, 0]) == 0b111


def test_word_packing_bit_order():
    m = np.zeros((2, 128), bool)
    m[0, 0] = m[0, 63] = m[0, 64] = m[1, 127] = True
    w = o.mask_to_words(m, 64)
    assert w.dtype == np.uint64
    assert int(w[0, 0]) == 1 | (1 << 63)
    assert int(w[0, 1]) == 1
    assert int(w[1, 1]) == 1 << 63 and int(w[1, 0]) == 0
    np.testing.assert_array_equal(o.words_to_mask(w, 64), m)


def test_invalid_arguments():
    p = np.zeros((1, 128), np.float32)
    with pytest.raises(ValueError):
        o.bank_topk_mask(p, 64, 0)
    with pytest.raises(ValueError):
        o.bank_topk_mask(p, 64, 65)
    with pytest.raises(ValueError):
        o.bank_topk_mask(p, 48, 16)


def test_logit_gap_closed_form():
    v = np.arange(64, dtype=np.float32)[::-1].copy()
    v[16] = v[15] - 0.25       # 16th largest 48, 17th largest 47.75
    g = o.logit_gap(v[None], 64, 16)
    assert g.shape == (1, 1) and g[0, 0] == 0.25
