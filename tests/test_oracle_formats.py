"""Pins for the oracle's number formats: bf16 rounding, widening, sigmoid."""
import math
import os

import numpy as np
import pytest
import torch

import oracle as o


def _load_bf16_vectors(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "bf16_rne_vectors.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            val, bits = line.split()[:2]
            rows.append((float(val), int(bits, 16)))
    return rows


def test_bf16_golden_vectors(golden_dir):
    rows = _load_bf16_vectors(golden_dir)
    assert len(rows) >= 15
    vals = np.array([r[0] for r in rows])
    want = np.array([r[1] for r in rows], dtype=np.uint16)
    got = o.bf16_bits_of(o.round_to_bf16(vals))
    for v, g, w in zip(vals, got, want):
        assert g == w, f"{v!r}: got {g:#06x}, want {w:#06x}"


def test_bf16_nan_stays_nan():
    r = o.round_to_bf16(np.array([np.nan, -np.nan]))
    assert np.isnan(r).all()


def test_bf16_matches_torch_conversion_on_fp32_inputs():
    # torch's CPU float -> bfloat16 cast is a library round-to-nearest-even
    rng = np.random.default_rng(123)
    mant = rng.standard_normal(200_000)
    expo = rng.integers(-140, 128, size=mant.shape)
    a = (mant * np.exp2(expo.astype(np.float64))).astype(np.float32)
    a = a[np.isfinite(a)]
    # plus every tie pattern: low 16 bits exactly 0x8000
    ties = (rng.integers(0, 2**16, size=5000).astype(np.uint32) << 16 | 0x8000)
    ties = ties.view(np.float32)
    ties = ties[np.isfinite(ties)]
    a = np.concatenate([a, ties])
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = o.bf16_bits_of(o.round_to_bf16(a.astype(np.float64)))
    np.testing.assert_array_equal(got, want)


def test_bf16_values_are_fixed_points():
    bits = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    vals = o.widen(bits)
    fin = np.isfinite(vals)
    r = o.round_to_bf16(vals[fin])
    np.testing.assert_array_equal(o.bf16_bits_of(r), bits[fin])


def test_widen_closed_forms():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x4049], dtype=np.uint16)
    v = o.widen(bits)
    assert v[0] == 1.0 and v[1] == -2.0
    assert v[2] == math.inf and v[3] == -math.inf
    assert v[4] == 2.0 ** -133
    assert v[5] == 0.0 and math.copysign(1.0, v[5]) == -1.0
    assert v[6] == 3.140625
    f = np.array([1.5, -0.25], dtype=np.float32)
    assert o.widen(f).dtype == np.float64 and list(o.widen(f)) == [1.5, -0.25]


def test_sigmoid_closed_forms():
    assert o.sigmoid(np.array(0.0)) == 0.5
    assert abs(o.sigmoid(np.array(math.log(3.0))) - 0.75) < 1e-15
    assert abs(o.sigmoid(np.array(-math.log(3.0))) - 0.25) < 1e-15
    a = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(o.sigmoid(-a), 1.0 - o.sigmoid(a), atol=1e-15)
    big = o.sigmoid(np.array([-np.inf, -1000.0, 1000.0, np.inf]))
    np.testing.assert_array_equal(big, [0.0, 0.0, 1.0, 1.0])
    # derivative identity s' = s (1 - s), checked by central differences
    x = np.linspace(-6, 6, 25)
    hstep = 1e-6
    num = (o.sigmoid(x + hstep) - o.sigmoid(x - hstep)) / (2 * hstep)
    s = o.sigmoid(x)
    np.testing.assert_allclose(num, s * (1 - s), rtol=0, atol=1e-9)
