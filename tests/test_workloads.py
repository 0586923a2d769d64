"""The seeded input recipe: determinism, shapes and the stated distributions."""
import numpy as np

import oracle as o
import workloads as wl


def test_deterministic_and_seed_dependent():
    a = wl.make_layer(wl.TINY, seed=0)
    b = wl.make_layer(wl.TINY, seed=0)
    c = wl.make_layer(wl.TINY, seed=1)
    for n in ("A", "B", "W_g", "W_u", "W_d"):
        np.testing.assert_array_equal(getattr(a, n), getattr(b, n))
        assert (getattr(a, n) != getattr(c, n)).mean() > 0.99
    np.testing.assert_array_equal(wl.make_tokens(wl.TINY, 8, 3), wl.make_tokens(wl.TINY, 8, 3))


def test_shapes_dtypes_and_variances():
    s = wl.LayerShape(d=1024, d_i=2048, rank=128)
    L = wl.make_layer(s, seed=0, bias_var=0.5)
    assert L.A.shape == (128, 1024) and L.B.shape == (2048, 128)
    assert L.W_g.shape == L.W_u.shape == (2048, 1024) and L.W_d.shape == (1024, 2048)
    for n, fan in (("A", 1024), ("B", 128), ("W_g", 1024), ("W_u", 1024), ("W_d", 2048)):
        w = getattr(L, n)
        assert w.dtype == np.uint16
        std = o.widen(w).std()
        assert abs(std * np.sqrt(fan) - 1) < 0.03, n
    assert abs(L.bias.var() - 0.5) < 0.05
    x = wl.make_tokens(s, 64, seed=0)
    assert x.dtype == np.uint16 and abs(o.widen(x).std() - 1) < 0.03
    t = wl.make_tokens(wl.TINY, 8, seed=0)
    assert t.dtype == np.float32 and t.shape == (8, 256)


def test_outlier_columns():
    x = o.widen(wl.make_tokens(wl.FULL, 256, seed=0, outlier_frac=0.01))
    cols = wl.outlier_columns(wl.FULL, seed=0)
    assert len(cols) == 41
    std = x.std(axis=0)
    assert (std[cols] > 15).all()
    rest = np.setdiff1d(np.arange(4096), cols)
    assert (std[rest] < 1.5).all()


def test_stress_logits_have_exact_ties_in_every_bank():
    p = wl.make_stress_logits(T=64, d_i=14336, seed=0)
    v = np.sort(p.reshape(64, 224, 64), axis=-1)
    dup = (np.diff(v, axis=-1) == 0).sum(-1)
    assert (dup >= 1).all()
    assert dup.mean() >= 2.5        # 3 copies per bank, sometimes onto each other
    np.testing.assert_array_equal(p, wl.make_stress_logits(T=64, d_i=14336, seed=0))


def test_tie_logits():
    p = wl.make_tie_logits(T=16, d_i=1024, seed=0)
    assert set(np.unique(p)) <= set(range(-4, 5))
    assert np.signbit(p[p == 0]).any()


def test_boundary_ties_straddle_the_keep_boundary():
    """The boundary variant of the stress logits: in every bank keep - 1
    values lie above the keep-th largest and 1 + 3 equal it, so the top-k must
    break a tie across the boundary (3 of the 4 tied channels dropped)."""
    for keep in (16, 5):
        p = wl.make_stress_logits(T=96, d_i=2048, seed=4, ties="boundary", keep=keep)
        v = p.reshape(96, 32, 64)
        kth = np.sort(v, axis=-1)[..., 64 - keep]
        assert ((v > kth[..., None]).sum(-1) == keep - 1).all()
        assert ((v == kth[..., None]).sum(-1) == 4).all()
        np.testing.assert_array_equal(p, wl.make_stress_logits(T=96, d_i=2048, seed=4, ties="boundary",
                                                               keep=keep))
    # the oracle keeps the lowest-index tied channel only
    p = wl.make_stress_logits(T=8, d_i=1024, seed=1, ties="boundary")
    m = o.bank_topk_mask(p, 64, 16)
    v = p.reshape(8, 16, 64)
    kth = np.sort(v, axis=-1)[..., 48]
    tied = v == kth[..., None]
    kept_tied = m.reshape(8, 16, 64) & tied
    assert (kept_tied.sum(-1) == 1).all()
    first = np.argmax(tied, axis=-1)
    assert (np.argmax(kept_tied, axis=-1) == first).all()
    # the random-copy variant is unchanged by the new option
    np.testing.assert_array_equal(wl.make_stress_logits(T=16, d_i=1024, seed=2),
                                  wl.make_stress_logits(T=16, d_i=1024, seed=2, ties="random"))
