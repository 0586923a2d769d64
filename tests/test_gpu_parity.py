"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars (the layer's correctness criteria):
* bank top-k masks are bit-exact when both sides get the same fp32 logits;
* end-to-end, a (token, bank) mask may differ from the oracle's only where
  the oracle's keep-th / (keep+1)-th logit gap is below 1e-3;
* y is within relative L2 2e-2 of the oracle, per token with the GPU's mask
  pinned into the oracle, and over the whole tensor end to end.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle as o
import workloads as wl
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

REL_L2 = 2e-2
GAP = 1e-3
SNAN = np.array([0x7F800001], dtype=np.uint32).view(np.float32)[0]      # signaling NaN bits
NEG_NAN = np.array([0xFFC00000], dtype=np.uint32).view(np.float32)[0]   # quiet NaN, sign set


def dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def words(t):
    return t.cpu().numpy().view(np.uint64)


def make_ffn(layer, bias=True, keep=16, gate="pred"):
    import activation_sparse_ffn_amd as sffn
    L = layer
    return sffn.SparseFFN(dev(L.W_g), dev(L.W_u), dev(L.W_d), dev(L.A), dev(L.B),
                          dev(L.bias) if (bias and L.bias is not None) else None,
                          keep=keep, gate=gate)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_forward(layer, x, y, mask, logits, tokens=None, bias=True, keep=16, gate="pred"):
    """Compare one GPU forward with the oracle on the chosen token rows."""
    L = layer
    b = L.bias if bias else None
    T = x.shape[0]
    rows = np.arange(T) if tokens is None else np.asarray(tokens)
    gw = words(mask)
    gl = host(logits)
    yg = o.widen(host(y))
    # 1. the GPU's own logits give the GPU's mask (bit-exact top-k)
    np.testing.assert_array_equal(o.mask_to_words(o.bank_topk_mask(gl[rows], 64, keep)), gw[rows])
    assert (np.bitwise_count(gw[rows]) == keep).all()
    # 2. end-to-end masks differ only where the oracle's logit gap is tiny
    r = o.forward(x, L.A, L.B, L.W_g, L.W_u, L.W_d, bias=b, keep=keep, gate=gate, tokens=rows)
    gap = o.logit_gap(r["p"], 64, keep)
    diff = gw[rows] != r["words"]
    assert (gap[diff] < GAP).all(), f"mask differs with gap {gap[diff].max()}"
    # the logits themselves agree closely (fp32 accumulation vs float64)
    scale = np.abs(r["p"]).max()
    assert np.abs(gl[rows].astype(np.float64) - r["p"]).max() <= 2e-3 * max(scale, 1.0)
    # 3. y per token with the GPU's mask pinned into the oracle
    y_pin = r["y"].copy()
    bad = np.flatnonzero(diff.any(axis=1))
    if len(bad):
        rp = o.forward(x, L.A, L.B, L.W_g, L.W_u, L.W_d, bias=b, keep=keep, gate=gate,
                       mask_in=gw, tokens=rows[bad])
        y_pin[bad] = rp["y"]
    for n, t in enumerate(rows):
        e = rel_l2(yg[t], y_pin[n])
        assert e <= REL_L2, f"token {t}: rel-L2 {e:.3e} (mask pinned)"
    # 4. end to end over the whole tensor
    assert rel_l2(yg[rows], r["y"]) <= REL_L2
    return r, int(diff.sum())


# ---------------------------------------------------------------------------
# fixtures
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def full_layer():
    return wl.make_layer(wl.FULL, seed=0, bias_var=0.5)


@pytest.fixture(scope="module")
def ffn_full(full_layer):
    return make_ffn(full_layer, bias=False)


@pytest.fixture(scope="module")
def ffn_full_bias(full_layer):
    return make_ffn(full_layer, bias=True)


MID = wl.LayerShape(d=512, d_i=2048, rank=64)


@pytest.fixture(scope="module")
def mid_layer():
    return wl.make_layer(MID, seed=4, bias_var=0.5)


# ---------------------------------------------------------------------------
# bank top-k alone
# ---------------------------------------------------------------------------

def _specials(T=6, d_i=256):
    rng = np.random.default_rng(11)
    p = rng.standard_normal((T, d_i)).astype(np.float32)
    p[0, :64] = np.nan
    p[1, :64:3] = np.inf
    p[1, 1:64:3] = -np.inf
    p[2, :64] = np.where(np.arange(64) % 2, -0.0, 0.0)
    p[3, 64:128] = 1.0
    p[4, 5:60] = np.nan
    p[5, 128:192] = np.arange(64, dtype=np.float32)[::-1]
    p[5, 192:256] = np.float32(1e-45) * (np.arange(64) % 3 - 1)   # subnormals and zeros
    p[3, 0:64:5] = SNAN                                              # signaling and negative NaNs
    p[3, 1:64:7] = NEG_NAN
    return p


@pytest.mark.parametrize("keep", [1, 7, 16, 48, 63, 64])
def test_bank_topk_bit_exact(keep):
    import activation_sparse_ffn_amd as sffn
    cases = [np.random.default_rng(1).standard_normal((37, 1024)).astype(np.float32),
             wl.make_tie_logits(T=29, d_i=2048, seed=5),
             wl.make_stress_logits(T=13, d_i=14336, seed=6),
             _specials()]
    for p in cases:
        mask, ids = sffn.bank_topk(dev(p), keep=keep, return_ids=True)
        torch.cuda.synchronize()
        m = o.bank_topk_mask(p, 64, keep)
        np.testing.assert_array_equal(words(mask), o.mask_to_words(m))
        ids_np = ids.cpu().numpy().view(np.uint16)
        for t in range(p.shape[0]):
            np.testing.assert_array_equal(ids_np[t], np.flatnonzero(m[t]))


@pytest.mark.parametrize("keep", [1, 16, 64])
def test_bank_topk_many_banks_per_wave(keep):
    """Above 65536 (token, bank) words each lane ranks one bank of a
    64-word chunk; a ragged tail (4099 x 16 words is not a multiple of 64),
    special values and ties included."""
    import activation_sparse_ffn_amd as sffn
    p = wl.make_tie_logits(T=4099, d_i=1024, seed=8)
    p[::7] = np.random.default_rng(3).standard_normal((len(p[::7]), 1024)).astype(np.float32)
    p[5, :64] = np.nan                        # a bank of NaNs only
    p[6, :50] = np.nan                        # fewer than 64 - keep numbers
    p[6, 64:128:5] = np.nan
    p[7, ::3] = np.inf
    p[8, 1::2] = -np.inf
    p[9, :64] = np.where(np.arange(64) % 2, -0.0, 0.0)
    p[10, 128:192] = np.float32(1e-45) * (np.arange(64) % 3 - 1)
    p[11, 0:64:3] = SNAN
    p[11, 1:64:5] = NEG_NAN
    p[12, 64:128] = SNAN                      # a bank of signaling NaNs only
    mask, ids = sffn.bank_topk(dev(p), keep=keep, return_ids=True)
    torch.cuda.synchronize()
    m = o.bank_topk_mask(p, 64, keep)
    np.testing.assert_array_equal(words(mask), o.mask_to_words(m))
    ids_np = ids.cpu().numpy().view(np.uint16).astype(np.int64)
    want = np.nonzero(m)[1].reshape(len(p), -1)
    np.testing.assert_array_equal(ids_np, want)


@pytest.mark.parametrize("T,keep", [(4096, 16), (16387, 16), (16387, 5)])
def test_bank_topk_persistent_chunks(T, keep):
    """The many-banks kernel at its lower size bound (4096 x 16 = 65536
    words, whole 64-word chunks) and where each wave walks several chunks
    and the last chunk is partial (16387 x 16 words = 4096 chunks + 48)."""
    import activation_sparse_ffn_amd as sffn
    p = wl.make_tie_logits(T=T, d_i=1024, seed=20 + keep)
    p[::5] = np.random.default_rng(21).standard_normal((len(p[::5]), 1024)).astype(np.float32)
    p[T - 1, 960:] = np.nan                   # the very last bank: NaNs only
    p[T - 2, 0:64:2] = -np.inf
    p[T - 3, 0:64:4] = SNAN
    mask, ids = sffn.bank_topk(dev(p), keep=keep, return_ids=True)
    torch.cuda.synchronize()
    m = o.bank_topk_mask(p, 64, keep)
    np.testing.assert_array_equal(words(mask), o.mask_to_words(m))
    ids_np = ids.cpu().numpy().view(np.uint16).astype(np.int64)
    np.testing.assert_array_equal(ids_np, np.nonzero(m)[1].reshape(len(p), -1))


def assert_topk_valid_on_gpu(mask, logits, keep=16, rows_per_pass=4096):
    """Every row of a GPU mask is THE bank top-k of its NaN-free fp32 logits,
    checked on the GPU: exactly `keep` bits per word; the smallest kept logit
    of a bank is >= its largest dropped one (IEEE compare: -0 == +0); and
    where they are equal, every kept channel holding that value has a lower
    index than every dropped one. These conditions single out the unique
    mask of the ranking (value, then lower index). Returns the number of
    banks whose keep boundary falls inside a tie."""
    T, nb = mask.shape
    assert logits.shape == (T, nb * 64)
    assert not bool(torch.isnan(logits).any()), "the check covers NaN-free logits"
    ties = 0
    lanes = torch.arange(64, device=mask.device)
    for r0 in range(0, T, rows_per_pass):
        m = mask[r0:r0 + rows_per_pass]
        v = logits[r0:r0 + rows_per_pass].view(-1, nb, 64)
        bits = ((m.unsqueeze(-1) >> lanes) & 1).bool()
        assert bool((bits.sum(-1) == keep).all()), "popcount"
        kmin = torch.where(bits, v, torch.full_like(v, float("inf"))).amin(-1)
        dmax = torch.where(bits, torch.full_like(v, float("-inf")), v).amax(-1)
        assert bool((kmin >= dmax).all()), "a dropped logit above a kept one"
        tie = dmax == kmin
        idx = lanes.expand_as(v)
        at_kmin = v == kmin.unsqueeze(-1)
        last_kept = torch.where(bits & at_kmin, idx, torch.full_like(idx, -1)).amax(-1)
        first_dropped = torch.where(~bits & at_kmin, idx, torch.full_like(idx, 99)).amin(-1)
        assert bool((last_kept[tie] < first_dropped[tie]).all()), "tie not broken to the lower index"
        ties += int(tie.sum())
    return ties


@pytest.mark.parametrize("ties", ["random", "boundary"])
def test_bank_topk_stress_full_size(ties):
    """32768 x 14336 fp32 logits with 5% exact ties per bank (copies of
    random in-bank values, or 3 copies of each bank's 16th-largest value on
    positions below it, so that every bank's boundary falls inside a tie):
    the oracle on a seeded sample of tokens, and the complete validity check
    of the unique mask on every bank, on the GPU."""
    import activation_sparse_ffn_amd as sffn
    cfg = wl.CONFIGS["topk_stress" if ties == "random" else "topk_stress_boundary"]
    p = wl.make_stress_logits(T=cfg["T"], d_i=cfg["d_i"], seed=0, tie_frac=cfg["tie_frac"], ties=ties)
    pd = dev(p)
    mask, ids = sffn.bank_topk(pd, keep=16, return_ids=True)
    torch.cuda.synchronize()
    w = words(mask)
    assert w.shape == (32768, 224)
    assert (np.bitwise_count(w) == 16).all()
    sample = np.sort(np.random.default_rng(0).choice(32768, size=96, replace=False))
    sample = np.concatenate([[0], sample, [32767]])
    np.testing.assert_array_equal(w[sample], o.mask_to_words(o.bank_topk_mask(p[sample], 64, 16)))
    n_ties = assert_topk_valid_on_gpu(mask, pd, 16)
    assert n_ties > 0
    if ties == "boundary":
        assert n_ties == 32768 * 224           # every bank breaks a tie at its boundary
    ids_np = ids.cpu().numpy().view(np.uint16)
    for t in sample[:8]:
        np.testing.assert_array_equal(ids_np[t], np.flatnonzero(o.words_to_mask(w[t:t + 1])[0]))


# ---------------------------------------------------------------------------
# whole forward
# ---------------------------------------------------------------------------

def test_forward_tiny_fp32():
    """fp32 layers take the gather path at every T (here up to 257 tokens)."""
    layer = wl.make_layer(wl.TINY, seed=0)
    ffn = make_ffn(layer)
    for T in (8, 1, 3, 64, 257):
        x = wl.make_tokens(wl.TINY, T, seed=T)
        y, mask, logits = ffn(dev(x), return_mask=True, return_logits=True)
        torch.cuda.synchronize()
        r, ndiff = check_forward(layer, x, y, mask, logits)
        assert ndiff == 0
        assert rel_l2(o.widen(host(y)), r["y"]) < 1e-5      # fp32 layer: fp32-level agreement


@pytest.mark.parametrize("T", [1, 3])
def test_forward_decode_full(full_layer, ffn_full, T):
    x = wl.make_tokens(wl.FULL, T, seed=100 + T)
    y, mask, logits = ffn_full(dev(x), return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    check_forward(full_layer, x, y, mask, logits, bias=False)


@pytest.mark.parametrize("T", [32, 33, 64])
def test_forward_batched_full(full_layer, ffn_full_bias, T):
    """The skinny path at the full layer shape: one 32-token tile (T = 32)
    and two (33: a single token in the second, 64: both full) in the fused
    predictor-2 + top-k kernel, gate/up and down; every token checked."""
    x = wl.make_tokens(wl.FULL, T, seed=200 + T)
    y, mask, logits = ffn_full_bias(dev(x), return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    check_forward(full_layer, x, y, mask, logits, bias=True)
    union = np.bitwise_or.reduce(words(mask), axis=0)
    frac = np.bitwise_count(union).sum() / 14336
    assert 0.5 < frac <= 1.0     # partial overlap across tokens


def test_concurrent_forwards_on_two_streams(ffn_full_bias):
    """Forwards of one layer on two streams at once, each with its own
    workspace (the interface allows it), give the bits of the same forwards
    run one after another: decode, the skinny path and the MFMA path."""
    Ts = [1, 32, 300, 1, 32, 300]
    xs = [dev(wl.make_tokens(wl.FULL, T, seed=900 + i)) for i, T in enumerate(Ts)]
    ref = []
    for x in xs:
        ref.append(ffn_full_bias(x, return_mask=True))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [torch.empty(ffn_full_bias.workspace_size(300), dtype=torch.uint8, device="cuda") for _ in streams]
    outs = [None] * len(xs)
    for s_ in streams:
        s_.wait_stream(torch.cuda.current_stream())
    for i, x in enumerate(xs):
        k = i % 2
        with torch.cuda.stream(streams[k]):
            y = torch.empty_like(x)
            mask = torch.empty((x.shape[0], 224), dtype=torch.int64, device="cuda")
            ffn_full_bias(x, y=y, mask=mask, workspace=wss[k])
            outs[i] = (y, mask)
    torch.cuda.synchronize()
    for (y, m), (yr, mr) in zip(outs, ref):
        assert torch.equal(m, mr)
        assert torch.equal(y.view(torch.int16), yr.view(torch.int16))


@pytest.mark.parametrize("T", [5, 40, 64, 130, 300])
def test_forward_mfma_ragged_full(full_layer, ffn_full, T):
    x = wl.make_tokens(wl.FULL, T, seed=300 + T)
    y, mask, logits = ffn_full(dev(x), return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    rows = None if T <= 8 else [r for r in (0, 1, 31, 32, 39, 63, 64, 127, 128, 129, 255, 256, 299) if r < T]
    check_forward(full_layer, x, y, mask, logits, tokens=rows, bias=False)


def test_forward_prefill_chunk(full_layer, ffn_full):
    cfg = wl.CONFIGS["prefill"]
    x = wl.make_tokens(wl.FULL, cfg["T"], seed=0, outlier_frac=cfg["outlier_frac"])
    y, mask, logits = ffn_full(dev(x), return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    rows = np.concatenate([[0, 127, 128, 4095],
                           np.random.default_rng(1).choice(4096, size=8, replace=False)])
    check_forward(full_layer, x, y, mask, logits, tokens=rows, bias=False)
    # every row's mask is the bank top-k of the logits that were ranked
    assert_topk_valid_on_gpu(mask, logits, 16)


def test_forward_long_context_chunks(full_layer, ffn_full):
    """32768 tokens through one handle in 8 chunks of 4096: sampled tokens of
    every chunk against the oracle, and chunking does not change any row."""
    cfg = wl.CONFIGS["longctx"]
    T, C = cfg["T"], cfg["chunk"]
    x = wl.make_tokens(wl.FULL, T, seed=7, outlier_frac=cfg["outlier_frac"])
    xd = dev(x)
    ys, masks, logits = [], [], []
    for c in range(T // C):
        y, m, lg = ffn_full(xd[c * C:(c + 1) * C], return_mask=True, return_logits=True)
        ys.append(y.clone()); masks.append(m.clone()); logits.append(lg.clone())
    y = torch.cat(ys); mask = torch.cat(masks); lg = torch.cat(logits)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    rows = np.sort(np.concatenate([c * C + rng.choice(C, size=2, replace=False) for c in range(T // C)]))
    check_forward(full_layer, x, y, mask, lg, tokens=rows, bias=False)
    # every one of the 32768 rows' masks is the bank top-k of its logits
    assert_topk_valid_on_gpu(mask, lg, 16)
    # the same tokens in one 4096-row call at another offset give identical rows
    y2 = ffn_full(xd[C // 2:C // 2 + C])
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), y[C // 2:C // 2 + C].view(torch.int16))


def test_forward_many_tiles_ragged(full_layer, ffn_full):
    """2500 tokens: more 256 x 128 gate/up tiles than compute units (each
    workgroup walks several tiles) and a ragged last row tile. Sampled rows
    against the oracle, and the first 256 rows equal a separate 256-token
    call (one tile per workgroup) bit for bit."""
    T = 2500
    x = wl.make_tokens(wl.FULL, T, seed=2500, outlier_frac=0.01)
    xd = dev(x)
    y, mask, logits = ffn_full(xd, return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    rows = [0, 1, 255, 256, 1023, 2303, 2304, 2305, 2450, 2499]
    check_forward(full_layer, x, y, mask, logits, tokens=rows, bias=False)
    y256 = ffn_full(xd[:256])
    torch.cuda.synchronize()
    assert torch.equal(y256.view(torch.int16), y[:256].view(torch.int16))


@pytest.mark.parametrize("gate,keep", [("silu", 16), ("pred", 40), ("pred", 41)])
def test_forward_persistent_gate_up(full_layer, gate, keep):
    """600 tokens: 336 gate/up tiles of 256 x 128, more than the compute
    units, so with compact gate tiles (keep <= 40) each workgroup walks up to
    two tiles and requests the next tile's first slab during the epilogue;
    keep = 41 (full fp16 tiles) runs one tile per workgroup. The last row
    tile holds 88 tokens. Sampled rows against the oracle, and the first 256
    rows equal a 256-token call (112 tiles, one per workgroup) bit for bit."""
    ffn = make_ffn(full_layer, bias=True, keep=keep, gate=gate)
    T = 600
    x = wl.make_tokens(wl.FULL, T, seed=3100 + keep, outlier_frac=0.01)
    xd = dev(x)
    y, mask, logits = ffn(xd, return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    rows = [0, 255, 256, 300, 511, 512, 599]
    check_forward(full_layer, x, y, mask, logits, tokens=rows, bias=True, keep=keep, gate=gate)
    y256 = ffn(xd[:256])
    torch.cuda.synchronize()
    assert torch.equal(y256.view(torch.int16), y[:256].view(torch.int16))


@pytest.mark.parametrize("d", [64, 576])
def test_forward_gate_up_k_step_counts(d):
    """Gate/up over 272 tiles of 256 x 128 (d_i = 2048, 4352 tokens) with a
    single K step (d = 64: persistent workgroups; the gate tile comes after
    that step's barrier and the next tile's first slab is requested during
    the epilogue) and with an odd count of K steps (d = 576: nine, one tile
    per workgroup). Sampled rows, the last row tile's included, against the
    oracle."""
    shape = wl.LayerShape(d=d, d_i=2048, rank=64)
    layer = wl.make_layer(shape, seed=40 + d, bias_var=0.5)
    ffn = make_ffn(layer, bias=True)
    T = 4352
    x = wl.make_tokens(shape, T, seed=41 + d)
    y, mask, logits = ffn(dev(x), return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    check_forward(layer, x, y, mask, logits, tokens=[0, 255, 256, 2000, 4095, 4096, 4351], bias=True)


@pytest.mark.parametrize("T", [1, 2, 4, 5, 64, 200, 300])
@pytest.mark.parametrize("gate", ["pred", "silu"])
def test_forward_mid_shapes(mid_layer, T, gate):
    ffn = make_ffn(mid_layer, bias=True, gate=gate)
    x = wl.make_tokens(MID, T, seed=T)
    y, mask, logits = ffn(dev(x), return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    check_forward(mid_layer, x, y, mask, logits, bias=True, gate=gate)


@pytest.mark.parametrize("keep", [4, 32])
@pytest.mark.parametrize("T", [1, 5, 300])
@pytest.mark.parametrize("gate", ["pred", "silu"])
def test_forward_other_keep(mid_layer, keep, T, gate):
    """keep other than 16 and 64 on every path: the generic gather kernels
    (T = 1), the skinny MFMA path (T = 5) and the fused predictor-2 + top-k
    GEMM, whose selection then takes the full 64-sort (T = 300)."""
    ffn = make_ffn(mid_layer, bias=True, keep=keep, gate=gate)
    x = wl.make_tokens(MID, T, seed=70 + T + keep)
    y, mask, logits = ffn(dev(x), return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    check_forward(mid_layer, x, y, mask, logits, bias=True, keep=keep, gate=gate)


@pytest.mark.parametrize("keep", [7, 40, 41])
@pytest.mark.parametrize("gate", ["pred", "silu"])
def test_forward_gate_tile_formats(mid_layer, keep, gate):
    """The gate tiles that the fused predictor-2 + top-k GEMM hands to the
    256-wide gate/up GEMM (T >= 256) in both layouts: compact rows of kept
    channel positions and gate values (keep <= 40; 7 leaves padding after
    both, 40 is the largest compact row and takes three groups of 16) and
    the full fp16 tile (41). T = 300 leaves the second 256-row tile partly
    filled."""
    ffn = make_ffn(mid_layer, bias=True, keep=keep, gate=gate)
    x = wl.make_tokens(MID, 300, seed=90 + keep)
    y, mask, logits = ffn(dev(x), return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    check_forward(mid_layer, x, y, mask, logits, bias=True, keep=keep, gate=gate)


@pytest.mark.parametrize("T", [2, 16])
@pytest.mark.parametrize("gate", ["pred", "silu"])
def test_keep_all_channels_is_dense(mid_layer, T, gate):
    """keep = 64: the predictor-gated dense FFN (every channel kept)."""
    ffn = make_ffn(mid_layer, bias=True, keep=64, gate=gate)
    x = wl.make_tokens(MID, T, seed=50 + T)
    y, mask, logits = ffn(dev(x), return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    assert (words(mask) == np.uint64(2**64 - 1)).all()
    check_forward(mid_layer, x, y, mask, logits, bias=True, keep=64, gate=gate)


@pytest.mark.parametrize("T", [1, 3, 32, 300])
@pytest.mark.parametrize("gate", ["pred", "silu"])
def test_dense_modes_full(full_layer, T, gate):
    """keep = 64: with the predictor gate, the predictor-gated dense FFN; with
    the silu gate, the plain dense SwiGLU, for which no predictor or top-k
    runs unless the logits are asked for. y does not depend on asking for the
    mask or the logits (bit for bit), the mask is all ones, and sampled rows
    match the oracle (T = 1, 3: gather path; 32: skinny; 300: 256-wide
    tiles)."""
    ffn = make_ffn(full_layer, bias=True, keep=64, gate=gate)
    x = wl.make_tokens(wl.FULL, T, seed=640 + T)
    xd = dev(x)
    y0 = ffn(xd)
    y1, m1 = ffn(xd, return_mask=True)
    y2, m2, lg = ffn(xd, return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(y0), host(y2))
    np.testing.assert_array_equal(host(y1), host(y2))
    assert (words(m1) == np.uint64(0xFFFFFFFFFFFFFFFF)).all()
    np.testing.assert_array_equal(words(m1), words(m2))
    rows = None if T <= 4 else [0, 1, T // 2, T - 1]
    check_forward(full_layer, x, y2, m2, lg, tokens=rows, bias=True, keep=64, gate=gate)


@pytest.mark.parametrize("T", [1, 32])
def test_gate_silu_full(full_layer, T):
    ffn = make_ffn(full_layer, bias=True, gate="silu")
    x = wl.make_tokens(wl.FULL, T, seed=400 + T)
    y, mask, logits = ffn(dev(x), return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    check_forward(full_layer, x, y, mask, logits, bias=True, gate="silu")


@pytest.mark.parametrize("T", [1, 32])
def test_poisoned_skipped_weights(mid_layer, T):
    """Inactive channels are exactly zero: NaN in every weight row the batch
    does not keep leaves y bit-identical. Decode reads kept rows only; the
    batched (skinny) path reads the rows of the batch's union only, for gate,
    up and down alike."""
    L = mid_layer
    x = dev(wl.make_tokens(MID, T, seed=60 + T))
    ffn = make_ffn(L)
    y0, mask = ffn(x, return_mask=True)
    torch.cuda.synchronize()
    union = o.words_to_mask(np.bitwise_or.reduce(words(mask), axis=0)[None])[0]
    dead = ~union
    assert dead.any()
    Wg, Wu, Wd = (o.widen(w).astype(np.float32) for w in (L.W_g, L.W_u, L.W_d))
    Wg[dead] = np.nan
    Wu[dead] = np.nan
    Wd[:, dead] = np.nan
    to_bf = wl.bf16_bits_from_f32
    poisoned = wl.Layer(L.shape, L.A, L.B, to_bf(Wg), to_bf(Wu), to_bf(Wd), L.bias)
    y1 = make_ffn(poisoned)(x)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert bool(torch.isfinite(y1.float()).all())


@pytest.mark.parametrize("T", [1, 32])
def test_deterministic_and_power_of_two_scaling(mid_layer, T):
    L = mid_layer
    x = dev(wl.make_tokens(MID, T, seed=70 + T))
    ffn = make_ffn(L)
    y0 = ffn(x).clone()
    y1 = ffn(x).clone()
    Wu2 = wl.bf16_bits_from_f32(2 * o.widen(L.W_u).astype(np.float32))
    y2 = make_ffn(wl.Layer(L.shape, L.A, L.B, L.W_g, Wu2, L.W_d, L.bias))(x)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert torch.equal((2 * y0.float()).view(torch.int32), y2.float().view(torch.int32))


def test_errors_reported_through_the_abi(mid_layer):
    import activation_sparse_ffn_amd as sffn
    ffn = make_ffn(mid_layer)
    x = dev(wl.make_tokens(MID, 4, seed=1))
    need = ffn.workspace_size(4)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(sffn.SparseFFNError) as e:
        ffn(x, workspace=small)
    assert e.value.status == sffn.SFFN_ERR_WORKSPACE
    lib = sffn.load_library()
    y = torch.empty_like(x)
    ws = ffn.workspace(4)
    st = lib.sparse_ffn_forward(ffn._h, ctypes.c_void_p(x.data_ptr() + 2), 4, ctypes.c_void_p(y.data_ptr()),
                                None, None, ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert st == sffn.SFFN_ERR_INVALID_ARG
    assert ffn(x[:0]).shape == (0, MID.d)     # T = 0 is a no-op


def test_stage_events_time_every_stage(mid_layer):
    ffn = make_ffn(mid_layer)
    x = dev(wl.make_tokens(MID, 1, seed=1))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(10)]
    for e in evs:
        e.record()          # materialise the underlying hipEvent_t
    torch.cuda.synchronize()
    ffn.set_stage_events([e.cuda_event for e in evs])
    ffn(x)
    torch.cuda.synchronize()
    ts = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(5)]
    assert all(0 < t < 100 for t in ts), ts
    assert ffn.stage_names(1)[2] == "gateup" and ffn.stage_names(64)[3] == "gateup_gemm"
    ffn.set_stage_events(None)


@pytest.mark.parametrize("T", [1, 32, 300])
def test_graph_capture_replays_match_eager(mid_layer, full_layer, ffn_full, T):
    """Forwards captured in a HIP graph replay bit-identically to eager runs,
    replay after replay, with other eager work and synchronisations between
    the replays (no library call inside the graph may depend on state that
    only the first replay sees)."""
    ffn = ffn_full if T == 1 else make_ffn(mid_layer)
    d = ffn.d
    x = dev(wl.make_tokens(wl.FULL if T == 1 else MID, T, seed=500 + T))
    other = dev(wl.make_tokens(wl.FULL if T == 1 else MID, T, seed=600 + T))
    y_eager = ffn(x).clone()
    m_eager = ffn(x, return_mask=True)[1].clone()
    y = torch.empty_like(x)
    mask = torch.empty((T, ffn.d_i // 64), dtype=torch.int64, device="cuda")
    ws = torch.empty(ffn.workspace_size(T), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ffn(x, y=y, mask=mask, workspace=ws)          # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ffn(x, y=y, mask=mask, workspace=ws)
    for r in range(4):
        y.zero_()
        mask.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), f"replay {r}"
        assert torch.equal(mask, m_eager), f"replay {r}"
        ffn(other, workspace=ws)                      # eager work reusing the workspace
        torch.cuda.synchronize()
    assert y.shape == (T, d)


@pytest.mark.parametrize("T", [256, 300])
def test_mask_and_output_do_not_depend_on_logits_request(full_layer, ffn_full_bias, T):
    """With T >= 256 the bank top-k runs inside predictor layer 2 and the
    logits reach memory only when asked for: the mask and y must be the
    same either way, and the returned logits must give that mask."""
    x = dev(wl.make_tokens(wl.FULL, T, seed=21))
    y0, m0 = ffn_full_bias(x, return_mask=True)
    y1, m1, p1 = ffn_full_bias(x, return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(words(m0), words(m1))
    np.testing.assert_array_equal(host(y0), host(y1))
    gl = host(p1)
    np.testing.assert_array_equal(o.mask_to_words(o.bank_topk_mask(gl, 64, 16)), words(m1))
    assert ffn_full_bias.stage_names(T)[1] == "pred2_topk_gemm"


# d_i = 2112 = 16.5 x 128: the last 128-column gate/up tile of the 256-wide
# kernel is half outside the layer, and no gate tiles exist (they need whole
# 128-column tiles).
HALF_TILE = wl.LayerShape(d=512, d_i=2112, rank=64)


@pytest.fixture(scope="module")
def half_tile_layer():
    return wl.make_layer(HALF_TILE, seed=9, bias_var=0.5)


@pytest.mark.parametrize("T", [300, 257])
@pytest.mark.parametrize("ask", [False, True])
def test_dense_fallback_half_gate_tile(half_tile_layer, T, ask):
    """keep = 64 with the silu gate (the dense fallback: no predictor, no
    top-k) when d_i is not a multiple of 128: the 256-wide gate/up epilogue
    must not write past the layer's last channel into the next token's row
    or past the intermediate. Every row against the oracle, with and
    without the mask and logits asked for."""
    L = half_tile_layer
    ffn = make_ffn(L, bias=True, keep=64, gate="silu")
    x = wl.make_tokens(HALF_TILE, T, seed=T)
    xd = dev(x)
    if ask:
        y, mask, logits = ffn(xd, return_mask=True, return_logits=True)
    else:
        y = ffn(xd)
    torch.cuda.synchronize()
    r = o.forward(x, L.A, L.B, L.W_g, L.W_u, L.W_d, bias=L.bias, keep=64, gate="silu")
    yg = o.widen(host(y))
    for t in range(T):
        assert rel_l2(yg[t], r["y"][t]) <= REL_L2, f"token {t}"
    if ask:
        assert (words(mask) == np.uint64(0xFFFFFFFFFFFFFFFF)).all()
        check_forward(L, x, y, mask, logits, bias=True, keep=64, gate="silu")


@pytest.mark.parametrize("gate", ["pred", "silu"])
def test_sparse_half_gate_tile(half_tile_layer, gate):
    """keep = 16 at T = 300 with d_i % 128 == 64: predictor layer 2 as a
    separate fp32 GEMM, the stand-alone bank top-k and the general gate/up
    epilogue (mask and logits read per element), every row checked."""
    L = half_tile_layer
    ffn = make_ffn(L, bias=True, keep=16, gate=gate)
    x = wl.make_tokens(HALF_TILE, 300, seed=77)
    y, mask, logits = ffn(dev(x), return_mask=True, return_logits=True)
    torch.cuda.synchronize()
    assert ffn.stage_names(300)[2] == "bank_topk"
    check_forward(L, x, y, mask, logits, bias=True, keep=16, gate=gate)
