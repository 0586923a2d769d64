"""Host logic of bench.py: the algorithmic bytes and flops its roofline
figures divide by, against the figures the layer's shapes fix (d = 4096,
d_i = 14336, rank 448, banks of 64, 16 kept), and the HBM traffic it reads
from the committed counter summary."""
import dataclasses

import bench
import workloads as wl

FULL = wl.FULL


def test_decode_bytes_per_token():
    a = bench.algorithmic("decode", FULL, 1)
    # A (448 x 4096) + B (14336 x 448) + kept rows of W_g, W_u and W_d^T
    # (3 x 3584 rows of 4096), all bf16
    assert a["pred_a"] == 448 * 4096 * 2 == 3_670_016
    assert a["pred_b"] == 14336 * 448 * 2 == 12_845_056
    assert a["gateup"] == 2 * 3584 * 4096 * 2 == 58_720_256
    assert a["down"] == 3584 * 4096 * 2 == 29_360_128
    assert a["bytes"] == 104_595_456
    # the fused kernel's share: B and the gathered rows
    assert a["pred_b"] + a["gateup"] + a["down"] == 100_925_440
    assert a["flops"] == 2 * (448 * 4096 + 14336 * 448 + 3 * 3584 * 4096)


def test_prefill_flops_per_chunk():
    a = bench.algorithmic("prefill", FULL, 4096, masks_union_frac=1.0)
    # executed: the predictor and the dense gate/up/down of 4096 tokens
    assert a["executed_flops"] == 1_510_754_746_368
    # algorithmic: the kept channels only
    assert a["flops"] == 2 * 4096 * (448 * 4096 + 14336 * 448 + 3 * 3584 * 4096)
    assert a["flops"] == 428_422_987_776


def test_batched_bytes_follow_the_union():
    for frac in (0.25, 0.93, 1.0):
        a = bench.algorithmic("batched", FULL, 32, masks_union_frac=frac)
        rows = frac * 14336
        assert a["pred"] == 16_515_072
        assert a["gateup"] == int(2 * rows * 4096 * 2)
        assert a["down"] == int(rows * 4096 * 2)
        assert a["bytes"] == a["pred"] + a["gateup"] + a["down"]


def test_dense_and_amplitude_modes():
    dense = dataclasses.replace(FULL, keep=64)
    a = bench.algorithmic("decode", dense, 1, gate="silu")
    assert a["pred"] == 0                       # keep 64 with the silu gate needs no predictor
    assert a["bytes"] == 3 * 14336 * 4096 * 2
    amp = bench.algorithmic("decode", FULL, 1, gate="amplitude")
    assert amp["gateup"] == 2 * 14336 * 4096 * 2  # every channel's gate and up rows
    assert amp["down"] == 3584 * 4096 * 2
    assert amp["pred"] == 0


def test_decode_traffic_from_the_committed_counters():
    t = bench.profiled_traffic("k_bank_fused")
    assert t is not None
    alg = 100_925_440                            # what the fused kernel must read
    assert 1.0 <= t / alg <= 1.1                 # reads plus the 3.7 MB of partial rows
    assert bench.profiled_traffic("no_such_kernel") is None
