#!/usr/bin/env python3
"""Throughput of the predictor-gated bank-wise sparse SwiGLU FFN forward on
one MI355X, with the CPU oracle timed beside it.

    python bench.py [--steps K] [--warmup W] [--workload decode|batched|prefill|long|...]

A step is one whole forward of the layer (predictor, bank top-k, gate/up on
kept rows, down on kept columns) over one batch of synthetic tokens already
resident in HBM:

  decode   1 token per step (d = 4096, d_i = 14336, rank 448, 16 of 64 kept);
           32 independently drawn layers (the depth of a model of this
           width) are rotated and every step gets a fresh token, so neither
           the ~105 MB a token touches nor the 16.5 MB of predictor weights
           per layer (528 MB over the 32 layers) are served from the 256 MB
           Infinity Cache. This is the default and the headline.
  batched  32 tokens per step, predictor output bias b ~ N(0, 0.5).
  prefill  4096 tokens per step with 1% outlier feature columns.
  long     32768 tokens per step with the same outliers, run as 8 forwards of
           4096-token chunks through one handle (stage times and the
           roofline entry are per chunk).
  topk     the bank top-k alone over 32768 x 14336 fp32 logits with 5% exact
           ties per bank (mask output), as GB/s against HBM.
  copy     not the layer: a plain 1 GiB device-to-device copy, timed and
           used to scale the HBM byte counters (FETCH_SIZE / WRITE_SIZE) of
           a profiler run against a kernel of known traffic.

The timed region replays a HIP graph of the steps (launch overhead removed).
A second pass of the same steps launches each kernel with start/stop events
(hipExtLaunchKernel) to get every stage's own duration; the dominant stage
gives the roofline entry. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-FFN tokens/s per layer (d_i=14336) + achieved HBM GB/s / MFMA % of peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA

WORKLOADS = {
    "decode": dict(T=1, layers=32, bias=False, outliers=0.0),
    "batched": dict(T=32, layers=8, bias=True, outliers=0.0),
    "prefill": dict(T=4096, layers=2, bias=False, outliers=0.01),
    # a 32768-token forward as 8 chunks of 4096 through one handle
    "long": dict(T=32768, chunk=4096, layers=2, bias=False, outliers=0.01),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", choices=sorted(WORKLOADS) + ["topk", "copy", "backward"], default="decode")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the oracle's bounded CPU sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead")
    ap.add_argument("--streams", type=int, default=1,
                    help="chunked workloads: streams the chunks alternate over (each with its "
                         "own workspace), so that one chunk's kernels can fill another's gaps")
    ap.add_argument("--keep", type=int, default=16,
                    help="channels kept per 64-channel bank (64: the dense modes)")
    ap.add_argument("--only", action="store_true",
                    help="time the chosen workload alone (a default run adds the batched, prefill, "
                         "long-context, top-k stress and backward workloads as sub-records)")
    ap.add_argument("--ties", choices=["random", "boundary"], default="random",
                    help="topk workload: where the 5%% exact ties per bank are planted")
    ap.add_argument("--gate", choices=["pred", "silu", "amplitude"], default="pred",
                    help="gate of the kept channels: sigmoid of the predictor logit or of u; "
                         "amplitude: the Dense-4x post-hoc baseline (no predictor)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic(wl_name, shape, T, masks_union_frac=None, gate="pred"):
    """Algorithmic bytes and flops of one step.

    Weights touched per token (bf16): predictor A and B in full, and for each
    of the d_s kept channels one row of W_g, one of W_u and one of W_d^T. The
    dense fallback (every channel kept, SiLU gate) needs no predictor.
    """
    d, d_i, r, ds = shape.d, shape.d_i, shape.rank, shape.d_s
    e = 2
    if gate == "amplitude":
        # Dense-4x baseline: gate and up for every channel, down on kept ones
        row = d * e
        gateup = 2 * d_i * row
        if wl_name == "decode":
            gateup, down = gateup * T, ds * row * T
        else:
            down = int(masks_union_frac * d_i * row)
        out = dict(pred=0, gateup=gateup, down=down, bytes=gateup + down,
                   flops=2 * T * (2 * d_i * d + ds * d))
        if wl_name != "decode":
            out["executed_flops"] = 2 * T * 3 * d_i * d
        return out
    no_pred = gate == "silu" and shape.keep == shape.bank
    pred = 0 if no_pred else (r * d + d_i * r) * e
    if no_pred:
        r = 0
    row = d * e
    if wl_name == "decode":
        gateup = 2 * ds * row * T
        down = ds * row * T
        return dict(pred=pred * T, pred_a=r * d * e * T, pred_b=d_i * r * e * T, gateup=gateup,
                    down=down, bytes=pred * T + gateup + down,
                    flops=2 * T * (r * d + d_i * r + 3 * ds * d))
    # batched / prefill: weights of the union of the batch's kept channels
    u = masks_union_frac * d_i
    gateup = int(2 * u * row)
    down = int(u * row)
    return dict(pred=pred, gateup=gateup, down=down, bytes=pred + gateup + down,
                flops=2 * T * (r * d + d_i * r + 3 * ds * d),
                executed_flops=2 * T * (r * d + d_i * r + 3 * d_i * d))


def profiled_traffic(kernel):
    """HBM bytes per launch of `kernel` (scaled FETCH_SIZE + WRITE_SIZE) from the
    committed rocprofv3 counter summary, or None when it is not listed."""
    path = os.path.join(ROOT, "profiles", "decode_T1_hbm_counters.md")
    try:
        for line in open(path):
            cells = [c.strip() for c in line.split("|")]
            if len(cells) > 5 and cells[1] == f"`{kernel}`":
                return int(cells[4].replace(",", "")) + int(cells[5].replace(",", ""))
    except (OSError, ValueError):
        pass
    return None


def host_cpu():
    """The host the oracle runs on: logical CPUs, the ones this process may
    use, the CPU model and whether SMT is on."""
    info = {"nproc": os.cpu_count() or 1}
    try:
        info["affinity"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        info["smt"] = open("/sys/devices/system/cpu/smt/active").read().strip() == "1"
    except OSError:
        pass
    return info


def cpu_baseline(layer, T, budget_s, keep=16, gate="pred"):
    """The oracle, as it stands, on a bounded sample of the same workload.
    `cores` is the number of threads the oracle's BLAS calls run on."""
    import oracle as o
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    n_tok = 0
    t0 = time.perf_counter()
    seed = 1000
    chunk = min(T, 4)
    while time.perf_counter() - t0 < budget_s:
        x = wl.make_tokens(layer.shape, chunk, seed=seed)
        seed += 1
        o.forward(x, layer.A, layer.B, layer.W_g, layer.W_u, layer.W_d, bias=layer.bias, keep=keep, gate=gate)
        n_tok += chunk
    el = time.perf_counter() - t0
    out = dict(value=n_tok / el, unit="tokens/s", cores=int(cores), kind="oracle",
               sample=f"{n_tok} tokens of the same layer in groups of {chunk}, "
                      f"{el:.1f} s wall, float64 numpy oracle", **host_cpu())
    # the same on one thread, over a third of the budget
    try:
        from threadpoolctl import threadpool_limits
        n1 = 0
        with threadpool_limits(1):
            t1 = time.perf_counter()
            while time.perf_counter() - t1 < budget_s / 3:
                x = wl.make_tokens(layer.shape, chunk, seed=seed)
                seed += 1
                o.forward(x, layer.A, layer.B, layer.W_g, layer.W_u, layer.W_d, bias=layer.bias, keep=keep,
                          gate=gate)
                n1 += chunk
            out["value_1_thread"] = n1 / (time.perf_counter() - t1)
    except ImportError:
        pass
    return out


def copy_calibration(args):
    """Attainable HBM bandwidth of a plain copy (read N + write N bytes)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k = max(args.steps // 64, 4)
    e0.record()
    for _ in range(k):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / k
    gbs = 2 * n / (ms * 1e-3) / 1e9
    print(json.dumps({"metric": "device copy bandwidth (read + write)", "value": round(gbs, 1),
                      "unit": "GB/s", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                      "copies": k, "ms_per_copy": round(ms, 4), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}),
          flush=True)
    del src, dst
    # library bf16 GEMM of the down projection's shape (M = 4096 tokens,
    # N = 4096, K = 14336): the attainable matrix-core rate for reference
    a = torch.randn(4096, 14336, device="cuda").to(torch.bfloat16)
    b = torch.randn(4096, 14336, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b.t())
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        torch.matmul(a, b.t())
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    tf = 2 * 4096 * 4096 * 14336 / (ms * 1e-3) / 1e12
    print(json.dumps({"metric": "library bf16 GEMM 4096 x 4096 x 14336 (torch.matmul)", "value": round(tf, 1),
                      "unit": "TFLOP/s", "ms": round(ms, 4), "frac_of_peak": round(tf / BF16_PEAK_TFLOPS, 4)}),
          flush=True)


def prime(stream):
    """Enqueue ~0.1 ms of GPU spinning on `stream` (not part of any step)."""
    import torch
    with torch.cuda.stream(stream):
        torch.cuda._sleep(250_000)


def dev(a):
    """A numpy array (bf16 bit patterns as uint16, or fp32) as a GPU tensor."""
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def topk_stress(steps, warmup, ties="random"):
    """bank_topk alone on the stress logits: bytes read + mask bytes written."""
    import numpy as np
    import torch
    import activation_sparse_ffn_amd as sffn
    import workloads as wl
    cfg = wl.CONFIGS["topk_stress" if ties == "random" else "topk_stress_boundary"]
    t0 = time.time()
    p = torch.from_numpy(wl.make_stress_logits(cfg["T"], cfg["d_i"], seed=0, tie_frac=cfg["tie_frac"],
                                               ties=ties)).cuda()
    T, d_i = p.shape
    mask = torch.empty((T, d_i // 64), dtype=torch.int64, device="cuda")
    log(f"topk setup {time.time() - t0:.1f}s ({ties} ties)")
    for _ in range(warmup):
        sffn.bank_topk(p, 16, mask_out=mask)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    prime(torch.cuda.current_stream())
    e0.record()
    for _ in range(steps):
        sffn.bank_topk(p, 16, mask_out=mask)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = p.numel() * 4 + mask.numel() * 8
    gbs = nbytes / (ms * 1e-3) / 1e9
    w = mask.cpu().numpy().view(np.uint64)
    assert (np.bitwise_count(w) == 16).all()
    del p
    return {"metric": "bank_topk stress: 32768 x 14336 fp32 logits, keep 16 of 64",
            "value": round(gbs, 1), "unit": "GB/s", "steps": steps, "warmup": warmup,
            "ms_per_step": round(ms, 4), "banks_per_s": round(T * d_i / 64 / (ms * 1e-3), 1),
            "bytes_per_step": nbytes, "ties": f"5% per bank ({ties})",
            "roofline": {"kernel": "k_bank_topk_lanes", "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def backward_bench(ffns, steps, warmup, keep, gate):
    """One backward pass (soft surrogate through the bank top-k) of a
    4096-token chunk of the full layer, rotating the given layers (created
    with for_backward=True); executed TFLOP/s."""
    import torch
    import workloads as wl

    T, n_layers = 4096, len(ffns)
    shape = wl.FULL
    d, d_i, r = shape.d, shape.d_i, shape.rank
    x = dev(wl.make_tokens(shape, T, seed=1, outlier_frac=0.01))
    gy = dev(wl.make_tokens(shape, T, seed=2))
    masks = []
    for f in ffns:
        _, m = f(x, return_mask=True)
        masks.append(m)
    ws = torch.empty(ffns[0]._lib.sparse_ffn_backward_workspace_size(ffns[0]._h, T), dtype=torch.uint8,
                     device="cuda")
    log(f"backward workspace {ws.numel() / 2**30:.2f} GiB")
    K, W = max(1, min(steps, 64)), max(1, min(warmup, 8))
    for i in range(W):
        ffns[i % n_layers].backward(x, gy, masks[i % n_layers], workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    prime(torch.cuda.current_stream())
    e0.record()
    for i in range(K):
        ffns[i % n_layers].backward(x, gy, masks[i % n_layers], workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    # executed: recomputed z, p, U and V; g_h; the weight gradients; g_z, g_A; g_x
    fl = 2 * T * (d * r + r * d_i + 2 * d * d_i + d * d_i + d * d_i + 2 * d * d_i
                  + d_i * r + d_i * r + r * d + d * r + 2 * d * d_i)
    tf = fl / (ms * 1e-3) / 1e12
    del ws
    return {"metric": "sparse-FFN backward (soft surrogate top-k), 4096-token chunk",
            "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "steps": K,
            "warmup": W, "ms_per_step": round(ms, 4), "dtype": "bf16",
            "config": {"workload": f"backward: {T} tokens, d={d}, d_i={d_i}, rank={r}, "
                                   f"keep {keep} of 64, gate {gate}, tau 1",
                       "layers_rotated": n_layers},
            "executed_flops": fl,
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4)}}


def forward_bench(name, ffns, shape, K, W, keep, gate, graph=True, n_streams=1):
    """Time K steps of workload `name` (decode, batched, prefill, long) over
    the given layers, then time every kernel stage with start/stop events;
    returns the record (without the CPU baseline)."""
    import numpy as np
    import torch
    import activation_sparse_ffn_amd as sffn
    import workloads as wl

    cfg = WORKLOADS[name]
    T = cfg["T"]
    n_layers = len(ffns)
    t0 = time.time()
    n_x = 64 if T == 1 else (16 if T <= 32 else (2 if T <= 4096 else 1))
    xs = [dev(wl.make_tokens(shape, T, seed=10_000 + i, outlier_frac=cfg["outliers"])) for i in range(n_x)]
    ys = [torch.empty_like(x) for x in xs]
    chunk = cfg.get("chunk", T)
    n_chunks = T // chunk
    n_streams = max(1, min(n_streams, n_chunks))
    wss = [torch.empty(ffns[0].workspace_size(chunk), dtype=torch.uint8, device="cuda")
           for _ in range(n_streams)]
    masks = [torch.empty((T, shape.n_banks), dtype=torch.int64, device="cuda") for _ in range(n_x)]
    log(f"{name}: tokens {time.time() - t0:.1f}s: {n_layers} layers, {n_x} token batches of T={T}"
        + (f" in {n_chunks} chunks of {chunk} over {n_streams} stream(s)" if n_chunks > 1 else ""))

    G = n_x * n_layers // np.gcd(n_x, n_layers)     # steps per graph: every (x, layer) pair once
    G = min(G, 64, K)                               # K <= 64: the timed region is one replay

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    side = [stream] + [torch.cuda.Stream() for _ in range(n_streams - 1)]

    def step(i, streams=None):
        j = i % n_x
        f = ffns[i % n_layers]
        if n_chunks == 1:
            f(xs[j], y=ys[j], mask=masks[j], workspace=wss[0])
            return
        streams = streams or side
        for s_ in streams[1:]:
            s_.wait_stream(stream)
        for c in range(n_chunks):
            k = c % len(streams)
            sl = slice(c * chunk, (c + 1) * chunk)
            with torch.cuda.stream(streams[k]):
                f(xs[j][sl], y=ys[j][sl], mask=masks[j][sl], workspace=wss[k])
        for s_ in streams[1:]:
            stream.wait_stream(s_)
    with torch.cuda.stream(stream):
        for i in range(W):
            step(i)
    torch.cuda.synchronize()

    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(G):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        # the graph reproduces eager results bit for bit
        y_graph = [y.clone() for y in ys]
        with torch.cuda.stream(stream):
            for i in range(G):
                step(i)
        torch.cuda.synchronize()
        for a, b in zip(y_graph, ys):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "graph replay differs"
        del y_graph

    # ---- timed region -------------------------------------------------------
    reps, rem = divmod(K, G) if g is not None else (0, K)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        # an untimed spin of ~0.1 ms ahead of the start event keeps the GPU
        # busy while the host submits the timed steps, so that the events
        # time the steps' execution and not the host's launch of the first
        prime(stream)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        for i in range(rem):
            step(i)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    ms_per_step = ms / K
    tokens_per_s = T * K / (ms / 1e3)
    log(f"{name}: timed {K} steps: {ms:.3f} ms, {ms_per_step * 1e3:.2f} us/step, {tokens_per_s:.1f} tokens/s")

    # ---- union of kept channels (batched / prefill bytes) -------------------
    union_frac = None
    if T > 1:
        fr = []
        for m in masks:
            w = m.cpu().numpy().view(np.uint64).reshape(-1, chunk, shape.n_banks)
            fr.append(np.mean([np.bitwise_count(np.bitwise_or.reduce(c, axis=0)).sum() / shape.d_i for c in w]))
        union_frac = float(np.mean(fr))
    alg = algorithmic(name, shape, chunk if n_chunks > 1 else T, union_frac, gate)
    if n_chunks > 1:
        # every chunk streams the weights of its own union again
        for key in ("pred", "gateup", "down", "bytes", "flops", "executed_flops"):
            if key in alg:
                alg[key] *= n_chunks

    # ---- per-stage durations (kernel start/stop events) ---------------------
    n_ev = 2 * sffn.SFFN_STAGES
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    with torch.cuda.stream(stream):
        for e in evs:
            e.record(stream)
    torch.cuda.synchronize()
    for f in ffns:
        f.set_stage_events([e.cuda_event for e in evs])
    stage_ms = np.zeros(sffn.SFFN_STAGES)
    n_prof = min(K, 256)
    with torch.cuda.stream(stream):
        for i in range(n_prof):
            step(i, streams=[stream])      # chunks in order: the events time the last one
            stream.synchronize()
            stage_ms += [evs[2 * s].elapsed_time(evs[2 * s + 1]) for s in range(sffn.SFFN_STAGES)]
    for f in ffns:
        f.set_stage_events(None)
    stage_us = stage_ms / n_prof * 1e3
    names = ffns[0].stage_names(chunk)
    stages = {n: round(float(u), 3) for n, u in zip(names, stage_us) if n != "none"}
    log(f"{name}: stages (us): {stages}")

    # ---- roofline of the dominant kernel, and of the whole step --------------
    step_s = ms_per_step * 1e-3
    if name == "decode":
        if "bank_fused" in names:
            dom, kname = "bank_fused", "k_bank_fused"
            nbytes = alg["pred_b"] + alg["gateup"] + alg["down"]
        else:
            dom = next(n for n in names if n.startswith("gateup"))
            kname = "k_gateup"
            nbytes = alg["gateup"]
        dur_s = stage_us[names.index(dom)] * 1e-6
        achieved = nbytes / dur_s / 1e9
        traffic = profiled_traffic(kname) if (keep == 16 and gate == "pred") else None
        roof = dict(kernel=kname, bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                    unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                    bytes_per_launch=nbytes, avg_us=round(float(stage_us[names.index(dom)]), 3))
        if traffic is not None:
            roof["traffic_from"] = "profiles/decode_T1_hbm_counters.md (rocprofv3 --pmc FETCH_SIZE, WRITE_SIZE)"
        gbs = alg["bytes"] / step_s / 1e9
        step_roof = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(gbs / HBM_PEAK_GBS, 4), bytes_per_step=alg["bytes"])
    elif name == "batched":
        # a T = 32 batch is bound by streaming the union's weight rows
        dom = next(n for n in names if n.startswith("gateup"))
        dur_s = stage_us[names.index(dom)] * 1e-6
        gb = alg["gateup"] / dur_s / 1e9
        roof = dict(kernel="k_skinny<SK_GATEUP>", bound="hbm", achieved=round(gb, 1), peak=HBM_PEAK_GBS,
                    unit="GB/s", frac=round(gb / HBM_PEAK_GBS, 4), traffic=None, bytes_per_launch=alg["gateup"],
                    avg_us=round(float(stage_us[names.index(dom)]), 3))
        gbs = alg["bytes"] / step_s / 1e9
        step_roof = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(gbs / HBM_PEAK_GBS, 4), bytes_per_step=alg["bytes"])
    else:
        dom = next(n for n in names if n.startswith("gateup"))
        dur_s = stage_us[names.index(dom)] * 1e-6
        fl = 2 * chunk * 2 * shape.d_i * shape.d    # executed per launch: dense gate and up
        achieved = fl / dur_s / 1e12
        roof = dict(kernel="k_gemm256<EPI_GATEUP>", bound="mfma", achieved=round(achieved, 1),
                    peak=BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=round(achieved / BF16_PEAK_TFLOPS, 4),
                    traffic=None, flops_per_launch=fl, avg_us=round(float(stage_us[names.index(dom)]), 3))
        if "down_gemm" in names:
            dd = stage_us[names.index("down_gemm")] * 1e-6
            fd = 2 * chunk * shape.d_i * shape.d
            roof["down_gemm"] = dict(avg_us=round(dd * 1e6, 3), achieved=round(fd / dd / 1e12, 1),
                                     frac=round(fd / dd / 1e12 / BF16_PEAK_TFLOPS, 4))
        ex = alg["executed_flops"] / step_s / 1e12
        al = alg["flops"] / step_s / 1e12
        step_roof = dict(bound="mfma", achieved=round(ex, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                         frac=round(ex / BF16_PEAK_TFLOPS, 4), executed_flops_per_step=alg["executed_flops"],
                         algorithmic=round(al, 1), algorithmic_frac=round(al / BF16_PEAK_TFLOPS, 4),
                         algorithmic_flops_per_step=alg["flops"])

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0, 1/fan_in) weights, N(0, 1) tokens)",
        "config": {
            "workload": f"{name}: {T} token(s) per step, d=4096, d_i=14336, rank=448, "
                        f"keep {keep} of 64 per bank, gate {gate}, {n_layers} layers rotated"
                        + (", predictor bias N(0, 0.5)" if cfg["bias"] else "")
                        + (", 1% outlier feature columns x20" if cfg["outliers"] else ""),
            "tokens_per_step": T, "layers_rotated": n_layers, "graph": g is not None,
            **({"chunk": chunk, "streams": n_streams} if n_chunks > 1 else {}),
        },
        "step_algorithmic_bytes": alg["bytes"],
        "stages_us": stages,
        "roofline": roof,
        "step_roofline": step_roof,
    }
    if union_frac is not None:
        out["union_frac"] = round(union_frac, 4)
    del xs, ys, wss, masks
    return out


def make_layers(shape, n, keep, gate, bias_layers=0, backward_layers=0):
    """n layers drawn with seeds 0 .. n-1 and packed for the GPU; the first
    `bias_layers` also packed with their predictor bias, the first
    `backward_layers` also packed for the backward pass. Returns the three
    lists and layer 0's host arrays (for the CPU baseline)."""
    import torch
    import activation_sparse_ffn_amd as sffn
    import workloads as wl
    plain, biased, bwd, layer0 = [], [], [], None
    for li in range(n):
        L = wl.make_layer(shape, seed=li, bias_var=0.5)
        W = [dev(a) for a in (L.W_g, L.W_u, L.W_d, L.A, L.B)]
        plain.append(sffn.SparseFFN(*W, None, keep=keep, gate=gate))
        if li < bias_layers:
            biased.append(sffn.SparseFFN(*W, dev(L.bias), keep=keep, gate=gate))
        if li < backward_layers and gate != "amplitude":
            bwd.append(sffn.SparseFFN(*W, None, keep=keep, gate=gate, for_backward=True))
        if li == 0:
            layer0 = wl.Layer(L.shape, L.A, L.B, L.W_g, L.W_u, L.W_d, None)
        del L, W
        torch.cuda.empty_cache()
    return plain, biased, bwd, layer0


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the layer would shard by tokens, with no exchange, or by banks, with one "
              "all-reduce of y).", file=sys.stderr)
        sys.exit(2)
    import torch

    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.workload == "copy":
        copy_calibration(args)
        return
    K, W = args.steps, args.warmup
    if args.workload == "topk":
        print(json.dumps(topk_stress(K, W, args.ties)), flush=True)
        return
    shape = dataclasses.replace(wl.FULL, keep=args.keep)
    if args.workload == "backward":
        _, _, bwd, _ = make_layers(shape, args.layers or 2, args.keep, args.gate, backward_layers=args.layers or 2)
        rec = backward_bench(bwd, K, W, args.keep, args.gate)
        rec.update(n_gpus=1, higher_is_better=True)
        print(json.dumps(rec), flush=True)
        return

    # the headline workload, and in a default run the others as sub-records
    subs = [] if args.only else ["batched", "prefill", "long", "topk", "backward"]
    n_layers = args.layers or WORKLOADS[args.workload]["layers"]
    want_bias = WORKLOADS[args.workload]["bias"]
    n_bias = max(n_layers if want_bias else 0, WORKLOADS["batched"]["layers"] if "batched" in subs else 0)
    n_bwd = 2 if "backward" in subs else 0
    t0 = time.time()
    plain, biased, bwd, layer0 = make_layers(shape, max(n_layers, 2), args.keep, args.gate,
                                             bias_layers=n_bias, backward_layers=n_bwd)
    log(f"setup {time.time() - t0:.1f}s: {len(plain)} layers (+{len(biased)} with bias, +{len(bwd)} for backward)")
    head = biased[:n_layers] if want_bias else plain[:n_layers]
    out = forward_bench(args.workload, head, shape, K, W, args.keep, args.gate, graph=not args.no_graph,
                        n_streams=args.streams)
    sub = {}
    Ks, Ws = max(K, 8), max(W, 2)
    for name in subs:
        if name == args.workload:
            continue
        t1 = time.time()
        if name == "topk":
            sub[name] = topk_stress(Ks, Ws)
        elif name == "backward":
            sub[name] = backward_bench(bwd, Ks, Ws, args.keep, args.gate)
        else:
            layers = biased[:WORKLOADS[name]["layers"]] if WORKLOADS[name]["bias"] else plain[:WORKLOADS[name]["layers"]]
            rec = forward_bench(name, layers, shape, Ks, Ws, args.keep, args.gate, graph=not args.no_graph)
            for k in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "dtype", "data"):
                rec.pop(k, None)
            sub[name] = rec
        sub[name]["wall_s"] = round(time.time() - t1, 1)
        torch.cuda.empty_cache()
    if sub:
        out["sub"] = sub
    if not args.no_cpu_baseline:
        log("cpu baseline ...")
        out["cpu_baseline"] = cpu_baseline(layer0, WORKLOADS[args.workload]["T"], args.cpu_seconds, args.keep,
                                           args.gate)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
