"""Benchmark of the low-bit dequant-GEMM hot path on one MI355X.

One step = one pass of the whole path over the DiT attention-projection
workload (W 3072x3072 bf16 ~ N(0, 0.02^2), 4-bit, group 128):
  1. quantize + pack W                      (ddg_quantize_pack)
  2. Y = X W_hat^T for X of 4096 tokens    (ddg_dequant_gemm, bf16 out)
  3. Y = X W_hat^T for X of 16 tokens      (ddg_dequant_gemm, bf16 out)
Inputs are resident in HBM before timing.  Each step uses other copies of
the weights (round robin over enough copies to exceed 1 GiB, 4x the 256 MB
last-level cache), so the M=16 product streams its packed weights from HBM.

Timing, all with HIP events on the stream the kernels are launched on:
  * ms_per_step: K whole steps back to back between two events (plus a
    device synchronize on both sides);
  * per-kernel averages: for each of the three launches, K launches of that
    kernel alone back to back between two events, divided by K, the median
    of 5 such bursts.  This is the kernel's own duration (what rocprofv3
    --kernel-trace reports per launch), without the dispatch gap an event
    pair around a single launch includes.
value = dequant-GEMM TFLOP/s at M=4096 (2*M*N*K / its average duration); the
JSON line also carries the M=16 packed-weight GB/s, the quantize/pack GB/s,
the roofline of the dominant kernel and the CPU oracle timed on a bounded
sample.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --suite block16     (the four linears of a DiT block at M=16)
    python bench.py --suite block --tokens 1024   (the same at M > 64, one by one and grouped)
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

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
M_BIG, M_SMALL, N, K, BITS = 4096, 16, 3072, 3072, 4
REPEATS = 5
ROTATE_BYTES = 1 << 30
# a burst of back-to-back launches holds at least this many launches, or at
# least this long a stretch of them, whichever is reached first
BURST_MIN_LAUNCHES = 100
BURST_MIN_MS = 200.0


def burst_count(ms_one, steps):
    """Launches per timed burst for a kernel of about ms_one per launch:
    --steps, raised to BURST_MIN_LAUNCHES or to BURST_MIN_MS of launches
    (whichever needs fewer)."""
    import math
    need = min(BURST_MIN_LAUNCHES, math.ceil(BURST_MIN_MS / max(ms_one, 1e-6)))
    return max(steps, need)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other workloads' keys (workloads 3, 4 and 5)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="bound on the oracle's GEMM sample time")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles",
                                                      "dequant_gemm_attnproj3072_traffic.md"),
                    help="profile summary holding the measured HBM bytes per launch of the "
                         "dominant kernel (used only while the kernel sources are unchanged)")
    ap.add_argument("--tokens", type=int, default=1024,
                    help="block: tokens per product (M > 64: the large-M kernel)")
    ap.add_argument("--ways", type=int, default=8,
                    help="shard: the number of GPUs the block's linears are split over along N")
    ap.add_argument("--suite", choices=["block16", "block", "alloc", "rotate", "w4a8", "shard"], default=None,
                    help="block16: instead of the bench line, time the four linears of a "
                         "Wan-14B block (qkv, o, up, down, their drawn bit widths) at 16 tokens, "
                         "one by one and grouped, one JSON line each; alloc: error tables of a "
                         "synthetic 4-block model on the GPU and the PD-guided bit allocation; "
                         "rotate: the block-Hadamard activation pre-pass against HBM, its cost next "
                         "to the product, and its accuracy on the outlier workload; w4a8: FP4 "
                         "weights x FP8 per-token activations on the scaled matrix cores; shard: "
                         "one GPU's share of the block's linears split --ways ways along N, at "
                         "16 and 32760 tokens")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (3 times), to scale the "
                         "FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


PRODUCT_KERNEL_SOURCES = ("api.hip", "ddg_device.hpp", "ddg_kernels.hpp", "inst_bits.hip")


def kernel_source_hash() -> str:
    """sha256 (first 16 hex digits) over the sources that define and dispatch
    the dequant-GEMM kernels, in this order."""
    import hashlib
    h = hashlib.sha256()
    for f in PRODUCT_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "dit_dequant_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(path: str):
    """HBM bytes per launch from a committed counter summary, or None when the
    summary is missing or was taken on other kernel sources."""
    if not path or not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic_json:"):
            rec = json.loads(line.split(":", 1)[1])
            if rec.get("source_hash") == kernel_source_hash():
                return int(rec["bytes_per_launch"])
    return None


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, three times: counter reference."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": src.numel() * 4, "launches": 3}), flush=True)


def _steady_ms(torch, stream, fn, steps, warmup):
    """Average duration of back-to-back calls fn(i), with i a running call
    index (the suites that rotate weight copies pick copy i):
    `warmup` calls, then more warm-up calls of the same products until 100 ms
    of them have run (the first launches after set-up run slower while the
    clock settles), then at least `steps` calls, or BURST_MIN_MS of them,
    between two HIP events on `stream`.  Returns (ms per call, calls timed)."""
    i = 0
    for _ in range(warmup):
        fn(i)
        i += 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < 0.1 or n < 3:
        fn(i)
        i += 1
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    one_ms = (time.perf_counter() - t0) * 1e3 / n
    count = max(steps, int(BURST_MIN_MS / max(one_ms, 1e-3)))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(count):
        fn(i)
        i += 1
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / count, count


def block_suite(tokens, steps, warmup):
    """The four linears of one DiT block (Wan-14B shapes, drawn widths) at
    `tokens` > 64 tokens: each product alone, the four one by one, and the four
    as one grouped call (one launch of the large-M kernel's tiles)."""
    import torch

    from dit_dequant_gemm_amd import api, synth
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    bits_of = synth.config5_bits()
    lins = []
    for name in ("qkv", "o", "up", "down"):
        w = torch.from_numpy(synth.config5_weights(name)).to(dev, torch.bfloat16)
        qw = api.quantize_pack(w, bits_of[name])
        del w
        x = torch.from_numpy(synth.config5_x(name, tokens)).to(dev, torch.bfloat16)
        y = torch.empty((tokens, qw.n), dtype=torch.bfloat16, device=dev)
        lins.append({"name": name, "qw": qw, "x": x, "y": y})

    def timed(fn):
        return _steady_ms(torch, stream, lambda i: fn(), steps, warmup)

    def line(name, ls, timing):
        ms, count = timing
        flops = sum(2.0 * tokens * L["qw"].n * L["qw"].k for L in ls)
        tf = flops / (ms * 1e-3) / 1e12
        print(json.dumps({"suite": "dit-block", "tokens": tokens, "linear": name,
                          "shapes": [f"{L['qw'].n}x{L['qw'].k}@{L['qw'].bits}b" for L in ls],
                          "us": round(ms * 1e3, 2), "TFLOPs": round(tf, 1),
                          "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "steps": count}),
              flush=True)

    for L in lins:
        line(L["name"], [L], timed(lambda L=L: api.dequant_gemm(L["x"], L["qw"], out=L["y"])))
    line("qkv+o+up+down one by one", lins,
         timed(lambda: [api.dequant_gemm(L["x"], L["qw"], out=L["y"]) for L in lins]))
    line("qkv+o+up+down grouped", lins,
         timed(lambda: api.dequant_gemm_grouped([(L["x"], L["qw"], L["y"]) for L in lins])))


def block16_suite(steps, warmup):
    """The four linears of one DiT block at M = 16 tokens: packed-weight GB/s
    of each product (at least K back-to-back launches, or 200 ms of them, after
    100 ms of warm-up launches, over >= 1 GiB of weight copies),
    then the same four as one grouped call, and q, k, v as three 5120x5120
    tensors of different widths, one by one and grouped."""
    import torch

    from dit_dequant_gemm_amd import api, synth
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def timed(fn):
        return _steady_ms(torch, stream, fn, steps, warmup)[0]

    def resident(w_np, x_np, bits):
        """Weight copies totalling >= 1 GiB, X, Y for one linear."""
        w = torch.from_numpy(w_np).to(dev, torch.bfloat16)
        q0 = api.quantize_pack(w, bits)
        del w
        nbytes = q0.packed.numel() + q0.scales.numel() * 4
        copies = max(2, -(-ROTATE_BYTES // nbytes))
        qs = [q0] + [dataclasses.replace(q0, packed=q0.packed.clone(), scales=q0.scales.clone())
                     for _ in range(copies - 1)]
        x = torch.from_numpy(x_np).to(dev, torch.bfloat16)
        y = torch.empty((16, q0.n), dtype=torch.bfloat16, device=dev)
        return {"qs": qs, "x": x, "y": y, "bytes": nbytes, "bits": bits, "n": q0.n, "k": q0.k}

    def line(name, lins, us):
        nbytes = sum(L["bytes"] for L in lins)
        gbps = nbytes / (us * 1e-3) / 1e9
        print(json.dumps({"suite": "dit-block-m16", "linear": name,
                          "shapes": [f"{L['n']}x{L['k']}@{L['bits']}b" for L in lins], "m": 16,
                          "us": round(us * 1e3, 2), "packed_weight_GBps": round(gbps, 1),
                          "frac_of_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4), "steps": steps}),
              flush=True)

    def seq(lins):
        def fn(i):
            for L in lins:
                api.dequant_gemm(L["x"], L["qs"][i % len(L["qs"])], out=L["y"])
        return fn

    def grouped(lins):
        def fn(i):
            api.dequant_gemm_grouped([(L["x"], L["qs"][i % len(L["qs"])], L["y"]) for L in lins])
        return fn

    bits_of = synth.config5_bits()
    block = []
    for name in ("qkv", "o", "up", "down"):
        L = resident(synth.config5_weights(name), synth.config5_x(name, 16), bits_of[name])
        line(name, [L], timed(seq([L])))
        block.append(L)
    line("qkv+o+up+down one by one", block, timed(seq(block)))
    line("qkv+o+up+down grouped", block, timed(grouped(block)))
    del block
    torch.cuda.empty_cache()
    # q, k, v as separate tensors (rows of the fused qkv weight) at 5, 6, 4 bits
    w = synth.config5_weights("qkv")
    x = synth.config5_x("qkv", 16)
    qkv = [resident(w[5120 * i:5120 * (i + 1)], x, b) for i, b in enumerate((5, 6, 4))]
    line("q,k,v (5,6,4 bits) one by one", qkv, timed(seq(qkv)))
    line("q,k,v (5,6,4 bits) grouped", qkv, timed(grouped(qkv)))


def shard_suite(ways, steps, warmup):
    """One GPU's share of the block's four linears when each is split `ways`
    ways along N (column-parallel, no exchange: every GPU holds N/ways rows of
    the packed weight and scales and computes those columns of Y): the first
    N/ways rows of each drawn weight, at 16 tokens (packed-weight GB/s, >= 1 GiB
    of weight copies rotated) and at 32760 tokens (TFLOP/s), each product
    alone, the four one by one, and the four grouped."""
    import torch

    from dit_dequant_gemm_amd import api, synth
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def timed(fn):
        return _steady_ms(torch, stream, fn, steps, warmup)[0]

    bits_of = synth.config5_bits()
    shares = {}
    for name in ("qkv", "o", "up", "down"):
        n, k = synth.C5_SHAPES[name]
        if n % (16 * ways):
            raise SystemExit(f"{name}: {n} rows do not split into {ways} shares of whole 16-row blocks")
        w = torch.from_numpy(synth.config5_weights(name, rows=n // ways)).to(dev, torch.bfloat16)
        shares[name] = api.quantize_pack(w, bits_of[name])
        del w

    def line(tokens, name, ls, ms):
        nbytes = sum(L["bytes"] for L in ls)
        flops = sum(2.0 * tokens * L["q"].n * L["q"].k for L in ls)
        rec = {"suite": "dit-block-shard", "ways": ways, "tokens": tokens, "linear": name,
               "shapes": [f"{L['q'].n}x{L['q'].k}@{L['q'].bits}b" for L in ls], "us": round(ms * 1e3, 2)}
        if tokens <= 16:
            gbps = nbytes / (ms * 1e-3) / 1e9
            rec.update(packed_weight_GBps=round(gbps, 1), frac_of_hbm_peak=round(gbps / PEAK_HBM_GBPS, 4))
        else:
            tf = flops / (ms * 1e-3) / 1e12
            rec.update(TFLOPs=round(tf, 1), frac_of_bf16_peak=round(tf / PEAK_BF16_TFLOPS, 4))
        rec["steps"] = steps
        print(json.dumps(rec), flush=True)

    for tokens in (16, 32760):
        lins = []
        for name, q0 in shares.items():
            nbytes = q0.packed.numel() + q0.scales.numel() * 4
            copies = max(2, -(-ROTATE_BYTES // nbytes)) if tokens <= 16 else 1
            qs = [q0] + [dataclasses.replace(q0, packed=q0.packed.clone(), scales=q0.scales.clone())
                         for _ in range(copies - 1)]
            x = torch.from_numpy(synth.config5_x(name, tokens)).to(dev, torch.bfloat16)
            y = torch.empty((tokens, q0.n), dtype=torch.bfloat16, device=dev)
            lins.append({"name": name, "q": q0, "qs": qs, "x": x, "y": y, "bytes": nbytes})

        def seq(ls):
            return lambda i: [api.dequant_gemm(L["x"], L["qs"][i % len(L["qs"])], out=L["y"]) for L in ls]

        for L in lins:
            line(tokens, L["name"], [L], timed(seq([L])))
        line(tokens, "qkv+o+up+down one by one", lins, timed(seq(lins)))
        line(tokens, "qkv+o+up+down grouped", lins,
             timed(lambda i: api.dequant_gemm_grouped([(L["x"], L["qs"][i % len(L["qs"])], L["y"])
                                                       for L in lins])))
        del lins
        torch.cuda.empty_cache()


def _greedy_allocation(mse, nparams, target, candidates):
    """Reference only: marginal-gain greedy over convex error curves (start
    at the lowest width, add one width at a time where it buys the largest
    error drop per weight-bit) until the budget is spent."""
    import heapq

    import numpy as np
    nc = len(candidates)
    idx = np.zeros(len(nparams), dtype=np.int64)
    budget = (target - candidates[0]) * float(np.sum(nparams))
    heap = [(-(mse[i, 0] - mse[i, 1]) / (candidates[1] - candidates[0]), i) for i in range(len(nparams))]
    heapq.heapify(heap)
    spent = 0.0
    while heap:
        _, i = heapq.heappop(heap)
        cost = float(nparams[i]) * (candidates[idx[i] + 1] - candidates[idx[i]])
        if spent + cost > budget + 1e-6:
            continue
        spent += cost
        idx[i] += 1
        if idx[i] + 1 < nc:
            heapq.heappush(heap, (-(mse[i, idx[i]] - mse[i, idx[i] + 1])
                                  / (candidates[idx[i] + 1] - candidates[idx[i]]), i))
    return np.asarray(candidates)[idx]


def alloc_suite(args):
    """Error tables of a synthetic 4-block DiT (40 tensors, Wan-14B block
    shapes) on the GPU, then the PD-guided allocation at 5.0 bits/weight."""
    import numpy as np
    import torch

    import oracle as O
    from dit_dequant_gemm_amd import api
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    shapes = ([(5120, 5120)] * 8 + [(13824, 5120), (5120, 13824)]) * 4
    rng = np.random.default_rng(5)
    sigma = np.exp(rng.uniform(np.log(0.01), np.log(0.04), size=len(shapes)))
    spread = rng.uniform(0.0, 1.5, size=len(shapes))
    outl = rng.uniform(0.0, 2e-3, size=len(shapes))
    ws = []
    for i, (n, k) in enumerate(shapes):
        w = torch.randn((n, k), generator=gen, device=dev) * float(sigma[i])
        w *= torch.exp(float(spread[i]) * 0.5 * torch.randn((n, 1), generator=gen, device=dev))
        mask = torch.rand((n, k), generator=gen, device=dev) < float(outl[i])
        w = torch.where(mask, w * 10.0, w).to(torch.bfloat16)
        ws.append(w)
    nweights = sum(w.numel() for w in ws)
    api.sse_table(ws[:2])                                  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    sse, nparams = api.sse_table(ws)
    torch.cuda.synchronize()
    t_tables = time.perf_counter() - t0
    mse = sse / nparams[:, None].astype(np.float64)        # the oracle's per-weight tables
    # the dominant kernel alone: events around one tensor's table on the stream
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        api.quant_sse(ws[0])
    e1.record(stream)
    e1.synchronize()
    t_one = e0.elapsed_time(e1) / 5 * 1e-3
    t_init = 0.5 * np.random.default_rng(6).standard_normal((15, len(ws)))
    w_cpu = ws[0][:1024].float().cpu().numpy()
    t0 = time.perf_counter()
    O.mse_table([w_cpu])
    t_table_cpu = time.perf_counter() - t0
    out = {
        "suite": "pd-bit-allocation", "tensors": len(ws), "weights": nweights,
        "gpu_error_tables_s": round(t_tables, 4),
        "gpu_error_table_weight_GBps": round(2 * nweights / t_tables / 1e9, 1),
        "quant_sse_5120x5120_ms": round(t_one * 1e3, 3),
        "quant_sse_5120x5120_weight_GBps": round(2 * 5120 * 5120 / t_one / 1e9, 1),
        "oracle_table_1024x5120_s": round(t_table_cpu, 3),
        "allocation": {},
    }
    for target in (4.0, 5.0, 6.0):
        t0 = time.perf_counter()
        bits, info = api.pd_allocate(sse, nparams, target, t_init, iters=500)
        t_search = time.perf_counter() - t0
        # the oracle's search on the same tables (numpy on the host)
        t0 = time.perf_counter()
        ro = O.pd_search(mse, nparams, target, t_init, iters=500)
        t_search_cpu = time.perf_counter() - t0
        uniform = O.pd_objective(mse, nparams, [int(target)] * len(ws))[0]
        greedy = _greedy_allocation(mse, nparams, target, list(O.PD_CANDIDATES))
        e_greedy, p_greedy = O.pd_objective(mse, nparams, greedy)
        out["allocation"][str(target)] = {
            "mse": info["mse"], "bpw": info["bpw"],
            "widths": {int(b): int(np.sum(bits == b)) for b in O.PD_CANDIDATES},
            "vs_uniform": round(info["mse"] / uniform - 1.0, 4),
            "greedy_reference_vs_uniform": round(e_greedy / uniform - 1.0, 4),
            "greedy_bpw": p_greedy,
            "search_s": round(t_search, 4), "oracle_search_s": round(t_search_cpu, 3),
            "search_matches_oracle": bool(np.array_equal(bits, ro["bits"])),
        }
    # the allocation drives the block's widths: every tensor packed at its width
    # (5.0 bpw), then each block's ten products at 16 tokens in one grouped launch
    bits5, _ = api.pd_allocate(sse, nparams, 5.0, t_init, iters=500)
    qws = [api.quantize_pack(w, int(b)) for w, b in zip(ws, bits5)]
    del ws
    xs = {k: torch.randn((16, k), generator=gen, device=dev).to(torch.bfloat16) for k in (5120, 13824)}
    blocks = [[(xs[qw.k], qw) for qw in qws[10 * i:10 * i + 10]] for i in range(4)]
    outs_b = [api.dequant_gemm_grouped(b) for b in blocks]
    for _ in range(args.warmup):
        for b, o in zip(blocks, outs_b):
            api.dequant_gemm_grouped([(x, qw, y) for (x, qw), y in zip(b, o)])
    items_b = [[(x, qw, y) for (x, qw), y in zip(b, o)] for b, o in zip(blocks, outs_b)]
    reps = []
    for _ in range(5):
        e0.record(stream)
        for _ in range(args.steps):
            for it in items_b:
                api.dequant_gemm_grouped(it)
        e1.record(stream)
        e1.synchronize()
        reps.append(e0.elapsed_time(e1) * 1e-3 / args.steps)
    t_model = sorted(reps)[2]
    wbytes = sum(qw.packed.numel() + qw.scales.numel() * 4 for qw in qws)
    out["allocated_model_m16"] = {
        "blocks": 4, "launches_per_step": 4, "bpw": float(np.sum(nparams * bits5) / np.sum(nparams)),
        "us_per_step": round(t_model * 1e6, 2), "us_per_block": round(t_model * 1e6 / 4, 2),
        "packed_weight_GBps": round(wbytes / t_model / 1e9, 1),
        "frac_of_hbm_peak": round(wbytes / t_model / 8e12, 4),
        "packed_bytes": int(wbytes),
    }
    print(json.dumps(out), flush=True)


def rotate_suite(args):
    """The rotation row: the activation pre-pass (4096 x 3072 bf16, h = 128)
    against HBM (round-robin over copies totalling >= 1 GiB), its cost next to
    the 4-bit product it feeds, the offline weight rotation + quantization, and
    what it buys on the outlier workload: relative Frobenius error of the 4-bit
    product against the float32 product of the unquantized weight."""
    import numpy as np
    import torch

    from dit_dequant_gemm_amd import api, synth
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    h = 128

    def burst(fn, steps):
        for _ in range(args.warmup):
            fn()
        reps = []
        for _ in range(5):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                fn()
            e1.record(stream)
            e1.synchronize()
            reps.append(e0.elapsed_time(e1) / steps)
        return sorted(reps)[2]

    c2 = synth.config2()
    m, k = c2["x"].shape
    n = c2["w"].shape[0]
    perm, signs = synth.rpbh_draw(k, 1)
    pd, sd = torch.from_numpy(perm).to(dev), torch.from_numpy(signs).to(dev)
    x0 = torch.from_numpy(c2["x"]).to(dev, torch.bfloat16)
    copies = max(2, -(-ROTATE_BYTES // (x0.numel() * 2)))
    xs = [x0] + [x0.clone() for _ in range(copies - 1)]
    outs = [torch.empty_like(x0) for _ in range(copies)]
    api.rpbh_rotate(xs[0], pd, sd, h, out=outs[0])            # checks once through the binding
    # then the entry point itself with prepared arguments, so that the burst
    # measures the GPU rather than Python's argument handling
    lib = api.load_library()
    sp = torch.cuda.current_stream().cuda_stream
    calls = [(xs[i].data_ptr(), outs[i].data_ptr()) for i in range(copies)]
    it = [0]

    def rot():
        xp, op = calls[it[0] % copies]
        it[0] += 1
        st = lib.ddg_rpbh_rotate(xp, api.DDG_BF16, m, k, pd.data_ptr(), sd.data_ptr(), h, op,
                                 api.DDG_BF16, sp)
        if st:
            raise api.DDGError(st, "ddg_rpbh_rotate")

    ms_rot = burst(rot, args.steps)
    rot_bytes = m * k * 4
    # offline: rotate the weight (float32 out) and quantize it
    w = torch.from_numpy(c2["w"]).to(dev, torch.bfloat16)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    wr = api.rpbh_rotate(w, pd, sd, h, out_dtype=torch.float32)
    qw = api.quantize_pack(wr, 4)
    e1.record(stream)
    e1.synchronize()
    ms_offline = e0.elapsed_time(e1)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    ms_gemm = burst(lambda: api.dequant_gemm(outs[0], qw, out=y), args.steps)
    del xs, outs

    # accuracy on the outlier workload (first 1024 tokens)
    c4 = synth.config4()
    w4 = torch.from_numpy(c4["w"]).to(dev, torch.bfloat16)
    x4 = torch.from_numpy(c4["x"][:1024]).to(dev, torch.bfloat16)
    y_ref = x4.float() @ w4.float().t().contiguous()
    perm4, signs4 = synth.rpbh_draw(c4["w"].shape[1], 2)
    p4, s4 = torch.from_numpy(perm4).to(dev), torch.from_numpy(signs4).to(dev)

    def rel(a):
        return float(torch.linalg.norm(a.float() - y_ref) / torch.linalg.norm(y_ref))

    def wsnr(w_ref, qw_):
        d = api.dequantize(qw_).float()
        return float(10 * torch.log10((w_ref.float() ** 2).sum() / ((w_ref.float() - d) ** 2).sum()))

    acc = {}
    for bits in (3, 4):
        qp = api.quantize_pack(w4, bits)
        yp = api.dequant_gemm(x4, qp, torch.float32)
        wr4 = api.rpbh_rotate(w4, p4, s4, h, out_dtype=torch.float32)
        qr = api.quantize_pack(wr4, bits)
        yr = api.dequant_gemm(api.rpbh_rotate(x4, p4, s4, h), qr, torch.float32)
        acc[str(bits)] = {"plain_rel_err": round(rel(yp), 5), "rotated_rel_err": round(rel(yr), 5),
                          "plain_weight_snr_db": round(wsnr(w4, qp), 2),
                          "rotated_weight_snr_db": round(wsnr(wr4, qr), 2)}
    print(json.dumps({
        "suite": "rpbh-rotation", "h": h,
        "activation_prepass": {"shape": [m, k], "dtype": "bf16->bf16", "us": round(ms_rot * 1e3, 2),
                               "GBps": round(rot_bytes / ms_rot / 1e6, 1),
                               "frac_of_hbm_peak": round(rot_bytes / ms_rot / 1e6 / 8000.0, 4),
                               "copies_rotated": copies},
        "gemm_4bit_on_rotated_x_us": round(ms_gemm * 1e3, 2),
        "prepass_overhead_vs_gemm": round(ms_rot / ms_gemm, 4),
        "offline_weight_rotate_and_quantize_us": round(ms_offline * 1e3, 1),
        "outlier_workload_accuracy": acc,
    }), flush=True)


def w4a8_suite(args):
    """FP4 (E2M1) weights x per-token FP8 (E4M3) or FP6 (E2M3, E3M2)
    activations at the attention projection (4096 x 3072 x 3072): the
    activation quantizers against HBM, the products (row and tiled weight
    storage, float32 and power-of-two scales) against the dense matrix peaks,
    the 4-bit bf16 product beside them, and each path's error against the
    float32 product of the unquantized weight; then the main products at
    32760 x 5120 x 5120 (a second JSON line)."""
    import torch

    from dit_dequant_gemm_amd import api, synth
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def burst(fn, steps):
        for _ in range(args.warmup):
            fn()
        reps = []
        for _ in range(5):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                fn()
            e1.record(stream)
            e1.synchronize()
            reps.append(e0.elapsed_time(e1) / steps)
        return sorted(reps)[2]

    c = synth.config2()
    m, k = c["x"].shape
    n = c["w"].shape[0]
    x = torch.from_numpy(c["x"]).to(dev, torch.bfloat16)
    w = torch.from_numpy(c["w"]).to(dev, torch.bfloat16)
    qf = api.fp4_quantize_pack(w, "e2m1")
    xq, xs = api.fp8_quantize_rows(x)
    copies = max(2, -(-ROTATE_BYTES // (m * k * 2)))
    xcs = [x] + [x.clone() for _ in range(copies - 1)]
    xqs = [torch.empty_like(xq) for _ in range(copies)]
    xss = [torch.empty_like(xs) for _ in range(copies)]
    lib = api.load_library()
    sp = stream.cuda_stream
    it = [0]

    def quant_rows():
        i = it[0] % copies
        it[0] += 1
        st = lib.ddg_fp8_quantize_rows(xcs[i].data_ptr(), m, k, xqs[i].data_ptr(), xss[i].data_ptr(), sp)
        if st:
            raise api.DDGError(st, "ddg_fp8_quantize_rows")

    ms_q = burst(quant_rows, args.steps)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    ms_g = burst(lambda: api.w4a8_gemm(xq, xs, qf, out=y), args.steps)
    qp = api.fp4_quantize_pack(w, "e2m1", pow2=True)
    ms_p = burst(lambda: api.w4a8_gemm(xq, xs, qp, out=y), args.steps)
    qt = api.fp4_quantize_pack(w, "e2m1", tiled=True)
    ms_t = burst(lambda: api.w4a8_gemm(xq, xs, qt, out=y), args.steps)
    qtp = api.fp4_quantize_pack(w, "e2m1", pow2=True, tiled=True)
    ms_tp = burst(lambda: api.w4a8_gemm(xq, xs, qtp, out=y), args.steps)
    ms_fmt = {f: burst(lambda: api.w4a8_gemm(xq, xs, q, out=y), args.steps)
              for f, q in (("e3m0", api.fp4_quantize_pack(w, "e3m0", tiled=True)),
                           ("e1m2", api.fp4_quantize_pack(w, "e1m2", tiled=True)))}
    # W4A6: 6-bit activations (tiled E2M1 weights)
    ms_a6 = {}
    for f6 in ("e2m3", "e3m2"):
        x6, s6 = api.fp6_quantize_rows(x, f6)
        ms_a6[f6] = (burst(lambda: api.w4a6_gemm(x6, s6, f6, qt, out=y), args.steps),
                     burst(lambda: api.w4a6_gemm(x6, s6, f6, qtp, out=y), args.steps))
    x6, s6 = api.fp6_quantize_rows(x, "e2m3")
    # W4A6 with the lookup weight formats (FP8 B operands)
    ms_a6_lut = {f: burst(lambda: api.w4a6_gemm(x6, s6, "e2m3", q, out=y), args.steps)
                 for f, q in (("e3m0", api.fp4_quantize_pack(w, "e3m0", tiled=True)),
                              ("e1m2", api.fp4_quantize_pack(w, "e1m2", tiled=True)))}
    ms_q6 = burst(lambda: api.fp6_quantize_rows(x, "e2m3"), args.steps)
    # W6A8: FP6 weights (tiled 6-bit storage) x E4M3 activations
    q6w = {f6: (api.fp6_quantize_pack(w, f6), api.fp6_quantize_pack(w, f6, pow2=True)) for f6 in ("e2m3", "e3m2")}
    ms_w6 = {f6: (burst(lambda: api.w6a8_gemm(xq, xs, q6w[f6][0], out=y), args.steps),
                  burst(lambda: api.w6a8_gemm(xq, xs, q6w[f6][1], out=y), args.steps)) for f6 in ("e2m3", "e3m2")}
    qi = api.quantize_pack(w, 4)
    ms_i = burst(lambda: api.dequant_gemm(x, qi, out=y), args.steps)
    del xcs, xqs, xss
    # accuracy on the first 1024 tokens against the float32 product of the bf16 weight
    xr = x[:1024]
    yref = xr.float() @ w.float().t().contiguous()

    def rel(a):
        return float(torch.linalg.norm(a.float() - yref) / torch.linalg.norm(yref))

    e_w4a8 = rel(api.w4a8_gemm(xq[:1024], xs[:1024], qt, torch.float32))
    e_pow2 = rel(api.w4a8_gemm(xq[:1024], xs[:1024], qtp, torch.float32))
    e_a6 = {}
    for f6 in ("e2m3", "e3m2"):
        x6, s6 = api.fp6_quantize_rows(xr, f6)
        e_a6[f6] = rel(api.w4a6_gemm(x6, s6, f6, qt, torch.float32))
    e_w6 = {f6: rel(api.w6a8_gemm(xq[:1024], xs[:1024], q6w[f6][0], torch.float32)) for f6 in ("e2m3", "e3m2")}
    e_int4 = rel(api.dequant_gemm(xr, qi, torch.float32))
    flops = 2.0 * m * n * k
    print(json.dumps({
        "suite": "w4a8-fp4", "shape": [m, n, k], "weight_format": "e2m1", "activation_format": "e4m3",
        "fp8_quantize_rows_us": round(ms_q * 1e3, 2),
        "fp8_quantize_rows_GBps": round(m * k * 3 / ms_q / 1e6, 1),
        "w4a8_tiled_us": round(ms_t * 1e3, 2), "w4a8_tiled_TFLOPs": round(flops / ms_t / 1e9, 1),
        "w4a8_tiled_frac_of_fp8_peak": round(flops / ms_t / 1e9 / 5000.0, 4),
        "w4a8_tiled_pow2_us": round(ms_tp * 1e3, 2), "w4a8_tiled_pow2_TFLOPs": round(flops / ms_tp / 1e9, 1),
        "w4a8_rows_us": round(ms_g * 1e3, 2), "w4a8_rows_pow2_us": round(ms_p * 1e3, 2),
        "w4a8_e3m0_tiled_us": round(ms_fmt["e3m0"] * 1e3, 2), "w4a8_e1m2_tiled_us": round(ms_fmt["e1m2"] * 1e3, 2),
        "fp6_quantize_rows_us": round(ms_q6 * 1e3, 2),
        "w4a6_e2m3_us": round(ms_a6["e2m3"][0] * 1e3, 2), "w4a6_e2m3_TFLOPs": round(flops / ms_a6["e2m3"][0] / 1e9, 1),
        "w4a6_e2m3_pow2_us": round(ms_a6["e2m3"][1] * 1e3, 2),
        "w4a6_e2m3_pow2_TFLOPs": round(flops / ms_a6["e2m3"][1] / 1e9, 1),
        "w4a6_e3m2_us": round(ms_a6["e3m2"][0] * 1e3, 2), "w4a6_e3m2_pow2_us": round(ms_a6["e3m2"][1] * 1e3, 2),
        "w4a6_e3m0_weights_us": round(ms_a6_lut["e3m0"] * 1e3, 2), "w4a6_e1m2_weights_us": round(ms_a6_lut["e1m2"] * 1e3, 2),
        "w6a8_e2m3_us": round(ms_w6["e2m3"][0] * 1e3, 2), "w6a8_e2m3_TFLOPs": round(flops / ms_w6["e2m3"][0] / 1e9, 1),
        "w6a8_e2m3_frac_of_fp8_peak": round(flops / ms_w6["e2m3"][0] / 1e9 / 5000.0, 4),
        "w6a8_e2m3_pow2_us": round(ms_w6["e2m3"][1] * 1e3, 2),
        "w6a8_e3m2_us": round(ms_w6["e3m2"][0] * 1e3, 2), "w6a8_e3m2_pow2_us": round(ms_w6["e3m2"][1] * 1e3, 2),
        "int4_bf16_gemm_us": round(ms_i * 1e3, 2), "int4_bf16_TFLOPs": round(flops / ms_i / 1e9, 1),
        "w4a8_rel_err_vs_f32": round(e_w4a8, 5), "w4a8_pow2_rel_err_vs_f32": round(e_pow2, 5),
        "w4a6_e2m3_rel_err_vs_f32": round(e_a6["e2m3"], 5), "w4a6_e3m2_rel_err_vs_f32": round(e_a6["e3m2"], 5),
        "w6a8_e2m3_rel_err_vs_f32": round(e_w6["e2m3"], 5), "w6a8_e3m2_rel_err_vs_f32": round(e_w6["e3m2"], 5),
        "int4_w4a16_rel_err_vs_f32": round(e_int4, 5),
    }), flush=True)
    del x, w, xq, xs, y, qf, qp, qt, qtp, qi, q6w, x6, s6, xr, yref
    torch.cuda.empty_cache()

    # The same products at a Wan-14B block shape with many tile rounds (the o
    # projection, 32760 x 5120 x 5120), where a single wave of tiles no longer
    # bounds them: tiled E2M1 weights with E4M3 and E2M3 activations, E2M3
    # weights with E4M3 activations, and the 4-bit bf16 product.
    m, (n, k) = 32760, synth.C5_SHAPES["o"]
    x = torch.from_numpy(synth.config5_x("o", m)).to(dev, torch.bfloat16)
    w = torch.from_numpy(synth.config5_weights("o")).to(dev, torch.bfloat16)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    xq, xs = api.fp8_quantize_rows(x)
    x6, s6 = api.fp6_quantize_rows(x, "e2m3")
    qt = api.fp4_quantize_pack(w, "e2m1", tiled=True)
    qtp = api.fp4_quantize_pack(w, "e2m1", pow2=True, tiled=True)
    q6 = api.fp6_quantize_pack(w, "e2m3")
    q6p = api.fp6_quantize_pack(w, "e2m3", pow2=True)
    qi = api.quantize_pack(w, 4)
    steps = max(1, args.steps // 4)
    big = {"w4a8_tiled": burst(lambda: api.w4a8_gemm(xq, xs, qt, out=y), steps),
           "w4a8_tiled_pow2": burst(lambda: api.w4a8_gemm(xq, xs, qtp, out=y), steps),
           "w4a6_e2m3": burst(lambda: api.w4a6_gemm(x6, s6, "e2m3", qt, out=y), steps),
           "w4a6_e2m3_pow2": burst(lambda: api.w4a6_gemm(x6, s6, "e2m3", qtp, out=y), steps),
           "w6a8_e2m3": burst(lambda: api.w6a8_gemm(xq, xs, q6, out=y), steps),
           "w6a8_e2m3_pow2": burst(lambda: api.w6a8_gemm(xq, xs, q6p, out=y), steps),
           "int4_bf16": burst(lambda: api.dequant_gemm(x, qi, out=y), steps)}
    peak = {"w4a8_tiled": 5000.0, "w4a8_tiled_pow2": 5000.0, "w4a6_e2m3": 10100.0, "w4a6_e2m3_pow2": 10100.0,
            "w6a8_e2m3": 5000.0, "w6a8_e2m3_pow2": 5000.0, "int4_bf16": PEAK_BF16_TFLOPS}
    flops = 2.0 * m * n * k
    rec = {"suite": "w4a8-fp4", "shape": [m, n, k], "steps": steps}
    for key, ms in big.items():
        tf = flops / ms / 1e9
        rec[key] = {"us": round(ms * 1e3, 2), "TFLOPs": round(tf, 1), "frac_of_peak": round(tf / peak[key], 4)}
    print(json.dumps(rec), flush=True)


def _sysfs_clock_power():
    """Current shader clock (MHz: the starred line of the DPM table) and board
    power with its cap (W) from the amdgpu sysfs files; None where missing."""
    import glob
    mhz = power = cap = None
    for path in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"):
        try:
            with open(path) as fh:
                for line in fh:
                    line = line.strip()
                    if line.endswith("*") and ":" in line:
                        v = line.split(":", 1)[1].rstrip("*").strip().lower().replace("mhz", "")
                        mhz = max(mhz or 0, int(float(v)))
        except (OSError, ValueError):
            pass
    for name in ("power1_input", "power1_cap"):
        for path in glob.glob(f"/sys/class/drm/card*/device/hwmon/hwmon*/{name}"):
            try:
                with open(path) as fh:
                    w = int(fh.read().strip()) / 1e6
            except (OSError, ValueError):
                continue
            if name == "power1_input":
                power = max(power or 0.0, w)
            else:
                cap = max(cap or 0.0, w)
    return mhz, power, cap


def sample_under_load(torch, fn, seconds=0.3):
    """Median shader clock and board power read from sysfs by a thread while
    fn(i) runs back to back for about `seconds` (outside the timed region)."""
    import threading
    samples = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            samples.append(_sysfs_clock_power())
            time.sleep(0.005)

    th = threading.Thread(target=sampler, daemon=True)
    stream = torch.cuda.current_stream()
    i = 0
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            fn(i)
            i += 1
        stream.synchronize()
    stop.set()
    th.join()
    import statistics
    med = lambda vals: float(statistics.median(vals)) if vals else None
    mhz = [m for m, _, _ in samples if m]
    pw = [p for _, p, _ in samples if p]
    caps = [c for _, _, c in samples if c]
    return {"launches": i, "samples": len(samples),
            "gfx_clock_mhz_median": med(mhz),
            "board_power_w_median": None if not pw else round(med(pw), 1),
            "power_cap_w": None if not caps else round(max(caps), 1)}


def system_info(torch):
    """GPU name, clock and ROCm build; host CPU model."""
    info = {"gpu": torch.cuda.get_device_name(0), "hip": torch.version.hip,
            "torch": torch.__version__}
    try:
        props = torch.cuda.get_device_properties(0)
        info["gcn_arch"] = props.gcnArchName
        info["compute_units"] = props.multi_processor_count
        rate = getattr(props, "clock_rate", None)
        if rate:
            info["max_clock_mhz"] = round(rate / 1000.0)
    except Exception:                                   # pragma: no cover
        pass
    try:
        with open("/opt/rocm/.info/version") as fh:
            info["rocm"] = fh.read().strip()
    except OSError:
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return info


def cpu_baseline(w, x, budget_s):
    """The oracle as it stands on the host: quantize + pack + dequantize the
    whole weight, then the float64 product over row chunks of X until the time
    budget is used.  Rate = 2 * rows * N * K / product time."""
    import numpy as np

    import oracle as O
    blas = None
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        threads = max([d.get("num_threads", 1) for d in pools] + [1])
        blas = [f"{d.get('internal_api')} {d.get('version')} ({d.get('num_threads')} threads)"
                for d in pools if d.get("user_api") == "blas"]
    except Exception:                                   # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    packed, scales, _ = O.quantize_pack(w, BITS)
    t_q = time.perf_counter() - t0
    w16 = O.dequant_from_packed(packed, scales, BITS, N, K)
    # the float64 product over row chunks of X, cycling through the 4096 rows
    # until the budget is used (at least one full pass)
    rows, t_g = 0, 0.0
    chunk = 256
    while rows < x.shape[0] or t_g < budget_s:
        r0 = rows % x.shape[0]
        t1 = time.perf_counter()
        O.gemm_ref(x[r0:r0 + chunk], w16)
        t_g += time.perf_counter() - t1
        rows += chunk
    q_bytes = 2 * N * K + N * K * BITS // 8 + N * K // 32
    return {
        "value": round(2.0 * rows * N * K / t_g / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"float64 product of {rows} token rows (the 4096 rows of X, cycled) with the "
                   f"oracle's dequantized 3072x3072 weight ({t_g:.1f} s); oracle quantize+pack of the "
                   f"whole weight {t_q:.2f} s = {q_bytes / t_q / 1e9:.3f} GB/s (1 thread)"),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "blas": blas,
    }


def _median_burst_ms(torch, fn, count, repeats=REPEATS):
    """Median over `repeats` bursts of the average duration of `count`
    back-to-back calls fn(i), HIP events on the current stream."""
    import statistics
    stream = torch.cuda.current_stream()
    out = []
    for r in range(repeats):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(count):
            fn(r * count + i)
        e1.record(stream)
        e1.synchronize()
        out.append(e0.elapsed_time(e1) / count)
    return float(statistics.median(out))


def _copies(q0, nbytes):
    """Records of q0's weight totalling >= 1 GiB of packed bytes and scales."""
    n = max(2, -(-ROTATE_BYTES // nbytes))
    return [q0] + [dataclasses.replace(q0, packed=q0.packed.clone(), scales=q0.scales.clone())
                   for _ in range(n - 1)]


def workload_lines(api, synth, torch, steps, warmup):
    """The other workloads the metric is quoted over, each timed as back-to-back
    launches of its kernels (median of 5 bursts), weights rotated over >= 1 GiB
    of packed copies, inputs drawn on the GPU with the workloads' shapes and
    distributions (seeded; bf16):
      workload3_m4096   the MLP pair (up 12288x3072, down 3072x12288, Student-t
                        weights) at 3/5/6/7 bits, 4096 tokens: TFLOP/s;
      workload4_lowrank the rank-32 branch + 4-bit residual of a 3072x3072
                        weight at 4096 tokens: the fused call, and the residual's
                        product alone beside it (their difference is the branch:
                        the T pre-pass and the epilogue term), and the T pre-pass
                        alone (ddg_lowrank_down; X rotated over >= 1 GiB of copies):
                        GB/s of X, lora_down and T;
      workload5_m32760  the four Wan-14B block linears at their drawn widths,
                        32760 tokens (one by one and grouped): TFLOP/s;
      workload5_m16     the same at 16 tokens: packed-weight GB/s (one by one and
                        grouped)."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(2024)
    out = {}

    def randn(shape, std=1.0):
        return (torch.randn(shape, generator=gen, device=dev) * std).to(torch.bfloat16)

    def tflops(m, n, k, ms):
        t = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        return {"us": round(ms * 1e3, 2), "TFLOPs": round(t, 1), "frac_of_bf16_peak": round(t / PEAK_BF16_TFLOPS, 4)}

    def gbps(nbytes, ms):
        g = nbytes / (ms * 1e-3) / 1e9
        return {"us": round(ms * 1e3, 2), "packed_weight_GBps": round(g, 1),
                "frac_of_hbm_peak": round(g / PEAK_HBM_GBPS, 4)}

    def burst(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        one = _median_burst_ms(torch, fn, 1, repeats=1)
        return _median_burst_ms(torch, fn, burst_count(one, steps))

    # workload 3: Student-t(4) weights, std 0.02
    t4 = torch.distributions.StudentT(torch.tensor(4.0, device=dev))
    w3 = {}
    lines3 = {}
    for which, (n, k) in (("up", (12288, 3072)), ("down", (3072, 12288))):
        torch.manual_seed(3 + (which == "down"))
        w = (t4.sample((n, k)) * (0.02 / 2 ** 0.5)).to(torch.bfloat16)
        x = randn((4096, k))
        y = torch.empty((4096, n), dtype=torch.bfloat16, device=dev)
        for bits in (3, 5, 6, 7):
            q0 = api.quantize_pack(w, bits)
            qs = _copies(q0, q0.packed.numel() + q0.scales.numel() * 4)
            ms = burst(lambda i: api.dequant_gemm(x, qs[i % len(qs)], out=y))
            lines3.setdefault(which, {})[str(bits)] = tflops(4096, n, k, ms)
            del qs, q0
        del w, x, y
    out["workload3_m4096"] = lines3
    torch.cuda.empty_cache()

    # workload 4: outlier weight, rank-32 branch, 4-bit residual
    c4 = synth.config4(m=4096)
    w4 = torch.from_numpy(c4["w"]).to(dev)
    u, s_, v = torch.svd_lowrank(w4, q=40, niter=3)
    root = s_[:32].sqrt()
    lora_up = (u[:, :32] * root).to(torch.bfloat16).contiguous()             # N x r = L2^T
    lora_down = (v[:, :32] * root).t().contiguous().to(torch.bfloat16)        # r x K = L1^T
    resid = (w4 - lora_up.float() @ lora_down.float()).contiguous()
    q0 = api.quantize_pack(resid, 4)
    qs = _copies(q0, q0.packed.numel() + q0.scales.numel() * 4)
    x4 = torch.from_numpy(c4["x"]).to(dev, torch.bfloat16)
    y4 = torch.empty((4096, 3072), dtype=torch.bfloat16, device=dev)
    wsp = torch.empty(api.workspace_bytes(4096, 3072, 3072, 32), dtype=torch.uint8, device=dev)
    ms_f = burst(lambda i: api.lowrank_fused_gemm(x4, qs[i % len(qs)], lora_down, lora_up,
                                                  out=y4, workspace=wsp))
    ms_m = burst(lambda i: api.dequant_gemm(x4, qs[i % len(qs)], out=y4))
    # the T pre-pass alone (ddg_lowrank_down), over copies of X totalling
    # >= 1 GiB so that every launch reads X from HBM: HBM-bound, X's bytes
    xs4 = [x4] + [x4.clone() for _ in range(max(1, -(-ROTATE_BYTES // (x4.numel() * 2)) - 1))]
    t4 = torch.empty((4096, 32), dtype=torch.bfloat16, device=dev)
    ms_t = burst(lambda i: api.lowrank_down(xs4[i % len(xs4)], lora_down, out=t4))
    t_bytes = x4.numel() * 2 + lora_down.numel() * 2 + t4.numel() * 2
    fl_lr = 2.0 * 4096 * 32 * (3072 + 3072)
    out["workload4_lowrank_m4096"] = {
        "fused": dict(tflops(4096, 3072, 3072, ms_f),
                      TFLOPs_with_branch=round((2.0 * 4096 * 3072 * 3072 + fl_lr) / (ms_f * 1e-3) / 1e12, 1)),
        "residual_product_alone": tflops(4096, 3072, 3072, ms_m),
        "branch_us": round((ms_f - ms_m) * 1e3, 2), "rank": 32,
        "t_prepass_alone": {"us": round(ms_t * 1e3, 2),
                            "GBps": round(t_bytes / (ms_t * 1e-3) / 1e9, 1),
                            "frac_of_hbm_peak": round(t_bytes / (ms_t * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                            "x_copies_rotated": len(xs4)}}
    del qs, q0, w4, resid, x4, y4, wsp, xs4, t4
    torch.cuda.empty_cache()

    # workload 5: the block's linears at their drawn widths
    bits_of = synth.config5_bits()
    recs = {}
    for name, (n, k) in synth.C5_SHAPES.items():
        q0 = api.quantize_pack(randn((n, k), 0.02), bits_of[name])
        recs[name] = (q0, _copies(q0, q0.packed.numel() + q0.scales.numel() * 4))
    big, grouped_big = {}, []
    for name, (n, k) in synth.C5_SHAPES.items():
        x = randn((32760, k))
        y = torch.empty((32760, n), dtype=torch.bfloat16, device=dev)
        q = recs[name][1][:2]
        ms = burst(lambda i: api.dequant_gemm(x, q[i % 2], out=y))
        big[name] = dict(tflops(32760, n, k, ms), bits=bits_of[name])
        grouped_big.append((x, q[0], y))
    ms = burst(lambda i: api.dequant_gemm_grouped(grouped_big))
    flops = sum(2.0 * 32760 * n * k for n, k in synth.C5_SHAPES.values())
    big["grouped"] = {"us": round(ms * 1e3, 2), "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
                      "frac_of_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    out["workload5_m32760"] = big
    del grouped_big, x, y
    torch.cuda.empty_cache()
    small, lins = {}, []
    for name, (n, k) in synth.C5_SHAPES.items():
        x = randn((16, k))
        y = torch.empty((16, n), dtype=torch.bfloat16, device=dev)
        q0, qs = recs[name]
        nbytes = q0.packed.numel() + q0.scales.numel() * 4
        ms = burst(lambda i: api.dequant_gemm(x, qs[i % len(qs)], out=y))
        small[name] = dict(gbps(nbytes, ms), bits=bits_of[name], copies_rotated=len(qs))
        lins.append((x, qs, y, nbytes))
    ms = burst(lambda i: api.dequant_gemm_grouped([(x, qs[i % len(qs)], y) for x, qs, y, _ in lins]))
    small["grouped"] = gbps(sum(L[3] for L in lins), ms)
    out["workload5_m16"] = small
    del recs, lins
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the product "
              "shards along the output dimension with no exchange, see the design notes",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from dit_dequant_gemm_amd import api, synth
    if not os.path.exists(api.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    api.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.suite == "block16":
        block16_suite(args.steps, args.warmup)
        return
    if args.suite == "block":
        block_suite(args.tokens, args.steps, args.warmup)
        return
    if args.suite == "alloc":
        alloc_suite(args)
        return
    if args.suite == "rotate":
        rotate_suite(args)
        return
    if args.suite == "w4a8":
        w4a8_suite(args)
        return
    if args.suite == "shard":
        shard_suite(args.ways, args.steps, args.warmup)
        return

    c = synth.config2(m=M_BIG)
    w_np, x_np = c["w"], c["x"]
    w_bytes = N * K * 2
    p_bytes = N * K * BITS // 8
    s_bytes = N * K // 128 * 4
    # bf16 weight copies for the quantizer (>= 1 GiB with its outputs) and
    # packed records for the products (>= 1 GiB of packed bytes and scales
    # alone: the M=16 product reads nothing else)
    n_w = max(2, -(-ROTATE_BYTES // (w_bytes + p_bytes + s_bytes)))
    n_copies = max(n_w, -(-ROTATE_BYTES // (p_bytes + s_bytes)))
    w0 = torch.from_numpy(w_np).to(dev, torch.bfloat16)
    ws = [w0.clone() for _ in range(n_w)]
    qws = [api.quantize_pack(ws[i % n_w], BITS) for i in range(n_copies)]
    x_big = torch.from_numpy(x_np).to(dev, torch.bfloat16)
    x_small = x_big[:M_SMALL].contiguous()
    y_big = torch.empty((M_BIG, N), dtype=torch.bfloat16, device=dev)
    y_small = torch.empty((M_SMALL, N), dtype=torch.bfloat16, device=dev)

    def quantize_into(i):
        q = qws[i % n_copies]
        st = api.load_library().ddg_quantize_pack(
            ws[i % n_w].data_ptr(), api.DDG_BF16, N, K, BITS, q.packed.data_ptr(),
            q.scales.data_ptr(), torch.cuda.current_stream().cuda_stream)
        if st:
            raise api.DDGError(st, "ddg_quantize_pack")

    stream = torch.cuda.current_stream()

    def gemm_big(i):
        api.dequant_gemm(x_big, qws[i % n_copies], out=y_big)

    def gemm_small(i):
        # packed weights not touched for a while (the big product of step i
        # reads copy i): M=16 streams them from HBM
        api.dequant_gemm(x_small, qws[(i + n_copies // 2) % n_copies], out=y_small)

    def step(i):
        quantize_into(i)
        gemm_big(i)
        gemm_small(i)

    def burst_ms(fn, count, offset):
        """Average duration of `count` back-to-back launches of fn, after
        --warmup untimed launches of the same kernel (the first launches
        after another kernel's burst run slower while the clock settles)."""
        for i in range(args.warmup):
            fn(offset + i)
        offset += args.warmup
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(count):
            fn(offset + i)
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / count

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = ev0.elapsed_time(ev1) / args.steps

    # per-kernel averages: median over REPEATS bursts of at least
    # BURST_MIN_LAUNCHES launches each (all three kernels take well under
    # BURST_MIN_MS / BURST_MIN_LAUNCHES per launch), each burst after its own
    # warm-up launches
    base = args.warmup + args.steps
    n_burst = max(args.steps, BURST_MIN_LAUNCHES)
    reps = {"q": [], "g": [], "s": []}
    for r in range(REPEATS):
        off = base + r * (n_burst + args.warmup)
        reps["q"].append(burst_ms(quantize_into, n_burst, off))
        reps["g"].append(burst_ms(gemm_big, n_burst, off))
        reps["s"].append(burst_ms(gemm_small, n_burst, off))
    t_q, t_g, t_s = (float(np.median(reps[k])) for k in ("q", "g", "s"))

    # context, not a target: torch's dense bf16 product of the same shape on
    # the dequantized weight (no dequantization inside)
    w_t = api.dequantize(qws[0]).t().contiguous()       # K x N, a plain row-major operand
    for _ in range(3):
        torch.matmul(x_big, w_t)
    t_dense = burst_ms(lambda i: torch.matmul(x_big, w_t), args.steps, 0)
    del w_t

    flops = 2.0 * M_BIG * N * K
    tflops = flops / (t_g * 1e-3) / 1e12
    gbps_small = (p_bytes + s_bytes) / (t_s * 1e-3) / 1e9
    gbps_q = (w_bytes + p_bytes + s_bytes) / (t_q * 1e-3) / 1e9

    traffic = measured_traffic(args.traffic)
    # shader clock and board power during a burst of the 4096-token product
    # (sysfs, read by a thread; not part of any timed figure)
    try:
        under_load = sample_under_load(torch, gemm_big)
    except Exception as e:                              # pragma: no cover
        under_load = {"error": repr(e)[:200]}

    out = {
        "metric": "dequant-GEMM TFLOP/s (M=4096) + packed-weight GB/s (M=16), % of roofline",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "DiT attention projection: W 3072x3072 bf16 ~N(0,0.02^2), 4-bit per-group(128) "
                        "fp32 scales, X 4096x3072 bf16 ~N(0,1) (+ its first 16 rows)",
            "m": M_BIG, "m_small": M_SMALL, "n": N, "k": K, "bits": BITS, "y_dtype": "bf16",
            "weight_copies_rotated": n_copies,
            "packed_bytes_rotated": n_copies * (p_bytes + s_bytes),
        },
        "kernels_ms": {"quantize_pack": round(t_q, 5), "dequant_gemm_m4096": round(t_g, 5),
                       "dequant_gemm_m16": round(t_s, 5)},
        "kernels_ms_repeats": {k: [round(v, 5) for v in reps[k2]]
                               for k, k2 in (("quantize_pack", "q"), ("dequant_gemm_m4096", "g"),
                                             ("dequant_gemm_m16", "s"))},
        "launches_per_burst": n_burst,
        "context_torch_matmul_bf16_dense_TFLOPs": round(flops / (t_dense * 1e-3) / 1e12, 1),
        "system": system_info(torch),
        "clock_power_under_load": dict(under_load, kernel="dequant_gemm_m4096"),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "m16_packed_weight_GBps": round(gbps_small, 2),
        "m16_frac_of_hbm_peak": round(gbps_small / PEAK_HBM_GBPS, 4),
        "quantize_pack_GBps": round(gbps_q, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    del ws, qws
    torch.cuda.empty_cache()
    if not args.no_workloads:
        out.update(workload_lines(api, synth, torch, args.steps, args.warmup))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w_np, x_np, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
