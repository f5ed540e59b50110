"""Benchmark of the FP8 (E4M3) 128x128 block-scaled decode GEMM on one MI355X.

One step = one fused-cast GEMM Y = X . W^T (bf16 X cast per row per 128
columns inside the kernel, E4M3 weights with fp32 128x128 block scales,
bf16 Y) on device-resident inputs. The default workload is the square
projection M=8, K=N=5120. Weight quantization is a one-off per weight and
is not part of a step.

Every timed GEMM reads weights that are not in any cache: the steps cycle
through a pool of distinct quantized weights of at least --pool-gib GiB,
larger than the 256 MB Infinity Cache. The steps are captured once in a HIP
graph and the graph is replayed (the decode-step launch pattern); the eager
per-call time is reported beside it.

Prints one JSON line (see the fields at the end of main()).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/GEMM and achieved HBM GB/s (% of 8 TB/s) at M=8, K=5120 FP8 block-scaled"
HBM_PEAK_GBPS = 8000.0
PATH_NAMES = {5: "prefill", 1: "mfma", 2: "dot", 3: "mfma_rows", 4: "mfma_stream"}
FP8_DENSE_PEAK_TFLOPS = 5000.0

WORKLOAD_DESCR = {
    "square": "square projection, K=N=5120, e4m3 weights with 128x128 fp32 block scales, "
              "bf16 activations cast per row per 128 columns inside the GEMM",
    "mlp_up": "MLP up/gate projection, K=5120, N=34816",
    "mlp_down": "MLP down projection, K=17408, N=5120",
    "vocab": "vocabulary output layer, K=5120, N=248320",
    "tiny": "tiny reference, K=1024, N=512",
}


def kernel_source_hash() -> str:
    """Hash of the HIP sources, to tell whether stored counter results still
    describe the current kernels."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_block_scaled_fp8bs_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".h", ".hip")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode())
                h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, m: int, layout: str) -> dict | None:
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources and weight layout."""
    path = os.path.join(ROOT, "profiles", f"gemm_{workload}_m{m}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha") != kernel_source_hash():
        return None
    if vals.get("weight_layout", "rows") != layout:
        return None
    try:
        return {"bytes_per_launch": float(vals["hbm_bytes_per_launch"]),
                "fetch_bytes": float(vals["fetch_bytes_per_launch"]),
                "write_bytes": float(vals["write_bytes_per_launch"])}
    except KeyError:
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(workload, m: int, budget_s: float) -> dict:
    """Time the CPU oracle (cast + fp64 GEMM) on the same workload: on every
    host core the process may use (BLAS threads set to that count), then on
    one core."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    w_bits = workload.weight()
    x_bits = workload.act(m)
    wq, ws = oracle.quantize_weight_ref(w_bits)     # one-off, not timed (as on the GPU)
    cores = len(os.sched_getaffinity(0))

    def timed(budget, limit):
        with threadpool_limits(limits=limit):
            oracle.gemm_fused_ref(x_bits, wq, ws)           # warm-up
            times = []
            t_end = time.perf_counter() + budget
            while len(times) < 3 or (time.perf_counter() < t_end and len(times) < 1000):
                t0 = time.perf_counter()
                oracle.gemm_fused_ref(x_bits, wq, ws)
                times.append(time.perf_counter() - t0)
            threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        return float(np.median(times)), len(times), int(threads)

    med, count, threads = timed(budget_s, cores)
    med1, count1, threads1 = timed(budget_s / 3, 1)
    nbytes = workload.algorithmic_bytes(m)
    return {
        "value": nbytes / med / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{count} full oracle GEMMs (per-row cast + fp64 block GEMM) of the timed "
                  f"workload, median {med * 1e3:.1f} ms each, on {threads} BLAS threads; host "
                  f"{cpu_model()}, {cores} cores visible",
        "us_per_gemm": med * 1e6,
        "one_core": {"value": nbytes / med1 / 1e9, "unit": "GB/s", "cores": threads1,
                     "us_per_gemm": med1 * 1e6, "gemms": count1},
        "cpu_model": cpu_model(),
    }


def step_mix(args, fp8bs, dev) -> int:
    """Decode-step mix: 256 GEMMs drawn from the square, MLP-up, MLP-down and
    vocabulary shapes in a fixed seeded order, run back to back on one
    stream as one captured HIP graph per M. Each shape cycles through its own
    pool of distinct quantized weights (at least --pool-gib GiB, or one
    weight when a single weight is larger), so no weight is served from the
    Infinity Cache. Reports microseconds per step and aggregate algorithmic
    GB/s, with per-shape subtotals of the bytes."""
    import torch

    from workloads import STEP_SHAPES, WORKLOADS, step_order

    order = step_order(256, 0)
    gemm = fp8bs.gemm_tiles if args.weight_layout == "tiles" else fp8bs.gemm
    pools = {}
    gen = torch.Generator(device=dev)
    gen.manual_seed(1400)
    for name in STEP_SHAPES:
        wl = WORKLOADS[name]
        count = max(1, math.ceil(args.pool_gib * (1 << 30) / (wl.n * wl.k)))
        pool = []
        for _ in range(count):
            w = (torch.randn((wl.n, wl.k), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
            wq, wsc = fp8bs.quantize_weight(w)
            del w
            pool.append((fp8bs.pack_weight(wq), wsc) if args.weight_layout == "tiles" else (wq, wsc))
            del wq
        pools[name] = pool
    torch.cuda.synchronize()
    for m in [int(v) for v in args.step_m.split(",")]:
        xs = {name: torch.randn((m, WORKLOADS[name].k), generator=gen, device=dev,
                                dtype=torch.float32).to(torch.bfloat16) for name in STEP_SHAPES}
        ys = {name: torch.empty((m, WORKLOADS[name].n), dtype=torch.bfloat16, device=dev)
              for name in STEP_SHAPES}
        ws_bytes = max(fp8bs.workspace_bytes(m, WORKLOADS[nm].n, WORKLOADS[nm].k) for nm in STEP_SHAPES)
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        cursor = {name: 0 for name in STEP_SHAPES}

        def one_step():
            for name in order:
                pool = pools[name]
                wq, wsc = pool[cursor[name] % len(pool)]
                cursor[name] += 1
                gemm(xs[name], wq, wsc, out=ys[name], workspace=workspace)

        for _ in range(2):
            one_step()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                one_step()
        stream.wait_stream(cap)
        g.replay()
        torch.cuda.synchronize()
        reps = max(3, args.steps // 40)
        graph_us, eager_us = [], []
        for _ in range(reps):
            # the same 256 GEMMs as one graph replay, then as 256 stream
            # launches from the host (eager), each timed on the stream
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            graph_us.append(e0.elapsed_time(e1) * 1e3)
            e0.record(stream)
            one_step()
            e1.record(stream)
            torch.cuda.synchronize()
            eager_us.append(e0.elapsed_time(e1) * 1e3)
        us = sorted(graph_us)[len(graph_us) // 2]
        us_eager = sorted(eager_us)[len(eager_us) // 2]
        by_shape = {name: order.count(name) * WORKLOADS[name].algorithmic_bytes(m) for name in STEP_SHAPES}
        total = sum(by_shape.values())
        print(json.dumps({
            "mode": "step_mix", "m": m, "gemms_per_step": len(order),
            "counts": {name: order.count(name) for name in STEP_SHAPES},
            "us_per_step": round(us, 1), "algorithmic_bytes_per_step": total,
            "GBps": round(total / (us * 1e3), 1), "pct_of_8TBps": round(100 * total / (us * 1e3) / HBM_PEAK_GBPS, 2),
            "eager_us_per_step": round(us_eager, 1),
            "graph_saves_us_per_step": round(us_eager - us, 1),
            "graph_saves_pct": round(100 * (us_eager - us) / us_eager, 2),
            "eager_gap_us_per_launch": round((us_eager - us) / len(order), 3),
            "bytes_by_shape": by_shape, "replays": reps,
            "timing": "median over replays: one captured HIP graph of the 256-GEMM step, "
                      "and the same 256 calls launched eagerly from the host"}), flush=True)
        del xs, ys, workspace, g
    return 0


# One GPU's share of each shape when the GEMM is split over 8 GPUs: whole
# 128-row weight blocks per GPU (column split; the largest share), or whole
# K blocks (row split of MLP down, whose partials would meet in a rank-order
# sum). (name, description, n, k, full shape it comes from)
SHARD_SHAPES = (
    ("vocab_col8", "vocabulary layer, one GPU's column share of 8: 243 of 1,940 block rows",
     31104, 5120, "vocab"),
    ("mlp_up_col8", "MLP up/gate, one GPU's column share of 8: 34 of 272 block rows", 4352, 5120,
     "mlp_up"),
    ("mlp_down_row8", "MLP down, one GPU's K share of 8: 17 of 136 K blocks", 5120, 2176,
     "mlp_down"),
    ("square_col8", "square projection, one GPU's column share of 8: 5 of 40 block rows", 640,
     5120, "square"),
)


def shards(args, fp8bs, dev) -> int:
    """The GEMM at one GPU's share of each shape under an 8-way split (the
    per-GPU kernel of the sharded path; nothing here runs on more than one
    GPU): the table's configuration on tile-layout weights over a rotating
    pool of at least --pool-gib GiB, K calls captured in one graph, the
    median of 5 replays. One JSON line per (shape, m), with the algorithmic
    GB/s of the share and, beside it, the time of the full shape divided by
    8 (what a perfect split would give per GPU)."""
    import torch

    from workloads import WORKLOADS

    stream = torch.cuda.current_stream()

    def timed(fn, steps):
        for i in range(2):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(steps):
                    fn(i)
        stream.wait_stream(cap)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t = []
        for _ in range(5):
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e3 / steps)
        return sorted(t)[2]

    gen = torch.Generator(device=dev)
    gen.manual_seed(1700)
    ms = [int(v) for v in args.shard_m.split(",")]
    for name, descr, n, k, full in SHARD_SHAPES:
        count = max(1, math.ceil(args.pool_gib * (1 << 30) / (n * k)))
        pool = []
        for _ in range(count):
            w = (torch.randn((n, k), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
            wq, wsc = fp8bs.quantize_weight(w)
            pool.append((fp8bs.pack_weight(wq), wsc))
            del w, wq
        fw = WORKLOADS[full]
        fcount = max(1, math.ceil(args.pool_gib * (1 << 30) / (fw.n * fw.k)))
        fpool = []
        for _ in range(fcount):
            w = (torch.randn((fw.n, fw.k), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
            wq, wsc = fp8bs.quantize_weight(w)
            fpool.append((fp8bs.pack_weight(wq), wsc))
            del w, wq
        torch.cuda.synchronize()
        for m in ms:
            x = torch.randn((m, k), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
            fx = torch.randn((m, fw.k), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            fy = torch.empty((m, fw.n), dtype=torch.bfloat16, device=dev)
            work = torch.empty(max(fp8bs.workspace_bytes(m, n, k), 16), dtype=torch.uint8, device=dev)
            fwork = torch.empty(max(fp8bs.workspace_bytes(m, fw.n, fw.k), 16), dtype=torch.uint8,
                                device=dev)
            P, FP = len(pool), len(fpool)
            steps = 200 if n * k < (1 << 28) else 40
            us = timed(lambda i: fp8bs.gemm_tiles(x, pool[i % P][0], pool[i % P][1], out=y,
                                                  workspace=work), steps)
            us_full = timed(lambda i: fp8bs.gemm_tiles(fx, fpool[i % FP][0], fpool[i % FP][1],
                                                       out=fy, workspace=fwork), steps)
            cfg = fp8bs.tiles_select_config(m, n, k)
            nbytes = n * k + 4 * (n // 128) * (k // 128) + 2 * m * k + 2 * m * n
            gbps = nbytes / (us * 1e3)
            print(json.dumps({
                "mode": "shard", "shape": name, "of": full, "description": descr, "m": m, "n": n,
                "k": k, "us": round(us, 3), "GBps": round(gbps, 1),
                "pct_of_8TBps": round(100 * gbps / HBM_PEAK_GBPS, 2), "algorithmic_bytes": nbytes,
                "full_shape_us": round(us_full, 3), "full_shape_us_over_8": round(us_full / 8, 3),
                "share_vs_perfect_split": round(us_full / 8 / us, 3),
                "kernel": {"path": PATH_NAMES.get(cfg.path, str(cfg.path)), "tiles_n": cfg.tiles_n,
                           "waves_n": cfg.waves_n, "waves_k": cfg.waves_k, "depth": cfg.depth,
                           "split_k": cfg.split_k},
                "weight_layout": "tiles", "weight_pool": P,
                "timing": f"graph of {steps} calls over the rotating pool, median of 5 replays"}),
                flush=True)
            del x, fx, y, fy, work, fwork
        del pool, fpool
        torch.cuda.empty_cache()
    return 0


def library_reference(args, x, n, k, gen, dev, stream) -> dict:
    """The same product with bf16 weights through torch.nn.functional.linear
    (hipBLASLt on ROCm), timed the same way as the kernel under test: a
    captured graph of calls over a rotating pool of distinct weights of at
    least --pool-gib GiB (one weight when a single one is larger)."""
    import torch

    m = x.shape[0]
    bf_bytes = 2 * n * k
    count = max(1, math.ceil(args.pool_gib * (1 << 30) / bf_bytes))
    pool = [(torch.randn((n, k), generator=gen, device=dev, dtype=torch.float32) * 0.02)
            .to(torch.bfloat16) for _ in range(count)]
    steps = max(10, min(200, args.steps // 2))

    def run():
        for i in range(steps):
            torch.nn.functional.linear(x, pool[i % count])

    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            run()
    stream.wait_stream(cap)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = bf_bytes + 2 * m * k + 2 * m * n
    del g, pool
    return {"op": "torch.nn.functional.linear, bf16 weights (hipBLASLt)", "us_per_gemm": round(us, 3),
            "GBps": round(nbytes / (us * 1e3), 1), "bytes": nbytes, "weight_pool": count,
            "timing": "hip graph of the calls, replayed"}


def mlp_swiglu(args, fp8bs, dev) -> int:
    """MLP up/gate projection with the SwiGLU epilogue and the FP8 cast of its
    output (one fp8bs_gemm_swiglu call), at every M of the step mix, on the
    5120 -> 34816 shape (inter 17408) with a rotating weight pool of at least
    --pool-gib GiB. Timed beside it, with the same launches in captured
    graphs: the plain GEMM alone, the GEMM followed by the standalone
    epilogue call, the epilogue inside the GEMM launch, and the fused call on
    the same weights in the tile layout (fp8bs_gemm_swiglu_tiles). One JSON
    line per M. Algorithmic bytes of the fused call: weight codes and scales, bf16 X,
    bf16 y (gate and up), h codes and h scales."""
    import dataclasses

    import torch

    from workloads import WORKLOADS

    wl = WORKLOADS["mlp_up"]
    n, k = wl.n, wl.k
    inter = n // 2
    gen = torch.Generator(device=dev)
    gen.manual_seed(1500)
    count = max(1, math.ceil(args.pool_gib * (1 << 30) / (n * k)))
    pool = []
    for _ in range(count):
        w = (torch.randn((n, k), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
        pool.append(fp8bs.quantize_weight(w))
        del w
    tiles = [fp8bs.pack_weight(wq) for wq, _ in pool]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(fn, steps):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(steps):
                    fn(i)
        stream.wait_stream(cap)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = float("inf")
        for _ in range(3):
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / steps)
        return best

    steps = max(10, min(100, args.steps // 4))
    for m in [int(v) for v in args.step_m.split(",")]:
        x = torch.randn((m, k), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        hq = torch.empty((m, inter), dtype=torch.uint8, device=dev)
        hs = torch.empty((m, inter // 128), dtype=torch.float32, device=dev)
        cfg = fp8bs.swiglu_select_config(m, n, k)
        inside = dataclasses.replace(cfg, epilogue=fp8bs.EPILOGUE_IN_GEMM) if cfg.split_k == 1 else None
        ws_bytes = max(max(fp8bs.swiglu_workspace_bytes(m, n, k, c) for c in (cfg, inside) if c),
                       fp8bs.workspace_bytes(m, n, k))
        work = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        P = len(pool)
        fused = timed(lambda i: fp8bs.gemm_swiglu(x, pool[i % P][0], pool[i % P][1], out=y,
                                                  h=(hq, hs), workspace=work), steps)
        plain = timed(lambda i: fp8bs.gemm(x, pool[i % P][0], pool[i % P][1], out=y,
                                           workspace=work), steps)
        two = timed(lambda i: (fp8bs.gemm(x, pool[i % P][0], pool[i % P][1], out=y, workspace=work),
                               fp8bs.swiglu_quant(y, h=(hq, hs))), steps)
        in_gemm = (timed(lambda i: fp8bs.gemm_swiglu_ex(inside, pool[i % P][0], pool[i % P][1], x=x,
                                                        out=y, h=(hq, hs), workspace=work), steps)
                   if inside is not None else None)
        fused_tiles = (timed(lambda i: fp8bs.gemm_swiglu_tiles(x, tiles[i % P], pool[i % P][1], out=y,
                                                               h=(hq, hs), workspace=work), steps)
                       if m <= 32 else None)
        nbytes = (n * k + 4 * (n // 128) * (k // 128) + 2 * m * k + 2 * m * n + m * inter
                  + 4 * m * (inter // 128))
        print(json.dumps({
            "mode": "mlp_swiglu", "m": m, "n": n, "k": k, "inter": inter,
            "config": dataclasses.asdict(cfg),
            "us_fused_call": round(fused, 3), "GBps": round(nbytes / (fused * 1e3), 1),
            "pct_of_8TBps": round(100 * nbytes / (fused * 1e3) / HBM_PEAK_GBPS, 2),
            "algorithmic_bytes": nbytes,
            "us_plain_gemm": round(plain, 3),
            "us_gemm_then_epilogue_call": round(two, 3),
            "us_epilogue_in_gemm": round(in_gemm, 3) if in_gemm is not None else None,
            "us_fused_call_tiles": round(fused_tiles, 3) if fused_tiles is not None else None,
            "config_tiles": dataclasses.asdict(fp8bs.tiles_select_config(m, n, k)) if m <= 32 else None,
            "timing": f"captured graph of {steps} calls over a {P}-weight pool, best of 3 replays"}),
            flush=True)
        del x, y, hq, hs, work
    return 0


def mlp_pair(args, fp8bs, dev) -> int:
    """The wide-then-narrow MLP pair as one chain, at every M of the step
    mix: the up/gate projection 5120 -> 34816 with the SwiGLU epilogue and
    the FP8 cast of h (one gemm_swiglu call), then the down projection
    17408 -> 5120 on those codes (gemm_q), captured in one graph per M over
    rotating weight pools of at least --pool-gib GiB each. Timed on
    tile-layout and on row-major weights. Algorithmic bytes of the pair:
    both weights (codes and scales), bf16 X, the bf16 up/gate output y, h
    (codes and scales) written once and read once, and the bf16 output."""
    import dataclasses

    import torch

    from workloads import WORKLOADS

    up, down = WORKLOADS["mlp_up"], WORKLOADS["mlp_down"]
    assert down.k == up.n // 2 and down.n == up.k
    gen = torch.Generator(device=dev)
    gen.manual_seed(1600)

    def make_pool(n, k):
        count = max(1, math.ceil(args.pool_gib * (1 << 30) / (n * k)))
        pool = []
        for _ in range(count):
            w = (torch.randn((n, k), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
            wq, wsc = fp8bs.quantize_weight(w)
            del w
            pool.append((wq, fp8bs.pack_weight(wq), wsc))
        return pool

    pu, pd = make_pool(up.n, up.k), make_pool(down.n, down.k)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    inter = up.n // 2
    for m in [int(v) for v in args.step_m.split(",")]:
        x = torch.randn((m, up.k), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        y = torch.empty((m, up.n), dtype=torch.bfloat16, device=dev)
        hq = torch.empty((m, inter), dtype=torch.uint8, device=dev)
        hs = torch.empty((m, inter // 128), dtype=torch.float32, device=dev)
        out = torch.empty((m, down.n), dtype=torch.bfloat16, device=dev)
        wsb = max(fp8bs.workspace_bytes(m, up.n, up.k), fp8bs.workspace_bytes(m, down.n, down.k),
                  fp8bs.swiglu_workspace_bytes(m, up.n, up.k))
        work = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        res = {}
        for layout in ("tiles", "rows"):
            def pair(i):
                wu, wd = pu[i % len(pu)], pd[i % len(pd)]
                if layout == "tiles":
                    fp8bs.gemm_swiglu_tiles(x, wu[1], wu[2], out=y, h=(hq, hs), workspace=work)
                    fp8bs.gemm_q_tiles(hq, hs, wd[1], wd[2], out=out, workspace=work)
                else:
                    fp8bs.gemm_swiglu(x, wu[0], wu[2], out=y, h=(hq, hs), workspace=work)
                    fp8bs.gemm_q(hq, hs, wd[0], wd[2], out=out, workspace=work)
            for i in range(3):
                pair(i)
            torch.cuda.synchronize()
            steps = max(10, min(100, args.steps // 4))
            g = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream()
            cap.wait_stream(stream)
            with torch.cuda.stream(cap):
                with torch.cuda.graph(g, stream=cap):
                    for i in range(steps):
                        pair(i)
            stream.wait_stream(cap)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            best = float("inf")
            for _ in range(3):
                e0.record(stream)
                g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                best = min(best, e0.elapsed_time(e1) * 1e3 / steps)
            res[layout] = best
            del g
        hbytes = m * inter + 4 * m * (inter // 128)
        nbytes = (up.n * up.k + 4 * (up.n // 128) * (up.k // 128) + 2 * m * up.k + 2 * m * up.n
                  + 2 * hbytes + down.n * down.k + 4 * (down.n // 128) * (down.k // 128)
                  + 2 * m * down.n)
        print(json.dumps({
            "mode": "mlp_pair", "m": m, "up": [up.n, up.k], "down": [down.n, down.k],
            "us_per_pair": round(res["tiles"], 3), "GBps": round(nbytes / (res["tiles"] * 1e3), 1),
            "pct_of_8TBps": round(100 * nbytes / (res["tiles"] * 1e3) / HBM_PEAK_GBPS, 2),
            "algorithmic_bytes": nbytes, "weight_layout": "tiles",
            "us_per_pair_row_major": round(res["rows"], 3),
            "config_up": dataclasses.asdict(fp8bs.tiles_select_config(m, up.n, up.k)),
            "config_down": dataclasses.asdict(fp8bs.tiles_select_config(m, down.n, down.k)),
            "timing": "captured graph of the two calls per step over rotating weight pools, best of 3 replays"}),
            flush=True)
        del x, y, hq, hs, out, work
    return 0


def _find_csv(root: str, suffix: str) -> list:
    out = []
    for d, _, files in os.walk(root):
        out += [os.path.join(d, f) for f in files if f.endswith(suffix)]
    return sorted(out)


def _pct(v: list, q: float) -> float:
    v = sorted(v)
    return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]


def summarize_trace(root: str, last: int, by_grid: bool = False) -> int:
    """Print a markdown summary of a rocprofv3 --kernel-trace CSV directory:
    per kernel, all dispatches (calls, mean, min, max) and the last `last`
    dispatches (median, p10, p90), in ns. by_grid: one row per kernel and
    grid size (work-items in x, y, z), which separates shapes that share a
    kernel."""
    import csv
    files = _find_csv(root, "kernel_trace.csv")
    if not files:
        print(f"no kernel_trace.csv under {root}", file=sys.stderr)
        return 1
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    by = {}
    for r in rows:
        key = r["Kernel_Name"]
        if by_grid:
            key = f"{key[:90]} grid {r['Grid_Size_X']}x{r['Grid_Size_Y']}x{r['Grid_Size_Z']}"
        by.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    print("| kernel | calls | mean ns | min ns | max ns |")
    print("|---|---|---|---|---|")
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{k[:130]}` | {len(v)} | {sum(v) / len(v):.0f} | {min(v)} | {max(v)} |")
    print()
    for k, v in by.items():
        if "fp8bs::" in k and ("gemm" in k or "splitk" in k or "swiglu" in k or "diag_stream" in k):
            t = v[-last:]
            print(f"- `{k[:130]}`: last {len(t)} dispatches: median {_pct(t, 0.5):.0f} ns, "
                  f"p10 {_pct(t, 0.1):.0f} ns, p90 {_pct(t, 0.9):.0f} ns, mean {sum(t) / len(t):.0f} ns")
    return 0


def summarize_pmc(root: str, counter: str) -> int:
    """Print per-kernel medians (over dispatches) of one rocprofv3 --pmc
    counter from a counter_collection CSV directory."""
    import csv
    files = _find_csv(root, "counter_collection.csv")
    if not files:
        print(f"no counter_collection.csv under {root}", file=sys.stderr)
        return 1
    per = {}
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter:
                    continue
                key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id", "")))
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    by = {}
    for (k, _), v in per.items():
        by.setdefault(k, []).append(v)
    for k, v in sorted(by.items(), key=lambda kv: -len(kv[1])):
        print(f"- `{k[:110]}`: {counter} median {_pct(v, 0.5):.2f} over {len(v)} dispatches "
              f"(min {min(v):.2f}, max {max(v):.2f})")
    return 0


MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 matrix peak


def prefill(args, fp8bs, dev) -> int:
    """Prefill sizes (m > 32: the tiled matrix-core kernel, activations cast
    first): the square, MLP-up and MLP-down weight shapes at several m. Times
    the fused call (cast + GEMM, two kernels) and the GEMM on pre-quantized
    activations, each as a captured graph of calls over a rotating weight
    pool, plus torch.nn.functional.linear with bf16 weights (hipBLASLt) on the
    same shape, and the library's FP8 GEMM with one scale per tensor
    (torch._scaled_mm) on the same codes. One JSON line per (shape, m), with
    TFLOP/s = 2 m n k / time against the dense FP8 peak."""
    import torch

    from workloads import WORKLOADS

    stream = torch.cuda.current_stream()

    def timed(fn, steps):
        for i in range(2):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(steps):
                    fn(i)
        stream.wait_stream(cap)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = float("inf")
        for _ in range(3):
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / steps)
        return best

    gen = torch.Generator(device=dev)
    gen.manual_seed(1600)
    for name in args.prefill_shapes.split(","):
        wl = WORKLOADS[name]
        n, k = wl.n, wl.k
        count = max(1, math.ceil(args.pool_gib * (1 << 30) / (n * k)))
        pool = []
        for _ in range(count):
            w = (torch.randn((n, k), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
            pool.append(fp8bs.quantize_weight(w))
            del w
        tiles = [fp8bs.pack_weight(wq) for wq, _ in pool]
        wbf = (torch.randn((n, k), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
        P = len(pool)
        for m in [int(v) for v in args.prefill_m.split(",")]:
            x = torch.randn((m, k), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
            xq, xs = fp8bs.quantize_act(x)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            work = torch.empty(max(fp8bs.workspace_bytes(m, n, k), 16), dtype=torch.uint8, device=dev)
            flop = 2.0 * m * n * k
            steps = max(5, min(50, int(2e13 / flop)))
            t_fused = timed(lambda i: fp8bs.gemm(x, pool[i % P][0], pool[i % P][1], out=y,
                                                 workspace=work), steps)
            t_q = timed(lambda i: fp8bs.gemm_q(xq, xs, pool[i % P][0], pool[i % P][1], out=y), steps)
            t_qt = timed(lambda i: fp8bs.gemm_q_tiles(xq, xs, tiles[i % P], pool[i % P][1], out=y,
                                                      workspace=work), steps)
            t_lib = timed(lambda i: torch.nn.functional.linear(x, wbf), steps)
            # the vendor library's FP8 GEMM on the same codes with one scale
            # per tensor (hipBLASLt through torch._scaled_mm): not the
            # block-scaled product, a reference for the FP8 matrix path alone
            one = torch.ones((), dtype=torch.float32, device=dev)
            xf8 = xq.view(torch.float8_e4m3fn)
            t_f8 = None
            try:
                t_f8 = timed(lambda i: torch._scaled_mm(
                    xf8, pool[i % P][0].view(torch.float8_e4m3fn).t(), scale_a=one, scale_b=one,
                    out_dtype=torch.bfloat16), steps)
            except (RuntimeError, TypeError):
                pass
            cfg = fp8bs.select_config(m, n, k)
            print(json.dumps({
                "mode": "prefill", "shape": name, "m": m, "n": n, "k": k,
                "path": PATH_NAMES.get(cfg.path, str(cfg.path)),
                "us_fused_call": round(t_fused, 2), "TFLOPs_fused_call": round(flop / (t_fused * 1e6), 1),
                "us_gemm_q": round(t_q, 2), "TFLOPs_gemm_q": round(flop / (t_q * 1e6), 1),
                "pct_of_fp8_peak_gemm_q": round(100 * flop / (t_q * 1e6) / MFMA_FP8_PEAK_TFLOPS, 2),
                "us_gemm_q_tiles": round(t_qt, 2), "TFLOPs_gemm_q_tiles": round(flop / (t_qt * 1e6), 1),
                "bf16_library_us": round(t_lib, 2), "bf16_library_TFLOPs": round(flop / (t_lib * 1e6), 1),
                "fp8_per_tensor_library_us": round(t_f8, 2) if t_f8 else None,
                "fp8_per_tensor_library_TFLOPs": round(flop / (t_f8 * 1e6), 1) if t_f8 else None,
                "timing": f"captured graph of {steps} calls over a {P}-weight pool, best of 3 replays"}),
                flush=True)
            del x, xq, xs, y, work
        del pool, tiles, wbf
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="square", choices=sorted(WORKLOAD_DESCR))
    ap.add_argument("--m", type=int, default=8)
    ap.add_argument("--pool-gib", type=float, default=1.0)
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-library-ref", action="store_true",
                    help="skip the bf16 torch.nn.functional.linear reference")
    ap.add_argument("--eager-only", action="store_true", help="time stream launches only")
    ap.add_argument("--diag-copy-mib", type=int, default=0,
                    help="run only the plain copy kernel over this many MiB (counter calibration)")
    ap.add_argument("--step-mix", action="store_true",
                    help="decode-step mix: 256 GEMMs over the four shapes per step, at every M; "
                         "prints one JSON line per M")
    ap.add_argument("--step-m", default="1,2,4,8,16,32", help="M values of the step mix")
    ap.add_argument("--shards", action="store_true",
                    help="the GEMM at one GPU's share of each shape under an 8-way split")
    ap.add_argument("--shard-m", default="1,8,16", help="M values of --shards")
    ap.add_argument("--prefill", action="store_true",
                    help="prefill sizes (m > 32) on the square and MLP shapes; one JSON line each")
    ap.add_argument("--prefill-m", default="128,512,2048,8192", help="m values of --prefill")
    ap.add_argument("--prefill-shapes", default="square,mlp_up,mlp_down",
                    help="weight shapes of --prefill")
    ap.add_argument("--config", default="",
                    help="explicit GEMM configuration 'path,tiles_n,waves_n,waves_k,depth[,split_k[,reduce]]' "
                         "for the GEMM line instead of the table's (analysis runs)")
    ap.add_argument("--weight-layout", default="tiles", choices=("tiles", "rows"),
                    help="weight codes for the GEMM and step-mix modes: the tile layout "
                         "(fp8bs_pack_weight, rearranged once before timing) or row-major")
    ap.add_argument("--mlp-pair", action="store_true",
                    help="the MLP pair as one chain: up/gate + SwiGLU + FP8 cast, then the down "
                         "projection on those codes, at every M; one JSON line per M")
    ap.add_argument("--mlp-swiglu", action="store_true",
                    help="MLP up/gate projection with the SwiGLU epilogue at every M; "
                         "prints one JSON line per M")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print a summary of a rocprofv3 --kernel-trace CSV directory and exit")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="print per-kernel medians of --counter from a rocprofv3 --pmc directory")
    ap.add_argument("--counter", default="FETCH_SIZE")
    ap.add_argument("--last", type=int, default=200,
                    help="dispatches per kernel counted as the timed ones in --summarize-trace")
    ap.add_argument("--by-grid", action="store_true",
                    help="--summarize-trace: one row per kernel and grid size")
    args = ap.parse_args()

    if args.summarize_trace:
        return summarize_trace(args.summarize_trace, args.last, args.by_grid)
    if args.summarize_pmc:
        return summarize_pmc(args.summarize_pmc, args.counter)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs on one GPU; --shards times one GPU's share of each shape).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import fp8_block_scaled_fp8bs_amd as fp8bs
    from workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fp8bs.load()

    if args.shards:
        return shards(args, fp8bs, dev)
    if args.step_mix:
        return step_mix(args, fp8bs, dev)
    if args.mlp_swiglu:
        return mlp_swiglu(args, fp8bs, dev)
    if args.mlp_pair:
        return mlp_pair(args, fp8bs, dev)
    if args.prefill:
        return prefill(args, fp8bs, dev)

    if args.diag_copy_mib:
        nbytes = args.diag_copy_mib << 20
        src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            fp8bs.diag_copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(src, dst)
        print(json.dumps({"diag_copy_bytes": nbytes, "launches": 5}))
        return 0

    wl = WORKLOADS[args.workload]
    m, n, k = args.m, wl.n, wl.k
    if m not in range(1, 33):
        print("--m must be in 1..32", file=sys.stderr)
        return 2
    alg_bytes = wl.algorithmic_bytes(m)
    floor_us = alg_bytes / (HBM_PEAK_GBPS * 1e3)
    print(f"# workload {args.workload} m={m} n={n} k={k}: {alg_bytes} algorithmic bytes, "
          f"floor {floor_us:.2f} us at 8 TB/s, 80% target {floor_us / 0.8:.2f} us", file=sys.stderr, flush=True)

    # --- inputs, resident on the device before timing ---------------------
    w_bits, x_bits = wl.weight(), wl.act(m)
    w0 = torch.from_numpy(w_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    code_bytes = n * k
    pool_n = max(1, math.ceil(args.pool_gib * (1 << 30) / code_bytes))
    tiles = args.weight_layout == "tiles"
    layout = "tiles" if tiles else "rows"

    def prepared(w):
        # quantized once; in the tile layout, rearranged once (neither is
        # timed). The other layout's codes are kept for the comparison line.
        wq, wsc = fp8bs.quantize_weight(w)
        wt = fp8bs.pack_weight(wq)
        return (wt, wsc, wq) if tiles else (wq, wsc, wt)

    pool = [prepared(w0)]
    del w0
    gen = torch.Generator(device=dev)
    gen.manual_seed(1400)
    for _ in range(pool_n - 1):
        wi = (torch.randn((n, k), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
        pool.append(prepared(wi))
        del wi
    torch.cuda.synchronize()
    cfg = fp8bs.tiles_select_config(m, n, k) if tiles else fp8bs.select_config(m, n, k)
    gemm = fp8bs.gemm_tiles if tiles else fp8bs.gemm
    ws_bytes = fp8bs.workspace_bytes(m, n, k)
    if args.config:
        # an explicit kernel configuration instead of the table's (analysis runs)
        from fp8_block_scaled_fp8bs_amd import GemmConfig
        cfg = GemmConfig(*[int(v) for v in args.config.split(",")],
                         weight_layout=fp8bs.LAYOUT_TILES if tiles else fp8bs.LAYOUT_ROWS)
        ws_bytes = fp8bs.config_workspace_bytes(cfg, m, n, k)

        def gemm(x_, wq_, wsc_, out, workspace):
            return fp8bs.gemm_ex(cfg, wq_, wsc_, x=x_, out=out, workspace=workspace)
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    print(f"# pool {pool_n} weights ({pool_n * code_bytes / 2**30:.2f} GiB), config {cfg}",
          file=sys.stderr, flush=True)

    calls = [0]

    def step(i):
        wq, wsc, _ = pool[i % pool_n]
        gemm(x, wq, wsc, out=y, workspace=workspace)
        calls[0] += 1

    launches0 = fp8bs.launch_count("gemm_mfma") + fp8bs.launch_count("gemm_dot")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # --- eager: stream launches --------------------------------------------
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / args.steps

    # --- graph: the same K steps captured once and replayed ------------------
    # One graph holds LEAD untimed steps, a timestamp kernel, exactly the K
    # timed steps and a second timestamp kernel; the two read the GPU's
    # constant-rate wall clock when they run. The timed region therefore
    # starts while the GPU is already busy and holds the K GEMMs back to
    # back: the graph launch latency stays outside it, whatever K is.
    graph_ms = None
    spread = None
    LEAD = 200
    stamps = torch.zeros(2, dtype=torch.int64, device=dev)
    clock_hz = fp8bs.diag_timestamp_hz()
    timing_note = f"two wall-clock timestamp kernels inside one graph, after {LEAD}+ lead steps"

    def capture(fn, count, lead=0):
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(lead):
                    fn(count + i)
                fp8bs.diag_timestamp(stamps[0:1])
                for i in range(count):
                    fn(i)
                fp8bs.diag_timestamp(stamps[1:2])
        stream.wait_stream(cap)
        return g

    def timed_graph(fn, count):
        """Per-call ms of `count` back-to-back calls, and a function that
        replays the graph once more and returns the next per-call time."""
        g = capture(fn, count, lead=max(LEAD, count))
        g.replay()
        torch.cuda.synchronize()

        def again():
            g.replay()
            torch.cuda.synchronize()
            t = stamps.cpu().tolist()
            return (t[1] - t[0]) / clock_hz * 1e3 / count
        return again(), again

    if not args.eager_only:
        graph_ms, again = timed_graph(step, args.steps)
        # spread: 20 more replays of the same graph, each window timed alone
        per = sorted(again() * 1e3 for _ in range(20))
        spread = {"replays": 20, "gemms_per_replay": args.steps,
                  "us_per_gemm_p10": round(per[2], 3), "us_per_gemm_median": round(per[10], 3),
                  "us_per_gemm_p90": round(per[18], 3)}
        # the same measurement with 400 timed steps, as a check that the
        # per-GEMM time does not depend on K
        t400, _ = timed_graph(step, 400)
        spread["us_per_gemm_400_steps"] = round(t400 * 1e3, 3)

    launches = fp8bs.launch_count("gemm_mfma") + fp8bs.launch_count("gemm_dot") - launches0
    # every host-side GEMM call (warm-up, eager steps, graph captures; replays
    # make none) must have launched the GEMM kernel once
    expected = calls[0]
    if launches != expected:
        print(f"kernel launch count {launches} != expected {expected}", file=sys.stderr)
        return 1
    maps = fp8bs.hip_runtime_mappings()
    if len(maps["libamdhip64"]) != 1 or len(maps["libfp8bs"]) != 1:
        print(f"unexpected runtime mappings: {maps}", file=sys.stderr)
        return 1

    # --- streaming-read ceiling over the same bytes ----------------------------
    # A plain read of the weight codes of each step, timed exactly like the
    # GEMM: a graph of K launches over the same rotating pool behind a lead
    # graph. One workgroup of 512 threads per compute unit (or two), each
    # reading a contiguous range with non-temporal 16-byte loads, 2 x depth
    # in flight per lane; or one workgroup of 4 waves per compute unit
    # requesting its range straight into LDS. The best one is the ceiling.
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    ceiling = {}
    if not args.eager_only:
        for blocks, depth in ((256, 4), (256, 8), (256, 16), (512, 4), (256, 0)):
            def rd(i, blocks=blocks, depth=depth):
                fp8bs.diag_stream(pool[i % pool_n][0], sink, blocks=blocks, depth=depth)
            ms_r, _ = timed_graph(rd, args.steps)
            us_r = ms_r * 1e3
            name = f"{blocks}x256_lds" if depth == 0 else f"{blocks}x512_depth{depth}"
            ceiling[name] = {"us": round(us_r, 3), "GBps": round(code_bytes / (us_r * 1e3), 1)}
    best = max(ceiling.values(), key=lambda v: v["GBps"]) if ceiling else None

    # --- the other weight layout: the same weights and activations through
    # the other call (row-major fp8bs_gemm, or fp8bs_gemm_tiles), with its own
    # table configuration, timed exactly like the GEMM steps
    other = None
    if not args.eager_only and not args.config:
        o_tiles = not tiles
        o_gemm = fp8bs.gemm_tiles if o_tiles else fp8bs.gemm
        o_cfg = fp8bs.tiles_select_config(m, n, k) if o_tiles else fp8bs.select_config(m, n, k)
        o_before = fp8bs.launch_count("gemm_mfma") + fp8bs.launch_count("gemm_dot")
        o_calls = [0]
        o_work = torch.empty(max(fp8bs.config_workspace_bytes(o_cfg, m, n, k), 16),
                             dtype=torch.uint8, device=dev)

        def o_step(i):
            _, wsc, wo = pool[i % pool_n]
            o_gemm(x, wo, wsc, out=y, workspace=o_work)
            o_calls[0] += 1

        o_ms, _ = timed_graph(o_step, args.steps)
        o_launches = fp8bs.launch_count("gemm_mfma") + fp8bs.launch_count("gemm_dot") - o_before
        if o_launches != o_calls[0]:
            print(f"kernel launch count {o_launches} != expected {o_calls[0]} (other layout)",
                  file=sys.stderr)
            return 1
        o_us = o_ms * 1e3
        o_gbps = alg_bytes / (o_us * 1e3)
        other = {"weight_layout": "tiles" if o_tiles else "rows",
                 "call": "fp8bs_gemm_tiles" if o_tiles else "fp8bs_gemm",
                 "us_per_gemm": round(o_us, 3), "GBps": round(o_gbps, 1),
                 "pct_of_8TBps": round(100 * o_gbps / HBM_PEAK_GBPS, 2),
                 "kernel": {"path": PATH_NAMES.get(o_cfg.path, str(o_cfg.path)),
                            "tiles_n": o_cfg.tiles_n, "waves_n": o_cfg.waves_n,
                            "waves_k": o_cfg.waves_k, "depth": o_cfg.depth,
                            "split_k": o_cfg.split_k},
                 "timing": "the same weights and activations, timed exactly like the GEMM steps"}

    # --- library reference: the same product in bf16 through torch (hipBLASLt)
    lib_ref = None if args.no_library_ref else library_reference(args, x, n, k, gen, dev, stream)

    step_ms = graph_ms if graph_ms is not None else eager_ms
    us = step_ms * 1e3
    gbps = alg_bytes / (us * 1e3)
    traffic = stored_traffic(args.workload, m, layout)
    roofline = {
        "bound": "hbm",
        "achieved": round(gbps, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(gbps / HBM_PEAK_GBPS, 4),
        "traffic": round(traffic["bytes_per_launch"]) if traffic else None,
    }
    cpu = None if args.no_cpu else cpu_baseline(wl, m, args.cpu_budget_s)
    out = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {WORKLOAD_DESCR[args.workload]}; M={m}",
            "m": m, "n": n, "k": k,
            "algorithmic_bytes": alg_bytes,
            "weight_pool": pool_n,
            "kernel": {"path": PATH_NAMES.get(cfg.path, str(cfg.path)), "tiles_n": cfg.tiles_n,
                       "waves_n": cfg.waves_n, "waves_k": cfg.waves_k, "depth": cfg.depth,
                       "split_k": cfg.split_k,
                       "launches_per_gemm": 2 if cfg.split_k > 1 and cfg.reduce == 0 else 1,
                       "explicit": bool(args.config)},
            "weight_layout": layout,
            "timing": (f"hip graph replay, K steps timed with {timing_note}" if graph_ms is not None
                       else "stream launches"),
        },
        "us_per_gemm": round(us, 3),
        "pct_of_8TBps": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "eager_us_per_gemm": round(eager_ms * 1e3, 3),
        "replay_spread": spread,
        "other_layout": other,
        "stream_read_ceiling": ({"bytes": code_bytes, "best_us": best["us"], "best_GBps": best["GBps"],
                                 "gemm_frac_of_ceiling": round(best["us"] / us, 4),
                                 "configs": ceiling,
                                 "timing": "K launches timed exactly like the GEMM steps"}
                                if best else None),
        "bf16_library_reference": (dict(lib_ref, fp8_speedup=round(lib_ref["us_per_gemm"] / us, 2))
                                   if lib_ref else None),
        "mfma_flops_frac": round(2 * m * n * k / (us * 1e-6) / (FP8_DENSE_PEAK_TFLOPS * 1e12), 6),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
