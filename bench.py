"""Benchmark: fp32 SGEMM throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--cfg ID]

A step is one C = alpha*A*B + beta*C call of the library (the whole hot path)
on the workload's seeded inputs, already resident in device memory.  Each
step writes its own copy of the pristine C, so every timed launch does the
full read-modify-write on fresh data and the last output can be checked
against the CPU oracle.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fp32 SGEMM GFLOP/s at 4096^3 and % of MI355X fp32 peak (1 GPU)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed launches first; in a fresh process the first launches after "
                         "only ten warm-ups still run 5-10%% slower")
    ap.add_argument("--workload", default="sq4096")
    ap.add_argument("--cfg", type=int, default=-1, help="force a configuration id")
    ap.add_argument("--tile", default=None,
                    help="force the configuration with this comma-separated tuple")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-context", action="store_true", help="skip the context timings (torch.mm, cold caches)")
    ap.add_argument("--ladder", action="store_true",
                    help="only time the four ladder rungs on the workload (one JSON line)")
    ap.add_argument("--oracle-timing", action="store_true",
                    help="only time the CPU oracle on every workload (one JSON line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 28  # 2^28 floats = 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": 4 * n, "launches": 3}), flush=True)


def cpu_baseline(w, A, B, C, target_s):
    """The oracle, as it stands, on the first R rows of the same workload."""
    from oracle import oracle
    oracle.build(force=False)
    threads = oracle.max_threads()
    rows = 8
    t0 = time.perf_counter()
    oracle.sgemm(A[:rows], B, C[:rows], w.alpha, w.beta)
    probe = time.perf_counter() - t0
    rows = int(max(8, min(w.M, rows * max(1.0, (target_s - probe) / max(probe, 1e-3)))))
    t0 = time.perf_counter()
    oracle.sgemm(A[:rows], B, C[:rows], w.alpha, w.beta)
    dt = time.perf_counter() - t0
    # Where the whole product takes well under the target, repeat it (the
    # same call on the same inputs) until about the target has been spent.
    passes = 1
    while rows == w.M and dt < 0.9 * target_s and dt / passes < target_s:
        oracle.sgemm(A, B, C, w.alpha, w.beta)
        passes += 1
        dt = time.perf_counter() - t0
    gflops = 2.0 * rows * w.N * w.K * passes / dt / 1e9
    what = (f"first {rows} of {w.M} rows of the same {w.M}x{w.N}x{w.K} product" if rows < w.M
            else f"the whole {w.M}x{w.N}x{w.K} product, {passes} pass{'es' if passes > 1 else ''}")
    return {"value": round(gflops, 3), "unit": "GFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} (fp64 accumulation, OpenMP over rows), {dt:.1f} s"}


def oracle_timing(inputs, model, max_seconds=20.0):
    """The oracle, as it stands, on every workload: the whole product where it
    takes at most `max_seconds`, else the first rows scaled to that time; one
    thread as well for the two smallest squares.  Reported only."""
    from oracle import oracle
    oracle.build(force=False)
    threads = oracle.max_threads()
    model_name = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model_name = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    out = []

    def run(w, A, B, C, nthreads):
        oracle.set_threads(nthreads)
        rows = min(w.M, 8)
        t0 = time.perf_counter()
        oracle.sgemm(A[:rows], B, C[:rows], w.alpha, w.beta)
        probe = max(time.perf_counter() - t0, 1e-4)
        rows = int(min(w.M, max(rows, rows * max_seconds / probe)))
        t0 = time.perf_counter()
        oracle.sgemm(A[:rows], B, C[:rows], w.alpha, w.beta)
        dt = time.perf_counter() - t0
        return {"workload": w.name, "threads": nthreads, "rows": rows, "of_rows": w.M,
                "seconds": round(dt, 4), "GFLOP/s": round(2.0 * rows * w.N * w.K / dt / 1e9, 3)}

    for name, w in inputs.WORKLOADS.items():
        A, B, C = inputs.make(w)
        out.append(run(w, A, B, C, threads))
        if name in ("sq256", "sq1024"):
            out.append(run(w, A, B, C, 1))
        print(json.dumps(out[-1]), file=sys.stderr, flush=True)
    oracle.set_threads(threads)
    print(json.dumps({"oracle_timing": out, "cores": threads, "cpu_model": model_name,
                      "kind": "oracle", "note": "fp64 accumulation, OpenMP over rows; reported only"}),
          flush=True)


def ladder(fg, inputs, model, w, dev, args):
    """Time the kernel ladder (the pages' progression rebuilt for wave64)."""
    import numpy as np
    import torch
    A, B, C = inputs.make(w)
    Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    C0 = torch.from_numpy(C).to(dev)
    Cd = C0.clone()
    stream = torch.cuda.current_stream(dev)
    names = {1: "shared-memory tiling, 1 output/lane, 32x32",
             2: "VALU 128x128x8, 8x8 per lane, A transposed, float4",
             3: "VALU warp tiling 128x64x16, 64x64 waves, 4x4 patches",
             4: "tuned MFMA dispatch"}
    out = {"ladder": [], "workload": w.name}
    flops = model.flops(w.M, w.N, w.K)
    for rung in (1, 2, 3, 4):
        reps = max(3, min(args.steps, 20))
        # Ten warm-ups per rung: the first launches after a switch run at a
        # lower clock.
        for _ in range(10):
            fg.ladder(rung, Ad, Bd, Cd, w.alpha, w.beta, stream=stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(reps):
            fg.ladder(rung, Ad, Bd, Cd, w.alpha, w.beta, stream=stream)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        ms = float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))
        out["ladder"].append({"rung": rung, "kernel": names[rung], "ms": round(ms, 4),
                              "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                              "pct_of_peak": round(100 * flops / (ms * 1e-3) / 1e12
                                                   / model.PEAK_FP32_TFLOPS, 2)})
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the benchmark runs the single-GPU kernel on exactly one GPU; "
              f"--gpus {args.gpus} (WORLD_SIZE={world}) is not supported", file=sys.stderr, flush=True)
        sys.exit(2)

    if args.oracle_timing:
        from fp32_gemm_amd import inputs, model
        oracle_timing(inputs, model)
        return

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration()
        return

    import fp32_gemm_amd as fg
    from fp32_gemm_amd import inputs, model

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if fg.device_check() != 0:
        raise SystemExit("bench.py: current device is not gfx950")
    if args.tile:
        want = tuple(int(x) for x in args.tile.split(","))
        ids = [c["id"] for c in fg.configs() if c["tuple"][:len(want)] == want]
        if not ids:
            raise SystemExit(f"bench.py: no compiled configuration {want}")
        args.cfg = ids[0]
    w = inputs.WORKLOADS[args.workload]
    if args.ladder:
        ladder(fg, inputs, model, w, dev, args)
        return
    A, B, C = inputs.make(w)
    Ad = torch.from_numpy(A).to(dev)
    Bd = torch.from_numpy(B).to(dev)
    C0 = torch.from_numpy(C).to(dev)
    total = args.warmup + args.steps
    # One pristine C per launch (cold in the caches, and beta * C never
    # compounds), within an 8 GiB budget; past it buffers are reused and the
    # timed ones are refilled after the warm-up.
    pool = max(1, min(total, (8 << 30) // max(1, C0.numel() * 4)))
    Cs = [C0.clone() for _ in range(pool)]
    stream = torch.cuda.current_stream(dev)
    plan = fg.binding.plan(w.M, w.N, w.K, Ad.data_ptr(), w.K, Bd.data_ptr(), w.N,
                           Cs[0].data_ptr(), w.N, args.cfg)
    info = fg.config_info(plan["cfg_id"])

    def step(i):
        fg.sgemm_ex(Ad, Bd, Cs[i % pool], w.alpha, w.beta, stream=stream, cfg_id=args.cfg)

    for i in range(args.warmup):
        step(i)
    if pool < total:
        # Buffers are reused: give the timed steps pristine C again.
        for i in range(args.steps):
            Cs[(args.warmup + i) % pool].copy_(C0)
    torch.cuda.synchronize()

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])  # ms
    avg_ms = float(ev[0].elapsed_time(ev[-1])) / args.steps

    # Parity of the last timed output against the oracle on sampled entries.
    from oracle import oracle
    last = Cs[(total - 1) % pool].cpu().numpy()
    rows, cols = inputs.sample_indices(w.M, w.N, 2000, seed=w.seed + 100)
    _, e64 = oracle.entries(rows, cols, A, B, C, w.alpha, w.beta)
    parity = oracle.rel_error(last[rows, cols], e64, w.K, np.abs(A).max(), np.abs(B).max())

    flops = model.flops(w.M, w.N, w.K)
    value = flops * args.steps / wall / 1e9
    achieved = flops / (avg_ms * 1e-3) / 1e12
    peak = model.PEAK_FP32_TFLOPS
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tr = json.load(f)
        key = f"{args.workload}:{'/'.join(map(str, info['tuple']))}"
        if key in tr:
            traffic = tr[key]["bytes_per_launch"]

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"sgemm {w.M}x{w.N}x{w.K} alpha={w.alpha} beta={w.beta} "
                        f"A,B ~ {'U[-1,1]' if w.dist == 'uniform' else 'N(0,1)'} seed {w.seed}",
            "M": w.M, "N": w.N, "K": w.K, "alpha": w.alpha, "beta": w.beta,
            "cfg_id": info["id"], "path": info["path_name"], "tile": list(info["tuple"]),
            "vector_variant": plan["vector_variant"], "grid": plan["grid"],
        },
        "pct_of_peak": round(100.0 * value / 1e3 / peak, 2),
        "roofline": {
            "bound": "mfma" if info["path"] != 0 else "alu",
            "achieved": round(achieved, 2),
            "peak": round(peak, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
        },
        "timing_ms": {"event_avg": round(avg_ms, 4), "median": round(float(np.median(per)), 4),
                      "min": round(float(per.min()), 4), "max": round(float(per.max()), 4),
                      "spread": round(float((per.max() - per.min()) / np.median(per)), 4)},
        "parity_err": parity,
    }
    if not args.no_context:
        # The same warm-up and launch count as the timed kernel above, so the
        # vendor library is compared at its steady clock too.  torch.mm is
        # the plain product (no alpha, no beta read of C).
        Cm = torch.empty_like(C0)
        mm_warm, mm_reps = max(args.warmup, 10), max(args.steps, 20)
        for _ in range(mm_warm):
            torch.mm(Ad, Bd, out=Cm)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(mm_reps):
            torch.mm(Ad, Bd, out=Cm)
        e1.record(stream)
        torch.cuda.synchronize()
        mm = flops / (e0.elapsed_time(e1) / mm_reps * 1e-3) / 1e12
        # Cold caches: a 512 MiB write between launches evicts A, B and C
        # from the L2s and the 256 MiB Infinity Cache; each launch is timed
        # alone, on a pristine C written before the eviction.  Three untimed
        # launches before each eviction hold the clock: isolated launches
        # after a synchronisation otherwise start ~25 % slower and take about
        # thirty launches to recover, whatever the caches hold.
        scratch = torch.empty(128 << 20, dtype=torch.float32, device=dev)
        spare = torch.empty_like(C0)

        def cold_times(f):
            t = []
            for i in range(10):
                Cs[i % pool].copy_(C0)
                for _ in range(3):
                    f(spare)
                scratch.fill_(float(i))
                e0.record(stream)
                f(Cs[i % pool])
                e1.record(stream)
                torch.cuda.synchronize()
                t.append(e0.elapsed_time(e1))
            return float(np.median(t))

        cold_ms = cold_times(lambda Cx: fg.sgemm_ex(Ad, Bd, Cx, w.alpha, w.beta, stream=stream,
                                                    cfg_id=args.cfg))
        cold_mm_ms = cold_times(lambda Cx: torch.mm(Ad, Bd, out=Cx))
        del scratch, spare
        out["context"] = {"torch_mm_tflops": round(mm, 2),
                          "this_vs_torch_mm": round(achieved / mm, 3),
                          "torch_mm_launches": {"warmup": mm_warm, "timed": mm_reps},
                          "cold_cache_tflops": round(flops / (cold_ms * 1e-3) / 1e12, 2),
                          "cold_cache_ms_median": round(cold_ms, 4),
                          "torch_mm_cold_cache_tflops": round(flops / (cold_mm_ms * 1e-3) / 1e12, 2),
                          "note": "vendor BLAS timing (plain A*B), context only; never used for "
                                  "dispatch or parity"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, A, B, C, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
