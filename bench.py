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
    ap.add_argument("--ramp", action="store_true",
                    help="only time, after an idle gap, 30 back-to-back launches of this library "
                         "and of the vendor library one by one (clock ramp; one JSON line)")
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


# The sources that make up the kernels' code (not the dispatch table):
# traffic counters in profiles/traffic.json count only for the kernel code
# they were taken on.
KERNEL_SOURCES = ("sgemm_kernels.hpp", "tile_maps.hpp", "tile_config.hpp", "registry.hpp")


def kernel_fingerprint():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "fp32_gemm_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        return "unknown"


def oracle_product(w, A, B, C, target_s):
    """The oracle, as it stands, on the whole product of the same workload:
    one pass gives the fp64 result every GPU output is checked against; more
    passes of the same call (when target_s > 0) bring the CPU sample to about
    target_s seconds for the reported baseline.  Returns (C64, baseline)."""
    from oracle import oracle
    oracle.build(force=False)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    _, C64 = oracle.sgemm(A, B, C, w.alpha, w.beta)
    dt = time.perf_counter() - t0
    passes = 1
    while target_s > 0 and dt < 0.9 * target_s and dt / passes < target_s:
        oracle.sgemm(A, B, C, w.alpha, w.beta)
        passes += 1
        dt = time.perf_counter() - t0
    gflops = 2.0 * w.M * w.N * w.K * passes / dt / 1e9
    base = {"value": round(gflops, 3), "unit": "GFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"the whole {w.M}x{w.N}x{w.K} product, {passes} pass"
                      f"{'es' if passes > 1 else ''} (fp64 accumulation, OpenMP over rows), "
                      f"{dt:.1f} s; the first pass is also the parity reference"}
    return C64, base


def oracle_timing(inputs, model, max_seconds=20.0):
    """The oracle, as it stands, on every workload: the whole product where it
    takes at most `max_seconds`, else the first rows scaled to that time; one
    thread as well for the two smallest squares.  Reported only."""
    from oracle import oracle
    oracle.build(force=False)
    threads = oracle.max_threads()
    model_name = cpu_model()
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


def kernel_resources(fg, info, plan, dev):
    """Registers, scratch, LDS and residency of the kernel the launch ran."""
    import torch
    vec = bool(plan["vector_variant"])
    attr = fg.binding.kernel_attributes(info["id"], 1 if vec else 0)
    rep = next((c for c in fg.configs() if c["id"] == info["id"]), {})
    res = rep.get("resources_vec" if vec else "resources_scalar") or {}
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    return {"vgprs": res.get("VGPRs"), "agprs": res.get("AGPRs"),
            "sgprs": res.get("TotalSGPRs"), "scratch_bytes_per_lane": attr["scratch_bytes"],
            "lds_bytes": attr["lds_bytes"], "waves_per_simd": res.get("Occupancy"),
            "workgroups_per_cu": plan["slots"] // cus if plan["slots"] else None,
            "compute_units": cus, "threads_per_workgroup": info["NT"]}


def ramp(fg, inputs, w, dev, launches=30, idle_s=3.0, rounds=2):
    """Per-launch times of back-to-back launches after an idle gap, for this
    library and for the vendor library in turn: how long the clock takes to
    settle, and whether it settles the same way for both."""
    import numpy as np
    import torch
    A, B, C = inputs.make(w)
    Ad, Bd, C0 = (torch.from_numpy(x).to(dev) for x in (A, B, C))
    Cs = [C0.clone() for _ in range(launches)]
    stream = torch.cuda.current_stream(dev)
    fg.sgemm_ex(Ad, Bd, Cs[0], w.alpha, w.beta, stream=stream)   # first-use set-up, untimed
    torch.mm(Ad, Bd, out=Cs[0])
    out = {"workload": w.name, "launches": launches, "idle_s": idle_s, "series": []}
    for r in range(rounds):
        for name, f in (("vendor torch.mm", lambda Cx: torch.mm(Ad, Bd, out=Cx)),
                        ("this library", lambda Cx: fg.sgemm_ex(Ad, Bd, Cx, w.alpha, w.beta,
                                                               stream=stream))):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(launches + 1)]
            torch.cuda.synchronize()
            time.sleep(idle_s)
            ev[0].record(stream)
            for i in range(launches):
                f(Cs[i])
                ev[i + 1].record(stream)
            torch.cuda.synchronize()
            ms = [round(ev[i].elapsed_time(ev[i + 1]), 4) for i in range(launches)]
            out["series"].append({"round": r, "kernel": name, "ms": ms,
                                  "first5_median": float(np.median(ms[:5])),
                                  "last5_median": float(np.median(ms[-5:]))})
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
    if args.ramp:
        ramp(fg, inputs, w, dev)
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

    last = Cs[(total - 1) % pool].cpu().numpy()

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
        if key in tr and tr[key].get("kernel") == kernel_fingerprint():
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
                      "spread": round(float((per.max() - per.min()) / np.median(per)), 4),
                      "per_launch": [round(float(x), 4) for x in per]},
        "kernel": kernel_resources(fg, info, plan, dev),
    }
    if not args.no_context:
        # Warm caches: the two libraries alternate in batches of five
        # launches (eight batches each, after a warm-up of each), so clock
        # and temperature drift affect them alike.  torch.mm is the plain
        # product (no alpha, no beta read of C).
        Cm = torch.empty_like(C0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ours = lambda Cx: fg.sgemm_ex(Ad, Bd, Cx, w.alpha, w.beta, stream=stream, cfg_id=args.cfg)
        vendor = lambda Cx: torch.mm(Ad, Bd, out=Cx)
        mm_warm, batches, batch = 10, 8, 5
        for _ in range(mm_warm):
            vendor(Cm)
        warm, warm_mm = [], []
        use = 0
        for _ in range(batches):
            for f, acc in ((ours, warm), (vendor, warm_mm)):
                torch.cuda.synchronize()
                e0.record(stream)
                for _ in range(batch):
                    f(Cs[use % pool] if f is ours else Cm)
                    use += 1
                e1.record(stream)
                torch.cuda.synchronize()
                acc.append(e0.elapsed_time(e1) / batch)
        warm_ms, mm_ms = float(np.median(warm)), float(np.median(warm_mm))
        mm = flops / (mm_ms * 1e-3) / 1e12
        # Cold caches: a 512 MiB write between launches evicts A, B and C
        # from the L2s and the 256 MiB Infinity Cache; each launch is timed
        # alone, on a pristine C written before the eviction.  Three untimed
        # launches before each eviction hold the clock (isolated launches
        # after a synchronisation otherwise start slower), and the two
        # libraries alternate launch by launch, so a clock still settling
        # favours neither.
        scratch = torch.empty(128 << 20, dtype=torch.float32, device=dev)
        spare = torch.empty_like(C0)

        def cold_once(f, i):
            Cs[i % pool].copy_(C0)
            for _ in range(3):
                f(spare)
            scratch.fill_(float(i))
            e0.record(stream)
            f(Cs[i % pool])
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)

        cold, cold_mm = [], []
        for i in range(10):
            cold.append(cold_once(ours, i))
            cold_mm.append(cold_once(vendor, i))
        cold_ms, cold_mm_ms = float(np.median(cold)), float(np.median(cold_mm))
        del scratch, spare
        out["context"] = {"interleaved_tflops": round(flops / (warm_ms * 1e-3) / 1e12, 2),
                          "torch_mm_tflops": round(mm, 2),
                          "this_vs_torch_mm": round(mm_ms / warm_ms, 3),
                          "interleaved_launches": {"torch_mm_warmup": mm_warm, "batches": batches,
                                                   "per_batch": batch},
                          "cold_cache_tflops": round(flops / (cold_ms * 1e-3) / 1e12, 2),
                          "cold_cache_ms_median": round(cold_ms, 4),
                          "torch_mm_cold_cache_tflops": round(flops / (cold_mm_ms * 1e-3) / 1e12, 2),
                          "cold_cache_this_vs_torch_mm": round(cold_mm_ms / cold_ms, 3),
                          "note": "vendor BLAS timing (plain A*B), context only; never used for "
                                  "dispatch or parity"}
    # Parity: every output of the last timed launch against the oracle's
    # whole product (the first pass of the CPU baseline's sample).
    from oracle import oracle
    C64, base = oracle_product(w, A, B, C, 0.0 if args.no_cpu_baseline else args.cpu_seconds)
    out["parity_err"] = oracle.rel_error(last, C64, w.K, np.abs(A).max(), np.abs(B).max())
    out["parity_outputs"] = f"all {w.M * w.N} outputs of the last timed launch"
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = base
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
