"""Autotuner over the compiled tile tuples.

For each shape and each compiled configuration whose kernels do not spill:
launch once on integer-valued inputs and check sampled outputs exactly
(every partial sum of small integers is exact in fp32, so a correct kernel
matches int64 arithmetic bit for bit), then warm up and time on the
workload's own inputs with HIP events.  The fastest few are re-timed with the
longer protocol and the winner per shape goes into the dispatch table.  The
page "Autotuning: Searching the Tile-Shape Space" (code listing and section
"What The Sweep Found") describes the same launch / verify / time / record
loop with a shorter warm-up for the sweep than for the final benchmark.

    python -m fp32_gemm_amd.tune [--workloads a,b] [--out results.jsonl]
                                 [--table-out tuned_table.inc]
    python -m fp32_gemm_amd.tune --workloads a,b --retime results.jsonl[,more.jsonl]
                                 [--top 5] [--table-out tuned_table.inc]
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np
import torch

from . import binding as fg
from . import inputs, model

SHORT = (3, 10)   # warm-up, timed reps during the sweep
LONG = (20, 60)   # re-timing of the finalists


def _time(fn, warm, reps, stream):
    for _ in range(warm):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(reps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])
    return float(np.median(per)), float(per.min()), float(per.max())


def _exact_inputs(M, N, K, dev, samples=1500):
    """Integer-valued inputs on the device and the expected sampled outputs
    from int64 arithmetic; drawn once per shape and shared by every
    configuration's check."""
    A, B, C = inputs.make_small_int(M, N, K, seed=4242)
    rows, cols = inputs.sample_indices(M, N, samples, seed=4243)
    s = np.einsum("ij,ji->i", A[rows].astype(np.int64), B[:, cols].astype(np.int64))
    want = (0.5 * s + 3.0 * C[rows, cols].astype(np.float64)).astype(np.float32)
    dev_in = tuple(torch.from_numpy(x).to(dev) for x in (A, B, C))
    return dev_in, torch.from_numpy(rows).to(dev), torch.from_numpy(cols).to(dev), want


def _exact_check(cfg_id, chk):
    """Sampled outputs of one configuration on the shared integer inputs must
    equal the int64 result bit for bit."""
    (Ad, Bd, C0), rows, cols, want = chk
    Cd = C0.clone()
    fg.sgemm_ex(Ad, Bd, Cd, 0.5, 3.0, cfg_id=cfg_id)
    got = Cd[rows, cols].cpu().numpy()
    return bool(np.array_equal(got.view(np.uint32), want.view(np.uint32)))


def usable_configs(vector_variant=True):
    """Compiled configurations whose kernel for this variant does not spill."""
    out = []
    for c in fg.configs():
        r = c["resources_vec"] if vector_variant else c["resources_scalar"]
        if r is None or r.get("ScratchSize", 1) > 0:
            continue
        out.append(c)
    return out


def tune_shape(w, dev, configs, log, finalists=6, progress=None):
    """Sweep one shape: exact check and short timing of every configuration,
    then the `finalists` fastest of each path re-timed interleaved with the
    long protocol, path by path.  Returns (best overall, best per path, all
    records)."""
    A, B, C = inputs.make(w)
    Ad, Bd = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    Cd = torch.from_numpy(C).to(dev)
    stream = torch.cuda.current_stream(dev)
    flops = model.flops(w.M, w.N, w.K)
    results = []
    chk = _exact_inputs(w.M, w.N, w.K, dev)
    t0 = time.time()
    for i, c in enumerate(configs):
        ok = _exact_check(c["id"], chk)
        rec = {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "cfg_id": c["id"],
               "tuple": list(c["tuple"]), "path": c["path_name"], "exact": ok}
        if ok:
            med, lo, hi = _time(lambda: fg.sgemm_ex(Ad, Bd, Cd, w.alpha, w.beta, stream=stream,
                                                    cfg_id=c["id"]), *SHORT, stream)
            rec.update(ms=med, ms_min=lo, ms_max=hi, tflops=flops / (med * 1e-3) / 1e12,
                       protocol="short")
        results.append(rec)
        log(rec)
        if progress and (i + 1) % 50 == 0:
            progress(f"[tune] {w.name}: {i + 1}/{len(configs)} swept ({time.time() - t0:.0f} s)")
    by_path = {}
    for r in sorted((r for r in results if r["exact"]), key=lambda r: r["ms"]):
        by_path.setdefault(r["path"], []).append(r)
    # Each path's finalists are timed interleaved (one batch of each in turn,
    # repeated), so clock and temperature drift affect them alike.  The
    # paths are timed in separate groups: a VALU batch draws less power than
    # an MFMA batch, and alternating the two shifts the clock between
    # batches, which skewed the MFMA finalists' order by up to 2 %.
    warm, reps = LONG
    batch = 5
    for group in by_path.values():
        ok = group[:finalists]
        fns = [lambda r=r: fg.sgemm_ex(Ad, Bd, Cd, w.alpha, w.beta, stream=stream,
                                       cfg_id=r["cfg_id"]) for r in ok]
        for f in fns:
            for _ in range(warm):
                f()
        samples = [[] for _ in ok]
        for _ in range(reps // batch):
            for i, f in enumerate(fns):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(batch):
                    f()
                e1.record(stream)
                torch.cuda.synchronize()
                samples[i].append(e0.elapsed_time(e1) / batch)
        for r, smp in zip(ok, samples):
            med = float(np.median(smp))
            fin = dict(r, ms=med, ms_min=float(min(smp)), ms_max=float(max(smp)),
                       tflops=flops / (med * 1e-3) / 1e12, protocol="long")
            results.append(fin)
            log(fin)
    longs = [r for r in results if r.get("protocol") == "long"]
    best_by_path = {}
    for r in longs:
        if r["path"] not in best_by_path or r["ms"] < best_by_path[r["path"]]["ms"]:
            best_by_path[r["path"]] = r
    for path, b in best_by_path.items():
        b["swept"] = sum(1 for r in results if r.get("protocol") == "short" and r["path"] == path)
        b["failed_exact"] = sum(1 for r in results if not r["exact"] and r["path"] == path)
    best = min(longs, key=lambda r: r["ms"])
    return best, best_by_path, results


def write_summary(best_by_shape_path, path, command, finalists=6):
    """Markdown table of the best tuple per (shape, path)."""
    lines = ["# Autotuner winners per (shape, path)", "",
             f"Command: `{command}`", "",
             "Every compiled, non-spilling configuration of each path was checked exactly on "
             "integer-valued inputs and timed with the short protocol (3 warm-up, 10 timed "
             f"launches); the {finalists} fastest of each path were then re-timed interleaved, path "
             "by path (20 warm-up, 12 batches of 5). Times are the long protocol's median.", "",
             "| shape | path | swept | best tuple (BM,BN,BK,WM,WN,WNITER,TM,TN,NT,path,swz,opt) "
             "| ms | TFLOP/s | % of 157.3 |",
             "|---|---|---|---|---|---|---|"]
    for (shape, pth), b in best_by_shape_path.items():
        lines.append(f"| {shape} {b['M']}x{b['N']}x{b['K']} | {pth} | {b['swept']} | "
                     f"{','.join(str(x) for x in b['tuple'])} | {b['ms']:.4f} | "
                     f"{b['tflops']:.1f} | {100 * b['tflops'] / model.PEAK_FP32_TFLOPS:.1f} |")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def retime(names, shapes, dev, results_path, top, summary_path, command):
    """Interleaved re-timing, per shape, of the tuned dispatch's choice and the
    `top` fastest matrix-core tuples of previous sweeps (short protocol
    records in `results_path`, comma-separated files): 20 warm-up launches each, then rounds of one
    5-launch batch of each in turn (30 rounds; 12 above 2 * 4096^3 FLOP)."""
    recs = [json.loads(l) for path in results_path.split(",") for l in open(path)]
    ids = {c["tuple"]: c["id"] for c in fg.configs()}
    stream = torch.cuda.current_stream(dev)
    lines = ["# Tuned-table rules: interleaved re-timing against each shape's best sweep candidates", "",
             f"Command: `{command}`", "",
             f"Per shape: the tuned dispatch's choice (marked `*`) and the {top} fastest MFMA tuples of the "
             "sweep in the results file, 20 warm-up launches each, then rounds of one 5-launch batch of "
             "each in turn (30 rounds; 12 at 8192^3), on the workload's own inputs; medians in TFLOP/s.", "",
             "| shape | tuple (BM,BN,BK,WM,WN,WNITER,TM,TN,NT,path,swz,opt) | TFLOP/s |", "|---|---|---|"]
    results = {}
    for name in names:
        w = shapes[name]
        A, B, C = inputs.make(w)
        Ad, Bd, Cd = (torch.from_numpy(x).to(dev) for x in (A, B, C))
        chosen = fg.plan(w.M, w.N, w.K, Ad.data_ptr(), w.K, Bd.data_ptr(), w.N, Cd.data_ptr(),
                         w.N)["cfg_id"]
        chosen_t = fg.config_info(chosen)["tuple"]
        short = sorted((r for r in recs if r["workload"] == name and r.get("protocol") == "short"
                        and r["exact"] and r["path"] != "valu"), key=lambda r: r["ms"])
        cands = list(dict.fromkeys([chosen_t] + [tuple(r["tuple"]) for r in short[:top]]))
        cands = [t for t in cands if t in ids]
        fns = [lambda i=ids[t]: fg.sgemm_ex(Ad, Bd, Cd, w.alpha, w.beta, stream=stream, cfg_id=i)
               for t in cands]
        for f in fns:
            for _ in range(20):
                f()
        flops = model.flops(w.M, w.N, w.K)
        rounds = 30 if flops <= 2 * 4096 ** 3 else 12
        samples = [[] for _ in fns]
        for _ in range(rounds):
            for i, f in enumerate(fns):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(5):
                    f()
                e1.record(stream)
                torch.cuda.synchronize()
                samples[i].append(e0.elapsed_time(e1) / 5)
        rows = sorted(((flops / (float(np.median(v)) * 1e-3) / 1e12, t) for t, v in zip(cands, samples)),
                      reverse=True)
        results[(w.M, w.N, w.K)] = (chosen_t, rows, name)
        for tf, t in rows:
            mark = " *" if t == chosen_t else ""
            lines.append(f"| {name} | {','.join(str(x) for x in t)}{mark} | {tf:.2f} |")
            print(f"[retime] {name} {t}{mark} {tf:.2f} TFLOP/s", flush=True)
    if summary_path:
        with open(summary_path, "w") as f:
            f.write("\n".join(lines) + "\n")
    return results


_RULE = re.compile(r"^(\s*)\{(\d+), (\d+), (\d+), \{([-\d, ]+)\}\},\s*// ([^:]*):.*$")


def off_table(seed, dev, out_path, summary_path, command, count=36, aligned=False, shapes=None,
              mix="standard", n4=False):
    """Dispatch study on seeded shapes that no rule was tuned on.  The
    standard mix: a third each with M, N, K uniform in [512, 8192],
    log-uniform in [256, 16384], and M, N in [1024, 8192] with K in
    [64, 1024] (shapes above 8192^3's work skipped).  The large mix, all
    log-uniform: a third each with M, N, K in [4096, 16384], M, N in
    [4096, 16384] with K in [16, 512], and M, N in [2048, 16384] with K in
    [8192, 65536] (shapes above 16384^3's work skipped).  The grid mix: M and
    N drawn from 512, 1024, 1536, 2048, 3072, 4096, 6144, 8192, 12288 and
    16384, K from 64, 128, 256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096,
    6144, 8192, 12288 and 16384 (above 16384^3's work skipped; each shape
    once).  The short-K grid, not drawn but enumerated (seed and count
    unused): every M, N in 4096, 6144, 8192, 12288, 16384 with K in 128,
    192, 256, 384, 512, 768.  With `aligned`, N
    and K are rounded up to multiples of 4, so every shape runs the float4
    variant; with `n4`, N is rounded up to a multiple of 4 and K moved to the
    next number when it is one (the scalar variant with 16-byte B loads).  Per shape the tuned dispatch's choice, the tuple of every
    table rule and torch.mm are timed interleaved (3 warm-up launches each,
    then 6 rounds of one 3-launch batch of each in turn; A, B normal, beta
    = 0); the summary reports the dispatch's rate against the best rule's
    and against torch.mm.  `shapes`, a list of (M, N, K), replaces the
    seeded shapes."""
    rules = []
    for line in open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc",
                                  "tuned_table.inc")):
        m = _RULE.match(line)
        if m:
            rules.append(tuple(int(x) for x in m.group(5).split(", ")))
    ids = {c["tuple"]: c["id"] for c in fg.configs()}
    rng = np.random.default_rng(seed)
    stream = torch.cuda.current_stream(dev)
    recs = []
    def log_uniform(lo, hi):
        return int(round(np.exp(rng.uniform(np.log(lo), np.log(hi)))))

    cap = 16384 ** 3 if mix in ("large", "grid") else 8192 ** 3
    grid_mn = (512, 1024, 1536, 2048, 3072, 4096, 6144, 8192, 12288, 16384)
    grid_k = (64, 128, 256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096, 6144, 8192, 12288, 16384)
    done = set()
    if mix == "grid-short-k":
        shapes = [(M, N, K) for M in (4096, 6144, 8192, 12288, 16384)
                  for N in (4096, 6144, 8192, 12288, 16384) for K in (128, 192, 256, 384, 512, 768)]
    for i in range(len(shapes) if shapes else count):
        if shapes:
            M, N, K = shapes[i]
        elif mix == "grid":
            M, N = (int(x) for x in rng.choice(grid_mn, 2))
            K = int(rng.choice(grid_k))
            if (M, N, K) in done:
                continue
            done.add((M, N, K))
        elif mix == "large":
            if i % 3 == 0:
                M, N, K = (log_uniform(4096, 16384) for _ in range(3))
            elif i % 3 == 1:
                M, N, K = log_uniform(4096, 16384), log_uniform(4096, 16384), log_uniform(16, 512)
            else:
                M, N, K = log_uniform(2048, 16384), log_uniform(2048, 16384), log_uniform(8192, 65536)
        elif i % 3 == 0:
            M, N, K = (int(x) for x in rng.integers(512, 8193, 3))
        elif i % 3 == 1:
            M, N, K = (log_uniform(256, 16384) for _ in range(3))
        else:
            M, N = (int(x) for x in rng.integers(1024, 8193, 2))
            K = int(rng.integers(64, 1025))
        if aligned:
            N, K = -(-N // 4) * 4, -(-K // 4) * 4
        if n4:
            N, K = -(-N // 4) * 4, K + 1 if K % 4 == 0 else K
        if not shapes and M * N * K > cap:
            continue
        A = torch.randn(M, K, device=dev)
        B = torch.randn(K, N, device=dev)
        C = torch.randn(M, N, device=dev)
        chosen = fg.plan(M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N)["cfg_id"]
        cands = sorted({ids[t] for t in rules if t in ids} | {chosen})
        fns = {c: (lambda c=c: fg.sgemm_ex(A, B, C, 1.0, 0.0, stream=stream, cfg_id=c)) for c in cands}
        Cm = torch.empty_like(C)
        fns["torch.mm"] = lambda: torch.mm(A, B, out=Cm)
        for f in fns.values():
            for _ in range(3):
                f()
        samples = {k: [] for k in fns}
        for _ in range(6):
            for k, f in fns.items():
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(3):
                    f()
                e1.record(stream)
                torch.cuda.synchronize()
                samples[k].append(e0.elapsed_time(e1) / 3)
        rate = {k: model.flops(M, N, K) / (float(np.median(v)) * 1e-3) / 1e12 for k, v in samples.items()}
        best = max(cands, key=lambda c: rate[c])
        rec = dict(M=M, N=N, K=K, vec=bool(N % 4 == 0 and K % 4 == 0), chosen=fg.config_info(chosen)["tuple"],
                   chosen_tflops=round(rate[chosen], 2), best=fg.config_info(best)["tuple"],
                   best_tflops=round(rate[best], 2), torch_tflops=round(rate["torch.mm"], 2))
        # Every candidate's rate and launch plan, so another selection policy
        # can be scored against the same timings.
        key = lambda c: ",".join(map(str, fg.config_info(c)["tuple"]))
        rec["rates"] = {key(c): round(rate[c], 2) for c in cands}
        rec["plans"] = {key(c): {k: v for k, v in fg.plan(M, N, K, A.data_ptr(), K, B.data_ptr(), N,
                                                          C.data_ptr(), N, c).items()
                                 if k in ("grid", "slots", "tiles_full", "splits")} for c in cands}
        recs.append(rec)
        print(f"[off-table] {M}x{N}x{K} dispatch {rec['chosen_tflops']:.1f}, best rule "
              f"{rec['best_tflops']:.1f}, torch.mm {rec['torch_tflops']:.1f}", flush=True)
    if out_path:
        with open(out_path, "w") as f:
            for r in recs:
                f.write(json.dumps(r) + "\n")
    if summary_path:
        g = lambda xs: float(np.exp(np.mean(np.log(xs))))
        of_best = [r["chosen_tflops"] / r["best_tflops"] for r in recs]
        vs_torch = [r["chosen_tflops"] / r["torch_tflops"] for r in recs]
        kind = "aligned " if aligned else "N % 4 == 0 scalar-variant " if n4 else ""
        title = (f"the {mix} shapes" if mix == "grid-short-k" else "given shapes" if shapes
                 else f"seeded {kind}off-table shapes ({mix} mix, seed {seed})")
        lines = [f"# Dispatch on {title}", "", f"Command: `{command}`", "",
                 off_table.__doc__.split("\n\n")[0].replace("\n    ", " ").strip(), "",
                 f"{len(recs)} shapes ({sum(not r['vec'] for r in recs)} scalar-variant). The dispatch's "
                 f"choice reaches {g(of_best):.3f} of the best table rule's rate (geometric mean; worst "
                 f"{min(of_best):.3f}) and {g(vs_torch):.3f}x torch.mm (worst {min(vs_torch):.3f}x).", "",
                 "| M | N | K | variant | dispatch tuple | TFLOP/s | best rule tuple | TFLOP/s | torch.mm |",
                 "|---|---|---|---|---|---|---|---|---|"]
        for r in recs:
            lines.append(f"| {r['M']} | {r['N']} | {r['K']} | {'float4' if r['vec'] else 'scalar'} | "
                         f"{','.join(map(str, r['chosen']))} | {r['chosen_tflops']:.1f} | "
                         f"{','.join(map(str, r['best']))} | {r['best_tflops']:.1f} | {r['torch_tflops']:.1f} |")
        with open(summary_path, "w") as f:
            f.write("\n".join(lines) + "\n")
    return recs


def write_rate_table(records, path, command):
    """The measured-rate table that the dispatch consults off the rules: per
    variant, one row per shape of the off-table studies' records, with each
    column tile's rate as a percentage (at least 1) of the row's fastest
    column.  The columns are the tuples timed on every shape.  A shape
    measured twice keeps its first record."""
    rows, seen = [], set()
    for r in records:
        key = (r["M"], r["N"], r["K"])
        if key in seen:
            continue
        seen.add(key)
        rows.append(r)
    if not rows:
        raise ValueError("no records with rates")
    common = set(rows[0]["rates"])
    for r in rows[1:]:
        common &= set(r["rates"])
    cols = sorted(common, key=lambda t: tuple(int(x) for x in t.split(",")))
    lines = [
        "// measured_rates.inc -- measured-rate table for shapes off the rules.",
        "//",
        f"// Written by `{command}`",
        "// from off-table dispatch studies (tune.py --off-table): each row is a",
        "// seeded shape, with every column tile's rate there as a percentage of",
        "// the row's fastest column (at least 1); kScalarRows hold shapes that run",
        "// the scalar variant, kVectorRows shapes that run the float4 variant.",
        "// select_config in sgemm_api.hip describes how the dispatch reads them.",
        "// Tile order: {BM, BN, BK, WM, WN, WNITER, TM, TN, NT, path, swz, opt}.",
        "",
        "static constexpr Tile kRateTiles[] = {",
    ]
    for i, t in enumerate(cols):
        lines.append("    {%s},  // column %d" % (t.replace(",", ", "), i))
    lines.append("};")
    counts = {}
    for name, vec in (("kScalarRows", False), ("kVectorRows", True)):
        sel = sorted((r for r in rows if bool(r["vec"]) == vec), key=lambda r: (r["M"], r["N"], r["K"]))
        counts[vec] = len(sel)
        lines += ["", f"static const RateRow {name}[] = {{"]
        for r in sel:
            best = max(r["rates"][t] for t in cols)
            pct = [max(1, int(round(100.0 * r["rates"][t] / best))) for t in cols]
            lines.append("    {%d, %d, %d, {%s}},  // best %.1f TFLOP/s" % (
                r["M"], r["N"], r["K"], ", ".join(map(str, pct)), best))
        if not sel:
            lines.append("    {0, 0, 0, {}},  // none measured")
        lines.append("};")
    lines.append("")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return cols, counts[False], counts[True]


_RATE_ROW = re.compile(r"^(\s*)\{(\d+), (\d+), (\d+), \{([\d, ]+)\}\},\s*// best ([\d.]+) TFLOP/s$")


def read_rate_table(path):
    """The columns of a measured-rate table (tuples) and its rows per
    variant: {"scalar": [(M, N, K, pcts)], "vector": [...]}."""
    cols, rows, kind = [], {"scalar": [], "vector": []}, None
    for line in open(path):
        if "// column" in line:
            cols.append(tuple(int(x) for x in line.split("{")[1].split("}")[0].split(",")))
        elif "kScalarRows[]" in line:
            kind = "scalar"
        elif "kVectorRows[]" in line:
            kind = "vector"
        else:
            m = _RATE_ROW.match(line.rstrip("\n"))
            if m and kind:
                rows[kind].append((int(m.group(2)), int(m.group(3)), int(m.group(4)),
                                   [int(x) for x in m.group(5).split(", ")]))
    return cols, rows


def retime_rate_column(dev, path, column, kind="scalar"):
    """Re-times one column of the measured-rate table on every row of one
    variant, beside the row's fastest other column, with the off-table
    studies' protocol (A, B, C ~ N(0,1), beta = 0; 3 warm-up launches each,
    then 6 rounds of one 3-launch batch of each in turn).  For a column
    whose kernel changed since the table was measured.  Scalar rows with
    N % 4 == 0 are skipped: such shapes run the scalar kernels with 16-byte
    B loads, while the dispatch reads the scalar rows only for N % 4 != 0.
    Returns {(M, N, K): (column rate, anchor column, anchor rate)} in
    TFLOP/s."""
    cols, rows = read_rate_table(path)
    ids = {c["tuple"]: c["id"] for c in fg.configs()}
    stream = torch.cuda.current_stream(dev)
    out = {}
    for M, N, K, pct in rows[kind]:
        if kind == "scalar" and N % 4 == 0:
            continue
        anchor = max((j for j in range(len(cols)) if j != column), key=lambda j: pct[j])
        A = torch.randn(M, K, device=dev)
        B = torch.randn(K, N, device=dev)
        C = torch.randn(M, N, device=dev)
        fns = [lambda c=ids[cols[j]]: fg.sgemm_ex(A, B, C, 1.0, 0.0, stream=stream, cfg_id=c)
               for j in (column, anchor)]
        for f in fns:
            for _ in range(3):
                f()
        samples = [[], []]
        for _ in range(6):
            for i, f in enumerate(fns):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(3):
                    f()
                e1.record(stream)
                torch.cuda.synchronize()
                samples[i].append(e0.elapsed_time(e1) / 3)
        r = [model.flops(M, N, K) / (float(np.median(v)) * 1e-3) / 1e12 for v in samples]
        out[(M, N, K)] = (round(r[0], 2), anchor, round(r[1], 2))
        print(f"[rate-column] {M}x{N}x{K} column {column} {r[0]:.1f}, column {anchor} {r[1]:.1f}",
              flush=True)
    return out


def refresh_rate_column(path, column, kind, retimed, command):
    """Rewrites the rows of one variant that `retimed` covers: the column's
    percentage becomes its new rate over its anchor column's, both timed
    side by side, times the anchor's stored percentage; where that passes
    100 the row is rescaled so that its fastest column is 100 again (every
    percentage at least 1).  The other columns keep their ratios, and the
    command joins the table's header.  Scalar rows with N % 4 == 0 are left
    as they are, as retime_rate_column skips them.  Returns the rows whose
    fastest column changed."""
    lines = open(path).read().split("\n")
    out, cur, moved = [], None, []
    for line in lines:
        if "kScalarRows[]" in line:
            cur = "scalar"
        elif "kVectorRows[]" in line:
            cur = "vector"
        m = _RATE_ROW.match(line)
        key = tuple(int(m.group(i)) for i in (2, 3, 4)) if m else None
        if m and cur == kind and key in retimed and not (kind == "scalar" and key[1] % 4 == 0):
            pct = [int(x) for x in m.group(5).split(", ")]
            rate, anchor, anchor_rate = retimed[key]
            rel = [float(x) for x in pct]
            rel[column] = pct[anchor] * rate / anchor_rate
            top = max(rel)
            new = [max(1, int(round(100.0 * x / top))) for x in rel]
            if new.index(100) != pct.index(100):
                moved.append(key)
            best = float(m.group(6)) * top / 100.0
            line = "%s{%d, %d, %d, {%s}},  // best %.1f TFLOP/s" % (
                m.group(1), *key, ", ".join(map(str, new)), best)
        out.append(line)
    at = next(i for i, l in enumerate(out) if l.startswith("// Tile order"))
    out[at:at] = [f"// Column {column} of the {kind} rows re-timed by `{command}`"]
    with open(path, "w") as f:
        f.write("\n".join(out))
    return moved


def write_rate_table_gap(swept, path, command):
    """Markdown table: per swept shape, the fastest of every swept tuple
    against the fastest tile of the measured-rate table (short protocol)."""
    table = set()
    for line in open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc",
                                  "measured_rates.inc")):
        if "// column" in line:
            table.add(tuple(int(x) for x in line.split("{")[1].split("}")[0].split(",")))
    lines = ["# The measured-rate table's tiles against a sweep of every tuple", "",
             f"Command: `{command}`", "",
             "Per shape, every swept tuple was checked exactly and timed with the short protocol "
             "(3 warm-up, 10 timed launches; A, B ~ N(0,1), beta = 0); the fastest of them against "
             "the fastest of the measured-rate table's tiles.", "",
             "| shape | swept | fastest tuple | TFLOP/s | fastest table tile | TFLOP/s | ratio |",
             "|---|---|---|---|---|---|---|"]
    for name, rs in swept.items():
        top = max(rs, key=lambda r: r["tflops"])
        tab = [r for r in rs if tuple(r["tuple"]) in table]
        tb = max(tab, key=lambda r: r["tflops"]) if tab else None
        lines.append(f"| {name} | {len(rs)} | {','.join(map(str, top['tuple']))} | {top['tflops']:.1f} | "
                     + (f"{','.join(map(str, tb['tuple']))} | {tb['tflops']:.1f} | "
                        f"{tb['tflops'] / top['tflops']:.3f} |" if tb else "- | - | - |"))
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def update_table(path, results, lead=0.01):
    """Rewrites the rules of the re-timed shapes in an existing table: a rule
    moves to the fastest re-timed tuple only where that tuple leads the
    rule's own by more than `lead` (the re-timing's spread between runs is
    about 1 %); every rule re-timed gets its measured rate in its comment.
    A re-timed shape without a rule gets one, with its fastest tuple, at the
    end of the table.  Rules of other shapes and the default tiles are left
    as they are."""
    out, changed, seen = [], [], set()
    in_rules = False
    with open(path) as f:
        text = f.read()
    for line in text.split("\n"):
        m = _RULE.match(line)
        in_rules = in_rules or m is not None
        key = tuple(int(m.group(i)) for i in (2, 3, 4)) if m else None
        if key in results:
            seen.add(key)
            chosen, rows = results[key][:2]
            rate = {t: tf for tf, t in rows}
            best_tf, best = rows[0]
            pick = best if best_tf > rate[chosen] * (1 + lead) else chosen
            if pick != chosen:
                changed.append((key, chosen, pick))
            line = "%s{%d, %d, %d, {%s}},  // %s: %.1f TFLOP/s (re-timed)" % (
                m.group(1), *key, ", ".join(str(x) for x in pick), m.group(6), rate[pick])
        if in_rules and line.startswith("};"):
            in_rules = False
            for key, (chosen, rows, name) in results.items():
                if key in seen:
                    continue
                best_tf, best = rows[0]
                out.append("    {%d, %d, %d, {%s}},  // %s (tuning only): %.1f TFLOP/s (re-timed)" % (
                    *key, ", ".join(str(x) for x in best), name, best_tf))
                changed.append((key, None, best))
                seen.add(key)
        out.append(line)
    with open(path, "w") as f:
        f.write("\n".join(out))
    return changed


def write_table(best_by_shape, path, defaults):
    lines = [
        "// tuned_table.inc -- dispatch table for the tuned choice of tile tuple.",
        "//",
        "// kTuned lists shapes with the tuple the autotuner measured fastest on",
        "// them (fp32_gemm_amd/tune.py); other shapes choose among the rules, or",
        "// from the measured-rate table of measured_rates.inc, as select_config in",
        "// sgemm_api.hip describes.  Tuple order:",
        "// {BM, BN, BK, WM, WN, WNITER, TM, TN, NT, path, swz, opt}.",
        "",
        "static const TunedRule kTuned[] = {",
    ]
    for b in best_by_shape:
        t = b["tuple"]
        lines.append("    {%d, %d, %d, {%s}},  // %s: %.3f ms, %.1f TFLOP/s" % (
            b["M"], b["N"], b["K"], ", ".join(str(x) for x in t), b["workload"], b["ms"],
            b["tflops"]))
    lines.append("};")
    lines.append("")
    for name, t in defaults:
        lines.append("static constexpr Tile %s{%s};" % (name, ", ".join(str(x) for x in t)))
    lines.append("")
    with open(path, "w") as f:
        f.write("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default=",".join(list(inputs.WORKLOADS) + list(inputs.TUNING_EXTRA)))
    ap.add_argument("--out", default="tune_results.jsonl")
    ap.add_argument("--table-out", default=None,
                    help="write the dispatch table from the sweep; with --retime, update the "
                         "re-timed shapes' rules in this existing table instead")
    ap.add_argument("--paths", default="valu,mfma32,mfma16")
    ap.add_argument("--prune-above", type=float, default=float("inf"),
                    help="shapes with more FLOP than this only try the best --keep configs per "
                         "path of the --prune-from shape's short sweep (default: no pruning)")
    ap.add_argument("--prune-from", default="sq4096",
                    help="the shape whose ranking prunes larger shapes (swept first)")
    ap.add_argument("--keep", type=int, default=32)
    ap.add_argument("--summary-out", default=None,
                    help="write a markdown table of the best tuple per (shape, path)")
    ap.add_argument("--top-from", default=None,
                    help="only try tuples ranked in the top --top of a previous results file "
                         "(per workload, short protocol)")
    ap.add_argument("--top", type=int, default=24)
    ap.add_argument("--filter", default=None,
                    help="Python expression over a config dict c (e.g. \"c['BK'] == 32\")")
    ap.add_argument("--finalists", type=int, default=6,
                    help="tuples per path re-timed interleaved with the long protocol; the "
                         "sweep's short timings are noisier than the gaps between the best tuples")
    ap.add_argument("--retime", default=None,
                    help="re-time, per shape in --workloads, the tuned dispatch's choice against the "
                         "--top fastest matrix-core tuples of these results files (comma-separated; "
                         "no sweep)")
    ap.add_argument("--best", default=None,
                    help="print the best tuple recorded for this workload in --out and exit")
    ap.add_argument("--off-table", type=int, default=None, metavar="SEED",
                    help="dispatch study on seeded shapes off the table (writes --out and "
                         "--summary-out), no sweep")
    ap.add_argument("--shapes", default=None,
                    help="shapes MxNxK, comma-separated: with --off-table, time these instead of "
                         "seeded ones; otherwise sweep them (instead of --workloads) and write to "
                         "--summary-out the fastest tuple against the fastest measured-rate table "
                         "tile")
    ap.add_argument("--mix", default="standard", choices=("standard", "large", "grid", "grid-short-k"),
                    help="with --off-table: the distribution of the seeded shapes")
    ap.add_argument("--n4", action="store_true",
                    help="with --off-table: N a multiple of 4, K not (scalar variant, 16-byte B loads)")
    ap.add_argument("--aligned", action="store_true",
                    help="with --off-table: round N and K up to multiples of 4 (float4 variant)")
    ap.add_argument("--rate-table", default=None, metavar="FILES",
                    help="write --rate-table-out from these off-table records (comma-separated "
                         "JSONL files of --off-table runs); no GPU needed")
    ap.add_argument("--rate-table-out", default=None)
    ap.add_argument("--rate-column", type=int, default=None, metavar="COLUMN",
                    help="re-time this column of csrc/measured_rates.inc on the --rate-kind rows "
                         "beside each row's fastest other column; writes --out")
    ap.add_argument("--rate-kind", default="scalar", choices=("scalar", "vector"))
    ap.add_argument("--rate-retimed", default=None, metavar="FILE",
                    help="with --rate-column: rewrite those rows of csrc/measured_rates.inc from "
                         "this --out file of a --rate-column run; no GPU needed")
    args = ap.parse_args()
    if args.rate_column is not None and args.rate_retimed:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "measured_rates.inc")
        retimed = {(r["M"], r["N"], r["K"]): (r["rate"], r["anchor"], r["anchor_rate"])
                   for r in map(json.loads, open(args.rate_retimed)) if r}
        moved = refresh_rate_column(path, args.rate_column, args.rate_kind, retimed,
                                    f"python -m fp32_gemm_amd.tune --rate-column {args.rate_column} "
                                    f"--rate-kind {args.rate_kind} --out "
                                    f"{os.path.basename(args.rate_retimed)}")
        print(f"[rate-column] {len(retimed)} re-timed rows read, {len(moved)} rows with a new fastest "
              "column")
        return 0
    if args.rate_table:
        recs = [json.loads(l) for f in args.rate_table.split(",") for l in open(f) if l.strip()]
        # The command as written into the table names the record files
        # without their directory.
        names = ",".join(os.path.basename(f) for f in args.rate_table.split(","))
        cols, ns, nv = write_rate_table(recs, args.rate_table_out,
                                        f"python -m fp32_gemm_amd.tune --rate-table {names} "
                                        f"--rate-table-out {args.rate_table_out}")
        print(f"[rate-table] {ns} scalar and {nv} float4 rows x {len(cols)} columns -> "
              f"{args.rate_table_out}")
        return 0
    if args.best:
        recs = [json.loads(l) for l in open(args.out)]
        fin = [r for r in recs if r["workload"] == args.best and r.get("protocol") == "long"]
        print(",".join(str(x) for x in min(fin, key=lambda r: r["ms"])["tuple"]))
        return 0
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if fg.device_check() != 0:
        raise SystemExit("tune: current device is not gfx950")
    if args.rate_column is not None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "measured_rates.inc")
        retimed = retime_rate_column(dev, path, args.rate_column, args.rate_kind)
        with open(args.out, "w") as f:
            for (M, N, K), (r, j, rj) in retimed.items():
                f.write(json.dumps(dict(M=M, N=N, K=K, rate=r, anchor=j, anchor_rate=rj)) + "\n")
        return 0
    if args.off_table is not None:
        off_table(args.off_table, dev, args.out, args.summary_out,
                  "python -m fp32_gemm_amd.tune " + " ".join(sys.argv[1:]), aligned=args.aligned,
                  shapes=[tuple(int(x) for x in sh.split("x")) for sh in args.shapes.split(",")]
                  if args.shapes else None, mix=args.mix, n4=args.n4)
        return 0
    if args.retime:
        shapes = {**inputs.WORKLOADS, **inputs.TUNING_EXTRA}
        results = retime(args.workloads.split(","), shapes, dev, args.retime, args.top,
                         args.summary_out, "python -m fp32_gemm_amd.tune " + " ".join(sys.argv[1:]))
        if args.table_out:
            for key, old_t, new_t in update_table(args.table_out, results):
                print(f"[retime] rule {key}: {old_t} -> {new_t}", flush=True)
        return 0
    paths = set(args.paths.split(","))
    configs = {v: [c for c in usable_configs(v) if c["path_name"] in paths] for v in (True, False)}
    if args.top_from:
        prev = [json.loads(l) for l in open(args.top_from)]
        keep = set()
        for wl in {r["workload"] for r in prev}:
            rs = sorted((r for r in prev if r["workload"] == wl and r.get("protocol") == "short"
                         and r["exact"]), key=lambda r: r["ms"])
            keep |= {tuple(r["tuple"]) for r in rs[:args.top]}
        configs = {v: [c for c in cs if tuple(c["tuple"]) in keep] for v, cs in configs.items()}
    if args.filter:
        configs = {v: [c for c in cs if eval(args.filter, {}, {"c": c})]
                   for v, cs in configs.items()}
    os.makedirs(os.path.dirname(args.out) or ".", exist_ok=True)
    fout = open(args.out, "a")

    def log(rec):
        fout.write(json.dumps(rec) + "\n")
        fout.flush()
        if rec.get("protocol") == "long" or not rec["exact"]:
            print(json.dumps(rec), flush=True)

    bests, per_path, swept = [], {}, {}
    ranked = None  # the --prune-from shape's configurations, fastest first per path
    shapes = {**inputs.WORKLOADS, **inputs.TUNING_EXTRA}
    if args.shapes:
        # Ad-hoc shapes: A, B ~ N(0, 1), C ~ U[-1, 1], alpha 1, beta 0.
        adhoc = [tuple(int(x) for x in sh.split("x")) for sh in args.shapes.split(",")]
        shapes = {f"{M}x{N}x{K}": inputs.Workload(f"{M}x{N}x{K}", M, N, K, "normal", "uniform", 1.0,
                                                  0.0, 7) for M, N, K in adhoc}
        args.workloads = ",".join(shapes)
    names = sorted(args.workloads.split(","), key=lambda n: (n != args.prune_from, model.flops(
        shapes[n].M, shapes[n].N, shapes[n].K)))
    progress = lambda msg: print(msg, flush=True)
    for name in names:
        w = shapes[name]
        t0 = time.time()
        use = configs[w.K % 4 == 0 and w.N % 4 == 0]
        if model.flops(w.M, w.N, w.K) > args.prune_above:
            if ranked is None:
                raise SystemExit(f"tune: pruning {name} needs --prune-from {args.prune_from} "
                                 f"in --workloads")
            ids = {c["id"] for c in use}
            use = [c for pth in ranked for c in ranked[pth][:args.keep] if c["id"] in ids]
        print(f"[tune] {name}: {len(use)} configs", flush=True)
        best, best_path, results = tune_shape(w, dev, use, log, finalists=args.finalists,
                                              progress=progress)
        if name == args.prune_from:
            order = sorted((r for r in results if r.get("protocol") == "short" and r["exact"]),
                           key=lambda r: r["ms"])
            by_id = {c["id"]: c for c in configs[True] + configs[False]}
            ranked = {}
            for r in order:
                ranked.setdefault(r["path"], []).append(by_id[r["cfg_id"]])
        for pth, b in best_path.items():
            per_path[(name, pth)] = b
            print(f"[tune] {name} {pth}: best cfg {b['cfg_id']} {b['tuple']} {b['ms']:.4f} ms "
                  f"{b['tflops']:.1f} TFLOP/s of {b['swept']} swept", flush=True)
        print(f"[tune] {name}: best cfg {best['cfg_id']} {best['tuple']} {best['ms']:.4f} ms "
              f"{best['tflops']:.1f} TFLOP/s ({time.time() - t0:.0f} s)", flush=True)
        bests.append(best)
        swept[name] = [r for r in results if r.get("protocol") == "short" and r["exact"]]
    if args.shapes and args.summary_out:
        write_rate_table_gap(swept, args.summary_out, "python -m fp32_gemm_amd.tune " +
                             " ".join(sys.argv[1:]))
    elif args.summary_out:
        write_summary(per_path, args.summary_out, "python -m fp32_gemm_amd.tune " +
                      " ".join(sys.argv[1:]), args.finalists)
    if args.table_out:
        by = {b["workload"]: b["tuple"] for b in bests}
        large = by.get("sq4096", bests[0]["tuple"])
        medium = by.get("sq1024", large)
        small = by.get("sq256", medium)
        write_table(bests, args.table_out, [("kDefaultLarge", large), ("kDefaultMedium", medium),
                                            ("kDefaultSmall", small)])
    fout.close()


if __name__ == "__main__":
    sys.exit(main())
