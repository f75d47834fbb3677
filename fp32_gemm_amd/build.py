"""Build libfp32_gemm_amd.so (HIP for gfx950) in-tree.

The candidate tile tuples below are written into generated instance
translation units; each candidate passes through the C++ legality checker at
compile time and only legal ones instantiate kernels.  The units compile in
parallel with hipcc and link into ``fp32_gemm_amd/libfp32_gemm_amd.so``.  The
compiler's per-kernel resource report (VGPRs, AGPRs, scratch, occupancy) is
saved to ``fp32_gemm_amd/_build/resources.json``.

Usage: ``python -m fp32_gemm_amd.build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os
import re
import shutil
import subprocess
import sys
import zlib

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfp32_gemm_amd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 VALU instructions are kept out of every kernel (the
# target-feature switch below); hipcc's host pass warns that it does not know
# the feature, which is harmless.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

VALU, MFMA32, MFMA16 = 0, 1, 2


# Tuples whose kernel (in either variant) the compiler had to spill to
# scratch memory: written by build() from the compiler's resource report and
# left out of the compiled table, so no configuration a caller can select
# spills.  A build that finds a new spilling tuple adds it here and compiles
# the affected units again.
SPILLING = os.path.join(PKG, "spilling_tuples.json")


def _spilling():
    if not os.path.exists(SPILLING):
        return set()
    with open(SPILLING) as f:
        return {tuple(t) for t in json.load(f)["tuples"]}


def valu_grid():
    """The VALU sweep grid: BM, BN in {64, 128, 256}, BK in {8, 16, 32}, WM, WN
    in {32 .. 256}, WNITER in {1, 2, 4}, TM, TN in {4, 8}, 128, 256 or 512
    threads, and 32 to 128 accumulators per lane (32-bank swizzle, no
    schedule options).  Only the cheap necessary conditions are applied here
    (warp tiles inside the block, one wave per warp tile); the C++ checker
    decides legality when the instance units compile."""
    import itertools
    out = []
    for BM, BN, BK, WM, WN, WNITER, TM, TN, NT in itertools.product(
            (64, 128, 256), (64, 128, 256), (8, 16, 32), (32, 64, 128, 256), (32, 64, 128, 256),
            (1, 2, 4), (4, 8), (4, 8), (128, 256, 512)):
        if WM > BM or WN > BN or (BM // WM) * (BN // WN) * 64 != NT:
            continue
        if not 32 <= WM * WN // 64 <= 128:
            continue
        out.append((BM, BN, BK, WM, WN, WNITER, TM, TN, NT, VALU, 32, 0))
    return out


def candidates(include_spilling=False):
    """Candidate tuples (BM, BN, BK, WM, WN, WNITER, TM, TN, NT, path, swz, opt)."""
    out = _all_candidates()
    if include_spilling:
        return out
    bad = _spilling()
    return [t for t in out if t not in bad]


def _all_candidates():
    out = []
    # MFMA 32x32x2: every block/warp tile split into 1, 2, 4 or 8 waves.
    for BM, BN in [(256, 256), (256, 128), (128, 256), (128, 128), (128, 64), (64, 128), (64, 64)]:
        for BK in (8, 16, 32):
            for WM in (32, 64, 128):
                for WN in (32, 64, 128):
                    if WM > BM or WN > BN:
                        continue
                    waves = (BM // WM) * (BN // WN)
                    if waves not in (1, 2, 4, 8):
                        continue
                    base = (BM, BN, BK, WM, WN, WN // 32, 16, 1, 64 * waves, MFMA32, 32)
                    out.append(base + (0,))
                    # Schedule options on the larger tiles.
                    if BM * BN >= 128 * 128 and BK >= 16:
                        out += [base + (1,), base + (2,), base + (3,)]
    # MFMA 16x16x4: a few block shapes.
    for BM, BN, WM, WN in [(128, 128, 64, 64), (256, 128, 128, 64), (256, 256, 128, 128),
                           (64, 64, 32, 32), (128, 64, 64, 32)]:
        for BK in (16, 32):
            waves = (BM // WM) * (BN // WN)
            base = (BM, BN, BK, WM, WN, WN // 16, 4, 1, 64 * waves, MFMA16, 32)
            out += [base + (0,), base + (3,)]
    # VALU outer products: wave64 analogues of the page's shapes.
    for t in [
        (128, 128, 8, 32, 128, 1, 8, 8, 256),   # the vectorized kernel's thread map (no warp tiling)
        (128, 128, 8, 64, 64, 1, 8, 8, 256),    # the page's square 128x128 tile, 8x8 lanes
        (128, 128, 16, 64, 64, 1, 8, 8, 256),
        (128, 64, 16, 64, 64, 2, 4, 4, 128),    # the page's winning shape, WN widened for 64 lanes
        (128, 64, 8, 64, 64, 2, 4, 4, 128),
        (128, 128, 16, 64, 64, 2, 4, 4, 256),
        (64, 64, 16, 64, 64, 2, 4, 4, 64),
        (128, 128, 16, 128, 64, 2, 8, 4, 128),
        (256, 128, 16, 128, 64, 2, 8, 4, 256),
        (128, 128, 32, 64, 64, 2, 4, 4, 256),
        # 8x16 and 16x8 lane patches: 0.75 LDS bytes per FMA instead of 1.
        (128, 128, 16, 64, 128, 1, 8, 16, 128),
        (128, 128, 8, 64, 128, 1, 8, 16, 128),
        (128, 256, 16, 64, 128, 1, 8, 16, 256),
        (256, 256, 16, 128, 128, 1, 8, 16, 256),
        (128, 128, 16, 128, 64, 1, 16, 8, 128),
        (256, 128, 16, 128, 64, 1, 16, 8, 256),
    ]:
        out.append(t + (VALU, 32, 0))
        out.append(t + (VALU, 32, 2))
    # The ladder's VALU rungs in the pages' unswizzled LDS layout.
    out.append((128, 128, 8, 32, 128, 1, 8, 8, 256, VALU, 0, 0))
    out.append((128, 64, 16, 64, 64, 2, 4, 4, 128, VALU, 0, 0))
    # Split-K of a partly filled last wave, on the shapes ragged or small
    # problems use.
    for base in [(256, 256, 32, 64, 128, 4, 16, 1, 512, MFMA32, 32),
                 (256, 256, 16, 64, 128, 4, 16, 1, 512, MFMA32, 32),
                 (128, 128, 32, 32, 64, 2, 16, 1, 512, MFMA32, 32),
                 (128, 128, 16, 32, 64, 2, 16, 1, 512, MFMA32, 32),
                 (128, 128, 32, 64, 64, 2, 16, 1, 256, MFMA32, 32),
                 (128, 256, 32, 64, 128, 4, 16, 1, 256, MFMA32, 32),
                 (256, 128, 32, 128, 64, 2, 16, 1, 256, MFMA32, 32),
                 (64, 64, 32, 32, 32, 1, 16, 1, 256, MFMA32, 32),
                 (128, 128, 16, 64, 64, 4, 4, 1, 256, MFMA16, 32)]:
        out += [base + (8,), base + (9,), base + (11,), base + (15,)]
    # The same schedules with the global loads left to the compiler.
    for base in [(256, 256, 32, 64, 128, 4, 16, 1, 512, MFMA32, 32),
                 (256, 256, 32, 128, 64, 2, 16, 1, 512, MFMA32, 32),
                 (128, 128, 32, 32, 64, 2, 16, 1, 512, MFMA32, 32),
                 (256, 256, 16, 64, 128, 4, 16, 1, 512, MFMA32, 32)]:
        out += [base + (4,), base + (7,)]
    # Direct global-to-LDS staging (MFMA 32x32x2), plain and XCD-aware.
    for BM, BN in [(256, 256), (256, 128), (128, 256), (128, 128)]:
        for BK in (16, 32, 64):
            for WM in (32, 64, 128):
                for WN in (32, 64, 128):
                    if WM > BM or WN > BN or (BM // WM) * (BN // WN) not in (4, 8):
                        continue
                    base = (BM, BN, BK, WM, WN, WN // 32, 16, 1, 64 * (BM // WM) * (BN // WN),
                            MFMA32, 32)
                    out += [base + (16,), base + (18,)]
    for base in [(256, 256, 32, 64, 128, 4, 16, 1, 512, MFMA32, 32),
                 (256, 256, 32, 128, 64, 2, 16, 1, 512, MFMA32, 32),
                 (128, 128, 32, 32, 64, 2, 16, 1, 512, MFMA32, 32),
                 (128, 128, 32, 64, 64, 2, 16, 1, 256, MFMA32, 32)]:
        out += [base + (20,), base + (24,), base + (26,)]
    # Direct-LDS on smaller tiles (more workgroups per CU for mid-size shapes).
    for BM, BN in [(128, 64), (64, 128), (64, 64)]:
        for BK in (16, 32, 64):
            for WM in (32, 64):
                for WN in (32, 64):
                    waves = (BM // WM) * (BN // WN)
                    if WM > BM or WN > BN or waves not in (2, 4, 8):
                        continue
                    base = (BM, BN, BK, WM, WN, WN // 32, 16, 1, 64 * waves, MFMA32, 32)
                    out += [base + (16,), base + (18,), base + (24,)]
    # Sixteen waves per workgroup (four per SIMD), direct-to-LDS staging.
    for BM, BN, WM, WN in [(256, 256, 64, 64), (256, 256, 128, 32), (256, 256, 32, 128),
                           (256, 128, 64, 32), (128, 256, 32, 64), (128, 128, 32, 32)]:
        for BK in (16, 32):
            base = (BM, BN, BK, WM, WN, WN // 32, 16, 1, 1024, MFMA32, 32)
            out += [base + (16,), base + (18,)]
            if BK == 16:
                out.append(base + (18 | 32,))
    # Direct-LDS staging on MFMA 16x16x4: sixteen independent accumulator
    # chains per wave on 64x64 wave tiles (the 32x32x2 tiles above carry four
    # or eight), under both bank models.
    for BM, BN, WM, WN in [(128, 128, 64, 64), (256, 128, 64, 64), (128, 256, 64, 64),
                           (256, 256, 64, 64), (256, 256, 128, 64), (128, 128, 64, 32),
                           (128, 128, 32, 64)]:
        waves = (BM // WM) * (BN // WN)
        for BK in (16, 32, 64):
            for swz in (32, 64):
                base = (BM, BN, BK, WM, WN, WN // 16, 4, 1, 64 * waves, MFMA16, swz)
                out += [base + (16,), base + (18,), base + (24,), base + (26,)]
                if BM * BN <= 128 * 128:
                    out.append(base + (18 | 128,))
                if BK == 16:
                    out.append(base + (18 | 32,))
    # Direct-LDS with the k-group pipeline (opt bit 1): the slice's last
    # k-group multiplied across the barrier.
    for base in [(256, 256, 32, 128, 32, 1, 16, 1, 1024, MFMA32, 32),
                 (256, 256, 16, 128, 32, 1, 16, 1, 1024, MFMA32, 32),
                 (256, 256, 32, 64, 64, 2, 16, 1, 1024, MFMA32, 32),
                 (256, 256, 32, 128, 64, 2, 16, 1, 512, MFMA32, 32),
                 (256, 256, 32, 64, 128, 4, 16, 1, 512, MFMA32, 32),
                 (128, 128, 32, 64, 64, 2, 16, 1, 256, MFMA32, 32),
                 (256, 256, 32, 128, 64, 4, 4, 1, 512, MFMA16, 32),
                 (256, 256, 32, 64, 64, 4, 4, 1, 1024, MFMA16, 64),
                 (128, 256, 16, 64, 64, 4, 4, 1, 512, MFMA16, 32),
                 (128, 256, 32, 64, 64, 4, 4, 1, 512, MFMA16, 32),
                 (128, 128, 16, 64, 64, 4, 4, 1, 256, MFMA16, 32),
                 (128, 128, 32, 64, 64, 4, 4, 1, 256, MFMA16, 32),
                 (128, 128, 64, 64, 32, 2, 4, 1, 512, MFMA16, 64),
                 (64, 64, 64, 32, 32, 1, 16, 1, 256, MFMA32, 32),
                 (64, 64, 32, 32, 32, 1, 16, 1, 256, MFMA32, 32),
                 (64, 128, 32, 64, 32, 1, 16, 1, 256, MFMA32, 32),
                 (128, 64, 32, 32, 64, 2, 16, 1, 256, MFMA32, 32),
                 (64, 64, 64, 32, 32, 2, 4, 1, 256, MFMA16, 32),
                 (128, 128, 64, 64, 64, 4, 4, 1, 256, MFMA16, 32)]:
        out += [base + (17,), base + (19,), base + (25,), base + (27,)]
        if base[0] * base[1] <= 128 * 128:
            out.append(base + (19 | 128,))
        if base[2] == 16:
            out.append(base + (19 | 32,))
    # Direct-LDS stage rings of 3 and 4 stages (opt field 32 / 64).
    for base in [(256, 256, 16, 128, 64, 2, 16, 1, 512, MFMA32, 32),
                 (256, 256, 16, 64, 128, 4, 16, 1, 512, MFMA32, 32),
                 (256, 128, 16, 128, 32, 1, 16, 1, 512, MFMA32, 32),
                 (128, 256, 16, 128, 32, 1, 16, 1, 512, MFMA32, 32),
                 (128, 256, 16, 64, 64, 2, 16, 1, 512, MFMA32, 32),
                 (128, 256, 32, 128, 32, 1, 16, 1, 512, MFMA32, 32),
                 (128, 128, 32, 64, 32, 1, 16, 1, 512, MFMA32, 32),
                 (128, 128, 32, 32, 64, 2, 16, 1, 512, MFMA32, 32),
                 (128, 128, 32, 128, 32, 1, 16, 1, 256, MFMA32, 32),
                 (128, 128, 16, 64, 32, 1, 16, 1, 512, MFMA32, 32)]:
        for ring in (32, 64):
            out += [base + (16 | ring,), base + (18 | ring,)]
    # Residency requests (opt field 128 * b: b + 1 workgroups per CU) on tiles
    # whose occupancy the compiler's register use limits.
    for t in [(128, 128, 16, 32, 64, 2, 16, 1, 512, MFMA32, 32, 16),
              (128, 128, 16, 64, 32, 1, 16, 1, 512, MFMA32, 32, 16),
              (128, 128, 32, 64, 32, 1, 16, 1, 512, MFMA32, 32, 18),
              (128, 128, 32, 128, 32, 1, 16, 1, 256, MFMA32, 32, 16),
              (128, 256, 16, 128, 32, 1, 16, 1, 512, MFMA32, 32, 16),
              (128, 128, 32, 32, 64, 2, 16, 1, 512, MFMA32, 32, 7),
              (64, 64, 32, 32, 32, 1, 16, 1, 256, MFMA32, 32, 0),
              (64, 64, 16, 32, 32, 1, 16, 1, 256, MFMA32, 32, 0),
              (128, 128, 16, 64, 64, 1, 8, 8, 256, VALU, 32, 0),
              (128, 64, 16, 64, 64, 2, 4, 4, 128, VALU, 32, 0),
              (128, 128, 16, 64, 64, 2, 4, 4, 256, VALU, 32, 0)]:
        for b in (1, 2, 3):
            out.append(t[:11] + (t[11] | (b << 7),))
    # Bank-model variants of the headline shapes: unswizzled, and 64 banks.
    for base in [(256, 256, 16, 128, 128, 4, 16, 1, 256, MFMA32),
                 (256, 256, 32, 128, 128, 4, 16, 1, 256, MFMA32),
                 (128, 128, 16, 64, 64, 2, 16, 1, 256, MFMA32),
                 (128, 128, 16, 64, 64, 4, 4, 1, 256, MFMA16),
                 (128, 64, 16, 64, 64, 2, 4, 4, 128, VALU)]:
        for swz in (0, 64):
            out.append(base + (swz, 0))
            if base[9] != VALU:
                out.append(base + (swz, 3))
    # One wave per SIMD with the whole 128 x 128 wave tile in accumulator
    # registers, k-group pipelined.
    for base in [(256, 256, 32, 128, 128, 4, 16, 1, 256, MFMA32, 32),
                 (256, 256, 16, 128, 128, 4, 16, 1, 256, MFMA32, 32),
                 (256, 256, 32, 128, 128, 8, 4, 1, 256, MFMA16, 32),
                 (256, 256, 32, 128, 128, 8, 4, 1, 256, MFMA16, 64)]:
        out += [base + (opt,) for opt in (17, 19, 25, 27)]
    # Direct-LDS staging on the VALU path (A transposed by 4-byte loads), on
    # the register-staged sweep's best VALU tiles: 2 and 3 LDS stages, plain
    # and XCD-aware order.
    for base in [(256, 256, 16, 128, 64, 2, 4, 4, 512, VALU, 32),
                 (256, 256, 8, 32, 256, 1, 8, 4, 512, VALU, 32),
                 (256, 128, 16, 128, 64, 1, 4, 8, 256, VALU, 32),
                 (128, 128, 16, 128, 64, 1, 4, 8, 128, VALU, 32),
                 (128, 256, 16, 128, 64, 2, 4, 4, 256, VALU, 32),
                 (128, 256, 16, 32, 128, 2, 4, 4, 512, VALU, 32),
                 (128, 256, 32, 64, 64, 2, 8, 4, 512, VALU, 32),
                 (256, 256, 16, 128, 64, 1, 4, 8, 512, VALU, 32),
                 (128, 128, 16, 64, 64, 1, 8, 8, 256, VALU, 32),
                 (128, 128, 32, 64, 32, 1, 8, 4, 512, VALU, 32)]:
        out += [base + (opt,) for opt in (16, 18, 48, 50)]
    # K-sliced workgroups (opt bit 9): two wave groups split the K slices of
    # one tile, for shapes with about one tile per compute unit.
    KS = 512
    for base in [(64, 64, 64, 32, 32, 1, 16, 1, 512, MFMA32, 32),
                 (64, 64, 32, 32, 32, 1, 16, 1, 512, MFMA32, 32),
                 (64, 64, 16, 32, 32, 1, 16, 1, 512, MFMA32, 32),
                 (64, 64, 64, 32, 32, 2, 4, 1, 512, MFMA16, 32),
                 (64, 64, 32, 32, 32, 2, 4, 1, 512, MFMA16, 32),
                 (128, 64, 32, 64, 32, 1, 16, 1, 512, MFMA32, 32),
                 (64, 128, 32, 32, 64, 2, 16, 1, 512, MFMA32, 32),
                 (128, 128, 32, 64, 64, 2, 16, 1, 512, MFMA32, 32),
                 (128, 128, 32, 64, 64, 4, 4, 1, 512, MFMA16, 32),
                 (128, 128, 32, 64, 32, 2, 4, 1, 1024, MFMA16, 64)]:
        out += [base + (opt | KS,) for opt in (16, 17, 18, 19)]
    out += valu_grid()
    seen, uniq = set(), []
    for t in out:
        if t not in seen:
            seen.add(t)
            uniq.append(t)
    return uniq


def _write_if_changed(path, text):
    if os.path.exists(path):
        with open(path) as f:
            if f.read() == text:
                return
    with open(path, "w") as f:
        f.write(text)


def generate(n_units=24):
    os.makedirs(BUILD, exist_ok=True)
    cands = candidates()
    # Each tuple's unit is a hash of the tuple, so dropping one tuple changes
    # only its own unit.
    units = [[] for _ in range(n_units)]
    for t in cands:
        units[zlib.crc32(repr(t).encode()) % n_units].append(t)
    srcs = []
    for ui, unit in enumerate(units):
        lines = ['#include "registry.hpp"', "namespace fp32gemm {",
                 f"extern ConfigEntry kEntries{ui}[] = {{"]
        for t in unit:
            lines.append("  candidate<%s>()," % ", ".join(str(x) for x in t))
        lines += ["};", f"extern const int kCount{ui} = {len(unit)};", "}  // namespace fp32gemm", ""]
        path = os.path.join(BUILD, f"instances_{ui:02d}.hip")
        _write_if_changed(path, "\n".join(lines))
        srcs.append(path)
    idx = ["namespace fp32gemm {"]
    for ui in range(len(units)):
        idx.append(f"extern ConfigEntry kEntries{ui}[]; extern const int kCount{ui};")
    idx.append("static const EntryTable kTables[] = {")
    for ui in range(len(units)):
        idx.append(f"  {{kEntries{ui}, kCount{ui}}},")
    idx += ["};", "}  // namespace fp32gemm", ""]
    # kCount is a run-time value across units; the table is read after static init.
    _write_if_changed(os.path.join(BUILD, "instances_index.inc"), "\n".join(idx))
    return srcs


_REMARK = re.compile(r"remark: (?:\s*)(Function Name|TotalSGPRs|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]): (\S+)")


def _compile(src, obj, remarks):
    cmd = [HIPCC, *HIP_FLAGS, "-I", CSRC, "-I", BUILD, "-c", src, "-o", obj]
    if remarks:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{p.stderr[-6000:]}")
    res, cur = {}, None
    for m in _REMARK.finditer(p.stderr):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = val
            res[cur] = {}
        elif cur is not None:
            res[cur][key.split(" ")[0]] = int(val)
    return res


_TILE_NAME = re.compile(r"TileCfgILi" + r"ELi".join([r"(\d+)"] * 12) + r"EEELb(\d)")


def build(verbose=True, jobs=None):
    """Compile every HIP source for gfx950 and link the shared library.  If a
    tuple's kernel spills, it is recorded in spilling_tuples.json and the
    units are compiled again without it."""
    for attempt in range(3):
        resources = _build_once(verbose, jobs)
        new = set()
        for name, v in resources.items():
            m = _TILE_NAME.search(name)
            if m and v.get("ScratchSize", 0) > 0:
                new.add(tuple(int(x) for x in m.groups()[:12]))
        if not new:
            return LIB
        bad = sorted(_spilling() | new)
        with open(SPILLING, "w") as f:
            json.dump({"note": "tuples whose kernel spilled to scratch in the compiler's resource "
                               "report; left out of the compiled table",
                       "tuples": [list(t) for t in bad]}, f, indent=0)
        if verbose:
            print(f"[build] {len(new)} spilling tuples excluded; compiling again", flush=True)
    raise RuntimeError("build: spilling tuples remain after three passes")


def _build_once(verbose, jobs):
    t_srcs = generate()
    jobs = jobs or min(16, os.cpu_count() or 4)
    api = os.path.join(CSRC, "sgemm_api.hip")
    work = [(api, os.path.join(BUILD, "sgemm_api.o"), False),
            (os.path.join(CSRC, "ladder.hip"), os.path.join(BUILD, "ladder.o"), True)]
    work += [(s, s[:-4] + ".o", True) for s in t_srcs]
    resources = {}
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {ex.submit(_compile, s, o, r): s for s, o, r in work}
        for f in cf.as_completed(futs):
            resources.update(f.result())
            if verbose:
                print(f"[build] compiled {os.path.basename(futs[f])}", flush=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [o for _, o, _ in work]
    p = subprocess.run(link, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n" + p.stderr[-4000:])
    os.replace(tmp, LIB)
    with open(os.path.join(BUILD, "resources.json"), "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    spills = {k: v for k, v in resources.items() if v.get("ScratchSize", 0) > 0}
    if verbose:
        print(f"[build] {LIB}: {len(resources)} kernels, {len(spills)} with scratch", flush=True)
    return resources


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)
    if os.path.exists(LIB):
        os.remove(LIB)


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
