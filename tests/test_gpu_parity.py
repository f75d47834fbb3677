"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: max|C_gpu - C64| / (K * max|A| * max|B|) <= 1e-6, bit-exact equality on
inputs whose sums are exact in fp32 (small integers, identity, all-ones,
rank-1), and every byte of C outside the M x N window untouched.
"""
import os
import sys
import time

import numpy as np
import pytest
import torch

from fp32_gemm_amd import inputs

pytestmark = pytest.mark.gpu

TOL = 1e-6
CANARY = 0x7FC0DEAD  # a NaN payload no computation produces


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def fg(dev):
    import fp32_gemm_amd
    assert fp32_gemm_amd.device_check() == 0, "current device is not gfx950"
    return fp32_gemm_amd


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle
    oracle.build(force=False)
    return oracle


class Canvas:
    """C placed inside a larger allocation: `guard` canary rows above and
    below, and canary padding columns [N, ldc)."""

    def __init__(self, C, ldc, guard, dev):
        M, N = C.shape
        self.M, self.N, self.guard = M, N, guard
        self.big = torch.full((M + 2 * guard, ldc), CANARY, dtype=torch.int32, device=dev)
        self.view = self.big.view(torch.float32)[guard:guard + M, :N]
        self.view.copy_(torch.from_numpy(C))

    def result(self):
        return self.view.cpu().numpy()

    def untouched(self):
        b = self.big.cpu().numpy().copy()
        b[self.guard:self.guard + self.M, :self.N] = CANARY
        return bool(np.all(b == CANARY))


def to_dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def check_close(got, C64, K, A, B, what):
    """The parity bar.  With a zero denominator (K == 0, or an all-zero A or
    B) there is no scale to measure against, and the result must equal the
    oracle's correctly rounded value exactly."""
    err = _err(got, C64, K, A, B)
    if err is None:
        want = np.asarray(C64, dtype=np.float64).astype(np.float32)
        assert np.array_equal(np.asarray(got, np.float32), want), f"{what}: zero scale, not exact"
        return 0.0
    assert err <= TOL, f"{what}: err={err}"
    return err


def same_ints(got, want):
    """Bitwise equality of integer-valued results, except that -0 and +0
    count as one value.  Every partial sum is exact, so any summation order
    gives the same number; only an exactly zero output may differ in sign:
    a zero sum of opposite-signed terms rounds to +0 while -0 + -0 stays -0,
    so with a negative alpha or beta a configuration that adds its K
    segments into beta * C one by one can end at +0 where the single sum
    alpha * (A B) + beta * C gives -0."""
    g = np.asarray(got, np.float32) + np.float32(0.0)
    w = np.asarray(want, np.float32) + np.float32(0.0)
    return np.array_equal(g.view(np.uint32), w.view(np.uint32))


def _err(got, C64, K, A, B):
    from oracle import oracle
    den = (K, float(np.abs(A).max()) if A.size else 0.0, float(np.abs(B).max()) if B.size else 0.0)
    return oracle.rel_error(got, C64, *den)


# ---------------------------------------------------------------------------
# Every compiled configuration, both variants, on a shape with ragged edges
# in M, N and K (several tiles in each direction for every tile size).

SHAPE_VEC = (600, 600, 100)     # K % 4 == N % 4 == 0: float4 variant
SHAPE_SCALAR = (601, 599, 99)   # scalar variant, N % 4 != 0: 4-byte B loads
SHAPE_SCALAR_N4 = (601, 600, 99)  # scalar variant, N % 4 == 0: 16-byte B loads


@pytest.fixture(scope="module")
def ragged_cases(orc):
    cases = {}
    for name, (M, N, K) in (("vec", SHAPE_VEC), ("scalar", SHAPE_SCALAR), ("scalar_n4", SHAPE_SCALAR_N4)):
        A, B, C = inputs.make_random(M, N, K, seed=900 + M)
        r32, r64 = orc.sgemm(A, B, C, 0.5, 3.0)
        Ai, Bi, Ci = inputs.make_small_int(M, N, K, seed=901 + M)
        i32, _ = orc.sgemm(Ai, Bi, Ci, 0.5, 3.0)
        cases[name] = dict(shape=(M, N, K), rnd=(A, B, C, r64), ints=(Ai, Bi, Ci, i32))
    return cases


def run(fg, dev, A, B, C, alpha, beta, cfg=-1, ldc_pad=5, guard=3):
    M, N = C.shape
    cv = Canvas(C, N + ldc_pad, guard, dev)
    fg.sgemm_ex(to_dev(A, dev), to_dev(B, dev), cv.view, alpha, beta, cfg_id=cfg)
    torch.cuda.synchronize()
    return cv


CHUNKS = 12


@pytest.mark.parametrize("chunk", range(CHUNKS))
def test_every_config_both_variants(fg, dev, ragged_cases, chunk):
    cfgs = [c for c in fg.configs() if c["id"] % CHUNKS == chunk]
    log(f"[parity] chunk {chunk}: {len(cfgs)} configs x 3 shapes")
    worst = 0.0
    for c in cfgs:
        for variant in ("vec", "scalar", "scalar_n4"):
            case = ragged_cases[variant]
            M, N, K = case["shape"]
            log(f"[parity] cfg {c['id']} {c['path_name']} {c['tuple']} {variant} {M}x{N}x{K}")
            A, B, C, r64 = case["rnd"]
            cv = run(fg, dev, A, B, C, 0.5, 3.0, cfg=c["id"], ldc_pad=4 if variant == "vec" else 5)
            assert cv.untouched(), f"cfg {c['id']} {variant}: wrote outside C"
            worst = max(worst, check_close(cv.result(), r64, K, A, B, f"cfg {c['id']} {variant}"))
            Ai, Bi, Ci, i32 = case["ints"]
            cv = run(fg, dev, Ai, Bi, Ci, 0.5, 3.0, cfg=c["id"], ldc_pad=4 if variant == "vec" else 5)
            got = cv.result()
            assert np.array_equal(got.view(np.uint32), i32.view(np.uint32)), \
                f"cfg {c['id']} {variant}: integer inputs not bit-exact"
    log(f"[parity] worst err {worst:.3e}")


@pytest.mark.parametrize("variant", ["vec", "scalar", "scalar_n4"])
def test_every_config_reads_inside_K(fg, dev, orc, variant):
    # A and B sit in NaN-filled buffers: NaN in the lda / ldb padding and in
    # the rows after B's K rows.  A read of any element outside the logical
    # K range would put a NaN into a stored output; the results must instead
    # match the oracle.  (Reads past M or N could only reach outputs that are
    # never stored; the buffer resources bound those.)  scalar_n4: K odd and
    # odd leading dimensions with N % 4 == 0, so the scalar variant's 16-byte
    # loads run at 4-byte-aligned addresses.
    M, N, K, pad = {"vec": (130, 100, 76, 4), "scalar": (130, 97, 75, 3),
                    "scalar_n4": (130, 100, 75, 3)}[variant]
    A, B, C = inputs.make_random(M, N, K, seed=77 + K)
    _, r64 = orc.sgemm(A, B, C, 0.5, 3.0)
    Abig = torch.full((M + 8, K + pad), float("nan"), device=dev)
    Bbig = torch.full((K + 8, N + pad), float("nan"), device=dev)
    Abig[:M, :K] = torch.from_numpy(A).to(dev)
    Bbig[:K, :N] = torch.from_numpy(B).to(dev)
    cfgs = fg.configs()
    log(f"[nan-padding] {variant} {M}x{N}x{K}: {len(cfgs)} configs")
    for c in cfgs:
        cv = Canvas(C, N + pad, 2, dev)
        fg.sgemm_ex(Abig[:M, :K], Bbig[:K, :N], cv.view, 0.5, 3.0, cfg_id=c["id"])
        torch.cuda.synchronize()
        assert cv.untouched(), f"cfg {c['id']}: wrote outside C"
        got = cv.result()
        assert np.isfinite(got).all(), f"cfg {c['id']} {c['tuple']}: read outside K"
        check_close(got, r64, K, A, B, f"cfg {c['id']} {variant}")


def test_split_configs_with_whole_and_split_tiles(fg, dev, orc):
    """Every split-K configuration on a shape whose tiles overflow the
    resident workgroups by a small tail, so whole tiles and atomically summed
    K segments meet in one launch: integer inputs must stay bit-exact and
    nothing outside C may change."""
    M, N, K = 4097, 4095, 130
    A, B, C = inputs.make_small_int(M, N, K, seed=31)
    want, _ = orc.sgemm(A, B, C, 0.5, 3.0)
    seen = 0
    for c in fg.configs():
        if not c["opt"] & 8:
            continue
        for ldc_pad in (0, 3):   # vector (N % 4 != 0 -> scalar anyway) and padded
            cv = run(fg, dev, A, B, C, 0.5, 3.0, cfg=c["id"], ldc_pad=ldc_pad, guard=1)
            plan = fg.plan(M, N, K, 1 << 40, K, 2 << 40, N, 4 << 40, N + ldc_pad, c["id"])
            log(f"[split] cfg {c['id']} {c['tuple']} tiles_full={plan['tiles_full']} "
                f"splits={plan['splits']}")
            assert cv.untouched(), f"cfg {c['id']}: wrote outside C"
            got = cv.result()
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), c["id"]
            seen += plan["splits"] > 1 and plan["tiles_full"] > 0
    assert seen > 0, "no configuration split a tail"


def test_split_configs_random_inputs_within_tolerance(fg, dev, orc):
    M, N, K = 1000, 1500, 777
    A, B, C = inputs.make_random(M, N, K, seed=33)
    _, r64 = orc.sgemm(A, B, C, 1.0, 1.0)
    _, r64b = orc.sgemm(A, B, C, 0.5, 0.0)
    for c in fg.configs():
        if not c["opt"] & 8:
            continue
        cv = run(fg, dev, A, B, C, 1.0, 1.0, cfg=c["id"])
        assert cv.untouched()
        check_close(cv.result(), r64, K, A, B, f"split cfg {c['id']}")
        cv = run(fg, dev, A, B, C, 0.5, 0.0, cfg=c["id"])
        check_close(cv.result(), r64b, K, A, B, f"split cfg {c['id']} beta=0")


@pytest.mark.parametrize("variant", ["vec", "scalar", "scalar_n4"])
def test_direct_lds_configs_short_and_ragged_K(fg, dev, orc, variant):
    # Direct-to-LDS configs run their K slices partial-first: slice 0 holds the
    # K % BK remainder (masked in both operands) and every later slice is
    # whole.  K = 0 (no slice), K below one slice, a one-column tail and a
    # tail one past a whole slice, on ragged M and N, for both load widths;
    # K = 196 / 197 gives BK = 64 tiles an even slice count and BK = 32 an
    # odd one (the two-slice K loop and its one-slice tail).  scalar_n4:
    # N % 4 == 0 with an odd ldc, so the scalar variant runs with 16-byte B
    # loads, with K % 4 == 0 (a whole-float4 slice 0) and K % 4 != 0.
    cfgs = [c for c in fg.configs() if c["opt"] & 16]
    N = 91 if variant == "scalar" else 92
    pad = 4 if variant == "vec" else 5
    Ks = {"vec": (0, 4, 36, 64, 196), "scalar": (0, 1, 33, 65, 197),
          "scalar_n4": (0, 1, 4, 33, 65, 196, 197)}[variant]
    for K in Ks:
        log(f"[direct-lds] {variant} 70x{N}x{K}: {len(cfgs)} configs")
        if K == 0:
            C = inputs.make_random(70, N, 1, seed=1700)[2]
            want = (3.0 * C.astype(np.float64)).astype(np.float32)
            A0 = torch.empty((70, 0), dtype=torch.float32, device=dev)
            B0 = torch.empty((0, N), dtype=torch.float32, device=dev)
            for c in cfgs:
                cv = Canvas(C, N + pad, 3, dev)
                fg.sgemm_ex(A0, B0, cv.view, 0.5, 3.0, cfg_id=c["id"])
                torch.cuda.synchronize()
                assert cv.untouched() and np.array_equal(cv.result(), want), f"cfg {c['id']} K=0"
            continue
        A, B, C = inputs.make_random(70, N, K, seed=1700 + K)
        Ai, Bi, Ci = inputs.make_small_int(70, N, K, seed=1800 + K)
        r64 = orc.sgemm(A, B, C, 0.5, 3.0)[1]
        i32 = orc.sgemm(Ai, Bi, Ci, 0.5, 3.0)[0]
        for c in cfgs:
            cv = run(fg, dev, A, B, C, 0.5, 3.0, cfg=c["id"], ldc_pad=pad)
            assert cv.untouched(), f"cfg {c['id']} K={K}: wrote outside C"
            check_close(cv.result(), r64, K, A, B, f"cfg {c['id']} K={K}")
            cv = run(fg, dev, Ai, Bi, Ci, 0.5, 3.0, cfg=c["id"], ldc_pad=pad)
            assert np.array_equal(cv.result().view(np.uint32), i32.view(np.uint32)), \
                f"cfg {c['id']} K={K}: integer inputs not bit-exact"


@pytest.mark.parametrize("rung", [1, 2, 3, 4])
def test_ladder_rungs(fg, dev, orc, rung):
    """Each rung of the kernel ladder on ragged shapes: within tolerance on
    random inputs, bit-exact on integer inputs, C outside M x N untouched."""
    for (M, N, K) in [(300, 260, 200), (1000, 1500, 777), (512, 512, 512)]:
        A, B, C = inputs.make_random(M, N, K, seed=M + rung)
        _, r64 = orc.sgemm(A, B, C, 0.5, 3.0)
        cv = Canvas(C, N + 5, 2, dev)
        fg.ladder(rung, to_dev(A, dev), to_dev(B, dev), cv.view, 0.5, 3.0)
        torch.cuda.synchronize()
        assert cv.untouched()
        check_close(cv.result(), r64, K, A, B, f"rung {rung} {M}x{N}x{K}")
        Ai, Bi, Ci = inputs.make_small_int(M, N, K, seed=M + 7 * rung)
        i32, _ = orc.sgemm(Ai, Bi, Ci, 0.5, 3.0)
        cv = Canvas(Ci, N, 1, dev)
        fg.ladder(rung, to_dev(Ai, dev), to_dev(Bi, dev), cv.view, 0.5, 3.0)
        torch.cuda.synchronize()
        assert np.array_equal(cv.result().view(np.uint32), i32.view(np.uint32)), f"rung {rung}"


# ---------------------------------------------------------------------------
# The workload configurations, through the tuned dispatch, compared with the
# oracle's whole product on every output.


def guard_rows(fg):
    """Canary rows above and below C: one block tile of the tallest compiled
    configuration, so a workgroup that strayed a whole tile out of the window
    would still land in the guard."""
    return max(c["BM"] for c in fg.configs())


def full_parity(fg, dev, orc, w, A, B, C, tag):
    """Tuned dispatch on the workload with C inside one-tile guard bands, once
    with tight ldc (the launch the benchmark times) and once with padded ldc
    (same configuration and variant: the pad keeps ldc % 4); every output
    against the oracle's fp64 product, every other byte of the allocation
    unchanged."""
    t0 = time.time()
    _, r64 = orc.sgemm(A, B, C, w.alpha, w.beta)
    log(f"[{tag}] oracle {w.M}x{w.N}x{w.K}: {time.time() - t0:.1f} s")
    guard = guard_rows(fg)
    worst = 0.0
    for pad in (0, 4 if w.N % 4 == 0 else 5):
        cv = run(fg, dev, A, B, C, w.alpha, w.beta, ldc_pad=pad, guard=guard)
        assert cv.untouched(), f"{tag}: wrote outside C (ldc pad {pad})"
        worst = max(worst, check_close(cv.result(), r64, w.K, A, B, f"{tag} ldc pad {pad}"))
        del cv
    return worst


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload(fg, dev, orc, name):
    w = inputs.WORKLOADS[name]
    log(f"[workload] {name} {w.M}x{w.N}x{w.K} alpha={w.alpha} beta={w.beta}")
    A, B, C = inputs.make(w)
    err = full_parity(fg, dev, orc, w, A, B, C, name)
    log(f"[workload] {name} err={err:.3e} over all {w.M * w.N} outputs")


@pytest.mark.parametrize("name", list(inputs.TUNING_EXTRA))
def test_tuning_only_shape(fg, dev, orc, name):
    # The dispatch table's tuning-only shapes run their own rule's tuple
    # (split-K for most).
    w = inputs.TUNING_EXTRA[name]
    log(f"[tuning shape] {name} {w.M}x{w.N}x{w.K} alpha={w.alpha} beta={w.beta}")
    A, B, C = inputs.make(w)
    err = full_parity(fg, dev, orc, w, A, B, C, name)
    log(f"[tuning shape] {name} err={err:.3e}")


@pytest.mark.parametrize("shape", [(4097, 4095, 4093), (1000, 1500, 777), (4096, 4096, 4096)])
def test_integer_inputs_bit_exact_full_size(fg, dev, orc, shape):
    # Every partial sum is an exact integer in fp32, so every output must equal
    # the oracle's bit for bit.
    M, N, K = shape
    log(f"[int] {M}x{N}x{K}")
    A, B, C = inputs.make_small_int(M, N, K, seed=77)
    want, _ = orc.sgemm(A, B, C, 0.5, 3.0)
    cv = run(fg, dev, A, B, C, 0.5, 3.0, ldc_pad=3, guard=guard_rows(fg))
    assert cv.untouched()
    assert np.array_equal(cv.result().view(np.uint32), want.view(np.uint32))


def test_random_shapes_tuned_dispatch(fg, dev, orc):
    """Seeded shapes off every table (half with M, N, K log-uniform in
    [1, 2500], mostly thin; half uniform in [200, 2500]),
    random alpha / beta (beta = 0 on a quarter of them), A and B inside
    NaN-filled buffers with padded leading dimensions, C inside canaries:
    the tuned dispatch must meet the parity bar on every output, and on
    integer-valued inputs, with alpha and beta that keep every product and
    sum exact in fp32, match the oracle bit for bit (but for the sign of an
    exactly zero output)."""
    rng = np.random.default_rng(2024)
    for case in range(24):
        if case % 2 == 0:
            M, N, K = (int(round(np.exp(rng.uniform(0, np.log(2500))))) for _ in range(3))
        else:
            M, N, K = (int(x) for x in rng.integers(200, 2501, 3))
        alpha = float(np.float32(rng.uniform(-2, 2)))
        beta = 0.0 if case % 4 == 3 else float(np.float32(rng.uniform(-2, 2)))
        pa, pb, pc = (int(x) for x in rng.integers(0, 8, 3))
        log(f"[random] case {case}: {M}x{N}x{K} alpha={alpha:.4f} beta={beta:.4f} pads {pa},{pb},{pc}")
        for ints in (False, True):
            a, b = alpha, beta
            if ints:
                A, B, C = inputs.make_small_int(M, N, K, seed=3000 + case)
                a = (0.5, -1.0, 2.0, 0.25)[case % 4]
                b = (3.0, -1.5, 0.5, 0.0)[case % 4]
            else:
                A, B, C = inputs.make_random(M, N, K, seed=3000 + case)
            want32, want64 = orc.sgemm(A, B, C, a, b)
            Abig = torch.full((M, K + pa), float("nan"), device=dev)
            Bbig = torch.full((K, N + pb), float("nan"), device=dev)
            Abig[:, :K] = to_dev(A, dev)
            Bbig[:, :N] = to_dev(B, dev)
            cv = Canvas(C, N + pc, 2, dev)
            fg.sgemm_ex(Abig[:, :K], Bbig[:, :N], cv.view, a, b)
            torch.cuda.synchronize()
            assert cv.untouched(), f"case {case}: wrote outside C"
            got = cv.result()
            if ints:
                assert same_ints(got, want32), f"case {case}: integer inputs not bit-exact"
            else:
                check_close(got, want64, K, A, B, f"case {case} {M}x{N}x{K}")


def test_zero_operand_exact(fg, dev, orc):
    # An all-zero A makes the parity scale zero: the result must then equal
    # the oracle's correctly rounded beta * C exactly.
    M, N, K = 300, 260, 200
    _, B, C = inputs.make_random(M, N, K, seed=19)
    A = np.zeros((M, K), np.float32)
    _, r64 = orc.sgemm(A, B, C, 0.5, 3.0)
    cv = run(fg, dev, A, B, C, 0.5, 3.0)
    assert cv.untouched()
    assert check_close(cv.result(), r64, K, A, B, "zero A") == 0.0


def test_maximum_leading_dimension(fg, dev, orc):
    """Leading dimensions at the library's limit (2^21 - 1 elements, and the
    largest multiple of 4 below it for the float4 variant) on a 256-row
    product, so the tallest block tile's in-tile offsets reach their largest
    values: every output against the oracle, C's padding untouched."""
    lim = (1 << 21) - 1
    M, N, K = 256, 260, 300
    A, B, C = inputs.make_random(M, N, K, seed=23)
    _, r64 = orc.sgemm(A, B, C, 0.5, 3.0)
    cfgs = [-1] + [c["id"] for c in fg.configs() if c["BM"] == 256 and c["opt"] & 16][:1]
    for ld in (lim, lim - 3):
        Abig = torch.full((M, ld), float("nan"), device=dev)
        Abig[:, :K] = to_dev(A, dev)
        for cfg in cfgs:
            cv = Canvas(C, ld, 1, dev)
            fg.sgemm_ex(Abig[:, :K], to_dev(B, dev), cv.view, 0.5, 3.0, cfg_id=cfg)
            torch.cuda.synchronize()
            pl = fg.plan(M, N, K, Abig.data_ptr(), ld, 1 << 40, N, cv.view.data_ptr(), ld, cfg)
            log(f"[max ld] ld={ld} cfg {pl['cfg_id']} vector={pl['vector_variant']}")
            assert pl["vector_variant"] == (ld % 4 == 0 and N % 4 == 0)
            assert cv.untouched(), f"ld {ld} cfg {cfg}: wrote outside C"
            check_close(cv.result(), r64, K, A, B, f"ld {ld} cfg {cfg}")
            del cv
        del Abig
        torch.cuda.empty_cache()


def test_operands_beyond_4GiB(fg, dev, orc):
    """Every operand spans more than 2^32 bytes, so tile base addresses lie
    past what a 32-bit buffer offset reaches (the kernels form bases in 64
    bits and keep only in-tile offsets in 32).  Default dispatch in both
    variants; sampled outputs, including the rows just past each 4 GiB
    boundary of A and C (every output reads B's last rows, which lie past
    it), bit-exact against the oracle on integer inputs; the guard rows and
    padding columns around C unchanged."""
    M, N, K, pad = 32800, 32900, 32780, 4
    A, B, Cin = inputs.make_small_int_device(M, N, K, seed=55, device=dev)
    big = torch.full((M + 2, N + pad), CANARY, dtype=torch.int32, device=dev)
    Cv = big.view(torch.float32)[1:1 + M, :N]
    assert min(M * K, K * N, M * (N + pad)) * 4 > 1 << 32
    rng = np.random.default_rng(56)
    ra, rc = (1 << 32) // (4 * K), (1 << 32) // (4 * (N + pad))
    rows = sorted({0, 1, 255, 256, ra - 1, ra, ra + 1, rc - 1, rc, rc + 1, M - 2, M - 1}
                  | set(rng.integers(0, M, 20).tolist()))
    cols = sorted({0, 255, 256, N - 5, N - 2, N - 1} | set(rng.integers(0, N, 26).tolist()))
    ri, ci = (x.ravel() for x in np.meshgrid(np.arange(len(rows)), np.arange(len(cols)), indexing="ij"))
    rt, ct = torch.tensor(rows, device=dev), torch.tensor(cols, device=dev)
    for variant, A_, B_ in (("vec", A, B), ("scalar", A[:, 1:], B[1:, :])):
        Kv = A_.shape[1]
        Cv.copy_(Cin)
        pl = fg.plan(M, N, Kv, A_.data_ptr(), K, B_.data_ptr(), N, Cv.data_ptr(), N + pad)
        log(f"[4GiB] {variant} {M}x{N}x{Kv}: cfg {pl['cfg_id']} vector={pl['vector_variant']}")
        assert pl["vector_variant"] == (variant == "vec")
        Asub = A_.index_select(0, rt).cpu().numpy()
        Bsub = B_.index_select(1, ct).cpu().numpy()
        Csub = Cin.index_select(0, rt).index_select(1, ct).cpu().numpy()
        e32, _ = orc.entries(ri, ci, Asub, Bsub, Csub, 0.5, 3.0)
        fg.sgemm_ex(A_, B_, Cv, 0.5, 3.0)
        torch.cuda.synchronize()
        got = Cv.index_select(0, rt).index_select(1, ct).cpu().numpy()
        assert np.array_equal(got[ri, ci].view(np.uint32), e32.view(np.uint32)), variant
        assert bool((big[0] == CANARY).all()) and bool((big[M + 1] == CANARY).all())
        assert bool((big[:, N:] == CANARY).all()), variant
    del A, B, Cin, big, Cv
    torch.cuda.empty_cache()


def test_c_client_runs_sgemm(dev, orc, tmp_path):
    """The library from plain C: a C99 program (tests/c_client) copies
    integer-valued inputs to hipMalloc'd buffers and calls sgemm() on the
    null stream, no Python or torch on that path; bit-exact against the
    oracle."""
    import subprocess
    client = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "sgemm_client")
    if not os.path.exists(client):
        pytest.fail("tests/c_client/sgemm_client is missing: run __graft_entry__.build()")
    M, N, K = 333, 260, 129
    A, B, C = inputs.make_small_int(M, N, K, seed=61)
    files = [str(tmp_path / f"{n}.bin") for n in ("A", "B", "C", "out")]
    for x, f in zip((A, B, C), files):
        x.tofile(f)
    log(f"[c client] {M}x{N}x{K}")
    r = subprocess.run([client, "run", str(M), str(N), str(K), "0.5", "3", *files],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    got = np.fromfile(files[3], dtype=np.float32).reshape(M, N)
    want, _ = orc.sgemm(A, B, C, 0.5, 3.0)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------------------
# Closed forms at full size.

@pytest.mark.parametrize("M,N", [(4096, 4096), (777, 1500)])
def test_identity_gives_B(fg, dev, M, N):
    K = M
    B = inputs.make_random(1, N, K, seed=5)[1]
    A = np.eye(M, dtype=np.float32)
    cv = run(fg, dev, A, B, np.zeros((M, N), np.float32), 1.0, 0.0)
    assert np.array_equal(cv.result().view(np.uint32), B.view(np.uint32))


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (4097, 4095, 4093), (8192, 2048, 4096)])
def test_all_ones_gives_K(fg, dev, M, N, K):
    A = torch.ones((M, K), dtype=torch.float32, device=dev)
    B = torch.ones((K, N), dtype=torch.float32, device=dev)
    C = torch.full((M, N), 2.0, dtype=torch.float32, device=dev)
    fg.sgemm(A, B, C, 0.5, 3.0)
    torch.cuda.synchronize()
    assert torch.all(C == 0.5 * K + 6.0).item()


def test_rank1_is_correctly_rounded(fg, dev):
    M, N = 513, 257
    rng = np.random.default_rng(3)
    a = rng.uniform(-1, 1, (M, 1)).astype(np.float32)
    b = rng.uniform(-1, 1, (1, N)).astype(np.float32)
    for c in fg.configs():
        cv = run(fg, dev, a, b, np.zeros((M, N), np.float32), 1.0, 0.0, cfg=c["id"])
        assert np.array_equal(cv.result(), a * b), f"cfg {c['id']} {c['path_name']}"


# ---------------------------------------------------------------------------
# Edge cases.

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (1, 300, 7), (300, 1, 7), (5, 5, 1), (33, 65, 17),
                                   (257, 129, 3), (64, 64, 64)])
def test_tiny_and_thin(fg, dev, orc, M, N, K):
    A, B, C = inputs.make_random(M, N, K, seed=M * 1000 + N + K)
    _, r64 = orc.sgemm(A, B, C, 0.5, 3.0)
    cv = run(fg, dev, A, B, C, 0.5, 3.0)
    assert cv.untouched()
    check_close(cv.result(), r64, K, A, B, f"{M}x{N}x{K}")


def test_K_zero_scales_C(fg, dev):
    C = inputs.make_random(70, 90, 1, seed=2)[2]
    A = torch.empty((70, 0), dtype=torch.float32, device=dev)
    B = torch.empty((0, 90), dtype=torch.float32, device=dev)
    cv = Canvas(C, 95, 2, dev)
    fg.sgemm(A, B, cv.view, 0.5, 3.0)
    torch.cuda.synchronize()
    assert cv.untouched()
    assert np.array_equal(cv.result(), (3.0 * C.astype(np.float64)).astype(np.float32))


def test_M_or_N_zero_touches_nothing(fg, dev):
    big = torch.full((10, 10), CANARY, dtype=torch.int32, device=dev)
    f = big.view(torch.float32)
    A = torch.ones((0, 4), dtype=torch.float32, device=dev)
    B = torch.ones((4, 10), dtype=torch.float32, device=dev)
    fg.sgemm(A, B, f[:0], 1.0, 1.0)
    fg.sgemm(torch.ones((10, 4), device=dev), torch.ones((4, 0), device=dev), f[:, :0], 1.0, 1.0)
    torch.cuda.synchronize()
    assert torch.all(big == CANARY).item()


def test_alpha_zero_and_beta_zero(fg, dev, orc):
    M, N, K = 300, 200, 100
    A, B, C = inputs.make_random(M, N, K, seed=4)
    cv = run(fg, dev, A, B, C, 0.0, 3.0)
    assert np.array_equal(cv.result(), (3.0 * C.astype(np.float64)).astype(np.float32))
    # beta == 0: the old C must not matter (finite "dirty" C).
    _, r64 = orc.sgemm(A, B, np.zeros_like(C), 1.0, 0.0)
    cv = run(fg, dev, A, B, C, 1.0, 0.0)
    check_close(cv.result(), r64, K, A, B, "beta=0 dirty C")
    # Bit-for-bit against zero C with a deterministic configuration (split-K
    # tiles commit their atomics in any order).
    det = fg.plan(M, N, K, 1 << 40, K, 2 << 40, N, 4 << 40, N)["cfg_id"]
    if fg.config_info(det)["opt"] & 8:
        det = [c["id"] for c in fg.configs() if not c["opt"] & 8][0]
    cv = run(fg, dev, A, B, C, 1.0, 0.0, cfg=det)
    cv0 = run(fg, dev, A, B, np.zeros_like(C), 1.0, 0.0, cfg=det)
    assert np.array_equal(cv.result(), cv0.result())


def _nonfinite_like(C):
    bad = np.full(C.shape, np.nan, dtype=np.float32)
    bad.reshape(-1)[1::3] = np.inf
    bad.reshape(-1)[2::3] = -np.inf
    return bad


def test_beta_zero_never_reads_C(fg, dev, orc):
    """With beta == 0 the old C is not read, so NaN and infinities in it must
    not reach the result.  One configuration of every (path, options) class
    in both variants on ragged shapes, a split-K configuration whose tail is
    split (the pre-pass writes zeros), the default dispatch, and K == 0
    (an empty sum: zeros).  Integer inputs, so each result is exact."""
    for M, N, K in (SHAPE_VEC, SHAPE_SCALAR):
        A, B, C = inputs.make_small_int(M, N, K, seed=41 + M)
        want, _ = orc.sgemm(A, B, np.zeros_like(C), 0.5, 0.0)
        bad = _nonfinite_like(C)
        seen = {}
        for c in fg.configs():
            seen.setdefault((c["path"], c["opt"]), c["id"])
        for cfg in [-1] + sorted(seen.values()):
            cv = run(fg, dev, A, B, bad, 0.5, 0.0, cfg=cfg)
            assert cv.untouched(), f"cfg {cfg}: wrote outside C"
            got = cv.result()
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (M, N, K, cfg)
        log(f"[beta0] {M}x{N}x{K}: {len(seen)} configuration classes")
    M, N, K = 4097, 4095, 130
    A, B, C = inputs.make_small_int(M, N, K, seed=43)
    want, _ = orc.sgemm(A, B, np.zeros_like(C), 0.5, 0.0)
    split = None
    for c in fg.configs():
        if c["opt"] & 8:
            plan = fg.plan(M, N, K, 1 << 40, K, 2 << 40, N, 4 << 40, N, c["id"])
            if plan["splits"] > 1 and plan["tiles_full"] > 0:
                split = c["id"]
                break
    assert split is not None, "no configuration split a tail"
    for cfg in (split, -1):
        cv = run(fg, dev, A, B, _nonfinite_like(C), 0.5, 0.0, cfg=cfg, ldc_pad=0, guard=1)
        assert cv.untouched()
        got = cv.result()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), cfg
    cv = Canvas(_nonfinite_like(np.zeros((70, 90), np.float32)), 95, 2, dev)
    fg.sgemm(torch.empty((70, 0), device=dev), torch.empty((0, 90), device=dev), cv.view, 0.5, 0.0)
    torch.cuda.synchronize()
    assert cv.untouched()
    assert np.array_equal(cv.result(), np.zeros((70, 90), np.float32))


def test_alpha_beta_linearity(fg, dev, orc):
    M, N, K = 384, 320, 256
    A, B, C = inputs.make_random(M, N, K, seed=8)
    P = run(fg, dev, A, B, np.zeros_like(C), 1.0, 0.0).result().astype(np.float64)
    for alpha, beta in [(0.5, 3.0), (-2.0, 0.25)]:
        got = run(fg, dev, A, B, C, alpha, beta).result().astype(np.float64)
        want = alpha * P + beta * C.astype(np.float64)
        assert np.max(np.abs(got - want)) / (K * np.abs(A).max() * np.abs(B).max()) <= 2 * TOL


@pytest.mark.parametrize("pad", [3, 64])
def test_padded_leading_dimensions(fg, dev, orc, pad):
    M, N, K = 515, 260, 300
    A, B, C = inputs.make_random(M, N, K, seed=pad)
    _, r64 = orc.sgemm(A, B, C, 0.5, 3.0)
    Abig = torch.full((M, K + pad), float("nan"), device=dev)
    Bbig = torch.full((K, N + pad), float("nan"), device=dev)
    Abig[:, :K] = torch.from_numpy(A).to(dev)
    Bbig[:, :N] = torch.from_numpy(B).to(dev)
    cv = Canvas(C, N + pad, 2, dev)
    fg.sgemm(Abig[:, :K], Bbig[:, :N], cv.view, 0.5, 3.0)
    torch.cuda.synchronize()
    assert cv.untouched()
    check_close(cv.result(), r64, K, A, B, f"pad {pad}")


def test_misaligned_pointers_use_scalar_variant(fg, dev, orc):
    M, N, K = 200, 256, 128
    A, B, C = inputs.make_random(M, N, K, seed=9)
    _, r64 = orc.sgemm(A, B, C, 1.0, 1.0)
    Abuf = torch.zeros(M * K + 1, device=dev)
    Abuf[1:] = torch.from_numpy(A.ravel()).to(dev)
    Aoff = Abuf[1:].view(M, K)
    assert Aoff.data_ptr() % 16 != 0
    cv = Canvas(C, N, 1, dev)
    fg.sgemm(Aoff, to_dev(B, dev), cv.view, 1.0, 1.0)
    torch.cuda.synchronize()
    check_close(cv.result(), r64, K, A, B, "misaligned A")


def test_misaligned_operands_every_direct_lds_config(fg, dev, orc):
    # A and B 4, 8 or 12 bytes past a 16-byte boundary (aligned shape and
    # leading dimensions): the scalar variant, whose direct-LDS matrix-core
    # kernels issue 16-byte loads at these 4-byte-aligned addresses.  NaN
    # fills the buffers around the operands; C sits inside canaries.
    M, N, K = 200, 256, 128
    A, B, C = inputs.make_random(M, N, K, seed=19)
    _, r64 = orc.sgemm(A, B, C, 0.5, 3.0)
    cfgs = [c for c in fg.configs() if c["opt"] & 16]
    for offa, offb in ((1, 2), (3, 1)):
        log(f"[misaligned] A +{4 * offa} B +{4 * offb} bytes: {len(cfgs)} configs")
        Abuf = torch.full((M * K + 8,), float("nan"), device=dev)
        Bbuf = torch.full((K * N + 8,), float("nan"), device=dev)
        Abuf[offa:offa + M * K] = to_dev(A.ravel(), dev)
        Bbuf[offb:offb + K * N] = to_dev(B.ravel(), dev)
        Aoff = Abuf[offa:offa + M * K].view(M, K)
        Boff = Bbuf[offb:offb + K * N].view(K, N)
        pl = fg.plan(M, N, K, Aoff.data_ptr(), K, Boff.data_ptr(), N, 1 << 40, N)
        assert pl["vector_variant"] == 0
        for c in cfgs:
            cv = Canvas(C, N, 2, dev)
            fg.sgemm_ex(Aoff, Boff, cv.view, 0.5, 3.0, cfg_id=c["id"])
            torch.cuda.synchronize()
            assert cv.untouched(), f"cfg {c['id']}: wrote outside C"
            check_close(cv.result(), r64, K, A, B, f"cfg {c['id']} misaligned {offa},{offb}")


def test_split_plan_uses_the_launched_kernels_occupancy(fg, dev):
    # The two variants of a tuple launch different kernels whose occupancies
    # can differ; the plan's resident slots must be the launched kernel's
    # (its workgroups per CU times the CUs), for N odd and N % 4 == 0 alike.
    fake = 1 << 40
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    seen = checked = 0
    for c in fg.configs():
        t = c["tuple"]
        if not (t[11] & 16 and t[9] != 0 and t[8] == 256):
            continue
        occ_s = c["resources_scalar"]["Occupancy"]
        occ_v = c["resources_vec"]["Occupancy"]
        if (160 * 1024) // c["lds_bytes"] < max(occ_s, occ_v):
            continue  # LDS, not registers, bounds the residency
        p0 = fg.plan(2000, 2001, 999, fake, 999, 2 * fake, 2001, 4 * fake, 2001, c["id"])
        p1 = fg.plan(2000, 2000, 999, fake, 999, 2 * fake, 2000, 4 * fake, 2000, c["id"])
        pv = fg.plan(2000, 2000, 1000, fake, 1000, 2 * fake, 2000, 4 * fake, 2000, c["id"])
        assert p0["vector_variant"] == 0 and p1["vector_variant"] == 0 and pv["vector_variant"] == 1
        # 256 threads are one wave per SIMD: workgroups per CU = waves per SIMD.
        assert p0["slots"] == cus * occ_s, (t, p0["slots"], occ_s)
        assert p1["slots"] == cus * occ_s, (t, p1["slots"], occ_s)
        assert pv["slots"] == cus * occ_v, (t, pv["slots"], occ_v)
        seen += occ_s != occ_v
        checked += 1
    log(f"[occupancy] {checked} tuples checked, {seen} whose two variants differ in occupancy")
    assert checked > 0


def test_transpose_identity_bit_exact(fg, dev):
    M, N, K = 8192 // 4, 2048 // 2, 777
    A, B, C = inputs.make_small_int(M, N, K, seed=10)
    Z = np.zeros((M, N), np.float32)
    c1 = run(fg, dev, A, B, Z, 1.0, 0.0).result()
    c2 = run(fg, dev, np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), Z.T.copy(), 1.0, 0.0).result()
    assert np.array_equal(c1.view(np.uint32), np.ascontiguousarray(c2.T).view(np.uint32))


def test_overlap_rejected(fg, dev):
    X = torch.zeros((256, 256), device=dev)
    with pytest.raises(fg.SgemmError) as e:
        fg.sgemm(X, X, X, 1.0, 0.0)
    assert e.value.status == 3


def _launch_efficiency(c, M, N, K, slots):
    """Busy share of the resident slots, as the launcher splits a partly
    filled last wave of a split-K configuration; 0 for a launch that splits
    every tile."""
    tiles = -(-M // c["BM"]) * -(-N // c["BN"])
    grid = tiles
    if c["opt"] & 8:
        tail, nk = tiles % slots, -(-K // c["BK"])
        if tail and 2 * tail <= slots and nk >= 2:
            s = min(slots // tail, nk)
            if s >= 2:
                if tail == tiles:
                    return 0.0
                grid = tiles - tail + tail * s
    return grid / (-(-grid // slots) * slots)


def test_rule_dispatch_fills_the_device(fg, dev):
    # Aligned shapes outside the measured-rate table's range (M or N below
    # 128) with at least 2^30 FLOP and K >= 256 choose among the aligned
    # rules: of those whose launch keeps at least 85 % of the resident slots
    # busy (the split of a partly filled last wave counted, a launch that
    # splits every tile not), one with the largest block tile; with none,
    # the nearest rule in (log M, log N, log K).
    import math
    import re
    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                             "fp32_gemm_amd", "csrc", "tuned_table.inc")).read()
    rules = {(int(M), int(N), int(K)): tuple(int(x) for x in t.split(","))
             for M, N, K, t in re.findall(r"\{(\d+), (\d+), (\d+), \{([\d, ]+)\}\}", text)
             if int(N) % 4 == 0 and int(K) % 4 == 0}
    ids = {tuple(c["tuple"]): c["id"] for c in fg.configs()}
    fake = 1 << 40
    for M, N, K in [(100, 8192, 8192), (120, 16384, 4096), (8192, 100, 8192), (64, 30000, 4096)]:
        assert (M, N, K) not in rules and 2 * M * N * K >= 1 << 30
        p = fg.plan(M, N, K, fake, K, 2 * fake, N, 4 * fake, N)
        c = fg.config_info(p["cfg_id"])
        eff = {}
        for t in set(rules.values()):
            ci = fg.config_info(ids[t])
            slots = fg.plan(M, N, K, fake, K, 2 * fake, N, 4 * fake, N, ids[t])["slots"]
            assert slots > 0
            eff[t] = _launch_efficiency(ci, M, N, K, slots)
        fit = [t for t, e in eff.items() if e >= 0.85]
        log(f"[rule fill] {M}x{N}x{K}: {c['tuple']}, {len(fit)} rules fill the device")
        if fit:
            assert eff[tuple(c["tuple"])] >= 0.85, (M, N, K, c["tuple"])
            assert c["BM"] * c["BN"] == max(t[0] * t[1] for t in fit), (M, N, K, c["tuple"])
        else:
            d = {s: sum(math.log2(a / b) ** 2 for a, b in zip((M, N, K), s)) for s in rules}
            assert tuple(c["tuple"]) == rules[min(d, key=d.get)], (M, N, K, c["tuple"])


def test_graph_capture_replays(fg, dev, orc):
    # sgemm_ex records into a stream capture like any launch on that stream
    # (the split-K pre-pass is a kernel, not a memset).  Each replay, with
    # eager work and synchronisation in between, must reproduce the eager
    # result: bit for bit where the configuration is deterministic, within
    # the tolerance for a split configuration (its atomics commit in any
    # order).
    M, N, K = 600, 520, 300
    A, B, C = inputs.make_random(M, N, K, seed=31)
    _, r64 = orc.sgemm(A, B, C, 0.5, 3.0)
    Ad, Bd, C0 = to_dev(A, dev), to_dev(B, dev), to_dev(C, dev)
    split = [c["id"] for c in fg.configs() if c["opt"] & 8 and c["opt"] & 16][0]
    for cfg in (-1, split):
        log(f"[graph] cfg {cfg}")
        Ce = C0.clone()
        fg.sgemm_ex(Ad, Bd, Ce, 0.5, 3.0, cfg_id=cfg)
        torch.cuda.synchronize()
        eager = Ce.cpu().numpy()
        check_close(eager, r64, K, A, B, f"eager cfg {cfg}")
        Cg = C0.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fg.sgemm_ex(Ad, Bd, Cg, 0.5, 3.0, cfg_id=cfg)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fg.sgemm_ex(Ad, Bd, Cg, 0.5, 3.0, cfg_id=cfg)
        for rep in range(4):
            Cg.copy_(C0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = Cg.cpu().numpy()
            chosen = cfg if cfg >= 0 else fg.plan(M, N, K, Ad.data_ptr(), K, Bd.data_ptr(), N,
                                                  Cg.data_ptr(), N)["cfg_id"]
            if fg.config_info(chosen)["opt"] & 8:
                check_close(got, r64, K, A, B, f"replay {rep} cfg {cfg}")
            else:
                assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), f"replay {rep}"


def test_side_stream(fg, dev, orc):
    M, N, K = 512, 512, 512
    A, B, C = inputs.make_random(M, N, K, seed=11)
    _, r64 = orc.sgemm(A, B, C, 0.5, 3.0)
    s = torch.cuda.Stream()
    Ad, Bd, Cd = to_dev(A, dev), to_dev(B, dev), to_dev(C, dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        fg.sgemm_ex(Ad, Bd, Cd, 0.5, 3.0, stream=s)
    s.synchronize()
    check_close(Cd.cpu().numpy(), r64, K, A, B, "side stream")
