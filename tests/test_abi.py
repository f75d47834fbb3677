"""The C ABI on the CPU: the library loads, exports every function the header
declares, and validates arguments before touching any device."""
import ctypes
import json
import math
import os
import re
import subprocess

import pytest

import fp32_gemm_amd as fg
from fp32_gemm_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp32_gemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sgemm\w*)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_api():
    names = declared_functions()
    assert "sgemm" in names and "sgemm_ex" in names
    assert names == binding.exported_symbols()


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fg.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fg.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (sgemm\w*)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


FAKE = 1 << 40  # a well-aligned, never-dereferenced address


def plan(M, N, K, lda, ldb, ldc, A=FAKE, B=FAKE * 2, C=FAKE * 4, cfg=-1):
    try:
        return 0, binding.plan(M, N, K, A, lda, B, ldb, C, ldc, cfg)
    except fg.SgemmError as e:
        return e.status, None


@pytest.mark.parametrize("args,code", [
    ((-1, 4, 4, 4, 4, 4), -1),
    ((4, -1, 4, 4, 4, 4), -2),
    ((4, 4, -1, 4, 4, 4), -3),
    ((4, 4, 8, 7, 4, 4), -6),
    ((4, 8, 4, 4, 7, 8), -8),
    ((4, 8, 4, 4, 8, 7), -11),
    ((4, 4, 4, 1 << 21, 4, 4), 5),
    ((2 ** 30 + 1, 4, 4, 4, 4, 4), 5),
])
def test_argument_codes(args, code):
    assert plan(*args)[0] == code


def test_tile_count_beyond_int32_is_unsupported():
    # 2^30 x (2^21 - 1) outputs need more than 2^31 - 1 workgroups with any
    # compiled tile; the sizes themselves are within the limits.
    M, N = 1 << 30, (1 << 21) - 1
    for cfg in (0, fg.num_configs() - 1):
        assert plan(M, N, 4, 4, N, N, cfg=cfg)[0] == 5
    assert plan(M, 64, 4, 4, 64, 64, cfg=0)[0] == 0


def test_null_pointers():
    assert plan(4, 4, 4, 4, 4, 4, A=None)[0] == -5
    assert plan(4, 4, 4, 4, 4, 4, B=None)[0] == -7
    assert plan(4, 4, 4, 4, 4, 4, C=None)[0] == -10
    # Empty operands may be NULL.
    assert plan(4, 4, 0, 1, 4, 4, A=None, B=None)[0] == 0
    assert plan(0, 0, 4, 4, 1, 1, A=None, B=FAKE, C=None)[0] == 0


def test_overlap_is_rejected():
    # C's extent starts inside A's extent.
    assert plan(64, 64, 64, 64, 64, 64, A=FAKE, B=FAKE * 2, C=FAKE + 1024)[0] == 3
    assert plan(64, 64, 64, 64, 64, 64, A=FAKE, B=FAKE * 2, C=FAKE * 2 + 64)[0] == 3
    # Adjacent but disjoint.
    assert plan(64, 64, 64, 64, 64, 64, A=FAKE, B=FAKE * 2, C=FAKE + 64 * 64 * 4)[0] == 0


def test_variant_selection():
    code, p = plan(256, 256, 256, 256, 256, 256)
    assert code == 0 and p["vector_variant"] == 1
    assert plan(256, 256, 255, 255, 256, 256)[1]["vector_variant"] == 0   # K % 4
    assert plan(256, 255, 256, 256, 255, 255)[1]["vector_variant"] == 0   # N % 4
    assert plan(256, 256, 256, 260, 256, 258)[1]["vector_variant"] == 0   # ldc % 4
    assert plan(256, 256, 256, 256, 256, 256, A=FAKE + 4)[1]["vector_variant"] == 0  # alignment


def test_bad_config_id():
    assert plan(4, 4, 4, 4, 4, 4, cfg=fg.num_configs())[0] == 2
    with pytest.raises(fg.SgemmError):
        fg.config_info(-1)


def test_tuned_dispatch_picks_a_compiled_config():
    for M, N, K in [(4096, 4096, 4096), (256, 256, 256), (1000, 1500, 777), (8192, 2048, 4096),
                    (1, 1, 1), (4097, 4095, 4093)]:
        code, p = plan(M, N, K, K, N, N)
        assert code == 0
        info = fg.config_info(p["cfg_id"])
        assert p["block"] == info["NT"]
        assert p["grid"] == -(-M // info["BM"]) * -(-N // info["BN"])


def test_tuned_table_tuples_are_compiled():
    # Every rule and default of the tuned table names a compiled tuple, and
    # each tuned shape dispatches to exactly that tuple.
    text = open(os.path.join(ROOT, "fp32_gemm_amd", "csrc", "tuned_table.inc")).read()
    compiled = {tuple(c["tuple"]) for c in fg.configs()}
    rules = re.findall(r"\{(\d+), (\d+), (\d+), \{([\d, ]+)\}\}", text)
    assert rules
    for M, N, K, tup in rules:
        t = tuple(int(x) for x in tup.split(","))
        assert t in compiled, t
        code, p = plan(int(M), int(N), int(K), int(K), int(N), int(N))
        assert code == 0 and tuple(fg.config_info(p["cfg_id"])["tuple"]) == t
    for d in re.findall(r"Tile kDefault\w+\{([\d, ]+)\}", text):
        assert tuple(int(x) for x in d.split(",")) in compiled


def test_off_table_rules_follow_the_variant():
    # Outside the measured-rate table's range (M or N below 128, or K below
    # 32) a shape takes a rule tuned on a shape of its own variant: the
    # ragged rules (tuned where only the 4-byte scalar variant runs) serve
    # unaligned shapes, the aligned rules aligned ones, even where a ragged
    # rule's shape is nearer.  Without a device the fill check (it needs the
    # device's occupancy) counts every launch as full, and the nearest such
    # rule is reported.
    rules = _table_rules()
    import torch
    if torch.cuda.is_available():
        pytest.skip("the fill check changes the choice on a device")

    def nearest(M, N, K, aligned=None):
        d = {s: sum(math.log2(a / b) ** 2 for a, b in zip((M, N, K), s))
             for s in rules if aligned is None or (s[2] % 4 == 0 and s[1] % 4 == 0) == aligned}
        return min(d, key=d.get)

    # 120 x 1500 x 776 lies nearest the ragged 1000 x 1500 x 777 rule.
    assert nearest(120, 1500, 776) == (1000, 1500, 777)
    code, p = plan(120, 1500, 776, 776, 1500, 1500)
    assert code == 0 and p["vector_variant"] == 1
    assert tuple(fg.config_info(p["cfg_id"])["tuple"]) == rules[nearest(120, 1500, 776, True)]
    assert nearest(120, 1500, 776, True) != (1000, 1500, 777)
    for M, N, K in ((100, 3001, 2999), (5000, 64, 777), (3000, 3001, 20)):
        code, p = plan(M, N, K, K, N, N)
        assert code == 0 and p["vector_variant"] == 0
        assert tuple(fg.config_info(p["cfg_id"])["tuple"]) == rules[nearest(M, N, K, False)], (M, N, K)


def _table_rules():
    text = open(os.path.join(ROOT, "fp32_gemm_amd", "csrc", "tuned_table.inc")).read()
    return {(int(M), int(N), int(K)): tuple(int(x) for x in t.split(","))
            for M, N, K, t in re.findall(r"\{(\d+), (\d+), (\d+), \{([\d, ]+)\}\}", text)}


def _rate_table():
    text = open(os.path.join(ROOT, "fp32_gemm_amd", "csrc", "measured_rates.inc")).read()
    tiles_text = text[text.index("kRateTiles[]"):text.index("kScalarRows[]")]
    cols = [tuple(int(x) for x in t.split(",")) for t in re.findall(r"\{([\d, ]+)\},\s*// column", tiles_text)]

    def rows(body):
        return [((int(M), int(N), int(K)), [int(x) for x in pct.split(",")])
                for M, N, K, pct in re.findall(r"\{(\d+), (\d+), (\d+), \{([\d, ]+)\}\}", body)]

    scalar = rows(text[text.index("kScalarRows[]"):text.index("kVectorRows[]")])
    vector = rows(text[text.index("kVectorRows[]"):])
    return cols, scalar, vector


def test_rate_table_is_well_formed():
    # Every column names a compiled tuple; every row is a distinct shape of
    # its variant (N or K not a multiple of 4 for the scalar rows, both
    # multiples of 4 for the float4 rows), holds one percentage per column,
    # and has its fastest column at 100.
    cols, scalar, vector = _rate_table()
    compiled = {tuple(c["tuple"]) for c in fg.configs()}
    assert cols and scalar and vector and len(cols) <= 32
    assert all(c in compiled for c in cols)
    for rows, aligned in ((scalar, False), (vector, True)):
        assert len({s for s, _ in rows}) == len(rows)
        for (M, N, K), pct in rows:
            assert (N % 4 == 0 and K % 4 == 0) == aligned, (M, N, K)
            assert len(pct) == len(cols) and max(pct) == 100 and min(pct) >= 1


def test_off_rule_shapes_follow_the_rate_table():
    # A shape without an exact rule, with M, N >= 128 and K >= 32, takes the
    # column with the highest sum over the 16 nearest rows (in log2 M, log2 N
    # and log2 K, the K difference weighing one half) of
    # exp(-squared distance) * log(percentage / 100); a shape that is a row
    # takes that row's fastest column.  Float4 shapes read the float4 rows;
    # scalar-variant shapes read them too, among the tiles whose scalar
    # kernel keeps 16-byte loads (direct-LDS matrix-core tiles).
    # The choice needs no device, so this holds on any host.
    cols, scalar, vector = _rate_table()
    rules = _table_rules()

    def hybrid(t):
        return bool(t[11] & 16) and t[9] != 0

    def expected(M, N, K, vec):
        rows = vector
        allowed = [c for c in range(len(cols)) if vec or hybrid(cols[c])]
        x = (math.log2(M), math.log2(N), math.log2(K))
        d = sorted(((x[0] - math.log2(s[0])) ** 2 + (x[1] - math.log2(s[1])) ** 2 +
                    0.5 * (x[2] - math.log2(s[2])) ** 2, i) for i, (s, _) in enumerate(rows))[:16]
        if d[0][0] == 0.0:
            pct = rows[d[0][1]][1]
            return cols[max(allowed, key=lambda c: pct[c])]
        score = {c: sum(math.exp(-dd) * math.log(rows[i][1][c] / 100.0) for dd, i in d) for c in allowed}
        return cols[max(allowed, key=lambda c: score[c])]

    cases = [(4000, 4001, 4003), (3603, 2045, 218), (1269, 7747, 321), (706, 1029, 963), (128, 129, 32),
             (20001, 300, 5001), (1000, 1000, 1001), (4000, 4000, 4000), (12288, 12288, 1024),
             (128, 128, 32), (894, 324, 5236), (30000, 20000, 8192), (8192, 8192, 8191)]
    cases += [s for s, _ in scalar[:2]] + [s for s, _ in vector[:2]]
    kinds = set()
    for M, N, K in cases:
        assert (M, N, K) not in rules
        code, p = plan(M, N, K, K, N, N)
        assert code == 0 and p["vector_variant"] == (N % 4 == 0 and K % 4 == 0)
        vec = p["vector_variant"] == 1
        kinds.add("vec" if vec else "b16" if N % 4 == 0 else "scalar")
        assert tuple(fg.config_info(p["cfg_id"])["tuple"]) == expected(M, N, K, vec), (M, N, K)
    assert kinds == {"vec", "b16", "scalar"}
    # Unaligned operands of an aligned shape: the scalar variant, N % 4 == 0.
    code, p = plan(4000, 4000, 4000, 4001, 4000, 4000)
    assert code == 0 and p["vector_variant"] == 0
    t = tuple(fg.config_info(p["cfg_id"])["tuple"])
    assert t == expected(4000, 4000, 4000, False) and hybrid(t)
    # An exact rule still wins over the table.
    for s, t in rules.items():
        code, p = plan(*s, s[2], s[1], s[1])
        assert tuple(fg.config_info(p["cfg_id"])["tuple"]) == t


def test_quick_return_and_no_device():
    # M == 0: nothing to do, success without a device.
    assert binding.sgemm_raw(0, 4, 4, 1.0, FAKE, 4, FAKE * 2, 4, 0.0, FAKE * 4, 4) == 0
    # Only where the library's own device check fails: then sgemm returns
    # before any launch, so the never-mapped addresses are not touched.
    if fg.device_check() != 0:
        assert fg.device_check() == 1
        assert binding.sgemm_raw(4, 4, 4, 1.0, FAKE, 4, FAKE * 2, 4, 0.0, FAKE * 4, 4) == 1


def test_status_strings():
    for code in (0, -1, -2, -3, -5, -6, -7, -8, -10, -11, 1, 2, 3, 4, 5):
        s = fg.status_string(code)
        assert s and s != "unknown status"
    assert fg.status_string(12345) == "unknown status"


def test_config_table_contents():
    cfgs = fg.configs()
    paths = {c["path_name"] for c in cfgs}
    assert paths == {"valu", "mfma32", "mfma16"}
    for c in cfgs:
        assert c["WMITER"] * c["WSUBM"] == c["WM"] and c["WNITER"] * c["WSUBN"] == c["WN"]
        assert c["lds_bytes"] <= 160 * 1024
        assert c["resources_vec"] is not None and c["resources_scalar"] is not None


def test_scalar_variant_kernels_per_tuple():
    # Every tuple has one scalar-variant kernel in the build's resource
    # report; for the direct-LDS matrix-core tuples it is the hybrid kernel
    # (16-byte loads but for slice 0's A), one per tuple.
    with open(fg.binding._RESOURCES) as f:
        names = list(json.load(f))
    hyb = sum(1 for n in names if "sgemm_tile_kernel_hyb" in n)
    hybrid = 0
    for c in fg.configs():
        t = c["tuple"]
        assert c["resources_scalar"] is not None
        hybrid += bool(t[11] & 16 and t[9] != 0)
    assert hybrid > 0 and hyb == hybrid


def test_default_configs_do_not_spill():
    for M, N, K in [(4096, 4096, 4096), (256, 256, 256), (1024, 1024, 1024)]:
        _, p = plan(M, N, K, K, N, N)
        c = fg.config_info(p["cfg_id"])
        res = [x for x in fg.configs() if x["id"] == c["id"]][0]
        assert res["resources_vec"]["ScratchSize"] == 0
        assert res["resources_scalar"]["ScratchSize"] == 0


def test_ladder_argument_handling():
    lib = ctypes.CDLL(fg.library_path())
    f = lib.sgemm_ladder
    f.argtypes = binding._SIGS["sgemm_ladder"][0]
    f.restype = ctypes.c_int
    # bad rung before anything else
    assert f(0, 4, 4, 4, 1.0, FAKE, 4, FAKE * 2, 4, 0.0, FAKE * 4, 4, None) == 2
    assert f(5, 4, 4, 4, 1.0, FAKE, 4, FAKE * 2, 4, 0.0, FAKE * 4, 4, None) == 2
    # argument validation, same codes as sgemm_ex
    assert f(1, -1, 4, 4, 1.0, FAKE, 4, FAKE * 2, 4, 0.0, FAKE * 4, 4, None) == -1
    assert f(1, 4, 4, 8, 1.0, FAKE, 7, FAKE * 2, 4, 0.0, FAKE * 4, 4, None) == -6
    assert f(1, 0, 4, 4, 1.0, FAKE, 4, FAKE * 2, 4, 0.0, FAKE * 4, 4, None) == 0
    import torch
    if not torch.cuda.is_available():
        assert f(1, 4, 4, 4, 1.0, FAKE, 4, FAKE * 2, 4, 0.0, FAKE * 4, 4, None) == 1


def test_binding_rejects_overlapping_rows():
    """Expanded or overlapping rows have no leading dimension; the binding
    refuses them instead of describing them as a dense matrix (which would
    make the kernels read past the storage)."""
    import torch
    with pytest.raises(ValueError, match="overlap"):
        binding._operand(torch.zeros(1, 8).expand(4, 8), "A")
    with pytest.raises(ValueError, match="overlap"):
        binding._operand(torch.zeros(64).as_strided((4, 8), (4, 1)), "C")
    with pytest.raises(ValueError, match="column stride"):
        binding._operand(torch.zeros(8, 4).t(), "B")
    # A row slice of a wider buffer and a single expanded row are valid
    # layouts: they pass every layout check and stop at the device check.
    for ok in (torch.zeros(4, 12)[:, :8], torch.zeros(1, 8).expand(1, 8), torch.zeros(5, 1)):
        with pytest.raises(ValueError, match="GPU device"):
            binding._operand(ok, "B")


CLIENT = os.path.join(ROOT, "tests", "c_client", "sgemm_client")


def test_header_is_strict_c99():
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                    "-x", "c", HEADER], check=True)


def test_c_client_device_free_calls():
    """A plain C program built against the header and the library (built by
    __graft_entry__.build()) sees the same configuration table, plan and
    status strings as the Python binding."""
    if not os.path.exists(CLIENT):
        pytest.fail("tests/c_client/sgemm_client is missing: run __graft_entry__.build()")
    out = subprocess.run([CLIENT, "info"], capture_output=True, text=True, check=True, timeout=60).stdout
    assert int(re.search(r"^configs (\d+)$", out, flags=re.M).group(1)) == fg.num_configs()
    m = re.search(r"^plan (-?\d+) cfg (\d+) vector (\d+) grid (\d+) block (\d+)$", out, flags=re.M)
    p = binding.plan(4096, 4096, 4096, FAKE, 4096, FAKE * 2, 4096, FAKE * 4, 4096)
    assert (int(m.group(1)), int(m.group(2)), int(m.group(3)), int(m.group(4)), int(m.group(5))) == \
        (0, p["cfg_id"], p["vector_variant"], p["grid"], p["block"])
    assert f"status -6 {fg.status_string(-6)}" in out
