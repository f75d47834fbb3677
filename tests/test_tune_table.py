"""The re-timing's table update (host only)."""
import shutil

from fp32_gemm_amd import tune

TABLE = "fp32_gemm_amd/csrc/tuned_table.inc"


def _rules(path):
    out = {}
    for line in open(path).read().split("\n"):
        m = tune._RULE.match(line)
        if m:
            out[tuple(int(m.group(i)) for i in (2, 3, 4))] = (
                tuple(int(x) for x in m.group(5).split(", ")), line)
    return out


def test_update_moves_only_rules_with_a_clear_lead(tmp_path):
    path = tmp_path / "table.inc"
    shutil.copy(TABLE, path)
    before = _rules(path)
    assert len(before) >= 8
    (k1, (t1, _)), (k2, (t2, _)) = list(before.items())[:2]
    other = (64, 128, 32, 64, 32, 1, 16, 1, 256, 1, 32, 24)
    assert other not in (t1, t2)
    new_key = (3001, 2999, 997)
    assert new_key not in before
    results = {
        k1: (t1, [(102.0, other), (100.0, t1)], "a"),     # leads by 2 %: the rule moves
        k2: (t2, [(100.5, other), (100.0, t2)], "b"),     # 0.5 %: the rule stays
        new_key: (t2, [(90.0, other), (88.0, t2)], "odd3001"),  # no rule yet: added
    }
    changed = tune.update_table(str(path), results)
    after = _rules(path)
    assert changed == [(k1, t1, other), (new_key, None, other)]
    assert after[new_key][0] == other and "odd3001 (tuning only): 90.0" in after[new_key][1]
    assert f"{{{', '.join(map(str, other))}}}}}," in after[new_key][1]
    assert len(after) == len(before) + 1
    assert after[k1][0] == other and "102.0 TFLOP/s (re-timed)" in after[k1][1]
    assert after[k2][0] == t2 and "100.0 TFLOP/s (re-timed)" in after[k2][1]
    for k in before:
        if k not in (k1, k2):
            assert after[k] == before[k]
    text = path.read_text()
    assert "kDefaultLarge" in text and text.count("{") == open(TABLE).read().count("{") + 2


def test_rate_table_rows_and_columns(tmp_path):
    # Rows per variant, each shape once (the first record), the columns the
    # tuples timed on every row, percentages of the row's best rounded and
    # floored at 1; a variant without records gets an empty marker row.
    a, b, c = "64,64,16,32,32,1,16,1,256,1,32,18", "128,128,16,64,64,4,4,1,256,2,64,24", \
        "256,256,32,128,64,2,16,1,512,1,32,27"
    recs = [
        dict(M=1000, N=1001, K=999, vec=False, rates={a: 50.0, b: 100.0, c: 0.4}),
        dict(M=300, N=301, K=302, vec=False, rates={a: 80.0, b: 40.0}),
        dict(M=1000, N=1001, K=999, vec=False, rates={a: 100.0, b: 10.0}),   # repeat: ignored
        dict(M=512, N=512, K=512, vec=True, rates={a: 1.0, b: 2.0, c: 3.0}),
    ]
    path = tmp_path / "rates.inc"
    cols, ns, nv = tune.write_rate_table(recs, str(path), "cmd")
    assert cols == [a, b] and ns == 2 and nv == 1
    text = path.read_text()
    assert "{64, 64, 16, 32, 32, 1, 16, 1, 256, 1, 32, 18},  // column 0" in text
    scalar = text[text.index("kScalarRows[]"):text.index("kVectorRows[]")]
    vector = text[text.index("kVectorRows[]"):]
    assert "{300, 301, 302, {100, 50}}" in scalar and "{1000, 1001, 999, {50, 100}}" in scalar
    assert scalar.index("{300, 301, 302") < scalar.index("{1000, 1001, 999")
    assert "{512, 512, 512, {50, 100}}" in vector and "`cmd`" in text
    cols, ns, nv = tune.write_rate_table(recs[:2], str(path), "cmd")
    assert nv == 0 and "{0, 0, 0, {}},  // none measured" in path.read_text()


def test_rate_table_gap_summary(tmp_path):
    # The sweep summary for ad-hoc shapes names the fastest swept tuple and
    # the fastest tile that the measured-rate table lists.
    text = open("fp32_gemm_amd/csrc/measured_rates.inc").read()
    first = text[text.index("kRateTiles[]"):].split("{", 2)[2].split("}")[0]
    in_table = [int(x) for x in first.split(",")]
    other = [1, 2, 3]
    swept = {"100x200x300": [dict(tuple=other, tflops=50.0), dict(tuple=in_table, tflops=40.0)]}
    path = tmp_path / "gap.md"
    tune.write_rate_table_gap(swept, str(path), "cmd")
    row = [l for l in path.read_text().split("\n") if l.startswith("| 100x200x300")][0]
    assert "| 1,2,3 | 50.0 |" in row and f"| {','.join(map(str, in_table))} | 40.0 | 0.800 |" in row


def test_rate_column_refresh(tmp_path):
    # A re-timed column takes its rate over its anchor's, times the anchor's
    # stored percentage; a column that now leads rescales the row to 100.
    # Rows of the other variant and rows not re-timed stay as they were.
    a, b, c = "64,64,16,32,32,1,16,1,256,1,32,18", "128,128,16,64,64,4,4,1,256,2,64,24", \
        "256,256,32,128,64,2,16,1,512,1,32,27"
    recs = [
        dict(M=1000, N=1001, K=999, vec=False, rates={a: 50.0, b: 100.0, c: 20.0}),
        dict(M=2000, N=2001, K=1999, vec=False, rates={a: 80.0, b: 40.0, c: 10.0}),
        dict(M=3000, N=3001, K=2999, vec=False, rates={a: 80.0, b: 40.0, c: 10.0}),
        dict(M=512, N=512, K=512, vec=True, rates={a: 1.0, b: 2.0, c: 1.0}),
    ]
    path = tmp_path / "rates.inc"
    tune.write_rate_table(recs, str(path), "cmd")
    cols, rows = tune.read_rate_table(str(path))
    assert [",".join(map(str, t)) for t in cols] == [a, b, c]
    assert rows["scalar"][1] == (2000, 2001, 1999, [100, 50, 12])
    assert rows["vector"] == [(512, 512, 512, [50, 100, 50])]
    # Row 1: column 2 at 0.6 of its anchor (column 1, 100 %) -> 60.
    # Row 2: column 2 at 1.5x its anchor (column 0, 100 %) -> leads; the
    # others scale by 1/1.5 and the best rate by 1.5.
    moved = tune.refresh_rate_column(str(path), 2, "scalar",
                                     {(1000, 1001, 999): (60.0, 1, 100.0),
                                      (2000, 2001, 1999): (150.0, 0, 100.0)}, "recmd")
    assert moved == [(2000, 2001, 1999)]
    cols2, rows2 = tune.read_rate_table(str(path))
    assert cols2 == cols
    assert rows2["scalar"][0][3] == [50, 100, 60]
    assert rows2["scalar"][1][3] == [67, 33, 100]
    assert rows2["scalar"][2] == rows["scalar"][2] and rows2["vector"] == rows["vector"]
    text = path.read_text()
    assert "{2000, 2001, 1999, {67, 33, 100}},  // best 120.0 TFLOP/s" in text
    assert "// Column 2 of the scalar rows re-timed by `recmd`" in text
    # A scalar row with N % 4 == 0 is not rewritten.
    recs[2]["N"] = 3000
    tune.write_rate_table(recs, str(path), "cmd")
    tune.refresh_rate_column(str(path), 2, "scalar", {(3000, 3000, 2999): (150.0, 0, 100.0)}, "x")
    assert tune.read_rate_table(str(path))[1]["scalar"][2] == (3000, 3000, 2999, [100, 50, 12])
