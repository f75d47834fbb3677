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
