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
    results = {
        k1: (t1, [(102.0, other), (100.0, t1)]),     # leads by 2 %: the rule moves
        k2: (t2, [(100.5, other), (100.0, t2)]),     # 0.5 %: the rule stays
    }
    changed = tune.update_table(str(path), results)
    after = _rules(path)
    assert changed == [(k1, t1, other)]
    assert after[k1][0] == other and "102.0 TFLOP/s (re-timed)" in after[k1][1]
    assert after[k2][0] == t2 and "100.0 TFLOP/s (re-timed)" in after[k2][1]
    for k in before:
        if k not in (k1, k2):
            assert after[k] == before[k]
    text = path.read_text()
    assert "kDefaultLarge" in text and text.count("{") == open(TABLE).read().count("{")
