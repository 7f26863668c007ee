"""CPU tests of the bench regression check (tests/bench_regression.py)."""
import json

import bench_regression as br


def _line(step_ms, prefill_ms, extra_name="prefill_C4"):
    return {"metric": "m", "ms_per_step": step_ms,
            "extra": {extra_name: {"ms_per_step": prefill_ms + 0.01,
                                   "prefill_call_ms": {"mean": prefill_ms, "median": prefill_ms}},
                      "decode_F1": {"decode_only_call_ms": {"median": 0.03}}}}


def _write(tmp_path, name, obj, wrap=False, noise=False):
    p = tmp_path / name
    text = json.dumps({"parsed": obj} if wrap else obj)
    if noise:
        text = "[bench] building\n[bench] timing\n" + text + "\n"
    p.write_text(text)
    return str(p)


def test_identical_results_pass(tmp_path):
    a = _write(tmp_path, "a.json", _line(0.046, 0.100))
    assert br.main([a, a]) == 0


def test_eleven_percent_slower_fails_nine_percent_passes(tmp_path):
    base = _write(tmp_path, "a.json", _line(0.046, 0.100))
    slow = _write(tmp_path, "b.json", _line(0.046, 0.111))
    ok = _write(tmp_path, "c.json", _line(0.046 * 1.09, 0.109))
    assert br.main([base, slow]) == 1
    assert br.main([base, ok]) == 0
    assert br.main([base, slow, "--threshold", "0.2"]) == 0


def test_faster_is_not_a_regression(tmp_path):
    base = _write(tmp_path, "a.json", _line(0.046, 0.100))
    fast = _write(tmp_path, "b.json", _line(0.030, 0.050))
    assert br.main([base, fast]) == 0


def test_reads_driver_records_and_bench_logs(tmp_path):
    base = _write(tmp_path, "a.json", _line(0.046, 0.100), wrap=True)
    new = _write(tmp_path, "b.json", _line(0.060, 0.100), noise=True)
    rows, regressed, _ = br.compare(br.load_line(base), br.load_line(new))
    assert regressed == ["ms_per_step"]
    assert {r[0] for r in rows} == {"ms_per_step", "prefill_C4.ms_per_step",
                                    "prefill_C4.prefill_call_ms.median",
                                    "decode_F1.decode_only_call_ms.median"}


def test_one_sided_quantities_are_skipped(tmp_path):
    base = _write(tmp_path, "a.json", _line(0.046, 0.100, extra_name="prefill_C4"))
    new = _write(tmp_path, "b.json", _line(0.046, 0.500, extra_name="prefill_C4i8"))
    rows, regressed, only = br.compare(br.load_line(base), br.load_line(new))
    assert not regressed and "prefill_C4i8.prefill_call_ms.median" in only
    assert br.main([base, new]) == 0


def test_unreadable_input(tmp_path):
    p = tmp_path / "x.json"
    p.write_text("not json at all\n")
    assert br.main([str(p), str(p)]) == 2
