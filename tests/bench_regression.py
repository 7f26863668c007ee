"""Bench regression check: compare two benchmark results and fail when a
timed quantity got more than a threshold (default 10%) slower.

The check of TinyLoop's "Current Status" table, row "Performance regression
tracker" (a 10% default threshold), for this library's bench output.  Each
input is a file holding bench.py's JSON line (the last line that parses as
a JSON object is used) or a driver record that wraps it under "parsed".

Compared, when both sides carry them (lower is better for all):
  * the headline step time, ms_per_step;
  * for every entry of "extra": ms_per_step and the median of every
    "*_call_ms" record (decode, prefill, mixed, append calls).
Quantities present on one side only are listed and skipped.

    python tests/bench_regression.py BASE.json NEW.json [--threshold 0.10]

Exit status 0 when nothing regressed, 1 when something did, 2 for
unreadable input.  Runs on the CPU only (it reads JSON).
"""
from __future__ import annotations

import argparse
import json
import sys


def load_line(path: str) -> dict:
    """The bench line in `path`: a bench.py output file or a driver record."""
    with open(path) as f:
        text = f.read()
    try:
        obj = json.loads(text)
        return obj.get("parsed", obj) if isinstance(obj, dict) else {}
    except json.JSONDecodeError:
        pass
    for line in reversed(text.splitlines()):
        line = line.strip()
        if line.startswith("{"):
            try:
                obj = json.loads(line)
            except json.JSONDecodeError:
                continue
            if isinstance(obj, dict):
                return obj.get("parsed", obj)
    raise ValueError(f"{path}: no JSON object found")


def timed_quantities(line: dict) -> dict:
    """{name: milliseconds} of every timed quantity the line carries."""
    out = {}
    if isinstance(line.get("ms_per_step"), (int, float)):
        out["ms_per_step"] = float(line["ms_per_step"])
    extra = line.get("extra") or {}
    for key, rec in extra.items():
        if not isinstance(rec, dict):
            continue
        if isinstance(rec.get("ms_per_step"), (int, float)):
            out[f"{key}.ms_per_step"] = float(rec["ms_per_step"])
        for field, val in rec.items():
            if field.endswith("_call_ms") and isinstance(val, dict) and \
                    isinstance(val.get("median"), (int, float)):
                out[f"{key}.{field}.median"] = float(val["median"])
    return out


def compare(base: dict, new: dict, threshold: float = 0.10):
    """Returns (rows, regressed): rows of (name, base_ms, new_ms, ratio) for
    the quantities on both sides, and the names more than `threshold`
    slower (new > base * (1 + threshold))."""
    b, n = timed_quantities(base), timed_quantities(new)
    rows, regressed = [], []
    for name in sorted(set(b) & set(n)):
        ratio = n[name] / b[name] if b[name] > 0 else float("inf")
        rows.append((name, b[name], n[name], ratio))
        if ratio > 1.0 + threshold:
            regressed.append(name)
    only = sorted(set(b) ^ set(n))
    return rows, regressed, only


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("base")
    ap.add_argument("new")
    ap.add_argument("--threshold", type=float, default=0.10,
                    help="allowed slowdown as a fraction (default 0.10)")
    args = ap.parse_args(argv)
    try:
        base, new = load_line(args.base), load_line(args.new)
    except (OSError, ValueError) as e:
        print(f"bench_regression: {e}", file=sys.stderr)
        return 2
    rows, regressed, only = compare(base, new, args.threshold)
    for name, b, n, r in rows:
        flag = "  SLOWER" if name in regressed else ""
        print(f"{name:60s} {b * 1e3:10.2f} us -> {n * 1e3:10.2f} us  x{r:.3f}{flag}")
    for name in only:
        print(f"{name:60s} (one side only; skipped)")
    if not rows:
        print("bench_regression: no timed quantity on both sides", file=sys.stderr)
        return 2
    if regressed:
        print(f"{len(regressed)} of {len(rows)} timed quantities more than "
              f"{args.threshold:.0%} slower", file=sys.stderr)
        return 1
    print(f"no regression beyond {args.threshold:.0%} ({len(rows)} quantities)")
    return 0


if __name__ == "__main__":
    sys.exit(main())
