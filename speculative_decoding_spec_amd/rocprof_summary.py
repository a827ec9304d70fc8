"""Short text summaries of rocprofv3 results (the rocpd SQLite output).

    python -m speculative_decoding_spec_amd.rocprof_summary trace DB [--match S ...]
        per kernel: calls, average / min / max duration (us), grid, workgroup
    python -m speculative_decoding_spec_amd.rocprof_summary counters DB [--match S ...]
        per kernel and counter: dispatches and average value per dispatch
    python -m speculative_decoding_spec_amd.rocprof_summary derived DB [--match S ...]
        per kernel, from SQ_WAVES, SQ_INSTS_VALU, SQ_INSTS_SALU, TCC_HIT_sum and
        TCC_MISS_sum: waves per dispatch, VALU and SALU instructions per wave,
        and the L2 hit rate of its requests
    python -m speculative_decoding_spec_amd.rocprof_summary traffic \
            --fetch DB --write DB --copy-fetch DB --copy-write DB \
            --copy-bytes N --match S --source FILE [--mix GRID_X:N ...]
        HBM bytes per launch of the matching kernels (optionally a weighted
        mix of launches told apart by grid size): FETCH_SIZE and
        WRITE_SIZE (KiB per dispatch) each scaled by the ratio of known bytes
        to what the same counter reads for a plain copy kernel of N bytes
        (read once, written once); FILE's sha256 records the kernel source
        the counters belong to.

Only reads the database; kernel names are shortened to their template id.
"""
from __future__ import annotations

import argparse
import re
import sqlite3
import sys


def short_name(name: str) -> str:
    """'void spec::(anonymous namespace)::qmv_kernel<4, 4, 2>(...)' -> 'qmv_kernel<4, 4, 2>'."""
    s = name
    depth, cut = 0, len(s)
    for i, ch in enumerate(s):          # drop the argument list
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and i > 0 and s[i - 1] not in ": ":
            cut = i
            break
    s = s[:cut]
    s = re.sub(r"^void ", "", s)
    s = s.split("::")[-1] if "<" not in s else s[s.rfind("::", 0, s.find("<")) + 2:]
    return s[:80]


def _matches(name: str, match) -> bool:
    return not match or any(m in name for m in match)


def trace_rows(db: str, match=None):
    con = sqlite3.connect(db)
    rows = con.execute(
        "select name, duration, grid_x, grid_y, workgroup_x from kernels").fetchall()
    agg: dict = {}
    for name, dur, gx, gy, wx in rows:
        if not _matches(name, match):
            continue
        key = (short_name(name), gx, gy, wx)
        agg.setdefault(key, []).append(dur / 1000.0)
    out = []
    for (n, gx, gy, wx), d in agg.items():
        out.append(dict(kernel=n, grid=f"{gx}x{gy}", wg=wx, calls=len(d),
                        avg_us=sum(d) / len(d), min_us=min(d), max_us=max(d),
                        total_us=sum(d)))
    out.sort(key=lambda r: -r["total_us"])
    return out


def counter_rows(db: str, match=None):
    con = sqlite3.connect(db)
    tables = {r[0] for r in con.execute("select name from sqlite_master")}
    table = "counters_collection" if "counters_collection" in tables else None
    if table is None:
        raise SystemExit("no counter collection in this database")
    cols = [r[1] for r in con.execute(f"pragma table_info({table})")]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    rows = con.execute(
        f"select {name_col}, counter_name, value, dispatch_id, grid_size_x, grid_size_y "
        f"from {table}" if "grid_size_x" in cols else
        f"select {name_col}, counter_name, value, dispatch_id, 0, 0 from {table}").fetchall()
    per: dict = {}
    for name, counter, value, disp, gx, gy in rows:
        if not _matches(name, match):
            continue
        key = (short_name(name), gx, gy, counter)
        per.setdefault(key, {}).setdefault(disp, 0.0)
        per[key][disp] += value      # sum over instances of one dispatch
    out = []
    for (n, gx, gy, c), d in per.items():
        vals = list(d.values())
        out.append(dict(kernel=n, grid=f"{gx}x{gy}", counter=c, dispatches=len(vals),
                        avg=sum(vals) / len(vals)))
    out.sort(key=lambda r: (r["kernel"], r["grid"], r["counter"]))
    return out


def _per_dispatch(db: str, counter: str, match, grid=None):
    """{dispatch_id: summed value} of one counter over the matching kernels
    (and, if given, the launches of total grid size `grid` in x)."""
    con = sqlite3.connect(db)
    cols = [r[1] for r in con.execute("pragma table_info(counters_collection)")]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    gx = "grid_size_x" if "grid_size_x" in cols else "0"
    d: dict = {}
    for name, c, v, disp, g in con.execute(
            f"select {name_col}, counter_name, value, dispatch_id, {gx} from counters_collection"):
        if c == counter and _matches(name, match) and (grid is None or g == grid):
            d[disp] = d.get(disp, 0.0) + v
    return d


def _mix_average(db: str, counter: str, match, mix):
    """Per-launch average of a counter over a launch mix: `mix` maps grid
    size to launches per step; each grid's dispatches are averaged first."""
    if not mix:
        vals = list(_per_dispatch(db, counter, match).values())
        return sum(vals) / len(vals), len(vals)
    total, count, seen = 0.0, 0, 0
    for grid, n in mix.items():
        vals = list(_per_dispatch(db, counter, match, grid).values())
        if not vals:
            raise SystemExit(f"no {counter} dispatches with grid {grid}")
        total += n * sum(vals) / len(vals)
        count += n
        seen += len(vals)
    return total / count, seen


def traffic(a) -> None:
    import hashlib
    cf = _per_dispatch(a.copy_fetch, "FETCH_SIZE", None)
    cw = _per_dispatch(a.copy_write, "WRITE_SIZE", None)
    # the copy is the dispatch that moved the most bytes
    copy_fetch_kib, copy_write_kib = max(cf.values()), max(cw.values())
    fetch_factor = a.copy_bytes / (copy_fetch_kib * 1024.0)
    write_factor = a.copy_bytes / (copy_write_kib * 1024.0)
    mix = {}
    for item in a.mix or []:
        g, n = item.split(":")
        mix[int(g)] = int(n)
    fk, nf = _mix_average(a.fetch, "FETCH_SIZE", a.match, mix)
    wk, nw = _mix_average(a.write, "WRITE_SIZE", a.match, mix)
    with open(a.source, "rb") as fh:
        sha = hashlib.sha256(fh.read()).hexdigest()
    print(f"kernel_match: {' '.join(a.match)}")
    print(f"source: {a.source}")
    print(f"source_sha256: {sha}")
    print(f"copy_bytes: {a.copy_bytes}")
    print(f"copy_fetch_kib: {copy_fetch_kib:.1f}")
    print(f"copy_write_kib: {copy_write_kib:.1f}")
    print(f"fetch_factor: {fetch_factor:.4f}")
    print(f"write_factor: {write_factor:.4f}")
    if mix:
        print("launch_mix: " + " ".join(f"{g}:{n}" for g, n in mix.items()))
    print(f"launches_fetch: {nf}")
    print(f"launches_write: {nw}")
    print(f"fetch_kib_per_launch: {fk:.1f}")
    print(f"write_kib_per_launch: {wk:.1f}")
    print(f"hbm_read_bytes_per_launch: {fk * 1024 * fetch_factor:.0f}")
    print(f"hbm_write_bytes_per_launch: {wk * 1024 * write_factor:.0f}")
    print(f"traffic_bytes_per_launch: {fk * 1024 * fetch_factor + wk * 1024 * write_factor:.0f}")


def derived(db: str, match=None):
    """Per kernel and grid: instructions per wave and L2 hit rate."""
    per: dict = {}
    for r in counter_rows(db, match):
        per.setdefault((r["kernel"], r["grid"]), {})[r["counter"]] = r["avg"]
    print(f"{'kernel':<44} {'grid':>14} {'waves':>8} {'VALU/wave':>10} {'SALU/wave':>10} "
          f"{'L2 hit %':>9}")
    for (k, g), c in sorted(per.items()):
        waves = c.get("SQ_WAVES", 0.0)
        hit, miss = c.get("TCC_HIT_sum"), c.get("TCC_MISS_sum")
        v = c.get("SQ_INSTS_VALU", 0.0) / waves if waves else float("nan")
        sa = c.get("SQ_INSTS_SALU", 0.0) / waves if waves else float("nan")
        h = 100.0 * hit / (hit + miss) if hit is not None and miss is not None and hit + miss else float("nan")
        print(f"{k:<44} {g:>14} {waves:>8.0f} {v:>10.1f} {sa:>10.1f} {h:>9.1f}")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["trace", "counters", "traffic", "derived"])
    ap.add_argument("db", nargs="?")
    ap.add_argument("--match", nargs="*")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-bytes", type=int)
    ap.add_argument("--source")
    ap.add_argument("--mix", nargs="*", help="GRID_X:LAUNCHES pairs weighting the per-grid averages")
    a = ap.parse_args(argv)
    if a.mode == "traffic":
        traffic(a)
    elif a.mode == "derived":
        derived(a.db, a.match)
    elif a.mode == "trace":
        print(f"{'kernel':<44} {'grid':>14} {'wg':>5} {'calls':>6} {'avg_us':>9} "
              f"{'min_us':>9} {'max_us':>9} {'total_us':>10}")
        for r in trace_rows(a.db, a.match):
            print(f"{r['kernel']:<44} {r['grid']:>14} {r['wg']:>5} {r['calls']:>6} "
                  f"{r['avg_us']:>9.2f} {r['min_us']:>9.2f} {r['max_us']:>9.2f} {r['total_us']:>10.1f}")
    else:
        print(f"{'kernel':<44} {'grid':>14} {'counter':<24} {'dispatches':>10} {'avg_per_dispatch':>18}")
        for r in counter_rows(a.db, a.match):
            print(f"{r['kernel']:<44} {r['grid']:>14} {r['counter']:<24} {r['dispatches']:>10} "
                  f"{r['avg']:>18.1f}")


if __name__ == "__main__":
    sys.exit(main())
