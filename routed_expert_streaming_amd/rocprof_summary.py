"""Summarise a rocprofv3 result database (rocpd SQLite) as plain text.

  python -m routed_expert_streaming_amd.rocprof_summary RESULTS.db [--by-grid | --counters | --timeline | --copies]

Prints one line per kernel: dispatches, average / min / max duration, share of
GPU time, grid, workgroup size and VGPRs (with --by-grid, one line per kernel
and grid size, which tells launches of one kernel on different shapes apart);
with --counters, the average of every
PMC counter per kernel (per kernel and grid size with --by-grid) (as collected by ``rocprofv3 --pmc ...``); with
--timeline, per kernel the average duration and the average idle gap between
the end of the previous dispatch and its start (over the last two thirds of the
trace, gaps under 20 us, so set-up and host pauses are left out); with --copies
(a trace taken with --memory-copy-trace), per copy direction the number of
copies, their average size, duration and rate, and over the last two thirds of
the trace the average idle gap between consecutive copies (gaps under 1 ms) and
the share of that span the copies were running; with --events N AT, N kernels
and copies in start order from the AT-th dispatch of the router partial kernel
counted from the end (1 = the last), times in microseconds from the first one.
"""
from __future__ import annotations

import argparse
import collections
import re
import sqlite3


def short_name(name: str) -> str:
    s = name.replace("(anonymous namespace)::", "")
    m = re.match(r"(?:void )?([\w:]+(?:<[^()]*>)?)", s)
    return (m.group(1) if m else s)[:90]


def kernel_stats(db: str, by_grid: bool = False):
    c = sqlite3.connect(db)
    rows = c.execute("select name, duration, grid_x, grid_y, grid_z, workgroup_x, vgpr_count, lds_size "
                     "from kernels").fetchall()
    agg = collections.defaultdict(list)
    meta = {}
    for name, dur, gx, gy, gz, wx, vgpr, lds in rows:
        k = short_name(name)
        if by_grid:
            k = f"{k[:70]} [{gx * gy * gz}]"
        agg[k].append(dur)
        meta[k] = (gx * gy * gz, wx, vgpr, lds)
    total = sum(sum(v) for v in agg.values()) or 1
    out = []
    for k, durs in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        g, w, v, l = meta[k]
        out.append((k, len(durs), sum(durs) / len(durs) / 1e3, min(durs) / 1e3, max(durs) / 1e3,
                    100.0 * sum(durs) / total, g, w, v, l))
    return out


def counter_stats(db: str, by_grid: bool = False):
    """Per kernel (and grid size, with by_grid): dispatch count and the average of
    every counter per dispatch."""
    c = sqlite3.connect(db)
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for name, grid, ctr, val in c.execute("select kernel_name, grid_size, counter_name, value "
                                          "from counters_collection"):
        k = short_name(name)
        agg[f"{k[:70]} [{grid}]" if by_grid else k][ctr].append(val)
    return {k: ({ctr: sum(v) / len(v) for ctr, v in d.items()}, max(len(v) for v in d.values()))
            for k, d in agg.items()}


def timeline_stats(db: str):
    c = sqlite3.connect(db)
    rows = c.execute("select name, start, end from kernels order by start").fetchall()
    dur = collections.defaultdict(list)
    gap = collections.defaultdict(list)
    prev_end = None
    for name, start, end in rows[len(rows) // 3:]:
        k = short_name(name)
        dur[k].append(end - start)
        if prev_end is not None and 0 <= start - prev_end < 20000:
            gap[k].append(start - prev_end)
        prev_end = end
    return [(k, len(d), sum(d) / len(d) / 1e3, (sum(gap[k]) / len(gap[k]) / 1e3) if gap[k] else 0.0)
            for k, d in dur.items()]


def copy_stats(db: str):
    c = sqlite3.connect(db)
    rows = c.execute("select src_agent_type, dst_agent_type, size, start, end from memory_copies "
                     "order by start").fetchall()
    by_dir = collections.defaultdict(list)
    for src, dst, size, start, end in rows:
        by_dir[f"{src}->{dst}"].append((start, end, size))
    out = []
    for d, cps in by_dir.items():
        tail = cps[len(cps) // 3:]
        gaps = [b[0] - a[1] for a, b in zip(tail, tail[1:]) if 0 <= b[0] - a[1] < 1_000_000]
        span = (tail[-1][1] - tail[0][0]) if tail else 0
        busy = sum(e - s0 for s0, e, _ in tail)
        n = len(cps)
        avg_size = sum(x[2] for x in cps) / n
        avg_dur = sum(x[1] - x[0] for x in cps) / n
        out.append((d, n, avg_size, avg_dur / 1e3, avg_size / avg_dur if avg_dur else 0.0,
                    (sum(gaps) / len(gaps) / 1e3) if gaps else 0.0, busy / span if span else 0.0))
    return out


def events(db: str, n: int, at: int, anchor: str = "router_partial_kernel"):
    c = sqlite3.connect(db)
    ev = [(s, e, "K " + short_name(name)[:60]) for name, s, e in c.execute("select name, start, end from kernels")]
    tabs = {r[0] for r in c.execute("select name from sqlite_master where type in ('table', 'view')")}
    if "memory_copies" in tabs:
        ev += [(s, e, f"C {size}") for s, e, size in c.execute("select start, end, size from memory_copies")]
    ev.sort()
    starts = [i for i, x in enumerate(ev) if anchor in x[2]]
    if not starts:
        return []
    i0 = starts[-min(at, len(starts))]
    t0 = ev[i0][0]
    return [((s - t0) / 1e3, (e - t0) / 1e3, (e - s) / 1e3, name) for s, e, name in ev[i0:i0 + n]]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--by-grid", action="store_true")
    ap.add_argument("--counters", action="store_true")
    ap.add_argument("--timeline", action="store_true")
    ap.add_argument("--copies", action="store_true")
    ap.add_argument("--events", nargs=2, type=int, metavar=("N", "AT"))
    args = ap.parse_args()
    if args.events:
        print(f"{'start_us':>9s} {'end_us':>9s} {'dur_us':>8s}  event")
        for s0, e, d, name in events(args.db, *args.events):
            print(f"{s0:9.2f} {e:9.2f} {d:8.2f}  {name}")
        return
    if args.copies:
        print(f"{'direction':14s} {'copies':>7s} {'avg_bytes':>11s} {'avg_us':>9s} {'GB/s':>7s} "
              f"{'gap_us':>8s} {'busy':>6s}")
        for d, n, sz, us, rate, gap, busy in copy_stats(args.db):
            print(f"{d:14s} {n:7d} {sz:11.0f} {us:9.2f} {rate:7.2f} {gap:8.2f} {busy:6.3f}")
        return
    if args.timeline:
        print(f"{'kernel':60s} {'calls':>6s} {'avg_us':>9s} {'gap_before_us':>14s}")
        for k, n, d, g in timeline_stats(args.db):
            print(f"{k[:60]:60s} {n:6d} {d:9.3f} {g:14.3f}")
        return
    if args.counters:
        for k, (d, n) in sorted(counter_stats(args.db, args.by_grid).items()):
            print(f"{k}  ({n} dispatches)")
            print("    " + "  ".join(f"{ctr}={v:.6g}" for ctr, v in sorted(d.items())))
        return
    print(f"{'kernel':90s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s} "
          f"{'threads':>8s} {'wg':>4s} {'vgpr':>4s} {'lds':>6s}")
    for k, n, avg, mn, mx, pct, g, w, v, l in kernel_stats(args.db, args.by_grid):
        print(f"{k:90s} {n:6d} {avg:9.3f} {mn:9.3f} {mx:9.3f} {pct:6.2f} {g:8d} {w:4d} {v:4d} {l:6d}")


if __name__ == "__main__":
    main()
