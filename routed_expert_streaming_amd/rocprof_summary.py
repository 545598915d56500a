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
counted from the end (1 = the last), times in microseconds from the first one;
with --copy-gaps ANCHOR (a trace taken with --memory-copy-trace), per step
(a step starts at a dispatch of the kernel named ANCHOR that follows more than
5 ms without one) the H2D slab copies (over 1 MB) of both copy streams merged
into busy intervals: the step's span, bytes, busy time and rate over it, the
head (step start to first copy), the tail (last copy to the step's last kernel
end), the idle gaps between busy intervals, and the time with one and with two
copies in flight; then the gaps over 100 us of the last step with the kernels
that ran in them.
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


def copy_gaps(db: str, anchor: str):
    c = sqlite3.connect(db)
    ks = sorted((s, e, short_name(n)) for n, s, e in c.execute("select name, start, end from kernels"))
    cps = sorted((s, e, z) for s, e, z in c.execute("select start, end, size from memory_copies where size > 1000000"))
    marks = [s for s, e, n in ks if n.startswith(anchor)]
    if not marks:
        return [], []
    starts = [marks[0]] + [b for a, b in zip(marks, marks[1:]) if b - a > 5_000_000]
    end_all = max(e for s, e, n in ks)
    rows, last_gaps = [], []
    for i, t0 in enumerate(starts):
        t1 = starts[i + 1] if i + 1 < len(starts) else end_all + 1
        cp = [x for x in cps if t0 <= x[0] < t1]
        kk = [x for x in ks if t0 <= x[0] < t1]
        if not cp or not kk:
            continue
        merged = []
        for s, e, _ in cp:
            if merged and s <= merged[-1][1]:
                merged[-1][1] = max(merged[-1][1], e)
            else:
                merged.append([s, e])
        busy = sum(e - s for s, e in merged)
        gaps = [(a[1], b[0]) for a, b in zip(merged, merged[1:])]
        kend = max(e for s, e, n in kk)
        level, last, in_flight = 0, cp[0][0], collections.Counter()
        for t, d in sorted([(s, 1) for s, e, z in cp] + [(e, -1) for s, e, z in cp]):
            in_flight[min(level, 2)] += t - last
            level += d
            last = t
        nbytes = sum(z for s, e, z in cp)
        rows.append((i, (kend - t0) / 1e6, len(cp), nbytes / 1e9, busy / 1e6, nbytes / busy, (merged[0][0] - t0) / 1e6,
                     (kend - merged[-1][1]) / 1e6, len(gaps), sum(b - a for a, b in gaps) / 1e6, in_flight[1] / 1e6,
                     in_flight[2] / 1e6))
        last_gaps = [((a - t0) / 1e3, (b - a) / 1e3, [n for s, e, n in kk if s < b and e > a])
                     for a, b in gaps if b - a > 100_000]
    return rows, last_gaps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db")
    ap.add_argument("--by-grid", action="store_true")
    ap.add_argument("--counters", action="store_true")
    ap.add_argument("--timeline", action="store_true")
    ap.add_argument("--copies", action="store_true")
    ap.add_argument("--events", nargs=2, type=int, metavar=("N", "AT"))
    ap.add_argument("--copy-gaps", metavar="ANCHOR")
    args = ap.parse_args()
    if args.copy_gaps:
        rows, gaps = copy_gaps(args.db, args.copy_gaps)
        print(f"{'step':>4s} {'span_ms':>9s} {'copies':>6s} {'GB':>6s} {'busy_ms':>9s} {'GB/s':>6s} {'head_ms':>8s} "
              f"{'tail_ms':>8s} {'gaps':>5s} {'gap_ms':>7s} {'one_ms':>7s} {'two_ms':>8s}")
        for r in rows:
            print(f"{r[0]:4d} {r[1]:9.2f} {r[2]:6d} {r[3]:6.2f} {r[4]:9.2f} {r[5]:6.2f} {r[6]:8.3f} {r[7]:8.3f} "
                  f"{r[8]:5d} {r[9]:7.3f} {r[10]:7.2f} {r[11]:8.2f}")
        print("gaps over 100 us in the last step (start us after its first anchor, length us, kernels in the gap):")
        for at, length, names in gaps:
            print(f"  {at:10.1f} {length:8.1f}  {' | '.join(n[:32] for n in names[:6])}")
        return
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
