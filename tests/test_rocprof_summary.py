"""The rocprofv3 summary tool on a small hand-made result database (host only)."""
import sqlite3

import pytest

from routed_expert_streaming_amd import rocprof_summary as R


@pytest.fixture
def db(tmp_path):
    path = str(tmp_path / "run_results.db")
    c = sqlite3.connect(path)
    c.execute("create table kernels(name, start, end)")
    c.execute("create table memory_copies(start, end, size)")
    for step in range(2):
        t = step * 30_000_000
        # two routers, then copies on two streams with one 400 us hole after the 3rd pair
        c.execute("insert into kernels values(?,?,?)", ("void router_mfma_kernel(int)", t, t + 1000))
        c.execute("insert into kernels values(?,?,?)", ("void router_mfma_kernel(int)", t + 1000, t + 2000))
        at = t + 10_000
        for i in range(6):
            c.execute("insert into memory_copies values(?,?,?)", (at, at + 100_000, 2_000_000))
            c.execute("insert into memory_copies values(?,?,?)", (at + 50_000, at + 150_000, 2_000_000))
            at += 150_000 + (400_000 if i == 2 else 0)
        c.execute("insert into kernels values(?,?,?)", ("void ffn_kernel<2>(int)", t + 500_000, t + 600_000))  # in the hole
        c.execute("insert into kernels values(?,?,?)", ("void ffn_kernel<1>(int)", at - 200_000, at + 30_000))
        c.execute("insert into memory_copies values(?,?,?)", (t + 5000, t + 6000, 4096))  # small: not a slab copy
    c.commit()
    return path


def test_copy_gaps_merges_both_streams_and_splits_steps(db):
    rows, gaps = R.copy_gaps(db, "router_mfma")
    assert len(rows) == 2
    for i, span, n, gb, busy, rate, head, tail, ngaps, gap_ms, one, two in rows:
        assert n == 12 and gb == pytest.approx(0.024)
        # 6 pairs of 150 us busy each, the 400 us hole splits them into two runs
        assert busy == pytest.approx(0.9) and ngaps == 1 and gap_ms == pytest.approx(0.4)
        assert head == pytest.approx(0.01) and tail == pytest.approx(0.03)
        # each pair: 50 us one copy, 50 us two, 50 us one
        assert one == pytest.approx(0.6) and two == pytest.approx(0.3)
        assert rate == pytest.approx(24e6 / 0.9e6)
    assert len(gaps) == 1 and gaps[0][1] == pytest.approx(400.0) and gaps[0][2] == ["ffn_kernel<2>"]
