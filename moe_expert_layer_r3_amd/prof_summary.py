"""Summaries of rocprofv3 result databases (rocpd SQLite) as plain text.

  python -m moe_expert_layer_r3_amd.prof_summary trace  <results.db>
      per-kernel call count and average / min / max duration (ns)
  python -m moe_expert_layer_r3_amd.prof_summary counters <results.db> [scale]
      per-kernel average of each collected counter per dispatch (the rocprofv3
      FETCH_SIZE / WRITE_SIZE unit is KiB); `scale` multiplies the values (the
      calibration factor from a plain copy of known size)."""

import sqlite3
import sys


def trace(path):
    db = sqlite3.connect(path)
    rows = db.execute(
        "select name, count(*), avg(duration), min(duration), max(duration) from kernels "
        "group by name order by sum(duration) desc").fetchall()
    print(f"{'calls':>5} {'avg_ns':>12} {'min_ns':>10} {'max_ns':>10}  kernel")
    for name, n, a, mn, mx in rows:
        print(f"{n:5d} {a:12.0f} {mn:10.0f} {mx:10.0f}  {name}")


def counters(path, scale=1.0):
    db = sqlite3.connect(path)
    rows = db.execute(
        "select kernel_name, counter_name, count(*), avg(value) from counters_collection "
        "group by kernel_name, counter_name order by avg(value) desc").fetchall()
    print(f"{'counter':12s} {'n':>3} {'avg/dispatch':>14} {'x scale':>14}  kernel")
    for name, ctr, n, a in rows:
        print(f"{ctr:12s} {n:3d} {a:14.1f} {a * scale:14.1f}  {name}")


if __name__ == "__main__":
    mode, path = sys.argv[1], sys.argv[2]
    if mode == "trace":
        trace(path)
    else:
        counters(path, float(sys.argv[3]) if len(sys.argv) > 3 else 1.0)
