"""Summaries of rocprofv3 result databases (rocpd SQLite) as plain text.

  python -m moe_expert_layer_r3_amd.prof_summary trace  <results.db>
      per-kernel call count and average / min / max duration (ns)
  python -m moe_expert_layer_r3_amd.prof_summary counters <results.db> [scale]
      per-kernel average of each collected counter per dispatch (the rocprofv3
      FETCH_SIZE / WRITE_SIZE unit is KiB); `scale` multiplies the values (the
      calibration factor from a plain copy of known size)
  python -m moe_expert_layer_r3_amd.prof_summary split <results.db> <name-part> <n> [count]
      launches of the kernels whose name contains <name-part>, in dispatch
      order (the first `count` of them), grouped by position modulo n: for a
      kernel launched n times per step with different shapes (the two weight
      gradient products, say), the average duration of each launch of a step,
      and of each collected counter when the database holds counters
  python -m moe_expert_layer_r3_amd.prof_summary traffic <fetch.db> <write.db> <copy_fetch.db>
          <copy_write.db> <name-part> <n> <pos> <key> <workload> <sources> <out.json>
      HBM bytes per launch of one kernel (the launches at position <pos> modulo
      <n> among those whose name contains <name-part>): FETCH_SIZE and
      WRITE_SIZE per dispatch, each scaled so that a plain 1 GiB device copy
      (the copy databases) reads as 1 GiB; written as JSON with the sha256 of
      the kernel's sources (comma-separated names under csrc/), which bench.py
      checks before it reports the figure
  python -m moe_expert_layer_r3_amd.prof_summary derived <results.db> [<results.db> ...] -- <name-part> <n> <pos>
      per-launch averages of the counters collected over one or more runs (the
      launches at position <pos> modulo <n> among kernels named like
      <name-part>) and the figures derived from them: shader cycles per
      launch (GRBM_GUI_ACTIVE counts on each of the 8 XCDs), MFMA busy share of
      the SIMD cycles (SQ_VALU_MFMA_BUSY_CYCLES is 32 cycles per 16x16x128
      MFMA, over 1024 SIMDs), wait shares of the wave cycles, texture
      addresser busy share (256 TAs), L2 read latency, L1 -> L2 read bytes per
      clock and CU (128-byte requests), VALU instructions per MFMA, LDS bank
      conflict share"""

import json
import os
import re
import sqlite3
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def code_sha256(paths):
    """sha256 of the sources' code: comments and blank lines removed, each line
    stripped, so that a comment edit does not orphan a profile while any
    change to the code does."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        text = re.sub(r"/\*.*?\*/", "", open(p).read(), flags=re.S)
        for line in text.splitlines():
            line = re.sub(r"//.*", "", line).strip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()


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


def split(path, part, n, count=None):
    db = sqlite3.connect(path)
    tables = {r[0] for r in db.execute("select name from sqlite_master where type in ('table', 'view')")}
    if "kernels" in tables:
        rows = db.execute("select name, duration from kernels where name like ? order by start",
                          (f"%{part}%",)).fetchall()
        rows = rows[:count] if count else rows
        print(f"{'pos':>3} {'n':>3} {'avg_ns':>12}  kernel")
        for i in range(n):
            sel = rows[i::n]
            if sel:
                avg = sum(d for _, d in sel) / len(sel)
                print(f"{i:3d} {len(sel):3d} {avg:12.0f}  {sel[0][0][:100]}")
    if "counters_collection" in tables:
        rows = db.execute("select dispatch_id, counter_name, value, kernel_name from counters_collection "
                          "where kernel_name like ? order by dispatch_id", (f"%{part}%",)).fetchall()
        disp = {}
        for d, c, v, k in rows:
            e = disp.setdefault(d, {"kernel": k})
            e[c] = e.get(c, 0.0) + v
        ds = sorted(disp)
        ds = ds[:count] if count else ds
        print(f"{'pos':>3} {'n':>3} {'counter':14s} {'avg/dispatch':>14}  kernel")
        for i in range(n):
            sel = [disp[d] for d in ds[i::n]]
            if not sel:
                continue
            for c in sorted(k for k in sel[0] if k != "kernel"):
                avg = sum(e.get(c, 0.0) for e in sel) / len(sel)
                print(f"{i:3d} {len(sel):3d} {c:14s} {avg:14.1f}  {sel[0]['kernel'][:80]}")


def _per_dispatch(path, counter, part):
    db = sqlite3.connect(path)
    rows = db.execute("select dispatch_id, sum(value) from counters_collection where counter_name = ? and "
                      "kernel_name like ? group by dispatch_id order by dispatch_id",
                      (counter, f"%{part}%")).fetchall()
    return [v for _, v in rows]


def traffic(fetch_db, write_db, cfetch_db, cwrite_db, part, n, pos, key, workload, sources, out):
    gib_kib = float(1 << 20)  # 1 GiB in the counters' KiB
    cf = [v for v in _per_dispatch(cfetch_db, "FETCH_SIZE", "copyBuffer") if v > 0.25 * gib_kib]
    cw = [v for v in _per_dispatch(cwrite_db, "WRITE_SIZE", "copyBuffer") if v > 0.25 * gib_kib]
    if not cf or not cw:
        raise SystemExit("no 1 GiB copy dispatch in the calibration databases")
    fs, ws = gib_kib / (sum(cf) / len(cf)), gib_kib / (sum(cw) / len(cw))
    f = _per_dispatch(fetch_db, "FETCH_SIZE", part)[pos::n]
    w = _per_dispatch(write_db, "WRITE_SIZE", part)[pos::n]
    srcs = sources.split(",")
    rec = {
        "kernel": key,
        "workload": workload,
        "match": f"launches {pos} mod {n} of kernels named like '{part}'",
        "dispatches": [len(f), len(w)],
        "sources": srcs,
        "code_sha256": code_sha256([os.path.join(CSRC, x) for x in srcs]),
        "fetch_bytes_per_launch": sum(f) / len(f) * fs * 1024.0,
        "write_bytes_per_launch": sum(w) / len(w) * ws * 1024.0,
        "fetch_scale": fs,
        "write_scale": ws,
    }
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def derived(paths, part, n, pos):
    tot = {}
    for path in paths:
        db = sqlite3.connect(path)
        rows = db.execute("select dispatch_id, counter_name, sum(value) from counters_collection "
                          "where kernel_name like ? group by dispatch_id, counter_name order by dispatch_id",
                          (f"%{part}%",)).fetchall()
        disp = {}
        for d, c, v in rows:
            disp.setdefault(d, {})[c] = v
        ds = sorted(disp)[pos::n]
        for c in sorted({c for d in ds for c in disp[d]}):
            vals = [disp[d][c] for d in ds if c in disp[d]]
            tot.setdefault(c, []).extend(vals)
    a = {c: sum(v) / len(v) for c, v in tot.items()}
    for c in sorted(a):
        print(f"  {c:32s} {a[c]:16.1f}   ({len(tot[c])} launches)")
    g = a.get("GRBM_GUI_ACTIVE")
    if g:
        cyc = g / 8.0
        print(f"  shader cycles per launch           {cyc:16.0f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in a:
            print(f"  MFMA busy share of SIMD cycles     {a['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * cyc):16.3f}")
        if "TA_TA_BUSY_sum" in a:
            print(f"  texture addresser busy share       {a['TA_TA_BUSY_sum'] / (256 * cyc):16.3f}")
        if "TCP_TCC_READ_REQ_sum" in a:
            print(f"  L1 -> L2 read bytes / clock / CU   {a['TCP_TCC_READ_REQ_sum'] * 128 / 256 / cyc:16.1f}")
    if "SQ_WAVE_CYCLES" in a:
        for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS"):
            if c in a:
                print(f"  {c + ' / wave cycles':34s} {a[c] / a['SQ_WAVE_CYCLES']:16.3f}")
    if "TCP_TCC_READ_REQ_LATENCY_sum" in a and a.get("TCP_TCC_READ_REQ_sum"):
        print(f"  L2 read latency (cycles)           {a['TCP_TCC_READ_REQ_LATENCY_sum'] / a['TCP_TCC_READ_REQ_sum']:16.0f}")
    if "TCP_TCC_WRITE_REQ_LATENCY_sum" in a and a.get("TCP_TCC_WRITE_REQ_sum"):
        print(f"  L2 write latency (cycles)          {a['TCP_TCC_WRITE_REQ_LATENCY_sum'] / a['TCP_TCC_WRITE_REQ_sum']:16.0f}")
    if a.get("SQ_INSTS_MFMA"):
        print(f"  VALU instructions per MFMA         {a.get('SQ_INSTS_VALU', 0) / a['SQ_INSTS_MFMA']:16.2f}")
    if a.get("SQ_LDS_IDX_ACTIVE"):
        print(f"  LDS bank conflict share            {a.get('SQ_LDS_BANK_CONFLICT', 0) / a['SQ_LDS_IDX_ACTIVE']:16.3f}")


if __name__ == "__main__":
    mode, path = sys.argv[1], sys.argv[2]
    if mode == "derived":
        k = sys.argv.index("--")
        derived(sys.argv[2:k], sys.argv[k + 1], int(sys.argv[k + 2]), int(sys.argv[k + 3]))
    elif mode == "traffic":
        a = sys.argv[2:]
        traffic(a[0], a[1], a[2], a[3], a[4], int(a[5]), int(a[6]), a[7], a[8], a[9], a[10])
    elif mode == "trace":
        trace(path)
    elif mode == "split":
        split(path, sys.argv[3], int(sys.argv[4]), int(sys.argv[5]) if len(sys.argv) > 5 else None)
    else:
        counters(path, float(sys.argv[3]) if len(sys.argv) > 3 else 1.0)
