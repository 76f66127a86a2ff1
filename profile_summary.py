"""Summaries of rocprofv3 result databases (kernel trace and PMC counter runs).

python profile_summary.py trace DB [--kernel NAME]
python profile_summary.py traffic FETCH_DB WRITE_DB --calib-bytes N
    [--kernel NAME] [--out JSON] [--workload W] [--kernel-sha SHA]
python profile_summary.py mfma DB --trace TRACE_DB [--kernel NAME]

`trace` prints per-kernel call counts and durations. `traffic` scales the
FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) of one kernel by the
ratio the same counters read for a plain device copy of known size, giving
HBM bytes per launch. `mfma` reads SQ_VALU_MFMA_BUSY_CYCLES,
SQ_INSTS_VALU_MFMA_MOPS_BF16 / _F32 and GRBM_GUI_ACTIVE per dispatch of one
kernel: matrix-core busy fraction (busy cycles over active cycles times the
1024 SIMDs; the stored GRBM_GUI_ACTIVE is the sum over the 8 XCDs, so one XCD's
active cycles are a eighth of it) and MFMA flops (512 per counted op), priced
against the kernel's mean duration from a kernel-trace database.
"""
from __future__ import annotations

import argparse
import json
import sqlite3
import statistics
import sys


def _con(path):
    return sqlite3.connect(path)


def kernel_stats(db: str):
    con = _con(db)
    rows = con.execute("select name, total_calls, total_duration, average, percentage from top_kernels").fetchall()
    out = []
    for name, calls, total, avg, pct in rows:
        durs = [r[0] for r in con.execute("select duration from kernels where name = ?", (name,))]
        out.append({"name": name, "calls": calls, "total_us": total / 1e3 if total > 1e6 else total,
                    "avg_ns": None if not durs else statistics.mean(durs),
                    "min_ns": None if not durs else min(durs),
                    "max_ns": None if not durs else max(durs), "pct": pct})
    return out


def counters(db: str, counter: str):
    con = _con(db)
    return con.execute("select dispatch_id, kernel_name, grid_size, value, duration from counters_collection "
                       "where counter_name = ? order by dispatch_id", (counter,)).fetchall()


def _is_copy(name: str) -> bool:
    # the runtime's device copy and the probe library's copy kernel; not torch's dtype
    # conversions, whose names also hold "copy_kernel" and which read other byte counts
    return "copyBuffer" in name or "bw_copy_kernel" in name


def traffic(fetch_db: str, write_db: str, calib_bytes: int, kernel: str = "kda_fwd_kernel"):
    f = counters(fetch_db, "FETCH_SIZE")
    w = counters(write_db, "WRITE_SIZE")
    kf = [v for _, n, _, v, _ in f if kernel in n]
    kw = [v for _, n, _, v, _ in w if kernel in n]
    # the calibration copies are the largest copy dispatches
    cf = sorted([v for _, n, g, v, _ in f if _is_copy(n)])[-3:]
    cw = sorted([v for _, n, g, v, _ in w if _is_copy(n)])[-3:]
    if not kf or not kw or not cf or not cw:
        raise SystemExit("missing kernel or calibration dispatches in the counter databases")
    calib_kib = calib_bytes / 1024.0
    f_scale = calib_kib / statistics.mean(cf)          # true bytes read per counted KiB
    w_scale = calib_kib / statistics.mean(cw)
    fetch = statistics.mean(kf) * 1024 * f_scale
    write = statistics.mean(kw) * 1024 * w_scale
    return {"fetch_kib_per_dispatch": statistics.mean(kf), "write_kib_per_dispatch": statistics.mean(kw),
            "copy_fetch_kib": statistics.mean(cf), "copy_write_kib": statistics.mean(cw),
            "copy_bytes": calib_bytes, "fetch_scale": f_scale, "write_scale": w_scale,
            "fetch_bytes": fetch, "write_bytes": write, "bytes_per_launch": fetch + write,
            "dispatches": len(kf)}


SIMD_NUM = 1024     # 256 CUs x 4 SIMDs
XCD_NUM = 8


def mfma(db: str, trace_db: str, kernel: str):
    def per_dispatch(name):
        vals = [v for _, n, _, v, _ in counters(db, name) if kernel in n]
        return statistics.mean(vals) if vals else None
    busy = per_dispatch("SQ_VALU_MFMA_BUSY_CYCLES")
    gui = per_dispatch("GRBM_GUI_ACTIVE")
    bf16 = per_dispatch("SQ_INSTS_VALU_MFMA_MOPS_BF16") or 0.0
    f32 = per_dispatch("SQ_INSTS_VALU_MFMA_MOPS_F32") or 0.0
    durs = [k for k in kernel_stats(trace_db) if kernel in k["name"]]
    avg_ns = durs[0]["avg_ns"] if durs else None
    rec = {"kernel": kernel, "mfma_busy_cycles": busy, "gui_active_cycles": gui,
           "mfma_busy_frac": (busy / (gui / XCD_NUM * SIMD_NUM)) if busy and gui else None,
           "bf16_flops": bf16 * 512, "f32_flops": f32 * 512, "avg_ns": avg_ns}
    if avg_ns:
        rec["bf16_tflops"] = bf16 * 512 / (avg_ns * 1e-9) / 1e12
        rec["f32_tflops"] = f32 * 512 / (avg_ns * 1e-9) / 1e12
    return rec


def counter_means(db: str, kernel: str):
    """Mean per dispatch of every counter collected in `db`, over the dispatches of `kernel`."""
    con = _con(db)
    names = [r[0] for r in con.execute("select distinct counter_name from counters_collection")]
    out = {}
    for name in names:
        vals = [v for _, n, _, v, _ in counters(db, name) if kernel in n]
        if vals:
            out[name] = statistics.mean(vals)
    out["dispatches"] = max((len([1 for _, n, _, _, _ in counters(db, nm) if kernel in n]) for nm in names),
                            default=0)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    c = sub.add_parser("traffic")
    c.add_argument("fetch_db")
    c.add_argument("write_db")
    c.add_argument("--calib-bytes", type=int, required=True)
    c.add_argument("--kernel", default="kda_fwd_kernel")
    c.add_argument("--out")
    c.add_argument("--workload", default="")
    c.add_argument("--kernel-sha", default="")
    m = sub.add_parser("mfma")
    m.add_argument("db")
    m.add_argument("--trace", required=True)
    m.add_argument("--kernel", default="kda_wy_chain_kernel")
    k = sub.add_parser("counters")
    k.add_argument("db")
    k.add_argument("--kernel", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        print(json.dumps({"kernel": a.kernel, **counter_means(a.db, a.kernel)}, indent=1))
        return 0
    if a.cmd == "mfma":
        print(json.dumps(mfma(a.db, a.trace, a.kernel), indent=1))
        return 0
    if a.cmd == "trace":
        for k in kernel_stats(a.db):
            print(f"{k['calls']:6d} calls  avg {k['avg_ns'] / 1e3:10.2f} us  min {k['min_ns'] / 1e3:10.2f} us  "
                  f"max {k['max_ns'] / 1e3:10.2f} us  {k['pct']:6.2f}%  {k['name'][:110]}")
    else:
        rec = traffic(a.fetch_db, a.write_db, a.calib_bytes, a.kernel)
        rec.update({"workload": a.workload, "kernel_sha": a.kernel_sha})
        txt = json.dumps(rec, indent=1)
        print(txt)
        if a.out:
            open(a.out, "w").write(txt + "\n")


if __name__ == "__main__":
    sys.exit(main())
