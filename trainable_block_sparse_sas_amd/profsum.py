"""Summaries of rocprofv3 result databases for the text files under profiles/.

  python -m trainable_block_sparse_sas_amd.profsum stats DB --cmd "..." [--by-grid]
      kernel-trace table: launches, average and total duration per kernel
      (per kernel and launch shape with --by-grid).
  python -m trainable_block_sparse_sas_amd.profsum traffic-by-grid --fetch DB --write DB
         --match decode_mfma topk_runs ... --cmd-fetch "..." --cmd-write "..."
      HBM bytes per dispatch for every matching kernel and launch shape.
  python -m trainable_block_sparse_sas_amd.profsum traffic --fetch DB --write DB
         --kernel bwd_dkdv --workload train-32k-sparse --cmd-fetch "..." --cmd-write "..."
      HBM bytes per launch of one kernel from a FETCH_SIZE run and a WRITE_SIZE
      run, each scaled by what the same counter reads for a plain copy kernel
      that reads and writes 1 GiB (bench.py --copy-probe).

  python -m trainable_block_sparse_sas_amd.profsum counters DB --cmd "..." --match fwd_sel bwd_dkdv ...
      per-kernel counter totals per dispatch (summed over counter instances)
      with the kernel's duration; SQ_INSTS_MFMA gives the executed matrix
      work (each v_mfma_f32_16x16x32_bf16 is 16384 flops).

Reads only the SQLite views rocprofv3 writes (kernels, pmc_events).
"""
from __future__ import annotations

import argparse
import hashlib
import os
import re
import sqlite3

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30
KERNEL_SOURCES = {"fwd_sel": "attn_fwd_sel.hip", "fwd_mfma": "attn_fwd_mfma.hip",
                  "bwd_dq": "attn_bwd_mfma.hip", "bwd_dkdv": "attn_bwd_mfma.hip"}


def short_name(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", n).strip()


def _grid(cols, r):
    """Workgroups of a dispatch as 'x,y,z' (grid sizes are in work-items)."""
    if "grid_x" not in cols:
        return ""
    gx, gy, gz = (r[cols.index(c)] for c in ("grid_x", "grid_y", "grid_z"))
    wx = r[cols.index("workgroup_x")] if "workgroup_x" in cols else 1
    return f"{gx // max(wx, 1)},{gy},{gz}"


def kernel_rows(db, by_grid=False):
    con = sqlite3.connect(db)
    cols = [r[1] for r in con.execute("pragma table_info(kernels)")]
    ni = cols.index("name") if "name" in cols else cols.index("kernel_name")
    si, ei = cols.index("start"), cols.index("end")
    for r in con.execute("select * from kernels order by start"):
        n = short_name(r[ni])
        if by_grid:
            n = f"{n} [{_grid(cols, r)}]"
        yield n, (r[ei] - r[si]) / 1e3  # us


def stats(db, cmd, by_grid=False):
    """Per kernel: launches, average, average without the kernel's first
    launch (which runs cold: the command's warm-up), total and share."""
    agg = {}
    for n, us in kernel_rows(db, by_grid):
        a = agg.setdefault(n, [0, 0.0, None])
        a[0] += 1
        a[1] += us
        if a[2] is None:
            a[2] = us
    tot = sum(v[1] for v in agg.values())
    out = ["# Kernel trace summary", "", "Command:", "", "```", cmd, "```", "",
           "| kernel | launches | avg us | avg us after the first launch | total ms | share |",
           "|---|---:|---:|---:|---:|---:|"]
    for n, (c, t, first) in sorted(agg.items(), key=lambda x: -x[1][1]):
        if t / tot < 1e-4:
            continue
        warm = f"{(t - first) / (c - 1):.1f}" if c > 1 else "-"
        out.append(f"| `{n[:120]}` | {c} | {t / c:.1f} | {warm} | {t / 1e3:.3f} | {100 * t / tot:.1f}% |")
    return "\n".join(out) + "\n"


def counter_per_dispatch(db, counter):
    """{kernel short name: mean counter value per dispatch}."""
    con = sqlite3.connect(db)
    per = {}
    for name, disp, cn, cv in con.execute(
            "select name, dispatch_id, counter_name, counter_value from pmc_events"):
        if cn != counter:
            continue
        d = per.setdefault(short_name(name), {})
        d[disp] = d.get(disp, 0.0) + cv
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def source_hash(kernel):
    csrc = os.path.join(HERE, "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "common.h", "mfma.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _pick(vals, key):
    hits = [k for k in vals if key in k]
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {key!r}, found {hits}")
    return hits[0], vals[hits[0]]


def traffic(fetch_db, write_db, kernel, workload, cmd_fetch, cmd_write):
    f = counter_per_dispatch(fetch_db, "FETCH_SIZE")
    w = counter_per_dispatch(write_db, "WRITE_SIZE")
    kname, kf = _pick(f, kernel + "_kernel<")
    _, kw = _pick(w, kernel + "_kernel<")
    cname, cf = _pick(f, "bitwise_not")
    _, cw = _pick(w, "bitwise_not")
    sf = COPY_BYTES / (cf * 1024.0)
    sw = COPY_BYTES / (cw * 1024.0)
    total = int(kf * 1024.0 * sf + kw * 1024.0 * sw)
    lines = [
        f"# HBM traffic of `{kernel}` on {workload}", "",
        "FETCH_SIZE and WRITE_SIZE (KiB per dispatch, rocprofv3 --pmc, one counter per run), each",
        "scaled by the same counter's reading for a plain copy kernel that reads and writes",
        "1 GiB (torch bitwise_not over 2^28 int32, run first by bench.py --copy-probe).", "",
        "Commands:", "", "```", cmd_fetch, cmd_write, "```", "",
        f"- kernel: `{kname}`",
        f"- fetch_kib_per_dispatch: {kf:.1f}",
        f"- write_kib_per_dispatch: {kw:.1f}",
        f"- copy_kernel: `{cname[:80]}`",
        f"- copy_fetch_kib: {cf:.1f}",
        f"- copy_write_kib: {cw:.1f}",
        f"- fetch_scale: {sf:.4f}",
        f"- write_scale: {sw:.4f}",
        f"- hbm_bytes_per_launch: {total}",
        f"- source_sha256_16: `{source_hash(kernel)}`",
    ]
    return "\n".join(lines) + "\n"


def counters(db, cmd, match):
    con = sqlite3.connect(db)
    per = {}  # kernel -> dispatch -> {counter: total}, durations
    durs = {}
    for name, disp, dur, cn, cv in con.execute(
            "select name, dispatch_id, duration, counter_name, counter_value from pmc_events"):
        n = short_name(name)
        if not any(m + "_kernel<" in n or n.endswith(m + "_kernel") for m in match):
            continue
        d = per.setdefault(n, {}).setdefault(disp, {})
        d[cn] = d.get(cn, 0.0) + cv
        durs.setdefault(n, {})[disp] = dur / 1e3  # us
    names = sorted({c for k in per.values() for d in k.values() for c in d})
    out = ["# Counter summary", "", "Command:", "", "```", cmd, "```", "",
           "Per dispatch, summed over counter instances, averaged over dispatches. Duration is",
           "the profiled dispatch (counters slow kernels down; use the kernel trace for time).", "",
           "| kernel | dispatches | duration us | " + " | ".join(names) + " | MFMA TFLOP/s executed | VALU per MFMA |",
           "|---|---:|---:|" + "---:|" * len(names) + "---:|---:|"]
    for k in sorted(per):
        disp = per[k]
        avg = {c: sum(d.get(c, 0.0) for d in disp.values()) / len(disp) for c in names}
        dur = sum(durs[k].values()) / len(durs[k])
        mf = avg.get("SQ_INSTS_MFMA", 0.0)
        va = avg.get("SQ_INSTS_VALU", 0.0)
        tf = mf * 16384 / (dur * 1e-6) / 1e12 if dur else 0.0
        vpm = f"{va / mf:.2f}" if mf else "-"
        out.append(f"| `{k[:70]}` | {len(disp)} | {dur:.1f} | " + " | ".join(f"{avg[c]:.4g}" for c in names)
                   + f" | {tf:.1f} | {vpm} |")
    return "\n".join(out) + "\n"


def counter_by_grid(db, counter):
    """{(kernel short name, workgroups): mean counter value per dispatch}."""
    con = sqlite3.connect(db)
    cols = [r[1] for r in con.execute("pragma table_info(pmc_events)")]
    per = {}
    for r in con.execute("select * from pmc_events"):
        if r[cols.index("counter_name")] != counter:
            continue
        key = (short_name(r[cols.index("name")]), _grid(cols, r))
        d = per.setdefault(key, {})
        disp = r[cols.index("dispatch_id")]
        d[disp] = d.get(disp, 0.0) + r[cols.index("counter_value")]
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def traffic_by_grid(fetch_db, write_db, match, cmd_fetch, cmd_write):
    """HBM bytes per dispatch of every kernel matching one of `match`, per
    launch shape (workgroups), scaled by the copy kernel's readings."""
    f = counter_by_grid(fetch_db, "FETCH_SIZE")
    w = counter_by_grid(write_db, "WRITE_SIZE")
    cf = [v for (n, _), v in f.items() if "bitwise_not" in n]
    cw = [v for (n, _), v in w.items() if "bitwise_not" in n]
    if len(cf) != 1 or len(cw) != 1:
        raise SystemExit("expected one copy-probe dispatch in each database")
    sf = COPY_BYTES / (cf[0] * 1024.0)
    sw = COPY_BYTES / (cw[0] * 1024.0)
    lines = ["# HBM traffic per dispatch, by kernel and launch shape", "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch, one counter per run), each scaled by",
             "the same counter's reading for a plain copy kernel that reads and writes 1 GiB",
             "(bench.py --copy-probe).", "", "Commands:", "", "```", cmd_fetch, cmd_write, "```", "",
             f"fetch scale {sf:.4f}, write scale {sw:.4f}", "",
             "| kernel | workgroups | read bytes | written bytes | total bytes |", "|---|---|---:|---:|---:|"]
    for (n, g) in sorted(f):
        if not any(m in n for m in match) or (n, g) not in w:
            continue
        rb = f[(n, g)] * 1024.0 * sf
        wb = w[(n, g)] * 1024.0 * sw
        lines.append(f"| `{n[:70]}` | {g} | {rb:.4g} | {wb:.4g} | {rb + wb:.4g} |")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("db")
    a.add_argument("--cmd", required=True)
    a.add_argument("--by-grid", action="store_true", help="one row per kernel and launch shape")
    t = sub.add_parser("traffic-by-grid")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--match", nargs="+", required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--cmd-fetch", required=True)
    b.add_argument("--cmd-write", required=True)
    cn = sub.add_parser("counters")
    cn.add_argument("db")
    cn.add_argument("--cmd", required=True)
    cn.add_argument("--match", nargs="+", required=True)
    args = ap.parse_args()
    if args.what == "counters":
        print(counters(args.db, args.cmd, args.match), end="")
        return
    if args.what == "traffic-by-grid":
        print(traffic_by_grid(args.fetch, args.write, args.match, args.cmd_fetch, args.cmd_write), end="")
        return
    if args.what == "stats":
        print(stats(args.db, args.cmd, args.by_grid), end="")
    else:
        print(traffic(args.fetch, args.write, args.kernel, args.workload, args.cmd_fetch,
                      args.cmd_write), end="")


if __name__ == "__main__":
    main()
