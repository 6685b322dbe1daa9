"""Summaries of rocprofv3 output for the profiles/ directory.

    python -m bit_moe_expert_02_amd.profile_summary trace DB OUT.md --title T --command C
        per-kernel durations from a --kernel-trace database
    python -m bit_moe_expert_02_amd.profile_summary traffic FETCH_DB WRITE_DB OUT.json \\
        --kernel NAME --calib-mib M --command-fetch C1 --command-write C2
        HBM bytes per launch of NAME from two --pmc runs (FETCH_SIZE, then WRITE_SIZE),
        each scaled by what the same counter reads for a device copy of M MiB
        (the run's largest copy dispatch); records a hash of the kernel sources so
        a reader can tell whether the numbers still describe the code.
    python -m bit_moe_expert_02_amd.profile_summary counters DB OUT.md --kernel NAME --title T --command C
        per-dispatch medians of every counter of a --pmc run for dispatches of NAME

Reads the rocpd SQLite views that rocprofv3 writes (kernels, counters_collection).
"""

import argparse
import hashlib
import json
import os
import sqlite3
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")


def source_hash():
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _counter_rows(db):
    c = sqlite3.connect(db)
    return c.execute("select dispatch_id, kernel_name, value from counters_collection").fetchall()


def traffic(fetch_db, write_db, kernel, calib_mib):
    """(fetch_bytes, write_bytes, fetch_factor, write_factor, launches) per launch of `kernel`."""
    calib = calib_mib << 20
    out = []
    for db in (fetch_db, write_db):
        rows = _counter_rows(db)
        copies = [v for _, k, v in rows if "copyBuffer" in k]
        ref_kb = max(copies)          # the calibration copy is the run's largest copy
        vals = [v for _, k, v in rows if k.split("(")[0].endswith(kernel) or kernel in k.split("(")[0]]
        if not vals:
            raise SystemExit(f"no dispatch of {kernel} in {db}")
        out.append((statistics.median(vals), ref_kb, len(vals)))
    (f_kb, f_ref, n), (w_kb, w_ref, _) = out
    return dict(fetch_kb_per_launch=f_kb, write_kb_per_launch=w_kb, launches=n,
                calib_copy_mib=calib_mib, fetch_factor=calib / 1024 / f_ref,
                write_factor=calib / 1024 / w_ref)


def counters_md(db, kernel, title, command):
    """Median over the dispatches of `kernel` of each counter in a --pmc run,
    with the wave-cycle shares the SQ counters give."""
    c = sqlite3.connect(db)
    cols = [r[1] for r in c.execute("pragma table_info(counters_collection)").fetchall()]
    name_col = "counter_name" if "counter_name" in cols else "name"
    rows = c.execute(f"select dispatch_id, kernel_name, {name_col}, value from counters_collection").fetchall()
    per = {}
    for _, k, n, v in rows:
        if kernel in k.split("(")[0]:
            per.setdefault(n, []).append(v)
    if not per:
        raise SystemExit(f"no dispatch of {kernel} in {db}")
    med = {n: statistics.median(v) for n, v in per.items()}
    lines = [f"# {title}", "", "Command (repository root on the MI355X):", "", "```", command, "```", "",
             f"Per-dispatch medians over {max(len(v) for v in per.values())} dispatches of `{kernel}`.", "",
             "| counter | median per dispatch |", "|---|---|"]
    for n in sorted(med):
        lines.append(f"| `{n}` | {med[n]:.6g} |")
    wc = med.get("SQ_WAVE_CYCLES")
    if wc:
        lines += ["", "| share of wave cycles | |", "|---|---|"]
        for n, what in (("SQ_WAIT_ANY", "waiting (memory, dependencies, barriers)"),
                        ("SQ_WAIT_INST_ANY", "waiting to issue"),
                        ("SQ_ACTIVE_INST_ANY", "issuing"),
                        ("SQ_ACTIVE_INST_VALU", "issuing VALU"),
                        ("SQ_ACTIVE_INST_LDS", "issuing LDS")):
            if n in med:
                lines.append(f"| {what} (`{n}`) | {100 * med[n] / wc:.1f} % |")
    return "\n".join(lines) + "\n"


def trace_md(db, title, command):
    c = sqlite3.connect(db)
    rows = c.execute("select name, count(*), avg(end-start), min(end-start), max(end-start), "
                     "sum(end-start) from kernels group by name order by sum(end-start) desc").fetchall()
    tot = sum(r[5] for r in rows)
    lines = [f"# {title}", "", "Command (repository root on the MI355X):", "", "```", command, "```", "",
             "| kernel | calls | avg µs | min µs | max µs | share of GPU time |", "|---|---|---|---|---|---|"]
    for name, n, avg, mn, mx, s in rows:
        short = name.split("(")[0].replace("void ", "")
        if "moe::" not in short:
            continue
        lines.append(f"| `{short}` | {n} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | {100 * s / tot:.1f}% |")
    return "\n".join(lines) + "\n"


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("out")
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    q = sub.add_parser("traffic")
    q.add_argument("fetch_db")
    q.add_argument("write_db")
    q.add_argument("out")
    q.add_argument("--kernel", required=True)
    q.add_argument("--calib-mib", type=int, required=True)
    q.add_argument("--command-fetch", required=True)
    q.add_argument("--command-write", required=True)
    k = sub.add_parser("counters")
    k.add_argument("db")
    k.add_argument("out")
    k.add_argument("--kernel", required=True)
    k.add_argument("--title", required=True)
    k.add_argument("--command", required=True)
    a = p.parse_args(argv)
    if a.what == "counters":
        with open(a.out, "w") as f:
            f.write(counters_md(a.db, a.kernel, a.title, a.command))
        return 0
    if a.what == "trace":
        with open(a.out, "w") as f:
            f.write(trace_md(a.db, a.title, a.command))
    else:
        d = traffic(a.fetch_db, a.write_db, a.kernel, a.calib_mib)
        d.update(kernel=a.kernel, source_sha256=source_hash(),
                 traffic_bytes_per_launch=int(d["fetch_kb_per_launch"] * 1024 * d["fetch_factor"]
                                              + d["write_kb_per_launch"] * 1024 * d["write_factor"]),
                 command_fetch=a.command_fetch, command_write=a.command_write)
        with open(a.out, "w") as f:
            json.dump(d, f, indent=1)
            f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
