"""Turn rocprofv3 CSV output into the short summaries kept under ``profiles/``.

* ``ktrace``: per-kernel duration statistics of a ``--kernel-trace --stats``
  run, plus the mean over dispatches ``[skip, skip + timed)`` of the named
  kernel (the bench's timed window: after its warmup launches, before the
  launches it times one by one).
* ``traffic``: HBM bytes per dispatch of a kernel from two ``--pmc`` runs
  (FETCH_SIZE, then WRITE_SIZE, both in KiB per dispatch), each scaled by what
  the same counter reads for a plain copy kernel of known size.  The record
  carries a digest of the kernel's sources so that ``bench.py`` reports it
  only while the kernel is unchanged.
* ``traffic-table``: the same scaled bytes for several kernels of one run, as
  a markdown table against each kernel's algorithmic bytes.
* ``traffic-grid``: the same, summed over every dispatch of each kernel, with
  each dispatch's algorithmic bytes from its grid size (for runs that launch
  one kernel at several sizes).

Usage::

    python -m collective_reduction_ring_amd.profiling ktrace --trace T.csv --stats S.csv \\
        --kernel fold_kernel --skip 10 --timed 100 --command "..." --out profiles/x.md
    python -m collective_reduction_ring_amd.profiling traffic --fetch F.csv --write W.csv \\
        --cal-fetch CF.csv --cal-write CW.csv --kernel fold_kernel --cal-kernel gather_kernel \\
        --cal-bytes 1073741824 --algorithmic-bytes 2415919104 --commands "..." --out profiles/x.json
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# Sources that determine the reduce-scatter fold kernel's machine code.
FOLD_SOURCES = ("fold_impl.h", "fold_f32.hip", "mem.h", "rsx_internal.h")


def kernel_source_digest(files=FOLD_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def counter_per_dispatch(path: str, counter: str, kernel: str) -> list[float]:
    """Values of `counter` for every dispatch whose name contains `kernel`."""
    return [float(r["Counter_Value"]) for r in _rows(path)
            if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]]


def ktrace_summary(trace: str, stats: str, kernel: str, skip: int, timed: int, command: str) -> str:
    srows = _rows(stats)
    rows = sorted((r for r in _rows(trace) if kernel and kernel in r["Kernel_Name"]),
                  key=lambda r: int(r["Start_Timestamp"]))
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    last = durs[skip:skip + timed] if timed else durs[skip:]
    lines = [
        "# rocprofv3 kernel trace summary",
        "",
        "Command:",
        "",
        "```",
        command,
        "```",
        "",
        "| kernel | calls | average (us) | min (us) | max (us) | share |",
        "|---|---|---|---|---|---|",
    ]
    for r in srows:
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f}% |")
    if not kernel:
        return "\n".join(lines + [""])
    lines += [
        "",
        f"`{kernel}`: {len(durs)} dispatches; mean of dispatches {skip}..{skip + len(last) - 1} "
        f"(the timed window): "
        f"**{statistics.mean(last):.1f} us**, median {statistics.median(last):.1f} us, "
        f"min {min(last):.1f} us.",
        "",
    ]
    return "\n".join(lines)


def traffic_record(fetch: str, write: str, cal_fetch: str, cal_write: str, kernel: str,
                   cal_kernel: str, cal_bytes: int, algorithmic_bytes: int, commands: str) -> dict:
    f = counter_per_dispatch(fetch, "FETCH_SIZE", kernel)
    w = counter_per_dispatch(write, "WRITE_SIZE", kernel)
    cf = counter_per_dispatch(cal_fetch, "FETCH_SIZE", cal_kernel)
    cw = counter_per_dispatch(cal_write, "WRITE_SIZE", cal_kernel)
    if not (f and w and cf and cw):
        raise SystemExit("missing counter rows for the kernel or the calibration kernel")
    fk, wk = statistics.mean(f), statistics.mean(w)
    cfk, cwk = statistics.mean(cf), statistics.mean(cw)
    f_scale = cal_bytes / (cfk * 1024.0)
    w_scale = cal_bytes / (cwk * 1024.0)
    fetch_b = fk * 1024.0 * f_scale
    write_b = wk * 1024.0 * w_scale
    return {
        "kernel": kernel,
        "kernel_source_sha256": kernel_source_digest(),
        "dispatches": {"fetch": len(f), "write": len(w)},
        "FETCH_SIZE_KiB_per_dispatch": round(fk, 3),
        "WRITE_SIZE_KiB_per_dispatch": round(wk, 3),
        "calibration": {
            "kernel": cal_kernel,
            "bytes_read_and_written_per_dispatch": cal_bytes,
            "FETCH_SIZE_KiB_per_dispatch": round(cfk, 3),
            "WRITE_SIZE_KiB_per_dispatch": round(cwk, 3),
            "fetch_scale": round(f_scale, 6),
            "write_scale": round(w_scale, 6),
        },
        "fetch_bytes_per_launch": round(fetch_b),
        "write_bytes_per_launch": round(write_b),
        "traffic_bytes_per_launch": round(fetch_b + write_b),
        "algorithmic_bytes_per_launch": algorithmic_bytes,
        "traffic_over_algorithmic": round((fetch_b + write_b) / algorithmic_bytes, 5),
        "commands": commands,
    }


def traffic_table(fetch: str, write: str, cal_fetch: str, cal_write: str, cal_kernel: str,
                  cal_bytes: int, kernels: list[tuple[str, int]], commands: str) -> str:
    """Markdown table of HBM bytes per dispatch for (kernel, algorithmic bytes) pairs."""
    cf = counter_per_dispatch(cal_fetch, "FETCH_SIZE", cal_kernel)
    cw = counter_per_dispatch(cal_write, "WRITE_SIZE", cal_kernel)
    if not (cf and cw):
        raise SystemExit("missing counter rows for the calibration kernel")
    f_scale = cal_bytes / (statistics.mean(cf) * 1024.0)
    w_scale = cal_bytes / (statistics.mean(cw) * 1024.0)
    lines = ["# rocprofv3 HBM traffic per dispatch", "", "Commands:", "", "```", commands, "```", "",
             f"Scale factors from the calibration kernel `{cal_kernel}` ({cal_bytes} bytes read and written "
             f"per dispatch): FETCH_SIZE x {f_scale:.5f}, WRITE_SIZE x {w_scale:.5f}.", "",
             "| kernel | dispatches | fetch bytes | write bytes | traffic | algorithmic | traffic / algorithmic |",
             "|---|---|---|---|---|---|---|"]
    for kernel, algo in kernels:
        f = counter_per_dispatch(fetch, "FETCH_SIZE", kernel)
        w = counter_per_dispatch(write, "WRITE_SIZE", kernel)
        if not (f and w):
            raise SystemExit(f"missing counter rows for {kernel}")
        fb = statistics.mean(f) * 1024.0 * f_scale
        wb = statistics.mean(w) * 1024.0 * w_scale
        lines.append(f"| `{kernel}` | {len(f)} | {fb:,.0f} | {wb:,.0f} | {fb + wb:,.0f} | {algo:,} | "
                     f"{(fb + wb) / algo:.4f} |")
    return "\n".join(lines) + "\n"


def _dispatches(path: str, counter: str, kernel: str) -> list[tuple[int, float]]:
    """(grid size in work-items, counter value) of every dispatch whose name contains `kernel`."""
    return [(int(r["Grid_Size"]), float(r["Counter_Value"])) for r in _rows(path)
            if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]]


def traffic_grid_table(fetch: str, write: str, cal_fetch: str, cal_write: str, cal_kernel: str,
                       cal_bytes: int, kernels: list[tuple[str, str, int]], commands: str) -> str:
    """HBM bytes against algorithmic bytes summed over every dispatch of each kernel.

    `kernels`: (name, "lane" | "dispatch", bytes): the algorithmic bytes of a
    dispatch are its grid size times `bytes` ("lane": the kernel moves a fixed
    number of 16-byte vectors per work-item) or `bytes` itself ("dispatch").
    Summing over dispatches handles runs that launch one kernel at several
    sizes (buckets of different lengths)."""
    cf = counter_per_dispatch(cal_fetch, "FETCH_SIZE", cal_kernel)
    cw = counter_per_dispatch(cal_write, "WRITE_SIZE", cal_kernel)
    if not (cf and cw):
        raise SystemExit("missing counter rows for the calibration kernel")
    f_scale = cal_bytes / (statistics.mean(cf) * 1024.0)
    w_scale = cal_bytes / (statistics.mean(cw) * 1024.0)
    lines = ["# rocprofv3 HBM traffic, summed over every dispatch", "", "Commands:", "", "```", commands, "```",
             "", f"Scale factors from the calibration kernel `{cal_kernel}` ({cal_bytes} bytes read and written "
             f"per dispatch): FETCH_SIZE x {f_scale:.5f}, WRITE_SIZE x {w_scale:.5f}.", "",
             "| kernel | dispatches | grid sizes | fetch bytes | write bytes | traffic | algorithmic | "
             "traffic / algorithmic |", "|---|---|---|---|---|---|---|---|"]
    for kernel, unit, nbytes in kernels:
        f = _dispatches(fetch, "FETCH_SIZE", kernel)
        w = _dispatches(write, "WRITE_SIZE", kernel)
        if not (f and w):
            raise SystemExit(f"missing counter rows for {kernel}")
        fb = sum(v for _, v in f) * 1024.0 * f_scale
        wb = sum(v for _, v in w) * 1024.0 * w_scale
        if sorted(g for g, _ in f) != sorted(g for g, _ in w):
            raise SystemExit(f"{kernel}: the FETCH_SIZE and WRITE_SIZE runs launched different dispatches")
        algo = sum((g * nbytes if unit == "lane" else nbytes) for g, _ in f)
        grids = sorted({g for g, _ in f})
        lines.append(f"| `{kernel}` | {len(f)} | {', '.join(f'{g:,}' for g in grids)} | {fb:,.0f} | "
                     f"{wb:,.0f} | {fb + wb:,.0f} | {algo:,.0f} | {(fb + wb) / algo:.4f} |")
    return "\n".join(lines) + "\n"


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("ktrace")
    k.add_argument("--trace", required=True)
    k.add_argument("--stats", required=True)
    k.add_argument("--kernel", default="", help="kernel whose timed window to summarise")
    k.add_argument("--skip", type=int, default=0)
    k.add_argument("--timed", type=int, default=0)
    k.add_argument("--command", required=True)
    k.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for name in ("fetch", "write", "cal-fetch", "cal-write", "kernel", "cal-kernel", "commands", "out"):
        t.add_argument(f"--{name}", required=True)
    t.add_argument("--cal-bytes", type=int, required=True)
    t.add_argument("--algorithmic-bytes", type=int, required=True)
    tt = sub.add_parser("traffic-table")
    for name in ("fetch", "write", "cal-fetch", "cal-write", "cal-kernel", "commands", "out"):
        tt.add_argument(f"--{name}", required=True)
    tt.add_argument("--cal-bytes", type=int, required=True)
    tt.add_argument("--kernel", action="append", required=True,
                    help="NAME=ALGORITHMIC_BYTES (NAME matches a substring of the kernel name); repeatable")
    tg = sub.add_parser("traffic-grid")
    for name in ("fetch", "write", "cal-fetch", "cal-write", "cal-kernel", "commands", "out"):
        tg.add_argument(f"--{name}", required=True)
    tg.add_argument("--cal-bytes", type=int, required=True)
    tg.add_argument("--kernel", action="append", required=True,
                    help="NAME=lane:BYTES or NAME=dispatch:BYTES (NAME matches a substring); repeatable")
    a = ap.parse_args()
    if a.cmd == "traffic-grid":
        trip = []
        for k in a.kernel:
            name, spec = k.rsplit("=", 1)
            unit, nbytes = spec.split(":")
            trip.append((name, unit, int(nbytes)))
        text = traffic_grid_table(a.fetch, a.write, a.cal_fetch, a.cal_write, a.cal_kernel, a.cal_bytes,
                                  trip, a.commands)
        with open(a.out, "w") as f:
            f.write(text)
        print(text)
    elif a.cmd == "traffic-table":
        pairs = [(k.rsplit("=", 1)[0], int(k.rsplit("=", 1)[1])) for k in a.kernel]
        text = traffic_table(a.fetch, a.write, a.cal_fetch, a.cal_write, a.cal_kernel, a.cal_bytes,
                             pairs, a.commands)
        with open(a.out, "w") as f:
            f.write(text)
        print(text)
    elif a.cmd == "ktrace":
        text = ktrace_summary(a.trace, a.stats, a.kernel, a.skip, a.timed, a.command)
        with open(a.out, "w") as f:
            f.write(text)
        print(text)
    else:
        rec = traffic_record(a.fetch, a.write, a.cal_fetch, a.cal_write, a.kernel, a.cal_kernel,
                             a.cal_bytes, a.algorithmic_bytes, a.commands)
        with open(a.out, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
