"""Text summaries of rocprofv3 result databases (SQLite, rocpd schema).

  python -m modulation_bf16_row_amd.profiling trace RESULTS.db OUT.txt --command "..."
      per-kernel dispatch statistics from a --kernel-trace run
  python -m modulation_bf16_row_amd.profiling traffic FETCH.db WRITE.db OUT.txt \
        --kernel k_ln_modulate [--grid N] --calib 'k_probe_copy<3>' \
        --calib-default 'k_probe_copy<2>' --calib-bytes 1073741824 --command "..."
      HBM bytes per dispatch of one kernel from FETCH_SIZE and WRITE_SIZE runs,
      each scaled by what the same counter reads for a copy dispatch of known
      size (calib-bytes read and calib-bytes written): FETCH_SIZE by the copy
      with nontemporal loads (--calib) and, for comparison, by the copy with
      default-policy loads (--calib-default), whose factor is also recorded

  python -m modulation_bf16_row_amd.profiling clock RESULTS.db OUT.txt --command "..."
      per kernel, from a --pmc GRBM_COUNT run: the effective core clock of
      each dispatch of 200 us or more (GRBM_COUNT, summed over the XCDs, /
      XCDs / duration),
      the core cycles it took (clock x duration), and how closely duration
      follows the clock across dispatches (a correlation near -1 means a
      fixed number of core cycles: the dispatch is bound by the core clock,
      not by HBM)

  python -m modulation_bf16_row_amd.profiling counters RESULTS.db OUT.txt --command "..."
      per kernel, from a --pmc run of any counters: the median value of each
      counter per dispatch, and per work-item of the dispatch (for the
      shader instruction counters, which count wave instructions, times 64
      gives instructions per lane)

The traffic summary records a hash of the code of the kernel's translation
unit (--source) or of all kernel sources; the benchmark only
reports it while the sources still match.
"""
import argparse
import hashlib
import os
import re
import sqlite3
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))


def _code_only(text):
    """Source text without comments and whitespace (string literals kept)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            if not c.isspace():
                out.append(c)
            i += 1
    return "".join(out)


CSRC = os.path.join(PKG, "csrc")


def unit_files(source):
    """The file `source` of csrc/ and every csrc/ header it includes,
    directly or through other headers (#include "...")."""
    seen, todo = set(), [source]
    while todo:
        name = todo.pop()
        if name in seen or not os.path.exists(os.path.join(CSRC, name)):
            continue
        seen.add(name)
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            todo += re.findall(r'^\s*#\s*include\s+"([^"]+)"', f.read(), flags=re.M)
    return sorted(seen)


def kernel_source_hash(source=None):
    """Hash of the code (comments and whitespace excluded) of the kernel
    sources: of one translation unit (`source`, e.g. "dit_ln.hip", and the
    headers it includes) or, with no argument, of every C++/HIP source in
    csrc/."""
    names = unit_files(source) if source else sorted(
        n for n in os.listdir(CSRC) if n.endswith((".hip", ".hpp", ".cpp", ".h")))
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _short(name):
    """Kernel name without return type, namespace and parameter list; template
    arguments are kept (for the row kernels: chunks, mode (0 = lossless,
    1 = fast), and for the LayerNorm producers whether the E4M3 copy is
    written)."""
    name = re.sub(r"\(.*$", "", name).strip()
    return re.sub(r"^void ", "", name).replace("dit::", "")


def kernel_stats(db):
    """Per (kernel, grid size in work-items) dispatch statistics, largest total first."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration, grid_x * grid_y * grid_z from kernels").fetchall()
    by = {}
    for name, dur, grid in rows:
        by.setdefault((_short(name), int(grid)), []).append(dur / 1000.0)
    out = []
    for (name, grid), d in by.items():
        d = sorted(d)
        pct = lambda q: d[min(len(d) - 1, int(q * (len(d) - 1) + 0.5))]
        out.append((name, grid, len(d), statistics.mean(d), statistics.median(d), pct(0.1),
                    pct(0.9), d[0], d[-1], sum(d)))
    return sorted(out, key=lambda r: -r[-1])


def counter_values(db, counter):
    """(kernel name, grid size) -> list of per-dispatch values of one counter."""
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, grid_size, value from counters_collection where "
                       "counter_name = ?", (counter,)).fetchall()
    by = {}
    for name, grid, v in rows:
        by.setdefault((_short(name), int(grid)), []).append(float(v))
    return by


def _match(by, pattern, grid=None):
    keys = [k for k in by if (re.search(pattern, k[0]) or k[0].startswith(pattern))
            and (grid is None or k[1] == grid)]
    if not keys:
        raise SystemExit(f"no dispatch of {pattern!r} (grid {grid}) in {sorted(by)}")
    vals = [v for k in keys for v in by[k]]
    return statistics.mean(vals), len(vals)


def write_trace(db, out, command):
    lines = [f"# rocprofv3 kernel-trace summary (durations in microseconds; grid in work-items)",
             f"# command: {command}",
             f"# kernel_source_hash = {kernel_source_hash()}",
             f"{'kernel':40s} {'grid':>10s} {'calls':>6s} {'avg_us':>9s} {'median_us':>9s} "
             f"{'p10_us':>9s} {'p90_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_us':>11s}"]
    for name, grid, n, avg, med, p10, p90, lo, hi, tot in kernel_stats(db):
        lines.append(f"{name[:40]:40s} {grid:10d} {n:6d} {avg:9.3f} {med:9.3f} {p10:9.3f} "
                     f"{p90:9.3f} {lo:9.3f} {hi:9.3f} {tot:11.1f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def write_traffic(fetch_db, write_db, out, kernel, calib, calib_bytes, command, grid=None,
                  source=None, calib_default=None):
    fetch = counter_values(fetch_db, "FETCH_SIZE")
    write = counter_values(write_db, "WRITE_SIZE")
    f_k, nf = _match(fetch, kernel, grid)
    w_k, nw = _match(write, kernel, grid)
    f_c, _ = _match(fetch, calib)
    w_c, _ = _match(write, calib)
    f_scale = calib_bytes / (f_c * 1024.0)
    w_scale = calib_bytes / (w_c * 1024.0)
    extra = []
    if calib_default:
        f_d, _ = _match(fetch, calib_default)
        extra = [f"calib_default_loads_kernel = {calib_default}",
                 f"calib_default_loads_fetch_kib = {f_d:.1f}",
                 f"fetch_scale_default_loads = {calib_bytes / (f_d * 1024.0):.4f}"]
    read_b = f_k * 1024.0 * f_scale
    write_b = w_k * 1024.0 * w_scale
    lines = [
        "# HBM traffic per dispatch from rocprofv3 memory counters",
        f"# command: {command}",
        f"# FETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is scaled by "
        f"calib_bytes / (counter of the copy dispatch)",
        f"kernel = {kernel}",
        f"grid_work_items = {grid if grid is not None else 'any'}",
        f"dispatches_fetch = {nf}",
        f"dispatches_write = {nw}",
        f"fetch_kib_per_dispatch = {f_k:.1f}",
        f"write_kib_per_dispatch = {w_k:.1f}",
        f"calib_kernel = {calib}",
        f"calib_bytes_each_way = {calib_bytes}",
        f"calib_fetch_kib = {f_c:.1f}",
        f"calib_write_kib = {w_c:.1f}",
        f"fetch_scale = {f_scale:.4f}",
        f"write_scale = {w_scale:.4f}",
        *extra,
        f"hbm_read_bytes_per_launch = {read_b:.0f}",
        f"hbm_write_bytes_per_launch = {write_b:.0f}",
        f"hbm_bytes_per_launch = {read_b + write_b:.0f}",
        f"kernel_source = {source or 'all of csrc'}",
        f"kernel_source_hash = {kernel_source_hash(source)}",
    ]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _pearson(xs, ys):
    mx, my = statistics.mean(xs), statistics.mean(ys)
    sxy = sum((x - mx) * (y - my) for x, y in zip(xs, ys))
    sxx = sum((x - mx) ** 2 for x in xs)
    syy = sum((y - my) ** 2 for y in ys)
    return sxy / (sxx * syy) ** 0.5 if sxx > 0 and syy > 0 else float("nan")


def clock_stats(db, xcds=8, min_us=200.0):
    """Per (kernel, grid): dispatches, median duration (us), median effective
    clock (GHz), median core cycles (thousands: us x GHz), and the correlation of
    duration with clock, over dispatches of at least min_us."""
    con = sqlite3.connect(db)
    rows = con.execute("select dispatch_id, kernel_name, grid_size, value, duration from "
                       "counters_collection where counter_name = 'GRBM_COUNT'").fetchall()
    by = {}
    for _, name, grid, v, dur in rows:
        if dur and dur / 1000.0 >= min_us:
            by.setdefault((_short(name), int(grid)), []).append((dur / 1000.0, v / xcds / dur))
    out = []
    for (name, grid), pts in by.items():
        if len(pts) < 4:
            continue
        d = [p[0] for p in pts]
        c = [p[1] for p in pts]
        cyc = [a * b for a, b in pts]
        out.append((name, grid, len(pts), statistics.median(d), statistics.median(c), min(c),
                    max(c), statistics.median(cyc), _pearson(d, c)))
    return sorted(out, key=lambda r: -r[2] * r[3])


def write_clock(db, out, command):
    lines = ["# effective core clock per dispatch from rocprofv3 --pmc GRBM_COUNT "
             "(summed over 8 XCDs), dispatches of 200 us or more (shorter ones read above "
             "the 2.4 GHz peak: the counter window outlasts the kernel)",
             f"# command: {command}",
             f"# kernel_source_hash = {kernel_source_hash()}",
             f"{'kernel':40s} {'grid':>10s} {'n':>4s} {'med_us':>9s} {'clk_GHz':>8s} "
             f"{'min_GHz':>8s} {'max_GHz':>8s} {'kcycles':>9s} {'corr(dur,clk)':>14s}"]
    for name, grid, n, d, c, lo, hi, cyc, r in clock_stats(db):
        lines.append(f"{name[:40]:40s} {grid:10d} {n:4d} {d:9.2f} {c:8.3f} {lo:8.3f} {hi:8.3f} "
                     f"{cyc:9.1f} {r:14.2f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counter_table(db):
    """{(kernel, grid): {counter: median value per dispatch}} over every
    counter of a --pmc run."""
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, grid_size, counter_name, value from "
                       "counters_collection").fetchall()
    by = {}
    for name, grid, cn, v in rows:
        by.setdefault((_short(name), int(grid)), {}).setdefault(cn, []).append(float(v))
    return {k: {cn: statistics.median(vs) for cn, vs in d.items()} for k, d in by.items()}


def write_counters(db, out, command, min_dispatches=4):
    table = counter_table(db)
    names = sorted({cn for d in table.values() for cn in d})
    lines = ["# shader counters per dispatch from rocprofv3 --pmc (median over dispatches); "
             "'/item' divides by the dispatch's work-items (x 64 = per lane for wave counts)",
             f"# command: {command}",
             f"# kernel_source_hash = {kernel_source_hash()}",
             f"{'kernel':40s} {'grid':>10s} " + " ".join(f"{n:>16s} {n[-8:] + '/item':>16s}"
                                                         for n in names)]
    con = sqlite3.connect(db)
    counts = dict(((_short(n), int(g)), c) for n, g, c in con.execute(
        "select kernel_name, grid_size, count(distinct dispatch_id) from counters_collection "
        "group by kernel_name, grid_size").fetchall())
    for (name, grid), d in sorted(table.items(), key=lambda kv: -kv[0][1]):
        if not name.startswith("k_") or counts.get((name, grid), 0) < min_dispatches:
            continue
        cells = []
        for n in names:
            v = d.get(n)
            cells.append(f"{v:16.0f} {v / grid:16.4f}" if v is not None else f"{'-':>16s} {'-':>16s}")
        lines.append(f"{name[:40]:40s} {grid:10d} " + " ".join(cells))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("out")
    t.add_argument("--command", default="")
    c = sub.add_parser("traffic")
    c.add_argument("fetch_db")
    c.add_argument("write_db")
    c.add_argument("out")
    c.add_argument("--kernel", required=True)
    c.add_argument("--calib", default="k_probe_copy<3>")
    c.add_argument("--calib-default", default=None,
                   help="copy dispatch with default-policy loads (its factor is recorded)")
    c.add_argument("--calib-bytes", type=float, default=float(1 << 30))
    c.add_argument("--grid", type=int, default=None,
                   help="only dispatches of this grid size (work-items)")
    c.add_argument("--source", default=None,
                   help="csrc file defining the kernel; its translation unit is hashed")
    c.add_argument("--command", default="")
    q = sub.add_parser("counters")
    q.add_argument("db")
    q.add_argument("out")
    q.add_argument("--command", default="")
    k = sub.add_parser("clock")
    k.add_argument("db")
    k.add_argument("out")
    k.add_argument("--command", default="")
    a = ap.parse_args()
    if a.cmd == "trace":
        write_trace(a.db, a.out, a.command)
    elif a.cmd == "clock":
        write_clock(a.db, a.out, a.command)
    elif a.cmd == "counters":
        write_counters(a.db, a.out, a.command)
    else:
        write_traffic(a.fetch_db, a.write_db, a.out, a.kernel, a.calib, a.calib_bytes, a.command,
                      a.grid, a.source, a.calib_default)


if __name__ == "__main__":
    main()
