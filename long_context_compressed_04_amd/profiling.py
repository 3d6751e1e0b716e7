"""Profile bookkeeping: which library kernel is which in a rocprofv3 trace, and the
summaries kept as text next to the code.

    python -m long_context_compressed_04_amd.profiling stats --db RUN.db --cmd "..." --out FILE
        kernel-trace summary (calls, average / min / max duration per kernel) of a
        `rocprofv3 --kernel-trace --stats` run, with the command that produced it.

    python -m long_context_compressed_04_amd.profiling counters --db RUN.db --cmd "..." --out FILE
        per-kernel averages of the counters (and derived metrics such as MfmaUtil) of a
        `rocprofv3 --pmc ...` run.

    python -m long_context_compressed_04_amd.profiling traffic --fetch F.db --write W.db \\
            --workload NAME --calib-bytes N --cmd-fetch "..." --cmd-write "..." --out FILE.json
        L2-to-fabric bytes per launch of each library kernel, from one `--pmc FETCH_SIZE`
        run and one `--pmc WRITE_SIZE` run.  Each counter is scaled by what it reads for a
        plain copy kernel of N bytes read and N bytes written in the same run (the
        calibration launch `bench.py --pmc-pass` makes).  The file records a hash of the
        kernel sources; a reader ignores it once those sources change.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sqlite3
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# library launch-timer name -> (regex on the demangled kernel name, source file)
KERNELS = {
    "index_scores_bf16": (r"index_scores_(mfma<\d+, false|lds<\d+, false|pf<)", "indexer.hip"),
    "index_rescore_bf16": (r"index_scores_lds<\d+, true", "indexer.hip"),
    "index_scores_mxfp4": (r"index_scores_mfma<\d+, true", "indexer.hip"),
    "index_scores_f32": (r"index_scores_f32", "indexer.hip"),
    "topk": (r"topk_", "topk.hip"),
    "mqa_bf16_w8": (r"mqa_w8_kernel", "mqa.hip"),
    "mqa_bf16_sd": (r"mqa_sd_kernel<false>", "mqa.hip"),
    "mqa_f8_sd": (r"mqa_sd_kernel<true>", "mqa.hip"),
    "mqa_bf16_h16": (r"mqa_bf16_kernel<", "mqa.hip"),
    "mqa_f32": (r"mqa_f32_kernel", "mqa.hip"),
    "mqa_combine": (r"mqa_combine_kernel", "mqa.hip"),
    "mqa_row_norms": (r"row_normalize_kernel", "mqa.hip"),
    "compress": (r"compress_kernel<", "compress.hip"),
    "mxfp4_quantize": (r"mxfp4_quantize_kernel", "compress.hip"),
    "fp8_quantize": (r"fp8_quantize_kernel", "compress.hip"),
}
# the calibration copy (a torch elementwise negation of an fp32 buffer)
CALIB_PATTERN = r"neg_kernel"
COMMON_SOURCES = ["csa_device.hpp", "csa_kernels.hpp", "select_device.hpp"]


def source_hash(kernel: str) -> str:
    """Hash of what decides the kernel's code: its source, the shared device headers,
    and the build script (compiler options, some per source)."""
    h = hashlib.sha256()
    src = KERNELS[kernel][1]
    paths = [os.path.join(CSRC, f) for f in ([src] if isinstance(src, str) else list(src)) + COMMON_SOURCES]
    for path in paths + [os.path.join(PKG, "build_lib.py")]:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def library_kernel(demangled: str):
    for name, (pat, _) in KERNELS.items():
        if re.search(pat, demangled):
            return name
    return None


def _kernel_rows(db):
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration from kernels").fetchall()
    con.close()
    return rows


def stats(db: str, cmd: str) -> str:
    agg = {}
    for name, dur in _kernel_rows(db):
        a = agg.setdefault(name, [0, 0.0, 1e30, 0.0])
        a[0] += 1
        a[1] += dur
        a[2] = min(a[2], dur)
        a[3] = max(a[3], dur)
    total = sum(a[1] for a in agg.values()) or 1.0
    lines = ["# rocprofv3 kernel-trace summary (durations in microseconds)",
             "# command: " + cmd, "#",
             "# %-20s %6s %10s %10s %10s %7s  %s" % ("library kernel", "calls", "avg_us", "min_us", "max_us",
                                                      "time%", "kernel")]
    for name, (n, s, mn, mx) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        lk = library_kernel(name) or "-"
        short = name if len(name) <= 90 else name[:87] + "..."
        lines.append("  %-20s %6d %10.2f %10.2f %10.2f %6.1f%%  %s" % (lk, n, s / n / 1e3, mn / 1e3, mx / 1e3,
                                                                      100.0 * s / total, short))
    return "\n".join(lines) + "\n"


def _counter_per_dispatch(db, counter):
    """{demangled kernel: [value per dispatch]} for one counter."""
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, dispatch_id, sum(value) from counters_collection "
                       "where counter_name = ? group by kernel_name, dispatch_id", (counter,)).fetchall()
    con.close()
    out = {}
    for name, _, v in rows:
        out.setdefault(name, []).append(float(v))
    return out


def traffic(fetch_db, write_db, calib_bytes, workload, cmd_fetch, cmd_write):
    fetch = _counter_per_dispatch(fetch_db, "FETCH_SIZE")
    write = _counter_per_dispatch(write_db, "WRITE_SIZE")

    def calib(per):
        vals = [max(v) for k, v in per.items() if re.search(CALIB_PATTERN, k)]
        if not vals:
            raise SystemExit("no calibration copy (%s) in the counter run" % CALIB_PATTERN)
        return max(vals)

    f_kib, w_kib = calib(fetch), calib(write)
    f_scale = calib_bytes / (f_kib * 1024.0)
    w_scale = calib_bytes / (w_kib * 1024.0)
    res = {"workload": workload, "counter_unit": "KiB per dispatch", "calibration_bytes": calib_bytes,
           "calibration_fetch_kib": f_kib, "calibration_write_kib": w_kib, "fetch_scale": f_scale,
           "write_scale": w_scale, "command_fetch": cmd_fetch, "command_write": cmd_write, "kernels": {}}
    for lk in KERNELS:
        fv = [v for k, vs in fetch.items() if library_kernel(k) == lk for v in vs]
        wv = [v for k, vs in write.items() if library_kernel(k) == lk for v in vs]
        if not fv or not wv:
            continue
        fa, wa = sum(fv) / len(fv), sum(wv) / len(wv)
        res["kernels"][lk] = {"dispatches": len(fv), "fetch_kib": round(fa, 1), "write_kib": round(wa, 1),
                              "bytes_per_launch": int(round(fa * 1024 * f_scale + wa * 1024 * w_scale)),
                              "source_hash": source_hash(lk)}
    return res


def counters(db: str, cmd: str) -> str:
    """Per library kernel: the average per dispatch of every counter (and derived metric)
    in a `rocprofv3 --pmc ...` run, as rocprofv3 reduced it over the GPU's instances."""
    con = sqlite3.connect(db)
    names = [r[0] for r in con.execute("select distinct counter_name from counters_collection order by counter_name")]
    con.close()
    per = {c: _counter_per_dispatch(db, c) for c in names}
    lines = ["# rocprofv3 counter summary (average per dispatch)", "# command: " + cmd, "#",
             "# %-20s %10s  %s" % ("library kernel", "dispatches", "  ".join("%18s" % c for c in names))]
    kernels = sorted({library_kernel(k) or "-" for c in names for k in per[c]})
    for lk in kernels:
        vals, n = [], 0
        for c in names:
            v = [x for k, xs in per[c].items() if (library_kernel(k) or "-") == lk for x in xs]
            n = max(n, len(v))
            vals.append(sum(v) / len(v) if v else float("nan"))
        lines.append("  %-20s %10d  %s" % (lk, n, "  ".join("%18.6g" % v for v in vals)))
    return "\n".join(lines) + "\n"


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--db", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--db", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    t.add_argument("--out", required=True)
    a = p.parse_args(argv)
    if a.what in ("stats", "counters"):
        text = (stats if a.what == "stats" else counters)(a.db, a.cmd)
        with open(a.out, "w") as f:
            f.write(text)
        sys.stdout.write(text)
    else:
        res = traffic(a.fetch, a.write, a.calib_bytes, a.workload, a.cmd_fetch, a.cmd_write)
        with open(a.out, "w") as f:
            json.dump(res, f, indent=1)
            f.write("\n")
        print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
