"""Host-side tools, on the CPU: the benchmark's one-GPU guard, and the profile bookkeeping
(kernel names -> library launch timers, the kernel-trace summary, the HBM-traffic scaling)."""
import os
import re
import sqlite3
import subprocess
import sys

import pytest

from long_context_compressed_04_amd import profiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def _profile_rows():
    """(library kernel, demangled name) of every row of the committed kernel-trace summaries."""
    rows = []
    for f in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if not f.startswith("kernels_"):
            continue
        for line in open(os.path.join(ROOT, "profiles", f)):
            if line.startswith("#") or not line.strip():
                continue
            m = re.match(r"\s*(\S+)\s+\d+\s+[\d.]+\s+[\d.]+\s+[\d.]+\s+[\d.]+%\s+(.*)$", line)
            assert m, line
            rows.append((m.group(1), m.group(2)))
    return rows


def test_committed_profiles_name_every_library_kernel():
    rows = _profile_rows()
    assert rows
    for lk, name in rows:
        if "csa::" in name:
            assert lk != "-", name                  # every library kernel has its timer name
        if not name.endswith("..."):                # (long names are cut in the summary)
            assert (profiling.library_kernel(name) or "-") == lk, name


def test_library_kernel_names():
    k = profiling.library_kernel
    assert k("void csa::mqa_sd_kernel<false>(csa::MqaArgs, csa::MqaLaunch, float*, float*)") == "mqa_bf16_sd"
    assert k("void csa::mqa_sd_kernel<true>(csa::MqaArgs, csa::MqaLaunch, float*, float*)") == "mqa_f8_sd"
    assert k("void csa::fp8_quantize_kernel<true>(void const*, long, unsigned char*)") == "fp8_quantize"
    assert k("void csa::index_scores_mfma<2, true, 8>(csa::IndexArgs, float*, int)") == "index_scores_mxfp4"
    assert k("void csa::index_scores_lds<2, false>(csa::IndexArgs, float*)") == "index_scores_bf16"
    assert k("void csa::index_scores_lds<2, true>(csa::IndexArgs, float*)") == "index_rescore_bf16"
    assert k("void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel>") is None


def _db(path, kernels=(), counters=()):
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, duration integer)")
    con.executemany("insert into kernels values (?, ?)", kernels)
    con.execute("create table counters_collection (kernel_name text, dispatch_id integer, counter_name text, "
                "value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", counters)
    con.commit()
    con.close()
    return path


def test_stats_summary(tmp_path):
    mqa = "void csa::mqa_sd_kernel<false>(csa::MqaArgs, csa::MqaLaunch, float*, float*)"
    db = _db(str(tmp_path / "k.db"), kernels=[(mqa, 10000), (mqa, 20000), ("other_kernel", 10000)])
    text = profiling.stats(db, "CMD")
    assert "# command: CMD" in text
    line = next(l for l in text.splitlines() if "mqa_sd_kernel" in l)
    # two calls, 15 us average, 10 / 20 us extremes, 75% of the time
    assert re.match(r"\s*mqa_bf16_sd\s+2\s+15\.00\s+10\.00\s+20\.00\s+75\.0%", line), line


def test_traffic_scales_by_the_calibration_copy(tmp_path):
    mqa = "void csa::mqa_sd_kernel<false>(csa::MqaArgs, csa::MqaLaunch, float*, float*)"
    calib = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel<float>>"
    # the copy moves 1 MiB each way; the counters read half of it for fetch, all of it for write
    f = _db(str(tmp_path / "f.db"), counters=[(calib, 1, "FETCH_SIZE", 512.0), (mqa, 2, "FETCH_SIZE", 100.0),
                                              (mqa, 3, "FETCH_SIZE", 300.0)])
    w = _db(str(tmp_path / "w.db"), counters=[(calib, 1, "WRITE_SIZE", 1024.0), (mqa, 2, "WRITE_SIZE", 10.0),
                                              (mqa, 3, "WRITE_SIZE", 30.0)])
    res = profiling.traffic(f, w, 1 << 20, "wl", "CF", "CW")
    assert res["fetch_scale"] == pytest.approx(2.0) and res["write_scale"] == pytest.approx(1.0)
    ent = res["kernels"]["mqa_bf16_sd"]
    assert ent["dispatches"] == 2 and ent["fetch_kib"] == 200.0 and ent["write_kib"] == 20.0
    assert ent["bytes_per_launch"] == 200 * 1024 * 2 + 20 * 1024
    assert ent["source_hash"] == profiling.source_hash("mqa_bf16_sd")
