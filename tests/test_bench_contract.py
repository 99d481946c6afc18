"""bench.py's contract logic, on the CPU: it refuses more than one GPU before
touching any device, and it reports a committed HBM-traffic figure only while
the kernel source and every local header it includes still hash to the
digest recorded with the counters."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_unchanged_sources(tmp_path, monkeypatch):
    import bench
    csrc = tmp_path / "ubatch_attention_paged_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "include").mkdir()
    (tmp_path / "profiles").mkdir()
    (csrc / "k.hip").write_text('#include "a.hpp"\n#include <hip/hip_runtime.h>\nkernel\n')
    (csrc / "a.hpp").write_text('#include "b.hpp"\n#include "api.h"\n')
    (csrc / "b.hpp").write_text("// b\n")
    (tmp_path / "include" / "api.h").write_text("// api\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    digest = bench.kernel_source_digest("k.hip")
    rec = {"source_digest": digest, "bytes_per_launch": 1234.4}
    (tmp_path / "profiles" / "k_x_traffic.json").write_text(json.dumps(rec))
    assert bench.committed_traffic("k_x", "k.hip") == 1234
    # a header two includes deep, then one under include/
    (csrc / "b.hpp").write_text("// b, changed\n")
    assert bench.kernel_source_digest("k.hip") != digest
    assert bench.committed_traffic("k_x", "k.hip") is None
    (csrc / "b.hpp").write_text("// b\n")
    assert bench.committed_traffic("k_x", "k.hip") == 1234
    (tmp_path / "include" / "api.h").write_text("// api, changed\n")
    assert bench.committed_traffic("k_x", "k.hip") is None
    # no summary at all
    assert bench.committed_traffic("k_y", "k.hip") is None


def test_committed_summaries_record_a_digest():
    for name in ("k_attn_mfma_traffic.json", "k_attn_valu_traffic.json"):
        rec = json.load(open(os.path.join(ROOT, "profiles", name)))
        assert len(rec["source_digest"]) == 64 and rec["bytes_per_launch"] > 0


def test_trace_average_is_reported_only_for_unchanged_sources(tmp_path, monkeypatch):
    import bench
    csrc = tmp_path / "ubatch_attention_paged_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "include").mkdir()
    (tmp_path / "profiles").mkdir()
    (csrc / "k.hip").write_text("kernel\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"source_digest": bench.kernel_source_digest("k.hip"), "legs": {"prefill": {"avg_ns": 250000.0}}}
    (tmp_path / "profiles" / "k_x_trace.json").write_text(json.dumps(rec))
    assert abs(bench.committed_trace_ms("k_x", "k.hip", "prefill") - 0.25) < 1e-12
    assert bench.committed_trace_ms("k_x", "k.hip", "cb_decode") is None
    (csrc / "k.hip").write_text("kernel, changed\n")
    assert bench.committed_trace_ms("k_x", "k.hip", "prefill") is None


def test_trace_stats_skips_warmup_dispatches(tmp_path):
    """--trace-stats keeps exactly the dispatches after the warm-up ones, of
    the named kernel only, in dispatch order."""
    import bench
    hdr = '"Kind","Dispatch_Id","Kernel_Name","Start_Timestamp","End_Timestamp"\n'
    rows = []
    for i in range(10):
        rows.append(f'"KERNEL_DISPATCH",{2 * i + 1},"void kvattn::k_attn_mfma<128, 2, false>(kvattn::AttnArgs)",'
                    f'{1000 * i},{1000 * i + 100 + i}\n')
        rows.append(f'"KERNEL_DISPATCH",{2 * i + 2},"kvattn::k_store_commit(kvattn::StoreArgs, kvattn::CsrArgs)",'
                    f'{1000 * i + 500},{1000 * i + 550}\n')
    p = tmp_path / "t.csv"
    p.write_text(hdr + "".join(reversed(rows)))
    r = bench.trace_stats(str(p), "k_attn_mfma", 3, 4)
    assert (r["n"], r["dispatches_total"], r["min_ns"], r["max_ns"]) == (4, 10, 103, 106)
    assert r["avg_ns"] == 104.5
    assert bench.trace_stats(str(p), "k_store_commit", 0, 0)["n"] == 10


def test_counter_stats_average_per_dispatch(tmp_path):
    """--counter-stats sums a kernel's counter rows per dispatch (rocprofv3
    may report one row per XCD) and averages over the selected dispatches."""
    import bench
    hdr = '"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n'
    rows = []
    for i in range(6):
        for part in (1.0, 2.0):       # two rows per dispatch and counter
            rows.append(f'{i},"void kvattn::k_attn_valu<128, 2>(kvattn::AttnArgs)","FETCH_SIZE",{part * (i + 1)}\n')
        rows.append(f'{i},"kvattn::k_store(kvattn::StoreArgs)","FETCH_SIZE",1000.0\n')
    p = tmp_path / "c.csv"
    p.write_text(hdr + "".join(rows))
    r = bench.counter_stats(str(p), "k_attn_valu", 2, 3)
    assert r["n"] == 3 and r["dispatches_total"] == 6
    assert abs(r["mean"]["FETCH_SIZE"] - 3.0 * (3 + 4 + 5) / 3) < 1e-9


def test_trace_table_covers_whole_steps(tmp_path):
    """--table lists every kernel of the steps holding the selected
    dispatches: from the step's first kernel to just before the next step,
    without the next bench leg's kernels."""
    import bench
    hdr = '"Kind","Dispatch_Id","Kernel_Name","Start_Timestamp","End_Timestamp"\n'
    rows, d = [], 0

    def add(name, dur):
        nonlocal d
        d += 1
        rows.append(f'"KERNEL_DISPATCH",{d},"{name}",{10 ** 6 * d},{10 ** 6 * d + 1000 * dur}\n')
    for step in range(5):
        add("kvattn::k_apply_updates(kvattn::CsrArgs, long)", 4)
        add("kvattn::k_store(kvattn::StoreArgs)", 5)
        add("void kvattn::k_attn_mfma<128, 2, false, 1>(kvattn::AttnArgs)", 50)
        add("void kvattn::k_attn_valu<128, 2>(kvattn::AttnArgs)", 100 + step)
        add("kvattn::k_attn_reduce(kvattn::AttnArgs, int)", 10)
    add("void at::native::vectorized_elementwise_kernel<8>(int)", 7)
    p = tmp_path / "t.csv"
    p.write_text(hdr + "".join(rows))
    t = bench.trace_table(str(p), "k_attn_valu", 2, 3, "k_apply_updates")
    lines = t.splitlines()[1:]
    calls = {ln[:62].strip(): int(ln[64:71]) for ln in lines}
    assert len(lines) == 5 and all(c == 3 for c in calls.values()), t
    assert "vectorized" not in t
    # the mean of the selected valu dispatches only (steps 2, 3, 4)
    valu = [ln for ln in lines if "k_attn_valu" in ln][0]
    assert float(valu[71:81]) == 103.0
