"""Host logic of bench.py that needs no GPU: the key that ties the committed HBM-traffic
counters to the dominant kernel's code, and the launch-gap analysis of a kernel trace."""
import os
import shutil
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.fixture
def sources(tmp_path, monkeypatch):
    copies = []
    for f in bench.GEMM_SOURCES:
        dst = tmp_path / os.path.basename(f)
        shutil.copy(f, dst)
        copies.append(str(dst))
    monkeypatch.setattr(bench, "GEMM_SOURCES", copies)
    return copies


def test_source_hash_ignores_comments_and_blank_lines(sources):
    h0 = bench.gemm_source_hash()
    with open(sources[0], "a", encoding="utf-8") as f:
        f.write("\n// a remark\n/* a block\n   remark */\n\n")
    assert bench.gemm_source_hash() == h0


def test_source_hash_follows_code(sources):
    h0 = bench.gemm_source_hash()
    with open(sources[1], "a", encoding="utf-8") as f:
        f.write("\nnamespace frt { constexpr int kUnused = 1; }\n")
    assert bench.gemm_source_hash() != h0


def _write_trace(path, decisions, kernels_per_decision, dur_ns, gap_ns, stall_at=None, stall_ns=0):
    """A kernel-trace CSV in rocprofv3's column names: each decision starts with the
    producer that reads no partials, then kernels of dur_ns each, gap_ns apart; one gap of
    stall_ns after dispatch stall_at of every decision."""
    t = 1_000_000
    with open(path, "w", encoding="utf-8") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for _ in range(decisions):
            for j in range(kernels_per_decision):
                name = "void frt::rnq_kernel<0, 1, 1>(frt::RnqParams)" if j == 0 else "void frt::other<1>(int)"
                f.write(f"\"{name}\",{t},{t + dur_ns}\n")
                t += dur_ns + (stall_ns if j == stall_at else gap_ns)
            t += 50_000  # between decisions (host side)


def test_trace_analysis_gap_shares(tmp_path):
    path = tmp_path / "trace.csv"
    # 3 decisions of 10 dispatches: 4 us kernels, 1 us gaps, one 20 us stall after dispatch 4
    _write_trace(path, 3, 10, 4000, 1000, stall_at=4, stall_ns=20000)
    res = bench.analyze_chain_trace(str(path))
    assert res["decisions"] == 3 and res["dispatches_per_decision"] == 10
    m = res["median"]
    span = 10 * 4.0 + 8 * 1.0 + 20.0            # 9 gaps: 8 of 1 us, one of 20 us
    assert m["span_us"] == pytest.approx(span)
    assert m["kernel_sum_us"] == pytest.approx(40.0)
    assert m["raw_gap_share"] == pytest.approx(round((span - 40.0) / span, 4))
    assert m["gaps_over_stall"] == 1
    assert m["gap_share_without_stalls"] == pytest.approx(round(8.0 / 48.0, 4))
    assert m["median_gap_us"] == pytest.approx(1.0)


def test_trace_analysis_abutting_kernels(tmp_path):
    path = tmp_path / "trace.csv"
    _write_trace(path, 2, 7, 3000, 0)
    m = bench.analyze_chain_trace(str(path))["median"]
    assert m["raw_gap_share"] == 0.0 and m["gaps_over_stall"] == 0 and m["median_gap_us"] == 0.0


def test_committed_profiles_are_read_only_for_matching_sources(tmp_path, monkeypatch):
    """The traffic and launch-gap figures come from the committed summaries only while the
    sources they were taken on are unchanged (the hash recorded with them)."""
    for name, getter in (("TRAFFIC_PROFILE", bench.measured_traffic), ("CHAIN_TRACE_PROFILE", bench.measured_launch_gaps)):
        text = open(getattr(bench, name), encoding="utf-8").read()
        stale = tmp_path / (name + ".md")
        stale.write_text("\n".join("source_sha256: 0000000000000000" if l.startswith("source_sha256:") else l
                                   for l in text.splitlines()), encoding="utf-8")
        monkeypatch.setattr(bench, name, str(stale))
        assert getter() is None, name
        monkeypatch.setattr(bench, name, str(tmp_path / "missing.md"))
        assert getter() is None, name


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
