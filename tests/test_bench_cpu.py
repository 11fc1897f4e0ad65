"""Host logic of bench.py that needs no GPU: the key that ties the committed HBM-traffic
counters to the dominant kernel's code."""
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



def test_bench_refuses_more_than_one_gpu():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
