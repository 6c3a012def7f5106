"""bench.py's host logic, without a GPU: the single-GPU refusal, the code hash
that ties a counter summary to the decode kernel's sources, and the HBM
traffic it derives from such a summary."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr and r.stdout == ""


def _sources(tmp_path, texts):
    paths = []
    for i, t in enumerate(texts):
        p = tmp_path / f"src{i}.hip"
        p.write_text(t)
        paths.append(str(p))
    return paths


def test_code_hash_ignores_comments_only(tmp_path, monkeypatch):
    versions = {
        "base": "int f(int a) {\n  return a + 1;  // one\n}\n/* block\n comment */\n",
        "comments": "int f(int a) {\n\n  return a + 1;   // another comment\n}\n/* x */\n",
        "code": "int f(int a) {\n  return a + 2;  // one\n}\n/* block\n comment */\n",
    }
    h = {}
    for name, text in versions.items():
        d = tmp_path / name
        d.mkdir()
        monkeypatch.setattr(bench, "GEMV_SOURCES", _sources(d, [text]))
        h[name] = bench.gemv_source_hash()
    assert h["comments"] == h["base"]
    assert h["code"] != h["base"]


def _summary(path, sha, kernel="gemv_stream"):
    path.write_text(
        "# counter summary\n"
        f"kernel = {kernel}\n"
        f"gemv_source_sha256_16 = {sha}\n"
        "profiled_algorithmic_bytes_per_dispatch = 1000000\n"
        "gemv_FETCH_SIZE_KiB_per_dispatch = 500.0\n"
        "gemv_WRITE_SIZE_KiB_per_dispatch = 10.0\n"
        "copy_bytes_each_way = 1048576\n"
        "copy_FETCH_SIZE_KiB = 512.0\n"
        "copy_WRITE_SIZE_KiB = 1024.0\n")


def test_traffic_from_a_matching_summary(tmp_path, monkeypatch):
    src = _sources(tmp_path, ["int g() { return 0; }\n"])
    monkeypatch.setattr(bench, "GEMV_SOURCES", src)
    summ = tmp_path / "{kernel}_pmc.txt"
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(summ))
    _summary(tmp_path / "gemv_stream_pmc.txt", bench.gemv_source_hash())
    t, note = bench.pmc_traffic(2_000_000, "gemv_stream")
    # FETCH scaled x2 (1 MiB copy read as 512 KiB), WRITE x1: (1000 + 10) KiB
    # per 1 MB of algorithmic bytes, carried over to a 2 MB launch
    assert t == pytest.approx(2 * (1000 + 10) * 1024)
    assert "x2.000 / x1.000" in note


def test_traffic_null_when_the_code_changed_or_summary_missing(tmp_path, monkeypatch):
    src = _sources(tmp_path, ["int g() { return 0; }\n"])
    monkeypatch.setattr(bench, "GEMV_SOURCES", src)
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "{kernel}_pmc.txt"))
    _summary(tmp_path / "gemv_stream_pmc.txt", "0123456789abcdef")
    assert bench.pmc_traffic(1, "gemv_stream")[0] is None
    _summary(tmp_path / "gemv_stream_pmc.txt", bench.gemv_source_hash(), kernel="gemv_chain")
    assert bench.pmc_traffic(1, "gemv_stream")[0] is None
    assert bench.pmc_traffic(1, "gemv_mfma") == (None, "no counter summary")
