"""Host-side logic of bench.py (no GPU): the one-GPU rule, and the rule that a committed traffic
summary counts only while the sources its kernel is built and planned from are unchanged."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr + r.stdout


def test_sources_per_workload():
    assert bench.kernel_sources("decode-8b")[0] == "decode.hip"
    assert bench.kernel_sources("shared-prefix-grouped")[0] == "decode.hip"
    assert bench.kernel_sources("prefill-chunk")[0] == "prefill.hip"
    assert bench.kernel_sources("block-copy")[0] == "blocks.hip"
    for w in ("decode-8b", "prefill-chunk", "block-copy"):
        assert "api.cpp" in bench.kernel_sources(w)
    assert "lds_tile.hpp" in bench.kernel_sources("prefill-chunk")
    assert "lds_tile.hpp" in bench.kernel_sources("decode-8b")
    assert bench.kernel_sources_sha("decode-8b") != bench.kernel_sources_sha("prefill-chunk")


def test_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    csrc = tmp_path / "paged_kv_cache_190_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("decode.hip", "common.hpp", "lds_tile.hpp", "launch.hpp", "api.cpp"):
        (csrc / f).write_text("int f(int x) { return x + 1; }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_sources_sha("decode-8b")
    (csrc / "decode.hip").write_text("// a comment\nint f(int x)   {\n  return x + 1; /* note */ }\n")
    assert bench.kernel_sources_sha("decode-8b") == h0
    (csrc / "api.cpp").write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_sources_sha("decode-8b") != h0


def test_traffic_counts_only_on_matching_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "paged_kv_cache_190_amd" / "csrc"
    csrc.mkdir(parents=True)
    prof = tmp_path / "profiles"
    prof.mkdir()
    for f in ("decode.hip", "common.hpp", "lds_tile.hpp", "launch.hpp", "api.cpp"):
        (csrc / f).write_text("int f(int x) { return x; }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.kernel_sources_sha("decode-8b")
    (prof / "traffic_decode-8b.md").write_text(
        f"traffic_bytes_per_launch: 6.4e+08\nkernel_sources_sha256: {sha}\n")
    assert bench.traffic_from_profile("decode-8b", 6.3e8) == 6.4e8
    assert bench.traffic_from_profile("decode-70b", 1e9) is None  # no summary for it
    (csrc / "decode.hip").write_text("int f(int x) { return x * 2; }\n")
    assert bench.traffic_from_profile("decode-8b", 6.3e8) is None

