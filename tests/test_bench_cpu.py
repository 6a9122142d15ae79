"""Host logic of bench.py (no GPU): the digest that ties recorded HBM traffic to
the kernel sources, the traffic lookup, and the one-GPU rule."""
from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_only_drops_comments_and_layout():
    src = 'int a = 1; // note\n/* block\n comment */ float b = 2.0f;\nconst char* s = "x // y /* z */";\n'
    got = bench._code_only(src)
    assert "note" not in got and "block" not in got
    assert '"x // y /* z */"' in got                 # string literals kept whole
    assert bench._code_only("int   a\n\n=  1;") == "int a = 1;"
    assert bench._code_only("a = '/'; // c") == "a = '/';"


def test_digest_follows_code_not_comments(tmp_path, monkeypatch):
    csrc = tmp_path / "rejection_sampling_verify_softmax_amd" / "csrc"
    csrc.mkdir(parents=True)
    f = csrc / "k.hip"
    f.write_text("// kernel\n__global__ void k(int* p) { p[0] = 1; }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.source_digest()
    f.write_text("// kernel, reworded\n__global__ void k(int* p) {\n    p[0] = 1;   /* store */\n}\n")
    assert bench.source_digest() == d0
    f.write_text("// kernel\n__global__ void k(int* p) { p[0] = 2; }\n")
    assert bench.source_digest() != d0


def test_traffic_lookup_matches_kernel_workload_and_digest(tmp_path, monkeypatch):
    digest = bench.source_digest()
    t = tmp_path / "traffic.txt"
    t.write_text("# header\n"
                 f"kernel=k_a workload=w1 sources={digest} bytes_per_launch=123\n"
                 "kernel=k_a workload=w2 sources=0000000000000000 bytes_per_launch=456\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(t))
    assert bench.load_traffic("k_a", "w1") == 123.0
    assert bench.load_traffic("k_a", "w2") is None     # taken on other sources
    assert bench.load_traffic("k_b", "w1") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.load_traffic("k_a", "w1") is None


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
