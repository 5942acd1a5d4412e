"""bench.py without a GPU: the multi-GPU refusal, and the rule that HBM traffic
figures are reported only when they were measured on the current kernel
sources."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "counters.json").write_text(json.dumps({
        "gqa_ring": {"csrc_hash": "aaaa", "bytes_per_launch": 123},
        "decode": {"csrc_hash": "bbbb", "bytes_per_launch": 456}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "csrc_hash", lambda workload=None: "aaaa")
    assert bench.load_traffic("gqa_ring") == 123
    assert bench.load_traffic("decode") is None          # taken on other sources
    assert bench.load_traffic("jagged") is None          # never measured


def test_source_hash_covers_every_kernel_file():
    h = bench.csrc_hash()
    assert len(h) == 16 and h == bench.csrc_hash()
    srcs = sorted(os.listdir(os.path.join(ROOT, "flash_attention_kv_amd", "csrc")))
    assert any(s.endswith(".hip") for s in srcs) and "fakv_device.h" in srcs


def test_counter_hash_follows_only_that_kernels_sources():
    d = os.path.join(ROOT, "flash_attention_kv_amd", "csrc")
    srcs = set(os.listdir(d))
    for w, fam in bench._WORKLOAD_FAMILY.items():
        files = bench._SHARED_SOURCES + bench._FAMILY_SOURCES[fam]
        assert set(files) <= srcs, w
        assert len(bench.csrc_hash(w)) == 16
    # the fp32 prefill is no part of the bf16 or decode counter entries
    assert all("prefill_f32.hip" not in f for f in bench._FAMILY_SOURCES.values())
    assert bench.csrc_hash("gqa_ring") == bench.csrc_hash("jagged") != bench.csrc_hash("decode")
    assert bench.csrc_hash("ring_tiny") == ""


def test_counter_hash_ignores_comments_and_layout(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one more\n}\n")
    b.write_text("/* the successor */\nint f(int x) { return x + 1; }\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench._code_text(str(a)) == bench._code_text(str(b))
    assert bench._code_text(str(a)) != bench._code_text(str(c))


def test_counter_hash_covers_build_flags():
    flags = bench._build_flags().decode()
    assert "FILE_FLAGS" in flags and "prefill_bf16_jagged.hip" in flags and "sched-strategy" in flags
    assert "/root" not in flags and "os.path" not in flags     # no machine-specific paths
