"""Host-side parts of bench.py: the one-GPU refusal, the kernel source hash
that ties committed counters to the kernels they were taken on, and the
lookup of those counters."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_without_touching_a_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_source_hash_ignores_comments_only():
    code = "int f(int x) { return x + 1; }"
    commented = "/* header\n comment */\nint f(int x) {  // the successor\n  return x + 1;\n}\n"
    changed = "int f(int x) { return x + 2; }"
    assert bench._code_only(code) == bench._code_only(commented)
    assert bench._code_only(code) != bench._code_only(changed)
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()


def test_counter_traffic_requires_the_current_sources(tmp_path, monkeypatch):
    rec = {"w": {"encode": {"hbm_bytes_per_launch": 123.0, "source_hash": bench.kernel_source_hash()},
                 "decode": {"hbm_bytes_per_launch": 456.0, "source_hash": "0" * 16}}}
    (tmp_path / "counters.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.counter_traffic("w", "encode") == 123.0
    assert bench.counter_traffic("w", "decode") is None      # taken on other kernel sources
    assert bench.counter_traffic("other", "encode") is None


def test_committed_counters_cover_every_bench_workload():
    with open(os.path.join(ROOT, "profiles", "counters.json")) as f:
        rec = json.load(f)
    for w in ("llama3_8b_4k", "llama3_8b_32k", "llama3_70b_16k", "qwen7b_paged"):
        for op in ("encode", "decode"):
            assert rec[w][op]["hbm_bytes_per_launch"] > 0


def test_pool_block_list_order():
    """The yardstick's block list: every block a paged call reads, slab by
    slab, request by request, block by block, as indices into L * 2 * NB."""
    import numpy as np
    from kv_cache_compression_kvc_amd import presets
    p = presets.preset("qwen7b_paged").with_(layers=2, block_size=16)
    table = np.array([[5, 1, 9, -1], [2, -1, -1, -1], [7, 8, 0, 3]], dtype=np.int32)
    lens = np.array([33, 0, 64], dtype=np.int32)
    got = bench.pool_block_list(p, table, lens, 10)
    one = [5, 1, 9, 7, 8, 0, 3]
    want = [s * 10 + b for s in range(4) for b in one]
    assert got.dtype == np.int32 and got.tolist() == want
