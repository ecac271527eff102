"""Host-side checks of the benchmark's own arithmetic and contract (CPU only)."""
import os
import subprocess
import sys

import numpy as np

import bench
import workload as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _pairs_by_enumeration(q, kv):
    """Visible (row, key) pairs of a bottom-right causal prefill, counted row by row."""
    return sum(kv - q + i + 1 for i in range(q))


def test_prefill_flops_match_visible_pairs():
    for name in ("tiny", "tail128", "tail16", "full8k", "full16k", "full32k"):
        w = W.get(name)
        pairs = sum(_pairs_by_enumeration(q, kv) for q, kv in zip(w.q_lens, w.kv_lens))
        assert bench.prefill_flops(w.q_lens, w.kv_lens, w.num_qo_heads) == 4 * 128 * w.num_qo_heads * pairs
    # the 16K causal prefill: 134,225,920 visible pairs per head, 2.199 TFLOP in all
    w = W.get("full16k")
    assert _pairs_by_enumeration(16384, 16384) == 134_225_920
    assert abs(bench.prefill_flops(w.q_lens, w.kv_lens, 32) - 2.199e12) < 1e9


def test_cache_bytes_per_token_and_head():
    # NVFP4: 64 packed bytes + 8 scale bytes for each of K and V; FP8: 128 + 128
    assert bench.KV_BYTES == {"nvfp4": 2 * (64 + 8), "fp8": 2 * 128}


def test_source_hash_ignores_commentary_only(tmp_path, monkeypatch):
    csrc = tmp_path / "attention_nvfp4_quantized_amd" / "csrc"
    csrc.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (csrc / "k.hip").write_text("// header\nint f(int x) { return x + 1; }  /* note */\n")
    h0 = bench.source_hash(["k.hip"])
    (csrc / "k.hip").write_text("// another header\n\nint f(int x) {\n  return x + 1;  // same code\n}\n")
    assert bench.source_hash(["k.hip"]) == h0
    (csrc / "k.hip").write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_hash(["k.hip"]) != h0


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
