"""Host-side parts of bench.py (no GPU): the code hash that ties stored counter data to
a kernel source, the single-GPU refusal, and the algorithmic flop counts the roofline
objects divide by."""
from __future__ import annotations

import os
import subprocess
import sys
from types import SimpleNamespace

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_hash_ignores_comments_and_whitespace_only():
    src = "int f(int x) {\n  return x + 1;  // one more\n}\n/* note */\n"
    same = "int f(int x){return x+1;}\n// another note\n"
    other = "int f(int x) {\n  return x + 2;  // one more\n}\n"
    h = bench.kernel_source_hash("x.hip", src)
    assert h == bench.kernel_source_hash("x.hip", same)
    assert h != bench.kernel_source_hash("x.hip", other)


def test_code_hash_of_the_kernel_sources_is_stable():
    for name in ("prefill64.hip", "decode.hip"):
        a = bench.kernel_source_hash(name)
        assert a == bench.kernel_source_hash(name) and len(a) == 16


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_flops_per_token_of_the_workloads():
    # packed prefill, Hk = 16, Hv = 32, K = V = 128, C = 64:
    # Hk 4 C K + Hv (2 C K + 4 C V + 6 K V)
    gdn = SimpleNamespace(shape=(1, 36112, 16, 32, 128, 128), num_householder=1)
    assert bench.prefill_flops_per_token(gdn, 64) == 16 * 4 * 64 * 128 + 32 * (
        2 * 64 * 128 + 4 * 64 * 128 + 6 * 128 * 128) == 5242880
    # gated delta product, n_h = 2, H = 32, K = V = 128, C = 128 tokens:
    # Hv ((4 n_h + 2) K V + 2 n_h^2 C (2 K + V) + 2 n_h C (K + V))
    gdp = SimpleNamespace(shape=(1, 65536, 32, 32, 128, 128), num_householder=2)
    assert bench.prefill_flops_per_token(gdp, 128) == 32 * (
        10 * 128 * 128 + 8 * 128 * 384 + 4 * 128 * 256) == 22020096
