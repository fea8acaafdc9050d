"""Host side of bench.py (no GPU): the CPU oracle baseline runs its worker
processes over a sampled set of heads and reports a throughput, and a
failure there is reported in the line instead of ending the run."""
import os
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from decode_kv_cache_head_amd import synth as S  # noqa: E402


def test_cpu_baseline_runs_worker_processes():
    w = S.workload("tiny")
    case = S.make_case(w, torch.device("cpu"))
    r = bench.cpu_baseline(case, w, 0.3, 2, every=1)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s"
    assert r["cores"] == 2          # two heads, one process each
    assert r["value"] > 0 and r["ms_per_step"] > 0
    # more processes than sampled heads: only those with a head are started
    r = bench.cpu_baseline(case, w, 0.2, 8, every=2)
    assert r["cores"] == 1 and r["value"] > 0


def test_cpu_baseline_failure_is_reported():
    w = S.workload("tiny")
    r = bench.cpu_baseline_or_error(None, w, 0.1, 2)
    assert r["kind"] == "oracle" and "error" in r


def test_kernel_bytes_fused_step_attention():
    # the step's attention launch reads only the dense window when the
    # compaction attended the sparse and condensed tiers
    import numpy as np
    w = S.workload("qwen8b_b1_16k")
    A = np.full((w.B, w.Hkv), w.T[0] - w.W, np.int64)
    k = A // 2
    fused = bench.kernel_bytes(w, A, k, "k_attn", True)
    unfused = bench.kernel_bytes(w, A, k, "k_attn", False)
    row = w.d * 2
    assert fused == 2 * w.W * row * w.B * w.Hkv + w.B * w.Hq * w.d * 2
    assert unfused > fused
