"""Host-side checks of bench.py (CPU only): the multi-GPU refusal and the
algorithmic byte count of the benchmark workload, recomputed from its
definition (every valid token's K row, V row and k_scale per KV head; v_scale;
Q, q_scale and the bf16 output per query row; the table entries and lengths)."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import torch

from fp8_paged_kv_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_algorithmic_bytes_of_the_benchmark_workload():
    cfg = synth.CONFIGS[1]
    inp = synth.make_gqa_inputs(cfg)
    seqs = inp["kv_act_seqs"].tolist()
    tokens = sum(seqs)
    per_token = cfg.nkv * (cfg.D + cfg.D + 4)                 # K row, V row (FP8) and k_scale, per KV head
    v_scale = cfg.B * cfg.nkv * cfg.D * 4
    queries = cfg.B * cfg.s1 * cfg.nq * (cfg.D * 2 + 4 + cfg.D * 2)   # bf16 q, q_scale, bf16 out
    table = 4 * sum((s + 127) // 128 for s in seqs) + 4 * cfg.B
    want = tokens * per_token + v_scale + queries + table
    assert synth.gqa_algorithmic_bytes(cfg, seqs) == want
    # the K / V / k_scale part equals the bytes of those tensors the valid tokens occupy
    k_rows = int(torch.tensor(seqs).sum()) * cfg.nkv * cfg.D
    assert tokens * per_token == 2 * k_rows + 4 * tokens * cfg.nkv


def test_cpu_baseline_fields_on_the_small_workload():
    """The oracle leg as bench.py reports it, on the small two-sequence workload:
    a multi-thread figure over a bounded sample and the single-thread one."""
    sys.path.insert(0, ROOT)
    import bench
    cfg = synth.CONFIGS[0]
    inp = synth.make_gqa_inputs(cfg)
    seqs = inp["kv_act_seqs"].tolist()
    r = bench.cpu_baseline(cfg, inp, seqs, target_s=5.0)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0
    assert 1 <= r["cores"] <= 16
    assert "sequences 0..1 of 2" in r["sample"]                       # both sequences fit the budget
    st = r["single_thread"]
    assert st["value"] > 0 and "1 thread" in st["sample"] and f"{seqs[0]} tokens" in st["sample"]
