"""Host-side checks of the benchmark (no GPU): the one-GPU guard, the
algorithmic byte count behind the roofline object, and the rule that stored
counter summaries apply only to the kernel sources they were taken on."""

import json
import os
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line for a configuration that was not measured


# Bytes per token written out by hand from the definition: each valid row
# reads its logits row (and teacher row) once and writes its gradient row
# once; accumulate mode also reads the old gradient; GSPO reads a valid row a
# second time; side inputs are the int64 label, the mask byte where the
# workload has a mask tensor, and fp32 old log-prob + advantage for policy losses.
HAND = {
    "ce_z_tiny_f32": 4 * 1024 + 4 * 1024 + 8,
    "ce_z_bf16": 2 * 128256 + 2 * 128256 + 8,
    "ce_z_f16": 2 * 128256 + 2 * 128256 + 8,
    "ce_fkl_bf16": 2 * 2 * 151936 + 2 * 151936 + 8,
    "ce_rkl_bf16": 2 * 2 * 151936 + 2 * 151936 + 8,
    "ce_fdce_bf16": 2 * 2 * 151936 + 2 * 151936 + 8,
    "ce_fkl_hinton_bf16": 2 * 2 * 151936 + 2 * 151936 + 8,
    "grpo_z_ent_bf16": 2 * 151936 + 2 * 151936 + 8 + 1 + 8,
    "ce_z_grpo_ent_bf16": 2 * 151936 + 2 * 151936 + 8 + 1 + 8,
    "gspo_z_ent_bf16": 2 * 2 * 151936 + 2 * 151936 + 8 + 1 + 8,
    "all_combined_bf16": 2 * 2 * 256000 + 2 * 2 * 256000 + 8 + 8,
}


@pytest.mark.parametrize("name", sorted(workloads.WORKLOADS))
def test_algorithmic_bytes_per_valid_token(name):
    w = workloads.WORKLOADS[name]
    assert name in HAND, "every benchmark workload needs its hand-computed byte count"
    assert workloads.algorithmic_bytes(w, n_valid_rows=w.N) == HAND[name] * w.N


def test_masked_rows_cost_their_gradient_write_only():
    w = workloads.WORKLOADS["grpo_z_ent_bf16"]
    row = 2 * w.V
    full = workloads.algorithmic_bytes(w, n_valid_rows=w.N)
    some_masked = workloads.algorithmic_bytes(w, n_valid_rows=w.N - 100)
    assert full - some_masked == 100 * row          # the read is skipped, the zero write stays
    acc = workloads.WORKLOADS["all_combined_bf16"]
    row = 2 * acc.V
    assert (workloads.algorithmic_bytes(acc, n_valid_rows=acc.N)
            - workloads.algorithmic_bytes(acc, n_valid_rows=acc.N - 10)) == 10 * 4 * row  # x, t, old grad, grad


def test_metrics_only_calls_read_each_valid_row_once():
    # no gradient: one read of each valid row's logits (and teacher), the side inputs;
    # GSPO without a gradient has no reloading backward, and accumulate mode no old-gradient read
    for name, tensors in (("grpo_z_ent_bf16", 1), ("gspo_z_ent_bf16", 1), ("ce_fkl_bf16", 2),
                          ("all_combined_bf16", 2)):
        w = workloads.WORKLOADS[name]
        row = 2 * w.V
        got = workloads.algorithmic_bytes(w, n_valid_rows=w.N - 7, with_grad=False)
        side = {"grpo_z_ent_bf16": 17, "gspo_z_ent_bf16": 17, "ce_fkl_bf16": 8, "all_combined_bf16": 16}[name]
        assert got == (w.N - 7) * tensors * row + w.N * side, name


def test_headline_launch_bytes_match_the_design_figure():
    # 16384 tokens, 5% of them masked in the generated batch: 15534 valid rows; the default
    # line runs the loss set the metric names on the GRPO configuration's inputs
    w = workloads.WORKLOADS[workloads.HEADLINE]
    assert w.name == "ce_z_grpo_ent_bf16"
    assert "+".join(bench.LOSS_NAMES[b] for b in bench.LOSS_NAMES if w.flags & b) == "CE+z+GRPO+entropy"
    assert workloads.seed_for(w.name) == workloads.seed_for("grpo_z_ent_bf16")
    assert workloads.algorithmic_bytes(w, n_valid_rows=15534) == 9699265024


def test_source_hash_is_stable_and_stored_traffic_needs_it():
    h = bench.source_hash()
    assert h == bench.source_hash() and len(h) == 16 and int(h, 16) >= 0
    w = workloads.WORKLOADS["grpo_z_ent_bf16"]
    assert bench.stored_traffic(w, "0" * 16) is None
    path = os.path.join(ROOT, "profiles", f"fused_kernel_{w.name}_pmc.json")
    with open(path) as f:
        stored = json.load(f)
    assert bench.stored_traffic(w, stored["src_hash"]) == stored["traffic_bytes_per_launch"]
