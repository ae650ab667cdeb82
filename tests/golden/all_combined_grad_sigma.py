"""Writes/checks workloads.ALL_COMBINED_GRAD_SIGMA with the fp64 oracle.

The all-combined workload accumulates into an existing bf16 gradient whose
entries are drawn from N(0, sigma^2); sigma is the rms of the fresh gradient
the oracle computes on a 64-row draw (seed 5000), so that the accumulated part
is of the same size as the existing one. Only oracle/ and the seeded
generator are called. Run: python tests/golden/all_combined_grad_sigma.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def sigma() -> float:
    w = workloads.WORKLOADS["all_combined_bf16"]
    inp = workloads.generate(w, "cpu", seed=5000, n_rows=64)
    x = inp["logits"].double().numpy()
    t = inp["teacher"].double().numpy()
    y = inp["labels"].numpy()
    spec = oracle.Spec(V=w.V, flags=w.flags & ~oracle.ACCUMULATE, w_ce=1.0, w_z=1e-4, w_distill=0.5,
                       w_grpo=1.0, grad_scale=1.0 / 32, temperature=w.temperature, eps=w.eps,
                       logit_scale=w.logit_scale, softcap=w.softcap)
    vals = oracle.row_values(spec, x, y)
    old = vals["logp"] + inp["old_noise"].double().numpy()
    _, _, _, g = oracle.rows_forward_backward(spec, x, float(w.N), y, None, t, old,
                                              inp["advantages"].double().numpy())
    return float(np.sqrt(np.mean(g * g)))


if __name__ == "__main__":
    s = sigma()
    print(f"rms of the fresh gradient: {s:.3e}  (stored: {workloads.ALL_COMBINED_GRAD_SIGMA:.3e})")
