"""Helpers for the GPU parity tests: run the HIP path, run the oracle on the
same stored inputs, compare at the tolerances the tests state."""

from __future__ import annotations

import sys

import numpy as np
import torch

import lm_head_vocab_amd as hl
import oracle
from oracle import SLOT

# Tolerances. fp32: scalars 1e-5 relative, gradient 1e-6 absolute. bf16:
# scalars 1e-4 relative, gradient rms-relative 4e-3 over the tensor and over
# its non-label entries alone (the label column carries most of the norm).
TOL = {
    "f32": dict(scalar_rel=1e-5, grad_abs=1e-6),
    "bf16": dict(scalar_rel=1e-4, grad_rms=4e-3),
    # fp16 (not among the stated tolerances): one fp16 rounding of the output is
    # at most 2^-11 = 4.9e-4 relative, so 1e-3 rms-relative; scalars as bf16.
    "f16": dict(scalar_rel=1e-4, grad_rms=1e-3),
}
# Slots whose batch mean can sit at or near zero (a KL against an identical or
# one-element distribution, a mean of signed advantages) are measured against
# max(|ref|, mean |per-row value|, NEAR_ZERO_FLOOR): an absolute error of
# rel * 1e-2 is allowed where the exact value is 0.
NEAR_ZERO_SLOTS = {"GRPO": "grpo", "ADV_MEAN": "adv", "KL_OLD_NEW": "k3", "DISTILL": "distill",
                   "NEWLOGP": "logp", "TOTAL": None}
NEAR_ZERO_FLOOR = 1e-2


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def spec_from(V, flags, w=None, **kw) -> oracle.Spec:
    w = w or {}
    return oracle.Spec(V=V, flags=flags, w_ce=w.get("ce", 1.0), w_z=w.get("z", 0.0),
                       w_distill=w.get("distill", 0.0), w_grpo=w.get("grpo", 0.0),
                       grad_scale=w.get("grad_scale", 1.0), divisor=w.get("divisor", 0.0),
                       temperature=kw.get("temperature", 1.0), eps=kw.get("eps", 0.2),
                       logit_scale=kw.get("logit_scale", 1.0), softcap=kw.get("softcap", 0.0))


def make_plan(spec: oracle.Spec, dtype, chunks: int = 0) -> hl.Plan:
    return hl.Plan(spec.V, dtype, spec.flags, ce=spec.w_ce, z=spec.w_z, distill=spec.w_distill,
                   grpo=spec.w_grpo, grad_scale=spec.grad_scale, divisor=spec.divisor,
                   temperature=spec.temperature, eps=spec.eps, logit_scale=spec.logit_scale,
                   softcap=spec.softcap, chunks=chunks)


def oracle_old_logprobs(spec, logits, labels, noise):
    """old = exact label log-prob (fp64 oracle) + noise, rounded to fp32."""
    vals = oracle.row_values(spec, to_np(logits), to_np(labels).astype(np.int64))
    old = vals["logp"] + to_np(noise)
    return torch.tensor(old, dtype=torch.float32)


def torch_old_logprobs(spec, logits, labels, noise, chunk=512):
    """old = label log-prob + noise for large batches, computed with torch in
    fp32 on the device (input synthesis only)."""
    N = logits.shape[0]
    out = torch.empty(N, dtype=torch.float32, device=logits.device)
    y = labels.clamp(min=0)
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        x = logits[r0:r1].float()
        s = spec.softcap * torch.tanh(x * (spec.logit_scale / spec.softcap)) if spec.softcap > 0 \
            else x * spec.logit_scale
        lp = torch.log_softmax(s, dim=1).gather(1, y[r0:r1, None])[:, 0]
        out[r0:r1] = lp
    return out + noise


def run_hip(plan, inputs, grad_mode="overwrite"):
    """grad_mode: 'overwrite' (fresh buffer), 'accumulate' (clone of grad_init),
    'none' (forward only)."""
    x = inputs["logits"]
    grad = None
    if grad_mode == "overwrite":
        grad = torch.full_like(x, float("nan"))
    elif grad_mode == "accumulate":
        grad = inputs["grad_init"].clone()
    sc = plan(x, labels=inputs.get("labels"), mask=inputs.get("mask"),
              teacher=inputs.get("teacher"), old_logprobs=inputs.get("old_logprobs"),
              advantages=inputs.get("advantages"), grad=grad)
    torch.cuda.synchronize()
    return sc.cpu().double().numpy(), grad


def run_oracle(spec, inputs, rows=None, n=None, want_grad=True):
    """Oracle on all rows (rows=None) or on a row subset with the batch divisor n."""
    def sel(key, as_int=False):
        t = inputs.get(key)
        if t is None:
            return None
        if rows is not None:
            t = t[rows]
        arr = to_np(t)
        return arr.astype(np.int64) if as_int else arr
    x = sel("logits")
    labels = sel("labels", as_int=True)
    mask = sel("mask")
    args = dict(labels=labels, mask=mask, teacher=sel("teacher"),
                old_logprobs=sel("old_logprobs"), advantages=sel("advantages"),
                grad_in=sel("grad_init") if spec.has(oracle.ACCUMULATE) else None,
                want_grad=want_grad)
    if rows is None:
        sc, g = oracle.forward_backward(spec, x, **args)
        return sc, g, None
    vals, valid, bad, g = oracle.rows_forward_backward(spec, x, n, **args)
    return None, g, (vals, valid, bad)


def scalar_errors(spec, got, ref, vals=None, valid=None):
    """Relative error per slot with the near-zero reading for mean slots."""
    errs = {}
    for name in oracle.SLOTS:
        i = SLOT[name]
        r, g = ref[i], got[i]
        denom = abs(r)
        key = NEAR_ZERO_SLOTS.get(name, "missing")
        if key == "distill" and vals is not None:
            key = "fkl" if spec.has(oracle.FKL) else ("rkl" if spec.has(oracle.RKL) else "fdce")
        if vals is not None and valid is not None and key not in (None, "missing") and key in vals:
            denom = max(denom, float(np.mean(np.abs(vals[key][valid]))) if valid.any() else 0.0)
        if key != "missing":
            denom = max(denom, NEAR_ZERO_FLOOR)
        errs[name] = abs(g - r) / denom if denom > 0 else abs(g - r)
    return errs


def assert_scalars(spec, got, ref, dtype, vals=None, valid=None, skip=()):
    rel = TOL[dtype]["scalar_rel"]
    errs = scalar_errors(spec, got, ref, vals, valid)
    for name in ("N_VALID", "N_BADLABEL"):
        assert got[SLOT[name]] == ref[SLOT[name]], (name, got[SLOT[name]], ref[SLOT[name]])
    bad = {k: v for k, v in errs.items() if v > rel and k not in ("N_VALID", "N_BADLABEL") and k not in skip}
    assert not bad, f"scalar errors above {rel}: {bad}\n got={got}\n ref={ref}"


def grad_check(got, ref, dtype, labels=None, valid=None, base=None, f32_abs=None):
    """Compare a gradient tensor with the oracle's. Returns a dict of metrics.
    ``f32_abs`` replaces the fp32 absolute gate where a test states why."""
    g = to_np(got)
    r = ref
    out = {}
    if dtype == "f32":
        out["max_abs"] = float(np.max(np.abs(g - r))) if g.size else 0.0
        assert out["max_abs"] <= (f32_abs or TOL["f32"]["grad_abs"]), out
        return out
    diff = g - r
    den = np.sqrt(np.mean(r * r)) if r.size else 0.0
    out["rms_rel"] = float(np.sqrt(np.mean(diff * diff)) / den) if den > 0 else float(np.sqrt(np.mean(diff * diff)))
    if labels is not None and r.size:
        y = np.asarray(labels).astype(np.int64)
        nonlab = np.ones_like(r, dtype=bool)
        rows = np.arange(r.shape[0])
        ok = (y >= 0) & (y < r.shape[1])
        nonlab[rows[ok], y[ok]] = False
        d2 = diff[nonlab]
        r2 = r[nonlab]
        den2 = np.sqrt(np.mean(r2 * r2)) if r2.size else 0.0
        if den2 > 0:
            out["rms_rel_nonlabel"] = float(np.sqrt(np.mean(d2 * d2)) / den2)
    tol = TOL[dtype]["grad_rms"]
    assert out["rms_rel"] <= tol, out
    assert out.get("rms_rel_nonlabel", 0.0) <= tol, out
    return out
