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
# Scalar gates. A slot is a mean of per-row values, so its error is measured
# against the larger of |mean| and the mean |per-row value| (the scale of
# the sum); TOTAL against the weighted sum of its terms' scales. Slots whose
# exact value can be 0 in an ordinary batch (a KL against an identical
# distribution, a policy loss or statistic with zero advantages or ratio 1,
# a mean of signed advantages) also take NEAR_ZERO_FLOOR as the scale's
# lower bound: an absolute error of rel * 1e-2 is allowed where the exact
# value is 0.
ROW_KEY = {"CE": "ce", "Z": "z", "DISTILL": "distill", "GRPO": "grpo", "NEWLOGP": "logp", "RATIO": "ratio",
           "KL_OLD_NEW": "k3", "ADV_MEAN": "adv", "ENTROPY": "entropy"}
ZERO_CAPABLE = ("DISTILL", "GRPO", "KL_OLD_NEW", "ADV_MEAN")
NEAR_ZERO_FLOOR = 1e-2
# per-row value columns whose values can be exactly 0 (the same reading, row by row)
ZERO_CAPABLE_ROWS = ("fkl", "rkl", "fdce", "grpo", "k3", "adv")


def row_value_scale(key, ref):
    """Scale of each per-row value of column `key` (ref: the oracle's values of
    the valid rows): max(|value|, 1e-2 * mean |value| of the column), and the
    near-zero floor for columns whose values can be exactly 0."""
    ref = np.asarray(ref, dtype=np.float64)
    col = 1e-2 * float(np.mean(np.abs(ref))) if ref.size else 0.0
    sc = np.maximum(np.abs(ref), col)
    if key in ZERO_CAPABLE_ROWS:
        sc = np.maximum(sc, NEAR_ZERO_FLOOR)
    return sc


def degenerate_allowance(spec, x, dtype="bf16") -> float:
    """Rows of one element (V = 1) in the 16-bit instances, a reading: the
    exact CE, new log-prob and every KL are 0 there, while those instances
    form them from fp32 statistics of magnitude S = max |s| (with a softcap
    c, max(max |s|, c)); a slot is accepted within 4 ulps of S times (1 + the
    weight sum). 0 for V > 1 and for fp32 inputs, whose instances form the
    statistics and coefficients in fp64 (measured: gradient errors below
    5e-10 on those rows), so the plain gates hold."""
    if spec.V != 1 or dtype == "f32" or x is None or np.size(x) == 0:
        return 0.0
    x = np.asarray(x, dtype=np.float64)
    s = spec.softcap * np.tanh(spec.logit_scale * x / spec.softcap) if spec.softcap > 0 else spec.logit_scale * x
    S = max(float(np.max(np.abs(s))), spec.softcap)
    wsum = 1.0 + abs(spec.w_ce) + abs(spec.w_z) + abs(spec.w_distill) + abs(spec.w_grpo)
    return 4 * 2.0 ** -23 * S * wsum


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def _f32(v) -> float:
    return float(np.float32(v))


def spec_from(V, flags, w=None, **kw) -> oracle.Spec:
    """The oracle's Spec for a plan. The C ABI takes every hyper-parameter
    (weights, scale, divisor, temperature, eps, logit scale, softcap) as fp32,
    so the plan holds their fp32 roundings; the oracle is evaluated at those
    same values (at the unrounded ones a weight of 1.44 alone moves an fp32
    gradient entry of magnitude 8 by 1.3e-6)."""
    w = w or {}
    return oracle.Spec(V=V, flags=flags, w_ce=_f32(w.get("ce", 1.0)), w_z=_f32(w.get("z", 0.0)),
                       w_distill=_f32(w.get("distill", 0.0)), w_grpo=_f32(w.get("grpo", 0.0)),
                       grad_scale=_f32(w.get("grad_scale", 1.0)), divisor=_f32(w.get("divisor", 0.0)),
                       temperature=_f32(kw.get("temperature", 1.0)), eps=_f32(kw.get("eps", 0.2)),
                       logit_scale=_f32(kw.get("logit_scale", 1.0)), softcap=_f32(kw.get("softcap", 0.0)))


def max_chunks(dtype: str, spec: oracle.Spec) -> int:
    """Chunks per row the split-vocab exchange allows (the documented rule of
    hl_plan_set_chunks): one wave polls every exchanged word of a row, at most
    64, and a chunk exchanges 3 statistics student-only, 6 with a teacher,
    one more for FDCE and one more for Hinton; fp32 plans also exchange the
    low parts of their one to three normalizers. Never more than 9."""
    teacher = bool(spec.flags & (oracle.FKL | oracle.RKL | oracle.FDCE))
    hinton = teacher and spec.has(oracle.HINTON)
    words = 3 if not teacher else 6 + int(spec.has(oracle.FDCE)) + int(hinton)
    if dtype == "f32":
        words += 1 if not teacher else (3 if hinton else 2)
    return min(9, 64 // words)


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
    """Relative error per slot, measured against the slot's scale (see above)."""
    scale = {}
    for name in oracle.SLOTS:
        sc = abs(ref[SLOT[name]])
        key = ROW_KEY.get(name)
        if key == "distill" and vals is not None:
            key = "fkl" if spec.has(oracle.FKL) else ("rkl" if spec.has(oracle.RKL) else "fdce")
        if vals is not None and valid is not None and key in (vals or {}) and valid.any():
            sc = max(sc, float(np.mean(np.abs(np.asarray(vals[key])[valid]))))
        scale[name] = sc
    scale["TOTAL"] = max(abs(ref[SLOT["TOTAL"]]), abs(spec.w_ce) * scale["CE"] + abs(spec.w_z) * scale["Z"]
                         + abs(spec.w_distill) * scale["DISTILL"] + abs(spec.w_grpo) * scale["GRPO"])
    for name in ZERO_CAPABLE:
        scale[name] = max(scale[name], NEAR_ZERO_FLOOR)
    errs = {}
    for name in oracle.SLOTS:
        i = SLOT[name]
        d = abs(got[i] - ref[i])
        errs[name] = d / scale[name] if scale[name] > 0 else d
    return errs


def assert_scalars(spec, got, ref, dtype, vals=None, valid=None, skip=(), x=None):
    """Scalar slots within the dtype's relative gate; with one-element rows
    (V = 1) also within degenerate_allowance(spec, x) absolute."""
    rel = TOL[dtype]["scalar_rel"]
    errs = scalar_errors(spec, got, ref, vals, valid)
    allow = degenerate_allowance(spec, x, dtype)
    for name in ("N_VALID", "N_BADLABEL"):
        assert got[SLOT[name]] == ref[SLOT[name]], (name, got[SLOT[name]], ref[SLOT[name]])
    bad = {k: v for k, v in errs.items()
           if v > rel and k not in ("N_VALID", "N_BADLABEL") and k not in skip
           and not abs(got[SLOT[k]] - ref[SLOT[k]]) <= allow}
    assert not bad, f"scalar errors above {rel}: {bad}\n got={got}\n ref={ref}"


def grad_check(got, ref, dtype, labels=None, valid=None, base=None):
    """Compare a gradient tensor with the oracle's. Returns a dict of metrics."""
    g = to_np(got)
    r = ref
    out = {}
    if dtype == "f32":
        d = np.abs(g - r)
        out["max_abs"] = float(np.max(d)) if g.size else 0.0
        out["max_ref"] = float(np.max(np.abs(r))) if r.size else 0.0
        assert out["max_abs"] <= TOL["f32"]["grad_abs"], out
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
