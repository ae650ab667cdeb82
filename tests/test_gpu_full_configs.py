"""Full-batch parity at the benchmark configurations: every row of the batch
through the fp64 oracle, in the launch configuration the benchmark times.

For each configuration the inputs are drawn on the device (as bench.py draws
them), one call runs through the C ABI with the plan's automatic variant, and
the rows stream device -> host in blocks of 1024 to 16 host threads that run
the oracle on 64 rows at a time (``oracle.rows_forward_backward`` with the
batch divisor). Compared:

* the 13 batch scalars against the oracle's, assembled from its per-row
  values over the whole batch (``oracle.scalars_from_rows``), at the scalar
  gates of the other parity tests;
* every valid row's per-row values (CE, z, distillation KL, new log-prob,
  ratio, GRPO objective, k3, advantage, entropy; with GSPO the segment values
  the row belongs to) against the oracle's, each within the scalar tolerance
  of max(|value|, 1e-2 * mean |value| of its column), with the scalar gates'
  near-zero floor (1e-2) for the columns whose values can be exactly 0 (KL,
  policy objective, k3, advantage); the clip flags exactly;
* the gradient: rms-relative error over the whole tensor and over its
  non-label entries (bf16 4e-3, fp16 1e-3; fp32 1e-6 absolute per entry),
  and every masked row +0.0 (overwrite) or untouched (accumulate).

Rows whose GRPO ratio (or GSPO segment ratio) lies within 1e-5 of 1 +/- eps
may take either clip branch; they are left out of the gradient and clip-flag
comparisons. The all-combined configuration (32768 x 256000, with teacher)
checks the scalars and the per-row values on every row and the gradient on a
stratified sample of 1024 rows (every 32nd row, so every XCD group and every
1024-token sequence is represented): its full gradient through the oracle
would take several minutes of host time. GSPO checks all 32 segments: the
oracle's segment step needs every row's new log-prob first, so its rows go
through the oracle twice (values, then gradient with the segment
coefficients).
"""

from __future__ import annotations

import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import TOL, assert_scalars, row_value_scale, say, spec_from, to_np, torch_old_logprobs
from oracle import SLOT

import lm_head_vocab_amd as hl

pytestmark = pytest.mark.gpu
DEV = "cuda"
BLOCK_ROWS = 1024         # rows per device -> host transfer
TASK_ROWS = 64            # rows per oracle task
THREADS = max(1, min(16, os.cpu_count() or 1))
INT_VIEW = {"f32": torch.int32, "bf16": torch.int16, "f16": torch.int16}
ROW_KEYS = ("ce", "z", "fkl", "rkl", "fdce", "grpo", "logp", "ratio", "clipped", "k3", "adv", "entropy")
# per-row value columns of hl_row_values, by oracle key
COLS = {"ce": 0, "z": 1, "distill": 2, "grpo": 3, "logp": 4, "ratio": 5, "k3": 7, "adv": 8, "entropy": 9}


def _spec(w):
    return spec_from(w.V, w.flags, dict(ce=w.weights.get("ce", 1.0),
                                        **{k: v for k, v in w.weights.items() if k != "ce"}),
                     temperature=w.temperature, eps=w.eps, logit_scale=w.logit_scale, softcap=w.softcap)


def _host_block(inp, r0, r1):
    """Rows [r0, r1) of every per-row input, as host tensors (logits in their own dtype)."""
    out = {}
    for k in ("logits", "teacher", "labels", "mask", "old_logprobs", "advantages", "grad_init"):
        t = inp.get(k)
        out[k] = None if t is None else t[r0:r1].cpu()
    return out


def _np(t, rows=None, f64=True):
    if t is None:
        return None
    if rows is not None:
        t = t[rows]
    return t.to(torch.float64).numpy() if f64 else t.numpy()


def _oracle_task(spec, n, blk, rows, want_grad, grad_gpu=None, gspo_dlogp=None, skip_rows=None):
    """Oracle on the rows `rows` (indices into the block). Returns per-row
    values (1-D arrays), validity, bad-label flags and, with a gradient, the
    sums of the squared error and squared reference over all entries and over
    the non-label entries (rows in skip_rows left out), or the max abs error."""
    x = _np(blk["logits"], rows)
    y = _np(blk["labels"], rows, f64=False).astype(np.int64)
    grad_in = _np(blk["grad_init"], rows) if spec.has(oracle.ACCUMULATE) else None
    vals, valid, bad, ref_g = oracle.rows_forward_backward(
        spec, x, n, labels=y, mask=_np(blk["mask"], rows, f64=False),
        teacher=_np(blk["teacher"], rows), old_logprobs=_np(blk["old_logprobs"], rows),
        advantages=_np(blk["advantages"], rows), grad_in=grad_in, want_grad=want_grad, gspo_dlogp=gspo_dlogp)
    out = {"vals": {k: np.asarray(vals[k]).reshape(-1).copy() for k in ROW_KEYS if k in vals},
           "valid": valid, "bad": bad}
    if want_grad:
        g = grad_gpu[rows].to(torch.float64).numpy()
        keep = np.ones(len(y), dtype=bool) if skip_rows is None else ~skip_rows
        d = (g - ref_g)[keep]
        r = ref_g[keep]
        lab = np.zeros_like(r, dtype=bool)
        yk = y[keep]
        ok = (yk >= 0) & (yk < spec.V)
        lab[np.arange(len(yk))[ok], yk[ok]] = True
        out["sums"] = (float(np.sum(d * d)), float(np.sum(r * r)),
                       float(np.sum(d[~lab] ** 2)), float(np.sum(r[~lab] ** 2)),
                       float(np.max(np.abs(d))) if d.size else 0.0, int(keep.sum()))
    return out


def _run(name):
    w = workloads.WORKLOADS[name]
    spec = _spec(w)
    say(f"[gpu] full parity {name}: N={w.N} V={w.V} {w.dtype} seed={workloads.seed_for(name)}")
    inp = workloads.generate(w, DEV)
    if w.flags & (workloads.GRPO | workloads.GSPO):
        inp["old_logprobs"] = torch_old_logprobs(spec, inp["logits"], inp["labels"], inp["old_noise"])
    plan = hl.Plan(w.V, w.torch_dtype, w.flags, ce=spec.w_ce, z=spec.w_z, distill=spec.w_distill,
                   grpo=spec.w_grpo, grad_scale=spec.grad_scale, divisor=spec.divisor,
                   temperature=spec.temperature, eps=spec.eps, logit_scale=spec.logit_scale, softcap=spec.softcap)
    acc = bool(w.flags & workloads.ACCUMULATE)
    grad = inp["grad_init"].clone() if acc else torch.full_like(inp["logits"], float("nan"))
    sc = plan(inp["logits"], labels=inp["labels"], mask=inp["mask"], teacher=inp["teacher"],
              old_logprobs=inp.get("old_logprobs"), advantages=inp["advantages"], grad=grad,
              seq_offsets=inp["seq_offsets"])
    torch.cuda.synchronize()
    sc = sc.cpu().double().numpy()
    rv = plan.row_values().cpu().double().numpy()
    say(f"[gpu] {name}: call done, plan={plan.describe()}")
    return w, spec, inp, plan, grad, sc, rv


def _check_rows_and_scalars(w, spec, sc, rv, vals, valid, bad, n, seam=None, boundary=None):
    dt = w.dtype
    tol = TOL[dt]["scalar_rel"]
    ref_sc = oracle.scalars_from_rows(spec, vals, valid, bad, n, seam)
    assert sc[SLOT["N_VALID"]] == ref_sc[SLOT["N_VALID"]] and sc[SLOT["N_BADLABEL"]] == ref_sc[SLOT["N_BADLABEL"]]
    scalar_vals = dict(vals)
    if seam is not None:
        seg = seam["segment"]
        scalar_vals.update(grpo=seam["loss"][seg], adv=seam["adv"][seg], k3=seam["k3"][seg],
                           ratio=seam["ratio"][seg])
    skip = ("CLIPFRAC",) if boundary is not None and boundary.any() else ()
    assert_scalars(spec, sc, ref_sc, dt, scalar_vals, valid, skip=skip)
    if not skip and (spec.has(oracle.GRPO) or spec.has(oracle.GSPO)):
        cnt = seam["n_seg"] if seam is not None else n
        assert round(sc[SLOT["CLIPFRAC"]] * cnt) == round(ref_sc[SLOT["CLIPFRAC"]] * cnt)
    # every valid row's per-row values
    checks = [("ce", "ce"), ("z", "z"), ("entropy", "entropy"), ("logp", "logp")]
    kl = "fkl" if spec.has(oracle.FKL) else "rkl" if spec.has(oracle.RKL) else "fdce" if spec.has(oracle.FDCE) else None
    if kl:
        checks.append((kl, "distill"))
    policy = spec.has(oracle.GRPO) or spec.has(oracle.GSPO)
    if policy:
        checks += [("grpo", "grpo"), ("ratio", "ratio"), ("k3", "k3"), ("adv", "adv")]
    worst = {}
    for key, col in checks:
        if key in ("ce", "logp") and not (spec.has(oracle.CE) or policy):
            continue
        if key == "entropy" and not spec.has(oracle.ENTROPY):
            continue
        ref = scalar_vals[key][valid]
        got = rv[valid, COLS[col]]
        scale = row_value_scale(key, ref)
        err = np.abs(got - ref) / np.where(scale > 0, scale, 1.0)
        worst[key] = float(err.max()) if err.size else 0.0
        bad_rows = np.nonzero(err > tol)[0]
        assert bad_rows.size == 0, (key, worst[key], np.nonzero(valid)[0][bad_rows[:5]])
    if policy:
        clip = (seam["clipped"][seam["segment"]] if seam is not None else vals["clipped"]).astype(bool)
        keep = valid & ~(boundary if boundary is not None else np.zeros_like(valid))
        assert np.array_equal(rv[keep, 6] != 0, clip[keep])
    say(f"[gpu] {w.name}: scalars ok; per-row worst relative errors "
        + ", ".join(f"{k} {v:.1e}" for k, v in worst.items()))


def _grad_gate(w, sums):
    d2, r2, d2n, r2n, dmax, count = (sum(s[i] for s in sums) for i in range(6))
    if w.dtype == "f32":
        say(f"[gpu] {w.name}: gradient over {count} rows, max abs error {dmax:.3e}")
        assert dmax <= TOL["f32"]["grad_abs"]
        return
    tol = TOL[w.dtype]["grad_rms"]
    rms, rms_nl = np.sqrt(d2 / r2), np.sqrt(d2n / r2n)
    say(f"[gpu] {w.name}: gradient over {count} rows, rms-relative {rms:.3e}, non-label {rms_nl:.3e}")
    assert rms <= tol and rms_nl <= tol, (rms, rms_nl)


def _masked_rows(w, inp, grad, valid):
    inval = torch.from_numpy(~valid).to(DEV)
    if not inval.any():
        return
    if w.flags & workloads.ACCUMULATE:
        assert torch.equal(grad[inval], inp["grad_init"][inval])
    else:
        assert torch.count_nonzero(grad[inval].view(INT_VIEW[w.dtype])).item() == 0


def _boundary(spec, ratio):
    return (np.abs(ratio - (1 + spec.eps)) < 1e-5) | (np.abs(ratio - (1 - spec.eps)) < 1e-5)


def _per_row_pass(spec, inp, grad, N, n, want_grad, grad_rows=None, dlogp=None, skip=None):
    """Stream rows through the oracle. want_grad: compare the gradient of the
    rows (all, or those in grad_rows). Returns per-row value arrays (when all
    rows are visited), validity, bad flags and the gradient sums."""
    results = {}
    sums = []
    t0 = time.time()
    with ThreadPoolExecutor(max_workers=THREADS) as ex:
        if grad_rows is None:
            for r0 in range(0, N, BLOCK_ROWS):
                r1 = min(N, r0 + BLOCK_ROWS)
                blk = _host_block(inp, r0, r1)
                g_blk = grad[r0:r1].cpu() if want_grad else None
                futs = []
                for t0r in range(0, r1 - r0, TASK_ROWS):
                    rows = np.arange(t0r, min(r1 - r0, t0r + TASK_ROWS))
                    futs.append((r0 + t0r, ex.submit(
                        _oracle_task, spec, n, blk, rows, want_grad, g_blk,
                        None if dlogp is None else dlogp[r0 + rows],
                        None if skip is None else skip[r0 + rows])))
                for start, f in futs:
                    results[start] = f.result()
                say(f"[gpu]   oracle rows {r1}/{N} ({time.time() - t0:.0f} s)")
        else:
            idx = np.asarray(grad_rows)
            blk = _host_block({k: (v[torch.from_numpy(idx).to(v.device)] if isinstance(v, torch.Tensor)
                                   and v.dim() >= 1 and v.shape[0] == N else None) for k, v in inp.items()},
                              0, len(idx))
            g_blk = grad[torch.from_numpy(idx).to(DEV)].cpu()
            futs = [ex.submit(_oracle_task, spec, n, blk, np.arange(t, min(len(idx), t + TASK_ROWS)), True,
                              g_blk, None, None if skip is None else skip[idx[t:t + TASK_ROWS]])
                    for t in range(0, len(idx), TASK_ROWS)]
            for i, f in enumerate(futs):
                results[i] = f.result()
            say(f"[gpu]   oracle gradient on {len(idx)} sampled rows ({time.time() - t0:.0f} s)")
    order = sorted(results)
    vals = {k: np.concatenate([results[s]["vals"][k] for s in order]) for k in results[order[0]]["vals"]}
    valid = np.concatenate([results[s]["valid"] for s in order])
    bad = np.concatenate([results[s]["bad"] for s in order])
    sums = [results[s]["sums"] for s in order if "sums" in results[s]]
    return vals, valid, bad, sums


FULL = ["ce_z_tiny_f32", "ce_z_bf16", "ce_z_f16", "ce_fkl_bf16", "ce_rkl_bf16", "ce_fdce_bf16",
        "ce_fkl_hinton_bf16", "grpo_z_ent_bf16", "ce_z_grpo_ent_bf16"]


@pytest.mark.parametrize("name", FULL)
def test_full_batch_parity(name):
    w, spec, inp, plan, grad, sc, rv = _run(name)
    N = w.N
    labels = to_np(inp["labels"]).astype(np.int64)
    valid0, _ = oracle.row_validity(N, w.V, labels, to_np(inp["mask"]))
    n = spec.divisor if spec.divisor > 0 else float(valid0.sum())
    skip = None
    if spec.has(oracle.GRPO):
        # the clip decision at the boundary may differ: those rows leave the gradient comparison
        skip = _boundary(spec, rv[:, COLS["ratio"]]) & valid0
    vals, valid, bad, sums = _per_row_pass(spec, inp, grad, N, n, want_grad=True, skip=skip)
    assert np.array_equal(valid, valid0)
    boundary = _boundary(spec, vals["ratio"]) & valid if "ratio" in vals else None
    _check_rows_and_scalars(w, spec, sc, rv, vals, valid, bad, n, boundary=boundary)
    _grad_gate(w, sums)
    _masked_rows(w, inp, grad, valid)


def test_full_batch_parity_all_combined():
    """32768 x 256000 with teacher, softcap, accumulate: scalars and per-row
    values on every row; the gradient on every 32nd row (1024 rows)."""
    name = "all_combined_bf16"
    w, spec, inp, plan, grad, sc, rv = _run(name)
    N = w.N
    labels = to_np(inp["labels"]).astype(np.int64)
    valid0, _ = oracle.row_validity(N, w.V, labels, to_np(inp["mask"]))
    n = float(valid0.sum())
    vals, valid, bad, _ = _per_row_pass(spec, inp, grad, N, n, want_grad=False)
    boundary = _boundary(spec, vals["ratio"]) & valid
    _check_rows_and_scalars(w, spec, sc, rv, vals, valid, bad, n, boundary=boundary)
    sample = np.arange(0, N, 32)
    _, _, _, sums = _per_row_pass(spec, inp, grad, N, n, want_grad=True, grad_rows=sample, skip=boundary)
    _grad_gate(w, sums)
    _masked_rows(w, inp, grad, valid)


def test_full_batch_parity_gspo():
    """GSPO over the 32 sequences of 512 tokens: every row's values, the
    segment step for all 32 segments, the whole gradient."""
    name = "gspo_z_ent_bf16"
    w, spec, inp, plan, grad, sc, rv = _run(name)
    N = w.N
    labels = to_np(inp["labels"]).astype(np.int64)
    valid0, _ = oracle.row_validity(N, w.V, labels, to_np(inp["mask"]))
    n = float(valid0.sum())
    vals, valid, bad, _ = _per_row_pass(spec, inp, grad, N, n, want_grad=False)
    offs = inp["seq_offsets"].cpu().numpy().astype(np.int64)
    seam = oracle.gspo_seam(spec, vals["logp"], to_np(inp["old_logprobs"]), to_np(inp["advantages"]), valid, offs)
    near = _boundary(spec, seam["ratio"]) & seam["nonempty"]
    boundary = near[seam["segment"]] & valid
    say(f"[gpu] {name}: {seam['n_seg']} segments, {int(near.sum())} within 1e-5 of the clip boundary")
    _check_rows_and_scalars(w, spec, sc, rv, vals, valid, bad, n, seam=seam, boundary=boundary)
    _, _, _, sums = _per_row_pass(spec, inp, grad, N, n, want_grad=True, dlogp=seam["dlogp"], skip=boundary)
    _grad_gate(w, sums)
    _masked_rows(w, inp, grad, valid)
