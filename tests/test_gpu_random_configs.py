"""Seeded random configurations through the C ABI against the fp64 oracle.

Each case draws, from its own seed, an element type, a loss combination, a
batch (1-24 rows) and a vocabulary size (log-uniform over 1-300000; a
second set 100-600 rows over 1000-40000, several rows per XCD group), the
logit scale, softcap and temperature, overwrite / accumulate / no gradient,
GSPO segments for the policy combinations, and the byte offsets of logits,
teacher and gradient (mostly 16-byte aligned, sometimes a common or a
differing misalignment). That spans the kernel paths together: register-
resident slices with and without the chunk exchange, the streaming forward,
the load-mode backward and the row-wise kernel. Tolerances are those of the
other parity tests (fp32: scalars 1e-5 relative, gradient 1e-6 absolute;
bf16: scalars 1e-4 relative, gradient rms-relative 4e-3 over the tensor and
over its non-label entries; fp16: 1e-3); masked rows must be +0.0 or
untouched.

One configuration the fixed gates do not fit, a reading stated here: rows of
one element (V = 1) in bf16 and fp16 (fp32 rows of one element take the plain
gates: those instances form the statistics in fp64). There the exact CE, new
log-prob and every KL are 0 and every gradient term but the z-loss's cancels
exactly (q = 1), while the 16-bit instances form them from fp32 statistics of
magnitude S = max |s| (with a
softcap c, max(max |s|, c): the element path forms s log2 e as
c log2 e - 2 c log2 e r, within a few ulps of c log2 e). On such cases a
scalar slot is accepted within its relative gate or within 4 ulps of S
times the weight sum, and the gradient per element within the output
rounding (2^-7 relative) plus 4 ulps of L2 = log2(e) (S + max |lse|) times
grad_scale k (1 + sum of weights) / n; the test prints the measured error.
Every fp32 case uses the plain gates. fp16 stores magnitudes below
2^-14 as subnormals 2^-24 apart (a z-loss-only plan with a small weight puts
its whole gradient there): the fp16 rms bounds add that spacing,
rms(g - ref) <= 1e-3 rms(ref) + 2^-24, over the tensor and over its
non-label entries.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import (TOL, assert_scalars, degenerate_allowance, grad_check, make_plan, oracle_old_logprobs,
                         say, scalar_errors, spec_from, to_np)
from oracle import SLOT

pytestmark = pytest.mark.gpu
DEV = "cuda"
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
INT_VIEW = {"f32": torch.int32, "bf16": torch.int16, "f16": torch.int16}
CE, Z, FKL, RKL, FDCE, GRPO, GSPO, ENT, ACC, HINTON = (oracle.CE, oracle.ZLOSS, oracle.FKL, oracle.RKL, oracle.FDCE,
                                                       oracle.GRPO, oracle.GSPO, oracle.ENTROPY, oracle.ACCUMULATE,
                                                       oracle.HINTON)
DISTILL = FKL | RKL | FDCE
N_CASES = 400


N_BATCH_CASES = 40


def _draw(i):
    rng = np.random.default_rng(20261202 + i)
    dtype = ["f32", "bf16", "f16"][rng.integers(3)]
    if i >= N_CASES:
        # larger batches: several rows per XCD group and many rows' chunks in flight at once
        V = int(np.exp(rng.uniform(np.log(1000), np.log(40_000))))
        N = int(rng.integers(100, 601))
    else:
        V = int(np.exp(rng.uniform(0.0, np.log(300_000))))
        N = int(rng.integers(1, 25))
    flags = 0
    w = dict(ce=0.0, z=0.0, distill=0.0, grpo=0.0, grad_scale=float(rng.choice([1.0, 0.5, 2.0])))
    if rng.random() < 0.7:
        flags |= CE
        w["ce"] = float(rng.uniform(0.2, 1.5))
    if rng.random() < 0.5:
        flags |= Z
        w["z"] = float(rng.choice([1e-4, 1e-2, 0.3]))
    d = rng.integers(5)
    if d < 3:
        flags |= (FKL, RKL, FDCE)[d]
        w["distill"] = float(rng.uniform(0.2, 1.5))
        if rng.random() < 0.3:
            flags |= HINTON
    pol = rng.integers(4)
    if pol == 1:
        flags |= GRPO
        w["grpo"] = float(rng.uniform(0.3, 1.5))
    elif pol == 2:
        flags |= GSPO
        w["grpo"] = float(rng.uniform(0.3, 1.5))
    if rng.random() < 0.4:
        flags |= ENT
    if flags & (CE | Z | DISTILL | GRPO | GSPO) == 0:
        flags |= CE
        w["ce"] = 1.0
    if dtype == "f16":
        w["grad_scale"] *= 1024.0      # a loss scale keeps small gradients in fp16's normal range
    mode = ["overwrite", "overwrite", "accumulate", "none"][rng.integers(4)]
    if mode == "accumulate":
        flags |= ACC
    cap = float(rng.choice([0.0, 0.0, 10.0, 30.0]))
    scale = float(rng.choice([1.0, 1.0, 0.5, 1.3]))
    tau = float(rng.choice([1.0, 0.7, 2.0]))
    lay = rng.integers(8)
    offs = (0, 0, 0) if lay < 5 else ((1, 1, 17) if lay == 5 else tuple(int(v) for v in rng.integers(0, 8, 3)))
    return dict(dtype=dtype, V=V, N=N, flags=flags, w=w, mode=mode, cap=cap, scale=scale, tau=tau, offs=offs,
                seed=int(rng.integers(1 << 30)), mask_frac=float(rng.choice([0.0, 0.2])))


def _place(t, off):
    if t is None:
        return None, None
    es = t.element_size()
    buf = torch.empty(t.numel() * es + off * es + 64, dtype=torch.uint8, device=DEV)
    v = buf[off * es: off * es + t.numel() * es].view(t.dtype).view(t.shape)
    v.copy_(t.to(DEV))
    return buf, v


@pytest.mark.parametrize("i", range(N_CASES + N_BATCH_CASES))
def test_random_configuration(i):
    c = _draw(i)
    dtype, N, V, flags = c["dtype"], c["N"], c["V"], c["flags"]
    spec = spec_from(V, flags, c["w"], temperature=c["tau"], eps=0.2, logit_scale=c["scale"], softcap=c["cap"])
    gspo = bool(flags & GSPO)
    inp = workloads.small_inputs(N, V, dtype, "cpu", c["seed"], teacher=bool(flags & DISTILL),
                                 grpo=bool(flags & (GRPO | GSPO)), accumulate=bool(flags & ACC),
                                 mask_frac=c["mask_frac"], bad_labels=1 if N > 3 else 0)
    offsets = None
    if gspo:
        offsets = workloads.segment_offsets(N, c["seed"] % 1000, max_len=5)
    if flags & (GRPO | GSPO):
        inp["old_logprobs"] = oracle_old_logprobs(spec, inp["logits"], inp["labels"], inp["old_noise"])
    plan = make_plan(spec, TDT[dtype])
    say(f"[gpu] case {i}: {dtype} N={N} V={V} flags={flags:#x} mode={c['mode']} cap={c['cap']} "
        f"scale={c['scale']} tau={c['tau']} offsets={c['offs']} {plan.describe()}")
    ox, ot, og = c["offs"]
    keep = []
    b, x = _place(inp["logits"], ox)
    keep.append(b)
    b, t = _place(inp.get("teacher"), ot)
    keep.append(b)
    grad = None
    if c["mode"] == "overwrite":
        b, grad = _place(torch.full_like(inp["logits"], float("nan")), og)
        keep.append(b)
    elif c["mode"] == "accumulate":
        b, grad = _place(inp["grad_init"], og)
        keep.append(b)
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    sc = plan(x, labels=dev["labels"], mask=dev["mask"], teacher=t, old_logprobs=dev.get("old_logprobs"),
              advantages=dev.get("advantages"), grad=grad,
              seq_offsets=offsets.to(DEV) if offsets is not None else None)
    torch.cuda.synchronize()
    got = sc.cpu().double().numpy()

    y = to_np(inp["labels"]).astype(np.int64)
    mask = to_np(inp["mask"])
    valid, _ = oracle.row_validity(N, V, y, mask)
    args = dict(labels=y, mask=mask, teacher=to_np(inp.get("teacher")), old_logprobs=to_np(inp.get("old_logprobs")),
                advantages=to_np(inp.get("advantages")),
                grad_in=to_np(inp["grad_init"]) if flags & ACC else None, want_grad=c["mode"] != "none")
    if gspo:
        args["seq_offsets"] = offsets.numpy()
    ref_sc, ref_g = oracle.forward_backward(spec, to_np(inp["logits"]), **args)
    vals = oracle.row_values(spec, to_np(inp["logits"]), y, args["teacher"], args["old_logprobs"],
                             args["advantages"])
    # tokens (GRPO) or segments (GSPO) within 1e-5 of the clip boundary may take either branch
    boundary = np.zeros(N, dtype=bool)
    if flags & GRPO:
        r = vals["ratio"]
        boundary = ((np.abs(r - 1.2) < 1e-5) | (np.abs(r - 0.8) < 1e-5)) & valid
    if gspo:
        seam = oracle.gspo_seam(spec, vals["logp"], args["old_logprobs"], args["advantages"], valid,
                                args["seq_offsets"])
        near = ((np.abs(seam["ratio"] - 1.2) < 1e-5) | (np.abs(seam["ratio"] - 0.8) < 1e-5)) & seam["nonempty"]
        boundary = near[seam["segment"]] & valid
        vals = dict(vals, grpo=seam["loss"][seam["segment"]], adv=seam["adv"][seam["segment"]],
                    k3=seam["k3"][seam["segment"]])
    # magnitudes the fp32 statistics are formed from (valid rows)
    x64 = to_np(inp["logits"])[valid]
    s64 = (c["cap"] * np.tanh(c["scale"] * x64 / c["cap"]) if c["cap"] > 0 else c["scale"] * x64) \
        if valid.any() else np.zeros((1, 1))
    smax = max(float(np.max(np.abs(s64))), c["cap"])
    lmax = float(np.max(np.abs(np.log(np.sum(np.exp(s64 - s64.max(1, keepdims=True)), 1)) + s64.max(1))))
    wsum = 1.0 + sum(abs(v) for k, v in c["w"].items() if k != "grad_scale")
    rel = TOL[dtype]["scalar_rel"]
    errs = scalar_errors(spec, got, ref_sc, vals, valid)
    allow = degenerate_allowance(spec, to_np(inp["logits"])[valid] if valid.any() else None, dtype)
    for name, e in errs.items():
        if e > rel and name not in ("N_VALID", "N_BADLABEL"):
            say(f"[scalar-v1] case {i} {name} got={got[SLOT[name]]!r} ref={ref_sc[SLOT[name]]!r} "
                f"abs={abs(got[SLOT[name]] - ref_sc[SLOT[name]]):.3e} allowance={allow:.3e} V={V}")
    assert_scalars(spec, got, ref_sc, dtype, vals, valid, skip=("CLIPFRAC",) if boundary.any() else (),
                   x=to_np(inp["logits"])[valid] if valid.any() else None)
    if grad is None:
        return
    gk = grad.detach().cpu()
    keep_rows = ~boundary
    l2 = 1.4427 * (smax + lmax)
    if V == 1 and dtype != "f32":
        n = max(1, int(valid.sum()))
        floor = 4 * l2 * 2.0 ** -23 * c["w"]["grad_scale"] * c["scale"] * wsum / n
        gd = to_np(gk[torch.from_numpy(keep_rows)])
        rd = ref_g[keep_rows]
        say(f"[v1-grad] case {i} max_abs={float(np.max(np.abs(gd - rd))) if gd.size else 0.0:.3e} floor={floor:.3e}")
        assert np.all(np.abs(gd - rd) <= 2.0 ** -7 * np.abs(rd) + floor), (np.max(np.abs(gd - rd)), floor)
    elif dtype == "f16":
        gd = to_np(gk[torch.from_numpy(keep_rows)])
        rd = ref_g[keep_rows]
        tol = TOL["f16"]["grad_rms"]
        nonlab = np.ones_like(rd, dtype=bool)
        yk = y[keep_rows]
        ok_y = (yk >= 0) & (yk < V)
        nonlab[np.arange(rd.shape[0])[ok_y], yk[ok_y]] = False
        for sel in (np.ones_like(rd, dtype=bool), nonlab):
            if sel.any():
                err = float(np.sqrt(np.mean((gd[sel] - rd[sel]) ** 2)))
                assert err <= tol * float(np.sqrt(np.mean(rd[sel] ** 2))) + 2.0 ** -24, (err, float(np.abs(rd[sel]).max()))
    else:
        met = grad_check(gk[torch.from_numpy(keep_rows)], ref_g[keep_rows], dtype, labels=y[keep_rows])
        if "max_abs" in met:
            say(f"[f32-err] case {i} max_abs={met['max_abs']:.3e} "
                f"max|g|={float(np.max(np.abs(ref_g))) if ref_g.size else 0.0:.3e}")
    inval = torch.from_numpy(~valid)
    if c["mode"] == "overwrite":
        assert torch.equal(gk[inval].view(INT_VIEW[dtype]), torch.zeros_like(gk[inval]).view(INT_VIEW[dtype]))
    else:
        assert torch.equal(gk[inval], inp["grad_init"][inval])
