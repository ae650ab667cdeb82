"""Pins for the fp64 oracle, against things other than the oracle itself.

Every check here is one of: an exact closed form (uniform logits, a
hand-worked example in tests/golden/), a torch library routine that computes
the same named quantity (cross_entropy, Categorical.entropy, kl_div,
log_softmax), central finite differences of the total loss, an independent
torch autograd of the total loss, or an invariant the mathematics fixes
(shift invariance, identity teacher, ratio one, clipped tokens,
superposition, accumulation). The last section plants mistakes in the oracle
and checks that these pins catch them.

KL_OLD_NEW and ADV_MEAN have no definition on the pages; they are checked
against the closed forms of the readings taken (k3 estimator, mean
advantage) only: parity unpinned by the pages.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import headloss_oracle as ho
from oracle import SLOT, Spec

HERE = os.path.dirname(os.path.abspath(__file__))
ALL_LOSSES = oracle.CE | oracle.ZLOSS | oracle.GRPO | oracle.ENTROPY


def _eval(expr):
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log}))


def _rng(seed):
    return np.random.default_rng(seed)


def _grpo_inputs(rng, x, labels, spec, spread=0.05):
    """old_logprobs near the current label log-prob, advantages ~ N(0,1)."""
    vals = ho.row_values(spec, x, labels)
    old = vals["logp"] + rng.normal(0.0, spread, size=x.shape[0])
    adv = rng.normal(0.0, 1.0, size=x.shape[0])
    return old, adv


# ---------------------------------------------------------------------------
# Hand-worked example (tests/golden/hand_example_v4.json)
# ---------------------------------------------------------------------------
def test_golden_hand_example():
    with open(os.path.join(HERE, "golden", "hand_example_v4.json")) as f:
        g = json.load(f)
    sp = g["spec"]
    flags = 0
    for name in sp["flags"]:
        flags |= getattr(oracle, name)
    spec = Spec(V=sp["V"], flags=flags, w_ce=sp["w_ce"], w_z=sp["w_z"],
                w_distill=sp["w_distill"], w_grpo=sp["w_grpo"],
                grad_scale=sp["grad_scale"], temperature=sp["temperature"],
                eps=sp["eps"], logit_scale=sp["logit_scale"], softcap=sp["softcap"])
    inp = g["inputs"]
    x = np.array([[_eval(e) for e in row] for row in inp["logits"]])
    t = np.array([[_eval(e) for e in row] for row in inp["teacher"]])
    y = np.array(inp["labels"], dtype=np.int64)
    old = np.array([_eval(e) for e in inp["old_logprobs"]])
    adv = np.array([_eval(e) for e in inp["advantages"]])
    scalars, grad = oracle.forward_backward(spec, x, y, None, t, old, adv)
    for name, expr in g["expected_scalars"].items():
        assert scalars[SLOT[name]] == pytest.approx(_eval(expr), abs=1e-12), name
    exp_grad = np.array([[_eval(e) for e in row] for row in g["expected_grad"]])
    np.testing.assert_allclose(grad, exp_grad, atol=1e-14, rtol=0)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("V", [1024, 151936])
def test_uniform_logits_closed_forms(V):
    spec = Spec(V=V, flags=oracle.CE | oracle.ZLOSS | oracle.ENTROPY, w_z=1.0)
    x = np.zeros((2, V))
    y = np.array([0, V - 1])
    sc, grad = oracle.forward_backward(spec, x, y)
    logV = math.log(V)
    assert sc[SLOT["CE"]] == pytest.approx(logV, rel=1e-14)
    assert sc[SLOT["Z"]] == pytest.approx(logV ** 2, rel=1e-14)
    assert sc[SLOT["ENTROPY"]] == pytest.approx(logV, rel=1e-13)
    # CE grad: (1/V - delta)/n ; z grad: 2 log V / V / n
    expect = np.full((2, V), (1.0 / V + 2 * logV / V) / 2)
    expect[0, 0] -= 0.5
    expect[1, V - 1] -= 0.5
    np.testing.assert_allclose(grad, expect, atol=1e-15, rtol=1e-12)


def test_uniform_values_from_the_survey_table():
    # all-zero logits: CE = log V (1024 -> 6.9315, 151936 -> 11.9312), z = (log V)^2
    assert math.log(1024) == pytest.approx(6.9315, abs=1e-4)
    assert math.log(151936) == pytest.approx(11.9312, abs=1e-4)
    assert math.log(1024) ** 2 == pytest.approx(48.045, abs=1e-3)


def test_entropy_extremes():
    V = 300
    spec = Spec(V=V, flags=oracle.ENTROPY)
    x = np.zeros((1, V))
    x[0, 17] = 50.0  # one dominant logit: entropy ~ 0
    sc, _ = oracle.forward_backward(spec, x, want_grad=False)
    assert 0.0 <= sc[SLOT["ENTROPY"]] < 1e-17 * V * 60


# ---------------------------------------------------------------------------
# torch library routines computing the same named quantity
# ---------------------------------------------------------------------------
def test_ce_value_and_grad_vs_torch_cross_entropy():
    rng = _rng(1)
    N, V = 23, 41
    x = rng.normal(0, 2.0, size=(N, V))
    y = rng.integers(0, V, size=N)
    y[[3, 7, 11]] = -100
    w, G = 0.7, 0.37
    spec = Spec(V=V, flags=oracle.CE, w_ce=w, grad_scale=G)
    sc, grad = oracle.forward_backward(spec, x, y)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    ce = F.cross_entropy(xt, torch.tensor(y), ignore_index=-100, reduction="mean")
    (G * w * ce).backward()
    assert sc[SLOT["CE"]] == pytest.approx(ce.item(), rel=1e-13)
    np.testing.assert_allclose(grad, xt.grad.numpy(), atol=1e-15, rtol=1e-11)
    assert sc[SLOT["N_VALID"]] == N - 3


def test_entropy_vs_torch_categorical():
    rng = _rng(2)
    x = rng.normal(0, 3.0, size=(9, 77))
    spec = Spec(V=77, flags=oracle.ENTROPY)
    vals = ho.row_values(spec, x)
    ref = torch.distributions.Categorical(logits=torch.tensor(x)).entropy().numpy()
    np.testing.assert_allclose(vals["entropy"], ref, rtol=1e-12)


@pytest.mark.parametrize("tau", [1.0, 2.0, 0.5])
def test_kl_vs_torch_kl_div(tau):
    rng = _rng(3)
    N, V = 7, 53
    t = rng.normal(0, 3.0, size=(N, V))
    x = 0.8 * t + rng.normal(0, 1.0, size=(N, V))
    spec = Spec(V=V, flags=oracle.FKL, temperature=tau)
    vals = ho.row_values(spec, x, teacher=t)
    logq = torch.log_softmax(torch.tensor(x), -1)
    logp = torch.log_softmax(torch.tensor(t) / tau, -1)
    fkl = F.kl_div(logq, logp, log_target=True, reduction="none").sum(-1).numpy()
    rkl = F.kl_div(logp, logq, log_target=True, reduction="none").sum(-1).numpy()
    np.testing.assert_allclose(vals["fkl"], fkl, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(vals["rkl"], rkl, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("tau", [1.0, 2.0])
def test_fdce_vs_torch_soft_target_cross_entropy(tau):
    """From-distribution CE: torch's cross_entropy with probability targets,
    and the identity FDCE = FKL + H(teacher) with H from Categorical."""
    rng = _rng(19)
    N, V = 6, 43
    t = rng.normal(0, 3.0, size=(N, V))
    x = 0.8 * t + rng.normal(0, 1.0, size=(N, V))
    spec = Spec(V=V, flags=oracle.FDCE, w_ce=0.0, w_distill=0.7, temperature=tau, grad_scale=0.3)
    sc, grad = oracle.forward_backward(spec, x, teacher=t)
    p = torch.softmax(torch.tensor(t) / tau, -1)
    xt = torch.tensor(x, requires_grad=True)
    ce = F.cross_entropy(xt, p, reduction="mean")
    (0.3 * 0.7 * ce).backward()
    assert sc[SLOT["DISTILL"]] == pytest.approx(ce.item(), rel=1e-12)
    np.testing.assert_allclose(grad, xt.grad.numpy(), atol=1e-15, rtol=1e-11)
    vals = ho.row_values(spec, x, teacher=t)
    h_t = torch.distributions.Categorical(probs=p).entropy().numpy()
    np.testing.assert_allclose(vals["fdce"], vals["fkl"] + h_t, rtol=1e-12)


def test_newlogp_vs_torch_log_softmax():
    rng = _rng(4)
    N, V = 11, 29
    x = rng.normal(0, 2.0, size=(N, V))
    y = rng.integers(0, V, size=N)
    spec = Spec(V=V, flags=oracle.GRPO, w_ce=0.0, w_grpo=1.0, logit_scale=0.5, softcap=3.0)
    old, adv = _grpo_inputs(rng, x, y, spec)
    sc, _ = oracle.forward_backward(spec, x, y, None, None, old, adv, want_grad=False)
    s = spec.softcap * torch.tanh(torch.tensor(x) * spec.logit_scale / spec.softcap)
    ref = torch.log_softmax(s, -1)[torch.arange(N), torch.tensor(y)].mean().item()
    assert sc[SLOT["NEWLOGP"]] == pytest.approx(ref, rel=1e-12)


# ---------------------------------------------------------------------------
# Independent torch autograd of the total loss (pins every hand gradient)
# ---------------------------------------------------------------------------
def _torch_total(spec, x, y, mask, t, old, adv, offsets=None):
    """The weighted total, built from torch library pieces, differentiated by autograd."""
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    k, c = spec.logit_scale, spec.softcap
    s = c * torch.tanh(k * xt / c) if c > 0 else k * xt
    yv = torch.tensor(y) if y is not None else None
    valid = torch.ones(x.shape[0], dtype=torch.bool)
    if mask is not None:
        valid &= torch.tensor(mask) != 0
    if yv is not None:
        valid &= (yv != -100) & (yv >= 0) & (yv < spec.V)
    n = spec.divisor if spec.divisor > 0 else float(valid.sum())
    sv = s[valid]
    total = torch.zeros((), dtype=torch.float64)
    logq = torch.log_softmax(sv, -1)
    if spec.flags & oracle.CE:
        total = total + spec.w_ce * F.cross_entropy(sv, yv[valid], reduction="sum") / n
    if spec.flags & oracle.ZLOSS:
        total = total + spec.w_z * (torch.logsumexp(sv, -1) ** 2).sum() / n
    if spec.flags & oracle.DISTILL_FLAGS:
        tau = spec.temperature
        logp = torch.log_softmax(torch.tensor(t)[valid] / tau, -1)
        hinton = bool(spec.flags & oracle.HINTON)
        sd = sv / tau if hinton else sv
        logq_d = torch.log_softmax(sd, -1)
        if spec.flags & oracle.FKL:
            kl = F.kl_div(logq_d, logp, log_target=True, reduction="sum")
        elif spec.flags & oracle.RKL:
            kl = F.kl_div(logp, logq_d, log_target=True, reduction="sum")
        else:
            kl = F.cross_entropy(sd, logp.exp(), reduction="sum")
        if hinton:
            kl = kl * tau * tau
        total = total + spec.w_distill * kl / n
    if spec.flags & oracle.GRPO:
        lp = logq.gather(-1, yv[valid][:, None])[:, 0]
        r = torch.exp(lp - torch.tensor(old)[valid])
        A = torch.tensor(adv)[valid]
        obj = torch.minimum(r * A, torch.clamp(r, 1 - spec.eps, 1 + spec.eps) * A)
        total = total + spec.w_grpo * (-obj).sum() / n
    if spec.flags & oracle.GSPO:
        # sequence-level ratio: exp of the mean token log-ratio of each
        # segment's valid tokens; the loss averages over nonempty segments
        lq_all = torch.log_softmax(s, -1)
        yc = torch.clamp(yv, 0, spec.V - 1)
        lp = lq_all.gather(-1, yc[:, None])[:, 0]
        objs = []
        for i in range(len(offsets) - 1):
            idx = [r for r in range(offsets[i], offsets[i + 1]) if bool(valid[r])]
            if not idx:
                continue
            idx = torch.tensor(idx)
            log_s = (lp[idx] - torch.tensor(old)[idx]).mean()
            r = torch.exp(log_s)
            A = torch.tensor(adv)[idx].mean()
            objs.append(torch.minimum(r * A, torch.clamp(r, 1 - spec.eps, 1 + spec.eps) * A))
        if objs:
            total = total + spec.w_grpo * (-torch.stack(objs)).mean()
    (spec.grad_scale * total).backward()
    return xt.grad.numpy()


@pytest.mark.parametrize("mode", ["fkl", "rkl", "fdce"])
@pytest.mark.parametrize("softcap", [0.0, 4.0])
def test_total_gradient_vs_torch_autograd(mode, softcap):
    rng = _rng(5)
    N, V = 13, 37
    t = rng.normal(0, 3.0, size=(N, V))
    x = 0.7 * t + rng.normal(0, 1.5, size=(N, V))
    y = rng.integers(0, V, size=N)
    y[2] = -100
    mask = np.ones(N, dtype=np.uint8)
    mask[5] = 0
    flags = oracle.CE | oracle.ZLOSS | oracle.GRPO | oracle.ENTROPY
    flags |= {"fkl": oracle.FKL, "rkl": oracle.RKL, "fdce": oracle.FDCE}[mode]
    spec = Spec(V=V, flags=flags, w_ce=1.0, w_z=0.3, w_distill=0.5, w_grpo=0.8,
                grad_scale=0.25, temperature=1.5, eps=0.2, logit_scale=0.5,
                softcap=softcap)
    old, adv = _grpo_inputs(rng, x, y, spec, spread=0.3)
    _, grad = oracle.forward_backward(spec, x, y, mask, t, old, adv)
    ref = _torch_total(spec, x, y, mask, t, old, adv)
    np.testing.assert_allclose(grad, ref, atol=1e-15, rtol=1e-10)


# ---------------------------------------------------------------------------
# Central finite differences of the oracle's own total
# ---------------------------------------------------------------------------
def _fd_check(spec, x, y, mask, t, old, adv, h=1e-6, tol=2e-8):
    _, grad = oracle.forward_backward(spec, x, y, mask, t, old, adv)
    fd = np.zeros_like(x)
    for i in range(x.shape[0]):
        for j in range(x.shape[1]):
            xp = x.copy(); xp[i, j] += h
            xm = x.copy(); xm[i, j] -= h
            fp = oracle.total_loss(spec, xp, y, mask, t, old, adv)
            fm = oracle.total_loss(spec, xm, y, mask, t, old, adv)
            fd[i, j] = (fp - fm) / (2 * h)
    np.testing.assert_allclose(grad, fd, atol=tol, rtol=0)


@pytest.mark.parametrize("mode", ["fkl", "rkl", "fdce"])
@pytest.mark.parametrize("softcap,scale", [(0.0, 1.0), (2.5, 0.7)])
def test_finite_differences_all_losses(mode, softcap, scale):
    rng = _rng(6)
    N, V = 4, 9
    t = rng.normal(0, 2.0, size=(N, V))
    x = rng.normal(0, 2.0, size=(N, V))
    y = rng.integers(0, V, size=N)
    flags = ALL_LOSSES | {"fkl": oracle.FKL, "rkl": oracle.RKL, "fdce": oracle.FDCE}[mode]
    spec = Spec(V=V, flags=flags, w_ce=0.9, w_z=0.2, w_distill=0.6, w_grpo=1.1,
                grad_scale=0.5, temperature=1.7, eps=0.2, logit_scale=scale,
                softcap=softcap)
    old, adv = _grpo_inputs(rng, x, y, spec, spread=0.05)
    _fd_check(spec, x, y, None, t, old, adv)


def test_finite_differences_clipped_grpo_tokens():
    rng = _rng(7)
    N, V = 3, 8
    x = rng.normal(0, 2.0, size=(N, V))
    y = rng.integers(0, V, size=N)
    spec = Spec(V=V, flags=oracle.GRPO, w_ce=0.0, w_grpo=1.0, eps=0.2)
    vals = ho.row_values(spec, x, y)
    # ratio 1.5 with A>0 (clipped, flat), ratio 0.5 with A<0 (clipped, flat),
    # ratio 1.5 with A<0 (unclipped, flows)
    old = vals["logp"] - np.log(np.array([1.5, 0.5, 1.5]))
    adv = np.array([1.0, -1.0, -1.0])
    _, grad = oracle.forward_backward(spec, x, y, None, None, old, adv)
    assert np.all(grad[0] == 0) and np.all(grad[1] == 0)
    assert np.abs(grad[2]).max() > 0.1
    _fd_check(spec, x, y, None, None, old, adv)


# ---------------------------------------------------------------------------
# Invariants and special cases
# ---------------------------------------------------------------------------
def test_shift_invariance():
    rng = _rng(8)
    N, V = 6, 31
    t = rng.normal(0, 3, size=(N, V))
    x = rng.normal(0, 3, size=(N, V))
    y = rng.integers(0, V, size=N)
    flags = oracle.CE | oracle.RKL | oracle.GRPO | oracle.ENTROPY
    spec = Spec(V=V, flags=flags, w_distill=0.5, w_grpo=1.0, temperature=2.0)
    old, adv = _grpo_inputs(rng, x, y, spec)
    sc0, g0 = oracle.forward_backward(spec, x, y, None, t, old, adv)
    shift = rng.normal(0, 10, size=(N, 1))
    sc1, g1 = oracle.forward_backward(spec, x + shift, y, None, t + 3 * shift, old, adv)
    for name in ("CE", "DISTILL", "GRPO", "ENTROPY", "NEWLOGP", "RATIO", "TOTAL"):
        assert sc1[SLOT[name]] == pytest.approx(sc0[SLOT[name]], rel=1e-11, abs=1e-12), name
    np.testing.assert_allclose(g1, g0, atol=1e-13)


def test_z_loss_is_not_shift_invariant():
    rng = _rng(9)
    x = rng.normal(0, 1, size=(3, 20))
    spec = Spec(V=20, flags=oracle.ZLOSS, w_ce=0.0, w_z=1.0)
    v0 = ho.row_values(spec, x)
    v1 = ho.row_values(spec, x + 2.5)
    np.testing.assert_allclose(v1["z"], (v0["lse"] + 2.5) ** 2, rtol=1e-13)


def test_identity_teacher_gives_zero_kl_and_zero_distill_grad():
    rng = _rng(10)
    N, V = 5, 64
    x = rng.normal(0, 3, size=(N, V))
    for flag in (oracle.FKL, oracle.RKL):
        spec = Spec(V=V, flags=flag, w_ce=0.0, w_distill=1.0, temperature=1.0)
        sc, grad = oracle.forward_backward(spec, x, teacher=x)
        assert abs(sc[SLOT["DISTILL"]]) < 1e-14
        assert np.abs(grad).max() < 1e-16


def test_kl_nonnegative_and_uniform_teacher_limit():
    rng = _rng(11)
    N, V = 8, 40
    t = rng.normal(0, 3, size=(N, V))
    x = rng.normal(0, 3, size=(N, V))
    spec = Spec(V=V, flags=oracle.FKL, temperature=1.0)
    v = ho.row_values(spec, x, teacher=t)
    assert np.all(v["fkl"] >= 0) and np.all(v["rkl"] >= 0)
    # tau -> infinity: the teacher is uniform, FKL = -log V - mean_j log q_j
    spec_inf = Spec(V=V, flags=oracle.FKL, temperature=1e12)
    vi = ho.row_values(spec_inf, x, teacher=t)
    expect = -math.log(V) - v["logq"].mean(axis=1)
    np.testing.assert_allclose(vi["fkl"], expect, rtol=1e-9)


def test_grpo_ratio_one_reduces_to_policy_gradient():
    rng = _rng(12)
    N, V = 10, 25
    x = rng.normal(0, 2, size=(N, V))
    y = rng.integers(0, V, size=N)
    spec = Spec(V=V, flags=oracle.GRPO, w_ce=0.0, w_grpo=1.0)
    vals = ho.row_values(spec, x, y)
    old = vals["logp"].copy()
    adv = rng.normal(0, 1, size=N)
    sc, grad = oracle.forward_backward(spec, x, y, None, None, old, adv)
    assert sc[SLOT["GRPO"]] == pytest.approx(-adv.mean(), rel=1e-12)
    assert sc[SLOT["RATIO"]] == pytest.approx(1.0, rel=1e-14)
    assert sc[SLOT["CLIPFRAC"]] == 0.0
    assert abs(sc[SLOT["KL_OLD_NEW"]]) < 1e-15
    assert sc[SLOT["ADV_MEAN"]] == pytest.approx(adv.mean(), rel=1e-14)
    # gradient = -A * d logp / dx / n, with d logp/dx from torch autograd
    xt = torch.tensor(x, requires_grad=True)
    lp = torch.log_softmax(xt, -1)[torch.arange(N), torch.tensor(y)]
    (-(torch.tensor(adv) * lp).sum() / N).backward()
    np.testing.assert_allclose(grad, xt.grad.numpy(), atol=1e-15, rtol=1e-11)


def test_grpo_zero_advantage_and_clipped_closed_forms():
    rng = _rng(13)
    N, V = 4, 12
    x = rng.normal(0, 2, size=(N, V))
    y = rng.integers(0, V, size=N)
    spec = Spec(V=V, flags=oracle.GRPO, w_ce=0.0, w_grpo=1.0, eps=0.2)
    vals = ho.row_values(spec, x, y)
    old = vals["logp"] - np.log(1.5)             # ratio 1.5 everywhere
    sc, grad = oracle.forward_backward(spec, x, y, None, None, old, np.zeros(N))
    assert sc[SLOT["GRPO"]] == 0.0 and np.all(grad == 0)
    A = np.array([0.5, 1.0, 2.0, 3.0])           # all positive: clipped at 1+eps
    sc, grad = oracle.forward_backward(spec, x, y, None, None, old, A)
    assert sc[SLOT["GRPO"]] == pytest.approx(-(1.2 * A).mean(), rel=1e-14)
    assert np.all(grad == 0)
    assert sc[SLOT["CLIPFRAC"]] == 1.0
    assert sc[SLOT["KL_OLD_NEW"]] == pytest.approx(0.5 - math.log(1.5), rel=1e-12)


def test_softcap_and_scale_limits():
    rng = _rng(14)
    N, V = 5, 33
    x = rng.normal(0, 2, size=(N, V))
    y = rng.integers(0, V, size=N)
    base = dict(V=V, flags=oracle.CE | oracle.ZLOSS | oracle.ENTROPY, w_z=0.1)
    sc0, g0 = oracle.forward_backward(Spec(**base), x, y)
    sc1, g1 = oracle.forward_backward(Spec(**base, softcap=1e7), x, y)
    np.testing.assert_allclose(sc1, sc0, rtol=1e-10)
    np.testing.assert_allclose(g1, g0, atol=1e-12)
    # logit_scale k on raw logits equals scale 1 on k*x, with the chain factor k
    k = 0.37
    sc2, g2 = oracle.forward_backward(Spec(**base, logit_scale=k), x, y)
    sc3, g3 = oracle.forward_backward(Spec(**base), k * x, y)
    np.testing.assert_allclose(sc2, sc3, rtol=1e-13)
    np.testing.assert_allclose(g2, k * g3, atol=1e-15)


def test_superposition_of_single_loss_runs():
    rng = _rng(15)
    N, V = 9, 45
    t = rng.normal(0, 3, size=(N, V))
    x = 0.8 * t + rng.normal(0, 1, size=(N, V))
    y = rng.integers(0, V, size=N)
    y[0] = -100
    w = dict(w_ce=0.5, w_z=0.01, w_distill=1.0, w_grpo=0.7)
    full = Spec(V=V, flags=ALL_LOSSES | oracle.RKL, temperature=2.0, **w)
    old, adv = _grpo_inputs(rng, x, y, full)
    sc, g = oracle.forward_backward(full, x, y, None, t, old, adv)
    acc = np.zeros_like(x)
    for flag, key in ((oracle.CE, "w_ce"), (oracle.ZLOSS, "w_z"),
                      (oracle.RKL, "w_distill"), (oracle.GRPO, "w_grpo")):
        single = Spec(V=V, flags=flag, temperature=2.0,
                      **{k: (v if k == key else 0.0) for k, v in w.items()})
        _, gk = oracle.forward_backward(single, x, y, None, t, old, adv)
        acc += gk
    np.testing.assert_allclose(g, acc, atol=1e-15, rtol=1e-12)
    # a zero-weight loss still reports its scalar and adds nothing to the gradient
    zero = Spec(V=V, flags=ALL_LOSSES | oracle.RKL, temperature=2.0,
                **{**w, "w_grpo": 0.0})
    sc0, g0 = oracle.forward_backward(zero, x, y, None, t, old, adv)
    assert sc0[SLOT["GRPO"]] == sc[SLOT["GRPO"]] and sc0[SLOT["RATIO"]] == sc[SLOT["RATIO"]]
    nog = Spec(V=V, flags=ALL_LOSSES | oracle.RKL, temperature=2.0, **{**w, "w_grpo": 0.0})
    _, g_no_grpo = oracle.forward_backward(nog, x, y, None, t, old, adv)
    np.testing.assert_allclose(g0, g_no_grpo, atol=0)


def test_masking_accumulate_divisor_and_bad_labels():
    rng = _rng(16)
    N, V = 12, 20
    x = rng.normal(0, 2, size=(N, V))
    y = rng.integers(0, V, size=N)
    y[1] = -100
    y[2] = V + 5       # out of range: masked and counted
    y[3] = -7          # out of range: masked and counted
    mask = np.ones(N, dtype=np.uint8)
    mask[4] = 0
    y[4] = V + 1       # masked by the mask byte: not counted as bad
    existing = rng.normal(0, 1, size=(N, V))
    spec = Spec(V=V, flags=oracle.CE | oracle.ZLOSS | oracle.ACCUMULATE, w_z=0.1)
    sc, g_acc = oracle.forward_backward(spec, x, y, mask, grad_in=existing)
    spec_over = Spec(V=V, flags=oracle.CE | oracle.ZLOSS, w_z=0.1)
    sc2, g = oracle.forward_backward(spec_over, x, y, mask)
    assert sc[SLOT["N_VALID"]] == N - 4 and sc[SLOT["N_BADLABEL"]] == 2
    for r in (1, 2, 3, 4):
        assert np.all(g[r] == 0.0)
        assert np.array_equal(g_acc[r], existing[r])
    np.testing.assert_allclose(g_acc - existing, g, atol=1e-15)
    # divisor: scalars and gradient both use it
    spec_div = Spec(V=V, flags=oracle.CE | oracle.ZLOSS, w_z=0.1, divisor=100.0)
    sc3, g3 = oracle.forward_backward(spec_div, x, y, mask)
    np.testing.assert_allclose(sc3[SLOT["CE"]], sc2[SLOT["CE"]] * (N - 4) / 100.0, rtol=1e-14)
    np.testing.assert_allclose(g3, g * (N - 4) / 100.0, atol=1e-16)


def test_all_rows_masked_gives_zeros():
    x = np.random.default_rng(17).normal(size=(4, 10))
    y = np.full(4, -100)
    spec = Spec(V=10, flags=ALL_LOSSES, w_grpo=1.0)
    sc, g = oracle.forward_backward(spec, x, y, None, None, np.zeros(4), np.ones(4))
    assert np.all(sc == 0.0) and np.all(g == 0.0)


# ---------------------------------------------------------------------------
# Hinton temperature mode (opt-in: tau on both softmaxes, times tau^2)
# ---------------------------------------------------------------------------
MODES = {"fkl": oracle.FKL, "rkl": oracle.RKL, "fdce": oracle.FDCE}


def _distill_case(seed, N=7, V=23, softcap=0.0, scale=1.0, tau=1.7, hinton=True, mode="fkl"):
    rng = _rng(seed)
    t = rng.normal(0, 3.0, size=(N, V))
    x = 0.6 * t + rng.normal(0, 1.5, size=(N, V))
    y = rng.integers(0, V, size=N)
    y[1] = -100
    flags = oracle.CE | oracle.ZLOSS | MODES[mode] | (oracle.HINTON if hinton else 0)
    spec = Spec(V=V, flags=flags, w_ce=0.7, w_z=0.05, w_distill=1.3, grad_scale=0.5,
                temperature=tau, logit_scale=scale, softcap=softcap)
    return spec, x, y, t


@pytest.mark.parametrize("mode", list(MODES))
def test_hinton_at_tau_one_is_the_plain_mode(mode):
    spec_h, x, y, t = _distill_case(21, tau=1.0, mode=mode)
    spec_p, _, _, _ = _distill_case(21, tau=1.0, mode=mode, hinton=False)
    sc_h, g_h = oracle.forward_backward(spec_h, x, y, None, t)
    sc_p, g_p = oracle.forward_backward(spec_p, x, y, None, t)
    np.testing.assert_allclose(sc_h, sc_p, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(g_h, g_p, rtol=1e-13, atol=1e-16)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("softcap,tau", [(0.0, 1.7), (4.0, 0.6), (0.0, 3.0)])
def test_hinton_gradient_vs_torch_autograd(mode, softcap, tau):
    spec, x, y, t = _distill_case(22, softcap=softcap, scale=0.8, tau=tau, mode=mode)
    _, grad = oracle.forward_backward(spec, x, y, None, t)
    ref = _torch_total(spec, x, y, None, t, None, None)
    np.testing.assert_allclose(grad, ref, atol=1e-15, rtol=1e-10)


@pytest.mark.parametrize("mode", ["fkl", "rkl"])
def test_hinton_identity_teacher_has_zero_kl_at_any_tau(mode):
    """With the teacher equal to the (unscaled, uncapped) student both tempered
    distributions coincide, so the Hinton KL and its gradient vanish for every
    tau; the teacher-only temperature reading does not have this property."""
    for tau in (0.5, 2.0, 7.0):
        spec, x, y, _ = _distill_case(23, tau=tau, mode=mode)
        spec.flags &= ~(oracle.CE | oracle.ZLOSS)
        sc, g = oracle.forward_backward(spec, x, None, None, x.copy())
        assert abs(sc[SLOT["DISTILL"]]) < 1e-13
        assert np.abs(g).max() < 1e-15
        spec_p, _, _, _ = _distill_case(23, tau=tau, mode=mode, hinton=False)
        spec_p.flags &= ~(oracle.CE | oracle.ZLOSS)
        sc_p, _ = oracle.forward_backward(spec_p, x, None, None, x.copy())
        assert sc_p[SLOT["DISTILL"]] > 1e-3


@pytest.mark.parametrize("mode", list(MODES))
def test_hinton_finite_differences(mode):
    spec, x, y, t = _distill_case(24, N=3, V=8, softcap=3.0, scale=0.9, tau=2.3, mode=mode)
    _fd_check(spec, x, y, None, t, None, None)


def test_hinton_planted_tau_factor_is_caught(monkeypatch):
    orig = ho.loss_gradients_wrt_s

    def tau_squared_gradient(spec, vals):
        g = orig(spec, vals)
        if "distill" in g and spec.has(oracle.HINTON):
            g["distill"] = g["distill"] * spec.temperature      # tau^2 instead of tau
        return g

    monkeypatch.setattr(ho, "loss_gradients_wrt_s", tau_squared_gradient)
    with pytest.raises(AssertionError):
        test_hinton_gradient_vs_torch_autograd("fkl", 0.0, 1.7)
    monkeypatch.setattr(ho, "loss_gradients_wrt_s", orig)


# ---------------------------------------------------------------------------
# GSPO (sequence-level ratio, per-segment step between forward and backward)
# ---------------------------------------------------------------------------
GSPO_OFFSETS = [0, 3, 3, 7, 8, 13]     # an empty segment and a one-token one


def _gspo_case(seed=11, N=13, V=29, softcap=0.0, flags=None, spread=0.3):
    rng = _rng(seed)
    t = rng.normal(0, 3.0, size=(N, V))
    x = 0.7 * t + rng.normal(0, 1.5, size=(N, V))
    y = rng.integers(0, V, size=N)
    y[4] = -100
    mask = np.ones(N, dtype=np.uint8)
    mask[min(9, N - 1)] = 0
    flags = flags if flags is not None else (oracle.CE | oracle.ZLOSS | oracle.GSPO | oracle.ENTROPY)
    spec = Spec(V=V, flags=flags, w_ce=0.6, w_z=0.2, w_distill=0.5, w_grpo=1.3,
                grad_scale=0.5, temperature=1.5, eps=0.2, logit_scale=0.8, softcap=softcap)
    vals = ho.row_values(spec, x, y)
    old = vals["logp"] + rng.normal(0, spread, size=N)
    # one advantage per segment, repeated over its tokens
    adv = np.zeros(N)
    for i in range(len(GSPO_OFFSETS) - 1):
        adv[GSPO_OFFSETS[i]:GSPO_OFFSETS[i + 1]] = rng.normal()
    return spec, x, y, mask, t, old, adv


@pytest.mark.parametrize("softcap", [0.0, 4.0])
@pytest.mark.parametrize("extra", [0, oracle.RKL, oracle.FKL])
def test_gspo_gradient_vs_torch_autograd(softcap, extra):
    spec, x, y, mask, t, old, adv = _gspo_case(softcap=softcap)
    spec.flags |= extra
    _, grad = oracle.forward_backward(spec, x, y, mask, t, old, adv, seq_offsets=GSPO_OFFSETS)
    ref = _torch_total(spec, x, y, mask, t, old, adv, offsets=GSPO_OFFSETS)
    np.testing.assert_allclose(grad, ref, atol=1e-15, rtol=1e-10)


def test_gspo_one_token_segments_equal_grpo():
    rng = _rng(12)
    N, V = 11, 17
    x = rng.normal(0, 2.0, size=(N, V))
    y = rng.integers(0, V, size=N)
    y[3] = -100
    mask = np.ones(N, dtype=np.uint8)
    mask[7] = 0
    base = dict(V=V, w_ce=0.4, w_z=0.1, w_grpo=1.0, grad_scale=0.7, eps=0.2)
    sp_g = Spec(flags=oracle.CE | oracle.ZLOSS | oracle.GRPO, **base)
    sp_s = Spec(flags=oracle.CE | oracle.ZLOSS | oracle.GSPO, **base)
    old, adv = _grpo_inputs(rng, x, y, sp_g, spread=0.4)
    sc_g, g_g = oracle.forward_backward(sp_g, x, y, mask, None, old, adv)
    sc_s, g_s = oracle.forward_backward(sp_s, x, y, mask, None, old, adv, seq_offsets=np.arange(N + 1))
    assert sc_g[SLOT["CLIPFRAC"]] > 0            # the case exercises the clip
    np.testing.assert_allclose(sc_s, sc_g, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(g_s, g_g, rtol=1e-12, atol=1e-16)


def test_gspo_ratio_one_closed_forms():
    spec, x, y, mask, t, old, adv = _gspo_case(flags=oracle.GSPO)
    spec.w_ce = 0.0
    vals = ho.row_values(spec, x, y)
    old = vals["logp"].copy()                     # every sequence ratio is 1
    sc, grad = oracle.forward_backward(spec, x, y, mask, None, old, adv, seq_offsets=GSPO_OFFSETS)
    valid, _ = ho.row_validity(len(y), spec.V, y, mask)
    seg_adv, counts = [], []
    for i in range(len(GSPO_OFFSETS) - 1):
        rows = [r for r in range(GSPO_OFFSETS[i], GSPO_OFFSETS[i + 1]) if valid[r]]
        if rows:
            seg_adv.append(adv[rows[0]])
            counts.append((rows, len(rows)))
    n_seg = len(seg_adv)
    assert n_seg == 4                             # the empty segment does not count
    assert sc[SLOT["RATIO"]] == pytest.approx(1.0, abs=1e-15)
    assert sc[SLOT["CLIPFRAC"]] == 0.0
    assert sc[SLOT["KL_OLD_NEW"]] == pytest.approx(0.0, abs=1e-15)
    assert sc[SLOT["GRPO"]] == pytest.approx(-np.mean(seg_adv), abs=1e-14)
    assert sc[SLOT["ADV_MEAN"]] == pytest.approx(np.mean(seg_adv), abs=1e-14)
    # gradient = -(A_i / (n_i n_seg)) (onehot(y) - q) times the chain factor k
    q = vals["q"]
    expect = np.zeros_like(x)
    for (rows, n_i), A in zip(counts, seg_adv):
        for r in rows:
            oh = np.zeros(spec.V)
            oh[y[r]] = 1.0
            expect[r] = -spec.grad_scale * spec.w_grpo * A / (n_i * n_seg) * (oh - q[r]) * spec.logit_scale
    np.testing.assert_allclose(grad, expect, atol=1e-16, rtol=1e-12)


def test_gspo_sequence_ratio_and_clip_closed_forms():
    spec, x, y, mask, t, old, adv = _gspo_case(flags=oracle.GSPO)
    vals = ho.row_values(spec, x, y)
    valid, _ = ho.row_validity(len(y), spec.V, y, mask)
    # segment [0, 3): token log-ratios 0.1, 0.3, 0.5 -> s = e^0.3 > 1 + eps
    old = vals["logp"].copy()
    old[0:3] = vals["logp"][0:3] - np.array([0.1, 0.3, 0.5])
    adv[0:3] = 2.0
    seam = ho.gspo_seam(spec, vals["logp"], old, adv, valid, GSPO_OFFSETS)
    assert seam["ratio"][0] == pytest.approx(math.exp(0.3), rel=1e-14)
    assert seam["loss"][0] == pytest.approx(-(1.0 + spec.eps) * 2.0, rel=1e-14)
    assert not seam["active"][0] and seam["clipped"][0]
    _, grad = oracle.forward_backward(spec, x, y, mask, None, old, adv, seq_offsets=GSPO_OFFSETS)
    assert np.all(grad[0:3] == 0.0)               # clipped with A > 0: no gradient
    assert np.abs(grad[5:7]).max() > 0            # other segments still flow
    # the same log-ratios with A < 0 flow through the unclipped term
    adv[0:3] = -2.0
    _, grad = oracle.forward_backward(spec, x, y, mask, None, old, adv, seq_offsets=GSPO_OFFSETS)
    assert np.abs(grad[0:3]).max() > 0


def test_gspo_finite_differences():
    spec, x, y, mask, t, old, adv = _gspo_case(seed=13, N=8, V=7, spread=0.1,
                                                flags=oracle.CE | oracle.GSPO | oracle.RKL)
    offsets = [0, 2, 2, 5, 8]
    mask[:] = 1
    mask[3] = 0
    y[4] = 1
    _, grad = oracle.forward_backward(spec, x, y, mask, t, old, adv, seq_offsets=offsets)
    h = 1e-6
    fd = np.zeros_like(x)
    for i in range(x.shape[0]):
        for j in range(x.shape[1]):
            xp = x.copy()
            xp[i, j] += h
            xm = x.copy()
            xm[i, j] -= h
            fp = oracle.total_loss(spec, xp, y, mask, t, old, adv, seq_offsets=offsets)
            fm = oracle.total_loss(spec, xm, y, mask, t, old, adv, seq_offsets=offsets)
            fd[i, j] = (fp - fm) / (2 * h)
    np.testing.assert_allclose(grad, fd, atol=2e-8, rtol=0)
    assert np.all(grad[3] == 0.0)


def test_gspo_all_masked_and_bad_offsets():
    spec, x, y, mask, t, old, adv = _gspo_case(flags=oracle.GSPO)
    mask[:] = 0
    sc, grad = oracle.forward_backward(spec, x, y, mask, None, old, adv, seq_offsets=GSPO_OFFSETS)
    assert np.all(sc[:11] == 0.0) and np.all(grad == 0.0)
    for bad in ([1, 13], [0, 12], [0, 5, 4, 13], [0]):
        with pytest.raises(ValueError):
            oracle.forward_backward(spec, x, y, None, None, old, adv, seq_offsets=bad)
    with pytest.raises(ValueError):
        oracle.forward_backward(Spec(V=spec.V, flags=oracle.GRPO | oracle.GSPO), x, y, None, None,
                                old, adv, seq_offsets=GSPO_OFFSETS)


# ---------------------------------------------------------------------------
# Planted mistakes: each mutation of the oracle must be caught by a pin above
# ---------------------------------------------------------------------------
def _mutant_total_grad_fails(monkeypatch, target, replacement):
    monkeypatch.setattr(ho, target, replacement)
    try:
        for mode in ("fkl", "rkl"):
            for sc in (0.0, 4.0):
                test_total_gradient_vs_torch_autograd(mode, sc)
    except AssertionError:
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    orig_grads = ho.loss_gradients_wrt_s
    orig_deriv = ho.transform_derivative
    orig_values = ho.row_values

    def wrong_rkl_sign(spec, vals):
        g = orig_grads(spec, vals)
        if "distill" in g and spec.has(oracle.RKL):
            g["distill"] = vals["q"] * (vals["logq"] - vals["logp_t"] + vals["rkl"][:, None])
        return g

    def dropped_z_factor(spec, vals):
        g = orig_grads(spec, vals)
        if "z" in g:
            g["z"] = vals["lse"][:, None] * vals["q"]
        return g

    def wrong_label_index(spec, vals):
        vals = dict(vals)
        vals["y"] = (vals["y"] + 1) % vals["q"].shape[1]
        return orig_grads(spec, vals)

    def chain_without_tanh(x, spec):
        return np.full_like(np.asarray(x, dtype=np.float64), spec.logit_scale)

    def grpo_always_active(spec, *a, **k):
        v = orig_values(spec, *a, **k)
        if "grpo_active" in v:
            v["grpo_active"] = np.ones_like(v["grpo_active"])
        return v

    for target, repl in (("loss_gradients_wrt_s", wrong_rkl_sign),
                         ("loss_gradients_wrt_s", dropped_z_factor),
                         ("loss_gradients_wrt_s", wrong_label_index),
                         ("transform_derivative", chain_without_tanh)):
        assert _mutant_total_grad_fails(monkeypatch, target, repl), target
        monkeypatch.setattr(ho, "loss_gradients_wrt_s", orig_grads)
        monkeypatch.setattr(ho, "transform_derivative", orig_deriv)

    monkeypatch.setattr(ho, "row_values", grpo_always_active)
    with pytest.raises(AssertionError):
        test_finite_differences_clipped_grpo_tokens()
    monkeypatch.setattr(ho, "row_values", orig_values)


def test_gspo_planted_mistakes_are_caught(monkeypatch):
    orig = ho.gspo_seam

    def per_token_mean_ratio(spec, logp, old, A, valid, offsets):
        # mean of the token ratios instead of the exponential of the mean log-ratio
        out = orig(spec, logp, old, A, valid, offsets)
        seg = out["segment"]
        r_tok = np.exp(np.asarray(logp) - np.asarray(old))
        for i in np.nonzero(out["nonempty"])[0]:
            rows = (seg == i) & np.asarray(valid)
            r = r_tok[rows].mean()
            d = -out["adv"][i] * r / (rows.sum() * out["n_seg"]) if out["active"][i] else 0.0
            out["dlogp"][rows] = d
        return out

    def no_length_norm(spec, logp, old, A, valid, offsets):
        out = orig(spec, logp, old, A, valid, offsets)
        out["dlogp"] = out["dlogp"] * np.take(out["n_tokens"], out["segment"])
        return out

    def token_count_divisor(spec, logp, old, A, valid, offsets):
        out = orig(spec, logp, old, A, valid, offsets)
        out["dlogp"] = out["dlogp"] * out["n_seg"] / max(int(np.asarray(valid).sum()), 1)
        return out

    for mutant in (per_token_mean_ratio, no_length_norm, token_count_divisor):
        monkeypatch.setattr(ho, "gspo_seam", mutant)
        with pytest.raises(AssertionError):
            test_gspo_gradient_vs_torch_autograd(0.0, 0)
    monkeypatch.setattr(ho, "gspo_seam", orig)
