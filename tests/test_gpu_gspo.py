"""GPU parity of the GSPO path against the fp64 oracle.

The path behind hl_forward_backward_segments: the fused kernel in
forward-only mode (row statistics), the segment step (sequence ratios and
per-token label-column coefficients) and the fused kernel again in load mode
(statistics read back, slice reloaded, gradient written), as in the GSPO case
of Fast-LLM PR #558 (section Design).

Tolerances are those of the other parity tests (fp32: scalars 1e-5 relative,
gradient 1e-6 absolute; bf16: scalars 1e-4 relative, gradient rms-relative
4e-3 over the tensor and over its non-label entries; fp16 as bf16 with a
1e-3 gradient gate). A segment whose sequence ratio lies within 1e-5 of
1 +/- eps may take either clip branch (both sides decide in floating point);
its rows are left out of the gradient comparison and the clip count.
"""

import numpy as np
import pytest
import torch

import lm_head_vocab_amd as hl
import oracle
import workloads
from gpu_support import (TOL, assert_scalars, grad_check, make_plan, oracle_old_logprobs, say,
                         spec_from, to_np, torch_old_logprobs)
from oracle import SLOT

pytestmark = pytest.mark.gpu
DEV = "cuda"
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
INT_VIEW = {"f32": torch.int32, "bf16": torch.int16, "f16": torch.int16}
F16_LOSS_SCALE = 1024.0

CE, Z, FKL, RKL, FDCE, GRPO, GSPO, ENT, ACC = (oracle.CE, oracle.ZLOSS, oracle.FKL, oracle.RKL, oracle.FDCE,
                                               oracle.GRPO, oracle.GSPO, oracle.ENTROPY, oracle.ACCUMULATE)
DISTILL = FKL | RKL | FDCE

COMBOS = {
    "gspo": (GSPO, dict(ce=0.0, grpo=1.0)),
    "gspo_z_ent": (GSPO | Z | ENT, dict(ce=0.0, z=0.01, grpo=1.0)),
    "all_gspo_rkl": (CE | Z | RKL | GSPO | ENT, dict(ce=1.0, z=1e-3, distill=0.5, grpo=1.0, grad_scale=0.25)),
    "all_gspo_fkl": (CE | Z | FKL | GSPO | ENT, dict(ce=0.7, z=1e-2, distill=0.9, grpo=0.6, grad_scale=2.0)),
    "ce_gspo_fdce": (CE | FDCE | GSPO, dict(ce=0.5, distill=1.0, grpo=1.3)),
    "all_gspo_rkl_h": (CE | Z | RKL | GSPO | ENT | oracle.HINTON,
                       dict(ce=1.0, z=1e-3, distill=0.5, grpo=1.0, grad_scale=0.25)),
}
SHAPES = [(37, 1000), (16, 4099), (9, 33000), (5, 3), (3, 1), (64, 300)]


def _segment_index(offs, N):
    o = offs.tolist()
    seg = np.zeros(N, dtype=np.int64)
    for i in range(len(o) - 1):
        seg[o[i]:o[i + 1]] = i
    return seg


def _case(dtype, combo, N, V, seed, softcap=0.0, scale=1.0, accumulate=False, mask_frac=0.15,
          broadcast_adv=True, max_len=8, eps=0.2, offsets=None, **gen):
    flags, w = COMBOS[combo]
    if dtype == "f16":
        w = dict(w, grad_scale=w.get("grad_scale", 1.0) * F16_LOSS_SCALE)
    if accumulate:
        flags |= ACC
    spec = spec_from(V, flags, w, temperature=1.5, eps=eps, logit_scale=scale, softcap=softcap)
    inp = workloads.small_inputs(N, V, dtype, "cpu", seed, teacher=bool(flags & DISTILL), grpo=True,
                                 accumulate=accumulate, mask_frac=mask_frac, **gen)
    offs = workloads.segment_offsets(N, seed + 1, max_len=max_len) if offsets is None \
        else torch.tensor(offsets, dtype=torch.int32)
    if broadcast_adv and N:
        # one advantage per sequence, repeated over its tokens
        seg = torch.from_numpy(_segment_index(offs, N))
        inp["advantages"] = inp["advantages"][seg].contiguous()
    inp["old_logprobs"] = oracle_old_logprobs(spec, inp["logits"], inp["labels"], inp["old_noise"])
    inp["seq_offsets"] = offs
    return spec, inp


def _run(plan, inp, grad_mode):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    x = d["logits"]
    grad = None
    if grad_mode == "overwrite":
        grad = torch.full_like(x, float("nan"))
    elif grad_mode == "accumulate":
        grad = d["grad_init"].clone()
    sc = plan(x, labels=d["labels"], mask=d["mask"], teacher=d["teacher"], old_logprobs=d["old_logprobs"],
              advantages=d["advantages"], grad=grad, seq_offsets=d["seq_offsets"])
    torch.cuda.synchronize()
    return sc.cpu().double().numpy(), grad


def _oracle(spec, inp, want_grad=True):
    y = to_np(inp["labels"]).astype(np.int64)
    args = dict(labels=y, mask=to_np(inp["mask"]), teacher=to_np(inp["teacher"]),
                old_logprobs=to_np(inp["old_logprobs"]), advantages=to_np(inp["advantages"]),
                grad_in=to_np(inp["grad_init"]) if spec.has(ACC) else None, want_grad=want_grad,
                seq_offsets=inp["seq_offsets"].numpy())
    sc, g = oracle.forward_backward(spec, to_np(inp["logits"]), **args)
    x = to_np(inp["logits"])
    N = x.shape[0]
    valid, _ = oracle.row_validity(N, spec.V, y, args["mask"])
    vals = oracle.row_values(spec, x, y, args["teacher"])
    seam = oracle.gspo_seam(spec, vals["logp"] if N else np.zeros(0), args["old_logprobs"],
                            args["advantages"], valid, args["seq_offsets"])
    return sc, g, vals, valid, seam


def _boundary_rows(spec, seam, valid):
    r = seam["ratio"]
    near = (np.abs(r - (1 + spec.eps)) < 1e-5) | (np.abs(r - (1 - spec.eps)) < 1e-5)
    near &= seam["nonempty"]
    return near[seam["segment"]] & valid, bool(near.any())


def _scalar_vals(vals, seam):
    """Per-row view of the segment values, used only to scale near-zero slots."""
    seg = seam["segment"]
    out = dict(vals)
    out["grpo"] = seam["loss"][seg]
    out["adv"] = seam["adv"][seg]
    out["k3"] = seam["k3"][seg]
    return out


def _check(spec, inp, dtype, chunks=0, grad_mode=None, variant=None):
    grad_mode = grad_mode or ("accumulate" if spec.has(ACC) else "overwrite")
    plan = make_plan(spec, TDT[dtype], chunks)
    if variant is not None:
        plan.set_variant(*variant)
    N = inp["logits"].shape[0]
    say(f"[gpu] gspo N={N} V={spec.V} S={inp['seq_offsets'].numel() - 1} {dtype} flags={spec.flags:#x} "
        f"{plan.describe()} grad={grad_mode}")
    sc, g = _run(plan, inp, grad_mode)
    ref_sc, ref_g, vals, valid, seam = _oracle(spec, inp, want_grad=grad_mode != "none")
    boundary, any_boundary = _boundary_rows(spec, seam, valid) if N else (np.zeros(0, bool), False)
    assert_scalars(spec, sc, ref_sc, dtype, _scalar_vals(vals, seam) if N else None, valid, x=to_np(inp["logits"]),
                   skip=("CLIPFRAC",) if any_boundary else ())
    if not any_boundary:
        ns = seam["n_seg"]
        assert round(sc[SLOT["CLIPFRAC"]] * ns) == round(ref_sc[SLOT["CLIPFRAC"]] * ns)
    if grad_mode == "none":
        return plan, sc, None, seam, valid
    gk = g.detach().cpu()
    keep = ~boundary
    metrics = grad_check(gk[torch.from_numpy(keep)], ref_g[keep], dtype,
                         labels=to_np(inp["labels"])[keep])
    inval = torch.from_numpy(~valid)
    if grad_mode == "overwrite":
        assert torch.equal(gk[inval].view(INT_VIEW[dtype]), torch.zeros_like(gk[inval]).view(INT_VIEW[dtype]))
    else:
        assert torch.equal(gk[inval], inp["grad_init"][inval])
    return plan, sc, metrics, seam, valid


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{n}x{v}" for n, v in SHAPES])
@pytest.mark.parametrize("combo", list(COMBOS))
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_gspo_small_parity(dtype, combo, shape):
    N, V = shape
    spec, inp = _case(dtype, combo, N, V, seed=13 * N + V, bad_labels=1 if N > 4 else 0,
                      mask_frac=0.15 if N > 8 else 0.0)
    _check(spec, inp, dtype)


@pytest.mark.parametrize("combo", ["gspo_z_ent", "all_gspo_rkl", "all_gspo_fkl", "ce_gspo_fdce"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_gspo_softcap_scale_and_accumulate(dtype, combo):
    spec, inp = _case(dtype, combo, 24, 2053, seed=7, softcap=7.0, scale=0.5, broadcast_adv=False)
    _check(spec, inp, dtype)
    spec, inp = _case(dtype, combo, 19, 20011, seed=3, accumulate=True, mask_frac=0.2, softcap=30.0, scale=0.5)
    _check(spec, inp, dtype)


@pytest.mark.parametrize("chunks", [2, 4])
@pytest.mark.parametrize("combo", ["gspo_z_ent", "all_gspo_rkl", "ce_gspo_fdce"])
def test_gspo_split_vocab_forward(combo, chunks):
    spec, inp = _case("bf16", combo, 12, 60013, seed=50 + chunks, softcap=15.0, scale=0.8, mask_frac=0.2)
    _check(spec, inp, "bf16", chunks=chunks)


@pytest.mark.parametrize("chunks", [4, 8])
@pytest.mark.parametrize("V", [13, 41])
@pytest.mark.parametrize("combo", ["gspo_z_ent", "all_gspo_rkl", "ce_gspo_fdce"])
def test_gspo_split_vocab_short_rows(combo, V, chunks):
    """Load mode on rows with more chunks than 16-byte body vectors (empty
    chunks, head and tail on chunk 0), with and without a teacher."""
    spec, inp = _case("bf16", combo, 14, V, seed=V + chunks, mask_frac=0.2)
    _check(spec, inp, "bf16", chunks=chunks)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gspo_one_token_segments_match_grpo(dtype):
    """With one token per segment the sequence ratio is the token ratio: GSPO
    and GRPO give the same scalars and gradient (through different kernels)."""
    N, V = 40, 5003
    spec, inp = _case(dtype, "gspo_z_ent", N, V, seed=77, offsets=list(range(N + 1)), mask_frac=0.2)
    plan_s, sc_s, _, _, valid = _check(spec, inp, dtype)
    spec_g = spec_from(V, GRPO | Z | ENT, dict(ce=0.0, z=0.01, grpo=1.0), eps=spec.eps)
    plan_g = make_plan(spec_g, TDT[dtype])
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    g_g = torch.full_like(d["logits"], float("nan"))
    sc_g = plan_g(d["logits"], labels=d["labels"], mask=d["mask"], old_logprobs=d["old_logprobs"],
                  advantages=d["advantages"], grad=g_g).cpu().double().numpy()
    _, g_s = _run(plan_s, inp, "overwrite")
    for name in ("GRPO", "NEWLOGP", "RATIO", "CLIPFRAC", "KL_OLD_NEW", "ADV_MEAN", "Z", "ENTROPY", "TOTAL"):
        a, b = sc_s[SLOT[name]], sc_g[SLOT[name]]
        assert abs(a - b) <= TOL[dtype]["scalar_rel"] * max(abs(b), 1e-2), (name, a, b)
    ref_g = g_g.cpu().double().numpy()
    if dtype == "f32":
        assert np.max(np.abs(g_s.cpu().double().numpy() - ref_g)) <= 1e-6
    else:
        grad_check(g_s.cpu(), ref_g, dtype, labels=to_np(inp["labels"]))


@pytest.mark.parametrize("chunks", [0, 3])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gspo_per_token_values(dtype, chunks):
    """Per-token outputs: new log-prob per token; the policy columns hold the
    token's segment loss, sequence ratio, clip flag, k3 and advantage."""
    spec, inp = _case(dtype, "all_gspo_rkl", 45, 20011, seed=41 + chunks, mask_frac=0.2, bad_labels=2,
                      softcap=9.0, scale=0.7, broadcast_adv=False)
    plan, _, _, seam, valid = _check(spec, inp, dtype, chunks=chunks, grad_mode="none")
    rv = plan.row_values().cpu().double().numpy()
    _, _, vals, _, _ = _oracle(spec, inp, want_grad=False)
    seg = seam["segment"]
    np.testing.assert_array_equal(rv[:, 10], valid.astype(float))
    assert np.all(rv[~valid] == 0.0)
    rel = TOL[dtype]["scalar_rel"]
    for key, col, ref_all in (("logp", 4, vals["logp"]), ("grpo", 3, seam["loss"][seg]),
                              ("ratio", 5, seam["ratio"][seg]), ("k3", 7, seam["k3"][seg]),
                              ("adv", 8, seam["adv"][seg])):
        ref = ref_all[valid]
        got = rv[valid, col]
        scale = np.maximum(np.abs(ref), 1e-2 * max(1.0, float(np.max(np.abs(ref)))))
        err = float(np.max(np.abs(got - ref) / scale))
        assert err <= rel, (key, err)
    boundary, _ = _boundary_rows(spec, seam, valid)
    keep = valid & ~boundary
    np.testing.assert_array_equal(rv[keep, 6] != 0, seam["clipped"][seg][keep])


def test_gspo_forward_only_and_determinism():
    spec, inp = _case("bf16", "all_gspo_fkl", 33, 40000, seed=8, accumulate=True, softcap=20.0)
    plan, sc_fo, _, _, _ = _check(spec, inp, "bf16", grad_mode="none")
    sc1, g1 = _run(plan, inp, "accumulate")
    sc2, g2 = _run(plan, inp, "accumulate")
    np.testing.assert_array_equal(sc1, sc2)
    np.testing.assert_array_equal(sc_fo, sc1)
    assert torch.equal(g1.view(torch.int16), g2.view(torch.int16))


@pytest.mark.parametrize("case", [("bf16", "all_gspo_rkl", 737_288), ("f32", "gspo_z_ent", 737_284)],
                         ids=["bf16-rkl-737288", "f32-z-737284"])
def test_gspo_rows_past_every_exchanged_slice(case):
    """GSPO on rows longer than any slice the chunk exchange serves: the same
    streamed forward and segment step, then a load-mode backward with more
    chunks than the exchange allows."""
    dtype, combo, V = case
    spec, inp = _case(dtype, combo, 9, V, seed=V % 991, bad_labels=1, max_len=4)
    plan, _, _, _, _ = _check(spec, inp, dtype)
    d = plan.describe()
    assert d["block"] == 1024 and d["chunks"] > 9


def test_gspo_changing_batches_and_segments():
    """One plan, calls with different row and segment counts."""
    spec, _ = _case("bf16", "all_gspo_rkl", 4, 30011, seed=1)
    plan = make_plan(spec, torch.bfloat16)
    for i, (N, max_len) in enumerate(((20, 6), (7, 3), (33, 40), (12, 1), (5, 9))):
        _, inp = _case("bf16", "all_gspo_rkl", N, 30011, seed=200 + i, max_len=max_len, mask_frac=0.2)
        say(f"[gpu] gspo changing batch N={N} S={inp['seq_offsets'].numel() - 1}")
        sc, g = _run(plan, inp, "overwrite")
        ref_sc, ref_g, vals, valid, seam = _oracle(spec, inp)
        boundary, any_b = _boundary_rows(spec, seam, valid)
        assert_scalars(spec, sc, ref_sc, "bf16", _scalar_vals(vals, seam), valid,
                       skip=("CLIPFRAC",) if any_b else ())
        keep = ~boundary
        grad_check(g.cpu()[torch.from_numpy(keep)], ref_g[keep], "bf16", labels=to_np(inp["labels"])[keep])


def test_gspo_malformed_offsets_make_results_nan_and_the_plan_recovers():
    """Offsets are checked on the device: a decreasing offset or a last offset
    short of n_rows turns every float scalar and every valid row's gradient
    into NaN; masked rows still read +0.0; the next good call is exact."""
    N, V = 16, 2000
    spec, inp = _case("f32", "gspo_z_ent", N, V, seed=90, mask_frac=0.25, offsets=[0, 4, 9, N])
    plan = make_plan(spec, torch.float32)
    _, _, _, _, valid = _check(spec, inp, "f32")
    for bad in ([0, 9, 4, N], [0, 4, 9, N - 1], [1, 4, 9, N]):
        bad_inp = dict(inp, seq_offsets=torch.tensor(bad, dtype=torch.int32))
        say(f"[gpu] malformed offsets {bad}")
        sc, g = _run(plan, bad_inp, "overwrite")
        assert np.all(np.isnan(sc[:11])), sc
        gk = g.cpu()
        assert torch.isnan(gk[torch.from_numpy(valid)]).all()
        assert torch.count_nonzero(gk[torch.from_numpy(~valid)].view(torch.int32)).item() == 0
    sc, g = _run(plan, inp, "overwrite")
    ref_sc, ref_g, _, _, _ = _oracle(spec, inp)
    assert not np.any(np.isnan(sc))
    assert np.max(np.abs(g.cpu().double().numpy() - ref_g)) <= 1e-6


def test_gspo_empty_batch_and_all_masked():
    spec = spec_from(100, GSPO | Z, dict(ce=0.0, z=0.1, grpo=1.0))
    plan = make_plan(spec, torch.bfloat16)
    say("[gpu] gspo empty batch")
    e = torch.empty(0, dtype=torch.float32, device=DEV)
    sc = plan(torch.empty(0, 100, dtype=torch.bfloat16, device=DEV),
              labels=torch.empty(0, dtype=torch.int64, device=DEV), old_logprobs=e, advantages=e,
              seq_offsets=torch.zeros(1, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert torch.all(sc.cpu() == 0)
    spec, inp = _case("bf16", "all_gspo_rkl", 10, 777, seed=1, ignore_frac=1.0)
    _check(spec, inp, "bf16")


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_gspo_load_mode_with_lds_held_slices(dtype, accumulate):
    """The reloading backward of a Hinton GSPO call on slices of 9 register
    vectors plus 4 LDS vectors per tensor (2 chunks x 512 threads at
    V = 100001): the LDS slots are read in pass 2 without a pass 1."""
    spec, inp = _case(dtype, "all_gspo_rkl_h", 12, 100001, seed=29 + accumulate, accumulate=accumulate,
                      mask_frac=0.2)
    plan, _, _, _, _ = _check(spec, inp, dtype, variant=(2, 512))
    d = plan.describe()
    assert (d["chunks"], d["block"], d["vec_per_thread"]) == (2, 512, 13)
