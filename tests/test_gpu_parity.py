"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small batches are compared element by element, at sizes that span several
workgroup tiles and ragged row tails; the full benchmark configurations are
compared row by row in test_gpu_full_configs.py.

Tolerances: fp32 inputs, scalars 1e-5 relative and gradient 1e-6 absolute;
bf16 inputs, scalars 1e-4 relative and gradient rms-relative 4e-3 over the
tensor and over its non-label entries. Slots whose batch mean can sit at or
near zero (distillation KL, GRPO objective and statistics, the total) are
measured against max(|mean|, mean |per-row value|, 1e-2). A GRPO token
whose ratio lies within 1e-5 of 1 +/- eps may take either branch (both
sides decide in floating point); such rows are excluded from the gradient
and clip-count comparisons.
"""

import numpy as np
import pytest
import torch

import lm_head_vocab_amd as hl
import oracle
import workloads
from gpu_support import (TOL, assert_scalars, grad_check, make_plan, max_chunks, oracle_old_logprobs,
                         run_hip, run_oracle, say, spec_from, to_np, torch_old_logprobs)
from oracle import SLOT

pytestmark = pytest.mark.gpu
DEV = "cuda"
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
INT_VIEW = {"f32": torch.int32, "bf16": torch.int16, "f16": torch.int16}
# fp16 gradients of small softmax entries sit below fp16's normal range; the
# fp16 cases use a loss scale (grad_scale) of 1024, as fp16 training does.
F16_LOSS_SCALE = 1024.0

CE, Z, FKL, RKL, GRPO, ENT, ACC = (oracle.CE, oracle.ZLOSS, oracle.FKL, oracle.RKL, oracle.GRPO,
                                   oracle.ENTROPY, oracle.ACCUMULATE)
FDCE = oracle.FDCE
HINTON = oracle.HINTON
DISTILL = FKL | RKL | FDCE

COMBOS = {
    "ce": (CE, dict(ce=1.0)),
    "ce_z": (CE | Z, dict(ce=1.0, z=0.1)),
    "z_ent": (Z | ENT, dict(ce=0.0, z=1.0)),
    "grpo_z_ent": (GRPO | Z | ENT, dict(ce=0.0, z=0.01, grpo=1.0)),
    "ce_fkl": (CE | FKL, dict(ce=0.5, distill=1.0)),
    "ce_rkl": (CE | RKL, dict(ce=0.5, distill=1.0)),
    "fkl_ent": (FKL | ENT, dict(ce=0.0, distill=1.0)),
    "all_rkl": (CE | Z | RKL | GRPO | ENT, dict(ce=1.0, z=1e-3, distill=0.5, grpo=1.0, grad_scale=0.25)),
    "all_fkl": (CE | Z | FKL | GRPO | ENT, dict(ce=0.7, z=1e-2, distill=0.9, grpo=0.6, grad_scale=2.0)),
    "ce_fdce": (CE | FDCE, dict(ce=0.5, distill=1.0)),
    "all_fdce": (CE | Z | FDCE | GRPO | ENT, dict(ce=0.3, z=1e-3, distill=1.1, grpo=0.8, grad_scale=0.5)),
    # Hinton temperature mode: tau on both softmaxes of the distillation term, times tau^2
    "ce_fkl_h": (CE | FKL | HINTON, dict(ce=0.5, distill=1.0)),
    "all_rkl_h": (CE | Z | RKL | GRPO | ENT | HINTON, dict(ce=1.0, z=1e-3, distill=0.5, grpo=1.0, grad_scale=0.25)),
    "all_fdce_h": (CE | Z | FDCE | GRPO | ENT | HINTON, dict(ce=0.3, z=1e-3, distill=1.1, grpo=0.8, grad_scale=0.5)),
}
HINTON_COMBOS = ["ce_fkl_h", "all_rkl_h", "all_fdce_h"]
# (N, V): aligned and ragged rows, tiny rows, both block sizes
SHAPES = [(37, 1000), (16, 4099), (9, 33000), (5, 3), (3, 1), (64, 300), (11, 2053)]


def _grpo_boundary_rows(spec, inp_cpu, eps_tol=1e-5):
    if not spec.has(GRPO):
        return np.zeros(inp_cpu["logits"].shape[0], dtype=bool)
    vals = oracle.row_values(spec, to_np(inp_cpu["logits"]), to_np(inp_cpu["labels"]).astype(np.int64),
                             None, to_np(inp_cpu["old_logprobs"]), to_np(inp_cpu["advantages"]))
    r = vals["ratio"]
    return (np.abs(r - (1 + spec.eps)) < eps_tol) | (np.abs(r - (1 - spec.eps)) < eps_tol)


def _small(dtype, combo, N, V, seed, softcap=0.0, scale=1.0, accumulate=False, temperature=1.5,
           logit_std=2.0, **gen):
    flags, w = COMBOS[combo]
    if dtype == "f16":
        w = dict(w, grad_scale=w.get("grad_scale", 1.0) * F16_LOSS_SCALE)
    if accumulate:
        flags |= ACC
    spec = spec_from(V, flags, w, temperature=temperature, eps=0.2, logit_scale=scale, softcap=softcap)
    inp = workloads.small_inputs(N, V, dtype, "cpu", seed, teacher=bool(flags & DISTILL),
                                 grpo=bool(flags & GRPO), accumulate=accumulate,
                                 logit_std=logit_std, **gen)
    if flags & GRPO:
        inp["old_logprobs"] = oracle_old_logprobs(spec, inp["logits"], inp["labels"], inp["old_noise"])
    return spec, inp


def _to_dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def _check_small(spec, inp, dtype, chunks=0, grad_mode=None, skip_scalars=()):
    grad_mode = grad_mode or ("accumulate" if spec.has(ACC) else "overwrite")
    plan = make_plan(spec, TDT[dtype], chunks)
    say(f"[gpu] N={inp['logits'].shape[0]} V={spec.V} {dtype} flags={spec.flags:#x} "
        f"chunks={plan.describe()} grad={grad_mode}")
    sc, g = run_hip(plan, _to_dev(inp), grad_mode)
    ref_sc, ref_g, _ = run_oracle(spec, inp, want_grad=grad_mode != "none")
    vals = oracle.row_values(spec, to_np(inp["logits"]),
                             to_np(inp["labels"]).astype(np.int64) if inp["labels"] is not None else None,
                             to_np(inp["teacher"]), to_np(inp.get("old_logprobs")), to_np(inp.get("advantages")))
    valid, _ = oracle.row_validity(inp["logits"].shape[0], spec.V,
                                   to_np(inp["labels"]).astype(np.int64) if inp["labels"] is not None else None,
                                   to_np(inp["mask"]))
    boundary = _grpo_boundary_rows(spec, inp) & valid
    assert_scalars(spec, sc, ref_sc, dtype, vals, valid,
                   skip=tuple(skip_scalars) + (("CLIPFRAC",) if boundary.any() else ()), x=to_np(inp["logits"]))
    if spec.has(GRPO) and not boundary.any():
        n = ref_sc[SLOT["N_VALID"]] if spec.divisor <= 0 else spec.divisor
        assert round(sc[SLOT["CLIPFRAC"]] * n) == round(ref_sc[SLOT["CLIPFRAC"]] * n)
    if grad_mode == "none":
        return plan, sc, None
    gk = g.detach().cpu()
    keep = ~boundary
    metrics = grad_check(gk[torch.from_numpy(keep)], ref_g[keep], dtype,
                         labels=to_np(inp["labels"])[keep] if inp["labels"] is not None else None)
    # masked rows: +0.0 in overwrite mode, bit-identical existing values in accumulate mode
    inval = torch.from_numpy(~valid)
    if grad_mode == "overwrite":
        assert torch.equal(gk[inval].view(INT_VIEW[dtype]), torch.zeros_like(gk[inval]).view(INT_VIEW[dtype]))
    else:
        assert torch.equal(gk[inval], inp["grad_init"][inval])
    return plan, sc, metrics


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{n}x{v}" for n, v in SHAPES])
@pytest.mark.parametrize("combo", list(COMBOS))
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_small_parity(dtype, combo, shape):
    N, V = shape
    spec, inp = _small(dtype, combo, N, V, seed=11 * N + V, bad_labels=1 if N > 4 else 0,
                       mask_frac=0.15 if N > 8 else 0.0)
    _check_small(spec, inp, dtype)


@pytest.mark.parametrize("logit_std", [2.0, 40.0], ids=["poly", "exp_branch"])
@pytest.mark.parametrize("combo", ["ce_z", "all_rkl", "all_fkl", "grpo_z_ent", "all_fdce"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_softcap_and_scale(dtype, combo, logit_std):
    spec, inp = _small(dtype, combo, 24, 2053, seed=7, softcap=7.0, scale=0.5, logit_std=logit_std)
    _check_small(spec, inp, dtype)


@pytest.mark.parametrize("combo", ["ce_z", "all_rkl", "all_fkl", "z_ent", "all_fdce"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("V", [1000, 20011])
def test_accumulate(dtype, combo, V):
    spec, inp = _small(dtype, combo, 19, V, seed=3, accumulate=True, mask_frac=0.2, softcap=30.0, scale=0.5)
    _check_small(spec, inp, dtype)


@pytest.mark.parametrize("combo", ["ce_z", "all_rkl", "grpo_z_ent"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_only_matches_and_writes_nothing(dtype, combo):
    """Without a gradient the statistics come from the streaming kernel, with
    a different summation order than the register-resident fused kernel of a
    gradient call: the scalars agree to float rounding (2e-6 relative), and
    repeated forward-only calls agree bit for bit."""
    spec, inp = _small(dtype, combo, 21, 3001, seed=5)
    plan_fo, sc_fo, _ = _check_small(spec, inp, dtype, grad_mode="none")
    sc_fo2, _ = run_hip(plan_fo, _to_dev(inp), "none")
    np.testing.assert_array_equal(sc_fo, sc_fo2)
    plan = make_plan(spec, TDT[dtype])
    sc_full, _ = run_hip(plan, _to_dev(inp), "overwrite")
    np.testing.assert_allclose(sc_fo, sc_full, rtol=2e-6, atol=1e-7)


FWD_COMBOS = ["ce_z", "z_ent", "grpo_z_ent", "all_rkl", "all_fkl", "fkl_ent", "all_fdce_h"]
FWD_SHAPES = SHAPES + [(3, 300_007)]   # long ragged rows every fp32 teacher mode takes


@pytest.mark.parametrize("shape", FWD_SHAPES, ids=[f"{n}x{v}" for n, v in FWD_SHAPES])
@pytest.mark.parametrize("combo", FWD_COMBOS)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_forward_only_streaming(dtype, combo, shape):
    """Forward only: the streaming statistics kernel (one workgroup per row,
    double-buffered batches of 16-byte vectors, no chunk exchange) against the
    oracle, scalars and per-row values, on aligned, ragged, tiny and very long
    rows, with softcap on the reverse-KL combination."""
    N, V = shape
    spec, inp = _small(dtype, combo, N, V, seed=3 * N + V, softcap=15.0 if combo == "all_rkl" else 0.0,
                       bad_labels=1 if N > 4 else 0, mask_frac=0.2 if N > 8 else 0.0)
    plan, _, _ = _check_small(spec, inp, dtype, grad_mode="none")
    y = to_np(inp["labels"]).astype(np.int64)
    vals = oracle.row_values(spec, to_np(inp["logits"]), y, to_np(inp["teacher"]),
                             to_np(inp.get("old_logprobs")), to_np(inp.get("advantages")))
    valid, _ = oracle.row_validity(N, V, y, to_np(inp["mask"]))
    ok = valid & ~_grpo_boundary_rows(spec, inp)
    rows = plan.row_values().cpu().double().numpy()
    tol = TOL[dtype]["scalar_rel"]
    np.testing.assert_allclose(rows[ok, 0], vals["ce"][ok], rtol=tol, atol=tol)
    if spec.has(ENT):
        np.testing.assert_allclose(rows[ok, 9], vals["entropy"][ok], rtol=tol, atol=tol)
    for key, flag in (("fkl", FKL), ("rkl", RKL), ("fdce", FDCE)):
        if spec.has(flag):
            np.testing.assert_allclose(rows[ok, 2], vals[key][ok], rtol=tol, atol=tol)
    assert np.all(rows[~valid] == 0.0)


@pytest.mark.parametrize("chunks", [2, 3, 5, 9])
@pytest.mark.parametrize("combo", ["ce_z", "all_rkl", "all_fkl", "ce_fkl", "all_fdce"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_split_vocab_variant(dtype, combo, chunks):
    # forced chunking exercises the cross-workgroup combine at small sizes;
    # fp32 teacher slices hold at most 8 vectors per tensor, so the wider
    # fp32 rows are 60000 elements (two chunks of 1024 x 8 x 4); a count above
    # what the mode's exchange allows is taken at that maximum
    wide = 60000 if dtype == "f32" else 70000
    for V, N in ((20011, 7), (wide, 5)):
        spec, inp = _small(dtype, combo, N, V, seed=chunks * 100 + N, softcap=15.0, scale=0.8)
        _check_small(spec, inp, dtype, chunks=min(chunks, max_chunks(dtype, spec)))


@pytest.mark.parametrize("chunks", [2, 4, 8])
@pytest.mark.parametrize("V", [3, 13, 20, 41])
@pytest.mark.parametrize("combo", ["ce_fkl", "all_rkl", "all_fdce_h"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_vocab_short_rows(dtype, combo, V, chunks):
    """More chunks than 16-byte body vectors: some chunks of a row own no
    vector at all (their loads point at the workspace and every value is
    discarded), head and tail elements sit with chunk 0, and every row still
    merges all of its chunks."""
    spec, inp = _small(dtype, combo, 9, V, seed=V * 10 + chunks, mask_frac=0.2, softcap=6.0, scale=0.9)
    _check_small(spec, inp, dtype, chunks=min(chunks, max_chunks(dtype, spec)))


@pytest.mark.parametrize("variant", [(2, 512), (4, 512), (3, 1024), (1, 1024), (8, 256)])
@pytest.mark.parametrize("combo", ["ce_z", "all_rkl", "grpo_z_ent", "ce_fkl"])
def test_forced_variants(combo, variant):
    """Every (chunks, threads per workgroup) layout gives the same answer
    (each of these layouts has an instance at V = 60013; a layout without
    one is refused on the host, tested in test_abi)."""
    chunks, block = variant
    spec, inp = _small("bf16", combo, 6, 60013, seed=31 + chunks, softcap=12.0, scale=0.9, mask_frac=0.2)
    plan = make_plan(spec, torch.bfloat16)
    plan.set_variant(chunks, block)
    say(f"[gpu] variant {variant} -> {plan.describe()}")
    sc, g = run_hip(plan, _to_dev(inp), "overwrite")
    ref_sc, ref_g, _ = run_oracle(spec, inp)
    valid, _ = oracle.row_validity(6, spec.V, to_np(inp["labels"]).astype(np.int64), to_np(inp["mask"]))
    vals = oracle.row_values(spec, to_np(inp["logits"]), to_np(inp["labels"]).astype(np.int64),
                             to_np(inp["teacher"]), to_np(inp.get("old_logprobs")), to_np(inp.get("advantages")))
    assert_scalars(spec, sc, ref_sc, "bf16", vals, valid)
    grad_check(g.cpu(), ref_g, "bf16", labels=to_np(inp["labels"]))


@pytest.mark.parametrize("variant", [(5, 512), (7, 512), (8, 512), (9, 512)])
@pytest.mark.parametrize("combo", ["ce_fkl", "all_rkl", "all_fdce"])
def test_teacher_slice_layouts(combo, variant):
    """Teacher slices of 6, 8 and 10 vectors per thread at 512 threads, at a
    full-length vocabulary row."""
    chunks, block = variant
    spec, inp = _small("bf16", combo, 4, 151936, seed=61 + chunks, softcap=12.0, scale=0.9)
    plan = make_plan(spec, torch.bfloat16)
    plan.set_variant(chunks, block)
    say(f"[gpu] teacher layout {variant} -> {plan.describe()}")
    sc, g = run_hip(plan, _to_dev(inp), "overwrite")
    ref_sc, ref_g, _ = run_oracle(spec, inp)
    valid, _ = oracle.row_validity(4, spec.V, to_np(inp["labels"]).astype(np.int64), None)
    vals = oracle.row_values(spec, to_np(inp["logits"]), to_np(inp["labels"]).astype(np.int64),
                             to_np(inp["teacher"]), to_np(inp.get("old_logprobs")), to_np(inp.get("advantages")))
    assert_scalars(spec, sc, ref_sc, "bf16", vals, valid)
    grad_check(g.cpu(), ref_g, "bf16", labels=to_np(inp["labels"]))


@pytest.mark.parametrize("V, nvec", [(95003, 12), (100001, 13)])
@pytest.mark.parametrize("mode", ["overwrite", "accumulate"])
@pytest.mark.parametrize("combo", HINTON_COMBOS)
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_lds_held_slices(dtype, combo, mode, V, nvec):
    """Hinton slices of 9 register vectors plus 3 or 4 LDS vectors per tensor
    (two chunks of 512 threads, ragged rows): the LDS slots take part in both
    passes, the labels of rows 0 and 1 sit in the LDS part of chunk 0 and of
    chunk 1, and accumulate mode reads the old gradient beside them."""
    spec, inp = _small(dtype, combo, 8, V, seed=V % 997 + nvec, softcap=12.0, scale=0.9, temperature=2.0,
                       accumulate=mode == "accumulate", mask_frac=0.0, ignore_frac=0.0)
    half = -(-(V // 8) // 2)                       # body vectors per chunk (about)
    inp["labels"][0] = (9 * 512 + 700) * 8 + 3     # slot 9 of chunk 0
    inp["labels"][1] = (half + 11 * 512 + 5) * 8   # slot 11 of chunk 1
    if spec.flags & GRPO:
        inp["old_logprobs"] = oracle_old_logprobs(spec, inp["logits"], inp["labels"], inp["old_noise"])
    plan = make_plan(spec, TDT[dtype])
    plan.set_variant(2, 512)
    d = plan.describe()
    say(f"[gpu] LDS-held slice {dtype} {combo} {mode} V={V} -> {d}")
    assert (d["chunks"], d["block"], d["vec_per_thread"]) == (2, 512, nvec)
    sc, g = run_hip(plan, _to_dev(inp), mode)
    ref_sc, ref_g, _ = run_oracle(spec, inp)
    y = to_np(inp["labels"]).astype(np.int64)
    valid, _ = oracle.row_validity(8, spec.V, y, to_np(inp["mask"]))
    vals = oracle.row_values(spec, to_np(inp["logits"]), y, to_np(inp["teacher"]), to_np(inp.get("old_logprobs")),
                             to_np(inp.get("advantages")))
    assert_scalars(spec, sc, ref_sc, dtype, vals, valid)
    grad_check(g.cpu(), ref_g, dtype, labels=y)


@pytest.mark.parametrize("chunks", [0, 3])
@pytest.mark.parametrize("combo", ["all_rkl", "all_fkl", "all_fdce"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_per_token_values(dtype, combo, chunks):
    """hl_row_values: every per-token column (CE, z, KL, GRPO objective, new
    log-prob, ratio, clip flag, k3, advantage, entropy, valid) row by row."""
    spec, inp = _small(dtype, combo, 29, 20011, seed=41 + chunks, mask_frac=0.2, bad_labels=2,
                       softcap=9.0, scale=0.7)
    plan = make_plan(spec, TDT[dtype], chunks)
    say(f"[gpu] per-token values {dtype} {combo} {plan.describe()}")
    run_hip(plan, _to_dev(inp), "none")
    rv = plan.row_values().cpu().double().numpy()
    N = inp["logits"].shape[0]
    y = to_np(inp["labels"]).astype(np.int64)
    valid, _ = oracle.row_validity(N, spec.V, y, to_np(inp["mask"]))
    vals = oracle.row_values(spec, to_np(inp["logits"]), y, to_np(inp["teacher"]),
                             to_np(inp["old_logprobs"]), to_np(inp["advantages"]))
    kl = "fkl" if spec.has(FKL) else ("rkl" if spec.has(RKL) else "fdce")
    rel = TOL[dtype]["scalar_rel"]
    np.testing.assert_array_equal(rv[:, 10], valid.astype(float))
    assert np.all(rv[~valid] == 0.0)
    for key, col in (("ce", 0), ("z", 1), (kl, 2), ("grpo", 3), ("logp", 4), ("ratio", 5),
                     ("k3", 7), ("adv", 8), ("entropy", 9)):
        ref = vals[key][valid]
        got = rv[valid, col]
        scale = np.maximum(np.abs(ref), 1e-2 * max(1.0, float(np.max(np.abs(ref)))))
        err = np.max(np.abs(got - ref) / scale)
        assert err <= rel, (key, err)
    boundary = (np.abs(vals["ratio"] - 1.2) < 1e-5) | (np.abs(vals["ratio"] - 0.8) < 1e-5)
    keep = valid & ~boundary
    np.testing.assert_array_equal(rv[keep, 6] != 0, vals["clipped"][keep])


def test_split_vocab_calls_with_changing_batch_sizes():
    """One plan, calls of different sizes: the workspace layout moves between
    calls and every call must still combine only its own chunk records."""
    spec, _ = _small("bf16", "all_fkl", 2, 60013, seed=1)
    plan = make_plan(spec, torch.bfloat16, chunks=3)
    for i, N in enumerate((8, 3, 8, 12, 5)):
        _, inp = _small("bf16", "all_fkl", N, 60013, seed=100 + i, mask_frac=0.2)
        say(f"[gpu] changing batch N={N}")
        sc, g = run_hip(plan, _to_dev(inp), "overwrite")
        ref_sc, ref_g, _ = run_oracle(spec, inp)
        valid, _ = oracle.row_validity(N, spec.V, to_np(inp["labels"]).astype(np.int64), to_np(inp["mask"]))
        vals = oracle.row_values(spec, to_np(inp["logits"]), to_np(inp["labels"]).astype(np.int64),
                                 to_np(inp["teacher"]), to_np(inp["old_logprobs"]), to_np(inp["advantages"]))
        assert_scalars(spec, sc, ref_sc, "bf16", vals, valid)
        grad_check(g.cpu(), ref_g, "bf16", labels=to_np(inp["labels"]))


def test_split_vocab_accumulate_and_masking():
    spec, inp = _small("bf16", "all_rkl", 12, 50003, seed=9, accumulate=True, mask_frac=0.3, bad_labels=2)
    _check_small(spec, inp, "bf16", chunks=4)


@pytest.mark.parametrize("tau", [0.7, 2.5])
@pytest.mark.parametrize("chunks", [2, 5, 8])
@pytest.mark.parametrize("combo", HINTON_COMBOS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_hinton_split_vocab_and_temperatures(dtype, combo, chunks, tau):
    """The tempered student sums travel through the split-vocab exchange (up
    to 8 chunks, the cap of the 8-statistic from-distribution mode; fp32
    plans, which also exchange the normalizers' low parts, up to their own
    caps). fp32 Hinton slices hold at most 4 vectors per tensor: the wider
    fp32 rows are 30011 elements (two chunks of 1024 x 4 x 4)."""
    wide = 30011 if dtype == "f32" else 70000
    for V, N in ((20011, 7), (wide, 5)):
        spec, inp = _small(dtype, combo, N, V, seed=chunks * 10 + N, softcap=15.0, scale=0.8,
                           temperature=tau, mask_frac=0.2)
        _check_small(spec, inp, dtype, chunks=min(chunks, max_chunks(dtype, spec)))


@pytest.mark.parametrize("combo", HINTON_COMBOS)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_hinton_accumulate_and_per_token_values(dtype, combo):
    spec, inp = _small(dtype, combo, 19, 20011, seed=13, accumulate=True, mask_frac=0.2, softcap=30.0,
                       scale=0.5, temperature=2.0)
    _check_small(spec, inp, dtype)
    spec, inp = _small(dtype, combo, 23, 4099, seed=14, mask_frac=0.2, temperature=3.0)
    plan, _, _ = _check_small(spec, inp, dtype, grad_mode="none")
    rv = plan.row_values().cpu().double().numpy()
    y = to_np(inp["labels"]).astype(np.int64)
    valid, _ = oracle.row_validity(23, spec.V, y, to_np(inp["mask"]))
    vals = oracle.row_values(spec, to_np(inp["logits"]), y, to_np(inp["teacher"]),
                             to_np(inp.get("old_logprobs")), to_np(inp.get("advantages")))
    key = "fkl" if spec.has(FKL) else ("rkl" if spec.has(RKL) else "fdce")
    ref = vals[key][valid]
    err = np.max(np.abs(rv[valid, 2] - ref) / np.maximum(np.abs(ref), 1e-2))
    assert err <= TOL[dtype]["scalar_rel"], err


@pytest.mark.parametrize("chunks", [0, 3])
@pytest.mark.parametrize("combo", ["ce_z", "all_rkl", "all_fkl", "all_fdce"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("mode", ["gradient", "forward_only"])
def test_outlier_logits(dtype, combo, chunks, mode):
    """A logit (or teacher logit) far above the rest of its row, placed after
    the first vector of a wave, in the ragged head/tail, or in the first
    vector: the softmax shift is taken from each wave's first vector, and a
    wave whose sums would overflow from that shift sums again from its true
    maximum."""
    N, V = 10, 20011
    spec, inp = _small(dtype, combo, N, V, seed=71 + chunks, mask_frac=0.0, ignore_frac=0.0)
    # student outlier 60 (x log2 e = 87, beyond 64 above a first vector whose
    # maximum is about 9 in log2 units), half of it on odd rows (35 above:
    # kept from the provisional shift); teacher outlier 100 (/ tau 1.5 =
    # 96 log2 units)
    big, tbig = 60.0, 100.0
    x = inp["logits"].float()
    t = inp["teacher"].float() if inp["teacher"] is not None else None
    # row r: an outlier at a position spread over the row (first vector,
    # later vectors, the last element of the row, i.e. the ragged tail)
    pos = [0, 5, 700, 4099, 9000, 15000, 19999, V - 1, 3, 12345]
    for r in range(N):
        x[r, pos[r]] = big if r % 2 == 0 else big / 2
        if t is not None and r % 3 == 0:
            t[r, pos[(r + 4) % N]] = tbig
    inp["logits"] = x.to(TDT[dtype])
    if t is not None:
        inp["teacher"] = t.to(TDT[dtype])
    if spec.has(GRPO):
        inp["old_logprobs"] = oracle_old_logprobs(spec, inp["logits"], inp["labels"], inp["old_noise"])
    # fp32 gradient: the plain 1e-6 absolute gate (the fp32 instances form
    # exponents with fp64 constants, sum the normalizers in fp64 and write
    # each element from fp64 coefficients, so an outlier's exponent keeps its
    # low bits).
    #
    # Entropy: these rows are nearly one-hot, so the exact entropy is ~1e-7
    # nats, while the entropy sum S and (in the 16-bit instances) Z are fp32
    # sums whose every rounding moves the result by up to 2^-24 nats through
    # up to ~20 merges, so the entropy is checked to 2e-6 nats absolute
    # instead of relative to its near-zero value.
    ref_sc, ref_g, _ = run_oracle(spec, inp)
    gm = None if mode == "gradient" else "none"
    _, sc, met = _check_small(spec, inp, dtype, chunks=chunks, grad_mode=gm, skip_scalars=("ENTROPY",))
    if met is not None and "max_abs" in met:
        say(f"[f32-err] outlier max_abs={met['max_abs']:.3e} max|g|={float(np.max(np.abs(ref_g))):.3e}")
    e = SLOT["ENTROPY"]
    assert abs(sc[e] - ref_sc[e]) <= 2e-6 + TOL[dtype]["scalar_rel"] * abs(ref_sc[e]), (sc[e], ref_sc[e])
    spec_c, inp_c = _small(dtype, combo, N, V, seed=71 + chunks, softcap=30.0, scale=0.5)
    inp_c["logits"] = inp["logits"]
    inp_c["teacher"] = inp["teacher"]
    if spec_c.has(GRPO):
        inp_c["old_logprobs"] = oracle_old_logprobs(spec_c, inp_c["logits"], inp_c["labels"], inp_c["old_noise"])
    ref_sc, ref_c, _ = run_oracle(spec_c, inp_c)
    _, sc, met = _check_small(spec_c, inp_c, dtype, chunks=chunks, grad_mode=gm, skip_scalars=("ENTROPY",))
    if met is not None and "max_abs" in met:
        say(f"[f32-err] outlier softcap max_abs={met['max_abs']:.3e} max|g|={float(np.max(np.abs(ref_c))):.3e}")
    assert abs(sc[e] - ref_sc[e]) <= 2e-6 + TOL[dtype]["scalar_rel"] * abs(ref_sc[e]), (sc[e], ref_sc[e])


# the longest rows each mode supports: 9 chunks x 1024 threads x 20 vectors
# (student), x 10 vectors (teacher), 8 chunks for from-distribution CE with
# the Hinton temperature (8 exchanged statistics per chunk); fp32 teacher
# slices of at most 8 vectors (4 Hinton) and the fp32 chunk caps (8 for the
# KL modes, 5 for Hinton FDCE)
MAX_V = [("bf16", "ce_z", 1_474_560, (9, 1024, 20)), ("bf16", "ce_z", 1_474_553, (9, 1024, 20)),
         ("f32", "ce_z", 737_280, (9, 1024, 20)), ("bf16", "all_rkl", 737_280, (9, 1024, 10)),
         ("bf16", "all_fdce_h", 655_360, (8, 1024, 10)), ("f32", "ce_fkl", 262_144, (8, 1024, 8)),
         ("f32", "all_fdce_h", 81_920, (5, 1024, 4))]


@pytest.mark.parametrize("case", MAX_V, ids=[f"{d}-{c}-{v}" for d, c, v, _ in MAX_V])
def test_maximum_vocabulary(case):
    dtype, combo, V, geo = case
    spec, inp = _small(dtype, combo, 3, V, seed=V % 1000, mask_frac=0.0, ignore_frac=0.0)
    plan, _, _ = _check_small(spec, inp, dtype)
    d = plan.describe()
    assert (d["chunks"], d["block"], d["vec_per_thread"]) == geo


# one vector past the longest slices the chunk exchange serves: statistics
# streamed, then the gradient from the fused kernel in load mode
LONG_ROWS = [("bf16", "ce_z", 1_474_569, False), ("bf16", "all_rkl", 737_288, True),
             ("f32", "ce_fkl", 368_644, False), ("bf16", "all_fdce_h", 655_368, False),
             ("f32", "all_fdce_h", 81_924, False)]


@pytest.mark.parametrize("case", LONG_ROWS, ids=[f"{d}-{c}-{v}" for d, c, v, _ in LONG_ROWS])
def test_rows_past_every_slice(case):
    """Rows longer than every slice the chunk exchange serves: the statistics
    streamed first, the gradient from the fused kernel in load mode with as many
    chunks as the row needs; forward-only calls stream only. Misaligned bases
    on such rows take the row-wise kernel."""
    dtype, combo, V, acc = case
    spec, inp = _small(dtype, combo, 3, V, seed=V % 997, softcap=20.0 if acc else 0.0, scale=0.7 if acc else 1.0,
                       accumulate=acc, bad_labels=1, mask_frac=0.0)
    plan, _, _ = _check_small(spec, inp, dtype)
    d = plan.describe()
    assert d["block"] == 1024 and d["chunks"] > max_chunks(dtype, spec)
    _check_small(spec, inp, dtype, grad_mode="none")
    # the same rows with a gradient buffer misaligned against the logits: row-wise
    ref_sc, ref_g, _ = run_oracle(spec, inp)
    dev = _to_dev(inp)
    es = dev["logits"].element_size()
    buf = torch.empty(dev["logits"].numel() * es + 64, dtype=torch.uint8, device=DEV)
    g = buf[es: es + dev["logits"].numel() * es].view(dev["logits"].dtype).view(dev["logits"].shape)
    g.copy_(inp["grad_init"].to(DEV) if acc else torch.zeros_like(dev["logits"]))
    sc = plan(dev["logits"], labels=dev["labels"], mask=dev["mask"], teacher=dev["teacher"],
              old_logprobs=dev.get("old_logprobs"), advantages=dev.get("advantages"), grad=g)
    torch.cuda.synchronize()
    assert_scalars(spec, sc.cpu().double().numpy(), ref_sc, dtype)
    grad_check(g.detach().cpu(), ref_g, dtype, labels=to_np(inp["labels"]))


def test_two_plans_on_two_streams():
    """Two split-vocab plans (a teacher row set in 4 chunks, a student row set in
    2) run concurrently on two streams of default priority, calls interleaved:
    each result is bitwise the one its plan gives alone. The chunks of a row
    wait for each other on the device; with two kernels in flight their
    workgroups share the CUs, and the in-order dispatch of each kernel keeps
    every wait finite (a broken wait would surface as NaN, not a hang)."""
    spec_a, inp_a = _small("bf16", "ce_fkl", 512, 151936, seed=3, mask_frac=0.1)
    spec_b, inp_b = _small("bf16", "grpo_z_ent", 768, 151936, seed=4, mask_frac=0.1)
    plan_a, plan_b = make_plan(spec_a, torch.bfloat16), make_plan(spec_b, torch.bfloat16)
    assert plan_a.describe()["chunks"] == 4 and plan_b.describe()["chunks"] == 2
    da, db = _to_dev(inp_a), _to_dev(inp_b)
    sc_a, g_a = run_hip(plan_a, da, "overwrite")
    sc_b, g_b = run_hip(plan_b, db, "overwrite")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(4):
        ga, gb = torch.empty_like(g_a), torch.empty_like(g_b)
        with torch.cuda.stream(s1):
            ra = plan_a(da["logits"], labels=da["labels"], mask=da["mask"], teacher=da["teacher"], grad=ga)
        with torch.cuda.stream(s2):
            rb = plan_b(db["logits"], labels=db["labels"], mask=db["mask"], old_logprobs=db["old_logprobs"],
                        advantages=db["advantages"], grad=gb)
        outs.append((ra, ga, rb, gb))
    torch.cuda.synchronize()
    say(f"[gpu] two streams: {len(outs)} interleaved call pairs")
    for ra, ga, rb, gb in outs:
        np.testing.assert_array_equal(ra.cpu().double().numpy(), sc_a)
        np.testing.assert_array_equal(rb.cpu().double().numpy(), sc_b)
        assert torch.equal(ga.view(torch.int16), g_a.view(torch.int16))
        assert torch.equal(gb.view(torch.int16), g_b.view(torch.int16))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_cases(dtype):
    dt = TDT[dtype]
    # empty batch: every slot 0
    spec = spec_from(100, CE | Z | ENT, dict(ce=1.0, z=0.1))
    plan = make_plan(spec, dt)
    say(f"[gpu] empty batch {dtype}")
    sc = plan(torch.empty(0, 100, dtype=dt, device=DEV), labels=torch.empty(0, dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    assert torch.all(sc.cpu() == 0)
    # every row masked: zeros, zero gradient
    spec, inp = _small(dtype, "all_rkl", 6, 777, seed=1, ignore_frac=1.0)
    _check_small(spec, inp, dtype)
    # single row, V = 1 (softmax is exactly 1)
    spec, inp = _small(dtype, "ce_z", 1, 1, seed=2, ignore_frac=0.0)
    _check_small(spec, inp, dtype)
    # bad labels are counted and masked
    spec, inp = _small(dtype, "ce", 30, 500, seed=3, bad_labels=5)
    plan, sc, _ = _check_small(spec, inp, dtype)
    assert sc[SLOT["N_BADLABEL"]] == 5
    # a caller divisor replaces the valid-row count
    spec, inp = _small(dtype, "all_fkl", 10, 999, seed=4)
    spec.divisor = 123.0
    _check_small(spec, inp, dtype)


@pytest.mark.parametrize("N", [15, 16, 16383, 16384, 16401, 40000])
@pytest.mark.parametrize("layout", ["aligned", "offset_views", "no_mask"])
def test_valid_row_count_paths(N, layout):
    """The valid-row and bad-label counts (tiled 16-byte loads when labels and
    mask are 16-byte aligned, one row at a time otherwise; ragged last tiles)
    against the oracle's row validity, with the CE mean as a cross-check."""
    V = 37
    spec = spec_from(V, CE, dict(ce=1.0))
    g = torch.Generator().manual_seed(N)
    y = torch.randint(0, V, (N + 3,), generator=g, dtype=torch.int64)
    y[torch.rand(N + 3, generator=g) < 0.1] = -100
    bad = torch.rand(N + 3, generator=g) < 0.05
    y[bad] = torch.where(torch.rand(N + 3, generator=g)[bad] < 0.5, V + 7, -5)
    m = (torch.rand(N + 3, generator=g) >= 0.2).to(torch.uint8)
    x = torch.randn(N, V, generator=g).to(torch.bfloat16)
    if layout == "offset_views":          # 8-byte (labels) / 1-byte (mask) aligned views
        yv, mv = y.to(DEV)[1:N + 1], m.to(DEV)[3:N + 3]
        y_c, m_c = y[1:N + 1], m[3:N + 3]
    else:
        yv, mv = y[:N].to(DEV), m[:N].to(DEV)
        y_c, m_c = y[:N], m[:N]
    if layout == "no_mask":
        mv, m_c = None, None
    plan = make_plan(spec, torch.bfloat16)
    say(f"[gpu] count N={N} layout={layout}")
    sc = plan(x.to(DEV), labels=yv, mask=mv).cpu().double().numpy()
    torch.cuda.synchronize()
    valid, bad_rows = oracle.row_validity(N, V, y_c.numpy(), None if m_c is None else m_c.numpy())
    assert sc[SLOT["N_VALID"]] == valid.sum()
    assert sc[SLOT["N_BADLABEL"]] == bad_rows.sum()
    ref = oracle.forward_backward(spec, x.double().numpy(), y_c.numpy(), None if m_c is None else m_c.numpy(),
                                  want_grad=False)[0]
    assert abs(sc[SLOT["CE"]] - ref[SLOT["CE"]]) <= 1e-4 * abs(ref[SLOT["CE"]])


@pytest.mark.parametrize("chunks", [0, 3])
@pytest.mark.parametrize("combo", ["ce_z", "all_rkl"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nonfinite_logits(dtype, combo, chunks):
    """NaN and Inf inputs propagate without sanitizing: a masked row that holds
    them changes nothing (its gradient row is +0.0, the scalars match the
    oracle on the other rows); a valid row with a NaN makes its own gradient
    row and the means of its per-row values NaN and leaves every other row's
    gradient as the oracle computes it."""
    N, V = 9, 3001
    spec, inp = _small(dtype, combo, N, V, seed=91 + chunks, ignore_frac=0.0, mask_frac=0.0)
    x = inp["logits"].clone()
    x[2, 5] = float("nan")
    x[2, 700] = float("inf")
    x[2, 2000] = float("-inf")
    inp["logits"] = x
    if inp.get("teacher") is not None:
        inp["teacher"][2, 9] = float("nan")
    labels = inp["labels"].clone()
    labels[2] = -100                     # row 2 masked through its label
    inp["labels"] = labels
    if spec.has(GRPO):
        inp["old_logprobs"] = oracle_old_logprobs(spec, x.nan_to_num(0.0), labels, inp["old_noise"])
    # masked non-finite row: parity everywhere, +0.0 gradient on that row
    _check_small(spec, inp, dtype, chunks=chunks)

    # the same NaN in a valid row
    labels2 = labels.clone()
    labels2[2] = 11
    inp2 = dict(inp, labels=labels2)
    plan = make_plan(spec, TDT[dtype], chunks)
    say(f"[gpu] non-finite valid row {dtype} {combo} {plan.describe()}")
    sc, g = run_hip(plan, _to_dev(inp2), "overwrite")
    _, ref_g, _ = run_oracle(spec, inp2)
    assert np.isnan(sc[SLOT["CE"]]) and np.isnan(sc[SLOT["TOTAL"]])
    assert sc[SLOT["N_VALID"]] == N
    gk = to_np(g.detach().cpu())
    assert np.isnan(gk[2]).all()
    keep = np.ones(N, dtype=bool)
    keep[2] = False
    grad_check(g.detach().cpu()[torch.from_numpy(keep)], ref_g[keep], dtype, labels=to_np(labels2)[keep])
    # without a gradient (the streaming statistics kernel): the same scalars' fate, and the
    # per-row values of the other rows as the oracle computes them
    sc_fo, _ = run_hip(plan, _to_dev(inp2), "none")
    assert np.isnan(sc_fo[SLOT["CE"]]) and np.isnan(sc_fo[SLOT["TOTAL"]])
    assert sc_fo[SLOT["N_VALID"]] == N
    rows = plan.row_values().cpu().double().numpy()
    assert np.isnan(rows[2, 0])
    vals = oracle.row_values(spec, to_np(inp2["logits"]), to_np(labels2).astype(np.int64),
                             to_np(inp2.get("teacher")), to_np(inp2.get("old_logprobs")),
                             to_np(inp2.get("advantages")))
    np.testing.assert_allclose(rows[keep, 0], vals["ce"][keep], rtol=TOL[dtype]["scalar_rel"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_weight_keeps_scalars_and_drops_gradient_term(dtype):
    spec, inp = _small(dtype, "all_rkl", 17, 1500, seed=21)
    spec0 = spec_from(spec.V, spec.flags, dict(ce=1.0, z=1e-3, distill=0.5, grpo=0.0, grad_scale=0.25),
                      temperature=spec.temperature)
    plan_full, sc_full, _ = _check_small(spec, inp, dtype)
    plan0, sc0, _ = _check_small(spec0, inp, dtype)
    for name in ("GRPO", "NEWLOGP", "RATIO", "CLIPFRAC", "KL_OLD_NEW", "ADV_MEAN"):
        assert sc0[SLOT[name]] == sc_full[SLOT[name]], name


def test_bitwise_determinism():
    for chunks, combo in ((0, "grpo_z_ent"), (3, "all_rkl")):
        spec, inp = _small("bf16", combo, 33, 40000, seed=8, accumulate=True, softcap=20.0)
        plan = make_plan(spec, torch.bfloat16, chunks)
        d = _to_dev(inp)
        say(f"[gpu] determinism chunks={chunks} {combo}")
        sc1, g1 = run_hip(plan, d, "accumulate")
        sc2, g2 = run_hip(plan, d, "accumulate")
        np.testing.assert_array_equal(sc1, sc2)
        assert torch.equal(g1.view(torch.int16), g2.view(torch.int16))
        rv1 = plan.row_values().clone()
        run_hip(plan, d, "accumulate")
        assert torch.equal(rv1, plan.row_values())


@pytest.mark.parametrize("combo", ["ce_z", "all_rkl", "all_fkl", "all_fdce"])
def test_fused_equals_separate_passes(combo):
    """The per-loss loop (one single-loss plan per loss, accumulating into one
    fp32 buffer) equals the fused pass up to rounding (fp32 inputs)."""
    spec, inp = _small("f32", combo, 29, 3333, seed=12)
    d = _to_dev(inp)
    fused = make_plan(spec, torch.float32)
    sc_f, g_f = run_hip(fused, d, "overwrite")
    weights = {CE: ("ce", spec.w_ce), Z: ("z", spec.w_z), FKL: ("distill", spec.w_distill),
               RKL: ("distill", spec.w_distill), FDCE: ("distill", spec.w_distill), GRPO: ("grpo", spec.w_grpo)}
    g = torch.zeros_like(d["logits"])
    first = True
    for flag, (key, wv) in weights.items():
        if not spec.has(flag):
            continue
        w = dict(ce=0.0, grad_scale=spec.grad_scale)
        w[key] = wv
        single = spec_from(spec.V, flag | (0 if first else ACC), w, temperature=spec.temperature)
        p = make_plan(single, torch.float32)
        p(d["logits"], labels=d["labels"], mask=d["mask"], teacher=d["teacher"],
          old_logprobs=d.get("old_logprobs"), advantages=d.get("advantages"), grad=g)
        first = False
    torch.cuda.synchronize()
    assert (g - g_f).abs().max().item() <= 1e-6


@pytest.mark.parametrize("reads, block, vpt", [(1, 1024, 10), (2, 512, 13), (2, 1024, 8), (1, 512, 9), (2, 512, 6)])
def test_stream_ceiling_moves_every_byte(reads, block, vpt):
    """The memory-system reference writes the xor of its inputs over the
    whole buffer (several workgroups and a ragged last one), bit for bit."""
    n = 3 * block * vpt + 37                      # 16-byte vectors
    gen = torch.Generator(device="cpu").manual_seed(block + vpt + reads)
    a = torch.randint(-2**31, 2**31 - 1, (n, 4), dtype=torch.int32, generator=gen).to(DEV)
    b = torch.randint(-2**31, 2**31 - 1, (n, 4), dtype=torch.int32, generator=gen).to(DEV) if reads == 2 else None
    out = torch.zeros_like(a)
    say(f"[gpu] stream ceiling reads={reads} block={block} vec={vpt} n={n}")
    ms = hl.stream_ceiling(a, b, out, block, vpt, reps=2)
    ref = a ^ b if b is not None else a
    assert torch.equal(out, ref)
    assert ms > 0.0


# signs and zeros of the probability, teacher and reverse-KL coefficients
# (the 16-bit instances fold the coefficient's magnitude into the exponent and
# apply its sign to the packed output; reverse KL with rho2 = 0 takes the plain
# element path)
SIGN_CASES = [
    ("ce", dict(ce=-0.7)),                                           # alpha < 0, no teacher
    ("ce_fkl", dict(ce=-0.7, distill=1.0)),                          # alpha < 0 < gam
    ("ce_fkl", dict(ce=0.5, distill=-0.8)),                          # gam < 0 < alpha
    ("ce_fkl", dict(ce=-0.5, distill=-0.8)),                         # both negative
    ("ce_fdce", dict(ce=0.0, distill=-1.1)),                         # alpha = gam < 0
    ("ce_fkl", dict(ce=0.5, distill=0.0)),                           # gam = 0
    ("all_rkl", dict(ce=1.0, z=1e-3, distill=0.0, grpo=1.0)),        # rho2 = 0: plain path
    ("all_rkl", dict(ce=1.0, z=1e-3, distill=-0.5, grpo=1.0)),       # rho2 < 0
    ("ce_rkl", dict(ce=-0.5, distill=0.7)),                          # c0 < 0 < rho2
]


@pytest.mark.parametrize("mode", ["overwrite", "accumulate"])
@pytest.mark.parametrize("case", SIGN_CASES, ids=[f"{c}-{'_'.join(f'{k}{v}' for k, v in w.items())}" for c, w in SIGN_CASES])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_coefficient_signs_and_zeros(dtype, case, mode):
    combo, w = case
    flags = COMBOS[combo][0] | (ACC if mode == "accumulate" else 0)
    w = dict(w)
    if dtype == "f16":
        w["grad_scale"] = w.get("grad_scale", 1.0) * F16_LOSS_SCALE
    N, V = 9, 20011
    spec = spec_from(V, flags, w, temperature=1.5, eps=0.2, logit_scale=0.9, softcap=0.0)
    inp = workloads.small_inputs(N, V, dtype, "cpu", 500 + len(combo) * 7 + N, teacher=bool(flags & DISTILL),
                                 grpo=bool(flags & GRPO), accumulate=mode == "accumulate", mask_frac=0.2)
    if flags & GRPO:
        inp["old_logprobs"] = oracle_old_logprobs(spec, inp["logits"], inp["labels"], inp["old_noise"])
    for chunks in (0, 3):
        _check_small(spec, inp, dtype, chunks=chunks)
