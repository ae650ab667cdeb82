"""GPU parity for logits, teacher and gradient bases that are not 16-byte
aligned.

The fused kernel splits every row into 16-byte vectors at the same
boundaries in the three tensors, so it runs whenever their base addresses
agree modulo 16 bytes (a common misalignment shifts the split); when they
do not, the row-wise kernel runs (element loads and stores). Both are
compared with the fp64 oracle at the tolerances of the other parity tests
(fp32: scalars 1e-5 relative, gradient 1e-6 absolute; bf16: scalars 1e-4
relative, gradient rms-relative 4e-3 over the tensor and over its non-label
entries), with each tensor copied into a larger buffer at a chosen byte
offset. Masked rows must be +0.0 (overwrite) or untouched (accumulate), as
everywhere else.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_support import assert_scalars, grad_check, make_plan, run_oracle, say, to_np
from test_gpu_gspo import _boundary_rows, _case, _oracle, _scalar_vals
from test_gpu_parity import _grpo_boundary_rows, _small

pytestmark = pytest.mark.gpu
DEV = "cuda"
TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
INT_VIEW = {"f32": torch.int32, "bf16": torch.int16, "f16": torch.int16}
GRPO, ACC = oracle.GRPO, oracle.ACCUMULATE

# byte offsets (in element sizes) of logits, teacher, gradient: the first two
# keep the three bases congruent modulo 16 bytes (fused kernel), the others
# do not (row-wise kernel)
LAYOUTS = {
    "common_1": (1, 1, 1),
    "common_3_plus_16": (3, 3 + 16, 3 + 32),
    "teacher_off": (0, 1, 0),
    "grad_off": (0, 0, 3),
    "all_differ": (1, 2, 3),
}
ROWWISE = {"teacher_off", "grad_off", "all_differ"}


def _place(t, off_elems):
    """A device copy of t starting off_elems elements past a fresh (512-byte
    aligned) allocation; returns (keep-alive buffer, view)."""
    if t is None:
        return None, None
    es = t.element_size()
    buf = torch.empty(t.numel() * es + off_elems * es + 64, dtype=torch.uint8, device=DEV)
    v = buf[off_elems * es: off_elems * es + t.numel() * es].view(t.dtype).view(t.shape)
    v.copy_(t.to(DEV))
    return buf, v


def _run_placed(plan, inp, layout, grad_mode, seq_offsets=None):
    ox, ot, og = LAYOUTS[layout]
    keep = []
    b, x = _place(inp["logits"], ox)
    keep.append(b)
    b, t = _place(inp.get("teacher"), ot)
    keep.append(b)
    grad = None
    if grad_mode == "overwrite":
        b, grad = _place(torch.full_like(inp["logits"], float("nan")), og)
        keep.append(b)
    elif grad_mode == "accumulate":
        b, grad = _place(inp["grad_init"], og)
        keep.append(b)
    dev = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    # the layout does what its name says: congruent bases, or at least one that differs
    bases = [q.data_ptr() % 16 for q in (t, grad) if q is not None]
    differs = any(m != x.data_ptr() % 16 for m in bases)
    assert differs == (layout in ROWWISE and (layout != "teacher_off" or t is not None)
                       and (layout != "grad_off" or grad is not None))
    sc = plan(x, labels=dev["labels"], mask=dev["mask"], teacher=t, old_logprobs=dev.get("old_logprobs"),
              advantages=dev.get("advantages"), grad=grad, seq_offsets=seq_offsets)
    torch.cuda.synchronize()
    return sc.cpu().double().numpy(), grad


CASES = [
    # (dtype, combo, N, V, softcap, scale, accumulate)
    ("f32", "ce_z", 13, 4099, 0.0, 1.0, False),
    ("bf16", "ce_z", 13, 4099, 0.0, 1.0, False),
    ("bf16", "grpo_z_ent", 21, 2053, 0.0, 1.0, False),
    ("f32", "all_rkl", 9, 33000, 20.0, 0.5, True),
    ("bf16", "all_rkl", 9, 33000, 20.0, 0.5, True),
    ("bf16", "all_fkl", 12, 1000, 0.0, 1.0, False),
    ("bf16", "all_fdce_h", 7, 4099, 0.0, 1.0, False),
    ("f16", "ce_fkl_h", 7, 2053, 0.0, 1.0, False),
    # degenerate rows and the largest vocabulary of the benchmark configurations
    ("bf16", "all_rkl", 5, 3, 0.0, 1.0, False),
    ("f32", "ce_z", 4, 1, 0.0, 1.0, False),
    ("bf16", "all_rkl", 3, 256000, 30.0, 0.5, True),
]


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}x{c[3]}" + ("-acc" if c[6] else "")
                                             for c in CASES])
def test_unaligned_bases_match_the_oracle(case, layout):
    dtype, combo, N, V, cap, scale, acc = case
    spec, inp = _small(dtype, combo, N, V, seed=7 * N + V, softcap=cap, scale=scale, accumulate=acc,
                       bad_labels=1, mask_frac=0.2)
    grad_mode = "accumulate" if acc else "overwrite"
    plan = make_plan(spec, TDT[dtype])
    say(f"[gpu] layout={layout} N={N} V={V} {dtype} {combo} grad={grad_mode} {plan.describe()}")
    sc, g = _run_placed(plan, inp, layout, grad_mode)
    ref_sc, ref_g, _ = run_oracle(spec, inp)
    y = to_np(inp["labels"]).astype(np.int64)
    vals = oracle.row_values(spec, to_np(inp["logits"]), y, to_np(inp["teacher"]),
                             to_np(inp.get("old_logprobs")), to_np(inp.get("advantages")))
    valid, _ = oracle.row_validity(N, V, y, to_np(inp["mask"]))
    boundary = _grpo_boundary_rows(spec, inp) & valid
    assert_scalars(spec, sc, ref_sc, dtype, vals, valid, skip=("CLIPFRAC",) if boundary.any() else (),
                   x=to_np(inp["logits"]))
    gk = g.detach().cpu()
    keep = ~boundary
    grad_check(gk[torch.from_numpy(keep)], ref_g[keep], dtype, labels=y[keep])
    inval = torch.from_numpy(~valid)
    if grad_mode == "overwrite":
        assert torch.equal(gk[inval].view(INT_VIEW[dtype]), torch.zeros_like(gk[inval]).view(INT_VIEW[dtype]))
    else:
        assert torch.equal(gk[inval], inp["grad_init"][inval])


@pytest.mark.parametrize("layout", ["common_1", "all_differ"])
def test_unaligned_forward_only_and_per_row_values(layout):
    """Forward only (no gradient): the kernel is chosen from logits and
    teacher alone; the per-row values match the oracle's."""
    spec, inp = _small("bf16", "all_rkl", 11, 4099, seed=5, bad_labels=1, mask_frac=0.2)
    plan = make_plan(spec, torch.bfloat16)
    sc, _ = _run_placed(plan, inp, layout, "none")
    ref_sc, _, _ = run_oracle(spec, inp, want_grad=False)
    y = to_np(inp["labels"]).astype(np.int64)
    vals = oracle.row_values(spec, to_np(inp["logits"]), y, to_np(inp["teacher"]),
                             to_np(inp.get("old_logprobs")), to_np(inp.get("advantages")))
    valid, _ = oracle.row_validity(11, 4099, y, to_np(inp["mask"]))
    boundary = _grpo_boundary_rows(spec, inp) & valid
    assert_scalars(spec, sc, ref_sc, "bf16", vals, valid, skip=("CLIPFRAC",) if boundary.any() else ())
    rows = plan.row_values().cpu().double().numpy()
    ok = valid & ~boundary
    np.testing.assert_allclose(rows[ok, 0], vals["ce"][ok], rtol=1e-4, atol=1e-4)
    np.testing.assert_allclose(rows[ok, 2], vals["rkl"][ok], rtol=1e-4, atol=1e-4)
    np.testing.assert_allclose(rows[ok, 9], vals["entropy"][ok], rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("layout", ["common_3_plus_16", "grad_off", "all_differ"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned_gspo(dtype, layout):
    """GSPO (forward, segment step, load-mode backward) on unaligned bases."""
    spec, inp = _case(dtype, "all_gspo_rkl", 19, 4099, seed=31, bad_labels=1)
    plan = make_plan(spec, TDT[dtype])
    say(f"[gpu] gspo layout={layout} {dtype} {plan.describe()}")
    sc, g = _run_placed(plan, inp, layout, "overwrite", seq_offsets=inp["seq_offsets"].to(DEV))
    ref_sc, ref_g, vals, valid, seam = _oracle(spec, inp)
    boundary, any_b = _boundary_rows(spec, seam, valid)
    assert_scalars(spec, sc, ref_sc, dtype, _scalar_vals(vals, seam), valid,
                   skip=("CLIPFRAC",) if any_b else ())
    gk = g.detach().cpu()
    keep = ~boundary
    grad_check(gk[torch.from_numpy(keep)], ref_g[keep], dtype, labels=to_np(inp["labels"])[keep])
    inval = torch.from_numpy(~valid)
    assert torch.equal(gk[inval].view(INT_VIEW[dtype]), torch.zeros_like(gk[inval]).view(INT_VIEW[dtype]))


def test_rowwise_and_fused_agree_closely():
    """The same inputs through both kernels (aligned vs relatively misaligned
    gradient): every scalar within 2e-6 relative, gradients within one bf16
    rounding step of each other almost everywhere."""
    spec, inp = _small("bf16", "all_fkl", 16, 33000, seed=99, bad_labels=1, mask_frac=0.1)
    plan = make_plan(spec, torch.bfloat16)
    sc_a, g_a = _run_placed(plan, inp, "common_1", "overwrite")
    sc_b, g_b = _run_placed(plan, inp, "grad_off", "overwrite")
    np.testing.assert_allclose(sc_a, sc_b, rtol=2e-6, atol=1e-7)
    a = g_a.detach().cpu().float().numpy()
    b = g_b.detach().cpu().float().numpy()
    close = np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-30
    assert close.mean() > 0.999, close.mean()
