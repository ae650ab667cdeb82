"""hl_forward_backward_noalloc, the entry point for callers that cannot
allocate device memory, against the allocating entry point
(hl_forward_backward_segments with the plan's own workspace): two calls in a
row on one plan, the second with a smaller input, each bit-identical to the
allocating call's scalars and gradient (same kernels) and within the parity
tolerances of the fp64 oracle. The cases cover the split-vocab exchange (its
words live in the static array), a student-only row set, GSPO (forward,
segment step, load-mode backward) and fp32; calls of different plans and
layouts follow each other on the one static array per GPU.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_support import assert_scalars, grad_check, make_plan, oracle_old_logprobs, say, spec_from, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}
CE, Z, FKL, RKL, GRPO, GSPO, ENT = (oracle.CE, oracle.ZLOSS, oracle.FKL, oracle.RKL, oracle.GRPO, oracle.GSPO,
                                    oracle.ENTROPY)

# name, dtype, flags, weights, V, chunks, (first N, second N)
CASES = [
    ("split_vocab_fkl", "bf16", CE | FKL, dict(ce=0.5, distill=1.0), 60013, 4, (40, 17)),
    ("student_grpo_z_ent", "bf16", GRPO | Z | ENT, dict(ce=0.0, z=0.01, grpo=1.0), 151936, 0, (48, 20)),
    ("gspo_rkl", "bf16", CE | RKL | GSPO | ENT, dict(ce=1.0, distill=0.5, grpo=1.0), 20011, 0, (30, 11)),
    ("fp32_ce_z_softcap", "f32", CE | Z, dict(ce=1.0, z=0.1), 4099, 3, (37, 9)),
]


def _inputs(spec, dtype, N, seed):
    inp = workloads.small_inputs(N, spec.V, dtype, "cpu", seed, teacher=bool(spec.flags & (FKL | RKL)),
                                 grpo=bool(spec.flags & (GRPO | GSPO)), mask_frac=0.2, bad_labels=1)
    if spec.flags & (GRPO | GSPO):
        inp["old_logprobs"] = oracle_old_logprobs(spec, inp["logits"], inp["labels"], inp["old_noise"])
    if spec.flags & GSPO:
        inp["seq_offsets"] = workloads.segment_offsets(N, seed + 1, max_len=6)
    return inp


def _call(plan, inp, noalloc):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    grad = torch.full_like(d["logits"], float("nan"))
    sc = plan(d["logits"], labels=d["labels"], mask=d["mask"], teacher=d["teacher"],
              old_logprobs=d.get("old_logprobs"), advantages=d["advantages"], grad=grad,
              seq_offsets=d.get("seq_offsets"), noalloc=noalloc)
    torch.cuda.synchronize()
    return sc.cpu(), grad.cpu()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_the_allocating_entry_point(case):
    name, dtype, flags, w, V, chunks, sizes = case
    cap = 20.0 if dtype == "f32" else 0.0
    spec = spec_from(V, flags, w, temperature=1.5, eps=0.2, logit_scale=0.8 if cap else 1.0, softcap=cap)
    plan = make_plan(spec, TDT[dtype], chunks)
    for k, N in enumerate(sizes):
        inp = _inputs(spec, dtype, N, seed=900 + 10 * k + len(name))
        say(f"[gpu] noalloc {name} call {k + 1}: N={N} V={V} {plan.describe()} "
            f"workspace={plan.workspace_bytes(N)} B")
        sc_ref, g_ref = _call(plan, inp, noalloc=False)
        sc, g = _call(plan, inp, noalloc=True)
        # the same kernels on the same inputs: bit for bit
        assert torch.equal(sc.view(torch.int32), sc_ref.view(torch.int32)), (sc, sc_ref)
        iv = torch.int32 if dtype == "f32" else torch.int16
        assert torch.equal(g.view(iv), g_ref.view(iv))
        # and the oracle's values within the parity tolerances
        y = to_np(inp["labels"]).astype(np.int64)
        args = dict(labels=y, mask=to_np(inp["mask"]), teacher=to_np(inp["teacher"]),
                    old_logprobs=to_np(inp.get("old_logprobs")), advantages=to_np(inp["advantages"]))
        if flags & GSPO:
            args["seq_offsets"] = inp["seq_offsets"].numpy()
        ref_sc, ref_g = oracle.forward_backward(spec, to_np(inp["logits"]), **args)
        vals = oracle.row_values(spec, to_np(inp["logits"]), y, args["teacher"], args["old_logprobs"],
                                 args["advantages"])
        valid, _ = oracle.row_validity(N, V, y, args["mask"])
        skip = ("CLIPFRAC", "GRPO", "RATIO", "KL_OLD_NEW", "ADV_MEAN") if flags & GSPO else ()
        r = vals.get("ratio")
        near = r is not None and bool(np.any(((np.abs(r - 1.2) < 1e-5) | (np.abs(r - 0.8) < 1e-5)) & valid))
        assert_scalars(spec, sc.double().numpy(), ref_sc, dtype, vals, valid,
                       skip=skip + (("CLIPFRAC",) if near else ()), x=to_np(inp["logits"]))
        if not (flags & GSPO) and not near:
            grad_check(g, ref_g, dtype, labels=y)


def test_oversized_call_is_refused_with_the_sizes():
    """A call whose workspace would exceed the static array is refused on the
    host (HL_ERR_WORKSPACE, before anything is enqueued or read) with the
    sizes in hl_last_error; the next call of a size that fits works."""
    import ctypes

    import lm_head_vocab_amd as hl
    spec = spec_from(151936, CE | FKL, dict(ce=0.5, distill=1.0), temperature=2.0)
    plan = make_plan(spec, torch.bfloat16)
    n_big = 1
    while plan.workspace_bytes(n_big) <= (32 << 20):
        n_big *= 2
    lib = hl.load_library()
    buf = torch.zeros(64, dtype=torch.int64, device=DEV)     # never read: the call is refused first
    p = ctypes.c_void_p(buf.data_ptr())
    st = lib.hl_forward_backward_noalloc(plan._h, n_big, p, p, None, p, None, None, None, 0, p, p,
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == hl.HL_ERR_WORKSPACE
    assert "HL_STATIC_WORKSPACE_BYTES" in lib.hl_last_error().decode()
    inp = _inputs(spec, "bf16", 8, seed=5)
    sc_ref, g_ref = _call(plan, inp, noalloc=False)
    sc, g = _call(plan, inp, noalloc=True)
    assert torch.equal(sc.view(torch.int32), sc_ref.view(torch.int32))
    assert torch.equal(g.view(torch.int16), g_ref.view(torch.int16))
