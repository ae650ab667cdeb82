"""GPU tests of the split-vocab exchange's failure path and of one workspace
shared by several plans.

A row spread over several workgroups combines its softmax statistics on the
device with a bounded wait. The failure path is forced from the host through
hl_plan_set_exchange_test: a short spin limit, and one chunk of one row that
does not publish its statistics. Every workgroup of that row then gives up
(each polls its own words as well), so the row's gradient and values must be
NaN and every float scalar NaN; all kernels still end. Rows that are not
withheld must match the fp64 oracle, and the next normal call must be exact.

The exchange words carry the epoch of the call that wrote them; the epoch and
the extent of the words known to be clean live in the workspace's control
words, so two plans of different layouts can take turns on one workspace. The
regression case: plan A runs, plan B's first call on the same workspace
restarts the epoch, and A's older words (now carrying epochs the next calls
reach again) must not be taken for a sibling's current statistics. A withheld
chunk makes that visible: it must give NaN, not a finite stale result.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_support import assert_scalars, grad_check, make_plan, run_hip, run_oracle, say, to_np
from test_gpu_parity import _small, _to_dev
from oracle import SLOT

pytestmark = pytest.mark.gpu

FLOAT_SLOTS = [s for s in oracle.SLOTS if s not in ("N_VALID", "N_BADLABEL")]


def _expect_row_failed(plan, sc, g, row, n_valid, dtype_int):
    for name in FLOAT_SLOTS:
        assert np.isnan(sc[SLOT[name]]), (name, sc[SLOT[name]])
    assert sc[SLOT["N_VALID"]] == n_valid
    gk = g.detach().cpu().float()
    assert torch.isnan(gk[row]).all(), int(torch.isnan(gk[row]).sum())
    rv = plan.row_values().cpu()
    assert torch.isnan(rv[row, 0])


@pytest.mark.parametrize("case", [("bf16", "ce_fkl", 60013, 4), ("bf16", "grpo_z_ent", 151936, 2),
                                  ("f32", "all_rkl", 30011, 3), ("bf16", "all_fdce_h", 20011, 8),
                                  ("f32", "all_fdce_h", 20011, 5)],
                         ids=lambda c: f"{c[0]}-{c[1]}-{c[3]}chunks")
def test_withheld_chunk_gives_nan_then_recovers(case):
    dtype, combo, V, chunks = case
    N, row, hold = 12, 5, chunks - 1
    spec, inp = _small(dtype, combo, N, V, seed=300 + chunks, mask_frac=0.0, ignore_frac=0.0)
    plan = make_plan(spec, {"f32": torch.float32, "bf16": torch.bfloat16}[dtype], chunks)
    assert plan.describe()["chunks"] == chunks
    d = _to_dev(inp)
    plan.set_exchange_test(spin_limit=64, withhold_row=row, withhold_chunk=hold)
    say(f"[gpu] withheld chunk {hold} of row {row}: {dtype} {combo} V={V} {plan.describe()}")
    sc, g = run_hip(plan, d, "overwrite")
    _expect_row_failed(plan, sc, g, row, N, None)
    # the other rows are untouched by the failure
    ref_sc, ref_g, _ = run_oracle(spec, inp)
    keep = np.ones(N, dtype=bool)
    keep[row] = False
    grad_check(g.detach().cpu()[torch.from_numpy(keep)], ref_g[keep], dtype, labels=to_np(inp["labels"])[keep])
    # the same plan, hook cleared: exact again
    plan.set_exchange_test()
    sc2, g2 = run_hip(plan, d, "overwrite")
    assert_scalars(spec, sc2, ref_sc, dtype)
    grad_check(g2.detach().cpu(), ref_g, dtype, labels=to_np(inp["labels"]))


def test_withheld_chunk_metrics_only_and_accumulate():
    """A failed row in accumulate mode: its existing gradient is replaced by
    NaN where the row's chunks gave up (a finite wrong sum is never left)."""
    spec, inp = _small("bf16", "all_rkl", 9, 50003, seed=17, accumulate=True, mask_frac=0.0, ignore_frac=0.0)
    plan = make_plan(spec, torch.bfloat16, 4)
    plan.set_exchange_test(spin_limit=16, withhold_row=0, withhold_chunk=0)
    say(f"[gpu] withheld chunk, accumulate {plan.describe()}")
    sc, g = run_hip(plan, _to_dev(inp), "accumulate")
    _expect_row_failed(plan, sc, g, 0, 9, None)
    plan.set_exchange_test()
    ref_sc, ref_g, _ = run_oracle(spec, inp)
    sc2, g2 = run_hip(plan, _to_dev(inp), "accumulate")
    assert_scalars(spec, sc2, ref_sc, "bf16")
    grad_check(g2.detach().cpu(), ref_g, "bf16", labels=to_np(inp["labels"]))


def test_two_plans_share_one_workspace():
    """Plans of different split-vocab layouts alternate on one workspace:
    every call matches the oracle, and after the second plan's first call has
    restarted the epoch, the first plan's older words are never taken as
    current (a withheld chunk then gives NaN, not a stale finite row)."""
    spec_a, _ = _small("bf16", "ce_fkl", 2, 20011, seed=1)
    spec_b, _ = _small("bf16", "grpo_z_ent", 2, 30011, seed=2)
    plan_a = make_plan(spec_a, torch.bfloat16, 4)
    plan_b = make_plan(spec_b, torch.bfloat16, 2)
    na, nb = 16, 6
    need = max(plan_a.workspace_bytes(na), plan_b.workspace_bytes(nb))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    plan_a.set_workspace(ws)
    plan_b.set_workspace(ws)

    def check(spec, plan, n, seed, dtype="bf16"):
        _, inp = _small(dtype, "ce_fkl" if plan is plan_a else "grpo_z_ent", n, spec.V, seed=seed, mask_frac=0.1)
        sc, g = run_hip(plan, _to_dev(inp), "overwrite")
        ref_sc, ref_g, _ = run_oracle(spec, inp)
        assert_scalars(spec, sc, ref_sc, dtype)
        grad_check(g.detach().cpu(), ref_g, dtype, labels=to_np(inp["labels"]))
        return inp

    say("[gpu] shared workspace: A, A, B (first call, epoch restarts), A withheld, A, B, A")
    check(spec_a, plan_a, na, 10)
    check(spec_a, plan_a, na, 11)
    check(spec_b, plan_b, nb, 12)
    # A's words from its last call are stale; with a chunk withheld its siblings must give up
    _, inp = _small("bf16", "ce_fkl", na, spec_a.V, seed=13, mask_frac=0.0, ignore_frac=0.0)
    plan_a.set_exchange_test(spin_limit=64, withhold_row=3, withhold_chunk=1)
    sc, g = run_hip(plan_a, _to_dev(inp), "overwrite")
    _expect_row_failed(plan_a, sc, g, 3, na, None)
    plan_a.set_exchange_test()
    check(spec_a, plan_a, na, 14)
    check(spec_b, plan_b, nb, 15)
    check(spec_a, plan_a, na, 16)
