"""fp64 CPU oracle for the fused LM-head loss (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package. The HIP library never does.
"""

from .headloss_oracle import (  # noqa: F401
    ACCUMULATE, CE, DISTILL_FLAGS, ENTROPY, FDCE, FKL, GRPO, GSPO, HINTON, IGNORE_INDEX, POLICY_FLAGS,
    READINGS, RKL, SLOT,
    SLOTS, ZLOSS, Spec, batch_divisor, forward_backward, log_softmax_rows,
    gspo_seam, logsumexp_rows, loss_gradients_wrt_s, row_validity, row_values,
    segment_of_rows,
    rows_forward_backward, scalars_from_rows, total_loss, transform,
    transform_derivative,
)
