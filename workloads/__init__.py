"""Seeded synthetic inputs for the fused LM-head loss.

The shapes, dtypes, value distributions and structure (confident columns,
label mixes, masking rates, per-sequence advantages, teacher correlation) of
the five benchmark configurations, drawn with torch generators so that the
same seed gives the same tensors on the GPU and on the host.

Segments (GSPO) are contiguous row ranges given by int32 offsets; the
benchmark segments are the workload's sequences.

This module holds none of the loss arithmetic. GRPO needs old log-probs near
the current policy's label log-prob; the generator draws only the noise
(``old_noise``) and the caller adds the label log-prob it computes itself
(``old_logprobs = logp_label + old_noise``).

The pages name no dataset or evaluation suite; these synthetic tensors are
the whole workload.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

CE, ZLOSS, FKL, RKL, GRPO, ENTROPY, FDCE, GSPO, ACCUMULATE, HINTON = 1, 2, 4, 8, 16, 32, 64, 128, 1 << 16, 1 << 17


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    V: int
    dtype: str                      # "f32" | "bf16"
    flags: int
    weights: dict = field(default_factory=dict)   # ce, z, distill, grpo, grad_scale, divisor
    temperature: float = 1.0
    eps: float = 0.2
    logit_scale: float = 1.0
    softcap: float = 0.0
    seq_len: int = 0                # tokens per sequence (advantages are per sequence)
    old_noise_std: float = 0.0
    description: str = ""

    @property
    def torch_dtype(self):
        return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    "ce_z_tiny_f32": Workload(
        "ce_z_tiny_f32", N=64, V=1024, dtype="f32", flags=CE | ZLOSS,
        weights=dict(ce=1.0, z=0.1),
        description="CE + z-loss (0.1), fp32 logits ~ N(0, 2^2), uniform labels, ~10% label=-100"),
    "ce_z_bf16": Workload(
        "ce_z_bf16", N=8192, V=128256, dtype="bf16", flags=CE | ZLOSS,
        weights=dict(ce=1.0, z=1e-4),
        description="CE + z-loss (1e-4), logits ~ N(0, 3^2) with one +8 confident column per row; "
                    "label = that column on 70% of rows; 10% label=-100"),
    "ce_z_f16": Workload(
        "ce_z_f16", N=8192, V=128256, dtype="f16", flags=CE | ZLOSS,
        weights=dict(ce=1.0, z=1e-4, grad_scale=float(2 ** 24)),
        description="the ce_z_bf16 recipe with fp16 logits and gradient; loss scale 2^24 keeps the "
                    "gradient inside fp16's normal range"),
    "ce_fkl_bf16": Workload(
        "ce_fkl_bf16", N=4096, V=151936, dtype="bf16", flags=CE | FKL,
        weights=dict(ce=0.5, distill=1.0), temperature=2.0,
        description="CE (0.5) + forward-KL (1.0), tau 2; teacher ~ N(0, 3^2), student 0.8 T + N(0, 1); "
                    "label = argmax teacher on 60% of rows"),
    "ce_rkl_bf16": Workload(
        "ce_rkl_bf16", N=4096, V=151936, dtype="bf16", flags=CE | RKL,
        weights=dict(ce=0.5, distill=1.0), temperature=2.0,
        description="the forward-KL inputs with reverse-KL distillation"),
    "ce_fdce_bf16": Workload(
        "ce_fdce_bf16", N=4096, V=151936, dtype="bf16", flags=CE | FDCE,
        weights=dict(ce=0.5, distill=1.0), temperature=2.0,
        description="the forward-KL inputs with from-distribution cross-entropy distillation"),
    "ce_fkl_hinton_bf16": Workload(
        "ce_fkl_hinton_bf16", N=4096, V=151936, dtype="bf16", flags=CE | FKL | HINTON,
        weights=dict(ce=0.5, distill=1.0), temperature=2.0,
        description="the forward-KL inputs with the Hinton temperature mode (student tempered too, "
                    "times tau^2)"),
    "grpo_z_ent_bf16": Workload(
        "grpo_z_ent_bf16", N=16384, V=151936, dtype="bf16", flags=GRPO | ZLOSS | ENTROPY,
        weights=dict(ce=0.0, z=0.01, grpo=1.0), eps=0.2, seq_len=512, old_noise_std=0.05,
        description="GRPO (eps 0.2) + z-loss (0.01) + entropy + ratio/clamp stats; 32 x 512 tokens; "
                    "logits ~ N(0, 2.5^2); uniform labels; old = label logprob + N(0, 0.05^2); "
                    "advantage per sequence ~ N(0, 1); 5% of tokens masked by the mask byte"),
    "ce_z_grpo_ent_bf16": Workload(
        "ce_z_grpo_ent_bf16", N=16384, V=151936, dtype="bf16", flags=CE | ZLOSS | GRPO | ENTROPY,
        weights=dict(ce=1.0, z=0.01, grpo=1.0), eps=0.2, seq_len=512, old_noise_std=0.05,
        description="the GRPO inputs (32 x 512 tokens) with the loss set the headline metric names: "
                    "CE (weight 1.0, not stated: a reading) + z-loss (0.01) + GRPO (eps 0.2) + entropy"),
    "gspo_z_ent_bf16": Workload(
        "gspo_z_ent_bf16", N=16384, V=151936, dtype="bf16", flags=GSPO | ZLOSS | ENTROPY,
        weights=dict(ce=0.0, z=0.01, grpo=1.0), eps=0.002, seq_len=512, old_noise_std=0.05,
        description="the GRPO inputs (32 x 512 tokens) with GSPO over the 32 sequences; eps 0.002 "
                    "(a sequence ratio moves by about 0.05 / sqrt(512), so some sequences clip)"),
    "all_combined_bf16": Workload(
        "all_combined_bf16", N=32768, V=256000, dtype="bf16",
        flags=CE | ZLOSS | RKL | GRPO | ENTROPY | ACCUMULATE,
        weights=dict(ce=1.0, z=1e-4, distill=0.5, grpo=1.0, grad_scale=1.0 / 32),
        temperature=1.5, eps=0.2, logit_scale=0.5, softcap=30.0, seq_len=1024, old_noise_std=0.1,
        description="scale 0.5 then tanh softcap 30; CE + z (1e-4) + reverse-KL tau 1.5 (0.5) + GRPO + "
                    "entropy; teacher ~ N(0, 3^2), student 0.7 T + N(0, 1.5^2); grad scale 1/32 "
                    "accumulated into an existing bf16 gradient"),
}

# Standard deviation of the pre-existing gradient of all_combined_bf16: the rms
# of the fresh gradient that the fp64 oracle gives on a 64-row draw with seed
# 5000 and n = 32768 (tests/golden/all_combined_grad_sigma.py recomputes it).
ALL_COMBINED_GRAD_SIGMA = 2.44e-09

# The benchmark's default line: the loss set the headline metric names
# (CE + z + GRPO + entropy) on the GRPO configuration's inputs.
HEADLINE = "ce_z_grpo_ent_bf16"


def seed_for(name: str, subcase: int = 0) -> int:
    order = ["ce_z_tiny_f32", "ce_z_bf16", "ce_fkl_bf16", "grpo_z_ent_bf16", "all_combined_bf16"]
    base = {"ce_rkl_bf16": "ce_fkl_bf16", "ce_fdce_bf16": "ce_fkl_bf16", "ce_z_f16": "ce_z_bf16",
            "ce_fkl_hinton_bf16": "ce_fkl_bf16",
            "gspo_z_ent_bf16": "grpo_z_ent_bf16", "ce_z_grpo_ent_bf16": "grpo_z_ent_bf16"}.get(name, name)
    return 1000 * (order.index(base) + 1) + subcase


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def generate(w: Workload | str, device="cpu", seed: int | None = None, n_rows: int | None = None,
             chunk_rows: int = 1024) -> dict:
    """Draw one batch of inputs for workload ``w`` (``n_rows`` overrides N).

    Returns a dict with logits, labels, mask, teacher, advantages, old_noise,
    grad_init and seq_offsets (None where the workload has no such input).
    Float tensors are drawn in fp32 and cast once to the workload dtype.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    device = torch.device(device)
    seed = seed_for(w.name) if seed is None else seed
    g = _gen(device, seed)
    N = w.N if n_rows is None else n_rows
    V = w.V
    dt = w.torch_dtype
    out = {"logits": None, "labels": None, "mask": None, "teacher": None,
           "advantages": None, "old_noise": None, "grad_init": None, "seq_offsets": None}

    def rows_normal(std):
        t = torch.empty((N, V), dtype=dt, device=device)
        for r0 in range(0, N, chunk_rows):
            r1 = min(N, r0 + chunk_rows)
            t[r0:r1] = torch.empty((r1 - r0, V), dtype=torch.float32, device=device).normal_(
                0.0, std, generator=g).to(dt)
        return t

    def uniform_labels(n):
        return torch.randint(0, V, (n,), generator=g, device=device, dtype=torch.int64)

    def bernoulli(n, p):
        return torch.rand((n,), generator=g, device=device) < p

    if w.name == "ce_z_tiny_f32":
        out["logits"] = rows_normal(2.0)
        y = uniform_labels(N)
        y[bernoulli(N, 0.1)] = -100
        out["labels"] = y
    elif w.name in ("ce_z_bf16", "ce_z_f16"):
        x = torch.empty((N, V), dtype=dt, device=device)
        cols = uniform_labels(N)
        for r0 in range(0, N, chunk_rows):
            r1 = min(N, r0 + chunk_rows)
            blk = torch.empty((r1 - r0, V), dtype=torch.float32, device=device).normal_(0.0, 3.0, generator=g)
            blk[torch.arange(r1 - r0, device=device), cols[r0:r1]] += 8.0
            x[r0:r1] = blk.to(dt)
        out["logits"] = x
        y = torch.where(bernoulli(N, 0.7), cols, uniform_labels(N))
        y[bernoulli(N, 0.1)] = -100
        out["labels"] = y
    elif w.name in ("ce_fkl_bf16", "ce_rkl_bf16", "ce_fdce_bf16", "ce_fkl_hinton_bf16"):
        t = torch.empty((N, V), dtype=dt, device=device)
        x = torch.empty((N, V), dtype=dt, device=device)
        for r0 in range(0, N, chunk_rows):
            r1 = min(N, r0 + chunk_rows)
            tb = torch.empty((r1 - r0, V), dtype=torch.float32, device=device).normal_(0.0, 3.0, generator=g)
            nb = torch.empty((r1 - r0, V), dtype=torch.float32, device=device).normal_(0.0, 1.0, generator=g)
            t[r0:r1] = tb.to(dt)
            x[r0:r1] = (0.8 * tb + nb).to(dt)
        out["logits"], out["teacher"] = x, t
        # argmax of the stored teacher row (first maximal index on ties)
        amax = torch.argmax(t.float(), dim=1)
        out["labels"] = torch.where(bernoulli(N, 0.6), amax, uniform_labels(N))
    elif w.name in ("grpo_z_ent_bf16", "gspo_z_ent_bf16", "ce_z_grpo_ent_bf16"):
        out["logits"] = rows_normal(2.5)
        out["labels"] = uniform_labels(N)
        out["mask"] = (~bernoulli(N, 0.05)).to(torch.uint8)
        n_seq = (N + w.seq_len - 1) // w.seq_len
        adv_seq = torch.empty(n_seq, dtype=torch.float32, device=device).normal_(0.0, 1.0, generator=g)
        out["advantages"] = adv_seq.repeat_interleave(w.seq_len)[:N].contiguous()
        out["old_noise"] = torch.empty(N, dtype=torch.float32, device=device).normal_(
            0.0, w.old_noise_std, generator=g)
    elif w.name == "all_combined_bf16":
        t = torch.empty((N, V), dtype=dt, device=device)
        x = torch.empty((N, V), dtype=dt, device=device)
        for r0 in range(0, N, chunk_rows):
            r1 = min(N, r0 + chunk_rows)
            tb = torch.empty((r1 - r0, V), dtype=torch.float32, device=device).normal_(0.0, 3.0, generator=g)
            nb = torch.empty((r1 - r0, V), dtype=torch.float32, device=device).normal_(0.0, 1.5, generator=g)
            t[r0:r1] = tb.to(dt)
            x[r0:r1] = (0.7 * tb + nb).to(dt)
        out["logits"], out["teacher"] = x, t
        out["labels"] = uniform_labels(N)
        n_seq = (N + w.seq_len - 1) // w.seq_len
        adv_seq = torch.empty(n_seq, dtype=torch.float32, device=device).normal_(0.0, 1.0, generator=g)
        out["advantages"] = adv_seq.repeat_interleave(w.seq_len)[:N].contiguous()
        out["old_noise"] = torch.empty(N, dtype=torch.float32, device=device).normal_(
            0.0, w.old_noise_std, generator=g)
        out["grad_init"] = rows_normal(ALL_COMBINED_GRAD_SIGMA)
    else:
        raise KeyError(w.name)
    if w.flags & GSPO:
        starts = torch.arange(0, N, w.seq_len, device=device)
        out["seq_offsets"] = torch.cat([starts, torch.tensor([N], device=device)]).to(torch.int32)
    return out


def segment_offsets(N: int, seed: int, max_len: int = 8, empty_frac: float = 0.1,
                    device="cpu") -> torch.Tensor:
    """Seeded contiguous segments covering N rows: int32 offsets [S + 1] from 0
    to N with lengths in [1, max_len], some empty segments mixed in, and never
    more segments than rows."""
    g = _gen(torch.device("cpu"), seed)
    offs = [0]
    while offs[-1] < N:
        if len(offs) - 1 < N - 1 and torch.rand((1,), generator=g).item() < empty_frac:
            offs.append(offs[-1])
        ln = int(torch.randint(1, max_len + 1, (1,), generator=g).item())
        offs.append(min(N, offs[-1] + ln))
    while len(offs) - 1 > max(N, 1):        # drop empty segments beyond the row count
        for i in range(1, len(offs)):
            if offs[i] == offs[i - 1]:
                del offs[i]
                break
    return torch.tensor(offs, dtype=torch.int32, device=device)


def algorithmic_bytes(w: Workload, n_valid_rows: int, n_rows: int | None = None,
                      with_grad: bool = True) -> int:
    """Bytes the fused pass must move: one read of each valid row's logits
    (and teacher), one write of every gradient row (a masked row's write is
    its zero fill; in accumulate mode masked rows are skipped and valid rows
    also read the existing gradient once), plus the per-token side inputs."""
    N = w.N if n_rows is None else n_rows
    row = w.V * w.elem_bytes
    tensors_read = 1 + (1 if w.flags & (FKL | RKL | FDCE) else 0)
    b = n_valid_rows * tensors_read * row
    if with_grad:
        if w.flags & ACCUMULATE:
            b += n_valid_rows * 2 * row
        else:
            b += N * row
    if with_grad and w.flags & GSPO:
        # the backward reloads every valid row once the segment ratios are known
        b += n_valid_rows * tensors_read * row
    side = 8  # labels
    if w.name in ("grpo_z_ent_bf16", "gspo_z_ent_bf16", "ce_z_grpo_ent_bf16"):
        side += 1  # mask byte
    if w.flags & (GRPO | GSPO):
        side += 8  # old_logprobs + advantages
    return b + N * side


def small_inputs(N: int, V: int, dtype: str, device="cpu", seed: int = 0, *, teacher: bool = False,
                 grpo: bool = False, accumulate: bool = False, ignore_frac: float = 0.1,
                 mask_frac: float = 0.0, bad_labels: int = 0, logit_std: float = 2.0,
                 old_noise_std: float = 0.3, grad_init_std: float = 1e-5) -> dict:
    """Small seeded batches for element-by-element parity checks.

    Logits ~ N(0, logit_std^2); teacher = student / 0.8 + N(0, 1) when asked;
    uniform labels with a fraction set to -100 and ``bad_labels`` rows set to
    out-of-range values; an optional mask byte; per-token advantages ~ N(0, 1)
    and old-logprob noise for GRPO; an existing gradient for accumulation.
    """
    device = torch.device(device)
    g = _gen(device, seed)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    x32 = torch.empty((N, V), dtype=torch.float32, device=device).normal_(0.0, logit_std, generator=g)
    out = {"logits": x32.to(dt), "labels": None, "mask": None, "teacher": None,
           "advantages": None, "old_noise": None, "grad_init": None}
    y = torch.randint(0, V, (N,), generator=g, device=device, dtype=torch.int64)
    if N:
        y[torch.rand((N,), generator=g, device=device) < ignore_frac] = -100
        for i in range(min(bad_labels, N)):
            y[(7 * i + 3) % N] = V + i if i % 2 == 0 else -(i + 2)
    out["labels"] = y
    if mask_frac > 0:
        out["mask"] = (torch.rand((N,), generator=g, device=device) >= mask_frac).to(torch.uint8)
    if teacher:
        nz = torch.empty((N, V), dtype=torch.float32, device=device).normal_(0.0, 1.0, generator=g)
        out["teacher"] = (x32 / 0.8 + nz).to(dt)
    if grpo:
        out["advantages"] = torch.empty(N, dtype=torch.float32, device=device).normal_(0.0, 1.0, generator=g)
        out["old_noise"] = torch.empty(N, dtype=torch.float32, device=device).normal_(
            0.0, old_noise_std, generator=g)
    if accumulate:
        out["grad_init"] = torch.empty((N, V), dtype=torch.float32, device=device).normal_(
            0.0, grad_init_std, generator=g).to(dt)
    return out
