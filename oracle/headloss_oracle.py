"""CPU fp64 oracle for the monolithic fused LM-head loss.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or
links this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, constants or
helpers with the HIP library under ``lm_head_vocab_amd/``.

What it computes is the plain definition of each loss and metric, written out
row by row in float64 with numpy, and the analytic gradient of each loss taken
separately and then summed with its weight. The fused kernel reaches the same
numbers by a different route (one shared softmax, two per-row coefficients);
the oracle deliberately does not use that route.

Sources (the pages describe the losses by name only; no page gives an
equation for any of them, so every formula below is the standard definition
of the named quantity, and each reading of an open point is listed in the
``READINGS`` table at the bottom of this module):

* [#507] Fast-LLM issue #507, "Monolithic fused head-loss kernel for
  combinable losses + metrics", sections Problem and Proposed direction: the
  losses and metrics that share one vocabulary softmax (cross-entropy,
  z-loss, distillation, GRPO clipped objective, GRPO ratio/KL/clamp/advantage
  statistics, entropy).
* [#549] Fast-LLM PR #549, "Monolithic fused head-loss kernel
  (torch.compile)", sections Approach (fp32 accumulation, one cast; one
  softmax per logit scale), Loss coverage (label CE, z-loss, forward-KL /
  reverse-KL distillation with temperature, GRPO objective, new_logprobs,
  GRPO metrics, entropy), Correctness (masking, logit scaling, softcap) and
  Bundled fix (the temperature must be honoured).
* [#558] Fast-LLM PR #558, the Triton kernel for the monolithic loss,
  section Design (the gradient is prob_coeff * softmax_j - label_coeff *
  delta(j, label); z-loss adds to prob_coeff only; CE and GRPO share the
  label column) and Validation (masking, logit/grad scaling, gradient
  accumulation, a zero-weight loss that still reports its diagnostics).

Parity status: every function here is pinned by ``tests/test_oracle.py``
(closed forms, a hand-worked example in ``tests/golden/``, torch library
routines, finite differences, invariants). The two GRPO statistics
``KL_OLD_NEW`` and ``ADV_MEAN`` have no definition on the pages at all; their
formulas are readings (k3 estimator, plain mean of the advantages) and are
pinned only against those readings' closed forms, so they are marked
"parity unpinned by the pages" in the test module and in the design notes.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# Flags and output slots. These mirror the C ABI's public numbering (a format
# both sides must agree on); the values are typed out here independently of
# the library headers.
# ---------------------------------------------------------------------------
CE = 1
ZLOSS = 2
FKL = 4
RKL = 8
GRPO = 16
ENTROPY = 32
FDCE = 64
ACCUMULATE = 1 << 16
DISTILL_FLAGS = FKL | RKL | FDCE

IGNORE_INDEX = -100

SLOTS = (
    "CE", "Z", "DISTILL", "GRPO", "NEWLOGP", "RATIO", "CLIPFRAC",
    "KL_OLD_NEW", "ADV_MEAN", "ENTROPY", "TOTAL", "N_VALID", "N_BADLABEL",
)
SLOT = {name: i for i, name in enumerate(SLOTS)}


@dataclass
class Spec:
    """The loss set and its hyper-parameters (one plan in the C ABI)."""

    V: int
    flags: int
    w_ce: float = 1.0
    w_z: float = 0.0
    w_distill: float = 0.0
    w_grpo: float = 0.0
    grad_scale: float = 1.0
    divisor: float = 0.0          # <= 0: divide by the number of valid rows
    temperature: float = 1.0
    eps: float = 0.2
    logit_scale: float = 1.0
    softcap: float = 0.0          # 0: no softcap

    def has(self, flag: int) -> bool:
        return bool(self.flags & flag)


# ---------------------------------------------------------------------------
# Elementary definitions
# ---------------------------------------------------------------------------
def transform(x: np.ndarray, spec: Spec) -> np.ndarray:
    """Student logits as the softmax sees them: s = k*x, or c*tanh(k*x/c).

    [#549 Correctness] lists logit scaling and softcap among the validated
    head variants; the order "scale, then tanh softcap" is the reading used
    throughout (see READINGS["softcap"]).
    """
    k = spec.logit_scale
    if spec.softcap > 0:
        c = spec.softcap
        return c * np.tanh(k * x / c)
    return k * x


def transform_derivative(x: np.ndarray, spec: Spec) -> np.ndarray:
    """ds/dx of ``transform``: k, or k*(1 - tanh(k*x/c)**2)."""
    k = spec.logit_scale
    if spec.softcap > 0:
        c = spec.softcap
        th = np.tanh(k * x / c)
        return k * (1.0 - th * th)
    return np.full_like(x, k)


def logsumexp_rows(s: np.ndarray) -> np.ndarray:
    """log(sum_j exp(s_j)) per row, computed with the max shifted out."""
    m = np.max(s, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(s - m), axis=-1, keepdims=True)))[..., 0]


def log_softmax_rows(s: np.ndarray) -> np.ndarray:
    return s - logsumexp_rows(s)[..., None]


# ---------------------------------------------------------------------------
# Row validity ([#549 Correctness] / [#558 Validation]: "masking")
# ---------------------------------------------------------------------------
def row_validity(n_rows: int, V: int, labels=None, mask=None):
    """Return (valid[bool N], bad_label[bool N]).

    A row is valid unless its mask byte is 0 or its label is the ignore index
    -100 (READINGS["masking"]). An unmasked row whose label is neither -100
    nor in [0, V) is treated as masked and counted as a bad label
    (READINGS["bad_labels"]).
    """
    unmasked = np.ones(n_rows, dtype=bool)
    if mask is not None:
        unmasked &= np.asarray(mask).reshape(n_rows) != 0
    bad = np.zeros(n_rows, dtype=bool)
    valid = unmasked.copy()
    if labels is not None:
        y = np.asarray(labels, dtype=np.int64).reshape(n_rows)
        ignored = y == IGNORE_INDEX
        out_of_range = (~ignored) & ((y < 0) | (y >= V))
        bad = unmasked & out_of_range
        valid &= ~ignored & ~out_of_range
    return valid, bad


# ---------------------------------------------------------------------------
# Per-row loss and metric values
# ---------------------------------------------------------------------------
def row_values(spec: Spec, x, labels=None, teacher=None, old_logprobs=None,
               advantages=None) -> dict:
    """Every per-row quantity the head can report, for every row given.

    ``x`` and ``teacher`` are [R, V] arrays (any float dtype, converted to
    float64 exactly). Rows that are invalid still get values here; the caller
    decides which rows count. Quantities whose inputs are missing are absent
    from the result.
    """
    x = np.asarray(x, dtype=np.float64)
    s = transform(x, spec)
    lse = logsumexp_rows(s)
    logq = s - lse[:, None]
    q = np.exp(logq)
    out = {"s": s, "lse": lse, "logq": logq, "q": q}

    # [#507 Problem], [#549 Loss coverage]: z-loss is a function of the
    # student's sum_exp_logits; its standard form is the squared
    # log-partition (READINGS["z_loss"]).
    out["z"] = lse * lse
    # [#507 Problem] "entropy metric": Shannon entropy of the student softmax.
    out["entropy"] = -np.sum(q * logq, axis=-1)

    if labels is not None:
        y = np.asarray(labels, dtype=np.int64).reshape(-1)
        y_safe = np.where((y >= 0) & (y < spec.V), y, 0)
        rows = np.arange(x.shape[0])
        logp_y = logq[rows, y_safe]
        out["y"] = y_safe
        # [#549 Loss coverage] label cross-entropy: -log q_y.
        out["ce"] = -logp_y
        # [#549 Loss coverage] new_logprobs: log q_y in the transformed space.
        out["logp"] = logp_y

    if teacher is not None:
        t = np.asarray(teacher, dtype=np.float64)
        # READINGS["temperature"]: the temperature divides the teacher logits
        # only; the student keeps its single softmax.
        tt = t / spec.temperature
        logp_t = log_softmax_rows(tt)
        p = np.exp(logp_t)
        out["p"] = p
        out["logp_t"] = logp_t
        # READINGS["kl_direction"]: forward = KL(teacher || student),
        # reverse = KL(student || teacher).
        out["fkl"] = np.sum(p * (logp_t - logq), axis=-1)
        out["rkl"] = np.sum(q * (logq - logp_t), axis=-1)
        # [#549 Loss coverage] "from-distribution cross-entropy": the cross
        # entropy of the student against the teacher distribution.
        out["fdce"] = -np.sum(p * logq, axis=-1)

    if labels is not None and old_logprobs is not None and advantages is not None:
        old = np.asarray(old_logprobs, dtype=np.float64).reshape(-1)
        A = np.asarray(advantages, dtype=np.float64).reshape(-1)
        eps = spec.eps
        logp = out["logp"]
        r = np.exp(logp - old)
        # [#507 Proposed direction] "GRPO clipped objective": the per-token
        # PPO-clip surrogate, loss = -min(r*A, clip(r, 1-eps, 1+eps)*A)
        # (READINGS["grpo"]).
        unclipped = r * A
        clipped = np.clip(r, 1.0 - eps, 1.0 + eps) * A
        out["grpo"] = -np.minimum(unclipped, clipped)
        out["ratio"] = r
        # The gradient flows through the unclipped term unless the clip is
        # strictly active in the direction the advantage pushes
        # (READINGS["grpo_ties"]).
        out["grpo_active"] = ~(((A > 0) & (r > 1.0 + eps)) | ((A < 0) & (r < 1.0 - eps)))
        # READINGS["clip_stat"]: the clamp statistic counts |r - 1| > eps.
        out["clipped"] = np.abs(r - 1.0) > eps
        # READINGS["kl_stat"]: k3 estimator of KL(new || old) per token.
        out["k3"] = (r - 1.0) - (logp - old)
        out["adv"] = A
    return out


# ---------------------------------------------------------------------------
# Per-row gradients, one loss at a time
# ---------------------------------------------------------------------------
def _onehot(y: np.ndarray, V: int) -> np.ndarray:
    oh = np.zeros((y.shape[0], V), dtype=np.float64)
    oh[np.arange(y.shape[0]), y] = 1.0
    return oh


def loss_gradients_wrt_s(spec: Spec, vals: dict) -> dict:
    """d(per-row loss)/d(s_j) for each enabled loss, as separate arrays.

    Each is the textbook derivative of that loss alone:
      CE:   q - onehot(y)
      z:    2 * lse * q
      FKL:  q - p
      FDCE: q - p          (the teacher entropy does not depend on the student)
      RKL:  q * (log q - log p - RKL)
      GRPO: -act * A * r * (onehot(y) - q)      (d logp_y / ds = onehot - q)
    """
    q = vals["q"]
    V = q.shape[1]
    g = {}
    if spec.has(CE):
        g["ce"] = q - _onehot(vals["y"], V)
    if spec.has(ZLOSS):
        g["z"] = 2.0 * vals["lse"][:, None] * q
    if spec.has(FKL) or spec.has(FDCE):
        g["distill"] = q - vals["p"]
    if spec.has(RKL):
        g["distill"] = q * (vals["logq"] - vals["logp_t"] - vals["rkl"][:, None])
    if spec.has(GRPO):
        a = np.where(vals["grpo_active"], vals["adv"] * vals["ratio"], 0.0)
        g["grpo"] = -a[:, None] * (_onehot(vals["y"], V) - q)
    return g


def _check_inputs(spec: Spec, labels, teacher, old_logprobs, advantages):
    if bin(spec.flags & DISTILL_FLAGS).count("1") > 1:
        raise ValueError("at most one distillation loss per plan")
    if (spec.has(CE) or spec.has(GRPO)) and labels is None:
        raise ValueError("CE and GRPO need labels")
    if (spec.flags & DISTILL_FLAGS) and teacher is None:
        raise ValueError("distillation needs teacher logits")
    if spec.has(GRPO) and (old_logprobs is None or advantages is None):
        raise ValueError("GRPO needs old_logprobs and advantages")


def rows_forward_backward(spec: Spec, x, n: float, labels=None, mask=None,
                          teacher=None, old_logprobs=None, advantages=None,
                          grad_in=None, want_grad=True):
    """Per-row values and gradient rows for a subset of a batch.

    ``n`` is the batch-level divisor (valid rows of the whole batch, or the
    caller's divisor); it is an argument so that sampled rows of a large batch
    can be checked one by one. Returns (vals, valid, bad, grad) where grad is
    None when ``want_grad`` is False.
    """
    _check_inputs(spec, labels, teacher, old_logprobs, advantages)
    x = np.asarray(x, dtype=np.float64)
    R, V = x.shape
    assert V == spec.V
    valid, bad = row_validity(R, V, labels, mask)
    vals = row_values(spec, x, labels, teacher, old_logprobs, advantages)
    grad = None
    if want_grad:
        weights = {"ce": spec.w_ce, "z": spec.w_z, "distill": spec.w_distill,
                   "grpo": spec.w_grpo}
        per_loss = loss_gradients_wrt_s(spec, vals)
        g_s = np.zeros_like(x)
        for name, gk in per_loss.items():
            if weights[name] != 0.0:
                g_s += weights[name] * gk
        scale = spec.grad_scale / n if n > 0 else 0.0
        g_x = scale * transform_derivative(x, spec) * g_s
        g_x[~valid] = 0.0
        if grad_in is not None and spec.has(ACCUMULATE):
            base = np.asarray(grad_in, dtype=np.float64)
            # masked rows keep the existing values (READINGS["masked_accumulate"])
            grad = np.where(valid[:, None], base + g_x, base)
        else:
            grad = g_x
    return vals, valid, bad, grad


def batch_divisor(spec: Spec, n_valid: int) -> float:
    """READINGS["divisor"]: mean over valid rows unless the caller gives one."""
    if spec.divisor > 0:
        return float(spec.divisor)
    return float(n_valid)


def scalars_from_rows(spec: Spec, vals: dict, valid: np.ndarray, bad: np.ndarray,
                      n: float) -> np.ndarray:
    """The 13 output slots: per-loss batch means, the weighted total, counts."""
    out = np.zeros(len(SLOTS), dtype=np.float64)
    n_valid = int(valid.sum())

    def mean(key):
        if key not in vals or n <= 0:
            return 0.0
        return float(np.sum(vals[key][valid]) / n)

    if spec.has(CE):
        out[SLOT["CE"]] = mean("ce")
    if spec.has(ZLOSS):
        out[SLOT["Z"]] = mean("z")
    if spec.has(FKL):
        out[SLOT["DISTILL"]] = mean("fkl")
    if spec.has(RKL):
        out[SLOT["DISTILL"]] = mean("rkl")
    if spec.has(FDCE):
        out[SLOT["DISTILL"]] = mean("fdce")
    if spec.has(GRPO):
        out[SLOT["GRPO"]] = mean("grpo")
        out[SLOT["NEWLOGP"]] = mean("logp")
        out[SLOT["RATIO"]] = mean("ratio")
        if n > 0:
            out[SLOT["CLIPFRAC"]] = float(np.sum(vals["clipped"][valid]) / n)
        out[SLOT["KL_OLD_NEW"]] = mean("k3")
        out[SLOT["ADV_MEAN"]] = mean("adv")
    if spec.has(ENTROPY):
        out[SLOT["ENTROPY"]] = mean("entropy")
    # [#549 Approach] each loss stores its own scalar; the weighted total is
    # what the combined gradient differentiates. Entropy is a metric only.
    out[SLOT["TOTAL"]] = (spec.w_ce * out[SLOT["CE"]] + spec.w_z * out[SLOT["Z"]]
                          + spec.w_distill * out[SLOT["DISTILL"]]
                          + spec.w_grpo * out[SLOT["GRPO"]])
    out[SLOT["N_VALID"]] = n_valid
    out[SLOT["N_BADLABEL"]] = int(bad.sum())
    return out


def forward_backward(spec: Spec, x, labels=None, mask=None, teacher=None,
                     old_logprobs=None, advantages=None, grad_in=None,
                     want_grad=True):
    """Whole-batch oracle: (scalars float64[13], grad float64[N, V] or None)."""
    x = np.asarray(x, dtype=np.float64)
    valid, _ = row_validity(x.shape[0], spec.V, labels, mask)
    n = batch_divisor(spec, int(valid.sum()))
    vals, valid, bad, grad = rows_forward_backward(
        spec, x, n, labels, mask, teacher, old_logprobs, advantages,
        grad_in, want_grad)
    return scalars_from_rows(spec, vals, valid, bad, n), grad


def total_loss(spec: Spec, x, labels=None, mask=None, teacher=None,
               old_logprobs=None, advantages=None) -> float:
    """The scalar the combined gradient differentiates, times grad_scale."""
    sc, _ = forward_backward(spec, x, labels, mask, teacher, old_logprobs,
                             advantages, want_grad=False)
    return spec.grad_scale * sc[SLOT["TOTAL"]]


# ---------------------------------------------------------------------------
# Readings of points the pages leave open (mirrored in the design notes)
# ---------------------------------------------------------------------------
READINGS = {
    "divisor": "Batch means divide by the number of valid rows; a positive caller divisor replaces it for scalars and gradient alike.",
    "empty": "With no valid row every scalar is 0 and the gradient is 0.",
    "masking": "A row is masked when its mask byte is 0 or its label is -100; the mask applies to every loss and metric.",
    "bad_labels": "An unmasked label outside [0, V) other than -100 masks the row and is counted in N_BADLABEL.",
    "z_loss": "z-loss per row is lse**2 (the squared log of sum_exp_logits).",
    "temperature": "The temperature divides the teacher logits only, with no tau**2 factor.",
    "teacher_transform": "Logit scale and softcap apply to the student only.",
    "kl_direction": "Forward KL = KL(teacher || student); reverse KL = KL(student || teacher).",
    "fdce": "From-distribution cross-entropy = -sum_j p_j log q_j with the tempered teacher p; gradient q - p.",
    "grpo": "Per-token PPO-clip with symmetric eps, no KL penalty, loss = -objective, mean over valid tokens.",
    "grpo_ties": "At r exactly 1 +/- eps the gradient flows (clip only on a strict inequality).",
    "clip_stat": "CLIPFRAC = mean of [|r - 1| > eps].",
    "kl_stat": "KL_OLD_NEW = mean of k3 = (r - 1) - log r; ADV_MEAN = mean advantage over valid rows.",
    "entropy": "Entropy is a metric: no gradient, no weight, excluded from TOTAL.",
    "softcap": "s = c * tanh(k * x / c): scale first, then cap; c = 0 disables it.",
    "weights": "Slots are unweighted means; TOTAL and the gradient use the weights.",
    "rounding": "The gradient is formed in fp32 and rounded once to the output dtype; accumulate adds in fp32 and rounds once.",
    "masked_accumulate": "Masked rows: overwrite mode writes +0.0, accumulate mode leaves the buffer untouched.",
    "nan": "NaN and Inf inputs propagate; nothing is sanitised.",
    "newlogp_space": "new_logprobs live in the transformed (scaled, softcapped) space, the same softmax the losses use.",
}
