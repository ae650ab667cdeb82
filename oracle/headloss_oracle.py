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
  The same Design section lists three dispatch cases; in the GSPO case a
  per-segment step runs between the forward and a backward that reloads the
  logits, and hands that backward a per-token coefficient on the shared
  label column. The pages name GSPO without a formula; ``gspo_seam`` follows
  the published sequence-level definition (READINGS["gspo"]).

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
GSPO = 128
ACCUMULATE = 1 << 16
HINTON = 1 << 17
DISTILL_FLAGS = FKL | RKL | FDCE
POLICY_FLAGS = GRPO | GSPO

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
        # only; the student keeps its single softmax. With the HINTON mode bit
        # (READINGS["hinton"]) the distillation term also tempers the student,
        # softmax(s / tau), and is multiplied by tau^2.
        tau = spec.temperature
        tt = t / tau
        logp_t = log_softmax_rows(tt)
        p = np.exp(logp_t)
        out["p"] = p
        out["logp_t"] = logp_t
        if spec.has(HINTON):
            logq_d = log_softmax_rows(s / tau)
            scale_d = tau * tau
        else:
            logq_d = logq
            scale_d = 1.0
        q_d = np.exp(logq_d)
        out["logq_d"] = logq_d
        out["q_d"] = q_d
        # READINGS["kl_direction"]: forward = KL(teacher || student),
        # reverse = KL(student || teacher).
        out["kl_d_rev"] = np.sum(q_d * (logq_d - logp_t), axis=-1)     # unscaled reverse KL
        out["fkl"] = scale_d * np.sum(p * (logp_t - logq_d), axis=-1)
        out["rkl"] = scale_d * out["kl_d_rev"]
        # [#549 Loss coverage] "from-distribution cross-entropy": the cross
        # entropy of the student against the teacher distribution.
        out["fdce"] = -scale_d * np.sum(p * logq_d, axis=-1)

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
    With HINTON the distillation student is q_tau = softmax(s / tau) and the
    loss carries tau^2, so d/ds = tau^2 * (1 / tau) * (the same form in q_tau):
      FKL, FDCE: tau * (q_tau - p);   RKL: tau * q_tau * (log q_tau - log p - KL_tau)
    """
    q = vals["q"]
    V = q.shape[1]
    g = {}
    if spec.has(CE):
        g["ce"] = q - _onehot(vals["y"], V)
    if spec.has(ZLOSS):
        g["z"] = 2.0 * vals["lse"][:, None] * q
    f_d = spec.temperature if spec.has(HINTON) else 1.0
    if spec.has(FKL) or spec.has(FDCE):
        g["distill"] = f_d * (vals["q_d"] - vals["p"])
    if spec.has(RKL):
        g["distill"] = f_d * vals["q_d"] * (vals["logq_d"] - vals["logp_t"] - vals["kl_d_rev"][:, None])
    if spec.has(GRPO):
        a = np.where(vals["grpo_active"], vals["adv"] * vals["ratio"], 0.0)
        g["grpo"] = -a[:, None] * (_onehot(vals["y"], V) - q)
    return g


def _check_inputs(spec: Spec, labels, teacher, old_logprobs, advantages):
    if bin(spec.flags & DISTILL_FLAGS).count("1") > 1:
        raise ValueError("at most one distillation loss per plan")
    if spec.has(HINTON) and not (spec.flags & DISTILL_FLAGS):
        raise ValueError("the Hinton temperature mode needs a distillation loss")
    if spec.has(GRPO) and spec.has(GSPO):
        raise ValueError("at most one policy loss per plan")
    if (spec.flags & (CE | POLICY_FLAGS)) and labels is None:
        raise ValueError("CE, GRPO and GSPO need labels")
    if (spec.flags & DISTILL_FLAGS) and teacher is None:
        raise ValueError("distillation needs teacher logits")
    if (spec.flags & POLICY_FLAGS) and (old_logprobs is None or advantages is None):
        raise ValueError("GRPO and GSPO need old_logprobs and advantages")


# ---------------------------------------------------------------------------
# GSPO: the per-segment step between the forward and the backward
# ---------------------------------------------------------------------------
def segment_of_rows(offsets, n_rows: int) -> np.ndarray:
    """Row -> segment index for contiguous segments [o_i, o_{i+1}).

    ``offsets`` has S+1 entries, starts at 0, never decreases and ends at the
    row count (READINGS["segments"]); an empty segment (o_i == o_{i+1}) owns
    no row.
    """
    o = np.asarray(offsets, dtype=np.int64).reshape(-1)
    if o.size < 2 or o[0] != 0 or o[-1] != n_rows or np.any(np.diff(o) < 0):
        raise ValueError("segment offsets must run from 0 to n_rows without decreasing")
    seg = np.empty(n_rows, dtype=np.int64)
    for i in range(o.size - 1):
        seg[o[i]:o[i + 1]] = i
    return seg


def gspo_seam(spec: Spec, logp, old_logprobs, advantages, valid, offsets,
              n_seg_total: int | None = None) -> dict:
    """Per-segment GSPO values and d(batch GSPO loss)/d(logp_t) per row.

    For segment i with valid tokens T_i (n_i = |T_i| > 0), READINGS["gspo"]:
      log s_i = (1/n_i) sum_{t in T_i} (logp_t - old_t)      (length-normalised
                                                               sequence ratio)
      A_i     = (1/n_i) sum_{t in T_i} A_t                   (READINGS["gspo_adv"])
      loss_i  = -min(s_i A_i, clip(s_i, 1-eps, 1+eps) A_i)
    and the batch loss is the mean of loss_i over the segments with n_i > 0.
    Its derivative with respect to logp_t (t in T_i) is -act_i A_i s_i /
    (n_i n_seg), act_i as for the per-token clip (READINGS["grpo_ties"]).
    Segments with no valid token contribute nothing and are not counted.
    ``n_seg_total`` replaces n_seg when the rows given are only some whole
    segments of a larger batch (sampled checks of large batches).
    """
    logp = np.asarray(logp, dtype=np.float64).reshape(-1)
    old = np.asarray(old_logprobs, dtype=np.float64).reshape(-1)
    A = np.asarray(advantages, dtype=np.float64).reshape(-1)
    valid = np.asarray(valid, dtype=bool).reshape(-1)
    N = logp.size
    seg = segment_of_rows(offsets, N)
    S = len(offsets) - 1
    eps = spec.eps
    n_i = np.zeros(S, dtype=np.int64)
    sum_d = np.zeros(S)
    sum_a = np.zeros(S)
    for t in range(N):
        if valid[t]:
            i = seg[t]
            n_i[i] += 1
            sum_d[i] += logp[t] - old[t]
            sum_a[i] += A[t]
    nonempty = n_i > 0
    n_seg = int(nonempty.sum()) if n_seg_total is None else int(n_seg_total)
    safe_n = np.where(nonempty, n_i, 1)
    log_s = np.where(nonempty, sum_d / safe_n, 0.0)
    ratio = np.exp(log_s)
    adv = np.where(nonempty, sum_a / safe_n, 0.0)
    loss = -np.minimum(ratio * adv, np.clip(ratio, 1.0 - eps, 1.0 + eps) * adv)
    active = ~(((adv > 0) & (ratio > 1.0 + eps)) | ((adv < 0) & (ratio < 1.0 - eps)))
    clipped = np.abs(ratio - 1.0) > eps
    k3 = (ratio - 1.0) - log_s
    dlogp = np.zeros(N)
    if n_seg > 0:
        for t in range(N):
            i = seg[t]
            if valid[t] and active[i]:
                dlogp[t] = -adv[i] * ratio[i] / (n_i[i] * n_seg)
    z = ~nonempty
    return {
        "segment": seg, "n_tokens": n_i, "nonempty": nonempty, "n_seg": n_seg,
        "log_ratio": log_s, "ratio": ratio, "adv": adv,
        "loss": np.where(z, 0.0, loss), "active": active,
        "clipped": clipped & nonempty, "k3": np.where(z, 0.0, k3),
        "dlogp": dlogp,
    }


def rows_forward_backward(spec: Spec, x, n: float, labels=None, mask=None,
                          teacher=None, old_logprobs=None, advantages=None,
                          grad_in=None, want_grad=True, gspo_dlogp=None):
    """Per-row values and gradient rows for a subset of a batch.

    ``n`` is the batch-level divisor (valid rows of the whole batch, or the
    caller's divisor); it is an argument so that sampled rows of a large batch
    can be checked one by one. With GSPO, ``gspo_dlogp`` is the per-row
    derivative of the batch GSPO loss with respect to logp_t from
    ``gspo_seam`` (it depends on whole segments, so the caller computes it).
    Returns (vals, valid, bad, grad) where grad is None when ``want_grad`` is
    False.
    """
    _check_inputs(spec, labels, teacher, old_logprobs, advantages)
    if spec.has(GSPO) and want_grad and gspo_dlogp is None:
        raise ValueError("GSPO needs the per-row derivative from gspo_seam")
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
        g_s *= scale
        if spec.has(GSPO) and spec.w_grpo != 0.0:
            # d logp_t / d s_j = onehot(y)_j - q_j; the seam's derivative
            # already carries the segment means' own normalisation.
            d = np.asarray(gspo_dlogp, dtype=np.float64).reshape(-1)
            g_s += (spec.grad_scale * spec.w_grpo) * d[:, None] * (_onehot(vals["y"], V) - vals["q"])
        g_x = transform_derivative(x, spec) * g_s
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
                      n: float, seam: dict | None = None) -> np.ndarray:
    """The 13 output slots: per-loss batch means, the weighted total, counts.

    With GSPO the policy slots hold segment means (READINGS["gspo_slots"]):
    the loss, ratio, clip fraction, k3 of the sequence ratio and advantage
    average over the nonempty segments of ``seam``; NEWLOGP stays a token
    mean.
    """
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
    if spec.has(GSPO):
        out[SLOT["NEWLOGP"]] = mean("logp")
        ns = seam["n_seg"]
        if ns > 0:
            ne = seam["nonempty"]
            out[SLOT["GRPO"]] = float(np.sum(seam["loss"][ne]) / ns)
            out[SLOT["RATIO"]] = float(np.sum(seam["ratio"][ne]) / ns)
            out[SLOT["CLIPFRAC"]] = float(np.sum(seam["clipped"][ne]) / ns)
            out[SLOT["KL_OLD_NEW"]] = float(np.sum(seam["k3"][ne]) / ns)
            out[SLOT["ADV_MEAN"]] = float(np.sum(seam["adv"][ne]) / ns)
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
                     want_grad=True, seq_offsets=None):
    """Whole-batch oracle: (scalars float64[13], grad float64[N, V] or None).

    GSPO needs ``seq_offsets`` (S+1 row offsets of contiguous segments).
    """
    x = np.asarray(x, dtype=np.float64)
    valid, _ = row_validity(x.shape[0], spec.V, labels, mask)
    n = batch_divisor(spec, int(valid.sum()))
    seam = None
    if spec.has(GSPO):
        if seq_offsets is None:
            raise ValueError("GSPO needs segment offsets")
        _check_inputs(spec, labels, teacher, old_logprobs, advantages)
        logp = log_softmax_rows(transform(x, spec))[
            np.arange(x.shape[0]), np.clip(np.asarray(labels, dtype=np.int64).reshape(-1), 0, spec.V - 1)]
        seam = gspo_seam(spec, logp, old_logprobs, advantages, valid, seq_offsets)
    vals, valid, bad, grad = rows_forward_backward(
        spec, x, n, labels, mask, teacher, old_logprobs, advantages,
        grad_in, want_grad, gspo_dlogp=None if seam is None else seam["dlogp"])
    return scalars_from_rows(spec, vals, valid, bad, n, seam), grad


def total_loss(spec: Spec, x, labels=None, mask=None, teacher=None,
               old_logprobs=None, advantages=None, seq_offsets=None) -> float:
    """The scalar the combined gradient differentiates, times grad_scale."""
    sc, _ = forward_backward(spec, x, labels, mask, teacher, old_logprobs,
                             advantages, want_grad=False, seq_offsets=seq_offsets)
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
    "segments": "GSPO segments are contiguous row ranges given by S+1 offsets from 0 to n_rows; empty segments are allowed and own no row.",
    "gspo": "GSPO: sequence ratio s_i = exp(mean over the segment's valid tokens of logp - old); loss_i = -min(s_i A_i, clip(s_i, 1-eps, 1+eps) A_i); batch loss = mean over segments with a valid token; same clip/tie rule as GRPO.",
    "gspo_adv": "A segment's advantage is the mean of its valid tokens' advantages (the broadcast value when the caller repeats one per sequence).",
    "gspo_slots": "With GSPO the policy slots are segment means (loss, ratio, clip fraction, k3 of the sequence ratio, advantage); NEWLOGP stays a token mean; GSPO ignores the caller divisor.",
    "policy_exclusive": "GRPO and GSPO are two policy losses of one kind: a plan holds at most one.",
    "hinton": "Opt-in HINTON mode bit: the distillation term uses softmax(s / tau) for the student as well and is multiplied by tau^2 (so its gradient keeps the tau-independent scale); CE, z-loss, GRPO/GSPO and entropy keep the untempered student softmax; the DISTILL slot reports the tau^2-scaled value.",
}
