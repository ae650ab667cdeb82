/*
 * headloss.h - C ABI of the MI355X fused language-model head loss.
 *
 * One call takes one row of logits per token over the whole vocabulary,
 * computes the student softmax once in fp32, and from that one shared softmax
 * emits every requested loss / metric scalar and the single combined logits
 * gradient. This is the "monolithic" head loss of Fast-LLM issue #507
 * ("Monolithic fused head-loss kernel for combinable losses + metrics",
 * section Proposed direction: run the softmax once, emit all requested
 * scalars and the combined gradient in one pass), with the loss set of
 * Fast-LLM PR #549 ("Monolithic fused head-loss kernel (torch.compile)",
 * section Loss coverage) and the gradient split of Fast-LLM PR #558 (the
 * Triton kernel for the monolithic loss, section Design):
 *
 *     grad_j = prob_coeff * softmax_j - label_coeff * delta(j, label)
 *              + distillation term
 *
 * Conventions for every entry point:
 *  - Pointers named dev_* or documented as "device" point to GPU memory
 *    allocated by the caller (e.g. by PyTorch); the library never frees them
 *    and keeps no reference to them after the call returns.
 *  - Every check is made on the host, before anything is enqueued; a call
 *    that returns an error has enqueued nothing. No kernel traps.
 *  - Calls that enqueue work are asynchronous on the given HIP stream
 *    (NULL = the default stream); results are valid after the stream is
 *    synchronised.
 */
#ifndef HEADLOSS_H
#define HEADLOSS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
typedef enum {
    HL_OK = 0,
    HL_ERR_INVALID_ARG = 1,   /* a value or pointer is out of its documented range */
    HL_ERR_MISSING_INPUT = 2, /* an enabled loss lacks one of its inputs */
    HL_ERR_UNSUPPORTED = 3,   /* a valid request this build does not implement */
    HL_ERR_WORKSPACE = 4,     /* no workspace, or one too small for n_rows */
    HL_ERR_HIP = 5            /* a HIP runtime call or kernel launch failed */
} hl_status;

/* Element type of logits, teacher logits and gradient (all three share it).
 * fp16 inputs are among the dtypes the monolithic kernel is validated with
 * (#558 Validation); an fp16 gradient underflows below 6e-8 (use grad_scale).
 * HL_F32 plans keep the softmax statistics, the per-row coefficients and each
 * gradient element in fp64 internally and round once on output; bf16 and fp16
 * plans compute in fp32 (#549 Approach: fp32 accumulation, one cast). */
typedef enum { HL_F32 = 0, HL_BF16 = 1, HL_F16 = 2 } hl_dtype;

/* Loss and metric flags (#507 Proposed direction: a flag set naming the
 * losses and metrics to emit). At most one of HL_FKL, HL_RKL, HL_FDCE per plan
 * (#558 What it does: at most one loss of each kind). */
enum {
    HL_CE = 1u << 0,       /* label cross-entropy  -log softmax_y            */
    HL_ZLOSS = 1u << 1,    /* z-loss  (log sum_j exp s_j)^2                  */
    HL_FKL = 1u << 2,      /* distillation, KL(teacher || student)           */
    HL_RKL = 1u << 3,      /* distillation, KL(student || teacher)           */
    HL_GRPO = 1u << 4,     /* GRPO clipped objective + new-logprob/ratio/
                              clamp/KL/advantage statistics                  */
    HL_ENTROPY = 1u << 5,  /* entropy metric (no gradient)                   */
    HL_FDCE = 1u << 6,     /* distillation, cross-entropy of the student
                              against the teacher distribution, -sum p log q
                              (#549 Loss coverage: from-distribution
                              cross-entropy); gradient as HL_FKL            */
    HL_GSPO = 1u << 7,     /* GSPO: the clipped objective on the sequence-
                              level ratio s_i = exp(mean over segment i's
                              valid tokens of logp - old), averaged over
                              segments; needs hl_forward_backward_segments.
                              At most one of HL_GRPO, HL_GSPO per plan.     */
    HL_ACCUMULATE = 1u << 16, /* mode bit: add into grad_out instead of
                                overwriting it (#558 Validation: gradient
                                accumulation)                                */
    HL_HINTON = 1u << 17     /* mode bit, with a distillation flag: the
                                distillation term also tempers the student,
                                softmax(s / temperature), and is multiplied by
                                temperature^2 (the DISTILL slot reports that
                                scaled value); CE, z-loss, policy losses and
                                entropy keep the untempered softmax. Without
                                it the temperature divides the teacher only
                                (#549 Loss coverage: distillation with
                                temperature; both readings are offered).     */
};

/* Loss weights and gradient scaling. Each scalar slot reports its loss
 * unweighted (#558 Design: every loss stores its own forward scalar); the
 * weights enter TOTAL and the gradient only. A zero weight keeps the loss's
 * scalars and removes its gradient term (#558 Validation: a zero-weight loss
 * still logs its diagnostics). */
typedef struct {
    float ce;         /* weight of HL_CE                                    */
    float z;          /* weight of HL_ZLOSS                                 */
    float distill;    /* weight of HL_FKL / HL_RKL / HL_FDCE                */
    float grpo;       /* weight of HL_GRPO or HL_GSPO                       */
    float grad_scale; /* extra factor on the gradient only (G)              */
    float divisor;    /* > 0: divide sums by this; <= 0: by the number of
                         valid rows of the call                             */
} hl_weights;

/* Output slots of scalars_out (device float[HL_NUM_SCALARS]). Slots of
 * losses that are not enabled are written as 0. With HL_GSPO the policy slots
 * GRPO (the GSPO loss), RATIO, CLIPFRAC, KL_OLD_NEW and ADV_MEAN are means
 * over the segments that hold a valid token, of the segment's loss, sequence
 * ratio s_i, clipped flag |s_i - 1| > eps, (s_i - 1) - log s_i and advantage;
 * NEWLOGP stays a mean over valid tokens. */
enum {
    HL_S_CE = 0, HL_S_Z, HL_S_DISTILL, HL_S_GRPO, HL_S_NEWLOGP, HL_S_RATIO,
    HL_S_CLIPFRAC, HL_S_KL_OLD_NEW, HL_S_ADV_MEAN, HL_S_ENTROPY, HL_S_TOTAL,
    HL_S_N_VALID, HL_S_N_BADLABEL,
    HL_NUM_SCALARS
};

/* Per-row value columns (see hl_row_values). */
enum {
    HL_R_CE = 0, HL_R_Z, HL_R_DISTILL, HL_R_GRPO, HL_R_NEWLOGP, HL_R_RATIO,
    HL_R_CLIPPED, HL_R_K3, HL_R_ADV, HL_R_ENTROPY, HL_R_VALID, HL_R_PAD,
    HL_NUM_ROW_COLS
};

typedef struct hl_plan_s* hl_plan_t;

/*
 * hl_plan - validate a loss set and choose the kernel variant for it.
 *
 * Defines the operation of #507 Proposed direction (one softmax, every
 * requested scalar, one combined gradient) for rows of length V.
 *   out          receives the plan handle (host pointer, must not be NULL).
 *   V            vocabulary size, >= 1.
 *   dtype        element type of logits / teacher / gradient.
 *   loss_flags   OR of HL_* loss flags (at least one loss or metric) and
 *                optionally HL_ACCUMULATE.
 *   weights      host pointer; all fields finite.
 *   temperature  divides the teacher logits (distillation only), > 0
 *                (#549 Bundled fix: the temperature is honoured).
 *   eps          GRPO / GSPO clip range, 0 < eps < 1 (policy losses only).
 *   logit_scale  student logits are multiplied by it, finite and > 0; one
 *                plan = one scale (#549 Approach: one softmax = one scale).
 *   softcap      0 = off; > 0: s = softcap * tanh(logit_scale * x / softcap).
 * Makes no HIP call. Errors: HL_ERR_INVALID_ARG (V < 1, unknown flag bits,
 * no loss flag, two distillation flags, HL_GRPO with HL_GSPO, HL_HINTON
 * without a distillation flag, temperature <= 0 with distillation, eps outside (0,1) with a policy loss, bad scale or
 * softcap, non-finite weight),
 * HL_ERR_UNSUPPORTED (V >= 2^31: element indices within a row are 32-bit).
 * Rows longer than the slices the on-device chunk exchange serves (9 chunks
 * x 1024 threads x 20 student or 10 student + teacher vectors of 16 bytes;
 * 8 chunks for HL_FDCE with HL_HINTON) take two launches: the statistics are
 * streamed first, then the fused kernel writes the gradient from them with
 * as many chunks as the row needs (each row read twice); hl_plan_describe
 * reports that chunk count.
 */
hl_status hl_plan(hl_plan_t* out, int64_t V, hl_dtype dtype, uint32_t loss_flags,
                  const hl_weights* weights, float temperature, float eps,
                  float logit_scale, float softcap);

/* Release a plan and any workspace the library allocated for it. NULL is a
 * no-op. The caller must have synchronised work that uses the plan. */
void hl_plan_destroy(hl_plan_t plan);

/* Bytes of device workspace a call with n_rows rows needs (0 on a NULL plan
 * or negative n_rows). Independent of the data. */
size_t hl_workspace_bytes(hl_plan_t plan, int64_t n_rows);

/* Give the plan caller-owned device workspace (256-byte aligned, at least
 * hl_workspace_bytes(plan, n_rows) for every later call). Replaces any
 * workspace the library allocated. Makes no HIP call: the next call clears
 * whatever part of the workspace must start at zero, on its own stream.
 * Several plans may share one workspace (their calls must not overlap in
 * time): the workspace's own control words record what its split-vocab
 * region holds, whichever plan wrote it last.
 * Errors: HL_ERR_INVALID_ARG (NULL plan or pointer, misaligned pointer). */
hl_status hl_plan_set_workspace(hl_plan_t plan, void* dev_workspace, size_t bytes);

/*
 * hl_forward_backward - the fused pass (#507 Proposed direction; #549
 * Approach; #558 Design).
 *   n_rows          number of tokens N >= 0 (0: scalars are all written 0).
 *   logits          device [N, V] row-major contiguous, plan dtype, base
 *                   aligned to the element size. Raw student logits.
 *   labels          device int64[N] or NULL; -100 = ignored token. Needed by
 *                   HL_CE, HL_GRPO and HL_GSPO. An unmasked label outside [0, V) that
 *                   is not -100 masks the row and counts in N_BADLABEL.
 *   mask            device uint8[N] or NULL; 0 = masked token. Masking
 *                   applies to every loss and metric.
 *   teacher_logits  device [N, V], plan dtype, element-aligned base, or
 *                   NULL; needed by HL_FKL / HL_RKL / HL_FDCE.
 *   old_logprobs    device float[N] or NULL; needed by HL_GRPO.
 *   advantages      device float[N] (per token) or NULL; needed by HL_GRPO.
 *   grad_out        device [N, V], plan dtype, element-aligned base, or NULL
 *                   (NULL: metrics only, no gradient written; the row
 *                   statistics then come from a streaming kernel, so the
 *                   scalars agree with a gradient call's to float rounding,
 *                   not bit for bit). Overwrite
 *                   mode writes every element (masked rows +0.0);
 *                   HL_ACCUMULATE adds in fp32 (HL_F32 plans: fp64) and
 *                   rounds once, and leaves masked rows untouched.
 *   scalars_out     device float[HL_NUM_SCALARS], must not be NULL.
 *   stream          HIP stream for all work of the call.
 * Alignment: rows are split into 16-byte vectors (plus a head and a tail of
 * single elements when V * element size is not a multiple of 16); this needs
 * the logits, teacher and gradient bases to agree modulo 16 bytes (as 16-byte
 * aligned allocations, PyTorch's among them, do). When they do not, a row-wise
 * kernel with element loads and stores computes the same results, more
 * slowly; it is never an error.
 * Gradient with respect to the raw logits of a valid row:
 *   grad_scale / n * ds/dx * sum_k weight_k * dloss_k/ds
 * with n the number of valid rows (or weights.divisor when > 0).
 * Split-vocab rows (several workgroups per row) combine their statistics on
 * the device with a bounded wait. If a workgroup gives up waiting (its
 * siblings were never scheduled beside it), it writes NaN into its part of
 * the row's gradient (and, for the row's first part, the row's values), and
 * every float scalar of the call is NaN: a failed combine never yields a
 * finite wrong result in the parts it writes.
 * Errors: HL_ERR_INVALID_ARG (NULL plan, n_rows < 0, NULL logits or
 * scalars_out, a base not aligned to the element size), HL_ERR_MISSING_INPUT (see above),
 * HL_ERR_WORKSPACE (a workspace that is too small was set by the caller),
 * HL_ERR_HIP. Allocates device memory only when no workspace was set (first
 * call, or a larger n_rows than before); the allocation is kept by the plan.
 * Concurrent calls with one plan race on its workspace: use one plan per
 * stream.
 */
hl_status hl_forward_backward(hl_plan_t plan, int64_t n_rows, const void* logits,
                              const int64_t* labels, const uint8_t* mask,
                              const void* teacher_logits, const float* old_logprobs,
                              const float* advantages, void* grad_out,
                              float* scalars_out, hipStream_t stream);

/*
 * hl_forward_backward_segments - hl_forward_backward with sequence segments,
 * required by HL_GSPO (and accepted, then ignored, by every other plan).
 * The GSPO case of #558 Design: a forward pass computes every row's softmax
 * statistics, a per-segment step turns them into sequence ratios and a
 * per-token label-column coefficient, and a backward that reloads the logits
 * writes the combined gradient. The logits (and teacher) are therefore read
 * twice.
 *   seq_offsets  device int32[n_segments + 1]: segment i is rows
 *                [seq_offsets[i], seq_offsets[i+1]); the offsets start at 0,
 *                never decrease and end at n_rows (empty segments allowed).
 *                Needed by HL_GSPO. Checked on the device: malformed offsets
 *                make every float scalar and the gradient NaN.
 *   n_segments   1 <= n_segments <= n_rows when n_rows > 0 (0 allowed when
 *                n_rows == 0).
 *   old_logprobs, advantages: per token, as for HL_GRPO; a segment's
 *                advantage is the mean over its valid tokens.
 * The GSPO gradient of a valid token t in segment i is
 *   grad_scale * weights.grpo * act_i * A_i * s_i / (n_i * n_seg)
 *   * ds/dx * (softmax - onehot(label)),
 * with n_i the segment's valid tokens, n_seg the segments holding a valid
 * token, act_i = 0 when the clip is strictly active in the advantage's
 * direction (weights.divisor does not apply to GSPO).
 * Other arguments, errors and asynchrony as hl_forward_backward, plus
 * HL_ERR_INVALID_ARG (n_segments out of range) and HL_ERR_MISSING_INPUT
 * (HL_GSPO without seq_offsets). hl_forward_backward on an HL_GSPO plan
 * returns HL_ERR_MISSING_INPUT.
 */
hl_status hl_forward_backward_segments(hl_plan_t plan, int64_t n_rows, const void* logits,
                                       const int64_t* labels, const uint8_t* mask,
                                       const void* teacher_logits, const float* old_logprobs,
                                       const float* advantages, const int32_t* seq_offsets,
                                       int64_t n_segments, void* grad_out,
                                       float* scalars_out, hipStream_t stream);

/* Size of the library's static per-GPU workspace used by
 * hl_forward_backward_noalloc. */
#define HL_STATIC_WORKSPACE_BYTES (32u * 1024u * 1024u)

/*
 * hl_forward_backward_noalloc - hl_forward_backward_segments for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The call makes no device allocation
 * and no allocating library call: its workspace is a fixed device array of
 * HL_STATIC_WORKSPACE_BYTES inside the library, one per GPU, held from the
 * first such call on that GPU until the process ends (the current device's
 * copy is used; the stream must belong to that device). Arguments, results,
 * asynchrony and kernels are those of hl_forward_backward_segments
 * (seq_offsets may be NULL and n_segments 0 for plans without HL_GSPO), and
 * the plan's own workspace, if any, is not touched; hl_row_values then points
 * into the static array. Every call on one GPU, from any plan, shares that
 * GPU's array and leaves its contents for the next call (each call clears
 * what must start at zero itself): calls that overlap in time on one GPU
 * race and must not be issued. Errors: those of
 * hl_forward_backward_segments, plus HL_ERR_WORKSPACE when the call needs
 * more than HL_STATIC_WORKSPACE_BYTES (hl_workspace_bytes(plan, n_rows) tells
 * in advance; hl_last_error names the sizes), HL_ERR_UNSUPPORTED for a device
 * index above 63, HL_ERR_HIP if the array's address cannot be obtained.
 */
hl_status hl_forward_backward_noalloc(hl_plan_t plan, int64_t n_rows, const void* logits,
                                      const int64_t* labels, const uint8_t* mask,
                                      const void* teacher_logits, const float* old_logprobs,
                                      const float* advantages, const int32_t* seq_offsets,
                                      int64_t n_segments, void* grad_out, float* scalars_out,
                                      hipStream_t stream);

/* Device pointer to the per-row values of the plan's last call: float
 * [n_rows, HL_NUM_ROW_COLS] inside the workspace (masked rows are all 0,
 * HL_R_VALID is 1 for counted rows; HL_R_ENTROPY is 0 unless HL_ENTROPY is
 * requested; with HL_GSPO the policy columns hold the row's segment values). Valid until the next call with the plan
 * or a workspace change. These are the per-token values the batch means of
 * #549 Loss coverage are taken over (new_logprobs, entropy, ratio, ...).
 * Returns NULL before the plan's first call. The values live in the
 * workspace the call used (the plan's, or the static one of
 * hl_forward_backward_noalloc). */
const float* hl_row_values(hl_plan_t plan);

/* Override the number of vocabulary chunks per row (0 = automatic). More than
 * one chunk selects the split-vocab variant: each row is spread over several
 * workgroups whose softmax statistics are combined before the gradient pass
 * (the looped multi-block path of #558 Validation). A successful change
 * releases a library-owned workspace; a caller-owned one must be set again
 * with hl_plan_set_workspace before the next call (HL_ERR_WORKSPACE until
 * then). Errors: HL_ERR_INVALID_ARG (chunks < 0 or > 9),
 * HL_ERR_UNSUPPORTED (no variant fits V with that many chunks, or more
 * chunks than the exchange serves: one wave polls all of a row's exchanged
 * words, at most 64, and a chunk exchanges 3 statistics without a teacher,
 * 6 with one, one more with HL_FDCE and one more with HL_HINTON; HL_F32 plans
 * add the low parts of their 1 to 3 normalizers. So at most 8 chunks with
 * HL_FDCE | HL_HINTON, and for HL_F32 plans 9 / 8 / 7 / 6 / 5 chunks without a
 * teacher / forward or reverse KL / FDCE / Hinton KL / Hinton FDCE). */
hl_status hl_plan_set_chunks(hl_plan_t plan, int chunks);

/* Tuning form of hl_plan_set_chunks that also fixes the threads per
 * workgroup (256, 512 or 1024; 0 = automatic, which requires chunks = 0 too
 * or picks the smallest block that fits). Same errors as hl_plan_set_chunks,
 * plus HL_ERR_INVALID_ARG for another block size or a block without chunks. */
hl_status hl_plan_set_variant(hl_plan_t plan, int chunks, int block);

/* Describe the chosen variant: chunks per row, threads per workgroup, 16-byte
 * vectors held per thread per tensor. Any pointer may be NULL. */
hl_status hl_plan_describe(hl_plan_t plan, int* chunks, int* block, int* vec_per_thread);

/* Record the two events (hipEvent_t, may be NULL to stop) immediately before
 * and after the fused kernel of every later call (with HL_GSPO: before the
 * forward launch and after the load-mode launch of the fused kernel), on the
 * call's stream, so a profiler can time the dominant kernel alone. */
hl_status hl_plan_set_timing_events(hl_plan_t plan, hipEvent_t before, hipEvent_t after);

/* Failure handling test hook (split-vocab rows): bound the device-side
 * wait of later calls to spin_limit polls (>= 1; the default is 2^20), and
 * make the workgroup that owns vocabulary chunk withhold_chunk of row
 * withhold_row skip publishing its statistics (withhold_row < 0: none), so
 * that every workgroup of that row gives up its wait and the call takes the
 * failure path described at hl_forward_backward; every kernel still ends.
 * Errors: HL_ERR_INVALID_ARG (NULL plan, spin_limit 0). */
hl_status hl_plan_set_exchange_test(hl_plan_t plan, uint32_t spin_limit, int64_t withhold_row,
                                    int withhold_chunk);

/* Measurement aid (Fast-LLM PR #549, section Performance: the fused path
 * is judged by the memory traffic it moves): the memory system's rate for
 * the fused kernel's traffic shape, with no arithmetic. Each workgroup of
 * `block` threads (512 or 1024) reads vec_per_thread (4, 6, 8, 9 or 10; 13
 * at 512 threads) 16-byte vectors per thread from read0 (and read1, if not NULL) into
 * registers, issuing every load before any use, then writes their bitwise
 * xor to `write`; each buffer holds `bytes` bytes (a multiple of 16, 16-byte
 * aligned device pointers; `write` is overwritten). One warm-up launch, then
 * `reps` timed launches on `stream` (this call synchronizes it);
 * *ms_per_launch receives the mean. Errors: HL_ERR_INVALID_ARG (NULL
 * pointer, size or alignment), HL_ERR_UNSUPPORTED (another block or vector
 * count), HL_ERR_HIP (see hl_last_error). */
hl_status hl_stream_ceiling(const void* read0, const void* read1, void* write, int64_t bytes, int block,
                            int vec_per_thread, int reps, hipStream_t stream, float* ms_per_launch);

/* Text of the last HIP failure seen by this thread (which call, the HIP
 * error string and code), or of the last workspace-size refusal of
 * hl_forward_backward_noalloc, or "" if none. Valid until the next failing
 * call. */
const char* hl_last_error(void);

/* Static text for a status code. */
const char* hl_status_str(hl_status status);

#ifdef __cplusplus
}
#endif

#endif /* HEADLOSS_H */
