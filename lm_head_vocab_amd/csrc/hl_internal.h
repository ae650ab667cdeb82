// Internal types shared by the host library and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hl {

// Distillation mode baked into a kernel instance. The _H modes temper the
// distillation student as well (softmax(s / tau), loss times tau^2).
enum TeacherMode : int {
    TM_NONE = 0, TM_FKL = 1, TM_RKL = 2, TM_FDCE = 3, TM_FKL_H = 4, TM_RKL_H = 5, TM_FDCE_H = 6
};

constexpr bool is_hinton(int t) { return t >= TM_FKL_H; }
constexpr int base_mode(int t) { return is_hinton(t) ? t - 3 : t; }
// Forward KL and from-distribution CE share the gradient q - p.
constexpr bool fkl_like(int t) { return base_mode(t) == TM_FKL || base_mode(t) == TM_FDCE; }
// Modes that carry the teacher entropy sum St.
constexpr bool has_st(int t) { return base_mode(t) == TM_FDCE; }
// Statistics a chunk publishes: M, Z, S (+ Mt, Zt, SX (+ St) (+ Zs)); the fp32
// instances (hp) also carry the low parts of the normalizers Z (+ Zt (+ Zs)).
constexpr int xwords_used(int t, bool hp = false) {
    return (t == TM_NONE ? 3 : 6 + (has_st(t) ? 1 : 0) + (is_hinton(t) ? 1 : 0)) +
           (hp ? (t == TM_NONE ? 1 : (is_hinton(t) ? 3 : 2)) : 0);
}

// Loss bits (same values as the public HL_* flags).
enum : uint32_t {
    F_CE = 1u << 0, F_Z = 1u << 1, F_FKL = 1u << 2, F_RKL = 1u << 3,
    F_GRPO = 1u << 4, F_ENT = 1u << 5, F_FDCE = 1u << 6, F_GSPO = 1u << 7, F_ACC = 1u << 16,
    F_HINTON = 1u << 17,
    F_DISTILL = F_FKL | F_RKL | F_FDCE,
};

// Per-row value columns (same order as the public HL_R_* enum).
enum RowCol : int {
    RC_CE = 0, RC_Z, RC_KL, RC_GRPO, RC_LOGP, RC_RATIO, RC_CLIP, RC_K3, RC_ADV,
    RC_ENT, RC_VALID, RC_PAD, NCOL
};
constexpr int NSUM = RC_VALID;        // columns the batch reduction sums
constexpr int NSCALARS = 13;

// Softmax statistics of a slice of one row, in the log2 domain:
//   M  = shift, Z = sum 2^(A_j - M), S = sum 2^(A_j - M) (A_j - M)
//   Mt, Zt = the same for the teacher, SX = the distillation cross sum.
//   St = sum 2^(U_j - Mt) (U_j - Mt), the teacher entropy sum (FDCE only).
//   Zs = sum 2^((A_j - M) b), b = 1 / tau: the tempered student's sum
//        (Hinton modes only; its shift is M b).
//   Zl, Ztl, Zsl: the fp32 instances keep the normalizers Z, Zt, Zs as
//        hi + lo pairs (sums and merges in fp64, carried as two floats);
//        0 in every other instance.
// The per-row record written by the fused kernel adds the raw label logit
// and a valid flag.
enum RecField : int { R_M = 0, R_Z, R_S, R_MT, R_ZT, R_SX, R_ST, R_XY, R_VALID, R_ZS, R_ZL, R_ZTL, R_ZSL, REC };

// Control words at the start of the workspace. CTRL_NSEG counts the GSPO
// segments that hold a valid row. CTRL_ERROR: 1 = a split-vocab row never saw
// all of its chunks, 2 = malformed segment offsets. CTRL_EPOCH tags the
// split-vocab words of the current call; CTRL_CLEAN_LO/HI (a 64-bit count)
// is how many leading split-vocab words are known to hold zeros or words of
// earlier epochs (both belong to the workspace, whichever plan calls).
// CTRL_SPIN, CTRL_HOLD_ROW, CTRL_HOLD_CHUNK: the bound of the split-vocab
// wait and the test hook of a withheld chunk, written by the count kernel
// and read by the exchange where it needs them (as kernel arguments they
// would stay live in scalar registers through the whole fused kernel).
enum Ctrl : int {
    CTRL_NVALID = 0, CTRL_NBAD = 1, CTRL_EPOCH = 2, CTRL_ERROR = 3, CTRL_DONE = 4, CTRL_NSEG = 5,
    CTRL_CLEAN_LO = 6, CTRL_CLEAN_HI = 7, CTRL_SPIN = 8, CTRL_HOLD_ROW = 9, CTRL_HOLD_CHUNK = 10,
    NCTRL = 64
};

// Per-segment GSPO record (fp64): loss, sequence ratio, clipped flag, k3 of
// the ratio, segment advantage, nonempty flag, the per-token coefficient
// act * A * s / n_i, and the valid-token count n_i.
enum SegField : int { SG_LOSS = 0, SG_RATIO, SG_CLIP, SG_K3, SG_ADV, SG_NONEMPTY, SG_DERIV, SG_COUNT, SEGREC };

// Split-vocab exchange: each chunk publishes its statistics as 64-bit words
// (float bits low, call epoch high), XWORDS apart (XWORDS_HP in the fp32
// instances, up to 11 words). One wave polls all of a row's words, so a mode
// allows at most 64 / xwords_used chunks.
constexpr int XWORDS = 8;
constexpr int XWORDS_HP = 16;
constexpr int xwords_stride(bool hp) { return hp ? XWORDS_HP : XWORDS; }
constexpr int kMaxChunks = 9;
constexpr int max_chunks_for(int t, bool hp = false) {
    return 64 / xwords_used(t, hp) < kMaxChunks ? 64 / xwords_used(t, hp) : kMaxChunks;
}
static_assert(kMaxChunks * xwords_used(TM_FDCE) <= 64, "one wave polls every exchanged word of a row");
static_assert(xwords_used(TM_FDCE_H, true) <= XWORDS_HP && xwords_used(TM_FDCE_H) <= XWORDS, "words per chunk");

struct Geometry {
    int chunks;      // workgroups per row
    int block;       // threads per workgroup
    int nvec;        // 16-byte vectors per thread per tensor
};

struct FusedParams {
    const void* logits;
    const void* teacher;
    const int64_t* labels;
    const uint8_t* mask;
    const float* old_logprobs;
    const float* advantages;
    void* grad;
    float* row_rec;           // [N, REC]
    uint64_t* chunk_words;    // [N, C, XWORDS] (XWORDS_HP in the fp32 instances)
    uint32_t* ctrl;           // [NCTRL]
    const float* row_coef;    // [N] GSPO label-column coefficient per row, or nullptr
    int load_mode;            // 1: statistics from row_rec (second launch of a GSPO call)
    int64_t n_rows;
    int64_t V;
    int chunks;
    int rows_per_xcd;     // split-vocab item mapping: rows handled per XCD group
    int accumulate;
    uint32_t flags;
    float k;          // logit scale
    float K1;         // k * log2(e)
    float K2;         // log2(e) / temperature
    float beta;       // 1 / temperature for the tempered distillation student (Hinton modes), else 1
    double K1d, K2d, betad;   // the same three in fp64 (used by the fp32 instances)
    float tau;        // temperature (the Hinton gradient carries tau)
    float cap;        // softcap c (0 = off)
    float kc;         // k / c
    float kc2;        // 2 k log2(e) / c: exp2 of kc2 x is exp(2 k x / c)
    float cl;         // c log2(e)
    float w_ce, w_z, w_d, w_g;
    float grad_scale;
    float divisor;
    float eps;
};

// Default bound of the split-vocab wait, in polls.
constexpr uint32_t kSpinLimit = 1u << 20;

struct CountParams {
    const int64_t* labels;
    const uint8_t* mask;
    uint32_t* ctrl;
    int64_t n_rows;
    int64_t V;
    // First call of a plan on a workspace: its control words may hold
    // anything, so the epoch restarts at 1 and the call's split-vocab words
    // are zero-filled whatever CTRL_CLEAN says.
    int reset;
    uint64_t* fill;        // the call's split-vocab words
    int64_t fill_words;    // their number (0 without a chunk exchange); even
    int vec;   // labels (and mask, if any) 16-byte aligned: the tiled load path
    // Bounded wait of the split-vocab exchange (polls), and a test hook: the
    // chunk hold_chunk of row hold_row does not publish its statistics
    // (hold_row 0xffffffff: none), so that every chunk of that row gives up.
    uint32_t spin_limit;
    uint32_t hold_row;
    uint32_t hold_chunk;
};

constexpr int kReduceBlock = 256;   // rows per reduction workgroup

struct ReduceParams {
    const float* row_rec;     // [N, REC] from the fused kernel
    double* partials;         // [G, NSUM] per-workgroup sums
    const int64_t* labels;
    const float* old_logprobs;
    const float* advantages;
    const double* seg_rec;    // [S, SEGREC] (GSPO only)
    const int32_t* seg_of_row;// [N] (GSPO only)
    int64_t n_segments;
    uint32_t* ctrl;
    float* rows;              // [N, NCOL] per-row values (written)
    float* scalars;
    int64_t n_rows;
    uint32_t flags;
    float k, cap, eps;
    float tau;                // Hinton modes: the distillation value is scaled by tau^2
    float w_ce, w_z, w_d, w_g;
    float divisor;
};

constexpr int kSeamBlock = 256;     // one wave per segment, 4 segments per workgroup

struct SeamParams {
    const float* row_rec;     // [N, REC] from the forward pass
    const float* old_logprobs;
    const float* advantages;
    const int32_t* offsets;   // [S + 1]
    double* seg_rec;          // [S, SEGREC] (written)
    float* row_coef;          // [N] (written)
    int32_t* seg_of_row;      // [N] (written)
    uint32_t* ctrl;
    int64_t n_rows;
    int64_t n_segments;
    float k, cap, eps;
};

typedef hipError_t (*FusedLauncher)(const FusedParams&, dim3 grid, hipStream_t);

// One getter per (dtype, teacher mode) translation unit; nullptr when the
// requested (block, nvec, softcap) instance does not exist.
FusedLauncher get_fused_f32_none(int block, int nvec, bool softcap);
FusedLauncher get_fused_f32_fkl(int block, int nvec, bool softcap);
FusedLauncher get_fused_f32_rkl(int block, int nvec, bool softcap);
FusedLauncher get_fused_bf16_none(int block, int nvec, bool softcap);
FusedLauncher get_fused_bf16_fkl(int block, int nvec, bool softcap);
FusedLauncher get_fused_bf16_rkl(int block, int nvec, bool softcap);
FusedLauncher get_fused_f16_none(int block, int nvec, bool softcap);
FusedLauncher get_fused_f16_fkl(int block, int nvec, bool softcap);
FusedLauncher get_fused_f16_rkl(int block, int nvec, bool softcap);
FusedLauncher get_fused_f32_fdce(int block, int nvec, bool softcap);
FusedLauncher get_fused_bf16_fdce(int block, int nvec, bool softcap);
FusedLauncher get_fused_f16_fdce(int block, int nvec, bool softcap);
FusedLauncher get_fused_f32_fklh(int block, int nvec, bool softcap);
FusedLauncher get_fused_f32_rklh(int block, int nvec, bool softcap);
FusedLauncher get_fused_f32_fdceh(int block, int nvec, bool softcap);
FusedLauncher get_fused_bf16_fklh(int block, int nvec, bool softcap);
FusedLauncher get_fused_bf16_rklh(int block, int nvec, bool softcap);
FusedLauncher get_fused_bf16_fdceh(int block, int nvec, bool softcap);
FusedLauncher get_fused_f16_fklh(int block, int nvec, bool softcap);
FusedLauncher get_fused_f16_rklh(int block, int nvec, bool softcap);
FusedLauncher get_fused_f16_fdceh(int block, int nvec, bool softcap);
// Row-wise kernel (inputs whose base addresses differ modulo 16 bytes), by
// teacher mode, one getter per element type.
FusedLauncher get_rowwise_f32(int tmode, bool softcap);
FusedLauncher get_rowwise_bf16(int tmode, bool softcap);
FusedLauncher get_rowwise_f16(int tmode, bool softcap);
// Forward-only streaming statistics kernel (no gradient; GSPO's forward).
FusedLauncher get_stream_f32(int tmode, bool softcap);
FusedLauncher get_stream_bf16(int tmode, bool softcap);
FusedLauncher get_stream_f16(int tmode, bool softcap);

hipError_t launch_count(const CountParams& p, hipStream_t s);
hipError_t launch_reduce(const ReduceParams& p, hipStream_t s);
hipError_t launch_seam(const SeamParams& p, hipStream_t s);

}  // namespace hl

#include "headloss.h"

namespace hl {

// Host side (hl_host.cpp): one call's arguments (those of
// hl_forward_backward_segments), its checks, its workspace size, and the
// enqueue of its kernels on a given workspace. `reset`: the workspace's
// control words are undefined (a plan's first call on it).
struct CallArgs {
    int64_t n_rows;
    const void* logits;
    const int64_t* labels;
    const uint8_t* mask;
    const void* teacher;
    const float* old_logprobs;
    const float* advantages;
    const int32_t* seq_offsets;
    int64_t n_segments;
    void* grad;
    float* scalars;
};
hl_status check_call(hl_plan_t plan, const CallArgs& a);
size_t call_workspace_bytes(hl_plan_t plan, int64_t n_rows);
hl_status enqueue_call(hl_plan_t plan, const CallArgs& a, void* ws, bool reset, hipStream_t stream);
void set_last_error(const char* msg);

// Threads per workgroup of the row-wise kernel (one workgroup per row).
constexpr int kRowwiseBlock = 256;
// Longest row any kernel takes: element indices within a row are 32-bit.
constexpr int64_t kMaxRowElements = 0x7fffffffLL;

// Vector counts that have a kernel instance, per block size.
constexpr int kSmallBlock = 256;
constexpr int kMidBlock = 512;
constexpr int kLargeBlock = 1024;
constexpr int kSmallNvec[] = {1, 2, 4};
constexpr int kMidNvecStudent[] = {10, 12, 16, 20};
// (12 and 13: 9 register vectors plus 3 or 4 held in LDS; 16-bit Hinton
// instances only, the one family where the larger slice measured faster)
constexpr int kMidNvecTeacher[] = {6, 8, 9, 10, 12, 13};
constexpr int kLargeNvecStudent[] = {2, 4, 6, 8, 10, 12, 14, 16, 18, 20};
constexpr int kLargeNvecTeacher[] = {2, 4, 6, 8, 10};
// fp32 slices with a teacher hold at most this many vectors per tensor (the
// fp64 element path of the fp32 instances needs the registers): 8, or 4 in
// the Hinton modes (three exponentials per element).
constexpr int kF32TeacherNvec = 8;
constexpr int kF32HintonNvec = 4;

}  // namespace hl
