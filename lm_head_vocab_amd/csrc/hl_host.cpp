// Host side of the C ABI declared in include/headloss.h: plan validation,
// kernel-variant choice, workspace layout and the per-call launch sequence.
#include "headloss.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>

#include "hl_internal.h"

using namespace hl;

struct hl_plan_s {
    int64_t V;
    hl_dtype dtype;
    uint32_t flags;
    hl_weights w;
    float temperature;
    float eps;
    float logit_scale;
    float softcap;
    int tmode;
    int forced_chunks;
    int forced_block;
    Geometry geo;
    FusedLauncher fused;
    FusedLauncher rowwise;   // inputs whose base addresses differ modulo 16 bytes
    FusedLauncher stream;    // forward only: row statistics streamed, one workgroup per row
    bool long_rows;          // V past every slice the chunk exchange serves: statistics streamed first,
                             // then the gradient from the records (fused kernel, load mode, many chunks)
    void* ws;
    size_t ws_bytes;
    bool ws_owned;
    bool ws_stale;      // the variant changed after a caller workspace was set
    bool ws_reset;      // the next call is the plan's first on ws: its control words are undefined
    const void* last_ws;// workspace of the last call (the plan's, or the static one)
    int64_t last_rows;
    hipEvent_t ev_before;
    hipEvent_t ev_after;
    uint32_t spin_limit;    // bound of the split-vocab wait (polls)
    int64_t withhold_row;   // test hook: this row's chunk withhold_chunk does not publish (-1: none)
    int withhold_chunk;
};

namespace {

thread_local char g_last_error[256] = "";

hl_status hip_fail(const char* where, hipError_t e) {
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
    return HL_ERR_HIP;
}

constexpr uint32_t kDistillBits = HL_FKL | HL_RKL | HL_FDCE;
constexpr uint32_t kPolicyBits = HL_GRPO | HL_GSPO;
constexpr uint32_t kLossBits = HL_CE | HL_ZLOSS | kDistillBits | kPolicyBits | HL_ENTROPY;
constexpr uint32_t kKnownBits = kLossBits | HL_ACCUMULATE | HL_HINTON;
constexpr int kTwoPerCuNvec = 10;         // 64 VGPRs at 1024 threads: two workgroups per CU
constexpr int kTwoPerCuNvecSoftcap = 8;   // the softcap instances need a few more registers

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
    size_t ctrl, chunk_rec, row_rec, rows, partials, row_coef, seg_of_row, seg_rec, total;
};

// Chunks of a row that exchange their records on the device (1 when the
// statistics are streamed first and the fused kernel only runs in load mode).
int exchange_chunks(const hl_plan_s* p) { return p->long_rows ? 1 : p->geo.chunks; }

// Workspace regions, in order: control words, split-vocab exchange words,
// per-row softmax records, per-row values, reduction partials, and for GSPO
// the per-row coefficient, the row -> segment map and the segment records
// (sized for the most segments a call may pass, n_rows).
Layout layout_for(const hl_plan_s* p, int64_t n) {
    Layout L;
    const size_t N = n > 0 ? (size_t)n : 0;
    L.ctrl = 0;
    L.chunk_rec = align256(NCTRL * sizeof(uint32_t));
    const size_t rec_bytes =
        exchange_chunks(p) > 1 ? N * p->geo.chunks * xwords_stride(p->dtype == HL_F32) * sizeof(uint64_t) : 0;
    L.row_rec = L.chunk_rec + align256(rec_bytes);
    L.rows = L.row_rec + align256(N * REC * sizeof(float));
    L.partials = L.rows + align256(N * NCOL * sizeof(float));
    const size_t groups = N > 0 ? (N + kReduceBlock - 1) / kReduceBlock : 1;
    L.row_coef = L.partials + align256(groups * NSUM * sizeof(double));
    const bool gspo = (p->flags & HL_GSPO) != 0u;
    L.seg_of_row = L.row_coef + (gspo ? align256(N * sizeof(float)) : 0);
    L.seg_rec = L.seg_of_row + (gspo ? align256(N * sizeof(int32_t)) : 0);
    L.total = L.seg_rec + (gspo ? align256(N * SEGREC * sizeof(double)) : 0);
    return L;
}

// The smallest entry of set that is >= need and <= cap (-1: none).
int round_up_to(const int* set, int n_set, int need, int cap = 1 << 30) {
    for (int i = 0; i < n_set; ++i)
        if (set[i] >= need && set[i] <= cap) return set[i];
    return -1;
}

// Largest slice (16-byte vectors per thread per tensor) an instance of this
// element type and mode holds.
int nvec_cap(hl_dtype dt, int tmode) {
    if (dt != HL_F32 || tmode == TM_NONE) return 1 << 30;
    return is_hinton(tmode) ? kF32HintonNvec : kF32TeacherNvec;
}

typedef FusedLauncher (*Getter)(int, int, bool);

// [dtype][teacher mode] instance getters (one translation unit each)
const Getter kGetters[3][7] = {
    {get_fused_f32_none, get_fused_f32_fkl, get_fused_f32_rkl, get_fused_f32_fdce,
     get_fused_f32_fklh, get_fused_f32_rklh, get_fused_f32_fdceh},
    {get_fused_bf16_none, get_fused_bf16_fkl, get_fused_bf16_rkl, get_fused_bf16_fdce,
     get_fused_bf16_fklh, get_fused_bf16_rklh, get_fused_bf16_fdceh},
    {get_fused_f16_none, get_fused_f16_fkl, get_fused_f16_rkl, get_fused_f16_fdce,
     get_fused_f16_fklh, get_fused_f16_rklh, get_fused_f16_fdceh},
};

FusedLauncher lookup_rowwise(hl_dtype dt, int tmode, bool softcap) {
    return dt == HL_F32 ? get_rowwise_f32(tmode, softcap)
         : dt == HL_BF16 ? get_rowwise_bf16(tmode, softcap) : get_rowwise_f16(tmode, softcap);
}

FusedLauncher lookup_stream(hl_dtype dt, int tmode, bool softcap) {
    return dt == HL_F32 ? get_stream_f32(tmode, softcap)
         : dt == HL_BF16 ? get_stream_bf16(tmode, softcap) : get_stream_f16(tmode, softcap);
}

FusedLauncher lookup(hl_dtype dt, int tmode, int block, int nvec, bool softcap) {
    return kGetters[(int)dt][tmode](block, nvec, softcap);
}

// Geometry for C chunks per row with a given block size (0: the smallest
// block that fits), or chunks = 0 when none fits. The register budget per
// thread is 20 vectors (80 VGPRs) for the student alone and 10 + 10 with a
// teacher, so that a 1024-thread workgroup stays within 128 VGPRs.
Geometry geometry_for(int64_t V, hl_dtype dt, int tmode, int C, int block = 0) {
    const int vec = dt == HL_F32 ? 4 : 8;
    const int cap = nvec_cap(dt, tmode);
    int64_t nvec_row = V / vec;
    if (nvec_row < 1) nvec_row = 1;
    const int64_t per = (nvec_row + C - 1) / C;
    Geometry g{0, 0, 0};
    if ((block == 0 || block == kSmallBlock) && per <= (int64_t)kSmallBlock * 4) {
        const int need = (int)((per + kSmallBlock - 1) / kSmallBlock);
        return Geometry{C, kSmallBlock, round_up_to(kSmallNvec, 3, need)};
    }
    if (block == kMidBlock) {
        const int* set = tmode == TM_NONE ? kMidNvecStudent : kMidNvecTeacher;
        const int n_set = tmode == TM_NONE ? 4 : (is_hinton(tmode) && dt != HL_F32 ? 6 : 4);
        const int64_t need = (per + kMidBlock - 1) / kMidBlock;
        if (need > (1 << 20)) return g;
        const int nv = round_up_to(set, n_set, (int)need, cap);
        return nv < 0 ? g : Geometry{C, kMidBlock, nv};
    }
    if (block != 0 && block != kLargeBlock) return g;
    const int* set = tmode == TM_NONE ? kLargeNvecStudent : kLargeNvecTeacher;
    const int n_set = tmode == TM_NONE ? 10 : 5;
    const int64_t need = (per + kLargeBlock - 1) / kLargeBlock;
    if (need > (1 << 20)) return g;
    const int nv = round_up_to(set, n_set, (int)need, cap);
    return nv < 0 ? g : Geometry{C, kLargeBlock, nv};
}

// Automatic choice: the fewest chunks per row whose slice fits the register
// budget while two workgroups still share a CU (one loads while the other
// computes): a student-only slice at 1024 threads holds at most 10 vectors
// per thread (8 with softcap, 64 VGPRs); a slice with a teacher uses 512
// threads and at most 10 + 10 vectors (about 113 VGPRs). Short rows use one
// 256-thread workgroup.
hl_status choose(hl_plan_s* p) {
    const int max_chunks = max_chunks_for(p->tmode, p->dtype == HL_F32);
    if (p->forced_chunks > max_chunks) return HL_ERR_UNSUPPORTED;
    if (p->forced_chunks > 0) {
        Geometry g = geometry_for(p->V, p->dtype, p->tmode, p->forced_chunks, p->forced_block);
        if (g.chunks == 0) return HL_ERR_UNSUPPORTED;
        p->geo = g;
    } else {
        Geometry g{0, 0, 0};
        for (int C = 1; C <= max_chunks; ++C) {
            g = geometry_for(p->V, p->dtype, p->tmode, C);
            if (g.chunks == 0) continue;
            if (g.block == kSmallBlock) break;
            if (p->tmode == TM_NONE) {
                if (g.nvec <= (p->softcap > 0.f ? kTwoPerCuNvecSoftcap : kTwoPerCuNvec)) break;
            } else {
                const Geometry mid = geometry_for(p->V, p->dtype, p->tmode, C, kMidBlock);
                if (mid.chunks != 0) {
                    g = mid;
                    break;
                }
            }
            g = Geometry{0, 0, 0};
        }
        if (g.chunks == 0) {   // very long rows: the fewest chunks that fit at all
            for (int C = 1; C <= max_chunks && g.chunks == 0; ++C) g = geometry_for(p->V, p->dtype, p->tmode, C);
        }
        p->long_rows = g.chunks == 0;
        if (p->long_rows) {
            // Rows longer than every slice the chunk exchange serves: the
            // statistics are streamed first (stream_stats_kernel), and the
            // gradient comes from the fused kernel in load mode, which needs
            // no exchange, with as many 1024-thread chunks as the row needs.
            const int vec = p->dtype == HL_F32 ? 4 : 8;
            int nmax = p->tmode == TM_NONE ? kLargeNvecStudent[9] : kLargeNvecTeacher[4];
            if (nmax > nvec_cap(p->dtype, p->tmode)) nmax = nvec_cap(p->dtype, p->tmode);
            const int64_t per_chunk = (int64_t)kLargeBlock * nmax;
            const int64_t nvec_row = p->V / vec;
            const int64_t C = (nvec_row + per_chunk - 1) / per_chunk;
            g = geometry_for(p->V, p->dtype, p->tmode, (int)C, kLargeBlock);
            if (g.chunks == 0) return HL_ERR_UNSUPPORTED;
        }
        p->geo = g;
    }
    if (p->forced_chunks > 0) p->long_rows = false;
    p->fused = lookup(p->dtype, p->tmode, p->geo.block, p->geo.nvec, p->softcap > 0.f);
    p->rowwise = lookup_rowwise(p->dtype, p->tmode, p->softcap > 0.f);
    p->stream = lookup_stream(p->dtype, p->tmode, p->softcap > 0.f);
    return (p->fused && p->rowwise && p->stream) ? HL_OK : HL_ERR_UNSUPPORTED;
}

bool finite(float x) { return std::isfinite(x); }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t elem_size(hl_dtype dt) { return dt == HL_F32 ? 4 : 2; }
bool elem_aligned(const void* p, size_t es) { return (reinterpret_cast<uintptr_t>(p) % es) == 0; }
uintptr_t mod16(const void* p) { return reinterpret_cast<uintptr_t>(p) & 15u; }

// The workspace layout depends on the variant: a library-owned buffer is
// released (the next call allocates a zeroed one); a caller's buffer must be
// handed over again with hl_plan_set_workspace.
void invalidate_workspace(hl_plan_s* p) {
    if (p->ws == nullptr) return;
    if (p->ws_owned) {
        (void)hipFree(p->ws);
        p->ws = nullptr;
        p->ws_bytes = 0;
        p->ws_owned = false;
    } else {
        p->ws_stale = true;
    }
}

}  // namespace

namespace hl {

void set_last_error(const char* msg) { std::snprintf(g_last_error, sizeof(g_last_error), "%s", msg); }

size_t call_workspace_bytes(hl_plan_t plan, int64_t n_rows) { return layout_for(plan, n_rows).total; }

hl_status check_call(hl_plan_t plan, const CallArgs& a) {
    if (plan == nullptr || a.n_rows < 0 || a.scalars == nullptr) return HL_ERR_INVALID_ARG;
    const int64_t n_rows = a.n_rows;
    if (n_rows > 0 && a.logits == nullptr) return HL_ERR_INVALID_ARG;
    const uint32_t f = plan->flags;
    if (f & HL_GSPO) {
        if (n_rows > 0 && a.seq_offsets == nullptr) return HL_ERR_MISSING_INPUT;
        if (a.n_segments < 0 || a.n_segments > n_rows || (n_rows > 0 && a.n_segments < 1)) return HL_ERR_INVALID_ARG;
    }
    if (n_rows > 0) {
        if ((f & (HL_CE | kPolicyBits)) && a.labels == nullptr) return HL_ERR_MISSING_INPUT;
        if ((f & kDistillBits) && a.teacher == nullptr) return HL_ERR_MISSING_INPUT;
        if ((f & kPolicyBits) && (a.old_logprobs == nullptr || a.advantages == nullptr)) return HL_ERR_MISSING_INPUT;
        const size_t es = elem_size(plan->dtype);
        if (!elem_aligned(a.logits, es)) return HL_ERR_INVALID_ARG;
        if (plan->tmode != TM_NONE && !elem_aligned(a.teacher, es)) return HL_ERR_INVALID_ARG;
        if (a.grad != nullptr && !elem_aligned(a.grad, es)) return HL_ERR_INVALID_ARG;
        if ((uint64_t)(n_rows + 7) * (uint64_t)plan->geo.chunks > 0x7fffffffull) return HL_ERR_UNSUPPORTED;
    }
    return HL_OK;
}

// Enqueue the kernels of a checked call on the workspace `wsv` (at least
// call_workspace_bytes(plan, n_rows), 256-byte aligned).
hl_status enqueue_call(hl_plan_t plan, const CallArgs& a, void* wsv, bool reset, hipStream_t stream) {
    const int64_t n_rows = a.n_rows;
    const void* logits = a.logits;
    const int64_t* labels = a.labels;
    const uint8_t* mask = a.mask;
    const void* teacher_logits = a.teacher;
    const float* old_logprobs = a.old_logprobs;
    const float* advantages = a.advantages;
    const int32_t* seq_offsets = a.seq_offsets;
    const int64_t n_segments = a.n_segments;
    void* grad_out = a.grad;
    float* scalars_out = a.scalars;
    const uint32_t f = plan->flags;
    const bool gspo = (f & HL_GSPO) != 0u;
    const Layout L = layout_for(plan, n_rows);
    plan->last_ws = wsv;
    plan->last_rows = n_rows;
    char* ws = static_cast<char*>(wsv);
    uint32_t* ctrl = reinterpret_cast<uint32_t*>(ws + L.ctrl);
    uint64_t* chunk_words = reinterpret_cast<uint64_t*>(ws + L.chunk_rec);
    float* row_rec = reinterpret_cast<float*>(ws + L.row_rec);
    float* rows = reinterpret_cast<float*>(ws + L.rows);
    const int C = plan->geo.chunks;
    const int CX = exchange_chunks(plan);   // chunks whose records travel through the exchange words

    CountParams cp;
    cp.labels = labels;
    cp.mask = mask;
    cp.ctrl = ctrl;
    cp.n_rows = n_rows;
    cp.V = plan->V;
    // The count kernel bumps the workspace's epoch and zero-fills this call's
    // split-vocab words where the workspace may hold anything but such words
    // (its control words decide; `reset` when they are undefined).
    cp.reset = reset ? 1 : 0;
    cp.spin_limit = plan->spin_limit;
    cp.hold_row = plan->withhold_row < 0 ? 0xffffffffu : (uint32_t)plan->withhold_row;
    cp.hold_chunk = plan->withhold_row < 0 ? 0xffffffffu : (uint32_t)plan->withhold_chunk;
    cp.vec = (labels != nullptr && aligned16(labels) && (mask == nullptr || aligned16(mask))) ? 1 : 0;
    cp.fill = chunk_words;
    cp.fill_words = CX > 1 ? n_rows * CX * xwords_stride(plan->dtype == HL_F32) : 0;
    hipError_t e = launch_count(cp, stream);
    if (e != hipSuccess) return hip_fail("count kernel launch", e);

    if (n_rows > 0) {
        FusedParams fp;
        fp.logits = logits;
        fp.teacher = plan->tmode != TM_NONE ? teacher_logits : nullptr;
        fp.labels = labels;
        fp.mask = mask;
        fp.old_logprobs = (f & HL_GRPO) ? old_logprobs : nullptr;
        fp.advantages = (f & HL_GRPO) ? advantages : nullptr;
        // GSPO: the fused kernel only computes the row statistics; the
        // gradient waits for the segment step
        fp.grad = gspo ? nullptr : grad_out;
        fp.row_rec = row_rec;
        fp.row_coef = nullptr;
        fp.load_mode = 0;
        fp.chunk_words = chunk_words;
        fp.ctrl = ctrl;
        fp.n_rows = n_rows;
        fp.V = plan->V;
        fp.chunks = C;
        fp.rows_per_xcd = (int)((n_rows + 7) / 8);
        fp.accumulate = (f & HL_ACCUMULATE) ? 1 : 0;
        fp.flags = f;
        constexpr double kLog2eD = 1.4426950408889634074;
        fp.k = plan->logit_scale;
        fp.K1d = (double)plan->logit_scale * kLog2eD;
        fp.K2d = kLog2eD / (double)plan->temperature;
        fp.betad = (f & HL_HINTON) ? 1.0 / (double)plan->temperature : 1.0;
        fp.K1 = (float)fp.K1d;
        fp.K2 = (float)fp.K2d;
        fp.beta = (float)fp.betad;
        fp.tau = plan->temperature;
        fp.cap = plan->softcap;
        fp.kc = plan->softcap > 0.f ? plan->logit_scale / plan->softcap : 0.f;
        fp.kc2 = plan->softcap > 0.f ? (float)(2.0 * (double)plan->logit_scale * 1.4426950408889634 /
                                               (double)plan->softcap)
                                     : 0.f;
        fp.cl = (float)((double)plan->softcap * 1.4426950408889634);
        fp.w_ce = plan->w.ce;
        fp.w_z = plan->w.z;
        fp.w_d = plan->w.distill;
        fp.w_g = plan->w.grpo;
        fp.grad_scale = plan->w.grad_scale;
        fp.divisor = plan->w.divisor;
        fp.eps = plan->eps;
        // The fused kernel splits every row at the same 16-byte boundaries in
        // logits, teacher and gradient, which exist only when the three base
        // addresses agree modulo 16; otherwise the row-wise kernel runs (one
        // workgroup per row, element loads and stores).
        const uintptr_t xa = mod16(logits);
        const bool teacher_ok = plan->tmode == TM_NONE || mod16(teacher_logits) == xa;
        const bool rowwise = !teacher_ok || (grad_out != nullptr && mod16(grad_out) != xa);
        // the streaming forward reads logits and teacher only, at any row length
        const bool stream_ok = teacher_ok;
        // rows past every exchanged slice: statistics streamed, then the
        // gradient from the records (the fused kernel in load mode)
        const bool two_pass = plan->long_rows && !rowwise;
        const FusedLauncher launch = rowwise ? plan->rowwise : plan->fused;
        // split-vocab: 8 XCD groups of rows_per_xcd rows, C workgroups per row
        const dim3 grid(rowwise ? (unsigned)n_rows
                        : C > 1 ? (unsigned)(8 * fp.rows_per_xcd * C) : (unsigned)n_rows);
        // A launch without a gradient (no grad_out, or GSPO's forward) keeps
        // nothing of the row after its sums: the streaming kernel reads each
        // row once with one workgroup and no chunk exchange.
        const bool fwd_only = fp.grad == nullptr;
        const bool stream_first = stream_ok && (fwd_only || two_pass);
        const FusedLauncher first = stream_first ? plan->stream : launch;
        const dim3 first_grid = stream_first ? dim3((unsigned)n_rows) : grid;
        if (plan->ev_before && (e = hipEventRecord(plan->ev_before, stream)) != hipSuccess)
            return hip_fail("hipEventRecord(before)", e);
        e = first(fp, first_grid, stream);
        if (e != hipSuccess) return hip_fail("fused kernel launch", e);
        if (gspo) {
            SeamParams sp;
            sp.row_rec = row_rec;
            sp.old_logprobs = old_logprobs;
            sp.advantages = advantages;
            sp.offsets = seq_offsets;
            sp.seg_rec = reinterpret_cast<double*>(ws + L.seg_rec);
            sp.row_coef = reinterpret_cast<float*>(ws + L.row_coef);
            sp.seg_of_row = reinterpret_cast<int32_t*>(ws + L.seg_of_row);
            sp.ctrl = ctrl;
            sp.n_rows = n_rows;
            sp.n_segments = n_segments;
            sp.k = plan->logit_scale;
            sp.cap = plan->softcap;
            sp.eps = plan->eps;
            e = launch_seam(sp, stream);
            if (e != hipSuccess) return hip_fail("segment kernel launch", e);
            if (grad_out != nullptr) {
                // the backward: the fused kernel again, in load mode, with the
                // per-row GSPO coefficient on the label column
                fp.grad = grad_out;
                fp.row_coef = sp.row_coef;
                fp.load_mode = 1;
                e = launch(fp, grid, stream);
                if (e != hipSuccess) return hip_fail("fused kernel launch (load mode)", e);
            }
        } else if (two_pass && grad_out != nullptr) {
            fp.load_mode = 1;
            e = launch(fp, grid, stream);
            if (e != hipSuccess) return hip_fail("fused kernel launch (load mode)", e);
        }
        if (plan->ev_after && (e = hipEventRecord(plan->ev_after, stream)) != hipSuccess)
            return hip_fail("hipEventRecord(after)", e);
    }

    ReduceParams rp;
    rp.row_rec = row_rec;
    rp.partials = reinterpret_cast<double*>(ws + L.partials);
    rp.labels = labels;
    rp.old_logprobs = (f & HL_GRPO) ? old_logprobs : nullptr;
    rp.advantages = (f & HL_GRPO) ? advantages : nullptr;
    rp.seg_rec = gspo ? reinterpret_cast<const double*>(ws + L.seg_rec) : nullptr;
    rp.seg_of_row = gspo ? reinterpret_cast<const int32_t*>(ws + L.seg_of_row) : nullptr;
    rp.n_segments = gspo ? n_segments : 0;
    rp.rows = rows;
    rp.ctrl = ctrl;
    rp.k = plan->logit_scale;
    rp.cap = plan->softcap;
    rp.eps = plan->eps;
    rp.tau = plan->temperature;
    rp.scalars = scalars_out;
    rp.n_rows = n_rows;
    rp.flags = f;
    rp.w_ce = plan->w.ce;
    rp.w_z = plan->w.z;
    rp.w_d = plan->w.distill;
    rp.w_g = plan->w.grpo;
    rp.divisor = plan->w.divisor;
    e = launch_reduce(rp, stream);
    if (e != hipSuccess) return hip_fail("reduce kernel launch", e);
    return HL_OK;
}

}  // namespace hl

extern "C" {

hl_status hl_plan(hl_plan_t* out, int64_t V, hl_dtype dtype, uint32_t loss_flags,
                  const hl_weights* weights, float temperature, float eps,
                  float logit_scale, float softcap) {
    if (out == nullptr) return HL_ERR_INVALID_ARG;
    *out = nullptr;
    if (V < 1 || weights == nullptr) return HL_ERR_INVALID_ARG;
    if (V > kMaxRowElements) return HL_ERR_UNSUPPORTED;
    if (dtype != HL_F32 && dtype != HL_BF16 && dtype != HL_F16) return HL_ERR_INVALID_ARG;
    if ((loss_flags & ~kKnownBits) != 0u || (loss_flags & kLossBits) == 0u) return HL_ERR_INVALID_ARG;
    const uint32_t dbits = loss_flags & kDistillBits;
    if (dbits & (dbits - 1u)) return HL_ERR_INVALID_ARG;   // at most one distillation loss
    const bool distill = dbits != 0u;
    if ((loss_flags & HL_HINTON) && !distill) return HL_ERR_INVALID_ARG;   // the mode tempers distillation
    if (distill && !(finite(temperature) && temperature > 0.f)) return HL_ERR_INVALID_ARG;
    if ((loss_flags & kPolicyBits) == kPolicyBits) return HL_ERR_INVALID_ARG;   // one policy loss
    if ((loss_flags & kPolicyBits) && !(finite(eps) && eps > 0.f && eps < 1.f)) return HL_ERR_INVALID_ARG;
    if (!(finite(logit_scale) && logit_scale > 0.f)) return HL_ERR_INVALID_ARG;
    if (!(finite(softcap) && softcap >= 0.f)) return HL_ERR_INVALID_ARG;
    const hl_weights& w = *weights;
    if (!(finite(w.ce) && finite(w.z) && finite(w.distill) && finite(w.grpo) &&
          finite(w.grad_scale) && finite(w.divisor)))
        return HL_ERR_INVALID_ARG;

    hl_plan_s* p = new (std::nothrow) hl_plan_s;
    if (p == nullptr) return HL_ERR_INVALID_ARG;
    std::memset(p, 0, sizeof(*p));
    p->V = V;
    p->dtype = dtype;
    p->flags = loss_flags;
    p->w = w;
    p->temperature = distill ? temperature : 1.f;
    p->eps = eps;
    p->logit_scale = logit_scale;
    p->softcap = softcap;
    p->spin_limit = kSpinLimit;
    p->withhold_row = -1;
    p->withhold_chunk = -1;
    p->tmode = (loss_flags & HL_FKL) ? TM_FKL
             : (loss_flags & HL_RKL) ? TM_RKL
             : (loss_flags & HL_FDCE) ? TM_FDCE : TM_NONE;
    if (loss_flags & HL_HINTON) p->tmode += TM_FKL_H - TM_FKL;
    const hl_status st = choose(p);
    if (st != HL_OK) {
        delete p;
        return st;
    }
    *out = p;
    return HL_OK;
}

void hl_plan_destroy(hl_plan_t plan) {
    if (plan == nullptr) return;
    if (plan->ws_owned && plan->ws) (void)hipFree(plan->ws);
    delete plan;
}

size_t hl_workspace_bytes(hl_plan_t plan, int64_t n_rows) {
    if (plan == nullptr || n_rows < 0) return 0;
    return layout_for(plan, n_rows).total;
}

hl_status hl_plan_set_workspace(hl_plan_t plan, void* dev_workspace, size_t bytes) {
    if (plan == nullptr || dev_workspace == nullptr) return HL_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(dev_workspace) & 255u) != 0) return HL_ERR_INVALID_ARG;
    if (plan->ws_owned && plan->ws) (void)hipFree(plan->ws);
    plan->ws = dev_workspace;
    plan->ws_bytes = bytes;
    plan->ws_owned = false;
    plan->ws_stale = false;
    plan->ws_reset = true;
    return HL_OK;
}

hl_status hl_plan_set_chunks(hl_plan_t plan, int chunks) {
    if (plan == nullptr || chunks < 0 || chunks > kMaxChunks) return HL_ERR_INVALID_ARG;
    const int prev = plan->forced_chunks, prev_b = plan->forced_block;
    const Geometry prev_geo = plan->geo;
    const FusedLauncher prev_fn = plan->fused;
    plan->forced_chunks = chunks;
    plan->forced_block = 0;
    const hl_status st = choose(plan);
    if (st != HL_OK) {
        plan->forced_chunks = prev;
        plan->forced_block = prev_b;
        plan->geo = prev_geo;
        plan->fused = prev_fn;
    } else {
        invalidate_workspace(plan);
    }
    return st;
}

hl_status hl_plan_set_variant(hl_plan_t plan, int chunks, int block) {
    if (plan == nullptr || chunks < 0 || chunks > kMaxChunks) return HL_ERR_INVALID_ARG;
    if (block != 0 && block != kSmallBlock && block != kMidBlock && block != kLargeBlock) return HL_ERR_INVALID_ARG;
    if (block != 0 && chunks == 0) return HL_ERR_INVALID_ARG;
    const int prev_c = plan->forced_chunks, prev_b = plan->forced_block;
    const Geometry prev_geo = plan->geo;
    const FusedLauncher prev_fn = plan->fused;
    plan->forced_chunks = chunks;
    plan->forced_block = block;
    const hl_status st = choose(plan);
    if (st != HL_OK) {
        plan->forced_chunks = prev_c;
        plan->forced_block = prev_b;
        plan->geo = prev_geo;
        plan->fused = prev_fn;
    } else {
        invalidate_workspace(plan);
    }
    return st;
}

hl_status hl_plan_describe(hl_plan_t plan, int* chunks, int* block, int* vec_per_thread) {
    if (plan == nullptr) return HL_ERR_INVALID_ARG;
    if (chunks) *chunks = plan->geo.chunks;
    if (block) *block = plan->geo.block;
    if (vec_per_thread) *vec_per_thread = plan->geo.nvec;
    return HL_OK;
}

hl_status hl_plan_set_timing_events(hl_plan_t plan, hipEvent_t before, hipEvent_t after) {
    if (plan == nullptr) return HL_ERR_INVALID_ARG;
    plan->ev_before = before;
    plan->ev_after = after;
    return HL_OK;
}

hl_status hl_plan_set_exchange_test(hl_plan_t plan, uint32_t spin_limit, int64_t withhold_row,
                                    int withhold_chunk) {
    if (plan == nullptr || spin_limit < 1 || withhold_row >= 0xffffffffLL) return HL_ERR_INVALID_ARG;
    plan->spin_limit = spin_limit;
    plan->withhold_row = withhold_row < 0 ? -1 : withhold_row;
    plan->withhold_chunk = withhold_row < 0 ? -1 : withhold_chunk;
    return HL_OK;
}

const float* hl_row_values(hl_plan_t plan) {
    if (plan == nullptr || plan->last_ws == nullptr) return nullptr;
    const Layout L = layout_for(plan, plan->last_rows);
    return reinterpret_cast<const float*>(static_cast<const char*>(plan->last_ws) + L.rows);
}

hl_status hl_forward_backward(hl_plan_t plan, int64_t n_rows, const void* logits,
                              const int64_t* labels, const uint8_t* mask,
                              const void* teacher_logits, const float* old_logprobs,
                              const float* advantages, void* grad_out,
                              float* scalars_out, hipStream_t stream) {
    return hl_forward_backward_segments(plan, n_rows, logits, labels, mask, teacher_logits, old_logprobs,
                                        advantages, nullptr, 0, grad_out, scalars_out, stream);
}

hl_status hl_forward_backward_segments(hl_plan_t plan, int64_t n_rows, const void* logits,
                                       const int64_t* labels, const uint8_t* mask,
                                       const void* teacher_logits, const float* old_logprobs,
                                       const float* advantages, const int32_t* seq_offsets,
                                       int64_t n_segments, void* grad_out,
                                       float* scalars_out, hipStream_t stream) {
    const CallArgs a{n_rows, logits, labels, mask, teacher_logits, old_logprobs, advantages,
                     seq_offsets, n_segments, grad_out, scalars_out};
    hl_status st = check_call(plan, a);
    if (st != HL_OK) return st;
    const size_t need = call_workspace_bytes(plan, n_rows);
    if (plan->ws_stale) return HL_ERR_WORKSPACE;
    if (plan->ws == nullptr || plan->ws_bytes < need) {
        if (plan->ws != nullptr && !plan->ws_owned) return HL_ERR_WORKSPACE;
        if (plan->ws_owned && plan->ws) {
            (void)hipFree(plan->ws);
            plan->ws = nullptr;
            plan->ws_bytes = 0;
        }
        void* mem = nullptr;
        hipError_t me = hipMalloc(&mem, need);
        if (me != hipSuccess) return hip_fail("hipMalloc(workspace)", me);
        plan->ws = mem;
        plan->ws_bytes = need;
        plan->ws_owned = true;
        plan->ws_reset = true;
    }
    st = enqueue_call(plan, a, plan->ws, plan->ws_reset, stream);
    if (st == HL_OK) plan->ws_reset = false;
    return st;
}

const char* hl_last_error(void) { return g_last_error; }

const char* hl_status_str(hl_status status) {
    switch (status) {
        case HL_OK: return "ok";
        case HL_ERR_INVALID_ARG: return "invalid argument";
        case HL_ERR_MISSING_INPUT: return "an enabled loss is missing one of its inputs";
        case HL_ERR_UNSUPPORTED: return "unsupported request";
        case HL_ERR_WORKSPACE: return "workspace missing or too small";
        case HL_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

}  // extern "C"
