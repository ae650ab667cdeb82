// Host-only driver of the C ABI for a sanitizer build (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host library, hl_host.cpp). The kernel
// launchers are replaced by stubs that record their parameters and return
// success, so every host path runs without a GPU and without device code:
// plan validation and variant choice, workspace layout, the per-call checks
// and the whole enqueue sequence on a stand-in workspace (never dereferenced
// by the host). Exit status 0 and no sanitizer report = pass.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "headloss.h"
#include "hl_internal.h"

namespace {
int g_fails = 0;
int g_fused_calls = 0, g_count_calls = 0, g_reduce_calls = 0, g_seam_calls = 0;
hl::FusedParams g_last_fused;
hl::CountParams g_last_count;

#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++g_fails;                                                           \
        }                                                                        \
    } while (0)

hipError_t stub_fused(const hl::FusedParams& p, dim3, hipStream_t) {
    ++g_fused_calls;
    g_last_fused = p;
    return hipSuccess;
}
}  // namespace

// stand-ins for the launchers of the device translation units
namespace hl {
#define STUB_GETTER(NAME) \
    FusedLauncher NAME(int, int, bool) { return &stub_fused; }
STUB_GETTER(get_fused_f32_none) STUB_GETTER(get_fused_f32_fkl) STUB_GETTER(get_fused_f32_rkl)
STUB_GETTER(get_fused_bf16_none) STUB_GETTER(get_fused_bf16_fkl) STUB_GETTER(get_fused_bf16_rkl)
STUB_GETTER(get_fused_f16_none) STUB_GETTER(get_fused_f16_fkl) STUB_GETTER(get_fused_f16_rkl)
STUB_GETTER(get_fused_f32_fdce) STUB_GETTER(get_fused_bf16_fdce) STUB_GETTER(get_fused_f16_fdce)
STUB_GETTER(get_fused_f32_fklh) STUB_GETTER(get_fused_f32_rklh) STUB_GETTER(get_fused_f32_fdceh)
STUB_GETTER(get_fused_bf16_fklh) STUB_GETTER(get_fused_bf16_rklh) STUB_GETTER(get_fused_bf16_fdceh)
STUB_GETTER(get_fused_f16_fklh) STUB_GETTER(get_fused_f16_rklh) STUB_GETTER(get_fused_f16_fdceh)
FusedLauncher get_rowwise_f32(int, bool) { return &stub_fused; }
FusedLauncher get_rowwise_bf16(int, bool) { return &stub_fused; }
FusedLauncher get_rowwise_f16(int, bool) { return &stub_fused; }
FusedLauncher get_stream_f32(int, bool) { return &stub_fused; }
FusedLauncher get_stream_bf16(int, bool) { return &stub_fused; }
FusedLauncher get_stream_f16(int, bool) { return &stub_fused; }
hipError_t launch_count(const CountParams& p, hipStream_t) {
    ++g_count_calls;
    g_last_count = p;
    return hipSuccess;
}
hipError_t launch_reduce(const ReduceParams&, hipStream_t) {
    ++g_reduce_calls;
    return hipSuccess;
}
hipError_t launch_seam(const SeamParams&, hipStream_t) {
    ++g_seam_calls;
    return hipSuccess;
}
}  // namespace hl

namespace {

hl_weights W(float ce, float z, float d, float g) { return hl_weights{ce, z, d, g, 1.0f, 0.0f}; }

void* fake(size_t addr) { return reinterpret_cast<void*>(addr); }

void plans_and_variants() {
    const hl_weights w = W(1, 0.1f, 0.5f, 1);
    const hl_dtype dts[] = {HL_F32, HL_BF16, HL_F16};
    const uint32_t sets[] = {HL_CE, HL_CE | HL_ZLOSS | HL_ENTROPY, HL_CE | HL_FKL, HL_CE | HL_RKL | HL_HINTON,
                             HL_CE | HL_FDCE, HL_GRPO | HL_ZLOSS, HL_GSPO | HL_RKL, HL_CE | HL_ACCUMULATE};
    const int64_t Vs[] = {1, 3, 1000, 4099, 60013, 151936, 256000, 737288, 1474569};
    for (hl_dtype dt : dts)
        for (uint32_t f : sets)
            for (int64_t V : Vs) {
                hl_plan_t p = nullptr;
                const hl_status st = hl_plan(&p, V, dt, f, &w, 1.5f, 0.2f, 0.8f, (V % 2) ? 10.0f : 0.0f);
                CHECK(st == HL_OK);
                if (st != HL_OK) continue;
                int c = 0, b = 0, n = 0;
                CHECK(hl_plan_describe(p, &c, &b, &n) == HL_OK);
                CHECK(c >= 1 && (b == 256 || b == 512 || b == 1024) && n >= 1);
                CHECK(hl_workspace_bytes(p, 1000) > 0);
                for (int chunks = 0; chunks <= 10; ++chunks) (void)hl_plan_set_chunks(p, chunks);
                for (int blk : {0, 256, 512, 1024, 300}) (void)hl_plan_set_variant(p, 3, blk);
                hl_plan_destroy(p);
            }
    // refusals
    hl_plan_t p = nullptr;
    CHECK(hl_plan(nullptr, 10, HL_BF16, HL_CE, &w, 1, 0.2f, 1, 0) == HL_ERR_INVALID_ARG);
    CHECK(hl_plan(&p, 0, HL_BF16, HL_CE, &w, 1, 0.2f, 1, 0) == HL_ERR_INVALID_ARG && p == nullptr);
    CHECK(hl_plan(&p, 10, HL_BF16, HL_FKL | HL_RKL, &w, 1, 0.2f, 1, 0) == HL_ERR_INVALID_ARG);
    CHECK(hl_plan(&p, 10, HL_BF16, HL_GRPO, &w, 1, 1.5f, 1, 0) == HL_ERR_INVALID_ARG);
    CHECK(hl_plan(&p, 10, HL_BF16, HL_CE, &w, 1, 0.2f, NAN, 0) == HL_ERR_INVALID_ARG);
    CHECK(hl_plan(&p, int64_t(1) << 31, HL_BF16, HL_CE, &w, 1, 0.2f, 1, 0) == HL_ERR_UNSUPPORTED);
    for (int s = 0; s <= 6; ++s) CHECK(std::strlen(hl_status_str((hl_status)s)) > 0);
}

// The enqueue sequence on a stand-in workspace: the stubs see the launches.
void enqueue_paths() {
    const hl_weights w = W(1, 0.01f, 0.5f, 1);
    hl_plan_t p = nullptr;
    CHECK(hl_plan(&p, 151936, HL_BF16, HL_CE | HL_ZLOSS | HL_FKL | HL_GRPO | HL_ENTROPY, &w, 2.0f, 0.2f, 1.0f,
                  0.0f) == HL_OK);
    int c = 0;
    hl_plan_describe(p, &c, nullptr, nullptr);
    const int64_t N = 4096;
    const size_t need = hl_workspace_bytes(p, N);
    CHECK(hl_plan_set_workspace(p, fake(1 << 20), need) == HL_OK);
    void* x = fake(0x100000000ull);
    void* t = fake(0x200000000ull);
    void* g = fake(0x300000000ull);
    const int64_t* y = static_cast<const int64_t*>(fake(0x400000000ull));
    const float* old = static_cast<const float*>(fake(0x500000000ull));
    const float* adv = static_cast<const float*>(fake(0x500100000ull));
    float* sc = static_cast<float*>(fake(0x600000000ull));
    const int before = g_fused_calls;
    CHECK(hl_forward_backward(p, N, x, y, nullptr, t, old, adv, g, sc, nullptr) == HL_OK);
    CHECK(g_fused_calls == before + 1 && g_count_calls >= 1 && g_reduce_calls >= 1);
    // the first call on a workspace resets its control words; later calls do not
    CHECK(g_last_count.reset == 1);
    CHECK(g_last_count.fill_words == N * c * hl::XWORDS || c == 1);
    CHECK(hl_forward_backward(p, N, x, y, nullptr, t, old, adv, g, sc, nullptr) == HL_OK);
    CHECK(g_last_count.reset == 0);
    // the exponent constants in fp64 and their fp32 roundings
    CHECK(std::fabs(g_last_fused.K1d - 1.4426950408889634) < 1e-15);
    CHECK(std::fabs(g_last_fused.K2d - 1.4426950408889634 / 2.0) < 1e-15);
    CHECK(g_last_fused.K1 == (float)g_last_fused.K1d && g_last_fused.K2 == (float)g_last_fused.K2d);
    // the test hook reaches the count kernel's parameters
    CHECK(hl_plan_set_exchange_test(p, 64, 7, 1) == HL_OK);
    CHECK(hl_forward_backward(p, N, x, y, nullptr, t, old, adv, g, sc, nullptr) == HL_OK);
    CHECK(g_last_count.spin_limit == 64 && g_last_count.hold_row == 7 && g_last_count.hold_chunk == 1);
    CHECK(hl_plan_set_exchange_test(p, hl::kSpinLimit, -1, -1) == HL_OK);
    // a metrics-only call, an empty batch, misaligned bases (the row-wise path)
    CHECK(hl_forward_backward(p, N, x, y, nullptr, t, old, adv, nullptr, sc, nullptr) == HL_OK);
    CHECK(hl_forward_backward(p, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, sc, nullptr) ==
          HL_OK);
    CHECK(hl_forward_backward(p, N, x, y, nullptr, fake(0x200000002ull), old, adv, g, sc, nullptr) == HL_OK);
    // workspace too small, then a larger batch than it holds
    CHECK(hl_plan_set_workspace(p, fake(1 << 20), 8) == HL_OK);
    CHECK(hl_forward_backward(p, N, x, y, nullptr, t, old, adv, g, sc, nullptr) == HL_ERR_WORKSPACE);
    CHECK(hl_row_values(p) != nullptr);
    hl_plan_destroy(p);

    // GSPO: forward, segment step, load-mode backward
    CHECK(hl_plan(&p, 20011, HL_BF16, HL_CE | HL_RKL | HL_GSPO, &w, 1.5f, 0.2f, 1.0f, 0.0f) == HL_OK);
    CHECK(hl_plan_set_workspace(p, fake(1 << 20), hl_workspace_bytes(p, 64)) == HL_OK);
    const int32_t* offs = static_cast<const int32_t*>(fake(0x700000000ull));
    const int seam_before = g_seam_calls;
    CHECK(hl_forward_backward_segments(p, 64, x, y, nullptr, t, old, adv, offs, 8, g, sc, nullptr) == HL_OK);
    CHECK(g_seam_calls == seam_before + 1 && g_last_fused.load_mode == 1);
    CHECK(hl_forward_backward(p, 64, x, y, nullptr, t, old, adv, g, sc, nullptr) == HL_ERR_MISSING_INPUT);
    hl_plan_destroy(p);
    hl_plan_destroy(nullptr);
}

}  // namespace

int main() {
    plans_and_variants();
    enqueue_paths();
    if (g_fails) {
        std::fprintf(stderr, "%d check(s) failed\n", g_fails);
        return 1;
    }
    std::printf("host ABI checks passed\n");
    return 0;
}
