// hl_forward_backward_noalloc: the fused call with its workspace in a fixed
// device array of the library, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc). The kernels and launch sequence are those of
// hl_forward_backward_segments; only the workspace differs.
#include <cstdio>
#include <mutex>

#include "hl_internal.h"

// The workspace: one copy per GPU the library runs on, held until the process
// ends. Host code must not use this name as an address (it is a host-side
// stand-in): the device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[HL_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchSlot {
    void* ptr;    // device address of `scratch` on this device (nullptr: not looked up yet)
    bool used;    // a call has run on it: its control words are defined
};

std::mutex g_mu;
ScratchSlot g_slots[kMaxDevices];

hl_status fail(const char* where, hipError_t e) {
    char msg[256];
    std::snprintf(msg, sizeof(msg), "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
    hl::set_last_error(msg);
    return HL_ERR_HIP;
}

}  // namespace

extern "C" hl_status hl_forward_backward_noalloc(hl_plan_t plan, int64_t n_rows, const void* logits,
                                                 const int64_t* labels, const uint8_t* mask,
                                                 const void* teacher_logits, const float* old_logprobs,
                                                 const float* advantages, const int32_t* seq_offsets,
                                                 int64_t n_segments, void* grad_out, float* scalars_out,
                                                 hipStream_t stream) {
    const hl::CallArgs a{n_rows, logits, labels, mask, teacher_logits, old_logprobs, advantages,
                         seq_offsets, n_segments, grad_out, scalars_out};
    hl_status st = hl::check_call(plan, a);
    if (st != HL_OK) return st;
    const size_t need = hl::call_workspace_bytes(plan, n_rows);
    if (need > (size_t)HL_STATIC_WORKSPACE_BYTES) {
        char msg[256];
        std::snprintf(msg, sizeof(msg),
                      "hl_forward_backward_noalloc: %lld rows need %zu bytes of workspace; the static "
                      "workspace holds %zu (HL_STATIC_WORKSPACE_BYTES)",
                      (long long)n_rows, need, (size_t)HL_STATIC_WORKSPACE_BYTES);
        hl::set_last_error(msg);
        return HL_ERR_WORKSPACE;
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail("hipGetDevice", e);
    if (dev < 0 || dev >= kMaxDevices) return HL_ERR_UNSUPPORTED;
    void* ws = nullptr;
    bool reset = false;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        ScratchSlot& slot = g_slots[dev];
        if (slot.ptr == nullptr) {
            // first call on this device (the current one): its copy's address
            void* ptr = nullptr;
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return fail("hipGetSymbolAddress(static workspace)", e);
            slot.ptr = ptr;
        }
        ws = slot.ptr;
        reset = !slot.used;
    }
    st = hl::enqueue_call(plan, a, ws, reset, stream);
    if (st == HL_OK) {
        std::lock_guard<std::mutex> lock(g_mu);
        g_slots[dev].used = true;
    }
    return st;
}
