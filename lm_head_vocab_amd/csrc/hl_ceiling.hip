// Memory-system reference for the roofline: the fused kernel's traffic shape
// with no arithmetic. Each workgroup reads its block of 16-byte vectors from
// one or two tensors into registers (all loads issued before any use, as the
// fused kernel does with its register-resident slice), combines them with a
// bitwise xor, and writes one tensor. Its rate is what HBM gives this
// read/write mix and burst length, the ceiling the fused kernel is compared
// with besides the vendor peak.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "headloss.h"
#include "hl_internal.h"

namespace hl {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <int NREAD, int BLOCK, int B>
__global__ __launch_bounds__(BLOCK) void ceiling_kernel(const v4u* __restrict__ a, const v4u* __restrict__ b,
                                                        v4u* __restrict__ out, int64_t n) {
    // this workgroup's block: [start, start + B * BLOCK) vectors, `rem` of them in range
    const int64_t start = (int64_t)blockIdx.x * B * BLOCK;
    const int64_t left = n - start;
    const int rem = left < (int64_t)B * BLOCK ? (int)left : B * BLOCK;
    const v4u* pa = a + start;
    const v4u* pb = b + start;
    v4u* po = out + start;
    const int tid = threadIdx.x;
    v4u x[B], y[NREAD == 2 ? B : 1];
#pragma unroll
    for (int u = 0; u < B; ++u) {
        // every slot loads (no branch); a slot past the range re-reads the last vector
        const int i = u * BLOCK + tid < rem ? u * BLOCK + tid : rem - 1;
        x[u] = __builtin_nontemporal_load(pa + i);
        if (NREAD == 2) y[u] = __builtin_nontemporal_load(pb + i);
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
        if (u * BLOCK + tid < rem) {
            v4u v = x[u];
            if (NREAD == 2) v ^= y[u];
            __builtin_nontemporal_store(v, po + u * BLOCK + tid);
        }
    }
}

typedef void (*CeilingKernel)(const v4u*, const v4u*, v4u*, int64_t);

// 13 vectors per thread only where the fused kernel has them (two tensors at
// 512 threads; at 1024 threads 26 vectors would not fit the registers)
template <int NREAD, int BLOCK>
CeilingKernel pick_b(int b) {
    switch (b) {
        case 4: return ceiling_kernel<NREAD, BLOCK, 4>;
        case 6: return ceiling_kernel<NREAD, BLOCK, 6>;
        case 8: return ceiling_kernel<NREAD, BLOCK, 8>;
        case 9: return ceiling_kernel<NREAD, BLOCK, 9>;
        case 10: return ceiling_kernel<NREAD, BLOCK, 10>;
        case 13:
            if constexpr (BLOCK == 512) return ceiling_kernel<NREAD, BLOCK, 13>;
            else return nullptr;
        default: return nullptr;
    }
}

CeilingKernel pick(int n_reads, int block, int b) {
    if (n_reads == 1) return block == 512 ? pick_b<1, 512>(b) : block == 1024 ? pick_b<1, 1024>(b) : nullptr;
    if (n_reads == 2) return block == 512 ? pick_b<2, 512>(b) : block == 1024 ? pick_b<2, 1024>(b) : nullptr;
    return nullptr;
}

}  // namespace
}  // namespace hl

extern "C" hl_status hl_stream_ceiling(const void* read0, const void* read1, void* write, int64_t bytes, int block,
                                       int vec_per_thread, int reps, hipStream_t stream, float* ms_per_launch) {
    using namespace hl;
    if (read0 == nullptr || write == nullptr || ms_per_launch == nullptr || bytes <= 0 || reps < 1 ||
        (bytes & 15) != 0 || ((reinterpret_cast<uintptr_t>(read0) | reinterpret_cast<uintptr_t>(write) |
                               reinterpret_cast<uintptr_t>(read1)) & 15) != 0)
        return HL_ERR_INVALID_ARG;
    const int n_reads = read1 != nullptr ? 2 : 1;
    CeilingKernel k = pick(n_reads, block, vec_per_thread);
    if (k == nullptr) return HL_ERR_UNSUPPORTED;
    const int64_t n = bytes / 16;
    const int64_t per = (int64_t)block * vec_per_thread;
    const int64_t groups = (n + per - 1) / per;
    if (groups > 0x7fffffff) return HL_ERR_UNSUPPORTED;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    const v4u* a = static_cast<const v4u*>(read0);
    const v4u* b = static_cast<const v4u*>(read1 != nullptr ? read1 : read0);
    v4u* o = static_cast<v4u*>(write);
    if (e == hipSuccess) {
        (void)hipGetLastError();
        hipLaunchKernelGGL(k, dim3((unsigned)groups), dim3(block), 0, stream, a, b, o, n);   // warm-up
        e = hipEventRecord(e0, stream);
    }
    for (int r = 0; r < reps && e == hipSuccess; ++r) {
        hipLaunchKernelGGL(k, dim3((unsigned)groups), dim3(block), 0, stream, a, b, o, n);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, stream);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (e != hipSuccess) {
        char msg[192];
        std::snprintf(msg, sizeof(msg), "hl_stream_ceiling: %s (%d)", hipGetErrorString(e), (int)e);
        set_last_error(msg);
        return HL_ERR_HIP;
    }
    *ms_per_launch = ms / (float)reps;
    return HL_OK;
}
