// Launchers of the valid-row count and the batch reduction kernels.
#include "hl_device.cuh"

namespace hl {

// ---------------------------------------------------------------------------
// count_kernel: one workgroup of 1024 threads. With 16-byte aligned labels
// (and mask), thread t takes rows [16 t, 16 t + 16) of every 16384-row tile
// with eight 16-byte label loads and one 16-byte mask load, all issued before
// any is used, so a tile costs one memory latency; a ragged last tile and
// unaligned inputs go one row at a time.
//
// It also keeps the split-vocab words safe to reuse. A chunk takes a
// sibling's word once the word carries the current call's epoch, so no word
// left in the workspace may carry it: every call bumps the epoch (a 32-bit
// counter in the workspace's control words, whichever plan calls), and the
// words are trusted only where the workspace held zeros or such words
// before. CTRL_CLEAN counts the leading words known to be so. When the
// call's words reach past it (another call's layout kept other data there),
// on a plan's first call on a workspace (control words undefined: `reset`),
// and when the epoch wraps, this kernel zero-fills the call's words first.
// Afterwards CTRL_CLEAN is the call's own word count: its other regions
// follow its words. One workgroup reads the control words, fills and writes
// them, so no other workgroup can see them half updated.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void count_row(int64_t y, bool unmasked, int64_t V, uint32_t& nv, uint32_t& nb) {
    const bool in_range = (y >= 0) && (y < V);
    nv += (unmasked && in_range) ? 1u : 0u;
    nb += (unmasked && !in_range && y != -100) ? 1u : 0u;
}

__global__ __launch_bounds__(1024) void count_kernel(const CountParams p) {
    __shared__ uint32_t s_v[16], s_b[16];
    // every thread reads the control words before thread 0 rewrites them
    // (after the barrier of the count below)
    const uint32_t old_epoch = p.reset ? 0u : p.ctrl[CTRL_EPOCH];
    const uint64_t clean = p.reset ? 0ull
                                   : (((uint64_t)p.ctrl[CTRL_CLEAN_HI] << 32) | (uint64_t)p.ctrl[CTRL_CLEAN_LO]);
    const bool wrap = old_epoch == 0xffffffffu;
    if (p.fill_words > 0 && (p.reset || wrap || clean < (uint64_t)p.fill_words)) {
        // the words start 256-byte aligned and come in groups of 8 per (row, chunk)
        const u32x4 z = {0u, 0u, 0u, 0u};
        u32x4* w = reinterpret_cast<u32x4*>(p.fill);
        for (int64_t i = threadIdx.x; i < p.fill_words / 2; i += 1024) w[i] = z;
    }
    uint32_t nv = 0, nb = 0;
    if (p.vec) {
        for (int64_t base = 0; base < p.n_rows; base += 16384) {
            const int64_t r0 = base + 16 * (int64_t)threadIdx.x;
            if (r0 + 16 <= p.n_rows) {
                const u32x4* lv = reinterpret_cast<const u32x4*>(p.labels + r0);
                u32x4 L[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) L[k] = lv[k];
                u32x4 m = {~0u, ~0u, ~0u, ~0u};
                if (p.mask != nullptr) m = *reinterpret_cast<const u32x4*>(p.mask + r0);
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint64_t lo = L[j >> 1][2 * (j & 1)], hi = L[j >> 1][2 * (j & 1) + 1];
                    const int64_t y = (int64_t)((hi << 32) | lo);
                    const bool unmasked = ((m[j >> 2] >> (8 * (j & 3))) & 0xffu) != 0u;
                    count_row(y, unmasked, p.V, nv, nb);
                }
            } else {
                for (int64_t r = r0; r < p.n_rows && r < r0 + 16; ++r)
                    count_row(p.labels[r], p.mask == nullptr || p.mask[r] != 0, p.V, nv, nb);
            }
        }
    } else {
        for (int64_t r = threadIdx.x; r < p.n_rows; r += 1024) {
            bool valid, bad;
            int64_t y;
            row_status(p.labels, p.mask, r, p.V, p.ctrl, valid, bad, y);
            nv += valid;
            nb += bad;
        }
    }
    for (int m = 32; m >= 1; m >>= 1) {
        nv += __shfl_xor(nv, m, 64);
        nb += __shfl_xor(nb, m, 64);
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) { s_v[wave] = nv; s_b[wave] = nb; }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t tv = 0, tb = 0;
        for (int w = 0; w < 16; ++w) { tv += s_v[w]; tb += s_b[w]; }
        p.ctrl[CTRL_NVALID] = tv;
        p.ctrl[CTRL_NBAD] = tb;
        // this call's epoch: words carry epochs >= 1, a zero-filled word epoch 0
        p.ctrl[CTRL_EPOCH] = (p.reset || wrap) ? 1u : old_epoch + 1u;
        p.ctrl[CTRL_CLEAN_LO] = (uint32_t)((uint64_t)p.fill_words & 0xffffffffu);
        p.ctrl[CTRL_CLEAN_HI] = (uint32_t)((uint64_t)p.fill_words >> 32);
        p.ctrl[CTRL_ERROR] = 0u;
        p.ctrl[CTRL_DONE] = 0u;
        p.ctrl[CTRL_NSEG] = 0u;
        p.ctrl[CTRL_SPIN] = p.spin_limit;
        p.ctrl[CTRL_HOLD_ROW] = p.hold_row;
        p.ctrl[CTRL_HOLD_CHUNK] = p.hold_chunk;
    }
}

// ---------------------------------------------------------------------------
// seam_kernel (GSPO): one wave per segment [o_i, o_{i+1}). From the final row
// records it forms each valid token's log-ratio logp_t - old_t in fp64, sums
// them with the advantages in a fixed order (lane-strided, then an xor
// butterfly, which leaves the same bits in every lane), and derives the
// sequence ratio s_i = exp(mean log-ratio), the segment advantage (mean of
// its tokens' advantages), the clipped objective and the per-token
// coefficient act * A_i * s_i / n_i that the load-mode backward adds to the
// label column. Malformed offsets raise CTRL_ERROR (the scalars and the
// gradient then come out NaN); every access stays inside [0, n_rows).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSeamBlock) void seam_kernel(const SeamParams p) {
    constexpr double LN2 = 0.69314718055994530942;
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * (kSeamBlock / 64) + (threadIdx.x >> 6);
    if (i >= p.n_segments) return;
    const int64_t o0 = p.offsets[i], o1 = p.offsets[i + 1];
    const bool ok = o0 >= 0 && o1 >= o0 && o1 <= p.n_rows && (i != 0 || o0 == 0) &&
                    (i != p.n_segments - 1 || o1 == p.n_rows);
    if (!ok) {
        if (lane == 0) __hip_atomic_store(&p.ctrl[CTRL_ERROR], 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    double sd = 0.0, sa = 0.0;
    uint32_t cnt = 0;
    for (int64_t t = o0 + lane; t < o1; t += 64) {
        const float* rec = p.row_rec + t * REC;
        if (rec[R_VALID] != 0.f) {
            const double lse = ((double)rec[R_M] + log2((double)rec[R_Z] + (double)rec[R_ZL])) * LN2;
            const double xy = rec[R_XY];
            const double sy = p.cap > 0.f ? (double)p.cap * tanh((double)p.k * xy / (double)p.cap)
                                          : (double)p.k * xy;
            sd += (sy - lse) - (double)p.old_logprobs[t];
            sa += (double)p.advantages[t];
            ++cnt;
        }
    }
    for (int m = 1; m < 64; m <<= 1) {
        sd = __dadd_rn(sd, __shfl_xor(sd, m, 64));
        sa = __dadd_rn(sa, __shfl_xor(sa, m, 64));
        cnt += __shfl_xor(cnt, m, 64);
    }
    double loss = 0.0, ratio = 0.0, clip = 0.0, k3 = 0.0, adv = 0.0, deriv = 0.0;
    if (cnt > 0u) {
        const double ls = sd / (double)cnt;
        const double eps = p.eps;
        ratio = exp(ls);
        adv = sa / (double)cnt;
        const double rc = ratio < 1.0 - eps ? 1.0 - eps : (ratio > 1.0 + eps ? 1.0 + eps : ratio);
        const double un = ratio * adv, cl = rc * adv;
        loss = -(un < cl ? un : cl);
        const bool active = !((adv > 0.0 && ratio > 1.0 + eps) || (adv < 0.0 && ratio < 1.0 - eps));
        clip = fabs(ratio - 1.0) > eps ? 1.0 : 0.0;
        k3 = expm1(ls) - ls;
        deriv = active ? adv * ratio / (double)cnt : 0.0;
    }
    if (lane == 0) {
        double* sr = p.seg_rec + i * SEGREC;
        sr[SG_LOSS] = loss;
        sr[SG_RATIO] = ratio;
        sr[SG_CLIP] = clip;
        sr[SG_K3] = k3;
        sr[SG_ADV] = adv;
        sr[SG_NONEMPTY] = cnt > 0u ? 1.0 : 0.0;
        sr[SG_DERIV] = deriv;
        sr[SG_COUNT] = (double)cnt;
        if (cnt > 0u) atomicAdd(&p.ctrl[CTRL_NSEG], 1u);
    }
    const float dc = (float)deriv;
    for (int64_t t = o0 + lane; t < o1; t += 64) {
        p.row_coef[t] = p.row_rec[t * REC + R_VALID] != 0.f ? dc : 0.f;
        p.seg_of_row[t] = (int32_t)i;
    }
}

// ---------------------------------------------------------------------------
// reduce_kernel: one row per thread, kReduceBlock rows per workgroup. Turns
// each row's softmax record into the reported per-row values in fp64 (lse =
// M + log2 Z in the log2 domain, entropy, KL, CE, new log-prob, GRPO
// objective and statistics), stores them for hl_row_values, and sums them:
// a fixed butterfly inside each wave, the waves in order, then the last
// workgroup to finish adds the workgroup sums in workgroup order. Every step
// has a fixed order, so the scalars are identical run to run.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kReduceBlock) void reduce_kernel(const ReduceParams p) {
    constexpr double LN2 = 0.69314718055994530942;
    constexpr int NWR = kReduceBlock / 64;
    __shared__ double s_acc[NWR][NSUM];
    __shared__ double s_sum[NSUM];
    __shared__ uint32_t s_last;
    const uint32_t f = p.flags;
    const int64_t r = (int64_t)blockIdx.x * kReduceBlock + threadIdx.x;
    double v[NCOL];
#pragma unroll
    for (int c = 0; c < NCOL; ++c) v[c] = 0.0;
    if (r < p.n_rows) {
        // every input of the row first, in one round of loads (a masked row's
        // record is all zeros), then the arithmetic
        const float* recp = p.row_rec + r * REC;
        float rec[REC];
#pragma unroll
        for (int c = 0; c < REC; ++c) rec[c] = recp[c];
        const bool grpo_in = (f & F_GRPO) && p.labels != nullptr;
        const float adv_r = grpo_in ? p.advantages[r] : 0.f;
        const float old_r = grpo_in ? p.old_logprobs[r] : 0.f;
        const int64_t sid = (f & F_GSPO) ? (int64_t)p.seg_of_row[r] : -1;
        if (rec[R_VALID] != 0.f) {
            const double Z = (double)rec[R_Z] + (double)rec[R_ZL];   // hi + lo (lo = 0 below fp32)
            const double l2Z = log2(Z);
            const double lse = ((double)rec[R_M] + l2Z) * LN2;
            v[RC_Z] = lse * lse;
            if (f & F_ENT) v[RC_ENT] = LN2 * (l2Z - (double)rec[R_S] / Z);   // S is formed only then
            if (f & F_DISTILL) {
                const double Zt = (double)rec[R_ZT] + (double)rec[R_ZTL];
                const double l2Zt = log2(Zt);
                // the distillation student: the shared softmax, or the tempered
                // one (Hinton mode; its shift is M / tau), whose value carries tau^2
                const bool hinton = (f & F_HINTON) != 0u;
                const double Zd = hinton ? (double)rec[R_ZS] + (double)rec[R_ZSL] : Z;
                const double l2Zd = hinton ? log2(Zd) : l2Z;
                const double sc = hinton ? (double)p.tau * (double)p.tau : 1.0;
                if (f & F_RKL) {
                    v[RC_KL] = sc * LN2 * ((double)rec[R_SX] / Zd - l2Zd + l2Zt);
                } else {
                    v[RC_KL] = LN2 * ((double)rec[R_SX] / Zt - l2Zt + l2Zd);      // forward KL
                    if (f & F_FDCE)                                                 // + teacher entropy
                        v[RC_KL] += LN2 * (l2Zt - (double)rec[R_ST] / Zt);
                    v[RC_KL] *= sc;
                }
            }
            if (p.labels != nullptr) {
                const double xy = rec[R_XY];
                const double sy = p.cap > 0.f ? (double)p.cap * tanh((double)p.k * xy / (double)p.cap)
                                              : (double)p.k * xy;
                v[RC_CE] = lse - sy;
                v[RC_LOGP] = sy - lse;
                if (f & F_GRPO) {
                    const double adv = adv_r;
                    const double d = v[RC_LOGP] - (double)old_r;
                    const double ratio = exp(d);
                    const double eps = p.eps;
                    const double rc = ratio < 1.0 - eps ? 1.0 - eps : (ratio > 1.0 + eps ? 1.0 + eps : ratio);
                    const double un = ratio * adv, cl = rc * adv;
                    v[RC_GRPO] = -(un < cl ? un : cl);
                    v[RC_RATIO] = ratio;
                    v[RC_CLIP] = fabs(ratio - 1.0) > eps ? 1.0 : 0.0;
                    v[RC_K3] = expm1(d) - d;
                    v[RC_ADV] = adv;
                }
            }
            if (f & F_GSPO) {
                // per-token view of the token's segment
                const bool in = sid >= 0 && sid < p.n_segments;
                const double* sr = p.seg_rec + (in ? sid : 0) * SEGREC;
                const double qnan = __builtin_nan("");
                v[RC_GRPO] = in ? sr[SG_LOSS] : qnan;
                v[RC_RATIO] = in ? sr[SG_RATIO] : qnan;
                v[RC_CLIP] = in ? sr[SG_CLIP] : qnan;
                v[RC_K3] = in ? sr[SG_K3] : qnan;
                v[RC_ADV] = in ? sr[SG_ADV] : qnan;
            }
            v[RC_VALID] = 1.0;
        }
        float* out = p.rows + r * NCOL;
#pragma unroll
        for (int c = 0; c < NCOL; ++c) out[c] = (float)v[c];
    }
    if (f & F_GSPO) {
        // the policy columns are summed over segments, not rows: thread r
        // contributes segment r (there are never more segments than rows)
        v[RC_GRPO] = v[RC_RATIO] = v[RC_CLIP] = v[RC_K3] = v[RC_ADV] = 0.0;
        if (r < p.n_segments) {
            const double* sr = p.seg_rec + r * SEGREC;
            if (sr[SG_NONEMPTY] != 0.0) {
                v[RC_GRPO] = sr[SG_LOSS];
                v[RC_RATIO] = sr[SG_RATIO];
                v[RC_CLIP] = sr[SG_CLIP];
                v[RC_K3] = sr[SG_K3];
                v[RC_ADV] = sr[SG_ADV];
            }
        }
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int c = 0; c < NSUM; ++c) {
        double x = v[c];
        for (int m = 1; m < 64; m <<= 1) x = __dadd_rn(x, __shfl_xor(x, m, 64));
        if (lane == 0) s_acc[wave][c] = x;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double* mine = p.partials + (int64_t)blockIdx.x * NSUM;
        for (int c = 0; c < NSUM; ++c) {
            double x = 0.0;
            for (int w = 0; w < NWR; ++w) x += s_acc[w][c];
            mine[c] = x;
        }
        __threadfence();
        const uint32_t done = atomicAdd(&p.ctrl[CTRL_DONE], 1u);
        s_last = (done == gridDim.x - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (s_last == 0u) return;
    __threadfence();
    // last workgroup: thread t adds workgroup sums t, t + 256, ... in order,
    // then a fixed pairwise tree over the 256 threads
    __shared__ double s_tree[NSUM][kReduceBlock];
    {
        double acc2[NSUM];
#pragma unroll
        for (int c = 0; c < NSUM; ++c) acc2[c] = 0.0;
        for (uint32_t g = threadIdx.x; g < gridDim.x; g += kReduceBlock) {
#pragma unroll
            for (int c = 0; c < NSUM; ++c) {
                const uint64_t bits = __hip_atomic_load(
                    reinterpret_cast<const uint64_t*>(p.partials + (int64_t)g * NSUM + c),
                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                acc2[c] += __longlong_as_double((long long)bits);
            }
        }
#pragma unroll
        for (int c = 0; c < NSUM; ++c) s_tree[c][threadIdx.x] = acc2[c];
    }
    __syncthreads();
    for (int half = kReduceBlock / 2; half >= 1; half >>= 1) {
        if ((int)threadIdx.x < half) {
#pragma unroll
            for (int c = 0; c < NSUM; ++c) s_tree[c][threadIdx.x] += s_tree[c][threadIdx.x + half];
        }
        __syncthreads();
    }
    if (threadIdx.x < NSUM) s_sum[threadIdx.x] = s_tree[threadIdx.x][0];
    __syncthreads();
    if (threadIdx.x != 0) return;
    const double* sum = s_sum;
    const uint32_t n_valid = p.ctrl[CTRL_NVALID];
    const double n = p.divisor > 0.f ? (double)p.divisor : (double)n_valid;
    float out[NSCALARS];
    for (int i = 0; i < NSCALARS; ++i) out[i] = 0.f;
    if (n_valid > 0 && n > 0.0) {
        const double inv = 1.0 / n;
        double ce = 0, z = 0, kl = 0, grpo = 0;
        if (f & F_CE) { ce = sum[RC_CE] * inv; out[0] = (float)ce; }
        if (f & F_Z) { z = sum[RC_Z] * inv; out[1] = (float)z; }
        if (f & F_DISTILL) { kl = sum[RC_KL] * inv; out[2] = (float)kl; }
        if (f & F_GRPO) {
            grpo = sum[RC_GRPO] * inv;
            out[3] = (float)grpo;
            out[4] = (float)(sum[RC_LOGP] * inv);
            out[5] = (float)(sum[RC_RATIO] * inv);
            out[6] = (float)(sum[RC_CLIP] * inv);
            out[7] = (float)(sum[RC_K3] * inv);
            out[8] = (float)(sum[RC_ADV] * inv);
        }
        if (f & F_GSPO) {
            out[4] = (float)(sum[RC_LOGP] * inv);
            const uint32_t n_seg = p.ctrl[CTRL_NSEG];
            if (n_seg > 0u) {
                const double is = 1.0 / (double)n_seg;
                grpo = sum[RC_GRPO] * is;
                out[3] = (float)grpo;
                out[5] = (float)(sum[RC_RATIO] * is);
                out[6] = (float)(sum[RC_CLIP] * is);
                out[7] = (float)(sum[RC_K3] * is);
                out[8] = (float)(sum[RC_ADV] * is);
            }
        }
        if (f & F_ENT) out[9] = (float)(sum[RC_ENT] * inv);
        out[10] = (float)((double)p.w_ce * ce + (double)p.w_z * z + (double)p.w_d * kl +
                          (double)p.w_g * grpo);
    }
    out[11] = (float)n_valid;
    out[12] = (float)p.ctrl[CTRL_NBAD];
    if (p.ctrl[CTRL_ERROR] != 0u) {
        // a split-vocab row never saw all of its chunks, or the segment
        // offsets were malformed: nothing is trustworthy
        for (int i = 0; i < 11; ++i) out[i] = __builtin_nanf("");
    }
    for (int i = 0; i < NSCALARS; ++i) p.scalars[i] = out[i];
}

hipError_t launch_count(const CountParams& p, hipStream_t s) {
    (void)hipGetLastError();   // drop an error left by an earlier, unrelated call
    hipLaunchKernelGGL(count_kernel, dim3(1), dim3(1024), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_seam(const SeamParams& p, hipStream_t s) {
    (void)hipGetLastError();
    constexpr int per = kSeamBlock / 64;
    const int64_t groups = (p.n_segments + per - 1) / per;
    hipLaunchKernelGGL(seam_kernel, dim3((unsigned)groups), dim3(kSeamBlock), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t s) {
    (void)hipGetLastError();
    const int64_t groups = p.n_rows > 0 ? (p.n_rows + kReduceBlock - 1) / kReduceBlock : 1;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)groups), dim3(kReduceBlock), 0, s, p);
    return hipGetLastError();
}

}  // namespace hl
