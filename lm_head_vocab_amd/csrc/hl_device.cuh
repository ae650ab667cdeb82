// Device code of the fused LM-head loss for gfx950 (CDNA4).
//
// Three kernels per call, all on the caller's stream:
//   count_kernel   valid-row count and bad-label count (the batch divisor
//                  must be known before any gradient is written);
//   fused_kernel   one workgroup per (row, vocabulary chunk): loads its slice
//                  of the row into registers once, computes the softmax
//                  statistics (max, sum-exp, entropy sum, teacher sums) with
//                  wave64 DPP reductions, combines them across waves (and,
//                  in the split-vocab variant, across the row's chunks), forms
//                  the per-row coefficients and writes the gradient from the
//                  registers it already holds;
//   reduce_kernel  fixed-order fp64 sum of the per-row values into the batch
//                  scalars.
// A call without a gradient computes the statistics with stream_stats_kernel
// instead (one workgroup per row, the row streamed once, no chunk exchange).
// With GSPO that kernel runs first (row statistics), then, after a segment
// kernel has turned the statistics into per-segment ratios and per-row
// coefficients, the fused kernel in load mode (the statistics read back from
// the row records, the slice reloaded, the gradient written); rows longer
// than every slice the chunk exchange serves take the same two launches
// without the segment step. Inputs whose base addresses differ modulo 16
// bytes take rowwise_kernel in place of the fused kernel.
//
// The gradient is written in the two-coefficient form of Fast-LLM PR #558
// (Triton kernel for the monolithic loss, section Design): prob_coeff times
// the softmax minus label_coeff at the label column, plus the distillation
// term, formed in fp32 and rounded once (Fast-LLM PR #549, "Monolithic fused
// head-loss kernel (torch.compile)", section Approach).
#pragma once

#include <type_traits>

#include "hl_internal.h"

namespace hl {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2f = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// Element formats. A 16-byte vector holds VEC elements.
// ---------------------------------------------------------------------------
struct F32T {
    static constexpr int VEC = 4;
    static constexpr int ESIZE = 4;
    __device__ static __forceinline__ float get(const u32x4& w, int e) {
        return __uint_as_float(w[e]);
    }
    __device__ static __forceinline__ float load1(const char* rowbase, int64_t i) {
        return reinterpret_cast<const float*>(rowbase)[i];
    }
    __device__ static __forceinline__ uint32_t raw1(const char* rowbase, int64_t i) {
        return reinterpret_cast<const uint32_t*>(rowbase)[i];
    }
    __device__ static __forceinline__ float from_raw(uint32_t b) { return __uint_as_float(b); }
    __device__ static __forceinline__ void store1(char* rowbase, int64_t i, float g) {
        reinterpret_cast<float*>(rowbase)[i] = g;
    }
    // running max over the 4 elements of a vector
    __device__ static __forceinline__ float vmax(float acc, const u32x4& w) {
        return fmaxf(fmaxf(acc, fmaxf(__uint_as_float(w[0]), __uint_as_float(w[1]))),
                     fmaxf(__uint_as_float(w[2]), __uint_as_float(w[3])));
    }
    __device__ static __forceinline__ u32x4 pack(const float* g) {
        u32x4 r;
        r[0] = __float_as_uint(g[0]);
        r[1] = __float_as_uint(g[1]);
        r[2] = __float_as_uint(g[2]);
        r[3] = __float_as_uint(g[3]);
        return r;
    }
};

struct BF16T {
    static constexpr int VEC = 8;
    static constexpr int ESIZE = 2;
    // bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32.
    __device__ static __forceinline__ float get(const u32x4& w, int e) {
        const uint32_t word = w[e >> 1];
        return (e & 1) ? __uint_as_float(word & 0xffff0000u) : __uint_as_float(word << 16);
    }
    __device__ static __forceinline__ float load1(const char* rowbase, int64_t i) {
        const uint32_t h = reinterpret_cast<const uint16_t*>(rowbase)[i];
        return __uint_as_float(h << 16);
    }
    __device__ static __forceinline__ uint32_t raw1(const char* rowbase, int64_t i) {
        return reinterpret_cast<const uint16_t*>(rowbase)[i];
    }
    __device__ static __forceinline__ float from_raw(uint32_t b) { return __uint_as_float(b << 16); }
    // Running max over the 8 elements of a vector, used only as the softmax
    // shift: the odd element is read as the whole 32-bit word (its bf16 bits
    // plus the even element's bits below them), which is within one bf16 ulp
    // of it; the even element is exact.
    __device__ static __forceinline__ float vmax(float acc, const u32x4& w) {
#pragma unroll
        for (int k = 0; k < 4; ++k) acc = fmaxf(acc, fmaxf(__uint_as_float(w[k]), __uint_as_float(w[k] << 16)));
        return acc;
    }
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
        f32x2 v = {lo, hi};
        bf16x2 b = __builtin_convertvector(v, bf16x2);   // v_cvt_pk_bf16_f32, RNE
        return __builtin_bit_cast(uint32_t, b);
    }
    __device__ static __forceinline__ void store1(char* rowbase, int64_t i, float g) {
        reinterpret_cast<uint16_t*>(rowbase)[i] = static_cast<uint16_t>(pack2(g, 0.0f) & 0xffffu);
    }
    __device__ static __forceinline__ u32x4 pack(const float* g) {
        u32x4 r;
        r[0] = pack2(g[0], g[1]);
        r[1] = pack2(g[2], g[3]);
        r[2] = pack2(g[4], g[5]);
        r[3] = pack2(g[6], g[7]);
        return r;
    }
};

struct F16T {
    static constexpr int VEC = 8;
    static constexpr int ESIZE = 2;
    __device__ static __forceinline__ float get(const u32x4& w, int e) {
        const uint32_t word = w[e >> 1];
        const uint16_t h = (e & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xffffu);
        return (float)__builtin_bit_cast(_Float16, h);
    }
    __device__ static __forceinline__ float load1(const char* rowbase, int64_t i) {
        return (float)reinterpret_cast<const _Float16*>(rowbase)[i];
    }
    __device__ static __forceinline__ uint32_t raw1(const char* rowbase, int64_t i) {
        return reinterpret_cast<const uint16_t*>(rowbase)[i];
    }
    __device__ static __forceinline__ float from_raw(uint32_t b) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
    }
    __device__ static __forceinline__ float vmax(float acc, const u32x4& w) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) acc = fmaxf(acc, fmaxf(get(w, e), get(w, e + 1)));
        return acc;
    }
    __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
        f32x2 v = {lo, hi};
        f16x2 h = __builtin_convertvector(v, f16x2);   // round to nearest even
        return __builtin_bit_cast(uint32_t, h);
    }
    __device__ static __forceinline__ void store1(char* rowbase, int64_t i, float g) {
        reinterpret_cast<_Float16*>(rowbase)[i] = (_Float16)g;
    }
    __device__ static __forceinline__ u32x4 pack(const float* g) {
        u32x4 r;
        r[0] = pack2(g[0], g[1]);
        r[1] = pack2(g[2], g[3]);
        r[2] = pack2(g[4], g[5]);
        r[3] = pack2(g[6], g[7]);
        return r;
    }
};

__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_stream(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ float fast_exp2(float a) { return __builtin_amdgcn_exp2f(a); }

// 2^a in fp64: 2^a = 2^n 2^u with n = rint(a), |u| <= 1/2, and 2^u = e^(u ln 2)
// from the Taylor series of the exponential to degree 8 (remainder below
// 2^-32 relative, ample for a result that is rounded to fp32). Branch-free:
// arguments below -1100 (-Inf included) are clamped there and give 0 from
// the final scaling; a NaN argument gives NaN.
__device__ __forceinline__ double exp2_hp(double a) {
    constexpr double LN2 = 0.69314718055994530942;
    a = a < -1100.0 ? -1100.0 : a;
    const double n = rint(a);
    const double v = (a - n) * LN2;
    double e = 1.0 / 40320.0;
    e = fma(e, v, 1.0 / 5040.0);
    e = fma(e, v, 1.0 / 720.0);
    e = fma(e, v, 1.0 / 120.0);
    e = fma(e, v, 1.0 / 24.0);
    e = fma(e, v, 1.0 / 6.0);
    e = fma(e, v, 0.5);
    e = fma(e, v, 1.0);
    e = fma(e, v, 1.0);
    return ldexp(e, (int)n);
}

// tanh from its definition: the odd Taylor polynomial (coefficients
// 2^(2n) (2^(2n)-1) B_2n / (2n)!, terms z .. z^9) for |z| < 0.25, where the
// truncation error is below 1e-8 relative and the fp32 result within 1.2e-7,
// and 1 - 2 / (exp(2|z|) + 1) above, where that form has no damaging
// cancellation (within 2.6e-7 relative).
__device__ __forceinline__ float hl_tanh(float z) {
    const float az = fabsf(z);
    float r;
    if (az < 0.25f) {
        const float z2 = z * z;
        float p = 0.021869488536155203f;
        p = fmaf(p, z2, -0.05396825396825397f);
        p = fmaf(p, z2, 0.13333333333333333f);
        p = fmaf(p, z2, -0.3333333333333333f);
        r = fmaf(z * z2, p, z);
    } else {
        const float e = fast_exp2(az * (2.0f * kLog2e));
        r = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
        r = copysignf(r, z);
    }
    return r;
}

// Softcap on the element paths, branch-free: with r = 1 / (exp(2 k x / c) + 1),
// tanh(k x / c) = 1 - 2 r, so the log2-domain logit is s log2(e) =
// c log2(e) - 2 c log2(e) r and the chain factor 1 - tanh^2 is 4 r (1 - r).
// 1 - 2 r is exact given r, so the absolute error of tanh stays within a few
// 2^-24 for every argument; the relative error near zero is larger than the
// polynomial's above, but the softmax, the z-loss and the entropy see s only
// through differences and through s itself. exp overflow gives r = 0
// (tanh = 1) and underflow r = 1 (tanh = -1), each with a zero chain factor.
__device__ __forceinline__ float cap_r(float x, float kc2) {
    return __builtin_amdgcn_rcpf(fast_exp2(x * kc2) + 1.0f);
}

// ---------------------------------------------------------------------------
// Wave64 reductions. Within a row of 16 lanes: DPP quad_perm (xor 1, xor 2),
// row_half_mirror, row_mirror; across rows: permlane swaps. Every lane ends
// with the same value, combined in the same pairing order.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // row_half_mirror
constexpr int DPP_MIRROR = 0x140;       // row_mirror

// Across the four 16-lane rows: v_permlane16_swap exchanges odd rows of one
// copy with even rows of the other, and v_permlane32_swap the two 32-lane
// halves, so each lane receives its own value and its partner's (row r and
// r ^ 1, resp. half h and h ^ 1) without an LDS round trip; combining the pair
// gives every lane the same bits (the combines are commutative).
struct LanePair {
    float a, b;
};
__device__ __forceinline__ LanePair pair16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return LanePair{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair pair32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return LanePair{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<DPP_XOR1>(v));
    v = fmaxf(v, dpp<DPP_XOR2>(v));
    v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
    v = fmaxf(v, dpp<DPP_MIRROR>(v));
    LanePair q = pair16(v);
    v = fmaxf(q.a, q.b);
    q = pair32(v);
    return fmaxf(q.a, q.b);
}

__device__ __forceinline__ float wave_sum(float v) {
    v = __fadd_rn(v, dpp<DPP_XOR1>(v));
    v = __fadd_rn(v, dpp<DPP_XOR2>(v));
    v = __fadd_rn(v, dpp<DPP_HALF_MIRROR>(v));
    v = __fadd_rn(v, dpp<DPP_MIRROR>(v));
    LanePair q = pair16(v);
    v = __fadd_rn(q.a, q.b);
    q = pair32(v);
    return __fadd_rn(q.a, q.b);
}

// The same butterfly in fp64 (the fp32 instances' normalizer sums): each
// step moves the two 32-bit halves.
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xf, 0xf, false);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double pair_sum_d16(double v) {
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)__double2loint(v), (uint32_t)__double2loint(v), false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)__double2hiint(v), (uint32_t)__double2hiint(v), false, false);
    return __dadd_rn(__hiloint2double((int)hi[0], (int)lo[0]), __hiloint2double((int)hi[1], (int)lo[1]));
}
__device__ __forceinline__ double pair_sum_d32(double v) {
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)__double2loint(v), (uint32_t)__double2loint(v), false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)__double2hiint(v), (uint32_t)__double2hiint(v), false, false);
    return __dadd_rn(__hiloint2double((int)hi[0], (int)lo[0]), __hiloint2double((int)hi[1], (int)lo[1]));
}
__device__ __forceinline__ double wave_sum_d(double v) {
    v = __dadd_rn(v, dpp_d<DPP_XOR1>(v));
    v = __dadd_rn(v, dpp_d<DPP_XOR2>(v));
    v = __dadd_rn(v, dpp_d<DPP_HALF_MIRROR>(v));
    v = __dadd_rn(v, dpp_d<DPP_MIRROR>(v));
    v = pair_sum_d16(v);
    return pair_sum_d32(v);
}

// An fp64 value as a hi + lo pair of floats.
__device__ __forceinline__ void split_hl(double v, float& hi, float& lo) {
    hi = (float)v;
    lo = (float)(v - (double)hi);
}

// 2^d for a shift difference d. The fp32 instances (HP) use integer shifts,
// so d is an integer (exact: both shifts are integers below 2^24 in
// magnitude, or the factor is 0 anyway) and the factor an exact power of
// two; -Inf and NaN (an empty side) give 0.
template <bool HP>
__device__ __forceinline__ float shift_int(float m) {
    if constexpr (HP) return ceilf(m);
    else return m;
}
template <bool HP>
__device__ __forceinline__ float pow2_of(float d) {
    if constexpr (HP) return ldexpf(1.0f, (int)fmaxf(d, -1000.0f));
    else return fast_exp2(d);
}

// ---------------------------------------------------------------------------
// Softmax-statistics record and its merge (the max-rescaling combine of an
// online softmax). Written with non-contracted operations so that
// merge(a, b) == merge(b, a) bit for bit; an empty slice has Z == 0.
// ---------------------------------------------------------------------------
struct Rec {
    float M, Z, S, Mt, Zt, SX, St, Zs;
    float Zl, Ztl, Zsl;   // low parts of Z, Zt, Zs (fp32 instances; 0 otherwise)
};

__device__ __forceinline__ Rec rec_empty() {
    return Rec{kNegInf, 0.f, 0.f, kNegInf, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
}

// Merge two records (beta = 1 / tau, used by the tempered student sums of the
// Hinton modes, whose offsets move by beta times the student's shift change).
// HP (the fp32 instances): the shifts are integers and the normalizers Z, Zt,
// Zs are merged in fp64 from their hi + lo parts (betad = 1 / tau in fp64).
template <int TMODE, bool HP = false>
__device__ __forceinline__ Rec rec_merge(const Rec& a, const Rec& b, float beta, double betad = 1.0) {
    const bool ea = (a.Z == 0.f), eb = (b.Z == 0.f);
    Rec r;
    const float M = fmaxf(a.M, b.M);
    const float da = __fsub_rn(a.M, M), db = __fsub_rn(b.M, M);
    const float fa = pow2_of<HP>(da), fb = pow2_of<HP>(db);
    r.M = M;
    r.Z = __fadd_rn(__fmul_rn(a.Z, fa), __fmul_rn(b.Z, fb));
    r.S = __fadd_rn(__fmul_rn(fa, __fadd_rn(a.S, __fmul_rn(da, a.Z))),
                    __fmul_rn(fb, __fadd_rn(b.S, __fmul_rn(db, b.Z))));
    if (TMODE != TM_NONE) {
        const float Mt = fmaxf(a.Mt, b.Mt);
        const float dta = __fsub_rn(a.Mt, Mt), dtb = __fsub_rn(b.Mt, Mt);
        const float fta = pow2_of<HP>(dta), ftb = pow2_of<HP>(dtb);
        r.Mt = Mt;
        r.Zt = __fadd_rn(__fmul_rn(a.Zt, fta), __fmul_rn(b.Zt, ftb));
        r.Zs = 0.f;
        if (is_hinton(TMODE)) {
            // tempered student offsets (A_j - M) beta move by d beta
            const float dsa = __fmul_rn(da, beta), dsb = __fmul_rn(db, beta);
            const float fsa = fast_exp2(dsa), fsb = fast_exp2(dsb);
            r.Zs = __fadd_rn(__fmul_rn(a.Zs, fsa), __fmul_rn(b.Zs, fsb));
            if (fkl_like(TMODE)) {
                // SX = sum_j 2^u_j (u_j - a_j beta)
                r.SX = __fadd_rn(__fmul_rn(fta, __fadd_rn(a.SX, __fmul_rn(__fsub_rn(dta, dsa), a.Zt))),
                                 __fmul_rn(ftb, __fadd_rn(b.SX, __fmul_rn(__fsub_rn(dtb, dsb), b.Zt))));
            } else {
                // SX = sum_j 2^(a_j beta) (a_j beta - u_j)
                r.SX = __fadd_rn(__fmul_rn(fsa, __fadd_rn(a.SX, __fmul_rn(__fsub_rn(dsa, dta), a.Zs))),
                                 __fmul_rn(fsb, __fadd_rn(b.SX, __fmul_rn(__fsub_rn(dsb, dtb), b.Zs))));
            }
        } else if (fkl_like(TMODE)) {
            // SX = sum_j 2^u_j (u_j - a_j): both offsets move
            r.SX = __fadd_rn(__fmul_rn(fta, __fadd_rn(a.SX, __fmul_rn(__fsub_rn(dta, da), a.Zt))),
                             __fmul_rn(ftb, __fadd_rn(b.SX, __fmul_rn(__fsub_rn(dtb, db), b.Zt))));
        } else {
            // SX = sum_j 2^a_j (a_j - u_j)
            r.SX = __fadd_rn(__fmul_rn(fa, __fadd_rn(a.SX, __fmul_rn(__fsub_rn(da, dta), a.Z))),
                             __fmul_rn(fb, __fadd_rn(b.SX, __fmul_rn(__fsub_rn(db, dtb), b.Z))));
        }
        // St = sum_j 2^u_j u_j: the teacher offset moves, as S does for the student
        r.St = has_st(TMODE)
                   ? __fadd_rn(__fmul_rn(fta, __fadd_rn(a.St, __fmul_rn(dta, a.Zt))),
                               __fmul_rn(ftb, __fadd_rn(b.St, __fmul_rn(dtb, b.Zt))))
                   : 0.f;
    } else {
        r.Mt = 0.f; r.Zt = 0.f; r.SX = 0.f; r.St = 0.f; r.Zs = 0.f;
    }
    r.Zl = 0.f; r.Ztl = 0.f; r.Zsl = 0.f;
    if constexpr (HP) {
        // integer shifts: each side is rescaled exactly, the sum rounded once
        // in fp64; the tempered sums move by d / tau, an fp64 exponential
        split_hl((double)a.Z * fa + (double)a.Zl * fa + ((double)b.Z * fb + (double)b.Zl * fb), r.Z, r.Zl);
        if (TMODE != TM_NONE) {
            const double fta = pow2_of<HP>(__fsub_rn(a.Mt, r.Mt)), ftb = pow2_of<HP>(__fsub_rn(b.Mt, r.Mt));
            split_hl((double)a.Zt * fta + (double)a.Ztl * fta + ((double)b.Zt * ftb + (double)b.Ztl * ftb), r.Zt,
                     r.Ztl);
            if (is_hinton(TMODE)) {
                const double fsa = exp2_hp((double)da * betad), fsb = exp2_hp((double)db * betad);
                split_hl(((double)a.Zs + (double)a.Zsl) * fsa + ((double)b.Zs + (double)b.Zsl) * fsb, r.Zs, r.Zsl);
            }
        }
    }
    if (ea) r = b;
    if (eb) r = a;
    return r;
}

template <int CTRL, int TMODE, bool HP = false>
__device__ __forceinline__ Rec rec_dpp_step(const Rec& a, float beta, double betad = 1.0) {
    Rec b;
    b.M = dpp<CTRL>(a.M);
    b.Z = dpp<CTRL>(a.Z);
    b.S = dpp<CTRL>(a.S);
    if (TMODE != TM_NONE) {
        b.Mt = dpp<CTRL>(a.Mt);
        b.Zt = dpp<CTRL>(a.Zt);
        b.SX = dpp<CTRL>(a.SX);
        b.St = has_st(TMODE) ? dpp<CTRL>(a.St) : 0.f;
        b.Zs = is_hinton(TMODE) ? dpp<CTRL>(a.Zs) : 0.f;
    } else {
        b.Mt = 0.f; b.Zt = 0.f; b.SX = 0.f; b.St = 0.f; b.Zs = 0.f;
    }
    b.Zl = 0.f; b.Ztl = 0.f; b.Zsl = 0.f;
    if constexpr (HP) {
        b.Zl = dpp<CTRL>(a.Zl);
        if (TMODE != TM_NONE) b.Ztl = dpp<CTRL>(a.Ztl);
        if (is_hinton(TMODE)) b.Zsl = dpp<CTRL>(a.Zsl);
    }
    return rec_merge<TMODE, HP>(a, b, beta, betad);
}

// Merge the records held by lanes 0..n-1 of every 16-lane row (lanes n..15
// hold empty records); all lanes end with the same result. A step whose
// partners are all empty is skipped: merging with an empty record returns
// the other one unchanged, so the result is the same for any n.
template <int TMODE, bool HP = false>
__device__ __forceinline__ Rec rec_reduce16(Rec r, float beta, int n, double betad = 1.0) {
    if (n > 1) r = rec_dpp_step<DPP_XOR1, TMODE, HP>(r, beta, betad);
    if (n > 2) r = rec_dpp_step<DPP_XOR2, TMODE, HP>(r, beta, betad);
    if (n > 4) r = rec_dpp_step<DPP_HALF_MIRROR, TMODE, HP>(r, beta, betad);
    if (n > 8) r = rec_dpp_step<DPP_MIRROR, TMODE, HP>(r, beta, betad);
    return r;
}

// ---------------------------------------------------------------------------
// Row validity (shared by the count and fused kernels): masked when the mask
// byte is 0, the label is -100, or the label is outside [0, V).
// ---------------------------------------------------------------------------
// Both the mask byte and the label are loaded, without a branch, before
// either is used (a missing input reads the 8-byte-aligned word at `spare`,
// any readable device memory, and its value is ignored), so the row's status
// costs one memory latency, not two.
__device__ __forceinline__ void row_status(const int64_t* labels, const uint8_t* mask, int64_t row,
                                           int64_t V, const void* spare, bool& valid, bool& bad,
                                           int64_t& y) {
    const uint8_t* mp = mask != nullptr ? mask + row : static_cast<const uint8_t*>(spare);
    const int64_t* lp = labels != nullptr ? labels + row : static_cast<const int64_t*>(spare);
    const uint32_t mk = *mp;
    const int64_t yl = *lp;
    const bool has_l = labels != nullptr;
    const bool unmasked = (mask == nullptr) || (mk != 0u);
    y = has_l ? yl : -1;
    const bool in_range = !has_l || ((y >= 0) && (y < V));
    valid = unmasked && in_range;
    bad = unmasked && !in_range && (y != -100);
}

// ---------------------------------------------------------------------------
// Per-row gradient coefficients and the per-element gradient
// ---------------------------------------------------------------------------
// The gradient of the weighted loss with respect to the raw logit x_j is
//   G k / n * c_j * (P q_j - L [j == y] - w_fkl p_j + w_rkl q_j (lq_j - lp_j - RKL))
// with P = w_ce + 2 w_z lse + w_g a + w_fkl, L = w_ce + w_g a, a = act * A * r,
// c_j = 1 (or 1 - tanh^2 with softcap). Fast-LLM PR #558 (Triton kernel for
// the monolithic loss), section Design: every loss only adds to the
// probability coefficient and the label-column coefficient. In the Hinton
// modes the distillation term is written in the tempered student
// q^tau_j = softmax(s / tau)_j instead: tau w (q^tau_j - p_j), or
// tau w q^tau_j (lq^tau_j - lp_j - KL_tau) for the reverse KL (the tau^2 on
// the loss times the 1 / tau of d(s / tau) / ds).
//
// Precision of the fp32 instances (HP). An fp32 exponent x k log2(e) - B2 is
// off by up to |x k log2 e| 2^-24 through the rounding of k log2(e) alone,
// and by up to |B2| 2^-24 through that of the log-partition B2, which moves
// every softmax entry by as much relatively; the GRPO ratio exp(s_y - lse -
// old) suffers the same from lse, and the hardware exp2 and every fp32
// product add about an ulp each. The fp32 instances therefore take
// k log2(e), log2(e) / tau and 1 / tau in fp64 (K1d, K2d, betad), shift each
// wave by the ceiling of its exact maximum (an integer, so records merge by
// exact powers of two), sum the normalizers Z, Zt, Zs in fp64 and carry them
// as hi + lo float pairs, form the per-row coefficients in fp64 and evaluate
// each gradient element in fp64 from the fp32 inputs (and, with softcap, the
// same fp32 cap_r value pass 1 summed), rounding it once.
template <typename R>
struct CoefsT {
    R alpha;   // probability coefficient, times G k / n
    R beta;    // label-column coefficient, times G k / n
    R gam;     // forward-KL teacher coefficient, times G k / n
    R gq;      // tempered student coefficient (Hinton forward KL / FDCE)
    R rho2;    // reverse-KL log-ratio coefficient (log2 domain)
    R c0;      // reverse-KL probability coefficient
    R sB;      // pass-2 student exponent offset: -B2, or c log2(e) - B2 with softcap
    R sBd;     // tempered student offset: -Bd, or c log2(e) beta - Bd with softcap
    R sBt;     // pass-2 teacher exponent offset: -Bt2
    R cd;      // HP Hinton: the tempered exponent is aq beta + cd, cd = log2(Z) beta - log2(Zs)
};
using Coefs = CoefsT<float>;
using CoefsD = CoefsT<double>;

// All data registers are live where the fused kernel calls this, so only
// single-instruction hardware log2 / exp2 / rcp are used; the reported
// per-row values are recomputed in fp64 by the reduction from the same record.
template <int TMODE, bool SOFTCAP>
__device__ __forceinline__ Coefs row_coefs_fast(const FusedParams& p, const Rec& r, int64_t y, float xy,
                                                float old, float adv) {
    const uint32_t f = p.flags;
    const float l2Z = __builtin_amdgcn_logf(r.Z);
    Coefs k;
    const float B2 = r.M + l2Z;
    const float lse = B2 * kLn2f;
    float Bt2 = 0.f, Bd = 0.f;
    float kl = 0.f;
    if (TMODE != TM_NONE) {
        const float l2Zt = __builtin_amdgcn_logf(r.Zt);
        Bt2 = r.Mt + l2Zt;
        if (is_hinton(TMODE)) {
            const float l2Zs = __builtin_amdgcn_logf(r.Zs);
            Bd = fmaf(r.M, p.beta, l2Zs);
            if (base_mode(TMODE) == TM_RKL) kl = kLn2f * (r.SX * __builtin_amdgcn_rcpf(r.Zs) - l2Zs + l2Zt);
        } else if (TMODE == TM_RKL) {
            kl = kLn2f * (r.SX * __builtin_amdgcn_rcpf(r.Z) - l2Z + l2Zt);
        }
    }
    k.sB = SOFTCAP ? p.cl - B2 : -B2;
    k.sBd = SOFTCAP ? fmaf(p.cl, p.beta, -Bd) : -Bd;
    k.sBt = -Bt2;
    k.cd = 0.f;
    float a_g = 0.f;
    if ((f & F_GRPO) && y >= 0) {
        const float sy = SOFTCAP ? p.cap * hl_tanh(xy * p.kc) : p.k * xy;
        const float d = (sy - lse) - old;
        const float ratio = fast_exp2(d * kLog2e);
        const bool active = !((adv > 0.f && ratio > 1.f + p.eps) || (adv < 0.f && ratio < 1.f - p.eps));
        a_g = active ? adv * ratio : 0.f;
    }
    const uint32_t n_valid = p.ctrl[CTRL_NVALID];
    const float n = p.divisor > 0.f ? p.divisor : (float)n_valid;
    const float scale = p.grad_scale * p.k / n;
    float P = 0.f, L = 0.f, wd = 0.f;
    if ((f & F_CE) && p.w_ce != 0.f) { P += p.w_ce; L += p.w_ce; }
    if ((f & F_Z) && p.w_z != 0.f) P += 2.f * p.w_z * lse;
    if ((f & F_GRPO) && p.w_g != 0.f) { P += p.w_g * a_g; L += p.w_g * a_g; }
    if ((f & F_DISTILL) && p.w_d != 0.f) wd = p.w_d;
    if (fkl_like(TMODE) && !is_hinton(TMODE)) P += wd;
    k.alpha = scale * P;
    k.beta = scale * L;
    if (is_hinton(TMODE)) {
        const float wt = wd * p.tau;
        k.gam = scale * wt;
        k.gq = scale * wt;
        k.rho2 = scale * wt * kLn2f;
        k.c0 = -scale * wt * kl;
    } else {
        k.gam = scale * wd;
        k.gq = 0.f;
        k.rho2 = scale * wd * kLn2f;
        k.c0 = scale * (P - wd * kl);
    }
    return k;
}

// The fp32 instances' coefficients: the same quantities in fp64.
template <int TMODE, bool SOFTCAP>
__device__ __forceinline__ CoefsD row_coefs_hp(const FusedParams& p, const Rec& r, int64_t y, float xy,
                                               float old, float adv) {
    constexpr double LN2 = 0.69314718055994530942;
    const uint32_t f = p.flags;
    CoefsD k;
    const double l2Z = log2((double)r.Z + (double)r.Zl);
    const double B2 = (double)r.M + l2Z;
    const double lse = B2 * LN2;
    k.sB = (SOFTCAP ? (double)p.cl : 0.0) - B2;
    k.sBd = 0.0;
    k.sBt = 0.0;
    k.cd = 0.0;
    double kl = 0.0;
    if (TMODE != TM_NONE) {
        const double Ztd = (double)r.Zt + (double)r.Ztl;
        const double l2Zt = log2(Ztd);
        k.sBt = -((double)r.Mt + l2Zt);
        if (is_hinton(TMODE)) {
            const double Zsd = (double)r.Zs + (double)r.Zsl;
            const double l2Zs = log2(Zsd);
            k.cd = l2Z * p.betad - l2Zs;
            if (base_mode(TMODE) == TM_RKL) kl = LN2 * ((double)r.SX / Zsd - l2Zs + l2Zt);
        } else if (TMODE == TM_RKL) {
            kl = LN2 * ((double)r.SX / ((double)r.Z + (double)r.Zl) - l2Z + l2Zt);
        }
    }
    double a_g = 0.0;
    if ((f & F_GRPO) && y >= 0) {
        const double sy = SOFTCAP ? (double)p.cap * tanh((double)p.k * (double)xy / (double)p.cap)
                                  : (double)p.k * (double)xy;
        const double ratio = exp((sy - lse) - (double)old);
        const double eps = p.eps;
        const bool active = !((adv > 0.f && ratio > 1.0 + eps) || (adv < 0.f && ratio < 1.0 - eps));
        a_g = active ? (double)adv * ratio : 0.0;
    }
    const uint32_t n_valid = p.ctrl[CTRL_NVALID];
    const double n = p.divisor > 0.f ? (double)p.divisor : (double)n_valid;
    const double scale = (double)p.grad_scale * (double)p.k / n;
    double P = 0.0, L = 0.0, wd = 0.0;
    if ((f & F_CE) && p.w_ce != 0.f) { P += p.w_ce; L += p.w_ce; }
    if ((f & F_Z) && p.w_z != 0.f) P += 2.0 * (double)p.w_z * lse;
    if ((f & F_GRPO) && p.w_g != 0.f) { P += (double)p.w_g * a_g; L += (double)p.w_g * a_g; }
    if ((f & F_DISTILL) && p.w_d != 0.f) wd = p.w_d;
    if (fkl_like(TMODE) && !is_hinton(TMODE)) P += wd;
    k.alpha = scale * P;
    k.beta = scale * L;
    if (is_hinton(TMODE)) {
        const double wt = wd * (double)p.tau;
        k.gam = scale * wt;
        k.gq = k.gam;
        k.rho2 = scale * wt * LN2;
        k.c0 = -scale * wt * kl;
    } else {
        k.gam = scale * wd;
        k.gq = 0.0;
        k.rho2 = scale * wd * LN2;
        k.c0 = scale * (P - wd * kl);
    }
    return k;
}

template <bool HP>
using CoefsFor = typename std::conditional<HP, CoefsD, Coefs>::type;

template <int TMODE, bool SOFTCAP, bool HP>
__device__ __forceinline__ CoefsFor<HP> row_coefs(const FusedParams& p, const Rec& r, int64_t y, float xy,
                                                  float old, float adv) {
    if constexpr (HP) return row_coefs_hp<TMODE, SOFTCAP>(p, r, y, xy, old, adv);
    else return row_coefs_fast<TMODE, SOFTCAP>(p, r, y, xy, old, adv);
}


// Pass-2 constants with the probability coefficient folded into the
// exponent (the 16-bit instances outside the Hinton modes). With A the
// coefficient that multiplies q (alpha; in reverse KL rho2) and sA its sign,
// each element's gradient is sA * h, where
//   h = 2^(aq + log2|A|)                                (no teacher)
//   h = 2^(aq + log2|A|) - sA sg 2^(up + log2|gam|)     (forward KL, FDCE)
//   h = 2^(aq') (aq' - up'')                            (reverse KL)
// with aq' = aq + log2|A| and up'' = up + log2|A| - c0 / rho2, so that
// aq' - up'' = (aq - up) + c0 / rho2 and rho2 q (aq - up) + c0 q = sA h. The
// sign is applied to the packed output (one xor per two elements, skipped
// when sA = +1), so the multiply by the coefficient disappears. A zero
// coefficient folds to 2^-Inf = 0, a NaN one to NaN. ok = false (reverse KL
// with rho2 = 0 or not finite) selects the plain element path.
struct Fold {
    float sBq;       // student exponent offset + log2|A|
    float sBp;       // teacher exponent offset (+ log2|gam|, or + log2|A| - c0 / rho2)
    float m;         // forward KL / FDCE: -sA sg
    float sA;        // +1 or -1
    uint32_t flip;   // sign bits of two packed 16-bit values when sA = -1, else 0
    bool ok;
};

template <int TMODE>
__device__ __forceinline__ Fold fold_coefs(const Coefs& k) {
    Fold f;
    const float A = TMODE == TM_RKL ? k.rho2 : k.alpha;
    f.sA = A < 0.f ? -1.f : 1.f;
    f.flip = A < 0.f ? 0x80008000u : 0u;
    const float lA = __builtin_amdgcn_logf(fabsf(A));
    f.sBq = k.sB + lA;
    f.sBp = 0.f;
    f.m = 0.f;
    f.ok = true;
    if (fkl_like(TMODE)) {
        f.sBp = k.sBt + __builtin_amdgcn_logf(fabsf(k.gam));
        f.m = (k.gam < 0.f) == (A < 0.f) ? -1.f : 1.f;
    } else if (TMODE == TM_RKL) {
        f.sBp = k.sBt + lA - k.c0 / k.rho2;
        f.ok = A != 0.f && __builtin_isfinite(A) && __builtin_isfinite(f.sBp);
    }
    return f;
}

// sA times the gradient of one element that is not the label (see Fold).
template <int TMODE, bool SOFTCAP>
__device__ __forceinline__ float grad_folded(const FusedParams& p, const Fold& f, float x, float t) {
    float aq, r = 0.f;
    if (SOFTCAP) {
        r = cap_r(x, p.kc2);
        aq = fmaf(r, -2.0f * p.cl, f.sBq);
    } else {
        aq = fmaf(x, p.K1, f.sBq);
    }
    const float q = fast_exp2(aq);
    float h;
    if (TMODE == TM_NONE) h = q;
    else if (fkl_like(TMODE)) h = fmaf(f.m, fast_exp2(fmaf(t, p.K2, f.sBp)), q);
    else h = q * (aq - fmaf(t, p.K2, f.sBp));
    return SOFTCAP ? (r * fmaf(-4.0f, r, 4.0f)) * h : h;
}

// Gradient of one element; lab = the label-column coefficient at the label,
// else 0. The fp32 instances (HP) compute in fp64 and return the unrounded
// value (the caller adds the existing gradient, if any, and rounds once).
template <int TMODE, bool SOFTCAP, bool HP>
__device__ __forceinline__ typename std::conditional<HP, double, float>::type
grad_one(const FusedParams& p, const CoefsFor<HP>& k, float x, float t,
         typename std::conditional<HP, double, float>::type lab) {
    if constexpr (HP) {
        double aq, cf = 1.0;          // log2 of the student's softmax entry
        if (SOFTCAP) {
            const double r = (double)cap_r(x, p.kc2);
            aq = fma(r, -2.0 * (double)p.cl, k.sB);
            cf = r * (4.0 - 4.0 * r);
        } else {
            aq = fma((double)x, p.K1d, k.sB);
        }
        const double q = exp2_hp(aq);
        double up = 0.0;              // log2 of the teacher's softmax entry
        if (TMODE != TM_NONE) up = fma((double)t, p.K2d, k.sBt);
        double g;
        if (is_hinton(TMODE)) {
            const double aqd = fma(aq, p.betad, k.cd);
            const double qd = exp2_hp(aqd);
            if (fkl_like(TMODE)) g = k.alpha * q + k.gq * qd - k.gam * exp2_hp(up) - lab;
            else g = k.alpha * q + qd * (k.rho2 * (aqd - up) + k.c0) - lab;
        } else if (TMODE == TM_NONE) {
            g = k.alpha * q - lab;
        } else if (fkl_like(TMODE)) {
            g = k.alpha * q - k.gam * exp2_hp(up) - lab;
        } else {
            g = q * (k.rho2 * (aq - up) + k.c0) - lab;
        }
        return SOFTCAP ? cf * g : g;
    } else {
        float aq, r = 0.f, cf = 1.0f;     // aq = log2 of the student's softmax entry
        if (SOFTCAP) {
            r = cap_r(x, p.kc2);
            aq = fmaf(r, -2.0f * p.cl, k.sB);
            cf = r * fmaf(-4.0f, r, 4.0f);
        } else {
            aq = fmaf(x, p.K1, k.sB);
        }
        const float q = fast_exp2(aq);
        float up = 0.f;                   // log2 of the teacher's softmax entry
        if (TMODE != TM_NONE) up = fmaf(t, p.K2, k.sBt);
        float g;
        if (is_hinton(TMODE)) {
            const float aqd = SOFTCAP ? fmaf(r, -2.0f * p.cl * p.beta, k.sBd) : fmaf(x, p.K1 * p.beta, k.sBd);
            const float qd = fast_exp2(aqd);
            if (fkl_like(TMODE)) g = fmaf(k.alpha, q, fmaf(k.gq, qd, fmaf(-k.gam, fast_exp2(up), -lab)));
            else g = fmaf(k.alpha, q, fmaf(qd, fmaf(k.rho2, aqd - up, k.c0), -lab));
        } else if (TMODE == TM_NONE) {
            g = fmaf(k.alpha, q, -lab);
        } else if (fkl_like(TMODE)) {
            g = fmaf(k.alpha, q, fmaf(-k.gam, fast_exp2(up), -lab));
        } else {
            g = fmaf(q, fmaf(k.rho2, aq - up, k.c0), -lab);
        }
        return SOFTCAP ? cf * g : g;
    }
}

// One element's terms of the pass-1 sums, in the log2 domain, relative to
// the student shift M and the teacher shift Mt: Z += 2^a, S += 2^a a (only
// when WS: the entropy sum), Zt += 2^u, the distillation cross sum SX (and
// St = sum 2^u u, Zs = sum 2^(a / tau) in the modes that need them), with
// a = s log2(e) - M the student's and u = t log2(e) / tau - Mt the teacher's
// offset. HP (the fp32 instances): the offsets in fp64 with the fp64
// constants, the normalizer terms from the fp64 exp2, and Z, Zt, Zs
// accumulated in fp64 (A = double); S, SX, St stay fp32 sums.
template <int TMODE, bool SOFTCAP, bool WS, bool HP, typename A>
__device__ __forceinline__ void stat_term(const FusedParams& p, float M, float Mt, float x, float t, A& z,
                                          float& s, A& zt, float& sx, float& st, A& zs) {
    if constexpr (HP) {
        const double ad = SOFTCAP ? fma((double)cap_r(x, p.kc2), -2.0 * (double)p.cl, (double)p.cl - (double)M)
                                  : fma((double)x, p.K1d, -(double)M);
        const double exd = exp2_hp(ad);
        z += exd;
        const float a = (float)ad, ex = (float)exd;
        if (WS) s = fmaf(ex, a, s);
        if (TMODE != TM_NONE) {
            const double ud = fma((double)t, p.K2d, -(double)Mt);
            const double etd = exp2_hp(ud);
            zt += etd;
            const float u = (float)ud, et = (float)etd;
            if (is_hinton(TMODE)) {
                const double add = ad * p.betad;   // tempered student, shift M beta
                const double edd = exp2_hp(add);
                zs += edd;
                const float ad32 = (float)add, ed = (float)edd;
                if (fkl_like(TMODE)) sx = fmaf(et, u - ad32, sx);
                else sx = fmaf(ed, ad32 - u, sx);
            } else if (fkl_like(TMODE)) {
                sx = fmaf(et, u - a, sx);
            } else {
                sx = fmaf(ex, a - u, sx);
            }
            if (has_st(TMODE)) st = fmaf(et, u, st);
        }
    } else {
        const float a = SOFTCAP ? fmaf(cap_r(x, p.kc2), -2.0f * p.cl, p.cl - M) : fmaf(x, p.K1, -M);
        const float ex = fast_exp2(a);
        z += ex;
        if (WS) s = fmaf(ex, a, s);
        if (TMODE != TM_NONE) {
            const float u = fmaf(t, p.K2, -Mt);
            const float et = fast_exp2(u);
            zt += et;
            if (is_hinton(TMODE)) {
                const float ad = a * p.beta;          // tempered student, shift M beta
                const float ed = fast_exp2(ad);
                zs += ed;
                if (fkl_like(TMODE)) sx = fmaf(et, u - ad, sx);
                else sx = fmaf(ed, ad - u, sx);
            } else if (fkl_like(TMODE)) {
                sx = fmaf(et, u - a, sx);
            } else {
                sx = fmaf(ex, a - u, sx);
            }
            if (has_st(TMODE)) st = fmaf(et, u, st);
        }
    }
}

// ---------------------------------------------------------------------------
// fused_kernel
// ---------------------------------------------------------------------------


// Waves per SIMD the register allocation must allow (the second
// __launch_bounds__ argument): student-only slices of at most 10 vectors per
// thread (8 with softcap) are held to 64 VGPRs, i.e. 8 waves per SIMD, so that
// 32 waves (two 1024-thread or four 512-thread workgroups) share a CU; every
// other instance is held to 128 VGPRs (4 waves per SIMD), which all fit. The
// fp32 instances form their per-row coefficients in fp64 (HP) and take the
// 128-VGPR budget too.
template <typename T, int BLOCK, int NVEC, int TMODE, bool SOFTCAP>
constexpr int min_waves_per_simd() {
    return (!std::is_same<T, F32T>::value && TMODE == TM_NONE && NVEC <= (SOFTCAP ? 8 : 10)) ? 8 : 4;
}

// Slots of the slice held in LDS instead of registers: 16-bit teacher
// instances at 512 threads with slices of 9 register vectors plus up to 4
// LDS vectors per tensor (NVEC 11..13; 2 x 4 x 512 x 16 B = 64 KiB of LDS,
// so two workgroups still share a CU). A larger slice per workgroup means
// fewer chunks per row and fewer exchanges; on the V = 151936 rows that
// measured 4.5% faster for the Hinton modes (3 x 512 x 13 against
// 4 x 512 x 10) and no faster for the others, so only the Hinton modes
// instantiate them.
template <typename T, int BLOCK, int NVEC, int TMODE>
constexpr int lds_slots() {
    return (!std::is_same<T, F32T>::value && TMODE != TM_NONE && BLOCK == 512 && NVEC > 10) ? NVEC - 9 : 0;
}

template <typename T, int BLOCK, int NVEC, int TMODE, bool SOFTCAP>
__global__ __launch_bounds__(BLOCK, (min_waves_per_simd<T, BLOCK, NVEC, TMODE, SOFTCAP>()))
void fused_kernel(const FusedParams p) {
    constexpr int VEC = T::VEC;
    constexpr int ES = T::ESIZE;
    constexpr int NW = BLOCK / 64;
    constexpr bool HP = std::is_same<T, F32T>::value;   // fp32: fp64 constants, sums and coefficients
    static_assert(NW <= 16, "at most 16 waves per workgroup");
    constexpr int NL = lds_slots<T, BLOCK, NVEC, TMODE>();   // slots 0..NR-1 in registers, NR.. in LDS
    constexpr int NR = NVEC - NL;
    static_assert(NL <= 4 && NR >= 1, "slice split");

    __shared__ float s_rec[16][REC];
    __shared__ float s_fin[REC];
    __shared__ float s_xw[kMaxChunks * XWORDS];
    __shared__ float s_row[8];
    __shared__ float s_lrec[REC];
    // Accumulate mode reads the existing gradient in pass 2. Loaded slot by
    // slot next to the stores, every load would wait for the stores before
    // it as well (they share one counter); teacher instances whose slots fit
    // in 72 KiB of LDS stage the whole old slice there with direct-to-LDS
    // loads issued before the first store, one latency per workgroup.
    constexpr bool STAGE_OLD = TMODE != TM_NONE && NL == 0 && (size_t)NVEC * BLOCK * 16 <= 73728;
    __shared__ u32x4 s_old[STAGE_OLD ? NVEC : 1][STAGE_OLD ? BLOCK : 1];
    // the LDS part of the slice: [logits slots..., teacher slots...][thread]
    __shared__ u32x4 s_ext[NL > 0 ? 2 * NL : 1][NL > 0 ? BLOCK : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // Which (row, chunk) this workgroup owns. With several chunks per row the
    // chunks of one row are consecutive workgroups of one XCD: workgroups are
    // dealt to the 8 XCDs round-robin (blockIdx mod 8) and each XCD starts its
    // own in order, so XCD x takes rows [x * rows_per_xcd, ...) one row's
    // chunks after another. A workgroup then only waits for siblings that its
    // XCD starts right next to it; the wait below is bounded regardless.
    int64_t row;
    int c;
    if (p.chunks > 1) {
        const uint32_t x = blockIdx.x & 7u, k = blockIdx.x >> 3;
        const uint32_t rloc = k / (uint32_t)p.chunks;
        c = (int)(k % (uint32_t)p.chunks);
        row = (int64_t)x * p.rows_per_xcd + rloc;
        if (rloc >= (uint32_t)p.rows_per_xcd || row >= p.n_rows) return;
    } else {
        row = blockIdx.x;
        c = 0;
    }

    bool valid, bad;
    int64_t y;
    row_status(p.labels, p.mask, row, p.V, p.ctrl, valid, bad, y);

    // Row geometry: an unaligned head (< VEC elements), full 16-byte body
    // vectors, a tail (< VEC elements). Head and tail belong to chunk 0.
    const int64_t V = p.V;
    const int64_t rowoff = row * V;
    const int mis = (int)((reinterpret_cast<uintptr_t>(p.logits) + (uint64_t)rowoff * ES) & 15);
    int head = mis ? (16 - mis) / ES : 0;
    if (head > V) head = (int)V;
    const int64_t nbv = (V - head) / VEC;
    const int tail = (int)(V - head - nbv * VEC);
    const int64_t cv = (nbv + p.chunks - 1) / p.chunks;
    const int64_t vb = (int64_t)c * cv;
    int64_t ve = vb + cv;
    if (ve > nbv) ve = nbv;
    const int nv = ve > vb ? (int)(ve - vb) : 0;
    const int n_extra = (c == 0) ? head + tail : 0;
    const bool has_e = tid < n_extra;
    // row-local element index of this thread's head/tail element (rows are
    // shorter than 2^31 elements: the plan caps V far below that)
    const int eidx = (tid < head) ? tid : head + (int)nbv * VEC + (tid - head);

    const char* xrow = static_cast<const char*>(p.logits) + rowoff * ES;
    const char* trow = static_cast<const char*>(p.teacher) + rowoff * ES;
    char* grow = static_cast<char*>(p.grad) + rowoff * ES;
    const u32x4* xv = reinterpret_cast<const u32x4*>(xrow + (int64_t)head * ES) + vb;
    const u32x4* tv = reinterpret_cast<const u32x4*>(trow + (int64_t)head * ES) + vb;
    u32x4* gv = reinterpret_cast<u32x4*>(grow + (int64_t)head * ES) + vb;

    if (!valid) {
        if (p.grad != nullptr && !p.accumulate) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            for (int i = tid; i < nv; i += BLOCK) st_stream(gv + i, z);
            if (has_e) T::store1(grow, eidx, 0.0f);
        }
        if (c == 0 && tid < REC) p.row_rec[row * REC + tid] = 0.0f;
        return;
    }

    // ---- loads, in the order their values are needed ----
    // Vector loads complete in issue order, so the small loads go first and
    // are consumed only after the slice's loads are in flight: threads 0..2
    // fetch the per-row scalars (label logit, old log-prob, advantage), in
    // load mode threads 8.. the row's statistics, and the head/tail lanes
    // their element.
    uint32_t small_b = 0u;
    if (tid == 0) {
        if (y >= 0) small_b = T::raw1(xrow, y);
    } else if (tid == 1) {
        if (p.old_logprobs) small_b = __float_as_uint(p.old_logprobs[row]);
    } else if (tid == 2) {
        if (p.advantages) small_b = __float_as_uint(p.advantages[row]);
    } else if (p.load_mode && tid >= 8 && tid < 8 + REC) {
        small_b = __float_as_uint(p.row_rec[row * REC + (tid - 8)]);
    }
    uint32_t xe_b = 0u, te_b = 0u;
    if (has_e) {
        xe_b = T::raw1(xrow, eidx);
        if (TMODE != TM_NONE) te_b = T::raw1(trow, eidx);
    }

    // The slice into registers (read once). Vector v of thread tid is element
    // v * BLOCK + tid of the slice, so each wave instruction covers 1 KiB of
    // consecutive bytes.
    //
    // With a teacher every slot is loaded, without a branch (a skipped load
    // would leave the compiler unable to wait for the first vectors alone), so
    // that pass 1 starts on the first vectors while later ones are still
    // arriving: a slot past the slice re-reads the slice's own last vector
    // (the lanes of one instruction that share it make one request, and no
    // byte outside the slice is fetched) and its value is never used; an
    // empty slice points the loads at the workspace's row records. A
    // student-only slice loads only its own slots and starts once all have
    // arrived: timed on the student rows, the extra requests and the earlier
    // start were each about 1% slower, while on the teacher rows the early
    // start is 5-8% faster.
    u32x4 xs[NR];
    u32x4 ts[TMODE != TM_NONE ? NR : 1];
    if (TMODE == TM_NONE) {
#pragma unroll
        for (int v = 0; v < NR; ++v)
            if (tid < nv - v * BLOCK) xs[v] = ld_stream(xv + v * BLOCK + tid);
    } else {
        const bool body = nv > 0;
        const u32x4* xb = body ? xv : reinterpret_cast<const u32x4*>(p.row_rec);
        const u32x4* tb = body ? tv : reinterpret_cast<const u32x4*>(p.row_rec);
        const int lastv = body ? nv - 1 : 0;
#pragma unroll
        for (int v = 0; v < NR; ++v) {
            int i = v * BLOCK + tid;
            i = i < lastv ? i : lastv;
            xs[v] = ld_stream(xb + i);
            ts[v] = ld_stream(tb + i);
        }
        // LDS slots: direct-to-LDS loads after the register slots (each
        // wave fills its own 64 x 16 B of every slot row, in lane order, and
        // later reads back only its own lanes)
#pragma unroll
        for (int v = NR; v < NVEC; ++v) {
            int i = v * BLOCK + tid;
            i = i < lastv ? i : lastv;
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(xb + i),
                                             (__attribute__((address_space(3))) void*)&s_ext[v - NR][wave * 64],
                                             16, 0, 2);
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(tb + i),
                                             (__attribute__((address_space(3))) void*)&s_ext[NL + v - NR][wave * 64],
                                             16, 0, 2);
        }
    }
    // slot v of this thread: registers, or (after lds_ready) LDS
    auto slot_x = [&](int v) -> u32x4 { return v < NR ? xs[v < NR ? v : 0] : s_ext[v >= NR ? v - NR : 0][tid]; };
    auto slot_t = [&](int v) -> u32x4 {
        if constexpr (TMODE == TM_NONE) return xs[0];
        else return v < NR ? ts[v < NR ? v : 0] : s_ext[NL + (v >= NR ? v - NR : 0)][tid];
    };
    // the LDS slots have landed once this wave's vector loads are done
    auto lds_ready = [&]() {
        if constexpr (NL > 0) {
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt unconstrained
            asm volatile("" ::: "memory");
        }
    };
    if (tid < 3) s_row[tid] = tid == 0 ? T::from_raw(small_b) : __uint_as_float(small_b);
    if (p.load_mode && tid >= 8 && tid < 8 + REC) s_lrec[tid - 8] = __uint_as_float(small_b);
    const float xe = has_e ? T::from_raw(xe_b) : 0.f;
    const float te = (has_e && TMODE != TM_NONE) ? T::from_raw(te_b) : 0.f;

    Rec r;
    if (p.load_mode) {
        // Load mode (the backward of a two-launch call): the row's statistics
        // are final already, in the record the forward launch wrote; only the
        // slice is needed again, for pass 2.
        __syncthreads();   // s_row and s_lrec, written above
        r.M = s_lrec[R_M]; r.Z = s_lrec[R_Z]; r.S = s_lrec[R_S];
        r.Mt = s_lrec[R_MT]; r.Zt = s_lrec[R_ZT]; r.SX = s_lrec[R_SX]; r.St = s_lrec[R_ST];
        r.Zs = s_lrec[R_ZS];
        r.Zl = s_lrec[R_ZL]; r.Ztl = s_lrec[R_ZTL]; r.Zsl = s_lrec[R_ZSL];
    } else {
    // ---- pass 1: sums relative to a provisional wave shift, log2 domain ----
    // The shift is the wave's maximum over its first vector, not the row
    // maximum: any shift gives the same statistics once records are merged
    // with rescaling, and this one needs no separate pass over the slice.
    // If some term could overflow (the wave's sum exceeds 2^64, i.e. an
    // element lies more than 64 above the shift; the sum is also non-finite
    // for Inf or NaN inputs) or the wave holds no element of its first
    // vector, the wave takes the true maximum and sums again. The entropy sum
    // S is formed only when the entropy metric is requested.
    float mx = kNegInf, mt = kNegInf;
    if (HP) {
        // fp32: the wave's exact maxima (its largest elements then sit at
        // offset ~0, where the fp32 offsets are exact)
#pragma unroll
        for (int v = 0; v < NR; ++v) {   // (no LDS slots in the fp32 instances)
            if (tid < nv - v * BLOCK) {
                mx = T::vmax(mx, xs[v]);
                if (TMODE != TM_NONE) mt = T::vmax(mt, ts[v]);
            }
        }
        if (has_e) {
            mx = fmaxf(mx, xe);
            if (TMODE != TM_NONE) mt = fmaxf(mt, te);
        }
    } else if (tid < nv) {
        mx = T::vmax(mx, xs[0]);
        if (TMODE != TM_NONE) mt = T::vmax(mt, ts[0]);
    }
    const float mx0 = wave_max(mx);
    const float mt0 = TMODE != TM_NONE ? wave_max(mt) : 0.f;
    auto shift_of = [&](float m) -> float {
        return shift_int<HP>(SOFTCAP ? (p.cap * hl_tanh(m * p.kc)) * kLog2e : m * p.K1);
    };
    float M = shift_of(mx0);
    float Mt = TMODE != TM_NONE ? shift_int<HP>(mt0 * p.K2) : 0.f;
    const bool early = mx0 != kNegInf && (TMODE == TM_NONE || mt0 != kNegInf);
    const bool want_s = (p.flags & F_ENT) != 0u;

    // normalizer accumulators: fp64 in the fp32 instances
    using Acc = typename std::conditional<HP, double, float>::type;
    float Z = 0.f, S = 0.f, Zt = 0.f, SX = 0.f, St = 0.f, Zs = 0.f;
    float Zl = 0.f, Ztl = 0.f, Zsl = 0.f;
    // one term of every sum; the entropy term only when WS
    auto term = [&](auto want_s_tag, float x, float t, Acc& z, float& s, Acc& zt, float& sx, float& st,
                    Acc& zs) {
        stat_term<TMODE, SOFTCAP, decltype(want_s_tag)::value, HP>(p, M, Mt, x, t, z, s, zt, sx, st, zs);
    };
    auto accumulate = [&](float x, float t, Acc& z, float& s, Acc& zt, float& sx, float& st, Acc& zs) {
        term(std::true_type(), x, t, z, s, zt, sx, st, zs);
    };
    auto wave_sums = [&](bool ws, Acc z0, float s0, Acc zt0, float sx0, float st0, Acc zs0) {
        if constexpr (HP) {
            split_hl(wave_sum_d(z0), Z, Zl);
            if (TMODE != TM_NONE) split_hl(wave_sum_d(zt0), Zt, Ztl);
            if (is_hinton(TMODE)) split_hl(wave_sum_d(zs0), Zs, Zsl);
        } else {
            Z = wave_sum(z0);
            if (TMODE != TM_NONE) Zt = wave_sum(zt0);
            if (is_hinton(TMODE)) Zs = wave_sum(zs0);
        }
        if (ws) S = wave_sum(s0);
        if (TMODE != TM_NONE) SX = wave_sum(sx0);
        if (has_st(TMODE)) St = wave_sum(st0);
    };
    // one call site per variant (below), so the slice stays in registers
    auto sweep = [&](auto want_s_tag) __attribute__((always_inline)) {
        constexpr bool WS = decltype(want_s_tag)::value;
        auto acc = [&](float x, float t, Acc& z, float& s, Acc& zt, float& sx, float& st, Acc& zs) {
            term(want_s_tag, x, t, z, s, zt, sx, st, zs);
        };
        Acc z0 = 0, zt0 = 0, zs0 = 0;
        float s0 = 0.f, sx0 = 0.f, st0 = 0.f;
#pragma unroll
        for (int v = 0; v < NVEC; ++v) {
            if (v == NR) lds_ready();
            if (tid < nv - v * BLOCK) {
                const u32x4 xw = slot_x(v), tw = slot_t(v);
                if constexpr (HP) {
                    // fp64 sums: straight into the thread's totals
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        acc(T::get(xw, e), TMODE != TM_NONE ? T::get(tw, e) : 0.f, z0, s0, zt0, sx0, st0, zs0);
                } else {
                    Acc z = 0, zt = 0, zs = 0;
                    float s = 0.f, sx = 0.f, st = 0.f;
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        acc(T::get(xw, e), TMODE != TM_NONE ? T::get(tw, e) : 0.f, z, s, zt, sx, st, zs);
                    z0 += z; s0 += s; zt0 += zt; sx0 += sx; st0 += st; zs0 += zs;
                }
            }
        }
        if (has_e) acc(xe, te, z0, s0, zt0, sx0, st0, zs0);
        wave_sums(WS, z0, s0, zt0, sx0, st0, zs0);
    };
    if (early) {
        if (want_s) sweep(std::true_type());
        else sweep(std::false_type());
    }
    constexpr float kSumLimit = 18446744073709551616.0f;   // 2^64
    if (!early || !(Z <= kSumLimit) || (TMODE != TM_NONE && !(Zt <= kSumLimit)) ||
        (is_hinton(TMODE) && !(Zs <= kSumLimit))) {
        // Rare: the true maximum, then the sums from it. This path reads the
        // slice again from memory so that the register copy keeps a single
        // use above (the slice must not be spilled to make room for a second).
        mx = kNegInf;
        mt = kNegInf;
        for (int i = tid; i < nv; i += BLOCK) {
            mx = T::vmax(mx, xv[i]);
            if (TMODE != TM_NONE) mt = T::vmax(mt, tv[i]);
        }
        if (has_e) {
            mx = fmaxf(mx, xe);
            if (TMODE != TM_NONE) mt = fmaxf(mt, te);
        }
        M = shift_of(wave_max(mx));
        if (TMODE != TM_NONE) Mt = shift_int<HP>(wave_max(mt) * p.K2);
        Acc z0 = 0, zt0 = 0, zs0 = 0;
        float s0 = 0.f, sx0 = 0.f, st0 = 0.f;
        for (int i = tid; i < nv; i += BLOCK) {
            const u32x4 w = xv[i];
            u32x4 wt = {0u, 0u, 0u, 0u};
            if (TMODE != TM_NONE) wt = tv[i];
            for (int e = 0; e < VEC; ++e)
                accumulate(T::get(w, e), TMODE != TM_NONE ? T::get(wt, e) : 0.f, z0, s0, zt0, sx0, st0, zs0);
        }
        if (has_e) accumulate(xe, te, z0, s0, zt0, sx0, st0, zs0);
        wave_sums(true, z0, s0, zt0, sx0, st0, zs0);
    }
    if (lane == 0) {
        s_rec[wave][0] = M;
        s_rec[wave][1] = Z;
        s_rec[wave][2] = S;
        s_rec[wave][3] = Mt;
        s_rec[wave][4] = Zt;
        s_rec[wave][5] = SX;
        s_rec[wave][6] = St;
        s_rec[wave][7] = Zs;
        if (HP) {
            s_rec[wave][8] = Zl;
            s_rec[wave][9] = Ztl;
            s_rec[wave][10] = Zsl;
        }
    }
    __syncthreads();

    // ---- combine the waves' records, then (split-vocab) the chunks' ----
    // Wave 0 alone merges (the other waves wait at the barrier below, so
    // their SIMDs are free for the other workgroups of the CU) and leaves the
    // row's final statistics in shared memory.
    //
    // Split-vocab exchange: each statistic travels as one 64-bit atomic word,
    // its float bits and the call's epoch (bumped by the count kernel before
    // this kernel starts). A sibling's word is taken once it carries the
    // current epoch, so nothing depends on the order in which different
    // words become visible, and no L2 write-back or invalidate is needed.
    // Wave 0 polls all C x words in one load per lane per round, then merges
    // the C records with the same fixed DPP tree in every workgroup of the row.
    if (wave == 0) {
        Rec wr = rec_empty();
        {
            const int w = lane & 15;
            if (w < NW) {
                wr.M = s_rec[w][0];
                wr.Z = s_rec[w][1];
                wr.S = s_rec[w][2];
                if (TMODE != TM_NONE) {
                    wr.Mt = s_rec[w][3];
                    wr.Zt = s_rec[w][4];
                    wr.SX = s_rec[w][5];
                    if (has_st(TMODE)) wr.St = s_rec[w][6];
                    if (is_hinton(TMODE)) wr.Zs = s_rec[w][7];
                }
                if (HP) {
                    wr.Zl = s_rec[w][8];
                    if (TMODE != TM_NONE) wr.Ztl = s_rec[w][9];
                    if (is_hinton(TMODE)) wr.Zsl = s_rec[w][10];
                }
                if (wr.Z == 0.f) wr = rec_empty();
            }
            wr = rec_reduce16<TMODE, HP>(wr, p.beta, NW, p.betad);
        }
        if (p.chunks > 1) {
            // statistics this mode exchanges: M, Z, S (+ Mt, Zt, SX (+ St) (+ Zs)),
            // packed in that order, then (fp32 instances) Zl (+ Ztl (+ Zsl))
            constexpr int NX0 = xwords_used(TMODE);
            constexpr int NXW = xwords_used(TMODE, HP);
            constexpr int XS = xwords_stride(HP);
            constexpr int POS_ZS = has_st(TMODE) ? 7 : 6;
            const uint64_t epoch = (uint64_t)p.ctrl[CTRL_EPOCH] << 32;
            const uint32_t spin_limit = p.ctrl[CTRL_SPIN];
            const bool held = (uint32_t)row == p.ctrl[CTRL_HOLD_ROW] && (uint32_t)c == p.ctrl[CTRL_HOLD_CHUNK];
            uint64_t* words = p.chunk_words + (int64_t)row * p.chunks * XS;
            uint64_t* mine = words + c * XS;
            if (lane == 0 && !held) {
                float f[XS] = {wr.M, wr.Z, wr.S, wr.Mt, wr.Zt, wr.SX, has_st(TMODE) ? wr.St : wr.Zs, wr.Zs};
                if (HP) {
                    f[NX0] = wr.Zl;
                    if (TMODE != TM_NONE) f[NX0 + 1] = wr.Ztl;
                    if (is_hinton(TMODE)) f[NX0 + 2] = wr.Zsl;
                }
#pragma unroll
                for (int i = 0; i < NXW; ++i)
                    __hip_atomic_store(mine + i, epoch | __float_as_uint(f[i]), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            // lane l polls word (l % NXW) of chunk (l / NXW)
            const int nwords = p.chunks * NXW;
            const int lw = (lane / NXW) * XS + lane % NXW;
            // Polls are device-scope loads that travel to memory and take
            // microseconds under a full memory pipe; a pause of 32 x 64 clocks
            // between them measured 1.2% faster on the teacher rows than back-
            // to-back polls (fewer of them compete with the slice traffic),
            // while several polls in flight measured 9% slower.
            uint64_t w = 0;
            uint32_t spins = 0;
            bool gave_up = false;
            while (true) {
                if (lane < nwords) w = __hip_atomic_load(words + lw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const bool ok = (lane >= nwords) || ((w & 0xffffffff00000000ull) == epoch);
                if (__all(ok)) break;
                __builtin_amdgcn_s_sleep(32);
                if (++spins > spin_limit) {
                    gave_up = true;
                    break;
                }
            }
            if (gave_up) {
                // A sibling never published: this chunk's statistics become NaN
                // (so its gradient slice and, for chunk 0, the row record are
                // NaN), its words are republished as NaN for any sibling still
                // polling, and the error word makes every scalar NaN.
                if (lane == 0)
                    __hip_atomic_store(&p.ctrl[CTRL_ERROR], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (lane < NXW)
                    __hip_atomic_store(mine + lane, epoch | 0x7fc00000ull, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                w = epoch | 0x7fc00000ull;
            }
            if (lane < nwords) s_xw[lane] = __uint_as_float((uint32_t)w);
            // lane l of every 16-lane row holds chunk l's record (empty beyond C)
            const int l = lane & 15;
            Rec cr = rec_empty();
            if (l < p.chunks) {
                cr.M = s_xw[l * NXW + 0]; cr.Z = s_xw[l * NXW + 1]; cr.S = s_xw[l * NXW + 2];
                if (TMODE != TM_NONE) {
                    cr.Mt = s_xw[l * NXW + 3]; cr.Zt = s_xw[l * NXW + 4]; cr.SX = s_xw[l * NXW + 5];
                    if (has_st(TMODE)) cr.St = s_xw[l * NXW + 6];
                    if (is_hinton(TMODE)) cr.Zs = s_xw[l * NXW + POS_ZS];
                }
                if (HP) {
                    cr.Zl = s_xw[l * NXW + NX0];
                    if (TMODE != TM_NONE) cr.Ztl = s_xw[l * NXW + NX0 + 1];
                    if (is_hinton(TMODE)) cr.Zsl = s_xw[l * NXW + NX0 + 2];
                }
                if (cr.Z == 0.f) cr = rec_empty();
            }
            wr = rec_reduce16<TMODE, HP>(cr, p.beta, p.chunks, p.betad);
        }
        if (lane == 0) {
            s_fin[0] = wr.M; s_fin[1] = wr.Z; s_fin[2] = wr.S;
            s_fin[3] = wr.Mt; s_fin[4] = wr.Zt; s_fin[5] = wr.SX; s_fin[6] = wr.St;
            s_fin[7] = wr.Zs;
            if (HP) {
                s_fin[8] = wr.Zl; s_fin[9] = wr.Ztl; s_fin[10] = wr.Zsl;
            }
            // per-row record for the batch reduction (s_row[0] was written by
            // this thread)
            if (c == 0) {
                float* out = p.row_rec + row * REC;
                out[R_M] = wr.M; out[R_Z] = wr.Z; out[R_S] = wr.S;
                out[R_MT] = wr.Mt; out[R_ZT] = wr.Zt; out[R_SX] = wr.SX; out[R_ST] = wr.St;
                out[R_ZS] = wr.Zs;
                out[R_XY] = s_row[0];
                out[R_VALID] = 1.0f;
                out[R_ZL] = HP ? wr.Zl : 0.f;
                out[R_ZTL] = HP ? wr.Ztl : 0.f;
                out[R_ZSL] = HP ? wr.Zsl : 0.f;
            }
        }
    }
    __syncthreads();
    r.M = s_fin[0]; r.Z = s_fin[1]; r.S = s_fin[2];
    r.Mt = s_fin[3]; r.Zt = s_fin[4]; r.SX = s_fin[5]; r.St = s_fin[6]; r.Zs = s_fin[7];
    r.Zl = 0.f; r.Ztl = 0.f; r.Zsl = 0.f;
    if (HP) {
        r.Zl = s_fin[8]; r.Ztl = s_fin[9]; r.Zsl = s_fin[10];
    }
    }   // pass 1
    if (p.grad == nullptr) return;

    // ---- gradient coefficients (every thread; fp64 in the fp32 instances) ----
    using CT = typename std::conditional<HP, double, float>::type;
    CoefsFor<HP> kf = row_coefs<TMODE, SOFTCAP, HP>(p, r, y, s_row[0], s_row[1], s_row[2]);
    if (p.row_coef != nullptr && p.w_g != 0.f) {
        // GSPO: d(loss)/d(logp_t) = -coef_t / n_seg; d logp_t / d s_j = [j == y] - q_j
        const uint32_t n_seg = p.ctrl[CTRL_NSEG];
        const CT e = n_seg > 0u ? (CT)p.grad_scale * (CT)p.k * (CT)p.w_g * (CT)p.row_coef[row] / (CT)n_seg
                                : (CT)0;
        kf.alpha += e;
        kf.beta += e;
        if (TMODE == TM_RKL) kf.c0 += e;   // there c0 multiplies q (alpha is unused); in the
                                           // Hinton reverse KL it multiplies the tempered q
    }
    if (p.load_mode && p.ctrl[CTRL_ERROR] != 0u) {
        // statistics or segments are not trustworthy: make the gradient say so
        kf.alpha = kf.beta = kf.c0 = (CT)__builtin_nanf("");
    }
    auto grad_elem = [&](float x, float t, CT lab) -> CT {
        return grad_one<TMODE, SOFTCAP, HP>(p, kf, x, t, lab);
    };
    const CT beta = kf.beta;

    if (STAGE_OLD && p.accumulate && nv > 0) {
        // slots past the slice re-read its last vector (in bounds, unused)
        const char* gc = reinterpret_cast<const char*>(gv);
#pragma unroll
        for (int v = 0; v < NVEC; ++v) {
            int i = v * BLOCK + tid;
            i = i < nv - 1 ? i : nv - 1;
            __builtin_amdgcn_global_load_lds(static_cast<const void*>(gc + (int64_t)i * 16),
                                             (__attribute__((address_space(3))) void*)&s_old[v][wave * 64],
                                             16, 0, 2);
        }
        // wait here, once, for the staged slice (no store is outstanding yet)
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt unconstrained
    }

    // label position relative to this chunk's body vectors (-1: not here)
    int yv = -1;
    int ly = 0;
    if (y >= head + vb * VEC && y < head + ve * VEC) {
        yv = (int)((y - head) / VEC - vb);
        ly = (int)((y - head) % VEC);
    }

    // Folded path (see Fold): every 16-bit instance outside the Hinton modes;
    // the reverse-KL ones fall back to the plain path when rho2 = 0. A
    // non-finite coefficient (the poisoned load-mode call) folds to NaN.
    constexpr bool FOLD = !HP && !is_hinton(TMODE);
    constexpr bool FOLD_ONLY = FOLD && TMODE != TM_RKL;
    Fold fd{};
    if constexpr (FOLD) fd = fold_coefs<TMODE>(kf);
    auto folded_pass = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < NVEC; ++v) {
            if (tid < nv - v * BLOCK) {
                const u32x4 xw = slot_x(v), tw = slot_t(v);
                float g[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    g[e] = grad_folded<TMODE, SOFTCAP>(p, fd, T::get(xw, e), TMODE != TM_NONE ? T::get(tw, e) : 0.f);
                if (tid == yv - v * BLOCK) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        if (e == ly)
                            g[e] = fd.sA * (float)grad_elem(T::get(xw, e), TMODE != TM_NONE ? T::get(tw, e) : 0.f,
                                                            beta);
                }
                u32x4 out;
                if (p.accumulate) {
                    const u32x4 old = STAGE_OLD ? s_old[v][tid] : ld_stream(gv + v * BLOCK + tid);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) g[e] = fmaf(fd.sA, g[e], T::get(old, e));
                    out = T::pack(g);
                } else {
                    out = T::pack(g);
                    if (fd.flip) {
#pragma unroll
                        for (int c = 0; c < 4; ++c) out[c] ^= fd.flip;
                    }
                }
                st_stream(gv + v * BLOCK + tid, out);
            }
        }
    };
    auto plain_pass = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < NVEC; ++v) {
        if (tid < nv - v * BLOCK) {
            const u32x4 xw = slot_x(v), tw = slot_t(v);
            CT gd[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                gd[e] = grad_elem(T::get(xw, e), TMODE != TM_NONE ? T::get(tw, e) : 0.f, (CT)0);
            if (tid == yv - v * BLOCK) {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    if (e == ly)
                        gd[e] = grad_elem(T::get(xw, e), TMODE != TM_NONE ? T::get(tw, e) : 0.f, beta);
            }
            if (p.accumulate) {
                const u32x4 old = STAGE_OLD ? s_old[v][tid] : ld_stream(gv + v * BLOCK + tid);
#pragma unroll
                for (int e = 0; e < VEC; ++e) gd[e] = (CT)T::get(old, e) + gd[e];
            }
            float g[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) g[e] = (float)gd[e];   // the one rounding
            st_stream(gv + v * BLOCK + tid, T::pack(g));
        }
    }
    };
    lds_ready();   // load mode skips pass 1
    if constexpr (FOLD_ONLY) {
        folded_pass();
    } else if constexpr (FOLD) {
        if (fd.ok) folded_pass();
        else plain_pass();
    } else {
        plain_pass();
    }
    if (has_e) {
        CT g = grad_elem(xe, te, (int64_t)eidx == y ? beta : (CT)0);
        if (p.accumulate) g = (CT)T::load1(grow, eidx) + g;
        T::store1(grow, eidx, (float)g);
    }
}

template <typename T, int BLOCK, int NVEC, int TMODE, bool SOFTCAP>
hipError_t launch_fused(const FusedParams& p, dim3 grid, hipStream_t s) {
    (void)hipGetLastError();   // drop an error left by an earlier, unrelated call
    hipLaunchKernelGGL((fused_kernel<T, BLOCK, NVEC, TMODE, SOFTCAP>), grid, dim3(BLOCK), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// rowwise_kernel: the same losses, row records and gradient for inputs whose
// base addresses differ modulo 16 bytes, where no split of a row into 16-byte
// vectors is aligned in all of logits, teacher and gradient at once. One
// 256-thread workgroup per row with element loads and stores; the row is read
// three times (exact maxima, sums, gradient). The statistics are taken
// relative to the exact row maxima, merged over the waves in wave order; the
// coefficients and the per-element gradient are the fused kernel's.
// ---------------------------------------------------------------------------
template <typename T, int TMODE, bool SOFTCAP>
__global__ __launch_bounds__(kRowwiseBlock) void rowwise_kernel(const FusedParams p) {
    constexpr int NW = kRowwiseBlock / 64;
    constexpr int ES = T::ESIZE;
    constexpr bool HP = std::is_same<T, F32T>::value;
    __shared__ float s_m[NW][2];
    __shared__ float s_rec[NW][11];
    __shared__ float s_fin[11];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t row = blockIdx.x;
    const int64_t V = p.V;

    bool valid, bad;
    int64_t y;
    row_status(p.labels, p.mask, row, V, p.ctrl, valid, bad, y);
    const char* xrow = static_cast<const char*>(p.logits) + row * V * ES;
    const char* trow = TMODE != TM_NONE ? static_cast<const char*>(p.teacher) + row * V * ES : nullptr;
    char* grow = p.grad != nullptr ? static_cast<char*>(p.grad) + row * V * ES : nullptr;
    if (!valid) {
        if (grow != nullptr && !p.accumulate)
            for (int64_t j = tid; j < V; j += kRowwiseBlock) T::store1(grow, j, 0.0f);
        if (tid < REC) p.row_rec[row * REC + tid] = 0.0f;
        return;
    }
    const float xy = y >= 0 ? T::load1(xrow, y) : 0.f;
    const float old = p.old_logprobs != nullptr ? p.old_logprobs[row] : 0.f;
    const float adv = p.advantages != nullptr ? p.advantages[row] : 0.f;

    Rec r;
    if (p.load_mode) {
        const float* rec = p.row_rec + row * REC;
        r.M = rec[R_M]; r.Z = rec[R_Z]; r.S = rec[R_S];
        r.Mt = rec[R_MT]; r.Zt = rec[R_ZT]; r.SX = rec[R_SX]; r.St = rec[R_ST]; r.Zs = rec[R_ZS];
        r.Zl = rec[R_ZL]; r.Ztl = rec[R_ZTL]; r.Zsl = rec[R_ZSL];
    } else {
        float mx = kNegInf, mt = kNegInf;
        for (int64_t j = tid; j < V; j += kRowwiseBlock) {
            mx = fmaxf(mx, T::load1(xrow, j));
            if (TMODE != TM_NONE) mt = fmaxf(mt, T::load1(trow, j));
        }
        mx = wave_max(mx);
        if (TMODE != TM_NONE) mt = wave_max(mt);
        if (lane == 0) {
            s_m[wave][0] = mx;
            s_m[wave][1] = mt;
        }
        __syncthreads();
        mx = s_m[0][0];
        mt = s_m[0][1];
        for (int w = 1; w < NW; ++w) {
            mx = fmaxf(mx, s_m[w][0]);
            mt = fmaxf(mt, s_m[w][1]);
        }
        const float M = shift_int<HP>(SOFTCAP ? (p.cap * hl_tanh(mx * p.kc)) * kLog2e : mx * p.K1);
        const float Mt = TMODE != TM_NONE ? shift_int<HP>(mt * p.K2) : 0.f;
        using Acc = typename std::conditional<HP, double, float>::type;
        Acc z = 0, zt = 0, zs = 0;
        float sv = 0.f, sx = 0.f, st = 0.f;
        for (int64_t j = tid; j < V; j += kRowwiseBlock) {
            const float x = T::load1(xrow, j);
            const float t = TMODE != TM_NONE ? T::load1(trow, j) : 0.f;
            stat_term<TMODE, SOFTCAP, true, HP>(p, M, Mt, x, t, z, sv, zt, sx, st, zs);
        }
        float zh = 0.f, zl = 0.f, zth = 0.f, ztl = 0.f, zsh = 0.f, zsl = 0.f;
        if constexpr (HP) {
            split_hl(wave_sum_d(z), zh, zl);
            if (TMODE != TM_NONE) split_hl(wave_sum_d(zt), zth, ztl);
            if (is_hinton(TMODE)) split_hl(wave_sum_d(zs), zsh, zsl);
        } else {
            zh = wave_sum(z);
            if (TMODE != TM_NONE) zth = wave_sum(zt);
            if (is_hinton(TMODE)) zsh = wave_sum(zs);
        }
        sv = wave_sum(sv);
        if (TMODE != TM_NONE) sx = wave_sum(sx);
        if (has_st(TMODE)) st = wave_sum(st);
        if (lane == 0) {
            s_rec[wave][0] = M; s_rec[wave][1] = zh; s_rec[wave][2] = sv; s_rec[wave][3] = Mt;
            s_rec[wave][4] = zth; s_rec[wave][5] = sx; s_rec[wave][6] = st; s_rec[wave][7] = zsh;
            s_rec[wave][8] = zl; s_rec[wave][9] = ztl; s_rec[wave][10] = zsl;
        }
        __syncthreads();
        if (tid == 0) {
            Rec acc = rec_empty();
            for (int w = 0; w < NW; ++w) {
                Rec b;
                b.M = s_rec[w][0]; b.Z = s_rec[w][1]; b.S = s_rec[w][2];
                if (TMODE != TM_NONE) {
                    b.Mt = s_rec[w][3]; b.Zt = s_rec[w][4]; b.SX = s_rec[w][5];
                    b.St = has_st(TMODE) ? s_rec[w][6] : 0.f;
                    b.Zs = is_hinton(TMODE) ? s_rec[w][7] : 0.f;
                } else {
                    b.Mt = 0.f; b.Zt = 0.f; b.SX = 0.f; b.St = 0.f; b.Zs = 0.f;
                }
                b.Zl = s_rec[w][8]; b.Ztl = s_rec[w][9]; b.Zsl = s_rec[w][10];
                if (b.Z == 0.f) b = rec_empty();
                acc = rec_merge<TMODE, HP>(acc, b, p.beta, p.betad);
            }
            s_fin[0] = acc.M; s_fin[1] = acc.Z; s_fin[2] = acc.S; s_fin[3] = acc.Mt;
            s_fin[4] = acc.Zt; s_fin[5] = acc.SX; s_fin[6] = acc.St; s_fin[7] = acc.Zs;
            s_fin[8] = acc.Zl; s_fin[9] = acc.Ztl; s_fin[10] = acc.Zsl;
            float* out = p.row_rec + row * REC;
            out[R_M] = acc.M; out[R_Z] = acc.Z; out[R_S] = acc.S;
            out[R_MT] = acc.Mt; out[R_ZT] = acc.Zt; out[R_SX] = acc.SX; out[R_ST] = acc.St;
            out[R_ZS] = acc.Zs;
            out[R_XY] = xy;
            out[R_VALID] = 1.0f;
            out[R_ZL] = acc.Zl; out[R_ZTL] = acc.Ztl; out[R_ZSL] = acc.Zsl;
        }
        __syncthreads();
        r.M = s_fin[0]; r.Z = s_fin[1]; r.S = s_fin[2]; r.Mt = s_fin[3];
        r.Zt = s_fin[4]; r.SX = s_fin[5]; r.St = s_fin[6]; r.Zs = s_fin[7];
        r.Zl = s_fin[8]; r.Ztl = s_fin[9]; r.Zsl = s_fin[10];
    }
    if (grow == nullptr) return;

    using CT = typename std::conditional<HP, double, float>::type;
    CoefsFor<HP> kf = row_coefs<TMODE, SOFTCAP, HP>(p, r, y, xy, old, adv);
    if (p.row_coef != nullptr && p.w_g != 0.f) {
        // GSPO: the per-token coefficient of the segment step on the label column
        const uint32_t n_seg = p.ctrl[CTRL_NSEG];
        const CT e = n_seg > 0u ? (CT)p.grad_scale * (CT)p.k * (CT)p.w_g * (CT)p.row_coef[row] / (CT)n_seg
                                : (CT)0;
        kf.alpha += e;
        kf.beta += e;
        if (TMODE == TM_RKL) kf.c0 += e;
    }
    if (p.load_mode && p.ctrl[CTRL_ERROR] != 0u) kf.alpha = kf.beta = kf.c0 = (CT)__builtin_nanf("");
    for (int64_t j = tid; j < V; j += kRowwiseBlock) {
        const float x = T::load1(xrow, j);
        const float t = TMODE != TM_NONE ? T::load1(trow, j) : 0.f;
        CT g = grad_one<TMODE, SOFTCAP, HP>(p, kf, x, t, j == y ? kf.beta : (CT)0);
        if (p.accumulate) g = (CT)T::load1(grow, j) + g;
        T::store1(grow, j, (float)g);
    }
}

template <typename T, int TMODE, bool SOFTCAP>
hipError_t launch_rowwise(const FusedParams& p, dim3 grid, hipStream_t s) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((rowwise_kernel<T, TMODE, SOFTCAP>), grid, dim3(kRowwiseBlock), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// stream_stats_kernel: the forward-only pass (row statistics and records, no
// gradient), used when no gradient is requested and for the forward launch
// of a GSPO call. Nothing of the row is needed after its sums, so instead of
// holding a register-resident slice per (row, chunk) this kernel gives each
// row one workgroup that streams it in batches of SU 16-byte vectors per
// thread and tensor, the next batch's loads in flight while the
// current one is summed: no chunk exchange, one read of every byte. The sums
// use the wave's provisional shift (the maximum of its first vectors) with
// the fused kernel's overflow fallback; records merge over the waves in
// order. Same record format as the fused kernel.
// ---------------------------------------------------------------------------
// Batches of 4 vectors (2 per tensor with a teacher) keep two double-buffered
// batches within 64 VGPRs, so two 1024-thread workgroups share a CU (the fp32
// instances, whose normalizer sums run in fp64, take 128 VGPRs and one).
constexpr int kStreamBlock = 1024;

template <typename T, int TMODE, bool SOFTCAP>
__global__ __launch_bounds__(kStreamBlock, (std::is_same<T, F32T>::value ? 4 : 8)) void stream_stats_kernel(
    const FusedParams p) {
    constexpr int VEC = T::VEC;
    constexpr int ES = T::ESIZE;
    constexpr int NW = kStreamBlock / 64;
    constexpr int SU = TMODE == TM_NONE ? 4 : 2;
    constexpr bool HP = std::is_same<T, F32T>::value;
    __shared__ float s_rec[16][11];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t row = blockIdx.x;
    const int64_t V = p.V;

    bool valid, bad;
    int64_t y;
    row_status(p.labels, p.mask, row, V, p.ctrl, valid, bad, y);
    if (!valid) {
        if (tid < REC) p.row_rec[row * REC + tid] = 0.0f;
        return;
    }
    // the fused kernel's row geometry (head, 16-byte body vectors, tail)
    const int64_t rowoff = row * V;
    const int mis = (int)((reinterpret_cast<uintptr_t>(p.logits) + (uint64_t)rowoff * ES) & 15);
    int head = mis ? (16 - mis) / ES : 0;
    if (head > V) head = (int)V;
    const int64_t nbv = (V - head) / VEC;
    const int tail = (int)(V - head - nbv * VEC);
    const bool has_e = tid < head + tail;
    const int eidx = (tid < head) ? tid : head + (int)nbv * VEC + (tid - head);
    const char* xrow = static_cast<const char*>(p.logits) + rowoff * ES;
    const char* trow = static_cast<const char*>(p.teacher) + rowoff * ES;
    const u32x4* xv = reinterpret_cast<const u32x4*>(xrow + (int64_t)head * ES);
    const u32x4* tv = reinterpret_cast<const u32x4*>(trow + (int64_t)head * ES);

    uint32_t xy_b = 0u, xe_b = 0u, te_b = 0u;
    if (tid == 0 && y >= 0) xy_b = T::raw1(xrow, y);
    if (has_e) {
        xe_b = T::raw1(xrow, eidx);
        if (TMODE != TM_NONE) te_b = T::raw1(trow, eidx);
    }
    // batch b of thread tid: vectors (b * SU + u) * BLOCK + tid; loads past
    // the row re-read its last vector (in bounds, never summed); a row with no
    // body vector points them at the workspace's row records
    const bool body = nbv > 0;
    const u32x4* xb = body ? xv : reinterpret_cast<const u32x4*>(p.row_rec);
    const u32x4* tb = body ? tv : reinterpret_cast<const u32x4*>(p.row_rec);
    const int64_t lastv = body ? nbv - 1 : 0;
    const int64_t nbatch = (nbv + (int64_t)SU * kStreamBlock - 1) / ((int64_t)SU * kStreamBlock);
    u32x4 xa[SU], ta[TMODE != TM_NONE ? SU : 1];
    auto load_batch = [&](int64_t b, u32x4* xd, u32x4* td) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            int64_t i = (b * SU + u) * kStreamBlock + tid;
            i = i < lastv ? i : lastv;
            xd[u] = ld_stream(xb + i);
            if (TMODE != TM_NONE) td[u] = ld_stream(tb + i);
        }
    };
    load_batch(0, xa, ta);
    const float xe = has_e ? T::from_raw(xe_b) : 0.f;
    const float te = (has_e && TMODE != TM_NONE) ? T::from_raw(te_b) : 0.f;

    // provisional shift: the wave's maximum over its first vectors
    float mx = kNegInf, mt = kNegInf;
    if (tid < nbv) {
        mx = T::vmax(mx, xa[0]);
        if (TMODE != TM_NONE) mt = T::vmax(mt, ta[0]);
    }
    const float mx0 = wave_max(mx);
    const float mt0 = TMODE != TM_NONE ? wave_max(mt) : 0.f;
    auto shift_of = [&](float m) -> float {
        return shift_int<HP>(SOFTCAP ? (p.cap * hl_tanh(m * p.kc)) * kLog2e : m * p.K1);
    };
    float M = shift_of(mx0);
    float Mt = TMODE != TM_NONE ? shift_int<HP>(mt0 * p.K2) : 0.f;
    const bool early = mx0 != kNegInf && (TMODE == TM_NONE || mt0 != kNegInf);
    using Acc = typename std::conditional<HP, double, float>::type;
    Acc z = 0, zt = 0, zs = 0;
    float sv = 0.f, sx = 0.f, st = 0.f;
    if (early) {
        for (int64_t b = 0; b < nbatch; ++b) {
            u32x4 xn[SU], tn[TMODE != TM_NONE ? SU : 1];
            if (b + 1 < nbatch) load_batch(b + 1, xn, tn);
#pragma unroll
            for (int u = 0; u < SU; ++u) {
                if ((b * SU + u) * kStreamBlock + tid < nbv) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        stat_term<TMODE, SOFTCAP, true, HP>(p, M, Mt, T::get(xa[u], e),
                                                        TMODE != TM_NONE ? T::get(ta[u], e) : 0.f,
                                                        z, sv, zt, sx, st, zs);
                }
            }
            if (b + 1 < nbatch) {
#pragma unroll
                for (int u = 0; u < SU; ++u) {
                    xa[u] = xn[u];
                    if (TMODE != TM_NONE) ta[u] = tn[u];
                }
            }
        }
        if (has_e) stat_term<TMODE, SOFTCAP, true, HP>(p, M, Mt, xe, te, z, sv, zt, sx, st, zs);
    }
    float zh = 0.f, zl = 0.f, zth = 0.f, ztl = 0.f, zsh = 0.f, zsl = 0.f;
    auto wave_sums = [&]() {
        if constexpr (HP) {
            split_hl(wave_sum_d(z), zh, zl);
            if (TMODE != TM_NONE) split_hl(wave_sum_d(zt), zth, ztl);
            if (is_hinton(TMODE)) split_hl(wave_sum_d(zs), zsh, zsl);
        } else {
            zh = wave_sum(z);
            if (TMODE != TM_NONE) zth = wave_sum(zt);
            if (is_hinton(TMODE)) zsh = wave_sum(zs);
        }
        sv = wave_sum(sv);
        if (TMODE != TM_NONE) sx = wave_sum(sx);
        if (has_st(TMODE)) st = wave_sum(st);
    };
    wave_sums();
    constexpr float kSumLimit = 18446744073709551616.0f;   // 2^64
    if (!early || !(zh <= kSumLimit) || (TMODE != TM_NONE && !(zth <= kSumLimit)) ||
        (is_hinton(TMODE) && !(zsh <= kSumLimit))) {
        // rare: the true maxima of the wave's vectors, then the sums again
        mx = kNegInf;
        mt = kNegInf;
        for (int64_t i = tid; i < nbv; i += kStreamBlock) {
            mx = T::vmax(mx, xv[i]);
            if (TMODE != TM_NONE) mt = T::vmax(mt, tv[i]);
        }
        if (has_e) {
            mx = fmaxf(mx, xe);
            if (TMODE != TM_NONE) mt = fmaxf(mt, te);
        }
        M = shift_of(wave_max(mx));
        if (TMODE != TM_NONE) Mt = shift_int<HP>(wave_max(mt) * p.K2);
        z = zt = zs = 0;
        sv = sx = st = 0.f;
        for (int64_t i = tid; i < nbv; i += kStreamBlock) {
            const u32x4 w = xv[i];
            u32x4 wt = {0u, 0u, 0u, 0u};
            if (TMODE != TM_NONE) wt = tv[i];
            for (int e = 0; e < VEC; ++e)
                stat_term<TMODE, SOFTCAP, true, HP>(p, M, Mt, T::get(w, e), TMODE != TM_NONE ? T::get(wt, e) : 0.f,
                                                z, sv, zt, sx, st, zs);
        }
        if (has_e) stat_term<TMODE, SOFTCAP, true, HP>(p, M, Mt, xe, te, z, sv, zt, sx, st, zs);
        wave_sums();
    }
    if (lane == 0) {
        s_rec[wave][0] = M; s_rec[wave][1] = zh; s_rec[wave][2] = sv; s_rec[wave][3] = Mt;
        s_rec[wave][4] = zth; s_rec[wave][5] = sx; s_rec[wave][6] = st; s_rec[wave][7] = zsh;
        if (HP) {
            s_rec[wave][8] = zl; s_rec[wave][9] = ztl; s_rec[wave][10] = zsl;
        }
    }
    __syncthreads();
    if (wave == 0) {
        Rec wr = rec_empty();
        const int w = lane & 15;
        if (w < NW) {
            wr.M = s_rec[w][0];
            wr.Z = s_rec[w][1];
            wr.S = s_rec[w][2];
            if (TMODE != TM_NONE) {
                wr.Mt = s_rec[w][3];
                wr.Zt = s_rec[w][4];
                wr.SX = s_rec[w][5];
                if (has_st(TMODE)) wr.St = s_rec[w][6];
                if (is_hinton(TMODE)) wr.Zs = s_rec[w][7];
            }
            if (HP) {
                wr.Zl = s_rec[w][8];
                if (TMODE != TM_NONE) wr.Ztl = s_rec[w][9];
                if (is_hinton(TMODE)) wr.Zsl = s_rec[w][10];
            }
            if (wr.Z == 0.f) wr = rec_empty();
        }
        wr = rec_reduce16<TMODE, HP>(wr, p.beta, NW, p.betad);
        if (lane == 0) {
            float* out = p.row_rec + row * REC;
            out[R_M] = wr.M; out[R_Z] = wr.Z; out[R_S] = wr.S;
            out[R_MT] = wr.Mt; out[R_ZT] = wr.Zt; out[R_SX] = wr.SX; out[R_ST] = wr.St;
            out[R_ZS] = wr.Zs;
            out[R_XY] = T::from_raw(xy_b);
            out[R_VALID] = 1.0f;
            out[R_ZL] = HP ? wr.Zl : 0.f;
            out[R_ZTL] = HP ? wr.Ztl : 0.f;
            out[R_ZSL] = HP ? wr.Zsl : 0.f;
        }
    }
}

template <typename T, int TMODE, bool SOFTCAP>
hipError_t launch_stream_stats(const FusedParams& p, dim3 grid, hipStream_t s) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((stream_stats_kernel<T, TMODE, SOFTCAP>), grid, dim3(kStreamBlock), 0, s, p);
    return hipGetLastError();
}

}  // namespace hl

// Instance getter, by teacher mode and softcap, of a one-workgroup-per-row kernel
// (LAUNCH: hl::launch_rowwise or hl::launch_stream_stats) for one element type.
#define HL_ROW_KERNEL_GETTER(NAME, LAUNCH, T)                                             \
    FusedLauncher NAME(int tmode, bool softcap) {                                         \
        switch (tmode) {                                                                  \
            case hl::TM_NONE:                                                             \
                return softcap ? &LAUNCH<T, hl::TM_NONE, true>                            \
                               : &LAUNCH<T, hl::TM_NONE, false>;                          \
            case hl::TM_FKL:                                                              \
                return softcap ? &LAUNCH<T, hl::TM_FKL, true>                             \
                               : &LAUNCH<T, hl::TM_FKL, false>;                           \
            case hl::TM_RKL:                                                              \
                return softcap ? &LAUNCH<T, hl::TM_RKL, true>                             \
                               : &LAUNCH<T, hl::TM_RKL, false>;                           \
            case hl::TM_FDCE:                                                             \
                return softcap ? &LAUNCH<T, hl::TM_FDCE, true>                            \
                               : &LAUNCH<T, hl::TM_FDCE, false>;                          \
            case hl::TM_FKL_H:                                                            \
                return softcap ? &LAUNCH<T, hl::TM_FKL_H, true>                           \
                               : &LAUNCH<T, hl::TM_FKL_H, false>;                         \
            case hl::TM_RKL_H:                                                            \
                return softcap ? &LAUNCH<T, hl::TM_RKL_H, true>                           \
                               : &LAUNCH<T, hl::TM_RKL_H, false>;                         \
            case hl::TM_FDCE_H:                                                           \
                return softcap ? &LAUNCH<T, hl::TM_FDCE_H, true>                          \
                               : &LAUNCH<T, hl::TM_FDCE_H, false>;                        \
        }                                                                                 \
        return nullptr;                                                                   \
    }

// Instantiation helper for the per-(dtype, mode) translation units.
#define HL_FUSED_CASE(T, BLOCK, NVEC, TMODE)                                 \
    if (block == BLOCK && nvec == NVEC)                                      \
        return softcap ? &hl::launch_fused<T, BLOCK, NVEC, TMODE, true>      \
                       : &hl::launch_fused<T, BLOCK, NVEC, TMODE, false>;
