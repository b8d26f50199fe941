// device.hpp -- binary32 building blocks shared by the gfx950 kernels.
//
// Numerics (Open-1B summary on onedev.kr, section "How"): one fixed reduction
// order, multiply and add never fused, subnormals flushed to zero.  The
// kernels are compiled with the f32 denormal mode "flush inputs and outputs"
// and contraction off, so a plain `a + b` / `a * b` is one v_add_f32 /
// v_mul_f32 that rounds to nearest even and flushes.  Division is the
// compiler's correctly rounded binary32 sequence (the only place where an fp32
// multiply-add appears: inside it, between v_div_scale_f32 and
// v_div_fixup_f32); square root goes through binary64 (correctly rounded
// there, and 53 >= 2*24+2 makes the second rounding to binary32 innocuous)
// with explicit flushing on both sides.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace brl {

typedef float vf4 __attribute__((ext_vector_type(4)));   // 16-byte vector

constexpr int kBlock = 32;      // CanonSum block width
constexpr int kQmax = 127;      // int8 quantiser range [-127, 127]

// s_waitcnt with vmcnt <= N, expcnt and lgkmcnt left unconstrained (gfx9
// encoding): waits for this wave's older global loads, including the direct
// global -> LDS ones.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ float flush_f32(float x) {
    return (__builtin_fabsf(x) < 1.17549435e-38f) ? __builtin_copysignf(0.0f, x) : x;
}

__device__ __forceinline__ float f_add(float a, float b) { return a + b; }
__device__ __forceinline__ float f_sub(float a, float b) { return a - b; }
__device__ __forceinline__ float f_mul(float a, float b) { return a * b; }

// One correctly rounded binary32 division.  In the flush mode its operands
// read subnormals as zeros of the same sign and a subnormal quotient is
// flushed; a quotient of two binary32 values never falls strictly between
// 2^-126 (1 - 2^-24) and 2^-126, the band where flushing before and after
// rounding would differ, so the result is the one f_div of binary64 gives.
__device__ __forceinline__ float f_div(float a, float b) { return a / b; }

// a / b for a divisor b fixed across many calls, given rb = fl64(1/flush(b)):
// the same correctly rounded binary32 quotient as f_div (see Quantizer below
// for why the binary64 product lands in the right rounding interval).
__device__ __forceinline__ float f_div_by(float a, double rb) {
    return flush_f32((float)((double)flush_f32(a) * rb));
}

__device__ __forceinline__ float f_sqrt(float a) {
    double r = __builtin_sqrt((double)flush_f32(a));
    return flush_f32((float)r);
}

__device__ __forceinline__ float f_rne(float t) { return __builtin_rintf(t); }

// LSQ quantiser with step s: q = clamp(rne(v/s), -127, 127),
// in = (-127 <= v/s <= 127); a zero step maps everything to q = 0, in range.
//
// Exact path.  The quotient comes from the binary64 reciprocal of the step:
// fl32(fl64(v * fl64(1/s))) is the correctly rounded binary32 v/s.  The
// binary64 product is within 2^-51.9 (relative) of v/s, while the exact
// quotient of two binary32 numbers that is not itself a rounding boundary
// is at least 2^-49 (relative) away from every one of them: the midpoints
// between neighbouring binary32 values and the underflow threshold.  So the
// product lies in the same rounding interval as v/s.
//
// Fast path.  t = v * fl32(1/s) in binary32 is within 3 * 2^-24 |v/s| of the
// correctly rounded quotient T (two roundings in t, one in T).  For |v/s| <=
// 128 that is under 2^-15, so when t lies at least 2^-15 from every midpoint
// k + 1/2 (the points where rne changes), T lies strictly on the same side of
// each of them and rne(T) = rne(t); likewise for the range test when t lies
// at least 2^-15 from +-127.  Above 128 in magnitude both give the clamped
// code and an out-of-range mask (and the 2^-15 test is only conservative).
// The fast forms report `unsure` when t is closer than that; callers then
// redo their values on the exact path (a wave at a time: about 1 in 16000
// uniformly placed quotients is unsure).  Subnormal v reads as zero in both.
struct Quantizer {
    float s;
    double rs;
    float rf;
    __device__ __forceinline__ explicit Quantizer(float step)
        : s(flush_f32(step)), rs(s == 0.0f ? 0.0 : 1.0 / (double)s), rf(s == 0.0f ? 0.0f : 1.0f / s) {}
    __device__ __forceinline__ float quotient(float v) const {
        return flush_f32((float)((double)flush_f32(v) * rs));
    }
    __device__ __forceinline__ int q(float v, bool* in_range) const {
        if (s == 0.0f) { *in_range = true; return 0; }
        const float t = quotient(v);
        *in_range = (t >= -(float)kQmax) && (t <= (float)kQmax);
        float r = f_rne(t);
        r = r > (float)kQmax ? (float)kQmax : r;
        r = r < -(float)kQmax ? -(float)kQmax : r;
        return (int)r;
    }
    __device__ __forceinline__ bool in_range(float v) const {
        if (s == 0.0f) return true;
        const float t = quotient(v);
        return (t >= -(float)kQmax) && (t <= (float)kQmax);
    }
    // q(v) when *unsure stays false; sets *unsure (never clears it) otherwise
    __device__ __forceinline__ int q_fast(float v, bool* unsure) const {
        const float t = v * rf;                  // s == 0: rf = 0, t = 0, q = 0
        const float r = f_rne(t);
        *unsure |= __builtin_fabsf(t - r) > 0.5f - 0x1p-15f;
        float c = r > (float)kQmax ? (float)kQmax : r;
        c = c < -(float)kQmax ? -(float)kQmax : c;
        return (int)c;
    }
    // in_range(v) when *unsure stays false; sets *unsure otherwise
    __device__ __forceinline__ bool in_range_fast(float v, bool* unsure) const {
        const float t = v * rf;
        *unsure |= __builtin_fabsf(__builtin_fabsf(t) - (float)kQmax) < 0x1p-15f;
        return s == 0.0f || __builtin_fabsf(t) <= (float)kQmax;
    }
};

// The weight step from S = CanonSum(|w|) over `count` weights:
// s_w = (2 * (S / fl(count))) / fl(sqrt(127)).
__device__ __forceinline__ float weight_step(float S, float count_f) {
    const float mu = f_div(S, count_f);
    return f_div(f_mul(2.0f, mu), f_sqrt((float)kQmax));
}

// ---- the library's own binary32 exp (SwiGLU) ------------------------------
// E(x): Cody-Waite reduction x = k*ln2 + r with k = rne(x * log2(e)), ln2
// split into a 16-bit head (so k*head is exact) and a binary32 tail; degree-7
// Taylor polynomial sum r^i/i! in Horner form; scaling by 2^k as two exact
// power-of-two multiplies.  x > 89 gives +inf, x < -104 gives +0.
struct ExpConsts {
    float l2e, ln2_hi, ln2_lo;
    float c[8];
};

// x is clamped into [-104, 89]: the steps give +0 at -104 and +inf at 89,
// as the definition does beyond them, so only NaN is selected afterwards and
// a wave takes no branch.  The scaling by 2^k is one ldexp: p * 2^k is exact
// while it is a normal number, overflows to +inf as the two multiplies do,
// and below 2^-126 is flushed to +0 by the FTZ mode either way.
__device__ __forceinline__ float own_exp(float x, const ExpConsts& K) {
    const float xr = __builtin_fminf(__builtin_fmaxf(x, -104.0f), 89.0f);
    float k = f_rne(f_mul(xr, K.l2e));
    float r = f_sub(f_sub(xr, f_mul(k, K.ln2_hi)), f_mul(k, K.ln2_lo));
    float p = K.c[7];
#pragma unroll
    for (int i = 6; i >= 0; --i) p = f_add(f_mul(p, r), K.c[i]);
    const float y = __builtin_amdgcn_ldexpf(p, (int)k);
    return x != x ? x : y;
}

// SwiGLU forward pieces: s = 1/(1 + E(-g)), h = g*s, a = h*u.
__device__ __forceinline__ float swiglu_sigma(float g, const ExpConsts& K) {
    float e = own_exp(-g, K);
    return f_div(1.0f, f_add(1.0f, e));
}

// ---- CanonSum helpers -------------------------------------------------------
// Pairwise tree, level by level with odd carry, over `count` values held in
// LDS (count <= blockDim.x).  Every thread of the workgroup must call it.
// Returns the root in thread 0 (other threads get unspecified values).
__device__ __forceinline__ float wg_pair_tree(float v, int count, float* lds) {
    const int t = threadIdx.x;
    lds[t] = v;
    __syncthreads();
    while (count > 1) {
        const int h = count >> 1;
        float nv = 0.0f;
        if (t < h) nv = f_add(lds[2 * t], lds[2 * t + 1]);
        else if (t == h && (count & 1)) nv = lds[count - 1];
        __syncthreads();
        if (t < h || (t == h && (count & 1))) lds[t] = nv;
        __syncthreads();
        count = h + (count & 1);
    }
    float r = lds[0];
    __syncthreads();
    return r;
}

// CanonSum root of Q leaves by one workgroup of blockDim.x threads
// (Q <= RUN * blockDim.x): thread t first reduces the aligned run [t*RUN,
// (t+1)*RUN) in registers, level by level (a complete subtree of the
// canonical tree, or for the short last run the canonical tree of its own
// leaves, which is the same thing), then the workgroup tree combines the run
// roots.  Every thread must call it; the root is returned in thread 0.
// leaf(j) returns leaf j.
template <int RUN, class Leaf>
__device__ __forceinline__ float canon_runs_tree(Leaf leaf, int64_t Q, float* lds) {
    const int64_t first = (int64_t)threadIdx.x * RUN;
    const int64_t left = Q - first;
    const int cnt = left <= 0 ? 0 : (left < RUN ? (int)left : RUN);
    float v[RUN];
#pragma unroll
    for (int i = 0; i < RUN; ++i) v[i] = i < cnt ? leaf(first + i) : 0.0f;
#pragma unroll
    for (int w = 1; w < RUN; w *= 2)
#pragma unroll
        for (int i = 0; i + w < RUN; i += 2 * w)
            if (i + w < cnt) v[i] = f_add(v[i], v[i + w]);
    const int runs = (int)((Q + RUN - 1) / RUN);
    return wg_pair_tree(v[0], runs, lds);
}

}  // namespace brl
