// probe.hip -- measurements behind the rooflines the library reports, and the
// matrix-core behaviour that fixes how the backward uses the matrix cores.
//
// probe_rate_kernel<WHAT>: sustained issue rates of the units the kernels
// run on, over a grid that fills the chip (4096 workgroups of 256 threads),
// each thread running 8 independent chains for `iters` steps:
//   WHAT 0: v_add_f32          (x_i <- x_i + c)          8 ops per step
//   WHAT 1: v_mul_f32          (x_i <- x_i * c)          8 ops per step
//           (c is held in a vector register, as the kernels' operands are)
//   WHAT 2: v_mfma_f32_16x16x1_4b_f32 (the backward's K = 1 product engine),
//           8 accumulating MFMAs per step, 1024 products each per wave
//   WHAT 3: v_mfma_i32_32x32x32_i8 (the forward's GEMM), 8 accumulating
//           MFMAs per step, 65536 integer ops each per wave
//   WHAT 4: 32-bit integer VALU (x_i <- x_i ^ (x_i >> 3): v_lshrrev_b32 and
//           v_xor_b32), 16 instructions per step
//   WHAT 5: v_add_f32 as WHAT 0 but with c in a scalar register
//   WHAT 7: v_mfma_i32_32x32x32_i8 on operands that change from one MFMA to
//           the next, as a GEMM's do: 16 A and 8 B fragments of hashed bits
//           held in registers, each step four rounds of a 4 x 2 grid of
//           them (32 MFMAs, 8 accumulators, no other instructions).  The
//           matrix core's power, and so the clock it sustains, depends on
//           how many operand bits toggle
//   WHAT 6: the backward's product engine without its memory traffic: per
//           step 4 K = 1 fp32 MFMAs with a -0 accumulator and the 64 v_add_f32
//           that add their products into 4 running sums (4096 multiply-adds
//           per wave)
//   WHAT 8: the same engine on operands that change from one MFMA to the
//           next, as the backward's do: 16 A and 16 B values per lane of
//           hashed sign and significand (magnitudes in [1, 2)), each step
//           four rounds of 4 MFMAs (16 distinct operand pairs) and their
//           256 adds per lane (16384 multiply-adds per wave)
// The results are stored so that no chain is dead code.
//
// probe_mfma_fma_kernel: the K = 1 fp32 MFMA with a non-zero accumulator
// input, out[i] = A*B + C for A = B = a[i], C = b[i].  It rounds the product
// and the sum once (the fused result); this is why the backward feeds it an
// accumulator of -0 and adds the products on the VALU, where every add is one
// binary32 rounding.
#include "internal.hpp"

#pragma clang fp contract(off)

namespace brl {

typedef float v16fp __attribute__((ext_vector_type(16)));
typedef int v4ip __attribute__((ext_vector_type(4)));
typedef int v16ip __attribute__((ext_vector_type(16)));

constexpr int kRateBlocks = 4096;
constexpr int kRateThreads = 256;

static_assert((int64_t)kRateBlocks * kRateThreads <= (1 << 30), "(threadIdx.x * blockIdx.x) >> 30 must stay 0");

template <int WHAT>
__global__ __launch_bounds__(kRateThreads) void probe_rate_kernel(int64_t iters, float c, float* __restrict__ out) {
    const int64_t gid = (int64_t)blockIdx.x * kRateThreads + threadIdx.x;
    float r = 0.0f;
    if constexpr (WHAT == 0 || WHAT == 1 || WHAT == 5) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (float)(threadIdx.x + i) * 0.25f + 1.0f;
        // (threadIdx.x * blockIdx.x) >> 30 is 0 for every launch of this
        // kernel, but not known to the compiler: cv is a per-lane register
        const float cv = WHAT == 5 ? c : f_add(c, (float)((threadIdx.x * blockIdx.x) >> 30));
        for (int64_t s = 0; s < iters; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = WHAT == 1 ? f_mul(x[i], cv) : f_add(x[i], cv);
#pragma unroll
        for (int i = 0; i < 8; ++i) r = f_add(r, x[i]);
    } else if constexpr (WHAT == 2) {
        v16fp acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
        const float a = c * (float)(threadIdx.x & 7), b = c;
        for (int64_t s = 0; s < iters; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x1f32(a, b, acc[i], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) r = f_add(r, acc[i][e]);
    } else if constexpr (WHAT == 6) {
        v16fp acc[4], p[4], cneg;
#pragma unroll
        for (int e = 0; e < 16; ++e) cneg[e] = -0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = cneg;
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = c * (float)((threadIdx.x & 7) * (i + 1));
        const float b = c;
        for (int64_t s = 0; s < iters; ++s) {
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_mfma_f32_16x16x1f32(a[i], b, cneg, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][e] = f_add(acc[i][e], p[i][e]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) r = f_add(r, acc[i][e]);
    } else if constexpr (WHAT == 8) {
        v16fp acc[4], p[4], cneg;
#pragma unroll
        for (int e = 0; e < 16; ++e) cneg[e] = -0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = cneg;
        // operand f of side `ab` (0: A, 1: B): a xorshift of a hash of
        // (thread, 2f + ab), sign and significand kept, exponent 0
        float av[16], bv[16];
#pragma unroll
        for (int f = 0; f < 16; ++f)
#pragma unroll
            for (int ab = 0; ab < 2; ++ab) {
                unsigned x = ((unsigned)gid + 1u) * 0x9E3779B1u + (unsigned)(2 * f + ab + 1) * 0x85EBCA77u;
                x ^= x << 13;
                x ^= x >> 17;
                x ^= x << 5;
                const float v = __int_as_float((int)((x & 0x807FFFFFu) | 0x3F800000u));
                if (ab == 0) av[f] = v;
                else bv[f] = v;
            }
        for (int64_t s = 0; s < iters; ++s)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_mfma_f32_16x16x1f32(av[4 * u + i], bv[4 * u + i], cneg, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[i][e] = f_add(acc[i][e], p[i][e]);
            }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) r = f_add(r, acc[i][e]);
    } else if constexpr (WHAT == 4) {
        unsigned x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (unsigned)gid * 8u + (unsigned)i + 1u;
        for (int64_t s = 0; s < iters; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] ^= x[i] >> 3;
        unsigned t = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) t ^= x[i];
        r = (float)(t & 0xFFFFFFu);
    } else if constexpr (WHAT == 7) {
        v16ip acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][e] = 0;
        // fragment f (A: f < 16, B: f >= 16), register k: a xorshift of a
        // hash of (thread, f, k)
        v4ip fr[24];
#pragma unroll
        for (int f = 0; f < 24; ++f)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                unsigned x = ((unsigned)gid + 1u) * 0x9E3779B1u + (unsigned)(4 * f + k + 1) * 0x85EBCA77u;
                x ^= x << 13;
                x ^= x >> 17;
                x ^= x << 5;
                fr[f][k] = (int)x;
            }
        for (int64_t s = 0; s < iters; ++s)
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    acc[q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fr[4 * p + q / 2], fr[16 + 2 * p + q % 2], acc[q], 0, 0, 0);
        unsigned t = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) t += (unsigned)acc[i][e];
        r = (float)(t & 0xFFFFFFu);
    } else {
        v16ip acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][e] = 0;
        const int v = (int)c + (int)(threadIdx.x & 3);
        const v4ip a = {v, v + 1, v + 2, v + 3}, b = {v + 4, v, v + 1, v + 2};
        for (int64_t s = 0; s < iters; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[i], 0, 0, 0);
        int t = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) t += acc[i][e];
        r = (float)t;
    }
    out[gid] = r;
}

hipError_t launch_probe_rate(int what, int64_t iters, float c, float* out, hipStream_t st) {
    const dim3 g(kRateBlocks), b(kRateThreads);
    switch (what) {
        case 0: hipLaunchKernelGGL(probe_rate_kernel<0>, g, b, 0, st, iters, c, out); break;
        case 1: hipLaunchKernelGGL(probe_rate_kernel<1>, g, b, 0, st, iters, c, out); break;
        case 2: hipLaunchKernelGGL(probe_rate_kernel<2>, g, b, 0, st, iters, c, out); break;
        case 3: hipLaunchKernelGGL(probe_rate_kernel<3>, g, b, 0, st, iters, c, out); break;
        case 4: hipLaunchKernelGGL(probe_rate_kernel<4>, g, b, 0, st, iters, c, out); break;
        case 5: hipLaunchKernelGGL(probe_rate_kernel<5>, g, b, 0, st, iters, c, out); break;
        case 6: hipLaunchKernelGGL(probe_rate_kernel<6>, g, b, 0, st, iters, c, out); break;
        case 7: hipLaunchKernelGGL(probe_rate_kernel<7>, g, b, 0, st, iters, c, out); break;
        case 8: hipLaunchKernelGGL(probe_rate_kernel<8>, g, b, 0, st, iters, c, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int64_t probe_rate_threads() { return (int64_t)kRateBlocks * kRateThreads; }

// Each wave takes 64 (a, b) pairs.  Lane l feeds a[l] as A row l and as B
// column l % 16 of the 16x16x1 MFMA (four 16x16 blocks, block beta = lanes
// 16beta .. 16beta+15); pair 16beta + t lands at row t, column t of block beta,
// which is lane 16(t/4) + t, register 4beta + t%4; that accumulator element
// starts as b of the pair, every other one as -0.
__global__ __launch_bounds__(64) void probe_mfma_fma_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                                            float* __restrict__ out, int64_t n) {
    const int lane = threadIdx.x;
    const int64_t base = (int64_t)blockIdx.x * 64;
    const float x = base + lane < n ? a[base + lane] : 0.0f;
    const int t = lane & 15;
    const bool diag = (lane >> 4) == (t >> 2);
    v16fp c;
#pragma unroll
    for (int beta = 0; beta < 4; ++beta)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t i = base + 16 * beta + t;
            c[4 * beta + e] = (diag && e == (t & 3) && i < n) ? b[i] : -0.0f;
        }
    const v16fp d = __builtin_amdgcn_mfma_f32_16x16x1f32(x, x, c, 0, 0, 0);
    if (diag) {
#pragma unroll
        for (int beta = 0; beta < 4; ++beta) {
            const int64_t i = base + 16 * beta + t;
            if (i < n) out[i] = d[4 * beta + (t & 3)];
        }
    }
}

hipError_t launch_probe_mfma_fma(const float* a, const float* b, float* out, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(probe_mfma_fma_kernel, dim3((unsigned)ceil_div(n, 64)), dim3(64), 0, st, a, b, out, n);
    return hipGetLastError();
}

}  // namespace brl
