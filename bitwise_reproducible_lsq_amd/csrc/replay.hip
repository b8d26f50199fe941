// replay.hip -- streaming kernels of the single-device audit replay of the
// gradient reduction (Open-1B summary on onedev.kr, "Limits", audit
// paragraph): the running sum of each replica over its shards, the TreeFold
// across replicas in recursive-doubling pairing order, and the clip scale
// pass of the global-norm clip (same page, recipe paragraph).
//
// All three are elementwise and bound by HBM: 16-byte vector loads and
// stores, non-temporal (each byte is touched once per pass), grid-stride
// loops over a fixed number of workgroups.
#include "internal.hpp"

#pragma clang fp contract(off)

namespace brl {

constexpr int kStreamThreads = 256;

static unsigned stream_grid(int64_t n4) {
    int64_t want = ceil_div(n4, kStreamThreads);
    int64_t cap = stream_wgs();
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    return (unsigned)want;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// A <- A + G
__global__ __launch_bounds__(kStreamThreads) void accumulate_v4_kernel(vf4* __restrict__ A,
                                                                       const vf4* __restrict__ G,
                                                                       int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
    for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n4; i += stride) {
        vf4 a = __builtin_nontemporal_load(A + i);
        vf4 g = __builtin_nontemporal_load(G + i);
        a.x = f_add(a.x, g.x);
        a.y = f_add(a.y, g.y);
        a.z = f_add(a.z, g.z);
        a.w = f_add(a.w, g.w);
        __builtin_nontemporal_store(a, A + i);
    }
}

__global__ __launch_bounds__(kStreamThreads) void accumulate_scalar_kernel(float* __restrict__ A,
                                                                           const float* __restrict__ G,
                                                                           int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
    for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += stride)
        A[i] = f_add(A[i], G[i]);
}

hipError_t launch_accumulate(float* A, const float* G, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    if (aligned16(A) && aligned16(G)) {
        int64_t n4 = n / 4;
        if (n4 > 0)
            hipLaunchKernelGGL(accumulate_v4_kernel, dim3(stream_grid(n4)), dim3(kStreamThreads), 0,
                               st, reinterpret_cast<vf4*>(A), reinterpret_cast<const vf4*>(G), n4);
        if (n - n4 * 4 > 0)
            hipLaunchKernelGGL(accumulate_scalar_kernel, dim3(1), dim3(kStreamThreads), 0, st,
                               A + n4 * 4, G + n4 * 4, n - n4 * 4);
    } else {
        hipLaunchKernelGGL(accumulate_scalar_kernel, dim3(stream_grid(ceil_div(n, 4))),
                           dim3(kStreamThreads), 0, st, A, G, n);
    }
    return hipGetLastError();
}

// TreeFold of R replica partials (the last one optionally still to be added
// to g_last): leaves L_i = A_i + A_{i+P} for i < R-P, else A_i; then the
// pairwise tree over the P leaves.  P = largest power of two <= R.
template <int P>
__device__ __forceinline__ float fold_one(const FoldPtrs& p, int R, const float* g_last, int64_t e) {
    float L[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        float a = p.a[i][e];
        if (i == R - 1 && g_last) a = f_add(a, g_last[e]);
        if (i + P < R) {
            float b = p.a[i + P][e];
            if (i + P == R - 1 && g_last) b = f_add(b, g_last[e]);
            a = f_add(a, b);
        }
        L[i] = a;
    }
#pragma unroll
    for (int w = 1; w < P; w *= 2)
#pragma unroll
        for (int i = 0; i < P; i += 2 * w) L[i] = f_add(L[i], L[i + w]);
    return L[0];
}

template <int P>
__global__ __launch_bounds__(kStreamThreads) void fold_kernel(FoldPtrs p, int R, const float* g_last,
                                                              float* __restrict__ out, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
    for (int64_t e = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; e < n; e += stride)
        out[e] = fold_one<P>(p, R, g_last, e);
}

// Vector version for R = 6 (the replay's mesh): 16-byte loads.
__global__ __launch_bounds__(kStreamThreads) void fold6_v4_kernel(FoldPtrs p, const float* g_last,
                                                                  vf4* __restrict__ out, int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
    const vf4* a0 = reinterpret_cast<const vf4*>(p.a[0]);
    const vf4* a1 = reinterpret_cast<const vf4*>(p.a[1]);
    const vf4* a2 = reinterpret_cast<const vf4*>(p.a[2]);
    const vf4* a3 = reinterpret_cast<const vf4*>(p.a[3]);
    const vf4* a4 = reinterpret_cast<const vf4*>(p.a[4]);
    const vf4* a5 = reinterpret_cast<const vf4*>(p.a[5]);
    const vf4* gl = reinterpret_cast<const vf4*>(g_last);
    for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n4; i += stride) {
        vf4 v0 = __builtin_nontemporal_load(a0 + i), v1 = __builtin_nontemporal_load(a1 + i);
        vf4 v2 = __builtin_nontemporal_load(a2 + i), v3 = __builtin_nontemporal_load(a3 + i);
        vf4 v4 = __builtin_nontemporal_load(a4 + i), v5 = __builtin_nontemporal_load(a5 + i);
        if (gl) {
            vf4 g = __builtin_nontemporal_load(gl + i);
            v5.x = f_add(v5.x, g.x); v5.y = f_add(v5.y, g.y);
            v5.z = f_add(v5.z, g.z); v5.w = f_add(v5.w, g.w);
        }
        vf4 r;
#define FOLD6(c) r.c = f_add(f_add(f_add(v0.c, v4.c), f_add(v1.c, v5.c)), f_add(v2.c, v3.c))
        FOLD6(x); FOLD6(y); FOLD6(z); FOLD6(w);
#undef FOLD6
        __builtin_nontemporal_store(r, out + i);
    }
}

hipError_t launch_fold(const FoldPtrs& p, int R, const float* g_last, float* out, int64_t n,
                       hipStream_t st) {
    if (n <= 0) return hipSuccess;
    bool al = aligned16(out) && (!g_last || aligned16(g_last));
    for (int i = 0; i < R; ++i) al = al && aligned16(p.a[i]);
    int64_t done = 0;
    if (R == 6 && al && n >= 4) {
        int64_t n4 = n / 4;
        hipLaunchKernelGGL(fold6_v4_kernel, dim3(stream_grid(n4)), dim3(kStreamThreads), 0, st, p,
                           g_last, reinterpret_cast<vf4*>(out), n4);
        done = n4 * 4;
    }
    if (done < n) {
        FoldPtrs q = p;
        for (int i = 0; i < R; ++i) q.a[i] = p.a[i] + done;
        const float* gl = g_last ? g_last + done : nullptr;
        int64_t m = n - done;
        dim3 grid(stream_grid(ceil_div(m, 4))), blk(kStreamThreads);
        int P = 1;
        while (P * 2 <= R) P *= 2;
        switch (P) {
            case 1: hipLaunchKernelGGL(fold_kernel<1>, grid, blk, 0, st, q, R, gl, out + done, m); break;
            case 2: hipLaunchKernelGGL(fold_kernel<2>, grid, blk, 0, st, q, R, gl, out + done, m); break;
            case 4: hipLaunchKernelGGL(fold_kernel<4>, grid, blk, 0, st, q, R, gl, out + done, m); break;
            case 8: hipLaunchKernelGGL(fold_kernel<8>, grid, blk, 0, st, q, R, gl, out + done, m); break;
            case 16: hipLaunchKernelGGL(fold_kernel<16>, grid, blk, 0, st, q, R, gl, out + done, m); break;
            case 32: hipLaunchKernelGGL(fold_kernel<32>, grid, blk, 0, st, q, R, gl, out + done, m); break;
            default: hipLaunchKernelGGL(fold_kernel<64>, grid, blk, 0, st, q, R, gl, out + done, m); break;
        }
    }
    return hipGetLastError();
}

// g <- g * kappa when the norm exceeded the bound (decided on the device).
__global__ __launch_bounds__(kStreamThreads) void clip_v4_kernel(vf4* __restrict__ g, int64_t n4,
                                                                 const Scalars* __restrict__ s) {
    if (!s->clip) return;
    const float k = s->kappa;
    const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
    for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n4; i += stride) {
        vf4 v = __builtin_nontemporal_load(g + i);
        v.x = f_mul(v.x, k); v.y = f_mul(v.y, k); v.z = f_mul(v.z, k); v.w = f_mul(v.w, k);
        __builtin_nontemporal_store(v, g + i);
    }
}

__global__ __launch_bounds__(kStreamThreads) void clip_scalar_kernel(float* __restrict__ g, int64_t n,
                                                                     const Scalars* __restrict__ s) {
    if (!s->clip) return;
    const float k = s->kappa;
    const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
    for (int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += stride)
        g[i] = f_mul(g[i], k);
}

hipError_t launch_clip(float* g, int64_t n, const Scalars* scal, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t done = 0;
    if (aligned16(g)) {
        int64_t n4 = n / 4;
        if (n4 > 0)
            hipLaunchKernelGGL(clip_v4_kernel, dim3(stream_grid(n4)), dim3(kStreamThreads), 0, st,
                               reinterpret_cast<vf4*>(g), n4, scal);
        done = n4 * 4;
    }
    if (done < n)
        hipLaunchKernelGGL(clip_scalar_kernel, dim3(stream_grid(ceil_div(n - done, 4))),
                           dim3(kStreamThreads), 0, st, g + done, n - done, scal);
    return hipGetLastError();
}

// ---- conformance probe ---------------------------------------------------------
__global__ void probe_kernel(int op, const float* __restrict__ a, const float* __restrict__ b,
                             float* __restrict__ out, int64_t n, ExpConsts ek) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float x = a[i];
    float y = b ? b[i] : 0.0f;
    float r;
    switch (op) {
        case 0: r = f_add(x, y); break;
        case 1: r = f_sub(x, y); break;
        case 2: r = f_mul(x, y); break;
        case 3: r = f_div(x, y); break;
        case 4: r = f_sqrt(x); break;
        case 5: r = (float)__float_as_int(x); break;
        case 6: r = f_rne(x); break;
        default: r = own_exp(x, ek); break;
    }
    out[i] = r;
}

hipError_t launch_probe(int op, const float* a, const float* b, float* out, int64_t n,
                        const ExpConsts& ek, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(probe_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, op, a, b,
                       out, n, ek);
    return hipGetLastError();
}

}  // namespace brl
