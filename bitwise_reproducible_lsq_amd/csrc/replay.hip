// replay.hip -- streaming kernels of the single-device audit replay of the
// gradient reduction (Open-1B summary on onedev.kr, "Limits", audit
// paragraph): the running sum of each replica over its shards, the TreeFold
// across replicas in recursive-doubling pairing order, and the clip scale
// pass of the global-norm clip (same page, recipe paragraph).
//
// All are elementwise and bound by HBM: 16-byte non-temporal vector loads and
// stores (each byte is touched once per pass) in one-shot grids, one vector
// per thread by default -- the fastest shape measured on MI355X for these
// read/write mixes.
#include "internal.hpp"

#pragma clang fp contract(off)

namespace brl {

constexpr int kStreamThreads = 256;

// One-shot grids: each thread handles V 16-byte vectors, V = the stream
// vector knob (1 by default: the fastest shape measured on MI355X).
static unsigned stream_grid(int64_t n4, int V) {
    int64_t g = ceil_div(n4, (int64_t)kStreamThreads * V);
    return (unsigned)(g < 1 ? 1 : g);
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <int V>
__device__ __forceinline__ int64_t vec_index(int u) {
    return ((int64_t)blockIdx.x * V + u) * kStreamThreads + threadIdx.x;
}

// A <- X + G (X is A itself, or the deferred first shard of the replica)
template <int V>
__global__ __launch_bounds__(kStreamThreads) void accumulate_v4_kernel(vf4* A, const vf4* X,
                                                                       const vf4* __restrict__ G,
                                                                       int64_t n4) {
    vf4 a[V], g[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int64_t i = vec_index<V>(u);
        if (i < n4) { a[u] = __builtin_nontemporal_load(X + i); g[u] = __builtin_nontemporal_load(G + i); }
    }
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int64_t i = vec_index<V>(u);
        if (i < n4) {
            vf4 r;
            r.x = f_add(a[u].x, g[u].x);
            r.y = f_add(a[u].y, g[u].y);
            r.z = f_add(a[u].z, g[u].z);
            r.w = f_add(a[u].w, g[u].w);
            __builtin_nontemporal_store(r, A + i);
        }
    }
}

// A <- G (the first shard of a replica)
template <int V>
__global__ __launch_bounds__(kStreamThreads) void copy_v4_kernel(vf4* __restrict__ A, const vf4* __restrict__ G,
                                                                 int64_t n4) {
    vf4 g[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int64_t i = vec_index<V>(u);
        if (i < n4) g[u] = __builtin_nontemporal_load(G + i);
    }
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int64_t i = vec_index<V>(u);
        if (i < n4) __builtin_nontemporal_store(g[u], A + i);
    }
}

__global__ __launch_bounds__(kStreamThreads) void accumulate_scalar_kernel(float* A, const float* X,
                                                                           const float* __restrict__ G,
                                                                           int64_t n, int first) {
    const int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    if (i < n) A[i] = first ? G[i] : f_add(X[i], G[i]);
}

hipError_t launch_accumulate(float* A, const float* X, const float* G, int64_t n, int first, int vec,
                             hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t done = 0;
    if (aligned16(A) && aligned16(X) && aligned16(G)) {
        const int64_t n4 = n / 4;
        const int V = vec;
        if (n4 > 0) {
            vf4* a4 = reinterpret_cast<vf4*>(A);
            const vf4* x4 = reinterpret_cast<const vf4*>(X);
            const vf4* g4 = reinterpret_cast<const vf4*>(G);
            const dim3 grid(stream_grid(n4, V)), blk(kStreamThreads);
            if (first) {
                if (V == 4) hipLaunchKernelGGL(copy_v4_kernel<4>, grid, blk, 0, st, a4, g4, n4);
                else if (V == 2) hipLaunchKernelGGL(copy_v4_kernel<2>, grid, blk, 0, st, a4, g4, n4);
                else hipLaunchKernelGGL(copy_v4_kernel<1>, grid, blk, 0, st, a4, g4, n4);
            } else {
                if (V == 4) hipLaunchKernelGGL(accumulate_v4_kernel<4>, grid, blk, 0, st, a4, x4, g4, n4);
                else if (V == 2) hipLaunchKernelGGL(accumulate_v4_kernel<2>, grid, blk, 0, st, a4, x4, g4, n4);
                else hipLaunchKernelGGL(accumulate_v4_kernel<1>, grid, blk, 0, st, a4, x4, g4, n4);
            }
        }
        done = n4 * 4;
    }
    if (done < n)
        hipLaunchKernelGGL(accumulate_scalar_kernel, dim3((unsigned)ceil_div(n - done, kStreamThreads)),
                           dim3(kStreamThreads), 0, st, A + done, X + done, G + done, n - done, first);
    return hipGetLastError();
}

// The running sum of a replica whose S partials are all resident, in one
// pass: ((G_0 + G_1) + G_2) + ... + G_{S-1}, the same binary32 adds in the
// same order as one accumulate pass per shard.  The loads of up to 8
// partials are issued before their adds.
__device__ __forceinline__ vf4 runsum_vec(const FoldPtrs& parts, int S, int64_t i) {
    vf4 acc = __builtin_nontemporal_load(reinterpret_cast<const vf4*>(parts.a[0]) + i);
    for (int s0 = 1; s0 < S; s0 += 8) {
        vf4 g[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < S) g[u] = __builtin_nontemporal_load(reinterpret_cast<const vf4*>(parts.a[s0 + u]) + i);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < S) {
                acc.x = f_add(acc.x, g[u].x); acc.y = f_add(acc.y, g[u].y);
                acc.z = f_add(acc.z, g[u].z); acc.w = f_add(acc.w, g[u].w);
            }
    }
    return acc;
}

__device__ __forceinline__ float runsum_one(const FoldPtrs& parts, int S, int64_t e) {
    float acc = parts.a[0][e];
    for (int s = 1; s < S; ++s) acc = f_add(acc, parts.a[s][e]);
    return acc;
}

__global__ __launch_bounds__(kStreamThreads) void runsum_v4_kernel(vf4* __restrict__ A, FoldPtrs parts, int S,
                                                                   int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    if (i < n4) __builtin_nontemporal_store(runsum_vec(parts, S, i), A + i);
}

__global__ __launch_bounds__(kStreamThreads) void runsum_scalar_kernel(float* __restrict__ A, FoldPtrs parts,
                                                                       int S, int64_t n) {
    const int64_t e = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    if (e < n) A[e] = runsum_one(parts, S, e);
}

static FoldPtrs offset_ptrs(const FoldPtrs& p, int count, int64_t d) {
    FoldPtrs q{};
    for (int i = 0; i < count; ++i) q.a[i] = p.a[i] + d;
    return q;
}

hipError_t launch_runsum(float* A, const FoldPtrs& parts, int S, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    if (S < 1 || S > 64) return hipErrorInvalidValue;
    bool al = aligned16(A);
    for (int s = 0; s < S; ++s) al = al && aligned16(parts.a[s]);
    int64_t done = 0;
    if (al) {
        const int64_t n4 = n / 4;
        if (n4 > 0)
            hipLaunchKernelGGL(runsum_v4_kernel, dim3(stream_grid(n4, 1)), dim3(kStreamThreads), 0, st,
                               reinterpret_cast<vf4*>(A), parts, S, n4);
        done = n4 * 4;
    }
    if (done < n)
        hipLaunchKernelGGL(runsum_scalar_kernel, dim3((unsigned)ceil_div(n - done, kStreamThreads)),
                           dim3(kStreamThreads), 0, st, A + done, offset_ptrs(parts, S, done), S, n - done);
    return hipGetLastError();
}

// TreeFold of R replica partials (the last one optionally still to be added
// to g_last): leaves L_i = A_i + A_{i+P} for i < R-P, else A_i; then the
// pairwise tree over the P leaves.  P = largest power of two <= R.
// Replica R-1's value at e: its resident partials' running sum, or A_{R-1}
// completed with g_last when given.
__device__ __forceinline__ float last_replica(const FoldPtrs& p, int R, const float* g_last, const FoldPtrs& last,
                                              int nlast, int64_t e) {
    if (nlast > 0) return runsum_one(last, nlast, e);
    float a = p.a[R - 1][e];
    if (g_last) a = f_add(a, g_last[e]);
    return a;
}

template <int P>
__device__ __forceinline__ float fold_one(const FoldPtrs& p, int R, const float* g_last, const FoldPtrs& last,
                                          int nlast, int64_t e) {
    float L[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        float a = i == R - 1 ? last_replica(p, R, g_last, last, nlast, e) : p.a[i][e];
        if (i + P < R) {
            const float b = i + P == R - 1 ? last_replica(p, R, g_last, last, nlast, e) : p.a[i + P][e];
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
__global__ __launch_bounds__(kStreamThreads) void fold_kernel(FoldPtrs p, int R, const float* g_last, FoldPtrs last,
                                                              int nlast, float* __restrict__ out, int64_t n) {
    const int64_t e = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    if (e < n) out[e] = fold_one<P>(p, R, g_last, last, nlast, e);
}

// Vector version for R = 6 (the replay's mesh): one 16-byte vector of each
// input per thread.  T = ((A0+A4)+(A1+A5))+(A2+A3), A5 first completed with
// the last partial when it is given.
__global__ __launch_bounds__(kStreamThreads) void fold6_v4_kernel(FoldPtrs p, const float* g_last, FoldPtrs last,
                                                                  int nlast, vf4* __restrict__ out, int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    if (i >= n4) return;
    const vf4* a0 = reinterpret_cast<const vf4*>(p.a[0]);
    const vf4* a1 = reinterpret_cast<const vf4*>(p.a[1]);
    const vf4* a2 = reinterpret_cast<const vf4*>(p.a[2]);
    const vf4* a3 = reinterpret_cast<const vf4*>(p.a[3]);
    const vf4* a4 = reinterpret_cast<const vf4*>(p.a[4]);
    vf4 v0 = __builtin_nontemporal_load(a0 + i), v1 = __builtin_nontemporal_load(a1 + i);
    vf4 v2 = __builtin_nontemporal_load(a2 + i), v3 = __builtin_nontemporal_load(a3 + i);
    vf4 v4 = __builtin_nontemporal_load(a4 + i);
    vf4 v5;
    if (nlast > 0) {
        v5 = runsum_vec(last, nlast, i);
    } else {
        v5 = __builtin_nontemporal_load(reinterpret_cast<const vf4*>(p.a[5]) + i);
        if (g_last) {
            const vf4 g = __builtin_nontemporal_load(reinterpret_cast<const vf4*>(g_last) + i);
            v5.x = f_add(v5.x, g.x); v5.y = f_add(v5.y, g.y);
            v5.z = f_add(v5.z, g.z); v5.w = f_add(v5.w, g.w);
        }
    }
    vf4 r;
#define FOLD6(c) r.c = f_add(f_add(f_add(v0.c, v4.c), f_add(v1.c, v5.c)), f_add(v2.c, v3.c))
    FOLD6(x); FOLD6(y); FOLD6(z); FOLD6(w);
#undef FOLD6
    __builtin_nontemporal_store(r, out + i);
}

hipError_t launch_fold(const FoldPtrs& p, int R, const float* g_last, const FoldPtrs& last, int nlast,
                       float* out, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    if (nlast < 0 || nlast > 64) return hipErrorInvalidValue;
    bool al = aligned16(out) && (!g_last || aligned16(g_last));
    // replica R-1's accumulator is read only without resident partials
    for (int i = 0; i < (nlast > 0 ? R - 1 : R); ++i) al = al && aligned16(p.a[i]);
    for (int s = 0; s < nlast; ++s) al = al && aligned16(last.a[s]);
    int64_t done = 0;
    if (R == 6 && al && n >= 4) {
        const int64_t n4 = n / 4;
        hipLaunchKernelGGL(fold6_v4_kernel, dim3(stream_grid(n4, 1)), dim3(kStreamThreads), 0, st, p,
                           g_last, last, nlast, reinterpret_cast<vf4*>(out), n4);
        done = n4 * 4;
    }
    if (done < n) {
        const FoldPtrs q = offset_ptrs(p, R, done);
        const FoldPtrs ql = offset_ptrs(last, nlast, done);
        const float* gl = g_last ? g_last + done : nullptr;
        const int64_t m = n - done;
        const dim3 grid((unsigned)ceil_div(m, kStreamThreads)), blk(kStreamThreads);
        int P = 1;
        while (P * 2 <= R) P *= 2;
        float* o = out + done;
        switch (P) {
            case 1: hipLaunchKernelGGL(fold_kernel<1>, grid, blk, 0, st, q, R, gl, ql, nlast, o, m); break;
            case 2: hipLaunchKernelGGL(fold_kernel<2>, grid, blk, 0, st, q, R, gl, ql, nlast, o, m); break;
            case 4: hipLaunchKernelGGL(fold_kernel<4>, grid, blk, 0, st, q, R, gl, ql, nlast, o, m); break;
            case 8: hipLaunchKernelGGL(fold_kernel<8>, grid, blk, 0, st, q, R, gl, ql, nlast, o, m); break;
            case 16: hipLaunchKernelGGL(fold_kernel<16>, grid, blk, 0, st, q, R, gl, ql, nlast, o, m); break;
            case 32: hipLaunchKernelGGL(fold_kernel<32>, grid, blk, 0, st, q, R, gl, ql, nlast, o, m); break;
            default: hipLaunchKernelGGL(fold_kernel<64>, grid, blk, 0, st, q, R, gl, ql, nlast, o, m); break;
        }
    }
    return hipGetLastError();
}

// g <- g * kappa when the norm exceeded the bound (decided on the device).
template <int V>
__global__ __launch_bounds__(kStreamThreads) void clip_v4_kernel(vf4* __restrict__ g, int64_t n4,
                                                                 const Scalars* __restrict__ s) {
    if (!s->clip) return;
    const float k = s->kappa;
    vf4 v[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int64_t i = vec_index<V>(u);
        if (i < n4) v[u] = __builtin_nontemporal_load(g + i);
    }
#pragma unroll
    for (int u = 0; u < V; ++u) {
        const int64_t i = vec_index<V>(u);
        if (i < n4) {
            vf4 r;
            r.x = f_mul(v[u].x, k); r.y = f_mul(v[u].y, k); r.z = f_mul(v[u].z, k); r.w = f_mul(v[u].w, k);
            __builtin_nontemporal_store(r, g + i);
        }
    }
}

__global__ __launch_bounds__(kStreamThreads) void clip_scalar_kernel(float* __restrict__ g, int64_t n,
                                                                     const Scalars* __restrict__ s) {
    if (!s->clip) return;
    const int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    if (i < n) g[i] = f_mul(g[i], s->kappa);
}

hipError_t launch_clip(float* g, int64_t n, const Scalars* scal, int vec, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t done = 0;
    if (aligned16(g)) {
        const int64_t n4 = n / 4;
        const int V = vec;
        if (n4 > 0) {
            vf4* g4 = reinterpret_cast<vf4*>(g);
            const dim3 grid(stream_grid(n4, V)), blk(kStreamThreads);
            if (V == 4) hipLaunchKernelGGL(clip_v4_kernel<4>, grid, blk, 0, st, g4, n4, scal);
            else if (V == 2) hipLaunchKernelGGL(clip_v4_kernel<2>, grid, blk, 0, st, g4, n4, scal);
            else hipLaunchKernelGGL(clip_v4_kernel<1>, grid, blk, 0, st, g4, n4, scal);
        }
        done = n4 * 4;
    }
    if (done < n)
        hipLaunchKernelGGL(clip_scalar_kernel, dim3((unsigned)ceil_div(n - done, kStreamThreads)),
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
