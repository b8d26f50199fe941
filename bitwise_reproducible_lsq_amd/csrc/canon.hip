// canon.hip -- CanonSum of a flat vector (weight-step mean of |w|, gradient
// squared norm), in the order the method fixes for every reduction (Open-1B
// summary on onedev.kr, "How"): 32-wide blocks summed left to right from their
// first term, then a level-by-level pairwise tree over the block sums.
//
// Work split: pass 1 gives each workgroup an aligned run of WGB block sums and
// reduces them to one subtree root; while more than 4096 roots remain, further
// passes reduce aligned runs of WGB roots (coalesced); one single-workgroup
// pass then reduces the rest (each thread an aligned run of at most 4 roots in
// registers, then the workgroup tree).  Aligned power-of-two runs are
// complete subtrees of the canonical tree (and a short final run is the
// canonical tree of its own leaves), so the result is independent of the
// split.  The last pass also computes the scalar that follows the sum (weight
// step, or norm and clip coefficient).
#include "internal.hpp"

#pragma clang fp contract(off)

namespace brl {

template <int MAP>
__device__ __forceinline__ float canon_map(float v) {
    if constexpr (MAP == kMapAbs) return __builtin_fabsf(v);
    else return f_mul(v, v);
}

// Pass 1: thread t of workgroup w sums block j = w*WGB + t.  The workgroup's
// WGB*32 elements are loaded coalesced (16-byte vectors when aligned) and
// transposed through LDS rows of 33 floats, so that each thread then walks
// its own 32 consecutive elements left to right without bank conflicts.
template <int MAP, int WGB>
__global__ __launch_bounds__(WGB) void canon_pass1_kernel(const float* __restrict__ x, int64_t n,
                                                         float* __restrict__ roots, int last,
                                                         CanonFinishArgs fin) {
    constexpr int kRow = kBlock + 1;
    __shared__ float tile[WGB * kRow];
    __shared__ float lds[WGB];
    const int t = threadIdx.x;
    const int64_t base = (int64_t)blockIdx.x * WGB * kBlock;
    const int64_t avail = n - base;
    const int span = avail < (int64_t)WGB * kBlock ? (int)avail : WGB * kBlock;
    const float* src = x + base;
    if (span == WGB * kBlock && ((reinterpret_cast<uintptr_t>(src) & 15) == 0)) {
        const vf4* s4 = reinterpret_cast<const vf4*>(src);
#pragma unroll
        for (int k = 0; k < kBlock / 4; ++k) {
            const int v = t + k * WGB;              // vector index in the span
            const vf4 q = __builtin_nontemporal_load(s4 + v);
            const int e = 4 * v, b = e >> 5, o = e & 31;
            float* d = &tile[b * kRow + o];
            d[0] = q.x; d[1] = q.y; d[2] = q.z; d[3] = q.w;
        }
    } else {
        for (int e = t; e < span; e += WGB) tile[(e >> 5) * kRow + (e & 31)] = src[e];
    }
    __syncthreads();
    float s = 0.0f;
    const int len = span - t * kBlock;               // elements of this thread's block
    if (len > 0) {
        const float* p = &tile[t * kRow];
        s = canon_map<MAP>(p[0]);
        if (len >= kBlock) {
#pragma unroll
            for (int i = 1; i < kBlock; ++i) s = f_add(s, canon_map<MAP>(p[i]));
        } else {
            for (int i = 1; i < len; ++i) s = f_add(s, canon_map<MAP>(p[i]));
        }
    }
    const int64_t J = (n + kBlock - 1) / kBlock;
    const int64_t rem = J - (int64_t)blockIdx.x * WGB;
    const int count = rem < WGB ? (int)(rem < 0 ? 0 : rem) : WGB;
    float r = wg_pair_tree(s, count, lds);
    if (t == 0) {
        if (last) canon_finish(r, fin);
        else roots[blockIdx.x] = r;
    }
}

// Later passes: aligned runs of WGB roots.
template <int WGB>
__global__ __launch_bounds__(WGB) void canon_tree_kernel(const float* __restrict__ in, int64_t Q,
                                                        float* __restrict__ out, int last,
                                                        CanonFinishArgs fin) {
    __shared__ float lds[WGB];
    const int64_t j = (int64_t)blockIdx.x * WGB + threadIdx.x;
    float s = j < Q ? in[j] : 0.0f;
    int64_t rem = Q - (int64_t)blockIdx.x * WGB;
    const int count = rem < WGB ? (int)rem : WGB;
    float r = wg_pair_tree(s, count, lds);
    if (threadIdx.x == 0) {
        if (last) canon_finish(r, fin);
        else out[blockIdx.x] = r;
    }
}

// Final pass in one workgroup of kTailThreads: thread t first reduces the
// aligned run of RUN roots [t*RUN, (t+1)*RUN) in registers, level by level
// (a complete subtree, or for the short last run the canonical tree of its
// own leaves), then the workgroup tree combines the run roots.  One launch
// replaces the chain of canon_tree_kernel passes once Q <= kTailThreads*RUN.
// Runs stay short: each thread's loads are strided by RUN, and longer runs
// (measured: 32 roots per thread, 15.7 us) cost more than a coalesced pass.
constexpr int kTailThreads = 1024;
constexpr int kTailMaxRun = 4;

template <int RUN>
__global__ __launch_bounds__(kTailThreads) void canon_tail_kernel(const float* __restrict__ in, int64_t Q,
                                                                  CanonFinishArgs fin) {
    __shared__ float lds[kTailThreads];
    const float r = canon_runs_tree<RUN>([&](int64_t j) { return in[j]; }, Q, lds);
    if (threadIdx.x == 0) canon_finish(r, fin);
}

static hipError_t launch_canon_tail(const float* in, int64_t Q, const CanonFinishArgs& fin, hipStream_t st) {
    int run = 1;
    while ((int64_t)run * kTailThreads < Q) run *= 2;
    const dim3 g(1), b(kTailThreads);
    switch (run) {
        case 1: hipLaunchKernelGGL(canon_tail_kernel<1>, g, b, 0, st, in, Q, fin); break;
        case 2: hipLaunchKernelGGL(canon_tail_kernel<2>, g, b, 0, st, in, Q, fin); break;
        case 4: hipLaunchKernelGGL(canon_tail_kernel<4>, g, b, 0, st, in, Q, fin); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int64_t canon_partials(int64_t n) {
    const int64_t wgb = 64;   // smallest allowed WGB gives the largest count
    int64_t J = ceil_div(n, kBlock);
    int64_t q = ceil_div(J, wgb);
    int64_t total = q + 1;
    while (q > 1) { q = ceil_div(q, wgb); total += q + 1; }
    return total + 64;
}

template <int WGB>
static hipError_t canon_run(int map, const float* x, int64_t n, float* partials,
                            const CanonFinishArgs& fin, hipStream_t st) {
    const int64_t J = ceil_div(n, kBlock);
    int64_t q = J > 0 ? ceil_div(J, WGB) : 1;
    int last = q == 1;
    if (map == kMapAbs)
        hipLaunchKernelGGL((canon_pass1_kernel<kMapAbs, WGB>), dim3((unsigned)q), dim3(WGB), 0, st,
                           x, n, partials, last, fin);
    else
        hipLaunchKernelGGL((canon_pass1_kernel<kMapSquare, WGB>), dim3((unsigned)q), dim3(WGB), 0, st,
                           x, n, partials, last, fin);
    float* in = partials;
    float* out = partials + q + 1;
    while (q > (int64_t)kTailThreads * kTailMaxRun) {
        int64_t nq = ceil_div(q, WGB);
        hipLaunchKernelGGL((canon_tree_kernel<WGB>), dim3((unsigned)nq), dim3(WGB), 0, st,
                           in, q, out, 0, fin);
        in = out;
        out = out + nq + 1;
        q = nq;
    }
    if (q > 1) return launch_canon_tail(in, q, fin, st);
    return hipGetLastError();
}

hipError_t launch_canon(int map, const float* x, int64_t n, float* partials,
                        const CanonFinishArgs& fin, int wg_blocks, hipStream_t st) {
    switch (wg_blocks) {
        case 64: return canon_run<64>(map, x, n, partials, fin, st);
        case 128: return canon_run<128>(map, x, n, partials, fin, st);
        default: return canon_run<256>(map, x, n, partials, fin, st);
    }
}

}  // namespace brl
