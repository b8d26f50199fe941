// bwd.hip -- straight-through backward of the int8 LSQ linear layer on gfx950.
//
// dX[m,k] = in_x ? CanonSum_n(G[m,n] * What[n,k]) : +0
// dW[n,k] = in_w ? CanonSum_m(G[m,n] * Xhat[m,k]) : +0
// with What = fl(q_w*s_w), Xhat = fl(q_x*s_x) and CanonSum the method's fixed
// order (Open-1B summary on onedev.kr, "How": one reduction order, multiply
// and add never fused, FTZ).  Every product is rounded on its own and every
// add is one binary32 add in a fixed sequence.
//
// Two engines give the same bits:
//
// ste_mfma_kernel<A_RMAJ, D> (matrix cores for the products): a 16x16x1 fp32
// MFMA with a K of one and an accumulator input of -0 returns fl(a*b) for
// each of its 1024 (a, b) pairs -- one product, one rounding, and -0 is the
// exact additive identity -- which on gfx950 (FTZ mode) is bit-identical to
// v_mul_f32, so the matrix cores form the products and the VALU only adds
// them, in order, into the running block sums.  Workgroup tile 64x64, wave w
// owns columns 16w..16w+15 of all 64 rows (4 MFMA blocks of 16x16 stacked
// in rows sharing the B values); lane l feeds A row l and B column l % 16 and
// receives 16 outputs.  Operand blocks move global -> LDS with direct loads
// (no staging registers) through a 3-stage ring; B comes pre-dequantised.
//
// ste_chunk_kernel<A_RMAJ, D> (VALU products; any shape and alignment): a
// workgroup of 256 threads owns a 64x64 output tile, each thread 4x4 outputs
// (4 consecutive rows, 4 consecutive columns).  Per 32-block it streams the
// block's 32 reduction steps from LDS (A as [r][i] and B as [r][j], pitch 68,
// both double-buffered; dX's A arrives i-major and is transposed on the LDS
// store, B is dequantised on the store), forming the block sums left to right
// from the first product.
//
// Both: a workgroup owns one chunk of 2^D consecutive 32-blocks of the
// reduction; finished block sums enter a binary-counter stack of depth D held
// in registers, which builds exactly the pairwise tree of the chunk.  An
// aligned run of 2^D blocks is a complete subtree of the canonical tree (a
// short last run is the canonical tree of its own blocks), so the chunk roots
// combined by the same pairwise tree (ste_finish_kernel) give the canonical
// result for any D.  Reduction steps past the end read A = -0 and B = +0,
// whose product -0 leaves every binary32 sum unchanged.
#include "internal.hpp"

#pragma clang fp contract(off)

namespace brl {

constexpr int kTile = 64;         // output tile edge per workgroup
constexpr int kPitchAr = 68;      // floats per LDS row of A ([r][64 i] + pad)
constexpr int kLdsA = kBlock * kPitchAr;
constexpr int kPitchB = 68;       // floats per LDS row of B ([r][64 j] + pad)
constexpr int kFinishLevels = 10; // finish pass handles up to 2^10 chunk roots

// Binary-counter stack: after block index bi (0-based) completes with value t,
// merge it with the stored subtrees of equal size.  st[L] is valid while bit L
// of the completed-block count is set.  V is a float or a clang float vector
// (elementwise binary32 adds).
template <class V, int L, int D>
__device__ __forceinline__ void stack_push(V (&st)[D + 1], V& t, unsigned bi) {
    if constexpr (L == D) {
        st[D] = t;
    } else {
        if (bi & (1u << L)) {
            t = st[L] + t;
            stack_push<V, L + 1, D>(st, t, bi);
        } else {
            st[L] = t;
        }
    }
}

// Final right-to-left merge of the stored subtrees for `count` blocks.
template <class V, int L, int D>
__device__ __forceinline__ void stack_final(const V (&st)[D + 1], unsigned count, V& root, bool have) {
    if constexpr (L <= D) {
        if (count & (1u << L)) {
            root = have ? st[L] + root : st[L];
            have = true;
        }
        stack_final<V, L + 1, D>(st, count, root, have);
    }
}

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float vf1 __attribute__((ext_vector_type(1)));

__device__ __forceinline__ float mask_select(float v, const float* src, int64_t idx,
                                             const float* s_dev, float s_host) {
    const float s = s_dev ? *s_dev : s_host;
    return Quantizer(s).in_range(src[idx]) ? v : 0.0f;
}

template <bool A_RMAJ, int D>
__global__ __launch_bounds__(256) void ste_chunk_kernel(SteArgs a, int64_t nblk, int final_out) {
    __shared__ __attribute__((aligned(16))) float As[2][kLdsA];
    __shared__ __attribute__((aligned(16))) float Bs[2][kBlock * kPitchB];

    const int tid = threadIdx.x;
    const int tj = tid & 15, ti = tid >> 4;
    const int64_t j0 = (int64_t)blockIdx.x * kTile;
    const int64_t i0 = (int64_t)blockIdx.y * kTile;
    const int64_t chunk = blockIdx.z;
    const int64_t b_begin = chunk << D;
    const int64_t b_end = (b_begin + (1 << D)) < nblk ? (b_begin + (1 << D)) : nblk;
    const float bscale = a.b_scale_dev ? *a.b_scale_dev : a.b_scale_host;

    // global -> register staging for one 32-block
    float ra[8];
    uint2 rb;
    // A whole 32-block inside the operand (every row of the tile, every
    // reduction step) loads without per-element predicates; 16-byte vectors
    // when the host saw the rows 16-byte aligned.
    const bool rows_full = i0 + kTile <= a.I;
    auto gload = [&](int64_t blk) {
        const int64_t r0 = blk * kBlock;
        if (rows_full && r0 + kBlock <= a.R) {
            const float* p;
            if constexpr (A_RMAJ)
                p = a.A + (i0 + (tid >> 2)) * a.lda + r0 + (tid & 3) * 8;
            else
                p = a.A + (r0 + (tid >> 3)) * a.lda + i0 + (tid & 7) * 8;
            if (a.a_vec) {
                const float4 u = reinterpret_cast<const float4*>(p)[0];
                const float4 v = reinterpret_cast<const float4*>(p)[1];
                ra[0] = u.x; ra[1] = u.y; ra[2] = u.z; ra[3] = u.w;
                ra[4] = v.x; ra[5] = v.y; ra[6] = v.z; ra[7] = v.w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) ra[e] = p[e];
            }
        } else if constexpr (A_RMAJ) {
            // A(r, i) = A[i*lda + r]: row ii, 8 consecutive r
            const int ii = tid >> 2, seg = (tid & 3) * 8;
            const int64_t i = i0 + ii, r = r0 + seg;
            const float* p = a.A + i * a.lda + r;
#pragma unroll
            for (int e = 0; e < 8; ++e) ra[e] = (i < a.I && r + e < a.R) ? p[e] : -0.0f;
        } else {
            // A(r, i) = A[r*lda + i]: row rr, 8 consecutive i
            const int rr = tid >> 3, seg = (tid & 7) * 8;
            const int64_t r = r0 + rr, i = i0 + seg;
            const float* p = a.A + r * a.lda + i;
#pragma unroll
            for (int e = 0; e < 8; ++e) ra[e] = (r < a.R && i + e < a.I) ? p[e] : -0.0f;
        }
        {
            const int rr = tid >> 3, seg = (tid & 7) * 8;
            rb = *reinterpret_cast<const uint2*>(a.Bq + (r0 + rr) * a.ldb + j0 + seg);
        }
    };
    auto sstore = [&](int buf) {
        if constexpr (A_RMAJ) {
            // transpose into the r-major tile: 8 consecutive r of row ii
            const int ii = tid >> 2, seg = (tid & 3) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) As[buf][(seg + e) * kPitchAr + ii] = ra[e];
        } else {
            // r-major like the source: row rr, 8 consecutive i
            const int rr = tid >> 3, seg = (tid & 7) * 8;
            float4* d = reinterpret_cast<float4*>(&As[buf][rr * kPitchAr + seg]);
            d[0] = make_float4(ra[0], ra[1], ra[2], ra[3]);
            d[1] = make_float4(ra[4], ra[5], ra[6], ra[7]);
        }
        {
            const int rr = tid >> 3, seg = (tid & 7) * 8;
            float f[8];
            const uint32_t w0 = rb.x, w1 = rb.y;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[e] = f_mul((float)(int8_t)(w0 >> (8 * e)), bscale);
                f[4 + e] = f_mul((float)(int8_t)(w1 >> (8 * e)), bscale);
            }
            float4* d = reinterpret_cast<float4*>(&Bs[buf][rr * kPitchB + seg]);
            d[0] = make_float4(f[0], f[1], f[2], f[3]);
            d[1] = make_float4(f[4], f[5], f[6], f[7]);
        }
    };

    v16f st[D + 1];
    v16f acc;

    gload(b_begin);
    sstore(0);
    __syncthreads();

    for (int64_t blk = b_begin; blk < b_end; ++blk) {
        const int cur = (int)((blk - b_begin) & 1);
        if (blk + 1 < b_end) gload(blk + 1);
        const float* Ab = &As[cur][0];
        const float* Bb = &Bs[cur][tj * 4];
#pragma unroll
        for (int rs = 0; rs < kBlock; rs += 4) {
            // av[s]: A of this thread's 4 rows at step rs+s; bv[s]: its 4 columns of B
            float4 av[4], bv[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) av[s] = *reinterpret_cast<const float4*>(Ab + (rs + s) * kPitchAr + 4 * ti);
#pragma unroll
            for (int s = 0; s < 4; ++s) bv[s] = *reinterpret_cast<const float4*>(Bb + (rs + s) * kPitchB);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 asrc = av[s];
                    const float x = q == 0 ? asrc.x : q == 1 ? asrc.y : q == 2 ? asrc.z : asrc.w;
                    const float p0 = f_mul(x, bv[s].x), p1 = f_mul(x, bv[s].y);
                    const float p2 = f_mul(x, bv[s].z), p3 = f_mul(x, bv[s].w);
                    if (rs == 0 && s == 0) {
                        acc[4 * q + 0] = p0; acc[4 * q + 1] = p1;
                        acc[4 * q + 2] = p2; acc[4 * q + 3] = p3;
                    } else {
                        acc[4 * q + 0] = f_add(acc[4 * q + 0], p0);
                        acc[4 * q + 1] = f_add(acc[4 * q + 1], p1);
                        acc[4 * q + 2] = f_add(acc[4 * q + 2], p2);
                        acc[4 * q + 3] = f_add(acc[4 * q + 3], p3);
                    }
                }
            }
        }
        stack_push<v16f, 0, D>(st, acc, (unsigned)(blk - b_begin));
        if (blk + 1 < b_end) sstore(cur ^ 1);
        __syncthreads();
    }

    v16f root;
    stack_final<v16f, 0, D>(st, (unsigned)(b_end - b_begin), root, false);

    const int64_t plane = a.I * a.Jn;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t i = i0 + 4 * ti + q;
        if (i >= a.I) continue;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t j = j0 + tj * 4 + c;
            if (j >= a.Jn) continue;
            const int64_t idx = i * a.Jn + j;
            float v = root[4 * q + c];
            if (final_out) {
                v = mask_select(v, a.mask_src, idx, a.mask_scale_dev, a.mask_scale_host);
                if (a.accumulate) v = f_add(a.out[idx], v);
                a.out[idx] = v;
            } else {
                a.roots[chunk * plane + idx] = v;
            }
        }
    }
}

// ---- matrix-core products ---------------------------------------------------------
constexpr int kMStages = 3;                       // LDS ring depth (blocks in flight: 2)
constexpr int kMTileA = kTile * kBlock;           // floats of A per block (64 x 32)
constexpr int kMTileB = kBlock * kTile;           // floats of B per block (32 x 64)
constexpr int kMStage = kMTileA + kMTileB;        // 16 KB

// Source of the 16-byte pieces of A past the end of the reduction.
__device__ __attribute__((aligned(16))) float kNegZero4[4] = {-0.0f, -0.0f, -0.0f, -0.0f};

// i-major A tile: row i holds 8 chunks of 4 reduction steps, chunk c stored
// at slot c ^ ((i >> 1) & 7), so the 16-byte reads of 16 consecutive rows hit
// 16 distinct bank groups.
__device__ __forceinline__ int mswz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

template <bool A_RMAJ, int D>
__global__ __launch_bounds__(256, 3) void ste_mfma_kernel(SteArgs a, int64_t nblk, int final_out) {
    __shared__ __attribute__((aligned(16))) float smem[kMStages * kMStage];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t j0 = (int64_t)blockIdx.x * kTile;
    const int64_t i0 = (int64_t)blockIdx.y * kTile;
    const int64_t chunk = blockIdx.z;
    const int64_t b_begin = chunk << D;
    const int64_t b_end = (b_begin + (1 << D)) < nblk ? (b_begin + (1 << D)) : nblk;

    // Direct loads of one 32-block into a stage: per operand 8 KB = 8 groups
    // of 1 KB, wave w moving groups w and w + 4 (64 lanes x 16 bytes each).
    // A 16-byte piece of A holds 4 consecutive reduction steps (dX, R % 4 ==
    // 0) or 4 consecutive rows (dW, I % 4 == 0), so each piece is wholly
    // inside or outside the operand.  Pieces past R load four -0 from
    // kNegZero4 (then A = -0 meets B = +0 in B's zero padding: product -0);
    // pieces of rows past I load element 0 of a valid row and only feed
    // outputs that are never stored.
    auto issue = [&](int64_t blk, int stage) {
        float* sA = smem + stage * kMStage;
        float* sB = sA + kMTileA;
        const int64_t r0 = blk * kBlock;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int g = k * 4 + wave;
            const float* src;
            if constexpr (A_RMAJ) {
                // G[i][r]: group g = rows 8g..8g+7, lane -> (row, slot)
                const int row = g * 8 + (lane >> 3), c = mswz(row, lane & 7);
                int64_t i = i0 + row;
                const int64_t r = r0 + 4 * c;
                if (i >= a.I) i = a.I - 1;
                src = r < a.R ? a.A + i * a.lda + r : kNegZero4;
            } else {
                // G[r][i]: group g = reduction rows 4g..4g+3, 16 chunks each
                const int row = g * 4 + (lane >> 4);
                const int64_t r = r0 + row;
                int64_t i = i0 + 4 * (lane & 15);
                if (i >= a.I) i = 0;
                src = r < a.R ? a.A + r * a.lda + i : kNegZero4;
            }
            __builtin_amdgcn_global_load_lds(src, sA + g * 256, 16, 0, 0);
            const int brow = g * 4 + (lane >> 4);
            const float* bsrc = a.Bf + (r0 + brow) * a.ldb + j0 + 4 * (lane & 15);
            __builtin_amdgcn_global_load_lds(bsrc, sB + g * 256, 16, 0, 0);
        }
    };
    constexpr int kLoads = 4;   // direct loads per wave per block

    v16f cneg;
#pragma unroll
    for (int r = 0; r < 16; ++r) cneg[r] = -0.0f;
    v16f st[D + 1];
    v16f acc;

    const int bcol = 16 * wave + (lane & 15);
    issue(b_begin, 0);
    if (b_begin + 1 < b_end) issue(b_begin + 1, 1);

    for (int64_t blk = b_begin; blk < b_end; ++blk) {
        const int t = (int)(blk - b_begin);
        const int stage = t % kMStages;
        // block blk landed for this wave (the next one may stay in flight),
        // then for every wave; the stage written next was read in the
        // previous iteration, which every wave has finished
        if (blk + 1 < b_end) wait_vmcnt<kLoads>();
        else wait_vmcnt<0>();
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        if (blk + 2 < b_end) issue(blk + 2, (t + 2) % kMStages);

        const float* sA = smem + stage * kMStage;
        const float* sB = sA + kMTileA;

        // operands of 4 steps are read one group ahead; the product of step
        // s+1 is formed (into the other of two product buffers) before the
        // adds of step s, so matrix-core and VALU work of one wave interleave
        float av[kBlock], bv[kBlock];
        auto read_group = [&](int rs) {
            if constexpr (A_RMAJ) {
                const vf4 v = *reinterpret_cast<const vf4*>(sA + lane * kBlock + 4 * mswz(lane, rs >> 2));
                av[rs] = v.x; av[rs + 1] = v.y; av[rs + 2] = v.z; av[rs + 3] = v.w;
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) av[rs + s] = sA[(rs + s) * kTile + lane];
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) bv[rs + s] = sB[(rs + s) * kTile + bcol];
        };
        v16f p[2];
        read_group(0);
        p[0] = __builtin_amdgcn_mfma_f32_16x16x1f32(av[0], bv[0], cneg, 0, 0, 0);
#pragma unroll
        for (int s = 0; s < kBlock; ++s) {
            if ((s & 3) == 0 && s + 4 < kBlock) read_group(s + 4);
            if (s + 1 < kBlock) p[(s + 1) & 1] = __builtin_amdgcn_mfma_f32_16x16x1f32(av[s + 1], bv[s + 1], cneg, 0, 0, 0);
            if (s == 0) acc = p[0];
            else acc = acc + p[s & 1];
        }
        stack_push<v16f, 0, D>(st, acc, (unsigned)t);
    }

    v16f root;
    stack_final<v16f, 0, D>(st, (unsigned)(b_end - b_begin), root, false);

    // lane l, register 4*beta + e holds row 16*beta + 4*(l / 16) + e, column l % 16
    const int64_t plane = a.I * a.Jn;
    const int64_t j = j0 + bcol;
    if (j < a.Jn) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t i = i0 + 16 * (r >> 2) + 4 * (lane >> 4) + (r & 3);
            if (i >= a.I) continue;
            const int64_t idx = i * a.Jn + j;
            float v = root[r];
            if (final_out) {
                v = mask_select(v, a.mask_src, idx, a.mask_scale_dev, a.mask_scale_host);
                if (a.accumulate) v = f_add(a.out[idx], v);
                a.out[idx] = v;
            } else {
                a.roots[chunk * plane + idx] = v;
            }
        }
    }
}

// Conformance probe of the matrix-core product: each wave takes 64 pairs,
// lane l feeding a[l] as A row l and b[l] as B column l % 16 of the 16x16x1
// MFMA (four 16x16 blocks, block beta = lanes 16beta..16beta+15, C = -0).
// The product of pair 16beta + t sits at row t, column t of block beta: lane
// 16(t/4) + t, register 4beta + t%4.
__global__ __launch_bounds__(64) void probe_mfma_kernel(const float* __restrict__ a, const float* __restrict__ b,
                                                        float* __restrict__ out, int64_t n) {
    const int lane = threadIdx.x;
    const int64_t base = (int64_t)blockIdx.x * 64;
    const float x = base + lane < n ? a[base + lane] : 0.0f;
    // B column c of block beta comes from lane 16beta + c: give it b of pair 16beta + c
    const float y = base + lane < n ? b[base + lane] : 0.0f;
    v16f cneg;
#pragma unroll
    for (int r = 0; r < 16; ++r) cneg[r] = -0.0f;
    const v16f d = __builtin_amdgcn_mfma_f32_16x16x1f32(x, y, cneg, 0, 0, 0);
    const int t = lane & 15;
    if (lane == 16 * (t >> 2) + t) {
#pragma unroll
        for (int beta = 0; beta < 4; ++beta) {
            const int64_t i = base + 16 * beta + t;
            const int r = 4 * beta + (t & 3);
            if (i < n) out[i] = d[r];
        }
    }
}

hipError_t launch_probe_mfma(const float* a, const float* b, float* out, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)ceil_div(n, 64)), dim3(64), 0, st, a, b, out, n);
    return hipGetLastError();
}

// Pairwise tree over the Q chunk roots of each output, then mask (+ running
// sum).  V consecutive outputs per thread (V = 4 needs the plane size to be a
// multiple of 4 so that every root vector is 16-byte aligned); the roots of
// up to 8 chunks are loaded before they enter the stack.
template <class T, int V>
__global__ __launch_bounds__(256) void ste_finish_kernel(SteArgs a, int64_t Q) {
    const int64_t plane = a.I * a.Jn;
    const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
    if (idx >= plane) return;
    T st[kFinishLevels + 1];
    for (int64_t c0 = 0; c0 < Q; c0 += 8) {
        T t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (c0 + u < Q) t[u] = *reinterpret_cast<const T*>(a.roots + (c0 + u) * plane + idx);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (c0 + u < Q) stack_push<T, 0, kFinishLevels>(st, t[u], (unsigned)(c0 + u));
    }
    T root;
    stack_final<T, 0, kFinishLevels>(st, (unsigned)Q, root, false);
    // one quantiser per thread (its reciprocals are formed once); the mask on
    // the fast path, redone on the exact one for a wave with a value whose
    // quotient lies near +-127; 16-byte mask loads and output stores when
    // both tensors allow them
    const Quantizer qz(a.mask_scale_dev ? *a.mask_scale_dev : a.mask_scale_host);
    const bool vec = V == 4 && ((reinterpret_cast<uintptr_t>(a.mask_src) | reinterpret_cast<uintptr_t>(a.out)) & 15) == 0;
    if constexpr (V == 4) {
        if (vec) {
            const vf4 x = *reinterpret_cast<const vf4*>(a.mask_src + idx);
            vf4 o;
            bool unsure = false;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = qz.in_range_fast(x[e], &unsure) ? root[e] : 0.0f;
            if (__ballot(unsure)) {
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = qz.in_range(x[e]) ? root[e] : 0.0f;
            }
            if (a.accumulate) {
                const vf4 prev = *reinterpret_cast<const vf4*>(a.out + idx);
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = f_add(prev[e], o[e]);
            }
            *reinterpret_cast<vf4*>(a.out + idx) = o;
            return;
        }
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
        float v = qz.in_range(a.mask_src[idx + e]) ? root[e] : 0.0f;
        if (a.accumulate) v = f_add(a.out[idx + e], v);
        a.out[idx + e] = v;
    }
}

int64_t ste_chunks(int64_t R, int D) {
    return ceil_div(ceil_div(R, kBlock), (int64_t)1 << D);
}

int64_t ste_root_floats(int64_t I, int64_t R, int64_t Jn, int D) {
    const int64_t Q = ste_chunks(R, D);
    return Q > 1 ? Q * I * Jn : 0;
}

// Empty reduction (no rows): every output is CanonSum of nothing = +0.
__global__ __launch_bounds__(256) void ste_empty_kernel(float* __restrict__ out, int64_t n, int accumulate) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n) return;
    out[idx] = accumulate ? f_add(out[idx], 0.0f) : 0.0f;
}

template <bool A_RMAJ>
static void ste_launch_chunk(const SteArgs& a, int D, dim3 grid, int64_t nblk, int final_out, hipStream_t st) {
    switch (D) {
        case 1: hipLaunchKernelGGL((ste_chunk_kernel<A_RMAJ, 1>), grid, dim3(256), 0, st, a, nblk, final_out); break;
        case 2: hipLaunchKernelGGL((ste_chunk_kernel<A_RMAJ, 2>), grid, dim3(256), 0, st, a, nblk, final_out); break;
        case 3: hipLaunchKernelGGL((ste_chunk_kernel<A_RMAJ, 3>), grid, dim3(256), 0, st, a, nblk, final_out); break;
        case 4: hipLaunchKernelGGL((ste_chunk_kernel<A_RMAJ, 4>), grid, dim3(256), 0, st, a, nblk, final_out); break;
        case 6: hipLaunchKernelGGL((ste_chunk_kernel<A_RMAJ, 6>), grid, dim3(256), 0, st, a, nblk, final_out); break;
        case 7: hipLaunchKernelGGL((ste_chunk_kernel<A_RMAJ, 7>), grid, dim3(256), 0, st, a, nblk, final_out); break;
        default: hipLaunchKernelGGL((ste_chunk_kernel<A_RMAJ, 5>), grid, dim3(256), 0, st, a, nblk, final_out); break;
    }
}

template <bool A_RMAJ>
static void ste_launch_mfma(const SteArgs& a, int D, dim3 grid, int64_t nblk, int final_out, hipStream_t st) {
    switch (D) {
        case 1: hipLaunchKernelGGL((ste_mfma_kernel<A_RMAJ, 1>), grid, dim3(256), 0, st, a, nblk, final_out); break;
        case 2: hipLaunchKernelGGL((ste_mfma_kernel<A_RMAJ, 2>), grid, dim3(256), 0, st, a, nblk, final_out); break;
        case 3: hipLaunchKernelGGL((ste_mfma_kernel<A_RMAJ, 3>), grid, dim3(256), 0, st, a, nblk, final_out); break;
        case 4: hipLaunchKernelGGL((ste_mfma_kernel<A_RMAJ, 4>), grid, dim3(256), 0, st, a, nblk, final_out); break;
        case 6: hipLaunchKernelGGL((ste_mfma_kernel<A_RMAJ, 6>), grid, dim3(256), 0, st, a, nblk, final_out); break;
        case 7: hipLaunchKernelGGL((ste_mfma_kernel<A_RMAJ, 7>), grid, dim3(256), 0, st, a, nblk, final_out); break;
        default: hipLaunchKernelGGL((ste_mfma_kernel<A_RMAJ, 5>), grid, dim3(256), 0, st, a, nblk, final_out); break;
    }
}

hipError_t launch_ste(const SteArgs& a, int engine, int D, hipStream_t st) {
    if (a.I <= 0 || a.Jn <= 0) return hipSuccess;
    if (D < 1 || D > 7) return hipErrorInvalidValue;
    const int64_t nblk = ceil_div(a.R, kBlock);
    if (nblk == 0) {
        const int64_t plane = a.I * a.Jn;
        hipLaunchKernelGGL(ste_empty_kernel, dim3((unsigned)ceil_div(plane, 256)), dim3(256), 0, st,
                           a.out, plane, a.accumulate);
        return hipGetLastError();
    }
    const int64_t Q = ceil_div(nblk, (int64_t)1 << D);
    dim3 grid((unsigned)ceil_div(a.Jn, kTile), (unsigned)ceil_div(a.I, kTile), (unsigned)Q);
    const int final_out = Q == 1;
    if (engine == 2) {
        if (a.a_rmaj) ste_launch_mfma<true>(a, D, grid, nblk, final_out, st);
        else ste_launch_mfma<false>(a, D, grid, nblk, final_out, st);
    } else {
        if (a.a_rmaj) ste_launch_chunk<true>(a, D, grid, nblk, final_out, st);
        else ste_launch_chunk<false>(a, D, grid, nblk, final_out, st);
    }
    if (!final_out) {
        const int64_t plane = a.I * a.Jn;
        if (plane % 4 == 0)
            hipLaunchKernelGGL((ste_finish_kernel<vf4, 4>), dim3((unsigned)ceil_div(plane / 4, 256)), dim3(256), 0,
                               st, a, Q);
        else
            hipLaunchKernelGGL((ste_finish_kernel<vf1, 1>), dim3((unsigned)ceil_div(plane, 256)), dim3(256), 0, st,
                               a, Q);
    }
    return hipGetLastError();
}

// ---- SwiGLU backward (pre-activation gradient) ---------------------------------
// du = dA*h, dg = (dA*u) * (s*(1 + g*(1 - s))), s = 1/(1 + E(-g)), h = g*s.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ dA,
                                                         const float* __restrict__ ypre, int64_t M,
                                                         int64_t N, float* __restrict__ G, ExpConsts ek) {
    const int64_t H = N / 2;
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= H) return;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        const float g = ypre[m * N + j], u = ypre[m * N + H + j], d = dA[m * H + j];
        const float s = swiglu_sigma(g, ek);
        const float h = f_mul(g, s);
        G[m * N + H + j] = f_mul(d, h);
        const float ds = f_mul(s, f_add(1.0f, f_mul(g, f_sub(1.0f, s))));
        G[m * N + j] = f_mul(f_mul(d, u), ds);
    }
}

hipError_t launch_swiglu_bwd(const float* dA, const float* ypre, int64_t M, int64_t N, float* G,
                             const ExpConsts& ek, hipStream_t st) {
    const int64_t H = N / 2;
    if (M <= 0 || H <= 0) return hipSuccess;
    const unsigned gy = (unsigned)(M < 65535 ? M : 65535);
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)ceil_div(H, 256), gy), dim3(256), 0, st, dA,
                       ypre, M, N, G, ek);
    return hipGetLastError();
}

}  // namespace brl
