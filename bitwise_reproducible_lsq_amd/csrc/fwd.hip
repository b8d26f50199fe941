// fwd.hip -- LSQ int8 quantisation-aware linear forward on gfx950.
//
// Method (Open-1B summary on onedev.kr, "Use"): 8-bit weights and activations
// on every attention/FFN linear, the weight step 2*mean(|w|)/sqrt(127)
// recomputed from the weights; the SwiGLU gate and up projections are one
// GEMM.  Numerics ("How"): the dequantisation multiply and any add stay
// separate roundings.
//
// Kernels:
//   quantize_kernel  fp32 -> int8 with the LSQ rounding (RNE, clamp to
//                    [-127,127]); writes zero-padded, GEMM-ready operands.
//   gemm_i8_kernel   int8 x int8 -> exact int32 on v_mfma_i32_32x32x32_i8,
//                    LDS-staged double-buffered tiles, dequantising epilogue
//                    (and the SwiGLU activation when asked).
// The integer product is exact and order-free, so any tiling gives the same
// int32 accumulators; every floating-point step after it is elementwise.
#include "internal.hpp"

#pragma clang fp contract(off)

namespace brl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// ---- quantiser ------------------------------------------------------------------
// Thread -> 16 consecutive columns of one padded output row; grid x walks
// the columns, grid y (with a stride loop) the rows.
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ v, int64_t rows,
                                                       int64_t cols, const float* __restrict__ s_dev,
                                                       float s_host, int8_t* __restrict__ q,
                                                       int64_t rows_p, int64_t cols_p,
                                                       int64_t swiglu_half) {
    const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 16;
    if (c0 >= cols_p) return;
    const float s = s_dev ? *s_dev : s_host;
    const bool vec_rows = ((cols & 3) == 0) && ((reinterpret_cast<uintptr_t>(v) & 15) == 0);
    for (int64_t ro = blockIdx.y; ro < rows_p; ro += gridDim.y) {
        int64_t r = ro;
        bool valid = ro < rows;
        if (swiglu_half > 0) {
            const int64_t t = ro >> 7, w = ro & (2 * kSwigluGroup - 1);
            const int64_t j = t * kSwigluGroup + (w & (kSwigluGroup - 1));
            valid = j < swiglu_half;
            r = (w < kSwigluGroup) ? j : swiglu_half + j;
        }
        union { int8_t b[16]; v4i v; } out;
#pragma unroll
        for (int e = 0; e < 16; ++e) out.b[e] = 0;
        if (valid) {
            const float* src = v + r * cols;
            if (vec_rows && c0 + 16 <= cols) {
                const vf4* s4 = reinterpret_cast<const vf4*>(src + c0);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    vf4 x = s4[g];
                    bool in;
                    out.b[4 * g + 0] = (int8_t)quantize_q(x.x, s, &in);
                    out.b[4 * g + 1] = (int8_t)quantize_q(x.y, s, &in);
                    out.b[4 * g + 2] = (int8_t)quantize_q(x.z, s, &in);
                    out.b[4 * g + 3] = (int8_t)quantize_q(x.w, s, &in);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    if (c0 + e < cols) {
                        bool in;
                        out.b[e] = (int8_t)quantize_q(src[c0 + e], s, &in);
                    }
                }
            }
        }
        *reinterpret_cast<v4i*>(q + ro * cols_p + c0) = out.v;
    }
}

hipError_t launch_quantize(const float* v, int64_t rows, int64_t cols, const float* s_dev,
                           float s_host, int8_t* q, int64_t rows_p, int64_t cols_p,
                           int64_t swiglu_half, hipStream_t st) {
    if (rows_p <= 0 || cols_p <= 0) return hipSuccess;
    const unsigned gx = (unsigned)ceil_div(cols_p / 16, 256);
    const unsigned gy = (unsigned)(rows_p < 65535 ? rows_p : 65535);
    hipLaunchKernelGGL(quantize_kernel, dim3(gx, gy), dim3(256), 0, st, v, rows, cols, s_dev, s_host,
                       q, rows_p, cols_p, swiglu_half);
    return hipGetLastError();
}

// ---- int8 GEMM ---------------------------------------------------------------------
// Workgroup tile BM x BN, K step 64 (two MFMA k-steps of 32), waves of WM x WN,
// each wave a (WM/32) x (WN/32) grid of 32x32 MFMA tiles.
// LDS rows are 64 bytes of k padded to 80 so that 16-byte fragment reads of
// consecutive rows fall in distinct banks.
constexpr int kBK = 64;
constexpr int kLdsPitch = 80;

template <int BM, int BN, int WM, int WN>
struct GemmCfg {
    static constexpr int kWavesM = BM / WM, kWavesN = BN / WN;
    static constexpr int kThreads = kWavesM * kWavesN * 64;
    static constexpr int kTM = WM / 32, kTN = WN / 32;
    static constexpr int kAChunks = BM * (kBK / 16) / kThreads;   // 16-byte chunks per thread
    static constexpr int kBChunks = BN * (kBK / 16) / kThreads;
    static constexpr int kLdsA = BM * kLdsPitch, kLdsB = BN * kLdsPitch;
};

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256, 1) void gemm_i8_kernel(GemmArgs a) {
    using C = GemmCfg<BM, BN, WM, WN>;
    static_assert(C::kThreads == 256, "the GEMM runs 4 waves per workgroup");
    extern __shared__ __attribute__((aligned(16))) int8_t smem[];
    int8_t* As = smem;                       // [2][BM][pitch]
    int8_t* Bs = smem + 2 * C::kLdsA;        // [2][BN][pitch]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / C::kWavesN, wn = wave % C::kWavesN;

    // tile of this workgroup; consecutive ids walk down M inside a column of
    // tiles so that workgroups running together share the weight tile
    const unsigned tilesM = (unsigned)(a.Mp / BM);
    const int64_t tm_ = blockIdx.x % tilesM;
    const int64_t tn_ = blockIdx.x / tilesM;
    const int64_t m0 = tm_ * BM, n0 = tn_ * BN;

    const int8_t* gA = a.qx + m0 * a.Kp;
    const int8_t* gB = a.qw + n0 * a.Kp;
    const int64_t KT = a.Kp / kBK;

    v4i ra[C::kAChunks], rb[C::kBChunks];
    auto gload = [&](int64_t kt) {
#pragma unroll
        for (int c = 0; c < C::kAChunks; ++c) {
            const int idx = tid + c * C::kThreads;
            const int row = idx >> 2, seg = (idx & 3) * 16;
            ra[c] = *reinterpret_cast<const v4i*>(gA + row * a.Kp + kt * kBK + seg);
        }
#pragma unroll
        for (int c = 0; c < C::kBChunks; ++c) {
            const int idx = tid + c * C::kThreads;
            const int row = idx >> 2, seg = (idx & 3) * 16;
            rb[c] = *reinterpret_cast<const v4i*>(gB + row * a.Kp + kt * kBK + seg);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int c = 0; c < C::kAChunks; ++c) {
            const int idx = tid + c * C::kThreads;
            const int row = idx >> 2, seg = (idx & 3) * 16;
            *reinterpret_cast<v4i*>(As + buf * C::kLdsA + row * kLdsPitch + seg) = ra[c];
        }
#pragma unroll
        for (int c = 0; c < C::kBChunks; ++c) {
            const int idx = tid + c * C::kThreads;
            const int row = idx >> 2, seg = (idx & 3) * 16;
            *reinterpret_cast<v4i*>(Bs + buf * C::kLdsB + row * kLdsPitch + seg) = rb[c];
        }
    };

    v16i acc[C::kTM][C::kTN];
#pragma unroll
    for (int i = 0; i < C::kTM; ++i)
#pragma unroll
        for (int j = 0; j < C::kTN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    gload(0);
    sstore(0);
    __syncthreads();

    const int frow = lane & 31;            // fragment row (A) / column (B)
    const int fk = (lane >> 5) * 16;       // byte offset of this lane's 16 k-values
    for (int64_t kt = 0; kt < KT; ++kt) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < KT) gload(kt + 1);
        const int8_t* Ab = As + cur * C::kLdsA + (wm * WM + frow) * kLdsPitch + fk;
        const int8_t* Bb = Bs + cur * C::kLdsB + (wn * WN + frow) * kLdsPitch + fk;
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 32) {
            v4i fa[C::kTM], fb[C::kTN];
#pragma unroll
            for (int i = 0; i < C::kTM; ++i)
                fa[i] = *reinterpret_cast<const v4i*>(Ab + i * 32 * kLdsPitch + kk);
#pragma unroll
            for (int j = 0; j < C::kTN; ++j)
                fb[j] = *reinterpret_cast<const v4i*>(Bb + j * 32 * kLdsPitch + kk);
#pragma unroll
            for (int i = 0; i < C::kTM; ++i)
#pragma unroll
                for (int j = 0; j < C::kTN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) sstore(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: Y = fl(acc) * s_y (+ addend), or the SwiGLU activation ----
    const float s_y = a.scal->s_y;
    const int col_l = lane & 31;
    const int row_q = (lane >> 5) * 4;
    if (a.epilogue == BRL_EPILOGUE_SWIGLU) {
        // wave columns: tiles [0, kTN/2) are gate, [kTN/2, kTN) the matching up
        const int64_t H = a.N / 2;
#pragma unroll
        for (int i = 0; i < C::kTM; ++i)
#pragma unroll
            for (int j = 0; j < C::kTN / 2; ++j) {
                const int64_t vcol = n0 + wn * WN + j * 32 + col_l;       // virtual gate column
                const int64_t gcol = (vcol / (2 * kSwigluGroup)) * kSwigluGroup + (vcol % kSwigluGroup);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = m0 + wm * WM + i * 32 + (r >> 2) * 8 + row_q + (r & 3);
                    if (row < a.M && gcol < H) {
                        float g = f_mul((float)acc[i][j][r], s_y);
                        float u = f_mul((float)acc[i][j + C::kTN / 2][r], s_y);
                        if (a.addend) {
                            g = f_add(g, a.addend[row * a.N + gcol]);
                            u = f_add(u, a.addend[row * a.N + H + gcol]);
                        }
                        if (a.Ypre) {
                            a.Ypre[row * a.N + gcol] = g;
                            a.Ypre[row * a.N + H + gcol] = u;
                        }
                        const float s = swiglu_sigma(g, a.ek);
                        a.Y[row * H + gcol] = f_mul(f_mul(g, s), u);
                    }
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < C::kTM; ++i)
#pragma unroll
            for (int j = 0; j < C::kTN; ++j) {
                const int64_t col = n0 + wn * WN + j * 32 + col_l;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = m0 + wm * WM + i * 32 + (r >> 2) * 8 + row_q + (r & 3);
                    if (row < a.M && col < a.N) {
                        float y = f_mul((float)acc[i][j][r], s_y);
                        if (a.addend) y = f_add(y, a.addend[row * a.N + col]);
                        a.Y[row * a.N + col] = y;
                    }
                }
            }
    }
}

hipError_t launch_gemm_i8(const GemmArgs& a, hipStream_t st) {
    constexpr int BM = 256, BN = 256, WM = 128, WN = 128;
    using C = GemmCfg<BM, BN, WM, WN>;
    static_assert(C::kAChunks * C::kThreads == BM * 4, "A tile load split");
    static_assert(C::kBChunks * C::kThreads == BN * 4, "B tile load split");
    const size_t lds = 2 * (size_t)(C::kLdsA + C::kLdsB);
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_i8_kernel<BM, BN, WM, WN>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        attr = true;
    }
    const int64_t tiles = (a.Mp / BM) * (a.Nvp / BN);
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, WM, WN>), dim3((unsigned)tiles), dim3(C::kThreads), lds,
                       st, a);
    return hipGetLastError();
}

}  // namespace brl
