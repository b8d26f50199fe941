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

// ---- dequantised operand for the backward ------------------------------------------
// out[r][c] = fl(q(v[r][c]) * s) with q the LSQ quantiser, zero rows and
// columns past the data; thread -> 4 consecutive columns of one padded row.
__global__ __launch_bounds__(256) void dequant_kernel(const float* __restrict__ v, int64_t rows, int64_t cols,
                                                      const float* __restrict__ s_dev, float s_host,
                                                      float* __restrict__ out, int64_t rows_p, int64_t cols_p) {
    const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (c0 >= cols_p) return;
    const float s = s_dev ? *s_dev : s_host;
    const bool vec_rows = ((cols & 3) == 0) && ((reinterpret_cast<uintptr_t>(v) & 15) == 0);
    for (int64_t r = blockIdx.y; r < rows_p; r += gridDim.y) {
        vf4 o = {0.0f, 0.0f, 0.0f, 0.0f};
        if (r < rows) {
            const float* src = v + r * cols;
            bool in;
            if (vec_rows && c0 + 4 <= cols) {
                const vf4 x = *reinterpret_cast<const vf4*>(src + c0);
                o.x = f_mul((float)quantize_q(x.x, s, &in), s);
                o.y = f_mul((float)quantize_q(x.y, s, &in), s);
                o.z = f_mul((float)quantize_q(x.z, s, &in), s);
                o.w = f_mul((float)quantize_q(x.w, s, &in), s);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c0 + e < cols) o[e] = f_mul((float)quantize_q(src[c0 + e], s, &in), s);
            }
        }
        *reinterpret_cast<vf4*>(out + r * cols_p + c0) = o;
    }
}

hipError_t launch_dequant(const float* v, int64_t rows, int64_t cols, const float* s_dev, float s_host,
                          float* out, int64_t rows_p, int64_t cols_p, hipStream_t st) {
    if (rows_p <= 0 || cols_p <= 0) return hipSuccess;
    const unsigned gx = (unsigned)ceil_div(cols_p / 4, 256);
    const unsigned gy = (unsigned)(rows_p < 8192 ? rows_p : 8192);
    hipLaunchKernelGGL(dequant_kernel, dim3(gx, gy), dim3(256), 0, st, v, rows, cols, s_dev, s_host, out,
                       rows_p, cols_p);
    return hipGetLastError();
}

// ---- int8 GEMM ---------------------------------------------------------------------
// Workgroup tile BM x BN (256 x 256), K step 64 bytes (two MFMA k-steps of 32),
// 4 waves of 128 x 128, each a 4 x 4 grid of v_mfma_i32_32x32x32_i8 tiles.
// Operand tiles move global -> LDS with global_load_lds_dwordx4 (no staging
// registers) through a ring of kStages LDS stages, so loads run kStages-1
// tiles ahead of the MFMAs.  LDS rows are 64 bytes, unpadded; the four
// 16-byte chunks of row r are stored XOR-swizzled by (r >> 1) & 3, which puts
// the 16-byte fragment reads of 8 consecutive rows in 8 distinct bank groups.
constexpr int kBK = 64;
constexpr int kStages = 4;

template <int BM, int BN, int WM, int WN>
struct GemmCfg {
    static constexpr int kWavesM = BM / WM, kWavesN = BN / WN;
    static constexpr int kThreads = kWavesM * kWavesN * 64;
    static constexpr int kWaves = kThreads / 64;
    static constexpr int kTM = WM / 32, kTN = WN / 32;
    static constexpr int kTileA = BM * kBK, kTileB = BN * kBK;      // bytes per stage
    static constexpr int kStage = kTileA + kTileB;
    // one load instruction moves 64 lanes x 16 bytes = 16 rows of 64 bytes
    static constexpr int kLoadsA = BM / 16 / kWaves, kLoadsB = BN / 16 / kWaves;
    static constexpr int kLoads = kLoadsA + kLoadsB;                // per wave per stage
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 3); }

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_i8_kernel(GemmArgs a) {
    using C = GemmCfg<BM, BN, WM, WN>;
    static_assert(C::kThreads == 256, "the GEMM runs 4 waves per workgroup");
    extern __shared__ __attribute__((aligned(16))) int8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index kept wave-uniform (scalar), so LDS bases for the direct
    // loads are computed on the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::kWavesN, wn = wave % C::kWavesN;

    // tile of this workgroup; consecutive ids walk down M inside a column of
    // tiles so that workgroups running together share the weight tile
    const unsigned tilesM = (unsigned)(a.Mp / BM);
    const int64_t tm_ = blockIdx.x % tilesM;
    const int64_t tn_ = blockIdx.x / tilesM;
    const int64_t m0 = tm_ * BM, n0 = tn_ * BN;

    const int8_t* gA = a.qx + m0 * a.Kp;
    const int8_t* gB = a.qw + n0 * a.Kp;
    const int KT = (int)(a.Kp / kBK);

    // this lane's share of one load instruction: row (lane >> 2) of a 16-row
    // group, LDS slot (lane & 3), holding global chunk swz(row, slot)
    const int lrow = lane >> 2, lslot = lane & 3;
    auto issue = [&](int kt, int stage) {
        int8_t* sA = smem + stage * C::kStage;
        int8_t* sB = sA + C::kTileA;
#pragma unroll
        for (int i = 0; i < C::kLoadsA; ++i) {
            const int r0 = (wave * C::kLoadsA + i) * 16;
            const int r = r0 + lrow;
            const int8_t* g = gA + (int64_t)r * a.Kp + kt * kBK + 16 * swz(r, lslot);
            __builtin_amdgcn_global_load_lds(g, sA + r0 * kBK, 16, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < C::kLoadsB; ++i) {
            const int r0 = (wave * C::kLoadsB + i) * 16;
            const int r = r0 + lrow;
            const int8_t* g = gB + (int64_t)r * a.Kp + kt * kBK + 16 * swz(r, lslot);
            __builtin_amdgcn_global_load_lds(g, sB + r0 * kBK, 16, 0, 0);
        }
    };

    v16i acc[C::kTM][C::kTN];
#pragma unroll
    for (int i = 0; i < C::kTM; ++i)
#pragma unroll
        for (int j = 0; j < C::kTN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int frow = lane & 31;            // fragment row (A) / column (B)
    const int fchunk = lane >> 5;          // this lane's 16-byte k chunk within a 32-k step
    // Fragments of one 32-k step (4 of A, 4 of B) live in registers.  The
    // reads of the next step are issued before the 16 MFMAs of the current
    // one, so LDS latency hides behind matrix work; the barrier that lands
    // the next tile sits between a tile's two steps, with MFMAs in flight.
    using Frag = v4i[C::kTM + C::kTN];
    auto read_frags = [&](int stage, int ks, Frag& F) {
        const int8_t* sA = smem + stage * C::kStage;
        const int8_t* sB = sA + C::kTileA;
        const int chunk = fchunk + 2 * ks;
#pragma unroll
        for (int i = 0; i < C::kTM; ++i) {
            const int r = wm * WM + i * 32 + frow;
            F[i] = *reinterpret_cast<const v4i*>(sA + r * kBK + 16 * swz(r, chunk));
        }
#pragma unroll
        for (int j = 0; j < C::kTN; ++j) {
            const int r = wn * WN + j * 32 + frow;
            F[C::kTM + j] = *reinterpret_cast<const v4i*>(sB + r * kBK + 16 * swz(r, chunk));
        }
    };
    auto mfmas = [&](const Frag& F) {
#pragma unroll
        for (int i = 0; i < C::kTM; ++i)
#pragma unroll
            for (int j = 0; j < C::kTN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(F[i], F[C::kTM + j], acc[i][j], 0, 0, 0);
    };
    // wait until tile t has landed in LDS for every wave (loads of the tiles
    // after it, up to min(KT-1, newest), may stay in flight), then barrier
    auto land = [&](int t, int newest) {
        const int last = newest < KT - 1 ? newest : KT - 1;
        const int ahead = last - t;
        if (ahead >= 2) wait_vmcnt<2 * C::kLoads>();
        else if (ahead == 1) wait_vmcnt<C::kLoads>();
        else wait_vmcnt<0>();
        // bare barrier: a fence here would wait for every load in flight
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };

    static_assert(kBK == 64, "two k-steps per tile");
    Frag F0, F1;
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < KT) issue(s, s);
    land(0, kStages - 2);
    read_frags(0, 0, F0);
    // every tile but the last hands over to the next one; the last is peeled
    // so that the loop body has no branch between LDS reads and their use
    for (int kt = 0; kt < KT - 1; ++kt) {
        read_frags(kt % kStages, 1, F1);
        mfmas(F0);
        // tile kt-1's stage is free once every wave passes this barrier
        land(kt + 1, kt + kStages - 2);
        if (kt + kStages - 1 < KT) issue(kt + kStages - 1, (kt + kStages - 1) % kStages);
        read_frags((kt + 1) % kStages, 0, F0);
        mfmas(F1);
    }
    read_frags((KT - 1) % kStages, 1, F1);
    mfmas(F0);
    mfmas(F1);

    // ---- epilogue: Y = fl(acc) * s_y (+ addend), or the SwiGLU activation ----
    const float s_y = a.scal->s_y;
    const int col_l = lane & 31;
    const int row_q = (lane >> 5) * 4;
    if constexpr (EPI == BRL_EPILOGUE_SWIGLU) {
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
        // whole tile inside Y and no addend: branch-free stores
        const bool full = (m0 + BM <= a.M) && (n0 + BN <= a.N) && !a.addend;
        if (full) {
            float* Yw = a.Y + (m0 + wm * WM + row_q) * a.N + n0 + wn * WN + col_l;
#pragma unroll
            for (int i = 0; i < C::kTM; ++i)
#pragma unroll
                for (int j = 0; j < C::kTN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        Yw[(int64_t)(i * 32 + (r >> 2) * 8 + (r & 3)) * a.N + j * 32] =
                            f_mul((float)acc[i][j][r], s_y);
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
}

template <int EPI>
static hipError_t launch_gemm_epi(const GemmArgs& a, hipStream_t st) {
    constexpr int BM = 256, BN = 256, WM = 128, WN = 128;
    using C = GemmCfg<BM, BN, WM, WN>;
    static_assert(C::kLoadsA * C::kWaves * 16 == BM && C::kLoadsB * C::kWaves * 16 == BN, "load split");
    static_assert(2 * C::kLoads < 64, "vmcnt range");
    const size_t lds = (size_t)kStages * C::kStage;
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_i8_kernel<BM, BN, WM, WN, EPI>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        attr = true;
    }
    const int64_t tiles = (a.Mp / BM) * (a.Nvp / BN);
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, WM, WN, EPI>), dim3((unsigned)tiles), dim3(C::kThreads), lds,
                       st, a);
    return hipGetLastError();
}

hipError_t launch_gemm_i8(const GemmArgs& a, hipStream_t st) {
    if (a.epilogue == BRL_EPILOGUE_SWIGLU) return launch_gemm_epi<BRL_EPILOGUE_SWIGLU>(a, st);
    return launch_gemm_epi<BRL_EPILOGUE_NONE>(a, st);
}

}  // namespace brl
