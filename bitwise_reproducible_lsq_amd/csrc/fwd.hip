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
// Thread -> 4 consecutive columns (one 16-byte load, one 4-byte store) of
// kQRows padded output rows, whose loads are all issued before any of them
// is quantised; grid x walks the column quads, grid y (with a stride loop)
// the row blocks.  A wave reads 1 KiB and writes 256 B contiguously.
constexpr int kQRows = 4;

__device__ __forceinline__ int64_t quantize_src_row(int64_t ro, int64_t rows, int64_t swiglu_half, bool* valid) {
    if (swiglu_half > 0) {
        // stacked gate/up weight rows interleaved in groups of kSwigluGroup
        const int64_t t = ro >> 7, w = ro & (2 * kSwigluGroup - 1);
        const int64_t j = t * kSwigluGroup + (w & (kSwigluGroup - 1));
        *valid = j < swiglu_half;
        return (w < kSwigluGroup) ? j : swiglu_half + j;
    }
    *valid = ro < rows;
    return ro;
}

// The quantiser's work of block (bx, by) of a (., gy) grid.
__device__ __forceinline__ void quantize_part(const float* __restrict__ v, int64_t rows, int64_t cols,
                                              const Quantizer& qz, int8_t* __restrict__ q, int64_t rows_p,
                                              int64_t cols_p, int64_t swiglu_half, int64_t bx, int64_t by,
                                              int64_t gy) {
    const int64_t c0 = (bx * 256 + threadIdx.x) * 4;
    if (c0 >= cols_p) return;
    const bool vec = ((cols & 3) == 0) && ((reinterpret_cast<uintptr_t>(v) & 15) == 0) && c0 + 4 <= cols;
    for (int64_t rb = by * kQRows; rb < rows_p; rb += gy * kQRows) {
        vf4 x[kQRows];
        bool ok[kQRows];
#pragma unroll
        for (int u = 0; u < kQRows; ++u) {
            x[u] = vf4{0.0f, 0.0f, 0.0f, 0.0f};
            bool valid;
            const int64_t r = quantize_src_row(rb + u, rows, swiglu_half, &valid);
            ok[u] = valid && rb + u < rows_p;
            if (!ok[u]) continue;
            const float* src = v + r * cols;
            if (vec) {
                x[u] = __builtin_nontemporal_load(reinterpret_cast<const vf4*>(src + c0));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c0 + e < cols) x[u][e] = src[c0 + e];
            }
        }
        // codes on the fast path; a wave with any value near a rounding
        // midpoint redoes all of its values on the exact path
        uint32_t packed[kQRows];
        bool unsure = false;
#pragma unroll
        for (int u = 0; u < kQRows; ++u) {
            packed[u] = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int qv = (ok[u] && c0 + e < cols) ? qz.q_fast(x[u][e], &unsure) : 0;
                packed[u] |= (uint32_t)(uint8_t)(int8_t)qv << (8 * e);
            }
        }
        if (__ballot(unsure)) {
#pragma unroll
            for (int u = 0; u < kQRows; ++u) {
                packed[u] = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bool in;
                    const int qv = (ok[u] && c0 + e < cols) ? qz.q(x[u][e], &in) : 0;
                    packed[u] |= (uint32_t)(uint8_t)(int8_t)qv << (8 * e);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kQRows; ++u) {
            if (rb + u >= rows_p) break;
            *reinterpret_cast<uint32_t*>(q + (rb + u) * cols_p + c0) = packed[u];
        }
    }
}

__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ v, int64_t rows,
                                                       int64_t cols, const float* __restrict__ s_dev,
                                                       float s_host, int8_t* __restrict__ q,
                                                       int64_t rows_p, int64_t cols_p,
                                                       int64_t swiglu_half) {
    const Quantizer qz(s_dev ? *s_dev : s_host);
    quantize_part(v, rows, cols, qz, q, rows_p, cols_p, swiglu_half, blockIdx.x, blockIdx.y, gridDim.y);
}

hipError_t launch_quantize(const float* v, int64_t rows, int64_t cols, const float* s_dev,
                           float s_host, int8_t* q, int64_t rows_p, int64_t cols_p,
                           int64_t swiglu_half, hipStream_t st) {
    if (rows_p <= 0 || cols_p <= 0) return hipSuccess;
    const unsigned gx = (unsigned)ceil_div(cols_p / 4, 256);
    // at most 2048 row groups of workgroups, so large inputs take a few
    // grid-stride iterations per thread: X of the QKV layer 35.3 -> 33.5 us,
    // of the down projection 90 -> 84 us, against one iteration per thread
    const int64_t blocks = ceil_div(rows_p, kQRows);
    const unsigned gy = (unsigned)(blocks < 2048 ? blocks : 2048);
    hipLaunchKernelGGL(quantize_kernel, dim3(gx, gy), dim3(256), 0, st, v, rows, cols, s_dev, s_host,
                       q, rows_p, cols_p, swiglu_half);
    return hipGetLastError();
}

// ---- the forward's preparation in one launch ----------------------------------------
// The weight step, the W codes and the X codes of one forward call in one grid
// of 256-thread workgroups, in four consecutive ranges of workgroup ids:
//   [0, P)         CanonSum of |W|: workgroup b reduces the aligned run of 256
//                  32-blocks that starts at block 256 b to one subtree root
//                  and publishes it;
//   P              the tail: waits for the P roots, reduces them in the
//                  canonical order (canon_runs_tree), forms s_w and s_y and
//                  publishes s_w;
//   [P+1, P+1+XB)  the X quantiser (its step is the caller's s_x);
//   [P+1+XB, ...)  the W quantiser (at most 1024 workgroups), which first
//                  waits for s_w.
// Each published value travels with its own ready tag in one 64-bit word
// (tag in the high half, the float's bits in the low half), written and read
// as a relaxed device-scope atomic: the reader needs that one word and
// nothing else, so no fence is needed.  (A device-scope release or acquire
// writes back or invalidates a whole L2; one per workgroup made this launch
// slower than the separate launches it replaces.)  fwd_prep_clear_kernel
// zeroes the words first.
//
// Only the tail and the W range wait, and only on work of lower ranges whose
// workgroups never wait: once running, they finish.  Waiters number at most
// 1 + min(1024, 4 per CU), fewer workgroups than the device holds at once
// (this kernel fits 7 per CU, its scalar registers being the limit: 1792 on
// 256 CUs), so the workgroups they wait for always find room to run even when
// every waiter is resident; each wait is bounded all the same
// (kPrepSpinLimit polls, about a second; then the error word records it and
// the GEMM writes NaN for every output), so every wave exits.  Measured on the MI355X (forward call, QKV / SwiGLU gate+up / down
// projection at 16384 tokens): 150 / 560 / 261 us against 158 / 575 / 276 us
// for the four separate launches; the W range before the X range, or at most
// 512 W workgroups, measured 1-2% slower.
constexpr int64_t kPrepMaxWgW = 1024;
constexpr uint32_t kPrepSpinLimit = 1u << 20;
constexpr uint64_t kPrepReady = 1ull << 32;

__device__ __forceinline__ uint64_t prep_word(float v) {
    return kPrepReady | (uint64_t)__builtin_bit_cast(uint32_t, v);
}

// The float published in *w, once its tag is up (bounded wait: on giving up,
// records it in *err and returns whatever the word holds).
__device__ __forceinline__ float prep_wait(const uint64_t* w, uint64_t* err) {
    uint64_t v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t polls = 0;
    while (v < kPrepReady) {
        if (++polls == kPrepSpinLimit) {
            __hip_atomic_store(err, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(16);
        v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return __builtin_bit_cast(float, (uint32_t)v);
}

// |w| of the 32 weights of one block, held 4 per lane by 8 consecutive lanes
// (lane 8j + k holds weights 4k .. 4k+3 of block j), summed left to right from
// the first term: the running sum moves one lane up per step (row_shr:1 stays
// inside a group of 8 lanes, which never straddles a 16-lane DPP row).  The
// block sum ends in lane 8j + 7.
__device__ __forceinline__ float prep_block_chain(vf4 x, int lane) {
    const int k = lane & 7;
    float c = 0.0f;
#pragma unroll
    for (int step = 0; step < 8; ++step) {
        const float prev = __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, c), 0x111, 0xF, 0xF, false));
        if (k == step) {
            float v = step == 0 ? __builtin_fabsf(x.x) : f_add(prev, __builtin_fabsf(x.x));
            v = f_add(v, __builtin_fabsf(x.y));
            v = f_add(v, __builtin_fabsf(x.z));
            c = f_add(v, __builtin_fabsf(x.w));
        }
    }
    return c;
}

// First range, workgroup b: the subtree root of 32-blocks [256 b, 256 b + 256)
// of |W| (flat, row-major), published in root word b.
__device__ void prep_abs_run(const PrepArgs& a, int64_t b, float* lds, float* blk) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t nW = a.N * a.K;
    const int64_t base = b * kPrepRunBlocks * kBlock;
    const float* src = a.W + base;
    int count;
    float v;
    if (base + kPrepRunBlocks * kBlock <= nW && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
        // wave w: weights [2048 w, 2048 w + 2048) of the run as 8 coalesced
        // 1 KiB loads; load i, lane l holds block 64 w + 8 i + l / 8
        const vf4* s4 = reinterpret_cast<const vf4*>(src) + w * 512 + lane;
        vf4 x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = s4[64 * i];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float c = prep_block_chain(x[i], lane);
            if ((lane & 7) == 7) blk[w * 64 + i * 8 + (lane >> 3)] = c;
        }
        __syncthreads();
        v = blk[t];
        count = (int)kPrepRunBlocks;
    } else {
        // the short last run (or an unaligned W): thread t walks its own block
        const int64_t e0 = base + (int64_t)t * kBlock;
        const int64_t left = nW - e0;
        const int len = left <= 0 ? 0 : (left < kBlock ? (int)left : kBlock);
        v = 0.0f;
        if (len > 0) {
            v = __builtin_fabsf(a.W[e0]);
            for (int i = 1; i < len; ++i) v = f_add(v, __builtin_fabsf(a.W[e0 + i]));
        }
        const int64_t blocks = (nW + kBlock - 1) / kBlock - b * kPrepRunBlocks;
        count = blocks < kPrepRunBlocks ? (int)blocks : (int)kPrepRunBlocks;
    }
    const float r = wg_pair_tree(v, count, lds);
    if (t == 0) __hip_atomic_store(&a.sync[kPrepRootWord + b], prep_word(r), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
}

// The tail: CanonSum of the P roots, then s_w (published) and s_y.  Each
// thread issues the loads of its RUN root words together and polls again only
// for the words not yet published.
template <int RUN>
__device__ float prep_tail_sum(const PrepArgs& a, float* lds) {
    const uint64_t* roots = a.sync + kPrepRootWord;
    uint64_t* err = a.sync + kPrepErrWord;
    const int64_t first = (int64_t)threadIdx.x * RUN;
    uint64_t w[RUN];
#pragma unroll
    for (int i = 0; i < RUN; ++i)
        w[i] = first + i < a.P ? __hip_atomic_load(roots + first + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                               : kPrepReady;
    float vals[RUN];
#pragma unroll
    for (int i = 0; i < RUN; ++i)
        vals[i] = w[i] >= kPrepReady ? __builtin_bit_cast(float, (uint32_t)w[i]) : prep_wait(roots + first + i, err);
    return canon_runs_tree<RUN>([&](int64_t j) { return vals[j - first]; }, a.P, lds);
}

__device__ void prep_tail(const PrepArgs& a, float* lds) {
    float S;
    if (a.P <= 256) S = prep_tail_sum<1>(a, lds);
    else if (a.P <= 512) S = prep_tail_sum<2>(a, lds);
    else if (a.P <= 1024) S = prep_tail_sum<4>(a, lds);
    else if (a.P <= 2048) S = prep_tail_sum<8>(a, lds);
    else S = prep_tail_sum<16>(a, lds);
    if (threadIdx.x == 0) {
        canon_finish(S, a.fin);
        __hip_atomic_store(&a.sync[kPrepStepWord], prep_word(a.fin.scal->s_w), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
}

__global__ __launch_bounds__(256) void fwd_prep_kernel(PrepArgs a) {
    __shared__ float lds[256];
    __shared__ float blk[256];
    int64_t i = blockIdx.x;
    if (i < a.P) {
        prep_abs_run(a, i, lds, blk);
        return;
    }
    if (i == a.P) {
        prep_tail(a, lds);
        return;
    }
    i -= a.P + 1;
    const int64_t nx = a.xgx * a.xgy;
    if (i < nx) {
        const Quantizer qz(a.s_x);
        const uint32_t iu = (uint32_t)i, gx = (uint32_t)a.xgx;   // 32-bit: no float-assisted 64-bit divide
        quantize_part(a.X, a.M, a.K, qz, a.qx, a.Mp, a.Kp, 0, iu % gx, iu / gx, a.xgy);
        return;
    }
    i -= nx;
    if (threadIdx.x == 0) lds[0] = prep_wait(a.sync + kPrepStepWord, a.sync + kPrepErrWord);
    __syncthreads();
    const Quantizer qz(lds[0]);
    const uint32_t iu = (uint32_t)i, gx = (uint32_t)a.wgx;
    quantize_part(a.W, a.N, a.K, qz, a.qw, a.Nvp, a.Kp, a.swiglu_half, iu % gx, iu / gx, a.wgy);
}

// zeroes the step, error and root words of a launch with P roots
__global__ __launch_bounds__(256) void fwd_prep_clear_kernel(uint64_t* sync, int64_t words) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j < words) sync[j] = 0ull;
}

hipError_t launch_fwd_prep(PrepArgs a, hipStream_t st) {
    const int64_t nW = a.N * a.K;
    a.P = ceil_div(ceil_div(nW, kBlock), kPrepRunBlocks);
    if (a.P < 1 || a.P > kPrepMaxRoots || a.Mp <= 0 || a.Nvp <= 0 || a.Kp <= 0) return hipErrorInvalidValue;
    // the W range (the waiters) also stays within 4 workgroups per CU of the
    // stream's device, of the 7 it holds of this kernel at once, so the
    // bound holds on a device with fewer CUs (a partition of the chip, say)
    int64_t max_w = kPrepMaxWgW;
    hipDevice_t dev = 0;
    int cus = 0;
    if (hipStreamGetDevice(st, &dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0 &&
        4 * (int64_t)cus < max_w)
        max_w = 4 * (int64_t)cus;
    (void)hipGetLastError();   // a failed query leaves the default and no pending error
    a.wgx = ceil_div(a.Kp / 4, 256);
    if (a.wgx > max_w) return hipErrorInvalidValue;
    const int64_t wrows = ceil_div(a.Nvp, kQRows);
    const int64_t wcap = max_w / a.wgx;
    a.wgy = wrows < wcap ? wrows : wcap;
    a.xgx = a.wgx;
    const int64_t xrows = ceil_div(a.Mp, kQRows);
    a.xgy = xrows < 2048 ? xrows : 2048;
    const int64_t grid = a.P + 1 + a.wgx * a.wgy + a.xgx * a.xgy;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    const int64_t words = kPrepRootWord + a.P;
    hipLaunchKernelGGL(fwd_prep_clear_kernel, dim3((unsigned)ceil_div(words, 256)), dim3(256), 0, st, a.sync,
                       words);
    if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL(fwd_prep_kernel, dim3((unsigned)grid), dim3(256), 0, st, a);
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
    const Quantizer qz(s);
    const bool vec_rows = ((cols & 3) == 0) && ((reinterpret_cast<uintptr_t>(v) & 15) == 0);
    for (int64_t r = blockIdx.y; r < rows_p; r += gridDim.y) {
        vf4 x = {0.0f, 0.0f, 0.0f, 0.0f};
        if (r < rows) {
            const float* src = v + r * cols;
            if (vec_rows && c0 + 4 <= cols) {
                x = *reinterpret_cast<const vf4*>(src + c0);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c0 + e < cols) x[e] = src[c0 + e];
            }
        }
        // zeros past the data quantise to 0 and dequantise to +0
        vf4 o;
        bool unsure = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = f_mul((float)qz.q_fast(x[e], &unsure), s);
        if (__ballot(unsure)) {
            bool in;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = f_mul((float)qz.q(x[e], &in), s);
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
// Workgroup tile BM x BN, K step 64 bytes (two MFMA k-steps of 32), 4 waves of
// WM x WN, each a (WM/32) x (WN/32) grid of v_mfma_i32_32x32x32_i8 tiles.
// Operand tiles move global -> LDS with buffer_load_dwordx4 ... lds (no
// staging registers; per-lane offsets fixed for the whole loop, the k offset
// in a scalar register) through a ring of STAGES LDS stages, so loads run
// STAGES-1 tiles ahead of the MFMAs.  LDS rows are 64 bytes, unpadded; the
// four 16-byte chunks of row r are stored XOR-swizzled by (r >> 2) & 3.  The
// LDS serves a 16-byte-per-lane read 16 lanes per clock across its 64 banks;
// the swizzle puts the fragment reads of 16 consecutive rows (4 rows per
// 256-byte bank window, 4 distinct chunk slots each) on 16 distinct 16-byte
// bank groups, so the reads are conflict-free.
//
// Schedule: with few waves per SIMD, any instruction that stalls a wave
// idles its matrix core, so every k-step issues its MFMAs with the memory
// instructions of the pipeline placed between them (scheduling barriers keep
// the compiler from regrouping them): the fragment reads of the next k-step,
// and in the second k-step of each tile the loads of the tile STAGES-1
// ahead.  Past the last tile those loads repeat the last tile
// into a stage that is never read again, so the loop has no branch.
constexpr int kBK = 64;

template <int BM, int BN, int WM, int WN, int STAGES>
struct GemmCfg {
    static constexpr int kWavesM = BM / WM, kWavesN = BN / WN;
    static constexpr int kThreads = kWavesM * kWavesN * 64;
    static constexpr int kWaves = kThreads / 64;
    static constexpr int kTM = WM / 32, kTN = WN / 32;
    static constexpr int kMfma = kTM * kTN;                          // MFMAs per wave per k-step
    static constexpr int kReads = kTM + kTN;                         // fragment reads per k-step
    static constexpr int kTileA = BM * kBK, kTileB = BN * kBK;      // bytes per stage
    static constexpr int kStage = kTileA + kTileB;
    static constexpr int kLds = STAGES * kStage;
    // one load instruction moves 64 lanes x 16 bytes = 16 rows of 64 bytes
    static constexpr int kLoadsA = BM / 16 / kWaves, kLoadsB = BN / 16 / kWaves;
    static constexpr int kLoads = kLoadsA + kLoadsB;                // per wave per stage
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

// 16 bytes per lane from base[off + soff] (a raw buffer over `bytes` bytes;
// reads past the end return zero) into LDS at lds + 16 * lane
__device__ __forceinline__ void gemm_load_lds(const int8_t* base, int bytes, uint32_t off, uint32_t soff,
                                              int8_t* lds) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(base), (short)0, bytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, soff, 0, 0);
}

#define GEMM_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

template <int BM, int BN, int WM, int WN, int STAGES, int MINB, int EPI>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64, MINB) void gemm_i8_kernel(GemmArgs a) {
    using C = GemmCfg<BM, BN, WM, WN, STAGES>;
    static_assert(C::kThreads == 256 || C::kThreads == 512, "the GEMM runs 4 or 8 waves per workgroup");
    static_assert(C::kReads <= C::kMfma && C::kLoads <= C::kMfma,
                  "every fragment read and tile load of a k-step follows one of its MFMAs");
    static_assert(STAGES >= 3 && 2 * C::kLoads * (STAGES - 2) < 64, "pipeline depth and vmcnt range");
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
    const int bytesA = (int)(BM * a.Kp), bytesB = (int)(BN * a.Kp);
    const int KT = (int)(a.Kp / kBK);

    // this lane's share of load instruction i: row (lane >> 2) of a 16-row
    // group, LDS slot (lane & 3), holding global chunk swz(row, slot)
    const int lrow = lane >> 2, lslot = lane & 3;
    uint32_t off[C::kLoads];
#pragma unroll
    for (int i = 0; i < C::kLoads; ++i) {
        const int r = i < C::kLoadsA ? (wave * C::kLoadsA + i) * 16 + lrow
                                     : (wave * C::kLoadsB + (i - C::kLoadsA)) * 16 + lrow;
        off[i] = (uint32_t)(r * a.Kp + 16 * swz(r, lslot));
    }
    auto load1 = [&](int kt, int stage, int i) {
        int8_t* sA = smem + stage * C::kStage;
        if (i < C::kLoadsA) {
            const int r0 = (wave * C::kLoadsA + i) * 16;
            gemm_load_lds(gA, bytesA, off[i], (uint32_t)(kt * kBK), sA + r0 * kBK);
        } else {
            const int r0 = (wave * C::kLoadsB + (i - C::kLoadsA)) * 16;
            gemm_load_lds(gB, bytesB, off[i], (uint32_t)(kt * kBK), sA + C::kTileA + r0 * kBK);
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
    using Frag = v4i[C::kReads];
    // fragment q of k-step ks in `stage`: A rows for q < kTM, else B rows
    auto read1 = [&](int stage, int ks, Frag& F, int q) {
        const int8_t* sA = smem + stage * C::kStage;
        const int chunk = fchunk + 2 * ks;
        if (q < C::kTM) {
            const int r = wm * WM + q * 32 + frow;
            F[q] = *reinterpret_cast<const v4i*>(sA + r * kBK + 16 * swz(r, chunk));
        } else {
            const int r = wn * WN + (q - C::kTM) * 32 + frow;
            F[q] = *reinterpret_cast<const v4i*>(sA + C::kTileA + r * kBK + 16 * swz(r, chunk));
        }
    };
    // one k-step: the kMfma MFMAs on Fc; MFMA q is followed by fragment read
    // q of (rs, rk) into Fn (q < kReads) and, when ld, by the loads of tile
    // lkt into stage ls spread evenly over the MFMAs
    auto kstep = [&](const Frag& Fc, Frag& Fn, bool rd, int rs, int rk, bool ld, int lkt, int ls) {
#pragma unroll
        for (int q = 0; q < C::kMfma; ++q) {
            const int i = q / C::kTN, j = q % C::kTN;
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(Fc[i], Fc[C::kTM + j], acc[i][j], 0, 0, 0);
            if (rd && q < C::kReads) read1(rs, rk, Fn, q);
            constexpr int nl = C::kLoads, nm = C::kMfma;
            if (ld && (q + 1) * nl / nm > q * nl / nm) load1(lkt, ls, q * nl / nm);
            GEMM_SCHED_FENCE();
        }
    };
    auto barrier = [] {
        // bare barrier: a fence here would wait for every load in flight
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };

    static_assert(kBK == 64, "two k-steps per tile");
    Frag F0, F1;
    // tiles 0 .. STAGES-2 in flight before the loop
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
#pragma unroll
        for (int i = 0; i < C::kLoads; ++i) load1(s < KT ? s : KT - 1, s, i);
    wait_vmcnt<(STAGES - 2) * C::kLoads>();   // tile 0 landed
    barrier();
#pragma unroll
    for (int q = 0; q < C::kReads; ++q) read1(0, 0, F0, q);
    GEMM_SCHED_FENCE();
    for (int kt = 0; kt < KT - 1; ++kt) {
        kstep(F0, F1, true, kt % STAGES, 1, false, 0, 0);
        // tile kt+1 landed for every wave, and every wave is past its reads
        // of tile kt-1, whose stage the loads below refill
        wait_vmcnt<(STAGES - 3) * C::kLoads>();
        barrier();
        const int lkt = kt + STAGES - 1 < KT ? kt + STAGES - 1 : KT - 1;
        kstep(F1, F0, true, (kt + 1) % STAGES, 0, true, lkt, (kt + STAGES - 1) % STAGES);
    }
    kstep(F0, F1, true, (KT - 1) % STAGES, 1, false, 0, 0);
    kstep(F1, F0, false, 0, 0, false, 0, 0);
    wait_vmcnt<0>();                       // no load into LDS outlives the loop

    // ---- epilogue: Y = fl(acc) * s_y (+ addend), or the SwiGLU activation ----
    // a preparation wait that gave up (see fwd_prep_kernel) poisons Y with NaN
    const float s_y = (a.prep_err && *a.prep_err) ? __builtin_nanf("") : a.scal->s_y;
    const int col_l = lane & 31;
    const int row_q = (lane >> 5) * 4;
    if constexpr (EPI == BRL_EPILOGUE_SWIGLU) {
        // wave columns: tiles [0, kTN/2) are gate, [kTN/2, kTN) the matching up
        const int64_t H = a.N / 2;
        // whole tile inside Y (its rows, and the gate columns of its virtual
        // column groups), no addend, offsets within the tile below 2^29:
        // branch-free stores at 32-bit offsets from the tile's corner
        const bool full = (m0 + BM <= a.M) && (n0 / 2 + BN / 2 <= H) && !a.addend &&
                          (int64_t)BM * a.N < ((int64_t)1 << 29);   // byte offsets below 2^31
        if (full) {
            // a wave's virtual columns are one gate/up group pair: gate
            // column gcol0 + c and up column H + gcol0 + c, c < kSwigluGroup;
            // stores at 32-bit byte offsets from uniform bases
            const int64_t gcol0 = (n0 + wn * WN) / 2;
            const unsigned N4 = 4u * (unsigned)a.N, H4 = 4u * (unsigned)H;
            char* Yt = reinterpret_cast<char*>(a.Y + m0 * H + gcol0);
            auto tile = [&](auto pre) {
                char* Pt = reinterpret_cast<char*>(a.Ypre + m0 * a.N + gcol0);
#pragma unroll
                for (int i = 0; i < C::kTM; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const unsigned rl = (unsigned)(wm * WM + i * 32 + (r >> 2) * 8 + row_q + (r & 3));
#pragma unroll
                        for (int j = 0; j < C::kTN / 2; ++j) {
                            const unsigned c4 = 4u * (unsigned)(j * 32 + col_l);
                            const float g = f_mul((float)acc[i][j][r], s_y);
                            const float u = f_mul((float)acc[i][j + C::kTN / 2][r], s_y);
                            if constexpr (decltype(pre)::value) {
                                *reinterpret_cast<float*>(Pt + (rl * N4 + c4)) = g;
                                *reinterpret_cast<float*>(Pt + (rl * N4 + H4 + c4)) = u;
                            }
                            const float sg = swiglu_sigma(g, a.ek);
                            *reinterpret_cast<float*>(Yt + (rl * H4 + c4)) = f_mul(f_mul(g, sg), u);
                        }
                    }
            };
            if (a.Ypre) tile(std::true_type{});
            else tile(std::false_type{});
            return;
        }
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

// Launch shape: 256 x 256 workgroup tiles of 8 waves, two per SIMD, so that
// one wave's waits (fragment reads, the tile barrier, the vmcnt wait) are
// covered by the MFMAs of the other; a ring of four 32 KB stages, one
// workgroup per CU.  Plain epilogue: waves of 128 x 64; SwiGLU epilogue: waves
// of 64 x 128 (a wave's columns are one interleaved gate/up group pair).
// Measured on the MI355X against 4 waves of 128 x 128 (one per SIMD): QKV
// forward 173 -> 167 us, SwiGLU gate+up forward 787 -> 669 us (against
// 128 x 256 tiles at two workgroups per CU), down projection unchanged.
template <int BM, int BN, int WM, int WN, int STAGES, int MINB, int EPI>
static hipError_t launch_gemm_cfg(const GemmArgs& a, hipStream_t st) {
    using C = GemmCfg<BM, BN, WM, WN, STAGES>;
    static_assert(C::kLoadsA * C::kWaves * 16 == BM && C::kLoadsB * C::kWaves * 16 == BN, "load split");
    static_assert(kRowPad % BM == 0 && kRowPad % BN == 0, "padded operands hold whole tiles");
    static_assert(EPI != BRL_EPILOGUE_SWIGLU || WN == 2 * kSwigluGroup,
                  "a wave's columns are one interleaved gate/up group pair");
    const size_t lds = (size_t)C::kLds;
    // operand panels are addressed through 32-bit buffer offsets
    if ((int64_t)(BM > BN ? BM : BN) * a.Kp > INT32_MAX) return hipErrorInvalidValue;
    const void* fn = reinterpret_cast<const void*>(&gemm_i8_kernel<BM, BN, WM, WN, STAGES, MINB, EPI>);
    // the limit is set on every call: it is per device, and the call is cheap
    if (const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        e != hipSuccess)
        return e;
    const int64_t tiles = (a.Mp / BM) * (a.Nvp / BN);
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, WM, WN, STAGES, MINB, EPI>), dim3((unsigned)tiles),
                       dim3(C::kThreads), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_gemm_i8(const GemmArgs& a, hipStream_t st) {
    if (a.epilogue == BRL_EPILOGUE_SWIGLU)
        return launch_gemm_cfg<256, 256, 64, 128, 4, 1, BRL_EPILOGUE_SWIGLU>(a, st);
    return launch_gemm_cfg<256, 256, 128, 64, 4, 1, BRL_EPILOGUE_NONE>(a, st);
}

}  // namespace brl
