// internal.hpp -- host-side launchers shared between the translation units of
// libbrlsq.  Nothing here is part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device.hpp"
#include "brlsq.h"

namespace brl {

// Scalars kept in device memory by one call (never read back by the host).
struct Scalars {
    float s_w;      // weight step
    float s_y;      // s_x * s_w
    float nu;       // global norm
    float kappa;    // clip coefficient (1 when not clipping)
    int32_t clip;   // 1 when kappa applies
    int32_t pad[11];
};

inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Launch shapes of one call (never change results), resolved from the
// caller's brl_tuning with the defaults filled in.
struct Tuning {
    int chunk_log2;   // backward chunk = 2^chunk_log2 32-blocks; 0 = per engine (6 matrix cores, 4 VALU)
    int wg_blocks;    // 32-blocks per workgroup in CanonSum passes (64, 128, 256)
    int vec;          // 16-byte vectors per thread in streaming kernels (1, 2, 4)
    int engine;       // backward products: 1 VALU, 2 matrix cores (when the operands allow)
    int fwd_prep;     // forward preparation: 1 one launch (where it fits), 2 separate launches
};
// false for a value outside its range
bool resolve_tuning(const brl_tuning* t, Tuning* out);
// chunk depth of the backward on `engine` (1 or 2); engine 0 gives the
// smaller depth of the two, which bounds the chunk roots for the workspace
int bwd_chunk_log2(const Tuning& t, int engine);

// ---- CanonSum over a flat vector -------------------------------------------
enum CanonMap { kMapAbs = 0, kMapSquare = 1 };
enum CanonFinish { kFinishScale = 0, kFinishNorm = 1 };

struct CanonFinishArgs {
    int mode;               // CanonFinish
    float count_f;          // fl(number of summed elements) (scale)
    float s_x;              // activation step (scale)
    float max_norm, eps;    // (norm)
    Scalars* scal;          // receives s_w/s_y or nu/kappa/clip
    float* s_w_out;         // optional copy of s_w
    float* nu_out;          // optional copy of nu
};

// The scalar that follows a CanonSum S (one thread): the weight step s_w and
// s_y = s_x * s_w, or the norm nu = sqrt(S) and the clip coefficient.
__device__ __forceinline__ void canon_finish(float S, const CanonFinishArgs& f) {
    if (f.mode == kFinishScale) {
        const float s_w = weight_step(S, f.count_f);
        f.scal->s_w = s_w;
        f.scal->s_y = f_mul(f.s_x, s_w);
        if (f.s_w_out) *f.s_w_out = s_w;
    } else {
        float nu = f_sqrt(S);
        int clip = nu > f.max_norm;
        f.scal->nu = nu;
        f.scal->clip = clip;
        f.scal->kappa = clip ? f_div(f.max_norm, f_add(nu, f.eps)) : 1.0f;
        if (f.nu_out) *f.nu_out = nu;
    }
}

// Partial buffer floats needed by launch_canon for n elements.
int64_t canon_partials(int64_t n);
hipError_t launch_canon(int map, const float* x, int64_t n, float* partials,
                        const CanonFinishArgs& fin, int wg_blocks, hipStream_t st);

// ---- quantisation and the int8 GEMM ------------------------------------------
// GEMM tiling (forward): K padded to kKPad, rows of both operands to kRowPad.
constexpr int kKPad = 64;
constexpr int kRowPad = 256;
constexpr int kSwigluGroup = 64;   // gate/up columns interleaved in groups of 64

// q[r_out, :] for every padded output row r_out < rows_p (zero rows and
// columns past the data).  swiglu_half > 0 interleaves rows in groups of
// kSwigluGroup: output rows [128t, 128t+64) = gate rows [64t, 64t+64),
// [128t+64, 128t+128) = up rows half + [64t, 64t+64).
hipError_t launch_quantize(const float* v, int64_t rows, int64_t cols, const float* s_dev,
                           float s_host, int8_t* q, int64_t rows_p, int64_t cols_p,
                           int64_t swiglu_half, hipStream_t st);

// out[r][c] = fl(q(v[r][c]) * s) for r < rows, c < cols; +0 up to rows_p x cols_p
// (cols_p a multiple of 4).
hipError_t launch_dequant(const float* v, int64_t rows, int64_t cols, const float* s_dev, float s_host,
                          float* out, int64_t rows_p, int64_t cols_p, hipStream_t st);

// The forward's preparation in one launch (weight step, W codes, X codes);
// see fwd_prep_kernel.  sync: kPrepSyncWords 64-bit words (the step word,
// the error word, then one word per |W| run root), cleared by the launcher.
constexpr int64_t kPrepRunBlocks = 256;                   // 32-blocks per first-range workgroup
constexpr int64_t kPrepMaxRoots = 256 * 16;               // roots the in-kernel tail reduces
constexpr int64_t kPrepStepWord = 0, kPrepErrWord = 1, kPrepRootWord = 2;
constexpr int64_t kPrepSyncWords = kPrepRootWord + kPrepMaxRoots;
struct PrepArgs {
    const float* X;
    const float* W;
    int64_t M, K, N;       // N = stacked width
    float s_x;
    int8_t* qx;            // [Mp, Kp]
    int8_t* qw;            // [Nvp, Kp]
    int64_t Mp, Kp, Nvp, swiglu_half;
    uint64_t* sync;        // kPrepSyncWords words
    int64_t P;             // first-range workgroups (|W| run roots)
    int64_t wgx, wgy;      // W quantiser grid
    int64_t xgx, xgy;      // X quantiser grid
    CanonFinishArgs fin;
};
// true when one launch can prepare a forward with N*K weights
inline bool fwd_prep_fits(int64_t nW) { return ceil_div(ceil_div(nW, kBlock), kPrepRunBlocks) <= kPrepMaxRoots; }
hipError_t launch_fwd_prep(PrepArgs a, hipStream_t st);

struct GemmArgs {
    const int8_t* qx;     // [Mp, Kp]
    const int8_t* qw;     // [Nvp, Kp] (interleaved for SwiGLU)
    int64_t M, N, Kp;     // N = true stacked width
    int64_t Mp, Nvp;      // padded row counts
    const Scalars* scal;  // s_y
    const float* addend;  // [M, N] or null
    float* Y;             // [M, N] or [M, N/2]
    float* Ypre;          // SwiGLU pre-activation [M, N] or null
    int epilogue;
    ExpConsts ek;
    const uint64_t* prep_err;   // the one-launch preparation's error word, or null
};
hipError_t launch_gemm_i8(const GemmArgs& a, hipStream_t st);

// ---- straight-through backward ---------------------------------------------
struct SteArgs {
    // C[i][j] = CanonSum_r A(r,i) * B(r,j) for r in [0, R)
    const float* A;        // dY / G
    int64_t lda;
    bool a_rmaj;           // A(r,i) = A[i*lda + r] (dX) else A[r*lda + i] (dW)
    bool a_vec;            // A and lda allow 16-byte row loads
    int64_t I, R, Jn;
    const int8_t* Bq;      // [>= round_up(R,32), ldb] int8, zero padded (VALU engine)
    const float* Bf;       // [>= round_up(R,32), ldb] fl(q*s), zero padded (matrix-core engine)
    int64_t ldb;
    const float* b_scale_dev;  // step of B (device) or null
    float b_scale_host;
    // mask and output
    const float* mask_src; // [I, Jn] values whose in-range decides the mask
    const float* mask_scale_dev;
    float mask_scale_host;
    float* out;            // [I, Jn]
    int accumulate;
    float* roots;          // workspace for chunk roots [Q, I, Jn]
};
// reduction chunks of 2^D 32-blocks over R terms
int64_t ste_chunks(int64_t R, int D);
int64_t ste_root_floats(int64_t I, int64_t R, int64_t Jn, int D);
// engine 2 needs Bf, a_vec and I % 4 == 0 when A is r-major, R % 4 == 0 when i-major;
// D = chunk depth (1..7)
hipError_t launch_ste(const SteArgs& a, int engine, int D, hipStream_t st);

hipError_t launch_swiglu_bwd(const float* dA, const float* ypre, int64_t M, int64_t N, float* G,
                             const ExpConsts& ek, hipStream_t st);

// ---- state hash (SHA-256 tree) -------------------------------------------------
constexpr int64_t kHashLeafBytes = 4096;    // bytes of a tensor per leaf
constexpr int64_t kHashFanIn = 16;          // digests per node
constexpr int kHashBatch = 64;              // tensors per leaf launch
struct HashBatch {
    const void* ptr[kHashBatch];
    int64_t len[kHashBatch];
    int64_t first_leaf[kHashBatch];   // first leaf of each tensor, counted from the batch's first leaf
    int32_t n;                        // tensors in the batch
    int32_t pad;
    int64_t first_tensor;             // index of ptr[0] in the state
    int64_t leaf_base;                // index of the batch's first leaf among all leaves
    int64_t leaves;                   // leaves in the batch
};
hipError_t launch_hash_leaves(const HashBatch& hb, bool vec, uint8_t* digests, int64_t* lens, hipStream_t st);
hipError_t launch_hash_nodes(const uint8_t* in, int64_t n_in, uint8_t* out, hipStream_t st);
hipError_t launch_hash_root(const uint8_t* top, const int64_t* lens, int64_t count, uint8_t* out, hipStream_t st);
void sha256_constants(uint32_t* k64, uint32_t* h8);

// ---- AdamW --------------------------------------------------------------------
hipError_t launch_adamw(float* p, const float* g, float* m, float* v, int64_t n, const brl_adamw_scalars& s,
                        int decay, hipStream_t st);
void adamw_scalars(int64_t step, double tokens, const brl_adamw_config& c, brl_adamw_scalars* out);

// ---- replay -------------------------------------------------------------------
// first = 1: A <- G; otherwise A <- X + G (X = A, or a deferred first shard).
hipError_t launch_accumulate(float* A, const float* X, const float* G, int64_t n, int first, int vec,
                             hipStream_t st);
struct FoldPtrs { const float* a[64]; };
// TreeFold of A_0..A_{R-1} into out.  Replica R-1's value: with nlast > 0
// the running sum of its resident partials last.a[0..nlast) (A_{R-1} is not
// read), else A_{R-1} completed with g_last when given.
hipError_t launch_fold(const FoldPtrs& p, int R, const float* g_last, const FoldPtrs& last, int nlast,
                       float* out, int64_t n, hipStream_t st);
// A <- running sum of parts.a[0..S): ((G_0 + G_1) + G_2) + ..., S >= 1
hipError_t launch_runsum(float* A, const FoldPtrs& parts, int S, int64_t n, hipStream_t st);
hipError_t launch_clip(float* g, int64_t n, const Scalars* scal, int vec, hipStream_t st);

// out[i] = a[i] * b[i] formed by the matrix-core product of the backward
hipError_t launch_probe_mfma(const float* a, const float* b, float* out, int64_t n, hipStream_t st);
hipError_t launch_probe(int op, const float* a, const float* b, float* out, int64_t n,
                        const ExpConsts& ek, hipStream_t st);
// out[i] = a[i]*a[i] + b[i] as the K=1 fp32 MFMA forms it (accumulator input b[i])
hipError_t launch_probe_mfma_fma(const float* a, const float* b, float* out, int64_t n, hipStream_t st);
// sustained-rate probes (probe.hip): what 0 v_add_f32, 1 v_mul_f32, 2 K=1 fp32
// MFMA, 3 i8 MFMA 32x32x32; out has probe_rate_threads() floats
hipError_t launch_probe_rate(int what, int64_t iters, float c, float* out, hipStream_t st);
int64_t probe_rate_threads();

ExpConsts exp_constants();

// error reporting for entry points outside api.hip (thread-local last error)
brl_status report_error(brl_status s, const char* msg);
brl_status report_hip(hipError_t e, const char* what);

// ---- attention (int8 P.V) ----------------------------------------------------
// workspace of attn_fwd: one slot of stored logits per workgroup of its grid,
// then the q_v codes of every key tile
size_t attn_fwd_ws_bytes(int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t window);
// logits the forward can keep for the backward: one slot per (query block,
// batch x query head) item, in the forward's item order
size_t attn_keep_bytes(int64_t B, int64_t S, int64_t Hq, int64_t window);
// keep (nullable): the forward writes every item's logits there instead of
// its per-workgroup slots; the backward reads them instead of recomputing
hipError_t launch_attn_fwd(const float* Q, const float* K, const float* V, int64_t B, int64_t S, int64_t Hq,
                           int64_t Hkv, int64_t ldq, int64_t ldk, int64_t ldv, int64_t window, float s_v,
                           float* O, int64_t ldo, float* stats, float* logits, float* keep, const ExpConsts& ek,
                           hipStream_t st);
hipError_t launch_attn_bwd_dq(const float* Q, const float* K, const float* V, const float* O, const float* dO,
                              const float* stats, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t ldq,
                              int64_t ldk, int64_t ldv, int64_t ldo, int64_t window, float s_v, float* dQ,
                              const float* keep, const ExpConsts& ek, hipStream_t st);
hipError_t launch_attn_bwd_dkdv(const float* Q, const float* K, const float* V, const float* O, const float* dO,
                                const float* stats, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t ldq,
                                int64_t ldk, int64_t ldv, int64_t ldo, int64_t window, float s_v, float* dK,
                                float* dV, int64_t ldg, const float* keep, const ExpConsts& ek, hipStream_t st);

}  // namespace brl
