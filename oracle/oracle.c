/*
 * oracle.c -- plain, slow, CPU reference for the bitwise-reproducible int8 LSQ
 * linear layer and the ordered gradient reduction of "OPEN-1B: A Fully
 * Auditable Training Run" (Donaghy et al., Gensyn).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file.  Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or constant
 * generator with the HIP library.
 *
 * Sources followed (the pages give no code; everything here is written from
 * the prose):
 *   - onedev.kr "Open-1B" summary, section "How" (RepOps): one fixed reduction
 *     order, multiply and add never fused, subnormals flushed to zero.
 *   - same page, section "Use": LSQ int8 QAT on every attention/FFN linear,
 *     8-bit weights and activations, weight step 2*mean(|w|)/sqrt(q_max)
 *     recomputed every step; SwiGLU gate and up as one GEMM.
 *   - same page, "Limits" paragraphs: global L2 gradient-norm clip at 1.0;
 *     audit replay = running-sum reduce-scatter over virtual ranks in mesh
 *     order (replica-major, shard-minor), then TreeFold in the pairing order
 *     of a recursive-doubling all-reduce.
 * Points the pages leave open take these readings: RNE everywhere, clamp
 * to [-127,127], 32-wide sequential blocks then a level-by-level pairwise
 * tree, STE mask = select +0.
 *
 * Arithmetic model.  Every binary32 operation (add, sub, mul, div, sqrt) is
 * computed in IEEE double from the (DAZ-flushed) float operands and rounded
 * once to float.  Because 53 >= 2*24+2 that double rounding is innocuous, so
 * the result is the correctly rounded binary32 result.  A result that is tiny
 * (below 2^-126 after rounding to 24 bits with an unbounded exponent, the
 * IEEE 754 after-rounding definition) is replaced by a zero of the same sign
 * (FTZ).  Nothing relies on the x87/SSE control word except the
 * round-to-nearest-even mode, which each entry point resets explicitly.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * Parallelism is across independent outputs only; every output's operation
 * order is fixed, so results do not depend on the thread count.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Floating-point environment: round-to-nearest-even, no hardware FTZ/DAZ.  */
/* (MXCSR bits 6 = DAZ, 13-14 = rounding control, 15 = FTZ.)                */
/* ------------------------------------------------------------------------ */
static void fp_env_default(void) { _mm_setcsr(0x1F80u); }

#define PARALLEL_BEGIN _Pragma("omp parallel") { fp_env_default();
#define PARALLEL_END }

/* ------------------------------------------------------------------------ */
/* binary32 primitives (onedev.kr, "How": FTZ everywhere, no fusion)        */
/* ------------------------------------------------------------------------ */
static inline float flush(float x) {
    /* subnormal operand -> zero of the same sign; zeros, normals, inf, nan pass */
    return (fabsf(x) < FLT_MIN) ? copysignf(0.0f, x) : x;
}

/* Round a binary64 value to binary32 with flush-to-zero.  x is the exact
 * result (add, sub, mul of binary32 operands are exact in binary64) or its
 * binary64 rounding (div, sqrt; innocuous, see the header).  Tininess is
 * detected after rounding, as IEEE 754 defines it: x is first rounded to 24
 * significant bits as if the exponent range were unbounded, and a result of
 * magnitude below 2^-126 becomes a zero of the same sign. */
static float round_flush(double x) {
    if (fabs(x) < 0x1p-100) {
        float r = (float)(x * 0x1p100);          /* exact scaling, then 24-bit rounding */
        if (fabsf(r) < 0x1p-26f) return signbit(x) ? -0.0f : 0.0f;
        return (float)((double)r * 0x1p-100);    /* exact: a normal binary32 */
    }
    return (float)x;
}

float or_add(float a, float b) { return round_flush((double)flush(a) + (double)flush(b)); }
float or_sub(float a, float b) { return round_flush((double)flush(a) - (double)flush(b)); }
float or_mul(float a, float b) { return round_flush((double)flush(a) * (double)flush(b)); }
float or_div(float a, float b) { return round_flush((double)flush(a) / (double)flush(b)); }
float or_sqrt(float a) { return round_flush(sqrt((double)flush(a))); }

/* int32 -> binary32, round to nearest even (exact for |x| <= 2^24). */
float or_i2f(int32_t x) { return (float)(double)x; }

/* Round a binary32 value to the nearest integer, ties to even, written out
 * from the definition (floor, then compare the remainder with one half). */
float or_rne(float t) {
    if (!(fabsf(t) < 8388608.0f)) return t;          /* |t| >= 2^23 is integral; nan/inf pass */
    double f = floor((double)t);
    double d = (double)t - f;                        /* exact: both in double, |t| < 2^23 */
    double r;
    if (d > 0.5) r = f + 1.0;
    else if (d < 0.5) r = f;
    else r = (fmod(f, 2.0) == 0.0) ? f : f + 1.0;    /* tie: the even neighbour */
    return copysignf((float)r, t);                   /* keeps -0 for t in (-0.5, -0] */
}

/* ------------------------------------------------------------------------ */
/* CanonSum: 32-wide sequential blocks, then a pairwise tree level by level  */
/* ------------------------------------------------------------------------ */
#define OR_BLOCK 32

/* Sequential sum of one block, left to right, starting from its first term. */
static float block_sum(const float* p, int64_t n) {
    float s = p[0];
    for (int64_t i = 1; i < n; ++i) s = or_add(s, p[i]);
    return s;
}

/* Pairwise tree over b[0..J): each level adds neighbours (0,1), (2,3), ...;
 * an odd last node is carried up unchanged.  Works in place. */
static float pair_tree(float* b, int64_t J) {
    if (J == 0) return 0.0f;
    while (J > 1) {
        int64_t h = J / 2;
        for (int64_t i = 0; i < h; ++i) b[i] = or_add(b[2 * i], b[2 * i + 1]);
        if (J & 1) { b[h] = b[J - 1]; J = h + 1; } else { J = h; }
    }
    return b[0];
}

float or_pair_tree(float* b, int64_t J) { fp_env_default(); return pair_tree(b, J); }

/* CanonSum of p[0..n).  n == 0 gives +0. */
static float canon_sum(const float* p, int64_t n, float* scratch) {
    if (n == 0) return 0.0f;
    int64_t J = (n + OR_BLOCK - 1) / OR_BLOCK;
    for (int64_t j = 0; j < J; ++j) {
        int64_t len = n - j * OR_BLOCK;
        if (len > OR_BLOCK) len = OR_BLOCK;
        scratch[j] = block_sum(p + j * OR_BLOCK, len);
    }
    return pair_tree(scratch, J);
}

float or_canon_sum(const float* p, int64_t n) {
    fp_env_default();
    int64_t J = (n + OR_BLOCK - 1) / OR_BLOCK;
    float* b = (float*)malloc(sizeof(float) * (size_t)(J > 0 ? J : 1));
    float r = canon_sum(p, n, b);
    free(b);
    return r;
}

/* ------------------------------------------------------------------------ */
/* LSQ weight step and quantiser (onedev.kr, "Use"; "Limits" last paragraph) */
/* ------------------------------------------------------------------------ */
#define OR_QMAX 127

/* s_w = (2 * mean|w|) / sqrt(127), mean = CanonSum(|w|) / fl(count) over the
 * row-major weight; recomputed from the weight on every call. */
float or_weight_scale(const float* w, int64_t count) {
    fp_env_default();
    if (count <= 0) return 0.0f;
    int64_t J = (count + OR_BLOCK - 1) / OR_BLOCK;
    float* b = (float*)malloc(sizeof(float) * (size_t)J);
    PARALLEL_BEGIN
    #pragma omp for schedule(static)
    for (int64_t j = 0; j < J; ++j) {
        int64_t len = count - j * OR_BLOCK;
        if (len > OR_BLOCK) len = OR_BLOCK;
        const float* p = w + j * OR_BLOCK;
        float s = fabsf(p[0]);
        for (int64_t i = 1; i < len; ++i) s = or_add(s, fabsf(p[i]));
        b[j] = s;
    }
    PARALLEL_END
    float S = pair_tree(b, J);
    free(b);
    float mu = or_div(S, (float)(double)count);
    return or_div(or_mul(2.0f, mu), or_sqrt((float)OR_QMAX));
}

/* t = v / s; q = clamp(rne(t), -127, 127); in = (-127 <= t <= 127).
 * A zero step (all-zero weights) quantises everything to 0 and in range. */
static void quantize_one(float v, float s, int8_t* q, uint8_t* in) {
    if (s == 0.0f) { *q = 0; *in = 1; return; }
    float t = or_div(v, s);
    float r = or_rne(t);
    if (r > (float)OR_QMAX) r = (float)OR_QMAX;
    if (r < -(float)OR_QMAX) r = -(float)OR_QMAX;
    *q = (int8_t)(int)r;
    *in = (uint8_t)(t >= -(float)OR_QMAX && t <= (float)OR_QMAX);
}

void or_quantize(const float* v, int64_t n, float s, int8_t* q, uint8_t* in) {
    PARALLEL_BEGIN
    #pragma omp for schedule(static)
    for (int64_t i = 0; i < n; ++i) quantize_one(v[i], s, &q[i], &in[i]);
    PARALLEL_END
}

/* ------------------------------------------------------------------------ */
/* int8 GEMM by its plain definition: int64 dot products                     */
/* ------------------------------------------------------------------------ */
/* acc[m,n] = sum_k qx[m,k] * qw[n,k]; returns the largest |acc| seen. */
int64_t or_gemm_i8(const int8_t* qx, const int8_t* qw, int64_t M, int64_t K, int64_t N, int64_t* acc) {
    int64_t amax = 0;
    PARALLEL_BEGIN
    int64_t local = 0;
    #pragma omp for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int64_t)qx[m * K + k] * (int64_t)qw[n * K + k];
            acc[m * N + n] = s;
            if (llabs(s) > local) local = llabs(s);
        }
    #pragma omp critical
    { if (local > amax) amax = local; }
    PARALLEL_END
    return amax;
}

/* ------------------------------------------------------------------------ */
/* Own binary32 exp for SiLU (the pages name no transcendental).             */
/* Cody-Waite reduction x = k*ln2 + r, degree-7 Taylor polynomial in Horner  */
/* form, scaling by 2^k in two exact power-of-two steps.  Every step is one  */
/* of the binary32 primitives above.                                         */
/* ------------------------------------------------------------------------ */
static float pow2f(int e) {          /* 2^e for -126 <= e <= 127, from the exponent field */
    uint32_t bits = (uint32_t)(e + 127) << 23;
    float f; memcpy(&f, &bits, 4); return f;
}

static float e_l2e, e_ln2_hi, e_ln2_lo, e_c[8];
static int e_ready = 0;

static void e_init(void) {
    if (e_ready) return;
    /* log2(e) and ln 2 from the mathematical constants (long double), then
     * rounded to binary32; ln2_hi keeps 16 significant bits so k*ln2_hi is
     * exact for |k| < 2^8. */
    const long double LN2 = 0.693147180559945309417232121458176568L;
    e_l2e = (float)(1.0L / LN2);
    long double hi = floorl(LN2 * 65536.0L) / 65536.0L;      /* 16 fraction bits: ln2 < 1 */
    e_ln2_hi = (float)hi;
    e_ln2_lo = (float)(LN2 - hi);
    long double f = 1.0L;
    for (int i = 0; i < 8; ++i) { if (i > 0) f *= (long double)i; e_c[i] = (float)(1.0L / f); }
    e_ready = 1;
}

float or_exp(float x) {
    e_init();
    if (x != x) return x;
    if (x > 89.0f) return INFINITY;
    if (x < -104.0f) return 0.0f;
    float k = or_rne(or_mul(x, e_l2e));
    float r = or_sub(or_sub(x, or_mul(k, e_ln2_hi)), or_mul(k, e_ln2_lo));
    float p = e_c[7];
    for (int i = 6; i >= 0; --i) p = or_add(or_mul(p, r), e_c[i]);
    int ki = (int)k;
    int k1 = ki / 2;                 /* truncates toward zero */
    int k2 = ki - k1;
    return or_mul(or_mul(p, pow2f(k1)), pow2f(k2));
}

void or_exp_constants(float* out) {   /* l2e, ln2_hi, ln2_lo, c0..c7 */
    e_init();
    out[0] = e_l2e; out[1] = e_ln2_hi; out[2] = e_ln2_lo;
    for (int i = 0; i < 8; ++i) out[3 + i] = e_c[i];
}

/* SwiGLU forward on one (gate, up) pair: a = (g * sigma(g)) * u with
 * sigma(g) = 1 / (1 + E(-g)). */
static void swiglu_fwd_one(float g, float u, float* a, float* h_out, float* s_out) {
    float e = or_exp(-g);
    float s = or_div(1.0f, or_add(1.0f, e));
    float h = or_mul(g, s);
    *a = or_mul(h, u);
    if (h_out) *h_out = h;
    if (s_out) *s_out = s;
}

/* SwiGLU backward: du = dA*h; dsig' = s*(1 + g*(1 - s)); dg = (dA*u)*dsig'. */
static void swiglu_bwd_one(float g, float u, float dA, float* dg, float* du) {
    float a, h, s;
    swiglu_fwd_one(g, u, &a, &h, &s);
    *du = or_mul(dA, h);
    float d = or_mul(s, or_add(1.0f, or_mul(g, or_sub(1.0f, s))));
    *dg = or_mul(or_mul(dA, u), d);
}

void or_swiglu_fwd(const float* ypre, int64_t rows, int64_t N, float* act) {
    int64_t H = N / 2;
    e_init();
    PARALLEL_BEGIN
    #pragma omp for schedule(static)
    for (int64_t m = 0; m < rows; ++m)
        for (int64_t j = 0; j < H; ++j)
            swiglu_fwd_one(ypre[m * N + j], ypre[m * N + H + j], &act[m * H + j], NULL, NULL);
    PARALLEL_END
}

void or_swiglu_bwd(const float* ypre, const float* dact, int64_t rows, int64_t N, float* dypre) {
    int64_t H = N / 2;
    e_init();
    PARALLEL_BEGIN
    #pragma omp for schedule(static)
    for (int64_t m = 0; m < rows; ++m)
        for (int64_t j = 0; j < H; ++j)
            swiglu_bwd_one(ypre[m * N + j], ypre[m * N + H + j], dact[m * H + j],
                           &dypre[m * N + j], &dypre[m * N + H + j]);
    PARALLEL_END
}

/* ------------------------------------------------------------------------ */
/* QAT linear forward, for a list of rows of Y                               */
/* ------------------------------------------------------------------------ */
/* Y[m,:] for m in rows: acc = sum_k qx*qw (int64, asserted < 2^31),
 * Y = fl(acc) * (s_x * s_w), then + addend if given (unfused).
 * epilogue 1 (stacked SwiGLU): ypre gets Y, act gets SwiGLU(Y).
 * s_w is the weight step of the whole W (or_weight_scale).
 * Returns 0, or -1 if an accumulator would not fit in int32. */
int or_fwd_rows(const float* X, const float* W, int64_t M, int64_t K, int64_t N, float s_x,
                float s_w, const float* addend, int epilogue, const int64_t* rows, int64_t nrows,
                float* Y, float* ypre) {
    (void)M;
    fp_env_default();
    int8_t* qw = (int8_t*)malloc((size_t)(N * K));
    uint8_t* inw = (uint8_t*)malloc((size_t)(N * K));
    or_quantize(W, N * K, s_w, qw, inw);
    float s_y = or_mul(s_x, s_w);
    int bad = 0;
    e_init();
    PARALLEL_BEGIN
    int8_t* qx = (int8_t*)malloc((size_t)K);
    uint8_t* inx = (uint8_t*)malloc((size_t)K);
    float* row = (float*)malloc(sizeof(float) * (size_t)N);
    #pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t m = rows[r];
        for (int64_t k = 0; k < K; ++k) quantize_one(X[m * K + k], s_x, &qx[k], &inx[k]);
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) acc += (int64_t)qx[k] * (int64_t)qw[n * K + k];
            if (acc >= 2147483648LL || acc < -2147483648LL) bad = 1;
            float y = or_mul(or_i2f((int32_t)acc), s_y);
            if (addend) y = or_add(y, addend[m * N + n]);
            row[n] = y;
        }
        if (epilogue == 1) {
            int64_t H = N / 2;
            memcpy(&ypre[r * N], row, sizeof(float) * (size_t)N);
            for (int64_t j = 0; j < H; ++j) swiglu_fwd_one(row[j], row[H + j], &Y[r * H + j], NULL, NULL);
        } else {
            memcpy(&Y[r * N], row, sizeof(float) * (size_t)N);
        }
    }
    free(qx); free(inx); free(row);
    PARALLEL_END
    free(qw); free(inw);
    return bad ? -1 : 0;
}

/* Y[:, n] for n in cols (no activation): the same definition column-wise,
 * for sampling columns of a large product.  Ycols is [ncols, M]. */
int or_fwd_cols(const float* X, const float* W, int64_t M, int64_t K, int64_t N, float s_x,
                float s_w, const int64_t* cols, int64_t ncols, float* Ycols) {
    (void)N;
    fp_env_default();
    int8_t* qx = (int8_t*)malloc((size_t)(M * K > 0 ? M * K : 1));
    uint8_t* inx = (uint8_t*)malloc((size_t)(M * K > 0 ? M * K : 1));
    or_quantize(X, M * K, s_x, qx, inx);
    float s_y = or_mul(s_x, s_w);
    int bad = 0;
    PARALLEL_BEGIN
    int8_t* qw = (int8_t*)malloc((size_t)K);
    #pragma omp for schedule(dynamic, 1)
    for (int64_t c = 0; c < ncols; ++c) {
        int64_t n = cols[c];
        for (int64_t k = 0; k < K; ++k) { uint8_t in; quantize_one(W[n * K + k], s_w, &qw[k], &in); }
        for (int64_t m = 0; m < M; ++m) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) acc += (int64_t)qx[m * K + k] * (int64_t)qw[k];
            if (acc >= 2147483648LL || acc < -2147483648LL) bad = 1;
            Ycols[c * M + m] = or_mul(or_i2f((int32_t)acc), s_y);
        }
    }
    free(qw);
    PARALLEL_END
    free(qx); free(inx);
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Straight-through backward                                                 */
/* ------------------------------------------------------------------------ */
/* dX[m,k] = in_x[m,k] ? CanonSum_n(dY[m,n] * What[n,k]) : +0, What = fl(q_w*s_w),
 * for m in rows.  dY holds the pre-activation gradient rows [nrows, N]
 * (already through the SwiGLU backward where that applies). */
void or_dx_rows(const float* dY_rows, const float* X, const float* W, int64_t K, int64_t N,
                float s_x, float s_w, const int64_t* rows, int64_t nrows, float* dX) {
    fp_env_default();
    int8_t* qw = (int8_t*)malloc((size_t)(N * K));
    uint8_t* inw = (uint8_t*)malloc((size_t)(N * K));
    or_quantize(W, N * K, s_w, qw, inw);
    float* What = (float*)malloc(sizeof(float) * (size_t)(N * K));
    for (int64_t i = 0; i < N * K; ++i) What[i] = or_mul(or_i2f(qw[i]), s_w);
    PARALLEL_BEGIN
    float* p = (float*)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
    float* sc = (float*)malloc(sizeof(float) * (size_t)(N / OR_BLOCK + 2));
    #pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t m = rows[r];
        for (int64_t k = 0; k < K; ++k) {
            int8_t q; uint8_t in;
            quantize_one(X[m * K + k], s_x, &q, &in);
            float v = 0.0f;
            if (in) {
                for (int64_t n = 0; n < N; ++n) p[n] = or_mul(dY_rows[r * N + n], What[n * K + k]);
                v = canon_sum(p, N, sc);
            }
            dX[r * K + k] = v;
        }
    }
    free(p); free(sc);
    PARALLEL_END
    free(qw); free(inw); free(What);
}

/* dW[n,k] for n in wrows.  dY_cols holds, for each selected n, the column
 * dY[0..M, n] as a contiguous [M] vector.  The M rows are taken as
 * microbatches of mb rows each (mb = M for a single batch): per microbatch
 * b, dW_b[n,k] = in_w[n,k] ? CanonSum over its rows of dY[m,n]*Xhat[m,k] : +0,
 * Xhat = fl(q_x*s_x); then D = dW_0, D = D + dW_b for b = 1, 2, ... */
void or_dw_rows(const float* dY_cols, const float* X, const float* W, int64_t M, int64_t K,
                float s_x, float s_w, const int64_t* wrows, int64_t nrows, int64_t mb, float* dW) {
    fp_env_default();
    if (mb <= 0) mb = M;
    float* Xhat = (float*)malloc(sizeof(float) * (size_t)(M * K > 0 ? M * K : 1));
    PARALLEL_BEGIN
    #pragma omp for schedule(static)
    for (int64_t i = 0; i < M * K; ++i) {
        int8_t q; uint8_t in;
        quantize_one(X[i], s_x, &q, &in);
        Xhat[i] = or_mul(or_i2f(q), s_x);
    }
    PARALLEL_END
    int64_t nb = (M + mb - 1) / mb;
    PARALLEL_BEGIN
    float* p = (float*)malloc(sizeof(float) * (size_t)(mb > 0 ? mb : 1));
    float* sc = (float*)malloc(sizeof(float) * (size_t)(mb / OR_BLOCK + 2));
    #pragma omp for schedule(dynamic, 1) collapse(2)
    for (int64_t r = 0; r < nrows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            int64_t n = wrows[r];
            int8_t q; uint8_t in;
            quantize_one(W[n * K + k], s_w, &q, &in);
            float D = 0.0f;
            for (int64_t b = 0; b < nb; ++b) {
                int64_t m0 = b * mb, len = M - m0 < mb ? M - m0 : mb;
                float v = 0.0f;
                if (in) {
                    for (int64_t i = 0; i < len; ++i) p[i] = or_mul(dY_cols[r * M + m0 + i], Xhat[(m0 + i) * K + k]);
                    v = canon_sum(p, len, sc);
                }
                D = (b == 0) ? v : or_add(D, v);
            }
            dW[r * K + k] = D;
        }
    free(p); free(sc);
    PARALLEL_END
    free(Xhat);
}

/* ------------------------------------------------------------------------ */
/* Audit replay of the gradient reduction (onedev.kr, "Limits", audit ¶)     */
/* ------------------------------------------------------------------------ */
/* Running sum for virtual rank v = r*S + s in mesh order:
 * A_r = G_v when s == 0 (first), else A_r = A_r + G_v. */
void or_replay_accumulate(float* A, const float* G, int64_t len, int first) {
    PARALLEL_BEGIN
    #pragma omp for schedule(static)
    for (int64_t i = 0; i < len; ++i) A[i] = first ? G[i] : or_add(A[i], G[i]);
    PARALLEL_END
}

/* TreeFold: simulate the cluster's recursive-doubling all-reduce over R
 * replica ranks, element by element.  p = largest power of two <= R; ranks
 * i >= p first send to rank i - p, which adds; then for k = 1, 2, 4, ... < p
 * rank i exchanges with rank i xor k and both add what they hold.  Every
 * rank ends with the same bits; the result is rank 0's.  Returns 0, or -1 if
 * two ranks ever disagree. */
int or_treefold(const float* const* A, int R, int64_t len, float* T) {
    if (R <= 0 || R > 64) return -2;
    int p = 1;
    while (p * 2 <= R) p *= 2;
    int bad = 0;
    PARALLEL_BEGIN
    float v[64], nv[64];
    #pragma omp for schedule(static)
    for (int64_t e = 0; e < len; ++e) {
        for (int i = 0; i < R; ++i) v[i] = A[i][e];
        for (int i = 0; i + p < R; ++i) v[i] = or_add(v[i], v[i + p]);
        for (int k = 1; k < p; k *= 2) {
            for (int i = 0; i < p; ++i) nv[i] = or_add(v[i], v[i ^ k]);
            for (int i = 0; i < p; ++i) v[i] = nv[i];
        }
        for (int i = 1; i < p; ++i)
            if (memcmp(&v[i], &v[0], 4) != 0) bad = 1;
        T[e] = v[0];
    }
    PARALLEL_END
    return bad ? -1 : 0;
}

/* Global L2 norm: nu = sqrt(CanonSum(T_i * T_i)) over the flat vector. */
float or_l2norm(const float* T, int64_t len) {
    fp_env_default();
    if (len <= 0) return 0.0f;
    int64_t J = (len + OR_BLOCK - 1) / OR_BLOCK;
    float* b = (float*)malloc(sizeof(float) * (size_t)J);
    PARALLEL_BEGIN
    #pragma omp for schedule(static)
    for (int64_t j = 0; j < J; ++j) {
        int64_t n = len - j * OR_BLOCK;
        if (n > OR_BLOCK) n = OR_BLOCK;
        const float* t = T + j * OR_BLOCK;
        float s = or_mul(t[0], t[0]);
        for (int64_t i = 1; i < n; ++i) s = or_add(s, or_mul(t[i], t[i]));
        b[j] = s;
    }
    PARALLEL_END
    float Q = pair_tree(b, J);
    free(b);
    return or_sqrt(Q);
}

/* Clip to max_norm: when nu > max_norm, kappa = max_norm / (nu + eps) and
 * T_i = T_i * kappa; otherwise T is left as it is.  Returns kappa (1 when
 * no clipping happens). */
float or_clip(float* T, int64_t len, float nu, float max_norm, float eps) {
    fp_env_default();
    if (!(nu > max_norm)) return 1.0f;
    float kappa = or_div(max_norm, or_add(nu, eps));
    PARALLEL_BEGIN
    #pragma omp for schedule(static)
    for (int64_t i = 0; i < len; ++i) T[i] = or_mul(T[i], kappa);
    PARALLEL_END
    return kappa;
}

/* ---- AdamW update in a fixed operation order ---------------------------------
 * Recipe: AdamW with beta1 0.9, beta2 0.95, eps 1e-8, decoupled weight decay
 * 0.1 (not on the input embedding, the norm weights or the RoPE table), after
 * the global clip; peak learning rate 4.5e-4 after a linear warm-up of about
 * 2.1B tokens, then one cosine decay to 10% of the peak at the 400B-token
 * budget, keyed to consumed tokens (onedev.kr summary, "Limits", recipe
 * paragraph).  The pages fix neither the operation order nor how the step's
 * scalars are formed; the reading taken:
 *   step scalars, in binary64 from the step t >= 1 and the tokens consumed,
 *   each rounded once to binary32: lr, c1 = 1 - beta1, c2 = 1 - beta2,
 *   bc1 = 1 - beta1^t, bc2 = 1 - beta2^t, d = lr * wd;
 *   per element, each operation one binary32 operation (flushed), in order:
 *     m = (beta1 * m) + (c1 * g)
 *     v = (beta2 * v) + (c2 * (g * g))
 *     u = (m / bc1) / (sqrt(v / bc2) + eps)
 *     p = p - (d * p)            (only for tensors that decay)
 *     p = p - (lr * u)                                                      */
void or_adamw(float* p, const float* g, float* m, float* v, int64_t n, float beta1, float beta2, float c1,
              float c2, float bc1, float bc2, float eps, float lr, float d, int decay) {
    fp_env_default();
    PARALLEL_BEGIN
    #pragma omp for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const float mi = or_add(or_mul(beta1, m[i]), or_mul(c1, g[i]));
        const float vi = or_add(or_mul(beta2, v[i]), or_mul(c2, or_mul(g[i], g[i])));
        const float u = or_div(or_div(mi, bc1), or_add(or_sqrt(or_div(vi, bc2)), eps));
        float pi = p[i];
        if (decay) pi = or_sub(pi, or_mul(d, pi));
        pi = or_sub(pi, or_mul(lr, u));
        m[i] = mi;
        v[i] = vi;
        p[i] = pi;
    }
    PARALLEL_END
}

/* ------------------------------------------------------------------------ */
/* Attention with int8 P.V (onedev.kr summary, "Use", attention paragraph:   */
/* the P.V product of flash attention on int8 tensor cores, the QK^T logits  */
/* and the softmax kept in high precision; GQA with 16 query heads sharing   */
/* 4 KV heads; 512-token sliding window, full causal on some layers).        */
/* ------------------------------------------------------------------------ */
/* Element (b, i, h, d) of Q is Q[(b*S + i)*ldq + h*D + d]; K, V, O alike.
 * Query head h reads KV head h / (Hq / Hkv).  Row i attends to keys
 * j in [lo, i], lo = max(0, i - window + 1) (window <= 0: lo = 0).
 * Readings (the pages fix none of these steps):
 *   s_ij = CanonSum_d(q_id * k_jd) * c,  c = 1 / sqrt(D) (each op rounded);
 *   m_i  = max over the row's keys (the first key, then strictly larger ones);
 *   p_ij = E(s_ij - m_i) for the row's keys, +0 for every other key;
 *   l_i  = CanonSum over the whole key axis j = 0..S-1 of p_ij;
 *   q_p  = clamp(rne(p * 127), 0, 127);  q_v = the LSQ quantiser with step s_v;
 *   acc_id = sum_j q_p,ij * q_v,jd       (exact integers);
 *   O_id = (fl(acc_id) * s_v) / (l_i * 127).                                 */
/* One output row (b, i, h) of the attention: O row (D floats) into o. */
static int attn_row(const float* Q, const float* K, const int8_t* qv, int64_t S, int64_t Hq, int64_t Hkv,
                    int64_t D, int64_t ldq, int64_t ldk, int64_t window, float s_v, float c, int64_t b, int64_t i,
                    int64_t h, float* prod, float* p, float* s, float* scratch, int64_t* acc, float* o) {
    const int64_t hk = h / (Hq / Hkv);
    const int64_t lo = (window > 0 && i - window + 1 > 0) ? i - window + 1 : 0;
    const float* q = Q + (b * S + i) * ldq + h * D;
    for (int64_t j = lo; j <= i; ++j) {
        const float* k = K + (b * S + j) * ldk + hk * D;
        for (int64_t d = 0; d < D; ++d) prod[d] = or_mul(q[d], k[d]);
        s[j] = or_mul(canon_sum(prod, D, scratch), c);
    }
    float m = s[lo];
    for (int64_t j = lo + 1; j <= i; ++j)
        if (s[j] > m) m = s[j];
    for (int64_t j = 0; j < S; ++j) p[j] = 0.0f;
    for (int64_t j = lo; j <= i; ++j) p[j] = or_exp(or_sub(s[j], m));
    const float l = canon_sum(p, S, scratch);
    for (int64_t d = 0; d < D; ++d) acc[d] = 0;
    for (int64_t j = lo; j <= i; ++j) {
        float r = or_rne(or_mul(p[j], 127.0f));
        if (r > 127.0f) r = 127.0f;
        if (r < 0.0f) r = 0.0f;
        const int64_t qp = (int64_t)r;
        const int8_t* vq = qv + ((b * S + j) * Hkv + hk) * D;
        for (int64_t d = 0; d < D; ++d) acc[d] += qp * (int64_t)vq[d];
    }
    const float t = or_mul(l, 127.0f);
    int bad = 0;
    for (int64_t d = 0; d < D; ++d) {
        if (acc[d] > INT32_MAX || acc[d] < INT32_MIN) bad = 1;
        o[d] = or_div(or_mul(or_i2f((int32_t)acc[d]), s_v), t);
    }
    return bad;
}

/* Quantised V, [B, S, Hkv, D]. */
static int8_t* attn_quantize_v(const float* V, int64_t B, int64_t S, int64_t Hkv, int64_t D, int64_t ldv,
                               float s_v) {
    int8_t* qv = (int8_t*)malloc((size_t)(B * S * Hkv * D > 0 ? B * S * Hkv * D : 1));
    PARALLEL_BEGIN
    #pragma omp for schedule(static)
    for (int64_t r = 0; r < B * S; ++r)
        for (int64_t h = 0; h < Hkv; ++h)
            for (int64_t d = 0; d < D; ++d) {
                uint8_t in;
                quantize_one(V[r * ldv + h * D + d], s_v, &qv[(r * Hkv + h) * D + d], &in);
            }
    PARALLEL_END
    return qv;
}

/* Rows given as flat ids (b*S + i)*Hq + h, or every row when rows == NULL
 * (then out row r is O row r).  out: nrows x D floats, row pitch ldo. */
int or_attn_fwd_rows(const float* Q, const float* K, const float* V, int64_t B, int64_t S, int64_t Hq,
                     int64_t Hkv, int64_t D, int64_t ldq, int64_t ldk, int64_t ldv, int64_t window, float s_v,
                     const int64_t* rows, int64_t nrows, float* out, int64_t ldo) {
    fp_env_default();
    e_init();
    if (Hkv <= 0 || Hq % Hkv != 0) return -1;
    const float c = or_div(1.0f, or_sqrt((float)(double)D));
    int8_t* qv = attn_quantize_v(V, B, S, Hkv, D, ldv, s_v);
    int bad = 0;
    PARALLEL_BEGIN
    float* prod = (float*)malloc(sizeof(float) * (size_t)D);
    float* p = (float*)malloc(sizeof(float) * (size_t)S);
    float* s = (float*)malloc(sizeof(float) * (size_t)S);
    float* scratch = (float*)malloc(sizeof(float) * (size_t)(S / OR_BLOCK + D / OR_BLOCK + 2));
    int64_t* acc = (int64_t*)malloc(sizeof(int64_t) * (size_t)D);
    #pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t row = rows ? rows[r] : r;
        const int64_t h = row % Hq, i = (row / Hq) % S, b = row / (Hq * S);
        if (attn_row(Q, K, qv, S, Hq, Hkv, D, ldq, ldk, window, s_v, c, b, i, h, prod, p, s, scratch, acc,
                     out + r * ldo)) {
            #pragma omp atomic write
            bad = 1;
        }
    }
    free(prod); free(p); free(s); free(scratch); free(acc);
    PARALLEL_END
    free(qv);
    return bad ? -2 : 0;
}

/* Attention with int8 P.V (onedev.kr summary, "Use", attention paragraph;
 * readings above attn_row): every row, O row (b, i, h) at
 * O[(b*S + i)*ldo + h*D]. */
int or_attn_fwd(const float* Q, const float* K, const float* V, int64_t B, int64_t S, int64_t Hq,
                int64_t Hkv, int64_t D, int64_t ldq, int64_t ldk, int64_t ldv, int64_t window, float s_v,
                float* O, int64_t ldo) {
    if (ldo != Hq * D) return -1;     /* rows are then O + row * D */
    return or_attn_fwd_rows(Q, K, V, B, S, Hq, Hkv, D, ldq, ldk, ldv, window, s_v, NULL, B * S * Hq, O, D);
}

/* ∇Q of the attention (onedev.kr summary, "Use", attention paragraph: the
 * attention backward accumulates ∇Q in 64-bit fixed point).  Readings, with
 * s, m, p, l, q_v as in the forward and O the forward's output:
 *   P_ij  = p_ij / l_i
 *   dP_ij = CanonSum_d(dO_id * V^_jd),  V^ = fl(q_v * s_v)
 *   Delta_i = CanonSum_d(dO_id * O_id)
 *   dS_ij = P_ij * (dP_ij - Delta_i) on the row's keys, +0 on other keys
 *   u_igd = CanonSum over the 64 key positions 64g .. 64g+63 of dS_ij * K_jd
 *           (zeros past the row's keys and past S)
 *   dQ_id = (fl(sum_g rne(u_igd * 2^40)) * 2^-40) * c
 * The tile sums u are fixed-point numbers with 40 fraction bits, summed as
 * exact int64 (any order gives the same sum); the total is rounded once to
 * binary32.  Returns -3 if a term or the sum leaves the int64 range. */
#define OR_ATTN_TILE 64
#define OR_DQ_FRAC 40
int or_attn_bwd_dq_rows(const float* Q, const float* K, const float* V, const float* O, const float* dO,
                        int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t ldq, int64_t ldk,
                        int64_t ldv, int64_t ldo, int64_t window, float s_v, const int64_t* rows, int64_t nrows,
                        float* out, int64_t ldout) {
    fp_env_default();
    e_init();
    if (Hkv <= 0 || Hq % Hkv != 0) return -1;
    const int64_t group = Hq / Hkv;
    const float c = or_div(1.0f, or_sqrt((float)(double)D));
    int8_t* qv = attn_quantize_v(V, B, S, Hkv, D, ldv, s_v);
    const int64_t ntile = (S + OR_ATTN_TILE - 1) / OR_ATTN_TILE;
    int bad = 0;
    PARALLEL_BEGIN
    float* prod = (float*)malloc(sizeof(float) * (size_t)(D > OR_ATTN_TILE ? D : OR_ATTN_TILE));
    float* p = (float*)malloc(sizeof(float) * (size_t)S);
    float* s = (float*)malloc(sizeof(float) * (size_t)S);
    float* ds = (float*)malloc(sizeof(float) * (size_t)(ntile * OR_ATTN_TILE));
    float* scratch = (float*)malloc(sizeof(float) * (size_t)(S / OR_BLOCK + D / OR_BLOCK + 4));
    int64_t* acc = (int64_t*)malloc(sizeof(int64_t) * (size_t)D);
    #pragma omp for schedule(dynamic, 8)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t row = rows ? rows[r] : r;
        const int64_t h = row % Hq, i = (row / Hq) % S, b = row / (Hq * S);
        const int64_t hk = h / group;
        const int64_t lo = (window > 0 && i - window + 1 > 0) ? i - window + 1 : 0;
        const float* q = Q + (b * S + i) * ldq + h * D;
        const float* go = dO + (b * S + i) * ldo + h * D;
        const float* o = O + (b * S + i) * ldo + h * D;
        /* forward quantities */
        for (int64_t j = lo; j <= i; ++j) {
            const float* k = K + (b * S + j) * ldk + hk * D;
            for (int64_t d = 0; d < D; ++d) prod[d] = or_mul(q[d], k[d]);
            s[j] = or_mul(canon_sum(prod, D, scratch), c);
        }
        float m = s[lo];
        for (int64_t j = lo + 1; j <= i; ++j)
            if (s[j] > m) m = s[j];
        for (int64_t j = 0; j < S; ++j) p[j] = 0.0f;
        for (int64_t j = lo; j <= i; ++j) p[j] = or_exp(or_sub(s[j], m));
        const float l = canon_sum(p, S, scratch);
        /* backward */
        for (int64_t d = 0; d < D; ++d) prod[d] = or_mul(go[d], o[d]);
        const float delta = canon_sum(prod, D, scratch);
        for (int64_t j = 0; j < ntile * OR_ATTN_TILE; ++j) ds[j] = 0.0f;
        for (int64_t j = lo; j <= i; ++j) {
            const int8_t* vq = qv + ((b * S + j) * Hkv + hk) * D;
            for (int64_t d = 0; d < D; ++d) prod[d] = or_mul(go[d], or_mul(or_i2f(vq[d]), s_v));
            const float dp = canon_sum(prod, D, scratch);
            ds[j] = or_mul(or_div(p[j], l), or_sub(dp, delta));
        }
        for (int64_t d = 0; d < D; ++d) acc[d] = 0;
        for (int64_t g = 0; g < ntile; ++g) {
            for (int64_t d = 0; d < D; ++d) {
                for (int64_t t = 0; t < OR_ATTN_TILE; ++t) {
                    const int64_t j = g * OR_ATTN_TILE + t;
                    const float kv = j < S ? K[(b * S + j) * ldk + hk * D + d] : 0.0f;
                    prod[t] = or_mul(ds[j], kv);
                }
                const float u = canon_sum(prod, OR_ATTN_TILE, scratch);
                const double x = rint((double)u * 0x1p40);
                if (!(fabs(x) < 0x1p62)) {
                    #pragma omp atomic write
                    bad = 3;
                    continue;
                }
                const int64_t fx = (int64_t)x;
                if (__builtin_add_overflow(acc[d], fx, &acc[d])) {
                    #pragma omp atomic write
                    bad = 3;
                }
            }
        }
        float* dq = out + r * ldout;
        for (int64_t d = 0; d < D; ++d)
            dq[d] = or_mul(or_mul(round_flush((double)(float)acc[d]), 0x1p-40f), c);
    }
    free(prod); free(p); free(s); free(ds); free(scratch); free(acc);
    PARALLEL_END
    free(qv);
    return bad ? -bad : 0;
}

/* dK and dV of the attention (onedev.kr summary, "Use", attention paragraph:
 * the pages give the 64-bit fixed-point accumulation for the query gradient
 * and say nothing of the key and value gradients).  Readings, with s, m, p,
 * l, q_v, V^, P, dP, Delta and dS as in or_attn_bwd_dq_rows:
 *   w_hgjd = CanonSum over the 64 query positions 64g .. 64g+63 of
 *            P_ij * dO_id   (query head h of j's group; +0 terms for rows
 *            that do not attend key j and past S)
 *   z_hgjd = the same sum of dS_ij * Q_id
 *   dV_jd  = q_v in range ? fl(sum_{h,g} rne(w * 2^40)) * 2^-40 : +0
 *   dK_jd  = (fl(sum_{h,g} rne(z * 2^40)) * 2^-40) * c
 * i.e. the query-tile sums take the fixed-point format of dQ, and the sum
 * over tiles and over the group's query heads is exact (order-free).  The
 * masks are the STE of the LSQ quantiser of V; the quantiser of p is passed
 * straight through (P = p / l, as in dS).
 * Key rows by flat id (b*S + j)*Hkv + hk (all rows when rows == NULL);
 * out rows r: dK at dk + r*ldout, dV at dv + r*ldout.  Returns -3 if a term
 * or a sum leaves the int64 range. */
static void attn_row_stats(const float* Q, const float* K, const float* O, const float* dO, int64_t S,
                           int64_t Hq, int64_t Hkv, int64_t D, int64_t ldq, int64_t ldk, int64_t ldo,
                           int64_t window, float c, int64_t b, int64_t i, int64_t h, float* s, float* p,
                           float* prod, float* scratch, float* out3) {
    const int64_t hk = h / (Hq / Hkv);
    const int64_t lo = (window > 0 && i - window + 1 > 0) ? i - window + 1 : 0;
    const float* q = Q + (b * S + i) * ldq + h * D;
    for (int64_t j = lo; j <= i; ++j) {
        const float* k = K + (b * S + j) * ldk + hk * D;
        for (int64_t d = 0; d < D; ++d) prod[d] = or_mul(q[d], k[d]);
        s[j] = or_mul(canon_sum(prod, D, scratch), c);
    }
    float m = s[lo];
    for (int64_t j = lo + 1; j <= i; ++j)
        if (s[j] > m) m = s[j];
    for (int64_t j = 0; j < S; ++j) p[j] = 0.0f;
    for (int64_t j = lo; j <= i; ++j) p[j] = or_exp(or_sub(s[j], m));
    const float* go = dO + (b * S + i) * ldo + h * D;
    const float* o = O + (b * S + i) * ldo + h * D;
    for (int64_t d = 0; d < D; ++d) prod[d] = or_mul(go[d], o[d]);
    out3[0] = m;
    out3[1] = canon_sum(p, S, scratch);
    out3[2] = canon_sum(prod, D, scratch);
}

static int fx_add(int64_t* acc, float u) {
    const double x = rint((double)u * 0x1p40);
    if (!(fabs(x) < 0x1p62)) return 1;
    return __builtin_add_overflow(*acc, (int64_t)x, acc) ? 1 : 0;
}

int or_attn_bwd_dkdv_rows(const float* Q, const float* K, const float* V, const float* O, const float* dO,
                          int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t ldq, int64_t ldk,
                          int64_t ldv, int64_t ldo, int64_t window, float s_v, const int64_t* rows,
                          int64_t nrows, float* dk, float* dv, int64_t ldout) {
    fp_env_default();
    e_init();
    if (Hkv <= 0 || Hq % Hkv != 0) return -1;
    const int64_t group = Hq / Hkv;
    const float c = or_div(1.0f, or_sqrt((float)(double)D));
    int8_t* qv = attn_quantize_v(V, B, S, Hkv, D, ldv, s_v);
    /* (m_i, l_i, Delta_i) of every query row that attends one of the key rows */
    const int64_t nq = B * S * Hq;
    float* st = (float*)malloc(sizeof(float) * (size_t)(3 * nq > 0 ? 3 * nq : 1));
    uint8_t* need = (uint8_t*)calloc((size_t)(nq > 0 ? nq : 1), 1);
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t row = rows ? rows[r] : r;
        const int64_t hk = row % Hkv, j = (row / Hkv) % S, b = row / (Hkv * S);
        const int64_t ihi = (window > 0 && j + window - 1 < S - 1) ? j + window - 1 : S - 1;
        for (int64_t i = j; i <= ihi; ++i)
            for (int64_t h = hk * group; h < (hk + 1) * group; ++h) need[(b * S + i) * Hq + h] = 1;
    }
    int bad = 0;
    PARALLEL_BEGIN
    float* prod = (float*)malloc(sizeof(float) * (size_t)(D > OR_ATTN_TILE ? D : OR_ATTN_TILE));
    float* p = (float*)malloc(sizeof(float) * (size_t)S);
    float* s = (float*)malloc(sizeof(float) * (size_t)S);
    float* scratch = (float*)malloc(sizeof(float) * (size_t)(S / OR_BLOCK + D / OR_BLOCK + 4));
    float* tw = (float*)malloc(sizeof(float) * (size_t)(OR_ATTN_TILE * D));
    float* tz = (float*)malloc(sizeof(float) * (size_t)(OR_ATTN_TILE * D));
    int64_t* accv = (int64_t*)malloc(sizeof(int64_t) * (size_t)D);
    int64_t* acck = (int64_t*)malloc(sizeof(int64_t) * (size_t)D);
    #pragma omp for schedule(dynamic, 16)
    for (int64_t qrow = 0; qrow < nq; ++qrow) {
        if (!need[qrow]) continue;
        const int64_t h = qrow % Hq, i = (qrow / Hq) % S, b = qrow / (Hq * S);
        attn_row_stats(Q, K, O, dO, S, Hq, Hkv, D, ldq, ldk, ldo, window, c, b, i, h, s, p, prod, scratch,
                       st + 3 * qrow);
    }
    #pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t row = rows ? rows[r] : r;
        const int64_t hk = row % Hkv, j = (row / Hkv) % S, b = row / (Hkv * S);
        const float* k = K + (b * S + j) * ldk + hk * D;
        const int8_t* vq = qv + ((b * S + j) * Hkv + hk) * D;
        for (int64_t d = 0; d < D; ++d) accv[d] = acck[d] = 0;
        for (int64_t h = hk * group; h < (hk + 1) * group; ++h) {
            for (int64_t g = j / OR_ATTN_TILE; g * OR_ATTN_TILE < S; ++g) {
                /* terms of the tile's 64 query positions, position-major */
                int any = 0;
                for (int64_t t = 0; t < OR_ATTN_TILE; ++t) {
                    const int64_t i = g * OR_ATTN_TILE + t;
                    const int64_t lo = (window > 0 && i - window + 1 > 0) ? i - window + 1 : 0;
                    float P = 0.0f, dS = 0.0f;
                    if (i < S && j <= i && j >= lo) {
                        any = 1;
                        const float* st3 = st + 3 * ((b * S + i) * Hq + h);
                        const float* q = Q + (b * S + i) * ldq + h * D;
                        const float* go = dO + (b * S + i) * ldo + h * D;
                        for (int64_t d = 0; d < D; ++d) prod[d] = or_mul(q[d], k[d]);
                        const float sij = or_mul(canon_sum(prod, D, scratch), c);
                        P = or_div(or_exp(or_sub(sij, st3[0])), st3[1]);
                        for (int64_t d = 0; d < D; ++d) prod[d] = or_mul(go[d], or_mul(or_i2f(vq[d]), s_v));
                        const float dp = canon_sum(prod, D, scratch);
                        dS = or_mul(P, or_sub(dp, st3[2]));
                    }
                    for (int64_t d = 0; d < D; ++d) {
                        const float gv = i < S ? dO[(b * S + i) * ldo + h * D + d] : 0.0f;
                        const float qd = i < S ? Q[(b * S + i) * ldq + h * D + d] : 0.0f;
                        tw[d * OR_ATTN_TILE + t] = or_mul(P, gv);
                        tz[d * OR_ATTN_TILE + t] = or_mul(dS, qd);
                    }
                }
                if (!any) break;     /* no later tile attends key j either */
                for (int64_t d = 0; d < D; ++d) {
                    int e = fx_add(&accv[d], canon_sum(tw + d * OR_ATTN_TILE, OR_ATTN_TILE, scratch));
                    e |= fx_add(&acck[d], canon_sum(tz + d * OR_ATTN_TILE, OR_ATTN_TILE, scratch));
                    if (e) {
                        #pragma omp atomic write
                        bad = 3;
                    }
                }
            }
        }
        float* ok = dk + r * ldout;
        float* ov = dv + r * ldout;
        for (int64_t d = 0; d < D; ++d) {
            int8_t q;
            uint8_t in;
            quantize_one(V[(b * S + j) * ldv + hk * D + d], s_v, &q, &in);
            ov[d] = in ? or_mul(round_flush((double)(float)accv[d]), 0x1p-40f) : 0.0f;
            ok[d] = or_mul(or_mul(round_flush((double)(float)acck[d]), 0x1p-40f), c);
        }
    }
    free(prod); free(p); free(s); free(scratch); free(tw); free(tz); free(accv); free(acck);
    PARALLEL_END
    free(st); free(need); free(qv);
    return bad ? -bad : 0;
}

void or_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int or_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
