// optim.hip -- AdamW update in a fixed operation order, after the global clip.
//
// Recipe (Open-1B summary on onedev.kr, "Limits", recipe paragraph): AdamW
// with beta1 0.9, beta2 0.95, eps 1e-8, decoupled weight decay 0.1 (not on the
// input embedding, the norm weights or the RoPE table); peak learning rate
// 4.5e-4 after a linear warm-up of about 2.1B tokens, then one cosine decay to
// 10% of the peak at the 400B-token budget, keyed to consumed tokens.  The
// pages fix neither the operation order nor how the step's scalars are
// formed; this library's reading:
//   step scalars (host, binary64, each rounded once to binary32): lr,
//   c1 = 1 - beta1, c2 = 1 - beta2, bc1 = 1 - beta1^t, bc2 = 1 - beta2^t,
//   d = lr * wd;
//   per element, one binary32 operation at a time (no fusion, FTZ):
//     m = (beta1 * m) + (c1 * g)
//     v = (beta2 * v) + (c2 * (g * g))
//     u = (m / bc1) / (sqrt(v / bc2) + eps)
//     p = p - (d * p)            (tensors that decay only)
//     p = p - (lr * u)
// Elementwise and HBM-bound: 16-byte vectors of p, g, m, v in, p, m, v out.
#include <math.h>

#include "internal.hpp"

#pragma clang fp contract(off)

namespace brl {

// rbc1, rbc2: binary64 reciprocals of the bias corrections (nonzero for
// step >= 1), so m / bc1 and v / bc2 cost one binary64 multiply each
__device__ __forceinline__ void adamw_elem(float& p, float g, float& m, float& v, const brl_adamw_scalars& s,
                                           double rbc1, double rbc2, int decay) {
    m = f_add(f_mul(s.beta1, m), f_mul(s.c1, g));
    v = f_add(f_mul(s.beta2, v), f_mul(s.c2, f_mul(g, g)));
    const float u = f_div(f_div_by(m, rbc1), f_add(f_sqrt(f_div_by(v, rbc2)), s.eps));
    if (decay) p = f_sub(p, f_mul(s.d, p));
    p = f_sub(p, f_mul(s.lr, u));
}

__global__ __launch_bounds__(256) void adamw_v4_kernel(vf4* __restrict__ p, const vf4* __restrict__ g,
                                                       vf4* __restrict__ m, vf4* __restrict__ v, int64_t n4,
                                                       brl_adamw_scalars s, int decay) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const double rbc1 = 1.0 / (double)flush_f32(s.bc1), rbc2 = 1.0 / (double)flush_f32(s.bc2);
    vf4 pp = __builtin_nontemporal_load(p + i), gg = __builtin_nontemporal_load(g + i);
    vf4 mm = __builtin_nontemporal_load(m + i), vv = __builtin_nontemporal_load(v + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float pe = pp[e], me = mm[e], ve = vv[e];
        adamw_elem(pe, gg[e], me, ve, s, rbc1, rbc2, decay);
        pp[e] = pe; mm[e] = me; vv[e] = ve;
    }
    __builtin_nontemporal_store(pp, p + i);
    __builtin_nontemporal_store(mm, m + i);
    __builtin_nontemporal_store(vv, v + i);
}

__global__ __launch_bounds__(256) void adamw_scalar_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                           float* __restrict__ m, float* __restrict__ v,
                                                           int64_t n, brl_adamw_scalars s, int decay) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const double rbc1 = 1.0 / (double)flush_f32(s.bc1), rbc2 = 1.0 / (double)flush_f32(s.bc2);
    float pe = p[i], me = m[i], ve = v[i];
    adamw_elem(pe, g[i], me, ve, s, rbc1, rbc2, decay);
    p[i] = pe; m[i] = me; v[i] = ve;
}

static bool al16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; }

hipError_t launch_adamw(float* p, const float* g, float* m, float* v, int64_t n, const brl_adamw_scalars& s,
                        int decay, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t done = 0;
    if (al16(p) && al16(g) && al16(m) && al16(v)) {
        const int64_t n4 = n / 4;
        if (n4 > 0)
            hipLaunchKernelGGL(adamw_v4_kernel, dim3((unsigned)ceil_div(n4, 256)), dim3(256), 0, st,
                               reinterpret_cast<vf4*>(p), reinterpret_cast<const vf4*>(g),
                               reinterpret_cast<vf4*>(m), reinterpret_cast<vf4*>(v), n4, s, decay);
        done = n4 * 4;
    }
    if (done < n)
        hipLaunchKernelGGL(adamw_scalar_kernel, dim3((unsigned)ceil_div(n - done, 256)), dim3(256), 0, st,
                           p + done, g + done, m + done, v + done, n - done, s, decay);
    return hipGetLastError();
}

// ---- the step's scalars (host, binary64, rounded once) -----------------------------
static double lr_at(double tokens, const brl_adamw_config& c) {
    if (tokens < c.warmup_tokens) return c.peak_lr * tokens / c.warmup_tokens;
    double frac = (tokens - c.warmup_tokens) / (c.total_tokens - c.warmup_tokens);
    if (frac > 1.0) frac = 1.0;
    return c.min_lr + (c.peak_lr - c.min_lr) * 0.5 * (1.0 + cos(M_PI * frac));
}

void adamw_scalars(int64_t step, double tokens, const brl_adamw_config& c, brl_adamw_scalars* out) {
    const double lr = lr_at(tokens, c);
    out->beta1 = (float)c.beta1;
    out->beta2 = (float)c.beta2;
    out->c1 = (float)(1.0 - c.beta1);
    out->c2 = (float)(1.0 - c.beta2);
    out->bc1 = (float)(1.0 - pow(c.beta1, (double)step));
    out->bc2 = (float)(1.0 - pow(c.beta2, (double)step));
    out->eps = (float)c.eps;
    out->lr = (float)lr;
    out->d = (float)(lr * c.wd);
}

}  // namespace brl
