// api.hip -- the C ABI of libbrlsq (declared in include/brlsq.h): argument
// checks, workspace carving and the launch sequence of each call.  No call
// allocates device memory or synchronises the host.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "internal.hpp"

namespace brl {

// ---- launch shapes of one call ---------------------------------------------------
bool resolve_tuning(const brl_tuning* t, Tuning* out) {
    Tuning r{0, 256, 1, 2, 1};
    if (t) {
        if (t->bwd_chunk_log2 < 0 || t->bwd_chunk_log2 > 7) return false;
        r.chunk_log2 = t->bwd_chunk_log2;
        if (t->reduce_wg_blocks != 0) {
            if (t->reduce_wg_blocks != 64 && t->reduce_wg_blocks != 128 && t->reduce_wg_blocks != 256) return false;
            r.wg_blocks = t->reduce_wg_blocks;
        }
        if (t->stream_vec != 0) {
            if (t->stream_vec != 1 && t->stream_vec != 2 && t->stream_vec != 4) return false;
            r.vec = t->stream_vec;
        }
        if (t->bwd_engine != 0) {
            if (t->bwd_engine != 1 && t->bwd_engine != 2) return false;
            r.engine = t->bwd_engine;
        }
        if (t->fwd_prep != 0) {
            if (t->fwd_prep != 1 && t->fwd_prep != 2) return false;
            r.fwd_prep = t->fwd_prep;
        }
    }
    *out = r;
    return true;
}

int bwd_chunk_log2(const Tuning& t, int engine) {
    if (t.chunk_log2 > 0) return t.chunk_log2;
    // defaults.  Matrix-core engine: the deepest stack (fewest chunks, so the
    // fewest chunk roots and, for reductions of at most 4096 steps, no finish
    // pass); measured on the MI355X on the three Open-1B layers against depth
    // 6, interleaved and warm: dX 0.7-2.7% faster, dW within noise.  Its upper
    // stack levels spill at 3 workgroups per CU, which still beats 2
    // workgroups without spills by 2-4%.
    if (engine == 2) return 7;
    return 4;   // VALU engine, and the bound over both engines (more chunk roots)
}

// ---- the SwiGLU exp constants, derived from ln 2 ---------------------------------
ExpConsts exp_constants() {
    ExpConsts k;
    const long double ln2 = logl(2.0L);
    k.l2e = (float)(1.0L / ln2);
    const long double head = floorl(ln2 * 65536.0L) / 65536.0L;   // 16 significant bits
    k.ln2_hi = (float)head;
    k.ln2_lo = (float)(ln2 - head);
    long double fact = 1.0L;
    for (int i = 0; i < 8; ++i) {
        if (i > 1) fact *= (long double)i;
        k.c[i] = (float)(1.0L / fact);
    }
    return k;
}

static thread_local char g_err[512];

static brl_status fail(brl_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
static brl_status fail(brl_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

static brl_status check_hip(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(BRL_EDEVICE, "%s: %s", what, hipGetErrorString(e));
    return BRL_OK;
}

static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3) == 0; }
static bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255) == 0; }

// error reporting for the entry points defined in other translation units
brl_status report_error(brl_status s, const char* msg) { return fail(s, "%s", msg); }
brl_status report_hip(hipError_t e, const char* what) { return check_hip(e, what); }

// ---- workspace layout --------------------------------------------------------------
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <class T> T* take(size_t count) {
        off = (off + 255) & ~(size_t)255;
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += count * sizeof(T);
        return p;
    }
};

struct FwdLayout {
    int64_t Kp, Mp, Nvp;
    Scalars* scal;
    uint64_t* sync;
    float* partials;
    int8_t* qx;
    int8_t* qw;
    size_t bytes;
};

static FwdLayout fwd_layout(void* ws, int64_t M, int64_t K, int64_t N, int epilogue) {
    FwdLayout L;
    L.Kp = round_up(K, kKPad);
    L.Mp = round_up(M, kRowPad);
    const int64_t nv = epilogue == BRL_EPILOGUE_SWIGLU ? 2 * round_up(N / 2, kSwigluGroup) : N;
    L.Nvp = round_up(nv, kRowPad);
    Carver c(ws);
    L.scal = c.take<Scalars>(1);
    L.sync = c.take<uint64_t>((size_t)kPrepSyncWords);
    L.partials = c.take<float>((size_t)canon_partials(N * K));
    L.qx = c.take<int8_t>((size_t)(L.Mp * L.Kp));
    L.qw = c.take<int8_t>((size_t)(L.Nvp * L.Kp));
    L.bytes = c.off + 256;
    return L;
}

struct BwdLayout {
    int64_t Kp, Mp, Np;
    Scalars* scal;
    float* partials;
    void* bx;      // X operand: int8 q_x (VALU engine) or fp32 fl(q_x*s_x) (matrix-core engine), [Mp, Kp]
    void* bw;      // W operand likewise, [Np, Kp]
    float* G;
    float* roots;
    size_t bytes;
};

// D: the chunk depth that sizes the chunk roots (the bound over both engines
// when the engine is not known yet)
static BwdLayout bwd_layout(void* ws, int64_t M, int64_t K, int64_t N, int epilogue, int D) {
    BwdLayout L;
    L.Kp = round_up(K, kKPad);
    L.Mp = round_up(M, kRowPad);
    L.Np = round_up(N, kRowPad);
    Carver c(ws);
    L.scal = c.take<Scalars>(1);
    L.partials = c.take<float>((size_t)canon_partials(N * K));
    L.bx = c.take<float>((size_t)(L.Mp * L.Kp));
    L.bw = c.take<float>((size_t)(L.Np * L.Kp));
    L.G = epilogue == BRL_EPILOGUE_SWIGLU ? c.take<float>((size_t)(M * N)) : nullptr;
    int64_t r1 = ste_root_floats(M, N, K, D);   // dX: I = M, R = N
    int64_t r2 = ste_root_floats(N, M, K, D);   // dW: I = N, R = M
    L.roots = c.take<float>((size_t)(r1 > r2 ? r1 : r2));
    L.bytes = c.off + 256;
    return L;
}

static size_t norm_bytes(int64_t len) {
    Carver c(nullptr);
    c.take<Scalars>(1);
    c.take<float>((size_t)canon_partials(len));
    return c.off + 256;
}

static bool sizes_ok(int64_t M, int64_t K, int64_t N) {
    const int64_t lim = (int64_t)1 << 40;
    return M >= 0 && K >= 1 && N >= 1 && M < lim && K < lim && N < lim && M * K < lim &&
           N * K < lim && M * N < lim;
}

}  // namespace brl

using namespace brl;

extern "C" {

// State hash workspace: every level of digests (level 0 = the leaves) and
// the tensor lengths.
struct HashLayout {
    int64_t levels[24];      // digests per level
    uint8_t* level_ptr[24];
    int nlev;
    int64_t* lens;
    size_t bytes;
};

static HashLayout hash_layout(void* ws, int64_t leaves, int64_t count) {
    HashLayout L{};
    Carver c(ws);
    int64_t n = leaves;
    L.nlev = 0;
    while (true) {
        L.levels[L.nlev] = n;
        L.level_ptr[L.nlev] = c.take<uint8_t>((size_t)(n * 32));
        ++L.nlev;
        if (n <= 1) break;
        n = ceil_div(n, kHashFanIn);
    }
    L.lens = c.take<int64_t>((size_t)count);
    L.bytes = c.off + 256;
    return L;
}

size_t brl_workspace_bytes(int32_t op, int64_t M, int64_t K, int64_t N, const brl_tuning* tune) {
    Tuning t;
    if (!resolve_tuning(tune, &t)) return 0;
    switch (op) {
        case BRL_OP_HASH:
            if (M < 0 || K < 1 || K > ((int64_t)1 << 31)) return 0;
            return hash_layout(nullptr, M / kHashLeafBytes + K, K).bytes;
        case BRL_OP_FWD: return sizes_ok(M, K, N) ? fwd_layout(nullptr, M, K, N, BRL_EPILOGUE_SWIGLU).bytes : 0;
        case BRL_OP_BWD:
            return sizes_ok(M, K, N) ? bwd_layout(nullptr, M, K, N, BRL_EPILOGUE_SWIGLU, bwd_chunk_log2(t, 0)).bytes : 0;
        case BRL_OP_NORM: return M >= 0 ? norm_bytes(M) : 0;
        default: return 0;
    }
}

brl_status qat_linear_fwd(const float* X, const float* W, int64_t M, int64_t K, int64_t N, float s_x,
                          const float* addend, int32_t epilogue, float* Y, float* Ypre, float* s_w_out,
                          void* ws, size_t ws_bytes, const brl_tuning* tune, void* stream) {
    Tuning tn;
    if (!resolve_tuning(tune, &tn)) return fail(BRL_EINVAL, "qat_linear_fwd: tuning value out of range");
    if (!sizes_ok(M, K, N)) return fail(BRL_ESHAPE, "qat_linear_fwd: bad sizes M=%lld K=%lld N=%lld",
                                        (long long)M, (long long)K, (long long)N);
    if (K > 133144) return fail(BRL_ESHAPE, "qat_linear_fwd: K=%lld could overflow int32 accumulators", (long long)K);
    if (epilogue != BRL_EPILOGUE_NONE && epilogue != BRL_EPILOGUE_SWIGLU)
        return fail(BRL_EINVAL, "qat_linear_fwd: unknown epilogue %d", epilogue);
    if (epilogue == BRL_EPILOGUE_SWIGLU && (N & 1)) return fail(BRL_ESHAPE, "qat_linear_fwd: SwiGLU needs even N");
    if (!(s_x > 0.0f) || !isfinite(s_x)) return fail(BRL_EINVAL, "qat_linear_fwd: s_x must be finite and > 0");
    if (!W || (M > 0 && (!X || !Y))) return fail(BRL_EINVAL, "qat_linear_fwd: null tensor");
    if (!aligned4(X) || !aligned4(W) || !aligned4(Y) || !aligned4(addend) || !aligned4(Ypre) || !aligned4(s_w_out))
        return fail(BRL_EINVAL, "qat_linear_fwd: pointers must be 4-byte aligned");
    const FwdLayout need = fwd_layout(nullptr, M, K, N, BRL_EPILOGUE_SWIGLU);
    if (!aligned256(ws)) return fail(BRL_EINVAL, "qat_linear_fwd: workspace must be 256-byte aligned");
    if (!ws || ws_bytes < need.bytes)
        return fail(BRL_EWORKSPACE, "qat_linear_fwd: workspace %zu < %zu bytes", ws_bytes, need.bytes);
    FwdLayout L = fwd_layout(ws, M, K, N, epilogue);
    hipStream_t st = static_cast<hipStream_t>(stream);

    const int64_t swiglu_half = epilogue == BRL_EPILOGUE_SWIGLU ? N / 2 : 0;
    CanonFinishArgs fin{};
    fin.mode = kFinishScale;
    fin.count_f = (float)(double)(N * K);
    fin.s_x = s_x;
    fin.scal = L.scal;
    fin.s_w_out = s_w_out;
    brl_status s = BRL_OK;
    const bool one_launch = M > 0 && tn.fwd_prep == 1 && fwd_prep_fits(N * K);
    if (one_launch) {
        // weight step, W codes and X codes in one launch
        PrepArgs p{};
        p.X = X; p.W = W; p.M = M; p.K = K; p.N = N; p.s_x = s_x;
        p.qx = L.qx; p.qw = L.qw; p.Mp = L.Mp; p.Kp = L.Kp; p.Nvp = L.Nvp; p.swiglu_half = swiglu_half;
        p.sync = L.sync; p.fin = fin;
        s = check_hip(launch_fwd_prep(p, st), "forward preparation");
        if (s) return s;
    } else {
        s = check_hip(launch_canon(kMapAbs, W, N * K, L.partials, fin, tn.wg_blocks, st), "weight step");
        if (s || M == 0) return s;
        s = check_hip(launch_quantize(W, N, K, &L.scal->s_w, 0.0f, L.qw, L.Nvp, L.Kp, swiglu_half, st),
                      "quantize W");
        if (s) return s;
        s = check_hip(launch_quantize(X, M, K, nullptr, s_x, L.qx, L.Mp, L.Kp, 0, st), "quantize X");
        if (s) return s;
    }
    GemmArgs g{};
    g.qx = L.qx; g.qw = L.qw; g.M = M; g.N = N; g.Kp = L.Kp; g.Mp = L.Mp; g.Nvp = L.Nvp;
    g.scal = L.scal; g.addend = addend; g.Y = Y; g.Ypre = Ypre; g.epilogue = epilogue;
    g.ek = exp_constants();
    g.prep_err = one_launch ? L.sync + kPrepErrWord : nullptr;
    return check_hip(launch_gemm_i8(g, st), "int8 GEMM");
}

brl_status qat_linear_bwd(const float* dOut, const float* X, const float* W, const float* Ypre,
                          int64_t M, int64_t K, int64_t N, float s_x, int32_t epilogue, float* dX,
                          float* dW, int32_t dW_accumulate, void* ws, size_t ws_bytes, const brl_tuning* tune,
                          void* stream) {
    Tuning tn;
    if (!resolve_tuning(tune, &tn)) return fail(BRL_EINVAL, "qat_linear_bwd: tuning value out of range");
    if (!sizes_ok(M, K, N)) return fail(BRL_ESHAPE, "qat_linear_bwd: bad sizes M=%lld K=%lld N=%lld",
                                        (long long)M, (long long)K, (long long)N);
    if (epilogue != BRL_EPILOGUE_NONE && epilogue != BRL_EPILOGUE_SWIGLU)
        return fail(BRL_EINVAL, "qat_linear_bwd: unknown epilogue %d", epilogue);
    if (epilogue == BRL_EPILOGUE_SWIGLU && (N & 1)) return fail(BRL_ESHAPE, "qat_linear_bwd: SwiGLU needs even N");
    if (!(s_x > 0.0f) || !isfinite(s_x)) return fail(BRL_EINVAL, "qat_linear_bwd: s_x must be finite and > 0");
    if (!W || (M > 0 && (!X || !dOut)) || (epilogue == BRL_EPILOGUE_SWIGLU && M > 0 && !Ypre))
        return fail(BRL_EINVAL, "qat_linear_bwd: null tensor");
    if (dW_accumulate != 0 && dW_accumulate != 1) return fail(BRL_EINVAL, "qat_linear_bwd: dW_accumulate must be 0 or 1");
    if (!aligned4(dOut) || !aligned4(X) || !aligned4(W) || !aligned4(Ypre) || !aligned4(dX) || !aligned4(dW))
        return fail(BRL_EINVAL, "qat_linear_bwd: pointers must be 4-byte aligned");
    // the engine is fixed by the operands before anything is sized, and the
    // chunk depth read once: the layout and the launches use the same values
    const float* G = dOut;
    const bool g_vec_shape = N % 4 == 0;
    // (with SwiGLU, G is the workspace's copy, carved at a 256-byte offset)
    const void* g_src = epilogue == BRL_EPILOGUE_SWIGLU ? ws : static_cast<const void*>(dOut);
    const bool g_al16 = (reinterpret_cast<uintptr_t>(g_src) & 15) == 0;
    // The matrix-core engine loads 16-byte pieces of G rows directly into
    // LDS: it needs N % 4 == 0 and a 16-byte aligned G (the workspace copy
    // is aligned); otherwise the VALU engine runs (same bits).
    const bool g_vec = g_vec_shape && g_al16;
    const int engine = (tn.engine == 2 && g_vec) ? 2 : 1;
    const int D = bwd_chunk_log2(tn, engine);
    const int64_t Qx = ste_chunks(N, D), Qw = ste_chunks(M, D);
    if (Qx > 1024 || Qw > 1024)
        return fail(BRL_ESHAPE, "qat_linear_bwd: reduction too long for the chunk setting (%lld, %lld chunks)",
                    (long long)Qx, (long long)Qw);
    const BwdLayout need = bwd_layout(nullptr, M, K, N, BRL_EPILOGUE_SWIGLU, D);
    if (!aligned256(ws)) return fail(BRL_EINVAL, "qat_linear_bwd: workspace must be 256-byte aligned");
    if (!ws || ws_bytes < need.bytes)
        return fail(BRL_EWORKSPACE, "qat_linear_bwd: workspace %zu < %zu bytes", ws_bytes, need.bytes);
    BwdLayout L = bwd_layout(ws, M, K, N, epilogue, D);
    hipStream_t st = static_cast<hipStream_t>(stream);

    CanonFinishArgs fin{};
    fin.mode = kFinishScale;
    fin.count_f = (float)(double)(N * K);
    fin.s_x = s_x;
    fin.scal = L.scal;
    brl_status s = check_hip(launch_canon(kMapAbs, W, N * K, L.partials, fin, tn.wg_blocks, st), "weight step");
    if (s) return s;
    if (epilogue == BRL_EPILOGUE_SWIGLU && M > 0) G = L.G;
    if (engine == 2) {
        s = check_hip(launch_dequant(W, N, K, &L.scal->s_w, 0.0f, static_cast<float*>(L.bw), L.Np, L.Kp, st),
                      "dequantise W");
        if (s) return s;
        s = check_hip(launch_dequant(X, M, K, nullptr, s_x, static_cast<float*>(L.bx), L.Mp, L.Kp, st),
                      "dequantise X");
    } else {
        s = check_hip(launch_quantize(W, N, K, &L.scal->s_w, 0.0f, static_cast<int8_t*>(L.bw), L.Np, L.Kp, 0, st),
                      "quantize W");
        if (s) return s;
        s = check_hip(launch_quantize(X, M, K, nullptr, s_x, static_cast<int8_t*>(L.bx), L.Mp, L.Kp, 0, st),
                      "quantize X");
    }
    if (s) return s;
    if (epilogue == BRL_EPILOGUE_SWIGLU && M > 0) {
        s = check_hip(launch_swiglu_bwd(dOut, Ypre, M, N, L.G, exp_constants(), st), "SwiGLU backward");
        if (s) return s;
    }
    if (dX && M > 0) {
        SteArgs a{};
        a.A = G; a.lda = N; a.a_rmaj = true; a.a_vec = g_vec; a.I = M; a.R = N; a.Jn = K;
        a.Bq = static_cast<const int8_t*>(L.bw); a.Bf = static_cast<const float*>(L.bw);
        a.ldb = L.Kp; a.b_scale_dev = &L.scal->s_w;
        a.mask_src = X; a.mask_scale_dev = nullptr; a.mask_scale_host = s_x;
        a.out = dX; a.accumulate = 0; a.roots = L.roots;
        s = check_hip(launch_ste(a, engine, D, st), "dX");
        if (s) return s;
    }
    if (dW) {
        SteArgs a{};
        a.A = G; a.lda = N; a.a_rmaj = false; a.a_vec = g_vec; a.I = N; a.R = M; a.Jn = K;
        a.Bq = static_cast<const int8_t*>(L.bx); a.Bf = static_cast<const float*>(L.bx);
        a.ldb = L.Kp; a.b_scale_dev = nullptr; a.b_scale_host = s_x;
        a.mask_src = W; a.mask_scale_dev = &L.scal->s_w;
        a.out = dW; a.accumulate = dW_accumulate; a.roots = L.roots;
        s = check_hip(launch_ste(a, engine, D, st), "dW");
        if (s) return s;
    }
    return BRL_OK;
}

brl_status brl_reduce_init(brl_reduce_state* st, int32_t replicas, int32_t shards, int64_t len,
                           float* const* acc) {
    if (!st || !acc) return fail(BRL_EINVAL, "brl_reduce_init: null argument");
    if (replicas < 1 || replicas > BRL_MAX_REPLICAS || shards < 1 || len < 0 ||
        (int64_t)replicas * shards > (int64_t)1 << 30)
        return fail(BRL_ESHAPE, "brl_reduce_init: bad mesh %d x %d or length", replicas, shards);
    memset(st, 0, sizeof(*st));
    st->replicas = replicas;
    st->shards = shards;
    st->len = len;
    st->next = 0;
    for (int r = 0; r < replicas; ++r) {
        if (!acc[r] && len > 0) return fail(BRL_EINVAL, "brl_reduce_init: null buffer for replica %d", r);
        if (!aligned4(acc[r])) return fail(BRL_EINVAL, "brl_reduce_init: misaligned buffer");
        st->acc[r] = acc[r];
    }
    return BRL_OK;
}

brl_status ordered_reduce(brl_reduce_state* sp, const float* partial, float* out, void* stream) {
    if (!sp) return fail(BRL_EINVAL, "ordered_reduce: null state");
    const int R = sp->replicas, S = sp->shards;
    if (R < 1 || R > BRL_MAX_REPLICAS || S < 1 || sp->len < 0)
        return fail(BRL_EINVAL, "ordered_reduce: state not initialised");
    const int64_t total = (int64_t)R * S;
    if (sp->next < 0 || sp->next >= total)
        return fail(BRL_EORDER, "ordered_reduce: all %lld virtual ranks already reduced", (long long)total);
    const int64_t v = sp->next;
    const int r = (int)(v / S), s = (int)(v % S);
    const bool last = v == total - 1;
    const int64_t n = sp->len;
    if (n > 0 && !partial) return fail(BRL_EINVAL, "ordered_reduce: null partial");
    if (last && n > 0 && !out) return fail(BRL_EINVAL, "ordered_reduce: last rank needs out");
    if (!aligned4(partial) || !aligned4(out)) return fail(BRL_EINVAL, "ordered_reduce: misaligned pointer");
    Tuning tn;
    if (!resolve_tuning(&sp->tune, &tn)) return fail(BRL_EINVAL, "ordered_reduce: tuning value out of range");
    hipStream_t st = static_cast<hipStream_t>(stream);
    brl_status rc = BRL_OK;
    const bool resident = (sp->flags & BRL_REDUCE_REPLICA_RESIDENT) && S > 1 && S <= BRL_MAX_SHARDS;
    const bool defer = !resident && (sp->flags & (BRL_REDUCE_PARTIALS_PERSIST | BRL_REDUCE_REPLICA_RESIDENT)) && S > 1;
    if (s == 0) sp->pending = nullptr;
    if (resident) {
        // the replica's partials stay resident: its last shard's call forms
        // the whole running sum in one pass (for the last replica, inside
        // the TreeFold)
        sp->shard_part[s] = partial;
        if (n > 0 && s == S - 1) {
            FoldPtrs parts{};
            for (int i = 0; i < S; ++i) parts.a[i] = sp->shard_part[i];
            if (!last) {
                rc = check_hip(launch_runsum(sp->acc[r], parts, S, n, st), "running sum (resident shards)");
            } else {
                FoldPtrs p{};
                for (int i = 0; i < R; ++i) p.a[i] = sp->acc[i];
                rc = check_hip(launch_fold(p, R, nullptr, parts, S, out, n, st), "TreeFold");
            }
        }
    } else if (n > 0) {
        if (s == 0 && defer) {
            // A_r = G_{r,0} is formed together with the next shard's add
            sp->pending = partial;
        } else if (!last) {
            const bool joint = s == 1 && sp->pending;
            rc = check_hip(launch_accumulate(sp->acc[r], joint ? sp->pending : sp->acc[r], partial, n, s == 0, tn.vec, st),
                           s == 0 ? "running sum (first shard)" : "running sum");
        } else {
            FoldPtrs p{};
            for (int i = 0; i < R; ++i) p.a[i] = sp->acc[i];
            const float* g_last = partial;
            if (s == 0) {
                p.a[R - 1] = partial;
                g_last = nullptr;
            } else if (s == 1 && sp->pending) {
                rc = check_hip(launch_accumulate(sp->acc[r], sp->pending, partial, n, 0, tn.vec, st), "running sum");
                g_last = nullptr;
            }
            if (rc == BRL_OK) rc = check_hip(launch_fold(p, R, g_last, FoldPtrs{}, 0, out, n, st), "TreeFold");
        }
    }
    if (s >= 1) sp->pending = nullptr;
    if (rc == BRL_OK) sp->next = (int32_t)(v + 1);
    return rc;
}

// The squared-norm CanonSum and the clip, on a workspace already checked to
// hold norm_bytes(len) bytes at a 256-byte aligned address.
static brl_status norm_clip_launch(float* g, int64_t len, float max_norm, float eps, float* norm_out, void* ws,
                                   const Tuning& tn, hipStream_t st) {
    Carver c(ws);
    Scalars* scal = c.take<Scalars>(1);
    float* partials = c.take<float>((size_t)canon_partials(len));
    CanonFinishArgs fin{};
    fin.mode = kFinishNorm;
    fin.max_norm = max_norm;
    fin.eps = eps;
    fin.scal = scal;
    fin.nu_out = norm_out;
    brl_status s = check_hip(launch_canon(kMapSquare, g, len, partials, fin, tn.wg_blocks, st), "squared norm");
    if (s) return s;
    return check_hip(launch_clip(g, len, scal, tn.vec, st), "clip");
}

static brl_status norm_clip_check(const char* who, const float* g, int64_t len, float max_norm, float eps,
                                  const float* norm_out) {
    if (len < 0 || len > ((int64_t)1 << 40)) return fail(BRL_ESHAPE, "%s: bad length", who);
    if (len > 0 && !g) return fail(BRL_EINVAL, "%s: null gradient", who);
    if (!(max_norm > 0.0f) || !isfinite(max_norm) || !(eps >= 0.0f) || !isfinite(eps))
        return fail(BRL_EINVAL, "%s: max_norm must be finite > 0 and eps finite >= 0", who);
    if (!aligned4(g) || !aligned4(norm_out)) return fail(BRL_EINVAL, "%s: misaligned pointer", who);
    return BRL_OK;
}

brl_status grad_l2norm_clip(float* g, int64_t len, float max_norm, float eps, float* norm_out, void* ws,
                            size_t ws_bytes, const brl_tuning* tune, void* stream) {
    Tuning tn;
    if (!resolve_tuning(tune, &tn)) return fail(BRL_EINVAL, "grad_l2norm_clip: tuning value out of range");
    if (brl_status s = norm_clip_check("grad_l2norm_clip", g, len, max_norm, eps, norm_out)) return s;
    const size_t need = norm_bytes(len);
    if (!aligned256(ws)) return fail(BRL_EINVAL, "grad_l2norm_clip: workspace must be 256-byte aligned");
    if (!ws || ws_bytes < need)
        return fail(BRL_EWORKSPACE, "grad_l2norm_clip: workspace %zu < %zu bytes", ws_bytes, need);
    return norm_clip_launch(g, len, max_norm, eps, norm_out, ws, tn, static_cast<hipStream_t>(stream));
}

// ---- the norm and clip without a caller workspace ---------------------------------
// For callers that cannot allocate (graph capture, tight serving loops): the
// squared-norm CanonSum's roots and the call's scalars live in `scratch`, a
// file-scope device array of kNormScratchBytes that every device the library
// runs on holds for the life of the process.  Its device address is taken once
// per device with hipGetSymbolAddress (the array's name in host code is only a
// host-side stand-in) and kept in g_scratch_dev.  Calls on one device share the
// array: calls that overlap in time on one device race.  Nothing in it needs
// clearing: every root and scalar is written before it is read in the call.
constexpr size_t kNormScratchBytes = (size_t)2 << 20;
constexpr int kScratchDevices = 64;
static __device__ __align__(256) char scratch[kNormScratchBytes];
static std::atomic<void*> g_scratch_dev[kScratchDevices];

static brl_status scratch_for_current_device(void** out) {
    int dev = -1;
    if (const hipError_t e = hipGetDevice(&dev); e != hipSuccess)
        return check_hip(e, "grad_l2norm_clip_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kScratchDevices)
        return fail(BRL_EDEVICE, "grad_l2norm_clip_noalloc: device %d beyond the %d the library tracks", dev,
                    kScratchDevices);
    void* p = g_scratch_dev[dev].load(std::memory_order_acquire);
    if (!p) {
        if (const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess)
            return check_hip(e, "grad_l2norm_clip_noalloc: hipGetSymbolAddress");
        if (!p || !aligned256(p)) return fail(BRL_EDEVICE, "grad_l2norm_clip_noalloc: bad scratch address");
        g_scratch_dev[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return BRL_OK;
}

brl_status grad_l2norm_clip_noalloc(float* g, int64_t len, float max_norm, float eps, float* norm_out,
                                    const brl_tuning* tune, void* stream) {
    Tuning tn;
    if (!resolve_tuning(tune, &tn)) return fail(BRL_EINVAL, "grad_l2norm_clip_noalloc: tuning value out of range");
    if (brl_status s = norm_clip_check("grad_l2norm_clip_noalloc", g, len, max_norm, eps, norm_out)) return s;
    const size_t need = norm_bytes(len);
    if (need > kNormScratchBytes)
        return fail(BRL_ESHAPE,
                    "grad_l2norm_clip_noalloc: len %lld needs %zu bytes of scratch, more than its %zu (at most "
                    "%lld elements)",
                    (long long)len, need, kNormScratchBytes, (long long)BRL_NOALLOC_NORM_MAX_LEN);
    void* ws = nullptr;
    if (brl_status s = scratch_for_current_device(&ws)) return s;
    return norm_clip_launch(g, len, max_norm, eps, norm_out, ws, tn, static_cast<hipStream_t>(stream));
}

brl_status brl_probe_f32(int32_t op, const float* a, const float* b, float* out, int64_t n, void* stream) {
    if (op < 0 || op > 9) return fail(BRL_EINVAL, "brl_probe_f32: unknown op %d", op);
    if (n < 0) return fail(BRL_ESHAPE, "brl_probe_f32: n < 0");
    if (n > 0 && (!a || !out || ((op <= 3 || op >= 8) && !b))) return fail(BRL_EINVAL, "brl_probe_f32: null pointer");
    if (op == 8)
        return check_hip(launch_probe_mfma(a, b, out, n, static_cast<hipStream_t>(stream)), "probe");
    if (op == 9)
        return check_hip(launch_probe_mfma_fma(a, b, out, n, static_cast<hipStream_t>(stream)), "probe");
    return check_hip(launch_probe(op, a, b, out, n, exp_constants(), static_cast<hipStream_t>(stream)), "probe");
}

brl_status brl_probe_rate(int32_t what, int64_t iters, float* out, int64_t out_len, void* stream) {
    if (what < 0 || what > 8) return fail(BRL_EINVAL, "brl_probe_rate: unknown unit %d", what);
    if (iters < 1 || iters > ((int64_t)1 << 30)) return fail(BRL_ESHAPE, "brl_probe_rate: iters out of range");
    if (!out || !aligned4(out)) return fail(BRL_EINVAL, "brl_probe_rate: bad output pointer");
    if (out_len < probe_rate_threads())
        return fail(BRL_ESHAPE, "brl_probe_rate: out needs %lld floats", (long long)probe_rate_threads());
    // c: a step that keeps every chain finite for any iteration count
    const float c = (what == 1 || what == 3) ? 1.0f : 0.5f;
    return check_hip(launch_probe_rate(what, iters, c, out, static_cast<hipStream_t>(stream)), "rate probe");
}

int64_t brl_probe_rate_threads(void) { return probe_rate_threads(); }

brl_status brl_state_hash(const void* const* tensors, const int64_t* nbytes, int32_t count, uint8_t* digest,
                          void* ws, size_t ws_bytes, void* stream) {
    if (count < 1 || !tensors || !nbytes) return fail(BRL_EINVAL, "brl_state_hash: need count >= 1 tensors");
    if (!digest) return fail(BRL_EINVAL, "brl_state_hash: null digest");
    int64_t total = 0, leaves = 0;
    bool vec = true;
    for (int32_t i = 0; i < count; ++i) {
        if (nbytes[i] < 0) return fail(BRL_ESHAPE, "brl_state_hash: nbytes[%d] < 0", (int)i);
        if (nbytes[i] > 0 && !tensors[i]) return fail(BRL_EINVAL, "brl_state_hash: tensor %d is null", (int)i);
        if (!aligned4(tensors[i])) return fail(BRL_EINVAL, "brl_state_hash: tensor %d not 4-byte aligned", (int)i);
        if ((reinterpret_cast<uintptr_t>(tensors[i]) & 15) != 0) vec = false;
        total += nbytes[i];
        leaves += nbytes[i] == 0 ? 1 : ceil_div(nbytes[i], kHashLeafBytes);
    }
    const HashLayout need = hash_layout(nullptr, leaves, count);
    if (!aligned256(ws)) return fail(BRL_EINVAL, "brl_state_hash: workspace must be 256-byte aligned");
    if (!ws || ws_bytes < need.bytes)
        return fail(BRL_EWORKSPACE, "brl_state_hash: workspace %zu < %zu bytes", ws_bytes, need.bytes);
    HashLayout L = hash_layout(ws, leaves, count);
    hipStream_t st = static_cast<hipStream_t>(stream);
    // leaves, 64 tensors per launch
    int64_t leaf_base = 0;
    for (int32_t t0 = 0; t0 < count; t0 += kHashBatch) {
        HashBatch hb{};
        hb.n = (count - t0) < kHashBatch ? (count - t0) : kHashBatch;
        hb.first_tensor = t0;
        hb.leaf_base = leaf_base;
        int64_t acc = 0;
        for (int i = 0; i < hb.n; ++i) {
            hb.ptr[i] = tensors[t0 + i];
            hb.len[i] = nbytes[t0 + i];
            hb.first_leaf[i] = acc;
            acc += nbytes[t0 + i] == 0 ? 1 : ceil_div(nbytes[t0 + i], kHashLeafBytes);
        }
        hb.leaves = acc;
        brl_status s = check_hip(launch_hash_leaves(hb, vec, L.level_ptr[0], L.lens, st), "hash leaves");
        if (s) return s;
        leaf_base += acc;
    }
    for (int l = 1; l < L.nlev; ++l) {
        brl_status s = check_hip(launch_hash_nodes(L.level_ptr[l - 1], L.levels[l - 1], L.level_ptr[l], st),
                                 "hash nodes");
        if (s) return s;
    }
    (void)total;
    return check_hip(launch_hash_root(L.level_ptr[L.nlev - 1], L.lens, count, digest, st), "hash root");
}

brl_status brl_adamw_scalars_for_step(int64_t step, double tokens, const brl_adamw_config* cfg,
                                      brl_adamw_scalars* out) {
    static const brl_adamw_config recipe = {0.9, 0.95, 1e-8, 0.1, 4.5e-4, 4.5e-5, 2.1e9, 400e9};
    const brl_adamw_config& c = cfg ? *cfg : recipe;
    if (!out) return fail(BRL_EINVAL, "brl_adamw_scalars_for_step: null output");
    if (step < 1) return fail(BRL_EINVAL, "brl_adamw_scalars_for_step: step must be >= 1");
    if (!(tokens >= 0.0) || !isfinite(tokens)) return fail(BRL_EINVAL, "brl_adamw_scalars_for_step: bad token count");
    if (!(c.beta1 >= 0.0 && c.beta1 < 1.0) || !(c.beta2 >= 0.0 && c.beta2 < 1.0) || !(c.eps > 0.0) ||
        !(c.wd >= 0.0) || !(c.peak_lr >= 0.0) || !(c.min_lr >= 0.0) || !(c.warmup_tokens > 0.0) ||
        !(c.total_tokens > c.warmup_tokens))
        return fail(BRL_EINVAL, "brl_adamw_scalars_for_step: bad configuration");
    adamw_scalars(step, tokens, c, out);
    return BRL_OK;
}

brl_status adamw_step(float* p, const float* g, float* m, float* v, int64_t n, const brl_adamw_scalars* sc,
                      int32_t decay, void* stream) {
    if (n < 0) return fail(BRL_ESHAPE, "adamw_step: n < 0");
    if (!sc) return fail(BRL_EINVAL, "adamw_step: null scalars");
    if (n > 0 && (!p || !g || !m || !v)) return fail(BRL_EINVAL, "adamw_step: null tensor");
    if (!aligned4(p) || !aligned4(g) || !aligned4(m) || !aligned4(v))
        return fail(BRL_EINVAL, "adamw_step: pointers must be 4-byte aligned");
    return check_hip(launch_adamw(p, g, m, v, n, *sc, decay != 0, static_cast<hipStream_t>(stream)), "AdamW");
}

static brl_status attn_check(const char* who, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                             int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo, float s_v) {
    if (B < 0 || S < 0) return fail(BRL_ESHAPE, "%s: B, S must be >= 0", who);
    if (D != 128) return fail(BRL_ESHAPE, "%s: head dimension must be 128", who);
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return fail(BRL_ESHAPE, "%s: Hq must be a positive multiple of Hkv", who);
    if (S > 133143) return fail(BRL_ESHAPE, "%s: S too large for int32 P.V accumulators", who);
    if (ldq < Hq * D || ldo < Hq * D || ldk < Hkv * D || ldv < Hkv * D)
        return fail(BRL_ESHAPE, "%s: row stride smaller than heads * D", who);
    if ((ldq | ldk | ldv | ldo) & 3) return fail(BRL_EINVAL, "%s: row strides must be multiples of 4", who);
    if (!(s_v == s_v)) return fail(BRL_EINVAL, "%s: s_v is NaN", who);
    return BRL_OK;
}

static bool al16p(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

size_t attn_fwd_workspace_bytes(int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t window) {
    if (B < 0 || S < 0 || S > 133143 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return 0;
    if (B * Hq * ((S + 63) / 64) > 0xffffffffLL) return 0;
    return attn_fwd_ws_bytes(B, S, Hq, Hkv, window);
}

size_t attn_logits_bytes(int64_t B, int64_t S, int64_t Hq, int64_t window) {
    if (B < 0 || S < 0 || S > 133143 || Hq <= 0) return 0;
    if (B * Hq * ((S + 63) / 64) > 0xffffffffLL) return 0;
    return attn_keep_bytes(B, S, Hq, window);
}

// kept logits: device, 256-byte aligned, at least attn_logits_bytes
static brl_status check_logits(const char* who, const void* logits, size_t bytes, int64_t B, int64_t S, int64_t Hq,
                               int64_t window) {
    const size_t need = attn_keep_bytes(B, S, Hq, window);
    if (!logits) return fail(BRL_EINVAL, "%s: null logits", who);
    if (!aligned256(logits)) return fail(BRL_EINVAL, "%s: logits must be 256-byte aligned", who);
    if (bytes < need) return fail(BRL_ESHAPE, "%s: logits %zu < %zu bytes", who, bytes, need);
    return BRL_OK;
}

static brl_status attn_fwd_impl(const char* who, const float* Q, const float* K, const float* V, int64_t B,
                                int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t ldq, int64_t ldk, int64_t ldv,
                                int64_t window, float s_v, float* O, int64_t ldo, float* stats, float* keep,
                                size_t keep_bytes, void* ws, size_t ws_bytes, void* stream) {
    brl_status rc = attn_check(who, B, S, Hq, Hkv, D, ldq, ldk, ldv, ldo, s_v);
    if (rc != BRL_OK) return rc;
    if (B * S == 0) return BRL_OK;
    if (!Q || !K || !V || !O) return fail(BRL_EINVAL, "%s: null tensor", who);
    if (!al16p(Q) || !al16p(K) || !al16p(V) || !al16p(O))
        return fail(BRL_EINVAL, "%s: pointers must be 16-byte aligned", who);
    if (stats && !aligned4(stats)) return fail(BRL_EINVAL, "%s: stats must be 4-byte aligned", who);
    if (B * Hq * ((S + 63) / 64) > 0xffffffffLL) return fail(BRL_ESHAPE, "%s: too many query blocks", who);
    if (keep && (rc = check_logits(who, keep, keep_bytes, B, S, Hq, window)) != BRL_OK) return rc;
    const size_t need = attn_fwd_ws_bytes(B, S, Hq, Hkv, window);
    if (!aligned256(ws)) return fail(BRL_EINVAL, "%s: workspace must be 256-byte aligned", who);
    if (!ws || ws_bytes < need) return fail(BRL_EWORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes, need);
    return check_hip(launch_attn_fwd(Q, K, V, B, S, Hq, Hkv, ldq, ldk, ldv, window, s_v, O, ldo, stats,
                                     static_cast<float*>(ws), keep, exp_constants(),
                                     static_cast<hipStream_t>(stream)),
                     "attention");
}

brl_status attn_fwd(const float* Q, const float* K, const float* V, int64_t B, int64_t S, int64_t Hq,
                    int64_t Hkv, int64_t D, int64_t ldq, int64_t ldk, int64_t ldv, int64_t window, float s_v,
                    float* O, int64_t ldo, float* stats, void* ws, size_t ws_bytes, void* stream) {
    return attn_fwd_impl("attn_fwd", Q, K, V, B, S, Hq, Hkv, D, ldq, ldk, ldv, window, s_v, O, ldo, stats, nullptr,
                         0, ws, ws_bytes, stream);
}

brl_status attn_fwd_keep_logits(const float* Q, const float* K, const float* V, int64_t B, int64_t S, int64_t Hq,
                                int64_t Hkv, int64_t D, int64_t ldq, int64_t ldk, int64_t ldv, int64_t window,
                                float s_v, float* O, int64_t ldo, float* stats, float* logits, size_t logits_bytes,
                                void* ws, size_t ws_bytes, void* stream) {
    if (!logits && B * S != 0) return fail(BRL_EINVAL, "attn_fwd_keep_logits: null logits");
    return attn_fwd_impl("attn_fwd_keep_logits", Q, K, V, B, S, Hq, Hkv, D, ldq, ldk, ldv, window, s_v, O, ldo,
                         stats, logits, logits_bytes, ws, ws_bytes, stream);
}

static brl_status attn_bwd_dq_impl(const char* who, const float* Q, const float* K, const float* V, const float* O,
                                   const float* dO, const float* stats, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                   int64_t D, int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo, int64_t window,
                                   float s_v, float* dQ, const float* keep, size_t keep_bytes, void* stream) {
    brl_status rc = attn_check(who, B, S, Hq, Hkv, D, ldq, ldk, ldv, ldo, s_v);
    if (rc != BRL_OK) return rc;
    if (B * S == 0) return BRL_OK;
    if (!Q || !K || !V || !O || !dO || !stats || !dQ) return fail(BRL_EINVAL, "%s: null tensor", who);
    if (!al16p(Q) || !al16p(K) || !al16p(V) || !al16p(O) || !al16p(dO) || !al16p(dQ))
        return fail(BRL_EINVAL, "%s: pointers must be 16-byte aligned", who);
    if (!aligned4(stats)) return fail(BRL_EINVAL, "%s: stats must be 4-byte aligned", who);
    if (keep && (rc = check_logits(who, keep, keep_bytes, B, S, Hq, window)) != BRL_OK) return rc;
    return check_hip(launch_attn_bwd_dq(Q, K, V, O, dO, stats, B, S, Hq, Hkv, ldq, ldk, ldv, ldo, window, s_v, dQ,
                                        keep, exp_constants(), static_cast<hipStream_t>(stream)),
                     "attention dQ");
}

brl_status attn_bwd_dq(const float* Q, const float* K, const float* V, const float* O, const float* dO,
                       const float* stats, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t ldq,
                       int64_t ldk, int64_t ldv, int64_t ldo, int64_t window, float s_v, float* dQ,
                       void* stream) {
    return attn_bwd_dq_impl("attn_bwd_dq", Q, K, V, O, dO, stats, B, S, Hq, Hkv, D, ldq, ldk, ldv, ldo, window, s_v,
                            dQ, nullptr, 0, stream);
}

brl_status attn_bwd_dq_logits(const float* Q, const float* K, const float* V, const float* O, const float* dO,
                              const float* stats, const float* logits, size_t logits_bytes, int64_t B, int64_t S,
                              int64_t Hq, int64_t Hkv, int64_t D, int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo,
                              int64_t window, float s_v, float* dQ, void* stream) {
    if (!logits && B * S != 0) return fail(BRL_EINVAL, "attn_bwd_dq_logits: null logits");
    return attn_bwd_dq_impl("attn_bwd_dq_logits", Q, K, V, O, dO, stats, B, S, Hq, Hkv, D, ldq, ldk, ldv, ldo,
                            window, s_v, dQ, logits, logits_bytes, stream);
}

static brl_status attn_bwd_dkdv_impl(const char* who, const float* Q, const float* K, const float* V, const float* O,
                                     const float* dO, const float* stats, int64_t B, int64_t S, int64_t Hq,
                                     int64_t Hkv, int64_t D, int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo,
                                     int64_t window, float s_v, float* dK, float* dV, int64_t ldg, const float* keep,
                                     size_t keep_bytes, void* stream) {
    brl_status rc = attn_check(who, B, S, Hq, Hkv, D, ldq, ldk, ldv, ldo, s_v);
    if (rc != BRL_OK) return rc;
    if (ldg < Hkv * D) return fail(BRL_ESHAPE, "%s: row stride smaller than heads * D", who);
    if (ldg & 3) return fail(BRL_EINVAL, "%s: row strides must be multiples of 4", who);
    if (B * S == 0) return BRL_OK;
    if (!Q || !K || !V || !O || !dO || !stats || !dK || !dV) return fail(BRL_EINVAL, "%s: null tensor", who);
    if (!al16p(Q) || !al16p(K) || !al16p(V) || !al16p(O) || !al16p(dO) || !al16p(dK) || !al16p(dV))
        return fail(BRL_EINVAL, "%s: pointers must be 16-byte aligned", who);
    if (!aligned4(stats)) return fail(BRL_EINVAL, "%s: stats must be 4-byte aligned", who);
    if (keep && (rc = check_logits(who, keep, keep_bytes, B, S, Hq, window)) != BRL_OK) return rc;
    return check_hip(launch_attn_bwd_dkdv(Q, K, V, O, dO, stats, B, S, Hq, Hkv, ldq, ldk, ldv, ldo, window, s_v,
                                          dK, dV, ldg, keep, exp_constants(), static_cast<hipStream_t>(stream)),
                     "attention dK/dV");
}

brl_status attn_bwd_dkdv(const float* Q, const float* K, const float* V, const float* O, const float* dO,
                         const float* stats, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                         int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo, int64_t window, float s_v, float* dK,
                         float* dV, int64_t ldg, void* stream) {
    return attn_bwd_dkdv_impl("attn_bwd_dkdv", Q, K, V, O, dO, stats, B, S, Hq, Hkv, D, ldq, ldk, ldv, ldo, window,
                              s_v, dK, dV, ldg, nullptr, 0, stream);
}

brl_status attn_bwd_dkdv_logits(const float* Q, const float* K, const float* V, const float* O, const float* dO,
                                const float* stats, const float* logits, size_t logits_bytes, int64_t B, int64_t S,
                                int64_t Hq, int64_t Hkv, int64_t D, int64_t ldq, int64_t ldk, int64_t ldv,
                                int64_t ldo, int64_t window, float s_v, float* dK, float* dV, int64_t ldg,
                                void* stream) {
    if (!logits && B * S != 0) return fail(BRL_EINVAL, "attn_bwd_dkdv_logits: null logits");
    return attn_bwd_dkdv_impl("attn_bwd_dkdv_logits", Q, K, V, O, dO, stats, B, S, Hq, Hkv, D, ldq, ldk, ldv, ldo,
                              window, s_v, dK, dV, ldg, logits, logits_bytes, stream);
}

const char* brl_status_string(brl_status s) {
    switch (s) {
        case BRL_OK: return "ok";
        case BRL_EINVAL: return "invalid argument";
        case BRL_ESHAPE: return "bad shape";
        case BRL_EORDER: return "out of mesh order";
        case BRL_EDEVICE: return "device error";
        case BRL_EWORKSPACE: return "workspace too small";
        default: return "unknown status";
    }
}

const char* brl_last_error(void) { return g_err; }

}  // extern "C"
