/*
 * brlsq.h -- C ABI of the bit-exact int8 LSQ linear layer and ordered
 * gradient reduction for AMD Instinct MI355X (gfx950).
 *
 * What is computed follows "OPEN-1B: A Fully Auditable Training Run"
 * (Donaghy et al., Gensyn), as summarised on onedev.kr:
 *   - section "How": every reduction in one fixed order, multiply and add
 *     never fused, subnormals flushed to zero on every backend;
 *   - section "Use": LSQ int8 QAT on every attention/FFN linear (8-bit
 *     weights and activations), weight step 2*mean(|w|)/sqrt(q_max) recomputed
 *     from the weights every step, SwiGLU gate and up as one GEMM;
 *   - section "Limits", recipe paragraph: global L2 gradient-norm clip at 1.0;
 *   - section "Limits", audit paragraph: single-device replay of the gradient
 *     reduction -- running-sum reduce-scatter over virtual ranks in mesh order
 *     (replica-major, shard-minor), then TreeFold over replicas in the
 *     pairing order of a recursive-doubling all-reduce.
 *
 * Numerics contract (every output, bit for bit, on every call):
 *   binary32 add/sub/mul/div/sqrt are each rounded to nearest even and then
 *   flushed to a zero of the same sign when the rounded result is below
 *   2^-126; subnormal operands read as zeros of the same sign; no operation is
 *   fused.  CanonSum(p_0..p_{n-1}) = sequential left-to-right sums of 32-wide
 *   blocks (each starting from its first term), then a pairwise tree over the
 *   block sums, level by level, (0,1),(2,3),..., an odd last node carried up
 *   unchanged; CanonSum of nothing is +0.  Results do not depend on tile
 *   sizes, launch shapes or the number of compute units.
 *
 * Memory and ownership.  All tensor pointers are device pointers, row-major,
 * dense (row pitch = the row length).  The caller owns every buffer,
 * including the workspace, whose size comes from brl_workspace_bytes().  The
 * library allocates no device memory and holds no state between calls
 * (besides the calling thread's last error message).  Every call is asynchronous on the given
 * HIP stream (a hipStream_t passed as void*; NULL = the null stream) and never
 * synchronises the host.  Pointers must be 4-byte aligned.
 *
 * Errors.  Arguments are checked before anything is launched; a bad argument
 * returns a negative status and launches nothing.  A failed launch returns
 * BRL_EDEVICE.  brl_last_error() gives a message for the calling thread.
 * Inputs must be finite; NaN and Inf propagate by IEEE rules and are not
 * checked.
 */
#ifndef BRLSQ_H
#define BRLSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define BRL_API __attribute__((visibility("default")))
#else
#define BRL_API
#endif

typedef int32_t brl_status;

#define BRL_OK          0
#define BRL_EINVAL     (-1)   /* null pointer, bad scalar, bad enum */
#define BRL_ESHAPE     (-2)   /* non-positive or inconsistent sizes, overflow risk */
#define BRL_EORDER     (-3)   /* ordered_reduce called out of mesh order */
#define BRL_EDEVICE    (-4)   /* HIP launch or runtime error */
#define BRL_EWORKSPACE (-5)   /* workspace missing or too small */

/* Epilogues of the forward (and the matching backward prologue). */
#define BRL_EPILOGUE_NONE   0
/* Stacked SwiGLU: W rows [0, N/2) are the gate, rows [N/2, N) the up
 * projection (the pages' "gate and up as one GEMM").  The activation is
 * A[m,j] = (g * sigma(g)) * u with g = Y[m,j], u = Y[m,j+N/2],
 * sigma(g) = 1 / (1 + E(-g)) and E the library's own binary32 exp (Cody-Waite
 * reduction with ln2 split at 16 bits, degree-7 Taylor polynomial in Horner
 * form, scaling by 2^k in two exact steps; every step one binary32 op). */
#define BRL_EPILOGUE_SWIGLU 1

/* Workspace query operations. */
#define BRL_OP_FWD  0
#define BRL_OP_BWD  1
#define BRL_OP_NORM 2
#define BRL_OP_HASH 3

/* Launch-shape choices of one call.  They change only how work is split
 * across workgroups or which units form the backward's products, never the
 * results.  A zero field selects its default; a NULL pointer selects every
 * default.  The library keeps no tuning state of its own: each call reads the
 * struct once, at its start, and a bad value fails the call with BRL_EINVAL. */
typedef struct brl_tuning {
    int32_t bwd_chunk_log2;    /* 32-blocks per backward reduction chunk: 2^v, v in 1..7
                                  (0: 7 on the matrix-core engine, 4 on the VALU engine) */
    int32_t reduce_wg_blocks;  /* 32-blocks per workgroup in CanonSum passes: 64, 128 or 256 (0: 256) */
    int32_t stream_vec;        /* 16-byte vectors per thread in the streaming kernels: 1, 2 or 4 (0: 1) */
    int32_t bwd_engine;        /* backward products on 1 the VALU, 2 the matrix cores (0: 2; the matrix
                                  cores need N % 4 == 0 and a 16-byte aligned dOut, else 1 runs) */
    int32_t fwd_prep;          /* forward weight step and quantisers in 1 one launch (used while
                                  N*K <= 2^25 and M > 0), 2 separate launches (0: 1) */
} brl_tuning;

/* Bytes of device workspace needed by an operation run with `tune` (NULL:
 * the defaults; the backward's chunk roots grow as bwd_chunk_log2 shrinks).
 * For BRL_OP_FWD and BRL_OP_BWD, M, K, N are the layer sizes (N = stacked
 * width for SwiGLU); for BRL_OP_NORM, M is the vector length and K, N are
 * ignored; for BRL_OP_HASH, M is the total byte length of the state and K
 * its tensor count (N ignored).  Returns 0 for bad sizes or tuning. */
BRL_API size_t brl_workspace_bytes(int32_t op, int64_t M, int64_t K, int64_t N, const brl_tuning* tune);

/*
 * qat_linear_fwd -- LSQ int8 quantisation-aware linear forward.
 *   s_w = (2 * mu) / fl(sqrt(127)),  mu = CanonSum(|W|) / fl(N*K) over
 *         row-major W, recomputed on every call;
 *   q_w = clamp(rne(W / s_w), -127, 127), q_x = clamp(rne(X / s_x), -127, 127)
 *         (a zero s_w quantises every weight to 0);
 *   acc = q_x . q_w^T in exact int32 (int8 matrix cores);
 *   Y   = fl(acc) * (s_x * s_w), then Y + addend when addend != NULL
 *         (a separate rounding; never fused).
 * X [M,K], W [N,K] (nn.Linear layout), addend [M,N] or NULL.
 * epilogue NONE: Y [M,N]; Ypre ignored.
 * epilogue SWIGLU: N even; Y [M,N/2] receives the activation and, when
 *   Ypre != NULL, Ypre [M,N] receives the pre-activation (needed by the
 *   backward).  addend (if any) is added before the activation.
 * s_x: the activation step, finite and > 0.
 * s_w_out: NULL or a device float that receives s_w.
 * ws: device workspace of at least brl_workspace_bytes(BRL_OP_FWD, M, K, N,
 * tune) bytes, owned by the caller; calls that overlap in time must not
 * share one.  tune: NULL or the call's launch shapes (see brl_tuning).
 * Requires |acc| < 2^31, guaranteed for K <= 133144.
 * With the one-launch preparation (tune->fwd_prep 0 or 1), workgroups of one
 * kernel wait on values other workgroups of it publish in the workspace; the
 * waits are bounded (about a second), and a wait that gives up, which needs
 * the device to leave those workgroups unscheduled that long, makes every
 * element of Y NaN instead of returning wrong numbers.
 */
BRL_API brl_status qat_linear_fwd(const float* X, const float* W, int64_t M, int64_t K, int64_t N,
                          float s_x, const float* addend, int32_t epilogue,
                          float* Y, float* Ypre, float* s_w_out,
                          void* ws, size_t ws_bytes, const brl_tuning* tune, void* stream);

/*
 * qat_linear_bwd -- straight-through backward of qat_linear_fwd.
 *   G   = dOut [M,N] (epilogue NONE), or for SWIGLU the pre-activation
 *         gradient from dOut [M,N/2] and Ypre [M,N]:
 *           du = dA*h,  dg = (dA*u) * (s*(1 + g*(1 - s))),  s = sigma(g), h = g*s;
 *   What = fl(q_w * s_w), Xhat = fl(q_x * s_x)   (recomputed from W, X, s_x);
 *   dX[m,k] = in_x[m,k] ? CanonSum_n(G[m,n] * What[n,k]) : +0
 *   dW[n,k] = in_w[n,k] ? CanonSum_m(G[m,n] * Xhat[m,k]) : +0
 *   with in_v = (-127 <= v/s <= 127) for the value's own step.
 * dX [M,K] and dW [N,K] may each be NULL (not computed).
 * dW_accumulate = 1: dW <- dW + (new dW), one binary32 add per element (the
 *   ascending microbatch running sum); 0: dW is overwritten.
 * ws: at least brl_workspace_bytes(BRL_OP_BWD, M, K, N, tune) bytes, owned
 * by the caller and not shared by overlapping calls.  tune: NULL or the
 * call's launch shapes.
 */
BRL_API brl_status qat_linear_bwd(const float* dOut, const float* X, const float* W, const float* Ypre,
                          int64_t M, int64_t K, int64_t N, float s_x, int32_t epilogue,
                          float* dX, float* dW, int32_t dW_accumulate,
                          void* ws, size_t ws_bytes, const brl_tuning* tune, void* stream);

#define BRL_MAX_REPLICAS 64

/* Caller-owned host struct describing one replay.  acc[r] are device
 * buffers of len floats (A_r), owned by the caller; next is the virtual rank
 * v = r*shards + s that ordered_reduce expects next.  flags: 0,
 * BRL_REDUCE_PARTIALS_PERSIST or BRL_REDUCE_REPLICA_RESIDENT, set by the
 * caller after brl_reduce_init; tune: the launch shapes of the replay's
 * kernels (zeroed by brl_reduce_init: the defaults; the caller may set it
 * afterwards); pending and shard_part are the library's own bookkeeping. */
#define BRL_REDUCE_PARTIALS_PERSIST 1u
#define BRL_REDUCE_REPLICA_RESIDENT 2u
#define BRL_MAX_SHARDS 64
typedef struct brl_reduce_state {
    int32_t replicas;
    int32_t shards;
    int64_t len;
    int32_t next;
    uint32_t flags;
    const float* pending;
    float* acc[BRL_MAX_REPLICAS];
    brl_tuning tune;
    const float* shard_part[BRL_MAX_SHARDS];   /* the library's bookkeeping (BRL_REDUCE_REPLICA_RESIDENT) */
} brl_reduce_state;

/* Fill a reduce state: 1 <= replicas <= 64, shards >= 1, len >= 0, acc[0..replicas)
 * non-NULL device buffers of len floats.  Sets next = 0. */
BRL_API brl_status brl_reduce_init(brl_reduce_state* st, int32_t replicas, int32_t shards, int64_t len,
                           float* const* acc);

/*
 * ordered_reduce -- one step of the audit replay of the gradient reduction.
 * Takes the partial gradient G_v [len] of virtual rank v = st->next,
 * r = v / shards, s = v % shards (mesh order: replica-major, shard-minor):
 *   s == 0: A_r = G_v;   s > 0: A_r = A_r + G_v   (binary32, elementwise).
 * After the last rank (v = replicas*shards - 1) it writes the TreeFold of
 * A_0..A_{R-1} to out [len]: with p the largest power of two <= R, leaves
 * L_i = A_i + A_{i+p} for i < R - p, else A_i, then the pairwise tree over
 * L_0..L_{p-1} -- the value every rank of a recursive-doubling all-reduce
 * holds.  For R = 6: ((A0+A4)+(A1+A5))+(A2+A3).  out may be NULL before the
 * last rank and must be non-NULL for it; the last A_r is not written back.
 * Advances st->next; a call with st->next >= replicas*shards returns
 * BRL_EORDER and launches nothing.  partial is only read during the call's
 * stream-ordered work and may be reused after it -- except with
 * BRL_REDUCE_PARTIALS_PERSIST in st->flags (and shards > 1): then the
 * shard-0 partial of each replica must stay valid and unchanged until the
 * shard-1 call of that replica has run on the stream; the shard-0 call
 * launches nothing and the shard-1 call forms A_r = G_{r,0} + G_{r,1} in one
 * pass (same bits, one copy pass fewer per replica).  With
 * BRL_REDUCE_REPLICA_RESIDENT in st->flags (and 1 < shards <=
 * BRL_MAX_SHARDS; otherwise it acts as BRL_REDUCE_PARTIALS_PERSIST), every
 * partial of a replica must stay valid and unchanged until that replica's
 * last-shard call has run on the stream: the replica's other calls launch
 * nothing, and its last-shard call forms the whole running sum
 * A_r = (((G_{r,0} + G_{r,1}) + G_{r,2}) + ...) + G_{r,S-1} in one pass over
 * the S partials -- for the last replica inside the TreeFold itself.  Same
 * bits; per element a replica then moves 4 (S + 1) bytes instead of 12 (S - 1).
 */
BRL_API brl_status ordered_reduce(brl_reduce_state* st, const float* partial, float* out, void* stream);

/*
 * grad_l2norm_clip -- global L2 norm and clip of one flat gradient.
 *   nu = fl(sqrt(CanonSum(g_i * g_i))) over g [len];
 *   when nu > max_norm: kappa = max_norm / (nu + eps), g_i <- g_i * kappa;
 *   otherwise g is left unchanged.
 * norm_out: NULL or a device float receiving nu (before clipping).
 * max_norm > 0 and eps >= 0, both finite.
 * ws: at least brl_workspace_bytes(BRL_OP_NORM, len, 0, 0, tune) bytes,
 * owned by the caller and not shared by overlapping calls.  tune: NULL or
 * the call's launch shapes.
 */
BRL_API brl_status grad_l2norm_clip(float* g, int64_t len, float max_norm, float eps, float* norm_out,
                            void* ws, size_t ws_bytes, const brl_tuning* tune, void* stream);

/*
 * grad_l2norm_clip_noalloc -- grad_l2norm_clip for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation and the same bits,
 * with no workspace argument.  The call allocates nothing; its CanonSum roots
 * and scalars live in a 2 MiB device array inside the library, one per device,
 * held until the process ends, so len is limited to BRL_NOALLOC_NORM_MAX_LEN
 * elements (a longer len returns BRL_ESHAPE and launches nothing).  The
 * stream must belong to the calling thread's current device.  Every call on
 * one device uses that device's array: calls that overlap in time on one
 * device race, and must be ordered by the caller (one stream, or events).
 */
#define BRL_NOALLOC_NORM_MAX_LEN 1056565248LL
BRL_API brl_status grad_l2norm_clip_noalloc(float* g, int64_t len, float max_norm, float eps, float* norm_out,
                                            const brl_tuning* tune, void* stream);

/*
 * brl_state_hash -- on-device hash of a training state (a list of tensors).
 * The pages store a hash of the state after every step and require a
 * replayed step to reproduce it; they name moving that hashing from the host
 * (about 6 s per step) onto the device as future work (onedev.kr summary,
 * sections "Use" and "Limits"; rit.work article body).  They do not name the
 * function; this library computes SHA-256 (FIPS 180-4) arranged as a tree:
 *   leaf  = SHA-256(4 KiB piece of one tensor's bytes || 0x00), pieces in
 *           order, the last piece of a tensor shorter, an empty tensor one
 *           empty piece; the leaves of all tensors, tensor after tensor;
 *   node  = SHA-256(16 consecutive digests (fewer for the last) || 0x01),
 *           level after level until one digest remains;
 *   root  = SHA-256(top || le64(count) || le64(nbytes[0]) ... || 0x02).
 * tensors: count (>= 1) device pointers, 4-byte aligned, read as raw bytes
 * (tensors[i] may be NULL when nbytes[i] == 0); nbytes: host array of byte
 * lengths >= 0; digest: device pointer receiving the 32 root bytes.  The host
 * arrays are read during the call only.  Workspace from
 * brl_workspace_bytes(BRL_OP_HASH, sum of nbytes, count, 0, NULL).
 */
BRL_API brl_status brl_state_hash(const void* const* tensors, const int64_t* nbytes, int32_t count,
                                  uint8_t* digest, void* ws, size_t ws_bytes, void* stream);

/*
 * AdamW update in a fixed operation order (the step after the clip).  The
 * recipe (onedev.kr summary, "Limits", recipe paragraph): AdamW with beta1
 * 0.9, beta2 0.95, eps 1e-8, decoupled weight decay 0.1 except on the input
 * embedding, the norm weights and the RoPE table; learning rate linear to
 * 4.5e-4 over about 2.1B tokens, then one cosine decay to 10% of the peak at
 * 400B tokens, keyed to consumed tokens.  The pages fix neither the operation
 * order nor the scalars' arithmetic; this library's reading:
 *   brl_adamw_scalars_for_step: lr(tokens) as above, c1 = 1 - beta1,
 *   c2 = 1 - beta2, bc1 = 1 - beta1^step, bc2 = 1 - beta2^step, d = lr * wd,
 *   each computed in binary64 and rounded once to binary32 (step >= 1);
 *   adamw_step, per element, binary32 operations in this order:
 *     m = (beta1 * m) + (c1 * g)
 *     v = (beta2 * v) + (c2 * (g * g))
 *     u = (m / bc1) / (sqrt(v / bc2) + eps)
 *     p = p - (d * p)           only when decay != 0
 *     p = p - (lr * u)
 * p, m, v (updated in place) and g: device arrays of n floats; sc: host
 * struct (copied into the launch).  cfg NULL selects the recipe.
 */
typedef struct brl_adamw_config {
    double beta1, beta2, eps, wd, peak_lr, min_lr, warmup_tokens, total_tokens;
} brl_adamw_config;
typedef struct brl_adamw_scalars {
    float beta1, beta2, c1, c2, bc1, bc2, eps, lr, d;
} brl_adamw_scalars;
BRL_API brl_status brl_adamw_scalars_for_step(int64_t step, double tokens, const brl_adamw_config* cfg,
                                              brl_adamw_scalars* out);
BRL_API brl_status adamw_step(float* p, const float* g, float* m, float* v, int64_t n,
                              const brl_adamw_scalars* sc, int32_t decay, void* stream);

/*
 * Attention with int8 P.V (onedev.kr summary, "Use", attention paragraph:
 * the P.V product of flash attention on int8 matrix units, QK^T logits and
 * softmax in high precision; grouped-query heads; causal, with a sliding
 * window on most layers).  The pages fix no step of the arithmetic; this
 * library's reading, every binary32 operation rounded on its own (FTZ):
 *   s_ij = CanonSum_d(q_id * k_jd) * c,  c = fl(1 / fl(sqrt(D)))
 *   m_i  = max_j s_ij over the row's keys j in [lo_i, i],
 *          lo_i = max(0, i - window + 1) (window <= 0: lo_i = 0)
 *   p_ij = E(s_ij - m_i) on the row's keys, +0 on all other keys
 *          (E: the library's binary32 exp, as in the SwiGLU epilogue)
 *   l_i  = CanonSum_j p_ij over the whole key axis j = 0 .. S-1
 *   q_p  = clamp(rne(p * 127), 0, 127); q_v = LSQ quantiser, step s_v
 *   O_id = (fl(sum_j q_p,ij * q_v,jd) * s_v) / (l_i * 127)
 * Layout: element (b, i, h, d) of Q at Q[(b*S + i)*ldq + h*D + d] (K, V, O
 * alike, with Hkv heads for K and V); query head h reads KV head
 * h / (Hq / Hkv).  The QKV projection's output [B*S, (Hq + 2*Hkv)*D] serves
 * directly: Q, K, V at column offsets 0, Hq*D, (Hq + Hkv)*D, ld = row width.
 * D must be 128; Hq a positive multiple of Hkv; S <= 133143 (int32 P.V
 * accumulators); every ld a multiple of 4 and >= heads*D; Q, K, V, O device
 * pointers 16-byte aligned; O must not overlap Q, K or V.  Inputs must be
 * finite.  stats (nullable, device, [B*S*Hq][2] floats, row (b*S + i)*Hq + h)
 * receives (m_i, l_i) for the backward.  ws: device workspace of at least
 * attn_fwd_workspace_bytes(B, S, Hq, Hkv, window) bytes, 256-byte aligned,
 * caller-owned, used only during the call (it holds the exact logits between
 * the two passes); BRL_EWORKSPACE if too small.  Asynchronous on `stream`.
 */
BRL_API brl_status attn_fwd(const float* Q, const float* K, const float* V, int64_t B, int64_t S, int64_t Hq,
                            int64_t Hkv, int64_t D, int64_t ldq, int64_t ldk, int64_t ldv, int64_t window,
                            float s_v, float* O, int64_t ldo, float* stats, void* ws, size_t ws_bytes,
                            void* stream);

/* Bytes of workspace attn_fwd needs for these sizes (0 for sizes it rejects).
 * It grows with the longest key walk of a query block (the window, or S for
 * full causal attention) and not with B or the head count beyond 512
 * (query block, head) items. */
BRL_API size_t attn_fwd_workspace_bytes(int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t window);

/*
 * attn_fwd that also keeps its exact logits s_ij (as defined above) for the
 * backward, which then need not form them again (attn_bwd_dq_logits,
 * attn_bwd_dkdv_logits).  The pages keep the logits in high precision
 * (onedev.kr summary, "Use", attention paragraph); keeping them in HBM trades
 * memory for one of the backward's products.  logits: device, 256-byte
 * aligned, at least attn_logits_bytes(B, S, Hq, window) bytes, caller-owned;
 * it receives one slot per (query block qb, batch b, query head h), slot
 * index (ceil(S/64) - 1 - qb) * (B*Hq) + b*Hq + h, each slot the block's key
 * tiles from its first (64 x 64 binary32, row-major by query), entries off
 * the row's keys unspecified.  BRL_ESHAPE if too small.  O and stats are the
 * same bits as attn_fwd's; other arguments and requirements as attn_fwd.
 * Asynchronous on `stream`.
 */
BRL_API brl_status attn_fwd_keep_logits(const float* Q, const float* K, const float* V, int64_t B, int64_t S,
                                        int64_t Hq, int64_t Hkv, int64_t D, int64_t ldq, int64_t ldk, int64_t ldv,
                                        int64_t window, float s_v, float* O, int64_t ldo, float* stats,
                                        float* logits, size_t logits_bytes, void* ws, size_t ws_bytes,
                                        void* stream);

/* Bytes of the logits attn_fwd_keep_logits keeps for these sizes (0 for sizes
 * it rejects): ceil(S/64) * B * Hq slots of (longest key walk of a query block,
 * in 64-key tiles) * 16 KB. */
BRL_API size_t attn_logits_bytes(int64_t B, int64_t S, int64_t Hq, int64_t window);

/*
 * dQ of attn_fwd with 64-bit fixed-point accumulation (onedev.kr summary,
 * "Use", attention paragraph: the attention backward accumulates the query
 * gradient in 64-bit fixed point).  This library's reading, with s, m, p, l,
 * q_v as in attn_fwd, O its output and dO the output gradient:
 *   P_ij = p_ij / l_i;  V^_jd = fl(q_v,jd * s_v)
 *   dP_ij = CanonSum_d(dO_id * V^_jd);  Delta_i = CanonSum_d(dO_id * O_id)
 *   dS_ij = P_ij * (dP_ij - Delta_i) on the row's keys, +0 elsewhere
 *   u_igd = CanonSum over key positions 64g .. 64g+63 of dS_ij * K_jd
 *   dQ_id = (fl(sum_g rne(u_igd * 2^40)) * 2^-40) * c
 * The tile sums are int64 fixed-point numbers with 40 fraction bits, added
 * exactly (their order cannot change the sum); the total is rounded once.
 * Valid while every |u| < 2^22 and |sum| < 2^23 (gradient scale; not
 * checked).  stats: the (m_i, l_i) that attn_fwd wrote for the same Q, K, V,
 * window.  O, dO and dQ share the layout and row stride ldo of Q's shape;
 * other arguments and requirements as attn_fwd.  dQ must not overlap the
 * inputs.  Asynchronous on `stream`.
 */
BRL_API brl_status attn_bwd_dq(const float* Q, const float* K, const float* V, const float* O, const float* dO,
                               const float* stats, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                               int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo, int64_t window, float s_v,
                               float* dQ, void* stream);

/* attn_bwd_dq reading the logits that attn_fwd_keep_logits kept for the same
 * Q, K, V, B, S, Hq, window (logits, logits_bytes as there) instead of forming
 * them again; the same bits as attn_bwd_dq. */
BRL_API brl_status attn_bwd_dq_logits(const float* Q, const float* K, const float* V, const float* O,
                                      const float* dO, const float* stats, const float* logits, size_t logits_bytes,
                                      int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t ldq,
                                      int64_t ldk, int64_t ldv, int64_t ldo, int64_t window, float s_v, float* dQ,
                                      void* stream);

/*
 * dK and dV of attn_fwd (onedev.kr summary, "Use", attention paragraph: the
 * pages give 64-bit fixed-point accumulation for the query gradient and
 * nothing for the key and value gradients; this library reads the same
 * format into both).  With P, dP, Delta and dS as in attn_bwd_dq:
 *   w_hgjd = CanonSum over the 64 query positions 64g .. 64g+63 of P_ij * dO_id
 *   z_hgjd = the same sum of dS_ij * Q_id
 *   dV_jd  = (-127 <= v_jd / s_v <= 127) ? fl(sum_{h,g} rne(w * 2^40)) * 2^-40 : +0
 *   dK_jd  = (fl(sum_{h,g} rne(z * 2^40)) * 2^-40) * c
 * summed over the query heads h of KV head j's group and every query tile g
 * (+0 terms for rows that do not attend key j and past S); the int64 sums
 * are exact, so their order cannot change them.  The range mask is the
 * straight-through estimator of V's LSQ quantiser; p's quantiser passes
 * straight through (P = p / l).  Valid while every |w|, |z| < 2^22 and each
 * sum < 2^23 in magnitude (gradient scale; not checked).
 * dK and dV: [B, S, Hkv, D] with row stride ldg (a multiple of 4, >= Hkv*D),
 * e.g. column slices of a [B*S, (Hq + 2*Hkv)*D] gradient buffer; they must
 * not overlap each other or the inputs.  Other arguments and requirements as
 * attn_bwd_dq.  Asynchronous on `stream`.
 */
BRL_API brl_status attn_bwd_dkdv(const float* Q, const float* K, const float* V, const float* O, const float* dO,
                                 const float* stats, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D,
                                 int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo, int64_t window, float s_v,
                                 float* dK, float* dV, int64_t ldg, void* stream);

/* attn_bwd_dkdv reading the logits that attn_fwd_keep_logits kept (as
 * attn_bwd_dq_logits); the same bits as attn_bwd_dkdv. */
BRL_API brl_status attn_bwd_dkdv_logits(const float* Q, const float* K, const float* V, const float* O,
                                        const float* dO, const float* stats, const float* logits,
                                        size_t logits_bytes, int64_t B, int64_t S, int64_t Hq, int64_t Hkv,
                                        int64_t D, int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo,
                                        int64_t window, float s_v, float* dK, float* dV, int64_t ldg,
                                        void* stream);

/*
 * Topology-invariant data stream (onedev.kr summary, "What differs": one
 * canonical stream independent of world size and rank, three generators --
 * source interleaving seeded by the training seed alone, shard order seeded
 * by (seed, SHA-256(source name), epoch), document order seeded by (seed,
 * SHA-256(source name), epoch, shard) -- documents joined with a separator
 * and cut into windows of 4,097 tokens; rank r of R owns windows m with
 * m mod R = r; a rank-independent resume record) with counter-based draws
 * ("How": values as pure functions of the seed and a logical position).
 * This library's reading:
 *   draw(key, stream, i): word i mod 4 of Philox4x32-10 (Salmon et al.,
 *     SC'11) with counter (i div 4 as two 32-bit words, stream, 0);
 *   bounded(x, n) = (x * n) >> 32;
 *   an order of n items: Fisher-Yates from the top, draw t (stream 0)
 *     swapping position n-1-t with bounded(draw, n-t);
 *   shard-order key: first 8 bytes, little endian, of SHA-256("shard" |
 *     le64 seed | SHA-256(name) | le64 epoch); document-order key likewise
 *     from "doc" | ... | le64 shard;
 *   source of document draw t: the first source whose cumulative weight
 *     exceeds bounded(draw(seed, 0x6d6978, t), total weight);
 *   a source moves to its next epoch when a document is requested after its
 *     last shard; shards without documents are skipped.
 * The corpus stays caller-owned and must outlive the stream (it is read,
 * never copied).  A source: NUL-terminated UTF-8 name, weight >= 0, shard
 * document counts, shard-major ascending token offsets (one more than the
 * document count), token ids.  Every source with weight > 0 needs a
 * document.  The stream object is host memory owned by the caller (create /
 * destroy); calls on one stream must not overlap.
 */
#define BRL_STREAM_WINDOW 4097
typedef struct brl_stream brl_stream;
typedef struct brl_stream_source {
    const char* name;
    int64_t weight;
    int32_t n_shards;
    const int64_t* shard_docs;    /* [n_shards] */
    const int64_t* doc_offsets;   /* [sum(shard_docs) + 1] */
    const int32_t* tokens;
} brl_stream_source;
BRL_API brl_status brl_stream_create(uint64_t seed, int32_t separator, const brl_stream_source* sources,
                                     int32_t n_sources, brl_stream** out);
BRL_API void brl_stream_destroy(brl_stream* s);
/* The next `count` windows of the global stream into out (host, count x 4097
 * int32); *first_window (nullable) receives the index m of the first. */
BRL_API brl_status brl_stream_next(brl_stream* s, int64_t count, int32_t* out, int64_t* first_window);
/* One global batch of `global_batch` windows (a multiple of ranks); out
 * (host, global_batch / ranks x 4097) receives the windows of `rank`. */
BRL_API brl_status brl_stream_step(brl_stream* s, int64_t global_batch, int32_t ranks, int32_t rank,
                                   int32_t* out);
/* Resume record: "BRLSTRM1" | le64 seed | le32 sources | le32 separator |
 * le64 next window | le64 mix draws | per source: SHA-256(name), le64 epoch,
 * le64 shard position, le64 document position, le64 documents consumed |
 * le64 buffered tokens | buffered tokens (le32; the tail of the last
 * document taken, which can exceed one window).  Independent of R.  Loading
 * checks seed, separator and source digests. */
BRL_API int64_t brl_stream_record_bytes(const brl_stream* s);
BRL_API brl_status brl_stream_save(const brl_stream* s, uint8_t* buf, int64_t cap);
BRL_API brl_status brl_stream_load(brl_stream* s, const uint8_t* buf, int64_t n);
/* Device draws: out[k] = draw(key, stream, first + k) for k < n (device
 * pointer, 4-byte aligned). */
BRL_API brl_status brl_philox_u32(uint64_t key, uint32_t stream, uint64_t first, int64_t n, uint32_t* out,
                                  void* hip_stream);

/* Conformance probe of the device's binary32 operations, as the kernels use
 * them: out[i] = op(a[i], b[i]) for op 0 add, 1 sub, 2 mul, 3 div, 4 sqrt (a),
 * 5 int32 bits of a -> float, 6 round-to-nearest-even integral (a),
 * 7 the SwiGLU exp E(a), 8 the product a*b as the backward's matrix-core
 * engine forms it (K=1 fp32 MFMA with a -0 accumulator), 9 a*a + b from the
 * same K=1 MFMA with the accumulator input b (the library never uses it that
 * way: it rounds product and sum once, which the method forbids).  Device
 * pointers, n >= 0. */
BRL_API brl_status brl_probe_f32(int32_t op, const float* a, const float* b, float* out, int64_t n,
                         void* stream);

/* Sustained-rate probe of the units the kernels run on, behind the rooflines
 * the library's benchmark reports: a grid that fills the chip
 * (brl_probe_rate_threads() threads), each thread running 8 independent
 * chains of `iters` steps of: what 0 v_add_f32 (8 binary32 adds per step),
 * 1 v_mul_f32 (8 multiplies per step), 2 the K=1 fp32 MFMA (8 per step per
 * wave, 1024 products each), 3 the i8 MFMA 32x32x32 (8 per step per wave,
 * 65536 integer ops each), 4 32-bit integer VALU (a shift and an xor, 16
 * instructions per step), 5 v_add_f32 with a scalar-register operand,
 * 6 the backward's product engine without memory traffic (4 K=1 fp32 MFMAs
 * with a -0 accumulator and the 64 v_add_f32 that sum their products: 4096
 * multiply-adds per wave per step), 7 the i8 MFMA on operands that change
 * from one MFMA to the next (32 per step per wave, 65536 integer ops each),
 * 8 the product engine of 6 on operands that change from one MFMA to the
 * next (16 MFMAs and their 256 adds per lane per step: 16384 multiply-adds
 * per wave per step).
 * out: device, at least brl_probe_rate_threads()
 * floats, receives each thread's chain results (values of no meaning).  The
 * caller times the call with events on `stream`. */
BRL_API brl_status brl_probe_rate(int32_t what, int64_t iters, float* out, int64_t out_len, void* stream);
BRL_API int64_t brl_probe_rate_threads(void);

BRL_API const char* brl_status_string(brl_status s);
BRL_API const char* brl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BRLSQ_H */
