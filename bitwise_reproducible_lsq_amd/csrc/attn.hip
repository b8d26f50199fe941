// attn.hip -- attention with int8 P.V, high-precision logits and softmax.
//
// Open-1B summary on onedev.kr, "Use", attention paragraph: inside flash
// attention the P.V product runs on int8 matrix units while the QK^T logits
// and the softmax stay in high precision; grouped-query attention (16 query
// heads over 4 KV heads), a 512-token sliding window with full causal
// attention on some layers.  The pages fix no step of the arithmetic; this
// library's reading (every binary32 operation rounded on its own, FTZ):
//   s_ij = CanonSum_d(q_id * k_jd) * c,       c = 1 / sqrt(D)
//   m_i  = max of s_ij over the row's keys j in [lo_i, i]
//   p_ij = E(s_ij - m_i) on the row's keys, +0 on every other key
//   l_i  = CanonSum of p_ij over the whole key axis j = 0 .. S-1
//   q_p  = clamp(rne(p * 127), 0, 127),  q_v = LSQ quantiser with step s_v
//   O_id = (fl(sum_j q_p,ij * q_v,jd) * s_v) / (l_i * 127)
// with E the library's own binary32 exp.  The integer product is exact and
// order-free, so only the logits and l_i carry an order, and both are fixed
// by absolute positions (d, and the key index j), not by tiles.
//
// Forward: a persistent grid of workgroups, each walking (batch, query head,
// block of 64 queries) items, longest first; two passes over the 64-key
// tiles that meet the block's key range:
//   pass 1: exact logits on the product engine below (the matrix cores form
//           each product, rounded on its own; the VALU adds d-blocks of 32
//           left to right, then the pairwise tree), stored in the
//           workgroup's slot of the workspace; each lane keeps running
//           maxima of its rows (order-free integer maxima), reduced over
//           the workgroup once per item;
//   pass 2: the stored logits -> p -> the 32-key block sums, each two
//           16-add chains of one row's consecutive keys joined by a DPP
//           shift; a tile's two blocks are a complete pair (their absolute
//           indices are 2kt, 2kt+1), so their sum is pushed on the row's
//           binary-counter stack of pairs at index kt; q_p and q_v staged as
//           int8 in LDS and multiplied on v_mfma_i32_32x32x32_i8 into int32
//           accumulators.
// Pass 2 reads the logits with another thread mapping (one row and 16 keys
// per thread) after a workgroup barrier.
// Pairs before the first real one are +0 subtrees (the stack starts zeroed)
// and merging with +0 is exact, so this is CanonSum over the whole axis.
// LDS is kept under 80 KB so that two workgroups share a CU.
//
// Backward (further down): dQ, dK and dV with 64-bit fixed-point
// accumulation, their products formed on the matrix cores.
#include "internal.hpp"

#pragma clang fp contract(off)

namespace brl {

typedef int v4i_a __attribute__((ext_vector_type(4)));
typedef unsigned v4u_a __attribute__((ext_vector_type(4)));
typedef int v16i_a __attribute__((ext_vector_type(16)));

constexpr int kAD = 128;          // head dimension
constexpr int kAQ = 64;           // queries per workgroup
constexpr int kAK = 64;           // keys per tile
constexpr int kAStack = 12;       // pair-stack levels: up to 2^12 key tiles

typedef float v16f_a __attribute__((ext_vector_type(16)));

constexpr int kKvThreads = 512;
constexpr int kKvRow = kAD + 4;     // floats per LDS row of K, Q and dO
constexpr int kKvRowQ = kAD + 16;   // bytes per LDS row of q_v
constexpr int kKvRowT = kAQ + 4;    // floats per LDS row of the key-major tiles

struct AttnArgs {
    const float* Q;
    const float* K;
    const float* V;
    float* O;
    float* stats;          // optional (m_i, l_i) per row (b*S + i)*Hq + h
    float* logits;         // slot_floats floats per workgroup: [tile][64 rows][64 keys]
    float* keep;           // optional: slot_floats floats per item, kept for the backward
    const int8_t* vcodes;  // q_v tiles [B][Hkv][tiles][kAD * kAK], laid out as sm.u.pv.vq
    int64_t B, S, Hq, Hkv, ldq, ldk, ldv, ldo, window, slot_floats, vtiles;
    float c, s_v;
    ExpConsts ek;
};

struct AttnSmem {
    union {
        struct {
            float qr[kAQ][kKvRow];  // Q tile, row-major
            float kr[kAK][kKvRow];  // K tile, key-major
        } a;                        // pass 1
        struct {
            int8_t pq[2][kAQ][kAK]; // q_p, rows of 64 keys, 16-byte chunks swizzled
            int8_t vq[2][kAD][kAK]; // q_v transposed: row d holds 64 keys, swizzled
        } pv;                       // pass 2, double-buffered by key tile
    } u;
    float st[kAQ][kAStack];         // per-row stacks of key-tile pair sums
    int rowmax[kAQ];                // row maxima as order-preserving integer images
    float rowdiv[kAQ];              // l_i * 127
};
static_assert(sizeof(AttnSmem) <= 81920, "two workgroups per CU");

__device__ __forceinline__ int aswz(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

// left-to-right running sum handed from lane to lane + 1 within a 16-lane row
__device__ __forceinline__ float dpp_shr1(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, false));
}
__device__ __forceinline__ float dpp_shr2(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, false));
}
__device__ __forceinline__ float dpp_shr8(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, false));
}

// q_v of one 64-key tile of V (keys j0 .. j0+63 of rows base + j, KV head
// hk) into the tile layout the P.V product reads: row d holds the 64 keys'
// codes, its 16-byte chunks swizzled by aswz.  Each of the 256 threads owns
// items of 4 keys x 4 d, stored as four 4-byte key runs.  Codes on the
// quantiser's fast path; a wave with a value near a rounding midpoint redoes
// its values on the exact path.  Keys at or past S quantise zeros (code 0).
__device__ __forceinline__ void attn_quant_v_tile(const float* V, int64_t ldv, int64_t base, int64_t j0, int64_t S,
                                                  int64_t hk, const Quantizer& qz, int8_t* tile) {
#pragma unroll
    for (int it = 0; it < (kAK / 4) * (kAD / 4) / 256; ++it) {
        const int e = threadIdx.x + 256 * it;
        const int rq = e & 15, dq = e >> 4;
        vf4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t j = j0 + 4 * rq + u;
            v[u] = vf4{0.0f, 0.0f, 0.0f, 0.0f};
            if (j < S) v[u] = *reinterpret_cast<const vf4*>(V + (base + j) * ldv + hk * kAD + 4 * dq);
        }
        uint32_t packed[4];
        bool unsure = false;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            packed[w] = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                packed[w] |= (uint32_t)(uint8_t)(int8_t)qz.q_fast(v[u][w], &unsure) << (8 * u);
        }
        if (__ballot(unsure)) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                packed[w] = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    bool in;
                    packed[w] |= (uint32_t)(uint8_t)(int8_t)qz.q(v[u][w], &in) << (8 * u);
                }
            }
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int d = 4 * dq + w, r = 4 * rq;
            *reinterpret_cast<uint32_t*>(tile + d * kAK + 16 * aswz(d, r >> 4) + (r & 15)) = packed[w];
        }
    }
}

// q_v of every key tile, once per (batch, KV head): workgroup (b, hk, kt)
// writes tile kt of [B][Hkv][tiles][kAD * kAK] codes
__global__ __launch_bounds__(256) void attn_quant_v_kernel(const float* __restrict__ V, int64_t ldv, int64_t S,
                                                           int64_t Hkv, int64_t tiles, float s_v,
                                                           int8_t* __restrict__ codes) {
    // 32-bit unsigned index arithmetic (the host checks that the grid fits)
    const unsigned t = (unsigned)tiles, bh = blockIdx.x / t;
    const int64_t kt = blockIdx.x % t;
    const int64_t hk = bh % (unsigned)Hkv, b = bh / (unsigned)Hkv;
    const Quantizer qz(s_v);
    attn_quant_v_tile(V, ldv, b * S, kt * kAK, S, hk, qz, codes + blockIdx.x * (int64_t)(kAD * kAK));
}

// ---- the product engine shared by the forward's logits and the backward ----
// A 16x16x1 fp32 MFMA with a K of one and an accumulator input of -0 forms
// fl(a*b) for each of its 1024 (a, b) pairs, bit-identical to v_mul_f32
// (FTZ); the VALU adds the products in the canonical order.  Lane l feeds A
// row l and B column l % 16; register 4*beta + e of lane l receives row
// 16*beta + 4*(l / 16) + e, column l % 16.
__device__ __forceinline__ v16f_a mfma_prod(float a, float b) {
    v16f_a cneg;
#pragma unroll
    for (int r = 0; r < 16; ++r) cneg[r] = -0.0f;
    return __builtin_amdgcn_mfma_f32_16x16x1f32(a, b, cneg, 0, 0, 0);
}

// Both phases run one product chain per wave, software-pipelined: the MFMA
// of step s + 1 is issued before the adds of step s, and the operands of the
// next 4 steps are read while the current 4 are consumed.  KV_STEP(acc)
// keeps the adds of a step at their place in the program (an empty asm that
// takes the running sums in and out); without it the compiler hoists all
// MFMAs of a block ahead of the adds and runs out of registers.
#define KV_STEP(acc) __asm__ volatile("" : "+v"(acc))

// four B operands (d .. d+3) of one key row: fp32, or q_v dequantised as
// fl(q_v * s_v)
template <bool DQV>
__device__ __forceinline__ vf4 kv_b4(const float* brow, const int8_t* bq, float s_v, int d) {
    vf4 bv;
    if constexpr (DQV) {
        const int q4 = *reinterpret_cast<const int*>(bq + d);
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] = f_mul((float)(int8_t)(q4 >> (8 * e)), s_v);
    } else {
        bv = *reinterpret_cast<const vf4*>(brow + d);
    }
    return bv;
}

// phase 1 of one wave: CanonSum over d of A[lane][d] * B[key][d] for 64
// rows x 16 keys: d-blocks of 32 left to right, then (b0 + b1) + (b2 + b3)
template <bool DQV>
__device__ __forceinline__ v16f_a kv_phase1(const float* arow, const float* brow, const int8_t* bq, float s_v) {
    v16f_a b01, b2, acc;
#pragma unroll 1
    for (int blk = 0; blk < kAD / 32; ++blk) {
        const int d0 = 32 * blk;
        v16f_a n;
        vf4 a_cur = *reinterpret_cast<const vf4*>(arow + d0), b_cur = kv_b4<DQV>(brow, bq, s_v, d0), a_nxt, b_nxt;
        v16f_a p = mfma_prod(a_cur[0], b_cur[0]);
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            if (g + 1 < 8) {
                a_nxt = *reinterpret_cast<const vf4*>(arow + d0 + 4 * (g + 1));
                b_nxt = kv_b4<DQV>(brow, bq, s_v, d0 + 4 * (g + 1));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int st = 4 * g + e;
                if (st + 1 < 32) n = e < 3 ? mfma_prod(a_cur[e + 1], b_cur[e + 1]) : mfma_prod(a_nxt[0], b_nxt[0]);
                if (st == 0) acc = p;
                else acc = acc + p;
                KV_STEP(acc);
                p = n;
            }
            a_cur = a_nxt;
            b_cur = b_nxt;
        }
        if (blk == 0) b01 = acc;
        else if (blk == 1) b01 = b01 + acc;
        else if (blk == 2) b2 = acc;
    }
    return b01 + (b2 + acc);
}

// half of kv_phase1: the d-blocks at d_first and d_first + 32, left to right
// within each, then b_first + b_second (so kv_phase1 = pair(0) + pair(64))
template <bool DQV>
__device__ __forceinline__ v16f_a kv_phase1_pair(const float* arow, const float* brow, const int8_t* bq, float s_v,
                                                 int d_first) {
    v16f_a first, acc;
#pragma unroll 1
    for (int blk = 0; blk < 2; ++blk) {
        const int d0 = d_first + 32 * blk;
        v16f_a n;
        vf4 a_cur = *reinterpret_cast<const vf4*>(arow + d0), b_cur = kv_b4<DQV>(brow, bq, s_v, d0), a_nxt, b_nxt;
        v16f_a p = mfma_prod(a_cur[0], b_cur[0]);
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            if (g + 1 < 8) {
                a_nxt = *reinterpret_cast<const vf4*>(arow + d0 + 4 * (g + 1));
                b_nxt = kv_b4<DQV>(brow, bq, s_v, d0 + 4 * (g + 1));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int st = 4 * g + e;
                if (st + 1 < 32) n = e < 3 ? mfma_prod(a_cur[e + 1], b_cur[e + 1]) : mfma_prod(a_nxt[0], b_nxt[0]);
                if (st == 0) acc = p;
                else acc = acc + p;
                KV_STEP(acc);
                p = n;
            }
            a_cur = a_nxt;
            b_cur = b_nxt;
        }
        if (blk == 0) first = acc;
    }
    return first + acc;
}

// rows 16w .. 16w+15 of one head for wave w (rows past `rows_left` as
// zeros), row-major into dst: the rows that wave's products read
__device__ __forceinline__ void attn_load_wave_rows(const float* src, int64_t ld, int64_t row0, int64_t rows_left,
                                                    int64_t head, float (*dst)[kKvRow], int wave, int lane) {
#pragma unroll
    for (int e = lane; e < 16 * (kAD / 4); e += 64) {
        const int row = 16 * wave + e / (kAD / 4), d4 = (e % (kAD / 4)) * 4;
        vf4 v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (row < rows_left) v = *reinterpret_cast<const vf4*>(src + (row0 + row) * ld + head * kAD + d4);
        *reinterpret_cast<vf4*>(&dst[row][d4]) = v;
    }
}

// 64 rows of one head (rows past `rows_left` as zeros), row-major into dst
__device__ __forceinline__ void attn_load_rows(const float* src, int64_t ld, int64_t row0, int64_t rows_left,
                                               int64_t head, float (*dst)[kKvRow]) {
#pragma unroll 4
    for (int e = threadIdx.x; e < kAQ * (kAD / 4); e += 256) {
        const int row = e / (kAD / 4), d4 = (e % (kAD / 4)) * 4;
        vf4 v = {0.0f, 0.0f, 0.0f, 0.0f};
        if (row < rows_left) v = *reinterpret_cast<const vf4*>(src + (row0 + row) * ld + head * kAD + d4);
        *reinterpret_cast<vf4*>(&dst[row][d4]) = v;
    }
}

// order-preserving integer image of a binary32 value (negative values:
// bits ^ 0x7fffffff), so that an integer maximum is the float maximum
__device__ __forceinline__ int max_image(float f) {
    const int b = __float_as_int(f);
    return b >= 0 ? b : b ^ 0x7fffffff;
}
// the larger of k and k from the lane `sh` places away in its DPP row of 16
// lanes (row_ror:sh): four of these give every lane its row's maximum
template <int SH>
__device__ __forceinline__ int max_ror(int k) {
    const int o = __builtin_amdgcn_update_dpp(0, k, 0x120 + SH, 0xf, 0xf, false);
    return o > k ? o : k;
}
__device__ __forceinline__ float from_max_image(int k) { return __int_as_float(k >= 0 ? k : k ^ 0x7fffffff); }

// key tiles [kt0, kt1] that meet the key ranges of query block qb
__host__ __device__ __forceinline__ void attn_tile_range(int64_t S, int64_t window, int64_t qb, int64_t* kt0,
                                                         int64_t* kt1) {
    const int64_t q0 = qb * kAQ;
    const int64_t qrows = S - q0 < kAQ ? S - q0 : kAQ;
    const int64_t klo = window > 0 ? (q0 - window + 1 > 0 ? q0 - window + 1 : 0) : 0;
    *kt0 = klo / kAK;
    *kt1 = (q0 + qrows - 1) / kAK;
}

__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    AttnSmem& sm = *reinterpret_cast<AttnSmem*>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // items in 32-bit unsigned arithmetic (the host checks that they fit);
    // query blocks slowest and from the last, so that the longest walks
    // (last blocks, causal) start first
    const unsigned nqb = (unsigned)((a.S + kAQ - 1) / kAQ);
    const unsigned nbh = (unsigned)(a.B * a.Hq), hq = (unsigned)a.Hq;
    const unsigned nitems = nqb * nbh;
    const int mt = wave & 1, nt0 = (wave >> 1) * 2;
    const int frow = lane & 31, fchunk = lane >> 5;

    for (unsigned item = blockIdx.x; item < nitems; item += gridDim.x) {
        // the item's logits: in the workgroup's slot, or kept per item
        float* slot = a.keep ? a.keep + (int64_t)item * a.slot_floats : a.logits + (int64_t)blockIdx.x * a.slot_floats;
        const unsigned qb = nqb - 1 - item / nbh;
        const unsigned bh = item % nbh;
        const int64_t h = bh % hq;
        const int64_t b = bh / hq;
        const int64_t hk = (unsigned)h / (hq / (unsigned)a.Hkv);
        const int64_t q0 = (int64_t)qb * kAQ;
        const int64_t qrows = a.S - q0 < kAQ ? a.S - q0 : kAQ;
        const int64_t base = b * a.S;                // first row of this batch entry
        int64_t kt0, kt1;
        attn_tile_range(a.S, a.window, qb, &kt0, &kt1);

        // row il of the block may attend key jl of the tile at key offset
        // dlt = j0 - q0 (32-bit: the host bounds S); `full`: every row of the
        // block may attend every key of the tile
        const int nrows = (int)qrows;
        const int win = (a.window <= 0 || a.window >= a.S) ? 0 : (int)a.window;   // 0: no window
        auto allowed = [&](int dlt, int il, int jl) {
            const int t = dlt + jl - il;                      // key - row
            return (il < nrows) & (t <= 0) & ((win == 0) | (t > -win));
        };
        auto full_tile = [&](int dlt) {
            return nrows == kAQ && dlt + kAK - 1 <= 0 && (win == 0 || dlt - (kAQ - 1) > -win);
        };

        __syncthreads();                             // the previous item is done with LDS
        attn_load_rows(a.Q, a.ldq, base + q0, qrows, h, sm.u.a.qr);
        for (int e = tid; e < kAQ * kAStack; e += 256) sm.st[e / kAStack][e % kAStack] = 0.0f;
        if (tid < kAQ) sm.rowmax[tid] = max_image(__int_as_float(0xff800000));

        // ---- pass 1: exact logits on the product engine, stored; row maxima ----
        // wave w: keys 16w .. 16w+15 of the tile for all 64 rows; register r
        // of lane l holds row 16(r >> 2) + 4(l >> 4) + (r & 3), key 16w + l % 16
        const int jl = 16 * wave + (lane & 15);
        // this lane's maxima of its 16 rows over its keys of every tile, as
        // order-preserving integer images (any order gives the same bits)
        int kmax[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) kmax[r] = max_image(__int_as_float(0xff800000));
        __syncthreads();                             // the Q tile is in LDS
        for (int64_t kt = kt0; kt <= kt1; ++kt) {
            const int64_t j0 = kt * kAK;
            const int dlt = (int)(j0 - q0);
            // each wave reads only its own 16 key rows, so it loads them itself
            // (after its own reads of the previous tile's rows): no workgroup
            // barrier inside pass 1
            attn_load_wave_rows(a.K, a.ldk, base + j0, a.S - j0, hk, sm.u.a.kr, wave, lane);
            const v16f_a sx = kv_phase1<false>(&sm.u.a.qr[lane][0], &sm.u.a.kr[jl][0], nullptr, 0.0f);
            float* dst = slot + (kt - kt0) * (kAQ * kAK) + 4 * (lane >> 4) * kAK + jl;
            const bool full = full_tile(dlt);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int il = 16 * (r >> 2) + 4 * (lane >> 4) + (r & 3);
                const float v = f_mul(sx[r], a.c);
                dst[(16 * (r >> 2) + (r & 3)) * kAK] = v;
                const int k = (full | allowed(dlt, il, jl)) ? max_image(v) : max_image(__int_as_float(0xff800000));
                kmax[r] = k > kmax[r] ? k : kmax[r];
            }
        }
        // each row's maximum over the 16 lanes of its lane group (rotations
        // within a DPP row of 16 lanes), then over the four waves
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            int k = kmax[r];
            k = max_ror<1>(k);
            k = max_ror<2>(k);
            k = max_ror<4>(k);
            k = max_ror<8>(k);
            if ((lane & 15) == 0) atomicMax(&sm.rowmax[16 * (r >> 2) + 4 * (lane >> 4) + (r & 3)], k);
        }
        // the maxima, and every thread's logit stores, visible to the workgroup
        __syncthreads();
        // pass 2 thread mapping: row pi = tid / 4 (wave w: rows 16w .. 16w+15),
        // keys 16 pk .. 16 pk + 15 of each tile
        const int pi = tid >> 2, pk = tid & 3;
        const float mrow = from_max_image(sm.rowmax[pi]);

        // ---- pass 2: p, row sums, int8 P.V ----
        v16i_a acc[2];
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[n][r] = 0;
        // a tile's logits of this thread's 16 keys, stored in pass 1 by the
        // lanes of the product engine (the barrier after pass 1 made them
        // visible to the workgroup), and its q_v codes (8 KB, copied into LDS
        // as they lie), loaded one tile ahead of their use
        const v4i_a* vbase = reinterpret_cast<const v4i_a*>(a.vcodes + (b * a.Hkv + hk) * a.vtiles *
                                                                            (int64_t)(kAD * kAK));
        vf4 svn[4];
        v4i_a vtn[2];
        auto fetch = [&](int64_t kt) {
            const float* src = slot + (kt - kt0) * (kAQ * kAK);
#pragma unroll
            for (int u = 0; u < 4; ++u) svn[u] = *reinterpret_cast<const vf4*>(src + pi * kAK + 16 * pk + 4 * u);
            const v4i_a* vsrc = vbase + kt * (kAD * kAK / 16);
#pragma unroll
            for (int k = 0; k < 2; ++k) vtn[k] = vsrc[tid + 256 * k];
        };
        fetch(kt0);
        for (int64_t kt = kt0; kt <= kt1; ++kt) {
            const int64_t j0 = kt * kAK;
            const int dlt = (int)(j0 - q0);
            const bool full = full_tile(dlt);
            const int buf = (int)((kt - kt0) & 1);
            vf4 sv[4];
            v4i_a vt[2];
#pragma unroll
            for (int x = 0; x < 4; ++x) sv[x] = svn[x];
#pragma unroll
            for (int k = 0; k < 2; ++k) vt[k] = vtn[k];
            if (kt < kt1) fetch(kt + 1);
            // buffer `buf` was last read by the P.V of tile kt - 2, which every
            // wave finished before the barrier of tile kt - 1 (for the first
            // two tiles: pass 1's reads, finished before the barrier after it)
#pragma unroll
            for (int k = 0; k < 2; ++k) reinterpret_cast<v4i_a*>(&sm.u.pv.vq[buf][0][0])[tid + 256 * k] = vt[k];
            float p[16];
            uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float ex = own_exp(f_sub(sv[e >> 2][e & 3], mrow), a.ek);
                p[e] = (full | allowed(dlt, pi, 16 * pk + e)) ? ex : 0.0f;
                float r = f_rne(f_mul(p[e], 127.0f));
                r = r > 127.0f ? 127.0f : (r < 0.0f ? 0.0f : r);
                packed[e >> 2] |= (uint32_t)(int)r << (8 * (e & 3));
            }
            *reinterpret_cast<v4u_a*>(&sm.u.pv.pq[buf][pi][16 * aswz(pi, pk)]) =
                v4u_a{packed[0], packed[1], packed[2], packed[3]};
            // 32-key block sums, left to right: block k's keys lie in lanes
            // pk = 2k (first half) and 2k + 1.  Every lane forms both chains;
            // the first half's sum is kept from lanes pk even, the block's from
            // lanes pk odd.
            float h = p[0];
#pragma unroll
            for (int e = 1; e < 16; ++e) h = f_add(h, p[e]);
            float blk = f_add(dpp_shr1(h), p[0]);
#pragma unroll
            for (int e = 1; e < 16; ++e) blk = f_add(blk, p[e]);
            // lane pk = 3: block 0's sum (from lane pk = 1) + block 1's, the
            // complete subtree of blocks 2kt, 2kt + 1, pushed on the row's stack
            const float pair = f_add(dpp_shr2(blk), blk);
            if (pk == 3) {
                float v = pair;
                unsigned cnt = (unsigned)kt;
                int L = 0;
                while (cnt & 1u) {
                    v = f_add(sm.st[pi][L], v);
                    cnt >>= 1;
                    ++L;
                }
                sm.st[pi][L] = v;
            }
            __syncthreads();
            // P.V on the matrix cores: this wave's 32 rows x 64 columns, k = 64 keys
#pragma unroll
            for (int ks = 0; ks < kAK / 32; ++ks) {
                const int chunk = fchunk + 2 * ks;
                const int ar = mt * 32 + frow;
                const v4i_a A = *reinterpret_cast<const v4i_a*>(&sm.u.pv.pq[buf][ar][16 * aswz(ar, chunk)]);
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const int br = (nt0 + n) * 32 + frow;
                    const v4i_a Bf = *reinterpret_cast<const v4i_a*>(&sm.u.pv.vq[buf][br][16 * aswz(br, chunk)]);
                    acc[n] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, Bf, acc[n], 0, 0, 0);
                }
            }
        }
        __syncthreads();
        // l_i: final merge of the pair stack at the absolute tile count
        if (tid < kAQ) {
            const unsigned count = (unsigned)(kt1 + 1);
            float root = 0.0f;
            bool have = false;
            for (int L = 0; L < kAStack; ++L)
                if (count & (1u << L)) {
                    root = have ? f_add(sm.st[tid][L], root) : sm.st[tid][L];
                    have = true;
                }
            sm.rowdiv[tid] = f_mul(root, 127.0f);
            if (a.stats && tid < qrows) {
                float* st2 = a.stats + 2 * ((base + q0 + tid) * a.Hq + h);
                st2[0] = from_max_image(sm.rowmax[tid]);
                st2[1] = root;
            }
        }
        __syncthreads();
        // O = (fl(acc) * s_v) / (l * 127)
        const int col_l = lane & 31, row_q = (lane >> 5) * 4;
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = mt * 32 + (r >> 2) * 8 + row_q + (r & 3);
                const int d = (nt0 + n) * 32 + col_l;
                if (i < qrows) {
                    const float y = f_div(f_mul((float)acc[n][r], a.s_v), sm.rowdiv[i]);
                    a.O[(base + q0 + i) * a.ldo + h * kAD + d] = y;
                }
            }
    }
}

// Tiles of the longest key walk of any query block, and the persistent grid:
// two workgroups per CU on the 256 CUs of an MI355X (each walks items until
// none is left, so the grid size changes only the split of the work)
constexpr int64_t kAttnGrid = 512;

int64_t attn_fwd_max_tiles(int64_t S, int64_t window) {
    int64_t best = 0;
    for (int64_t qb = 0; qb * kAQ < S; ++qb) {
        int64_t kt0, kt1;
        attn_tile_range(S, window, qb, &kt0, &kt1);
        best = kt1 - kt0 + 1 > best ? kt1 - kt0 + 1 : best;
    }
    return best;
}

int64_t attn_fwd_grid(int64_t B, int64_t S, int64_t Hq) {
    const int64_t items = B * Hq * ceil_div(S, kAQ);
    return items < kAttnGrid ? items : kAttnGrid;
}

// logits kept for the backward: one slot per (query block, batch x head)
// item, in the forward's item order
size_t attn_keep_bytes(int64_t B, int64_t S, int64_t Hq, int64_t window) {
    if (B <= 0 || S <= 0) return 0;
    return (size_t)(B * Hq * ceil_div(S, kAQ)) * (size_t)attn_fwd_max_tiles(S, window) * (size_t)(kAQ * kAK) *
           sizeof(float);
}

// workspace: the logit slots, then the q_v codes (both 256-byte aligned)
static size_t attn_fwd_slots_bytes(int64_t B, int64_t S, int64_t Hq, int64_t window) {
    return (size_t)attn_fwd_grid(B, S, Hq) * (size_t)attn_fwd_max_tiles(S, window) * (size_t)(kAQ * kAK) *
           sizeof(float);
}

size_t attn_fwd_ws_bytes(int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t window) {
    if (B <= 0 || S <= 0) return 256;
    return attn_fwd_slots_bytes(B, S, Hq, window) + (size_t)(B * Hkv * ceil_div(S, kAK)) * (kAD * kAK) + 256;
}

hipError_t launch_attn_fwd(const float* Q, const float* K, const float* V, int64_t B, int64_t S, int64_t Hq,
                           int64_t Hkv, int64_t ldq, int64_t ldk, int64_t ldv, int64_t window, float s_v,
                           float* O, int64_t ldo, float* stats, float* logits, float* keep, const ExpConsts& ek,
                           hipStream_t st) {
    if (B == 0 || S == 0) return hipSuccess;
    AttnArgs a;
    a.Q = Q; a.K = K; a.V = V; a.O = O; a.stats = stats; a.logits = logits; a.keep = keep;
    a.B = B; a.S = S; a.Hq = Hq; a.Hkv = Hkv; a.ldq = ldq; a.ldk = ldk; a.ldv = ldv; a.ldo = ldo; a.window = window;
    a.slot_floats = attn_fwd_max_tiles(S, window) * (kAQ * kAK);
    a.vtiles = ceil_div(S, kAK);
    int8_t* codes = reinterpret_cast<int8_t*>(logits) + attn_fwd_slots_bytes(B, S, Hq, window);
    a.vcodes = codes;
    // c = fl(1 / fl(sqrt(D))): both binary64 results are rounded once more to
    // binary32, which is innocuous for sqrt and division (53 >= 2 * 24 + 2)
    a.c = (float)(1.0 / (double)(float)sqrt((double)kAD));
    a.s_v = s_v;
    a.ek = ek;
    // the limit is set on every call: it is per device, and the call is cheap
    if (const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(AttnSmem));
        e != hipSuccess)
        return e;
    if (B * Hq * ceil_div(S, kAQ) > 0xffffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(attn_quant_v_kernel, dim3((unsigned)(B * Hkv * a.vtiles)), dim3(256), 0, st, V, ldv, S, Hkv,
                       a.vtiles, s_v, codes);
    hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)attn_fwd_grid(B, S, Hq)), dim3(256), sizeof(AttnSmem), st, a);
    return hipGetLastError();
}

// ---- dQ with 64-bit fixed-point accumulation ------------------------------------
// The attention backward accumulates dQ in 64-bit fixed point (onedev.kr
// summary, "Use", attention paragraph).  This library's reading, with s, m,
// p, l as in the forward (m and l from the forward's stats) and O its output:
//   P_ij = p_ij / l_i;  dP_ij = CanonSum_d(dO_id * V^_jd), V^ = fl(q_v * s_v);
//   Delta_i = CanonSum_d(dO_id * O_id);
//   dS_ij = P_ij * (dP_ij - Delta_i) on the row's keys, +0 elsewhere;
//   u_igd = CanonSum over the 64 key positions of tile g of dS_ij * K_jd;
//   dQ_id = (fl(sum_g rne(u_igd * 2^40)) * 2^-40) * c.
// The tile sums become int64 with 40 fraction bits and add exactly, in any
// order (the kernel follows the key and value gradients below, on the same
// matrix-core engine).

struct AttnBwdArgs {
    const float* Q;
    const float* K;
    const float* V;
    const float* O;
    const float* dO;
    const float* stats;
    float* dQ;
    const float* keep;     // optional: the logits the forward kept, keep_slot floats per item
    int64_t S, Hq, Hkv, B, ldq, ldk, ldv, ldo, window, keep_slot;
    float c, s_v;
    ExpConsts ek;
};

// dK and dV of the attention.  The pages give the 64-bit fixed-point
// accumulation for dQ only; this library reads the same format into the key
// and value gradients (s, m, p, l, P, dP, Delta, dS as for dQ):
//   w_hgjd = CanonSum over the 64 query positions of tile g of P_ij * dO_id
//   z_hgjd = the same sum of dS_ij * Q_id
//   dV_jd  = V_jd in the quantiser's range ? fl(sum_{h,g} rne(w * 2^40)) * 2^-40 : +0
//   dK_jd  = (fl(sum_{h,g} rne(z * 2^40)) * 2^-40) * c
// over the query heads h of the KV head and every query tile g; rows that do
// not attend key j give +0 terms.  The sum over tiles and heads is exact, so
// one workgroup per (key tile, batch, KV head) walks its heads and query
// tiles in any order.  K and q_v stay in LDS for the whole walk; each visit
// brings one query tile of Q and dO.
//
// Every product is formed on the matrix cores, as in the linear backward: a
// 16x16x1 fp32 MFMA with a K of one and an accumulator input of -0 returns
// fl(a*b) for each of its (a, b) pairs, bit-identical to v_mul_f32 (FTZ), and
// the VALU adds the products in the canonical order.  Lane l feeds A row l
// and B column l % 16; register 4*beta + e of lane l receives row
// 16*beta + 4*(l / 16) + e, column l % 16 (64 rows x 16 columns per MFMA).
//   phase 1 (8 waves): logits (waves 0-3) and dP (waves 4-7) for key slab
//     16*(w % 4) .. +15, the four d-blocks left to right, then
//     (b0 + b1) + (b2 + b3); stored key-major;
//   an elementwise pass forms P and dS for the 64 x 64 tile;
//   phase 2 (8 waves): the tile sums over the 64 query positions (two
//     32-blocks, then the pair) of P x dO, then of dS x Q, for d slab
//     16*w .. +15, each into 16 int64 accumulators.
struct AttnKvArgs {
    const float* Q;
    const float* K;
    const float* V;
    const float* O;
    const float* dO;
    const float* stats;
    float* dK;
    float* dV;
    const float* keep;     // optional: the logits the forward kept, keep_slot floats per item
    int64_t S, Hq, Hkv, B, ldq, ldk, ldv, ldo, ldg, window, keep_slot;
    float c, s_v;
    ExpConsts ek;
};

struct AttnKvSmem {
    float kr[kAK][kKvRow];          // K tile, key-major
    float qr[kAQ][kKvRow];          // Q tile, row-major
    float gr[kAQ][kKvRow];          // dO tile, row-major
    float pt[kAK][kKvRowT];         // logits, then P (key-major)
    float dt[kAK][kKvRowT];         // dP, then dS (key-major)
    int8_t vq[kAK][kKvRowQ];        // q_v tile, key-major
    float rowm[kAQ], rowl[kAQ], rowdelta[kAQ];
};
static_assert(sizeof(AttnKvSmem) <= 163840, "LDS of one CU");

// phase 2 of one wave: the tile sum over the 64 query positions of
// T[key][i] * R[i][dcol] (keys from the lanes), two 32-blocks left to right
// and then the pair, into int64 accumulators with 40 fraction bits
__device__ __forceinline__ void kv_phase2(const float (*T)[kKvRowT], const float (*R)[kKvRow], int lane, int dcol,
                                          int64_t (&fx)[16]) {
    v16f_a acc, first;
#pragma unroll 1
    for (int bb = 0; bb < 2; ++bb) {
        const int i0 = 32 * bb;
        v16f_a n;
        vf4 a_cur = *reinterpret_cast<const vf4*>(&T[lane][i0]), a_nxt;
        float r_cur[4], r_nxt[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r_cur[e] = R[i0 + e][dcol];
        v16f_a p = mfma_prod(a_cur[0], r_cur[0]);
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            if (g + 1 < 8) {
                a_nxt = *reinterpret_cast<const vf4*>(&T[lane][i0 + 4 * (g + 1)]);
#pragma unroll
                for (int e = 0; e < 4; ++e) r_nxt[e] = R[i0 + 4 * (g + 1) + e][dcol];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int st = 4 * g + e;
                if (st + 1 < 32) n = e < 3 ? mfma_prod(a_cur[e + 1], r_cur[e + 1]) : mfma_prod(a_nxt[0], r_nxt[0]);
                if (st == 0) acc = p;
                else acc = acc + p;
                KV_STEP(acc);
                p = n;
            }
            a_cur = a_nxt;
#pragma unroll
            for (int e = 0; e < 4; ++e) r_cur[e] = r_nxt[e];
        }
        if (bb == 0) first = acc;
    }
    const v16f_a u = first + acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) fx[r] += (int64_t)__builtin_rint((double)u[r] * 0x1p40);
}

// 64 rows of Q and dO (query head h) from row `row0` on, row-major into qr
// and gr; zeros for rows past `rows`
__device__ __forceinline__ void kv_load_qg(const float* Q, int64_t ldq, const float* dO, int64_t ldo, int64_t row0,
                                           int64_t rows, int64_t h, float (*qr)[kKvRow], float (*gr)[kKvRow]) {
    for (int e = threadIdx.x; e < kAQ * (kAD / 4); e += kKvThreads) {
        const int row = e / (kAD / 4), d4 = (e % (kAD / 4)) * 4;
        vf4 q = {0.0f, 0.0f, 0.0f, 0.0f}, g = q;
        if (row < rows) {
            q = *reinterpret_cast<const vf4*>(Q + (row0 + row) * ldq + h * kAD + d4);
            g = *reinterpret_cast<const vf4*>(dO + (row0 + row) * ldo + h * kAD + d4);
        }
        *reinterpret_cast<vf4*>(&qr[row][d4]) = q;
        *reinterpret_cast<vf4*>(&gr[row][d4]) = g;
    }
}

// 64 rows of K and of q_v (KV head hk) from row `row0` on, key-major into kr
// and vq; zeros (and q_v = 0) for rows past `rows`
__device__ __forceinline__ void kv_load_kv(const float* K, int64_t ldk, const float* V, int64_t ldv, int64_t row0,
                                           int64_t rows, int64_t hk, const Quantizer& qz, float (*kr)[kKvRow],
                                           int8_t (*vq)[kKvRowQ]) {
    for (int e = threadIdx.x; e < kAK * (kAD / 4); e += kKvThreads) {
        const int row = e / (kAD / 4), d4 = (e % (kAD / 4)) * 4;
        vf4 k = {0.0f, 0.0f, 0.0f, 0.0f}, v = k;
        if (row < rows) {
            k = *reinterpret_cast<const vf4*>(K + (row0 + row) * ldk + hk * kAD + d4);
            v = *reinterpret_cast<const vf4*>(V + (row0 + row) * ldv + hk * kAD + d4);
        }
        *reinterpret_cast<vf4*>(&kr[row][d4]) = k;
        // the exact fast path, with the exact quotient where a lane is unsure
        unsigned q4 = 0;
        bool unsure = false;
#pragma unroll
        for (int u = 0; u < 4; ++u) q4 |= (unsigned)(uint8_t)(int8_t)qz.q_fast(v[u], &unsure) << (8 * u);
        if (__ballot(unsure)) {
            q4 = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                bool in;
                q4 |= (unsigned)(uint8_t)(int8_t)qz.q(v[u], &in) << (8 * u);
            }
        }
        *reinterpret_cast<unsigned*>(&vq[row][d4]) = row < rows ? q4 : 0u;
    }
}

// (m_i, l_i) from the forward's statistics and Delta_i = CanonSum_d(dO * O)
// for 64 rows from `row0` on (query head h): four lanes per row hold the
// d-blocks, then the pair tree through two lane swaps; rows past `rows` get
// (0, 1, 0).  Threads 0 .. 255 (four whole waves) take part.
__device__ __forceinline__ void kv_row_stats(const float* dO, const float* O, int64_t ldo, const float* stats,
                                             int64_t Hq, int64_t row0, int64_t rows, int64_t h, float* rowm,
                                             float* rowl, float* rowdelta) {
    const int tid = threadIdx.x;
    if (tid >= 4 * kAQ) return;
    const int row = tid >> 2, blk = tid & 3;
    float x = 0.0f;
    if (row < rows) {
        const float* go = dO + (row0 + row) * ldo + h * kAD + 32 * blk;
        const float* o = O + (row0 + row) * ldo + h * kAD + 32 * blk;
        x = f_mul(go[0], o[0]);
        for (int d = 1; d < 32; ++d) x = f_add(x, f_mul(go[d], o[d]));
    }
    x = f_add(x, __shfl_xor(x, 1));
    x = f_add(x, __shfl_xor(x, 2));
    if (blk == 0) {
        float m = 0.0f, l = 1.0f;
        if (row < rows) {
            const int64_t r = (row0 + row) * Hq + h;
            m = stats[2 * r];
            l = stats[2 * r + 1];
        }
        rowm[row] = m;
        rowl[row] = l;
        rowdelta[row] = row < rows ? x : 0.0f;
    }
}

template <bool KEEP>
__global__ __launch_bounds__(kKvThreads) void attn_bwd_dkdv_kernel(AttnKvArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    AttnKvSmem& sm = *reinterpret_cast<AttnKvSmem*>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    // key tiles slowest, so that the longest walks (first tiles, causal) start first
    const unsigned nbh = (unsigned)(a.B * a.Hkv), hkv = (unsigned)a.Hkv;
    const unsigned kt = blockIdx.x / nbh;
    const unsigned bh = blockIdx.x % nbh;
    const int64_t hk = bh % hkv;
    const int64_t b = bh / hkv;
    const int64_t group = (unsigned)a.Hq / hkv;
    const int64_t j0 = (int64_t)kt * kAK;
    const int64_t krows = a.S - j0 < kAK ? a.S - j0 : kAK;
    const int64_t base = b * a.S;
    const int64_t ihi_all = a.window > 0 ? (j0 + krows - 1 + a.window - 1 < a.S - 1 ? j0 + krows - 1 + a.window - 1
                                                                                   : a.S - 1)
                                         : a.S - 1;
    const int64_t qt0 = j0 / kAQ, qt1 = ihi_all / kAQ;
    const int s32 = (int)a.S;
    const int win = (a.window <= 0 || a.window >= a.S) ? 0 : (int)a.window;   // 0: no window

    // K rows and q_v rows of the key tile (zeros past S)
    const Quantizer qz(a.s_v);
    kv_load_kv(a.K, a.ldk, a.V, a.ldv, base + j0, krows, hk, qz, sm.kr, sm.vq);

    // wave roles: phase 1 (logits or dP, key slab), phase 2 (d slab)
    const int p1_dp = w >> 2, p1_slab = w & 3;
    const int jcol = 16 * p1_slab + (lane & 15);
    const int dcol = 16 * w + (lane & 15);
    int64_t fv[16], fk[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) fv[r] = fk[r] = 0;

    for (int64_t h = hk * group; h < (hk + 1) * group; ++h) {
        for (int64_t qt = qt0; qt <= qt1; ++qt) {
            const int64_t i0 = qt * kAQ;
            const int64_t qrows = a.S - i0 < kAQ ? a.S - i0 : kAQ;
            __syncthreads();
            kv_load_qg(a.Q, a.ldq, a.dO, a.ldo, base + i0, qrows, h, sm.qr, sm.gr);
            kv_row_stats(a.dO, a.O, a.ldo, a.stats, a.Hq, base + i0, qrows, h, sm.rowm, sm.rowl, sm.rowdelta);
            __syncthreads();
            // phase 1: logits and dP of the 64 x 64 tile, stored key-major.
            // With kept logits, dP only: wave w forms the d-blocks of half
            // w / 4 for its key slab, the halves go to dt and pt and are added
            // in the pass below, (b0 + b1) + (b2 + b3) as kv_phase1 adds them.
            {
                v16f_a part;
                if constexpr (KEEP)
                    part = kv_phase1_pair<true>(&sm.gr[lane][0], nullptr, &sm.vq[jcol][0], a.s_v, 64 * p1_dp);
                else
                    part = p1_dp ? kv_phase1<true>(&sm.gr[lane][0], nullptr, &sm.vq[jcol][0], a.s_v)
                                 : kv_phase1<false>(&sm.qr[lane][0], &sm.kr[jcol][0], nullptr, a.s_v);
                float (*T)[kKvRowT] = (p1_dp != 0) == KEEP ? sm.pt : sm.dt;
#pragma unroll
                for (int beta = 0; beta < 4; ++beta)
                    *reinterpret_cast<vf4*>(&T[jcol][16 * beta + 4 * (lane >> 4)]) =
                        vf4{part[4 * beta], part[4 * beta + 1], part[4 * beta + 2], part[4 * beta + 3]};
            }
            __syncthreads();
            // the kept logits of this (query block, head) item's tile: items
            // in the forward's order, tiles from the block's first key tile
            const float* kept = nullptr;
            if constexpr (KEEP) {
                int64_t kq0, kq1;
                attn_tile_range(a.S, a.window, qt, &kq0, &kq1);
                const int64_t nqb = (a.S + kAQ - 1) / kAQ;
                const int64_t item = (nqb - 1 - qt) * (a.B * a.Hq) + b * a.Hq + h;
                kept = a.keep + item * a.keep_slot + ((int64_t)kt - kq0) * (kAQ * kAK);
            }
            // P and dS of the tile (32-bit positions: S < 2^31)
#pragma unroll
            for (int e = 0; e < (kAQ * kAK) / kKvThreads; ++e) {
                const int idx = tid + kKvThreads * e;
                const int jl = idx >> 6, il = idx & 63;
                const int i = (int)i0 + il, j = (int)j0 + jl;
                float P = 0.0f, dS = 0.0f;
                if (i < s32 && j <= i && (win == 0 || j > i - win)) {
                    const float sl = KEEP ? kept[il * kAK + jl] : f_mul(sm.pt[jl][il], a.c);
                    const float dP = KEEP ? f_add(sm.dt[jl][il], sm.pt[jl][il]) : sm.dt[jl][il];
                    const float p = own_exp(f_sub(sl, sm.rowm[il]), a.ek);
                    P = f_div(p, sm.rowl[il]);
                    dS = f_mul(P, f_sub(dP, sm.rowdelta[il]));
                }
                sm.pt[jl][il] = P;
                sm.dt[jl][il] = dS;
            }
            __syncthreads();
            // phase 2: tile sums of P x dO (dV) and dS x Q (dK)
            kv_phase2(sm.pt, sm.gr, lane, dcol, fv);
            kv_phase2(sm.dt, sm.qr, lane, dcol, fk);
        }
    }
    // lane l, register r: key 16*(r/4) + 4*(l/16) + r%4 of the tile, d = dcol
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int jl = 16 * (r >> 2) + 4 * (lane >> 4) + (r & 3);
        if (jl >= krows) continue;
        const int64_t row = base + j0 + jl;
        a.dK[row * a.ldg + hk * kAD + dcol] = f_mul(f_mul((float)fk[r], 0x1p-40f), a.c);
        const float v = a.V[row * a.ldv + hk * kAD + dcol];
        a.dV[row * a.ldg + hk * kAD + dcol] = qz.in_range(v) ? f_mul((float)fv[r], 0x1p-40f) : 0.0f;
    }
}

hipError_t launch_attn_bwd_dkdv(const float* Q, const float* K, const float* V, const float* O, const float* dO,
                                const float* stats, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t ldq,
                                int64_t ldk, int64_t ldv, int64_t ldo, int64_t window, float s_v, float* dK,
                                float* dV, int64_t ldg, const float* keep, const ExpConsts& ek, hipStream_t st) {
    if (B == 0 || S == 0) return hipSuccess;
    AttnKvArgs a;
    a.Q = Q; a.K = K; a.V = V; a.O = O; a.dO = dO; a.stats = stats; a.dK = dK; a.dV = dV;
    a.keep = keep;
    a.keep_slot = attn_fwd_max_tiles(S, window) * (kAQ * kAK);
    a.S = S; a.Hq = Hq; a.Hkv = Hkv; a.B = B;
    a.ldq = ldq; a.ldk = ldk; a.ldv = ldv; a.ldo = ldo; a.ldg = ldg; a.window = window;
    a.c = (float)(1.0 / (double)(float)sqrt((double)kAD));
    a.s_v = s_v;
    a.ek = ek;
    // the limit is set on every call: it is per device, and the call is cheap
    const void* fn = keep ? reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<true>)
                          : reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<false>);
    if (const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(AttnKvSmem));
        e != hipSuccess)
        return e;
    const int64_t blocks = B * Hkv * ceil_div(S, kAK);
    if (blocks > 0xffffffffLL) return hipErrorInvalidValue;
    if (keep)
        hipLaunchKernelGGL(attn_bwd_dkdv_kernel<true>, dim3((unsigned)blocks), dim3(kKvThreads), sizeof(AttnKvSmem),
                           st, a);
    else
        hipLaunchKernelGGL(attn_bwd_dkdv_kernel<false>, dim3((unsigned)blocks), dim3(kKvThreads), sizeof(AttnKvSmem),
                           st, a);
    return hipGetLastError();
}

// dQ on the same engine.  One workgroup (8 waves) per (batch, query head,
// block of 64 queries) keeps the Q and dO rows and walks the key tiles; per
// tile: phase 1 as for dK/dV (logits and dP of the 64 x 64 tile, stored
// row-major), dS elementwise, then each wave's tile sum over the 64 key
// positions of dS x K for d slab 16*w .. +15 into 16 int64 accumulators.
struct AttnDqSmem {
    float qr[kAQ][kKvRow];          // Q rows of the block
    float gr[kAQ][kKvRow];          // dO rows of the block
    float kr[kAK][kKvRow];          // K tile, key-major
    float st[kAQ][kKvRowT];         // logits of the tile (row-major)
    float dt[kAQ][kKvRowT];         // dP, then dS (row-major)
    int8_t vq[kAK][kKvRowQ];        // q_v tile, key-major
    float rowm[kAQ], rowl[kAQ], rowdelta[kAQ];
};
static_assert(sizeof(AttnDqSmem) <= 163840, "LDS of one CU");

template <bool KEEP>
__global__ __launch_bounds__(kKvThreads) void attn_bwd_dq_kernel(AttnBwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    AttnDqSmem& sm = *reinterpret_cast<AttnDqSmem*>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    // query blocks slowest and from the last, so that the longest walks
    // (last blocks, causal) start first
    const unsigned nqb = (unsigned)((a.S + kAQ - 1) / kAQ), hq = (unsigned)a.Hq;
    const unsigned nbh = (unsigned)(a.B * a.Hq);
    const unsigned qb = nqb - 1 - blockIdx.x / nbh;
    const unsigned bh = blockIdx.x % nbh;
    const int64_t h = bh % hq;
    const int64_t b = bh / hq;
    const int64_t hk = (unsigned)h / (hq / (unsigned)a.Hkv);
    const int64_t q0 = (int64_t)qb * kAQ;
    const int64_t qrows = a.S - q0 < kAQ ? a.S - q0 : kAQ;
    const int64_t base = b * a.S;
    const int64_t klo = a.window > 0 ? (q0 - a.window + 1 > 0 ? q0 - a.window + 1 : 0) : 0;
    const int64_t khi = q0 + qrows - 1;
    const int64_t kt0 = klo / kAK, kt1 = khi / kAK;
    const int s32 = (int)a.S;
    const int win = (a.window <= 0 || a.window >= a.S) ? 0 : (int)a.window;   // 0: no window

    kv_load_qg(a.Q, a.ldq, a.dO, a.ldo, base + q0, qrows, h, sm.qr, sm.gr);
    kv_row_stats(a.dO, a.O, a.ldo, a.stats, a.Hq, base + q0, qrows, h, sm.rowm, sm.rowl, sm.rowdelta);

    const Quantizer qz(a.s_v);
    const int p1_dp = w >> 2, p1_slab = w & 3;
    const int jcol = 16 * p1_slab + (lane & 15);
    const int dcol = 16 * w + (lane & 15);
    int64_t fx[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) fx[r] = 0;

    for (int64_t kt = kt0; kt <= kt1; ++kt) {
        const int64_t j0 = kt * kAK;
        const int64_t krows = a.S - j0 < kAK ? a.S - j0 : kAK;
        __syncthreads();
        kv_load_kv(a.K, a.ldk, a.V, a.ldv, base + j0, krows, hk, qz, sm.kr, sm.vq);
        __syncthreads();
        // phase 1: logits and dP of the 64 x 64 tile, stored row-major.
        // With kept logits, dP only: wave w forms the d-blocks of half w / 4
        // for its key slab, the halves go to dt and st and are added in the
        // dS pass, (b0 + b1) + (b2 + b3) as kv_phase1 adds them.
        {
            v16f_a part;
            if constexpr (KEEP)
                part = kv_phase1_pair<true>(&sm.gr[lane][0], nullptr, &sm.vq[jcol][0], a.s_v, 64 * p1_dp);
            else
                part = p1_dp ? kv_phase1<true>(&sm.gr[lane][0], nullptr, &sm.vq[jcol][0], a.s_v)
                             : kv_phase1<false>(&sm.qr[lane][0], &sm.kr[jcol][0], nullptr, a.s_v);
            float (*T)[kKvRowT] = (p1_dp != 0) == KEEP ? sm.st : sm.dt;
#pragma unroll
            for (int r = 0; r < 16; ++r) T[16 * (r >> 2) + 4 * (lane >> 4) + (r & 3)][jcol] = part[r];
        }
        __syncthreads();
        // the kept logits of this item's tile (this grid's order is the
        // forward's item order; tiles from the block's first key tile)
        const float* kept = KEEP ? a.keep + (int64_t)blockIdx.x * a.keep_slot + (kt - kt0) * (kAQ * kAK) : nullptr;
        // dS of the tile (32-bit positions: S < 2^31)
#pragma unroll
        for (int e = 0; e < (kAQ * kAK) / kKvThreads; ++e) {
            const int idx = tid + kKvThreads * e;
            const int il = idx >> 6, jl = idx & 63;
            const int i = (int)q0 + il, j = (int)j0 + jl;
            float dS = 0.0f;
            if (i < s32 && j <= i && (win == 0 || j > i - win)) {
                const float sl = KEEP ? kept[il * kAK + jl] : f_mul(sm.st[il][jl], a.c);
                const float dP = KEEP ? f_add(sm.dt[il][jl], sm.st[il][jl]) : sm.dt[il][jl];
                const float p = own_exp(f_sub(sl, sm.rowm[il]), a.ek);
                dS = f_mul(f_div(p, sm.rowl[il]), f_sub(dP, sm.rowdelta[il]));
            }
            sm.dt[il][jl] = dS;
        }
        __syncthreads();
        // phase 2: tile sums of dS x K
        kv_phase2(sm.dt, sm.kr, lane, dcol, fx);
    }
    // dQ = (fl(acc) * 2^-40) * c; lane l, register r: row 16*(r/4) + 4*(l/16) + r%4
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int il = 16 * (r >> 2) + 4 * (lane >> 4) + (r & 3);
        if (il >= qrows) continue;
        a.dQ[(base + q0 + il) * a.ldo + h * kAD + dcol] = f_mul(f_mul((float)fx[r], 0x1p-40f), a.c);
    }
}

hipError_t launch_attn_bwd_dq(const float* Q, const float* K, const float* V, const float* O, const float* dO,
                              const float* stats, int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t ldq,
                              int64_t ldk, int64_t ldv, int64_t ldo, int64_t window, float s_v, float* dQ,
                              const float* keep, const ExpConsts& ek, hipStream_t st) {
    if (B == 0 || S == 0) return hipSuccess;
    AttnBwdArgs a;
    a.Q = Q; a.K = K; a.V = V; a.O = O; a.dO = dO; a.stats = stats; a.dQ = dQ;
    a.keep = keep;
    a.keep_slot = attn_fwd_max_tiles(S, window) * (kAQ * kAK);
    a.S = S; a.Hq = Hq; a.Hkv = Hkv; a.B = B;
    a.ldq = ldq; a.ldk = ldk; a.ldv = ldv; a.ldo = ldo; a.window = window;
    a.c = (float)(1.0 / (double)(float)sqrt((double)kAD));
    a.s_v = s_v;
    a.ek = ek;
    // the limit is set on every call: it is per device, and the call is cheap
    const void* fn = keep ? reinterpret_cast<const void*>(&attn_bwd_dq_kernel<true>)
                          : reinterpret_cast<const void*>(&attn_bwd_dq_kernel<false>);
    if (const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(AttnDqSmem));
        e != hipSuccess)
        return e;
    const int64_t blocks = B * Hq * ceil_div(S, kAQ);
    if (blocks > 0xffffffffLL) return hipErrorInvalidValue;
    if (keep)
        hipLaunchKernelGGL(attn_bwd_dq_kernel<true>, dim3((unsigned)blocks), dim3(kKvThreads), sizeof(AttnDqSmem), st,
                           a);
    else
        hipLaunchKernelGGL(attn_bwd_dq_kernel<false>, dim3((unsigned)blocks), dim3(kKvThreads), sizeof(AttnDqSmem), st,
                           a);
    return hipGetLastError();
}

}  // namespace brl
