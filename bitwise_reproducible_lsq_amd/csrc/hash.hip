// hash.hip -- on-device state hash: SHA-256 (FIPS 180-4) arranged as a tree.
//
// The pages store a hash of the training state after every step, require a
// replayed step to reproduce it, and name moving the host-side hashing (about
// 6 s per step) onto the device as the way to remove its cost (onedev.kr
// summary, sections "Use" and "Limits"; rit.work article body).  They do not
// name the function.  This library's reading, chosen so that every lane of
// the GPU can hash its own piece:
//
//   leaves  each tensor's bytes cut into 4 KiB pieces (last one shorter, an
//           empty tensor one empty piece): SHA-256(piece || 0x00)
//   nodes   consecutive groups of 16 digests (512 bytes): SHA-256(group || 0x01),
//           level after level until one digest remains
//
// Small leaves spread a state over many lanes (a lane's hash is one long
// dependency chain, so lanes, not bytes per lane, give the throughput), and
// a small fan-in keeps the upper levels, which have few lanes, short.
//   root    SHA-256(top || le64(count) || le64(length of each tensor) || 0x02)
//
// One lane hashes one leaf or one node; the root is one lane.  SHA-256's
// round constants and initial value are the first 32 fractional bits of the
// cube and square roots of the first primes; the host derives them exactly
// (integer roots) and passes them in as kernel arguments.
#include "internal.hpp"

namespace brl {

struct ShaConsts {
    uint32_t k[64];
    uint32_t h0[8];
};

__device__ __forceinline__ uint32_t rotr(uint32_t x, int n) { return __builtin_amdgcn_alignbit(x, x, n); }
// three-input XOR in one v_bitop3_b32 (truth table 0x96)
__device__ __forceinline__ uint32_t xor3(uint32_t x, uint32_t y, uint32_t z) {
    return __builtin_amdgcn_bitop3_b32(x, y, z, 0x96);
}

// One 64-byte block (16 big-endian words) into the state.
__device__ __forceinline__ void sha_block(uint32_t (&h)[8], uint32_t (&w)[16], const ShaConsts& c) {
    uint32_t a = h[0], b = h[1], cc = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
#pragma unroll
    for (int t = 0; t < 64; ++t) {
        uint32_t wt;
        if (t < 16) {
            wt = w[t];
        } else {
            const uint32_t w15 = w[(t + 1) & 15], w2 = w[(t + 14) & 15];
            const uint32_t s0 = xor3(rotr(w15, 7), rotr(w15, 18), w15 >> 3);
            const uint32_t s1 = xor3(rotr(w2, 17), rotr(w2, 19), w2 >> 10);
            wt = w[t & 15] + s0 + w[(t + 9) & 15] + s1;
            w[t & 15] = wt;
        }
        const uint32_t S1 = xor3(rotr(e, 6), rotr(e, 11), rotr(e, 25));
        const uint32_t ch = (e & f) ^ (~e & g);
        const uint32_t t1 = hh + S1 + ch + c.k[t] + wt;
        const uint32_t S0 = xor3(rotr(a, 2), rotr(a, 13), rotr(a, 22));
        const uint32_t maj = (a & b) ^ (a & cc) ^ (b & cc);
        const uint32_t t2 = S0 + maj;
        hh = g; g = f; f = e; e = d + t1; d = cc; cc = b; b = a; a = t1 + t2;
    }
    h[0] += a; h[1] += b; h[2] += cc; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
}

__device__ __forceinline__ uint32_t bswap(uint32_t x) { return __builtin_bswap32(x); }

// SHA-256 of (bytes[0..n) || tag) where bytes live in global memory, written
// as 32 big-endian bytes to out.  Whole 64-byte blocks load as 16-byte
// vectors when VEC (16-byte aligned source); the tail byte by byte.
template <bool VEC>
__device__ void sha_piece(const uint8_t* __restrict__ src, int64_t n, uint8_t tag, const ShaConsts& c,
                          uint8_t* __restrict__ out) {
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = c.h0[i];
    uint32_t w[16];
    const int64_t full = n >> 6;
    if constexpr (VEC) {
        // the next block's 64 bytes load while this one is compressed
        uint4 nxt[4];
        if (full > 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) nxt[q] = reinterpret_cast<const uint4*>(src)[q];
        }
        for (int64_t blk = 0; blk < full; ++blk) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                w[4 * q + 0] = bswap(nxt[q].x); w[4 * q + 1] = bswap(nxt[q].y);
                w[4 * q + 2] = bswap(nxt[q].z); w[4 * q + 3] = bswap(nxt[q].w);
            }
            if (blk + 1 < full) {
                const uint4* p = reinterpret_cast<const uint4*>(src + ((blk + 1) << 6));
#pragma unroll
                for (int q = 0; q < 4; ++q) nxt[q] = p[q];
            }
            sha_block(h, w, c);
        }
    } else {
        for (int64_t blk = 0; blk < full; ++blk) {
            const uint8_t* p = src + (blk << 6);
#pragma unroll
            for (int q = 0; q < 16; ++q) w[q] = bswap(reinterpret_cast<const uint32_t*>(p)[q]);
            sha_block(h, w, c);
        }
    }
    // tail: rem message bytes, the tag, 0x80, zeros, 64-bit big-endian bit length
    const int rem = (int)(n & 63);
    const uint64_t bits = (uint64_t)(n + 1) * 8;
    const int nblk = (rem + 1 + 1 + 8 > 64) ? 2 : 1;
    const uint8_t* p = src + (full << 6);
    for (int b = 0; b < nblk; ++b) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int pos = b * 64 + 4 * q + e;       // byte position in the tail blocks
                uint32_t byte;
                if (pos < rem) byte = p[pos];
                else if (pos == rem) byte = tag;
                else if (pos == rem + 1) byte = 0x80;
                else if (pos >= nblk * 64 - 8) byte = (uint32_t)(bits >> (8 * (nblk * 64 - 1 - pos))) & 0xFF;
                else byte = 0;
                word = (word << 8) | byte;
            }
            w[q] = word;
        }
        sha_block(h, w, c);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) reinterpret_cast<uint32_t*>(out)[i] = bswap(h[i]);
}

// ---- leaves -------------------------------------------------------------------------
struct LeafRef {
    const uint8_t* src;
    int64_t n;
};

__device__ __forceinline__ LeafRef leaf_ref(const HashBatch& hb, int64_t g) {
    // the tensor holding leaf g: last t with first_leaf[t] <= g
    int t = 0;
    for (int s = 32; s > 0; s >>= 1)
        if (t + s < hb.n && hb.first_leaf[t + s] <= g) t += s;
    const int64_t off = (g - hb.first_leaf[t]) * kHashLeafBytes;
    const int64_t left = hb.len[t] - off;
    return {static_cast<const uint8_t*>(hb.ptr[t]) + off, left < kHashLeafBytes ? left : kHashLeafBytes};
}

// Lane -> leaf g of the batch.
template <bool VEC>
__global__ __launch_bounds__(256) void hash_leaf_kernel(HashBatch hb, ShaConsts c, uint8_t* __restrict__ digests,
                                                        int64_t* __restrict__ lens_out) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blockIdx.x == 0 && threadIdx.x < hb.n) lens_out[hb.first_tensor + threadIdx.x] = hb.len[threadIdx.x];
    if (g >= hb.leaves) return;
    const LeafRef l = leaf_ref(hb, g);
    sha_piece<VEC>(l.src, l.n, 0x00, c, digests + (hb.leaf_base + g) * 32);
}

// ---- one level of nodes: groups of kHashFanIn digests -------------------------------
__global__ __launch_bounds__(256) void hash_node_kernel(const uint8_t* __restrict__ in, int64_t n_in,
                                                        uint8_t* __restrict__ out, ShaConsts c) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t first = g * kHashFanIn;
    if (first >= n_in) return;
    const int64_t cnt = (n_in - first) < kHashFanIn ? (n_in - first) : kHashFanIn;
    sha_piece<true>(in + first * 32, cnt * 32, 0x01, c, out + g * 32);
}

// ---- root: SHA-256(top || le64(count) || le64(len_i)... || 0x02), one lane ----------
__global__ __launch_bounds__(64) void hash_root_kernel(const uint8_t* __restrict__ top,
                                                       const int64_t* __restrict__ lens, int64_t count,
                                                       ShaConsts c, uint8_t* __restrict__ out) {
    if (threadIdx.x != 0) return;
    // message bytes: [0,32) top, [32,40) count, [40, 40+8count) lengths, then 0x02
    const int64_t n = 32 + 8 + 8 * count;     // bytes before the tag
    auto byte_at = [&](int64_t pos) -> uint32_t {
        if (pos < 32) return top[pos];
        if (pos < 40) return (uint32_t)((uint64_t)count >> (8 * (pos - 32))) & 0xFF;
        const int64_t q = pos - 40;
        return (uint32_t)((uint64_t)lens[q >> 3] >> (8 * (q & 7))) & 0xFF;
    };
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = c.h0[i];
    uint32_t w[16];
    const uint64_t bits = (uint64_t)(n + 1) * 8;
    const int64_t total = ((n + 1 + 8) + 63) / 64 * 64;   // padded length
    for (int64_t base = 0; base < total; base += 64) {
        for (int q = 0; q < 16; ++q) {
            uint32_t word = 0;
            for (int e = 0; e < 4; ++e) {
                const int64_t pos = base + 4 * q + e;
                uint32_t byte;
                if (pos < n) byte = byte_at(pos);
                else if (pos == n) byte = 0x02;
                else if (pos == n + 1) byte = 0x80;
                else if (pos >= total - 8) byte = (uint32_t)(bits >> (8 * (total - 1 - pos))) & 0xFF;
                else byte = 0;
                word = (word << 8) | byte;
            }
            w[q] = word;
        }
        sha_block(h, w, c);
    }
    for (int i = 0; i < 8; ++i) reinterpret_cast<uint32_t*>(out)[i] = bswap(h[i]);
}

// ---- constants from their definition -------------------------------------------------
static uint64_t icbrt(unsigned __int128 x) {       // floor(cube root of x)
    uint64_t r = (uint64_t)cbrtl((long double)x);
    while ((unsigned __int128)r * r * r > x) --r;
    while ((unsigned __int128)(r + 1) * (r + 1) * (r + 1) <= x) ++r;
    return r;
}
static uint64_t isqrt(unsigned __int128 x) {       // floor(square root of x)
    uint64_t r = (uint64_t)sqrtl((long double)x);
    while ((unsigned __int128)r * r > x) --r;
    while ((unsigned __int128)(r + 1) * (r + 1) <= x) ++r;
    return r;
}

// Built once, on first use; a function-local static's initialisation is
// thread-safe, so concurrent first calls see the complete table.
static const ShaConsts& sha_consts() {
    static const ShaConsts c = [] {
        ShaConsts t{};
        int primes[64], np = 0;
        for (int v = 2; np < 64; ++v) {
            bool prime = true;
            for (int d = 2; d * d <= v; ++d)
                if (v % d == 0) { prime = false; break; }
            if (prime) primes[np++] = v;
        }
        for (int i = 0; i < 64; ++i)   // first 32 fractional bits of cbrt(p): floor(cbrt(p * 2^96)) mod 2^32
            t.k[i] = (uint32_t)icbrt((unsigned __int128)primes[i] << 96);
        for (int i = 0; i < 8; ++i)    // first 32 fractional bits of sqrt(p): floor(sqrt(p * 2^64)) mod 2^32
            t.h0[i] = (uint32_t)isqrt((unsigned __int128)primes[i] << 64);
        return t;
    }();
    return c;
}

void sha256_constants(uint32_t* k64, uint32_t* h8) {
    const ShaConsts& c = sha_consts();
    for (int i = 0; i < 64; ++i) k64[i] = c.k[i];
    for (int i = 0; i < 8; ++i) h8[i] = c.h0[i];
}

hipError_t launch_hash_leaves(const HashBatch& hb, bool vec, uint8_t* digests, int64_t* lens, hipStream_t st) {
    const ShaConsts& c = sha_consts();
    if (hb.leaves <= 0) return hipSuccess;
    const dim3 grid((unsigned)ceil_div(hb.leaves, 256));
    if (vec) hipLaunchKernelGGL(hash_leaf_kernel<true>, grid, dim3(256), 0, st, hb, c, digests, lens);
    else hipLaunchKernelGGL(hash_leaf_kernel<false>, grid, dim3(256), 0, st, hb, c, digests, lens);
    return hipGetLastError();
}

hipError_t launch_hash_nodes(const uint8_t* in, int64_t n_in, uint8_t* out, hipStream_t st) {
    const ShaConsts& c = sha_consts();
    const int64_t groups = ceil_div(n_in, (int64_t)kHashFanIn);
    hipLaunchKernelGGL(hash_node_kernel, dim3((unsigned)ceil_div(groups, 256)), dim3(256), 0, st, in, n_in, out, c);
    return hipGetLastError();
}

hipError_t launch_hash_root(const uint8_t* top, const int64_t* lens, int64_t count, uint8_t* out, hipStream_t st) {
    const ShaConsts& c = sha_consts();
    hipLaunchKernelGGL(hash_root_kernel, dim3(1), dim3(64), 0, st, top, lens, count, c, out);
    return hipGetLastError();
}

}  // namespace brl
