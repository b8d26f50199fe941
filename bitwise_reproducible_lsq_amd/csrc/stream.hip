// stream.hip -- the topology-invariant data stream and counter-based draws.
//
// Open-1B summary on onedev.kr: section "How" (random values as pure
// functions of the seed and a fixed logical position, Philox, so the stream
// does not depend on tensor sizes, lane splits or the device) and section
// "What differs" (one canonical data stream independent of world size and
// rank; source interleaving from a mix generator seeded by the training seed
// alone; shard order seeded by (seed, SHA-256 of the source name, epoch);
// document order seeded by (seed, SHA-256 of the source name, epoch, shard);
// documents joined with a separator into a flat buffer cut into 4,097-token
// windows; rank r of R owns windows m with m mod R = r; a rank-independent
// resume record).  This library's reading of the open steps:
//   draw(key, stream, i) = word i mod 4 of Philox4x32-10 with counter
//     (i div 4 as two words, stream, 0) and the 64-bit key;
//   bounded(x, n) = (x * n) >> 32;
//   orders: Fisher-Yates from the top, draw t swapping position n-1-t with
//     bounded(draw(key, 0, t), n-t);
//   keys: first 8 bytes (little endian) of SHA-256("shard" | le64 seed |
//     SHA-256(name) | le64 epoch), and of SHA-256("doc" | ... | le64 shard);
//   mixing: draw t of (seed, "mix") picks the source whose cumulative
//     weight first exceeds bounded(draw, total weight);
//   a source's epoch advances when its next document is requested after
//     its last shard is done.
// Host code: the stream itself is sequential integer bookkeeping over the
// caller's corpus.  Device code: bulk draws (philox_u32_kernel).
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "internal.hpp"

namespace brl {

// ---- Philox4x32-10 ----------------------------------------------------------------
constexpr uint32_t kPhM0 = 0xD2511F53u, kPhM1 = 0xCD9E8D57u;
constexpr uint32_t kPhW0 = 0x9E3779B9u, kPhW1 = 0xBB67AE85u;

__host__ __device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)kPhM0 * c[0];
        const uint64_t p1 = (uint64_t)kPhM1 * c[2];
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = (uint32_t)p1;
        c[2] = n2;
        c[3] = (uint32_t)p0;
        k0 += kPhW0;
        k1 += kPhW1;
    }
}

static uint32_t draw_host(uint64_t key, uint32_t stream, uint64_t i) {
    const uint64_t blk = i >> 2;
    uint32_t c[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), stream, 0u};
    philox4x32_10(c, (uint32_t)key, (uint32_t)(key >> 32));
    return c[i & 3];
}

// out[k] = draw(key, stream, first + k): one lane per 4-word block
__global__ __launch_bounds__(256) void philox_u32_kernel(uint64_t key, uint32_t stream, uint64_t first, int64_t n,
                                                         uint32_t* __restrict__ out) {
    const uint64_t b0 = first >> 2;
    const uint64_t blk = b0 + (uint64_t)blockIdx.x * 256 + threadIdx.x;
    const uint64_t pos0 = blk << 2;
    if (pos0 >= first + (uint64_t)n) return;
    uint32_t c[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), stream, 0u};
    philox4x32_10(c, (uint32_t)key, (uint32_t)(key >> 32));
    if (pos0 >= first && pos0 + 4 <= first + (uint64_t)n && ((pos0 - first) & 3) == 0 &&
        (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
        *reinterpret_cast<uint4*>(out + (pos0 - first)) = uint4{c[0], c[1], c[2], c[3]};
        return;
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint64_t pos = pos0 + w;
        if (pos >= first && pos < first + (uint64_t)n) out[pos - first] = c[w];
    }
}

hipError_t launch_philox_u32(uint64_t key, uint32_t stream, uint64_t first, int64_t n, uint32_t* out,
                             hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const uint64_t blocks = ((first + (uint64_t)n + 3) >> 2) - (first >> 2);
    const uint64_t grid = (blocks + 255) / 256;
    if (grid > 0xffffffffull) return hipErrorInvalidValue;
    hipLaunchKernelGGL(philox_u32_kernel, dim3((unsigned)grid), dim3(256), 0, st, key, stream, first, n, out);
    return hipGetLastError();
}

// ---- host SHA-256 (for source names and key derivation) -----------------------------
static void sha256_host(const uint8_t* msg, size_t n, uint8_t out[32]) {
    struct Tables { uint32_t K[64], H0[8]; };
    static const Tables tab = [] { Tables t; sha256_constants(t.K, t.H0); return t; }();   // thread-safe init
    const uint32_t* K = tab.K;
    const uint32_t* H0 = tab.H0;
    auto rotr = [](uint32_t x, int r) { return (x >> r) | (x << (32 - r)); };
    uint32_t h[8];
    memcpy(h, H0, sizeof(h));
    std::vector<uint8_t> m(msg, msg + n);
    m.push_back(0x80);
    while (m.size() % 64 != 56) m.push_back(0);
    const uint64_t bits = (uint64_t)n * 8;
    for (int i = 7; i >= 0; --i) m.push_back((uint8_t)(bits >> (8 * i)));
    for (size_t off = 0; off < m.size(); off += 64) {
        uint32_t w[64];
        for (int t = 0; t < 16; ++t)
            w[t] = (uint32_t)m[off + 4 * t] << 24 | (uint32_t)m[off + 4 * t + 1] << 16 |
                   (uint32_t)m[off + 4 * t + 2] << 8 | m[off + 4 * t + 3];
        for (int t = 16; t < 64; ++t) {
            const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
            const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
            w[t] = w[t - 16] + s0 + w[t - 7] + s1;
        }
        uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
        for (int t = 0; t < 64; ++t) {
            const uint32_t t1 = hh + (rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25)) + ((e & f) ^ (~e & g)) + K[t] + w[t];
            const uint32_t t2 = (rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22)) + ((a & b) ^ (a & c) ^ (b & c));
            hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
        }
        h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
    }
    for (int i = 0; i < 8; ++i)
        for (int j = 0; j < 4; ++j) out[4 * i + j] = (uint8_t)(h[i] >> (24 - 8 * j));
}

static void put_le64(std::vector<uint8_t>& v, uint64_t x) {
    for (int i = 0; i < 8; ++i) v.push_back((uint8_t)(x >> (8 * i)));
}

static uint64_t key_from(const char* tag, uint64_t seed, const uint8_t digest[32], uint64_t epoch, bool with_shard,
                         uint64_t shard) {
    std::vector<uint8_t> m(tag, tag + strlen(tag));
    put_le64(m, seed);
    m.insert(m.end(), digest, digest + 32);
    put_le64(m, epoch);
    if (with_shard) put_le64(m, shard);
    uint8_t h[32];
    sha256_host(m.data(), m.size(), h);
    uint64_t k = 0;
    for (int i = 7; i >= 0; --i) k = k << 8 | h[i];
    return k;
}

static void fisher_yates(uint64_t key, int64_t n, std::vector<int64_t>& p) {
    p.resize((size_t)n);
    for (int64_t i = 0; i < n; ++i) p[(size_t)i] = i;
    for (int64_t t = 0; t + 1 < n; ++t) {
        const int64_t k = n - 1 - t;
        const int64_t j = (int64_t)(((uint64_t)draw_host(key, 0, (uint64_t)t) * (uint64_t)(k + 1)) >> 32);
        std::swap(p[(size_t)k], p[(size_t)j]);
    }
}

}  // namespace brl

// ---- the stream object (C ABI) --------------------------------------------------------
struct brl_stream {
    struct Src {
        std::string name;
        uint8_t digest[32];
        int64_t weight;
        std::vector<int64_t> shard_docs, shard_first;   // documents per shard, first document index
        const int64_t* doc_offsets;
        const int32_t* tokens;
        // state
        uint64_t epoch = 0, shard_pos = 0, doc_pos = 0, consumed = 0;
        // cached orders
        uint64_t shard_order_epoch = ~0ull;
        std::vector<int64_t> shard_order;
        uint64_t doc_order_epoch = ~0ull, doc_order_shard = ~0ull;
        std::vector<int64_t> doc_order;
    };
    uint64_t seed;
    int32_t sep;
    std::vector<Src> src;
    std::vector<int64_t> cum;
    int64_t total = 0;
    uint64_t window = 0, mix_draws = 0;
    std::vector<int32_t> buf;
    size_t head = 0;
};

namespace brl {

static const uint32_t kMixStream = 0x6D6978u;   // "mix"

static int pick_source(brl_stream* s) {
    const uint64_t r = ((uint64_t)draw_host(s->seed, kMixStream, s->mix_draws) * (uint64_t)s->total) >> 32;
    ++s->mix_draws;
    for (size_t k = 0; k < s->cum.size(); ++k)
        if ((int64_t)r < s->cum[k]) return (int)k;
    return (int)s->cum.size() - 1;   // unreachable for a positive total
}

// the next document of source k: [first, last) token offsets
static void next_document(brl_stream* s, int k, int64_t* first, int64_t* last) {
    brl_stream::Src& c = s->src[(size_t)k];
    const int64_t n_shards = (int64_t)c.shard_docs.size();
    for (;;) {
        if (c.shard_pos == (uint64_t)n_shards) {
            ++c.epoch;
            c.shard_pos = 0;
        }
        if (c.shard_order_epoch != c.epoch) {
            fisher_yates(key_from("shard", s->seed, c.digest, c.epoch, false, 0), n_shards, c.shard_order);
            c.shard_order_epoch = c.epoch;
        }
        const int64_t shard = c.shard_order[(size_t)c.shard_pos];
        const int64_t nd = c.shard_docs[(size_t)shard];
        if ((int64_t)c.doc_pos < nd) {
            if (c.doc_order_epoch != c.epoch || c.doc_order_shard != (uint64_t)shard) {
                fisher_yates(key_from("doc", s->seed, c.digest, c.epoch, true, (uint64_t)shard), nd, c.doc_order);
                c.doc_order_epoch = c.epoch;
                c.doc_order_shard = (uint64_t)shard;
            }
            const int64_t doc = c.shard_first[(size_t)shard] + c.doc_order[(size_t)c.doc_pos];
            ++c.doc_pos;
            ++c.consumed;
            if ((int64_t)c.doc_pos == nd) {
                c.doc_pos = 0;
                ++c.shard_pos;
            }
            *first = c.doc_offsets[doc];
            *last = c.doc_offsets[doc + 1];
            return;
        }
        c.doc_pos = 0;
        ++c.shard_pos;
    }
}

static void next_window(brl_stream* s, int32_t* out) {
    while (s->buf.size() - s->head < (size_t)BRL_STREAM_WINDOW) {
        const int k = pick_source(s);
        int64_t a, b;
        next_document(s, k, &a, &b);
        const int32_t* t = s->src[(size_t)k].tokens;
        s->buf.insert(s->buf.end(), t + a, t + b);
        s->buf.push_back(s->sep);
    }
    if (out) memcpy(out, s->buf.data() + s->head, sizeof(int32_t) * BRL_STREAM_WINDOW);
    s->head += BRL_STREAM_WINDOW;
    if (s->head > (1u << 20)) {
        s->buf.erase(s->buf.begin(), s->buf.begin() + (std::ptrdiff_t)s->head);
        s->head = 0;
    }
    ++s->window;
}

}  // namespace brl

// ---- C ABI --------------------------------------------------------------------------
using namespace brl;

extern "C" {

brl_status brl_stream_create(uint64_t seed, int32_t separator, const brl_stream_source* sources,
                             int32_t n_sources, brl_stream** out) {
    if (!out) return report_error(BRL_EINVAL, "brl_stream_create: null out");
    *out = nullptr;
    if (n_sources <= 0 || !sources) return report_error(BRL_EINVAL, "brl_stream_create: no sources");
    brl_stream* s = new brl_stream();
    s->seed = seed;
    s->sep = separator;
    int64_t total = 0;
    for (int32_t k = 0; k < n_sources; ++k) {
        const brl_stream_source& in = sources[k];
        if (!in.name || in.weight < 0 || in.n_shards <= 0 || !in.shard_docs || !in.doc_offsets ||
            (!in.tokens && in.doc_offsets[0] != 0)) {
            delete s;
            return report_error(BRL_EINVAL, "brl_stream_create: bad source description");
        }
        brl_stream::Src c;
        c.name = in.name;
        sha256_host(reinterpret_cast<const uint8_t*>(in.name), strlen(in.name), c.digest);
        c.weight = in.weight;
        int64_t first = 0;
        for (int32_t j = 0; j < in.n_shards; ++j) {
            if (in.shard_docs[j] < 0) {
                delete s;
                return report_error(BRL_EINVAL, "brl_stream_create: negative document count");
            }
            c.shard_first.push_back(first);
            c.shard_docs.push_back(in.shard_docs[j]);
            first += in.shard_docs[j];
        }
        for (int64_t d = 0; d < first; ++d)
            if (in.doc_offsets[d + 1] < in.doc_offsets[d]) {
                delete s;
                return report_error(BRL_EINVAL, "brl_stream_create: token offsets must ascend");
            }
        if (in.weight > 0 && in.doc_offsets[first] == in.doc_offsets[0] && first == 0) {
            delete s;
            return report_error(BRL_EINVAL, "brl_stream_create: a weighted source has no documents");
        }
        c.doc_offsets = in.doc_offsets;
        c.tokens = in.tokens;
        total += in.weight;
        s->cum.push_back(total);
        s->src.push_back(std::move(c));
    }
    if (total <= 0 || total > 0xffffffffLL) {
        delete s;
        return report_error(BRL_EINVAL, "brl_stream_create: total weight must be in [1, 2^32)");
    }
    s->total = total;
    *out = s;
    return BRL_OK;
}

void brl_stream_destroy(brl_stream* s) { delete s; }

brl_status brl_stream_next(brl_stream* s, int64_t count, int32_t* out, int64_t* first_window) {
    if (!s || count < 0 || (count > 0 && !out)) return report_error(BRL_EINVAL, "brl_stream_next: bad arguments");
    if (first_window) *first_window = (int64_t)s->window;
    for (int64_t k = 0; k < count; ++k) next_window(s, out + k * BRL_STREAM_WINDOW);
    return BRL_OK;
}

brl_status brl_stream_step(brl_stream* s, int64_t global_batch, int32_t ranks, int32_t rank, int32_t* out) {
    if (!s || ranks <= 0 || rank < 0 || rank >= ranks || global_batch < 0)
        return report_error(BRL_EINVAL, "brl_stream_step: bad arguments");
    if (global_batch % ranks) return report_error(BRL_ESHAPE, "brl_stream_step: global batch not a multiple of ranks");
    if (global_batch > 0 && !out) return report_error(BRL_EINVAL, "brl_stream_step: null out");
    int64_t j = 0;
    for (int64_t k = 0; k < global_batch; ++k) {
        const bool mine = (int64_t)(s->window % (uint64_t)ranks) == rank;
        next_window(s, mine ? out + (j++) * BRL_STREAM_WINDOW : nullptr);
    }
    return BRL_OK;
}

int64_t brl_stream_record_bytes(const brl_stream* s) {
    if (!s) return -1;
    return 8 + 8 + 4 + 4 + 8 + 8 + (int64_t)s->src.size() * (32 + 32) + 8 +
           4 * (int64_t)(s->buf.size() - s->head);
}

brl_status brl_stream_save(const brl_stream* s, uint8_t* buf, int64_t cap) {
    if (!s || !buf) return report_error(BRL_EINVAL, "brl_stream_save: null argument");
    if (cap < brl_stream_record_bytes(s)) return report_error(BRL_EWORKSPACE, "brl_stream_save: buffer too small");
    std::vector<uint8_t> v;
    const char* magic = "BRLSTRM1";
    v.insert(v.end(), magic, magic + 8);
    put_le64(v, s->seed);
    for (int i = 0; i < 4; ++i) v.push_back((uint8_t)((uint32_t)s->src.size() >> (8 * i)));
    for (int i = 0; i < 4; ++i) v.push_back((uint8_t)((uint32_t)s->sep >> (8 * i)));
    put_le64(v, s->window);
    put_le64(v, s->mix_draws);
    for (const auto& c : s->src) {
        v.insert(v.end(), c.digest, c.digest + 32);
        put_le64(v, c.epoch);
        put_le64(v, c.shard_pos);
        put_le64(v, c.doc_pos);
        put_le64(v, c.consumed);
    }
    const size_t nb = s->buf.size() - s->head;
    put_le64(v, nb);
    for (size_t i = 0; i < nb; ++i)
        for (int b = 0; b < 4; ++b) v.push_back((uint8_t)((uint32_t)s->buf[s->head + i] >> (8 * b)));
    memcpy(buf, v.data(), v.size());
    return BRL_OK;
}

static uint64_t get_le(const uint8_t* p, int bytes) {
    uint64_t x = 0;
    for (int i = bytes - 1; i >= 0; --i) x = x << 8 | p[i];
    return x;
}

brl_status brl_stream_load(brl_stream* s, const uint8_t* buf, int64_t n) {
    if (!s || !buf) return report_error(BRL_EINVAL, "brl_stream_load: null argument");
    const int64_t fixed = 8 + 8 + 4 + 4 + 8 + 8 + (int64_t)s->src.size() * 64 + 8;
    if (n < fixed || memcmp(buf, "BRLSTRM1", 8) != 0) return report_error(BRL_EINVAL, "brl_stream_load: not a record");
    const uint8_t* p = buf + 8;
    if (get_le(p, 8) != s->seed || get_le(p + 8, 4) != s->src.size() || (int32_t)get_le(p + 12, 4) != s->sep)
        return report_error(BRL_EINVAL, "brl_stream_load: record of another stream (seed, sources or separator)");
    p += 16;
    const uint64_t window = get_le(p, 8), mix = get_le(p + 8, 8);
    p += 16;
    for (const auto& c : s->src) {
        if (memcmp(p, c.digest, 32) != 0) return report_error(BRL_EINVAL, "brl_stream_load: source names differ");
        const uint64_t shard_pos = get_le(p + 40, 8), doc_pos = get_le(p + 48, 8);
        if (shard_pos > c.shard_docs.size()) return report_error(BRL_EINVAL, "brl_stream_load: bad shard position");
        (void)doc_pos;
        p += 64;
    }
    const uint64_t nb = get_le(p, 8);
    p += 8;
    if (nb > (uint64_t)(n - fixed) / 4 || n < fixed + 4 * (int64_t)nb)
        return report_error(BRL_EINVAL, "brl_stream_load: bad buffer length");
    s->window = window;
    s->mix_draws = mix;
    const uint8_t* q = buf + 8 + 16 + 16;
    for (auto& c : s->src) {
        c.epoch = get_le(q + 32, 8);
        c.shard_pos = get_le(q + 40, 8);
        c.doc_pos = get_le(q + 48, 8);
        c.consumed = get_le(q + 56, 8);
        c.shard_order_epoch = c.doc_order_epoch = c.doc_order_shard = ~0ull;
        q += 64;
    }
    s->buf.assign((size_t)nb, 0);
    s->head = 0;
    for (uint64_t i = 0; i < nb; ++i) s->buf[(size_t)i] = (int32_t)(uint32_t)get_le(p + 4 * i, 4);
    return BRL_OK;
}

brl_status brl_philox_u32(uint64_t key, uint32_t stream, uint64_t first, int64_t n, uint32_t* out, void* hip_stream) {
    if (n < 0) return report_error(BRL_ESHAPE, "brl_philox_u32: n < 0");
    if (n > 0 && (!out || (reinterpret_cast<uintptr_t>(out) & 3)))
        return report_error(BRL_EINVAL, "brl_philox_u32: null or unaligned out");
    if (first + (uint64_t)n < first) return report_error(BRL_ESHAPE, "brl_philox_u32: position range overflows");
    return report_hip(launch_philox_u32(key, stream, first, n, out, static_cast<hipStream_t>(hip_stream)),
                      "philox draws");
}

}  // extern "C"
