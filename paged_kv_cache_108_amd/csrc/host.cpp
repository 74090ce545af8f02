// Host side of libpkv: error reporting, the block allocator, the block-table
// and slot builders, and the tail-waste arithmetic. CPU only; no HIP calls.
//
// The allocator follows the pages' statement of the problem:
//  * a fixed pool of equal blocks, all allocated at start, handed out from a
//    plain free list ("PagedAttention" daily term, "Pros"; "03 ·
//    PagedAttention", "Blocks and block tables");
//  * a block is taken only when the sequence's previous block is full
//    (same section: the 17th token takes a block, 18-32 take none);
//  * forks share blocks by reference count and a write into a shared,
//    partially filled block copies it first ("03 · PagedAttention", "Sharing:
//    copy-on-write"; daily term, copy-on-write figure);
//  * running out of blocks is reported, not handled: preemption is the
//    scheduler's decision ("03 · PagedAttention", "When the pool runs dry").
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "common.h"

namespace pkv {

static thread_local std::string g_last_error;

pkv_status fail(pkv_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

pkv_status ok() {
    g_last_error.clear();
    return PKV_OK;
}

}  // namespace pkv

using pkv::fail;
using pkv::ok;

extern "C" const char* pkv_last_error(void) { return pkv::g_last_error.c_str(); }
extern "C" const char* pkv_version(void) { return "pkv 0.1.0 (gfx950)"; }

// ----------------------------------------------------------------------------
// SHA-256, written from FIPS 180-4 (sections 4.1.2, 4.2.2, 5.1.1, 6.2). The
// round constants and the initial hash value are the first 32 bits of the
// fractional parts of the cube roots of the first 64 primes and of the square
// roots of the first 8 primes; they are computed here rather than tabulated.
// ----------------------------------------------------------------------------
namespace {

struct Sha256Consts {
    uint32_t k[64];
    uint32_t h0[8];
    Sha256Consts() {
        int primes[64], n = 0;
        for (int c = 2; n < 64; ++c) {
            bool prime = true;
            for (int d = 2; d * d <= c; ++d)
                if (c % d == 0) { prime = false; break; }
            if (prime) primes[n++] = c;
        }
        for (int i = 0; i < 64; ++i) k[i] = frac32(std::cbrt((long double)primes[i]), primes[i], 3);
        for (int i = 0; i < 8; ++i) h0[i] = frac32(std::sqrt((long double)primes[i]), primes[i], 2);
    }
    // first 32 fraction bits of the real root r of x^e = p; the long double
    // estimate is corrected to the exact integer answer with integer arithmetic
    static uint32_t frac32(long double r, int p, int e) {
        unsigned __int128 v = (unsigned __int128)(r * 4294967296.0L);       // root * 2^32, approx.
        auto pw = [&](unsigned __int128 x) {                                // x^e vs p * 2^(32e)
            unsigned __int128 y = 1;
            for (int t = 0; t < e; ++t) y *= x;
            return y;
        };
        const unsigned __int128 target = (unsigned __int128)p << (32 * e);
        while (pw(v + 1) <= target) ++v;
        while (pw(v) > target) --v;                                         // v = floor(root * 2^32)
        return (uint32_t)(v & 0xFFFFFFFFu);
    }
};
const Sha256Consts& sha_consts() {
    static const Sha256Consts c;
    return c;
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

struct Sha256 {
    uint32_t h[8];
    uint8_t buf[64];
    size_t used = 0;
    uint64_t total = 0;
    Sha256() { std::memcpy(h, sha_consts().h0, sizeof h); }
    void block(const uint8_t* m) {
        const uint32_t* k = sha_consts().k;
        uint32_t w[64];
        for (int t = 0; t < 16; ++t)
            w[t] = (uint32_t)m[4 * t] << 24 | (uint32_t)m[4 * t + 1] << 16 | (uint32_t)m[4 * t + 2] << 8 | m[4 * t + 3];
        for (int t = 16; t < 64; ++t) {
            const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
            const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
            w[t] = w[t - 16] + s0 + w[t - 7] + s1;
        }
        uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
        for (int t = 0; t < 64; ++t) {
            const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
            const uint32_t ch = (e & f) ^ (~e & g);
            const uint32_t t1 = hh + S1 + ch + k[t] + w[t];
            const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
            const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
            const uint32_t t2 = S0 + maj;
            hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
        }
        h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
    }
    void update(const void* data, size_t n) {
        const uint8_t* p = static_cast<const uint8_t*>(data);
        total += n;
        while (n > 0) {
            const size_t take = std::min(n, (size_t)64 - used);
            std::memcpy(buf + used, p, take);
            used += take; p += take; n -= take;
            if (used == 64) { block(buf); used = 0; }
        }
    }
    void finish(uint8_t out[32]) {
        const uint64_t bits = total * 8;
        const uint8_t one = 0x80, zero = 0;
        update(&one, 1);
        while (used != 56) update(&zero, 1);
        uint8_t len[8];
        for (int i = 0; i < 8; ++i) len[i] = (uint8_t)(bits >> (56 - 8 * i));
        update(len, 8);
        for (int i = 0; i < 8; ++i)
            for (int j = 0; j < 4; ++j) out[4 * i + j] = (uint8_t)(h[i] >> (24 - 8 * j));
    }
};

struct Hash32 {
    uint8_t b[32];
    bool operator==(const Hash32& o) const { return std::memcmp(b, o.b, 32) == 0; }
};
struct Hash32Hasher {
    size_t operator()(const Hash32& h) const {
        size_t v;
        std::memcpy(&v, h.b, sizeof v);
        return v;
    }
};

// Hash of one full block: SHA-256 over the parent block's hash (32 zero bytes
// for the first block), the block's bs token ids as little-endian int32, and
// the caller's extra key bytes.
Hash32 block_hash(const Hash32& parent, const int32_t* tokens, int32_t bs, const uint8_t* extra,
                  int32_t extra_len) {
    Sha256 sh;
    sh.update(parent.b, 32);
    for (int32_t t = 0; t < bs; ++t) {
        const uint32_t u = (uint32_t)tokens[t];
        const uint8_t le[4] = {(uint8_t)u, (uint8_t)(u >> 8), (uint8_t)(u >> 16), (uint8_t)(u >> 24)};
        sh.update(le, 4);
    }
    if (extra_len > 0) sh.update(extra, (size_t)extra_len);
    Hash32 h;
    sh.finish(h.b);
    return h;
}

}  // namespace

struct pkv_allocator {
    struct Seq {
        std::vector<int32_t> blocks;   // logical block j -> physical block
        int64_t len = 0;               // tokens held
    };
    struct Entry {
        int32_t block;
        uint32_t stamp;                // live while it equals stamp[block] and the block is free
    };
    int32_t P = 0;
    int32_t bs = 0;
    std::vector<Entry> free_stack;     // back() is the next block handed out (stale entries skipped)
    std::vector<uint32_t> stamp;       // bumped on every push of the block
    std::vector<int32_t> ref;          // tables referencing each block (0: free)
    int32_t n_free = 0;
    std::unordered_map<int64_t, Seq> seqs;
    // prefix cache: hash of a full block -> block; a block keeps its hash while
    // it is in use and while it is free, until it is handed out again
    std::unordered_map<Hash32, int32_t, Hash32Hasher> cached;
    std::vector<Hash32> hash_of;
    std::vector<uint8_t> has_hash;
    int64_t hit_blocks = 0, miss_blocks = 0;

    void push(int32_t b) {
        free_stack.push_back(Entry{b, ++stamp[b]});
        ++n_free;
    }
    int32_t pop() {
        while (true) {
            const Entry e = free_stack.back();
            free_stack.pop_back();
            if (ref[e.block] == 0 && e.stamp == stamp[e.block]) {
                const int32_t b = e.block;
                ref[b] = 1;
                --n_free;
                forget(b);             // its contents are about to change
                return b;
            }
        }
    }
    void forget(int32_t b) {
        if (!has_hash[b]) return;
        auto it = cached.find(hash_of[b]);
        if (it != cached.end() && it->second == b) cached.erase(it);
        has_hash[b] = 0;
    }
    void remember(int32_t b, const Hash32& h) {
        auto it = cached.find(h);
        if (it != cached.end() && it->second != b) has_hash[it->second] = 0;
        cached[h] = b;
        hash_of[b] = h;
        has_hash[b] = 1;
    }
};

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

extern "C" pkv_status pkv_allocator_create(int32_t P, int32_t bs, pkv_allocator** out) {
    if (!out) return fail(PKV_E_INVALID, "allocator_create: out is NULL");
    if (P <= 0 || bs <= 0)
        return fail(PKV_E_INVALID, "allocator_create: P=%d and bs=%d must be positive", P, bs);
    auto* a = new pkv_allocator;
    a->P = P;
    a->bs = bs;
    a->stamp.assign(P, 0);
    a->ref.assign(P, 0);
    a->hash_of.resize(P);
    a->has_hash.assign(P, 0);
    a->free_stack.reserve(P);
    for (int32_t k = 0; k < P; ++k) a->push(P - 1 - k);   // first pop -> 0
    *out = a;
    return ok();
}

extern "C" void pkv_allocator_destroy(pkv_allocator* a) { delete a; }

extern "C" pkv_status pkv_seq_create(pkv_allocator* a, int64_t seq_id) {
    if (!a) return fail(PKV_E_INVALID, "seq_create: allocator is NULL");
    if (a->seqs.count(seq_id)) return fail(PKV_E_STATE, "seq_create: sequence %lld exists", (long long)seq_id);
    a->seqs.emplace(seq_id, pkv_allocator::Seq{});
    return ok();
}

extern "C" pkv_status pkv_seq_append(pkv_allocator* a, int64_t seq_id, int32_t n_tokens,
                                     int64_t* slots_out, int32_t* cow_src, int32_t* cow_dst,
                                     int32_t* n_cow) {
    if (!a) return fail(PKV_E_INVALID, "seq_append: allocator is NULL");
    if (n_tokens < 0) return fail(PKV_E_INVALID, "seq_append: n_tokens=%d < 0", n_tokens);
    if (n_tokens > 0 && !slots_out) return fail(PKV_E_INVALID, "seq_append: slots_out is NULL");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end()) return fail(PKV_E_NOT_FOUND, "seq_append: sequence %lld not found", (long long)seq_id);
    auto& s = it->second;
    const int64_t bs = a->bs;
    const bool cow = n_tokens > 0 && s.len % bs != 0 && a->ref[s.blocks.back()] > 1;
    if (cow && (!cow_src || !cow_dst || !n_cow))
        return fail(PKV_E_INVALID, "seq_append: copy-on-write needed but cow outputs are NULL");
    const int64_t need = ceil_div(s.len + n_tokens, bs) - ceil_div(s.len, bs) + (cow ? 1 : 0);
    if (need > (int64_t)a->n_free)
        return fail(PKV_E_NO_BLOCKS, "seq_append: need %lld blocks, %d free", (long long)need, a->n_free);
    if (n_cow) *n_cow = 0;
    if (cow) {
        int32_t src = s.blocks.back();
        int32_t dst = a->pop();
        a->ref[src] -= 1;
        s.blocks.back() = dst;
        *cow_src = src;
        *cow_dst = dst;
        *n_cow = 1;
    }
    for (int64_t k = 0; k < n_tokens; ++k) {
        int64_t p = s.len + k;
        size_t j = (size_t)(p / bs);
        if (j == s.blocks.size()) s.blocks.push_back(a->pop());
        slots_out[k] = (int64_t)s.blocks[j] * bs + p % bs;
    }
    s.len += n_tokens;
    return ok();
}

extern "C" pkv_status pkv_seq_fork(pkv_allocator* a, int64_t parent, int64_t child) {
    if (!a) return fail(PKV_E_INVALID, "seq_fork: allocator is NULL");
    auto it = a->seqs.find(parent);
    if (it == a->seqs.end()) return fail(PKV_E_NOT_FOUND, "seq_fork: parent %lld not found", (long long)parent);
    if (a->seqs.count(child)) return fail(PKV_E_STATE, "seq_fork: child %lld exists", (long long)child);
    pkv_allocator::Seq c = it->second;        // copy before emplace may rehash
    for (int32_t b : c.blocks) a->ref[b] += 1;
    a->seqs.emplace(child, std::move(c));
    return ok();
}

extern "C" pkv_status pkv_seq_free(pkv_allocator* a, int64_t seq_id) {
    if (!a) return fail(PKV_E_INVALID, "seq_free: allocator is NULL");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end()) return fail(PKV_E_NOT_FOUND, "seq_free: sequence %lld not found", (long long)seq_id);
    const auto& blocks = it->second.blocks;
    for (auto r = blocks.rbegin(); r != blocks.rend(); ++r)
        if (a->ref[*r] <= 0) return fail(PKV_E_STATE, "seq_free: block %d has refcount %d", *r, a->ref[*r]);
    for (auto r = blocks.rbegin(); r != blocks.rend(); ++r) {
        if (--a->ref[*r] == 0) a->push(*r);
    }
    a->seqs.erase(it);
    return ok();
}

extern "C" pkv_status pkv_seq_info(const pkv_allocator* a, int64_t seq_id, int64_t* length,
                                   int32_t* num_blocks) {
    if (!a) return fail(PKV_E_INVALID, "seq_info: allocator is NULL");
    auto it = a->seqs.find(seq_id);
    if (it == a->seqs.end()) return fail(PKV_E_NOT_FOUND, "seq_info: sequence %lld not found", (long long)seq_id);
    if (length) *length = it->second.len;
    if (num_blocks) *num_blocks = (int32_t)it->second.blocks.size();
    return ok();
}

extern "C" pkv_status pkv_build_block_tables(const pkv_allocator* a, const int64_t* seq_ids,
                                             int32_t S, int32_t max_blocks,
                                             int32_t* tables_out, int32_t* lens_out) {
    if (!a) return fail(PKV_E_INVALID, "build_block_tables: allocator is NULL");
    if (S < 0 || max_blocks <= 0) return fail(PKV_E_INVALID, "build_block_tables: S=%d max_blocks=%d", S, max_blocks);
    if (S > 0 && (!seq_ids || !tables_out || !lens_out))
        return fail(PKV_E_INVALID, "build_block_tables: NULL pointer");
    std::vector<const pkv_allocator::Seq*> rows(S);
    for (int32_t i = 0; i < S; ++i) {
        auto it = a->seqs.find(seq_ids[i]);
        if (it == a->seqs.end())
            return fail(PKV_E_NOT_FOUND, "build_block_tables: sequence %lld not found", (long long)seq_ids[i]);
        if ((int64_t)it->second.blocks.size() > max_blocks)
            return fail(PKV_E_INVALID, "build_block_tables: sequence %lld holds %zu blocks > max_blocks %d",
                        (long long)seq_ids[i], it->second.blocks.size(), max_blocks);
        if (it->second.len > INT32_MAX)
            return fail(PKV_E_INVALID, "build_block_tables: sequence %lld too long", (long long)seq_ids[i]);
        rows[i] = &it->second;
    }
    for (int32_t i = 0; i < S; ++i) {
        int32_t* row = tables_out + (size_t)i * max_blocks;
        const auto& b = rows[i]->blocks;
        std::copy(b.begin(), b.end(), row);
        std::fill(row + b.size(), row + max_blocks, -1);
        lens_out[i] = (int32_t)rows[i]->len;
    }
    return ok();
}

extern "C" pkv_status pkv_slots_from_tables(const int32_t* tables, const int32_t* positions,
                                            int32_t S, int32_t max_blocks, int32_t bs,
                                            int64_t* slots_out) {
    if (S < 0 || max_blocks <= 0 || bs <= 0)
        return fail(PKV_E_INVALID, "slots_from_tables: S=%d max_blocks=%d bs=%d", S, max_blocks, bs);
    if (S > 0 && (!tables || !positions || !slots_out))
        return fail(PKV_E_INVALID, "slots_from_tables: NULL pointer");
    for (int32_t i = 0; i < S; ++i) {
        int32_t p = positions[i];
        if (p < 0) continue;
        int32_t j = p / bs;
        if (j >= max_blocks)
            return fail(PKV_E_INVALID, "slots_from_tables: position %d of row %d beyond the table", p, i);
        if (tables[(size_t)i * max_blocks + j] < 0)
            return fail(PKV_E_INVALID, "slots_from_tables: row %d block %d unallocated", i, j);
    }
    for (int32_t i = 0; i < S; ++i) {
        int32_t p = positions[i];
        slots_out[i] = p < 0 ? -1 : (int64_t)tables[(size_t)i * max_blocks + p / bs] * bs + p % bs;
    }
    return ok();
}

extern "C" pkv_status pkv_shared_prefix_plan(const int32_t* tables, const int32_t* lens, int32_t S,
                                             int32_t max_blocks, int32_t group_size, int32_t bs,
                                             int32_t* prefix_tables, int32_t* prefix_lens,
                                             int32_t* suffix_tables, int32_t* suffix_lens) {
    if (S < 0 || max_blocks <= 0 || bs <= 0 || group_size < 1 || S % group_size != 0)
        return fail(PKV_E_INVALID, "shared_prefix_plan: S=%d max_blocks=%d bs=%d group_size=%d", S,
                    max_blocks, bs, group_size);
    if (S > 0 && (!tables || !lens || !prefix_tables || !prefix_lens || !suffix_tables || !suffix_lens))
        return fail(PKV_E_INVALID, "shared_prefix_plan: NULL pointer");
    for (int32_t i = 0; i < S; ++i)
        if ((int64_t)lens[i] > (int64_t)max_blocks * bs)
            return fail(PKV_E_INVALID, "shared_prefix_plan: length %d of row %d beyond the table", lens[i], i);
    const int32_t n_groups = S / group_size;
    for (int32_t g = 0; g < n_groups; ++g) {
        const int32_t first = g * group_size;
        // blocks before every member's last one, listed with the same id by all
        int32_t full = max_blocks;
        for (int32_t m = 0; m < group_size; ++m) {
            const int32_t L = lens[first + m];
            full = std::min(full, L > 0 ? (L - 1) / bs : 0);
        }
        int32_t k = 0;
        for (; k < full; ++k) {
            const int32_t id = tables[(size_t)first * max_blocks + k];
            bool same = id >= 0;
            for (int32_t m = 1; m < group_size && same; ++m)
                same = tables[(size_t)(first + m) * max_blocks + k] == id;
            if (!same) break;
        }
        int32_t* pre = prefix_tables + (size_t)g * max_blocks;
        for (int32_t j = 0; j < max_blocks; ++j) pre[j] = j < k ? tables[(size_t)first * max_blocks + j] : -1;
        prefix_lens[g] = k * bs;
        for (int32_t m = 0; m < group_size; ++m) {
            const int32_t i = first + m;
            const int32_t L = std::max(lens[i], 0);
            const int32_t nb = (L + bs - 1) / bs;
            int32_t* suf = suffix_tables + (size_t)i * max_blocks;
            for (int32_t j = 0; j < max_blocks; ++j)
                suf[j] = k + j < nb ? tables[(size_t)i * max_blocks + k + j] : -1;
            suffix_lens[i] = L - k * bs;
        }
    }
    return ok();
}

extern "C" pkv_status pkv_allocator_stats(const pkv_allocator* a, pkv_stats* out) {
    if (!a || !out) return fail(PKV_E_INVALID, "allocator_stats: NULL pointer");
    std::vector<int32_t> fill(a->P, 0);   // a shared block holds the same prefix in every table
    for (const auto& kv : a->seqs) {
        const auto& s = kv.second;
        for (size_t j = 0; j < s.blocks.size(); ++j) {
            int64_t f = std::min<int64_t>(a->bs, s.len - (int64_t)j * a->bs);
            fill[s.blocks[j]] = std::max<int32_t>(fill[s.blocks[j]], (int32_t)f);
        }
    }
    int64_t tokens = 0;
    for (int32_t f : fill) tokens += f;
    out->num_blocks = a->P;
    out->free_blocks = a->n_free;
    out->used_blocks = a->P - out->free_blocks;
    out->slots_allocated = (int64_t)out->used_blocks * a->bs;
    out->tokens_stored = tokens;
    out->waste = out->slots_allocated ? 1.0 - (double)tokens / (double)out->slots_allocated : 0.0;
    return ok();
}

extern "C" pkv_status pkv_waste_stats(const int32_t* lens, int32_t n, int32_t bs, int32_t max_len,
                                      int64_t* paged_slots, int64_t* naive_slots, int64_t* used,
                                      double* waste_paged, double* waste_naive) {
    if (n < 0 || bs <= 0 || max_len < 0)
        return fail(PKV_E_INVALID, "waste_stats: n=%d bs=%d max_len=%d", n, bs, max_len);
    if (n > 0 && !lens) return fail(PKV_E_INVALID, "waste_stats: lens is NULL");
    int64_t paged = 0, u = 0;
    for (int32_t i = 0; i < n; ++i) {
        int64_t L = std::max<int32_t>(lens[i], 0);
        paged += ceil_div(L, bs) * bs;
        u += L;
    }
    int64_t naive = (int64_t)n * max_len;
    if (paged_slots) *paged_slots = paged;
    if (naive_slots) *naive_slots = naive;
    if (used) *used = u;
    if (waste_paged) *waste_paged = paged ? 1.0 - (double)u / (double)paged : 0.0;
    if (waste_naive) *waste_naive = naive ? 1.0 - (double)u / (double)naive : 0.0;
    return ok();
}

// ----------------------------------------------------------------------------
// Prefix caching: a full block is named by the hash of its tokens and of the
// prefix before it, so a later request with the same prefix reuses the block
// ("PagedAttention" daily term, the prefix-caching paragraph after the
// copy-on-write figure; "Serving: vLLM and PagedAttention", section 2.6).
// ----------------------------------------------------------------------------

extern "C" pkv_status pkv_block_hashes(const int32_t* tokens, int32_t n_tokens, int32_t bs,
                                       const uint8_t* extra, int32_t extra_len, uint8_t* hashes_out) {
    if (n_tokens < 0 || bs <= 0 || extra_len < 0)
        return fail(PKV_E_INVALID, "block_hashes: n_tokens=%d bs=%d extra_len=%d", n_tokens, bs, extra_len);
    const int32_t m = n_tokens / bs;
    if ((m > 0 && (!tokens || !hashes_out)) || (extra_len > 0 && !extra))
        return fail(PKV_E_INVALID, "block_hashes: NULL pointer");
    Hash32 h{};
    for (int32_t k = 0; k < m; ++k) {
        h = block_hash(h, tokens + (size_t)k * bs, bs, extra, extra_len);
        std::memcpy(hashes_out + 32 * (size_t)k, h.b, 32);
    }
    return ok();
}

extern "C" pkv_status pkv_seq_create_prefixed(pkv_allocator* a, int64_t seq_id, const int32_t* tokens,
                                              int32_t n_tokens, const uint8_t* extra, int32_t extra_len,
                                              int64_t* slots_out, int32_t* n_cached_out) {
    if (!a) return fail(PKV_E_INVALID, "seq_create_prefixed: allocator is NULL");
    if (n_tokens < 0 || extra_len < 0)
        return fail(PKV_E_INVALID, "seq_create_prefixed: n_tokens=%d extra_len=%d", n_tokens, extra_len);
    if ((n_tokens > 0 && (!tokens || !slots_out)) || (extra_len > 0 && !extra) || !n_cached_out)
        return fail(PKV_E_INVALID, "seq_create_prefixed: NULL pointer");
    if (a->seqs.count(seq_id)) return fail(PKV_E_STATE, "seq_create_prefixed: sequence %lld exists", (long long)seq_id);
    const int32_t bs = a->bs;
    const int32_t m = n_tokens / bs;                       // full blocks
    std::vector<Hash32> hs(m);
    Hash32 h{};
    for (int32_t k = 0; k < m; ++k) hs[k] = h = block_hash(h, tokens + (size_t)k * bs, bs, extra, extra_len);
    // the longest run of leading blocks whose hashes are cached
    int32_t hit = 0;
    std::vector<int32_t> hit_ids;
    while (hit < m) {
        auto it = a->cached.find(hs[hit]);
        if (it == a->cached.end()) break;
        hit_ids.push_back(it->second);
        ++hit;
    }
    int64_t revive = 0;
    for (int32_t b : hit_ids) revive += a->ref[b] == 0;
    const int64_t fresh = ceil_div(n_tokens, bs) - hit;
    if (revive + fresh > a->n_free)
        return fail(PKV_E_NO_BLOCKS, "seq_create_prefixed: need %lld blocks, %d free",
                    (long long)(revive + fresh), a->n_free);
    pkv_allocator::Seq s;
    for (int32_t b : hit_ids) {                         // shared, or taken back from the free list
        if (a->ref[b] == 0) --a->n_free;                // its stack entry goes stale
        a->ref[b] += 1;
        s.blocks.push_back(b);
    }
    for (int64_t j = hit; j < ceil_div(n_tokens, bs); ++j) {
        const int32_t b = a->pop();
        if (j < m) a->remember(b, hs[j]);
        s.blocks.push_back(b);
    }
    for (int32_t p = 0; p < n_tokens; ++p) slots_out[p] = (int64_t)s.blocks[p / bs] * bs + p % bs;
    s.len = n_tokens;
    a->seqs.emplace(seq_id, std::move(s));
    a->hit_blocks += hit;
    a->miss_blocks += m - hit;
    *n_cached_out = hit * bs;
    return ok();
}

extern "C" pkv_status pkv_prefix_cache_stats(const pkv_allocator* a, int64_t* hit_blocks,
                                             int64_t* miss_blocks, int32_t* cached_blocks) {
    if (!a) return fail(PKV_E_INVALID, "prefix_cache_stats: allocator is NULL");
    if (hit_blocks) *hit_blocks = a->hit_blocks;
    if (miss_blocks) *miss_blocks = a->miss_blocks;
    if (cached_blocks) *cached_blocks = (int32_t)a->cached.size();
    return ok();
}
