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

struct pkv_allocator {
    struct Seq {
        std::vector<int32_t> blocks;   // logical block j -> physical block
        int64_t len = 0;               // tokens held
    };
    int32_t P = 0;
    int32_t bs = 0;
    std::vector<int32_t> free_stack;   // back() is the next block handed out
    std::vector<int32_t> ref;          // tables referencing each block
    std::unordered_map<int64_t, Seq> seqs;

    int32_t pop() {
        int32_t b = free_stack.back();
        free_stack.pop_back();
        ref[b] = 1;
        return b;
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
    a->free_stack.resize(P);
    for (int32_t k = 0; k < P; ++k) a->free_stack[k] = P - 1 - k;   // first pop -> 0
    a->ref.assign(P, 0);
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
    if (need > (int64_t)a->free_stack.size())
        return fail(PKV_E_NO_BLOCKS, "seq_append: need %lld blocks, %zu free", (long long)need,
                    a->free_stack.size());
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
        if (--a->ref[*r] == 0) a->free_stack.push_back(*r);
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
    out->free_blocks = (int32_t)a->free_stack.size();
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
