// Host work plan for the planned decode step (pkv_build_paged_decode_plan):
// the balanced split of the decode attention work, computed on the CPU from
// the host copy of the context lengths, as step a0 builds the block tables
// and the slot mapping. The planned kernel reads each wave's chunk list and
// the merge descriptors from the plan instead of deriving them from the
// lengths on the device; the split is the same one (split.h), position for
// position, so with the same wave count the result is the unplanned kernel's,
// bit for bit (with another wave count the pieces differ and the result agrees
// within rounding).
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "common.h"
#include "split.h"

using pkv::fail;
using pkv::ok;
using namespace pkv_split;

namespace {

struct Entry {
    int32_t i, g, kc, L;
    int flags;
};

// One step's plan, or the number of int32 words it needs: decode (n_q = 0)
// or a window of n_q queries per sequence over G query heads per kv head.
pkv_status build_plan(const char* fn, const int32_t* lens, int32_t S, int32_t n_q, int32_t G, int32_t Hkv,
                      int32_t d, pkv_dtype cache_dtype, int32_t max_context_len, int32_t n_workers, int32_t* plan,
                      size_t plan_bytes, size_t* plan_bytes_needed) {
    if (S <= 0 || Hkv <= 0 || n_workers <= 0 || max_context_len < 0)
        return fail(PKV_E_INVALID, "%s: S=%d Hkv=%d n_workers=%d max_context_len=%d", fn, S, Hkv, n_workers,
                    max_context_len);
    if (!pkv::is_head_dim(d)) return fail(PKV_E_INVALID, "%s: d=%d not in {64,128}", fn, d);
    int kv;
    if (cache_dtype == PKV_F32) kv = kKvF32;
    else if (cache_dtype == PKV_BF16) kv = kKvBf16;
    else if (cache_dtype == PKV_FP8_E4M3) kv = kKvFp8;
    else return fail(PKV_E_INVALID, "%s: unsupported cache dtype %d", fn, cache_dtype);
    if (!lens) return fail(PKV_E_INVALID, "%s: NULL pointer", fn);
    if (n_workers > (1 << 20)) return fail(PKV_E_INVALID, "%s: n_workers=%d too large", fn, n_workers);
    // chunk counts are formed in 32-bit arithmetic (split.h)
    if (max_context_len > (1 << 30))
        return fail(PKV_E_INVALID, "%s: max_context_len=%d above 2^30", fn, max_context_len);
    const int cost = seg_cost(kv, d);
    // decode: one segment per (sequence, kv head); a window: n_qg per kv head
    // (one or two 16-column tiles each), the kv head's groups next to each other
    const QueryGroups qgr = n_q > 0 ? query_groups_in(n_q, G, window_plan_tiles(n_q, G)) : QueryGroups{1, 1, G};
    const int64_t HS64 = (int64_t)Hkv * qgr.n_qg;
    if (HS64 > 0xFFFF) return fail(PKV_E_INVALID, "%s: %lld segments per sequence", fn, (long long)HS64);
    const int32_t HS = (int32_t)HS64;

    // positions, sequence-major, as the kernel enumerates them
    std::vector<int32_t> L(S);
    uint64_t V64 = 0;
    for (int32_t i = 0; i < S; ++i) {
        L[i] = std::min(lens[i], max_context_len);
        V64 += (uint64_t)span_of(L[i], cost) * (uint64_t)HS;
    }
    if (V64 > 0x7FFFFFFFull) return fail(PKV_E_INVALID, "%s: too many work positions", fn);
    const unsigned V = (unsigned)V64;
    const unsigned W = V > 0 ? waves_used(V, (unsigned)n_workers) : 0u;

    // each wave's chunks, in order
    std::vector<std::vector<Entry>> waves(W);
    std::vector<int32_t> desc((size_t)S * HS * 2, 0);
    if (W > 0) {
        const Split split(V, W);
        unsigned pos = 0;
        for (int32_t i = 0; i < S; ++i) {
            const unsigned sp = span_of(L[i], cost);
            if (sp == 0) continue;
            const int nch = (L[i] + 15) >> 4;
            for (int32_t g = 0; g < HS; ++g) {
                // the segment's chunks sit at positions pos + cost .. pos + sp - 1
                const unsigned p0 = pos + (unsigned)cost;
                const unsigned w_lo = split.owner(p0), w_hi = split.owner(pos + sp - 1);
                for (int kc = 0; kc < nch; ++kc) {
                    const unsigned w = split.owner(p0 + (unsigned)kc);
                    waves[w].push_back(Entry{i, g, kc, L[i], 0});
                }
                // w_lo's record is 2 w_lo when the segment holds its first chunk
                const bool lo_first = split.start(w_lo) + (unsigned)cost >= p0;
                desc[((size_t)i * HS + g) * 2] = (int32_t)(2 * w_lo + (lo_first ? 0 : 1));
                desc[((size_t)i * HS + g) * 2 + 1] = (int32_t)(w_hi - w_lo + 1);
                pos += sp;
            }
        }
        // flags: pieces are runs of one segment inside a wave
        for (unsigned w = 0; w < W; ++w) {
            auto& e = waves[w];
            const size_t n = e.size();
            size_t a = 0;
            while (a < n) {
                size_t b = a;
                while (b + 1 < n && e[b + 1].i == e[a].i && e[b + 1].g == e[a].g) ++b;
                const int nch = (e[a].L + 15) >> 4;
                const bool whole = e[a].kc == 0 && e[b].kc == nch - 1;
                e[a].flags |= kFirst;
                e[b].flags |= kLast | (whole ? kWhole : 0);
                if (a != 0)
                    for (size_t k = a; k <= b; ++k) e[k].flags |= kOdd;
                a = b + 1;
            }
        }
    }
    size_t stride = 1;
    for (const auto& e : waves) stride = std::max(stride, e.size());
    const size_t words = (size_t)kPlanHeader + (size_t)n_workers * stride * 4 + desc.size();
    if (plan_bytes_needed) *plan_bytes_needed = words * sizeof(int32_t);
    if (!plan || plan_bytes < words * sizeof(int32_t))
        return fail(PKV_E_WORKSPACE, "%s: plan buffer %zu bytes, need %zu", fn, plan_bytes,
                    words * sizeof(int32_t));
    int32_t* h = plan;
    std::memset(h, 0, kPlanHeader * sizeof(int32_t));
    h[0] = kPlanMagic;
    h[1] = kPlanVersion;
    h[2] = n_workers;
    h[3] = (int32_t)W;
    h[4] = S;
    h[5] = Hkv;
    h[6] = cost;
    h[7] = (int32_t)stride;
    h[8] = max_context_len;
    h[9] = d;
    h[10] = kv;
    if (n_q > 0) {
        h[11] = n_q;
        h[12] = G;
        h[13] = qgr.qgs;
        h[14] = qgr.n_qg;
    }
    int32_t* ent = plan + kPlanHeader;
    for (size_t w = 0; w < (size_t)n_workers; ++w) {
        for (size_t k = 0; k < stride; ++k) {
            int32_t* x = ent + (w * stride + k) * 4;
            if (w < waves.size() && k < waves[w].size()) {
                const Entry& e = waves[w][k];
                x[0] = e.i;
                x[1] = e.g | (e.flags << 16);
                x[2] = e.kc;
                x[3] = e.L;
            } else {
                x[0] = -1;
                x[1] = 0;
                x[2] = 0;
                x[3] = 0;
            }
        }
    }
    std::memcpy(ent + (size_t)n_workers * stride * 4, desc.data(), desc.size() * sizeof(int32_t));
    return ok();
}

}  // namespace

extern "C" pkv_status pkv_build_paged_decode_plan(const int32_t* context_lens, int32_t S, int32_t Hkv, int32_t d,
                                                  pkv_dtype cache_dtype, int32_t max_context_len,
                                                  int32_t n_workers, void* plan, size_t plan_bytes,
                                                  size_t* plan_bytes_needed) {
    return build_plan("build_paged_decode_plan", context_lens, S, 0, 0, Hkv, d, cache_dtype, max_context_len,
                      n_workers, static_cast<int32_t*>(plan), plan_bytes, plan_bytes_needed);
}

extern "C" pkv_status pkv_build_paged_window_plan(const int32_t* context_lens, int32_t S, int32_t n_q, int32_t Hq,
                                                  int32_t Hkv, int32_t d, pkv_dtype cache_dtype,
                                                  int32_t max_context_len, int32_t n_workers, void* plan,
                                                  size_t plan_bytes, size_t* plan_bytes_needed) {
    const char* fn = "build_paged_window_plan";
    if (n_q <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Hq / Hkv > 16)
        return fail(PKV_E_INVALID, "%s: n_q=%d Hq=%d Hkv=%d (need n_q > 0 and 1 <= Hq/Hkv <= 16)", fn, n_q, Hq,
                    Hkv);
    return build_plan(fn, context_lens, S, n_q, Hq / Hkv, Hkv, d, cache_dtype, max_context_len, n_workers,
                      static_cast<int32_t*>(plan), plan_bytes, plan_bytes_needed);
}

extern "C" pkv_status pkv_plan_mark_shared_blocks(void* plan, size_t plan_bytes, const int32_t* block_tables,
                                                  const int32_t* context_lens, int32_t S, int32_t max_blocks,
                                                  int32_t bs, int32_t* shared) {
    const char* fn = "plan_mark_shared_blocks";
    if (!plan || !block_tables || !context_lens || S <= 0 || max_blocks <= 0 || bs <= 0)
        return fail(PKV_E_INVALID, "%s: NULL pointer or S=%d max_blocks=%d bs=%d", fn, S, max_blocks, bs);
    if (plan_bytes < kPlanHeader * sizeof(int32_t))
        return fail(PKV_E_INVALID, "%s: plan of %zu bytes", fn, plan_bytes);
    int32_t* h = static_cast<int32_t*>(plan);
    if (h[0] != kPlanMagic || h[1] != kPlanVersion || h[4] != S)
        return fail(PKV_E_INVALID, "%s: not a plan for S=%d", fn, S);
    // the blocks each sequence reads: ceil(L / bs) entries of its row
    const int32_t max_len = h[8];
    std::vector<int32_t> seen;
    seen.reserve(1024);
    for (int32_t i = 0; i < S; ++i) {
        const int64_t L = std::min(context_lens[i], max_len);
        const int32_t nb = L > 0 ? (int32_t)std::min<int64_t>((L + bs - 1) / bs, max_blocks) : 0;
        for (int32_t j = 0; j < nb; ++j) seen.push_back(block_tables[(size_t)i * max_blocks + j]);
    }
    std::sort(seen.begin(), seen.end());
    const bool dup = std::adjacent_find(seen.begin(), seen.end()) != seen.end();
    h[kPlanFlagsWord] = dup ? (h[kPlanFlagsWord] | kPlanSharedBlocks) : (h[kPlanFlagsWord] & ~kPlanSharedBlocks);
    if (shared) *shared = dup ? 1 : 0;
    return ok();
}
