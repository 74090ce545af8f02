// The balanced split of the decode attention work, shared by the device
// kernels (which compute it from the context lengths on the device) and the
// host plan builder (which computes the same split on the CPU, so that the
// planned kernel runs exactly the work of the unplanned one).
//
// Work positions run sequence-major, then kv head, then position inside the
// (sequence, kv head) segment. A segment of n 16-token chunks has
// seg_cost + n positions: the first seg_cost stand for the fixed cost of
// starting and finishing a segment (q load, epilogue, partly filled last
// chunk). V positions in all are cut into W
// near-equal contiguous ranges, one per wave, range w being
// [start(w), start(w + 1)) with the first V % W ranges one longer.
#pragma once

#include <cstdint>

#ifdef __HIPCC__
#define PKV_HD __host__ __device__
#else
#define PKV_HD
#endif

namespace pkv_split {

// Cache element kinds (the same numbering as the kernels' KvKind).
enum : int { kKvF32 = 0, kKvBf16 = 1, kKvFp8 = 2 };

#ifndef PKV_MIN_POS
#define PKV_MIN_POS 4
#endif
// Positions per wave, at least: a short input is cut into fewer, longer
// ranges, so that a merged row has fewer records.
constexpr unsigned kMinPositions = PKV_MIN_POS;

// Positions a segment costs beyond its chunks: its fixed work (the q rows,
// the epilogue and its record, the pipeline refill), which grows with d as
// the chunk does, weighs as much as streaming 128 * d bytes of K and V. That
// is 4 / (cache element bytes) chunks whatever d: 1 for fp32, 2 for bf16, 4
// for fp8 caches (measured: half or double these weights leave the waves of
// a call ending less evenly).
PKV_HD constexpr int seg_cost(int kv, int) { return kv == kKvF32 ? 1 : kv == kKvBf16 ? 2 : 4; }

// Positions of one (sequence, kv head) segment of L tokens.
PKV_HD inline unsigned span_of(int L, int cost) { return L > 0 ? (unsigned)cost + (unsigned)((L + 15) >> 4) : 0u; }

// Waves that get a range: all of them, unless the input is short.
PKV_HD inline unsigned waves_used(unsigned V, unsigned W_all) {
    const unsigned w = (V + kMinPositions - 1) / kMinPositions;
    return W_all < (w > 1u ? w : 1u) ? W_all : (w > 1u ? w : 1u);
}

// n positions cut into W ranges (32-bit: callers keep positions below 2^31).
struct Split {
    unsigned q, r;
    PKV_HD Split(unsigned n, unsigned W) : q(n / W), r(n % W) {}
    PKV_HD unsigned start(unsigned w) const { return w * q + (w < r ? w : r); }
    PKV_HD unsigned owner(unsigned c) const {
        const unsigned big = r * (q + 1);
        return c < big ? c / (q + 1) : r + (c - big) / q;
    }
};

// Query windows (n_q queries per sequence): the (query, head) pairs of one kv
// head are cut into n_qg groups of qgs queries, so that a group's cols =
// G * qgs columns fit `tiles` 16-column MFMA tiles; each group is a segment
// of its own, with the chunks of the whole sequence. Decode is n_q = 1: one
// group of G columns.
struct QueryGroups {
    int qgs, n_qg, cols;
};
PKV_HD inline QueryGroups query_groups_in(int n_q, int G, int tiles) {
    QueryGroups r;
    const int per = 16 * tiles / G;
    r.qgs = n_q < (per > 1 ? per : 1) ? n_q : (per > 1 ? per : 1);
    r.n_qg = (n_q + r.qgs - 1) / r.qgs;
    r.cols = G * r.qgs;
    return r;
}

// Tiles per query group of a window plan: one when the window's n_q * G
// columns fit one 16-column tile, else two (32 columns per group, as the
// unplanned window call takes per pass).
PKV_HD inline int window_plan_tiles(int n_q, int G) { return (long long)n_q * G <= 16 ? 1 : 2; }

// ---------------------------------------------------------------------------
// The work plan (pkv_build_paged_decode_plan, pkv_build_paged_window_plan;
// int32 words):
//   header[16]: kPlanMagic, kPlanVersion, n_workers (waves of the grid it was
//               built for), W (waves with a range), S, Hkv, seg_cost, stride
//               (entries per wave), max_context_len, d, kv kind, then for a
//               window plan n_q, G, qgs, n_qg (0 0 0 0 in a decode plan),
//               then flags (kPlanSharedBlocks)
//   entries[n_workers][stride][4]: wave w's chunks in processing order, each
//               {sequence i, segment column group g2 | flags << 16, chunk
//               index kc, L_i}, g2 = kv head * n_qg + query group (the kv
//               head in a decode plan); unused entries have i = -1
//   desc[S * Hkv * n_qg][2]: per segment (first record, record count) for
//               the merge (a count of 1 or less: processed whole)
// ---------------------------------------------------------------------------
constexpr int32_t kPlanMagic = 0x504B5650;   // "PKVP"
constexpr int32_t kPlanVersion = 1;
constexpr int kPlanHeader = 16;
constexpr int kPlanFlagsWord = 15;
// flags: some physical block is listed by more than one sequence (or twice
// in one), so the kernels read K/V with cacheable loads, and sequences that
// read the same block can meet in L2
constexpr int32_t kPlanSharedBlocks = 1;
// entry flags
constexpr int kFirst = 1;    // the first chunk of this wave's piece of the segment
constexpr int kLast = 2;     // the last chunk of this wave's piece
constexpr int kWhole = 4;    // the piece is the whole segment (rows are written directly)
constexpr int kOdd = 8;      // the piece's partial record is 2w + 1 (else 2w)

}  // namespace pkv_split
