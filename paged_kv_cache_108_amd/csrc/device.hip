// Device side of libpkv: the KV-cache write and paged decode attention for
// gfx950 (CDNA4), with their argument validation and launchers.
//
// Paged decode attention ("03 · PagedAttention", "The part the analogy hides:
// the kernel"; "PagedAttention" daily term, decode-step figure): for every
// (sequence, kv head) the kernel walks the block table, gathers each block's
// K and V tile and accumulates softmax(q K^T) V for the G query heads that share
// the kv head. The pages' own kernel targets other hardware; this one is built
// for wave64 + MFMA:
//
//  * The unit of work is a 16-token chunk of one (sequence, kv head): one MFMA
//    tile of scores S^T[16 tokens][16 columns] = K_chunk . Q^T (bf16 16x16x32,
//    or fp32 16x16x4 for an fp32 cache; fp8 codes are converted exactly to
//    bf16). Columns are the G query heads (padded to 16), or (query, head)
//    pairs for windows of several queries. The K operand rows are tokens, so a
//    lane's K fragment is consecutive channels of one token: 16-byte loads.
//  * The MFMA result layout is exactly the B operand of the P.V MFMA
//    (O^T[dims][columns] += V^T[dims][tokens] . P^T[tokens][columns]), so P
//    never leaves registers. V tiles are channel-major inside sub-tiles of
//    min(bs, 16) tokens, so the V^T operand is 4 consecutive tokens of one
//    channel and a chunk reads one whole sub-tile.
//  * P keeps float32 accuracy: for bf16/fp8 caches it is split into hi + lo
//    bf16 parts that one MFMA takes together (rounding P to bf16 alone costs
//    about 2e-3 relative error).
//  * Softmax max and sum across the 4 token groups of a column use gfx950's
//    v_permlane16_swap / v_permlane32_swap.
//  * Default split (paged_attn_stream_kernel, partition_size =
//    PKV_PARTITION_BALANCED): the chunks of all segments, plus a fixed cost per
//    segment, are cut into one equal contiguous range per wave, with one
//    4-wave workgroup per CU. Each wave streams its chunks through a two-stage
//    register pipeline with nontemporal loads; pieces of split segments write
//    partial records that paged_attn_merge_kernel combines in fixed order.
//    Instantiations: decode, query windows, and the decode step with the write
//    of the new tokens fused in.
//  * Fixed partitions (paged_attn_partition_kernel): partition p covers tokens
//    [p*part, (p+1)*part), items (sequence, kv head, partition) over a
//    persistent grid, merged by the same merge kernel.
//  * Shared prefixes: a window pass over a group's shared blocks and a decode
//    pass over each sequence's own blocks, combined exactly by log-sum-exp
//    (shared_prefix_merge_kernel, merge_states_kernel).
//  * No atomics anywhere: every split depends only on the lengths and every
//    record has a fixed slot, so results are bit-reproducible.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "attn_kernels.h"

using pkv::fail;
using pkv::ok;

namespace {

using namespace pkv_dev;

// ----------------------------------------------------------------------------
// Block copy (copy-on-write)
// ----------------------------------------------------------------------------

// blockIdx.x = pair, blockIdx.y = pool (0: K, 1: V); a block of one pool is
// one contiguous run of `bytes` (a multiple of 16) bytes.
__global__ void __launch_bounds__(256)
copy_blocks_kernel(char* __restrict__ k_cache, char* __restrict__ v_cache,
                   const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
                   int P, size_t bytes) {
    const int s = src[blockIdx.x];
    const int d = dst[blockIdx.x];
    if (s < 0 || s >= P || d < 0 || d >= P) return;
    char* pool = blockIdx.y == 0 ? k_cache : v_cache;
    const uint4* from = reinterpret_cast<const uint4*>(pool + (size_t)s * bytes);
    uint4* to = reinterpret_cast<uint4*>(pool + (size_t)d * bytes);
    const size_t n = bytes / 16;
    for (size_t e = threadIdx.x; e < n; e += blockDim.x) to[e] = from[e];
}

// ----------------------------------------------------------------------------
// KV-cache write
// ----------------------------------------------------------------------------

// One workgroup per new token; threads stride over its Hkv*d elements.
template <int SRC, int CACHE>
__global__ void __launch_bounds__(256)
kv_cache_write_kernel(const void* __restrict__ k_new, const void* __restrict__ v_new,
                      void* __restrict__ k_cache, void* __restrict__ v_cache,
                      const int64_t* __restrict__ slot_mapping,
                      int Hkv, int d, int bs, long long n_slots,
                      float k_inv, float v_inv) {
    const long long t = blockIdx.x;
    const long long slot = slot_mapping[t];
    if (slot < 0 || slot >= n_slots) return;
    const long long b = slot / bs;
    const int o = (int)(slot - b * bs);
    const int n = Hkv * d;
    for (int e = threadIdx.x; e < n; e += blockDim.x) {
        const int h = e / d;
        const int c = e - h * d;
        const size_t src = (size_t)t * n + e;
        const size_t kd = (((size_t)b * Hkv + h) * bs + o) * d + c;
        // V tile: [bs / vs][d][vs] with vs = min(bs, 16) tokens per sub-tile
        const int vs = bs < 16 ? bs : 16;
        const size_t vd = ((size_t)b * Hkv + h) * bs * d + (size_t)(o / vs) * vs * d + (size_t)c * vs + o % vs;
        if constexpr (CACHE == KV_F32) {
            static_cast<float*>(k_cache)[kd] = static_cast<const float*>(k_new)[src];
            static_cast<float*>(v_cache)[vd] = static_cast<const float*>(v_new)[src];
        } else if constexpr (CACHE == KV_BF16) {
            static_cast<uint16_t*>(k_cache)[kd] = static_cast<const uint16_t*>(k_new)[src];
            static_cast<uint16_t*>(v_cache)[vd] = static_cast<const uint16_t*>(v_new)[src];
        } else {
            float kx, vx;
            if constexpr (SRC == KV_BF16) {
                kx = bf16_bits_to_f32(static_cast<const uint16_t*>(k_new)[src]);
                vx = bf16_bits_to_f32(static_cast<const uint16_t*>(v_new)[src]);
            } else {
                kx = static_cast<const float*>(k_new)[src];
                vx = static_cast<const float*>(v_new)[src];
            }
            static_cast<uint8_t*>(k_cache)[kd] = (uint8_t)e4m3_encode(kx * k_inv);
            static_cast<uint8_t*>(v_cache)[vd] = (uint8_t)e4m3_encode(vx * v_inv);
        }
    }
}

// Merge partial records into output rows: one wave per (sequence, q head).
// Fixed partitions: a sequence with n > 1 partitions has records
// (i*Hkv + g)*n_part + p, p < n. Balanced: a segment split over waves
// w_lo..w_hi has record 2*w_lo + (1 if w_lo's range starts before the
// segment) and 2*w for the others; the attention kernel left the first record
// and the count in the segment's descriptor. Records are combined in that
// fixed order.
//
// Planned calls whose segments fit take the descriptors in the merge
// kernel's arguments instead (paged_attn_merge_args_kernel), packed first
// record | count << 13 (records are below 2 * kMaxWorkers = 8192, counts at
// most kMaxWorkers); a workgroup reads its segment's word with the other
// arguments at the start, so the records follow in one round trip. A segment
// with one record or none (an empty sequence) needs no merge, so the lengths
// are not read.
constexpr int kArgDescs = 768;
struct MergeArgDesc {
    uint32_t d[kArgDescs];
};

// Merge row h (column r of its segment) from its n records, the first rec0
// (balanced: then 2 * (w_lo + k) for k >= 1; partitions: rec0 + k). KB:
// records whose columns one round trip loads beyond the first eight (32, or
// 8 for a kernel that wants fewer registers and more resident waves); the
// records are summed in the same order either way.
template <int D, int KB = 32>
__device__ __forceinline__ void merge_records(const AttnParams& p, long long h, int r, int n, int rec0,
                                              bool balanced) {
    const int lane = threadIdx.x & 63;
    const long long w_lo = rec0 >> 1;
    // record k of this segment
    // record k of this segment; k past the last is read as the last one, so
    // loads the compiler issues ahead of their use stay inside this call's
    // records (their values are never used)
    auto rec_of = [&](int k) -> size_t {
        k = min(k, n - 1);
        if (balanced) return k == 0 ? (size_t)rec0 : (size_t)(2 * (w_lo + k));
        return (size_t)(rec0 + k);
    };
    const size_t nrec = (size_t)p.n_rec;
    const int G = p.cols;                     // record rows (columns)
    auto m_at = [&](int k) { return p.ws[nrec * G * D + rec_of(k) * G + r]; };
    auto l_at = [&](int k) { return p.ws[nrec * G * (D + 1) + rec_of(k) * G + r]; };
    constexpr int PER = D / 64;
    float num[PER] = {};
    float den = 0.f;
    if (n <= 8) {
        // up to 8 records: every load of the row is issued before any is used
        float mv[8], lv[8], ov[8][PER];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const bool in = k < n;
            mv[k] = in ? m_at(k) : -INFINITY;
            lv[k] = in ? l_at(k) : 0.f;
#pragma unroll
            for (int x = 0; x < PER; ++x)
                ov[k][x] = in ? p.ws[(rec_of(k) * G + r) * D + lane + 64 * x] : 0.f;
        }
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < 8; ++k) M = fmaxf(M, mv[k]);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (k < n) {
                const float wt = __builtin_amdgcn_exp2f(mv[k] - M);
                den += wt * lv[k];
#pragma unroll
                for (int x = 0; x < PER; ++x) num[x] += wt * ov[k][x];
            }
        }
#pragma unroll
        for (int x = 0; x < PER; ++x) p.out[h * D + lane + 64 * x] = num[x] / den;
        if (p.lse && lane == 0) p.lse[h] = M + __log2f(den);
        return;
    }
    if (n <= 32) {
        // up to 32 records, KB per round trip: lane k reads record k's m and
        // l, and every lane its PER adjacent columns of every record
        using VT = typename std::conditional<PER == 2, float2, float>::type;
        const float mk = lane < n ? m_at(lane) : -INFINITY;
        const float lk = lane < n ? l_at(lane) : 0.f;
        float M = mk;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
        const float wl = lane < n ? __builtin_amdgcn_exp2f(mk - M) : 0.f;
        float dn = wl * lk;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) dn += __shfl_xor(dn, off);
        float acc[PER] = {};
#pragma unroll
        for (int b0 = 0; b0 < 32; b0 += KB) {
            if (b0 >= n) break;
            VT ov[KB];
#pragma unroll
            for (int u0 = 0; u0 < KB; u0 += 8) {
                if (b0 + u0 < n) {            // whole groups of 8 past the last record are skipped
#pragma unroll
                    for (int u = u0; u < u0 + 8; ++u)
                        ov[u] = *reinterpret_cast<const VT*>(p.ws + (rec_of(b0 + u) * G + r) * D + PER * lane);
                } else {
#pragma unroll
                    for (int u = u0; u < u0 + 8; ++u) ov[u] = VT{};
                }
            }
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                if (b0 + u < n) {
                    const float wt = __shfl(wl, b0 + u);
                    if constexpr (PER == 2) {
                        acc[0] += wt * ov[u].x;
                        acc[1] += wt * ov[u].y;
                    } else {
                        acc[0] += wt * ov[u];
                    }
                }
            }
        }
        float* orow = p.out + h * D + PER * lane;
        if constexpr (PER == 2) *reinterpret_cast<float2*>(orow) = make_float2(acc[0] / dn, acc[1] / dn);
        else orow[0] = acc[0] / dn;
        if (p.lse && lane == 0) p.lse[h] = M + __log2f(dn);
        return;
    }
    float M = -INFINITY;
    for (int k0 = 0; k0 < n; k0 += 64)
        if (k0 + lane < n) M = fmaxf(M, m_at(k0 + lane));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    for (int k0 = 0; k0 < n; k0 += 64) {
        const int kn = min(64, n - k0);
        const float wl = k0 + lane < n ? __builtin_amdgcn_exp2f(m_at(k0 + lane) - M) : 0.f;
        den += wl * (k0 + lane < n ? l_at(k0 + lane) : 0.f);
        int k = 0;
        for (; k + KB <= kn; k += KB) {
            // long rows: KB records per memory round trip
            float ov[KB][PER];
#pragma unroll
            for (int u = 0; u < KB; ++u)
#pragma unroll
                for (int x = 0; x < PER; ++x)
                    ov[u][x] = p.ws[(rec_of(k0 + k + u) * G + r) * D + lane + 64 * x];
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                const float wt = __shfl(wl, (k + u) & 63);
#pragma unroll
                for (int x = 0; x < PER; ++x) num[x] += wt * ov[u][x];
            }
        }
        for (; k < kn; k += 8) {
            float ov[8][PER];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int x = 0; x < PER; ++x)
                    ov[u][x] = k + u < kn ? p.ws[(rec_of(k0 + k + u) * G + r) * D + lane + 64 * x] : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float wt = __shfl(wl, (k + u) & 63);
#pragma unroll
                for (int x = 0; x < PER; ++x) num[x] += wt * ov[u][x];
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
#pragma unroll
    for (int x = 0; x < PER; ++x) p.out[h * D + lane + 64 * x] = num[x] / den;
    if (p.lse && lane == 0) p.lse[h] = M + __log2f(den);
}

template <int D>
__global__ void __launch_bounds__(kThreads)
paged_attn_merge_kernel(AttnParams p) {
    const bool balanced = p.balanced != 0;

    // output row h = (i * n_q + j) * Hq + head
    const long long h = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (h >= (long long)p.S * p.n_q * p.Hq) return;
    const int i = (int)(h / ((long long)p.n_q * p.Hq));
    const int jh = (int)(h - (long long)i * p.n_q * p.Hq);
    const int j = jh / p.Hq;
    const int head = jh - j * p.Hq;
    const int g = head / p.G;
    const int qg = j / p.qgs;
    const int r = (j - qg * p.qgs) * p.G + (head - g * p.G);     // column of this row
    // the length and (balanced) the segment's descriptor are read together:
    // one memory round trip before the records
    const int seg = (i * p.Hkv + g) * p.n_qg + qg;
    int2 dsc = make_int2(0, 0);
    if (balanced) dsc = *reinterpret_cast<const int2*>(p.desc + 2 * seg);
    const int L = min(p.lens[i], p.max_len);
    if (L <= 0) return;
    int n, rec0;                              // records rec0 .. (see below), n of them
    if (balanced) {
        rec0 = dsc.x;
        n = dsc.y;
        if (n <= 1) return;                   // one wave wrote the rows
    } else {
        if (L <= p.part_tokens) return;       // written by the partition kernel
        n = (L + p.part_tokens - 1) / p.part_tokens;
        rec0 = (i * p.Hkv + g) * p.n_part;
    }
    // eight records per round trip: 72 VGPRs at d 128 instead of 129, so
    // seven waves per SIMD instead of three for the many rows of a window
    // (one wave per row)
    merge_records<D, 8>(p, h, r, n, rec0, balanced);
}

// Planned calls whose segments fit the arguments: workgroup (s, y) merges
// rows 4y .. 4y + 3 of (sequence, kv head) segment s, one per wave, and reads
// the segment's descriptor at once by its index.
template <int D>
__global__ void __launch_bounds__(kThreads)
paged_attn_merge_args_kernel(AttnParams p, MergeArgDesc md) {
    const uint32_t x = md.d[blockIdx.x];
    // every argument the merge reads, loaded together with the descriptor
    // (the compiler would otherwise wait for each before the next branch)
    const float* ws = p.ws;
    float* out = p.out;
    float* lse = p.lse;
    const int nrec = p.n_rec, cols = p.cols, Hkv = p.Hkv, Hq = p.Hq, G = p.G, n_q = p.n_q, qgs = p.qgs,
              n_qg = p.n_qg;
    asm volatile("" : : "s"(x), "s"(ws), "s"(out), "s"(lse), "s"(nrec), "s"(cols), "s"(Hkv), "s"(Hq), "s"(G),
                 "s"(n_q), "s"(qgs), "s"(n_qg));
    const int n = (int)(x >> 13);
    if (n <= 1) return;                       // whole, or an empty sequence
    const int rec0 = (int)(x & 0x1FFFu);
    // segment (sequence i, kv head g, query group qg); column r of its cols is
    // query qg * qgs + r / G of the window, head g * G + r % G
    const int HS = Hkv * n_qg;
    const int i = (int)blockIdx.x / HS;
    const int g2 = (int)blockIdx.x - i * HS;
    const int g = g2 / n_qg;
    const int qg = g2 - g * n_qg;
    const int r = kWaves * (int)blockIdx.y + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (r >= cols) return;
    const int jr = r / G;
    const int j = qg * qgs + jr;
    if (j >= n_q) return;
    merge_records<D>(p, ((long long)i * n_q + j) * Hq + g * G + (r - jr * G), r, n, rec0, true);
}

// Two attention states of the same rows over disjoint token sets (a shared
// prefix and a private suffix): out = (2^la a + 2^lb b) / (2^la + 2^lb) per
// row, with la, lb the rows' base-2 log softmax sums. A side with lse = -inf
// saw no token and gets weight 0; a row with both -inf is 0. One wave per row.
template <int D>
__global__ void __launch_bounds__(kThreads)
merge_states_kernel(float* __restrict__ out, float* __restrict__ lse_out, const float* __restrict__ a,
                    const float* __restrict__ lse_a, const float* __restrict__ b,
                    const float* __restrict__ lse_b, long long rows) {
    const long long r = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (r >= rows) return;
    const int lane = threadIdx.x & 63;
    const float la = lse_a[r], lb = lse_b[r];
    const float M = fmaxf(la, lb);
    constexpr int PER = D / 64;
    if (M == -INFINITY) {
#pragma unroll
        for (int x = 0; x < PER; ++x) out[r * D + lane + 64 * x] = 0.f;
        if (lse_out && lane == 0) lse_out[r] = -INFINITY;
        return;
    }
    const float wa = __builtin_amdgcn_exp2f(la - M);
    const float wb = __builtin_amdgcn_exp2f(lb - M);
    const float den = wa + wb;
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const size_t e = r * D + lane + 64 * x;
        out[e] = (wa * a[e] + wb * b[e]) / den;
    }
    if (lse_out && lane == 0) lse_out[r] = M + __log2f(den);
}

// One side of a shared-prefix merge: where the attention state of an output
// row over one token set lies after a stream pass whose merge was not run.
// A segment one wave processed whole left the normalised row and its lse; a
// split segment left n partial records (see paged_attn_merge_kernel).
struct SideState {
    const float* rows;   // normalised rows [.][D] (whole segments)
    const float* lse;    // their base-2 log softmax sums
    const float* ws;     // partial records
    size_t nrec;         // record slots in ws
    int C;               // columns (rows) per record
    int col;             // this row's column
    int n;               // 0: no tokens; 1: whole; > 1: records
    int rec0;            // first record (descriptor)
};

// Record k of a side (k past the last is read as the last one, so loads
// issued ahead of their use stay inside this call's records).
template <int D>
__device__ __forceinline__ size_t side_rec(const SideState& x, int k) {
    k = min(k, max(x.n - 1, 0));
    return k == 0 ? (size_t)x.rec0 : (size_t)(2 * ((x.rec0 >> 1) + k));
}

// Source k of a side as a record (m, l, o): a whole row is (lse, 1, row).
template <int D>
__device__ __forceinline__ void side_source(const SideState& x, long long h, int k, int lane, float& m,
                                            float& l, float (&o)[D / 64]) {
    if (x.n == 1) {
        m = x.lse[h];
        l = 1.f;
#pragma unroll
        for (int u = 0; u < D / 64; ++u) o[u] = x.rows[h * D + lane + 64 * u];
        return;
    }
    const size_t rr = side_rec<D>(x, k) * x.C + x.col;
    m = x.ws[x.nrec * x.C * D + rr];
    l = x.ws[x.nrec * x.C * (D + 1) + rr];
#pragma unroll
    for (int u = 0; u < D / 64; ++u) o[u] = x.ws[rr * D + lane + 64 * u];
}

// Shared-prefix decode, final step: each output row (sequence i = group g,
// member m; head) combines its state over the group's shared prefix (window
// pass a, column m's head) with its state over its own suffix (decode pass b).
// Both passes ran without their merge; this kernel merges the records of
// both in one go: out = sum_k 2^(m_k - M) o_k / sum_k 2^(m_k - M) l_k over
// every source k of either side. One wave per row.
template <int D>
__global__ void __launch_bounds__(kThreads)
shared_prefix_merge_kernel(AttnParams a, AttnParams b, float* __restrict__ out, int M) {
    const long long h = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (h >= (long long)b.S * b.Hq) return;
    const int lane = threadIdx.x & 63;
    const int i = (int)(h / b.Hq);
    const int head = (int)(h - (long long)i * b.Hq);
    const int G = b.G;
    const int kvh = head / G;
    const int r = head - kvh * G;
    const int g = i / M;
    const int mm = i - g * M;
    const int qg = mm / a.qgs;
    const int seg_a = (g * a.Hkv + kvh) * a.n_qg + qg;
    const int seg_b = i * b.Hkv + kvh;
    // one round trip: both lengths and both descriptors
    const int La = min(a.lens[g], a.max_len);
    const int Lb = min(b.lens[i], b.max_len);
    const int2 da = *reinterpret_cast<const int2*>(a.desc + 2 * seg_a);
    const int2 db = *reinterpret_cast<const int2*>(b.desc + 2 * seg_b);
    SideState x[2];
    // a descriptor is this call's only where its side has tokens; otherwise
    // its record index is not used (and is set to 0)
    const int na = La > 0 ? max(da.y, 1) : 0, nb = Lb > 0 ? max(db.y, 1) : 0;
    x[0] = SideState{a.out, a.lse, a.ws, (size_t)a.n_rec, a.cols, (mm - qg * a.qgs) * G + r, na,
                     na > 1 ? da.x : 0};
    x[1] = SideState{b.out, b.lse, b.ws, (size_t)b.n_rec, b.cols, r, nb, nb > 1 ? db.x : 0};
    constexpr int PER = D / 64;
    float num[PER] = {};
    float den = 0.f, Mx = -INFINITY;
    if (x[0].n <= 8 && x[1].n <= 8) {
        // every load of both sides is issued before any is used
        float mv[16], lv[16], ov[16][PER];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = 8 * s + k;
                mv[e] = -INFINITY;
                lv[e] = 0.f;
#pragma unroll
                for (int u = 0; u < PER; ++u) ov[e][u] = 0.f;
                if (k < x[s].n) side_source<D>(x[s], h, k, lane, mv[e], lv[e], ov[e]);
            }
#pragma unroll
        for (int e = 0; e < 16; ++e) Mx = fmaxf(Mx, mv[e]);
        if (Mx != -INFINITY) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                if (mv[e] != -INFINITY) {
                    const float wt = __builtin_amdgcn_exp2f(mv[e] - Mx);
                    den += wt * lv[e];
#pragma unroll
                    for (int u = 0; u < PER; ++u) num[u] += wt * ov[e][u];
                }
            }
        }
    } else {
        // long sides: sources one at a time with a running maximum
        for (int s = 0; s < 2; ++s)
            for (int k = 0; k < x[s].n; ++k) {
                float m, l, o[PER];
                side_source<D>(x[s], h, k, lane, m, l, o);
                if (m == -INFINITY) continue;
                const float m_new = fmaxf(Mx, m);
                const float alpha = __builtin_amdgcn_exp2f(Mx - m_new);
                const float wt = __builtin_amdgcn_exp2f(m - m_new);
                den = den * alpha + wt * l;
#pragma unroll
                for (int u = 0; u < PER; ++u) num[u] = num[u] * alpha + wt * o[u];
                Mx = m_new;
            }
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) out[h * D + lane + 64 * u] = den > 0.f ? num[u] / den : 0.f;
}

// ----------------------------------------------------------------------------
// Dispatch
// ----------------------------------------------------------------------------

// The instantiations live in attn_inst.hip, one translation unit per (cache
// type, head dim).
AttnKernel pick(int kv, int d, int bs, int mode, int tiles, bool partition, bool cached = false) {
    if (kv == KV_F32) return d == 64 ? pick_kernel<KV_F32, 64>(bs, mode, tiles, partition, cached)
                                     : pick_kernel<KV_F32, 128>(bs, mode, tiles, partition, cached);
    if (kv == KV_BF16) return d == 64 ? pick_kernel<KV_BF16, 64>(bs, mode, tiles, partition, cached)
                                      : pick_kernel<KV_BF16, 128>(bs, mode, tiles, partition, cached);
    return d == 64 ? pick_kernel<KV_FP8, 64>(bs, mode, tiles, partition, cached)
                   : pick_kernel<KV_FP8, 128>(bs, mode, tiles, partition, cached);
}

AttnKernel pick_gather(int kv, int d, int bs, bool cached) {
    if (kv == KV_F32)
        return d == 64 ? pick_gather_kernel<KV_F32, 64>(bs, cached) : pick_gather_kernel<KV_F32, 128>(bs, cached);
    if (kv == KV_BF16)
        return d == 64 ? pick_gather_kernel<KV_BF16, 64>(bs, cached) : pick_gather_kernel<KV_BF16, 128>(bs, cached);
    return d == 64 ? pick_gather_kernel<KV_FP8, 64>(bs, cached) : pick_gather_kernel<KV_FP8, 128>(bs, cached);
}

AttnKernel pick_plan(int kv, int d, int bs, int mode, bool cached = false) {
    if (kv == KV_F32)
        return d == 64 ? pick_plan_kernel<KV_F32, 64>(bs, mode, cached) : pick_plan_kernel<KV_F32, 128>(bs, mode, cached);
    if (kv == KV_BF16)
        return d == 64 ? pick_plan_kernel<KV_BF16, 64>(bs, mode, cached)
                       : pick_plan_kernel<KV_BF16, 128>(bs, mode, cached);
    return d == 64 ? pick_plan_kernel<KV_FP8, 64>(bs, mode, cached) : pick_plan_kernel<KV_FP8, 128>(bs, mode, cached);
}

// Compute units of the current device (cached per device).
int compute_units() {
    static int cache[64] = {};
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    std::lock_guard<std::mutex> lock(mu);
    if (dev < 64 && cache[dev] > 0) return cache[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (dev < 64) cache[dev] = cus;
    return cus;
}

// Workgroups of `kern` the current device holds at once (cached per kernel,
// LDS size and device).
int resident_workgroups(AttnKernel kern, size_t lds) {
    struct Entry { AttnKernel k; size_t lds; int dev; int n; };
    static Entry cache[64];
    static int used = 0;
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    std::lock_guard<std::mutex> lock(mu);
    for (int e = 0; e < used; ++e)
        if (cache[e].k == kern && cache[e].lds == lds && cache[e].dev == dev) return cache[e].n;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                      kThreads, lds) != hipSuccess) return -1;
    const int n = cus * (per_cu > 0 ? per_cu : 1);
    if (used < 64) cache[used++] = Entry{kern, lds, dev, n};
    return n;
}

// Balanced split: partial records of up to kMaxWorkers waves, two each
// (256-byte multiple); the segment descriptors follow them.
size_t balanced_records_bytes(size_t G, int d) {
    const size_t b = 2 * (size_t)kMaxWorkers * G * (size_t)(d + 2) * sizeof(float);
    return (b + 255) / 256 * 256;
}

// Records of a balanced call with n_workers waves (256-byte multiple).
size_t grid_records_bytes(int n_workers, size_t G, int d) {
    const size_t b = 2 * (size_t)n_workers * G * (size_t)(d + 2) * sizeof(float);
    return (b + 255) / 256 * 256;
}

int64_t n_partitions(int32_t max_len, int32_t partition_size) {
    if (partition_size <= 0 || max_len <= 0) return 1;
    return ((int64_t)max_len + partition_size - 1) / partition_size;
}

}  // namespace

// ----------------------------------------------------------------------------
// C ABI
// ----------------------------------------------------------------------------

extern "C" pkv_status pkv_kv_cache_write(const void* k_new, const void* v_new, void* k_cache,
                                         void* v_cache, const int64_t* slot_mapping, int32_t T,
                                         int32_t Hkv, int32_t d, int32_t bs, int32_t P,
                                         pkv_dtype src_dtype, pkv_dtype cache_dtype,
                                         float k_inv_scale, float v_inv_scale, void* stream) {
    if (T < 0) return fail(PKV_E_INVALID, "kv_cache_write: T=%d < 0", T);
    if (Hkv <= 0 || P <= 0) return fail(PKV_E_INVALID, "kv_cache_write: Hkv=%d P=%d must be positive", Hkv, P);
    if (!pkv::is_head_dim(d)) return fail(PKV_E_INVALID, "kv_cache_write: d=%d not in {64,128}", d);
    if (!pkv::is_pow2_block(bs)) return fail(PKV_E_INVALID, "kv_cache_write: bs=%d not in {8,16,32,64,128}", bs);
    const bool same = src_dtype == cache_dtype && (src_dtype == PKV_F32 || src_dtype == PKV_BF16);
    const bool quant = cache_dtype == PKV_FP8_E4M3 && src_dtype == PKV_BF16;
    if (!same && !quant)
        return fail(PKV_E_INVALID, "kv_cache_write: unsupported src/cache dtypes %d/%d", src_dtype, cache_dtype);
    if (quant && !(std::isfinite(k_inv_scale) && std::isfinite(v_inv_scale) && k_inv_scale > 0.f &&
                   v_inv_scale > 0.f))
        return fail(PKV_E_INVALID, "kv_cache_write: fp8 inverse scales must be finite and > 0");
    if (T == 0) return ok();
    if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping)
        return fail(PKV_E_INVALID, "kv_cache_write: NULL pointer");
    auto st = static_cast<hipStream_t>(stream);
    const long long n_slots = (long long)P * bs;
    if (cache_dtype == PKV_F32)
        hipLaunchKernelGGL((kv_cache_write_kernel<KV_F32, KV_F32>), dim3(T), dim3(256), 0, st, k_new,
                           v_new, k_cache, v_cache, slot_mapping, Hkv, d, bs, n_slots, 1.f, 1.f);
    else if (cache_dtype == PKV_BF16)
        hipLaunchKernelGGL((kv_cache_write_kernel<KV_BF16, KV_BF16>), dim3(T), dim3(256), 0, st, k_new,
                           v_new, k_cache, v_cache, slot_mapping, Hkv, d, bs, n_slots, 1.f, 1.f);
    else
        hipLaunchKernelGGL((kv_cache_write_kernel<KV_BF16, KV_FP8>), dim3(T), dim3(256), 0, st, k_new,
                           v_new, k_cache, v_cache, slot_mapping, Hkv, d, bs, n_slots, k_inv_scale,
                           v_inv_scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_E_HIP, "kv_cache_write: launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Streaming read: every 16-byte unit of src once, with the nontemporal
// 16-byte loads the attention kernels stream the cache with, grid-stride
// (thread t reads units t, t + T, ...), U loads in flight per thread. Each
// thread xor-folds the words it loaded, so the loads stay, and writes sink[0]
// only when its fold hits one fixed value.
template <int U>
__global__ void __launch_bounds__(256) stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                          uint32_t* sink) {
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const size_t nt = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    unsigned acc = 0;
    for (; i + (U - 1) * nt < n16; i += U * nt) {
        v4u v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(src + i + u * nt));
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += nt) {
        const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(src + i));
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

extern "C" pkv_status pkv_stream_read(const void* src, size_t bytes, int32_t blocks, int32_t unroll,
                                      uint32_t* sink, void* stream) {
    if (!src || !sink) return fail(PKV_E_INVALID, "stream_read: NULL pointer");
    if (reinterpret_cast<uintptr_t>(src) % 16 != 0) return fail(PKV_E_INVALID, "stream_read: src not 16-byte aligned");
    if (blocks < 1 || blocks > (1 << 20)) return fail(PKV_E_INVALID, "stream_read: blocks=%d not in [1, 2^20]", blocks);
    const size_t n16 = bytes / 16;
    if (n16 == 0) return ok();
    auto st = static_cast<hipStream_t>(stream);
    const auto s = reinterpret_cast<const uint4*>(src);
    if (unroll == 4) hipLaunchKernelGGL(stream_read_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, st, s, n16, sink);
    else if (unroll == 8) hipLaunchKernelGGL(stream_read_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, st, s, n16, sink);
    else if (unroll == 16) hipLaunchKernelGGL(stream_read_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, st, s, n16, sink);
    else return fail(PKV_E_INVALID, "stream_read: unroll=%d not in {4, 8, 16}", unroll);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_E_HIP, "stream_read: launch failed: %s", hipGetErrorString(e));
    return ok();
}

extern "C" pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src,
                                      const int32_t* dst, int32_t n, int32_t P, int32_t Hkv,
                                      int32_t d, int32_t bs, pkv_dtype cache_dtype, void* stream) {
    if (n < 0) return fail(PKV_E_INVALID, "copy_blocks: n=%d < 0", n);
    if (Hkv <= 0 || P <= 0) return fail(PKV_E_INVALID, "copy_blocks: Hkv=%d P=%d must be positive", Hkv, P);
    if (!pkv::is_head_dim(d)) return fail(PKV_E_INVALID, "copy_blocks: d=%d not in {64,128}", d);
    if (!pkv::is_pow2_block(bs)) return fail(PKV_E_INVALID, "copy_blocks: bs=%d not in {8,16,32,64,128}", bs);
    size_t elem;
    if (cache_dtype == PKV_F32) elem = 4;
    else if (cache_dtype == PKV_BF16) elem = 2;
    else if (cache_dtype == PKV_FP8_E4M3) elem = 1;
    else return fail(PKV_E_INVALID, "copy_blocks: unsupported cache dtype %d", cache_dtype);
    if (n == 0) return ok();
    if (!k_cache || !v_cache || !src || !dst) return fail(PKV_E_INVALID, "copy_blocks: NULL pointer");
    if (n > P || n > (1 << 20))
        return fail(PKV_E_INVALID, "copy_blocks: n=%d above min(P=%d, 2^20)", n, P);
    const size_t bytes = (size_t)Hkv * bs * d * elem;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)n, 2), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<char*>(k_cache),
                       static_cast<char*>(v_cache), src, dst, P, bytes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_E_HIP, "copy_blocks: launch failed: %s", hipGetErrorString(e));
    return ok();
}

namespace {

// Query window layout of the balanced split: qgs queries per group (G * qgs
// MFMA columns in `tiles` tiles of 16) and n_qg groups, each one pass over
// the sequence's blocks. A window that fits one 16-column tile takes one
// tile; a larger one takes wide_tiles(d) tiles (32 columns) per pass.
struct QueryGroups {
    int qgs, n_qg, cols, tiles;
};
QueryGroups query_groups(int32_t n_q, int32_t G, int32_t d) {
    QueryGroups r;
    r.tiles = (int64_t)n_q * G <= 16 ? 1 : wide_tiles(d);
    const pkv_split::QueryGroups q = pkv_split::query_groups_in(n_q, G, r.tiles);
    r.qgs = q.qgs;
    r.n_qg = q.n_qg;
    r.cols = q.cols;
    return r;
}

size_t attn_workspace_size(int32_t S, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t d,
                           int32_t max_context_len, int32_t partition_size) {
    if (S <= 0 || n_q <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv != 0) return 0;
    const int32_t G = Hq / Hkv;
    if (partition_size == PKV_PARTITION_BALANCED) {
        const QueryGroups qg = query_groups(n_q, G, d);
        return balanced_records_bytes((size_t)qg.cols, d) +
               2 * (size_t)S * (size_t)Hkv * (size_t)qg.n_qg * sizeof(int);
    }
    const int64_t n = n_partitions(max_context_len, partition_size);
    if (n <= 1) return 0;
    return (size_t)S * (size_t)Hq * (size_t)n * (size_t)(d + 2) * sizeof(float);
}

// Validation and launch shared by the single-query and multi-query entry
// points (n_q > 1 always takes the balanced split).
// The new tokens a decode step writes (k_new == nullptr: no write).
struct StepWrite {
    const void* k_new = nullptr;
    const void* v_new = nullptr;
    float k_inv = 1.f, v_inv = 1.f;
};

pkv_status attn_launch(const char* fn, float* out, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                       int32_t S, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t d, int32_t bs,
                       int32_t P, int32_t max_blocks, int32_t max_context_len, float softmax_scale,
                       float k_scale, float v_scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                       int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream,
                       const StepWrite& step = StepWrite(), float* lse = nullptr,
                       bool causal = true, bool run_merge = true, AttnParams* used = nullptr,
                       bool validate_only = false, bool grid_sized_workspace = false) {
    const bool is_step = step.k_new != nullptr || step.v_new != nullptr;
    if (S < 0 || Hq <= 0 || Hkv <= 0) return fail(PKV_E_INVALID, "%s: S=%d Hq=%d Hkv=%d", fn, S, Hq, Hkv);
    if (n_q < 1 || n_q > 4096) return fail(PKV_E_INVALID, "%s: n_q=%d outside [1, 4096]", fn, n_q);
    if (Hq % Hkv != 0) return fail(PKV_E_INVALID, "%s: Hq=%d not a multiple of Hkv=%d", fn, Hq, Hkv);
    const int32_t G = Hq / Hkv;
    if (G > 16) return fail(PKV_E_INVALID, "%s: Hq/Hkv=%d > 16", fn, G);
    if (!pkv::is_head_dim(d)) return fail(PKV_E_INVALID, "%s: d=%d not in {64,128}", fn, d);
    if (!pkv::is_pow2_block(bs)) return fail(PKV_E_INVALID, "%s: bs=%d not in {8,16,32,64,128}", fn, bs);
    if (P <= 0 || max_blocks <= 0) return fail(PKV_E_INVALID, "%s: P=%d max_blocks=%d", fn, P, max_blocks);
    if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks * bs)
        return fail(PKV_E_INVALID, "%s: max_context_len=%d outside [0, max_blocks*bs=%lld]", fn,
                    max_context_len, (long long)max_blocks * bs);
    // the kernels form chunk counts in 32-bit arithmetic (split.h)
    if (max_context_len > (1 << 30))
        return fail(PKV_E_INVALID, "%s: max_context_len=%d above 2^30", fn, max_context_len);
    int kv;
    if (q_dtype == PKV_F32 && cache_dtype == PKV_F32) kv = KV_F32;
    else if (q_dtype == PKV_BF16 && cache_dtype == PKV_BF16) kv = KV_BF16;
    else if (q_dtype == PKV_BF16 && cache_dtype == PKV_FP8_E4M3) kv = KV_FP8;
    else return fail(PKV_E_INVALID, "%s: unsupported q/cache dtypes %d/%d", fn, q_dtype, cache_dtype);
    const bool balanced = partition_size == PKV_PARTITION_BALANCED;
    if (!balanced && (partition_size < 0 || partition_size % 32 != 0))
        return fail(PKV_E_INVALID, "%s: partition_size=%d not 0, a multiple of 32 or "
                    "PKV_PARTITION_BALANCED", fn, partition_size);
    if (!std::isfinite(softmax_scale)) return fail(PKV_E_INVALID, "%s: softmax_scale not finite", fn);
    if (kv == KV_FP8 && !(std::isfinite(k_scale) && std::isfinite(v_scale)))
        return fail(PKV_E_INVALID, "%s: fp8 scales not finite", fn);
    if (is_step && kv == KV_FP8 && !(std::isfinite(step.k_inv) && std::isfinite(step.v_inv) &&
                                     step.k_inv > 0.f && step.v_inv > 0.f))
        return fail(PKV_E_INVALID, "%s: fp8 inverse scales must be finite and > 0", fn);
    if (S == 0) return ok();
    if (is_step && (!step.k_new || !step.v_new)) return fail(PKV_E_INVALID, "%s: NULL pointer", fn);
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
        return fail(PKV_E_INVALID, "%s: NULL pointer", fn);
    const QueryGroups qgr = query_groups(n_q, G, d);
    const int64_t n_part = balanced ? 1 : n_partitions(max_context_len, partition_size);
    // grid_sized_workspace (balanced only): the records are sized to this
    // call's grid, not to the largest one, and checked once the grid is known
    const size_t need = grid_sized_workspace ? 0
                      : attn_workspace_size(S, n_q, Hq, Hkv, d, max_context_len, partition_size);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PKV_E_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, need);
    // upper bound on work items (fixed partitions) or positions (balanced)
    const int64_t n_upper = balanced ? (int64_t)S * Hkv * qgr.n_qg *
                                           (((int64_t)max_context_len + 15) / 16 + kSegCostMax)
                                     : n_part * (int64_t)S * Hkv;
    if (n_upper > 0x7FFFFFFFLL) return fail(PKV_E_INVALID, "%s: too many work items", fn);
    if (validate_only) return ok();

    AttnParams prm{};
    prm.out = out;
    prm.q = q;
    prm.k = k_cache;
    prm.v = v_cache;
    prm.tables = block_tables;
    prm.lens = context_lens;
    prm.ws = static_cast<float*>(workspace);
    prm.desc = balanced ? reinterpret_cast<int*>(static_cast<char*>(workspace) +
                                                 balanced_records_bytes((size_t)qgr.cols, d))
                        : nullptr;
    prm.S = S;
    prm.Hq = Hq;
    prm.Hkv = Hkv;
    prm.G = G;
    prm.P = P;
    prm.max_blocks = max_blocks;
    prm.max_len = max_context_len;
    prm.n_q = n_q;
    prm.qgs = qgr.qgs;
    prm.n_qg = qgr.n_qg;
    prm.cols = qgr.cols;
    // single pass: one partition long enough for any sequence (whole chunks)
    prm.part_tokens = partition_size > 0 ? partition_size : ((max(max_context_len, 1) + 31) / 32) * 32;
    prm.n_part = (int)n_part;
    prm.balanced = balanced ? 1 : 0;
    prm.k_new = step.k_new;
    prm.v_new = step.v_new;
    prm.k_inv = step.k_inv;
    prm.v_inv = step.v_inv;
    const float ks = kv == KV_FP8 ? k_scale : 1.f;
    prm.qk_scale = softmax_scale * ks * kLog2e;
    prm.v_scale = kv == KV_FP8 ? v_scale : 1.f;
    prm.lse = lse;
    prm.causal = causal ? 1 : 0;
    prm.cache_lens = S <= kMaxCachedLens;

    AttnKernel kern;
    size_t lds;
    if (balanced) {
        const int mode = is_step ? SM_STEP : n_q > 1 ? SM_WINDOW : SM_DECODE;
        const int tiles = mode == SM_WINDOW ? qgr.tiles : 1;
        // a wide window of several passes: plain loads, so that a pass can
        // find the blocks the neighbouring pass's segments just read
        const bool cached = mode == SM_WINDOW && tiles > 1 && qgr.n_qg > 1;
        kern = pick(kv, d, bs, mode, tiles, false, cached);
        lds = (size_t)(prm.cache_lens ? S : 0) * sizeof(int);
    } else {
        kern = pick(kv, d, bs, SM_DECODE, 1, true);
        lds = (size_t)(2 * kWaves * 16 + kWaves * G * d + (prm.cache_lens ? S : 0)) * sizeof(float);
    }
    auto st = static_cast<hipStream_t>(stream);
    const int resident = resident_workgroups(kern, lds);
    if (resident <= 0) return fail(PKV_E_HIP, "%s: occupancy query failed", fn);
    int64_t grid = n_upper < resident ? n_upper : resident;
    if (balanced) {
        // One workgroup per compute unit: a single wave per SIMD streams at the
        // same rate as any other (several resident waves per SIMD do not get
        // equal shares of memory bandwidth, which equal static ranges cannot
        // absorb). Idle ranges exit at once.
        const int cus = compute_units();
        if (cus <= 0) return fail(PKV_E_HIP, "%s: device query failed", fn);
        grid = cus < resident ? cus : resident;
        if (grid * kWaves > kMaxWorkers) grid = kMaxWorkers / kWaves;
    }
    if (grid < 1) grid = 1;
    prm.n_workers = (int)(balanced ? grid * kWaves : grid);
    prm.n_rec = balanced ? 2 * prm.n_workers : (int)(n_part * (int64_t)S * Hkv);
    if (balanced && grid_sized_workspace) {
        const size_t rec = grid_records_bytes(prm.n_workers, (size_t)qgr.cols, d);
        const size_t need_g = rec + 2 * (size_t)S * (size_t)Hkv * (size_t)qgr.n_qg * sizeof(int);
        if (!workspace || workspace_bytes < need_g)
            return fail(PKV_E_WORKSPACE, "%s: this call needs %zu bytes of workspace (%d waves, %d columns, "
                        "d %d, %d sequences x %d kv heads); %zu are available", fn, need_g, prm.n_workers,
                        qgr.cols, d, S, Hkv, workspace_bytes);
        prm.desc = reinterpret_cast<int*>(static_cast<char*>(workspace) + rec);
    }
    if (used) *used = prm;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, st, prm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_E_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    if (run_merge && (balanced || n_part > 1)) {
        const unsigned rgrid = (unsigned)(((int64_t)S * n_q * Hq + kWaves - 1) / kWaves);
        if (d == 64)
            hipLaunchKernelGGL(paged_attn_merge_kernel<64>, dim3(rgrid), dim3(kThreads), 0, st, prm);
        else
            hipLaunchKernelGGL(paged_attn_merge_kernel<128>, dim3(rgrid), dim3(kThreads), 0, st, prm);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(PKV_E_HIP, "%s: merge launch failed: %s", fn, hipGetErrorString(e));
    }
    return ok();
}

}  // namespace

extern "C" size_t pkv_paged_decode_attn_workspace_size(int32_t S, int32_t Hq, int32_t Hkv, int32_t d,
                                                       int32_t max_context_len,
                                                       int32_t partition_size) {
    return attn_workspace_size(S, 1, Hq, Hkv, d, max_context_len, partition_size);
}

extern "C" pkv_status pkv_paged_decode_attn(float* out, const void* q, const void* k_cache,
                                            const void* v_cache, const int32_t* block_tables,
                                            const int32_t* context_lens, int32_t S, int32_t Hq,
                                            int32_t Hkv, int32_t d, int32_t bs, int32_t P,
                                            int32_t max_blocks, int32_t max_context_len,
                                            float softmax_scale, float k_scale, float v_scale,
                                            pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                            int32_t partition_size, void* workspace,
                                            size_t workspace_bytes, void* stream) {
    return attn_launch("paged_decode_attn", out, q, k_cache, v_cache, block_tables, context_lens, S, 1,
                       Hq, Hkv, d, bs, P, max_blocks, max_context_len, softmax_scale, k_scale, v_scale,
                       q_dtype, cache_dtype, partition_size, workspace, workspace_bytes, stream);
}

extern "C" size_t pkv_paged_multi_query_attn_workspace_size(int32_t S, int32_t n_q, int32_t Hq,
                                                            int32_t Hkv, int32_t d) {
    return attn_workspace_size(S, n_q, Hq, Hkv, d, 0, PKV_PARTITION_BALANCED);
}

extern "C" pkv_status pkv_paged_multi_query_attn(float* out, const void* q, const void* k_cache,
                                                 const void* v_cache, const int32_t* block_tables,
                                                 const int32_t* context_lens, int32_t S, int32_t n_q,
                                                 int32_t Hq, int32_t Hkv, int32_t d, int32_t bs,
                                                 int32_t P, int32_t max_blocks,
                                                 int32_t max_context_len, float softmax_scale,
                                                 float k_scale, float v_scale, pkv_dtype q_dtype,
                                                 pkv_dtype cache_dtype, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
    return attn_launch("paged_multi_query_attn", out, q, k_cache, v_cache, block_tables, context_lens, S,
                       n_q, Hq, Hkv, d, bs, P, max_blocks, max_context_len, softmax_scale, k_scale,
                       v_scale, q_dtype, cache_dtype, PKV_PARTITION_BALANCED, workspace, workspace_bytes,
                       stream);
}

extern "C" pkv_status pkv_paged_decode_step(float* out, const void* q, const void* k_new,
                                            const void* v_new, void* k_cache, void* v_cache,
                                            const int32_t* block_tables, const int32_t* context_lens,
                                            int32_t S, int32_t Hq, int32_t Hkv, int32_t d, int32_t bs,
                                            int32_t P, int32_t max_blocks, int32_t max_context_len,
                                            float softmax_scale, float k_scale, float v_scale,
                                            float k_inv_scale, float v_inv_scale, pkv_dtype q_dtype,
                                            pkv_dtype cache_dtype, void* workspace,
                                            size_t workspace_bytes, void* stream) {
    StepWrite w;
    w.k_new = k_new;
    w.v_new = v_new;
    w.k_inv = cache_dtype == PKV_FP8_E4M3 ? k_inv_scale : 1.f;
    w.v_inv = cache_dtype == PKV_FP8_E4M3 ? v_inv_scale : 1.f;
    if (S > 0 && (!k_new || !v_new)) return fail(PKV_E_INVALID, "paged_decode_step: NULL pointer");
    return attn_launch("paged_decode_step", out, q, k_cache, v_cache, block_tables, context_lens, S, 1,
                       Hq, Hkv, d, bs, P, max_blocks, max_context_len, softmax_scale, k_scale, v_scale,
                       q_dtype, cache_dtype, PKV_PARTITION_BALANCED, workspace, workspace_bytes, stream, w);
}

// ----------------------------------------------------------------------------
// Decode step without any allocation: the records and descriptors of the
// balanced split live in a file-scope device array instead of a caller
// workspace. Each device that runs it holds its own copy of the array for the
// life of the process; its address on a device is looked up once, with that
// device current, and kept.
// ----------------------------------------------------------------------------

namespace {

constexpr size_t kScratchBytes = (size_t)PKV_STEP_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Address of this device's copy of `scratch` (nullptr and *err set on failure).
void* scratch_on_current_device(hipError_t* err) {
    static void* addr[64] = {};
    static std::mutex mu;
    int dev = 0;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= 64) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        addr[dev] = ptr;
    }
    return addr[dev];
}

}  // namespace

extern "C" size_t pkv_paged_decode_step_scratch_bytes(void) { return kScratchBytes; }

extern "C" pkv_status pkv_paged_decode_step_noalloc(float* out, const void* q, const void* k_new,
                                                    const void* v_new, void* k_cache, void* v_cache,
                                                    const int32_t* block_tables,
                                                    const int32_t* context_lens, int32_t S, int32_t Hq,
                                                    int32_t Hkv, int32_t d, int32_t bs, int32_t P,
                                                    int32_t max_blocks, int32_t max_context_len,
                                                    float softmax_scale, float k_scale, float v_scale,
                                                    float k_inv_scale, float v_inv_scale,
                                                    pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                                    void* stream) {
    const char* fn = "paged_decode_step_noalloc";
    StepWrite w;
    w.k_new = k_new;
    w.v_new = v_new;
    w.k_inv = cache_dtype == PKV_FP8_E4M3 ? k_inv_scale : 1.f;
    w.v_inv = cache_dtype == PKV_FP8_E4M3 ? v_inv_scale : 1.f;
    if (S > 0 && (!k_new || !v_new)) return fail(PKV_E_INVALID, "%s: NULL pointer", fn);
    // every argument check first (no HIP call), then the scratch address
    pkv_status rc = attn_launch(fn, out, q, k_cache, v_cache, block_tables, context_lens, S, 1, Hq, Hkv, d,
                                bs, P, max_blocks, max_context_len, softmax_scale, k_scale, v_scale, q_dtype,
                                cache_dtype, PKV_PARTITION_BALANCED, nullptr, 0, stream, w, nullptr, true,
                                true, nullptr, true, true);
    if (rc != PKV_OK || S == 0) return rc;
    hipError_t e = hipSuccess;
    void* ws = scratch_on_current_device(&e);
    if (!ws) return fail(PKV_E_HIP, "%s: scratch address lookup failed: %s", fn, hipGetErrorString(e));
    return attn_launch(fn, out, q, k_cache, v_cache, block_tables, context_lens, S, 1, Hq, Hkv, d, bs, P,
                       max_blocks, max_context_len, softmax_scale, k_scale, v_scale, q_dtype, cache_dtype,
                       PKV_PARTITION_BALANCED, ws, kScratchBytes, stream, w, nullptr, true, true, nullptr,
                       false, true);
}

// ----------------------------------------------------------------------------
// Planned decode: the balanced split read from a host-built plan
// ----------------------------------------------------------------------------

namespace {

// Waves of the planned kernel's grid on the current device: one 4-wave
// workgroup per compute unit, as the stream kernel, or two where a chunk is
// 2 KiB or less (fp8 at d 64) and both fit. Measured: such chunks stream
// faster with twice the waves in flight (`small` fp8 24.7 -> 22.1 us), larger
// ones slower (`llama8b` 69.4 -> 71.0 us, `long` 356 -> 364 us).
// The step and the attention-only kernels share the grid (one plan serves
// both): the smaller of their residencies decides.
int plan_workers(int kv, int d, int bs) {
    // the smallest residency of the planned kernel's variants: a plan serves
    // any of them
    int resident = 1 << 30;
    for (int mode : {PM_ATTN, PM_STEP, PM_WINDOW, PM_WINDOW2})
        for (bool cached : {false, true}) {
            if (mode == PM_WINDOW && cached) continue;
            const AttnKernel k = pick_plan(kv, d, bs, mode, cached);
            if (!k) return -1;
            const int r = resident_workgroups(k, 0);
            if (r < resident) resident = r;
        }
    const int cus = compute_units();
    if (resident <= 0 || cus <= 0) return -1;
    const int chunk_bytes = 16 * 2 * d * (kv == KV_F32 ? 4 : kv == KV_BF16 ? 2 : 1);
    const int per_cu = chunk_bytes <= 2048 ? 2 : 1;
    int grid = cus * per_cu < resident ? cus * per_cu : resident;
    if (grid * kWaves > kMaxWorkers) grid = kMaxWorkers / kWaves;
    return grid * kWaves;
}

// The plan's header against the call (S, Hkv, d, cache kind, max_context_len,
// the window: n_q queries over G heads per kv head, 0 for a decode plan; its
// size) and this device's wave count; n_workers, stride and the query
// grouping (qgs, n_qg; 1 and 1 for decode) from it.
pkv_status check_plan(const char* fn, const void* plan_host, const void* plan_dev, size_t plan_bytes, int32_t S,
                      int32_t n_q, int32_t G, int32_t Hkv, int32_t d, int32_t bs, int kv, int32_t max_context_len,
                      int32_t* n_workers, int32_t* stride, int32_t* qgs, int32_t* n_qg) {
    if (!plan_host || !plan_dev) return fail(PKV_E_INVALID, "%s: NULL plan", fn);
    if (plan_bytes < pkv_split::kPlanHeader * sizeof(int32_t))
        return fail(PKV_E_INVALID, "%s: plan of %zu bytes", fn, plan_bytes);
    const int32_t* h = static_cast<const int32_t*>(plan_host);
    if (h[0] != pkv_split::kPlanMagic || h[1] != pkv_split::kPlanVersion)
        return fail(PKV_E_INVALID, "%s: not a decode plan (magic %#x version %d)", fn, h[0], h[1]);
    if (h[4] != S || h[5] != Hkv || h[8] != max_context_len || h[9] != d || h[10] != kv)
        return fail(PKV_E_INVALID, "%s: the plan was built for S=%d Hkv=%d max_context_len=%d d=%d kv=%d, "
                    "not S=%d Hkv=%d max_context_len=%d d=%d kv=%d", fn, h[4], h[5], h[8], h[9], h[10], S, Hkv,
                    max_context_len, d, kv);
    if (h[11] != n_q || (n_q > 0 && h[12] != G))
        return fail(PKV_E_INVALID, "%s: the plan was built for a window of %d queries over %d heads per kv head "
                    "(0: a decode plan), not %d over %d", fn, h[11], h[12], n_q, G);
    *qgs = 1;
    *n_qg = 1;
    if (n_q > 0) {
        const pkv_split::QueryGroups q = pkv_split::query_groups_in(n_q, G, pkv_split::window_plan_tiles(n_q, G));
        if (h[13] != q.qgs || h[14] != q.n_qg)
            return fail(PKV_E_INVALID, "%s: the plan's query groups (%d x %d) are not those of %d queries over %d "
                        "heads", fn, h[14], h[13], n_q, G);
        *qgs = q.qgs;
        *n_qg = q.n_qg;
    }
    *n_workers = h[2];
    *stride = h[7];
    const size_t words = (size_t)pkv_split::kPlanHeader + (size_t)*n_workers * *stride * 4 +
                         (size_t)S * Hkv * (size_t)*n_qg * 2;
    if (*stride <= 0 || *n_workers <= 0 || plan_bytes < words * sizeof(int32_t))
        return fail(PKV_E_INVALID, "%s: plan of %zu bytes, its header describes %zu", fn, plan_bytes,
                    words * sizeof(int32_t));
    const int workers = plan_workers(kv, d, bs);
    if (workers <= 0) return fail(PKV_E_HIP, "%s: device query failed", fn);
    if (workers != *n_workers)
        return fail(PKV_E_INVALID, "%s: the plan was built for %d waves, this device runs %d "
                    "(pkv_paged_decode_plan_workers)", fn, *n_workers, workers);
    return ok();
}

// A planned call: the decode step or attention (n_q = 0, a decode plan) or a
// query window of n_q queries per sequence (a window plan; no write).
pkv_status plan_launch(const char* fn, float* out, const void* q, const void* k_new, const void* v_new,
                       void* k_cache, void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                       int32_t S, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t d, int32_t bs, int32_t P,
                       int32_t max_blocks,
                       int32_t max_context_len, float softmax_scale, float k_scale, float v_scale,
                       float k_inv_scale, float v_inv_scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                       const void* plan_host, const void* plan_dev, size_t plan_bytes, void* workspace,
                       size_t workspace_bytes, void* stream, void* attn_done_event) {
    const bool is_step = k_new != nullptr || v_new != nullptr;
    StepWrite wr;
    wr.k_new = k_new;
    wr.v_new = v_new;
    wr.k_inv = cache_dtype == PKV_FP8_E4M3 ? k_inv_scale : 1.f;
    wr.v_inv = cache_dtype == PKV_FP8_E4M3 ? v_inv_scale : 1.f;
    // the arguments shared with the unplanned call, checked the same way
    if (n_q > 0 && is_step) return fail(PKV_E_INVALID, "%s: a window call writes no new tokens", fn);
    pkv_status rc = attn_launch(fn, out, q, k_cache, v_cache, block_tables, context_lens, S, n_q > 0 ? n_q : 1, Hq,
                                Hkv, d, bs, P, max_blocks, max_context_len, softmax_scale, k_scale, v_scale, q_dtype,
                                cache_dtype, PKV_PARTITION_BALANCED, nullptr, 0, stream, wr, nullptr, true, true,
                                nullptr, true, true);
    if (rc != PKV_OK || S == 0) return rc;
    const int kv = cache_dtype == PKV_F32 ? KV_F32 : cache_dtype == PKV_BF16 ? KV_BF16 : KV_FP8;
    const int32_t G = Hq / Hkv;
    int32_t n_workers = 0, stride = 0, qgs = 1, n_qg = 1;
    rc = check_plan(fn, plan_host, plan_dev, plan_bytes, S, n_q, G, Hkv, d, bs, kv, max_context_len, &n_workers,
                    &stride, &qgs, &n_qg);
    if (rc != PKV_OK) return rc;
    const int32_t cols = G * qgs;             // record rows per piece
    const size_t need = grid_records_bytes(n_workers, (size_t)cols, d);
    if (!workspace || workspace_bytes < need)
        return fail(PKV_E_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, need);

    AttnParams prm{};
    prm.out = out;
    prm.q = q;
    prm.k = k_cache;
    prm.v = v_cache;
    prm.tables = block_tables;
    prm.lens = context_lens;
    prm.ws = static_cast<float*>(workspace);
    const int32_t* pd = static_cast<const int32_t*>(plan_dev);
    prm.plan = pd + pkv_split::kPlanHeader;
    prm.plan_stride = stride;
    prm.desc = const_cast<int*>(pd + pkv_split::kPlanHeader + (size_t)n_workers * stride * 4);
    prm.S = S;
    prm.Hq = Hq;
    prm.Hkv = Hkv;
    prm.G = G;
    prm.P = P;
    prm.max_blocks = max_blocks;
    prm.max_len = max_context_len;
    prm.n_q = n_q > 0 ? n_q : 1;
    prm.qgs = qgs;
    prm.n_qg = n_qg;
    prm.cols = cols;
    prm.part_tokens = 32;
    prm.n_part = 1;
    prm.balanced = 1;
    prm.k_new = k_new;
    prm.v_new = v_new;
    prm.k_inv = wr.k_inv;
    prm.v_inv = wr.v_inv;
    prm.qk_scale = softmax_scale * (kv == KV_FP8 ? k_scale : 1.f) * kLog2e;
    prm.v_scale = kv == KV_FP8 ? v_scale : 1.f;
    prm.causal = 1;
    prm.n_workers = n_workers;
    prm.n_rec = 2 * n_workers;
    auto st = static_cast<hipStream_t>(stream);
    const int mode = n_q > 0 ? (cols > 16 ? PM_WINDOW2 : PM_WINDOW) : is_step ? PM_STEP : PM_ATTN;
    // cacheable K/V loads for a decode plan that lists shared blocks, and for
    // a window of several query groups per kv head (neighbouring segments
    // that read the same blocks at about the same time)
    const bool cached =
        n_q == 0 ? (static_cast<const int32_t*>(plan_host)[pkv_split::kPlanFlagsWord] & pkv_split::kPlanSharedBlocks) != 0
                 : mode == PM_WINDOW2 && n_qg > 1;
    hipLaunchKernelGGL(pick_plan(kv, d, bs, mode, cached), dim3((unsigned)(n_workers / kWaves)), dim3(kThreads), 0,
                       st, prm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_E_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    if (attn_done_event) {
        e = hipEventRecord(static_cast<hipEvent_t>(attn_done_event), st);
        if (e != hipSuccess) return fail(PKV_E_HIP, "%s: event record failed: %s", fn, hipGetErrorString(e));
    }
    const unsigned rgrid = (unsigned)(((int64_t)S * prm.n_q * Hq + kWaves - 1) / kWaves);
    const int64_t n_seg = (int64_t)S * Hkv * n_qg;
    if (n_seg <= kArgDescs) {
        // the plan's descriptors by value (the host copy holds them)
        MergeArgDesc md;
        const int32_t* hd = static_cast<const int32_t*>(plan_host) + pkv_split::kPlanHeader +
                            (size_t)n_workers * stride * 4;
        for (int64_t x = 0; x < n_seg; ++x) {
            const uint32_t rec0 = (uint32_t)hd[2 * x], cnt = (uint32_t)hd[2 * x + 1];
            md.d[x] = cnt <= 1 ? 0u : (rec0 & 0x1FFFu) | (cnt << 13);
        }
        const dim3 sgrid((unsigned)n_seg, (unsigned)((cols + kWaves - 1) / kWaves));
        if (d == 64)
            hipLaunchKernelGGL(paged_attn_merge_args_kernel<64>, sgrid, dim3(kThreads), 0, st, prm, md);
        else
            hipLaunchKernelGGL(paged_attn_merge_args_kernel<128>, sgrid, dim3(kThreads), 0, st, prm, md);
    } else if (d == 64) {
        hipLaunchKernelGGL(paged_attn_merge_kernel<64>, dim3(rgrid), dim3(kThreads), 0, st, prm);
    } else {
        hipLaunchKernelGGL(paged_attn_merge_kernel<128>, dim3(rgrid), dim3(kThreads), 0, st, prm);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_E_HIP, "%s: merge launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" int32_t pkv_paged_decode_plan_workers(int32_t d, int32_t bs, pkv_dtype cache_dtype) {
    if (!pkv::is_head_dim(d) || !pkv::is_pow2_block(bs)) return -1;
    const int kv = cache_dtype == PKV_F32 ? KV_F32 : cache_dtype == PKV_BF16 ? KV_BF16
                 : cache_dtype == PKV_FP8_E4M3 ? KV_FP8 : -1;
    if (kv < 0) return -1;
    return plan_workers(kv, d, bs);
}

extern "C" size_t pkv_paged_decode_plan_workspace_size(int32_t n_workers, int32_t Hq, int32_t Hkv, int32_t d) {
    if (n_workers <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || !pkv::is_head_dim(d)) return 0;
    return grid_records_bytes(n_workers, (size_t)(Hq / Hkv), d);
}

extern "C" pkv_status pkv_paged_gather_read(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                            int32_t S, int32_t Hkv, int32_t d, int32_t bs, int32_t P,
                                            int32_t max_blocks, int32_t max_context_len, pkv_dtype cache_dtype,
                                            const void* plan_host, const void* plan_dev, size_t plan_bytes,
                                            uint32_t* sink, void* stream) {
    const char* fn = "paged_gather_read";
    if (S <= 0 || Hkv <= 0 || P <= 0 || max_blocks <= 0 || max_context_len < 0)
        return fail(PKV_E_INVALID, "%s: S=%d Hkv=%d P=%d max_blocks=%d max_context_len=%d", fn, S, Hkv, P,
                    max_blocks, max_context_len);
    if (!pkv::is_head_dim(d)) return fail(PKV_E_INVALID, "%s: d=%d not in {64,128}", fn, d);
    if (!pkv::is_pow2_block(bs)) return fail(PKV_E_INVALID, "%s: bs=%d not in {8,16,32,64,128}", fn, bs);
    if (cache_dtype != PKV_F32 && cache_dtype != PKV_BF16 && cache_dtype != PKV_FP8_E4M3)
        return fail(PKV_E_INVALID, "%s: unsupported cache dtype %d", fn, cache_dtype);
    if (!k_cache || !v_cache || !block_tables || !sink) return fail(PKV_E_INVALID, "%s: NULL pointer", fn);
    if ((int64_t)max_context_len > (int64_t)max_blocks * bs || max_context_len > (1 << 30))
        return fail(PKV_E_INVALID, "%s: max_context_len=%d exceeds max_blocks*bs=%lld or 2^30", fn, max_context_len,
                    (long long)max_blocks * bs);
    const int kv = cache_dtype == PKV_F32 ? KV_F32 : cache_dtype == PKV_BF16 ? KV_BF16 : KV_FP8;
    int32_t n_workers = 0, stride = 0, qgs = 1, n_qg = 1;
    pkv_status rc = check_plan(fn, plan_host, plan_dev, plan_bytes, S, 0, 0, Hkv, d, bs, kv, max_context_len,
                               &n_workers, &stride, &qgs, &n_qg);
    if (rc != PKV_OK) return rc;
    AttnParams prm{};
    prm.k = k_cache;
    prm.v = v_cache;
    prm.tables = block_tables;
    prm.ws = reinterpret_cast<float*>(sink);
    prm.plan = static_cast<const int32_t*>(plan_dev) + pkv_split::kPlanHeader;
    prm.plan_stride = stride;
    prm.S = S;
    prm.Hkv = Hkv;
    prm.P = P;
    prm.max_blocks = max_blocks;
    prm.max_len = max_context_len;
    const bool cached = static_cast<const int32_t*>(plan_host)[pkv_split::kPlanFlagsWord] & pkv_split::kPlanSharedBlocks;
    const AttnKernel kern = pick_gather(kv, d, bs, cached);
    if (!kern) return fail(PKV_E_INVALID, "%s: no kernel for d=%d bs=%d", fn, d, bs);
    hipLaunchKernelGGL(kern, dim3((unsigned)(n_workers / kWaves)), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       prm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_E_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

extern "C" pkv_status pkv_paged_decode_step_planned(
    float* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    const int32_t* block_tables, const int32_t* context_lens, int32_t S, int32_t Hq, int32_t Hkv, int32_t d,
    int32_t bs, int32_t P, int32_t max_blocks, int32_t max_context_len, float softmax_scale, float k_scale,
    float v_scale, float k_inv_scale, float v_inv_scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
    const void* plan_host, const void* plan_dev, size_t plan_bytes, void* workspace, size_t workspace_bytes,
    void* stream, void* attn_done_event) {
    if (S > 0 && (k_new == nullptr) != (v_new == nullptr))
        return fail(PKV_E_INVALID, "paged_decode_step_planned: k_new and v_new must both be given or both be NULL");
    return plan_launch("paged_decode_step_planned", out, q, k_new, v_new, k_cache, v_cache, block_tables,
                       context_lens, S, 0, Hq, Hkv, d, bs, P, max_blocks, max_context_len, softmax_scale, k_scale,
                       v_scale, k_inv_scale, v_inv_scale, q_dtype, cache_dtype, plan_host, plan_dev, plan_bytes,
                       workspace, workspace_bytes, stream, attn_done_event);
}

extern "C" size_t pkv_paged_window_plan_workspace_size(int32_t n_workers, int32_t n_q, int32_t Hq, int32_t Hkv,
                                                      int32_t d) {
    if (n_workers <= 0 || n_q <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Hq / Hkv > 16 || !pkv::is_head_dim(d))
        return 0;
    const int32_t G = Hq / Hkv;
    const pkv_split::QueryGroups q = pkv_split::query_groups_in(n_q, G, pkv_split::window_plan_tiles(n_q, G));
    return grid_records_bytes(n_workers, (size_t)q.cols, d);
}

extern "C" pkv_status pkv_paged_multi_query_attn_planned(
    float* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
    const int32_t* context_lens, int32_t S, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t d, int32_t bs, int32_t P,
    int32_t max_blocks, int32_t max_context_len, float softmax_scale, float k_scale, float v_scale,
    pkv_dtype q_dtype, pkv_dtype cache_dtype, const void* plan_host, const void* plan_dev, size_t plan_bytes,
    void* workspace, size_t workspace_bytes, void* stream) {
    if (n_q <= 0) return fail(PKV_E_INVALID, "paged_multi_query_attn_planned: n_q=%d", n_q);
    return plan_launch("paged_multi_query_attn_planned", out, q, nullptr, nullptr, const_cast<void*>(k_cache),
                       const_cast<void*>(v_cache), block_tables, context_lens, S, n_q, Hq, Hkv, d, bs, P,
                       max_blocks, max_context_len, softmax_scale, k_scale, v_scale, 1.f, 1.f, q_dtype,
                       cache_dtype, plan_host, plan_dev, plan_bytes, workspace, workspace_bytes, stream, nullptr);
}

extern "C" pkv_status pkv_paged_decode_attn_lse(float* out, float* lse, const void* q,
                                                const void* k_cache, const void* v_cache,
                                                const int32_t* block_tables,
                                                const int32_t* context_lens, int32_t S, int32_t Hq,
                                                int32_t Hkv, int32_t d, int32_t bs, int32_t P,
                                                int32_t max_blocks, int32_t max_context_len,
                                                float softmax_scale, float k_scale, float v_scale,
                                                pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                                void* workspace, size_t workspace_bytes,
                                                void* stream) {
    if (S > 0 && !lse) return fail(PKV_E_INVALID, "paged_decode_attn_lse: NULL pointer");
    return attn_launch("paged_decode_attn_lse", out, q, k_cache, v_cache, block_tables, context_lens, S,
                       1, Hq, Hkv, d, bs, P, max_blocks, max_context_len, softmax_scale, k_scale,
                       v_scale, q_dtype, cache_dtype, PKV_PARTITION_BALANCED, workspace,
                       workspace_bytes, stream, StepWrite(), lse, true);
}

extern "C" pkv_status pkv_paged_shared_prefix_attn(float* out, float* lse, const void* q,
                                                   const void* k_cache, const void* v_cache,
                                                   const int32_t* prefix_tables,
                                                   const int32_t* prefix_lens, int32_t n_groups,
                                                   int32_t M, int32_t Hq, int32_t Hkv, int32_t d,
                                                   int32_t bs, int32_t P, int32_t max_blocks,
                                                   int32_t max_prefix_len, float softmax_scale,
                                                   float k_scale, float v_scale, pkv_dtype q_dtype,
                                                   pkv_dtype cache_dtype, void* workspace,
                                                   size_t workspace_bytes, void* stream) {
    if (n_groups > 0 && !lse) return fail(PKV_E_INVALID, "paged_shared_prefix_attn: NULL pointer");
    return attn_launch("paged_shared_prefix_attn", out, q, k_cache, v_cache, prefix_tables, prefix_lens,
                       n_groups, M, Hq, Hkv, d, bs, P, max_blocks, max_prefix_len, softmax_scale,
                       k_scale, v_scale, q_dtype, cache_dtype, PKV_PARTITION_BALANCED, workspace,
                       workspace_bytes, stream, StepWrite(), lse, false);
}

extern "C" pkv_status pkv_merge_attn_states(float* out, float* lse_out, const float* a,
                                            const float* lse_a, const float* b, const float* lse_b,
                                            int64_t rows, int32_t d, void* stream) {
    if (rows < 0) return fail(PKV_E_INVALID, "merge_attn_states: rows=%lld < 0", (long long)rows);
    if (!pkv::is_head_dim(d)) return fail(PKV_E_INVALID, "merge_attn_states: d=%d not in {64,128}", d);
    if (rows == 0) return ok();
    if (!out || !a || !lse_a || !b || !lse_b) return fail(PKV_E_INVALID, "merge_attn_states: NULL pointer");
    if (rows > (int64_t)0x7FFFFFFF * kWaves) return fail(PKV_E_INVALID, "merge_attn_states: too many rows");
    const unsigned grid = (unsigned)((rows + kWaves - 1) / kWaves);
    auto st = static_cast<hipStream_t>(stream);
    if (d == 64)
        hipLaunchKernelGGL(merge_states_kernel<64>, dim3(grid), dim3(kThreads), 0, st, out, lse_out, a,
                           lse_a, b, lse_b, (long long)rows);
    else
        hipLaunchKernelGGL(merge_states_kernel<128>, dim3(grid), dim3(kThreads), 0, st, out, lse_out, a,
                           lse_a, b, lse_b, (long long)rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_E_HIP, "merge_attn_states: launch failed: %s", hipGetErrorString(e));
    return ok();
}

namespace {

// Workspace of pkv_paged_shared_prefix_decode: the prefix pass's balanced
// workspace (with room for the descriptors of every prefix and suffix
// segment, for the one-launch form), the suffix pass's, then both passes'
// rows and lse values.
struct SharedPrefixLayout {
    size_t a, b, out_a, lse_a, out_b, lse_b, total;
};
SharedPrefixLayout shared_prefix_layout(int32_t n_groups, int32_t M, int32_t Hq, int32_t Hkv, int32_t d) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    SharedPrefixLayout L{};
    const size_t S = (size_t)n_groups * (size_t)M;
    const size_t rows = S * (size_t)Hq;
    L.a = 0;
    L.b = L.a + up(attn_workspace_size(n_groups, M, Hq, Hkv, d, 0, PKV_PARTITION_BALANCED) +
                   2 * S * (size_t)Hkv * sizeof(int));
    L.out_a = L.b + up(attn_workspace_size((int32_t)S, 1, Hq, Hkv, d, 0, PKV_PARTITION_BALANCED));
    L.lse_a = L.out_a + up(rows * d * sizeof(float));
    L.out_b = L.lse_a + up(rows * sizeof(float));
    L.lse_b = L.out_b + up(rows * d * sizeof(float));
    L.total = L.lse_b + up(rows * sizeof(float));
    return L;
}

}  // namespace

extern "C" size_t pkv_paged_shared_prefix_decode_workspace_size(int32_t n_groups, int32_t M, int32_t Hq,
                                                                int32_t Hkv, int32_t d) {
    if (n_groups <= 0 || M <= 0 || M > 4096 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 ||
        !pkv::is_head_dim(d) || (int64_t)n_groups * M > 0x7FFFFFFF)
        return 0;
    return shared_prefix_layout(n_groups, M, Hq, Hkv, d).total;
}

extern "C" pkv_status pkv_paged_shared_prefix_decode(
    float* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    const int32_t* prefix_tables, const int32_t* prefix_lens, int32_t prefix_max_blocks,
    int32_t max_prefix_len, const int32_t* suffix_tables, const int32_t* suffix_lens,
    int32_t suffix_max_blocks, int32_t max_suffix_len, int32_t n_groups, int32_t M, int32_t Hq,
    int32_t Hkv, int32_t d, int32_t bs, int32_t P, float softmax_scale, float k_scale, float v_scale,
    float k_inv_scale, float v_inv_scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, void* workspace,
    size_t workspace_bytes, void* stream) {
    const char* fn = "paged_shared_prefix_decode";
    if (n_groups < 0 || M < 1 || M > 4096)
        return fail(PKV_E_INVALID, "%s: n_groups=%d M=%d (need n_groups >= 0, 1 <= M <= 4096)", fn, n_groups, M);
    if ((int64_t)n_groups * M > 0x7FFFFFFF) return fail(PKV_E_INVALID, "%s: too many sequences", fn);
    if ((k_new == nullptr) != (v_new == nullptr))
        return fail(PKV_E_INVALID, "%s: k_new and v_new must both be given or both be NULL", fn);
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || !pkv::is_head_dim(d))
        return fail(PKV_E_INVALID, "%s: Hq=%d Hkv=%d d=%d", fn, Hq, Hkv, d);
    if (n_groups == 0) return ok();
    if (!out || !q || !k_cache || !v_cache || !prefix_tables || !prefix_lens || !suffix_tables || !suffix_lens)
        return fail(PKV_E_INVALID, "%s: NULL pointer", fn);
    const SharedPrefixLayout lay = shared_prefix_layout(n_groups, M, Hq, Hkv, d);
    if (!workspace || workspace_bytes < lay.total)
        return fail(PKV_E_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, lay.total);
    char* ws = static_cast<char*>(workspace);
    float* out_a = reinterpret_cast<float*>(ws + lay.out_a);
    float* lse_a = reinterpret_cast<float*>(ws + lay.lse_a);
    float* out_b = reinterpret_cast<float*>(ws + lay.out_b);
    float* lse_b = reinterpret_cast<float*>(ws + lay.lse_b);
    const int32_t S = n_groups * M;
    // the suffixes first: they hold each sequence's last block, so this pass
    // also writes the step's new tokens (when given) before the prefix pass
    StepWrite step;
    step.k_new = k_new;
    step.v_new = v_new;
    step.k_inv = cache_dtype == PKV_FP8_E4M3 ? k_inv_scale : 1.f;
    step.v_inv = cache_dtype == PKV_FP8_E4M3 ? v_inv_scale : 1.f;
    AttnParams pb, pa;
    const int32_t G = Hq / Hkv;
    const QueryGroups qa = query_groups(M, G, d);
    // A group's M queries fit one 16-column tile: prefixes and suffixes go
    // through one launch of the stream kernel (the prefix segments as windows
    // without a causal mask, the suffix segments as decode-step segments).
    // Otherwise two launches: the suffix pass, then the prefix pass.
    const bool one_launch = qa.tiles == 1 && (int64_t)n_groups + S <= 0x7FFFFFFF;
    // both passes' arguments are checked before anything is launched
    for (int launch = 0; launch < 2; ++launch) {
        const bool check_only = launch == 0 || one_launch;
        pkv_status rc = attn_launch(fn, out_b, q, k_cache, v_cache, suffix_tables, suffix_lens, S, 1, Hq, Hkv,
                                    d, bs, P, suffix_max_blocks, max_suffix_len, softmax_scale, k_scale,
                                    v_scale, q_dtype, cache_dtype, PKV_PARTITION_BALANCED, ws + lay.b,
                                    lay.out_a - lay.b, stream, step, lse_b, true, false, &pb, check_only);
        if (rc != PKV_OK) return rc;
        rc = attn_launch(fn, out_a, q, k_cache, v_cache, prefix_tables, prefix_lens, n_groups, M, Hq, Hkv, d,
                         bs, P, prefix_max_blocks, max_prefix_len, softmax_scale, k_scale, v_scale, q_dtype,
                         cache_dtype, PKV_PARTITION_BALANCED, ws + lay.a, lay.b - lay.a, stream, StepWrite(),
                         lse_a, false, false, &pa, check_only);
        if (rc != PKV_OK) return rc;
    }
    if (one_launch) {
        const int64_t n_seq = (int64_t)n_groups + S;
        const int64_t n_upper = n_seq * Hkv * (((int64_t)std::max(max_prefix_len, max_suffix_len) + 15) / 16 +
                                               kSegCostMax);
        if (n_upper > 0x7FFFFFFFLL) return fail(PKV_E_INVALID, "%s: too many work items", fn);
        const int kv = cache_dtype == PKV_F32 ? KV_F32 : cache_dtype == PKV_BF16 ? KV_BF16 : KV_FP8;
        AttnKernel kern = pick(kv, d, bs, SM_SHARED, 1, false);
        AttnParams prm{};
        prm.out = out_a;
        prm.lse = lse_a;
        prm.out2 = out_b;
        prm.lse2 = lse_b;
        prm.q = q;
        prm.k = k_cache;
        prm.v = v_cache;
        prm.tables = prefix_tables;
        prm.lens = prefix_lens;
        prm.max_blocks = prefix_max_blocks;
        prm.max_len = max_prefix_len;
        prm.tables2 = suffix_tables;
        prm.lens2 = suffix_lens;
        prm.max_blocks2 = suffix_max_blocks;
        prm.max_len2 = max_suffix_len;
        prm.n_pre = n_groups;
        prm.S = (int)n_seq;
        prm.Hq = Hq;
        prm.Hkv = Hkv;
        prm.G = G;
        prm.P = P;
        prm.n_q = M;
        prm.qgs = qa.qgs;
        prm.n_qg = qa.n_qg;
        prm.cols = qa.cols;
        prm.part_tokens = 32;
        prm.n_part = 1;
        prm.balanced = 1;
        prm.causal = 0;
        prm.ws = reinterpret_cast<float*>(ws + lay.a);
        prm.desc = reinterpret_cast<int*>(ws + lay.a + balanced_records_bytes((size_t)qa.cols, d));
        prm.k_new = k_new;
        prm.v_new = v_new;
        prm.k_inv = step.k_inv;
        prm.v_inv = step.v_inv;
        prm.qk_scale = softmax_scale * (cache_dtype == PKV_FP8_E4M3 ? k_scale : 1.f) * kLog2e;
        prm.v_scale = cache_dtype == PKV_FP8_E4M3 ? v_scale : 1.f;
        prm.cache_lens = n_seq <= kMaxCachedLens;
        const size_t lds = (size_t)(prm.cache_lens ? n_seq : 0) * sizeof(int);
        const int resident = resident_workgroups(kern, lds);
        const int cus = compute_units();
        if (resident <= 0 || cus <= 0) return fail(PKV_E_HIP, "%s: device query failed", fn);
        int64_t grid = std::min(cus, resident);
        if (grid * kWaves > kMaxWorkers) grid = kMaxWorkers / kWaves;
        prm.n_workers = (int)(grid * kWaves);
        prm.n_rec = 2 * prm.n_workers;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, static_cast<hipStream_t>(stream), prm);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(PKV_E_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
        // the merge's two views of the one launch: prefix rows and records,
        // and suffix rows with the same records and the suffix descriptors
        pa = prm;
        pa.S = n_groups;
        pb = prm;
        pb.out = out_b;
        pb.lse = lse_b;
        pb.lens = suffix_lens;
        pb.max_len = max_suffix_len;
        pb.S = S;
        pb.n_pre = 0;
        pb.desc = prm.desc + 2 * (size_t)n_groups * Hkv * qa.n_qg;
    }
    const unsigned grid = (unsigned)(((int64_t)S * Hq + kWaves - 1) / kWaves);
    auto st = static_cast<hipStream_t>(stream);
    if (d == 64)
        hipLaunchKernelGGL(shared_prefix_merge_kernel<64>, dim3(grid), dim3(kThreads), 0, st, pa, pb, out, M);
    else
        hipLaunchKernelGGL(shared_prefix_merge_kernel<128>, dim3(grid), dim3(kThreads), 0, st, pa, pb, out, M);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_E_HIP, "%s: merge launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}
