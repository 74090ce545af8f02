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
//  * Work item = (sequence i, kv head g, partition p); one 256-thread
//    workgroup (4 waves) per item. Waves take the item's 16-token chunks
//    round-robin, each keeping its own online-softmax state; the four states
//    are merged exactly through LDS at the end.
//  * Scores: S^T[16 tokens][16 heads] = K_chunk . Q^T with one MFMA chain
//    (bf16 16x16x32, or fp32 16x16x4 for an fp32 cache). The K operand rows
//    are tokens, so each lane's K fragment is 8 (bf16), 16 (fp8) or 4 (fp32)
//    consecutive channels of one token: 16-byte global loads, 64 contiguous
//    bytes per token row per instruction. Heads G..15 of the MFMA are padding.
//  * The MFMA result layout (lane = head + 16*token_group, 4 tokens per lane)
//    is exactly the B-operand layout of the P.V MFMA
//    (O^T[dims][heads] += V^T[dims][tokens] . P^T[tokens][heads]), so P never
//    leaves registers. V tiles are stored channel-major ([d][bs] per block and
//    head) so the V^T operand is 4 consecutive tokens of one channel.
//  * P stays float32 to the accuracy of the product: for bf16/fp8 caches it is
//    split into hi + lo bf16 parts and both are multiplied (two MFMAs), since
//    rounding P alone to bf16 costs ~2e-3 relative error.
//  * Softmax max and sum across the 4 token groups of a head use gfx950's
//    v_permlane16_swap / v_permlane32_swap (no LDS traffic).
//  * Split-K: partition p covers tokens [p*part, (p+1)*part); a sequence with
//    more than one partition writes (m, l, o) partials and a second kernel
//    merges them in fixed partition order. No atomics anywhere: results are
//    bit-reproducible.
//  * Work order: items of the last partition index first, so full-length
//    items of long sequences start early and short items fill the tail.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "common.h"

using pkv::fail;
using pkv::ok;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;

enum KvKind { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

// ----------------------------------------------------------------------------
// Small device helpers
// ----------------------------------------------------------------------------

// OCP E4M3 encoder written from the format definition: round to nearest,
// ties to even mantissa, |y| > 448 (and infinities) saturate to 448, NaN keeps
// its sign with the all-ones code, zero keeps its sign.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const float a = fabsf(y);
    if (!(a == a)) return sign | 0x7Fu;
    if (a > 448.0f) return sign | 0x7Eu;
    if (a < 0.015625f) {                        // below 2^-6: subnormal quantum 2^-9
        const float q = rintf(a * 512.0f);      // exact scaling, round half to even
        return sign | (uint32_t)q;              // q == 8 is the smallest normal, code 0x08
    }
    uint32_t ua = __float_as_uint(a);
    ua += 0x7FFFFu + ((ua >> 20) & 1u);         // round the 23-bit mantissa to 3 bits, RNE
    const uint32_t e = (ua >> 23) - 120u;       // rebias 127 -> 7
    const uint32_t m = (ua >> 20) & 7u;
    return sign | (e << 3) | m;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// Reduction over the 4 lanes that hold one head (lanes h, h+16, h+32, h+48).
__device__ __forceinline__ float head_max(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float head_sum(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Two fp8 codes (low or high 16 bits of `w`) -> two bf16 (exact).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 r = {(__bf16)a, (__bf16)b};          // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo_as_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_as_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

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
        const size_t vd = (((size_t)b * Hkv + h) * d + c) * bs + o;
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

// ----------------------------------------------------------------------------
// Paged decode attention
// ----------------------------------------------------------------------------

struct AttnParams {
    float* out;
    const void* q;
    const void* k;
    const void* v;
    const int32_t* tables;
    const int32_t* lens;
    float* ws;             // partials: o [S][Hq][n_part][D], m [...], l [...]
    int S, Hq, Hkv, G, P, max_blocks, max_len, part_tokens, n_part;
    float qk_scale;        // softmax_scale * k_scale * log2(e): scores in the log2 domain
    float v_scale;
};

// Per-cache-type register fragments of one 16-token chunk.
template <int KV, int D> struct Frag;

template <int D> struct Frag<KV_F32, D> {
    float4 k[D / 16];      // token r16, channels 16f + 4j4 .. +3
    float4 v[D / 16];      // channel 16s + r16, tokens 4j4 .. +3
};
template <int D> struct Frag<KV_BF16, D> {
    uint4 k[D / 32];       // token r16, channels 32s + 8j4 .. +7
    uint2 v[D / 16];       // channel 16s + r16, tokens 4j4 .. +3
};
template <int D> struct Frag<KV_FP8, D> {
    uint4 k[D / 64];       // token r16, channels 64f + 16j4 .. +15
    uint32_t v[D / 16];    // channel 16s + r16, tokens 4j4 .. +3
};

template <int KV> struct QFragT;
template <> struct QFragT<KV_F32> { using T = float4; };
template <> struct QFragT<KV_BF16> { using T = uint4; };
template <> struct QFragT<KV_FP8> { using T = uint4; };

// Number of 16-byte q loads per lane, matching the K fragment's channel map.
template <int KV, int D> constexpr int q_loads() { return KV == KV_F32 ? D / 16 : D / 32; }

template <int BS>
__device__ __forceinline__ int clamp_block(int b, int P) { return min(max(b, 0), P - 1); }

// Load the K and V fragments of the chunk starting at token `tc` (absolute).
// b0 is the physical block holding token tc; for bs 8, b1 holds token tc + 8.
template <int KV, int D, int BS>
__device__ __forceinline__ void load_chunk(Frag<KV, D>& f, const AttnParams& p, int b0, int b1,
                                           int tc, int g, int r16, int j4) {
    using E = typename std::conditional<KV == KV_F32, float,
              typename std::conditional<KV == KV_BF16, uint16_t, uint8_t>::type>::type;
    const E* kbase = static_cast<const E*>(p.k);
    const E* vbase = static_cast<const E*>(p.v);
    int bk, bv;            // physical blocks for this lane's K row and V tokens
    int ok_, ov;           // offsets within those blocks
    if constexpr (BS == 8) {
        bk = r16 < 8 ? b0 : b1;
        ok_ = r16 & 7;
        bv = j4 < 2 ? b0 : b1;
        ov = (4 * j4) & 7;
    } else {
        bk = b0;
        bv = b0;
        ok_ = (tc % BS) + r16;
        ov = (tc % BS) + 4 * j4;
    }
    const size_t tile = (size_t)BS * D;
    const E* krow = kbase + ((size_t)bk * p.Hkv + g) * tile + (size_t)ok_ * D;
    const E* vt = vbase + ((size_t)bv * p.Hkv + g) * tile + ov;
    if constexpr (KV == KV_F32) {
#pragma unroll
        for (int x = 0; x < D / 16; ++x)
            f.k[x] = *reinterpret_cast<const float4*>(krow + 16 * x + 4 * j4);
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            f.v[s] = *reinterpret_cast<const float4*>(vt + (size_t)(16 * s + r16) * BS);
    } else if constexpr (KV == KV_BF16) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
            f.k[s] = *reinterpret_cast<const uint4*>(krow + 32 * s + 8 * j4);
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            f.v[s] = *reinterpret_cast<const uint2*>(vt + (size_t)(16 * s + r16) * BS);
    } else {
#pragma unroll
        for (int x = 0; x < D / 64; ++x)
            f.k[x] = *reinterpret_cast<const uint4*>(krow + 64 * x + 16 * j4);
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            f.v[s] = *reinterpret_cast<const uint32_t*>(vt + (size_t)(16 * s + r16) * BS);
    }
}

// Scores of the chunk: S^T[token 4*j4+i][head r16] in acc[i].
template <int KV, int D>
__device__ __forceinline__ f32x4 chunk_scores(const Frag<KV, D>& f,
                                              const typename QFragT<KV>::T* qf) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KV == KV_F32) {
#pragma unroll
        for (int x = 0; x < D / 16; ++x) {
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.k[x].x, qf[x].x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.k[x].y, qf[x].y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.k[x].z, qf[x].z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.k[x].w, qf[x].w, acc, 0, 0, 0);
        }
    } else if constexpr (KV == KV_BF16) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.k[s]),
                                                          __builtin_bit_cast(bf16x8, qf[s]),
                                                          acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int x = 0; x < D / 64; ++x) {
            const uint32_t w[4] = {f.k[x].x, f.k[x].y, f.k[x].z, f.k[x].w};
            uint4 lo, hi;          // channels +0..7 and +8..15 as bf16
            lo.x = fp8x2_to_bf16x2<false>(w[0]); lo.y = fp8x2_to_bf16x2<true>(w[0]);
            lo.z = fp8x2_to_bf16x2<false>(w[1]); lo.w = fp8x2_to_bf16x2<true>(w[1]);
            hi.x = fp8x2_to_bf16x2<false>(w[2]); hi.y = fp8x2_to_bf16x2<true>(w[2]);
            hi.z = fp8x2_to_bf16x2<false>(w[3]); hi.w = fp8x2_to_bf16x2<true>(w[3]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, lo),
                                                          __builtin_bit_cast(bf16x8, qf[2 * x]),
                                                          acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, hi),
                                                          __builtin_bit_cast(bf16x8, qf[2 * x + 1]),
                                                          acc, 0, 0, 0);
        }
    }
    return acc;
}

// O^T += V^T . P^T for the chunk; `tail_mask` zeroes V of tokens >= t_end.
template <int KV, int D>
__device__ __forceinline__ void chunk_pv(Frag<KV, D>& f, const float p[4], f32x4* o,
                                         bool tail, int first_tok, int t_end) {
    if constexpr (KV == KV_F32) {
        if (tail) {
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                f.v[s].x = first_tok + 0 < t_end ? f.v[s].x : 0.f;
                f.v[s].y = first_tok + 1 < t_end ? f.v[s].y : 0.f;
                f.v[s].z = first_tok + 2 < t_end ? f.v[s].z : 0.f;
                f.v[s].w = first_tok + 3 < t_end ? f.v[s].w : 0.f;
            }
        }
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            o[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.v[s].x, p[0], o[s], 0, 0, 0);
            o[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.v[s].y, p[1], o[s], 0, 0, 0);
            o[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.v[s].z, p[2], o[s], 0, 0, 0);
            o[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.v[s].w, p[3], o[s], 0, 0, 0);
        }
    } else {
        // P = hi + lo, both bf16 (|lo| <= 2^-9 |P|, so the pair carries ~16 bits).
        const uint32_t h01 = pack_bf16x2(p[0], p[1]);
        const uint32_t h23 = pack_bf16x2(p[2], p[3]);
        const uint32_t l01 = pack_bf16x2(p[0] - bf16_lo_as_f32(h01), p[1] - bf16_hi_as_f32(h01));
        const uint32_t l23 = pack_bf16x2(p[2] - bf16_lo_as_f32(h23), p[3] - bf16_hi_as_f32(h23));
        const s16x4 phi = __builtin_bit_cast(s16x4, make_uint2(h01, h23));
        const s16x4 plo = __builtin_bit_cast(s16x4, make_uint2(l01, l23));
        // keep-masks for the two bf16 halves of each 32-bit word (tokens +0/+1, +2/+3)
        uint32_t m01 = 0xFFFFFFFFu, m23 = 0xFFFFFFFFu;
        uint32_t m8 = 0xFFFFFFFFu;
        if (tail) {
            m01 = (first_tok + 0 < t_end ? 0x0000FFFFu : 0u) | (first_tok + 1 < t_end ? 0xFFFF0000u : 0u);
            m23 = (first_tok + 2 < t_end ? 0x0000FFFFu : 0u) | (first_tok + 3 < t_end ? 0xFFFF0000u : 0u);
            m8 = (first_tok + 0 < t_end ? 0x000000FFu : 0u) | (first_tok + 1 < t_end ? 0x0000FF00u : 0u) |
                 (first_tok + 2 < t_end ? 0x00FF0000u : 0u) | (first_tok + 3 < t_end ? 0xFF000000u : 0u);
        }
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            uint2 vv;
            if constexpr (KV == KV_BF16) {
                vv = make_uint2(f.v[s].x & m01, f.v[s].y & m23);
            } else {
                const uint32_t w = f.v[s] & m8;   // masked codes become +0
                vv = make_uint2(fp8x2_to_bf16x2<false>(w), fp8x2_to_bf16x2<true>(w));
            }
            const s16x4 a = __builtin_bit_cast(s16x4, vv);
            o[s] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, phi, o[s], 0, 0, 0);
            o[s] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, plo, o[s], 0, 0, 0);
        }
    }
}

template <int KV, int D, int BS>
__global__ void __launch_bounds__(kThreads)
paged_attn_partition_kernel(AttnParams p) {
    extern __shared__ float smem[];          // m[4][16], l[4][16], o[4][G][D]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int r16 = lane & 15;               // MFMA row / column index
    const int j4 = lane >> 4;                // token group (scores) / k-group (operands)

    const int per = p.S * p.Hkv;
    const int part = p.n_part - 1 - (int)(blockIdx.x / per);   // last partitions first
    const int rem = (int)(blockIdx.x % per);
    const int i = rem / p.Hkv;
    const int g = rem - i * p.Hkv;
    const int G = p.G;

    const int L = min(p.lens[i], p.max_len);
    const int t0 = part * p.part_tokens;
    if (L <= 0) {                            // empty sequence: zero rows, once
        if (part == 0)
            for (int e = threadIdx.x; e < G * D; e += kThreads)
                p.out[((size_t)i * p.Hq + g * G) * D + e] = 0.f;
        return;
    }
    if (t0 >= L) return;
    const int t1 = min(L, t0 + p.part_tokens);
    const int n_chunks = (t1 - t0 + 15) >> 4;
    const bool split = L > p.part_tokens;
    const int32_t* __restrict__ row = p.tables + (size_t)i * p.max_blocks;

    // q fragment for head r16 (zero for padding heads), channel map = K's.
    using QF = typename QFragT<KV>::T;
    QF qf[q_loads<KV, D>()];
    {
        const bool live = r16 < G;
        const size_t qoff = ((size_t)i * p.Hq + g * G + (live ? r16 : 0)) * D;
#pragma unroll
        for (int x = 0; x < q_loads<KV, D>(); ++x) {
            int c;
            if constexpr (KV == KV_F32) c = 16 * x + 4 * j4;
            else if constexpr (KV == KV_BF16) c = 32 * x + 8 * j4;
            else c = 64 * (x >> 1) + 16 * j4 + 8 * (x & 1);
            QF val;
            if constexpr (KV == KV_F32)
                val = *reinterpret_cast<const float4*>(static_cast<const float*>(p.q) + qoff + c);
            else
                val = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.q) + qoff + c);
            if (!live) val = QF{};
            qf[x] = val;
        }
    }

    f32x4 o[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) o[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    auto process = [&](Frag<KV, D>& f, int c) {
        const int tc = t0 + 16 * c;
        const f32x4 sc = chunk_scores<KV, D>(f, qf);
        const bool tail = tc + 16 > t1;
        const int first_tok = tc + 4 * j4;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = sc[e] * p.qk_scale;
            if (tail && first_tok + e >= t1) x[e] = -INFINITY;
        }
        const float cm = head_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        const float m_new = fmaxf(m_run, cm);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float pr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pr[e] = __builtin_amdgcn_exp2f(x[e] - m_new);
        l_run = l_run * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
        m_run = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
            for (int s = 0; s < D / 16; ++s) o[s] *= alpha;
        }
        chunk_pv<KV, D>(f, pr, o, tail, first_tok, t1);
    };

    // This wave's chunks are c_k = wave + 4k, k < nk. Their block ids are
    // fetched once per 64 chunks (lane k holds chunk c_k's ids) and read back
    // with v_readlane, so no table load sits between a chunk's data loads.
    const int nk = n_chunks > wave ? (n_chunks - wave + kWaves - 1) / kWaves : 0;
    for (int kb = 0; kb < nk; kb += 64) {
        const int nw = min(64, nk - kb);
        int id0 = 0, id1 = 0;
        if (lane < nw) {
            const int tc = t0 + 16 * (wave + kWaves * (kb + lane));
            if constexpr (BS == 8) {
                id0 = row[tc / 8];
                id1 = tc + 8 < t1 ? row[tc / 8 + 1] : id0;   // only read entries that exist
            } else {
                id0 = row[tc / BS];
            }
            id0 = min(max(id0, 0), p.P - 1);
            id1 = min(max(id1, 0), p.P - 1);
        }
        auto chunk_tc = [&](int k) { return t0 + 16 * (wave + kWaves * (kb + k)); };
        // The scheduling barriers keep each prefetch at its place in program
        // order: nothing of the next chunk's math moves above it (which would
        // make the prefetch wait for that chunk's data).
        auto issue = [&](Frag<KV, D>& f, int k) {
            __builtin_amdgcn_sched_barrier(0);
            const int b0 = __builtin_amdgcn_readlane(id0, k);
            const int b1 = BS == 8 ? __builtin_amdgcn_readlane(id1, k) : b0;
            load_chunk<KV, D, BS>(f, p, b0, b1, chunk_tc(k), g, r16, j4);
            __builtin_amdgcn_sched_barrier(0);
        };
        // Two register buffers: chunk k+1 loads while chunk k computes. Every
        // load inside the loop is unconditional, so each wait the compiler
        // places covers exactly the buffer about to be used; the last one or
        // two chunks run after the loop.
        Frag<KV, D> fa, fb;
        issue(fa, 0);
        int k = 0;
        for (; k + 2 < nw; k += 2) {
            issue(fb, k + 1);
            process(fa, wave + kWaves * (kb + k));
            issue(fa, k + 2);
            process(fb, wave + kWaves * (kb + k + 1));
        }
        if (k + 1 < nw) {
            issue(fb, k + 1);
            process(fa, wave + kWaves * (kb + k));
            process(fb, wave + kWaves * (kb + k + 1));
        } else {
            process(fa, wave + kWaves * (kb + k));
        }
    }

    // ---- merge the 4 waves' states (exact rescaling to a common max) ----
    const float l_tot = head_sum(l_run);
    float* sm_m = smem;                       // [4][16]
    float* sm_l = smem + kWaves * 16;         // [4][16]
    float* sm_o = smem + 2 * kWaves * 16;     // [4][G][D]
    if (j4 == 0) {
        sm_m[wave * 16 + r16] = m_run;
        sm_l[wave * 16 + r16] = l_tot;
    }
    if (r16 < G) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            *reinterpret_cast<f32x4*>(sm_o + ((size_t)wave * G + r16) * D + 16 * s + 4 * j4) = o[s];
    }
    __syncthreads();

    for (int e = threadIdx.x; e < G * D; e += kThreads) {
        const int r = e / D;
        const int ch = e - r * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w * 16 + r]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float wt = __builtin_amdgcn_exp2f(sm_m[w * 16 + r] - M);
            num += wt * sm_o[((size_t)w * G + r) * D + ch];
            den += wt * sm_l[w * 16 + r];
        }
        const size_t h = (size_t)i * p.Hq + g * G + r;
        if (!split) {
            p.out[h * D + ch] = num / den * p.v_scale;
        } else {
            const size_t slot = h * p.n_part + part;
            p.ws[slot * D + ch] = num * p.v_scale;
            if (ch == 0) {
                const size_t nrow = (size_t)p.S * p.Hq * p.n_part;
                p.ws[nrow * D + slot] = M;
                p.ws[nrow * (D + 1) + slot] = den;
            }
        }
    }
}

// Merge the partitions of every split sequence: one wave per (sequence, head).
// Lanes hold one partition's (m, l) each (64 partitions per pass); the output
// loop keeps 8 partitions' loads in flight. Fixed order throughout.
template <int D>
__global__ void __launch_bounds__(256)
paged_attn_reduce_kernel(AttnParams p) {
    const int lane = threadIdx.x & 63;
    const size_t h = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);    // (i, head)
    if (h >= (size_t)p.S * p.Hq) return;
    const int i = (int)(h / p.Hq);
    const int L = min(p.lens[i], p.max_len);
    if (L <= p.part_tokens) return;            // written by the partition kernel
    const int n = (L + p.part_tokens - 1) / p.part_tokens;
    const size_t nrow = (size_t)p.S * p.Hq * p.n_part;
    const float* pm = p.ws + nrow * D + h * p.n_part;
    const float* pl = p.ws + nrow * (D + 1) + h * p.n_part;
    const float* po = p.ws + h * p.n_part * D;
    float M = -INFINITY;
    for (int k0 = 0; k0 < n; k0 += 64)
        if (k0 + lane < n) M = fmaxf(M, pm[k0 + lane]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    constexpr int PER = D / 64;
    float num[PER] = {};
    float den = 0.f;
    for (int k0 = 0; k0 < n; k0 += 64) {
        const int kn = min(64, n - k0);
        const float wl = k0 + lane < n ? __builtin_amdgcn_exp2f(pm[k0 + lane] - M) : 0.f;
        den += wl * (k0 + lane < n ? pl[k0 + lane] : 0.f);
        for (int k = 0; k < kn; k += 8) {
            float ov[8][PER];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int x = 0; x < PER; ++x)
                    ov[u][x] = k + u < kn ? po[(size_t)(k0 + k + u) * D + lane + 64 * x] : 0.f;
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
}

// ----------------------------------------------------------------------------
// Dispatch
// ----------------------------------------------------------------------------

using AttnKernel = void (*)(AttnParams);

template <int KV, int D>
AttnKernel pick_bs(int bs) {
    switch (bs) {
        case 8: return paged_attn_partition_kernel<KV, D, 8>;
        case 16: return paged_attn_partition_kernel<KV, D, 16>;
        case 32: return paged_attn_partition_kernel<KV, D, 32>;
    }
    return nullptr;
}

template <int KV>
AttnKernel pick_d(int d, int bs) {
    return d == 64 ? pick_bs<KV, 64>(bs) : pick_bs<KV, 128>(bs);
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
    if (!pkv::is_pow2_block(bs)) return fail(PKV_E_INVALID, "kv_cache_write: bs=%d not in {8,16,32}", bs);
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

extern "C" size_t pkv_paged_decode_attn_workspace_size(int32_t S, int32_t Hq, int32_t d,
                                                       int32_t max_context_len,
                                                       int32_t partition_size) {
    if (S <= 0 || Hq <= 0 || d <= 0) return 0;
    const int64_t n = n_partitions(max_context_len, partition_size);
    if (n <= 1) return 0;
    return (size_t)S * (size_t)Hq * (size_t)n * (size_t)(d + 2) * sizeof(float);
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
    if (S < 0 || Hq <= 0 || Hkv <= 0) return fail(PKV_E_INVALID, "paged_decode_attn: S=%d Hq=%d Hkv=%d", S, Hq, Hkv);
    if (Hq % Hkv != 0) return fail(PKV_E_INVALID, "paged_decode_attn: Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
    const int32_t G = Hq / Hkv;
    if (G > 16) return fail(PKV_E_INVALID, "paged_decode_attn: Hq/Hkv=%d > 16", G);
    if (!pkv::is_head_dim(d)) return fail(PKV_E_INVALID, "paged_decode_attn: d=%d not in {64,128}", d);
    if (!pkv::is_pow2_block(bs)) return fail(PKV_E_INVALID, "paged_decode_attn: bs=%d not in {8,16,32}", bs);
    if (P <= 0 || max_blocks <= 0) return fail(PKV_E_INVALID, "paged_decode_attn: P=%d max_blocks=%d", P, max_blocks);
    if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks * bs)
        return fail(PKV_E_INVALID, "paged_decode_attn: max_context_len=%d outside [0, max_blocks*bs=%lld]",
                    max_context_len, (long long)max_blocks * bs);
    int kv;
    if (q_dtype == PKV_F32 && cache_dtype == PKV_F32) kv = KV_F32;
    else if (q_dtype == PKV_BF16 && cache_dtype == PKV_BF16) kv = KV_BF16;
    else if (q_dtype == PKV_BF16 && cache_dtype == PKV_FP8_E4M3) kv = KV_FP8;
    else return fail(PKV_E_INVALID, "paged_decode_attn: unsupported q/cache dtypes %d/%d", q_dtype, cache_dtype);
    if (partition_size < 0 || partition_size % 32 != 0)
        return fail(PKV_E_INVALID, "paged_decode_attn: partition_size=%d not 0 or a multiple of 32", partition_size);
    if (!std::isfinite(softmax_scale)) return fail(PKV_E_INVALID, "paged_decode_attn: softmax_scale not finite");
    if (kv == KV_FP8 && !(std::isfinite(k_scale) && std::isfinite(v_scale)))
        return fail(PKV_E_INVALID, "paged_decode_attn: fp8 scales not finite");
    if (S == 0) return ok();
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
        return fail(PKV_E_INVALID, "paged_decode_attn: NULL pointer");
    const int64_t n_part = n_partitions(max_context_len, partition_size);
    const size_t need = pkv_paged_decode_attn_workspace_size(S, Hq, d, max_context_len, partition_size);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(PKV_E_WORKSPACE, "paged_decode_attn: workspace %zu bytes, need %zu", workspace_bytes, need);
    const int64_t grid = n_part * (int64_t)S * Hkv;
    if (grid > 0x7FFFFFFFLL) return fail(PKV_E_INVALID, "paged_decode_attn: grid too large");

    AttnParams prm;
    prm.out = out;
    prm.q = q;
    prm.k = k_cache;
    prm.v = v_cache;
    prm.tables = block_tables;
    prm.lens = context_lens;
    prm.ws = static_cast<float*>(workspace);
    prm.S = S;
    prm.Hq = Hq;
    prm.Hkv = Hkv;
    prm.G = G;
    prm.P = P;
    prm.max_blocks = max_blocks;
    prm.max_len = max_context_len;
    // single pass: one partition long enough for any sequence (whole chunks)
    prm.part_tokens = partition_size > 0 ? partition_size : ((max(max_context_len, 1) + 31) / 32) * 32;
    prm.n_part = (int)n_part;
    const float ks = kv == KV_FP8 ? k_scale : 1.f;
    prm.qk_scale = softmax_scale * ks * kLog2e;
    prm.v_scale = kv == KV_FP8 ? v_scale : 1.f;

    AttnKernel kern = kv == KV_F32 ? pick_d<KV_F32>(d, bs)
                    : kv == KV_BF16 ? pick_d<KV_BF16>(d, bs) : pick_d<KV_FP8>(d, bs);
    const size_t lds = (size_t)(2 * kWaves * 16 + kWaves * G * d) * sizeof(float);
    auto st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, st, prm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_E_HIP, "paged_decode_attn: launch failed: %s", hipGetErrorString(e));
    if (n_part > 1) {
        const unsigned rgrid = (unsigned)(((int64_t)S * Hq + 3) / 4);
        if (d == 64)
            hipLaunchKernelGGL(paged_attn_reduce_kernel<64>, dim3(rgrid), dim3(256), 0, st, prm);
        else
            hipLaunchKernelGGL(paged_attn_reduce_kernel<128>, dim3(rgrid), dim3(256), 0, st, prm);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(PKV_E_HIP, "paged_decode_attn: reduce launch failed: %s", hipGetErrorString(e));
    }
    return ok();
}
