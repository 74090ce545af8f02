/*
 * pkv.h - C ABI of libpkv.so: paged decode attention for AMD Instinct MI355X
 * (gfx950), the KV-cache write, and the host-side block allocator.
 *
 * What is computed follows the pages' statement of PagedAttention:
 *  - "03 · PagedAttention" (sunilkunchoor.github.io), sections "Blocks and
 *    block tables", "The part the analogy hides: the kernel", "Sharing:
 *    copy-on-write" and "When the pool runs dry";
 *  - "PagedAttention" daily term (mlapandio.dev), the decode-step figure
 *    (gather K and V through the block table, score q against every key,
 *    write the new K and V into the current block) and "Pros" (a plain free
 *    list; not an approximation);
 *  - "Serving: vLLM and PagedAttention" (henryfzh-note.com), section 2.2
 *    (block table as page table, last-block fill, coalesced in-block reads).
 *
 * Conventions for every function:
 *  - The return value is a pkv_status; PKV_OK (0) is success. On any other
 *    value pkv_last_error() returns a message for the calling thread.
 *  - Every argument check runs before any HIP call: an invalid call returns
 *    PKV_E_INVALID / PKV_E_WORKSPACE synchronously and launches nothing.
 *  - Device functions take device pointers the caller owns, enqueue their
 *    kernels on `stream` (a hipStream_t; NULL is the default stream), never
 *    allocate device memory and never synchronise. A launch failure returns
 *    PKV_E_HIP with HIP's error string.
 *  - Host allocator functions run on the CPU only and are not thread-safe:
 *    the caller serialises calls on one allocator.
 *
 * Notation: S sequences, Hq query heads, Hkv kv heads (Hq % Hkv == 0, query
 * head h uses kv head h / (Hq/Hkv)), d head dim, bs tokens per block, P
 * blocks in the pool, L_i the context length of sequence i.
 *
 * Pool layout (the pages fix none; tokens of a block are contiguous in both):
 *   k_cache[P][Hkv][bs][d]           each (block, kv head) tile token-major
 *   v_cache[P][Hkv][bs/vs][d][vs]    each (block, kv head) tile in sub-tiles of
 *                                    vs = min(bs, 16) tokens, each channel-major
 *                                    (for bs <= 16: v_cache[P][Hkv][d][bs])
 * A 16-token chunk of a block then reads whole rows of K and one whole V
 * sub-tile, whatever the block size.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_OK = 0,
    PKV_E_INVALID = 1,    /* bad argument; nothing was changed or launched      */
    PKV_E_WORKSPACE = 2,  /* workspace missing or smaller than required          */
    PKV_E_NO_BLOCKS = 3,  /* pool exhausted; allocator state unchanged           */
    PKV_E_NOT_FOUND = 4,  /* unknown sequence id                                 */
    PKV_E_STATE = 5,      /* operation conflicts with current state              */
    PKV_E_HIP = 6         /* a HIP call or kernel launch failed                  */
} pkv_status;

typedef enum {
    PKV_F32 = 0,          /* IEEE binary32                                       */
    PKV_BF16 = 1,         /* bfloat16 (upper half of binary32)                   */
    PKV_FP8_E4M3 = 2      /* OCP 8-bit E4M3 ("fn": no inf, NaN = S.1111.111)     */
} pkv_dtype;

/* partition_size value selecting the balanced split (see pkv_paged_decode_attn). */
#define PKV_PARTITION_BALANCED (-1)

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* pkv_last_error(void);
/* Library version string. */
const char* pkv_version(void);

/* ------------------------------------------------------------------------ */
/* Device operations                                                         */
/* ------------------------------------------------------------------------ */

/*
 * KV-cache write: scatter each new token's K and V into its physical slot
 * ("PagedAttention" daily term, decode-step figure: "write the new K and V
 * into the current block").
 *
 * For each t < T with 0 <= slot_mapping[t] < P*bs: (b, o) = divmod(slot, bs);
 *   k_cache[b][h][o][c]                 = cvt(k_new[t][h][c])
 *   v_cache[b][h][o / vs][c][o % vs]    = cvt(v_new[t][h][c])     (vs = min(bs, 16);
 *                                         for bs <= 16 that is v_cache[b][h][c][o])
 * for all h < Hkv, c < d. Any other slot value (-1 by convention) skips the
 * token. Every other byte of the pools is left unchanged.
 *
 * cvt: a bit copy when src_dtype == cache_dtype (F32->F32, BF16->BF16);
 * for BF16 -> FP8_E4M3: e4m3(float32(x) * inv_scale), rounded to nearest with
 * ties to even, |value| > 448 (and +-inf) saturating to +-448, NaN -> 0x7F
 * with its sign, the sign of zero kept. k_inv_scale / v_inv_scale are used only
 * for an FP8 cache and must then be finite and > 0.
 *
 * k_new, v_new: [T][Hkv][d] in src_dtype. slot_mapping: int64 [T].
 * Two tokens with the same slot race (the result is one of them).
 * T == 0 is a no-op. Requires T >= 0, Hkv > 0, d in {64, 128},
 * bs in {8, 16, 32, 64, 128}, P > 0.
 */
pkv_status pkv_kv_cache_write(const void* k_new, const void* v_new,
                              void* k_cache, void* v_cache,
                              const int64_t* slot_mapping,
                              int32_t T, int32_t Hkv, int32_t d, int32_t bs, int32_t P,
                              pkv_dtype src_dtype, pkv_dtype cache_dtype,
                              float k_inv_scale, float v_inv_scale, void* stream);

/*
 * Bytes of workspace pkv_paged_decode_attn needs for these sizes:
 *  - partition_size == PKV_PARTITION_BALANCED: R + 2 * S * Hkv * 4, where
 *    R = 2 * 4096 * (Hq/Hkv) * (d + 2) * 4 rounded up to a multiple of 256
 *    (two partial records per wave, at most 4096 waves) and the rest holds
 *    one (first record, record count) descriptor per (sequence, kv head);
 *  - otherwise 0 when no sequence can span more than one partition
 *    (partition_size == 0 or max_context_len <= partition_size), else
 *    S * Hq * n_part * (d + 2) * 4 with n_part = ceil(max_context_len / partition_size).
 * Returns 0 for invalid sizes.
 */
size_t pkv_paged_decode_attn_workspace_size(int32_t S, int32_t Hq, int32_t Hkv, int32_t d,
                                            int32_t max_context_len,
                                            int32_t partition_size);

/*
 * Paged decode attention: one new query per sequence attends to the
 * sequence's L_i cached tokens, gathered block by block through the block
 * table ("03 · PagedAttention", "The part the analogy hides: the kernel";
 * "PagedAttention" daily term, decode-step figure). The result is the
 * ordinary attention over the tokens in logical order:
 *
 *   s_t   = softmax_scale * k_scale * sum_c q[i][h][c] * K_i[t][g][c]
 *   out[i][h][c] = v_scale * sum_t exp(s_t - max s) V_i[t][g][c] / sum_t exp(s_t - max s)
 *
 * with g = h / (Hq / Hkv), K_i[t] the token at position t (0-based) of
 * sequence i: logical block t / bs at offset t % bs, physical block
 * block_tables[i][t / bs]. For an FP8 cache K and V are the decoded E4M3
 * values and k_scale / v_scale the per-tensor scales; for F32 and BF16
 * caches k_scale and v_scale are ignored (taken as 1).
 *
 * out:           float32 [S][Hq][d]; a row with L_i <= 0 is written as 0.
 * q:             [S][Hq][d] in q_dtype.
 * k_cache, v_cache: the pools (layout above) in cache_dtype.
 * block_tables:  int32 [S][max_blocks]; entries j >= ceil(L_i/bs) are never read.
 * context_lens:  int32 [S] (device); the caller guarantees
 *                L_i <= max_context_len. Lengths above it are clamped to it and
 *                block ids outside [0, P) are clamped into range, so the kernel
 *                never reads outside the table row or the pool; the output of
 *                such a sequence is then unspecified.
 * Supported (q_dtype, cache_dtype): (F32, F32), (BF16, BF16), (BF16, FP8_E4M3).
 * Requires S > 0, Hkv > 0, Hq % Hkv == 0, 1 <= Hq/Hkv <= 16, d in {64, 128},
 * bs in {8, 16, 32, 64, 128}, P > 0, max_blocks > 0, 0 <= max_context_len <=
 * min(max_blocks * bs, 2^30), softmax_scale finite; for FP8 finite k_scale,
 * v_scale.
 *
 * partition_size selects how sequences are split across workgroups (split-K);
 * partial results are always merged exactly (running max, sum of
 * exponentials, unnormalised output) in a fixed order:
 *  - 0: every (sequence, kv head) in one pass, no split;
 *  - a positive multiple of 32: fixed partitions of that many tokens; a
 *    sequence longer than partition_size is split into
 *    ceil(L_i / partition_size) partitions;
 *  - PKV_PARTITION_BALANCED: all (sequence, kv head, 16-token chunk) work,
 *    with each (sequence, kv head) weighted by 1, 2 or 4 extra chunks (fp32,
 *    bf16, fp8 caches) for its fixed costs, is cut into equal contiguous
 *    shares, one per wave of a grid of one
 *    workgroup per compute unit; a long sequence is split wherever the shares
 *    cut it, and every wave finishes at about the same time.
 * workspace: device memory of at least
 * pkv_paged_decode_attn_workspace_size(...) bytes (may be NULL when that is 0);
 * its contents on entry do not matter. Calls that overlap in time must not
 * share a workspace.
 *
 * The result is deterministic for a given GPU: no atomics, fixed reduction
 * order (the balanced split depends on the number of compute units).
 */
pkv_status pkv_paged_decode_attn(float* out, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int32_t S, int32_t Hq, int32_t Hkv, int32_t d, int32_t bs,
                                 int32_t P, int32_t max_blocks, int32_t max_context_len,
                                 float softmax_scale, float k_scale, float v_scale,
                                 pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                 int32_t partition_size,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step in one call: write each sequence's new token and attend
 * over the context including it, as a single launch of the attention kernel
 * ("PagedAttention" daily term, decode-step figure: gather, score and the
 * write of the new K/V in one launch for the batch). The result equals
 * pkv_kv_cache_write of token i at position L_i - 1 of sequence i (its slot
 * taken from block_tables) followed by pkv_paged_decode_attn with
 * PKV_PARTITION_BALANCED. The new token's slot may hold anything on entry:
 * the kernel takes that token's K/V from k_new/v_new (encoded as the write
 * encodes them) and writes the slot concurrently.
 *
 * k_new, v_new:  [S][Hkv][d], F32 for an F32 cache, BF16 for BF16 and
 *                FP8_E4M3 caches; k_inv_scale / v_inv_scale are the fp8
 *                write's inverse scales (ignored otherwise).
 * Other arguments and the workspace as for pkv_paged_decode_attn with
 * partition_size = PKV_PARTITION_BALANCED (same workspace size). Sequences with
 * L_i <= 0 get zero rows and no write. The new token's block must not be
 * shared with another sequence (copy-on-write first: pkv_copy_blocks).
 */
pkv_status pkv_paged_decode_step(float* out, const void* q, const void* k_new, const void* v_new,
                                 void* k_cache, void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int32_t S, int32_t Hq, int32_t Hkv, int32_t d, int32_t bs,
                                 int32_t P, int32_t max_blocks, int32_t max_context_len,
                                 float softmax_scale, float k_scale, float v_scale,
                                 float k_inv_scale, float v_inv_scale,
                                 pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Planned decode step. The balanced split of pkv_paged_decode_step (the
 * decode attention work cut into equal cost-weighted ranges, one per wave)
 * depends only on the context lengths, so a caller that holds them on the
 * host -- as the scheduler does when it builds the block tables and the slot
 * mapping ("03 · PagedAttention", "Blocks and block tables") -- can compute it
 * there, once per step, with pkv_build_paged_decode_plan. The planned kernel
 * then reads each wave's chunk list from the plan instead of scanning the
 * lengths and searching its positions on the device, and the merge reads the
 * plan's descriptors. It still walks the block tables, gathers every K/V
 * tile and writes the new tokens. Its pools are those of
 * pkv_paged_decode_step byte for byte, and so are its outputs (or, without
 * new tokens, those of pkv_paged_decode_attn with the balanced split) when
 * both run the same number of waves: one 4-wave workgroup per compute unit.
 * Where a 16-token chunk is 2 KiB or less (fp8 at d 64) the planned kernel
 * runs two workgroups per compute unit; its split into pieces then differs
 * and the outputs agree to rounding.
 *
 * pkv_paged_decode_plan_workers: the number of waves the planned kernel runs
 * on the current device for this head dim, block size and cache type (the
 * plan is built for it); -1 on an invalid argument or a failed device query.
 */
int32_t pkv_paged_decode_plan_workers(int32_t d, int32_t bs, pkv_dtype cache_dtype);

/*
 * Build the plan on the host. context_lens: host int32 [S], the same lengths
 * the call passes on the device (clamped to max_context_len as the kernels
 * clamp them); n_workers from pkv_paged_decode_plan_workers. plan: caller-
 * owned host memory of plan_bytes; *plan_bytes_needed (when not NULL) gets
 * the size the plan needs, and a call with plan NULL or too small returns
 * PKV_E_WORKSPACE after setting it. The plan is int32 words: a 16-word header
 * (magic "PKVP", version, n_workers, waves used, S, Hkv, segment cost, entries
 * per wave, max_context_len, d, cache kind, four window words that are zero
 * here, flags), then per wave its chunk entries
 * {sequence, kv head | flags << 16, chunk index, L} (unused: sequence -1),
 * then one (first record, record count) descriptor per (sequence, kv head).
 * Requires S > 0, Hkv > 0, d in {64, 128}, n_workers > 0 and
 * 0 <= max_context_len <= 2^30; PKV_E_INVALID otherwise.
 */
pkv_status pkv_build_paged_decode_plan(const int32_t* context_lens, int32_t S, int32_t Hkv, int32_t d,
                                       pkv_dtype cache_dtype, int32_t max_context_len, int32_t n_workers,
                                       void* plan, size_t plan_bytes, size_t* plan_bytes_needed);

/*
 * Mark in a decode plan whether its batch shares physical blocks: whether any
 * block id appears more than once among the blocks the sequences read (the
 * first ceil(min(L_i, max_context_len) / bs) entries of each table row) --
 * the prefix blocks of beams or of sequences forked from one prompt ("03 ·
 * PagedAttention", "Sharing: copy-on-write": a shared block is listed by
 * every table that uses it). block_tables: host int32 [S][max_blocks], the
 * tables the call passes on the device; context_lens: host int32 [S]. Sets
 * or clears the plan's flags word (header word 15) and *shared (when not
 * NULL). A plan so marked runs its decode kernels with cacheable K/V loads,
 * so that the waves reading one shared block can meet in L2 instead of each
 * reading it from HBM; unmarked plans keep streaming (evict-first) loads,
 * which are faster when every block is read once. The result is the same
 * either way, bit for bit; upload the plan after marking it.
 */
pkv_status pkv_plan_mark_shared_blocks(void* plan, size_t plan_bytes, const int32_t* block_tables,
                                       const int32_t* context_lens, int32_t S, int32_t max_blocks, int32_t bs,
                                       int32_t* shared);

/*
 * The plan of a query window (pkv_paged_multi_query_attn_planned): n_q
 * queries per sequence, query j at position L_i - n_q + j seeing the tokens
 * up to it, as in pkv_paged_multi_query_attn ("Serving: vLLM and
 * PagedAttention", sections 2.4 and 2.7). The (query,
 * head) pairs of each kv head are cut into n_qg groups of qgs queries, qgs =
 * min(n_q, max(1, 16 * T / G)) with G = Hq / Hkv and T = 1 16-column MFMA
 * tile per group when n_q * G <= 16, else T = 2 (the grouping of
 * pkv_paged_multi_query_attn), and every group is a segment of the balanced
 * split with the sequence's whole chunk list, the kv head's groups next to
 * each other. The
 * layout is that of the decode plan, with header words 11..14 = n_q, G, qgs,
 * n_qg (zero in a decode plan), entry field g2 = kv head * n_qg + group, and
 * one descriptor per (sequence, kv head, group). n_workers from
 * pkv_paged_decode_plan_workers. Requires n_q > 0, 1 <= Hq/Hkv <= 16 and what
 * pkv_build_paged_decode_plan requires.
 */
pkv_status pkv_build_paged_window_plan(const int32_t* context_lens, int32_t S, int32_t n_q, int32_t Hq,
                                       int32_t Hkv, int32_t d, pkv_dtype cache_dtype, int32_t max_context_len,
                                       int32_t n_workers, void* plan, size_t plan_bytes,
                                       size_t* plan_bytes_needed);

/* Workspace bytes of a planned window call: 2 * n_workers * cols * (d + 2) * 4
 * rounded up to a multiple of 256, cols = G * qgs (the partial records); 0
 * for invalid sizes. */
size_t pkv_paged_window_plan_workspace_size(int32_t n_workers, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t d);

/*
 * pkv_paged_multi_query_attn with its work split by a window plan built on
 * the host (pkv_build_paged_window_plan), in the planned kernel. Arguments,
 * layouts and result as for pkv_paged_multi_query_attn, plus plan_host (its
 * header is checked against the call: S, n_q, Hq/Hkv, Hkv, d, cache type,
 * max_context_len and this device's wave count) and plan_dev (a device copy
 * of all plan_bytes, read by the kernels). Both calls group the columns alike
 * and, with the same number of waves, split the work alike, so their outputs
 * are equal bit for bit. A window of several groups per kv head reads K/V
 * with cacheable loads (its groups read the same blocks). The workspace
 * (pkv_paged_window_plan_workspace_size bytes) need not be initialised; calls
 * that overlap in time must not share it.
 */
pkv_status pkv_paged_multi_query_attn_planned(float* out, const void* q, const void* k_cache, const void* v_cache,
                                              const int32_t* block_tables, const int32_t* context_lens, int32_t S,
                                              int32_t n_q, int32_t Hq, int32_t Hkv, int32_t d, int32_t bs,
                                              int32_t P, int32_t max_blocks, int32_t max_context_len,
                                              float softmax_scale, float k_scale, float v_scale, pkv_dtype q_dtype,
                                              pkv_dtype cache_dtype, const void* plan_host, const void* plan_dev,
                                              size_t plan_bytes, void* workspace, size_t workspace_bytes,
                                              void* stream);

/* Workspace bytes of a planned call: 2 * n_workers * (Hq/Hkv) * (d + 2) * 4,
 * rounded up to a multiple of 256 (the partial records); 0 for invalid sizes. */
size_t pkv_paged_decode_plan_workspace_size(int32_t n_workers, int32_t Hq, int32_t Hkv, int32_t d);

/*
 * The planned step. Arguments as for pkv_paged_decode_step, plus the plan:
 * plan_host (its host copy; only the header is read, to check that it was
 * built for these S, Hkv, d, cache type and max_context_len and for this
 * device's wave count) and plan_dev (a device copy of all plan_bytes, read by
 * the kernels; the caller uploads it). k_new and v_new may both be NULL: the
 * attention alone, with no write. Contents of the workspace on entry do not
 * matter; calls that overlap in time must not share it. attn_done_event:
 * NULL, or a hipEvent_t that the call records on stream after the attention
 * kernel and before the merge kernel, so that a caller can time the two
 * apart (the call's work is the same either way). Over an FP8_E4M3 cache the
 * wave that holds a sequence's last chunk writes that token and then reads
 * it back from the pool instead of taking it from k_new/v_new; the result
 * is the same, bit for bit, except for a token whose table entry lies
 * outside [0, P): it is not stored, and that sequence's output is then
 * unspecified (as for any out-of-range entry).
 */
pkv_status pkv_paged_decode_step_planned(float* out, const void* q, const void* k_new, const void* v_new,
                                         void* k_cache, void* v_cache,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         int32_t S, int32_t Hq, int32_t Hkv, int32_t d, int32_t bs,
                                         int32_t P, int32_t max_blocks, int32_t max_context_len,
                                         float softmax_scale, float k_scale, float v_scale,
                                         float k_inv_scale, float v_inv_scale,
                                         pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                         const void* plan_host, const void* plan_dev, size_t plan_bytes,
                                         void* workspace, size_t workspace_bytes, void* stream,
                                         void* attn_done_event);

/*
 * pkv_paged_decode_step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step, the same kernels and the same result as
 * pkv_paged_decode_step, with no workspace argument. The balanced split's
 * partial records and segment descriptors go to a file-scope device array of
 * PKV_STEP_SCRATCH_BYTES (16 MiB) that every GPU the library runs on holds
 * from the library's load until the process ends; the call allocates nothing.
 *
 * A call needs R + 2 * S * Hkv * 4 bytes of it, R = 2 * W * (Hq/Hkv) * (d + 2) * 4
 * rounded up to a multiple of 256, with W = 4 waves per compute unit (1024 on
 * MI355X): Hq/Hkv up to 8 at d 128 and 16 at d 64 fit, for up to hundreds of
 * thousands of (sequence, kv head) pairs. A call that needs more returns
 * PKV_E_WORKSPACE (nothing launched); pkv_paged_decode_step takes any size.
 *
 * Every call on one GPU uses that GPU's one array, and the array keeps what
 * the last call left in it (nothing in it needs clearing: each call writes
 * every record and descriptor it reads). Calls whose execution overlaps on one
 * GPU (different streams, no ordering between them) race on the array and
 * may return wrong results: serialise them. Arguments and result otherwise
 * exactly as for pkv_paged_decode_step.
 */
#define PKV_STEP_SCRATCH_BYTES (16u << 20)
size_t pkv_paged_decode_step_scratch_bytes(void);
pkv_status pkv_paged_decode_step_noalloc(float* out, const void* q, const void* k_new, const void* v_new,
                                         void* k_cache, void* v_cache,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         int32_t S, int32_t Hq, int32_t Hkv, int32_t d, int32_t bs,
                                         int32_t P, int32_t max_blocks, int32_t max_context_len,
                                         float softmax_scale, float k_scale, float v_scale,
                                         float k_inv_scale, float v_inv_scale,
                                         pkv_dtype q_dtype, pkv_dtype cache_dtype, void* stream);

/*
 * Bytes of workspace pkv_paged_multi_query_attn needs: R + 2 * S * Hkv * n_qg * 4
 * with G = Hq/Hkv, T = 1 column tile when n_q * G <= 16 and otherwise T = 2,
 * qgs = min(n_q, max(1, 16 * T / G)) queries per
 * pass, n_qg = ceil(n_q / qgs) passes and R = 2 * 4096 * G * qgs * (d + 2) * 4
 * rounded up to a multiple of 256. Returns 0 for invalid sizes.
 */
size_t pkv_paged_multi_query_attn_workspace_size(int32_t S, int32_t n_q, int32_t Hq, int32_t Hkv,
                                                 int32_t d);

/*
 * Paged attention for a window of n_q consecutive new queries per sequence,
 * causal inside the window: the chunks of chunked prefill and the candidate
 * windows of speculative decoding, which reuse the decode gather ("Serving:
 * vLLM and PagedAttention", sections 2.4 and 2.7). Query j (0-based) of
 * sequence i sits at position L_i - n_q + j and attends to the cached tokens at
 * positions 0 .. L_i - n_q + j (the window's own K/V are written beforehand,
 * e.g. by pkv_kv_cache_write with one slot per query token):
 *
 *   out[i][j][h][c] = v_scale * sum_{t <= L_i - n_q + j} exp(s_t - max s) V_i[t][g][c]
 *                              / sum_{t <= L_i - n_q + j} exp(s_t - max s)
 *
 * with s_t, g and the pools as in pkv_paged_decode_attn. n_q = 1 is exactly
 * decode attention.
 *
 * out: float32 [S][n_q][Hq][d]; q: [S][n_q][Hq][d] in q_dtype; the other
 * arguments as for pkv_paged_decode_attn, which this shares its kernels with:
 * the balanced split is always used, and workspace must hold
 * pkv_paged_multi_query_attn_workspace_size(S, n_q, Hq, Hkv, d) bytes.
 * Requires 1 <= n_q <= 4096 and, per sequence, L_i >= n_q or L_i <= 0 (zero
 * rows); rows of a query that sees no token are otherwise unspecified.
 * The G query heads of a kv head and up to qgs queries of the window share
 * each pass over the sequence's blocks, as T tiles of 16 MFMA columns (T and
 * qgs as for the workspace size); a longer window takes ceil(n_q / qgs)
 * passes.
 */
pkv_status pkv_paged_multi_query_attn(float* out, const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t S, int32_t n_q, int32_t Hq, int32_t Hkv, int32_t d,
                                      int32_t bs, int32_t P, int32_t max_blocks,
                                      int32_t max_context_len, float softmax_scale, float k_scale,
                                      float v_scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention over sequences that share leading blocks (beams, parallel
 * samples: several block tables list the same physical blocks for a common
 * prefix, "03 · PagedAttention", "Sharing: copy-on-write"; "PagedAttention"
 * daily term, "Pros"). The pages share such blocks in memory; these three
 * calls also read them once per step instead of once per sequence:
 *
 *   1. pkv_paged_shared_prefix_attn: for each group of M sequences, attention of
 *      all M queries over the group's shared prefix, every query seeing every
 *      prefix token (one pass over the prefix blocks serves G*M columns);
 *   2. pkv_paged_decode_attn_lse: each sequence's attention over its own
 *      tokens after the prefix (tables and lengths of the suffixes);
 *   3. pkv_merge_attn_states: the exact combination of the two states.
 *
 * For a row (sequence i, head h) the result is the decode attention of
 * pkv_paged_decode_attn over all L_i tokens: with A = the prefix tokens and
 * B = the suffix tokens, out = (2^la o_A + 2^lb o_B) / (2^la + 2^lb), where
 * o_X and lx = log2 sum_{t in X} exp(s_t) (the scores s_t as in
 * pkv_paged_decode_attn, including k_scale) are what calls 1 and 2 return.
 */

/* Call 2: pkv_paged_decode_attn with the balanced split (same workspace size,
 * partition_size PKV_PARTITION_BALANCED) that also writes lse[S][Hq] (float32,
 * device): log2 of each row's sum of exp(s_t) over its tokens; -inf for a
 * sequence with L_i <= 0 (whose row is zero). */
pkv_status pkv_paged_decode_attn_lse(float* out, float* lse, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t S, int32_t Hq,
                                     int32_t Hkv, int32_t d, int32_t bs, int32_t P,
                                     int32_t max_blocks, int32_t max_context_len,
                                     float softmax_scale, float k_scale, float v_scale,
                                     pkv_dtype q_dtype, pkv_dtype cache_dtype, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Call 1: n_groups groups of M queries each. q: [n_groups][M][Hq][d] (query m
 * of group g is the g*M + m-th sequence's q); prefix_tables [n_groups]
 * [max_blocks] and prefix_lens [n_groups] describe each group's shared prefix
 * (a whole number of blocks). out: float32 [n_groups][M][Hq][d]; lse:
 * float32 [n_groups][M][Hq] as for call 2. Every query attends to all
 * prefix_lens[g] tokens (no causal mask). workspace as
 * pkv_paged_multi_query_attn_workspace_size(n_groups, M, Hq, Hkv, d); other
 * arguments and limits as for pkv_paged_multi_query_attn (1 <= M <= 4096). */
pkv_status pkv_paged_shared_prefix_attn(float* out, float* lse, const void* q, const void* k_cache,
                                        const void* v_cache, const int32_t* prefix_tables,
                                        const int32_t* prefix_lens, int32_t n_groups, int32_t M,
                                        int32_t Hq, int32_t Hkv, int32_t d, int32_t bs, int32_t P,
                                        int32_t max_blocks, int32_t max_prefix_len,
                                        float softmax_scale, float k_scale, float v_scale,
                                        pkv_dtype q_dtype, pkv_dtype cache_dtype, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* Call 3: out[r] = (2^la[r] a[r] + 2^lb[r] b[r]) / (2^la[r] + 2^lb[r]) for rows
 * r < rows of d floats (device, float32); a side with lse -inf has weight 0
 * and a row with both -inf is zero. lse_out (optional, may be NULL) receives
 * log2(2^la + 2^lb). out may alias a or b. d in {64, 128}. */
pkv_status pkv_merge_attn_states(float* out, float* lse_out, const float* a, const float* lse_a,
                                 const float* b, const float* lse_b, int64_t rows, int32_t d,
                                 void* stream);

/*
 * The three calls above in one, plus the decode step's write, with a single
 * merge: groups of M consecutive sequences (sequence g*M + m is member m of
 * group g) whose tables start with the same blocks. prefix_tables/prefix_lens
 * ([n_groups][prefix_max_blocks], [n_groups]) list each group's shared
 * blocks; suffix_tables/suffix_lens ([S][suffix_max_blocks], [S], S =
 * n_groups*M) list each sequence's blocks after them. A sequence's context is
 * its group's prefix followed by its suffix; out[S][Hq][d] (float32) is the
 * decode attention of pkv_paged_decode_attn over that whole context.
 *
 * k_new/v_new ([S][Hkv][d], as for pkv_kv_cache_write; both NULL: no write)
 * are each sequence's new token: it is written at the suffix's last position
 * (suffix_lens[i] - 1; sequences with an empty suffix write nothing) and
 * attended to, as by pkv_paged_decode_step. So a plan whose suffixes keep each
 * sequence's last block (the one that takes the new token) makes this one
 * decode step.
 *
 * Launches on `stream`: when a group's M queries fit one 16-column MFMA tile
 * (M * Hq/Hkv <= 16), one attention kernel takes the prefixes (every query of
 * a group sees every prefix token) and the suffixes (with the write) together;
 * otherwise the suffix pass (with the write) runs first, then the prefix
 * pass. Then one merge kernel combines the partial states of both. A new
 * token's slot must lie in its sequence's suffix blocks (the plan of
 * pkv_shared_prefix_plan guarantees it), since prefix blocks may be read
 * while the write runs. workspace: pkv_paged_shared_prefix_decode_workspace_size
 * bytes (device, caller-owned, any contents). Limits and dtypes as for
 * pkv_paged_decode_step and pkv_paged_multi_query_attn (1 <= M <= 4096);
 * k_inv_scale/v_inv_scale are used only for an fp8 cache with a write.
 */
size_t pkv_paged_shared_prefix_decode_workspace_size(int32_t n_groups, int32_t M, int32_t Hq,
                                                     int32_t Hkv, int32_t d);

pkv_status pkv_paged_shared_prefix_decode(
    float* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
    const int32_t* prefix_tables, const int32_t* prefix_lens, int32_t prefix_max_blocks,
    int32_t max_prefix_len, const int32_t* suffix_tables, const int32_t* suffix_lens,
    int32_t suffix_max_blocks, int32_t max_suffix_len, int32_t n_groups, int32_t M, int32_t Hq,
    int32_t Hkv, int32_t d, int32_t bs, int32_t P, float softmax_scale, float k_scale, float v_scale,
    float k_inv_scale, float v_inv_scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * Copy whole blocks inside both pools: for each k < n, block dst[k] becomes a
 * copy of block src[k] (every kv head, K and V). This is the device half of
 * copy-on-write: pkv_seq_append reports the (src, dst) pair when a sequence
 * writes into a shared, partly filled last block, and the caller copies it
 * before writing the new token ("03 · PagedAttention", "Sharing:
 * copy-on-write"; "PagedAttention" daily term, copy-on-write figure).
 *
 * k_cache, v_cache: the pools (layout above) in cache_dtype (any of the three).
 * src, dst:      int32 [n] device arrays of block ids. A pair with an id
 *                outside [0, P) is skipped (checked on the device). Within one
 *                call the copies run concurrently: the dst ids must be distinct
 *                and no dst may also be a src of the same call.
 * Requires 0 <= n <= min(P, 2^20) (n == 0 launches nothing), Hkv > 0,
 * d in {64, 128}, bs in {8, 16, 32, 64, 128}, P > 0.
 */
pkv_status pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst,
                           int32_t n, int32_t P, int32_t Hkv, int32_t d, int32_t bs,
                           pkv_dtype cache_dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Host block allocator and builders (CPU only)                              */
/* ------------------------------------------------------------------------ */

/*
 * A pool of P equal blocks of bs tokens, all free at creation; a LIFO free
 * list whose first pop returns block 0 ("PagedAttention" daily term, "Pros":
 * uniform blocks, a simple free list, no search).
 */
typedef struct pkv_allocator pkv_allocator;

typedef struct {
    int32_t num_blocks;       /* P                                              */
    int32_t free_blocks;      /* blocks on the free list                        */
    int32_t used_blocks;      /* P - free_blocks                                */
    int64_t slots_allocated;  /* used_blocks * bs                               */
    int64_t tokens_stored;    /* tokens held in used blocks (a shared block counted once) */
    double waste;             /* 1 - tokens_stored / slots_allocated (0 if none) */
} pkv_stats;

/* Create an allocator over a pool of P blocks of bs tokens, all free, set up
 * once for the whole cache ("03 · PagedAttention", "Blocks and block tables":
 * the pool is carved into equal blocks up front). P > 0, bs > 0; *out (host)
 * receives the handle, which the caller owns until pkv_allocator_destroy. */
pkv_status pkv_allocator_create(int32_t P, int32_t bs, pkv_allocator** out);
/* Destroy an allocator and every sequence in it; NULL is ignored. */
void pkv_allocator_destroy(pkv_allocator* a);

/* Register an empty sequence: a block table with no entries, blocks taken on
 * demand as tokens arrive ("03 · PagedAttention", "Blocks and block tables").
 * PKV_E_STATE if the id exists. */
pkv_status pkv_seq_create(pkv_allocator* a, int64_t seq_id);

/*
 * Append n_tokens positions to a sequence, taking a new block only when the
 * previous one is full ("03 · PagedAttention", "Blocks and block tables": the
 * 17th token takes a block, tokens 18-32 take none). slots_out[k] receives the
 * slot (block*bs + offset) of the k-th appended position (may be NULL when
 * n_tokens == 0).
 *
 * Copy-on-write ("03 · PagedAttention", "Sharing: copy-on-write"; daily term,
 * copy-on-write figure): if the sequence's last block is partially filled and
 * shared (refcount > 1), a new block is taken first, the (src, dst) pair is
 * written to *cow_src / *cow_dst with *n_cow = 1, the sequence's table points
 * at dst and src's refcount drops by one; the caller copies the block's data
 * (the pair is reported, not copied). Otherwise *n_cow = 0. cow_src, cow_dst
 * and n_cow may be NULL only if the caller never shares blocks; a CoW with
 * NULL outputs returns PKV_E_INVALID without changing anything.
 *
 * All or nothing: if fewer blocks are free than the append needs,
 * PKV_E_NO_BLOCKS and no state changes (the scheduler's cue to preempt:
 * "03 · PagedAttention", "When the pool runs dry").
 */
pkv_status pkv_seq_append(pkv_allocator* a, int64_t seq_id, int32_t n_tokens,
                          int64_t* slots_out, int32_t* cow_src, int32_t* cow_dst,
                          int32_t* n_cow);

/* Fork: child shares every block of parent (refcount + 1 each) and its
 * length, so both tables list the same physical blocks until one of them
 * writes into a shared, partly filled block and pkv_seq_append reports the
 * copy-on-write pair ("03 · PagedAttention", "Sharing: copy-on-write";
 * "PagedAttention" daily term, copy-on-write figure: beams and parallel
 * samples start from one prompt's blocks).
 * PKV_E_NOT_FOUND if parent is unknown, PKV_E_STATE if child exists; nothing
 * changes on an error. */
pkv_status pkv_seq_fork(pkv_allocator* a, int64_t parent, int64_t child);

/* Release a finished sequence: refcount - 1 for each of its blocks, last
 * logical block first; a block whose count reaches 0 goes back on the free
 * list, where the next append can take it ("PagedAttention" daily term,
 * "Pros": a plain free list of blocks; "03 · PagedAttention", "Sharing:
 * copy-on-write": a shared block is freed only when no table lists it).
 * PKV_E_NOT_FOUND for an unknown id; nothing changes then. */
pkv_status pkv_seq_free(pkv_allocator* a, int64_t seq_id);

/* Current context length and block count of a sequence. */
pkv_status pkv_seq_info(const pkv_allocator* a, int64_t seq_id, int64_t* length,
                        int32_t* num_blocks);

/*
 * Block tables for the listed sequences, the per-sequence map from logical
 * block j (token positions j*bs .. j*bs + bs - 1) to the physical block that
 * holds it ("03 · PagedAttention", "Blocks and block tables"; "Serving: vLLM
 * and PagedAttention", section 2.2, the block table as a page table):
 * tables_out int32 [S][max_blocks] (row i = sequence seq_ids[i]'s physical
 * blocks in logical order, padded with -1) and lens_out int32 [S] (their
 * lengths, the token being written this step included). Both are host
 * arrays the caller owns. PKV_E_INVALID if a sequence holds more than
 * max_blocks blocks or is longer than INT32_MAX; PKV_E_NOT_FOUND for an
 * unknown id. Outputs are written only on success.
 */
pkv_status pkv_build_block_tables(const pkv_allocator* a, const int64_t* seq_ids,
                                  int32_t S, int32_t max_blocks,
                                  int32_t* tables_out, int32_t* lens_out);

/*
 * Slot mapping: the flat slot of token position positions[i] (0-based) of each
 * sequence from its table row, tables[i][p / bs] * bs + p % bs: logical block
 * p / bs at offset p % bs ("03 · PagedAttention", "Blocks and block tables";
 * "Serving: vLLM and PagedAttention", section 2.2, the last block filled
 * from its start). A negative position gives -1 (pkv_kv_cache_write skips
 * it). tables, positions and slots_out are host arrays the caller owns.
 * PKV_E_INVALID if p / bs >= max_blocks or the entry is negative (nothing
 * written then). For a decode step the position is L_i - 1, the token being
 * written.
 */
pkv_status pkv_slots_from_tables(const int32_t* tables, const int32_t* positions,
                                 int32_t S, int32_t max_blocks, int32_t bs,
                                 int64_t* slots_out);

/*
 * Host plan for pkv_paged_shared_prefix_decode (shared blocks, "03 ·
 * PagedAttention", "Sharing: copy-on-write"): rows g*group_size ..
 * (g+1)*group_size - 1 of tables [S][max_blocks] (lengths lens[S]) form group
 * g. Its prefix is the longest run of leading blocks that every member lists
 * with the same id (>= 0), not counting any member's last block (the one that
 * takes the step's new token; copy-on-write keeps it private):
 * prefix_tables[g][0..k) = those ids, prefix_lens[g] = k*bs. Member i's suffix
 * is the rest of its row: suffix_tables[i][j] = tables[i][k + j] for
 * k + j < ceil(L_i/bs), suffix_lens[i] = L_i - k*bs (L_i <= 0: 0). Unused
 * entries are -1. All arrays are caller-owned host memory: prefix_tables
 * [S/group_size][max_blocks], prefix_lens [S/group_size], suffix_tables
 * [S][max_blocks], suffix_lens [S]. PKV_E_INVALID if S is not a multiple of
 * group_size or a length exceeds max_blocks*bs (nothing written then).
 */
pkv_status pkv_shared_prefix_plan(const int32_t* tables, const int32_t* lens, int32_t S,
                                  int32_t max_blocks, int32_t group_size, int32_t bs,
                                  int32_t* prefix_tables, int32_t* prefix_lens,
                                  int32_t* suffix_tables, int32_t* suffix_lens);

/*
 * Prefix caching ("PagedAttention" daily term, the prefix-caching paragraph
 * after the copy-on-write figure; "Serving: vLLM and PagedAttention",
 * section 2.6): a full block is named by a hash of its tokens and of the
 * prefix before it, so a later request whose prompt starts the same way reuses
 * the cached blocks instead of recomputing them.
 *
 * Block hash k of a token sequence (reading of the pages' components: parent
 * hash, block token ids, extra keys) is
 *   SHA-256( hash_{k-1} || tokens[k*bs .. k*bs+bs) as little-endian int32 || extra )
 * with hash_{-1} = 32 zero bytes; extra is any caller key (adapter id, tenant
 * salt, ...) and may be empty. Only full blocks have hashes.
 *
 * pkv_block_hashes writes the n_tokens / bs hashes of a sequence to
 * hashes_out[n_tokens / bs][32].
 */
pkv_status pkv_block_hashes(const int32_t* tokens, int32_t n_tokens, int32_t bs,
                            const uint8_t* extra, int32_t extra_len, uint8_t* hashes_out);

/*
 * Create sequence seq_id holding a prompt of n_tokens tokens. The longest run
 * of leading full blocks whose hashes are cached is shared (reference count + 1;
 * a cached block that is free again is taken back off the free list); the rest
 * of the prompt gets fresh blocks, and each fresh full block is registered
 * under its hash. slots_out[n_tokens] receives every position's slot;
 * *n_cached_out the number of leading tokens whose K/V are already in the
 * cache (a multiple of bs) -- the caller writes only the others.
 * A block keeps its hash while in use and after it is freed, until the free
 * list hands it out again. All or nothing: PKV_E_NO_BLOCKS changes nothing;
 * PKV_E_STATE if seq_id exists.
 */
pkv_status pkv_seq_create_prefixed(pkv_allocator* a, int64_t seq_id, const int32_t* tokens,
                                   int32_t n_tokens, const uint8_t* extra, int32_t extra_len,
                                   int64_t* slots_out, int32_t* n_cached_out);

/* Prefix-cache counters: leading blocks found and not found by
 * pkv_seq_create_prefixed, and blocks holding a hash now. */
pkv_status pkv_prefix_cache_stats(const pkv_allocator* a, int64_t* hit_blocks,
                                  int64_t* miss_blocks, int32_t* cached_blocks);

/* Pool-wide statistics ("03 · PagedAttention", "In Production": the block
 * pool's fill is the capacity signal). */
pkv_status pkv_allocator_stats(const pkv_allocator* a, pkv_stats* out);

/*
 * Tail-waste arithmetic for n lengths at block size bs ("paged-attention"
 * lesson, worked example; "03 · PagedAttention", waste table):
 *   paged_slots = sum ceil(L/bs)*bs, naive_slots = n*max_len, used = sum L,
 *   waste_paged = 1 - used/paged_slots, waste_naive = 1 - used/naive_slots.
 * Negative lengths count as 0. Any output pointer may be NULL.
 */
pkv_status pkv_waste_stats(const int32_t* lens, int32_t n, int32_t bs, int32_t max_len,
                           int64_t* paged_slots, int64_t* naive_slots, int64_t* used,
                           double* waste_paged, double* waste_naive);

/*
 * Gather only: read the K/V chunks that a decode plan lists -- every chunk of
 * every (sequence, kv head) the step attends over, through the block tables --
 * with the planned kernel's loads (cacheable ones for a plan marked by
 * pkv_plan_mark_shared_blocks), pipeline and grid, and no arithmetic. Its
 * time is the read rate of the step's own scattered tiles: the ceiling of the
 * planned step without its compute, q loads, new-token write, records and
 * merge, timed next to it. A decode step reads the whole cache of every
 * active sequence through its block table ("Serving: vLLM and
 * PagedAttention", section 4.2, the step-time model; "03 · PagedAttention",
 * "Blocks and block tables"). Arguments as for pkv_paged_decode_step_planned
 * (the plan must be built for this S, Hkv, d, cache type, max_context_len
 * and device); sink: one device uint32 that a thread writes only when the xor
 * of the words it loaded equals 0x9E3779B9. Nothing is written otherwise;
 * nothing allocated.
 */
pkv_status pkv_paged_gather_read(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                 int32_t S, int32_t Hkv, int32_t d, int32_t bs, int32_t P, int32_t max_blocks,
                                 int32_t max_context_len, pkv_dtype cache_dtype, const void* plan_host,
                                 const void* plan_dev, size_t plan_bytes, uint32_t* sink, void* stream);

/*
 * Streaming read of `bytes` of device memory at src (16-byte aligned; the
 * floor(bytes / 16) whole 16-byte units are read, each once), with the same
 * nontemporal 16-byte loads the attention kernels stream the cache with:
 * the practical read ceiling of the device, timed next to a decode step over
 * the same byte count. A decode step is bound by reading the whole cache of
 * every active sequence, so its time is about those bytes over the achieved
 * bandwidth ("Serving: vLLM and PagedAttention", section 4.2, the step-time
 * model). blocks: workgroups of 256 threads, 1 .. 2^20; unroll: loads in
 * flight per thread, 4, 8 or 16. sink: one device uint32 that a thread
 * writes only when the xor of the words it loaded equals 0x9E3779B9 (it
 * keeps the loads from being dropped). Enqueued on stream; nothing allocated.
 */
pkv_status pkv_stream_read(const void* src, size_t bytes, int32_t blocks, int32_t unroll, uint32_t* sink,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
