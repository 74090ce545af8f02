"""fp64 paged decode attention: reassemble each sequence's K/V, then attend.

Test infrastructure only (see the package docstring).

What is computed (the pages' statement of the problem):

* A sequence's cache is a list of fixed-size blocks found through its block
  table: logical block j holds token positions [j*bs, (j+1)*bs) and lives in
  physical block ``table[j]`` ("03 · PagedAttention", "Blocks and block tables";
  "Serving: vLLM and PagedAttention", section 2.2).
* One decode step scores the new query against every key of the sequence,
  gathering K and V from the listed blocks ("PagedAttention" daily term,
  decode-step figure).
* The result is the ordinary attention over the sequence's tokens in logical
  order: only the layout differs from a contiguous cache ("paged-attention"
  lesson, closing paragraph; "PagedAttention" daily term, "Pros": not an
  approximation).

So: out[i, h] = sum_t softmax_t(sigma * q[i,h] . K_i[t, g]) * V_i[t, g] with
g = h // G (grouped-query attention, consecutive grouping), over the L_i tokens
of sequence i; a row with L_i <= 0 is zero.

Storage layout of the pools (the pages fix none; the reading taken):
  k_cache[P][Hkv][bs][d]          token-major within each (block, kv-head) tile
  v_cache[P][Hkv][bs/vs][d][vs]   channel-major within each sub-tile of vs =
                                  min(bs, 16) tokens; for bs <= 16 that is
                                  [P][Hkv][d][bs], and may be given so
Both tiles are contiguous, and the bs tokens of a block sit together in each.

Element storage: "f32" float32, "bf16" uint16 bit patterns, "fp8" uint8 OCP
E4M3 codes whose value is decode(code) * scale (one float32 scale per tensor).
"""

import numpy as np

from .codecs import bf16_bits_to_f64, f32_to_f64, e4m3_decode
from .layout import v_view5


def widen(arr, dtype, scale=1.0):
    """Stored elements -> exact float64 values (fp8 includes the tensor scale)."""
    if dtype == "f32":
        return f32_to_f64(arr)
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "fp8":
        # decode(code) has at most 4 significant bits and the scale 24, so the
        # float64 product is exact.
        return e4m3_decode(arr) * np.float64(np.float32(scale))
    raise ValueError(f"unknown dtype {dtype!r}")


def reassemble(pool, table_row, L, bs, which):
    """Gather one sequence's K or V into logical order: [L][Hkv][d] (storage dtype).

    ``which`` is "k" for the [P][Hkv][bs][d] pool and "v" for the
    [P][Hkv][bs/vs][d][vs] pool (or [P][Hkv][d][bs] when bs <= 16). Position p
    lives in logical block p // bs at offset p % bs (0-based positions); in V
    that is sub-tile (p % bs) // vs, column (p % bs) % vs.
    """
    if which == "v":
        pool = v_view5(pool, bs)
    P = pool.shape[0]
    n = -(-L // bs)
    ids = np.asarray(table_row[:n], dtype=np.int64)
    if n and (ids.min() < 0 or ids.max() >= P):
        raise ValueError("block table entry outside the pool")
    tiles = pool[ids]
    if which == "k":            # [n][Hkv][bs][d] -> [n][bs][Hkv][d]
        tiles = tiles.transpose(0, 2, 1, 3)
    elif which == "v":          # [n][Hkv][bs/vs][d][vs] -> [n][bs/vs][vs][Hkv][d]
        tiles = tiles.transpose(0, 2, 4, 1, 3)
    else:
        raise ValueError(which)
    flat = tiles.reshape(n * bs, tiles.shape[-2], tiles.shape[-1])
    return flat[:L]


def contiguous_decode_attn(q_i, K, V, sigma):
    """Textbook single-query attention over contiguous float64 K/V.

    q_i: [Hq][d]; K, V: [L][Hkv][d]; sigma: the softmax scale. Returns [Hq][d].
    """
    Hq, d = q_i.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    if L <= 0:
        return np.zeros((Hq, d))
    qg = q_i.reshape(Hkv, G, d)
    Kh = K.transpose(1, 0, 2)              # [Hkv][L][d]
    Vh = V.transpose(1, 0, 2)
    s = sigma * (qg @ Kh.transpose(0, 2, 1))   # [Hkv][G][L]
    m = s.max(axis=-1, keepdims=True)
    p = np.exp(s - m)
    o = (p @ Vh) / p.sum(axis=-1, keepdims=True)
    return o.reshape(Hq, d)


def paged_decode_attn(q, k_cache, v_cache, block_tables, context_lens, *, bs,
                      softmax_scale, q_dtype, cache_dtype, k_scale=1.0, v_scale=1.0,
                      seqs=None):
    """Oracle output, float64 [S][Hq][d] (or only the rows in ``seqs``).

    softmax_scale is taken as the float32 value the kernel receives, widened.
    """
    S, Hq, d = q.shape
    sigma = np.float64(np.float32(softmax_scale))
    ks = k_scale if cache_dtype == "fp8" else 1.0
    vs = v_scale if cache_dtype == "fp8" else 1.0
    rows = range(S) if seqs is None else seqs
    out = np.zeros((S, Hq, d)) if seqs is None else np.zeros((len(seqs), Hq, d))
    for r, i in enumerate(rows):
        L = int(context_lens[i])
        if L <= 0:
            continue
        K = widen(reassemble(k_cache, block_tables[i], L, bs, "k"), cache_dtype, ks)
        V = widen(reassemble(v_cache, block_tables[i], L, bs, "v"), cache_dtype, vs)
        qi = widen(q[i], q_dtype)
        out[r] = contiguous_decode_attn(qi, K, V, sigma)
    return out


def paged_multi_query_attn(q, k_cache, v_cache, block_tables, context_lens, *, bs, softmax_scale,
                           q_dtype, cache_dtype, k_scale=1.0, v_scale=1.0, seqs=None):
    """Oracle output, float64 [S][n_q][Hq][d], for a window of n_q new queries
    per sequence ("Serving: vLLM and PagedAttention", sections 2.4 and 2.7:
    prefill chunks and verification windows reuse the decode gather).

    Query j of sequence i sits at position L_i - n_q + j and is causal: it is the
    single-query decode attention of ``paged_decode_attn`` over the first
    L_i - n_q + j + 1 tokens of the same block table. Sequences with L_i <= 0
    give zero rows.
    """
    S, n_q, Hq, d = q.shape
    rows = list(range(S)) if seqs is None else list(seqs)
    out = np.zeros((len(rows), n_q, Hq, d))
    lens = np.asarray(context_lens, dtype=np.int64)
    for j in range(n_q):
        lens_j = np.where(lens > 0, lens - n_q + 1 + j, 0)
        out[:, j] = paged_decode_attn(q[:, j], k_cache, v_cache, block_tables, lens_j, bs=bs,
                                      softmax_scale=softmax_scale, q_dtype=q_dtype,
                                      cache_dtype=cache_dtype, k_scale=k_scale, v_scale=v_scale,
                                      seqs=rows)
    return out


def contiguous_decode_lse(q_i, K, sigma):
    """[Hq]: log2 of each head's softmax denominator, log2 sum_t exp(s_t), over
    contiguous float64 K ([L][Hkv][d]) with s_t = sigma * q . K_t; -inf when
    L <= 0. This is the state that lets two attentions over disjoint token sets
    be combined exactly (``merge_attn_states``)."""
    Hq, d = q_i.shape
    L, Hkv, _ = K.shape
    if L <= 0:
        return np.full(Hq, -np.inf)
    G = Hq // Hkv
    s = sigma * (q_i.reshape(Hkv, G, d) @ K.transpose(1, 2, 0))   # [Hkv][G][L]
    m = s.max(axis=-1)
    return ((m + np.log(np.exp(s - m[..., None]).sum(axis=-1))) / np.log(2.0)).reshape(Hq)


def paged_decode_lse(q, k_cache, block_tables, context_lens, *, bs, softmax_scale, q_dtype,
                     cache_dtype, k_scale=1.0, seqs=None):
    """Oracle [S][Hq] (or the rows in ``seqs``): ``contiguous_decode_lse`` of each
    sequence's reassembled K, scores as in ``paged_decode_attn`` (k_scale
    included for fp8 caches)."""
    S, Hq, d = q.shape
    sigma = np.float64(np.float32(softmax_scale))
    ks = k_scale if cache_dtype == "fp8" else 1.0
    rows = list(range(S)) if seqs is None else list(seqs)
    out = np.full((len(rows), Hq), -np.inf)
    for r, i in enumerate(rows):
        L = int(context_lens[i])
        if L <= 0:
            continue
        K = widen(reassemble(k_cache, block_tables[i], L, bs, "k"), cache_dtype, ks)
        out[r] = contiguous_decode_lse(widen(q[i], q_dtype), K, sigma)
    return out


def merge_attn_states(o_a, lse_a, o_b, lse_b):
    """Combine the attentions of one query over two disjoint token sets A and B
    into its attention over A and B together. With Z_X = sum_{t in X} exp(s_t)
    = 2^lse_X, the softmax over A and B weighs o_A by Z_A / (Z_A + Z_B) and o_B
    by Z_B / (Z_A + Z_B); the new lse is log2(Z_A + Z_B). A side with lse -inf
    (no tokens) has weight 0; a row with no tokens on either side is zero.
    o_*: [..., d]; lse_*: [...]. Returns (o, lse) in float64.

    This is how shared prefix blocks ("03 · PagedAttention", "Sharing:
    copy-on-write") are attended once for all sequences that list them.
    """
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(la, lb)
    empty = m == -np.inf
    m_safe = np.where(empty, 0.0, m)
    wa = np.where(la == -np.inf, 0.0, np.exp2(la - m_safe))
    wb = np.where(lb == -np.inf, 0.0, np.exp2(lb - m_safe))
    den = wa + wb
    den_safe = np.where(empty, 1.0, den)
    o = (wa[..., None] * np.asarray(o_a, dtype=np.float64)
         + wb[..., None] * np.asarray(o_b, dtype=np.float64)) / den_safe[..., None]
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, -np.inf, m_safe + np.log2(den_safe))
    return o, lse
