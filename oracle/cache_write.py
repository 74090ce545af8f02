"""The KV-cache write: scatter each new token's K and V into its physical slot.

Test infrastructure only (see the package docstring).

The decode-step figure of the "PagedAttention" daily term puts "write the new K
and V into the current block" in the same per-step launch as the gather. A slot
is the flat index block * bs + offset; slot -1 means "skip this token" (padding).

Per token t with slot >= 0: (b, o) = divmod(slot, bs), then for every kv head h
and channel c
    K[b][h][o][c] = enc(K_new[t][h][c])                  (k_cache [P][Hkv][bs][d])
    V[b][h][o // vs][c][o % vs] = enc(V_new[t][h][c])    (v_cache [P][Hkv][bs/vs][d][vs])
with vs = min(bs, 16); for bs <= 16 the V pool may also be given as
[P][Hkv][d][bs], the same memory. Every other element of the pools is left as
it was.

Copy-on-write ("03 · PagedAttention", "Sharing: copy-on-write"; the daily
term's copy-on-write figure): before a sequence writes into a shared, partly
filled block, the block is duplicated for it. ``copy_blocks`` is that
duplication: for each (src, dst) pair, every element of block dst (all kv
heads, K and V) takes the value of block src.

enc is the identity on the stored bits when source and cache dtypes agree
(f32 -> f32, bf16 -> bf16). For an fp8 cache the source (bf16) value x becomes
e4m3_encode(float32(x) * float32(inv_scale)): one float32 multiplication rounded
to nearest-even, then the codec of ``codecs.py``.
"""

import numpy as np

from .codecs import bf16_bits_to_f64, e4m3_encode
from .layout import v_view5


def quantise(x_bits, src_dtype, inv_scale):
    """Source elements -> E4M3 codes, exactly as the write stores them."""
    if src_dtype == "bf16":
        x = bf16_bits_to_f64(x_bits).astype(np.float32)    # exact
    elif src_dtype == "f32":
        x = np.asarray(x_bits, dtype=np.float32)
    else:
        raise ValueError(src_dtype)
    y = x * np.float32(inv_scale)                          # float32 product, RNE
    return e4m3_encode(y)


def kv_cache_write(k_new, v_new, k_cache, v_cache, slot_mapping, *, bs, src_dtype,
                   cache_dtype, k_inv_scale=1.0, v_inv_scale=1.0):
    """Return (k_cache', v_cache'): copies of the pools with the new tokens written.

    k_new, v_new: [T][Hkv][d] in the source storage dtype; slot_mapping: int64[T].
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    v5 = v_view5(v_out, bs)                                # a view: writes land in v_out
    if cache_dtype == "fp8":
        kq = quantise(k_new, src_dtype, k_inv_scale)
        vq = quantise(v_new, src_dtype, v_inv_scale)
    elif cache_dtype == src_dtype:
        kq = np.asarray(k_new)
        vq = np.asarray(v_new)
    else:
        raise ValueError(f"unsupported write {src_dtype} -> {cache_dtype}")
    P = k_cache.shape[0]
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        b, o = divmod(int(slot), bs)
        if b >= P:
            raise ValueError("slot outside the pool")
        k_out[b, :, o, :] = kq[t]
        v5[b, :, o // v5.shape[4], :, o % v5.shape[4]] = vq[t]
    return k_out, v_out


def copy_blocks(k_cache, v_cache, pairs):
    """Return (k_cache', v_cache'): copies of the pools in which block dst of
    each (src, dst) pair holds block src's contents. Pairs are applied in
    order; a dst that is also a src of the same call is rejected (the copies of
    one call are independent of each other)."""
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    P = k_cache.shape[0]
    srcs = {int(a) for a, _ in pairs}
    dsts = [int(b) for _, b in pairs]
    if len(set(dsts)) != len(dsts) or srcs & set(dsts):
        raise ValueError("dst blocks must be distinct and not among the sources")
    for a, b in pairs:
        a, b = int(a), int(b)
        if not (0 <= a < P and 0 <= b < P):
            continue                      # outside the pool: skipped
        k_out[b] = k_cache[a]
        v_out[b] = v_cache[a]
    return k_out, v_out
