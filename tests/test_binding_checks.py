"""The Python binding rejects tensors whose dtypes, shapes or devices do not go
together, before anything reaches the library.

The C ABI takes one cache dtype (from the K pool) and one source dtype: a V
pool of another dtype, or new K/V or q of the wrong dtype, would be read or
written with the wrong element size. These checks run on CPU tensors: each
mismatch must raise ValueError naming it, before the device-pointer check.
"""

import pytest
import torch

import paged_kv_cache_108_amd as pkv
from paged_kv_cache_108_amd import api

P, Hkv, bs, d, S, Hq = 6, 2, 16, 64, 3, 4


def pools(dtype=torch.bfloat16, v_dtype=None, v_shape=None):
    k = torch.zeros((P, Hkv, bs, d), dtype=dtype)
    v = torch.zeros(v_shape or (P, Hkv, d, bs), dtype=v_dtype or dtype)
    return k, v


def attn_args(q_dtype=torch.bfloat16):
    q = torch.zeros((S, Hq, d), dtype=q_dtype)
    out = torch.zeros((S, Hq, d), dtype=torch.float32)
    tab = torch.zeros((S, 2), dtype=torch.int32)
    lens = torch.ones(S, dtype=torch.int32)
    return out, q, tab, lens


def test_v_pool_of_another_dtype_is_rejected():
    k, v = pools(torch.bfloat16, v_dtype=torch.uint8)
    out, q, tab, lens = attn_args()
    kn = torch.zeros((S, Hkv, d), dtype=torch.bfloat16)
    slots = torch.zeros(S, dtype=torch.int64)
    with pytest.raises(ValueError, match="v_cache dtype"):
        pkv.kv_cache_write(kn, kn, k, v, slots)
    with pytest.raises(ValueError, match="v_cache dtype"):
        pkv.paged_decode_attn(out, q, k, v, tab, lens, max_context_len=1, softmax_scale=0.1)
    with pytest.raises(ValueError, match="v_cache dtype"):
        pkv.paged_decode_step(out, q, kn, kn, k, v, tab, lens, max_context_len=1, softmax_scale=0.1)
    with pytest.raises(ValueError, match="v_cache dtype"):
        pkv.copy_blocks(k, v, torch.zeros(1, dtype=torch.int32), torch.ones(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="v_cache dtype"):
        api.paged_multi_query_attn(out.unsqueeze(1), q.unsqueeze(1), k, v, tab, lens, max_context_len=1,
                                   softmax_scale=0.1)


def test_v_pool_of_another_shape_is_rejected():
    k, v = pools(v_shape=(P, Hkv, d, bs // 2))
    out, q, tab, lens = attn_args()
    with pytest.raises(ValueError, match="v_cache shape"):
        pkv.paged_decode_attn(out, q, k, v, tab, lens, max_context_len=1, softmax_scale=0.1)
    lse = torch.zeros((S, Hq), dtype=torch.float32)
    with pytest.raises(ValueError, match="v_cache shape"):
        api.paged_decode_attn_lse(out, lse, q, k, v, tab, lens, max_context_len=1, softmax_scale=0.1)


def test_new_tokens_must_match_the_cache():
    kn32 = torch.zeros((S, Hkv, d), dtype=torch.float32)
    knb = torch.zeros((S, Hkv, d), dtype=torch.bfloat16)
    slots = torch.zeros(S, dtype=torch.int64)
    out, q, tab, lens = attn_args()
    for dt in (torch.bfloat16, torch.uint8):        # bf16 and fp8 caches take bf16 new tokens
        k, v = pools(dt)
        with pytest.raises(ValueError, match="k_new dtype"):
            pkv.kv_cache_write(kn32, kn32, k, v, slots)
        with pytest.raises(ValueError, match="v_new dtype"):
            pkv.kv_cache_write(knb, kn32, k, v, slots)
        with pytest.raises(ValueError, match="v_new dtype"):
            pkv.paged_decode_step(out, q, knb, kn32, k, v, tab, lens, max_context_len=1, softmax_scale=0.1)
    k, v = pools(torch.float32)                     # an f32 cache takes f32 new tokens
    with pytest.raises(ValueError, match="k_new dtype"):
        pkv.kv_cache_write(knb, knb, k, v, slots)


def test_q_must_match_the_cache():
    out, q32, tab, lens = attn_args(torch.float32)
    for dt in (torch.bfloat16, torch.uint8):
        k, v = pools(dt)
        with pytest.raises(ValueError, match="q dtype"):
            pkv.paged_decode_attn(out, q32, k, v, tab, lens, max_context_len=1, softmax_scale=0.1)
    k, v = pools(torch.float32)
    out, qb, tab, lens = attn_args(torch.bfloat16)
    with pytest.raises(ValueError, match="q dtype"):
        pkv.paged_decode_attn(out, qb, k, v, tab, lens, max_context_len=1, softmax_scale=0.1)


def test_shapes_of_out_tables_and_lengths():
    k, v = pools()
    out, q, tab, lens = attn_args()
    with pytest.raises(ValueError, match="out must be float32"):
        pkv.paged_decode_attn(out[:2], q, k, v, tab, lens, max_context_len=1, softmax_scale=0.1)
    with pytest.raises(ValueError, match="tables/lengths"):
        pkv.paged_decode_attn(out, q, k, v, tab[:2], lens, max_context_len=1, softmax_scale=0.1)
    with pytest.raises(ValueError, match="int32"):
        pkv.paged_decode_attn(out, q, k, v, tab.long(), lens, max_context_len=1, softmax_scale=0.1)
    with pytest.raises(ValueError, match="q must be"):
        pkv.paged_decode_attn(out, torch.zeros((S, Hq, 2 * d), dtype=torch.bfloat16), k, v, tab, lens,
                              max_context_len=1, softmax_scale=0.1)


def test_one_device_for_every_tensor():
    api_one_device = api._one_device
    a = torch.zeros(1)
    b = torch.zeros(1, device="meta")
    api_one_device("x", a, None, a)                  # one device: fine
    with pytest.raises(ValueError, match="several devices"):
        api_one_device("x", a, b)
