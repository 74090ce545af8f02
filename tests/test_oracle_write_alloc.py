"""Pins of the oracle's cache write, slot mapping and allocator twin."""

import numpy as np
import pytest
import torch

import oracle
from oracle import TwinAllocator, NoBlocks


# ----------------------------------------------------------------------- slots
def test_block_table_listing(golden):
    g = golden("block_table_listing.json")
    bs = g["block_size"]
    B = g["sequence_B"]
    tab = np.array([B["table"]])
    L = B["length"]
    # newest token of a 20-token sequence: position 19, logical block 1, offset 3
    assert oracle.decode_slots(tab, [L], bs)[0] == B["table"][1] * bs + 3
    assert L - (len(B["table"]) - 1) * bs == B["last_block_used"]
    A = g["sequence_A_as_printed"]
    # reading: a 35-token sequence fills 3 slots of its third block
    assert 35 - 2 * bs == 3
    assert oracle.slots_for_positions(np.array([A["table"]]), [34], bs)[0] == 893 * bs + 2


def test_slots_every_position():
    rng = np.random.default_rng(0)
    for bs in (8, 16, 32):
        tab = rng.permutation(50)[:10].reshape(1, 10)
        for p in range(10 * bs):
            s = oracle.slots_for_positions(tab, [p], bs)[0]
            assert s // bs == tab[0, p // bs] and s % bs == p % bs
    assert oracle.decode_slots(np.array([[3, -1]]), [0], 16)[0] == -1


# ----------------------------------------------------------------------- write
def _pools(P, Hkv, bs, d, dtype=np.float32):
    rng = np.random.default_rng(1)
    return (rng.standard_normal((P, Hkv, bs, d)).astype(dtype),
            rng.standard_normal((P, Hkv, d, bs)).astype(dtype))


def test_write_places_each_token_and_nothing_else():
    P, Hkv, bs, d = 9, 3, 8, 4
    kc, vc = _pools(P, Hkv, bs, d)
    rng = np.random.default_rng(2)
    kn = rng.standard_normal((4, Hkv, d)).astype(np.float32)
    vn = rng.standard_normal((4, Hkv, d)).astype(np.float32)
    slots = np.array([5 * bs + 3, -1, 0, P * bs - 1])
    k2, v2 = oracle.kv_cache_write(kn, vn, kc, vc, slots, bs=bs, src_dtype="f32", cache_dtype="f32")
    expect_k, expect_v = kc.copy(), vc.copy()
    for t, (b, o) in {0: (5, 3), 2: (0, 0), 3: (P - 1, bs - 1)}.items():
        for h in range(Hkv):
            for c in range(d):
                expect_k[b, h, o, c] = kn[t, h, c]
                expect_v[b, h, c, o] = vn[t, h, c]
    assert np.array_equal(k2, expect_k) and np.array_equal(v2, expect_v)
    assert np.array_equal(kc, _pools(P, Hkv, bs, d)[0])      # inputs untouched


def test_write_bf16_is_a_bit_copy():
    P, Hkv, bs, d = 4, 2, 16, 8
    kc = np.arange(P * Hkv * bs * d, dtype=np.uint16).reshape(P, Hkv, bs, d)
    vc = np.arange(P * Hkv * d * bs, dtype=np.uint16).reshape(P, Hkv, d, bs)
    kn = np.full((1, Hkv, d), 0x7FC1, dtype=np.uint16)       # a NaN payload survives
    vn = np.full((1, Hkv, d), 0x8001, dtype=np.uint16)
    k2, v2 = oracle.kv_cache_write(kn, vn, kc, vc, np.array([17]), bs=bs, src_dtype="bf16",
                                   cache_dtype="bf16")
    assert np.all(k2[1, :, 1, :] == 0x7FC1) and np.all(v2[1, :, :, 1] == 0x8001)
    assert np.sum(k2 != kc) == Hkv * d and np.sum(v2 != vc) == Hkv * d


def test_write_large_block_lands_in_its_v_sub_tile():
    # bs 64: V tiles are 4 sub-tiles of 16 tokens, each [d][16]; token offset
    # 37 of block 2 is sub-tile 2, column 5
    P, Hkv, bs, d = 3, 2, 64, 8
    kc = np.zeros((P, Hkv, bs, d), dtype=np.uint16)
    vc = np.zeros((P, Hkv, bs // 16, d, 16), dtype=np.uint16)
    kn = np.arange(1, Hkv * d + 1, dtype=np.uint16).reshape(1, Hkv, d)
    vn = kn + 1000
    k2, v2 = oracle.kv_cache_write(kn, vn, kc, vc, np.array([2 * bs + 37]), bs=bs, src_dtype="bf16",
                                   cache_dtype="bf16")
    assert np.array_equal(k2[2, :, 37, :], kn[0]) and np.sum(k2 != 0) == Hkv * d
    assert np.array_equal(v2[2, :, 2, :, 5], vn[0]) and np.sum(v2 != 0) == Hkv * d
    flat = v2.reshape(P, Hkv, bs * d)                     # tile memory order
    for h in range(Hkv):
        for c in range(d):
            assert flat[2, h, 2 * 16 * d + c * 16 + 5] == vn[0, h, c]
    # a [P][Hkv][d][bs] pool does not describe bs > 16
    with pytest.raises(ValueError):
        oracle.kv_cache_write(kn, vn, kc, np.zeros((P, Hkv, d, bs), np.uint16), np.array([0]), bs=bs,
                              src_dtype="bf16", cache_dtype="bf16")


def test_write_fp8_quantises_with_one_float32_product():
    P, Hkv, bs, d = 3, 2, 16, 64
    kc = np.zeros((P, Hkv, bs, d), dtype=np.uint8)
    vc = np.zeros((P, Hkv, d, bs), dtype=np.uint8)
    rng = np.random.default_rng(4)
    x = torch.from_numpy(rng.standard_normal((2, Hkv, d)).astype(np.float32) * 3).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    inv = np.float32(448.0 / 11.0)
    k2, v2 = oracle.kv_cache_write(bits, bits, kc, vc, np.array([0, 33]), bs=bs, src_dtype="bf16",
                                   cache_dtype="fp8", k_inv_scale=inv, v_inv_scale=inv)
    y = (x.float() * float(inv))                             # float32 product, RNE
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()   # |y| < 448 here
    assert np.array_equal(k2[0, :, 0, :], ref[0]) and np.array_equal(k2[2, :, 1, :], ref[1])
    assert np.array_equal(v2[0, :, :, 0], ref[0]) and np.array_equal(v2[2, :, :, 1], ref[1])


def test_write_rejects_slot_outside_pool():
    kc, vc = _pools(2, 1, 4, 2)
    with pytest.raises(ValueError):
        oracle.kv_cache_write(np.zeros((1, 1, 2), np.float32), np.zeros((1, 1, 2), np.float32),
                              kc, vc, np.array([8]), bs=4, src_dtype="f32", cache_dtype="f32")


# ----------------------------------------------------------------------- allocator
def test_on_demand_allocation():
    a = TwinAllocator(10, 16)
    a.create(1)
    a.append(1, 16)
    assert a.stats()["used_blocks"] == 1
    a.append(1, 1)                      # the 17th token takes a block
    assert a.stats()["used_blocks"] == 2
    for _ in range(15):                 # tokens 18..32 take none
        a.append(1, 1)
    assert a.stats()["used_blocks"] == 2
    a.append(1, 1)
    assert a.stats()["used_blocks"] == 3
    a.create(2)
    a.append(2, 80)                     # 80 tokens use 5 blocks
    assert len(a.seqs[2][0]) == 5


def test_lifo_order_and_slots():
    a = TwinAllocator(8, 4)
    a.create(0)
    slots, cow = a.append(0, 6)
    assert a.seqs[0][0] == [0, 1] and slots == [0, 1, 2, 3, 4, 5] and cow == []
    a.create(1)
    a.append(1, 1)
    assert a.seqs[1][0] == [2]
    a.release(0)                        # pushes 1 then 0: next pops give 0, then 1
    a.create(2)
    a.append(2, 5)
    assert a.seqs[2][0] == [0, 1]


def test_worked_example_through_allocator(golden):
    g = golden("worked_example.json")
    a = TwinAllocator(g["pool_slots"] // 16, 16)
    for i, L in enumerate(g["lengths"]):
        a.create(i)
        a.append(i, L)
    st = a.stats()
    assert st["used_blocks"] == sum(g["pages"])
    assert st["slots_allocated"] == g["paged_alloc"]
    assert st["tokens_stored"] == g["used"]
    assert round(100 * st["waste"], 1) == g["paged_waste_pct_1dp"]


def test_fork_and_copy_on_write():
    # the daily term's figure: 3 samples share a prefix; s1 writes into the
    # shared, partially filled block: it gets a copy, the original's count drops.
    a = TwinAllocator(20, 16)
    a.create("s1")
    a.append("s1", 40)                  # blocks 0,1,2; block 2 holds 8 tokens
    a.fork("s1", "s2")
    a.fork("s1", "s3")
    assert [a.ref[b] for b in (0, 1, 2)] == [3, 3, 3]
    slots, cow = a.append("s1", 1)
    assert cow == [(2, 3)]
    assert a.seqs["s1"][0] == [0, 1, 3] and a.seqs["s2"][0] == [0, 1, 2]
    assert a.ref[2] == 2 and a.ref[3] == 1
    assert slots == [3 * 16 + 8]
    _, cow = a.append("s1", 1)          # now private: no further copy
    assert cow == []
    # a block-aligned shared prefix never copies
    b = TwinAllocator(10, 16)
    b.create(0)
    b.append(0, 32)
    b.fork(0, 1)
    _, cow = b.append(1, 3)
    assert cow == [] and b.seqs[1][0] == [0, 1, 2]


def test_copy_on_write_keeps_every_sequence_equal_to_its_own_tokens():
    # Beams forked from a prefix that ends inside a block, then each appends
    # its own token through the allocator: after copying each reported pair and
    # writing the new tokens, every beam's reassembled K/V must be exactly the
    # prefix followed by its own token, and the parent's prefix is untouched
    # (the copy-on-write rule of "Sharing: copy-on-write"). Built against
    # sequences assembled directly from the token values, not from the pool.
    from oracle import copy_blocks, kv_cache_write, reassemble
    rng = np.random.default_rng(5)
    bs, Hkv, d, P, L0 = 16, 2, 64, 40, 100          # 100 = 6 blocks + 4 tokens
    prefix_k = rng.standard_normal((L0, Hkv, d)).astype(np.float32)
    prefix_v = rng.standard_normal((L0, Hkv, d)).astype(np.float32)
    own_k = rng.standard_normal((4, Hkv, d)).astype(np.float32)
    own_v = rng.standard_normal((4, Hkv, d)).astype(np.float32)
    kc = np.full((P, Hkv, bs, d), np.nan, np.float32)
    vc = np.full((P, Hkv, d, bs), np.nan, np.float32)
    a = TwinAllocator(P, bs)
    a.create(0)
    slots, _ = a.append(0, L0)
    kc, vc = kv_cache_write(prefix_k, prefix_v, kc, vc, np.array(slots), bs=bs, src_dtype="f32",
                            cache_dtype="f32")
    for b in (1, 2, 3):
        a.fork(0, b)
    pairs, new_slots = [], []
    for b in range(4):
        s_, cow = a.append(b, 1)
        pairs += cow
        new_slots += s_
    assert len(pairs) == 3                          # the last writer owns the block by then
    kc, vc = copy_blocks(kc, vc, pairs)
    kc, vc = kv_cache_write(own_k, own_v, kc, vc, np.array(new_slots), bs=bs, src_dtype="f32",
                            cache_dtype="f32")
    tabs, lens = a.tables([0, 1, 2, 3], 8)
    for b in range(4):
        got_k = reassemble(kc, tabs[b], lens[b], bs, "k")
        got_v = reassemble(vc, tabs[b], lens[b], bs, "v")
        assert np.array_equal(got_k, np.concatenate([prefix_k, own_k[b:b + 1]]))
        assert np.array_equal(got_v, np.concatenate([prefix_v, own_v[b:b + 1]]))
    # a copy pair with a block outside the pool is skipped; overlapping pairs are refused
    k2, v2 = copy_blocks(kc, vc, [(0, P + 3)])
    assert np.array_equal(k2, kc, equal_nan=True) and np.array_equal(v2, vc, equal_nan=True)
    with pytest.raises(ValueError):
        copy_blocks(kc, vc, [(1, 2), (2, 3)])


def test_exhaustion_is_all_or_nothing():
    a = TwinAllocator(3, 16)
    a.create(0)
    a.append(0, 20)
    before = (list(a.free), list(a.ref), [list(a.seqs[0][0]), a.seqs[0][1]])
    with pytest.raises(NoBlocks):
        a.append(0, 40)                 # needs 3 more blocks, 1 free
    assert (list(a.free), list(a.ref), [list(a.seqs[0][0]), a.seqs[0][1]]) == before
    a.fork(0, 1)
    a.append(0, 12)                     # shared partial block 1: CoW takes the last free block
    with pytest.raises(NoBlocks):
        a.append(1, 13)                 # block 1 is private again; 33 tokens need a 3rd block
    assert len(a.free) == 0


def _check_invariants(a):
    count = [0] * a.P
    for blocks, length in a.seqs.values():
        assert len(blocks) == -(-length // a.bs)
        for b in blocks:
            count[b] += 1
    assert count == a.ref
    used = {b for blocks, _ in a.seqs.values() for b in blocks}
    assert not (used & set(a.free))
    assert len(a.free) + len(used) == a.P
    assert len(set(a.free)) == len(a.free)


def test_random_op_invariants():
    rng = np.random.default_rng(12)
    a = TwinAllocator(64, 8)
    live, nxt = [], 0
    for _ in range(3000):
        op = rng.integers(4)
        try:
            if op == 0 or not live:
                a.create(nxt)
                live.append(nxt)
                nxt += 1
            elif op == 1:
                a.append(live[rng.integers(len(live))], int(rng.integers(0, 20)))
            elif op == 2:
                a.fork(live[rng.integers(len(live))], nxt)
                live.append(nxt)
                nxt += 1
            else:
                s = live.pop(int(rng.integers(len(live))))
                a.release(s)
        except NoBlocks:
            pass
        _check_invariants(a)


def test_prefix_cache_reuses_the_longest_cached_prefix():
    # A later request with the same prefix points at the blocks already holding
    # it (the daily term's prefix-caching paragraph; "Serving", section 2.6):
    # only full blocks, only a run of leading ones, only with the same extra key.
    rng = np.random.default_rng(8)
    prompt = list(rng.integers(0, 50000, 100))          # 6 full blocks of 16 + 4 tokens
    a = TwinAllocator(64, 16)
    s1, c1 = a.create_prefixed("r1", prompt)
    assert c1 == 0 and len(s1) == 100
    s2, c2 = a.create_prefixed("r2", prompt[:96] + list(rng.integers(0, 50000, 30)))
    assert c2 == 96                                     # 6 shared blocks, not the partial 7th
    t1, t2 = a.seqs["r1"][0], a.seqs["r2"][0]
    assert t2[:6] == t1[:6] and t2[6] != t1[6]
    assert all(a.ref[b] == 2 for b in t1[:6]) and a.ref[t1[6]] == 1
    # differing in block 3 keeps blocks 0-2 only (the hashes chain)
    p3 = list(prompt)
    p3[50] += 1
    _, c3 = a.create_prefixed("r3", p3)
    assert c3 == 48 and a.seqs["r3"][0][:3] == t1[:3] and a.seqs["r3"][0][3] != t1[3]
    # another extra key (tenant salt, adapter id) shares nothing
    _, c4 = a.create_prefixed("r4", prompt, extra=b"tenant-b")
    assert c4 == 0
    # freed blocks stay cached: a new request takes them back off the free list
    a.release("r1"); a.release("r2"); a.release("r3")
    free_before = a.n_free
    _, c5 = a.create_prefixed("r5", prompt)
    assert c5 == 96 and a.seqs["r5"][0][:6] == t1[:6]
    assert a.n_free == free_before - 7                  # 6 taken back + 1 fresh for the tail
    assert not set(a.seqs["r5"][0]) & set(a.free)
    _check_invariants(a)


def test_prefix_cache_forgets_reused_blocks_and_is_all_or_nothing():
    a = TwinAllocator(10, 4)
    p = list(range(16))                                 # 4 full blocks
    a.create_prefixed(0, p)
    a.release(0)                                        # blocks free but still cached
    assert sorted(a.cached.values()) == [0, 1, 2, 3]
    a.create(1)
    a.append(1, 20)                                     # pops 0..4: the cached blocks are reused
    assert a.cached == {}                               # ... and no longer named
    _, c = a.create_prefixed(2, p)
    assert c == 0
    before = (list(a.free), list(a.ref), dict(a.cached))
    with pytest.raises(NoBlocks):
        a.create_prefixed(3, list(range(100, 140)))
    assert (list(a.free), list(a.ref), dict(a.cached)) == before
    _check_invariants(a)


def test_twin_block_hash_is_chained_sha256():
    # the hash of block k covers its parent's hash, its tokens and the extra key
    import hashlib, struct
    toks = [7, 8, 9, 10, 11, 12, 13, 14]
    h0 = hashlib.sha256(bytes(32) + struct.pack("<4i", 7, 8, 9, 10) + b"x").digest()
    h1 = hashlib.sha256(h0 + struct.pack("<4i", 11, 12, 13, 14) + b"x").digest()
    assert TwinAllocator.block_hashes(toks, 4, b"x") == [h0, h1]
    assert len(TwinAllocator.block_hashes(toks[:7], 4)) == 1      # only full blocks
