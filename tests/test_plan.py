"""The host work plan (pkv_build_paged_decode_plan) against an independent
re-derivation of the balanced split in Python, word for word, and its
invariants: every chunk of every segment is listed exactly once, each wave's
entries are consecutive positions, pieces and descriptors agree.

The split (the library's, restated here from its definition): work positions
run sequence-major, then kv head, then position in the (sequence, kv head)
segment; a segment of n 16-token chunks has c + n positions, the first c
standing for its fixed cost (c = 4 / cache element bytes: 1 for fp32, 2 for
bf16, 4 for fp8); V positions are cut into W = min(n_workers,
max(1, ceil(V / 4))) ranges, the first V mod W of them one longer.
"""

import numpy as np
import pytest

import paged_kv_cache_108_amd as pkv
from paged_kv_cache_108_amd import workloads as W

KIND = {"f32": 0, "bf16": 1, "fp8": 2}
ELEM = {"f32": 4, "bf16": 2, "fp8": 1}


def seg_cost(dtype, d):
    return 4 // ELEM[dtype]


def reference_plan(lens, Hkv, d, dtype, max_len, n_workers, n_q=0, G=0):
    """The plan, from the definition (plain Python). n_q > 0: a window plan,
    whose segments are (sequence, kv head, query group) with groups of
    qgs = min(n_q, max(1, 16 T // G)) queries: T = 1 16-column tile when the
    window's n_q G columns fit one, else T = 2."""
    c = seg_cost(dtype, d)
    L = [min(int(x), max_len) for x in lens]
    S = len(L)
    T = 1 if n_q * G <= 16 else 2
    qgs = min(n_q, max(1, 16 * T // G)) if n_q else 1
    n_qg = -(-n_q // qgs) if n_q else 1
    HS = Hkv * n_qg                           # segments per sequence
    segs = []                                 # (i, g2, first position, n chunks)
    pos = 0
    for i in range(S):
        n = -(-L[i] // 16) if L[i] > 0 else 0
        if n == 0:
            continue
        for g in range(HS):
            segs.append((i, g, pos, n))
            pos += c + n
    V = pos
    Wn = min(n_workers, max(1, -(-V // 4))) if V else 0
    q, r = (V // Wn, V % Wn) if Wn else (0, 0)
    start = [w * q + min(w, r) for w in range(Wn + 1)]

    def owner(x):
        big = r * (q + 1)
        return x // (q + 1) if x < big else r + (x - big) // q

    waves = [[] for _ in range(Wn)]
    desc = np.zeros((S * HS, 2), dtype=np.int64)
    for i, g, p, n in segs:
        p0 = p + c
        for kc in range(n):
            waves[owner(p0 + kc)].append([i, g, kc, L[i], 0])
        w_lo, w_hi = owner(p0), owner(p0 + n - 1)
        desc[i * HS + g] = (2 * w_lo + (0 if start[w_lo] >= p else 1), w_hi - w_lo + 1)
    for ent in waves:
        a = 0
        while a < len(ent):
            b = a
            while b + 1 < len(ent) and ent[b + 1][:2] == ent[a][:2]:
                b += 1
            n = -(-ent[a][3] // 16)
            ent[a][4] |= 1
            ent[b][4] |= 2 | (4 if ent[a][2] == 0 and ent[b][2] == n - 1 else 0)
            if a:
                for k in range(a, b + 1):
                    ent[k][4] |= 8
            a = b + 1
    stride = max([len(e) for e in waves] + [1])
    window = [n_q, G, qgs, n_qg] if n_q else [0, 0, 0, 0]
    out = [0x504B5650, 1, n_workers, Wn, S, Hkv, c, stride, max_len, d, KIND[dtype]] + window + [0]
    for w in range(n_workers):
        ent = waves[w] if w < Wn else []
        for k in range(stride):
            if k < len(ent):
                i, g, kc, Li, f = ent[k]
                out += [i, g | (f << 16), kc, Li]
            else:
                out += [-1, 0, 0, 0]
    out += list(desc.reshape(-1))
    return np.array(out, dtype=np.int64)


CASES = [
    ("tiny", None, 1024), ("small", None, 1024), ("llama8b", None, 1024), ("llama8b", "fp8", 1024),
    ("beam", None, 1024), ("llama8b", None, 256), ("small", "fp8", 512),
]


@pytest.mark.parametrize("name,kv,workers", CASES)
def test_plan_matches_the_definition(name, kv, workers):
    w = W.make(name, cache_dtype=kv)
    s = w.spec
    got = pkv.build_paged_decode_plan(w.context_lens, s.Hkv, s.d, KIND[s.cache_dtype], w.max_context_len, workers)
    want = reference_plan(w.context_lens, s.Hkv, s.d, s.cache_dtype, w.max_context_len, workers)
    assert got.shape == want.shape
    assert np.array_equal(got.astype(np.int64), want)


@pytest.mark.parametrize("lens,Hkv,d,dtype,workers", [
    ([0, 1, 17, 0, 300], 2, 64, "bf16", 1024),        # empty sequences, short input: few waves
    ([5000, 3, 3, 3], 8, 128, "fp8", 64),
    ([16] * 700, 1, 64, "f32", 128),                  # many one-chunk segments
    ([0, 0, 0], 4, 128, "bf16", 1024),                # nothing at all
    ([32768] * 4, 8, 128, "bf16", 1024),              # several windows per wave
])
def test_plan_edges(lens, Hkv, d, dtype, workers):
    max_len = max(lens)
    got = pkv.build_paged_decode_plan(lens, Hkv, d, KIND[dtype], max_len, workers)
    want = reference_plan(lens, Hkv, d, dtype, max_len, workers)
    assert np.array_equal(got.astype(np.int64), want)
    # invariants: every (sequence, head, chunk) once; flags consistent
    stride, Wn = int(got[7]), int(got[3])
    ent = got[16:16 + workers * stride * 4].reshape(workers, stride, 4)
    seen = {}
    for w in range(workers):
        rows = [e for e in ent[w] if e[0] >= 0]
        if w >= Wn:
            assert not rows
        for e in rows:
            key = (int(e[0]), int(e[1]) & 0xFFFF, int(e[2]))
            assert key not in seen
            seen[key] = w
    n_chunks = sum((-(-L // 16)) * Hkv for L in lens if L > 0)
    assert len(seen) == n_chunks


def test_plan_clamps_lengths_and_rejects_bad_arguments():
    a = pkv.build_paged_decode_plan([100, 40], 2, 128, 1, 64, 256)
    b = pkv.build_paged_decode_plan([64, 40], 2, 128, 1, 64, 256)
    assert np.array_equal(a, b)                      # lengths above max_context_len count as it
    for bad in [dict(Hkv=0), dict(d=96), dict(workers=0)]:
        kw = dict(Hkv=2, d=128, workers=16)
        kw.update(bad)
        with pytest.raises(pkv.PkvError):
            pkv.build_paged_decode_plan([10, 20], kw["Hkv"], kw["d"], 1, 32, kw["workers"])


@pytest.mark.parametrize("name,kv,n_q,workers", [
    ("llama8b", None, 4, 1024), ("llama8b", None, 8, 1024), ("llama8b", None, 16, 1024),
    ("small", None, 4, 1024), ("small", "fp8", 3, 2048), ("tiny", None, 20, 1024),
])
def test_window_plan_matches_the_definition(name, kv, n_q, workers):
    w = W.make(name, cache_dtype=kv)
    s = w.spec
    G = s.Hq // s.Hkv
    got = pkv.build_paged_window_plan(w.context_lens, n_q, s.Hq, s.Hkv, s.d, KIND[s.cache_dtype],
                                      w.max_context_len, workers)
    want = reference_plan(w.context_lens, s.Hkv, s.d, s.cache_dtype, w.max_context_len, workers, n_q=n_q, G=G)
    assert got.shape == want.shape
    assert np.array_equal(got.astype(np.int64), want)
    qgs = int(got[13])
    assert got[11] == n_q and got[12] == G and got[14] * qgs >= n_q
    # one tile when the window fits it, else two tiles (32 columns) per group
    assert qgs * G <= (16 if n_q * G <= 16 else 32) and (n_q * G <= 16 or qgs == min(n_q, max(1, 32 // G)))


def test_window_plan_long_lengths():
    # the long-context shape (16 x 32768 tokens, 8 kv heads, G 8), lengths only
    lens = [32768] * 16
    got = pkv.build_paged_window_plan(lens, 3, 64, 8, 128, 1, 32768, 1024)
    want = reference_plan(lens, 8, 128, "bf16", 32768, 1024, n_q=3, G=8)
    assert np.array_equal(got.astype(np.int64), want)


def test_window_plan_of_one_query_is_the_decode_plan_but_the_header():
    w = W.make("llama8b")
    s = w.spec
    dec = pkv.build_paged_decode_plan(w.context_lens, s.Hkv, s.d, 1, w.max_context_len, 1024)
    win = pkv.build_paged_window_plan(w.context_lens, 1, s.Hq, s.Hkv, s.d, 1, w.max_context_len, 1024)
    assert np.array_equal(dec[16:], win[16:]) and np.array_equal(dec[:11], win[:11])
    assert list(win[11:15]) == [1, s.Hq // s.Hkv, 1, 1] and list(dec[11:15]) == [0, 0, 0, 0]


def test_window_plan_rejects_bad_arguments():
    for kw in [dict(n_q=0), dict(Hq=12, Hkv=8), dict(Hq=34, Hkv=2)]:
        a = dict(n_q=2, Hq=8, Hkv=2)
        a.update(kw)
        with pytest.raises(pkv.PkvError):
            pkv.build_paged_window_plan([10, 20], a["n_q"], a["Hq"], a["Hkv"], 64, 1, 32, 16)


def test_shared_blocks_mark():
    """pkv_plan_mark_shared_blocks sets the flags word (header word 15) exactly
    when a block id repeats among the blocks the sequences read, and changes no
    other word."""
    beam = W.make("beam")
    s = beam.spec
    plan = pkv.build_paged_decode_plan(beam.context_lens, s.Hkv, s.d, 1, beam.max_context_len, 1024)
    before = plan.copy()
    assert pkv.plan_mark_shared_blocks(plan, beam.block_tables, beam.context_lens, s.bs)
    assert plan[15] == 1 and np.array_equal(np.delete(plan, 15), np.delete(before, 15))
    w = W.make("llama8b")
    s = w.spec
    plan = pkv.build_paged_decode_plan(w.context_lens, s.Hkv, s.d, 1, w.max_context_len, 1024)
    assert not pkv.plan_mark_shared_blocks(plan, w.block_tables, w.context_lens, s.bs) and plan[15] == 0
    # a repeat past a row's read range does not count; one inside it does
    tables = np.array([[3, 4, 5, -1], [6, 7, 3, -1]], dtype=np.int32)
    lens = [40, 20]                                          # 3 and 2 blocks of 16 are read
    plan = pkv.build_paged_decode_plan(lens, 1, 64, 1, 64, 16)
    assert not pkv.plan_mark_shared_blocks(plan, tables, lens, 16)
    assert pkv.plan_mark_shared_blocks(plan, tables, [40, 40], 16) and plan[15] == 1
    assert not pkv.plan_mark_shared_blocks(plan, tables, [40, 20], 16) and plan[15] == 0    # cleared again
    same_row = np.array([[9, 9, -1, -1], [1, 2, -1, -1]], dtype=np.int32)
    assert pkv.plan_mark_shared_blocks(plan, same_row, [20, 20], 16)


def test_plan_rejects_lengths_past_two_to_the_thirty():
    big = 2**31 - 1
    with pytest.raises(pkv.PkvError):
        pkv.build_paged_decode_plan([big, 5], 1, 64, 1, big, 16)
    with pytest.raises(pkv.PkvError):
        pkv.build_paged_window_plan([big, 5], 2, 4, 1, 64, 1, big, 16)
    # lengths past max_context_len are clamped, and the mark reads no more of a
    # table row than it holds
    plan = pkv.build_paged_decode_plan([big, 5], 1, 64, 1, 64, 16)
    tables = np.array([[3, 4], [5, -1]], dtype=np.int32)
    assert not pkv.plan_mark_shared_blocks(plan, tables, [big, 5], 16)
    assert pkv.plan_mark_shared_blocks(plan, np.array([[3, 4], [4, -1]], dtype=np.int32), [big, 5], 16)


@pytest.mark.parametrize("n_q,Hq,Hkv,d", [(1, 32, 8, 128), (4, 32, 8, 128), (5, 32, 8, 128), (8, 32, 8, 128),
                                          (16, 32, 8, 128), (5, 14, 2, 64), (3, 16, 1, 128), (20, 2, 2, 64)])
def test_window_plan_workspace_matches_its_grouping(n_q, Hq, Hkv, d):
    """The planned window call's workspace holds two records per wave of the
    plan's G * qgs columns, with the grouping the plan header states, which is
    the unplanned call's (its workspace has the same column count)."""
    n_workers = 1024
    plan = pkv.build_paged_window_plan([300, 40, 7000], n_q, Hq, Hkv, d, 1, 8192, n_workers)
    G = Hq // Hkv
    qgs, n_qg = int(plan[13]), int(plan[14])
    cols = G * qgs
    want = -(-(2 * n_workers * cols * (d + 2) * 4) // 256) * 256
    got = int(pkv.lib().pkv_paged_window_plan_workspace_size(n_workers, n_q, Hq, Hkv, d))
    assert got == want
    T = 1 if n_q * G <= 16 else 2
    assert cols <= 16 * T and qgs == min(n_q, max(1, 16 * T // G)) and n_qg == -(-n_q // qgs)
