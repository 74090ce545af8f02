"""CPU tests of the C ABI: exports, host allocator against the oracle's twin,
builders against the oracle, and every argument check of the device entry
points (all of which return before any HIP call)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import paged_kv_cache_108_amd as pkv
from paged_kv_cache_108_amd import _lib
from paged_kv_cache_108_amd import workloads as W

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 16
    handle = ctypes.CDLL(pkv.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"
    assert pkv.version().startswith("pkv")


# ------------------------------------------------------------------ allocator parity
def _run_both(ops, P, bs):
    a, t = pkv.Allocator(P, bs), oracle.TwinAllocator(P, bs)
    for op in ops:
        kind = op[0]
        if kind == "create":
            a.create(op[1]); t.create(op[1])
        elif kind == "append":
            try:
                got = a.append(op[1], op[2])
                got = (list(got[0]), got[1])
            except pkv.NoBlocks:
                got = "noblocks"
            try:
                want = t.append(op[1], op[2])
            except oracle.NoBlocks:
                want = "noblocks"
            assert got == want, op
        elif kind == "fork":
            a.fork(op[1], op[2]); t.fork(op[1], op[2])
        elif kind == "free":
            a.release(op[1]); t.release(op[1])
    return a, t


def _random_ops(seed, n=1500):
    rng = np.random.default_rng(seed)
    ops, live, nxt = [], [], 0
    for _ in range(n):
        k = rng.integers(5)
        if k == 0 or not live:
            ops.append(("create", nxt)); live.append(nxt); nxt += 1
        elif k in (1, 2):
            ops.append(("append", int(live[rng.integers(len(live))]), int(rng.integers(0, 40))))
        elif k == 3:
            ops.append(("fork", int(live[rng.integers(len(live))]), nxt)); live.append(nxt); nxt += 1
        else:
            ops.append(("free", int(live.pop(int(rng.integers(len(live)))))))
    return ops


@pytest.mark.parametrize("seed,P,bs", [(0, 64, 8), (1, 200, 16), (2, 30, 32), (3, 500, 16)])
def test_allocator_matches_twin(seed, P, bs):
    ops = _random_ops(seed)
    a, t = _run_both(ops, P, bs)
    ids = sorted(t.seqs)
    maxb = max([len(t.seqs[s][0]) for s in ids] + [1])
    tab, lens = a.tables(ids, maxb)
    ttab, tlens = t.tables(ids, maxb)
    assert np.array_equal(tab, np.array(ttab, dtype=np.int32).reshape(len(ids), maxb))
    assert list(lens) == tlens
    sa, st = a.stats(), t.stats()
    for k in ("num_blocks", "free_blocks", "used_blocks", "slots_allocated", "tokens_stored"):
        assert sa[k] == st[k], k
    assert abs(sa["waste"] - st["waste"]) < 1e-12


def test_allocator_reproduces_beam_layout():
    # The generator's beam tables are the sequential ids a first-pop-0 pool
    # hands out for: prefix append, 3 forks, private appends.
    private = np.random.default_rng([108, 4, 0]).integers(1, 201, 128)
    for bs in (8, 16, 32):
        seq_tab, lens, used = W.beam_layout(bs, private)
        a = pkv.Allocator(used, bs)
        for g in range(32):
            a.create(4 * g)
            a.append(4 * g, 1024)
            for b in (1, 2, 3):
                a.fork(4 * g, 4 * g + b)
            for b in range(4):
                _, cow = a.append(4 * g + b, int(private[4 * g + b]))
                assert cow == []                       # block-aligned prefix: never copies
        tab, L = a.tables(list(range(128)), seq_tab.shape[1])
        assert np.array_equal(tab, seq_tab) and np.array_equal(L, lens)
        assert a.stats()["free_blocks"] == 0


def test_allocator_reproduces_churned_pool():
    ops = W.churn_ops()
    a = pkv.Allocator(36045, 16)
    for op in ops:
        if op[0] == "alloc":
            a.create(op[1] + 10**6)
            a.append(op[1] + 10**6, op[2] * 16)
        else:
            a.release(op[1] + 10**6)
    for s in range(16):
        a.create(s)
    for j in range(2048):
        for s in range(16):
            a.append(s, 16)
    tab, lens = a.tables(list(range(16)), 2048)
    assert np.array_equal(tab, W.churned_tables()) and set(lens) == {32768}


def test_allocator_cow_pair_and_errors():
    a = pkv.Allocator(6, 16)
    a.create(1)
    a.append(1, 20)
    a.fork(1, 2)
    slots, cow = a.append(2, 1)
    assert cow == [(1, 2)] and list(slots) == [2 * 16 + 4]
    assert a.info(2) == (21, 2)
    with pytest.raises(pkv.PkvError, match="PKV_E_STATE"):
        a.create(1)
    with pytest.raises(pkv.PkvError, match="PKV_E_NOT_FOUND"):
        a.append(99, 1)
    with pytest.raises(pkv.PkvError, match="PKV_E_NOT_FOUND"):
        a.release(99)
    with pytest.raises(pkv.PkvError, match="PKV_E_STATE"):
        a.fork(1, 2)
    with pytest.raises(pkv.PkvError, match="PKV_E_INVALID"):
        a.append(1, -1)
    before = a.stats()
    with pytest.raises(pkv.NoBlocks):
        a.append(1, 16 * 10)
    assert a.stats() == before
    with pytest.raises(pkv.PkvError, match="PKV_E_INVALID"):
        a.tables([1, 2], 1)                          # 2 blocks > max_blocks
    with pytest.raises(pkv.PkvError, match="PKV_E_INVALID"):
        pkv.Allocator(0, 16)
    # a CoW with no place to report it is refused without changing anything
    lib = pkv.lib()
    slots = np.zeros(1, dtype=np.int64)
    a.fork(2, 3)
    st = lib.pkv_seq_append(a._h, 3, 1, slots.ctypes.data_as(_lib.P_i64), None, None, None)
    assert st == _lib.PKV_E_INVALID and a.info(3) == (21, 2)


def test_slots_and_waste_match_oracle(golden):
    g = golden("worked_example.json")
    w = pkv.waste_stats(g["lengths"], 16, g["reserve_max_len"])
    assert (w["paged_slots"], w["naive_slots"], w["used"]) == (2608, 10240, 2581)
    assert abs(w["waste_paged"] - oracle.waste_fraction(g["lengths"], 2608)) < 1e-15
    assert round(100 * w["waste_naive"], 1) == 74.8
    rng = np.random.default_rng(0)
    for bs in (8, 16, 32):
        tab = rng.permutation(400)[:120].reshape(6, 20).astype(np.int32)
        pos = rng.integers(-2, 20 * bs, 6).astype(np.int32)
        got = pkv.slots_from_tables(tab, pos, bs)
        assert np.array_equal(got, oracle.slots_for_positions(tab, pos, bs))
    with pytest.raises(pkv.PkvError):
        pkv.slots_from_tables(np.array([[3, -1]]), np.array([20]), 16)   # unallocated block
    with pytest.raises(pkv.PkvError):
        pkv.slots_from_tables(np.array([[3]]), np.array([16]), 16)       # beyond the table


def test_decode_slots_for_workloads_match_oracle():
    w = W.make("tiny")
    got = pkv.slots_from_tables(w.block_tables, w.context_lens - 1, w.spec.bs)
    assert np.array_equal(got, oracle.decode_slots(w.block_tables, w.context_lens, w.spec.bs))


# ------------------------------------------------------------------ device argument checks
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def _attn(**kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, tab=FAKE, lens=FAKE, S=4, Hq=8, Hkv=2, d=128, bs=16,
             P=100, maxb=10, maxlen=160, scale=0.1, ks=1.0, vs=1.0, qd=1, cd=1, part=512,
             ws=FAKE, wsb=0, stream=None)
    a.update(kw)
    return pkv.lib().pkv_paged_decode_attn(
        a["out"], a["q"], a["k"], a["v"], a["tab"], a["lens"], a["S"], a["Hq"], a["Hkv"], a["d"],
        a["bs"], a["P"], a["maxb"], a["maxlen"], a["scale"], a["ks"], a["vs"], a["qd"], a["cd"],
        a["part"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(Hq=7), dict(Hq=34, Hkv=2), dict(d=96), dict(bs=4), dict(bs=48), dict(bs=256), dict(P=0),
    dict(maxb=0), dict(maxlen=161), dict(maxlen=-1), dict(qd=0), dict(qd=1, cd=0),
    dict(qd=2, cd=2), dict(part=16), dict(part=-32), dict(part=-2), dict(scale=float("inf")),
    dict(qd=1, cd=2, ks=float("nan")), dict(out=None), dict(tab=None), dict(S=-1), dict(Hkv=0),
    dict(maxb=1 << 24, bs=128, maxlen=(1 << 30) + 1),          # above 2^30, within the table
])
def test_attn_rejects_invalid_arguments(kw):
    assert _attn(**kw) == _lib.PKV_E_INVALID
    assert pkv.last_error()


def test_attn_workspace_checks():
    need = pkv.paged_decode_attn_workspace_size(4, 8, 2, 128, 2000, 512)
    assert need == 4 * 8 * 4 * 130 * 4
    assert pkv.paged_decode_attn_workspace_size(4, 8, 2, 128, 512, 512) == 0
    assert pkv.paged_decode_attn_workspace_size(4, 8, 2, 128, 2000, 0) == 0
    bal = pkv.paged_decode_attn_workspace_size(4, 8, 2, 128, 2000, pkv.PKV_PARTITION_BALANCED)
    assert bal == 2 * 4096 * 4 * 130 * 4 + 2 * 4 * 2 * 4     # records + segment descriptors
    assert pkv.paged_decode_attn_workspace_size(4, 7, 2, 128, 2000, 512) == 0     # invalid
    assert _attn(part=pkv.PKV_PARTITION_BALANCED, wsb=bal - 1) == _lib.PKV_E_WORKSPACE
    assert _attn(maxb=200, maxlen=2000, wsb=need - 1) == _lib.PKV_E_WORKSPACE
    assert _attn(maxb=200, maxlen=2000, ws=None, wsb=need) == _lib.PKV_E_WORKSPACE
    assert _attn(S=0) == _lib.PKV_OK                 # nothing to do, nothing launched


def _write(**kw):
    a = dict(kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, sm=FAKE, T=3, Hkv=2, d=64, bs=16, P=10, sd=1,
             cd=1, ki=1.0, vi=1.0)
    a.update(kw)
    return pkv.lib().pkv_kv_cache_write(a["kn"], a["vn"], a["kc"], a["vc"], a["sm"], a["T"],
                                        a["Hkv"], a["d"], a["bs"], a["P"], a["sd"], a["cd"],
                                        a["ki"], a["vi"], None)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(Hkv=0), dict(d=32), dict(bs=12), dict(P=0), dict(sd=0, cd=1),
    dict(sd=2, cd=2), dict(sd=0, cd=2), dict(sd=1, cd=2, ki=0.0), dict(sd=1, cd=2, vi=float("inf")),
    dict(kn=None), dict(sm=None),
])
def test_write_rejects_invalid_arguments(kw):
    assert _write(**kw) == _lib.PKV_E_INVALID


def test_write_zero_tokens_is_a_noop():
    assert _write(T=0, kn=None, vn=None, kc=None, vc=None, sm=None) == _lib.PKV_OK


def _copy(**kw):
    a = dict(kc=FAKE, vc=FAKE, src=FAKE, dst=FAKE, n=3, P=10, Hkv=2, d=64, bs=16, cd=1)
    a.update(kw)
    return pkv.lib().pkv_copy_blocks(a["kc"], a["vc"], a["src"], a["dst"], a["n"], a["P"], a["Hkv"],
                                     a["d"], a["bs"], a["cd"], None)


@pytest.mark.parametrize("kw", [
    dict(n=-1), dict(n=11), dict(P=0), dict(Hkv=0), dict(d=96), dict(bs=4), dict(cd=7),
    dict(kc=None), dict(dst=None),
])
def test_copy_blocks_rejects_invalid_arguments(kw):
    assert _copy(**kw) == _lib.PKV_E_INVALID
    assert "copy_blocks" in pkv.last_error()


def test_copy_blocks_zero_pairs_is_a_noop():
    assert _copy(n=0, kc=None, vc=None, src=None, dst=None) == _lib.PKV_OK


# ------------------------------------------------------------------ prefix caching
def test_block_hashes_match_sha256_of_the_chain():
    # lengths of parent + tokens + extra cross every SHA-256 padding boundary
    rng = np.random.default_rng(3)
    for bs in (1, 2, 8, 16):
        for extra_len in (0, 1, 3, 7, 8, 19, 20, 23, 24, 55, 56, 64, 120):
            toks = rng.integers(-2**31, 2**31, 3 * bs + 1).astype(np.int32)
            extra = bytes(rng.integers(0, 256, extra_len, dtype=np.uint8))
            got = pkv.block_hashes(toks, bs, extra)
            want = oracle.TwinAllocator.block_hashes(list(toks), bs, extra)
            assert [bytes(r) for r in got] == want, (bs, extra_len)
    assert pkv.block_hashes(np.arange(5, dtype=np.int32), 16).shape == (0, 32)


def _prefixed_ops(seed, n=600):
    rng = np.random.default_rng(seed)
    prefixes = [list(rng.integers(0, 1000, 80)) for _ in range(4)]
    ops, live, nxt = [], [], 0
    for _ in range(n):
        k = rng.integers(6)
        if k <= 1 or not live:
            base = prefixes[rng.integers(4)]
            cut = int(rng.integers(0, 81))
            toks = base[:cut] + list(rng.integers(0, 1000, rng.integers(0, 40)))
            extra = b"" if rng.integers(4) else b"salt"
            ops.append(("prefixed", nxt, toks, extra)); live.append(nxt); nxt += 1
        elif k == 2:
            ops.append(("append", int(live[rng.integers(len(live))]), int(rng.integers(0, 20))))
        elif k == 3:
            ops.append(("fork", int(live[rng.integers(len(live))]), nxt)); live.append(nxt); nxt += 1
        else:
            ops.append(("free", int(live.pop(int(rng.integers(len(live)))))))
    return ops


@pytest.mark.parametrize("seed,P,bs", [(0, 48, 8), (1, 120, 16), (2, 30, 4)])
def test_prefix_allocator_matches_twin(seed, P, bs):
    a, t = pkv.Allocator(P, bs), oracle.TwinAllocator(P, bs)
    for op in _prefixed_ops(seed):
        if op[0] == "prefixed":
            try:
                s_, c = a.create_prefixed(op[1], op[2], op[3])
                got = (list(s_), c)
            except pkv.NoBlocks:
                got = "noblocks"
            try:
                want = t.create_prefixed(op[1], op[2], op[3])
            except oracle.NoBlocks:
                want = "noblocks"
            assert got == want, op[:2]
            if got == "noblocks":
                a.create(op[1]); t.create(op[1])
        elif op[0] == "append":
            try:
                g = a.append(op[1], op[2]); g = (list(g[0]), g[1])
            except pkv.NoBlocks:
                g = "noblocks"
            try:
                wnt = t.append(op[1], op[2])
            except oracle.NoBlocks:
                wnt = "noblocks"
            assert g == wnt
        elif op[0] == "fork":
            a.fork(op[1], op[2]); t.fork(op[1], op[2])
        else:
            a.release(op[1]); t.release(op[1])
    ids = sorted(t.seqs)
    maxb = max([len(t.seqs[s][0]) for s in ids] + [1])
    tab, lens = a.tables(ids, maxb)
    ttab, tlens = t.tables(ids, maxb)
    assert np.array_equal(tab, np.array(ttab, dtype=np.int32).reshape(len(ids), maxb))
    assert a.prefix_stats() == t.prefix_stats()
    assert a.prefix_stats()["hit_blocks"] > 0
    sa, st = a.stats(), t.stats()
    assert sa["free_blocks"] == st["free_blocks"] and sa["tokens_stored"] == st["tokens_stored"]


def test_decode_step_rejects_invalid_arguments():
    lib = pkv.lib()

    def step(**kw):
        a = dict(kn=FAKE, vn=FAKE, cd=1, qd=1, ki=1.0, vi=1.0, wsb=1 << 30)
        a.update(kw)
        return lib.pkv_paged_decode_step(FAKE, FAKE, a["kn"], a["vn"], FAKE, FAKE, FAKE, FAKE, 4, 8, 2,
                                         128, 16, 100, 10, 160, 0.1, 1.0, 1.0, a["ki"], a["vi"],
                                         a["qd"], a["cd"], FAKE, a["wsb"], None)
    assert step(kn=None) == _lib.PKV_E_INVALID
    assert step(vn=None) == _lib.PKV_E_INVALID
    assert step(cd=2, ki=0.0) == _lib.PKV_E_INVALID
    assert step(cd=2, vi=float("inf")) == _lib.PKV_E_INVALID
    assert step(wsb=16) == _lib.PKV_E_WORKSPACE


def _shared(**kw):
    a = dict(out=FAKE, q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, ptab=FAKE, plen=FAKE, pmaxb=64,
             pmax=1024, stab=FAKE, slen=FAKE, smaxb=16, smax=200, ng=8, M=4, Hq=32, Hkv=8, d=128, bs=16,
             P=4000, scale=0.1, ks=1.0, vs=1.0, ki=1.0, vi=1.0, qd=1, cd=1, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return pkv.lib().pkv_paged_shared_prefix_decode(
        a["out"], a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["ptab"], a["plen"], a["pmaxb"], a["pmax"],
        a["stab"], a["slen"], a["smaxb"], a["smax"], a["ng"], a["M"], a["Hq"], a["Hkv"], a["d"], a["bs"],
        a["P"], a["scale"], a["ks"], a["vs"], a["ki"], a["vi"], a["qd"], a["cd"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=0), _lib.PKV_E_INVALID), (dict(M=4097), _lib.PKV_E_INVALID), (dict(ng=-1), _lib.PKV_E_INVALID),
    (dict(kn=None), _lib.PKV_E_INVALID), (dict(vn=None), _lib.PKV_E_INVALID),
    (dict(Hq=30), _lib.PKV_E_INVALID), (dict(d=96), _lib.PKV_E_INVALID), (dict(bs=12), _lib.PKV_E_INVALID),
    (dict(pmaxb=0), _lib.PKV_E_INVALID), (dict(pmax=1025), _lib.PKV_E_INVALID),
    (dict(smax=257), _lib.PKV_E_INVALID), (dict(qd=0), _lib.PKV_E_INVALID),
    (dict(cd=2, ki=0.0), _lib.PKV_E_INVALID), (dict(scale=float("nan")), _lib.PKV_E_INVALID),
    (dict(ptab=None), _lib.PKV_E_INVALID), (dict(slen=None), _lib.PKV_E_INVALID),
    (dict(wsb=1024), _lib.PKV_E_WORKSPACE), (dict(ws=None), _lib.PKV_E_WORKSPACE),
])
def test_shared_prefix_decode_rejects_invalid_arguments(kw, status):
    # every check, of both passes, runs before any launch
    assert _shared(**kw) == status
    assert "shared_prefix_decode" in pkv.last_error()


def test_shared_prefix_decode_workspace_and_empty_call():
    lib = pkv.lib()
    n = lib.pkv_paged_shared_prefix_decode_workspace_size(32, 4, 32, 8, 128)
    pre = lib.pkv_paged_multi_query_attn_workspace_size(32, 4, 32, 8, 128)
    suf = lib.pkv_paged_decode_attn_workspace_size(128, 32, 8, 128, 0, pkv.PKV_PARTITION_BALANCED)
    rows = 128 * 32
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    assert n == up(pre + 2 * 128 * 8 * 4) + up(suf) + 2 * (up(rows * 128 * 4) + up(rows * 4))
    assert lib.pkv_paged_shared_prefix_decode_workspace_size(0, 4, 32, 8, 128) == 0
    assert lib.pkv_paged_shared_prefix_decode_workspace_size(4, 4, 30, 8, 128) == 0
    assert _shared(ng=0, out=None, q=None, ws=None, wsb=0) == _lib.PKV_OK     # nothing to do


def test_lse_and_merge_entry_points_reject_invalid_arguments():
    lib = pkv.lib()
    rc = lib.pkv_paged_decode_attn_lse(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 2, 128, 16, 100, 10,
                                       160, 0.1, 1.0, 1.0, 1, 1, FAKE, 1 << 30, None)
    assert rc == _lib.PKV_E_INVALID                                   # lse is required
    rc = lib.pkv_paged_shared_prefix_attn(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 8, 2, 128, 16, 100,
                                          10, 160, 0.1, 1.0, 1.0, 1, 1, FAKE, 1 << 30, None)
    assert rc == _lib.PKV_E_INVALID
    rc = lib.pkv_merge_attn_states(FAKE, None, FAKE, FAKE, FAKE, FAKE, -1, 128, None)
    assert rc == _lib.PKV_E_INVALID
    rc = lib.pkv_merge_attn_states(FAKE, None, FAKE, FAKE, FAKE, FAKE, 10, 96, None)
    assert rc == _lib.PKV_E_INVALID
    rc = lib.pkv_merge_attn_states(FAKE, None, None, FAKE, FAKE, FAKE, 10, 128, None)
    assert rc == _lib.PKV_E_INVALID
    assert lib.pkv_merge_attn_states(None, None, None, None, None, None, 0, 128, None) == _lib.PKV_OK


def _plan_properties_hold(tab, lens, M, bs):
    """Every member's prefix blocks followed by its suffix blocks are exactly its
    own first ceil(L/bs) table entries; the prefix never holds a member's last
    block; prefixes are whole blocks."""
    pre_tab, pre_len, suf_tab, suf_len = pkv.shared_prefix_plan(tab, lens, M, bs)
    for g in range(len(pre_len)):
        assert pre_len[g] % bs == 0
        k = pre_len[g] // bs
        for i in range(g * M, (g + 1) * M):
            L = max(int(lens[i]), 0)
            nb = -(-L // bs)
            assert k <= max(nb - 1, 0)
            assert pre_len[g] + suf_len[i] == L
            joined = list(pre_tab[g, :k]) + list(suf_tab[i, :nb - k])
            assert joined == list(tab[i, :nb])
            assert np.all(suf_tab[i, nb - k:] == -1)
        assert np.all(pre_tab[g, k:] == -1)
    return pre_tab, pre_len, suf_tab, suf_len


def test_shared_prefix_plan_on_the_beam_layout():
    for bs in (8, 16, 32):
        w = W.make("beam", bs=bs)
        pre_tab, pre_len, suf_tab, suf_len = _plan_properties_hold(w.block_tables, w.context_lens, 4, bs)
        assert np.all(pre_len == 1024)                  # each group's whole prompt, every block size
        assert np.array_equal(suf_len, w.context_lens - 1024)
        assert np.array_equal(pre_tab[:, :1024 // bs], w.block_tables[::4, :1024 // bs])


def test_shared_prefix_plan_edges():
    bs = 4
    tab = np.full((6, 8), -1, dtype=np.int32)
    tab[0, :4] = [10, 11, 12, 13]        # group 0 (M = 3): members share blocks 10, 11, 12
    tab[1, :5] = [10, 11, 12, 20, 21]
    tab[2, :4] = [10, 11, 12, 30]
    tab[3, :2] = [40, 41]                # group 1: differs at block 0 -> nothing shared
    tab[4, :2] = [50, 41]
    lens = np.array([16, 18, 13, 8, 6, 0])
    pre_tab, pre_len, suf_tab, suf_len = _plan_properties_hold(tab, lens, 3, bs)
    # member 0 fills block 13 exactly (L = 16): its last block is 13, so the
    # prefix stops before it, at 3 blocks
    assert list(pre_len) == [12, 0]
    assert list(suf_len) == [4, 6, 1, 8, 6, 0]
    # groups of one: everything before the last block is "shared"
    _, pre1, _, suf1 = _plan_properties_hold(tab, lens, 1, bs)
    assert list(pre1) == [12, 16, 12, 4, 4, 0] and list(suf1) == [4, 2, 1, 4, 2, 0]
    # groups of two: rows 0/1 share 3 blocks, rows 2/3 none, rows 4/5 none (row 5 is empty)
    _, pre2, _, _ = _plan_properties_hold(tab, lens, 2, bs)
    assert list(pre2) == [12, 0, 0]
    with pytest.raises(ValueError):
        pkv.shared_prefix_plan(tab, lens, 4, bs)         # 6 rows are not groups of 4
    out = [np.empty(48, dtype=np.int32), np.empty(6, dtype=np.int32)] * 2
    ptr = lambda a: a.ctypes.data_as(_lib.P_i32)          # noqa: E731
    t32, l32 = np.ascontiguousarray(tab), lens.astype(np.int32)
    assert pkv.lib().pkv_shared_prefix_plan(ptr(t32), ptr(l32), 6, 8, 4, bs, *map(ptr, out)) == _lib.PKV_E_INVALID
    with pytest.raises(pkv.PkvError):
        pkv.shared_prefix_plan(tab, np.array([33, 0, 0, 0, 0, 0]), 3, bs)   # beyond 8 blocks of 4
