"""Pins of the oracle's paged decode attention.

The pages print no attention outputs. What they fix, and what pins the oracle:
* the result is ordinary attention over the sequence in logical order, whatever
  the layout: brute force (pure-Python loops) and PyTorch's
  scaled_dot_product_attention on contiguous K/V built independently of the
  oracle's reassembly;
* the output does not change when physical block ids are permuted or when
  sequences share prefix blocks instead of holding private copies;
* closed forms (one token, constant V, equal keys, zero query, empty sequence);
* the split-K merge equals the single pass;
* the log-sum-exp state: closed forms and brute force; merging the states of a
  prefix and a suffix (found through their own tables) gives the whole
  sequence's attention.
Mutation checks at the end plant plausible mistakes in the oracle and confirm
that one of these pins catches each.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt


def _scatter(Kc, Vc, bs, P, rng, shared_prefix=None):
    """Place contiguous per-sequence K/V (lists of [L][Hkv][d] float32) into pools
    in the documented layout, one token at a time, with a random block order."""
    S = len(Kc)
    Hkv, d = Kc[0].shape[1], Kc[0].shape[2]
    nb = [-(-len(k) // bs) for k in Kc]
    maxb = max(max(nb), 1)
    perm = list(rng.permutation(P))
    kpool = np.full((P, Hkv, bs, d), np.nan, dtype=np.float32)
    # V: sub-tiles of vs = min(bs, 16) tokens, channel-major; [P][Hkv][d][bs] for bs <= 16
    vs = min(bs, 16)
    vpool = np.full((P, Hkv, bs // vs, d, vs), np.nan, dtype=np.float32)
    tables = np.full((S, maxb), -1, dtype=np.int32)
    for i in range(S):
        for j in range(nb[i]):
            tables[i, j] = perm.pop()
        for t in range(len(Kc[i])):
            b, o = tables[i, t // bs], t % bs
            for h in range(Hkv):
                for c in range(d):
                    kpool[b, h, o, c] = Kc[i][t, h, c]
                    vpool[b, h, o // vs, c, o % vs] = Vc[i][t, h, c]
    if bs <= 16:
        vpool = vpool.reshape(P, Hkv, d, bs)
    return kpool, vpool, tables


def _sdpa(q_i, K, V, sigma):
    """torch SDPA in float64; kv head h // G serves q head h."""
    Hq, d = q_i.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    if L == 0:
        return np.zeros((Hq, d))
    q = torch.from_numpy(q_i).reshape(1, Hq, 1, d)
    k = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
    v = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=float(sigma))
    return o.reshape(Hq, d).numpy()


def _loops(q_i, K, V, sigma):
    """Pure-Python attention, one head and one token at a time."""
    Hq, d = q_i.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    out = np.zeros((Hq, d))
    for h in range(Hq):
        g = h // G
        s = [sigma * sum(float(q_i[h, c]) * float(K[t, g, c]) for c in range(d)) for t in range(L)]
        if not s:
            continue
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = sum(w)
        for c in range(d):
            out[h, c] = sum(w[t] * float(V[t, g, c]) for t in range(L)) / z
    return out


def _case(seed, lens, Hq, Hkv, d, bs, pool_extra=7):
    rng = np.random.default_rng(seed)
    Kc = [rng.standard_normal((L, Hkv, d)).astype(np.float32) for L in lens]
    Vc = [rng.standard_normal((L, Hkv, d)).astype(np.float32) for L in lens]
    q = rng.standard_normal((len(lens), Hq, d)).astype(np.float32)
    P = sum(-(-L // bs) for L in lens) + pool_extra
    kp, vp, tab = _scatter(Kc, Vc, bs, P, rng)
    return q, Kc, Vc, kp, vp, tab


CASES = [
    (1, [5, 17, 1, 33], 4, 4, 8, 4),
    (2, [16, 3, 40], 8, 2, 16, 8),
    (3, [100, 2], 6, 3, 8, 16),
    (4, [31, 32, 33, 0, 1], 7, 1, 4, 16),
    (5, [64, 9], 16, 2, 32, 32),
]


@pytest.mark.parametrize("seed,lens,Hq,Hkv,d,bs", CASES)
def test_against_sdpa(seed, lens, Hq, Hkv, d, bs):
    q, Kc, Vc, kp, vp, tab = _case(seed, lens, Hq, Hkv, d, bs)
    sigma = np.float32(1 / math.sqrt(d))
    out = oracle.paged_decode_attn(q, kp, vp, tab, np.array(lens), bs=bs, softmax_scale=sigma,
                                   q_dtype="f32", cache_dtype="f32")
    for i, L in enumerate(lens):
        ref = _sdpa(q[i].astype(np.float64), Kc[i].astype(np.float64), Vc[i].astype(np.float64),
                    np.float64(sigma))
        np.testing.assert_allclose(out[i], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed,lens,Hq,Hkv,d,bs", CASES[:3])
def test_against_loops(seed, lens, Hq, Hkv, d, bs):
    q, Kc, Vc, kp, vp, tab = _case(seed, lens, Hq, Hkv, d, bs)
    sigma = np.float32(0.37)
    out = oracle.paged_decode_attn(q, kp, vp, tab, np.array(lens), bs=bs, softmax_scale=sigma,
                                   q_dtype="f32", cache_dtype="f32")
    for i in range(len(lens)):
        ref = _loops(q[i], Kc[i], Vc[i], float(sigma))
        np.testing.assert_allclose(out[i], ref, rtol=1e-12, atol=1e-12)


def test_bf16_storage_widens_exactly():
    q, Kc, Vc, kp, vp, tab = _case(11, [20, 7], 4, 2, 16, 8)
    lens = np.array([20, 7])

    def bits(x):
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    def back(x):
        return torch.from_numpy(x).to(torch.bfloat16).double().numpy()

    out = oracle.paged_decode_attn(bits(q), bits(kp), bits(vp), tab, lens, bs=8,
                                   softmax_scale=0.25, q_dtype="bf16", cache_dtype="bf16")
    for i, L in enumerate(lens):
        ref = _sdpa(back(q[i]), back(Kc[i]), back(Vc[i]), 0.25)
        np.testing.assert_allclose(out[i], ref, rtol=1e-12, atol=1e-12)


def test_block_permutation_invariance():
    q, Kc, Vc, kp, vp, tab = _case(21, [70, 3, 48, 16], 8, 4, 16, 16, pool_extra=20)
    lens = np.array([70, 3, 48, 16])
    kw = dict(bs=16, softmax_scale=0.25, q_dtype="f32", cache_dtype="f32")
    base = oracle.paged_decode_attn(q, kp, vp, tab, lens, **kw)
    P = kp.shape[0]
    for seed in range(3):
        pi = np.random.default_rng(seed).permutation(P)
        kp2 = np.empty_like(kp)
        vp2 = np.empty_like(vp)
        kp2[pi] = kp
        vp2[pi] = vp
        tab2 = np.where(tab >= 0, pi[np.maximum(tab, 0)], -1)
        out = oracle.paged_decode_attn(q, kp2, vp2, tab2, lens, **kw)
        assert np.array_equal(out, base)


def test_shared_prefix_equals_private_copies():
    # 3 sequences share a 2-block prefix (refcount 3) and hold private tails.
    rng = np.random.default_rng(5)
    bs, Hkv, d, Hq = 8, 2, 16, 4
    prefix_k = rng.standard_normal((16, Hkv, d)).astype(np.float32)
    prefix_v = rng.standard_normal((16, Hkv, d)).astype(np.float32)
    tails = [5, 8, 13]
    Kc = [np.concatenate([prefix_k, rng.standard_normal((t, Hkv, d)).astype(np.float32)]) for t in tails]
    Vc = [np.concatenate([prefix_v, rng.standard_normal((t, Hkv, d)).astype(np.float32)]) for t in tails]
    q = rng.standard_normal((3, Hq, d)).astype(np.float32)
    lens = np.array([16 + t for t in tails])
    kw = dict(bs=bs, softmax_scale=0.3, q_dtype="f32", cache_dtype="f32")
    # private copies
    kp, vp, tab = _scatter(Kc, Vc, bs, 20, rng)
    private = oracle.paged_decode_attn(q, kp, vp, tab, lens, **kw)
    # shared: sequences 1 and 2 point at sequence 0's prefix blocks
    tab_sh = tab.copy()
    tab_sh[1, :2] = tab[0, :2]
    tab_sh[2, :2] = tab[0, :2]
    kp_sh, vp_sh = kp.copy(), vp.copy()
    for i in (1, 2):
        for b in tab[i, :2]:
            kp_sh[b] = np.nan          # the private prefix copies are now unused
            vp_sh[b] = np.nan
    shared = oracle.paged_decode_attn(q, kp_sh, vp_sh, tab_sh, lens, **kw)
    assert np.array_equal(private, shared)


def test_closed_forms():
    rng = np.random.default_rng(9)
    Hq, Hkv, d, bs = 4, 2, 8, 4
    q = rng.standard_normal((1, Hq, d)).astype(np.float32)
    kw = dict(bs=bs, softmax_scale=0.5, q_dtype="f32", cache_dtype="f32")
    # one token: out = v0 exactly
    K1 = [rng.standard_normal((1, Hkv, d)).astype(np.float32)]
    V1 = [rng.standard_normal((1, Hkv, d)).astype(np.float32)]
    kp, vp, tab = _scatter(K1, V1, bs, 3, rng)
    out = oracle.paged_decode_attn(q, kp, vp, tab, np.array([1]), **kw)
    for h in range(Hq):
        assert np.array_equal(out[0, h], V1[0][0, h // 2].astype(np.float64))
    # constant V: out = that constant
    L = 13
    Kc = [rng.standard_normal((L, Hkv, d)).astype(np.float32)]
    c = rng.standard_normal((Hkv, d)).astype(np.float32)
    Vc = [np.broadcast_to(c, (L, Hkv, d)).copy()]
    kp, vp, tab = _scatter(Kc, Vc, bs, 6, rng)
    out = oracle.paged_decode_attn(q, kp, vp, tab, np.array([L]), **kw)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], c[h // 2], rtol=1e-15, atol=1e-15)
    # equal keys, or a zero query: the mean of V
    Kc = [np.broadcast_to(rng.standard_normal((1, Hkv, d)).astype(np.float32), (L, Hkv, d)).copy()]
    Vc = [rng.standard_normal((L, Hkv, d)).astype(np.float32)]
    kp, vp, tab = _scatter(Kc, Vc, bs, 6, rng)
    mean = Vc[0].astype(np.float64).mean(axis=0)
    for qq in (q, np.zeros_like(q)):
        out = oracle.paged_decode_attn(qq, kp, vp, tab, np.array([L]), **kw)
        for h in range(Hq):
            np.testing.assert_allclose(out[0, h], mean[h // 2], rtol=1e-14, atol=1e-14)
    # empty sequence: zero row, tables never read
    out = oracle.paged_decode_attn(q, kp, vp, np.full((1, 4), -1, np.int32), np.array([0]), **kw)
    assert np.array_equal(out, np.zeros_like(out))


@pytest.mark.parametrize("L,part", [(1, 16), (100, 16), (513, 512), (1500, 512), (2048, 256)])
def test_splitk_merge_equals_single_pass(L, part):
    rng = np.random.default_rng(L)
    Hq, Hkv, d = 8, 2, 16
    K = rng.standard_normal((L, Hkv, d)) * 3
    V = rng.standard_normal((L, Hkv, d))
    q = rng.standard_normal((Hq, d))
    a = oracle.contiguous_decode_attn(q, K, V, 0.25)
    b = oracle.partition_then_merge(q, K, V, 0.25, part)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- planted mistakes
def _pins_pass():
    """True when the brute-force and invariance pins all hold for the oracle."""
    try:
        test_against_sdpa(*CASES[1])
        test_against_sdpa(*CASES[3])
        test_closed_forms()
        test_bf16_storage_widens_exactly()
    except AssertionError:
        return False
    return True


def test_pins_hold_for_the_oracle():
    assert _pins_pass()


def test_planted_gqa_mapping_mistake_is_caught(monkeypatch):
    orig = oatt.contiguous_decode_attn

    def wrong(q_i, K, V, sigma):    # kv head h % Hkv instead of h // G
        Hq, d = q_i.shape
        Hkv = K.shape[1]
        G = Hq // Hkv
        perm = np.array([(h % Hkv) * G + h // Hkv for h in range(Hq)])
        return orig(q_i[perm], K, V, sigma)[np.argsort(perm)]
    monkeypatch.setattr(oatt, "contiguous_decode_attn", wrong)
    assert not _pins_pass()


def test_planted_v_layout_mistake_is_caught(monkeypatch):
    orig = oatt.reassemble

    def wrong(pool, table_row, L, bs, which):   # read V as if it were token-major
        if which == "v":
            P, H, d, b = pool.shape
            pool = pool.reshape(P, H, b, d)
            return orig(pool, table_row, L, bs, "k")
        return orig(pool, table_row, L, bs, which)
    monkeypatch.setattr(oatt, "reassemble", wrong)
    assert not _pins_pass()


def test_planted_position_offset_mistake_is_caught(monkeypatch):
    orig = oatt.reassemble

    def wrong(pool, table_row, L, bs, which):   # drop the first token, duplicate the last
        x = orig(pool, table_row, L, bs, which)
        return np.concatenate([x[1:], x[-1:]]) if L > 1 else x
    monkeypatch.setattr(oatt, "reassemble", wrong)
    assert not _pins_pass()


def test_planted_missing_scale_is_caught(monkeypatch):
    orig = oatt.contiguous_decode_attn
    monkeypatch.setattr(oatt, "contiguous_decode_attn", lambda q, K, V, s: orig(q, K, V, 1.0))
    assert not _pins_pass()


def test_planted_bf16_truncation_mistake_is_caught(monkeypatch):
    from oracle import codecs

    def wrong(bits):                # read bf16 as if it were the low half of a float32
        b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return b.view(np.float32).astype(np.float64)
    monkeypatch.setattr(oatt, "bf16_bits_to_f64", wrong)
    assert not _pins_pass()
    assert codecs.bf16_bits_to_f64 is not wrong


# ------------------------------------------------------------------ query windows
def _sdpa_window(q_w, K, V, sigma):
    """All n_q queries of a window at once through torch SDPA with an explicit
    boolean mask: query j (position L - n_q + j) may see token t iff t <= that
    position. float64; kv head h // G serves q head h."""
    n_q, Hq, d = q_w.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    q = torch.from_numpy(q_w).permute(1, 0, 2).unsqueeze(0).contiguous()          # [1][Hq][n_q][d]
    k = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
    v = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
    pos = torch.arange(L - n_q, L).unsqueeze(1)                                   # [n_q][1]
    mask = torch.arange(L).unsqueeze(0) <= pos                                    # [n_q][L]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=float(sigma))
    return o[0].permute(1, 0, 2).numpy()                                          # [n_q][Hq][d]


WINDOWS = [
    (21, [5, 17, 33], 4, 4, 8, 4, 3),
    (22, [16, 40, 9], 8, 2, 16, 8, 5),
    (23, [64, 30], 6, 3, 8, 16, 1),
    (24, [20, 20], 16, 2, 32, 16, 20),        # the window is the whole sequence
]


@pytest.mark.parametrize("seed,lens,Hq,Hkv,d,bs,n_q", WINDOWS)
def test_multi_query_against_masked_sdpa(seed, lens, Hq, Hkv, d, bs, n_q):
    rng = np.random.default_rng(seed)
    _, Kc, Vc, kp, vp, tab = _case(seed, lens, Hq, Hkv, d, bs)
    q = rng.standard_normal((len(lens), n_q, Hq, d)).astype(np.float32)
    sigma = np.float32(1 / math.sqrt(d))
    out = oracle.paged_multi_query_attn(q, kp, vp, tab, np.array(lens), bs=bs, softmax_scale=sigma,
                                        q_dtype="f32", cache_dtype="f32")
    for i in range(len(lens)):
        ref = _sdpa_window(q[i].astype(np.float64), Kc[i].astype(np.float64), Vc[i].astype(np.float64),
                           np.float64(sigma))
        np.testing.assert_allclose(out[i], ref, rtol=1e-12, atol=1e-12)


def test_multi_query_last_query_is_decode_and_empty_rows():
    _, Kc, Vc, kp, vp, tab = _case(25, [30, 0, 12], 4, 2, 8, 4)
    q = np.random.default_rng(26).standard_normal((3, 4, 4, 8)).astype(np.float32)
    lens = np.array([30, 0, 12])
    mq = oracle.paged_multi_query_attn(q, kp, vp, tab, lens, bs=4, softmax_scale=0.3,
                                       q_dtype="f32", cache_dtype="f32")
    dec = oracle.paged_decode_attn(q[:, -1], kp, vp, tab, lens, bs=4, softmax_scale=0.3,
                                   q_dtype="f32", cache_dtype="f32")
    assert np.array_equal(mq[:, -1], dec)
    assert np.all(mq[1] == 0.0)


def test_planted_causal_offset_mistake_is_caught(monkeypatch):
    # a window whose queries saw one token too many would disagree with SDPA
    real = oatt.paged_decode_attn

    def shifted(q, kc, vc, tab, lens, **kw):
        return real(q, kc, vc, tab, np.where(np.asarray(lens) > 0, np.asarray(lens) + 1, 0), **kw)

    seed, lens, Hq, Hkv, d, bs, n_q = WINDOWS[0]
    rng = np.random.default_rng(seed)
    _, Kc, Vc, kp, vp, tab = _case(seed, lens, Hq, Hkv, d, bs)
    q = rng.standard_normal((len(lens), n_q, Hq, d)).astype(np.float32)
    monkeypatch.setattr(oatt, "paged_decode_attn", shifted)
    out = oatt.paged_multi_query_attn(q, kp, vp, tab, np.array(lens), bs=bs, softmax_scale=0.35,
                                      q_dtype="f32", cache_dtype="f32")
    ref = _sdpa_window(q[0].astype(np.float64), Kc[0].astype(np.float64), Vc[0].astype(np.float64),
                       np.float64(np.float32(0.35)))
    assert not np.allclose(out[0], ref, rtol=1e-6, atol=1e-6)


# ------------------------------------------------ log-sum-exp states and their merge (shared prefixes)
def _lse_loops(q_i, K, sigma):
    """Pure-Python log2 sum_t exp(s_t) per head."""
    Hq, d = q_i.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    out = []
    for h in range(Hq):
        s = [sigma * sum(float(q_i[h, c]) * float(K[t, h // G, c]) for c in range(d)) for t in range(L)]
        out.append(math.log2(sum(math.exp(x) for x in s)) if s else -math.inf)
    return np.array(out)


def _lse_closed_forms_hold():
    rng = np.random.default_rng(41)
    ok = True
    for L in (1, 2, 7, 100):
        K = rng.standard_normal((L, 2, 8))
        # q = 0: every score is 0, the sum of exponentials is L
        ok &= bool(np.allclose(oatt.contiguous_decode_lse(np.zeros((4, 8)), K, 0.5), math.log2(L),
                               rtol=0, atol=1e-13))
    # one token: the sum is exp(s_0), so lse = s_0 / ln 2
    q = rng.standard_normal((4, 8))
    K = rng.standard_normal((1, 2, 8))
    want = [0.3 * float(q[h] @ K[0, h // 2]) / math.log(2) for h in range(4)]
    ok &= bool(np.allclose(oatt.contiguous_decode_lse(q, K, 0.3), want, rtol=0, atol=1e-13))
    ok &= bool(np.all(oatt.contiguous_decode_lse(q, K[:0], 0.3) == -np.inf))
    return ok


def test_lse_closed_forms():
    assert _lse_closed_forms_hold()


@pytest.mark.parametrize("seed,lens,Hq,Hkv,d,bs", CASES)
def test_lse_against_loops(seed, lens, Hq, Hkv, d, bs):
    q, Kc, _, kp, _, tab = _case(seed, lens, Hq, Hkv, d, bs)
    sigma = np.float32(1 / math.sqrt(d))
    got = oracle.paged_decode_lse(q, kp, tab, np.array(lens), bs=bs, softmax_scale=sigma,
                                  q_dtype="f32", cache_dtype="f32")
    for i, L in enumerate(lens):
        want = _lse_loops(q[i].astype(np.float64), Kc[i].astype(np.float64), float(sigma))
        np.testing.assert_allclose(got[i], want, rtol=1e-12, atol=1e-12)


def _split_error(seed=51, lens=(40, 17, 64, 8), Hq=6, Hkv=2, d=16, bs=8, cut_blocks=(2, 1, 5, 1)):
    """Largest difference between the whole-sequence oracle attention and the
    merge of its states over the first cut_blocks[i] blocks and over the rest,
    both found through block tables (the rest through a table that starts at
    the cut). Returns (output error, lse error)."""
    q, _, _, kp, vp, tab = _case(seed, list(lens), Hq, Hkv, d, bs)
    lens = np.array(lens)
    kw = dict(bs=bs, softmax_scale=0.31, q_dtype="f32", cache_dtype="f32")
    cut = np.minimum(np.array(cut_blocks) * bs, lens)
    pre_tab = tab.copy()
    suf_tab = np.full_like(tab, -1)
    for i in range(len(lens)):
        nb = -(-int(lens[i]) // bs)
        k = int(cut[i]) // bs
        suf_tab[i, :nb - k] = tab[i, k:nb]
    o_a = oracle.paged_decode_attn(q, kp, vp, pre_tab, cut, **kw)
    o_b = oracle.paged_decode_attn(q, kp, vp, suf_tab, lens - cut, **kw)
    la = oracle.paged_decode_lse(q, kp, pre_tab, cut, **kw)
    lb = oracle.paged_decode_lse(q, kp, suf_tab, lens - cut, **kw)
    o, lse = oracle.merge_attn_states(o_a, la, o_b, lb)
    whole = oracle.paged_decode_attn(q, kp, vp, tab, lens, **kw)
    lse_whole = oracle.paged_decode_lse(q, kp, tab, lens, **kw)
    return float(np.max(np.abs(o - whole))), float(np.max(np.abs(lse - lse_whole)))


def test_merge_of_prefix_and_suffix_states_is_the_whole_attention():
    # cuts inside, at the end of (nothing after) and past nothing (all after)
    eo, el = _split_error()
    assert eo < 1e-12 and el < 1e-12
    eo, el = _split_error(cut_blocks=(0, 3, 8, 1))
    assert eo < 1e-12 and el < 1e-12


def test_merge_attn_states_empty_sides():
    o_a = np.arange(6.0).reshape(3, 2)
    o_b = -np.arange(6.0).reshape(3, 2)
    la = np.array([1.5, -np.inf, -np.inf])
    lb = np.array([-np.inf, 0.25, -np.inf])
    o, lse = oracle.merge_attn_states(o_a, la, o_b, lb)
    assert np.array_equal(o[0], o_a[0]) and lse[0] == 1.5
    assert np.array_equal(o[1], o_b[1]) and lse[1] == 0.25
    assert np.all(o[2] == 0) and lse[2] == -np.inf
    # equal weights: the mean, and lse grows by exactly one (a doubled sum)
    o, lse = oracle.merge_attn_states(o_a[:1], np.array([3.0]), o_b[:1], np.array([3.0]))
    assert np.array_equal(o[0], (o_a[0] + o_b[0]) / 2) and lse[0] == 4.0


def test_planted_natural_log_lse_is_caught(monkeypatch):
    real = oatt.contiguous_decode_lse
    monkeypatch.setattr(oatt, "contiguous_decode_lse", lambda q, K, s: real(q, K, s) * math.log(2))
    assert not _lse_closed_forms_hold()


def test_planted_swapped_merge_weights_are_caught(monkeypatch):
    real = oatt.merge_attn_states
    monkeypatch.setattr(oracle, "merge_attn_states", lambda a, la, b, lb: real(a, lb, b, la))
    eo, _ = _split_error()
    assert eo > 1e-6
