"""GPU parity of the fp8 (OCP E4M3) cache paths against the fp64 oracle.

* Edge shapes at every V sub-tile arrangement: bs 8 (element loads), 16 (one
  sub-tile), 32 and 128 (several sub-tiles per block), with G 1 and 4 and
  lengths ending inside a chunk, for the write + attention and for the fused
  step (which patches the new token into whichever row it lands in).
* K and V with scales two orders of magnitude apart: a swapped or shared scale
  in the kernels would fail the 2e-2 row tolerance.
* The write's encoder on every bf16 bit pattern, at inverse scale 1 (which
  holds every E4M3 midpoint exactly), at 1 + 2^-23 and 1 - 2^-24 (whose float32
  products are the midpoints' float32 neighbours) and at the scales of the
  seeded workloads: byte-exact against the oracle's quantisation, through the
  separate write and through the fused step.
* A fused step whose table lists no block (-1) for a new token's position
  leaves every block of both pools unchanged there, as the separate write does.
"""

import numpy as np
import pytest

import oracle
import paged_kv_cache_108_amd as pkv
from paged_kv_cache_108_amd import workloads as W
from helpers import (TOL, DeviceStep, assert_rows_close, device_decode_step, need_gpu, oracle_pools,
                     same_bits, to_dev, to_host)

pytestmark = pytest.mark.gpu
BAL = pkv.PKV_PARTITION_BALANCED


@pytest.fixture(autouse=True)
def _gpu_present():
    need_gpu()


def _listed_blocks(w, seqs=None):
    rows = range(w.spec.S) if seqs is None else seqs
    b = np.unique(w.block_tables[list(rows)].reshape(-1))
    return b[b >= 0]


def _fp8_case(w, partitions, step=False):
    """Write (or fused step) + attention on an fp8 cache; pools byte-exact on
    every listed block, rows within the fp8 tolerance."""
    s = w.spec
    print(f"[case] fp8 {s.name} lens={list(w.context_lens)[:8]} G={s.Hq // s.Hkv} d={s.d} bs={s.bs} "
          f"step={step} scales=({w.k_scale:.4g}, {w.v_scale:.4g})", flush=True)
    kc, vc = oracle_pools(w)
    ref = oracle.paged_decode_attn(w.q, kc, vc, w.block_tables, w.context_lens, bs=s.bs,
                                   softmax_scale=w.softmax_scale, q_dtype=s.q_dtype, cache_dtype="fp8",
                                   k_scale=w.k_scale, v_scale=w.v_scale)
    blocks = _listed_blocks(w)
    dev = DeviceStep(w)
    outs = []
    if step:
        outs.append(("step", to_host(device_decode_step(dev)).copy()))
    else:
        dev.write()
    assert np.array_equal(to_host(dev.k_cache)[blocks], kc[blocks]), "K pool differs"
    assert np.array_equal(to_host(dev.v_cache)[blocks], vc[blocks]), "V pool differs"
    for part in partitions:
        outs.append((part, to_host(dev.attend(part)).copy()))
    e = 0.0
    for name, got in outs:
        e = max(e, assert_rows_close(got, ref, TOL["fp8"], f"fp8 {name}"))
    if step:                                   # the fused step equals write + balanced attention
        assert np.array_equal(outs[0][1], dict(outs)[BAL])
    for i, L in enumerate(w.context_lens):
        if L <= 0:
            assert all(np.all(o[i] == 0.0) for _, o in outs)
    print(f"[case] max row err {e:.3e}", flush=True)


FP8_EDGE = [
    # lens, Hq, Hkv, d, bs
    ([1, 17, 33, 65, 700, 0], 4, 4, 128, 8),
    ([1, 2, 17, 33, 65, 700], 16, 4, 128, 8),
    ([1, 15, 16, 17, 33, 65, 700], 8, 2, 64, 16),
    ([1, 17, 33, 65, 700, 0], 4, 4, 64, 32),
    ([1, 31, 32, 33, 65, 700], 16, 4, 128, 32),
    ([1, 17, 33, 65, 127, 128, 129, 700], 4, 1, 128, 128),
    ([1, 17, 33, 65, 700], 16, 4, 64, 128),
]


@pytest.mark.parametrize("lens,Hq,Hkv,d,bs", FP8_EDGE)
def test_fp8_edge_shapes(lens, Hq, Hkv, d, bs):
    w = W.make_custom(lens=lens, Hq=Hq, Hkv=Hkv, d=d, bs=bs, cache_dtype="fp8", cfg=1100 + bs + Hq + d)
    _fp8_case(w, [0, 512, 32, BAL])


@pytest.mark.parametrize("lens,Hq,Hkv,d,bs", FP8_EDGE)
def test_fp8_decode_step_edge_shapes(lens, Hq, Hkv, d, bs):
    w = W.make_custom(lens=lens, Hq=Hq, Hkv=Hkv, d=d, bs=bs, cache_dtype="fp8", cfg=1200 + bs + Hq + d)
    _fp8_case(w, [BAL], step=True)


@pytest.mark.parametrize("bs,G", [(16, 4), (8, 1), (32, 8)])
def test_fp8_distinct_k_and_v_scales(bs, G):
    # K values 0.05 x N(0,1), V values 20 x N(0,1): k_scale and v_scale differ
    # by a factor of 400
    lens = [1, 9, 40, 300, 1100]
    w = W.make_custom(lens=lens, Hq=2 * G, Hkv=2, d=128, bs=bs, cache_dtype="fp8", cfg=1300 + bs + G,
                      value_scales=(0.05, 20.0))
    assert w.v_scale / w.k_scale > 100
    _fp8_case(w, [0, 512, BAL])
    _fp8_case(w, [BAL], step=True)


# ------------------------------------------------------------------ the encoder on every bf16 pattern
def _inverse_scales():
    small = W.make("small", cache_dtype="fp8")
    scales = [1.0, float(np.float32(1 + 2.0 ** -23)), float(np.float32(1 - 2.0 ** -24)),
              small.k_inv_scale, small.v_inv_scale, float(np.float32(448.0 / 5.25)),
              float(np.float32(2.0 ** -7)), float(np.float32(1e4))]
    return scales


def _all_bf16_patterns(T, Hkv, d, seed):
    bits = np.arange(1 << 16, dtype=np.uint16)
    bits = bits[np.random.default_rng(seed).permutation(len(bits))]
    return bits.reshape(T, Hkv, d)


def test_fp8_write_every_bf16_pattern():
    torch = need_gpu()
    T, Hkv, d, bs = 64, 8, 128, 16
    P = T // bs
    kn, vn = _all_bf16_patterns(T, Hkv, d, 1), _all_bf16_patterns(T, Hkv, d, 2)
    slots = np.arange(T, dtype=np.int64)[np.random.default_rng(3).permutation(T)]
    gkn, gvn, gslots = to_dev(kn), to_dev(vn), to_dev(slots)
    kc = torch.zeros((P, Hkv, bs, d), dtype=torch.uint8, device="cuda")
    vc = torch.zeros((P, Hkv, d, bs), dtype=torch.uint8, device="cuda")
    zk = np.zeros((P, Hkv, bs, d), np.uint8)
    zv = np.zeros((P, Hkv, d, bs), np.uint8)
    for inv_k in _inverse_scales():
        inv_v = float(np.float32(inv_k * 1.5))
        print(f"[case] every bf16 pattern, write, inv ({inv_k!r}, {inv_v!r})", flush=True)
        pkv.kv_cache_write(gkn, gvn, kc, vc, gslots, k_inv_scale=inv_k, v_inv_scale=inv_v)
        torch.cuda.synchronize()
        ok_, ov = oracle.kv_cache_write(kn, vn, zk, zv, slots, bs=bs, src_dtype="bf16", cache_dtype="fp8",
                                        k_inv_scale=inv_k, v_inv_scale=inv_v)
        assert np.array_equal(to_host(kc), ok_), f"K codes differ at inverse scale {inv_k!r}"
        assert np.array_equal(to_host(vc), ov), f"V codes differ at inverse scale {inv_v!r}"


@pytest.mark.parametrize("planned", [False, True])
def test_fp8_fused_step_write_every_bf16_pattern(planned):
    # 64 sequences x 8 kv heads x 128 channels: one step writes every bf16
    # pattern once into K and once into V (the unplanned step's stream kernel
    # and the planned kernel each carry their own copy of the write)
    torch = need_gpu()
    S, Hkv, d, bs = 64, 8, 128, 16
    lens = [1 + 37 * i % 300 for i in range(S)]
    w = W.make_custom(lens=lens, Hq=Hkv * 4, Hkv=Hkv, d=d, bs=bs, cache_dtype="fp8", cfg=1400)
    w.k_new[:] = _all_bf16_patterns(S, Hkv, d, 4)
    w.v_new[:] = _all_bf16_patterns(S, Hkv, d, 5)
    dev = DeviceStep(w)
    slots = oracle.decode_slots(w.block_tables, w.context_lens, bs)
    ws = pkv.paged_decode_attn_workspace(S, w.spec.Hq, Hkv, d, w.max_context_len, BAL)
    plan = pkv.DecodePlan(w.context_lens, Hq=w.spec.Hq, Hkv=Hkv, d=d, bs=bs, cache_dtype_code=pkv.PKV_FP8_E4M3,
                          max_context_len=w.max_context_len) if planned else None
    for inv_k in _inverse_scales():
        inv_v = float(np.float32(inv_k * 0.75))
        print(f"[case] every bf16 pattern, {'planned' if planned else 'fused'} step, inv ({inv_k!r}, {inv_v!r})",
              flush=True)
        if planned:
            plan(dev.out, dev.q, dev.k_cache, dev.v_cache, dev.tables, dev.lens, softmax_scale=w.softmax_scale,
                 k_new=dev.k_new, v_new=dev.v_new, k_inv_scale=inv_k, v_inv_scale=inv_v)
        else:
            pkv.paged_decode_step(dev.out, dev.q, dev.k_new, dev.v_new, dev.k_cache, dev.v_cache, dev.tables,
                                  dev.lens, max_context_len=w.max_context_len, softmax_scale=w.softmax_scale,
                                  k_scale=1.0, v_scale=1.0, k_inv_scale=inv_k, v_inv_scale=inv_v, workspace=ws)
        torch.cuda.synchronize()
        gk, gv = to_host(dev.k_cache), to_host(dev.v_cache)
        want_k = oracle.quantise(w.k_new, "bf16", inv_k)
        want_v = oracle.quantise(w.v_new, "bf16", inv_v)
        for i, slot in enumerate(slots):
            b, o = divmod(int(slot), bs)
            assert np.array_equal(gk[b, :, o, :], want_k[i]), f"K codes of token {i} at inverse scale {inv_k!r}"
            assert np.array_equal(gv[b, :, :, o], want_v[i]), f"V codes of token {i} at inverse scale {inv_v!r}"


# ------------------------------------------------------------------ a table entry outside the pool
@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_decode_step_skips_a_new_token_without_a_block(dt):
    # sequence 0's new token (position 32) would open its third block, but the
    # table lists -1 there: the fused step must not store it anywhere. Every
    # other sequence's token is written as usual; every other byte is unchanged.
    need_gpu()
    lens = [33, 17, 1, 64, 200]
    w = W.make_custom(lens=lens, Hq=8, Hkv=2, d=128, bs=16, cache_dtype=dt, cfg=1500)
    dev = DeviceStep(w)
    w.block_tables[0, 2] = -1
    dev.tables = to_dev(w.block_tables)
    before_k, before_v = to_host(dev.k_cache).copy(), to_host(dev.v_cache).copy()
    print(f"[case] decode step with a -1 entry, {dt}", flush=True)
    device_decode_step(dev)
    slots = np.array([-1] + list(oracle.decode_slots(w.block_tables[1:], w.context_lens[1:], 16)))
    want_k, want_v = oracle.kv_cache_write(
        w.k_new, w.v_new, before_k, before_v, slots, bs=16, src_dtype="bf16",
        cache_dtype=dt, k_inv_scale=w.k_inv_scale, v_inv_scale=w.v_inv_scale)
    assert same_bits(to_host(dev.k_cache), want_k), "K pool: a byte outside the written slots changed"
    assert same_bits(to_host(dev.v_cache), want_v), "V pool: a byte outside the written slots changed"
