"""GPU parity of planned query windows (pkv_paged_multi_query_attn_planned).

A window plan cuts each kv head's (query, head) columns into groups of one
16-column tile (a window of n_q * G <= 16 columns) or two (a wider one) and
makes each group a segment of the balanced split, as the unplanned window call
groups them per pass. Where both run the same number of waves the split is the
same one and the planned outputs must equal the unplanned call's bit for bit;
otherwise they agree within the tolerance. Every case is checked against the
fp64 oracle's windowed attention. A decode plan, or a window plan for another
window, is refused.
"""

import numpy as np
import pytest

import oracle
import paged_kv_cache_108_amd as pkv
from paged_kv_cache_108_amd import workloads as W
from helpers import TOL, DeviceStep, assert_rows_close, need_gpu, oracle_pools, to_dev, to_host

pytestmark = pytest.mark.gpu
CODE = {"f32": 0, "bf16": 1, "fp8": 2}


@pytest.fixture(autouse=True)
def _gpu_present():
    need_gpu()


def _window_q(w, n_q):
    s = w.spec
    rng = np.random.default_rng([108, 955, n_q, s.S])
    qf = rng.standard_normal((s.S, n_q, s.Hq, s.d)).astype(np.float32)
    return qf if s.q_dtype == "f32" else W.to_bf16_bits(qf)


def _plan(w, n_q):
    s = w.spec
    return pkv.WindowPlan(w.context_lens, n_q=n_q, Hq=s.Hq, Hkv=s.Hkv, d=s.d, bs=s.bs,
                          cache_dtype_code=CODE[s.cache_dtype], max_context_len=w.max_context_len)


def _case(w, n_q):
    torch = need_gpu()
    s = w.spec
    G = s.Hq // s.Hkv
    print(f"[case] planned window {s.name} n_q={n_q} G={G} bs={s.bs} cache={s.cache_dtype} S={s.S}", flush=True)
    dev = DeviceStep(w)
    dev.write()                               # the window's last token: attention reads up to L - 1
    q = _window_q(w, n_q)
    qd = to_dev(q)
    want = torch.full((s.S, n_q, s.Hq, s.d), float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_multi_query_attn(want, qd, dev.k_cache, dev.v_cache, dev.tables, dev.lens,
                               max_context_len=w.max_context_len, softmax_scale=w.softmax_scale,
                               k_scale=w.k_scale, v_scale=w.v_scale)
    plan = _plan(w, n_q)
    got = torch.full_like(want, float("nan"))
    plan(got, qd, dev.k_cache, dev.v_cache, dev.tables, dev.lens, softmax_scale=w.softmax_scale,
         k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    got_h, want_h = to_host(got).copy(), to_host(want).copy()
    same_split = plan.n_workers == 4 * torch.cuda.get_device_properties(0).multi_processor_count
    print(f"[case] {plan.n_workers} waves, {int(plan.host[14])} query groups of {int(plan.host[13])}; "
          f"same split as the unplanned call: {same_split}", flush=True)
    if same_split:
        assert np.array_equal(got_h, want_h), "planned window differs from the unplanned call"
    else:
        assert_rows_close(got_h, want_h.astype(np.float64), TOL[s.cache_dtype], "planned vs unplanned window")
    assert np.array_equal(to_host(plan.dev), plan.host), "the call changed its plan"
    kc, vc = oracle_pools(w)
    ref = oracle.paged_multi_query_attn(q, kc, vc, w.block_tables, w.context_lens, bs=s.bs,
                                        softmax_scale=w.softmax_scale, q_dtype=s.q_dtype,
                                        cache_dtype=s.cache_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    e = assert_rows_close(got_h, ref, TOL[s.cache_dtype], f"planned window {s.name} n_q={n_q}")
    print(f"[case] max row err {e:.3e}", flush=True)
    return got_h


# one tile per group: llama8b (G 4) up to 4 queries, small (G 7) 2, tiny (G 1)
# 4 (its shortest sequence holds 4 tokens; a window may not be longer)
@pytest.mark.parametrize("name,cache,n_q", [
    ("llama8b", None, 1), ("llama8b", None, 4), ("llama8b", "fp8", 4), ("small", None, 2), ("small", "fp8", 2),
    ("tiny", None, 4),
])
def test_planned_window_one_tile(name, cache, n_q):
    _case(W.make(name, cache_dtype=cache), n_q)


# two tiles per group (more than 16 columns), and several groups per kv head
# (one pass over the blocks for each)
@pytest.mark.parametrize("name,cache,n_q", [
    ("llama8b", None, 8), ("llama8b", None, 16), ("llama8b", None, 20), ("small", None, 5), ("small", None, 12),
    ("llama8b", "fp8", 8), ("small", "fp8", 5),
])
def test_planned_window_several_groups(name, cache, n_q):
    _case(W.make(name, cache_dtype=cache), n_q)


def test_planned_window_long_fp8():
    _case(W.make("long", cache_dtype="fp8"), 3)


@pytest.mark.parametrize("lens,Hq,Hkv,d,bs,dt,n_q", [
    ([16, 17, 40, 300, 0, 20], 4, 4, 64, 16, "f32", 16),      # G 1: the whole window in one group
    ([20, 21, 100, 600], 2, 2, 64, 8, "f32", 20),             # G 1, two groups
    ([4, 5, 17, 33, 1000, 0], 32, 8, 128, 16, "bf16", 4),     # L = n_q exactly
    ([9, 64, 65, 700], 14, 2, 64, 32, "bf16", 9),             # G 7: five groups of 2 queries
    ([3, 3, 50, 129], 16, 1, 128, 128, "fp8", 3),             # G 16: one query per group
    ([7, 300, 16, 0, 1], 8, 2, 64, 16, "fp8", 1),             # fp8 at d 64: two workgroups per CU
    ([7, 8, 90, 333, 0], 12, 4, 64, 16, "bf16", 7),           # G 3: 21 columns, a tile boundary inside a query
    ([6, 41, 500, 1200], 10, 2, 128, 32, "fp8", 6),           # G 5: 30 columns in two tiles
    ([12, 13, 64, 260], 4, 2, 128, 8, "f32", 12),             # G 2, bs 8: 24 columns
])
def test_planned_window_edge_shapes(lens, Hq, Hkv, d, bs, dt, n_q):
    w = W.make_custom(lens=lens, Hq=Hq, Hkv=Hkv, d=d, bs=bs, q_dtype="f32" if dt == "f32" else "bf16",
                      cache_dtype=dt, cfg=1960 + n_q + Hq)
    got = _case(w, n_q)
    for i, L in enumerate(lens):
        if L <= 0:
            assert np.all(got[i] == 0.0)


def test_planned_window_repeated_calls_give_the_same_bits():
    torch = need_gpu()
    w = W.make("llama8b")
    s = w.spec
    dev = DeviceStep(w)
    dev.write()
    qd = to_dev(_window_q(w, 8))
    plan = _plan(w, 8)
    first = None
    for _ in range(4):
        out = torch.full((s.S, 8, s.Hq, s.d), float("nan"), dtype=torch.float32, device="cuda")
        plan(out, qd, dev.k_cache, dev.v_cache, dev.tables, dev.lens, softmax_scale=w.softmax_scale)
        torch.cuda.synchronize()
        got = to_host(out).copy()
        if first is None:
            first = got
            assert not np.isnan(first).any()
        else:
            assert np.array_equal(got, first), "a later call differs"


def test_window_plan_of_another_kind_is_refused():
    torch = need_gpu()
    w = W.make_custom(lens=[5, 40, 300], Hq=8, Hkv=2, d=128, bs=16, cfg=1990)
    s = w.spec
    dev = DeviceStep(w)
    qd = to_dev(_window_q(w, 4))
    out = torch.zeros((s.S, 4, s.Hq, s.d), dtype=torch.float32, device="cuda")
    good = _plan(w, 4)
    dec = pkv.DecodePlan(w.context_lens, Hq=s.Hq, Hkv=s.Hkv, d=s.d, bs=s.bs, cache_dtype_code=1,
                         max_context_len=w.max_context_len)
    other = _plan(w, 3)
    for plan in (dec, other):
        with pytest.raises(pkv.PkvError):
            pkv.paged_multi_query_attn_planned(out, qd, dev.k_cache, dev.v_cache, dev.tables, dev.lens,
                                               max_context_len=w.max_context_len, softmax_scale=w.softmax_scale,
                                               plan_host=plan.host, plan_dev=plan.dev, workspace=good.workspace)
    # a window plan given to the decode step
    out1 = torch.zeros((s.S, s.Hq, s.d), dtype=torch.float32, device="cuda")
    with pytest.raises(pkv.PkvError):
        pkv.paged_decode_step_planned(out1, dev.q, None, None, dev.k_cache, dev.v_cache, dev.tables, dev.lens,
                                      max_context_len=w.max_context_len, softmax_scale=w.softmax_scale,
                                      plan_host=good.host, plan_dev=good.dev, workspace=dec.workspace)
    torch.cuda.synchronize()
    assert np.all(to_host(out) == 0) and np.all(to_host(out1) == 0)      # nothing ran
