"""The decode step that allocates nothing (pkv_paged_decode_step_noalloc),
called through the C ABI, against pkv_paged_decode_step on the same inputs.

Both run the same kernels on the same values, so outputs must be identical
bit for bit (and within the oracle's tolerance), and the pools after the two
steps identical byte for byte. Two calls in a row, the second on a smaller
input, so the second call runs on the scratch array as the first left it. A
call that needs more than the scratch array holds is refused before any
launch.
"""

import ctypes

import numpy as np
import pytest

import oracle
import paged_kv_cache_108_amd as pkv
from paged_kv_cache_108_amd import workloads as W
from helpers import (TOL, DeviceStep, assert_rows_close, device_decode_step, need_gpu, oracle_pools,
                     same_bits, to_host)

pytestmark = pytest.mark.gpu


def _noalloc_step(dev, out):
    """One pkv_paged_decode_step_noalloc call through ctypes."""
    torch = need_gpu()
    w = dev.w
    s = w.spec
    lib = pkv.lib()
    code = {torch.float32: pkv.PKV_F32, torch.bfloat16: pkv.PKV_BF16, torch.uint8: pkv.PKV_FP8_E4M3}
    st = lib.pkv_paged_decode_step_noalloc(
        out.data_ptr(), dev.q.data_ptr(), dev.k_new.data_ptr(), dev.v_new.data_ptr(), dev.k_cache.data_ptr(),
        dev.v_cache.data_ptr(), dev.tables.data_ptr(), dev.lens.data_ptr(), s.S, s.Hq, s.Hkv, s.d, s.bs, w.P,
        w.max_blocks, w.max_context_len, ctypes.c_float(w.softmax_scale), ctypes.c_float(w.k_scale),
        ctypes.c_float(w.v_scale), ctypes.c_float(w.k_inv_scale), ctypes.c_float(w.v_inv_scale),
        code[dev.q.dtype], code[dev.k_cache.dtype], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return st


def _compare(w, seqs=None):
    torch = need_gpu()
    s = w.spec
    print(f"[case] noalloc step {s.name} S={s.S} cache={s.cache_dtype}", flush=True)
    ref_dev = DeviceStep(w)
    want = to_host(device_decode_step(ref_dev)).copy()
    dev = DeviceStep(w)
    out = torch.full((s.S, s.Hq, s.d), float("nan"), dtype=torch.float32, device="cuda")
    assert _noalloc_step(dev, out) == 0, pkv.last_error()
    got = to_host(out)
    assert np.array_equal(got, want), "no-alloc step differs from pkv_paged_decode_step"
    assert same_bits(to_host(dev.k_cache), to_host(ref_dev.k_cache))
    assert same_bits(to_host(dev.v_cache), to_host(ref_dev.v_cache))
    kc, vc = oracle_pools(w, seqs)
    ref = oracle.paged_decode_attn(w.q, kc, vc, w.block_tables, w.context_lens, bs=s.bs,
                                   softmax_scale=w.softmax_scale, q_dtype=s.q_dtype, cache_dtype=s.cache_dtype,
                                   k_scale=w.k_scale, v_scale=w.v_scale, seqs=seqs)
    assert_rows_close(got if seqs is None else got[seqs], ref, TOL[s.cache_dtype], "no-alloc step")


def test_noalloc_step_twice_second_smaller():
    need_gpu()
    _compare(W.make("llama8b"), seqs=[0, 9, 31, 63])
    _compare(W.make("small"), seqs=list(range(0, 256, 15)))


def test_noalloc_step_fp8_then_tiny():
    need_gpu()
    _compare(W.make_custom(lens=[1, 17, 700, 3000, 0], Hq=16, Hkv=2, d=128, bs=16, cache_dtype="fp8",
                           cfg=1600))
    _compare(W.make("tiny"))


def test_noalloc_step_refuses_a_call_beyond_the_scratch():
    # 16 query heads per kv head at d 128: 2 x 1024 waves x 16 x 130 x 4 bytes
    # of records, above the 16 MiB array on a 256-CU part
    torch = need_gpu()
    assert pkv.lib().pkv_paged_decode_step_scratch_bytes() == 16 << 20
    n_waves = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    need = 2 * n_waves * 16 * 130 * 4
    w = W.make_custom(lens=[5, 40], Hq=16, Hkv=1, d=128, bs=16, cfg=1601)
    dev = DeviceStep(w)
    out = torch.zeros((2, 16, 128), dtype=torch.float32, device="cuda")
    before = to_host(dev.k_cache).copy()
    st = _noalloc_step(dev, out)
    if need + 8 > 16 << 20:
        assert st == 2, "expected PKV_E_WORKSPACE"            # PKV_E_WORKSPACE, nothing launched
        assert "workspace" in pkv.last_error()
        assert np.all(to_host(out) == 0) and same_bits(to_host(dev.k_cache), before)
    else:
        assert st == 0
