"""Pins of where the oracle applies the fp8 scales.

An fp8 KV cache stores one E4M3 code per element and one float32 scale per
tensor, K and V each their own ("Serving: vLLM and PagedAttention", section
3.1, the ``kv_cache_dtype`` knob; the one-scale-per-tensor reading): a K
element's value is decode(code) * k_scale and a V element's decode(code) *
v_scale, and the write stores encode(float32(x) * inv_scale) with K's and V's
own inverse scales.

The references here decode the codes with PyTorch's ``float8_e4m3fn`` (a
library routine written independently of the oracle's table), multiply each
tensor by its own scale in float64, and attend with PyTorch's
``scaled_dot_product_attention`` / ``logsumexp`` over contiguous K/V that the
test scatters into the pools itself. The scales differ by orders of magnitude
(k_scale 0.01, v_scale 3.0), so a swapped pair or one shared scale moves every
output far outside the 1e-12 agreement. The planted mistakes at the end swap
them inside the oracle and confirm the pins catch it.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from oracle import cache_write as ocw

K_SCALE, V_SCALE = 0.01, 3.0


def _e4m3_torch(codes):
    """uint8 codes -> float64 values via torch's float8_e4m3fn."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).double().numpy()


def _finite_codes(rng, shape):
    """Random E4M3 codes without the two NaN codes."""
    c = rng.integers(0, 254, shape, dtype=np.int64)
    c = np.where(c >= 0x7F, c + 1, c)             # 0..0x7E and 0x80..0xFE
    return c.astype(np.uint8)


def _case(seed, lens, Hq, Hkv, d, bs):
    """Contiguous per-sequence codes scattered into fp8 pools in the library
    layout (K [P][Hkv][bs][d]; V [P][Hkv][bs/vs][d][vs], vs = min(bs, 16)),
    with random block ids; unused slots hold the NaN code."""
    rng = np.random.default_rng(seed)
    S = len(lens)
    nb = [-(-L // bs) for L in lens]
    P = sum(nb) + 5
    vs = min(bs, 16)
    kpool = np.full((P, Hkv, bs, d), 0x7F, dtype=np.uint8)
    vpool = np.full((P, Hkv, bs // vs, d, vs), 0x7F, dtype=np.uint8)
    tables = np.full((S, max(max(nb), 1)), -1, dtype=np.int32)
    perm = list(rng.permutation(P))
    Kc, Vc = [], []
    for i, L in enumerate(lens):
        kc = _finite_codes(rng, (L, Hkv, d))
        vc = _finite_codes(rng, (L, Hkv, d))
        Kc.append(kc)
        Vc.append(vc)
        for j in range(nb[i]):
            tables[i, j] = perm.pop()
        for t in range(L):
            b, o = tables[i, t // bs], t % bs
            kpool[b, :, o, :] = kc[t]
            vpool[b, :, o // vs, :, o % vs] = vc[t]
    if bs <= 16:
        vpool = vpool.reshape(P, Hkv, d, bs)
    q = (rng.standard_normal((S, Hq, d)) * 4).astype(np.float32)
    return q, Kc, Vc, kpool, vpool, tables, np.array(lens)


def _sdpa(q_i, K, V, sigma, mask=None):
    """torch SDPA in float64; q_i [n][Hq][d] queries, kv head h // G."""
    n, Hq, d = q_i.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    q = torch.from_numpy(q_i).permute(1, 0, 2).unsqueeze(0)                  # [1][Hq][n][d]
    k = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0).contiguous()
    v = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0).unsqueeze(0).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=float(sigma))
    return o[0].permute(1, 0, 2).numpy()                                      # [n][Hq][d]


CASES = [
    (11, [1, 5, 16, 33], 4, 2, 16, 8),
    (12, [3, 17, 40], 8, 1, 32, 16),
    (13, [50, 2], 6, 3, 16, 32),
]


def _decode_error(seed, lens, Hq, Hkv, d, bs, k_scale=K_SCALE, v_scale=V_SCALE):
    q, Kc, Vc, kp, vp, tab, L = _case(seed, lens, Hq, Hkv, d, bs)
    sigma = np.float32(1 / math.sqrt(d))
    got = oracle.paged_decode_attn(q, kp, vp, tab, L, bs=bs, softmax_scale=sigma, q_dtype="f32",
                                   cache_dtype="fp8", k_scale=k_scale, v_scale=v_scale)
    worst = 0.0
    for i in range(len(lens)):
        K = _e4m3_torch(Kc[i]) * float(np.float32(k_scale))
        V = _e4m3_torch(Vc[i]) * float(np.float32(v_scale))
        want = _sdpa(q[i][None].astype(np.float64), K, V, float(sigma))[0]
        worst = max(worst, float(np.max(np.abs(got[i] - want)) / max(np.max(np.abs(want)), 1e-30)))
    return worst


def _lse_error(seed, lens, Hq, Hkv, d, bs, k_scale=K_SCALE):
    q, Kc, _, kp, _, tab, L = _case(seed, lens, Hq, Hkv, d, bs)
    sigma = np.float32(1 / math.sqrt(d))
    got = oracle.paged_decode_lse(q, kp, tab, L, bs=bs, softmax_scale=sigma, q_dtype="f32",
                                  cache_dtype="fp8", k_scale=k_scale)
    worst = 0.0
    G = Hq // Hkv
    for i in range(len(lens)):
        K = torch.from_numpy(_e4m3_torch(Kc[i]) * float(np.float32(k_scale)))      # [L][Hkv][d]
        qi = torch.from_numpy(q[i].astype(np.float64))
        Kh = K[:, torch.arange(Hq) // G, :]                                          # [L][Hq][d]
        s = float(sigma) * torch.einsum("hc,lhc->hl", qi, Kh)
        want = (torch.logsumexp(s, dim=-1) / math.log(2.0)).numpy()
        worst = max(worst, float(np.max(np.abs(got[i] - want))))
    return worst


def _window_error(seed, lens, Hq, Hkv, d, bs, n_q, k_scale=K_SCALE, v_scale=V_SCALE):
    q, Kc, Vc, kp, vp, tab, L = _case(seed, lens, Hq, Hkv, d, bs)
    rng = np.random.default_rng(seed + 100)
    qw = (rng.standard_normal((len(lens), n_q, Hq, d)) * 4).astype(np.float32)
    sigma = np.float32(1 / math.sqrt(d))
    got = oracle.paged_multi_query_attn(qw, kp, vp, tab, L, bs=bs, softmax_scale=sigma, q_dtype="f32",
                                        cache_dtype="fp8", k_scale=k_scale, v_scale=v_scale)
    worst = 0.0
    for i, Li in enumerate(lens):
        K = _e4m3_torch(Kc[i]) * float(np.float32(k_scale))
        V = _e4m3_torch(Vc[i]) * float(np.float32(v_scale))
        # query j sits at position Li - n_q + j and sees positions <= it
        pos = np.arange(Li)[None, :] <= (Li - n_q + np.arange(n_q))[:, None]
        want = _sdpa(qw[i].astype(np.float64), K, V, float(sigma), mask=torch.from_numpy(pos))
        worst = max(worst, float(np.max(np.abs(got[i] - want) / np.maximum(
            np.max(np.abs(want), axis=-1, keepdims=True), 1e-30))))
    return worst


def _write_mismatches(k_inv=np.float32(448.0 / 0.37), v_inv=np.float32(448.0 / 9.5)):
    """Number of codes where the oracle's fp8 write differs from torch's
    float8_e4m3fn conversion of the float32 product x * inv_scale (K and V
    each with their own inverse scale)."""
    rng = np.random.default_rng(21)
    P, Hkv, bs, d, T = 5, 2, 16, 32, 4
    kx = torch.from_numpy((rng.standard_normal((T, Hkv, d)) * 0.1).astype(np.float32)).to(torch.bfloat16)
    vx = torch.from_numpy((rng.standard_normal((T, Hkv, d)) * 3.0).astype(np.float32)).to(torch.bfloat16)
    kbits = kx.view(torch.int16).numpy().view(np.uint16)
    vbits = vx.view(torch.int16).numpy().view(np.uint16)
    kc = np.zeros((P, Hkv, bs, d), dtype=np.uint8)
    vc = np.zeros((P, Hkv, d, bs), dtype=np.uint8)
    slots = np.array([0, 17, 3 * bs + 15, 4 * bs + 2])
    k2, v2 = oracle.kv_cache_write(kbits, vbits, kc, vc, slots, bs=bs, src_dtype="bf16",
                                   cache_dtype="fp8", k_inv_scale=k_inv, v_inv_scale=v_inv)
    # torch: float32 product (one rounding), then the saturating fp8 cast
    ky = (kx.float() * float(k_inv)).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    vy = (vx.float() * float(v_inv)).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = 0
    for t, slot in enumerate(slots):
        b, o = divmod(int(slot), bs)
        bad += int(np.sum(k2[b, :, o, :] != ky[t])) + int(np.sum(v2[b, :, :, o] != vy[t]))
    return bad


# ------------------------------------------------------------------ the pins
@pytest.mark.parametrize("seed,lens,Hq,Hkv,d,bs", CASES)
def test_fp8_decode_against_sdpa_with_distinct_scales(seed, lens, Hq, Hkv, d, bs):
    assert _decode_error(seed, lens, Hq, Hkv, d, bs) < 1e-12


@pytest.mark.parametrize("seed,lens,Hq,Hkv,d,bs", CASES)
def test_fp8_lse_against_logsumexp_with_k_scale(seed, lens, Hq, Hkv, d, bs):
    assert _lse_error(seed, lens, Hq, Hkv, d, bs) < 1e-11


@pytest.mark.parametrize("n_q", [1, 3, 5])
def test_fp8_window_against_masked_sdpa_with_distinct_scales(n_q):
    assert _window_error(14, [5, 9, 33], 8, 2, 16, 16, n_q) < 1e-12


def test_fp8_write_uses_each_tensors_inverse_scale():
    assert _write_mismatches() == 0


# ------------------------------------------------------------------ planted mistakes
def test_planted_swapped_attention_scales_are_caught(monkeypatch):
    real = oatt.paged_decode_attn

    def swapped(*a, k_scale=1.0, v_scale=1.0, **kw):
        return real(*a, k_scale=v_scale, v_scale=k_scale, **kw)
    monkeypatch.setattr(oatt, "paged_decode_attn", swapped)
    monkeypatch.setattr(oracle, "paged_decode_attn", swapped)
    assert _decode_error(*CASES[1]) > 1e-3
    assert _window_error(14, [5, 9, 33], 8, 2, 16, 16, 3) > 1e-3


def test_planted_shared_scale_is_caught(monkeypatch):
    real = oatt.widen

    def one_scale(arr, dtype, scale=1.0):       # every fp8 tensor dequantised with k_scale
        return real(arr, dtype, K_SCALE if dtype == "fp8" else scale)
    monkeypatch.setattr(oatt, "widen", one_scale)
    assert _decode_error(*CASES[2]) > 1e-3


def test_planted_v_scale_in_scores_is_caught(monkeypatch):
    real = oatt.paged_decode_lse

    def wrong(*a, k_scale=1.0, **kw):            # scores scaled by v_scale
        return real(*a, k_scale=V_SCALE, **kw)
    monkeypatch.setattr(oracle, "paged_decode_lse", wrong)
    assert _lse_error(*CASES[0]) > 1e-3


def test_planted_swapped_write_scales_are_caught(monkeypatch):
    real = ocw.kv_cache_write

    def swapped(*a, k_inv_scale=1.0, v_inv_scale=1.0, **kw):
        return real(*a, k_inv_scale=v_inv_scale, v_inv_scale=k_inv_scale, **kw)
    monkeypatch.setattr(oracle, "kv_cache_write", swapped)
    assert _write_mismatches() > 0
