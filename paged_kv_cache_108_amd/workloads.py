"""Seeded synthetic decode workloads: lengths, block tables, pools, queries.

This module only draws inputs. It holds none of the computation under test:
no attention, no cache write, no slot arithmetic, no codec. Both the HIP path
and the CPU oracle are fed from it.

Every random stream is ``numpy.random.default_rng([108, cfg, stream])``:
0 lengths (or private-token counts), 1 block permutation or pool churn, 2 q,
3 K pool, 4 V pool, 5 new K, 6 new V. Values are float32 standard normal;
bf16 storage is the round-to-nearest-even of those float32 values.

Workload shapes (the pages measure none on a GPU; these stand in for the
decode batches they describe: lognormal lengths with a long right tail as in
"03 · PagedAttention", Experiment 1, and "Serving: vLLM and PagedAttention",
section 2.1; beams and shared prefixes as in the copy-on-write figure of the
"PagedAttention" daily term):

  tiny     5 seqs {512, 37, 1900, 128, 4} (the "paged-attention" lesson's worked
           example), 8 q / 8 kv heads, d 64, fp32, bs 16, pool 256 blocks
  small    256 seqs, lognormal(median 300, sigma 1.0) in [1, 4096],
           14 q / 2 kv heads, d 64, bf16, bs 16, pool 1.1x the blocks used
  llama8b  64 seqs, lognormal(median 500, sigma 1.2) in [1, 8192],
           32 q / 8 kv heads, d 128, bf16, bs 16, pool 1.1x
  beam     32 prompts x 4 beams: 1024 shared prefix tokens + 1..200 private,
           32 q / 8 kv heads, d 128, bf16, bs 8 / 16 / 32, pool 1.1x
  long     16 seqs x 32768, 64 q / 8 kv heads, d 128, bf16 or fp8 (e4m3, one
           float32 scale per tensor), bs 16, pool 36045 blocks fragmented by a
           seeded allocate/free churn

Unused slots (free blocks, tails of last blocks, and the slot the step's new
token is about to be written to) hold NaN, so a kernel that reads one as data
instead of masking it produces NaN.

Table construction is the input recipe: sequential block ids (the order a pool
hands out blocks when its first free block is 0 and it grows sequences in the
stated order) mapped through a seeded permutation, or, for ``long``, a plain
stack simulation of allocate/free churn. The library's allocator is checked
against the same op sequences in the tests; it is not used here.
"""

from dataclasses import dataclass, field, replace
import math
import re

import numpy as np

F32, BF16, FP8 = "f32", "bf16", "fp8"
BF16_NAN = np.uint16(0x7FC0)


@dataclass(frozen=True)
class Spec:
    name: str
    cfg: int
    S: int
    Hq: int
    Hkv: int
    d: int
    bs: int
    q_dtype: str
    cache_dtype: str
    src_dtype: str
    partition_size: int
    description: str = ""


SPECS = {
    "tiny": Spec("tiny", 1, 5, 8, 8, 64, 16, F32, F32, F32, 0,
                 "5 seqs {512,37,1900,128,4}, 8/8 heads, d64, fp32, bs16, P=256"),
    "small": Spec("small", 2, 256, 14, 2, 64, 16, BF16, BF16, BF16, 512,
                  "256 seqs lognormal(300,1.0), 14/2 heads, d64, bf16, bs16"),
    "llama8b": Spec("llama8b", 3, 64, 32, 8, 128, 16, BF16, BF16, BF16, 512,
                    "64 seqs lognormal(500,1.2) <=8192, 32/8 heads, d128, bf16, bs16"),
    "beam": Spec("beam", 4, 128, 32, 8, 128, 16, BF16, BF16, BF16, 512,
                 "32 prompts x 4 beams, 1024 shared + 1..200 private, 32/8, d128, bf16"),
    "long": Spec("long", 5, 16, 64, 8, 128, 16, BF16, BF16, BF16, 512,
                 "16 seqs x 32768, 64/8 heads, d128, bs16, churned pool"),
}


def spec(name, **overrides):
    s = SPECS[name]
    return replace(s, **overrides) if overrides else s


def _rng(cfg, stream):
    return np.random.default_rng([108, cfg, stream])


def to_bf16_bits(x):
    """float32 array -> uint16 bf16 bits (round to nearest even, via torch)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _store(x, dtype):
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype in (BF16, FP8):      # fp8 pools are drawn as bf16 values, then quantised
        return to_bf16_bits(x)
    raise ValueError(dtype)


# --------------------------------------------------------------------------- lengths
def lognormal_lengths(cfg, S, median, sigma, lo, hi):
    r = _rng(cfg, 0)
    x = np.floor(r.lognormal(math.log(median), sigma, S)).astype(np.int64)
    return np.clip(x, lo, hi).astype(np.int64)


def _ceil_div(a, b):
    return -(-a // b)


# --------------------------------------------------------------------------- tables
def _tables_from_permutation(lens, bs, P, perm):
    """Sequence i takes the next ceil(L_i/bs) ids of ``perm`` in order."""
    nb = [_ceil_div(int(L), bs) for L in lens]
    maxb = max(max(nb), 1)
    tab = np.full((len(lens), maxb), -1, dtype=np.int32)
    k = 0
    for i, n in enumerate(nb):
        tab[i, :n] = perm[k:k + n]
        k += n
    return tab


def beam_layout(bs, private):
    """Sequential ids for 32 groups x 4 beams: shared prefix then private blocks.

    Order: group g's 1024-token prefix, then beam 0..3's private tokens. Returns
    (tables [128][maxb] with sequential ids, lengths, blocks used).
    """
    pre = 1024 // bs
    rows, lens = [], []
    nxt = 0
    for g in range(32):
        prefix = list(range(nxt, nxt + pre))
        nxt += pre
        for b in range(4):
            k = 4 * g + b
            n = _ceil_div(int(private[k]), bs)
            rows.append(prefix + list(range(nxt, nxt + n)))
            nxt += n
            lens.append(1024 + int(private[k]))
    maxb = max(len(r) for r in rows)
    tab = np.full((128, maxb), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        tab[i, :len(r)] = r
    return tab, np.array(lens, dtype=np.int64), nxt


def churn_ops(P=36045, steps=4000, cfg=5):
    """The seeded allocate/free churn of the ``long`` pool, as a list of ops.

    Each step draws u; if ghost sequences are live and u < 0.5 one of them
    (chosen uniformly among live ids in creation order) is freed, otherwise a
    ghost of 1..256 blocks is allocated if that many blocks are free. Then the
    remaining ghosts are freed in a seeded random order. Ops: ("alloc", id, n)
    and ("free", id). Free-block counting is the only state kept here.
    """
    r = _rng(cfg, 1)
    free = P
    live = []            # ghost ids in creation order
    size = {}
    ops = []
    nxt = 0
    for _ in range(steps):
        u = r.random()
        if live and u < 0.5:
            gid = live.pop(int(r.integers(len(live))))
            ops.append(("free", gid))
            free += size.pop(gid)
        else:
            n = int(r.integers(1, 257))
            if n <= free:
                ops.append(("alloc", nxt, n))
                size[nxt] = n
                live.append(nxt)
                free -= n
                nxt += 1
    for idx in r.permutation(len(live)):
        gid = live[int(idx)]
        ops.append(("free", gid))
    return ops


def churned_tables(P=36045, S=16, blocks_per_seq=2048, cfg=5):
    """Replay ``churn_ops`` on a stack pool (first pop = block 0; a freed
    sequence pushes its blocks last-first), then grow S sequences one block at a
    time, interleaved: for j < blocks_per_seq, for s < S, pop one block."""
    stack = list(range(P - 1, -1, -1))
    held = {}
    for op in churn_ops(P, cfg=cfg):
        if op[0] == "alloc":
            held[op[1]] = [stack.pop() for _ in range(op[2])]
        else:
            for b in reversed(held.pop(op[1])):
                stack.append(b)
    tab = np.full((S, blocks_per_seq), -1, dtype=np.int32)
    for j in range(blocks_per_seq):
        for s in range(S):
            tab[s, j] = stack.pop()
    return tab


# --------------------------------------------------------------------------- workload
@dataclass
class Workload:
    spec: Spec
    P: int
    q: np.ndarray              # [S][Hq][d]      f32 or bf16 bits
    k_pool: np.ndarray         # [P][Hkv][bs][d] f32 or bf16 bits (fp8: values to quantise)
    v_pool: np.ndarray         # [P][Hkv][d][bs] for bs <= 16, else [P][Hkv][bs/16][d][16]
    block_tables: np.ndarray   # int32 [S][maxB], -1 padded
    context_lens: np.ndarray   # int32 [S], includes this step's new token
    k_new: np.ndarray          # [S][Hkv][d] source dtype
    v_new: np.ndarray
    k_scale: float = 1.0       # fp8 only: value = decode(code) * scale
    v_scale: float = 1.0
    k_inv_scale: float = 1.0   # fp8 only: code = encode(x * inv_scale)
    v_inv_scale: float = 1.0
    softmax_scale: float = 1.0
    extra: dict = field(default_factory=dict)

    @property
    def max_blocks(self):
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self):
        return int(self.context_lens.max()) if len(self.context_lens) else 0


def _valid_mask(tables, lens, bs, P):
    """bool [P][bs]: slots holding a token of some sequence."""
    valid = np.zeros((P, bs), dtype=bool)
    for i, L in enumerate(lens):
        L = int(L)
        n = _ceil_div(L, bs)
        if n <= 0:
            continue
        ids = tables[i, :n].astype(np.int64)
        valid[ids[:-1], :] = True
        valid[ids[-1], :L - (n - 1) * bs] = True
    return valid


def v_pool_shape(P, Hkv, d, bs):
    """V pool shape: one channel-major tile per (block, kv head), in sub-tiles of
    16 tokens when bs > 16 (the library's layout)."""
    return (P, Hkv, d, bs) if bs <= 16 else (P, Hkv, bs // 16, d, 16)


def _poison(pool_k, pool_v, valid, dtype):
    nan = np.float32(np.nan) if dtype == F32 else BF16_NAN
    inv = ~valid                                   # [P][bs]
    b_idx, o_idx = np.nonzero(inv)
    pool_k[b_idx, :, o_idx, :] = nan
    if pool_v.ndim == 4:
        pool_v[b_idx, :, :, o_idx] = nan
    else:
        pool_v[b_idx, :, o_idx // 16, :, o_idx % 16] = nan


def generate(s, tables, lens, P, *, extra=None, poison_new=True, value_scales=(1.0, 1.0)):
    """Draw q, pools and new tokens for a spec with given tables and lengths.
    K values (pool and new tokens) are N(0, 1) times value_scales[0], V values
    times value_scales[1]."""
    cfg, S, Hq, Hkv, d, bs = s.cfg, s.S, s.Hq, s.Hkv, s.d, s.bs
    assert tables.shape[0] == S and len(lens) == S
    ks, vs = (np.float32(x) for x in value_scales)
    q32 = _rng(cfg, 2).standard_normal((S, Hq, d), dtype=np.float32)
    k32 = _rng(cfg, 3).standard_normal((P, Hkv, bs, d), dtype=np.float32)
    v32 = _rng(cfg, 4).standard_normal(v_pool_shape(P, Hkv, d, bs), dtype=np.float32)
    kn32 = _rng(cfg, 5).standard_normal((S, Hkv, d), dtype=np.float32)
    vn32 = _rng(cfg, 6).standard_normal((S, Hkv, d), dtype=np.float32)
    if ks != 1.0:
        k32 *= ks
        kn32 *= ks
    if vs != 1.0:
        v32 *= vs
        vn32 *= vs
    pool_dtype = F32 if s.cache_dtype == F32 else BF16
    k_pool = _store(k32, pool_dtype)
    del k32
    v_pool = _store(v32, pool_dtype)
    del v32
    valid = _valid_mask(tables, lens, bs, P)
    if poison_new:
        # The step's new token (position L-1) is not in the pool yet.
        for i, L in enumerate(lens):
            L = int(L)
            if L > 0:
                b = int(tables[i, (L - 1) // bs])
                valid[b, (L - 1) % bs] = False
    _poison(k_pool, v_pool, valid, pool_dtype)
    w = Workload(
        spec=s, P=P, q=_store(q32, s.q_dtype), k_pool=k_pool, v_pool=v_pool,
        block_tables=np.ascontiguousarray(tables, dtype=np.int32),
        context_lens=np.asarray(lens, dtype=np.int32),
        k_new=_store(kn32, s.src_dtype), v_new=_store(vn32, s.src_dtype),
        softmax_scale=float(np.float32(1.0 / math.sqrt(d))), extra=dict(extra or {}))
    if s.cache_dtype == FP8:
        _fp8_scales(w, valid)
    return w


def _bf16_abs_max(bits):
    """Largest finite |value| among bf16 bit patterns (NaNs ignored)."""
    mag = (np.asarray(bits, dtype=np.uint16) & np.uint16(0x7FFF))
    mag = mag[mag < 0x7F80]
    if mag.size == 0:
        return 0.0
    top = np.uint32(mag.max()) << np.uint32(16)
    return float(np.array([top], dtype=np.uint32).view(np.float32)[0])


def _fp8_scales(w, valid):
    """One float32 scale per tensor: amax/448 over the values that will be stored."""
    for which, pool, new in (("k", w.k_pool, w.k_new), ("v", w.v_pool, w.v_new)):
        amax = max(_bf16_abs_max(pool), _bf16_abs_max(new))
        scale = np.float32(amax / 448.0)
        inv = np.float32(448.0 / amax)
        setattr(w, f"{which}_scale", float(scale))
        setattr(w, f"{which}_inv_scale", float(inv))


def _described(base, s):
    """s with its description naming the block size and cache type it was made
    with, where they differ from the named workload's."""
    text = s.description
    if s.bs != base.bs:
        text = re.sub(r"\bbs\d+\b", f"bs{s.bs}", text) if re.search(r"\bbs\d+\b", text) else f"{text}, bs{s.bs}"
    if s.cache_dtype != base.cache_dtype:
        text = f"{text}, {s.cache_dtype} cache"
    return replace(s, description=text)


def make(name, *, bs=None, cache_dtype=None, poison_new=True):
    """The named workload (see the module docstring)."""
    s = SPECS[name]
    if bs is not None:
        s = replace(s, bs=bs)
    if cache_dtype is not None:
        s = replace(s, cache_dtype=cache_dtype)
    s = _described(SPECS[name], s)
    if name == "tiny":
        lens = np.array([512, 37, 1900, 128, 4], dtype=np.int64)
        P = 256
        perm = _rng(1, 1).permutation(P)
        tables = _tables_from_permutation(lens, s.bs, P, perm)
        extra = {}
    elif name in ("small", "llama8b"):
        med, sig, hi = (300, 1.0, 4096) if name == "small" else (500, 1.2, 8192)
        lens = lognormal_lengths(s.cfg, s.S, med, sig, 1, hi)
        used = int(sum(_ceil_div(int(L), s.bs) for L in lens))
        P = int(math.ceil(1.1 * used))
        perm = _rng(s.cfg, 1).permutation(P)
        tables = _tables_from_permutation(lens, s.bs, P, perm)
        extra = {"blocks_used": used}
    elif name == "beam":
        private = _rng(4, 0).integers(1, 201, 128)
        seq_tab, lens, used = beam_layout(s.bs, private)
        P = int(math.ceil(1.1 * used))
        perm = _rng(4, 1).permutation(P).astype(np.int32)
        tables = np.where(seq_tab >= 0, perm[np.maximum(seq_tab, 0)], -1).astype(np.int32)
        extra = {"blocks_used": used, "private": private, "sequential_tables": seq_tab}
    elif name == "long":
        P = 36045
        tables = churned_tables(P, s.S, 32768 // s.bs, cfg=5)
        lens = np.full(s.S, 32768, dtype=np.int64)
        extra = {"blocks_used": int(s.S * 32768 // s.bs)}
    else:
        raise KeyError(name)
    return generate(s, tables, lens, P, extra=extra, poison_new=poison_new)


def make_custom(*, lens, Hq, Hkv, d, bs, q_dtype=BF16, cache_dtype=BF16, cfg=900,
                pool_factor=1.5, partition_size=512, poison_new=True, value_scales=(1.0, 1.0)):
    """A small ad-hoc workload (edge cases): ``lens`` may hold zeros; ids permuted.
    value_scales multiplies the K and the V values (see ``generate``)."""
    dtype_src = F32 if cache_dtype == F32 else BF16
    s = Spec("custom", cfg, len(lens), Hq, Hkv, d, bs, q_dtype, cache_dtype, dtype_src,
             partition_size)
    lens = np.asarray(lens, dtype=np.int64)
    used = int(sum(_ceil_div(max(int(L), 0), bs) for L in lens))
    P = max(int(math.ceil(pool_factor * used)), 1)
    perm = _rng(cfg, 1).permutation(P)
    tables = _tables_from_permutation(np.maximum(lens, 0), bs, P, perm)
    return generate(s, tables, lens, P, poison_new=poison_new, value_scales=value_scales)
