#!/usr/bin/env python3
"""Benchmark one decode step of paged attention on one MI355X.

A step is the whole hot path over one batch: the KV-cache write of each
sequence's new token and paged decode attention over every sequence's context
including that token. By default one pkv_paged_decode_step_planned call does
both (the planned attention kernel with the write fused in, then the merge
kernel), with the work plan built on the host before the timed region, as the
block tables are; --step fused times the unplanned pkv_paged_decode_step
(the stream kernel derives the same split on the device); --step split times
pkv_kv_cache_write, then pkv_paged_decode_attn (balanced split by default;
--partition N selects fixed partitions of N tokens). Inputs are seeded
synthetic workloads already resident in HBM.

Timing: W untimed warm-up steps, then K timed steps (50 by default). Before
each timed step (outside its event pair) a 1 GiB buffer is read so neither the
256 MB Infinity Cache nor L2 still holds the KV pool; each step is bracketed by
HIP events on the stream the kernels run on (with --step split, a third event
between the write and the attention call). Python's garbage collector is off
while the timed steps are enqueued. `value` uses the median step time.
Bytes are algorithmic: what the method must move (each valid token's K and V
once, shared blocks once, q, the fp32 output, the table entries and lengths;
for the write, the new tokens read and stored and the slot mapping).

Alongside the step (unless --no-companions), in the same process and with the
same flush and event protocol: pkv_stream_read over the step's byte count in
a few launch shapes (the practical read ceiling), pkv_paged_gather_read of the
plan's chunks (the step's own scattered reads without arithmetic), the
attention call with 512-token partitions, and the unplanned fused step.

Prints ONE JSON line.
"""

import argparse
import contextlib
import gc
import json
import math
import os
import statistics
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published peak

ELEM = {"f32": 4, "bf16": 2, "fp8": 1}

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_cache_108_amd", "csrc")
# every file of device code: the counters hold only while all of them are unchanged
DEVICE_SOURCES = [os.path.join(CSRC, f) for f in ("device.hip", "attn_kernels.h", "attn_inst.hip", "split.h")]


def _code_only(text):
    """C++ source text without its comments, blank lines and trailing blanks: a
    comment edit leaves the compiled kernels, and so the counters, unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                         # string or character literal, kept whole
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (line.rstrip() for line in "".join(out).split("\n"))
    return "\n".join(line for line in lines if line)


def device_source_sha256(paths=None):
    """SHA-256 over the code of the device sources (comments left out), in order."""
    import hashlib
    h = hashlib.sha256()
    for path in paths or DEVICE_SOURCES:
        with open(path, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()

# HBM traffic of one measured call (its two kernels), from
# rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE runs of this script's default
# command, in KiB per call, and the scale that turns each counter into bytes
# (what the counter reads for a plain copy of known size). Reported only while
# the kernel source is the one the counters were taken with.
MEASURED_TRAFFIC = {
    ("beam", "bf16", 16, -1, "planned"): {
        "source_sha256": "820800b3ff5373f9f148bf35ac40925d69bcc578f999c8d58b411164ae5ff0dd",
        "fetch_kib": 245784.3, "write_kib": 10434.2, "fetch_scale": 2.0, "write_scale": 1.0,
    },
    ("llama8b", "bf16", 16, -1, "planned"): {
        "source_sha256": "820800b3ff5373f9f148bf35ac40925d69bcc578f999c8d58b411164ae5ff0dd",
        "fetch_kib": 170306.3, "write_kib": 5939.4, "fetch_scale": 2.0, "write_scale": 1.0,
    },
    ("small", "bf16", 16, -1, "planned"): {
        "source_sha256": "820800b3ff5373f9f148bf35ac40925d69bcc578f999c8d58b411164ae5ff0dd",
        "fetch_kib": 34303.6, "write_kib": 4412.8, "fetch_scale": 2.0, "write_scale": 1.0,
    },
    ("llama8b", "fp8", 16, -1, "planned"): {
        "source_sha256": "820800b3ff5373f9f148bf35ac40925d69bcc578f999c8d58b411164ae5ff0dd",
        "fetch_kib": 86285.4, "write_kib": 4806.0, "fetch_scale": 2.0, "write_scale": 1.0,
    },
    ("small", "fp8", 16, -1, "planned"): {
        "source_sha256": "820800b3ff5373f9f148bf35ac40925d69bcc578f999c8d58b411164ae5ff0dd",
        "fetch_kib": 18918.9, "write_kib": 5530.5, "fetch_scale": 2.0, "write_scale": 1.0,
    },
    ("long", "bf16", 16, -1, "planned"): {
        "source_sha256": "820800b3ff5373f9f148bf35ac40925d69bcc578f999c8d58b411164ae5ff0dd",
        "fetch_kib": 1054201.7, "write_kib": 5730.8, "fetch_scale": 2.0, "write_scale": 1.0,
    },
    ("long", "fp8", 16, -1, "planned"): {
        "source_sha256": "820800b3ff5373f9f148bf35ac40925d69bcc578f999c8d58b411164ae5ff0dd",
        "fetch_kib": 529611.1, "write_kib": 5453.8, "fetch_scale": 2.0, "write_scale": 1.0,
    },
}


def measured_traffic(name, cache_dtype, bs, part, step="planned"):
    """Bytes per attention call from the counters, or None when none were taken
    for this configuration or the kernel source has changed since."""
    m = MEASURED_TRAFFIC.get((name, cache_dtype, bs, part, step))
    if m is None:
        return None
    if device_source_sha256() != m["source_sha256"]:
        return None
    return int(round(1024 * (m["fetch_kib"] * m["fetch_scale"] + m["write_kib"] * m["write_scale"])))


def algorithmic_bytes(w, cache_dtype):
    """(attention bytes, write bytes, logical KV bytes) for one step of workload w."""
    s = w.spec
    bs, Hkv, d = s.bs, s.Hkv, s.d
    fill = {}
    n_entries = 0
    for i, L in enumerate(w.context_lens):
        L = int(L)
        n = -(-L // bs) if L > 0 else 0
        n_entries += n
        for j in range(n):
            b = int(w.block_tables[i, j])
            f = min(bs, L - j * bs)
            if f > fill.get(b, 0):
                fill[b] = f
    unique_tokens = sum(fill.values())
    logical_tokens = int(np.maximum(w.context_lens, 0).sum())
    kv_elem = ELEM[cache_dtype]
    kv = unique_tokens * 2 * Hkv * d * kv_elem
    q = s.S * s.Hq * d * ELEM[s.q_dtype]
    out = s.S * s.Hq * d * 4
    attn = kv + q + out + 4 * n_entries + 4 * s.S
    T = s.S
    write = T * 2 * Hkv * d * (ELEM[s.src_dtype] + kv_elem) + 8 * T
    return attn, write, logical_tokens * 2 * Hkv * d * kv_elem, unique_tokens


def _oracle_pools(w, cache_dtype, seqs):
    """The oracle's own pools after this step's write, for the listed sequences'
    blocks (fp8: the oracle quantises those blocks itself). Not timed."""
    import oracle
    s = w.spec
    slots = oracle.decode_slots(w.block_tables, w.context_lens, s.bs)
    if cache_dtype != "fp8":
        return oracle.kv_cache_write(w.k_new, w.v_new, w.k_pool, w.v_pool, slots, bs=s.bs,
                                     src_dtype=s.src_dtype, cache_dtype=cache_dtype)
    blocks = np.unique(w.block_tables[seqs].reshape(-1))
    blocks = blocks[blocks >= 0]
    kq = np.zeros(w.k_pool.shape, dtype=np.uint8)
    vq = np.zeros(w.v_pool.shape, dtype=np.uint8)
    kq[blocks] = oracle.quantise(w.k_pool[blocks], "bf16", w.k_inv_scale)
    vq[blocks] = oracle.quantise(w.v_pool[blocks], "bf16", w.v_inv_scale)
    return oracle.kv_cache_write(w.k_new, w.v_new, kq, vq, slots, bs=s.bs, src_dtype="bf16",
                                 cache_dtype="fp8", k_inv_scale=w.k_inv_scale,
                                 v_inv_scale=w.v_inv_scale)


def cpu_baseline(w, cache_dtype, budget_s=12.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of sequences:
    sequences in order, one call each, until the time budget is spent."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] + [1])
    except Exception:
        threads = 1
    s = w.spec
    # sequences the budget can plausibly cover (bounded prep for big pools)
    est = max(1, min(s.S, int(budget_s * 2e8 / max(1, 2 * s.Hkv * s.d * 8 * np.mean(w.context_lens)))))
    kc, vc = _oracle_pools(w, cache_dtype, list(range(min(s.S, est + 2))))
    done, t_used, kv_bytes = [], 0.0, 0
    sample = list(range(min(s.S, est + 2)))
    for n in range(10**6):                 # passes over the sample until the budget is spent
        i = sample[n % len(sample)]
        t0 = time.perf_counter()
        oracle.paged_decode_attn(w.q, kc, vc, w.block_tables, w.context_lens, bs=s.bs,
                                 softmax_scale=w.softmax_scale, q_dtype=s.q_dtype,
                                 cache_dtype=cache_dtype, k_scale=w.k_scale, v_scale=w.v_scale,
                                 seqs=[i])
        t_used += time.perf_counter() - t0
        done.append(i)
        kv_bytes += int(w.context_lens[i]) * 2 * s.Hkv * s.d * ELEM[cache_dtype] \
            + s.Hq * s.d * (ELEM[s.q_dtype] + 4)
        if t_used >= budget_s:
            break
    return {
        "value": round(len(done) / t_used, 3), "unit": "seq-steps/s",
        "gbs": round(kv_bytes / t_used / 1e9, 4), "cores": int(threads),
        "affinity_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
        "sample": f"oracle paged_decode_attn, {len(done)} calls of one sequence each over "
                  f"sequences 0..{len(sample) - 1} of {s.S} "
                  f"({int(sum(int(w.context_lens[i]) for i in done))} tokens), {t_used:.1f} s",
    }


@contextlib.contextmanager
def _no_gc():
    """Python's collector off while a timed loop enqueues work: a full
    collection over the objects torch holds pauses the host for tens of ms,
    and an event pair that waits on the host then times an idle GPU."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


def _timed(args, torch, fn, flush, stream, steps=None, warmup=None):
    """Mean, median and min event time in ms of fn over the timed calls (after
    the warm-up calls), each preceded by the flush read outside the events;
    also the wall time of the timed region."""
    steps = args.steps if steps is None else steps
    for _ in range(args.warmup if warmup is None else warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    with _no_gc():
        wall0 = time.perf_counter()
        for a, b in ev:
            if not args.no_flush:
                flush.max()
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
    ms = [a.elapsed_time(b) for a, b in ev]
    return statistics.mean(ms), statistics.median(ms), min(ms), wall


# Launch shapes of the streaming-read reference (unroll, workgroups); the best
# median is reported. Measured on MI355X: each is the best at one of the byte
# counts of the workloads here (66 MB .. 2.1 GB).
READ_SHAPES = [(4, 512), (8, 256), (16, 2048), (16, 8192)]


def companions(args, torch, pkv, w, flush, stream, bufs, step_bytes, attn_bytes, plan=None):
    """The read ceiling over step_bytes, the gather of the step's own chunks
    (with a plan), the 512-token-partition attention call and the unplanned
    fused step, each timed like the step (median)."""
    s = w.spec
    q, k_new, v_new, k_cache, v_cache, tables, lens, out = bufs
    res = {}
    if plan is not None:
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        _, med, _, _ = _timed(args, torch, lambda: plan.gather(k_cache, v_cache, tables, sink, stream=stream),
                              flush, stream)
        chunks = int(sum(-(-int(L) // 16) for L in np.minimum(w.context_lens, w.max_context_len) if L > 0)) * s.Hkv
        kv_bytes = chunks * 16 * 2 * s.d * ELEM[s.cache_dtype]
        res["gather_ceiling"] = {
            "kernel": "pkv_paged_gather_read: the plan's K/V chunks through the block tables with the planned "
                      "kernel's loads, pipeline and grid, no arithmetic",
            "bytes_read": kv_bytes, "ms_median": round(med, 5), "gbs": round(kv_bytes / (med * 1e-3) / 1e9, 1)}
    src = torch.empty(step_bytes + 16, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    shapes = []
    for unroll, blocks in READ_SHAPES:
        _, med, mn, _ = _timed(args, torch, lambda: pkv.stream_read(src, sink, nbytes=step_bytes, blocks=blocks,
                                                                     unroll=unroll, stream=stream),
                               flush, stream)
        shapes.append({"unroll": unroll, "workgroups": blocks, "ms_median": round(med, 5),
                       "gbs": round(step_bytes / (med * 1e-3) / 1e9, 1)})
    best = max(shapes, key=lambda x: x["gbs"])
    res["read_ceiling"] = {
        "kernel": "pkv_stream_read (nontemporal 16-byte loads, grid-stride)", "bytes": int(step_bytes),
        "gbs": best["gbs"], "ms_median": best["ms_median"], "frac_of_peak": round(best["gbs"] / HBM_PEAK_GBS, 4),
        "best_shape": {"unroll": best["unroll"], "workgroups": best["workgroups"]}, "shapes": shapes,
    }
    del src
    # attention alone with 512-token partitions (split-K), and the unplanned fused step
    ws512 = pkv.paged_decode_attn_workspace(s.S, s.Hq, s.Hkv, s.d, w.max_context_len, 512)
    _, med, _, _ = _timed(args, torch, lambda: pkv.paged_decode_attn(
        out, q, k_cache, v_cache, tables, lens, max_context_len=w.max_context_len, softmax_scale=w.softmax_scale,
        k_scale=w.k_scale, v_scale=w.v_scale, partition_size=512, workspace=ws512, stream=stream), flush, stream)
    g = attn_bytes / (med * 1e-3) / 1e9
    res["partition_512_attention"] = {
        "call": "pkv_paged_decode_attn, partition_size 512 (partition kernel + merge kernel), no write",
        "bytes": int(attn_bytes), "ms_median": round(med, 5), "gbs": round(g, 1),
        "pct_of_peak": round(100 * g / HBM_PEAK_GBS, 2)}
    wsb = pkv.paged_decode_attn_workspace(s.S, s.Hq, s.Hkv, s.d, w.max_context_len, pkv.PKV_PARTITION_BALANCED)
    _, med, _, _ = _timed(args, torch, lambda: pkv.paged_decode_step(
        out, q, k_new, v_new, k_cache, v_cache, tables, lens, max_context_len=w.max_context_len,
        softmax_scale=w.softmax_scale, k_scale=w.k_scale, v_scale=w.v_scale, k_inv_scale=w.k_inv_scale,
        v_inv_scale=w.v_inv_scale, workspace=wsb, stream=stream), flush, stream)
    g = step_bytes / (med * 1e-3) / 1e9
    res["unplanned_fused_step"] = {
        "call": "pkv_paged_decode_step (stream kernel deriving the split on the device + merge kernel)",
        "bytes": int(step_bytes), "ms_median": round(med, 5), "gbs": round(g, 1),
        "pct_of_peak": round(100 * g / HBM_PEAK_GBS, 2)}
    return res


def run_other_op(args, w, torch, pkv):
    """--op window / --op copy: one JSON line for that call on workload w."""
    from paged_kv_cache_108_amd import workloads as W
    s = w.spec
    cache_dtype = s.cache_dtype

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    if cache_dtype == "fp8":
        vk, vv = dev(w.k_pool), dev(w.v_pool)
        k_cache = torch.empty(vk.shape, dtype=torch.uint8, device="cuda")
        v_cache = torch.empty(vv.shape, dtype=torch.uint8, device="cuda")
        pkv.quantise_pool(vk, vv, k_cache, v_cache, k_inv_scale=w.k_inv_scale,
                          v_inv_scale=w.v_inv_scale)
        del vk, vv
    else:
        k_cache, v_cache = dev(w.k_pool), dev(w.v_pool)
    flush = torch.ones(1 << 27, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    kv_elem = ELEM[cache_dtype]
    if args.op == "window":
        n_q = args.window
        G = s.Hq // s.Hkv
        tiles = 1 if n_q * G <= 16 else 2             # 16-column tiles per pass (as the library)
        qgs = min(n_q, max(16 * tiles // G, 1))
        n_qg = -(-n_q // qgs)
        rng = np.random.default_rng([108, 951, n_q])
        qf = rng.standard_normal((s.S, n_q, s.Hq, s.d)).astype(np.float32)
        q = dev(qf if s.q_dtype == "f32" else W.to_bf16_bits(qf))
        tables, lens = dev(w.block_tables), dev(w.context_lens)
        out = torch.empty((s.S, n_q, s.Hq, s.d), dtype=torch.float32, device="cuda")
        ws = pkv.paged_multi_query_attn_workspace(s.S, n_q, s.Hq, s.Hkv, s.d)
        plan = pkv.WindowPlan(w.context_lens, n_q=n_q, Hq=s.Hq, Hkv=s.Hkv, d=s.d, bs=s.bs,
                              cache_dtype_code={"f32": 0, "bf16": 1, "fp8": 2}[cache_dtype],
                              max_context_len=w.max_context_len)

        def fn_unplanned():
            pkv.paged_multi_query_attn(out, q, k_cache, v_cache, tables, lens,
                                       max_context_len=w.max_context_len,
                                       softmax_scale=w.softmax_scale, k_scale=w.k_scale,
                                       v_scale=w.v_scale, workspace=ws, stream=stream)

        def fn_planned():
            plan(out, q, k_cache, v_cache, tables, lens, softmax_scale=w.softmax_scale, k_scale=w.k_scale,
                 v_scale=w.v_scale, stream=stream)
        # both calls group the window's columns alike (one or two 16-column
        # tiles per pass); the planned one is the faster at every width measured
        planned = args.window_call == "planned"
        fn, other = (fn_planned, fn_unplanned) if planned else (fn_unplanned, fn_planned)
        if planned:
            qgs, n_qg = int(plan.host[13]), int(plan.host[14])
            tiles = 1 if qgs * G <= 16 else 2
        attn, _, _, unique_tokens = algorithmic_bytes(w, cache_dtype)
        dec_q = s.S * s.Hq * s.d * ELEM[s.q_dtype]
        dec_out = s.S * s.Hq * s.d * 4
        once = attn - dec_q - dec_out                 # K/V, tables, lengths: read once
        byts = once + n_q * (dec_q + dec_out)
        passes = once * n_qg + n_q * (dec_q + dec_out)
        metric = "paged multi-query (window) attention: achieved HBM GB/s at 1 GPU"
        kernel = ("paged_multi_query_attn_planned call (planned kernel, window mode + merge kernel)" if planned
                  else "paged_multi_query_attn call (stream kernel, window instantiation + merge kernel)")
        cfg = {"window": n_q, "call": "planned" if planned else "unplanned", "column_tiles": tiles,
               "queries_per_pass": qgs, "passes": n_qg, "bytes_with_passes": passes,
               "note": "value counts K/V once; a window needing several passes reads K/V once per pass "
                       "(bytes_with_passes)"}
    elif args.op == "shared":
        q, k_new, v_new = dev(w.q), dev(w.k_new), dev(w.v_new)
        run = pkv.SharedPrefixDecode(w.block_tables, w.context_lens, args.group, s.bs, s.Hq, s.Hkv, s.d)
        out = torch.empty((s.S, s.Hq, s.d), dtype=torch.float32, device="cuda")

        def fn():
            run(out, q, k_cache, v_cache, softmax_scale=w.softmax_scale, k_scale=w.k_scale,
                v_scale=w.v_scale, k_new=k_new, v_new=v_new, k_inv_scale=w.k_inv_scale,
                v_inv_scale=w.v_inv_scale, stream=stream)
        attn, write, logical, unique_tokens = algorithmic_bytes(w, cache_dtype)
        byts = attn + write                  # unique K/V once, q, out, tables, lengths; the write
        metric = "shared-prefix decode step (write + attention): achieved HBM GB/s at 1 GPU"
        kernel = ("pkv_paged_shared_prefix_decode call (suffix stream kernel with the write, prefix "
                  "window kernel, shared-prefix merge kernel)")
        cfg = {"group": args.group, "prefix_tokens": run.prefix_tokens, "unique_tokens": int(unique_tokens),
               "context_tokens": int(w.context_lens.sum()), "kv_bytes_logical": int(logical)}
    else:
        per_pool = s.Hkv * s.bs * s.d * kv_elem           # one block of one pool
        n = min(args.pairs, w.P // 2)
        perm = np.random.default_rng([108, 952]).permutation(w.P)
        src = torch.from_numpy(perm[:n].astype(np.int32)).cuda()
        dst = torch.from_numpy(perm[n:2 * n].astype(np.int32)).cuda()

        def fn():
            pkv.copy_blocks(k_cache, v_cache, src, dst, stream=stream)
        byts = n * 2 * 2 * per_pool                        # both pools, read + write
        metric = "copy-on-write block copies: achieved HBM GB/s at 1 GPU"
        kernel = "copy_blocks call (copy_blocks_kernel)"
        cfg = {"pairs": n, "bytes_per_pair": 4 * per_pool}
    mean, med, mn, wall = _timed(args, torch, fn, flush, stream)
    gbs = byts / (mean * 1e-3) / 1e9
    if args.op == "window":
        # the other window call on the same inputs, for comparison
        o_mean, o_med, _, _ = _timed(args, torch, other, flush, stream)
        cfg["other_call"] = {"call": "unplanned" if planned else "planned", "ms_mean": round(o_mean, 5),
                             "ms_median": round(o_med, 5)}
    print(json.dumps({
        "metric": metric, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(mean, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 KV, bf16 q"}[cache_dtype],
        "data": "synthetic (seeded)",
        "config": dict({"workload": f"{s.name}: {s.description}", "block_size": s.bs,
                        "kv_dtype": cache_dtype, "cache_flush_between_steps": not args.no_flush}, **cfg),
        "timing": {"ms_mean": round(mean, 5), "ms_median": round(med, 5), "ms_min": round(mn, 5),
                   "wall_s_timed_region": round(wall, 4)},
        "bytes": {"algorithmic": int(byts)},
        "roofline": {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "device": torch.cuda.get_device_name(0),
    }), flush=True)


def run_prefix(args):
    """--op prefix: admission of requests that share a system prompt through the
    host allocator's prefix cache (chained block hashes, cached full blocks).
    Host code only; one JSON line."""
    import paged_kv_cache_108_amd as pkv
    bs, n_req, shared = 16, 64, 1024
    rng = np.random.default_rng([108, 953])
    system = rng.integers(0, 32000, shared)
    private = np.clip(np.floor(np.exp(rng.normal(np.log(500), 1.0, n_req))), 1, 4096).astype(int)
    prompts = [np.concatenate([system, rng.integers(0, 32000, int(n))]).astype(np.int32) for n in private]
    blocks_needed = sum(-(-len(t) // bs) for t in prompts) + 64
    reps = max(args.steps, 1)
    times, hits, misses, hashed = [], 0, 0, 0
    for _ in range(reps):
        alloc = pkv.Allocator(blocks_needed, bs)
        t0 = time.perf_counter()
        for k, t in enumerate(prompts):
            alloc.create_prefixed(k, t)
        times.append(time.perf_counter() - t0)
        st = alloc.prefix_stats()
        hits, misses = st["hit_blocks"], st["miss_blocks"]
        alloc.close()
    hashed = sum(len(t) // bs for t in prompts)
    mean = statistics.mean(times)
    print(json.dumps({
        "metric": "prefix-cache admission (host): requests/s and hashed blocks/s", "value": round(n_req / mean, 1),
        "unit": "requests/s", "n_gpus": 0, "steps": reps, "warmup": 0, "ms_per_step": round(1e3 * mean, 4),
        "higher_is_better": True, "scaling": "none", "vs_baseline": None, "dtype": "int32 tokens",
        "data": "synthetic (seeded)",
        "config": {"workload": f"{n_req} requests sharing a {shared}-token system prompt, lognormal(500, 1.0) "
                               f"private tokens, bs {bs}", "tokens": int(sum(len(t) for t in prompts)),
                   "full_blocks_hashed": hashed, "hit_blocks": hits, "miss_blocks": misses},
        "timing": {"s_mean": round(mean, 6), "s_min": round(min(times), 6),
                   "us_per_hashed_block": round(1e6 * mean / hashed, 3)},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="llama8b",
                    choices=["tiny", "small", "llama8b", "beam", "long"])
    ap.add_argument("--bs", type=int, default=None)
    ap.add_argument("--kv", default=None, choices=[None, "bf16", "fp8", "f32"])
    ap.add_argument("--partition", type=int, default=-1,
                    help="partition_size for paged_decode_attn: -1 = balanced split (default), "
                         "0 = one pass per (sequence, kv head), else tokens per partition")
    ap.add_argument("--step", choices=["planned", "fused", "split"], default="planned",
                    help="planned: one pkv_paged_decode_step_planned call writes the new tokens and attends, "
                         "its plan built on the host before the timed region (default); fused: one "
                         "pkv_paged_decode_step call (balanced split derived on the device); split: "
                         "pkv_kv_cache_write, then pkv_paged_decode_attn")
    ap.add_argument("--no-companions", action="store_true",
                    help="skip the read ceiling, the 512-partition call and the unplanned step")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--op", choices=["step", "window", "copy", "prefix", "shared"], default="step",
                    help="step: the decode step (default); window: pkv_paged_multi_query_attn over "
                         "windows of --window queries per sequence; copy: pkv_copy_blocks of --pairs "
                         "(src, dst) block pairs; prefix: host-side prefix-cache admission "
                         "(pkv_seq_create_prefixed), no GPU; shared: shared-prefix decode step "
                         "(pkv_paged_shared_prefix_decode) for groups of --group sequences")
    ap.add_argument("--window", type=int, default=4, help="queries per sequence for --op window")
    ap.add_argument("--window-call", default="planned", choices=["planned", "unplanned"],
                    help="--op window: the call timed (default: the planned call); the other is timed beside it")
    ap.add_argument("--pairs", type=int, default=1024, help="block pairs for --op copy")
    ap.add_argument("--group", type=int, default=4, help="sequences per group for --op shared")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)

    if args.op == "prefix":
        run_prefix(args)
        return

    import torch
    import paged_kv_cache_108_amd as pkv
    from paged_kv_cache_108_amd import workloads as W

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)

    if args.copy_calibration:
        # A plain copy of known size: under rocprofv3 --pmc its FETCH_SIZE and
        # WRITE_SIZE per dispatch give the counters' scale (bytes = MiB * 2^20).
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "dispatches": max(args.steps, 1)}))
        return

    w = W.make(args.config, bs=args.bs, cache_dtype=args.kv)
    s = w.spec
    if args.op != "step":
        run_other_op(args, w, torch, pkv)
        return
    cache_dtype = s.cache_dtype
    part = args.partition
    one_call = args.step in ("planned", "fused")
    if one_call and part != pkv.PKV_PARTITION_BALANCED:
        print(json.dumps({"error": f"--step {args.step} takes the balanced split (--partition -1)"}))
        sys.exit(2)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    q = dev(w.q)
    tables = dev(w.block_tables)
    lens = dev(w.context_lens)
    k_new, v_new = dev(w.k_new), dev(w.v_new)
    if cache_dtype == "fp8":
        vk, vv = dev(w.k_pool), dev(w.v_pool)
        k_cache = torch.empty(vk.shape, dtype=torch.uint8, device="cuda")
        v_cache = torch.empty(vv.shape, dtype=torch.uint8, device="cuda")
        pkv.quantise_pool(vk, vv, k_cache, v_cache, k_inv_scale=w.k_inv_scale,
                          v_inv_scale=w.v_inv_scale)
        del vk, vv
    else:
        k_cache, v_cache = dev(w.k_pool), dev(w.v_pool)
    slots = dev(pkv.slots_from_tables(w.block_tables, w.context_lens - 1, s.bs))
    out = torch.empty((s.S, s.Hq, s.d), dtype=torch.float32, device="cuda")
    need = pkv.paged_decode_attn_workspace_size(s.S, s.Hq, s.Hkv, s.d, w.max_context_len, part)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda") if need else None
    # 1 GiB read between timed steps: the Infinity Cache and L2 then hold only
    # clean lines of this buffer (a write flush would leave dirty lines whose
    # write-back the next kernel pays for)
    flush = torch.ones(1 << 27, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()

    def write():
        pkv.kv_cache_write(k_new, v_new, k_cache, v_cache, slots, k_inv_scale=w.k_inv_scale,
                           v_inv_scale=w.v_inv_scale, stream=stream)

    def attend():
        pkv.paged_decode_attn(out, q, k_cache, v_cache, tables, lens,
                              max_context_len=w.max_context_len, softmax_scale=w.softmax_scale,
                              k_scale=w.k_scale, v_scale=w.v_scale, partition_size=part,
                              workspace=ws, stream=stream)

    def fused_step():
        pkv.paged_decode_step(out, q, k_new, v_new, k_cache, v_cache, tables, lens,
                              max_context_len=w.max_context_len, softmax_scale=w.softmax_scale,
                              k_scale=w.k_scale, v_scale=w.v_scale, k_inv_scale=w.k_inv_scale,
                              v_inv_scale=w.v_inv_scale, workspace=ws, stream=stream)

    plan_info = None
    if args.step == "planned":
        # step a0 on the host, before the timed region: the plan from the host
        # lengths (as the block tables are built), uploaded once
        code = {"f32": pkv.PKV_F32, "bf16": pkv.PKV_BF16, "fp8": pkv.PKV_FP8_E4M3}[cache_dtype]
        t0 = time.perf_counter()
        plan = pkv.DecodePlan(w.context_lens, Hq=s.Hq, Hkv=s.Hkv, d=s.d, bs=s.bs, cache_dtype_code=code,
                              max_context_len=w.max_context_len, block_tables=w.block_tables)
        torch.cuda.synchronize()
        t_plan = time.perf_counter() - t0
        t0 = time.perf_counter()
        pkv.build_paged_decode_plan(w.context_lens, s.Hkv, s.d, code, w.max_context_len, plan.n_workers)
        t_build = time.perf_counter() - t0
        plan_info = {"host_build_ms": round(1e3 * t_build, 3), "build_and_upload_ms": round(1e3 * t_plan, 3),
                     "bytes": int(plan.host.nbytes), "waves": int(plan.n_workers),
                     "shared_blocks": plan.shared_blocks,
                     "note": "built on the host from the host lengths before the timed region (step a0, as the "
                             "block tables), and marked from the host tables when sequences share blocks "
                             "(cacheable K/V loads); one plan serves every layer of a step"}

        def planned_step():
            plan(out, q, k_cache, v_cache, tables, lens, softmax_scale=w.softmax_scale, k_new=k_new,
                 v_new=v_new, k_scale=w.k_scale, v_scale=w.v_scale, k_inv_scale=w.k_inv_scale,
                 v_inv_scale=w.v_inv_scale, stream=stream)

    one = planned_step if args.step == "planned" else fused_step
    for _ in range(args.warmup):
        if one_call:
            one()
        else:
            write()
            attend()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    with _no_gc():
        wall0 = time.perf_counter()
        for k in range(args.steps):
            if not args.no_flush:
                flush.max()
            a, b, c = ev[k]
            a.record(stream)
            if one_call:
                one()
            else:
                write()
                b.record(stream)
                attend()
            c.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0

    # The planned call's own kernels, timed apart: a second timed loop whose
    # calls record an event between the attention kernel and the merge kernel
    # (kept out of the loop above, so the step's time has no extra event).
    split_ms = None
    if args.step == "planned":
        ev2 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for _, mid, _ in ev2:
            mid.record(stream)                 # creates the event the call records
        torch.cuda.synchronize()
        with _no_gc():
            for a, mid, c in ev2:
                if not args.no_flush:
                    flush.max()
                a.record(stream)
                plan(out, q, k_cache, v_cache, tables, lens, softmax_scale=w.softmax_scale, k_new=k_new,
                     v_new=v_new, k_scale=w.k_scale, v_scale=w.v_scale, k_inv_scale=w.k_inv_scale,
                     v_inv_scale=w.v_inv_scale, stream=stream, attn_done_event=mid)
                c.record(stream)
            torch.cuda.synchronize()
        split_ms = ([a.elapsed_time(mid) for a, mid, c in ev2], [mid.elapsed_time(c) for a, mid, c in ev2])

    step_ms = [a.elapsed_time(c) for a, b, c in ev]
    if one_call:                               # one call does both
        write_ms, attn_ms = None, step_ms
    else:
        write_ms = [a.elapsed_time(b) for a, b, c in ev]
        attn_ms = [b.elapsed_time(c) for a, b, c in ev]
    step_mean = statistics.mean(step_ms)
    step_med = statistics.median(step_ms)
    attn_mean = statistics.mean(attn_ms)

    attn_bytes, write_bytes, logical_kv, unique_tokens = algorithmic_bytes(w, cache_dtype)
    step_bytes = attn_bytes + write_bytes
    value = step_bytes / (step_med * 1e-3) / 1e9
    attn_gbs = attn_bytes / (attn_mean * 1e-3) / 1e9
    if args.step == "planned":
        kernel_name = ("paged_attn_plan_kernel (the planned attention kernel with the write fused in), mean "
                       "event time from the call's start to the event the call records after it")
        split = "balanced: equal cost-weighted chunk ranges, one per wave, listed in a host-built plan"
        attn_gbs = step_bytes / (statistics.mean(split_ms[0]) * 1e-3) / 1e9   # the kernel moves the write's bytes too
    elif one_call:
        kernel_name = ("paged_decode_step call (stream kernel with the write fused in + merge kernel), "
                       "mean event time")
        split = "balanced: equal cost-weighted chunk ranges, one per wave"
        attn_gbs = step_bytes / (step_mean * 1e-3) / 1e9     # the call moves the write's bytes too
    elif part == pkv.PKV_PARTITION_BALANCED:
        kernel_name = "paged_decode_attn call (balanced stream kernel + merge kernel)"
        split = "balanced: equal cost-weighted chunk ranges, one per wave"
    else:
        n_part = -(-w.max_context_len // part) if part else 1
        kernel_name = "paged_decode_attn call (partition kernel" + (" + merge kernel)" if n_part > 1 else ")")
        split = f"partitions of {part} tokens" if part else "one pass per (sequence, kv head)"

    result = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) and seq-steps/sec at 1 GPU",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_med, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 KV, bf16 q"}[cache_dtype],
        "data": "synthetic (seeded; N(0,1) values, lognormal lengths)",
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(s.S / (step_med * 1e-3), 1),
        "config": {
            "workload": f"{s.name}: {s.description}",
            "sequences": s.S, "q_heads": s.Hq, "kv_heads": s.Hkv, "head_dim": s.d,
            "block_size": s.bs, "kv_dtype": cache_dtype, "partition_size": part, "split": split,
            "step": {"planned": "one planned call (write + attention)", "fused": "one fused call (write + attention)",
                     "split": "write call, then attention call"}[args.step],
            "context_tokens": int(w.context_lens.sum()), "unique_tokens": int(unique_tokens),
            "max_context_len": w.max_context_len, "pool_blocks": w.P,
            "cache_flush_between_steps": not args.no_flush,
        },
        "timing": {
            "value_from": "median step time",
            "step_ms_mean": round(step_mean, 5), "step_ms_median": round(step_med, 5),
            "step_ms_min": round(min(step_ms), 5),
            "write_ms_mean": None if write_ms is None else round(statistics.mean(write_ms), 5),
            "attn_ms_mean": round(attn_mean, 5), "attn_ms_median": round(statistics.median(attn_ms), 5),
            "attn_ms_min": round(min(attn_ms), 5),
            "wall_s_timed_region": round(wall, 4),
        },
        "kernels": None if split_ms is None else {
            "note": "a second timed loop of the planned call with an event recorded between its two kernels",
            "attention_ms_mean": round(statistics.mean(split_ms[0]), 5),
            "attention_ms_median": round(statistics.median(split_ms[0]), 5),
            "merge_ms_mean": round(statistics.mean(split_ms[1]), 5),
            "merge_ms_median": round(statistics.median(split_ms[1]), 5),
        },
        "bytes": {"attn_algorithmic": attn_bytes, "write_algorithmic": write_bytes,
                  "kv_logical": logical_kv},
        "roofline": {
            "kernel": kernel_name,
            "bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(s.name, cache_dtype, s.bs, part, args.step),
            "call_achieved": round(step_bytes / (step_mean * 1e-3) / 1e9, 1),
        },
        "device": torch.cuda.get_device_name(0),
    }
    if plan_info is not None:
        result["plan"] = plan_info
    if not args.no_companions:
        comp = companions(args, torch, pkv, w, flush, stream, (q, k_new, v_new, k_cache, v_cache, tables, lens, out),
                          step_bytes, attn_bytes, plan if args.step == "planned" else None)
        comp["step_over_read_ceiling"] = round(value / comp["read_ceiling"]["gbs"], 4)
        if "gather_ceiling" in comp:
            comp["gather_ms_over_step_ms"] = round(comp["gather_ceiling"]["ms_median"] / step_med, 4)
        result["companions"] = comp
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, cache_dtype, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
