"""Python names for the C ABI of libpkv.so (argument marshalling only).

Device functions take torch tensors that already live on the GPU (their data
pointers and torch's current HIP stream are passed through); every step of
the computation runs in the library's kernels. Host functions take numpy
arrays. Errors from the library raise PkvError with its message.
"""

import ctypes

import numpy as np

from ._lib import (lib, check, PkvError, PkvStats, PKV_F32, PKV_BF16, PKV_FP8_E4M3, PKV_OK,
                   PKV_PARTITION_BALANCED,
                   PKV_E_NO_BLOCKS, P_i32, P_i64, P_f64, c_vp, c_i64, c_i32, c_f64)

__all__ = [
    "kv_cache_write", "copy_blocks", "paged_decode_attn", "paged_decode_step", "paged_decode_step_noalloc",
    "paged_decode_plan_workers", "build_paged_decode_plan", "paged_decode_step_planned", "DecodePlan",
    "build_paged_window_plan", "paged_multi_query_attn_planned", "WindowPlan", "plan_mark_shared_blocks",
    "paged_decode_attn_workspace_size",
    "paged_decode_attn_workspace", "paged_multi_query_attn", "paged_multi_query_attn_workspace",
    "Allocator",
    "slots_from_tables", "waste_stats", "block_hashes", "last_error", "version", "quantise_pool",
    "PkvError", "NoBlocks", "PKV_PARTITION_BALANCED",
]


class NoBlocks(PkvError):
    """The pool has fewer free blocks than the append needs (nothing changed)."""


def last_error():
    return lib().pkv_last_error().decode()


def version():
    return lib().pkv_version().decode()


# ------------------------------------------------------------------ device ops
def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PKV_FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _event(ev):
    if ev is None:
        return None
    handle = int(ev.cuda_event)
    if handle == 0:
        raise ValueError("attn_done_event: record the event once first, so that it exists")
    return ctypes.c_void_p(handle)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def v_shape_ok(v_cache, P, Hkv, d, bs):
    """The V pool holds one tile per (block, kv head) in sub-tiles of
    vs = min(bs, 16) tokens, each [d][vs]: shape [P][Hkv][bs/vs][d][vs], or
    [P][Hkv][d][bs] when bs <= 16 (the same memory)."""
    shp = tuple(v_cache.shape)
    vs = min(bs, 16)
    if shp == (P, Hkv, bs // vs, d, vs):
        return True
    return bs <= 16 and shp == (P, Hkv, d, bs)


def _pools(fn, k_cache, v_cache):
    """(P, Hkv, bs, d) of a K pool [P][Hkv][bs][d] and the V pool that goes with
    it: same dtype, same device, V in the layout v_shape_ok describes."""
    if k_cache.dim() != 4:
        raise ValueError(f"{fn}: k_cache must be [P][Hkv][bs][d]")
    P, Hkv, bs, d = k_cache.shape
    if v_cache.dtype != k_cache.dtype:
        raise ValueError(f"{fn}: v_cache dtype {v_cache.dtype} differs from k_cache dtype {k_cache.dtype}")
    if not v_shape_ok(v_cache, P, Hkv, d, bs):
        raise ValueError(f"{fn}: v_cache shape {tuple(v_cache.shape)} does not match k_cache {tuple(k_cache.shape)}")
    _dtype_code(k_cache)
    return P, Hkv, bs, d


def _src_dtype_ok(fn, name, t, k_cache):
    """New K/V (and q) elements: float32 for a float32 cache, bfloat16 for a
    bfloat16 or fp8 cache."""
    import torch
    want = torch.float32 if k_cache.dtype == torch.float32 else torch.bfloat16
    if t.dtype != want:
        raise ValueError(f"{fn}: {name} dtype {t.dtype} does not go with a {k_cache.dtype} cache (needs {want})")


def _one_device(fn, *tensors):
    devs = {t.device for t in tensors if t is not None}
    if len(devs) > 1:
        raise ValueError(f"{fn}: tensors on several devices {sorted(str(x) for x in devs)}")


def kv_cache_write(k_new, v_new, k_cache, v_cache, slot_mapping, *, k_inv_scale=1.0,
                   v_inv_scale=1.0, stream=None):
    """pkv_kv_cache_write. k_new/v_new [T][Hkv][d]; k_cache [P][Hkv][bs][d];
    v_cache as v_shape_ok describes; slot_mapping int64 [T]."""
    import torch
    P, Hkv, bs, d = _pools("kv_cache_write", k_cache, v_cache)
    if k_new.dim() != 3 or tuple(k_new.shape[1:]) != (Hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("kv_cache_write: k_new and v_new must both be [T][Hkv][d]")
    T = k_new.shape[0]
    _src_dtype_ok("kv_cache_write", "k_new", k_new, k_cache)
    _src_dtype_ok("kv_cache_write", "v_new", v_new, k_cache)
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("kv_cache_write: slot_mapping must be int64 [T]")
    _one_device("kv_cache_write", k_new, v_new, k_cache, v_cache, slot_mapping)
    check(lib().pkv_kv_cache_write(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(slot_mapping, "slot_mapping"), T, Hkv, d, bs, P,
        _dtype_code(k_new), _dtype_code(k_cache), float(k_inv_scale), float(v_inv_scale),
        _stream(stream)))


def copy_blocks(k_cache, v_cache, src, dst, *, stream=None):
    """pkv_copy_blocks: block dst[k] of both pools becomes a copy of block
    src[k]. src, dst: int32 device tensors [n]; the dst ids must be distinct
    and none of them a src of the same call."""
    import torch
    P, Hkv, bs, d = _pools("copy_blocks", k_cache, v_cache)
    if src.dtype != torch.int32 or dst.dtype != torch.int32 or src.shape != dst.shape or src.dim() != 1:
        raise ValueError("copy_blocks: src and dst must be int32 [n]")
    _one_device("copy_blocks", k_cache, v_cache, src, dst)
    n = src.shape[0]
    if n == 0:
        return
    check(lib().pkv_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(src, "src"),
                                _dev(dst, "dst"), n, P, Hkv, d, bs, _dtype_code(k_cache),
                                _stream(stream)))


def stream_read(src, sink, *, nbytes=None, blocks=512, unroll=4, stream=None):
    """pkv_stream_read: read the first nbytes (default all) of the device tensor
    src once with the cache-streaming loads; sink: an int32 device tensor of at
    least one element (a thread writes it only when the xor of its words is a
    fixed value)."""
    import torch
    if not src.is_cuda or not sink.is_cuda or sink.numel() < 1 or sink.element_size() != 4:
        raise ValueError("stream_read: src and sink must be device tensors, sink 32-bit with one element")
    _one_device("stream_read", src, sink)
    total = src.numel() * src.element_size()
    n = total if nbytes is None else int(nbytes)
    if n < 0 or n > total:
        raise ValueError(f"stream_read: nbytes={n} outside [0, {total}]")
    check(lib().pkv_stream_read(_dev(src, "src"), n, int(blocks), int(unroll), _dev(sink, "sink"),
                                _stream(stream)))


def paged_decode_attn_workspace_size(S, Hq, Hkv, d, max_context_len, partition_size):
    return int(lib().pkv_paged_decode_attn_workspace_size(S, Hq, Hkv, d, max_context_len,
                                                          partition_size))


def paged_decode_attn_workspace(S, Hq, Hkv, d, max_context_len, partition_size, device="cuda"):
    """A uint8 device tensor of the size pkv_paged_decode_attn needs (None when
    it needs none); reusable by any later call with the same or smaller needs."""
    import torch
    need = paged_decode_attn_workspace_size(S, Hq, Hkv, d, max_context_len, partition_size)
    return torch.empty(need, dtype=torch.uint8, device=device) if need else None


def _attn_args(fn, out, q, k_cache, block_tables, context_lens, d, n_q=None):
    """Check q ([S][Hq][d], or [S][n_q][Hq][d] when n_q is given), the float32
    output of the same shape, int32 tables [S][max_blocks] and lengths [S];
    returns (S, Hq)."""
    import torch
    want_dim = 3 if n_q is None else 4
    if q.dim() != want_dim or q.shape[-1] != d:
        raise ValueError(f"{fn}: q must be {'[S][Hq][d]' if n_q is None else '[S][n_q][Hq][d]'} with d={d}")
    S, Hq = q.shape[0], q.shape[-2]
    if tuple(out.shape) != tuple(q.shape) or out.dtype != torch.float32:
        raise ValueError(f"{fn}: out must be float32 of q's shape {tuple(q.shape)}")
    _src_dtype_ok(fn, "q", q, k_cache)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError(f"{fn}: tables and lengths must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError(f"{fn}: tables/lengths shape mismatch")
    return S, Hq


def paged_decode_attn(out, q, k_cache, v_cache, block_tables, context_lens, *, max_context_len,
                      softmax_scale, k_scale=1.0, v_scale=1.0, partition_size=PKV_PARTITION_BALANCED,
                      workspace=None, stream=None):
    """pkv_paged_decode_attn. out float32 [S][Hq][d]; q [S][Hq][d]; tables int32
    [S][max_blocks]; context_lens int32 [S]; workspace a uint8 device tensor of at
    least paged_decode_attn_workspace_size(...) bytes (paged_decode_attn_workspace
    makes one); None allocates one for this call when one is needed (pass one in
    loops that must not allocate);
    partition_size PKV_PARTITION_BALANCED (default: equal cost-weighted chunk
    ranges, one per wave), 0 (one pass per sequence and kv head) or a multiple
    of 32 (fixed partitions of that many tokens)."""
    P, Hkv, bs, d = _pools("paged_decode_attn", k_cache, v_cache)
    S, Hq = _attn_args("paged_decode_attn", out, q, k_cache, block_tables, context_lens, d)
    _one_device("paged_decode_attn", out, q, k_cache, v_cache, block_tables, context_lens, workspace)
    if workspace is None:                     # convenience: a fresh zeroed one for this call
        workspace = paged_decode_attn_workspace(S, Hq, Hkv, d, int(max_context_len),
                                                int(partition_size), device=q.device)
    ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    check(lib().pkv_paged_decode_attn(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"),
        S, Hq, Hkv, d, bs, P, block_tables.shape[1], int(max_context_len),
        float(softmax_scale), float(k_scale), float(v_scale), _dtype_code(q),
        _dtype_code(k_cache), int(partition_size), ws_ptr, ws_bytes, _stream(stream)))


def paged_decode_step(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, *,
                      max_context_len, softmax_scale, k_scale=1.0, v_scale=1.0, k_inv_scale=1.0,
                      v_inv_scale=1.0, workspace=None, stream=None):
    """pkv_paged_decode_step: write each sequence's new token (k_new, v_new
    [S][Hkv][d]) at position L_i - 1 and attend, in one launch. Same result as
    kv_cache_write followed by paged_decode_attn with the balanced split."""
    P, Hkv, bs, d = _pools("paged_decode_step", k_cache, v_cache)
    S, Hq = _attn_args("paged_decode_step", out, q, k_cache, block_tables, context_lens, d)
    if tuple(k_new.shape) != (S, Hkv, d) or tuple(v_new.shape) != (S, Hkv, d):
        raise ValueError("paged_decode_step: k_new/v_new must be [S][Hkv][d]")
    _src_dtype_ok("paged_decode_step", "k_new", k_new, k_cache)
    _src_dtype_ok("paged_decode_step", "v_new", v_new, k_cache)
    _one_device("paged_decode_step", out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                workspace)
    if workspace is None:
        workspace = paged_decode_attn_workspace(S, Hq, Hkv, d, int(max_context_len),
                                                PKV_PARTITION_BALANCED, device=q.device)
    check(lib().pkv_paged_decode_step(
        _dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
        _dev(context_lens, "context_lens"), S, Hq, Hkv, d, bs, P, block_tables.shape[1],
        int(max_context_len), float(softmax_scale), float(k_scale), float(v_scale),
        float(k_inv_scale), float(v_inv_scale), _dtype_code(q), _dtype_code(k_cache),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))


def paged_decode_step_noalloc(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, *,
                              max_context_len, softmax_scale, k_scale=1.0, v_scale=1.0, k_inv_scale=1.0,
                              v_inv_scale=1.0, stream=None):
    """pkv_paged_decode_step_noalloc: paged_decode_step with no workspace; its
    records live in the library's per-GPU scratch array (calls on one GPU must
    not overlap). Raises PkvError (PKV_E_WORKSPACE) for a call that needs more
    than pkv_paged_decode_step_scratch_bytes()."""
    P, Hkv, bs, d = _pools("paged_decode_step_noalloc", k_cache, v_cache)
    S, Hq = _attn_args("paged_decode_step_noalloc", out, q, k_cache, block_tables, context_lens, d)
    if tuple(k_new.shape) != (S, Hkv, d) or tuple(v_new.shape) != (S, Hkv, d):
        raise ValueError("paged_decode_step_noalloc: k_new/v_new must be [S][Hkv][d]")
    _src_dtype_ok("paged_decode_step_noalloc", "k_new", k_new, k_cache)
    _src_dtype_ok("paged_decode_step_noalloc", "v_new", v_new, k_cache)
    _one_device("paged_decode_step_noalloc", out, q, k_new, v_new, k_cache, v_cache, block_tables,
                context_lens)
    check(lib().pkv_paged_decode_step_noalloc(
        _dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
        _dev(context_lens, "context_lens"), S, Hq, Hkv, d, bs, P, block_tables.shape[1],
        int(max_context_len), float(softmax_scale), float(k_scale), float(v_scale),
        float(k_inv_scale), float(v_inv_scale), _dtype_code(q), _dtype_code(k_cache), _stream(stream)))


def paged_decode_plan_workers(d, bs, cache_dtype_code):
    """pkv_paged_decode_plan_workers: waves of the planned kernel's grid on the
    current device (the plan is built for this many)."""
    n = int(lib().pkv_paged_decode_plan_workers(d, bs, cache_dtype_code))
    if n <= 0:
        raise PkvError(PKV_E_INVALID, f"paged_decode_plan_workers: no grid for d={d} bs={bs}")
    return n


def build_paged_decode_plan(context_lens, Hkv, d, cache_dtype_code, max_context_len, n_workers):
    """pkv_build_paged_decode_plan on host lengths: the plan as an int32 numpy array."""
    lens = _i32(context_lens)
    S = len(lens)
    need = ctypes.c_size_t(0)
    st = lib().pkv_build_paged_decode_plan(_ptr(lens, P_i32), S, Hkv, d, cache_dtype_code, int(max_context_len),
                                           int(n_workers), None, 0, ctypes.byref(need))
    if st not in (PKV_OK, 2):                  # 2: PKV_E_WORKSPACE, the size query
        check(st)
    plan = np.zeros(need.value // 4, dtype=np.int32)
    check(lib().pkv_build_paged_decode_plan(_ptr(lens, P_i32), S, Hkv, d, cache_dtype_code, int(max_context_len),
                                            int(n_workers), plan.ctypes.data_as(c_vp), plan.nbytes,
                                            ctypes.byref(need)))
    return plan


def plan_mark_shared_blocks(plan, block_tables, context_lens, bs):
    """pkv_plan_mark_shared_blocks on a host plan (int32 numpy, changed in
    place) from the host tables [S][max_blocks] and lengths [S]; returns
    whether the batch shares blocks."""
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = _i32(context_lens)
    if tables.ndim != 2 or tables.shape[0] != len(lens):
        raise ValueError("plan_mark_shared_blocks: tables must be [S][max_blocks] with S = len(context_lens)")
    shared = ctypes.c_int32(0)
    check(lib().pkv_plan_mark_shared_blocks(plan.ctypes.data_as(c_vp), plan.nbytes, _ptr(tables, P_i32),
                                            _ptr(lens, P_i32), len(lens), tables.shape[1], int(bs),
                                            ctypes.byref(shared)))
    return bool(shared.value)


def build_paged_window_plan(context_lens, n_q, Hq, Hkv, d, cache_dtype_code, max_context_len, n_workers):
    """pkv_build_paged_window_plan on host lengths: the plan as an int32 numpy array."""
    lens = _i32(context_lens)
    S = len(lens)
    need = ctypes.c_size_t(0)
    st = lib().pkv_build_paged_window_plan(_ptr(lens, P_i32), S, int(n_q), Hq, Hkv, d, cache_dtype_code,
                                           int(max_context_len), int(n_workers), None, 0, ctypes.byref(need))
    if st not in (PKV_OK, 2):                  # 2: PKV_E_WORKSPACE, the size query
        check(st)
    plan = np.zeros(need.value // 4, dtype=np.int32)
    check(lib().pkv_build_paged_window_plan(_ptr(lens, P_i32), S, int(n_q), Hq, Hkv, d, cache_dtype_code,
                                            int(max_context_len), int(n_workers), plan.ctypes.data_as(c_vp),
                                            plan.nbytes, ctypes.byref(need)))
    return plan


def paged_decode_step_planned(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, *,
                              max_context_len, softmax_scale, plan_host, plan_dev, workspace, k_scale=1.0,
                              v_scale=1.0, k_inv_scale=1.0, v_inv_scale=1.0, stream=None, attn_done_event=None):
    """pkv_paged_decode_step_planned. plan_host: the int32 numpy plan; plan_dev:
    its device copy (int32 tensor); k_new/v_new None for attention alone;
    attn_done_event: None, or a torch.cuda.Event (already recorded once, so
    that it exists) that the call records between its two kernels."""
    import torch
    P, Hkv, bs, d = _pools("paged_decode_step_planned", k_cache, v_cache)
    S, Hq = _attn_args("paged_decode_step_planned", out, q, k_cache, block_tables, context_lens, d)
    if (k_new is None) != (v_new is None):
        raise ValueError("paged_decode_step_planned: give both k_new and v_new, or neither")
    if k_new is not None:
        if tuple(k_new.shape) != (S, Hkv, d) or tuple(v_new.shape) != (S, Hkv, d):
            raise ValueError("paged_decode_step_planned: k_new/v_new must be [S][Hkv][d]")
        _src_dtype_ok("paged_decode_step_planned", "k_new", k_new, k_cache)
        _src_dtype_ok("paged_decode_step_planned", "v_new", v_new, k_cache)
    plan_host = np.ascontiguousarray(plan_host, dtype=np.int32)
    if plan_dev.dtype != torch.int32 or plan_dev.numel() != plan_host.size:
        raise ValueError("paged_decode_step_planned: plan_dev must be the int32 device copy of plan_host")
    _one_device("paged_decode_step_planned", out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                plan_dev, workspace)
    check(lib().pkv_paged_decode_step_planned(
        _dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new") if k_new is not None else None,
        _dev(v_new, "v_new") if v_new is not None else None, _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"), S, Hq, Hkv, d, bs, P,
        block_tables.shape[1], int(max_context_len), float(softmax_scale), float(k_scale), float(v_scale),
        float(k_inv_scale), float(v_inv_scale), _dtype_code(q), _dtype_code(k_cache),
        plan_host.ctypes.data_as(c_vp), _dev(plan_dev, "plan_dev"), plan_host.nbytes,
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream),
        _event(attn_done_event)))


def paged_multi_query_attn_planned(out, q, k_cache, v_cache, block_tables, context_lens, *, max_context_len,
                                   softmax_scale, plan_host, plan_dev, workspace, k_scale=1.0, v_scale=1.0,
                                   stream=None):
    """pkv_paged_multi_query_attn_planned: pkv_paged_multi_query_attn with a
    window plan (build_paged_window_plan). out float32 [S][n_q][Hq][d]; q
    [S][n_q][Hq][d]; plan_host the int32 numpy plan, plan_dev its int32 device
    copy; workspace of pkv_paged_window_plan_workspace_size bytes."""
    import torch
    P, Hkv, bs, d = _pools("paged_multi_query_attn_planned", k_cache, v_cache)
    S, Hq = _attn_args("paged_multi_query_attn_planned", out, q, k_cache, block_tables, context_lens, d, n_q=True)
    n_q = q.shape[1]
    plan_host = np.ascontiguousarray(plan_host, dtype=np.int32)
    if plan_dev.dtype != torch.int32 or plan_dev.numel() != plan_host.size:
        raise ValueError("paged_multi_query_attn_planned: plan_dev must be the int32 device copy of plan_host")
    _one_device("paged_multi_query_attn_planned", out, q, k_cache, v_cache, block_tables, context_lens, plan_dev,
                workspace)
    check(lib().pkv_paged_multi_query_attn_planned(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"), S, n_q, Hq, Hkv, d, bs, P,
        block_tables.shape[1], int(max_context_len), float(softmax_scale), float(k_scale), float(v_scale),
        _dtype_code(q), _dtype_code(k_cache), plan_host.ctypes.data_as(c_vp), _dev(plan_dev, "plan_dev"),
        plan_host.nbytes, _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def paged_gather_read(k_cache, v_cache, block_tables, sink, *, max_context_len, plan_host, plan_dev, stream=None):
    """pkv_paged_gather_read: the plan's K/V chunks read through the tables, no
    arithmetic (the step's own read pattern, for timing). sink: an int32
    device tensor of at least one element."""
    import torch
    P, Hkv, bs, d = _pools("paged_gather_read", k_cache, v_cache)
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2:
        raise ValueError("paged_gather_read: block_tables must be int32 [S][max_blocks]")
    if sink.dtype != torch.int32 or sink.numel() < 1:
        raise ValueError("paged_gather_read: sink must be an int32 tensor of at least one element")
    _one_device("paged_gather_read", k_cache, v_cache, block_tables, sink, plan_dev)
    plan_host = np.ascontiguousarray(plan_host, dtype=np.int32)
    if plan_dev.dtype != torch.int32 or plan_dev.numel() != plan_host.size:
        raise ValueError("paged_gather_read: plan_dev must be the int32 device copy of plan_host")
    S = block_tables.shape[0]
    check(lib().pkv_paged_gather_read(
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"), S, Hkv, d, bs, P,
        block_tables.shape[1], int(max_context_len), _dtype_code(k_cache), plan_host.ctypes.data_as(c_vp),
        _dev(plan_dev, "plan_dev"), plan_host.nbytes, _dev(sink, "sink"), _stream(stream)))


class DecodePlan:
    """A decode step's work plan: built on the host from the host lengths (as
    the block tables are), uploaded once, with the workspace it needs. Holds
    while the lengths do: the next step (one more token per sequence) needs a
    new plan. __call__ runs pkv_paged_decode_step_planned."""

    def __init__(self, context_lens, *, Hq, Hkv, d, bs, cache_dtype_code, max_context_len, block_tables=None,
                 device="cuda"):
        """block_tables: the host copy of the tables (optional); when given, the
        plan records whether the batch shares blocks (plan_mark_shared_blocks),
        which selects cacheable K/V loads."""
        import torch
        self.n_workers = paged_decode_plan_workers(d, bs, cache_dtype_code)
        self.max_context_len = int(max_context_len)
        self.host = build_paged_decode_plan(context_lens, Hkv, d, cache_dtype_code, self.max_context_len,
                                            self.n_workers)
        self.shared_blocks = (plan_mark_shared_blocks(self.host, block_tables, context_lens, bs)
                              if block_tables is not None else False)
        self.dev = torch.from_numpy(self.host).to(device)
        need = int(lib().pkv_paged_decode_plan_workspace_size(self.n_workers, Hq, Hkv, d))
        self.workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)

    def gather(self, k_cache, v_cache, block_tables, sink, *, stream=None):
        """pkv_paged_gather_read of this plan's chunks (no arithmetic)."""
        paged_gather_read(k_cache, v_cache, block_tables, sink, max_context_len=self.max_context_len,
                          plan_host=self.host, plan_dev=self.dev, stream=stream)

    def __call__(self, out, q, k_cache, v_cache, block_tables, context_lens, *, softmax_scale, k_new=None,
                 v_new=None, k_scale=1.0, v_scale=1.0, k_inv_scale=1.0, v_inv_scale=1.0, stream=None,
                 attn_done_event=None):
        paged_decode_step_planned(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                                  max_context_len=self.max_context_len, softmax_scale=softmax_scale,
                                  plan_host=self.host, plan_dev=self.dev, workspace=self.workspace,
                                  k_scale=k_scale, v_scale=v_scale, k_inv_scale=k_inv_scale,
                                  v_inv_scale=v_inv_scale, stream=stream, attn_done_event=attn_done_event)


class WindowPlan:
    """A query window's work plan (build_paged_window_plan), uploaded once, with
    the workspace it needs; __call__ runs pkv_paged_multi_query_attn_planned."""

    def __init__(self, context_lens, *, n_q, Hq, Hkv, d, bs, cache_dtype_code, max_context_len, device="cuda"):
        import torch
        self.n_q = int(n_q)
        self.n_workers = paged_decode_plan_workers(d, bs, cache_dtype_code)
        self.max_context_len = int(max_context_len)
        self.host = build_paged_window_plan(context_lens, self.n_q, Hq, Hkv, d, cache_dtype_code,
                                            self.max_context_len, self.n_workers)
        self.dev = torch.from_numpy(self.host).to(device)
        need = int(lib().pkv_paged_window_plan_workspace_size(self.n_workers, self.n_q, Hq, Hkv, d))
        if need == 0:
            raise ValueError("WindowPlan: invalid sizes")
        self.workspace = torch.empty(need, dtype=torch.uint8, device=device)

    def __call__(self, out, q, k_cache, v_cache, block_tables, context_lens, *, softmax_scale, k_scale=1.0,
                 v_scale=1.0, stream=None):
        paged_multi_query_attn_planned(out, q, k_cache, v_cache, block_tables, context_lens,
                                       max_context_len=self.max_context_len, softmax_scale=softmax_scale,
                                       plan_host=self.host, plan_dev=self.dev, workspace=self.workspace,
                                       k_scale=k_scale, v_scale=v_scale, stream=stream)


def paged_multi_query_attn_workspace(S, n_q, Hq, Hkv, d, device="cuda"):
    """A uint8 device tensor of the size pkv_paged_multi_query_attn needs."""
    import torch
    need = int(lib().pkv_paged_multi_query_attn_workspace_size(S, n_q, Hq, Hkv, d))
    if need == 0:
        raise ValueError("paged_multi_query_attn: invalid sizes")
    return torch.empty(need, dtype=torch.uint8, device=device)


def paged_multi_query_attn(out, q, k_cache, v_cache, block_tables, context_lens, *, max_context_len,
                           softmax_scale, k_scale=1.0, v_scale=1.0, workspace=None, stream=None):
    """pkv_paged_multi_query_attn. out float32 [S][n_q][Hq][d]; q [S][n_q][Hq][d]:
    query j of sequence i sits at position L_i - n_q + j and sees the tokens up to
    it (causal inside the window). workspace as from paged_multi_query_attn_workspace
    (None allocates one for this call)."""
    P, Hkv, bs, d = _pools("paged_multi_query_attn", k_cache, v_cache)
    S, Hq = _attn_args("paged_multi_query_attn", out, q, k_cache, block_tables, context_lens, d, n_q=True)
    n_q = q.shape[1]
    _one_device("paged_multi_query_attn", out, q, k_cache, v_cache, block_tables, context_lens, workspace)
    if workspace is None:
        workspace = paged_multi_query_attn_workspace(S, n_q, Hq, Hkv, d, device=q.device)
    check(lib().pkv_paged_multi_query_attn(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"),
        S, n_q, Hq, Hkv, d, bs, P, block_tables.shape[1], int(max_context_len),
        float(softmax_scale), float(k_scale), float(v_scale), _dtype_code(q), _dtype_code(k_cache),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream)))


def paged_decode_attn_lse(out, lse, q, k_cache, v_cache, block_tables, context_lens, *,
                          max_context_len, softmax_scale, k_scale=1.0, v_scale=1.0, workspace=None,
                          stream=None):
    """pkv_paged_decode_attn_lse: balanced decode attention that also writes
    lse float32 [S][Hq], the base-2 log of each row's softmax sum."""
    import torch
    P, Hkv, bs, d = _pools("paged_decode_attn_lse", k_cache, v_cache)
    S, Hq = _attn_args("paged_decode_attn_lse", out, q, k_cache, block_tables, context_lens, d)
    if tuple(lse.shape) != (S, Hq) or lse.dtype != torch.float32:
        raise ValueError("paged_decode_attn_lse: lse must be float32 [S][Hq]")
    _one_device("paged_decode_attn_lse", out, lse, q, k_cache, v_cache, block_tables, context_lens, workspace)
    if workspace is None:
        workspace = paged_decode_attn_workspace(S, Hq, Hkv, d, int(max_context_len),
                                                PKV_PARTITION_BALANCED, device=q.device)
    check(lib().pkv_paged_decode_attn_lse(
        _dev(out, "out"), _dev(lse, "lse"), _dev(q, "q"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"),
        S, Hq, Hkv, d, bs, P, block_tables.shape[1], int(max_context_len), float(softmax_scale),
        float(k_scale), float(v_scale), _dtype_code(q), _dtype_code(k_cache), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def paged_shared_prefix_attn(out, lse, q, k_cache, v_cache, prefix_tables, prefix_lens, *,
                             max_prefix_len, softmax_scale, k_scale=1.0, v_scale=1.0, workspace=None,
                             stream=None):
    """pkv_paged_shared_prefix_attn: q [n_groups][M][Hq][d]; every query of a
    group attends to all of the group's prefix tokens. out float32
    [n_groups][M][Hq][d], lse float32 [n_groups][M][Hq]."""
    import torch
    P, Hkv, bs, d = _pools("paged_shared_prefix_attn", k_cache, v_cache)
    n_groups, Hq = _attn_args("paged_shared_prefix_attn", out, q, k_cache, prefix_tables, prefix_lens, d,
                              n_q=True)
    M = q.shape[1]
    if tuple(lse.shape) != (n_groups, M, Hq) or lse.dtype != torch.float32:
        raise ValueError("paged_shared_prefix_attn: lse must be float32 [n_groups][M][Hq]")
    _one_device("paged_shared_prefix_attn", out, lse, q, k_cache, v_cache, prefix_tables, prefix_lens,
                workspace)
    if workspace is None:
        workspace = paged_multi_query_attn_workspace(n_groups, M, Hq, Hkv, d, device=q.device)
    check(lib().pkv_paged_shared_prefix_attn(
        _dev(out, "out"), _dev(lse, "lse"), _dev(q, "q"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(prefix_tables, "prefix_tables"), _dev(prefix_lens, "prefix_lens"),
        n_groups, M, Hq, Hkv, d, bs, P, prefix_tables.shape[1], int(max_prefix_len), float(softmax_scale),
        float(k_scale), float(v_scale), _dtype_code(q), _dtype_code(k_cache), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def merge_attn_states(out, a, lse_a, b, lse_b, *, lse_out=None, stream=None):
    """pkv_merge_attn_states over rows of d floats: a, b, out float32 [..., d];
    lse_a, lse_b (and lse_out) float32 with one value per row."""
    import torch
    d = a.shape[-1]
    rows = a.numel() // d
    for t, name in ((out, "out"), (a, "a"), (b, "b")):
        if t.dtype != torch.float32 or t.numel() != rows * d:
            raise ValueError(f"merge_attn_states: {name} must be float32 with {rows} rows of {d}")
    for t, name in ((lse_a, "lse_a"), (lse_b, "lse_b")) + (((lse_out, "lse_out"),) if lse_out is not None else ()):
        if t.dtype != torch.float32 or t.numel() != rows:
            raise ValueError(f"merge_attn_states: {name} must be float32 with {rows} values")
    check(lib().pkv_merge_attn_states(
        _dev(out, "out"), _dev(lse_out, "lse_out") if lse_out is not None else None, _dev(a, "a"),
        _dev(lse_a, "lse_a"), _dev(b, "b"), _dev(lse_b, "lse_b"), rows, d, _stream(stream)))


def shared_prefix_plan(block_tables, context_lens, group_size, bs):
    """pkv_shared_prefix_plan (host): for groups of group_size consecutive
    sequences (beams, parallel samples), the leading blocks that every member
    lists with the same id, not counting any member's last block (it takes this
    step's new token, and copy-on-write keeps it private). Returns (prefix
    tables [n_groups][max_blocks], prefix lengths [n_groups], suffix tables
    [S][max_blocks], suffix lengths [S]) as int32 numpy arrays; a group that
    shares nothing gets a prefix of length 0."""
    tables = _i32(block_tables)
    lens = _i32(context_lens)
    S, max_blocks = tables.shape
    if group_size < 1 or S % group_size:
        raise ValueError("shared_prefix_plan: S must be a multiple of group_size")
    n_groups = S // group_size
    pre_tab = np.empty((n_groups, max_blocks), dtype=np.int32)
    pre_len = np.empty(n_groups, dtype=np.int32)
    suf_tab = np.empty((S, max_blocks), dtype=np.int32)
    suf_len = np.empty(S, dtype=np.int32)
    check(lib().pkv_shared_prefix_plan(_ptr(tables, P_i32), _ptr(lens, P_i32), S, max_blocks, group_size, bs,
                                       _ptr(pre_tab, P_i32), _ptr(pre_len, P_i32), _ptr(suf_tab, P_i32),
                                       _ptr(suf_len, P_i32)))
    return pre_tab, pre_len, suf_tab, suf_len


def paged_shared_prefix_decode_workspace(n_groups, M, Hq, Hkv, d, device="cuda"):
    import torch
    n = lib().pkv_paged_shared_prefix_decode_workspace_size(n_groups, M, Hq, Hkv, d)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def paged_shared_prefix_decode(out, q, k_cache, v_cache, prefix_tables, prefix_lens, suffix_tables,
                               suffix_lens, group_size, *, max_prefix_len, max_suffix_len, softmax_scale,
                               k_scale=1.0, v_scale=1.0, k_new=None, v_new=None, k_inv_scale=1.0,
                               v_inv_scale=1.0, workspace=None, stream=None):
    """pkv_paged_shared_prefix_decode: decode attention (and, with k_new/v_new,
    the step's write) for groups of group_size sequences over their group's
    prefix blocks followed by their own suffix blocks. out float32 [S][Hq][d]."""
    import torch
    P, Hkv, bs, d = _pools("paged_shared_prefix_decode", k_cache, v_cache)
    S, Hq = _attn_args("paged_shared_prefix_decode", out, q, k_cache, suffix_tables, suffix_lens, d)
    M = int(group_size)
    if M < 1 or S % M:
        raise ValueError("paged_shared_prefix_decode: S must be a multiple of group_size")
    n_groups = S // M
    for t, name in ((prefix_tables, "prefix_tables"), (prefix_lens, "prefix_lens"),
                    (suffix_tables, "suffix_tables"), (suffix_lens, "suffix_lens")):
        if t.dtype != torch.int32:
            raise ValueError(f"paged_shared_prefix_decode: {name} must be int32")
    if prefix_tables.shape[0] != n_groups or prefix_lens.shape != (n_groups,):
        raise ValueError("paged_shared_prefix_decode: prefix tables/lengths shape mismatch")
    if suffix_tables.shape[0] != S or suffix_lens.shape != (S,):
        raise ValueError("paged_shared_prefix_decode: suffix tables/lengths shape mismatch")
    if (k_new is None) != (v_new is None):
        raise ValueError("paged_shared_prefix_decode: give both k_new and v_new, or neither")
    if k_new is not None:
        for t, name in ((k_new, "k_new"), (v_new, "v_new")):
            if tuple(t.shape) != (S, Hkv, d):
                raise ValueError(f"paged_shared_prefix_decode: {name} must be [S][Hkv][d]")
            _src_dtype_ok("paged_shared_prefix_decode", name, t, k_cache)
    _one_device("paged_shared_prefix_decode", out, q, k_new, v_new, k_cache, v_cache, prefix_tables, prefix_lens,
                suffix_tables, suffix_lens, workspace)
    if workspace is None:
        workspace = paged_shared_prefix_decode_workspace(n_groups, M, Hq, Hkv, d, device=q.device)
    check(lib().pkv_paged_shared_prefix_decode(
        _dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new") if k_new is not None else None,
        _dev(v_new, "v_new") if v_new is not None else None, _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(prefix_tables, "prefix_tables"), _dev(prefix_lens, "prefix_lens"),
        prefix_tables.shape[1], int(max_prefix_len), _dev(suffix_tables, "suffix_tables"),
        _dev(suffix_lens, "suffix_lens"), suffix_tables.shape[1], int(max_suffix_len), n_groups, M, Hq,
        Hkv, d, bs, P, float(softmax_scale), float(k_scale), float(v_scale), float(k_inv_scale),
        float(v_inv_scale), _dtype_code(q), _dtype_code(k_cache), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))


class SharedPrefixDecode:
    """Decode steps for groups of group_size consecutive sequences that share
    leading blocks, reading the shared blocks once per group
    (pkv_paged_shared_prefix_decode). The plan (host tables, see
    shared_prefix_plan) is built and uploaded once here, with the workspace,
    and holds while the tables and lengths do: a step that changes them needs
    a new plan. __call__ runs one step: with k_new/v_new the write of each
    sequence's new token and the attention, without them the attention alone."""

    def __init__(self, block_tables, context_lens, group_size, bs, Hq, Hkv, d, device="cuda"):
        import torch
        pre_tab, pre_len, suf_tab, suf_len = shared_prefix_plan(block_tables, context_lens, group_size, bs)
        S = len(suf_len)
        self.M, self.n_groups, self.S, self.Hq, self.d = group_size, S // group_size, S, Hq, d
        self.max_prefix = int(pre_len.max()) if len(pre_len) else 0
        self.max_suffix = int(suf_len.max()) if len(suf_len) else 0
        self.prefix_tokens = int(pre_len.sum())
        self.pre_tab = torch.from_numpy(pre_tab).to(device)
        self.pre_len = torch.from_numpy(pre_len).to(device)
        self.suf_tab = torch.from_numpy(suf_tab).to(device)
        self.suf_len = torch.from_numpy(suf_len).to(device)
        self.ws = paged_shared_prefix_decode_workspace(self.n_groups, group_size, Hq, Hkv, d, device=device)

    def __call__(self, out, q, k_cache, v_cache, *, softmax_scale, k_scale=1.0, v_scale=1.0, k_new=None,
                 v_new=None, k_inv_scale=1.0, v_inv_scale=1.0, stream=None):
        paged_shared_prefix_decode(out, q, k_cache, v_cache, self.pre_tab, self.pre_len, self.suf_tab,
                                   self.suf_len, self.M, max_prefix_len=self.max_prefix,
                                   max_suffix_len=self.max_suffix, softmax_scale=softmax_scale,
                                   k_scale=k_scale, v_scale=v_scale, k_new=k_new, v_new=v_new,
                                   k_inv_scale=k_inv_scale, v_inv_scale=v_inv_scale, workspace=self.ws,
                                   stream=stream)


def quantise_pool(values_k, values_v, codes_k, codes_v, *, k_inv_scale, v_inv_scale, stream=None):
    """Fill whole fp8 pools from bf16 pools of the same layout, through the
    library's cache write (every slot written once, in order)."""
    import torch
    P, Hkv, bs, d = values_k.shape
    tok_k = values_k.permute(0, 2, 1, 3).reshape(P * bs, Hkv, d).contiguous()
    if values_v.dim() == 4:                    # [P][Hkv][d][bs] (bs <= 16)
        tok_v = values_v.permute(0, 3, 1, 2)
    else:                                      # [P][Hkv][bs/vs][d][vs]
        tok_v = values_v.permute(0, 2, 4, 1, 3)
    tok_v = tok_v.reshape(P * bs, Hkv, d).contiguous()
    slots = torch.arange(P * bs, dtype=torch.int64, device=values_k.device)
    kv_cache_write(tok_k, tok_v, codes_k, codes_v, slots, k_inv_scale=k_inv_scale,
                   v_inv_scale=v_inv_scale, stream=stream)


# ------------------------------------------------------------------ host side
def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a, ctype):
    return a.ctypes.data_as(ctype)


def slots_from_tables(tables, positions, bs):
    """pkv_slots_from_tables -> int64 [S]."""
    tables = _i32(tables)
    positions = _i32(positions)
    S, maxb = tables.shape
    out = np.empty(S, dtype=np.int64)
    check(lib().pkv_slots_from_tables(_ptr(tables, P_i32), _ptr(positions, P_i32), S, maxb, bs,
                                      _ptr(out, P_i64)))
    return out


def waste_stats(lens, bs, max_len):
    """pkv_waste_stats -> dict."""
    lens = _i32(lens)
    p, nv, u = c_i64(), c_i64(), c_i64()
    wp, wn = c_f64(), c_f64()
    check(lib().pkv_waste_stats(_ptr(lens, P_i32), len(lens), bs, max_len, ctypes.byref(p),
                                ctypes.byref(nv), ctypes.byref(u), ctypes.byref(wp),
                                ctypes.byref(wn)))
    return {"paged_slots": p.value, "naive_slots": nv.value, "used": u.value,
            "waste_paged": wp.value, "waste_naive": wn.value}


def block_hashes(tokens, bs, extra=b""):
    """pkv_block_hashes -> uint8 [n_tokens // bs][32]."""
    tokens = _i32(tokens)
    m = len(tokens) // bs
    out = np.zeros((max(m, 1), 32), dtype=np.uint8)
    ex = bytes(extra)
    check(lib().pkv_block_hashes(_ptr(tokens, P_i32), len(tokens), bs, ex if ex else None, len(ex),
                                 out.ctypes.data_as(c_vp)))
    return out[:m]


class Allocator:
    """The library's host block allocator (pkv_allocator_*)."""

    def __init__(self, num_blocks, block_size):
        h = c_vp()
        check(lib().pkv_allocator_create(num_blocks, block_size, ctypes.byref(h)))
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if self._h:
            lib().pkv_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def create(self, seq_id):
        check(lib().pkv_seq_create(self._h, seq_id))

    def append(self, seq_id, n_tokens):
        """Returns (slots int64[n], cow_pairs list of (src, dst))."""
        slots = np.empty(max(n_tokens, 1), dtype=np.int64)
        src, dst, n = c_i32(), c_i32(), c_i32()
        st = lib().pkv_seq_append(self._h, seq_id, n_tokens, _ptr(slots, P_i64), ctypes.byref(src),
                                  ctypes.byref(dst), ctypes.byref(n))
        if st == PKV_E_NO_BLOCKS:
            raise NoBlocks(st, last_error())
        check(st)
        return slots[:n_tokens], ([(src.value, dst.value)] if n.value else [])

    def fork(self, parent, child):
        check(lib().pkv_seq_fork(self._h, parent, child))

    def release(self, seq_id):
        check(lib().pkv_seq_free(self._h, seq_id))

    def info(self, seq_id):
        L, n = c_i64(), c_i32()
        check(lib().pkv_seq_info(self._h, seq_id, ctypes.byref(L), ctypes.byref(n)))
        return L.value, n.value

    def tables(self, seq_ids, max_blocks):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        S = len(ids)
        tab = np.empty((S, max_blocks), dtype=np.int32)
        lens = np.empty(S, dtype=np.int32)
        check(lib().pkv_build_block_tables(self._h, _ptr(ids, P_i64), S, max_blocks,
                                           _ptr(tab, P_i32), _ptr(lens, P_i32)))
        return tab, lens

    def create_prefixed(self, seq_id, tokens, extra=b""):
        """pkv_seq_create_prefixed -> (slots int64[n], n_cached)."""
        tokens = _i32(tokens)
        n = len(tokens)
        slots = np.empty(max(n, 1), dtype=np.int64)
        n_cached = c_i32()
        ex = bytes(extra)
        st = lib().pkv_seq_create_prefixed(self._h, seq_id, _ptr(tokens, P_i32), n, ex if ex else None,
                                           len(ex), _ptr(slots, P_i64), ctypes.byref(n_cached))
        if st == PKV_E_NO_BLOCKS:
            raise NoBlocks(st, last_error())
        check(st)
        return slots[:n], n_cached.value

    def prefix_stats(self):
        h, m, c = c_i64(), c_i64(), c_i32()
        check(lib().pkv_prefix_cache_stats(self._h, ctypes.byref(h), ctypes.byref(m), ctypes.byref(c)))
        return {"hit_blocks": h.value, "miss_blocks": m.value, "cached_blocks": c.value}

    def stats(self):
        s = PkvStats()
        check(lib().pkv_allocator_stats(self._h, ctypes.byref(s)))
        return {k: getattr(s, k) for k, _ in PkvStats._fields_}
