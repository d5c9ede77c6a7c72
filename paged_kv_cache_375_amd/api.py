"""Python face of the C ABI (same names, argument marshalling only).

Device buffers are torch tensors; kernels run on torch's current HIP stream
unless a stream is given.  Shapes and dtypes are checked here so that a
mistake fails before any launch; the library checks again on its side.
"""
import ctypes

import numpy as np
import torch

from . import _lib
from ._lib import PA_F16, PA_F32, PA_FP8_E4M3, PaAllocatorStats, PaKVCache, check, lib

TORCH_DTYPE = {PA_F32: torch.float32, PA_F16: torch.float16, PA_FP8_E4M3: torch.uint8}
DTYPE_CODE = {torch.float32: PA_F32, torch.float16: PA_F16, torch.uint8: PA_FP8_E4M3}
NAME_CODE = {"f32": PA_F32, "f16": PA_F16, "e4m3": PA_FP8_E4M3}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, dtype, name, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


class KVCache:
    """A K pool and a V pool, each [num_blocks][num_kv_heads][block_size][head_dim]."""

    def __init__(self, num_blocks, block_size, num_kv_heads, head_dim, kv_dtype, device="cuda",
                 k_scale=1.0, v_scale=1.0, k_inv_scale=1.0, v_inv_scale=1.0, k=None, v=None):
        kv_dtype = NAME_CODE.get(kv_dtype, kv_dtype)
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        tdt = TORCH_DTYPE[kv_dtype]
        self.k = torch.zeros(shape, dtype=tdt, device=device) if k is None else _dev(k, tdt, "k", shape)
        self.v = torch.zeros(shape, dtype=tdt, device=device) if v is None else _dev(v, tdt, "v", shape)
        self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim = shape[0], block_size, num_kv_heads, head_dim
        self.kv_dtype = kv_dtype
        self.struct = PaKVCache(self.k.data_ptr(), self.v.data_ptr(), num_blocks, block_size, num_kv_heads, head_dim,
                                kv_dtype, k_scale, v_scale, k_inv_scale, v_inv_scale)

    def with_pools(self, k, v):
        """The same description over another pair of pools of the same shape."""
        s = self.struct
        return KVCache(self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim, self.kv_dtype,
                       k_scale=s.k_scale, v_scale=s.v_scale, k_inv_scale=s.k_inv_scale, v_inv_scale=s.v_inv_scale,
                       k=k, v=v)


def _act(t):
    if t.dtype not in (torch.float32, torch.float16):
        raise TypeError("activations must be float32 or float16")
    return DTYPE_CODE[t.dtype]


def kv_append(cache: KVCache, k_new, v_new, block_tables, context_lens, stream=None):
    B = context_lens.shape[0]
    act = _act(k_new)
    shape = (B, cache.num_kv_heads, cache.head_dim)
    _dev(k_new, k_new.dtype, "k_new", shape)
    _dev(v_new, k_new.dtype, "v_new", shape)
    _dev(block_tables, torch.int32, "block_tables")
    _dev(context_lens, torch.int32, "context_lens", (B,))
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq]")
    check(lib().pa_kv_append(ctypes.byref(cache.struct), _ptr(k_new), _ptr(v_new), act, _ptr(block_tables),
                             _ptr(context_lens), B, block_tables.shape[1], _stream(stream)))


def kv_write_prompt(cache: KVCache, k_src, v_src, src_row, start_pos, count, block_tables, max_count, stream=None):
    B = count.shape[0]
    act = _act(k_src)
    _dev(k_src, k_src.dtype, "k_src")
    _dev(v_src, k_src.dtype, "v_src", k_src.shape)
    if k_src.dim() != 3 or tuple(k_src.shape[1:]) != (cache.num_kv_heads, cache.head_dim):
        raise ValueError("k_src must be [rows][num_kv_heads][head_dim]")
    _dev(src_row, torch.int64, "src_row", (B,))
    _dev(start_pos, torch.int32, "start_pos", (B,))
    _dev(count, torch.int32, "count", (B,))
    _dev(block_tables, torch.int32, "block_tables")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq]")
    check(lib().pa_kv_write_prompt(ctypes.byref(cache.struct), _ptr(k_src), _ptr(v_src), act, _ptr(src_row),
                                   _ptr(start_pos), _ptr(count), _ptr(block_tables), B, block_tables.shape[1],
                                   int(max_count), _stream(stream)))


def copy_blocks(cache: KVCache, src_dst_pairs, stream=None):
    _dev(src_dst_pairs, torch.int32, "src_dst_pairs")
    if src_dst_pairs.dim() != 2 or src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be [n][2]")
    check(lib().pa_copy_blocks(ctypes.byref(cache.struct), _ptr(src_dst_pairs), src_dst_pairs.shape[0],
                               _stream(stream)))


def swap_blocks(cache: KVCache, host_k, host_v, block_ids, direction, stream=None):
    """Move whole blocks between the pool and pinned host memory (pa_swap_blocks).

    host_k/host_v: pinned CPU tensors [n][num_kv_heads][block_size][head_dim]
    of the pool dtype (entry i is block block_ids[i]); block_ids: device int32 [n];
    direction "out" (pool -> host) or "in" (host -> pool)."""
    _dev(block_ids, torch.int32, "block_ids")
    if block_ids.dim() != 1:
        raise ValueError("block_ids must be [n]")
    n = block_ids.shape[0]
    shape = (n, cache.num_kv_heads, cache.block_size, cache.head_dim)
    for name, h in (("host_k", host_k), ("host_v", host_v)):
        if h.device.type != "cpu" or not h.is_pinned() or not h.is_contiguous():
            raise ValueError(f"{name} must be a contiguous pinned CPU tensor")
        if tuple(h.shape) != shape or h.dtype != cache.k.dtype:
            raise ValueError(f"{name} must be {shape} of {cache.k.dtype}")
    direction = {"out": _lib.PA_SWAP_OUT, "in": _lib.PA_SWAP_IN}[direction]
    check(lib().pa_swap_blocks(ctypes.byref(cache.struct), _ptr(host_k), _ptr(host_v), _ptr(block_ids), n, direction,
                               _stream(stream)))


def decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len):
    return int(lib().pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len))


def new_workspace(num_seqs, num_q_heads, head_dim, max_context_len, device="cuda"):
    """A zero-filled decode workspace (its arrival counters must start at zero)."""
    need = decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len)
    return torch.zeros(max(need, 1), dtype=torch.uint8, device=device)


def _decode_args(cache, q, block_tables, context_lens, max_context_len, out, workspace):
    B, hq, d = q.shape
    _dev(q, q.dtype, "q", (B, hq, cache.head_dim))
    _dev(block_tables, torch.int32, "block_tables")
    _dev(context_lens, torch.int32, "context_lens", (B,))
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq]")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, q.dtype, "out", q.shape)
    if workspace is None:
        workspace = new_workspace(B, hq, d, max_context_len, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    return out, workspace, ws_bytes


def decode(cache: KVCache, q, block_tables, context_lens, max_context_len, sm_scale, out=None, workspace=None,
           stream=None):
    """Attention of every sequence's query over its paged context (pa_decode)."""
    B, hq, d = q.shape
    act = _act(q)
    out, workspace, ws_bytes = _decode_args(cache, q, block_tables, context_lens, max_context_len, out, workspace)
    check(lib().pa_decode(ctypes.byref(cache.struct), _ptr(q), _ptr(out), act, hq, _ptr(block_tables),
                          _ptr(context_lens), B, block_tables.shape[1], int(max_context_len), float(sm_scale),
                          _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def decode_step(cache: KVCache, q, k_new, v_new, block_tables, context_lens, max_context_len, sm_scale, out=None,
                workspace=None, stream=None):
    """Append of the new K/V and decode in one launch (pa_decode_step)."""
    B, hq, d = q.shape
    act = _act(q)
    shape = (B, cache.num_kv_heads, cache.head_dim)
    _dev(k_new, q.dtype, "k_new", shape)
    _dev(v_new, q.dtype, "v_new", shape)
    out, workspace, ws_bytes = _decode_args(cache, q, block_tables, context_lens, max_context_len, out, workspace)
    check(lib().pa_decode_step(ctypes.byref(cache.struct), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), act, hq,
                               _ptr(block_tables), _ptr(context_lens), B, block_tables.shape[1],
                               int(max_context_len), float(sm_scale), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def decode_step_noalloc(cache: KVCache, q, k_new, v_new, block_tables, context_lens, max_context_len, sm_scale,
                        out, stream=None):
    """pa_decode_step with the library's own per-device scratch in place of a
    workspace (pa_decode_step_noalloc); `out` must be given (nothing is
    allocated)."""
    B, hq, d = q.shape
    act = _act(q)
    shape = (B, cache.num_kv_heads, cache.head_dim)
    _dev(k_new, q.dtype, "k_new", shape)
    _dev(v_new, q.dtype, "v_new", shape)
    _dev(q, q.dtype, "q", (B, hq, cache.head_dim))
    _dev(block_tables, torch.int32, "block_tables")
    _dev(context_lens, torch.int32, "context_lens", (B,))
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [num_seqs][max_blocks_per_seq]")
    _dev(out, q.dtype, "out", q.shape)
    check(lib().pa_decode_step_noalloc(ctypes.byref(cache.struct), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), act,
                                       hq, _ptr(block_tables), _ptr(context_lens), B, block_tables.shape[1],
                                       int(max_context_len), float(sm_scale), _stream(stream)))
    return out


def shared_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len, max_shared_tokens):
    return int(lib().pa_decode_shared_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
                                                     max_shared_tokens))


def decode_shared_prefix(cache: KVCache, q, block_tables, context_lens, max_context_len, sm_scale, group_start,
                         group_shared_blocks, k_new=None, v_new=None, out=None, workspace=None, stream=None):
    """Decode (with the append when k_new/v_new are given) of a batch whose sequence groups
    [group_start[g], group_start[g + 1]) share their first group_shared_blocks[g] blocks
    (pa_decode_shared_prefix)."""
    B, hq, d = q.shape
    act = _act(q)
    gs = np.ascontiguousarray(group_start, dtype=np.int32)
    gb = np.ascontiguousarray(group_shared_blocks, dtype=np.int32)
    if gs.ndim != 1 or gb.ndim != 1 or len(gs) != len(gb) + 1:
        raise ValueError("group_start needs one more entry than group_shared_blocks")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        shape = (B, cache.num_kv_heads, cache.head_dim)
        _dev(k_new, q.dtype, "k_new", shape)
        _dev(v_new, q.dtype, "v_new", shape)
    if workspace is None:
        need = shared_workspace_size(B, hq, d, max_context_len, int(gb.max(initial=0)) * cache.block_size)
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    out, workspace, ws_bytes = _decode_args(cache, q, block_tables, context_lens, max_context_len, out, workspace)
    check(lib().pa_decode_shared_prefix(ctypes.byref(cache.struct), _ptr(q), _ptr(k_new) if k_new is not None else None,
                                        _ptr(v_new) if v_new is not None else None, _ptr(out), act, hq,
                                        _ptr(block_tables), _ptr(context_lens), B, block_tables.shape[1],
                                        int(max_context_len), float(sm_scale), len(gb),
                                        gs.ctypes.data_as(ctypes.c_void_p), gb.ctypes.data_as(ctypes.c_void_p),
                                        _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def read_probe(cache: KVCache, block_tables, context_lens, max_context_len, mode, sink, stream=None):
    """Measurement only (pa_read_probe): read the pools with the decode's load
    pattern (mode 0, "paged") or start to end (mode 1, "linear")."""
    mode = {"paged": 0, "linear": 1}.get(mode, mode)
    _dev(sink, torch.int32, "sink", (1024,))
    B = context_lens.shape[0]
    check(lib().pa_read_probe(ctypes.byref(cache.struct), _ptr(block_tables), _ptr(context_lens), B,
                              block_tables.shape[1], int(max_context_len), int(mode), _ptr(sink), _stream(stream)))


def timing_enable(on=True):
    check(lib().pa_timing_enable(1 if on else 0))


def timing_read():
    """(decode kernel ms summed, launches) since the last read."""
    ms, n = ctypes.c_double(), ctypes.c_int32()
    check(lib().pa_timing_read(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


class OutOfBlocks(_lib.PagedAttnError):
    pass


class Allocator:
    """The library's host block allocator (C++), with the same methods as the reference model."""

    def __init__(self, num_blocks, block_size, free_order=None):
        h = ctypes.c_void_p()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("free_order must have num_blocks entries")
        check(lib().pa_allocator_create(num_blocks, block_size,
                                        order.ctypes.data_as(ctypes.c_void_p) if order is not None else None,
                                        ctypes.byref(h)))
        self._h = h
        self._destroy = lib().pa_allocator_destroy  # kept: the module may be torn down before __del__
        self._order = order
        self.num_blocks, self.block_size = num_blocks, block_size

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._destroy(h)
            self._h = None

    def _call(self, status):
        if status == _lib.PA_ERR_OUT_OF_BLOCKS:
            raise OutOfBlocks(status, lib().pa_last_error().decode())
        return check(status)

    def num_free(self):
        return lib().pa_allocator_num_free(self._h)

    def allocate(self, seq, num_tokens):
        self._call(lib().pa_seq_allocate(self._h, seq, num_tokens))

    def allocate_cached(self, seq, tokens):
        """A new sequence with prompt token ids `tokens`, reusing cached full blocks of the same
        beginning; returns how many leading tokens the reused blocks already hold."""
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        cached = ctypes.c_int32()
        self._call(lib().pa_seq_allocate_cached(self._h, seq, toks.ctypes.data_as(ctypes.c_void_p), len(toks),
                                                ctypes.byref(cached)))
        return cached.value

    def prefix_cache_size(self):
        return lib().pa_prefix_cache_size(self._h)

    def fork(self, parent, child):
        self._call(lib().pa_seq_fork(self._h, parent, child))

    def append_slot(self, seq):
        src, dst = ctypes.c_int32(), ctypes.c_int32()
        self._call(lib().pa_seq_append_slot(self._h, seq, ctypes.byref(src), ctypes.byref(dst)))
        return (src.value, dst.value)

    def free_seq(self, seq):
        self._call(lib().pa_seq_free(self._h, seq))

    def _swap(self, fn, seq):
        n = ctypes.c_int32()
        status = fn(self._h, seq, None, 0, ctypes.byref(n))
        if status == _lib.PA_ERR_INVALID_ARGUMENT and n.value > 0:  # sized: call again with room
            buf = np.zeros(n.value, dtype=np.int32)
            self._call(fn(self._h, seq, buf.ctypes.data_as(ctypes.c_void_p), n.value, ctypes.byref(n)))
            return buf.tolist()
        self._call(status)
        return []

    def swap_out(self, seq):
        """Release every block of seq, keep its length; its former blocks in logical order."""
        return self._swap(lib().pa_seq_swap_out, seq)

    def swap_in(self, seq):
        """Fresh blocks for a swapped-out seq's whole length, all or none; in logical order."""
        return self._swap(lib().pa_seq_swap_in, seq)

    def table(self, seq):
        n, c = ctypes.c_int32(), ctypes.c_int32()
        self._call(lib().pa_seq_get(self._h, seq, None, 0, ctypes.byref(n), ctypes.byref(c)))
        buf = np.zeros(max(1, n.value), dtype=np.int32)
        self._call(lib().pa_seq_get(self._h, seq, buf.ctypes.data_as(ctypes.c_void_p), n.value, ctypes.byref(n),
                                    ctypes.byref(c)))
        return buf[: n.value].tolist()

    def export(self, seqs, max_blocks):
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        t = np.zeros((len(seqs), max_blocks), dtype=np.int32)
        c = np.zeros(len(seqs), dtype=np.int32)
        self._call(lib().pa_export_tables(self._h, seqs.ctypes.data_as(ctypes.c_void_p), len(seqs), max_blocks,
                                          t.ctypes.data_as(ctypes.c_void_p), c.ctypes.data_as(ctypes.c_void_p)))
        return t, c

    def refcount(self, block):
        return lib().pa_block_refcount(self._h, block)

    def stats(self):
        s = PaAllocatorStats()
        check(lib().pa_allocator_get_stats(self._h, ctypes.byref(s)))
        return s

    def latest_arrival(self):
        r = lib().pa_latest_arrival(self._h)
        return None if r < 0 else r


def simulate_arrivals(num_blocks, block_size, arrivals, lengths, trace_rounds=0):
    """The toy machine's arrival simulator (pa_simulate_arrivals), run over the library's allocator.

    Returns dict(max_concurrent, utilisation, rounds, preemptions, trace), trace holding
    (running, tokens held, slots reserved) for the first trace_rounds rounds."""
    arr = np.ascontiguousarray(arrivals, dtype=np.int32)
    lens = np.ascontiguousarray(lengths, dtype=np.int32)
    if arr.shape != lens.shape or arr.ndim != 1:
        raise ValueError("arrivals and lengths must be 1-D of equal length")
    out = _lib.PaArrivalReadout()
    tr = np.zeros((max(1, trace_rounds), 3), dtype=np.int32)
    check(lib().pa_simulate_arrivals(num_blocks, block_size, arr.ctypes.data_as(ctypes.c_void_p),
                                     lens.ctypes.data_as(ctypes.c_void_p), len(arr), ctypes.byref(out),
                                     tr.ctypes.data_as(ctypes.c_void_p), trace_rounds))
    return {"max_concurrent": out.max_concurrent, "utilisation": out.utilisation, "rounds": out.rounds,
            "preemptions": out.preemptions,
            "trace": [tuple(int(x) for x in row) for row in tr[: min(trace_rounds, out.rounds)]]}
