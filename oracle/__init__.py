"""Reference oracle for paged KV-cache decode — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and
this package imports nothing from the product.

What lives here:
  * ``oracle.c`` (loaded through ctypes below): append, prompt write, block
    copy and decode attention in plain scalar C, every value in double.
  * ``allocator.py``: the block allocator's bookkeeping in plain Python.
  * ``brute.py``: contiguous (unpaged) textbook attention in pure Python, the
    independent check of the paged decode on tiny inputs.
  * ``two_layer.py``: the two-layer cached-vs-recomputed model of the "KV 缓存"
    topic page (aiinfact.com), level-3 script, with its multiply-accumulate
    counters.

Pool layout indexed here: K and V each [num_blocks][num_kv_heads][block_size]
[head_dim].  Dtype codes: 0 f32, 1 f16, 2 OCP E4M3, 3 f64 (oracle only).
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, F16, E4M3, F64 = 0, 1, 2, 3
_NP = {F32: np.float32, F16: np.float16, E4M3: np.uint8, F64: np.float64}

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        vp, i32, f32, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = f64
        L.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_to_f64.restype = f64
        L.oracle_e4m3_encode.argtypes = [f32]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_quantize.argtypes = [f32, f32]
        L.oracle_e4m3_quantize.restype = ctypes.c_uint8
        L.oracle_append.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, i32, vp, i32, vp, i32, f32, f32]
        L.oracle_append.restype = i32
        L.oracle_write_tokens.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, i32, vp, vp, vp, vp, i32, i32, f32, f32]
        L.oracle_write_tokens.restype = i32
        L.oracle_copy_blocks.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, i32]
        L.oracle_copy_blocks.restype = i32
        L.oracle_decode.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, i32, i32, vp, i32, vp, i32,
                                    f64, f64, f64, vp, ctypes.POINTER(ctypes.c_longlong)]
        L.oracle_decode.restype = i32
        L.oracle_decode_pairs.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, i32, i32, vp, i32, vp, i32,
                                          f64, f64, f64, vp, vp, i32, vp]
        L.oracle_decode_pairs.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def dtype_code(np_dtype):
    np_dtype = np.dtype(np_dtype)
    for code, t in _NP.items():
        if np.dtype(t) == np_dtype:
            return code
    raise ValueError(f"no oracle dtype for {np_dtype}")


# ---- scalar formats ------------------------------------------------------

def f16_to_f64(bits):
    return lib().oracle_f16_to_f64(int(bits))


def e4m3_to_f64(code):
    return lib().oracle_e4m3_to_f64(int(code))


def e4m3_encode(y):
    """binary32 -> E4M3 byte, nearest-even, saturating to +-448."""
    return lib().oracle_e4m3_encode(float(np.float32(y)))


def e4m3_quantize(x, inv_scale):
    """The FP8 store rule: e4m3(f32(x) * inv_scale), one binary32 multiply."""
    return lib().oracle_e4m3_quantize(float(np.float32(x)), float(np.float32(inv_scale)))


def e4m3_decode_array(codes):
    L = lib()
    return np.array([L.oracle_e4m3_to_f64(int(c)) for c in np.asarray(codes).ravel()],
                    dtype=np.float64).reshape(np.shape(codes))


# ---- pool operations (in place on numpy arrays) --------------------------

def append(k_pool, v_pool, k_new, v_new, tables, ctx_lens, block_size, k_inv_scale=1.0, v_inv_scale=1.0):
    """Store token ctx_lens[s]-1 of every sequence; pools are modified in place."""
    nb, hkv, bs, d = k_pool.shape
    assert bs == block_size and v_pool.shape == k_pool.shape and v_pool.dtype == k_pool.dtype
    tables = _c(tables, np.int32)
    ctx = _c(ctx_lens, np.int32)
    k_new = np.ascontiguousarray(k_new)
    v_new = np.ascontiguousarray(v_new)
    assert k_new.shape == (len(ctx), hkv, d) and v_new.dtype == k_new.dtype
    rc = lib().oracle_append(_ptr(k_pool), _ptr(v_pool), dtype_code(k_pool.dtype), nb, bs, hkv, d,
                             _ptr(k_new), _ptr(v_new), dtype_code(k_new.dtype),
                             _ptr(tables), tables.shape[1], _ptr(ctx), len(ctx),
                             float(k_inv_scale), float(v_inv_scale))
    if rc:
        raise ValueError("oracle_append: table entry or position out of range")


def write_tokens(k_pool, v_pool, k_src, v_src, src_row, start, count, tables, k_inv_scale=1.0, v_inv_scale=1.0):
    """Prompt write: sequence s stores rows src_row[s]..+count[s] at positions start[s].."""
    nb, hkv, bs, d = k_pool.shape
    tables = _c(tables, np.int32)
    src_row = _c(src_row, np.int64)
    start = _c(start, np.int32)
    count = _c(count, np.int32)
    k_src = np.ascontiguousarray(k_src)
    v_src = np.ascontiguousarray(v_src)
    assert k_src.shape[1:] == (hkv, d) and v_src.shape == k_src.shape
    rc = lib().oracle_write_tokens(_ptr(k_pool), _ptr(v_pool), dtype_code(k_pool.dtype), nb, bs, hkv, d,
                                   _ptr(k_src), _ptr(v_src), dtype_code(k_src.dtype),
                                   _ptr(src_row), _ptr(start), _ptr(count), _ptr(tables), tables.shape[1],
                                   len(start), float(k_inv_scale), float(v_inv_scale))
    if rc:
        raise ValueError("oracle_write_tokens: table entry or position out of range")


def copy_blocks(k_pool, v_pool, pairs):
    nb, hkv, bs, d = k_pool.shape
    pairs = _c(np.asarray(pairs).reshape(-1, 2), np.int32)
    rc = lib().oracle_copy_blocks(_ptr(k_pool), _ptr(v_pool), dtype_code(k_pool.dtype), nb, bs, hkv, d,
                                  _ptr(pairs), pairs.shape[0])
    if rc:
        raise ValueError("oracle_copy_blocks: block id out of range")


def decode(k_pool, v_pool, q, tables, ctx_lens, sm_scale, k_scale=1.0, v_scale=1.0, count_macs=False):
    """Paged decode attention; returns [num_seqs][hq][d] float64 (and the MAC count)."""
    nb, hkv, bs, d = k_pool.shape
    q = np.ascontiguousarray(q)
    B, hq, dq = q.shape
    assert dq == d
    tables = _c(tables, np.int32)
    ctx = _c(ctx_lens, np.int32)
    assert tables.shape[0] == B and ctx.shape == (B,)
    out = np.zeros((B, hq, d), dtype=np.float64)
    macs = ctypes.c_longlong(0)
    rc = lib().oracle_decode(_ptr(k_pool), _ptr(v_pool), dtype_code(k_pool.dtype), nb, bs, hkv, d,
                             _ptr(q), dtype_code(q.dtype), hq, _ptr(tables), tables.shape[1], _ptr(ctx), B,
                             float(sm_scale), float(k_scale), float(v_scale), _ptr(out),
                             ctypes.byref(macs))
    if rc:
        raise ValueError("oracle_decode: bad arguments or table entry out of range")
    return (out, macs.value) if count_macs else out


def decode_pairs(k_pool, v_pool, q, tables, ctx_lens, sm_scale, seqs, heads, k_scale=1.0, v_scale=1.0):
    """Decode only the listed (sequence, head) pairs; returns [n][d] float64."""
    nb, hkv, bs, d = k_pool.shape
    q = np.ascontiguousarray(q)
    B, hq, _ = q.shape
    tables = _c(tables, np.int32)
    ctx = _c(ctx_lens, np.int32)
    seqs = _c(seqs, np.int32)
    heads = _c(heads, np.int32)
    out = np.zeros((len(seqs), d), dtype=np.float64)
    rc = lib().oracle_decode_pairs(_ptr(k_pool), _ptr(v_pool), dtype_code(k_pool.dtype), nb, bs, hkv, d,
                                   _ptr(q), dtype_code(q.dtype), hq, _ptr(tables), tables.shape[1], _ptr(ctx), B,
                                   float(sm_scale), float(k_scale), float(v_scale),
                                   _ptr(seqs), _ptr(heads), len(seqs), _ptr(out))
    if rc:
        raise ValueError("oracle_decode_pairs: bad arguments")
    return out
