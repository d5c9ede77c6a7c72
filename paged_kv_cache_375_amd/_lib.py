"""ctypes binding of libpagedattn.so: argument marshalling only.

Every computation runs in the library's HIP kernels; torch tensors are used
for device memory and the current stream.  Loading fails loudly when the
library has not been built — there is no fallback.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpagedattn.so")

PA_OK, PA_ERR_INVALID_ARGUMENT, PA_ERR_OUT_OF_BLOCKS, PA_ERR_UNKNOWN_SEQ = 0, 1, 2, 3
PA_ERR_WORKSPACE_TOO_SMALL, PA_ERR_UNSUPPORTED, PA_ERR_HIP, PA_ERR_HOST_MEMORY = 4, 5, 6, 7
PA_F32, PA_F16, PA_FP8_E4M3 = 0, 1, 2
PA_SWAP_OUT, PA_SWAP_IN = 0, 1

# every symbol the public header declares
EXPORTS = (
    "pa_kv_append", "pa_kv_write_prompt", "pa_copy_blocks", "pa_swap_blocks", "pa_decode_workspace_size", "pa_decode",
    "pa_decode_step", "pa_decode_step_noalloc", "pa_decode_shared_prefix", "pa_decode_shared_workspace_size", "pa_allocator_create", "pa_allocator_destroy", "pa_allocator_num_free", "pa_seq_allocate",
    "pa_seq_allocate_cached", "pa_prefix_cache_size", "pa_seq_fork", "pa_seq_append_slot", "pa_seq_free",
    "pa_seq_swap_out", "pa_seq_swap_in", "pa_seq_get", "pa_export_tables", "pa_block_refcount",
    "pa_allocator_get_stats", "pa_latest_arrival", "pa_simulate_arrivals", "pa_status_str", "pa_last_error",
    "pa_timing_enable", "pa_timing_read", "pa_read_probe",
)


class PaKVCache(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("k_inv_scale", ctypes.c_float), ("v_inv_scale", ctypes.c_float),
    ]


class PaAllocatorStats(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int32), ("num_free", ctypes.c_int32), ("num_shared", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32), ("tokens_held", ctypes.c_int64), ("slots_allocated", ctypes.c_int64),
    ]


class PaArrivalReadout(ctypes.Structure):
    _fields_ = [
        ("max_concurrent", ctypes.c_int32), ("rounds", ctypes.c_int32), ("preemptions", ctypes.c_int32),
        ("reserved0", ctypes.c_int32), ("utilisation", ctypes.c_double),
    ]


class PagedAttnError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{status_str(status)}: {detail}")
        self.status = status


_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    P = ctypes.POINTER
    st = ctypes.c_int
    sig = {
        "pa_kv_append": (st, [P(PaKVCache), vp, vp, i32, vp, vp, i32, i32, vp]),
        "pa_kv_write_prompt": (st, [P(PaKVCache), vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, vp]),
        "pa_copy_blocks": (st, [P(PaKVCache), vp, i32, vp]),
        "pa_swap_blocks": (st, [P(PaKVCache), vp, vp, vp, i32, i32, vp]),
        "pa_decode_workspace_size": (ctypes.c_size_t, [i32, i32, i32, i32]),
        "pa_decode": (st, [P(PaKVCache), vp, vp, i32, i32, vp, vp, i32, i32, i32, f32, vp, ctypes.c_size_t, vp]),
        "pa_decode_step": (st, [P(PaKVCache), vp, vp, vp, vp, i32, i32, vp, vp, i32, i32, i32, f32, vp,
                                ctypes.c_size_t, vp]),
        "pa_decode_step_noalloc": (st, [P(PaKVCache), vp, vp, vp, vp, i32, i32, vp, vp, i32, i32, i32, f32, vp]),
        "pa_decode_shared_prefix": (st, [P(PaKVCache), vp, vp, vp, vp, i32, i32, vp, vp, i32, i32, i32, f32, i32, vp,
                                         vp, vp, ctypes.c_size_t, vp]),
        "pa_decode_shared_workspace_size": (ctypes.c_size_t, [i32, i32, i32, i32, i32]),
        "pa_allocator_create": (st, [i32, i32, vp, P(vp)]),
        "pa_allocator_destroy": (None, [vp]),
        "pa_allocator_num_free": (i32, [vp]),
        "pa_seq_allocate": (st, [vp, i32, i32]),
        "pa_seq_allocate_cached": (st, [vp, i32, vp, i32, P(i32)]),
        "pa_prefix_cache_size": (i32, [vp]),
        "pa_seq_fork": (st, [vp, i32, i32]),
        "pa_seq_append_slot": (st, [vp, i32, P(i32), P(i32)]),
        "pa_seq_free": (st, [vp, i32]),
        "pa_seq_swap_out": (st, [vp, i32, vp, i32, P(i32)]),
        "pa_seq_swap_in": (st, [vp, i32, vp, i32, P(i32)]),
        "pa_seq_get": (st, [vp, i32, vp, i32, P(i32), P(i32)]),
        "pa_export_tables": (st, [vp, vp, i32, i32, vp, vp]),
        "pa_block_refcount": (i32, [vp, i32]),
        "pa_allocator_get_stats": (st, [vp, P(PaAllocatorStats)]),
        "pa_latest_arrival": (i32, [vp]),
        "pa_simulate_arrivals": (st, [i32, i32, vp, vp, i32, P(PaArrivalReadout), vp, i32]),
        "pa_status_str": (ctypes.c_char_p, [st]),
        "pa_last_error": (ctypes.c_char_p, []),
        "pa_timing_enable": (st, [i32]),
        "pa_timing_read": (st, [P(ctypes.c_double), P(i32)]),
        "pa_read_probe": (st, [P(PaKVCache), vp, vp, i32, i32, i32, i32, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def status_str(s):
    return lib().pa_status_str(int(s)).decode()


def check(status):
    if status != PA_OK:
        raise PagedAttnError(status, lib().pa_last_error().decode())
    return status
