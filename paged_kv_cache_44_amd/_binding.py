"""ctypes declarations of the C ABI in include/pa.h (argument marshalling
only; every computation happens in the HIP library)."""

import ctypes
import os

from .build import LIB_PATH

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_NO_SPACE = range(6)
#: size of the fixed device array pa_decode_no_alloc uses (PA_DECODE_NO_ALLOC_MAX_BYTES)
DECODE_NO_ALLOC_MAX_BYTES = 64 << 20
PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = range(4)
PA_COPY_D2D, PA_COPY_H2D, PA_COPY_D2H, PA_COPY_H2D_KERNEL, PA_COPY_D2H_KERNEL = range(5)

#: every function the header declares
EXPORTED = ("pa_write_kv", "pa_decode", "pa_decode_attend", "pa_decode_merge", "pa_decode_no_alloc",
            "pa_decode_partition_tokens", "pa_decode_workspace_size", "pa_decode_shared",
            "pa_decode_shared_workspace_size", "pa_prefill",
            "pa_copy_blocks", "pa_copy_blocks_staged", "pa_copy_staging_size",
            "pa_host_pool_mapped", "pa_status_string", "pa_version",
            # pa_blocks.h
            "pa_bm_create", "pa_bm_destroy", "pa_bm_num_free", "pa_bm_add", "pa_bm_fork",
            "pa_bm_append", "pa_bm_blocks_needed", "pa_bm_copy_last_block", "pa_bm_release",
            "pa_bm_table", "pa_bm_newest_running", "pa_bm_swap_out", "pa_bm_swap_out_done",
            "pa_bm_swap_in")


class PaKvCache(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("dtype", ctypes.c_int),
        ("num_blocks", ctypes.c_int32),
        ("num_layers", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_stride", ctypes.c_int64),
        ("layer_stride", ctypes.c_int64),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libpa.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m paged_kv_cache_44_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(PaKvCache)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.pa_write_kv.argtypes = [P, i32, vp, vp, ctypes.c_int, vp, i32, vp]
    lib.pa_write_kv.restype = ctypes.c_int
    dec = [P, i32, vp, ctypes.c_int, vp, vp, i32, vp, i32, i32, i32, f32, vp, sz, vp]
    for name in ("pa_decode", "pa_decode_attend", "pa_decode_merge"):
        getattr(lib, name).argtypes = dec
        getattr(lib, name).restype = ctypes.c_int
    lib.pa_decode_no_alloc.argtypes = dec[:12] + [vp]
    lib.pa_decode_no_alloc.restype = ctypes.c_int
    lib.pa_decode_shared.argtypes = dec[:12] + [i32] + dec[12:]
    lib.pa_decode_shared.restype = ctypes.c_int
    lib.pa_decode_shared_workspace_size.argtypes = [P, i32, i32]
    lib.pa_decode_shared_workspace_size.restype = sz
    lib.pa_prefill.argtypes = [P, i32, vp, ctypes.c_int, vp, vp, i32, vp, i32, vp, i32, i32, i32,
                               i32, f32, vp]
    lib.pa_prefill.restype = ctypes.c_int
    # host block manager (pa_blocks.h)
    vpp = ctypes.POINTER(ctypes.c_void_p)
    pi32, pi64 = ctypes.POINTER(i32), ctypes.POINTER(i64)
    sig = {
        "pa_bm_create": ([i32, i32, vp, i32, vpp], ctypes.c_int),
        "pa_bm_destroy": ([vp], None),
        "pa_bm_num_free": ([vp, i32], i32),
        "pa_bm_add": ([vp, i64], ctypes.c_int),
        "pa_bm_fork": ([vp, i64, i64], ctypes.c_int),
        "pa_bm_append": ([vp, i64, i32, vp, vp, pi32], ctypes.c_int),
        "pa_bm_blocks_needed": ([vp, i64, i32], i32),
        "pa_bm_copy_last_block": ([vp, i64, vp], ctypes.c_int),
        "pa_bm_release": ([vp, i64], ctypes.c_int),
        "pa_bm_table": ([vp, i64, vp, i32, pi32, pi32], ctypes.c_int),
        "pa_bm_newest_running": ([vp, pi64], ctypes.c_int),
        "pa_bm_swap_out": ([vp, i64, vp, i32, pi32], ctypes.c_int),
        "pa_bm_swap_out_done": ([vp, i64], ctypes.c_int),
        "pa_bm_swap_in": ([vp, i64, vp, i32, pi32], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        getattr(lib, name).argtypes = args
        getattr(lib, name).restype = res
    lib.pa_decode_partition_tokens.argtypes = [P, i32, i32, i32]
    lib.pa_decode_partition_tokens.restype = i32
    lib.pa_decode_workspace_size.argtypes = [P, i32, i32, i32]
    lib.pa_decode_workspace_size.restype = sz
    lib.pa_copy_blocks.argtypes = [P, P, vp, i32, ctypes.c_int, vp]
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_copy_blocks_staged.argtypes = [P, P, vp, i32, ctypes.c_int, vp, sz, vp]
    lib.pa_copy_blocks_staged.restype = ctypes.c_int
    lib.pa_copy_staging_size.argtypes = [P, i32]
    lib.pa_copy_staging_size.restype = sz
    lib.pa_host_pool_mapped.argtypes = [P]
    lib.pa_host_pool_mapped.restype = ctypes.c_int32
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_version.argtypes = []
    lib.pa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


class PaError(RuntimeError):
    def __init__(self, status: int, what: str):
        lib = load_library()
        super().__init__(f"{what}: {lib.pa_status_string(status).decode()}")
        self.status = status


def check(status: int, what: str) -> None:
    if status != PA_OK:
        raise PaError(status, what)
