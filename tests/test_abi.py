"""The C-ABI library on the CPU: it loads, exports every function the
headers under include/ declare, and rejects bad arguments before any HIP call (so no
GPU is needed here)."""

import ctypes
import os
import re

import pytest

from paged_kv_cache_44_amd import _binding as B

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
FAKE = 0x100000          # aligned, never dereferenced: every call below fails or
                         # returns before touching memory


def declared_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_and_binding_agree():
    assert declared_functions() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol(pa_lib):
    for name in declared_functions():
        assert hasattr(pa_lib, name), name
    assert pa_lib.pa_version().decode().count(".") == 2


def test_status_strings(pa_lib):
    for s in range(6):
        assert pa_lib.pa_status_string(s).decode().startswith("PA_")
    assert b"unknown" in pa_lib.pa_status_string(99)


def _cache(dtype=B.PA_BF16, blocks=100, layers=1, heads=8, bs=16, dim=128, ks=1.0, vs=1.0):
    ls = heads * bs * dim
    return B.PaKvCache(FAKE, FAKE, dtype, blocks, layers, heads, bs, dim, layers * ls, ls, ks, vs)


def test_workspace_and_partition_queries(pa_lib):
    # matrix-core path (bf16 pool, bf16 queries): splits at 16-token chunks and
    # always needs a workspace (partials + chunk prefix sums)
    c = _cache()
    assert pa_lib.pa_decode_partition_tokens(ctypes.byref(c), 256, 32, 4000) == 16
    ws = pa_lib.pa_decode_workspace_size(ctypes.byref(c), 256, 32, 4000)
    assert ws >= (256 * 8 * 4) * (128 + 2) * 4 + 257 * 4
    assert pa_lib.pa_decode_workspace_size(ctypes.byref(c), 4, 32, 16) > 0
    # VALU path (fp32 pool): fixed partitions; one partition needs no workspace
    f = _cache(dtype=B.PA_F32, dim=64, heads=4)
    p = pa_lib.pa_decode_partition_tokens(ctypes.byref(f), 64, 4, 4000)
    assert p >= 64 and p % 64 == 0
    parts = -(-4000 // p)
    ws = pa_lib.pa_decode_workspace_size(ctypes.byref(f), 64, 4, 4000)
    assert parts > 1 and ws >= 64 * 4 * parts * (64 + 2) * 4
    assert pa_lib.pa_decode_workspace_size(ctypes.byref(f), 4, 4, 16) == 0
    # invalid geometry -> 0
    bad = _cache(bs=12)
    assert pa_lib.pa_decode_partition_tokens(ctypes.byref(bad), 4, 32, 100) == 0


def _decode(lib, c, q_dtype=B.PA_BF16, hq=32, seqs=4, max_ctx=100, ws=None, ws_bytes=0,
            q=FAKE, out=FAKE, tables=FAKE, ctx=FAKE, scale=0.1, layer=0):
    return lib.pa_decode(ctypes.byref(c), layer, q, q_dtype, out, tables, 8, ctx, max_ctx, seqs,
                         hq, scale, ws, ws_bytes, None)


def test_decode_argument_errors(pa_lib):
    c = _cache()
    assert _decode(pa_lib, c, seqs=0) == B.PA_OK                      # nothing to do
    assert _decode(pa_lib, c, hq=30) == B.PA_ERR_INVALID_ARG          # not a multiple of 8
    assert _decode(pa_lib, c, hq=8 * 16) == B.PA_ERR_WORKSPACE        # group of 16: matrix cores
    assert _decode(pa_lib, c, hq=8 * 32) == B.PA_ERR_UNSUPPORTED      # group of 32
    f32 = _cache(dtype=B.PA_F32, dim=64, heads=4)
    assert _decode(pa_lib, f32, q_dtype=B.PA_F32, hq=4 * 16) == B.PA_ERR_UNSUPPORTED   # VALU: <= 8
    assert _decode(pa_lib, c, q_dtype=B.PA_F16) == B.PA_ERR_UNSUPPORTED
    assert _decode(pa_lib, c, layer=1) == B.PA_ERR_INVALID_ARG
    assert _decode(pa_lib, c, q=None) == B.PA_ERR_INVALID_ARG
    assert _decode(pa_lib, c, scale=float("inf")) == B.PA_ERR_INVALID_ARG
    assert _decode(pa_lib, c, max_ctx=5000) == B.PA_ERR_WORKSPACE     # needs a workspace
    assert _decode(pa_lib, c, max_ctx=5, ws=FAKE, ws_bytes=64) == B.PA_ERR_WORKSPACE
    assert _decode(pa_lib, _cache(dim=96)) == B.PA_ERR_UNSUPPORTED
    assert _decode(pa_lib, _cache(dtype=B.PA_F32, dim=128), q_dtype=B.PA_F32) == B.PA_ERR_UNSUPPORTED
    assert _decode(pa_lib, _cache(ks=0.5)) == B.PA_ERR_INVALID_ARG    # scale on a bf16 pool
    assert _decode(pa_lib, _cache(dtype=B.PA_FP8_E4M3, ks=0.0)) == B.PA_ERR_INVALID_ARG


def test_write_argument_errors(pa_lib):
    c = _cache()
    w = lambda **kw: pa_lib.pa_write_kv(ctypes.byref(kw.get("c", c)), kw.get("layer", 0), FAKE,
                                        FAKE, kw.get("src", B.PA_BF16), FAKE, kw.get("n", 5), None)
    assert w(n=0) == B.PA_OK
    assert w(n=-1) == B.PA_ERR_INVALID_ARG
    assert w(src=B.PA_F16) == B.PA_ERR_INVALID_ARG          # no conversion into a bf16 pool
    assert w(layer=3) == B.PA_ERR_INVALID_ARG
    f8 = _cache(dtype=B.PA_FP8_E4M3, ks=0.1, vs=0.2)
    assert w(c=f8, src=B.PA_FP8_E4M3, n=0) == B.PA_OK
    assert w(c=_cache(bs=0)) == B.PA_ERR_INVALID_ARG


def test_host_copy_pairs_validated_before_any_copy(pa_lib):
    c = _cache(blocks=10)
    h = _cache(blocks=4)

    def run(pairs, direction=B.PA_COPY_H2D, dst=c, src=h):
        arr = (ctypes.c_int64 * (2 * len(pairs)))(*[x for p in pairs for x in p])
        return pa_lib.pa_copy_blocks(ctypes.byref(dst), ctypes.byref(src), arr, len(pairs),
                                     direction, None)
    assert run([(0, 10)]) == B.PA_ERR_INVALID_ARG            # dst out of range
    assert run([(4, 1)]) == B.PA_ERR_INVALID_ARG             # src out of range
    assert run([(0, 3), (1, 3)]) == B.PA_ERR_INVALID_ARG     # duplicate destination
    assert run([(0, 1)], direction=7) == B.PA_ERR_INVALID_ARG
    other = _cache(blocks=4, bs=8)
    assert run([(0, 1)], src=other) == B.PA_ERR_INVALID_ARG  # geometry differs
    assert run([], direction=B.PA_COPY_D2D) == B.PA_OK


def test_pool_layouts_block_major_and_layer_major(pa_lib):
    heads, bs, dim, nb, L = 8, 16, 128, 10, 4
    slab = heads * bs * dim

    def status(block_stride, layer_stride, blocks=nb, layers=L):
        c = B.PaKvCache(FAKE, FAKE, B.PA_BF16, blocks, layers, heads, bs, dim, block_stride,
                        layer_stride, 1.0, 1.0)
        return pa_lib.pa_copy_blocks(ctypes.byref(c), ctypes.byref(c), None, 0, B.PA_COPY_D2D, None)
    assert status(L * slab, slab) == B.PA_OK                       # block-major, packed
    assert status(L * (slab + 32) + 64, slab + 32) == B.PA_OK       # block-major, padded
    assert status(slab, nb * slab) == B.PA_OK                       # layer-major
    assert status(slab + 64, nb * (slab + 64)) == B.PA_OK           # layer-major, padded
    assert status(slab, slab) == B.PA_ERR_INVALID_ARG               # layers and blocks collide
    assert status(L * slab - 8, slab) == B.PA_ERR_INVALID_ARG       # blocks overlap
    assert status(slab, (nb - 1) * slab) == B.PA_ERR_INVALID_ARG    # layers overlap
    assert status(slab - 8, 0, layers=1) == B.PA_ERR_INVALID_ARG    # blocks overlap
    assert status(0, slab - 8, blocks=1) == B.PA_ERR_INVALID_ARG    # layers overlap
    assert status(0, 0, blocks=1, layers=1) == B.PA_OK


def test_host_pool_mapped_rejects_invalid_pool_without_device_calls(pa_lib):
    assert pa_lib.pa_host_pool_mapped(ctypes.byref(_cache(bs=0))) == 0
    assert pa_lib.pa_host_pool_mapped(None) == 0


def test_staged_copy_arguments_checked_before_device_work(pa_lib):
    heads, bs, dim, L = 8, 16, 128, 4
    slab = heads * bs * dim
    dev = B.PaKvCache(FAKE, FAKE, B.PA_BF16, 10, L, heads, bs, dim, slab, 10 * slab, 1.0, 1.0)
    host = B.PaKvCache(FAKE, FAKE, B.PA_BF16, 6, L, heads, bs, dim, L * slab, slab, 1.0, 1.0)
    one = 2 * L * slab * 2                              # bytes of one block, K and V
    assert pa_lib.pa_copy_staging_size(ctypes.byref(dev), 3) == 3 * one
    assert pa_lib.pa_copy_staging_size(ctypes.byref(dev), 0) == 0

    def run(pairs, direction=B.PA_COPY_D2H, dst=host, src=dev, staging=FAKE, nbytes=one):
        arr = (ctypes.c_int64 * (2 * len(pairs)))(*[x for p in pairs for x in p])
        return pa_lib.pa_copy_blocks_staged(ctypes.byref(dst), ctypes.byref(src), arr, len(pairs),
                                            direction, staging, nbytes, None)
    assert run([]) == B.PA_OK
    assert run([(0, 1)], direction=B.PA_COPY_D2D) == B.PA_ERR_INVALID_ARG
    assert run([(0, 1)], direction=B.PA_COPY_D2H_KERNEL) == B.PA_ERR_INVALID_ARG
    assert run([(0, 1)], staging=None) == B.PA_ERR_INVALID_ARG
    assert run([(0, 1)], staging=FAKE + 8) == B.PA_ERR_UNSUPPORTED
    assert run([(0, 1)], nbytes=one - 16) == B.PA_ERR_WORKSPACE
    assert run([(0, 6)]) == B.PA_ERR_INVALID_ARG             # host id out of range
    assert run([(0, 1), (2, 1)]) == B.PA_ERR_INVALID_ARG     # duplicate destination
    # the host pool's layers must be contiguous within a block
    assert run([(0, 1)], dst=dev, src=dev) == B.PA_ERR_UNSUPPORTED
    assert run([(1, 0)], direction=B.PA_COPY_H2D, dst=dev, src=host, nbytes=0) == \
        B.PA_ERR_WORKSPACE


def test_shared_decode_arguments(pa_lib):
    c = _cache()
    n = pa_lib.pa_decode_shared_workspace_size(ctypes.byref(c), 256, 32)
    assert n > pa_lib.pa_decode_workspace_size(ctypes.byref(c), 256, 32, 4000)
    f32 = _cache(dtype=B.PA_F32, dim=64, heads=4)
    assert pa_lib.pa_decode_shared_workspace_size(ctypes.byref(f32), 8, 4) == 0

    def run(cache=c, q_dtype=B.PA_BF16, reuse=0, ws=FAKE, nbytes=n, hq=32, S=256):
        return pa_lib.pa_decode_shared(ctypes.byref(cache), 0, FAKE, q_dtype, FAKE, FAKE, 8, FAKE,
                                       128, S, hq, ctypes.c_float(0.1), reuse, ws, nbytes, None)
    assert run(S=0) == B.PA_OK
    assert run(reuse=2) == B.PA_ERR_INVALID_ARG
    assert run(cache=f32, q_dtype=B.PA_F32, hq=4) == B.PA_ERR_UNSUPPORTED
    assert run(q_dtype=B.PA_F16) == B.PA_ERR_UNSUPPORTED      # bf16 pool, f16 queries
    assert run(hq=30) == B.PA_ERR_INVALID_ARG                 # not a multiple of the KV heads
    assert run(nbytes=n - 256) == B.PA_ERR_WORKSPACE
    assert run(ws=None) == B.PA_ERR_WORKSPACE
    assert run(ws=FAKE + 64) == B.PA_ERR_WORKSPACE


def test_decode_no_alloc_argument_errors(pa_lib):
    """pa_decode_no_alloc checks its arguments as pa_decode does, and refuses
    sizes whose workspace exceeds its fixed array, all before any HIP call."""
    c = _cache()

    def call(seqs=4, hq=32, max_ctx=100, q_dtype=B.PA_BF16, q=FAKE, out=FAKE):
        return pa_lib.pa_decode_no_alloc(ctypes.byref(c), 0, q, q_dtype, out, FAKE, 8, FAKE,
                                         max_ctx, seqs, hq, 0.1, None)
    assert call(seqs=0) == B.PA_OK
    assert call(hq=30) == B.PA_ERR_INVALID_ARG
    assert call(q=None) == B.PA_ERR_INVALID_ARG
    assert call(q_dtype=B.PA_F16) == B.PA_ERR_UNSUPPORTED           # bf16 pool, f16 queries
    assert call(hq=8 * 32) == B.PA_ERR_UNSUPPORTED
    # 8,192 sequences x 8 KV heads x groups of 4 need far more than the array
    big = pa_lib.pa_decode_workspace_size(ctypes.byref(c), 8192, 32, 4000)
    assert big > B.DECODE_NO_ALLOC_MAX_BYTES
    assert call(seqs=8192, max_ctx=4000) == B.PA_ERR_WORKSPACE
