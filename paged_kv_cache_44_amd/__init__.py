"""Paged KV cache for MI355X: Python binding of the C ABI in include/pa.h.

The three operations are hand-written HIP kernels in ``libpa.so``; this
module only turns torch tensors into pointers, sizes and the current HIP
stream, and raises on a non-OK status. torch supplies device memory, pinned
host memory and streams.

    cache = KVCache(k_pool, v_pool, "bf16", num_blocks, 1, 8, 16, 128)
    write_kv(cache, 0, k_new, v_new, slot_mapping)
    out = decode(cache, 0, q, block_tables, context_lens, max_context_len, scale)
    copy_blocks(cache, cache, pairs, "d2d")

If the library has not been built, every call raises: there is no fallback.
"""

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _binding as B

DTYPES = {"f32": B.PA_F32, "f16": B.PA_F16, "bf16": B.PA_BF16, "fp8_e4m3": B.PA_FP8_E4M3}
TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
               "fp8_e4m3": torch.uint8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}

__all__ = ["KVCache", "write_kv", "decode", "decode_attend", "decode_merge", "decode_no_alloc",
           "decode_workspace_size", "decode_partition_tokens", "copy_blocks", "version"]


def _lib():
    return B.load_library()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _alloc_on(stream, fn):
    """Run the allocation `fn` with `stream` current, so torch's caching
    allocator ties the memory to the stream the kernels run on: once the
    tensor is dropped, the block is handed out again only in that stream's
    order (after the kernels that use it), never to another stream while
    they may still run."""
    if stream is None:
        return fn()
    with torch.cuda.stream(stream):
        return fn()


def dtype_name(t: torch.Tensor) -> str:
    for k, v in TORCH_DTYPE.items():
        if t.dtype == v:
            return k
    if t.dtype == torch.float8_e4m3fn:
        return "fp8_e4m3"
    raise ValueError(f"unsupported tensor dtype {t.dtype}")


@dataclass
class KVCache:
    """A K pool and a V pool (device, or pinned host for swap space).

    Element (layer l, block b, head h, slot o, dim d) sits at flat index
    b * block_stride + l * layer_stride + (h * block_size + o) * head_dim + d;
    strides default to the block-major packed layout.
    """
    k: torch.Tensor
    v: torch.Tensor
    dtype: str
    num_blocks: int
    num_layers: int
    num_kv_heads: int
    block_size: int
    head_dim: int
    block_stride: int = -1
    layer_stride: int = -1
    k_scale: float = 1.0
    v_scale: float = 1.0

    def __post_init__(self):
        if self.layer_stride < 0:
            self.layer_stride = self.num_kv_heads * self.block_size * self.head_dim
        if self.block_stride < 0:
            self.block_stride = self.num_layers * self.layer_stride
        need = self.required_elements()
        eb = ELEM_BYTES[self.dtype]
        for name, t in (("k", self.k), ("v", self.v)):
            if not t.is_contiguous():
                raise ValueError(f"pool {name} must be contiguous")
            if t.element_size() != eb:
                raise ValueError(f"pool {name} has {t.element_size()}-byte elements, "
                                 f"{self.dtype} needs {eb}")
            if t.numel() < need:
                raise ValueError(f"pool {name} holds {t.numel()} elements, geometry needs {need}")

    def required_elements(self) -> int:
        """Elements the geometry addresses (the last block's last element + 1)."""
        if self.num_blocks <= 0:
            return 0
        return ((self.num_blocks - 1) * self.block_stride + (self.num_layers - 1) * self.layer_stride
                + self.num_kv_heads * self.block_size * self.head_dim)

    @property
    def is_device(self) -> bool:
        return self.k.is_cuda and self.v.is_cuda

    @classmethod
    def empty(cls, dtype: str, num_blocks: int, num_layers: int, num_kv_heads: int,
              block_size: int, head_dim: int, device="cuda", pin_memory=False,
              k_scale=1.0, v_scale=1.0) -> "KVCache":
        n = num_blocks * num_layers * num_kv_heads * block_size * head_dim
        kw = dict(dtype=TORCH_DTYPE[dtype])
        if pin_memory:
            k = torch.empty(n, pin_memory=True, **kw)
            v = torch.empty(n, pin_memory=True, **kw)
        else:
            k = torch.empty(n, device=device, **kw)
            v = torch.empty(n, device=device, **kw)
        return cls(k, v, dtype, num_blocks, num_layers, num_kv_heads, block_size, head_dim,
                   k_scale=k_scale, v_scale=v_scale)

    def struct(self) -> B.PaKvCache:
        return B.PaKvCache(self.k.data_ptr(), self.v.data_ptr(), DTYPES[self.dtype],
                           self.num_blocks, self.num_layers, self.num_kv_heads,
                           self.block_size, self.head_dim, self.block_stride,
                           self.layer_stride, self.k_scale, self.v_scale)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _on_device(*ts):
    for t in ts:
        _need(t.is_cuda and t.is_contiguous(), "tensors must be contiguous device tensors")


def write_kv(cache: KVCache, layer: int, k: torch.Tensor, v: torch.Tensor,
             slot_mapping: torch.Tensor, stream=None) -> None:
    """Store k, v [T][H_kv][D] at their slots (int64 [T], negative = skip)."""
    _need(cache.is_device, "write_kv needs a device pool")
    _on_device(k, v, slot_mapping)
    T = int(slot_mapping.numel())
    shape = (T, cache.num_kv_heads, cache.head_dim)
    _need(tuple(k.shape) == shape and tuple(v.shape) == shape, f"k, v must be {shape}")
    _need(k.dtype == v.dtype, "k and v dtypes differ")
    _need(slot_mapping.dtype == torch.int64, "slot_mapping must be int64")
    c = cache.struct()
    st = _lib().pa_write_kv(ctypes.byref(c), layer, _ptr(k), _ptr(v), DTYPES[dtype_name(k)],
                            _ptr(slot_mapping), int(slot_mapping.numel()), _stream(stream))
    B.check(st, "pa_write_kv")


def decode_workspace_size(cache: KVCache, num_seqs: int, num_q_heads: int,
                          max_context_len: int) -> int:
    c = cache.struct()
    return int(_lib().pa_decode_workspace_size(ctypes.byref(c), num_seqs, num_q_heads,
                                               max_context_len))


def decode_partition_tokens(cache: KVCache, num_seqs: int, num_q_heads: int,
                            max_context_len: int) -> int:
    c = cache.struct()
    return int(_lib().pa_decode_partition_tokens(ctypes.byref(c), num_seqs, num_q_heads,
                                                 max_context_len))


def _decode_call(fn_name, cache, layer, q, block_tables, context_lens, max_context_len, scale,
                 out, workspace, stream):
    _need(cache.is_device, "decode needs a device pool")
    _need(q.dim() == 3 and q.shape[2] == cache.head_dim, "q must be [S][H_q][head_dim]")
    S, Hq, D = q.shape
    _on_device(q, block_tables, context_lens)
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S, "block_tables must be int32 [S][max_blocks]")
    _need(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (S,),
          "context_lens must be int32 [S]")
    if out is not None:
        _on_device(out)
        _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    if out is None:
        out = _alloc_on(stream, lambda: torch.empty_like(q))
    if workspace is None:
        n = decode_workspace_size(cache, S, Hq, max_context_len)
        workspace = _alloc_on(stream, lambda: torch.empty(max(n, 1), dtype=torch.uint8,
                                                          device=q.device))
    else:
        _on_device(workspace)
    c = cache.struct()
    st = getattr(_lib(), fn_name)(
        ctypes.byref(c), layer, _ptr(q), DTYPES[dtype_name(q)], _ptr(out), _ptr(block_tables),
        int(block_tables.shape[1]) if block_tables.dim() == 2 else 0, _ptr(context_lens),
        int(max_context_len), S, Hq, float(scale), _ptr(workspace), int(workspace.numel()),
        _stream(stream))
    B.check(st, fn_name)
    return out, workspace


def decode(cache: KVCache, layer: int, q: torch.Tensor, block_tables: torch.Tensor,
           context_lens: torch.Tensor, max_context_len: int, scale: float,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """Paged decode attention: q [S][H_q][D] -> out [S][H_q][D] (q's dtype)."""
    return _decode_call("pa_decode", cache, layer, q, block_tables, context_lens,
                        max_context_len, scale, out, workspace, stream)[0]


def decode_no_alloc(cache: KVCache, layer: int, q: torch.Tensor, block_tables: torch.Tensor,
                    context_lens: torch.Tensor, max_context_len: int, scale: float,
                    out: torch.Tensor, stream=None) -> torch.Tensor:
    """pa_decode_no_alloc: the result of :func:`decode` into the caller's
    ``out``, with the library's fixed device array as workspace (no
    allocation anywhere; see include/pa.h for the size limit and for calls
    that overlap on one GPU)."""
    _need(cache.is_device, "decode needs a device pool")
    _need(q.dim() == 3 and q.shape[2] == cache.head_dim, "q must be [S][H_q][head_dim]")
    S, Hq, D = q.shape
    _on_device(q, block_tables, context_lens, out)
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S, "block_tables must be int32 [S][max_blocks]")
    _need(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (S,),
          "context_lens must be int32 [S]")
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    c = cache.struct()
    st = _lib().pa_decode_no_alloc(
        ctypes.byref(c), layer, _ptr(q), DTYPES[dtype_name(q)], _ptr(out), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(context_lens), int(max_context_len), S, Hq,
        float(scale), _stream(stream))
    B.check(st, "pa_decode_no_alloc")
    return out


def decode_shared_workspace_size(cache: KVCache, num_seqs: int, num_q_heads: int) -> int:
    c = cache.struct()
    return int(_lib().pa_decode_shared_workspace_size(ctypes.byref(c), num_seqs, num_q_heads))


def decode_shared(cache: KVCache, layer: int, q: torch.Tensor, block_tables: torch.Tensor,
                  context_lens: torch.Tensor, max_context_len: int, scale: float,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  reuse_plan: bool = False, stream=None) -> torch.Tensor:
    """pa_decode_shared: the result of :func:`decode`, reading the prefix that
    runs of consecutive sequences share (same leading blocks in their tables)
    once per group of up to 32 / G of them. ``reuse_plan`` keeps the sharing
    found by the previous call with this workspace (same tables and lengths)."""
    _need(cache.is_device, "decode needs a device pool")
    _need(q.dim() == 3 and q.shape[2] == cache.head_dim, "q must be [S][H_q][head_dim]")
    S, Hq, D = q.shape
    _on_device(q, block_tables, context_lens)
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S, "block_tables must be int32 [S][max_blocks]")
    _need(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (S,),
          "context_lens must be int32 [S]")
    if out is None:
        out = _alloc_on(stream, lambda: torch.empty_like(q))
    else:
        _on_device(out)
        _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    if workspace is None:
        n = decode_shared_workspace_size(cache, S, Hq)
        workspace = _alloc_on(stream, lambda: torch.empty(max(n, 1), dtype=torch.uint8,
                                                          device=q.device))
    else:
        _on_device(workspace)
    c = cache.struct()
    st = _lib().pa_decode_shared(
        ctypes.byref(c), layer, _ptr(q), DTYPES[dtype_name(q)], _ptr(out), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(context_lens), int(max_context_len), S, Hq,
        float(scale), 1 if reuse_plan else 0, _ptr(workspace), int(workspace.numel()),
        _stream(stream))
    B.check(st, "pa_decode_shared")
    return out


def decode_attend(cache, layer, q, block_tables, context_lens, max_context_len, scale,
                  out, workspace, stream=None):
    """Phase 1 of :func:`decode` (partition attention). ``out`` and
    ``workspace`` are required: :func:`decode_merge` must see the same ones."""
    _need(out is not None and workspace is not None, "decode_attend needs out and workspace")
    _decode_call("pa_decode_attend", cache, layer, q, block_tables, context_lens,
                 max_context_len, scale, out, workspace, stream)


def decode_merge(cache, layer, q, block_tables, context_lens, max_context_len, scale,
                 out, workspace, stream=None):
    """Phase 2 of :func:`decode` (merge of partition partials): the ``out``
    and ``workspace`` that :func:`decode_attend` was given."""
    _need(out is not None and workspace is not None, "decode_merge needs out and workspace")
    _decode_call("pa_decode_merge", cache, layer, q, block_tables, context_lens,
                 max_context_len, scale, out, workspace, stream)


def prefill(cache: KVCache, layer: int, q: torch.Tensor, block_tables: torch.Tensor,
            context_lens: torch.Tensor, max_context_len: int, query_start_loc: torch.Tensor,
            max_query_len: int, scale: float, out: torch.Tensor = None, stream=None) -> torch.Tensor:
    """Paged prefill: causal attention of each sequence's newest positions
    (pa_prefill). q, out [num_q_tokens][H_q][D]; query_start_loc int32 [S+1]
    (device): rows query_start_loc[s] .. query_start_loc[s+1]-1 are positions
    context_lens[s] - n_s .. context_lens[s] - 1 of sequence s."""
    _need(cache.is_device, "prefill needs a device pool")
    _need(q.dim() == 3 and q.shape[2] == cache.head_dim, "q must be [T][H_q][head_dim]")
    T, Hq, D = q.shape
    _on_device(q, block_tables, context_lens, query_start_loc)
    S = int(context_lens.shape[0]) if context_lens.dim() == 1 else -1
    _need(context_lens.dtype == torch.int32 and context_lens.dim() == 1, "context_lens must be int32 [S]")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S, "block_tables must be int32 [S][max_blocks]")
    _need(query_start_loc.dtype == torch.int32 and tuple(query_start_loc.shape) == (S + 1,),
          "query_start_loc must be int32 [S + 1]")
    if out is None:
        out = _alloc_on(stream, lambda: torch.empty_like(q))
    else:
        _on_device(out)
        _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    c = cache.struct()
    st = _lib().pa_prefill(ctypes.byref(c), layer, _ptr(q), DTYPES[dtype_name(q)], _ptr(out),
                           _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens),
                           int(max_context_len), _ptr(query_start_loc), int(max_query_len), S, T,
                           Hq, float(scale), _stream(stream))
    B.check(st, "pa_prefill")
    return out


_DIRS = {"d2d": B.PA_COPY_D2D, "h2d": B.PA_COPY_H2D, "d2h": B.PA_COPY_D2H,
         "h2d_kernel": B.PA_COPY_H2D_KERNEL, "d2h_kernel": B.PA_COPY_D2H_KERNEL}


def copy_blocks(dst: KVCache, src: KVCache, pairs: torch.Tensor, direction: str = "d2d",
                stream=None) -> None:
    """Copy whole blocks: pairs int64 [N][2] = (src_block, dst_block); device
    memory for "d2d", host memory for "h2d" / "d2h" (the DMA engines) and
    "h2d_kernel" / "d2h_kernel" (one copy kernel; the host pool must be
    pinned and device-mapped)."""
    _need(pairs.dtype == torch.int64 and pairs.is_contiguous() and
          (pairs.numel() == 0 or (pairs.dim() == 2 and pairs.shape[1] == 2)),
          "pairs must be contiguous int64 [N][2]")
    if direction == "d2d":
        _need(dst.is_device and src.is_device and pairs.is_cuda, "d2d needs device pools and pairs")
    elif direction in ("h2d", "h2d_kernel"):
        _need(dst.is_device and not src.is_device and not pairs.is_cuda,
              "h2d copies a host pool into a device pool with host pairs")
    elif direction in ("d2h", "d2h_kernel"):
        _need(src.is_device and not dst.is_device and not pairs.is_cuda,
              "d2h copies a device pool into a host pool with host pairs")
    else:
        raise ValueError(f"unknown direction {direction!r}")
    d, s = dst.struct(), src.struct()
    n = int(pairs.shape[0]) if pairs.dim() == 2 else 0
    st = _lib().pa_copy_blocks(ctypes.byref(d), ctypes.byref(s), _ptr(pairs), n,
                               _DIRS[direction], _stream(stream))
    B.check(st, "pa_copy_blocks")


def copy_staging_size(pool: KVCache, num_pairs: int) -> int:
    """Bytes of staging that let :func:`copy_blocks_staged` move num_pairs
    blocks in one chunk."""
    c = pool.struct()
    return int(_lib().pa_copy_staging_size(ctypes.byref(c), int(num_pairs)))


def copy_blocks_staged(dst: KVCache, src: KVCache, pairs: torch.Tensor, direction: str,
                       staging: torch.Tensor, stream=None) -> None:
    """Swap through a device staging buffer (pa_copy_blocks_staged): "d2h"
    gathers the device blocks into ``staging`` and moves runs of host blocks
    by DMA; "h2d" the reverse. pairs int64 [N][2] in host memory."""
    _need(pairs.dtype == torch.int64 and pairs.is_contiguous() and not pairs.is_cuda and
          (pairs.numel() == 0 or (pairs.dim() == 2 and pairs.shape[1] == 2)),
          "pairs must be contiguous host int64 [N][2]")
    _need(direction in ("h2d", "d2h"), "direction must be 'h2d' or 'd2h'")
    dev_pool, host_pool = (dst, src) if direction == "h2d" else (src, dst)
    _need(dev_pool.is_device and not host_pool.is_device, f"{direction} pools on the wrong sides")
    _on_device(staging)
    d, s = dst.struct(), src.struct()
    n = int(pairs.shape[0]) if pairs.dim() == 2 else 0
    st = _lib().pa_copy_blocks_staged(ctypes.byref(d), ctypes.byref(s), _ptr(pairs), n,
                                      _DIRS[direction], _ptr(staging),
                                      staging.numel() * staging.element_size(), _stream(stream))
    B.check(st, "pa_copy_blocks_staged")


def host_pool_mapped(pool: KVCache) -> bool:
    """Whether the copy kernel can move blocks to and from this host pool."""
    c = pool.struct()
    return bool(_lib().pa_host_pool_mapped(ctypes.byref(c)))


def version() -> str:
    return _lib().pa_version().decode()
