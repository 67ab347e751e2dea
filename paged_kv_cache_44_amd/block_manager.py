"""Python binding of the host block manager (pa_blocks.h): argument
marshalling only; every decision is made by the native library."""

import ctypes

import numpy as np

from . import _binding as B


class BlockManager:
    """Device blocks (FIFO free list in ``order``, default 0, 1, ...) and
    host blocks for swapped-out sequences; sequences named by int ids.
    Failing calls raise :class:`PaError` (``status == PA_ERR_NO_SPACE`` when
    blocks are short) and change nothing."""

    def __init__(self, num_blocks: int, block_size: int, order=None, num_host_blocks: int = 0):
        self._lib = B.load_library()
        self.block_size = block_size
        h = ctypes.c_void_p()
        o = None
        if order is not None:
            self._order = np.ascontiguousarray(order, dtype=np.int32)
            o = self._order.ctypes.data_as(ctypes.c_void_p)
        B.check(self._lib.pa_bm_create(num_blocks, block_size, o, num_host_blocks, ctypes.byref(h)),
                "pa_bm_create")
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def num_free(self, host: bool = False) -> int:
        return int(self._lib.pa_bm_num_free(self._h, 1 if host else 0))

    def add(self, seq: int) -> None:
        B.check(self._lib.pa_bm_add(self._h, seq), "pa_bm_add")

    def fork(self, parent: int, child: int) -> None:
        B.check(self._lib.pa_bm_fork(self._h, parent, child), "pa_bm_fork")

    def blocks_needed(self, seq: int, n: int = 1) -> int:
        return int(self._lib.pa_bm_blocks_needed(self._h, seq, n))

    def append(self, seq: int, n: int = 1):
        """Reserve n positions: (slots int64 [n], list of (src, dst) copies)."""
        slots = np.zeros(max(n, 1), dtype=np.int64)
        cow = np.zeros(2, dtype=np.int64)
        nc = ctypes.c_int32()
        B.check(self._lib.pa_bm_append(self._h, seq, n, slots.ctypes.data_as(ctypes.c_void_p),
                                       cow.ctypes.data_as(ctypes.c_void_p), ctypes.byref(nc)),
                "pa_bm_append")
        return slots[:n], [(int(cow[0]), int(cow[1]))] if nc.value else []

    def copy_last_block(self, seq: int):
        pair = np.zeros(2, dtype=np.int64)
        B.check(self._lib.pa_bm_copy_last_block(self._h, seq, pair.ctypes.data_as(ctypes.c_void_p)),
                "pa_bm_copy_last_block")
        return int(pair[0]), int(pair[1])

    def release(self, seq: int) -> None:
        B.check(self._lib.pa_bm_release(self._h, seq), "pa_bm_release")

    def table(self, seq: int):
        """(block ids int32 [num_blocks], num_tokens)."""
        nb, nt = ctypes.c_int32(), ctypes.c_int32()
        cap = 1 << 12
        while True:
            t = np.zeros(cap, dtype=np.int32)
            st = self._lib.pa_bm_table(self._h, seq, t.ctypes.data_as(ctypes.c_void_p), cap,
                                       ctypes.byref(nb), ctypes.byref(nt))
            if st == B.PA_OK:
                return t[:nb.value].copy(), int(nt.value)
            if cap >= 1 << 26:
                B.check(st, "pa_bm_table")
            cap *= 16

    def newest_running(self):
        s = ctypes.c_int64()
        st = self._lib.pa_bm_newest_running(self._h, ctypes.byref(s))
        return int(s.value) if st == B.PA_OK else None

    def _pairs(self, fn, seq: int, cap: int):
        pairs = np.zeros((max(cap, 1), 2), dtype=np.int64)
        n = ctypes.c_int32()
        B.check(getattr(self._lib, fn)(self._h, seq, pairs.ctypes.data_as(ctypes.c_void_p),
                                       max(cap, 1), ctypes.byref(n)), fn)
        return pairs[:n.value].copy()

    def swap_out(self, seq: int):
        """Plan (device block, host block) pairs; call swap_out_done after
        the copy has completed."""
        return self._pairs("pa_bm_swap_out", seq, len(self.table(seq)[0]))

    def swap_out_done(self, seq: int) -> None:
        B.check(self._lib.pa_bm_swap_out_done(self._h, seq), "pa_bm_swap_out_done")

    def swap_in(self, seq: int):
        """(host block, device block) pairs into fresh device blocks."""
        nt = self.table(seq)[1]
        return self._pairs("pa_bm_swap_in", seq, -(-nt // self.block_size))
