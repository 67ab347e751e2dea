"""A tiny block manager (oracle; test infrastructure only).

Plain bookkeeping of a paged KV cache as the pages describe it, used to replay
their worked example and to drive scenario tests:

* a pool of fixed-size physical blocks with a free list ("Continuous Batching
  and PagedAttention", section "Fixed-size blocks make every free block
  usable": any free block serves any request);
* per-sequence block tables that fill left to right; a new block is taken
  only when the last one is full ("Efficient Memory Management for Large
  Language Model Serving with PagedAttention", block-table paragraph);
* reference counts for shared blocks and copy-on-write before writing into a
  shared block (same page, sampling and prefix paragraphs);
* release without zeroing; releasing exclusive blocks makes them allocatable
  again ("When KV Capacity Runs Out", section "Pause requests and release KV
  blocks", Figure 2);
* eviction is all-or-nothing ("41 · Preemption, Recomputation & KV Pressure",
  §2);
* swap-out copies a victim's blocks to host blocks before its device blocks
  are released, swap-in restores them into freshly allocated, possibly
  different, device blocks ("When KV Capacity Runs Out", section "Restore KV
  stored outside the GPU", Figure 4).

Slots are encoded as ``physical_block * block_size + offset``.
"""

from collections import deque


class NoFreeBlock(RuntimeError):
    """The pool has no free block left."""


class BlockPool:
    """Physical blocks, a FIFO free list and reference counts."""

    def __init__(self, num_blocks: int, block_size: int, order=None):
        self.num_blocks = num_blocks
        self.block_size = block_size
        ids = list(range(num_blocks)) if order is None else [int(b) for b in order]
        if sorted(ids) != list(range(num_blocks)):
            raise ValueError("order must be a permutation of the block ids")
        self.free_list = deque(ids)
        self.refcount = [0] * num_blocks

    @property
    def num_free(self) -> int:
        return len(self.free_list)

    def allocate(self) -> int:
        if not self.free_list:
            raise NoFreeBlock("no free block")
        b = self.free_list.popleft()
        self.refcount[b] = 1
        return b

    def share(self, b: int) -> None:
        if self.refcount[b] <= 0:
            raise ValueError("sharing a free block")
        self.refcount[b] += 1

    def release(self, b: int) -> None:
        """Drop one reference; at zero the block becomes allocatable again.
        Its contents are left as they are (no zeroing)."""
        if self.refcount[b] <= 0:
            raise ValueError("releasing a free block")
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free_list.append(b)


class Sequence:
    """One request's KV: a block table and the number of KV positions held."""

    def __init__(self, pool: BlockPool, name: str = ""):
        self.pool = pool
        self.name = name
        self.table = []
        self.num_tokens = 0

    # -- capacity ---------------------------------------------------------
    def blocks_for_next(self) -> int:
        """Free blocks the next append needs (0 or 1)."""
        B = self.pool.block_size
        if self.num_tokens % B == 0:
            return 1                       # last block full (or no block yet)
        if self.pool.refcount[self.table[-1]] > 1:
            return 1                       # shared partial block: copy first
        return 0

    def can_append(self) -> bool:
        return self.blocks_for_next() <= self.pool.num_free

    # -- growth -----------------------------------------------------------
    def append(self):
        """Reserve the slot of the next position.

        Returns ``(slot, cow)`` where ``cow`` is ``(src_block, dst_block)``
        when the last block was shared and had to be copied before writing,
        else ``None``. Raises :class:`NoFreeBlock` when a block is needed and
        none is free (nothing changes then).
        """
        B = self.pool.block_size
        cow = None
        if self.num_tokens % B == 0:
            self.table.append(self.pool.allocate())
        elif self.pool.refcount[self.table[-1]] > 1:
            new = self.pool.allocate()
            old = self.table[-1]
            self.pool.release(old)
            self.table[-1] = new
            cow = (old, new)
        slot = self.table[-1] * B + self.num_tokens % B
        self.num_tokens += 1
        return slot, cow

    def extend(self, n: int):
        """Append n positions; returns the list of slots and of CoW pairs."""
        slots, cows = [], []
        for _ in range(n):
            s, c = self.append()
            slots.append(s)
            if c is not None:
                cows.append(c)
        return slots, cows

    def slots(self):
        """Slot of every stored position, in position order."""
        B = self.pool.block_size
        return [self.table[t // B] * B + t % B for t in range(self.num_tokens)]

    # -- sharing ----------------------------------------------------------
    def fork(self, name: str = "") -> "Sequence":
        """A new sequence mapping the same physical blocks (parallel sampling
        from one prompt)."""
        child = Sequence(self.pool, name)
        for b in self.table:
            self.pool.share(b)
        child.table = list(self.table)
        child.num_tokens = self.num_tokens
        return child

    def copy_last_block(self):
        """Copy-on-write of the last block now, even if it is full (used for a
        workload that privatises the last shared block up front). Returns the
        (src, dst) pair: dst is a freshly allocated block (reference count 1)
        that replaces src as the table's last entry, and src loses exactly the
        one reference this sequence held. Only a shared block is copied ("a
        private copy for a writer to a shared block"); a sequence with no
        block, or whose last block it alone holds, raises ValueError."""
        if not self.table:
            raise ValueError("copy-on-write of a sequence that holds no block")
        if self.pool.refcount[self.table[-1]] <= 1:
            raise ValueError("copy-on-write of a block no other sequence shares")
        new = self.pool.allocate()
        old = self.table[-1]
        self.pool.release(old)
        self.table[-1] = new
        return (old, new)

    # -- release / preemption ---------------------------------------------
    def free_all(self):
        """Release every block at once (eviction is all or nothing). The
        token count drops to 0; the caller keeps the token history."""
        released = list(self.table)
        for b in released:
            self.pool.release(b)
        self.table = []
        self.num_tokens = 0
        return released

    def swap_out(self, host_pool: BlockPool):
        """Copy plan of a swap-out: one host block per device block. Returns
        ``(pairs, saved_tokens)`` with pairs = [(device_block, host_block)].
        The device blocks are released only by :meth:`finish_swap_out`, after
        the copy has completed."""
        pairs = [(b, host_pool.allocate()) for b in self.table]
        return pairs, self.num_tokens

    def finish_swap_out(self):
        return self.free_all()

    def swap_in(self, host_pool: BlockPool, host_blocks, saved_tokens: int):
        """Allocate fresh device blocks for the saved host blocks. Returns
        pairs [(host_block, device_block)]; host blocks are released."""
        if len(host_blocks) > self.pool.num_free:
            raise NoFreeBlock("not enough free blocks to swap in")
        pairs = []
        for hb in host_blocks:
            db = self.pool.allocate()
            self.table.append(db)
            pairs.append((hb, db))
            host_pool.release(hb)
        self.num_tokens = saved_tokens
        return pairs


def blocks_for_tokens(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of num_tokens positions occupies (the last may be
    partial)."""
    return -(-num_tokens // block_size)


def wasted_slots(num_tokens: int, block_size: int) -> int:
    """Allocated but unfilled slots: at most block_size - 1, in the last
    block ("Continuous Batching and PagedAttention", section "Growth on
    demand")."""
    return blocks_for_tokens(num_tokens, block_size) * block_size - num_tokens
