"""Pins of the oracle's copy-on-write (oracle/blocks.py), worked by hand.

What the pages fix ("Efficient Memory Management for Large Language Model
Serving with PagedAttention", sampling paragraph; "Continuous Batching and
PagedAttention", section "Sharing, the part that goes beyond fixing what
broke"): samples of one prompt map the same physical blocks, each block
counting its holders; a sequence about to write into a block that others
also hold first gets a private copy in a newly allocated block, and the
shared block loses that one holder; a block with a single holder is written
in place. The expected values below are written out by hand for a six-block
pool, not computed by the oracle, and each planted mistake (the kinds a
bookkeeping slip produces) must fail at least one of them.
"""

import pytest

from oracle import blocks
from oracle.blocks import BlockPool, Sequence

# free-list order of the six-block pool: FIFO, so allocations take 3, 0, 5, 1 ...
ORDER = [3, 0, 5, 1, 4, 2]


def _forked(tokens: int):
    """A parent of `tokens` positions (block size 4) and one fork of it."""
    pool = BlockPool(6, 4, order=ORDER)
    parent = Sequence(pool, "parent")
    parent.extend(tokens)
    child = parent.fork("child")
    return pool, parent, child


def check_full_block_cow(seq_cls=Sequence):
    """As the shared-prefix workload does: the last shared block is full (8 tokens in blocks 3 and
    0, both held twice); the child privatises it up front."""
    pool = BlockPool(6, 4, order=ORDER)
    parent = seq_cls(pool, "parent")
    parent.extend(8)
    child = parent.fork("child")
    assert parent.table == [3, 0] and child.table == [3, 0]
    assert pool.refcount == [2, 0, 0, 2, 0, 0]
    pair = child.copy_last_block()
    assert pair == (0, 5)                     # src = old last block, dst = head of the free list
    assert child.table == [3, 5]              # last entry repointed, first kept
    assert parent.table == [3, 0]             # the sibling still maps the original
    assert pool.refcount == [1, 0, 0, 2, 0, 1]   # src lost exactly one holder; copy held once
    assert list(pool.free_list) == [1, 4, 2]  # src, still held, is not freed
    assert child.num_tokens == parent.num_tokens == 8
    # the child's next position opens a fresh block (its copy is full)
    slot, cow = child.append()
    assert (slot, cow) == (1 * 4 + 0, None) and child.table == [3, 5, 1]
    # the parent, now the only holder of block 0 (full), also opens a new block
    slot, cow = parent.append()
    assert (slot, cow) == (4 * 4 + 0, None) and parent.table == [3, 0, 4]
    # releasing the parent frees block 0 and 4 but only drops block 3 to one holder
    parent.free_all()
    assert pool.refcount == [0, 1, 0, 1, 0, 1] and list(pool.free_list) == [2, 0, 4]


def check_partial_block_cow(seq_cls=Sequence):
    """The shared last block is partial (6 tokens: block 0 holds positions
    4, 5): the child's append copies it and writes slot 2 of the copy; the
    parent, then the only holder, writes slot 2 of the original in place."""
    pool = BlockPool(6, 4, order=ORDER)
    parent = seq_cls(pool, "parent")
    parent.extend(6)
    child = parent.fork("child")
    slot, cow = child.append()
    assert cow == (0, 5) and slot == 5 * 4 + 2
    assert child.table == [3, 5] and parent.table == [3, 0]
    assert pool.refcount == [1, 0, 0, 2, 0, 1]
    slot, cow = parent.append()
    assert cow is None and slot == 0 * 4 + 2 and parent.table == [3, 0]
    assert pool.refcount == [1, 0, 0, 2, 0, 1] and list(pool.free_list) == [1, 4, 2]


def check_three_holders(seq_cls=Sequence):
    """Three holders: the first copy leaves the block with two, the second
    with one, and the last holder may no longer copy it (nothing shared)."""
    pool = BlockPool(6, 4, order=ORDER)
    a = seq_cls(pool, "a")
    a.extend(4)
    b, c = a.fork("b"), a.fork("c")
    assert pool.refcount[3] == 3
    assert b.copy_last_block() == (3, 0) and pool.refcount[3] == 2
    assert c.copy_last_block() == (3, 5) and pool.refcount[3] == 1
    assert (a.table, b.table, c.table) == ([3], [0], [5])
    with pytest.raises(ValueError):
        a.copy_last_block()
    assert a.table == [3] and pool.refcount == [1, 0, 0, 1, 0, 1]


def check_refusals(seq_cls=Sequence):
    """No block, or a block held once: refused, nothing changes."""
    pool = BlockPool(6, 4, order=ORDER)
    s = seq_cls(pool, "s")
    with pytest.raises(ValueError):
        s.copy_last_block()
    s.extend(3)
    with pytest.raises(ValueError):
        s.copy_last_block()
    assert s.table == [3] and pool.refcount == [0, 0, 0, 1, 0, 0]
    assert list(pool.free_list) == [0, 5, 1, 4, 2]


CHECKS = [check_full_block_cow, check_partial_block_cow, check_three_holders, check_refusals]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_oracle_cow_pins(check):
    check()


# ---------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin
# ---------------------------------------------------------------------------

class _NoRelease(Sequence):
    """Forgets to drop the source's reference."""
    def copy_last_block(self):
        if not self.table or self.pool.refcount[self.table[-1]] <= 1:
            raise ValueError("nothing shared")
        new = self.pool.allocate()
        old = self.table[-1]
        self.table[-1] = new
        return (old, new)


class _NoRepoint(Sequence):
    """Releases the source but keeps mapping it."""
    def copy_last_block(self):
        if not self.table or self.pool.refcount[self.table[-1]] <= 1:
            raise ValueError("nothing shared")
        new = self.pool.allocate()
        old = self.table[-1]
        self.pool.release(old)
        return (old, new)


class _DoubleRelease(Sequence):
    """Drops two references of the source (one too many)."""
    def copy_last_block(self):
        if not self.table or self.pool.refcount[self.table[-1]] <= 1:
            raise ValueError("nothing shared")
        new = self.pool.allocate()
        old = self.table[-1]
        self.pool.release(old)
        if self.pool.refcount[old] > 0:
            self.pool.release(old)
        self.table[-1] = new
        return (old, new)


class _SwappedPair(Sequence):
    """Returns the pair as (dst, src): the copy would run backwards."""
    def copy_last_block(self):
        old, new = Sequence.copy_last_block(self)
        return (new, old)


class _CopiesUnshared(Sequence):
    """Copies even a block it alone holds."""
    def copy_last_block(self):
        if not self.table:
            raise ValueError("no block")
        new = self.pool.allocate()
        old = self.table[-1]
        self.pool.release(old)
        self.table[-1] = new
        return (old, new)


class _FirstEntry(Sequence):
    """Repoints the first table entry instead of the last."""
    def copy_last_block(self):
        if not self.table or self.pool.refcount[self.table[-1]] <= 1:
            raise ValueError("nothing shared")
        new = self.pool.allocate()
        old = self.table[-1]
        self.pool.release(old)
        self.table[0] = new
        return (old, new)


class _AppendNoCow(Sequence):
    """Writes into a shared partial block without copying it."""
    def append(self):
        B = self.pool.block_size
        if self.num_tokens % B == 0:
            self.table.append(self.pool.allocate())
        slot = self.table[-1] * B + self.num_tokens % B
        self.num_tokens += 1
        return slot, None


class _AppendAlwaysCow(Sequence):
    """Copies a partial last block even when it is the only holder."""
    def append(self):
        B = self.pool.block_size
        cow = None
        if self.num_tokens % B == 0:
            self.table.append(self.pool.allocate())
        else:
            new = self.pool.allocate()
            old = self.table[-1]
            self.pool.release(old)
            self.table[-1] = new
            cow = (old, new)
        slot = self.table[-1] * B + self.num_tokens % B
        self.num_tokens += 1
        return slot, cow


MUTANTS = [_NoRelease, _NoRepoint, _DoubleRelease, _SwappedPair, _CopiesUnshared, _FirstEntry,
           _AppendNoCow, _AppendAlwaysCow]


def _fork_as(cls):
    """Sequence.fork builds a plain Sequence; give the fork the mutant's class."""
    def fork(self, name=""):
        child = cls(self.pool, name)
        for b in self.table:
            self.pool.share(b)
        child.table = list(self.table)
        child.num_tokens = self.num_tokens
        return child
    return fork


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda c: c.__name__)
def test_planted_cow_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(mutant, "fork", _fork_as(mutant))
    failed = 0
    for check in CHECKS:
        try:
            check(mutant)
        except (AssertionError, ValueError, blocks.NoFreeBlock, pytest.fail.Exception):
            failed += 1
    assert failed > 0, f"{mutant.__name__} passed every pin"
