"""The pages' block-accounting worked example, replayed with the oracle's
block manager; expected numbers are in tests/golden/worked_example.json
(transcribed from "When KV Capacity Runs Out", Figures 1-5)."""

import json
import os

import pytest

from oracle.blocks import BlockPool, NoFreeBlock, Sequence

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))
NAME = {i: n for i, n in enumerate(GOLD["pool"]["names"])}


def _setup():
    pool = BlockPool(GOLD["pool"]["num_blocks"], GOLD["pool"]["block_size"])
    a, b = Sequence(pool, "A"), Sequence(pool, "B")
    a.extend(GOLD["figure1"]["initial_positions"]["A"])
    b.extend(GOLD["figure1"]["initial_positions"]["B"])
    return pool, a, b


def test_figure1_pool_runs_dry_at_position_8():
    f1 = GOLD["figure1"]
    pool, a, b = _setup()
    assert len(a.table) == len(b.table) == f1["blocks_each"]
    assert set(a.table).isdisjoint(b.table)
    assert len(a.table) * pool.block_size == f1["allocated_slots_each"]
    assert pool.num_free == f1["free_blocks"]
    # with 0 free blocks both can still take their next input (empty slot)
    assert a.can_append() and b.can_append()
    a.append()
    b.append()
    assert (a.num_tokens, b.num_tokens) == tuple(f1["after_one_step_positions"].values())
    assert pool.num_free == f1["new_blocks_available"]
    # position 8 needs a third block and none is left
    assert a.num_tokens == f1["position_needing_new_block"]
    assert a.blocks_for_next() == 1 and not a.can_append() and not b.can_append()
    with pytest.raises(NoFreeBlock):
        a.append()
    assert a.num_tokens == 8 and len(a.table) == 2


def test_figure2_release_b_then_a_grows():
    f2 = GOLD["figure2"]
    pool, a, b = _setup()
    a.append(), b.append()
    # skipping B's execution alone frees nothing
    assert pool.num_free == f2["skip_only_free_blocks"]
    released = b.free_all()
    assert [NAME[x] for x in released] == f2["released_blocks_of_B"]
    assert pool.num_free == f2["free_after_release"]
    slot, cow = a.append()
    assert cow is None
    assert NAME[a.table[-1]] == f2["block_given_to_A"]
    assert slot == a.table[-1] * pool.block_size + 0          # first slot of P2
    assert a.num_tokens == f2["A_positions"] and len(a.table) == f2["A_blocks"]
    assert pool.num_free == f2["free_after"]
    assert NAME[pool.free_list[0]] == f2["remaining_free_block"]


def test_figure3_recompute_rebuilds_nine_positions_in_three_blocks():
    f3 = GOLD["figure3"]
    pool, a, b = _setup()
    a.append(), b.append()
    history = ["p%d" % i for i in range(7)] + ["x0", "x1"]
    assert len(history) == f3["B_history_tokens"]
    assert b.num_tokens == f3["B_kv_positions_before"]
    b.free_all()
    a.free_all()          # A completes later and releases its blocks
    b.extend(len(history))  # one prefill pass over the whole history
    assert len(b.table) == f3["blocks_after_recompute"] and b.num_tokens == 9


def test_figure4_swap_out_and_restore_elsewhere():
    f4 = GOLD["figure4"]
    pool, a, b = _setup()
    a.append(), b.append()
    host = BlockPool(4, pool.block_size)
    pairs_out, saved = b.swap_out(host)
    assert saved == f4["swapped_positions"] and len(pairs_out) == 2
    old_blocks = [d for d, _ in pairs_out]
    # blocks are released only after the copy finished
    assert pool.num_free == 0
    b.finish_swap_out()
    assert pool.num_free == 2
    a.append()            # A takes one of them meanwhile
    a.free_all()          # ... and later completes
    pairs_in = b.swap_in(host, [h for _, h in pairs_out], saved)
    assert len(pairs_in) == f4["restored_blocks"]
    assert b.num_tokens == 8
    slot, _ = b.append()  # x1 needs a third block
    assert len(b.table) == f4["restored_blocks"] + f4["extra_block_for_x1"]
    assert b.num_tokens == f4["positions_after"]
    assert slot % pool.block_size == 0
    # the restored blocks are not the ones the data left (A used one of them
    # in between), which the block table absorbs
    assert sorted(b.table[:2]) != sorted(old_blocks)


def test_figure5_a_grows_to_twelve_within_three_blocks():
    f5 = GOLD["figure5"]
    pool, a, b = _setup()
    a.append(), b.append()
    b.free_all()
    a.append()
    assert a.num_tokens == f5["A_grows_from"]
    while a.num_tokens < f5["A_grows_to"]:
        assert a.blocks_for_next() == 0
        a.append()
    assert len(a.table) == f5["A_blocks"]
    a.free_all()
    assert pool.num_free == 4
    b.extend(9)
    assert len(b.table) == f5["B_blocks_after_A_completes"]


def test_copy_on_write_of_shared_partial_block():
    pool = BlockPool(8, 4)
    parent = Sequence(pool)
    parent.extend(6)                       # 2 blocks, last one half full
    kids = [parent.fork() for _ in range(2)]
    assert pool.refcount[parent.table[-1]] == 3
    slot, cow = kids[0].append()
    assert cow is not None and cow[0] == parent.table[-1]
    assert kids[0].table[-1] == cow[1] and slot == cow[1] * 4 + 2
    assert pool.refcount[parent.table[-1]] == 2
    assert pool.refcount[parent.table[0]] == 3   # full prompt block stays shared
    kids[1].append()
    _, cow = parent.append()
    assert cow is None                       # last owner writes in place


def test_eviction_releases_every_block():
    pool = BlockPool(6, 4)
    s = Sequence(pool)
    s.extend(10)
    s.free_all()
    assert s.table == [] and pool.num_free == 6
