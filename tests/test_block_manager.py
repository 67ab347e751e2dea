"""The native host block manager (pa_blocks.h) against the pages' worked
example and, operation by operation, against the oracle's block manager.

Worked example: "When KV Capacity Runs Out", Figures 1-5 (numbers in
tests/golden/worked_example.json). Differential test: random sequences of
admissions, appends, forks, copy-on-write, releases and swaps give identical
block tables, slots, copy pairs, swap pairs and free counts in both, and the
native manager refuses exactly the appends the oracle cannot complete. Host
code only: these run without a GPU."""

import copy
import json
import os
import random

import numpy as np
import pytest

from oracle.blocks import BlockPool, NoFreeBlock, Sequence
from paged_kv_cache_44_amd import _binding as B
from paged_kv_cache_44_amd.block_manager import BlockManager

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")))
NAME = {i: n for i, n in enumerate(GOLD["pool"]["names"])}
A, Bq = 1, 2


def _setup():
    bm = BlockManager(GOLD["pool"]["num_blocks"], GOLD["pool"]["block_size"], num_host_blocks=4)
    bm.add(A)
    bm.add(Bq)
    bm.append(A, GOLD["figure1"]["initial_positions"]["A"])
    bm.append(Bq, GOLD["figure1"]["initial_positions"]["B"])
    return bm


def _no_space(fn, *a):
    with pytest.raises(B.PaError) as e:
        fn(*a)
    assert e.value.status == B.PA_ERR_NO_SPACE


def test_figure1_pool_runs_dry_at_position_8():
    f1 = GOLD["figure1"]
    bm = _setup()
    ta, _ = bm.table(A)
    tb, _ = bm.table(Bq)
    assert len(ta) == len(tb) == f1["blocks_each"] and set(ta).isdisjoint(tb)
    assert bm.num_free() == f1["free_blocks"]
    bm.append(A)
    bm.append(Bq)
    assert (bm.table(A)[1], bm.table(Bq)[1]) == tuple(f1["after_one_step_positions"].values())
    assert bm.table(A)[1] == f1["position_needing_new_block"]
    assert bm.blocks_needed(A, 1) == 1 and bm.num_free() == 0
    _no_space(bm.append, A, 1)
    assert bm.table(A)[1] == 8 and len(bm.table(A)[0]) == 2     # unchanged


def test_figure2_release_newest_then_a_grows():
    f2 = GOLD["figure2"]
    bm = _setup()
    bm.append(A)
    bm.append(Bq)
    victim = bm.newest_running()
    assert victim == Bq                                  # the most recent arrival
    released = bm.table(Bq)[0]
    bm.release(Bq)
    assert [NAME[int(x)] for x in released] == f2["released_blocks_of_B"]
    assert bm.num_free() == f2["free_after_release"]
    slots, cow = bm.append(A)
    ta, n = bm.table(A)
    assert not cow and NAME[int(ta[-1])] == f2["block_given_to_A"]
    assert slots[0] == ta[-1] * 4                        # first slot of P2
    assert n == f2["A_positions"] and len(ta) == f2["A_blocks"]
    assert bm.num_free() == f2["free_after"]


def test_figure3_recompute_rebuilds_nine_positions_in_three_blocks():
    f3 = GOLD["figure3"]
    bm = _setup()
    bm.append(A)
    bm.append(Bq)
    bm.release(Bq)
    bm.release(A)
    bm.add(Bq)
    bm.append(Bq, f3["B_history_tokens"])                # one prefill over the history
    assert len(bm.table(Bq)[0]) == f3["blocks_after_recompute"]


def test_figure4_swap_out_and_restore_elsewhere():
    f4 = GOLD["figure4"]
    bm = _setup()
    bm.append(A)
    bm.append(Bq)
    pairs_out = bm.swap_out(Bq)
    assert len(pairs_out) == 2 and bm.num_free() == 0   # held until the copy is done
    assert bm.num_free(host=True) == 2
    bm.swap_out_done(Bq)
    assert bm.num_free() == 2 and bm.table(Bq) [1] == f4["swapped_positions"]
    bm.append(A)                                          # A takes one meanwhile
    bm.release(A)
    pairs_in = bm.swap_in(Bq)
    assert len(pairs_in) == f4["restored_blocks"]
    assert [int(h) for h, _ in pairs_in] == [int(h) for _, h in pairs_out]
    slots, _ = bm.append(Bq)
    tb, n = bm.table(Bq)
    assert len(tb) == f4["restored_blocks"] + f4["extra_block_for_x1"] and n == f4["positions_after"]
    assert slots[0] % 4 == 0
    assert sorted(tb[:2].tolist()) != sorted(pairs_out[:, 0].tolist())


def test_figure5_a_grows_to_twelve_within_three_blocks():
    f5 = GOLD["figure5"]
    bm = _setup()
    bm.append(A)
    bm.append(Bq)
    bm.release(Bq)
    bm.append(A)
    while bm.table(A)[1] < f5["A_grows_to"]:
        assert bm.blocks_needed(A, 1) == 0
        bm.append(A)
    assert len(bm.table(A)[0]) == f5["A_blocks"]
    bm.release(A)
    bm.add(Bq)
    bm.append(Bq, 9)
    assert len(bm.table(Bq)[0]) == f5["B_blocks_after_A_completes"]


def test_errors_change_nothing():
    bm = BlockManager(4, 4, num_host_blocks=1)
    bm.add(1)
    bm.append(1, 6)
    before = (bm.table(1)[0].tolist(), bm.table(1)[1], bm.num_free())
    for fn, args in [(bm.add, (1,)), (bm.fork, (9, 10)), (bm.release, (9,)),
                     (bm.swap_out_done, (1,)), (bm.swap_in, (1,))]:
        with pytest.raises(B.PaError) as e:
            fn(*args)
        assert e.value.status == B.PA_ERR_INVALID_ARG
    _no_space(bm.append, 1, 11)                           # needs 3 more blocks, 2 free
    _no_space(bm.swap_out, 1)                             # 2 blocks, 1 host block
    assert (bm.table(1)[0].tolist(), bm.table(1)[1], bm.num_free()) == before
    with pytest.raises(B.PaError):
        BlockManager(3, 4, order=[0, 0, 1])               # not a permutation


class _Mirror:
    """The oracle's block manager under caller ids, plus admission order."""

    def __init__(self, n, B_, order, nh):
        self.pool = BlockPool(n, B_, order)
        self.host = BlockPool(nh, B_)
        self.seqs = {}
        self.saved = {}                                    # id -> (host blocks, tokens)
        self.admitted = {}
        self.clock = 0


def test_differential_against_oracle_manager():
    for trial in range(60):
        rnd = random.Random(trial)
        nblk, Bs, nh = rnd.choice([4, 8, 13, 32]), rnd.choice([1, 2, 4, 16]), rnd.choice([0, 3, 16])
        order = rnd.sample(range(nblk), nblk)
        bm = BlockManager(nblk, Bs, order=order, num_host_blocks=nh)
        m = _Mirror(nblk, Bs, order, nh)
        next_id = 100
        for step in range(120):
            running = [i for i in m.seqs if i not in m.saved]
            op = rnd.choice(["add", "append", "append", "append", "fork", "cow", "release",
                             "swap", "swapin"])
            if op == "add" or not m.seqs:
                bm.add(next_id)
                m.seqs[next_id] = Sequence(m.pool)
                m.clock += 1
                m.admitted[next_id] = m.clock
                next_id += 1
            elif op == "append" and running:
                sid = rnd.choice(running)
                n = rnd.choice([1, 1, 2, 5, 17])
                trial_seq = copy.deepcopy((m.pool, m.seqs[sid]))
                try:
                    trial_seq[1].extend(n)
                    fits = True
                except NoFreeBlock:
                    fits = False
                if fits:
                    slots, cow = bm.append(sid, n)
                    ref_slots, ref_cow = m.seqs[sid].extend(n)
                    assert slots.tolist() == ref_slots and cow == ref_cow
                else:
                    _no_space(bm.append, sid, n)
            elif op == "fork" and running:
                sid = rnd.choice(running)
                bm.fork(sid, next_id)
                m.seqs[next_id] = m.seqs[sid].fork()
                m.clock += 1
                m.admitted[next_id] = m.clock
                next_id += 1
            elif op == "cow" and running:
                sid = rnd.choice(running)
                sq = m.seqs[sid]
                if sq.table and m.pool.refcount[sq.table[-1]] > 1 and m.pool.num_free:
                    assert bm.copy_last_block(sid) == sq.copy_last_block()
                elif not sq.table or m.pool.refcount[sq.table[-1]] <= 1:
                    # nothing shared to copy: both refuse and change nothing
                    with pytest.raises(ValueError):
                        sq.copy_last_block()
                    with pytest.raises(B.PaError) as e:
                        bm.copy_last_block(sid)
                    assert e.value.status == B.PA_ERR_INVALID_ARG
                else:
                    _no_space(bm.copy_last_block, sid)
            elif op == "release" and m.seqs:
                sid = rnd.choice(list(m.seqs))
                bm.release(sid)
                if sid in m.saved:
                    for hb in m.saved.pop(sid)[0]:
                        m.host.release(hb)
                else:
                    m.seqs[sid].free_all()
                del m.seqs[sid]
                m.admitted.pop(sid)
            elif op == "swap" and running:
                sid = m_victim = max(running, key=lambda i: m.admitted[i])
                assert bm.newest_running() == m_victim
                if len(m.seqs[sid].table) <= m.host.num_free:
                    pairs = bm.swap_out(sid)
                    ref_pairs, saved = m.seqs[sid].swap_out(m.host)
                    assert [tuple(p) for p in pairs.tolist()] == ref_pairs
                    bm.swap_out_done(sid)
                    m.seqs[sid].finish_swap_out()
                    m.saved[sid] = ([h for _, h in ref_pairs], saved)
                else:
                    _no_space(bm.swap_out, sid)
            elif op == "swapin" and m.saved:
                sid = rnd.choice(list(m.saved))
                hbs, saved = m.saved[sid]
                if len(hbs) <= m.pool.num_free:
                    pairs = bm.swap_in(sid)
                    ref = m.seqs[sid].swap_in(m.host, hbs, saved)
                    assert [tuple(p) for p in pairs.tolist()] == ref
                    del m.saved[sid]
                    m.clock += 1
                    m.admitted[sid] = m.clock
                else:
                    _no_space(bm.swap_in, sid)
            # state agrees after every operation
            assert bm.num_free() == m.pool.num_free and bm.num_free(host=True) == m.host.num_free
            for sid, sq in m.seqs.items():
                t, n = bm.table(sid)
                if sid in m.saved:
                    assert t.tolist() == [] and n == m.saved[sid][1]
                else:
                    assert t.tolist() == sq.table and n == sq.num_tokens
        bm.close()


def test_accounting_pins_on_the_native_manager():
    """Block math on the native manager: a 300-token request takes 19 blocks
    of 16 (304 slots, 4 wasted; "Continuous Batching and PagedAttention",
    section "Growth on demand"); 1,500 tokens take 94 ("41 · Preemption,
    Recomputation & KV Pressure", section 3); 100 decoding requests at B = 16
    draw 6.25 new blocks per step on average (same page, section 1);
    releasing a sequence frees every block it held and swapping it out moves
    every block (all or nothing, same page, section 2)."""
    bm = BlockManager(200, 16, num_host_blocks=120)
    bm.add(1)
    bm.append(1, 300)
    t, n = bm.table(1)
    assert len(t) == 19 and n == 300 and len(t) * 16 - n == 4
    bm.add(2)
    bm.append(2, 1500)
    assert len(bm.table(2)[0]) == 94 and bm.num_free() == 200 - 19 - 94
    pairs = bm.swap_out(2)
    assert len(pairs) == 94 and bm.num_free(host=True) == 120 - 94
    bm.swap_out_done(2)
    bm.release(1)
    assert bm.num_free() == 200 and bm.table(2)[0].shape == (0,)
    assert len(bm.swap_in(2)) == 94 and bm.num_free(host=True) == 120
    bm.release(2)
    assert bm.num_free() == 200

    bm = BlockManager(2000, 16)
    rng = np.random.default_rng(12)
    for s in range(100):
        bm.add(s)
        bm.append(s, int(rng.integers(1, 200)))
    drawn = []
    for step in range(16 * 8):
        before = bm.num_free()
        for s in range(100):
            bm.append(s, 1)
        drawn.append(before - bm.num_free())
    assert np.mean(drawn) == 100 / 16 == 6.25
