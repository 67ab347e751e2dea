"""The seeded generators: determinism, shapes and the length mixes they
promise (the pages' workloads, stood in for by synthetic draws)."""

import numpy as np

import workloads


def _check_layout(wl):
    B = wl.block_size
    ctx = wl.context_lens
    nb = -(-ctx.astype(np.int64) // B)
    used = np.concatenate([wl.block_tables[s, :nb[s]] for s in range(wl.num_seqs)])
    assert used.min() >= 0 and used.max() < wl.num_blocks
    return used


def test_config1_shape():
    wl = workloads.config1()
    assert wl.num_blocks == 4 and wl.block_size == 4 and list(wl.context_lens) == [7, 8]
    used = _check_layout(wl)
    assert sorted(used.tolist()) == [0, 1, 2, 3]                 # disjoint blocks
    assert wl.q.shape == (2, 4, 64) and wl.write_k.shape == (15, 4, 64)
    assert wl.scale == 0.125
    assert len(set(wl.write_slots.tolist())) == 15


def test_generators_are_deterministic():
    a, b = workloads.config2(num_seqs=4), workloads.config2(num_seqs=4)
    assert np.array_equal(a.write_k, b.write_k) and np.array_equal(a.block_tables, b.block_tables)


def test_config2_lengths_and_pool():
    wl = workloads.config2()
    assert wl.context_lens.min() >= 128 and wl.context_lens.max() <= 2048
    used = _check_layout(wl)
    assert len(np.unique(used)) == len(used)                     # no sharing
    assert wl.num_blocks == -(-len(used) * 11 // 10)
    assert wl.spare_block not in set(used.tolist())


def test_config3_length_mix():
    rng = np.random.default_rng(0)
    lens = workloads.gqa_lengths(rng, 200000)
    assert abs(lens.mean() - (850 + 125.5)) < 3.0                # prompt mean 850 + answer mean
    wl = workloads.config3(num_seqs=16)
    _check_layout(wl)
    assert wl.num_q_heads == 32 and wl.num_kv_heads == 8


def test_config3_block_sizes_keep_the_lengths():
    # the block-size sweep's layouts: the same lengths, disjoint blocks, and
    # every slot inside the sequence's own blocks
    base = workloads.config3(num_seqs=16)
    for B in (8, 64, 256):
        wl = workloads.config3(num_seqs=16, block_size=B)
        assert wl.block_size == B and np.array_equal(wl.context_lens, base.context_lens)
        used = _check_layout(wl)
        assert len(np.unique(used)) == len(used)
        assert np.all(np.isin(wl.write_slots // B, used))


def test_config4_sharing_structure():
    wl = workloads.config4(groups=2, samples=8)
    used = _check_layout(wl)
    tb = wl.block_tables
    for g in range(2):
        rows = tb[g * 8:(g + 1) * 8]
        assert np.all(rows[:, :63] == rows[0, :63])              # shared prompt blocks
        last = rows[:, 63]
        assert len(set(last.tolist())) == 8                      # 7 copies + the original
        assert last[7] == wl.extra["prefix_blocks"][g][63]
    assert wl.extra["cow_pairs"].shape == (14, 2)
    assert np.all(wl.context_lens >= 1024 + 64) and np.all(wl.context_lens <= 1024 + 256)


def test_config4_partial_prefix_variant():
    wl = workloads.config4(groups=1, samples=4, prefix_tokens=1020, copied_samples=3)
    # the first private token lands in slot 12 of the (copied) last prompt block
    first_priv = wl.extra["num_prefix_tokens_written"]
    assert wl.write_slots[first_priv] % 16 == 12


def test_config5_victim():
    wl = workloads.config5(num_seqs=2, ctx_min=100, ctx_max=200)
    assert wl.extra["victim_blocks_before"].shape == (94,)
    assert set(wl.extra["victim_blocks_before"]).isdisjoint(set(wl.extra["victim_blocks_after"]))
    assert wl.context_lens[-1] == 1500
    assert 0 < wl.k_scale < 0.1 and 0 < wl.v_scale < 0.1
