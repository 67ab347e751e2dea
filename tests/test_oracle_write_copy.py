"""Pins of the oracle's slot-mapped write and whole-block copy.

The layout check goes through numpy reshapes / strided views of the pool
(a route independent of the oracle's index arithmetic): element (block, layer,
head, slot, dim) of a block-major pool is ``pool5[block, layer, head, slot,
dim]``.
"""

import numpy as np
import pytest

from oracle import codecs, paged


def _view5(pool, geom):
    bs, ls = geom.strides()
    it = pool.itemsize
    return np.lib.stride_tricks.as_strided(
        pool, shape=(geom.num_blocks, geom.num_layers, geom.num_kv_heads, geom.block_size,
                     geom.head_dim),
        strides=(bs * it, ls * it, geom.block_size * geom.head_dim * it, geom.head_dim * it, it),
        writeable=False)


@pytest.mark.parametrize("layers,bstride_pad", [(1, 0), (3, 0), (2, 40)])
def test_write_lands_in_its_slot_and_nowhere_else(layers, bstride_pad):
    rng = np.random.default_rng(layers)
    B, H, D, nblk = 4, 3, 8, 7
    base = paged.Geometry(nblk, layers, H, B, D)
    bs, ls = base.strides()
    geom = paged.Geometry(nblk, layers, H, B, D, block_stride=bs + bstride_pad, layer_stride=ls)
    pool = np.full(geom.pool_elements(), codecs.NAN_CODE[codecs.F16], np.uint16)
    T = 13
    slots = rng.choice(nblk * B, size=T, replace=False).astype(np.int64)
    slots[3] = -1                                   # padding token
    k = rng.integers(0, 0x7C00, size=(T, H, D)).astype(np.uint16)
    v = rng.integers(0, 0x7C00, size=(T, H, D)).astype(np.uint16)
    layer = layers - 1
    pk, pv = paged.write_kv(pool, pool.copy(), geom, codecs.F16, layer, k, v, codecs.F16, slots)
    k5, v5 = _view5(pk, geom), _view5(pv, geom)
    touched = np.zeros(pk.shape, bool)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        b, o = divmod(int(s), B)
        assert np.array_equal(k5[b, layer, :, o, :], k[i])
        assert np.array_equal(v5[b, layer, :, o, :], v[i])
        for h in range(H):
            st = b * geom.block_stride + layer * ls + (h * B + o) * D
            touched[st:st + D] = True
    assert np.all(pk[~touched] == codecs.NAN_CODE[codecs.F16])
    assert np.all(pv[~touched] == codecs.NAN_CODE[codecs.F16])


def test_write_skips_negative_and_out_of_pool_slots_and_rejects_duplicates():
    geom = paged.Geometry(2, 1, 1, 4, 4)
    pool = np.zeros(geom.pool_elements(), np.uint32)
    k = np.ones((3, 1, 4), np.uint32)
    pk, _ = paged.write_kv(pool, pool, geom, codecs.F32, 0, k, k, codecs.F32, [-5, 8, 100])
    assert np.array_equal(pk, pool)
    with pytest.raises(ValueError):
        paged.write_kv(pool, pool, geom, codecs.F32, 0, k, k, codecs.F32, [1, 1, 2])


def test_fp8_write_stores_quantised_codes():
    rng = np.random.default_rng(3)
    geom = paged.Geometry(3, 1, 2, 4, 16)
    pool = np.full(geom.pool_elements(), 0x7F, np.uint8)
    x = rng.standard_normal((5, 2, 16)).astype(np.float32)
    src = x.view(np.uint32)
    slots = np.array([0, 5, 11, 2, 7])
    pk, pv = paged.write_kv(pool, pool.copy(), geom, codecs.FP8, 0, src, src, codecs.F32,
                            slots, k_scale=0.02, v_scale=0.5)
    k5, v5 = _view5(pk, geom), _view5(pv, geom)
    for i, s in enumerate(slots):
        b, o = divmod(int(s), 4)
        assert np.array_equal(k5[b, 0, :, o, :], codecs.quantize_e4m3(x[i], 0.02))
        assert np.array_equal(v5[b, 0, :, o, :], codecs.quantize_e4m3(x[i], 0.5))


def test_gather_after_write_round_trips():
    rng = np.random.default_rng(4)
    B, H, D = 4, 2, 8
    geom = paged.Geometry(6, 2, H, B, D)
    pool = np.full(geom.pool_elements(), codecs.NAN_CODE[codecs.BF16], np.uint16)
    table = np.array([4, 1, 5], dtype=np.int32)
    n = 10
    t = np.arange(n)
    slots = table[t // B].astype(np.int64) * B + t % B
    k = rng.integers(0, 0x7F00, size=(n, H, D)).astype(np.uint16)
    pk, pv = paged.write_kv(pool, pool.copy(), geom, codecs.BF16, 1, k, k, codecs.BF16, slots)
    got = paged.gather(pk, geom, codecs.BF16, 1, table, n)
    assert np.array_equal(got, codecs.decode(k, codecs.BF16))


def test_copy_blocks_brute_force():
    rng = np.random.default_rng(5)
    geom = paged.Geometry(8, 2, 2, 4, 4)
    src_k = rng.integers(0, 2**16, size=geom.pool_elements()).astype(np.uint16)
    src_v = rng.integers(0, 2**16, size=geom.pool_elements()).astype(np.uint16)
    pairs = [(1, 6), (3, 0), (2, 7)]
    dk, dv = paged.copy_blocks(src_k, src_v, geom, src_k, src_v, geom, pairs, same_pool=True)
    s5k, d5k = _view5(src_k, geom), _view5(dk, geom)
    s5v, d5v = _view5(src_v, geom), _view5(dv, geom)
    dst_set = {d for _, d in pairs}
    for b in range(8):
        if b not in dst_set:
            assert np.array_equal(d5k[b], s5k[b]) and np.array_equal(d5v[b], s5v[b])
    for s, d in pairs:
        assert np.array_equal(d5k[d], s5k[s]) and np.array_equal(d5v[d], s5v[s])


def test_copy_between_pools_with_different_strides():
    rng = np.random.default_rng(6)
    g1 = paged.Geometry(4, 2, 1, 4, 4)
    bs, ls = g1.strides()
    g2 = paged.Geometry(5, 2, 1, 4, 4, block_stride=bs + 8, layer_stride=ls + 4)
    src_k = rng.integers(0, 2**8, size=g1.pool_elements()).astype(np.uint8)
    dst = np.zeros(g2.pool_elements(), np.uint8)
    dk, dv = paged.copy_blocks(dst, dst, g2, src_k, src_k, g1, [(3, 4), (0, 1)])
    assert np.array_equal(_view5(dk, g2)[4], _view5(src_k, g1)[3])
    assert np.array_equal(_view5(dk, g2)[1], _view5(src_k, g1)[0])
    assert np.all(_view5(dk, g2)[[0, 2, 3]] == 0)


def test_copy_rejects_bad_pairs():
    geom = paged.Geometry(4, 1, 1, 2, 2)
    p = np.zeros(geom.pool_elements(), np.uint8)
    for pairs, same in (([(0, 1), (2, 1)], False), ([(0, 4)], False), ([(0, 1), (1, 2)], True)):
        with pytest.raises(ValueError):
            paged.copy_blocks(p, p, geom, p, p, geom, pairs, same_pool=same)
