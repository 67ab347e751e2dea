"""Pins of the oracle's paged decode.

The pages define the paged result as that of ordinary attention over the same
tokens ("Efficient Memory Management for Large Language Model Serving with
PagedAttention", kernel paragraph; "Continuous Batching and PagedAttention",
FAQ "Is PagedAttention an attention algorithm?"). The oracle is checked here
against torch's scaled_dot_product_attention on the unpaged tensors, against
closed forms, against independence from physical placement ("Continuous
Batching and PagedAttention", section "Fixed-size blocks ..."; "When KV
Capacity Runs Out", section "Restore KV stored outside the GPU": restored
blocks may sit elsewhere) and against never-written bytes ("When KV Capacity
Runs Out", section "Pause requests ...": release does not zero).
"""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import codecs, paged
from tests.oracle_helpers import random_paged, sdpa_reference


def _oracle(geom, pk, pv, tables, ctx, q, scale, dtype=codecs.F32, pool_dtype=None,
            k_scale=1.0, v_scale=1.0):
    return paged.decode(q, dtype, pk, pv, geom, pool_dtype or dtype, 0, tables, ctx, scale,
                        k_scale, v_scale)


@pytest.mark.parametrize("hq,hkv,B,d", [(4, 4, 4, 64), (8, 2, 16, 32), (8, 1, 8, 16),
                                        (6, 3, 2, 8)])
def test_matches_sdpa_on_unpaged_tensors(hq, hkv, B, d):
    rng = np.random.default_rng(hq * 100 + B)
    ctx = [1, B - 1 if B > 1 else 1, B, B + 1, 3 * B + 2, 47]
    geom, pk, pv, tables, ctx, q, dk, dv = random_paged(rng, ctx, hq, hkv, d, B)
    scale = 1.0 / np.sqrt(d)
    got = _oracle(geom, pk, pv, tables, ctx, q, scale)
    ref = sdpa_reference(codecs.decode(q, codecs.F32), dk, dv, scale)
    assert np.max(np.abs(got - ref)) < 1e-12


@pytest.mark.parametrize("dtype", [codecs.F16, codecs.BF16])
def test_matches_sdpa_16bit_storage(dtype):
    rng = np.random.default_rng(11)
    geom, pk, pv, tables, ctx, q, dk, dv = random_paged(rng, [5, 33, 64], 8, 2, 32, 16, dtype=dtype)
    got = _oracle(geom, pk, pv, tables, ctx, q, 0.17, dtype=dtype)
    ref = sdpa_reference(codecs.decode(q, dtype), dk, dv, 0.17)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_matches_sdpa_fp8_storage():
    rng = np.random.default_rng(12)
    geom, pk, pv, tables, ctx, q, dk, dv = random_paged(
        rng, [1, 17, 40], 8, 1, 32, 16, dtype=codecs.BF16, pool_dtype=codecs.FP8,
        k_scale=0.011, v_scale=0.013)
    got = paged.decode(q, codecs.BF16, pk, pv, geom, codecs.FP8, 0, tables, ctx, 0.2,
                       0.011, 0.013)
    ref = sdpa_reference(codecs.decode(q, codecs.BF16), dk, dv, 0.2)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_context_one_returns_first_value_exactly():
    rng = np.random.default_rng(2)
    geom, pk, pv, tables, ctx, q, dk, dv = random_paged(rng, [1, 1], 4, 2, 16, 4)
    got = _oracle(geom, pk, pv, tables, ctx, q, 0.3)
    for s in range(2):
        for h in range(4):
            assert np.array_equal(got[s, h], dv[s][0, h // 2])


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(3)
    geom, pk, pv, tables, ctx, q, dk, dv = random_paged(rng, [9, 30], 2, 2, 8, 4)
    q = np.zeros_like(q)
    got = _oracle(geom, pk, pv, tables, ctx, q, 1.0)
    for s in range(2):
        assert np.max(np.abs(got[s] - dv[s].mean(axis=0))) < 1e-15


def test_equal_keys_give_mean_and_equal_values_give_that_row():
    rng = np.random.default_rng(4)
    B, d, n = 4, 8, 11
    geom = paged.Geometry(4, 1, 1, B, d)
    table = np.array([[2, 0, 3]], dtype=np.int32)
    t = np.arange(n)
    slots = table[0][t // B].astype(np.int64) * B + t % B
    krow = rng.standard_normal(d).astype(np.float32)
    k = np.tile(krow, (n, 1)).reshape(n, 1, d).view(np.uint32)
    v = rng.standard_normal((n, 1, d)).astype(np.float32).view(np.uint32)
    pk = np.zeros(geom.pool_elements(), np.uint32)
    pk, pv = paged.write_kv(pk, pk.copy(), geom, codecs.F32, 0, k, v, codecs.F32, slots)
    q = rng.standard_normal((1, 1, d)).astype(np.float32).view(np.uint32)
    got = paged.decode(q, codecs.F32, pk, pv, geom, codecs.F32, 0, table, [n], 0.5)
    mean = codecs.decode(v, codecs.F32).reshape(n, d).mean(axis=0)
    assert np.max(np.abs(got[0, 0] - mean)) < 1e-15
    vrow = rng.standard_normal(d).astype(np.float32)
    v2 = np.tile(vrow, (n, 1)).reshape(n, 1, d).view(np.uint32)
    k2 = rng.standard_normal((n, 1, d)).astype(np.float32).view(np.uint32)
    pk, pv = paged.write_kv(pk, pk.copy(), geom, codecs.F32, 0, k2, v2, codecs.F32, slots)
    got = paged.decode(q, codecs.F32, pk, pv, geom, codecs.F32, 0, table, [n], 0.5)
    assert np.max(np.abs(got[0, 0] - vrow.astype(np.float64))) < 1e-15


def test_two_tokens_closed_form():
    rng = np.random.default_rng(5)
    geom, pk, pv, tables, ctx, q, dk, dv = random_paged(rng, [2], 1, 1, 16, 1)
    scale = 0.25
    got = _oracle(geom, pk, pv, tables, ctx, q, scale)[0, 0]
    qv = codecs.decode(q, codecs.F32)[0, 0]
    z0 = scale * float(np.dot(qv, dk[0][0, 0]))
    z1 = scale * float(np.dot(qv, dk[0][1, 0]))
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))
    ref = sig(z0 - z1) * dv[0][0, 0] + sig(z1 - z0) * dv[0][1, 0]
    assert np.max(np.abs(got - ref)) < 1e-14


def test_zero_context_gives_zero_row():
    rng = np.random.default_rng(6)
    geom, pk, pv, tables, ctx, q, dk, dv = random_paged(rng, [0, 5], 4, 2, 8, 4)
    got = _oracle(geom, pk, pv, tables, ctx, q, 0.3)
    assert np.array_equal(got[0], np.zeros_like(got[0]))
    assert np.all(np.isfinite(got[1]))


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(7)
    hq, hkv, d, B = 8, 2, 16, 4
    g = hq // hkv
    geom, pk, pv, tables, ctx, q, dk, dv = random_paged(rng, [13, 6], hq, hkv, d, B)
    got = _oracle(geom, pk, pv, tables, ctx, q, 0.4)
    # repeat every KV head g times in a second pool with hq KV heads
    geom2 = paged.Geometry(geom.num_blocks, 1, hq, B, d)
    k5 = pk.reshape(geom.num_blocks, 1, hkv, B, d)
    v5 = pv.reshape(geom.num_blocks, 1, hkv, B, d)
    pk2 = np.repeat(k5, g, axis=2).reshape(-1)
    pv2 = np.repeat(v5, g, axis=2).reshape(-1)
    got2 = paged.decode(q, codecs.F32, pk2, pv2, geom2, codecs.F32, 0, tables, ctx, 0.4)
    assert np.array_equal(got, got2)


def test_placement_invariance_bitwise():
    rng = np.random.default_rng(8)
    hq, hkv, d, B = 4, 2, 16, 4
    ctx = np.array([11, 16, 3], dtype=np.int32)
    T = int(ctx.sum())
    k = rng.standard_normal((T, hkv, d)).astype(np.float32).view(np.uint32)
    v = rng.standard_normal((T, hkv, d)).astype(np.float32).view(np.uint32)
    q = rng.standard_normal((3, hq, d)).astype(np.float32).view(np.uint32)
    nbs = [-(-int(n) // B) for n in ctx]
    nblk = sum(nbs) + 2
    outs = []
    for trial in range(3):
        perm = np.random.default_rng(100 + trial).permutation(nblk)
        tables = np.zeros((3, max(nbs)), np.int32)
        slots, pos = [], 0
        for s, nb in enumerate(nbs):
            tables[s, :nb] = perm[pos:pos + nb]
            pos += nb
            t = np.arange(int(ctx[s]))
            slots.append(tables[s][t // B].astype(np.int64) * B + t % B)
        geom = paged.Geometry(nblk, 1, hkv, B, d)
        pk = np.full(geom.pool_elements(), codecs.NAN_CODE[codecs.F32], np.uint32)
        pk, pv = paged.write_kv(pk, pk.copy(), geom, codecs.F32, 0, k, v, codecs.F32,
                                np.concatenate(slots))
        outs.append(paged.decode(q, codecs.F32, pk, pv, geom, codecs.F32, 0, tables, ctx, 0.3))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_never_written_bytes_do_not_matter():
    rng = np.random.default_rng(9)
    geom, pk, pv, tables, ctx, q, dk, dv = random_paged(rng, [5, 9, 2], 4, 4, 8, 4, spare=3)
    nan_out = _oracle(geom, pk, pv, tables, ctx, q, 0.3)
    # replace every never-written code by zeros, then by random codes
    written = pk != codecs.NAN_CODE[codecs.F32]
    for fill in (0, 0x3F800000):
        pk2 = np.where(written, pk, np.uint32(fill))
        pv2 = np.where(pv != codecs.NAN_CODE[codecs.F32], pv, np.uint32(fill))
        assert np.array_equal(_oracle(geom, pk2, pv2, tables, ctx, q, 0.3), nan_out)
    assert np.all(np.isfinite(nan_out))


def test_bad_tables_raise():
    geom = paged.Geometry(4, 1, 1, 4, 8)
    pool = np.zeros(geom.pool_elements(), np.uint32)
    q = np.zeros((1, 1, 8), np.uint32)
    with pytest.raises(ValueError):
        paged.decode(q, codecs.F32, pool, pool, geom, codecs.F32, 0, [[0, 1]], [9], 1.0)
    with pytest.raises(ValueError):
        paged.decode(q, codecs.F32, pool, pool, geom, codecs.F32, 0, [[0, 4]], [5], 1.0)


@settings(max_examples=60, deadline=None)
@given(B=st.sampled_from([1, 2, 4, 8, 16, 32]), d=st.sampled_from([8, 16, 64]),
       g=st.sampled_from([1, 2, 4, 8]), hkv=st.sampled_from([1, 2]),
       ctx=st.lists(st.integers(0, 300), min_size=1, max_size=3),
       seed=st.integers(0, 2**31 - 1))
def test_property_matches_sdpa(B, d, g, hkv, ctx, seed):
    rng = np.random.default_rng(seed)
    geom, pk, pv, tables, ctxa, q, dk, dv = random_paged(rng, ctx, g * hkv, hkv, d, B)
    scale = 1.0 / np.sqrt(d)
    got = _oracle(geom, pk, pv, tables, ctxa, q, scale)
    ref = sdpa_reference(codecs.decode(q, codecs.F32), dk, dv, scale)
    assert np.max(np.abs(got - ref), initial=0.0) < 1e-12


# ---------------------------------------------------------------------------
# planted mistakes: each mutation of the oracle must fail one of the pins
# ---------------------------------------------------------------------------

def _mutant_attention(kind):
    def attention(q, k, v, scale):
        Hq, D = q.shape
        n, Hkv, _ = k.shape
        g = Hq // Hkv
        out = np.zeros((Hq, D))
        if n == 0:
            return out
        for h in range(Hq):
            kvh = (h % Hkv) if kind == "head_map" else h // g
            z = scale * (k[:, kvh, :] @ q[h])
            if kind == "no_scale":
                z = k[:, kvh, :] @ q[h]
            if kind == "drop_last":
                z = z[:-1] if n > 1 else z
            p = np.exp(z - z.max())
            vv = v[:len(p), kvh, :]
            if kind == "no_norm":
                out[h] = p @ vv
            else:
                out[h] = (p @ vv) / p.sum()
        return out
    return attention


@pytest.mark.parametrize("kind", ["head_map", "no_scale", "drop_last", "no_norm"])
def test_planted_attention_mistakes_are_caught(monkeypatch, kind):
    rng = np.random.default_rng(21)
    geom, pk, pv, tables, ctx, q, dk, dv = random_paged(rng, [7, 20], 8, 2, 16, 4)
    monkeypatch.setattr(paged, "attention", _mutant_attention(kind))
    got = _oracle(geom, pk, pv, tables, ctx, q, 0.25)
    ref = sdpa_reference(codecs.decode(q, codecs.F32), dk, dv, 0.25)
    assert np.max(np.abs(got - ref)) > 1e-6


def test_planted_gather_mistake_is_caught(monkeypatch):
    """A gather that reads slot t % B from the wrong logical block (off by one
    in the table index) must fail the dense comparison."""
    rng = np.random.default_rng(22)
    geom, pk, pv, tables, ctx, q, dk, dv = random_paged(rng, [9, 12], 2, 2, 8, 4)
    real_index = geom.index

    def wrong_gather(pool, geom_, pool_dtype, layer, table_row, n, scale=1.0):
        t = np.arange(n)
        blk = np.asarray(table_row)[np.minimum((t + 1) // geom_.block_size,
                                               -(-n // geom_.block_size) - 1)]
        idx = real_index(blk[:, None, None], layer, np.arange(geom_.num_kv_heads)[None, :, None],
                         (t % geom_.block_size)[:, None, None],
                         np.arange(geom_.head_dim)[None, None, :])
        return codecs.decode(np.asarray(pool)[idx], pool_dtype)
    monkeypatch.setattr(paged, "gather", wrong_gather)
    got = _oracle(geom, pk, pv, tables, ctx, q, 0.3)
    ref = sdpa_reference(codecs.decode(q, codecs.F32), dk, dv, 0.3)
    assert not np.max(np.abs(got - ref)) < 1e-12
