"""Seeded random shapes against the oracle: plain decode (one call and the
two-launch form, which must agree bit for bit), shared-prefix decode and
prefill (whole prompts, later chunks, single rows, empty query sets),
over every supported pool / query dtype pair, head dim, group size, KV head
count (odd ones too), block size from 1 to 128, batch size and context mix
(short, long-tailed, one long sequence among tiny ones, empty rows). Each
case is small enough for the oracle; together they reach range lengths of
every parity at the wave level, segments cut at every kind of boundary, and
chunks that straddle blocks. The pages fix the result: paged attention
equals ordinary attention over the same tokens, whether or not blocks are
shared ("Efficient Memory Management for Large Language Model Serving with
PagedAttention", kernel and sampling paragraphs)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_44_amd as pa
import workloads
from oracle import codecs, paged
from tests.gpu_helpers import (DeviceState, TOL, codes_to_tensor, max_err, max_err_stored, say,
                               tensor_codes)

pytestmark = pytest.mark.gpu

PAIRS = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("fp8_e4m3", "bf16"),
         ("fp8_e4m3", "f16"), ("fp8_e4m3", "f32")]
BUDGET = 240_000            # sum(context) x query heads: keeps each oracle run short


@pytest.fixture(autouse=True)
def _announce(request, gpu):
    say(f"\n[gpu] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def _tol(pool, q):
    return TOL["fp8_e4m3"] if pool == "fp8_e4m3" else TOL[q]


def _err(got, ref, pool, q, rows):
    return max_err(got, ref, rows=rows) if q == "f32" else max_err_stored(got, ref, q, _tol(pool, q), rows=rows)


def _decode_case(seed):
    r = np.random.default_rng(7000 + seed)
    pool, q = PAIRS[int(r.integers(len(PAIRS)))]
    D = 64 if pool == "f32" else int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 4, 8]))
    hkv = int(r.choice([1, 2, 3, 4, 5, 8]))
    B = int(r.choice([1, 2, 4, 8, 16, 32, 64, 128]))
    S = int(r.integers(1, 49))
    kind = int(r.integers(5))
    if kind == 0:
        ctx = r.integers(1, 301, S)
    elif kind == 1:
        ctx = np.clip(r.lognormal(np.log(400.0), 0.8, S), 1, 3000).astype(np.int64)
    elif kind == 2:
        ctx = r.integers(1, 21, S)
        ctx[int(r.integers(S))] = int(r.integers(1000, 4001))
    elif kind == 3:
        ctx = r.integers(1, 21, S)
    else:
        ctx = r.integers(1, 2049, S)
    ctx = ctx.astype(np.int64)
    while ctx.sum() * G * hkv > BUDGET:
        ctx = np.maximum(ctx // 2, 1)
    zero = sorted(set(int(x) for x in r.integers(0, S, int(r.integers(0, 3)))))
    return pool, q, D, G, hkv, B, ctx, zero


@pytest.mark.parametrize("seed", range(24))
def test_random_shape_decode(seed):
    pool, q, D, G, hkv, B, ctx, zero = _decode_case(seed)
    say(f"pool {pool} q {q} D {D} G {G} H_kv {hkv} B {B} S {len(ctx)} "
        f"ctx sum {int(ctx.sum())} max {int(ctx.max())} empty rows {zero}")
    wl = workloads.custom(seed, ctx, pool_dtype=pool, q_dtype=q, num_q_heads=G * hkv,
                          num_kv_heads=hkv, head_dim=D, block_size=B)
    st = DeviceState(wl)
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    assert st.pools_equal_oracle()[0]
    run = wl.context_lens.copy()
    run[zero] = 0
    mc = int(wl.context_lens.max())
    got = st.decode(ctx=run, max_ctx=mc)
    assert np.array_equal(got, st.decode(ctx=run, max_ctx=mc, split=True))
    assert np.all(got[zero] == 0)
    live = [s for s in range(wl.num_seqs) if run[s] > 0]
    ref = st.oracle_decode(ctx=run, seqs=live)
    err = _err(got, ref, pool, q, live)
    say(f"max error {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= _tol(pool, q)


def _shared_case(seed):
    r = np.random.default_rng(9000 + seed)
    pool, q = [("f16", "f16"), ("bf16", "bf16"), ("fp8_e4m3", "bf16"), ("fp8_e4m3", "f16")][
        int(r.integers(4))]
    D = int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 4, 8]))
    hkv = int(r.choice([1, 2, 3, 4]))
    B = int(r.choice([4, 8, 16, 32, 64]))
    groups = []
    for _ in range(int(r.integers(1, 7))):
        prompt = int(r.integers(1, 700))
        groups.append((prompt, [int(x) for x in r.integers(0, 121, int(r.integers(1, 12)))]))
    def tokens(gs):
        return sum(p + t for p, priv in gs for t in priv) * G * hkv
    while tokens(groups) > BUDGET and len(groups) > 1:
        groups.pop()
    return pool, q, D, G, hkv, B, groups


@pytest.mark.parametrize("seed", range(8))
def test_random_shape_shared_decode(seed):
    pool, q, D, G, hkv, B, groups = _shared_case(seed)
    say(f"pool {pool} q {q} D {D} G {G} H_kv {hkv} B {B} groups {groups}")
    wl = workloads.shared_prefix(seed, groups, pool_dtype=pool, q_dtype=q, num_q_heads=G * hkv,
                                 num_kv_heads=hkv, head_dim=D, block_size=B)
    st = DeviceState(wl)
    for op in workloads.fill_plan(wl):
        if op[0] == "write":
            st.write(op[1], op[2], op[3])
        else:
            st.copy_d2d(op[1])
    qt = codes_to_tensor(wl.q, wl.q_dtype)
    tt = torch.from_numpy(np.ascontiguousarray(wl.block_tables, dtype=np.int32)).cuda()
    ct = torch.from_numpy(np.ascontiguousarray(wl.context_lens, dtype=np.int32)).cuda()
    mc = int(wl.context_lens.max())
    out = pa.decode_shared(st.cache, wl.layer, qt, tt, ct, mc, wl.scale)
    torch.cuda.synchronize()
    got = codecs.decode(tensor_codes(out), wl.q_dtype)
    ref = st.oracle_decode()
    err = max_err_stored(got, ref, q, _tol(pool, q))
    say(f"{wl.num_seqs} sequences, max error beyond output rounding {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= _tol(pool, q)
    # the same batch through the plain decode agrees within the tolerance too
    plain = st.decode()
    assert max_err_stored(plain, ref, q, _tol(pool, q)) <= _tol(pool, q)


def _prefill_case(seed):
    r = np.random.default_rng(11000 + seed)
    pool, q = [("f16", "f16"), ("bf16", "bf16"), ("fp8_e4m3", "bf16"), ("fp8_e4m3", "f16")][
        int(r.integers(4))]
    D = int(r.choice([64, 128]))
    G = int(r.choice([1, 2, 4, 8, 16]))
    hkv = int(r.choice([1, 2, 3]))
    B = int(r.choice([1, 2, 4, 8, 16, 32, 64, 128]))
    S = int(r.integers(1, 13))
    ctx = r.integers(1, 700, S)
    # query rows: the whole context, a later chunk, one row, or none
    nq = np.array([[c, int(r.integers(1, c + 1)), 1, 0][int(r.integers(4))] for c in ctx])
    while int((ctx * nq).sum()) * G * hkv > 20 * BUDGET:
        ctx = np.maximum(ctx // 2, 1)
        nq = np.minimum(nq, ctx)
    return pool, q, D, G, hkv, B, ctx, nq


@pytest.mark.parametrize("seed", range(10))
def test_random_shape_prefill(seed):
    pool, q, D, G, hkv, B, ctx, nq = _prefill_case(seed)
    say(f"pool {pool} q {q} D {D} G {G} H_kv {hkv} B {B} ctx {ctx.tolist()} rows {nq.tolist()}")
    wl = workloads.custom(seed, ctx, pool_dtype=pool, q_dtype=q, num_q_heads=G * hkv,
                          num_kv_heads=hkv, head_dim=D, block_size=B)
    st = DeviceState(wl)
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    qc, qsl = workloads.prefill_queries(wl, nq.tolist(), seed + 1)
    if int(qsl[-1]) == 0:
        return                                   # nothing to attend for
    qt = codes_to_tensor(qc, q)
    out = torch.empty_like(qt)
    tt = torch.from_numpy(np.ascontiguousarray(wl.block_tables, dtype=np.int32)).cuda()
    ct = torch.from_numpy(np.ascontiguousarray(wl.context_lens, dtype=np.int32)).cuda()
    qs = torch.from_numpy(np.ascontiguousarray(qsl, dtype=np.int32)).cuda()
    pa.prefill(st.cache, wl.layer, qt, tt, ct, int(ctx.max()), qs, max(int(np.max(np.diff(qsl))), 1),
               wl.scale, out=out)
    torch.cuda.synchronize()
    got = codecs.decode(tensor_codes(out), q)
    ref = paged.prefill(qc, q, st.ok, st.ov, st.geom, pool, wl.layer, wl.block_tables,
                        wl.context_lens, qsl, wl.scale, wl.k_scale, wl.v_scale)
    err = max_err_stored(got, ref, q, _tol(pool, q))
    say(f"{int(qsl[-1])} rows, max error beyond output rounding {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= _tol(pool, q)


@pytest.mark.parametrize("pool,q,D,hkv,B", [
    ("bf16", "bf16", 128, 8, 16),
    ("f16", "f16", 64, 1, 8),
    ("fp8_e4m3", "bf16", 128, 2, 32),
    ("fp8_e4m3", "f16", 64, 3, 1),
])
def test_group_of_16_decode(pool, q, D, hkv, B):
    """Sixteen query heads per KV head (the whole matrix-core tile holds one
    group, no padding columns)."""
    r = np.random.default_rng(hkv * 131 + B)
    S = 20
    ctx = np.concatenate([r.integers(1, 40, 10), r.integers(200, 1500, 10)]).astype(np.int64)
    while ctx.sum() * 16 * hkv > BUDGET:
        ctx = np.maximum(ctx // 2, 1)
    wl = workloads.custom(int(hkv * 17 + B), ctx, pool_dtype=pool, q_dtype=q,
                          num_q_heads=16 * hkv, num_kv_heads=hkv, head_dim=D, block_size=B)
    st = DeviceState(wl)
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    run = wl.context_lens.copy()
    run[3] = 0
    mc = int(wl.context_lens.max())
    got = st.decode(ctx=run, max_ctx=mc)
    assert np.array_equal(got, st.decode(ctx=run, max_ctx=mc, split=True))
    assert np.all(got[3] == 0)
    live = [s for s in range(S) if run[s] > 0]
    ref = st.oracle_decode(ctx=run, seqs=live)
    err = max_err_stored(got, ref, q, _tol(pool, q), rows=live)
    say(f"{S} sequences, max error beyond output rounding {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= _tol(pool, q)


@pytest.mark.parametrize("pool,q", [("bf16", "bf16"), ("fp8_e4m3", "f16"), ("f32", "f32")])
def test_block_size_256(pool, q):
    """The largest block size the pool takes: decode (both forms) and, for
    the matrix-core dtypes, prefill."""
    D = 64 if pool == "f32" else 128
    ctx = np.array([1, 255, 256, 257, 700, 1300, 40, 512])
    wl = workloads.custom(256, ctx, pool_dtype=pool, q_dtype=q, num_q_heads=8, num_kv_heads=2,
                          head_dim=D, block_size=256)
    st = DeviceState(wl)
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    assert st.pools_equal_oracle()[0]
    got = st.decode()
    assert np.array_equal(got, st.decode(split=True))
    ref = st.oracle_decode()
    err = _err(got, ref, pool, q, None)
    say(f"decode max error {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= _tol(pool, q)
    if pool == "f32":
        return
    nq = [1, 255, 3, 257, 1, 600, 40, 0]
    qc, qsl = workloads.prefill_queries(wl, nq, 257)
    qt = codes_to_tensor(qc, q)
    out = torch.empty_like(qt)
    tt = torch.from_numpy(np.ascontiguousarray(wl.block_tables, dtype=np.int32)).cuda()
    ct = torch.from_numpy(np.ascontiguousarray(wl.context_lens, dtype=np.int32)).cuda()
    qs = torch.from_numpy(np.ascontiguousarray(qsl, dtype=np.int32)).cuda()
    pa.prefill(st.cache, wl.layer, qt, tt, ct, int(ctx.max()), qs, max(nq), wl.scale, out=out)
    torch.cuda.synchronize()
    got = codecs.decode(tensor_codes(out), q)
    ref = paged.prefill(qc, q, st.ok, st.ov, st.geom, pool, wl.layer, wl.block_tables,
                        wl.context_lens, qsl, wl.scale, wl.k_scale, wl.v_scale)
    err = max_err_stored(got, ref, q, _tol(pool, q))
    say(f"prefill max error beyond output rounding {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= _tol(pool, q)


SMALL_BATCHES = [
    ("bf16", "bf16", 128, 4, 8, [1000]),
    ("bf16", "bf16", 128, 4, 8, [7000]),
    ("fp8_e4m3", "bf16", 128, 8, 2, [6000, 7000]),
    ("f16", "f16", 64, 1, 4, [1, 17, 30000]),
    ("f16", "f16", 128, 2, 1, [40000, 3, 60000]),
    ("bf16", "bf16", 64, 16, 2, [5000]),
    ("fp8_e4m3", "f16", 64, 2, 3, [1, 2, 3, 4, 5, 6, 7, 8]),
    ("f16", "f16", 128, 8, 4, [16, 17, 15, 1, 2000, 33]),
]


@pytest.mark.parametrize("case", range(len(SMALL_BATCHES)))
def test_small_batch_grids(case):
    """Batches of a few sequences: the call launches only as many workgroups
    as its chunk count needs (sized from max_context_len), and few long
    segments are merged one workgroup per (segment, KV head, query head).
    The same batch decoded with a 4x larger max_context_len (a larger grid,
    a different split) must match the oracle as well."""
    pool, q, D, G, hkv, ctx = SMALL_BATCHES[case]
    ctx = np.asarray(ctx, dtype=np.int64)
    assert ctx.sum() * G * hkv <= BUDGET
    say(f"pool {pool} q {q} D {D} G {G} H_kv {hkv} contexts {ctx.tolist()}")
    wl = workloads.custom(900 + case, ctx, pool_dtype=pool, q_dtype=q, num_q_heads=G * hkv,
                          num_kv_heads=hkv, head_dim=D, block_size=16)
    st = DeviceState(wl)
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    mc = int(ctx.max())
    live = list(range(len(ctx)))
    ref = st.oracle_decode(seqs=live)
    for bound in (mc, 4 * mc):
        got = st.decode(max_ctx=bound)
        assert np.array_equal(got, st.decode(max_ctx=bound, split=True))
        err = max_err_stored(got, ref, q, _tol(pool, q), rows=live)
        say(f"max_context_len {bound}: error beyond output rounding {err:.3e}")
        assert np.all(np.isfinite(got)) and err <= _tol(pool, q)
