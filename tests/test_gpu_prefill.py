"""Paged prefill on the GPU through the C ABI, checked against the oracle's
causal attention of each sequence's newest positions: whole prompts, later
chunks, single rows and empty query sets over every supported pool / query
dtype, head dim, group size and block size; a 1,500-token recompute (the
long FP8 workload's swap victim brought back by recomputation instead, "When
KV Capacity Runs Out", section "Recompute KV from token history"); invalid
device data."""

import zlib

import numpy as np
import pytest
import torch

import paged_kv_cache_44_amd as pa
import workloads
from oracle import codecs, paged
from tests.gpu_helpers import (DeviceState, TOL, codes_to_tensor, max_err, max_err_stored, say,
                               tensor_codes)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request, gpu):
    say(f"\n[gpu] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def _run(st, q_codes, qsl, tables=None, ctx=None, max_q=None, out_fill=None, out=None):
    wl = st.wl
    tables = wl.block_tables if tables is None else tables
    ctx = wl.context_lens if ctx is None else ctx
    q = codes_to_tensor(q_codes, wl.q_dtype)
    out = torch.empty_like(q) if out is None else out
    if out_fill is not None:
        out.view(torch.int16).fill_(out_fill)
    tt = torch.from_numpy(np.ascontiguousarray(tables, dtype=np.int32)).cuda()
    ct = torch.from_numpy(np.ascontiguousarray(ctx, dtype=np.int32)).cuda()
    qt = torch.from_numpy(np.ascontiguousarray(qsl, dtype=np.int32)).cuda()
    mq = int(np.max(np.diff(qsl))) if max_q is None else max_q
    pa.prefill(st.cache, wl.layer, q, tt, ct, int(np.max(ctx)), qt, max(mq, 1), wl.scale, out=out)
    torch.cuda.synchronize()
    return out


def _oracle(st, q_codes, qsl, tables=None, ctx=None, seqs=None, rows=None):
    wl = st.wl
    return paged.prefill(q_codes, wl.q_dtype, st.ok, st.ov, st.geom, wl.pool_dtype, wl.layer,
                         wl.block_tables if tables is None else tables,
                         wl.context_lens if ctx is None else ctx, qsl, wl.scale,
                         wl.k_scale, wl.v_scale, seqs=seqs, rows=rows)


COMBOS = [
    # pool,      q,      D,   G, B,  H_kv
    ("f16", "f16", 128, 1, 16, 3),
    ("f16", "f16", 64, 2, 8, 2),
    ("bf16", "bf16", 128, 4, 16, 2),
    ("bf16", "bf16", 64, 8, 32, 1),
    ("bf16", "bf16", 128, 2, 1, 1),
    ("bf16", "bf16", 128, 16, 16, 1),
    ("fp8_e4m3", "bf16", 128, 8, 16, 1),
    ("fp8_e4m3", "f16", 64, 4, 16, 2),
    ("fp8_e4m3", "bf16", 128, 1, 4, 2),
]


@pytest.mark.parametrize("pool,q,D,G,B,HKV", COMBOS)
def test_prefill_matches_oracle(pool, q, D, G, B, HKV):
    ctx = [1, 2, 15, 16, 17, 33, 100, 257, 40, 64]
    nq = [1, 2, 15, 16, 5, 33, 37, 257, 1, 0]        # whole, whole, ..., a chunk, ..., a decode row, none
    seed = zlib.crc32(repr((pool, q, D, G, B)).encode()) % 1000
    wl = workloads.custom(seed, ctx, pool_dtype=pool, q_dtype=q, num_q_heads=G * HKV,
                          num_kv_heads=HKV, head_dim=D, block_size=B)
    st = DeviceState(wl)
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    qc, qsl = workloads.prefill_queries(wl, nq, seed + 1)
    out = _run(st, qc, qsl)
    got = codecs.decode(tensor_codes(out), q)
    ref = _oracle(st, qc, qsl)
    assert np.all(np.isfinite(got))
    err = max_err(got, ref)
    ex = max_err_stored(got, ref, q, TOL[pool])
    say(f"{int(qsl[-1])} rows, max abs err {err:.3e}, beyond output rounding {ex:.3e}")
    assert ex <= TOL[pool]


@pytest.mark.parametrize("pool,q,D", [("bf16", "bf16", 128), ("f16", "f16", 64),
                                      ("fp8_e4m3", "bf16", 128)])
def test_prefill_output_alignment(pool, q, D):
    """Rows leave the kernel as 16-byte pieces when the output is 16-byte
    aligned and element by element otherwise: an output 4 bytes off that
    alignment (the least the call accepts) gets the same values bit for bit,
    and nothing around it is written."""
    ctx, nq = [1, 40, 257, 100], [1, 40, 200, 33]
    wl = workloads.custom(321, ctx, pool_dtype=pool, q_dtype=q, num_q_heads=8, num_kv_heads=2,
                          head_dim=D, block_size=16)
    st = DeviceState(wl)
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    qc, qsl = workloads.prefill_queries(wl, nq, 322)
    ref = _run(st, qc, qsl)
    assert ref.data_ptr() % 16 == 0
    n = ref.numel()
    buf = torch.full((n + 16,), -7, dtype=torch.int16, device=ref.device)
    out = buf[2:2 + n].view(ref.dtype).view(ref.shape)
    assert out.data_ptr() % 16 == 4
    _run(st, qc, qsl, out=out)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert bool((buf[:2] == -7).all()) and bool((buf[2 + n:] == -7).all())
    got = codecs.decode(tensor_codes(ref), q)
    assert max_err_stored(got, _oracle(st, qc, qsl), q, TOL[pool]) <= TOL[pool]


def test_prefill_recompute_long_fp8():
    """The long FP8 workload's 1,500-token victim recomputed: its keys and
    values written into fresh blocks, then one prefill pass over every
    position; sampled rows against the oracle."""
    wl = workloads.custom(505, [1500], pool_dtype="fp8_e4m3", q_dtype="bf16", num_q_heads=64,
                          num_kv_heads=8, head_dim=128, block_size=16)
    st = DeviceState(wl)
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    qc, qsl = workloads.prefill_queries(wl, [1500], 506)
    out = _run(st, qc, qsl)
    got = codecs.decode(tensor_codes(out), "bf16")
    rows = sorted({0, 1, 15, 16, 17, 255, 256, 511, 777, 1023, 1024, 1300, 1498, 1499} |
                  set(np.random.default_rng(7).choice(1500, 10, replace=False).tolist()))
    ref = _oracle(st, qc, qsl, rows=rows)
    assert np.all(np.isfinite(got))
    err = max_err(got, ref, rows=rows)
    ex = max_err_stored(got, ref, "bf16", TOL["fp8_e4m3"], rows=rows)
    say(f"rows {rows}: max abs err {err:.3e}, beyond output rounding {ex:.3e}")
    assert ex <= TOL["fp8_e4m3"]


def test_prefill_invalid_data():
    """A context shorter than its query rows and a table naming a block
    outside the pool give NaN rows for that sequence only; a sequence whose
    rows leave the packed query array is skipped (its rows untouched)."""
    ctx = [30, 20, 40, 25]
    nq = [10, 20, 5, 25]
    wl = workloads.custom(31, ctx, pool_dtype="bf16", q_dtype="bf16", num_q_heads=8,
                          num_kv_heads=2, head_dim=128, block_size=16)
    st = DeviceState(wl)
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    qc, qsl = workloads.prefill_queries(wl, nq, 32)
    tables = wl.block_tables.copy()
    tables[2, 1] = wl.num_blocks + 3                  # bad id inside the context of sequence 2
    ctx_bad = np.array(ctx, dtype=np.int32)
    ctx_bad[1] = 12                                   # fewer positions than its 20 rows
    qsl_bad = qsl.copy()
    qsl_bad[4] = qsl[4] + 7                           # sequence 3 runs past the packed rows
    out = _run(st, qc, qsl_bad, tables=tables, ctx=ctx_bad, max_q=32, out_fill=0x1234)
    codes = tensor_codes(out)
    got = codecs.decode(codes, "bf16")
    assert np.all(np.isnan(got[qsl[1]:qsl[2]])) and np.all(np.isnan(got[qsl[2]:qsl[3]]))
    assert np.all(codes[qsl[3]:qsl[4]] == 0x1234)
    ref = _oracle(st, qc, qsl, seqs=[0])
    assert max_err(got[qsl[0]:qsl[1]], ref[qsl[0]:qsl[1]]) <= TOL["bf16"]


def test_prefill_argument_errors():
    wl = workloads.custom(41, [8], pool_dtype="bf16", q_dtype="bf16", num_q_heads=4,
                          num_kv_heads=2, head_dim=128, block_size=16)
    st = DeviceState(wl)
    qc, qsl = workloads.prefill_queries(wl, [8], 42)
    q = codes_to_tensor(qc, "bf16")
    tt = torch.from_numpy(wl.block_tables).cuda()
    ct = torch.from_numpy(wl.context_lens).cuda()
    qt = torch.from_numpy(qsl).cuda()
    with pytest.raises(pa._binding.PaError):                    # fp32 queries are not supported here
        pa.prefill(st.cache, 0, q.float(), tt, ct, 8, qt, 8, 0.1)
    with pytest.raises(pa._binding.PaError):                    # bad layer
        pa.prefill(st.cache, 3, q, tt, ct, 8, qt, 8, 0.1)
    with pytest.raises(ValueError):                    # query_start_loc of the wrong length
        pa.prefill(st.cache, 0, q, tt, ct, 8, qt[:1], 8, 0.1)


LARGE_GRID = [
    # pool,      q,      D,   G, B
    ("bf16", "bf16", 128, 4, 16),
    ("f16", "f16", 64, 2, 8),
    ("fp8_e4m3", "bf16", 128, 8, 16),
    ("fp8_e4m3", "f16", 64, 1, 4),
    ("bf16", "bf16", 128, 16, 32),
    # blocks smaller than the 4 key rows (D = 128; 8 at D = 64) one wave
    # instruction stages straight into LDS: the rows of one instruction
    # come from different blocks
    ("f16", "f16", 128, 4, 2),
    ("bf16", "bf16", 64, 8, 1),
    ("bf16", "bf16", 128, 2, 4),
]


@pytest.mark.parametrize("pool,q,D,G,B", LARGE_GRID)
def test_prefill_large_grid_matches_oracle(pool, q, D, G, B):
    """A batch whose grid has more than four workgroups per compute unit
    (200 sequences x 8 KV heads), so the kernel runs its 32-key tiles at
    three waves per SIMD; whole prompts, later chunks and single rows, every
    row against the oracle."""
    rng = np.random.default_rng(zlib.crc32(repr((pool, q, D, G, B)).encode()) % 1000)
    ctx = rng.integers(1, 200, 200)
    nq = np.where(rng.random(200) < 0.5, ctx, np.maximum(1, (ctx * rng.random(200)).astype(np.int64)))
    wl = workloads.custom(int(rng.integers(1000)), ctx, pool_dtype=pool, q_dtype=q,
                          num_q_heads=8 * G, num_kv_heads=8, head_dim=D, block_size=B)
    st = DeviceState(wl)
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    qc, qsl = workloads.prefill_queries(wl, nq, 17)
    out = _run(st, qc, qsl)
    got = codecs.decode(tensor_codes(out), q)
    ref = _oracle(st, qc, qsl)
    assert np.all(np.isfinite(got))
    err = max_err(got, ref)
    ex = max_err_stored(got, ref, q, TOL[pool])
    say(f"{int(qsl[-1])} rows, max abs err {err:.3e}, with the output-rounding allowance {ex:.3e}")
    assert ex <= TOL[pool]


# (sequences, KV heads) for each workgroup order: pairs dealt round-robin
# over the 8 XCDs when the KV heads are a multiple of 8, (pair, row tile)
# items dealt in turn otherwise (including item counts that leave padding
# slots in the last round).
ORDERS = [(1, 3), (5, 1), (3, 5), (11, 3), (40, 1), (2, 8), (3, 16)]


@pytest.mark.parametrize("S,HKV", ORDERS)
def test_prefill_workgroup_orders(S, HKV):
    """Every workgroup order of the launch covers each (sequence, KV head,
    row tile) exactly once: prompts of mixed lengths, every row against the
    oracle."""
    rng = np.random.default_rng(31 * S + HKV)
    ctx = rng.integers(1, 300, S)
    ctx[0] = 300                                   # one long prompt sets the row tiles of all
    wl = workloads.custom(int(rng.integers(1000)), ctx, pool_dtype="bf16", q_dtype="bf16",
                          num_q_heads=4 * HKV, num_kv_heads=HKV, head_dim=128, block_size=16)
    st = DeviceState(wl)
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    qc, qsl = workloads.prefill_queries(wl, ctx, 19)
    out = _run(st, qc, qsl)
    got = codecs.decode(tensor_codes(out), "bf16")
    ref = _oracle(st, qc, qsl)
    assert np.all(np.isfinite(got))
    ex = max_err_stored(got, ref, "bf16", TOL["bf16"])
    say(f"{S} x {HKV} pairs, {int(qsl[-1])} rows, error with the output-rounding allowance {ex:.3e}")
    assert ex <= TOL["bf16"]
