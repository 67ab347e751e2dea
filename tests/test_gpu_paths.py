"""GPU parity of decode paths that the workload tests do not reach, through
the C ABI, each against the oracle:

* batches of more than 8,192 sequences, which pa_decode serves with the VALU
  kernel for 16-bit and FP8 pools;
* every E4M3 code through the matrix-core kernel's own conversions, for K
  (with bf16 and f16 queries) and for V;
* paged prefill at the benchmarked shape (the GQA bf16 workload's 256
  contexts, up to ~4,000 tokens, prefilled whole), on sampled rows;
* decode launched on a side stream while the default stream allocates.

"Efficient Memory Management for Large Language Model Serving with
PagedAttention", kernel paragraph: whatever the blocks' placement, the
result is that of ordinary attention over the same tokens.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_44_amd as pa
import workloads
from oracle import codecs
from tests.gpu_helpers import (DeviceState, TOL, codes_to_tensor, max_err, max_err_stored, say,
                               tensor_codes)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request, gpu):
    say(f"\n[gpu] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# more than 8,192 sequences: the VALU kernel with 16-bit and FP8 pools
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("pool,q", [("bf16", "bf16"), ("f16", "f16"), ("fp8_e4m3", "bf16"),
                                    ("fp8_e4m3", "f16")])
def test_decode_beyond_8192_sequences(pool, q):
    """9,000 sequences of 1..40 tokens (GQA 8 / 2 heads x 128, block 16): past
    the matrix-core kernel's batch limit, so the VALU kernel runs; sampled
    rows (and the first and last) against the oracle at the stated bound."""
    rng = np.random.default_rng(9000)
    ctx = rng.integers(1, 41, 9000)
    wl = workloads.custom(9001, ctx, pool_dtype=pool, q_dtype=q, num_q_heads=8, num_kv_heads=2,
                          head_dim=128, block_size=16)
    st = DeviceState(wl)
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    assert st.pools_equal_oracle()[0]
    # the VALU kernel splits contexts into partitions of 64+ tokens; the
    # matrix-core kernel reports 16
    assert pa.decode_partition_tokens(st.cache, wl.num_seqs, wl.num_q_heads,
                                      wl.max_context_len) != 16
    got = st.decode()
    assert np.array_equal(got, st.decode(split=True))
    seqs = sorted({0, 1, 8191, 8192, 8193, wl.num_seqs - 1} |
                  set(rng.choice(wl.num_seqs, 400, replace=False).tolist()))
    ref = st.oracle_decode(seqs=seqs)
    tol = TOL["fp8_e4m3"] if pool == "fp8_e4m3" else TOL[q]
    err = max_err(got, ref, rows=seqs)
    ex = max_err_stored(got, ref, q, tol, rows=seqs)
    say(f"{pool}/{q}: {len(seqs)} of {wl.num_seqs} rows, max abs err {err:.3e}, "
        f"with the output-rounding allowance {ex:.3e}")
    assert np.all(np.isfinite(got[seqs])) and ex <= tol


# ---------------------------------------------------------------------------
# every E4M3 code through the matrix-core kernel's conversions
# ---------------------------------------------------------------------------

H_Q, D, B = 8, 128, 16          # G = 8 query heads over one KV head: the matrix-core tile
E4M3_ONE = 0x38                 # code of 1.0 (exponent 7 = bias, mantissa 0)


def _fp8_workload(S, ctx, q_codes, q_dtype, seed):
    """S sequences of `ctx` tokens, one block each, at shuffled block ids of a
    pool with one spare block; softmax scale 1, k_scale = v_scale = 1."""
    perm = np.random.default_rng(seed).permutation(S + 1)
    return workloads.Workload(
        name="fp8_codes", seed=seed, pool_dtype="fp8_e4m3", src_dtype="bf16", q_dtype=q_dtype,
        num_q_heads=H_Q, num_kv_heads=1, head_dim=D, block_size=B, num_blocks=S + 1,
        num_layers=1, layer=0, scale=1.0, context_lens=np.full(S, ctx, np.int32),
        block_tables=perm[:S].astype(np.int32).reshape(S, 1), q=q_codes,
        write_k=np.zeros((0, 1, D), np.uint16), write_v=np.zeros((0, 1, D), np.uint16),
        write_slots=np.zeros(0, np.int64), k_scale=1.0, v_scale=1.0,
        spare_block=int(perm[S]))


def _set_pools(st, kpool, vpool):
    st.cache.k.copy_(torch.from_numpy(kpool))
    st.cache.v.copy_(torch.from_numpy(vpool))
    st.ok, st.ov = kpool, vpool


@pytest.mark.parametrize("q", ["bf16", "f16"])
def test_fp8_value_codes_exact_on_matrix_cores(q):
    """Context 1: each output row is its sequence's only value row, code by
    code, exactly (every E4M3 value is a bf16 and an f16 value; the single
    weight is 1). Two sequences hold the 256 codes in their 128 dims; NaN
    codes give NaN."""
    codes = np.arange(256, dtype=np.uint8).reshape(2, D)
    qv = np.random.default_rng(3).standard_normal((2, H_Q, D)).astype(np.float32)
    wl = _fp8_workload(2, 1, workloads.to_codes(qv, q), q, seed=11)
    st = DeviceState(wl)
    kp, vp = tensor_codes(st.cache.k), tensor_codes(st.cache.v)
    for s in range(2):
        base = int(wl.block_tables[s, 0]) * wl.block_stride()
        kp[base:base + D] = E4M3_ONE
        vp[base:base + D] = codes[s]
    _set_pools(st, kp, vp)
    got = st.decode()
    for s in range(2):
        want = codecs.E4M3_TABLE[codes[s]]
        for h in range(H_Q):
            assert np.array_equal(got[s, h], want, equal_nan=True), (s, h)
    ref = st.oracle_decode()
    assert np.array_equal(got, ref, equal_nan=True)


@pytest.mark.parametrize("q", ["bf16", "f16"])
def test_fp8_key_codes_on_matrix_cores(q):
    """Every E4M3 code as a key, through the score product's own conversion
    (to the query's 16-bit type). Sequence c holds two tokens: key 0 = code c
    in every dim, value 1; key 1 = 0, value 0. Query head h is alpha_c at one
    dim (8c + h mod 128, so the code is read at every dim position) and 0
    elsewhere, alpha_c the power of two that puts alpha_c * |value(c)| in
    [1, 2). The output is then sigma(alpha_c * value(c)) in every dim: a
    code read as a neighbouring one moves the score by at least 1/8, hence
    the output by more than twice the 4e-3 checked here; NaN codes give NaN
    rows."""
    S = 256
    val = codecs.E4M3_TABLE[np.arange(S)]
    finite = np.isfinite(val)
    alpha = np.ones(S)
    nz = finite & (val != 0)
    alpha[nz] = 2.0 ** -np.floor(np.log2(np.abs(val[nz])))
    qv = np.zeros((S, H_Q, D), np.float32)
    for c in range(S):
        for h in range(H_Q):
            qv[c, h, (8 * c + h) % D] = alpha[c]
    wl = _fp8_workload(S, 2, workloads.to_codes(qv, q), q, seed=12)
    assert np.array_equal(codecs.decode(wl.q, q), qv.astype(np.float64))   # alphas exact in q
    st = DeviceState(wl)
    kp, vp = tensor_codes(st.cache.k), tensor_codes(st.cache.v)
    for c in range(S):
        base = int(wl.block_tables[c, 0]) * wl.block_stride()
        kp[base:base + D] = c                    # key 0
        kp[base + D:base + 2 * D] = 0            # key 1
        vp[base:base + D] = E4M3_ONE             # value 0 = 1
        vp[base + D:base + 2 * D] = 0            # value 1 = 0
    _set_pools(st, kp, vp)
    got = st.decode()
    ref = st.oracle_decode()
    # the test's power: reading code c as c +- 1 (same sign, finite) moves the
    # oracle's own output by more than twice the bound
    sig = lambda z: 1.0 / (1.0 + np.exp(-z))
    for c in np.nonzero(nz)[0]:
        for d in (-1, 1):
            n = c + d
            if 0 <= n < S and np.isfinite(val[n]) and (n >> 7) == (c >> 7):
                assert abs(sig(alpha[c] * val[n]) - sig(alpha[c] * val[c])) > 8e-3, (c, n)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.all(np.isnan(got[~finite])) and np.all(np.isfinite(got[finite]))
    err = max_err(got[finite], ref[finite])
    say(f"{q}: max abs err over the {int(finite.sum())} finite codes {err:.3e}")
    assert err <= 4e-3


# ---------------------------------------------------------------------------
# prefill at the benchmarked shape
# ---------------------------------------------------------------------------

def test_prefill_at_benchmarked_shape_sampled_rows():
    """The GQA bf16 workload's 256 contexts (lognormal ~850-token prompts plus
    1..250 generated tokens, up to ~4,000) prefilled whole in one call, the
    queries drawn as the prefill benchmark draws them; sampled rows against
    the oracle at the bf16 bound: the longest sequence's first, middle and
    last rows, and rows at tile and chunk edges of 24 other sequences."""
    wl = workloads.make(3)
    st = DeviceState(wl)
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    ql = wl.context_lens.copy()
    qc, qsl = workloads.prefill_queries(wl, ql, 77)
    say(f"{wl.num_seqs} sequences, {int(qsl[-1])} query rows, longest context {wl.max_context_len}")
    dev = torch.device("cuda")
    q = codes_to_tensor(qc, wl.q_dtype)
    tables = torch.from_numpy(wl.block_tables).to(dev)
    ctx = torch.from_numpy(wl.context_lens).to(dev)
    qs = torch.from_numpy(qsl).to(dev)
    out = pa.prefill(st.cache, wl.layer, q, tables, ctx, wl.max_context_len, qs, int(ql.max()),
                     wl.scale)
    torch.cuda.synchronize()
    got = codecs.decode(tensor_codes(out), wl.q_dtype)
    del q, out
    rng = np.random.default_rng(78)
    longest = int(np.argmax(wl.context_lens))
    seqs = sorted({longest} | set(rng.choice(wl.num_seqs, 24, replace=False).tolist()))
    rows = []
    for s in seqs:
        n, r0 = int(wl.context_lens[s]), int(qsl[s])
        picks = {0, n - 1, n // 2, min(15, n - 1), min(16, n - 1), min(31, n - 1),
                 min(32, n - 1), int(rng.integers(n))}
        rows += [r0 + j for j in sorted(picks)]
    ref = st.oracle_prefill(qc, qsl, seqs=seqs, rows=rows)
    err = max_err(got, ref, rows=rows)
    ex = max_err_stored(got, ref, wl.q_dtype, TOL["bf16"], rows=rows)
    say(f"{len(rows)} rows of {len(seqs)} sequences: max abs err {err:.3e}, "
        f"with the output-rounding allowance {ex:.3e}")
    assert np.all(np.isfinite(got[rows])) and ex <= TOL["bf16"]


# ---------------------------------------------------------------------------
# a side stream
# ---------------------------------------------------------------------------

def test_decode_on_a_side_stream_while_the_default_stream_allocates():
    """decode(stream=side) lets the binding allocate the output and the
    workspace, and drops the workspace on return while the kernels still
    run on `side`. Right after each call the default stream allocates
    tensors of the same sizes and overwrites them: the allocator must not
    hand out the workspace there. Every output matches the oracle."""
    rng = np.random.default_rng(52)
    ctx = rng.integers(1500, 3000, 64)
    wl = workloads.custom(53, ctx, pool_dtype="bf16", q_dtype="bf16", num_q_heads=32,
                          num_kv_heads=8, head_dim=128, block_size=16)
    st = DeviceState(wl)
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    qt = codes_to_tensor(wl.q, "bf16")
    tt = torch.from_numpy(wl.block_tables).cuda()
    ct = torch.from_numpy(wl.context_lens).cuda()
    mc = int(ctx.max())
    nws = pa.decode_workspace_size(st.cache, wl.num_seqs, wl.num_q_heads, mc)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs, junk = [], []
    for _ in range(4):
        outs.append(pa.decode(st.cache, wl.layer, qt, tt, ct, mc, wl.scale, stream=side))
        w = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
        w.fill_(0xFF)                                    # NaN bytes
        o = torch.empty_like(qt)
        o.fill_(float("nan"))
        junk += [w, o]
    side.synchronize()
    torch.cuda.synchronize()
    ref = st.oracle_decode()
    for i, out in enumerate(outs):
        got = codecs.decode(tensor_codes(out), "bf16")
        ex = max_err_stored(got, ref, "bf16", TOL["bf16"])
        say(f"call {i}: error {ex:.3e}")
        assert np.all(np.isfinite(got)) and ex <= TOL["bf16"]
