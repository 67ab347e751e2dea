"""Pins of the oracle's paged prefill (causal attention of each sequence's
newest positions).

Recompute runs the prompt and the generated tokens again as one prefill pass
("When KV Capacity Runs Out", section "Recompute KV from token history";
"KV Cache Preemption in vLLM", section "Swap versus recompute"); each position
attends to itself and the positions before it. The oracle is checked against
torch's scaled_dot_product_attention on the unpaged tensors, with
``is_causal`` for whole prefills and an explicit position mask for later
chunks, against closed forms, and against planted mistakes.
"""

import numpy as np
import pytest
import torch

from oracle import codecs, paged
from tests.oracle_helpers import random_paged


def _setup(rng, ctx, nq, hq, hkv, d, B, dtype=codecs.F32):
    """Random paged pool of the given contexts plus packed query rows, nq[s]
    of them for sequence s."""
    geom, pk, pv, tables, ctx, _, dk, dv = random_paged(rng, ctx, hq, hkv, d, B, dtype=dtype)
    qsl = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    x = rng.standard_normal((int(qsl[-1]), hq, d)).astype(np.float32)
    if dtype == codecs.F32:
        q = x.view(np.uint32)
    else:
        q = torch.from_numpy(x).to(torch.bfloat16 if dtype == codecs.BF16 else torch.float16)
        q = q.view(torch.int16).numpy().view(np.uint16)
    return geom, pk, pv, tables, ctx, qsl, q, dk, dv


def _sdpa(q64, qsl, dk, dv, scale, causal_full):
    """Dense reference: torch SDPA in float64, KV heads repeated; whole
    prefills use is_causal, chunks a boolean mask key <= position."""
    out = np.zeros_like(q64)
    for s in range(len(dk)):
        r0, r1 = int(qsl[s]), int(qsl[s + 1])
        if r1 == r0:
            continue
        k = torch.from_numpy(dk[s])
        v = torch.from_numpy(dv[s])
        n, hkv, d = k.shape
        hq = q64.shape[1]
        g = hq // hkv
        kr = k.permute(1, 0, 2).repeat_interleave(g, dim=0).contiguous()     # [hq, n, d]
        vr = v.permute(1, 0, 2).repeat_interleave(g, dim=0).contiguous()
        qq = torch.from_numpy(q64[r0:r1]).permute(1, 0, 2).contiguous()       # [hq, nq, d]
        nq = r1 - r0
        if causal_full and nq == n:
            o = torch.nn.functional.scaled_dot_product_attention(qq, kr, vr, is_causal=True, scale=scale)
        else:
            pos = torch.arange(n - nq, n).unsqueeze(1)
            mask = torch.arange(n).unsqueeze(0) <= pos                        # [nq, n]
            o = torch.nn.functional.scaled_dot_product_attention(qq, kr, vr, attn_mask=mask, scale=scale)
        out[r0:r1] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("hq,hkv,B,d", [(4, 4, 4, 16), (8, 2, 16, 32), (8, 1, 8, 16)])
def test_whole_prefill_matches_causal_sdpa(hq, hkv, B, d):
    rng = np.random.default_rng(hq * 10 + B)
    ctx = [1, 5, B, 2 * B + 3, 40]
    geom, pk, pv, tables, ctx, qsl, q, dk, dv = _setup(rng, ctx, ctx, hq, hkv, d, B)
    got = paged.prefill(q, codecs.F32, pk, pv, geom, codecs.F32, 0, tables, ctx, qsl, 0.3)
    ref = _sdpa(codecs.decode(q, codecs.F32), qsl, dk, dv, 0.3, causal_full=True)
    assert np.max(np.abs(got - ref)) < 1e-12


@pytest.mark.parametrize("dtype", [codecs.BF16, codecs.F16])
def test_chunked_prefill_matches_masked_sdpa(dtype):
    rng = np.random.default_rng(7)
    ctx = [9, 33, 64, 20, 1]
    nq = [3, 33, 1, 7, 0]                       # later chunks, a whole prefill, a decode step, none
    geom, pk, pv, tables, ctx, qsl, q, dk, dv = _setup(rng, ctx, nq, 8, 2, 32, 16, dtype=dtype)
    got = paged.prefill(q, dtype, pk, pv, geom, dtype, 0, tables, ctx, qsl, 0.17)
    ref = _sdpa(codecs.decode(q, dtype), qsl, dk, dv, 0.17, causal_full=False)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_first_position_returns_its_value_exactly():
    rng = np.random.default_rng(8)
    geom, pk, pv, tables, ctx, qsl, q, dk, dv = _setup(rng, [6, 11], [6, 11], 4, 2, 16, 4)
    got = paged.prefill(q, codecs.F32, pk, pv, geom, codecs.F32, 0, tables, ctx, qsl, 0.5)
    for s in range(2):
        for h in range(4):
            assert np.array_equal(got[qsl[s], h], dv[s][0, h // 2])


def test_last_row_is_the_decode_of_the_whole_context():
    rng = np.random.default_rng(9)
    geom, pk, pv, tables, ctx, qsl, q, dk, dv = _setup(rng, [13, 30], [4, 30], 8, 2, 16, 8)
    got = paged.prefill(q, codecs.F32, pk, pv, geom, codecs.F32, 0, tables, ctx, qsl, 0.25)
    last = q.reshape(-1, 8, 16)[qsl[1:] - 1]
    dec = paged.decode(last, codecs.F32, pk, pv, geom, codecs.F32, 0, tables, ctx, 0.25)
    assert np.array_equal(got[qsl[1:] - 1], dec)


def test_bad_query_rows_raise():
    rng = np.random.default_rng(10)
    geom, pk, pv, tables, ctx, qsl, q, dk, dv = _setup(rng, [4, 4], [2, 2], 2, 2, 8, 4)
    with pytest.raises(ValueError):
        paged.prefill(q, codecs.F32, pk, pv, geom, codecs.F32, 0, tables, np.array([1, 4]), qsl, 1.0)
    with pytest.raises(ValueError):
        paged.prefill(q, codecs.F32, pk, pv, geom, codecs.F32, 0, tables, ctx, np.array([0, 3, 2]), 1.0)


@pytest.mark.parametrize("kind", ["strict_causal", "position_from_start"])
def test_planted_prefill_mistakes_are_caught(monkeypatch, kind):
    """Two plausible mistakes fail the dense reference: a strict causal bound
    (a position not attending to itself) and chunk rows placed at the start of
    the context instead of its end."""
    rng = np.random.default_rng(11)
    geom, pk, pv, tables, ctx, qsl, q, dk, dv = _setup(rng, [12, 25], [5, 25], 4, 1, 8, 4)
    real = paged.attention

    def mutant(qrow, k, v, scale):
        if kind == "strict_causal":
            return real(qrow, k[:-1], v[:-1], scale)
        return real(qrow, k[:max(1, len(k) - 7)], v[:max(1, len(v) - 7)], scale)
    monkeypatch.setattr(paged, "attention", mutant)
    got = paged.prefill(q, codecs.F32, pk, pv, geom, codecs.F32, 0, tables, ctx, qsl, 0.3)
    ref = _sdpa(codecs.decode(q, codecs.F32), qsl, dk, dv, 0.3, causal_full=False)
    assert np.max(np.abs(got - ref)) > 1e-6
