"""Helpers shared by the oracle tests: tiny random paged workloads built
with the oracle's own write, and torch's scaled_dot_product_attention as an
independent dense reference (float64, CPU)."""

import numpy as np
import torch

from oracle import codecs, paged


def random_paged(rng, ctx_lens, hq, hkv, d, B, dtype=codecs.F32, spare=3,
                 pool_dtype=None, k_scale=1.0, v_scale=1.0):
    """Random Q/K/V of the given dtype, written at a random physical placement.

    Returns (geom, pool_k, pool_v, tables, ctx, q_codes, dense_k, dense_v)
    where dense_k/v are the per-sequence float64 values of the tokens as
    stored (list of [n][H_kv][D])."""
    pool_dtype = pool_dtype or dtype
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    nbs = [-(-int(n) // B) for n in ctx_lens]
    nblk = sum(nbs) + spare
    geom = paged.Geometry(nblk, 1, hkv, B, d)
    perm = rng.permutation(nblk)
    width = max(1, max(nbs) + 1)
    tables = np.full((len(ctx_lens), width), perm[-1] if spare else 0, dtype=np.int32)
    pos = 0
    slots = []
    for s, nb in enumerate(nbs):
        tables[s, :nb] = perm[pos:pos + nb]
        pos += nb
        t = np.arange(int(ctx_lens[s]))
        slots.append(tables[s][t // B].astype(np.int64) * B + t % B)
    slots = np.concatenate(slots) if slots else np.zeros(0, np.int64)
    T = int(ctx_lens.sum())
    def draw(shape):
        x = rng.standard_normal(shape).astype(np.float32)
        if dtype == codecs.F32:
            return x.view(np.uint32)
        tt = torch.from_numpy(x).to(torch.float16 if dtype == codecs.F16 else torch.bfloat16)
        return tt.view(torch.int16).numpy().view(np.uint16)
    q = draw((len(ctx_lens), hq, d))
    k = draw((T, hkv, d))
    v = draw((T, hkv, d))
    pk = np.full(geom.pool_elements(), codecs.NAN_CODE[pool_dtype], dtype=codecs.CODE_TYPE[pool_dtype])
    pv = pk.copy()
    pk, pv = paged.write_kv(pk, pv, geom, pool_dtype, 0, k, v, dtype, slots, k_scale, v_scale)
    starts = np.concatenate([[0], np.cumsum(ctx_lens)]).astype(int)
    dk, dv = [], []
    for s in range(len(ctx_lens)):
        kk = codecs.decode(codecs.encode_for_store(k[starts[s]:starts[s + 1]], dtype, pool_dtype, k_scale), pool_dtype)
        vv = codecs.decode(codecs.encode_for_store(v[starts[s]:starts[s + 1]], dtype, pool_dtype, v_scale), pool_dtype)
        if pool_dtype == codecs.FP8:
            kk = kk * np.float64(np.float32(k_scale))
            vv = vv * np.float64(np.float32(v_scale))
        dk.append(kk.reshape(-1, hkv, d))
        dv.append(vv.reshape(-1, hkv, d))
    return geom, pk, pv, tables, ctx_lens, q, dk, dv


def sdpa_reference(q64, dense_k, dense_v, scale):
    """torch.nn.functional.scaled_dot_product_attention in float64 on the
    dense tensors, KV heads repeated to the query heads."""
    S, hq, d = q64.shape
    out = np.zeros((S, hq, d))
    for s in range(S):
        k = torch.from_numpy(dense_k[s])       # [n, hkv, d]
        v = torch.from_numpy(dense_v[s])
        n, hkv, _ = k.shape
        if n == 0:
            continue
        g = hq // hkv
        kr = k.permute(1, 0, 2).repeat_interleave(g, dim=0).contiguous()   # [hq, n, d]
        vr = v.permute(1, 0, 2).repeat_interleave(g, dim=0).contiguous()
        qq = torch.from_numpy(q64[s]).unsqueeze(1)                          # [hq, 1, d]
        o = torch.nn.functional.scaled_dot_product_attention(qq, kr, vr, scale=scale)
        out[s] = o.squeeze(1).numpy()
    return out
