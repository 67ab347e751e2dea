"""Paged KV-cache operations, plainly (oracle; test infrastructure only).

A pool is a flat numpy array of storage codes plus a :class:`Geometry`.
Element (layer l, block b, kv head h, slot o, dim d) sits at

    b * block_stride + l * layer_stride + (h * block_size + o) * head_dim + d

Blocks are fixed-size and may sit anywhere ("Continuous Batching and
PagedAttention", section "Fixed-size blocks make every free block usable").
Positions are 0-based: token t lives in logical block t // block_size at slot
t % block_size ("When KV Capacity Runs Out", section "Running out of KV space
during generation", Figure 1: positions count from 0). The summary page of
"Efficient Memory Management for Large Language Model Serving with
PagedAttention" numbers tokens from 1 in its kernel paragraph; both readings
describe the same blocks.

Where the pages are silent this module takes these readings:
* slot = physical_block * block_size + offset, int64, negative = skip;
* a context length counts the token the current step has just written;
* context length 0 gives an all-zero output row;
* query head h uses KV head h // (H_q / H_kv) (contiguous GQA groups);
* the caller passes the softmax scale; no mask beyond the context length;
* an FP8 code means code_value * scale (one fp32 scale per K or V tensor);
* slots never written and blocks never referenced hold undefined bytes that
  must never influence a result;
* duplicate destination slots / blocks in one call are caller errors.
"""

from dataclasses import dataclass

import numpy as np

from . import codecs


@dataclass(frozen=True)
class Geometry:
    num_blocks: int
    num_layers: int
    num_kv_heads: int
    block_size: int
    head_dim: int
    block_stride: int = -1      # elements; -1 = block-major default
    layer_stride: int = -1      # elements; -1 = dense default

    def strides(self):
        ls = self.layer_stride if self.layer_stride >= 0 else \
            self.num_kv_heads * self.block_size * self.head_dim
        bs = self.block_stride if self.block_stride >= 0 else self.num_layers * ls
        return bs, ls

    def pool_elements(self) -> int:
        """Smallest flat length that holds every element of the pool."""
        bs, ls = self.strides()
        last = (self.num_blocks - 1) * bs + (self.num_layers - 1) * ls + \
            self.num_kv_heads * self.block_size * self.head_dim
        return int(last)

    def index(self, block, layer, head, slot, dim):
        """Flat element index (numpy-broadcasting)."""
        bs, ls = self.strides()
        block = np.asarray(block, dtype=np.int64)
        return (block * bs + np.int64(layer) * ls
                + (np.asarray(head, dtype=np.int64) * self.block_size
                   + np.asarray(slot, dtype=np.int64)) * self.head_dim
                + np.asarray(dim, dtype=np.int64))


# --------------------------------------------------------------------------
# slot-mapped write
# --------------------------------------------------------------------------

def write_kv(pool_k, pool_v, geom: Geometry, pool_dtype: str, layer: int,
             k_src, v_src, src_dtype: str, slot_mapping,
             k_scale: float = 1.0, v_scale: float = 1.0):
    """Return copies of the pools after storing tokens at their slots.

    For token i with slot_mapping[i] >= 0: block = slot // B, offset = slot % B;
    K[i, h, :] and V[i, h, :] go to (layer, block, h, offset, :) for every KV
    head h ("When KV Capacity Runs Out", Figure 2: the KV of position 8 goes
    into the first slot of the block just attached; section "Restore KV stored
    outside the GPU": processing x1 writes its new KV into a fresh block).
    Tokens with a negative slot are skipped; slots beyond the pool are skipped.
    Same dtype: bytes are stored unchanged. FP8 pool: the quantiser of
    :func:`codecs.quantize_e4m3`.
    """
    B, H, D = geom.block_size, geom.num_kv_heads, geom.head_dim
    slots = np.asarray(slot_mapping, dtype=np.int64).reshape(-1)
    T = slots.shape[0]
    k_src = np.asarray(k_src).reshape(T, H, D)
    v_src = np.asarray(v_src).reshape(T, H, D)
    if not 0 <= layer < geom.num_layers:
        raise ValueError("layer out of range")
    live = slots >= 0
    live &= slots < np.int64(geom.num_blocks) * B
    live_slots = slots[live]
    if np.unique(live_slots).shape[0] != live_slots.shape[0]:
        raise ValueError("duplicate destination slots in one write")
    out_k = np.array(pool_k, copy=True)
    out_v = np.array(pool_v, copy=True)
    if live_slots.shape[0] == 0:
        return out_k, out_v
    kc = codecs.encode_for_store(k_src[live], src_dtype, pool_dtype, k_scale)
    vc = codecs.encode_for_store(v_src[live], src_dtype, pool_dtype, v_scale)
    blk = live_slots // B
    off = live_slots % B
    idx = geom.index(blk[:, None, None], layer, np.arange(H)[None, :, None],
                     off[:, None, None], np.arange(D)[None, None, :])
    out_k[idx] = kc
    out_v[idx] = vc
    return out_k, out_v


# --------------------------------------------------------------------------
# whole-block copy
# --------------------------------------------------------------------------

def copy_blocks(dst_k, dst_v, dst_geom: Geometry, src_k, src_v, src_geom: Geometry,
                pairs, same_pool: bool = False):
    """Return copies of the destination pools after dst[d] <- src[s] for every
    pair (s, d): K and V, every layer, head, slot and dim, as raw codes.

    Copy-on-write gives a writer to a shared block its own copy ("Efficient
    Memory Management for Large Language Model Serving with PagedAttention",
    sampling paragraph); swap moves a victim's blocks out and back, possibly
    into other blocks ("When KV Capacity Runs Out", section "Restore KV stored
    outside the GPU").
    """
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    for g1, g2 in ((dst_geom, src_geom),):
        if (g1.num_layers, g1.num_kv_heads, g1.block_size, g1.head_dim) != \
           (g2.num_layers, g2.num_kv_heads, g2.block_size, g2.head_dim):
            raise ValueError("pools differ in geometry")
    src_ids, dst_ids = pairs[:, 0], pairs[:, 1]
    if np.any(src_ids < 0) or np.any(src_ids >= src_geom.num_blocks) or \
       np.any(dst_ids < 0) or np.any(dst_ids >= dst_geom.num_blocks):
        raise ValueError("block id out of range")
    if np.unique(dst_ids).shape[0] != dst_ids.shape[0]:
        raise ValueError("duplicate destination blocks")
    if same_pool and np.intersect1d(src_ids, dst_ids).shape[0] != 0:
        raise ValueError("a block is both source and destination")
    out_k = np.array(dst_k, copy=True)
    out_v = np.array(dst_v, copy=True)
    H, B, D = src_geom.num_kv_heads, src_geom.block_size, src_geom.head_dim
    for s, d in pairs:
        for layer in range(src_geom.num_layers):
            si = src_geom.index(s, layer, 0, 0, 0)
            di = dst_geom.index(d, layer, 0, 0, 0)
            n = H * B * D
            out_k[di:di + n] = np.asarray(src_k)[si:si + n]
            out_v[di:di + n] = np.asarray(src_v)[si:si + n]
    return out_k, out_v


# --------------------------------------------------------------------------
# gather + attention
# --------------------------------------------------------------------------

def check_table(geom: Geometry, table_row, ctx: int):
    """Validate one sequence's block table for a context of ctx tokens."""
    nb = -(-ctx // geom.block_size)
    if ctx < 0:
        raise ValueError("negative context length")
    if nb > len(table_row):
        raise ValueError("context longer than the block table")
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    if np.any(ids < 0) or np.any(ids >= geom.num_blocks):
        raise ValueError("block id out of range")


def gather(pool, geom: Geometry, pool_dtype: str, layer: int, table_row, ctx: int,
           scale: float = 1.0) -> np.ndarray:
    """Keys (or values) of one sequence as float64 [ctx][H_kv][D].

    Token t comes from block table_row[t // B], slot t % B ("Continuous
    Batching and PagedAttention", section "The block table is a page table":
    logical block index -> physical block). FP8 codes are multiplied by the
    tensor's scale (exact in float64).
    """
    check_table(geom, table_row, ctx)
    B, H, D = geom.block_size, geom.num_kv_heads, geom.head_dim
    t = np.arange(ctx, dtype=np.int64)
    blk = np.asarray(table_row, dtype=np.int64)[t // B] if ctx > 0 else t
    idx = geom.index(blk[:, None, None], layer, np.arange(H)[None, :, None],
                     (t % B)[:, None, None], np.arange(D)[None, None, :])
    vals = codecs.decode(np.asarray(pool)[idx], pool_dtype)
    if pool_dtype == codecs.FP8:
        vals = vals * np.float64(np.float32(scale))
    return vals


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Ordinary softmax attention of one decode query, float64.

    q [H_q][D]; k, v [n][H_kv][D]. Query head h reads KV head h // (H_q/H_kv).
    z_t = scale * <q_h, k_t>, out_h = sum_t exp(z_t - max z) v_t / sum_t
    exp(z_t - max z); n == 0 gives zeros.
    """
    Hq, D = q.shape
    n, Hkv, _ = k.shape
    if Hq % Hkv:
        raise ValueError("query heads not a multiple of KV heads")
    g = Hq // Hkv
    out = np.zeros((Hq, D), dtype=np.float64)
    if n == 0:
        return out
    for h in range(Hq):
        kvh = h // g
        z = np.float64(scale) * (k[:, kvh, :] @ q[h])          # [n]
        p = np.exp(z - z.max())
        out[h] = (p @ v[:, kvh, :]) / p.sum()
    return out


def decode(q_codes, q_dtype: str, pool_k, pool_v, geom: Geometry, pool_dtype: str,
           layer: int, block_tables, context_lens, scale: float,
           k_scale: float = 1.0, v_scale: float = 1.0, seqs=None) -> np.ndarray:
    """Paged decode: every (sequence, query head) output in float64.

    Gathers each sequence's keys and values through its block table into
    contiguous float64 arrays, then runs :func:`attention` on them: the paged
    result is defined to equal ordinary attention over the same tokens
    ("Efficient Memory Management for Large Language Model Serving with
    PagedAttention", kernel paragraph). ``seqs`` restricts the work to a subset
    of sequence indices (the returned array still has every row; others are
    NaN).
    """
    q = codecs.decode(q_codes, q_dtype)
    S, Hq, D = q.shape
    out = np.full((S, Hq, D), np.nan)
    tables = np.asarray(block_tables)
    ctx = np.asarray(context_lens)
    for s in (range(S) if seqs is None else seqs):
        n = int(ctx[s])
        k = gather(pool_k, geom, pool_dtype, layer, tables[s], n, k_scale)
        v = gather(pool_v, geom, pool_dtype, layer, tables[s], n, v_scale)
        out[s] = attention(q[s], k, v, scale)
    return out


def prefill(q_codes, q_dtype: str, pool_k, pool_v, geom: Geometry, pool_dtype: str,
            layer: int, block_tables, context_lens, query_start_loc, scale: float,
            k_scale: float = 1.0, v_scale: float = 1.0, seqs=None, rows=None) -> np.ndarray:
    """Paged prefill (and chunked prefill, and recompute): causal attention of
    the newest positions of each sequence, float64.

    Sequence s has n_s = query_start_loc[s+1] - query_start_loc[s] query rows,
    rows query_start_loc[s] .. +n_s - 1 of q [rows][H_q][D]; row j holds
    position p = ctx_s - n_s + j and attends to the sequence's positions
    0 .. p. Recompute runs the prompt and every generated token again as one
    prefill pass ("When KV Capacity Runs Out", section "Recompute KV from
    token history"; "Continuous Batching and PagedAttention": prefill is one
    wide parallel pass over the prompt); the keys and values of all positions
    are in the pool (written first, as in decode), reached through the block
    table. n_s = ctx_s is a whole prefill, n_s < ctx_s a later chunk, n_s = 1
    a decode step. ``seqs`` restricts the work to some sequences and ``rows``
    to some query rows (the others stay NaN).
    """
    q = codecs.decode(q_codes, q_dtype)
    R, Hq, D = q.shape
    out = np.full((R, Hq, D), np.nan)
    tables = np.asarray(block_tables)
    ctx = np.asarray(context_lens)
    qsl = np.asarray(query_start_loc)
    S = ctx.shape[0]
    if qsl.shape[0] != S + 1 or qsl[0] != 0 or qsl[-1] != R or np.any(np.diff(qsl) < 0):
        raise ValueError("query_start_loc must run from 0 to the row count, nondecreasing")
    want = None if rows is None else set(int(r) for r in rows)
    for s in (range(S) if seqs is None else seqs):
        n = int(ctx[s])
        nq = int(qsl[s + 1] - qsl[s])
        if nq > n:
            raise ValueError("more query rows than context positions")
        js = [j for j in range(nq) if want is None or int(qsl[s]) + j in want]
        if not js:
            continue
        k = gather(pool_k, geom, pool_dtype, layer, tables[s], n, k_scale)
        v = gather(pool_v, geom, pool_dtype, layer, tables[s], n, v_scale)
        for j in js:
            p = n - nq + j
            out[qsl[s] + j] = attention(q[qsl[s] + j], k[:p + 1], v[:p + 1], scale)
    return out

