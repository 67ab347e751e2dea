"""Seeded synthetic inputs for the paged KV-cache operations.

This module only draws inputs: context lengths, physical block placements,
slot mappings, block tables, and random query / key / value codes. It holds
none of the arithmetic the operations perform (no attention, no quantisation,
no block copies), so both the CPU oracle and the GPU library can be fed from
it without sharing code. The pages publish no datasets to run; the shapes and
length mixes below stand in for the workloads they describe:

1. ``tiny``      — the worked example's pool: 4 physical blocks x 4 slots, two
   requests holding 7 and 8 positions in disjoint blocks ("When KV Capacity
   Runs Out", Figure 1), fp32, 4 heads x 64.
2. ``mha_fp16``  — hidden size 5,120 as 40 heads x 128 ("Efficient Memory
   Management for Large Language Model Serving with PagedAttention", per-token
   size paragraph), 64 sequences, contexts uniform in [128, 2048].
3. ``gqa_bf16``  — 8 KV heads x 128 in bf16 ("Continuous Batching and
   PagedAttention", section "Sizing the KV cache for the running 70B model"),
   32 query heads, 256 sequences of an ~850-token prompt plus a 1..250-token
   answer ("KV Cache Preemption in vLLM", section "How much KV cache a token
   costs").
4. ``shared_prefix_fp16`` — parallel sampling: 32 prompts x 8 samples sharing
   the prompt's blocks (same summary page, sampling paragraph; "Continuous
   Batching and PagedAttention", section "Sharing, ...").
5. ``long_fp8``  — 64/8 heads x 128 with an FP8 KV cache, 8 sequences of 8k-32k
   tokens, plus a 1,500-token victim swapped back in from host memory
   ("41 · Preemption, Recomputation & KV Pressure", §3: 94 blocks).

Recipe common to all: ``numpy.random.default_rng(seed)`` with seed = config
number, drawing in the order lengths -> block permutation -> Q -> K -> V (->
victim K, V). Values are N(0, 1) float32 rounded to the storage type with
round-to-nearest-even (torch's CPU casts). Physical block ids come from one
permutation of the pool, handed out in order to sequence 0, 1, ...; the pool
is 10 % larger than needed and the spare blocks stay unwritten. Block-table
padding points at a spare block.
"""

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

F32, F16, BF16, FP8 = "f32", "f16", "bf16", "fp8_e4m3"
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2, FP8: 1}
CODE_TYPE = {F32: np.uint32, F16: np.uint16, BF16: np.uint16, FP8: np.uint8}
#: a NaN code per dtype: fills every pool slot before writes, so bytes that
#: were never written are NaN and any read of them shows up
NAN_CODE = {F32: 0x7FC00000, F16: 0x7E00, BF16: 0x7FC0, FP8: 0x7F}

CONFIG_NAMES = {1: "tiny_fp32", 2: "mha_fp16", 3: "gqa_bf16",
                4: "shared_prefix_fp16", 5: "long_fp8"}


# --------------------------------------------------------------------------
# value drawing
# --------------------------------------------------------------------------

def to_codes(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to a 16/32-bit storage type (RNE); return codes."""
    x = np.ascontiguousarray(x_f32, dtype=np.float32)
    if dtype == F32:
        return x.view(np.uint32).copy()
    t = torch.from_numpy(x)
    if dtype == F16:
        return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16).copy()
    if dtype == BF16:
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"no direct draw for {dtype}")


def normal_codes(rng, shape, dtype: str) -> np.ndarray:
    return to_codes(rng.standard_normal(size=shape, dtype=np.float32), dtype)


def codes_as_f32(codes: np.ndarray, dtype: str) -> np.ndarray:
    """Widen 16/32-bit codes to float32 (used only to pick FP8 scales)."""
    t = torch.from_numpy(np.ascontiguousarray(codes).view(np.int16 if dtype != F32 else np.int32))
    if dtype == F32:
        return t.view(torch.float32).numpy()
    if dtype == F16:
        return t.view(torch.float16).float().numpy()
    return t.view(torch.bfloat16).float().numpy()


def fp8_scale(src_codes: np.ndarray, src_dtype: str) -> float:
    """Per-tensor FP8 scale of a source tensor: fp32(max |x|) / 448 in fp32."""
    m = np.float32(np.max(np.abs(codes_as_f32(src_codes, src_dtype))))
    return float(m / np.float32(448.0))


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    seed: int
    pool_dtype: str           # storage type of the KV pool
    src_dtype: str            # type of the key/value tokens handed to writes
    q_dtype: str              # query / output type
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    num_layers: int
    layer: int
    scale: float              # softmax scale
    context_lens: np.ndarray  # int32 [S]
    block_tables: np.ndarray  # int32 [S][max_blocks]
    q: np.ndarray             # codes [S][H_q][D]
    # tokens written into the pool before decode, in write order
    write_k: np.ndarray       # codes [T][H_kv][D] of src_dtype
    write_v: np.ndarray
    write_slots: np.ndarray   # int64 [T]
    k_scale: float = 1.0
    v_scale: float = 1.0
    spare_block: int = -1     # an unwritten block (block-table padding target)
    # index into write_* of each sequence's newest token (the token one decode
    # step writes before attending); -1 when that token is not in write_*
    step_token: Optional[np.ndarray] = None
    # extra scenario inputs (shared prefix: copy-on-write pairs; long FP8: the swap victim)
    extra: Dict[str, object] = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    def layer_stride(self) -> int:
        return self.num_kv_heads * self.block_size * self.head_dim

    def block_stride(self) -> int:
        return self.num_layers * self.layer_stride()

    def pool_elements(self) -> int:
        return self.num_blocks * self.block_stride()

    def empty_pool(self) -> np.ndarray:
        """A pool whose every code is NaN (never-written bytes)."""
        return np.full(self.pool_elements(), NAN_CODE[self.pool_dtype],
                       dtype=CODE_TYPE[self.pool_dtype])


def _tables_from_placement(blocks_per_seq: List[List[int]], pad_id: int) -> np.ndarray:
    width = max(1, max(len(b) for b in blocks_per_seq))
    t = np.full((len(blocks_per_seq), width), pad_id, dtype=np.int32)
    for s, b in enumerate(blocks_per_seq):
        t[s, :len(b)] = b
    return t


def _slots_of(blocks: List[int], ntok: int, B: int) -> np.ndarray:
    t = np.arange(ntok, dtype=np.int64)
    return np.asarray(blocks, dtype=np.int64)[t // B] * B + t % B


def _pool_size(needed: int) -> int:
    return -(-needed * 11 // 10)


def _paged_workload(name, seed, rng, ctx, *, pool_dtype, src_dtype, q_dtype,
                    hq, hkv, d, B, extra_blocks=0, num_blocks=None):
    """Lengths are drawn; this draws the permutation, Q, K, V and lays out."""
    ctx = np.asarray(ctx, dtype=np.int32)
    nbs = [-(-int(n) // B) for n in ctx]
    needed = sum(nbs) + extra_blocks
    nblk = num_blocks if num_blocks is not None else _pool_size(needed)
    perm = rng.permutation(nblk)
    placement, pos = [], 0
    for nb in nbs:
        placement.append([int(x) for x in perm[pos:pos + nb]])
        pos += nb
    spare = int(perm[needed]) if needed < nblk else -1
    pad = spare if spare >= 0 else int(perm[0])
    tables = _tables_from_placement(placement, pad)
    S = len(ctx)
    q = normal_codes(rng, (S, hq, d), q_dtype)
    T = int(ctx.sum())
    k = normal_codes(rng, (T, hkv, d), src_dtype)
    v = normal_codes(rng, (T, hkv, d), src_dtype)
    slots = np.concatenate([_slots_of(placement[s], int(ctx[s]), B) for s in range(S)]) \
        if T else np.zeros(0, np.int64)
    starts = np.concatenate([[0], np.cumsum(ctx)[:-1]]).astype(np.int64)
    step_token = np.where(ctx > 0, starts + ctx - 1, -1).astype(np.int64)
    wl = Workload(name=name, seed=seed, pool_dtype=pool_dtype, src_dtype=src_dtype,
                  q_dtype=q_dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                  block_size=B, num_blocks=nblk, num_layers=1, layer=0,
                  scale=float(np.float32(1.0) / np.sqrt(np.float32(d))),
                  context_lens=ctx, block_tables=tables, q=q, write_k=k, write_v=v,
                  write_slots=slots, spare_block=spare, step_token=step_token)
    wl.extra["perm"] = perm
    wl.extra["needed_blocks"] = needed
    return wl


# --------------------------------------------------------------------------
# the five configurations
# --------------------------------------------------------------------------

def config1(seed: int = 1) -> Workload:
    """Tiny fp32: 4 blocks x 4 slots, contexts 7 and 8, 4 heads x 64."""
    rng = np.random.default_rng(seed)
    ctx = np.array([7, 8], dtype=np.int32)
    return _paged_workload("tiny_fp32", seed, rng, ctx, pool_dtype=F32, src_dtype=F32,
                           q_dtype=F32, hq=4, hkv=4, d=64, B=4, num_blocks=4)


def config2(seed: int = 2, num_seqs: int = 64) -> Workload:
    """MHA fp16: 40 x 128, B 16, contexts uniform in [128, 2048]."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(128, 2048, size=num_seqs, endpoint=True).astype(np.int32)
    return _paged_workload("mha_fp16", seed, rng, ctx, pool_dtype=F16, src_dtype=F16,
                           q_dtype=F16, hq=40, hkv=40, d=128, B=16)


def gqa_lengths(rng, num_seqs: int, prompt_mean: float = 850.0, sigma: float = 0.5,
                gen_max: int = 250) -> np.ndarray:
    """Prompt ~ lognormal with the given mean (sigma 0.5), rounded, >= 1, plus
    an answer length uniform in [1, gen_max]."""
    mu = np.log(prompt_mean) - sigma * sigma / 2.0
    prompt = np.maximum(1, np.rint(rng.lognormal(mu, sigma, size=num_seqs))).astype(np.int64)
    gen = rng.integers(1, gen_max, size=num_seqs, endpoint=True)
    return (prompt + gen).astype(np.int32)


def config3(seed: int = 3, num_seqs: int = 256, block_size: int = 16) -> Workload:
    """GQA bf16: 32/8 x 128, B 16 (other block sizes for the block-size sweep),
    256 sequences, ~850-token prompt + answer."""
    rng = np.random.default_rng(seed)
    ctx = gqa_lengths(rng, num_seqs)
    return _paged_workload("gqa_bf16", seed, rng, ctx, pool_dtype=BF16, src_dtype=BF16,
                           q_dtype=BF16, hq=32, hkv=8, d=128, B=block_size)


def config4(seed: int = 4, groups: int = 32, samples: int = 8, prefix_tokens: int = 1024,
            private_min: int = 64, private_max: int = 256, copied_samples: int = 7) -> Workload:
    """Shared-prefix parallel sampling, fp16 GQA 32/8 x 128, B 16.

    Each group's prompt occupies ceil(prefix/16) blocks shared by its samples.
    ``copied_samples`` of them privatise the prompt's last block by
    copy-on-write before their own tokens are written; the others keep the
    shared block. Writes happen in three phases (prompt tokens, then the
    copies, then each sample's private tokens), described in ``extra``.
    """
    B, hq, hkv, d = 16, 32, 8, 128
    rng = np.random.default_rng(seed)
    priv = rng.integers(private_min, private_max, size=(groups, samples), endpoint=True)
    nb_prefix = -(-prefix_tokens // B)
    fill = prefix_tokens % B            # tokens in the prompt's last block
    needed = 0
    per_sample_priv_blocks = np.zeros((groups, samples), dtype=np.int64)
    for g in range(groups):
        needed += nb_prefix
        for s in range(samples):
            room = (B - fill) % B       # private tokens that fit the last prompt block
            nb = -(-max(0, int(priv[g, s]) - room) // B)
            per_sample_priv_blocks[g, s] = nb
            needed += nb + (1 if s < copied_samples else 0)
    nblk = _pool_size(needed)
    perm = rng.permutation(nblk)
    pos = 0

    def take(n):
        nonlocal pos
        out = [int(x) for x in perm[pos:pos + n]]
        pos += n
        return out

    prefix_blocks, cow_pairs, placements, ctx = [], [], [], []
    for g in range(groups):
        pb = take(nb_prefix)
        prefix_blocks.append(pb)
        for s in range(samples):
            tbl = list(pb)
            if s < copied_samples:
                nb_new = take(1)[0]
                cow_pairs.append((pb[-1], nb_new))
                tbl[-1] = nb_new
            tbl += take(int(per_sample_priv_blocks[g, s]))
            placements.append(tbl)
            ctx.append(prefix_tokens + int(priv[g, s]))
    spare = int(perm[needed]) if needed < nblk else -1
    tables = _tables_from_placement(placements, spare if spare >= 0 else int(perm[0]))
    ctx = np.asarray(ctx, dtype=np.int32)
    S = groups * samples
    q = normal_codes(rng, (S, hq, d), F16)
    # prompt tokens per group, then private tokens per sample
    kp = normal_codes(rng, (groups * prefix_tokens, hkv, d), F16)
    vp = normal_codes(rng, (groups * prefix_tokens, hkv, d), F16)
    npriv = int(priv.sum())
    kq = normal_codes(rng, (npriv, hkv, d), F16)
    vq = normal_codes(rng, (npriv, hkv, d), F16)
    prefix_slots = np.concatenate([_slots_of(prefix_blocks[g], prefix_tokens, B)
                                   for g in range(groups)])
    priv_slots = []
    for i, tbl in enumerate(placements):
        t = np.arange(prefix_tokens, int(ctx[i]), dtype=np.int64)
        priv_slots.append(np.asarray(tbl, dtype=np.int64)[t // B] * B + t % B)
    priv_slots = np.concatenate(priv_slots)
    wl = Workload(name="shared_prefix_fp16" if prefix_tokens % B == 0 else
                  f"shared_prefix_fp16_p{prefix_tokens}", seed=seed, pool_dtype=F16,
                  src_dtype=F16, q_dtype=F16, num_q_heads=hq, num_kv_heads=hkv,
                  head_dim=d, block_size=B, num_blocks=nblk, num_layers=1, layer=0,
                  scale=float(np.float32(1.0) / np.sqrt(np.float32(d))),
                  context_lens=ctx, block_tables=tables, q=q,
                  write_k=np.concatenate([kp, kq]), write_v=np.concatenate([vp, vq]),
                  write_slots=np.concatenate([prefix_slots, priv_slots]),
                  spare_block=spare)
    # the step token of a sample is its last private token
    starts = np.concatenate([[0], np.cumsum(priv.reshape(-1))[:-1]]).astype(np.int64)
    wl.step_token = groups * prefix_tokens + starts + priv.reshape(-1) - 1
    wl.extra.update(perm=perm, needed_blocks=needed, prefix_blocks=prefix_blocks,
                    cow_pairs=np.asarray(cow_pairs, dtype=np.int64).reshape(-1, 2),
                    num_prefix_tokens_written=groups * prefix_tokens,
                    groups=groups, samples=samples, prefix_tokens=prefix_tokens)
    return wl


def config5(seed: int = 5, num_seqs: int = 8, ctx_min: int = 8192, ctx_max: int = 32768,
            victim_tokens: int = 1500, host_blocks: int = 128) -> Workload:
    """Long-context FP8 KV: 64/8 x 128, B 16, bf16 queries and sources.

    Also draws a swap victim of ``victim_tokens`` positions: its keys/values
    (bf16 sources), the device blocks it held before being swapped out, the
    host blocks that keep it while it is paused, and the (different) device
    blocks it is restored into ("When KV Capacity Runs Out", section "Restore
    KV stored outside the GPU"). The victim is decoded as one more sequence
    after the swap-in.
    """
    B, hq, hkv, d = 16, 64, 8, 128
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ctx_min, ctx_max, size=num_seqs, endpoint=True).astype(np.int32)
    nvb = -(-victim_tokens // B)
    nbs = [-(-int(n) // B) for n in ctx]
    needed = sum(nbs) + 2 * nvb            # victim: original blocks + restore blocks
    nblk = _pool_size(needed)
    perm = rng.permutation(nblk)
    placement, pos = [], 0
    for nb in nbs:
        placement.append([int(x) for x in perm[pos:pos + nb]])
        pos += nb
    victim_before = [int(x) for x in perm[pos:pos + nvb]]
    pos += nvb
    victim_after = [int(x) for x in perm[pos:pos + nvb]]
    pos += nvb
    spare = int(perm[pos]) if pos < nblk else -1
    host_ids = [int(x) for x in rng.permutation(host_blocks)[:nvb]]
    S = num_seqs
    q = normal_codes(rng, (S + 1, hq, d), BF16)
    T = int(ctx.sum())
    k = normal_codes(rng, (T, hkv, d), BF16)
    v = normal_codes(rng, (T, hkv, d), BF16)
    vk = normal_codes(rng, (victim_tokens, hkv, d), BF16)
    vv = normal_codes(rng, (victim_tokens, hkv, d), BF16)
    k_scale = fp8_scale(np.concatenate([k, vk]), BF16)
    v_scale = fp8_scale(np.concatenate([v, vv]), BF16)
    slots = np.concatenate([_slots_of(placement[s], int(ctx[s]), B) for s in range(S)])
    ctx_all = np.concatenate([ctx, [victim_tokens]]).astype(np.int32)
    tables = _tables_from_placement(placement + [victim_after], spare)
    starts = np.concatenate([[0], np.cumsum(ctx)[:-1]]).astype(np.int64)
    wl = Workload(name="long_fp8", seed=seed, pool_dtype=FP8, src_dtype=BF16, q_dtype=BF16,
                  num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=B,
                  num_blocks=nblk, num_layers=1, layer=0,
                  scale=float(np.float32(1.0) / np.sqrt(np.float32(d))),
                  context_lens=ctx_all, block_tables=tables, q=q, write_k=k, write_v=v,
                  write_slots=slots, k_scale=k_scale, v_scale=v_scale, spare_block=spare,
                  step_token=np.concatenate([starts + ctx - 1, [-1]]).astype(np.int64))
    wl.extra.update(perm=perm, needed_blocks=needed, victim_k=vk, victim_v=vv,
                    victim_slots_before=_slots_of(victim_before, victim_tokens, B),
                    victim_blocks_before=np.asarray(victim_before, np.int64),
                    victim_blocks_after=np.asarray(victim_after, np.int64),
                    victim_host_blocks=np.asarray(host_ids, np.int64),
                    host_pool_blocks=host_blocks, victim_tokens=victim_tokens)
    return wl


def custom(seed: int, ctx, *, pool_dtype: str, q_dtype: str, num_q_heads: int,
           num_kv_heads: int, head_dim: int, block_size: int, src_dtype: str = None,
           scale_from_data: bool = True) -> Workload:
    """A small workload with given context lengths (edge cases, sweeps).

    FP8 pools take bf16 sources (unless ``src_dtype`` says otherwise) and
    per-tensor scales fp32(max |x|) / 448."""
    rng = np.random.default_rng(seed)
    src = src_dtype or (BF16 if pool_dtype == FP8 else pool_dtype)
    wl = _paged_workload(f"custom_{seed}", seed, rng, np.asarray(ctx, dtype=np.int32),
                         pool_dtype=pool_dtype, src_dtype=src, q_dtype=q_dtype,
                         hq=num_q_heads, hkv=num_kv_heads, d=head_dim, B=block_size)
    if pool_dtype == FP8 and scale_from_data and wl.write_k.shape[0]:
        wl.k_scale = fp8_scale(wl.write_k, src)
        wl.v_scale = fp8_scale(wl.write_v, src)
    return wl


def shared_prefix(seed: int, groups, *, pool_dtype: str, q_dtype: str, num_q_heads: int,
                  num_kv_heads: int, head_dim: int, block_size: int,
                  src_dtype: str = None) -> Workload:
    """Parallel samples of several prompts (the layout of the shared-prefix
    workload, any geometry). ``groups`` lists (prompt tokens, [private
    tokens of each sample]); a group's samples are consecutive sequences
    whose tables name the prompt's blocks. A sample that appends to a
    partly filled last prompt block first copies it (copy-on-write), so its
    table names the copy there. Writes run in three phases like
    :func:`fill_plan` expects: prompts, copies, private tokens."""
    rng = np.random.default_rng(seed)
    B = block_size
    src = src_dtype or (BF16 if pool_dtype == FP8 else pool_dtype)
    needed = 0
    for P, priv in groups:
        nbp = -(-P // B)
        needed += nbp
        for n in priv:
            cow = 1 if (P % B and n > 0) else 0
            room = (B - P % B) % B if not cow else (B - P % B)
            needed += cow + -(-max(0, n - room) // B)
    nblk = _pool_size(needed) + 1
    perm = rng.permutation(nblk)
    pos = 0

    def take(n):
        nonlocal pos
        out = [int(x) for x in perm[pos:pos + n]]
        pos += n
        return out

    placements, ctx, cow_pairs, prompt_slots, priv_slots = [], [], [], [], []
    for P, priv in groups:
        pb = take(-(-P // B))
        prompt_slots.append(_slots_of(pb, P, B))
        for n in priv:
            tbl = list(pb)
            if P % B and n > 0:
                nb_new = take(1)[0]
                cow_pairs.append((pb[-1], nb_new))
                tbl[-1] = nb_new
            extra = -(-max(0, P + n - len(tbl) * B) // B)
            tbl += take(extra)
            placements.append(tbl)
            ctx.append(P + n)
            t = np.arange(P, P + n, dtype=np.int64)
            priv_slots.append(np.asarray(tbl, dtype=np.int64)[t // B] * B + t % B)
    spare = int(perm[pos]) if pos < nblk else int(perm[0])
    tables = _tables_from_placement(placements, spare)
    ctx = np.asarray(ctx, dtype=np.int32)
    S = len(ctx)
    q = normal_codes(rng, (S, num_q_heads, head_dim), q_dtype)
    n0 = sum(P for P, _ in groups)
    npriv = int(sum(sum(p) for _, p in groups))
    k = normal_codes(rng, (n0 + npriv, num_kv_heads, head_dim), src)
    v = normal_codes(rng, (n0 + npriv, num_kv_heads, head_dim), src)
    slots = np.concatenate(prompt_slots + priv_slots) if n0 + npriv else np.zeros(0, np.int64)
    wl = Workload(name=f"shared_{seed}", seed=seed, pool_dtype=pool_dtype, src_dtype=src,
                  q_dtype=q_dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                  head_dim=head_dim, block_size=B, num_blocks=nblk, num_layers=1, layer=0,
                  scale=float(np.float32(1.0) / np.sqrt(np.float32(head_dim))),
                  context_lens=ctx, block_tables=tables, q=q, write_k=k, write_v=v,
                  write_slots=slots, spare_block=spare)
    wl.extra.update(cow_pairs=np.asarray(cow_pairs, dtype=np.int64).reshape(-1, 2),
                    num_prefix_tokens_written=n0)
    if pool_dtype == FP8 and k.shape[0]:
        wl.k_scale = fp8_scale(k, src)
        wl.v_scale = fp8_scale(v, src)
    return wl


def make(config: int, **kw) -> Workload:
    return {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}[config](**kw)


def fill_plan(wl: Workload):
    """Steps that put every context token of the workload into its pool, in
    order: ``("write", k, v, slots)`` and ``("copy", pairs)`` (device block
    copies). The shared-prefix workload writes its prompts, copies the last
    prompt block for the samples that privatise it, then writes the private
    tokens; the long FP8 workload's victim is written straight into the
    blocks it is restored into (the state after its swap-in)."""
    if "cow_pairs" in wl.extra:
        n0 = wl.extra["num_prefix_tokens_written"]
        return [("write", wl.write_k[:n0], wl.write_v[:n0], wl.write_slots[:n0]),
                ("copy", wl.extra["cow_pairs"]),
                ("write", wl.write_k[n0:], wl.write_v[n0:], wl.write_slots[n0:])]
    plan = [("write", wl.write_k, wl.write_v, wl.write_slots)]
    if "victim_k" in wl.extra:
        after = [int(b) for b in wl.extra["victim_blocks_after"]]
        plan.append(("write", wl.extra["victim_k"], wl.extra["victim_v"],
                     _slots_of(after, wl.extra["victim_tokens"], wl.block_size)))
    return plan


# --------------------------------------------------------------------------
# byte accounting of the measurements
# --------------------------------------------------------------------------

def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       elem_bytes: float) -> float:
    """Bytes of K and V one token leaves in the cache: 2 x layers x kv width x
    bytes per element ("KV Cache Preemption in vLLM", section "How much KV
    cache a token costs")."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def decode_bytes(wl: Workload, context_lens=None) -> int:
    """Bytes a decode call must move at the least: every context token's K and
    V for every KV head, the queries, the outputs, the block-table entries in
    use and the context lengths."""
    ctx = np.asarray(wl.context_lens if context_lens is None else context_lens, dtype=np.int64)
    S = ctx.shape[0]
    kv = int(ctx.sum()) * int(kv_bytes_per_token(1, wl.num_kv_heads, wl.head_dim,
                                                 ELEM_BYTES[wl.pool_dtype]))
    qo = S * wl.num_q_heads * wl.head_dim * 2 * ELEM_BYTES[wl.q_dtype]
    tables = int(np.sum(-(-ctx // wl.block_size))) * 4 + 4 * S
    return kv + qo + tables


def write_bytes(wl: Workload, num_tokens: int) -> int:
    """Bytes a slot write of num_tokens tokens moves: source K and V read,
    pool K and V written, slot indices read."""
    per_tok = wl.num_kv_heads * wl.head_dim * 2
    return num_tokens * (per_tok * (ELEM_BYTES[wl.src_dtype] + ELEM_BYTES[wl.pool_dtype]) + 8)


def copy_bytes(wl: Workload, num_pairs: int) -> int:
    """Bytes a block copy of num_pairs blocks moves (read + write)."""
    return 2 * num_pairs * 2 * wl.block_stride() * ELEM_BYTES[wl.pool_dtype]


def prefill_queries(wl: Workload, query_lens, seed: int):
    """Packed query rows for a prefill over the workload's pool: query_lens[s]
    rows for sequence s (its newest positions), N(0, 1) rounded to the query
    dtype. Returns (q codes [rows][H_q][D], query_start_loc int32 [S + 1])."""
    rng = np.random.default_rng(seed)
    ql = np.asarray(query_lens, dtype=np.int64)
    qsl = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    q = normal_codes(rng, (int(qsl[-1]), wl.num_q_heads, wl.head_dim), wl.q_dtype)
    return q, qsl

