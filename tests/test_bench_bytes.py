"""The roofline's numerator: the algorithmic bytes bench.py divides by the
measured times, counted here again from the workload's token and block
counts (host logic only)."""

import numpy as np

import bench
import workloads


def test_gqa_bf16_attention_bytes():
    wl = workloads.config3()
    ctx = wl.context_lens.astype(np.int64)
    tokens = int(ctx.sum())
    assert tokens == 253_123
    entries = sum(-(-int(c) // 16) for c in ctx)            # block-table entries read
    kv = tokens * 8 * 128 * 2 * 2                           # K and V, 8 KV heads x 128, bf16
    q = 256 * 32 * 128 * 2
    expect = kv + q + 4 * entries + 4 * 256                 # + the context lengths
    assert bench.attend_bytes(wl) == expect == 1_038_953_744
    # a decode call also writes every output row once
    assert workloads.decode_bytes(wl) - bench.attend_bytes(wl) == 256 * 32 * 128 * 2
    # the step adds the newest token's slot write: source read, pool written, slot index
    per_tok = 8 * 128 * 2 * (2 + 2) + 8
    assert workloads.write_bytes(wl, 256) == 256 * per_tok
    assert workloads.decode_bytes(wl) + workloads.write_bytes(wl, 256) == 1_043_150_096


def test_fp8_pool_counts_one_byte_per_element():
    wl = workloads.config5(num_seqs=2, ctx_min=100, ctx_max=200)
    ctx = wl.context_lens.astype(np.int64)
    kv = int(ctx.sum()) * wl.num_kv_heads * wl.head_dim * 2 * 1
    q = wl.num_seqs * wl.num_q_heads * wl.head_dim * 2      # bf16 queries
    tables = int(np.sum(-(-ctx // wl.block_size))) * 4 + 4 * wl.num_seqs
    assert bench.attend_bytes(wl) == kv + q + tables
