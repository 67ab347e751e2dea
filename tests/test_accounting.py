"""Pins of the byte and block accounting used by the measurements, against
the worked numbers the pages print."""

import numpy as np
import pytest

import workloads
from oracle.blocks import blocks_for_tokens, wasted_slots

KiB, MiB, GiB = 1024, 1024 ** 2, 1024 ** 3


def test_bytes_per_token_13b_class():
    # "Efficient Memory Management ... PagedAttention", per-token size
    # paragraph: 2 x 5,120 x 40 layers x 2 bytes = 800 KB; 2,048 tokens ~ 1.6 GB
    b = workloads.kv_bytes_per_token(40, 40, 128, 2)
    assert b == 800 * KiB
    assert 1.55e9 < 2048 * b < 1.7e9


def test_bytes_per_token_70b_gqa():
    # "Continuous Batching and PagedAttention", section "Sizing the KV cache":
    # 4 KiB per token per layer, 320 KiB over 80 layers, 1.25 GiB per 4,096
    assert workloads.kv_bytes_per_token(1, 8, 128, 2) == 4 * KiB
    assert workloads.kv_bytes_per_token(80, 8, 128, 2) == 320 * KiB
    assert 4096 * workloads.kv_bytes_per_token(80, 8, 128, 2) == 1.25 * GiB
    # plain multi-head attention: 64 KV heads, eight-fold
    assert workloads.kv_bytes_per_token(80, 64, 128, 2) == 8 * 320 * KiB


def test_bytes_per_token_7b():
    # "KV Cache Preemption in vLLM", section "How much KV cache a token costs"
    assert workloads.kv_bytes_per_token(32, 32, 128, 2) == 0.5 * MiB
    assert workloads.kv_bytes_per_token(32, 32, 128, 1) == 0.25 * MiB
    assert workloads.kv_bytes_per_token(32, 8, 128, 2) == 128 * KiB


def test_swap_victim_blocks_and_bytes():
    # "41 · Preemption, Recomputation & KV Pressure", §3: 1500 / 16 = 93.75
    # -> 94 blocks x 2 MiB = 188 MiB (128 KiB per token, 32 layers)
    assert blocks_for_tokens(1500, 16) == 94
    per_block = 16 * workloads.kv_bytes_per_token(32, 8, 128, 2)
    assert per_block == 2 * MiB and 94 * per_block == 188 * MiB
    # the long FP8 workload stacked to 64 layers moves the same bytes per block
    assert 16 * workloads.kv_bytes_per_token(64, 8, 128, 1) == 2 * MiB


def test_internal_fragmentation_300_tokens():
    # "Continuous Batching and PagedAttention", section "Growth on demand":
    # 300 tokens waste 4 of 304 allocated slots (~1.3 %); never more than 15
    assert blocks_for_tokens(300, 16) * 16 == 304
    assert wasted_slots(300, 16) == 4
    assert round(100 * 4 / 304, 1) == 1.3
    assert max(wasted_slots(n, 16) for n in range(1, 2000)) == 15
    # contiguous reservation of 2,048 for a 300-token answer wastes ~85 %
    assert round(100 * (2048 - 300) / 2048) == 85


def test_new_block_rate_per_step():
    # "41 · Preemption, Recomputation & KV Pressure", §1: 100 requests with
    # 16-token blocks need ~6.25 new blocks per step (block starts counted
    # over a 16-step window with the requests at staggered offsets)
    offsets = np.arange(100) % 16
    new_blocks = [np.sum((offsets + step) % 16 == 0) for step in range(16)]
    assert np.mean(new_blocks) == 100 / 16 == 6.25


def test_decode_bytes_formula_on_a_tiny_case():
    wl = workloads.config1()
    # 15 tokens x 4 kv heads x 64 x 4 B x (K and V) + q/out + table entries
    kv = 15 * 4 * 64 * 4 * 2
    qo = 2 * 4 * 64 * 4 * 2
    tables = (2 + 2) * 4 + 2 * 4
    assert workloads.decode_bytes(wl) == kv + qo + tables
