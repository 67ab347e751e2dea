"""Benchmark of the paged-decode hot path on one MI355X.

A step is one pass of the hot path over one batch: the slot write of every
sequence's newest token (pa_write_kv), then paged decode attention over every
sequence's whole context (pa_decode_attend + pa_decode_merge). The default
workload is the GQA bf16 decode batch: 256 sequences, 32 query / 8 KV heads x
128, block size 16, contexts of a lognormal ~850-token prompt plus a
1..250-token answer (seeded synthetic data; the pages publish no dataset).

Prints ONE JSON line: value = algorithmic bytes of a step / step time, in
GB/s (KV of every context token for every KV head, queries, outputs, block
table entries and context lengths, plus the slot write's source and pool
bytes). Inputs are resident in HBM before timing starts. Also reported:
the dominant kernel's roofline (HIP events on the launch stream), the CPU
oracle timed on a bounded sample, and an L2/Infinity-Cache-flushed per-call
decode time.

    python bench.py [--steps K] [--warmup W] [--config 1..5] [--no-cpu-baseline]
"""

import argparse
import hashlib
import json
import os
import sys
import time
import types

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s

# Figures the pages give for context (reported beside the measurements; none
# is a target here, and none was measured on this hardware).
PAGE_CONTEXT = [
    {"figure": "2-4x the request rate of Orca-class serving systems at similar latency",
     "context": "the vLLM authors' end-to-end serving measurements on their own GPUs, models "
                "(e.g. OPT-13B) and request traces (ShareGPT, Alpaca); whole serving systems, "
                "not one kernel",
     "source": "Efficient Memory Management for Large Language Model Serving with PagedAttention "
               "(summary page), results paragraph"},
    {"figure": "about 24 ms to recompute a 1,500-token request",
     "context": "idealised: 1,500 tokens x 16 GFLOP per token = 24 TFLOP for Llama 3.1 8B, all "
                "layers, at the 989 TFLOP/s H100 dense peak",
     "source": "41 - Preemption, Recomputation & KV Pressure, section 3"},
    {"figure": "about 3 ms each way to swap the same request",
     "context": "94 blocks x 2 MiB (all layers) = 188 MiB over PCIe Gen5 x16 at ~64 GB/s nominal",
     "source": "41 - Preemption, Recomputation & KV Pressure, section 3"},
]
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_44_amd", "csrc", f)
                  for f in ("pa_decode.hip", "pa_decode_mfma.hip", "pa_decode_sk.h", "pa_mfma.h", "pa_device.h",
                            "pa_internal.h")]


def attend_kernel_name(wl) -> str:
    """Which attention kernel the library runs for this workload: the matrix
    core kernel for 16-bit / FP8 pools with 16-bit queries, the VALU kernel
    otherwise."""
    mfma = (wl.pool_dtype in ("f16", "bf16", "fp8_e4m3") and wl.q_dtype in ("f16", "bf16")
            and (wl.pool_dtype == wl.q_dtype or wl.pool_dtype == "fp8_e4m3")
            and wl.head_dim in (64, 128) and wl.num_q_heads // wl.num_kv_heads in (1, 2, 4, 8, 16))
    return "attend_sk_kernel" if mfma else "attend_kernel"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target seconds of CPU oracle work for the baseline sample")
    ap.add_argument("--flush-iters", type=int, default=20)
    ap.add_argument("--print-source-hash", action="store_true",
                    help="print the hash of the attention kernel sources and exit")
    ap.add_argument("--swap", action="store_true",
                    help="time the long FP8 workload's swap-victim block moves between pinned "
                         "host memory and the device (1 layer and a 64-layer stack); one JSON "
                         "line per case")
    ap.add_argument("--shared", action="store_true",
                    help="decode with pa_decode_shared (prefixes shared by runs of consecutive "
                         "sequences read once per group; sharing planned every step)")
    ap.add_argument("--reuse-plan", action="store_true",
                    help="with --shared: plan the sharing once, then time calls that reuse the "
                         "plan (the later layers of a decode step, whose tables and lengths are "
                         "those of the first)")
    ap.add_argument("--swap-sweep", action="store_true",
                    help="swap moves of a 1,500-token FP8 victim for block sizes 8..128, one "
                         "layer and 64 layers, block-major and layer-major pools; then the "
                         "swap pipeline (copy stream beside decode); one JSON line per case")
    ap.add_argument("--prefill", action="store_true",
                    help="time paged prefill: the GQA bf16 workload's contexts prefilled whole "
                         "(bf16 pool, and an FP8 pool with bf16 queries), and the long FP8 "
                         "workload's 1,500-token victim recomputed; one JSON line each")
    ap.add_argument("--block-size-sweep", action="store_true",
                    help="the GQA bf16 decode step at block sizes 8..256: step and attention-kernel "
                         "time, and the slots the blocks hold beyond the context (one JSON line each)")
    ap.add_argument("--counters-summary", nargs=2, metavar=("KERNEL_WORKLOAD", "CSV"),
                    help="turn rocprofv3 --pmc counter CSVs (comma-separated paths) of a "
                         "decode run into profiles/traffic_<KERNEL_WORKLOAD>.json")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (torch) a few times: the "
                         "reference kernel for scaling HBM byte counters")
    return ap.parse_args()


def copy_calibration(reps: int = 5):
    """A plain device-to-device copy of 1 GiB (read 1 GiB, write 1 GiB), timed;
    its counter readings calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ms = float(np.median(ts))
    print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30,
                      "median_ms": round(ms, 4),
                      "GBps_read_plus_write": round(2 * (1 << 30) / (ms * 1e-3) / 1e9, 1)}),
          flush=True)


def codes_tensor(codes, dtype, device):
    import torch
    codes = np.ascontiguousarray(codes)
    if dtype == "fp8_e4m3":
        t = torch.from_numpy(codes.view(np.uint8))
    elif dtype == "f32":
        t = torch.from_numpy(codes.view(np.int32)).view(torch.float32)
    elif dtype == "f16":
        t = torch.from_numpy(codes.view(np.int16)).view(torch.float16)
    else:
        t = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def attend_bytes(wl) -> int:
    """Algorithmic bytes the attention kernel must move: every context token's
    K and V for every KV head, the queries, the block-table entries in use and
    the context lengths (outputs are excluded: the merge writes part of them)."""
    import workloads
    ctx = wl.context_lens.astype(np.int64)
    kv = int(ctx.sum()) * wl.num_kv_heads * wl.head_dim * 2 * workloads.ELEM_BYTES[wl.pool_dtype]
    q = wl.num_seqs * wl.num_q_heads * wl.head_dim * workloads.ELEM_BYTES[wl.q_dtype]
    tables = int(np.sum(-(-ctx // wl.block_size))) * 4 + 4 * wl.num_seqs
    return kv + q + tables


def load_traffic(kernel: str, workload: str):
    """Measured HBM bytes per launch from the committed counter summary, or
    None when it is missing or the kernel source changed since."""
    path = os.path.join(PROFILE_DIR, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def unique_decode_bytes(wl) -> int:
    """Bytes a decode call moves when every physical block's used slots are
    read once however many sequences share it (the shared-prefix workload's
    prompts): the logical count with each physical slot counted once."""
    import workloads
    B = wl.block_size
    used = {}
    for s in range(wl.num_seqs):
        n = int(wl.context_lens[s])
        for j in range(-(-n // B)):
            phys = int(wl.block_tables[s, j])
            used[phys] = max(used.get(phys, 0), min(B, n - j * B))
    per_tok = workloads.kv_bytes_per_token(1, wl.num_kv_heads, wl.head_dim,
                                           workloads.ELEM_BYTES[wl.pool_dtype])
    logical_kv = int(wl.context_lens.sum()) * int(per_tok)
    return workloads.decode_bytes(wl) - logical_kv + sum(used.values()) * int(per_tok)


def swap_bench(reps: int = 20):
    """Swap out / swap in of the long FP8 workload's 1,500-token victim (94
    blocks, their device ids shuffled) between pinned host blocks and device
    blocks ("When KV Capacity Runs Out", section "Restore KV stored outside the
    GPU"), for one layer and for a 64-layer stack of the same geometry.
    Bandwidth against the PCIe link the copy crosses."""
    import torch
    import paged_kv_cache_44_amd as pa
    import workloads
    wl = workloads.config5()
    ex = wl.extra
    nvb = len(ex["victim_host_blocks"])
    host_ids = np.asarray(ex["victim_host_blocks"], np.int64)
    dev_blocks = 2 * ex["host_pool_blocks"]
    dev_ids = np.random.default_rng(55).permutation(dev_blocks)[:nvb].astype(np.int64)
    for L in (1, 64):
        host = pa.KVCache.empty(wl.pool_dtype, ex["host_pool_blocks"], L, wl.num_kv_heads,
                                wl.block_size, wl.head_dim, pin_memory=True,
                                k_scale=wl.k_scale, v_scale=wl.v_scale)
        dev = pa.KVCache.empty(wl.pool_dtype, dev_blocks, L, wl.num_kv_heads, wl.block_size,
                               wl.head_dim, k_scale=wl.k_scale, v_scale=wl.v_scale)
        host.k.fill_(1)
        host.v.fill_(2)
        dev.k.fill_(3)
        dev.v.fill_(4)
        p_in = torch.from_numpy(np.stack([host_ids, dev_ids], 1).copy())
        p_out = torch.from_numpy(np.stack([dev_ids, host_ids], 1).copy())
        nbytes = nvb * 2 * dev.block_stride * workloads.ELEM_BYTES[wl.pool_dtype]
        res = {}
        for name, dst, src, pairs, d in (("h2d", dev, host, p_in, "h2d"),
                                         ("d2h", host, dev, p_out, "d2h")):
            for _ in range(3):
                pa.copy_blocks(dst, src, pairs, d)
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                pa.copy_blocks(dst, src, pairs, d)
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            ms = float(np.median(ts))
            res[name] = {"ms": round(ms, 4), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 2)}
        print(json.dumps({"metric": "swap block moves, GB/s over PCIe", "workload": "long_fp8 victim",
                          "blocks": nvb, "layers": L, "bytes_each_way": int(nbytes),
                          "h2d": res["h2d"], "d2h": res["d2h"],
                          "pcie_nominal_GBps": 64.0}), flush=True)
        del host, dev


def _time_ms(fn, reps: int, stream=None) -> float:
    """Median milliseconds of fn() between two events on ``stream``."""
    import torch
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts))


def _swap_pools(dtype, nvb, ndev, L, H, B, D, layout):
    """A pinned host pool of nvb packed blocks and a device pool of ndev
    blocks: block-major (a block's layers back to back) or layer-major (one
    packed array of blocks per layer)."""
    import torch
    import paged_kv_cache_44_amd as pa
    host = pa.KVCache.empty(dtype, nvb, L, H, B, D, pin_memory=True)
    slab = H * B * D
    if layout == "block_major":
        dev = pa.KVCache.empty(dtype, ndev, L, H, B, D)
    else:
        td = pa.TORCH_DTYPE[dtype]
        dev = pa.KVCache(torch.empty(ndev * L * slab, dtype=td, device="cuda"),
                         torch.empty(ndev * L * slab, dtype=td, device="cuda"), dtype, ndev, L, H,
                         B, D, block_stride=slab, layer_stride=ndev * slab)
    for t, c in ((host.k, 1), (host.v, 2), (dev.k, 3), (dev.v, 4)):
        t.view(torch.uint8).fill_(c)
    return host, dev


def swap_sweep(reps: int = 8):
    """Block-size sweep of swap moves ("41 · Preemption, Recomputation & KV
    Pressure", section 3; "Efficient Memory Management for Large Language
    Model Serving with PagedAttention", block-size paragraph): the long FP8
    workload's 1,500-token victim (8 KV heads, head dim 128) for B = 8 .. 128,
    one layer and a 64-layer stack, the device blocks scattered at random and
    the host blocks packed. Block-major pools move a whole block (every layer)
    per DMA transfer; layer-major pools, one layer of one block. Each move is
    timed by the DMA engines, by the copy kernel (one launch for every block
    and layer) and staged (a gather / scatter kernel beside a few large DMA
    transfers). One JSON line per case."""
    import torch
    import paged_kv_cache_44_amd as pa
    import workloads
    wl = workloads.config5()
    H, D, dt = wl.num_kv_heads, wl.head_dim, wl.pool_dtype
    eb = workloads.ELEM_BYTES[dt]
    tokens = 1500
    rng = np.random.default_rng(77)
    for L in (1, 64):
        for B in (8, 16, 32, 64, 128):
            nvb = -(-tokens // B)
            ndev = 4 * nvb
            for layout in (("block_major",) if L == 1 else ("block_major", "layer_major")):
                host, dev = _swap_pools(dt, nvb, ndev, L, H, B, D, layout)
                dev_ids = rng.permutation(ndev)[:nvb].astype(np.int64)
                host_ids = np.arange(nvb, dtype=np.int64)
                p_in = torch.from_numpy(np.stack([host_ids, dev_ids], 1).copy())
                p_out = torch.from_numpy(np.stack([dev_ids, host_ids], 1).copy())
                nbytes = nvb * 2 * L * H * B * D * eb
                transfers = 2 * nvb * (1 if layout == "block_major" else L)
                staging = torch.empty(pa.copy_staging_size(dev, nvb), dtype=torch.uint8,
                                      device="cuda")
                res = {}
                for name, dst, src, pairs in (("d2h", host, dev, p_out), ("h2d", dev, host, p_in)):
                    res[name] = {}
                    for method in ("dma", "kernel", "staged"):
                        def move():
                            if method == "staged":
                                pa.copy_blocks_staged(dst, src, pairs, name, staging)
                            else:
                                pa.copy_blocks(dst, src, pairs,
                                               name + ("_kernel" if method == "kernel" else ""))
                        for _ in range(2):
                            move()
                        torch.cuda.synchronize()
                        ms = _time_ms(move, reps)
                        res[name][method] = {"ms": round(ms, 4),
                                             "GBps": round(nbytes / (ms * 1e-3) / 1e9, 2)}
                print(json.dumps({"metric": "swap block moves, GB/s over PCIe",
                                  "workload": "1,500-token FP8 victim", "layers": L,
                                  "block_size": B, "blocks": nvb, "layout": layout,
                                  "bytes_each_way": int(nbytes),
                                  "host_pool_mapped": pa.host_pool_mapped(host),
                                  "dma_transfers": transfers,
                                  "bytes_per_dma_transfer": int(nbytes // transfers),
                                  "d2h": res["d2h"], "h2d": res["h2d"]}),
                      flush=True)
                del host, dev, staging
                torch.cuda.empty_cache()


def swap_overlap(steps: int = 40):
    """The swap pipeline: the 64-layer victim's blocks move out and back on a
    copy stream while decode steps of the long FP8 workload run on the
    compute stream; the copy stream waits on an event the compute stream
    records after the victim's last use, and the compute stream waits on the
    swap-in's completion event before the next step that reads the victim
    ("When KV Capacity Runs Out", section "Restore KV stored outside the
    GPU": blocks must not be reused before their copy has finished). Reports
    each side alone and both together, for the DMA engines, the copy kernel
    and the staged copy (gather kernel + large DMA transfers)."""
    import torch
    import paged_kv_cache_44_amd as pa
    import workloads
    wl = workloads.config5()
    dev = torch.device("cuda:0")
    pool = wl.empty_pool()
    cache = pa.KVCache(codes_tensor(pool, wl.pool_dtype, dev), codes_tensor(pool, wl.pool_dtype, dev),
                       wl.pool_dtype, wl.num_blocks, wl.num_layers, wl.num_kv_heads,
                       wl.block_size, wl.head_dim, k_scale=wl.k_scale, v_scale=wl.v_scale)
    for op in workloads.fill_plan(wl):
        if op[0] == "write":
            pa.write_kv(cache, wl.layer, codes_tensor(op[1], wl.src_dtype, dev),
                        codes_tensor(op[2], wl.src_dtype, dev), torch.from_numpy(op[3]).to(dev))
        else:
            pa.copy_blocks(cache, cache, torch.from_numpy(op[1]).to(dev), "d2d")
    q = codes_tensor(wl.q, wl.q_dtype, dev)
    out = torch.empty_like(q)
    tables = torch.from_numpy(wl.block_tables).to(dev)
    ctx = torch.from_numpy(wl.context_lens).to(dev)
    S, Hq, mc = wl.num_seqs, wl.num_q_heads, wl.max_context_len
    ws = torch.empty(max(1, pa.decode_workspace_size(cache, S, Hq, mc)), dtype=torch.uint8, device=dev)

    H, B, D, L = wl.num_kv_heads, wl.block_size, wl.head_dim, 64
    nvb = -(-1500 // B)
    host, sp = _swap_pools(wl.pool_dtype, nvb, 4 * nvb, L, H, B, D, "block_major")
    rng = np.random.default_rng(78)
    ids = rng.permutation(4 * nvb)[:2 * nvb].astype(np.int64)
    hid = np.arange(nvb, dtype=np.int64)
    p_out = torch.from_numpy(np.stack([ids[:nvb], hid], 1).copy())
    p_in = torch.from_numpy(np.stack([hid, ids[nvb:]], 1).copy())
    nbytes = nvb * 2 * L * H * B * D * workloads.ELEM_BYTES[wl.pool_dtype]
    copy_stream = torch.cuda.Stream()
    compute = torch.cuda.current_stream()

    def decode_steps():
        for _ in range(steps):
            pa.decode(cache, wl.layer, q, tables, ctx, mc, wl.scale, out=out, workspace=ws)

    decode_steps()
    torch.cuda.synchronize()
    dec_ms = _time_ms(decode_steps, 5, compute)
    res = {}
    staging = torch.empty(pa.copy_staging_size(sp, nvb), dtype=torch.uint8, device=dev)
    for method in ("dma", "kernel", "staged"):
        def swap_round_trip():
            if method == "staged":
                pa.copy_blocks_staged(host, sp, p_out, "d2h", staging, stream=copy_stream)
                pa.copy_blocks_staged(sp, host, p_in, "h2d", staging, stream=copy_stream)
            else:
                sfx = "_kernel" if method == "kernel" else ""
                pa.copy_blocks(host, sp, p_out, "d2h" + sfx, stream=copy_stream)
                pa.copy_blocks(sp, host, p_in, "h2d" + sfx, stream=copy_stream)

        swap_round_trip()
        torch.cuda.synchronize()
        swp_ms = _time_ms(swap_round_trip, 5, copy_stream)
        both = []
        for _ in range(5):
            a, b, c, d = (torch.cuda.Event(enable_timing=True) for _ in range(4))
            a.record(compute)
            copy_stream.wait_event(a)        # the victim's last use precedes its copy
            swap_round_trip()
            c.record(copy_stream)
            decode_steps()
            b.record(compute)
            compute.wait_event(c)            # a step reading the victim waits for its swap-in
            d.record(compute)
            torch.cuda.synchronize()
            both.append((a.elapsed_time(b), a.elapsed_time(c), a.elapsed_time(d)))
        both = np.median(np.array(both), axis=0)
        res[method] = {"swap_ms_alone": round(swp_ms, 3),
                       "swap_GBps_alone": round(2 * nbytes / (swp_ms * 1e-3) / 1e9, 2),
                       "decode_ms_during_swap": round(float(both[0]), 3),
                       "swap_ms_during_decode": round(float(both[1]), 3),
                       "both_ms": round(float(both[2]), 3),
                       "serial_ms": round(dec_ms + swp_ms, 3)}
    print(json.dumps({"metric": "swap pipeline overlap", "workload": "long_fp8 decode + 64-layer "
                      "1,500-token victim out and back", "decode_steps": steps,
                      "decode_ms_alone": round(dec_ms, 3), **res}), flush=True)


MFMA_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 / f16 matrix-core peak


def prefill_flops(context_lens, query_lens, num_q_heads: int, head_dim: int) -> int:
    """Algorithmic FLOPs of a causal prefill: each query row at position p
    takes p + 1 scores and p + 1 weighted values per head, 2 FLOPs per
    multiply-add over head_dim."""
    tot = 0
    for n, nq in zip(context_lens, query_lens):
        n, nq = int(n), int(nq)
        # positions n - nq .. n - 1 attend to p + 1 keys each
        tot += nq * (n - nq) + nq * (nq + 1) // 2
    return 4 * num_q_heads * head_dim * tot


def prefill_bench(steps: int, warmup: int):
    """Paged prefill timed with HIP events (median over steps): TFLOP/s
    against the matrix-core peak, and the key/value bytes it reads."""
    import torch
    import paged_kv_cache_44_amd as pa
    import workloads
    dev = torch.device("cuda:0")
    gqa = workloads.make(3)
    cases = [("prefill_gqa_bf16", gqa, None),
             ("prefill_gqa_fp8", workloads.custom(3, gqa.context_lens, pool_dtype="fp8_e4m3",
                                                  q_dtype="bf16", num_q_heads=32, num_kv_heads=8,
                                                  head_dim=128, block_size=16), None),
             ("recompute_fp8_1500", workloads.custom(505, [1500], pool_dtype="fp8_e4m3",
                                                     q_dtype="bf16", num_q_heads=64, num_kv_heads=8,
                                                     head_dim=128, block_size=16), None)]
    for name, wl, _ in cases:
        pool = wl.empty_pool()
        cache = pa.KVCache(codes_tensor(pool, wl.pool_dtype, dev), codes_tensor(pool, wl.pool_dtype, dev),
                           wl.pool_dtype, wl.num_blocks, wl.num_layers, wl.num_kv_heads,
                           wl.block_size, wl.head_dim, k_scale=wl.k_scale, v_scale=wl.v_scale)
        for op in workloads.fill_plan(wl):
            if op[0] == "write":
                pa.write_kv(cache, wl.layer, codes_tensor(op[1], wl.src_dtype, dev),
                            codes_tensor(op[2], wl.src_dtype, dev), torch.from_numpy(op[3]).to(dev))
            else:
                pa.copy_blocks(cache, cache, torch.from_numpy(op[1]).to(dev), "d2d")
        ql = wl.context_lens.copy()                       # whole prefills: every position
        qc, qsl = workloads.prefill_queries(wl, ql, 77)
        q = codes_tensor(qc, wl.q_dtype, dev)
        out = torch.empty_like(q)
        tables = torch.from_numpy(wl.block_tables).to(dev)
        ctx = torch.from_numpy(wl.context_lens).to(dev)
        qs = torch.from_numpy(qsl).to(dev)
        mq = int(ql.max())
        call = lambda: pa.prefill(cache, wl.layer, q, tables, ctx, wl.max_context_len, qs, mq,
                                  wl.scale, out=out)
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        # calls shorter than a millisecond are timed 8 back to back per sample
        # (as the layers of one pass would run), so that the host's share of
        # one call does not leave the GPU idle inside the timed region
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        torch.cuda.synchronize()
        reps = 1 if a.elapsed_time(b) > 1.0 else 8
        ts = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                call()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / reps)
        ms = float(np.median(ts))
        fl = prefill_flops(wl.context_lens, ql, wl.num_q_heads, wl.head_dim)
        kv = workloads.decode_bytes(wl) - wl.num_seqs * wl.num_q_heads * wl.head_dim * 2 * \
            workloads.ELEM_BYTES[wl.q_dtype]
        qo = int(qsl[-1]) * wl.num_q_heads * wl.head_dim * 2 * workloads.ELEM_BYTES[wl.q_dtype]
        tf = fl / (ms * 1e-3) / 1e12
        print(json.dumps({
            "metric": "paged prefill TFLOP/s", "workload": name, "value": round(tf, 2),
            "unit": "TFLOP/s", "ms": round(ms, 4), "p10_ms": round(float(np.percentile(ts, 10)), 4),
            "p90_ms": round(float(np.percentile(ts, 90)), 4),
            "dtype": {"bf16": "bf16", "fp8_e4m3": "fp8-e4m3 KV, bf16 q"}[wl.pool_dtype],
            "config": {"num_seqs": wl.num_seqs, "num_q_heads": wl.num_q_heads,
                       "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                       "block_size": wl.block_size, "query_rows": int(qsl[-1]),
                       "context_max": int(wl.max_context_len)},
            "calls_per_sample": reps, "flops": fl, "bytes": int(kv + qo),
            "GBps": round((kv + qo) / (ms * 1e-3) / 1e9, 1),
            "roofline": {"kernel": "prefill_kernel", "bound": "mfma", "achieved": round(tf, 2),
                         "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / MFMA_PEAK_TFLOPS, 4)}}), flush=True)
        del cache, q, out


def _counter_rows(paths):
    """Per-dispatch counter sums from rocprofv3 counter_collection CSVs:
    {(file, dispatch id): {"kernel": name, counter: value}}."""
    import csv
    rows = {}
    for path in paths:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                key = (path, r["Dispatch_Id"])
                d = rows.setdefault(key, {"kernel": r["Kernel_Name"]})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return rows


# Read and write request counters of the L2's memory interface (EA).
# TCC_EA0_RDREQ counts every read request, TCC_EA0_RDREQ_32B the 32-byte
# ones; on MI355X every other read request is 128 bytes: a 1 GiB device copy
# issues exactly 2^23 of them, and TCC_BUBBLE, which rocprofv3's FETCH_SIZE
# takes for the 128-byte count (valuing the rest at 64 bytes), reads 0 --
# hence FETCH_SIZE reports half the bytes read. Writes are 32 or 64 bytes
# (TCC_EA0_WRREQ_64B the 64-byte ones; the copy writes 2^24 of them for
# 1 GiB). *_DRAM counts the requests that went on to DRAM (the rest were
# served by the Infinity Cache).
READ_COUNTERS = ["TCC_BUBBLE_sum", "TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum",
                 "TCC_EA0_RDREQ_DRAM_sum"]
WRITE_COUNTERS = ["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_DRAM_sum"]


def request_bytes(c):
    """(read bytes, write bytes) from one dispatch's request counts."""
    r128, rall, r32 = c["TCC_BUBBLE_sum"], c["TCC_EA0_RDREQ_sum"], c["TCC_EA0_RDREQ_32B_sum"]
    if r128 == 0:             # MI355X: every read request that is not 32 bytes is 128
        read = 128 * (rall - r32) + 32 * r32
    else:
        read = 128 * r128 + 64 * (rall - r128 - r32) + 32 * r32
    wall, w64 = c["TCC_EA0_WRREQ_sum"], c["TCC_EA0_WRREQ_64B_sum"]
    write = 64 * w64 + 32 * (wall - w64)
    return read, write


def counters_summary(spec):
    """profiles/traffic_<kernel>_<workload>.json from two rocprofv3 --pmc
    runs of `bench.py --config N` (READ_COUNTERS, then WRITE_COUNTERS): the
    kernel's memory read and write bytes counted from the L2's requests by
    size (request_bytes), averaged over its dispatches, against its
    algorithmic bytes; and the share of read requests that reached DRAM."""
    name, csvs = spec
    kernel, workload = name.split(":")
    rows = _counter_rows(csvs.split(","))
    mine = [d for d in rows.values() if kernel in d["kernel"]]
    if not mine:
        raise SystemExit(f"no dispatch of {kernel} in {csvs}")

    def avg(c):
        v = [d[c] for d in mine if c in d]
        return float(np.mean(v)) if v else None
    counts = {c: avg(c) for c in READ_COUNTERS + WRITE_COUNTERS}
    missing = [c for c, v in counts.items() if v is None]
    if missing:
        raise SystemExit(f"counters missing from {csvs}: {missing}")
    read, write = request_bytes(counts)
    import workloads
    if workload == "copy_1GiB":         # bench.py --copy-calibration: 1 GiB read, 1 GiB written
        ab = 2 << 30
    else:
        wl = workloads.make(wl_config(workload))
        ab = unique_decode_bytes(wl) - (workloads.decode_bytes(wl) - attend_bytes(wl))
    rec = {"kernel": mine[0]["kernel"], "workload": workload,
           "kernel_source_sha": kernel_source_hash(),
           "dispatches": len(mine) // 2,
           "requests_per_launch": {c: round(v, 1) for c, v in counts.items()},
           "hbm_read_bytes_per_launch": int(read),
           "hbm_write_bytes_per_launch": int(write),
           "hbm_bytes_per_launch": int(read + write),
           "dram_share_of_read_requests": round(counts["TCC_EA0_RDREQ_DRAM_sum"] /
                                                counts["TCC_EA0_RDREQ_sum"], 4),
           "algorithmic_bytes_per_launch": ab,
           "traffic_over_algorithmic": round((read + write) / ab, 4),
           "commands": [f"rocprofv3 --pmc {' '.join(cs)} --output-format csv -d <out> -o run -- "
                        + ("python bench.py --copy-calibration" if workload == "copy_1GiB" else
                           f"python bench.py --no-cpu-baseline --config {wl_config(workload)} "
                           "--steps 5 --warmup 2 --flush-iters 0")
                        for cs in (READ_COUNTERS, WRITE_COUNTERS)]}
    path = os.path.join(PROFILE_DIR, f"traffic_{kernel}_{workload}.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def wl_config(workload: str) -> int:
    return {"tiny_fp32": 1, "mha_fp16": 2, "gqa_bf16": 3, "shared_prefix_fp16": 4,
            "long_fp8": 5}[workload]


def launch_avg_ms(fn, reps: int) -> float:
    """Mean duration of one launch of fn: reps launches back to back between
    two HIP events on the launch stream (torch's current stream, which the
    binding launches on), so the events' own cost is spread over reps."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def decode_setup(wl, dev):
    """Device pool filled with every context token (untimed, as the workload
    prescribes), the step's write of each sequence's newest token, queries,
    tables, lengths and the output."""
    import torch
    import paged_kv_cache_44_amd as pa
    import workloads
    pool = wl.empty_pool()
    cache = pa.KVCache(codes_tensor(pool, wl.pool_dtype, dev), codes_tensor(pool, wl.pool_dtype, dev),
                       wl.pool_dtype, wl.num_blocks, wl.num_layers, wl.num_kv_heads,
                       wl.block_size, wl.head_dim, k_scale=wl.k_scale, v_scale=wl.v_scale)
    for op in workloads.fill_plan(wl):
        if op[0] == "write":
            pa.write_kv(cache, wl.layer, codes_tensor(op[1], wl.src_dtype, dev),
                        codes_tensor(op[2], wl.src_dtype, dev), torch.from_numpy(op[3]).to(dev))
        else:
            pa.copy_blocks(cache, cache, torch.from_numpy(op[1]).to(dev), "d2d")
    # the step's own write: each sequence's newest token, stored again at its slot
    step_idx = wl.step_token[wl.step_token >= 0]
    q = codes_tensor(wl.q, wl.q_dtype, dev)
    return types.SimpleNamespace(
        cache=cache, step_idx=step_idx,
        step_k=codes_tensor(wl.write_k[step_idx], wl.src_dtype, dev),
        step_v=codes_tensor(wl.write_v[step_idx], wl.src_dtype, dev),
        step_slots=torch.from_numpy(wl.write_slots[step_idx]).to(dev),
        q=q, out=torch.empty_like(q), tables=torch.from_numpy(wl.block_tables).to(dev),
        ctx=torch.from_numpy(wl.context_lens).to(dev), max_ctx=wl.max_context_len)


def block_size_sweep(steps: int, warmup: int):
    """Decode block-size sweep ("Efficient Memory Management for Large Language
    Model Serving with PagedAttention", block-size paragraph: small blocks
    give the kernel less to read per block-table entry, large ones leave more
    of a sequence's last block empty). The GQA bf16 workload's lengths at
    each block size: the whole step (newest-token write, attend, merge) timed
    without events, the attention kernel alone from HIP events around a run
    of back-to-back launches,
    and the slots the sequences' blocks hold beyond their contexts."""
    import torch
    import paged_kv_cache_44_amd as pa
    import workloads
    dev = torch.device("cuda:0")
    rows = []
    for B in (8, 16, 32, 64, 128, 256):
        wl = workloads.config3(block_size=B)
        print(f"[bench] block size {B}: {wl.num_blocks} blocks", file=sys.stderr, flush=True)
        d = decode_setup(wl, dev)
        S, Hq = wl.num_seqs, wl.num_q_heads
        ws = torch.empty(max(1, pa.decode_workspace_size(d.cache, S, Hq, d.max_ctx)),
                         dtype=torch.uint8, device=dev)
        def attend():
            pa.decode_attend(d.cache, wl.layer, d.q, d.tables, d.ctx, d.max_ctx, wl.scale, d.out, ws)

        def step():
            pa.write_kv(d.cache, wl.layer, d.step_k, d.step_v, d.step_slots)
            attend()
            pa.decode_merge(d.cache, wl.layer, d.q, d.tables, d.ctx, d.max_ctx, wl.scale, d.out, ws)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        attend_ms = launch_avg_ms(attend, steps)
        step_bytes = workloads.decode_bytes(wl) + workloads.write_bytes(wl, len(d.step_idx))
        held = int(np.sum(-(-wl.context_lens.astype(np.int64) // B))) * B
        used = int(wl.context_lens.sum())
        rec = {"block_size": B, "ms_per_step": round(ms, 5),
               "step_GBps": round(step_bytes / (ms * 1e-3) / 1e9, 2),
               "attend_ms": round(attend_ms, 5),
               "attend_GBps": round(attend_bytes(wl) / (attend_ms * 1e-3) / 1e9, 2),
               "slots_held": held, "slots_used": used,
               "slots_unused_pct": round(100.0 * (held - used) / held, 2)}
        print(json.dumps(rec), flush=True)
        rows.append(rec)
        del d, ws
        torch.cuda.empty_cache()
    return rows


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (empty if unreadable)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def host_workers() -> int:
    """Worker processes for the pooled oracle run: the cores this process may
    run on, capped by OMP_NUM_THREADS where the host sets it (the CPU share
    a GPU machine gives one GPU)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


# the oracle's pools for the pooled run, inherited by forked workers
_ORACLE = {}


def _oracle_pools(wl):
    from oracle import paged
    import workloads
    geom = paged.Geometry(wl.num_blocks, wl.num_layers, wl.num_kv_heads, wl.block_size,
                          wl.head_dim)
    ok = wl.empty_pool()
    ov = ok.copy()
    for op in workloads.fill_plan(wl):
        if op[0] == "write":
            ok, ov = paged.write_kv(ok, ov, geom, wl.pool_dtype, wl.layer, op[1], op[2],
                                    wl.src_dtype, op[3], wl.k_scale, wl.v_scale)
        else:
            ok, ov = paged.copy_blocks(ok, ov, geom, ok, ov, geom, op[1], same_pool=True)
    return geom, ok, ov


def _oracle_seq(s: int) -> int:
    """One sequence's decode by the oracle (in a worker); returns its bytes."""
    from oracle import paged
    import workloads
    wl, geom, ok, ov = _ORACLE["wl"], _ORACLE["geom"], _ORACLE["ok"], _ORACLE["ov"]
    paged.decode(wl.q, wl.q_dtype, ok, ov, geom, wl.pool_dtype, wl.layer, wl.block_tables,
                 wl.context_lens, wl.scale, wl.k_scale, wl.v_scale, seqs=[s])
    return workloads.decode_bytes(wl, wl.context_lens[s:s + 1])


def _one_blas_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def cpu_baseline(wl, target_s: float):
    """The oracle, as it is, on the host cores. Its slot write builds the pool
    on the host; then its decode runs sequence by sequence (cycling through
    the workload) for about target_s seconds in one process with BLAS on one
    thread, and again for about target_s seconds in a pool of host_workers()
    forked processes (one BLAS thread each) that take sequences in turn.
    Must run before this process initialises the GPU (the pool forks)."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    geom, ok, ov = _oracle_pools(wl)
    _ORACLE.update(wl=wl, geom=geom, ok=ok, ov=ov)
    S = wl.num_seqs
    # one process
    done_bytes, seqs = 0, 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < target_s:
            done_bytes += _oracle_seq(seqs % S)
            seqs += 1
        dt1 = time.perf_counter() - t0
    one = {"value": round(done_bytes / dt1 / 1e9, 4), "seq_per_s": round(seqs / dt1, 3),
           "seconds": round(dt1, 2), "sequences": seqs}
    # a pool of forked workers, in rounds of whole passes over the batch (or
    # of one sequence per worker when a pass is long) until target_s is spent
    n = host_workers()
    ctx = mp.get_context("fork")
    pbytes, pseqs = 0, 0
    with ctx.Pool(n, initializer=_one_blas_thread) as pool:
        pool.map(_oracle_seq, [0] * n)                      # start-up outside the timing
        chunk = max(S, n)
        t0 = time.perf_counter()
        nxt = 0
        while time.perf_counter() - t0 < target_s:
            idx = [(nxt + i) % S for i in range(chunk)]
            nxt += chunk
            pbytes += sum(pool.map(_oracle_seq, idx, chunksize=max(1, len(idx) // (4 * n))))
            pseqs += chunk
        dtn = time.perf_counter() - t0
    _ORACLE.clear()
    pooled = {"value": round(pbytes / dtn / 1e9, 4), "seq_per_s": round(pseqs / dtn, 3),
              "seconds": round(dtn, 2), "sequences": pseqs, "workers": n}
    return {"value": pooled["value"], "unit": "GB/s", "cores": n, "kind": "oracle",
            "cpu_model": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0)),
            "sample": (f"the workload's sequences decoded one at a time by the numpy fp64 oracle, "
                       f"cycling through the batch: {pseqs} decodes in {dtn:.1f} s over {n} "
                       f"worker processes (one BLAS thread each); single process: {seqs} "
                       f"decodes in {dt1:.1f} s"),
            "single_process": one, "pooled": pooled}


def main():
    args = parse()
    if args.print_source_hash:
        print(kernel_source_hash())
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path; each GPU would decode its own share)",
              file=sys.stderr)
        sys.exit(2)
    if args.reuse_plan and not args.shared:
        print("--reuse-plan applies to --shared only", file=sys.stderr)
        sys.exit(2)
    import torch
    import paged_kv_cache_44_amd as pa
    import workloads

    if args.counters_summary:
        counters_summary(args.counters_summary)
        return
    plain = not (args.copy_calibration or args.swap or args.swap_sweep or args.block_size_sweep
                 or args.prefill)
    # the CPU oracle first, before this process touches the GPU (its worker
    # pool forks); the host measurement does not depend on the order
    cpu = None
    if plain and not args.no_cpu_baseline:
        cpu = cpu_baseline(workloads.make(args.config), args.cpu_seconds)
        print(f"[bench] cpu baseline: {cpu['value']} GB/s over {cpu['cores']} workers, "
              f"{cpu['single_process']['value']} GB/s in one process", file=sys.stderr, flush=True)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    if args.swap:
        swap_bench()
        return
    if args.swap_sweep:
        swap_sweep()
        swap_overlap()
        return
    if args.block_size_sweep:
        block_size_sweep(args.steps, args.warmup)
        return
    if args.prefill:
        prefill_bench(args.steps if args.steps != 50 else 20, args.warmup if args.warmup != 10 else 3)
        return
    dev = torch.device("cuda:0")
    t_setup = time.perf_counter()
    wl = workloads.make(args.config)
    print(f"[bench] workload {wl.name}: {wl.num_seqs} seqs, ctx mean "
          f"{wl.context_lens.mean():.1f} max {wl.max_context_len}, pool {wl.num_blocks} blocks",
          file=sys.stderr, flush=True)

    d = decode_setup(wl, dev)
    cache, step_idx, step_k, step_v, step_slots = d.cache, d.step_idx, d.step_k, d.step_v, d.step_slots
    q, out, tables, ctx, max_ctx = d.q, d.out, d.tables, d.ctx, d.max_ctx
    S, Hq = wl.num_seqs, wl.num_q_heads
    ws_n = (pa.decode_shared_workspace_size(cache, S, Hq) if args.shared
            else pa.decode_workspace_size(cache, S, Hq, max_ctx))
    ws = torch.empty(max(1, ws_n), dtype=torch.uint8, device=dev)
    part = pa.decode_partition_tokens(cache, S, Hq, max_ctx)
    torch.cuda.synchronize()
    print(f"[bench] setup {time.perf_counter() - t_setup:.1f} s; partition {part} tokens",
          file=sys.stderr, flush=True)

    planned = [False]

    def attend():
        if args.shared:     # planning (unless reused), prefix pass, suffix pass and merges
            pa.decode_shared(cache, wl.layer, q, tables, ctx, max_ctx, wl.scale, out=out,
                             workspace=ws, reuse_plan=args.reuse_plan and planned[0])
            planned[0] = True
        else:
            pa.decode_attend(cache, wl.layer, q, tables, ctx, max_ctx, wl.scale, out, ws)

    def step():
        pa.write_kv(cache, wl.layer, step_k, step_v, step_slots)
        attend()
        if not args.shared:
            pa.decode_merge(cache, wl.layer, q, tables, ctx, max_ctx, wl.scale, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    # the attention kernel's own duration (the timed steps above carry no
    # events: recording one costs the stream ~3 us)
    attend_ms = launch_avg_ms(attend, args.steps)

    # flushed per-call decode time: a 512 MiB scratch write evicts the L2s and
    # the Infinity Cache before each call (untimed)
    scratch = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    fl = []
    for _ in range(0 if args.shared else args.flush_iters):
        scratch.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        pa.decode_attend(cache, wl.layer, q, tables, ctx, max_ctx, wl.scale, out, ws)
        pa.decode_merge(cache, wl.layer, q, tables, ctx, max_ctx, wl.scale, out, ws)
        b.record()
        torch.cuda.synchronize()
        fl.append(a.elapsed_time(b))
    del scratch

    # the method's bytes: every physical slot in use read once, however many
    # sequences share it (equal to the logical count unless blocks are
    # shared, as the shared-prefix workload's prompts are)
    uniq = unique_decode_bytes(wl)
    wbytes = workloads.write_bytes(wl, len(step_idx))
    step_bytes = uniq + wbytes
    logical_step_bytes = workloads.decode_bytes(wl) + wbytes
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    ab = uniq - (workloads.decode_bytes(wl) - attend_bytes(wl))
    kname = attend_kernel_name(wl)
    traffic = load_traffic(kname, wl.name)
    if args.shared:
        # the whole shared decode (planning, both passes, merges) against the
        # bytes it must read at the least
        kname = ("decode_shared (prefix and suffix passes, merges; plan reused)" if args.reuse_plan
                 else "decode_shared (plan, prefix and suffix passes, merges)")
        traffic = None
    achieved = ab / (attend_ms * 1e-3) / 1e9
    rec = {
        "metric": "paged-decode KV GB/s and % of MI355X HBM peak; sequences/s at 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16", "bf16": "bf16", "fp8_e4m3": "fp8-e4m3 KV, bf16 q"}[wl.pool_dtype],
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": wl.num_kv_heads,
            "head_dim": wl.head_dim, "block_size": wl.block_size,
            "context_mean": round(float(wl.context_lens.mean()), 1),
            "context_max": max_ctx, "context_tokens": int(wl.context_lens.sum()),
            "partition_tokens": part, "parallelism": "single GPU",
            **({"decode": "pa_decode_shared" + (", sharing plan reused" if args.reuse_plan else "")}
               if args.shared else {}),
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_per_s": round(S / (ms_per_step * 1e-3), 1),
        "step_bytes": step_bytes,
        "unique_decode_bytes": uniq,
        "logical_step_bytes": logical_step_bytes,
        "logical_GBps": round(logical_step_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "attend_logical_GBps": round(attend_bytes(wl) / (attend_ms * 1e-3) / 1e9, 2),
        "decode_flushed_ms": ({"median": round(float(np.median(fl)), 5),
                               "p10": round(float(np.percentile(fl, 10)), 5),
                               "p90": round(float(np.percentile(fl, 90)), 5)} if fl else None),
        "roofline": {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": ab,
                     "avg_launch_ms": round(attend_ms, 5)},
        "cpu_baseline": cpu,
        "page_context": PAGE_CONTEXT,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
