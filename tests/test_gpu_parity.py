"""GPU parity of the five workloads against the oracle, through the C ABI.

Slot writes and block copies must match the oracle byte for byte over the
whole pool (never-written slots included); decode outputs must be finite and
within the max-abs tolerance of the workload's dtype: 1e-5 fp32, 2e-3 fp16,
1e-2 bf16, 3e-2 fp8 KV.
"""

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_helpers import DeviceState, TOL, max_err, say, codes_to_tensor, tensor_codes
from oracle import blocks as oblocks, codecs, paged

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request, gpu):
    say(f"\n[gpu] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def _fill(st):
    wl = st.wl
    st.write(wl.write_k, wl.write_v, wl.write_slots)
    same, _, _ = st.pools_equal_oracle()
    assert same, "pool bytes differ from the oracle after the write"


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_plain_configs_write_and_decode(cfg):
    wl = workloads.make(cfg)
    say(f"config {cfg} {wl.name}: S={wl.num_seqs} ctx mean {wl.context_lens.mean():.1f} "
        f"max {wl.max_context_len} blocks {wl.num_blocks}")
    st = DeviceState(wl)
    _fill(st)
    got = st.decode()
    ref = st.oracle_decode()
    assert np.all(np.isfinite(got))
    err = max_err(got, ref)
    say(f"config {cfg}: max abs err {err:.3e} (tol {TOL[wl.pool_dtype]})")
    assert err <= TOL[wl.pool_dtype]


def _shared_prefix_flow(wl):
    st = DeviceState(wl)
    n0 = wl.extra["num_prefix_tokens_written"]
    st.write(wl.write_k[:n0], wl.write_v[:n0], wl.write_slots[:n0])
    st.copy_d2d(wl.extra["cow_pairs"])
    st.write(wl.write_k[n0:], wl.write_v[n0:], wl.write_slots[n0:])
    return st


@pytest.mark.parametrize("prefix", [1024, 1020])
def test_shared_prefix_cow_write_and_decode(prefix):
    kw = {} if prefix == 1024 else dict(prefix_tokens=1020)
    wl = workloads.config4(**kw)
    say(f"shared-prefix fp16, prefix {prefix}: S={wl.num_seqs} cow pairs {len(wl.extra['cow_pairs'])}")
    st = _shared_prefix_flow(wl)
    same, _, _ = st.pools_equal_oracle()
    assert same
    got = st.decode()
    ref = st.oracle_decode()
    assert np.all(np.isfinite(got))
    err = max_err(got, ref)
    say(f"shared-prefix fp16: max abs err {err:.3e}")
    assert err <= TOL["f16"]


def test_shared_blocks_unchanged_by_private_writes():
    """Copy-on-write: after the copies and the private writes the shared
    prompt blocks still hold exactly the prompt's bytes."""
    wl = workloads.config4(groups=4, prefix_tokens=1020)
    st = DeviceState(wl)
    n0 = wl.extra["num_prefix_tokens_written"]
    st.write(wl.write_k[:n0], wl.write_v[:n0], wl.write_slots[:n0])
    torch.cuda.synchronize()
    before = tensor_codes(st.cache.k).copy()
    st.copy_d2d(wl.extra["cow_pairs"])
    st.write(wl.write_k[n0:], wl.write_v[n0:], wl.write_slots[n0:])
    torch.cuda.synchronize()
    after = tensor_codes(st.cache.k)
    bs = wl.block_stride()
    for g, pb in enumerate(wl.extra["prefix_blocks"]):
        for b in pb[:-1]:
            assert np.array_equal(before[b * bs:(b + 1) * bs], after[b * bs:(b + 1) * bs])
        # each copy equals the original block as it was when copied
        for src, dst in wl.extra["cow_pairs"]:
            if src == pb[-1]:
                blk = after[dst * bs:(dst + 1) * bs]
                orig = before[src * bs:(src + 1) * bs]
                # prompt slots (0..11) identical; slots 12.. hold the sample's own tokens
                s5 = blk.reshape(wl.num_kv_heads, wl.block_size, wl.head_dim)
                o5 = orig.reshape(wl.num_kv_heads, wl.block_size, wl.head_dim)
                assert np.array_equal(s5[:, :12], o5[:, :12])


def test_long_fp8_with_swap_in():
    wl = workloads.config5()
    ex = wl.extra
    say(f"long FP8: S={wl.num_seqs} ctx {list(wl.context_lens)} k_scale {wl.k_scale:.5g} "
        f"v_scale {wl.v_scale:.5g}")
    st = DeviceState(wl)
    _fill(st)
    # the victim first lives in its original blocks
    st.write(ex["victim_k"], ex["victim_v"], ex["victim_slots_before"])
    hb = ex["host_pool_blocks"]
    hgeom = paged.Geometry(hb, 1, wl.num_kv_heads, wl.block_size, wl.head_dim)
    hk0 = np.full(hgeom.pool_elements(), 0x7F, np.uint8)
    out_pairs = np.stack([ex["victim_blocks_before"], ex["victim_host_blocks"]], 1)
    hk, hv = paged.copy_blocks(hk0, hk0.copy(), hgeom, st.ok, st.ov, st.geom, out_pairs)
    # swap out to pinned host blocks
    host = type(st.cache).empty(wl.pool_dtype, hb, 1, wl.num_kv_heads, wl.block_size, wl.head_dim,
                                pin_memory=True, k_scale=wl.k_scale, v_scale=wl.v_scale)
    host.k.fill_(0x7F)
    host.v.fill_(0x7F)
    from paged_kv_cache_44_amd import copy_blocks
    copy_blocks(host, st.cache, torch.from_numpy(out_pairs.copy()), "d2h")
    # release and reuse: the original blocks are overwritten right after, on the
    # same stream; the host copy must already hold the victim's bytes
    junk = np.full((len(ex["victim_slots_before"]), wl.num_kv_heads, wl.head_dim), 0x3F80,
                   dtype=np.uint16)
    st.write(junk, junk, ex["victim_slots_before"])
    torch.cuda.synchronize()
    assert np.array_equal(tensor_codes(host.k), hk)
    assert np.array_equal(tensor_codes(host.v), hv)
    # swap in to different blocks
    in_pairs = np.stack([ex["victim_host_blocks"], ex["victim_blocks_after"]], 1)
    copy_blocks(st.cache, host, torch.from_numpy(in_pairs.copy()), "h2d")
    st.ok, st.ov = paged.copy_blocks(st.ok, st.ov, st.geom, hk, hv, hgeom, in_pairs)
    same, _, _ = st.pools_equal_oracle()
    assert same
    got = st.decode()
    ref = st.oracle_decode()
    assert np.all(np.isfinite(got))
    err = max_err(got, ref)
    say(f"long FP8: max abs err {err:.3e}")
    assert err <= TOL["fp8_e4m3"]
