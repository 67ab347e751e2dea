"""pa_decode_no_alloc on the GPU, through the C ABI: the same output as
pa_decode (bit for bit; both run the same kernels with the same launch
sizes) and within the stated bound of the oracle, for two calls in a row on
each path, the second with a smaller batch, so it starts from whatever the
first left in the library's fixed array."""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_44_amd as pa
import workloads
from oracle import codecs
from paged_kv_cache_44_amd import _binding as B
from tests.gpu_helpers import (DeviceState, TOL, codes_to_tensor, max_err, max_err_stored, say,
                               tensor_codes)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request, gpu):
    say(f"\n[gpu] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


def _no_alloc(st, q, tables, ctx, max_ctx):
    """One pa_decode_no_alloc call via ctypes; returns the output tensor."""
    wl = st.wl
    out = torch.full_like(q, float("nan"))
    c = st.cache.struct()
    lib = B.load_library()
    s = lib.pa_decode_no_alloc(
        ctypes.byref(c), wl.layer, ctypes.c_void_p(q.data_ptr()), pa.DTYPES[wl.q_dtype],
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(tables.data_ptr()),
        int(tables.shape[1]), ctypes.c_void_p(ctx.data_ptr()), int(max_ctx), int(q.shape[0]),
        int(q.shape[1]), float(wl.scale),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    B.check(s, "pa_decode_no_alloc")
    return out


CASES = [
    # name, pool, q, H_q, H_kv, D, B, first contexts, second (smaller) contexts
    ("gqa_bf16", "bf16", "bf16", 32, 8, 128, 16,
     list(np.random.default_rng(61).integers(200, 3000, 96)), [1, 17, 300, 40, 999]),
    ("long_fp8", "fp8_e4m3", "bf16", 64, 8, 128, 16, [8192, 20000, 12345, 31000], [5000, 700]),
    ("mha_f16", "f16", "f16", 40, 40, 128, 16,
     list(np.random.default_rng(62).integers(128, 2048, 32)), [1, 2047, 64]),
    ("valu_f32", "f32", "f32", 8, 2, 64, 16, [1, 900, 4000, 2500, 7], [3, 1500]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_no_alloc_matches_decode_twice(case):
    name, pool, q, hq, hkv, d, bs, ctx1, ctx2 = case
    for call, ctx in enumerate((ctx1, ctx2)):
        wl = workloads.custom(70 + call + 10 * CASES.index(case), ctx, pool_dtype=pool, q_dtype=q,
                              num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs)
        need = pa.decode_workspace_size(DeviceState(wl).cache, wl.num_seqs, hq, wl.max_context_len)
        assert need <= B.DECODE_NO_ALLOC_MAX_BYTES
        st = DeviceState(wl)
        st.write(wl.write_k, wl.write_v, wl.write_slots)
        qt = codes_to_tensor(wl.q, q)
        tt = torch.from_numpy(wl.block_tables).cuda()
        ct = torch.from_numpy(wl.context_lens).cuda()
        mc = wl.max_context_len
        out = _no_alloc(st, qt, tt, ct, mc)
        ref_out = pa.decode(st.cache, wl.layer, qt, tt, ct, mc, wl.scale)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), ref_out.view(torch.uint8)), \
            f"{name} call {call}: differs from pa_decode"
        got = codecs.decode(tensor_codes(out), q)
        ref = st.oracle_decode()
        tol = TOL["fp8_e4m3"] if pool == "fp8_e4m3" else TOL[q]
        ex = max_err(got, ref) if q == "f32" else max_err_stored(got, ref, q, tol)
        say(f"{name} call {call}: {wl.num_seqs} seqs (workspace {need} B), error {ex:.3e}")
        assert np.all(np.isfinite(got)) and ex <= tol
