"""Shared-prefix decode (pa_decode_shared) on the GPU against the oracle's
ordinary decode: parallel samples of several prompts (consecutive sequences
whose tables name the prompt's blocks, copy-on-write of a partly filled last
prompt block), over pool / query dtypes, head dims, group sizes and block
sizes; runs longer than one tile of samples, prefixes that are not a
multiple of 16, contexts that are all prefix, singletons, empty and invalid
rows inside runs, a reused plan, the split of the launch between the two
passes at its extremes (no sharing, one short prefix, contexts that are all
prefix), and the shared-prefix workload at full size on sampled sequences. The pages fix the result: sharing blocks does not
change the attention ("Efficient Memory Management for Large Language Model
Serving with PagedAttention", kernel and sampling paragraphs)."""

import numpy as np
import pytest
import torch

import paged_kv_cache_44_amd as pa
import workloads
from oracle import codecs
from tests.gpu_helpers import DeviceState, TOL, codes_to_tensor, max_err_stored, say, tensor_codes

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request, gpu):
    say(f"\n[gpu] {request.node.nodeid}")
    yield
    torch.cuda.synchronize()


GROUPS = [(40, [5, 0, 17]), (32, [0, 0]), (7, [3]), (100, [1, 2, 3, 4, 5, 6, 7, 8, 9]),
          (300, [20, 64, 0, 33, 16]), (16, [0, 40]), (64, [70])]

COMBOS = [
    # pool,       q,      D,  G,  B, H_kv
    ("f16", "f16", 128, 4, 16, 2),
    ("bf16", "bf16", 128, 8, 16, 1),
    ("bf16", "bf16", 64, 2, 8, 2),
    ("fp8_e4m3", "bf16", 128, 4, 32, 2),
    ("f16", "f16", 64, 1, 16, 3),
    ("fp8_e4m3", "f16", 64, 8, 16, 1),
    ("f16", "f16", 128, 2, 64, 2),
]


def _state(wl):
    st = DeviceState(wl)
    for op in workloads.fill_plan(wl):
        if op[0] == "write":
            st.write(op[1], op[2], op[3])
        else:
            st.copy_d2d(op[1])
    return st


def _shared(st, q_codes=None, ctx=None, max_ctx=None, reuse=False, ws=None):
    wl = st.wl
    q = codes_to_tensor(wl.q if q_codes is None else q_codes, wl.q_dtype)
    ctx = wl.context_lens if ctx is None else ctx
    tt = torch.from_numpy(np.ascontiguousarray(wl.block_tables, dtype=np.int32)).cuda()
    ct = torch.from_numpy(np.ascontiguousarray(ctx, dtype=np.int32)).cuda()
    mc = int(np.max(ctx)) if max_ctx is None else max_ctx
    out = pa.decode_shared(st.cache, wl.layer, q, tt, ct, mc, wl.scale, workspace=ws,
                           reuse_plan=reuse)
    torch.cuda.synchronize()
    return codecs.decode(tensor_codes(out), wl.q_dtype)


def _tol(wl):
    return TOL["fp8_e4m3"] if wl.pool_dtype == "fp8_e4m3" else TOL[wl.q_dtype]


@pytest.mark.parametrize("combo", COMBOS, ids=lambda c: "-".join(map(str, c)))
def test_shared_decode_matches_oracle(combo):
    pool, qd, D, G, B, hkv = combo
    wl = workloads.shared_prefix(11, GROUPS, pool_dtype=pool, q_dtype=qd,
                                 num_q_heads=hkv * G, num_kv_heads=hkv, head_dim=D,
                                 block_size=B)
    st = _state(wl)
    got = _shared(st)
    ref = st.oracle_decode()
    ex = max_err_stored(got, ref, wl.q_dtype, _tol(wl))
    say(f"{combo}: {wl.num_seqs} seqs, error beyond output rounding {ex:.3e}")
    assert np.all(np.isfinite(got)) and ex <= _tol(wl)


# Runs long enough to fill both 16-column tiles of a prefix slot and spill
# into further slots: a slot holds 32 / G samples (32 at G = 1, 16 at G = 2),
# so 40 samples take 32 + 8, 33 take 32 + 1; a partly filled last prompt
# block (200 tokens), and samples whose context is all prompt.
MANY = [(200, [int(x) for x in np.random.default_rng(5).integers(0, 50, 40)]),
        (33, [int(x) for x in np.random.default_rng(6).integers(0, 30, 17)]),
        (16, [0, 0, 0] + [5] * 30)]


@pytest.mark.parametrize("pool,q,G,hkv", [("f16", "f16", 1, 2), ("bf16", "bf16", 1, 1),
                                          ("fp8_e4m3", "bf16", 1, 2), ("bf16", "bf16", 2, 2)])
def test_runs_filling_both_prefix_tiles(pool, q, G, hkv):
    wl = workloads.shared_prefix(13, MANY, pool_dtype=pool, q_dtype=q, num_q_heads=hkv * G,
                                 num_kv_heads=hkv, head_dim=128, block_size=16)
    st = _state(wl)
    got = _shared(st)
    ref = st.oracle_decode()
    err = max_err_stored(got, ref, wl.q_dtype, _tol(wl))
    say(f"{wl.num_seqs} sequences, G {G}: error beyond output rounding {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= _tol(wl)


# The launch splits its workgroups between the passes by the plan's chunk
# counts: a batch with no sharing gives the prefix pass none; one short
# shared prefix among long private contexts gives it the least (one round
# of the XCDs); contexts that are all prefix give the suffix pass the least.
_R = np.random.default_rng(17)
SPLITS = {
    "no_sharing": [(int(p), [int(t)]) for p, t in zip(_R.integers(20, 600, 24), _R.integers(0, 60, 24))],
    "one_short_prefix": [(16, [3, 5])] + [(600, [int(t)]) for t in _R.integers(1, 80, 20)],
    "all_prefix": [(512, [0] * 8), (256, [0] * 8), (160, [0, 0, 0])],
}


@pytest.mark.parametrize("case", sorted(SPLITS))
@pytest.mark.parametrize("pool,q,G,hkv", [("f16", "f16", 4, 2), ("fp8_e4m3", "bf16", 8, 1)])
def test_split_extremes(case, pool, q, G, hkv):
    wl = workloads.shared_prefix(14, SPLITS[case], pool_dtype=pool, q_dtype=q, num_q_heads=hkv * G,
                                 num_kv_heads=hkv, head_dim=128, block_size=16)
    st = _state(wl)
    got = _shared(st)
    ref = st.oracle_decode()
    err = max_err_stored(got, ref, wl.q_dtype, _tol(wl))
    say(f"{case}: {wl.num_seqs} sequences, error beyond output rounding {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= _tol(wl)


def test_empty_and_invalid_rows_inside_runs_and_plan_reuse():
    groups = [(48, [4, 0, 9, 2]), (33, [1, 1, 1])]
    wl = workloads.shared_prefix(12, groups, pool_dtype="bf16", q_dtype="bf16", num_q_heads=8,
                                 num_kv_heads=2, head_dim=128, block_size=16)
    st = _state(wl)
    ctx = wl.context_lens.copy()
    ctx[1] = 0                                    # empty context inside the first run
    ctx[5] = 10_000                               # beyond max_context_len: invalid
    mc = int(wl.context_lens.max())
    got = _shared(st, ctx=ctx, max_ctx=mc)
    ok = [s for s in range(wl.num_seqs) if s not in (1, 5)]
    ref = st.oracle_decode(ctx=np.where(ctx > mc, 0, ctx), seqs=ok)
    assert np.all(got[1] == 0)
    assert np.all(np.isnan(got[5]))
    ex = max_err_stored(got, ref, "bf16", TOL["bf16"], rows=ok)
    say(f"error beyond output rounding {ex:.3e}")
    assert ex <= TOL["bf16"]
    # a second call with other queries reuses the plan left in the workspace
    ws = torch.empty(pa.decode_shared_workspace_size(st.cache, wl.num_seqs, wl.num_q_heads),
                     dtype=torch.uint8, device="cuda")
    _shared(st, ws=ws)
    q2 = workloads.normal_codes(np.random.default_rng(5), wl.q.shape, "bf16")
    got2 = _shared(st, q_codes=q2, ws=ws, reuse=True)
    ref2 = st.oracle_decode(q_codes=q2)
    ex2 = max_err_stored(got2, ref2, "bf16", TOL["bf16"])
    say(f"reused plan: error beyond output rounding {ex2:.3e}")
    assert ex2 <= TOL["bf16"]


def test_shared_prefix_workload_full_size_sampled():
    wl = workloads.config4()
    st = _state(wl)
    got = _shared(st)
    rng = np.random.default_rng(4)
    seqs = sorted(rng.choice(wl.num_seqs, 12, replace=False).tolist())
    ref = st.oracle_decode(seqs=seqs)
    ex = max_err_stored(got, ref, wl.q_dtype, TOL[wl.q_dtype], rows=seqs)
    say(f"shared-prefix workload, sequences {seqs}: error beyond output rounding {ex:.3e}")
    assert np.all(np.isfinite(got)) and ex <= TOL[wl.q_dtype]
    plain = st.decode()
    assert np.max(np.abs(plain - got)) <= 2 * TOL[wl.q_dtype]
