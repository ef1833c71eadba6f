"""Graph capture of the device-side path (MI355X only).

The library launches kernels only: no allocation, memset or synchronisation inside a
call, so a fixed plan's calls can be captured into a HIP graph and replayed.  Each case
captures one path, replays it several times with the program's own eager work and
synchronisations in between, and checks every replay bit for bit against the eager
result (the kernels are deterministic).
"""

import sys

import numpy as np
import pytest
import torch

import position_independent_kv_rope_amd as P
from position_independent_kv_rope_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()


def say(*a):
    print("[gpu-graph]", *a, flush=True)
    sys.stdout.flush()


def replay_and_compare(fn, outputs, reps=3):
    """Eager run, capture, then replays interleaved with eager work; every replay's
    outputs must equal the eager ones bit for bit."""
    fn()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as capture expects
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for rep in range(reps):
        for o in outputs:
            o.fill_(float("nan"))
        fn()  # eager work between replays
        torch.cuda.synchronize()
        for o in outputs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outputs, want):
            assert torch.equal(o, w), ("replay", rep)
        say("replay", rep, "matches the eager result")


@pytest.mark.parametrize("one_launch", [False, True], ids=["two_calls", "rope_splice"])
def test_graph_contiguous_step(one_launch):
    # restore K from a pristine copy, rotate, splice, attend: the whole one-batch path
    # (rotation and splice as two calls, or as the one pic_rope_splice launch)
    # 4 x 4096 + 64 tokens: keys split into segments, so the merge kernel is captured too
    wl = W.Workload("graph_ctx", "bf16", 32, 8, 128, 500000.0, 16, [W.Request([4096] * 4, 64)],
                    seed=93)
    r = wl.requests[0]
    plan = P.pic_build_index([r.chunk_lens], [r.q_len], wl.k, wl.h_q, wl.h_kv, n_cu=2)
    plan.to_device()
    assert plan[P.H_N_MERGE] > 0  # the merge kernel is part of the graph
    k0, v0 = (t.cuda() for t in W.context_tensors(wl))
    q, kf, vf = (t.cuda() for t in W.fresh_tensors(wl, plan.n_rows))
    k, v = k0.clone(), v0.clone()
    out = torch.empty_like(q)
    ws = P.attn_workspace(plan, wl.head_dim)
    say("contiguous step", plan.n_tokens, "tokens", plan.n_rows, "rows")

    def fn():
        k.copy_(k0)
        v.copy_(v0)
        if one_launch:
            P.pic_rope_splice(plan, k, v, kf, vf, wl.rope_base)
        else:
            P.pic_rope_delta(plan, k, wl.rope_base)
            P.pic_splice(plan, k, v, kf, vf)
        P.pic_selective_attn(plan, q, k, v, out, workspace=ws)

    replay_and_compare(fn, [out, k])


def _pool_case():
    lens = [3000, 17, 2600, 64, 1290, 250]
    reqs = [W.Request([lens[i] for i in ids], qn, chunk_ids=ids)
            for ids, qn in (([0, 2, 4], 40), ([5, 1, 0, 3], 9), ([2], 3))]
    wl = W.Workload("graph_pool", "bf16", 32, 4, 128, 500000.0, 8, reqs, pool_lens=lens,
                    block_size=16, pool_block_perm_seed=9, seed=91)
    plan = P.pic_build_index([r.chunk_lens for r in reqs], [r.q_len for r in reqs], wl.k,
                             wl.h_q, wl.h_kv, n_cu=256, chunk_ids_per_req=[r.chunk_ids for r in reqs])
    plan.to_device()
    cbp, blocks = W.pool_block_table(wl)
    pk, pv = (t.cuda() for t in W.pool_tensors(wl))
    q, kf, vf = (t.cuda() for t in W.fresh_tensors(wl, plan.n_rows))
    return wl, plan, pk, pv, torch.from_numpy(cbp).cuda(), torch.from_numpy(blocks).cuda(), q, kf, vf


def test_graph_paged_prefill():
    wl, plan, pk, pv, cbp, blocks, q, kf, vf = _pool_case()
    out = torch.empty_like(q)
    ws = P.attn_workspace(plan, wl.head_dim)
    say("paged prefill items=%d merges=%d" % (plan[P.H_N_ATTN_ITEMS], plan[P.H_N_MERGE]))
    assert plan[P.H_N_MERGE] > 0
    replay_and_compare(lambda: P.pic_selective_attn_paged(plan, q, pk, pv, cbp, blocks, kf, vf, out,
                                                          wl.rope_base, workspace=ws), [out])


def test_graph_decode():
    wl, plan, pk, pv, cbp, blocks, _, kf, vf = _pool_case()
    qn, kn, vn = (t.cuda() for t in W.decode_tensors(wl))
    out = torch.empty_like(qn)
    ws = P.decode_workspace(plan, wl.head_dim)
    say("decode pieces=%d records=%d" % (plan[P.H_N_DEC_PIECES], plan[P.H_N_DEC_RECS]))
    replay_and_compare(lambda: P.pic_decode_attn_paged(plan, qn, kn, vn, pk, pv, cbp, blocks, kf, vf,
                                                       out, wl.rope_base, workspace=ws), [out])


def test_graph_pool_gather():
    # the gather form of the pool path: pool blocks -> contiguous rotated K/V with the
    # fresh rows spliced in (paged plan), then the contiguous attention (plan of the same
    # requests without chunk ids)
    wl, plan, pk, pv, cbp, blocks, q, kf, vf = _pool_case()
    reqs = wl.requests
    cplan = P.pic_build_index([r.chunk_lens for r in reqs], [r.q_len for r in reqs], wl.k,
                              wl.h_q, wl.h_kv, n_cu=256)
    cplan.to_device()
    k = torch.empty((cplan.n_tokens, wl.h_kv, wl.head_dim), dtype=q.dtype, device="cuda")
    v = torch.empty_like(k)
    out = torch.empty_like(q)
    ws = P.attn_workspace(cplan, wl.head_dim)
    say("pool gather kblocks=%d, attention items=%d merges=%d"
        % (plan[P.H_N_KBLOCKS], cplan[P.H_N_ATTN_ITEMS], cplan[P.H_N_MERGE]))

    def fn():
        P.pic_rope_splice_pool(plan, pk, pv, cbp, blocks, k, v, kf, vf, wl.rope_base)
        P.pic_selective_attn(cplan, q, k, v, out, workspace=ws)

    replay_and_compare(fn, [out, k, v])
