"""GPU parity of the linear-layer state composition (pic_state_compose) against the CPU
oracle (MI355X only): every state after every chunk and every final state, fp32 I/O,
max-abs 1e-5 on states of magnitude O(1).
"""

import sys

import numpy as np
import pytest
import torch

import position_independent_kv_rope_amd as P
from position_independent_kv_rope_amd import workloads as W
from oracle import pic_oracle as O

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()


def say(*a):
    print("[gpu-state]", *a, flush=True)
    sys.stdout.flush()


def run_state(wl, n_heads, with_init=False, with_prefix=True, requests=None):
    reqs = [r.chunk_lens for r in wl.requests]
    ids = [r.chunk_ids for r in wl.requests]
    qs = [r.q_len for r in wl.requests]
    plan = P.pic_build_index(reqs, qs, wl.k, 8, 8, chunk_ids_per_req=ids)
    plan.to_device()
    t_pool, s_pool = W.state_pool_tensors(wl, n_heads)
    n_req, d = len(reqs), 128
    dev = "cuda"
    s_init = W.draw((n_req, n_heads, d, d), 91, torch.float32, 0.5) if with_init else None
    final = torch.full((n_req, n_heads, d, d), float("nan"), device=dev)
    prefix = (torch.full((plan[P.H_N_CHUNKS], n_heads, d, d), float("nan"), device=dev)
              if with_prefix else None)
    say(wl.name, "heads=%d chunks=%d init=%s" % (n_heads, plan[P.H_N_CHUNKS], with_init))
    P.pic_state_compose(plan, t_pool.to(dev), s_pool.to(dev), final, prefix_out=prefix,
                        s_init=None if s_init is None else s_init.to(dev))
    torch.cuda.synchronize()
    fin = final.cpu().double().numpy()
    pre = None if prefix is None else prefix.cpu().double().numpy()
    tp, sp = t_pool.double().numpy(), s_pool.double().numpy()
    rcp = [0] + list(np.cumsum([len(r.chunk_ids) for r in wl.requests]))
    worst = 0.0
    for b, r in enumerate(wl.requests):
        if requests is not None and b not in requests:
            continue
        for h in range(n_heads):
            s0 = None if s_init is None else s_init[b, h].double().numpy()
            states = O.compose_states([tp[i, h] for i in r.chunk_ids], [sp[i, h] for i in r.chunk_ids], s0)
            want_final = states[-1] if len(states) else (np.zeros((d, d)) if s0 is None else s0)
            err = float(np.max(np.abs(fin[b, h] - want_final)))
            if pre is not None and len(states):
                err = max(err, float(np.max(np.abs(pre[rcp[b]:rcp[b + 1], h] - states))))
            worst = max(worst, err)
            assert err <= TOL, ("request", b, "head", h, err)
    say(wl.name, "max-abs error", worst)


def small_pool_wl(seed=71):
    lens = [40, 17, 90, 33, 1, 64, 20]
    reqs = [W.Request([lens[i] for i in ids], 5, chunk_ids=ids)
            for ids in ([0, 1, 2, 3], [2, 2, 5], [6], [], [4, 0, 6, 1, 3, 5, 2])]
    return W.Workload("state_small", "f32", 8, 8, 128, 1e4, 2, reqs, pool_lens=lens, seed=seed)


def test_state_compose_small():
    run_state(small_pool_wl(), 3)


def test_state_compose_initial_state_and_no_prefix():
    run_state(small_pool_wl(73), 2, with_init=True)
    run_state(small_pool_wl(75), 2, with_prefix=False)


def test_state_compose_shared_pool():
    # the shared-pool batch (8 requests x 96-128 chunks from 256 pooled chunks), 4 heads
    run_state(W.shared_pool(), 4)
