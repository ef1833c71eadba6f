"""pic_selective_attn_noalloc (split-KV partials in the library's per-GPU scratch array)
against pic_selective_attn (caller workspace) through the C ABI: two calls in a row, the
second with a smaller input, each bit-identical to the workspace entry point on the same
inputs and within the bf16 bound of the oracle; plans beyond the scratch size are
refused before anything runs."""

import sys

import numpy as np
import pytest
import torch

import position_independent_kv_rope_amd as P
from position_independent_kv_rope_amd import workloads as W
from oracle import pic_oracle as O

TOL = 2e-2  # bf16 I/O


def say(*a):
    print("[no-alloc]", *a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def _spliced(wl):
    """Plan, rotated + spliced K/V on the device, Q, and the host inputs."""
    reqs = [r.chunk_lens for r in wl.requests]
    qs = [r.q_len for r in wl.requests]
    plan = P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, n_cu=256)
    plan.to_device()
    k_in, v_in = W.context_tensors(wl)
    q_h, kf_h, vf_h = W.fresh_tensors(wl, plan.n_rows)
    k, v = k_in.cuda(), v_in.cuda()
    P.pic_rope_splice(plan, k, v, kf_h.cuda(), vf_h.cuda(), wl.rope_base)
    return plan, k, v, q_h.cuda(), (k_in, v_in, q_h, kf_h, vf_h)


def _check_against_oracle(wl, plan, out, host, n_sample=24):
    k_in, v_in, q_h, kf_h, vf_h = host
    rng = np.random.default_rng(5)
    worst = 0.0
    for b, r in enumerate(wl.requests):
        tok0 = int(plan.req_tok_ptr[b])
        row0, row1 = int(plan.req_row_ptr[b]), int(plan.req_row_ptr[b + 1])
        offs = O.chunk_offsets(r.chunk_lens)
        ck = [f64(k_in[tok0 + offs[c]:tok0 + offs[c + 1]]) for c in range(len(r.chunk_lens))]
        cv = [f64(v_in[tok0 + offs[c]:tok0 + offs[c + 1]]) for c in range(len(r.chunk_lens))]
        rows = O.recompute_positions(r.chunk_lens, r.q_len, wl.k)
        kx, vx = O.splice(O.rope_delta(ck, wl.rope_base), O.concat_chunks(cv),
                          f64(kf_h[row0:row1]), f64(vf_h[row0:row1]), rows, offs[-1] + r.q_len)
        n = row1 - row0
        picks = sorted(set(rng.integers(0, n, size=min(n_sample, n)).tolist()) | {0, n - 1})
        heads = rng.integers(0, wl.h_q, size=len(picks))
        qb = f64(q_h[row0:row1])
        want = O.attn_rows_direct([qb[i, h] for i, h in zip(picks, heads)], kx, vx,
                                  [rows[i] for i in picks], heads // (wl.h_q // wl.h_kv))
        got = np.stack([f64(out[row0 + i, h]) for i, h in zip(picks, heads)])
        worst = max(worst, float(np.max(np.abs(got - want))))
    assert worst <= TOL, worst
    return worst


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # first call: the 32,896-token request at k = 16 (1,592 split slots, 101 MiB of
    # partials); second call: the 5,184-token request (160 slots), a smaller input
    for wl in (W.long_context(k=16), W.rag_single()):
        plan, k, v, q, host = _spliced(wl)
        need = P.pic_attn_workspace_bytes(plan, wl.head_dim)
        assert 0 < need <= P.PIC_ATTN_SCRATCH_BYTES
        ref = torch.full_like(q, float("nan"))
        P.pic_selective_attn(plan, q, k, v, ref, workspace=P.attn_workspace(plan, wl.head_dim))
        got = torch.full_like(q, float("nan"))
        say(wl.name, "tokens", plan.n_tokens, "partials bytes", need)
        P.pic_selective_attn_noalloc(plan, q, k, v, got)
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), ref.cpu())
        err = _check_against_oracle(wl, plan, got.cpu(), host)
        say(wl.name, "bit-identical to the workspace call; sampled max-abs vs oracle", err)


def test_noalloc_refuses_plans_beyond_the_scratch():
    # the 4 x ~50k batch at k = 16 needs ~287 MiB of partials: PIC_ENOSPC, checked
    # before any device call (so this runs without a GPU)
    import ctypes
    wl = W.epic_sweep(k=16)
    plan = P.pic_build_index([r.chunk_lens for r in wl.requests], [r.q_len for r in wl.requests],
                             wl.k, wl.h_q, wl.h_kv, n_cu=256)
    assert P.pic_attn_workspace_bytes(plan, 128) > P.PIC_ATTN_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)
    st = P.lib().pic_selective_attn_noalloc(plan.host_ptr(), fake, fake, fake, fake, fake,
                                            P.PIC_BF16, 128, 0.0, None)
    assert st == P.PIC_ENOSPC
