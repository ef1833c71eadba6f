"""GPU parity of the HIP path against the CPU oracle (MI355X only).

Every case calls the C ABI through the binding on seeded synthetic inputs and
compares with the oracle on the same bits: the index and the splice bit-exactly,
floating outputs to max-abs 1e-5 (fp32 I/O) or 2e-2 (bf16 I/O) on unit-variance
inputs.  Full-size workloads compare every rotated row and sampled attention rows.
"""

import sys

import numpy as np
import pytest
import torch

import position_independent_kv_rope_amd as P
from position_independent_kv_rope_amd import workloads as W
from oracle import pic_oracle as O

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
LAYOUTS = {"adjacent": P.PIC_ROPE_ADJACENT, "half": P.PIC_ROPE_HALF}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


class Run:
    """One pass of the path on the GPU, keeping every intermediate on the host."""

    def __init__(self, wl, layout="adjacent", n_cu=0, pos_base=0, scheme="delta", fused=False):
        # scheme "delta": cached K carries RoPE at local positions (rotation by delta);
        # scheme "nope": cached K is position-free and gets RoPE at the target positions
        self.wl = wl
        reqs = [r.chunk_lens for r in wl.requests]
        qs = [r.q_len for r in wl.requests]
        self.plan = P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, pos_base=pos_base,
                                      n_cu=n_cu)
        self.plan.to_device()
        self.k_in, self.v_in = W.context_tensors(wl)
        self.q, self.kf, self.vf = W.fresh_tensors(wl, self.plan.n_rows)
        dev = "cuda"
        k = self.k_in.to(dev)
        v = self.v_in.to(dev)
        q, kf, vf = self.q.to(dev), self.kf.to(dev), self.vf.to(dev)
        out = torch.full_like(q, float("nan"))
        ws = P.attn_workspace(self.plan, wl.head_dim)
        self.scheme = scheme
        if fused:
            # rotation and splice as one launch; the rotated-only K is the result with
            # the recomputed rows put back to their inputs (the rotation skips them)
            say(wl.name, "k=%d" % wl.k, layout, "rope_splice (one launch)", "rope_" + scheme)
            mode = P.PIC_ROPE_AT_POSITION if scheme == "nope" else P.PIC_ROPE_BY_DELTA
            P.pic_rope_splice(self.plan, k, v, kf, vf, wl.rope_base, LAYOUTS[layout], mode)
            torch.cuda.synchronize()
            self.k_spl, self.v_spl = k.cpu(), v.cpu()
            self.k_rot = self.k_spl.clone()
            rt = torch.as_tensor(np.asarray(self.plan.row_tok, dtype=np.int64))
            self.k_rot[rt] = self.k_in[rt]
        else:
            say(wl.name, "k=%d" % wl.k, layout, "rope_" + scheme)
            if scheme == "nope":
                P.pic_rope_apply(self.plan, k, wl.rope_base, LAYOUTS[layout])
            else:
                P.pic_rope_delta(self.plan, k, wl.rope_base, LAYOUTS[layout])
            torch.cuda.synchronize()
            self.k_rot = k.cpu()
            say(wl.name, "splice")
            P.pic_splice(self.plan, k, v, kf, vf)
            torch.cuda.synchronize()
            self.k_spl, self.v_spl = k.cpu(), v.cpu()
        say(wl.name, "selective_attn items=%d merges=%d" % (self.plan[P.H_N_ATTN_ITEMS],
                                                          self.plan[P.H_N_MERGE]))
        P.pic_selective_attn(self.plan, q, k, v, out, workspace=ws)
        torch.cuda.synchronize()
        self.out = out.cpu()
        self.layout = layout
        self.pos_base = pos_base
        self.dev = dict(q=q, k=k, v=v, out=out, ws=ws)

    def request_slices(self, b):
        r = self.wl.requests[b]
        tok0 = int(self.plan.req_tok_ptr[b])
        row0, row1 = int(self.plan.req_row_ptr[b]), int(self.plan.req_row_ptr[b + 1])
        return r, tok0, row0, row1

    def oracle_request(self, b):
        """Oracle K after rotation, spliced K/V, and attention output of request b."""
        r, tok0, row0, row1 = self.request_slices(b)
        offs = O.chunk_offsets(r.chunk_lens)
        kin = f64(self.k_in[tok0:tok0 + offs[-1]])
        vin = f64(self.v_in[tok0:tok0 + offs[-1]])
        chunks_k = [kin[offs[c]:offs[c + 1]] for c in range(len(r.chunk_lens))]
        chunks_v = [vin[offs[c]:offs[c + 1]] for c in range(len(r.chunk_lens))]
        rows = O.recompute_positions(r.chunk_lens, r.q_len, self.wl.k)
        if chunks_k and self.scheme == "nope":
            k_ctx = O.rope_apply(chunks_k, self.wl.rope_base, self.layout)
            v_ctx = O.concat_chunks(chunks_v)
        elif chunks_k:
            k_ctx = O.rope_delta(chunks_k, self.wl.rope_base, self.layout, self.pos_base)
            v_ctx = O.concat_chunks(chunks_v)
        else:
            k_ctx = np.zeros((0, self.wl.h_kv, self.wl.head_dim))
            v_ctx = k_ctx
        n_total = offs[-1] + r.q_len
        kx, vx = O.splice(k_ctx, v_ctx, f64(self.kf[row0:row1]), f64(self.vf[row0:row1]), rows,
                          n_total)
        return rows, k_ctx, kx, vx


def check_run(run, sample_rows=None):
    wl, plan = run.wl, run.plan
    tol = TOL[wl.dtype]
    # index: bit-exact
    flat = []
    for r in wl.requests:
        flat += O.recompute_positions(r.chunk_lens, r.q_len, wl.k)
    assert plan.rows.tolist() == flat
    worst = {"rope": 0.0, "attn": 0.0}
    for b in range(len(wl.requests)):
        r, tok0, row0, row1 = run.request_slices(b)
        rows, k_ctx, kx, vx = run.oracle_request(b)
        ctx = sum(r.chunk_lens)
        rec = set(rows)
        keep = np.array([j for j in range(ctx) if j not in rec], dtype=np.int64)
        # rotated K on the kept rows against the oracle; untouched rows bit-identical
        got = f64(run.k_rot[tok0:tok0 + ctx])
        if keep.size:
            err = float(np.max(np.abs(got[keep] - k_ctx[keep])))
            worst["rope"] = max(worst["rope"], err)
            assert err <= tol, ("rope_delta", b, err)
        n_total = ctx + r.q_len
        # rows the rotation must not touch: recomputed rows (the splice overwrites them)
        # and, with pos_base = 0, all of chunk 0 (delta_0 = 0)
        rec_t = torch.tensor(rows, dtype=torch.long) + tok0
        assert torch.equal(run.k_rot[rec_t], run.k_in[rec_t])
        if run.pos_base == 0 and r.chunk_lens and run.scheme == "delta":
            L0 = r.chunk_lens[0]
            assert torch.equal(run.k_rot[tok0:tok0 + L0], run.k_in[tok0:tok0 + L0])
        # splice: fresh rows bit-exact, V elsewhere unchanged, K elsewhere = rotated
        rows_t = torch.tensor(rows, dtype=torch.long) + tok0
        assert torch.equal(run.k_spl[rows_t], run.kf[row0:row1])
        assert torch.equal(run.v_spl[rows_t], run.vf[row0:row1])
        others = torch.tensor([tok0 + j for j in range(n_total) if j not in rec], dtype=torch.long)
        if others.numel():
            assert torch.equal(run.v_spl[others], run.v_in[others])
            assert torch.equal(run.k_spl[others], run.k_rot[others])
        # attention
        qb = f64(run.q[row0:row1])
        if sample_rows is None:
            want = O.selective_attn(qb, kx, vx, rows)
            got_o = f64(run.out[row0:row1])
        else:
            rng = np.random.default_rng(1234 + b)
            n = row1 - row0
            picks = sorted(set(rng.integers(0, n, size=min(sample_rows, n)).tolist()) |
                           {0, n - 1})
            heads = rng.integers(0, wl.h_q, size=len(picks))
            g = heads // (wl.h_q // wl.h_kv)
            want = O.attn_rows_direct([qb[i, h] for i, h in zip(picks, heads)], kx, vx,
                                      [rows[i] for i in picks], g)
            got_o = np.stack([f64(run.out[row0 + i, h]) for i, h in zip(picks, heads)])
        assert np.isfinite(got_o).all()
        err = float(np.max(np.abs(got_o - want))) if want.size else 0.0
        worst["attn"] = max(worst["attn"], err)
        assert err <= tol, ("selective_attn", b, err)
    say(wl.name, "k=%d" % wl.k, "max-abs errors", worst)
    return worst


@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_worked_example_fp32(layout):
    run = Run(W.worked_example(), layout)
    assert run.plan.rows.tolist() == [4, 5, 9, 10, 14, 15, 16]
    check_run(run)


def test_rag_single_bf16():
    check_run(Run(W.rag_single()))


@pytest.mark.parametrize("k", [2, 16])
def test_long_context_bf16(k):
    run = Run(W.long_context(k=k))
    assert run.plan[P.H_N_MERGE] > 0
    check_run(run)


def test_epic_sweep_full_size_sampled():
    # the launch configuration bench.py times (n_cu = 256), sampled attention rows
    run = Run(W.epic_sweep(k=16), n_cu=256)
    check_run(run, sample_rows=48)


def _custom(name, dtype, h_q, h_kv, d, base, k, reqs, seed=11, scale=1.0):
    return W.Workload(name, dtype, h_q, h_kv, d, base, k,
                      [W.Request(list(c), q) for c, q in reqs], value_scale=scale, seed=seed)


EDGE_CASES = [
    # ragged tails, zero-length chunks, q = 0 requests, k = 0, k >= chunk length
    ("ragged_bf16", "bf16", 32, 8, 128, 5e5, 3, [([37, 0, 101, 5], 9), ([64], 0), ([3, 3], 70)]),
    ("k0_bf16", "bf16", 32, 8, 128, 5e5, 0, [([300, 200], 17)]),
    ("k_ge_len_bf16", "bf16", 32, 8, 128, 5e5, 40, [([20, 33, 7], 5)]),
    ("gqa8_bf16", "bf16", 32, 4, 128, 5e5, 8, [([700, 650, 900], 128), ([513], 3)]),
    ("mha_bf16_d64", "bf16", 8, 8, 64, 1e4, 4, [([130, 77], 12)]),
    ("gqa2_bf16_d64", "bf16", 16, 8, 64, 1e6, 2, [([250, 250, 250], 40)]),
    ("f32_d32", "f32", 8, 2, 32, 1e4, 2, [([40, 41, 42], 11), ([5], 2)]),
    ("f32_d64", "f32", 16, 4, 64, 5e5, 5, [([300, 129], 33)]),
    ("f32_d128", "f32", 32, 8, 128, 5e5, 16, [([200, 180], 20)]),
    ("only_query_rows", "f32", 4, 4, 16, 1e4, 2, [([], 6), ([0], 3)]),
    # wide GQA groups: a wave owns 32/G rows with all G heads (G = 16, 32), or, past 32
    # heads per KV head, 32 consecutive head-major columns of the tile (G = 64, 128)
    ("gqa16_bf16", "bf16", 32, 2, 128, 5e5, 3, [([300, 257, 90], 21), ([130], 4)]),
    ("gqa32_bf16_d64", "bf16", 32, 1, 64, 1e4, 5, [([200, 333], 17)]),
    ("gqa64_bf16_d64", "bf16", 64, 1, 64, 1e4, 2, [([150, 180, 70], 9)]),
    ("gqa128_bf16_d64", "bf16", 128, 1, 64, 1e4, 2, [([90, 140], 5)]),
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_edge_cases(case):
    name, dtype, hq, hkv, d, base, k, reqs = case
    check_run(Run(_custom(name, dtype, hq, hkv, d, base, k, reqs)))


@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_half_layout_and_pos_base(layout):
    # LegoLink-0 style cached positions (first cached row at position 4): every chunk,
    # chunk 0 included, is rotated by off_c - 4 (negative for chunk 0)
    wl = _custom("pos_base", "bf16", 32, 8, 128, 5e5, 0, [([100, 90, 80], 20)])
    check_run(Run(wl, layout, pos_base=4))


def test_consistency_invariant_gpu():
    # cached K = RoPE(K0, local), fresh K/Q = RoPE(., global) (made by the oracle on the
    # CPU, rounded to fp32): the GPU link must reproduce full causal attention.
    rng = np.random.default_rng(21)
    lens, q_len, hq, hkv, d, base, k = [9, 14, 11, 6], 5, 8, 2, 32, 1e4, 2
    offs = O.chunk_offsets(lens)
    n = offs[-1] + q_len
    q0, k0, v = (rng.standard_normal((n, h, d)) for h in (hq, hkv, hkv))
    pos = np.arange(n)
    kg, qg = O.rope_rotate(k0, pos, base), O.rope_rotate(q0, pos, base)
    cached = np.concatenate([O.rope_rotate(k0[offs[c]:offs[c + 1]], np.arange(lens[c]), base)
                             for c in range(len(lens))] + [np.zeros((q_len, hkv, d))])
    plan = P.pic_build_index([lens], [q_len], k, hq, hkv)
    plan.to_device()
    rows = plan.rows.tolist()
    t = lambda a: torch.tensor(a, dtype=torch.float32, device="cuda").contiguous()
    kb, vb = t(cached), t(np.concatenate([v[:offs[-1]], np.zeros((q_len, hkv, d))]))
    q, kf, vf = t(qg[rows]), t(kg[rows]), t(v[rows])
    out = torch.empty_like(q)
    say("consistency_invariant")
    P.pic_rope_delta(plan, kb, base)
    P.pic_splice(plan, kb, vb, kf, vf)
    P.pic_selective_attn(plan, q, kb, vb, out, workspace=P.attn_workspace(plan, d))
    torch.cuda.synchronize()
    want = O.full_causal_attn(qg.astype(np.float32), kg.astype(np.float32),
                              v.astype(np.float32))[rows]
    assert np.max(np.abs(f64(kb) - kg)) < 1e-5
    assert np.max(np.abs(f64(out) - want)) < 1e-5


def test_attention_is_deterministic():
    run = Run(W.long_context(k=2))
    d = run.dev
    again = torch.full_like(d["out"], float("nan"))
    P.pic_selective_attn(run.plan, d["q"], d["k"], d["v"], again, workspace=d["ws"])
    torch.cuda.synchronize()
    assert torch.equal(again.cpu(), run.out)


# ---------------------------------------------------------------------------
# Scheme B: position-free cache, RoPE applied at the target positions
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_scheme_b_worked_example_fp32(layout):
    check_run(Run(W.worked_example(), layout, scheme="nope"))


def test_scheme_b_rag_single_bf16():
    check_run(Run(W.rag_single(), scheme="nope"))


def test_scheme_b_long_context_bf16_half():
    check_run(Run(W.long_context(k=2), "half", scheme="nope"), sample_rows=32)


def test_scheme_b_epic_sweep_full_size_sampled():
    # every kept row of the 4 x ~50k batch rotated at its global position (chunk 0
    # included), sampled attention rows, launched as bench.py launches it (n_cu = 256)
    check_run(Run(W.epic_sweep(k=16), n_cu=256, scheme="nope"), sample_rows=24)


# K/V of one request are addressed with 32-bit byte offsets: pic_selective_attn takes
# requests up to 0x7fff0000 bytes of K (N * h_kv * D * 2), and refuses larger ones
MAX_REQUEST_BYTES = 0x7FFF0000


def test_max_request_size_sampled():
    # the largest request the contiguous path takes: 1,048,544 tokens of 8 KV heads of
    # 128 (2 GiB of K and of V), 16 chunks, k = 2, in the launch configuration bench.py
    # times.  Rotated rows at the top of the buffer, every spliced row, and sampled
    # attention rows (the last query row among them) against the oracle.
    n_max = MAX_REQUEST_BYTES // (8 * 128 * 2)
    wl = W.single_huge(n_max)
    r = wl.requests[0]
    plan = P.pic_build_index([r.chunk_lens], [r.q_len], wl.k, wl.h_q, wl.h_kv, n_cu=256)
    plan.to_device()
    assert plan.n_tokens == n_max
    dev = "cuda"
    say("max request: drawing K/V on the device", plan.n_tokens, "tokens")
    k, v = W.device_context_tensors(wl, dev)
    q_h, kf_h, vf_h = W.fresh_tensors(wl, plan.n_rows)
    groups = [0, wl.h_kv - 1]  # KV heads checked against the oracle
    k_in = {g: k[:, g, :].cpu() for g in groups}
    v_in = {g: v[:, g, :].cpu() for g in groups}
    q, kf, vf = q_h.to(dev), kf_h.to(dev), vf_h.to(dev)
    out = torch.full_like(q, float("nan"))
    say("max request: rope_delta, splice, selective_attn (items=%d merges=%d)"
        % (plan[P.H_N_ATTN_ITEMS], plan[P.H_N_MERGE]))
    P.pic_rope_delta(plan, k, wl.rope_base)
    torch.cuda.synchronize()
    rows = O.recompute_positions(r.chunk_lens, r.q_len, wl.k)
    assert plan.rows.tolist() == rows
    offs = O.chunk_offsets(r.chunk_lens)
    ctx = offs[-1]
    # rotated K: the last 64 kept rows of the buffer and 64 random kept rows, all heads
    rec = set(rows)
    kept_tail = [j for j in range(ctx - 1, -1, -1) if j not in rec][:64]
    rng = np.random.default_rng(77)
    picks = sorted(set(kept_tail) | {int(j) for j in rng.integers(0, ctx, 64) if int(j) not in rec})
    pick_t = torch.tensor(picks, dtype=torch.long, device=dev)
    got_rot = f64(k.index_select(0, pick_t))
    say("max request: oracle rotation of", len(picks), "sampled rows")
    chunk_of = np.searchsorted(np.asarray(offs[1:]), np.asarray(picks), side="right")
    k_pre = {g: f64(k_in[g][picks]) for g in groups}
    for g in groups:
        want = O.rope_rotate(k_pre[g][:, None, :], np.asarray(offs)[chunk_of], wl.rope_base)[:, 0]
        err = float(np.max(np.abs(got_rot[:, g] - want)))
        say("rope_delta head", g, "max-abs error", err)
        assert err <= TOL["bf16"]
    P.pic_splice(plan, k, v, kf, vf)
    ws = P.attn_workspace(plan, wl.head_dim)
    P.pic_selective_attn(plan, q, k, v, out, workspace=ws)
    torch.cuda.synchronize()
    rows_t = torch.tensor(rows, dtype=torch.long, device=dev)
    assert torch.equal(k.index_select(0, rows_t).cpu(), kf_h)
    assert torch.equal(v.index_select(0, rows_t).cpu(), vf_h)
    out_h = out.cpu()
    assert torch.isfinite(out_h.float()).all()
    # attention: sampled (row, head) pairs in the checked KV heads, against the oracle
    # chained from the same inputs (rotation per chunk, splice of the fresh rows)
    n = len(rows)
    G = wl.h_q // wl.h_kv
    sample = sorted({0, n - 1, n - 2, n - 64, 1, 15, 29} | set(rng.integers(0, n, 5).tolist()))
    for g in groups:
        say("max request: oracle K/V of KV head", g)
        kin = f64(k_in[g])[:, None, :]
        vin = f64(v_in[g])[:, None, :]
        k_ctx = O.rope_delta([kin[offs[c]:offs[c + 1]] for c in range(len(r.chunk_lens))],
                             wl.rope_base)
        kx, vx = O.splice(k_ctx, vin[:ctx], f64(kf_h[:, g:g + 1]), f64(vf_h[:, g:g + 1]), rows,
                          plan.n_tokens)
        heads = [g * G + (i % G) for i in sample]
        want = O.attn_rows_direct([f64(q_h[i, h]) for i, h in zip(sample, heads)], kx, vx,
                                  [rows[i] for i in sample], [0] * len(sample))
        got = np.stack([f64(out_h[i, h]) for i, h in zip(sample, heads)])
        err = float(np.max(np.abs(got - want)))
        say("selective_attn head group", g, "max-abs error", err)
        assert err <= TOL["bf16"]


def _random_case(i):
    """Seeded random configuration: heads, GQA group, head_dim, dtype, layout, pos_base,
    k and ragged requests (empty chunks, chunk-free and query-free requests)."""
    rng = np.random.default_rng(4000 + i)
    dtype = "bf16" if i % 3 else "f32"
    d = int(rng.choice([64, 128] if dtype == "bf16" else [16, 32, 64, 128]))
    h_kv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    reqs = []
    for _ in range(int(rng.integers(1, 4))):
        n = int(rng.integers(0, 6))
        lens = [int(x) for x in rng.integers(0, 2500 if i % 2 else 500, size=n)]
        if n and rng.random() < 0.3:
            lens[int(rng.integers(0, n))] = 0
        reqs.append((lens, int(rng.integers(0, 60))))
    if sum(sum(l) + q for l, q in reqs) == 0:
        reqs[0] = ([37], 5)
    k = int(rng.integers(0, 20))
    base = float(rng.choice([1e4, 5e5, 1e6]))
    layout = "half" if rng.random() < 0.5 else "adjacent"
    pos_base = int(rng.integers(0, 8)) if rng.random() < 0.3 else 0
    wl = _custom("random%d" % i, dtype, g * h_kv, h_kv, d, base, k, reqs, seed=500 + i)
    return wl, layout, pos_base


@pytest.mark.parametrize("i", range(16))
def test_random_configurations(i):
    # every stage of the contiguous path on a seeded random configuration, against the
    # oracle (full compare), with the plan split for a few-CU launch as often as not
    wl, layout, pos_base = _random_case(i)
    say("random case", i, wl.dtype, "h_q=%d h_kv=%d D=%d k=%d" % (wl.h_q, wl.h_kv, wl.head_dim, wl.k),
        layout, "pos_base=%d" % pos_base, [(sum(r.chunk_lens), len(r.chunk_lens), r.q_len) for r in wl.requests])
    check_run(Run(wl, layout, n_cu=(2 if i % 2 else 0), pos_base=pos_base))


ONE_LAUNCH_CASES = [
    # (workload, layout, scheme, pos_base, n_cu)
    ("worked_example", "adjacent", "delta", 0, 0),
    ("worked_example", "half", "nope", 0, 0),
    ("ragged_bf16", "adjacent", "delta", 0, 2),
    ("f32_d64", "half", "delta", 4, 0),
    ("gqa8_bf16", "adjacent", "nope", 0, 0),
    ("only_query_rows", "adjacent", "delta", 0, 0),
    ("long_context_k16", "adjacent", "delta", 0, 256),
]


def _one_launch_workload(name):
    if name == "worked_example":
        return W.worked_example()
    if name == "long_context_k16":
        return W.long_context(k=16)
    case = [c for c in EDGE_CASES if c[0] == name][0]
    return _custom(*case)


@pytest.mark.parametrize("case", ONE_LAUNCH_CASES, ids=["-".join(map(str, c)) for c in ONE_LAUNCH_CASES])
def test_rope_splice_one_launch(case):
    # pic_rope_splice: the oracle checks of every stage, and its spliced K/V bit-equal to
    # the two calls it replaces on the same inputs
    name, layout, scheme, pos_base, n_cu = case
    wl = _one_launch_workload(name)
    fused = Run(wl, layout, n_cu=n_cu, pos_base=pos_base, scheme=scheme, fused=True)
    check_run(fused)
    apart = Run(wl, layout, n_cu=n_cu, pos_base=pos_base, scheme=scheme)
    assert torch.equal(fused.k_spl, apart.k_spl)
    assert torch.equal(fused.v_spl, apart.v_spl)
    assert torch.equal(fused.out, apart.out)


def test_rope_splice_epic_sweep_full_size_sampled():
    # the call bench.py times, at its size and launch configuration
    run = Run(W.epic_sweep(k=16), n_cu=256, fused=True)
    check_run(run, sample_rows=48)


@pytest.mark.parametrize("i", [16, 17, 18, 19, 20, 21])
def test_random_configurations_one_launch(i):
    # seeded random configurations through pic_rope_splice (rotation by delta or RoPE at
    # the target positions, then the splice, in one launch), every stage against the oracle
    wl, layout, pos_base = _random_case(i)
    scheme = "nope" if (i % 2 and pos_base == 0) else "delta"
    say("random case (one launch)", i, wl.dtype, "h_q=%d h_kv=%d D=%d k=%d" % (wl.h_q, wl.h_kv, wl.head_dim, wl.k),
        layout, scheme, "pos_base=%d" % pos_base)
    check_run(Run(wl, layout, n_cu=(2 if i % 3 else 0), pos_base=pos_base, scheme=scheme, fused=True))


# ---------------------------------------------------------------------------
# The fp32 angle at the offsets of long contexts (delta ~ 1e5 .. 5e5)
# ---------------------------------------------------------------------------
#
# The rotation's angle is delta * theta_i.  A plain fp32 product errs by ~1e-3 rad at
# delta ~ 1e5, far below what the bf16 bound of 2e-2 can see, so these cases check the
# rotation where the error would show: fp32 I/O at 1e-5, and bf16 output within one
# unit in the last place of the oracle's value rounded to bf16.  One KV head keeps the
# half-million-token request small (256 MB of fp32 K).

LONG_OFFSETS = [([100000, 700, 400000, 300], 16)]  # chunks at 0, 1e5, 100,700, 500,700


@pytest.mark.parametrize("scheme", ["delta", "nope"])
@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_fp32_rotation_at_long_offsets(layout, scheme):
    wl = _custom("long_offsets_f32", "f32", 4, 1, 128, 5e5, 2, LONG_OFFSETS, seed=41)
    worst = check_run(Run(wl, layout, n_cu=256, scheme=scheme), sample_rows=16)
    say("fp32 long offsets", layout, scheme, "rope max-abs", worst["rope"])


@pytest.mark.parametrize("scheme", ["delta", "nope"])
def test_fp32_rotation_one_launch_at_long_offsets(scheme):
    wl = _custom("long_offsets_f32", "f32", 4, 1, 128, 5e5, 2, LONG_OFFSETS, seed=43)
    check_run(Run(wl, "adjacent", n_cu=256, scheme=scheme, fused=True), sample_rows=8)


@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_fp32_rotation_at_delta_near_two_to_the_20(layout):
    # cached rows at local positions from -(2^20 - 3): every chunk rotates by
    # off_c + 2^20 - 3 (about 1.05e6)
    wl = _custom("pos_base_2e20_f32", "f32", 8, 2, 128, 5e5, 3, [([300, 257, 410], 33)], seed=45)
    check_run(Run(wl, layout, pos_base=-(1 << 20) + 3))


def _bf16_ulp(y):
    """Spacing of bf16 numbers at |y| (y already representable in bf16)."""
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(np.maximum(e, -126.0) - 7.0), np.exp2(-133.0))


@pytest.mark.parametrize("scheme", ["delta", "nope"])
def test_bf16_rotation_within_one_ulp_at_long_offsets(scheme):
    # The GPU rotates in fp32 and rounds once to bf16.  With an angle good to ~1e-6 rad
    # its fp32 value lies within E = 4e-6 * |pair| of the exact one, so each rotated
    # element is the oracle's value rounded to bf16 or one unit in the last place away,
    # up to E where the result nearly cancels; and a flip to the neighbouring bf16 value
    # happens only when the exact value lies within E of a rounding midpoint: for
    # ~1e-4 of the elements.  A plain fp32 product delta * theta flips ~13% of them at
    # these offsets, an angle error of 1e-3 rad ~30%.
    wl = _custom("long_offsets_bf16", "bf16", 4, 1, 128, 5e5, 2, LONG_OFFSETS, seed=47)
    run = Run(wl, "adjacent", n_cu=256, scheme=scheme)
    r, tok0, _, _ = run.request_slices(0)
    rows, k_ctx, _, _ = run.oracle_request(0)
    ctx = sum(r.chunk_lens)
    rec = set(rows)
    keep = np.array([j for j in range(ctx) if j not in rec], dtype=np.int64)
    exact = k_ctx[keep]
    want = torch.from_numpy(exact).to(torch.bfloat16).to(torch.float64).numpy()
    got = f64(run.k_rot[tok0:tok0 + ctx])[keep]
    pair = np.sqrt(exact[..., 0::2] ** 2 + exact[..., 1::2] ** 2).repeat(2, axis=-1)
    diff = np.abs(got - want)
    flipped = float(np.mean(diff > 0))
    say("bf16 long offsets", scheme, "max ulps", float(np.max(diff / _bf16_ulp(want))),
        "elements off the rounded oracle value: %.4f%%" % (100.0 * flipped))
    assert np.all(diff <= _bf16_ulp(want) + 4e-6 * pair)
    assert flipped <= 1e-3
