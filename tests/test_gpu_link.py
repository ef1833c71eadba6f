"""GPU parity of the multi-layer link (pic_qkv_rope, pic_out_proj, pic_link) against the
CPU oracle (MI355X only).

Each entry point is compared with the oracle on the same bf16 inputs to max-abs 2e-2
(bf16 I/O, unit-variance activations).  The whole link of several layers is compared
two ways: layer by layer (each GPU layer against the oracle layer fed the GPU's own
bf16 input), and end to end against the oracle chained in fp64, where every layer adds
its own bf16 roundings (x, Q/K/V, the rotated K and the attention output each rounded
once): 2e-2 per layer.  The residual stream grows layer by layer (x + O W_o^T), and a
bf16 rounding error is relative to the value, so both link bounds scale with the
reference's magnitude beyond the unit-variance range: 2e-2 * max(1, max|x| / 4).
"""

import sys

import numpy as np
import pytest
import torch

import position_independent_kv_rope_amd as P
from position_independent_kv_rope_amd import workloads as W
from oracle import pic_oracle as O

pytestmark = pytest.mark.gpu

TOL = 2e-2
LAYOUTS = {"adjacent": P.PIC_ROPE_ADJACENT, "half": P.PIC_ROPE_HALF}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()


def say(*a):
    print("[gpu-link]", *a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def small(h_q=4, h_kv=2, d=128, seed=61, reqs=None):
    reqs = reqs or [W.Request([40, 50, 33], 7), W.Request([20], 5), W.Request([], 3)]
    return W.Workload("link_small", "bf16", h_q, h_kv, d, 10000.0, 2, reqs, seed=seed)


def plan_of(wl, n_cu=0):
    plan = P.pic_build_index([r.chunk_lens for r in wl.requests], [r.q_len for r in wl.requests],
                             wl.k, wl.h_q, wl.h_kv, n_cu=n_cu)
    plan.to_device()
    return plan


@pytest.mark.parametrize("layout,d,h_q,h_kv", [("adjacent", 128, 4, 2), ("half", 128, 4, 2),
                                               ("adjacent", 64, 8, 2), ("half", 64, 8, 2)])
def test_qkv_rope_small(layout, d, h_q, h_kv):
    wl = small(h_q, h_kv, d)
    plan = plan_of(wl)
    d_model = 256
    x, w, _, _, _ = W.link_tensors(wl, 1, d_model, plan.n_rows)
    w = w[0]
    dev = "cuda"
    q = torch.full((plan.n_rows, h_q, d), float("nan"), dtype=torch.bfloat16, device=dev)
    kf = torch.full((plan.n_rows, h_kv, d), float("nan"), dtype=torch.bfloat16, device=dev)
    vf = torch.full_like(kf, float("nan"))
    say("qkv_rope", layout, "D=%d rows=%d" % (d, plan.n_rows))
    P.pic_qkv_rope(plan, x.to(dev), w.to(dev), q, kf, vf, wl.rope_base, LAYOUTS[layout])
    torch.cuda.synchronize()
    want = O.qkv_rope(f64(x), f64(w), plan.rows.tolist(), h_q, h_kv, wl.rope_base, layout)
    errs = [float(np.max(np.abs(f64(g) - w_))) for g, w_ in zip((q, kf, vf), want)]
    say("qkv_rope max-abs errors q/k/v", errs)
    assert max(errs) <= TOL


def test_out_proj_small():
    wl = small()
    plan = plan_of(wl)
    d_model = 384
    x, _, w_o, _, _ = W.link_tensors(wl, 1, d_model, plan.n_rows)
    o = W.draw((plan.n_rows, wl.h_q, wl.head_dim), 77, torch.bfloat16)
    xd = x.to("cuda")
    say("out_proj rows=%d d_model=%d" % (plan.n_rows, d_model))
    P.pic_out_proj(plan, o.to("cuda"), w_o[0].to("cuda"), xd)
    torch.cuda.synchronize()
    err = float(np.max(np.abs(f64(xd) - O.out_proj_residual(f64(o), f64(w_o[0]), f64(x)))))
    say("out_proj max-abs error", err)
    assert err <= TOL


def test_qkv_rope_full_size_sampled():
    # the bench batch's recomputed rows (4 x ~50k tokens, k = 16: 3,520 rows), a 4096-wide
    # model with 32/8 heads of 128: sampled rows against the oracle
    wl = W.epic_sweep(k=16)
    plan = plan_of(wl, n_cu=256)
    d_model = 4096
    x, w, _, _, _ = W.link_tensors(wl, 1, d_model, plan.n_rows)
    dev = "cuda"
    q = torch.empty((plan.n_rows, wl.h_q, wl.head_dim), dtype=torch.bfloat16, device=dev)
    kf = torch.empty((plan.n_rows, wl.h_kv, wl.head_dim), dtype=torch.bfloat16, device=dev)
    vf = torch.empty_like(kf)
    say("qkv_rope full size rows=%d" % plan.n_rows)
    P.pic_qkv_rope(plan, x.to(dev), w[0].to(dev), q, kf, vf, wl.rope_base)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    pick = np.sort(rng.choice(plan.n_rows, 96, replace=False))
    pick[-1] = plan.n_rows - 1  # the ragged last tile
    rows = plan.rows.tolist()
    want = O.qkv_rope(f64(x[pick]), f64(w[0]), [rows[i] for i in pick], wl.h_q, wl.h_kv,
                      wl.rope_base)
    errs = [float(np.max(np.abs(f64(g[pick]) - w_))) for g, w_ in zip((q, kf, vf), want)]
    say("qkv_rope full size max-abs errors q/k/v", errs)
    assert max(errs) <= TOL


def run_link(wl, n_layers, d_model, layout="adjacent", n_cu=0, requests=None, per_layer=True):
    plan = plan_of(wl, n_cu)
    x0, w_qkv, w_o, kc, vc = W.link_tensors(wl, n_layers, d_model, plan.n_rows)
    dev = "cuda"
    lay = LAYOUTS[layout]
    d, hq, hkv = wl.head_dim, wl.h_q, wl.h_kv
    q = torch.empty((plan.n_rows, hq, d), dtype=torch.bfloat16, device=dev)
    kf = torch.empty((plan.n_rows, hkv, d), dtype=torch.bfloat16, device=dev)
    vf, o = torch.empty_like(kf), torch.empty_like(q)
    wq_d = [w.to(dev) for w in w_qkv]
    wo_d = [w.to(dev) for w in w_o]
    req_rows = [(int(plan.req_row_ptr[b]), int(plan.req_row_ptr[b + 1])) for b in range(len(wl.requests))]
    req_tok = plan.req_tok_ptr.tolist()
    chosen = [b for b in range(len(wl.requests)) if requests is None or b in requests]

    def oracle_layers(x_in, layers, b):
        r = wl.requests[b]
        offs = O.chunk_offsets(r.chunk_lens)
        per = []
        for l in layers:
            t0 = req_tok[b]
            kch = [f64(kc[l][t0 + offs[c]:t0 + offs[c + 1]]) for c in range(len(r.chunk_lens))]
            vch = [f64(vc[l][t0 + offs[c]:t0 + offs[c + 1]]) for c in range(len(r.chunk_lens))]
            per.append({"w_qkv": f64(w_qkv[l]), "w_o": f64(w_o[l]), "k_chunks": kch, "v_chunks": vch})
        return O.link_layers(x_in, per, r.q_len, wl.k, hq, hkv, wl.rope_base, layout)["x"]

    worst = 0.0
    if per_layer:  # layer by layer: the oracle layer gets the GPU's own input
        x = x0.to(dev)
        for l in range(n_layers):
            x_in = f64(x)
            say(wl.name, layout, "layer %d/%d" % (l + 1, n_layers))
            P.pic_link(plan, x, wq_d[l:l + 1], wo_d[l:l + 1], [kc[l].to(dev)], [vc[l].to(dev)],
                       q, kf, vf, o, wl.rope_base, lay)
            torch.cuda.synchronize()
            got = f64(x)
            for b in chosen:
                r0, r1 = req_rows[b]
                want = oracle_layers(x_in[r0:r1], [l], b)
                err = float(np.max(np.abs(got[r0:r1] - want), initial=0.0))
                tol = TOL * max(1.0, float(np.max(np.abs(want), initial=0.0)) / 4)
                worst = max(worst, err)
                say("layer", l, "request", b, "max-abs error", err, "bound", tol)
                assert err <= tol, ("layer", l, "request", b, err)
        say(wl.name, "per-layer max-abs error", worst)
    # all layers in one call against the oracle chained in fp64
    x = x0.to(dev)
    say(wl.name, layout, "%d layers in one call" % n_layers)
    P.pic_link(plan, x, wq_d, wo_d, [t.to(dev) for t in kc], [t.to(dev) for t in vc], q, kf, vf,
               o, wl.rope_base, lay)
    torch.cuda.synchronize()
    got = f64(x)
    assert np.isfinite(got).all()
    e2e = 0.0
    for b in chosen:
        r0, r1 = req_rows[b]
        want = oracle_layers(f64(x0)[r0:r1], range(n_layers), b)
        err = float(np.max(np.abs(got[r0:r1] - want), initial=0.0))
        tol = TOL * n_layers * max(1.0, float(np.max(np.abs(want), initial=0.0)) / 4)
        e2e = max(e2e, err)
        say("end to end request", b, "max-abs error", err, "bound", tol)
        assert err <= tol, ("end to end", b, err)
    say(wl.name, "end-to-end max-abs error", e2e)
    return worst, e2e


@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_link_three_layers_small(layout):
    run_link(small(), 3, 256, layout)


def test_link_gqa4_d64_and_split_attention():
    # D = 64 with G = 4; long enough rows that attention splits keys (n_cu = 2 forces it)
    reqs = [W.Request([300, 700, 260], 40), W.Request([900], 9)]
    run_link(small(h_q=8, h_kv=2, d=64, seed=63, reqs=reqs), 2, 512, n_cu=2)


def test_link_full_size_sampled():
    # the bench batch (4 x ~50k tokens, k = 16, 32/8 heads of 128) through two layers of a
    # 4096-wide model; request 0 against the oracle end to end
    run_link(W.epic_sweep(k=16), 2, 4096, n_cu=256, requests=[0], per_layer=False)
