"""GPU parity of the paged shared-chunk path (pic_selective_attn_paged) against the
oracle: chunks gathered from the pool, rotated by R(delta_c), spliced with the fresh
rows, then selective attention -- bf16 I/O, max-abs <= 2e-2.  The pool is read-only:
it is checked to be bit-identical after the call."""

import sys

import numpy as np
import pytest
import torch

import position_independent_kv_rope_amd as P
from position_independent_kv_rope_amd import workloads as W
from oracle import pic_oracle as O

pytestmark = pytest.mark.gpu
TOL = 2e-2      # bf16 I/O
TOL_F32 = 1e-5  # fp32 I/O


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    P.lib()


def say(*a):
    print("[gpu-paged]", *a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def _drop_last_block(cbp, blocks, i):
    """A CSR block table whose row i lists one block fewer; every other row still lists
    its own blocks (the ids after row i move up by one place)."""
    keep = np.ones(len(blocks), dtype=bool)
    keep[cbp[i + 1] - 1] = False
    cbp = cbp.copy()
    cbp[i + 1:] -= 1
    return cbp, blocks[keep]


def _gather_or_zeros(pool64, cbp, blocks, i, L, h_kv, d):
    """The oracle's gather of pool chunk i; rows whose block its table row does not list
    read as zeros."""
    listed = min(L, (cbp[i + 1] - cbp[i]) * pool64.shape[1])
    g = O.gather_paged_chunk(pool64, blocks[cbp[i]:cbp[i + 1]], listed) if listed > 0 \
        else np.zeros((0, h_kv, d))
    if g.shape[0] < L:
        g = np.concatenate([g, np.zeros((L - g.shape[0], h_kv, d))])
    return g


def run_paged(wl, layout="adjacent", pos_base=0, nan_slack=False, n_cu=0, sample_rows=None,
              drop_last_block_of=None):
    reqs = [r.chunk_lens for r in wl.requests]
    ids = [r.chunk_ids for r in wl.requests]
    qs = [r.q_len for r in wl.requests]
    plan = P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, pos_base=pos_base, n_cu=n_cu,
                             chunk_ids_per_req=ids)
    plan.to_device()
    cbp, blocks = W.pool_block_table(wl)
    pk, pv = W.pool_tensors(wl)
    # the block table the kernel walks: enough blocks per chunk, ids inside the pool
    bs = wl.block_size
    assert len(cbp) == len(wl.pool_lens) + 1
    assert all(cbp[i + 1] - cbp[i] >= -(-L // bs) for i, L in enumerate(wl.pool_lens))
    assert blocks.min(initial=0) >= 0 and blocks.max(initial=0) < pk.shape[0]
    assert all(0 <= c < len(wl.pool_lens) for r in wl.requests for c in r.chunk_ids)
    if nan_slack:  # slots past a chunk's length hold NaN: they must not leak into outputs
        bs = wl.block_size
        for i, L in enumerate(wl.pool_lens):
            if L % bs:
                last = blocks[cbp[i + 1] - 1]
                pk[last, L % bs:] = float("nan")
                pv[last, L % bs:] = float("nan")
    if drop_last_block_of is not None:
        cbp, blocks = _drop_last_block(cbp, blocks, drop_last_block_of)
    q, kf, vf = W.fresh_tensors(wl, plan.n_rows)
    dev = "cuda"
    pkd, pvd = pk.to(dev), pv.to(dev)
    out = torch.full((plan.n_rows, wl.h_q, wl.head_dim), float("nan"), dtype=q.dtype, device=dev)
    ws = P.attn_workspace(plan, wl.head_dim)
    say(wl.name, "k=%d" % wl.k, layout, "pos_base=%d" % pos_base, "items=%d merges=%d" %
        (plan[P.H_N_ATTN_ITEMS], plan[P.H_N_MERGE]))
    lay = P.PIC_ROPE_HALF if layout == "half" else P.PIC_ROPE_ADJACENT
    P.pic_selective_attn_paged(plan, q.to(dev), pkd, pvd, torch.from_numpy(cbp).to(dev),
                               torch.from_numpy(blocks).to(dev), kf.to(dev), vf.to(dev), out,
                               wl.rope_base, layout=lay, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(torch.nan_to_num(pkd.cpu()), torch.nan_to_num(pk))  # pool untouched
    assert torch.equal(torch.nan_to_num(pvd.cpu()), torch.nan_to_num(pv))
    got_all = out.cpu()
    pk64, pv64 = f64(pk), f64(pv)
    worst = 0.0
    bs = wl.block_size
    for b, r in enumerate(wl.requests):
        row0, row1 = int(plan.req_row_ptr[b]), int(plan.req_row_ptr[b + 1])
        rows = O.recompute_positions(r.chunk_lens, r.q_len, wl.k)
        assert plan.rows[row0:row1].tolist() == rows
        if row1 == row0:
            continue
        ck = [_gather_or_zeros(pk64, cbp, blocks, i, wl.pool_lens[i], wl.h_kv, wl.head_dim)
              for i in r.chunk_ids]
        cv = [_gather_or_zeros(pv64, cbp, blocks, i, wl.pool_lens[i], wl.h_kv, wl.head_dim)
              for i in r.chunk_ids]
        offs = O.chunk_offsets(r.chunk_lens)
        if ck:
            k_ctx, v_ctx = O.rope_delta(ck, wl.rope_base, layout, pos_base), O.concat_chunks(cv)
        else:  # a request with only query tokens
            k_ctx = v_ctx = np.zeros((0, wl.h_kv, wl.head_dim))
        kx, vx = O.splice(k_ctx, v_ctx, f64(kf[row0:row1]), f64(vf[row0:row1]), rows,
                          offs[-1] + r.q_len)
        qb = f64(q[row0:row1])
        if sample_rows is None:
            want = O.selective_attn(qb, kx, vx, rows)
            got = f64(got_all[row0:row1])
        else:
            rng = np.random.default_rng(77 + b)
            n = row1 - row0
            picks = sorted(set(rng.integers(0, n, size=min(sample_rows, n)).tolist()) | {0, n - 1})
            heads = rng.integers(0, wl.h_q, size=len(picks))
            want = O.attn_rows_direct([qb[i, h] for i, h in zip(picks, heads)], kx, vx,
                                      [rows[i] for i in picks], heads // (wl.h_q // wl.h_kv))
            got = np.stack([f64(got_all[row0 + i, h]) for i, h in zip(picks, heads)])
        assert np.isfinite(got).all()
        err = float(np.max(np.abs(got - want)))
        worst = max(worst, err)
        if sample_rows is not None:
            say("request", b, "max-abs error", err)
        assert err <= (TOL_F32 if wl.dtype == "f32" else TOL), ("paged attention", b, err)
    say(wl.name, "max-abs error", worst)
    return worst


def small_pool(k, h_q=32, h_kv=4, d=128, seed=31, lens=None, n_req=3, dtype="bf16"):
    rng = np.random.default_rng(seed)
    lens = lens or [17, 33, 5, 64, 100, 48, 16, 1, 130, 77, 64, 15]
    reqs = []
    for b in range(n_req):
        m = int(rng.integers(2, len(lens)))
        ids = [int(x) for x in rng.permutation(len(lens))[:m]]
        reqs.append(W.Request([lens[i] for i in ids], int(rng.integers(1, 40)), chunk_ids=ids))
    return W.Workload("small_pool", dtype, h_q, h_kv, d, 500000.0, k, reqs, pool_lens=lens,
                      block_size=16, pool_block_perm_seed=seed + 1, seed=seed)


@pytest.mark.parametrize("k", [8, 3])
@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_paged_small(k, layout):
    run_paged(small_pool(k), layout)


def test_paged_nan_slack_and_pos_base():
    run_paged(small_pool(8, seed=41), nan_slack=True)
    run_paged(small_pool(0, h_q=16, h_kv=4, seed=43), pos_base=4)


def test_paged_edge_requests():
    # a lone chunk without query tokens, a request without chunks, a chunk used twice in
    # one request, chunks shorter than the seam window and exactly one pool block long
    lens = [16, 3, 200, 64, 1]
    reqs = [W.Request([200], 0, chunk_ids=[2]),
            W.Request([], 5, chunk_ids=[]),
            W.Request([16, 3, 16, 64, 1, 200], 7, chunk_ids=[0, 1, 0, 3, 4, 2])]
    wl = W.Workload("paged_edges", "bf16", 8, 2, 128, 10000.0, 8, reqs, pool_lens=lens,
                    block_size=16, pool_block_perm_seed=3, seed=53)
    run_paged(wl)


def test_paged_gqa4_d64():
    run_paged(small_pool(4, h_q=32, h_kv=8, d=64, seed=47))


@pytest.mark.parametrize("h_q", [32, 64])
def test_paged_wide_groups(h_q):
    # one KV head: G = 32 (a wave owns one row of the tile with all its heads) and G = 64
    # (32 consecutive head-major columns per wave)
    run_paged(small_pool(3, h_q=h_q, h_kv=1, d=64, seed=61 + h_q))


def test_paged_shared_pool_full_size_sampled():
    # the shared-pool workload (256 pooled chunks, 8 requests x ~116k tokens, w = 8) in
    # the launch configuration bench.py times (n_cu = 256), sampled rows
    run_paged(W.shared_pool(), n_cu=256, sample_rows=24)


# ---------------------------------------------------------------------------
# Decode step over the shared pool (pic_decode_attn_paged)
# ---------------------------------------------------------------------------


def run_decode(wl, layout="adjacent", nan_slack=False, n_cu=0, requests=None):
    reqs = [r.chunk_lens for r in wl.requests]
    ids = [r.chunk_ids for r in wl.requests]
    qs = [r.q_len for r in wl.requests]
    plan = P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, n_cu=n_cu, chunk_ids_per_req=ids)
    plan.to_device()
    cbp, blocks = W.pool_block_table(wl)
    pk, pv = W.pool_tensors(wl)
    bs = wl.block_size
    assert len(cbp) == len(wl.pool_lens) + 1
    assert all(cbp[i + 1] - cbp[i] >= -(-L // bs) for i, L in enumerate(wl.pool_lens))
    assert blocks.min(initial=0) >= 0 and blocks.max(initial=0) < pk.shape[0]
    if nan_slack:
        for i, L in enumerate(wl.pool_lens):
            if L % bs:
                last = blocks[cbp[i + 1] - 1]
                pk[last, L % bs:] = float("nan")
                pv[last, L % bs:] = float("nan")
    _, kf, vf = W.fresh_tensors(wl, plan.n_rows)
    qn, kn, vn = W.decode_tensors(wl)
    dev = "cuda"
    out = torch.full(qn.shape, float("nan"), dtype=qn.dtype, device=dev)
    say(wl.name, "decode", layout, "items=%d uses=%d pieces=%d workgroups=%d" % (
        plan[P.H_N_DEC_ITEMS], plan[P.H_N_DEC_USES], plan[P.H_N_DEC_PIECES], plan[P.H_N_DEC_WG]))
    lay = P.PIC_ROPE_HALF if layout == "half" else P.PIC_ROPE_ADJACENT
    P.pic_decode_attn_paged(plan, qn.to(dev), kn.to(dev), vn.to(dev), pk.to(dev), pv.to(dev),
                            torch.from_numpy(cbp).to(dev), torch.from_numpy(blocks).to(dev),
                            kf.to(dev), vf.to(dev), out, wl.rope_base, layout=lay)
    torch.cuda.synchronize()
    got_all = f64(out.cpu())
    assert np.isfinite(got_all).all()
    pk64, pv64 = f64(pk), f64(pv)
    worst = 0.0
    for b, r in enumerate(wl.requests):
        if requests is not None and b not in requests:
            continue
        row0, row1 = int(plan.req_row_ptr[b]), int(plan.req_row_ptr[b + 1])
        rows = O.recompute_positions(r.chunk_lens, r.q_len, wl.k)
        ck = [O.gather_paged_chunk(pk64, blocks[cbp[i]:cbp[i + 1]], wl.pool_lens[i]) for i in r.chunk_ids]
        cv = [O.gather_paged_chunk(pv64, blocks[cbp[i]:cbp[i + 1]], wl.pool_lens[i]) for i in r.chunk_ids]
        if ck:
            k_ctx, v_ctx = O.rope_delta(ck, wl.rope_base, layout), O.concat_chunks(cv)
        else:
            k_ctx = v_ctx = np.zeros((0, wl.h_kv, wl.head_dim))
        n_total = sum(r.chunk_lens) + r.q_len
        kx, vx = O.splice(k_ctx, v_ctx, f64(kf[row0:row1]), f64(vf[row0:row1]), rows, n_total)
        want = O.decode_attn(f64(qn[b]), kx, vx, f64(kn[b]), f64(vn[b]))
        err = float(np.max(np.abs(got_all[b] - want)))
        worst = max(worst, err)
        assert err <= TOL, ("decode", b, err)
    say(wl.name, "decode max-abs error", worst)
    return worst


@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_decode_small(layout):
    run_decode(small_pool(8), layout)


def test_decode_edges_nan_slack_and_gqa4_d64():
    run_decode(small_pool(8, seed=41), nan_slack=True)
    run_decode(small_pool(4, h_q=32, h_kv=8, d=64, seed=47))
    lens = [16, 3, 200, 64, 1]
    reqs = [W.Request([200], 0, chunk_ids=[2]),           # no recomputed rows at all
            W.Request([], 5, chunk_ids=[]),               # only query rows
            W.Request([16, 3, 16, 64, 1, 200], 7, chunk_ids=[0, 1, 0, 3, 4, 2])]
    run_decode(W.Workload("decode_edges", "bf16", 8, 2, 128, 10000.0, 8, reqs, pool_lens=lens,
                          block_size=16, pool_block_perm_seed=3, seed=53))


def test_decode_few_workgroups():
    # grids of 4 and 12 workgroups: each streams many pieces back to back and the equal
    # runs cut units in the middle, so one (use, kv head) leaves several records
    run_decode(small_pool(8, seed=59), n_cu=1)
    run_decode(small_pool(8, seed=61), layout="half", n_cu=3)


def test_decode_shared_pool_full_size():
    # the shared-pool batch (8 requests x ~116k tokens from 256 pooled chunks, w = 8):
    # every request's output against the oracle
    run_decode(W.shared_pool(), n_cu=256)


# pool K (and V) of pic_selective_attn_paged are addressed with 32-bit byte offsets:
# pool_blocks * 16 * h_kv * D * 2 <= 0x7fff0000 - 16 * h_kv * D * 2
POOL_LIMIT_BYTES = 0x7FFF0000


def test_largest_pool_prefill_and_decode():
    # a 2 GiB pool (131,066 blocks of 16 tokens, 4 KV heads of 128): one chunk in the
    # pool's last blocks in descending order, one on random blocks, one just below the
    # first; two requests splice them (one chunk shared).  Prefill of every row and the
    # decode step of both requests against the oracle.
    tok_bytes = 4 * 128 * 2
    n_blocks = (POOL_LIMIT_BYTES - 16 * tok_bytes) // (16 * tok_bytes)
    lens = [4100, 3000, 2500]
    need = [-(-L // 16) for L in lens]
    rng = np.random.default_rng(83)
    b0 = np.arange(n_blocks - 1, n_blocks - 1 - need[0], -1)
    b2 = np.arange(n_blocks - need[0] - need[2], n_blocks - need[0])
    rest = np.setdiff1d(np.arange(n_blocks), np.concatenate([b0, b2]))
    b1 = rng.choice(rest, need[1], replace=False)
    blocks = np.concatenate([b0, b1, b2]).astype(np.int32)
    cbp = np.concatenate([[0], np.cumsum(need)]).astype(np.int32)
    reqs = [W.Request([lens[0], lens[1], lens[2]], 64, chunk_ids=[0, 1, 2]),
            W.Request([lens[2], lens[0]], 32, chunk_ids=[2, 0])]
    wl = W.Workload("largest_pool", "bf16", 32, 4, 128, 500000.0, 8, reqs, pool_lens=lens,
                    block_size=16, seed=71)
    plan = P.pic_build_index([r.chunk_lens for r in reqs], [r.q_len for r in reqs], wl.k,
                             wl.h_q, wl.h_kv, n_cu=256, chunk_ids_per_req=[r.chunk_ids for r in reqs])
    plan.to_device()
    dev = "cuda"
    say("largest pool: drawing", n_blocks, "blocks on the device")
    shape = (n_blocks, 16, wl.h_kv, wl.head_dim)
    pk = W.device_draw(shape, 711, torch.bfloat16, dev)
    pv = W.device_draw(shape, 712, torch.bfloat16, dev)
    assert pk.numel() * 2 <= POOL_LIMIT_BYTES - 16 * tok_bytes
    used = torch.from_numpy(blocks.astype(np.int64)).to(dev)
    mini_k, mini_v = f64(pk.index_select(0, used)), f64(pv.index_select(0, used))
    mini_ids = np.arange(len(blocks))  # chunk i's blocks, in order, in the host copy
    q, kf, vf = W.fresh_tensors(wl, plan.n_rows)
    qn, kn, vn = W.decode_tensors(wl)
    out = torch.full((plan.n_rows, wl.h_q, wl.head_dim), float("nan"), dtype=q.dtype, device=dev)
    cbp_d, blocks_d = torch.from_numpy(cbp).to(dev), torch.from_numpy(blocks).to(dev)
    say("largest pool: prefill items=%d, decode pieces=%d" % (plan[P.H_N_ATTN_ITEMS],
                                                              plan[P.H_N_DEC_PIECES]))
    P.pic_selective_attn_paged(plan, q.to(dev), pk, pv, cbp_d, blocks_d, kf.to(dev), vf.to(dev),
                               out, wl.rope_base, workspace=P.attn_workspace(plan, wl.head_dim))
    dec = torch.full(qn.shape, float("nan"), dtype=qn.dtype, device=dev)
    P.pic_decode_attn_paged(plan, qn.to(dev), kn.to(dev), vn.to(dev), pk, pv, cbp_d, blocks_d,
                            kf.to(dev), vf.to(dev), dec, wl.rope_base)
    torch.cuda.synchronize()
    assert np.array_equal(f64(pk.index_select(0, used)), mini_k)  # pool untouched
    got_all, dec_all = f64(out.cpu()), f64(dec.cpu())
    assert np.isfinite(got_all).all() and np.isfinite(dec_all).all()
    for b, r in enumerate(reqs):
        row0, row1 = int(plan.req_row_ptr[b]), int(plan.req_row_ptr[b + 1])
        rows = O.recompute_positions(r.chunk_lens, r.q_len, wl.k)
        assert plan.rows[row0:row1].tolist() == rows
        ck = [O.gather_paged_chunk(mini_k, mini_ids[cbp[i]:cbp[i + 1]], lens[i]) for i in r.chunk_ids]
        cv = [O.gather_paged_chunk(mini_v, mini_ids[cbp[i]:cbp[i + 1]], lens[i]) for i in r.chunk_ids]
        k_ctx, v_ctx = O.rope_delta(ck, wl.rope_base), O.concat_chunks(cv)
        kx, vx = O.splice(k_ctx, v_ctx, f64(kf[row0:row1]), f64(vf[row0:row1]), rows,
                          sum(r.chunk_lens) + r.q_len)
        err = float(np.max(np.abs(got_all[row0:row1] - O.selective_attn(f64(q[row0:row1]), kx, vx, rows))))
        derr = float(np.max(np.abs(dec_all[b] - O.decode_attn(f64(qn[b]), kx, vx, f64(kn[b]), f64(vn[b])))))
        say("largest pool request", b, "prefill max-abs error", err, "decode", derr)
        assert err <= TOL and derr <= TOL


def _random_pool(i):
    """Seeded random pool and requests: chunk lengths from 1 row to several pool blocks,
    chunks shared between requests and repeated within one, chunk-free requests."""
    rng = np.random.default_rng(7000 + i)
    h_kv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    lens = [int(x) for x in rng.integers(1, 900, size=int(rng.integers(1, 10)))]
    reqs = []
    for _ in range(int(rng.integers(1, 5))):
        m = int(rng.integers(0, 7))
        ids = [int(x) for x in rng.integers(0, len(lens), size=m)]
        reqs.append(W.Request([lens[c] for c in ids], int(rng.integers(0 if m else 1, 50)), chunk_ids=ids))
    return W.Workload("random_pool%d" % i, "bf16", g * h_kv, h_kv, d, float(rng.choice([1e4, 5e5])),
                      int(rng.integers(0, 12)), reqs, pool_lens=lens, block_size=16,
                      pool_block_perm_seed=80 + i, seed=90 + i)


@pytest.mark.parametrize("i", range(8))
def test_random_pools(i):
    # paged prefill (every row), the gather form (every gathered row and output) and the
    # decode step (every request) on seeded random pools, both pair layouts, NaN in the
    # slack slots of every other case
    wl = _random_pool(i)
    layout = "half" if i % 2 else "adjacent"
    say("random pool", i, "h_q=%d h_kv=%d D=%d k=%d" % (wl.h_q, wl.h_kv, wl.head_dim, wl.k),
        layout, [(len(r.chunk_ids), r.q_len) for r in wl.requests])
    run_paged(wl, layout, nan_slack=bool(i % 2), n_cu=(256 if i % 3 == 0 else 2))
    run_pool_gather(wl, layout, nan_slack=bool(i % 2), n_cu=(2 if i % 3 == 0 else 256))
    if wl.h_q // wl.h_kv <= P.PIC_DECODE_COLS:
        run_decode(wl, layout, nan_slack=bool(i % 2), n_cu=(1 if i % 3 == 1 else 256))


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_paged_f32(layout, d):
    # fp32 I/O over the pool (keys rotated into the global frame as they are staged):
    # every row against the oracle at 1e-5, NaN in the slack slots, split items
    wl = small_pool(8, h_q=8, h_kv=2, d=d, seed=17 + d, dtype="f32")
    run_paged(wl, layout, nan_slack=True, n_cu=256)
    run_paged(small_pool(3, h_q=4, h_kv=4, d=d, seed=19 + d, dtype="f32"), layout, pos_base=2)
    # long chunks: keys split into ranges, so the fp32 merge runs over the pool too
    long = small_pool(8, h_q=8, h_kv=2, d=d, seed=23 + d, lens=[3000, 2600, 1290, 700, 64, 5],
                      dtype="f32")
    plan = P.pic_build_index([r.chunk_lens for r in long.requests], [r.q_len for r in long.requests],
                             long.k, long.h_q, long.h_kv, n_cu=256,
                             chunk_ids_per_req=[r.chunk_ids for r in long.requests])
    assert plan[P.H_N_MERGE] > 0
    run_paged(long, layout, n_cu=256)


@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_paged_f32_rotation_at_delta_near_two_to_the_20(layout):
    # pool chunks cached at local positions from -(2^20 - 5): each staged key is rotated
    # by off_c + 2^20 - 5 (about 1.05e6) on load; every row against the oracle at 1e-5
    wl = small_pool(4, h_q=8, h_kv=2, d=128, seed=29, dtype="f32")
    run_paged(wl, layout, pos_base=-(1 << 20) + 5, n_cu=256)


# ---------------------------------------------------------------------------
# Rotation + splice from the pool into contiguous buffers (pic_rope_splice_pool),
# then the contiguous selective attention over them
# ---------------------------------------------------------------------------


def run_pool_gather(wl, layout="adjacent", pos_base=0, nan_slack=False, n_cu=0,
                    sample_rows=None, drop_last_block_of=None):
    """Gather + rotate + splice from the pool with a paged plan, attend with the contiguous
    plan of the same requests; every row against the oracle.  drop_last_block_of: a pool
    chunk whose block-table row is cut by one block (its last rows must read as zeros)."""
    reqs = [r.chunk_lens for r in wl.requests]
    ids = [r.chunk_ids for r in wl.requests]
    qs = [r.q_len for r in wl.requests]
    pplan = P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, pos_base=pos_base, n_cu=n_cu,
                              chunk_ids_per_req=ids)
    cplan = P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, pos_base=pos_base, n_cu=n_cu)
    assert pplan.req_tok_ptr.tolist() == cplan.req_tok_ptr.tolist()
    assert pplan.rows.tolist() == cplan.rows.tolist()
    pplan.to_device()
    cplan.to_device()
    cbp, blocks = W.pool_block_table(wl)
    pk, pv = W.pool_tensors(wl)
    bs = wl.block_size
    if nan_slack:
        for i, L in enumerate(wl.pool_lens):
            if L % bs:
                last = blocks[cbp[i + 1] - 1]
                pk[last, L % bs:] = float("nan")
                pv[last, L % bs:] = float("nan")
    cbp_used = cbp.copy()
    if drop_last_block_of is not None:
        cbp_used, blocks = _drop_last_block(cbp, blocks, drop_last_block_of)
    q, kf, vf = W.fresh_tensors(wl, pplan.n_rows)
    dev = "cuda"
    k = torch.full((pplan.n_tokens, wl.h_kv, wl.head_dim), float("nan"), dtype=q.dtype, device=dev)
    v = torch.full_like(k, float("nan"))
    lay = P.PIC_ROPE_HALF if layout == "half" else P.PIC_ROPE_ADJACENT
    say(wl.name, "pool gather k=%d" % wl.k, layout, "pos_base=%d" % pos_base,
        "kblocks=%d" % pplan[P.H_N_KBLOCKS])
    P.pic_rope_splice_pool(pplan, pk.to(dev), pv.to(dev), torch.from_numpy(cbp_used).to(dev),
                           torch.from_numpy(blocks).to(dev), k, v, kf.to(dev), vf.to(dev),
                           wl.rope_base, layout=lay)
    out = torch.full((pplan.n_rows, wl.h_q, wl.head_dim), float("nan"), dtype=q.dtype, device=dev)
    P.pic_selective_attn(cplan, q.to(dev), k, v, out, workspace=P.attn_workspace(cplan, wl.head_dim))
    torch.cuda.synchronize()
    kg, vg, got_all = k.cpu(), v.cpu(), out.cpu()
    tol = TOL_F32 if wl.dtype == "f32" else TOL
    pk64, pv64 = f64(pk), f64(pv)
    worst = {"rope": 0.0, "attn": 0.0}
    for b, r in enumerate(wl.requests):
        tok0 = int(pplan.req_tok_ptr[b])
        row0, row1 = int(pplan.req_row_ptr[b]), int(pplan.req_row_ptr[b + 1])
        rows = O.recompute_positions(r.chunk_lens, r.q_len, wl.k)
        offs = O.chunk_offsets(r.chunk_lens)
        n_b = offs[-1] + r.q_len
        ck, cv = [], []
        for i in r.chunk_ids:  # blocks the table row does not list read as zeros
            ck.append(_gather_or_zeros(pk64, cbp_used, blocks, i, wl.pool_lens[i], wl.h_kv,
                                       wl.head_dim))
            cv.append(_gather_or_zeros(pv64, cbp_used, blocks, i, wl.pool_lens[i], wl.h_kv,
                                       wl.head_dim))
        if ck:
            k_ctx, v_ctx = O.rope_delta(ck, wl.rope_base, layout, pos_base), O.concat_chunks(cv)
        else:
            k_ctx = v_ctx = np.zeros((0, wl.h_kv, wl.head_dim))
        kx, vx = O.splice(k_ctx, v_ctx, f64(kf[row0:row1]), f64(vf[row0:row1]), rows, n_b)
        gk_b, gv_b = f64(kg[tok0:tok0 + n_b]), f64(vg[tok0:tok0 + n_b])
        assert np.isfinite(gk_b).all() and np.isfinite(gv_b).all()  # every row written
        rec = set(rows)
        keep = [j for j in range(offs[-1]) if j not in rec]
        if keep:
            err = float(np.max(np.abs(gk_b[keep] - kx[keep])))
            worst["rope"] = max(worst["rope"], err)
            assert err <= tol, ("pool rotation", b, err)
        assert np.array_equal(gv_b, vx)  # V and the fresh rows are bit copies
        assert np.array_equal(gk_b[rows], kx[rows])
        qb = f64(q[row0:row1])
        if row1 == row0:
            continue
        if sample_rows is None:
            want = O.selective_attn(qb, kx, vx, rows)
            got = f64(got_all[row0:row1])
        else:
            rng = np.random.default_rng(91 + b)
            n = row1 - row0
            picks = sorted(set(rng.integers(0, n, size=min(sample_rows, n)).tolist()) | {0, n - 1})
            heads = rng.integers(0, wl.h_q, size=len(picks))
            want = O.attn_rows_direct([qb[i, h] for i, h in zip(picks, heads)], kx, vx,
                                      [rows[i] for i in picks], heads // (wl.h_q // wl.h_kv))
            got = np.stack([f64(got_all[row0 + i, h]) for i, h in zip(picks, heads)])
        err = float(np.max(np.abs(got - want)))
        worst["attn"] = max(worst["attn"], err)
        assert err <= tol, ("attention over the gathered K/V", b, err)
    say(wl.name, "pool gather max-abs errors", worst)
    return worst


@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_pool_gather_small(layout):
    run_pool_gather(small_pool(8), layout, nan_slack=True)
    run_pool_gather(small_pool(3, h_q=16, h_kv=4, seed=43), layout, pos_base=4)


def test_pool_gather_f32_and_edges():
    run_pool_gather(small_pool(8, h_q=8, h_kv=2, d=64, seed=53, dtype="f32"), "adjacent",
                    nan_slack=True, n_cu=2)
    run_pool_gather(small_pool(2, h_q=4, h_kv=4, d=128, seed=57, dtype="f32"), "half",
                    pos_base=-(1 << 20) + 5)
    # a request without chunks (only query rows) and one without query rows
    wl = small_pool(4, seed=59)
    wl.requests.append(W.Request([], 9, chunk_ids=[]))
    wl.requests.append(W.Request([wl.pool_lens[2], wl.pool_lens[8]], 0, chunk_ids=[2, 8]))
    run_pool_gather(wl)


def test_undersized_block_table_row_reads_zeros():
    # pool chunk 8 (130 rows = 9 blocks) listed with 8 blocks: its last 2 rows read as
    # zeros, never the next chunk's first block -- through the gather and through the
    # paged attention kernel alike
    wl = small_pool(8, seed=61)
    wl.requests[0] = W.Request([wl.pool_lens[3], wl.pool_lens[8], wl.pool_lens[9]], 17,
                               chunk_ids=[3, 8, 9])
    run_pool_gather(wl, drop_last_block_of=8)
    run_paged(wl, drop_last_block_of=8)


def test_pool_gather_shared_pool_full_size_sampled():
    # the shared-pool batch (8 x ~116k tokens): every gathered row against the oracle,
    # sampled attention rows of the contiguous kernel over the result
    run_pool_gather(W.shared_pool(), n_cu=256, sample_rows=24)
