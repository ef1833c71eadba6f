"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each pin is chosen so a plausible mistake (dropped term, wrong sign or index,
transposed operand, off-by-one in k, top-left mask, positions restarted at 0)
fails at least one of them; the "planted" tests at the end plant such mistakes
into the oracle and check that a pin catches each one.  CPU only.
"""

import cmath
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import pic_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Recompute index
# ---------------------------------------------------------------------------


def test_worked_example_index():
    g = _golden("worked_example.json")
    assert O.chunk_offsets(g["chunk_lens"]) == g["offsets"]
    rows = O.recompute_positions(g["chunk_lens"], g["q_len"], g["k"])
    assert rows == g["recompute_positions"]
    assert len(rows) == g["n_recomputed"]
    assert O.chunk_offsets(g["chunk_lens"])[-1] == g["total_ctx_len"]
    assert g["total_ctx_len"] + g["q_len"] == g["n_total"]
    assert _recompute_by_chunk_walk(g["chunk_lens"], g["q_len"], g["k"]) == rows


def test_k_sweep_counts():
    g = _golden("k_sweep.json")
    assert sum(g["chunk_lens"]) + g["q_len"] == g["n_total"]
    for row in g["rows"]:
        rows = O.recompute_positions(g["chunk_lens"], g["q_len"], row["k"])
        assert len(rows) == row["recompute_tokens"]
        assert round(100.0 * len(rows) / g["n_total"], 1) == row["percent"]


def test_method_table_count_formula():
    # EPIC method table: LegoLink-k recomputes (chunks - 1) * k + q tokens when
    # every chunk has at least k tokens.
    rng = np.random.default_rng(0)
    for _ in range(200):
        k = int(rng.integers(0, 9))
        n = int(rng.integers(1, 7))
        lens = [int(x) for x in rng.integers(k, k + 10, size=n)]
        q = int(rng.integers(0, 6))
        assert len(O.recompute_positions(lens, q, k)) == (n - 1) * k + q


def _recompute_by_chunk_walk(chunk_lens, q_len, k):
    """Second formulation of the recompute set, chunk by chunk (the oracle scans
    positions): for each chunk after the first, its first min(k, L_c) positions, then
    the query positions."""
    out, off = [], 0
    for c, length in enumerate(chunk_lens):
        if c > 0:
            out.extend(off + j for j in range(min(k, length)))
        off += length
    return out + list(range(off, off + q_len))


def test_chunk_walk_formulation_exhaustive():
    import itertools
    for n in range(1, 4):
        for lens in itertools.product(range(0, 5), repeat=n):
            for q in range(0, 3):
                for k in range(0, 6):
                    a = O.recompute_positions(list(lens), q, k)
                    b = _recompute_by_chunk_walk(list(lens), q, k)
                    assert a == b, (lens, q, k)
                    assert a == sorted(set(a))


def test_chunk_zero_never_recomputed_and_queries_always():
    rng = np.random.default_rng(1)
    for _ in range(100):
        lens = [int(x) for x in rng.integers(0, 12, size=int(rng.integers(1, 6)))]
        q = int(rng.integers(0, 5))
        k = int(rng.integers(0, 20))
        rows = O.recompute_positions(lens, q, k)
        ctx = sum(lens)
        assert all(r >= lens[0] for r in rows)
        assert [r for r in rows if r >= ctx] == list(range(ctx, ctx + q))


# ---------------------------------------------------------------------------
# RoPE and the delta rotation
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_rope_two_dims_is_complex_multiplication(layout):
    # D = 2: theta_0 = 1, so RoPE at position p multiplies a + ib by e^{ip}.
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 3, 2))
    pos = rng.integers(-50, 50, size=7)
    got = O.rope_rotate(x, pos, 10000.0, layout)
    z = (x[..., 0] + 1j * x[..., 1]) * np.exp(1j * pos.astype(np.float64))[:, None]
    assert np.max(np.abs(got[..., 0] - z.real)) < 1e-13
    assert np.max(np.abs(got[..., 1] - z.imag)) < 1e-13


def test_rope_pair_layout_and_frequency_unit_vectors():
    # D = 4, base B: theta_1 = B^(-1/2).  Unit vector on the first member of pair 1.
    base, p = 10000.0, 3
    th1 = 1.0 / math.sqrt(base)
    x = np.zeros((1, 1, 4))
    x[0, 0, 2] = 1.0  # adjacent layout: pair 1 is (2, 3)
    got = O.rope_rotate(x, [p], base, "adjacent")[0, 0]
    assert np.allclose(got, [0.0, 0.0, math.cos(p * th1), math.sin(p * th1)], atol=1e-15)
    x = np.zeros((1, 1, 4))
    x[0, 0, 1] = 1.0  # half layout: pair 1 is (1, 3)
    got = O.rope_rotate(x, [p], base, "half")[0, 0]
    assert np.allclose(got, [0.0, math.cos(p * th1), 0.0, math.sin(p * th1)], atol=1e-15)
    # pair 0 rotates at theta_0 = 1 in both layouts
    x = np.zeros((1, 1, 4))
    x[0, 0, 0] = 1.0
    for layout, idx in (("adjacent", 1), ("half", 2)):
        got = O.rope_rotate(x, [p], base, layout)[0, 0]
        want = np.zeros(4)
        want[0], want[idx] = math.cos(p), math.sin(p)
        assert np.allclose(got, want, atol=1e-15)


def test_rope_theta_matches_footnote_inv_freq():
    # [RoPE-C] footnote 3 (HF Llama): inv_freq = 1 / base^(arange(0, D, 2) / D)
    for d, base in ((16, 1e4), (128, 5e5), (64, 1e6)):
        inv = 1.0 / (base ** (np.arange(0, d, 2, dtype=np.float64) / d))
        assert np.allclose(O.rope_theta(d, base), inv, rtol=1e-14, atol=0)


@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_rope_additivity_closed_form(layout):
    # R(delta) RoPE(x, p) = RoPE(x, p + delta): rotating a cached row from p by delta
    # equals rotating it directly at p + delta ([RoPE-C] 3.3), fp64 to 1e-10.
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 2, 128))
    p = rng.integers(0, 4096, size=64)
    delta = rng.integers(-131072, 131072, size=64)
    a = O.rope_rotate(O.rope_rotate(x, p, 5e5, layout), delta, 5e5, layout)
    b = O.rope_rotate(x, p + delta, 5e5, layout)
    assert np.max(np.abs(a - b)) < 1e-10
    # inverse and identity
    back = O.rope_rotate(O.rope_rotate(x, p, 5e5, layout), -p, 5e5, layout)
    assert np.max(np.abs(back - x)) < 1e-10
    assert np.array_equal(O.rope_rotate(x, np.zeros(64, dtype=np.int64), 5e5, layout), x)


@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_rope_norm_and_relative_position(layout):
    rng = np.random.default_rng(4)
    q = rng.standard_normal((32, 1, 64))
    k = rng.standard_normal((32, 1, 64))
    m = rng.integers(0, 70000, size=32)
    n = rng.integers(0, 70000, size=32)
    s = rng.integers(-20000, 20000, size=32)
    ia, ib = O.rope_pair_index(64, layout)
    rq = O.rope_rotate(q, m, 5e5, layout)
    # per-pair norm preserved
    assert np.allclose(rq[..., ia] ** 2 + rq[..., ib] ** 2, q[..., ia] ** 2 + q[..., ib] ** 2,
                       rtol=0, atol=1e-12)
    # <R(m) q, R(n) k> depends on n - m only ([RoPE-C] 2.2)
    d1 = np.sum(O.rope_rotate(q, m, 5e5, layout) * O.rope_rotate(k, n, 5e5, layout), axis=-1)
    d2 = np.sum(O.rope_rotate(q, m + s, 5e5, layout) * O.rope_rotate(k, n + s, 5e5, layout), axis=-1)
    assert np.max(np.abs(d1 - d2)) < 1e-10


@pytest.mark.parametrize("pos_base", [0, 4])
def test_rope_delta_restores_global_rotation(pos_base):
    # Cached chunk rows = RoPE(K0, pos_base + local t); after the delta rotation they
    # must equal RoPE(K0, global position) for every chunk, including chunk 0 when
    # pos_base != 0 (negative delta).
    rng = np.random.default_rng(5)
    lens = [5, 0, 7, 3]
    offs = O.chunk_offsets(lens)
    k0 = rng.standard_normal((offs[-1], 2, 32))
    cached = []
    for c, L in enumerate(lens):
        cached.append(O.rope_rotate(k0[offs[c]:offs[c] + L], pos_base + np.arange(L), 1e4))
    got = O.rope_delta(cached, 1e4, pos_base=pos_base)
    want = O.rope_rotate(k0, np.arange(offs[-1]), 1e4)
    assert np.max(np.abs(got - want)) < 1e-12


@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_scheme_b_equals_scheme_c(layout):
    # [RoPE-C] 3.2 and 3.3 reach the same K at the target positions: RoPE applied to the
    # position-free rows at global positions (scheme B) equals the delta rotation of
    # rows cached with RoPE at local positions (scheme C).
    rng = np.random.default_rng(8)
    lens = [6, 0, 9, 4, 1]
    offs = O.chunk_offsets(lens)
    nope = [rng.standard_normal((L, 2, 16)) for L in lens]
    cached = [O.rope_rotate(x, np.arange(x.shape[0]), 1e4, layout) for x in nope]
    got = O.rope_apply(nope, 1e4, layout)
    want = O.rope_delta(cached, 1e4, layout)
    assert got.shape == (offs[-1], 2, 16)
    assert np.max(np.abs(got - want)) < 1e-12


def test_scheme_b_two_dims_is_complex_rotation_by_global_position():
    # D = 2: one pair with theta_0 = 1, so row t of the concatenation turns by t radians.
    lens = [3, 2, 4]
    rng = np.random.default_rng(9)
    nope = [rng.standard_normal((L, 1, 2)) for L in lens]
    got = O.rope_apply(nope, 10000.0)
    t = 0
    for x in nope:
        for row in x:
            z = complex(row[0, 0], row[0, 1]) * cmath.exp(1j * t)
            assert abs(got[t, 0, 0] - z.real) < 1e-12 and abs(got[t, 0, 1] - z.imag) < 1e-12
            t += 1


def test_planted_scheme_b_local_positions_fails():
    # restarting positions at every chunk (forgetting the offsets) must break the pin
    rng = np.random.default_rng(10)
    nope = [rng.standard_normal((L, 1, 8)) for L in (5, 5)]
    wrong = np.concatenate([O.rope_rotate(x, np.arange(5), 1e4) for x in nope])
    assert np.max(np.abs(wrong - O.rope_apply(nope, 1e4))) > 0.1


# ---------------------------------------------------------------------------
# Splice layout and offset mask
# ---------------------------------------------------------------------------


def test_worked_example_splice_layout():
    g = _golden("worked_example.json")
    lens, q, k = g["chunk_lens"], g["q_len"], g["k"]
    rows = O.recompute_positions(lens, q, k)
    ctx = sum(lens)
    # tag every cached row with 1000 + position and every fresh row with 2000 + r
    v_ctx = (1000.0 + np.arange(ctx)).reshape(ctx, 1, 1)
    v_fresh = (2000.0 + np.arange(len(rows))).reshape(len(rows), 1, 1)
    _, vx = O.splice(v_ctx, v_ctx, v_fresh, v_fresh, rows, g["n_total"])
    src = g["spliced_row_source"]
    for key, positions in src.items():
        for p in positions:
            val = vx[p, 0, 0]
            if key.startswith("cached"):
                assert val == 1000.0 + p
            else:
                assert val == 2000.0 + rows.index(p)
    assert not np.isnan(vx).any()


def test_offset_mask_examples():
    g = _golden("offset_mask_exercise.json")
    for ex in g["examples"]:
        P, C = ex["past_len"], ex["new_len"]
        m = O.offset_mask(P, C)
        assert list(m.shape) == ex["score_shape"]
        assert list(m.sum(axis=1)) == ex["visible_keys"]
        top_left = np.tril(np.ones((C, P + C), dtype=bool))
        assert list(top_left.sum(axis=1)) == ex["top_left_visible_keys"]
        assert (P + np.arange(C)).tolist() == ex["query_positions"]


# ---------------------------------------------------------------------------
# Selective attention
# ---------------------------------------------------------------------------


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_full_recompute_equals_brute_force():
    # k >= every chunk length: every row after chunk 0 is fresh, so the selected rows
    # of the causal attention over the whole prompt (independent code) must match.
    rng = np.random.default_rng(6)
    lens, q_len, hq, hkv, d = [3, 4, 2], 2, 4, 2, 8
    n = sum(lens) + q_len
    q_all, k_all, v_all = _rand(rng, n, hq, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
    rows = O.recompute_positions(lens, q_len, 10)
    cached_k = [k_all[0:3], _rand(rng, 4, hkv, d), _rand(rng, 2, hkv, d)]
    cached_v = [v_all[0:3], _rand(rng, 4, hkv, d), _rand(rng, 2, hkv, d)]
    res = O.link_request(cached_k, cached_v, q_len, 10, k_all[rows], v_all[rows], q_all[rows], 1e4)
    want = O.full_causal_attn(q_all, k_all, v_all)[rows]
    assert np.max(np.abs(res["out"] - want)) < 1e-10


@pytest.mark.parametrize("k", [0, 1, 2, 5])
@pytest.mark.parametrize("layout", ["adjacent", "half"])
def test_consistency_invariant_any_k(k, layout):
    # One layer with pre-RoPE K0/Q0: cached K = RoPE(K0, local), fresh = RoPE(., global).
    # Delta rotation + splice rebuild RoPE(K0, global) exactly, so the selected rows
    # equal full causal attention for every k.  Pins rope_delta + splice + attention.
    rng = np.random.default_rng(7 + k)
    lens, q_len, hq, hkv, d, base = [4, 5, 5], 3, 4, 2, 16, 1e4
    offs = O.chunk_offsets(lens)
    n = offs[-1] + q_len
    q0, k0, v = _rand(rng, n, hq, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
    pos = np.arange(n)
    q_glob = O.rope_rotate(q0, pos, base, layout)
    k_glob = O.rope_rotate(k0, pos, base, layout)
    rows = O.recompute_positions(lens, q_len, k)
    cached_k = [O.rope_rotate(k0[offs[c]:offs[c + 1]], np.arange(lens[c]), base, layout)
                for c in range(len(lens))]
    cached_v = [v[offs[c]:offs[c + 1]] for c in range(len(lens))]
    res = O.link_request(cached_k, cached_v, q_len, k, k_glob[rows], v[rows], q_glob[rows],
                         base, layout)
    assert np.max(np.abs(res["kx"] - k_glob)) < 1e-12
    want = O.full_causal_attn(q_glob, k_glob, v)[rows]
    assert np.max(np.abs(res["out"] - want)) < 1e-10


def test_matches_torch_sdpa_with_explicit_mask():
    rng = np.random.default_rng(8)
    lens, q_len, hq, hkv, d = [6, 3, 7], 4, 6, 3, 16
    n = sum(lens) + q_len
    rows = O.recompute_positions(lens, q_len, 2)
    kx, vx = _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
    q = _rand(rng, len(rows), hq, d)
    got = O.selective_attn(q, kx, vx, rows)
    group = hq // hkv
    kt = torch.from_numpy(kx).permute(1, 0, 2).repeat_interleave(group, 0)  # [Hq, N, D]
    vt = torch.from_numpy(vx).permute(1, 0, 2).repeat_interleave(group, 0)
    qt = torch.from_numpy(q).permute(1, 0, 2)  # [Hq, R, D]
    mask = torch.arange(n)[None, :] <= torch.tensor(rows)[:, None]  # [R, N]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    assert np.max(np.abs(ref.permute(1, 0, 2).numpy() - got)) < 1e-12


def test_special_cases():
    rng = np.random.default_rng(9)
    d = 8
    # A request whose only chunk is empty and one query token: row 0 sees key 0 only.
    rows = O.recompute_positions([0], 1, 3)
    assert rows == [0]
    kx, vx = _rand(rng, 1, 1, d), _rand(rng, 1, 1, d)
    out = O.selective_attn(_rand(rng, 1, 2, d), kx, vx, rows)
    assert np.array_equal(out[0, 0], vx[0, 0]) and np.array_equal(out[0, 1], vx[0, 0])
    # identical V rows: output is that row whatever the scores
    lens, q_len = [5, 6], 3
    n = sum(lens) + q_len
    rows = O.recompute_positions(lens, q_len, 2)
    vrow = _rand(rng, 1, 1, d)
    vx = np.repeat(vrow, n, axis=0)
    out = O.selective_attn(_rand(rng, len(rows), 1, d) * 5, _rand(rng, n, 1, d), vx, rows)
    assert np.max(np.abs(out - vrow[0, 0])) < 1e-12


def test_causality_probe_and_input_immutability():
    # [KV-scratch] equivalence checks: changing the last token leaves earlier outputs
    # unchanged; the inputs are not modified.
    rng = np.random.default_rng(10)
    lens, q_len, hq, hkv, d = [4, 4, 4], 3, 2, 1, 8
    n = sum(lens) + q_len
    rows = O.recompute_positions(lens, q_len, 2)
    kx, vx, q = _rand(rng, n, hkv, d), _rand(rng, n, hkv, d), _rand(rng, len(rows), hq, d)
    copies = [a.copy() for a in (kx, vx, q)]
    a = O.selective_attn(q, kx, vx, rows)
    for x, c in zip((kx, vx, q), copies):
        assert np.array_equal(x, c)
    kx2, vx2, q2 = kx.copy(), vx.copy(), q.copy()
    kx2[-1] += 3.0
    vx2[-1] -= 2.0
    q2[-1] *= -1.0
    b = O.selective_attn(q2, kx2, vx2, rows)
    assert np.array_equal(a[:-1], b[:-1])
    assert not np.allclose(a[-1], b[-1])


def test_paged_gather_roundtrip():
    rng = np.random.default_rng(11)
    bs, L, h, d = 4, 10, 2, 8
    chunk = _rand(rng, L, h, d)
    n_blocks = 7
    pool = np.zeros((n_blocks, bs, h, d))
    blocks = [5, 1, 3]  # physical blocks of this chunk, in order
    for t in range(L):
        pool[blocks[t // bs], t % bs] = chunk[t]
    assert np.array_equal(O.gather_paged_chunk(pool, blocks, L), chunk)


# ---------------------------------------------------------------------------
# Planted mistakes: each must make a pin fail by far more than its tolerance
# ---------------------------------------------------------------------------


def _consistency_error(layout="adjacent", k=2):
    rng = np.random.default_rng(12)
    lens, q_len, hq, hkv, d, base = [4, 5, 5], 3, 4, 2, 16, 1e4
    offs = O.chunk_offsets(lens)
    n = offs[-1] + q_len
    q0, k0, v = _rand(rng, n, hq, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
    pos = np.arange(n)
    q_glob = O.rope_rotate(q0, pos, base, layout)
    k_glob = O.rope_rotate(k0, pos, base, layout)
    rows = O.recompute_positions(lens, q_len, k)
    cached_k = [O.rope_rotate(k0[offs[c]:offs[c + 1]], np.arange(lens[c]), base, layout)
                for c in range(len(lens))]
    cached_v = [v[offs[c]:offs[c + 1]] for c in range(len(lens))]
    res = O.link_request(cached_k, cached_v, q_len, k, k_glob[rows], v[rows], q_glob[rows],
                         base, layout)
    want = O.full_causal_attn(q_glob, k_glob, v)[rows]
    return float(np.max(np.abs(res["out"] - want)))


def test_planted_delta_zero_is_caught(monkeypatch):
    assert _consistency_error() < 1e-10
    monkeypatch.setattr(O, "rope_delta", lambda chunks, base, layout="adjacent", pos_base=0:
                        O.concat_chunks(chunks))
    assert _consistency_error() > 1e-2


def test_planted_top_left_mask_is_caught(monkeypatch):
    monkeypatch.setattr(O, "offset_mask",
                        lambda P, C: np.tril(np.ones((C, P + C), dtype=bool)))
    assert _consistency_error() > 1e-2


def test_planted_dropped_scale_is_caught(monkeypatch):
    real = O.selective_attn
    monkeypatch.setattr(O, "selective_attn", lambda q, kx, vx, rows, scale=None:
                        real(q, kx, vx, rows, 1.0))
    assert _consistency_error() > 1e-2


def test_planted_fresh_rows_at_local_positions_is_caught():
    # Fresh K/Q rotated at positions restarted from 0 (the [KV-scratch] "positions
    # reset" injection) instead of their global positions.
    rng = np.random.default_rng(15)
    lens, q_len, hq, hkv, d, base = [4, 5, 5], 3, 4, 2, 16, 1e4
    offs = O.chunk_offsets(lens)
    n = offs[-1] + q_len
    q0, k0, v = _rand(rng, n, hq, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
    k_glob = O.rope_rotate(k0, np.arange(n), base)
    q_glob = O.rope_rotate(q0, np.arange(n), base)
    rows = O.recompute_positions(lens, q_len, 2)
    restart = np.arange(len(rows))
    cached_k = [O.rope_rotate(k0[offs[c]:offs[c + 1]], np.arange(lens[c]), base)
                for c in range(len(lens))]
    cached_v = [v[offs[c]:offs[c + 1]] for c in range(len(lens))]
    res = O.link_request(cached_k, cached_v, q_len, 2,
                         O.rope_rotate(k0[rows], restart, base), v[rows],
                         O.rope_rotate(q0[rows], restart, base), base)
    want = O.full_causal_attn(q_glob, k_glob, v)[rows]
    assert np.max(np.abs(res["out"] - want)) > 1e-2


def test_planted_wrong_rotation_sign_is_caught(monkeypatch):
    real = O.rope_rotate
    monkeypatch.setattr(O, "rope_rotate", lambda x, p, base, layout="adjacent":
                        real(x, -np.asarray(p), base, layout))
    x = np.random.default_rng(13).standard_normal((3, 1, 2))
    pos = np.array([1, 2, 3])
    z = (x[..., 0] + 1j * x[..., 1]) * np.exp(1j * pos)[:, None]
    got = O.rope_rotate(x, pos, 1e4)
    assert np.max(np.abs(got[..., 1] - z.imag)) > 1e-2


def test_planted_gqa_map_is_caught(monkeypatch):
    rng = np.random.default_rng(14)
    lens, q_len, hq, hkv, d = [3, 4, 2], 2, 4, 2, 8
    n = sum(lens) + q_len
    q_all, k_all, v_all = _rand(rng, n, hq, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
    rows = O.recompute_positions(lens, q_len, 10)
    want = O.full_causal_attn(q_all, k_all, v_all)[rows]
    good = O.selective_attn(q_all[rows], k_all, v_all, rows)
    assert np.max(np.abs(good - want)) < 1e-10
    # interleaved head map (h % Hkv) instead of contiguous groups (h // G)
    k_perm = k_all[:, [0, 1], :]
    q_perm = q_all[rows][:, [0, 2, 1, 3], :]
    bad = O.selective_attn(q_perm, k_perm, v_all, rows)[:, [0, 2, 1, 3], :]
    assert np.max(np.abs(bad - want)) > 1e-2


def test_planted_k_off_by_one_is_caught():
    g = _golden("worked_example.json")
    assert O.recompute_positions(g["chunk_lens"], g["q_len"], g["k"] + 1) != g["recompute_positions"]
    assert O.recompute_positions(g["chunk_lens"], g["q_len"], g["k"] - 1) != g["recompute_positions"]


def test_attn_rows_direct_matches_selective_attn():
    # the one-row-at-a-time form used for sampled parity at full size is the same
    # definition as the run-based selective_attn (and so as the brute force)
    rng = np.random.default_rng(16)
    lens, q_len, hq, hkv, d = [7, 9, 4], 5, 8, 2, 16
    n = sum(lens) + q_len
    rows = O.recompute_positions(lens, q_len, 3)
    kx, vx = _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
    q = _rand(rng, len(rows), hq, d)
    full = O.selective_attn(q, kx, vx, rows)
    picks = [(i, h) for i in range(len(rows)) for h in (0, 3, 7)]
    got = O.attn_rows_direct([q[i, h] for i, h in picks], kx, vx, [rows[i] for i, _ in picks],
                             [h // (hq // hkv) for _, h in picks])
    want = np.stack([full[i, h] for i, h in picks])
    assert np.max(np.abs(got - want)) < 1e-12


# ---------------------------------------------------------------------------
# Decode after the link
# ---------------------------------------------------------------------------


def test_decode_attn_is_last_row_of_full_causal_attention():
    # the decode output equals the last row of plain causal attention over the spliced
    # sequence extended by the new token (brute force, N x N mask)
    rng = np.random.default_rng(11)
    n, hq, hkv, d = 13, 4, 2, 8
    k_all = rng.standard_normal((n + 1, hkv, d))
    v_all = rng.standard_normal((n + 1, hkv, d))
    q_all = rng.standard_normal((n + 1, hq, d))
    want = O.full_causal_attn(q_all, k_all, v_all)[n]
    got = O.decode_attn(q_all[n], k_all[:n], v_all[:n], k_all[n], v_all[n])
    assert np.max(np.abs(got - want)) < 1e-12


def test_decode_attn_single_key_and_planted_self_exclusion():
    rng = np.random.default_rng(12)
    d = 8
    k_new, v_new = rng.standard_normal((1, d)), rng.standard_normal((1, d))
    # no earlier keys: the output is the new token's own value
    got = O.decode_attn(rng.standard_normal((2, d)), np.zeros((0, 1, d)), np.zeros((0, 1, d)),
                        k_new[0][None], v_new[0][None])
    assert np.allclose(got, np.broadcast_to(v_new, (2, d)), atol=1e-12)
    # leaving the new token out of its own keys must change the result
    kx, vx = rng.standard_normal((6, 1, d)), rng.standard_normal((6, 1, d))
    q = rng.standard_normal((1, d))
    with_self = O.decode_attn(q, kx, vx, k_new, v_new)
    without = O.selective_attn(q[None], kx, vx, [5])[0]
    assert np.max(np.abs(with_self - without)) > 1e-3


# ---------------------------------------------------------------------------
# The multi-layer link: compute_qkv at global positions, splice, attention, residual
# ---------------------------------------------------------------------------


def _tiny_model(seed, n_layers, d_model=16, h_q=4, h_kv=2, d=4):
    rng = np.random.default_rng(seed)
    n_out = (h_q + 2 * h_kv) * d
    return [(rng.standard_normal((n_out, d_model)) / math.sqrt(d_model),
             rng.standard_normal((d_model, h_q * d)) / math.sqrt(h_q * d))
            for _ in range(n_layers)]


def _compiled_link(weights, x_chunks, x_query, k, base, layout, pos_base, h_q=4, h_kv=2,
                   link=None):
    """Compile every chunk alone at local positions pos_base.. ([EPIC] compile_chunk), then
    link the request: returns (link rows, link x, full-prefill x of the whole sequence)."""
    lens = [len(c) for c in x_chunks]
    per_layer = [{"w_qkv": w, "w_o": wo, "k_chunks": [], "v_chunks": []} for w, wo in weights]
    for xc in x_chunks:
        comp = O.prefill_layers(xc, weights, pos_base + np.arange(len(xc)), h_q, h_kv, base, layout)
        for layer, kc, vc in zip(per_layer, comp["k"], comp["v"]):
            layer["k_chunks"].append(kc)
            layer["v_chunks"].append(vc)
    x_all = np.concatenate(list(x_chunks) + [x_query], axis=0)
    rows = O.recompute_positions(lens, len(x_query), k)
    res = (link or O.link_layers)(x_all[rows], per_layer, len(x_query), k, h_q, h_kv, base,
                                  layout, pos_base)
    full = O.prefill_layers(x_all, weights, np.arange(len(x_all)), h_q, h_kv, base, layout)
    return res["rows"], res["x"], full["x"]


@pytest.mark.parametrize("layout,pos_base", [("adjacent", 0), ("half", 0), ("adjacent", 4)])
def test_link_layers_full_recompute_equals_prefill(layout, pos_base):
    # chunks compiled alone, then linked with k >= every chunk length: every row but
    # chunk 0's is recomputed, so after all layers the rows' hidden states equal a plain
    # causal prefill of the whole sequence ([EPIC] full recompute; fp64 1e-10)
    rng = np.random.default_rng(31)
    weights = _tiny_model(32, 3)
    x_chunks = [rng.standard_normal((n, 16)) for n in (4, 5, 5)]
    x_query = rng.standard_normal((3, 16))
    rows, got, full = _compiled_link(weights, x_chunks, x_query, 5, 1e4, layout, pos_base)
    assert rows == list(range(4, 17))
    assert np.max(np.abs(got - full[rows])) < 1e-10
    # with chunk 0 alone and pos_base 0, even k = 0 is exact (no seam to repair)
    rows0, got0, full0 = _compiled_link(weights, x_chunks[:1], x_query, 0, 1e4, layout, 0)
    assert np.max(np.abs(got0 - full0[rows0])) < 1e-10


def test_link_layers_seam_recompute_differs_from_full_recompute():
    # k < L: cached rows keep their chunk-local context, so the link is an approximation
    # of full recompute, and a visible one with random weights (the pins above are not
    # vacuous)
    rng = np.random.default_rng(33)
    weights = _tiny_model(34, 2)
    x_chunks = [rng.standard_normal((n, 16)) for n in (4, 5, 5)]
    x_query = rng.standard_normal((3, 16))
    rows, got, full = _compiled_link(weights, x_chunks, x_query, 2, 1e4, "adjacent", 0)
    assert rows == [4, 5, 9, 10, 14, 15, 16]
    assert np.max(np.abs(got - full[rows])) > 1e-3


def test_link_layers_one_layer_is_link_request_plus_projection():
    # one layer: the attention part is exactly the single-layer link of the rows' fresh
    # Q/K/V, and the layer adds O W_o^T to the hidden states
    rng = np.random.default_rng(35)
    (w, wo), = _tiny_model(36, 1)
    lens, q_len, k = [4, 5, 5], 3, 2
    kc = [rng.standard_normal((n, 2, 4)) for n in lens]
    vc = [rng.standard_normal((n, 2, 4)) for n in lens]
    rows = O.recompute_positions(lens, q_len, k)
    x = rng.standard_normal((len(rows), 16))
    q, kf, vf = O.qkv_rope(x, w, rows, 4, 2, 1e4)
    one = O.link_request(kc, vc, q_len, k, kf, vf, q, 1e4)
    got = O.link_layers(x, [{"w_qkv": w, "w_o": wo, "k_chunks": kc, "v_chunks": vc}], q_len, k,
                        4, 2, 1e4)["x"]
    assert np.max(np.abs(got - (x + one["out"].reshape(len(rows), -1) @ wo.T))) < 1e-12


def test_qkv_rope_split_and_rotation():
    # the projection's output features are Q heads, then K heads, then V heads; with an
    # identity-like weight each part is the matching slice of x, Q and K rotated at the
    # given positions and V untouched
    rng = np.random.default_rng(37)
    h_q, h_kv, d = 2, 1, 4
    x = rng.standard_normal((5, (h_q + 2 * h_kv) * d))
    w = np.eye(x.shape[1])
    pos = [0, 3, 7, 100, -2]
    q, k, v = O.qkv_rope(x, w, pos, h_q, h_kv, 1e4)
    assert np.allclose(q[0], x[0, :8].reshape(2, 4), atol=1e-15)  # position 0: identity
    assert np.allclose(v, x[:, 12:].reshape(5, 1, 4), atol=1e-15)
    # D = 4, pair i = (2i, 2i+1) rotated by p * theta_i: complex multiplication
    theta = [1.0, 1e4 ** -0.5]
    for t, p in enumerate(pos):
        for i in range(2):
            z = complex(x[t, 8 + 2 * i], x[t, 9 + 2 * i]) * cmath.exp(1j * p * theta[i])
            assert abs(complex(k[t, 0, 2 * i], k[t, 0, 2 * i + 1]) - z) < 1e-12


@pytest.mark.parametrize("mistake", ["local_positions", "no_residual", "layer_order"])
def test_planted_link_layer_mistakes_fail(mistake):
    rng = np.random.default_rng(39)
    weights = _tiny_model(40, 3)
    x_chunks = [rng.standard_normal((n, 16)) for n in (4, 5, 5)]
    x_query = rng.standard_normal((3, 16))

    def wrong(x_rows, layers, q_len, k, h_q, h_kv, base, layout, pos_base, scale=None):
        lens = [len(c) for c in layers[0]["k_chunks"]]
        rows = O.recompute_positions(lens, q_len, k)
        offs = O.chunk_offsets(lens)
        local = [r - max(o for o in offs[:-1] if o <= r) if r < offs[-1] else r for r in rows]
        x = np.asarray(x_rows, dtype=np.float64)
        seq = layers[::-1] if mistake == "layer_order" else layers
        for layer in seq:
            pos = local if mistake == "local_positions" else rows
            q, kf, vf = O.qkv_rope(x, layer["w_qkv"], pos, h_q, h_kv, base, layout)
            kx, vx = O.splice(O.rope_delta(layer["k_chunks"], base, layout, pos_base),
                              O.concat_chunks(layer["v_chunks"]), kf, vf, rows, offs[-1] + q_len)
            o = O.selective_attn(q, kx, vx, rows)
            x = (o.reshape(len(rows), -1) @ layer["w_o"].T if mistake == "no_residual"
                 else O.out_proj_residual(o, layer["w_o"], x))
        return {"rows": rows, "x": x}

    rows, got, full = _compiled_link(weights, x_chunks, x_query, 5, 1e4, "adjacent", 0, link=wrong)
    assert np.max(np.abs(got - full[rows])) > 1e-3


# ---------------------------------------------------------------------------
# HYPIC linear-layer state composition
# ---------------------------------------------------------------------------


def _delta_rule_tokens(rng, n, dk, dv):
    """Per-token transitions and writes of a gated delta rule (one of the linear
    attention families the composition covers): A_t = alpha_t (I - beta_t k k^T),
    W_t = beta_t k v^T with unit k."""
    a_list, w_list = [], []
    for _ in range(n):
        k = rng.standard_normal(dk)
        k /= np.linalg.norm(k)
        v = rng.standard_normal(dv)
        alpha, beta = rng.uniform(0.9, 1.0), rng.uniform(0.1, 0.9)
        a_list.append(alpha * (np.eye(dk) - beta * np.outer(k, k)))
        w_list.append(beta * np.outer(k, v))
    return a_list, w_list


def test_state_composition_equals_token_recurrence():
    # cached (T_C, S(C|0)) of independent segments, composed in prompt order, give the
    # state of the token-level recurrence over the whole prompt, after every segment
    rng = np.random.default_rng(41)
    dk, dv = 6, 5
    lens = [7, 1, 12, 4]
    segs = [_delta_rule_tokens(rng, n, dk, dv) for n in lens]
    summaries = [O.segment_summary(a, w, dv) for a, w in segs]
    got = O.compose_states([t for t, _ in summaries], [s for _, s in summaries])
    s = np.zeros((dk, dv))
    for j, (a, w) in enumerate(segs):
        s = O.linear_recurrence(a, w, s)
        assert np.max(np.abs(got[j] - s)) < 1e-12
    # a non-zero initial state enters through every T
    s0 = rng.standard_normal((dk, dv))
    got0 = O.compose_states([t for t, _ in summaries], [x for _, x in summaries], s0)
    a_all = [a for a, _ in segs for a in a]
    w_all = [w for _, w in segs for w in w]
    assert np.max(np.abs(got0[-1] - O.linear_recurrence(a_all, w_all, s0))) < 1e-12


def test_state_composition_special_cases_and_associativity():
    rng = np.random.default_rng(43)
    dk, dv = 4, 3
    t = [rng.standard_normal((dk, dk)) for _ in range(3)]
    s = [rng.standard_normal((dk, dv)) for _ in range(3)]
    # identity transitions: the states are running sums; one segment is its own state
    got = O.compose_states([np.eye(dk)] * 3, s)
    assert np.allclose(got, np.cumsum(np.stack(s), axis=0), atol=1e-14)
    assert np.array_equal(O.compose_states(t[:1], s[:1])[0], s[0])
    # composing (T, S) pairs is associative: merging the last two segments first
    # ((T3 T2, T3 S2 + S3)) gives the same final state
    merged = (t[2] @ t[1], t[2] @ s[1] + s[2])
    two = O.compose_states([t[0], merged[0]], [s[0], merged[1]])
    assert np.max(np.abs(two[-1] - O.compose_states(t, s)[-1])) < 1e-12


def test_planted_state_composition_mistakes_fail():
    # naive addition of zero-init states (T dropped) and a swapped segment order both
    # miss the true state by far more than any tolerance
    rng = np.random.default_rng(45)
    dk, dv = 6, 5
    segs = [_delta_rule_tokens(rng, n, dk, dv) for n in (30, 30)]
    summaries = [O.segment_summary(a, w, dv) for a, w in segs]
    want = O.linear_recurrence([a for a, _ in segs for a in a], [w for _, w in segs for w in w],
                               np.zeros((dk, dv)))
    naive = summaries[0][1] + summaries[1][1]
    assert np.max(np.abs(naive - want)) > 1e-2
    swapped = O.compose_states([summaries[1][0], summaries[0][0]], [summaries[1][1], summaries[0][1]])
    assert np.max(np.abs(swapped[-1] - want)) > 1e-2
