"""Plain CPU oracle for position-independent KV splicing (fp64, NumPy).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
GPU library never routes through this module, and this module imports nothing from
the GPU package: the two sides share no code.

Every function is the slow, obvious definition of one step of the link phase of
LegoLink / seam-window recompute, written from these pages:

* [EPIC] "EPIC: Efficient Position-Independent Caching for Serving Large Language
  Models" (Chinese walkthrough on juhe.plus): the worked 4+5+5+3 example, the
  ``link_legolink`` listing (Step 1 recompute positions, Step 2 global positions,
  Step 3 splice and attention), the method/complexity table and the Step 5 k sweep.
* [RoPE-C] 10100.com article on why RoPE breaks prefix caching: section 2.2 (RoPE
  rotates each adjacent dimension pair by an angle proportional to the position),
  section 3.2 (scheme B: cache K before RoPE, apply RoPE at the target positions on a
  hit), section 3.3 (scheme C, rotary correction by a delta rotation) and footnote 3
  (HF Llama ``inv_freq``).
* [HYPIC] joto.ai article on HYPIC: section 2.1 (linear layers: cached segment
  transition T_C and zero-init state S(C|0), composed as T(C2) S(C1) + S(C2)) and
  section 2.2 (seam window of w tokens at the head of every internal segment,
  default w = 8).
* [KV-scratch] "KV cache 从零实现：两层 Decoder、位置偏移与正确性验证": section on the
  offset causal mask (allowed[i, j] = [j <= P + i]) and the equivalence-testing
  method (fp64 re-runs, error injection).

Readings of places where the pages are silent, garbled or disagree:

1. RoPE pairs: [RoPE-C] 2.2 rotates pairs of neighbouring dimensions, so the default
   layout pairs (2i, 2i+1).  The HF Llama code cited in footnote 3 pairs (i, i+D/2);
   that layout is offered as ``layout="half"``.  Both rotate pair i by angle p*theta_i.
2. Frequencies: theta_i = base ** (-2i / D), i = 0 .. D/2-1 ([RoPE-C] footnote 3).
3. Rotation sign (the formula was lost in extraction): R(phi) = [[cos, -sin], [sin, cos]]
   acting on (x_a, x_b), so R(a) R(b) = R(a + b) and <R(m) q, R(n) k> depends on n - m
   only, as [RoPE-C] 2.2 and 3.3 state.
4. Cached K of a chunk sits at local positions pos_base .. pos_base + L - 1 (pos_base
   = 0 for plain compile, [EPIC] compile_chunk); the correction angle of chunk c is
   delta_c = off_c - pos_base.
5. Fresh Q/K of recomputed rows arrive already rotated at their global positions
   ([EPIC] Step 3: ``compute_qkv`` is called with the global positions); V never
   carries RoPE.
6. Mask: causal including self, j <= p_r ([EPIC] Step 3 listing applies a causal mask;
   [KV-scratch] offset mask).  The worked example's looser wording (the seven rows
   see all 17 positions) is read as: all keys that exist, filtered by that mask.
7. Scale 1/sqrt(D); no bias, soft-cap or dropout.
8. GQA: query head h reads KV head h // (Hq / Hkv) (contiguous groups).
9. Every recomputed row produces an output (seam outputs feed the next layer in the
   per-layer loop); the query rows are the last q of them.
10. Zero-length chunks are legal and contribute nothing; q = 0 is legal.
11. The layer of the multi-layer link is compute_qkv (projection, RoPE at the global
    positions) -> splice -> attention -> x + O W_o^T; the pages do not show the rest of
    a transformer block, and per-row maps after the attention would not change which
    rows are recomputed or how they are spliced.
"""

import math

import numpy as np

# ---------------------------------------------------------------------------
# Step 1 / Step 2 of [EPIC] link_legolink: offsets and recompute positions.
# ---------------------------------------------------------------------------


def chunk_offsets(chunk_lens):
    """Global start of every chunk, plus the total context length at the end.

    [EPIC] Step 1 walk-through: the running ``offset`` goes 0 -> 4 -> 9 -> 14 for
    chunks of 4, 5, 5 tokens, and total_ctx_len is the last value.
    """
    offs = [0]
    for length in chunk_lens:
        offs.append(offs[-1] + int(length))
    return offs


def recompute_positions(chunk_lens, q_len, k):
    """LegoLink-k recompute set, in ascending order.

    The rule ([EPIC] Step 1 and the worked 4+5+5+3 example; [HYPIC] 2.2 with k = w):
    a position j of the spliced prompt is recomputed exactly when it is a query
    position (j >= ctx), or when it lies in a chunk other than the first and is one of
    that chunk's first k tokens (j - off_c < k).  Positions are visited one by one;
    the chunk holding j is tracked as j advances (empty chunks hold no position).
    """
    offs = chunk_offsets(chunk_lens)
    ctx = offs[-1]
    k = int(k)
    out = []
    c = 0
    for j in range(ctx + int(q_len)):
        if j >= ctx:
            out.append(j)
            continue
        while j >= offs[c + 1]:
            c += 1
        if c >= 1 and j - offs[c] < k:
            out.append(j)
    return out


# ---------------------------------------------------------------------------
# RoPE definition ([RoPE-C] 2.2 and footnote 3).
# ---------------------------------------------------------------------------


def rope_theta(head_dim, base):
    """theta_i = base ** (-2 i / D) for i = 0 .. D/2 - 1, in fp64."""
    assert head_dim % 2 == 0
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / np.float64(head_dim))


def rope_pair_index(head_dim, layout="adjacent"):
    """Dimension indices (a_i, b_i) of pair i.

    "adjacent": (2i, 2i+1) -- the wording of [RoPE-C] 2.2.
    "half":     (i, i+D/2) -- the HF Llama layout referenced in footnote 3.
    """
    half = head_dim // 2
    i = np.arange(half)
    if layout == "adjacent":
        return 2 * i, 2 * i + 1
    if layout == "half":
        return i, i + half
    raise ValueError("unknown layout %r" % (layout,))


def rope_rotate(x, positions, base, layout="adjacent"):
    """Rotate every pair of every row of ``x`` by angle positions[t] * theta_i.

    x: [T, H, D] (any float dtype; computed in fp64).  positions: [T] integers
    (may be negative: rotating by -p undoes rotating by p).  Returns a new fp64 array.
    Pair (a, b) maps to (a cos phi - b sin phi, a sin phi + b cos phi).
    """
    x = np.asarray(x, dtype=np.float64)
    t_count, _, head_dim = x.shape
    theta = rope_theta(head_dim, base)
    ia, ib = rope_pair_index(head_dim, layout)
    pos = np.asarray(positions, dtype=np.float64).reshape(t_count, 1)
    phi = pos * theta[None, :]  # [T, D/2], fp64 angle
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    a = x[:, :, ia]
    b = x[:, :, ib]
    out = np.empty_like(x)
    out[:, :, ia] = a * c - b * s
    out[:, :, ib] = a * s + b * c
    return out


# ---------------------------------------------------------------------------
# Scheme C rotary correction ([RoPE-C] 3.3): cached K moved from local to global.
# ---------------------------------------------------------------------------


def rope_delta(cached_k_chunks, base, layout="adjacent", pos_base=0):
    """Concatenate the cached K of every chunk, each rotated by R(delta_c).

    cached_k_chunks: list of [L_c, Hkv, D] arrays whose rows carry RoPE at local
    positions pos_base .. pos_base + L_c - 1.  delta_c = off_c - pos_base, one
    direct rotation per row (not two stacked ones).  Returns [ctx, Hkv, D] fp64.
    """
    lens = [int(np.asarray(a).shape[0]) for a in cached_k_chunks]
    offs = chunk_offsets(lens)
    parts = []
    for c, kc in enumerate(cached_k_chunks):
        kc = np.asarray(kc, dtype=np.float64)
        delta = offs[c] - int(pos_base)
        parts.append(rope_rotate(kc, np.full(kc.shape[0], delta), base, layout))
    if not parts:
        raise ValueError("at least one chunk is required")
    return np.concatenate(parts, axis=0)


def rope_apply(nope_k_chunks, base, layout="adjacent"):
    """Scheme B ([RoPE-C] 3.2): concatenate the position-free ("nope") cached K of every
    chunk and apply RoPE at the global positions off_c + t.  Returns [ctx, Hkv, D] fp64.
    """
    lens = [int(np.asarray(a).shape[0]) for a in nope_k_chunks]
    if not lens:
        raise ValueError("at least one chunk is required")
    x = np.concatenate([np.asarray(a, dtype=np.float64) for a in nope_k_chunks], axis=0)
    return rope_rotate(x, np.arange(x.shape[0]), base, layout)


def concat_chunks(chunks):
    """Plain concatenation along tokens (V carries no RoPE, [RoPE-C] 3.2/3.3)."""
    return np.concatenate([np.asarray(a, dtype=np.float64) for a in chunks], axis=0)


# ---------------------------------------------------------------------------
# Step 3 of [EPIC]: splice and selective attention.
# ---------------------------------------------------------------------------


def splice(k_ctx, v_ctx, k_fresh, v_fresh, rows, n_total):
    """Build the full-length spliced K/V ([EPIC] Step 3: K_exp, V_exp).

    Rows 0..ctx-1 start as the (corrected) cached rows; rows ctx..N-1 do not exist
    in the cache and are filled only by fresh rows.  Then K_exp[rows] = K_new and
    V_exp[rows] = V_new.  Rows that no fresh row covers stay NaN so a missing
    overwrite cannot pass unnoticed.
    """
    k_ctx = np.asarray(k_ctx, dtype=np.float64)
    v_ctx = np.asarray(v_ctx, dtype=np.float64)
    ctx = k_ctx.shape[0]
    shape = (n_total,) + k_ctx.shape[1:]
    kx = np.full(shape, np.nan)
    vx = np.full(shape, np.nan)
    kx[:ctx] = k_ctx
    vx[:ctx] = v_ctx
    rows = np.asarray(rows, dtype=np.int64)
    kx[rows] = np.asarray(k_fresh, dtype=np.float64)
    vx[rows] = np.asarray(v_fresh, dtype=np.float64)
    return kx, vx


def contiguous_runs(rows):
    """Split an ascending position list into runs of consecutive positions.

    Returns (first_position, first_row_index, length) triples.
    """
    runs = []
    r = 0
    rows = list(rows)
    while r < len(rows):
        s = r
        while r + 1 < len(rows) and rows[r + 1] == rows[r] + 1:
            r += 1
        runs.append((rows[s], s, r - s + 1))
        r += 1
    return runs


def offset_mask(past_len, new_len):
    """allowed[i, j] = [j <= P + i] over keys 0 .. P + C - 1 ([KV-scratch] mask)."""
    qpos = past_len + np.arange(new_len)
    kpos = np.arange(past_len + new_len)
    return kpos[None, :] <= qpos[:, None]


def _softmax_rows(scores):
    m = np.max(scores, axis=-1, keepdims=True)
    e = np.exp(scores - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def selective_attn(q, kx, vx, rows, scale=None):
    """Causal attention of the recomputed rows over the spliced K/V.

    q: [R, Hq, D] (row r at global position rows[r]); kx, vx: [N, Hkv, D].
    For each query head h (KV head h // G) and each contiguous run of rows starting
    at position P: scores = Q K^T * scale over keys 0 .. P+m-1, masked with the
    offset mask, softmax, times V ([EPIC] Step 3; [KV-scratch] offset mask).
    Returns O: [R, Hq, D] fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    kx = np.asarray(kx, dtype=np.float64)
    vx = np.asarray(vx, dtype=np.float64)
    n_rows, hq, head_dim = q.shape
    hkv = kx.shape[1]
    assert hq % hkv == 0
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    out = np.zeros((n_rows, hq, head_dim))
    for start_pos, first_row, m in contiguous_runs(rows):
        allowed = offset_mask(start_pos, m)
        n_keys = start_pos + m
        for h in range(hq):
            g = h // group
            qr = q[first_row:first_row + m, h, :]
            kk = kx[:n_keys, g, :]
            vv = vx[:n_keys, g, :]
            scores = (qr @ kk.T) * scale
            scores = np.where(allowed, scores, -np.inf)
            out[first_row:first_row + m, h, :] = _softmax_rows(scores) @ vv
    return out


def full_causal_attn(q_all, k_all, v_all, scale=None):
    """Brute force: dense causal attention over every position (tiny inputs only).

    q_all: [N, Hq, D]; k_all, v_all: [N, Hkv, D].  Builds the explicit N x N mask
    j <= i for each head independently of ``selective_attn``.
    """
    q_all = np.asarray(q_all, dtype=np.float64)
    k_all = np.asarray(k_all, dtype=np.float64)
    v_all = np.asarray(v_all, dtype=np.float64)
    n_total, hq, head_dim = q_all.shape
    hkv = k_all.shape[1]
    group = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    out = np.zeros_like(q_all)
    for h in range(hq):
        g = h // group
        for i in range(n_total):
            s = np.array([np.dot(q_all[i, h], k_all[j, g]) * scale for j in range(i + 1)])
            w = np.exp(s - s.max())
            w = w / w.sum()
            acc = np.zeros(head_dim)
            for j in range(i + 1):
                acc += w[j] * v_all[j, g]
            out[i, h] = acc
    return out


def attn_rows_direct(q_rows, kx, vx, positions, heads, scale=None):
    """Attention output of selected (row, head) pairs, one at a time.

    Used for sampled parity at full size: q_rows[s] is the query vector [D] of
    sample s at global position positions[s] for query head heads[s]; kx/vx carry
    all group heads.  Same definition as ``selective_attn``.
    """
    kx = np.asarray(kx, dtype=np.float64)
    vx = np.asarray(vx, dtype=np.float64)
    head_dim = kx.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    out = []
    for qv, p, g in zip(q_rows, positions, heads):
        kk = kx[: int(p) + 1, int(g), :]
        vv = vx[: int(p) + 1, int(g), :]
        s = (kk @ np.asarray(qv, dtype=np.float64)) * scale
        w = np.exp(s - s.max())
        w = w / w.sum()
        out.append(w @ vv)
    return np.stack(out)


# ---------------------------------------------------------------------------
# Composition of one request ([EPIC] link_legolink, one layer).
# ---------------------------------------------------------------------------


def decode_attn(q_new, kx, vx, k_new, v_new, scale=None):
    """One decode step after the link: the next token, at position N right after the N
    spliced keys, attends over keys 0..N including itself ([KV-scratch] incremental
    decode with the offset mask for a single new row, P = N).  q_new: [Hq, D];
    k_new/v_new: [Hkv, D] (RoPE'd at N).  Returns [Hq, D] fp64."""
    kx = np.asarray(kx, dtype=np.float64)
    vx = np.asarray(vx, dtype=np.float64)
    n = kx.shape[0]
    kx2 = np.concatenate([kx, np.asarray(k_new, dtype=np.float64)[None]], axis=0)
    vx2 = np.concatenate([vx, np.asarray(v_new, dtype=np.float64)[None]], axis=0)
    return selective_attn(np.asarray(q_new, dtype=np.float64)[None], kx2, vx2, [n], scale)[0]


def link_request(cached_k_chunks, cached_v_chunks, q_len, k, k_fresh, v_fresh, q_fresh,
                 base, layout="adjacent", pos_base=0, scale=None):
    """Run the whole link for one request and one layer.

    Returns dict(rows, offsets, kx, vx, out).  k_fresh/v_fresh/q_fresh are in the
    order of ``rows`` (ascending positions).
    """
    lens = [int(np.asarray(a).shape[0]) for a in cached_k_chunks]
    offs = chunk_offsets(lens)
    rows = recompute_positions(lens, q_len, k)
    n_total = offs[-1] + int(q_len)
    k_ctx = rope_delta(cached_k_chunks, base, layout, pos_base)
    v_ctx = concat_chunks(cached_v_chunks)
    kx, vx = splice(k_ctx, v_ctx, k_fresh, v_fresh, rows, n_total)
    out = selective_attn(q_fresh, kx, vx, rows, scale)
    return {"rows": rows, "offsets": offs, "kx": kx, "vx": vx, "out": out}


# ---------------------------------------------------------------------------
# The layer loop of the link ([EPIC] Step 3 runs over the model's layers): per layer
# the recomputed rows' Q/K/V come from their hidden states with RoPE at the global
# positions (compute_qkv), are spliced and attend, and the attention output carries
# the rows' hidden states to the next layer.  The pages show only compute_qkv, the
# splice and the attention of a layer; the layer here is the plainest block that
# closes the loop: x <- x + O W_o^T (output projection plus residual), with the
# projections in the nn.Linear layout (weight rows are output features).
# ---------------------------------------------------------------------------


def qkv_rope(x, w_qkv, positions, h_q, h_kv, base, layout="adjacent"):
    """compute_qkv of [EPIC] Step 3: y = x W^T, split into Q (h_q heads), K and V (h_kv
    heads each), Q and K rotated at ``positions`` (the global positions), V not.

    x: [T, d_model]; w_qkv: [(h_q + 2 h_kv) * D, d_model].  Returns fp64
    q [T, h_q, D], k [T, h_kv, D], v [T, h_kv, D].
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_qkv, dtype=np.float64)
    n_out = w.shape[0]
    assert n_out % (h_q + 2 * h_kv) == 0
    head_dim = n_out // (h_q + 2 * h_kv)
    y = x @ w.T
    t_count = x.shape[0]
    q = y[:, :h_q * head_dim].reshape(t_count, h_q, head_dim)
    k = y[:, h_q * head_dim:(h_q + h_kv) * head_dim].reshape(t_count, h_kv, head_dim)
    v = y[:, (h_q + h_kv) * head_dim:].reshape(t_count, h_kv, head_dim)
    return rope_rotate(q, positions, base, layout), rope_rotate(k, positions, base, layout), v


def out_proj_residual(o, w_o, x):
    """Next hidden state of the rows: x + O W_o^T, O [T, h_q, D] read as [T, h_q * D];
    w_o: [d_model, h_q * D].  Returns [T, d_model] fp64."""
    o = np.asarray(o, dtype=np.float64)
    o2 = o.reshape(o.shape[0], -1)
    return np.asarray(x, dtype=np.float64) + o2 @ np.asarray(w_o, dtype=np.float64).T


def link_layers(x_rows, layers, q_len, k, h_q, h_kv, base, layout="adjacent", pos_base=0,
                scale=None):
    """The whole link of one request over several layers.

    x_rows: [R, d_model] hidden states of the recomputed rows (ascending positions)
    entering layer 0.  layers: one dict per layer with ``w_qkv``, ``w_o`` and the
    request's cached chunks ``k_chunks`` (K with RoPE at local positions pos_base..)
    and ``v_chunks``.  Per layer: compute_qkv at the global positions, rotate the
    cached K by delta_c, splice, selective attention, output projection + residual.
    Returns dict(rows, x) with the rows' hidden states after the last layer.
    """
    lens = [int(np.asarray(a).shape[0]) for a in layers[0]["k_chunks"]]
    rows = recompute_positions(lens, q_len, k)
    n_total = sum(lens) + int(q_len)
    x = np.asarray(x_rows, dtype=np.float64)
    for layer in layers:
        q, kf, vf = qkv_rope(x, layer["w_qkv"], rows, h_q, h_kv, base, layout)
        if lens:
            k_ctx = rope_delta(layer["k_chunks"], base, layout, pos_base)
            v_ctx = concat_chunks(layer["v_chunks"])
        else:
            k_ctx = np.zeros((0,) + kf.shape[1:])
            v_ctx = np.zeros((0,) + vf.shape[1:])
        kx, vx = splice(k_ctx, v_ctx, kf, vf, rows, n_total)
        o = selective_attn(q, kx, vx, rows, scale)
        x = out_proj_residual(o, layer["w_o"], x)
    return {"rows": rows, "x": x}


def prefill_layers(x_seq, weights, positions, h_q, h_kv, base, layout="adjacent", scale=None):
    """Dense causal prefill of a token sequence through the same layers, written apart
    from the link: every row is computed, with one explicit N x N causal mask.

    x_seq: [N, d_model] layer-0 hidden states; weights: list of (w_qkv, w_o);
    positions: [N] RoPE positions of the rows.  Run on one chunk at its local
    positions it is [EPIC] compile_chunk (returns the per-layer cached K, V); run on
    the whole spliced sequence at 0..N-1 it is full recompute.  Returns
    dict(x=[N, d_model], k=[per layer [N, h_kv, D]], v=[...]).
    """
    x = np.asarray(x_seq, dtype=np.float64)
    n = x.shape[0]
    ks, vs = [], []
    for w_qkv, w_o in weights:
        w_qkv = np.asarray(w_qkv, dtype=np.float64)
        head_dim = w_qkv.shape[0] // (h_q + 2 * h_kv)
        y = x @ w_qkv.T
        q = rope_rotate(y[:, :h_q * head_dim].reshape(n, h_q, head_dim), positions, base, layout)
        kk = rope_rotate(y[:, h_q * head_dim:(h_q + h_kv) * head_dim].reshape(n, h_kv, head_dim),
                         positions, base, layout)
        vv = y[:, (h_q + h_kv) * head_dim:].reshape(n, h_kv, head_dim)
        ks.append(kk)
        vs.append(vv)
        sc = (1.0 / math.sqrt(head_dim)) if scale is None else scale
        causal = np.tril(np.ones((n, n), dtype=bool))
        o = np.zeros((n, h_q, head_dim))
        for h in range(h_q):
            g = h // (h_q // h_kv)
            s = np.where(causal, (q[:, h, :] @ kk[:, g, :].T) * sc, -np.inf)
            s = np.exp(s - s.max(axis=1, keepdims=True))
            o[:, h, :] = (s / s.sum(axis=1, keepdims=True)) @ vv[:, g, :]
        x = x + o.reshape(n, h_q * head_dim) @ np.asarray(w_o, dtype=np.float64).T
    return {"x": x, "k": ks, "v": vs}


# ---------------------------------------------------------------------------
# Linear-attention layers of a hybrid model ([HYPIC] 2.1): a layer keeps one state
# matrix per head, S_t = A_t S_{t-1} + W_t (A_t the token's transition, W_t its write,
# e.g. beta_t k_t v_t^T).  A segment C is cached as its cumulative transition
# T_C = A_L ... A_1 and its zero-init final state S(C|0); after any prefix the state
# is S(prefix . C) = T_C S(prefix) + S(C|0).
# ---------------------------------------------------------------------------


def linear_recurrence(a_list, w_list, s0):
    """Token-level recurrence S_t = A_t S_{t-1} + W_t from S_0 = s0; returns S_N (fp64).
    a_list: [N][dk, dk]; w_list: [N][dk, dv]."""
    s = np.array(s0, dtype=np.float64)
    for a, w in zip(a_list, w_list):
        s = np.asarray(a, dtype=np.float64) @ s + np.asarray(w, dtype=np.float64)
    return s


def segment_summary(a_list, w_list, dv):
    """(T_C, S(C|0)) of one segment: T_C = A_L ... A_1 (the latest transition on the
    left) and the recurrence run from a zero state."""
    dk = np.asarray(a_list[0]).shape[0] if len(a_list) else None
    if dk is None:
        raise ValueError("a segment needs at least one token")
    t = np.eye(dk)
    for a in a_list:
        t = np.asarray(a, dtype=np.float64) @ t
    return t, linear_recurrence(a_list, w_list, np.zeros((dk, dv)))


def compose_states(t_list, s_list, s0=None):
    """States after each segment of a request: S_j = T_j S_{j-1} + S_j(0), S_{-1} = s0
    (zero when None).  t_list: [m][dk, dk]; s_list: [m][dk, dv].  Returns [m, dk, dv]."""
    out = []
    s = None if s0 is None else np.asarray(s0, dtype=np.float64)
    for t, s_seg in zip(t_list, s_list):
        s_seg = np.asarray(s_seg, dtype=np.float64)
        s = s_seg.copy() if s is None else np.asarray(t, dtype=np.float64) @ s + s_seg
        out.append(s)
    return np.stack(out) if out else np.zeros((0,) + np.asarray(s_list).shape[1:])


# ---------------------------------------------------------------------------
# Shared-chunk pool (paged storage): gather one chunk back to contiguous rows.
# ---------------------------------------------------------------------------


def gather_paged_chunk(pool, block_ids, length):
    """Rows 0..length-1 of a chunk stored in fixed-size pool blocks.

    pool: [n_blocks, block_size, H, D]; block_ids: the chunk's blocks in order.
    Token t lives in block block_ids[t // block_size], slot t % block_size.
    """
    pool = np.asarray(pool)
    bs = pool.shape[1]
    rows = [pool[int(block_ids[t // bs]), t % bs] for t in range(int(length))]
    if not rows:
        return np.zeros((0,) + pool.shape[2:], dtype=np.float64)
    return np.stack(rows).astype(np.float64)
