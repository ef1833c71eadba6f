"""Seeded synthetic workloads for position-independent KV splicing.

This module only draws random numbers and chunk lengths.  It holds none of the
method's arithmetic (no offsets, recompute sets, rotations or attention), so both
the GPU path and the CPU oracle can take their inputs from it without sharing any
of the computation.

The shapes follow the pages' workloads: RAG prompts assembled from independently
cached documents plus a user query (EPIC walkthrough, worked example and Step 5;
HYPIC section 2.2: segments usually longer than 512 tokens, seam window w = 8;
prompts of tens to hundreds of segments reaching ~100k tokens).  No dataset is
used: values are N(0, 1) draws (optionally scaled) rounded to the I/O dtype with
round-to-nearest-even.

Recipe (all draws use ``torch.Generator`` on the CPU, Mersenne Twister, seeded):
  * chunk lengths: ``numpy.random.default_rng(seed)`` integers, inclusive bounds;
  * tensors: ``torch.randn(float32) * scale`` then ``.to(dtype)`` (RNE for bf16);
  * the size-limit request's 2 GiB K/V buffers: the same on the GPU with torch's
    seeded device generator (``device_context_tensors``).
"""

from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class Request:
    chunk_lens: list
    q_len: int
    chunk_ids: list = None  # pool chunk id per chunk (paged workloads only)


@dataclass
class Workload:
    name: str
    dtype: str
    h_q: int
    h_kv: int
    head_dim: int
    rope_base: float
    k: int
    requests: list
    value_scale: float = 1.0
    seed: int = 0
    # paged shared-chunk pool (None for contiguous workloads)
    pool_lens: list = None
    block_size: int = 16
    pool_block_perm_seed: int = None
    extra: dict = field(default_factory=dict)

    @property
    def n_tokens(self):
        return sum(sum(r.chunk_lens) + r.q_len for r in self.requests)

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]


def _lengths_until(rng, lo, hi, target):
    lens = []
    while sum(lens) < target:
        lens.append(int(rng.integers(lo, hi + 1)))
    return lens


def worked_example(seed=1):
    """4+5+5 token chunks plus a 3-token query, k = 2, fp32, 4 heads of 16 dims."""
    return Workload("worked_example", "f32", 4, 4, 16, 10000.0, 2,
                    [Request([4, 5, 5], 3)], seed=seed)


def rag_single(seed=2):
    """One RAG request: 5 chunks of 1024 tokens + 64 query tokens, GQA 32/8, k = 16."""
    return Workload("rag_single", "bf16", 32, 8, 128, 500000.0, 16,
                    [Request([1024] * 5, 64)], value_scale=1.0 / np.sqrt(128.0), seed=seed)


def long_context(k=16, seed=3):
    """Batch 1: 32 chunks of 1024 tokens + 128 query tokens (32896 tokens)."""
    return Workload("long_context", "bf16", 32, 8, 128, 500000.0, k,
                    [Request([1024] * 32, 128)], seed=seed * 1000 + k)


def epic_sweep(k=16, n_req=4, seed=4):
    """4 independent requests of ~50k tokens; chunk lengths uniform in [512, 2048]."""
    rng = np.random.default_rng(seed * 1000 + k)
    reqs = [Request(_lengths_until(rng, 512, 2048, 50000), 256) for _ in range(n_req)]
    return Workload("epic_sweep", "bf16", 32, 8, 128, 500000.0, k, reqs, seed=seed * 1000 + k)


def shared_pool(n_pool=256, n_req=8, m_lo=96, m_hi=128, q_len=128, w=8, seed=5):
    """Paged shared-chunk pool: 256 chunks (lengths in [512, 1536]) stored once in
    16-token blocks; 8 requests each splice 96-128 distinct pool chunks in random
    order plus 128 query tokens; seam window w = 8; GQA 32/4."""
    rng = np.random.default_rng(seed)
    pool_lens = [int(x) for x in rng.integers(512, 1537, size=n_pool)]
    reqs = []
    for _ in range(n_req):
        m = int(rng.integers(m_lo, m_hi + 1))
        ids = [int(x) for x in rng.permutation(n_pool)[:m]]
        reqs.append(Request([pool_lens[i] for i in ids], q_len, chunk_ids=ids))
    return Workload("shared_pool", "bf16", 32, 4, 128, 500000.0, w, reqs,
                    pool_lens=pool_lens, block_size=16, pool_block_perm_seed=seed + 7,
                    seed=seed)


def single_huge(n_tokens, q_len=64, chunk=65536, k=2, seed=6):
    """One request of exactly ``n_tokens`` tokens (``q_len`` query tokens, the context
    in chunks of ``chunk`` tokens, the last one shorter), GQA 32/8, D = 128, bf16: the
    size-limit case.  Its K/V come from ``device_context_tensors``."""
    ctx = n_tokens - q_len
    lens = [chunk] * (ctx // chunk) + ([ctx % chunk] if ctx % chunk else [])
    return Workload("single_huge", "bf16", 32, 8, 128, 500000.0, k, [Request(lens, q_len)],
                    seed=seed)


def pool_block_table(wl):
    """Physical block ids of every pool chunk, in a shuffled physical order.

    Chunk i needs ceil(L_i / block_size) blocks; the physical ids are a seeded
    permutation of 0 .. n_blocks-1 so a gather is a real gather.  Returns
    (chunk_block_ptr [n_pool + 1], blocks [n_blocks]) as int32 arrays.
    """
    bs = wl.block_size
    counts = [(L + bs - 1) // bs for L in wl.pool_lens]
    ptr = np.zeros(len(counts) + 1, dtype=np.int64)
    ptr[1:] = np.cumsum(counts)
    n_blocks = int(ptr[-1])
    perm = np.random.default_rng(wl.pool_block_perm_seed).permutation(n_blocks)
    return ptr.astype(np.int32), perm.astype(np.int32)


def draw(shape, seed, dtype, scale=1.0):
    """N(0, 1) * scale rounded to ``dtype`` (a torch dtype); CPU tensor."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    x = torch.randn(tuple(int(s) for s in shape), generator=g, dtype=torch.float32)
    if scale != 1.0:
        x = x * float(scale)
    return x.to(dtype)


def context_tensors(wl):
    """Cached K/V buffers for a contiguous workload.

    Returns (k_buf, v_buf), each [n_tokens, Hkv, D] in the workload's dtype.  Request
    b's rows start where request b-1's end; within a request the chunks' cached rows
    come first in chunk order (each carrying RoPE at its own local positions, as the
    compile step leaves it), followed by q rows that only the splice fills.
    """
    shape = (wl.n_tokens, wl.h_kv, wl.head_dim)
    k_buf = draw(shape, wl.seed * 7 + 1, wl.torch_dtype, wl.value_scale)
    v_buf = draw(shape, wl.seed * 7 + 2, wl.torch_dtype, wl.value_scale)
    return k_buf, v_buf


def device_draw(shape, seed, dtype, device, scale=1.0):
    """N(0, 1) * scale rounded to ``dtype``, drawn on ``device`` with torch's seeded
    device generator (Philox): for buffers whose host draw would take minutes (slices
    are copied to the host for the oracle)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(int(s) for s in shape), generator=g, device=device,
                    dtype=torch.float32)
    if scale != 1.0:
        x.mul_(float(scale))
    return x.to(dtype)


def device_context_tensors(wl, device):
    """``context_tensors`` drawn on ``device`` (``device_draw``)."""
    shape = (wl.n_tokens, wl.h_kv, wl.head_dim)
    return tuple(device_draw(shape, wl.seed * 7 + j, wl.torch_dtype, device, wl.value_scale)
                 for j in (1, 2))


def fresh_tensors(wl, n_rows):
    """Fresh Q/K/V of the recomputed rows: Q [n_rows, Hq, D], K/V [n_rows, Hkv, D].

    ``n_rows`` is supplied by the caller (each side derives it from its own index)."""
    q = draw((n_rows, wl.h_q, wl.head_dim), wl.seed * 7 + 3, wl.torch_dtype, wl.value_scale)
    kf = draw((n_rows, wl.h_kv, wl.head_dim), wl.seed * 7 + 4, wl.torch_dtype, wl.value_scale)
    vf = draw((n_rows, wl.h_kv, wl.head_dim), wl.seed * 7 + 5, wl.torch_dtype, wl.value_scale)
    return q, kf, vf


def pool_tensors(wl):
    """Paged pool K/V: [n_blocks, block_size, Hkv, D] each."""
    bs = wl.block_size
    n_blocks = sum((L + bs - 1) // bs for L in wl.pool_lens)
    shape = (n_blocks, bs, wl.h_kv, wl.head_dim)
    return (draw(shape, wl.seed * 7 + 1, wl.torch_dtype, wl.value_scale),
            draw(shape, wl.seed * 7 + 2, wl.torch_dtype, wl.value_scale))


def decode_tensors(wl):
    """The next token of every request (decode step): Q [n_req, Hq, D], K/V
    [n_req, Hkv, D]."""
    n = len(wl.requests)
    return (draw((n, wl.h_q, wl.head_dim), wl.seed * 7 + 6, wl.torch_dtype, wl.value_scale),
            draw((n, wl.h_kv, wl.head_dim), wl.seed * 7 + 7, wl.torch_dtype, wl.value_scale),
            draw((n, wl.h_kv, wl.head_dim), wl.seed * 7 + 8, wl.torch_dtype, wl.value_scale))


def link_tensors(wl, n_layers, d_model, n_rows):
    """A random model for the multi-layer link (no trained weights exist here).

    Returns (x0, w_qkv, w_o, k_cache, v_cache): x0 [n_rows, d_model] layer-0 hidden
    states of the recomputed rows (N(0, 1)); per layer w_qkv [(Hq + 2 Hkv) D, d_model]
    and w_o [d_model, Hq D] (nn.Linear layout, N(0, 1/fan_in) so activations stay
    O(1)), and the cached K/V buffers [n_tokens, Hkv, D] as context_tensors lays
    them out.  ``n_rows`` is supplied by the caller."""
    hq, hkv, d = wl.h_q, wl.h_kv, wl.head_dim
    base = wl.seed * 7 + 100
    x0 = draw((n_rows, d_model), base, wl.torch_dtype)
    w_qkv, w_o, kc, vc = [], [], [], []
    shape = (wl.n_tokens, hkv, d)
    for l in range(n_layers):
        s = base + 10 * (l + 1)
        w_qkv.append(draw(((hq + 2 * hkv) * d, d_model), s, wl.torch_dtype, 1.0 / np.sqrt(d_model)))
        w_o.append(draw((d_model, hq * d), s + 1, wl.torch_dtype, 1.0 / np.sqrt(hq * d)))
        kc.append(draw(shape, s + 2, wl.torch_dtype, wl.value_scale))
        vc.append(draw(shape, s + 3, wl.torch_dtype, wl.value_scale))
    return x0, w_qkv, w_o, kc, vc


def state_pool_tensors(wl, n_heads, d=128, decay=0.9, noise=0.1, s_scale=0.1):
    """Cached linear-layer summaries of every pool chunk (no trained model exists here):
    T [n_pool, H, d, d] = decay * (I + noise * G / sqrt(d)) with G ~ N(0, 1), a
    contraction like a product of decaying token transitions, and S(C|0) [n_pool, H, d, d]
    ~ N(0, s_scale^2), so composed states stay O(1).  fp32 CPU tensors."""
    import torch
    n_pool = len(wl.pool_lens)
    g = draw((n_pool, n_heads, d, d), wl.seed * 7 + 200, torch.float32, noise / np.sqrt(d))
    t = decay * (g + torch.eye(d, dtype=torch.float32))
    sz = draw((n_pool, n_heads, d, d), wl.seed * 7 + 201, torch.float32, s_scale)
    return t, sz


CONFIGS = {
    "worked_example": worked_example,
    "rag_single": rag_single,
    "long_context": long_context,
    "epic_sweep": epic_sweep,
    "shared_pool": shared_pool,
}
