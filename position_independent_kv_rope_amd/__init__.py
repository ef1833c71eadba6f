"""Position-independent KV splicing on MI355X: thin Python binding of libpic.so.

The functions below carry the names of the C entry points in ``include/pic.h`` and
only marshal arguments: every step of the path runs in the HIP library.  PyTorch
supplies device memory and the current stream.  There is no fallback: if libpic.so
is missing or a call fails, a ``PicError`` is raised.
"""

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpic.so")

PIC_OK, PIC_EINVAL, PIC_ENOSPC, PIC_EUNSUPPORTED, PIC_EDEVICE = 0, -1, -2, -3, -4
PIC_F32, PIC_BF16 = 0, 1
PIC_ROPE_ADJACENT, PIC_ROPE_HALF = 0, 1
PIC_ROPE_BY_DELTA, PIC_ROPE_AT_POSITION = 0, 1
PIC_PLAN_MAGIC = 0x31434950
PIC_ATTN_TILE_M = 128

# header word indices (include/pic.h)
(H_MAGIC, H_WORDS, H_N_REQ, H_N_CHUNKS, H_N_ROWS, H_N_TOKENS, H_K, H_POS_BASE, H_H_Q, H_H_KV,
 H_TILE_ROWS, H_N_ROPE_TILES, H_N_ATTN_TILES, H_N_ATTN_ITEMS, H_N_MERGE, H_N_PARTIALS,
 H_MAX_TOKENS, H_O_REQ_CHUNK_PTR, H_O_CHUNK_OFF, H_O_REQ_TOK_PTR, H_O_REQ_ROW_PTR, H_O_ROWS,
 H_O_ROW_TOK, H_O_ROPE_TILES, H_O_ATTN_TILES, H_O_ATTN_ITEMS, H_O_MERGE, H_PAGED, H_O_SEGS,
 H_N_KBLOCKS, H_O_KBLOCKS, H_N_DEC_ITEMS, H_O_DEC_ITEMS, H_N_DEC_USES, H_O_DEC_USES,
 H_N_DEC_RECS, H_O_DEC_REC_PTR, H_N_DEC_PIECES, H_O_DEC_PIECES, H_O_DEC_PIECE_RECS,
 H_N_DEC_WG, H_O_DEC_WG_PTR) = range(42)
PIC_DECODE_COLS = 64
PIC_DECODE_BLOCK = 32
PIC_DECODE_WG_PER_CU = 4

EXPORTED = ("pic_build_index", "pic_rope_delta", "pic_rope_apply", "pic_splice",
            "pic_rope_splice", "pic_rope_splice_pool",
            "pic_attn_workspace_bytes",
            "pic_selective_attn", "pic_selective_attn_noalloc", "pic_selective_attn_paged",
            "pic_decode_workspace_bytes",
            "pic_decode_attn_paged", "pic_qkv_workspace_bytes", "pic_qkv_rope",
            "pic_out_proj", "pic_link_workspace_bytes", "pic_link", "pic_state_compose",
            "pic_strerror")


class PicError(RuntimeError):
    def __init__(self, fn, status):
        msg = "%s failed: %d (%s)" % (fn, status, strerror(status) if _lib else "?")
        super().__init__(msg)
        self.status = status


_lib = None
_NO_CHUNKS = ctypes.c_int32(0)


def lib():
    """Load libpic.so (built in-tree by build.py); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libpic.so not found at %s; build it with "
                           "`python -m position_independent_kv_rope_amd.build`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, p, f32, f64, sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_float, ctypes.c_double, ctypes.c_size_t)
    L.pic_build_index.argtypes = [i32, p, p, p, p, i32, i32, i32, i32, i32, p, i64,
                                  ctypes.POINTER(i64)]
    L.pic_build_index.restype = ctypes.c_int
    L.pic_rope_delta.argtypes = [p, p, p, i32, i32, i32, f64, p]
    L.pic_rope_delta.restype = ctypes.c_int
    L.pic_rope_apply.argtypes = [p, p, p, i32, i32, i32, f64, p]
    L.pic_rope_apply.restype = ctypes.c_int
    L.pic_splice.argtypes = [p, p, p, p, p, p, i32, i32, p]
    L.pic_splice.restype = ctypes.c_int
    L.pic_rope_splice.argtypes = [p, p, p, p, p, p, i32, i32, i32, f64, i32, p]
    L.pic_rope_splice.restype = ctypes.c_int
    L.pic_rope_splice_pool.argtypes = [p, p, p, p, i64, i32, p, i32, p, p, p, p, p, i32, i32, i32,
                                       f64, p]
    L.pic_rope_splice_pool.restype = ctypes.c_int
    L.pic_attn_workspace_bytes.argtypes = [p, i32]
    L.pic_attn_workspace_bytes.restype = sz
    L.pic_selective_attn.argtypes = [p, p, p, p, p, p, i32, i32, f32, p, sz, p]
    L.pic_selective_attn.restype = ctypes.c_int
    L.pic_selective_attn_noalloc.argtypes = [p, p, p, p, p, p, i32, i32, f32, p]
    L.pic_selective_attn_noalloc.restype = ctypes.c_int
    L.pic_selective_attn_paged.argtypes = [p, p, p, p, p, i64, i32, p, i32, p, p, p, p, i32, i32,
                                           i32, f64, f32, p, sz, p]
    L.pic_selective_attn_paged.restype = ctypes.c_int
    L.pic_decode_workspace_bytes.argtypes = [p, i32]
    L.pic_decode_workspace_bytes.restype = sz
    L.pic_decode_attn_paged.argtypes = [p, p, p, p, p, p, p, i64, i32, p, i32, p, p, p, p, i32,
                                        i32, i32, f64, f32, p, sz, p]
    L.pic_decode_attn_paged.restype = ctypes.c_int
    L.pic_qkv_workspace_bytes.argtypes = [p, i32]
    L.pic_qkv_workspace_bytes.restype = sz
    L.pic_qkv_rope.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, f64, p, sz, p]
    L.pic_qkv_rope.restype = ctypes.c_int
    L.pic_out_proj.argtypes = [p, p, p, p, i32, i32, i32, p]
    L.pic_out_proj.restype = ctypes.c_int
    L.pic_link_workspace_bytes.argtypes = [p, i32]
    L.pic_link_workspace_bytes.restype = sz
    L.pic_link.argtypes = [p, p, i32, p, p, p, p, p, p, p, p, p, i32, i32, i32, i32, f64, f32,
                           p, sz, p]
    L.pic_link.restype = ctypes.c_int
    L.pic_state_compose.argtypes = [p, p, i32, i32, i32, p, p, i32, p, p, p, i32, p]
    L.pic_state_compose.restype = ctypes.c_int
    L.pic_strerror.argtypes = [ctypes.c_int]
    L.pic_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def strerror(status):
    return lib().pic_strerror(int(status)).decode()


def _check(fn, status):
    if status != PIC_OK:
        raise PicError(fn, status)


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None and a.size else None


class Plan:
    """Host plan (int32 numpy array) written by pic_build_index, plus section views."""

    def __init__(self, words):
        self.words = words
        self.dev = None

    def __getitem__(self, i):
        return int(self.words[i])

    def _sec(self, off_field, n, width=1):
        o = self[off_field]
        return self.words[o:o + n * width].reshape(n, width) if width > 1 else self.words[o:o + n]

    @property
    def n_rows(self):
        return self[H_N_ROWS]

    @property
    def n_tokens(self):
        return self[H_N_TOKENS]

    @property
    def rows(self):
        return self._sec(H_O_ROWS, self[H_N_ROWS])

    @property
    def row_tok(self):
        return self._sec(H_O_ROW_TOK, self[H_N_ROWS])

    @property
    def chunk_off(self):
        return self._sec(H_O_CHUNK_OFF, self[H_N_CHUNKS] + self[H_N_REQ])

    @property
    def req_tok_ptr(self):
        return self._sec(H_O_REQ_TOK_PTR, self[H_N_REQ] + 1)

    @property
    def req_row_ptr(self):
        return self._sec(H_O_REQ_ROW_PTR, self[H_N_REQ] + 1)

    @property
    def rope_tiles(self):
        return self._sec(H_O_ROPE_TILES, self[H_N_ROPE_TILES], 4)

    @property
    def attn_tiles(self):
        return self._sec(H_O_ATTN_TILES, self[H_N_ATTN_TILES], 8)

    @property
    def attn_items(self):
        return self._sec(H_O_ATTN_ITEMS, self[H_N_ATTN_ITEMS], 8)

    @property
    def merges(self):
        return self._sec(H_O_MERGE, self[H_N_MERGE], 4)

    @property
    def paged(self):
        return bool(self[H_PAGED])

    @property
    def segments(self):
        return self._sec(H_O_SEGS, self[H_N_CHUNKS] if self.paged else 0, 8)

    @property
    def kblocks(self):
        return self._sec(H_O_KBLOCKS, self[H_N_KBLOCKS], 4)

    @property
    def dec_items(self):
        """[n][4]: source (pool chunk id, or -1-b), key count, first use, use count."""
        return self._sec(H_O_DEC_ITEMS, self[H_N_DEC_ITEMS], 4)

    @property
    def dec_uses(self):
        return self._sec(H_O_DEC_USES, self[H_N_DEC_USES], 1).reshape(-1)

    def _has_decode(self):
        return self.paged and self[H_H_Q] // self[H_H_KV] <= PIC_DECODE_COLS

    @property
    def dec_rec_ptr(self):
        n = self[H_N_REQ] * self[H_H_KV] + 1 if self._has_decode() else 0
        return self._sec(H_O_DEC_REC_PTR, n, 1)

    @property
    def dec_pieces(self):
        """[n][8]: item, kv head, first key, end key, record offset, 0, 0, 0."""
        return self._sec(H_O_DEC_PIECES, self[H_N_DEC_PIECES], 8)

    @property
    def dec_piece_recs(self):
        items = self.dec_items
        n = int(sum(items[p[0], 3] for p in self.dec_pieces)) if len(items) else 0
        return self._sec(H_O_DEC_PIECE_RECS, n, 1)

    @property
    def dec_wg_ptr(self):
        n = self[H_N_DEC_WG] + 1 if self._has_decode() and self[H_N_DEC_WG] > 0 else 0
        return self._sec(H_O_DEC_WG_PTR, n, 1)

    def to_device(self, device="cuda"):
        """Upload the plan (one int32 tensor) and keep it with the host copy."""
        import torch
        self.dev = torch.from_numpy(self.words).to(device)
        return self.dev

    def host_ptr(self):
        return self.words.ctypes.data_as(ctypes.c_void_p)

    def dev_ptr(self):
        if self.dev is None:
            raise RuntimeError("plan not uploaded: call Plan.to_device() first")
        return ctypes.c_void_p(self.dev.data_ptr())


def pic_build_index(chunk_lens_per_req, q_lens, k, h_q, h_kv, pos_base=0, n_cu=0,
                    chunk_ids_per_req=None):
    """Run the host planner.  chunk_lens_per_req: list (per request) of chunk-length lists;
    chunk_ids_per_req: pool chunk ids of the same shape for a paged pool, or None."""
    n_req = len(chunk_lens_per_req)
    ptr = np.zeros(n_req + 1, dtype=np.int64)
    ptr[1:] = np.cumsum([len(c) for c in chunk_lens_per_req])
    rcp = _i32(ptr)
    lens = _i32([x for c in chunk_lens_per_req for x in c])
    ql = _i32(q_lens)
    ids = None
    if chunk_ids_per_req is not None:
        ids = _i32([x for c in chunk_ids_per_req for x in c])
        if ids.size != lens.size:
            raise ValueError("chunk_ids_per_req must match chunk_lens_per_req")
    ids_p = ids.ctypes.data_as(ctypes.c_void_p) if ids is not None else None
    if ids is not None and ids.size == 0:
        ids_p = ctypes.cast(ctypes.pointer(_NO_CHUNKS), ctypes.c_void_p)  # paged, no chunks
    words = ctypes.c_int64(0)
    L = lib()
    st = L.pic_build_index(n_req, _ptr(rcp), _ptr(lens), _ptr(ql), ids_p, int(k), int(pos_base),
                           int(h_q), int(h_kv), int(n_cu), None, 0, ctypes.byref(words))
    _check("pic_build_index", st)
    plan = np.zeros(words.value, dtype=np.int32)
    st = L.pic_build_index(n_req, _ptr(rcp), _ptr(lens), _ptr(ql), ids_p, int(k), int(pos_base),
                           int(h_q), int(h_kv), int(n_cu), _ptr(plan), plan.size,
                           ctypes.byref(words))
    _check("pic_build_index", st)
    return Plan(plan)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return PIC_BF16
    if t.dtype == torch.float32:
        return PIC_F32
    raise TypeError("unsupported dtype %s" % (t.dtype,))


def _dev(t, name):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous device tensor" % name)
    return ctypes.c_void_p(t.data_ptr())


def _scale(scale):
    """None -> 0.0, which the library reads as its default 1/sqrt(head_dim)."""
    return 0.0 if scale is None else float(scale)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def pic_rope_delta(plan, k, rope_base, layout=PIC_ROPE_ADJACENT, stream=None):
    """In-place rotary correction of k ([n_tokens, h_kv, D]) on the current stream."""
    if k.shape[0] != plan.n_tokens or k.shape[1] != plan[H_H_KV]:
        raise ValueError("k shape %s does not match the plan" % (tuple(k.shape),))
    st = lib().pic_rope_delta(plan.host_ptr(), plan.dev_ptr(), _dev(k, "k"), _dtype_code(k),
                              int(k.shape[2]), int(layout), float(rope_base), _stream(stream))
    _check("pic_rope_delta", st)


def pic_rope_apply(plan, k, rope_base, layout=PIC_ROPE_ADJACENT, stream=None):
    """In-place RoPE at the global positions of the kept cached rows of a position-free
    ("nope") cache k ([n_tokens, h_kv, D]) on the current stream."""
    if k.shape[0] != plan.n_tokens or k.shape[1] != plan[H_H_KV]:
        raise ValueError("k shape %s does not match the plan" % (tuple(k.shape),))
    st = lib().pic_rope_apply(plan.host_ptr(), plan.dev_ptr(), _dev(k, "k"), _dtype_code(k),
                              int(k.shape[2]), int(layout), float(rope_base), _stream(stream))
    _check("pic_rope_apply", st)


def pic_splice(plan, k, v, k_fresh, v_fresh, stream=None):
    """k[row_tok[r]] = k_fresh[r], v[row_tok[r]] = v_fresh[r] for every recomputed row."""
    for t, n in ((k, plan.n_tokens), (v, plan.n_tokens), (k_fresh, plan.n_rows),
                 (v_fresh, plan.n_rows)):
        if t.shape[0] != n or t.dtype != k.dtype or tuple(t.shape[1:]) != tuple(k.shape[1:]):
            raise ValueError("buffer shapes/dtypes do not match the plan")
    st = lib().pic_splice(plan.host_ptr(), plan.dev_ptr(), _dev(k, "k"), _dev(v, "v"),
                          _dev(k_fresh, "k_fresh"), _dev(v_fresh, "v_fresh"), _dtype_code(k),
                          int(k.shape[2]), _stream(stream))
    _check("pic_splice", st)


def pic_rope_splice(plan, k, v, k_fresh, v_fresh, rope_base, layout=PIC_ROPE_ADJACENT,
                    mode=PIC_ROPE_BY_DELTA, stream=None):
    """pic_rope_delta (mode PIC_ROPE_BY_DELTA) or pic_rope_apply (PIC_ROPE_AT_POSITION),
    then pic_splice, as one launch on the current stream."""
    for t, n in ((k, plan.n_tokens), (v, plan.n_tokens), (k_fresh, plan.n_rows),
                 (v_fresh, plan.n_rows)):
        if t.shape[0] != n or t.dtype != k.dtype or tuple(t.shape[1:]) != tuple(k.shape[1:]):
            raise ValueError("buffer shapes/dtypes do not match the plan")
    if k.shape[1] != plan[H_H_KV]:
        raise ValueError("k shape %s does not match the plan" % (tuple(k.shape),))
    st = lib().pic_rope_splice(plan.host_ptr(), plan.dev_ptr(), _dev(k, "k"), _dev(v, "v"),
                               _dev(k_fresh, "k_fresh"), _dev(v_fresh, "v_fresh"),
                               _dtype_code(k), int(k.shape[2]), int(layout), float(rope_base),
                               int(mode), _stream(stream))
    _check("pic_rope_splice", st)


def pic_rope_splice_pool(plan, pool_k, pool_v, chunk_block_ptr, block_ids, k, v, k_fresh,
                         v_fresh, rope_base, layout=PIC_ROPE_ADJACENT, stream=None):
    """Rotation + splice of a paged plan's requests from the shared pool [blocks, 16, h_kv,
    D] (read-only) into contiguous k/v [n_tokens, h_kv, D]; pic_selective_attn with the
    matching contiguous plan then attends over them."""
    import torch
    if not plan.paged:
        raise ValueError("plan was not built with chunk ids (paged pool)")
    d = int(k.shape[2])
    if k.shape != (plan.n_tokens, plan[H_H_KV], d) or v.shape != k.shape:
        raise ValueError("k/v must be [n_tokens, h_kv, D]")
    if pool_k.dim() != 4 or pool_v.shape != pool_k.shape or pool_k.shape[2] != plan[H_H_KV] \
            or pool_k.shape[3] != d:
        raise ValueError("pool must be [blocks, block_size, h_kv, D]")
    if k_fresh.shape != (plan.n_rows, plan[H_H_KV], d) or v_fresh.shape != k_fresh.shape:
        raise ValueError("fresh K/V must be [n_rows, h_kv, D]")
    for t, name in ((chunk_block_ptr, "chunk_block_ptr"), (block_ids, "block_ids")):
        if t.dtype != torch.int32 or t.dim() != 1:
            raise ValueError(name + " must be a 1-D int32 tensor")
    for t in (pool_k, pool_v, v, k_fresh, v_fresh):
        if t.dtype != k.dtype:
            raise ValueError("all tensors must share one dtype")
    st = lib().pic_rope_splice_pool(
        plan.host_ptr(), plan.dev_ptr(), _dev(pool_k, "pool_k"), _dev(pool_v, "pool_v"),
        int(pool_k.shape[0]), int(pool_k.shape[1]), _dev(chunk_block_ptr, "chunk_block_ptr"),
        int(chunk_block_ptr.numel()) - 1, _dev(block_ids, "block_ids"), _dev(k, "k"),
        _dev(v, "v"), _dev(k_fresh, "k_fresh"), _dev(v_fresh, "v_fresh"), _dtype_code(k), d,
        int(layout), float(rope_base), _stream(stream))
    _check("pic_rope_splice_pool", st)


def pic_attn_workspace_bytes(plan, head_dim):
    return int(lib().pic_attn_workspace_bytes(plan.host_ptr(), int(head_dim)))


def pic_selective_attn(plan, q, k, v, out, scale=None, workspace=None, stream=None):
    """out[r, h] = causal attention of q[r, h] over the spliced k/v of its request."""
    d = int(q.shape[2])
    if q.shape[0] != plan.n_rows or out.shape != q.shape or q.shape[1] != plan[H_H_Q]:
        raise ValueError("q/out shapes do not match the plan")
    if k.shape[0] != plan.n_tokens or v.shape != k.shape or k.shape[1] != plan[H_H_KV]:
        raise ValueError("k/v shapes do not match the plan")
    for t in (k, v, out):
        if t.dtype != q.dtype:
            raise ValueError("q, k, v and out must share one dtype")
    ws, ws_bytes = None, 0
    if workspace is not None:
        ws, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    st = lib().pic_selective_attn(plan.host_ptr(), plan.dev_ptr(), _dev(q, "q"), _dev(k, "k"),
                                  _dev(v, "v"), _dev(out, "out"), _dtype_code(q), d,
                                  _scale(scale), ws, ws_bytes, _stream(stream))
    _check("pic_selective_attn", st)


PIC_ATTN_SCRATCH_BYTES = 128 << 20


def pic_selective_attn_noalloc(plan, q, k, v, out, scale=None, stream=None):
    """pic_selective_attn with the split-KV partials in the library's per-GPU scratch
    array (no workspace, no allocation); plans needing more than PIC_ATTN_SCRATCH_BYTES
    raise PicError (PIC_ENOSPC)."""
    d = int(q.shape[2])
    if q.shape[0] != plan.n_rows or out.shape != q.shape or q.shape[1] != plan[H_H_Q]:
        raise ValueError("q/out shapes do not match the plan")
    if k.shape[0] != plan.n_tokens or v.shape != k.shape or k.shape[1] != plan[H_H_KV]:
        raise ValueError("k/v shapes do not match the plan")
    for t in (k, v, out):
        if t.dtype != q.dtype:
            raise ValueError("q, k, v and out must share one dtype")
    st = lib().pic_selective_attn_noalloc(plan.host_ptr(), plan.dev_ptr(), _dev(q, "q"),
                                          _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                                          _dtype_code(q), d, _scale(scale), _stream(stream))
    _check("pic_selective_attn_noalloc", st)


def attn_workspace(plan, head_dim, device="cuda"):
    """Allocate the split-KV workspace a plan needs (a float32 device tensor or None)."""
    import torch
    n = pic_attn_workspace_bytes(plan, head_dim)
    if n == 0:
        return None
    return torch.empty(n // 4, dtype=torch.float32, device=device)


def pic_selective_attn_paged(plan, q, pool_k, pool_v, chunk_block_ptr, block_ids, k_fresh,
                             v_fresh, out, rope_base, layout=PIC_ROPE_ADJACENT, scale=None,
                             workspace=None, stream=None):
    """Selective attention over a shared paged pool [blocks, 16, h_kv, D] (read-only)."""
    import torch
    d = int(q.shape[2])
    if not plan.paged:
        raise ValueError("plan was not built with chunk ids (paged pool)")
    if q.shape[0] != plan.n_rows or out.shape != q.shape or q.shape[1] != plan[H_H_Q]:
        raise ValueError("q/out shapes do not match the plan")
    if pool_k.dim() != 4 or pool_v.shape != pool_k.shape or pool_k.shape[2] != plan[H_H_KV]:
        raise ValueError("pool must be [blocks, block_size, h_kv, D]")
    for t, name in ((chunk_block_ptr, "chunk_block_ptr"), (block_ids, "block_ids")):
        if t.dtype != torch.int32 or t.dim() != 1:
            raise ValueError(name + " must be a 1-D int32 tensor")
    if k_fresh.shape != (plan.n_rows, plan[H_H_KV], d) or v_fresh.shape != k_fresh.shape:
        raise ValueError("fresh K/V must be [n_rows, h_kv, D]")
    for t in (pool_k, pool_v, k_fresh, v_fresh, out):
        if t.dtype != q.dtype:
            raise ValueError("all tensors must share one dtype")
    ws, ws_bytes = None, 0
    if workspace is not None:
        ws, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    st = lib().pic_selective_attn_paged(
        plan.host_ptr(), plan.dev_ptr(), _dev(q, "q"), _dev(pool_k, "pool_k"),
        _dev(pool_v, "pool_v"), int(pool_k.shape[0]), int(pool_k.shape[1]),
        _dev(chunk_block_ptr, "chunk_block_ptr"), int(chunk_block_ptr.numel()) - 1,
        _dev(block_ids, "block_ids"),
        _dev(k_fresh, "k_fresh"), _dev(v_fresh, "v_fresh"), _dev(out, "out"), _dtype_code(q), d,
        int(layout), float(rope_base), _scale(scale), ws, ws_bytes, _stream(stream))
    _check("pic_selective_attn_paged", st)


def decode_workspace(plan, head_dim, device="cuda"):
    """Workspace tensor for pic_decode_attn_paged."""
    import torch
    n = int(lib().pic_decode_workspace_bytes(plan.host_ptr(), int(head_dim)))
    return torch.empty(max(1, (n + 3) // 4), dtype=torch.float32, device=device)


def pic_decode_attn_paged(plan, q_new, k_new, v_new, pool_k, pool_v, chunk_block_ptr, block_ids,
                          k_fresh, v_fresh, out, rope_base, layout=PIC_ROPE_ADJACENT, scale=None,
                          workspace=None, stream=None):
    """One decode step of every request of a paged plan: the next token (position N_b)
    attends over the request's pool chunks, recomputed rows and itself."""
    import torch
    d = int(q_new.shape[2])
    if not plan.paged:
        raise ValueError("plan was not built with chunk ids (paged pool)")
    n_req = plan[H_N_REQ]
    if q_new.shape != (n_req, plan[H_H_Q], d) or out.shape != q_new.shape:
        raise ValueError("q_new/out must be [n_req, h_q, D]")
    if k_new.shape != (n_req, plan[H_H_KV], d) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [n_req, h_kv, D]")
    if pool_k.dim() != 4 or pool_v.shape != pool_k.shape or pool_k.shape[2] != plan[H_H_KV]:
        raise ValueError("pool must be [blocks, block_size, h_kv, D]")
    if k_fresh.shape != (plan.n_rows, plan[H_H_KV], d) or v_fresh.shape != k_fresh.shape:
        raise ValueError("fresh K/V must be [n_rows, h_kv, D]")
    for t, name in ((chunk_block_ptr, "chunk_block_ptr"), (block_ids, "block_ids")):
        if t.dtype != torch.int32 or t.dim() != 1:
            raise ValueError(name + " must be a 1-D int32 tensor")
    for t in (k_new, v_new, pool_k, pool_v, k_fresh, v_fresh, out):
        if t.dtype != q_new.dtype:
            raise ValueError("all tensors must share one dtype")
    if workspace is None:
        workspace = decode_workspace(plan, d, q_new.device)
    st = lib().pic_decode_attn_paged(
        plan.host_ptr(), plan.dev_ptr(), _dev(q_new, "q_new"), _dev(k_new, "k_new"),
        _dev(v_new, "v_new"), _dev(pool_k, "pool_k"), _dev(pool_v, "pool_v"),
        int(pool_k.shape[0]), int(pool_k.shape[1]), _dev(chunk_block_ptr, "chunk_block_ptr"),
        int(chunk_block_ptr.numel()) - 1, _dev(block_ids, "block_ids"), _dev(k_fresh, "k_fresh"),
        _dev(v_fresh, "v_fresh"), _dev(out, "out"), _dtype_code(q_new), d, int(layout),
        float(rope_base), _scale(scale), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("pic_decode_attn_paged", st)


def _bytes_workspace(n, device):
    import torch
    return torch.empty(max(1, (int(n) + 3) // 4), dtype=torch.float32, device=device)


def pic_qkv_rope(plan, x, w_qkv, q, k_fresh, v_fresh, rope_base, layout=PIC_ROPE_ADJACENT,
                 workspace=None, stream=None):
    """compute_qkv of the recomputed rows: q/k_fresh/v_fresh from x [n_rows, d_model] and
    w_qkv [(h_q + 2 h_kv) * D, d_model], Q and K rotated at the rows' global positions."""
    d = int(q.shape[2])
    d_model = int(x.shape[1])
    hq, hkv = plan[H_H_Q], plan[H_H_KV]
    if x.shape[0] != plan.n_rows or q.shape != (plan.n_rows, hq, d):
        raise ValueError("x/q shapes do not match the plan")
    if k_fresh.shape != (plan.n_rows, hkv, d) or v_fresh.shape != k_fresh.shape:
        raise ValueError("k_fresh/v_fresh must be [n_rows, h_kv, D]")
    if w_qkv.shape != ((hq + 2 * hkv) * d, d_model):
        raise ValueError("w_qkv must be [(h_q + 2 h_kv) * D, d_model]")
    for t in (w_qkv, q, k_fresh, v_fresh):
        if t.dtype != x.dtype:
            raise ValueError("all tensors must share one dtype")
    if workspace is None:
        workspace = _bytes_workspace(lib().pic_qkv_workspace_bytes(plan.host_ptr(), d), x.device)
    st = lib().pic_qkv_rope(plan.host_ptr(), plan.dev_ptr(), _dev(x, "x"), _dev(w_qkv, "w_qkv"),
                            _dev(q, "q"), _dev(k_fresh, "k_fresh"), _dev(v_fresh, "v_fresh"),
                            _dtype_code(x), d_model, d, int(layout), float(rope_base),
                            _dev(workspace, "workspace"),
                            workspace.numel() * workspace.element_size(), _stream(stream))
    _check("pic_qkv_rope", st)


def pic_out_proj(plan, o, w_o, x, stream=None):
    """x += o W_o^T in place (o [n_rows, h_q, D], w_o [d_model, h_q * D])."""
    d = int(o.shape[2])
    d_model = int(x.shape[1])
    if o.shape != (plan.n_rows, plan[H_H_Q], d) or x.shape[0] != plan.n_rows:
        raise ValueError("o/x shapes do not match the plan")
    if w_o.shape != (d_model, plan[H_H_Q] * d):
        raise ValueError("w_o must be [d_model, h_q * D]")
    if w_o.dtype != x.dtype or o.dtype != x.dtype:
        raise ValueError("all tensors must share one dtype")
    st = lib().pic_out_proj(plan.host_ptr(), _dev(o, "o"), _dev(w_o, "w_o"), _dev(x, "x"),
                            _dtype_code(x), d_model, d, _stream(stream))
    _check("pic_out_proj", st)


def link_workspace(plan, head_dim, device="cuda"):
    """Workspace tensor for pic_link."""
    return _bytes_workspace(lib().pic_link_workspace_bytes(plan.host_ptr(), int(head_dim)), device)


def pic_link(plan, x, w_qkv, w_o, k_cache, v_cache, q, k_fresh, v_fresh, o, rope_base,
             layout=PIC_ROPE_ADJACENT, scale=None, workspace=None, stream=None):
    """The whole link over len(w_qkv) layers: per layer rope-delta, compute_qkv, splice,
    selective attention and output projection; x (the rows' hidden states) in place."""
    n_layers = len(w_qkv)
    if not (len(w_o) == len(k_cache) == len(v_cache) == n_layers):
        raise ValueError("one w_qkv, w_o, k_cache and v_cache per layer")
    d = int(q.shape[2])
    d_model = int(x.shape[1])
    hq, hkv = plan[H_H_Q], plan[H_H_KV]
    if x.shape[0] != plan.n_rows or q.shape != (plan.n_rows, hq, d) or o.shape != q.shape:
        raise ValueError("x/q/o shapes do not match the plan")
    if k_fresh.shape != (plan.n_rows, hkv, d) or v_fresh.shape != k_fresh.shape:
        raise ValueError("k_fresh/v_fresh must be [n_rows, h_kv, D]")
    for l in range(n_layers):
        if w_qkv[l].shape != ((hq + 2 * hkv) * d, d_model) or w_o[l].shape != (d_model, hq * d):
            raise ValueError("layer %d weight shapes" % l)
        if k_cache[l].shape != (plan.n_tokens, hkv, d) or v_cache[l].shape != k_cache[l].shape:
            raise ValueError("layer %d K/V must be [n_tokens, h_kv, D]" % l)
    for t in list(w_qkv) + list(w_o) + list(k_cache) + list(v_cache) + [q, k_fresh, v_fresh, o]:
        if t.dtype != x.dtype:
            raise ValueError("all tensors must share one dtype")
    arr = lambda ts, name: (ctypes.c_void_p * max(1, n_layers))(*[_dev(t, name).value for t in ts])
    if workspace is None:
        workspace = link_workspace(plan, d, x.device)
    st = lib().pic_link(plan.host_ptr(), plan.dev_ptr(), n_layers, _dev(x, "x"),
                        arr(w_qkv, "w_qkv"), arr(w_o, "w_o"), arr(k_cache, "k_cache"),
                        arr(v_cache, "v_cache"), _dev(q, "q"), _dev(k_fresh, "k_fresh"),
                        _dev(v_fresh, "v_fresh"), _dev(o, "o"), _dtype_code(x), d_model, d,
                        int(layout), float(rope_base), _scale(scale),
                        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                        _stream(stream))
    _check("pic_link", st)


def pic_state_compose(plan, t_pool, s_pool, final_out, prefix_out=None, s_init=None,
                      stream=None):
    """Linear-layer states over each request's chunks: S_c = T S_{c-1} + S(C|0).
    t_pool [n_pool, H, dk, dk], s_pool [n_pool, H, dk, dv], final_out [n_req, H, dk, dv],
    prefix_out [n_chunks, H, dk, dv] or None, s_init [n_req, H, dk, dv] or None."""
    if not plan.paged:
        raise ValueError("plan was not built with chunk ids (paged pool)")
    n_pool, n_heads, d_k, d_v = (int(x) for x in s_pool.shape)
    if t_pool.shape != (n_pool, n_heads, d_k, d_k):
        raise ValueError("t_pool must be [n_pool, H, dk, dk]")
    if final_out.shape != (plan[H_N_REQ], n_heads, d_k, d_v):
        raise ValueError("final_out must be [n_req, H, dk, dv]")
    if prefix_out is not None and prefix_out.shape != (plan[H_N_CHUNKS], n_heads, d_k, d_v):
        raise ValueError("prefix_out must be [n_chunks, H, dk, dv]")
    if s_init is not None and s_init.shape != final_out.shape:
        raise ValueError("s_init must be [n_req, H, dk, dv]")
    for t in (t_pool, final_out) + tuple(x for x in (prefix_out, s_init) if x is not None):
        if t.dtype != s_pool.dtype:
            raise ValueError("all tensors must share one dtype")
    opt = lambda t, n: None if t is None else _dev(t, n)
    st = lib().pic_state_compose(plan.host_ptr(), plan.dev_ptr(), n_heads, d_k, d_v,
                                 _dev(t_pool, "t_pool"), _dev(s_pool, "s_pool"), n_pool,
                                 opt(s_init, "s_init"), opt(prefix_out, "prefix_out"),
                                 _dev(final_out, "final_out"), _dtype_code(s_pool),
                                 _stream(stream))
    _check("pic_state_compose", st)
