"""C-ABI surface and host planner (pic_build_index), CPU only.

The planner is host code, so it runs here: its recompute index, offsets and
buffer rows must equal the oracle's bit for bit, and its launch schedules must
cover exactly the rows and keys the definition needs.  No kernel is launched.
"""

import ctypes
import itertools
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import position_independent_kv_rope_amd as P
from oracle import pic_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(P.LIB_PATH):
        from position_independent_kv_rope_amd import build
        build.build()


def _declared_symbols(header="pic.h"):
    with open(os.path.join(ROOT, "include", header)) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pic_[a-z_]+)\s*\(", text)))


def test_plain_c_caller_plans_the_worked_example(tmp_path):
    # the header compiles as C11 with warnings as errors, and a C program linked against
    # libpic.so plans the pages' worked example through the ABI alone (host only)
    import json
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    lib_dir = os.path.dirname(P.LIB_PATH)
    exe = str(tmp_path / "abi_worked_example")
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(root, "include"),
                    os.path.join(here, "c", "abi_worked_example.c"), "-o", exe,
                    "-L", lib_dir, "-lpic", "-Wl,-rpath," + lib_dir], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split("\n")
    gold = json.load(open(os.path.join(here, "golden", "worked_example.json")))
    assert out[0].split()[1:] == [str(p) for p in gold["recompute_positions"]]
    assert out[1].split()[1:] == [str(o) for o in gold["offsets"]]
    assert out[2] == "tokens %d" % gold["n_total"]
    assert out[3].startswith("bad plan: ") and len(out[3]) > len("bad plan: ")


def test_library_exports_every_declared_symbol():
    syms = _declared_symbols()
    assert set(syms) == set(P.EXPORTED), syms
    lib = ctypes.CDLL(P.LIB_PATH)
    for s in syms:
        assert hasattr(lib, s), s


def test_calibration_library_exports_and_host_checks():
    # libpic_calib.so (the bench's measured peaks) exports what pic_calib.h declares; its
    # argument checks and flop count run on the host (no launch for an invalid argument)
    from position_independent_kv_rope_amd import build
    if not os.path.exists(build.CALIB_LIB):
        build.build()
    syms = _declared_symbols("pic_calib.h")
    assert syms == sorted(["pic_calib_copy", "pic_calib_mfma", "pic_calib_mfma_flops",
                           "pic_calib_read", "pic_calib_read_sink_words", "pic_calib_update"])
    lib = ctypes.CDLL(build.CALIB_LIB)
    for s in syms:
        assert hasattr(lib, s), s
    i32, i64, p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.pic_calib_mfma_flops.argtypes = [i32, i32]
    lib.pic_calib_mfma_flops.restype = i64
    assert lib.pic_calib_mfma_flops(512, 4096) == 512 * 4 * 4096 * 4 * 2 * 32 * 32 * 16
    lib.pic_calib_read_sink_words.argtypes = [i64]
    lib.pic_calib_read_sink_words.restype = i64
    assert lib.pic_calib_read_sink_words(8) == 0
    assert lib.pic_calib_read_sink_words(16) == 4            # one workgroup, four waves
    assert lib.pic_calib_read_sink_words(1 << 31) == 4096 * 4  # grid capped at 4096
    lib.pic_calib_read.argtypes = [p, i64, p, p]
    lib.pic_calib_copy.argtypes = [p, p, i64, p]
    lib.pic_calib_mfma.argtypes = [p, p, i32, i32, p]
    assert lib.pic_calib_read(None, 16, None, None) == -1
    assert lib.pic_calib_read(p(16), 24, p(16), None) == -1    # not a multiple of 16
    assert lib.pic_calib_copy(p(16), None, 16, None) == -1
    lib.pic_calib_update.argtypes = [p, i64, p]
    assert lib.pic_calib_update(None, 16, None) == -1
    assert lib.pic_calib_update(p(16), 0, None) == -1
    assert lib.pic_calib_mfma(p(16), p(16), 4, 6, None) == -1  # rounds not a multiple of 4
    assert lib.pic_calib_mfma(p(16), p(16), 0, 4, None) == -1


def test_strerror_and_status_codes():
    assert P.strerror(P.PIC_OK) == "ok"
    for code in (P.PIC_EINVAL, P.PIC_ENOSPC, P.PIC_EUNSUPPORTED, P.PIC_EDEVICE):
        assert P.strerror(code) != "unknown status"
    assert P.strerror(12345) == "unknown status"


def _build_raw(rcp, lens, ql, k, h_q=4, h_kv=4, pos_base=0, cap=None):
    L = P.lib()
    rcp, lens, ql = (np.asarray(a, dtype=np.int32) for a in (rcp, lens, ql))
    words = ctypes.c_int64(0)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p) if a.size else None
    n_req = len(ql)
    st0 = L.pic_build_index(n_req, ptr(rcp), ptr(lens), ptr(ql), None, k, pos_base, h_q, h_kv,
                            0, None, 0, ctypes.byref(words))
    if st0 != 0 or cap is None:
        return st0, words.value
    buf = np.full(max(cap, 1), 0x5A5A5A5A, dtype=np.int32)
    st1 = L.pic_build_index(n_req, ptr(rcp), ptr(lens), ptr(ql), None, k, pos_base, h_q, h_kv,
                            0, ptr(buf), cap, ctypes.byref(words))
    return st1, buf


def test_build_index_error_paths():
    assert _build_raw([0, 1], [3], [2], -1)[0] == P.PIC_EINVAL       # k < 0
    assert _build_raw([0, 1], [-3], [2], 1)[0] == P.PIC_EINVAL       # negative length
    assert _build_raw([0, 1], [3], [-2], 1)[0] == P.PIC_EINVAL       # negative q
    assert _build_raw([1, 1], [3], [2], 1)[0] == P.PIC_EINVAL        # CSR not from 0
    assert _build_raw([0, 2, 1], [3, 3], [1, 1], 1)[0] == P.PIC_EINVAL  # CSR decreasing
    assert _build_raw([0, 1], [3], [2], 1, h_q=6, h_kv=4)[0] == P.PIC_EINVAL
    assert _build_raw([0, 1], [3], [2], 1, h_q=12, h_kv=4)[0] == P.PIC_EUNSUPPORTED  # G=3
    assert _build_raw([0, 1, 2], [3, 1 << 25], [1, 1], 1)[0] == P.PIC_OK  # chunk 0 of req 1
    assert _build_raw([0, 2], [1 << 25, 3], [1], 1)[0] == P.PIC_EUNSUPPORTED  # delta > 2^24
    st, need = _build_raw([0, 3], [4, 5, 5], [3], 2)
    assert st == P.PIC_OK and need > 32
    st, buf = _build_raw([0, 3], [4, 5, 5], [3], 2, cap=need - 1)
    assert st == P.PIC_ENOSPC and np.all(buf == 0x5A5A5A5A)  # untouched


def test_device_entry_points_reject_bad_arguments_without_launching():
    L = P.lib()
    plan = P.pic_build_index([[4, 5, 5]], [3], 2, 4, 4)
    hp = plan.host_ptr()
    bogus = np.zeros(64, dtype=np.int32)
    bp = bogus.ctypes.data_as(ctypes.c_void_p)
    fake = ctypes.c_void_p(0x1000)
    assert L.pic_rope_delta(bp, fake, fake, P.PIC_F32, 16, 0, 1e4, None) == P.PIC_EINVAL
    assert L.pic_rope_delta(hp, fake, fake, 7, 16, 0, 1e4, None) == P.PIC_EINVAL
    assert L.pic_rope_delta(hp, fake, fake, P.PIC_F32, 15, 0, 1e4, None) == P.PIC_EINVAL
    assert L.pic_rope_delta(hp, fake, fake, P.PIC_F32, 16, 2, 1e4, None) == P.PIC_EINVAL
    assert L.pic_rope_delta(hp, fake, fake, P.PIC_F32, 16, 0, -1.0, None) == P.PIC_EINVAL
    assert L.pic_rope_delta(hp, fake, fake, P.PIC_F32, 12, 0, 1e4, None) == P.PIC_EUNSUPPORTED
    assert L.pic_rope_delta(hp, fake, None, P.PIC_F32, 16, 0, 1e4, None) == P.PIC_EINVAL
    assert L.pic_splice(bp, fake, fake, fake, fake, fake, P.PIC_F32, 16, None) == P.PIC_EINVAL
    assert L.pic_splice(hp, fake, fake, None, fake, fake, P.PIC_F32, 16, None) == P.PIC_EINVAL
    assert L.pic_splice(hp, fake, fake, fake, fake, fake, P.PIC_F32, 12, None) == P.PIC_EUNSUPPORTED
    rs = L.pic_rope_splice
    f4 = (fake, fake, fake, fake)
    assert rs(bp, fake, *f4, P.PIC_F32, 16, 0, 1e4, 0, None) == P.PIC_EINVAL  # bad plan
    assert rs(hp, fake, *f4, P.PIC_F32, 16, 0, 1e4, 2, None) == P.PIC_EINVAL  # rope_mode
    assert rs(hp, fake, *f4, P.PIC_F32, 16, 2, 1e4, 0, None) == P.PIC_EINVAL  # layout
    assert rs(hp, fake, *f4, P.PIC_F32, 16, 0, 0.0, 1, None) == P.PIC_EINVAL  # base
    assert rs(hp, fake, *f4, 7, 16, 0, 1e4, 0, None) == P.PIC_EINVAL  # dtype
    assert rs(hp, fake, None, fake, fake, fake, P.PIC_F32, 16, 0, 1e4, 0, None) == P.PIC_EINVAL
    assert rs(hp, fake, fake, None, fake, fake, P.PIC_F32, 16, 0, 1e4, 0, None) == P.PIC_EINVAL
    assert rs(hp, fake, fake, fake, fake, None, P.PIC_F32, 16, 0, 1e4, 1, None) == P.PIC_EINVAL
    assert rs(hp, fake, *f4, P.PIC_F32, 12, 0, 1e4, 0, None) == P.PIC_EUNSUPPORTED
    args = (fake, fake, fake, fake)
    # scale: NaN or infinity is refused (a value <= 0 selects 1/sqrt(head_dim); the GPU
    # tests pass None, i.e. 0, and compare with the oracle at 1/sqrt(D))
    for bad in (float("nan"), float("inf"), float("-inf")):
        assert L.pic_selective_attn(hp, fake, *args, P.PIC_F32, 16, bad, None, 0, None) == P.PIC_EINVAL
    assert L.pic_selective_attn(hp, fake, *args, P.PIC_F32, 24, 0.25, None, 0, None) == P.PIC_EUNSUPPORTED
    assert L.pic_selective_attn(hp, fake, *args, P.PIC_BF16, 16, 0.25, None, 0, None) == P.PIC_EUNSUPPORTED
    assert L.pic_selective_attn(hp, None, *args, P.PIC_F32, 16, 0.25, None, 0, None) == P.PIC_EINVAL
    # a split plan without workspace is refused before launch
    big = P.pic_build_index([[1024] * 32], [128], 2, 32, 8)
    assert P.pic_attn_workspace_bytes(big, 128) > 0
    assert L.pic_selective_attn(big.host_ptr(), fake, *args, P.PIC_BF16, 128, 0.088, None, 0,
                                None) == P.PIC_ENOSPC
    assert L.pic_attn_workspace_bytes(bp, 128) == 0


def test_pool_gather_rejects_bad_arguments_without_launching():
    L = P.lib()
    f = ctypes.c_void_p(0x1000)
    paged = P.pic_build_index([[40, 50]], [7], 2, 8, 4, chunk_ids_per_req=[[0, 1]])
    contig = P.pic_build_index([[40, 50]], [7], 2, 8, 4)
    call = lambda plan, n_pool=2, bs=16, dtype=P.PIC_BF16, d=128, layout=P.PIC_ROPE_ADJACENT, \
        base=1e4, k=f, pool_blocks=64: L.pic_rope_splice_pool(
            plan.host_ptr(), f, f, f, pool_blocks, bs, f, n_pool, f, k, f, f, f, dtype, d,
            layout, base, None)
    assert call(contig) == P.PIC_EINVAL                 # needs a plan built with chunk ids
    assert call(paged, n_pool=1) == P.PIC_EINVAL        # chunk id 1 outside the table
    assert call(paged, dtype=7) == P.PIC_EINVAL
    assert call(paged, layout=2) == P.PIC_EINVAL
    assert call(paged, base=0.0) == P.PIC_EINVAL
    assert call(paged, base=float("nan")) == P.PIC_EINVAL
    assert call(paged, pool_blocks=-1) == P.PIC_EINVAL
    assert call(paged, d=130) == P.PIC_EUNSUPPORTED     # not a multiple of 8
    assert call(paged, bs=32) == P.PIC_EUNSUPPORTED     # 16-row pool blocks only
    assert call(paged, k=None) == P.PIC_EINVAL


def test_request_size_limit_is_checked_before_launch():
    # K/V of one request are addressed with 32-bit byte offsets: 0x7fff0000 bytes of K
    # (N * h_kv * D * 2) are taken, one token more is refused without a launch
    L = P.lib()
    f = ctypes.c_void_p(0x1000)
    n_max = 0x7FFF0000 // (8 * 128 * 2)
    for n, want in ((n_max + 1, P.PIC_EUNSUPPORTED), (n_max, P.PIC_EINVAL)):
        plan = P.pic_build_index([[n - 64]], [64], 2, 32, 8)
        assert plan.n_tokens == n
        # a null output pointer is the only other fault, so the size check comes first
        st = L.pic_selective_attn(plan.host_ptr(), f, f, f, f, None, P.PIC_BF16, 128, 0.088,
                                  f, 1 << 40, None)
        assert st == want


def test_pool_size_limit_is_checked_before_launch():
    # pool K/V are addressed with 32-bit byte offsets: a pool of up to 0x7fff0000 bytes
    # less one block is taken, one block more is refused without a launch
    L = P.lib()
    f = ctypes.c_void_p(0x1000)
    plan = P.pic_build_index([[40, 50]], [7], 2, 32, 4, chunk_ids_per_req=[[0, 1]])
    blk = 16 * 4 * 128 * 2
    n_max = (0x7FFF0000 - blk) // blk
    for nb, want in ((n_max + 1, P.PIC_EUNSUPPORTED), (n_max, P.PIC_EINVAL)):
        # a null output pointer is the only other fault, so the size check comes first
        st = L.pic_selective_attn_paged(plan.host_ptr(), f, f, f, f, nb, 16, f, 2, f, f, f,
                                        None, P.PIC_BF16, 128, P.PIC_ROPE_ADJACENT, 1e4, 0.088,
                                        f, 1 << 40, None)
        assert st == want


def test_paged_workspace_covers_partials_angles_and_key_block_records():
    # the paged call keeps split-KV partials, a cos/sin table per chunk and one 32-byte
    # record per key block in the caller's workspace; one byte short is refused
    L = P.lib()
    f = ctypes.c_void_p(0x1000)
    plan = P.pic_build_index([[3000, 7000, 2600], [9000]], [40, 9], 8, 8, 2,
                             chunk_ids_per_req=[[0, 1, 2], [3]], n_cu=2)
    d = 128
    ws = P.pic_attn_workspace_bytes(plan, d)
    partials = plan[P.H_N_PARTIALS] * P.PIC_ATTN_TILE_M * (d + 2) * 4
    angles = plan[P.H_N_CHUNKS] * (d // 2) * 8
    assert plan[P.H_N_PARTIALS] > 0 and plan[P.H_N_KBLOCKS] > 0
    assert ws >= partials + angles + 32 * plan[P.H_N_KBLOCKS]
    assert ws <= partials + angles + 32 * plan[P.H_N_KBLOCKS] + 32
    call = lambda wsb: L.pic_selective_attn_paged(
        plan.host_ptr(), f, f, f, f, 64, 16, f, 4, f, f, f, f, P.PIC_BF16, d,
        P.PIC_ROPE_ADJACENT, 1e4, 0.088, f, wsb, None)
    assert call(ws - 1) == P.PIC_ENOSPC


def test_state_compose_rejects_bad_arguments_without_launching():
    L = P.lib()
    f = ctypes.c_void_p(0x1000)
    plan = P.pic_build_index([[40, 50]], [7], 2, 8, 2, chunk_ids_per_req=[[0, 3]])
    hp = plan.host_ptr()
    call = lambda hp=hp, heads=4, dk=128, dv=128, n_pool=4, fin=f, dt=P.PIC_F32, t=f: \
        L.pic_state_compose(hp, f, heads, dk, dv, t, f, n_pool, None, None, fin, dt, None)
    contiguous = P.pic_build_index([[40, 50]], [7], 2, 8, 2)
    assert call(hp=contiguous.host_ptr()) == P.PIC_EINVAL   # needs chunk ids
    assert call(heads=0) == P.PIC_EINVAL
    assert call(n_pool=3) == P.PIC_EINVAL                   # chunk id 3 >= n_pool
    assert call(fin=None) == P.PIC_EINVAL
    assert call(t=None) == P.PIC_EINVAL
    assert call(dt=9) == P.PIC_EINVAL
    assert call(dt=P.PIC_BF16) == P.PIC_EUNSUPPORTED        # the scan is fp32
    assert call(dk=64, dv=64) == P.PIC_EUNSUPPORTED


def test_link_entry_points_reject_bad_arguments_without_launching():
    L = P.lib()
    plan = P.pic_build_index([[40, 50]], [7], 2, 8, 2)  # G = 4, h_kv * 128 = 256
    hp = plan.host_ptr()
    bogus = np.zeros(64, dtype=np.int32)
    bp = bogus.ctypes.data_as(ctypes.c_void_p)
    f = ctypes.c_void_p(0x1000)
    ws = P.lib().pic_qkv_workspace_bytes(hp, 128)
    assert ws >= plan.n_rows * 64 * 8 and L.pic_qkv_workspace_bytes(bp, 128) == 0
    qkv = lambda *a: L.pic_qkv_rope(*a)
    ok = (hp, f, f, f, f, f, f, P.PIC_BF16, 256, 128, 0, 1e4, f, ws, None)
    def with_(i, v):
        a = list(ok)
        a[i] = v
        return qkv(*a)
    assert with_(0, bp) == P.PIC_EINVAL                 # not a plan
    assert with_(7, 9) == P.PIC_EINVAL                  # dtype
    assert with_(7, P.PIC_F32) == P.PIC_EUNSUPPORTED    # the GEMMs are bf16
    assert with_(9, 96) == P.PIC_EUNSUPPORTED           # head_dim
    assert with_(8, 200) == P.PIC_EUNSUPPORTED          # d_model % 64
    assert with_(10, 3) == P.PIC_EINVAL                 # layout
    assert with_(11, 0.0) == P.PIC_EINVAL               # base
    assert with_(2, None) == P.PIC_EINVAL               # x
    assert with_(12, None) == P.PIC_EINVAL              # workspace
    assert with_(13, ws - 1) == P.PIC_ENOSPC
    small = P.pic_build_index([[40, 50]], [7], 2, 1, 1)  # h_q * 64 = 64: not whole tiles
    assert L.pic_qkv_rope(small.host_ptr(), f, f, f, f, f, f, P.PIC_BF16, 256, 64, 0, 1e4, f,
                          ws, None) == P.PIC_EUNSUPPORTED
    assert L.pic_out_proj(hp, f, f, f, P.PIC_BF16, 192, 128, None) == P.PIC_EUNSUPPORTED
    assert L.pic_out_proj(hp, None, f, f, P.PIC_BF16, 256, 128, None) == P.PIC_EINVAL
    assert L.pic_out_proj(bp, f, f, f, P.PIC_BF16, 256, 128, None) == P.PIC_EINVAL
    # pic_link: a bad layer pointer or short workspace is refused before any launch
    arr = (ctypes.c_void_p * 2)(0x1000, 0x1000)
    bad = (ctypes.c_void_p * 2)(0x1000, None)
    lws = L.pic_link_workspace_bytes(hp, 128)
    assert lws >= ws
    link = lambda wq, wsz, dt=P.PIC_BF16, sc=0.088: L.pic_link(
        hp, f, 2, f, wq, arr, arr, arr, f, f, f, f, dt, 256, 128, 0, 1e4, sc, f, wsz, None)
    assert link(bad, lws) == P.PIC_EINVAL
    assert link(arr, lws - 1) == P.PIC_ENOSPC
    assert link(arr, lws, dt=P.PIC_F32) == P.PIC_EUNSUPPORTED
    assert link(arr, lws, sc=float("nan")) == P.PIC_EINVAL
    paged = P.pic_build_index([[40, 50]], [7], 2, 8, 2, chunk_ids_per_req=[[0, 1]])
    assert L.pic_link(paged.host_ptr(), f, 2, f, arr, arr, arr, arr, f, f, f, f, P.PIC_BF16, 256,
                      128, 0, 1e4, 0.088, f, lws, None) == P.PIC_EINVAL


# ---------------------------------------------------------------------------
# Planner vs oracle
# ---------------------------------------------------------------------------


def check_plan(reqs, q_lens, k, h_q, h_kv, pos_base=0, n_cu=0):
    plan = P.pic_build_index(reqs, q_lens, k, h_q, h_kv, pos_base=pos_base, n_cu=n_cu)
    group = h_q // h_kv
    # index, offsets and pointers: bit-exact against the oracle
    exp_rows, exp_off, exp_tok, exp_rowptr = [], [], [0], [0]
    for lens, q in zip(reqs, q_lens):
        rows = O.recompute_positions(lens, q, k)
        offs = O.chunk_offsets(lens)
        exp_rows.append(rows)
        exp_off += offs
        exp_tok.append(exp_tok[-1] + offs[-1] + q)
        exp_rowptr.append(exp_rowptr[-1] + len(rows))
    flat_rows = [r for rr in exp_rows for r in rr]
    assert plan.rows.tolist() == flat_rows
    assert plan.chunk_off.tolist() == exp_off
    assert plan.req_tok_ptr.tolist() == exp_tok
    assert plan.req_row_ptr.tolist() == exp_rowptr
    assert plan.row_tok.tolist() == [exp_tok[b] + r for b, rr in enumerate(exp_rows) for r in rr]
    assert plan.n_tokens == exp_tok[-1] and plan.n_rows == len(flat_rows)

    # rope tiles: exactly the cached rows that keep their K, each with delta = off_c -
    # pos_base and its global position (rows of one tile are consecutive in one chunk)
    want = {}
    for b, (lens, q) in enumerate(zip(reqs, q_lens)):
        offs = O.chunk_offsets(lens)
        rec = set(exp_rows[b])
        for c, L_c in enumerate(lens):
            delta = offs[c] - pos_base
            for t in range(L_c):
                if offs[c] + t not in rec:
                    want[exp_tok[b] + offs[c] + t] = (delta, offs[c] + t)
    got = {}
    for tok0, n, delta, pos0 in plan.rope_tiles.tolist():
        assert 1 <= n <= 32
        for i, t in enumerate(range(tok0, tok0 + n)):
            assert t not in got
            got[t] = (delta, pos0 + i)
    assert got == want

    # attention tiles: every (row, head) once; items cover [0, p_last] of each tile
    tile_rows = P.PIC_ATTN_TILE_M // group
    seen = set()
    for ti, (req, r0, n, tokb, pf, pl, _, _) in enumerate(plan.attn_tiles.tolist()):
        assert 1 <= n <= tile_rows and tokb == exp_tok[req]
        assert exp_rowptr[req] <= r0 and r0 + n <= exp_rowptr[req + 1]
        assert pf == flat_rows[r0] and pl == flat_rows[r0 + n - 1]
        for r in range(r0, r0 + n):
            assert r not in seen
            seen.add(r)
    assert seen == set(range(len(flat_rows)))
    cover = {}
    slots = set()
    for tile, g, kb, ke, slot, _, _, _ in plan.attn_items.tolist():
        assert 0 <= g < h_kv and 0 <= kb < ke
        cover.setdefault((tile, g), []).append((kb, ke, slot))
        if slot >= 0:
            assert slot not in slots
            slots.add(slot)
    tiles = plan.attn_tiles.tolist()
    for ti in range(len(tiles)):
        for g in range(h_kv):
            ranges = sorted(cover[(ti, g)])
            assert ranges[0][0] == 0 and ranges[-1][1] == tiles[ti][5] + 1
            for (a0, a1, _), (b0, b1, _) in zip(ranges, ranges[1:]):
                assert a1 == b0
            if len(ranges) == 1:
                assert ranges[0][2] == -1
            else:
                assert all(s >= 0 for _, _, s in ranges)
    merges = plan.merges.tolist()
    assert len(merges) == sum(1 for v in cover.values() if len(v) > 1)
    for tile, g, base, n in merges:
        assert sorted(s for _, _, s in cover[(tile, g)]) == list(range(base, base + n))
    assert plan[P.H_N_PARTIALS] == len(slots)
    # dispatch order: items of one (request, kv head) stream run segment by segment
    streams = {}
    for tile, g, kb, ke, _, _, _, _ in plan.attn_items.tolist():
        streams.setdefault((tiles[tile][0], g), []).append(kb)
    for begins in streams.values():
        assert begins == sorted(begins)
    return plan


def test_plan_worked_example():
    plan = check_plan([[4, 5, 5]], [3], 2, 4, 4)
    assert plan.rows.tolist() == [4, 5, 9, 10, 14, 15, 16]


def test_plan_exhaustive_small_grids():
    for n in range(1, 4):
        for lens in itertools.product(range(0, 5), repeat=n):
            for q in range(0, 3):
                for k in (0, 1, 2, 5):
                    check_plan([list(lens)], [q], k, 4, 2)


def test_plan_multi_request_and_pos_base():
    check_plan([[3, 0, 4], [5], [2, 2, 2, 2], []], [2, 0, 3, 4], 1, 8, 2)
    check_plan([[4, 5, 5], [7, 1]], [3, 2], 0, 4, 4, pos_base=4)
    check_plan([[4, 5, 5]], [3], 2, 4, 4, pos_base=-3)


@pytest.mark.parametrize("k", [2, 16])
def test_plan_long_context_splits(k):
    plan = check_plan([[1024] * 32], [128], k, 32, 8)
    assert plan[P.H_N_MERGE] > 0  # a few hundred rows need split-KV to fill the GPU


def test_plan_epic_sweep_sizes():
    from position_independent_kv_rope_amd import workloads as W
    wl = W.epic_sweep(k=16)
    check_plan([r.chunk_lens for r in wl.requests], [r.q_len for r in wl.requests], 16, 32, 8)


@settings(max_examples=60, deadline=None)
@given(st.lists(st.lists(st.integers(0, 300), min_size=0, max_size=12), min_size=1, max_size=4),
       st.lists(st.integers(0, 70), min_size=4, max_size=4), st.integers(0, 20),
       st.sampled_from([(32, 8), (32, 4), (4, 4), (8, 1), (16, 16)]), st.integers(-5, 5))
def test_plan_property(reqs, qs, k, heads, pos_base):
    check_plan(reqs, qs[:len(reqs)], k, heads[0], heads[1], pos_base=pos_base, n_cu=8)


# ---------------------------------------------------------------------------
# Paged plans (shared chunk pool)
# ---------------------------------------------------------------------------


def check_paged_plan(reqs, ids, q_lens, k, h_q, h_kv, pos_base=0, n_cu=0):
    plan = P.pic_build_index(reqs, q_lens, k, h_q, h_kv, pos_base=pos_base, n_cu=n_cu,
                             chunk_ids_per_req=ids)
    assert plan.paged and plan[P.H_N_ROPE_TILES] == 0
    flat_rows = [r for lens, q in zip(reqs, q_lens) for r in O.recompute_positions(lens, q, k)]
    assert plan.rows.tolist() == flat_rows
    segs = plan.segments.tolist()
    kb = plan.kblocks.tolist()
    c = 0
    req_row_ptr = plan.req_row_ptr.tolist()
    for b, (lens, q) in enumerate(zip(reqs, q_lens)):
        offs = O.chunk_offsets(lens)
        for j, L in enumerate(lens):
            off, ln, seam, cid, delta, req = segs[c][:6]
            assert (off, ln, req, cid) == (offs[j], L, b, ids[b][j])
            assert seam == (0 if j == 0 else min(k, L)) and delta == offs[j] - pos_base
            c += 1
    # every key a request can see is covered exactly once: fresh rows by fresh blocks,
    # pool rows t >= n_seam by pool blocks (blocks may also hold masked keys)
    for b, (lens, q) in enumerate(zip(reqs, q_lens)):
        n_fresh = req_row_ptr[b + 1] - req_row_ptr[b]
        fresh_cov, pool_cov = [], []
        c0 = sum(len(r) for r in reqs[:b])
        for chunk, t0, first_pos, _ in kb:
            if chunk == -1:
                continue
            if segs[chunk][5] == b:
                off, ln, seam = segs[chunk][:3]
                assert first_pos == off + t0
                pool_cov += [off + t for t in range(t0, min(t0 + 64, ln)) if t >= seam]
        rows_b = flat_rows[req_row_ptr[b]:req_row_ptr[b + 1]]
        want_pool = [p for p in range(sum(lens)) if p not in set(rows_b)]
        assert sorted(pool_cov) == want_pool
    # items: per (tile, head) the block ranges cover the needed fresh and pool blocks
    tiles = plan.attn_tiles.tolist()
    for tile, g, b1, e1, slot, b2, e2, _ in plan.attn_items.tolist():
        assert 0 <= b1 <= e1 and 0 <= b2 <= e2
        for i in list(range(b1, e1)) + list(range(b2, e2)):
            assert kb[i][2] <= tiles[tile][5]  # no block starts after the tile's last row
    # decode items: every request chunk with keys is one use of exactly one item of its
    # pool chunk (at most PIC_DECODE_COLS / G uses, all of the chunk's keys), and every
    # request with fresh rows has one item of its own
    group = h_q // h_kv
    B = P.PIC_DECODE_BLOCK
    items, uses = plan.dec_items.tolist(), plan.dec_uses.tolist()
    n_chunks = plan[P.H_N_CHUNKS]
    assert plan[P.H_N_DEC_USES] == len(uses)
    flat_lens = [x for lens in reqs for x in lens]
    flat_ids = [x for c in ids for x in c]
    n_fresh = [int(plan.req_row_ptr[b + 1] - plan.req_row_ptr[b]) for b in range(len(reqs))]
    use_req = [segs[c][5] if c >= 0 else -1 - c for c in uses]
    seen, fresh = [], []
    for src, n_keys, u0, nu in items:
        assert 1 <= nu <= P.PIC_DECODE_COLS // group
        us = uses[u0:u0 + nu]
        if src >= 0:
            assert all(flat_ids[c] == src and flat_lens[c] == n_keys > 0 for c in us)
            seen += us
        else:
            assert us == [src] and n_keys == n_fresh[-1 - src] > 0
            fresh.append(-1 - src)
    assert sorted(seen) == [c for c, L in enumerate(flat_lens) if L > 0]
    assert fresh == [b for b in range(len(reqs)) if n_fresh[b] > 0]
    # pieces: the (item, kv head) units, in order, cut into B-key blocks; the block
    # sequence split into n_wg equal runs (min(blocks, n_cu * PIC_DECODE_WG_PER_CU) of
    # them); a piece is a unit's part of one run, and it writes one record per use
    pieces, wp = plan.dec_pieces.tolist(), plan.dec_wg_ptr.tolist()
    precs, rp = plan.dec_piece_recs.tolist(), plan.dec_rec_ptr.tolist()
    units = [(i, g, n_keys) for i, (_, n_keys, _, _) in enumerate(items) for g in range(h_kv)]
    total = sum((n + B - 1) // B for _, _, n in units)
    n_wg = plan[P.H_N_DEC_WG]
    assert n_wg == min(total, (n_cu if n_cu > 0 else 256) * P.PIC_DECODE_WG_PER_CU)
    if total == 0:
        assert pieces == [] and rp[-1] == 0
        return plan
    assert wp[0] == 0 and wp[-1] == len(pieces) and len(wp) == n_wg + 1
    cover = {}  # (item, g) -> blocks in piece order
    for w in range(n_wg):
        assert wp[w] < wp[w + 1]  # no idle workgroup
        run = 0
        for it, g, t0, t1, off, _, _, _ in pieces[wp[w]:wp[w + 1]]:
            n_keys = items[it][1]
            assert t0 % B == 0 and t0 < t1 and (t1 % B == 0 or t1 == n_keys) and t1 <= n_keys
            cover.setdefault((it, g), []).append((t0, t1))
            run += (t1 - t0 + B - 1) // B
        assert run in (total // n_wg, (total + n_wg - 1) // n_wg)
    for it, g, n_keys in units:  # each unit's pieces tile its keys in order
        spans = cover.pop((it, g))
        assert spans[0][0] == 0 and spans[-1][1] == n_keys
        assert all(a[1] == b[0] for a, b in zip(spans, spans[1:]))
    assert not cover
    # records: ids of (request b, kv head g) are the contiguous run [rp[b*h_kv+g], ..+1)
    assert rp[0] == 0 and rp == sorted(rp) and rp[-1] == plan[P.H_N_DEC_RECS]
    got = []
    for it, g, t0, t1, off, _, _, _ in pieces:
        _, _, u0, nu = items[it]
        for u in range(nu):
            b = use_req[u0 + u]
            r = precs[off + u]
            assert rp[b * h_kv + g] <= r < rp[b * h_kv + g + 1]
            got.append(r)
    assert sorted(got) == list(range(rp[-1]))
    return plan


def check_paged_tail_cut(reqs, ids, q_lens, k, h_q, h_kv, n_cu=256, tail_blocks=64):
    """Paged plans: every item's first range is pool blocks and its second range (only
    on a tile's first item) the request's fresh blocks; the final round of each die --
    its last 2 * n_cu / 8 items, workgroup i running on die i % 8 -- holds pieces of at
    most tail_blocks pool blocks (4,096 keys): the last-round cut acts on the pool range,
    and the fresh blocks stay with one piece."""
    plan = P.pic_build_index(reqs, q_lens, k, h_q, h_kv, n_cu=n_cu, chunk_ids_per_req=ids)
    items = plan.attn_items.tolist()
    kb = plan.kblocks.tolist()
    slots_per_die = 2 * n_cu // 8
    for _, _, b1, e1, _, b2, e2, _ in items:
        assert all(kb[i][0] >= 0 for i in range(b1, e1))   # first range: pool blocks
        assert all(kb[i][0] == -1 for i in range(b2, e2))  # second range: fresh blocks
    for d in range(8):
        for _, _, b1, e1, _, _, _, _ in items[d::8][-slots_per_die:]:
            assert e1 - b1 <= tail_blocks, (d, b1, e1)
    return plan


def test_paged_plan_tail_cut_acts_on_pool_blocks():
    # the shared-pool shape: 8 requests x 96-128 chunks of 512-1536 tokens
    rng = np.random.default_rng(11)
    pool = [int(x) for x in rng.integers(512, 1537, size=256)]
    ids = [[int(x) for x in rng.permutation(256)[:int(rng.integers(96, 129))]] for _ in range(8)]
    check_paged_tail_cut([[pool[i] for i in r] for r in ids], ids, [128] * 8, 8, 32, 4)
    # 64 requests of 8 x 1024 tokens: one 8,192-key range per tile, so every item is a
    # tile's first item (pool range plus fresh blocks) and the cut must shorten those
    ids = [[int(x) for x in rng.permutation(96)[:8]] for _ in range(64)]
    plan = check_paged_tail_cut([[1024] * 8 for _ in ids], ids, [128] * 64, 8, 32, 4)
    items = plan.attn_items.tolist()
    with_fresh = [(t, g) for t, g, _, _, _, b2, e2, _ in items if e2 > b2]
    assert sorted(with_fresh) == sorted(set((t, g) for t, g, *_ in items))  # one per tile+head
    assert max(e1 - b1 for _, _, b1, e1, *_ in items) == 128  # uncut items before the tail


def test_paged_plan_small():
    check_paged_plan([[37, 64, 5, 130], [130, 70]], [[3, 0, 7, 2], [2, 5]], [9, 4], 8, 32, 4)
    # one pool chunk read twice by one request, and by two requests
    check_paged_plan([[16, 3, 16, 64], [64, 16]], [[0, 1, 0, 3], [3, 0]], [7, 0], 8, 8, 2)
    check_paged_plan([[4, 5, 5]], [[0, 1, 2]], [3], 2, 4, 4, pos_base=3)
    # long chunks and fresh rows over a grid of few workgroups (runs cut inside units),
    # a chunk of exactly a whole number of blocks
    check_paged_plan([[300, 600, 256], [600, 10]], [[0, 1, 2], [1, 3]], [300, 0], 8, 16, 2,
                     n_cu=3)


def test_paged_plan_shared_pool_workload():
    from position_independent_kv_rope_amd import workloads as W
    wl = W.shared_pool()
    check_paged_plan([r.chunk_lens for r in wl.requests], [r.chunk_ids for r in wl.requests],
                     [r.q_len for r in wl.requests], wl.k, wl.h_q, wl.h_kv, n_cu=256)


def test_paged_plan_rejects_negative_ids():
    with pytest.raises(P.PicError):
        P.pic_build_index([[4, 5]], [1], 2, 4, 4, chunk_ids_per_req=[[0, -1]])


def test_paged_plan_rejects_inconsistent_chunk_lengths():
    # a pool chunk has one length wherever it is used
    with pytest.raises(P.PicError):
        P.pic_build_index([[4, 5], [6]], [1, 1], 2, 4, 4, chunk_ids_per_req=[[0, 1], [1]])


def test_bench_refuses_more_than_one_gpu():
    # the bench measures one GPU; asked for more it says so and exits non-zero, before
    # touching a device
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_split_length_fills_whole_rounds_of_slots():
    # small batches: the split segment is a half or a third of a fair share per workgroup
    # slot (>= 1024 keys), whichever packs the item count closer to whole rounds of the
    # 2 x n_cu slots; large batches keep the 8192-key segments
    from position_independent_kv_rope_amd import workloads as W

    def items(wl):
        p = P.pic_build_index([r.chunk_lens for r in wl.requests], [r.q_len for r in wl.requests],
                              wl.k, wl.h_q, wl.h_kv, n_cu=256)
        return p[P.H_N_ATTN_ITEMS], p[P.H_N_MERGE]

    n2, m2 = items(W.long_context(k=2))      # 6 tiles x 8 kv heads over 32,896 keys
    n16, m16 = items(W.long_context(k=16))   # 20 tiles x 8 kv heads
    assert (n2, m2) == (1016, 48)      # half share: 1,016 items = 1.98 rounds of 512
    assert (n16, m16) == (1600, 152)   # third share: 3.1 rounds (half share: 2.16)
    assert items(W.epic_sweep(k=16))[0] == 4600  # 8192-key segments, tail cut
