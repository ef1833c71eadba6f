"""Run the host planner's checks against an AddressSanitizer + UndefinedBehaviorSanitizer
build of pic_plan.cpp (CPU only).

Usage: python tests/plan_sanitized_driver.py <libpic_plan_san.so>

Started by tests/test_plan_sanitized.py with the sanitizer runtimes preloaded.  The
binding's library handle is replaced by the sanitized planner-only library (it exports
pic_build_index and pic_strerror, nothing that launches a kernel), then the planner
checks of test_abi_and_plan.py run against it: the worked example, exhaustive small
grids, error paths, the long-context and EPIC-scale sizes, paged plans, and hypothesis
searches over random batches (contiguous and paged).  Any sanitizer report aborts the
process with a non-zero status.
"""

import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import position_independent_kv_rope_amd as P  # noqa: E402


def load(path):
    L = ctypes.CDLL(path)
    i32, i64, p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    L.pic_build_index.argtypes = [i32, p, p, p, p, i32, i32, i32, i32, i32, p, i64,
                                  ctypes.POINTER(i64)]
    L.pic_build_index.restype = ctypes.c_int
    L.pic_strerror.argtypes = [ctypes.c_int]
    L.pic_strerror.restype = ctypes.c_char_p
    return L


def epic_like(rng, n_req, lo, hi, target, q):
    reqs = []
    for _ in range(n_req):
        lens = []
        while sum(lens) < target:
            lens.append(int(rng.integers(lo, hi + 1)))
        reqs.append(lens)
    return reqs, [q] * n_req


def pool_like(rng, n_pool, n_req, m_lo, m_hi):
    pool = [int(x) for x in rng.integers(512, 1537, size=n_pool)]
    lens, ids = [], []
    for _ in range(n_req):
        m = int(rng.integers(m_lo, m_hi + 1))
        c = [int(x) for x in rng.permutation(n_pool)[:m]]
        ids.append(c)
        lens.append([pool[i] for i in c])
    return lens, ids


def main():
    P._lib = load(sys.argv[1])
    import test_abi_and_plan as T
    from hypothesis import given, settings, strategies as st

    T.test_strerror_and_status_codes()
    T.test_build_index_error_paths()
    T.test_plan_worked_example()
    T.test_plan_exhaustive_small_grids()
    T.test_plan_multi_request_and_pos_base()
    for k in (0, 2, 16):
        T.check_plan([[1024] * 32], [128], k, 32, 8, n_cu=256)
    rng = np.random.default_rng(2024)
    for k in (2, 4, 8, 16):  # EPIC-scale batches: 4 x ~50k tokens of 512-2048-token chunks
        reqs, qs = epic_like(rng, 4, 512, 2048, 50000, 256)
        T.check_plan(reqs, qs, k, 32, 8, n_cu=256)
    T.test_paged_plan_small()
    T.test_paged_plan_rejects_negative_ids()
    T.test_paged_plan_rejects_inconsistent_chunk_lengths()
    lens, ids = pool_like(rng, 256, 8, 96, 128)  # the shared-pool batch's shape
    T.check_paged_plan(lens, ids, [128] * 8, 8, 32, 4, n_cu=256)
    T.check_paged_tail_cut(lens, ids, [128] * 8, 8, 32, 4, n_cu=256)

    @settings(max_examples=300, deadline=None, database=None)
    @given(st.lists(st.lists(st.integers(0, 400), min_size=0, max_size=14), min_size=1,
                    max_size=5),
           st.lists(st.integers(0, 90), min_size=5, max_size=5), st.integers(0, 24),
           st.sampled_from([(32, 8), (32, 4), (4, 4), (8, 1), (16, 16), (64, 8)]),
           st.integers(-6, 6), st.sampled_from([1, 3, 8, 256]))
    def contiguous(reqs, qs, k, heads, pos_base, n_cu):
        T.check_plan(reqs, qs[:len(reqs)], k, heads[0], heads[1], pos_base=pos_base, n_cu=n_cu)

    @settings(max_examples=150, deadline=None, database=None)
    @given(st.lists(st.integers(1, 700), min_size=1, max_size=9),
           st.lists(st.lists(st.integers(0, 8), min_size=0, max_size=6), min_size=1,
                    max_size=4),
           st.lists(st.integers(0, 70), min_size=4, max_size=4), st.integers(0, 12),
           st.sampled_from([(32, 8), (32, 4), (8, 2), (4, 4)]), st.integers(-4, 4),
           st.sampled_from([2, 5, 64]))
    def paged(pool, picks, qs, k, heads, pos_base, n_cu):
        ids = [[i % len(pool) for i in req] for req in picks]
        lens = [[pool[i] for i in req] for req in ids]
        T.check_paged_plan(lens, ids, qs[:len(ids)], k, heads[0], heads[1], pos_base=pos_base,
                           n_cu=n_cu)

    contiguous()
    paged()
    print("sanitized planner: ok", flush=True)


if __name__ == "__main__":
    main()
