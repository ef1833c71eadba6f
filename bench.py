"""Benchmark of the position-independent KV splicing hot path on one MI355X.

One step = one pass of the whole link path over one batch of synthetic requests:
host planner (recompute index + schedules) and plan upload, rotary correction of the
cached K, splice of the fresh rows, selective attention (+ split-KV merge).  Inputs
are resident in HBM before the timed region.  The planner of step i+1 runs on the host
while the GPU executes step i (pinned, double-buffered, asynchronous plan upload).
Prints ONE JSON line.

Default workload: 4 independent requests of ~50k tokens each (chunks of 512-2048
tokens, 256 query tokens), GQA 32/8, head_dim 128, bf16, k = 16.  The default run also
measures the other configurations of the same path and adds them to the one line as
"sub_records", each with its own roofline and a bounded cpu_baseline: the same batch
shape at k = 2, 4, 8; one 32,896-token request (32 chunks of 1024 + 128 query tokens)
at k = 2 and 16; and the shared-pool batch below.  Every contiguous record also times
the rotation + splice launch right after a 512 MB read that evicts the
Infinity Cache.

--workload shared_pool: 256 chunks stored once in a paged pool of 16-token blocks,
8 requests each splicing 96-128 of them (~116k tokens) + 128 query tokens, seam
window w = 8, GQA 32/4.  The pool is never rotated or written: one step is the
planner, the plan upload and pic_selective_attn_paged (rotation on load, fresh rows
read in place).  With --gather one step is instead the planner (a paged plan for the
gather, a contiguous plan for the attention), both uploads, pic_rope_splice_pool (pool
blocks -> contiguous rotated K/V with the fresh rows spliced in) and pic_selective_attn;
the default run adds it as the "shared_pool_gathered_k8" sub-record.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "spliced context tokens/s + selective-attn TFLOP/s (1 GPU, % of roofline)"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
CSRC = "position_independent_kv_rope_amd/csrc/"
ATTN_SOURCES = [CSRC + "pic_attn.hip", CSRC + "pic_attn_common.h"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="epic_sweep",
                    choices=["rag_single", "long_context", "epic_sweep", "shared_pool"])
    ap.add_argument("--k", type=int, default=None,
                    help="recompute count (default 16; the seam window 8 for shared_pool)")
    ap.add_argument("--rope-scheme", default="delta", choices=["delta", "nope"],
                    help="delta: cached K carries RoPE at local positions and is rotated by "
                         "delta (pic_rope_delta); nope: cached K is position-free and gets "
                         "RoPE at the target positions (pic_rope_apply)")
    ap.add_argument("--decode", action="store_true",
                    help="shared_pool only: time one decode step of every request "
                         "(pic_decode_attn_paged) instead of the link")
    ap.add_argument("--graph", action="store_true",
                    help="with --decode: capture the step's launches in a HIP graph once "
                         "(the plan is fixed) and replay it every step")
    ap.add_argument("--link-layers", type=int, default=0,
                    help="contiguous workloads: time the whole multi-layer link (pic_link: "
                         "per layer rope-delta, compute_qkv, splice, attention, output "
                         "projection) of a random model with this many layers")
    ap.add_argument("--d-model", type=int, default=0,
                    help="model width for --link-layers (default h_q * head_dim)")
    ap.add_argument("--state-compose", action="store_true",
                    help="shared_pool only: time the linear-layer state composition over "
                         "every request's chunks (pic_state_compose), --heads heads")
    ap.add_argument("--heads", type=int, default=32,
                    help="linear-attention heads for --state-compose")
    ap.add_argument("--gather", action="store_true",
                    help="shared_pool only: gather the pool chunks into contiguous K/V "
                         "(pic_rope_splice_pool), then pic_selective_attn")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub-records", action="store_true",
                    help="default workload only: skip the sub-records of the other "
                         "configurations (k sweep, 32k-token request, shared pool)")
    ap.add_argument("--cpu-sample-rows", type=int, default=0,
                    help="recomputed rows per request whose attention the oracle times "
                         "(0 = all; the time is scaled to all rows by causal-pair count)")
    ap.add_argument("--peaks-only", action="store_true",
                    help="run only the measured peaks (calibration streams, MFMA loop, "
                         "vendor GEMM) and print them as one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (5 launches) to calibrate "
                         "rocprofv3 FETCH_SIZE/WRITE_SIZE against known bytes")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)


def calib_lib():
    """libpic_calib.so (include/pic_calib.h): streaming read/copy and MFMA-loop kernels."""
    import ctypes
    path = os.path.join(ROOT, "position_independent_kv_rope_amd", "libpic_calib.so")
    if not os.path.exists(path):
        raise RuntimeError("libpic_calib.so not found at %s; build it with "
                           "`python -m position_independent_kv_rope_amd.build`" % path)
    L = ctypes.CDLL(path)
    i32, i64, p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    L.pic_calib_read_sink_words.argtypes = [i64]
    L.pic_calib_read_sink_words.restype = i64
    L.pic_calib_read.argtypes = [p, i64, p, p]
    L.pic_calib_read.restype = ctypes.c_int
    L.pic_calib_copy.argtypes = [p, p, i64, p]
    L.pic_calib_copy.restype = ctypes.c_int
    L.pic_calib_update.argtypes = [p, i64, p]
    L.pic_calib_update.restype = ctypes.c_int
    L.pic_calib_mfma_flops.argtypes = [i32, i32]
    L.pic_calib_mfma_flops.restype = i64
    L.pic_calib_mfma.argtypes = [p, p, i32, i32, p]
    L.pic_calib_mfma.restype = ctypes.c_int
    return L


def measured_peaks():
    """Rates this GPU reaches, measured live (context for the spec-peak fractions, never
    the denominator of `frac`): with the calibration kernels a plain streaming read of
    2 GiB, a 1 GiB copy and a 1 GiB in-place update (read + write bytes), and an MFMA
    loop on random bf16 operands (v_mfma_f32_32x32x16_bf16, two waves per SIMD); and an
    8192^3 bf16 GEMM of random operands through the vendor BLAS."""
    import torch
    dev = "cuda"
    C = calib_lib()
    stream = lambda: ctypes_stream(torch)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    def ok(st, name):
        if st != 0:
            raise RuntimeError("%s failed: %d" % (name, st))

    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: ok(C.pic_calib_copy(src.data_ptr(), dst.data_ptr(), n, stream()),
                              "pic_calib_copy"), 10)
    t_update = timed(lambda: ok(C.pic_calib_update(src.data_ptr(), n, stream()),
                                "pic_calib_update"), 10)
    del dst, src
    big = torch.ones(n // 2, dtype=torch.float32, device=dev)
    sink = torch.empty(int(C.pic_calib_read_sink_words(2 * n)), dtype=torch.int32, device=dev)
    t_read = timed(lambda: ok(C.pic_calib_read(big.data_ptr(), 2 * n, sink.data_ptr(), stream()),
                              "pic_calib_read"), 10)
    del big, sink
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    n_wg, iters = 2 * n_cu, 4096
    g = torch.Generator(device="cpu").manual_seed(7)
    ops = torch.randn(8 * 64 * 8, generator=g).to(torch.bfloat16).to(dev)
    fsink = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)
    t_mfma = timed(lambda: ok(C.pic_calib_mfma(ops.data_ptr(), fsink.data_ptr(), n_wg, iters,
                                               stream()), "pic_calib_mfma"), 10)
    mfma_flops = float(C.pic_calib_mfma_flops(n_wg, iters))
    del ops, fsink
    m = 8192
    a = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
    b = torch.randn(m, m, dtype=torch.bfloat16, device=dev)
    t_gemm = timed(lambda: torch.matmul(a, b), 10)
    del a, b
    torch.cuda.empty_cache()
    return {"read_GB_s": round(2 * n / t_read / 1e9, 1),
            "copy_GB_s": round(2 * n / t_copy / 1e9, 1),
            "update_GB_s": round(2 * n / t_update / 1e9, 1),
            "mfma_loop_bf16_TFLOP_s": round(mfma_flops / t_mfma / 1e12, 1),
            "gemm_bf16_TFLOP_s": round(2.0 * m ** 3 / t_gemm / 1e12, 1),
            "how": ("libpic_calib.so: streaming read of 2 GiB, copy of 1 GiB and in-place "
                    "update of 1 GiB (read + write bytes), MFMA loop (%d workgroups x 4 waves "
                    "x %d rounds of 4 v_mfma_f32_32x32x16_bf16 on random operands); vendor "
                    "BLAS: torch.matmul 8192^3 bf16 with random operands; 10 launches each, "
                    "HIP events" % (n_wg, iters))}


def ctypes_stream(torch):
    return torch.cuda.current_stream().cuda_stream


def with_measured(rec, peaks):
    """Add fractions of the measured rates next to the spec fractions: MFMA-bound records
    against the MFMA loop and the vendor GEMM, HBM-bound ones against the streaming read
    (a read-dominated call) and every HBM-bound kernel entry against the in-place update
    (the rotation reads and writes its rows in place; the splice and the pool gather
    write rows they did not read, for which the copy rate is given as well)."""
    if not peaks:
        return rec
    roof = rec.get("roofline", {})
    if roof.get("unit") == "TFLOP/s" and rec.get("dtype") == "bf16":
        roof["frac_of_measured_mfma"] = round(roof["achieved"] / peaks["mfma_loop_bf16_TFLOP_s"], 4)
        roof["frac_of_measured_gemm"] = round(roof["achieved"] / peaks["gemm_bf16_TFLOP_s"], 4)
    elif roof.get("unit") == "GB/s":
        roof["frac_of_measured_read"] = round(roof["achieved"] / peaks["read_GB_s"], 4)
    for kr in rec.get("kernels", {}).values():
        if isinstance(kr, dict) and "GB_s" in kr and "hbm_frac" in kr:
            kr["frac_of_measured_update"] = round(kr["GB_s"] / peaks["update_GB_s"], 4)
            kr["frac_of_measured_copy"] = round(kr["GB_s"] / peaks["copy_GB_s"], 4)
    return rec


def make_workload(name, k):
    from position_independent_kv_rope_amd import workloads as W
    if name == "shared_pool":
        return W.shared_pool(w=8 if k is None else k)
    k = 16 if k is None else k
    if name == "rag_single":
        wl = W.rag_single()
        wl.k = k
        return wl
    if name == "long_context":
        return W.long_context(k=k)
    return W.epic_sweep(k=k)


def pct(times_ms):
    """p50 / p95 of per-step event times (ms)."""
    t = np.asarray(times_ms, dtype=np.float64)
    return {"p50_ms": round(float(np.percentile(t, 50)), 4),
            "p95_ms": round(float(np.percentile(t, 95)), 4)}


def load_traffic(kernel, workload, sources=None):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from position_independent_kv_rope_amd.profiling import src_hash
    if rec.get("source_hash") != src_hash(rec.get("sources", sources or ATTN_SOURCES)):
        return None
    return rec.get("bytes_per_launch")


class PlanUploader:
    """Host planner output -> device plan, pipelined: the plan words go through one of two
    pinned host buffers and are copied asynchronously on the compute stream, so the host
    plans step i+1 while the GPU still runs step i and the GPU runs the kernels of a step
    back to back (the events around each call then time GPU work only).  A buffer is
    reused only after the copy that read it has completed."""

    def __init__(self, n_words, device):
        import torch
        self.torch = torch
        self.dev = torch.empty(n_words, dtype=torch.int32, device=device)
        self.host = [torch.empty(n_words, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.done = [None, None]
        self.i = 0

    def upload(self, plan):
        torch = self.torch
        b = self.i % 2
        self.i += 1
        if self.done[b] is not None:
            self.done[b].synchronize()
        n = plan.words.size
        if n > self.dev.numel():
            raise ValueError("plan grew beyond the preallocated device buffer")
        self.host[b].numpy()[:n] = plan.words
        self.dev[:n].copy_(self.host[b][:n], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        self.done[b] = ev
        plan.dev = self.dev
        return plan


def _threads():
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])


def _sample_rows(rows, n_att):
    """The last n_att rows (the longest ones) when sampling, else all of them."""
    return slice(len(rows) - n_att, len(rows)) if 0 < n_att < len(rows) else slice(0, len(rows))


def cpu_baseline(wl, k_in, v_in, q, kf, vf, plan, requests, sample_rows, scheme="delta"):
    """Time the CPU oracle (as it stands) on the given requests of the same inputs:
    index, rotation (or Scheme B), splice and selective attention.  With sample_rows > 0
    only the last sample_rows recomputed rows of each request attend, and the attention
    time is scaled to all rows by causal-pair count (flops)."""
    import torch
    from oracle import pic_oracle as O
    f64 = lambda t: t.to(torch.float64).numpy()
    t_meas = t_full = 0.0
    n_tokens = n_rows = n_att_rows = 0
    for b in requests:
        r = wl.requests[b]
        tok0 = int(plan.req_tok_ptr[b])
        row0, row1 = int(plan.req_row_ptr[b]), int(plan.req_row_ptr[b + 1])
        offs = O.chunk_offsets(r.chunk_lens)
        kin = f64(k_in[tok0:tok0 + offs[-1]])
        vin = f64(v_in[tok0:tok0 + offs[-1]])
        ck = [kin[offs[c]:offs[c + 1]] for c in range(len(r.chunk_lens))]
        cv = [vin[offs[c]:offs[c + 1]] for c in range(len(r.chunk_lens))]
        qb, kfb, vfb = f64(q[row0:row1]), f64(kf[row0:row1]), f64(vf[row0:row1])
        t0 = time.perf_counter()
        rows = O.recompute_positions(r.chunk_lens, r.q_len, wl.k)
        k_ctx = O.rope_apply(ck, wl.rope_base) if scheme == "nope" else O.rope_delta(ck, wl.rope_base)
        v_ctx = O.concat_chunks(cv)
        kx, vx = O.splice(k_ctx, v_ctx, kfb, vfb, rows, offs[-1] + r.q_len)
        t1 = time.perf_counter()
        sel = _sample_rows(rows, sample_rows)
        O.selective_attn(qb[sel], kx, vx, rows[sel])
        t2 = time.perf_counter()
        pairs = float(sum(p + 1 for p in rows))
        pairs_s = float(sum(p + 1 for p in rows[sel]))
        t_meas += t2 - t0
        t_full += (t1 - t0) + (t2 - t1) * (pairs / pairs_s if pairs_s else 1.0)
        n_tokens += offs[-1] + r.q_len
        n_rows += len(rows)
        n_att_rows += len(rows[sel])
    scaled = n_att_rows < n_rows
    return {"value": round(n_tokens / t_full, 1), "unit": "tokens/s", "cores": _threads(),
            "kind": "oracle", "seconds": round(t_meas, 3),
            "seconds_all_rows": round(t_full, 3),
            "sample": "%d of %d requests of the batch (%d tokens, %d recomputed rows%s), fp64 "
                      "NumPy oracle: index, %s, splice and selective attention"
                      % (len(requests), len(wl.requests), n_tokens, n_rows,
                         "; the last %d rows of each request attend and the attention time is "
                         "scaled to all %d rows by causal-pair count" % (sample_rows, n_rows)
                         if scaled else "", "RoPE at the target positions" if scheme == "nope"
                         else "rotation"),
            "host_cpus": os.cpu_count()}


def cpu_baseline_paged(wl, pk, pv, cbp, blocks, q, kf, vf, plan, sample_rows):
    """Time the CPU oracle (as it stands) on request 0 of the paged batch: gather of the
    request's chunks from the pool, rotation, splice and selective attention (the last
    sample_rows rows, the attention time scaled to all rows by causal-pair count)."""
    import torch
    from oracle import pic_oracle as O
    r = wl.requests[0]
    row0, row1 = int(plan.req_row_ptr[0]), int(plan.req_row_ptr[1])
    f64 = lambda t: t.to(torch.float64).numpy()
    qb, kfb, vfb = f64(q[row0:row1]), f64(kf[row0:row1]), f64(vf[row0:row1])
    # the request's pool blocks only (the rest of the pool is not part of its work)
    t0 = time.perf_counter()
    ck, cv = [], []
    for i in r.chunk_ids:
        ids = blocks[cbp[i]:cbp[i + 1]]
        sub = torch.from_numpy(ids.astype(np.int64))
        ck.append(O.gather_paged_chunk(f64(pk[sub]), np.arange(len(ids)), wl.pool_lens[i]))
        cv.append(O.gather_paged_chunk(f64(pv[sub]), np.arange(len(ids)), wl.pool_lens[i]))
    rows = O.recompute_positions(r.chunk_lens, r.q_len, wl.k)
    offs = O.chunk_offsets(r.chunk_lens)
    k_ctx = O.rope_delta(ck, wl.rope_base)
    v_ctx = O.concat_chunks(cv)
    kx, vx = O.splice(k_ctx, v_ctx, kfb, vfb, rows, offs[-1] + r.q_len)
    t1 = time.perf_counter()
    sel = _sample_rows(rows, sample_rows)
    O.selective_attn(qb[sel], kx, vx, rows[sel])
    t2 = time.perf_counter()
    pairs, pairs_s = float(sum(p + 1 for p in rows)), float(sum(p + 1 for p in rows[sel]))
    t_full = (t1 - t0) + (t2 - t1) * (pairs / pairs_s if pairs_s else 1.0)
    n_tokens = offs[-1] + r.q_len
    n_att = len(rows[sel])
    return {"value": round(n_tokens / t_full, 1), "unit": "tokens/s", "cores": _threads(),
            "kind": "oracle", "seconds": round(t2 - t0, 3),
            "seconds_all_rows": round(t_full, 3),
            "sample": "request 0 of the batch (%d tokens in %d pooled chunks, %d recomputed "
                      "rows%s), fp64 NumPy oracle: pool gather, index, rotation, splice and "
                      "selective attention"
                      % (n_tokens, len(r.chunk_ids), len(rows),
                         "; the last %d rows attend and the attention time is scaled to all "
                         "rows by causal-pair count" % n_att if n_att < len(rows) else ""),
            "host_cpus": os.cpu_count()}


def bench_paged(args, wl):
    run = run_pool_gathered if args.gather else run_paged
    peaks = measured_peaks()
    rec = with_measured(run(wl, args.steps, args.warmup,
                            None if args.no_cpu_baseline else args.cpu_sample_rows), peaks)
    rec["measured_peaks"] = peaks
    print(json.dumps(rec), flush=True)


def run_pool_gathered(wl, steps, warmup, cpu_sample_rows):
    """One step = planner (a paged plan with chunk ids for the gather, a contiguous plan of
    the same requests for the attention) + both uploads + pic_rope_splice_pool +
    pic_selective_attn over the shared-pool batch; returns the record."""
    import torch
    import position_independent_kv_rope_amd as P
    from position_independent_kv_rope_amd import workloads as W
    reqs = [r.chunk_lens for r in wl.requests]
    ids = [r.chunk_ids for r in wl.requests]
    qs = [r.q_len for r in wl.requests]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    plans = lambda: (P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, n_cu=n_cu,
                                       chunk_ids_per_req=ids),
                     P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, n_cu=n_cu))
    pplan, cplan = plans()
    cbp, blocks = W.pool_block_table(wl)
    pk_h, pv_h = W.pool_tensors(wl)
    q_h, kf_h, vf_h = W.fresh_tensors(wl, cplan.n_rows)
    dev = "cuda"
    pk, pv = pk_h.to(dev), pv_h.to(dev)
    cbp_d, blocks_d = torch.from_numpy(cbp).to(dev), torch.from_numpy(blocks).to(dev)
    q, kf, vf = q_h.to(dev), kf_h.to(dev), vf_h.to(dev)
    k = torch.empty((cplan.n_tokens, wl.h_kv, wl.head_dim), dtype=q.dtype, device=dev)
    v = torch.empty_like(k)
    out = torch.empty_like(q)
    ws = P.attn_workspace(cplan, wl.head_dim)
    up_p, up_c = PlanUploader(pplan.words.size, dev), PlanUploader(cplan.words.size, dev)
    torch.cuda.synchronize()

    s = wl.torch_dtype.itemsize
    D, hq, hkv = wl.head_dim, wl.h_q, wl.h_kv
    rows = cplan.rows.astype(np.int64)
    attn_flops = 4.0 * D * hq * float(np.sum(rows + 1))
    attn_bytes = 2.0 * s * hkv * D * cplan.n_tokens + 2.0 * s * hq * D * cplan.n_rows
    # the gather reads every context row of K and V from the pool and the fresh rows, and
    # writes every row of K and V once
    n_ctx = int(sum(sum(r.chunk_lens) for r in wl.requests))
    row_bytes = s * hkv * D
    gather_bytes = 2.0 * row_bytes * (n_ctx + cplan.n_rows) + 2.0 * row_bytes * cplan.n_tokens
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    plan_s = []

    def step(i=None):
        t0 = time.perf_counter()
        pp, cp = plans()
        plan_s.append(time.perf_counter() - t0)
        up_p.upload(pp)
        up_c.upload(cp)
        e = ev[i] if i is not None else None
        if e: e[0].record()
        P.pic_rope_splice_pool(pp, pk, pv, cbp_d, blocks_d, k, v, kf, vf, wl.rope_base)
        if e: e[1].record()
        P.pic_selective_attn(cp, q, k, v, out, workspace=ws)
        if e: e[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / steps
    l_g = [e[0].elapsed_time(e[1]) for e in ev]
    l_attn = [e[1].elapsed_time(e[2]) for e in ev]
    t_g, t_attn = float(np.mean(l_g)), float(np.mean(l_attn))
    tokens = cplan.n_tokens
    attn_tflops = attn_flops / (t_attn * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[wl.dtype]
    rec = {
        "metric": METRIC,
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": "shared_pool (gathered)", "requests": len(wl.requests),
                   "tokens": tokens, "pool_chunks": len(wl.pool_lens),
                   "pool_blocks": int(blocks.size), "block_size": wl.block_size,
                   "recomputed_rows": cplan.n_rows, "seam_window": wl.k, "h_q": hq,
                   "h_kv": hkv, "head_dim": D, "rope_base": wl.rope_base,
                   "parallelism": "none (1 GPU)"},
        "attn_tflops": round(attn_tflops, 2),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4),
                     "traffic": load_traffic("attn", "shared_pool_gathered_k%d" % wl.k),
                     "kernel": "pic_selective_attn call (attn_bf16_kernel + merge_kernel)",
                     "algorithmic_flops": attn_flops, "algorithmic_bytes": attn_bytes},
        "kernels": {
            "rope_splice_pool": {"ms": round(t_g, 4), **pct(l_g), "bytes": gather_bytes,
                                 "GB_s": round(gather_bytes / (t_g * 1e-3) / 1e9, 1),
                                 "hbm_frac": round(gather_bytes / (t_g * 1e-3) / 1e9
                                                   / HBM_PEAK_GBS, 4)},
            "selective_attn": {"ms": round(t_attn, 4), **pct(l_attn), "flops": attn_flops,
                               "TFLOP_s": round(attn_tflops, 2),
                               "items": cplan[P.H_N_ATTN_ITEMS], "merges": cplan[P.H_N_MERGE]},
            "host_plan_ms": round(1e3 * float(np.mean(plan_s)), 4),
            "gpu_idle_ms": round(ms_step - t_g - t_attn, 4),
        },
    }
    del pk, pv, q, kf, vf, k, v, out, ws
    torch.cuda.empty_cache()
    rec["cpu_baseline"] = None if cpu_sample_rows is None else cpu_baseline_paged(
        wl, pk_h, pv_h, cbp, blocks, q_h, kf_h, vf_h, cplan, cpu_sample_rows)
    return rec


def run_paged(wl, steps, warmup, cpu_sample_rows):
    """One step = planner (with chunk ids) + plan upload + pic_selective_attn_paged over
    the shared-pool batch; returns the record (cpu_sample_rows None: no cpu_baseline)."""
    import torch
    import position_independent_kv_rope_amd as P
    from position_independent_kv_rope_amd import workloads as W
    reqs = [r.chunk_lens for r in wl.requests]
    ids = [r.chunk_ids for r in wl.requests]
    qs = [r.q_len for r in wl.requests]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    plan = P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, n_cu=n_cu, chunk_ids_per_req=ids)
    cbp, blocks = W.pool_block_table(wl)
    pk_h, pv_h = W.pool_tensors(wl)
    q_h, kf_h, vf_h = W.fresh_tensors(wl, plan.n_rows)
    dev = "cuda"
    pk, pv = pk_h.to(dev), pv_h.to(dev)
    cbp_d, blocks_d = torch.from_numpy(cbp).to(dev), torch.from_numpy(blocks).to(dev)
    q, kf, vf = q_h.to(dev), kf_h.to(dev), vf_h.to(dev)
    out = torch.empty_like(q)
    ws = P.attn_workspace(plan, wl.head_dim)
    uploader = PlanUploader(plan.words.size, dev)
    torch.cuda.synchronize()

    s = wl.torch_dtype.itemsize
    D, hq, hkv = wl.head_dim, wl.h_q, wl.h_kv
    rows = plan.rows.astype(np.int64)
    attn_flops = 4.0 * D * hq * float(np.sum(rows + 1))
    # every request reads its chunks' K/V once, plus Q and O of the recomputed rows
    attn_bytes = 2.0 * s * hkv * D * plan.n_tokens + 2.0 * s * hq * D * plan.n_rows
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    plan_s = []

    def step(i=None):
        t0 = time.perf_counter()
        p = P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, n_cu=n_cu, chunk_ids_per_req=ids)
        plan_s.append(time.perf_counter() - t0)
        uploader.upload(p)
        e = ev[i] if i is not None else None
        if e: e[0].record()
        P.pic_selective_attn_paged(p, q, pk, pv, cbp_d, blocks_d, kf, vf, out, wl.rope_base,
                                   workspace=ws)
        if e: e[1].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / steps
    l_attn = [e[0].elapsed_time(e[1]) for e in ev]
    t_attn = float(np.mean(l_attn))
    tokens = plan.n_tokens
    attn_tflops = attn_flops / (t_attn * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[wl.dtype]
    rec = {
        "metric": METRIC,
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": "shared_pool", "requests": len(wl.requests), "tokens": tokens,
                   "pool_chunks": len(wl.pool_lens), "pool_blocks": int(blocks.size),
                   "block_size": wl.block_size, "recomputed_rows": plan.n_rows,
                   "seam_window": wl.k, "h_q": hq, "h_kv": hkv, "head_dim": D,
                   "rope_base": wl.rope_base, "parallelism": "none (1 GPU)"},
        "attn_tflops": round(attn_tflops, 2),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4),
                     "traffic": load_traffic("attn_paged", "shared_pool_k%d" % wl.k),
                     "kernel": "pic_selective_attn_paged call (paged_angles_kernel + "
                               "paged_blocks_kernel + attn_bf16_paged_kernel + merge_kernel)",
                     "algorithmic_flops": attn_flops, "algorithmic_bytes": attn_bytes},
        "kernels": {
            "selective_attn_paged": {"ms": round(t_attn, 4), **pct(l_attn), "flops": attn_flops,
                                     "TFLOP_s": round(attn_tflops, 2),
                                     "items": plan[P.H_N_ATTN_ITEMS], "merges": plan[P.H_N_MERGE]},
            "host_plan_ms": round(1e3 * float(np.mean(plan_s)), 4),
            "gpu_idle_ms": round(ms_step - t_attn, 4),
        },
    }
    del pk, pv, q, kf, vf, out, ws
    torch.cuda.empty_cache()
    rec["cpu_baseline"] = None if cpu_sample_rows is None else cpu_baseline_paged(
        wl, pk_h, pv_h, cbp, blocks, q_h, kf_h, vf_h, plan, cpu_sample_rows)
    return rec


def bench_decode(args, wl):
    """One decode step of every request of the shared-pool batch: its next token attends
    over the request's pool chunks (rotated on load), recomputed rows and itself."""
    import torch
    import position_independent_kv_rope_amd as P
    from position_independent_kv_rope_amd import workloads as W
    from oracle import pic_oracle as O
    reqs = [r.chunk_lens for r in wl.requests]
    ids = [r.chunk_ids for r in wl.requests]
    qs = [r.q_len for r in wl.requests]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    plan = P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, n_cu=n_cu, chunk_ids_per_req=ids)
    plan.to_device()
    cbp, blocks = W.pool_block_table(wl)
    pk_h, pv_h = W.pool_tensors(wl)
    _, kf_h, vf_h = W.fresh_tensors(wl, plan.n_rows)
    qn_h, kn_h, vn_h = W.decode_tensors(wl)
    dev = "cuda"
    pk, pv = pk_h.to(dev), pv_h.to(dev)
    cbp_d, blocks_d = torch.from_numpy(cbp).to(dev), torch.from_numpy(blocks).to(dev)
    kf, vf = kf_h.to(dev), vf_h.to(dev)
    qn, kn, vn = qn_h.to(dev), kn_h.to(dev), vn_h.to(dev)
    out = torch.empty_like(qn)
    ws = P.decode_workspace(plan, wl.head_dim)
    torch.cuda.synchronize()

    s = wl.torch_dtype.itemsize
    D, hq, hkv = wl.head_dim, wl.h_q, wl.h_kv
    row_bytes = s * hkv * D  # one token's K (or V) for all KV heads
    used = sorted({i for r in wl.requests for i in r.chunk_ids})
    pool_used_tokens = sum(wl.pool_lens[i] for i in used)
    # chunk-major minimum: every used pool chunk once, the fresh rows, the new tokens, Q/O
    dec_bytes = (2.0 * row_bytes * (pool_used_tokens + plan.n_rows + len(wl.requests))
                 + 2.0 * s * hq * D * len(wl.requests))
    per_request_bytes = 2.0 * row_bytes * (plan.n_tokens + len(wl.requests))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]

    def call():
        P.pic_decode_attn_paged(plan, qn, kn, vn, pk, pv, cbp_d, blocks_d, kf, vf, out,
                                wl.rope_base, workspace=ws)

    graph = None
    if args.graph:  # the step's launches captured once (fixed plan), replayed per step
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        torch.cuda.synchronize()

    def step(i=None):
        e = ev[i] if i is not None else None
        if e: e[0].record()
        if graph is not None:
            graph.replay()
        else:
            call()
        if e: e[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t0) / args.steps
    l_dec = [e[0].elapsed_time(e[1]) for e in ev]
    t_dec = float(np.mean(l_dec))
    gbs = dec_bytes / (t_dec * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(plan.n_tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": "shared_pool_decode", "requests": len(wl.requests),
                   "context_tokens": plan.n_tokens, "pool_chunks": len(wl.pool_lens),
                   "pool_chunks_used": len(used), "seam_window": wl.k, "h_q": hq, "h_kv": hkv,
                   "head_dim": D, "parallelism": "none (1 GPU)",
                   "launch": "hip graph replay" if graph is not None else "eager"},
        "decode_steps_per_s": round(1e3 / ms_step, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("decode", "shared_pool_k%d" % wl.k),
                     "kernel": "pic_decode_attn_paged call (paged_angles_kernel + "
                               "dec_attn_kernel + dec_merge_kernel)",
                     "algorithmic_bytes": dec_bytes,
                     "per_request_streaming_bytes": per_request_bytes},
        "kernels": {"decode_attn": {"ms": round(t_dec, 4), **pct(l_dec), "GB_s": round(gbs, 1),
                                    "items": plan[P.H_N_DEC_ITEMS], "uses": plan[P.H_N_DEC_USES],
                                    "pieces": plan[P.H_N_DEC_PIECES],
                                    "workgroups": plan[P.H_N_DEC_WG],
                                    "records": plan[P.H_N_DEC_RECS]}},
    }
    if not args.no_cpu_baseline:
        # the oracle's decode of request 0: pool gather, rotation, splice, attention
        t1 = time.perf_counter()
        r = wl.requests[0]
        row0, row1 = int(plan.req_row_ptr[0]), int(plan.req_row_ptr[1])
        f64 = lambda t: t.to(torch.float64).numpy()
        ck, cv = [], []
        for i in r.chunk_ids:
            sub = torch.from_numpy(blocks[cbp[i]:cbp[i + 1]].astype(np.int64))
            ck.append(O.gather_paged_chunk(f64(pk_h[sub]), np.arange(len(sub)), wl.pool_lens[i]))
            cv.append(O.gather_paged_chunk(f64(pv_h[sub]), np.arange(len(sub)), wl.pool_lens[i]))
        rows = O.recompute_positions(r.chunk_lens, r.q_len, wl.k)
        kx, vx = O.splice(O.rope_delta(ck, wl.rope_base), O.concat_chunks(cv),
                          f64(kf_h[row0:row1]), f64(vf_h[row0:row1]), rows,
                          sum(r.chunk_lens) + r.q_len)
        O.decode_attn(f64(qn_h[0]), kx, vx, f64(kn_h[0]), f64(vn_h[0]))
        dt = time.perf_counter() - t1
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        n0 = sum(r.chunk_lens) + r.q_len
        rec["cpu_baseline"] = {"value": round(n0 / dt, 1), "unit": "tokens/s", "cores": int(threads),
                               "kind": "oracle", "seconds": round(dt, 3),
                               "sample": "decode step of request 0 (%d context tokens): pool "
                                         "gather, rotation, splice, attention of the new token"
                                         % n0, "host_cpus": os.cpu_count()}
    else:
        rec["cpu_baseline"] = None
    peaks = measured_peaks()
    rec = with_measured(rec, peaks)
    rec["measured_peaks"] = peaks
    print(json.dumps(rec), flush=True)


def bench_link(args, wl):
    """The whole link of a random model with args.link_layers layers: per step the host
    planner, the plan upload and one pic_link call (per layer: rope-delta of that layer's
    cached K, compute_qkv of the recomputed rows at their global positions, splice,
    selective attention, output projection + residual)."""
    import torch
    import position_independent_kv_rope_amd as P
    from position_independent_kv_rope_amd import workloads as W
    from oracle import pic_oracle as O
    n_layers = args.link_layers
    D, hq, hkv = wl.head_dim, wl.h_q, wl.h_kv
    d_model = args.d_model or hq * D
    reqs = [r.chunk_lens for r in wl.requests]
    qs = [r.q_len for r in wl.requests]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    plan = P.pic_build_index(reqs, qs, wl.k, hq, hkv, n_cu=n_cu)
    x0_h, wq_h, wo_h, kc_h, vc_h = W.link_tensors(wl, n_layers, d_model, plan.n_rows)
    dev = "cuda"
    x0 = x0_h.to(dev)
    x = x0.clone()
    wq = [t.to(dev) for t in wq_h]
    wo = [t.to(dev) for t in wo_h]
    kc = [t.to(dev) for t in kc_h]
    vc = [t.to(dev) for t in vc_h]
    q = torch.empty((plan.n_rows, hq, D), dtype=wl.torch_dtype, device=dev)
    kf = torch.empty((plan.n_rows, hkv, D), dtype=wl.torch_dtype, device=dev)
    vf, o = torch.empty_like(kf), torch.empty_like(q)
    ws = P.link_workspace(plan, D, dev)
    qkv_ws = P._bytes_workspace(P.lib().pic_qkv_workspace_bytes(plan.host_ptr(), D), dev)
    attn_ws = P.attn_workspace(plan, D, dev)
    uploader = PlanUploader(plan.words.size, dev)
    torch.cuda.synchronize()

    rows = plan.rows.astype(np.int64)
    attn_flops = 4.0 * D * hq * float(np.sum(rows + 1))
    qkv_flops = 2.0 * plan.n_rows * d_model * (hq + 2 * hkv) * D
    out_flops = 2.0 * plan.n_rows * hq * D * d_model
    link_flops = n_layers * (attn_flops + qkv_flops + out_flops)
    s = wl.torch_dtype.itemsize
    attn_bytes = 2.0 * s * hkv * D * plan.n_tokens + 2.0 * s * hq * D * plan.n_rows
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    plan_s = []

    def step(i=None):
        t0 = time.perf_counter()
        p = P.pic_build_index(reqs, qs, wl.k, hq, hkv, n_cu=n_cu)
        plan_s.append(time.perf_counter() - t0)
        uploader.upload(p)
        x.copy_(x0)  # every step starts from the same hidden states
        e = ev[i] if i is not None else None
        if e: e[0].record()
        P.pic_link(p, x, wq, wo, kc, vc, q, kf, vf, o, wl.rope_base, workspace=ws)
        if e: e[1].record()

    # The caches and weights stay resident; repeated steps rotate the caches again (a
    # rotation keeps every row's norm).  The hidden states are restored before every
    # step: left to grow, the residual stream would make the softmax ever more peaked,
    # and the MFMA units draw less power (and clock higher) on such near-zero operands.
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t0) / args.steps
    l_link = [e[0].elapsed_time(e[1]) for e in ev]
    t_link = float(np.mean(l_link))

    # per-kernel breakdown: the same entry points pic_link calls, one event between each
    names = ("qkv_rope", "rope_splice", "selective_attn", "out_proj")
    reps = 3
    plan.to_device()
    bev = [[[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_layers)]
           for _ in range(reps)]
    for rr in range(reps):
        x.copy_(x0)
        for l in range(n_layers):
            e = bev[rr][l]
            e[0].record()
            P.pic_qkv_rope(plan, x, wq[l], q, kf, vf, wl.rope_base, workspace=qkv_ws)
            e[1].record()
            P.pic_rope_splice(plan, kc[l], vc[l], kf, vf, wl.rope_base)
            e[2].record()
            P.pic_selective_attn(plan, q, kc[l], vc[l], o, workspace=attn_ws)
            e[3].record()
            P.pic_out_proj(plan, o, wo[l], x)
            e[4].record()
    torch.cuda.synchronize()
    t = {n: float(np.mean([bev[rr][l][j].elapsed_time(bev[rr][l][j + 1])
                           for rr in range(reps) for l in range(n_layers)]))
         for j, n in enumerate(names)}
    attn_tflops = attn_flops / (t["selective_attn"] * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[wl.dtype]

    # the vendor library (torch -> hipBLASLt) on the same two GEMM shapes, plain (no RoPE
    # epilogue, no residual): a same-shape reference for the projection kernels
    import torch.nn.functional as F

    def lib_ms(a, w):
        for _ in range(2):
            F.linear(a, w)
        le = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(10)]
        for e in le:
            e[0].record()
            F.linear(a, w)
            e[1].record()
        torch.cuda.synchronize()
        return float(np.mean([e[0].elapsed_time(e[1]) for e in le]))

    lib_qkv = lib_ms(x, wq[0])
    lib_out = lib_ms(o.reshape(plan.n_rows, hq * D), wo[0])
    rec = {
        "metric": METRIC,
        "value": round(plan.n_tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload + "_link", "requests": len(wl.requests),
                   "tokens": plan.n_tokens, "recomputed_rows": plan.n_rows, "k": wl.k,
                   "layers": n_layers, "d_model": d_model, "h_q": hq, "h_kv": hkv,
                   "head_dim": D, "rope_base": wl.rope_base, "parallelism": "none (1 GPU)"},
        "link_ms": round(t_link, 4),
        "link_p50_ms": pct(l_link)["p50_ms"], "link_p95_ms": pct(l_link)["p95_ms"],
        "link_tflops": round(link_flops / (t_link * 1e-3) / 1e12, 2),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4),
                     "traffic": load_traffic("attn", args.workload + "_k%d" % wl.k),
                     "kernel": "pic_selective_attn call (attn_bf16_kernel + merge_kernel), "
                               "per layer",
                     "algorithmic_flops": attn_flops, "algorithmic_bytes": attn_bytes},
        "kernels": {
            "qkv_rope": {"ms": round(t["qkv_rope"], 4), "flops": qkv_flops,
                         "TFLOP_s": round(qkv_flops / (t["qkv_rope"] * 1e-3) / 1e12, 2),
                         "library_same_shape_TFLOP_s": round(qkv_flops / (lib_qkv * 1e-3) / 1e12, 2),
                         "frac_of_library": round(lib_qkv / t["qkv_rope"], 3)},
            "rope_splice": {"ms": round(t["rope_splice"], 4)},
            "selective_attn": {"ms": round(t["selective_attn"], 4), "flops": attn_flops,
                               "TFLOP_s": round(attn_tflops, 2)},
            "out_proj": {"ms": round(t["out_proj"], 4), "flops": out_flops,
                         "TFLOP_s": round(out_flops / (t["out_proj"] * 1e-3) / 1e12, 2),
                         "library_same_shape_TFLOP_s": round(out_flops / (lib_out * 1e-3) / 1e12, 2),
                         "frac_of_library": round(lib_out / t["out_proj"], 3)},
            "library_reference": "torch.nn.functional.linear (hipBLASLt) on the same [rows x "
                                 "d_in] x [d_out x d_in]^T shapes, bf16, 10 launches, HIP "
                                 "events; plain GEMM without the RoPE epilogue or residual",
            "per_layer_ms": round(sum(t.values()), 4),
            "host_plan_ms": round(1e3 * float(np.mean(plan_s)), 4),
        },
    }
    if not args.no_cpu_baseline:
        # the oracle's link of request 0 through the first (up to) two layers, scaled to
        # all layers: compute_qkv, rotation, splice, attention, output projection
        r = wl.requests[0]
        f64 = lambda t: t.to(torch.float64).numpy()
        offs = O.chunk_offsets(r.chunk_lens)
        n_run = min(2, n_layers)
        r0, r1 = int(plan.req_row_ptr[0]), int(plan.req_row_ptr[1])
        t1 = time.perf_counter()
        layers = [{"w_qkv": f64(wq_h[l]), "w_o": f64(wo_h[l]),
                   "k_chunks": [f64(kc_h[l][offs[c]:offs[c + 1]]) for c in range(len(r.chunk_lens))],
                   "v_chunks": [f64(vc_h[l][offs[c]:offs[c + 1]]) for c in range(len(r.chunk_lens))]}
                  for l in range(n_run)]
        O.link_layers(f64(x0_h[r0:r1]), layers, r.q_len, wl.k, hq, hkv, wl.rope_base)
        dt = (time.perf_counter() - t1) * n_layers / n_run
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        n0 = sum(r.chunk_lens) + r.q_len
        rec["cpu_baseline"] = {"value": round(n0 / dt, 1), "unit": "tokens/s", "cores": int(threads),
                               "kind": "oracle", "seconds": round(dt, 3),
                               "sample": "request 0 (%d tokens) through %d of the %d layers, "
                                         "scaled to all: compute_qkv, rotation, splice, "
                                         "attention, output projection" % (n0, n_run, n_layers),
                               "host_cpus": os.cpu_count()}
    else:
        rec["cpu_baseline"] = None
    peaks = measured_peaks()
    rec = with_measured(rec, peaks)
    rec["measured_peaks"] = peaks
    print(json.dumps(rec), flush=True)


def bench_state(args, wl):
    """HYPIC linear-layer state composition over the shared-pool batch: every request's
    chunks composed in prompt order from cached (T_C, S(C|0)) per head, writing the state
    after every chunk and the final states (fp32)."""
    import torch
    import position_independent_kv_rope_amd as P
    from position_independent_kv_rope_amd import workloads as W
    from oracle import pic_oracle as O
    H, d = args.heads, 128
    reqs = [r.chunk_lens for r in wl.requests]
    ids = [r.chunk_ids for r in wl.requests]
    qs = [r.q_len for r in wl.requests]
    plan = P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, chunk_ids_per_req=ids)
    plan.to_device()
    t_h, s_h = W.state_pool_tensors(wl, H, d)
    dev = "cuda"
    t_pool, s_pool = t_h.to(dev), s_h.to(dev)
    n_req, n_chunks = len(reqs), plan[P.H_N_CHUNKS]
    final = torch.empty((n_req, H, d, d), dtype=torch.float32, device=dev)
    prefix = torch.empty((n_chunks, H, d, d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    steps = n_chunks * H  # (chunk, head) products
    flops = steps * 2.0 * d * d * d
    used = sorted({i for r in wl.requests for i in r.chunk_ids})
    mat = 4.0 * d * d
    # every used chunk's T and S(C|0) once, the state after every chunk and the finals
    alg_bytes = len(used) * H * 2 * mat + steps * mat + n_req * H * mat
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]

    def step(i=None):
        e = ev[i] if i is not None else None
        if e: e[0].record()
        P.pic_state_compose(plan, t_pool, s_pool, final, prefix_out=prefix)
        if e: e[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t0) / args.steps
    l_call = [e[0].elapsed_time(e[1]) for e in ev]
    t_call = float(np.mean(l_call))
    tflops = flops / (t_call * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS["f32"]
    rec = {
        "metric": METRIC,
        "value": round(plan.n_tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "shared_pool_state_compose", "requests": n_req,
                   "context_tokens": plan.n_tokens, "chunks": n_chunks, "pool_chunks": len(wl.pool_lens),
                   "heads": H, "d_k": d, "d_v": d, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
                     "traffic": load_traffic("state", "shared_pool_h%d" % H,
                                             ["position_independent_kv_rope_amd/csrc/pic_state.hip"]),
                     "kernel": "pic_state_compose call (state_compose_kernel)",
                     "algorithmic_flops": flops, "algorithmic_bytes": alg_bytes,
                     "hbm_GB_s_at_algorithmic_bytes": round(alg_bytes / (t_call * 1e-3) / 1e9, 1)},
        "kernels": {"state_compose": {"ms": round(t_call, 4), **pct(l_call),
                                      "TFLOP_s": round(tflops, 2),
                                      "products": steps}},
    }
    if not args.no_cpu_baseline:
        # the oracle's composition of request 0, every head
        t1 = time.perf_counter()
        r = wl.requests[0]
        tp = [t_h[i].double().numpy() for i in r.chunk_ids]
        sp = [s_h[i].double().numpy() for i in r.chunk_ids]
        for h in range(H):
            O.compose_states([t[h] for t in tp], [s[h] for s in sp])
        dt = time.perf_counter() - t1
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        n0 = sum(r.chunk_lens) + r.q_len
        rec["cpu_baseline"] = {"value": round(n0 / dt, 1), "unit": "tokens/s", "cores": int(threads),
                               "kind": "oracle", "seconds": round(dt, 3),
                               "sample": "request 0 (%d chunks, %d tokens), all %d heads: fp64 "
                                         "composition of the cached (T, S) pairs"
                                         % (len(r.chunk_ids), n0, H),
                               "host_cpus": os.cpu_count()}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


SUB_RECORDS = [("epic_sweep", 2), ("epic_sweep", 4), ("epic_sweep", 8),
               ("long_context", 2), ("long_context", 16), ("shared_pool", 8),
               ("shared_pool_gathered", 8)]
MALL_EVICT_BYTES = 512 << 20  # twice the 256 MB Infinity Cache


def run_contiguous(wl, workload, steps, warmup, rope_scheme="delta", cpu_requests=None,
                   cpu_sample_rows=0, evict_passes=20):
    """One step = host planner + plan upload + pic_rope_splice + pic_selective_attn over one
    batch of a contiguous workload.  Returns the record (cpu_requests None: no
    cpu_baseline).  After the timed steps: the two calls the fused launch stands for,
    timed separately, and evict_passes rotation + splice launches each timed right after
    a 512 MB read that evicts the Infinity Cache (MALL)."""
    import torch
    import position_independent_kv_rope_amd as P
    from position_independent_kv_rope_amd import workloads as W
    reqs = [r.chunk_lens for r in wl.requests]
    qs = [r.q_len for r in wl.requests]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    plan = P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, n_cu=n_cu)
    k_in, v_in = W.context_tensors(wl)
    q_h, kf_h, vf_h = W.fresh_tensors(wl, plan.n_rows)
    dev = "cuda"
    k, v = k_in.to(dev), v_in.to(dev)
    q, kf, vf = q_h.to(dev), kf_h.to(dev), vf_h.to(dev)
    out = torch.empty_like(q)
    ws = P.attn_workspace(plan, wl.head_dim)
    uploader = PlanUploader(plan.words.size, dev)
    torch.cuda.synchronize()

    s = wl.torch_dtype.itemsize
    D, hq, hkv = wl.head_dim, wl.h_q, wl.h_kv
    rows = plan.rows.astype(np.int64)
    attn_flops = 4.0 * D * hq * float(np.sum(rows + 1))
    tiles = plan.rope_tiles if plan[P.H_N_ROPE_TILES] else np.zeros((0, 4), dtype=np.int64)
    # rows the rotation touches: tiles with delta != 0 (by delta), every kept row (nope)
    rotated = tiles if rope_scheme == "nope" else tiles[tiles[:, 2] != 0]
    rope_rows = int(rotated[:, 1].sum())
    rope_bytes = 2.0 * s * hkv * D * rope_rows
    splice_bytes = 4.0 * s * hkv * D * plan.n_rows
    attn_bytes = 2.0 * s * hkv * D * plan.n_tokens + 2.0 * s * hq * D * plan.n_rows

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    plan_s = []
    mode = P.PIC_ROPE_AT_POSITION if rope_scheme == "nope" else P.PIC_ROPE_BY_DELTA

    def step(i=None):
        t0 = time.perf_counter()
        p = P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, n_cu=n_cu)
        plan_s.append(time.perf_counter() - t0)
        uploader.upload(p)
        e = ev[i] if i is not None else None
        if e: e[0].record()
        P.pic_rope_splice(p, k, v, kf, vf, wl.rope_base, mode=mode)
        if e: e[1].record()
        P.pic_selective_attn(p, q, k, v, out, workspace=ws)
        if e: e[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / steps

    l_rs = [e[0].elapsed_time(e[1]) for e in ev]
    l_attn = [e[1].elapsed_time(e[2]) for e in ev]
    t_rs, t_attn = float(np.mean(l_rs)), float(np.mean(l_attn))

    # breakdown after the timed steps: the two calls pic_rope_splice stands for, timed
    # separately on the same buffers (each pass rotates K again: the bytes are the same),
    # each pair followed by the attention call as in a step
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    dplan = uploader.upload(P.pic_build_index(reqs, qs, wl.k, wl.h_q, wl.h_kv, n_cu=n_cu))
    for e in sev:
        e[0].record()
        if rope_scheme == "nope":
            P.pic_rope_apply(dplan, k, wl.rope_base)
        else:
            P.pic_rope_delta(dplan, k, wl.rope_base)
        e[1].record()
        P.pic_splice(dplan, k, v, kf, vf)
        e[2].record()
        P.pic_selective_attn(dplan, q, k, v, out, workspace=ws)
    torch.cuda.synchronize()
    l_rope = [e[0].elapsed_time(e[1]) for e in sev]
    l_splice = [e[1].elapsed_time(e[2]) for e in sev]
    t_rope, t_splice = float(np.mean(l_rope)), float(np.mean(l_splice))
    rs_bytes = rope_bytes + splice_bytes
    # the fused rotation + splice from HBM: before each timed launch a 512 MB buffer
    # (written once, before the passes) is read, which evicts the Infinity Cache (K and V
    # of the smaller batches would otherwise be served from it) and leaves it holding
    # clean lines, so the timed launch pays for no write-back of the eviction pass; one
    # untimed pass first
    l_ev = []
    if evict_passes > 0:
        scratch = torch.ones(MALL_EVICT_BYTES // 4, dtype=torch.int32, device=dev)
        xev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(evict_passes)]
        scratch.sum()
        P.pic_rope_splice(dplan, k, v, kf, vf, wl.rope_base, mode=mode)
        for e in xev:
            scratch.sum()
            e[0].record()
            P.pic_rope_splice(dplan, k, v, kf, vf, wl.rope_base, mode=mode)
            e[1].record()
        torch.cuda.synchronize()
        l_ev = [e[0].elapsed_time(e[1]) for e in xev]
        del scratch
    tokens = plan.n_tokens
    value = tokens / (ms_step * 1e-3)
    attn_tflops = attn_flops / (t_attn * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[wl.dtype]
    traffic = load_traffic("attn", workload + "_k%d" % wl.k)
    gbs = lambda nbytes, ms: round(nbytes / (ms * 1e-3) / 1e9, 1)
    frac = lambda nbytes, ms: round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    fused = "pic_rope_splice (%s + splice, one launch)" % (
        "rope_apply" if rope_scheme == "nope" else "rope_delta")
    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": workload, "requests": len(wl.requests), "tokens": tokens,
                   "recomputed_rows": plan.n_rows, "k": wl.k, "h_q": hq, "h_kv": hkv,
                   "head_dim": D, "rope_base": wl.rope_base, "rope_scheme": rope_scheme,
                   "parallelism": "none (1 GPU)"},
        "attn_tflops": round(attn_tflops, 2),
        "splice_pass_tokens_per_s": round(tokens / (t_rs * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4),
                     "traffic": traffic,
                     "kernel": "pic_selective_attn call (attn_bf16_kernel + merge_kernel)",
                     "algorithmic_flops": attn_flops, "algorithmic_bytes": attn_bytes},
        "kernels": {
            "rope_splice": {"ms": round(t_rs, 4), **pct(l_rs), "bytes": rs_bytes,
                            "GB_s": gbs(rs_bytes, t_rs), "hbm_frac": frac(rs_bytes, t_rs),
                            "call": fused + ", inside the steps"},
            ("rope_apply" if rope_scheme == "nope" else "rope_delta"): {
                "ms": round(t_rope, 4), **pct(l_rope), "bytes": rope_bytes,
                "GB_s": gbs(rope_bytes, t_rope), "hbm_frac": frac(rope_bytes, t_rope),
                "call": "separate call, timed after the steps"},
            "splice": {"ms": round(t_splice, 4), **pct(l_splice), "bytes": splice_bytes,
                       "GB_s": gbs(splice_bytes, t_splice), "hbm_frac": frac(splice_bytes, t_splice),
                       "call": "separate call, timed after the steps"},
            "selective_attn": {"ms": round(t_attn, 4), **pct(l_attn), "flops": attn_flops,
                               "TFLOP_s": round(attn_tflops, 2),
                               "items": plan[P.H_N_ATTN_ITEMS], "merges": plan[P.H_N_MERGE]},
            "host_plan_ms": round(1e3 * float(np.mean(plan_s)), 4),
            "gpu_idle_ms": round(ms_step - t_rs - t_attn, 4),
        },
    }
    if l_ev:
        t_ev = float(np.mean(l_ev))
        rec["kernels"]["rope_splice_mall_evicted"] = {
            "ms": round(t_ev, 4), **pct(l_ev), "bytes": rs_bytes, "GB_s": gbs(rs_bytes, t_ev),
            "hbm_frac": frac(rs_bytes, t_ev),
            "call": fused + ", each launch right after a 512 MB read (Infinity Cache evicted, "
                    "no dirty lines left)"}
    del k, v, q, kf, vf, out, ws
    torch.cuda.empty_cache()
    rec["cpu_baseline"] = None if cpu_requests is None else cpu_baseline(
        wl, k_in, v_in, q_h, kf_h, vf_h, plan, cpu_requests, cpu_sample_rows, rope_scheme)
    return rec


def sub_record(rec):
    """The per-configuration fields of a record (what a sub-record keeps)."""
    keep = ("value", "unit", "ms_per_step", "steps", "warmup", "config", "attn_tflops",
            "splice_pass_tokens_per_s", "roofline", "kernels", "cpu_baseline")
    return {k: rec[k] for k in keep if k in rec}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import position_independent_kv_rope_amd as P

    if args.copy_calibration:
        return copy_calibration()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    P.lib()
    if args.peaks_only:
        print(json.dumps({"measured_peaks": measured_peaks()}), flush=True)
        return
    wl = make_workload(args.workload, args.k)
    if wl.pool_lens is not None:
        if args.state_compose:
            return bench_state(args, wl)
        return bench_decode(args, wl) if args.decode else bench_paged(args, wl)
    if args.decode:
        print("--decode needs --workload shared_pool", file=sys.stderr)
        sys.exit(2)
    if args.link_layers > 0:
        return bench_link(args, wl)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = list(range(len(wl.requests)))
    peaks = measured_peaks()
    rec = with_measured(run_contiguous(wl, args.workload, args.steps, args.warmup,
                                       args.rope_scheme, cpu, args.cpu_sample_rows), peaks)
    rec["measured_peaks"] = peaks
    headline = (args.workload == "epic_sweep" and args.k is None and args.rope_scheme == "delta"
                and not args.no_sub_records)
    if headline:
        # the other configurations of the same path, each with its own roofline and a
        # bounded cpu_baseline sample, as sub-records of the one line
        sub_steps, sub_warm = max(3, min(args.steps, 10)), max(1, min(args.warmup, 3))
        subs = {}
        for name, k in SUB_RECORDS:
            gathered = name == "shared_pool_gathered"
            w = make_workload("shared_pool" if gathered else name, k)
            print("[bench] sub-record %s k=%d" % (name, k), file=sys.stderr, flush=True)
            if w.pool_lens is not None:
                r = (run_pool_gathered if gathered else run_paged)(
                    w, sub_steps, sub_warm, None if args.no_cpu_baseline else 96)
            else:
                r = run_contiguous(w, name, sub_steps, sub_warm, "delta",
                                   None if args.no_cpu_baseline else [0],
                                   0 if name == "long_context" else 128)
            subs["%s_k%d" % (name, k)] = sub_record(with_measured(r, peaks))
        rec["sub_records"] = subs
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
