"""Summaries of rocprofv3 output for the kernels of libpic.so.

    python -m position_independent_kv_rope_amd.profiling stats <kernel_stats.csv>
    python -m position_independent_kv_rope_amd.profiling counters <counter_collection.csv> ...
    python -m position_independent_kv_rope_amd.profiling report --kernel attn_bf16 \
        --stats <kernel_stats.csv> --counters <csv> ... --copy-fetch <csv> --copy-write <csv> \
        --algo-bytes B --algo-flops F --title T --cmdline "..." [--cmdline "..."]
    python -m position_independent_kv_rope_amd.profiling traffic \
        --fetch <bench FETCH_SIZE csv> --write <bench WRITE_SIZE csv> \
        --copy-fetch <copy FETCH_SIZE csv> --copy-write <copy WRITE_SIZE csv> \
        --kernel attn_bf16_kernel,merge_kernel --out profiles/traffic_attn_<workload>.json \
        --sources position_independent_kv_rope_amd/csrc/pic_attn.hip \
                  position_independent_kv_rope_amd/csrc/pic_attn_common.h

``traffic`` scales the per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the kernels of one
call (summed) by what the same counters read for a plain device copy of known size, and
records the sha256 of the kernel sources' code (comments and white space removed) so a
stale measurement is not reused after a code change.
"""

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SHORT = [("pool_rope_splice_kernel", "rope_splice_pool"), ("rope_splice_kernel", "rope_splice"),
         ("qkv_rope_gemm_kernel", "qkv_rope_gemm"), ("out_proj_gemm_kernel", "out_proj_gemm"),
         ("state_compose_kernel", "state_compose"),
         ("row_angles_kernel", "row_angles"),
         ("attn_bf16_paged_kernel", "attn_bf16_paged"), ("paged_angles_kernel", "paged_angles"),
         ("paged_blocks_kernel", "paged_blocks"),
         ("dec_attn_kernel", "dec_attn"), ("dec_merge_kernel", "dec_merge"),
         ("attn_bf16_kernel", "attn_bf16"), ("attn_f32_kernel", "attn_f32"),
         ("merge_kernel", "merge"), ("rope_delta_kernel", "rope_delta"),
         ("splice_kernel", "splice"), ("copyBuffer", "copy (calibration)"),
         ("calib_mfma_kernel", "calib_mfma"), ("calib_read_kernel", "calib_read"),
         ("calib_copy_kernel", "calib_copy"), ("calib_update_kernel", "calib_update")]


def short_name(name):
    m = re.search(r"rope_kernelI\w+?Lb[01]ELb([01])E", name)  # rope_kernel<T, half, absolute>
    if m:
        return "rope_apply" if m.group(1) == "1" else "rope_delta"
    for key, s in SHORT:
        if key in name:
            return s
    return name[:48]


def read_csv(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def kernel_stats(path):
    out = []
    for r in read_csv(path):
        out.append({"kernel": short_name(r["Name"]), "calls": int(r["Calls"]),
                    "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                    "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return out


def counters(paths):
    """Mean per dispatch of every counter, per kernel (a counter's rows of one dispatch --
    one per hardware instance when rocprofv3 reports them apart -- are summed first).
    Each counter run also gives the mean dispatch duration of its own dispatches, in ns,
    under the key "duration_ns:<counter run file>"."""
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for p in paths:
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        dur, kname = {}, {}
        for r in read_csv(p):
            d = r.get("Dispatch_Id", str(len(dur)))
            per[d][r["Counter_Name"]] += float(r["Counter_Value"])
            kname[d] = short_name(r["Kernel_Name"])
            if "Start_Timestamp" in r and "End_Timestamp" in r:
                dur[d] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
        for d, cs in per.items():
            for c, v in cs.items():
                agg[kname[d]][c].append(v)
            if d in dur:
                agg[kname[d]]["duration_ns:" + os.path.basename(os.path.dirname(p))].append(dur[d])
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in agg.items()}


# MI355X: 32 shader engines (8 XCDs x 4) each count SQ_BUSY_CYCLES, and 1024 SIMDs (256
# CUs x 4) each count SQ_VALU_MFMA_BUSY_CYCLES, so per dispatch
#   shader clock  = SQ_BUSY_CYCLES / 32 / duration
#   MFMA busy     = SQ_VALU_MFMA_BUSY_CYCLES / 1024 / (SQ_BUSY_CYCLES / 32)
N_SE, N_SIMD = 32, 1024


def derived(c):
    """Clock, MFMA-busy fraction, instruction mix and wait fractions from one kernel's
    counters (None where a counter is missing)."""
    out = {}
    dur = [v for k, v in c.items() if k.startswith("duration_ns:") and "SQ" in k]
    busy = c.get("SQ_BUSY_CYCLES")
    if busy and dur:
        out["shader_clock_GHz"] = busy / N_SE / dur[0]
    if busy and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        out["mfma_busy"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / (busy / N_SE)
    if c.get("SQ_INSTS_MFMA"):
        out["valu_per_mfma"] = c.get("SQ_INSTS_VALU", 0.0) / c["SQ_INSTS_MFMA"]
        if "SQ_INSTS_LDS" in c:
            out["lds_per_mfma"] = c["SQ_INSTS_LDS"] / c["SQ_INSTS_MFMA"]
    if c.get("SQ_WAVE_CYCLES"):
        for k, name in (("SQ_WAIT_ANY", "wave_cycles_in_waitcnt"),
                        ("SQ_WAIT_INST_ANY", "wave_cycles_waiting_to_issue")):
            if k in c:
                out[name] = c[k] / c["SQ_WAVE_CYCLES"]
    return out


def src_hash(paths):
    """sha256 of the sources' code with comments and white space removed, so that a
    counter run stays valid across comment-only edits and goes stale with any code
    change."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(re.sub(r"\s+", "", text).encode())
    return h.hexdigest()[:16]


def traffic(args):
    fetch = counters([args.fetch])
    write = counters([args.write])
    cf = counters([args.copy_fetch])["copy (calibration)"]["FETCH_SIZE"]
    cw = counters([args.copy_write])["copy (calibration)"]["WRITE_SIZE"]
    copy_kib = args.copy_bytes / 1024.0
    f_scale, w_scale = copy_kib / cf, copy_kib / cw
    ks = [short_name(k) for k in args.kernel.split(",")]  # the kernels of one call, summed
    fb = sum(fetch[k]["FETCH_SIZE"] for k in ks) * f_scale * 1024.0
    wb = sum(write[k]["WRITE_SIZE"] for k in ks) * w_scale * 1024.0
    rec = {"kernel": " + ".join(ks), "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
           "bytes_per_launch": fb + wb, "fetch_scale": f_scale, "write_scale": w_scale,
           "copy_bytes": args.copy_bytes, "sources": args.sources,
           "source_hash": src_hash(args.sources), "command": args.command}
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def report(args):
    """Markdown summary of one kernel: trace statistics, counters, scaled HBM traffic."""
    stats = {r["kernel"]: r for r in kernel_stats(args.stats)}
    cs = counters(args.counters)
    k = short_name(args.kernel)
    st = stats[k]
    c = cs.get(k, {})
    copy_kib = float(1 << 30) / 1024.0
    f_scale = copy_kib / counters([args.copy_fetch])["copy (calibration)"]["FETCH_SIZE"]
    w_scale = copy_kib / counters([args.copy_write])["copy (calibration)"]["WRITE_SIZE"]
    out = ["# %s" % args.title, "", "Commands (run from /tmp with TMPDIR=/tmp; R = repository root):", ""]
    out += ["    " + cl for cl in args.cmdlines]
    out += ["", "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
            "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for r in kernel_stats(args.stats):
        out.append("| %s | %d | %.1f | %.1f | %.1f | %.2f |" % (r["kernel"], r["calls"], r["avg_us"],
                                                                 r["min_us"], r["max_us"], r["pct"]))
    avg_s = st["avg_us"] * 1e-6
    out += ["", "## %s per launch" % k, ""]
    if args.algo_flops:
        out.append("- algorithmic flops: %.4g -> %.1f TFLOP/s at the average duration" %
                   (args.algo_flops, args.algo_flops / avg_s / 1e12))
    if args.algo_bytes:
        out.append("- algorithmic bytes: %.4g -> %.1f GB/s at the average duration" %
                   (args.algo_bytes, args.algo_bytes / avg_s / 1e9))
    if "FETCH_SIZE" in c:
        fb = c["FETCH_SIZE"] * f_scale * 1024
        wb = c.get("WRITE_SIZE", 0.0) * w_scale * 1024
        out.append("- HBM traffic from counters: fetch %.4g B + write %.4g B = %.4g B "
                   "(FETCH_SIZE x %.3f, WRITE_SIZE x %.3f, factors from a 1 GiB device copy)"
                   % (fb, wb, fb + wb, f_scale, w_scale))
        if args.algo_bytes:
            out.append("- counter traffic / algorithmic bytes: %.2f" % ((fb + wb) / args.algo_bytes))
    if "TCC_HIT" in c and "TCC_MISS" in c:
        out.append("- L2 hit rate: %.1f%%" % (100.0 * c["TCC_HIT"] / (c["TCC_HIT"] + c["TCC_MISS"])))
    dv = derived(c)
    if "shader_clock_GHz" in dv:
        out.append("- shader clock during the SQ counter run: %.2f GHz (SQ_BUSY_CYCLES / 32 "
                   "shader engines / dispatch duration)" % dv["shader_clock_GHz"])
    if "mfma_busy" in dv:
        out.append("- MFMA busy: %.1f%% of busy cycles (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs "
                   "over SQ_BUSY_CYCLES / 32)" % (100 * dv["mfma_busy"]))
    if "valu_per_mfma" in dv:
        out.append("- VALU instructions per MFMA (SQ_INSTS_VALU counts the MFMAs too): %.2f%s" % (
            dv["valu_per_mfma"], "; LDS instructions per MFMA: %.2f" % dv["lds_per_mfma"]
            if "lds_per_mfma" in dv else ""))
    if "wave_cycles_in_waitcnt" in dv:
        out.append("- wave cycles in s_waitcnt: %.1f%%; waiting to issue: %.1f%% "
                   "(SQ_WAIT_ANY, SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES)" % (
                       100 * dv["wave_cycles_in_waitcnt"],
                       100 * dv.get("wave_cycles_waiting_to_issue", 0.0)))
    if c:
        out += ["", "Raw counters (mean per dispatch): " +
                ", ".join("%s=%.6g" % kv for kv in sorted(c.items())
                          if not kv[0].startswith("duration_ns:"))]
    text = "\n".join(out) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--kernel", "--out"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    t.add_argument("--sources", nargs="+", required=True,
                   help="the kernel sources whose code the record stays valid for")
    t.add_argument("--command", default="")
    r = sub.add_parser("report")
    r.add_argument("--kernel", required=True)
    r.add_argument("--stats", required=True)
    r.add_argument("--counters", nargs="*", default=[])
    r.add_argument("--copy-fetch", required=True)
    r.add_argument("--copy-write", required=True)
    r.add_argument("--algo-bytes", type=float, default=0.0)
    r.add_argument("--algo-flops", type=float, default=0.0)
    r.add_argument("--title", required=True)
    r.add_argument("--cmdline", action="append", dest="cmdlines", default=[])
    r.add_argument("--out", default="")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print("| kernel | calls | avg us | min us | max us | % time |")
        print("|---|---|---|---|---|---|")
        for r in kernel_stats(a.csv):
            print("| %s | %d | %.1f | %.1f | %.1f | %.2f |" % (r["kernel"], r["calls"], r["avg_us"],
                                                             r["min_us"], r["max_us"], r["pct"]))
    elif a.cmd == "counters":
        for k, cs in counters(a.csv).items():
            print("%s: %s" % (k, ", ".join("%s=%.6g" % kv for kv in sorted(cs.items()))))
    elif a.cmd == "report":
        report(a)
    else:
        traffic(a)


if __name__ == "__main__":
    sys.exit(main())
