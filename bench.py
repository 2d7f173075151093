"""Benchmark of the masked paged-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  * prefill: one 16384-token sequence (no prefix), 40 query / 40 KV heads,
    headSize 128, blockSize 128, bf16, ALiBi slopes 2^(-8(h+1)/40): one
    PrefixEncoder launch with the sqrt ALiBi mask and one with the left-aligned
    ALiBi mask, over the same inputs;
  * decode: MLA on the latent paged cache (batch 64, 128 heads, q_len 1, 576/512,
    blockSize 128, contextLens ~ U[1024,8192], bf16), split + combine, reading one
    of two rotated KV caches (2 x 340 MB > the 256 MB Infinity Cache) so the cache
    is cold.
value = valid prefill FLOPs of the two launches (4 * headSize per visible
(query, key) pair) / their kernel time; the decode rate (algorithmic bytes / MLA
call time) is reported beside it.  Kernel times come from HIP events that each
call records on its own kernels' dispatch packets (start of its first kernel,
end of its last) inside the timed region, so no event command sits between the
calls on the stream; the step time comes from two stream events around the whole
timed region (it includes each call's copy of its launch plan into its workspace).
Before the W warm-up steps the step runs untimed for half a second, so that the
timed steps see the GPU's working clocks rather than its ramp from idle.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-extra] [--no-cpu-baseline]
"""

import argparse
import csv
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "valid-FLOP attention TFLOP/s + % MFMA peak (prefill); decode GB/s + % HBM"
PEAK_MFMA_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


# ---------------------------------------------------------------------------
# Work accounting (closed forms; pinned by tests/test_bench_accounting.py).
# ---------------------------------------------------------------------------

def visible_pairs(seq_len, kv_seq_len, causal):
    """Visible (query row, key) pairs of one head: row i of sequence b sees
    min(kv, kv - L + i + 1) keys when causal, kv otherwise."""
    tot = 0
    for L, kv in zip(seq_len, kv_seq_len):
        L, kv = int(L), int(kv)
        if causal:
            P = kv - L
            tot += L * P + L * (L + 1) // 2
        else:
            tot += L * kv
    return tot


def prefill_valid_flops(seq_len, kv_seq_len, causal, head_num, head_size):
    """2*D for q.k plus 2*D for p*v per visible pair, every query head."""
    return visible_pairs(seq_len, kv_seq_len, causal) * head_num * 4 * head_size


def prefill_valid_flops_chunked(seq_len, kv_seq_len, chunk, head_num, head_size):
    """Valid FLOPs of the chunked local causal mask: row a sees a - chunk*floor(a/chunk) + 1 keys."""
    pairs = 0
    for L, kv in zip(seq_len, kv_seq_len):
        a = np.arange(int(kv) - int(L), int(kv), dtype=np.int64)
        pairs += int((a - (a // chunk) * chunk + 1).sum())
    return pairs * head_num * 4 * head_size


def padding_positions(lengths, padded_to):
    """B * Lmax - sum L_i (padding count of a padded batch)."""
    return len(lengths) * int(padded_to) - int(np.sum(lengths))


def mla_bytes(context_lens, q_tokens, head_num, elem=2, with_lse=True, max_blocks=None):
    """Algorithmic HBM bytes of one MLA call: every latent row (512 + 64 values)
    once, the query (576), the output (512), the LSE (fp32) and the block table."""
    kv = int(np.sum(context_lens)) * 576 * elem
    q = q_tokens * head_num * 576 * elem
    o = q_tokens * head_num * 512 * elem
    lse = q_tokens * head_num * 4 if with_lse else 0
    bt = len(context_lens) * (max_blocks or 0) * 4
    return kv + q + o + lse + bt


def mla_bytes_int8(context_lens, q_tokens, head_num, elem=2, max_blocks=None):
    """Algorithmic HBM bytes of one MLA call over the int8 latent cache: every
    latent row once (512 int8 + 64 rope values), the query (512 int8 + 64), the
    output (512), the LSE (fp32), the block table and the two per-head descales."""
    kv = int(np.sum(context_lens)) * (512 + 64 * elem)
    q = q_tokens * head_num * (512 + 64 * elem)
    o = q_tokens * head_num * 512 * elem
    lse = q_tokens * head_num * 4
    bt = len(context_lens) * (max_blocks or 0) * 4
    return kv + q + o + lse + bt + 2 * head_num * 4


def mla_flops(context_lens, q_seq_len, head_num, spec):
    """2*576 + 2*512 flops per visible (token, key) pair per head."""
    pairs = 0
    for b, ctx in enumerate(context_lens):
        ql = 1 if q_seq_len is None else int(q_seq_len[b])
        for t in range(ql):
            pairs += (int(ctx) - ql + t + 1) if spec else int(ctx)
    return pairs * head_num * (2 * 576 + 2 * 512)


# ---------------------------------------------------------------------------
# rocprofv3 summaries (the text files under profiles/) and the HBM traffic they hold.
# ---------------------------------------------------------------------------

# Everything that decides what the kernels do on the GPU: a change to any of these
# files invalidates hardware counters taken before it.
KERNEL_FILES = ("masked_paged_attention_amd/csrc/prefill_fwd.hip",
                "masked_paged_attention_amd/csrc/mla_decode.hip",
                "masked_paged_attention_amd/csrc/device.h",
                "masked_paged_attention_amd/csrc/kernels.h",
                "masked_paged_attention_amd/csrc/planner.cpp",
                "masked_paged_attention_amd/csrc/api.cpp")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_alibi16384_mla_decode.txt")
KERNEL_KEYS = ("prefill_dma_kernel", "prefill_fwd_kernel", "mla_split_kernel", "mla_combine_kernel")


def kernel_source_digest():
    h = hashlib.sha256()
    for f in KERNEL_FILES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_kernel_name(mangled):
    """'..prefill_fwd_kernelIDF16bLi128ELi9EEE..' -> 'prefill_fwd_kernel<bf16,128,9>'."""
    for key in KERNEL_KEYS:
        k = mangled.find(key)
        if k >= 0:
            rest = mangled[k + len(key):]
            args = []
            if rest.startswith("I"):  # mangled template arguments
                for m in re.finditer(r"DF16b|DF16_|Li(\d+)E|Lb([01])E", rest[:40]):
                    t = m.group(0)
                    args.append("bf16" if t == "DF16b" else "fp16" if t == "DF16_" else
                                m.group(1) if m.group(1) else ("true" if m.group(2) == "1" else "false"))
            elif rest.startswith("<"):  # demangled
                inner = rest[1:rest.find(">")] if ">" in rest else ""
                parts = [a.strip() for a in inner.split(",")]
                i = 0
                while i < len(parts):
                    a = parts[i]
                    i += 1
                    # rocprofv3 prints the mangled __bf16 (DF16b) as "bool _Accum" and
                    # the mangled true (Lb1E) as the two pieces "bool", "E"
                    if a == "bool" and i < len(parts) and parts[i] == "E":
                        args.append("true")
                        i += 1
                        continue
                    args.append("bf16" if "bf" in a.lower() or "_Accum" in a else
                                "fp16" if "16" in a and "float" in a.lower() else a)
            return key + ("<" + ",".join(args) + ">" if args else "")
    return mangled


def summarize_kernel_stats(stats_csv, command, last=0):
    """Text summary of a rocprofv3 --kernel-trace --stats kernel_stats.csv; with
    last > 0 also the mean duration of each kernel's last `last` dispatches, from
    the kernel_trace.csv beside it (the timed steps of a bench run: the earlier
    dispatches include the untimed pre-warm and warm-up)."""
    rows = list(csv.DictReader(open(stats_csv)))
    out = ["# rocprofv3 kernel statistics", "# command:", "#   " + command,
           f"# kernel sources digest: {kernel_source_digest()}", "",
           f"{'kernel':44s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'share%':>7s}"]
    for r in rows:
        out.append(f"{short_kernel_name(r['Name']):44s} {int(r['Calls']):6d} "
                   f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                   f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):7.2f}")
    trace_csv = stats_csv.replace("kernel_stats.csv", "kernel_trace.csv")
    if last > 0 and os.path.exists(trace_csv):
        per = {}
        for r in csv.DictReader(open(trace_csv)):
            per.setdefault(short_kernel_name(r["Kernel_Name"]), []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        out += ["", f"# mean of each kernel's last {last} dispatches (in launch order)",
                f"{'kernel':44s} {'calls':>6s} {'avg_us':>10s}"]
        for k, v in per.items():
            d = [x[1] for x in sorted(v)[-last:]]
            out.append(f"{k:44s} {len(d):6d} {float(np.mean(d)) / 1e3:10.2f}")
    return "\n".join(out) + "\n"


def _pmc_per_kernel(pmc_csv, counter):
    """Per-dispatch values of one counter, grouped by short kernel name, plus the
    value on the largest device-copy dispatch (the calibration copy)."""
    per = {}
    copy = (0, None)
    for r in csv.DictReader(open(pmc_csv)):
        if r["Counter_Name"] != counter:
            continue
        v = float(r["Counter_Value"])
        if "copyBuffer" in r["Kernel_Name"]:
            g = int(r["Grid_Size"])
            if g > copy[0]:
                copy = (g, v)
            continue
        per.setdefault(short_kernel_name(r["Kernel_Name"]), []).append(v)
    return per, copy[1]


def summarize_traffic(fetch_csv, write_csv, command, copy_bytes=1 << 30):
    """HBM bytes per dispatch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by
    what the same counters read for a device copy of copy_bytes."""
    fetch, cf = _pmc_per_kernel(fetch_csv, "FETCH_SIZE")
    write, cw = _pmc_per_kernel(write_csv, "WRITE_SIZE")
    if not cf or not cw:
        raise SystemExit("no calibration copy in the counter files (run bench.py with --calibrate-copy)")
    ff = copy_bytes / 1024.0 / cf
    fw = copy_bytes / 1024.0 / cw
    out = ["# HBM traffic per dispatch from rocprofv3 hardware counters", "# commands:"]
    out += ["#   " + c for c in command.split(" ;; ")]
    out += [f"# calibration: a {copy_bytes >> 20} MiB device copy reads FETCH_SIZE {cf:.1f} KiB and "
            f"WRITE_SIZE {cw:.1f} KiB, so fetch_factor {ff:.3f}, write_factor {fw:.3f}",
            "# bytes = (FETCH_SIZE * fetch_factor + WRITE_SIZE * write_factor) * 1024, averaged over dispatches",
            "", f"source_digest {kernel_source_digest()}",
            f"{'# key':30s} {'kernel':40s} {'dispatches':>10s} {'fetch_KiB_raw':>14s} {'write_KiB_raw':>14s} {'hbm_bytes':>14s}"]
    for k in sorted(fetch):
        f = float(np.mean(fetch[k]))
        w = float(np.mean(write.get(k, [0.0])))
        b = (f * ff + w * fw) * 1024.0
        out.append(f"{'traffic':30s} {k:40s} {len(fetch[k]):10d} {f:14.1f} {w:14.1f} {b:14.0f}")
    return "\n".join(out) + "\n"


XCDS = 8  # accelerator complex dies of an MI355X, each with its own GRBM_GUI_ACTIVE
CUS = 256  # compute units of an MI355X


def summarize_counters(pmc_csv, command):
    """Per-kernel means over dispatches of every counter in a rocprofv3 --pmc
    counter_collection.csv (device copies left out).  With GRBM_GUI_ACTIVE among
    them, also the engine clock of each dispatch: its active cycles, summed over
    the dies, per ns of the dispatch's own timestamps, divided by the die count
    (meaningful for dispatches much longer than the counter window's few-us
    overhang, i.e. not for the short merge kernels); with SQ_LDS_IDX_ACTIVE too,
    the LDS busy share of each dispatch: cycles the LDS served indexed reads and
    writes, summed over the compute units, per compute-unit cycle (rocprofv3's
    LdsUtil, with the per-die active cycles taken as their mean).  These two are
    medians over the dispatches, so that the first, cold dispatch of a process
    does not weigh in."""
    vals = {}
    per = {}  # (kernel, dispatch) -> {counter: value, "dur": ns}
    for r in csv.DictReader(open(pmc_csv)):
        if "copyBuffer" in r["Kernel_Name"]:
            continue
        k = short_kernel_name(r["Kernel_Name"])
        v = float(r["Counter_Value"])
        vals.setdefault((k, r["Counter_Name"]), []).append(v)
        d = per.setdefault((k, r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = v
        d["dur"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    clock, lds = {}, {}
    for (k, _), d in per.items():
        if "GRBM_GUI_ACTIVE" in d:
            clock.setdefault(k, []).append(d["GRBM_GUI_ACTIVE"] / max(d["dur"], 1) / XCDS)
            if "SQ_LDS_IDX_ACTIVE" in d:
                lds.setdefault(k, []).append(
                    100.0 * d["SQ_LDS_IDX_ACTIVE"] / max(d["GRBM_GUI_ACTIVE"] / XCDS * CUS, 1.0))
    for k, v in clock.items():
        vals[(k, "clock_GHz")] = [float(np.median(v))]
    for k, v in lds.items():
        vals[(k, "lds_busy_pct")] = [float(np.median(v))]
    counters = sorted({c for _, c in vals})
    kernels = sorted({k for k, _ in vals})
    out = ["# rocprofv3 hardware counters, mean per dispatch", "# command:", "#   " + command,
           f"# kernel sources digest: {kernel_source_digest()}", "",
           f"{'kernel':40s} {'dispatches':>10s} " + " ".join(f"{c:>16s}" for c in counters)]
    for k in kernels:
        n = max(len(vals.get((k, c), [])) for c in counters)
        out.append(f"{k:40s} {n:10d} " + " ".join(
            f"{float(np.mean(vals[(k, c)])):16.4g}" if (k, c) in vals else f"{'-':>16s}" for c in counters))
    return "\n".join(out) + "\n"


def read_traffic(kernel_prefix, path=TRAFFIC_SUMMARY):
    """HBM bytes per dispatch of the first kernel whose short name starts with
    kernel_prefix, from the committed counter summary; None when the summary is
    missing or was taken on other kernel sources."""
    if not os.path.exists(path):
        return None
    digest = None
    for line in open(path):
        f = line.split()
        if len(f) == 2 and f[0] == "source_digest":
            digest = f[1]
        elif len(f) == 6 and f[0] == "traffic" and f[1].startswith(kernel_prefix):
            return int(float(f[5])) if digest == kernel_source_digest() else None
    return None


# ---------------------------------------------------------------------------


PREWARM_S = 0.5  # untimed steps before the warm-up steps (clock ramp)
EXTRA_PREWARM_S = 0.25  # the same before each of the other workloads


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_op(torch, run, iters, warmup, prewarm_s=EXTRA_PREWARM_S):
    """Average ms of run() over iters launches, events on the current stream (for
    calls without an operation object); about prewarm_s seconds of untimed calls
    first (clock ramp, as in time_ops)."""
    t0 = time.perf_counter()
    run()
    torch.cuda.synchronize()
    n = max(warmup, int(prewarm_s / max(time.perf_counter() - t0, 1e-4)))
    for _ in range(n):
        run()
    torch.cuda.synchronize()
    evs = [_events(torch) for _ in range(iters)]
    for a, b in evs:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs]))


def launch_events(torch, n):
    """n pairs of timing events, created (HIP events exist only after a first record)."""
    evs = [_events(torch) for _ in range(n)]
    for a, b in evs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    return evs


def time_ops(torch, ops, iters, warmup, prewarm_s=EXTRA_PREWARM_S):
    """Average ms of one call over iters back-to-back calls of the operations in turn,
    from events recorded on each call's own kernels (its first kernel's start, its
    last kernel's end: mpaOperationSetLaunchEvents), so no command sits between the
    calls on the stream.  The warm-up calls carry the same events: the first
    launch that records a given event that way runs several times slower, and
    must not be a timed one.  Before them, about prewarm_s seconds of untimed
    calls run back to back, so that the clocks have left their idle state (the
    inputs of each workload are made on the host first, and the GPU idles
    meanwhile)."""
    evs = launch_events(torch, iters)
    if prewarm_s > 0:
        t0 = time.perf_counter()
        ops[0].set_launch_events(*evs[0])
        ops[0].run()
        torch.cuda.synchronize()
        n = max(1, int(prewarm_s / max(time.perf_counter() - t0, 1e-4)))
        for i in range(n):
            op = ops[i % len(ops)]
            op.set_launch_events(*evs[i % iters])
            op.run()
        torch.cuda.synchronize()
    for i in range(max(warmup, iters)):
        op = ops[i % len(ops)]
        op.set_launch_events(*evs[i % iters])
        op.run()
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        op = ops[i % len(ops)]
        op.set_launch_events(a, b)
        op.run()
    torch.cuda.synchronize()
    for op in ops:
        op.set_launch_events(None, None)
    return float(np.mean([a.elapsed_time(b) for a, b in evs]))


_CPU_CASE = None  # oracle arguments of the workload the CPU baseline samples (set before forking)


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    global _CPU_LIMIT
    _CPU_LIMIT = threadpool_limits(1)  # one BLAS thread per worker process


def _cpu_pair(bh):
    """Oracle output of every row of one (sequence, head) pair; returns the pair's
    valid FLOPs."""
    import oracle
    b, h = bh
    args = _CPU_CASE
    L = int(args["seq_len"][b])
    oracle.prefix_encoder_rows(rows=[(b, i, h) for i in range(L)], **args)
    return prefill_valid_flops([L], [int(args["kv_seq_len"][b])], True, 1, args["query"].shape[-1])


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, name, max_workers=16, max_pairs=40):
    """The fp64 oracle, as it is, on a bounded sample of the workload: up to
    max_pairs whole (sequence, head) pairs (every row of the pair; for the
    16384-token workload that is all 40 heads), spread over worker processes
    with one BLAS thread each, as many workers as the host allows (at most
    max_workers), timed by the wall clock."""
    import multiprocessing as mp
    global _CPU_CASE
    _CPU_CASE = case.oracle_args()
    n_cpu = os.cpu_count() or 1
    workers = max(1, min(max_workers, n_cpu))
    pairs = [(b, h) for b in range(case.batch) for h in range(case.head_num)]
    order = np.random.default_rng(0).permutation(len(pairs))[:max_pairs]
    todo = [pairs[k] for k in order]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
        flops = sum(pool.map(_cpu_pair, todo, chunksize=1))
    dt = time.perf_counter() - t0
    _CPU_CASE = None
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"{len(todo)} whole (sequence, head) pairs of the {name} workload, all rows each "
                      f"({len(todo)} of {len(pairs)} pairs; fp64 numpy), {workers} worker processes "
                      f"x 1 BLAS thread, {dt:.1f} s wall",
            "cpu_model": _cpu_model(), "os_cpu_count": n_cpu, "threads_per_worker": 1,
            "seconds": round(dt, 2), "valid_flops": int(flops)}


def measure_peaks(torch, command, iters=20):
    """Achievable rates of the GPU, as context for the published peaks the roofline
    uses: a 1 GiB device-to-device copy (HBM read + write) and an 8192^3 bf16
    GEMM through torch (the vendor BLAS), each timed with events over `iters`
    calls after a warm-up."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lines = [f"command: {command}" if command else "command: python bench.py --peaks",
             f"device: {torch.cuda.get_device_name(dev)}"]
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)

    def timed(fn):
        for _ in range(5):
            fn()
        a, b = _events(torch)
        torch.cuda.synchronize()
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    ms = timed(lambda: dst.copy_(src))
    gbs = 2 * (1 << 30) / (ms * 1e-3) / 1e9
    lines.append(f"copy 1 GiB -> 1 GiB: {ms:.4f} ms per copy, {gbs:.1f} GB/s read + write "
                 f"({gbs / 8000:.3f} of 8 TB/s)")
    del src, dst
    n = 8192
    g = torch.Generator(device=dev).manual_seed(5)
    a = torch.randn(n, n, dtype=torch.bfloat16, device=dev, generator=g)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=dev, generator=g)
    ms = timed(lambda: torch.matmul(a, b))
    tf = 2 * n ** 3 / (ms * 1e-3) / 1e12
    lines.append(f"bf16 GEMM {n}x{n}x{n} (torch.matmul): {ms:.4f} ms, {tf:.1f} TFLOP/s "
                 f"({tf / 2500:.3f} of 2.5 PFLOP/s dense)")
    return "\n".join(lines) + "\n"


def _sum_or_none(*xs):
    return None if any(x is None for x in xs) else int(sum(xs))


# The step's prefill workload (the sqrt call; the left-aligned call reads the same inputs).
HEADLINE = "alibi_sqrt_16384"



def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB device copy first (reference for HBM byte counters)")
    ap.add_argument("--summarize-stats", metavar="KERNEL_STATS_CSV",
                    help="print a text summary of a rocprofv3 kernel_stats.csv and exit")
    ap.add_argument("--last", type=int, default=0,
                    help="with --summarize-stats: also the mean of each kernel's last N dispatches")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print HBM bytes per dispatch from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-counters", metavar="COUNTER_CSV",
                    help="print per-kernel means of a rocprofv3 --pmc counter_collection.csv and exit")
    ap.add_argument("--command", default="", help="the profiling command(s), recorded in a summary")
    ap.add_argument("--peaks", action="store_true",
                    help="measure the achievable HBM copy rate and bf16 GEMM rate of the GPU and exit")
    args = ap.parse_args()
    if args.summarize_stats:
        sys.stdout.write(summarize_kernel_stats(args.summarize_stats, args.command, args.last))
        return
    if args.summarize_traffic:
        sys.stdout.write(summarize_traffic(*args.summarize_traffic, args.command))
        return
    if args.summarize_counters:
        sys.stdout.write(summarize_counters(args.summarize_counters, args.command))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W

    if args.peaks:
        sys.stdout.write(measure_peaks(torch, args.command))
        return

    # Inputs of the headline prefill workload, generated on the host; the CPU
    # baseline runs the oracle on them before anything touches the GPU (its
    # worker processes are forked from this one).
    print("bench: generating inputs", file=sys.stderr, flush=True)
    hc = W.make_prefill_config(HEADLINE)
    cpu = None
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(hc, "1 x 16384-token sqrt ALiBi (40 heads, headSize 128, bf16)")
        print(f"bench: cpu baseline {cpu['value']:.3e} TFLOP/s on {cpu['cores']} processes "
              f"({cpu['seconds']} s)", file=sys.stderr, flush=True)

    import masked_paged_attention_amd as mpa
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # --- prefill: the 16384-token sequence, sqrt and left-aligned ALiBi (same inputs) ---
    pc = hc.to(dev)
    del hc
    p_out = torch.empty_like(pc.query)
    p_lse = torch.empty((pc.n_tokens, pc.head_num), dtype=torch.float32, device=dev)
    p_slopes = torch.as_tensor(pc.slopes, device=dev)
    p_ops = [mpa.PrefixEncoder(pc.query, pc.key, pc.value, pc.block_tables, pc.seq_len, pc.kv_seq_len,
                               mask_type=mt, qk_scale=pc.qk_scale, slopes=p_slopes, out=p_out, lse=p_lse)
             for mt in (mpa.MASK_ALIBI_SQRT, mpa.MASK_ALIBI_LEFT)]
    p_flops = prefill_valid_flops(pc.seq_len, pc.kv_seq_len, True, pc.head_num, pc.head_size)  # per call

    # --- decode workload: two independent caches, rotated per step ---
    mcs = [W.make_mla_config("mla_decode_q1", device=dev)]
    m2 = W.make_mla_config("mla_decode_q1", device="cpu")
    # second copy: the same values relocated to other blocks (other memory), so
    # consecutive steps never find the previous step's KV in the Infinity Cache
    perm = torch.randperm(m2.ct_kv.shape[0], generator=torch.Generator().manual_seed(77))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(perm.numel())
    import dataclasses
    m2 = dataclasses.replace(m2, ct_kv=m2.ct_kv[perm].contiguous(), k_rope=m2.k_rope[perm].contiguous(),
                             block_tables=inv[m2.block_tables.long()].to(torch.int32))
    mcs.append(m2.to(dev))
    m_out = torch.empty_like(mcs[0].q_nope)
    m_lse = torch.empty((mcs[0].n_tokens, mcs[0].head_num), dtype=torch.float32, device=dev)
    m_ops = [mpa.MLA(m.q_nope, m.q_rope, m.ct_kv, m.k_rope, m.block_tables, m.context_lens,
                     qk_scale=m.qk_scale, out=m_out, lse=m_lse) for m in mcs]
    m0 = mcs[0]
    m_bytes = mla_bytes(m0.context_lens, m0.n_tokens, m0.head_num, max_blocks=m0.max_block_num)
    m_flops = mla_flops(m0.context_lens, None, m0.head_num, False)

    # Per-call times come from events recorded on the calls' own kernels (start of
    # the first, end of the last: mpaOperationSetLaunchEvents), so nothing but the
    # calls' own commands sits on the stream inside the timed region.
    def step(i, ev=None):
        if ev is not None:
            for op, e in zip(p_ops, ev[:2]):
                op.set_launch_events(*e)
            m_ops[i % 2].set_launch_events(*ev[2])
        for op in p_ops:
            op.run()
        m_ops[i % 2].run()

    # The GPU leaves its idle clocks over the first few tens of milliseconds of
    # work (the first calls of a fresh process run up to 3x slower): the step runs
    # untimed, back to back, for about PREWARM_S seconds before the W warm-up
    # steps.
    print("bench: clock pre-warm + warmup", file=sys.stderr, flush=True)
    # (the timing events exist before the warm-up: creating them between the
    # warm-up and the timed steps would leave the GPU idle there)
    evs = [launch_events(torch, 3) for _ in range(args.steps)]
    t_start, t_end = _events(torch)
    t_pw = time.perf_counter()
    step(0)
    torch.cuda.synchronize()
    t_one = max(time.perf_counter() - t_pw, 1e-3)
    # (the untimed steps carry the timed steps' events: the first launch that
    # records a given event on its kernel runs several times slower, and must
    # not be a timed one)
    for i in range(max(1, int(PREWARM_S / t_one))):
        step(i, evs[i % args.steps])
    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i, evs[i % args.steps])
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(i, evs[i])
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    sq_all = [e[0][0].elapsed_time(e[0][1]) for e in evs]
    lf_all = [e[1][0].elapsed_time(e[1][1]) for e in evs]
    m_all = [e[2][0].elapsed_time(e[2][1]) for e in evs]
    sq_ms, lf_ms, m_ms = float(np.mean(sq_all)), float(np.mean(lf_all)), float(np.mean(m_all))

    def spread(ts):
        # the spread of one call's launches over the timed steps (the rates above
        # use the mean of all of them)
        return {"ms_median": round(float(np.median(ts)), 5), "ms_min": round(float(np.min(ts)), 5),
                "ms_max": round(float(np.max(ts)), 5)}
    for op in p_ops + m_ops:
        op.set_launch_events(None, None)
    p_tflops = 2 * p_flops / ((sq_ms + lf_ms) * 1e-3) / 1e12
    sq_tf = p_flops / (sq_ms * 1e-3) / 1e12
    lf_tf = p_flops / (lf_ms * 1e-3) / 1e12
    m_gbs = m_bytes / (m_ms * 1e-3) / 1e9
    print(f"bench: prefill sqrt {sq_ms:.4f} ms {sq_tf:.1f} TFLOP/s, left {lf_ms:.4f} ms {lf_tf:.1f} TFLOP/s; "
          f"decode {m_ms:.4f} ms {m_gbs:.0f} GB/s", file=sys.stderr, flush=True)
    # the dominant kernel of the step: the slower of the two prefill launches
    dom_name, dom_ms, dom_tf = max([("prefill_dma_kernel<bf16,4>", sq_ms, sq_tf),
                                    ("prefill_dma_kernel<bf16,5>", lf_ms, lf_tf)], key=lambda x: x[1])
    del pc, p_out, p_lse, p_ops
    torch.cuda.empty_cache()

    extra = {}
    if not args.no_extra:
        def prefill_extra(name, c, tile=None, fl=None):
            sl = torch.as_tensor(c.slopes, device=dev) if c.slopes is not None else None
            op = mpa.PrefixEncoder(c.query, c.key, c.value, c.block_tables, c.seq_len, c.kv_seq_len,
                                   mask_type=c.mask_type, qk_scale=c.qk_scale, slopes=sl,
                                   q_start_loc=c.q_start_loc, return_lse=True, compressed_mask=tile,
                                   attention_chunk=c.chunk if c.chunk else None)
            ms = time_ops(torch, [op], 10, 3)
            if fl is None:
                fl = prefill_valid_flops(c.seq_len, c.kv_seq_len, True, c.head_num, c.head_size)
            tf = fl / (ms * 1e-3) / 1e12
            e = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_mfma": round(tf / PEAK_MFMA_TFLOPS, 4)}
            if c.q_start_loc is not None:
                e["padding_positions"] = padding_positions(c.seq_len, 8192)
            extra[name] = e
            op.close()
            torch.cuda.empty_cache()

        # the prefix-encoder causal GQA workload, then the same call reading the
        # page's compressed norm tile
        print("bench: extra prefix_gqa_causal", file=sys.stderr, flush=True)
        c = W.make_prefill_config("prefix_gqa_causal", device=dev)
        prefill_extra("prefix_gqa_causal", c)
        prefill_extra("prefix_gqa_causal_norm_tile", c, W.compressed_tile(c.mask_type, c.dtype).to(dev))
        extra["prefix_gqa_causal"]["valid_flops"] = int(
            prefill_valid_flops(c.seq_len, c.kv_seq_len, True, c.head_num, c.head_size))
        del c
        print("bench: extra alibi_right_4x4096", file=sys.stderr, flush=True)
        c = W.make_prefill_config("alibi_right_4x4096", device=dev)
        prefill_extra("alibi_right_4x4096", c)
        prefill_extra("alibi_right_4x4096_tile", c, W.compressed_tile(c.mask_type, c.dtype).to(dev))
        del c
        # the 16384-token calls reading the [256,256] compressed tiles
        for name in ["alibi_sqrt_16384", "alibi_left_16384"]:
            print(f"bench: extra {name}_tile", file=sys.stderr, flush=True)
            c = W.make_prefill_config(name, device=dev)
            prefill_extra(name + "_tile", c, W.compressed_tile(c.mask_type, c.dtype).to(dev))
            del c
        # the same sqrt call over a cache of 16-key blocks (4 blocks per 64-key tile)
        print("bench: extra alibi_sqrt_16384_bs16", file=sys.stderr, flush=True)
        c = W.make_prefill(1003, np.array([16384]), np.array([16384]), 40, 40, 128, 16, "bf16", 4,
                           1.0 / np.sqrt(128.0), slopes="alibi").to(dev)
        prefill_extra("alibi_sqrt_16384_bs16", c)
        del c
        for name in ["alibi_sqrt_varlen16", "alibi_sqrt_padded16", "alibi_left_varlen16", "alibi_left_padded16"]:
            print(f"bench: extra {name}", file=sys.stderr, flush=True)
            c = W.make_prefill_config(name, device=dev)
            prefill_extra(name, c)
            del c
        # chunked local causal mask over one 16384-token bf16 sequence, 40 heads, chunk 2048
        print("bench: extra chunked_16384_c2048", file=sys.stderr, flush=True)
        cc = W.make_prefill(87, np.array([16384]), np.array([16384]), 40, 40, 128, 128, "bf16", 9,
                            1.0 / np.sqrt(128.0), chunk=2048).to(dev)
        prefill_extra("chunked_16384_c2048", cc,
                      fl=prefill_valid_flops_chunked(cc.seq_len, cc.kv_seq_len, cc.chunk, cc.head_num,
                                                     cc.head_size))
        del cc
        print("bench: extra mla_spec_q4", file=sys.stderr, flush=True)
        m4 = W.make_mla_config("mla_spec_q4", device=dev)
        op4 = mpa.MLA(m4.q_nope, m4.q_rope, m4.ct_kv, m4.k_rope, m4.block_tables, m4.context_lens,
                      qk_scale=m4.qk_scale, q_seq_len=m4.q_seq_len, mask_type=m4.mask_type,
                      return_lse=True)
        ms = time_ops(torch, [op4], 10, 3)
        fl = mla_flops(m4.context_lens, m4.q_seq_len, m4.head_num, True)
        by = mla_bytes(m4.context_lens, m4.n_tokens, m4.head_num, max_blocks=m4.max_block_num)
        extra["mla_spec_q4"] = {"ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                                "frac_mfma": round(fl / (ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
                                "gbs": round(by / (ms * 1e-3) / 1e9, 1)}
        op4.close()
        del m4, op4
        # MLA calcType PREFILL: 4 prompts of 256 new tokens over 1-4k keys, causal.
        print("bench: extra mla_prefill", file=sys.stderr, flush=True)
        ctx_p = np.array([1024, 2048, 3072, 4096], dtype=np.int32)
        ql_p = np.full(4, 256, dtype=np.int32)
        mp = W.make_mla(81, ctx_p, ql_p, 128, 128, "bf16", 1, 3, 1, 1.0 / np.sqrt(192.0)).to(dev)
        opp = mpa.MLA(mp.q_nope, mp.q_rope, mp.ct_kv, mp.k_rope, mp.block_tables, mp.context_lens,
                      qk_scale=mp.qk_scale, q_seq_len=mp.q_seq_len, mask_type=mp.mask_type,
                      calc_type=mp.calc_type, return_lse=True)
        ms = time_ops(torch, [opp], 10, 3)
        fl = mla_flops(mp.context_lens, mp.q_seq_len, mp.head_num, True)
        extra["mla_prefill"] = {"ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                                "frac_mfma": round(fl / (ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
                                "shape": "4 x 256 tokens, ctx 1024..4096, 128 heads, causal"}
        opp.close()
        del mp, opp
        # MLA decode over the int8 latent cache, the decode workload's shape; two
        # caches alternate (2 x 189 MB > the 256 MB Infinity Cache).
        print("bench: extra mla_int8_decode_q1", file=sys.stderr, flush=True)
        rng8 = np.random.default_rng(1001)
        ctx8 = rng8.integers(1024, 8192, size=64, endpoint=True)
        m8 = [W.make_mla_int8(3101 + i, ctx8, None, 128, 128, "bf16", 0, 0, 1.0 / np.sqrt(192.0),
                              max_block_num=64).to(dev) for i in range(2)]
        o8 = torch.empty((m8[0].n_tokens, 128, 512), dtype=torch.bfloat16, device=dev)
        l8 = torch.empty((m8[0].n_tokens, 128), dtype=torch.float32, device=dev)
        ops8 = [mpa.MLA(m.q_nope, m.q_rope, m.ct_kv, m.k_rope, m.block_tables, m.context_lens,
                        qk_scale=m.qk_scale, out=o8, lse=l8,
                        qk_descale=torch.as_tensor(m.qk_descale, device=dev),
                        pv_descale=torch.as_tensor(m.pv_descale, device=dev)) for m in m8]
        ms = time_ops(torch, ops8, 20, 4)
        by = mla_bytes_int8(ctx8, m8[0].n_tokens, 128, max_blocks=64)
        fl = mla_flops(ctx8, None, 128, False)
        extra["mla_int8_decode_q1"] = {"ms": round(ms, 4), "gbs": round(by / (ms * 1e-3) / 1e9, 1),
                                       "frac_hbm": round(by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                       "tflops": round(fl / (ms * 1e-3) / 1e12, 1), "bytes": by}
        for op8 in ops8:
            op8.close()
        del m8, ops8, o8, l8
        # LSE merge of 8 partials shaped like the prefix-encoder workload's output
        # (4624 tokens x 32 heads x 128; HBM-bound; 8 x 38 MB of partials)
        print("bench: extra lse_merge", file=sys.stderr, flush=True)
        n_parts, n_tok, n_h, hd = 8, 4624, 32, 128
        rows = n_tok * n_h
        g = torch.Generator(device=dev).manual_seed(5)
        o_parts = torch.randn((n_parts, n_tok, n_h, hd), generator=g, device=dev).to(torch.bfloat16)
        l_parts = torch.randn((n_parts, n_tok, n_h), generator=g, device=dev) * 4.0
        mo = torch.empty_like(o_parts[0])
        ml = torch.empty_like(l_parts[0])
        ms = time_op(torch, lambda: mpa.lse_merge(o_parts, l_parts, out=mo, lse=ml), 20, 3)
        by = (n_parts + 1) * rows * (hd * 2 + 4)
        extra["lse_merge"] = {"ms": round(ms, 4), "gbs": round(by / (ms * 1e-3) / 1e9, 1),
                              "frac_hbm": round(by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                              "parts": n_parts, "rows": rows, "head_dim": hd}
        del o_parts, l_parts, mo, ml

    res = {
        "metric": METRIC,
        "value": round(p_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "long-sequence ALiBi prefill: 1 x 16384 tokens (no prefix), 40/40 heads, headSize 128, "
                        "blockSize 128, bf16, slopes 2^(-8(h+1)/40), one sqrt-ALiBi call and one left-aligned "
                        "ALiBi call per step (value = valid FLOPs of both / their kernel time) + MLA decode "
                        "(batch 64, 128 heads, q_len 1, 576/512, blockSize 128, contextLens~U[1024,8192], "
                        "bf16, cold KV)",
            "prefill_tokens": 16384,
            "prefill_valid_flops_per_call": int(p_flops),
            "decode_batch": int(m0.batch),
            "decode_kv_keys": int(np.sum(m0.context_lens)),
        },
        "roofline": {"bound": "mfma", "kernel": dom_name,
                     "achieved": round(dom_tf, 2), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(dom_tf / PEAK_MFMA_TFLOPS, 4),
                     "traffic": read_traffic(dom_name),
                     "per_launch_flops": int(p_flops), "ms": round(dom_ms, 5)},
        "prefill": {"sqrt": {"ms": round(sq_ms, 5), "tflops": round(sq_tf, 1),
                             "frac_mfma": round(sq_tf / PEAK_MFMA_TFLOPS, 4),
                             "traffic": read_traffic("prefill_dma_kernel<bf16,4>"), **spread(sq_all)},
                    "left": {"ms": round(lf_ms, 5), "tflops": round(lf_tf, 1),
                             "frac_mfma": round(lf_tf / PEAK_MFMA_TFLOPS, 4),
                             "traffic": read_traffic("prefill_dma_kernel<bf16,5>"), **spread(lf_all)},
                    "target": "50% of dense bf16 MFMA peak (<= 2.2 ms per call)"},
        "decode": {"value": round(m_gbs, 1), "unit": "GB/s", "frac_hbm": round(m_gbs / PEAK_HBM_GBS, 4),
                   "ms": round(m_ms, 5), "bytes": int(m_bytes), **spread(m_all),
                   "tflops": round(m_flops / (m_ms * 1e-3) / 1e12, 1),
                   "traffic": _sum_or_none(read_traffic("mla_split_kernel"), read_traffic("mla_combine_kernel")),
                   "target": "70% of HBM",
                   "note": "whole MLA call (split + combine kernels)"},
        "extra": extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
