"""Benchmark: bf16 GEMM C = A.B at M = N = K = 8192 on one MI355X.

One step = one pass of the hot path over the 8192^3 workload: the planned
(XCD-grouped) GEMM kernel -- LDS staging, MFMA inner loop and epilogue in one
launch -- on inputs already resident in HBM.  Plan creation happens once,
before the timed region.

Prints ONE JSON line with the metric, the kernel's roofline position (HIP
events on the launch stream; algorithmic flops = 2*M*N*K per launch; peak =
2.5 PFLOP/s dense bf16), the HBM traffic from the committed rocprofv3 counter
summary of the workload when it was taken on the current kernel source, and the CPU oracle
timed on a bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--per-launch N]
      (defaults: warm up for about 0.5 s of launches, then time at least 50
      launches and 0.1 s; the JSON line reports the counts used.  Then N = 50
      single launches are timed warm and N cold -- each after a 1 GiB read
      that evicts L2 and the MALL -- and their median and minimum reported
      as per_launch_ms)
  python bench.py --workload NAME      other workloads (reported, not the headline);
                                       attn32x2048 is the fused attention forward
  python bench.py --tilecast           tile fan-out microbenchmark (JSON lines)
  python bench.py --profile            short run for rocprofv3 (GEMM + a copy kernel of known size)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
HEADLINE = "gemm8192"
KERNEL_SOURCES = {kind: [os.path.join(ROOT, "attention_scores_amd", "csrc", f)
                          for f in mains + ("schedule.hpp", "tile.hpp")]
                  for kind, mains in (("gemm", ("gemm.hip", "splitk.hip")), ("attn", ("attn.hip",)))}


def kernel_kind(name: str) -> str:
    from workloads import ATTN_WORKLOADS
    return "attn" if name in ATTN_WORKLOADS else "gemm"


def kernel_source_hash(kind: str = "gemm") -> str:
    """Hash of the sources of the kernel a workload runs (for stale-summary checks)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kind]:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_file(name: str) -> str:
    return os.path.join(ROOT, "profiles", "traffic_%s.txt" % name)


def read_traffic(name: str):
    """HBM bytes per launch of workload `name` from its committed counter
    summary, if that summary was taken on the current kernel source."""
    path = traffic_file(name)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(kernel_kind(name)):
        return None
    try:
        return {"read_bytes": float(vals["hbm_read_bytes_per_launch"]),
                "write_bytes": float(vals["hbm_write_bytes_per_launch"]),
                "scale": float(vals["copy_scale_factor"])}
    except (KeyError, ValueError):
        return None


def _gpu_inputs(w, dev):
    import torch
    from workloads import operands
    A, B = operands(w)
    return A.to(dev), B.to(dev)


def _plan(asl, w, flags=0):
    c_t = asl.AS_BF16 if w.out == "bf16" else asl.AS_F32
    sb = w.b_strides()
    if w.kind == "sscore":                       # B = K^T: B[d, j] = K[j, d]
        sb = (1, sb[0], sb[2])
    return asl.gemm_create(w.M, w.N, w.K, w.batch, w.a_strides(), sb, (w.N, 1, w.M * w.N),
                           asl.AS_BF16, asl.AS_BF16, c_t, flags)


WARMUP_S = 0.5      # default warm-up: launches for about this long, so the clocks settle
TIMED_S = 0.1       # default timed region: at least this long (and at least 50 launches)
PER_LAUNCH_N = 0    # after the timed region: this many single launches timed warm and cold (0: none)
FLUSH_BYTES = 1 << 30   # cold launches: this many bytes read first (4x the 256 MB MALL)
GRAPH_LAUNCHES = 20     # graph timing: launches recorded into one HIP graph
LAST_PER_LAUNCH = None  # per-launch statistics of the last _timed call, when PER_LAUNCH_N > 0


def _timed(run, steps, warmup, stream):
    """(wall ms per step, event ms per launch, steps, warmup) of launches of
    run(); steps / warmup None: sized from a short calibration (WARMUP_S,
    TIMED_S).  HIP events are recorded on the launch stream."""
    import torch
    if warmup is None or steps is None:
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        for _ in range(10):
            run()
        torch.cuda.synchronize()
        per = max((time.perf_counter() - c0) / 10, 1e-6)
        if warmup is None:
            warmup = max(30, min(20000, int(WARMUP_S / per)))
        if steps is None:
            steps = max(50, min(20000, int(TIMED_S / per)))
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        run()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if PER_LAUNCH_N > 0:
        _per_launch(run, PER_LAUNCH_N, stream)
    return (t1 - t0) * 1e3 / steps, ev0.elapsed_time(ev1) / steps, steps, warmup


def _per_launch(run, n, stream):
    """Median and minimum of n single launches (HIP events around each, on the
    launch stream), warm and then cold: before each cold launch a FLUSH_BYTES
    buffer is read on the same stream, which evicts L2 and the MALL.  It is
    read, not written: a write leaves the caches full of dirty lines that the
    measured kernel would then have to write back (the attention scores took
    a third longer after a 1 GiB write than after a 1 GiB read).  Then the
    launch time without the host: GRAPH_LAUNCHES launches recorded into one
    HIP graph (run(stream handle) launches on the capturing stream), each
    replay timed with events; reported per launch."""
    import statistics
    import torch
    global LAST_PER_LAUNCH
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=stream.device)
    sink = torch.empty((), dtype=torch.float32, device=stream.device)
    torch.cuda.synchronize()
    stats = {"launches": n, "flush_bytes_read": FLUSH_BYTES}
    for kind in ("warm", "cold"):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i, (e0, e1) in enumerate(evs):
            if kind == "cold":
                torch.amax(flush, dim=0, out=sink)
            e0.record(stream)
            run()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = [e0.elapsed_time(e1) for e0, e1 in evs]
        stats[kind + "_median"] = round(statistics.median(ms), 4)
        stats[kind + "_min"] = round(min(ms), 4)
    del flush, sink
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        for _ in range(GRAPH_LAUNCHES):
            run(cs)
    g.replay()                                   # the first replay uploads the graph
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(max(5, n // 5))]
    for e0, e1 in evs:
        e0.record(stream)
        g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) / GRAPH_LAUNCHES for e0, e1 in evs]
    stats["graph_launches"] = GRAPH_LAUNCHES
    stats["graph_median"] = round(statistics.median(ms), 4)
    stats["graph_min"] = round(min(ms), 4)
    del g
    LAST_PER_LAUNCH = stats


def time_attention(w, steps, warmup):
    """(wall ms, event ms, steps, warmup) for attention workload w."""
    import torch
    import attention_scores_amd as asl
    from workloads import attn_operands
    dev = torch.device("cuda:0")
    Q, K, V = (t.to(dev) for t in attn_operands(w))
    od = torch.bfloat16 if w.out == "bf16" else torch.float32
    O = torch.empty((w.batch, w.Lq, w.dv), dtype=od, device=dev)
    stream = torch.cuda.current_stream(dev)
    sq, sk, sv, so = w.strides()
    o_t = asl.AS_BF16 if w.out == "bf16" else asl.AS_F32
    args = (Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), w.batch, w.kv_group, w.Lq, w.Lk, w.d, w.dv,
            sq, sk, sv, so, w.scale, asl.AS_BF16, o_t, asl.AS_ATTN_CAUSAL if w.causal else 0, stream.cuda_stream)

    def run(s=None):
        asl.attn_fwd_run_gqa(*args[:-1], stream.cuda_stream if s is None else s)
    out = _timed(run, steps, warmup, stream)
    del Q, K, V, O
    return out


def time_workload(w, steps, warmup, flags=0):
    """(wall ms per step, event ms per launch, plan info, steps, warmup) for
    workload w.  steps / warmup None: sized from a short calibration so that
    the warm-up lasts WARMUP_S and the timed region at least TIMED_S (the GPU
    raises its clocks over tens of milliseconds of load, which 30 launches of
    a 0.1 ms kernel do not reach)."""
    import torch
    import attention_scores_amd as asl
    dev = torch.device("cuda:0")
    A, B = _gpu_inputs(w, dev)
    od = torch.bfloat16 if w.out == "bf16" else torch.float32
    C = torch.empty((w.batch, w.M, w.N), dtype=od, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    a, b, c = A.data_ptr(), B.data_ptr(), C.data_ptr()
    if w.kind == "sscore" and flags == 0:
        s_t = asl.AS_BF16 if w.out == "bf16" else asl.AS_F32
        sq, sk, ss = w.a_strides(), w.b_strides(), (w.N, 1, w.M * w.N)
        # the plan sscore_run makes internally, for reporting only
        plan = asl.gemm_create(w.M, w.N, w.K, w.batch, sq, (1, sk[0], sk[2]), ss, asl.AS_BF16, asl.AS_BF16, s_t)
        info = asl.gemm_plan_info(plan) + (1,)
        asl.gemm_destroy(plan)

        def run(s=None):
            asl.sscore_run(a, b, c, w.batch, w.M, w.N, w.K, sq, sk, ss, asl.AS_BF16, s_t, sh if s is None else s)
    else:
        # (the attention scores with flags, e.g. the grouping ablation: the
        # plan sscore_run makes -- A = Q, B = K^T, no split -- with the flags)
        plan = _plan(asl, w, flags | (asl.AS_FLAG_NO_SPLIT_K if w.kind == "sscore" else 0))
        info = asl.gemm_plan_info(plan) + (asl.gemm_plan_split_k(plan)[0],)

        def run(s=None):
            asl.gemm_run(plan, a, b, c, sh if s is None else s)
    wall_ms, ev_ms, steps, warmup = _timed(run, steps, warmup, stream)
    if w.kind != "sscore" or flags:
        asl.gemm_destroy(plan)
    del A, B, C
    return wall_ms, ev_ms, info, steps, warmup


# The oracle's threads: a one-GPU job gets a 16-core share of its host,
# whatever the machine reports in all (both counts are recorded).
ORACLE_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def host_cpu():
    """What the CPU baseline ran on: the machine's CPU count, the cores this
    process may use, and the CPU model."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": model}


def _oracle_rows(w, a, b, r0, nrows, threads):
    """Seconds the oracle takes for output rows r0 .. r0+nrows-1 of workload
    w (a GEMM: rows of C, whatever A's layout -- a row offset into A's storage
    with the workload's strides; the attention scores: whole slices)."""
    import oracle
    sa, sb = w.a_strides(), w.b_strides()
    t = time.perf_counter()
    if w.kind == "sscore":
        s0, ns = r0 // w.M, nrows // w.M
        oracle.sscore(a[s0 * sa[2]:], b[s0 * sb[2]:], ns, w.M, w.N, w.K, sa, sb, nthreads=threads)
    else:
        oracle.gemm(a[r0 * sa[0]:], b, 1, nrows, w.N, w.K, sa, sb, want_T=True, nthreads=threads)
    return time.perf_counter() - t


def cpu_baseline(w, target_s=15.0, single_thread_s=None):
    """The oracle, as it stands, on a bounded sample of workload w's output
    rows (the attention scores: whole slices), on ORACLE_THREADS threads;
    with single_thread_s, also a single-thread run of about that long."""
    from workloads import bits, operands
    A, B = operands(w)
    a, b = bits(A).reshape(-1), bits(B).reshape(-1)
    unit = w.M if w.kind == "sscore" else 1            # rows per sampling unit
    total_rows = w.batch * w.M
    flop_per_row = 2.0 * w.N * w.K

    def sample(threads, seconds):
        probe = max(unit, (threads + unit - 1) // unit * unit)
        t_probe = _oracle_rows(w, a, b, 0, probe, threads)
        n = int(probe * seconds / max(t_probe, 1e-3)) // probe * probe
        n = max(0, min(n, total_rows - probe))
        t_main = _oracle_rows(w, a, b, probe, n, threads) if n else 0.0
        rows, secs = probe + n, t_probe + t_main
        return rows, secs, rows * flop_per_row / secs / 1e12

    rows, secs, value = sample(ORACLE_THREADS, target_s)
    what = ("%d of %d slices of the %d x %dx%dx%d scores" % (rows // w.M, w.batch, w.batch, w.M, w.N, w.K)
            if w.kind == "sscore" else
            "%d of %d output rows of the %dx%dx%d product" % (rows, w.M, w.M, w.N, w.K))
    out = {"value": value, "unit": "TFLOP/s", "cores": ORACLE_THREADS, "kind": "oracle",
           "sample": "%s (fp64 oracle incl. the sum|a*b| pass), %.1f s on %d threads"
                     % (what, secs, ORACLE_THREADS)}
    out.update(host_cpu())
    if single_thread_s:
        rows1, secs1, value1 = sample(1, single_thread_s)
        out["single_thread"] = {"value": value1, "unit": "TFLOP/s", "rows": rows1, "seconds": round(secs1, 2)}
    return out


def cpu_baseline_attn(w, target_s=12.0):
    """The attention oracle, as it stands, on a bounded sample of query rows of w."""
    import numpy as np
    import oracle
    from workloads import attn_operands, bits
    Q, K, V = (bits(t) for t in attn_operands(w))
    threads = ORACLE_THREADS
    sq, sk, sv, _ = w.strides()

    order = np.random.default_rng(7).permutation(w.batch * w.Lq)  # rows of every cost, in any prefix

    def rows_job(r0, n):
        flat = order[r0:r0 + n]
        rows = np.stack([flat // w.Lq, flat % w.Lq], axis=1)
        t = time.perf_counter()
        oracle.attention(Q, K, V, w.batch, w.Lq, w.Lk, w.d, w.dv, sq, sk, sv, w.scale, rows=rows,
                         nthreads=threads, causal=w.causal, kv_group=w.kv_group)
        secs = time.perf_counter() - t
        keys = (rows[:, 1] + (w.Lk - w.Lq) + 1).sum() if w.causal else n * w.Lk   # keys each row sees
        return secs, 2.0 * float(keys) * (w.d + w.dv)

    probe = threads
    t_probe, f_probe = rows_job(0, probe)
    n = max(threads, int(probe * target_s / max(t_probe, 1e-3)) // threads * threads)
    n = min(n, w.batch * w.Lq - probe)
    t_main, f_main = rows_job(probe, n)
    rows, secs, flop = probe + n, t_probe + t_main, f_probe + f_main
    out = {"value": flop / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": "%d of %d query rows (fp64 oracle incl. the sum p|v| pass), %.1f s on %d threads"
                     % (rows, w.batch * w.Lq, secs, threads)}
    out.update(host_cpu())
    return out


def tilecast_report(iters=5000):
    """Fan-out microbenchmark: grouped vs ungrouped, hot-tile and streaming."""
    import torch
    import attention_scores_amd as asl
    dev = torch.device("cuda:0")
    lines = []
    for rows, cols, label in ((4096, 4096, "32MiB"), (32768, 16384, "1GiB")):
        buf = torch.randint(-32768, 32768, (rows, cols), dtype=torch.int16, device=dev).view(torch.bfloat16)
        tile_bytes = 128 * 64 * 2
        for stride_kind in ("hot", "stream"):
            for group in (1, 2, 4, 8, 16, 32):
                for grouped in (True, False):
                    if group == 1 and not grouped:
                        continue
                    stride = 0 if stride_kind == "hot" else 256 // group
                    out = torch.zeros(512, dtype=torch.int32, device=dev)
                    asl.tilecast(buf, 128, 64, 256, group, grouped, 50, 0, stride, out)
                    torch.cuda.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    asl.tilecast(buf, 128, 64, 256, group, grouped, iters, 0, stride, out)
                    e1.record()
                    torch.cuda.synchronize()
                    ms = e0.elapsed_time(e1)
                    delivered = 256 * iters * tile_bytes
                    lines.append({"bench": "tilecast", "matrix": label, "scenario": stride_kind, "group": group,
                                  "grouped": grouped, "ms": ms, "delivered_GBps": delivered / ms / 1e6,
                                  "consumers": 256, "iters": iters, "tile": "128x64 bf16"})
        del buf
    return lines


def profile_run(steps, name=HEADLINE, flags=0):
    """Short run for counter collection: one workload, then a copy kernel of known size."""
    import torch
    from workloads import ATTN_WORKLOADS, WORKLOADS
    if name in ATTN_WORKLOADS:
        time_attention(ATTN_WORKLOADS[name], steps, 1)
    else:
        time_workload(WORKLOADS[name], steps, 1, flags)
    n = 1 << 29                                  # 1 GiB of bf16 read, 1 GiB written
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"profile": "done", "gemm_launches": steps + 1, "copy_bytes_each_way": 2 * n,
                      "copy_launches": steps}))


METRIC = "bf16 GEMM TFLOP/s at 8192^3 (MFMA util %); HBM bytes read / compulsory bytes"


def attention_line(w, args):
    """The JSON line for a fused-attention workload (MFMA-bound: 2*(d+dv) flop per visible
    (query, key) pair, b*Lq*Lk of them without the causal mask)."""
    import attention_scores_amd as asl
    wall_ms, ev_ms, steps, warmup = time_attention(w, args.steps, args.warmup)
    qw, kps, wgs = asl.attn_fwd_plan_info(w.batch, w.Lq, asl.AS_ATTN_CAUSAL if w.causal else 0)
    achieved = w.flop / (ev_ms * 1e-3) / 1e12
    traffic = read_traffic(w.name)
    out = {
        "metric": METRIC,
        "value": round(w.flop / (wall_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, %s)" % w.dist,
        "config": {"workload": w.description, "batch": w.batch, "Lq": w.Lq, "Lk": w.Lk, "d": w.d, "dv": w.dv,
                   "causal": w.causal, "kv_group": w.kv_group, "queries_per_workgroup": qw, "keys_per_stage": kps,
                   "workgroups": wgs},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": (traffic["read_bytes"] + traffic["write_bytes"]) if traffic else None,
                     "kernel_ms": round(ev_ms, 4)},
        "hbm_bytes_per_s_compulsory": round((w.bytes_in + w.bytes_out) / (ev_ms * 1e-3) / 1e9, 1),
        "hbm_read_over_compulsory": (round(traffic["read_bytes"] / w.bytes_in, 3) if traffic else None),
    }
    if LAST_PER_LAUNCH:
        out["per_launch_ms"] = LAST_PER_LAUNCH
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_attn(w)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed launches (default: >= 50 and >= %.1f s)" % TIMED_S)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed launches first (default: about %.1f s worth, >= 30)" % WARMUP_S)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tilecast", action="store_true")
    ap.add_argument("--profile", action="store_true")
    ap.add_argument("--flags", type=int, default=0)
    ap.add_argument("--per-launch", type=int, default=50,
                    help="single launches timed warm and cold after the timed region (0: skip)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path; "
              "got --gpus %d" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_scores_amd as asl
    from workloads import WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    asl.lib()

    if args.profile:
        profile_run(args.steps if args.steps else 3, args.workload, args.flags)
        return
    if args.tilecast:
        for line in tilecast_report():
            print(json.dumps(line))
        return

    global PER_LAUNCH_N
    PER_LAUNCH_N = max(0, args.per_launch)
    from workloads import ATTN_WORKLOADS
    if args.workload in ATTN_WORKLOADS:
        print(json.dumps(attention_line(ATTN_WORKLOADS[args.workload], args)))
        return
    w = WORKLOADS[args.workload]
    wall_ms, ev_ms, info, steps, warmup = time_workload(w, args.steps, args.warmup, args.flags)
    flop = w.flop
    value = flop / (wall_ms * 1e-3) / 1e12
    achieved = flop / (ev_ms * 1e-3) / 1e12
    traffic = read_traffic(w.name)
    compulsory_read = w.bytes_a + w.bytes_b
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": (traffic["read_bytes"] + traffic["write_bytes"]) if traffic else None,
                "kernel_ms": round(ev_ms, 4)}
    if w.name != HEADLINE and w.flop / (w.bytes_a + w.bytes_b + w.bytes_c) < PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3:
        gbs = (w.bytes_a + w.bytes_b + w.bytes_c) / (ev_ms * 1e-3) / 1e9
        roofline.update({"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4)})
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "strong",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, %s)" % w.dist,
        "config": {"workload": w.description, "M": w.M, "N": w.N, "K": w.K, "batch": w.batch,
                   "tile": "%dx%dx%d" % (info[0], info[1], info[2]), "tiles": info[3], "workgroups": info[4],
                   "split_k": info[5],
                   "grouping": "none" if args.flags & asl.AS_FLAG_NO_GROUPING else "xcd-grouped"},
        "roofline": roofline,
        "mfma_util": round(achieved / PEAK_BF16_TFLOPS, 4),
        "hbm_read_over_compulsory": (round(traffic["read_bytes"] / compulsory_read, 3) if traffic else None),
    }
    if LAST_PER_LAUNCH:
        out["per_launch_ms"] = LAST_PER_LAUNCH
    if not args.no_cpu_baseline:
        # single-thread times too where they take seconds (512^3, the attention scores)
        out["cpu_baseline"] = cpu_baseline(w, single_thread_s=(8.0 if w.flop < 1e11 else None))
    print(json.dumps(out))


if __name__ == "__main__":
    main()
