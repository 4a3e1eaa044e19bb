"""Benchmark of the smooth-K low-precision Ulysses pack/unpack on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input held in HBM:
the Q/K statistics (grouped amax + boundary min/max, every rank), the boundary derive, the
pack of every rank into the all-to-all buffer, and the unpack of every destination.  Two
forms of the step give identical bytes: the one-read form (statistics and the pack from
one read of Q, K and V; then derive with the pack of the slots that waited for it; then
the unpack: three launches), whose K timed steps give ms_per_step, and the separate form
(statistics, derive, pack, unpack: four launches, the pages' own sequence), timed the same
way after it.  The default workload is the largest configuration, long_unaligned (B=1,
world_size 8, L=9360, H=40, D=128, bf16, used 74000).  Inputs and outputs rotate over
several buffer sets so that each step reads data last touched several steps earlier (the
sets together exceed the 256 MB last-level cache).

Timing uses HIP events on the stream every launch goes to, placed only at the two ends of
each timed region (an event recorded between two launches costs about 2 us of GPU time,
more than 5 % of a small workload's kernel).  After the steps, K launches of each kernel
alone give its average duration (pack_ms, unpack_ms, stats_ms, derive_ms; the roofline
figure uses pack_ms), and K back-to-back pack+unpack pairs give the reported value:
pack+unpack algorithmic bytes / average pair time.  Each of these per-kernel loops is
preceded by three untimed calls and timed five times; the median loop is reported.  The
global K mean (an input of the step) is timed the same way, as k_mean GB/s.  The CPU
oracle is timed on the host's cores on the same inputs (cpu_baseline).  Prints one JSON
line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E peak
REPS = 5                        # timed loops per kernel figure (the median loop is reported)
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["precision_attention_input_amd/csrc/pack.hip",
                  "precision_attention_input_amd/csrc/ulp_device.h",
                  "precision_attention_input_amd/csrc/pack_device.h"]


def algorithmic_bytes(w, v_scale: bool = False) -> dict:
    """Bytes the method must move (read + write), per step, by kernel.
    N = B*S*H*D elements per tensor, e = 2 bytes, sigma = slots(L), W = scale width."""
    import precision_attention_input_amd as ulp
    e = 2
    B, P, L, H, D = w.B, w.P, w.L, w.H, w.D
    S = P * L
    N = B * S * H * D
    sigma = ulp.slots(L)
    Wd = ulp.scale_widths(w.scale_sequence or S)[0]
    spad = (S + 63) // 64 * 64
    pack = 3 * e * N + 8 * B * H * sigma * P + P * e * B * H * D + 3 * N + 8 * B * H * sigma * P
    if v_scale:
        pack += P * 4 * B * H * D          # every rank reads the caller's [B,H,D] V scale
    unpack = 3 * N + 8 * B * H * Wd + 2 * N + B * D * H * spad + 8 * B * H * Wd
    # fused statistics: read Q and K once, the mean per rank; write both amax tensors and
    # both boundary min/max tensors
    stats = 2 * e * N + P * e * B * H * D + 2 * 4 * B * H * sigma * P + 2 * 4 * P * B * H * 4 * D
    # global K mean: read the live rows of K once, write the binary32 and dtype means
    used = w.used or S
    k_mean = e * B * used * H * D + (4 + e) * B * H * D
    return dict(pack=pack, unpack=unpack, stats=stats, k_mean=k_mean, N=N)


UNPACK_SOURCES = ["precision_attention_input_amd/csrc/unpack.hip",
                  "precision_attention_input_amd/csrc/ulp_device.h"]


def kernel_hash(sources=None) -> str:
    """Hash of a kernel's source (the pack's by default) with comments and whitespace
    removed, so that the recorded traffic stays attached to the code it was measured on,
    not to its comments."""
    import re
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes measured with rocprofv3 counters for the current kernel sources:
    (pack: copy-scaled FETCH_SIZE + WRITE_SIZE, pack: DRAM request bytes, unpack: DRAM
    request bytes), each per launch, or None where not recorded for the current source."""
    path = os.path.join(PROFILES, f"pack_kernel_{workload}_traffic.json")
    if not os.path.exists(path):
        return None, None, None
    with open(path) as f:
        rec = json.load(f)
    pack_ok = rec.get("kernel_hash") == kernel_hash()
    unpack_ok = rec.get("unpack_kernel_hash") == kernel_hash(UNPACK_SOURCES)
    return (rec.get("hbm_bytes_per_launch") if pack_ok else None,
            rec.get("dram_request_bytes_per_launch") if pack_ok else None,
            rec.get("unpack_dram_request_bytes_per_launch") if unpack_ok else None)


def _pmc_means(paths: list[str], kernel: str) -> dict:
    """Mean value per dispatch of every counter recorded for the kernels whose name contains
    `kernel`, over rocprofv3 counter_collection.csv files."""
    import csv
    vals: dict = {}
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                if kernel in r["Kernel_Name"]:
                    vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no counter rows for {kernel} in {paths}")
    return {c: sum(v) / len(v) for c, v in vals.items()}


def _need(table: dict, *names):
    missing = [n for n in names if n not in table]
    if missing:
        raise SystemExit(f"counters missing from the files: {missing}")


def record_traffic(args):
    """HBM bytes per pack launch from rocprofv3 --pmc counter files: the counter_collection.csv
    files of runs of this script on the workload (--record-traffic) and of --copy-calibration
    MIB, a plain device copy of known size (--copy-counters), recorded under profiles/ with
    the pack kernel's source hash.  Two
    measures, both per launch:
      - FETCH_SIZE and WRITE_SIZE (KiB), each scaled by copy bytes / what the same counter
        reads for the copy.  On gfx950 the read factor is 2: FETCH_SIZE counts 128-byte read
        requests through TCC_BUBBLE, which reads 0 here, so each such request is taken as a
        64-byte one (the copy's TCC_EA0_RDREQ_128B equals its bytes / 128);
      - the L2's requests to memory in 32-byte units, TCC_EA0_RDREQ_DRAM_32B and
        TCC_EA0_WRREQ_WRITE_DRAM_32B, times 32, with no calibration (they read the copy's
        bytes exactly).
    Both count what leaves the L2 for memory, last-level (Infinity Cache) hits included."""
    from precision_attention_input_amd import workloads as W
    w = W.BY_NAME[args.workload] if args.workload else W.LONG_UNALIGNED
    copy_bytes = args.copy_calibration * 2 ** 20
    if not copy_bytes:
        raise SystemExit("--record-traffic needs --copy-calibration MIB (the copy's size)")
    if not args.copy_counters:
        raise SystemExit("--record-traffic needs --copy-counters (the copy run's files)")
    copy = _pmc_means(args.copy_counters, "copyBuffer")
    pack = _pmc_means(args.record_traffic, "::pack_kernel<")
    for t in (copy, pack):
        _need(t, "FETCH_SIZE", "WRITE_SIZE", "TCC_EA0_RDREQ_DRAM_32B_sum",
              "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")
    f_scale = copy_bytes / (1024 * copy["FETCH_SIZE"])
    w_scale = copy_bytes / (1024 * copy["WRITE_SIZE"])
    read = 1024 * pack["FETCH_SIZE"] * f_scale
    write = 1024 * pack["WRITE_SIZE"] * w_scale
    dram_read = 32 * pack["TCC_EA0_RDREQ_DRAM_32B_sum"]
    dram_write = 32 * pack["TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"]
    unpack = _pmc_means(args.record_traffic, "::unpack_kernel<")
    _need(unpack, "TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")
    unpack_req = 32 * (unpack["TCC_EA0_RDREQ_DRAM_32B_sum"] +
                       unpack["TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"])
    rec = {"kernel": "pack_kernel", "workload": w.name, "kernel_hash": kernel_hash(),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "copy_dram_request_bytes": round(32 * (copy["TCC_EA0_RDREQ_DRAM_32B_sum"] +
                                                  copy["TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"])),
           "copy_bytes": 2 * copy_bytes,
           "hbm_read_bytes_per_launch": round(read), "hbm_write_bytes_per_launch": round(write),
           "hbm_bytes_per_launch": round(read + write),
           "dram_request_read_bytes_per_launch": round(dram_read),
           "dram_request_write_bytes_per_launch": round(dram_write),
           "dram_request_bytes_per_launch": round(dram_read + dram_write),
           "algorithmic_bytes_per_launch": algorithmic_bytes(w)["pack"],
           "unpack_kernel_hash": kernel_hash(UNPACK_SOURCES),
           "unpack_dram_request_bytes_per_launch": round(unpack_req),
           "unpack_algorithmic_bytes_per_launch": algorithmic_bytes(w)["unpack"]}
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"pack_kernel_{w.name}_traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def _timed_reps(fn, min_s: float) -> tuple[float, int]:
    """Mean seconds per call of fn over repetitions totalling at least min_s (at least one)."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            return dt / n, n


def cpu_baseline(w, d, nb: dict, min_s: float):
    """The CPU oracle, unchanged, on the host's cores: the ranks' (and destinations')
    independent calls run side by side on a thread pool (ctypes releases the interpreter
    lock during each C call), so at most world_size of them run at once.
      - pack+unpack: the whole workload, every rank's pack then every destination's unpack;
      - amax: the statistics step, every rank's grouped amax (Q raw, K centered) and
        boundary min/max of Q and K;
      - single-thread figures of both on a sample: rank 0's pack + destination 0's unpack,
        rank 0's statistics (1/world_size of the work).
    Each figure repeats its work for at least min_s seconds.  GB/s use the GPU figures'
    algorithmic bytes."""
    import torch
    import oracle
    from oracle import pipeline

    P, L = w.P, w.L
    host_cores = len(os.sched_getaffinity(0))
    threads = max(1, min(16, host_cores))
    used_threads = min(threads, P)
    qs, ks, vs = (pipeline.shards(d[n], P) for n in ("Q", "K", "V"))
    mean = d["mean"]
    _, _, q_amax, k_amax = pipeline.run_stats(qs, ks, mean, world_size=P,
                                              used_sequence=w.used, threads=threads)

    def pack_rank(r):
        return oracle.pack(qs[r], ks[r], vs[r], mean, q_amax[r], k_amax[r], rank=r,
                           world_size=P)

    def unpack_dest(sends, p):
        recv = torch.stack([sends[r][p] for r in range(P)])
        return oracle.unpack_for_sage(recv, batch_size=w.B, local_sequence=L, local_heads=w.h,
                                      head_dim=w.D, world_size=P,
                                      scale_sequence=w.scale_sequence)

    def pack_unpack_all():
        sends = pipeline._map(pack_rank, range(P), threads)
        pipeline._map(lambda p: unpack_dest(sends, p), range(P), threads)

    sends0 = pipeline._map(pack_rank, range(P), threads)   # destination 0's receive buffer

    def pack_unpack_one():
        pack_rank(0)
        unpack_dest(sends0, 0)

    def stats_all():
        pipeline.run_stats(qs, ks, mean, world_size=P, used_sequence=w.used, threads=threads)

    def stats_one():
        kw = dict(rank=0, world_size=P, used_sequence=w.used)
        oracle.boundary_minmax(qs[0], **kw)
        oracle.boundary_minmax(ks[0], **kw)
        oracle.k_grouped_amax(qs[0], None, **kw)
        oracle.k_grouped_amax(ks[0], mean, **kw)

    pu_bytes = nb["pack"] + nb["unpack"]
    t_pu, n_pu = _timed_reps(pack_unpack_all, min_s)
    t_st, n_st = _timed_reps(stats_all, min_s / 2)
    t_pu1, n_pu1 = _timed_reps(pack_unpack_one, min_s / 2)
    t_st1, n_st1 = _timed_reps(stats_one, min_s / 4)
    return {
        "value": round(pu_bytes / t_pu / 1e9, 4), "unit": "GB/s", "cores": used_threads,
        "kind": "oracle",
        "sample": f"pack+unpack: the whole workload (pack of all {P} ranks, unpack of all {P} "
                  f"destinations; {n_pu} repetitions, {t_pu:.3f} s each) with the ranks on "
                  f"{used_threads} threads of the {host_cores} host cores; single-thread: "
                  f"rank 0's pack + destination 0's unpack ({n_pu1} repetitions); amax: the "
                  f"statistics of every rank, Q and K ({n_st} repetitions on {used_threads} "
                  f"threads; single-thread: rank 0, {n_st1} repetitions)",
        "single_thread_gbps": round(pu_bytes / P / t_pu1 / 1e9, 4),
        "amax_gbps": round(nb["stats"] / t_st / 1e9, 4),
        "amax_single_thread_gbps": round(nb["stats"] / P / t_st1 / 1e9, 4),
        "host_cores": host_cores,
    }


MFMA_PEAK_TFLOPS = 5000.0       # MI355X dense int8 / fp8 matrix peak


def consumer_bench(args, w, d, dev):
    """K back-to-back launches of the consumer check over every destination's unpacked
    tensors (one launch per destination), HIP events at the two ends."""
    import torch

    import precision_attention_input_amd as ulp
    from precision_attention_input_amd import workloads as W

    P, L, B, H, D = w.P, w.L, w.B, w.H, w.D
    used = w.used or w.S
    st = {n: W.stacked_shards(d[n], P).to(dev) for n in ("Q", "K", "V")}
    mean = d["mean"].to(dev)
    qa, ka, qm, km = ulp.group_stats(st["Q"], st["K"], mean, world_size=P, used_sequence=w.used)
    ulp.group_derive(qa, ka, qm, km, mean, local_sequence=L, world_size=P)
    grp = ulp.group_pack(st["Q"], st["K"], st["V"], mean, qa, ka, world_size=P)
    outs = ulp.group_unpack(grp, batch_size=B, local_sequence=L, local_heads=w.h, head_dim=D,
                            world_size=P, aligned=w.aligned, scale_sequence=w.scale_sequence)
    res = [torch.empty(B, used, w.h, D, dtype=torch.float32, device=dev) for _ in range(P)]

    def run():
        for p in range(P):
            ulp.consumer_attention(*(t[p] for t in outs), used=used, out=res[p])

    for _ in range(args.warmup):
        run()
    # Small launches finish before the GPU's clocks have risen: keep warming up until about
    # --warm-ms of launches have run.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if args.warm_ms > 0:
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        for _ in range(min(2000, int(args.warm_ms / max(e0.elapsed_time(e1), 1e-3)))):
            run()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (args.steps * P)          # one destination's launch
    flops = 4.0 * B * w.h * used * used * D                # Q.K and P.V, per destination
    tflops = flops / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "consumer check attention TFLOP/s (INT8 Q.K + FP8 P.V on MFMA)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_launch": round(ms, 5), "higher_is_better": True,
        "dtype": "i8/fp8", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "local_heads": w.h, "used_sequence": used,
                   "head_dim": D, "launches_per_step": P},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
                     "flops_per_launch": flops},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="workload name (default: long_unaligned, the largest configuration, "
                         "B=1, world_size 8, L=9360, H=40, D=128, bf16, used 74000)")
    ap.add_argument("--sets", type=int, default=0, help="rotating buffer sets (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="seconds of repetitions behind the CPU oracle's pack+unpack figure "
                         "(the amax and single-thread figures take half and a quarter of it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm-ms", type=float, default=300.0,
                    help="with --consumer: extra warm-up launches until about this many ms "
                         "of them have run (0: only --warmup)")
    ap.add_argument("--consumer", action="store_true",
                    help="time the MFMA consumer check (INT8 Q.K, FP8 P.V attention over every "
                         "destination's unpacked tensors) instead of the path; prints its own "
                         "JSON line (TFLOP/s against the 5.0 PFLOP/s int8/fp8 dense peak)")
    ap.add_argument("--graph", action="store_true",
                    help="capture every timed loop into a HIP graph once and time its replays "
                         "(removes the host's per-launch cost; matters for launch-bound "
                         "workloads such as the tiny one)")
    ap.add_argument("--v-scale", action="store_true",
                    help="pass a caller-held [B,H,D] V scale to the pack (V divided before "
                         "E4M3); the default converts V unscaled")
    ap.add_argument("--record-traffic", nargs="+", metavar="CSV",
                    help="rocprofv3 --pmc counter_collection files of runs of this script on the "
                         "workload, holding FETCH_SIZE, WRITE_SIZE, "
                         "TCC_EA0_RDREQ_DRAM_32B_sum and TCC_EA0_WRREQ_WRITE_DRAM_32B_sum: write "
                         "the pack kernel's HBM bytes per launch under profiles/ and exit")
    ap.add_argument("--copy-counters", nargs="+", metavar="CSV",
                    help="with --record-traffic: the counter_collection files of the "
                         "--copy-calibration run")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB per step (the reference "
                         "kernel for scaling HBM byte counters), then exit")
    args = ap.parse_args()

    if args.record_traffic:
        record_traffic(args)
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (the whole Ulysses group is held "
              f"by one device; world_size only shapes the byte layout); --gpus {args.gpus} "
              f"is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import precision_attention_input_amd as ulp
    from precision_attention_input_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration * 2 ** 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n,
                          "dispatches": args.warmup + args.steps}), flush=True)
        return

    w = W.BY_NAME[args.workload] if args.workload else W.LONG_UNALIGNED
    d = W.generate(w)
    if args.consumer:
        consumer_bench(args, w, d, dev)
        return
    nb = algorithmic_bytes(w, args.v_scale)
    vsc = W.v_scale(w).to(dev) if args.v_scale else None
    set_bytes = 12 * nb["N"]      # stacked Q/K/V (6N) + all-to-all buffer (3N) + outputs (3N)
    nsets = args.sets or max(2, min(8, -(-1024 * 2 ** 20 // set_bytes)))
    P, L, B, H, D = w.P, w.L, w.B, w.H, w.D

    sets = []
    for i in range(nsets):
        s = {n: W.stacked_shards(d[n], P).to(dev) for n in ("Q", "K", "V")}
        s["mean"] = d["mean"].to(dev)
        f = dict(dtype=torch.float32, device=dev)
        sl = ulp.slots(L)
        s["stats"] = (torch.empty(P, B, H, sl, **f), torch.empty(P, B, H, sl, **f),
                      torch.empty(P, B, H, 2, 2, D, **f), torch.empty(P, B, H, 2, 2, D, **f))
        s["group"] = ulp.group_buffer(B, L, H, D, P, dev)
        s["out"] = ulp._alloc_unpack(dev, ulp.unpack_shapes(B, L, w.h, D, P, w.scale_sequence),
                                     lead=(P,))
        sets.append(s)

    def stats(s):
        return ulp.group_stats(s["Q"], s["K"], s["mean"], world_size=P, used_sequence=w.used,
                               out=s["stats"])

    def derive(s):
        qa, ka, qm, km = s["stats"]
        ulp.group_derive(qa, ka, qm, km, s["mean"], local_sequence=L, world_size=P)

    def pack(s):
        ulp.group_pack(s["Q"], s["K"], s["V"], s["mean"], s["stats"][0], s["stats"][1],
                       world_size=P, v_scale=vsc, group=s["group"])

    def unpack(s):
        ulp.group_unpack(s["group"], batch_size=B, local_sequence=L, local_heads=w.h,
                         head_dim=D, world_size=P, aligned=w.aligned,
                         scale_sequence=w.scale_sequence, out=s["out"])

    def step(s):
        stats(s)
        derive(s)
        pack(s)
        unpack(s)

    def pack_unpack(s):
        pack(s)
        unpack(s)

    def timed(fn, n, reps=1, warm=3):
        """Average ms per call over n back-to-back calls on rotating buffer sets, with HIP
        events (on the current stream, where every launch goes) only at the two ends of the
        region: an event recorded between two launches costs about 2 us of GPU time.  `warm`
        untimed calls of the same loop come first; with reps > 1 the loop of n calls is
        timed reps times and the median loop is returned (one late dispatch or clock dip in
        a loop of small kernels otherwise moves a single loop's average by a percent)."""
        for i in range(warm):
            fn(sets[i % nsets])

        def loop():
            for i in range(n):
                fn(sets[i % nsets])

        run = loop
        if args.graph:
            # the n calls captured once into a HIP graph and replayed: no host launch cost
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                loop()
            graph.replay()                      # one untimed replay
            run = graph.replay
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        loops, walls = [], []
        for _ in range(reps):
            torch.cuda.synchronize()
            w0 = time.perf_counter()
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            walls.append((time.perf_counter() - w0) * 1e3 / n)
            loops.append(e0.elapsed_time(e1) / n)
        timed.wall_ms = statistics.median(walls)
        return statistics.median(loops)

    # The one-read step: statistics and the pack of every slot that derive cannot change
    # from one read of Q, K and V, then derive together with the pack of the slots that
    # waited for it, then the unpack (the same outputs as the separate step above).
    def stats_pack(s):
        ulp.group_stats_pack(s["Q"], s["K"], s["V"], s["mean"], world_size=P,
                             used_sequence=w.used, v_scale=vsc, out=s["stats"],
                             group=s["group"])

    def derive_pack(s):
        qa, ka, qm, km = s["stats"]
        ulp.group_derive_pack(s["Q"], s["K"], s["mean"], qa, ka, qm, km, world_size=P,
                              group=s["group"], used_sequence=w.used)

    def one_read_step(s):
        stats_pack(s)
        derive_pack(s)
        unpack(s)

    # Warm-up: W steps of each form (at least one per buffer set, so that every set holds
    # valid statistics for the per-kernel loops below).
    for i in range(max(args.warmup, nsets)):
        step(sets[i % nsets])
    for i in range(max(args.warmup, nsets)):
        one_read_step(sets[i % nsets])
    torch.cuda.synchronize()

    # The timed steps: the whole path, exactly K steps of the one-read form (ms_per_step,
    # host clock around them, synchronized on both sides), then K of the separate form.
    K = args.steps
    or_step_ms = timed(one_read_step, K, warm=0)
    ms_per_step = timed.wall_ms
    step_ms = timed(step, K, warm=0)
    sep_step_wall_ms = timed.wall_ms

    # Each kernel on its own, and pack+unpack as a pair: loops of K launches on the same
    # sets, the median of REPS loops.
    stats_ms = timed(stats, K, REPS)
    derive_ms = timed(derive, K, REPS)
    pack_ms = timed(pack, K, REPS)
    unpack_ms = timed(unpack, K, REPS)
    pu_ms = timed(pack_unpack, K, REPS)

    # The global K mean, an input of the step (formed once per K tensor), timed on its own.
    ws = torch.empty(int(ulp.lib().ulp_k_mean_workspace_bytes(B, L, H, D, P, ulp._none(w.used))),
                     dtype=torch.uint8, device=dev)
    km_out = (torch.empty(B, H, D, dtype=torch.float32, device=dev),
              torch.empty(B, H, D, dtype=w.dtype, device=dev))

    def k_mean(s):
        ulp.k_mean(s["K"], world_size=P, used_sequence=w.used, workspace=ws, out=km_out)

    for i in range(args.warmup):
        k_mean(sets[i % nsets])
    k_mean_ms = timed(k_mean, K)

    # Statistics together with the K mean: the mean then the statistics (two reads of K),
    # and the one-read entry point that forms both from one pass over K.
    ws2 = torch.empty(int(ulp.lib().ulp_group_stats_with_mean_workspace_bytes(B, L, H, D, P)),
                      dtype=torch.uint8, device=dev)
    sm_out = tuple(t.clone() for t in sets[0]["stats"]) + km_out

    def stats_mean_separate(s):
        k_mean(s)
        ulp.group_stats(s["Q"], s["K"], km_out[1], world_size=P, used_sequence=w.used,
                        out=s["stats"])

    def stats_mean_one_read(s):
        ulp.group_stats_with_mean(s["Q"], s["K"], world_size=P, used_sequence=w.used,
                                  workspace=ws2, out=sm_out)

    for i in range(args.warmup):
        stats_mean_separate(sets[i % nsets])
        stats_mean_one_read(sets[i % nsets])
    sm_sep_ms = timed(stats_mean_separate, K)
    sm_one_ms = timed(stats_mean_one_read, K)

    # The one-read step's two pack launches, each alone.
    sp_ms = timed(stats_pack, K, REPS)
    pd_ms = timed(derive_pack, K, REPS)

    pu_bytes = nb["pack"] + nb["unpack"]
    value = pu_bytes / (pu_ms * 1e-3) / 1e9
    pack_gbps = nb["pack"] / (pack_ms * 1e-3) / 1e9
    traffic, traffic_req, unpack_req = (None, None, None) if args.v_scale else \
        load_traffic(w.name)
    # the pair's HBM bytes as the counters read them (pack + unpack, DRAM requests), when
    # both are recorded for the current sources
    pair_req = traffic_req + unpack_req if traffic_req and unpack_req else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, d, nb, args.cpu_seconds)

    line = {
        "metric": "pack+unpack GB/s and % of HBM peak per config; amax-kernel GB/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "fp16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "world_size": P, "local_sequence": L,
                   "heads": H, "head_dim": D, "used_sequence": w.used,
                   "scale_sequence": w.scale_sequence, "aligned": w.aligned,
                   "v_scale": bool(args.v_scale), "buffer_sets": nsets,
                   "hip_graph": bool(args.graph)},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "pct_hbm_peak_counters": (None if pair_req is None else
                                  round(100 * pair_req / (pu_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2)),
        "pack_unpack_bytes": pu_bytes,
        "pack_unpack_ms": round(pu_ms, 5),
        "pack_ms": round(pack_ms, 5),
        "unpack_ms": round(unpack_ms, 5),
        "stats_ms": round(stats_ms, 5),
        "derive_ms": round(derive_ms, 5),
        "amax_gbps": round(nb["stats"] / (stats_ms * 1e-3) / 1e9, 2),
        "k_mean_ms": round(k_mean_ms, 5),
        "k_mean_gbps": round(nb["k_mean"] / (k_mean_ms * 1e-3) / 1e9, 2),
        "stats_with_mean_ms": {"k_mean_then_stats": round(sm_sep_ms, 5),
                               "one_read_of_k": round(sm_one_ms, 5)},
        "one_read_step_ms": {"step": round(or_step_ms, 5),
                             "stats_pack": round(sp_ms, 5),
                             "derive_pack": round(pd_ms, 5),
                             "stats_pack_gbps": round(nb["pack"] / (sp_ms * 1e-3) / 1e9, 2)},
        "one_read_step_gbps": round((pu_bytes + nb["stats"] - 2 * 2 * nb["N"]) /
                                    (or_step_ms * 1e-3) / 1e9, 2),
        "separate_step_ms": {"events": round(step_ms, 5), "wall": round(sep_step_wall_ms, 5)},
        "step_gbps": round((pu_bytes + nb["stats"]) / (step_ms * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "kernel": "pack_kernel", "achieved": round(pack_gbps, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(pack_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "traffic_dram_requests": traffic_req,
                     "algorithmic_bytes_per_launch": nb["pack"]},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
