"""Benchmark of the gradient-bucket reduction path on one MI355X.

Default workload (the headline metric): ZeRO-2 gradient sync of K = 8
simulated ranks, 2,376,274,560 bf16 gradient elements per rank (~N(0, 1e-3),
seeded), in five 500M-element buckets through the scheduler; each bucket is
one fused ring-order reduce-scatter + /8 + fp32 cast into the ranks'
partitioned flat gradients. One step = the whole sync (all five buckets).

Byte model (the method's minimum traffic, each input read once, each output
written once): per element index K*2 bytes read + 4 bytes written = 20 B,
so 47.53 GB per step. `value` = those bytes / step time.

Other workloads (--workload):
  zero2_accum     the same sync as a later micro-step (adds into the partitions)
  zero2_overlap   the same sync under a synthetic backward pass: each bucket's
                  compute then its reduction, scheduler against one buffer
  zero3_ag        the 32-layer transformer all-gather in 162 prefetch buckets
  zero3_prefetch  the prefetch coordinator walking that model's trace, with a
                  synthetic compute per step; reports the pass time in ms
  allreduce64     K = 64, N = 1,000,000,007 fused in-place all-reduce
  flatten8        the 64-fragment bucket: flatten + reduce-scatter against the
                  discrete path, in microseconds per call (cache-resident)
  frags_layer     the discrete reduce-scatter over one layer's seven gradients
  flatten_layer   the bucket flatten of those seven gradients (bandwidth scale)
  frags_k64       256 fragments on K = 64: calls and plans with and without a
                  workspace-staged table (microseconds and launches per call)

Prints one JSON line. Only one GPU is used; --gpus above 1 exits.
"""
import argparse
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "gradient_sync_zr_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(name, src_hash, algorithmic, key="hbm_bytes_per_launch"):
    """HBM bytes per launch (or per step) from a committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a plain copy of known size),
    or None when it is missing, was taken on a different kernel source, or
    measured a workload whose algorithmic bytes differ from `algorithmic`."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != src_hash:
        return None
    algo_key = key.replace("hbm_bytes", "algorithmic_bytes")
    try:
        if abs(float(kv[algo_key]) - algorithmic) > 1e-3 * algorithmic:
            return None
        return int(float(kv[key]))
    except (KeyError, ValueError):
        return None


def host_cores():
    """Cores this process may run on (its affinity mask), all of them. The
    machine's hardware thread count (os.cpu_count()) is reported beside it:
    the two differ when the process is confined to part of the host."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, n)


def events_ms(pairs):
    return [a.elapsed_time(b) for a, b in pairs]


def copy_ceiling_gbps(gib=4, reps=10):
    """A plain streaming copy's read + write rate on this GPU, measured now:
    the practical ceiling of a bandwidth-bound kernel (the test kit's
    tk_copy, one block per 4 KiB). None when the test kit is not built."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "tests", "kit", "libtestkit.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.tk_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                            ctypes.c_void_p]
    nbytes = gib << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    s = torch.cuda.current_stream().cuda_stream
    ms = []
    for i in range(reps + 2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if lib.tk_copy(src.data_ptr(), dst.data_ptr(), nbytes, nbytes // 4096, s) != 0:
            return None
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            ms.append(e0.elapsed_time(e1))
    del src, dst
    return round(2 * nbytes / (sum(ms) / len(ms) * 1e-3) / 1e9, 1)


def mix_ceiling(reps=10, modes=("mix", "reads", "writes"), slices=4):
    """The test kit's matched-mix stream (tests/kit/mix_probe.py: the
    reduce-scatter's loads and stores at one bucket's shape, no arithmetic,
    in tiles of `slices` slices per wave), measured now: the rates of the
    requested modes ("mix", "reads", "writes", "accum"), or None when the kit
    is not built."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("mix_probe", os.path.join(ROOT, "tests", "kit",
                                                                            "mix_probe.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.measure(reps=reps, modes=modes, slices=slices)


# ----------------------------------------------------------------- zero2
def bench_zero2(args, accumulate=False):
    import numpy as np
    import torch

    import synth
    from gradient_sync_zr_amd.steps import Zero2GradSync
    from synth import workloads as W

    cfg = W.ZERO2
    K, N, bucket, sigma = cfg["K"], cfg["N_total"], cfg["bucket"], cfg["sigma"]
    seed = W.seed_of(3)
    grads = [torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    for r in range(K):
        synth.dev_normal_bf16(grads[r], seed, r, 0, sigma)
    buckets = W.zero2_buckets(N, bucket)
    P = sum(-(-n // K) for _, n in buckets)
    parts = [torch.empty(P, dtype=torch.float32, device="cuda") for _ in range(K)]
    # the headline: the reductions on the caller's own stream, the library's
    # default for a sync with no compute to overlap (the scheduler then
    # enqueues no cross-stream waits)
    sync = Zero2GradSync(grads, parts, bucket, chunk_shift=cfg["shift"], average=True)
    torch.cuda.synchronize()
    print(f"# zero2: K={K} N={N} buckets={len(buckets)} inputs resident", file=sys.stderr, flush=True)
    # an accumulation micro-step also reads the fp32 partition back
    per_elem = 2 * K + (8 if accumulate else 4)
    micro = 1 if accumulate else 0
    step_bytes = sum(n * per_elem for _, n in buckets)
    prod = torch.cuda.current_stream()

    def timed_steps(s, first):
        """W untimed steps, then K timed ones with nothing but the sync in
        them; one event per step boundary on the caller's stream (each step
        ends with that stream ordered after the step's reductions) gives
        every step's device time for the median and minimum. The first
        sync's first step writes the partitions (micro-step 0), so that an
        accumulating run adds to defined values; every later launch is of
        the timed kind."""
        if first:
            s.step()
        for _ in range(args.warmup):
            s.step(micro_step=micro)
        torch.cuda.synchronize()
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        t0 = time.perf_counter()
        marks[0].record(prod)
        for i in range(args.steps):
            s.step(micro_step=micro)
            marks[i + 1].record(prod)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) * 1e3 / args.steps, sorted(marks[i].elapsed_time(marks[i + 1])
                                                     for i in range(args.steps))

    ms_step, step_ms = timed_steps(sync, True)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    # the same steps with the reductions on a stream of their own, as a
    # training step that overlaps them with the backward pass runs them: each
    # bucket waits on the caller's stream and each step ends with the caller
    # waiting on the reduction stream
    red = torch.cuda.Stream()
    sync2 = Zero2GradSync(grads, parts, bucket, chunk_shift=cfg["shift"], average=True,
                          reduction_stream=red)
    ms_step2, step_ms2 = timed_steps(sync2, False)
    sync2.close()
    reduction_stream = {"ms_per_step": round(ms_step2, 4),
                        "step_ms_median": round(step_ms2[len(step_ms2) // 2], 4),
                        "step_ms_min": round(step_ms2[0], 4),
                        "GBps": round(step_bytes / (ms_step2 * 1e-3) / 1e9, 1)}
    # a separate instrumented pass of as many steps: an event pair around each
    # launch, after its stream has been ordered after the producer, so each
    # pair brackets the kernel alone
    timing = []
    for _ in range(args.steps):
        sync.step(timing=timing, micro_step=micro)
    torch.cuda.synchronize()
    launch_ms = events_ms(timing)
    launch_bytes = [n * per_elem for _, n in buckets] * args.steps
    achieved = sum(launch_bytes) / (sum(launch_ms) * 1e-3) / 1e9
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    # the 500M-element buckets alone (the last bucket is smaller)
    full = sorted(ms for ms, b in zip(launch_ms, launch_bytes) if b == max(launch_bytes))
    full_med, full_min = full[len(full) // 2], full[0]
    bytes_per_launch = sum(launch_bytes) / len(launch_bytes)
    # each bucket's rate over the instrumented steps (its launches are every nb-th)
    nb = len(buckets)
    per_bucket = [round(launch_bytes[b] * (len(launch_ms) // nb) / (sum(launch_ms[b::nb]) * 1e-3) / 1e9, 1)
                  for b in range(nb)]
    src = kernel_source_hash(["zr_rs.hip", "zr_fold.hpp", "zr_device.hpp"])
    traffic = read_traffic("rs_ring_bf16_f32_k8_zero2" + ("_accum" if accumulate else "") +
                           ".counters.txt", src, bytes_per_launch)
    print(f"# zero2: {ms_step:.3f} ms/step (median {step_ms[len(step_ms) // 2]:.3f}, min "
          f"{step_ms[0]:.3f}), kernel avg {avg_launch_ms:.3f} ms", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline and not accumulate:
        cpu = cpu_baseline_zero2(grads, parts, buckets[0], K, args)
        if cpu and cpu.get("value"):
            cpu["gpu_over_oracle"] = round(value / cpu["value"], 1)
    sync.close()
    del sync, grads, parts
    copy = copy_ceiling_gbps()
    # the kernel's own tile shape: one slice per wave for the plain sync,
    # four when the partitions are read back
    mix_slices = 4 if accumulate else 1
    mix = mix_ceiling(modes=("accum",) if accumulate else ("mix", "reads", "writes"), slices=mix_slices)
    mix_key = "accum" if accumulate else "mix"
    if accumulate:
        metric = ("reduce-scatter+avg+accumulate GB/s (gradient-accumulation micro-step), K=8, "
                  "2.38B-elem bf16 grads")
    else:
        metric = "reduce-scatter+avg+cast GB/s and % of HBM peak, K=8, 2.38B-elem bf16 grads"
    return {
        "metric": metric,
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic: seeded counter-based generator on the device, bf16 ~N(0,1e-3)",
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "step_ms_median": round(step_ms[len(step_ms) // 2], 4),
        "step_ms_min": round(step_ms[0], 4),
        "value_at_median_step_GBps": round(step_bytes / (step_ms[len(step_ms) // 2] * 1e-3) / 1e9, 1),
        "reduction_stream": reduction_stream,
        "reads_only_GBps": round(K * N * 2 / (ms_step * 1e-3) / 1e9, 1),
        "config": {"workload": "zero2_grad_sync: K=8 simulated ranks in one HBM, "
                               "2,376,274,560 bf16 grad elements per rank, 5 buckets of "
                               "500M elements via the ping-pong scheduler, ring-order "
                               "reduce-scatter + /8 + fp32 cast into the partitioned flat grad",
                   "K": K, "N_per_rank": N, "bucket_elems": bucket, "n_buckets": len(buckets),
                   "chunk_shift": 1, "io": "bf16 in, f32 out" + (", f32 partition read back and "
                                                                   "added" if accumulate else ""),
                   "bytes_per_step": step_bytes,
                   "parallelism": "1 GPU (K ranks simulated)"},
        "roofline": {"bound": "hbm", "kernel": "rs_kernel<bf16,f32,K=8,avg,ring>",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "avg_launch_ms": round(avg_launch_ms, 4),
                     "full_bucket_launch_ms_median": round(full_med, 4),
                     "full_bucket_launch_ms_min": round(full_min, 4),
                     "per_bucket_GBps": per_bucket,
                     "copy_ceiling_GBps": copy,
                     "of_copy_ceiling": round(achieved / copy, 4) if copy else None,
                     "mix_ceiling_GBps": mix[mix_key]["GBps"] if mix else None,
                     "mix_tile_slices": mix_slices,
                     "of_mix_ceiling": round(achieved / mix[mix_key]["GBps"], 4) if mix else None,
                     "mix_reads_only_GBps": mix["reads"]["GBps"] if mix and "reads" in mix else None,
                     "mix_writes_only_GBps": mix["writes"]["GBps"] if mix and "writes" in mix else None,
                     "timing": "per-launch event pairs from a separate instrumented pass of "
                               "the same number of steps; value and the step median/min come "
                               "from the uninstrumented steps",
                     "algorithmic_bytes_per_launch": int(bytes_per_launch),
                     "kernel_source_sha256_16": src},
        "cpu_baseline": cpu,
    }


def cpu_baseline_zero2(grads, parts, first_bucket, K, args):
    """The oracle on bucket 0 of the same resident inputs (copied to the host,
    not timed), split by chunk offset over every host core this process may
    use; then the same bucket on one core. Also checks the GPU partitions of
    that bucket bit for bit."""
    import numpy as np
    import torch

    import oracle
    start, n = first_bucket
    C = -(-n // K)
    M = min(C, args.cpu_sample_elems // K) if args.cpu_sample_elems else C
    # the sample: offsets [0, M) of every chunk of bucket 0, as its own
    # reduce-scatter problem with chunk size M (M = C: the whole bucket)
    xs = []
    for r in range(K):
        rows = [grads[r][start + j * C:start + j * C + M].view(torch.int16).cpu().numpy()
                for j in range(K)]
        xs.append(np.concatenate(rows).view(np.uint16))
    outs = [np.empty(M, dtype=np.float32) for _ in range(K)]
    T = host_cores()

    def work(i):
        lo, hi = i * M // T, (i + 1) * M // T
        oracle.reduce_scatter(xs, K * M, np.float32, shift=1, average=True, o_range=(lo, hi),
                              out=outs)

    th = [threading.Thread(target=work, args=(i,)) for i in range(T)]
    t0 = time.perf_counter()
    for t in th:
        t.start()
    for t in th:
        t.join()
    dt = time.perf_counter() - t0
    model_bytes = K * M * (2 * K + 4)
    gbs = model_bytes / dt / 1e9
    exact = all(np.array_equal(parts[q][:M].cpu().numpy().view(np.uint32), outs[q].view(np.uint32))
                for q in range(K))
    # one core on the same sample, whole
    t1 = time.perf_counter()
    oracle.reduce_scatter(xs, K * M, np.float32, shift=1, average=True, o_range=(0, M), out=outs)
    dt1 = time.perf_counter() - t1
    sample = ("all of bucket 0" if M == C else f"offsets [0,{M}) of each of the {K} chunks of bucket 0")
    return {"value": round(gbs, 2), "unit": "GB/s", "cores": T, "kind": "oracle",
            "host_cores": T, "threads_used": T, "hardware_threads": os.cpu_count(),
            "seconds": round(dt, 3),
            "single_core_GBps": round(model_bytes / dt1 / 1e9, 2),
            "single_core_seconds": round(dt1, 3),
            "single_core_sample": sample,
            "sample": f"{sample} ({K * M} element indices, {model_bytes / 1e9:.2f} GB under the same "
                      f"byte model); GPU partitions bit-exact on it: {exact}"}


# ----------------------------------------------------------------- zero3
def bench_zero3(args):
    import torch

    import synth
    from gradient_sync_zr_amd.steps import Zero3Gather
    from synth import workloads as W

    cfg = W.ZERO3
    K, sigma, shift = cfg["K"], cfg["sigma"], cfg["shift"]
    seed = W.seed_of(4)
    numels = [p.numel for p in W.llama_like_params()]
    shard_numel = sum(-(-n // K) for n in numels)
    full_numel = sum(numels)
    shards = [torch.zeros(shard_numel, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    fulls = [torch.empty(full_numel, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    soff = 0
    for p, n in enumerate(numels):
        C = -(-n // K)
        for r in range(K):
            j = (r + shift) % K
            cnt = max(0, min(C, n - j * C))
            if cnt:
                synth.dev_normal_bf16(shards[r][soff:soff + cnt], seed, p, j * C, sigma)
        soff += C
    gather = Zero3Gather(shards, fulls, numels, cfg["prefetch_bytes"] // cfg["elem_bytes"],
                         chunk_shift=shift)
    for _ in range(args.warmup):
        gather.step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        gather.step()
    e1.record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    step_bytes = full_numel * 2 + K * full_numel * 2   # shards read once + K full copies
    value = step_bytes / (ms_step * 1e-3) / 1e9
    kernel_ms = e0.elapsed_time(e1) / args.steps
    src = kernel_source_hash(["zr_ag.hip", "zr_device.hpp"])
    traffic = read_traffic("ag_bf16_k8_zero3.counters.txt", src, step_bytes, key="hbm_bytes_per_step")
    copy = copy_ceiling_gbps()
    return {
        "metric": "all-gather GB/s (shard read + K full writes), K=8, 6.74B-param transformer",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded generator, bf16 ~N(0,0.02)",
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "config": {"workload": "zero3_allgather: 226 params (32 layers, hidden 4096, FFN 11008, "
                               "vocab 32000), 1/8 shards, 162 greedy 50 MB prefetch buckets",
                   "K": K, "params": len(numels), "n_buckets": len(gather.buckets),
                   "bytes_per_step": step_bytes},
        "roofline": {"bound": "hbm", "kernel": "ag_kernel<bf16,K=8> (162 launches per step)",
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "achieved": round(step_bytes / (kernel_ms * 1e-3) / 1e9, 1),
                     "copy_ceiling_GBps": copy,
                     "of_copy_ceiling": round(step_bytes / (kernel_ms * 1e-3) / 1e9 / copy, 4) if copy else None,
                     "frac": round(step_bytes / (kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "traffic_unit": "bytes per step",
                     "kernel_source_sha256_16": src},
        "cpu_baseline": None,
    }


# --------------------------------------------------------- zero3_prefetch
def kit_delay():
    """delay(us, stream): the test kit's bounded wall-clock spin kernel, a
    stand-in for a module's compute, calibrated against events on the device."""
    import ctypes

    import torch
    L = ctypes.CDLL(os.path.join(ROOT, "tests", "kit", "libtestkit.so"))
    L.tk_delay.argtypes = [ctypes.c_longlong, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_void_p]
    L.tk_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int)]
    khz = ctypes.c_int(0)
    if L.tk_clock_khz(ctypes.byref(khz)) != 0 or khz.value <= 0:
        raise RuntimeError("wall clock rate unavailable")
    s = torch.cuda.current_stream()
    nominal = 2 * khz.value  # 2 ms at the reported rate
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ms = []
    for _ in range(3):
        e0.record(s)
        L.tk_delay(nominal, 50_000_000, None, s.cuda_stream)
        e1.record(s)
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    ticks_per_us = nominal / (sorted(ms)[1] * 1e3)

    def delay(us, stream):
        if L.tk_delay(int(us * ticks_per_us), 50_000_000, None, stream.cuda_stream) != 0:
            raise RuntimeError("delay launch failed")
    return delay


def bench_zero2_overlap(args):
    """The scheduler against the dependency the issue page reports: each
    bucket's backward compute (a calibrated spin of `compute_ratio` times that
    bucket's reduction time, on the producer stream) followed by its
    reduction. Two buffers let the compute of bucket i+1 run under the
    reduction of bucket i; one buffer makes every bucket's compute wait for
    the previous reduction, which is the serialisation the issue describes."""
    import torch

    import synth
    from gradient_sync_zr_amd.steps import Zero2GradSync
    from synth import workloads as W

    cfg = W.ZERO2
    K, N, bucket, sigma = cfg["K"], cfg["N_total"], cfg["bucket"], cfg["sigma"]
    seed = W.seed_of(3)
    grads = [torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    for r in range(K):
        synth.dev_normal_bf16(grads[r], seed, r, 0, sigma)
    buckets = W.zero2_buckets(N, bucket)
    P = sum(-(-n // K) for _, n in buckets)
    parts = [torch.empty(P, dtype=torch.float32, device="cuda") for _ in range(K)]
    red, prod = torch.cuda.Stream(), torch.cuda.Stream()
    syncs = {nb: Zero2GradSync(grads, parts, bucket, chunk_shift=cfg["shift"], average=True,
                               n_buffers=nb, reduction_stream=red) for nb in (1, 2)}
    delay = kit_delay()
    torch.cuda.synchronize()
    # each bucket's reduction time, alone
    syncs[2].step(producer_stream=prod)
    timing = []
    syncs[2].step(producer_stream=prod, timing=timing)
    torch.cuda.synchronize()
    red_ms = events_ms(timing)
    compute_us = [args.compute_ratio * ms * 1e3 for ms in red_ms]
    passes = max(1, min(args.steps, 10))

    def wall(fn):
        fn()  # warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(passes):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / passes

    def produce(i, stream):
        delay(compute_us[i], stream)

    def compute_only():
        for i in range(len(buckets)):
            delay(compute_us[i], prod)

    # the phases are 10 ms apart (idle, untimed), so a kernel trace shows them apart
    ms_compute = wall(compute_only)
    time.sleep(0.01)
    ms_reduce = wall(lambda: syncs[2].step(producer_stream=prod))
    time.sleep(0.01)
    ms_overlap = wall(lambda: syncs[2].step(producer_stream=prod, produce=produce))
    time.sleep(0.01)
    ms_serial = wall(lambda: syncs[1].step(producer_stream=prod, produce=produce))
    for s_ in syncs.values():
        s_.close()
    exposed = max(0.0, ms_overlap - ms_compute)
    return {
        "metric": "ZeRO-2 backward with bucket reductions overlapped by the scheduler: ms per "
                  "sync, K=8, 2.38B-elem bf16 grads",
        "value": round(ms_overlap, 3), "unit": "ms", "n_gpus": 1, "steps": passes, "warmup": 1,
        "ms_per_step": round(ms_overlap, 3), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic: seeded generator, bf16 ~N(0,1e-3); compute is a calibrated spin",
        "serial_one_buffer_ms": round(ms_serial, 3), "compute_only_ms": round(ms_compute, 3),
        "reductions_only_ms": round(ms_reduce, 3), "exposed_reduction_ms": round(exposed, 3),
        "hidden_fraction": round(1.0 - exposed / ms_reduce, 4),
        "bucket_reduction_ms": [round(x, 4) for x in red_ms],
        "config": {"workload": "zero2_overlap: K=8, 2,376,274,560 bf16 grad elements per rank, "
                               "5 buckets; per bucket a spin on the producer stream, then the "
                               "reduction through the scheduler (2 buffers, or 1 for the serial "
                               "line)",
                   "K": K, "n_buckets": len(buckets), "compute_ratio": args.compute_ratio},
        "roofline": None, "cpu_baseline": None,
    }


def bench_zero3_prefetch(args):
    """The ZeRO-3 fetch/prefetch coordinator on workload 4's full trace
    (forward then backward, one parameter per module visit) with a synthetic
    compute stream: each step's compute is a spin of `compute_ratio` times
    that step's all-gather time at the measured gather rate."""
    import torch

    import synth
    import gradient_sync_zr_amd as zr
    from synth import workloads as W

    cfg = W.ZERO3
    K, sigma, shift = cfg["K"], cfg["sigma"], cfg["shift"]
    seed = W.seed_of(4)
    numels = [p.numel for p in W.llama_like_params()]
    steps = W.zero3_trace(len(numels))
    offs, soff = [], 0
    for n in numels:
        offs.append(soff)
        soff += -(-n // K)
    shards = [torch.zeros(soff, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    for p, n in enumerate(numels):
        C = -(-n // K)
        for r in range(K):
            j = (r + shift) % K
            cnt = max(0, min(C, n - j * C))
            if cnt:
                synth.dev_normal_bf16(shards[r][offs[p]:offs[p] + cnt], seed, p, j * C, sigma)
    bucket = cfg["prefetch_bytes"] // cfg["elem_bytes"]
    caps = dict(prefetch_bucket_numel=bucket, max_live_numel=cfg["max_live"],
                max_reuse_numel=cfg["max_reuse"], max_ongoing_fetches=cfg["max_ongoing"])
    arena = args.arena_numel
    plan = zr.zr_pf_plan(numels, steps, bucket, cfg["max_live"], arena,
                         max_ongoing_fetches=cfg["max_ongoing"], max_reuse_numel=cfg["max_reuse"])
    arenas = [torch.empty(arena, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    gs, cs = torch.cuda.Stream(), torch.cuda.Stream()
    delay = kit_delay()
    # the gather rate, from one gathers-only pass (kernel time on the gather stream)
    visit_numel = sum(numels[p] for st in steps for p in st)

    def walk(serial=False, compute_us=None, gathers=True, passes=1):
        pf = zr.Prefetcher(numels, offs, shards, arenas, arena, steps, chunk_shift=shift,
                           gather_stream=cs if serial else gs, compute_stream=cs,
                           **caps) if gathers else None
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(passes):
            for t in range(len(steps)):
                if pf:
                    pf.fetch(t)
                if compute_us is not None:
                    delay(compute_us[t], cs)
                if pf:
                    pf.release(t)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / passes
        st = pf.stats() if pf else None
        if pf:
            pf.close()
        return ms, st

    passes = max(1, min(args.steps, 5))
    walk()  # warm-up
    ms_gather, st_g = walk(passes=passes)
    gathered = (st_g["prefetch_numel"] + st_g["immediate_numel"]) / passes
    gather_bytes = gathered * 2 * (K + 1)      # shard read once + K full copies
    rate = gather_bytes / (ms_gather * 1e-3)   # bytes per second, host loop included
    compute_us = [args.compute_ratio * sum(numels[p] for p in st) * 2 * (K + 1) / rate * 1e6
                  for st in steps]
    # the phases are 10 ms apart (idle, untimed), so a kernel trace shows them apart
    ms_compute, _ = walk(compute_us=compute_us, gathers=False, passes=passes)
    time.sleep(0.01)
    ms_overlap, st = walk(compute_us=compute_us, passes=passes)
    time.sleep(0.01)
    ms_serial, _ = walk(serial=True, compute_us=compute_us, passes=passes)
    exposed = max(0.0, ms_overlap - ms_compute)
    return {
        "metric": "ZeRO-3 fetch/prefetch: ms per forward+backward pass with the gathers "
                  "overlapped, K=8, 6.74B-param transformer",
        "value": round(ms_overlap, 3), "unit": "ms", "n_gpus": 1, "steps": passes,
        "warmup": 1, "ms_per_step": round(ms_overlap, 3), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded generator, bf16 ~N(0,0.02); compute is a calibrated spin",
        "serial_ms": round(ms_serial, 3), "compute_only_ms": round(ms_compute, 3),
        "gathers_only_ms": round(ms_gather, 3),
        "exposed_gather_ms": round(exposed, 3),
        "hidden_fraction": round(1.0 - exposed / ms_gather, 4),
        "gathers_only_GBps": round(rate / 1e9, 1),
        "coordinator": {k: st[k] // (passes if k in ("gathers", "immediate_gathers",
                                                     "immediate_numel", "prefetch_numel",
                                                     "host_syncs", "stream_waits", "retained",
                                                     "prefetch_trimmed") else 1)
                        for k in st},
        "plan_arena_peak": plan["arena_peak"],
        "config": {"workload": "zero3_prefetch: 226 params (32 layers, hidden 4096, FFN 11008, "
                               "vocab 32000), 452 module visits per pass, 1/8 shards",
                   "K": K, "prefetch_bucket_numel": bucket, "max_live_numel": cfg["max_live"],
                   "max_reuse_numel": cfg["max_reuse"], "max_ongoing_fetches": cfg["max_ongoing"],
                   "arena_numel": arena, "compute_ratio": args.compute_ratio,
                   "gathered_numel_per_pass": int(gathered), "visit_numel_per_pass": visit_numel},
        "roofline": None, "cpu_baseline": None,
    }


# ------------------------------------------------------------ allreduce64
def bench_allreduce64(args):
    import torch

    import synth
    import gradient_sync_zr_amd as zr
    from synth import workloads as W

    cfg = W.ALLREDUCE64
    K, N = cfg["K"], cfg["N"]
    seed = W.seed_of(5)
    stride = -(-N // 128) * 128
    buf = torch.empty(K * stride, dtype=torch.bfloat16, device="cuda")
    ranks = [buf[r * stride:r * stride + N] for r in range(K)]
    ptrs = [t.data_ptr() for t in ranks]

    def regen():
        for r in range(K):
            synth.dev_normal_bf16(ranks[r], seed, r, 0, cfg["sigma"], cfg["outlier_p"],
                                  cfg["outlier_mag"])

    times = []
    for i in range(args.warmup + args.steps):
        regen()  # in-place sums grow, so every step starts from the same inputs (untimed)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        zr.zr_allreduce(ptrs, ptrs, N, average=False, fused=True, dtype=torch.bfloat16)
        e1.record()
        torch.cuda.synchronize()
        if i >= args.warmup:
            times.append(e0.elapsed_time(e1))
    ms_step = sum(times) / len(times)
    step_bytes = 2 * K * N * 2
    value = step_bytes / (ms_step * 1e-3) / 1e9
    src = kernel_source_hash(["zr_ar.hip", "zr_fold.hpp", "zr_fold_any.hpp", "zr_device.hpp"])
    traffic = read_traffic("ar_ring_bf16_k64_allreduce64.counters.txt", src, step_bytes)
    copy = copy_ceiling_gbps()
    return {
        "metric": "fused all-reduce GB/s (K reads + K writes), K=64, 1e9 bf16 elements",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic: seeded generator, bf16 ~N(0,1) with 1% at +-1e4",
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "config": {"workload": "allreduce64: K=64, N=1,000,000,007 per rank, in place, ring "
                               "order, fp32 accumulation, bf16 out (step = the all-reduce; "
                               "inputs regenerated untimed between steps)",
                   "K": K, "N": N, "bytes_per_step": step_bytes},
        "roofline": {"bound": "hbm", "kernel": "ar_kernel<bf16,K=64,ring>", "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "achieved": round(value, 1),
                     "copy_ceiling_GBps": copy,
                     "of_copy_ceiling": round(value / copy, 4) if copy else None,
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": step_bytes,
                     "kernel_source_sha256_16": src},
        "cpu_baseline": None,
    }


# ------------------------------------------------------------ frags_layer
def bench_frags_layer(args):
    """Discrete path at bandwidth scale: the seven gradients of one transformer
    layer (q, k, v, o: 4096x4096; gate, up, down: 4096x11008) per rank, reduced
    straight from the fragments, against flatten-into-a-bucket + reduce-scatter."""
    import torch

    import synth
    import gradient_sync_zr_amd as zr
    from synth import workloads as W

    cfg = W.FRAGS_LAYER
    K = cfg["K"]
    sizes = W.frags_layer_numels()
    N = sum(sizes)          # 202,375,168: a multiple of 8
    seed = W.seed_of(cfg["seed_cfg"])
    frags = [[torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes] for _ in range(K)]
    for r in range(K):
        for p in range(len(sizes)):
            synth.dev_normal_bf16(frags[r][p], seed, W.frags_layer_stream(r, p), 0, cfg["sigma"])
    buckets = [torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    parts = [torch.empty(N // K, dtype=torch.float32, device="cuda") for _ in range(K)]
    fp = [[t.data_ptr() for t in row] for row in frags]
    bp = [t.data_ptr() for t in buckets]
    pp = [t.data_ptr() for t in parts]

    def discrete():
        zr.zr_reduce_scatter_frags(fp, sizes, N, pp, chunk_shift=1, average=True,
                                   in_dtype=torch.bfloat16, out_dtype=torch.float32)

    def flat_rs():
        zr.zr_flatten_bucket(fp, sizes, bp, N, dtype=torch.bfloat16)
        zr.zr_reduce_scatter_avg(bp, N, pp, chunk_shift=1, average=True, in_dtype=torch.bfloat16,
                                 out_dtype=torch.float32)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_flat = timed(flat_rs)
    ms = timed(discrete)
    step_bytes = N * (2 * K + 4)  # one launch per step
    value = step_bytes / (ms * 1e-3) / 1e9
    src = kernel_source_hash(["zr_rsf_kernel.hpp", "zr_rsf.hip", "zr_fold.hpp", "zr_fold_any.hpp", "zr_device.hpp"])
    traffic = read_traffic("rsf_ring_bf16_f32_k8_frags_layer.counters.txt", src, step_bytes)
    copy = copy_ceiling_gbps()
    return {
        "metric": "discrete reduce-scatter+avg+cast GB/s from 7 fragments per rank, K=8",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic: seeded generator, bf16 ~N(0,1e-3)",
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "flatten_then_rs_ms": round(ms_flat, 4),
        "speedup_over_flatten_then_rs": round(ms_flat / ms, 3),
        "config": {"workload": "frags_layer: K=8, one transformer layer's 7 gradients per rank "
                               f"({N} elements), bucket never materialised",
                   "K": K, "N": N, "bytes_per_step": step_bytes},
        "roofline": {"bound": "hbm", "kernel": "rsf_kernel<bf16,f32,avg,ring>", "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "achieved": round(value, 1),
                     "copy_ceiling_GBps": copy,
                     "of_copy_ceiling": round(value / copy, 4) if copy else None,
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel_source_sha256_16": src},
        "cpu_baseline": None,
    }


# -------------------------------------------------------------- flatten8
def wall_us(fn, steps, warmup):
    """Host wall time per call of `fn` (microseconds), the device drained
    before and after: what a caller's loop of such calls costs."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e6 / steps


def bench_flatten8(args):
    import torch

    import synth
    import gradient_sync_zr_amd as zr
    from synth import workloads as W

    K, F = W.FLATTEN8["K"], W.FLATTEN8["n_frag"]
    seed = W.seed_of(2)
    sizes = W.flatten8_numels(F)
    P = -(-sum(sizes) // K) * K
    frags = [[torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes] for _ in range(K)]
    for r in range(K):
        for p in range(F):
            synth.dev_normal_bf16(frags[r][p], seed, W.flatten8_frag_stream(r, p), 0, 1e-3)
    buckets = [torch.empty(P, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    parts = [torch.empty(P // K, dtype=torch.float32, device="cuda") for _ in range(K)]
    fp = [[t.data_ptr() for t in row] for row in frags]
    bp = zr.table([t.data_ptr() for t in buckets])
    pp = zr.table([t.data_ptr() for t in parts])
    ws = torch.empty(zr.zr_workspace_bytes(K, F), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(zr.zr_workspace_bytes(K, F), dtype=torch.uint8, device="cuda")
    bf, f32 = torch.bfloat16, torch.float32

    def rs():
        zr.zr_reduce_scatter_avg(bp, P, pp, chunk_shift=1, average=True, in_dtype=bf, out_dtype=f32)

    def step():
        zr.zr_flatten_bucket(fp, sizes, bp, P, dtype=bf)
        rs()

    def step_discrete():
        zr.zr_reduce_scatter_frags(fp, sizes, P, pp, chunk_shift=1, average=True, in_dtype=bf,
                                   out_dtype=f32)

    flat_args = zr.FlatPlan(fp, sizes, bp, P, dtype=bf)
    flat_ws = zr.FlatPlan(fp, sizes, bp, P, dtype=bf, workspace=ws)
    plan = zr.RsfPlan(fp, sizes, P, pp, chunk_shift=1, average=True, in_dtype=bf, out_dtype=f32)
    plan_ws = zr.RsfPlan(fp, sizes, P, pp, chunk_shift=1, average=True, in_dtype=bf, out_dtype=f32,
                         workspace=ws2)
    us = wall_us(step, args.steps, args.warmup)
    us_discrete = wall_us(step_discrete, args.steps, args.warmup)
    us_flatplan_rs = wall_us(lambda: (flat_args.launch(), rs()), args.steps, args.warmup)
    us_flatplan_ws_rs = wall_us(lambda: (flat_ws.launch(), rs()), args.steps, args.warmup)
    rs_plan = zr.RsPlan(bp, P, pp, chunk_shift=1, average=True, in_dtype=bf, out_dtype=f32)
    stream = torch.cuda.current_stream().cuda_stream
    us_plans = wall_us(lambda: (flat_ws.launch(stream), rs_plan.launch(stream)), args.steps, args.warmup)
    us_plan = wall_us(plan.launch, args.steps, args.warmup)
    us_plan_ws = wall_us(plan_ws.launch, args.steps, args.warmup)
    # the plan's launches captured once in a HIP graph and replayed
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.launch()
    us_graph = wall_us(graph.replay, args.steps, args.warmup)
    launches = {"flatten": flat_args.info()["launches"], "flatten_ws": flat_ws.info()["launches"],
                "discrete": plan.info()["launches"], "discrete_ws": plan_ws.info()["launches"],
                "reduce_scatter": 1}
    for p_ in (flat_args, flat_ws, plan, plan_ws, rs_plan):
        p_.close()
    return {
        "metric": "flatten + reduce-scatter-avg microseconds per bucket, K=8, 64 fragments",
        "value": round(us, 2), "unit": "us", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 5), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic: seeded generator, bf16 ~N(0,1e-3)",
        "flatten_plan_then_rs_us": round(us_flatplan_rs, 2),
        "flatten_plan_ws_then_rs_us": round(us_flatplan_ws_rs, 2),
        "flatten_plan_ws_then_rs_plan_us": round(us_plans, 2),
        "discrete_path_us": round(us_discrete, 2),
        "discrete_plan_us": round(us_plan, 2),
        "discrete_plan_ws_us": round(us_plan_ws, 2),
        "discrete_plan_graph_us": round(us_graph, 2),
        "launches": launches,
        "config": {"workload": f"flatten8: K=8, 64 log-uniform fragments ({sum(sizes)} elements), "
                               f"bucket padded to {P}, then RS + /8 + fp32 cast (cache-resident, "
                               "launch-bound; host wall time per call)", "K": K},
        "roofline": None, "cpu_baseline": None,
    }


# ------------------------------------------------------------- frags_k64
def bench_frags_k64(args):
    """A bucket of 256 log-uniform fragments on K = 64 ranks: the discrete
    reduce-scatter and the flatten, as one-shot calls and as plans, without a
    workspace (4 fragments per launch) and with one (the table staged, one
    launch): microseconds per call and launches per call."""
    import torch

    import synth
    import gradient_sync_zr_amd as zr
    from synth import log_uniform_sizes
    from synth import workloads as W

    K, F = 64, 256
    seed = W.seed_of(2)
    sizes = log_uniform_sizes(seed + 64, F)
    N = -(-sum(sizes) // K) * K
    frags = [[torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes] for _ in range(K)]
    for r in range(K):
        for p in range(F):
            synth.dev_normal_bf16(frags[r][p], seed + 64, r * 4096 + p, 0, 1e-3)
    parts = [torch.empty(N // K, dtype=torch.float32, device="cuda") for _ in range(K)]
    buckets = [torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    fp = [[t.data_ptr() for t in row] for row in frags]
    pp = zr.table([t.data_ptr() for t in parts])
    bp = zr.table([t.data_ptr() for t in buckets])
    need = zr.zr_workspace_bytes(K, F)
    ws = [torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(3)]
    kw = dict(chunk_shift=1, average=True, in_dtype=torch.bfloat16, out_dtype=torch.float32)
    plan = zr.RsfPlan(fp, sizes, N, pp, **kw)
    plan_ws = zr.RsfPlan(fp, sizes, N, pp, workspace=ws[0], **kw)
    fplan = zr.FlatPlan(fp, sizes, bp, N, dtype=torch.bfloat16)
    fplan_ws = zr.FlatPlan(fp, sizes, bp, N, dtype=torch.bfloat16, workspace=ws[1])
    steps, warm = max(10, args.steps), max(3, args.warmup)

    def device_ms(fn, reps=20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    res = {
        "discrete_call_us": wall_us(lambda: zr.zr_reduce_scatter_frags(fp, sizes, N, pp, **kw), steps, warm),
        "discrete_call_ws_us": wall_us(lambda: zr.zr_reduce_scatter_frags(fp, sizes, N, pp, workspace=ws[2], **kw),
                                       steps, warm),
        "discrete_plan_us": wall_us(plan.launch, steps, warm),
        "discrete_plan_ws_us": wall_us(plan_ws.launch, steps, warm),
        "flatten_plan_us": wall_us(fplan.launch, steps, warm),
        "flatten_plan_ws_us": wall_us(fplan_ws.launch, steps, warm),
        "discrete_plan_device_ms": device_ms(plan.launch),
        "discrete_plan_ws_device_ms": device_ms(plan_ws.launch),
    }
    launches = {"discrete": plan.info()["launches"], "discrete_ws": plan_ws.info()["launches"],
                "flatten": fplan.info()["launches"], "flatten_ws": fplan_ws.info()["launches"],
                "staged_table_bytes": plan_ws.info()["table_bytes"], "workspace_bytes": need}
    for p_ in (plan, plan_ws, fplan, fplan_ws):
        p_.close()
    return {
        "metric": "discrete reduce-scatter microseconds per call, K=64, 256 fragments, plan with a "
                  "workspace-staged table",
        "value": round(res["discrete_plan_ws_us"], 2), "unit": "us", "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": round(res["discrete_plan_ws_us"] / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic: seeded generator, bf16 ~N(0,1e-3)",
        **{k: round(v, 4 if k.endswith("_ms") else 2) for k, v in res.items()},
        "launches": launches,
        "config": {"workload": f"frags_k64: K=64, {F} log-uniform fragments in [1, 65536] "
                               f"({sum(sizes)} elements per rank), N padded to {N}; host wall time "
                               "per call, device time per plan launch", "K": K, "n_frag": F},
        "roofline": None, "cpu_baseline": None,
    }


# ---------------------------------------------------------- flatten_layer
def bench_flatten_layer(args):
    """The bucket flatten at bandwidth scale: one transformer layer's seven
    gradients per rank (q, k, v, o: 4096x4096; gate, up, down: 4096x11008)
    copied into a flat bucket per rank, K = 8. Every byte is read once and
    written once: K * N * 2 bytes each way."""
    import torch

    import synth
    import gradient_sync_zr_amd as zr
    from synth import workloads as W

    cfg = W.FRAGS_LAYER
    K = cfg["K"]
    sizes = W.frags_layer_numels()
    N = sum(sizes)
    seed = W.seed_of(cfg["seed_cfg"])
    frags = [[torch.empty(n, dtype=torch.bfloat16, device="cuda") for n in sizes] for _ in range(K)]
    for r in range(K):
        for p in range(len(sizes)):
            synth.dev_normal_bf16(frags[r][p], seed, W.frags_layer_stream(r, p), 0, cfg["sigma"])
    buckets = [torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    fp = [[t.data_ptr() for t in row] for row in frags]
    plan = zr.FlatPlan(fp, sizes, [t.data_ptr() for t in buckets], N, dtype=torch.bfloat16)
    for _ in range(args.warmup):
        plan.launch()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[2 * i].record(s)
        plan.launch()
        ev[2 * i + 1].record(s)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    launch_ms = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps))
    avg = sum(launch_ms) / len(launch_ms)
    step_bytes = 2 * K * N * 2
    ok = all(torch.equal(buckets[r][sum(sizes[:p]):sum(sizes[:p + 1])], frags[r][p])
             for r in range(K) for p in range(len(sizes)))
    plan.close()
    del frags, buckets
    src = kernel_source_hash(["zr_flatten.hip", "zr_device.hpp"])
    traffic = read_traffic("flatten_bf16_k8_flatten_layer.counters.txt", src, step_bytes)
    copy = copy_ceiling_gbps()
    achieved = step_bytes / (avg * 1e-3) / 1e9
    return {
        "metric": "bucket flatten GB/s (K fragment reads + K bucket writes), K=8, one layer's 7 "
                  "gradients per rank",
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded generator, bf16 ~N(0,1e-3)",
        "launch_ms_median": round(launch_ms[len(launch_ms) // 2], 4),
        "launch_ms_min": round(launch_ms[0], 4),
        "copied_exactly": ok,
        "config": {"workload": f"flatten_layer: K=8, 7 fragments per rank ({N} elements) into one "
                               "bucket per rank (a plan: one launch)", "K": K, "N": N,
                   "bytes_per_step": step_bytes},
        "roofline": {"bound": "hbm", "kernel": "flatten_kernel<bf16>", "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "achieved": round(achieved, 1),
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "avg_launch_ms": round(avg, 4),
                     "copy_ceiling_GBps": copy,
                     "of_copy_ceiling": round(achieved / copy, 4) if copy else None,
                     "algorithmic_bytes_per_launch": step_bytes,
                     "kernel_source_sha256_16": src},
        "cpu_baseline": None,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="zero2",
                    choices=["zero2", "zero2_accum", "zero2_overlap", "zero3_ag", "zero3_prefetch",
                             "allreduce64", "flatten8", "frags_layer", "frags_k64", "flatten_layer"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--compute-ratio", type=float, default=1.5,
                    help="zero3_prefetch, zero2_overlap: each step's synthetic compute, in units "
                         "of its gather or reduction time")
    ap.add_argument("--arena-numel", type=int, default=1_600_000_000,
                    help="zero3_prefetch: arena elements per rank")
    ap.add_argument("--cpu-sample-elems", type=int, default=0,
                    help="element indices in the CPU-baseline sample (default: all of bucket 0)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the K ranks are simulated on one GPU; --gpus {args.gpus} is not "
              "supported (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    fn = {"zero2": bench_zero2, "zero2_accum": lambda a: bench_zero2(a, accumulate=True),
          "zero2_overlap": bench_zero2_overlap,
          "zero3_ag": bench_zero3, "zero3_prefetch": bench_zero3_prefetch,
          "allreduce64": bench_allreduce64,
          "flatten8": bench_flatten8, "frags_layer": bench_frags_layer, "frags_k64": bench_frags_k64,
          "flatten_layer": bench_flatten_layer}[args.workload]
    print(json.dumps(fn(args)), flush=True)


if __name__ == "__main__":
    main()
