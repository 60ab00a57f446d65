"""Matched read:write-mix stream probe (test kit, not part of the library).

tk_mix replays the reduce-scatter's memory access pattern at the shape of one
500M-element bucket of the ZeRO-2 workload (K = 8, chunk C = 62,500,864, the
multiple of 4096 next to 62.5M) with no arithmetic: every tile loads eight
bf16 streams with 8-byte non-temporal loads and writes one fp32 block (4 KiB
with one slice per wave, 16 KiB with four: the kernel's two tile shapes) with
16-byte non-temporal stores, tiles numbered by pairs of chunks as the kernel
numbers them. Four modes, each timed with events over `reps` launches after
3 warm-ups:

  mix     loads + stores: 16 B read and 4 B written per element index
  reads   the loads alone (the reads' share of the ceiling)
  writes  the stores alone (the writes' share)
  accum   loads + each output word read back before its store: 20 B read and
          4 B written per element index, the accumulating reduce-scatter's mix

The mix rate is the practical ceiling of a stream with the reduce-scatter's
own traffic mix on this GPU, measured the way the kernel is measured.

    python tests/kit/mix_probe.py [--reps 20] [--slices 1|4]
"""
import argparse
import ctypes
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
K = 8
CHUNK = 15259 * 4096  # 62,500,864 elements: one 500M-element bucket's chunk, whole tiles


def measure(reps=20, C=CHUNK, modes=("mix", "reads", "writes"), slices=4):
    """{mode: {"avg_ms", "min_ms", "GBps"}} for the requested modes, with
    tiles of `slices` slices per wave (1 or 4), or None when the test kit is
    not built."""
    import torch
    path = os.path.join(HERE, "libtestkit.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.tk_mix.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong,
                         ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    n = K * C
    ins = [torch.ones(n, dtype=torch.bfloat16, device="cuda") for _ in range(K)]
    outs = [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(K)]
    sink = torch.empty(4 * K * (C // (1024 * slices)), dtype=torch.int32, device="cuda")  # a word per tile
    tin = (ctypes.c_void_p * K)(*[t.data_ptr() for t in ins])
    tout = (ctypes.c_void_p * K)(*[t.data_ptr() for t in outs])
    s = torch.cuda.current_stream().cuda_stream
    moved = {"mix": n * (2 * K + 4), "reads": n * 2 * K, "writes": n * 4, "accum": n * (2 * K + 8)}
    code = {"mix": 0, "reads": 1, "writes": 2, "accum": 3}
    res = {}
    for m in modes:
        def run():
            if L.tk_mix(tin, tout, sink.data_ptr(), C, code[m], slices, s) != 0:
                raise RuntimeError("tk_mix launch failed")
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        avg = sum(ms) / len(ms)
        res[m] = {"avg_ms": round(avg, 4), "min_ms": round(min(ms), 4),
                  "GBps": round(moved[m] / (avg * 1e-3) / 1e9, 1)}
    del ins, outs, sink
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--slices", type=int, default=4, choices=(1, 4))
    args = ap.parse_args()
    out = {"K": K, "C": CHUNK, "slices": args.slices, "element_indices": K * CHUNK,
           "bytes_mix": K * CHUNK * (2 * K + 4)}
    out.update(measure(args.reps, modes=("mix", "reads", "writes", "accum"), slices=args.slices))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
