"""Plain-copy and read-only HBM probes (test kit, not part of the library).

Runs tk_copy over a buffer of known size: its average kernel time gives the
practical copy bandwidth of the device, and under rocprofv3 --pmc its
FETCH_SIZE / WRITE_SIZE give the counter-to-bytes factor for known traffic
(exactly `bytes` read and `bytes` written per launch). By default the copy's
grid has one block per 4 KiB (one 16-byte unit per thread), the fastest
launch shape measured for a copy; --blocks-per-cu N > 0 gives it a
persistent grid of N blocks per CU striding over the buffer instead. The
read probe (tk_read, which also writes one partial sum per block) always
runs on a persistent grid of 8 blocks per CU.

    python tests/kit/hbm_copy.py [--gib 4] [--reps 20] [--blocks-per-cu 0]
"""
import argparse
import ctypes
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gib", type=float, default=4.0)
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--blocks-per-cu", type=int, default=0)
    args = ap.parse_args()
    import torch
    L = ctypes.CDLL(os.path.join(HERE, "libtestkit.so"))
    for f in (L.tk_copy, L.tk_read):
        f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                      ctypes.c_void_p]
    nbytes = int(args.gib * 2 ** 30) // 16 * 16
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = cus * args.blocks_per_cu if args.blocks_per_cu > 0 else nbytes // (16 * 256)
    read_blocks = cus * 8
    sink = torch.empty(read_blocks * 4, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    out = {"bytes": nbytes, "copy_blocks": blocks, "read_blocks": read_blocks}
    for name, fn, moved in (("copy", lambda: L.tk_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                                                        blocks, s), 2 * nbytes),
                            ("read", lambda: L.tk_read(src.data_ptr(), sink.data_ptr(), nbytes,
                                                        read_blocks, s), nbytes)):
        for _ in range(3):
            assert fn() == 0
        torch.cuda.synchronize()
        ms = []
        for _ in range(args.reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            assert fn() == 0
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        avg = sum(ms) / len(ms)
        out[name] = {"avg_ms": round(avg, 4), "GBps": round(moved / (avg * 1e-3) / 1e9, 1)}
    assert torch.equal(src, dst)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    sys.exit(main())
