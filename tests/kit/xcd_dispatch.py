"""Which XCD runs each block of a one-block-per-tile launch (test kit, not
part of the library).

Launches tk_xcd with one block per 4 KiB copy tile; each block records the
XCD it ran on (its XCC_ID hardware register). Prints, per run, how many
blocks ran on XCD (block index mod the number of XCDs seen), the blocks per
XCD, and the first 16 blocks' XCDs.

    python tests/kit/xcd_dispatch.py [--blocks 65536] [--runs 3]
"""
import argparse
import ctypes
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--blocks", type=int, default=65536)
    ap.add_argument("--runs", type=int, default=3)
    args = ap.parse_args()
    import torch
    L = ctypes.CDLL(os.path.join(HERE, "libtestkit.so"))
    L.tk_xcd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                         ctypes.c_void_p]
    n = args.blocks * 4096 // 4  # 4 KiB per block
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    xcd = torch.empty(args.blocks, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    for run in range(args.runs):
        xcd.fill_(-1)
        assert L.tk_xcd(src.data_ptr(), dst.data_ptr(), xcd.data_ptr(), args.blocks, s) == 0
        torch.cuda.synchronize()
        h = xcd.cpu().tolist()
        seen = sorted(set(h))
        nx = len(seen)
        match = sum(1 for i, x in enumerate(h) if x == i % nx)
        print(json.dumps({"run": run, "blocks": args.blocks, "xcds": nx,
                          "blocks_on_xcd_i_mod_n": match,
                          "per_xcd": {str(x): h.count(x) for x in seen}, "first_16": h[:16]}),
              flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
