"""Shapes, value recipes and seeds of the five gradient-bucket workloads.

Each workload is described by plain numbers only; values come from the
counter-based generator in :mod:`synth`. Seeds are ``0x5A520000 + id``.

1. ``ring4``      ring all-reduce, K=4, N=16 fp32 per rank, integers U[-8, 8].
2. ``flatten8``   K=8, 64 fragments per rank with log-uniform numel in
                  [1, 65536], bf16 ~N(0, 1e-3), flattened into one bucket
                  padded to a multiple of 8, reduce-scatter + average, fp32 out.
3. ``zero2_grad`` K=8, 2,376,274,560 bf16 elements per rank ~N(0, 1e-3),
                  buckets of 500,000,000 elements, ring reduce-scatter, /8,
                  fp32 partitions.
4. ``zero3_ag``   K=8 bf16 shards of a 32-layer transformer (hidden 4096,
                  FFN 11008, vocab 32000), weights ~N(0, 0.02), gathered in
                  50 MB prefetch buckets.
5. ``allreduce64`` K=64, N=1,000,000,007 bf16 ~N(0, 1) with 1% of the
                  elements set to +-1e4, ring all-reduce (sum), bf16 out.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

SEED_BASE = 0x5A520000


def seed_of(cfg_id: int) -> int:
    return SEED_BASE + cfg_id


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


# ------------------------------------------------------------------ cfg 1
RING4 = dict(id=1, K=4, N=16, lo=-8, hi=8)

# ------------------------------------------------------------------ cfg 2
FLATTEN8 = dict(id=2, K=8, n_frag=64, max_numel=65536, sigma=1e-3)


def flatten8_frag_stream(rank: int, frag: int) -> int:
    """Generator stream of fragment `frag` on rank `rank`."""
    return rank * 4096 + frag


def flatten8_numels(n_frag: int = 64) -> List[int]:
    from . import log_uniform_sizes
    return log_uniform_sizes(seed_of(2), n_frag)


# ------------------------------------------------------------------ cfg 3
ZERO2 = dict(id=3, K=8, N_total=2_376_274_560, bucket=500_000_000, sigma=1e-3, shift=1)


def zero2_buckets(n_total: int = ZERO2["N_total"], bucket: int = ZERO2["bucket"]
                  ) -> List[Tuple[int, int]]:
    """(start, numel) of each bucket of the flat per-rank gradient."""
    out, start = [], 0
    while start < n_total:
        n = min(bucket, n_total - start)
        out.append((start, n))
        start += n
    return out


# ------------------------------------------------------------------ cfg 4
@dataclass
class Param:
    name: str
    numel: int


def llama_like_params(layers: int = 32, hidden: int = 4096, ffn: int = 11008,
                      vocab: int = 32000) -> List[Param]:
    """Embedding, then per layer q, k, v, o (hidden x hidden) and gate, up, down
    (hidden x ffn), then an untied lm_head; norm vectors are left out."""
    ps = [Param("embed", vocab * hidden)]
    for i in range(layers):
        for n in ("q", "k", "v", "o"):
            ps.append(Param(f"l{i}.{n}", hidden * hidden))
        for n in ("gate", "up", "down"):
            ps.append(Param(f"l{i}.{n}", hidden * ffn))
    ps.append(Param("lm_head", vocab * hidden))
    return ps


ZERO3 = dict(id=4, K=8, sigma=0.02, shift=0, prefetch_bytes=50_000_000, elem_bytes=2,
             max_live=1_000_000_000, max_reuse=1_000_000_000, max_ongoing=2)


def zero3_trace(n_params: int) -> List[List[int]]:
    """One parameter per module visit: forward in order, then backward in
    reverse order."""
    fwd = [[p] for p in range(n_params)]
    return fwd + fwd[::-1]

# ------------------------------------------------------------------ cfg 5
ALLREDUCE64 = dict(id=5, K=64, N=1_000_000_007, sigma=1.0, outlier_p=0.01, outlier_mag=1e4)


# ------------------------------------------- discrete path at full scale
# The seven weight gradients of one transformer layer of the parameter set
# above (q, k, v, o, gate, up, down: 202,375,168 elements) per rank, reduced
# straight from the fragments; seeded under the ZeRO-2 gradient seed.
FRAGS_LAYER = dict(K=8, sigma=1e-3, shift=1, seed_cfg=3)


def frags_layer_numels() -> List[int]:
    return [p.numel for p in llama_like_params(layers=1)[1:8]]


def frags_layer_stream(rank: int, frag: int) -> int:
    return 1000 + rank * 8 + frag
