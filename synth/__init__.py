"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the attention method: it only names the
workload shapes, draws seeded N(0, 1) values and rounds them to bfloat16.
Both the HIP path and the CPU oracle receive the arrays it returns; neither
side generates its own inputs.

Recipe (same for every workload):

* ``numpy.random.Generator(PCG64(seed))``;
* draw order: K ``[b, S, n_kv, d]`` in global position order, then V (same
  shape), then Q ``[b, c, n_q, d]`` for the measured rank only, in that
  rank's local order (c = S / N);
* values are float32 ``standard_normal``; for bfloat16 workloads they are
  rounded to nearest-even, and the oracle sees exactly those bf16 values
  widened to float64.

Document-masked workloads (all-gather CP) also draw document lengths, from
``Generator(PCG64(seed + 2000))``: log-uniform between S/256 and S/4 tokens,
packed from position 0 until the sequence is full (the last one cut at S).
The pages only say that a training sequence packs several documents; this
mix of short and long documents is the stand-in.
"""

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    b: int
    S: int
    N: int
    kind: str          # "contiguous" | "zigzag" | "striped"
    n_q: int
    n_kv: int
    d: int
    dtype: str         # "f32" | "bf16"
    scale_mult: float  # softmax scale = scale_mult / sqrt(d)
    causal: bool
    seed: int
    rank: int = 0
    docs: bool = False  # document mask (all-gather CP workloads)

    @property
    def c(self):
        return self.S // self.N

    @property
    def scale(self):
        return float(np.float32(self.scale_mult / np.sqrt(self.d)))

    def with_(self, **kw):
        return replace(self, **kw)


# The five workloads: a tiny fp32 ring; Llama-3-8B and Llama-3-70B attention
# shapes (GQA 32/8 and 64/8) at 32K and 128K with zig-zag over 8 ranks; the
# Ulysses post-all-to-all shape (full 128K sequence, 8 query heads / 1 KV head,
# no ring); and a 1M-token sequence over 32 ranks with scores scaled by 4.
WORKLOADS = {
    "tiny_ring_f32": Workload("tiny_ring_f32", 1, 256, 4, "contiguous", 1, 1, 64,
                              "f32", 1.0, False, 1),
    "llama3_8b_32k_zigzag": Workload("llama3_8b_32k_zigzag", 1, 32768, 8, "zigzag",
                                     32, 8, 128, "bf16", 1.0, True, 2),
    "llama3_70b_128k_zigzag": Workload("llama3_70b_128k_zigzag", 1, 131072, 8, "zigzag",
                                       64, 8, 128, "bf16", 1.0, True, 3),
    "ulysses_local_128k": Workload("ulysses_local_128k", 1, 131072, 1, "contiguous",
                                   8, 1, 128, "bf16", 1.0, True, 4),
    "long_1m_zigzag": Workload("long_1m_zigzag", 1, 1048576, 32, "zigzag",
                               8, 1, 128, "bf16", 4.0, True, 5),
}

# All-gather CP with a document mask: the Llama-3 shapes, zig-zag queries
# (the 2 x CP chunking), K/V of the whole sequence, packed documents.
ALLGATHER_WORKLOADS = {
    "llama3_8b_32k_allgather_docs": Workload("llama3_8b_32k_allgather_docs", 1, 32768, 8,
                                             "zigzag", 32, 8, 128, "bf16", 1.0, True, 7,
                                             docs=True),
    "llama3_70b_128k_allgather_docs": Workload("llama3_70b_128k_allgather_docs", 1, 131072, 8,
                                               "zigzag", 64, 8, 128, "bf16", 1.0, True, 6,
                                               docs=True),
}


def doc_lengths(S, seed, lo=None, hi=None):
    """Seeded document lengths that pack [0, S) (see the module docstring)."""
    lo = max(1, S // 256) if lo is None else lo
    hi = max(lo, S // 4) if hi is None else hi
    rng = np.random.Generator(np.random.PCG64(seed + 2000))
    out, total = [], 0
    while total < S:
        L = int(np.exp(rng.uniform(np.log(lo), np.log(hi + 1))))
        L = max(1, min(L, S - total))
        out.append(L)
        total += L
    return np.array(out, dtype=np.int64)


def bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits):
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Inputs:
    """Seeded inputs of one workload.

    ``q``/``k``/``v`` are the device-side element arrays: float32 for f32
    workloads, uint16 bfloat16 bit patterns for bf16 ones. ``q64``/``k64``/
    ``v64`` are the identical values widened to float64 (for the oracle).
    K and V are in global position order.
    """
    w: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray

    def _wide(self, a):
        if self.w.dtype == "bf16":
            return bf16_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    @property
    def q64(self):
        return self._wide(self.q)

    @property
    def k64(self):
        return self._wide(self.k)

    @property
    def v64(self):
        return self._wide(self.v)


def draw(w, q_rows=None):
    """Draw the inputs of workload ``w`` (see the module docstring for the recipe).

    ``q_rows`` optionally returns only those local query rows (the full Q is
    still drawn so the values do not depend on the subset).
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    shape_kv = (w.b, w.S, w.n_kv, w.d)
    k = rng.standard_normal(shape_kv, dtype=np.float32)
    v = rng.standard_normal(shape_kv, dtype=np.float32)
    q = rng.standard_normal((w.b, w.c, w.n_q, w.d), dtype=np.float32)
    if q_rows is not None:
        q = q[:, q_rows]
    if w.dtype == "bf16":
        k, v, q = bf16_bits(k), bf16_bits(v), bf16_bits(q)
    return Inputs(w, q, k, v)


def sample_rows(c, count, seed, must=()):
    """Sorted distinct local query rows: ``must`` rows, 16 at each end, the rest
    uniform from ``Generator(PCG64(seed + 1000))``."""
    rows = set(int(r) for r in must if 0 <= r < c)
    rows.update(range(min(16, c)))
    rows.update(range(max(0, c - 16), c))
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    while len(rows) < min(count, c):
        rows.add(int(rng.integers(0, c)))
    return np.array(sorted(rows), dtype=np.int64)
