"""Helpers for the GPU parity tests: seeded inputs to device tensors and the
tolerance checks of the parity bar (O max-abs <= 1e-5 for float32 inputs,
<= 1e-2 for bfloat16; lse abs <= 2e-3; -inf rows exactly -inf with o = 0)."""

import numpy as np
import torch

import synth

TOL_O = {"f32": 1e-5, "bf16": 1e-2}
TOL_LSE = 2e-3


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def to_device(arr, dtype):
    """Host array -> device tensor. bf16 arrays are uint16 bit patterns."""
    from ring_attention_context_amd.runner import host_to_device
    return host_to_device(arr, dtype, "cuda")


def rand_inputs(shape, dtype, rng, mult=1.0):
    x = (rng.standard_normal(shape, dtype=np.float32) * np.float32(mult)).astype(np.float32)
    if dtype == "bf16":
        bits = synth.bf16_bits(x)
        return bits, synth.bf16_to_f32(bits).astype(np.float64)
    return x, x.astype(np.float64)


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    """Assert the parity bar; returns (max |dO|, max |dlse|) over finite rows."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    neg = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), neg), f"{what}: -inf pattern differs"
    assert not np.isnan(o_gpu).any() and not np.isnan(lse_gpu).any(), f"{what}: NaN"
    if neg.any():
        assert not o_gpu[neg].any(), f"{what}: rows without keys must have o = 0"
    do = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    fin = ~neg
    dl = float(np.max(np.abs(lse_gpu[fin] - lse_ref[fin]))) if fin.any() else 0.0
    assert do <= TOL_O[dtype], f"{what}: max |dO| = {do:.3g} > {TOL_O[dtype]}"
    assert dl <= TOL_LSE, f"{what}: max |dlse| = {dl:.3g} > {TOL_LSE}"
    return do, dl


def oracle_rows_threaded(fn, rows, q64, q_pos, elems_per_chunk=1 << 22):
    """fn(q_rows, q_pos_rows) -> (o, lse) for a row subset; run over chunks of
    ``rows`` in a thread pool (rows are independent, and NumPy's matrix
    products and ufuncs release the GIL), BLAS limited to one thread per
    worker. Returns (o, lse) of ``rows`` in their order."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    rows = np.asarray(rows)
    S = q_pos.max() + 1 if len(q_pos) else 1
    per = max(1, int(elems_per_chunk // max(1, S)))
    chunks = [rows[i:i + per] for i in range(0, len(rows), per)]
    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(chunks)))
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(lambda r: fn(q64[:, r], q_pos[r]), chunks))
    o = np.concatenate([p[0] for p in parts], axis=1)
    lse = np.concatenate([p[1] for p in parts], axis=1)
    return o, lse


_FWD_CACHE = {}


def oracle_forward_rows(w, rows=None):
    """The fp64 oracle's (o, lse) of workload ``w``'s rank on ``rows`` (every
    row when None), computed once per (workload, rows) in this process."""
    from oracle import attention as oatt
    from oracle import partition as opart
    key = (w, None if rows is None else tuple(int(r) for r in rows))
    if key not in _FWD_CACHE:
        inp = synth.draw(w)
        q64, k64, v64 = inp.q64, inp.k64, inp.v64
        q_pos = opart.partition_map(w.kind, w.S, w.N, w.rank)
        sel = np.arange(w.c) if rows is None else np.asarray(rows)
        _FWD_CACHE[key] = oracle_rows_threaded(
            lambda qr, qp: oatt.rows_attention(qr, k64, v64, qp, w.causal, w.scale), sel, q64,
            q_pos)
    return _FWD_CACHE[key]


def sample_keys(kind, S, N, count, seed):
    """Sorted distinct global key positions: the first and last key of every
    chunk half (zig-zag) or chunk, the sequence's ends, the rest uniform from
    Generator(PCG64(seed + 3000))."""
    from oracle import partition as opart
    keys = {0, S - 1}
    for j in range(N):
        m = opart.partition_map(kind, S, N, j)
        h = len(m) // 2
        keys.update(int(x) for x in (m[0], m[-1], m[max(h - 1, 0)], m[h]))
    rng = np.random.Generator(np.random.PCG64(seed + 3000))
    while len(keys) < min(count, S):
        keys.add(int(rng.integers(0, S)))
    return np.array(sorted(keys), dtype=np.int64)


def key_slots(kind, S, N, keys):
    """(chunk, local row) of each global key position under map ``kind``."""
    from oracle import partition as opart
    where = {}
    for j in range(N):
        for a, p in enumerate(opart.partition_map(kind, S, N, j)):
            where[int(p)] = (j, a)
    return [where[int(p)] for p in keys]
