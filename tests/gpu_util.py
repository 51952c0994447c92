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
