"""ra_ring_fwd_noalloc (the allocation-free ring forward) against ra_ring_fwd,
through the C ABI: two calls in a row, the second on a smaller ring, each
compared bit for bit with ra_ring_fwd on the same inputs (same kernels in the
same order) and with the fp64 oracle to the parity bar."""

import ctypes

import numpy as np
import pytest
import torch

import ring_attention_context_amd as ra
import synth
from gpu_util import compare, require_gpu
from oracle import attention as oatt
from oracle import partition as opart
from ring_attention_context_amd import runner

pytestmark = pytest.mark.gpu


def _run_case(S, N, rank, n_q, n_kv, seed):
    w = synth.Workload("noalloc", 1, S, N, "zigzag", n_q, n_kv, 128, "bf16", 1.0, True, seed=seed,
                       rank=rank)
    print(f"noalloc S={S} N={N} rank={rank} n_q={n_q} n_kv={n_kv}", flush=True)
    inp = synth.draw(w)
    q, kc, vc = runner.ring_inputs(inp.q, inp.k, inp.v, w.dtype, w.kind, w.N, "cuda")
    call = runner.RingCall(q, kc, vc, kind=w.kind, S=S, N=N, rank=rank, causal=True)
    o_ref, lse_ref = call()
    torch.cuda.synchronize()
    o_ref, lse_ref = o_ref.cpu().numpy(), lse_ref.cpu().numpy()
    desc, _ = ra.ring_desc(b=1, n_q=n_q, n_kv=n_kv, d=128, dtype=ra.RA_BF16, causal=True,
                           kind="zigzag", S=S, N=N, rank=rank)
    assert ra.ra_ring_workspace_bytes(desc) <= ra.RA_NOALLOC_SCRATCH_BYTES
    o = torch.full(tuple(call.o.shape), float("nan"), device="cuda")
    lse = torch.full(tuple(call.lse.shape), float("nan"), device="cuda")
    lib = ra.load_library()
    st = lib.ra_ring_fwd_noalloc(ctypes.byref(desc), ctypes.c_void_p(q.data_ptr()),
                                 ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(vc.data_ptr()),
                                 ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == ra.RA_OK, ra.ra_last_error()
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)
    q_pos = opart.partition_map(w.kind, S, N, rank)
    ro, rl = oatt.naive_attention(inp.q64, inp.k64, inp.v64, q_pos, np.arange(S), True, w.scale)
    do, dl = compare(o, lse, ro, rl, "bf16", f"noalloc S={S}")
    print(f"  bit-identical to ra_ring_fwd; max|dO| {do:.2e} max|dlse| {dl:.2e}", flush=True)


def test_ring_fwd_noalloc_two_calls_match_ring_fwd():
    require_gpu()
    _run_case(4096, 4, 1, 8, 2, seed=501)     # first call on the device
    _run_case(1024, 4, 2, 4, 1, seed=502)     # smaller ring, same scratch
