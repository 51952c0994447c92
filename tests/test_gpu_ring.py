"""GPU parity of ra_ring_fwd against the CPU oracle, through the C ABI.

Small rings are checked on every output; the five measured workloads run at
full size in the same launch configuration the benchmark times and are
checked on every row (the 32K shard) or 256 sampled query rows (all heads,
every element of o and lse)."""

import math

import numpy as np
import pytest
import torch

import ring_attention_context_amd as ra
import synth
from gpu_util import compare, oracle_forward_rows, require_gpu
from oracle import attention as oatt
from oracle import partition as opart
from ring_attention_context_amd import runner

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def device_inputs(w, inp):
    return runner.ring_inputs(inp.q, inp.k, inp.v, w.dtype, w.kind, w.N, "cuda")


def run_ring(w, q, kc, vc, flags=0, poison=False, step_events=False):
    call = runner.RingCall(q, kc, vc, kind=w.kind, S=w.S, N=w.N, rank=w.rank, causal=w.causal,
                           scale=w.scale, flags=flags, step_events=step_events)
    if poison:
        call.workspace.fill_(0xFF)   # NaN in every float / bf16 lane
        call.o.fill_(float("nan"))
        call.lse.fill_(float("nan"))
    o, lse = call()
    torch.cuda.synchronize()
    return call, o.cpu().numpy(), lse.cpu().numpy()


def test_tiny_ring_f32_full():
    """S = 256, N = 4 contiguous, rank 0, non-causal, fp32, d = 64: every output."""
    w = synth.WORKLOADS["tiny_ring_f32"]
    print(f"workload {w.name}", flush=True)
    inp = synth.draw(w)
    q, kc, vc = device_inputs(w, inp)
    _, o, lse = run_ring(w, q, kc, vc)
    ro, rl = oatt.ring_attention(inp.q64, inp.k64, inp.v64, w.kind, w.S, w.N, w.rank,
                                 w.causal, w.scale)
    do, dl = compare(o, lse, ro, rl, "f32", w.name)
    no, nl = oatt.naive_attention(inp.q64, inp.k64, inp.v64,
                                  opart.partition_map(w.kind, w.S, w.N, w.rank),
                                  np.arange(w.S), w.causal, w.scale)
    compare(o, lse, no, nl, "f32", w.name + " vs naive")
    print(f"  max|dO| {do:.2e} max|dlse| {dl:.2e}")


SMALL = []
for kind in ("contiguous", "zigzag", "striped"):
    for N in (1, 2, 4):
        for rank in sorted({0, N // 2, N - 1}):
            SMALL.append((kind, N, rank, True, "bf16"))
SMALL += [("zigzag", 4, 1, False, "bf16"), ("striped", 4, 2, True, "f32"),
          ("zigzag", 8, 7, True, "f32"), ("contiguous", 2, 1, False, "f32")]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_small_ring_matches_oracle(case):
    kind, N, rank, causal, dtype = case
    print(f"ring {case}", flush=True)
    S = 192 * 2 * N   # c = 384 per rank: several tiles, zig-zag halves of 192
    w = synth.Workload("small", 1, S, N, kind, 8, 2, 128, dtype, 1.0, causal, seed=40 + N,
                       rank=rank)
    inp = synth.draw(w)
    q, kc, vc = device_inputs(w, inp)
    _, o, lse = run_ring(w, q, kc, vc)
    ro, rl = oatt.naive_attention(inp.q64, inp.k64, inp.v64,
                                  opart.partition_map(kind, S, N, rank), np.arange(S), causal,
                                  w.scale)
    compare(o, lse, ro, rl, dtype, str(case))


@pytest.mark.parametrize("case", [("zigzag", 80, 4, 1), ("contiguous", 200, 2, 1),
                                  ("striped", 36, 3, 2), ("zigzag", 4 * 2 * 7, 4, 3)],
                         ids=lambda c: "-".join(map(str, c)))
def test_small_ring_rows_layout_fallback(case):
    """bf16 rings whose chunk length c is not a multiple of 8 keep V row-major
    (plain copies, transposing LDS reads) instead of the transposed staging."""
    kind, S, N, rank = case
    print(f"ring fallback {case}", flush=True)
    w = synth.Workload("odd_c", 1, S, N, kind, 8, 2, 128, "bf16", 1.0, True, seed=S + N,
                       rank=rank)
    assert w.c % 8 != 0
    inp = synth.draw(w)
    q, kc, vc = device_inputs(w, inp)
    _, o, lse = run_ring(w, q, kc, vc)
    ro, rl = oatt.naive_attention(inp.q64, inp.k64, inp.v64,
                                  opart.partition_map(kind, S, N, rank), np.arange(S), True,
                                  w.scale)
    compare(o, lse, ro, rl, "bf16", str(case))


def _flag_case(dtype="bf16"):
    w = synth.Workload("flags", 1, 4096, 4, "zigzag", 8, 1, 128, dtype, 1.0, True, seed=77,
                       rank=1)
    inp = synth.draw(w)
    return w, inp, device_inputs(w, inp)


def test_overlap_equals_serialized_bitwise():
    """Same kernels in the same order: any difference would be a copy/compute race.
    The chunks here are small, so the default runs the copies on `compute` and
    pairs visible steps in one launch; RA_RING_STEPWISE keeps one launch per
    step, the launches RA_RING_OVERLAP makes."""
    w, inp, dev = _flag_case()
    _, o1, l1 = run_ring(w, *dev, flags=ra.RA_RING_OVERLAP)
    _, o2, l2 = run_ring(w, *dev, flags=ra.RA_RING_SERIALIZE | ra.RA_RING_STEPWISE)
    _, o3, l3 = run_ring(w, *dev, flags=ra.RA_RING_SERIALIZE)
    _, o4, l4 = run_ring(w, *dev)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)


PAIRED = [("zigzag", 3960, 3, 2, True),       # odd N (a last step alone), ragged tiles
          ("zigzag", 4096, 4, 1, False),      # non-causal: every step visible
          ("contiguous", 4096, 4, 2, True),   # step 3 is empty: steps 0-1 paired, 2 alone
          ("striped", 4096, 4, 3, True),
          ("zigzag", 8192, 8, 0, True)]


@pytest.mark.parametrize("case", PAIRED, ids=lambda c: "-".join(map(str, c)))
def test_paired_steps_match_stepwise_and_oracle(case):
    """Two visible steps per launch (the default when the copies run on
    `compute`) against one launch per step and the fp64 oracle on every row:
    both within the parity bar, and apart only by rounding."""
    kind, S, N, rank, causal = case
    print(f"paired ring {case}", flush=True)
    w = synth.Workload("paired", 1, S, N, kind, 8, 2, 128, "bf16", 1.0, causal, seed=S + rank,
                       rank=rank)
    inp = synth.draw(w)
    dev = device_inputs(w, inp)
    _, o1, l1 = run_ring(w, *dev, flags=ra.RA_RING_SERIALIZE)
    _, o2, l2 = run_ring(w, *dev, flags=ra.RA_RING_SERIALIZE | ra.RA_RING_STEPWISE)
    ro, rl = oatt.naive_attention(inp.q64, inp.k64, inp.v64,
                                  opart.partition_map(kind, S, N, rank), np.arange(S), causal,
                                  w.scale)
    d1 = compare(o1, l1, ro, rl, "bf16", f"{case} paired")
    d2 = compare(o2, l2, ro, rl, "bf16", f"{case} stepwise")
    assert np.array_equal(np.isneginf(l1), np.isneginf(l2))
    fin = np.isfinite(l1)
    assert np.max(np.abs(l1[fin] - l2[fin])) <= 1e-4
    assert np.max(np.abs(o1 - o2)) <= 8e-3
    print(f"  paired max|dO| {d1[0]:.2e} |dlse| {d1[1]:.2e}; stepwise {d2[0]:.2e} {d2[1]:.2e}")


@pytest.mark.parametrize("flags", [ra.RA_RING_OVERLAP, 0])
def test_graph_replay_matches_eager(flags):
    """One ra_ring_fwd call captured as a HIP graph (the copy stream joining
    the capture when the copies overlap) and replayed three times, with eager
    work and synchronisations between the replays and the outputs poisoned
    before each: every replay equals the eager call bit for bit."""
    w, inp, dev = _flag_case()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        call = runner.RingCall(*dev, kind=w.kind, S=w.S, N=w.N, rank=w.rank, causal=w.causal,
                               scale=w.scale, flags=flags, compute=side)
        o_ref, l_ref = (t.clone() for t in call())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call()
    torch.cuda.synchronize()
    for i in range(3):
        call.o.fill_(float("nan"))
        call.lse.fill_(float("nan"))
        eager = run_ring(w, *dev, flags=flags)   # other eager work between the replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(call.o, o_ref) and torch.equal(call.lse, l_ref), i
        assert np.array_equal(eager[1], o_ref.cpu().numpy())


def test_poisoned_workspace_and_outputs():
    """NaN-filled workspace and outputs: a read before its write would surface as NaN."""
    w, inp, dev = _flag_case()
    _, o1, l1 = run_ring(w, *dev)
    _, o2, l2 = run_ring(w, *dev, poison=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    _, o3, l3 = run_ring(w, *dev, flags=ra.RA_RING_UNFUSED_MERGE, poison=True)
    assert not np.isnan(o3).any()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unfused_merge_matches_fused_and_oracle(dtype):
    w, inp, dev = _flag_case(dtype)
    _, o1, l1 = run_ring(w, *dev)
    _, o2, l2 = run_ring(w, *dev, flags=ra.RA_RING_UNFUSED_MERGE)
    q_pos = opart.partition_map(w.kind, w.S, w.N, w.rank)
    rows = synth.sample_rows(w.c, 96, w.seed, must=[0, w.c // 2 - 1, w.c // 2, w.c - 1])
    ro, rl = oatt.rows_attention(inp.q64[:, rows], inp.k64, inp.v64, q_pos[rows], True, w.scale)
    compare(o1[:, rows], l1[:, rows], ro, rl, dtype, "fused")
    compare(o2[:, rows], l2[:, rows], ro, rl, dtype, "unfused")


def test_step_events_record_every_step():
    w, inp, dev = _flag_case()
    call, _, _ = run_ring(w, *dev, step_events=True)
    ms = call.step_ms()
    assert len(ms) == w.N and all(t >= 0 for t in ms)


def test_empty_sequence_is_a_no_op():
    w = synth.Workload("empty", 1, 0, 4, "zigzag", 8, 1, 128, "bf16", 1.0, True, seed=1)
    q = torch.empty(1, 0, 8, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.empty(4, 1, 0, 1, 128, dtype=torch.bfloat16, device="cuda")
    call = runner.RingCall(q, kc, kc, kind=w.kind, S=0, N=4, rank=0, causal=True)
    call()
    torch.cuda.synchronize()


FULL = [
    ("llama3_8b_32k_zigzag", {}),
    ("llama3_70b_128k_zigzag", {}),
    ("llama3_70b_128k_zigzag", {"kind": "contiguous", "rank": 7}),
    ("llama3_70b_128k_zigzag", {"kind": "striped", "rank": 3}),
    ("ulysses_local_128k", {}),
    ("long_1m_zigzag", {}),
]


@pytest.mark.parametrize("name,over", FULL, ids=lambda x: str(x))
def test_full_workload_rows(name, over):
    """Full-size run (all rows computed on the GPU) in the benchmark's
    configuration. The 32K Llama-3-8B shard is compared on every row x every
    head; the larger workloads on 256 sampled rows (the zig-zag half boundaries
    and diagonals, 16 rows at each end, the rest seeded uniform) x all heads,
    every element of o and lse."""
    w = synth.WORKLOADS[name].with_(**over)
    print(f"workload {w.name} {over}", flush=True)
    inp = synth.draw(w)
    q, kc, vc = device_inputs(w, inp)
    _, o, lse = run_ring(w, q, kc, vc)
    del q, kc, vc
    torch.cuda.empty_cache()
    c = w.c
    every_row = name == "llama3_8b_32k_zigzag" and not over
    rows = np.arange(c) if every_row else synth.sample_rows(
        c, 256, w.seed, must=[0, 1, c // 2 - 1, c // 2, c // 2 + 1, c - 1])
    ro, rl = oracle_forward_rows(w, None if every_row else rows)
    do, dl = compare(o[:, rows], lse[:, rows], ro, rl, w.dtype, w.name)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    print(f"  rows {len(rows)} max|dO| {do:.2e} max|dlse| {dl:.2e}", flush=True)


@pytest.mark.parametrize("kind", opart.KINDS)
def test_device_position_maps_bit_exact(kind):
    """The position maps the ring writes into its workspace (the first S int32:
    rank j's c positions at [j*c, (j+1)*c)) equal the oracle's maps bit for
    bit, for N in {1, 2, 3, 4, 8, 32}; the backward's workspace the same."""
    for N in (1, 2, 3, 4, 8, 32):
        S = 2 * N * 24
        rank = N // 2
        print(f"positions {kind} N={N} S={S}", flush=True)
        w = synth.Workload("pos", 1, S, N, kind, 1, 1, 128, "bf16", 1.0, True, seed=N, rank=rank)
        inp = synth.draw(w)
        q, kc, vc = device_inputs(w, inp)
        call, _, _ = run_ring(w, q, kc, vc, poison=True)
        got = call.workspace[:S * 4].view(torch.int32).cpu().numpy().reshape(N, S // N)
        for j in range(N):
            assert np.array_equal(got[j], opart.partition_map(kind, S, N, j)), (kind, N, j)
        desc, _ = ra.ring_desc(b=1, n_q=1, n_kv=1, d=128, dtype=ra.RA_BF16, causal=True, kind=kind,
                               S=S, N=N, rank=rank)
        ws = torch.full((ra.ra_ring_bwd_workspace_bytes(desc),), 0xFF, dtype=torch.uint8,
                        device="cuda")
        dq = torch.empty(tuple(q.shape), device="cuda")
        dkc = torch.zeros(tuple(kc.shape), device="cuda")
        ra.ra_ring_bwd(desc, q, kc, vc, call.o, call.lse, q, dq, dkc, torch.zeros_like(dkc), ws)
        torch.cuda.synchronize()
        got = ws[:S * 4].view(torch.int32).cpu().numpy().reshape(N, S // N)
        for j in range(N):
            assert np.array_equal(got[j], opart.partition_map(kind, S, N, j)), ("bwd", kind, N, j)
