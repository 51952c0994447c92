"""GPU parity of the backward path (ra_attn_bwd_delta, ra_block_attn_bwd,
ra_ring_bwd) against the fp64 backward oracle, through the C ABI.

Tolerance: the MFMAs consume P and dS rounded to bf16 (relative error 2^-9 per
element) and accumulate in fp32, so each gradient is compared as
max |g - g_ref| <= 1e-2 * max |g_ref| + 1e-4: about five times the
per-element rounding, and far below what a wrong term, sign, scale or mask
produces (tests/test_oracle_bwd.py shows those move the gradients by O(1))."""

import math
import zlib

import numpy as np
import pytest
import torch

import ring_attention_context_amd as ra
import synth
from gpu_util import (key_slots, oracle_forward_rows, rand_inputs, require_gpu,
                      sample_keys, to_device)
from oracle import attention as oatt
from oracle import backward as obwd
from oracle import partition as opart
from ring_attention_context_amd import runner

pytestmark = pytest.mark.gpu

TOL_REL, TOL_ABS = 1e-2, 1e-4


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def grad_close(got, want, what):
    got = np.asarray(got, dtype=np.float64)
    assert not np.isnan(got).any(), f"{what}: NaN"
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    scale = float(np.max(np.abs(want))) if want.size else 0.0
    assert err <= TOL_REL * scale + TOL_ABS, f"{what}: max err {err:.3g} vs max |ref| {scale:.3g}"
    return err, scale


def test_delta_matches_numpy():
    rng = np.random.default_rng(1)
    for shape, dt in (((2, 77, 4, 128), "bf16"), ((1, 33, 3, 64), "f32"), ((1, 5, 2, 128), "f32")):
        print(f"delta {shape} {dt}", flush=True)
        do, do64 = rand_inputs(shape, dt, rng)
        o = rng.standard_normal(shape).astype(np.float32)
        tdo = to_device(do, dt)
        to = torch.from_numpy(o).cuda()
        delta = torch.full(shape[:-1], float("nan"), device="cuda")
        ra.ra_attn_bwd_delta(tdo, to, delta)
        torch.cuda.synchronize()
        want = obwd.delta(o, do64)
        np.testing.assert_allclose(delta.cpu().numpy(), want, rtol=1e-5, atol=1e-5)


def run_block_bwd(host, o, lse, q_pos, kv_pos, causal, scale):
    q, k, v, do = (to_device(x, "bf16") for x in host)
    b, s_q, n_q, d = q.shape
    s_kv, n_kv = k.shape[1], k.shape[2]
    to = torch.from_numpy(np.ascontiguousarray(o, dtype=np.float32)).cuda()
    tl = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).cuda()
    delta = torch.empty((b, s_q, n_q), device="cuda")
    ra.ra_attn_bwd_delta(do, to, delta)
    dq = torch.zeros((b, s_q, n_q, d), device="cuda")
    dk = torch.zeros((b, s_kv, n_kv, d), device="cuda")
    dv = torch.zeros((b, s_kv, n_kv, d), device="cuda")
    ra.ra_block_attn_bwd(q, k, v, do, tl, delta, dq, dk, dv, causal=causal, scale=scale,
                         q_pos=torch.from_numpy(q_pos).cuda(),
                         kv_pos=torch.from_numpy(kv_pos).cuda())
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


BWD_CASES = [
    # b, s_q, s_kv, n_q, n_kv, causal, score multiplier
    (1, 128, 256, 4, 1, False, 1.0),
    (1, 200, 333, 8, 2, False, 1.0),     # ragged q and kv tails, g = 4
    (2, 77, 130, 8, 4, True, 1.0),       # g = 2, batch 2, random positions
    (1, 300, 500, 3, 3, True, 1.0),      # g = 1
    (1, 96, 64, 12, 4, True, 1.0),       # g = 3
    (1, 257, 640, 8, 1, True, 1.0),      # g = 8, many tiles
    (1, 130, 700, 8, 1, True, 4.0),      # peaked softmax (scores x4)
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_block_bwd_matches_oracle(case):
    b, s_q, s_kv, n_q, n_kv, causal, mult = case
    print(f"block bwd {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(str(case).encode()))
    q, q64 = rand_inputs((b, s_q, n_q, 128), "bf16", rng)
    k, k64 = rand_inputs((b, s_kv, n_kv, 128), "bf16", rng)
    v, v64 = rand_inputs((b, s_kv, n_kv, 128), "bf16", rng)
    do, do64 = rand_inputs((b, s_q, n_q, 128), "bf16", rng)
    span = 2 * (s_q + s_kv) + 1
    q_pos = np.sort(rng.choice(span, s_q, replace=False)).astype(np.int32)
    kv_pos = np.sort(rng.choice(span, s_kv, replace=False)).astype(np.int32)
    scale = np.float32(mult / math.sqrt(128))
    o, lse = oatt.naive_attention(q64, k64, v64, q_pos, kv_pos, causal, scale)
    if causal:
        assert np.isneginf(lse).any() or q_pos[0] >= kv_pos[0]
    dq, dk, dv = run_block_bwd((q, k, v, do), o, lse, q_pos, kv_pos, causal, float(scale))
    rq, rk, rv = obwd.naive_attention_bwd(q64, k64, v64, do64, q_pos, kv_pos, causal, scale)
    for got, want, name in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        err, mag = grad_close(got, want, f"{case} {name}")
        print(f"  {name}: max err {err:.2e} (max |ref| {mag:.2e})")
    # rows with no visible key anywhere contribute nothing and get dq = 0
    empty = np.isneginf(lse)
    if empty.any():
        assert not dq[empty].any()


def test_block_bwd_accumulates():
    """The outputs are added to: two calls give twice one call."""
    rng = np.random.default_rng(7)
    q, q64 = rand_inputs((1, 64, 4, 128), "bf16", rng)
    k, k64 = rand_inputs((1, 96, 2, 128), "bf16", rng)
    v, v64 = rand_inputs((1, 96, 2, 128), "bf16", rng)
    do, do64 = rand_inputs((1, 64, 4, 128), "bf16", rng)
    pos_q = np.arange(32, 96, dtype=np.int32)
    pos_k = np.arange(96, dtype=np.int32)
    o, lse = oatt.naive_attention(q64, k64, v64, pos_q, pos_k, True, 1 / math.sqrt(128))
    tq, tk, tv, tdo = (to_device(x, "bf16") for x in (q, k, v, do))
    tl = torch.from_numpy(lse.astype(np.float32)).cuda()
    delta = torch.empty((1, 64, 4), device="cuda")
    ra.ra_attn_bwd_delta(tdo, torch.from_numpy(o.astype(np.float32)).cuda(), delta)
    outs = [torch.zeros((1, 64, 4, 128), device="cuda"), torch.zeros((1, 96, 2, 128), device="cuda"),
            torch.zeros((1, 96, 2, 128), device="cuda")]
    kw = dict(causal=True, q_pos=torch.from_numpy(pos_q).cuda(), kv_pos=torch.from_numpy(pos_k).cuda())
    ra.ra_block_attn_bwd(tq, tk, tv, tdo, tl, delta, *outs, **kw)
    once = [t.clone() for t in outs]
    ra.ra_block_attn_bwd(tq, tk, tv, tdo, tl, delta, *outs, **kw)
    torch.cuda.synchronize()
    for a, b2 in zip(once, outs):
        assert torch.equal(2 * a, b2)


# (kind, N, S): c = S / N; c = 200 and 150 end in a ragged query block and
# key tile.
RING_CASES = [("contiguous", 2, 768), ("zigzag", 4, 1536), ("striped", 4, 1536),
              ("zigzag", 1, 384), ("contiguous", 4, 1536), ("zigzag", 2, 400),
              ("contiguous", 2, 300)]


@pytest.mark.parametrize("case", RING_CASES, ids=lambda c: "-".join(map(str, c)))
def test_ring_bwd_all_ranks_reassemble_sequence_gradients(case):
    kind, N, S = case
    print(f"ring bwd {case}", flush=True)
    w = synth.Workload("bwd", 1, S, N, kind, 8, 2, 128, "bf16", 1.0, True, seed=60 + N)
    rng = np.random.default_rng(60 + N)
    full = synth.draw(w.with_(N=1, kind="contiguous", rank=0))      # q for every token
    k64, v64 = full.k64, full.v64
    do_bits = synth.bf16_bits(rng.standard_normal(full.q.shape, dtype=np.float32))
    do64 = synth.bf16_to_f32(do_bits).astype(np.float64)
    want = obwd.naive_attention_bwd(full.q64, k64, v64, do64, np.arange(S), np.arange(S), True,
                                    w.scale)
    kc = runner.chunk_kv(runner.host_to_device(full.k, "bf16", "cuda"), kind, N)
    vc = runner.chunk_kv(runner.host_to_device(full.v, "bf16", "cuda"), kind, N)
    dkc = torch.zeros((N,) + tuple(kc.shape[1:]), device="cuda")
    dvc = torch.zeros_like(dkc)
    for rank in range(N):
        pos = opart.partition_map(kind, S, N, rank)
        o, lse = oatt.naive_attention(full.q64[:, pos], k64, v64, pos, np.arange(S), True, w.scale)
        q = runner.host_to_device(full.q[:, pos], "bf16", "cuda")
        do = runner.host_to_device(do_bits[:, pos], "bf16", "cuda")
        desc, _ = ra.ring_desc(b=1, n_q=8, n_kv=2, d=128, dtype=ra.RA_BF16, causal=True, kind=kind,
                               S=S, N=N, rank=rank, scale=float(w.scale))
        ws = torch.empty(ra.ra_ring_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        ws.fill_(0xFF)
        dq = torch.full(q.shape, float("nan"), device="cuda")
        ra.ra_ring_bwd(desc, q, kc, vc, torch.from_numpy(o.astype(np.float32)).cuda(),
                       torch.from_numpy(lse.astype(np.float32)).cuda(), do, dq, dkc, dvc, ws)
        torch.cuda.synchronize()
        grad_close(dq.cpu().numpy(), want[0][:, pos], f"{case} rank {rank} dq")
    dk = np.zeros_like(k64)
    dv = np.zeros_like(v64)
    dkh, dvh = dkc.cpu().numpy(), dvc.cpu().numpy()
    for j in range(N):
        pj = opart.partition_map(kind, S, N, j)
        dk[:, pj] = dkh[j]
        dv[:, pj] = dvh[j]
    grad_close(dk, want[1], f"{case} dk")
    grad_close(dv, want[2], f"{case} dv")


def test_ring_bwd_32k_every_gradient_kind_against_oracle():
    """The ring backward of the 32K Llama-3-8B shard at full size, fed the
    oracle's o and lse of every row (rounded to float32, as the GPU receives
    them): dq on 32 sampled rows x all heads, and this rank's dK, dV
    contribution to 64+ sampled keys (chunk and half boundaries among them) x
    all KV heads, element by element. A key's gradient needs the lse and
    D = dout . o of every query that sees it, hence the full-row forward."""
    w = synth.WORKLOADS["llama3_8b_32k_zigzag"]
    print(f"workload {w.name} backward, oracle o / lse", flush=True)
    inp = synth.draw(w)
    q64, k64, v64 = inp.q64, inp.k64, inp.v64
    ro, rl = oracle_forward_rows(w)
    o32, lse32 = ro.astype(np.float32), rl.astype(np.float32)
    q, kc, vc = runner.ring_inputs(inp.q, inp.k, inp.v, w.dtype, w.kind, w.N, "cuda")
    rng = np.random.default_rng(w.seed + 1000)
    do_bits = synth.bf16_bits(rng.standard_normal(tuple(q.shape), dtype=np.float32))
    do64 = synth.bf16_to_f32(do_bits).astype(np.float64)
    desc, _ = ra.ring_desc(b=w.b, n_q=w.n_q, n_kv=w.n_kv, d=w.d, dtype=ra.RA_BF16,
                           causal=w.causal, kind=w.kind, S=w.S, N=w.N, rank=w.rank,
                           scale=w.scale)
    ws = torch.empty(ra.ra_ring_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    dq = torch.empty(tuple(q.shape), device="cuda")
    dkc = torch.zeros(tuple(kc.shape), device="cuda")
    dvc = torch.zeros_like(dkc)
    ra.ra_ring_bwd(desc, q, kc, vc, torch.from_numpy(o32).cuda(), torch.from_numpy(lse32).cuda(),
                   runner.host_to_device(do_bits, "bf16", "cuda"), dq, dkc, dvc, ws)
    torch.cuda.synchronize()
    dq, dkh, dvh = dq.cpu().numpy(), dkc.cpu().numpy(), dvc.cpu().numpy()
    del q, kc, vc, dkc, dvc, ws
    torch.cuda.empty_cache()
    c = w.c
    q_pos = opart.partition_map(w.kind, w.S, w.N, w.rank)
    rows = synth.sample_rows(c, 32, w.seed, must=[0, c // 2 - 1, c // 2, c - 1])
    rq = obwd.rows_dq(q64[:, rows], k64, v64, do64[:, rows], q_pos[rows], np.arange(w.S),
                      w.causal, w.scale)
    err, m = grad_close(dq[:, rows], rq, "32K dq rows")
    print(f"  dq rows {len(rows)}: max err {err:.2e} (max |ref| {m:.2e})", flush=True)
    keys = sample_keys(w.kind, w.S, w.N, 64, w.seed)
    D = obwd.delta(o32, do64)
    _, rk, rv = obwd.block_attention_bwd(q64, k64[:, keys], v64[:, keys], do64, lse32, D, q_pos,
                                         keys, w.causal, w.scale)
    slots = key_slots(w.kind, w.S, w.N, keys)
    got_k = np.stack([dkh[j][:, a] for j, a in slots], axis=1)
    got_v = np.stack([dvh[j][:, a] for j, a in slots], axis=1)
    for got, want, what in ((got_k, rk, "dk"), (got_v, rv, "dv")):
        err, m = grad_close(got, want, f"32K {what} keys")
        print(f"  {what} keys {len(keys)}: max err {err:.2e} (max |ref| {m:.2e})", flush=True)


@pytest.mark.parametrize("name", ["llama3_70b_128k_zigzag"])
def test_full_workload_bwd_sampled_rows_and_invariant(name):
    """The 128K ring backward at full size in the benchmark's configuration
    (the oracle cannot afford the lse of every row here): dq on 32 sampled
    rows x all heads against the oracle (a row's dq depends on that row only);
    sum_j dk_j = 0 over the rank's whole contribution to every block (each
    query's dx sums to zero over its visible keys); and sum_j dv_j equals the
    sum of dout over the queries of each KV head's group (each query's
    probabilities sum to one over its visible keys)."""
    w = synth.WORKLOADS[name]
    print(f"workload {w.name} backward", flush=True)
    inp = synth.draw(w)
    q, kc, vc = runner.ring_inputs(inp.q, inp.k, inp.v, w.dtype, w.kind, w.N, "cuda")
    call = runner.RingCall(q, kc, vc, kind=w.kind, S=w.S, N=w.N, rank=w.rank, causal=w.causal,
                           scale=w.scale)
    o, lse = call()
    rng = np.random.default_rng(w.seed + 1000)
    do_bits = synth.bf16_bits(rng.standard_normal(tuple(q.shape), dtype=np.float32))
    desc, _ = ra.ring_desc(b=w.b, n_q=w.n_q, n_kv=w.n_kv, d=w.d, dtype=ra.RA_BF16,
                           causal=w.causal, kind=w.kind, S=w.S, N=w.N, rank=w.rank,
                           scale=w.scale)
    ws = torch.empty(ra.ra_ring_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    dq = torch.empty(tuple(q.shape), device="cuda")
    dkc = torch.zeros(tuple(kc.shape), device="cuda")
    dvc = torch.zeros_like(dkc)
    ra.ra_ring_bwd(desc, q, kc, vc, o, lse, runner.host_to_device(do_bits, "bf16", "cuda"), dq,
                   dkc, dvc, ws)
    torch.cuda.synchronize()
    dq = dq.cpu().numpy()
    dk = dkc.cpu().numpy().astype(np.float64)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and torch.isfinite(dvc).all()
    dv_tot = dvc.sum(dim=(0, 1, 2)).double().cpu().numpy()       # [n_kv, d]
    del call, q, kc, vc, dkc, dvc, ws
    torch.cuda.empty_cache()
    tot = dk.sum(axis=(0, 1, 2))          # [n_kv, d]: every block, batch and key
    mag = np.abs(dk).sum(axis=(0, 1, 2))
    assert np.max(np.abs(tot) / mag) < 1e-3, np.max(np.abs(tot) / mag)
    do_grp = synth.bf16_to_f32(do_bits).astype(np.float64).sum(axis=(0, 1))     # [n_q, d]
    want_dv = do_grp.reshape(w.n_kv, w.n_q // w.n_kv, w.d).sum(axis=1)
    err_dv = float(np.max(np.abs(dv_tot - want_dv)))
    assert err_dv <= 1e-2 * float(np.max(np.abs(want_dv))), (err_dv, np.max(np.abs(want_dv)))
    c = w.c
    rows = synth.sample_rows(c, 32, w.seed, must=[0, c // 2 - 1, c // 2, c - 1])
    q_pos = opart.partition_map(w.kind, w.S, w.N, w.rank)
    do64 = synth.bf16_to_f32(do_bits).astype(np.float64)
    rq = obwd.rows_dq(inp.q64[:, rows], inp.k64, inp.v64, do64[:, rows], q_pos[rows],
                      np.arange(w.S), w.causal, w.scale)
    err, m = grad_close(dq[:, rows], rq, f"{name} dq rows")
    print(f"  dq rows {len(rows)}: max err {err:.2e} (max |ref| {m:.2e}); "
          f"max |sum dk| / sum |dk| {np.max(np.abs(tot) / mag):.2e}; "
          f"max |sum dv - sum dout| {err_dv:.2e} (max {np.max(np.abs(want_dv)):.2e})", flush=True)


def test_ring_bwd_128k_sampled_keys_against_oracle():
    """The 128K ring backward at full size, element by element on this rank's
    dK, dV contribution to 64+ sampled keys (chunk and half boundaries among
    them) x all KV heads (dq rows at this size are checked above, against the
    oracle's own forward).

    The backward is a function of (q, k, v, dout, o, lse); the oracle cannot
    afford the 128K forward of every row, so both sides get the same seeded
    o ~ N(0, 0.05^2) and lse = ln(pos + 1) + 1/2 (the expected log-sum-exp of
    pos + 1 unit-variance scores; any finite lse is a valid input) instead of
    the forward's. A key's gradient then needs only that lse and D = dout . o
    of every query that sees it."""
    w = synth.WORKLOADS["llama3_70b_128k_zigzag"]
    print(f"workload {w.name} backward, seeded o / lse, sampled keys", flush=True)
    inp = synth.draw(w)
    q_pos = opart.partition_map(w.kind, w.S, w.N, w.rank)
    rng = np.random.default_rng(w.seed + 2000)
    o32 = (0.05 * rng.standard_normal((w.b, w.c, w.n_q, w.d))).astype(np.float32)
    lse32 = np.broadcast_to((np.log(q_pos + 1.0) + 0.5)[None, :, None],
                            (w.b, w.c, w.n_q)).astype(np.float32)
    rng = np.random.default_rng(w.seed + 1000)
    do_bits = synth.bf16_bits(rng.standard_normal((w.b, w.c, w.n_q, w.d), dtype=np.float32))
    q, kc, vc = runner.ring_inputs(inp.q, inp.k, inp.v, w.dtype, w.kind, w.N, "cuda")
    desc, _ = ra.ring_desc(b=w.b, n_q=w.n_q, n_kv=w.n_kv, d=w.d, dtype=ra.RA_BF16,
                           causal=w.causal, kind=w.kind, S=w.S, N=w.N, rank=w.rank,
                           scale=w.scale)
    ws = torch.empty(ra.ra_ring_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    dq = torch.empty(tuple(q.shape), device="cuda")
    dkc = torch.zeros(tuple(kc.shape), device="cuda")
    dvc = torch.zeros_like(dkc)
    ra.ra_ring_bwd(desc, q, kc, vc, torch.from_numpy(o32).cuda(),
                   torch.from_numpy(np.ascontiguousarray(lse32)).cuda(),
                   runner.host_to_device(do_bits, "bf16", "cuda"), dq, dkc, dvc, ws)
    torch.cuda.synchronize()
    keys = sample_keys(w.kind, w.S, w.N, 64, w.seed)
    slots = key_slots(w.kind, w.S, w.N, keys)
    got_k = torch.stack([dkc[j][:, a] for j, a in slots], dim=1).cpu().numpy()
    got_v = torch.stack([dvc[j][:, a] for j, a in slots], dim=1).cpu().numpy()
    del q, kc, vc, dkc, dvc, ws
    torch.cuda.empty_cache()
    q64, k64, v64 = inp.q64, inp.k64, inp.v64
    do64 = synth.bf16_to_f32(do_bits).astype(np.float64)
    D = obwd.delta(o32, do64)
    _, rk, rv = obwd.block_attention_bwd(q64, k64[:, keys], v64[:, keys], do64, lse32, D, q_pos,
                                         keys, w.causal, w.scale)
    for got, want, what in ((got_k, rk, "dk"), (got_v, rv, "dv")):
        err, m = grad_close(got, want, f"128K {what} keys")
        print(f"  {what} keys {len(keys)}: max err {err:.2e} (max |ref| {m:.2e})", flush=True)


def test_block_bwd_offsets_past_2gib():
    """ra_block_attn_bwd over one (batch, kv head) of 8,388,672 keys, K and V
    past 2 GiB each (every K / V tile of the dq kernel through a descriptor of
    its own), with 40 causal queries near the end of the block: dq of every
    row and dK, dV of 64+ sampled keys (the last ones among them) against the
    oracle, fed the oracle's o and lse (rounded to float32). K and V hold
    seeded bf16 bit patterns of random sign, exponent and mantissa in
    +-[0.5, 2) (2^31 normal draws would take the host a minute)."""
    n = 2**23 + 64
    print(f"block backward, {n} keys (2.1 GB K, V)", flush=True)
    rng = np.random.default_rng(2**23 + 1)
    q, q64 = rand_inputs((1, 40, 1, 128), "bf16", rng)
    do, do64 = rand_inputs((1, 40, 1, 128), "bf16", rng)

    def bits():
        r = rng.integers(0, 1 << 16, size=(1, n, 1, 128), dtype=np.uint16)
        return (r & np.uint16(0x80FF)) | np.uint16(0x3F00)   # sign, exponent 126 or 127

    k, v = bits(), bits()
    k64 = synth.bf16_to_f32(k).astype(np.float64)
    v64 = synth.bf16_to_f32(v).astype(np.float64)
    q_pos = np.arange(n - 100, n - 60, dtype=np.int32)
    kv_pos = np.arange(n, dtype=np.int32)
    scale = 1 / math.sqrt(128)
    o, lse = oatt.naive_attention(q64, k64, v64, q_pos, kv_pos, True, scale)
    o32, lse32 = o.astype(np.float32), lse.astype(np.float32)
    tk, tv = to_device(k, "bf16"), to_device(v, "bf16")
    del k, v
    tdo = to_device(do, "bf16")
    delta = torch.empty((1, 40, 1), device="cuda")
    ra.ra_attn_bwd_delta(tdo, torch.from_numpy(o32).cuda(), delta)
    dq = torch.zeros((1, 40, 1, 128), device="cuda")
    dk = torch.zeros((1, n, 1, 128), device="cuda")
    dv = torch.zeros_like(dk)
    ra.ra_block_attn_bwd(to_device(q, "bf16"), tk, tv, tdo, torch.from_numpy(lse32).cuda(), delta,
                         dq, dk, dv, causal=True, q_pos=torch.from_numpy(q_pos).cuda(),
                         kv_pos=torch.from_numpy(kv_pos).cuda())
    torch.cuda.synchronize()
    keys = np.unique(np.concatenate([np.arange(n - 130, n, 8), np.arange(n - 100, n - 58),
                                     rng.integers(0, n, 16)]))
    idx = torch.from_numpy(keys).cuda()
    got_k = dk[:, idx].cpu().numpy()
    got_v = dv[:, idx].cpu().numpy()
    got_q = dq.cpu().numpy()
    del tk, tv, dk, dv, idx
    torch.cuda.empty_cache()
    rq = obwd.rows_dq(q64, k64, v64, do64, q_pos, kv_pos, True, scale)
    D = obwd.delta(o32, do64)
    _, rk, rv = obwd.block_attention_bwd(q64, k64[:, keys], v64[:, keys], do64, lse32, D, q_pos,
                                         keys, True, scale)
    # Each query spreads its weight over ~2^23 keys, so the gradients are tiny
    # (|dk| ~ 1e-5): compared relative to their largest magnitude, without the
    # absolute floor of grad_close.
    for got, want, what in ((got_q, rq, "dq"), (got_k, rk, "dk"), (got_v, rv, "dv")):
        err = float(np.max(np.abs(got - want)))
        m = float(np.max(np.abs(want)))
        assert m > 0 and err <= TOL_REL * m, f"{what}: max err {err:.3g} vs max |ref| {m:.3g}"
        print(f"  {what}: max err {err:.2e} (max |ref| {m:.2e})", flush=True)
    late = keys > q_pos[-1]            # keys after every query: no gradient at all
    assert late.any() and not got_k[:, late].any() and not got_v[:, late].any()


def test_ring_batched_forward_and_backward():
    """b = 2 through ra_ring_fwd and every rank's ra_ring_bwd (the [N, b, c, ...]
    chunk layout and the per-batch rows of every step), against naive attention
    and its backward over the whole sequence."""
    kind, N, S, b = "zigzag", 4, 1536, 2
    print(f"ring batched b={b} {kind} N={N} S={S}", flush=True)
    w = synth.Workload("bwd_b2", b, S, N, kind, 8, 2, 128, "bf16", 1.0, True, seed=77)
    rng = np.random.default_rng(77)
    full = synth.draw(w.with_(N=1, kind="contiguous", rank=0))      # q for every token
    k64, v64 = full.k64, full.v64
    assert full.q.shape[0] == b
    do_bits = synth.bf16_bits(rng.standard_normal(full.q.shape, dtype=np.float32))
    do64 = synth.bf16_to_f32(do_bits).astype(np.float64)
    want = obwd.naive_attention_bwd(full.q64, k64, v64, do64, np.arange(S), np.arange(S), True,
                                    w.scale)
    kc = runner.chunk_kv(runner.host_to_device(full.k, "bf16", "cuda"), kind, N)
    vc = runner.chunk_kv(runner.host_to_device(full.v, "bf16", "cuda"), kind, N)
    dkc = torch.zeros((N,) + tuple(kc.shape[1:]), device="cuda")
    dvc = torch.zeros_like(dkc)
    for rank in range(N):
        pos = opart.partition_map(kind, S, N, rank)
        o, lse = oatt.naive_attention(full.q64[:, pos], k64, v64, pos, np.arange(S), True, w.scale)
        q = runner.host_to_device(full.q[:, pos], "bf16", "cuda")
        if rank == 1:   # the forward of one rank, all steps
            call = runner.RingCall(q, kc, vc, kind=kind, S=S, N=N, rank=rank, causal=True,
                                   scale=float(w.scale))
            go, gl = call()
            torch.cuda.synchronize()
            assert np.abs(go.cpu().numpy() - o).max() <= 1e-2
            assert np.abs(gl.cpu().numpy() - lse).max() <= 2e-3
        do = runner.host_to_device(do_bits[:, pos], "bf16", "cuda")
        desc, _ = ra.ring_desc(b=b, n_q=8, n_kv=2, d=128, dtype=ra.RA_BF16, causal=True, kind=kind,
                               S=S, N=N, rank=rank, scale=float(w.scale))
        ws = torch.empty(ra.ra_ring_bwd_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        ws.fill_(0xFF)
        dq = torch.full(q.shape, float("nan"), device="cuda")
        ra.ra_ring_bwd(desc, q, kc, vc, torch.from_numpy(o.astype(np.float32)).cuda(),
                       torch.from_numpy(lse.astype(np.float32)).cuda(), do, dq, dkc, dvc, ws)
        torch.cuda.synchronize()
        grad_close(dq.cpu().numpy(), want[0][:, pos], f"b2 rank {rank} dq")
    dk = np.zeros_like(k64)
    dv = np.zeros_like(v64)
    dkh, dvh = dkc.cpu().numpy(), dvc.cpu().numpy()
    for j in range(N):
        pj = opart.partition_map(kind, S, N, j)
        dk[:, pj] = dkh[j]
        dv[:, pj] = dvh[j]
    grad_close(dk, want[1], "b2 dk")
    grad_close(dv, want[2], "b2 dv")


def test_ring_bwd_transfer_overlap_equals_serialized_bitwise():
    """The travelling block's receives and sends on a second stream (overlapped
    with the kernels) against the same copies on the compute stream: any
    difference would be a race between a transfer and a kernel. Slots start
    from nonzero "earlier ranks'" values and the workspace is NaN-poisoned;
    both maps that skip (contiguous) and that do not (zig-zag) are run."""
    for kind, rank in (("zigzag", 1), ("contiguous", 1)):
        N, S, n_q, n_kv = 4, 4096, 8, 2
        print(f"ring bwd transfer {kind} N={N} rank={rank}", flush=True)
        rng = np.random.default_rng(91)
        c = S // N
        q, _ = rand_inputs((1, c, n_q, 128), "bf16", rng)
        k, _ = rand_inputs((1, S, n_kv, 128), "bf16", rng)
        v, _ = rand_inputs((1, S, n_kv, 128), "bf16", rng)
        do, _ = rand_inputs((1, c, n_q, 128), "bf16", rng)
        tq, tdo = to_device(q, "bf16"), to_device(do, "bf16")
        kc = runner.chunk_kv(to_device(k, "bf16"), kind, N)
        vc = runner.chunk_kv(to_device(v, "bf16"), kind, N)
        call = runner.RingCall(tq, kc, vc, kind=kind, S=S, N=N, rank=rank, causal=True)
        o, lse = call()
        dk0 = torch.from_numpy(rng.standard_normal((N, 1, c, n_kv, 128)).astype(np.float32)).cuda()
        dv0 = torch.from_numpy(rng.standard_normal((N, 1, c, n_kv, 128)).astype(np.float32)).cuda()
        outs = []
        for serialize in (False, True):
            desc, _ = ra.ring_desc(b=1, n_q=n_q, n_kv=n_kv, d=128, dtype=ra.RA_BF16, causal=True,
                                   kind=kind, S=S, N=N, rank=rank,
                                   flags=ra.RA_RING_SERIALIZE if serialize else 0)
            ws = torch.full((ra.ra_ring_bwd_workspace_bytes(desc),), 0xFF, dtype=torch.uint8,
                            device="cuda")
            dq = torch.full(tuple(tq.shape), float("nan"), device="cuda")
            dkc, dvc = dk0.clone(), dv0.clone()
            ra.ra_ring_bwd(desc, tq, kc, vc, o, lse, tdo, dq, dkc, dvc, ws)
            torch.cuda.synchronize()
            outs.append((dq.cpu().numpy(), dkc.cpu().numpy(), dvc.cpu().numpy()))
        for a_, b_, what in zip(outs[0], outs[1], ("dq", "dk", "dv")):
            assert not np.isnan(a_).any(), (kind, what)
            assert np.array_equal(a_, b_), (kind, what)
        # the chunks this rank cannot see (contiguous: later ranks) are passed on unchanged
        for j in range(N):
            if j > rank and kind == "contiguous":
                assert np.array_equal(outs[0][1][j], dk0[j].cpu().numpy())
                assert np.array_equal(outs[0][2][j], dv0[j].cpu().numpy())
