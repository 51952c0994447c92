"""GPU parity of ra_lse_merge and ra_block_attn_fwd against the CPU oracle,
through the C ABI, on seeded inputs spanning several tiles, ragged tails,
GQA groupings, causal positions and the degenerate cases (empty blocks,
queries with no visible key)."""

import math
import zlib

import numpy as np
import pytest
import torch

import ring_attention_context_amd as ra
import synth
from gpu_util import TOL_O, compare, rand_inputs, require_gpu, to_device
from oracle import attention as oatt
from oracle import partition as opart

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _merge_case(rows, d, seed):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((rows, d)).astype(np.float32)
    ob = rng.standard_normal((rows, d)).astype(np.float32)
    lse = rng.uniform(-20, 20, rows).astype(np.float32)
    lseb = rng.uniform(-20, 20, rows).astype(np.float32)
    # stress rows: -inf on either side or both, |lse| = 80, equal values
    k = rows // 8
    lse[:k] = -np.inf
    lseb[k:2 * k] = -np.inf
    lse[2 * k:3 * k] = -np.inf
    lseb[2 * k:3 * k] = -np.inf
    o[2 * k:3 * k] = 0.0      # the identity carries o = 0
    ob[2 * k:3 * k] = 0.0
    lse[3 * k:4 * k] = 80.0
    lseb[3 * k:4 * k] = -80.0
    lse[4 * k:5 * k] = lseb[4 * k:5 * k]
    return o, lse, ob, lseb


@pytest.mark.parametrize("rows,d", [(1, 128), (1000, 128), (4099, 64), (64, 4), (33, 8),
                                    (5, 16), (777, 256)])
def test_lse_merge_matches_oracle(rows, d):
    o, lse, ob, lseb = _merge_case(rows, d, seed=rows + d)
    print(f"merge rows={rows} d={d}", flush=True)
    to, tl = torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda()
    ra.ra_lse_merge(to, tl, torch.from_numpy(ob).cuda(), torch.from_numpy(lseb).cuda())
    torch.cuda.synchronize()
    ro, rl = oatt.merge(o.astype(np.float64), lse.astype(np.float64), ob.astype(np.float64),
                        lseb.astype(np.float64))
    compare(to.cpu().numpy(), tl.cpu().numpy(), ro, rl, "f32", "merge")


def _block_case(dtype, b, s_q, s_kv, n_q, n_kv, d, causal, seed, pos=None):
    rng = np.random.default_rng(seed)
    q, q64 = rand_inputs((b, s_q, n_q, d), dtype, rng)
    k, k64 = rand_inputs((b, s_kv, n_kv, d), dtype, rng)
    v, v64 = rand_inputs((b, s_kv, n_kv, d), dtype, rng)
    if pos is None:
        span = 2 * (s_q + s_kv) + 1
        q_pos = np.sort(rng.choice(span, s_q, replace=False)).astype(np.int32)
        kv_pos = np.sort(rng.choice(span, s_kv, replace=False)).astype(np.int32)
    else:
        q_pos, kv_pos = pos
    return (q, k, v), (q64, k64, v64), q_pos, kv_pos


def _run_block(dtype, host, q_pos, kv_pos, causal, scale):
    q, k, v = (to_device(x, dtype) for x in host)
    b, s_q, n_q, d = q.shape
    o = torch.full((b, s_q, n_q, d), float("nan"), device="cuda")
    lse = torch.full((b, s_q, n_q), float("nan"), device="cuda")
    qp = torch.from_numpy(q_pos).cuda()
    kp = torch.from_numpy(kv_pos).cuda()
    ra.ra_block_attn_fwd(q, k, v, o, lse, causal=causal, scale=scale, q_pos=qp, kv_pos=kp)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


BLOCK_CASES = [
    # dtype, b, s_q, s_kv, n_q, n_kv, d, causal
    ("bf16", 1, 128, 256, 4, 1, 128, False),     # whole tiles
    ("bf16", 1, 200, 333, 8, 2, 128, False),     # ragged q and kv tails, g = 4
    ("bf16", 2, 77, 130, 8, 4, 128, True),       # g = 2, batch 2, random positions
    ("bf16", 1, 300, 500, 3, 3, 128, True),      # g = 1
    ("bf16", 1, 96, 64, 12, 4, 128, True),       # g = 3
    ("bf16", 1, 257, 1000, 8, 1, 128, True),     # g = 8, many tiles
    ("f32", 1, 64, 64, 1, 1, 64, False),
    ("f32", 1, 100, 77, 4, 2, 64, True),
    ("f32", 2, 45, 130, 2, 1, 128, True),
    ("f32", 1, 33, 300, 6, 3, 128, False),
]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=lambda c: "-".join(map(str, c)))
def test_block_attn_matches_oracle(case):
    dtype, b, s_q, s_kv, n_q, n_kv, d, causal = case
    print(f"block {case}", flush=True)
    host, wide, q_pos, kv_pos = _block_case(dtype, b, s_q, s_kv, n_q, n_kv, d, causal,
                                            seed=zlib.crc32(str(case).encode()))
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_block(dtype, host, q_pos, kv_pos, causal, 0.0)
    ro, rl = oatt.naive_attention(*wide, q_pos, kv_pos, causal, scale)
    compare(o, lse, ro, rl, dtype, str(case))
    if causal:
        assert np.isneginf(rl).any() or q_pos[0] >= kv_pos[0]


def test_block_attn_per_row_statistics_match_block_oracle():
    """Small case against the oracle's explicit per-block statistics (m_b, l_b, o_b, lse_b)."""
    host, wide, q_pos, kv_pos = _block_case("bf16", 1, 40, 90, 4, 2, 128, True, seed=5)
    o, lse = _run_block("bf16", host, q_pos, kv_pos, True, 0.3)
    ro, rl = oatt.block_attention(*wide, q_pos, kv_pos, True, np.float32(0.3))
    compare(o, lse, ro, rl, "bf16", "block stats")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_attn_zigzag_steps(dtype):
    """Every (rank, step) block of a zig-zag ring: full, diagonal and empty steps."""
    S, N = 512, 4
    d = 128
    rng = np.random.default_rng(9)
    for rank in (0, N - 1):
        q_pos = opart.partition_map("zigzag", S, N, rank).astype(np.int32)
        q, q64 = rand_inputs((1, len(q_pos), 8, d), dtype, rng)
        for src in opart.ring_sources(rank, N):
            kv_pos = opart.partition_map("zigzag", S, N, src).astype(np.int32)
            k, k64 = rand_inputs((1, len(kv_pos), 2, d), dtype, rng)
            v, v64 = rand_inputs((1, len(kv_pos), 2, d), dtype, rng)
            o, lse = _run_block(dtype, (q, k, v), q_pos, kv_pos, True, 0.0)
            ro, rl = oatt.naive_attention(q64, k64, v64, q_pos, kv_pos, True, 1 / math.sqrt(d))
            compare(o, lse, ro, rl, dtype, f"zigzag rank {rank} src {src}")


def test_block_attn_empty_key_block():
    """s_kv = 0: every row is the merge identity (0, -inf)."""
    q = torch.randn(1, 70, 4, 128, device="cuda").to(torch.bfloat16)
    k = torch.empty(1, 0, 2, 128, device="cuda", dtype=torch.bfloat16)
    o = torch.full((1, 70, 4, 128), 5.0, device="cuda")
    lse = torch.zeros(1, 70, 4, device="cuda")
    qp = torch.arange(70, dtype=torch.int32, device="cuda")
    ra.ra_block_attn_fwd(q, k, k, o, lse, causal=True, q_pos=qp,
                         kv_pos=torch.empty(0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_block_attn_all_keys_in_future():
    """Causal block entirely after the queries: no key visible anywhere."""
    rng = np.random.default_rng(3)
    q, _ = rand_inputs((1, 64, 4, 128), "bf16", rng)
    k, _ = rand_inputs((1, 130, 1, 128), "bf16", rng)
    v, _ = rand_inputs((1, 130, 1, 128), "bf16", rng)
    o, lse = _run_block("bf16", (q, k, v), np.arange(64, dtype=np.int32),
                        np.arange(1000, 1130, dtype=np.int32), True, 0.0)
    assert np.all(np.isneginf(lse)) and not o.any()


def test_block_attn_large_scores_stay_finite():
    """Scores scaled x4 with peaky softmax: exponentials must not overflow."""
    host, wide, q_pos, kv_pos = _block_case("bf16", 1, 130, 700, 8, 1, 128, True, seed=21)
    scale = 4.0 / math.sqrt(128)
    o, lse = _run_block("bf16", host, q_pos, kv_pos, True, scale)
    ro, rl = oatt.naive_attention(*wide, q_pos, kv_pos, True, np.float32(scale))
    compare(o, lse, ro, rl, "bf16", "x4 scores")


def test_block_attn_offsets_past_2gib():
    """Key blocks whose K and V span more than 2^31 bytes: every tile is then
    read through a descriptor of its own (the far path), with one (batch, kv
    head) of 8,388,672 keys (2.1 GB per tensor): row-major V at that length
    with causal queries near the end of the block (positions and diagonal
    tiles at the far end), and V^T at the longest length the transposed
    layout accepts (8,388,544 keys: its d rows of one head still fit 31-bit
    offsets) with non-causal ones. K and V hold seeded bf16 values of random sign,
    exponent and mantissa in +-[0.5, 2) (drawn as bit patterns: 2^31 normal
    draws would take a minute on the host), every key different, so a read
    from the wrong place or a zero-filled one moves the result."""
    n = 2**23 + 64
    n_vt = 2**23 - 64
    print(f"block attention, {n} keys (2.1 GB K, V)", flush=True)
    rng = np.random.default_rng(2**23)
    q, q64 = rand_inputs((1, 40, 1, 128), "bf16", rng)

    def bits():
        r = rng.integers(0, 1 << 16, size=(1, n, 1, 128), dtype=np.uint16)
        return (r & np.uint16(0x80FF)) | np.uint16(0x3F00)   # sign, exponent 126 or 127

    k, v = bits(), bits()
    tq = to_device(q, "bf16")
    tk = to_device(k, "bf16")
    tv = to_device(v, "bf16")
    cases = []
    for s_kv, vt, causal in ((n, False, True), (n_vt, True, False)):
        kv_pos = np.arange(s_kv, dtype=np.int32)
        q_pos = np.arange(s_kv - 100, s_kv - 60, dtype=np.int32)
        ks, vs = tk[:, :s_kv], tv[:, :s_kv]
        if vt:
            vs = torch.empty((1, 1, 128, s_kv), dtype=torch.bfloat16, device="cuda")
            ra.ra_v_transpose(tv[:, :s_kv].contiguous(), vs)
        o = torch.full((1, 40, 1, 128), float("nan"), device="cuda")
        lse = torch.full((1, 40, 1), float("nan"), device="cuda")
        ra.ra_block_attn_fwd(tq, ks, vs, o, lse, causal=causal,
                             q_pos=torch.from_numpy(q_pos).cuda(),
                             kv_pos=torch.from_numpy(kv_pos).cuda(), v_transposed=vt)
        torch.cuda.synchronize()
        cases.append((s_kv, vt, causal, q_pos, o.cpu().numpy(), lse.cpu().numpy()))
        del vs
    del tk, tv
    torch.cuda.empty_cache()
    k64 = synth.bf16_to_f32(k).astype(np.float64)
    del k
    v64 = synth.bf16_to_f32(v).astype(np.float64)
    del v
    for s_kv, vt, causal, q_pos, o, lse in cases:
        ro, rl = oatt.naive_attention(q64, k64[:, :s_kv], v64[:, :s_kv], q_pos,
                                      np.arange(s_kv), causal, 1 / math.sqrt(128))
        do, dl = compare(o, lse, ro, rl, "bf16", f"{s_kv} keys vt={vt} causal={causal}")
        print(f"  {s_kv} keys vt={vt} causal={causal}: max|dO| {do:.2e} max|dlse| {dl:.2e}",
              flush=True)
