"""GPU parity of the transposed-V path: ra_v_transpose moves every element bit
for bit, ra_block_attn_fwd with RA_V_TRANSPOSED matches the CPU oracle, and
both V layouts survive score ranges that force the kernel's lazy reference
update and its overflow fallback (a tile redone against its true row max)."""

import math
import zlib

import numpy as np
import pytest
import torch

import ring_attention_context_amd as ra
from gpu_util import compare, rand_inputs, require_gpu, to_device
from oracle import attention as oatt

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("shape,dtype", [
    ((1, 1000, 2, 128), torch.bfloat16),   # ragged token tail
    ((2, 64, 3, 128), torch.bfloat16),
    ((2, 200, 3, 72), torch.bfloat16),     # ragged channel tile (16-byte path)
    ((1, 77, 2, 64), torch.bfloat16),      # s % 8 != 0: element-wise path
    ((1, 77, 5, 72), torch.float32),       # ragged channel tile
    ((3, 130, 1, 64), torch.float32),
])
def test_v_transpose_bit_exact(shape, dtype):
    print(f"v_transpose {shape} {dtype}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(zlib.crc32(str(shape).encode()))
    v = torch.randn(shape, generator=g).to(dtype).cuda()
    b, s, h, d = shape
    vt = torch.full((b, h, d, s), float("nan"), dtype=dtype, device="cuda")
    ra.ra_v_transpose(v, vt)
    torch.cuda.synchronize()
    want = v.permute(0, 2, 3, 1).contiguous()
    assert torch.equal(vt.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       want.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))


def _run(host, q_pos, kv_pos, causal, scale, v_transposed):
    q, k, v = (to_device(x, "bf16") for x in host)
    b, s_q, n_q, d = q.shape
    if v_transposed:
        vt = torch.empty((b, v.shape[2], d, v.shape[1]), dtype=v.dtype, device="cuda")
        ra.ra_v_transpose(v, vt)
        v = vt
    o = torch.full((b, s_q, n_q, d), float("nan"), device="cuda")
    lse = torch.full((b, s_q, n_q), float("nan"), device="cuda")
    ra.ra_block_attn_fwd(q, k, v, o, lse, causal=causal, scale=scale,
                         q_pos=torch.from_numpy(q_pos).cuda(),
                         kv_pos=torch.from_numpy(kv_pos).cuda(), v_transposed=v_transposed)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


VT_CASES = [
    # b, s_q, s_kv, n_q, n_kv, causal   (s_kv % 8 == 0 for the V^T layout)
    (1, 128, 256, 4, 1, False),
    (1, 200, 328, 8, 2, False),     # ragged q tail, ragged last key tile
    (2, 77, 136, 8, 4, True),       # g = 2, batch 2
    (1, 300, 504, 3, 3, True),      # g = 1
    (1, 96, 64, 12, 4, True),       # g = 3
    (1, 257, 1000, 8, 1, True),     # g = 8, many tiles
]


@pytest.mark.parametrize("case", VT_CASES, ids=lambda c: "-".join(map(str, c)))
def test_block_attn_transposed_v_matches_oracle(case):
    b, s_q, s_kv, n_q, n_kv, causal = case
    print(f"block V^T {case}", flush=True)
    rng = np.random.default_rng(zlib.crc32(str(case).encode()))
    q, q64 = rand_inputs((b, s_q, n_q, 128), "bf16", rng)
    k, k64 = rand_inputs((b, s_kv, n_kv, 128), "bf16", rng)
    v, v64 = rand_inputs((b, s_kv, n_kv, 128), "bf16", rng)
    span = 2 * (s_q + s_kv) + 1
    q_pos = np.sort(rng.choice(span, s_q, replace=False)).astype(np.int32)
    kv_pos = np.sort(rng.choice(span, s_kv, replace=False)).astype(np.int32)
    o, lse = _run((q, k, v), q_pos, kv_pos, causal, 0.0, True)
    ro, rl = oatt.naive_attention(q64, k64, v64, q_pos, kv_pos, causal, 1 / math.sqrt(128))
    compare(o, lse, ro, rl, "bf16", f"V^T {case}")


def _ramp_case(seed, s_q, s_kv, jump):
    """Keys whose scale grows along the block: early tiles small, later tiles large.
    `jump`=True makes one step so large that a tile's sum exceeds 2^32 against the
    reference of the earlier tiles (the fallback path); otherwise the growth is
    gradual (the lazy reference update)."""
    rng = np.random.default_rng(seed)
    q, q64 = rand_inputs((1, s_q, 4, 128), "bf16", rng)
    if jump:
        mult = np.where(np.arange(s_kv) < 128, 0.05, 12.0).astype(np.float32)
    else:
        mult = np.linspace(0.05, 6.0, s_kv).astype(np.float32)
    kf = rng.standard_normal((1, s_kv, 1, 128), dtype=np.float32) * mult[None, :, None, None]
    import synth
    k = synth.bf16_bits(kf.astype(np.float32))
    k64 = synth.bf16_to_f32(k).astype(np.float64)
    v, v64 = rand_inputs((1, s_kv, 1, 128), "bf16", rng)
    return (q, k, v), (q64, k64, v64)


@pytest.mark.parametrize("jump", [False, True], ids=["gradual", "jump"])
@pytest.mark.parametrize("v_transposed", [False, True], ids=["v_rows", "v_t"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_block_attn_reference_updates(jump, v_transposed, causal):
    s_q, s_kv = 160, 640
    print(f"ramp jump={jump} vt={v_transposed} causal={causal}", flush=True)
    host, wide = _ramp_case(31 + 2 * jump + causal, s_q, s_kv, jump)
    # causal: queries at the end of the key range see every key up to themselves
    kv_pos = np.arange(s_kv, dtype=np.int32)
    q_pos = np.arange(s_kv - s_q, s_kv, dtype=np.int32)
    scale = 1.0 / math.sqrt(128)
    o, lse = _run(host, q_pos, kv_pos, causal, scale, v_transposed)
    ro, rl = oatt.naive_attention(*wide, q_pos, kv_pos, causal, np.float32(scale))
    # the row max moves far above the first tile's: the test is meaningful only if so
    assert np.max(rl) > 20.0
    compare(o, lse, ro, rl, "bf16", f"ramp jump={jump} vt={v_transposed} causal={causal}")
