"""The C-ABI library on the host: it loads without a GPU, exports every
symbol include/ringattn.h declares, ra_partition is bit-exact against the
oracle's maps, and argument errors are reported before any HIP call."""

import ctypes
import os
import re

import numpy as np
import pytest

import ring_attention_context_amd as ra
from ring_attention_context_amd import _lib
from oracle import partition as opart

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ringattn.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = ra.load_library()
    declared = header_functions()
    assert set(declared) == set(ra.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    # also visible to the dynamic linker as C symbols (no C++ mangling)
    handle = ctypes.CDLL(ra.LIB_PATH)
    for name in declared:
        assert ctypes.cast(getattr(handle, name), ctypes.c_void_p).value


def test_struct_layouts_match_header():
    # ra_attn_desc: 4 int32, 2 int64, 2 int32, float, int32, 3 pointers
    assert ctypes.sizeof(_lib.AttnDesc) == 16 + 16 + 8 + 8 + 24
    assert _lib.AttnDesc.q_pos.offset == 48 and _lib.AttnDesc.q_doc_start.offset == 64
    # ra_ring_desc: 8 x 4-byte fields, int64 S, 4 int32, 2 pointers
    assert _lib.RingDesc.S.offset == 32 and _lib.RingDesc.step_events.offset == 56
    assert _lib.RingDesc.doc_start.offset == 64
    assert ctypes.sizeof(_lib.RingDesc) == 72


@pytest.mark.parametrize("kind", opart.KINDS)
def test_partition_bit_exact_vs_oracle(kind):
    for N in (1, 2, 3, 4, 8, 32):
        for S in (0, 2 * N, 64 * N, 2 * N * 37):
            for rank in sorted({0, N // 2, N - 1}):
                got = ra.ra_partition(kind, S, N, rank)
                want = opart.partition_map(kind, S, N, rank)
                assert got.dtype == np.int32
                assert np.array_equal(got, want), (kind, S, N, rank)


def test_partition_bit_exact_at_workload_sizes():
    import synth
    for w in synth.WORKLOADS.values():
        for rank in sorted({0, w.N // 2, w.N - 1}):
            assert np.array_equal(ra.ra_partition(w.kind, w.S, w.N, rank),
                                  opart.partition_map(w.kind, w.S, w.N, rank))


@pytest.mark.parametrize("args", [
    ("contiguous", 10, 3, 0),      # S % N
    ("zigzag", 12, 4, 0),          # S % 2N
    ("striped", 8, 4, 4),          # rank >= N
    ("striped", 8, 4, -1),
    ("contiguous", 8, 0, 0),       # N < 1
    (7, 8, 2, 0),                  # unknown kind
    ("contiguous", 2**31, 2, 0),   # S too large for int32 positions
])
def test_partition_errors(args):
    with pytest.raises(ra.RingAttnError) as ei:
        ra.ra_partition(*args)
    assert ei.value.status == ra.RA_ERR_INVALID_ARG
    assert ra.ra_last_error()


def test_partition_null_output():
    lib = ra.load_library()
    assert lib.ra_partition(0, 8, 2, 0, None) == ra.RA_ERR_INVALID_ARG
    assert lib.ra_partition(0, 0, 2, 0, None) == ra.RA_OK   # nothing to write


def test_status_strings():
    for code in (ra.RA_OK, ra.RA_ERR_INVALID_ARG, ra.RA_ERR_UNSUPPORTED, ra.RA_ERR_HIP):
        assert ra.ra_status_str(code).startswith("RA_")
    assert "unknown" in ra.ra_status_str(99)


def _attn_desc(**kw):
    base = dict(b=1, n_q=4, n_kv=2, d=128, s_q=64, s_kv=64, dtype=ra.RA_BF16, causal=0,
                scale=0.0, v_layout=ra.RA_V_ROWS, q_pos=None, kv_pos=None)
    base.update(kw)
    return _lib.AttnDesc(**base)


FAKE = ctypes.c_void_p(0x1000)     # aligned, never dereferenced: validation fails first
UNALIGNED = ctypes.c_void_p(0x1004)


@pytest.mark.parametrize("kw,code", [
    (dict(d=64), ra.RA_ERR_UNSUPPORTED),            # bf16 needs d = 128
    (dict(dtype=ra.RA_F32, d=96), ra.RA_ERR_UNSUPPORTED),
    (dict(dtype=5), ra.RA_ERR_UNSUPPORTED),
    (dict(n_q=3), ra.RA_ERR_INVALID_ARG),           # n_q % n_kv
    (dict(n_kv=0), ra.RA_ERR_INVALID_ARG),
    (dict(s_q=-1), ra.RA_ERR_INVALID_ARG),
    (dict(scale=-1.0), ra.RA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), ra.RA_ERR_INVALID_ARG),
    (dict(causal=1), ra.RA_ERR_INVALID_ARG),        # causal without positions
    (dict(causal=2), ra.RA_ERR_INVALID_ARG),
    (dict(v_layout=2), ra.RA_ERR_INVALID_ARG),      # unknown V layout
    (dict(v_layout=1, dtype=ra.RA_F32), ra.RA_ERR_UNSUPPORTED),  # V^T is bf16 only
    (dict(v_layout=1, s_kv=60), ra.RA_ERR_INVALID_ARG),          # V^T rows 16-byte aligned
    (dict(v_layout=1, s_kv=2**23), ra.RA_ERR_UNSUPPORTED),       # V^T past 31-bit offsets
])
def test_block_attn_argument_errors(kw, code):
    lib = ra.load_library()
    desc = _attn_desc(**kw)
    st = lib.ra_block_attn_fwd(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == code, ra.ra_last_error()


def test_block_attn_pointer_errors():
    lib = ra.load_library()
    desc = _attn_desc()
    assert lib.ra_block_attn_fwd(ctypes.byref(desc), None, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.ra_block_attn_fwd(ctypes.byref(desc), UNALIGNED, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.ra_block_attn_fwd(ctypes.byref(desc), FAKE, FAKE, None, FAKE, FAKE, None) == 1
    assert lib.ra_block_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    # nothing to compute: OK without touching any pointer or the GPU
    empty = _attn_desc(s_q=0)
    assert lib.ra_block_attn_fwd(ctypes.byref(empty), None, FAKE, FAKE, None, None, None) == 0


def test_lse_merge_argument_errors():
    lib = ra.load_library()
    for d in (0, 3, 96, 512):
        assert lib.ra_lse_merge(4, d, FAKE, FAKE, FAKE, FAKE, None) == ra.RA_ERR_INVALID_ARG
    assert lib.ra_lse_merge(-1, 128, FAKE, FAKE, FAKE, FAKE, None) == ra.RA_ERR_INVALID_ARG
    assert lib.ra_lse_merge(4, 128, None, FAKE, FAKE, FAKE, None) == ra.RA_ERR_INVALID_ARG
    assert lib.ra_lse_merge(4, 128, UNALIGNED, FAKE, FAKE, FAKE, None) == ra.RA_ERR_INVALID_ARG
    assert lib.ra_lse_merge(0, 128, None, None, None, None, None) == ra.RA_OK


def _ring(**kw):
    base = dict(b=1, n_q=8, n_kv=2, d=128, dtype=ra.RA_BF16, causal=True, kind="zigzag",
                S=1024, N=4, rank=1)
    base.update(kw)
    return _lib.ring_desc(**base)[0]


def test_ring_workspace_bytes():
    def align(x):
        return (x + 255) // 256 * 256
    desc = _ring()
    chunk = 1 * 256 * 2 * 128 * 2
    # positions of all ranks, the rank's document starts, the double buffer
    assert ra.ra_ring_workspace_bytes(desc) == align(1024 * 4) + align(256 * 4) + 2 * 2 * align(chunk)
    unfused = _ring(flags=ra.RA_RING_UNFUSED_MERGE)
    rows = 256 * 8
    assert ra.ra_ring_workspace_bytes(unfused) == (ra.ra_ring_workspace_bytes(desc)
                                                   + align(rows * 128 * 4) + align(rows * 4))
    # N = 1 (one dense pass): bf16 still stages the transposed V chunk
    one_chunk = 1 * 1024 * 2 * 128 * 2
    assert ra.ra_ring_workspace_bytes(_ring(N=1, rank=0)) == (align(1024 * 4) + align(1024 * 4)
                                                              + 2 * 2 * align(one_chunk))
    # ... float32 reads K and V in place: no double buffer
    assert ra.ra_ring_workspace_bytes(_ring(N=1, rank=0, dtype=ra.RA_F32)) == 2 * align(1024 * 4)
    # ... and so does bf16 once a chunk's V^T rows leave 31-bit buffer offsets
    # (d * c * 2 >= 2^31 bytes: c >= 2^23 at d = 128); just below, it stages V^T
    for S, vt in ((2**23, False), (2**23 - 8, True)):
        got = ra.ra_ring_workspace_bytes(_ring(N=1, rank=0, S=S, n_kv=1, n_q=1))
        base = 2 * align(S * 4)
        assert got == base + (2 * 2 * align(S * 128 * 2) if vt else 0), (S, got)


@pytest.mark.parametrize("kw", [
    dict(S=1002), dict(S=1028, N=4), dict(rank=4), dict(N=0, rank=0), dict(kind=9),
    dict(flags=16), dict(flags=5), dict(d=64), dict(n_q=5), dict(S=-4),
])
def test_ring_argument_errors(kw):
    with pytest.raises(ra.RingAttnError):
        ra.ra_ring_workspace_bytes(_ring(**kw))


def test_ring_small_workspace_rejected_before_enqueue():
    lib = ra.load_library()
    desc = _ring()
    need = ra.ra_ring_workspace_bytes(desc)
    st = lib.ra_ring_fwd(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                         None, None)
    assert st == ra.RA_ERR_INVALID_ARG and "workspace" in ra.ra_last_error()
    st = lib.ra_ring_fwd(ctypes.byref(desc), FAKE, FAKE, None, FAKE, FAKE, FAKE, need, None, None)
    assert st == ra.RA_ERR_INVALID_ARG


def test_v_transpose_argument_errors():
    lib = ra.load_library()
    ok_args = (1, 64, 2, 128)
    assert lib.ra_v_transpose(*ok_args, 7, FAKE, ctypes.c_void_p(0x100000), None) == ra.RA_ERR_UNSUPPORTED
    assert lib.ra_v_transpose(-1, 64, 2, 128, ra.RA_BF16, FAKE, FAKE, None) == ra.RA_ERR_INVALID_ARG
    assert lib.ra_v_transpose(1, 64, 0, 128, ra.RA_BF16, FAKE, FAKE, None) == ra.RA_ERR_INVALID_ARG
    assert lib.ra_v_transpose(*ok_args, ra.RA_BF16, None, FAKE, None) == ra.RA_ERR_INVALID_ARG
    # overlapping source and destination
    assert lib.ra_v_transpose(*ok_args, ra.RA_BF16, FAKE, ctypes.c_void_p(0x1010), None) == ra.RA_ERR_INVALID_ARG
    assert lib.ra_v_transpose(300, 64, 256, 128, ra.RA_BF16, FAKE, FAKE, None) == ra.RA_ERR_INVALID_ARG
    # nothing to move: OK without pointers or a GPU
    assert lib.ra_v_transpose(1, 0, 2, 128, ra.RA_BF16, None, None, None) == ra.RA_OK


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ra.RingAttnError):
        _lib.load_library(str(tmp_path / "nope.so"))


def test_backward_argument_errors():
    lib = ra.load_library()
    # delta: d, dtype, pointers
    assert lib.ra_attn_bwd_delta(4, 96, ra.RA_BF16, FAKE, FAKE, FAKE, None) == ra.RA_ERR_UNSUPPORTED
    assert lib.ra_attn_bwd_delta(4, 128, 9, FAKE, FAKE, FAKE, None) == ra.RA_ERR_UNSUPPORTED
    assert lib.ra_attn_bwd_delta(4, 128, ra.RA_BF16, None, FAKE, FAKE, None) == ra.RA_ERR_INVALID_ARG
    assert lib.ra_attn_bwd_delta(0, 128, ra.RA_BF16, None, None, None, None) == ra.RA_OK
    # block backward: bf16 / d = 128 / row-major V only; validation before any launch
    for kw, code in ((dict(dtype=ra.RA_F32), ra.RA_ERR_UNSUPPORTED),
                     (dict(v_layout=ra.RA_V_TRANSPOSED), ra.RA_ERR_UNSUPPORTED),
                     (dict(n_q=3), ra.RA_ERR_INVALID_ARG)):
        desc = _attn_desc(**kw)
        st = lib.ra_block_attn_bwd(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, None)
        assert st == code, (kw, ra.ra_last_error())
    desc = _attn_desc()
    assert lib.ra_block_attn_bwd(ctypes.byref(desc), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                 FAKE, FAKE, None) == ra.RA_ERR_INVALID_ARG
    # ring backward: same ring validation, plus bf16 only and no merge flags
    with pytest.raises(ra.RingAttnError):
        ra.ra_ring_bwd_workspace_bytes(_ring(dtype=ra.RA_F32))
    with pytest.raises(ra.RingAttnError):
        ra.ra_ring_bwd_workspace_bytes(_ring(flags=ra.RA_RING_UNFUSED_MERGE))
    def align(x):
        return (x + 255) // 256 * 256
    # positions, D and log2 lse (head-major), document starts, and for N > 1 two
    # halves of the travelling block: K, V (bf16) and dK, dV (float32), one
    # [b, c, n_kv, d] chunk each
    r = _ring()
    chunk = r.b * (r.S // r.N) * r.n_kv * r.d
    half = 2 * align(chunk * 2) + 2 * align(chunk * 4)
    assert ra.ra_ring_bwd_workspace_bytes(r) == (align(1024 * 4) + align(2 * 256 * 8 * 4)
                                                 + align(256 * 4) + 2 * half)
    r1 = _ring(N=1, S=256, rank=0)
    assert ra.ra_ring_bwd_workspace_bytes(r1) == (align(256 * 4) + align(2 * 256 * 8 * 4)
                                                  + align(256 * 4))


def test_document_mask_argument_errors():
    """The document mask needs the causal rule."""
    lib = ra.load_library()
    for fn in (lambda d: lib.ra_block_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE,
                                               None),
               lambda d: lib.ra_block_attn_bwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE,
                                               FAKE, FAKE, FAKE, FAKE, None)):
        desc = _attn_desc(causal=0)
        desc.q_doc_start = FAKE.value
        assert fn(desc) == ra.RA_ERR_UNSUPPORTED, ra.ra_last_error()
    ring = _ring()
    ring.doc_start = FAKE.value
    for fn in (ra.ra_ring_workspace_bytes, ra.ra_allgather_workspace_bytes,
               ra.ra_ring_bwd_workspace_bytes, ra.ra_allgather_bwd_workspace_bytes):
        fn(ring)                                  # every ring / all-gather call takes it
    ring = _ring(causal=False)
    ring.doc_start = FAKE.value
    for fn in (ra.ra_ring_workspace_bytes, ra.ra_allgather_workspace_bytes,
               ra.ra_ring_bwd_workspace_bytes, ra.ra_allgather_bwd_workspace_bytes):
        with pytest.raises(ra.RingAttnError):
            fn(ring)


def test_allgather_workspace_and_errors():
    def align(x):
        return (x + 255) // 256 * 256
    # S = 1024, N = 4, c = 256; bf16 K/V of the sequence 1024 x 2 x 128 x 2 bytes each
    full = 1024 * 2 * 128 * 2
    # positions, key positions, document starts, K, V^T, the slot row of every position
    want = align(1024 * 4) * 2 + align(256 * 4) + 2 * align(full) + align(1024 * 4)
    assert ra.ra_allgather_workspace_bytes(_ring()) == want
    # float32: no transposed copy
    full32 = 1024 * 2 * 128 * 4
    assert ra.ra_allgather_workspace_bytes(_ring(dtype=ra.RA_F32)) == (
        align(1024 * 4) * 2 + align(256 * 4) + 2 * align(full32))
    for kw in (dict(flags=ra.RA_RING_SERIALIZE), dict(S=1002), dict(rank=4), dict(d=64)):
        with pytest.raises(ra.RingAttnError):
            ra.ra_allgather_workspace_bytes(_ring(**kw))
    lib = ra.load_library()
    desc = _ring()
    need = ra.ra_allgather_workspace_bytes(desc)
    st = lib.ra_allgather_fwd(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                              None)
    assert st == ra.RA_ERR_INVALID_ARG and "workspace" in ra.ra_last_error()
    st = lib.ra_allgather_fwd(ctypes.byref(desc), FAKE, None, FAKE, FAKE, FAKE, FAKE, need, None)
    assert st == ra.RA_ERR_INVALID_ARG


def test_allgather_bwd_workspace_and_errors():
    def align(x):
        return (x + 255) // 256 * 256
    elems = 1024 * 2 * 128
    want = (2 * align(1024 * 4) + align(256 * 4) + align(2 * 256 * 8 * 4)
            + 2 * align(elems * 2) + align(1024 * 4))
    assert ra.ra_allgather_bwd_workspace_bytes(_ring()) == want
    for kw in (dict(dtype=ra.RA_F32), dict(flags=ra.RA_RING_SERIALIZE), dict(S=1002)):
        with pytest.raises(ra.RingAttnError):
            ra.ra_allgather_bwd_workspace_bytes(_ring(**kw))
    lib = ra.load_library()
    desc = _ring()
    need = ra.ra_allgather_bwd_workspace_bytes(desc)
    args = [FAKE] * 9
    st = lib.ra_allgather_bwd(ctypes.byref(desc), *args, FAKE, need - 1, None)
    assert st == ra.RA_ERR_INVALID_ARG and "workspace" in ra.ra_last_error()
    args[6] = None       # dq
    st = lib.ra_allgather_bwd(ctypes.byref(desc), *args, FAKE, need, None)
    assert st == ra.RA_ERR_INVALID_ARG


def test_noalloc_rejects_rings_beyond_its_scratch():
    """ra_ring_fwd_noalloc checks the ring's workspace against the static
    scratch before touching the GPU, and validates the descriptor like
    ra_ring_fwd."""
    lib = ra.load_library()
    big = _ring(S=1 << 20, N=8, n_q=8, n_kv=8)        # ~1 GiB of double buffer
    assert ra.ra_ring_workspace_bytes(big) > ra.RA_NOALLOC_SCRATCH_BYTES
    st = lib.ra_ring_fwd_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == ra.RA_ERR_INVALID_ARG and "scratch" in ra.ra_last_error(), ra.ra_last_error()
    bad = _ring(N=3)                                     # 1024 % 6 != 0 for zig-zag
    assert lib.ra_ring_fwd_noalloc(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None) == ra.RA_ERR_INVALID_ARG
