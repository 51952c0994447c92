"""The CPU oracle against its pins (closed forms, brute force, a library
special case and the numbers the pages print). CPU only."""

import types

import numpy as np
import pytest

import oracle_pins as pins
from oracle import attention, partition


def oracle_namespace():
    ns = types.SimpleNamespace()
    for mod in (attention, partition):
        for name in dir(mod):
            if not name.startswith("_"):
                setattr(ns, name, getattr(mod, name))
    return ns


@pytest.mark.parametrize("pin", pins.ATTENTION_PINS + pins.PARTITION_PINS,
                         ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle_namespace())


def test_gqa_table_matches_workload_heads():
    from golden_values import read
    import synth
    gold = read("gqa_heads.txt")
    w8 = synth.WORKLOADS["llama3_8b_32k_zigzag"]
    w70 = synth.WORKLOADS["llama3_70b_128k_zigzag"]
    assert [w8.n_q, w8.n_kv] == [int(x) for x in gold["LLaMA-3 8B"]]
    assert [w70.n_q, w70.n_kv] == [int(x) for x in gold["LLaMA-3 70B"]]
    # the Ulysses-local and 1M shapes hold one eighth of the 70B heads (64/8 split)
    for name in ("ulysses_local_128k", "long_1m_zigzag"):
        w = synth.WORKLOADS[name]
        assert (w.n_q * 8, w.n_kv * 8) == (w70.n_q, w70.n_kv)


def test_partition_rejects_remainders():
    with pytest.raises(ValueError):
        partition.partition_map("contiguous", 10, 3, 0)
    with pytest.raises(ValueError):
        partition.partition_map("zigzag", 12, 4, 0)   # 12 % 8 != 0
    with pytest.raises(ValueError):
        partition.partition_map("striped", 8, 4, 4)


def test_ring_sources_visit_every_chunk_once():
    for N in (1, 2, 5, 8, 32):
        for rank in range(N):
            src = partition.ring_sources(rank, N)
            assert src[0] == rank and sorted(src) == list(range(N))


def test_workload_pair_counts():
    """Visible pairs of rank 0 for the measured workloads (exact integers)."""
    import synth
    expect = {"tiny_ring_f32": 64 * 256,
              "llama3_8b_32k_zigzag": 67_110_912,
              "llama3_70b_128k_zigzag": 1_073_750_016,
              "ulysses_local_128k": 131072 * 131073 // 2,
              "long_1m_zigzag": 17_179_885_568}
    for name, want in expect.items():
        w = synth.WORKLOADS[name]
        q_pos = partition.partition_map(w.kind, w.S, w.N, 0)
        got = partition.visible_pairs(q_pos, np.arange(w.S), w.causal)
        assert got == want, name
        # zig-zag: every rank S*c/2 + c/2 pairs exactly
        if w.kind == "zigzag":
            assert got == w.S * w.c // 2 + w.c // 2


def test_bf16_rounding_is_nearest_even():
    import synth
    # bf16 keeps 7 fraction bits: 1 + 2^-8 is a tie (rounds to the even 1.0),
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 1.0 + 2**-8 + 2**-12], np.float32)
    back = synth.bf16_to_f32(synth.bf16_bits(x))
    assert back.tolist() == [1.0, 1.0, 1.0 + 2**-6, -1.0, 1.0 + 2**-7]


def test_draw_is_seeded_and_subset_stable():
    import synth
    w = synth.WORKLOADS["tiny_ring_f32"]
    a, b = synth.draw(w), synth.draw(w)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k)
    rows = np.array([0, 5, 63])
    sub = synth.draw(w, q_rows=rows)
    assert np.array_equal(sub.q, a.q[:, rows])
