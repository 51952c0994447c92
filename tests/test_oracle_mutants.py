"""Plant plausible mistakes in the CPU oracle and check that the pins catch
each one. The mistakes are planted in the oracle, on the CPU, through
monkeypatching; nothing here touches the HIP path."""

import numpy as np
import pytest

import oracle_pins as pins
from oracle import attention, partition
from test_oracle import oracle_namespace

real_naive = attention.naive_attention
real_block = attention.block_attention
real_merge = attention.merge
real_map = partition.partition_map
real_rows = attention.rows_attention
real_tile_pairs = partition.tile_work_pairs
real_tile_inc = partition.tile_work_pairs_increasing
real_step_work = partition.step_work


def rows_kv_shifted(q, k, v, qp, c, s):
    """Keys placed one position later than their index."""
    return real_naive(q, k, v, qp, np.arange(k.shape[1]) + 1, c, s)


def rows_kv_reversed(q, k, v, qp, c, s):
    return real_naive(q, k, v, qp, np.arange(k.shape[1])[::-1], c, s)


def tile_pairs_diag_skipped(q_pos, kv_pos, Bq, Bk, causal=True):
    """Counts only fully visible tiles (drops the diagonal ones)."""
    cls = partition.tile_classes(q_pos, kv_pos, Bq, Bk, causal)
    total = 0
    for a in range(cls.shape[0]):
        rows = min(Bq, len(q_pos) - a * Bq)
        for t in range(cls.shape[1]):
            if cls[a, t] == partition.FULL:
                total += rows * min(Bk, len(kv_pos) - t * Bk)
    return total


def tile_inc_first_query(q_pos, kv_pos, Bq, Bk):
    """Tests a tile's first key against its FIRST query instead of its last."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.asarray(kv_pos, dtype=np.int64)
    c, s = q_pos.size, kv_pos.size
    qs, ks = np.arange(0, c, Bq), np.arange(0, s, Bk)
    keep = kv_pos[ks][None, :] <= q_pos[qs][:, None]
    rows = np.minimum(qs + Bq, c) - qs
    cols = np.minimum(ks + Bk, s) - ks
    return int((rows[:, None] * cols[None, :] * keep).sum())


def tile_inc_no_ragged(q_pos, kv_pos, Bq, Bk):
    """Counts every tile at its full size (ragged tails over-counted)."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.asarray(kv_pos, dtype=np.int64)
    c, s = q_pos.size, kv_pos.size
    qs, ks = np.arange(0, c, Bq), np.arange(0, s, Bk)
    keep = kv_pos[ks][None, :] <= q_pos[np.minimum(qs + Bq, c) - 1][:, None]
    return int((Bq * Bk * keep).sum())


def rank_work_columns(kind, S, N, causal=True):
    """Sums the per-step table over ranks instead of over steps."""
    return real_step_work(kind, S, N, causal).sum(axis=0)


def merge_wrong_sign(o, lse, o_b, lse_b):
    M = np.maximum(lse, lse_b)
    new_lse = M + np.log(np.exp(lse - M) + np.exp(lse_b - M))
    return (np.exp(lse - new_lse)[..., None] * o + np.exp(new_lse - lse_b)[..., None] * o_b,
            new_lse)


def merge_dropped_max(o, lse, o_b, lse_b):
    M = np.maximum(lse, lse_b)
    new_lse = np.log(np.exp(lse - M) + np.exp(lse_b - M))          # "+ M" dropped
    return (np.exp(lse - new_lse)[..., None] * o + np.exp(lse_b - new_lse)[..., None] * o_b,
            new_lse)


def merge_unweighted(o, lse, o_b, lse_b):
    new_o, new_lse = real_merge(o, lse, o_b, lse_b)
    return o + o_b, new_lse


MUTANTS = {
    # attention
    "naive_strict_causal": ("naive_attention",
                            lambda q, k, v, qp, kp, c, s: real_naive(q, k, v, np.asarray(qp) - 1, kp, c, s)),
    "naive_no_scale": ("naive_attention",
                       lambda q, k, v, qp, kp, c, s: real_naive(q, k, v, qp, kp, c, 1.0)),
    "naive_k_v_swapped": ("naive_attention",
                          lambda q, k, v, qp, kp, c, s: real_naive(q, v, k, qp, kp, c, s)),
    "block_future_visible": ("block_attention",
                             lambda q, k, v, qp, kp, c, s: real_block(q, k, v, np.asarray(qp) + 1, kp, c, s)),
    "block_half_scale": ("block_attention",
                         lambda q, k, v, qp, kp, c, s: real_block(q, k, v, qp, kp, c, 0.5 * s)),
    "merge_wrong_sign": ("merge", merge_wrong_sign),
    "merge_dropped_max": ("merge", merge_dropped_max),
    "merge_unweighted": ("merge", merge_unweighted),
    # partition
    "zigzag_wrong_partner": ("partition_map",
                             lambda kind, S, N, r: (np.concatenate(
                                 [np.split(np.arange(S), 2 * N)[r],
                                  np.split(np.arange(S), 2 * N)[(2 * N - 2 - r) % (2 * N)]])
                                 if kind == "zigzag" else real_map(kind, S, N, r))),
    "striped_off_by_one": ("partition_map",
                           lambda kind, S, N, r: (np.arange(S)[np.arange(S) % N == (r + 1) % N]
                                                  if kind == "striped" else real_map(kind, S, N, r))),
    "rows_kv_shifted": ("rows_attention", rows_kv_shifted),
    "rows_kv_reversed": ("rows_attention", rows_kv_reversed),
    "tile_pairs_diag_skipped": ("tile_work_pairs", tile_pairs_diag_skipped),
    "tile_inc_first_query": ("tile_work_pairs_increasing", tile_inc_first_query),
    "tile_inc_no_ragged": ("tile_work_pairs_increasing", tile_inc_no_ragged),
    "flops_half": ("causal_adjusted_flops", lambda b, n_q, d, pairs: 2 * b * n_q * d * pairs),
    "flops_per_head_missing": ("causal_adjusted_flops", lambda b, n_q, d, pairs: 4 * b * d * pairs),
    "rank_work_columns": ("rank_work", rank_work_columns),
    "contiguous_reversed": ("partition_map",
                            lambda kind, S, N, r: (real_map(kind, S, N, N - 1 - r)
                                                   if kind == "contiguous" else real_map(kind, S, N, r))),
}

PATCH_SITES = {
    "naive_attention": [attention],
    "block_attention": [attention],
    "merge": [attention],
    "partition_map": [attention, partition],
    "rows_attention": [attention],
    "tile_work_pairs": [partition],
    "tile_work_pairs_increasing": [partition],
    "causal_adjusted_flops": [partition],
    "rank_work": [partition],
}


def run_all_pins():
    failures = []
    for pin in pins.ATTENTION_PINS + pins.PARTITION_PINS:
        try:
            pin(oracle_namespace())
        except Exception as exc:  # noqa: BLE001 -- any failure counts as caught
            failures.append((pin.__name__, type(exc).__name__))
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    fname, fn = MUTANTS[name]
    for mod in PATCH_SITES[fname]:
        monkeypatch.setattr(mod, fname, fn)
    failures = run_all_pins()
    assert failures, f"no pin caught the planted mistake {name}"


def test_ring_sources_follow_the_described_protocol():
    """Each step every rank sends its current K/V to rank + 1 and receives from
    rank - 1; simulating that hand-off must give the oracle's source list."""
    for N in (1, 2, 3, 8):
        hold = list(range(N))
        for r in range(N):
            for i in range(N):
                assert partition.ring_sources(i, N)[r] == hold[i]
            hold = [hold[(i - 1) % N] for i in range(N)]
