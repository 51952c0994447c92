"""Token maps, visible-pair counts, tile classes and ring efficiency (fp64/int oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring. Plain NumPy, written
to be checked against the pages by eye.

Citations are to "Context Parallelism and Ring Attention" (hs-black.github.io)
unless stated otherwise.
"""

import numpy as np

KINDS = ("contiguous", "zigzag", "striped")


def partition_map(kind, S, N, rank):
    """Global positions of the tokens rank ``rank`` owns, in its local order.

    * contiguous -- §2: the sequence is cut into N consecutive segments and rank
      i keeps segment i, i.e. positions [i*c, (i+1)*c) with c = S/N.
    * zigzag -- §6 "Zig-zag": the sequence is cut into 2N chunks C_0..C_{2N-1}
      of c/2 tokens; rank i takes C_i and C_{2N-1-i}. Local order: C_i first,
      then C_{2N-1-i}, each ascending (the pages fix only which chunks; this
      ordering makes the map increasing).
    * striped -- §6 "Striped": token p goes to rank p mod N; local order is
      ascending p.

    Remainders are not treated by the pages; S % N != 0 (or S % 2N != 0 for
    zig-zag) raises ValueError.
    """
    if N <= 0 or not (0 <= rank < N):
        raise ValueError("need N > 0 and 0 <= rank < N")
    if S < 0 or S % N:
        raise ValueError("S must be a non-negative multiple of N")
    positions = np.arange(S, dtype=np.int64)
    if kind == "contiguous":
        segments = np.split(positions, N)
        return segments[rank]
    if kind == "zigzag":
        if S % (2 * N):
            raise ValueError("zig-zag needs S to be a multiple of 2N")
        chunks = np.split(positions, 2 * N)
        return np.concatenate([chunks[rank], chunks[2 * N - 1 - rank]])
    if kind == "striped":
        return positions[positions % N == rank]
    raise ValueError(f"unknown partition kind {kind!r}")


def ring_sources(rank, N):
    """§4: at step r (from 0) rank i holds the K/V that rank (i - r) mod N started with."""
    return [(rank - r) % N for r in range(N)]


def visible(q_pos, kv_pos, causal=True):
    """Boolean [len(q_pos), len(kv_pos)] matrix: key visible to query.

    §5: with causal attention token p only sees keys at positions <= p
    (diagonal included); §6 ("the cost of reordering"): the mask is decided by
    each token's position in the original sequence.
    """
    q_pos = np.asarray(q_pos)
    kv_pos = np.asarray(kv_pos)
    if not causal:
        return np.ones((q_pos.size, kv_pos.size), dtype=bool)
    return kv_pos[None, :] <= q_pos[:, None]


def visible_pairs(q_pos, kv_pos, causal=True):
    """Number of visible (query, key) pairs. Counts element by element."""
    q_pos = np.asarray(q_pos)
    kv_pos = np.asarray(kv_pos)
    if not causal:
        return int(q_pos.size) * int(kv_pos.size)
    # Count, for each query, the keys at or before it. Equivalent to
    # visible(q_pos, kv_pos).sum() but without the q x k matrix.
    kv_sorted = np.sort(kv_pos)
    return int(np.searchsorted(kv_sorted, q_pos, side="right").sum())


def step_work(kind, S, N, causal=True):
    """W[i, r] = visible pairs that rank i computes at ring step r (element level)."""
    maps = [partition_map(kind, S, N, i) for i in range(N)]
    W = np.zeros((N, N), dtype=np.int64)
    for i in range(N):
        for r, src in enumerate(ring_sources(i, N)):
            W[i, r] = visible_pairs(maps[i], maps[src], causal)
    return W


def rank_work(kind, S, N, causal=True):
    """Total visible pairs per rank over all ring steps."""
    return step_work(kind, S, N, causal).sum(axis=1)


def ring_efficiency(W):
    """§5 / §7: each step lasts as long as the busiest rank; efficiency is the
    useful work averaged over ranks divided by the sum of per-step maxima."""
    W = np.asarray(W, dtype=np.float64)
    N = W.shape[0]
    return (W.sum() / N) / W.max(axis=0).sum()


SKIP, FULL, DIAG = 0, 1, 2


def tile_classes(q_pos, kv_pos, Bq, Bk, causal=True):
    """Class of every (query tile, key tile) pair, decided element by element.

    SKIP: no visible pair in the tile; FULL: every pair visible; DIAG: some
    but not all (needs the element mask). Tiles are consecutive runs of Bq
    local query rows and Bk local key rows; the last tile may be ragged.
    §7 notes that real kernels skip per tile, discounting the diagonal.
    """
    vis = visible(q_pos, kv_pos, causal)
    nq = -(-len(q_pos) // Bq)
    nk = -(-len(kv_pos) // Bk)
    out = np.zeros((nq, nk), dtype=np.int8)
    for a in range(nq):
        for t in range(nk):
            blk = vis[a * Bq:(a + 1) * Bq, t * Bk:(t + 1) * Bk]
            if not blk.any():
                out[a, t] = SKIP
            elif blk.all():
                out[a, t] = FULL
            else:
                out[a, t] = DIAG
    return out


def tile_work_pairs(q_pos, kv_pos, Bq, Bk, causal=True):
    """(q, k) element slots inside non-skipped tiles: the work a tile-skipping
    kernel actually does (ragged tiles counted by their real size)."""
    cls = tile_classes(q_pos, kv_pos, Bq, Bk, causal)
    total = 0
    for a in range(cls.shape[0]):
        rows = min(Bq, len(q_pos) - a * Bq)
        for t in range(cls.shape[1]):
            if cls[a, t] != SKIP:
                total += rows * min(Bk, len(kv_pos) - t * Bk)
    return total


def tile_work_pairs_increasing(q_pos, kv_pos, Bq, Bk):
    """tile_work_pairs for causal attention when both position lists are
    strictly increasing (every map of §2 / §6 is): a tile then holds a
    visible pair exactly when its first key is not after its last query, so
    the tile test needs only the two end positions (§7's per-tile skip).
    Element slots of the non-skipped tiles; ragged tiles by their real size."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_pos = np.asarray(kv_pos, dtype=np.int64)
    c, s = q_pos.size, kv_pos.size
    if c == 0 or s == 0:
        return 0
    q_starts = np.arange(0, c, Bq)
    k_starts = np.arange(0, s, Bk)
    q_last = q_pos[np.minimum(q_starts + Bq, c) - 1]
    k_first = kv_pos[k_starts]
    rows = np.minimum(q_starts + Bq, c) - q_starts
    cols = np.minimum(k_starts + Bk, s) - k_starts
    keep = k_first[None, :] <= q_last[:, None]
    return int((rows[:, None] * cols[None, :] * keep).sum())


def tile_step_work(kind, S, N, Bq, Bk):
    """W[i, r]: element slots of the non-skipped (Bq x Bk) tiles that rank i
    computes at ring step r, causal (the tile-level counterpart of
    :func:`step_work`; §7: real kernels skip whole tiles, so the diagonal is
    discounted at tile granularity)."""
    maps = [partition_map(kind, S, N, i) for i in range(N)]
    W = np.zeros((N, N), dtype=np.int64)
    for i in range(N):
        for r, src in enumerate(ring_sources(i, N)):
            W[i, r] = tile_work_pairs_increasing(maps[i], maps[src], Bq, Bk)
    return W


def kv_bytes(b, s, n_kv, d_h, bytes_per_elem=2):
    """§8: full K/V of one layer is 2 * 2 * b * s * n_kv * d_h bytes in bf16
    (K and V, two bytes each)."""
    return 2 * bytes_per_elem * b * s * n_kv * d_h


def causal_adjusted_flops(b, n_q, d, pairs):
    """§4 "can communication be hidden": Q K^T and P V each cost 2*b*c^2*h flops
    for a full c x c block (h = n_q * d), i.e. 4 * n_q * d flops per (query,
    key) pair summed over heads; causal attention counts visible pairs only."""
    return 4 * b * n_q * d * pairs
