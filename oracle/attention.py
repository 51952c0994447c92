"""Softmax attention, block statistics, the log-sum-exp merge and the ring loop, in fp64.

TEST INFRASTRUCTURE ONLY -- see the package docstring. Nothing here is blocked,
fused or reordered beyond what the cited definitions state.

Citations are to "Context Parallelism and Ring Attention" (hs-black.github.io)
unless stated otherwise.

Conventions (readings where the pages are silent):

* layout [b, s, heads, d] for q, k, v and o; lse is [b, s, n_q];
* query head h uses key/value head h // (n_q // n_kv) (contiguous GQA groups;
  the "Tensor Parallelism" page's GQA table only says several query heads
  share one KV head);
* log is the natural log;
* a query that sees no key in a block gets o_b = 0 and lse_b = -inf (the
  empty-sum limit), which is also the identity of the merge.
"""

import numpy as np

from .partition import partition_map, ring_sources, visible


def _check_shapes(q, k, v, q_pos, kv_pos):
    b, c, n_q, d = q.shape
    bk, s, n_kv, dk = k.shape
    if v.shape != k.shape or bk != b or dk != d:
        raise ValueError("q [b,c,n_q,d] and k, v [b,s,n_kv,d] shapes disagree")
    if n_q % n_kv:
        raise ValueError("n_q must be a multiple of n_kv")
    if len(q_pos) != c or len(kv_pos) != s:
        raise ValueError("positions must match the row counts")
    return b, c, n_q, d, s, n_kv


def naive_attention(q, k, v, q_pos, kv_pos, causal, scale):
    """Primary oracle: one softmax over every visible key (§3 first equation).

    o = sum_j softmax(x)_j v_j with x_j = scale * q . k_j; the pages use
    scale = 1/sqrt(d_h). lse = log sum_j e^{x_j} (§3, block LSE equation
    applied to the whole key set), computed as m + log sum e^{x - m}.
    The visible set follows the causal rule of §5 on global positions.

    q: [b, c, n_q, d]; k, v: [b, s, n_kv, d]; q_pos: [c]; kv_pos: [s].
    Returns o [b, c, n_q, d] and lse [b, c, n_q], float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, c, n_q, d, s, n_kv = _check_shapes(q, k, v, q_pos, kv_pos)
    g = n_q // n_kv
    o = np.zeros((b, c, n_q, d))
    lse = np.full((b, c, n_q), -np.inf)
    if c == 0 or s == 0:
        return o, lse
    vis = visible(q_pos, kv_pos, causal)            # [c, s]
    has_key = vis.any(axis=1)
    for bi in range(b):
        for h in range(n_q):
            kvh = h // g
            x = scale * (q[bi, :, h, :] @ k[bi, :, kvh, :].T)   # [c, s]
            x = np.where(vis, x, -np.inf)
            m = np.max(x, axis=1, keepdims=True)
            m = np.where(has_key[:, None], m, 0.0)
            total = np.sum(np.exp(x - m), axis=1)
            with np.errstate(divide="ignore"):
                row_lse = m[:, 0] + np.log(total)               # -inf where no key
            weights = np.exp(x - np.where(has_key, row_lse, 0.0)[:, None])
            o[bi, :, h, :] = np.where(has_key[:, None], weights @ v[bi, :, kvh, :], 0.0)
            lse[bi, :, h] = np.where(has_key, row_lse, -np.inf)
    return o, lse


def block_attention(q, k_blk, v_blk, q_pos, kv_pos_blk, causal, scale):
    """Per-block statistics of §3: for the keys B of one block,

    m_b = max_{j in B} x_j,  l_b = sum_{j in B} e^{x_j - m_b},
    o_b = (1/l_b) sum_{j in B} e^{x_j - m_b} v_j,  lse_b = m_b + log l_b.

    Only keys visible to the query (§5 causal rule) belong to its block; a
    query with none gets (o_b, lse_b) = (0, -inf).
    """
    q = np.asarray(q, dtype=np.float64)
    k_blk = np.asarray(k_blk, dtype=np.float64)
    v_blk = np.asarray(v_blk, dtype=np.float64)
    b, c, n_q, d, s, n_kv = _check_shapes(q, k_blk, v_blk, q_pos, kv_pos_blk)
    g = n_q // n_kv
    o_b = np.zeros((b, c, n_q, d))
    lse_b = np.full((b, c, n_q), -np.inf)
    if s == 0:
        return o_b, lse_b
    vis = visible(q_pos, kv_pos_blk, causal)
    for bi in range(b):
        for h in range(n_q):
            kvh = h // g
            for a in range(c):
                keys = np.nonzero(vis[a])[0]
                if keys.size == 0:
                    continue
                x = scale * (k_blk[bi, keys, kvh, :] @ q[bi, a, h, :])
                m_b = x.max()
                e = np.exp(x - m_b)
                l_b = e.sum()
                o_b[bi, a, h, :] = (e @ v_blk[bi, keys, kvh, :]) / l_b
                lse_b[bi, a, h] = m_b + np.log(l_b)
    return o_b, lse_b


def merge(o, lse, o_b, lse_b):
    """The boxed two-block merge of §3 in its stable form.

    o = e^{lse_1 - lse} o_1 + e^{lse_2 - lse} o_2,
    lse = M + log(e^{lse_1 - M} + e^{lse_2 - M}),  M = max(lse_1, lse_2),
    so every exponent is <= 0. When both inputs are empty (M = -inf) the
    result stays the identity (0, -inf).
    """
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    M = np.maximum(lse, lse_b)
    empty = np.isneginf(M)
    M_safe = np.where(empty, 0.0, M)
    with np.errstate(divide="ignore"):      # log(0) only on empty rows, replaced below
        new_lse = M_safe + np.log(np.exp(lse - M_safe) + np.exp(lse_b - M_safe))
    new_lse = np.where(empty, -np.inf, new_lse)
    lse_ref = np.where(empty, 0.0, new_lse)
    w1 = np.where(empty, 0.0, np.exp(lse - lse_ref))
    w2 = np.where(empty, 0.0, np.exp(lse_b - lse_ref))
    new_o = w1[..., None] * o + w2[..., None] * o_b
    return new_o, new_lse


def merge_weights(lse, lse_b):
    """The two weights e^{lse_b - lse_total} of the boxed merge; §3 notes they sum to 1."""
    M = np.maximum(lse, lse_b)
    total = M + np.log(np.exp(lse - M) + np.exp(lse_b - M))
    return np.exp(lse - total), np.exp(lse_b - total)


def ring_attention(q, k, v, kind, S, N, rank, causal, scale, keep_steps=False):
    """Secondary oracle: the ring forward of §4, block then merge.

    q: [b, c, n_q, d] -- rank ``rank``'s queries in local order;
    k, v: [b, S, n_kv, d] -- the whole sequence in global order.
    The running (o, lse) starts at the merge identity (0, -inf) (the pages'
    ``None``). At step r the rank holds the K/V that rank (rank - r) mod N
    owns; its block statistics are merged in with :func:`merge`.
    Returns (o, lse) and, if keep_steps, the list of (src, o_b, lse_b).
    """
    q_pos = partition_map(kind, S, N, rank)
    b, c, n_q, d = q.shape
    o = np.zeros((b, c, n_q, d))
    lse = np.full((b, c, n_q), -np.inf)
    steps = []
    for src in ring_sources(rank, N):
        kv_pos = partition_map(kind, S, N, src)
        o_b, lse_b = block_attention(q, k[:, kv_pos], v[:, kv_pos], q_pos, kv_pos,
                                     causal, scale)
        o, lse = merge(o, lse, o_b, lse_b)
        if keep_steps:
            steps.append((src, o_b, lse_b))
    return (o, lse, steps) if keep_steps else (o, lse)


def rows_attention(q_rows, k, v, q_pos_rows, causal, scale):
    """Primary oracle on a subset of query rows against the whole sequence in
    global order (rows are independent, so this is :func:`naive_attention`
    with kv_pos = 0..S-1 applied to the chosen rows only)."""
    S = k.shape[1]
    return naive_attention(q_rows, k, v, q_pos_rows, np.arange(S), causal, scale)
