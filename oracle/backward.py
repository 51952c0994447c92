"""Gradients of softmax attention and the ring backward, in fp64.

TEST INFRASTRUCTURE ONLY -- see the package docstring. Nothing here is blocked,
fused or reordered beyond what the cited definitions state.

Source: "Context Parallelism and Ring Attention" (hs-black.github.io):

* §3, last paragraph (the backward needs only the lse). With the GLOBAL lse of
  a query, the probability of key j is p_j = e^{x_j - lse}, so it can be
  recomputed on any block alone. Each key then gets dv_j = sum_q p_j do and
  dx_j = p_j (do . v_j - D), where D = do . o is one scalar per query (also
  global). The rank keeps its queries' o and lse after the forward.
* §4: the K/V blocks travel the ring again. Each step yields the block's
  contribution to dQ (accumulated on the rank) and to that block's dK and dV;
  those accumulated dK, dV travel the ring with the block ("can communication
  be hidden": the backward moves dK, dV as well).

Readings where the pages stop:

* x_j = scale * q . k_j (§3), so by the chain rule dq = scale * sum_j dx_j k_j
  and dk_j = scale * sum_q dx_j q -- the pages give dx and dv only;
* the loss is L = sum(do * o): do is the upstream gradient of o;
* a query with no visible key anywhere (lse = -inf) has o = 0 and contributes
  no gradient;
* GQA: a key/value head's dk and dv sum the contributions of every query head
  that reads it (query head h reads key/value head h // (n_q // n_kv)).
"""

import numpy as np

from .partition import partition_map, ring_sources, visible


def _as64(*xs):
    return [np.asarray(x, dtype=np.float64) for x in xs]


def delta(o, do):
    """D = do . o per (token, query head) (§3 backward paragraph): [b, c, n_q]."""
    o, do = _as64(o, do)
    return np.sum(do * o, axis=-1)


def naive_attention_bwd(q, k, v, do, q_pos, kv_pos, causal, scale):
    """Primary backward oracle: the gradients of L = sum(do * o) for the plain
    definition o = softmax(x) v over the visible keys (§3 first equation, §5
    causal rule), written out by the chain rule on the whole key set:

    p = softmax(x), o = p v, D = rowsum(do * o),
    dv = p^T do, dp = do v^T, dx = p * (dp - D),
    dq = scale * dx k, dk = scale * dx^T q.

    q, do: [b, c, n_q, d]; k, v: [b, s, n_kv, d]. Returns dq [b, c, n_q, d] and
    dk, dv [b, s, n_kv, d], float64.
    """
    q, k, v, do = _as64(q, k, v, do)
    b, c, n_q, d = q.shape
    s, n_kv = k.shape[1], k.shape[2]
    g = n_q // n_kv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if c == 0 or s == 0:
        return dq, dk, dv
    vis = visible(q_pos, kv_pos, causal)               # [c, s]
    has_key = vis.any(axis=1)
    for bi in range(b):
        for h in range(n_q):
            kvh = h // g
            x = scale * (q[bi, :, h, :] @ k[bi, :, kvh, :].T)       # [c, s]
            x = np.where(vis, x, -np.inf)
            m = np.where(has_key, np.max(np.where(vis, x, -np.inf), axis=1), 0.0)
            e = np.where(vis, np.exp(x - m[:, None]), 0.0)
            tot = e.sum(axis=1)
            p = e / np.where(has_key, tot, 1.0)[:, None]             # 0 on rows without keys
            o = p @ v[bi, :, kvh, :]
            D = np.sum(do[bi, :, h, :] * o, axis=1)
            dv[bi, :, kvh, :] += p.T @ do[bi, :, h, :]
            dp = do[bi, :, h, :] @ v[bi, :, kvh, :].T
            dx = p * (dp - D[:, None])
            dq[bi, :, h, :] = scale * (dx @ k[bi, :, kvh, :])
            dk[bi, :, kvh, :] += scale * (dx.T @ q[bi, :, h, :])
    return dq, dk, dv


def block_attention_bwd(q, k_blk, v_blk, do, lse, D, q_pos, kv_pos_blk, causal, scale):
    """One block's gradient contributions, following §3's backward paragraph
    key by key: with the GLOBAL lse and D = do . o of the query,

    p_j = e^{x_j - lse},  dv_j += p_j do,  dx_j = p_j (do . v_j - D),
    dq += scale * dx_j k_j,  dk_j += scale * dx_j q,

    for every key j of the block visible to the query (§5). Queries with
    lse = -inf contribute nothing. Returns (dq, dk, dv) of this block.
    """
    q, k_blk, v_blk, do, lse, D = _as64(q, k_blk, v_blk, do, lse, D)
    b, c, n_q, d = q.shape
    s, n_kv = k_blk.shape[1], k_blk.shape[2]
    g = n_q // n_kv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k_blk)
    dv = np.zeros_like(v_blk)
    if s == 0 or c == 0:
        return dq, dk, dv
    vis = visible(q_pos, kv_pos_blk, causal)
    for bi in range(b):
        for h in range(n_q):
            kvh = h // g
            for a in range(c):
                if np.isneginf(lse[bi, a, h]):
                    continue
                keys = np.nonzero(vis[a])[0]
                if keys.size == 0:
                    continue
                x = scale * (k_blk[bi, keys, kvh, :] @ q[bi, a, h, :])
                p = np.exp(x - lse[bi, a, h])
                dv[bi, keys, kvh, :] += p[:, None] * do[bi, a, h, :][None, :]
                dx = p * (v_blk[bi, keys, kvh, :] @ do[bi, a, h, :] - D[bi, a, h])
                dq[bi, a, h, :] += scale * (dx @ k_blk[bi, keys, kvh, :])
                dk[bi, keys, kvh, :] += scale * dx[:, None] * q[bi, a, h, :][None, :]
    return dq, dk, dv


def ring_attention_bwd(q, k, v, do, o, lse, kind, S, N, rank, causal, scale):
    """The ring backward of §3 / §4 for rank ``rank``.

    q, do, o: [b, c, n_q, d] and lse [b, c, n_q] -- the rank's queries in
    local order, with the global o and lse its forward kept; k, v: [b, S,
    n_kv, d], the whole sequence in global order. D = do . o once; at step r
    the rank holds the block of rank (rank - r) mod N; its dq contribution is
    accumulated on the rank, and its dk, dv are added to that block's
    travelling gradient buffers.

    Returns dq [b, c, n_q, d] and dk_chunks, dv_chunks [N, b, c, n_kv, d]:
    this rank's contribution to every block's dk, dv, block j in rank j's
    local order (summing these over all ranks gives the sequence's dk, dv).
    """
    q, k, v, do, o, lse = _as64(q, k, v, do, o, lse)
    b, c, n_q, d = q.shape
    n_kv = k.shape[2]
    q_pos = partition_map(kind, S, N, rank)
    D = delta(o, do)
    dq = np.zeros_like(q)
    dk_chunks = np.zeros((N, b, c, n_kv, d))
    dv_chunks = np.zeros((N, b, c, n_kv, d))
    for src in ring_sources(rank, N):
        kv_pos = partition_map(kind, S, N, src)
        dq_b, dk_b, dv_b = block_attention_bwd(q, k[:, kv_pos], v[:, kv_pos], do, lse, D,
                                               q_pos, kv_pos, causal, scale)
        dq += dq_b
        dk_chunks[src] += dk_b
        dv_chunks[src] += dv_b
    return dq, dk_chunks, dv_chunks


def rows_dq(q_rows, k, v, do_rows, q_pos_rows, kv_pos, causal, scale):
    """dq of chosen query rows only, by the same chain rule as
    :func:`naive_attention_bwd` (a row's dq depends on that row alone:
    dq = scale * sum_j p_j (dp_j - D) k_j with p its softmax over the visible
    keys, dp_j = do . v_j, D = do . o). For full-size spot checks: each key /
    value head is copied once into contiguous memory for its query heads.
    Returns [b, r, n_q, d] float64."""
    q_rows, do_rows = _as64(q_rows, do_rows)
    b, r, n_q, d = q_rows.shape
    n_kv = k.shape[2]
    g = n_q // n_kv
    dq = np.zeros_like(q_rows)
    if r == 0 or k.shape[1] == 0:
        return dq
    vis = visible(q_pos_rows, kv_pos, causal)
    has_key = vis.any(axis=1)
    for bi in range(b):
        for kvh in range(n_kv):
            kk = np.ascontiguousarray(k[bi, :, kvh, :], dtype=np.float64)
            vv = np.ascontiguousarray(v[bi, :, kvh, :], dtype=np.float64)
            for h in range(kvh * g, (kvh + 1) * g):
                x = np.where(vis, scale * (q_rows[bi, :, h, :] @ kk.T), -np.inf)
                m = np.where(has_key, x.max(axis=1), 0.0)
                e = np.exp(x - m[:, None])
                p = e / np.where(has_key, e.sum(axis=1), 1.0)[:, None]
                D = np.sum(do_rows[bi, :, h, :] * (p @ vv), axis=1)
                dx = p * (do_rows[bi, :, h, :] @ vv.T - D[:, None])
                dq[bi, :, h, :] = scale * (dx @ kk)
    return dq
