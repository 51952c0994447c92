"""All-gather context parallelism with a document mask, in fp64.

TEST INFRASTRUCTURE ONLY -- see the package docstring. Nothing here is blocked,
fused or reordered beyond what the cited definitions state.

Source: "Context Parallelism and Ring Attention" (hs-black.github.io), §8
(all-gather CP). Instead of passing K/V around a ring, every rank gathers the
K and V of the whole sequence from its CP group before attention and attends
with its own queries (backward: a reduce-scatter of dK, dV). The queries keep
the load-balanced 2 x CP chunking of §6. The page gives the document mask as
the reason this form suits Llama 3: one training sequence packs several
documents and no token may attend across a document boundary; with the whole
K/V at hand the rank applies that mask directly on original positions.

The backward of all-gather CP (§8: a reduce-scatter of dK, dV) follows the
backward paragraph of §3 with the same mask: the gradients of L = sum(do * o)
by the chain rule (as in :mod:`oracle.backward`), the rank's dK, dV of the
whole sequence then cut back into the N chunks (this rank's share of the
reduce-scatter's input; summing every rank's shares gives the sequence's
dK, dV).

Readings where the page stops:

* documents are contiguous runs of positions that tile [0, S); a document id
  per position is non-decreasing (document 0 first);
* the document mask is combined with the causal rule of §5: key j is visible
  to query q iff doc(p_j) == doc(p_q) and p_j <= p_q (without the causal rule,
  iff the documents are equal);
* the gathered K/V are laid out in global position order;
* the visible-pair count of the FLOP convention (§4, see
  :func:`oracle.partition.causal_adjusted_flops`) counts pairs that pass both
  rules.
"""

import numpy as np

from .partition import partition_map


def doc_ids_from_lengths(lengths):
    """Document id of every position for documents of the given lengths, packed
    back to back from position 0 (readings above)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    if (lengths <= 0).any():
        raise ValueError("document lengths must be positive")
    return np.repeat(np.arange(lengths.size, dtype=np.int64), lengths)


def doc_start(doc_ids):
    """For every position, the first position of its document."""
    doc_ids = np.asarray(doc_ids)
    S = doc_ids.size
    out = np.zeros(S, dtype=np.int64)
    for p in range(1, S):
        out[p] = out[p - 1] if doc_ids[p] == doc_ids[p - 1] else p
    return out


def visible_docs(q_pos, kv_pos, doc_ids, causal=True):
    """Boolean [len(q_pos), len(kv_pos)]: key visible to query under the
    document mask (same document) and, if causal, the §5 rule on original
    positions (§6: masks are decided by original positions)."""
    q_pos = np.asarray(q_pos)
    kv_pos = np.asarray(kv_pos)
    doc_ids = np.asarray(doc_ids)
    same = doc_ids[q_pos][:, None] == doc_ids[kv_pos][None, :]
    if causal:
        same &= kv_pos[None, :] <= q_pos[:, None]
    return same


def masked_attention(q, k, v, vis, scale):
    """Softmax attention (§3 first equation) over an explicit visibility
    matrix vis [c, s]: o = sum_j softmax(x)_j v_j over the visible keys,
    lse = log sum_j e^{x_j} (m + log sum e^{x - m}); a query with no visible
    key gets (0, -inf). q: [b, c, n_q, d]; k, v: [b, s, n_kv, d]; query head
    h reads key/value head h // (n_q // n_kv)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, c, n_q, d = q.shape
    n_kv = k.shape[2]
    g = n_q // n_kv
    o = np.zeros((b, c, n_q, d))
    lse = np.full((b, c, n_q), -np.inf)
    if c == 0 or k.shape[1] == 0:
        return o, lse
    has_key = vis.any(axis=1)
    for bi in range(b):
        for h in range(n_q):
            kvh = h // g
            x = np.where(vis, scale * (q[bi, :, h, :] @ k[bi, :, kvh, :].T), -np.inf)
            m = np.where(has_key, x.max(axis=1), 0.0)
            e = np.exp(x - m[:, None])
            tot = e.sum(axis=1)
            with np.errstate(divide="ignore"):
                row_lse = np.where(has_key, m + np.log(np.where(has_key, tot, 1.0)), -np.inf)
            w = e / np.where(has_key, tot, 1.0)[:, None]
            o[bi, :, h, :] = w @ v[bi, :, kvh, :]
            lse[bi, :, h] = row_lse
    return o, lse


def allgather_kv(chunks, kind, S, N):
    """§8's all-gather on one GPU: chunks [N, b, c, n_kv, d] (chunk j = rank
    j's tokens in its local order, §6 maps) -> [b, S, n_kv, d] in global
    position order."""
    chunks = np.asarray(chunks)
    b, c = chunks.shape[1], chunks.shape[2]
    if N * c != S:
        raise ValueError("chunks do not cover the sequence")
    full = np.zeros((b, S) + chunks.shape[3:], dtype=chunks.dtype)
    for j in range(N):
        full[:, partition_map(kind, S, N, j)] = chunks[j]
    return full


def allgather_attention(q, k_chunks, v_chunks, kind, S, N, rank, doc_ids, causal, scale):
    """One rank of all-gather CP (§8): gather K and V of the whole sequence,
    then attend with the rank's queries (local order, map ``kind``) under the
    document mask. Returns o [b, c, n_q, d] and lse [b, c, n_q]."""
    k = allgather_kv(k_chunks, kind, S, N)
    v = allgather_kv(v_chunks, kind, S, N)
    q_pos = partition_map(kind, S, N, rank)
    vis = visible_docs(q_pos, np.arange(S), doc_ids, causal)
    return masked_attention(q, k, v, vis, scale)


def rows_attention_docs(q_rows, k, v, q_pos_rows, doc_ids, causal, scale):
    """The document-masked definition on chosen query rows against the whole
    sequence in global order (rows are independent)."""
    S = k.shape[1]
    vis = visible_docs(q_pos_rows, np.arange(S), doc_ids, causal)
    return masked_attention(q_rows, k, v, vis, scale)


def doc_visible_pairs(q_pos, doc_ids, causal=True):
    """Visible (query, key) pairs of queries at q_pos against every position of
    the sequence under the document mask: p - start(doc(p)) + 1 per query when
    causal, the document length otherwise."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    doc_ids = np.asarray(doc_ids)
    start = doc_start(doc_ids)
    if causal:
        return int((q_pos - start[q_pos] + 1).sum())
    lengths = np.bincount(doc_ids)
    return int(lengths[doc_ids[q_pos]].sum())


def masked_attention_bwd(q, k, v, do, vis, scale):
    """Gradients of L = sum(do * o) for o = softmax(x) v over an explicit
    visibility matrix vis [c, s] (x = scale q . k), by the chain rule:
    p = softmax(x), D = rowsum(do * o), dv = p^T do, dp = do v^T,
    dx = p * (dp - D), dq = scale dx k, dk = scale dx^T q. Query head h reads
    key/value head h // (n_q // n_kv); a key/value head sums its group's
    contributions. Rows with no visible key contribute nothing."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    b, c, n_q, d = q.shape
    n_kv = k.shape[2]
    g = n_q // n_kv
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    if c == 0 or k.shape[1] == 0:
        return dq, dk, dv
    has_key = vis.any(axis=1)
    for bi in range(b):
        for h in range(n_q):
            kvh = h // g
            x = np.where(vis, scale * (q[bi, :, h, :] @ k[bi, :, kvh, :].T), -np.inf)
            m = np.where(has_key, x.max(axis=1), 0.0)
            e = np.exp(x - m[:, None])
            p = e / np.where(has_key, e.sum(axis=1), 1.0)[:, None]
            o = p @ v[bi, :, kvh, :]
            D = np.sum(do[bi, :, h, :] * o, axis=1)
            dv[bi, :, kvh, :] += p.T @ do[bi, :, h, :]
            dx = p * (do[bi, :, h, :] @ v[bi, :, kvh, :].T - D[:, None])
            dq[bi, :, h, :] = scale * (dx @ k[bi, :, kvh, :])
            dk[bi, :, kvh, :] += scale * (dx.T @ q[bi, :, h, :])
    return dq, dk, dv


def allgather_attention_bwd(q, k_chunks, v_chunks, do, kind, S, N, rank, doc_ids, causal,
                            scale):
    """Backward of one rank of all-gather CP (§8) under the document mask.

    q, do: [b, c, n_q, d] (the rank's queries, local order); k_chunks,
    v_chunks: [N, b, c, n_kv, d]. Returns dq [b, c, n_q, d] and dk_chunks,
    dv_chunks [N, b, c, n_kv, d]: this rank's contribution to every chunk's
    dK, dV, chunk j in rank j's local order (what the reduce-scatter sums)."""
    k = allgather_kv(k_chunks, kind, S, N)
    v = allgather_kv(v_chunks, kind, S, N)
    q_pos = partition_map(kind, S, N, rank)
    vis = visible_docs(q_pos, np.arange(S), doc_ids, causal)
    dq, dk, dv = masked_attention_bwd(q, k, v, do, vis, scale)
    dk_chunks = np.stack([dk[:, partition_map(kind, S, N, j)] for j in range(N)])
    dv_chunks = np.stack([dv[:, partition_map(kind, S, N, j)] for j in range(N)])
    return dq, dk_chunks, dv_chunks
