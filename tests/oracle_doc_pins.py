"""Checks that pin the all-gather / document-mask oracle (oracle/documents.py)
to facts other than itself.

Each ``pin_*`` takes an object ``A`` exposing ``naive_attention`` (the primary
forward oracle, pinned on its own by tests/oracle_pins.py), ``partition_map``,
and the functions of oracle/documents.py (``doc_ids_from_lengths``,
``doc_start``, ``visible_docs``, ``masked_attention``, ``allgather_kv``,
``allgather_attention``, ``rows_attention_docs``, ``doc_visible_pairs``); it raises AssertionError when
the oracle disagrees.

What pins what ("Context Parallelism and Ring Attention", §8 all-gather CP):

* independence of documents: attention over the packed sequence under the
  document mask equals plain causal attention run on each document alone
  (positions restarted), concatenated -- the definition of "no attention
  across documents", computed without any document code;
* one document: the mask reduces to the causal rule, so the result equals
  the plain causal oracle;
* every token its own document: a query sees only its own key, so o is its
  own V row and lse its own score;
* brute force: Python loops with math.exp on tiny inputs (the whole
  sequence, and chosen rows through rows_attention_docs);
* the all-gather: gathering the chunks that the §6 maps cut from a sequence
  gives the sequence back bit for bit, for every map;
* zig-zag and striped reordering (§6, masks on original positions): every
  rank's all-gather result, put back at its positions, reassembles the
  whole sequence's document-masked attention;
* pair counts: brute-force counts of the mask, and the closed form
  sum_docs L (L + 1) / 2 over a whole sequence;
* backward: central finite differences of L = sum(do * o) through the
  masked forward; per-document independence against the plain backward
  oracle (oracle/backward.py, pinned on its own) run on each document
  alone; and every rank's all-gather backward, its dq put back at its
  positions and its chunk contributions summed, equals the whole sequence's
  document-masked gradients.
"""

import math

import numpy as np


def _qkv(rng, b, c, s, n_q, n_kv, d):
    return (rng.standard_normal((b, c, n_q, d)), rng.standard_normal((b, s, n_kv, d)),
            rng.standard_normal((b, s, n_kv, d)))


def pin_docs_independent_documents(A):
    rng = np.random.default_rng(201)
    for lengths in ([5, 1, 9, 3], [17], [2, 2, 2, 2, 2, 2], [1, 12, 4]):
        S = sum(lengths)
        q, k, v = _qkv(rng, 2, S, S, 4, 2, 6)
        ids = A.doc_ids_from_lengths(lengths)
        pos = np.arange(S)
        o, lse = A.masked_attention(q, k, v, A.visible_docs(pos, pos, ids, True), 0.45)
        lo = 0
        for L in lengths:
            sl = slice(lo, lo + L)
            rel = np.arange(L)
            o_d, lse_d = A.naive_attention(q[:, sl], k[:, sl], v[:, sl], rel, rel, True, 0.45)
            assert np.max(np.abs(o[:, sl] - o_d)) < 1e-12, f"document {lengths} at {lo}: o"
            assert np.max(np.abs(lse[:, sl] - lse_d)) < 1e-12, f"document {lengths} at {lo}: lse"
            lo += L


def pin_docs_one_document(A):
    rng = np.random.default_rng(202)
    S = 23
    q, k, v = _qkv(rng, 1, S, S, 6, 3, 5)
    ids = A.doc_ids_from_lengths([S])
    pos = np.arange(S)
    for causal in (True, False):
        o, lse = A.masked_attention(q, k, v, A.visible_docs(pos, pos, ids, causal), 0.3)
        o_r, lse_r = A.naive_attention(q, k, v, pos, pos, causal, 0.3)
        assert np.max(np.abs(o - o_r)) < 1e-12 and np.max(np.abs(lse - lse_r)) < 1e-12


def pin_docs_singletons(A):
    rng = np.random.default_rng(203)
    S = 9
    q, k, v = _qkv(rng, 1, S, S, 4, 2, 3)
    ids = A.doc_ids_from_lengths([1] * S)
    pos = np.arange(S)
    o, lse = A.masked_attention(q, k, v, A.visible_docs(pos, pos, ids, True), 0.7)
    for a in range(S):
        for h in range(4):
            assert np.allclose(o[0, a, h], v[0, a, h // 2], rtol=0, atol=1e-14)
            assert abs(lse[0, a, h] - 0.7 * q[0, a, h] @ k[0, a, h // 2]) < 1e-12


def pin_docs_brute_force(A):
    rng = np.random.default_rng(204)
    lengths = [3, 4, 1, 4]
    S = sum(lengths)
    ids = A.doc_ids_from_lengths(lengths)
    q_pos = np.array([1, 4, 7, 8, 11])
    q = rng.standard_normal((1, q_pos.size, 2, 3))
    k = rng.standard_normal((1, S, 1, 3))
    v = rng.standard_normal((1, S, 1, 3))
    scale = 0.6
    o, lse = A.masked_attention(q, k, v, A.visible_docs(q_pos, np.arange(S), ids, True), scale)
    doc_of = []
    for i, L in enumerate(lengths):
        doc_of += [i] * L
    for a, p in enumerate(q_pos):
        for h in range(2):
            xs = [(j, scale * sum(q[0, a, h, e] * k[0, j, 0, e] for e in range(3)))
                  for j in range(S) if doc_of[j] == doc_of[p] and j <= p]
            m = max(x for _, x in xs)
            tot = sum(math.exp(x - m) for _, x in xs)
            want_lse = m + math.log(tot)
            want_o = [sum(math.exp(x - want_lse) * v[0, j, 0, e] for j, x in xs) for e in range(3)]
            assert abs(lse[0, a, h] - want_lse) < 1e-12
            assert np.max(np.abs(o[0, a, h] - want_o)) < 1e-12


def pin_docs_allgather_inverse(A):
    rng = np.random.default_rng(205)
    for kind in ("contiguous", "zigzag", "striped"):
        for N in (1, 2, 4):
            S = 2 * N * 5
            full = rng.standard_normal((2, S, 3, 4))
            chunks = np.stack([full[:, A.partition_map(kind, S, N, j)] for j in range(N)])
            back = A.allgather_kv(chunks, kind, S, N)
            assert np.array_equal(back, full), f"{kind} N={N}"


def pin_docs_ranks_reassemble(A):
    rng = np.random.default_rng(206)
    lengths = [7, 3, 12, 1, 9, 16]
    S = sum(lengths)            # 48 = 2 * 4 * 6
    ids = A.doc_ids_from_lengths(lengths)
    n_q, n_kv, d = 4, 2, 5
    q_all, k, v = _qkv(rng, 1, S, S, n_q, n_kv, d)
    pos = np.arange(S)
    want_o, want_lse = A.masked_attention(q_all, k, v, A.visible_docs(pos, pos, ids, True), 0.5)
    for kind in ("contiguous", "zigzag", "striped"):
        N = 4
        kc = np.stack([k[:, A.partition_map(kind, S, N, j)] for j in range(N)])
        vc = np.stack([v[:, A.partition_map(kind, S, N, j)] for j in range(N)])
        got_o = np.zeros_like(want_o)
        got_lse = np.zeros_like(want_lse)
        for rank in range(N):
            qp = A.partition_map(kind, S, N, rank)
            o, lse = A.allgather_attention(q_all[:, qp], kc, vc, kind, S, N, rank, ids, True, 0.5)
            got_o[:, qp] = o
            got_lse[:, qp] = lse
        assert np.max(np.abs(got_o - want_o)) < 1e-12, kind
        assert np.max(np.abs(got_lse - want_lse)) < 1e-12, kind


def pin_docs_pair_counts(A):
    rng = np.random.default_rng(207)
    for lengths in ([4, 1, 6, 9], [20], [1] * 12, [3, 17, 5]):
        S = sum(lengths)
        ids = A.doc_ids_from_lengths(lengths)
        start = A.doc_start(ids)
        first = np.cumsum([0] + lengths[:-1])
        assert np.array_equal(start, np.repeat(first, lengths)), "document starts"
        for causal in (True, False):
            full = A.doc_visible_pairs(np.arange(S), ids, causal)
            closed = sum(L * (L + 1) // 2 if causal else L * L for L in lengths)
            assert full == closed, (lengths, causal, full, closed)
            qp = np.sort(rng.choice(S, max(1, S // 3), replace=False))
            brute = int(A.visible_docs(qp, np.arange(S), ids, causal).sum())
            assert A.doc_visible_pairs(qp, ids, causal) == brute


def pin_docs_rows(A):
    """rows_attention_docs on chosen rows equals brute force with the document
    mask on those rows, and the rows of the whole-sequence masked result."""
    rng = np.random.default_rng(208)
    lengths = [5, 2, 9, 4, 12]
    S = sum(lengths)
    ids = A.doc_ids_from_lengths(lengths)
    doc_of = np.repeat(np.arange(len(lengths)), lengths)
    q_all, k, v = _qkv(rng, 2, S, S, 4, 2, 3)
    pos = np.arange(S)
    rows = np.array([0, 4, 5, 6, 15, 20, S - 1])
    for causal in (True, False):
        o, lse = A.rows_attention_docs(q_all[:, rows], k, v, pos[rows], ids, causal, 0.65)
        want_o, want_lse = A.masked_attention(q_all, k, v, A.visible_docs(pos, pos, ids, causal),
                                              0.65)
        assert np.max(np.abs(o - want_o[:, rows])) < 1e-12, "rows vs whole-sequence rows"
        assert np.max(np.abs(lse - want_lse[:, rows])) < 1e-12
        for bi in range(2):
            for a, p in enumerate(rows):
                for h in range(4):
                    xs = [(j, 0.65 * sum(q_all[bi, p, h, e] * k[bi, j, h // 2, e] for e in range(3)))
                          for j in range(S) if doc_of[j] == doc_of[p] and (j <= p or not causal)]
                    tot = sum(math.exp(x) for _, x in xs)
                    assert abs(lse[bi, a, h] - math.log(tot)) < 1e-12, "rows brute-force lse"
                    for e in range(3):
                        want = sum(math.exp(x) / tot * v[bi, j, h // 2, e] for j, x in xs)
                        assert abs(o[bi, a, h, e] - want) < 1e-12, "rows brute-force o"


DOC_PINS = [pin_docs_rows, pin_docs_independent_documents, pin_docs_one_document, pin_docs_singletons,
            pin_docs_brute_force, pin_docs_allgather_inverse, pin_docs_ranks_reassemble,
            pin_docs_pair_counts]


def pin_docs_bwd_finite_differences(A):
    rng = np.random.default_rng(208)
    lengths = [3, 1, 4]
    S = sum(lengths)
    ids = A.doc_ids_from_lengths(lengths)
    q_pos = np.array([0, 2, 3, 5, 7])
    q = rng.standard_normal((1, 5, 2, 3))
    k = rng.standard_normal((1, S, 1, 3))
    v = rng.standard_normal((1, S, 1, 3))
    do = rng.standard_normal((1, 5, 2, 3))
    vis = A.visible_docs(q_pos, np.arange(S), ids, True)
    dq, dk, dv = A.masked_attention_bwd(q, k, v, do, vis, 0.8)

    def loss(qq, kk, vv):
        o, _ = A.masked_attention(qq, kk, vv, vis, 0.8)
        return float(np.sum(do * o))

    h = 1e-6
    for which, (x, g) in enumerate(((q, dq), (k, dk), (v, dv))):
        for idx in np.ndindex(x.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += h
            lp = loss(*args)
            args[which][idx] -= 2 * h
            lm = loss(*args)
            assert abs((lp - lm) / (2 * h) - g[idx]) < 1e-6, (which, idx)


def pin_docs_bwd_independent_documents(A):
    rng = np.random.default_rng(209)
    lengths = [6, 1, 9, 4]
    S = sum(lengths)
    ids = A.doc_ids_from_lengths(lengths)
    q, k, v = _qkv(rng, 1, S, S, 4, 2, 5)
    do = rng.standard_normal(q.shape)
    pos = np.arange(S)
    dq, dk, dv = A.masked_attention_bwd(q, k, v, do, A.visible_docs(pos, pos, ids, True), 0.35)
    lo = 0
    for L in lengths:
        sl = slice(lo, lo + L)
        rel = np.arange(L)
        rq, rk, rv = A.naive_attention_bwd(q[:, sl], k[:, sl], v[:, sl], do[:, sl], rel, rel,
                                           True, 0.35)
        for got, want in ((dq[:, sl], rq), (dk[:, sl], rk), (dv[:, sl], rv)):
            assert np.max(np.abs(got - want)) < 1e-12, f"document at {lo}"
        lo += L


def pin_docs_bwd_ranks_reassemble(A):
    rng = np.random.default_rng(210)
    lengths = [5, 11, 2, 14]
    S = sum(lengths)            # 32 = 2 * 4 * 4
    ids = A.doc_ids_from_lengths(lengths)
    q_all, k, v = _qkv(rng, 1, S, S, 4, 2, 3)
    do_all = rng.standard_normal(q_all.shape)
    pos = np.arange(S)
    want = A.masked_attention_bwd(q_all, k, v, do_all, A.visible_docs(pos, pos, ids, True), 0.5)
    for kind in ("contiguous", "zigzag", "striped"):
        N = 4
        kc = np.stack([k[:, A.partition_map(kind, S, N, j)] for j in range(N)])
        vc = np.stack([v[:, A.partition_map(kind, S, N, j)] for j in range(N)])
        dq = np.zeros_like(q_all)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        for rank in range(N):
            qp = A.partition_map(kind, S, N, rank)
            g_q, g_kc, g_vc = A.allgather_attention_bwd(q_all[:, qp], kc, vc, do_all[:, qp], kind,
                                                        S, N, rank, ids, True, 0.5)
            dq[:, qp] = g_q
            for j in range(N):
                pj = A.partition_map(kind, S, N, j)
                dk[:, pj] += g_kc[j]
                dv[:, pj] += g_vc[j]
        for got, w, name in ((dq, want[0], "dq"), (dk, want[1], "dk"), (dv, want[2], "dv")):
            assert np.max(np.abs(got - w)) < 1e-12, f"{kind} {name}"


DOC_PINS += [pin_docs_bwd_finite_differences, pin_docs_bwd_independent_documents,
             pin_docs_bwd_ranks_reassemble]
