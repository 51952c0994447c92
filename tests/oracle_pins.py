"""Checks that pin the CPU oracle to facts other than itself.

Each ``pin_*`` function takes an object ``O`` exposing the oracle functions
(``naive_attention``, ``rows_attention``, ``block_attention``, ``merge``,
``merge_weights``, ``ring_attention``, ``partition_map``, ``step_work``,
``rank_work``, ``visible_pairs``, ``tile_classes``, ``tile_work_pairs``,
``tile_work_pairs_increasing``, ``tile_step_work``, ``ring_efficiency``,
``causal_adjusted_flops``, ``kv_bytes``) and raises
AssertionError when the oracle disagrees with the pin. The tests run every
pin against the real oracle, and against copies with a planted mistake to
show that the pins catch them.

What pins what (citations: "Context Parallelism and Ring Attention",
hs-black.github.io, unless stated):

* brute force: triple loops with math.exp on tiny inputs (textbook softmax);
* library special case: torch's float64 CPU scaled_dot_product_attention;
* zero-query closed form: q = 0 makes every score 0, so lse = ln(#visible
  keys) and o = the mean of the visible V rows -- exact for every map, step
  and rank; pins the causal mask (§5), the per-block counts and the merge;
* single visible key: the query at global position 0 sees only key 0, so
  o = v_0 and lse = x_00;
* causality: changing keys after a query's position leaves it unchanged;
* merge closed forms (§3 boxed merge): equal lse gives lse + ln 2 and the
  average; the identity (0, -inf) leaves the other side unchanged; weights
  sum to 1 (§3); finite at |lse| = 700 (stable form);
* block-then-merge equals the one-shot softmax (§3 worked example, §4 "after
  N steps every Q has seen all K/V");
* maps and work counts against the numbers the pages print (tests/golden);
* per-rank work against its closed forms (contiguous, zig-zag, striped);
* tile-level work against brute-force loops over tiles and the causal
  triangle B^2 n (n + 1) / 2;
* the FLOP convention against counted multiply-adds, and against the
  communication-hiding thresholds the pages print (§4).
"""

import math

import numpy as np

from golden_values import read


def _rand(shape, rng):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- attention


def brute_force(q, k, v, q_pos, kv_pos, causal, scale):
    """Softmax attention with explicit Python loops and math.exp."""
    b, c, n_q, d = q.shape
    s, n_kv = k.shape[1], k.shape[2]
    g = n_q // n_kv
    o = np.zeros((b, c, n_q, d))
    lse = np.full((b, c, n_q), -math.inf)
    for bi in range(b):
        for a in range(c):
            for h in range(n_q):
                kvh = h // g
                xs = []
                for p in range(s):
                    if causal and kv_pos[p] > q_pos[a]:
                        continue
                    dot = 0.0
                    for e in range(d):
                        dot += float(q[bi, a, h, e]) * float(k[bi, p, kvh, e])
                    xs.append((p, scale * dot))
                if not xs:
                    continue
                denom = sum(math.exp(x) for _, x in xs)
                lse[bi, a, h] = math.log(denom)
                for p, x in xs:
                    w = math.exp(x) / denom
                    for e in range(d):
                        o[bi, a, h, e] += w * float(v[bi, p, kvh, e])
    return o, lse


def pin_bruteforce(O):
    rng = np.random.default_rng(11)
    b, c, s, n_q, n_kv, d = 2, 5, 7, 4, 2, 3
    q = _rand((b, c, n_q, d), rng)
    k = _rand((b, s, n_kv, d), rng)
    v = _rand((b, s, n_kv, d), rng)
    q_pos = np.array([0, 2, 3, 7, 9])
    kv_pos = np.array([0, 1, 4, 5, 6, 8, 9])
    for causal in (False, True):
        o, lse = O.naive_attention(q, k, v, q_pos, kv_pos, causal, 0.7)
        o_bf, lse_bf = brute_force(q, k, v, q_pos, kv_pos, causal, 0.7)
        assert np.allclose(o, o_bf, rtol=0, atol=1e-12), "naive vs brute force (o)"
        assert np.allclose(lse, lse_bf, rtol=0, atol=1e-12), "naive vs brute force (lse)"
        ob, lb = O.block_attention(q, k, v, q_pos, kv_pos, causal, 0.7)
        assert np.allclose(ob, o_bf, rtol=0, atol=1e-12), "block vs brute force (o)"
        assert np.allclose(lb, lse_bf, rtol=0, atol=1e-12), "block vs brute force (lse)"


def pin_torch_sdpa(O):
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(12)
    b, s, n_q, n_kv, d = 1, 24, 4, 2, 16
    q = _rand((b, s, n_q, d), rng)
    k = _rand((b, s, n_kv, d), rng)
    v = _rand((b, s, n_kv, d), rng)
    pos = np.arange(s)
    g = n_q // n_kv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    for causal in (False, True):
        ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)  # scale 1/sqrt(d)
        ref = ref.permute(0, 2, 1, 3).numpy()
        o, _ = O.naive_attention(q, k, v, pos, pos, causal, 1.0 / math.sqrt(d))
        assert np.allclose(o, ref, rtol=0, atol=1e-12), "naive vs torch sdpa"
        scores = (tq @ tk.transpose(-1, -2)) / math.sqrt(d)
        if causal:
            scores = scores.masked_fill(torch.ones(s, s, dtype=torch.bool).triu(1), -math.inf)
        ref_lse = torch.logsumexp(scores, dim=-1).permute(0, 2, 1).numpy()
        _, lse = O.naive_attention(q, k, v, pos, pos, causal, 1.0 / math.sqrt(d))
        assert np.allclose(lse, ref_lse, rtol=0, atol=1e-12), "naive lse vs torch logsumexp"


def pin_zero_query(O):
    """q = 0: every score is 0, so a query at global position P sees P + 1 keys
    (causal) with equal weight: lse = ln(P + 1), o = mean(v[0..P])."""
    rng = np.random.default_rng(13)
    b, n_q, n_kv, d = 1, 2, 1, 4
    for kind in ("contiguous", "zigzag", "striped"):
        for N in (1, 2, 4):
            S = 16 * N
            k = _rand((b, S, n_kv, d), rng)
            v = _rand((b, S, n_kv, d), rng)
            for rank in range(N):
                q_pos = O.partition_map(kind, S, N, rank)
                q = np.zeros((b, len(q_pos), n_q, d))
                o, lse, steps = O.ring_attention(q, k, v, kind, S, N, rank, True, 0.5,
                                                 keep_steps=True)
                for a, P in enumerate(q_pos):
                    assert abs(lse[0, a, 0] - math.log(P + 1)) < 1e-12, "zero-query lse"
                    assert np.allclose(o[0, a, 0], v[0, :P + 1, 0].mean(axis=0), atol=1e-12), \
                        "zero-query o"
                for src, o_b, lse_b in steps:
                    kv_pos = O.partition_map(kind, S, N, src)
                    for a, P in enumerate(q_pos):
                        vis = kv_pos[kv_pos <= P]
                        if vis.size == 0:
                            assert lse_b[0, a, 0] == -math.inf and not o_b[0, a, 0].any(), \
                                "empty block must be (0, -inf)"
                        else:
                            assert abs(lse_b[0, a, 0] - math.log(vis.size)) < 1e-12, \
                                "zero-query block lse"
                            assert np.allclose(o_b[0, a, 0], v[0, vis, 0].mean(axis=0),
                                               atol=1e-12), "zero-query block o"


def pin_single_key(O):
    rng = np.random.default_rng(14)
    S, N, d = 32, 4, 8
    k = _rand((1, S, 1, d), rng)
    v = _rand((1, S, 1, d), rng)
    q = _rand((1, S // N, 1, d), rng)
    for kind in ("contiguous", "zigzag", "striped"):
        o, lse = O.ring_attention(q, k, v, kind, S, N, 0, True, 0.3)
        # local row 0 of rank 0 is global position 0 for every map
        assert abs(lse[0, 0, 0] - 0.3 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-12, "single-key lse"
        assert np.allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-12), "single-key o"


def pin_causality(O):
    rng = np.random.default_rng(15)
    S, N, d = 32, 4, 8
    k = _rand((1, S, 2, d), rng)
    v = _rand((1, S, 2, d), rng)
    for kind in ("contiguous", "zigzag", "striped"):
        rank = 1
        q_pos = O.partition_map(kind, S, N, rank)
        q = _rand((1, len(q_pos), 4, d), rng)
        o, lse = O.ring_attention(q, k, v, kind, S, N, rank, True, 0.4)
        a = len(q_pos) // 2
        P = q_pos[a]
        k2, v2 = k.copy(), v.copy()
        k2[:, P + 1:] += 5.0
        v2[:, P + 1:] -= 3.0
        o2, lse2 = O.ring_attention(q, k2, v2, kind, S, N, rank, True, 0.4)
        assert np.array_equal(o[:, a], o2[:, a]) and np.array_equal(lse[:, a], lse2[:, a]), \
            "future keys changed a causal row"
        later = q_pos > P
        assert not np.allclose(o[:, later], o2[:, later]), "later rows must see the change"


def pin_ring_equals_naive(O):
    rng = np.random.default_rng(16)
    d = 8
    for kind in ("contiguous", "zigzag", "striped"):
        for N in (1, 2, 4, 8):
            S = 16 * N
            k = _rand((1, S, 2, d), rng)
            v = _rand((1, S, 2, d), rng)
            for rank in sorted({0, N // 2, N - 1}):
                q_pos = O.partition_map(kind, S, N, rank)
                q = _rand((1, len(q_pos), 4, d), rng)
                for causal in (True, False):
                    o, lse = O.ring_attention(q, k, v, kind, S, N, rank, causal, 0.35)
                    o_n, lse_n = O.naive_attention(q, k, v, q_pos, np.arange(S), causal, 0.35)
                    assert np.allclose(o, o_n, rtol=0, atol=1e-12), "ring vs naive (o)"
                    assert np.allclose(lse, lse_n, rtol=0, atol=1e-12), "ring vs naive (lse)"


def pin_random_split_merge(O):
    """Two blocks of random membership merged = one softmax over their union."""
    rng = np.random.default_rng(17)
    c, s, d = 6, 20, 5
    q = _rand((1, c, 1, d), rng)
    k = _rand((1, s, 1, d), rng)
    v = _rand((1, s, 1, d), rng)
    pos = np.arange(s)
    for _ in range(5):
        mask = rng.random(s) < 0.5
        b1, b2 = pos[mask], pos[~mask]
        q_pos = np.full(c, s)  # non-causal use: every key visible
        o1, l1 = O.block_attention(q, k[:, b1], v[:, b1], q_pos, b1, False, 0.8)
        o2, l2 = O.block_attention(q, k[:, b2], v[:, b2], q_pos, b2, False, 0.8)
        o, lse = O.merge(o1, l1, o2, l2)
        o_n, lse_n = O.naive_attention(q, k, v, q_pos, pos, False, 0.8)
        assert np.allclose(o, o_n, atol=1e-12) and np.allclose(lse, lse_n, atol=1e-12), \
            "two-block merge must equal the one-shot softmax"


def pin_merge_closed_forms(O):
    rng = np.random.default_rng(18)
    o1 = _rand((3, 4), rng)
    o2 = _rand((3, 4), rng)
    for L in (-700.0, -3.0, 0.0, 2.5, 700.0):
        lse = np.full(3, L)
        o, out = O.merge(o1, lse, o2, lse)
        assert np.allclose(out, L + math.log(2.0), atol=1e-12), "equal-lse merge: lse + ln 2"
        assert np.allclose(o, 0.5 * (o1 + o2), atol=1e-12), "equal-lse merge: average"
        # a block carrying e^{ln 3} more mass gets weight 3/4
        o, out = O.merge(o1, lse, o2, lse + math.log(3.0))
        assert np.allclose(out, L + math.log(4.0), atol=1e-12), "lse of 1:3 merge"
        assert np.allclose(o, 0.25 * o1 + 0.75 * o2, atol=1e-12), "1:3 merge weights"
    ident_o, ident_l = np.zeros((3, 4)), np.full(3, -math.inf)
    lse = np.array([1.0, -2.0, 700.0])
    o, out = O.merge(ident_o, ident_l, o2, lse)
    assert np.array_equal(out, lse) and np.allclose(o, o2, atol=1e-15), "identity on the left"
    o, out = O.merge(o1, lse, ident_o, ident_l)
    assert np.array_equal(out, lse) and np.allclose(o, o1, atol=1e-15), "identity on the right"
    o, out = O.merge(ident_o, ident_l, ident_o, ident_l)
    assert np.all(np.isneginf(out)) and not o.any() and not np.isnan(o).any(), "identity pair"


def pin_merge_weights(O):
    rng = np.random.default_rng(19)
    l1 = rng.uniform(-50, 50, 100)
    l2 = rng.uniform(-50, 50, 100)
    w1, w2 = O.merge_weights(l1, l2)
    assert np.allclose(w1 + w2, 1.0, atol=1e-14), "merge weights sum to 1"
    assert np.all(w1 > 0) and np.all(w2 > 0)
    assert np.allclose(w1 / w2, np.exp(l1 - l2), rtol=1e-12), "weight ratio e^{lse1-lse2}"


def pin_rows_attention(O):
    """rows_attention on chosen rows equals brute force on those rows against
    the whole sequence in global order, and the full naive result's rows."""
    rng = np.random.default_rng(20)
    S, N, d = 24, 4, 3
    k = _rand((2, S, 2, d), rng)
    v = _rand((2, S, 2, d), rng)
    for kind in ("contiguous", "zigzag", "striped"):
        for rank in (0, N - 1):
            q_pos = np.asarray(O.partition_map(kind, S, N, rank))
            q = _rand((2, q_pos.size, 4, d), rng)
            rows = np.array([0, 2, q_pos.size - 1])
            for causal in (True, False):
                o, lse = O.rows_attention(q[:, rows], k, v, q_pos[rows], causal, 0.55)
                o_bf, lse_bf = brute_force(q[:, rows], k, v, q_pos[rows], np.arange(S), causal,
                                           0.55)
                assert np.allclose(o, o_bf, rtol=0, atol=1e-12), "rows vs brute force (o)"
                assert np.allclose(lse, lse_bf, rtol=0, atol=1e-12), "rows vs brute force (lse)"
                o_n, lse_n = O.naive_attention(q, k, v, q_pos, np.arange(S), causal, 0.55)
                assert np.allclose(o, o_n[:, rows], rtol=0, atol=1e-12), "rows vs naive rows"
                assert np.allclose(lse, lse_n[:, rows], rtol=0, atol=1e-12)


ATTENTION_PINS = [pin_rows_attention, pin_bruteforce, pin_torch_sdpa, pin_zero_query, pin_single_key,
                  pin_causality, pin_ring_equals_naive, pin_random_split_merge,
                  pin_merge_closed_forms, pin_merge_weights]


# ---------------------------------------------------------------- partition


def pin_maps_are_permutations(O):
    for kind in ("contiguous", "zigzag", "striped"):
        for N in (1, 2, 3, 4, 8):
            S = 4 * N * 6
            maps = [np.asarray(O.partition_map(kind, S, N, i)) for i in range(N)]
            allpos = np.concatenate(maps)
            assert np.array_equal(np.sort(allpos), np.arange(S)), "maps must partition [0, S)"
            for m in maps:
                assert len(m) == S // N and np.all(np.diff(m) > 0), "map strictly increasing"


def pin_map_definitions(O):
    S, N = 64, 4
    c, h = S // N, S // (2 * N)
    for i in range(N):
        assert np.array_equal(O.partition_map("contiguous", S, N, i), np.arange(i * c, (i + 1) * c))
        assert np.array_equal(O.partition_map("striped", S, N, i),
                              [p for p in range(S) if p % N == i])
    z0 = O.partition_map("zigzag", S, N, 0)
    assert set(z0) == set(range(0, h)) | set(range(S - h, S)), "rank 0: first and last chunk"
    zl = O.partition_map("zigzag", S, N, N - 1)
    assert set(zl) == set(range((N - 1) * h, (N + 1) * h)), "rank N-1: the middle two chunks"


def pin_n4_rank_work(O):
    gold = read("ring_n4_rank_work.txt")
    N = int(gold["N"][0])
    for c in (8, 32, 128):
        S, unit = N * c, (c // 2) ** 2
        for kind in ("contiguous", "zigzag"):
            per_rank = np.asarray(O.rank_work(kind, S, N))
            assert np.array_equal(per_rank, np.asarray(O.step_work(kind, S, N)).sum(axis=1))
            # the figure counts each chunk's own diagonal block as half a block;
            # the exact count adds the diagonal itself: c/2 pairs per rank
            units = (per_rank - c // 2) / unit
            assert np.array_equal(units, [int(x) for x in gold[kind]]), (kind, units)


def pin_contiguous_efficiency(O):
    gold = read("ring_contiguous_efficiency.txt")
    for N, key in ((4, "N4_percent"), (8, "N8_percent")):
        c = 512
        eta = O.ring_efficiency(O.step_work("contiguous", N * c, N))
        assert round(100 * eta) == int(gold[key][0]), (N, eta)
        assert abs(eta - N / (2 * N - 1)) < 2.0 / c, "eta -> N / (2N - 1)"
        ez = O.ring_efficiency(O.step_work("zigzag", N * c, N))
        assert abs(ez - 1.0) < 1e-12, "zig-zag is perfectly balanced"
        # zig-zag is about 2 - 1/N times faster than the contiguous split
        tc = np.asarray(O.step_work("contiguous", N * c, N)).max(axis=0).sum()
        tz = np.asarray(O.step_work("zigzag", N * c, N)).max(axis=0).sum()
        assert abs(tc / tz - (2 - 1 / N)) < 4.0 / c


def pin_zigzag_table(O):
    gold = read("zigzag_step_table.txt")
    outcome = {"full": lambda blk: blk.all(),
               "skip": lambda blk: not blk.any(),
               "diag": lambda blk: blk.any() and not blk.all()}
    for N in (2, 4, 8):
        h = 6
        S = 2 * N * h
        for i in range(N):
            qmap = np.asarray(O.partition_map("zigzag", S, N, i))
            q_half = {"early": qmap[:h], "late": qmap[h:]}
            for j in range(N):
                kmap = np.asarray(O.partition_map("zigzag", S, N, j))
                k_half = {"early": kmap[:h], "late": kmap[h:]}
                col = 0 if j < i else (1 if j == i else 2)
                for key, vals in gold.items():
                    qh, kh = key.split()
                    blk = k_half[kh][None, :] <= q_half[qh][:, None]
                    assert outcome[vals[col]](blk), (N, i, j, key)
                pairs = O.visible_pairs(qmap, kmap)
                assert pairs == (2 * h * h if j != i else 2 * h * h + h), "c^2/2 per step"


def pin_zigzag_rectangles(O):
    """j < i: all queries x the first half of the keys; j > i: the second half of
    the queries x all keys (both unmasked rectangles); only j = i needs a mask."""
    N, h = 4, 5
    S = 2 * N * h
    for i in range(N):
        qmap = np.asarray(O.partition_map("zigzag", S, N, i))
        for j in range(N):
            kmap = np.asarray(O.partition_map("zigzag", S, N, j))
            vis = kmap[None, :] <= qmap[:, None]
            rect = np.zeros_like(vis)
            if j < i:
                rect[:, :h] = True
            elif j > i:
                rect[h:, :] = True
            else:
                continue
            assert np.array_equal(vis, rect), (i, j)


def pin_striped_balance(O):
    for N in (2, 4, 8):
        c = 10
        S = N * c
        per_rank = np.asarray(O.step_work("striped", S, N)).sum(axis=1)
        # rank i owns a*N + i: key b*N + j is visible iff b < a or (b == a and j <= i)
        expect = [N * c * (c - 1) // 2 + c * (i + 1) for i in range(N)]
        assert np.array_equal(per_rank, expect), "striped per-rank work"
        assert per_rank.max() - per_rank.min() == c * (N - 1), "differs only on the diagonal"
        eta = O.ring_efficiency(O.step_work("striped", S, N))
        assert abs(eta - (N * c + 1) / (N * c + N)) < 1e-12


def pin_causal_triangle_tiles(O):
    """One contiguous rank (N = 1) with square tiles is the textbook causal
    triangle: tiles below the diagonal full, on it diagonal, above it skipped."""
    S, B = 40, 8
    pos = O.partition_map("contiguous", S, 1, 0)
    cls = np.asarray(O.tile_classes(pos, pos, B, B))
    n = S // B
    for a in range(n):
        for t in range(n):
            want = 1 if t < a else (2 if t == a else 0)
            assert cls[a, t] == want, (a, t)


def pin_kv_bytes(O):
    gold = read("kv_buffer_bytes.txt")
    b, s, n_kv, d = (int(gold[x][0]) for x in ("b", "s", "n_kv", "d_h"))
    assert O.kv_bytes(b, s, n_kv, d) == int(gold["full_MiB"][0]) << 20
    assert O.kv_bytes(b, s, n_kv // 8, d) == int(gold["tp8_MiB"][0]) << 20


def pin_rank_work_closed_forms(O):
    """Per-rank visible pairs (§5, §6): contiguous rank i sees all of the i
    earlier segments plus its own triangle, i c^2 + c (c + 1) / 2; zig-zag
    gives every rank S c / 2 + c / 2; striped rank i (positions a N + i) sees
    N c (c - 1) / 2 + c (i + 1). Non-causal: c S for every rank."""
    for N in (1, 2, 3, 4, 8):
        for c in (2, 6, 10):
            S = N * c
            cont = np.asarray(O.rank_work("contiguous", S, N))
            assert np.array_equal(cont, [i * c * c + c * (c + 1) // 2 for i in range(N)])
            stri = np.asarray(O.rank_work("striped", S, N))
            assert np.array_equal(stri, [N * c * (c - 1) // 2 + c * (i + 1) for i in range(N)])
            zz = np.asarray(O.rank_work("zigzag", S, N))
            assert np.array_equal(zz, [S * c // 2 + c // 2] * N)
            for kind in ("contiguous", "zigzag", "striped"):
                assert np.array_equal(np.asarray(O.rank_work(kind, S, N, False)), [c * S] * N)


def _brute_tile_slots(q_pos, kv_pos, Bq, Bk, causal):
    """Element slots of tiles holding at least one visible pair, by loops."""
    total = 0
    for a0 in range(0, len(q_pos), Bq):
        for t0 in range(0, len(kv_pos), Bk):
            qs = q_pos[a0:a0 + Bq]
            ks = kv_pos[t0:t0 + Bk]
            if any((not causal) or kp <= qp for qp in qs for kp in ks):
                total += len(qs) * len(ks)
    return total


def pin_tile_work(O):
    """Tile-level work (§7: kernels skip whole tiles): brute-force loops over
    tiles; the causal triangle of one contiguous rank with square tiles,
    B^2 n (n + 1) / 2; the per-step table against those counts."""
    rng = np.random.default_rng(21)
    for _ in range(20):
        c, s = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        q_pos = np.sort(rng.choice(100, c, replace=False))
        kv_pos = np.sort(rng.choice(100, s, replace=False))
        Bq, Bk = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        for causal in (True, False):
            want = _brute_tile_slots(q_pos, kv_pos, Bq, Bk, causal)
            assert O.tile_work_pairs(q_pos, kv_pos, Bq, Bk, causal) == want, "tile_work_pairs"
        assert O.tile_work_pairs_increasing(q_pos, kv_pos, Bq, Bk) == \
            _brute_tile_slots(q_pos, kv_pos, Bq, Bk, True), "tile_work_pairs_increasing"
    for n, B in ((1, 4), (5, 8), (7, 3)):
        pos = np.arange(n * B)
        assert O.tile_work_pairs(pos, pos, B, B) == B * B * n * (n + 1) // 2, "triangle"
        assert O.tile_work_pairs_increasing(pos, pos, B, B) == B * B * n * (n + 1) // 2
    for kind in ("contiguous", "zigzag", "striped"):
        for N in (1, 2, 4):
            S = 2 * N * 12
            W = np.asarray(O.tile_step_work(kind, S, N, 4, 8))
            for i in range(N):
                q_pos = O.partition_map(kind, S, N, i)
                for r, src in enumerate(O.ring_sources(i, N)):
                    kv_pos = O.partition_map(kind, S, N, src)
                    assert W[i, r] == _brute_tile_slots(q_pos, kv_pos, 4, 8, True), (kind, i, r)


def _brute_flops(b, c, s, n_q, d, q_pos, kv_pos, causal):
    """Floating-point operations of the two matmuls, counted one multiply-add
    (2 flops) at a time over every visible pair: d for the score q . k and d
    for the output row p v."""
    fl = 0
    for _ in range(b):
        for a in range(c):
            for _h in range(n_q):
                for j in range(s):
                    if causal and kv_pos[j] > q_pos[a]:
                        continue
                    fl += 2 * d      # q . k
                    fl += 2 * d      # p * v accumulated into o
    return fl


def pin_causal_adjusted_flops(O):
    """The FLOP convention (§4): counted multiply-adds of the two matmuls over
    the visible pairs; and the page's hiding thresholds c = (C/W) n_kv / n_h
    (H100 node and cross-node, MHA and GQA 8/64), where the block's math
    (causal_adjusted_flops of a full c x c block) equals its K/V transfer
    (kv_bytes of one chunk)."""
    b, n_q, d = 2, 3, 5
    q_pos, kv_pos = np.array([1, 4, 6, 9]), np.array([0, 2, 4, 5, 7, 8, 10])
    for causal in (True, False):
        pairs = O.visible_pairs(q_pos, kv_pos, causal)
        assert O.causal_adjusted_flops(b, n_q, d, pairs) == \
            _brute_flops(b, len(q_pos), len(kv_pos), n_q, d, q_pos, kv_pos, causal)
    gold = {k: float(v[0]) for k, v in read("comm_hiding_threshold.txt").items()}
    C = gold["C_flops"]
    d_h, n_h = 128, 64
    for W, mha, gqa in ((gold["W_node_Bps"], gold["node_mha_tokens"], gold["node_gqa_8_64_tokens"]),
                        (gold["W_cross_Bps"], gold["cross_mha_tokens"],
                         gold["cross_gqa_8_64_tokens"])):
        for n_kv, want in ((n_h, mha), (8, gqa)):
            # T_math(c) = flops(c^2 pairs) / C grows as c^2, T_comm(c) = bytes(c) / W as c:
            # they meet at c* = (bytes per token / W) / (flops per pair / C)
            per_pair = O.causal_adjusted_flops(1, n_h, d_h, 1)
            per_token = O.kv_bytes(1, 1, n_kv, d_h)
            c_star = (per_token / W) / (per_pair / C)
            assert abs(c_star - want) / want < 0.02, (W, n_kv, c_star, want)


PARTITION_PINS = [pin_rank_work_closed_forms, pin_tile_work, pin_causal_adjusted_flops,
                  pin_maps_are_permutations, pin_map_definitions, pin_n4_rank_work,
                  pin_contiguous_efficiency, pin_zigzag_table, pin_zigzag_rectangles,
                  pin_striped_balance, pin_causal_triangle_tiles, pin_kv_bytes]
