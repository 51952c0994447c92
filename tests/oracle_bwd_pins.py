"""Checks that pin the backward oracle (oracle/backward.py) to facts other than itself.

Each ``pin_*`` takes an object ``B`` exposing the oracle functions
(``naive_attention`` -- the forward, ``naive_attention_bwd``,
``block_attention_bwd``, ``delta``, ``ring_attention_bwd``, ``partition_map``)
and raises AssertionError when the oracle disagrees with the pin.

What pins what:

* finite differences: central differences of L = sum(do * o) through the
  FORWARD oracle give the gradients independently of any backward formula;
* library special case: torch float64 autograd through its CPU
  scaled_dot_product_attention (non-causal, causal, and GQA by repeating K/V
  heads);
* invariants of the softmax gradient: each query's dx sums to 0 over its
  visible keys (sum_j p_j (dp_j - D) = D - D), hence the keys' dk sum to 0;
  zero do gives zero gradients, and the gradients are linear in do;
* the block decomposition of "Context Parallelism and Ring Attention" §3
  (backward paragraph): the blocks' contributions, each with the GLOBAL lse and
  D, add up to the one-shot gradients;
* the ring of §4: summing every rank's per-block dk, dv (and taking each rank's
  dq) reassembles the whole sequence's gradients;
* single visible key: the query at global position 0 (causal) sees only key 0,
  so its p = 1 and dx = do . v_0 - do . o = 0: its dq row is 0.
"""

import numpy as np


def _inputs(rng, b, c, s, n_q, n_kv, d):
    q = rng.standard_normal((b, c, n_q, d))
    k = rng.standard_normal((b, s, n_kv, d))
    v = rng.standard_normal((b, s, n_kv, d))
    do = rng.standard_normal((b, c, n_q, d))
    return q, k, v, do


def _loss(B, q, k, v, do, q_pos, kv_pos, causal, scale):
    o, _ = B.naive_attention(q, k, v, q_pos, kv_pos, causal, scale)
    return float(np.sum(do * o))


def _fd(B, q, k, v, do, q_pos, kv_pos, causal, scale, h=1e-5):
    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        x = base[which]
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            x0 = x[idx]
            x[idx] = x0 + h
            lp = _loss(B, *base, do, q_pos, kv_pos, causal, scale)
            x[idx] = x0 - h
            lm = _loss(B, *base, do, q_pos, kv_pos, causal, scale)
            x[idx] = x0
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


def pin_bwd_finite_differences(B):
    rng = np.random.default_rng(101)
    cases = [
        # c, s, n_q, n_kv, d, causal, q_pos, kv_pos
        (4, 6, 2, 1, 3, False, np.arange(4), np.arange(6)),
        (5, 7, 2, 2, 3, True, np.array([1, 3, 4, 8, 9]), np.array([0, 2, 3, 5, 6, 8, 10])),
        # query 0 sees no key at all (position before every key)
        (3, 4, 4, 2, 2, True, np.array([0, 5, 9]), np.array([2, 4, 6, 8])),
    ]
    for c, s, n_q, n_kv, d, causal, qp, kp in cases:
        q, k, v, do = _inputs(rng, 1, c, s, n_q, n_kv, d)
        scale = 0.7
        dq, dk, dv = B.naive_attention_bwd(q, k, v, do, qp, kp, causal, scale)
        fq, fk, fv = _fd(B, q, k, v, do, qp, kp, causal, scale)
        for got, want, name in ((dq, fq, "dq"), (dk, fk, "dk"), (dv, fv, "dv")):
            err = np.max(np.abs(got - want))
            assert err < 1e-7 + 1e-6 * np.max(np.abs(want)), f"{name} vs finite differences: {err}"


def pin_bwd_torch_autograd(B):
    import torch
    rng = np.random.default_rng(102)
    for causal, n_q, n_kv in ((False, 2, 2), (True, 2, 2), (True, 4, 2), (False, 6, 3)):
        c = s = 9
        d = 5
        q, k, v, do = _inputs(rng, 2, c, s, n_q, n_kv, d)
        scale = 0.4
        g = n_q // n_kv
        tq = torch.tensor(q.transpose(0, 2, 1, 3), requires_grad=True)        # [b, h, s, d]
        tk = torch.tensor(k.transpose(0, 2, 1, 3), requires_grad=True)
        tv = torch.tensor(v.transpose(0, 2, 1, 3), requires_grad=True)
        kk = tk.repeat_interleave(g, dim=1)
        vv = tv.repeat_interleave(g, dim=1)
        out = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, is_causal=causal,
                                                               scale=scale)
        out.backward(torch.tensor(do.transpose(0, 2, 1, 3)))
        pos = np.arange(c)
        dq, dk, dv = B.naive_attention_bwd(q, k, v, do, pos, pos, causal, scale)
        for got, t, name in ((dq, tq, "dq"), (dk, tk, "dk"), (dv, tv, "dv")):
            want = t.grad.numpy().transpose(0, 2, 1, 3)
            err = np.max(np.abs(got - want))
            assert err < 1e-10, f"{name} vs torch autograd (causal={causal}, g={g}): {err}"


def pin_bwd_invariants(B):
    rng = np.random.default_rng(103)
    c, s, n_q, n_kv, d = 11, 13, 4, 2, 6
    q, k, v, do = _inputs(rng, 2, c, s, n_q, n_kv, d)
    qp = np.sort(rng.choice(40, c, replace=False))
    kp = np.sort(rng.choice(40, s, replace=False))
    for causal in (False, True):
        dq, dk, dv = B.naive_attention_bwd(q, k, v, do, qp, kp, causal, 0.3)
        # keys' dk sum to zero (each query's dx sums to zero over its visible keys)
        assert np.max(np.abs(dk.sum(axis=1))) < 1e-10, "sum_j dk_j != 0"
        z = B.naive_attention_bwd(q, k, v, np.zeros_like(do), qp, kp, causal, 0.3)
        assert all(not np.any(t) for t in z), "zero do must give zero gradients"
        two = B.naive_attention_bwd(q, k, v, 2.5 * do, qp, kp, causal, 0.3)
        for a, b2 in zip((dq, dk, dv), two):
            assert np.allclose(2.5 * a, b2, rtol=1e-12, atol=1e-12), "gradients not linear in do"


def pin_bwd_blocks_sum_to_naive(B):
    rng = np.random.default_rng(104)
    c, s, n_q, n_kv, d = 10, 17, 4, 1, 5
    q, k, v, do = _inputs(rng, 1, c, s, n_q, n_kv, d)
    qp = np.sort(rng.choice(50, c, replace=False))
    kp = np.sort(rng.choice(50, s, replace=False))
    for causal in (False, True):
        scale = 0.6
        o, lse = B.naive_attention(q, k, v, qp, kp, causal, scale)
        D = B.delta(o, do)
        want = B.naive_attention_bwd(q, k, v, do, qp, kp, causal, scale)
        for cuts in ([5, 11], [1, 2, 16], list(range(1, s))):
            got = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)]
            bounds = [0] + cuts + [s]
            for lo, hi in zip(bounds[:-1], bounds[1:]):
                part = B.block_attention_bwd(q, k[:, lo:hi], v[:, lo:hi], do, lse, D, qp,
                                             kp[lo:hi], causal, scale)
                got[0] += part[0]
                got[1][:, lo:hi] += part[1]
                got[2][:, lo:hi] += part[2]
            for g_, w_, name in zip(got, want, ("dq", "dk", "dv")):
                err = np.max(np.abs(g_ - w_))
                assert err < 1e-10, f"blocks {cuts} {name}: {err}"


def pin_bwd_ring_all_ranks(B):
    rng = np.random.default_rng(105)
    n_q, n_kv, d = 4, 2, 4
    for kind in ("contiguous", "zigzag", "striped"):
        for N in (1, 2, 4):
            S = 2 * N * 3
            c = S // N
            k = rng.standard_normal((1, S, n_kv, d))
            v = rng.standard_normal((1, S, n_kv, d))
            q_all = rng.standard_normal((1, S, n_q, d))
            do_all = rng.standard_normal((1, S, n_q, d))
            scale = 0.5
            want = B.naive_attention_bwd(q_all, k, v, do_all, np.arange(S), np.arange(S), True,
                                         scale)
            dk = np.zeros_like(k)
            dv = np.zeros_like(v)
            for rank in range(N):
                pos = B.partition_map(kind, S, N, rank)
                q = q_all[:, pos]
                do = do_all[:, pos]
                o, lse = B.naive_attention(q, k, v, pos, np.arange(S), True, scale)
                dq, dkc, dvc = B.ring_attention_bwd(q, k, v, do, o, lse, kind, S, N, rank, True,
                                                    scale)
                assert np.max(np.abs(dq - want[0][:, pos])) < 1e-10, f"{kind} N={N} dq"
                for j in range(N):
                    pj = B.partition_map(kind, S, N, j)
                    dk[:, pj] += dkc[j]
                    dv[:, pj] += dvc[j]
            assert c == len(pos)
            assert np.max(np.abs(dk - want[1])) < 1e-10, f"{kind} N={N} dk"
            assert np.max(np.abs(dv - want[2])) < 1e-10, f"{kind} N={N} dv"


def pin_bwd_single_key(B):
    rng = np.random.default_rng(106)
    c = s = 6
    q, k, v, do = _inputs(rng, 1, c, s, 2, 1, 4)
    pos = np.arange(c)
    dq, dk, dv = B.naive_attention_bwd(q, k, v, do, pos, pos, True, 0.8)
    assert np.max(np.abs(dq[:, 0])) < 1e-12, "query 0 sees one key: its dq must be 0"
    # the last key is seen only by the last query, whose p for it is e^{x - lse}
    o, lse = B.naive_attention(q, k, v, pos, pos, True, 0.8)
    for h in range(2):
        p_last = np.exp(0.8 * q[0, -1, h] @ k[0, -1, 0] - lse[0, -1, h])
        np.testing.assert_allclose(dv[0, -1, 0], sum(
            np.exp(0.8 * q[0, -1, hh] @ k[0, -1, 0] - lse[0, -1, hh]) * do[0, -1, hh]
            for hh in range(2)), rtol=1e-12)
        assert 0 < p_last <= 1


def pin_bwd_rows_dq(B):
    """The row-subset dq equals the full backward's dq on those rows."""
    rng = np.random.default_rng(107)
    for causal in (True, False):
        c, s, n_q, n_kv, d = 9, 14, 6, 2, 5
        q, k, v, do = _inputs(rng, 2, c, s, n_q, n_kv, d)
        qp = np.sort(rng.choice(30, c, replace=False))
        kp = np.sort(rng.choice(30, s, replace=False))
        want = B.naive_attention_bwd(q, k, v, do, qp, kp, causal, 0.4)[0]
        rows = np.array([0, 3, 4, 8])
        got = B.rows_dq(q[:, rows], k, v, do[:, rows], qp[rows], kp, causal, 0.4)
        assert np.max(np.abs(got - want[:, rows])) < 1e-12, f"rows_dq causal={causal}"


BACKWARD_PINS = [pin_bwd_finite_differences, pin_bwd_torch_autograd, pin_bwd_invariants,
                 pin_bwd_blocks_sum_to_naive, pin_bwd_ring_all_ranks, pin_bwd_single_key,
                 pin_bwd_rows_dq]
