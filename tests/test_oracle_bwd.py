"""The backward oracle against its pins (tests/oracle_bwd_pins.py), and planted
mistakes in it that the pins must catch. Everything here runs on the CPU and
touches only the oracle."""

import types

import numpy as np
import pytest

import oracle_bwd_pins as pins
from oracle import attention, backward, partition


def namespace():
    """Late-bound view of the oracle: monkeypatched functions are seen."""
    return types.SimpleNamespace(
        naive_attention=lambda *a: attention.naive_attention(*a),
        naive_attention_bwd=lambda *a: backward.naive_attention_bwd(*a),
        block_attention_bwd=lambda *a: backward.block_attention_bwd(*a),
        delta=lambda *a: backward.delta(*a),
        ring_attention_bwd=lambda *a: backward.ring_attention_bwd(*a),
        rows_dq=lambda *a: backward.rows_dq(*a),
        partition_map=lambda *a: partition.partition_map(*a),
    )


@pytest.mark.parametrize("pin", pins.BACKWARD_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(namespace())


# ------------------------------------------------------------- planted mistakes

real_naive_bwd = backward.naive_attention_bwd
real_block_bwd = backward.block_attention_bwd
real_delta = backward.delta
real_ring_bwd = backward.ring_attention_bwd


def naive_bwd_no_delta(q, k, v, do, qp, kp, causal, scale):
    """dx = p * dp (the - D term dropped)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    b, c, n_q, d = q.shape
    n_kv = k.shape[2]
    g = n_q // n_kv
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    vis = partition.visible(qp, kp, causal)
    for bi in range(b):
        for h in range(n_q):
            kvh = h // g
            x = np.where(vis, scale * q[bi, :, h] @ k[bi, :, kvh].T, -np.inf)
            m = np.max(x, axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.where(vis, np.exp(x - m), 0.0)
            p = e / np.maximum(e.sum(axis=1, keepdims=True), 1e-300)
            dv[bi, :, kvh] += p.T @ do[bi, :, h]
            dx = p * (do[bi, :, h] @ v[bi, :, kvh].T)
            dq[bi, :, h] = scale * dx @ k[bi, :, kvh]
            dk[bi, :, kvh] += scale * dx.T @ q[bi, :, h]
    return dq, dk, dv


def naive_bwd_sign(*a):
    dq, dk, dv = real_naive_bwd(*a)
    return -dq, dk, dv


def naive_bwd_dk_unscaled(q, k, v, do, qp, kp, causal, scale):
    dq, dk, dv = real_naive_bwd(q, k, v, do, qp, kp, causal, scale)
    return dq, dk / scale, dv


def naive_bwd_no_mask(q, k, v, do, qp, kp, causal, scale):
    return real_naive_bwd(q, k, v, do, qp, kp, False, scale)


def block_bwd_local_lse(q, kb, vb, do, lse, D, qp, kp, causal, scale):
    """Uses the block's own log-sum-exp instead of the global one."""
    _, lse_b = attention.block_attention(q, kb, vb, qp, kp, causal, scale)
    return real_block_bwd(q, kb, vb, do, lse_b, D, qp, kp, causal, scale)


def block_bwd_no_mask(q, kb, vb, do, lse, D, qp, kp, causal, scale):
    return real_block_bwd(q, kb, vb, do, lse, D, qp, kp, False, scale)


def delta_with_v_sum(o, do):
    return np.sum(do, axis=-1)


def ring_bwd_wrong_chunk(q, k, v, do, o, lse, kind, S, N, rank, causal, scale):
    dq, dkc, dvc = real_ring_bwd(q, k, v, do, o, lse, kind, S, N, rank, causal, scale)
    return dq, np.roll(dkc, 1, axis=0), np.roll(dvc, 1, axis=0)


real_rows_dq = backward.rows_dq


def rows_dq_no_scale(q, k, v, do, qp, kp, causal, scale):
    return real_rows_dq(q, k, v, do, qp, kp, causal, scale) / scale


MUTANTS = {
    "rows_dq_no_scale": ("rows_dq", rows_dq_no_scale),
    "naive_bwd_no_delta": ("naive_attention_bwd", naive_bwd_no_delta),
    "naive_bwd_sign": ("naive_attention_bwd", naive_bwd_sign),
    "naive_bwd_dk_unscaled": ("naive_attention_bwd", naive_bwd_dk_unscaled),
    "naive_bwd_no_mask": ("naive_attention_bwd", naive_bwd_no_mask),
    "block_bwd_local_lse": ("block_attention_bwd", block_bwd_local_lse),
    "block_bwd_no_mask": ("block_attention_bwd", block_bwd_no_mask),
    "delta_with_v_sum": ("delta", delta_with_v_sum),
    "ring_bwd_wrong_chunk": ("ring_attention_bwd", ring_bwd_wrong_chunk),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_pins_catch_planted_mistake(name, monkeypatch):
    fname, fn = MUTANTS[name]
    monkeypatch.setattr(backward, fname, fn)
    caught = []
    for pin in pins.BACKWARD_PINS:
        try:
            pin(namespace())
        except Exception as exc:  # noqa: BLE001 -- any failure counts as caught
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin caught the planted mistake {name}"
