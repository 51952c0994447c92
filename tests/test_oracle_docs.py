"""The all-gather / document-mask oracle against its pins
(tests/oracle_doc_pins.py), and planted mistakes in it that the pins must
catch. CPU only; touches only the oracle."""

import types

import numpy as np
import pytest

import oracle_doc_pins as pins
from oracle import attention, backward, documents, partition


def namespace():
    """Late-bound view of the oracle: monkeypatched functions are seen."""
    names = ["doc_ids_from_lengths", "doc_start", "visible_docs", "masked_attention",
             "allgather_kv", "allgather_attention", "rows_attention_docs", "doc_visible_pairs",
             "masked_attention_bwd", "allgather_attention_bwd"]
    ns = {n: (lambda n: lambda *a: getattr(documents, n)(*a))(n) for n in names}
    ns["naive_attention"] = lambda *a: attention.naive_attention(*a)
    ns["naive_attention_bwd"] = lambda *a: backward.naive_attention_bwd(*a)
    ns["partition_map"] = lambda *a: partition.partition_map(*a)
    return types.SimpleNamespace(**ns)


@pytest.mark.parametrize("pin", pins.DOC_PINS, ids=lambda p: p.__name__)
def test_doc_oracle_pin(pin):
    pin(namespace())


# ------------------------------------------------------------- planted mistakes

real_visible = documents.visible_docs
real_gather = documents.allgather_kv
real_start = documents.doc_start
real_masked = documents.masked_attention


def visible_earlier_docs(q_pos, kv_pos, ids, causal=True):
    """Lets a query see earlier documents too (<= on document ids)."""
    q_pos, kv_pos, ids = np.asarray(q_pos), np.asarray(kv_pos), np.asarray(ids)
    m = ids[kv_pos][None, :] <= ids[q_pos][:, None]
    return m & (kv_pos[None, :] <= q_pos[:, None]) if causal else m


def visible_no_docs(q_pos, kv_pos, ids, causal=True):
    return partition.visible(q_pos, kv_pos, causal)


def visible_no_causal(q_pos, kv_pos, ids, causal=True):
    return real_visible(q_pos, kv_pos, ids, False)


def gather_shifted(chunks, kind, S, N):
    """Places chunk j at rank (j + 1)'s positions."""
    chunks = np.roll(np.asarray(chunks), 1, axis=0)
    return real_gather(chunks, kind, S, N)


def start_off_by_one(ids):
    s = real_start(ids)
    return np.where(s > 0, s + 1, s)


def masked_no_scale(q, k, v, vis, scale):
    return real_masked(q, k, v, vis, 1.0)


real_masked_bwd = documents.masked_attention_bwd


def masked_bwd_no_delta(q, k, v, do, vis, scale):
    """dx = p * dp (the - D term dropped)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    n_q, n_kv = q.shape[2], k.shape[2]
    g = n_q // n_kv
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for bi in range(q.shape[0]):
        for h in range(n_q):
            kvh = h // g
            x = np.where(vis, scale * (q[bi, :, h] @ k[bi, :, kvh].T), -np.inf)
            m = np.where(vis.any(axis=1), x.max(axis=1), 0.0)
            e = np.exp(x - m[:, None])
            p = e / np.maximum(e.sum(axis=1, keepdims=True), 1e-300)
            dv[bi, :, kvh] += p.T @ do[bi, :, h]
            dx = p * (do[bi, :, h] @ v[bi, :, kvh].T)
            dq[bi, :, h] = scale * dx @ k[bi, :, kvh]
            dk[bi, :, kvh] += scale * dx.T @ q[bi, :, h]
    return dq, dk, dv


def masked_bwd_dk_unscaled(q, k, v, do, vis, scale):
    dq, dk, dv = real_masked_bwd(q, k, v, do, vis, scale)
    return dq, dk / scale, dv


real_ag_bwd = documents.allgather_attention_bwd


def ag_bwd_chunks_rolled(*a):
    dq, dkc, dvc = real_ag_bwd(*a)
    return dq, np.roll(dkc, 1, axis=0), np.roll(dvc, 1, axis=0)


real_rows_docs = documents.rows_attention_docs


def rows_docs_no_causal(q, k, v, qp, ids, causal, scale):
    return real_rows_docs(q, k, v, qp, ids, False, scale)


def rows_docs_shifted_keys(q, k, v, qp, ids, causal, scale):
    """Document mask taken one position off for the keys."""
    vis = documents.visible_docs(qp, np.arange(k.shape[1]), np.roll(ids, 1), causal)
    return documents.masked_attention(q, k, v, vis, scale)


MUTANTS = {
    "rows_docs_no_causal": ("rows_attention_docs", rows_docs_no_causal),
    "rows_docs_shifted_keys": ("rows_attention_docs", rows_docs_shifted_keys),
    "masked_bwd_no_delta": ("masked_attention_bwd", masked_bwd_no_delta),
    "masked_bwd_dk_unscaled": ("masked_attention_bwd", masked_bwd_dk_unscaled),
    "ag_bwd_chunks_rolled": ("allgather_attention_bwd", ag_bwd_chunks_rolled),
    "visible_earlier_docs": ("visible_docs", visible_earlier_docs),
    "visible_no_docs": ("visible_docs", visible_no_docs),
    "visible_no_causal": ("visible_docs", visible_no_causal),
    "gather_shifted": ("allgather_kv", gather_shifted),
    "start_off_by_one": ("doc_start", start_off_by_one),
    "masked_no_scale": ("masked_attention", masked_no_scale),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_doc_pins_catch_planted_mistake(name, monkeypatch):
    fname, fn = MUTANTS[name]
    monkeypatch.setattr(documents, fname, fn)
    caught = []
    for pin in pins.DOC_PINS:
        try:
            pin(namespace())
        except Exception as exc:  # noqa: BLE001 -- any failure counts as caught
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin caught the planted mistake {name}"
