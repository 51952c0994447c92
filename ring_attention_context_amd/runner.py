"""Device-side plumbing around ra_ring_fwd: chunk layout, buffers, streams, events.

Reordering K/V into rank-chunk order is the one-time model-entry reordering
("Context Parallelism and Ring Attention" §6, "the cost of reordering"): a
gather by the positions ``ra_partition`` returns, done once with PyTorch
indexing before any timed call. Everything the ring computes runs in
libringattn's kernels.
"""

import ctypes

import numpy as np
import torch

from . import _lib

# hipEventDisableSystemFence: recording the event skips the system-scope fence
# (cache write-back and invalidate) that a default event performs, which at
# the 32K shard's short ring steps costs about 1 % of a call per event pair.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
_HIP = None


def _hip():
    """The HIP runtime PyTorch has loaded (the one libringattn runs on)."""
    global _HIP
    if _HIP is None:
        import glob
        import os
        libs = sorted(glob.glob(os.path.join(os.path.dirname(torch.__file__), "lib",
                                             "libamdhip64.so*")))
        _HIP = ctypes.CDLL(libs[0] if libs else "libamdhip64.so")
    return _HIP


class TimingEvent:
    """A HIP event used only to time work on the device (created with
    hipEventDisableSystemFence). Same interface as the parts of
    torch.cuda.Event used here: ``cuda_event`` (the handle the library records)
    and ``elapsed_time``."""

    def __init__(self):
        self._h = ctypes.c_void_p()
        rc = _hip().hipEventCreateWithFlags(ctypes.byref(self._h),
                                            ctypes.c_uint(HIP_EVENT_DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    @property
    def cuda_event(self):
        return self._h.value

    def elapsed_time(self, end):
        """Milliseconds from this event to ``end`` (both recorded and complete)."""
        ms = ctypes.c_float()
        rc = _hip().hipEventElapsedTime(ctypes.byref(ms), self._h, end._h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        try:
            if self._h.value and _HIP is not None:
                _HIP.hipEventDestroy(self._h)
        except Exception:  # noqa: BLE001  (interpreter shutdown)
            pass


def rank_positions(kind, S, N):
    """[N, c] int32 host array: the global positions of every rank's tokens."""
    return np.stack([_lib.ra_partition(kind, S, N, j) for j in range(N)])


def chunk_kv(x, kind, N):
    """[b, S, n_kv, d] in global order -> [N, b, c, n_kv, d], chunk j = rank j's
    tokens in rank j's local order."""
    b, S = x.shape[0], x.shape[1]
    idx = torch.from_numpy(rank_positions(kind, S, N).reshape(-1).astype(np.int64)).to(x.device)
    g = torch.index_select(x, 1, idx)                     # [b, N*c, n_kv, d]
    return g.view(b, N, S // N, *x.shape[2:]).transpose(0, 1).contiguous()


class RingCall:
    """Buffers and descriptor of one rank's ring forward.

    q: [b, c, n_q, d]; k_chunks, v_chunks: [N, b, c, n_kv, d] (same dtype).
    """

    def __init__(self, q, k_chunks, v_chunks, *, kind, S, N, rank, causal, scale=0.0, flags=0,
                 step_events=False, compute=None, copy=None):
        self.q, self.k, self.v = q, k_chunks, v_chunks
        b, c, n_q, d = q.shape
        n_kv = k_chunks.shape[3]
        dtype = _lib.RA_BF16 if q.dtype == torch.bfloat16 else _lib.RA_F32
        dev = q.device
        self.N = N
        self.compute = compute if compute is not None else torch.cuda.current_stream(dev)
        self.copy = copy if copy is not None else torch.cuda.Stream(dev)
        self.events = None
        if step_events:
            self.events = [TimingEvent() for _ in range(N + 1)]
        self.desc, self._keep = _lib.ring_desc(b=b, n_q=n_q, n_kv=n_kv, d=d, dtype=dtype,
                                               causal=causal, kind=kind, S=S, N=N, rank=rank,
                                               scale=scale, flags=flags,
                                               step_events=self.events)
        ws = _lib.ra_ring_workspace_bytes(self.desc)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.o = torch.empty((b, c, n_q, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((b, c, n_q), dtype=torch.float32, device=dev)

    def make_events(self):
        """A fresh set of N + 1 timing events for the step boundaries of one call."""
        return [TimingEvent() for _ in range(self.N + 1)]

    def __call__(self, events=None):
        """Enqueue one ring forward. ``events``: optional N + 1 events to record
        the step boundaries of this call (instead of the ones given at init)."""
        desc = self.desc
        keep = None
        if events is not None:
            desc = _lib.RingDesc.from_buffer_copy(self.desc)
            keep = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
            desc.step_events = ctypes.cast(keep, ctypes.c_void_p)
        _lib.ra_ring_fwd(desc, self.q, self.k, self.v, self.o, self.lse, self.workspace,
                         compute=self.compute, copy=self.copy)
        del keep
        return self.o, self.lse

    def step_ms(self):
        """Per-step times (ms) of the last call; needs step_events=True and a sync."""
        return [self.events[i].elapsed_time(self.events[i + 1]) for i in range(self.N)]


def doc_start_positions(lengths):
    """int32 host array [S]: for documents of these lengths packed from
    position 0, the first position of every position's document (the
    ``doc_start`` input of ra_ring_fwd / ra_allgather_fwd)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    first = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    return np.repeat(first, lengths).astype(np.int32)


class AllGatherCall:
    """Buffers and descriptor of one rank's all-gather CP forward.

    q: [b, c, n_q, d]; k_chunks, v_chunks: [N, b, c, n_kv, d]; doc_start:
    optional int32 device tensor [S] (document mask).
    """

    def __init__(self, q, k_chunks, v_chunks, *, kind, S, N, rank, causal, scale=0.0,
                 doc_start=None, stream=None):
        self.q, self.k, self.v = q, k_chunks, v_chunks
        b, c, n_q, d = q.shape
        n_kv = k_chunks.shape[3]
        dtype = _lib.RA_BF16 if q.dtype == torch.bfloat16 else _lib.RA_F32
        dev = q.device
        self.stream = stream if stream is not None else torch.cuda.current_stream(dev)
        self.doc_start = doc_start
        self.desc, _ = _lib.ring_desc(b=b, n_q=n_q, n_kv=n_kv, d=d, dtype=dtype, causal=causal,
                                      kind=kind, S=S, N=N, rank=rank, scale=scale,
                                      doc_start=doc_start)
        ws = _lib.ra_allgather_workspace_bytes(self.desc)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
        self.o = torch.empty((b, c, n_q, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((b, c, n_q), dtype=torch.float32, device=dev)

    def __call__(self, events=None):
        """Enqueue one all-gather forward; ``events``: optional 2 events recorded
        around its attention launch."""
        desc = self.desc
        keep = None
        if events is not None:
            desc = _lib.RingDesc.from_buffer_copy(self.desc)
            keep = (ctypes.c_void_p * 2)(*[e.cuda_event for e in events])
            desc.step_events = ctypes.cast(keep, ctypes.c_void_p)
        _lib.ra_allgather_fwd(desc, self.q, self.k, self.v, self.o, self.lse, self.workspace,
                              stream=self.stream)
        del keep
        return self.o, self.lse


def host_to_device(arr, dtype, device="cuda"):
    """Host array -> device tensor; bf16 arrays are given as uint16 bit patterns."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def ring_inputs(q, k, v, dtype, kind, N, device="cuda"):
    """Host q [b, c, n_q, d] (local order) and k, v [b, S, n_kv, d] (global order)
    -> device q and K/V in rank-chunk order [N, b, c, n_kv, d]."""
    qd = host_to_device(q, dtype, device)
    kc = chunk_kv(host_to_device(k, dtype, device), kind, N)
    vc = chunk_kv(host_to_device(v, dtype, device), kind, N)
    return qd, kc, vc
