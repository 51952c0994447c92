"""ctypes binding of libringattn (include/ringattn.h).

Argument marshalling only: tensors are passed by ``data_ptr()``, streams by
their HIP handle. Every step of the computation runs in the library's HIP
kernels; there is no fallback. If the shared library is missing or fails to
load, every call raises.
"""

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("RINGATTN_LIB", os.path.join(_PKG, "libringattn.so"))

RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_HIP = 0, 1, 2, 3
RA_PART_CONTIGUOUS, RA_PART_ZIGZAG, RA_PART_STRIPED = 0, 1, 2
RA_F32, RA_BF16 = 0, 1
RA_RING_SERIALIZE, RA_RING_UNFUSED_MERGE, RA_RING_OVERLAP, RA_RING_STEPWISE = 1, 2, 4, 8
RA_RING_SERIAL_CHUNK_BYTES = 16 << 20
RA_V_ROWS, RA_V_TRANSPOSED = 0, 1

KINDS = {"contiguous": RA_PART_CONTIGUOUS, "zigzag": RA_PART_ZIGZAG, "striped": RA_PART_STRIPED}

EXPORTED = ("ra_partition", "ra_block_attn_fwd", "ra_v_transpose", "ra_lse_merge",
            "ra_ring_workspace_bytes", "ra_ring_fwd", "ra_attn_bwd_delta", "ra_block_attn_bwd",
            "ra_ring_bwd_workspace_bytes", "ra_ring_bwd", "ra_allgather_workspace_bytes",
            "ra_allgather_fwd", "ra_allgather_bwd_workspace_bytes", "ra_allgather_bwd",
            "ra_ring_fwd_noalloc", "ra_status_str", "ra_last_error")
RA_NOALLOC_SCRATCH_BYTES = 64 << 20


class RingAttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} [status {status}]")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("s_q", ctypes.c_int64), ("s_kv", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
                ("v_layout", ctypes.c_int32), ("q_pos", ctypes.c_void_p),
                ("kv_pos", ctypes.c_void_p), ("q_doc_start", ctypes.c_void_p)]


class RingDesc(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("scale", ctypes.c_float), ("kind", ctypes.c_int32), ("S", ctypes.c_int64),
                ("N", ctypes.c_int32), ("rank", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("step_events", ctypes.c_void_p),
                ("doc_start", ctypes.c_void_p)]


_lib = None


def load_library(path=None):
    """Load libringattn.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RingAttnError(-1, f"libringattn not built: {p} is missing "
                                "(run ring_attention_context_amd.build.build())")
    lib = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.ra_partition.argtypes = [i32, i64, i32, i32, vp]
    lib.ra_block_attn_fwd.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp]
    lib.ra_v_transpose.argtypes = [i32, i64, i32, i32, i32, vp, vp, vp]
    lib.ra_lse_merge.argtypes = [i64, i32, vp, vp, vp, vp, vp]
    lib.ra_ring_workspace_bytes.argtypes = [ctypes.POINTER(RingDesc), ctypes.POINTER(ctypes.c_size_t)]
    lib.ra_ring_fwd.argtypes = [ctypes.POINTER(RingDesc), vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                vp, vp]
    lib.ra_attn_bwd_delta.argtypes = [i64, i32, i32, vp, vp, vp, vp]
    lib.ra_block_attn_bwd.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp]
    lib.ra_ring_bwd_workspace_bytes.argtypes = [ctypes.POINTER(RingDesc),
                                                ctypes.POINTER(ctypes.c_size_t)]
    lib.ra_ring_bwd.argtypes = [ctypes.POINTER(RingDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                ctypes.c_size_t, vp, vp]
    lib.ra_allgather_workspace_bytes.argtypes = [ctypes.POINTER(RingDesc),
                                                 ctypes.POINTER(ctypes.c_size_t)]
    lib.ra_allgather_fwd.argtypes = [ctypes.POINTER(RingDesc), vp, vp, vp, vp, vp, vp,
                                     ctypes.c_size_t, vp]
    lib.ra_allgather_bwd_workspace_bytes.argtypes = [ctypes.POINTER(RingDesc),
                                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.ra_allgather_bwd.argtypes = [ctypes.POINTER(RingDesc), vp, vp, vp, vp, vp, vp, vp, vp,
                                     vp, vp, ctypes.c_size_t, vp]
    lib.ra_ring_fwd_noalloc.argtypes = [ctypes.POINTER(RingDesc), vp, vp, vp, vp, vp, vp]
    for name in ("ra_ring_fwd_noalloc", "ra_partition", "ra_block_attn_fwd", "ra_v_transpose",
                 "ra_lse_merge",
                 "ra_ring_workspace_bytes", "ra_ring_fwd", "ra_attn_bwd_delta",
                 "ra_block_attn_bwd", "ra_ring_bwd_workspace_bytes", "ra_ring_bwd",
                 "ra_allgather_workspace_bytes", "ra_allgather_fwd",
                 "ra_allgather_bwd_workspace_bytes", "ra_allgather_bwd"):
        getattr(lib, name).restype = i32
    lib.ra_status_str.argtypes = [i32]
    lib.ra_status_str.restype = ctypes.c_char_p
    lib.ra_last_error.argtypes = []
    lib.ra_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(status):
    if status != RA_OK:
        lib = load_library()
        msg = lib.ra_last_error().decode() or lib.ra_status_str(status).decode()
        raise RingAttnError(status, msg)


def ra_status_str(status):
    return load_library().ra_status_str(status).decode()


def ra_last_error():
    return load_library().ra_last_error().decode()


def _kind(kind):
    return KINDS[kind] if isinstance(kind, str) else int(kind)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float32:
        return RA_F32
    raise RingAttnError(RA_ERR_UNSUPPORTED, f"unsupported tensor dtype {t.dtype}")


def _need_contiguous(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise RingAttnError(RA_ERR_INVALID_ARG, "tensors must be contiguous")


def ra_partition(kind, S, N, rank):
    """Host call: int32 numpy array of the c = S/N global positions of ``rank``."""
    c = S // N if N > 0 else 0
    out = np.empty(max(c, 0), dtype=np.int32)
    _check(load_library().ra_partition(_kind(kind), S, N, rank,
                                       out.ctypes.data_as(ctypes.c_void_p)))
    return out


def ra_block_attn_fwd(q, k, v, o_b, lse_b, *, causal, scale=0.0, q_pos=None, kv_pos=None,
                      v_transposed=False, q_doc_start=None, stream=None):
    """q [b, s_q, n_q, d], k [b, s_kv, n_kv, d] (bf16 or f32, same dtype); v like k, or
    [b, n_kv, d, s_kv] with ``v_transposed`` (bf16, see :func:`ra_v_transpose`);
    writes o_b float32 [b, s_q, n_q, d] and lse_b float32 [b, s_q, n_q].
    q_pos / kv_pos: int32 device tensors of global positions (causal only).
    q_doc_start: int32 device tensor [s_q], the position where each query's
    document starts (document mask; causal only)."""
    _need_contiguous(q, k, v, o_b, lse_b, q_pos, kv_pos, q_doc_start)
    desc = AttnDesc(b=q.shape[0], n_q=q.shape[2], n_kv=k.shape[2], d=q.shape[3],
                    s_q=q.shape[1], s_kv=k.shape[1], dtype=_dtype_code(q), causal=int(causal),
                    scale=scale, v_layout=RA_V_TRANSPOSED if v_transposed else RA_V_ROWS,
                    q_pos=None if q_pos is None else q_pos.data_ptr(),
                    kv_pos=None if kv_pos is None else kv_pos.data_ptr(),
                    q_doc_start=None if q_doc_start is None else q_doc_start.data_ptr())
    _check(load_library().ra_block_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(o_b), _ptr(lse_b), _stream(stream)))


def ra_v_transpose(v, vt, stream=None):
    """vt [b, n_kv, d, s] <- v [b, s, n_kv, d] (bf16 or f32, moved bit for bit)."""
    _need_contiguous(v, vt)
    b, s, n_kv, d = v.shape
    if tuple(vt.shape) != (b, n_kv, d, s) or vt.dtype != v.dtype:
        raise RingAttnError(RA_ERR_INVALID_ARG, "vt must be [b, n_kv, d, s] of v's dtype")
    _check(load_library().ra_v_transpose(b, s, n_kv, d, _dtype_code(v), _ptr(v), _ptr(vt),
                                         _stream(stream)))


def ra_lse_merge(o, lse, o_b, lse_b, stream=None):
    """In place (o, lse) <- merge((o, lse), (o_b, lse_b)); o [..., d], lse [...]."""
    _need_contiguous(o, lse, o_b, lse_b)
    d = o.shape[-1]
    rows = lse.numel()
    _check(load_library().ra_lse_merge(rows, d, _ptr(o), _ptr(lse), _ptr(o_b), _ptr(lse_b),
                                       _stream(stream)))


def ra_attn_bwd_delta(dout, o, delta, stream=None):
    """delta [..] <- sum over the last axis of dout * o (dout bf16 or f32, o f32)."""
    _need_contiguous(dout, o, delta)
    d = o.shape[-1]
    _check(load_library().ra_attn_bwd_delta(delta.numel(), d, _dtype_code(dout), _ptr(dout),
                                            _ptr(o), _ptr(delta), _stream(stream)))


def ra_block_attn_bwd(q, k, v, dout, lse, delta, dq, dk, dv, *, causal, scale=0.0, q_pos=None,
                      kv_pos=None, q_doc_start=None, stream=None):
    """dq, dk, dv (float32) += the gradient contributions of key block (k, v)
    for queries q with upstream gradient dout, global lse and delta = dout . o
    (q_doc_start: the document mask, as for :func:`ra_block_attn_fwd`)."""
    _need_contiguous(q, k, v, dout, lse, delta, dq, dk, dv, q_pos, kv_pos, q_doc_start)
    desc = AttnDesc(b=q.shape[0], n_q=q.shape[2], n_kv=k.shape[2], d=q.shape[3],
                    s_q=q.shape[1], s_kv=k.shape[1], dtype=_dtype_code(q), causal=int(causal),
                    scale=scale, v_layout=RA_V_ROWS,
                    q_pos=None if q_pos is None else q_pos.data_ptr(),
                    kv_pos=None if kv_pos is None else kv_pos.data_ptr(),
                    q_doc_start=None if q_doc_start is None else q_doc_start.data_ptr())
    _check(load_library().ra_block_attn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq),
                                            _ptr(dk), _ptr(dv), _stream(stream)))


def ring_desc(*, b, n_q, n_kv, d, dtype, causal, kind, S, N, rank, scale=0.0, flags=0,
              step_events=None, doc_start=None):
    """Build the C ring descriptor. ``step_events``: list of N + 1 torch.cuda.Event
    (each already recorded once so that its handle exists). ``doc_start``: int32
    device tensor [S], the first position of every position's document."""
    desc = RingDesc(b=b, n_q=n_q, n_kv=n_kv, d=d, dtype=dtype, causal=int(causal), scale=scale,
                    kind=_kind(kind), S=S, N=N, rank=rank, flags=flags, reserved=0,
                    step_events=None,
                    doc_start=None if doc_start is None else doc_start.data_ptr())
    keep = None
    if step_events is not None:
        keep = (ctypes.c_void_p * len(step_events))(*[e.cuda_event for e in step_events])
        desc.step_events = ctypes.cast(keep, ctypes.c_void_p)
    return desc, keep


def ra_ring_workspace_bytes(desc):
    out = ctypes.c_size_t(0)
    _check(load_library().ra_ring_workspace_bytes(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


def ra_ring_fwd(desc, q, k_chunks, v_chunks, o, lse, workspace, compute=None, copy=None):
    """Ring forward of one rank; see ringattn.h. ``desc`` from :func:`ring_desc`."""
    _need_contiguous(q, k_chunks, v_chunks, o, lse, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().ra_ring_fwd(ctypes.byref(desc), _ptr(q), _ptr(k_chunks),
                                      _ptr(v_chunks), _ptr(o), _ptr(lse), _ptr(workspace),
                                      ws_bytes, _stream(compute), _stream(copy)))


def ra_ring_fwd_noalloc(desc, q, k_chunks, v_chunks, o, lse, stream=None):
    """ra_ring_fwd with the library's static scratch as workspace and the copies
    on ``stream``; allocates nothing (see ringattn.h for the size limit)."""
    _need_contiguous(q, k_chunks, v_chunks, o, lse)
    _check(load_library().ra_ring_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_chunks),
                                              _ptr(v_chunks), _ptr(o), _ptr(lse),
                                              _stream(stream)))


def ra_ring_bwd_workspace_bytes(desc):
    out = ctypes.c_size_t(0)
    _check(load_library().ra_ring_bwd_workspace_bytes(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


_SIDE_STREAMS = {}


def side_stream(device=None):
    """A second stream of the device (default priority), kept for the process:
    the default copy stream of the ring backward."""
    import torch
    dev = torch.cuda.current_device() if device is None else torch.device(device).index
    if dev not in _SIDE_STREAMS:
        _SIDE_STREAMS[dev] = torch.cuda.Stream(device=dev)
    return _SIDE_STREAMS[dev]


def ra_ring_bwd(desc, q, k_chunks, v_chunks, o, lse, dout, dq, dk_chunks, dv_chunks, workspace,
                stream=None, copy=None):
    """Ring backward of one rank; see ringattn.h. dk_chunks / dv_chunks are added to.
    ``copy``: the stream of the travelling block's transfers (default: a side
    stream of q's device; pass ``stream`` itself to serialize)."""
    _need_contiguous(q, k_chunks, v_chunks, o, lse, dout, dq, dk_chunks, dv_chunks, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if copy is None:
        copy = side_stream(q.device)
    _check(load_library().ra_ring_bwd(ctypes.byref(desc), _ptr(q), _ptr(k_chunks),
                                      _ptr(v_chunks), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                      _ptr(dk_chunks), _ptr(dv_chunks), _ptr(workspace),
                                      ws_bytes, _stream(stream), _stream(copy)))


def ra_allgather_workspace_bytes(desc):
    out = ctypes.c_size_t(0)
    _check(load_library().ra_allgather_workspace_bytes(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


def ra_allgather_fwd(desc, q, k_chunks, v_chunks, o, lse, workspace, stream=None):
    """All-gather CP forward of one rank; see ringattn.h. ``desc`` from :func:`ring_desc`."""
    _need_contiguous(q, k_chunks, v_chunks, o, lse, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().ra_allgather_fwd(ctypes.byref(desc), _ptr(q), _ptr(k_chunks),
                                           _ptr(v_chunks), _ptr(o), _ptr(lse), _ptr(workspace),
                                           ws_bytes, _stream(stream)))


def ra_allgather_bwd_workspace_bytes(desc):
    out = ctypes.c_size_t(0)
    _check(load_library().ra_allgather_bwd_workspace_bytes(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


def ra_allgather_bwd(desc, q, k_chunks, v_chunks, o, lse, dout, dq, dk_chunks, dv_chunks,
                     workspace, stream=None):
    """All-gather CP backward of one rank; see ringattn.h. dk_chunks / dv_chunks are added to."""
    _need_contiguous(q, k_chunks, v_chunks, o, lse, dout, dq, dk_chunks, dv_chunks, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().ra_allgather_bwd(ctypes.byref(desc), _ptr(q), _ptr(k_chunks),
                                           _ptr(v_chunks), _ptr(o), _ptr(lse), _ptr(dout),
                                           _ptr(dq), _ptr(dk_chunks), _ptr(dv_chunks),
                                           _ptr(workspace), ws_bytes, _stream(stream)))
