"""libringattn: one context-parallel rank's Ring Attention forward on MI355X (gfx950).

The compute path is the HIP library ``libringattn.so`` (C ABI in
``include/ringattn.h``); this package only binds it (:mod:`._lib`) and lays
out device tensors for it with PyTorch (:mod:`.runner`). There is no CPU
fallback: without the built library every call raises.
"""

from ._lib import (  # noqa: F401
    EXPORTED,
    KINDS,
    RA_BF16,
    RA_ERR_HIP,
    RA_ERR_INVALID_ARG,
    RA_ERR_UNSUPPORTED,
    RA_F32,
    RA_NOALLOC_SCRATCH_BYTES,
    RA_OK,
    RA_PART_CONTIGUOUS,
    RA_PART_STRIPED,
    RA_PART_ZIGZAG,
    RA_RING_OVERLAP,
    RA_RING_SERIAL_CHUNK_BYTES,
    RA_RING_SERIALIZE,
    RA_RING_STEPWISE,
    RA_RING_UNFUSED_MERGE,
    RA_V_ROWS,
    RA_V_TRANSPOSED,
    LIB_PATH,
    RingAttnError,
    load_library,
    ra_allgather_bwd,
    ra_allgather_bwd_workspace_bytes,
    ra_allgather_fwd,
    ra_allgather_workspace_bytes,
    ra_attn_bwd_delta,
    ra_block_attn_bwd,
    ra_block_attn_fwd,
    ra_last_error,
    ra_lse_merge,
    ra_partition,
    ra_ring_bwd,
    ra_ring_bwd_workspace_bytes,
    ra_ring_fwd,
    ra_ring_fwd_noalloc,
    ra_ring_workspace_bytes,
    ra_status_str,
    ra_v_transpose,
    ring_desc,
    side_stream,
)
