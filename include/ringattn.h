/*
 * libringattn -- one context-parallel rank's Ring Attention forward on an
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow "Context Parallelism and Ring Attention"
 * (hs-black.github.io, posts/scaling-context-parallel):
 *   - ra_partition       -- §2 (contiguous split) and §6 (zig-zag, striped);
 *   - ra_block_attn_fwd  -- §3 block statistics (m_b, l_b, o_b, lse_b) of one
 *                           key block, with the §5 causal rule on original
 *                           positions (§6 "the cost of reordering");
 *   - ra_lse_merge       -- §3 boxed two-block merge, stable form;
 *   - ra_ring_fwd        -- §4 ring loop: N steps, step r uses the K/V of
 *                           rank (rank - r) mod N, each block merged into the
 *                           running (o, lse). On one GPU the neighbour's send
 *                           becomes a device-to-device prefetch into a double
 *                           buffer (§4 "memory": six blocks, double-buffered).
 *   - ra_allgather_fwd   -- §8 all-gather CP: the K/V of all ranks gathered
 *                           into the whole sequence, then one pass of the
 *                           rank's queries over it, optionally under the
 *                           document mask (no attention across documents).
 * With N = 1 the ring call is a single dense pass: the local attention of one
 * rank after the DeepSpeed-Ulysses all-to-all (§9; "DeepSpeed-Ulysses and
 * hybrids", t6page.pages.dev: full sequence, h/N heads).
 *
 * Conventions shared by every call:
 *   - Layouts are contiguous [b, s, heads, d] for q, k, v, o, o_b, and
 *     [b, s, n_q] for lse, lse_b. o, o_b, lse and lse_b are always float32.
 *   - Query head h reads key/value head h / (n_q / n_kv) (GQA groups are
 *     contiguous runs of query heads).
 *   - lse is a natural logarithm. A query that sees no key gets o = 0 and
 *     lse = -inf exactly; (0, -inf) is the identity of the merge.
 *   - Causal rule: key at global position p is visible to a query at global
 *     position P iff p <= P (diagonal included).
 *   - Device pointers must be 16-byte aligned. The caller owns every buffer;
 *     the library allocates no device memory.
 *   - Calls that take a stream are stream-ordered and return once the work
 *     is enqueued. Argument errors are reported before anything is enqueued
 *     (RA_ERR_INVALID_ARG / RA_ERR_UNSUPPORTED); a failed HIP call returns
 *     RA_ERR_HIP. Faults inside kernels surface at the caller's next
 *     synchronisation. ra_last_error() gives the message of the last failure
 *     on the calling thread.
 *   - Streams are hipStream_t values passed as void* (NULL = default stream).
 */
#ifndef RINGATTN_H
#define RINGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_ERR_INVALID_ARG = 1,  /* bad size, pointer, alignment or divisibility   */
  RA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (dtype / head dim)   */
  RA_ERR_HIP = 3           /* a HIP runtime call failed; see ra_last_error() */
} ra_status;

typedef enum {
  RA_PART_CONTIGUOUS = 0,  /* rank i owns positions [i*c, (i+1)*c)            */
  RA_PART_ZIGZAG = 1,      /* rank i owns chunks C_i and C_{2N-1-i} of c/2    */
  RA_PART_STRIPED = 2      /* rank i owns positions p with p mod N == i       */
} ra_partition_kind;

typedef enum { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

/* Layout of v in ra_block_attn_fwd. */
typedef enum {
  RA_V_ROWS = 0,        /* [b, s_kv, n_kv, d], the layout of k                */
  RA_V_TRANSPOSED = 1   /* [b, n_kv, d, s_kv]: element (i, s, h, e) at
                           ((i*n_kv + h)*d + e)*s_kv + s; bf16 only, and
                           s_kv % 8 == 0 (16-byte aligned rows), else
                           RA_ERR_INVALID_ARG; d * s_kv * 2 < 2^31 bytes (the
                           d rows of one head within 31-bit buffer offsets,
                           s_kv < 8,388,608 at d = 128), else
                           RA_ERR_UNSUPPORTED. Produced by ra_v_transpose.
                           The kernel then reads V^T tiles with plain
                           16-byte LDS reads.                                */
} ra_v_layout;

/*
 * ra_partition -- global positions of the c = S/N tokens rank `rank` owns, in
 * its local order ("Context Parallelism and Ring Attention" §2, §6).
 *   contiguous: pos[a] = rank*c + a
 *   zigzag:     the sequence is cut into 2N chunks of h = c/2 tokens; rank i
 *               holds C_i then C_{2N-1-i}, each ascending:
 *               pos[a] = i*h + a (a < h), (2N-1-i)*h + (a-h) (a >= h)
 *   striped:    token p goes to rank p mod N: pos[a] = a*N + rank
 * Every map is strictly increasing in a, and the N maps partition [0, S).
 * out_pos: HOST array of c int32, written by the call. Needs S < 2^31,
 * N >= 1, 0 <= rank < N, S % N == 0, and S % (2N) == 0 for zig-zag; the
 * pages do not treat remainders, so they are RA_ERR_INVALID_ARG.
 * Makes no HIP call (usable without a GPU).
 */
ra_status ra_partition(int32_t kind, int64_t S, int32_t N, int32_t rank, int32_t *out_pos);

/* One block of keys against a query shard. */
typedef struct ra_attn_desc {
  int32_t b;          /* batch                                               */
  int32_t n_q;        /* query heads                                         */
  int32_t n_kv;       /* key/value heads; n_q % n_kv == 0                    */
  int32_t d;          /* head dim: 128 for bf16; 64 or 128 for f32           */
  int64_t s_q;        /* query rows (tokens) of the shard, >= 0              */
  int64_t s_kv;       /* key rows of the block, >= 0                         */
  int32_t dtype;      /* ra_dtype of q, k and v                              */
  int32_t causal;     /* 1: apply the causal rule on q_pos / kv_pos          */
  float scale;        /* softmax scale; 0 selects 1/sqrt(d); must be >= 0    */
  int32_t v_layout;   /* ra_v_layout of v (RA_V_ROWS unless stated)         */
  const int32_t *q_pos;   /* device [s_q] global positions, non-decreasing   */
  const int32_t *kv_pos;  /* device [s_kv] global positions, non-decreasing  */
  const int32_t *q_doc_start;  /* device [s_q] or NULL: document mask. The
                           global position where the query's document starts
                           (<= its q_pos, non-decreasing); a key is visible
                           only if q_doc_start <= kv_pos. Needs causal = 1.  */
} ra_attn_desc;

/*
 * ra_block_attn_fwd -- block statistics of "Context Parallelism and Ring
 * Attention" §3 for the keys of one block:
 *   m_b = max x, l_b = sum e^{x - m_b}, o_b = (1/l_b) sum e^{x - m_b} v,
 *   lse_b = m_b + ln l_b,  x = scale * q.k  over the keys visible to the query.
 * q: device [b, s_q, n_q, d]; k: device [b, s_kv, n_kv, d] (dtype);
 * v: device [b, s_kv, n_kv, d], or [b, n_kv, d, s_kv] with RA_V_TRANSPOSED;
 * o_b: device float32 [b, s_q, n_q, d]; lse_b: device float32 [b, s_q, n_q],
 * both fully overwritten. Rows with no visible key get (0, -inf).
 * q_pos / kv_pos are read only when causal; positions out of order give
 * unspecified values (never an out-of-bounds access).
 * With q_doc_start, key j is visible to query a iff
 * q_doc_start[a] <= kv_pos[j] <= q_pos[a]: the causal rule plus the
 * document mask of §8 when documents are runs of consecutive positions.
 */
ra_status ra_block_attn_fwd(const ra_attn_desc *desc, const void *q, const void *k,
                            const void *v, float *o_b, float *lse_b, void *stream);

/*
 * ra_v_transpose -- vt <- v with the token and channel axes exchanged per
 * head: v [b, s, n_kv, d] -> vt [b, n_kv, d, s] (the RA_V_TRANSPOSED layout
 * of ra_block_attn_fwd). Values are moved bit for bit, not converted.
 * dtype RA_BF16 or RA_F32; v and vt are device buffers of b*s*n_kv*d
 * elements that must not overlap. b * n_kv <= 65535.
 */
ra_status ra_v_transpose(int32_t b, int64_t s, int32_t n_kv, int32_t d, int32_t dtype,
                         const void *v, void *vt, void *stream);

/*
 * ra_lse_merge -- in place (o, lse) <- merge((o, lse), (o_b, lse_b)), the
 * boxed merge of "Context Parallelism and Ring Attention" §3 in its stable
 * form: M = max(lse, lse_b), lse' = M + ln(e^{lse-M} + e^{lse_b-M}),
 * o' = e^{lse-lse'} o + e^{lse_b-lse'} o_b. A row with lse = lse_b = -inf
 * becomes (0, -inf).
 * rows: number of (token, head) rows; o, o_b: device float32 [rows, d],
 * 16-byte aligned; lse, lse_b: device float32 [rows]. d must be a power of
 * two in [4, 256]. Returns RA_ERR_INVALID_ARG for rows < 0, another d, a NULL
 * or misaligned pointer (rows == 0 is a no-op that reads no pointer).
 */
ra_status ra_lse_merge(int64_t rows, int32_t d, float *o, float *lse, const float *o_b,
                       const float *lse_b, void *stream);

/* ra_ring_desc.flags */
#define RA_RING_SERIALIZE 1      /* run the K/V prefetch copies on `compute`  */
#define RA_RING_UNFUSED_MERGE 2  /* write (o_b, lse_b) to the workspace and
                                    merge with ra_lse_merge's kernel, instead
                                    of merging in the attention epilogue     */
#define RA_RING_OVERLAP 4        /* ra_ring_fwd: run the copies on `copy` also
                                    for chunks of at most
                                    RA_RING_SERIAL_CHUNK_BYTES                */
#define RA_RING_STEPWISE 8       /* ra_ring_fwd: one attention launch per step
                                    also when the copies run on `compute`
                                    (see ra_ring_fwd)                        */
/* ra_ring_fwd runs the copies of K chunks up to this size on `compute` unless
 * RA_RING_OVERLAP is set: between two short steps the wait for the other
 * stream costs more than the copy itself. */
#define RA_RING_SERIAL_CHUNK_BYTES ((size_t)16 << 20)

typedef struct ra_ring_desc {
  int32_t b, n_q, n_kv, d;  /* as in ra_attn_desc                            */
  int32_t dtype;            /* ra_dtype of q and the K/V chunks              */
  int32_t causal;           /* 1: causal rule on global positions            */
  float scale;              /* 0 selects 1/sqrt(d)                           */
  int32_t kind;             /* ra_partition_kind of the sequence split       */
  int64_t S;                /* total tokens of the sequence                  */
  int32_t N;                /* ring size (context-parallel degree), >= 1     */
  int32_t rank;             /* the rank whose queries are computed           */
  int32_t flags;            /* RA_RING_* bits                                */
  int32_t reserved;         /* must be 0                                     */
  void **step_events;       /* optional: N+1 hipEvent_t, recorded on
                               `compute` before step 0 and after each step   */
  const int32_t *doc_start; /* optional device [S]: document mask (§8). For
                               every global position p, the first position
                               of p's document (0 <= doc_start[p] <= p,
                               non-decreasing: documents are runs of
                               consecutive positions). A key is visible only
                               within the query's document. Needs causal = 1.
                               Taken by the ring and all-gather calls, both
                               passes.                                       */
} ra_ring_desc;

/* Workspace bytes ra_ring_fwd needs for *desc (same validation as the call). */
ra_status ra_ring_workspace_bytes(const ra_ring_desc *desc, size_t *bytes);

/*
 * ra_ring_fwd -- the ring loop of "Context Parallelism and Ring Attention" §4
 * for rank `rank`, replayed on one GPU.
 * q:        device [b, c, n_q, d], the rank's tokens in its local order
 *           (c = S/N; see ra_partition for the order).
 * k_chunks, v_chunks: device [N, b, c, n_kv, d]; chunk j holds rank j's
 *           tokens in rank j's local order.
 * o, lse:   device float32 [b, c, n_q, d] and [b, c, n_q], overwritten with
 *           the merged result over all N blocks.
 * workspace: device, >= ra_ring_workspace_bytes(); holds the double buffer
 *           for the incoming K/V chunk and the position maps. Its contents on
 *           entry do not matter. For bf16 with c % 8 == 0 (and c < 8,388,608
 *           at d = 128, the RA_V_TRANSPOSED limit) the V half of each buffer
 *           holds the chunk transposed (RA_V_TRANSPOSED, written by the copy
 *           stream), including the rank's own chunk before step 0; otherwise
 *           V stays row-major.
 * Step r computes the block of chunk (rank - r) mod N; the copy of the next
 * step's chunk into the idle half of the double buffer runs on `copy` while
 * step r computes on `compute` (on `compute` with RA_RING_SERIALIZE, when
 * copy == compute, or when a K chunk is at most RA_RING_SERIAL_CHUNK_BYTES
 * and RA_RING_OVERLAP is not set; RA_RING_SERIALIZE with RA_RING_OVERLAP is
 * RA_ERR_INVALID_ARG).
 * When the copies run on `compute` (bf16 with V staged transposed, merge
 * fused, no document mask, RA_RING_STEPWISE not set), two consecutive steps
 * whose blocks the rank can see share one attention launch: the kernel scans
 * the keys of both blocks in one online softmax (§3: the same identity
 * applied within one GPU) and merges into (o, lse) once. The result equals
 * the stepwise one up to rounding (the order in which the two blocks'
 * statistics combine); both steps' events are recorded after that launch.
 * A causal step whose block no query of the rank can see (with the
 * contiguous map, every later rank's chunk) launches no kernel: merging its
 * statistics would be the identity. Its chunk still arrives on `copy`, as the
 * ring forwards it; its step event is recorded as usual.
 * After the call the workspace's first S int32 hold the position map of
 * every rank (rank j's c positions at [j*c, (j+1)*c)), as ra_partition
 * gives them.
 * On return all work is enqueued and `compute` is ordered after every copy;
 * `copy` first waits for the work already enqueued on `compute`.
 * Calls that share a workspace must be ordered on `compute`.
 */
ra_status ra_ring_fwd(const ra_ring_desc *desc, const void *q, const void *k_chunks,
                      const void *v_chunks, float *o, float *lse, void *workspace,
                      size_t workspace_bytes, void *compute, void *copy);

/* Size of the static device scratch of ra_ring_fwd_noalloc (64 MiB per GPU). */
#define RA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * ra_ring_fwd_noalloc -- ra_ring_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments and result as ra_ring_fwd, without the
 * workspace: the workspace is a static device array of
 * RA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends, and the chunk copies run on `stream` (as with
 * RA_RING_SERIALIZE). No call allocates memory, creates a stream or an event.
 * Returns RA_ERR_INVALID_ARG, before enqueueing anything, when
 * ra_ring_workspace_bytes(desc) exceeds RA_NOALLOC_SCRATCH_BYTES (for
 * example the 32K Llama-3-8B shard fits: about 33 MB).
 * Every call on one GPU shares the scratch: calls that may overlap on a GPU
 * (different streams, or threads without ordering) race and must be ordered
 * by the caller. Each call writes every scratch byte it reads first, so a
 * call does not depend on what an earlier one left there.
 */
ra_status ra_ring_fwd_noalloc(const ra_ring_desc *desc, const void *q, const void *k_chunks,
                              const void *v_chunks, float *o, float *lse, void *stream);

/* Workspace bytes ra_allgather_fwd needs for *desc (same validation as the call). */
ra_status ra_allgather_workspace_bytes(const ra_ring_desc *desc, size_t *bytes);

/*
 * ra_allgather_fwd -- all-gather context parallelism ("Context Parallelism
 * and Ring Attention" §8) for rank `rank`, replayed on one GPU: the K and V
 * chunks of all N ranks are gathered into the whole sequence in global
 * position order (the all-gather's result), then the rank's queries attend
 * over every key in one pass (no merge), with the causal rule and, when
 * desc->doc_start is set, the document mask.
 * Arguments as for ra_ring_fwd (flags must be 0); o and lse are
 * overwritten. step_events, if set, holds 2 hipEvent_t recorded on `stream`
 * just before and just after the attention launch. workspace: device, >= ra_allgather_workspace_bytes();
 * holds the positions, the gathered K and V of the sequence (for bf16 with
 * S % 8 == 0 and S < 8,388,608, V gathered straight into the transposed layout RA_V_TRANSPOSED,
 * with the chunk row of every position) and the queries' document starts.
 * Runs on `stream`.
 */
ra_status ra_allgather_fwd(const ra_ring_desc *desc, const void *q, const void *k_chunks,
                           const void *v_chunks, float *o, float *lse, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Backward ("Context Parallelism and Ring Attention" §3, backward paragraph;
 * §4 for the ring). With the GLOBAL lse of a query (the forward's output) the
 * probability of key j is p_j = e^{x_j - lse} on any block; with
 * D = dout . o per query:
 *   dv_j += p_j dout,  dx_j = p_j (dout . v_j - D),
 *   dq += scale sum_j dx_j k_j,  dk_j += scale sum_q dx_j q   (x = scale q.k).
 * The causal rule is the forward's.
 */

/*
 * ra_attn_bwd_delta -- delta[r] = sum_e dout[r, e] * o[r, e] (the scalar D).
 * rows = b * s * n_q; dout: device [rows, d] of dtype (RA_BF16 or RA_F32);
 * o: device float32 [rows, d]; delta: device float32 [rows]. d in {64, 128}.
 */
ra_status ra_attn_bwd_delta(int64_t rows, int32_t d, int32_t dtype, const void *dout,
                            const float *o, float *delta, void *stream);

/*
 * ra_block_attn_bwd -- one key block's gradient contributions, ADDED into
 * dq, dk and dv (callers accumulate blocks; zero them first for one block).
 * desc: as for ra_block_attn_fwd (bf16, d = 128, v_layout RA_V_ROWS only;
 * others are RA_ERR_UNSUPPORTED). q, dout: device [b, s_q, n_q, d] bf16;
 * k, v: device [b, s_kv, n_kv, d] bf16; lse: device float32 [b, s_q, n_q],
 * the query's global lse (natural log; -inf for a query with no visible key
 * anywhere); delta: device float32 [b, s_q, n_q] from ra_attn_bwd_delta;
 * dq: device float32 [b, s_q, n_q, d]; dk, dv: device float32
 * [b, s_kv, n_kv, d] (a key/value head collects every query head of its
 * group); dq, dk and dv must not overlap one another. Two kernels run in
 * order on `stream`.
 */
ra_status ra_block_attn_bwd(const ra_attn_desc *desc, const void *q, const void *k,
                            const void *v, const void *dout, const float *lse,
                            const float *delta, float *dq, float *dk, float *dv, void *stream);

/* Workspace bytes ra_ring_bwd needs: positions (S int32), D and the lse in
 * log2 units per query head (2*b*c*n_q floats, head-major), the queries'
 * document starts (c int32) and, for N > 1, the double buffer of
 * the travelling block: two halves of K, V (bf16) and dK, dV (float32), one
 * chunk each. */
ra_status ra_ring_bwd_workspace_bytes(const ra_ring_desc *desc, size_t *bytes);

/*
 * ra_ring_bwd -- the ring backward for rank `rank`, replayed on one GPU
 * ("Context Parallelism and Ring Attention" §3 backward paragraph and §4:
 * the accumulated dK, dV of a block travel around the ring with its K, V).
 * desc: as for ra_ring_fwd (bf16, d = 128; flags 0 or RA_RING_SERIALIZE;
 * doc_start optional).
 * q, dout: device [b, c, n_q, d] bf16, the rank's tokens in its local order;
 * o, lse: device float32 [b, c, n_q, d] and [b, c, n_q], the rank's forward
 * outputs (global o and lse); k_chunks, v_chunks: device [N, b, c, n_kv, d]
 * bf16 as for ra_ring_fwd.
 * dq: device float32 [b, c, n_q, d], overwritten with the rank's dQ.
 * dk_chunks, dv_chunks: device float32 [N, b, c, n_kv, d], slot j holding
 * block j's dK, dV accumulated so far; this rank's contribution is ADDED:
 * calling every rank on the same slots sums the sequence's dK, dV. dq,
 * dk_chunks and dv_chunks must not overlap one another.
 * Step r works on block (rank - r) mod N. With N > 1 the block's K, V and
 * slot dK, dV are received into half r % 2 of the workspace's double buffer
 * on `copy`, the step's two kernels run on `compute` against that half, and
 * the updated dK, dV are sent back to the slot on `copy` (on `compute` with
 * RA_RING_SERIALIZE or copy == compute); the result equals adding to the
 * slots in place. A causal step whose block no query of the rank can see
 * launches no kernel (its dK, dV pass through unchanged). After the call
 * the workspace's first S int32 hold every rank's position map, as for
 * ra_ring_fwd. N+1 step events (optional) are recorded on `compute` before
 * step 0 and after each step's kernels.
 * On return all work is enqueued and `compute` is ordered after every copy;
 * `copy` first waits for the work already enqueued on `compute`.
 */
ra_status ra_ring_bwd(const ra_ring_desc *desc, const void *q, const void *k_chunks,
                      const void *v_chunks, const float *o, const float *lse, const void *dout,
                      float *dq, float *dk_chunks, float *dv_chunks, void *workspace,
                      size_t workspace_bytes, void *compute, void *copy);

/* Workspace bytes ra_allgather_bwd needs for *desc (same validation as the call). */
ra_status ra_allgather_bwd_workspace_bytes(const ra_ring_desc *desc, size_t *bytes);

/*
 * ra_allgather_bwd -- the backward of all-gather context parallelism
 * ("Context Parallelism and Ring Attention" §8: K/V all-gathered before
 * attention, dK/dV reduce-scattered after) for rank `rank`, replayed on one
 * GPU, with the optional document mask of desc->doc_start.
 * desc: as for ra_allgather_fwd (bf16, d = 128). Arguments as for
 * ra_ring_bwd: dq is overwritten with the rank's dQ; this rank's
 * contribution to chunk j's dK, dV is ADDED to slot j of dk_chunks /
 * dv_chunks (the reduce-scatter's input: summing every rank's calls on the
 * same slots gives each chunk's dK, dV). workspace: >=
 * ra_allgather_bwd_workspace_bytes(): positions, D and the log2 lse
 * (head-major), document starts, the gathered K and V of the sequence
 * (bf16) and the chunk row of each
 * position (int32; the gradients go straight into the slots). One stream;
 * step_events unused.
 */
ra_status ra_allgather_bwd(const ra_ring_desc *desc, const void *q, const void *k_chunks,
                           const void *v_chunks, const float *o, const float *lse,
                           const void *dout, float *dq, float *dk_chunks, float *dv_chunks,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Static text of a status code. */
const char *ra_status_str(int32_t status);

/* Message of the last failing call on this thread ("" if none). */
const char *ra_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RINGATTN_H */
