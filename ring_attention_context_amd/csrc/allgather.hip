// ra_allgather_fwd: all-gather context parallelism ("Context Parallelism and
// Ring Attention" §8) for one rank, replayed on one GPU.
//
// Instead of passing K/V blocks around a ring, every rank gathers the K and
// V of the whole sequence from its context-parallel group before attention
// and attends with its own queries in one pass: no ring steps and no merge.
// The page gives two reasons for this form: document masks (a sequence that
// packs several documents must not attend across them) are easy to apply
// with every key at its original position, and with GQA the gathered K/V are
// small next to the O(S^2) attention. Here the gather reads the N rank chunks
// (each in its rank's local order, the layout ra_ring_fwd takes) and writes
// the sequence in global position order, the layout an all-gather followed by
// the inverse token permutation of §6 produces. For bf16 V goes from the
// chunks straight into the transposed layout the attention kernel reads
// fastest, in the same pass. Everything runs on one stream: positions, the
// queries' document starts, the gathers, one attention launch.
//
// ra_allgather_bwd is the backward of the same scheme (§8: the all-gather's
// backward is a reduce-scatter of dK, dV): the block backward of the rank's
// queries against the gathered sequence (the kernels of the ring backward,
// with K/V of all S keys). The dK/dV kernel adds each key's gradient straight
// into the caller's slot of the chunk that holds the key (a row map built
// from the positions), so the sequence's dK, dV never exist on their own:
// this rank's share of the reduce-scatter.
#include <cmath>

#include "ra_internal.h"

namespace ra {
namespace {

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// full[bi, pos[j*c + a], :] = chunks[j, bi, a, :] for every rank j, batch bi
// and local index a; rows of `row16` 16-byte units (n_kv * d elements). HBM
// bound: each byte is read once and written once; consecutive threads move
// consecutive 16-byte units of one row.
__global__ __launch_bounds__(256) void kv_gather_kernel(const uint4 *__restrict__ chunks,
                                                        uint4 *__restrict__ full,
                                                        const int32_t *__restrict__ pos,
                                                        int64_t c, int32_t b, int64_t S,
                                                        int64_t row16, int64_t total) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += stride) {
    const int64_t u = i % row16;
    const int64_t row = i / row16;         // (j * b + bi) * c + a
    const int64_t a = row % c;
    const int64_t jb = row / c;
    const int64_t bi = jb % b;
    const int64_t j = jb / b;
    const int64_t p = pos[j * c + a];
    full[(bi * S + p) * row16 + u] = chunks[i];
  }
}

hipError_t launch_kv_gather(const void *chunks, void *full, const int32_t *pos, int64_t c,
                            int32_t N, int32_t b, int64_t S, size_t row_bytes,
                            hipStream_t stream) {
  const int64_t row16 = static_cast<int64_t>(row_bytes / 16);
  const int64_t total = static_cast<int64_t>(N) * b * c * row16;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 256 * 32) blocks = 256 * 32;
  kv_gather_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
      static_cast<const uint4 *>(chunks), static_cast<uint4 *>(full), pos, c, b, S, row16, total);
  return hipGetLastError();
}

// row[pos[j*c + a]] = j*b*c + a: the row of chunk slot j (batch 0) that
// holds the key at each position of the sequence, so that the backward
// kernel adds each key's dK, dV straight into its chunk's slot.
__global__ __launch_bounds__(256) void slot_rows_kernel(const int32_t *__restrict__ pos,
                                                        int32_t *__restrict__ row, int64_t c,
                                                        int32_t b, int64_t S) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < S;
       i += stride) {
    const int64_t j = i / c, a = i % c;
    row[pos[i]] = static_cast<int32_t>(j * b * c + a);
  }
}

hipError_t launch_slot_rows(const int32_t *pos, int32_t *row, int64_t c, int32_t b, int64_t S,
                            hipStream_t stream) {
  if (S == 0) return hipSuccess;
  int64_t blocks = (S + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  slot_rows_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(pos, row, c, b, S);
  return hipGetLastError();
}

struct AgPlan {
  int64_t c = 0;
  size_t full_bytes = 0;    // K (or V) of the whole sequence [b, S, n_kv, d]
  size_t pos_off = 0, kvpos_off = 0, qlo_off = 0, k_off = 0, v_off = 0, vt_off = 0, row_off = 0,
         total = 0;
  bool vt = false;          // V gathered transposed to [b, n_kv, d, S] (else rows)
};

ra_status make_ag_plan(const ra_ring_desc *r, AgPlan *p) {
  ra_status st = check_ring_desc(r);
  if (st != RA_OK) return st;
  if (r->flags != 0) return fail(RA_ERR_INVALID_ARG, "all-gather: flags must be 0 (0x%x)", r->flags);
  const size_t esize = r->dtype == RA_BF16 ? 2 : 4;
  p->c = r->S / r->N;
  p->full_bytes = static_cast<size_t>(r->b) * r->S * r->n_kv * r->d * esize;
  // V^T rows of S keys: 16-byte aligned rows, and a head's d-rows addressable
  // with 32-bit buffer offsets.
  p->vt = r->dtype == RA_BF16 && r->S % 8 == 0 && r->S > 0 &&
          static_cast<int64_t>(r->b) * r->n_kv <= 65535 && vt_addressable(r->d, r->S);
  size_t off = 0;
  p->pos_off = off;
  off += align_up(static_cast<size_t>(r->S) * sizeof(int32_t));
  p->kvpos_off = off;
  off += align_up(static_cast<size_t>(r->S) * sizeof(int32_t));
  p->qlo_off = off;
  off += align_up(static_cast<size_t>(p->c) * sizeof(int32_t));
  p->k_off = off;
  off += align_up(p->full_bytes);
  if (p->vt) {  // V goes straight from the chunks to V^T through the slot rows
    p->vt_off = off;
    off += align_up(p->full_bytes);
    p->row_off = off;
    off += align_up(static_cast<size_t>(r->S) * sizeof(int32_t));
  } else {
    p->v_off = off;
    off += align_up(p->full_bytes);
  }
  p->total = off;
  return RA_OK;
}

struct AgBwdPlan {
  int64_t c = 0;
  size_t kv_bytes = 0;      // K (or V) of the sequence, bf16 [b, S, n_kv, d]
  size_t pos_off = 0, kvpos_off = 0, qlo_off = 0, delta_off = 0, k_off = 0, v_off = 0,
         row_off = 0, total = 0;
};

ra_status make_ag_bwd_plan(const ra_ring_desc *r, AgBwdPlan *p) {
  ra_status st = check_ring_desc(r);
  if (st != RA_OK) return st;
  if (r->flags != 0) return fail(RA_ERR_INVALID_ARG, "all-gather bwd: flags must be 0 (0x%x)", r->flags);
  if (r->dtype != RA_BF16 || r->d != 128)
    return fail(RA_ERR_UNSUPPORTED, "all-gather bwd: bf16 with d = 128 only");
  p->c = r->S / r->N;
  const size_t elems = static_cast<size_t>(r->b) * r->S * r->n_kv * r->d;
  p->kv_bytes = elems * 2;
  size_t off = 0;
  p->pos_off = off;
  off += align_up(static_cast<size_t>(r->S) * sizeof(int32_t));
  p->kvpos_off = off;
  off += align_up(static_cast<size_t>(r->S) * sizeof(int32_t));
  p->qlo_off = off;
  off += align_up(static_cast<size_t>(p->c) * sizeof(int32_t));
  p->delta_off = off;  // D, then the lse in log2 units: head-major [b, n_q, c] each
  off += align_up(2 * static_cast<size_t>(r->b) * p->c * r->n_q * sizeof(float));
  p->k_off = off;
  off += align_up(p->kv_bytes);
  p->v_off = off;
  off += align_up(p->kv_bytes);
  p->row_off = off;
  off += align_up(static_cast<size_t>(r->S) * sizeof(int32_t));
  p->total = off;
  return RA_OK;
}

}  // namespace
}  // namespace ra

extern "C" ra_status ra_allgather_workspace_bytes(const ra_ring_desc *desc, size_t *bytes) {
  ra::clear_error();
  if (!bytes) return ra::fail(RA_ERR_INVALID_ARG, "ra_allgather_workspace_bytes: bytes is NULL");
  ra::AgPlan p;
  ra_status st = ra::make_ag_plan(desc, &p);
  if (st != RA_OK) return st;
  *bytes = p.total;
  return RA_OK;
}

extern "C" ra_status ra_allgather_fwd(const ra_ring_desc *r, const void *q, const void *k_chunks,
                                      const void *v_chunks, float *o, float *lse, void *workspace,
                                      size_t workspace_bytes, void *stream) {
  using ra::fail;
  using ra::hip_check;
  ra::clear_error();
  ra::AgPlan P;
  ra_status st = ra::make_ag_plan(r, &P);
  if (st != RA_OK) return st;
  if (r->b == 0 || P.c == 0) return RA_OK;
  if (!q || !k_chunks || !v_chunks || !o || !lse)
    return fail(RA_ERR_INVALID_ARG, "ra_allgather_fwd: NULL q / k_chunks / v_chunks / o / lse");
  if (!ra::aligned16(q) || !ra::aligned16(k_chunks) || !ra::aligned16(v_chunks) ||
      !ra::aligned16(o))
    return fail(RA_ERR_INVALID_ARG, "ra_allgather_fwd: q / k / v / o not 16-byte aligned");
  const size_t esize = r->dtype == RA_BF16 ? 2 : 4;
  const size_t row_bytes = static_cast<size_t>(r->n_kv) * r->d * esize;
  if (row_bytes % 16)
    return fail(RA_ERR_INVALID_ARG, "ra_allgather_fwd: n_kv * d * element size not a multiple of 16");
  if (!workspace || !ra::aligned16(workspace))
    return fail(RA_ERR_INVALID_ARG, "ra_allgather_fwd: workspace NULL or not 16-byte aligned");
  if (workspace_bytes < P.total)
    return fail(RA_ERR_INVALID_ARG, "ra_allgather_fwd: workspace has %zu bytes, needs %zu",
                workspace_bytes, P.total);

  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char *ws = static_cast<unsigned char *>(workspace);
  int32_t *pos = reinterpret_cast<int32_t *>(ws + P.pos_off);
  int32_t *kv_pos = reinterpret_cast<int32_t *>(ws + P.kvpos_off);
  int32_t *qlo = reinterpret_cast<int32_t *>(ws + P.qlo_off);
  unsigned char *kfull = ws + P.k_off;
  unsigned char *vfull = ws + P.v_off;
  unsigned char *vtfull = ws + P.vt_off;
  const int32_t *q_pos = pos + static_cast<int64_t>(r->rank) * P.c;

  // Every rank's map (to place its chunk), and the identity map of the
  // gathered sequence (keys in global order).
  st = hip_check(ra::launch_positions(r->kind, r->S, r->N, pos, s), "ra_allgather_fwd: positions");
  if (st == RA_OK)
    st = hip_check(ra::launch_positions(RA_PART_CONTIGUOUS, r->S, 1, kv_pos, s),
                   "ra_allgather_fwd: key positions");
  if (st == RA_OK && r->doc_start)
    st = hip_check(ra::launch_gather_i32(r->doc_start, q_pos, qlo, P.c, s),
                   "ra_allgather_fwd: document starts");
  if (st == RA_OK)
    st = hip_check(ra::launch_kv_gather(k_chunks, kfull, pos, P.c, r->N, r->b, r->S, row_bytes, s),
                   "ra_allgather_fwd: K gather");
  if (st == RA_OK && P.vt) {
    int32_t *src_row = reinterpret_cast<int32_t *>(ws + P.row_off);
    st = hip_check(ra::launch_slot_rows(pos, src_row, P.c, r->b, r->S, s),
                   "ra_allgather_fwd: slot rows");
    if (st == RA_OK)
      st = hip_check(ra::launch_rows_to_vt(v_chunks, vtfull, src_row, P.c, r->b, r->S, r->n_kv,
                                           r->d, s),
                     "ra_allgather_fwd: V gather (transposed)");
  } else if (st == RA_OK) {
    st = hip_check(ra::launch_kv_gather(v_chunks, vfull, pos, P.c, r->N, r->b, r->S, row_bytes, s),
                   "ra_allgather_fwd: V gather");
  }
  if (st != RA_OK) return st;

  hipEvent_t *ev = reinterpret_cast<hipEvent_t *>(r->step_events);
  if (ev) {
    st = hip_check(hipEventRecord(ev[0], s), "ra_allgather_fwd: event");
    if (st != RA_OK) return st;
  }
  ra::AttnArgs a{};
  a.q = q;
  a.k = kfull;
  a.v = P.vt ? vtfull : vfull;
  a.v_layout = P.vt ? RA_V_TRANSPOSED : RA_V_ROWS;
  a.o = o;
  a.lse = lse;
  a.q_pos = q_pos;
  a.kv_pos = kv_pos;
  a.q_lo = r->doc_start ? qlo : nullptr;
  a.s_q = P.c;
  a.s_kv = r->S;
  a.b = r->b;
  a.n_q = r->n_q;
  a.n_kv = r->n_kv;
  a.d = r->d;
  a.scale = r->scale > 0.f ? r->scale : 1.0f / std::sqrt(static_cast<float>(r->d));
  a.causal = r->causal;
  a.merge = 0;
  hipError_t err = r->dtype == RA_BF16 ? ra::launch_attn_bf16(a, s) : ra::launch_attn_f32(a, s);
  st = hip_check(err, "ra_allgather_fwd: attention launch");
  if (st == RA_OK && ev) st = hip_check(hipEventRecord(ev[1], s), "ra_allgather_fwd: event");
  return st;
}

extern "C" ra_status ra_allgather_bwd_workspace_bytes(const ra_ring_desc *desc, size_t *bytes) {
  ra::clear_error();
  if (!bytes) return ra::fail(RA_ERR_INVALID_ARG, "ra_allgather_bwd_workspace_bytes: bytes is NULL");
  ra::AgBwdPlan p;
  ra_status st = ra::make_ag_bwd_plan(desc, &p);
  if (st != RA_OK) return st;
  *bytes = p.total;
  return RA_OK;
}

extern "C" ra_status ra_allgather_bwd(const ra_ring_desc *r, const void *q, const void *k_chunks,
                                      const void *v_chunks, const float *o, const float *lse,
                                      const void *dout, float *dq, float *dk_chunks,
                                      float *dv_chunks, void *workspace, size_t workspace_bytes,
                                      void *stream) {
  using ra::fail;
  using ra::hip_check;
  ra::clear_error();
  ra::AgBwdPlan P;
  ra_status st = ra::make_ag_bwd_plan(r, &P);
  if (st != RA_OK) return st;
  if (r->b == 0 || P.c == 0) return RA_OK;
  if (!q || !k_chunks || !v_chunks || !o || !lse || !dout || !dq || !dk_chunks || !dv_chunks)
    return fail(RA_ERR_INVALID_ARG, "ra_allgather_bwd: NULL input or output");
  const void *ptrs[] = {q, k_chunks, v_chunks, o, dout, dq, dk_chunks, dv_chunks};
  for (const void *p : ptrs)
    if (!ra::aligned16(p)) return fail(RA_ERR_INVALID_ARG, "ra_allgather_bwd: pointer not 16-byte aligned");
  if (!workspace || !ra::aligned16(workspace))
    return fail(RA_ERR_INVALID_ARG, "ra_allgather_bwd: workspace NULL or not 16-byte aligned");
  if (workspace_bytes < P.total)
    return fail(RA_ERR_INVALID_ARG, "ra_allgather_bwd: workspace has %zu bytes, needs %zu",
                workspace_bytes, P.total);

  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char *ws = static_cast<unsigned char *>(workspace);
  int32_t *pos = reinterpret_cast<int32_t *>(ws + P.pos_off);
  int32_t *kv_pos = reinterpret_cast<int32_t *>(ws + P.kvpos_off);
  int32_t *qlo = reinterpret_cast<int32_t *>(ws + P.qlo_off);
  float *delta = reinterpret_cast<float *>(ws + P.delta_off);
  unsigned char *kfull = ws + P.k_off;
  unsigned char *vfull = ws + P.v_off;
  int32_t *slot_row = reinterpret_cast<int32_t *>(ws + P.row_off);
  const int32_t *q_pos = pos + static_cast<int64_t>(r->rank) * P.c;
  const size_t row_bytes = static_cast<size_t>(r->n_kv) * r->d * 2;
  const int64_t rows = static_cast<int64_t>(r->b) * P.c * r->n_q;

  st = hip_check(ra::launch_positions(r->kind, r->S, r->N, pos, s), "ra_allgather_bwd: positions");
  if (st == RA_OK)
    st = hip_check(ra::launch_positions(RA_PART_CONTIGUOUS, r->S, 1, kv_pos, s),
                   "ra_allgather_bwd: key positions");
  if (st == RA_OK && r->doc_start)
    st = hip_check(ra::launch_gather_i32(r->doc_start, q_pos, qlo, P.c, s),
                   "ra_allgather_bwd: document starts");
  if (st == RA_OK)
    st = hip_check(ra::launch_bwd_prep(r->b, P.c, r->n_q, dout, o, lse, delta, delta + rows, s),
                   "ra_allgather_bwd: delta");
  if (st == RA_OK)
    st = hip_check(ra::launch_fill_zero(dq, rows * r->d, s), "ra_allgather_bwd: zero dq");
  if (st == RA_OK)
    st = hip_check(ra::launch_slot_rows(pos, slot_row, P.c, r->b, r->S, s),
                   "ra_allgather_bwd: slot rows");
  if (st == RA_OK)
    st = hip_check(ra::launch_kv_gather(k_chunks, kfull, pos, P.c, r->N, r->b, r->S, row_bytes, s),
                   "ra_allgather_bwd: K gather");
  if (st == RA_OK)
    st = hip_check(ra::launch_kv_gather(v_chunks, vfull, pos, P.c, r->N, r->b, r->S, row_bytes, s),
                   "ra_allgather_bwd: V gather");
  if (st != RA_OK) return st;

  ra::BwdArgs a{};
  a.q = q;
  a.k = kfull;
  a.v = vfull;
  a.dout = dout;
  a.lse = delta + rows;
  a.delta = delta;
  a.hm = 1;
  a.dq = dq;
  a.dk = dk_chunks;  // each key's dK, dV go straight into its chunk's slot
  a.dv = dv_chunks;
  a.kv_row = slot_row;
  a.kv_row_bstride = P.c;
  a.q_pos = q_pos;
  a.kv_pos = kv_pos;
  a.q_lo = r->doc_start ? qlo : nullptr;
  a.s_q = P.c;
  a.s_kv = r->S;
  a.b = r->b;
  a.n_q = r->n_q;
  a.n_kv = r->n_kv;
  a.d = r->d;
  a.scale = r->scale > 0.f ? r->scale : 1.0f / std::sqrt(static_cast<float>(r->d));
  a.causal = r->causal;
  st = hip_check(ra::launch_attn_bwd_bf16(a, s), "ra_allgather_bwd: backward launch");
  return st;
}
