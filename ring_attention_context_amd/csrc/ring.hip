// ra_ring_fwd: the ring loop of "Context Parallelism and Ring Attention" §4
// for one rank, replayed on one GPU.
//
// The pages' loop: at step r the rank holds the K/V block that rank
// (rank - r) mod N started with, computes its block statistics against the
// local queries, merges them into the running (o, lse) with the §3 merge, and
// meanwhile sends its block on and receives the next one (double buffer,
// §4 "memory"). Here the "receive" is a device-to-device copy of the next
// chunk into the idle half of a double buffer on a second stream, ordered by
// events against the compute stream:
//   copy(r+1 -> buf[(r+1)&1]) waits for step r-1 (the last reader of that half)
//   step r waits for copy(r -> buf[r&1]).
// For bf16 (with c % 8 == 0 and d * c * 2 < 2^31 bytes, the reach of one
// buffer descriptor) the copy of V is a transpose into the V^T
// layout the attention kernel reads fastest, and the rank's own V chunk is
// transposed into buffer half 0 before step 0 as well; K of step 0 is read in
// place. Step 0 writes (o, lse) directly (merging into the identity
// (0, -inf) is a no-op). Later steps merge in the attention kernel's
// epilogue, or, with RA_RING_UNFUSED_MERGE, write (o_b, lse_b) to the
// workspace and run the standalone merge kernel. With a document mask the
// rank's queries' document starts are gathered once; every step's block
// then applies the same per-query lower bound on key positions, which is
// what keeps the mask right for any chunk (§8 names this per-step mask as
// the ring's difficulty).
#include <climits>
#include <cmath>
#include <unordered_map>

#include "ra_internal.h"

namespace ra {
namespace {

constexpr size_t ALIGN = 256;
inline size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// Positions of every rank's tokens: pos[j * c + a] = map_j(a) (§2, §6).
__global__ void positions_kernel(int32_t kind, int64_t S, int32_t N, int32_t *pos) {
  const int64_t c = S / N;
  const int64_t h = c / 2;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < S;
       i += stride) {
    const int64_t j = i / c, a = i - j * c;
    int64_t p;
    if (kind == RA_PART_CONTIGUOUS)
      p = j * c + a;
    else if (kind == RA_PART_ZIGZAG)
      p = a < h ? j * h + a : (2 * static_cast<int64_t>(N) - 1 - j) * h + (a - h);
    else
      p = a * N + j;
    pos[i] = static_cast<int32_t>(p);
  }
}

struct Plan {
  int64_t c = 0;
  size_t esize = 0;
  size_t chunk_bytes = 0;   // one K (or V) chunk [b, c, n_kv, d]
  size_t pos_off = 0, qlo_off = 0, kv_off[2] = {0, 0}, ob_off = 0, lseb_off = 0, total = 0;
  bool fused = true, serialize = false;
  bool vt = false;          // V chunks staged transposed (bf16, c % 8 == 0)
  bool pairable = false;    // serialized steps may run two blocks per launch
};

}  // namespace

// Checks shared by every call that takes an ra_ring_desc (flags aside).
ra_status check_ring_desc(const ra_ring_desc *r) {
  if (!r) return fail(RA_ERR_INVALID_ARG, "ring: desc is NULL");
  if (r->N < 1) return fail(RA_ERR_INVALID_ARG, "ring: N = %d must be >= 1", r->N);
  if (r->rank < 0 || r->rank >= r->N)
    return fail(RA_ERR_INVALID_ARG, "ring: rank %d outside [0, %d)", r->rank, r->N);
  if (r->S < 0 || r->S > INT32_MAX - 1)
    return fail(RA_ERR_INVALID_ARG, "ring: S = %lld outside [0, 2^31 - 1)", (long long)r->S);
  if (r->S % r->N) return fail(RA_ERR_INVALID_ARG, "ring: S %% N != 0");
  if (r->kind == RA_PART_ZIGZAG && r->S % (2 * static_cast<int64_t>(r->N)))
    return fail(RA_ERR_INVALID_ARG, "ring: zig-zag needs S %% 2N == 0");
  if (r->kind != RA_PART_CONTIGUOUS && r->kind != RA_PART_ZIGZAG && r->kind != RA_PART_STRIPED)
    return fail(RA_ERR_INVALID_ARG, "ring: unknown partition kind %d", r->kind);
  if (r->reserved != 0) return fail(RA_ERR_INVALID_ARG, "ring: reserved must be 0");
  if (r->doc_start && r->causal != 1)
    return fail(RA_ERR_UNSUPPORTED, "ring: a document mask needs causal = 1");
  // Shape / dtype checks shared with the block call.
  ra_attn_desc ad{};
  ad.b = r->b;
  ad.n_q = r->n_q;
  ad.n_kv = r->n_kv;
  ad.d = r->d;
  ad.s_q = 0;
  ad.s_kv = 0;
  ad.dtype = r->dtype;
  ad.causal = r->causal;
  ad.scale = r->scale;
  return validate_attn(&ad, nullptr, nullptr, nullptr, nullptr, nullptr);
}

namespace {

ra_status make_plan(const ra_ring_desc *r, Plan *p) {
  ra_status st = check_ring_desc(r);
  if (st != RA_OK) return st;
  if (r->flags & ~(RA_RING_SERIALIZE | RA_RING_UNFUSED_MERGE | RA_RING_OVERLAP | RA_RING_STEPWISE))
    return fail(RA_ERR_INVALID_ARG, "ring: unknown flag bits 0x%x", r->flags);
  if ((r->flags & RA_RING_SERIALIZE) && (r->flags & RA_RING_OVERLAP))
    return fail(RA_ERR_INVALID_ARG, "ring: RA_RING_SERIALIZE and RA_RING_OVERLAP both set");
  p->c = r->S / r->N;
  p->esize = r->dtype == RA_BF16 ? 2 : 4;
  p->chunk_bytes = static_cast<size_t>(r->b) * p->c * r->n_kv * r->d * p->esize;
  p->fused = !(r->flags & RA_RING_UNFUSED_MERGE);
  p->serialize = (r->flags & RA_RING_SERIALIZE) != 0 ||
                 (!(r->flags & RA_RING_OVERLAP) && p->chunk_bytes <= RA_RING_SERIAL_CHUNK_BYTES);
  p->vt = r->dtype == RA_BF16 && p->c % 8 == 0 && p->c > 0 &&
          static_cast<int64_t>(r->b) * r->n_kv <= 65535 && vt_addressable(r->d, p->c);
  p->pairable = p->vt && p->fused && !r->doc_start && !(r->flags & RA_RING_STEPWISE);
  size_t off = 0;
  p->pos_off = off;
  off += align_up(static_cast<size_t>(r->S) * sizeof(int32_t));
  if (r->N > 1 || p->vt) {
    for (int i = 0; i < 2; ++i) {
      p->kv_off[i] = off;
      off += 2 * align_up(p->chunk_bytes);
    }
  }
  if (!p->fused && r->N > 1) {
    const size_t rows = static_cast<size_t>(r->b) * p->c * r->n_q;
    p->ob_off = off;
    off += align_up(rows * r->d * sizeof(float));
    p->lseb_off = off;
    off += align_up(rows * sizeof(float));
  }
  p->qlo_off = off;   // the rank's queries' document starts
  off += align_up(static_cast<size_t>(p->c) * sizeof(int32_t));
  p->total = off;
  return RA_OK;
}

struct RingEvents {
  hipEvent_t start, ready[2], freed[2];
};

// Per-thread, per-device events used to order the two streams.
ra_status ring_events(RingEvents **out) {
  thread_local std::unordered_map<int, RingEvents> cache;
  int dev = 0;
  ra_status st = hip_check(hipGetDevice(&dev), "ring: hipGetDevice");
  if (st != RA_OK) return st;
  auto it = cache.find(dev);
  if (it == cache.end()) {
    RingEvents ev{};
    hipEvent_t *all[5] = {&ev.start, &ev.ready[0], &ev.ready[1], &ev.freed[0], &ev.freed[1]};
    for (hipEvent_t *e : all) {
      st = hip_check(hipEventCreateWithFlags(e, hipEventDisableTiming), "ring: hipEventCreate");
      if (st != RA_OK) return st;
    }
    it = cache.emplace(dev, ev).first;
  }
  *out = &it->second;
  return RA_OK;
}

}  // namespace

__global__ void fill_zero_kernel(float *p, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    p[i] = 0.f;
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_zero_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(p, n);
  return hipGetLastError();
}

__global__ void gather_i32_kernel(const int32_t *src, const int32_t *idx, int32_t *out, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = src[idx[i]];
}

hipError_t launch_gather_i32(const int32_t *src, const int32_t *idx, int32_t *out, int64_t n,
                             hipStream_t stream) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  gather_i32_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(src, idx, out, n);
  return hipGetLastError();
}

hipError_t launch_positions(int32_t kind, int64_t S, int32_t N, int32_t *pos,
                            hipStream_t stream) {
  if (S == 0) return hipSuccess;
  int64_t blocks = (S + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  positions_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(kind, S, N, pos);
  return hipGetLastError();
}

}  // namespace ra

extern "C" ra_status ra_ring_workspace_bytes(const ra_ring_desc *desc, size_t *bytes) {
  ra::clear_error();
  if (!bytes) return ra::fail(RA_ERR_INVALID_ARG, "ra_ring_workspace_bytes: bytes is NULL");
  ra::Plan p;
  ra_status st = ra::make_plan(desc, &p);
  if (st != RA_OK) return st;
  *bytes = p.total;
  return RA_OK;
}

extern "C" ra_status ra_ring_fwd(const ra_ring_desc *r, const void *q, const void *k_chunks,
                                 const void *v_chunks, float *o, float *lse, void *workspace,
                                 size_t workspace_bytes, void *compute, void *copy) {
  using ra::fail;
  using ra::hip_check;
  ra::clear_error();
  ra::Plan P;
  ra_status st = ra::make_plan(r, &P);
  if (st != RA_OK) return st;
  const bool empty = r->b == 0 || P.c == 0;
  if (!empty) {
    if (!q || !k_chunks || !v_chunks || !o || !lse)
      return fail(RA_ERR_INVALID_ARG, "ra_ring_fwd: NULL q / k_chunks / v_chunks / o / lse");
    if (!ra::aligned16(q) || !ra::aligned16(k_chunks) || !ra::aligned16(v_chunks) ||
        !ra::aligned16(o))
      return fail(RA_ERR_INVALID_ARG, "ra_ring_fwd: q / k / v / o not 16-byte aligned");
    if (P.chunk_bytes % 16)
      return fail(RA_ERR_INVALID_ARG, "ra_ring_fwd: chunk size not a multiple of 16 bytes");
    if (!workspace || !ra::aligned16(workspace))
      return fail(RA_ERR_INVALID_ARG, "ra_ring_fwd: workspace NULL or not 16-byte aligned");
    if (workspace_bytes < P.total)
      return fail(RA_ERR_INVALID_ARG, "ra_ring_fwd: workspace has %zu bytes, needs %zu",
                  workspace_bytes, P.total);
  }
  hipStream_t sc = static_cast<hipStream_t>(compute);
  hipStream_t sp = static_cast<hipStream_t>(copy);
  const bool serialize = P.serialize || sp == sc;
  // With the copies on `compute`, two consecutive visible steps share one
  // launch (both blocks in one scan, one merge): at small chunks a launch's
  // prologue and its o / lse merge cost a fifth of the step.
  const bool pair = serialize && P.pairable;
  hipEvent_t *step_ev = reinterpret_cast<hipEvent_t *>(r->step_events);
  if (empty) {
    if (step_ev)
      for (int i = 0; i <= r->N; ++i) {
        st = hip_check(hipEventRecord(step_ev[i], sc), "ra_ring_fwd: step event");
        if (st != RA_OK) return st;
      }
    return RA_OK;
  }

  ra::RingEvents *ev = nullptr;
  if (!serialize && (r->N > 1 || P.vt)) {
    st = ra::ring_events(&ev);
    if (st != RA_OK) return st;
  }
  unsigned char *ws = static_cast<unsigned char *>(workspace);
  int32_t *pos = reinterpret_cast<int32_t *>(ws + P.pos_off);
  st = hip_check(ra::launch_positions(r->kind, r->S, r->N, pos, sc), "ra_ring_fwd: positions");
  if (st != RA_OK) return st;
  int32_t *qlo = reinterpret_cast<int32_t *>(ws + P.qlo_off);
  if (r->doc_start) {
    st = hip_check(ra::launch_gather_i32(r->doc_start, pos + static_cast<int64_t>(r->rank) * P.c,
                                         qlo, P.c, sc),
                   "ra_ring_fwd: document starts");
    if (st != RA_OK) return st;
  }
  if (ev) {
    // The copy stream reads k/v chunks the caller may have just written on `compute`.
    st = hip_check(hipEventRecord(ev->start, sc), "ra_ring_fwd: event record");
    if (st == RA_OK) st = hip_check(hipStreamWaitEvent(sp, ev->start, 0), "ra_ring_fwd: wait");
    if (st != RA_OK) return st;
  }
  if (step_ev) {
    st = hip_check(hipEventRecord(step_ev[0], sc), "ra_ring_fwd: step event");
    if (st != RA_OK) return st;
  }

  const unsigned char *kc = static_cast<const unsigned char *>(k_chunks);
  const unsigned char *vc = static_cast<const unsigned char *>(v_chunks);
  const size_t CB = P.chunk_bytes;
  unsigned char *kbuf[2] = {ws + P.kv_off[0], ws + P.kv_off[1]};
  unsigned char *vbuf[2] = {ws + P.kv_off[0] + ra::align_up(CB), ws + P.kv_off[1] + ra::align_up(CB)};
  float *o_b = reinterpret_cast<float *>(ws + P.ob_off);
  float *lse_b = reinterpret_cast<float *>(ws + P.lseb_off);
  const int N = r->N, rank = r->rank;

  ra::AttnArgs a{};
  a.q = q;
  a.s_q = P.c;
  a.s_kv = P.c;
  a.b = r->b;
  a.n_q = r->n_q;
  a.n_kv = r->n_kv;
  a.d = r->d;
  a.scale = r->scale > 0.f ? r->scale : 1.0f / std::sqrt(static_cast<float>(r->d));
  a.causal = r->causal;
  a.q_pos = pos + static_cast<int64_t>(rank) * P.c;
  a.q_lo = r->doc_start ? qlo : nullptr;

  // Fill buffer half (step & 1) with the chunk of `step` (K copied, V copied
  // or transposed); step 0 needs only its V, and only when transposing.
  hipStream_t cs = serialize ? sc : sp;
  auto uses_buf = [&](int step) { return step >= 1 || P.vt; };
  auto fill = [&](int step) -> ra_status {
    const int src = ((rank - step) % N + N) % N;
    const int buf = step & 1;
    ra_status s2 = RA_OK;
    if (!serialize && step >= 2 && uses_buf(step - 2))
      s2 = hip_check(hipStreamWaitEvent(sp, ev->freed[buf], 0), "ra_ring_fwd: wait freed");
    if (s2 == RA_OK && P.vt) {
      // V transposed and (from step 1 on) K copied by one launch.
      s2 = hip_check(ra::launch_rows_to_vt(vc + static_cast<size_t>(src) * CB, vbuf[buf], nullptr,
                                           P.c, r->b, P.c, r->n_kv, r->d, cs,
                                           kc + static_cast<size_t>(src) * CB, kbuf[buf],
                                           step >= 1 ? CB : 0),
                     "ra_ring_fwd: K copy and V transpose");
    } else if (s2 == RA_OK) {
      if (step >= 1)
        s2 = hip_check(hipMemcpyAsync(kbuf[buf], kc + static_cast<size_t>(src) * CB, CB,
                                      hipMemcpyDeviceToDevice, cs),
                       "ra_ring_fwd: K copy");
      if (s2 == RA_OK)
        s2 = hip_check(hipMemcpyAsync(vbuf[buf], vc + static_cast<size_t>(src) * CB, CB,
                                      hipMemcpyDeviceToDevice, cs),
                       "ra_ring_fwd: V copy");
    }
    if (s2 == RA_OK && !serialize)
      s2 = hip_check(hipEventRecord(ev->ready[buf], sp), "ra_ring_fwd: record ready");
    return s2;
  };
  if (P.vt) {
    st = fill(0);
    if (st != RA_OK) return st;
  }
  a.v_layout = P.vt ? RA_V_TRANSPOSED : RA_V_ROWS;

  // Chunks are filled in step order; fill(x) writes half x % 2, which the
  // launch of step x - 2 (enqueued before it) has finished with.
  int next_fill = 1;
  auto fill_upto = [&](int x) -> ra_status {
    for (; next_fill <= x && next_fill < N; ++next_fill) {
      ra_status s2 = fill(next_fill);
      if (s2 != RA_OK) return s2;
    }
    return RA_OK;
  };
  auto visible = [&](int step) {
    const int src = ((rank - step) % N + N) % N;
    return step == 0 || !r->causal || !ra::causally_empty(r->kind, r->S, N, rank, src);
  };
  auto record_step = [&](int step) -> ra_status {
    return step_ev ? hip_check(hipEventRecord(step_ev[step + 1], sc), "ra_ring_fwd: step event")
                   : RA_OK;
  };
  for (int step = 0; step < N;) {
    const int src = ((rank - step) % N + N) % N;
    if (pair && step + 1 < N && visible(step) && visible(step + 1)) {
      // Steps step and step + 1 in one launch; both chunks are in place
      // (serialized copies on `compute`).
      st = fill_upto(step + 1);
      if (st != RA_OK) return st;
      const int src2 = ((rank - step - 1) % N + N) % N;
      a.k = step == 0 ? kc + static_cast<size_t>(rank) * CB : kbuf[step & 1];
      a.v = vbuf[step & 1];
      a.kv_pos = pos + static_cast<int64_t>(src) * P.c;
      a.k2 = kbuf[(step + 1) & 1];
      a.v2 = vbuf[(step + 1) & 1];
      a.kv_pos2 = pos + static_cast<int64_t>(src2) * P.c;
      a.o = o;
      a.lse = lse;
      a.merge = step > 0 ? 1 : 0;
      st = hip_check(ra::launch_attn_bf16(a, sc), "ra_ring_fwd: attention launch (two blocks)");
      a.k2 = a.v2 = nullptr;
      a.kv_pos2 = nullptr;
      if (st == RA_OK) st = record_step(step);
      if (st == RA_OK) st = record_step(step + 1);
      if (st != RA_OK) return st;
      step += 2;
      continue;
    }
    // Prefetch the next step's chunk into the idle half of the double buffer.
    st = fill_upto(step + 1);
    if (st != RA_OK) return st;
    // A block that no query of this rank can see (causal rule; step 0 is the
    // rank's own chunk and never empty) adds nothing: its chunk still arrives
    // (the ring forwards it) but no kernel reads it.
    if (!visible(step)) {
      st = record_step(step);
      if (st != RA_OK) return st;
      ++step;
      continue;
    }
    if (uses_buf(step) && !serialize) {
      st = hip_check(hipStreamWaitEvent(sc, ev->ready[step & 1], 0), "ra_ring_fwd: wait ready");
      if (st != RA_OK) return st;
    }
    a.k = step == 0 ? kc + static_cast<size_t>(rank) * CB : kbuf[step & 1];
    a.v = uses_buf(step) ? vbuf[step & 1] : vc + static_cast<size_t>(rank) * CB;
    a.kv_pos = pos + static_cast<int64_t>(src) * P.c;
    const bool unfused_merge = !P.fused && step > 0;
    a.o = unfused_merge ? o_b : o;
    a.lse = unfused_merge ? lse_b : lse;
    a.merge = (P.fused && step > 0) ? 1 : 0;
    hipError_t err = r->dtype == RA_BF16 ? ra::launch_attn_bf16(a, sc) : ra::launch_attn_f32(a, sc);
    st = hip_check(err, "ra_ring_fwd: attention launch");
    if (st != RA_OK) return st;
    if (unfused_merge) {
      const int64_t rows = static_cast<int64_t>(r->b) * P.c * r->n_q;
      st = hip_check(ra::launch_lse_merge(rows, r->d, o, lse, o_b, lse_b, sc),
                     "ra_ring_fwd: merge launch");
      if (st != RA_OK) return st;
    }
    if (uses_buf(step) && !serialize) {
      st = hip_check(hipEventRecord(ev->freed[step & 1], sc), "ra_ring_fwd: record freed");
      if (st != RA_OK) return st;
    }
    st = record_step(step);
    if (st != RA_OK) return st;
    ++step;
  }
  // Order `compute` after the last chunk's arrival also when its step was
  // skipped (the next call reuses the buffers).
  if (uses_buf(N - 1) && !serialize) {
    st = hip_check(hipStreamWaitEvent(sc, ev->ready[(N - 1) & 1], 0), "ra_ring_fwd: join copies");
    if (st != RA_OK) return st;
  }
  return RA_OK;
}

// ---------------------------------------------------------------- backward ring
//
// The ring backward of "Context Parallelism and Ring Attention" §3 (backward
// paragraph) and §4 for one rank: D = dout . o once; at step r the rank holds
// the K/V block of rank (rank - r) mod N together with that block's
// accumulated dK, dV (on a ring they travel with it, §4 "can communication be
// hidden"), adds the block's contribution to its dQ and to the travelling
// dK, dV, and passes the block on. Replayed on one GPU, the caller's per-block
// slots hold the accumulated dK, dV; for N > 1, step r "receives" block src's
// K, V and accumulated dK, dV into half (r & 1) of a double buffer and, once
// both kernels of the step have run on that half, "sends" the updated dK, dV
// back to the slot. Receives and sends run on the copy stream, ordered by
// events against the compute stream:
//   receive(r)  into half r&1 follows send(r-2) out of it (same stream);
//   send(r)     waits for step r's kernels;
//   step r      waits for receive(r).
// The result equals adding this rank's contribution to the slots in place.

namespace ra {
namespace {

struct BwdPlan {
  int64_t c = 0;
  size_t chunk_elems = 0;  // one K (or V) chunk [b, c, n_kv, d]
  size_t pos_off = 0, delta_off = 0, qlo_off = 0, total = 0;
  size_t buf_off[2] = {0, 0};  // per half: K, V (bf16), dK, dV (fp32)
  size_t kb = 0, vb = 0, dkb = 0, dvb = 0;  // offsets inside a half
  bool ring = false;       // N > 1: the transfer is replayed through the buffer
};

ra_status make_bwd_plan(const ra_ring_desc *r, BwdPlan *p) {
  if (!r) return fail(RA_ERR_INVALID_ARG, "ring bwd: desc is NULL");
  if (r->flags & ~RA_RING_SERIALIZE)
    return fail(RA_ERR_INVALID_ARG, "ring bwd: only RA_RING_SERIALIZE may be set (0x%x)", r->flags);
  ra_ring_desc fwd = *r;
  fwd.flags = 0;
  Plan fp;
  ra_status st = make_plan(&fwd, &fp);
  if (st != RA_OK) return st;
  if (r->dtype != RA_BF16 || r->d != 128)
    return fail(RA_ERR_UNSUPPORTED, "ring bwd: bf16 with d = 128 only");
  p->c = fp.c;
  p->chunk_elems = static_cast<size_t>(r->b) * fp.c * r->n_kv * r->d;
  p->ring = r->N > 1;
  size_t off = 0;
  p->pos_off = off;
  off += align_up(static_cast<size_t>(r->S) * sizeof(int32_t));
  p->delta_off = off;  // D, then the lse in log2 units: head-major [b, n_q, c] each
  off += align_up(2 * static_cast<size_t>(r->b) * fp.c * r->n_q * sizeof(float));
  p->qlo_off = off;   // the rank's queries' document starts
  off += align_up(static_cast<size_t>(fp.c) * sizeof(int32_t));
  if (p->ring) {
    p->kb = 0;
    p->vb = align_up(p->chunk_elems * 2);
    p->dkb = 2 * align_up(p->chunk_elems * 2);
    p->dvb = p->dkb + align_up(p->chunk_elems * 4);
    const size_t half = p->dvb + align_up(p->chunk_elems * 4);
    for (int i = 0; i < 2; ++i) {
      p->buf_off[i] = off;
      off += half;
    }
  }
  p->total = off;
  return RA_OK;
}

struct BwdEvents {
  hipEvent_t start, ready[2], done[2], sent;
};

ra_status bwd_events(BwdEvents **out) {
  thread_local std::unordered_map<int, BwdEvents> cache;
  int dev = 0;
  ra_status st = hip_check(hipGetDevice(&dev), "ring bwd: hipGetDevice");
  if (st != RA_OK) return st;
  auto it = cache.find(dev);
  if (it == cache.end()) {
    BwdEvents ev{};
    hipEvent_t *all[6] = {&ev.start, &ev.ready[0], &ev.ready[1], &ev.done[0], &ev.done[1], &ev.sent};
    for (hipEvent_t *e : all) {
      st = hip_check(hipEventCreateWithFlags(e, hipEventDisableTiming), "ring bwd: hipEventCreate");
      if (st != RA_OK) return st;
    }
    it = cache.emplace(dev, ev).first;
  }
  *out = &it->second;
  return RA_OK;
}

}  // namespace
}  // namespace ra

extern "C" ra_status ra_ring_bwd_workspace_bytes(const ra_ring_desc *desc, size_t *bytes) {
  ra::clear_error();
  if (!bytes) return ra::fail(RA_ERR_INVALID_ARG, "ra_ring_bwd_workspace_bytes: bytes is NULL");
  ra::BwdPlan p;
  ra_status st = ra::make_bwd_plan(desc, &p);
  if (st != RA_OK) return st;
  *bytes = p.total;
  return RA_OK;
}

extern "C" ra_status ra_ring_bwd(const ra_ring_desc *r, const void *q, const void *k_chunks,
                                 const void *v_chunks, const float *o, const float *lse,
                                 const void *dout, float *dq, float *dk_chunks, float *dv_chunks,
                                 void *workspace, size_t workspace_bytes, void *compute,
                                 void *copy) {
  using ra::fail;
  using ra::hip_check;
  ra::clear_error();
  ra::BwdPlan P;
  ra_status st = ra::make_bwd_plan(r, &P);
  if (st != RA_OK) return st;
  hipStream_t sc = static_cast<hipStream_t>(compute);
  hipStream_t sp = static_cast<hipStream_t>(copy);
  const bool serialize = (r->flags & RA_RING_SERIALIZE) != 0 || sp == sc;
  hipEvent_t *step_ev = reinterpret_cast<hipEvent_t *>(r->step_events);
  const bool empty = r->b == 0 || P.c == 0;
  if (empty) {
    if (step_ev)
      for (int i = 0; i <= r->N; ++i) {
        st = hip_check(hipEventRecord(step_ev[i], sc), "ra_ring_bwd: step event");
        if (st != RA_OK) return st;
      }
    return RA_OK;
  }
  if (!q || !k_chunks || !v_chunks || !o || !lse || !dout || !dq || !dk_chunks || !dv_chunks)
    return fail(RA_ERR_INVALID_ARG, "ra_ring_bwd: NULL input or output");
  const void *ptrs[] = {q, k_chunks, v_chunks, o, dout, dq, dk_chunks, dv_chunks};
  for (const void *p : ptrs)
    if (!ra::aligned16(p)) return fail(RA_ERR_INVALID_ARG, "ra_ring_bwd: pointer not 16-byte aligned");
  if ((P.chunk_elems * 2) % 16)
    return fail(RA_ERR_INVALID_ARG, "ra_ring_bwd: chunk size not a multiple of 16 bytes");
  if (!workspace || !ra::aligned16(workspace))
    return fail(RA_ERR_INVALID_ARG, "ra_ring_bwd: workspace NULL or not 16-byte aligned");
  if (workspace_bytes < P.total)
    return fail(RA_ERR_INVALID_ARG, "ra_ring_bwd: workspace has %zu bytes, needs %zu",
                workspace_bytes, P.total);

  unsigned char *ws = static_cast<unsigned char *>(workspace);
  int32_t *pos = reinterpret_cast<int32_t *>(ws + P.pos_off);
  float *delta = reinterpret_cast<float *>(ws + P.delta_off);
  const int64_t rows = static_cast<int64_t>(r->b) * P.c * r->n_q;
  float *lse_t = delta + rows;
  st = hip_check(ra::launch_positions(r->kind, r->S, r->N, pos, sc), "ra_ring_bwd: positions");
  if (st == RA_OK)
    st = hip_check(ra::launch_bwd_prep(r->b, P.c, r->n_q, dout, o, lse, delta, lse_t, sc),
                   "ra_ring_bwd: delta");
  if (st == RA_OK)
    st = hip_check(ra::launch_fill_zero(dq, rows * r->d, sc), "ra_ring_bwd: zero dq");
  int32_t *qlo = reinterpret_cast<int32_t *>(ws + P.qlo_off);
  if (st == RA_OK && r->doc_start)
    st = hip_check(ra::launch_gather_i32(r->doc_start, pos + static_cast<int64_t>(r->rank) * P.c,
                                         qlo, P.c, sc),
                   "ra_ring_bwd: document starts");
  if (st != RA_OK) return st;

  ra::BwdEvents *ev = nullptr;
  if (P.ring && !serialize) {
    st = ra::bwd_events(&ev);
    // The copy stream reads slots the caller may have just written on `compute`.
    if (st == RA_OK) st = hip_check(hipEventRecord(ev->start, sc), "ra_ring_bwd: event record");
    if (st == RA_OK) st = hip_check(hipStreamWaitEvent(sp, ev->start, 0), "ra_ring_bwd: wait");
    if (st != RA_OK) return st;
  }
  if (step_ev) {
    st = hip_check(hipEventRecord(step_ev[0], sc), "ra_ring_bwd: step event");
    if (st != RA_OK) return st;
  }

  ra::BwdArgs a{};
  a.q = q;
  a.dout = dout;
  a.lse = lse_t;
  a.delta = delta;
  a.hm = 1;
  a.dq = dq;
  a.s_q = P.c;
  a.s_kv = P.c;
  a.b = r->b;
  a.n_q = r->n_q;
  a.n_kv = r->n_kv;
  a.d = r->d;
  a.scale = r->scale > 0.f ? r->scale : 1.0f / std::sqrt(static_cast<float>(r->d));
  a.causal = r->causal;
  a.q_pos = pos + static_cast<int64_t>(r->rank) * P.c;
  a.q_lo = r->doc_start ? qlo : nullptr;
  const unsigned char *kc = static_cast<const unsigned char *>(k_chunks);
  const unsigned char *vc = static_cast<const unsigned char *>(v_chunks);
  const int N = r->N, rank = r->rank;
  const size_t EB = P.chunk_elems * 2, FB = P.chunk_elems * 4;  // bf16 / fp32 chunk bytes
  auto src_of = [&](int step) { return ((rank - step) % N + N) % N; };
  auto half = [&](int step) { return ws + P.buf_off[step & 1]; };
  hipStream_t cs = serialize ? sc : sp;
  auto copy_bytes = [&](void *dst, const void *from, size_t n, const char *what) {
    return hip_check(hipMemcpyAsync(dst, from, n, hipMemcpyDeviceToDevice, cs), what);
  };
  // Receive block `step`'s K, V and accumulated dK, dV into its buffer half.
  auto receive = [&](int step) -> ra_status {
    const size_t j = static_cast<size_t>(src_of(step));
    unsigned char *h = half(step);
    ra_status s2 = copy_bytes(h + P.kb, kc + j * EB, EB, "ra_ring_bwd: receive K");
    if (s2 == RA_OK) s2 = copy_bytes(h + P.vb, vc + j * EB, EB, "ra_ring_bwd: receive V");
    if (s2 == RA_OK)
      s2 = copy_bytes(h + P.dkb, dk_chunks + j * P.chunk_elems, FB, "ra_ring_bwd: receive dK");
    if (s2 == RA_OK)
      s2 = copy_bytes(h + P.dvb, dv_chunks + j * P.chunk_elems, FB, "ra_ring_bwd: receive dV");
    if (s2 == RA_OK && !serialize)
      s2 = hip_check(hipEventRecord(ev->ready[step & 1], sp), "ra_ring_bwd: record ready");
    return s2;
  };
  // Send block `step`'s updated dK, dV on (back to its slot) once its kernels ran.
  auto send = [&](int step) -> ra_status {
    const size_t j = static_cast<size_t>(src_of(step));
    unsigned char *h = half(step);
    ra_status s2 = RA_OK;
    if (!serialize) s2 = hip_check(hipStreamWaitEvent(sp, ev->done[step & 1], 0), "ra_ring_bwd: wait done");
    if (s2 == RA_OK)
      s2 = copy_bytes(dk_chunks + j * P.chunk_elems, h + P.dkb, FB, "ra_ring_bwd: send dK");
    if (s2 == RA_OK)
      s2 = copy_bytes(dv_chunks + j * P.chunk_elems, h + P.dvb, FB, "ra_ring_bwd: send dV");
    return s2;
  };

  if (P.ring) {
    st = receive(0);
    if (st == RA_OK) st = receive(1);
    if (st != RA_OK) return st;
  }
  for (int step = 0; step < N; ++step) {
    const int src = src_of(step);
    // A block that no query of this rank can see (causal rule; step 0, the
    // rank's own chunk, never is) gets no contribution: no kernel runs, and
    // its dK, dV pass through unchanged.
    const bool skip = step > 0 && r->causal && ra::causally_empty(r->kind, r->S, N, rank, src);
    if (P.ring) {
      unsigned char *h = half(step);
      a.k = h + P.kb;
      a.v = h + P.vb;
      a.dk = reinterpret_cast<float *>(h + P.dkb);
      a.dv = reinterpret_cast<float *>(h + P.dvb);
      if (!serialize)
        st = hip_check(hipStreamWaitEvent(sc, ev->ready[step & 1], 0), "ra_ring_bwd: wait ready");
    } else {
      a.k = kc + static_cast<size_t>(src) * EB;
      a.v = vc + static_cast<size_t>(src) * EB;
      a.dk = dk_chunks + static_cast<size_t>(src) * P.chunk_elems;
      a.dv = dv_chunks + static_cast<size_t>(src) * P.chunk_elems;
    }
    a.kv_pos = pos + static_cast<int64_t>(src) * P.c;
    if (st == RA_OK && !skip)
      st = hip_check(ra::launch_attn_bwd_bf16(a, sc), "ra_ring_bwd: backward launch");
    if (st == RA_OK && P.ring && !serialize)
      st = hip_check(hipEventRecord(ev->done[step & 1], sc), "ra_ring_bwd: record done");
    if (st == RA_OK && step_ev)
      st = hip_check(hipEventRecord(step_ev[step + 1], sc), "ra_ring_bwd: step event");
    if (st == RA_OK && P.ring) st = send(step);
    if (st == RA_OK && P.ring && step + 2 < N) st = receive(step + 2);
    if (st != RA_OK) return st;
  }
  if (P.ring && !serialize) {
    // `compute` is ordered after the last send.
    st = hip_check(hipEventRecord(ev->sent, sp), "ra_ring_bwd: record sent");
    if (st == RA_OK) st = hip_check(hipStreamWaitEvent(sc, ev->sent, 0), "ra_ring_bwd: join copies");
  }
  return st;
}
