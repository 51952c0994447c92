// Internal declarations shared by the host entry points and the kernels of
// libringattn. Not part of the public interface (include/ringattn.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ringattn.h"

namespace ra {

// Arguments of one attention launch: the queries of a shard against one block
// of keys. Layouts as in ringattn.h; o / lse are the block outputs when
// merge == 0, or the running (o, lse) to merge into when merge == 1.
struct AttnArgs {
  const void *q;
  const void *k;
  const void *v;
  float *o;
  float *lse;
  const int32_t *q_pos;
  const int32_t *kv_pos;
  int64_t s_q;
  int64_t s_kv;
  int32_t b;
  int32_t n_q;
  int32_t n_kv;
  int32_t d;
  float scale;   // softmax scale (natural units), > 0
  int32_t causal;
  int32_t merge;
  int32_t v_layout;  // ra_v_layout of v (RA_V_TRANSPOSED: [b, n_kv, d, s_kv], bf16 only)
  const int32_t *q_lo;  // optional [s_q]: first visible key position (document start)
  // optional second key block of s_kv keys (bf16, V^T, no q_lo): scanned after
  // the first, so one launch covers both blocks (one merge into o / lse)
  const void *k2;
  const void *v2;
  const int32_t *kv_pos2;
};

// Arguments of one backward launch (one key block against a query shard):
// q, dout [b, s_q, n_q, d]; k, v [b, s_kv, n_kv, d]; lse, delta [b, s_q, n_q]
// (the global lse of the forward and D = dout . o) or, with hm, head-major
// [b, n_q, s_q] with the lse in log2 units (+inf for a query with no visible
// key); dq [b, s_q, n_q, d] and dk, dv [b, s_kv, n_kv, d] float32,
// accumulated into.
struct BwdArgs {
  const void *q;
  const void *k;
  const void *v;
  const void *dout;
  const float *lse;
  const float *delta;
  int32_t hm;
  float *dq;
  float *dk;
  float *dv;
  const int32_t *q_pos;
  const int32_t *kv_pos;
  const int32_t *q_lo;  // optional [s_q]: first visible key position (document start)
  // optional [s_kv]: the dk/dv row of key j for batch 0 (batch bi adds
  // bi * kv_row_bstride); without it key j of batch bi is row bi * s_kv + j
  const int32_t *kv_row;
  int64_t kv_row_bstride;
  int64_t s_q;
  int64_t s_kv;
  int32_t b;
  int32_t n_q;
  int32_t n_kv;
  int32_t d;
  float scale;
  int32_t causal;
};

// Records a failure message for ra_last_error() and returns the status.
ra_status fail(ra_status st, const char *fmt, ...);
// Checks a HIP return code; records the HIP error text on failure.
ra_status hip_check(hipError_t err, const char *what);
// Clears the thread's last-error message.
void clear_error();

// Validates an attention descriptor plus its data pointers.
ra_status validate_attn(const ra_attn_desc *d, const void *q, const void *k, const void *v,
                        const void *o, const void *lse);

// Kernel launchers (enqueue only; return the launch status).
hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t stream);
hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t stream);
hipError_t launch_lse_merge(int64_t rows, int32_t d, float *o, float *lse, const float *o_b,
                            const float *lse_b, hipStream_t stream);
// Checks shared by every call that takes an ra_ring_desc (all but its flags).
ra_status check_ring_desc(const ra_ring_desc *r);
hipError_t launch_positions(int32_t kind, int64_t S, int32_t N, int32_t *pos, hipStream_t stream);
// Host: global position of local token a of rank `rank` under map `kind`.
int64_t map_position(int32_t kind, int64_t S, int32_t N, int32_t rank, int64_t a);
// Host: true when no query of rank `rank` can see any key of rank `src`'s
// chunk under the causal rule (the maps are increasing, so this compares the
// chunk's first key with the rank's last query).
inline bool causally_empty(int32_t kind, int64_t S, int32_t N, int32_t rank, int32_t src) {
  const int64_t c = S / N;
  return c > 0 && map_position(kind, S, N, src, 0) > map_position(kind, S, N, rank, c - 1);
}
// D = dout . o per row (rows = b * s * n_q, d elements each; esize of dout 2 or 4).
hipError_t launch_bwd_delta(int64_t rows, int32_t d, int32_t esize, const void *dout,
                            const float *o, float *delta, hipStream_t stream);
// The backward's per-row arrays, head-major [b, n_q, s]: D = dout . o and the
// lse in log2 units (+inf for -inf); dout bf16 [b, s, n_q, 128], o, lse as
// for the forward's outputs.
hipError_t launch_bwd_prep(int32_t b, int64_t s, int32_t n_q, const void *dout, const float *o,
                           const float *lse, float *delta_t, float *lse_t, hipStream_t stream);
// dq, dk, dv += the gradient contributions of one key block (bf16, d = 128).
hipError_t launch_attn_bwd_bf16(const BwdArgs &a, hipStream_t stream);
// p[0 .. n) = 0 (a kernel, so that callers may capture it in a graph).
hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t stream);
// v [b, s, n_kv, d] -> vt [b, n_kv, d, s]; esize = 2 or 4 bytes per element.
// out[i] = src[idx[i]], i < n.
hipError_t launch_gather_i32(const int32_t *src, const int32_t *idx, int32_t *out, int64_t n,
                             hipStream_t stream);
hipError_t launch_v_transpose(int32_t b, int64_t s, int32_t n_kv, int32_t d, int32_t esize,
                              const void *v, void *vt, hipStream_t stream);
// bf16 rows -> V^T [b, n_kv, d, s] with 16-byte accesses (s % 8 == 0, d % 8 == 0):
// position p of batch bi is row (src_row ? src_row[p] : p) + bi * bstride of src.
// With k_bytes > 0 the same launch also copies k_bytes (16-byte aligned, a
// multiple of 16, at most b * s * n_kv * d * 2 rounded up to whole tiles)
// from k_src to k_dst.
hipError_t launch_rows_to_vt(const void *src, void *vt, const int32_t *src_row, int64_t bstride,
                             int32_t b, int64_t s, int32_t n_kv, int32_t d, hipStream_t stream,
                             const void *k_src = nullptr, void *k_dst = nullptr,
                             size_t k_bytes = 0);

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// V^T [.., d, s_kv] of one (batch, kv head) must be addressable with 31-bit
// buffer offsets: the attention kernel reads a V^T tile through one buffer
// descriptor whose records span all d rows of s_kv keys.
inline bool vt_addressable(int64_t d, int64_t s_kv) { return d * s_kv * 2 < (int64_t{1} << 31); }

}  // namespace ra
