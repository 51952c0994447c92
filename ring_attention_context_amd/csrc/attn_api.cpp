// ra_block_attn_fwd: argument checks and dispatch to the bf16 (MFMA) or
// float32 attention kernel. The block statistics computed are those of
// "Context Parallelism and Ring Attention" §3 (m_b, l_b, o_b, lse_b).
#include <cmath>

#include "ra_internal.h"

namespace ra {

ra_status validate_attn(const ra_attn_desc *d, const void *q, const void *k, const void *v,
                        const void *o, const void *lse) {
  if (!d) return fail(RA_ERR_INVALID_ARG, "attention: desc is NULL");
  if (d->b < 0 || d->n_q < 1 || d->n_kv < 1 || d->s_q < 0 || d->s_kv < 0)
    return fail(RA_ERR_INVALID_ARG, "attention: negative size or zero heads");
  if (d->n_q % d->n_kv)
    return fail(RA_ERR_INVALID_ARG, "attention: n_q = %d not a multiple of n_kv = %d", d->n_q,
                d->n_kv);
  if (d->s_q > INT32_MAX || d->s_kv > INT32_MAX)
    return fail(RA_ERR_INVALID_ARG, "attention: more than 2^31 - 1 rows");
  if (!(d->scale >= 0.f) || std::isinf(d->scale))
    return fail(RA_ERR_INVALID_ARG, "attention: scale must be finite and >= 0");
  if (d->v_layout != RA_V_ROWS && d->v_layout != RA_V_TRANSPOSED)
    return fail(RA_ERR_INVALID_ARG, "attention: unknown v_layout %d", d->v_layout);
  if (d->v_layout == RA_V_TRANSPOSED) {
    if (d->dtype != RA_BF16)
      return fail(RA_ERR_UNSUPPORTED, "attention: RA_V_TRANSPOSED needs bf16");
    if (d->s_kv % 8)
      return fail(RA_ERR_INVALID_ARG, "attention: RA_V_TRANSPOSED needs s_kv %% 8 == 0");
    if (!vt_addressable(d->d, d->s_kv))
      return fail(RA_ERR_UNSUPPORTED,
                  "attention: RA_V_TRANSPOSED needs d * s_kv * 2 < 2^31 bytes (s_kv = %lld)",
                  static_cast<long long>(d->s_kv));
  }
  if (d->causal != 0 && d->causal != 1)
    return fail(RA_ERR_INVALID_ARG, "attention: causal must be 0 or 1");
  if (d->q_doc_start && !d->causal)
    return fail(RA_ERR_UNSUPPORTED, "attention: a document mask needs causal = 1");
  if (d->dtype == RA_BF16) {
    if (d->d != 128) return fail(RA_ERR_UNSUPPORTED, "attention: bf16 needs d = 128 (got %d)", d->d);
  } else if (d->dtype == RA_F32) {
    if (d->d != 64 && d->d != 128)
      return fail(RA_ERR_UNSUPPORTED, "attention: f32 needs d = 64 or 128 (got %d)", d->d);
  } else {
    return fail(RA_ERR_UNSUPPORTED, "attention: unknown dtype %d", d->dtype);
  }
  const bool any_q = d->b > 0 && d->s_q > 0;
  if (any_q) {
    if (!q || !o || !lse) return fail(RA_ERR_INVALID_ARG, "attention: NULL q / o / lse");
    if (!aligned16(q) || !aligned16(o))
      return fail(RA_ERR_INVALID_ARG, "attention: q / o not 16-byte aligned");
    if (d->causal && !d->q_pos) return fail(RA_ERR_INVALID_ARG, "attention: causal needs q_pos");
  }
  if (d->b > 0 && d->s_kv > 0) {
    if (!k || !v) return fail(RA_ERR_INVALID_ARG, "attention: NULL k / v");
    if (!aligned16(k) || !aligned16(v))
      return fail(RA_ERR_INVALID_ARG, "attention: k / v not 16-byte aligned");
    if (d->causal && !d->kv_pos) return fail(RA_ERR_INVALID_ARG, "attention: causal needs kv_pos");
  }
  return RA_OK;
}

}  // namespace ra

extern "C" ra_status ra_block_attn_fwd(const ra_attn_desc *desc, const void *q, const void *k,
                                       const void *v, float *o_b, float *lse_b, void *stream) {
  ra::clear_error();
  ra_status st = ra::validate_attn(desc, q, k, v, o_b, lse_b);
  if (st != RA_OK) return st;
  if (desc->b == 0 || desc->s_q == 0) return RA_OK;
  ra::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o_b;
  a.lse = lse_b;
  a.q_pos = desc->q_pos;
  a.kv_pos = desc->kv_pos;
  a.q_lo = desc->q_doc_start;
  a.s_q = desc->s_q;
  a.s_kv = desc->s_kv;
  a.b = desc->b;
  a.n_q = desc->n_q;
  a.n_kv = desc->n_kv;
  a.d = desc->d;
  a.scale = desc->scale > 0.f ? desc->scale : 1.0f / std::sqrt(static_cast<float>(desc->d));
  a.causal = desc->causal;
  a.merge = 0;
  a.v_layout = desc->v_layout;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = desc->dtype == RA_BF16 ? ra::launch_attn_bf16(a, s) : ra::launch_attn_f32(a, s);
  return ra::hip_check(err, "ra_block_attn_fwd launch");
}
