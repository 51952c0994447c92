// Float32 block attention (correctness-grade path for float32 inputs).
//
// Computes the block statistics of "Context Parallelism and Ring Attention"
// §3 for one key block, scanning the keys tile by tile with the running
// max / sum / unnormalised output update the same section describes for a
// single GPU, then normalising: o_b = acc / l, lse_b = m + ln l. Causal
// masking follows §5 on the original positions (§6 "the cost of reordering").
//
// One workgroup = 32 query rows of one head; 8 threads per row. Q, K, V tiles
// and the probabilities of the current tile are staged in LDS. Plain fp32
// FMAs, expf / logf: this path exists for float32 accuracy, not speed.
#include <climits>

#include "ra_internal.h"

namespace ra {
namespace {

constexpr int F_BQ = 32;   // query rows per workgroup
constexpr int F_BK = 32;   // keys per tile
constexpr int F_TPR = 8;   // threads per query row

template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  __shared__ float qs[F_BQ][D + 1];
  __shared__ float ks[F_BK][D + 1];
  __shared__ float vs[F_BK][D + 1];
  __shared__ float ps[F_BQ][F_BK + 1];
  __shared__ int kpos[F_BK];

  constexpr int DPT = D / F_TPR;
  const int tid = threadIdx.x;
  const int r = tid / F_TPR;
  const int t8 = tid % F_TPR;

  const int64_t nqb = (a.s_q + F_BQ - 1) / F_BQ;
  const int64_t blk = blockIdx.x;
  const int64_t qb = blk % nqb;
  const int h = static_cast<int>((blk / nqb) % a.n_q);
  const int bi = static_cast<int>(blk / (nqb * a.n_q));
  const int g = a.n_q / a.n_kv;
  const int kvh = h / g;

  const int64_t tok0 = qb * F_BQ;
  const int64_t tok = tok0 + r;
  const bool tok_ok = tok < a.s_q;
  const float *q = static_cast<const float *>(a.q);
  const float *k = static_cast<const float *>(a.k);
  const float *v = static_cast<const float *>(a.v);

  // Query tile -> LDS (rows past s_q are zero and never stored).
  for (int i = tid; i < F_BQ * D; i += 256) {
    const int rr = i / D, e = i % D;
    const int64_t tt = tok0 + rr;
    qs[rr][e] = tt < a.s_q ? q[((bi * a.s_q + tt) * a.n_q + h) * D + e] : 0.f;
  }
  // Query position; non-causal uses the smallest value so every key is visible.
  const int qpos = !a.causal ? INT_MAX : (tok_ok ? a.q_pos[tok] : INT_MIN);
  // First visible key position (document mask); INT_MIN without one.
  const int qlo = a.q_lo && tok_ok ? a.q_lo[tok] : INT_MIN;

  float m_run = -INFINITY, l_run = 0.f;
  float acc[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) acc[i] = 0.f;

  for (int64_t key0 = 0; key0 < a.s_kv; key0 += F_BK) {
    __syncthreads();
    for (int i = tid; i < F_BK * D; i += 256) {
      const int kk = i / D, e = i % D;
      const int64_t key = key0 + kk;
      const bool ok = key < a.s_kv;
      const int64_t off = ((bi * a.s_kv + key) * a.n_kv + kvh) * D + e;
      ks[kk][e] = ok ? k[off] : 0.f;
      vs[kk][e] = ok ? v[off] : 0.f;
    }
    if (tid < F_BK) {
      const int64_t key = key0 + tid;
      // Keys past the block are never visible; non-causal keys always are.
      kpos[tid] = key >= a.s_kv ? INT_MAX : (a.causal ? a.kv_pos[key] : INT_MIN);
    }
    __syncthreads();

    // Scores of this row's keys t8, t8 + 8, t8 + 16, t8 + 24.
    float s[F_BK / F_TPR];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < F_BK / F_TPR; ++j) {
      const int kk = t8 + F_TPR * j;
      float dot = 0.f;
#pragma unroll 16
      for (int e = 0; e < D; ++e) dot = fmaf(qs[r][e], ks[kk][e], dot);
      const bool vis = kpos[kk] <= qpos && kpos[kk] >= qlo && key0 + kk < a.s_kv;
      s[j] = vis ? dot * a.scale : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
#pragma unroll
    for (int off = 1; off < F_TPR; off <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = expf(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < F_BK / F_TPR; ++j) {
      const float p = expf(s[j] - m_use);
      psum += p;
      ps[r][t8 + F_TPR * j] = p;
    }
#pragma unroll
    for (int off = 1; off < F_TPR; off <<= 1) psum += __shfl_xor(psum, off);
    l_run = alpha * l_run + psum;
    m_run = m_new;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      const int e = t8 + F_TPR * i;
      float x = alpha * acc[i];
#pragma unroll 8
      for (int kk = 0; kk < F_BK; ++kk) x = fmaf(ps[r][kk], vs[kk][e], x);
      acc[i] = x;
    }
  }

  if (!tok_ok) return;
  // A row with no visible key in this block merges the identity: unchanged.
  if (a.merge && !(l_run > 0.f)) return;
  const int64_t row = (bi * a.s_q + tok) * a.n_q + h;
  const float lse_new = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float w_old = 0.f, w_new = 1.f, lse_out = lse_new;
  if (a.merge) {
    const float lse_old = a.lse[row];
    const float m = fmaxf(lse_old, lse_new);
    if (m == -INFINITY) {
      w_new = 0.f;
      lse_out = -INFINITY;
    } else {
      lse_out = m + logf(expf(lse_old - m) + expf(lse_new - m));
      w_old = expf(lse_old - lse_out);
      w_new = expf(lse_new - lse_out);
    }
  }
  float *o = a.o + row * D;
#pragma unroll
  for (int i = 0; i < DPT; ++i) {
    const int e = t8 + F_TPR * i;
    const float onew = acc[i] * inv;
    o[e] = a.merge ? w_old * o[e] + w_new * onew : onew;
  }
  if (t8 == 0) a.lse[row] = lse_out;
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t stream) {
  const int64_t nqb = (a.s_q + F_BQ - 1) / F_BQ;
  const int64_t blocks = nqb * a.n_q * a.b;
  if (blocks == 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (a.d == 64)
    attn_f32_kernel<64><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(a);
  else
    attn_f32_kernel<128><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ra
