// ra_lse_merge: the boxed two-block merge of "Context Parallelism and Ring
// Attention" §3 in its stable form (every exponent <= 0):
//   M = max(lse, lse_b), lse' = M + ln(e^{lse-M} + e^{lse_b-M}),
//   o' = e^{lse-lse'} o + e^{lse_b-lse'} o_b,
// applied in place to float32 rows. The kernel is HBM-bound: per row it
// reads o, o_b, lse, lse_b and writes o, lse (12 d + 12 bytes). A thread
// owns U of the d/4 16-byte units of one row (U = min(4, d/4)), so the four
// transcendentals of the weights are paid once per 16 U bytes: with T = d/4/U
// threads per row, thread j takes units j, j + T, ..., so each load and store
// instruction of a wave covers contiguous runs of 16 T bytes. d is a power of
// two, so rows and units come from shifts. o and o_b are streamed with
// nontemporal loads and stores: every byte is touched once.
#include "ra_internal.h"

namespace ra {
namespace {
typedef float fv4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void lse_merge_kernel(int64_t n_units, int32_t shift,
                                                        int32_t d4, float *o, float *lse,
                                                        const float *o_b, const float *lse_b) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  fv4 *o4 = reinterpret_cast<fv4 *>(o);
  const fv4 *ob4 = reinterpret_cast<const fv4 *>(o_b);
  constexpr int LU = U == 4 ? 2 : U == 2 ? 1 : 0;
  const int32_t tpr = d4 >> LU;   // threads per row
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < n_units;
       u += stride) {
    const int64_t r = u >> (shift - LU);  // row (d4 = 1 << shift units per row)
    const int32_t c = static_cast<int32_t>(u & (tpr - 1));
    const int64_t i = (r << shift) + c;   // this thread's first unit; then every tpr-th
    fv4 x[U], y[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      x[k] = __builtin_nontemporal_load(o4 + i + k * tpr);
      y[k] = __builtin_nontemporal_load(ob4 + i + k * tpr);
    }
    const float l1 = lse[r];
    const float l2 = lse_b[r];
    const float m = fmaxf(l1, l2);
    float w1 = 0.f, w2 = 0.f, out = -INFINITY;
    if (m != -INFINITY) {
      out = m + logf(expf(l1 - m) + expf(l2 - m));
      w1 = expf(l1 - out);
      w2 = expf(l2 - out);
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      fv4 z;
#pragma unroll
      for (int j = 0; j < 4; ++j) z[j] = w1 * x[k][j] + w2 * y[k][j];
      __builtin_nontemporal_store(z, o4 + i + k * tpr);
    }
    // Every thread of a row sits in the same wave (tpr divides 64) and reads
    // lse[r] before this store is issued.
    if (c == 0) lse[r] = out;
  }
}

}  // namespace

hipError_t launch_lse_merge(int64_t rows, int32_t d, float *o, float *lse, const float *o_b,
                            const float *lse_b, hipStream_t stream) {
  const int32_t d4 = d / 4;  // a power of two, 1 .. 64
  int32_t shift = 0;
  while ((1 << shift) < d4) ++shift;
  const int U = d4 >= 4 ? 4 : d4;
  const int64_t n_units = rows * d4 / U;
  if (n_units == 0) return hipSuccess;
  int64_t blocks = (n_units + 255) / 256;
  // Enough waves to cover the 256 CUs several times; the rest is grid-stride.
  if (blocks > 256 * 16) blocks = 256 * 16;
  const unsigned g = static_cast<unsigned>(blocks);
  if (U == 4)
    lse_merge_kernel<4><<<g, 256, 0, stream>>>(n_units, shift, d4, o, lse, o_b, lse_b);
  else if (U == 2)
    lse_merge_kernel<2><<<g, 256, 0, stream>>>(n_units, shift, d4, o, lse, o_b, lse_b);
  else
    lse_merge_kernel<1><<<g, 256, 0, stream>>>(n_units, shift, d4, o, lse, o_b, lse_b);
  return hipGetLastError();
}

}  // namespace ra

extern "C" ra_status ra_lse_merge(int64_t rows, int32_t d, float *o, float *lse,
                                  const float *o_b, const float *lse_b, void *stream) {
  using ra::fail;
  ra::clear_error();
  if (rows < 0) return fail(RA_ERR_INVALID_ARG, "ra_lse_merge: rows < 0");
  if (d < 4 || d > 256 || (d & (d - 1)))
    return fail(RA_ERR_INVALID_ARG, "ra_lse_merge: d = %d must be a power of two in [4, 256]", d);
  if (rows == 0) return RA_OK;
  if (!o || !lse || !o_b || !lse_b) return fail(RA_ERR_INVALID_ARG, "ra_lse_merge: NULL pointer");
  if (!ra::aligned16(o) || !ra::aligned16(o_b))
    return fail(RA_ERR_INVALID_ARG, "ra_lse_merge: o / o_b must be 16-byte aligned");
  return ra::hip_check(
      ra::launch_lse_merge(rows, d, o, lse, o_b, lse_b, static_cast<hipStream_t>(stream)),
      "ra_lse_merge launch");
}
