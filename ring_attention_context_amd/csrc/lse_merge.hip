// ra_lse_merge: the boxed two-block merge of "Context Parallelism and Ring
// Attention" §3 in its stable form (every exponent <= 0):
//   M = max(lse, lse_b), lse' = M + ln(e^{lse-M} + e^{lse_b-M}),
//   o' = e^{lse-lse'} o + e^{lse_b-lse'} o_b,
// applied in place to float32 rows. The kernel is HBM-bound: per row it
// reads o, o_b, lse, lse_b and writes o, lse (12 d + 12 bytes). Each thread
// owns 16 bytes of a row, so a wave moves whole 512-byte rows at d = 128
// with fully coalesced accesses.
#include "ra_internal.h"

namespace ra {
namespace {

__global__ __launch_bounds__(256) void lse_merge_kernel(int64_t rows, int32_t d4, float *o,
                                                        float *lse, const float *o_b,
                                                        const float *lse_b) {
  const int64_t n = rows * d4;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  float4 *o4 = reinterpret_cast<float4 *>(o);
  const float4 *ob4 = reinterpret_cast<const float4 *>(o_b);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += stride) {
    const int64_t r = i / d4;
    const int32_t c = static_cast<int32_t>(i - r * d4);
    const float l1 = lse[r];
    const float l2 = lse_b[r];
    const float m = fmaxf(l1, l2);
    float w1 = 0.f, w2 = 0.f, out = -INFINITY;
    if (m != -INFINITY) {
      out = m + logf(expf(l1 - m) + expf(l2 - m));
      w1 = expf(l1 - out);
      w2 = expf(l2 - out);
    }
    const float4 x = o4[i];
    const float4 y = ob4[i];
    float4 z;
    z.x = w1 * x.x + w2 * y.x;
    z.y = w1 * x.y + w2 * y.y;
    z.z = w1 * x.z + w2 * y.z;
    z.w = w1 * x.w + w2 * y.w;
    o4[i] = z;
    // Every lane of a row sits in the same wave (d4 divides 64) and reads
    // lse[r] before this store is issued.
    if (c == 0) lse[r] = out;
  }
}

}  // namespace

hipError_t launch_lse_merge(int64_t rows, int32_t d, float *o, float *lse, const float *o_b,
                            const float *lse_b, hipStream_t stream) {
  const int32_t d4 = d / 4;
  const int64_t n = rows * d4;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  // Enough waves to cover the 256 CUs several times; the rest is grid-stride.
  if (blocks > 256 * 16) blocks = 256 * 16;
  lse_merge_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(rows, d4, o, lse, o_b,
                                                                       lse_b);
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
