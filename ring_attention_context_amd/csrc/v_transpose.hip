// ra_v_transpose: v [b, s, n_kv, d] -> vt [b, n_kv, d, s].
//
// Data movement only. The bf16 attention kernel reads V^T tiles (d-rows of
// keys) with plain 16-byte LDS reads; the ring produces that layout for each
// incoming chunk on its copy stream, and the all-gather forward gathers V
// straight into it. HBM-bound: each element is read once and written once,
// through a 64 x 64 LDS tile so that both the reads (along d) and the writes
// (along s) are contiguous across the wave.
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int TS = 64;  // tile edge (tokens and channels)

template <typename T>
__global__ __launch_bounds__(256) void v_transpose_kernel(const T *__restrict__ v,
                                                          T *__restrict__ vt, int64_t s,
                                                          int32_t n_kv, int32_t d) {
  // +2 elements of padding: a column read walks rows at an odd dword stride.
  __shared__ T tile[TS][TS + 2];
  const int tid = threadIdx.x;
  const int64_t s0 = static_cast<int64_t>(blockIdx.x) * TS;
  const int e0 = blockIdx.y * TS;
  const int bh = blockIdx.z;  // bi * n_kv + h
  const int bi = bh / n_kv, h = bh - bi * n_kv;
  const int c = tid & (TS - 1), r0 = tid >> 6;
#pragma unroll
  for (int i = 0; i < TS / 4; ++i) {
    const int r = r0 + 4 * i;
    const int64_t si = s0 + r;
    const int e = e0 + c;
    T x = T(0);
    if (si < s && e < d) x = v[((bi * s + si) * n_kv + h) * d + e];
    tile[r][c] = x;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TS / 4; ++i) {
    const int r = r0 + 4 * i;  // channel within the tile
    const int64_t si = s0 + c;
    const int e = e0 + r;
    if (si < s && e < d) vt[(static_cast<int64_t>(bh) * d + e) * s + si] = tile[c][r];
  }
}

// bf16 with s % 8 == 0 and d % 8 == 0: 16-byte accesses on both sides.
// Position p of batch bi is source row (src_row ? src_row[p] : p) + bi *
// bstride of `src` [rows, n_kv, d]; vt is [b, n_kv, d, s]. A workgroup moves a
// 64-position x 64-channel tile: 16-byte loads along the channels of each
// position's row, 16-byte stores along the positions of each channel row.
// 16-byte chunk k of tile row r sits at chunk k ^ (r/8 % 8), so the column
// reads of the store phase hit eight different chunks (no bank conflicts)
// while the row writes stay contiguous. Positions past s read as zero and are
// not stored (a stored 8-position chunk is whole).
// Optionally (k_bytes > 0, a multiple of 16) workgroup w also copies bytes
// [w * 8 KiB, (w + 1) * 8 KiB) of k_src to k_dst: a tile of V^T is 8 KiB, so
// the grid covers a K chunk of the same shape, and a ring step's K and V
// arrive in one launch.
__global__ __launch_bounds__(256) void rows_to_vt_kernel(const uint16_t *__restrict__ src,
                                                         uint16_t *__restrict__ vt,
                                                         const int32_t *__restrict__ src_row,
                                                         int64_t bstride, int64_t s,
                                                         int32_t n_kv, int32_t d,
                                                         const unsigned char *__restrict__ k_src,
                                                         unsigned char *__restrict__ k_dst,
                                                         uint64_t k_bytes) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[TS * TS];
  const int tid = threadIdx.x;
  if (k_bytes) {
    const uint64_t wg = (static_cast<uint64_t>(blockIdx.z) * gridDim.y + blockIdx.y) * gridDim.x +
                        blockIdx.x;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint64_t off = wg * (TS * TS * 2) + k * 4096 + tid * 16;
      if (off < k_bytes)
        *reinterpret_cast<uint4 *>(k_dst + off) = *reinterpret_cast<const uint4 *>(k_src + off);
    }
  }
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * TS;
  const int e0 = blockIdx.y * TS;
  const int bh = blockIdx.z;  // bi * n_kv + h
  const int bi = bh / n_kv, h = bh - bi * n_kv;
  const int c8 = tid & 7;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int r = (tid >> 3) + 32 * k;
    const int64_t p = p0 + r;
    uint4 x = uint4{0, 0, 0, 0};
    if (p < s && e0 + c8 * 8 < d) {
      const int64_t row = (src_row ? src_row[p] : p) + static_cast<int64_t>(bi) * bstride;
      x = *reinterpret_cast<const uint4 *>(src + (row * n_kv + h) * d + e0 + c8 * 8);
    }
    *reinterpret_cast<uint4 *>(tile + r * TS + ((c8 ^ ((r >> 3) & 7)) << 3)) = x;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int e = (tid >> 3) + 32 * k;  // channel row of the tile
    const int pc = c8;                  // 8-position chunk
    const int64_t p = p0 + pc * 8;
    if (p >= s || e0 + e >= d) continue;
    uint16_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)  // tile row pc*8 + i, whose (row / 8) % 8 is pc
      v[i] = tile[(pc * 8 + i) * TS + (((e >> 3) ^ pc) << 3) + (e & 7)];
    uint4 y;
    y.x = v[0] | (static_cast<uint32_t>(v[1]) << 16);
    y.y = v[2] | (static_cast<uint32_t>(v[3]) << 16);
    y.z = v[4] | (static_cast<uint32_t>(v[5]) << 16);
    y.w = v[6] | (static_cast<uint32_t>(v[7]) << 16);
    *reinterpret_cast<uint4 *>(vt + (static_cast<int64_t>(bh) * d + e0 + e) * s + p) = y;
  }
}

}  // namespace

hipError_t launch_rows_to_vt(const void *src, void *vt, const int32_t *src_row, int64_t bstride,
                             int32_t b, int64_t s, int32_t n_kv, int32_t d, hipStream_t stream,
                             const void *k_src, void *k_dst, size_t k_bytes) {
  if (b == 0 || s == 0) return hipSuccess;
  const int64_t gx = (s + TS - 1) / TS, gy = (d + TS - 1) / TS;
  const int64_t gz = static_cast<int64_t>(b) * n_kv;
  if (gx > INT32_MAX || gz > 65535 || s % 8 || d % 8) return hipErrorInvalidValue;
  // The K copy: 16-byte units, and no more than the grid's 8 KiB per workgroup.
  if (k_bytes && (k_bytes % 16 || !k_src || !k_dst ||
                  static_cast<uint64_t>(k_bytes) >
                      static_cast<uint64_t>(gx) * gy * gz * (TS * TS * 2) ||
                  ((reinterpret_cast<uintptr_t>(k_src) | reinterpret_cast<uintptr_t>(k_dst)) & 15)))
    return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy), static_cast<unsigned>(gz));
  rows_to_vt_kernel<<<grid, 256, 0, stream>>>(static_cast<const uint16_t *>(src),
                                              static_cast<uint16_t *>(vt), src_row, bstride, s,
                                              n_kv, d, static_cast<const unsigned char *>(k_src),
                                              static_cast<unsigned char *>(k_dst), k_bytes);
  return hipGetLastError();
}

hipError_t launch_v_transpose(int32_t b, int64_t s, int32_t n_kv, int32_t d, int32_t esize,
                              const void *v, void *vt, hipStream_t stream) {
  if (b == 0 || s == 0) return hipSuccess;
  const int64_t gx = (s + TS - 1) / TS;
  const int64_t gy = (d + TS - 1) / TS;
  const int64_t gz = static_cast<int64_t>(b) * n_kv;
  if (gx > INT32_MAX || gz > 65535) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy), static_cast<unsigned>(gz));
  const bool a16 = ((reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(vt)) & 15) == 0;
  if (esize == 2 && s % 8 == 0 && d % 8 == 0 && a16)
    return launch_rows_to_vt(v, vt, nullptr, s, b, s, n_kv, d, stream);
  if (esize == 2)
    v_transpose_kernel<uint16_t><<<grid, 256, 0, stream>>>(static_cast<const uint16_t *>(v),
                                                           static_cast<uint16_t *>(vt), s, n_kv, d);
  else
    v_transpose_kernel<uint32_t><<<grid, 256, 0, stream>>>(static_cast<const uint32_t *>(v),
                                                           static_cast<uint32_t *>(vt), s, n_kv, d);
  return hipGetLastError();
}

}  // namespace ra

extern "C" ra_status ra_v_transpose(int32_t b, int64_t s, int32_t n_kv, int32_t d, int32_t dtype,
                                    const void *v, void *vt, void *stream) {
  ra::clear_error();
  if (b < 0 || s < 0 || n_kv < 1 || d < 1)
    return ra::fail(RA_ERR_INVALID_ARG, "ra_v_transpose: negative size or zero heads / d");
  if (dtype != RA_BF16 && dtype != RA_F32)
    return ra::fail(RA_ERR_UNSUPPORTED, "ra_v_transpose: unknown dtype %d", dtype);
  if (static_cast<int64_t>(b) * n_kv > 65535)
    return ra::fail(RA_ERR_INVALID_ARG, "ra_v_transpose: b * n_kv > 65535");
  if (b == 0 || s == 0) return RA_OK;
  if (!v || !vt) return ra::fail(RA_ERR_INVALID_ARG, "ra_v_transpose: NULL v / vt");
  const int32_t esize = dtype == RA_BF16 ? 2 : 4;
  const uintptr_t bytes = static_cast<uintptr_t>(b) * s * n_kv * d * esize;
  const uintptr_t pv = reinterpret_cast<uintptr_t>(v), pt = reinterpret_cast<uintptr_t>(vt);
  if (pv < pt + bytes && pt < pv + bytes)
    return ra::fail(RA_ERR_INVALID_ARG, "ra_v_transpose: v and vt overlap");
  return ra::hip_check(ra::launch_v_transpose(b, s, n_kv, d, esize, v, vt,
                                              static_cast<hipStream_t>(stream)),
                       "ra_v_transpose launch");
}
