// ra_partition: the token maps of "Context Parallelism and Ring Attention"
// §2 (contiguous segments) and §6 (zig-zag: rank i holds chunks C_i and
// C_{2N-1-i} of c/2 tokens; striped: token p belongs to rank p mod N).
// Host only; no HIP call, so it also runs on machines without a GPU.
#include <cstdint>

#include "ra_internal.h"

extern "C" ra_status ra_partition(int32_t kind, int64_t S, int32_t N, int32_t rank,
                                  int32_t *out_pos) {
  using ra::fail;
  ra::clear_error();
  if (N < 1) return fail(RA_ERR_INVALID_ARG, "ra_partition: N = %d must be >= 1", N);
  if (rank < 0 || rank >= N)
    return fail(RA_ERR_INVALID_ARG, "ra_partition: rank %d outside [0, %d)", rank, N);
  if (S < 0 || S > INT32_MAX)
    return fail(RA_ERR_INVALID_ARG, "ra_partition: S = %lld outside [0, 2^31)", (long long)S);
  if (S % N) return fail(RA_ERR_INVALID_ARG, "ra_partition: S %% N != 0");
  const int64_t c = S / N;
  if (c > 0 && !out_pos) return fail(RA_ERR_INVALID_ARG, "ra_partition: out_pos is NULL");
  switch (kind) {
    case RA_PART_CONTIGUOUS:
      for (int64_t a = 0; a < c; ++a) out_pos[a] = static_cast<int32_t>(rank * c + a);
      return RA_OK;
    case RA_PART_ZIGZAG: {
      if (S % (2 * static_cast<int64_t>(N)))
        return fail(RA_ERR_INVALID_ARG, "ra_partition: zig-zag needs S %% 2N == 0");
      const int64_t h = c / 2;
      const int64_t late = 2 * static_cast<int64_t>(N) - 1 - rank;
      for (int64_t a = 0; a < h; ++a) out_pos[a] = static_cast<int32_t>(rank * h + a);
      for (int64_t a = 0; a < h; ++a) out_pos[h + a] = static_cast<int32_t>(late * h + a);
      return RA_OK;
    }
    case RA_PART_STRIPED:
      for (int64_t a = 0; a < c; ++a) out_pos[a] = static_cast<int32_t>(a * N + rank);
      return RA_OK;
    default:
      return fail(RA_ERR_INVALID_ARG, "ra_partition: unknown kind %d", kind);
  }
}

namespace ra {

// Global position of local token a of rank `rank` (the maps above; arguments
// already validated by the caller).
int64_t map_position(int32_t kind, int64_t S, int32_t N, int32_t rank, int64_t a) {
  const int64_t c = S / N;
  if (kind == RA_PART_CONTIGUOUS) return rank * c + a;
  if (kind == RA_PART_ZIGZAG) {
    const int64_t h = c / 2;
    return a < h ? rank * h + a : (2 * static_cast<int64_t>(N) - 1 - rank) * h + (a - h);
  }
  return a * N + rank;
}

}  // namespace ra
