// Backward of block attention on gfx950: the gradient contributions of one
// key block, following the backward paragraph of "Context Parallelism and
// Ring Attention" §3. With the GLOBAL lse of a query, the probability of key j
// is p_j = e^{x_j - lse}, recomputable on any block alone; then
//   dv_j += p_j do,   dx_j = p_j (do . v_j - D),   D = do . o (per query),
// and by the chain rule (x = scale q . k)
//   dq += scale sum_j dx_j k_j,   dk_j += scale sum_q dx_j q.
// The causal rule of §5 applies on original positions, as in the forward.
//
// Three kernels:
//   * bwd_delta_kernel: D = do . o per (token, head) (HBM-bound);
//   * bwd_dq_kernel (bf16, d = 128): shaped like the forward kernel. A wave
//     owns 32 queries of one head with q and do in registers; 8 waves share
//     each 64-key K/V tile, staged by buffer loads straight into LDS. Per tile:
//     S^T = K Q^T and dP^T = V dO^T (K and V rows by ds_read_b128),
//     P^T = 2^(S^T scale log2 e - lse log2 e), dS^T = P^T (dP^T - D), and
//     dQ^T += K^T dS^T (K^T operands by the transposing ds_read_b64_tr_b16).
//     Every lane holds one query, so lse and D are per-lane constants. As in
//     the forward, the MFMAs of two tiles form one matrix phase and the
//     element-wise work a vector phase, which the two waves of a SIMD run in
//     opposite orders;
//   * bwd_dkdv_kernel (bf16, d = 128): a workgroup owns 128 keys of one
//     key/value head in four groups of 32, one group per SIMD, and walks the
//     blocks of 64 queries (q, do, lse, D, positions, staged in LDS) of every
//     query head of the GQA group in 32-row sub-blocks. Each SIMD runs two
//     waves with split roles: the producer holds the group's K and V rows and
//     computes A, S = Q K^T and dP = dO V^T (Q and dO rows by ds_read_b128),
//     and B, P and dS on the VALU, which it hands over through LDS in the
//     B-operand lane order; the consumer holds the dK^T and dV^T accumulators
//     and computes C, dV^T += dO^T P and dK^T += Q^T dS (dO^T and Q^T by the
//     transposing read). One barrier per sub-block moves the pipeline on: the
//     producer runs A of the next and B of the current sub-block while the
//     consumer runs C of the previous one, so the producer's exponentials
//     overlap the consumer's MFMAs on the same SIMD.
// P and dS enter the MFMAs as bf16; every accumulation is fp32. dq, dk and dv
// are float32 and ACCUMULATED into (+=): the ring adds one block per step.
#include <climits>
#include <cmath>
#include <type_traits>

#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))
#define INLINE __attribute__((always_inline))

constexpr int D = 128;
constexpr int ROW_B = D * 2;                 // bytes per bf16 row of d elements
constexpr float LOG2E = 1.4426950408889634f;
constexpr int BUF_DWORD3 = 0x00020000;

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : static_cast<int32_t>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0), n,
                                           BUF_DWORD3);
}

__device__ __forceinline__ void wait_own_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }


// Number of entries < p (lower bound) / <= p (upper bound) in a non-decreasing array.
__device__ __forceinline__ int64_t count_lt(const int32_t *pos, int64_t n, int32_t p) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (pos[mid] < p) lo = mid + 1; else hi = mid;
  }
  return lo;
}
__device__ __forceinline__ int64_t count_le(const int32_t *pos, int64_t n, int32_t p) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (pos[mid] <= p) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// The same counts found by the 64 lanes of a wave together: each round probes
// 64 evenly spaced entries of the remaining range and keeps the gap between
// the last probe that counts and the first that does not (about log64(n)
// dependent loads). LE: entries <= p, else < p. Call with all lanes active;
// the result is uniform.
template <bool LE>
__device__ __forceinline__ int64_t wave_count(const int32_t *pos, int64_t n, int32_t p, int lane) {
  int64_t lo = 0, hi = n;  // the count lies in [lo, hi]
  while (lo < hi) {
    const int64_t step = (hi - lo + 63) / 64;
    const int64_t idx = lo + lane * step;
    bool in = false;
    if (idx < hi) {
      const int32_t v = pos[idx];
      in = LE ? v <= p : v < p;
    }
    const int cnt = __popcll(__ballot(in));  // the probes that count form a prefix
    const int64_t new_hi = min(hi, lo + cnt * step);
    lo = cnt == 0 ? lo : lo + (cnt - 1) * step + 1;
    hi = new_hi;
  }
  return lo;
}

// lse in log2 units; a query with no visible key (lse = -inf) gets +inf so
// that every probability 2^(x - lse) of it is 0.
__device__ __forceinline__ float lse_log2(float lse) {
  return lse == -INFINITY ? INFINITY : lse * LOG2E;
}

// Transposing-read offsets (as the forward's row-major V operand): in each
// 16-lane group gq, lane s reads 8 bytes of row r (4 rows per group) so that
// lane j of the group receives M[r0 + 0..3][col0 + j]; call c covers rows
// {0..3, 8..11} + 4*(gq>>1) of a 16-row step -- the k-slots an MFMA
// accumulator row block hands to its B operand.
__device__ __forceinline__ void tr_offsets(int lane, uint32_t (&off)[2][D / 32]) {
  const int gq = lane >> 4, s = lane & 15;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = ((gq >> 1) << 2) + (s >> 2) + 8 * c;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int lc = db * 4 + ((gq & 1) << 1) + ((s & 3) >> 1);
      off[c][db] = r * ROW_B + ((lc ^ swz(r)) << 4) + ((s & 1) << 3);
    }
  }
}

__device__ __forceinline__ bf16x8 tr_read(const unsigned char *base, const uint32_t (&off)[2][D / 32],
                                           int db, int row0) {
  const bf16x4 v0 =
      __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4 *)(base + off[0][db] + row0 * ROW_B));
  const bf16x4 v1 =
      __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4 *)(base + off[1][db] + row0 * ROW_B));
  return bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
}

// ---------------------------------------------------------------- D = do . o

// HM: instead of delta[r], write the head-major pair delta_t, lse_t
// [b, n_q, s] -- D and the row's lse in log2 units (+inf for a query with no
// visible key) -- the per-row arrays the dK/dV kernel stages, one contiguous
// run per head and query block.
template <typename T, int DD, bool HM>
__global__ __launch_bounds__(256) void bwd_delta_kernel(int64_t rows, const T *__restrict__ dout,
                                                        const float *__restrict__ o,
                                                        float *__restrict__ delta,
                                                        int64_t s, int32_t n_q,
                                                        const float *__restrict__ lse,
                                                        float *__restrict__ lse_t) {
  constexpr int TPR = DD / 8;  // threads per row, 8 elements each
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int t = threadIdx.x % TPR;
  for (int64_t i = tid; i < rows * TPR; i += stride) {
    const int64_t r = i / TPR;
    const float4 *op = reinterpret_cast<const float4 *>(o + r * DD + t * 8);
    const float4 o0 = op[0], o1 = op[1];
    float x[8];
    if constexpr (sizeof(T) == 2) {
      const u32x4 raw = *reinterpret_cast<const u32x4 *>(dout + r * DD + t * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = __uint_as_float(raw[j] << 16);
        x[2 * j + 1] = __uint_as_float(raw[j] & 0xffff0000u);
      }
    } else {
      const float4 *dp = reinterpret_cast<const float4 *>(dout + r * DD + t * 8);
      const float4 a = dp[0], b = dp[1];
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    float sum = x[0] * o0.x + x[1] * o0.y + x[2] * o0.z + x[3] * o0.w +
                x[4] * o1.x + x[5] * o1.y + x[6] * o1.z + x[7] * o1.w;
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) sum += __shfl_xor(sum, m);
    if (t == 0) {
      if constexpr (HM) {
        const int64_t h = r % n_q, bt = r / n_q;
        const int64_t hr = ((bt / s) * n_q + h) * s + bt % s;
        delta[hr] = sum;
        lse_t[hr] = lse_log2(lse[r]);
      } else {
        delta[r] = sum;
      }
    }
  }
}

// ---------------------------------------------------------------- dQ

constexpr int Q_WAVES = 8;
constexpr int Q_THREADS = Q_WAVES * 64;
constexpr int Q_QW = 32;
constexpr int Q_BK = 64;
constexpr int Q_TILE_B = Q_BK * ROW_B;
constexpr int Q_LOADS = Q_TILE_B / (1024 * Q_WAVES);
constexpr int Q_NSTAGE = 4;

// Waits until at most n (0..15) of this wave's vector-memory loads are in
// flight: the n most recent ones (loads complete in order).
__device__ __forceinline__ void wait_loads_upto(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
    case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
    case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
    case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
    case 13: __builtin_amdgcn_s_waitcnt(0x0F7D); break;
    case 14: __builtin_amdgcn_s_waitcnt(0x0F7E); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F7F); break;
  }
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// also wait for every load still in flight); the empty asm statements keep
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_keep_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// DOC: a document mask is given (a.q_lo); without it the mask code compiles away.
template <int HW, bool DOC>
__global__ __launch_bounds__(Q_THREADS, 1) void bwd_dq_kernel(BwdArgs a) {
  // One LDS object per stage and operand (a tile's key positions after its K
  // rows): the compiler then sees that the asynchronous loads into one stage
  // never alias the reads of the others. It tells at most eight apart.
  __shared__ __attribute__((aligned(16))) unsigned char k_lds0[Q_TILE_B + Q_BK * 4],
      k_lds1[Q_TILE_B + Q_BK * 4], k_lds2[Q_TILE_B + Q_BK * 4], k_lds3[Q_TILE_B + Q_BK * 4];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds0[Q_TILE_B], v_lds1[Q_TILE_B],
      v_lds2[Q_TILE_B], v_lds3[Q_TILE_B];
  auto k_stage = [&](auto s) INLINE -> unsigned char * {
    constexpr int v = decltype(s)::value;
    return v == 0 ? k_lds0 : v == 1 ? k_lds1 : v == 2 ? k_lds2 : k_lds3;
  };
  auto v_stage = [&](auto s) INLINE -> unsigned char * {
    constexpr int v = decltype(s)::value;
    return v == 0 ? v_lds0 : v == 1 ? v_lds1 : v == 2 ? v_lds2 : v_lds3;
  };
  auto p_stage = [&](auto s) INLINE -> int32_t * {
    return reinterpret_cast<int32_t *>(k_stage(s) + Q_TILE_B);
  };

  constexpr int TB = Q_WAVES / HW;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int lane = tid & 63;
  const int col = lane & 31;
  const int hi = lane >> 5;

  const int g = a.n_q / a.n_kv;
  const int hgroups = g / HW;
  const int64_t tok_per_wg = TB * Q_QW;
  const int64_t ntb = (a.s_q + tok_per_wg - 1) / tok_per_wg;
  const int64_t inner = static_cast<int64_t>(a.b) * a.n_kv * hgroups;
  const int64_t id = blockIdx.x;
  const int64_t tb = ntb - 1 - id / inner;  // latest (heaviest) token block first
  int64_t rem = id % inner;
  const int kvh = static_cast<int>(rem % a.n_kv);
  rem /= a.n_kv;
  const int hgi = static_cast<int>(rem % hgroups);
  const int bi = static_cast<int>(rem / hgroups);

  const int64_t wg_tok0 = tb * tok_per_wg;
  const int64_t wg_tok_last = min(wg_tok0 + tok_per_wg, a.s_q) - 1;
  const int h = kvh * g + hgi * HW + (wave % HW);
  const int64_t w_tok0 = wg_tok0 + (wave / HW) * Q_QW;
  const int64_t w_tok_last = min(w_tok0 + Q_QW, a.s_q) - 1;
  const bool wave_has_rows = w_tok0 < a.s_q;
  const int64_t tok = w_tok0 + col;
  const bool tok_ok = tok < a.s_q;

  // Keys up to the workgroup's last position; with a document mask, from the
  // tile holding the first query's document start.
  int64_t nkeys = a.s_kv;
  int64_t kbeg = 0;
  int32_t w_qmin = INT_MAX - 1, w_qmax = INT_MAX - 1;
  int32_t w_lomax = INT_MIN;
  if (a.causal) {
    nkeys = count_le(a.kv_pos, a.s_kv, a.q_pos[wg_tok_last]);
    if (DOC) kbeg = count_lt(a.kv_pos, a.s_kv, a.q_lo[wg_tok0]) / Q_BK * Q_BK;
    if (wave_has_rows) {
      w_qmin = a.q_pos[w_tok0];
      w_qmax = a.q_pos[w_tok_last];
      if (DOC) w_lomax = a.q_lo[w_tok_last];
    }
  }
  // (The searches read memory, so the compiler cannot see that their results
  // agree across lanes: say so, and the loop's decisions stay scalar.)
  nkeys = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(nkeys));
  kbeg = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(kbeg));
  const int nt = nkeys > kbeg ? static_cast<int>((nkeys - kbeg + Q_BK - 1) / Q_BK) : 0;
  // The wave's tiles: those whose first key is not after its last query.
  int w_nt = wave_has_rows ? nt : 0;
  if (a.causal && w_nt > 0) {
    const int64_t c = wave_count<true>(a.kv_pos + kbeg, nkeys - kbeg, w_qmax, lane);
    w_nt = min(w_nt, static_cast<int>((c + Q_BK - 1) / Q_BK));
  }

  // This lane's query and upstream gradient: the B operands of S^T and dP^T.
  const uint16_t *qg = static_cast<const uint16_t *>(a.q);
  const uint16_t *dg = static_cast<const uint16_t *>(a.dout);
  bf16x8 qreg[D / 16], dreg[D / 16];
  const int64_t row = (bi * a.s_q + (tok_ok ? tok : 0)) * a.n_q + h;
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds) {
    const u32x4 rq = tok_ok ? *reinterpret_cast<const u32x4 *>(qg + row * D + ds * 16 + hi * 8)
                            : u32x4{0, 0, 0, 0};
    const u32x4 rd = tok_ok ? *reinterpret_cast<const u32x4 *>(dg + row * D + ds * 16 + hi * 8)
                            : u32x4{0, 0, 0, 0};
    qreg[ds] = __builtin_bit_cast(bf16x8, rq);
    dreg[ds] = __builtin_bit_cast(bf16x8, rd);
  }
  const int32_t qpos = !a.causal ? INT_MAX - 1 : (tok_ok ? a.q_pos[tok] : INT_MIN);
  const int32_t qlo = DOC && tok_ok ? a.q_lo[tok] : INT_MIN;  // document start
  const int64_t hrow = (static_cast<int64_t>(bi) * a.n_q + h) * a.s_q + tok;
  const float lse2 = !tok_ok ? INFINITY : a.hm ? a.lse[hrow] : lse_log2(a.lse[row]);
  const float dlt = !tok_ok ? 0.f : a.hm ? a.delta[hrow] : a.delta[row];
  const float sl2 = a.scale * LOG2E;

  // Waves w and w + 4 share a SIMD and run the tile phases in opposite orders.
  const bool grp_b = wave >= Q_WAVES / 2;

  // K / V row operand of k-step ds: the swizzle is an XOR of the chunk index,
  // so one offset register serves every k-step (kept live by the pin in the
  // loop, which stops the compiler from hoisting eight offsets).
  uint32_t koff0 = col * ROW_B + ((hi ^ swz(col & 15)) << 4);
  auto koff = [&](int ds) INLINE -> uint32_t { return koff0 ^ (static_cast<uint32_t>(ds) << 5); };
  uint32_t toff[2][D / 32];
  tr_offsets(lane, toff);

  const unsigned char *kg = static_cast<const unsigned char *>(a.k);
  const unsigned char *vg = static_cast<const unsigned char *>(a.v);
  const int64_t kv_row_bytes = static_cast<int64_t>(a.n_kv) * D * 2;
  const int64_t kv_base = (static_cast<int64_t>(bi) * a.s_kv * a.n_kv + kvh) * D * 2;
  uint32_t goff[Q_LOADS];
#pragma unroll
  for (int i = 0; i < Q_LOADS; ++i) {
    const int r = 4 * (wave + Q_WAVES * i) + (lane >> 4);
    goff[i] = static_cast<uint32_t>(r * kv_row_bytes + (((lane & 15) ^ swz(r & 15)) << 4));
  }
  // K, V rows (and key positions, by wave 0 when causal) of tile t into
  // stage `stage`. Issued for every step, past the range too (the buffer
  // descriptors' bounds return zeros there), so every wave issues the same
  // loads per step and the waits below count them exactly.
  auto issue_tile = [&](int t, auto stage) INLINE {
    const int64_t key0 = kbeg + static_cast<int64_t>(t) * Q_BK;
    const int64_t left = a.s_kv - key0;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + kv_base + key0 * kv_row_bytes,
                                                (left - 1) * kv_row_bytes + D * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + kv_base + key0 * kv_row_bytes,
                                                (left - 1) * kv_row_bytes + D * 2);
#pragma unroll
    for (int i = 0; i < Q_LOADS; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (LDS_AS void *)(k_stage(stage) + 4 * (wave + Q_WAVES * i) * ROW_B), 16, goff[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (LDS_AS void *)(v_stage(stage) + 4 * (wave + Q_WAVES * i) * ROW_B), 16, goff[i], 0, 0, 0);
    }
    if (a.causal && wave == 0) {
      const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.kv_pos + key0, left * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (LDS_AS void *)p_stage(stage), 4, lane * 4,
                                               0, 0, 0);
    }
  };
  const int n_step = 2 * Q_LOADS + (a.causal && wave == 0 ? 1 : 0);  // loads per issue_tile

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  // S^T and dP^T of the tile whose dS comes next; dS^T (bf16 B operand per
  // k-step) of the tile whose dQ products come next.
  f32x16 s[2], dp[2];
  bf16x8 dsb[4];
  bool done = !wave_has_rows || w_nt == 0;

  // Item m of S^T, dP^T (32 MFMAs): k-step m/4, key block (m/2)%2; S^T from
  // the K rows when m is even, dP^T from the V rows when odd.
  auto rd_m1 = [&](const unsigned char *kb, const unsigned char *vb, int m) INLINE -> bf16x8 {
    return *reinterpret_cast<const bf16x8 *>(((m & 1) ? vb : kb) + koff(m >> 2) +
                                             ((m >> 1) & 1) * 32 * ROW_B);
  };
  auto mfma_m1 = [&](int m, const bf16x8 &o) INLINE {
    const int ds = m >> 2, j = (m >> 1) & 1;
    if (m & 1)
      dp[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, dreg[ds], ds == 0 ? f32x16{} : dp[j], 0, 0, 0);
    else
      s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, qreg[ds], ds == 0 ? f32x16{} : s[j], 0, 0, 0);
  };
  constexpr int DIST = 4;
  // S^T and dP^T of the tile in stage `st` alone (before the loop).
  auto m1_only = [&](auto st) INLINE {
    const unsigned char *kb = k_stage(st);
    const unsigned char *vb = v_stage(st);
    bf16x8 op[DIST + 1];
#pragma unroll
    for (int i = 0; i < DIST; ++i) op[i] = rd_m1(kb, vb, i);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i + DIST < 32) op[(i + DIST) % (DIST + 1)] = rd_m1(kb, vb, i + DIST);
      mfma_m1(i, op[i % (DIST + 1)]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Matrix phase: S^T, dP^T of the next tile (stage `sn`) interleaved with
  // dQ^T += K^T dS^T of the current one (stage `sc`, K^T by the transposing
  // read): two of the former, then one of the latter. Operands are read DIST
  // items ahead behind scheduling fences.
  auto xphase = [&](auto sn, auto sc) INLINE {
    const unsigned char *kn = k_stage(sn);
    const unsigned char *vn = v_stage(sn);
    const unsigned char *kc = k_stage(sc);
    auto rd = [&](int i) INLINE -> bf16x8 {
      if (i % 3 < 2) return rd_m1(kn, vn, 2 * (i / 3) + i % 3);
      const int c = i / 3;
      return tr_read(kc, toff, c & 3, (c >> 2) * 16);
    };
    bf16x8 op[DIST + 1];
#pragma unroll
    for (int i = 0; i < DIST; ++i) op[i] = rd(i);
#pragma unroll
    for (int i = 0; i < 48; ++i) {
      if (i + DIST < 48) op[(i + DIST) % (DIST + 1)] = rd(i + DIST);
      const bf16x8 o = op[i % (DIST + 1)];
      if (i % 3 < 2) {
        mfma_m1(2 * (i / 3) + i % 3, o);
      } else {
        const int c = i / 3, ks = c >> 2, db = c & 3;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, dsb[ks], acc[db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Vector phase for tile t (scores in s, dp; positions in stage `st`): the
  // element mask where needed, then dS^T = P^T (dP^T - D) into dsb: k-step ks
  // holds accumulator elements (ks%2)*8 .. +7 of key block ks/2.
  auto yphase = [&](int t, auto st) INLINE {
    // Element e4*4 + j of key block kb holds key kb*32 + e4*8 + hi*4 + j.
    const int64_t key0 = kbeg + static_cast<int64_t>(t) * Q_BK;
    const bool ragged = key0 + Q_BK > a.s_kv;
    const int32_t *pp = p_stage(st);
    if (ragged || (a.causal && pp[Q_BK - 1] > w_qmin) || (DOC && pp[0] < w_lomax)) {
      const int lim = ragged ? static_cast<int>(a.s_kv - key0) : Q_BK;
      const int32_t qp = a.causal ? qpos : INT_MAX;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int kk = j * 32 + e4 * 8 + hi * 4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool out = (kk + i >= lim) | (pp[kk + i] > qp) | (pp[kk + i] < qlo);
            s[j][e4 * 4 + i] = out ? -INFINITY : s[j][e4 * 4 + i];
          }
        }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = ks >> 1, el = (ks & 1) * 8 + u;
        const float p = exp2_fast(fmaf(s[j][el], sl2, -lse2));
        dsb[ks][u] = static_cast<__bf16>(p * (dp[j][el] - dlt));
      }
      asm volatile("" : "+v"(dsb[ks]));  // one k-step of fp32 values live at a time
    }
  };

  using St0 = std::integral_constant<int, 0>;
  using St1 = std::integral_constant<int, 1>;
  using St2 = std::integral_constant<int, 2>;
  using St3 = std::integral_constant<int, 3>;
  // ---- prologue: tiles 0..2 in flight, tile 0's scores (and, for the first
  // group, its dS) ----
  issue_tile(0, St0{});
  issue_tile(1, St1{});
  issue_tile(2, St2{});
  wait_loads_upto(2 * n_step);  // tile 0 has landed (this wave's share)
  barrier_keep_loads();         // ... and everyone's
  if (!done) {
    m1_only(St0{});
    if (!grp_b) yphase(0, St0{});
  }
  // ---- main loop: step t = 0 .. nt-1, tile t in stage t % 4 ----
  // Step t issues tile t + 3 into the stage tile t - 1 left and needs tiles t
  // (dQ products) and t + 1 (scores): its loads have had two steps to land.
  // The matrix phase runs the dQ products of tile t with the scores of tile
  // t + 1; the vector phase forms dS of the tile whose scores are at hand. The
  // first group runs matrix then vector (tile t + 1), the second vector (tile
  // t) then matrix, so one wave's exponentials overlap the other's MFMAs.
  auto step = [&](auto stage_c, int t) INLINE {
    constexpr int S = decltype(stage_c)::value;
    using SC = std::integral_constant<int, S>;
    using SN = std::integral_constant<int, (S + 1) % Q_NSTAGE>;
    using SP = std::integral_constant<int, (S + Q_NSTAGE - 1) % Q_NSTAGE>;
    wait_loads_upto(n_step);  // tile t + 1 has landed (tile t + 2 may be in flight)
    barrier_keep_loads();     // everyone's too; every wave is done with tile t - 1
    asm volatile("" : "+v"(koff0));  // pin: see koff
    issue_tile(t + 3, SP{});
    if (!done) {
      if (grp_b) yphase(t, SC{});
      // After the wave's last tile the scores computed here are of a tile past
      // its range and are dropped.
      __builtin_amdgcn_s_setprio(1);
      xphase(SN{}, SC{});
      __builtin_amdgcn_s_setprio(0);
      if (t + 1 < w_nt) {
        if (!grp_b) yphase(t + 1, SN{});
      } else {
        done = true;
      }
    }
  };
  // The body always runs all four steps (steps past nt only wait, synchronise
  // and issue loads past the range).
  for (int t = 0; t < nt; t += Q_NSTAGE) {
    step(St0{}, t);
    step(St1{}, t + 1);
    step(St2{}, t + 2);
    step(St3{}, t + 3);
  }
  wait_loads_upto(0);  // the loads past the range have landed before the wave ends

  // With a document mask many waves see no key at all: they skip the dq
  // update (adding zeros).
  if (!tok_ok || (DOC && w_nt == 0)) return;
  // Accumulator element e4*4 + j of block db holds d = db*32 + e4*8 + hi*4 + j.
  float *drow = a.dq + row * D + hi * 4;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      float4 *dst = reinterpret_cast<float4 *>(drow + db * 32 + e4 * 8);
      float4 r = *dst;
      r.x += a.scale * acc[db][e4 * 4 + 0];
      r.y += a.scale * acc[db][e4 * 4 + 1];
      r.z += a.scale * acc[db][e4 * 4 + 2];
      r.w += a.scale * acc[db][e4 * 4 + 3];
      *dst = r;
    }
}

// ---------------------------------------------------------------- dK, dV

constexpr int KV_GROUPS = 4;                 // key groups of 32 keys, one per SIMD
constexpr int KV_WAVES = 2 * KV_GROUPS;      // a producer and a consumer wave per group
constexpr int KV_THREADS = KV_WAVES * 64;
constexpr int KV_KW = 32;                    // keys per group
constexpr int KV_KT = KV_GROUPS * KV_KW;     // keys per workgroup
constexpr int KV_QB = 64;                    // queries per staged block (two 32-row sub-blocks)
constexpr int KV_SUB = 32;
constexpr int KV_TILE_B = KV_QB * ROW_B;     // 16 KiB (q or dout rows)
constexpr int KV_LOADS = KV_TILE_B / (1024 * KV_GROUPS);  // per consumer wave
constexpr int KV_NSTAGE = 3;
// LDS: KV_NSTAGE stages of one query block -- q rows, dout rows and, per row,
// the lse (log2 units), delta, position and document start -- then the P / dS
// hand-over buffers, two per group (P then dS, each two 1 KiB k-steps in the
// lane order of the B operand).
constexpr int ST_Q = 0;
constexpr int ST_D = ST_Q + KV_TILE_B;
constexpr int ST_L = ST_D + KV_TILE_B;
constexpr int ST_E = ST_L + KV_QB * 4;
constexpr int ST_P = ST_E + KV_QB * 4;
constexpr int ST_O = ST_P + KV_QB * 4;
constexpr int STAGE_B = ST_O + KV_QB * 4;
constexpr int XG_B = 4 * 1024;
constexpr int XCH = KV_NSTAGE * STAGE_B;
constexpr int KV_LDS_B = XCH + KV_GROUPS * 2 * XG_B;
static_assert(KV_LOADS * 1024 * KV_GROUPS == KV_TILE_B, "block split over the consumer waves");
static_assert(STAGE_B % 256 == 0, "stage bases leave the swizzled address bits alone");
static_assert(KV_LDS_B <= 160 * 1024, "LDS of one workgroup");

template <bool DOC>
__global__ __launch_bounds__(KV_THREADS, 1) void bwd_dkdv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[KV_LDS_B];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int lane = tid & 63;
  const int col = lane & 31;
  const int hi = lane >> 5;
  const int grp = wave & (KV_GROUPS - 1);
  const bool producer = wave < KV_GROUPS;

  // ---- workgroup -> (batch, kv head, key tile); earliest keys (most queries) first ----
  const int64_t inner = static_cast<int64_t>(a.b) * a.n_kv;
  const int64_t kt = blockIdx.x / inner;
  const int kvh = static_cast<int>(blockIdx.x % a.n_kv);
  const int bi = static_cast<int>((blockIdx.x / a.n_kv) % a.b);
  const int g = a.n_q / a.n_kv;

  const int64_t wg_key0 = kt * KV_KT;
  const int64_t w_key0 = wg_key0 + grp * KV_KW;
  const int64_t key = w_key0 + col;
  const bool key_ok = key < a.s_kv;
  const bool grp_has_keys = w_key0 < a.s_kv;
  const int32_t kpos = !key_ok ? INT_MAX : (a.causal ? a.kv_pos[key] : INT_MIN);
  // The group's first and last key positions (causal skips and masks).
  int32_t w_kmin = INT_MIN, w_kmax = INT_MIN;
  if (a.causal && grp_has_keys) {
    w_kmin = a.kv_pos[w_key0];
    w_kmax = a.kv_pos[min(w_key0 + KV_KW, a.s_kv) - 1];
  }

  // ---- query range that can see any key of the workgroup ----
  // Causal: from the first query at or after its first key. With a document
  // mask, up to the last query whose document starts at or before its last
  // key (document starts are non-decreasing). (The searches read memory, so
  // the compiler cannot see that their results agree across lanes: say so.)
  int64_t q_first = 0, q_end = a.s_q;
  if (a.causal) q_first = count_lt(a.q_pos, a.s_q, a.kv_pos[wg_key0]);
  if (DOC) q_end = count_le(a.q_lo, a.s_q, a.kv_pos[min(wg_key0 + KV_KT, a.s_kv) - 1]);
  const int64_t qb0 = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(q_first / KV_QB));
  const int64_t nqb = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((q_end + KV_QB - 1) / KV_QB));
  const int64_t n_blk = nqb > qb0 ? nqb - qb0 : 0;   // query blocks per head
  const int n_it = static_cast<int>(n_blk * g);
  const int n_sub = 2 * n_it;
  const int64_t qb_last = qb0 + n_blk - 1;

  // ---- the group's sub-blocks ----
  // Sub-block n = 2 it + h holds rows 32h .. 32h+31 of the block of iteration
  // it. A sub-block whose rows are all before the group's first key (causal),
  // or all start their document after its last key, or lie past the
  // sequence, sees none of the group's keys. In row terms the useful first
  // rows r (multiples of 32) satisfy c_vis - 31 <= r < r_end; they form one
  // range of blocks in the walk, whose first and last blocks may have one
  // useless half per head (those run fully masked and add nothing). n_lo ..
  // n_hi is that range in the walk. c_kmax / c_dmin decide which sub-blocks
  // need the element mask.
  int64_t c_vis = 0, c_kmax = 0, r_end = a.s_q, c_dmin = a.s_q;
  if (a.causal && grp_has_keys) {
    c_vis = wave_count<false>(a.q_pos, a.s_q, w_kmin, lane);
    c_kmax = wave_count<false>(a.q_pos, a.s_q, w_kmax, lane);
  }
  if (DOC && grp_has_keys) {
    r_end = min(r_end, wave_count<true>(a.q_lo, a.s_q, w_kmax, lane));
    c_dmin = wave_count<true>(a.q_lo, a.s_q, w_kmin, lane);
  }
  int64_t R_lo = (c_vis - 31 + 31) / 32;  // ceil((c_vis - 31) / 32) for c_vis >= 0
  if (c_vis < 31) R_lo = 0;
  int64_t R_hi = (r_end + 31) / 32 - 1;   // last useful 32-row unit
  R_lo = max(R_lo, 2 * qb0);
  R_hi = min(R_hi, 2 * qb_last + 1);
  int n_lo = 0, n_hi = 0;
  if (grp_has_keys && n_blk > 0 && R_lo <= R_hi) {
    const int64_t j_first = qb_last - R_hi / 2;          // walk block of the latest unit
    const int64_t h_min = max<int64_t>(0, R_lo - 2 * (qb_last - j_first));
    n_lo = static_cast<int>(2 * (j_first * g) + h_min);
    const int64_t j_last = qb_last - R_lo / 2;           // walk block of the earliest unit
    const int64_t h_max = min<int64_t>(1, R_hi - 2 * (qb_last - j_last));
    n_hi = static_cast<int>(2 * (j_last * g + g - 1) + h_max + 1);
  }
  n_lo = __builtin_amdgcn_readfirstlane(n_lo);
  n_hi = __builtin_amdgcn_readfirstlane(n_hi);
  const bool any = n_lo < n_hi;
  const bool w_ragged = w_key0 + KV_KW > a.s_kv;   // some key of the group past the block

  // ---- staging of one query block (iteration it -> head, block) ----
  // Iteration it -> (query block, head): blocks from the last one down, the g
  // heads of a block back to back. Every workgroup of a kv head then walks the
  // same blocks in the same order (they differ only in where they stop), so
  // workgroups resident together read each block while it is in L2. Block it
  // lives in stage it % 3.
  const unsigned char *qbytes = static_cast<const unsigned char *>(a.q);
  const unsigned char *dbytes = static_cast<const unsigned char *>(a.dout);
  const int64_t q_row_bytes = static_cast<int64_t>(a.n_q) * D * 2;
  uint32_t goff[KV_LOADS];
#pragma unroll
  for (int i = 0; i < KV_LOADS; ++i) {
    const int r = 4 * (grp + KV_GROUPS * i) + (lane >> 4);
    goff[i] = static_cast<uint32_t>(r * q_row_bytes + (((lane & 15) ^ swz(r & 15)) << 4));
  }
  auto stage_b = [&](int it) INLINE -> uint32_t {
    return static_cast<uint32_t>(it % KV_NSTAGE) * STAGE_B;
  };
  auto blk_of = [&](int it, int64_t *q0, int *h) INLINE {
    const int64_t j = it / g;
    *q0 = (qb0 + n_blk - 1 - j) * KV_QB;
    *h = kvh * g + static_cast<int>(it - j * g);
  };
  auto blk_q0 = [&](int it) INLINE -> int64_t { return (qb_last - it / g) * KV_QB; };
  // A block's loads: each consumer wave issues KV_LOADS 16-byte loads each
  // of its q and dout rows (the consumers wait at the barrier for the
  // producers anyway); producer waves 0-3 stage one per-row array each (lse,
  // delta, positions when causal, document starts with a document mask).
  auto issue_blk = [&](int it) INLINE {
    int64_t q0;
    int h;
    blk_of(it, &q0, &h);
    const int64_t left = a.s_q - q0;
    const int64_t rbase = (static_cast<int64_t>(bi) * a.s_q + q0) * a.n_q + h;
    const uint32_t sb = stage_b(it);
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(qbytes + rbase * D * 2, (left - 1) * q_row_bytes + D * 2);
    const __amdgpu_buffer_rsrc_t rd =
        make_rsrc(dbytes + rbase * D * 2, (left - 1) * q_row_bytes + D * 2);
    if (!producer) {
#pragma unroll
      for (int i = 0; i < KV_LOADS; ++i) {
        const uint32_t row_b = sb + 4 * (grp + KV_GROUPS * i) * ROW_B;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (LDS_AS void *)(smem + row_b + ST_Q), 16,
                                                 goff[i], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (LDS_AS void *)(smem + row_b + ST_D), 16,
                                                 goff[i], 0, 0, 0);
      }
      return;
    }
    // lse and delta of rows q0 + lane of head h: head-major runs (hm), else
    // rows with stride n_q floats; positions and document starts q0 + lane.
    const int64_t hbase = (static_cast<int64_t>(bi) * a.n_q + h) * a.s_q + q0;
    if (wave < 2) {
      const float *src = wave == 0 ? a.lse : a.delta;
      const __amdgpu_buffer_rsrc_t rr =
          a.hm ? make_rsrc(src + hbase, left * 4) : make_rsrc(src + rbase, ((left - 1) * a.n_q + 1) * 4);
      const uint32_t lo = a.hm ? lane * 4 : lane * a.n_q * 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (LDS_AS void *)(smem + sb + (wave == 0 ? ST_L : ST_E)),
                                               4, lo, 0, 0, 0);
    } else if (wave == 2 && a.causal) {
      const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.q_pos + q0, left * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (LDS_AS void *)(smem + sb + ST_P), 4, lane * 4,
                                               0, 0, 0);
    } else if (DOC && wave == 3) {
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.q_lo + q0, left * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ro, (LDS_AS void *)(smem + sb + ST_O), 4, lane * 4,
                                               0, 0, 0);
    }
  };
  // Unless the lse comes in log2 units already (hm), wave 0 converts each
  // block's lse in place (-inf, a query with no key, to +inf so that its
  // probabilities are 0) in the iteration before its first B.
  auto prescale_lse = [&](int it) INLINE {
    if (wave == 0 && !a.hm) {
      float *l = reinterpret_cast<float *>(smem + stage_b(it) + ST_L);
      l[lane] = lse_log2(l[lane]);
    }
  };
  // Iteration n (from -1 to n_sub): the producer runs A on sub-block n+1 and
  // B on n, the consumer C on n-1. Block j+3 goes into the stage of block j,
  // whose last C ran in iteration 2j+2: the producers' per-row loads are
  // issued at the start of iteration 2j+3, the consumers' q / dout rows at its
  // end (into registers, written to the stage at the end of 2j+4), and all
  // have landed by the barrier that ends iteration 2j+4 (every even iteration
  // waits for the loads in flight); wave 0 converts its lse in iteration
  // 2j+5, before B of its first sub-block in 2j+6. The barrier that ends each
  // iteration publishes the P and dS the producers wrote for the consumers'
  // next iteration.
  auto begin_iter = [&](int n) INLINE {
    if (producer && (n & 1) && n >= 3 && (n + 3) / 2 < n_it) issue_blk((n + 3) / 2);
    if ((n & 1) && (n + 1) / 2 < n_it) prescale_lse((n + 1) / 2);
  };
  auto end_iter = [&](int n) INLINE {
    if ((n & 1) == 0) wait_own_loads();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): LDS writes and reads done
    __builtin_amdgcn_s_barrier();
  };

  if (n_it > 0) issue_blk(0);
  if (n_it > 1) issue_blk(1);
  if (n_it > 2) issue_blk(2);
  wait_own_loads();
  __syncthreads();

  // Q / dO rows by ds_read_b128 (row = query col), chunk 2*ds + hi: the
  // swizzle is an XOR of the chunk index, so k-step ds reads at qoff0 with
  // bits 5..7 XORed by ds. Likewise the transposing reads of d block db are at
  // toff0 with bits 6..7 XORed by db. Stage bases and row offsets are
  // multiples of 256 and leave those bits alone.
  const uint32_t qoff0 = col * ROW_B + (((hi ^ swz(col & 15))) << 4);
  uint32_t toff0[2];
  {
    uint32_t toff[2][D / 32];
    tr_offsets(lane, toff);
    toff0[0] = toff[0][0];
    toff0[1] = toff[1][0];
  }
  // This group's hand-over buffers: parity x at xch + x * XG_B; P of k-step
  // ks at + ks * 1 KiB, dS at + 2 KiB + ks * 1 KiB, lane l at + 16 l.
  const uint32_t xch = XCH + grp * 2 * XG_B + lane * 16;
  const float sl2 = a.scale * LOG2E;
  constexpr int DIST = 4;  // operand reads ahead of their MFMA

  if (producer) {
    // ---- producer: A (S = Q K^T, dP = dO V^T) and B (P, dS) ----
    // This lane's key: the B operands of S = Q K^T and dP = dO V^T.
    const uint16_t *kg = static_cast<const uint16_t *>(a.k);
    const uint16_t *vg = static_cast<const uint16_t *>(a.v);
    bf16x8 kreg[D / 16], vreg[D / 16];
    const int64_t krow = (static_cast<int64_t>(bi) * a.s_kv + (key_ok ? key : 0)) * a.n_kv + kvh;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      const u32x4 rk = key_ok ? *reinterpret_cast<const u32x4 *>(kg + krow * D + ds * 16 + hi * 8)
                              : u32x4{0, 0, 0, 0};
      const u32x4 rv = key_ok ? *reinterpret_cast<const u32x4 *>(vg + krow * D + ds * 16 + hi * 8)
                              : u32x4{0, 0, 0, 0};
      kreg[ds] = __builtin_bit_cast(bf16x8, rk);
      vreg[ds] = __builtin_bit_cast(bf16x8, rv);
    }
    // S accumulator: lane holds key `col`; element e holds sub-block row
    // (e/4)*8 + hi*4 + e%4. Scores are double-buffered by sub-block parity.
    f32x16 s[2], dp[2];
    bf16x8 pb[2], dsb[2];   // P and dS of the sub-block in B, per k-step
    float4 l4[4], d4[4];    // its rows' lse (log2 units) and D
    // Operand of A item ai (k-step ai/2; S from the Q rows when ai is even, dP
    // from the dO rows when odd); qa = stage base + rows + qoff0.
    auto rd_a = [&](uint32_t qa, int ai) INLINE -> bf16x8 {
      const uint32_t off = (qa ^ (static_cast<uint32_t>(ai >> 1) << 5)) + ((ai & 1) ? ST_D : ST_Q);
      return *reinterpret_cast<const bf16x8 *>(smem + off);
    };
    auto mfma_a = [&](int par, int ai, const bf16x8 &o) INLINE {
      const int ds = ai >> 1;
      if (ai & 1)
        dp[par] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, vreg[ds], ds == 0 ? f32x16{} : dp[par], 0, 0, 0);
      else
        s[par] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, kreg[ds], ds == 0 ? f32x16{} : s[par], 0, 0, 0);
    };
    auto read_ld = [&](uint32_t sb, int rb) INLINE {
      const float *ll = reinterpret_cast<const float *>(smem + sb + ST_L) + rb;
      const float *ee = reinterpret_cast<const float *>(smem + sb + ST_E) + rb;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        l4[e4] = *reinterpret_cast<const float4 *>(ll + e4 * 8 + hi * 4);
        d4[e4] = *reinterpret_cast<const float4 *>(ee + e4 * 8 + hi * 4);
      }
    };
    // Two elements (el, el+1) of B: p = 2^(S scale log2 e - lse'),
    // ds = p (dP - D), converted to bf16 together.
    auto b_pair = [&](int par, int el) INLINE {
#pragma unroll
      for (int j = el; j < el + 2; ++j) {
        const float p = exp2_fast(fmaf(s[par][j], sl2, -l4[j >> 2][j & 3]));
        pb[j >> 3][j & 7] = static_cast<__bf16>(p);
        dsb[j >> 3][j & 7] = static_cast<__bf16>(p * (dp[par][j] - d4[j >> 2][j & 3]));
      }
      // Keep the pair here, between the MFMAs: otherwise the compiler sinks
      // all of B past the stream, where nothing overlaps it.
      asm volatile("" : "+v"(pb[el >> 3]), "+v"(dsb[el >> 3]));
    };
    auto write_x = [&](int par) INLINE {
      unsigned char *x = smem + xch + par * XG_B;
      *reinterpret_cast<bf16x8 *>(x) = pb[0];
      *reinterpret_cast<bf16x8 *>(x + 1024) = pb[1];
      *reinterpret_cast<bf16x8 *>(x + 2048) = dsb[0];
      *reinterpret_cast<bf16x8 *>(x + 3072) = dsb[1];
    };
    // A of one sub-block (16 MFMAs), with B of another interleaved (a pair
    // after every odd MFMA) when WITH_B.
    auto a_stream = [&](auto with_b, uint32_t qa, int pa, int pbp) INLINE {
      constexpr bool WB = decltype(with_b)::value;
      bf16x8 op[DIST + 1];
#pragma unroll
      for (int i = 0; i < DIST; ++i) op[i] = rd_a(qa, i);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + DIST < 16) op[(i + DIST) % (DIST + 1)] = rd_a(qa, i + DIST);
        mfma_a(pa, i, op[i % (DIST + 1)]);
        if (WB && (i & 1)) b_pair(pbp, i - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto b_only = [&](int pbp) INLINE {
#pragma unroll
      for (int el = 0; el < 16; el += 2) b_pair(pbp, el);
    };
    // Element mask of A's scores (sub-block at rows rb of the stage at sb,
    // block rows from q0): rows past the sequence, keys past the block, a
    // query before the key (causal), or a key before the query's document.
    auto mask_a = [&](uint32_t sb, int rb, int par, int64_t q0) INLINE {
      const int qlim = static_cast<int>(min<int64_t>(a.s_q - q0 - rb, KV_SUB));
      const int64_t row0 = q0 + rb;
      const bool need = qlim < KV_SUB || w_ragged || (a.causal && row0 < c_kmax) ||
                        (DOC && row0 + qlim - 1 >= c_dmin);
      if (need) {
        const int32_t *pp = reinterpret_cast<const int32_t *>(smem + sb + ST_P) + rb;
        const int32_t *lp = reinterpret_cast<const int32_t *>(smem + sb + ST_O) + rb;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int r0 = e4 * 8 + hi * 4;
          int4 p4 = int4{INT_MAX, INT_MAX, INT_MAX, INT_MAX};
          int4 o4 = int4{INT_MIN, INT_MIN, INT_MIN, INT_MIN};
          if (a.causal) p4 = *reinterpret_cast<const int4 *>(pp + r0);
          if (DOC) o4 = *reinterpret_cast<const int4 *>(lp + r0);
          const int32_t qp[4] = {p4.x, p4.y, p4.z, p4.w};
          const int32_t ql[4] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool out = (r0 + j >= qlim) | (kpos > qp[j]) | (kpos < ql[j]) | !key_ok;
            s[par][e4 * 4 + j] = out ? -INFINITY : s[par][e4 * 4 + j];
          }
        }
      }
    };
    // Iteration n with its parity PAR compile-time: B on sub-block n (scores
    // s[PAR]), A on n+1 (into s[1 - PAR]).
    auto step = [&](auto par_c, int n) INLINE {
      constexpr int PAR = decltype(par_c)::value;
      begin_iter(n);
      const bool do_a = n + 1 >= n_lo && n + 1 < n_hi;
      const bool do_b = n >= n_lo && n < n_hi;
      const int ja = (n + 1) >> 1, jb = n >> 1;
      const uint32_t sba = stage_b(ja), sbb = stage_b(jb);
      const uint32_t qa = sba + 32 * (1 - PAR) * ROW_B + qoff0;
      if (do_b) read_ld(sbb, 32 * PAR);
      if (do_a && do_b) {
        a_stream(std::true_type{}, qa, 1 - PAR, PAR);
      } else if (do_a) {
        a_stream(std::false_type{}, qa, 1 - PAR, PAR);
      } else if (do_b) {
        b_only(PAR);
      }
      if (do_b) write_x(PAR);
      if (do_a) mask_a(sba, 32 * (1 - PAR), 1 - PAR, blk_q0(ja));
      end_iter(n);
    };
    for (int n = -1; n <= n_sub; n += 2) {
      step(std::integral_constant<int, 1>{}, n);
      step(std::integral_constant<int, 0>{}, n + 1);
    }
    return;
  }

  // ---- consumer: C (dV^T += dO^T P, dK^T += Q^T dS) ----
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  bf16x8 pc[2], dsc[2];  // P and dS of the sub-block in C, per k-step
  // The q and dout rows of block j+3, loaded into registers at the end of
  // iteration 2j+3 (after its C, where the consumer would wait at the
  // barrier) and written to its stage at the end of 2j+4.
  u32x4 stg[2 * KV_LOADS];
  auto stg_load = [&](int it) INLINE {
    int64_t q0;
    int h;
    blk_of(it, &q0, &h);
    const int64_t left = a.s_q - q0;
    const int64_t rbase = (static_cast<int64_t>(bi) * a.s_q + q0) * a.n_q + h;
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(qbytes + rbase * D * 2, (left - 1) * q_row_bytes + D * 2);
    const __amdgpu_buffer_rsrc_t rd =
        make_rsrc(dbytes + rbase * D * 2, (left - 1) * q_row_bytes + D * 2);
#pragma unroll
    for (int i = 0; i < KV_LOADS; ++i) {
      stg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, goff[i], 0, 0));
      stg[KV_LOADS + i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rd, goff[i], 0, 0));
    }
  };
  auto stg_write = [&](int it) INLINE {
    const uint32_t sb = stage_b(it);
#pragma unroll
    for (int i = 0; i < KV_LOADS; ++i) {
      const uint32_t row_b = sb + 4 * (grp + KV_GROUPS * i) * ROW_B + lane * 16;
      *reinterpret_cast<u32x4 *>(smem + row_b + ST_Q) = stg[i];
      *reinterpret_cast<u32x4 *>(smem + row_b + ST_D) = stg[KV_LOADS + i];
    }
  };
  // Operand of C item ci (16-row step ci/8, d block (ci/2)%4; dV from dO^T
  // when ci is even, dK from Q^T when odd), by the transposing read; t0 / t1 =
  // stage base + rows + toff0[0 / 1].
  auto rd_c = [&](uint32_t t0, uint32_t t1, int ci) INLINE -> bf16x8 {
    const uint32_t x = static_cast<uint32_t>((ci >> 1) & 3) << 6;
    const uint32_t off = ((ci & 1) ? ST_Q : ST_D) + (ci >> 3) * 16 * ROW_B;
    const bf16x4 v0 =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4 *)(smem + (t0 ^ x) + off));
    const bf16x4 v1 =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4 *)(smem + (t1 ^ x) + off));
    return bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
  };
  auto step = [&](auto par_c, int n) INLINE {
    constexpr int PAR = decltype(par_c)::value;   // parity of n; C runs on n-1
    if (n - 1 >= n_lo && n - 1 < n_hi) {
      const unsigned char *x = smem + xch + (1 - PAR) * XG_B;
      pc[0] = *reinterpret_cast<const bf16x8 *>(x);
      pc[1] = *reinterpret_cast<const bf16x8 *>(x + 1024);
      dsc[0] = *reinterpret_cast<const bf16x8 *>(x + 2048);
      dsc[1] = *reinterpret_cast<const bf16x8 *>(x + 3072);
      const uint32_t base = stage_b((n - 1) >> 1) + 32 * (1 - PAR) * ROW_B;
      const uint32_t t0 = base + toff0[0], t1 = base + toff0[1];
      bf16x8 op[DIST + 1];
#pragma unroll
      for (int i = 0; i < DIST; ++i) op[i] = rd_c(t0, t1, i);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + DIST < 16) op[(i + DIST) % (DIST + 1)] = rd_c(t0, t1, i + DIST);
        const int ks = i >> 3, db = (i >> 1) & 3;
        if (i & 1)
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % (DIST + 1)], dsc[ks], dk[db], 0, 0, 0);
        else
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % (DIST + 1)], pc[ks], dv[db], 0, 0, 0);
      }
    }
    if (PAR == 0 && n >= 4 && (n + 2) / 2 < n_it) {
      wait_own_loads();
      stg_write((n + 2) / 2);
    }
    if (PAR == 1 && n >= 3 && (n + 3) / 2 < n_it) stg_load((n + 3) / 2);
    end_iter(n);
  };
  for (int n = -1; n <= n_sub; n += 2) {
    step(std::integral_constant<int, 1>{}, n);
    step(std::integral_constant<int, 0>{}, n + 1);
  }

  if (!key_ok || (DOC && !any)) return;
  // Accumulator element e4*4 + j of block dblk holds d = dblk*32 + e4*8 + hi*4 + j.
  const int64_t krow = (static_cast<int64_t>(bi) * a.s_kv + key) * a.n_kv + kvh;
  const int64_t orow = a.kv_row ? (a.kv_row[key] + bi * a.kv_row_bstride) * a.n_kv + kvh : krow;
  float *krow_out = a.dk + orow * D + hi * 4;
  float *vrow_out = a.dv + orow * D + hi * 4;
  // Per 32-column block, the eight 16-byte loads go out together before its
  // stores (dk and dv are separate arrays), so the block waits for memory once.
#pragma unroll
  for (int dblk = 0; dblk < D / 32; ++dblk) {
    float4 rk[4], rv[4];
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      rk[e4] = *reinterpret_cast<const float4 *>(krow_out + dblk * 32 + e4 * 8);
      rv[e4] = *reinterpret_cast<const float4 *>(vrow_out + dblk * 32 + e4 * 8);
    }
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      rk[e4].x += a.scale * dk[dblk][e4 * 4 + 0];
      rk[e4].y += a.scale * dk[dblk][e4 * 4 + 1];
      rk[e4].z += a.scale * dk[dblk][e4 * 4 + 2];
      rk[e4].w += a.scale * dk[dblk][e4 * 4 + 3];
      rv[e4].x += dv[dblk][e4 * 4 + 0];
      rv[e4].y += dv[dblk][e4 * 4 + 1];
      rv[e4].z += dv[dblk][e4 * 4 + 2];
      rv[e4].w += dv[dblk][e4 * 4 + 3];
      *reinterpret_cast<float4 *>(krow_out + dblk * 32 + e4 * 8) = rk[e4];
      *reinterpret_cast<float4 *>(vrow_out + dblk * 32 + e4 * 8) = rv[e4];
    }
  }
}

template <int HW>
hipError_t launch_dq(const BwdArgs &a, hipStream_t stream) {
  constexpr int TB = Q_WAVES / HW;
  const int64_t ntb = (a.s_q + TB * Q_QW - 1) / (TB * Q_QW);
  const int64_t blocks = ntb * a.b * a.n_kv * ((a.n_q / a.n_kv) / HW);
  if (blocks == 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (a.q_lo)
    bwd_dq_kernel<HW, true><<<static_cast<unsigned>(blocks), Q_THREADS, 0, stream>>>(a);
  else
    bwd_dq_kernel<HW, false><<<static_cast<unsigned>(blocks), Q_THREADS, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_delta(int64_t rows, int32_t d, int32_t esize, const void *dout,
                            const float *o, float *delta, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t threads = rows * (d / 8);
  int64_t blocks = (threads + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  const unsigned nb = static_cast<unsigned>(blocks);
  if (esize == 2 && d == 128)
    bwd_delta_kernel<uint16_t, 128, false><<<nb, 256, 0, stream>>>(
        rows, static_cast<const uint16_t *>(dout), o, delta, 1, 1, nullptr, nullptr);
  else if (esize == 2 && d == 64)
    bwd_delta_kernel<uint16_t, 64, false><<<nb, 256, 0, stream>>>(
        rows, static_cast<const uint16_t *>(dout), o, delta, 1, 1, nullptr, nullptr);
  else if (d == 128)
    bwd_delta_kernel<float, 128, false><<<nb, 256, 0, stream>>>(
        rows, static_cast<const float *>(dout), o, delta, 1, 1, nullptr, nullptr);
  else
    bwd_delta_kernel<float, 64, false><<<nb, 256, 0, stream>>>(
        rows, static_cast<const float *>(dout), o, delta, 1, 1, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(int32_t b, int64_t s, int32_t n_q, const void *dout, const float *o,
                           const float *lse, float *delta_t, float *lse_t, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(b) * s * n_q;
  if (rows == 0) return hipSuccess;
  int64_t blocks = (rows * (D / 8) + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  bwd_delta_kernel<uint16_t, D, true><<<static_cast<unsigned>(blocks), 256, 0, stream>>>(
      rows, static_cast<const uint16_t *>(dout), o, delta_t, s, n_q, lse, lse_t);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_bf16(const BwdArgs &a, hipStream_t stream) {
  if (a.b == 0 || a.s_q == 0 || a.s_kv == 0) return hipSuccess;
  const int g = a.n_q / a.n_kv;
  hipError_t err;
  if (g % 8 == 0)
    err = launch_dq<8>(a, stream);
  else if (g % 4 == 0)
    err = launch_dq<4>(a, stream);
  else if (g % 2 == 0)
    err = launch_dq<2>(a, stream);
  else
    err = launch_dq<1>(a, stream);
  if (err != hipSuccess) return err;
  const int64_t nkt = (a.s_kv + KV_KT - 1) / KV_KT;
  const int64_t blocks = nkt * a.b * a.n_kv;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (a.q_lo)
    bwd_dkdv_kernel<true><<<static_cast<unsigned>(blocks), KV_THREADS, 0, stream>>>(a);
  else
    bwd_dkdv_kernel<false><<<static_cast<unsigned>(blocks), KV_THREADS, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ra

extern "C" ra_status ra_attn_bwd_delta(int64_t rows, int32_t d, int32_t dtype, const void *dout,
                                       const float *o, float *delta, void *stream) {
  using ra::fail;
  ra::clear_error();
  if (rows < 0) return fail(RA_ERR_INVALID_ARG, "ra_attn_bwd_delta: rows < 0");
  if (d != 64 && d != 128) return fail(RA_ERR_UNSUPPORTED, "ra_attn_bwd_delta: d = %d (64 or 128)", d);
  if (dtype != RA_BF16 && dtype != RA_F32)
    return fail(RA_ERR_UNSUPPORTED, "ra_attn_bwd_delta: unknown dtype %d", dtype);
  if (rows == 0) return RA_OK;
  if (!dout || !o || !delta) return fail(RA_ERR_INVALID_ARG, "ra_attn_bwd_delta: NULL pointer");
  if (!ra::aligned16(dout) || !ra::aligned16(o))
    return fail(RA_ERR_INVALID_ARG, "ra_attn_bwd_delta: dout / o not 16-byte aligned");
  return ra::hip_check(ra::launch_bwd_delta(rows, d, dtype == RA_BF16 ? 2 : 4, dout, o, delta,
                                            static_cast<hipStream_t>(stream)),
                       "ra_attn_bwd_delta launch");
}

extern "C" ra_status ra_block_attn_bwd(const ra_attn_desc *desc, const void *q, const void *k,
                                       const void *v, const void *dout, const float *lse,
                                       const float *delta, float *dq, float *dk, float *dv,
                                       void *stream) {
  using ra::fail;
  ra::clear_error();
  ra_status st = ra::validate_attn(desc, q, k, v, dq, lse);
  if (st != RA_OK) return st;
  if (desc->dtype != RA_BF16 || desc->d != 128)
    return fail(RA_ERR_UNSUPPORTED, "ra_block_attn_bwd: bf16 with d = 128 only");
  if (desc->v_layout != RA_V_ROWS)
    return fail(RA_ERR_UNSUPPORTED, "ra_block_attn_bwd: v must be row-major (RA_V_ROWS)");
  if (desc->b == 0 || desc->s_q == 0 || desc->s_kv == 0) return RA_OK;
  if (!dout || !delta || !dk || !dv)
    return fail(RA_ERR_INVALID_ARG, "ra_block_attn_bwd: NULL dout / delta / dk / dv");
  if (!ra::aligned16(dout) || !ra::aligned16(dk) || !ra::aligned16(dv) || !ra::aligned16(dq))
    return fail(RA_ERR_INVALID_ARG, "ra_block_attn_bwd: dout / dq / dk / dv not 16-byte aligned");
  ra::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
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
  return ra::hip_check(ra::launch_attn_bwd_bf16(a, static_cast<hipStream_t>(stream)),
                       "ra_block_attn_bwd launch");
}
