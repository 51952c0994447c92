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
//     Every lane holds one query, so lse and D are per-lane constants;
//   * bwd_dkdv_kernel (bf16, d = 128): a wave owns 32 keys of one key/value
//     head, with its K and V rows in registers; 4 waves share each block of 64
//     queries (q, do, lse, D, positions) staged in LDS, for every query head of
//     the GQA group, and work through it in 32-row sub-blocks: A, S = Q K^T and
//     dP = dO V^T (Q and dO rows by ds_read_b128); B, P and dS on the VALU; C,
//     dV^T += dO^T P and dK^T += Q^T dS (dO^T and Q^T by the transposing read),
//     so each lane ends up holding d-values of one key. The sub-blocks run as
//     a software pipeline: A of the next and C of the previous sub-block share
//     one stream of MFMAs into which B of the current one is interleaved.
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

template <typename T, int DD>
__global__ __launch_bounds__(256) void bwd_delta_kernel(int64_t rows, const T *__restrict__ dout,
                                                        const float *__restrict__ o,
                                                        float *__restrict__ delta) {
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
    float s = x[0] * o0.x + x[1] * o0.y + x[2] * o0.z + x[3] * o0.w +
              x[4] * o1.x + x[5] * o1.y + x[6] * o1.z + x[7] * o1.w;
#pragma unroll
    for (int m = TPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if (t == 0) delta[r] = s;
  }
}

// ---------------------------------------------------------------- dQ

constexpr int Q_WAVES = 8;
constexpr int Q_THREADS = Q_WAVES * 64;
constexpr int Q_QW = 32;
constexpr int Q_BK = 64;
constexpr int Q_TILE_B = Q_BK * ROW_B;
constexpr int Q_LOADS = Q_TILE_B / (1024 * Q_WAVES);

// DOC: a document mask is given (a.q_lo); without it the mask code compiles away.
template <int HW, bool DOC>
__global__ __launch_bounds__(Q_THREADS, 1) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char k_lds0[Q_TILE_B], k_lds1[Q_TILE_B],
      k_lds2[Q_TILE_B];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds0[Q_TILE_B], v_lds1[Q_TILE_B],
      v_lds2[Q_TILE_B];
  __shared__ __attribute__((aligned(16))) int32_t p_lds0[Q_BK], p_lds1[Q_BK], p_lds2[Q_BK];
  auto k_stage = [&](auto s) INLINE -> unsigned char * {
    constexpr int v = decltype(s)::value;
    return v == 0 ? k_lds0 : v == 1 ? k_lds1 : k_lds2;
  };
  auto v_stage = [&](auto s) INLINE -> unsigned char * {
    constexpr int v = decltype(s)::value;
    return v == 0 ? v_lds0 : v == 1 ? v_lds1 : v_lds2;
  };
  auto p_stage = [&](auto s) INLINE -> int32_t * {
    constexpr int v = decltype(s)::value;
    return v == 0 ? p_lds0 : v == 1 ? p_lds1 : p_lds2;
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
  const float lse2 = tok_ok ? lse_log2(a.lse[row]) : INFINITY;
  const float dlt = tok_ok ? a.delta[row] : 0.f;
  const float sl2 = a.scale * LOG2E;

  uint32_t koff[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds)
    koff[ds] = col * ROW_B + ((((2 * ds + hi) ^ swz(col & 15))) << 4);
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

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};

  // Per tile: S^T and dP^T (32 MFMAs, K and V rows read a few MFMAs ahead),
  // the element mask where needed, then dQ^T += K^T dS^T (16 MFMAs, K^T by the
  // transposing read) with dS^T of the next k-step formed on the VALU between
  // them. Scheduling fences keep the reads ahead of their MFMAs: left to
  // itself the compiler waits for each read right before its MFMA.
  constexpr int DIST = 4;
  auto process = [&](int t, auto stage) INLINE {
    const unsigned char *kb = k_stage(stage);
    const unsigned char *vb = v_stage(stage);
    f32x16 s[2], dp[2];
    // Item i: k-step i/4, key block (i/2)%2; S^T from K when i is even, dP^T
    // from V when odd.
    auto rd_a = [&](int i) INLINE -> bf16x8 {
      const unsigned char *base = (i & 1) ? vb : kb;
      return *reinterpret_cast<const bf16x8 *>(base + koff[i >> 2] + ((i >> 1) & 1) * 32 * ROW_B);
    };
    {
      bf16x8 op[DIST + 1];
#pragma unroll
      for (int i = 0; i < DIST; ++i) op[i] = rd_a(i);
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i + DIST < 32) op[(i + DIST) % (DIST + 1)] = rd_a(i + DIST);
        const int ds = i >> 2, j = (i >> 1) & 1;
        const bf16x8 o = op[i % (DIST + 1)];
        if (i & 1)
          dp[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, dreg[ds], ds == 0 ? f32x16{} : dp[j], 0, 0, 0);
        else
          s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, qreg[ds], ds == 0 ? f32x16{} : s[j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Element e4*4 + j of key block kb holds key kb*32 + e4*8 + hi*4 + j.
    const int64_t key0 = kbeg + static_cast<int64_t>(t) * Q_BK;
    const bool ragged = key0 + Q_BK > a.s_kv;
    if (ragged || (a.causal && p_stage(stage)[Q_BK - 1] > w_qmin) ||
        (DOC && p_stage(stage)[0] < w_lomax)) {
      const int lim = ragged ? static_cast<int>(a.s_kv - key0) : Q_BK;
      const int32_t *pp = p_stage(stage);
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
    // dS^T = P^T (dP^T - D) as the bf16 B operand of dQ^T += K^T dS^T:
    // k-step ks holds accumulator elements (ks%2)*8 .. +7 of key block ks/2.
    bf16x8 dsb[4];
    auto ds_pair = [&](int ks, int e) INLINE {
#pragma unroll
      for (int u = e; u < e + 2; ++u) {
        const int j = ks >> 1, el = (ks & 1) * 8 + u;
        const float p = exp2_fast(fmaf(s[j][el], sl2, -lse2));
        dsb[ks][u] = static_cast<__bf16>(p * (dp[j][el] - dlt));
      }
      asm volatile("" : "+v"(dsb[ks]));  // keep it between the MFMAs
    };
#pragma unroll
    for (int e = 0; e < 8; e += 2) ds_pair(0, e);
    auto rd_c = [&](int i) INLINE -> bf16x8 { return tr_read(kb, toff, i & 3, (i >> 2) * 16); };
    {
      bf16x8 op[DIST + 1];
#pragma unroll
      for (int i = 0; i < DIST; ++i) op[i] = rd_c(i);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + DIST < 16) op[(i + DIST) % (DIST + 1)] = rd_c(i + DIST);
        const int ks = i >> 2, db = i & 3;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i % (DIST + 1)], dsb[ks], acc[db], 0, 0, 0);
        if (ks + 1 < 4) ds_pair(ks + 1, 2 * (i & 3));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  using St0 = std::integral_constant<int, 0>;
  using St1 = std::integral_constant<int, 1>;
  using St2 = std::integral_constant<int, 2>;
  if (nt > 0) issue_tile(0, St0{});
  if (nt > 1) issue_tile(1, St1{});
  auto step = [&](auto stage_c, int t) INLINE {
    constexpr int S = decltype(stage_c)::value;
    using SC = std::integral_constant<int, S>;
    using SL = std::integral_constant<int, (S + 2) % 3>;
    wait_own_loads();  // tiles t (and t+1) have landed in this wave's share ...
    __syncthreads();   // ... and in everyone's; every wave is done with tile t-1
    if (t + 2 < nt) issue_tile(t + 2, SL{});
    if (t < w_nt) process(t, SC{});
  };
  for (int t = 0; t < nt; t += 3) {
    step(St0{}, t);
    if (t + 1 < nt) step(St1{}, t + 1);
    if (t + 2 < nt) step(St2{}, t + 2);
  }

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

constexpr int KV_WAVES = 4;
constexpr int KV_THREADS = KV_WAVES * 64;
constexpr int KV_KW = 32;                    // keys per wave
constexpr int KV_KT = KV_WAVES * KV_KW;      // keys per workgroup
constexpr int KV_QB = 64;                    // queries per staged block (two 32-row sub-blocks)
constexpr int KV_SUB = 32;
constexpr int KV_TILE_B = KV_QB * ROW_B;     // 16 KiB (q or do)
constexpr int KV_LOADS = KV_TILE_B / (1024 * KV_WAVES);

template <bool DOC>
__global__ __launch_bounds__(KV_THREADS, 1) void bwd_dkdv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char q_lds0[KV_TILE_B], q_lds1[KV_TILE_B],
      q_lds2[KV_TILE_B];
  __shared__ __attribute__((aligned(16))) unsigned char d_lds0[KV_TILE_B], d_lds1[KV_TILE_B],
      d_lds2[KV_TILE_B];
  // per stage: lse (64 floats), delta (64 floats), positions (64 int32) of the block's rows
  __shared__ __attribute__((aligned(16))) float l_lds0[64], l_lds1[64], l_lds2[64];
  __shared__ __attribute__((aligned(16))) float e_lds0[64], e_lds1[64], e_lds2[64];
  __shared__ __attribute__((aligned(16))) int32_t p_lds0[64], p_lds1[64], p_lds2[64];
  // ... and the rows' document starts (document mask)
  __shared__ __attribute__((aligned(16))) int32_t o_lds0[64], o_lds1[64], o_lds2[64];
  auto q_stage = [&](auto s) INLINE -> unsigned char * {
    constexpr int v = decltype(s)::value;
    return v == 0 ? q_lds0 : v == 1 ? q_lds1 : q_lds2;
  };
  auto d_stage = [&](auto s) INLINE -> unsigned char * {
    constexpr int v = decltype(s)::value;
    return v == 0 ? d_lds0 : v == 1 ? d_lds1 : d_lds2;
  };
  auto l_stage = [&](auto s) INLINE -> float * {
    constexpr int v = decltype(s)::value;
    return v == 0 ? l_lds0 : v == 1 ? l_lds1 : l_lds2;
  };
  auto e_stage = [&](auto s) INLINE -> float * {
    constexpr int v = decltype(s)::value;
    return v == 0 ? e_lds0 : v == 1 ? e_lds1 : e_lds2;
  };
  auto p_stage = [&](auto s) INLINE -> int32_t * {
    constexpr int v = decltype(s)::value;
    return v == 0 ? p_lds0 : v == 1 ? p_lds1 : p_lds2;
  };
  auto lo_stage = [&](auto s) INLINE -> int32_t * {
    constexpr int v = decltype(s)::value;
    return v == 0 ? o_lds0 : v == 1 ? o_lds1 : o_lds2;
  };

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int hi = lane >> 5;

  // ---- workgroup -> (batch, kv head, key tile); earliest keys (most queries) first ----
  const int64_t nkt = (a.s_kv + KV_KT - 1) / KV_KT;
  const int64_t inner = static_cast<int64_t>(a.b) * a.n_kv;
  const int64_t kt = blockIdx.x / inner;
  const int kvh = static_cast<int>(blockIdx.x % a.n_kv);
  const int bi = static_cast<int>((blockIdx.x / a.n_kv) % a.b);
  (void)nkt;
  const int g = a.n_q / a.n_kv;

  const int64_t wg_key0 = kt * KV_KT;
  const int64_t w_key0 = wg_key0 + wave * KV_KW;
  const int64_t key = w_key0 + col;
  const bool key_ok = key < a.s_kv;
  const bool wave_has_keys = w_key0 < a.s_kv;
  const int32_t kpos = !key_ok ? INT_MAX : (a.causal ? a.kv_pos[key] : INT_MIN);
  // The wave's first and last key positions (causal skips and masks).
  int32_t w_kmin = INT_MIN, w_kmax = INT_MIN;
  if (a.causal && wave_has_keys) {
    w_kmin = a.kv_pos[w_key0];
    w_kmax = a.kv_pos[min(w_key0 + KV_KW, a.s_kv) - 1];
  }

  // ---- query range that can see any key of the workgroup ----
  // Causal: from the first query at or after its first key. With a document
  // mask, up to the last query whose document starts at or before its last
  // key (document starts are non-decreasing).
  int64_t q_first = 0, q_end = a.s_q;
  if (a.causal) q_first = count_lt(a.q_pos, a.s_q, a.kv_pos[wg_key0]);
  if (DOC) q_end = count_le(a.q_lo, a.s_q, a.kv_pos[min(wg_key0 + KV_KT, a.s_kv) - 1]);
  const int64_t qb0 = q_first / KV_QB;
  const int64_t nqb = (q_end + KV_QB - 1) / KV_QB;
  const int64_t n_blk = nqb > qb0 ? nqb - qb0 : 0;   // query blocks per head
  const int n_it = static_cast<int>(n_blk * g);

  // ---- this lane's key: B operands of S = Q K^T and dP = dO V^T ----
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
    asm volatile("" : "+a"(kreg[ds]), "+a"(vreg[ds]));  // they live in AGPRs (see mfma_a)
  }
  const float sl2 = a.scale * LOG2E;

  // Q / dO rows by ds_read_b128 (row = query col), chunk 2*ds + hi: the
  // swizzle is an XOR of the chunk index, so k-step ds reads at qoff0 with
  // bits 5..7 XORed by ds. Likewise the transposing reads of d block db are at
  // toff0 with bits 6..7 XORed by db. (`pin` keeps the compiler from hoisting
  // the XORs back into eight registers each.)
  uint32_t qoff0 = col * ROW_B + (((hi ^ swz(col & 15))) << 4);
  auto qoff = [&](int ds) INLINE -> uint32_t { return qoff0 ^ (static_cast<uint32_t>(ds) << 5); };
  uint32_t toff0[2];
  {
    uint32_t toff[2][D / 32];
    tr_offsets(lane, toff);
    toff0[0] = toff[0][0];
    toff0[1] = toff[1][0];
  }
  auto tread = [&](const unsigned char *base, int db, int row0) INLINE -> bf16x8 {
    const uint32_t x = static_cast<uint32_t>(db) << 6;
    const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (LDS_AS bf16x4 *)(base + (toff0[0] ^ x) + row0 * ROW_B));
    const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (LDS_AS bf16x4 *)(base + (toff0[1] ^ x) + row0 * ROW_B));
    return bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
  };

  // ---- staging of one query block (iteration it -> head, block) ----
  const unsigned char *qbytes = static_cast<const unsigned char *>(a.q);
  const unsigned char *dbytes = static_cast<const unsigned char *>(a.dout);
  const int64_t q_row_bytes = static_cast<int64_t>(a.n_q) * D * 2;
  uint32_t goff[KV_LOADS];
#pragma unroll
  for (int i = 0; i < KV_LOADS; ++i) {
    const int r = 4 * (wave + KV_WAVES * i) + (lane >> 4);
    goff[i] = static_cast<uint32_t>(r * q_row_bytes + (((lane & 15) ^ swz(r & 15)) << 4));
  }
  // Iteration it -> (query block, head): blocks from the last one down, the g
  // heads of a block back to back. Every workgroup of a kv head then walks the
  // same blocks in the same order (they differ only in where they stop), so
  // workgroups resident together read each block while it is in L2.
  auto blk_of = [&](int it, int64_t *q0, int *h) INLINE {
    const int64_t j = it / g;
    *q0 = (qb0 + n_blk - 1 - j) * KV_QB;
    *h = kvh * g + static_cast<int>(it - j * g);
  };
  auto issue_blk = [&](int it, auto stage) INLINE {
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
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rq, (LDS_AS void *)(q_stage(stage) + 4 * (wave + KV_WAVES * i) * ROW_B), 16, goff[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rd, (LDS_AS void *)(d_stage(stage) + 4 * (wave + KV_WAVES * i) * ROW_B), 16, goff[i], 0, 0, 0);
    }
    // lse and delta rows q0 + lane of head h (stride n_q floats); positions q0 + lane.
    if (wave == 0) {
      const __amdgpu_buffer_rsrc_t rl =
          make_rsrc(a.lse + rbase, ((left - 1) * a.n_q + 1) * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (LDS_AS void *)l_stage(stage), 4,
                                               lane * a.n_q * 4, 0, 0, 0);
    } else if (wave == 1) {
      const __amdgpu_buffer_rsrc_t re =
          make_rsrc(a.delta + rbase, ((left - 1) * a.n_q + 1) * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (LDS_AS void *)e_stage(stage), 4,
                                               lane * a.n_q * 4, 0, 0, 0);
    } else if (wave == 2 && a.causal) {
      const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.q_pos + q0, left * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (LDS_AS void *)p_stage(stage), 4, lane * 4,
                                               0, 0, 0);
    } else if (DOC && wave == 3) {
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q_lo + q0, left * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (LDS_AS void *)lo_stage(stage), 4, lane * 4,
                                               0, 0, 0);
    }
  };

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  // ---- the wave's sub-blocks ----
  // Sub-block n = 2 it + h holds rows 32h .. 32h+31 of the block of iteration
  // it. A sub-block whose rows are all before the wave's first key (causal),
  // or all start their document after its last key, or lie past the
  // sequence, sees none of the wave's keys. In row terms the useful first rows
  // r (multiples of 32) satisfy c_vis - 31 <= r < r_end; they form one range
  // of blocks in the walk, whose first and last blocks may have one useless
  // half per head (those run fully masked and add nothing). n_lo .. n_hi is
  // that range in the walk. c_kmax / c_dmin decide which sub-blocks need the
  // element mask.
  int64_t c_vis = 0, c_kmax = 0, r_end = a.s_q, c_dmin = a.s_q;
  if (a.causal && wave_has_keys) {
    c_vis = wave_count<false>(a.q_pos, a.s_q, w_kmin, lane);
    c_kmax = wave_count<false>(a.q_pos, a.s_q, w_kmax, lane);
  }
  if (DOC && wave_has_keys) {
    r_end = min(r_end, wave_count<true>(a.q_lo, a.s_q, w_kmax, lane));
    c_dmin = wave_count<true>(a.q_lo, a.s_q, w_kmin, lane);
  }
  const int64_t qb_last = qb0 + n_blk - 1;
  int64_t R_lo = (c_vis - 31 + 31) / 32;  // ceil((c_vis - 31) / 32) for c_vis >= 0
  if (c_vis < 31) R_lo = 0;
  int64_t R_hi = (r_end + 31) / 32 - 1;   // last useful 32-row unit
  R_lo = max(R_lo, 2 * qb0);
  R_hi = min(R_hi, 2 * qb_last + 1);
  int n_lo = 0, n_hi = 0;
  if (wave_has_keys && n_blk > 0 && R_lo <= R_hi) {
    const int64_t j_first = qb_last - R_hi / 2;          // walk block of the latest unit
    const int64_t h_min = max<int64_t>(0, R_lo - 2 * (qb_last - j_first));
    n_lo = static_cast<int>(2 * (j_first * g) + h_min);
    const int64_t j_last = qb_last - R_lo / 2;           // walk block of the earliest unit
    const int64_t h_max = min<int64_t>(1, R_hi - 2 * (qb_last - j_last));
    n_hi = static_cast<int>(2 * (j_last * g + g - 1) + h_max + 1);
  }
  const bool any = n_lo < n_hi;
  const bool w_ragged = w_key0 + KV_KW > a.s_kv;   // some key of the wave past the block

  // ---- software pipeline over sub-blocks ----
  // One wave per SIMD, so the wave itself must overlap its MFMAs with its
  // vector work. Iteration n runs one stream of 32 MFMAs, A(n+1) -- S = Q K^T
  // and dP = dO V^T of the next sub-block -- interleaved with C(n-1) --
  // dV^T += dO^T P and dK^T += Q^T dS of the previous one -- with operands
  // read a few MFMAs ahead, and after every MFMA the vector work of B(n): the
  // probabilities P and dS of one element of this sub-block. Scores, P and dS
  // are double-buffered by sub-block parity. The element mask (rare: the
  // diagonal, ragged rows or keys, a document start) is applied to A(n+1)'s
  // scores right after the stream.
  // S accumulator: lane holds key `col`; element a holds sub-block row
  // (a/4)*8 + hi*4 + a%4.
  f32x16 s[2], dp[2];
  bf16x8 pb[2][2], dsb[2][2];
  // P and dS start at zero: the first C of the wave's range (of the
  // sub-block before it) then adds nothing.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      pb[i][j] = bf16x8{};
      dsb[i][j] = bf16x8{};
    }
  float4 l4[4], d4[4];  // lse (log2 units) and D of the rows of the sub-block of B

  auto blk_q0 = [&](int it) INLINE -> int64_t { return (qb_last - it / g) * KV_QB; };
  auto read_ld = [&](auto stage, int rb) INLINE {
    const float *ll = l_stage(stage) + rb;
    const float *ee = e_stage(stage) + rb;
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
      pb[par][j >> 3][j & 7] = static_cast<__bf16>(p);
      dsb[par][j >> 3][j & 7] = static_cast<__bf16>(p * (dp[par][j] - d4[j >> 2][j & 3]));
    }
    // Keep the pair here, between the MFMAs: otherwise the compiler sinks all
    // of B past the stream, where nothing overlaps it.
    asm volatile("" : "+v"(pb[par][el >> 3]), "+v"(dsb[par][el >> 3]));
  };
  // Operand of A item a (k-step a/2; S from the Q rows when a is even, dP from
  // the dO rows when odd) for the sub-block at rows rb of `stage`.
  auto rd_a = [&](auto stage, int rb, int ai) INLINE -> bf16x8 {
    const unsigned char *base = ((ai & 1) ? d_stage(stage) : q_stage(stage)) + rb * ROW_B;
    return *reinterpret_cast<const bf16x8 *>(base + qoff(ai >> 1));
  };
  // Operand of C item c (16-row step c/8, d block (c/2)%4; dV from dO^T when
  // c is even, dK from Q^T when odd), by the transposing read.
  auto rd_c = [&](auto stage, int rb, int ci) INLINE -> bf16x8 {
    const unsigned char *base = (ci & 1) ? q_stage(stage) : d_stage(stage);
    return tread(base, (ci >> 1) & 3, rb + (ci >> 3) * 16);
  };
  // A's MFMAs are written out so that the K and V rows (read-only, the B
  // operands) sit in AGPRs and S, dP land in VGPRs, where B reads them:
  // left to itself the compiler keeps K, V in VGPRs and S, dP in AGPRs, and
  // moves all 32 results out of AGPRs on every sub-block. The compiler's
  // hazard checks do not see these MFMAs: their results are read by B one
  // iteration later (after several MFMAs), or by the element mask, which
  // first waits out their writes.
  auto mfma_a = [&](int par, int ai, const bf16x8 &o) INLINE {
    const int ds = ai >> 1;
    f32x16 &r = (ai & 1) ? dp[par] : s[par];
    const bf16x8 &b = (ai & 1) ? vreg[ds] : kreg[ds];
    if (ds == 0)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(r) : "v"(o), "a"(b));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(r) : "v"(o), "a"(b));
  };
  auto mfma_c = [&](int par, int ci, const bf16x8 &o) INLINE {
    const int ks = ci >> 3, db = (ci >> 1) & 3;
    if (ci & 1)
      dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, dsb[par][ks], dk[db], 0, 0, 0);
    else
      dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, pb[par][ks], dv[db], 0, 0, 0);
  };
  constexpr int DIST = 4;  // operand reads ahead of their MFMA
  // The full stream: A(n+1) on even slots, C(n-1) on odd slots, a pair of B(n)
  // elements after every fourth MFMA (the lse and D reads at the top of the
  // iteration land meanwhile).
  auto stream = [&](auto sa, int rb_a, int pa, auto sc, int rb_c, int pc, int pbp) INLINE {
    auto rd = [&](int i) INLINE -> bf16x8 {
      return (i & 1) ? rd_c(sc, rb_c, i >> 1) : rd_a(sa, rb_a, i >> 1);
    };
    bf16x8 op[DIST + 1];
#pragma unroll
    for (int i = 0; i < DIST; ++i) op[i] = rd(i);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i + DIST < 32) op[(i + DIST) % (DIST + 1)] = rd(i + DIST);
      if (i & 1)
        mfma_c(pc, i >> 1, op[i % (DIST + 1)]);
      else
        mfma_a(pa, i >> 1, op[i % (DIST + 1)]);
      if ((i & 3) == 3) b_pair(pbp, 2 * (i >> 2));
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // A alone (before the wave's first sub-block) and C alone (after its last).
  auto a_only = [&](auto sa, int rb_a, int pa) INLINE {
    bf16x8 op[DIST + 1];
#pragma unroll
    for (int i = 0; i < DIST; ++i) op[i] = rd_a(sa, rb_a, i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + DIST < 16) op[(i + DIST) % (DIST + 1)] = rd_a(sa, rb_a, i + DIST);
      mfma_a(pa, i, op[i % (DIST + 1)]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto c_only = [&](auto sc, int rb_c, int pc) INLINE {
    bf16x8 op[DIST + 1];
#pragma unroll
    for (int i = 0; i < DIST; ++i) op[i] = rd_c(sc, rb_c, i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + DIST < 16) op[(i + DIST) % (DIST + 1)] = rd_c(sc, rb_c, i + DIST);
      mfma_c(pc, i, op[i % (DIST + 1)]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Element mask of A's scores (sub-block at rows rb of `stage`, block rows
  // from q0): rows past the sequence, keys past the block, a query before the
  // key (causal), or a key before the query's document.
  auto mask_a = [&](auto stage, int rb, int par, int64_t q0) INLINE {
    const int64_t qlim = a.s_q - q0 - rb;
    const int64_t row0 = q0 + rb;
    const bool need = qlim < KV_SUB || w_ragged || (a.causal && row0 < c_kmax) ||
                      (DOC && row0 + min<int64_t>(KV_SUB, qlim) - 1 >= c_dmin);
    if (need) {
      // wait out the writes of the last A MFMAs (written out, see mfma_a)
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
      const int32_t *pp = p_stage(stage) + rb;
      const int32_t *lp = lo_stage(stage) + rb;
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

  // Wave 0 loads every block's lse and converts it in place to log2 units
  // (-inf, a query with no key, to +inf so that its probabilities are 0):
  // block 0 before the first barrier, block it+1 in the second iteration of
  // block it (it landed at the first one's barrier; the other waves read it
  // after the second one's).
  auto prescale_lse = [&](auto stage) INLINE {
    if (wave == 0) {
      float *l = l_stage(stage);
      l[lane] = lse_log2(l[lane]);
    }
  };

  using St0 = std::integral_constant<int, 0>;
  using St1 = std::integral_constant<int, 1>;
  using St2 = std::integral_constant<int, 2>;
  // Block it lives in stage it % 3. Blocks 0 and 1 start streaming now; block
  // it+2 is issued at the barrier of iteration 2 it, once every wave is done
  // with block it-1 (its C ran in that iteration).
  if (n_it > 0) issue_blk(0, St0{});
  if (n_it > 1) issue_blk(1, St1{});
  // Stage 2 is read (with zero P and dS) by the first iteration's C before any
  // block lands in it: clear it so that it holds finite values.
#pragma unroll
  for (int i = 0; i < KV_TILE_B / (16 * KV_THREADS); ++i) {
    reinterpret_cast<u32x4 *>(q_lds2)[tid + i * KV_THREADS] = u32x4{0, 0, 0, 0};
    reinterpret_cast<u32x4 *>(d_lds2)[tid + i * KV_THREADS] = u32x4{0, 0, 0, 0};
  }
  wait_own_loads();
  if (n_it > 0) prescale_lse(St0{});
  __syncthreads();
  if (n_lo == 0 && n_hi > 0) {
    a_only(St0{}, 0, 0);
    mask_a(St0{}, 0, 0, blk_q0(0));
  }
  const int n_sub = 2 * n_it;
  // Iteration n (n % 6 = K): B on sub-block n, A on n+1, C on n-1.
  auto step = [&](auto k_c, int n) INLINE {
    constexpr int K = decltype(k_c)::value;
    constexpr int H = K % 2;                 // half of its block
    using SB = std::integral_constant<int, (K / 2) % 3>;         // stage of n's block
    using SA = std::integral_constant<int, ((K + 1) / 2) % 3>;   // ... of n+1's
    using SC = std::integral_constant<int, ((K + 5) / 2) % 3>;   // ... of n-1's
    constexpr int RB = 32 * H, RB_O = 32 * (1 - H);  // rows of n; of n+1 and n-1
    constexpr int PB = H, PO = 1 - H;                // parity of n; of n+-1
    const int it = n >> 1;
    asm volatile("" : "+v"(qoff0), "+v"(toff0[0]), "+v"(toff0[1]));  // pin: see qoff
    // Inside the range the full stream runs; its A past the range computes
    // scores nobody reads, and its C before the range adds zero P and dS.
    if (n >= n_lo && n < n_hi) {
      read_ld(SB{}, RB);
      stream(SA{}, RB_O, PO, SC{}, RB_O, PO, PB);
      if (n + 1 < n_hi) mask_a(SA{}, RB_O, PO, blk_q0((n + 1) >> 1));
    } else if (n + 1 == n_lo) {
      a_only(SA{}, RB_O, PO);
      mask_a(SA{}, RB_O, PO, blk_q0((n + 1) >> 1));
    } else if (n == n_hi) {
      c_only(SC{}, RB_O, PO);
    }
    if constexpr (H == 0) {
      wait_own_loads();  // block it+1 has landed
      __syncthreads();
      if (it + 2 < n_it) issue_blk(it + 2, SC{});
    } else {
      if (it + 1 < n_it) prescale_lse(SA{});
      __syncthreads();
    }
  };
  for (int n = 0; n < n_sub; n += 6) {
    step(std::integral_constant<int, 0>{}, n);
    step(std::integral_constant<int, 1>{}, n + 1);
    if (n + 2 < n_sub) step(std::integral_constant<int, 2>{}, n + 2);
    if (n + 3 < n_sub) step(std::integral_constant<int, 3>{}, n + 3);
    if (n + 4 < n_sub) step(std::integral_constant<int, 4>{}, n + 4);
    if (n + 5 < n_sub) step(std::integral_constant<int, 5>{}, n + 5);
  }
  // C of the last sub-block (its block's stage is still intact).
  if (n_hi == n_sub && n_lo < n_hi) {
    const int st = (n_it - 1) % 3;
    if (st == 0)
      c_only(St0{}, 32, 1);
    else if (st == 1)
      c_only(St1{}, 32, 1);
    else
      c_only(St2{}, 32, 1);
  }

  if (!key_ok || (DOC && !any)) return;
  // Accumulator element e4*4 + j of block dblk holds d = dblk*32 + e4*8 + hi*4 + j.
  const int64_t orow = a.kv_row ? (a.kv_row[key] + bi * a.kv_row_bstride) * a.n_kv + kvh : krow;
  float *krow_out = a.dk + orow * D + hi * 4;
  float *vrow_out = a.dv + orow * D + hi * 4;
#pragma unroll
  for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      float4 *pk = reinterpret_cast<float4 *>(krow_out + dblk * 32 + e4 * 8);
      float4 *pv = reinterpret_cast<float4 *>(vrow_out + dblk * 32 + e4 * 8);
      float4 rk = *pk, rv = *pv;
      rk.x += a.scale * dk[dblk][e4 * 4 + 0];
      rk.y += a.scale * dk[dblk][e4 * 4 + 1];
      rk.z += a.scale * dk[dblk][e4 * 4 + 2];
      rk.w += a.scale * dk[dblk][e4 * 4 + 3];
      rv.x += dv[dblk][e4 * 4 + 0];
      rv.y += dv[dblk][e4 * 4 + 1];
      rv.z += dv[dblk][e4 * 4 + 2];
      rv.w += dv[dblk][e4 * 4 + 3];
      *pk = rk;
      *pv = rv;
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
    bwd_delta_kernel<uint16_t, 128><<<nb, 256, 0, stream>>>(rows, static_cast<const uint16_t *>(dout), o, delta);
  else if (esize == 2 && d == 64)
    bwd_delta_kernel<uint16_t, 64><<<nb, 256, 0, stream>>>(rows, static_cast<const uint16_t *>(dout), o, delta);
  else if (d == 128)
    bwd_delta_kernel<float, 128><<<nb, 256, 0, stream>>>(rows, static_cast<const float *>(dout), o, delta);
  else
    bwd_delta_kernel<float, 64><<<nb, 256, 0, stream>>>(rows, static_cast<const float *>(dout), o, delta);
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
