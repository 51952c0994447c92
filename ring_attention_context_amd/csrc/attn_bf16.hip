// bf16 block attention on gfx950 matrix cores.
//
// Computes, for the keys of one block, the statistics of "Context
// Parallelism and Ring Attention" §3: m_b = max x, l_b = sum e^{x - m_b},
// o_b = (1/l_b) sum e^{x - m_b} v, lse_b = m_b + ln l_b, scanning the block
// tile by tile with a running max, running sum and unnormalised output (the
// single-GPU form of the same identity, §3). The causal rule of §5 is applied
// on original positions (§6 "the cost of reordering"); positions are
// non-decreasing, so whole tiles past a query tile's last position are never
// loaded (the tile skipping of §7), and only tiles that straddle the
// diagonal, or the ragged last tile, evaluate the element mask.
//
// Work decomposition (d = 128):
//   * a wave owns 32 query tokens of one query head; a workgroup of 4 waves
//     owns TB = 4 / HW consecutive 32-token blocks of HW heads that share one
//     key/value head (GQA), so each K/V tile staged in LDS serves every
//     query row of the workgroup;
//   * K/V tiles of 64 keys: K is stored row-major ([key][d]) and V transposed
//     ([d][key]) in LDS, both padded so the 16-byte MFMA operand reads of a
//     wave are bank-conflict free;
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: each lane then holds 32 keys of ONE query, so
//     the row max and row sum are in-lane plus one exchange with the lane 32
//     away, and the fp32 probabilities convert in place into the B operand of
//     O^T = V^T P^T (the same MFMA shape), whose accumulator keeps one query
//     per lane -- the rescale by e^{m_old - m_new} is a per-lane scalar;
//   * exponentials run in base 2 (v_exp_f32) with the scale folded in:
//     p = 2^(s * scale * log2(e) - m), lse is converted back to natural log.
// Workgroups are ordered heaviest query tile first (later positions see more
// keys under the causal rule).
#include <climits>

#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr int QW = 32;                 // query tokens per wave
constexpr int WAVES = 4;
constexpr int THREADS = WAVES * 64;
constexpr int BK = 64;                 // keys per tile
constexpr int K_STRIDE = D * 2 + 16;   // bytes per key row of K in LDS
constexpr int VT_STRIDE = BK * 2 + 16; // bytes per d row of V^T in LDS
constexpr int K_BYTES = BK * K_STRIDE;
constexpr int VT_BYTES = D * VT_STRIDE;
constexpr int LDS_BYTES = K_BYTES + VT_BYTES + BK * 4;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float swap_halves(float x) {
  // Value of the lane 32 away (lanes l and l ^ 32 hold the two key halves of
  // the same query).
  return __shfl_xor(x, 32);
}

// Number of keys with position <= p in the non-decreasing kv_pos[0, n).
__device__ __forceinline__ int64_t count_le(const int32_t *kv_pos, int64_t n, int32_t p) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (kv_pos[mid] <= p)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

template <int HW>
__global__ __launch_bounds__(THREADS, 2) void attn_bf16_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char *k_lds = smem;
  unsigned char *vt_lds = smem + K_BYTES;
  int32_t *pos_lds = reinterpret_cast<int32_t *>(smem + K_BYTES + VT_BYTES);

  constexpr int TB = WAVES / HW;  // 32-token blocks per workgroup
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;  // query within the wave
  const int hi = lane >> 5;   // which half of the MFMA k-slots this lane holds

  // ---- workgroup -> (batch, kv head, head group, token block) ----
  const int g = a.n_q / a.n_kv;
  const int hgroups = g / HW;
  const int64_t tok_per_wg = TB * QW;
  const int64_t ntb = (a.s_q + tok_per_wg - 1) / tok_per_wg;
  const int64_t inner = static_cast<int64_t>(a.b) * a.n_kv * hgroups;
  const int64_t id = blockIdx.x;
  const int64_t tb = ntb - 1 - id / inner;  // heaviest (latest) token block first
  int64_t rem = id % inner;
  const int hgi = static_cast<int>(rem % hgroups);
  rem /= hgroups;
  const int kvh = static_cast<int>(rem % a.n_kv);
  const int bi = static_cast<int>(rem / a.n_kv);

  const int64_t wg_tok0 = tb * tok_per_wg;
  const int64_t wg_tok_last = min(wg_tok0 + tok_per_wg, a.s_q) - 1;
  const int h = kvh * g + hgi * HW + (wave % HW);
  const int64_t w_tok0 = wg_tok0 + (wave / HW) * QW;
  const int64_t w_tok_last = min(w_tok0 + QW, a.s_q) - 1;
  const bool wave_has_rows = w_tok0 < a.s_q;
  const int64_t tok = w_tok0 + col;
  const bool tok_ok = tok < a.s_q;

  // ---- key range of the workgroup (causal: keys up to its last position) ----
  // Non-causal: every valid key (position INT_MIN) is visible and keys past
  // the block (position INT_MAX) are not, so queries take INT_MAX - 1.
  int64_t nkeys = a.s_kv;
  int32_t w_qmin = INT_MAX - 1, w_qmax = INT_MAX - 1;
  if (a.causal) {
    nkeys = count_le(a.kv_pos, a.s_kv, a.q_pos[wg_tok_last]);
    if (wave_has_rows) {
      w_qmin = a.q_pos[w_tok0];
      w_qmax = a.q_pos[w_tok_last];
    }
  }
  const int ntiles = static_cast<int>((nkeys + BK - 1) / BK);

  // ---- this lane's query: B operand of S^T = K Q^T (8 bf16 per k-step) ----
  const uint16_t *qg = static_cast<const uint16_t *>(a.q);
  bf16x8 qreg[D / 16];
  {
    const int64_t qoff = ((bi * a.s_q + (tok_ok ? tok : 0)) * a.n_q + h) * D + hi * 8;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      u32x4 raw = tok_ok ? *reinterpret_cast<const u32x4 *>(qg + qoff + ds * 16) : u32x4{0, 0, 0, 0};
      qreg[ds] = __builtin_bit_cast(bf16x8, raw);
    }
  }
  const int32_t qpos = !a.causal ? INT_MAX - 1 : (tok_ok ? a.q_pos[tok] : INT_MIN);
  const float sl2 = a.scale * LOG2E;

  // ---- global -> register staging of one K/V tile ----
  // K: thread (chunk kc = tid % 16, rows kr + 16 j): 16 lanes read one 256-byte row.
  // V: thread (key quad vq = tid % 16, chunk vc = tid / 16): rows 4 vq + j, so the
  //    register transpose yields 4 consecutive keys of one d for an 8-byte LDS write.
  const int kc = tid & 15, kr = tid >> 4;
  const int vq = tid & 15, vc = tid >> 4;
  const uint16_t *kg = static_cast<const uint16_t *>(a.k);
  const uint16_t *vg = static_cast<const uint16_t *>(a.v);
  const int64_t kv_row_stride = static_cast<int64_t>(a.n_kv) * D;  // elements per token
  const int64_t kv_base = (static_cast<int64_t>(bi) * a.s_kv * a.n_kv + kvh) * D;
  u32x4 kst[4], vst[4];
  int32_t pst = 0;

  auto load_tile = [&](int t) {
    const int64_t key0 = static_cast<int64_t>(t) * BK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t key = key0 + kr + 16 * j;
      kst[j] = key < a.s_kv
                   ? *reinterpret_cast<const u32x4 *>(kg + kv_base + key * kv_row_stride + kc * 8)
                   : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t key = key0 + 4 * vq + j;
      vst[j] = key < a.s_kv
                   ? *reinterpret_cast<const u32x4 *>(vg + kv_base + key * kv_row_stride + vc * 8)
                   : u32x4{0, 0, 0, 0};
    }
    if (tid < BK) {
      const int64_t key = key0 + tid;
      pst = key >= a.s_kv ? INT_MAX : (a.causal ? a.kv_pos[key] : INT_MIN);
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4 *>(k_lds + (kr + 16 * j) * K_STRIDE + kc * 16) = kst[j];
    // Keys 4 vq .. 4 vq + 3 sit in a 16-key group; inside a group, position
    // (gg * 8 + hh * 4 + j) holds key (hh * 8 + gg * 4 + j), so the 8 keys an
    // MFMA lane needs for one k-step are contiguous.
    const int grp = vq >> 2, q4 = vq & 3;
    const int col_elem = grp * 16 + (q4 & 1) * 8 + (q4 >> 1) * 4;
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // dword w of each row = d pair (vc*8 + 2w, +1)
      const uint32_t x0 = vst[0][w], x1 = vst[1][w], x2 = vst[2][w], x3 = vst[3][w];
      const u32x2 even{(x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16)};
      const u32x2 odd{(x0 >> 16) | (x1 & 0xffff0000u), (x2 >> 16) | (x3 & 0xffff0000u)};
      const int d0 = vc * 8 + 2 * w;
      *reinterpret_cast<u32x2 *>(vt_lds + d0 * VT_STRIDE + col_elem * 2) = even;
      *reinterpret_cast<u32x2 *>(vt_lds + (d0 + 1) * VT_STRIDE + col_elem * 2) = odd;
    }
    if (tid < BK) pos_lds[tid] = pst;
  };

  // ---- running state: one query per lane ----
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;  // running max, in units of log2 (scaled scores)
  float l_run = 0.f;        // this lane's half of the running sum

  if (ntiles > 0) load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // every wave is done with the previous tile
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);

    const int64_t key0 = static_cast<int64_t>(t) * BK;
    const int32_t tile_pmin = pos_lds[0];
    const int32_t tile_pmax = pos_lds[BK - 1];
    // Tile entirely after this wave's last query: nothing visible.
    if (!wave_has_rows || tile_pmin > w_qmax) continue;
    const bool need_mask = key0 + BK > a.s_kv || tile_pmax > w_qmin;

    // S^T[key][query] = K Q^T; block kb covers keys kb*32 .. kb*32+31.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const unsigned char *krow = k_lds + (kb * 32 + col) * K_STRIDE + hi * 16;
#pragma unroll
      for (int ds = 0; ds < D / 16; ++ds) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(krow + ds * 32);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ds], s[kb], 0, 0, 0);
      }
    }
    // Accumulator element e of block kb is key kb*32 + (e/4)*8 + hi*4 + e%4.
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int32_t *pp = pos_lds + kb * 32 + e4 * 8 + hi * 4;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (pp[j] > qpos) s[kb][e4 * 4 + j] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m_run, mx * sl2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;

    // P (bf16) in the B-operand layout of O^T += V^T P^T: k-step ks covers
    // keys ks*16 .. ks*16+15 and uses accumulator elements (ks%2)*8 .. +7 of
    // block ks/2, i.e. keys {hi*4 + 0..3, 8 + hi*4 + 0..3} of the 16.
    bf16x8 pb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = exp2_fast(fmaf(s[ks >> 1][(ks & 1) * 8 + e], sl2, -m_use));
        l_run += p;
        pb[ks][e] = static_cast<__bf16>(p);
      }
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const unsigned char *vrow = vt_lds + (db * 32 + col) * VT_STRIDE + hi * 16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 va = *reinterpret_cast<const bf16x8 *>(vrow + ks * 32);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[ks], acc[db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: o_b = acc / l, lse_b = (m + log2 l) ln 2; optional merge ----
  const float l_tot = l_run + swap_halves(l_run);
  if (!tok_ok) return;
  const float lse_new = l_tot > 0.f ? (m_run + __log2f(l_tot)) * LN2 : -INFINITY;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t row = (bi * a.s_q + tok) * a.n_q + h;
  float w_old = 0.f, w_new = inv, lse_out = lse_new;
  if (a.merge) {
    const float lse_old = a.lse[row];
    const float m = fmaxf(lse_old, lse_new);
    if (m == -INFINITY) {
      w_new = 0.f;
      lse_out = -INFINITY;
    } else {
      lse_out = m + __logf(__expf(lse_old - m) + __expf(lse_new - m));
      w_old = __expf(lse_old - lse_out);
      w_new = __expf(lse_new - lse_out) * inv;
    }
  }
  float *orow = a.o + row * D + hi * 4;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      float4 *dst = reinterpret_cast<float4 *>(orow + db * 32 + e4 * 8);
      float4 r;
      r.x = w_new * acc[db][e4 * 4 + 0];
      r.y = w_new * acc[db][e4 * 4 + 1];
      r.z = w_new * acc[db][e4 * 4 + 2];
      r.w = w_new * acc[db][e4 * 4 + 3];
      if (a.merge) {
        const float4 old = *dst;
        r.x += w_old * old.x;
        r.y += w_old * old.y;
        r.z += w_old * old.z;
        r.w += w_old * old.w;
      }
      *dst = r;
    }
  if (hi == 0) a.lse[row] = lse_out;
}

template <int HW>
hipError_t launch_hw(const AttnArgs &a, hipStream_t stream) {
  constexpr int TB = WAVES / HW;
  const int64_t ntb = (a.s_q + TB * QW - 1) / (TB * QW);
  const int64_t blocks = ntb * a.b * a.n_kv * ((a.n_q / a.n_kv) / HW);
  if (blocks == 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  attn_bf16_kernel<HW><<<static_cast<unsigned>(blocks), THREADS, LDS_BYTES, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t stream) {
  const int g = a.n_q / a.n_kv;
  if (g % 4 == 0) return launch_hw<4>(a, stream);
  if (g % 2 == 0) return launch_hw<2>(a, stream);
  return launch_hw<1>(a, stream);
}

}  // namespace ra
