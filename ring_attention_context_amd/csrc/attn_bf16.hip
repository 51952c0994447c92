// bf16 block attention on gfx950 matrix cores.
//
// Computes, for the keys of one block, the statistics of "Context
// Parallelism and Ring Attention" §3: m_b = max x, l_b = sum e^{x - m_b},
// o_b = (1/l_b) sum e^{x - m_b} v, lse_b = m_b + ln l_b, scanning the block
// tile by tile with a running reference, running sum and unnormalised output
// (the single-GPU form of the same identity, §3). The causal rule of §5 is
// applied on original positions (§6 "the cost of reordering"); positions are
// non-decreasing, so tiles past a query tile's last position are never
// loaded (the tile skipping of §7), and only tiles that straddle the
// diagonal, or the ragged last tile, evaluate the element mask. With the
// document mask of §8 (all-gather CP) each query also carries the position
// where its document starts: the key range begins at the tile holding the
// first query's document start, and tiles that begin before a query's
// document start evaluate the element mask too.
//
// Work decomposition (d = 128):
//   * a wave owns 32 query tokens of one query head; a workgroup of 8 waves
//     owns TB = 8 / HW consecutive 32-token blocks of HW heads that share one
//     key/value head (GQA), so every K/V tile staged in LDS serves all eight
//     waves (two per SIMD);
//   * K/V tiles of 64 keys go from HBM straight into LDS (buffer loads with
//     the LDS destination, no register staging), K and V each through a ring
//     of four stages, one barrier per tile; out-of-range keys come back as
//     zeros from the buffer descriptor's bounds check. K is consumed a step
//     before V, so K is issued three tiles ahead and V two, and every load
//     has two steps to land: the barrier waits only for loads older than the
//     previous step's (a fence-free barrier; __syncthreads would drain all);
//   * K rows are row-major in LDS with the 16-byte chunks of each 256-byte row
//     XOR-swizzled by the row index, so the operand reads (ds_read_b128) are
//     bank-conflict free. V comes either row-major (read with the gfx950
//     transposing ds_read_b64_tr_b16) or already transposed, V^T [d, keys]
//     (VT = true; plain ds_read_b128 of 128-byte rows, swizzled the same way),
//     which moves a third of the LDS bytes per instruction of the former;
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: each lane then holds keys of ONE query, so
//     row reductions are in-lane plus one exchange with the lane 32 away
//     (v_permlane32_swap), and the probabilities convert in place into the B
//     operand of O^T = V^T P^T, whose accumulator keeps one query per lane.
//     With V^T the K rows are read in a permuted order (bits 2 and 3 of the
//     row swapped) so that each lane's probabilities are 8 consecutive keys,
//     the k-slots of one 16-byte V^T read;
//   * each tile runs in two phases: phase 1 issues the score MFMAs of tile
//     t+1 interleaved, k-step by k-step, with the exponentials of tile t;
//     phase 2 issues the P V MFMAs of tile t. Waves w and w+4 share a SIMD; the second group runs the two phases
//     in the opposite order (P V of tile t-1 first), so the pair overlaps one
//     wave's exponentials with the other's MFMAs. V of tile t-1 therefore
//     stays resident for that group while V of tile t+2 streams in;
//   * exponentials run in base 2 (v_exp_f32) with the scale folded into one
//     FMA. The reference of the exponentials is updated lazily from the tile
//     sum instead of a per-tile max: probabilities are formed against the
//     current reference, and when a row's tile sum exceeds 2^8 the reference
//     moves up by log2 of it, so later probabilities stay near 1. A tile is
//     redone with its true row max only when a row has no reference yet or
//     the sum leaves [0, 2^32] (a score far above the reference). The result
//     is exact for any reference (o = acc / l, lse = ref + log2 l) as long as
//     nothing overflows, which those bounds guarantee;
//   * two row sums: l over the fp32 probabilities gives lse, and l^ over the
//     bf16-rounded probabilities that enter P V (one v_dot2 per pair) divides
//     the accumulator, so o is a convex combination of V rows with exactly the
//     weights the MFMA used: a dominant key contributes its V row with no
//     rounding error, which matters for peaked rows.
// Workgroups are ordered heaviest query tile first (later positions see more
// keys under the causal rule); consecutive workgroups cover the KV heads of one
// token block, so with the round-robin dispatch over the 8 XCDs each XCD's L2
// serves a fixed KV head.
#include <climits>
#include <type_traits>

#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))
#define INLINE __attribute__((always_inline))

constexpr int D = 128;
constexpr int QW = 32;                       // query tokens per wave
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int BK = 64;                       // keys per tile
constexpr int ROW_B = D * 2;                 // bytes per key row
constexpr int VT_ROW_B = BK * 2;             // bytes per d-row of a V^T tile
constexpr int TILE_B = BK * ROW_B;           // 16 KiB
constexpr int NSTAGE = 4;
constexpr int LOADS_PER_WAVE = TILE_B / (1024 * WAVES);  // 1 KiB per wave instruction
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float TAU = 8.f;                   // lazy-rescale slack, log2 units
constexpr int BUF_DWORD3 = 0x00020000;       // raw buffer, 32-bit data format

static_assert(LOADS_PER_WAVE * 1024 * WAVES == TILE_B, "tile split over waves");

// 16-byte chunk swizzle of a 256-byte K row: a 4-bit rotation of the row index.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// 16-byte chunk swizzle of a 128-byte V^T row.
__device__ __forceinline__ int swz_vt(int r) { return (r >> 1) & 7; }
// K row read by lane column c when V is transposed: bits 2 and 3 swapped.
__device__ __forceinline__ int kperm(int c) { return (c & ~12) | ((c & 4) << 1) | ((c & 8) >> 1); }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum over the lane pair (l, l ^ 32), which holds the two key halves of a query.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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
// Number of keys with position < p.
__device__ __forceinline__ int64_t count_lt(const int32_t *kv_pos, int64_t n, int32_t p) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (kv_pos[mid] < p)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : static_cast<int32_t>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0), n,
                                           BUF_DWORD3);
}

// Waits until at most n (0..5) of this wave's HBM->LDS loads are still in
// flight: the n most recent ones (loads complete in order). Only vmcnt is
// waited on. A barrier after it publishes the older loads to all waves.
__device__ __forceinline__ void wait_loads_upto(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F75); break;
  }
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// also wait for every load still in flight). The empty asm statements keep
// the compiler from moving LDS accesses across it; LDS reads issued before it
// have been consumed, so they are complete.
__device__ __forceinline__ void barrier_keep_loads() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// DOC: a document mask is given (a.q_lo); without it the mask code compiles away.
template <int HW, bool VT, bool DOC>
__global__ __launch_bounds__(THREADS, 1) void attn_bf16_kernel(AttnArgs a) {
  // One LDS object per stage and operand (the key positions of a tile sit
  // after its K rows): the compiler then sees that the asynchronous loads into
  // one stage never alias the reads of the others and waits for exactly the
  // loads a read depends on. It tells at most eight such objects apart.
  __shared__ __attribute__((aligned(16))) unsigned char k_lds0[TILE_B + BK * 4],
      k_lds1[TILE_B + BK * 4], k_lds2[TILE_B + BK * 4], k_lds3[TILE_B + BK * 4];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds0[TILE_B], v_lds1[TILE_B],
      v_lds2[TILE_B], v_lds3[TILE_B];
  auto k_stage = [&](auto s) INLINE -> unsigned char * {
    constexpr int v = decltype(s)::value;
    return v == 0 ? k_lds0 : v == 1 ? k_lds1 : v == 2 ? k_lds2 : k_lds3;
  };
  auto v_stage = [&](auto s) INLINE -> unsigned char * {
    constexpr int v = decltype(s)::value;
    return v == 0 ? v_lds0 : v == 1 ? v_lds1 : v == 2 ? v_lds2 : v_lds3;
  };
  auto p_stage = [&](auto s) INLINE -> int32_t * {
    return reinterpret_cast<int32_t *>(k_stage(s) + TILE_B);
  };

  constexpr int TB = WAVES / HW;  // 32-token blocks per workgroup
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int lane = tid & 63;
  const int col = lane & 31;  // query within the wave
  const int hi = lane >> 5;   // which half of the MFMA k-slots this lane holds
  const bool grp_b = wave >= WAVES / 2;  // runs its tile phases in the opposite order

  // ---- workgroup -> (batch, kv head, head group, token block) ----
  const int g = a.n_q / a.n_kv;
  const int hgroups = g / HW;
  const int64_t tok_per_wg = TB * QW;
  const int64_t ntb = (a.s_q + tok_per_wg - 1) / tok_per_wg;
  const int64_t inner = static_cast<int64_t>(a.b) * a.n_kv * hgroups;
  const int64_t id = blockIdx.x;
  const int64_t tb = ntb - 1 - id / inner;  // heaviest (latest) token block first
  int64_t rem = id % inner;
  const int kvh = static_cast<int>(rem % a.n_kv);
  rem /= a.n_kv;
  const int hgi = static_cast<int>(rem % hgroups);
  const int bi = static_cast<int>(rem / hgroups);

  const int64_t wg_tok0 = tb * tok_per_wg;
  const int64_t wg_tok_last = min(wg_tok0 + tok_per_wg, a.s_q) - 1;
  const int h = kvh * g + hgi * HW + (wave % HW);
  const int64_t w_tok0 = wg_tok0 + (wave / HW) * QW;
  const int64_t w_tok_last = min(w_tok0 + QW, a.s_q) - 1;
  const bool wave_has_rows = w_tok0 < a.s_q;
  const int64_t tok = w_tok0 + col;
  const bool tok_ok = tok < a.s_q;

  // ---- key range of the workgroup (causal: keys up to its last position) ----
  // Non-causal: every key is visible, so a query takes position INT_MAX - 1
  // and the tile tests below never skip.
  // With a document mask the range starts at the tile holding the first key
  // of the first query's document (document starts are non-decreasing).
  int64_t nkeys = a.s_kv;
  int64_t kbeg = 0;
  int32_t w_qmin = INT_MAX - 1, w_qmax = INT_MAX - 1;
  int32_t w_lomax = INT_MIN;  // latest document start among the wave's queries
  if (a.causal) {
    nkeys = count_le(a.kv_pos, a.s_kv, a.q_pos[wg_tok_last]);
    if (DOC) kbeg = count_lt(a.kv_pos, a.s_kv, a.q_lo[wg_tok0]) / BK * BK;
    if (wave_has_rows) {
      w_qmin = a.q_pos[w_tok0];
      w_qmax = a.q_pos[w_tok_last];
      if (DOC) w_lomax = a.q_lo[w_tok_last];
    }
  }
  const int nt = nkeys > kbeg ? static_cast<int>((nkeys - kbeg + BK - 1) / BK) : 0;

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
  const int32_t qlo = DOC && tok_ok ? a.q_lo[tok] : INT_MIN;  // first visible key position
  const float sl2 = a.scale * LOG2E;

  // ---- per-lane LDS offsets of the MFMA operands (within one stage) ----
  // K: lane (col, hi) reads key row krow (+32 for the second key block),
  // logical chunk 2*ds + hi.
  const int krow = VT ? kperm(col) : col;
  uint32_t koff[D / 16];
#pragma unroll
  for (int ds = 0; ds < D / 16; ++ds)
    koff[ds] = krow * ROW_B + ((((2 * ds + hi) ^ swz(krow & 15))) << 4);
  // V^T operand of k-step ks: with V^T staged, lane (col, hi) reads d-row col
  // (+32 per d block), keys ks*16 + hi*8 .. +7. With V row-major, the
  // transposing read: in each 16-lane group gq, lane s reads 8 bytes of key
  // row r (4 rows per group) so that lane j of the group receives
  // V[k0 + 0..3][d0 + j]; call c covers keys {0..3, 8..11} + 4*(gq>>1) of a
  // 16-key step, matching the k-slots of P in the B operand.
  uint32_t voff[2][D / 32];
  if constexpr (VT) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) voff[0][ks] = col * VT_ROW_B + (((2 * ks + hi) ^ swz_vt(col)) << 4);
  } else {
    const int gq = lane >> 4, s = lane & 15;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int r = ((gq >> 1) << 2) + (s >> 2) + 8 * c;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int lc = db * 4 + ((gq & 1) << 1) + ((s & 3) >> 1);
        voff[c][db] = r * ROW_B + ((lc ^ swz(r)) << 4) + ((s & 1) << 3);
      }
    }
  }

  // ---- direct HBM -> LDS loads of one K/V tile (and its key positions) ----
  const unsigned char *kg = static_cast<const unsigned char *>(a.k);
  const unsigned char *vg = static_cast<const unsigned char *>(a.v);
  const int64_t kv_row_bytes = static_cast<int64_t>(a.n_kv) * D * 2;
  const int64_t kv_base = (static_cast<int64_t>(bi) * a.s_kv * a.n_kv + kvh) * D * 2;
  // V^T [b, n_kv, d, s_kv]: d-rows of s_kv keys.
  const int64_t vt_stride = a.s_kv * 2;
  const int64_t vt_base = (static_cast<int64_t>(bi) * a.n_kv + kvh) * D * vt_stride;
  uint32_t goff[LOADS_PER_WAVE], vgoff[LOADS_PER_WAVE];
#pragma unroll
  for (int i = 0; i < LOADS_PER_WAVE; ++i) {
    // K (and row-major V): 4 rows of 256 bytes per instruction.
    const int row = 4 * (wave + WAVES * i) + (lane >> 4);
    const int lc = (lane & 15) ^ swz(row & 15);
    goff[i] = static_cast<uint32_t>(row * kv_row_bytes + lc * 16);
    // V^T: 8 d-rows of 128 bytes per instruction.
    const int vrow = 8 * (wave + WAVES * i) + (lane >> 3);
    vgoff[i] = static_cast<uint32_t>(vrow * vt_stride + (((lane & 7) ^ swz_vt(vrow)) << 4));
  }
  // K rows (and key positions) of tile t into K stage `stage`: LOADS_PER_WAVE
  // loads per wave, plus one for wave 0 when causal.
  auto issue_k = [&](int t, auto stage) INLINE {
    const int64_t key0 = kbeg + static_cast<int64_t>(t) * BK;
    const int64_t left = a.s_kv - key0;  // rows before the end of the block
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + kv_base + key0 * kv_row_bytes,
                                                (left - 1) * kv_row_bytes + D * 2);
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (LDS_AS void *)(k_stage(stage) + 4 * (wave + WAVES * i) * ROW_B), 16, goff[i], 0, 0, 0);
    if (a.causal && wave == 0) {
      const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.kv_pos + key0, left * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (LDS_AS void *)p_stage(stage), 4, lane * 4,
                                               0, 0, 0);
    }
  };
  // V (or V^T) of tile t into V stage `stage`: LOADS_PER_WAVE loads per wave.
  auto issue_v = [&](int t, auto stage) INLINE {
    const int64_t key0 = kbeg + static_cast<int64_t>(t) * BK;
    const int64_t left = a.s_kv - key0;
    // V^T: keys past the block in a d-row read the next d-row's first keys
    // (finite values that meet a zero probability) or, for the last row,
    // zeros from the bounds check.
    const __amdgpu_buffer_rsrc_t rv =
        VT ? make_rsrc(vg + vt_base + key0 * 2, (D - 1) * vt_stride + left * 2)
           : make_rsrc(vg + kv_base + key0 * kv_row_bytes, (left - 1) * kv_row_bytes + D * 2);
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) {
      if constexpr (VT)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (LDS_AS void *)(v_stage(stage) + (wave + WAVES * i) * 1024), 16, vgoff[i], 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (LDS_AS void *)(v_stage(stage) + 4 * (wave + WAVES * i) * ROW_B), 16, goff[i], 0, 0, 0);
    }
  };
  const int nk = LOADS_PER_WAVE + (a.causal && wave == 0 ? 1 : 0);  // loads per issue_k
  constexpr int nv = LOADS_PER_WAVE;                                  // loads per issue_v

  // ---- running state: one query per lane ----
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;  // reference of the exponentials (log2 units)
  float l_run = 0.f;        // this lane's half of the running sum (fp32 probabilities)
  float lh_run = 0.f;       // ... of the bf16-rounded probabilities fed to P V
  float lt = 0.f;           // this lane's half of the current tile's sum
  float lht = 0.f;          // ... and of its bf16-rounded probabilities
  float alpha = 1.f;        // rescale factor pending for acc / l_run
  bool done = !wave_has_rows || nt == 0;
  bool pend = false;        // second group: P V of the previous tile still to do
  bool have_next = false;   // tile t+1 exists and is not entirely in the future
  bf16x8 pb[4];             // probabilities of the tile whose P V is next
  f32x16 sA[2], sB[2];      // scores of two consecutive tiles (roles alternate)

  auto tile_pos = [&](auto stage, int i) INLINE -> int32_t { return p_stage(stage)[i]; };
  // Whole tile after this wave's last query (causal): nothing visible here or later.
  auto tile_skip = [&](auto stage) INLINE -> bool { return a.causal && tile_pos(stage, 0) > w_qmax; };

  // Scores S^T = K Q^T of the K tile in `stage`.
  auto qk = [&](auto stage, f32x16 *s) INLINE {
    const unsigned char *kb_base = k_stage(stage);
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(kb_base + koff[ds] + kb * 32 * ROW_B);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ds], ds == 0 ? f32x16{} : s[kb], 0, 0, 0);
      }
  };

  // Element mask of a diagonal or ragged tile t held in `stage` (or one that
  // starts before a query's document). Accumulator element e4*4 + j of key
  // block kb holds key kk + j.
  auto mask = [&](int t, auto stage, f32x16 *s) INLINE {
    const int64_t key0 = kbeg + static_cast<int64_t>(t) * BK;
    const bool ragged = key0 + BK > a.s_kv;
    if (ragged || (a.causal && tile_pos(stage, BK - 1) > w_qmin) ||
        (DOC && tile_pos(stage, 0) < w_lomax)) {
      // Branch-free selects: key index past the block, position after the
      // query, or before the query's document.
      const int lim = ragged ? static_cast<int>(a.s_kv - key0) : BK;
      const int32_t *pp = p_stage(stage);
      const int32_t qp = a.causal ? qpos : INT_MAX;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int kk = VT ? kb * 32 + (e4 >> 1) * 16 + hi * 8 + (e4 & 1) * 4
                            : kb * 32 + e4 * 8 + hi * 4;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool out = (kk + j >= lim) | (pp[kk + j] > qp) | (pp[kk + j] < qlo);
            s[kb][e4 * 4 + j] = out ? -INFINITY : s[kb][e4 * 4 + j];
          }
        }
    }
  };

  // Row max of a tile (both key halves) in log2 units.
  auto rowmax = [&](const f32x16 *s) INLINE -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    return pair_max(mx) * sl2;
  };

  auto apply_rescale = [&]() INLINE {
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
      l_run *= alpha;
      lh_run *= alpha;
      alpha = 1.f;
    }
  };

  // P = 2^(S * scale * log2 e - ref) as the bf16 B operand of O^T += V^T P^T:
  // k-step ks covers keys ks*16 .. ks*16+15 and uses accumulator elements
  // (ks%2)*8 .. +7 of block ks/2. The tile sum uses the fp32 probabilities
  // (before bf16 rounding), so lse carries no bf16 error; four partial sums
  // keep the dependency chains short.
  auto softmax = [&](const f32x16 *s) INLINE {
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float lp[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = exp2_fast(fmaf(s[ks >> 1][(ks & 1) * 8 + e], sl2, -m_use));
        if (ks == 0 && e < 4)
          lp[e] = p;
        else
          lp[e & 3] += p;
        pb[ks][e] = static_cast<__bf16>(p);
      }
    }
    lt = (lp[0] + lp[1]) + (lp[2] + lp[3]);
    const bf16x2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
    float lh[2] = {0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        lh[e >> 2] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[ks][e], pb[ks][e + 1]}, one,
                                                     lh[e >> 2], false);
    lht = lh[0] + lh[1];
  };

  // Phase-1 body: the score MFMAs of the next tile interleaved with the
  // probabilities of the current one, one k-step at a time behind hard
  // scheduling fences (left to itself the compiler clusters the MFMAs and the
  // VALU work apart). Each k-step issues the K reads two steps ahead, the two
  // score MFMAs, then a quarter of one key block's probabilities (4 per
  // lane), which the VALU works through while the MFMAs run.
  auto qk_softmax = [&](auto stage, f32x16 *s, const f32x16 *cur) INLINE {
    const unsigned char *kb_base = k_stage(stage);
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    bf16x8 ka[3][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        ka[j][kb] = *reinterpret_cast<const bf16x8 *>(kb_base + koff[j] + kb * 32 * ROW_B);
    float lp[4] = {0.f, 0.f, 0.f, 0.f};
    float lh[2] = {0.f, 0.f};
    const bf16x2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
      if (ds + 2 < D / 16) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          ka[(ds + 2) % 3][kb] =
              *reinterpret_cast<const bf16x8 *>(kb_base + koff[ds + 2] + kb * 32 * ROW_B);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ds % 3][kb], qreg[ds],
                                                        ds == 0 ? f32x16{} : s[kb], 0, 0, 0);
      // probabilities of k-slots ks = ds / 2, e = (ds % 2) * 4 .. +3
      const int ks = ds >> 1, e0 = (ds & 1) * 4;
      float pf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pf[j] = exp2_fast(fmaf(cur[ks >> 1][(ks & 1) * 8 + e0 + j], sl2, -m_use));
        lp[j] += pf[j];
        pb[ks][e0 + j] = static_cast<__bf16>(pf[j]);
      }
#pragma unroll
      for (int j = 0; j < 4; j += 2)
        lh[j >> 1] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[ks][e0 + j], pb[ks][e0 + j + 1]},
                                                     one, lh[j >> 1], false);
      __builtin_amdgcn_sched_barrier(0);
    }
    lt = (lp[0] + lp[1]) + (lp[2] + lp[3]);
    lht = lh[0] + lh[1];
  };

  // O^T += V^T P^T with the V tile in `stage`. The V operand of MFMA i is read
  // two MFMAs ahead behind scheduling fences; left to itself the compiler
  // waits for each read right before its MFMA.
  auto pv = [&](auto stage) INLINE {
    const unsigned char *vb = v_stage(stage);
    constexpr int NDB = D / 32;  // d blocks per k-step
    auto rd = [&](int i) INLINE -> bf16x8 {
      const int ks = i / NDB, db = i % NDB;
      if constexpr (VT) {
        return *reinterpret_cast<const bf16x8 *>(vb + voff[0][ks] + db * 32 * VT_ROW_B);
      } else {
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4 *)(vb + voff[0][db] + ks * 16 * ROW_B));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4 *)(vb + voff[1][db] + ks * 16 * ROW_B));
        return bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      }
    };
    bf16x8 va[3];
    va[0] = rd(0);
    va[1] = rd(1);
#pragma unroll
    for (int i = 0; i < 4 * NDB; ++i) {
      if (i + 2 < 4 * NDB) va[(i + 2) % 3] = rd(i + 2);
      acc[i % NDB] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % 3], pb[i / NDB], acc[i % NDB], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Phase 1 of tile t: scores of tile t+1 (K in stage `sn`) on the matrix
  // cores, probabilities of tile t (scores in `cur`) on the VALU.
  auto phase1 = [&](int t, auto sn, const f32x16 *cur, f32x16 *nxt) INLINE {
    apply_rescale();
    have_next = t + 1 < nt && !tile_skip(sn);
    qk_softmax(sn, nxt, cur);
    const float lt_row = pair_sum(lt);
    if (__any((m_run == -INFINITY) | !(lt_row <= 0x1p32f))) {
      // No reference yet, or a score far above it: redo the tile against its
      // true row max (rescaling what is accumulated so far).
      const float m_new = fmaxf(m_run, rowmax(cur));
      const float al = (m_run == -INFINITY || m_new == -INFINITY) ? 1.f : exp2_fast(m_run - m_new);
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= al;
      l_run *= al;
      lh_run *= al;
      m_run = m_new;
      softmax(cur);
    }
    l_run += lt;
    lh_run += lht;
  };

  // Phase 2 of tile t: P V with V in stage `sc`; mask of tile t+1 (positions in
  // stage `sn`); lazy reference update from tile t's sum.
  auto phase2 = [&](int t, auto sc, auto sn, f32x16 *nxt) INLINE {
    if (have_next) mask(t + 1, sn, nxt);
    pv(sc);
    const float lt_row = pair_sum(lt);
    const bool need = lt_row > 0x1p8f;  // 2^TAU
    const float lg = __builtin_amdgcn_logf(lt_row);  // log2
    alpha = need ? exp2_fast(-lg) : 1.f;
    m_run = need ? m_run + lg : m_run;
    done = !have_next;
  };

  // ---- prologue: tiles 0 and 1 in flight; reference from tile 0's row max ----
  using St0 = std::integral_constant<int, 0>;
  using St1 = std::integral_constant<int, 1>;
  using St2 = std::integral_constant<int, 2>;
  using St3 = std::integral_constant<int, 3>;
  // Step t issues K of tile t+3 and V of tile t+2 and needs everything issued
  // up to step t-2, so each load has two steps to land. The prologue issues
  // what steps -3 .. -1 would have: K0; K1, V0; K2, V1. Loads are issued
  // unconditionally (a tile past the range reads zeros, or keys that are
  // never used, into a free stage): the compiler's own waits before LDS reads
  // then count the loads that follow exactly instead of assuming none did.
  const int n_step = nk + nv;  // loads this wave issues per step
  issue_k(0, St0{});
  issue_k(1, St1{});
  issue_v(0, St0{});
  wait_loads_upto(n_step);  // K0 has landed
  barrier_keep_loads();
  issue_k(2, St2{});
  issue_v(1, St1{});
  if (!done && tile_skip(St0{})) done = true;
  if (!done) {
    qk(St0{}, sA);
    mask(0, St0{}, sA);
    m_run = rowmax(sA);
  }
  static_assert(TAU == 8.f, "phase2 compares against 2^TAU");

  // ---- main loop: step t = 0 .. nt (step nt only finishes the second group's
  // last P V). Tile t lives in K and V stage t % 4; its scores are in sA (t
  // even) or sB.
  auto step = [&](auto stage_c, int t) INLINE {
    constexpr int S = decltype(stage_c)::value;
    using SC = std::integral_constant<int, S>;
    using SN = std::integral_constant<int, (S + 1) % NSTAGE>;
    using SP = std::integral_constant<int, (S + NSTAGE - 1) % NSTAGE>;
    using SL = std::integral_constant<int, (S + 2) % NSTAGE>;
    f32x16 *cur = (S & 1) == 0 ? sA : sB;
    f32x16 *nxt = (S & 1) == 0 ? sB : sA;
    // This wave's loads up to step t-2 (K and positions of tile t+1, V of
    // tile t) have landed, and after the barrier everyone's; every wave is done
    // with step t-1, so K stage t-1 and V stage t-2 are free.
    wait_loads_upto(n_step);
    barrier_keep_loads();
    issue_k(t + 3, SP{});
    issue_v(t + 2, SL{});
    if (grp_b && pend) {
      phase2(t - 1, SP{}, SC{}, cur);  // scores of tile t are in `cur`
      pend = false;
    }
    if (!done && t < nt) {
      phase1(t, SN{}, cur, nxt);
      if (grp_b)
        pend = true;
      else
        phase2(t, SC{}, SN{}, nxt);
    }
  };
  // The body always runs all four steps (steps past nt only wait, synchronise
  // and issue loads past the range), so the loads issued between two LDS reads
  // are the same on every path through the loop.
  for (int t = 0; t <= nt; t += NSTAGE) {
    step(St0{}, t);
    step(St1{}, t + 1);
    step(St2{}, t + 2);
    step(St3{}, t + 3);
  }
  wait_loads_upto(0);  // the loads past the range have landed before the wave ends
  apply_rescale();

  // ---- epilogue: o_b = acc / l^, lse_b = (ref + log2 l) ln 2; optional merge ----
  const float l_tot = pair_sum(l_run);
  const float lh_tot = pair_sum(lh_run);
  if (!tok_ok) return;
  const float lse_new = l_tot > 0.f ? (m_run + __log2f(l_tot)) * LN2 : -INFINITY;
  const float inv = l_tot > 0.f && lh_tot > 0.f ? 1.f / lh_tot : 0.f;
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
  // Accumulator element e4*4 + j of block db holds d = db*32 + e4*8 + hi*4 + j.
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

template <int HW, bool VT>
hipError_t launch_hw(const AttnArgs &a, hipStream_t stream) {
  constexpr int TB = WAVES / HW;
  const int64_t ntb = (a.s_q + TB * QW - 1) / (TB * QW);
  const int64_t blocks = ntb * a.b * a.n_kv * ((a.n_q / a.n_kv) / HW);
  if (blocks == 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (a.q_lo)
    attn_bf16_kernel<HW, VT, true><<<static_cast<unsigned>(blocks), THREADS, 0, stream>>>(a);
  else
    attn_bf16_kernel<HW, VT, false><<<static_cast<unsigned>(blocks), THREADS, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool VT>
hipError_t launch_vt(const AttnArgs &a, hipStream_t stream) {
  const int g = a.n_q / a.n_kv;
  if (g % 8 == 0) return launch_hw<8, VT>(a, stream);
  if (g % 4 == 0) return launch_hw<4, VT>(a, stream);
  if (g % 2 == 0) return launch_hw<2, VT>(a, stream);
  return launch_hw<1, VT>(a, stream);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs &a, hipStream_t stream) {
  return a.v_layout == RA_V_TRANSPOSED ? launch_vt<true>(a, stream) : launch_vt<false>(a, stream);
}

}  // namespace ra
