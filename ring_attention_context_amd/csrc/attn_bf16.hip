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
//     zeros from the buffer descriptor's bounds check. Step t loads tile t+3
//     into the stages tile t-1 left, so every load has two steps to land:
//     the barrier waits only for loads older than the previous step's (a
//     fence-free barrier; __syncthreads would drain all of them). The K
//     stage of tile t-1 is free a step before its V stage, so each wave
//     issues the K rows before the step's barrier, where it would otherwise
//     wait, and only the V rows after it;
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
//   * each step has a matrix phase, the score MFMAs of tile t+1 interleaved
//     with the P V MFMAs of tile t (operands read a few MFMAs ahead), and a
//     vector phase, the probabilities of the tile whose scores are at hand.
//     Waves w and w+4 share a SIMD and run the phases in opposite orders
//     (matrix then vector, vector then matrix), so one wave's exponentials
//     overlap the other's MFMAs; the matrix phase runs at raised priority.
//     The per-wave tile counts come from the key positions up front (64-lane
//     searches), so no LDS read decides a branch;
//   * exponentials run in base 2 (v_exp_f32) with the scale folded into one
//     FMA. The reference of the exponentials is updated lazily from the tile
//     sum instead of a per-tile max: probabilities are formed against the
//     current reference, and when a row's tile sum exceeds 2^8 the reference
//     moves up by log2 of it, so later probabilities stay near 1. A tile is
//     redone with its true row max only when a row has no reference yet or
//     the sum leaves [0, 2^32] (a score far above the reference). The result
//     is exact for any reference (o = acc / l, lse = ref + log2 l) as long as
//     nothing overflows, which those bounds guarantee. Each lane first tests
//     its own half of the row sum: while every half is at most 2^7 the row
//     sums are at most 2^8 and the tile needs neither, so the row sums (a
//     cross-lane exchange) and the logarithm are formed only on the rare
//     tiles where some half exceeds it;
//   * two row sums: l over the fp32 probabilities gives lse, and l^ over the
//     bf16-rounded probabilities that enter P V divides the accumulator, so o
//     is a convex combination of V rows with exactly the weights the MFMA
//     used: a dominant key contributes its V row with no rounding error, which
//     matters for peaked rows. l^ is formed on the matrix pipe by
//     v_mfma_f32_4x4x4_16b_bf16 against a ones operand (each lane's own four
//     values summed into element lane % 4 of its accumulator), eight per tile
//     beside the P V MFMAs: the VALU's v_dot2 executes on the matrix pipe as
//     well and cannot issue while another wave's MFMAs run, so one v_dot2 per
//     pair stalled the vector phase of the other wave;
//   * K / V loads use one buffer descriptor per operand for the workgroup's
//     whole key range when every offset fits in 31 bits; a tile adds its
//     offset to each lane's offset, so the loads after the barrier need no
//     scalar descriptor arithmetic.
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
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
constexpr int NDB = D / 32;                  // 32-wide d blocks of the output
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

// Number of keys with position <= p (LE) or < p in the non-decreasing
// kv_pos[0, n), found by the 64 lanes of a wave together: each round probes 64
// evenly spaced keys of the remaining range and keeps the gap between the
// last probe that counts and the first that does not, so a range of n keys
// takes about log64(n) dependent loads instead of the log2(n) of a binary
// search. Call with all lanes active; the result is uniform.
template <bool LE>
__device__ __forceinline__ int64_t wave_count(const int32_t *kv_pos, int64_t n, int32_t p, int lane) {
  int64_t lo = 0, hi = n;  // the count lies in [lo, hi]
  while (lo < hi) {
    const int64_t step = (hi - lo + 63) / 64;
    const int64_t idx = lo + lane * step;
    bool in = false;
    if (idx < hi) {
      const int32_t v = kv_pos[idx];
      in = LE ? v <= p : v < p;
    }
    const int cnt = __popcll(__ballot(in));  // the probes that count form a prefix
    const int64_t new_hi = min(hi, lo + cnt * step);
    lo = cnt == 0 ? lo : lo + (cnt - 1) * step + 1;
    hi = new_hi;
  }
  return lo;
}

// K independent counts of the same kind as wave_count (search k: keys of the
// non-decreasing arr[k][0, n) with position <= p[k], or < p[k] when lt[k]),
// advanced together: each round issues every active search's probe load
// before any is used, so the K searches cost the memory latency of one.
template <int K>
__device__ __forceinline__ void wave_counts(const int32_t *const (&arr)[K], int64_t n,
                                            const int32_t (&p)[K], const bool (&lt)[K],
                                            int64_t (&cnt)[K], int lane) {
  int64_t lo[K], hi[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    lo[k] = 0;
    hi[k] = n;
  }
  while (true) {
    bool active = false;
#pragma unroll
    for (int k = 0; k < K; ++k) active |= lo[k] < hi[k];
    if (!active) break;
    int64_t step[K], idx[K];
    int32_t v[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      step[k] = (hi[k] - lo[k] + 63) / 64;
      idx[k] = lo[k] + lane * step[k];
      v[k] = lo[k] < hi[k] && idx[k] < hi[k] ? arr[k][idx[k]] : 0;
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (lo[k] >= hi[k]) continue;
      const bool in = idx[k] < hi[k] && (lt[k] ? v[k] < p[k] : v[k] <= p[k]);
      const int c = __popcll(__ballot(in));
      const int64_t new_hi = min(hi[k], lo[k] + c * step[k]);
      lo[k] = c == 0 ? lo[k] : lo[k] + (c - 1) * step[k] + 1;
      hi[k] = new_hi;
    }
  }
#pragma unroll
  for (int k = 0; k < K; ++k) cnt[k] = lo[k];
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : static_cast<int32_t>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0), n,
                                           BUF_DWORD3);
}

// Waits until at most n (0..7) of this wave's HBM->LDS loads are still in
// flight: the n most recent ones (loads complete in order). Only vmcnt is
// waited on. A barrier after it publishes the older loads to all waves.
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
    default: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
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
// NEAR: the launcher has checked that every offset of the key range fits in 31 bits.
// PAIR: a second key block (a.k2, a.v2, a.kv_pos2, same length) follows the
// first: its tiles come after the first block's in the same scan, so the
// statistics of both blocks form in one pass and are merged (or written) once.
template <int HW, bool VT, bool DOC, bool NEAR, bool PAIR>
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
  // All the counts below come from one joint search (wave_counts): the
  // workgroup's range, then the wave's (c_hi: keys not after its last query,
  // c_lo: not after its first; c_d: before its latest document start), for
  // the second block too with PAIR. A wave without rows searches with the
  // workgroup's last query (its results are not used).
  int64_t nkeys = a.s_kv, nkeys2 = PAIR ? a.s_kv : 0;
  int64_t kbeg = 0;
  int32_t w_qmin = INT_MAX - 1, w_qmax = INT_MAX - 1;
  int32_t w_lomax = INT_MIN;  // latest document start among the wave's queries
  int64_t c_hi = 0, c_lo = 0, c_d = 0, c_hi2 = 0, c_lo2 = 0;
  if (a.causal) {
    const int32_t p_last = a.q_pos[wg_tok_last];
    w_qmin = wave_has_rows ? a.q_pos[w_tok0] : p_last;
    w_qmax = wave_has_rows ? a.q_pos[w_tok_last] : p_last;
    if constexpr (DOC) {
      w_lomax = a.q_lo[wave_has_rows ? w_tok_last : wg_tok_last];
      int64_t c[5];
      wave_counts<5>({a.kv_pos, a.kv_pos, a.kv_pos, a.kv_pos, a.kv_pos}, a.s_kv,
                     {p_last, a.q_lo[wg_tok0], w_qmax, w_qmin, w_lomax},
                     {false, true, false, false, true}, c, lane);
      nkeys = c[0];
      kbeg = c[1] / BK * BK;
      c_hi = c[2];
      c_lo = c[3];
      c_d = c[4];
    } else if constexpr (PAIR) {
      int64_t c[6];
      wave_counts<6>({a.kv_pos, a.kv_pos, a.kv_pos, a.kv_pos2, a.kv_pos2, a.kv_pos2}, a.s_kv,
                     {p_last, w_qmax, w_qmin, p_last, w_qmax, w_qmin},
                     {false, false, false, false, false, false}, c, lane);
      nkeys = c[0];
      c_hi = c[1];
      c_lo = c[2];
      nkeys2 = c[3];
      c_hi2 = c[4];
      c_lo2 = c[5];
    } else {
      int64_t c[3];
      wave_counts<3>({a.kv_pos, a.kv_pos, a.kv_pos}, a.s_kv, {p_last, w_qmax, w_qmin},
                     {false, false, false}, c, lane);
      nkeys = c[0];
      c_hi = c[1];
      c_lo = c[2];
    }
    if (!wave_has_rows) {
      w_qmin = INT_MAX - 1;
      w_qmax = INT_MAX - 1;
      w_lomax = INT_MIN;
    }
  }
  // nt1 tiles of the first block, then (PAIR) nt2 of the second.
  const int nt1 = nkeys > kbeg ? static_cast<int>((nkeys - kbeg + BK - 1) / BK) : 0;
  const int nt2 = PAIR ? static_cast<int>((nkeys2 + BK - 1) / BK) : 0;
  const int nt = nt1 + nt2;
  // Merging a block that no query of the workgroup can see leaves (o, lse) as
  // they are (its statistics are the merge identity): nothing to load or write.
  // nt is the same for every wave, so the whole workgroup leaves together.
  if (a.merge && nt == 0) return;
  // Tiles of this wave, from the same counts (positions are non-decreasing):
  // w_nt tiles hold a key not after its last query; tiles from j_diag on hold
  // a key after its first query, and tiles before j_doc a key before its
  // latest document start. Those (and a ragged last tile) take the element
  // mask.
  // PAIR: the wave's own range ends w_nt1 tiles into the first block (tiles
  // w_nt1 .. nt1-1 of the first block are masked whole for it) and w_nt2
  // tiles into the second, whose diagonal starts at tile j_diag2.
  int w_nt = nt, j_diag = INT_MAX, j_doc = 0;
  int w_nt1 = nt1, j_diag2 = INT_MAX;
  if (a.causal && wave_has_rows) {
    w_nt1 = c_hi > kbeg ? min(nt1, static_cast<int>((c_hi - kbeg + BK - 1) / BK)) : 0;
    w_nt = w_nt1;
    j_diag = c_lo > kbeg ? static_cast<int>((c_lo - kbeg) / BK) : 0;
    if (DOC) j_doc = c_d > kbeg ? static_cast<int>((c_d - kbeg + BK - 1) / BK) : 0;
    if (PAIR) {
      const int w_nt2 = min(nt2, static_cast<int>((c_hi2 + BK - 1) / BK));
      if (w_nt2 > 0) w_nt = nt1 + w_nt2;
      j_diag2 = static_cast<int>(c_lo2 / BK);
    }
  }

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
  // The swizzle is an XOR of the chunk index, so the offset of k-step ds is
  // that of k-step 0 with bits 5..7 XORed by ds: one register instead of
  // eight (kept live through the loop by `pin`, which stops the compiler from
  // hoisting the eight XORs back out).
  const int krow = VT ? kperm(col) : col;
  uint32_t koff0 = krow * ROW_B + (((hi ^ swz(krow & 15))) << 4);
  auto koff = [&](int ds) INLINE -> uint32_t { return koff0 ^ (static_cast<uint32_t>(ds) << 5); };
  // V^T operand of k-step ks: with V^T staged, lane (col, hi) reads d-row col
  // (+32 per d block), keys ks*16 + hi*8 .. +7. With V row-major, the
  // transposing read: in each 16-lane group gq, lane s reads 8 bytes of key
  // row r (4 rows per group) so that lane j of the group receives
  // V[k0 + 0..3][d0 + j]; call c covers keys {0..3, 8..11} + 4*(gq>>1) of a
  // 16-key step, matching the k-slots of P in the B operand.
  // With V^T the offset of k-step ks is that of k-step 0 with bits 5..6
  // XORed by ks, as for K.
  uint32_t voff[2][D / 32];
  uint32_t voff0 = col * VT_ROW_B + ((hi ^ swz_vt(col)) << 4);
  auto voff_vt = [&](int ks) INLINE -> uint32_t { return voff0 ^ (static_cast<uint32_t>(ks) << 5); };
  if constexpr (VT) {
    (void)voff;
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
  // NEAR (every byte offset of the key range fits in 31 bits): one buffer
  // descriptor per operand covers the workgroup's whole key range and stays in
  // scalar registers through the loop; tile t adds its offset to each lane's.
  // Keys past the block still fall outside the descriptor and read as zeros.
  // Otherwise each tile gets a descriptor of its own.
  const int64_t rows_left = a.s_kv - kbeg;
  const __amdgpu_buffer_rsrc_t rk_all = make_rsrc(
      kg + kv_base + kbeg * kv_row_bytes, rows_left > 0 ? (rows_left - 1) * kv_row_bytes + D * 2 : 0);
  const __amdgpu_buffer_rsrc_t rv_all =
      VT ? make_rsrc(vg + vt_base + kbeg * 2, rows_left > 0 ? (D - 1) * vt_stride + rows_left * 2 : 0)
         : make_rsrc(vg + kv_base + kbeg * kv_row_bytes,
                     rows_left > 0 ? (rows_left - 1) * kv_row_bytes + D * 2 : 0);
  const __amdgpu_buffer_rsrc_t rp_all = make_rsrc(a.kv_pos + kbeg, rows_left * 4);
  // PAIR: the second block's descriptors (the key range starts at 0 there).
  const unsigned char *kg2 = static_cast<const unsigned char *>(a.k2);
  const unsigned char *vg2 = static_cast<const unsigned char *>(a.v2);
  const int64_t all2 = PAIR ? a.s_kv : 0;
  const __amdgpu_buffer_rsrc_t rk_all2 =
      make_rsrc(PAIR ? kg2 + kv_base : kg, all2 > 0 ? (all2 - 1) * kv_row_bytes + D * 2 : 0);
  const __amdgpu_buffer_rsrc_t rv_all2 =
      make_rsrc(PAIR ? vg2 + vt_base : vg, all2 > 0 ? (D - 1) * vt_stride + all2 * 2 : 0);
  const __amdgpu_buffer_rsrc_t rp_all2 = make_rsrc(PAIR ? a.kv_pos2 : a.kv_pos, all2 * 4);
  // Tile t of the scan: the block it lies in (second when t >= nt1) and its
  // index there. Tiles past the scan fall past the second block's end.
  auto second = [&](int t) INLINE -> bool { return PAIR && t >= nt1; };
  auto local = [&](int t) INLINE -> int { return second(t) ? t - nt1 : t; };
  const uint32_t k_tile_b = static_cast<uint32_t>(BK * kv_row_bytes);
  auto issue_k = [&](int t, auto stage) INLINE {
    if constexpr (NEAR) {
      const bool sb = second(t);
      const uint32_t lt = static_cast<uint32_t>(local(t));
      const uint32_t toff = lt * k_tile_b;
      const __amdgpu_buffer_rsrc_t rk = sb ? rk_all2 : rk_all;
#pragma unroll
      for (int i = 0; i < LOADS_PER_WAVE; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (LDS_AS void *)(k_stage(stage) + 4 * (wave + WAVES * i) * ROW_B), 16,
            goff[i] + toff, 0, 0, 0);
      if (a.causal && wave == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sb ? rp_all2 : rp_all, (LDS_AS void *)p_stage(stage), 4,
                                                 lane * 4 + lt * (BK * 4), 0, 0, 0);
      return;
    }
    const bool sb = second(t);
    const int64_t key0 = (sb ? 0 : kbeg) + static_cast<int64_t>(local(t)) * BK;
    const int64_t left = a.s_kv - key0;  // rows before the end of the block
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((sb ? kg2 : kg) + kv_base + key0 * kv_row_bytes,
                                                (left - 1) * kv_row_bytes + D * 2);
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (LDS_AS void *)(k_stage(stage) + 4 * (wave + WAVES * i) * ROW_B), 16, goff[i], 0, 0, 0);
    if (a.causal && wave == 0) {
      const __amdgpu_buffer_rsrc_t rp = make_rsrc((sb ? a.kv_pos2 : a.kv_pos) + key0, left * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, (LDS_AS void *)p_stage(stage), 4, lane * 4,
                                               0, 0, 0);
    }
  };
  // V (or V^T) of tile t into V stage `stage`: LOADS_PER_WAVE loads per wave.
  auto issue_v = [&](int t, auto stage) INLINE {
    if constexpr (NEAR) {
      const uint32_t lt = static_cast<uint32_t>(local(t));
      const __amdgpu_buffer_rsrc_t rv = second(t) ? rv_all2 : rv_all;
#pragma unroll
      for (int i = 0; i < LOADS_PER_WAVE; ++i) {
        if constexpr (VT)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rv, (LDS_AS void *)(v_stage(stage) + (wave + WAVES * i) * 1024), 16,
              vgoff[i] + lt * (BK * 2), 0, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rv, (LDS_AS void *)(v_stage(stage) + 4 * (wave + WAVES * i) * ROW_B), 16,
              goff[i] + lt * k_tile_b, 0, 0, 0);
      }
      return;
    }
    const bool sb = second(t);
    const int64_t key0 = (sb ? 0 : kbeg) + static_cast<int64_t>(local(t)) * BK;
    const int64_t left = a.s_kv - key0;
    const unsigned char *vgb = sb ? vg2 : vg;
    // V^T: keys past the block in a d-row read the next d-row's first keys
    // (finite values that meet a zero probability) or, for the last row,
    // zeros from the bounds check.
    const __amdgpu_buffer_rsrc_t rv =
        VT ? make_rsrc(vgb + vt_base + key0 * 2, (D - 1) * vt_stride + left * 2)
           : make_rsrc(vgb + kv_base + key0 * kv_row_bytes, (left - 1) * kv_row_bytes + D * 2);
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
  float lt = 0.f;           // this lane's half of the current tile's sum
  // bf16 sums by 4x4x4 MFMAs (B = ones): lane l's own sum sits in element
  // l % 4, the other elements are other lanes' sums scaled by this lane's
  // factors and are never read.
  f32x4 lh4 = {};
  const bf16x4 ones4 = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f),
                        static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  float alpha = 1.f;        // rescale factor pending for acc / l_run
  bool pend = false;        // some lane has alpha != 1 (wave-uniform)
  float m_use = 0.f;        // m_run, or 0 while it is -inf (the exponentials' offset)
  bool done = !wave_has_rows || w_nt == 0;
  bf16x8 pb[4];             // probabilities of the tile whose P V is next
  f32x16 s[2];              // scores of the tile whose probabilities are next

  // Scores S^T = K Q^T of the K tile in `stage`.
  auto qk = [&](auto stage) INLINE {
    const unsigned char *kb_base = k_stage(stage);
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(kb_base + koff(ds) + kb * 32 * ROW_B);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ds], ds == 0 ? f32x16{} : s[kb], 0, 0, 0);
      }
  };

  // Element mask of tile t (positions in `stage`) when it straddles the
  // wave's diagonal, starts before a query's document, or is the ragged last
  // tile. Accumulator element e4*4 + j of key block kb holds key kk + j.
  auto mask = [&](int t, auto stage) INLINE {
    const bool sb = second(t);
    const int lt = local(t);
    const int64_t key0 = (sb ? 0 : kbeg) + static_cast<int64_t>(lt) * BK;
    const bool ragged = key0 + BK > a.s_kv;
    // PAIR: a first-block tile past the wave's own range is masked whole.
    const bool dead = PAIR && !sb && t >= w_nt1;
    if (ragged || dead || lt >= (sb ? j_diag2 : j_diag) || (DOC && t < j_doc)) {
      // Branch-free selects: key index past the block, position after the
      // query, or before the query's document.
      const int lim = dead ? 0 : ragged ? static_cast<int>(a.s_kv - key0) : BK;
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

  // Row max of the scores (both key halves) in log2 units.
  auto rowmax = [&]() INLINE -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    return pair_max(mx) * sl2;
  };

  auto apply_rescale = [&]() INLINE {
    if (pend) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
      l_run *= alpha;
      lh4 *= alpha;
      alpha = 1.f;
      pend = false;
    }
  };

  // P = 2^(S * scale * log2 e - ref) as the bf16 B operand of O^T += V^T P^T:
  // k-step ks covers keys ks*16 .. ks*16+15 and uses accumulator elements
  // (ks%2)*8 .. +7 of block ks/2. The tile sum uses the fp32 probabilities
  // (before bf16 rounding), so lse carries no bf16 error; four partial sums
  // keep the dependency chains short.
  auto softmax = [&]() INLINE {
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
      // Convert each k-step's probabilities as they are made, so that at most
      // one k-step of fp32 probabilities is live (the compiler would
      // otherwise compute all 32 first).
      asm volatile("" : "+v"(pb[ks]));
    }
    lt = (lp[0] + lp[1]) + (lp[2] + lp[3]);
    asm volatile("" : "+v"(lt));
  };

  // Matrix phase of step t: the score MFMAs of tile t+1 (K in stage `sn`)
  // interleaved with the P V MFMAs of tile t (V in stage `sc`). Operands are
  // read DIST MFMAs ahead behind scheduling fences; left to itself the
  // compiler waits for each read right before its MFMA.
  auto xphase = [&](auto sn, auto sc) INLINE {
    constexpr int NPV = 4 * NDB;          // P V MFMAs: 4 k-steps x NDB d blocks
    constexpr int N = 2 * NPV;            // the score MFMAs are as many
    constexpr int DIST = 4;
    const unsigned char *kbase = k_stage(sn);
    const unsigned char *vb = v_stage(sc);
    // Sequence slot i: even slots are score MFMA i/2 (k-step i/4, key block
    // (i/2)%2), odd slots P V MFMA i/2 (k-step i/2/NDB, d block i/2%NDB).
    auto rd = [&](int i) INLINE -> bf16x8 {
      if ((i & 1) == 0) {
        const int it = i >> 1;
        return *reinterpret_cast<const bf16x8 *>(kbase + koff(it >> 1) + (it & 1) * 32 * ROW_B);
      }
      const int pi = i >> 1;
      const int ks = pi / NDB, db = pi % NDB;
      if constexpr (VT) {
        return *reinterpret_cast<const bf16x8 *>(vb + voff_vt(ks) + db * 32 * VT_ROW_B);
      } else {
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4 *)(vb + voff[0][db] + ks * 16 * ROW_B));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4 *)(vb + voff[1][db] + ks * 16 * ROW_B));
        return bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      }
    };
    bf16x8 op[DIST + 1];
#pragma unroll
    for (int i = 0; i < DIST; ++i) op[i] = rd(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i + DIST < N) op[(i + DIST) % (DIST + 1)] = rd(i + DIST);
      const bf16x8 o = op[i % (DIST + 1)];
      if ((i & 1) == 0) {
        const int it = i >> 1, ds = it >> 1, kb = it & 1;
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, qreg[ds], ds == 0 ? f32x16{} : s[kb], 0, 0, 0);
      } else {
        const int pi = i >> 1, ks = pi / NDB, db = pi % NDB;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o, pb[ks], acc[db], 0, 0, 0);
        // The sum of the bf16 probabilities (the weights P V just used), four
        // per 4x4x4 MFMA, two per k-step.
        if ((db & 1) == 0)
          lh4 = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(
              db == 0 ? bf16x4{pb[ks][0], pb[ks][1], pb[ks][2], pb[ks][3]}
                      : bf16x4{pb[ks][4], pb[ks][5], pb[ks][6], pb[ks][7]},
              ones4, lh4, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Vector phase for the tile whose (masked) scores are in `s`: probabilities
  // and sums. The reference of the exponentials is updated
  // lazily from the tile sum: when a row's sum exceeds 2^TAU the reference
  // moves up by log2 of it, and the rescale of acc and the sums waits until
  // the P V of this tile has been added (the next vector phase). A tile is
  // redone against its true row max when a row has no reference yet or its
  // sum leaves [0, 2^32]. Both tests run only when some lane's half of its
  // row sum exceeds 2^(TAU-1) (or a reference is missing): otherwise every
  // row sum is at most 2^TAU and both would come out false.
  auto yphase = [&]() INLINE {
    apply_rescale();
    softmax();
    // Every half-row sum at most 2^(TAU-1) and every reference set: the row
    // sums are at most 2^TAU, so neither a redo nor a reference move is due.
    if (__any((m_run == -INFINITY) | !(lt <= 0x1p7f))) {
      float lt_row = pair_sum(lt);
      if (__any((m_run == -INFINITY) | !(lt_row <= 0x1p32f))) {
        const float m_new = fmaxf(m_run, rowmax());
        const float al = (m_run == -INFINITY || m_new == -INFINITY) ? 1.f : exp2_fast(m_run - m_new);
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[i] *= al;
        l_run *= al;
        lh4 *= al;
        m_run = m_new;
        m_use = m_run == -INFINITY ? 0.f : m_run;
        softmax();
        lt_row = pair_sum(lt);
      }
      const bool need = lt_row > 0x1p8f;  // 2^TAU
      const float lg = __builtin_amdgcn_logf(lt_row);  // log2
      alpha = need ? exp2_fast(-lg) : 1.f;
      m_run = need ? m_run + lg : m_run;
      m_use = m_run == -INFINITY ? 0.f : m_run;
      pend = __any(need);
    }
    l_run += lt;
  };
  static_assert(TAU == 8.f, "yphase compares against 2^TAU");

  // ---- prologue ----
  using St0 = std::integral_constant<int, 0>;
  using St1 = std::integral_constant<int, 1>;
  using St2 = std::integral_constant<int, 2>;
  using St3 = std::integral_constant<int, 3>;
  // Step t issues K (with positions) and V of tile t+3 into the stages tile
  // t-1 left (K before its barrier, V after it), and needs everything issued
  // up to step t-2: K of tile t+1 has two steps to land, V of tile t three. The loads are issued
  // unconditionally (a tile past the range reads zeros, or keys that are never
  // used, into a free stage): the compiler's own waits before LDS reads then
  // count the loads that follow exactly instead of assuming none did. The
  // prologue issues what steps -3 .. -1 would have.
  const int n_step = nk + nv;  // loads this wave issues per step
  issue_k(0, St0{});
  issue_v(0, St0{});
  issue_k(1, St1{});
  issue_v(1, St1{});
  wait_loads_upto(nv + nk + nv);  // K (and positions) of tile 0 have landed
  barrier_keep_loads();
  issue_k(2, St2{});
  issue_v(2, St2{});
  if (!done) {
    qk(St0{});
    mask(0, St0{});
    m_run = rowmax();
    m_use = m_run == -INFINITY ? 0.f : m_run;
  }

  // ---- main loop: step t = 0 .. nt-1 ----
  // Tile t lives in K and V stage t % 4. Each step has a matrix phase (scores
  // of tile t+1 and P V of tile t) and a vector phase (probabilities of the
  // tile whose scores are at hand). The two waves on a SIMD run them in
  // opposite orders: the first group matrix then vector (tile t+1), the
  // second vector (tile t) then matrix, so one wave's exponentials overlap the
  // other's MFMAs. The matrix phase runs at raised priority so that its MFMAs
  // go first.
  if (!grp_b && !done) yphase();
  auto step = [&](auto stage_c, int t) INLINE {
    constexpr int S = decltype(stage_c)::value;
    using SC = std::integral_constant<int, S>;
    using SN = std::integral_constant<int, (S + 1) % NSTAGE>;
    using SP = std::integral_constant<int, (S + NSTAGE - 1) % NSTAGE>;
    // K (and positions) of tile t-1 were last read in step t-2, which every
    // wave finished before the barrier of step t-1: their stage takes tile
    // t+3 before this step's barrier. Then this wave's loads up to step t-2
    // have landed, and after the barrier everyone's; every wave is done with
    // step t-1, so the V stage of tile t-1 is free too.
    issue_k(t + 3, SP{});
    wait_loads_upto(n_step + nk);
    barrier_keep_loads();
    asm volatile("" : "+v"(koff0), "+v"(voff0));  // pin: see koff
    issue_v(t + 3, SP{});
    if (!done) {
      if (grp_b) yphase();
      // After the wave's last tile the scores computed here are of a stage
      // holding no tile of its range and are dropped: one code path keeps the
      // accumulators in place.
      __builtin_amdgcn_s_setprio(1);
      xphase(SN{}, SC{});
      __builtin_amdgcn_s_setprio(0);
      if (t + 1 < w_nt) {
        mask(t + 1, SN{});
        if (!grp_b) yphase();
      } else {
        done = true;
      }
    }
  };
  // The body always runs all four steps (steps past nt only wait, synchronise
  // and issue loads past the range), so the loads issued between two LDS reads
  // are the same on every path through the loop.
  for (int t = 0; t < nt; t += NSTAGE) {
    step(St0{}, t);
    step(St1{}, t + 1);
    step(St2{}, t + 2);
    step(St3{}, t + 3);
  }
  wait_loads_upto(0);  // the loads past the range have landed before the wave ends
  apply_rescale();

  // ---- epilogue: o_b = acc / l^, lse_b = (ref + log2 l) ln 2; optional merge ----
  const float l_tot = pair_sum(l_run);
  const int own = lane & 3;
  const float lh_tot =
      pair_sum(own == 0 ? lh4[0] : own == 1 ? lh4[1] : own == 2 ? lh4[2] : lh4[3]);
  if (!tok_ok) return;
  // A row with no visible key in this block merges the identity: unchanged.
  if (a.merge && !(l_tot > 0.f)) return;
  const float lse_new = l_tot > 0.f ? (m_run + __log2f(l_tot)) * LN2 : -INFINITY;
  const float inv = l_tot > 0.f && lh_tot > 0.f ? 1.f / lh_tot : 0.f;
  const int64_t row = (bi * a.s_q + tok) * a.n_q + h;
  // Accumulator element e4*4 + j of block db holds d = db*32 + e4*8 + hi*4 + j.
  float *orow = a.o + row * D + hi * 4;
  // Merging: the old lse and all sixteen 16-byte pieces of the old o row go
  // out together, so the epilogue waits for memory once, not once per piece.
  float4 o_old[D / 32][4];
  float lse_old = -INFINITY;
  if (a.merge) {
    lse_old = a.lse[row];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        o_old[db][e4] = *reinterpret_cast<const float4 *>(orow + db * 32 + e4 * 8);
  }
  float w_old = 0.f, w_new = inv, lse_out = lse_new;
  if (a.merge) {
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
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      float4 r;
      r.x = w_new * acc[db][e4 * 4 + 0];
      r.y = w_new * acc[db][e4 * 4 + 1];
      r.z = w_new * acc[db][e4 * 4 + 2];
      r.w = w_new * acc[db][e4 * 4 + 3];
      if (a.merge) {
        const float4 old = o_old[db][e4];
        r.x += w_old * old.x;
        r.y += w_old * old.y;
        r.z += w_old * old.z;
        r.w += w_old * old.w;
      }
      *reinterpret_cast<float4 *>(orow + db * 32 + e4 * 8) = r;
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
  // NEAR: the byte offsets into K, V (or V^T) and the key positions stay below
  // 2^31 over the whole block plus the three tiles read past its end.
  const int64_t rows = a.s_kv + 3 * BK;
  const int64_t kv_row_bytes = static_cast<int64_t>(a.n_kv) * D * 2;
  const bool near = rows * kv_row_bytes < (int64_t{1} << 31) &&
                    (D - 1) * a.s_kv * 2 + rows * 2 < (int64_t{1} << 31);
  const unsigned grid = static_cast<unsigned>(blocks);
  if (a.k2) {
    // Two key blocks in one scan (V^T, no document mask; checked by the caller).
    if constexpr (VT) {
      if (near)
        attn_bf16_kernel<HW, true, false, true, true><<<grid, THREADS, 0, stream>>>(a);
      else
        attn_bf16_kernel<HW, true, false, false, true><<<grid, THREADS, 0, stream>>>(a);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (a.q_lo) {
    if (near)
      attn_bf16_kernel<HW, VT, true, true, false><<<grid, THREADS, 0, stream>>>(a);
    else
      attn_bf16_kernel<HW, VT, true, false, false><<<grid, THREADS, 0, stream>>>(a);
  } else {
    if (near)
      attn_bf16_kernel<HW, VT, false, true, false><<<grid, THREADS, 0, stream>>>(a);
    else
      attn_bf16_kernel<HW, VT, false, false, false><<<grid, THREADS, 0, stream>>>(a);
  }
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
