// attn_bf16.hip -- fused attention forward for bf16 storage on gfx950.
//
// Compiled once per key width: -DSFS_DK=16|32|64|128.  Each translation unit
// holds the Yat |k|^2 pre-pass for that width and the fused kernels for the
// three score-to-weight maps x four value widths.
//
// What is computed (per batch b, query head h, query row i; h_kv = h / g):
//   Yat     ("Softmax-Free Attention in JAX/Flax NNX", "One module, two
//            compatibility functions"): kappa = (q.k + b)^2 /
//            (max(|q|^2 + |k|^2 - 2 q.k, 0) + eps), masked kappa = 0,
//            out = sum kappa v / (sum kappa + 1e-9).
//   softmax ("NNX Scaled Dot-Product Attention", displayed equation):
//            softmax(q.k / sqrt(d_k)) with -inf on blocked keys.
//   s^tau   ("s^tau" forum post, core formula): phi = softplus(s) + 1e-6,
//            w = phi^tau / sum phi^tau, tau = softplus(log_tau) + 1.
//
// Design (gfx950 / CDNA4, wave64):
//   * A workgroup of 8 waves owns BM = 256 query rows of one (b, h); each wave
//     owns 32 rows, whose query fragments stay in registers as the B operand
//     of the score MFMA.  Key/value tiles of BN rows are staged HBM ->
//     registers -> LDS once for all 8 waves.  K is kept row-major, V is
//     transposed on the way in (V^T, keys contiguous), since the value MFMA
//     contracts over keys and wants 8 consecutive keys per lane.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: lane (half, col) then holds query col and 16
//     keys, so the score accumulator is already the B operand of the value
//     MFMA O^T = V^T P^T after an in-register bf16 conversion.  K rows are
//     written to LDS with bits 2 and 3 of the row index swapped; with that,
//     accumulator element r of 32-key block kb is key 32kb + 16(r/8) + 8 half
//     + r%8, i.e. eight consecutive keys per half per k-step of the second
//     MFMA, in natural order.
//   * The two halves of the workgroup run a "ping-pong" schedule (see the
//     kernel): on each SIMD one wave issues the matrix-core work of a tile
//     while its partner maps the previous scores to weights on the vector ALU.
//   * The Yat distance is built in registers from the same score tile.  The
//     score chain starts at b, so it yields u = q.k + b, and d2 = (|q|^2 + b)
//     + (|k|^2 + b) - 2u.  |k|^2 + b comes from a pre-pass (per query head)
//     and |q|^2 + b from the workgroup's own query fragments; both use the
//     same MFMA instruction, k-step order and start value as the score tile
//     (diagonals of X X^T), so for a key equal to its query the three terms
//     cancel to exactly 0 and the peak (|q|^2 + b)^2 / eps is reproduced.
//     Both row terms are held scaled by 2^-96, which lets the clamp at 0 and
//     the + eps ride on two FMAs (yat_den).
//   * Yat and s^tau accumulate sum(p v) and the mass in one pass with no
//     running maximum; softmax keeps a reference maximum that moves only when
//     a tile's maximum exceeds it by more than 2^8 (then O and the sum are
//     rescaled).
//   * Row statistics are per-lane partials over the lane's keys, combined
//     with the partner lane (lane ^ 32, v_permlane32_swap) once per tile
//     (softmax maximum) or once at the end (mass, max_score).
//   * Ragged tails: buffer loads past the end of a (b, h) slice return 0; the
//     mask zeroes keys >= T_k; query rows >= T_q are computed but not stored.
#include "bf16_common.h"

#include <type_traits>

#ifndef SFS_DK
#error "compile with -DSFS_DK=16, 32, 64 or 128"
#endif

#define SFS_CAT2(a, b) a##b
#define SFS_CAT(a, b) SFS_CAT2(a, b)

namespace sfs {
namespace {

// Softmax keeps exponentials relative to a reference maximum that is only
// moved when a tile's maximum exceeds it by more than this (log2 units):
// weights stay below 2^8 and most tiles skip the rescale of the accumulator.
constexpr float kRescaleSlack = 8.0f;

// Start value of the score accumulators.  Yat starts every MFMA chain -- the
// score q.k and the diagonals |q|^2 and |k|^2 -- at b: the chain then hands
// over u = q.k + b, the numerator's base, and the distance is
// d2 = (|q|^2 + b) + (|k|^2 + b) - 2u, with no add of b per element.  For a
// key equal to its query the three chains are the same instruction sequence
// from the same start, so d2 is still exactly 0.  The other maps start at 0.
template <int VAR>
__device__ __forceinline__ f32x16 score_init(float bias) {
  f32x16 c = {};
  if constexpr (is_yat(VAR)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) c[r] = bias;
  }
  return c;
}

// Yat's b of query head h (0 for the bias-free form).
__device__ __forceinline__ float yat_bias(const Problem& p, int h) {
  return p.yat_bias_free ? 0.f : softplus_precise(p.b_raw[h]);
}

// Yat with d_k <= 32 in the small-grid kernels: key norms formed in the
// kernel (no pre-pass).
__host__ __device__ constexpr bool yat_local_norms(int var, int dk) {
  return is_yat(var) && dk <= 32;
}

// Yat pre-pass: (|k_j|^2 + b_h) 2^-96 for every key row and query head, by the same
// MFMA sequence and start value as the score tile (see score_init).  One wave
// per 32 rows; grid (ceil(T_k / 128), Hq, B), 256 threads; output
// [B][Hq][nk_pitch(T_k)].
template <int DK>
__global__ __launch_bounds__(256) void yat_key_norms_bf16(Problem p) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int b = blockIdx.z, h = blockIdx.y, hk = h / (p.Hq / p.Hkv);
  const int row = blockIdx.x * 128 + 32 * w + col;
  const unsigned short* base =
      (const unsigned short*)p.k + (int64_t)b * p.ks[0] + (int64_t)hk * p.ks[1];
  const uint32_t bytes = slice_bytes(p.Tk, p.ks[2], DK);
  const rsrc_t r = make_rsrc(base, bytes);
  const uint32_t off = row < p.Tk ? (uint32_t)(((int64_t)row * p.ks[2] + 8 * half) * 2) : bytes;
  // the row's loads are issued before b is formed, so that the parameter
  // load and softplus run under them
  u32x4 x[DK / 16];
#pragma unroll
  for (int s = 0; s < DK / 16; ++s) x[s] = ld128(r, off + 32 * s);
  f32x16 g = score_init<kYat>(yat_bias(p, h));
#pragma unroll
  for (int s = 0; s < DK / 16; ++s)
    g = mfma32(__builtin_bit_cast(bf16x8, x[s]), __builtin_bit_cast(bf16x8, x[s]), g);
  if (row < p.Tk && holds_diag(col, half))
    p.nk[((int64_t)b * p.Hq + h) * nk_pitch(p.Tk) + row] = diag_of(g, col) * kNormScale;
}

// Fused forward, "ping-pong" schedule.
//
// A workgroup has 8 waves in two groups of 4 (group g = wave / 4); wave w and
// wave w + 4 share a SIMD.  Each wave owns 32 query rows; the workgroup owns
// BM = 256 rows of one (b, h) and streams key/value tiles of BN rows once for
// both groups.  The groups run half an iteration apart, separated by one
// workgroup barrier per phase:
//
//   phase 2t   : group 0 M(t)      group 1 W(t-1)
//   phase 2t+1 : group 0 W(t)      group 1 M(t)
//
// M(t) is matrix-core work -- O += V_{t-1}^T P_{t-1}^T and S_t = K_t Q^T --
// plus this group's share of the tile staging; W(t) is the score -> weight map
// of S_t on the vector ALU.  On every SIMD one wave therefore issues MFMAs
// while its partner issues VALU work.  Staging: group 0 writes K_{t+1} (and
// its |k|^2 rows) in phase 2t, group 1 writes V_t in phase 2t+1; K and V are
// double-buffered in LDS (K_t is read in phases 2t..2t+1, V_t in 2t+2..2t+3)
// and the |k|^2 rows triple-buffered (read in W phases up to 2t+2).  Global
// loads for a stage are issued one iteration before it is written.
template <int VAR, int DK, int DV, int BN>
__global__ __launch_bounds__(512, 1) void attn_fwd_bf16(Problem p) {
  constexpr int NW = 8;                  // waves per workgroup
  constexpr int BM = NW * 32;            // query rows per workgroup
  constexpr int GT = 256;                // threads per group
  constexpr int KS = DK / 16;            // k-steps of the score MFMA
  constexpr int DVP = DV < 32 ? 32 : DV; // value width padded to the MFMA block
  constexpr int DB = DVP / 32;           // 32-row blocks of O^T
  constexpr int KB = BN / 32;            // 32-key blocks per tile
  constexpr int KLD = DK + 8;            // LDS pitch of K rows (bf16), padded
  constexpr int VLD = BN + 8;            // LDS pitch of V^T rows (bf16), padded
  constexpr int KCH = DK / 8;            // 16-byte chunks per K row
  constexpr int K_UNITS = BN * KCH;
  constexpr int K_PER_T = (K_UNITS + GT - 1) / GT;
  constexpr int V_UNITS = (BN / 4) * (DV / 8);  // 4 keys x 8 values each
  constexpr int V_PER_T = (V_UNITS + GT - 1) / GT;
  static_assert(BN % 32 == 0 && BN <= 64, "tiles are 32 or 64 keys");

  __shared__ __attribute__((aligned(16))) unsigned short sK[2][BN * KLD];
  __shared__ __attribute__((aligned(16))) unsigned short sV[2][DVP * VLD];
  __shared__ __attribute__((aligned(16))) float sNK[3][BN];
  __shared__ float sNQ[BM];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int grp = w >> 2, gtid = tid & (GT - 1);
  const int col = lane & 31, half = lane >> 5;

  // Workgroup -> (query tile, batch, head) in XCD-aware head groups (the
  // resident workgroups of an XCD share 4 heads' K/V in its L2 instead of 8:
  // long_yat 476 -> 284 MB fetched per launch).  With a causal mask the
  // longest query tiles of a group go first.
  const int n_qt = (p.Tq + BM - 1) / BM;
  const int nbh = p.B * p.Hq;
  int qt, bh;
  grid_tile_slice(blockIdx.x, n_qt, nbh, qt, bh);
  if (p.causal) qt = n_qt - 1 - qt;
  const int b = bh / p.Hq, h = bh - b * p.Hq;
  const int hk = h / (p.Hq / p.Hkv);
  const int q0 = qt * BM, qw = q0 + 32 * w, my_q = qw + col;

  const unsigned short* qbase =
      (const unsigned short*)p.q + (int64_t)b * p.qs[0] + (int64_t)h * p.qs[1];
  const unsigned short* kbase =
      (const unsigned short*)p.k + (int64_t)b * p.ks[0] + (int64_t)hk * p.ks[1];
  const unsigned short* vbase =
      (const unsigned short*)p.v + (int64_t)b * p.vs[0] + (int64_t)hk * p.vs[1];
  const uint32_t q_bytes = slice_bytes(p.Tq, p.qs[2], DK);
  const uint32_t k_bytes = slice_bytes(p.Tk, p.ks[2], DK);
  const uint32_t v_bytes = slice_bytes(p.Tk, p.vs[2], DV);
  const rsrc_t rq = make_rsrc(qbase, q_bytes);
  const rsrc_t rk = make_rsrc(kbase, k_bytes);
  const rsrc_t rv = make_rsrc(vbase, v_bytes);
  const int kst = (int)p.ks[2], vst = (int)p.vs[2];

  // Per-head scalars, formed in the prologue once its loads are in flight.
  float bias = 0.f, eps = 0.f, tau = 0.f;
  auto head_scalars = [&]() {
    if (is_yat(VAR)) {
      bias = yat_bias(p, h);
      eps = softplus_precise(p.eps_raw[h]);
    } else if (VAR == kStau) {
      tau = softplus_precise(p.log_tau[h]) + 1.f;
    }
  };
  const float scale = 1.0f / sqrtf((float)DK);

  // Query fragments: lane (half, col) holds q[my_q][16 s + 8 half + 0..7]
  // (loaded in the prologue below).
  bf16x8 qf[KS];
  float nq = 0.f;
  // |k|^2 + b slice of this query head; padded to a multiple of 64 rows, so a
  // tile never reads past it (entries >= T_k are masked out).
  const float* nk_slice =
      is_yat(VAR) ? p.nk + ((int64_t)b * p.Hq + h) * nk_pitch(p.Tk) : nullptr;
  f32x16 sinit = {};  // score_init<VAR>(bias), set in the prologue

  const int kend = p.causal ? min(p.Tk, q0 + BM) : p.Tk;
  const int n_tiles = (kend + BN - 1) / BN;

  // Staging registers: group 0 stages K (+ |k|^2), group 1 stages V; one
  // array serves both, since a wave only ever stages one of them.
  constexpr int NSTG = K_PER_T > 4 * V_PER_T ? K_PER_T : 4 * V_PER_T;
  u32x4 stg[NSTG];
  f32x4 nkreg = {0.f, 0.f, 0.f, 0.f};

  // Tile loads.  A tile wholly inside T_k takes plain offsets (one add per
  // load); the last, partial tile points its rows >= T_k past the slice, where
  // buffer loads return 0.
  auto load_k = [&](int k0) {
    // this thread's rows are k0 + u / KCH for u = gtid + i GT: one base
    // offset, then steps of (GT / KCH) rows
    const uint32_t off0 = (uint32_t)(((k0 + gtid / KCH) * kst + 8 * (gtid % KCH)) * 2);
    const uint32_t step = (uint32_t)((GT / KCH) * kst * 2);
    if (k0 + BN <= p.Tk) {  // uniform
#pragma unroll
      for (int i = 0; i < K_PER_T; ++i)
        if (gtid + i * GT < K_UNITS) stg[i] = ld128(rk, off0 + i * step);
    } else {
#pragma unroll
      for (int i = 0; i < K_PER_T; ++i) {
        const int row = k0 + (gtid + i * GT) / KCH;
        if (gtid + i * GT < K_UNITS) stg[i] = ld128(rk, row < p.Tk ? off0 + i * step : k_bytes);
      }
    }
    if (is_yat(VAR) && gtid < BN / 4) nkreg = *(const f32x4*)(nk_slice + k0 + 4 * gtid);
  };
  auto store_k = [&](int t) {
    unsigned short* K = sK[t & 1];
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int u = gtid + i * GT;
      if (u < K_UNITS) {
        const int j = u / KCH, c = u % KCH;
        const int row = (j & ~31) | k_lds_row(j & 31);
        *(u32x4*)&K[row * KLD + 8 * c] = stg[i];
      }
    }
    if (is_yat(VAR) && gtid < BN / 4) *(f32x4*)&sNK[t % 3][4 * gtid] = nkreg;
  };
  auto load_v = [&](int k0) {
    const bool full = k0 + BN <= p.Tk;  // uniform
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = gtid + i * GT;
      if (u < V_UNITS) {
        const int g4 = u % (BN / 4), c = u / (BN / 4);
        const uint32_t off0 = (uint32_t)(((k0 + 4 * g4) * vst + 8 * c) * 2);
        if (full) {
#pragma unroll
          for (int r = 0; r < 4; ++r) stg[4 * i + r] = ld128(rv, off0 + (uint32_t)(r * vst * 2));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            stg[4 * i + r] = ld128(rv, k0 + 4 * g4 + r < p.Tk ? off0 + (uint32_t)(r * vst * 2)
                                                               : v_bytes);
        }
      }
    }
  };
  auto store_v = [&](int t) {
    unsigned short* Vt = sV[t & 1];
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = gtid + i * GT;
      if (u < V_UNITS) {
        const int g4 = u % (BN / 4), c = u / (BN / 4);
        // 4 keys x 8 values -> 8 value rows of 4 keys each.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned a0 = stg[4 * i][e], a1 = stg[4 * i + 1][e];
          const unsigned a2 = stg[4 * i + 2][e], a3 = stg[4 * i + 3][e];
          u32x2 lo, hi;
          lo[0] = lo_halves(a0, a1);
          lo[1] = lo_halves(a2, a3);
          hi[0] = hi_halves(a0, a1);
          hi[1] = hi_halves(a2, a3);
          *(u32x2*)&Vt[(8 * c + 2 * e) * VLD + 4 * g4] = lo;
          *(u32x2*)&Vt[(8 * c + 2 * e + 1) * VLD + 4 * g4] = hi;
        }
      }
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = f32x16{};
  f32x16 sacc[KB];          // S_t, from M(t) to W(t)
  bf16x8 pb[KB][2];         // P_t in bf16, from W(t) to M(t+1)
  float mass = 0.f;         // Yat: sum of weights; s^tau: of weights / (ln 2)^tau; softmax: sum exp2(x - mref)
  float mx = -INFINITY;     // Yat: max kappa; s^tau: max q.k; softmax: max of x = s*log2e/sqrt(dk)
  float mref = -INFINITY;   // softmax: reference maximum of the exponentials
  const MapConsts mc = map_consts(scale * kLog2e);
  const StauPoly sp = stau_poly();
  const float c_sm = mc.c_sm;

  // wave has work on tile t unless all its keys lie in the wave's future
  auto active = [&](int t) { return !(p.causal && t * BN > qw + 31); };

  // Matrix-core phases.  The A-operand fragments are read from LDS several
  // MFMAs ahead of use (the issue order is pinned with scheduling groups), so
  // the LDS latency is covered by MFMAs in flight instead of stalling each one.
  auto qk = [&](int t) {
    const unsigned short* K = sK[t & 1];
    constexpr int NF = KS * KB;   // fragments, in use order (s major, kb minor)
    constexpr int AHEAD = NF < 4 ? NF : 4;
    bf16x8 fa[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int s = i / KB, kb = i % KB;
      fa[i] = __builtin_bit_cast(
          bf16x8, *(const u32x4*)&K[(kb * 32 + col) * KLD + 16 * s + 8 * half]);
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] = sinit;
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int s = i / KB, kb = i % KB;
      sacc[kb] = mfma32(fa[i], qf[s], sacc[kb]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int i = 0; i < NF - AHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
  };
  auto pv = [&](int t) {
    const unsigned short* Vt = sV[t & 1];
    constexpr int NF = KB * 2 * DB;   // fragments, in use order ((kb, s) major, d minor)
    constexpr int AHEAD = DB;
    bf16x8 fa[NF];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int ks = i / DB, d = i % DB, kb = ks >> 1, s = ks & 1;
      fa[i] = __builtin_bit_cast(
          bf16x8, *(const u32x4*)&Vt[(32 * d + col) * VLD + kb * 32 + 16 * s + 8 * half]);
    }
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int ks = i / DB, d = i % DB, kb = ks >> 1, s = ks & 1;
      o[d] = mfma32(fa[i], pb[kb][s], o[d]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int i = 0; i < NF - AHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
  };

  // Score -> weight for tile t (vector ALU only).
  auto weights = [&](auto mask_tag, int t) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int k0 = t * BN;
    // key k0 + 8 half + o is allowed iff o <= lim (o: the element's offset,
    // a compile-time constant), so the mask is one compare per element
    const int lim = (p.causal ? min(my_q, p.Tk - 1) : p.Tk - 1) - (k0 + 8 * half);
    auto allowed = [&](int kb, int r) { return kb * 32 + 16 * (r >> 3) + (r & 7) <= lim; };
    if (VAR == kSoftmax) {
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sacc[kb][r] * c_sm;
          if (MASK) x = allowed(kb, r) ? x : -INFINITY;
          sacc[kb][r] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = pair_max(tmax);
      mx = fmaxf(mx, tmax);
      if (tmax > mref + kRescaleSlack) {  // first tile: mref = -inf
        const float alpha = __builtin_amdgcn_exp2f(mref - tmax);
        mass *= alpha;
#pragma unroll
        for (int d = 0; d < DB; ++d) o[d] *= alpha;
        mref = tmax;
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(sacc[kb][r] - mref);
          sacc[kb][r] = e;
          mass += e;
        }
    } else if (is_yat(VAR)) {
      const float* NK = sNK[t % 3];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        // (read as float vectors: this compiler mis-evaluates a bit_cast of a
        // single vector element)
        const f32x4 n0 = *(const f32x4*)&NK[kb * 32 + 8 * half];
        const f32x4 n1 = *(const f32x4*)&NK[kb * 32 + 8 * half + 4];
        const f32x4 n2 = *(const f32x4*)&NK[kb * 32 + 16 + 8 * half];
        const f32x4 n3 = *(const f32x4*)&NK[kb * 32 + 16 + 8 * half + 4];
        float nk[16];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          nk[e] = n0[e];
          nk[4 + e] = n1[e];
          nk[8 + e] = n2[e];
          nk[12 + e] = n3[e];
        }
        // In three stages over 8 elements (denominators, reciprocals,
        // numerators) so that the reciprocals issue back to back instead of
        // each stalling its own element.
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += 8) {
          float den[8], rc[8];
#pragma unroll
          for (int r = 0; r < 8; ++r)
            den[r] = yat_den(sacc[kb][r0 + r], nq + nk[r0 + r], eps, mc);
#pragma unroll
          for (int r = 0; r < 8; ++r) rc[r] = __builtin_amdgcn_rcpf(den[r]);
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const float u = sacc[kb][r0 + r];  // q.k + b
            float kap = yat_numerator<VAR>(u, p.yat_power) * rc[r];
            if (MASK) kap = allowed(kb, r0 + r) ? kap : 0.f;
            sacc[kb][r0 + r] = kap;
            mx = fmaxf(mx, kap);
          }
        }
      }
    } else {  // s^tau: weights phi^tau / (ln 2)^tau; max_score tracked on q.k
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = sacc[kb][r];
          float u = stau_weight2(x, tau, mc, sp);
          float xm = x;
          if (MASK) {
            const bool ok = allowed(kb, r);
            u = ok ? u : 0.f;
            xm = ok ? x : -INFINITY;
          }
          sacc[kb][r] = u;
          mx = fmaxf(mx, xm);
        }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 pw;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pw[e] = pack_bf16(sacc[kb][8 * s + 2 * e], sacc[kb][8 * s + 2 * e + 1]);
        // the mass (Yat, s^tau) is the sum of the bf16 weights the value MFMA takes
        if (is_yat(VAR) || VAR == kStau) {
#pragma unroll
          for (int e = 0; e < 4; ++e) mass = add_bf16_pair(pw[e], mass, mc);
        }
        pb[kb][s] = __builtin_bit_cast(bf16x8, pw);
      }
  };

  // Prologue: the query fragments and K_0 (group 0) or V_0 (group 1) in
  // flight together, one wait for all of them (so that none is outstanding on
  // entry to the main loop, where every score MFMA would otherwise wait for
  // the tile loads issued after them); then |q|^2 + b, K_0 into stage 0 and
  // K_1 into the staging registers.
  {
    const uint32_t off = my_q < p.Tq ? (uint32_t)(((int64_t)my_q * p.qs[2] + 8 * half) * 2)
                                     : q_bytes;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(bf16x8, ld128(rq, off + 32 * s));
  }
  if (grp == 0) load_k(0);
  else load_v(0);
  head_scalars();
  sinit = score_init<VAR>(bias);
  __builtin_amdgcn_s_waitcnt(0);
  if (is_yat(VAR)) {
    f32x16 g = sinit;
#pragma unroll
    for (int s = 0; s < KS; ++s) g = mfma32(qf[s], qf[s], g);
    if (holds_diag(col, half)) sNQ[32 * w + col] = diag_of(g, col) * kNormScale;
  }
  if (grp == 0) {
    store_k(0);
    if (n_tiles > 1) load_k(BN);
  }
  __syncthreads();
  if (is_yat(VAR)) nq = sNQ[32 * w + col];

  const int n_phases = 2 * n_tiles + 2;
  for (int ph = 0; ph < n_phases; ++ph) {
    const bool mphase = (ph & 1) == grp;
    if (mphase) {
      const int t = (ph - grp) >> 1;  // M(t)
      // the matrix-core wave issues first; its VALU partner fills the gaps
      __builtin_amdgcn_s_setprio(3);
      if (t >= 1 && active(t - 1)) pv(t - 1);
      if (t < n_tiles && active(t)) qk(t);
      if (grp == 0) {
        if (t + 1 < n_tiles) store_k(t + 1);
        if (t + 2 < n_tiles) load_k((t + 2) * BN);
      } else {
        if (t < n_tiles) store_v(t);
        if (t + 1 < n_tiles) load_v((t + 1) * BN);
      }
      __builtin_amdgcn_s_setprio(0);
    } else {
      const int t = (ph - 1 - grp) >> 1;  // W(t)
      if (t >= 0 && t < n_tiles && active(t)) {
        const int k0 = t * BN;
        const bool need_mask = (p.causal && k0 + BN - 1 > qw) || (k0 + BN > p.Tk);
        if (need_mask) weights(std::true_type{}, t);
        else weights(std::false_type{}, t);
      }
    }
    __syncthreads();
  }

  // Epilogue: combine the two lanes that share a query, normalise, store.
  float mass_all = pair_sum(mass);
  const float mx_all = pair_max(mx);
  if (VAR == kSoftmax) mass_all *= __builtin_amdgcn_exp2f(mref - mx_all);  // relative to the max
  float inv;
  if (is_yat(VAR)) inv = 1.f / (mass_all + 1e-9f);
  else if (VAR == kSoftmax) inv = 1.f / mass_all;
  else inv = mass_all > 0.f ? 1.f / mass_all : 0.f;
  // softmax: O holds sum exp2(x - mref) v; mass_all is relative to mx_all
  const float oscale = VAR == kSoftmax ? inv * __builtin_amdgcn_exp2f(mref - mx_all) : inv;
  if (my_q < p.Tq) {
    unsigned short* orow = (unsigned short*)p.out + (int64_t)b * p.os[0] +
                           (int64_t)h * p.os[1] + (int64_t)my_q * p.os[2];
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dv0 = 32 * d + 8 * g4 + 4 * half;
        if (dv0 < DV) {
          u32x2 st;
          st[0] = pack_bf16(o[d][4 * g4] * oscale, o[d][4 * g4 + 1] * oscale);
          st[1] = pack_bf16(o[d][4 * g4 + 2] * oscale, o[d][4 * g4 + 3] * oscale);
          *(u32x2*)&orow[dv0] = st;
        }
      }
    if (half == 0) {
      const int64_t ri = ((int64_t)b * p.Hq + h) * p.Tq + my_q;
      if (p.mass) p.mass[ri] = VAR == kStau ? mass_all * stau_unit(tau) : mass_all;
      if (p.max_score)
        p.max_score[ri] = VAR == kSoftmax ? mx_all * kLn2 : VAR == kStau ? mx_all * scale : mx_all;
    }
  }
}

// Fused forward for small grids (fewer query tiles than the ping-pong
// kernel needs to fill and balance the chip): NW waves x 32 query rows per
// workgroup, several workgroups per CU, one 64- or 32-key tile per iteration
// with two LDS stages.  Same layouts and score -> weight maps as above.
// PRE: every workgroup has at most kPreTiles tiles (short key ranges).  The
// prologue then issues all of its tile loads at once, next to the query
// fragments, and stores them to kPreTiles LDS stages: one memory latency per
// workgroup instead of one per tile, and no barrier inside the tile loop.
// It pays where the map is cheap (softmax); where the map is long (Yat,
// s^tau) the two-stage pipeline, which starts on the first tile while the
// next one loads, is as fast or faster, so the launcher keeps it there.
// KH = 2: two waves per 32 query rows, one per SIMD pair slot, each taking
// every other tile of the key range (the two tiles of an iteration are staged
// together), and their partial O, mass and maxima merged through LDS at the
// end.  A wave's chain of tiles -- which, with a causal mask, sets the time of
// the longest query tiles while the CU's other work has run out -- is then
// half as long.  One workgroup of 8 waves per CU instead of two of 4.
constexpr int kPreTiles = 4;

template <int VAR, int DK, int DV, int NW, int BN, bool PRE, int KH>
__global__ __attribute__((amdgpu_flat_work_group_size(KH * NW * 64, KH * NW * 64),
                          amdgpu_waves_per_eu(2, 2))) void attn_fwd_bf16_small(Problem p) {
  constexpr int BM = NW * 32;            // query rows per workgroup
  constexpr int NT = NW * 64;            // threads per key half
  constexpr int KS = DK / 16;            // k-steps of the score MFMA
  constexpr int DVP = DV < 32 ? 32 : DV; // value width padded to the MFMA block
  constexpr int DB = DVP / 32;           // 32-row blocks of O^T
  constexpr int KB = BN / 32;            // 32-key blocks per tile
  constexpr int KLD = DK + 8;            // LDS pitch of K rows (bf16), padded
  constexpr int VLD = BN + 8;            // LDS pitch of V^T rows (bf16), padded
  constexpr int KCH = DK / 8;            // 16-byte chunks per K row
  constexpr int K_UNITS = BN * KCH;
  constexpr int K_PER_T = (K_UNITS + NT - 1) / NT;
  constexpr int V_UNITS = (BN / 4) * (DV / 8);  // 4 keys x 8 values each
  constexpr int V_PER_T = (V_UNITS + NT - 1) / NT;
  static_assert(BN % 32 == 0 && BN <= 64, "tiles are 32 or 64 keys");
  constexpr int NSTG = PRE ? kPreTiles : 2;  // LDS stages
  constexpr int NSLOT = PRE ? kPreTiles : 1; // register sets of staged tiles
  static_assert(KH == 1 || (KH == 2 && !PRE), "key halves: 1, or 2 without PRE");

  // Yat with d_k <= 32 forms its key norms here, from the K fragments its
  // score MFMAs read anyway: the same instruction, k-step order and start
  // value as the pre-pass (ties still cancel), for KB KS more MFMAs per tile
  // and wave instead of a pre-pass launch, which costs more at these widths.
  constexpr bool NK_LOCAL = yat_local_norms(VAR, DK);

  // Two LDS stages (the tiles being computed and the next ones being
  // filled), or one per tile with PRE; each stage holds one tile per key half.
  __shared__ __attribute__((aligned(16))) unsigned short sK[NSTG][KH][BN * KLD];
  __shared__ __attribute__((aligned(16))) unsigned short sV[NSTG][KH][DVP * VLD];
  __shared__ __attribute__((aligned(16))) float sNK[NSTG][KH][BN];
  __shared__ __attribute__((aligned(16))) float sNKw[NK_LOCAL ? KH * NW : 1][NK_LOCAL ? BN : 4];
  __shared__ float sNQ[BM];
  // KH = 2 merge: the second half's O goes to sV, its row statistics to sK
  static_assert(KH == 1 || (NW * 64 * DB * 16 * 4 <= (int)sizeof(sV) &&
                            NW * 64 * 3 * 4 <= (int)sizeof(sK)), "merge buffers");

  // kh: the key half of this wave; tid, w: thread and wave within the half
  const int kh = (int)threadIdx.x / NT;
  const int tid = (int)threadIdx.x - kh * NT, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;

  // Workgroup -> (query tile, batch, head).  Heads vary fastest; with a causal
  // mask the longest query tiles are dispatched first.
  const int n_qt = (p.Tq + BM - 1) / BM;
  const int nbh = p.B * p.Hq;
  int qt = blockIdx.x / nbh;
  const int bh = blockIdx.x - qt * nbh;
  if (p.causal) qt = n_qt - 1 - qt;
  const int b = bh / p.Hq, h = bh - b * p.Hq;
  const int hk = h / (p.Hq / p.Hkv);
  const int q0 = qt * BM, qw = q0 + 32 * w, my_q = qw + col;

  const unsigned short* qbase =
      (const unsigned short*)p.q + (int64_t)b * p.qs[0] + (int64_t)h * p.qs[1];
  const unsigned short* kbase =
      (const unsigned short*)p.k + (int64_t)b * p.ks[0] + (int64_t)hk * p.ks[1];
  const unsigned short* vbase =
      (const unsigned short*)p.v + (int64_t)b * p.vs[0] + (int64_t)hk * p.vs[1];
  const uint32_t q_bytes = slice_bytes(p.Tq, p.qs[2], DK);
  const uint32_t k_bytes = slice_bytes(p.Tk, p.ks[2], DK);
  const uint32_t v_bytes = slice_bytes(p.Tk, p.vs[2], DV);
  const rsrc_t rq = make_rsrc(qbase, q_bytes);
  const rsrc_t rk = make_rsrc(kbase, k_bytes);
  const rsrc_t rv = make_rsrc(vbase, v_bytes);
  const int kst = (int)p.ks[2], vst = (int)p.vs[2];

  // Per-head scalars, formed in the prologue once its loads are in flight.
  float bias = 0.f, eps = 0.f, tau = 0.f;
  auto head_scalars = [&]() {
    if (is_yat(VAR)) {
      bias = yat_bias(p, h);
      eps = softplus_precise(p.eps_raw[h]);
    } else if (VAR == kStau) {
      tau = softplus_precise(p.log_tau[h]) + 1.f;
    }
  };
  const float scale = 1.0f / sqrtf((float)DK);

  // Query fragments: lane (half, col) holds q[my_q][16 s + 8 half + 0..7]
  // (loaded in the prologue below).
  bf16x8 qf[KS];
  float nq = 0.f;
  // |k|^2 + b slice of this query head; padded to a multiple of 64 rows, so a
  // tile never reads past it (entries >= T_k are masked out).
  const float* nk_slice =
      is_yat(VAR) ? p.nk + ((int64_t)b * p.Hq + h) * nk_pitch(p.Tk) : nullptr;
  f32x16 sinit = {};  // score_init<VAR>(bias), set in the prologue
  int b_sgpr = 0;     // bias as a wave-uniform bit pattern, set in the prologue

  const int kend = p.causal ? min(p.Tk, q0 + BM) : p.Tk;
  const int n_tiles = (kend + BN - 1) / BN;
  // With p.kv_splits > 1 this workgroup takes chunk blockIdx.y of its key
  // range, in whole tiles, and writes unnormalised partials.
  const int split = blockIdx.y;
  const int tps = (n_tiles + p.kv_splits - 1) / p.kv_splits;
  const int t_begin = min(split * tps, n_tiles);
  const int t_end = min(t_begin + tps, n_tiles);

  // Staging registers for the next key/value tile (PRE: for every tile).
  u32x4 kreg[NSLOT][K_PER_T];
  u32x4 vreg[NSLOT][V_PER_T][4];
  f32x4 nkreg[NSLOT];
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) nkreg[sl] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A tile wholly inside T_k takes plain offsets (one add per load); the
  // last, partial tile points its rows >= T_k past the slice (loads give 0).
  // `slot` (a compile-time index) names the register set.
  static_assert(NT % KCH == 0 && NT % (BN / 4) == 0, "load offsets step evenly");
  auto load_tile = [&](int k0, auto slot) {
    constexpr int SL = decltype(slot)::value;
    const bool full = k0 + BN <= p.Tk;
    const uint32_t koff = (uint32_t)(((k0 + tid / KCH) * kst + 8 * (tid % KCH)) * 2);
    const uint32_t kstep = (uint32_t)((NT / KCH) * kst * 2);
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      if (tid + i * NT < K_UNITS) {
        const int row = k0 + (tid + i * NT) / KCH;
        kreg[SL][i] = ld128(rk, full || row < p.Tk ? koff + i * kstep : k_bytes);
      }
    }
    const int g4 = tid % (BN / 4);
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      if (tid + i * NT < V_UNITS) {
        const int c = (tid + i * NT) / (BN / 4);
        const uint32_t voff = (uint32_t)(((k0 + 4 * g4) * vst + 8 * c) * 2);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = k0 + 4 * g4 + r;
          vreg[SL][i][r] = ld128(rv, full || row < p.Tk ? voff + (uint32_t)(r * vst * 2) : v_bytes);
        }
      }
    }
    if (is_yat(VAR) && !NK_LOCAL && tid < BN / 4)
      nkreg[SL] = *(const f32x4*)(nk_slice + k0 + 4 * tid);
  };

  auto store_tile = [&](int buf, auto slot) {
    constexpr int SL = decltype(slot)::value;
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int u = tid + i * NT;
      if (u < K_UNITS) {
        const int j = u / KCH, c = u % KCH;
        const int row = (j & ~31) | k_lds_row(j & 31);
        *(u32x4*)&sK[buf][kh][row * KLD + 8 * c] = kreg[SL][i];
      }
    }
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i) {
      const int u = tid + i * NT;
      if (u < V_UNITS) {
        const int g4 = u % (BN / 4), c = u / (BN / 4);
        // 4 keys x 8 values -> 8 value rows of 4 keys each.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned a0 = vreg[SL][i][0][e], a1 = vreg[SL][i][1][e];
          const unsigned a2 = vreg[SL][i][2][e], a3 = vreg[SL][i][3][e];
          u32x2 lo, hi;
          lo[0] = lo_halves(a0, a1);
          lo[1] = lo_halves(a2, a3);
          hi[0] = hi_halves(a0, a1);
          hi[1] = hi_halves(a2, a3);
          *(u32x2*)&sV[buf][kh][(8 * c + 2 * e) * VLD + 4 * g4] = lo;
          *(u32x2*)&sV[buf][kh][(8 * c + 2 * e + 1) * VLD + 4 * g4] = hi;
        }
      }
    }
    if (is_yat(VAR) && !NK_LOCAL && tid < BN / 4) *(f32x4*)&sNK[buf][kh][4 * tid] = nkreg[SL];
  };

  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = f32x16{};
  float mass = 0.f;       // Yat: sum of weights; s^tau: of weights / (ln 2)^tau; softmax: sum exp2(x - mref)
  float mx = -INFINITY;   // Yat: max kappa; s^tau: max q.k; softmax: max of x = s*log2e/sqrt(dk)
  float mref = -INFINITY; // softmax: reference maximum of the exponentials
  const MapConsts mc = map_consts(scale * kLog2e);
  const StauPoly sp = stau_poly();
  const float c_sm = mc.c_sm;

  // One tile of BN keys against the wave's 32 queries.
  auto compute = [&](auto mask_tag, int buf, int k0) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const unsigned short* K = sK[buf][kh];
    const unsigned short* Vt = sV[buf][kh];

    // S^T = K Q^T, the KB accumulation chains interleaved.
    f32x16 sacc[KB];
    if constexpr (is_yat(VAR)) {
      // the start values are rebuilt from a scalar for every tile (holding
      // them across the loop would cost 16 registers)
      int b_bits = b_sgpr;
      asm volatile("" : "+s"(b_bits));
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = __int_as_float(b_bits);
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sacc[kb] = f32x16{};
    }
    f32x16 gk[NK_LOCAL ? KB : 1];  // NK_LOCAL: K K^T of each 32-key block, from b
    if constexpr (NK_LOCAL) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) gk[kb] = sacc[kb];
    }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *(const u32x4*)&K[(kb * 32 + col) * KLD + 16 * s + 8 * half]);
        sacc[kb] = mfma32(a, qf[s], sacc[kb]);
        if constexpr (NK_LOCAL) gk[kb] = mfma32(a, a, gk[kb]);
      }
    if constexpr (NK_LOCAL) {
      // LDS row i of the tile holds key (i & ~31) | k_lds_row(i & 31); this
      // wave's own copy of the norms, in key order (read back by the same wave)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        if (holds_diag(col, half))
          sNKw[kh * NW + w][kb * 32 + k_lds_row(col)] = diag_of(gk[kb], col) * kNormScale;
    }

    // key k0 + 8 half + o is allowed iff o <= lim (o: the element's offset,
    // a compile-time constant), so the mask is one compare per element
    const int lim = (p.causal ? min(my_q, p.Tk - 1) : p.Tk - 1) - (k0 + 8 * half);
    auto allowed = [&](int kb, int r) { return kb * 32 + 16 * (r >> 3) + (r & 7) <= lim; };

    if (VAR == kSoftmax) {
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sacc[kb][r] * c_sm;
          if (MASK) x = allowed(kb, r) ? x : -INFINITY;
          sacc[kb][r] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = pair_max(tmax);
      mx = fmaxf(mx, tmax);
      if (tmax > mref + kRescaleSlack) {  // first tile: mref = -inf
        const float alpha = __builtin_amdgcn_exp2f(mref - tmax);
        mass *= alpha;
#pragma unroll
        for (int d = 0; d < DB; ++d) o[d] *= alpha;
        mref = tmax;
      }
      // (a row with no allowed key so far keeps mref = -inf; its masked
      // scores must give 0, not -inf - -inf)
      const float mref_f = fmaxf(mref, -3.0e38f);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(sacc[kb][r] - mref_f);
          sacc[kb][r] = e;
          mass += e;
        }
    } else if (is_yat(VAR)) {
      const float* NK = NK_LOCAL ? sNKw[NK_LOCAL ? kh * NW + w : 0] : sNK[buf][kh];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        // (read as float vectors: this compiler mis-evaluates a bit_cast of a
        // single vector element)
        const f32x4 n0 = *(const f32x4*)&NK[kb * 32 + 8 * half];
        const f32x4 n1 = *(const f32x4*)&NK[kb * 32 + 8 * half + 4];
        const f32x4 n2 = *(const f32x4*)&NK[kb * 32 + 16 + 8 * half];
        const f32x4 n3 = *(const f32x4*)&NK[kb * 32 + 16 + 8 * half + 4];
        float nk[16];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          nk[e] = n0[e];
          nk[4 + e] = n1[e];
          nk[8 + e] = n2[e];
          nk[12 + e] = n3[e];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float u = sacc[kb][r];  // q.k + b
          float kap = yat_numerator<VAR>(u, p.yat_power) *
                      __builtin_amdgcn_rcpf(yat_den(u, nq + nk[r], eps, mc));
          if (MASK) kap = allowed(kb, r) ? kap : 0.f;
          sacc[kb][r] = kap;
          mx = fmaxf(mx, kap);
        }
      }
    } else {  // s^tau: weights phi^tau / (ln 2)^tau; max_score tracked on q.k
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = sacc[kb][r];
          float u = stau_weight2(x, tau, mc, sp);
          float xm = x;
          if (MASK) {
            const bool ok = allowed(kb, r);
            u = ok ? u : 0.f;
            xm = ok ? x : -INFINITY;
          }
          sacc[kb][r] = u;
          mx = fmaxf(mx, xm);
        }
    }

    // O^T += V^T P^T.
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 pw;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pw[e] = pack_bf16(sacc[kb][8 * s + 2 * e], sacc[kb][8 * s + 2 * e + 1]);
        // the mass (Yat, s^tau) is the sum of the bf16 weights the value MFMA takes
        if (is_yat(VAR) || VAR == kStau) {
#pragma unroll
          for (int e = 0; e < 4; ++e) mass = add_bf16_pair(pw[e], mass, mc);
        }
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, *(const u32x4*)&Vt[(32 * d + col) * VLD + kb * 32 + 16 * s + 8 * half]);
          o[d] = mfma32(a, pb, o[d]);
        }
      }
  };

  // Prologue: the query fragments and the first tile (PRE: every tile) in
  // flight together, one wait for all of them (none outstanding on entry to
  // the main loop); then |q|^2 + b, the first tile into its stage, the next
  // into registers (PRE: every tile into its own stage).
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, (NSLOT > 1 ? 1 : 0)>;
  using S2 = std::integral_constant<int, (NSLOT > 2 ? 2 : 0)>;
  using S3 = std::integral_constant<int, (NSLOT > 3 ? 3 : 0)>;
  static_assert(!PRE || kPreTiles == 4, "the prologue names four slots");
  {
    const uint32_t off = my_q < p.Tq ? (uint32_t)(((int64_t)my_q * p.qs[2] + 8 * half) * 2)
                                     : q_bytes;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(bf16x8, ld128(rq, off + 32 * s));
  }
  if (t_begin + kh < t_end) load_tile((t_begin + kh) * BN, S0{});
  if constexpr (PRE) {
    if (t_begin + 1 < t_end) load_tile((t_begin + 1) * BN, S1{});
    if (t_begin + 2 < t_end) load_tile((t_begin + 2) * BN, S2{});
    if (t_begin + 3 < t_end) load_tile((t_begin + 3) * BN, S3{});
  }
  head_scalars();
  sinit = score_init<VAR>(bias);
  b_sgpr = __builtin_amdgcn_readfirstlane(__float_as_int(bias));
  __builtin_amdgcn_s_waitcnt(0);
  if (is_yat(VAR) && kh == 0) {
    f32x16 g = sinit;
#pragma unroll
    for (int s = 0; s < KS; ++s) g = mfma32(qf[s], qf[s], g);
    if (holds_diag(col, half)) sNQ[32 * w + col] = diag_of(g, col) * kNormScale;
  }
  if constexpr (PRE) {
    if (t_begin < t_end) store_tile(0, S0{});
    if (t_begin + 1 < t_end) store_tile(1, S1{});
    if (t_begin + 2 < t_end) store_tile(2, S2{});
    if (t_begin + 3 < t_end) store_tile(3, S3{});
  } else if (t_begin + kh < t_end) {
    store_tile(0, S0{});
    if (t_begin + KH + kh < t_end) load_tile((t_begin + KH + kh) * BN, S0{});
  }
  __syncthreads();
  if (is_yat(VAR)) nq = sNQ[32 * w + col];

  // Iteration it covers tiles t .. t + KH - 1, this wave tile t + kh.
  for (int t = t_begin, it = 0; t < t_end; t += KH, ++it) {
    const int tt = t + kh, k0 = tt * BN, buf = PRE ? t - t_begin : it & 1;
    // past the range, or every key of the tile in this wave's future: nothing to do
    if (tt < t_end && !(p.causal && k0 > qw + 31)) {
      const bool need_mask = (p.causal && k0 + BN - 1 > qw) || (k0 + BN > p.Tk);
      if (need_mask) compute(std::true_type{}, buf, k0);
      else compute(std::false_type{}, buf, k0);
    }
    if constexpr (!PRE) {
      if (tt + KH < t_end) {
        // Stage buf ^ 1 was last read in iteration it - 1, which every wave
        // finished before the barrier that ended it.
        store_tile(buf ^ 1, S0{});
        if (tt + 2 * KH < t_end) load_tile(k0 + 2 * KH * BN, S0{});
      }
      __syncthreads();
    }
  }

  // KH = 2: the second key half hands its partials to the first through LDS
  // (the stages are free: the loop's last barrier, or the prologue's, has
  // passed) and ends; the first merges them.  Yat and s^tau add O and the
  // mass; softmax first brings both to the larger reference maximum.
  if constexpr (KH == 2) {
    float* mo = reinterpret_cast<float*>(&sV[0][0][0]);
    float* ms = reinterpret_cast<float*>(&sK[0][0][0]);
    const int slot = w * 64 + lane;
    if (kh == 1) {
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = o[d][4 * g4 + e];
          *(f32x4*)&mo[((d * 4 + g4) * NT + slot) * 4] = v4;
        }
      ms[slot] = mass;
      ms[NT + slot] = mx;
      ms[2 * NT + slot] = mref;
    }
    __syncthreads();
    if (kh == 1) return;
    const float mass1 = ms[slot], mx1 = ms[NT + slot], mref1 = ms[2 * NT + slot];
    float f0 = 1.f, f1 = 1.f;
    if (VAR == kSoftmax) {
      const float m = fmaxf(mref, mref1);
      f0 = mref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mref - m);
      f1 = mref1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mref1 - m);
      mref = m;
    }
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 v4 = *(const f32x4*)&mo[((d * 4 + g4) * NT + slot) * 4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[d][4 * g4 + e] = VAR == kSoftmax ? o[d][4 * g4 + e] * f0 + v4[e] * f1
                                             : o[d][4 * g4 + e] + v4[e];
      }
    mass = VAR == kSoftmax ? mass * f0 + mass1 * f1 : mass + mass1;
    mx = fmaxf(mx, mx1);
  }

  // Epilogue: combine the two lanes that share a query, normalise, store.
  float mass_all = pair_sum(mass);
  const float mx_all = pair_max(mx);
  if (p.kv_splits > 1) {
    // partials of this chunk: O (relative to mref for softmax), mass, max, mref
    // (s^tau: O and mass in units of phi^tau, max as s, like the decode kernel's)
    const float ounit = VAR == kStau ? stau_unit(tau) : 1.f;
    if (my_q < p.Tq) {
      const int64_t R = (int64_t)p.B * p.Hq * p.Tq;
      const int64_t ri = ((int64_t)b * p.Hq + h) * p.Tq + my_q;
      float* po = p.part + ((int64_t)split * R + ri) * p.dv;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dv0 = 32 * d + 8 * g4 + 4 * half;
          if (dv0 < DV) {
            f32x4 st;
#pragma unroll
            for (int e = 0; e < 4; ++e) st[e] = VAR == kStau ? o[d][4 * g4 + e] * ounit
                                                              : o[d][4 * g4 + e];
            *(f32x4*)&po[dv0] = st;
          }
        }
      if (half == 0) {
        f32x4 st = {mass_all * ounit, VAR == kStau ? mx_all * scale : mx_all, mref, 0.f};
        *(f32x4*)&p.part[(int64_t)p.kv_splits * R * p.dv + ((int64_t)split * R + ri) * 4] = st;
      }
    }
    return;
  }
  if (VAR == kSoftmax) mass_all *= __builtin_amdgcn_exp2f(mref - mx_all);  // relative to the max
  float inv;
  if (is_yat(VAR)) inv = 1.f / (mass_all + 1e-9f);
  else if (VAR == kSoftmax) inv = 1.f / mass_all;
  else inv = mass_all > 0.f ? 1.f / mass_all : 0.f;
  // softmax: O holds sum exp2(x - mref) v; mass_all is relative to mx_all
  const float oscale = VAR == kSoftmax ? inv * __builtin_amdgcn_exp2f(mref - mx_all) : inv;
  if (my_q < p.Tq) {
    unsigned short* orow = (unsigned short*)p.out + (int64_t)b * p.os[0] +
                           (int64_t)h * p.os[1] + (int64_t)my_q * p.os[2];
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dv0 = 32 * d + 8 * g4 + 4 * half;
        if (dv0 < DV) {
          u32x2 st;
          st[0] = pack_bf16(o[d][4 * g4] * oscale, o[d][4 * g4 + 1] * oscale);
          st[1] = pack_bf16(o[d][4 * g4 + 2] * oscale, o[d][4 * g4 + 3] * oscale);
          *(u32x2*)&orow[dv0] = st;
        }
      }
    if (half == 0) {
      const int64_t ri = ((int64_t)b * p.Hq + h) * p.Tq + my_q;
      if (p.mass) p.mass[ri] = VAR == kStau ? mass_all * stau_unit(tau) : mass_all;
      if (p.max_score)
        p.max_score[ri] = VAR == kSoftmax ? mx_all * kLn2 : VAR == kStau ? mx_all * scale : mx_all;
    }
  }
}


// Keys per tile.
#ifndef SFS_BN
#define SFS_BN 64
#endif
// The 128-row small-grid kernel splits each workgroup's key range over two
// key halves (KH = 2) when that range spans at least this many 64-key tiles:
// stau_gqa 76.7 -> 72.2 us; with the 4 tiles of gpt_small it is slower.
constexpr int kKeyHalvesMinTiles = 8;

// the instantiations with PRE (others compile it as false)
template <int VAR, int DK, int DV>
constexpr bool kPreBuilt = VAR == kSoftmax && DK <= 64 && DV <= 64;

template <int VAR, int DV>
hipError_t launch_variant(const Problem& p, hipStream_t stream) {
  constexpr int DK = SFS_DK;
  constexpr int BN = SFS_BN;
  // (the small-grid kernels form the norms themselves at d_k <= 32)
  if (is_yat(VAR) && !(p.block_rows != 256 && yat_local_norms(VAR, DK)))
    hipLaunchKernelGGL(yat_key_norms_bf16<DK>, dim3((p.Tk + 127) / 128, p.Hq, p.B), dim3(256), 0,
                       stream, p);
  // p.block_rows and p.kv_splits come from the host plan (make_plan)
  const unsigned bh = (unsigned)p.B * (unsigned)p.Hq;
  const unsigned nq = (unsigned)((p.Tq + p.block_rows - 1) / p.block_rows) * bh;
  // short key ranges (every workgroup at most kPreTiles tiles) preload all
  // of their tiles with the softmax map; kept to d <= 64, where the staging
  // registers fit
  const int tile_keys = p.block_rows == 128 ? 64 : 32;
  const bool pre = VAR == kSoftmax && DK <= 64 && DV <= 64 && p.kv_splits == 1 &&
                   p.Tk <= kPreTiles * tile_keys;
  // 64-key tiles in the longest workgroup's key range (per key split)
  const int64_t span = p.causal ? min((int64_t)p.Tk, (int64_t)nq / bh * 128) : (int64_t)p.Tk;
  const int64_t tiles = ((span + 63) / 64 + p.kv_splits - 1) / p.kv_splits;
  const bool key_halves = tiles >= kKeyHalvesMinTiles;
  if (p.block_rows == 256) {
    hipLaunchKernelGGL((attn_fwd_bf16<VAR, DK, DV, BN>), dim3(nq), dim3(512), 0, stream, p);
  } else if (p.block_rows == 128) {
    if (pre)
      hipLaunchKernelGGL((attn_fwd_bf16_small<VAR, DK, DV, 4, 64, kPreBuilt<VAR, DK, DV>, 1>),
                         dim3(nq, p.kv_splits), dim3(256), 0, stream, p);
    else if (key_halves)
      hipLaunchKernelGGL((attn_fwd_bf16_small<VAR, DK, DV, 4, 64, false, 2>),
                         dim3(nq, p.kv_splits), dim3(512), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_fwd_bf16_small<VAR, DK, DV, 4, 64, false, 1>),
                         dim3(nq, p.kv_splits), dim3(256), 0, stream, p);
  } else {
    if (pre)
      hipLaunchKernelGGL((attn_fwd_bf16_small<VAR, DK, DV, 2, 32, kPreBuilt<VAR, DK, DV>, 1>),
                         dim3(nq, p.kv_splits), dim3(128), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_fwd_bf16_small<VAR, DK, DV, 2, 32, false, 1>),
                         dim3(nq, p.kv_splits), dim3(128), 0, stream, p);
  }
  return hipGetLastError();
}

template <int VAR>
hipError_t launch_dv(const Problem& p, hipStream_t stream) {
  switch (p.dv) {
    case 16: return launch_variant<VAR, 16>(p, stream);
    case 32: return launch_variant<VAR, 32>(p, stream);
    case 64: return launch_variant<VAR, 64>(p, stream);
    case 128: return launch_variant<VAR, 128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t SFS_CAT(launch_bf16_dk, SFS_DK)(const Problem& p, hipStream_t stream) {
  switch (p.variant) {
    case kSoftmax: return launch_dv<kSoftmax>(p, stream);
    case kYat: return p.yat_power > 1 ? launch_dv<kYatPow>(p, stream) : launch_dv<kYat>(p, stream);
    case kStau: return launch_dv<kStau>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace sfs
