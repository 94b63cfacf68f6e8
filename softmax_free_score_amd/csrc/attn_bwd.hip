// attn_bwd.hip -- attention backward for bf16 storage on gfx950.
//
// Compiled once per key width: -DSFS_DK=16|32|64|128.
//
// For L = sum(dout * out) and the forward defined in attn_bf16.hip, with the
// row values D_i = sum_j w_ij dp_ij (= dout_i . out_i; computed here from the
// recomputed weights) and the normaliser Z_i of the forward (see
// attn_bwd_aux.hip), every allowed pair (i, j) has
//   w_ij  the forward's weight,  dp_ij = dout_i . v_j,
//   du_ij = (dp_ij - D_i) / Z_i  (d L / d of the unnormalised weight u_ij),
// and the gradients are
//   dv_j = sum_i w_ij dout_i,
//   dq_i = sum_j g_ij k_j - c_i q_i,   dk_j = sum_i g_ij q_i - c'_j k_j,
// with the "gradient score" g and the corrections c per map:
//   softmax  u = e^(s - max), s = q.k / sqrt(d_k):
//            g = w (dp - D) / sqrt(d_k), c = 0;
//   s^tau    u = phi^tau, phi = softplus(s) + 1e-6:
//            g = w (dp - D) tau sigmoid(s) / phi / sqrt(d_k), c = 0;
//   Yat      u = kappa = (q.k + b)^2 / den, den = |q|^2 + |k|^2 - 2 q.k + eps
//            (d den / d q = 2 (q - k)):
//            g = A + B, A = 2 du (q.k + b) / den, B = 2 du kappa / den,
//            c_i = sum_j B_ij, c'_j = sum_i B_ij,
// i.e. d kappa / d q = [2 (q.k + b) k - 2 kappa (q - k)] / den.
// ("Softmax-Free Attention in JAX/Flax NNX", "One module, two compatibility
// functions", for the Yat map; "NNX Scaled Dot-Product Attention", displayed
// equation, for softmax; the "s^tau" forum post, core formula, for s^tau.)
//
// Design (gfx950 / CDNA4, wave64, v_mfma_f32_32x32x16_bf16 throughout):
//   * Two kernels, no atomics: attn_bwd_kv owns 128 keys of one (b, kv head)
//     per workgroup (32 per pair of waves, their k and v rows in registers)
//     and streams 32-query tiles of every query head of the group; attn_bwd_q owns 128
//     query rows of one (b, h) (32 per wave) and streams 32-key tiles.  Each
//     recomputes the score tile (and dp) it needs, so both the score and the
//     dp products are taken twice; in exchange every output is written once,
//     in a fixed summation order.
//   * attn_bwd_kv computes S = Q K^T with the query rows of the tile in LDS
//     (rows permuted by swapping bits 2 and 3, as the forward does for keys),
//     so the accumulator of lane (half, col) holds key col and queries
//     16 (r / 8) + 8 half + r % 8 in natural order: packed to bf16 it is the B
//     operand of dV^T += dO^T P and dK^T += Q^T G, whose A operands (dO^T,
//     Q^T) come from the same row-major tiles by transposing LDS reads.
//   * attn_bwd_q is the mirror image: S^T = K Q^T and dP^T = V dO^T with the
//     lane's query fragments in registers, then dQ^T += K^T G^T with K^T in
//     LDS.
//   * Yat's subtraction of c q (or c' k) cancels against the B part of the
//     product g k exactly where q = k only if both use the same B values.
//     g is rounded to bf16 for the matrix core; the correction uses
//     B' = bf16(g) - A, so that the kernel computes A k + B' (k - q) with the
//     difference (k - q) formed in exact arithmetic.
//   * Yat |q|^2 and |k|^2 come from the same MFMA pre-pass as the forward's,
//     so d2 = |q|^2 + |k|^2 - 2 q.k cancels to exactly 0 for a key equal to
//     its query.
//   * Parameter gradients: attn_bwd_q sums A/2 and B/2 (Yat) or
//     w (dp - D) log2(phi) (s^tau) per workgroup; a last kernel adds the
//     workgroup sums per head in a fixed order.
//   * Yat carries g/2 = A/2 (1 + u/den) and A/2 = (dp - D) Z u / den, u = q.k
//     + b, which needs neither kappa nor the factor 2 per pair; outputs and
//     sums are doubled at the end (exact in binary floating point).
#include "bf16_common.h"

#include <type_traits>

#ifndef SFS_DK
#error "compile with -DSFS_DK=16, 32, 64 or 128"
#endif

#define SFS_CAT2(a, b) a##b
#define SFS_CAT(a, b) SFS_CAT2(a, b)

namespace sfs {
namespace {

__device__ __forceinline__ float bf16_lo(unsigned x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(unsigned x) { return __uint_as_float(x & 0xffff0000u); }

// A-operand fragment of v_mfma_f32_32x32x16_bf16 whose matrix is the
// transpose of a row-major LDS tile R (32 rows, pitch `ld` elements, row j
// stored at position k_lds_row(j)): lane (half, col) receives column
// c0 + col of tile rows 16 s + 8 half .. 16 s + 8 half + 7.  Two
// ds_read_b64_tr_b16 per lane: within each group of 16 lanes, source lane c
// addresses tile row base + c / 4, columns cb + 4 (c % 4) .. + 3, and the
// hardware returns to lane i of the group column cb + i of rows base .. base
// + 3 (lane mapping measured on gfx950).
//
// The lane's part of the address is formed once by tr_lane_off (elements);
// tr_frag_at(R + off, ld, c0, s) then reads at (16 s + 8 j) ld + c0, j = 0, 1,
// offsets the reads carry as immediates.  (k_lds_row swaps row bits 2 and 3,
// so tile row 16 s + 8 (g >> 1) + 4 j + (c >> 2), g = lane / 16, sits at
// 16 s + 8 j + 4 (g >> 1) + (c >> 2).)  Needs c0 + 32 <= width, or c0 = 0 for
// a tile narrower than 32, whose columns at or past `width` wrap to
// width - 16 .. width - 1: those rows of the product are not used.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int tr_lane_off(int lane, int ld, int width) {
  const int g = lane >> 4, c = lane & 15;
  int cb = 16 * (g & 1) + 4 * (c & 3);
  if (cb >= width) cb -= 16;
  return (4 * (g >> 1) + (c >> 2)) * ld + cb;
}
__device__ __forceinline__ bf16x8 tr_frag_at(const unsigned short* R, int ld, int c0, int s) {
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(R + (16 * s + 8 * j) * ld + c0));
    const u32x2 xx = __builtin_bit_cast(u32x2, x);
    out[2 * j] = xx[0];
    out[2 * j + 1] = xx[1];
  }
  return __builtin_bit_cast(bf16x8, out);
}

// Per-head constants of a map.
struct HeadC {
  float bias, eps, tau, scale, c_sm;
};
template <int VAR, int DK>
__device__ __forceinline__ HeadC head_consts(const BwdProblem& p, int h) {
  HeadC c{0.f, 0.f, 0.f, 1.0f / sqrtf((float)DK), 0.f};
  c.c_sm = c.scale * kLog2e;
  if (is_yat(VAR)) {
    c.bias = softplus_precise(p.b_raw[h]);
    c.eps = softplus_precise(p.eps_raw[h]);
  } else if (VAR == kStau) {
    c.tau = softplus_precise(p.log_tau[h]) + 1.f;
  }
  return c;
}

// The forward's weight of one pair from the score sd, the row normaliser Z
// (softmax: L, the log2 normaliser) and, for Yat, nqk.  Yat's score chains
// start at b, as the forward's do: sd = u = q.k + b and nqk = ((|q|^2 + b) +
// (|k|^2 + b)) 2^-96, so d2 = 2^96 nqk - 2u; for softmax and s^tau sd = q.k.
template <int VAR>
__device__ __forceinline__ float pair_weight(float sd, float Z, float nqk, const HeadC& hc) {
  if constexpr (is_yat(VAR)) {
    const float rden = __builtin_amdgcn_rcpf(yat_den(sd, nqk, hc.eps));
    return sd * (sd * rden) * Z;
  } else if constexpr (VAR == kSoftmax) {
    return __builtin_amdgcn_exp2f(fmaf(sd, hc.c_sm, -Z));
  } else {
    const float s = sd * hc.scale;
    // softplus as the forward takes it: max(s, 0) + log1p(e), e = exp(-|s|),
    // with the rounding error of 1 + e corrected to first order
    const float e = __builtin_amdgcn_exp2f(-fabsf(s) * kLog2e);
    const float u1 = 1.f + e;
    const float c = (u1 - 1.f) - e;
    const float sp = fmaf(__builtin_amdgcn_logf(u1), kLn2, fmaxf(s, 0.f) - c);
    return __builtin_amdgcn_exp2f(hc.tau * __builtin_amdgcn_logf(sp + 1e-6f)) * Z;
  }
}

// The gradient score of one pair from sd, dp = dout.v, the row's D and Z and
// (Yat) nqk, before the 1/sqrt(d_k) of softmax and s^tau, plus the terms of
// the Yat correction and parameter sums (a, lt) and of the s^tau parameter
// sum (lt).
//   Yat:   returns g/2, a = A/2 and lt = B/2 (the kernels double the
//          results; exact): with r = 1/den, u = q.k + b:
//          A/2 = (dp - D) Z u r, B/2 = A/2 u r, g/2 = A/2 + B/2
//          (B/A = kappa/u = u r).
//   softmax: g = w (dp - D);  s^tau: g = w (dp - D) tau sigmoid(s) / phi,
//          lt = w (dp - D) log2(phi).
template <int VAR>
__device__ __forceinline__ void pair_grad(float sd, float dp, float D, float Z, float nqk,
                                          const HeadC& hc, float& g, float& a, float& lt) {
  if constexpr (is_yat(VAR)) {
    const float rden = __builtin_amdgcn_rcpf(yat_den(sd, nqk, hc.eps));
    const float ur = sd * rden;
    a = (dp - D) * Z * ur;
    lt = a * ur;
    g = a + lt;
  } else if constexpr (VAR == kSoftmax) {
    g = __builtin_amdgcn_exp2f(fmaf(sd, hc.c_sm, -Z)) * (dp - D);
    a = lt = 0.f;
  } else {
    const float s = sd * hc.scale;
    const float e = __builtin_amdgcn_exp2f(-fabsf(s) * kLog2e);
    const float u1 = 1.f + e;
    const float c = (u1 - 1.f) - e;
    const float sp = fmaf(__builtin_amdgcn_logf(u1), kLn2, fmaxf(s, 0.f) - c);
    const float phi = sp + 1e-6f;
    const float lp = __builtin_amdgcn_logf(phi);  // log2(phi)
    const float w = __builtin_amdgcn_exp2f(hc.tau * lp) * Z;
    const float sig = (s >= 0.f ? 1.f : e) * __builtin_amdgcn_rcpf(u1);  // sigmoid(s)
    const float dw = w * (dp - D);
    g = dw * hc.tau * sig * __builtin_amdgcn_rcpf(phi);
    lt = dw * lp;
    a = 0.f;
  }
}

// The forward's weight of one pair (as pair_weight) together with the factor
// the dK wave's gradient score needs from the same evaluation, so that the
// map runs once per pair in attn_bwd_kv:
//   Yat     mult = u r:                  A/2 = (dp - D) Z mult, g/2 = A/2 (1 + mult);
//   softmax mult = w:                    g = mult (dp - D);
//   s^tau   mult = w tau sigmoid(s)/phi: g = mult (dp - D).
template <int VAR>
__device__ __forceinline__ float pair_weight_mult(float sd, float Z, float nqk, const HeadC& hc,
                                                  float& mult) {
  if constexpr (is_yat(VAR)) {
    const float rden = __builtin_amdgcn_rcpf(yat_den(sd, nqk, hc.eps));
    const float ur = sd * rden;
    mult = ur;
    return sd * ur * Z;
  } else if constexpr (VAR == kSoftmax) {
    const float w = __builtin_amdgcn_exp2f(fmaf(sd, hc.c_sm, -Z));
    mult = w;
    return w;
  } else {
    const float s = sd * hc.scale;
    const float e = __builtin_amdgcn_exp2f(-fabsf(s) * kLog2e);
    const float u1 = 1.f + e;
    const float c = (u1 - 1.f) - e;
    const float sp = fmaf(__builtin_amdgcn_logf(u1), kLn2, fmaxf(s, 0.f) - c);
    const float phi = sp + 1e-6f;
    const float w = __builtin_amdgcn_exp2f(hc.tau * __builtin_amdgcn_logf(phi)) * Z;
    const float sig = (s >= 0.f ? 1.f : e) * __builtin_amdgcn_rcpf(u1);  // sigmoid(s)
    mult = w * hc.tau * sig * __builtin_amdgcn_rcpf(phi);
    return w;
  }
}
// The gradient score from that factor; Yat returns g/2 and sets a = A/2.
template <int VAR>
__device__ __forceinline__ float grad_from_mult(float mult, float dp, float D, float Z,
                                                float& a) {
  if constexpr (is_yat(VAR)) {
    a = (dp - D) * Z * mult;
    return fmaf(a, mult, a);
  } else {
    a = 0.f;
    return mult * (dp - D);
  }
}

// ---------------------------------------------------------------------------
// dK, dV: 8 waves in 4 pairs; pair p owns keys k0 + 32 p .. k0 + 32 p + 31 of
// one (b, kv head) and streams 32-query tiles of every query head of the
// group.  Wave p ("A") holds the pair's key rows and the dV^T accumulator;
// wave p + 4 ("B") holds the value rows and the dK^T accumulator.  Each
// keeps one row fragment and one accumulator, which is what lets two waves
// share a SIMD without spilling, and each issues 16 of a tile's 32 MFMAs.
// The two are pipelined one tile apart, one barrier per tile:
//
//   iteration t:  A: dV^T += dO_t^T P_t (P_t in its registers), S_{t+1} =
//                    Q_{t+1} K^T, the weights P_{t+1} -> registers and, per
//                    pair, the factor of B's gradient score -> LDS
//                 B: dP_t = dO_t V^T, the factors of tile t <- LDS, gradient
//                    scores, dK^T += Q^T G
//
// so on each SIMD one wave's matrix-core work overlaps the other's vector
// work, and the score -> weight map is evaluated once per pair (B's terms
// are two or three products of A's factor).  Tiles live in three LDS stages: tile t is read in iteration t (and
// its Q rows already in t - 1), tile t + 2 is written in iteration t from
// registers loaded in iteration t - 1.
template <int VAR, int DK, int DV>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512),
                          amdgpu_waves_per_eu(2, 2))) void attn_bwd_kv(BwdProblem p) {
  constexpr int NP = 4, NT = 128 * NP, BK = 32 * NP, BQ = 32, NS = 3;
  constexpr int KS = DK / 16, VS = DV / 16, FS = KS > VS ? KS : VS;
  constexpr int DKP = DK < 32 ? 32 : DK, DVP = DV < 32 ? 32 : DV;
  constexpr int KB = DKP / 32, VB = DVP / 32, AB = KB > VB ? KB : VB;
  constexpr int QLD = DK + 8, OLD = DV + 8;
  constexpr int Q_UNITS = (BQ / 4) * (DK / 8), O_UNITS = (BQ / 4) * (DV / 8);
  constexpr int UNITS = Q_UNITS + O_UNITS;
  constexpr int PER_T = (UNITS + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) unsigned short sQ[NS][BQ * QLD];
  __shared__ __attribute__((aligned(16))) unsigned short sO[NS][BQ * OLD];
  __shared__ __attribute__((aligned(16))) float sD[NS][BQ];
  __shared__ __attribute__((aligned(16))) float sZ[NS][BQ];
  __shared__ __attribute__((aligned(16))) float sNQ[NS][BQ];
  __shared__ f32x4 sS[2][NP][4][64];  // score tiles, in A's register layout

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const bool is_a = w < NP;
  const int trq = tr_lane_off(lane, QLD, DK), tro = tr_lane_off(lane, OLD, DV);
  const int pr = w & (NP - 1);
  // Workgroup -> (key tile, batch, kv head), heads fastest.  With a causal
  // mask the first key tiles have the most queries and go first.  (Grouping
  // heads per XCD as the forward does measured 1 % slower here.)
  const int nbh = p.B * p.Hkv;
  const int kt = blockIdx.x / nbh;
  const int bh = blockIdx.x - kt * nbh;
  const int b = bh / p.Hkv, hk = bh - b * p.Hkv;
  const int g = p.Hq / p.Hkv;
  const int k0 = kt * BK, kw = k0 + 32 * pr, my_k = kw + col;

  const unsigned short* kbase =
      (const unsigned short*)p.k + (int64_t)b * p.ks[0] + (int64_t)hk * p.ks[1];
  const unsigned short* vbase =
      (const unsigned short*)p.v + (int64_t)b * p.vs[0] + (int64_t)hk * p.vs[1];
  const uint32_t q_bytes = slice_bytes(p.Tq, p.qs[2], DK);
  const uint32_t o_bytes = slice_bytes(p.Tq, p.os[2], DV);
  const int qst = (int)p.qs[2], ost = (int)p.os[2];

  // A: this lane's key row, the B operand of S = Q K^T; B: its value row,
  // the B operand of dP = dO V^T.
  bf16x8 frag[FS];
  {
    const uint32_t k_bytes = slice_bytes(p.Tk, p.ks[2], DK);
    const uint32_t v_bytes = slice_bytes(p.Tk, p.vs[2], DV);
    const rsrc_t r = is_a ? make_rsrc(kbase, k_bytes) : make_rsrc(vbase, v_bytes);
    const int64_t rs = is_a ? p.ks[2] : p.vs[2];
    const uint32_t lim = is_a ? k_bytes : v_bytes;
    const uint32_t off = my_k < p.Tk ? (uint32_t)((my_k * rs + 8 * half) * 2) : lim;
#pragma unroll
    for (int s = 0; s < FS; ++s)
      if (s < (is_a ? KS : VS)) frag[s] = __builtin_bit_cast(bf16x8, ld128(r, off + 32 * s));
  }

  const int n_qt = (p.Tq + BQ - 1) / BQ;
  const int qt0 = p.causal ? k0 / BQ : 0;  // causal: T_q == T_k, so qt0 < n_qt
  const int per_head = n_qt - qt0;
  const int n_it = g * per_head;           // 0 when T_q == 0: only zeros are stored
  const int64_t qpitch = nk_pitch(p.Tq);
  // A, Yat: |k|^2 + b of this lane's key for the head being mapped
  float nk = 0.f;
  auto load_nk = [&](int gi) {
    if (is_yat(VAR) && my_k < p.Tk)
      nk = p.nk[((int64_t)b * p.Hq + hk * g + gi) * nk_pitch(p.Tk) + my_k];
  };

  // Tile it covers query head hk * g + it / per_head, query tile
  // qt0 + it % per_head; the loops below step these instead of dividing.
  struct Pos {
    int gi, qt;
  };
  auto advance = [&](Pos& x) {
    if (++x.qt == n_qt) {
      x.qt = qt0;
      ++x.gi;
    }
  };

  // Staging registers for a query tile.
  u32x4 st[PER_T][4];
  float st_d = 0.f, st_z = 0.f, st_nq = 0.f;
  auto load = [&](Pos x) {
    const int h = hk * g + x.gi, qb = x.qt * BQ;
    const rsrc_t rq = make_rsrc((const unsigned short*)p.q + (int64_t)b * p.qs[0] +
                                    (int64_t)h * p.qs[1], q_bytes);
    const rsrc_t ro = make_rsrc((const unsigned short*)p.dout + (int64_t)b * p.os[0] +
                                    (int64_t)h * p.os[1], o_bytes);
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int u = tid + i * NT;
      if (u < Q_UNITS) {
        const int g4 = u % (BQ / 4), c = u / (BQ / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = qb + 4 * g4 + r;
          st[i][r] = ld128(rq, row < p.Tq ? (uint32_t)((row * qst + 8 * c) * 2) : q_bytes);
        }
      } else if (u < UNITS) {
        const int u2 = u - Q_UNITS;
        const int g4 = u2 % (BQ / 4), c = u2 / (BQ / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = qb + 4 * g4 + r;
          st[i][r] = ld128(ro, row < p.Tq ? (uint32_t)((row * ost + 8 * c) * 2) : o_bytes);
        }
      }
    }
    if (tid < BQ) {
      const int64_t idx = ((int64_t)b * p.Hq + h) * qpitch + qb + tid;
      st_d = p.row_d[idx];
      st_z = p.row_z[idx];
      if (is_yat(VAR)) st_nq = p.nq[idx];
    }
  };
  // 4 rows x 8 columns -> 4 rows of the row-major tile (rows permuted)
  auto put = [&](const u32x4* rows, int g4, int c, unsigned short* R, int ld) {
#pragma unroll
    for (int r = 0; r < 4; ++r) *(u32x4*)&R[k_lds_row(4 * g4 + r) * ld + 8 * c] = rows[r];
  };
  auto store = [&](int slot) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int u = tid + i * NT;
      if (u < Q_UNITS) {
        put(st[i], u % (BQ / 4), u / (BQ / 4), sQ[slot], QLD);
      } else if (u < UNITS) {
        const int u2 = u - Q_UNITS;
        put(st[i], u2 % (BQ / 4), u2 / (BQ / 4), sO[slot], OLD);
      }
    }
    if (tid < BQ) {
      sD[slot][tid] = st_d;
      sZ[slot][tid] = st_z;
      sNQ[slot][tid] = st_nq;
    }
  };
  // a tile whose every query precedes every key of this pair: nothing to do
  auto active = [&](int qt) { return !(p.causal && qt * BQ + BQ - 1 < kw); };
  auto needs_mask = [&](int qb) { return (p.causal && qb < kw + 32) || qb + BQ > p.Tq; };

  // A: dV^T; B: dK^T (rows are value / key columns, the keys are the columns)
  f32x16 acc[AB];
#pragma unroll
  for (int i = 0; i < AB; ++i) acc[i] = f32x16{};
  // B, Yat: sums over the lane's queries of bf16(g/2) and of A/2; their
  // difference is the sum of B'/2 = bf16(g/2) - A/2
  float corr = 0.f, asum = 0.f;
  HeadC hc{};        // A: constants of query head hk g + hc_gi, the head last mapped
  int hc_gi = -1;

  // A: S = Q K^T of the tile in `slot`, its weights packed to bf16 into pk
  // and B's factors into sS[ss].  Masked pairs get weight and factor 0.
  auto weights = [&](auto mask_tag, int slot, int ss, int qb, u32x4* pk) {
    constexpr bool MASK = decltype(mask_tag)::value;
    f32x16 sacc = {};
    if (is_yat(VAR)) {
      // the chain starts at b (see pair_weight), from a scalar for every tile
      int bb = __builtin_amdgcn_readfirstlane(__float_as_int(hc.bias));
      asm volatile("" : "+s"(bb));
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = __int_as_float(bb);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sacc = mfma32(__builtin_bit_cast(bf16x8, *(const u32x4*)&sQ[slot][col * QLD + 16 * s + 8 * half]),
                    frag[s], sacc);
    f32x16 mult;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // accumulator elements 8 s .. 8 s + 7: queries qb + 16 s + 8 half + 0..7
      const int q8 = 16 * s + 8 * half;
      f32x4 n0 = {0.f, 0.f, 0.f, 0.f}, n1 = n0;
      const f32x4 z0 = *(const f32x4*)&sZ[slot][q8], z1 = *(const f32x4*)&sZ[slot][q8 + 4];
      if (is_yat(VAR)) {
        n0 = *(const f32x4*)&sNQ[slot][q8];
        n1 = *(const f32x4*)&sNQ[slot][q8 + 4];
      }
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float v[2];
#pragma unroll
        for (int o = 0; o < 2; ++o) {
          const int e = 2 * e2 + o, r = 8 * s + e;
          const float Z = e < 4 ? z0[e] : z1[e - 4];
          const float nq = e < 4 ? n0[e] : n1[e - 4];
          float m;
          v[o] = pair_weight_mult<VAR>(sacc[r], Z, nq + nk, hc, m);
          if (MASK) {
            const int qi = qb + q8 + e;
            const bool ok = qi < p.Tq && !(p.causal && my_k > qi);
            v[o] = ok ? v[o] : 0.f;
            m = ok ? m : 0.f;
          }
          mult[r] = m;
        }
        pk[s][e2] = pack_bf16(v[0], v[1]);
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
      sS[ss][pr][m][lane] = f32x4{mult[4 * m], mult[4 * m + 1], mult[4 * m + 2], mult[4 * m + 3]};
  };
  // A: dV^T += dO^T P of the tile in `slot`.
  auto dv_update = [&](int slot, const u32x4* pk) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 bop = __builtin_bit_cast(bf16x8, pk[s]);
#pragma unroll
      for (int i = 0; i < VB; ++i)
        acc[i] = mfma32(tr_frag_at(sO[slot] + tro, OLD, 32 * i, s), bop, acc[i]);
    }
  };
  // B: dP of the tile in `slot`, A's factors from sS[ss], the gradient scores
  // G and dK^T += Q^T G.  (Masked pairs have factor 0, hence G = 0.)
  auto grads = [&](int slot, int ss) {
    f32x16 pacc = {};
#pragma unroll
    for (int s = 0; s < VS; ++s)
      pacc = mfma32(__builtin_bit_cast(bf16x8, *(const u32x4*)&sO[slot][col * OLD + 16 * s + 8 * half]),
                    frag[s], pacc);
    f32x16 mult;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x4 x = sS[ss][pr][m][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) mult[4 * m + e] = x[e];
    }
    u32x4 pk[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int q8 = 16 * s + 8 * half;
      const f32x4 d0 = *(const f32x4*)&sD[slot][q8], d1 = *(const f32x4*)&sD[slot][q8 + 4];
      f32x4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = z0;
      if (is_yat(VAR)) {
        z0 = *(const f32x4*)&sZ[slot][q8];
        z1 = *(const f32x4*)&sZ[slot][q8 + 4];
      }
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float v[2], av[2];
#pragma unroll
        for (int o = 0; o < 2; ++o) {
          const int e = 2 * e2 + o, r = 8 * s + e;
          const float D = e < 4 ? d0[e] : d1[e - 4];
          const float Z = e < 4 ? z0[e] : z1[e - 4];
          v[o] = grad_from_mult<VAR>(mult[r], pacc[r], D, Z, av[o]);
        }
        pk[s][e2] = pack_bf16(v[0], v[1]);
        if (is_yat(VAR)) {
          corr = add_bf16_pair(pk[s][e2], corr);
          asum += av[0] + av[1];
        }
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 bop = __builtin_bit_cast(bf16x8, pk[s]);
#pragma unroll
      for (int i = 0; i < KB; ++i)
        acc[i] = mfma32(tr_frag_at(sQ[slot] + trq, QLD, 32 * i, s), bop, acc[i]);
    }
  };
  // A: S, weights and factors of the tile at `x` in `slot`
  auto map_tile = [&](Pos x, int slot, int ss, u32x4* pk) {
    const int qb = x.qt * BQ;
    if (needs_mask(qb)) weights(std::true_type{}, slot, ss, qb, pk);
    else weights(std::false_type{}, slot, ss, qb, pk);
  };

  // Prologue: tiles 0 and 1 into their stages, tile 2 into registers; A maps
  // tile 0.
  Pos cur{0, qt0};       // tile it
  Pos nxt = cur;         // tile it + 1
  Pos ld = cur;          // next tile to load
  u32x4 pk_cur[2] = {};  // A: P of tile it in bf16
  if (n_it > 0) {
    load(ld);
    store(0);
    advance(ld);
    if (n_it > 1) {
      load(ld);
      store(1);
      advance(ld);
    }
    if (n_it > 2) {
      load(ld);
      advance(ld);
    }
  }
  advance(nxt);
  __syncthreads();
  if (n_it > 0 && is_a && active(cur.qt)) {
    hc = head_consts<VAR, DK>(p, hk * g + cur.gi);
    hc_gi = cur.gi;
    load_nk(cur.gi);
    map_tile(cur, 0, 0, pk_cur);
  }
  __syncthreads();
  // Every load issued so far has landed (vmcnt 0).  Without this wait the
  // compiler cannot tell at the loop head that the fragments in `frag` are
  // complete (on the path with no tiles the prologue waits for nothing), and
  // makes each score or dP MFMA of the loop wait for all loads in flight,
  // including the staging loads issued earlier in the same iteration.
  __builtin_amdgcn_s_waitcnt(0x0f70);

  for (int it = 0; it < n_it; ++it) {
    const int slot = it % NS;
    // stage (it + 2) % 3 was last read in iteration it - 1
    if (it + 2 < n_it) store((it + 2) % NS);
    if (it + 3 < n_it) {
      load(ld);
      advance(ld);
    }
    const bool act = active(cur.qt);
    if (is_a) {
      if (act) dv_update(slot, pk_cur);
      if (it + 1 < n_it && active(nxt.qt)) {
        if (nxt.gi != hc_gi) {
          hc = head_consts<VAR, DK>(p, hk * g + nxt.gi);
          hc_gi = nxt.gi;
          load_nk(nxt.gi);
          // as before the loop: |k|^2 + b lands here, so that the maps of
          // the other iterations do not wait for the staging loads
          if (is_yat(VAR)) __builtin_amdgcn_s_waitcnt(0x0f70);
        }
        u32x4 pk_nxt[2];
        map_tile(nxt, (it + 1) % NS, (it + 1) & 1, pk_nxt);
        pk_cur[0] = pk_nxt[0];
        pk_cur[1] = pk_nxt[1];
      }
    } else if (act) {
      grads(slot, it & 1);
    }
    cur = nxt;
    advance(nxt);
    __syncthreads();
  }

  if (my_k < p.Tk) {
    if (is_a) {
      unsigned short* dvrow = (unsigned short*)p.dv_ + (int64_t)b * p.vs[0] +
                              (int64_t)hk * p.vs[1] + (int64_t)my_k * p.vs[2];
      // accumulator element 4 g4 + e of block i: row 32 i + 8 g4 + 4 half + e
#pragma unroll
      for (int i = 0; i < VB; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = 32 * i + 8 * g4 + 4 * half;
          if (d0 < DV) {
            u32x2 o;
            o[0] = pack_bf16(acc[i][4 * g4], acc[i][4 * g4 + 1]);
            o[1] = pack_bf16(acc[i][4 * g4 + 2], acc[i][4 * g4 + 3]);
            *(u32x2*)&dvrow[d0] = o;
          }
        }
    }
  }
  if (!is_a) {
    if (is_yat(VAR)) corr = 2.f * pair_sum(corr - asum);  // the kernel carries g/2 and A/2
    if (my_k < p.Tk) {
      unsigned short* dkrow = (unsigned short*)p.dk_ + (int64_t)b * p.ks[0] +
                              (int64_t)hk * p.ks[1] + (int64_t)my_k * p.ks[2];
      const unsigned short* krow = kbase + (int64_t)my_k * p.ks[2];
      const float sc = is_yat(VAR) ? 2.f : 1.0f / sqrtf((float)DK);
#pragma unroll
      for (int i = 0; i < KB; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = 32 * i + 8 * g4 + 4 * half;
          if (d0 < DK) {
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = acc[i][4 * g4 + e] * sc;
            if (is_yat(VAR)) {
              const u32x2 kk = *(const u32x2*)&krow[d0];
              x[0] -= corr * bf16_lo(kk[0]);
              x[1] -= corr * bf16_hi(kk[0]);
              x[2] -= corr * bf16_lo(kk[1]);
              x[3] -= corr * bf16_hi(kk[1]);
            }
            u32x2 o;
            o[0] = pack_bf16(x[0], x[1]);
            o[1] = pack_bf16(x[2], x[3]);
            *(u32x2*)&dkrow[d0] = o;
          }
        }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ and the parameter sums: 4 waves x 32 query rows; 32-key tiles.
//
// DELTA = true is a pass of its own before the gradient kernels: the same
// score tiles give D_i = sum_j w_ij dp_ij in fp32 from the weights as this
// file computes them.  In exact arithmetic D_i = dout_i . out_i, but the
// stored bf16 output is off by about 2^-9 |dp|, and every gradient score of
// the row carries that error through (dp - D): where the exact gradient
// cancels (a row whose weight sits on one key: dp - D = dp (1 - w), w ~ 1)
// it would be left at 2^-9 of the terms, and for Yat it is multiplied by
// d ln(kappa) / d q = 2 k / (q.k + b) - 2 (q - k) / den, unbounded where
// q.k + b -> 0.  With D from the same fp32 weights the cancellation is exact
// up to fp32 rounding.
template <int VAR, int DK, int DV, bool DELTA>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(2, 2))) void attn_bwd_q(BwdProblem p) {
  constexpr int NW = 4, NT = 64 * NW, BM = 32 * NW, BN = 32;
  static_assert(BM == kBwdQRows, "query rows per workgroup");
  constexpr int KS = DK / 16, VS = DV / 16;
  constexpr int DKP = DK < 32 ? 32 : DK;
  constexpr int KB = DKP / 32;
  constexpr int KLD = DK + 8, VLD = DV + 8;
  constexpr int K_UNITS = (BN / 4) * (DK / 8), V_UNITS = (BN / 4) * (DV / 8);
  constexpr int UNITS = K_UNITS + V_UNITS;
  constexpr int PER_T = (UNITS + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) unsigned short sK[2][BN * KLD];
  __shared__ __attribute__((aligned(16))) unsigned short sV[2][BN * VLD];
  __shared__ __attribute__((aligned(16))) float sNK[2][BN];
  __shared__ float sPrm[NW][2];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int trk = tr_lane_off(lane, KLD, DK);
  const int n_qt = (p.Tq + BM - 1) / BM;
  const int nbh = p.B * p.Hq;
  int qt = blockIdx.x / nbh;
  const int bh = blockIdx.x - qt * nbh;
  if (p.causal) qt = n_qt - 1 - qt;  // longest rows first
  const int b = bh / p.Hq, h = bh - b * p.Hq;
  const int hk = h / (p.Hq / p.Hkv);
  const int q0 = qt * BM, qw = q0 + 32 * w, my_q = qw + col;

  const unsigned short* qbase =
      (const unsigned short*)p.q + (int64_t)b * p.qs[0] + (int64_t)h * p.qs[1];
  const unsigned short* obase =
      (const unsigned short*)p.dout + (int64_t)b * p.os[0] + (int64_t)h * p.os[1];
  const uint32_t q_bytes = slice_bytes(p.Tq, p.qs[2], DK);
  const uint32_t o_bytes = slice_bytes(p.Tq, p.os[2], DV);
  const uint32_t k_bytes = slice_bytes(p.Tk, p.ks[2], DK);
  const uint32_t v_bytes = slice_bytes(p.Tk, p.vs[2], DV);
  const rsrc_t rk = make_rsrc((const unsigned short*)p.k + (int64_t)b * p.ks[0] +
                                  (int64_t)hk * p.ks[1], k_bytes);
  const rsrc_t rv = make_rsrc((const unsigned short*)p.v + (int64_t)b * p.vs[0] +
                                  (int64_t)hk * p.vs[1], v_bytes);
  const int kst = (int)p.ks[2], vst = (int)p.vs[2];

  // This lane's query and output-gradient rows: B operands of S^T and dP^T.
  bf16x8 qf[KS], of[VS];
  {
    const rsrc_t rq = make_rsrc(qbase, q_bytes);
    const rsrc_t ro = make_rsrc(obase, o_bytes);
    const uint32_t qo = my_q < p.Tq ? (uint32_t)(((int64_t)my_q * p.qs[2] + 8 * half) * 2)
                                    : q_bytes;
    const uint32_t oo = my_q < p.Tq ? (uint32_t)(((int64_t)my_q * p.os[2] + 8 * half) * 2)
                                    : o_bytes;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(bf16x8, ld128(rq, qo + 32 * s));
#pragma unroll
    for (int s = 0; s < VS; ++s) of[s] = __builtin_bit_cast(bf16x8, ld128(ro, oo + 32 * s));
  }
  float D = 0.f, Z = 0.f, nq = 0.f;
  const int64_t row_idx = ((int64_t)b * p.Hq + h) * nk_pitch(p.Tq) + my_q;
  if (my_q < p.Tq) {
    const int64_t idx = row_idx;
    if (!DELTA) D = p.row_d[idx];
    // the Yat and s^tau D pass forms the normaliser itself (below): its
    // weights are then kappa or phi^tau
    Z = DELTA && VAR != kSoftmax ? 1.f : p.row_z[idx];
    if (is_yat(VAR)) nq = p.nq[idx];
  }
  const HeadC hc = head_consts<VAR, DK>(p, h);
  const float* nk_slice =
      is_yat(VAR) ? p.nk + ((int64_t)b * p.Hq + h) * nk_pitch(p.Tk) : nullptr;  // |k|^2 + b
  const int b_bits = __builtin_amdgcn_readfirstlane(__float_as_int(hc.bias));

  const int kend = p.causal ? min(p.Tk, q0 + BM) : p.Tk;
  const int n_tiles = (kend + BN - 1) / BN;

  u32x4 st[PER_T][4];
  f32x4 st_nk = {0.f, 0.f, 0.f, 0.f};
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int u = tid + i * NT;
      if (u < K_UNITS) {
        const int g4 = u % (BN / 4), c = u / (BN / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = k0 + 4 * g4 + r;
          st[i][r] = ld128(rk, row < p.Tk ? (uint32_t)((row * kst + 8 * c) * 2) : k_bytes);
        }
      } else if (u < UNITS) {
        const int u2 = u - K_UNITS;
        const int g4 = u2 % (BN / 4), c = u2 / (BN / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = k0 + 4 * g4 + r;
          st[i][r] = ld128(rv, row < p.Tk ? (uint32_t)((row * vst + 8 * c) * 2) : v_bytes);
        }
      }
    }
    // the |k|^2 slice is padded to a multiple of 64 rows
    if (is_yat(VAR) && tid < BN / 4) st_nk = *(const f32x4*)(nk_slice + k0 + 4 * tid);
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int u = tid + i * NT;
      if (u < K_UNITS) {
        const int g4 = u % (BN / 4), c = u / (BN / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *(u32x4*)&sK[buf][k_lds_row(4 * g4 + r) * KLD + 8 * c] = st[i][r];
      } else if (u < UNITS) {
        const int u2 = u - K_UNITS;
        const int g4 = u2 % (BN / 4), c = u2 / (BN / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *(u32x4*)&sV[buf][k_lds_row(4 * g4 + r) * VLD + 8 * c] = st[i][r];
      }
    }
    if (is_yat(VAR) && tid < BN / 4) *(f32x4*)&sNK[buf][4 * tid] = st_nk;
  };

  f32x16 accQ[KB];
#pragma unroll
  for (int i = 0; i < KB; ++i) accQ[i] = f32x16{};
  float corr = 0.f;            // Yat: sum over the lane's keys of bf16(g/2) (minus sum0 below:
                               // the sum of B'/2 = bf16(g/2) - A/2)
  float sum0 = 0.f, sum1 = 0.f;  // Yat: sum A/2, sum B/2; s^tau: sum w (dp - D) log2(phi)
  float dsum = 0.f;            // DELTA: sum over the lane's keys of w dp (Yat: kappa dp)
  float msum = 0.f;            // DELTA, Yat, s^tau: sum over the lane's keys of kappa or phi^tau

  // Scores of one tile -> packed gradient scores (pg) and the row sums.
  auto scores = [&](auto mask_tag, int buf, int k0, u32x4* pg) {
    constexpr bool MASK = decltype(mask_tag)::value;
    f32x16 sacc = {}, pacc = {};
    if (is_yat(VAR)) {
      // the score chain starts at b (see pair_weight), rebuilt from a scalar
      // for every tile rather than held in 16 registers
      int bb = b_bits;
      asm volatile("" : "+s"(bb));
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = __int_as_float(bb);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sacc = mfma32(__builtin_bit_cast(bf16x8, *(const u32x4*)&sK[buf][col * KLD + 16 * s + 8 * half]),
                    qf[s], sacc);
#pragma unroll
    for (int s = 0; s < VS; ++s)
      pacc = mfma32(__builtin_bit_cast(bf16x8, *(const u32x4*)&sV[buf][col * VLD + 16 * s + 8 * half]),
                    of[s], pacc);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // accumulator elements 8 s .. 8 s + 7: keys k0 + 16 s + 8 half + 0..7
      const int k8 = 16 * s + 8 * half;
      f32x4 n0 = {0.f, 0.f, 0.f, 0.f}, n1 = n0;
      if (is_yat(VAR)) {
        n0 = *(const f32x4*)&sNK[buf][k8];
        n1 = *(const f32x4*)&sNK[buf][k8 + 4];
      }
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float gv[2], av[2], lv[2];
#pragma unroll
        for (int o = 0; o < 2; ++o) {
          const int e = 2 * e2 + o, r = 8 * s + e;
          const float nkv = e < 4 ? n0[e] : n1[e - 4];
          const int kj = k0 + k8 + e;
          const bool ok = !MASK || (my_q < p.Tq && kj < p.Tk && !(p.causal && kj > my_q));
          if (DELTA) {
            const float wv = ok ? pair_weight<VAR>(sacc[r], Z, nq + nkv, hc) : 0.f;
            dsum = fmaf(wv, pacc[r], dsum);
            if (VAR != kSoftmax) msum += wv;
            gv[o] = av[o] = lv[o] = 0.f;
          } else {
            pair_grad<VAR>(sacc[r], pacc[r], D, Z, nq + nkv, hc, gv[o], av[o], lv[o]);
            gv[o] = ok ? gv[o] : 0.f;
            av[o] = ok ? av[o] : 0.f;
            lv[o] = ok ? lv[o] : 0.f;
          }
        }
        if (DELTA) continue;
        pg[s][e2] = pack_bf16(gv[0], gv[1]);
        if (is_yat(VAR)) {
          // (g/2 and A/2: the sums are doubled where they are used)
          corr = add_bf16_pair(pg[s][e2], corr);
          sum0 += av[0] + av[1];
          sum1 += lv[0] + lv[1];
        } else if (VAR == kStau) {
          sum0 += lv[0] + lv[1];
        }
      }
    }
  };
  // dQ^T += K^T G^T (queries are the columns)
  auto accumulate = [&](int buf, const u32x4* pg) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 bg = __builtin_bit_cast(bf16x8, pg[s]);
#pragma unroll
      for (int i = 0; i < KB; ++i)
        accQ[i] = mfma32(tr_frag_at(sK[buf] + trk, KLD, 32 * i, s), bg, accQ[i]);
    }
  };

  // Staging as in attn_bwd_kv: tile t + 1 is written at the start of
  // iteration t, tile t + 2 loaded after iteration t's scores.
  if (n_tiles > 0) {
    load(0);
    store(0);
    if (n_tiles > 1) load(BN);
  }
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = t * BN, buf = t & 1;
    if (t + 1 < n_tiles) store(buf ^ 1);
    const bool active = !(p.causal && k0 > qw + 31);
    u32x4 pg[2];
    if (active) {
      const bool need_mask = (p.causal && k0 + BN - 1 > qw) || k0 + BN > p.Tk || qw + 32 > p.Tq;
      if (need_mask) scores(std::true_type{}, buf, k0, pg);
      else scores(std::false_type{}, buf, k0, pg);
    }
    if (t + 2 < n_tiles) load(k0 + 2 * BN);
    if (active && !DELTA) accumulate(buf, pg);
    __syncthreads();
  }

  if (DELTA) {
    dsum = pair_sum(dsum);
    if (is_yat(VAR)) {
      // Z = 1 / (sum_j kappa_ij + 1e-9) from these same kappa, so that a row's
      // weights add to mass / (mass + 1e-9) in this evaluation's rounding and
      // dp - D cancels where the exact gradient does (a row whose weight sits
      // on one key), whatever rounding the forward's kappa took
      const float z = 1.f / (pair_sum(msum) + 1e-9f);
      if (my_q < p.Tq && half == 0) {
        p.row_z[row_idx] = z;
        p.row_d[row_idx] = dsum * z;
      }
    } else if (VAR == kStau) {
      // Z = 1 / sum_j phi^tau from these same weights: the forward's mass
      // carries that kernel's own rounding (it takes log2(1 + t) from a
      // polynomial), which would otherwise scale every weight here and enter
      // the parameter sum through dp - D
      const float m = pair_sum(msum);
      const float z = m > 0.f ? 1.f / m : 0.f;
      if (my_q < p.Tq && half == 0) {
        p.row_z[row_idx] = z;
        p.row_d[row_idx] = dsum * z;
      }
    } else if (my_q < p.Tq && half == 0) {
      p.row_d[row_idx] = dsum;
    }
    return;
  }

  if (is_yat(VAR)) corr = 2.f * pair_sum(corr - sum0);  // the kernel carries g/2 and A/2
  if (my_q < p.Tq) {
    unsigned short* dqrow = (unsigned short*)p.dq + (int64_t)b * p.qs[0] +
                            (int64_t)h * p.qs[1] + (int64_t)my_q * p.qs[2];
    const unsigned short* qrow = qbase + (int64_t)my_q * p.qs[2];
    const float sc = is_yat(VAR) ? 2.f : 1.0f / sqrtf((float)DK);
#pragma unroll
    for (int i = 0; i < KB; ++i)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * i + 8 * g4 + 4 * half;
        if (d0 < DK) {
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = accQ[i][4 * g4 + e] * sc;
          if (is_yat(VAR)) {
            const u32x2 qq = *(const u32x2*)&qrow[d0];
            x[0] -= corr * bf16_lo(qq[0]);
            x[1] -= corr * bf16_hi(qq[0]);
            x[2] -= corr * bf16_lo(qq[1]);
            x[3] -= corr * bf16_hi(qq[1]);
          }
          u32x2 o;
          o[0] = pack_bf16(x[0], x[1]);
          o[1] = pack_bf16(x[2], x[3]);
          *(u32x2*)&dqrow[d0] = o;
        }
      }
  }

  // parameter sums of the workgroup: wave reduction, then the waves in order
  if (VAR != kSoftmax && p.prm_part) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      sum0 += __shfl_xor(sum0, m, 64);
      sum1 += __shfl_xor(sum1, m, 64);
    }
    if (lane == 0) {
      sPrm[w][0] = sum0;
      sPrm[w][1] = sum1;
    }
    __syncthreads();
    if (tid < 2) {
      double a = 0.0;
#pragma unroll
      for (int i = 0; i < NW; ++i) a += (double)sPrm[i][tid];
      p.prm_part[(((int64_t)h * p.B + b) * n_qt + qt) * 2 + tid] = a;
    }
  }
}

// Yat: (|x_j|^2 + b_h) 2^-96 for every row of the key or query slice that
// query head h reads (x head h / (Hq / Hx)), by the same MFMA sequence and
// start value b as the score chains (the scaling is the one yat_den takes).
// One wave per 32 rows; grid (ceil(T / 128), Hq, B), 256 threads; output
// [B][Hq][nk_pitch(T)].
template <int DK>
__global__ __launch_bounds__(256) void norms_plus_bias_bf16(const unsigned short* x, int64_t s0,
                                                            int64_t s1, int64_t s2, int Hx,
                                                            int T, int Hq, const float* b_raw,
                                                            float* out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int b = blockIdx.z, h = blockIdx.y, hx = h / (Hq / Hx);
  const int row = blockIdx.x * 128 + 32 * w + col;
  const unsigned short* base = x + (int64_t)b * s0 + (int64_t)hx * s1;
  const uint32_t bytes = slice_bytes(T, s2, DK);
  const rsrc_t r = make_rsrc(base, bytes);
  const uint32_t off = row < T ? (uint32_t)(((int64_t)row * s2 + 8 * half) * 2) : bytes;
  // the row's loads first: b's parameter load and softplus run under them
  u32x4 xr[DK / 16];
#pragma unroll
  for (int s = 0; s < DK / 16; ++s) xr[s] = ld128(r, off + 32 * s);
  const float bias = softplus_precise(b_raw[h]);  // as head_consts forms it
  f32x16 g;
#pragma unroll
  for (int i = 0; i < 16; ++i) g[i] = bias;
#pragma unroll
  for (int s = 0; s < DK / 16; ++s)
    g = mfma32(__builtin_bit_cast(bf16x8, xr[s]), __builtin_bit_cast(bf16x8, xr[s]), g);
  if (row < T && holds_diag(col, half))
    out[((int64_t)b * Hq + h) * nk_pitch(T) + row] = diag_of(g, col) * kNormScale;
}

template <int VAR, int DV>
hipError_t launch_bwd_variant(const BwdProblem& p, hipStream_t stream) {
  constexpr int DK = SFS_DK;
  if (is_yat(VAR) && p.Tq > 0) {
    hipLaunchKernelGGL(norms_plus_bias_bf16<DK>, dim3((p.Tk + 127) / 128, p.Hq, p.B), dim3(256),
                       0, stream, (const unsigned short*)p.k, p.ks[0], p.ks[1], p.ks[2], p.Hkv,
                       p.Tk, p.Hq, p.b_raw, p.nk);
    hipLaunchKernelGGL(norms_plus_bias_bf16<DK>, dim3((p.Tq + 127) / 128, p.Hq, p.B), dim3(256),
                       0, stream, (const unsigned short*)p.q, p.qs[0], p.qs[1], p.qs[2], p.Hq,
                       p.Tq, p.Hq, p.b_raw, p.nq);
  }
  const unsigned n_q = (unsigned)((p.Tq + kBwdQRows - 1) / kBwdQRows) * (unsigned)p.B *
                       (unsigned)p.Hq;
  // D_i in fp32 from the weights (see attn_bwd_q)
  if (p.Tq > 0)
    hipLaunchKernelGGL((attn_bwd_q<VAR, DK, DV, true>), dim3(n_q), dim3(256), 0, stream, p);
  const unsigned n_kv = (unsigned)((p.Tk + 127) / 128) * (unsigned)p.B * (unsigned)p.Hkv;
  hipLaunchKernelGGL((attn_bwd_kv<VAR, DK, DV>), dim3(n_kv), dim3(512), 0, stream, p);
  if (p.Tq == 0) return hipGetLastError();  // dk = dv = 0 written; no query rows
  hipLaunchKernelGGL((attn_bwd_q<VAR, DK, DV, false>), dim3(n_q), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int VAR>
hipError_t launch_bwd_dv(const BwdProblem& p, hipStream_t stream) {
  switch (p.dv) {
    case 16: return launch_bwd_variant<VAR, 16>(p, stream);
    case 32: return launch_bwd_variant<VAR, 32>(p, stream);
    case 64: return launch_bwd_variant<VAR, 64>(p, stream);
    case 128: return launch_bwd_variant<VAR, 128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t SFS_CAT(launch_bwd_bf16_dk, SFS_DK)(const BwdProblem& p, hipStream_t stream) {
  switch (p.variant) {
    case kSoftmax: return launch_bwd_dv<kSoftmax>(p, stream);
    case kYat: return launch_bwd_dv<kYat>(p, stream);
    case kStau: return launch_bwd_dv<kStau>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace sfs
