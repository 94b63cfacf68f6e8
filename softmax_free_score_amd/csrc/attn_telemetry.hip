// attn_telemetry.hip -- the telemetry pass of a finished bf16 forward
// (row entropy, row sparsity, per-head tau*), on the forward's score tiles.
//
// Compiled once per key width: -DSFS_DK=16|32|64|128.
#include "bf16_common.h"

#ifndef SFS_DK
#error "compile with -DSFS_DK=16, 32, 64 or 128"
#endif

#define SFS_CAT2(a, b) a##b
#define SFS_CAT(a, b) SFS_CAT2(a, b)

namespace sfs {
namespace {

// Telemetry pass over the score tiles of a finished forward (no values).
//
// With the forward's row normaliser (mass, and max_score for softmax) the
// weights of every allowed pair are recomputed exactly as the forward defines
// them (Yat: kappa rounded to bf16, s^tau: phi^tau / (ln 2)^tau rounded to
// bf16, as the tile kernels weight the values), and per row the pass
// accumulates sum w log2 w, the count of weights
// below the threshold and the count of allowed keys; per (head, batch, query
// tile) it accumulates the sums that give tau* = Cov(s, ln phi(s)) /
// Var(ln phi(s)) with s = q.k / sqrt(d_k), phi = softplus(s) + 1e-6 (the s^tau
// post's closed form), whatever the branch.  Entropy is normalised by ln n
// ("The Kernel Between the Roles", "The run": 0 for a row on one key, 1 for
// uniform weights).  64 query rows per workgroup (2 waves),
// 32-key tiles staged through LDS; the score tile and its layout are those of
// the forward.
template <int VAR, int DK>
__global__ __attribute__((amdgpu_flat_work_group_size(128, 128),
                          amdgpu_waves_per_eu(2, 2))) void attn_stats_bf16(Problem p) {
  constexpr int NW = 2, BM = 64, BN = 32, NT = 128;
  constexpr int KS = DK / 16;
  constexpr int KLD = DK + 8;
  constexpr int KCH = DK / 8;
  constexpr int K_UNITS = BN * KCH;
  constexpr int K_PER_T = (K_UNITS + NT - 1) / NT;
  static_assert(BM == kStatsRows, "rows per workgroup");

  __shared__ __attribute__((aligned(16))) unsigned short sK[2][BN * KLD];
  __shared__ __attribute__((aligned(16))) float sNK[2][BN];
  __shared__ float sNQ[BM];
  __shared__ float sTau[NW][6];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int n_qt = (p.Tq + BM - 1) / BM;
  const int nbh = p.B * p.Hq;
  const int qt = blockIdx.x / nbh;
  const int bh = blockIdx.x - qt * nbh;
  const int b = bh / p.Hq, h = bh - b * p.Hq;
  const int hk = h / (p.Hq / p.Hkv);
  const int q0 = qt * BM, qw = q0 + 32 * w, my_q = qw + col;

  const unsigned short* qbase =
      (const unsigned short*)p.q + (int64_t)b * p.qs[0] + (int64_t)h * p.qs[1];
  const unsigned short* kbase =
      (const unsigned short*)p.k + (int64_t)b * p.ks[0] + (int64_t)hk * p.ks[1];
  const uint32_t q_bytes = slice_bytes(p.Tq, p.qs[2], DK);
  const uint32_t k_bytes = slice_bytes(p.Tk, p.ks[2], DK);
  const rsrc_t rq = make_rsrc(qbase, q_bytes);
  const rsrc_t rk = make_rsrc(kbase, k_bytes);
  const int kst = (int)p.ks[2];

  float bias = 0.f, eps = 0.f, tau = 0.f;
  if (is_yat(VAR)) {
    bias = softplus_precise(p.b_raw[h]);
    eps = softplus_precise(p.eps_raw[h]);
  } else if (VAR == kStau) {
    tau = softplus_precise(p.log_tau[h]) + 1.f;
  }
  const float scale = 1.0f / sqrtf((float)DK);
  // s^tau: the tile kernels weight the values by phi^tau / (ln 2)^tau in bf16
  // and sum those for the mass; (ln 2)^tau brings them back to phi^tau
  const float tau_unit = VAR == kStau ? stau_unit(tau) : 1.f;
  constexpr float kLog2Ln2 = -0.52876637294031f;  // log2(ln 2)

  bf16x8 qf[KS];
  {
    const uint32_t off = my_q < p.Tq ? (uint32_t)(((int64_t)my_q * p.qs[2] + 8 * half) * 2)
                                     : q_bytes;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(bf16x8, ld128(rq, off + 32 * s));
    __builtin_amdgcn_s_waitcnt(0);
  }
  float nq = 0.f;
  const float* nk_slice =
      is_yat(VAR) ? p.nk + ((int64_t)b * p.Hkv + hk) * nk_pitch(p.Tk) : nullptr;
  if (is_yat(VAR)) {
    f32x16 g = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) g = mfma32(qf[s], qf[s], g);
    if (holds_diag(col, half)) sNQ[32 * w + col] = diag_of(g, col);
  }
  // this row's normaliser from the forward
  const int64_t ri = ((int64_t)b * p.Hq + h) * p.Tq + min(my_q, p.Tq - 1);
  const float row_mass = p.in_mass[ri];
  float inv_mass, xmax = 0.f;
  if (is_yat(VAR)) inv_mass = 1.f / (row_mass + 1e-9f);
  else inv_mass = row_mass > 0.f ? 1.f / row_mass : 0.f;
  if (VAR == kSoftmax) xmax = p.in_max[ri] * kLog2e;  // log2 units

  const int kend = p.causal ? min(p.Tk, q0 + BM) : p.Tk;
  const int n_tiles = (kend + BN - 1) / BN;

  u32x4 kreg[K_PER_T];
  f32x4 nkreg = {0.f, 0.f, 0.f, 0.f};
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int u = tid + i * NT;
      if (u < K_UNITS) {
        const int row = k0 + u / KCH, c = u % KCH;
        const uint32_t off = row < p.Tk ? (uint32_t)((row * kst + 8 * c) * 2) : k_bytes;
        kreg[i] = ld128(rk, off);
      }
    }
    if (is_yat(VAR) && tid < BN / 4) nkreg = *(const f32x4*)(nk_slice + k0 + 4 * tid);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int u = tid + i * NT;
      if (u < K_UNITS) {
        const int j = u / KCH, c = u % KCH;
        *(u32x4*)&sK[buf][k_lds_row(j) * KLD + 8 * c] = kreg[i];
      }
    }
    if (is_yat(VAR) && tid < BN / 4) *(f32x4*)&sNK[buf][4 * tid] = nkreg;
  };

  float ent = 0.f, n_sparse = 0.f, n_allowed = 0.f;  // per lane, this row (ent: sum w log2 w)
  float t_n = 0.f, t_s = 0.f, t_l = 0.f, t_ss = 0.f, t_ll = 0.f, t_sl = 0.f;  // tau sums

  load_tile(0);
  store_tile(0);
  if (n_tiles > 1) load_tile(BN);
  __syncthreads();
  if (is_yat(VAR)) nq = sNQ[32 * w + col];

  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = t * BN, buf = t & 1;
    if (!(p.causal && k0 > qw + 31)) {
      const unsigned short* K = sK[buf];
      f32x16 sacc = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, *(const u32x4*)&K[col * KLD + 16 * s + 8 * half]);
        sacc = mfma32(a, qf[s], sacc);
      }
      const f32x4 n0 = *(const f32x4*)&sNK[buf][8 * half];
      const f32x4 n1 = *(const f32x4*)&sNK[buf][8 * half + 4];
      const f32x4 n2 = *(const f32x4*)&sNK[buf][16 + 8 * half];
      const f32x4 n3 = *(const f32x4*)&sNK[buf][16 + 8 * half + 4];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 16 * (r >> 3) + 8 * half + (r & 7);
        const bool ok = !((p.causal && key > my_q) || key >= p.Tk) && my_q < p.Tq;
        const float sd = sacc[r];          // q.k
        const float s = sd * scale;        // the scaled score
        // log2 phi, phi = softplus(s) + 1e-6 as the forward's s^tau map forms
        // it: max(s, 0) + log1p(e^-|s|) with the rounding of 1 + e corrected
        const float e = __builtin_amdgcn_exp2f(-fabsf(s) * kLog2e);
        const float u1 = 1.f + e;
        const float c = (u1 - 1.f) - e;
        const float lp = __builtin_amdgcn_logf(
            fmaf(__builtin_amdgcn_logf(u1), kLn2, fmaxf(s, 0.f) - c) + 1e-6f);
        float wgt;
        if (is_yat(VAR)) {
          const float nkr = r < 4 ? n0[r] : r < 8 ? n1[r - 4] : r < 12 ? n2[r - 8] : n3[r - 12];
          const float d2 = fmaf(-2.f, sd, nq + nkr);
          const float u = sd + bias;
          // the tile kernels' value MFMA takes kappa in bf16, and their mass sums those
          const float kap =
              yat_numerator<VAR>(u, p.yat_power) * __builtin_amdgcn_rcpf(fmaxf(d2, 0.f) + eps);
          wgt = (float)(__bf16)kap * inv_mass;
        } else if (VAR == kSoftmax) {
          wgt = __builtin_amdgcn_exp2f(fmaf(sd, scale * kLog2e, -xmax)) * inv_mass;
        } else {
          const float zt = __builtin_amdgcn_exp2f(tau * (lp - kLog2Ln2));  // phi^tau / (ln 2)^tau
          wgt = (float)(__bf16)zt * tau_unit * inv_mass;
        }
        wgt = ok ? wgt : 0.f;
        // w log2 w (weights below the smallest normal float add nothing)
        ent += wgt >= 1.17549435e-38f ? wgt * __builtin_amdgcn_logf(wgt) : 0.f;
        n_sparse += ok && wgt < p.sparsity_threshold ? 1.f : 0.f;
        n_allowed += ok ? 1.f : 0.f;
        const float L = ok ? lp * kLn2 : 0.f;  // ln phi
        const float sm = ok ? s : 0.f;
        t_n += ok ? 1.f : 0.f;
        t_s += sm;
        t_l += L;
        t_ss = fmaf(sm, sm, t_ss);
        t_ll = fmaf(L, L, t_ll);
        t_sl = fmaf(sm, L, t_sl);
      }
    }
    if (t + 1 < n_tiles) {
      store_tile(buf ^ 1);
      if (t + 2 < n_tiles) load_tile(k0 + 2 * BN);
    }
    __syncthreads();
  }

  // rows: combine the two lanes of a query
  ent = pair_sum(ent);
  n_sparse = pair_sum(n_sparse);
  n_allowed = pair_sum(n_allowed);
  if (my_q < p.Tq && half == 0) {
    const int64_t r = ((int64_t)b * p.Hq + h) * p.Tq + my_q;
    if (p.row_entropy)
      p.row_entropy[r] = n_allowed > 1.f ? -ent * kLn2 / logf(n_allowed) : 0.f;  // ent in log2
    if (p.row_sparsity) p.row_sparsity[r] = n_sparse / n_allowed;
  }
  // tau sums of the workgroup: wave reduction, then the two waves in LDS
  if (p.tau_part) {
    float v6[6] = {t_n, t_s, t_l, t_ss, t_ll, t_sl};
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      float x = v6[i];
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
      v6[i] = x;
    }
    if (lane == 0)
#pragma unroll
      for (int i = 0; i < 6; ++i) sTau[w][i] = v6[i];
    __syncthreads();
    if (tid < 6) {
      double* dst = p.tau_part + (((int64_t)h * p.B + b) * n_qt + qt) * 8;
      dst[tid] = (double)sTau[0][tid] + (double)sTau[1][tid];
    }
  }
}

template <int VAR>
hipError_t launch_stats_variant(const Problem& p, hipStream_t stream) {
  constexpr int DK = SFS_DK;
  if (is_yat(VAR)) {
    const dim3 grid((p.Tk + 127) / 128, p.Hkv, p.B);
    hipLaunchKernelGGL(row_norms_bf16<DK>, grid, dim3(256), 0, stream,
                       (const unsigned short*)p.k, p.ks[0], p.ks[1], p.ks[2], p.Hkv, p.Tk, p.nk);
  }
  const unsigned n = (unsigned)((p.Tq + kStatsRows - 1) / kStatsRows) * (unsigned)p.B *
                     (unsigned)p.Hq;
  hipLaunchKernelGGL((attn_stats_bf16<VAR, DK>), dim3(n), dim3(128), 0, stream, p);
  return hipGetLastError();
}
}  // namespace

hipError_t SFS_CAT(launch_stats_bf16_dk, SFS_DK)(const Problem& p, hipStream_t stream) {
  switch (p.variant) {
    case kSoftmax: return launch_stats_variant<kSoftmax>(p, stream);
    case kYat: return launch_stats_variant<kYat>(p, stream);
    case kStau: return launch_stats_variant<kStau>(p, stream);
  }
  return hipErrorInvalidValue;
}
}  // namespace sfs
