// attn_decode.hip -- the forward for few query rows per key/value head
// (decode: one new query row per head against a long key cache), on the
// vector ALU.
//
// Compiled once per key width: -DSFS_DK=16|32|64|128.
//
// The matrix-core kernels tile 64 or more query rows per workgroup; with one
// row per head almost all of that work is padding, and it, not HBM, sets the
// time.  Here the g query heads that share a key/value head and their T_q
// rows (at most kDecodeRows together) are packed into one workgroup of four
// waves, which reads each key and value row of its 256-key chunk once, with
// every load coalesced (d/8 lanes x 16 bytes per row; a wave's key loads for
// its 64 keys are all issued at the start, its value loads after phase 1):
//   phase 1: lane (key sub-row kk = lane / (d_k/8), column block cb) forms
//            partial dot products of 8 columns with every packed query row
//            (broadcast from LDS) and the d_k/8 lanes of a key add them with
//            a fixed xor-shuffle tree; the map's weight goes to LDS;
//   phase 2: per-row maximum and mass over the chunk (fixed-order reductions);
//   phase 3: O = sum_j w_j v_j with the same lane split over value columns,
//            two keys per v_dot2 (bf16 weights), the four key sub-rows added
//            by shuffles and the waves in LDS.
// Each chunk writes unnormalised partials (O, mass, maximum, softmax
// reference maximum) in the layout of the key-split path, and combine_partials
// merges them.  Maps as in attn_bf16.hip ("Softmax-Free Attention in JAX/Flax
// NNX", "One module, two compatibility functions"; "NNX Scaled Dot-Product
// Attention", displayed equation; the "s^tau" forum post, core formula).
// |q|^2, |k|^2 and q.k are formed by the same per-lane v_dot2 order on the
// bf16 pairs and the same shuffle tree, so for a key equal to its query
// d2 = |q|^2 + |k|^2 - 2 q.k is exactly 0.
#include "bf16_common.h"

#ifndef SFS_DK
#error "compile with -DSFS_DK=16, 32, 64 or 128"
#endif

#define SFS_CAT2(a, b) a##b
#define SFS_CAT(a, b) SFS_CAT2(a, b)

namespace sfs {
namespace {

constexpr int kChunk = 256;  // keys per workgroup

// Key and value rows are read once per call: streaming (non-temporal) loads.
__device__ __forceinline__ u32x4 ld128_stream(rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2);
}

// Sum over the N (2, 4, 8 or 16) lanes of an aligned group with DPP moves:
// swap neighbours, swap pairs, then mirror within 8 and within 16 lanes.
// Each step adds two equal-sized partial sums, so every lane of the group
// ends with the same bits, and the tree is the same for every call.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                             0xf, 0xf, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror
  return x;
}
// Partial dot product of 8 bf16 columns held as 4 packed pairs (column 2e in
// the low half): one v_dot2_f32_bf16 per pair, pairs in column order, fp32
// accumulation.
__device__ __forceinline__ float dot8(const unsigned* a, const unsigned* b) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a[e]),
                                        __builtin_bit_cast(bf16x2, b[e]), s, false);
  return s;
}

// NR: packed rows the instantiation holds (1, 2, 4 or 8; R <= NR rows used).
template <int VAR, int DK, int DV, int NR>
__global__ __launch_bounds__(256) void attn_decode_bf16(Problem p) {
  constexpr int NT = 256, NW = NT / 64;
  constexpr int CB = DK / 8;            // 8-column blocks of a key row (<= 16)
  constexpr int KPI = 64 / CB;          // key rows per wave instruction
  constexpr int KIT = 64 / KPI;         // instructions for a wave's 64 keys
  constexpr int VB = DV / 8;            // 8-column blocks of a value row
  constexpr int VPI = 64 / VB;
  constexpr int VIT = 64 / VPI;
  __shared__ __attribute__((aligned(16))) unsigned sQ[NR][DK / 2];  // bf16 pairs
  __shared__ float sC[NR][4];           // |q|^2, b (Yat) / tau (s^tau), eps
  __shared__ float sP[NR][kChunk];      // weights of the chunk (softmax: exponent first)
  __shared__ float sRed[NW][NR][2];
  __shared__ float sStat[NR][2];        // mass, max
  __shared__ float sO[NW][NR][DV];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int chunk = blockIdx.x, S = gridDim.x;
  const int bh = blockIdx.y;
  const int b = bh / p.Hkv, hk = bh - b * p.Hkv;
  const int g = p.Hq / p.Hkv;
  const int R = g * p.Tq;  // packed rows, <= NR (checked on the host)
  const int j0 = chunk * kChunk;
  const float scale = 1.0f / sqrtf((float)DK);
  const int kk = lane / CB, cb = lane % CB;  // key sub-row, column block (phase 1)

  // Query rows into LDS as bf16 pairs; row r is query head hk g + r / T_q,
  // row r % T_q.
  for (int idx = tid; idx < R * DK / 2; idx += NT) {
    const int r = idx / (DK / 2), d = 2 * (idx - r * (DK / 2));
    const int h = hk * g + r / p.Tq, i = r - (r / p.Tq) * p.Tq;
    const unsigned short* qrow = (const unsigned short*)p.q + (int64_t)b * p.qs[0] +
                                 (int64_t)h * p.qs[1] + (int64_t)i * p.qs[2];
    sQ[r][d / 2] = (unsigned)qrow[d] | ((unsigned)qrow[d + 1] << 16);
  }

  // Issue this wave's key loads: instruction t covers keys j0 + 64 w + KPI t
  // + kk, columns 8 cb .. 8 cb + 7.
  const unsigned short* kbase =
      (const unsigned short*)p.k + (int64_t)b * p.ks[0] + (int64_t)hk * p.ks[1];
  const uint32_t k_bytes = slice_bytes(p.Tk, p.ks[2], DK);
  const rsrc_t rk = make_rsrc(kbase, k_bytes);
  u32x4 kr[KIT];
#pragma unroll
  for (int t = 0; t < KIT; ++t) {
    const int j = j0 + 64 * w + KPI * t + kk;
    kr[t] = ld128_stream(rk, j < p.Tk ? (uint32_t)(((int64_t)j * p.ks[2] + 8 * cb) * 2) : k_bytes);
  }
  __syncthreads();
  if (w == 0) {
    // |q|^2 of every packed row, by the same partial order and tree as q.k
    for (int r = kk; r < R; r += KPI) {
      const float nq = group_sum<CB>(dot8(&sQ[r][4 * cb], &sQ[r][4 * cb]));
      if (cb == 0) sC[r][0] = nq;
    }
    if (lane < R) {
      const int h = hk * g + lane / p.Tq;
      if (is_yat(VAR)) {
        sC[lane][1] = p.yat_bias_free ? 0.f : softplus_precise(p.b_raw[h]);
        sC[lane][2] = softplus_precise(p.eps_raw[h]);
      } else if (VAR == kStau) {
        sC[lane][1] = softplus_precise(p.log_tau[h]) + 1.f;
      }
    }
  }
  __syncthreads();

  // this lane's 8 columns (4 bf16 pairs) of every packed query row
  unsigned qf[NR][4];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) qf[r][e] = r < R ? sQ[r][4 * cb + e] : 0u;

  // Phase 1: scores and weights of this wave's 64 keys.  After the shuffle
  // tree every one of a key's CB lanes holds its scores, so the map is spread
  // over them: lane cb evaluates rows cb, cb + CB, ... (RPL of them) instead
  // of every lane evaluating every row.
  constexpr int RPL = (NR + CB - 1) / CB;
  float mx[RPL], rnq[RPL], rc1[RPL], rc2[RPL];
  int rqi[RPL];
#pragma unroll
  for (int q = 0; q < RPL; ++q) {
    const int rr = cb + q * CB, rc = rr < R ? rr : 0;  // rows >= R: any valid row, unused
    mx[q] = -INFINITY;
    rnq[q] = sC[rc][0];
    rc1[q] = sC[rc][1];
    rc2[q] = sC[rc][2];
    rqi[q] = rc - (rc / p.Tq) * p.Tq;
  }
#pragma unroll
  for (int t = 0; t < KIT; ++t) {
    const int jl = 64 * w + KPI * t + kk, j = j0 + jl;
    unsigned kf[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) kf[e] = kr[t][e];
    const float nk = is_yat(VAR) ? group_sum<CB>(dot8(kf, kf)) : 0.f;
    float sc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) sc[r] = r < R ? group_sum<CB>(dot8(qf[r], kf)) : 0.f;
#pragma unroll
    for (int q = 0; q < RPL; ++q) {
      const int rr = cb + q * CB;
      float x = sc[0];
#pragma unroll
      for (int r = 1; r < NR; ++r) x = rr == r ? sc[r] : x;
      const bool ok = rr < R && j < p.Tk && !(p.causal && j > rqi[q]);
      float val, m;
      if (is_yat(VAR)) {
        const float d2 = fmaf(-2.f, x, rnq[q] + nk);
        const float kap = yat_numerator<VAR>(x + rc1[q], p.yat_power) *
                          __builtin_amdgcn_rcpf(fmaxf(d2, 0.f) + rc2[q]);
        val = ok ? kap : 0.f;
        m = ok ? kap : -INFINITY;
      } else if (VAR == kSoftmax) {
        const float xs = x * (scale * kLog2e);
        val = ok ? xs : -INFINITY;
        m = val;
      } else {
        const float s = x * scale;
        const float e = __builtin_amdgcn_exp2f(-fabsf(s) * kLog2e);
        const float u1 = 1.f + e;
        const float cc = (u1 - 1.f) - e;
        const float sp = fmaf(__builtin_amdgcn_logf(u1), kLn2, fmaxf(s, 0.f) - cc);
        const float u = __builtin_amdgcn_exp2f(rc1[q] * __builtin_amdgcn_logf(sp + 1e-6f));
        val = ok ? u : 0.f;
        m = ok ? s : -INFINITY;
      }
      if (rr < R) sP[rr][jl] = val;
      mx[q] = fmaxf(mx[q], m);
    }
  }
  // Value loads for phase 3, issued now so that they overlap phase 2:
  // instruction t covers keys 64 w + VPI t + lane / VB, columns 8 (lane % VB) .. + 7.
  const unsigned short* vbase =
      (const unsigned short*)p.v + (int64_t)b * p.vs[0] + (int64_t)hk * p.vs[1];
  const uint32_t v_bytes = slice_bytes(p.Tk, p.vs[2], DV);
  const rsrc_t rv = make_rsrc(vbase, v_bytes);
  const int vk = lane / VB, vc = lane % VB;
  u32x4 vr[VIT];
#pragma unroll
  for (int t = 0; t < VIT; ++t) {
    const int j = j0 + 64 * w + VPI * t + vk;
    vr[t] = ld128_stream(rv, j < p.Tk ? (uint32_t)(((int64_t)j * p.vs[2] + 8 * vc) * 2) : v_bytes);
  }

  // Phase 2: row maxima and masses over the chunk (waves in order).
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (r < R) {
      float m = -INFINITY;  // this lane's maximum of row r, if it maps row r
#pragma unroll
      for (int q = 0; q < RPL; ++q) m = cb + q * CB == r ? mx[q] : m;
#pragma unroll
      for (int sh = 1; sh < 64; sh <<= 1) m = fmaxf(m, __shfl_xor(m, sh, 64));
      if (lane == 0) sRed[w][r][0] = m;
    }
  }
  __syncthreads();
  if (tid < R) {
    float m = sRed[0][tid][0];
    for (int v = 1; v < NW; ++v) m = fmaxf(m, sRed[v][tid][0]);
    sStat[tid][1] = m;
  }
  __syncthreads();
  // softmax: exponentials against the chunk's maximum (a row whose keys are
  // all masked here keeps -inf and gets weights 0); then the masses
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (r < R) {
      float v = sP[r][tid];
      if (VAR == kSoftmax) {
        v = __builtin_amdgcn_exp2f(v - fmaxf(sStat[r][1], -3.0e38f));
        sP[r][tid] = v;
      }
#pragma unroll
      for (int sh = 1; sh < 64; sh <<= 1) v += __shfl_xor(v, sh, 64);
      if (lane == 0) sRed[w][r][1] = v;
    }
  }
  __syncthreads();
  if (tid < R) {
    float s = sRed[0][tid][1];
    for (int v = 1; v < NW; ++v) s += sRed[v][tid][1];
    sStat[tid][0] = s;
  }

  // Phase 3: O = sum_j w_j v_j over this wave's keys; lanes of one column
  // block (lane % VB) then add their key sub-rows, waves add in LDS.
  float o[NR][8];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[r][e] = 0.f;
  // Two keys at a time (instructions t and t + 1 hold keys jl and jl + VPI in
  // the same columns): each column's two values form one bf16 pair (one byte
  // permute), the two weights another (rounded to bf16, as the matrix-core
  // kernels weight the values), and one v_dot2 adds both products.
  static_assert(VIT % 2 == 0, "key pairs");
#pragma unroll
  for (int t = 0; t < VIT; t += 2) {
    const int jl = 64 * w + VPI * t + vk;
    unsigned vp[8];  // column 2e: (key jl, key jl + VPI) pairs, then column 2e + 1
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vp[2 * e] = lo_halves(vr[t][e], vr[t + 1][e]);
      vp[2 * e + 1] = hi_halves(vr[t][e], vr[t + 1][e]);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (r < R) {
        // 0 for keys past T_k (masked)
        const bf16x2 wp = __builtin_bit_cast(bf16x2, pack_bf16(sP[r][jl], sP[r][jl + VPI]));
#pragma unroll
        for (int e = 0; e < 8; ++e)
          o[r][e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, vp[e]), wp,
                                                    o[r][e], false);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (r < R) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = o[r][e];
        for (int sh = VB; sh < 64; sh <<= 1) x += __shfl_xor(x, sh, 64);
        if (vk == 0) sO[w][r][8 * vc + e] = x;
      }
    }
  }
  __syncthreads();

  // Partials of this chunk, in the key-split layout: O [S][rows][d_v] then
  // statistics [S][rows][4] (mass, max, reference max), rows = B Hq Tq.
  const int64_t Rtot = (int64_t)p.B * p.Hq * p.Tq;
  for (int idx = tid; idx < R * DV; idx += NT) {
    const int r = idx / DV, c = idx - r * DV;
    const int h = hk * g + r / p.Tq, i = r - (r / p.Tq) * p.Tq;
    const int64_t ri = ((int64_t)b * p.Hq + h) * p.Tq + i;
    float sum = 0.f;
    for (int v = 0; v < NW; ++v) sum += sO[v][r][c];
    p.part[((int64_t)chunk * Rtot + ri) * p.dv + c] = sum;
  }
  if (tid < R) {
    const int h = hk * g + tid / p.Tq, i = tid - (tid / p.Tq) * p.Tq;
    const int64_t ri = ((int64_t)b * p.Hq + h) * p.Tq + i;
    const f32x4 st = {sStat[tid][0], sStat[tid][1], sStat[tid][1], 0.f};
    *(f32x4*)&p.part[(int64_t)S * Rtot * p.dv + ((int64_t)chunk * Rtot + ri) * 4] = st;
  }
}

template <int VAR, int DV>
hipError_t launch_decode_dv(const Problem& p, const dim3& grid, hipStream_t stream) {
  constexpr int DK = SFS_DK;
  const int R = p.Hq / p.Hkv * p.Tq;
  if (R <= 1) hipLaunchKernelGGL((attn_decode_bf16<VAR, DK, DV, 1>), grid, dim3(256), 0, stream, p);
  else if (R <= 2) hipLaunchKernelGGL((attn_decode_bf16<VAR, DK, DV, 2>), grid, dim3(256), 0, stream, p);
  else if (R <= 4) hipLaunchKernelGGL((attn_decode_bf16<VAR, DK, DV, 4>), grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((attn_decode_bf16<VAR, DK, DV, kDecodeRows>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int VAR>
hipError_t launch_decode_variant(const Problem& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.kv_splits, (unsigned)(p.B * p.Hkv));
  switch (p.dv) {
    case 16: return launch_decode_dv<VAR, 16>(p, grid, stream);
    case 32: return launch_decode_dv<VAR, 32>(p, grid, stream);
    case 64: return launch_decode_dv<VAR, 64>(p, grid, stream);
    case 128: return launch_decode_dv<VAR, 128>(p, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t SFS_CAT(launch_decode_bf16_dk, SFS_DK)(const Problem& p, hipStream_t stream) {
  switch (p.variant) {
    case kSoftmax: return launch_decode_variant<kSoftmax>(p, stream);
    case kYat:
      return p.yat_power > 1 ? launch_decode_variant<kYatPow>(p, stream)
                             : launch_decode_variant<kYat>(p, stream);
    case kStau: return launch_decode_variant<kStau>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace sfs
