// attn_combine.hip -- merges the key-chunk partials of the small-grid and decode kernels.
//
// When the keys of a workgroup are split into S chunks, chunk s of query row
// r leaves O_s (sum over its keys of w_j v_j, unnormalised), its mass m_s, its
// maximum score x_s and, for softmax, the reference maximum M_s its
// exponentials are taken against (O_s and m_s are relative to 2^M_s).
//
//   Yat, s^tau: the weights need no maximum, so the chunks add:
//               O = sum O_s, mass = sum m_s, max = max x_s
//               ("Softmax-Free Attention in JAX/Flax NNX", "One module, two
//               compatibility functions": out = O / (mass + 1e-9) for Yat;
//               s^tau forum post, core formula: out = O / mass).
//   softmax:    the log-sum-exp merge with M = max M_s:
//               O = sum 2^(M_s - M) O_s, l = sum 2^(M_s - M) m_s, out = O / l,
//               mass reported relative to the row maximum x = max x_s.
//
// One wave per row, chunks in batches of 32: a batch's statistics (one chunk
// per lane) and its partial O (lane c holds value columns c and c + 64) are
// loaded together, then the statistics are reduced across the wave and the
// partial O accumulated in chunk order.  Every reduction has a fixed order,
// so the result does not depend on scheduling.
#include "attn_launch.h"

namespace sfs {
namespace {

constexpr float kLn2c = 0.6931471805599453f;
typedef float f32x4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned short to_bf16(float x) {
  return __builtin_bit_cast(unsigned short, (__bf16)x);  // round to nearest even
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__global__ __launch_bounds__(256) void combine_partials(Problem p) {
  const int lane = threadIdx.x & 63;
  const int64_t R = (int64_t)p.B * p.Hq * p.Tq;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;  // whole waves
  const int S = p.kv_splits, dv = p.dv;
  const float* po = p.part;
  const float* ps = p.part + (int64_t)S * R * dv;

  // Chunks in batches of kBatch: every load of a batch -- the statistics of
  // chunk s0 + lane and the partial O of each chunk of the batch -- is issued
  // before any is used, so a batch costs one memory round trip.
  constexpr int kBatch = 32;
  float x = -INFINITY, M = -INFINITY, mass = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    const int nb = min(kBatch, S - s0);
    f32x4s st = {0.f, -INFINITY, -INFINITY, 0.f};
    if (lane < nb) st = *(const f32x4s*)(ps + ((int64_t)(s0 + lane) * R + r) * 4);
    float a0[kBatch], a1[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      a0[u] = a1[u] = 0.f;
      if (u < nb) {
        const float* row = po + ((int64_t)(s0 + u) * R + r) * dv;
        if (lane < dv) a0[u] = row[lane];
        if (lane + 64 < dv) a1[u] = row[lane + 64];
      }
    }
    // batch maxima; softmax rescales what the earlier batches summed
    const float xb = wave_max(st[1]), Mb = wave_max(st[2]);
    x = fmaxf(x, xb);
    float fo = 1.f;  // factor for the sums so far (softmax)
    if (p.variant == kSoftmax) {
      const float Mn = fmaxf(M, Mb);
      fo = M == -INFINITY ? 0.f : exp2f(M - Mn);
      M = Mn;
    }
    // lane l: the weight of chunk s0 + l
    float wgt = lane < nb ? 1.f : 0.f;
    if (p.variant == kSoftmax && lane < nb) wgt = st[2] == -INFINITY ? 0.f : exp2f(st[2] - M);
    mass = mass * fo + wave_sum(wgt * st[0]);
    o0 *= fo;
    o1 *= fo;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float wu = __shfl(wgt, u, 64);  // 0 past the last chunk
      o0 = fmaf(wu, a0[u], o0);
      o1 = fmaf(wu, a1[u], o1);
    }
  }
  float inv;
  if (is_yat(p.variant)) inv = 1.f / (mass + 1e-9f);
  else if (p.variant == kSoftmax) inv = 1.f / mass;
  else inv = mass > 0.f ? 1.f / mass : 0.f;

  const int64_t i = r % p.Tq, bh = r / p.Tq;
  const int64_t h = bh % p.Hq, b = bh / p.Hq;
  unsigned short* orow =
      (unsigned short*)p.out + b * p.os[0] + h * p.os[1] + i * p.os[2];
  if (lane < dv) orow[lane] = to_bf16(o0 * inv);
  if (lane + 64 < dv) orow[lane + 64] = to_bf16(o1 * inv);
  if (lane == 0) {
    // softmax: mass relative to the row maximum, max_score in natural units
    if (p.mass) p.mass[r] = p.variant == kSoftmax ? mass * exp2f(M - x) : mass;
    if (p.max_score) p.max_score[r] = p.variant == kSoftmax ? x * kLn2c : x;
  }
}

// tau* of query head h = blockIdx.x * 64 + lane from the per-(head, batch,
// query tile) sums of the telemetry pass, in a fixed order (the s^tau post:
// tau* = Cov(s, ln phi(s)) / Var(ln phi(s))).  NaN when Var = 0.
__global__ __launch_bounds__(64) void tau_star_kernel(Problem p, int n_qt) {
  const int h = blockIdx.x * 64 + threadIdx.x;
  if (h >= p.Hq) return;
  double a[6] = {0, 0, 0, 0, 0, 0};
  const double* src = p.tau_part + (int64_t)h * p.B * n_qt * 8;
  for (int64_t i = 0; i < (int64_t)p.B * n_qt; ++i)
    for (int j = 0; j < 6; ++j) a[j] += src[i * 8 + j];
  const double n = a[0];
  const double ms = a[1] / n, ml = a[2] / n;
  const double cov = a[5] / n - ms * ml;
  const double var = a[4] / n - ml * ml;
  p.tau_star[h] = var > 0.0 ? (float)(cov / var) : __builtin_nanf("");
}

}  // namespace

hipError_t launch_tau_star(const Problem& p, hipStream_t stream) {
  const int n_qt = (p.Tq + kStatsRows - 1) / kStatsRows;
  hipLaunchKernelGGL(tau_star_kernel, dim3((p.Hq + 63) / 64), dim3(64), 0, stream, p, n_qt);
  return hipGetLastError();
}

hipError_t launch_combine(const Problem& p, hipStream_t stream) {
  const int64_t R = (int64_t)p.B * p.Hq * p.Tq;
  hipLaunchKernelGGL(combine_partials, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sfs
