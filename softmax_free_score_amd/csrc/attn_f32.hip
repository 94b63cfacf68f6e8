// attn_f32.hip -- attention forward for fp32 storage on gfx950 (vector ALU).
//
// Same three maps as the bf16 path (see attn_bf16.hip for the formulas and
// the pages they come from), evaluated in fp32 with IEEE division and the
// accurate library exp/log/pow, for callers that keep fp32 tensors.  On
// MI355X the fp32 matrix-core rate equals the fp32 vector rate, so this path
// stays on the vector ALU.
//
// One workgroup (one wave) per query row.  Keys are taken 64 at a time, one
// per lane: each lane forms its score with a sequential fma chain over d (and
// |k|^2 with the same chain, so a key equal to its query cancels exactly in
// the Yat distance), maps it to a weight, and the wave then accumulates the
// weighted value rows with lanes over d_v.
#include "attn_launch.h"

namespace sfs {
namespace {

__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

template <int VAR>
__global__ __launch_bounds__(64) void attn_fwd_f32(Problem p) {
  __shared__ float sQ[128];
  __shared__ float sP[64];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;  // (b*Hq + h)*Tq + i
  const int i = (int)(row % p.Tq);
  const int bh = (int)(row / p.Tq);
  const int h = bh % p.Hq, b = bh / p.Hq;
  const int hk = h / (p.Hq / p.Hkv);
  const int dk = p.dk, dv = p.dv;
  const float* qrow = (const float*)p.q + (int64_t)b * p.qs[0] + (int64_t)h * p.qs[1] +
                      (int64_t)i * p.qs[2];
  const float* kb = (const float*)p.k + (int64_t)b * p.ks[0] + (int64_t)hk * p.ks[1];
  const float* vb = (const float*)p.v + (int64_t)b * p.vs[0] + (int64_t)hk * p.vs[1];

  for (int d = lane; d < dk; d += 64) sQ[d] = qrow[d];
  __syncthreads();

  float bias = 0.f, eps = 0.f, tau = 0.f, nq = 0.f;
  if (is_yat(VAR)) {
    bias = p.yat_bias_free ? 0.f : softplus_f(p.b_raw[h]);
    eps = softplus_f(p.eps_raw[h]);
    for (int d = 0; d < dk; ++d) nq = fmaf(sQ[d], sQ[d], nq);
  } else if (VAR == kStau) {
    tau = softplus_f(p.log_tau[h]) + 1.f;
  }
  const float scale = 1.0f / sqrtf((float)dk);
  const int n_keys = p.causal ? i + 1 : p.Tk;

  float o0 = 0.f, o1 = 0.f;  // value columns lane and lane + 64
  float mass = 0.f;          // per-lane partial (softmax: relative to m)
  float m = -INFINITY;       // softmax: running max of s; Yat/s^tau: lane max
  for (int k0 = 0; k0 < n_keys; k0 += 64) {
    const int j = k0 + lane;
    const bool allowed = j < n_keys;
    float s = 0.f, nk = 0.f;
    if (allowed) {
      const float* kr = kb + (int64_t)j * p.ks[2];
      for (int d = 0; d < dk; ++d) {
        const float x = kr[d];
        s = fmaf(sQ[d], x, s);
        nk = fmaf(x, x, nk);
      }
    }
    float w = 0.f;
    if (is_yat(VAR)) {
      if (allowed) {
        const float d2 = fmaf(-2.f, s, nq + nk);
        const float u = s + bias;
        w = yat_numerator<VAR>(u, p.yat_power) / (fmaxf(d2, 0.f) + eps);
        m = fmaxf(m, w);
      }
      mass += w;
    } else if (VAR == kStau) {
      if (allowed) {
        const float sc = s * scale;
        w = powf(softplus_f(sc) + 1e-6f, tau);
        m = fmaxf(m, sc);
      }
      mass += w;
    } else {
      const float sc = allowed ? s * scale : -INFINITY;
      const float mnew = fmaxf(m, wave_max(sc));
      const float alpha = expf(m - mnew);  // m = -inf on the first chunk: 0
      o0 *= alpha;
      o1 *= alpha;
      mass *= alpha;
      m = mnew;
      w = allowed ? expf(sc - m) : 0.f;
      mass += w;
    }
    sP[lane] = w;
    __syncthreads();
    const int nj = min(64, n_keys - k0);
    for (int jj = 0; jj < nj; ++jj) {
      const float* vr = vb + (int64_t)(k0 + jj) * p.vs[2];
      const float pj = sP[jj];
      if (lane < dv) o0 = fmaf(pj, vr[lane], o0);
      if (lane + 64 < dv) o1 = fmaf(pj, vr[lane + 64], o1);
    }
    __syncthreads();
  }

  const float mass_all = wave_sum(mass);
  const float mx = VAR == kSoftmax ? m : wave_max(m);
  float inv;
  if (is_yat(VAR)) inv = 1.f / (mass_all + 1e-9f);
  else if (VAR == kSoftmax) inv = 1.f / mass_all;
  else inv = mass_all > 0.f ? 1.f / mass_all : 0.f;
  float* orow = (float*)p.out + (int64_t)b * p.os[0] + (int64_t)h * p.os[1] + (int64_t)i * p.os[2];
  if (lane < dv) orow[lane] = o0 * inv;
  if (lane + 64 < dv) orow[lane + 64] = o1 * inv;
  if (lane == 0) {
    if (p.mass) p.mass[row] = mass_all;
    if (p.max_score) p.max_score[row] = mx;
  }
}

}  // namespace

hipError_t launch_f32(const Problem& p, hipStream_t stream) {
  const unsigned n = (unsigned)((int64_t)p.B * p.Hq * p.Tq);
  switch (p.variant) {
    case kSoftmax: hipLaunchKernelGGL(attn_fwd_f32<kSoftmax>, dim3(n), dim3(64), 0, stream, p); break;
    case kYat:
      if (p.yat_power > 1)
        hipLaunchKernelGGL(attn_fwd_f32<kYatPow>, dim3(n), dim3(64), 0, stream, p);
      else
        hipLaunchKernelGGL(attn_fwd_f32<kYat>, dim3(n), dim3(64), 0, stream, p);
      break;
    case kStau: hipLaunchKernelGGL(attn_fwd_f32<kStau>, dim3(n), dim3(64), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sfs
