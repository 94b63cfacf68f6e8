// bf16_common.h -- device helpers shared by the bf16 kernel translation
// units (forward, telemetry and backward): vector types, buffer loads, the
// 32x32x16 bf16 MFMA, bf16 packing, the row layout of score tiles in LDS and
// the |x|^2 pre-pass.  Every item has internal linkage in each unit.
#pragma once

#include "attn_launch.h"

namespace sfs {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Buffer-resource word 3 for raw (unformatted) dword access on gfx9.
constexpr int kRsrcWord3 = 0x00020000;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}
__device__ __forceinline__ u32x4 ld128(rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;  // round to nearest even
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(unsigned, v);
}
// Yat's denominator max(d2, 0) + eps in two instructions.  The row terms
// |q|^2 + b and |k|^2 + b are kept scaled by 2^-96 (exact: a power of two), so
// y = 2^-96 d2 comes from one FMA whose result the clamp modifier limits to
// [0, 1], and y 2^96 + eps is one more FMA with a single rounding: the same
// value as max(d2, 0) + eps computed unscaled, ties (d2 = 0) included.  Limits:
// d2 is capped at 2^96, and d2 below 2^-30 loses bits (denormal y); neither
// changes the denominator unless eps is below ~1e-15 or |q|^2 + |k|^2 exceeds
// the range where (q.k + b)^2 is finite.
constexpr float kNormScale = 0x1p-96f;
__device__ __forceinline__ float yat_den(float u, float nqk_scaled, float eps) {
  const float y = __builtin_amdgcn_fmed3f(fmaf(u, -2.f * kNormScale, nqk_scaled), 0.f, 1.f);
  return fmaf(y, 0x1p96f, eps);
}

// Map constants held in scalar registers.  -2 kNormScale, 2^96, the s^tau
// floor and the score scale are not inline constants, so an instruction
// would otherwise carry each as a 32-bit literal, which halves its issue rate;
// a scalar register operand costs nothing (one per instruction).
// The s^tau floor 1e-6 in base-2 units (see stau_weight2 below).
constexpr float kStauFloor2 = 1e-6f * kLog2e;
struct MapConsts {
  float m2s;    // -2 kNormScale
  float k96;    // 2^96
  float floor2; // kStauFloor2
  float c_sm;   // log2(e) / sqrt(d_k)
  unsigned ones;  // the bf16 pair (1, 1)
};
__device__ __forceinline__ MapConsts map_consts(float c_sm) {
  MapConsts c{-2.f * kNormScale, 0x1p96f, kStauFloor2, c_sm, 0x3f803f80u};
  // opaque to constant folding: the values stay in scalar registers
  asm volatile("" : "+s"(c.m2s), "+s"(c.k96), "+s"(c.floor2), "+s"(c.c_sm), "+s"(c.ones));
  return c;
}
__device__ __forceinline__ float yat_den(float u, float nqk_scaled, float eps,
                                         const MapConsts& mc) {
  const float y = __builtin_amdgcn_fmed3f(fmaf(u, mc.m2s, nqk_scaled), 0.f, 1.f);
  return fmaf(y, mc.k96, eps);
}

// s^tau ("s^tau" forum post, core formula): phi = softplus(s) + 1e-6 and the
// weight phi^tau, here in base-2 units.  With y = s log2(e) + c0 (c0 the floor
// 1e-6 in the same units),
//   Z = phi / ln 2 = max(y, c0) + log2(1 + 2^-|y|),
// which moves the floor into the fma that forms y (2^-|y| then differs from
// 2^-|s log2 e| by a relative 1e-6 at most).  With t = 2^-|y| in (0, 1],
// log2(1 + t) = t P(t), P a degree-4 polynomial for log2(1 + t) / t on [0, 1]
// that is minimax in relative error (Lawson's algorithm; the fit is
// softmax_free_score_amd/stau_poly.py): relative error below 5.7e-5 with fp32
// Horner (tau times that in the weight, well inside the 2^-9 rounding the
// weights take for the value MFMA), and t P(t) keeps that relative precision
// for small t, where
// Z ~ c0 + t / ln 2.  The weight returned is Z^tau = phi^tau / (ln 2)^tau: the
// constant factor of a head cancels in the normalised output; stau_unit gives
// it for the mass.  Three transcendentals: exp2, log2, exp2.
struct StauPoly {
  float c0, c1, c2, c3, c4;
};
__device__ __forceinline__ StauPoly stau_poly() {
  StauPoly s{1.4426132440567017f, -0.7169874310493469f, 0.44189882278442383f,
             -0.22711941599845886f, 0.05965153127908707f};
  // scalar registers rather than 32-bit literals, as MapConsts above
  asm("" : "+s"(s.c0), "+s"(s.c1), "+s"(s.c2), "+s"(s.c3), "+s"(s.c4));
  return s;
}
// x: the raw score q.k; mc.c_sm = log2(e) / sqrt(d_k).
__device__ __forceinline__ float stau_weight2(float x, float tau, const MapConsts& mc,
                                             const StauPoly& sp) {
  const float y = fmaf(x, mc.c_sm, mc.floor2);
  const float t = __builtin_amdgcn_exp2f(-fabsf(y));
  float l = fmaf(sp.c4, t, sp.c3);
  l = fmaf(l, t, sp.c2);
  l = fmaf(l, t, sp.c1);
  l = fmaf(l, t, sp.c0);
  const float z = fmaf(l, t, fmaxf(y, mc.floor2));
  return __builtin_amdgcn_exp2f(tau * __builtin_amdgcn_logf(z));
}
// (ln 2)^tau: stau_weight2 times this is phi^tau
__device__ __forceinline__ float stau_unit(float tau) {
  return exp2f(tau * -0.52876637294031f);  // log2(ln 2)
}

// acc + the two bf16 halves of x, in fp32, one instruction (v_dot2 with ones)
__device__ __forceinline__ float add_bf16_pair(unsigned x, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), ones, acc, false);
}
// The same with the pair of ones from a scalar register.
__device__ __forceinline__ float add_bf16_pair(unsigned x, float acc, const MapConsts& mc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x),
                                         __builtin_bit_cast(bf16x2, mc.ones), acc, false);
}
// Two bf16 words from two packed pairs, one byte permute each: the low
// halves of a and b (a's in the low half of the result), or the high halves.
__device__ __forceinline__ unsigned lo_halves(unsigned a, unsigned b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ unsigned hi_halves(unsigned a, unsigned b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
// log(1 + e^x) without overflow (fp32 library calls; used once per head).
__device__ __forceinline__ float softplus_precise(float x) {
  return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}
// Byte size of a (b, h) slice with rows of `d` elements at `row_stride`.
__device__ __forceinline__ uint32_t slice_bytes(int rows, int64_t row_stride, int d) {
  return (uint32_t)(((int64_t)(rows - 1) * row_stride + d) * 2);
}
// Row position inside a 32-row block of the K tile in LDS: bits 2 and 3 swapped.
__device__ __forceinline__ int k_lds_row(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}
// Diagonal of the 32x32 accumulator of X X^T: column n = col sits in the lane
// half (col >> 2) & 1, element 4 (col >> 3) + (col & 3).
__device__ __forceinline__ bool holds_diag(int col, int half) { return ((col >> 2) & 1) == half; }
__device__ __forceinline__ float diag_of(const f32x16& g, int col) {
  const int r = 4 * (col >> 3) + (col & 3);
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) d = (i == r) ? g[i] : d;
  return d;
}

// |k_j|^2 for every key row, by the same MFMA sequence as the score tile.
// One wave per 32 rows; grid (ceil(T/128), H, B), 256 threads.
template <int DK>
__global__ __launch_bounds__(256) void row_norms_bf16(const unsigned short* x, int64_t s0,
                                                      int64_t s1, int64_t s2, int H, int T,
                                                      float* out) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int b = blockIdx.z, h = blockIdx.y;
  const int row = blockIdx.x * 128 + 32 * w + col;
  const unsigned short* base = x + (int64_t)b * s0 + (int64_t)h * s1;
  const uint32_t bytes = slice_bytes(T, s2, DK);
  const rsrc_t r = make_rsrc(base, bytes);
  const uint32_t off = row < T ? (uint32_t)(((int64_t)row * s2 + 8 * half) * 2) : bytes;
  f32x16 g = {};
#pragma unroll
  for (int s = 0; s < DK / 16; ++s)
    g = mfma32(__builtin_bit_cast(bf16x8, ld128(r, off + 32 * s)),
               __builtin_bit_cast(bf16x8, ld128(r, off + 32 * s)), g);
  if (row < T && holds_diag(col, half))
    out[((int64_t)b * H + h) * nk_pitch(T) + row] = diag_of(g, col);
}

// Partner-lane exchange for row statistics: lanes l and l ^ 32 hold the same
// query.  v_permlane32_swap hands every lane both halves' values.
__device__ __forceinline__ float pair_sum(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)s[0]) + __builtin_bit_cast(float, (unsigned)s[1]);
}
__device__ __forceinline__ float pair_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)s[0]), __builtin_bit_cast(float, (unsigned)s[1]));
}

}  // namespace
}  // namespace sfs
