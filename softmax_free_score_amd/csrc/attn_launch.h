// attn_launch.h -- internal interface between the C ABI (attn_api.cpp) and
// the kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfs {

// kYatPow is internal: the Yat map with the numerator raised to a power
// m >= 2 (m = yat_power, a runtime value); kYat is the m = 1 kernel.
enum Variant : int { kSoftmax = 0, kYat = 1, kStau = 2, kYatPow = 3 };
__host__ __device__ constexpr bool is_yat(int v) { return v == kYat || v == kYatPow; }

// Yat numerator (s + b)^(2m) from u = s + b: u^2 for kYat, (u^2)^m for kYatPow.
template <int VAR>
__device__ __forceinline__ float yat_numerator(float u, int m) {
  const float u2 = u * u;
  if constexpr (VAR == kYatPow) {
    float num = u2;
    for (int i = 1; i < m; ++i) num *= u2;
    return num;
  } else {
    (void)m;
    return u2;
  }
}

// Row pitch (in floats) of the Yat |k|^2 workspace per (batch, kv head):
// T_k rounded up to 64, so a 64-key tile never reads past its slice.
__host__ __device__ inline int64_t nk_pitch(int64_t Tk) { return (Tk + 63) / 64 * 64; }

// Everything a launch needs, already validated by the ABI layer.  Offsets
// inside one (batch, head) slice fit in int32 (checked there); the per-slice
// base offsets are 64-bit.
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* mass;       // may be null
  float* max_score;  // may be null
  const float* b_raw;
  const float* eps_raw;
  const float* log_tau;
  float* nk;         // Yat: |k_j|^2 per key row [B*Hkv][nk_pitch(Tk)] (workspace)
  int64_t qs[3], ks[3], vs[3], os[3];  // element strides for (b, h, t)
  int B, Hq, Hkv, Tq, Tk, dk, dv;
  int variant;
  int causal;
  int block_rows;     // 0: choose by grid size; 64, 128, 256: force that kernel
  int yat_power;      // Yat numerator power m >= 1 ((s + b)^(2m))
  int yat_bias_free;  // Yat: b = 0 exactly (b_raw not read)
};

// Fused forward for fp32 storage (vector-ALU path).
hipError_t launch_f32(const Problem& p, hipStream_t stream);

// Per-dk launchers of the bf16 path: |k|^2 pre-pass (Yat) + fused forward on
// the matrix cores (one translation unit per d_k).
hipError_t launch_bf16_dk16(const Problem& p, hipStream_t stream);
hipError_t launch_bf16_dk32(const Problem& p, hipStream_t stream);
hipError_t launch_bf16_dk64(const Problem& p, hipStream_t stream);
hipError_t launch_bf16_dk128(const Problem& p, hipStream_t stream);

}  // namespace sfs
