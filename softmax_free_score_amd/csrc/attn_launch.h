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

// Work layout of the bf16 path, chosen on the host so that the workspace size
// and the launch agree.  rows: query rows per workgroup (256: ping-pong
// kernel; 128, 64: small-grid kernels).  splits: the keys of each workgroup
// are cut into this many chunks of whole tiles (small-grid kernels only);
// each chunk writes unnormalised partials that a combine kernel merges.
constexpr int kDeviceCUs = 256;
// Workgroup i of a grid of n_t tiles x n_s slices ((batch, head) pairs) runs
// on XCD i % kXcds, and each XCD has its own L2.  When the slices divide
// evenly, each XCD takes its slices in groups of kSliceGroup and runs a
// group's tiles together, slices fastest, so that its resident workgroups
// share a few slices' operands in L2; otherwise slices vary fastest over the
// whole grid.  t is the tile in dispatch order (0 first), s the slice.
constexpr int kXcds = 8, kSliceGroup = 4;
__device__ __forceinline__ void grid_tile_slice(int i, int n_t, int n_s, int& t, int& s) {
  if (n_s % (kXcds * kSliceGroup) == 0) {
    const int x = i % kXcds, l = i / kXcds;
    const int gi = l / (kSliceGroup * n_t), r = l - gi * (kSliceGroup * n_t);
    t = r / kSliceGroup;
    s = x + kXcds * (gi * kSliceGroup + r - t * kSliceGroup);
  } else {
    t = i / n_s;
    s = i - t * n_s;
  }
}
constexpr int kMaxKvSplits = 64;
// rows = kDecodeRows: the vector kernel for at most this many query rows per
// key/value head (the g heads of a group x T_q packed together), one
// workgroup per kDecodeChunk keys, always writing partials.
constexpr int kDecodeRows = 8;
constexpr int kDecodeChunk = 256;
struct Plan {
  int rows;
  int splits;
};
inline Plan make_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk, int causal,
                      int block_rows, int kv_splits) {
  const int64_t packed = (Hq / Hkv) * Tq;
  if (block_rows == kDecodeRows ||
      (block_rows == 0 && kv_splits == 0 && packed <= kDecodeRows))
    return Plan{kDecodeRows, (int)((Tk + kDecodeChunk - 1) / kDecodeChunk)};
  const int64_t bh = B * Hq;
  const int64_t n256 = (Tq + 255) / 256 * bh, n128 = (Tq + 127) / 128 * bh,
                n64 = (Tq + 63) / 64 * bh;
  Plan pl{block_rows, kv_splits > 0 ? kv_splits : 1};
  if (pl.rows == 0) {
    // 256-row workgroups when there are enough of them to fill the device
    // (with a causal mask, also to balance tiles of unequal length);
    // otherwise 128- or 64-row workgroups, several per CU.
    if (kv_splits <= 1 && n256 >= (causal ? 4 : 1) * kDeviceCUs) pl.rows = 256;
    else pl.rows = n128 >= kDeviceCUs ? 128 : 64;
  }
  if (kv_splits == 0 && pl.rows != 256) {
    // too few waves for the device (2 per SIMD) and long key ranges: split
    // the keys.  A workgroup of `rows` query rows has rows / 32 waves.
    const int64_t n_wg = pl.rows == 128 ? n128 : n64;
    const int64_t want = 8 * kDeviceCUs / (pl.rows / 32);  // workgroups that fill the device
    const int64_t tiles = (Tk + (pl.rows == 128 ? 63 : 31)) / (pl.rows == 128 ? 64 : 32);
    if (n_wg < want && tiles >= 8) {
      int64_t s = (want + n_wg - 1) / n_wg;
      s = s < tiles / 4 ? s : tiles / 4;  // at least 4 tiles per chunk
      s = s < kMaxKvSplits ? s : kMaxKvSplits;
      pl.splits = s > 1 ? (int)s : 1;
    }
  }
  return pl;
}

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
  float* nk;         // Yat (workspace): forward |k_j|^2 + b_h [B*Hq][nk_pitch(Tk)];
                     // telemetry |k_j|^2 [B*Hkv][nk_pitch(Tk)]
  int64_t qs[3], ks[3], vs[3], os[3];  // element strides for (b, h, t)
  int B, Hq, Hkv, Tq, Tk, dk, dv;
  int variant;
  int causal;
  int block_rows;     // query rows per workgroup: 64, 128 or 256, or kDecodeRows for
                      // the packed vector kernel (bf16; planned)
  int kv_splits;      // key chunks per workgroup (>= 1); > 1 writes partials
  float* part;        // kv_splits > 1: partial O [S][R][dv] then stats [S][R][4]
                      // (mass, max, reference max), R = B*Hq*Tq
  // telemetry pass (attn_telemetry): the forward's row statistics in, row
  // entropy / sparsity out, per-(head, batch, query tile) tau sums
  const float* in_mass;
  const float* in_max;
  float sparsity_threshold;
  float* row_entropy;
  float* row_sparsity;
  double* tau_part;   // [Hq][B][n_qt][8]: count, sum s, sum L, sum s^2, sum L^2, sum sL
  float* tau_star;
  int yat_power;      // Yat numerator power m >= 1 ((s + b)^(2m))
  int yat_bias_free;  // Yat: b = 0 exactly (b_raw not read)
};

// Device address of this GPU's scratch for attn_fwd_noalloc
// (ATTN_NOALLOC_SCRATCH_BYTES), taken once per device (attn_scratch.hip).
hipError_t scratch_address(void** ptr);

// Telemetry pass: per-row entropy and sparsity of the weights, tau sums.
hipError_t launch_stats_bf16_dk16(const Problem& p, hipStream_t stream);
hipError_t launch_stats_bf16_dk32(const Problem& p, hipStream_t stream);
hipError_t launch_stats_bf16_dk64(const Problem& p, hipStream_t stream);
hipError_t launch_stats_bf16_dk128(const Problem& p, hipStream_t stream);
// tau* per query head from the tau sums (fixed summation order).
hipError_t launch_tau_star(const Problem& p, hipStream_t stream);
// Query rows per workgroup of the telemetry pass.
constexpr int kStatsRows = 64;

// Merges the kv_splits partials of every row into out, mass and max_score.
hipError_t launch_combine(const Problem& p, hipStream_t stream);

// Forward for at most kDecodeRows query rows per key/value head (vector ALU,
// partials per kDecodeChunk keys; combine_partials merges them).
hipError_t launch_decode_bf16_dk16(const Problem& p, hipStream_t stream);
hipError_t launch_decode_bf16_dk32(const Problem& p, hipStream_t stream);
hipError_t launch_decode_bf16_dk64(const Problem& p, hipStream_t stream);
hipError_t launch_decode_bf16_dk128(const Problem& p, hipStream_t stream);

// Fused forward for fp32 storage (vector-ALU path).
hipError_t launch_f32(const Problem& p, hipStream_t stream);

// Per-dk launchers of the bf16 path: |k|^2 pre-pass (Yat) + fused forward on
// the matrix cores (one translation unit per d_k).
hipError_t launch_bf16_dk16(const Problem& p, hipStream_t stream);
hipError_t launch_bf16_dk32(const Problem& p, hipStream_t stream);
hipError_t launch_bf16_dk64(const Problem& p, hipStream_t stream);
hipError_t launch_bf16_dk128(const Problem& p, hipStream_t stream);

// Backward pass (bf16 storage).  Per query row i the API layer's first kernel
// leaves the row normaliser the forward used: Yat 1 / (mass + 1e-9), s^tau
// 1 / mass (0 if mass is 0), softmax L_i = max_score_i log2(e) + log2(mass_i)
// (weights exp2(s log2(e) - L_i)); a first pass over the score tiles then
// fills in D_i = sum_j w_ij dp_ij.
struct BwdProblem {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  void* dq;          // strides of q
  void* dk_;         // strides of k
  void* dv_;         // strides of v
  const float* b_raw;
  const float* eps_raw;
  const float* log_tau;
  const float* mass;
  const float* max_score;
  float* db_raw;     // Yat; may be null
  float* deps_raw;   // Yat; may be null
  float* dlog_tau;   // s^tau; may be null
  int64_t qs[3], ks[3], vs[3], os[3];  // os: strides of dout
  int B, Hq, Hkv, Tq, Tk, dk, dv;
  int variant;
  int causal;
  // workspace
  float* nq;         // Yat: |q_i|^2 + b_h [B*Hq][nk_pitch(Tq)]
  float* nk;         // Yat: |k_j|^2 + b_h per query head h [B*Hq][nk_pitch(Tk)]
  float* row_d;      // D_i = sum_j w_ij dp_ij [B*Hq][nk_pitch(Tq)] (0 past T_q)
  float* row_z;      // row normaliser [B*Hq][nk_pitch(Tq)] (0 past T_q)
  double* prm_part;  // [Hq][B][n_qt][2] per-workgroup sums for the parameter
                     // gradients (n_qt = query tiles of the dq kernel)
};
// Query rows per workgroup of the dq kernel.
constexpr int kBwdQRows = 128;

// The row normaliser of every query row, and D cleared (before the passes).
hipError_t launch_bwd_rows(const BwdProblem& p, hipStream_t stream);
// dk, dv (key-tile kernel) and dq plus parameter sums (query-tile kernel).
hipError_t launch_bwd_bf16_dk16(const BwdProblem& p, hipStream_t stream);
hipError_t launch_bwd_bf16_dk32(const BwdProblem& p, hipStream_t stream);
hipError_t launch_bwd_bf16_dk64(const BwdProblem& p, hipStream_t stream);
hipError_t launch_bwd_bf16_dk128(const BwdProblem& p, hipStream_t stream);
// Per-head parameter gradients from the per-workgroup sums (fixed order).
hipError_t launch_bwd_params(const BwdProblem& p, hipStream_t stream);

}  // namespace sfs
