// attn_api.cpp -- the C ABI declared in include/sfs_attn.h.
//
// Every argument is validated on the host before any HIP call, so a bad call
// returns its status code, enqueues nothing and writes nothing -- also on a
// machine without a GPU.  The library allocates nothing per call.
#include "sfs_attn.h"

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>

#include "attn_launch.h"

namespace {

thread_local char g_last_error[256] = "";

void set_error(const char* msg) {
  std::snprintf(g_last_error, sizeof g_last_error, "%s", msg);
}

bool head_dim_ok(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks one tensor's strides: non-negative multiples of 16 bytes, and the
// byte span of one (batch, head) slice below 2^31 (kernels use 32-bit offsets
// inside a slice).
bool strides_ok(const int64_t s[3], int64_t rows, int64_t d, int64_t elem) {
  const int64_t align = 16 / elem;
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || s[i] % align != 0) return false;
  if (s[2] < d) return false;  // rows of one slice may not overlap
  const int64_t span = ((rows - 1) * s[2] + d) * elem;
  return span < (int64_t(1) << 31);
}

// Sizes whose index and workspace arithmetic cannot overflow: every extent
// within 32 bits, B*Hq*Tq query rows within 32 bits, B*Hq*Tk within 2^40 and
// head sizes within 4096 (no kernel is built for more).  Tq may be 0 here.
bool sizes_fit(const attn_desc* d) {
  if (d->B < 0 || d->Hq <= 0 || d->Hkv <= 0 || d->Tq < 0 || d->Tk <= 0 || d->dk <= 0 ||
      d->dv <= 0)
    return false;
  if (d->B > INT32_MAX || d->Hq > INT32_MAX || d->Tq > INT32_MAX || d->Tk > INT32_MAX ||
      d->dk > 4096 || d->dv > 4096)
    return false;
  int64_t bh = 0, rows_q = 0, rows_k = 0;
  if (__builtin_mul_overflow(d->B, d->Hq, &bh) || __builtin_mul_overflow(bh, d->Tq, &rows_q) ||
      __builtin_mul_overflow(bh, d->Tk, &rows_k))
    return false;
  return rows_q <= INT32_MAX && rows_k <= (int64_t(1) << 40);
}

// Workspace layout of the bf16 path: Yat |k|^2 rows, then (key splits) the
// partials, each region 256-byte aligned.
struct WsLayout {
  sfs::Plan plan;
  size_t nk_bytes, part_off, total;
};
WsLayout ws_layout(const attn_desc* d, int variant, int causal) {
  WsLayout w{};
  w.plan = sfs::make_plan(d->B, d->Hq, d->Hkv, d->Tq, d->Tk, causal, d->block_rows,
                          d->kv_splits);
  // the decode kernel forms |k|^2 itself: no pre-pass
  const bool decode = w.plan.rows == sfs::kDecodeRows;
  w.nk_bytes = variant == ATTN_YAT && !decode
                   ? (size_t)(d->B * d->Hq * sfs::nk_pitch(d->Tk)) * 4 : 0;
  w.part_off = (w.nk_bytes + 255) / 256 * 256;
  w.total = w.nk_bytes;
  if (w.plan.splits > 1 || decode)
    w.total = w.part_off + (size_t)w.plan.splits * (size_t)(d->B * d->Hq * d->Tq) *
                               (size_t)(d->dv + 4) * sizeof(float);
  return w;
}
// The plan depends on the mask (a causal problem needs 4x more 256-row
// workgroups before it takes that kernel), which the workspace query does not
// know: size for the larger of the two.
size_t ws_need(const attn_desc* d, int variant) {
  const size_t a = ws_layout(d, variant, 0).total, c = ws_layout(d, variant, 1).total;
  return a > c ? a : c;
}

int validate(const attn_desc* d, const void* q, const void* k, const void* v, int variant,
             const float* b_raw, const float* eps_raw, const float* log_tau, int causal,
             const void* out, const float* mass, const float* max_score, const void* ws,
             size_t ws_bytes, bool yat_bias_free, bool* empty, int64_t ws_need = -1) {
  *empty = false;
  if (!d) {
    set_error("desc is NULL");
    return ATTN_ERR_NULL;
  }
  if (d->B < 0 || d->Hq <= 0 || d->Hkv <= 0 || d->Tq < 0 || d->Tk <= 0 || d->dk <= 0 ||
      d->dv <= 0) {
    set_error("a size is out of range (B >= 0, Hq, Hkv >= 1, Tq >= 0, Tk >= 1, dk, dv >= 1)");
    return ATTN_ERR_SHAPE;
  }
  if (d->Hq % d->Hkv != 0) {
    set_error("Hq must be a multiple of Hkv");
    return ATTN_ERR_SHAPE;
  }
  if (causal && d->Tq != d->Tk) {
    set_error("a causal mask needs Tq == Tk");
    return ATTN_ERR_SHAPE;
  }
  if (!sizes_fit(d)) {
    set_error("problem too large (B*Hq*Tq and each extent within 32 bits, B*Hq*Tk within "
              "2^40, head sizes within 4096)");
    return ATTN_ERR_UNSUPPORTED;
  }
  if (variant < ATTN_SOFTMAX || variant > ATTN_STAU) {
    set_error("unknown variant");
    return ATTN_ERR_UNSUPPORTED;
  }
  if (d->dtype != ATTN_F32 && d->dtype != ATTN_BF16) {
    set_error("unknown dtype");
    return ATTN_ERR_UNSUPPORTED;
  }
  if (d->block_rows != 0 && (d->dtype != ATTN_BF16 || (d->block_rows != 64 &&
                             d->block_rows != 128 && d->block_rows != 256 &&
                             d->block_rows != sfs::kDecodeRows))) {
    set_error("block_rows must be 0, or 8, 64, 128 or 256 with bf16 storage");
    return ATTN_ERR_UNSUPPORTED;
  }
  if (d->block_rows == sfs::kDecodeRows && d->Hq / d->Hkv * d->Tq > sfs::kDecodeRows) {
    set_error("block_rows = 8 needs at most 8 query rows per key/value head (Hq/Hkv * Tq)");
    return ATTN_ERR_UNSUPPORTED;
  }
  if (d->kv_splits < 0 || d->kv_splits > sfs::kMaxKvSplits || d->reserved != 0 ||
      (d->kv_splits > 1 && (d->dtype != ATTN_BF16 || d->block_rows == 256 ||
                            d->block_rows == sfs::kDecodeRows))) {
    set_error("kv_splits must be 0 .. 64; more than 1 needs bf16 and a 64- or 128-row kernel");
    return ATTN_ERR_UNSUPPORTED;
  }
  if (!head_dim_ok(d->dk) || !head_dim_ok(d->dv)) {
    set_error("dk and dv must be 16, 32, 64 or 128");
    return ATTN_ERR_UNSUPPORTED;
  }
  if (d->B == 0 || d->Tq == 0) {
    *empty = true;
    return ATTN_OK;
  }
  if (!q || !k || !v || !out) {
    set_error("q, k, v and out are required");
    return ATTN_ERR_NULL;
  }
  if (variant == ATTN_YAT && ((!b_raw && !yat_bias_free) || !eps_raw)) {
    set_error("the Yat map needs eps_raw, and b_raw unless it is bias-free");
    return ATTN_ERR_PARAM;
  }
  if (variant == ATTN_STAU && !log_tau) {
    set_error("the s^tau map needs log_tau");
    return ATTN_ERR_PARAM;
  }
  const int64_t elem = d->dtype == ATTN_BF16 ? 2 : 4;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(mass) & 3u) || (reinterpret_cast<uintptr_t>(max_score) & 3u)) {
    set_error("q, k, v, out must be 16-byte aligned; mass and max_score 4-byte aligned");
    return ATTN_ERR_UNSUPPORTED;
  }
  if (!strides_ok(d->q_stride, d->Tq, d->dk, elem) || !strides_ok(d->k_stride, d->Tk, d->dk, elem) ||
      !strides_ok(d->v_stride, d->Tk, d->dv, elem) || !strides_ok(d->o_stride, d->Tq, d->dv, elem)) {
    set_error("strides must be non-negative multiples of 16 bytes, row stride >= row width, "
              "and one (batch, head) slice must span less than 2^31 bytes");
    return ATTN_ERR_UNSUPPORTED;
  }
  const size_t need = ws_need >= 0 ? (size_t)ws_need : attn_fwd_workspace_bytes(d, variant);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) {
    set_error("workspace missing, misaligned or smaller than attn_fwd_workspace_bytes()");
    return ATTN_ERR_WORKSPACE;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_desc_init(attn_desc* d, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq, int64_t Tk,
                   int64_t dk, int64_t dv, int32_t dtype) {
  if (!d) return ATTN_ERR_NULL;
  std::memset(d, 0, sizeof *d);
  d->B = B; d->Hq = Hq; d->Hkv = Hkv; d->Tq = Tq; d->Tk = Tk; d->dk = dk; d->dv = dv;
  d->dtype = dtype;
  d->q_stride[2] = dk; d->q_stride[1] = Tq * dk; d->q_stride[0] = Hq * Tq * dk;
  d->k_stride[2] = dk; d->k_stride[1] = Tk * dk; d->k_stride[0] = Hkv * Tk * dk;
  d->v_stride[2] = dv; d->v_stride[1] = Tk * dv; d->v_stride[0] = Hkv * Tk * dv;
  d->o_stride[2] = dv; d->o_stride[1] = Tq * dv; d->o_stride[0] = Hq * Tq * dv;
  return ATTN_OK;
}

size_t attn_fwd_workspace_bytes(const attn_desc* d, int variant) {
  if (!d || d->dtype != ATTN_BF16 || !sizes_fit(d) || d->B == 0 || d->Tq == 0) return 0;
  return ws_need(d, variant);
}

}  // extern "C"

namespace {

int run(const attn_desc* d, const void* q, const void* k, const void* v, int variant,
        const float* b_raw, const float* eps_raw, const float* log_tau, int yat_power,
        int yat_bias_free, int causal, void* out, float* mass, float* max_score,
        void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  const int st = validate(d, q, k, v, variant, b_raw, eps_raw, log_tau, causal, out, mass,
                          max_score, workspace, workspace_bytes, yat_bias_free != 0, &empty);
  if (st != ATTN_OK || empty) return st;

  sfs::Problem p{};
  p.q = q; p.k = k; p.v = v; p.out = out;
  p.mass = mass; p.max_score = max_score;
  p.b_raw = b_raw; p.eps_raw = eps_raw; p.log_tau = log_tau;
  // bias-free Yat does not read b_raw; keep the pointer valid all the same
  if (variant == ATTN_YAT && yat_bias_free && !b_raw) p.b_raw = eps_raw;
  p.nk = static_cast<float*>(workspace);
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = d->q_stride[i]; p.ks[i] = d->k_stride[i];
    p.vs[i] = d->v_stride[i]; p.os[i] = d->o_stride[i];
  }
  p.B = (int)d->B; p.Hq = (int)d->Hq; p.Hkv = (int)d->Hkv;
  p.Tq = (int)d->Tq; p.Tk = (int)d->Tk; p.dk = (int)d->dk; p.dv = (int)d->dv;
  p.variant = variant;
  p.causal = causal ? 1 : 0;
  p.kv_splits = 1;
  if (d->dtype == ATTN_BF16) {
    const WsLayout w = ws_layout(d, variant, p.causal);
    p.block_rows = w.plan.rows;
    p.kv_splits = w.plan.splits;
    if (p.kv_splits > 1 || p.block_rows == sfs::kDecodeRows)
      p.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.part_off);
  }
  p.yat_power = yat_power;
  p.yat_bias_free = yat_bias_free ? 1 : 0;

  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (d->dtype == ATTN_F32) {
      e = sfs::launch_f32(p, s);
    } else {
      if (p.block_rows == sfs::kDecodeRows) {
        switch (p.dk) {
          case 16: e = sfs::launch_decode_bf16_dk16(p, s); break;
          case 32: e = sfs::launch_decode_bf16_dk32(p, s); break;
          case 64: e = sfs::launch_decode_bf16_dk64(p, s); break;
          default: e = sfs::launch_decode_bf16_dk128(p, s); break;
        }
      } else {
        switch (p.dk) {
          case 16: e = sfs::launch_bf16_dk16(p, s); break;
          case 32: e = sfs::launch_bf16_dk32(p, s); break;
          case 64: e = sfs::launch_bf16_dk64(p, s); break;
          default: e = sfs::launch_bf16_dk128(p, s); break;
        }
      }
      if (e == hipSuccess && (p.kv_splits > 1 || p.block_rows == sfs::kDecodeRows))
        e = sfs::launch_combine(p, s);
    }
  }
  if (e != hipSuccess) {
    char msg[256];
    std::snprintf(msg, sizeof msg, "HIP: %s (%s)", hipGetErrorName(e), hipGetErrorString(e));
    set_error(msg);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const attn_desc* d, const void* q, const void* k, const void* v, int variant,
             const float* b_raw, const float* eps_raw, const float* log_tau, int causal,
             void* out, float* mass, float* max_score, void* workspace, size_t workspace_bytes,
             void* stream) {
  return run(d, q, k, v, variant, b_raw, eps_raw, log_tau, 1, 0, causal, out, mass, max_score,
             workspace, workspace_bytes, stream);
}

int attn_fwd_yat(const attn_desc* d, const void* q, const void* k, const void* v,
                 const float* b_raw, const float* eps_raw, const attn_yat_opts* opts, int causal,
                 void* out, float* mass, float* max_score, void* workspace,
                 size_t workspace_bytes, void* stream) {
  const int power = opts ? opts->power : 1;
  const int bias_free = opts ? opts->bias_free : 0;
  if (power < 1 || power > ATTN_YAT_MAX_POWER) {
    set_error("Yat numerator power must be 1 .. ATTN_YAT_MAX_POWER");
    return ATTN_ERR_UNSUPPORTED;
  }
  return run(d, q, k, v, ATTN_YAT, b_raw, eps_raw, nullptr, power, bias_free, causal, out, mass,
             max_score, workspace, workspace_bytes, stream);
}

int attn_fwd_noalloc(const attn_desc* d, const void* q, const void* k, const void* v,
                     int variant, const float* b_raw, const float* eps_raw,
                     const float* log_tau, int causal, void* out, float* mass,
                     float* max_score, void* stream) {
  // the same checks as attn_fwd, with the scratch size in place of the
  // caller's workspace; nothing touches the GPU before they pass
  bool empty = false;
  const size_t need = d ? attn_fwd_workspace_bytes(d, variant) : 0;
  int st = validate(d, q, k, v, variant, b_raw, eps_raw, log_tau, causal, out, mass, max_score,
                    nullptr, 0, false, &empty, 0);
  if (st != ATTN_OK || empty) return st;
  if (need > ATTN_NOALLOC_SCRATCH_BYTES) {
    char msg[256];
    std::snprintf(msg, sizeof msg,
                  "attn_fwd_noalloc: this problem needs %zu bytes of scratch, more than the "
                  "%u of ATTN_NOALLOC_SCRATCH_BYTES (use attn_fwd with a workspace)",
                  need, (unsigned)ATTN_NOALLOC_SCRATCH_BYTES);
    set_error(msg);
    return ATTN_ERR_WORKSPACE;
  }
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = sfs::scratch_address(&scratch);
    if (e != hipSuccess) {
      char msg[256];
      std::snprintf(msg, sizeof msg, "HIP: %s (%s)", hipGetErrorName(e), hipGetErrorString(e));
      set_error(msg);
      return ATTN_ERR_HIP;
    }
  }
  return run(d, q, k, v, variant, b_raw, eps_raw, log_tau, 1, 0, causal, out, mass, max_score,
             scratch, need, stream);
}

size_t attn_telemetry_workspace_bytes(const attn_desc* d, int variant) {
  if (!d || d->dtype != ATTN_BF16 || !sizes_fit(d) || d->B == 0 || d->Tq == 0) return 0;
  const size_t nk = variant == ATTN_YAT ? (size_t)(d->B * d->Hkv * sfs::nk_pitch(d->Tk)) * 4 : 0;
  const size_t n_qt = (size_t)((d->Tq + sfs::kStatsRows - 1) / sfs::kStatsRows);
  return (nk + 255) / 256 * 256 + (size_t)(d->Hq * d->B) * n_qt * 8 * sizeof(double);
}

int attn_telemetry(const attn_desc* d, const void* q, const void* k, int variant,
                   const float* b_raw, const float* eps_raw, const float* log_tau, int causal,
                   const float* mass, const float* max_score, float sparsity_threshold,
                   float* row_entropy, float* row_sparsity, float* tau_star, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (d && d->dtype != ATTN_BF16) {
    set_error("telemetry is built for bf16 storage");
    return ATTN_ERR_UNSUPPORTED;
  }
  if (!mass || (variant == ATTN_SOFTMAX && !max_score) ||
      (!row_entropy && !row_sparsity && !tau_star)) {
    set_error("telemetry needs the forward's mass (and max_score for softmax) and an output");
    return ATTN_ERR_NULL;
  }
  if (!(sparsity_threshold > 0.f)) {
    set_error("sparsity_threshold must be > 0");
    return ATTN_ERR_PARAM;
  }
  for (const float* t : {row_entropy, row_sparsity, tau_star})
    if (reinterpret_cast<uintptr_t>(t) & 3u) {
      set_error("telemetry outputs must be 4-byte aligned");
      return ATTN_ERR_UNSUPPORTED;
    }
  bool empty = false;
  // v and out are not used: k stands in for their pointer checks
  const int st = validate(d, q, k, k, variant, b_raw, eps_raw, log_tau, causal, k, mass,
                          max_score, workspace, workspace_bytes, false, &empty,
                          (int64_t)attn_telemetry_workspace_bytes(d, variant));
  if (st != ATTN_OK || empty) return st;

  sfs::Problem p{};
  p.q = q; p.k = k;
  p.b_raw = b_raw; p.eps_raw = eps_raw; p.log_tau = log_tau;
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = d->q_stride[i]; p.ks[i] = d->k_stride[i];
  }
  p.B = (int)d->B; p.Hq = (int)d->Hq; p.Hkv = (int)d->Hkv;
  p.Tq = (int)d->Tq; p.Tk = (int)d->Tk; p.dk = (int)d->dk; p.dv = (int)d->dv;
  p.variant = variant;
  p.causal = causal ? 1 : 0;
  p.yat_power = 1;
  p.in_mass = mass; p.in_max = max_score;
  p.sparsity_threshold = sparsity_threshold;
  p.row_entropy = row_entropy; p.row_sparsity = row_sparsity; p.tau_star = tau_star;
  const size_t nk = variant == ATTN_YAT ? (size_t)(d->B * d->Hkv * sfs::nk_pitch(d->Tk)) * 4 : 0;
  p.nk = static_cast<float*>(workspace);
  if (tau_star)
    p.tau_part = reinterpret_cast<double*>(static_cast<char*>(workspace) + (nk + 255) / 256 * 256);

  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (p.dk) {
      case 16: e = sfs::launch_stats_bf16_dk16(p, s); break;
      case 32: e = sfs::launch_stats_bf16_dk32(p, s); break;
      case 64: e = sfs::launch_stats_bf16_dk64(p, s); break;
      default: e = sfs::launch_stats_bf16_dk128(p, s); break;
    }
    if (e == hipSuccess && tau_star) e = sfs::launch_tau_star(p, s);
  }
  if (e != hipSuccess) {
    char msg[256];
    std::snprintf(msg, sizeof msg, "HIP: %s (%s)", hipGetErrorName(e), hipGetErrorString(e));
    set_error(msg);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // extern "C"

namespace {

// Workspace of the backward: Yat |k|^2 and |q|^2 rows, the row values D and
// Z, and the parameter sums; each region 256-byte aligned.
struct BwdWs {
  size_t nk, nq, rd, rz, prm, total;
};
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
BwdWs bwd_ws(const attn_desc* d, int variant) {
  BwdWs w{};
  const size_t rows_q = (size_t)(d->B * d->Hq * sfs::nk_pitch(d->Tq)) * 4;
  const size_t n_qt = (size_t)((d->Tq + sfs::kBwdQRows - 1) / sfs::kBwdQRows);
  size_t off = 0;
  w.nk = off;
  if (variant == ATTN_YAT) off += align256((size_t)(d->B * d->Hq * sfs::nk_pitch(d->Tk)) * 4);
  w.nq = off;
  if (variant == ATTN_YAT) off += align256(rows_q);
  w.rd = off;
  off += align256(rows_q);
  w.rz = off;
  off += align256(rows_q);
  w.prm = off;
  if (variant != ATTN_SOFTMAX) off += (size_t)(d->Hq * d->B) * n_qt * 2 * sizeof(double);
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

size_t attn_bwd_workspace_bytes(const attn_desc* d, int variant) {
  if (!d || d->dtype != ATTN_BF16 || !sizes_fit(d) || d->B == 0 || d->Tq == 0) return 0;
  if (variant < ATTN_SOFTMAX || variant > ATTN_STAU) return 0;
  return bwd_ws(d, variant).total;
}

int attn_bwd(const attn_desc* d, const void* q, const void* k, const void* v,
             const void* dout, int variant, const float* b_raw, const float* eps_raw,
             const float* log_tau, int causal, const float* mass, const float* max_score,
             void* dq, void* dk, void* dv, float* db_raw, float* deps_raw, float* dlog_tau,
             void* workspace, size_t workspace_bytes, void* stream) {
  if (d && d->dtype != ATTN_BF16) {
    set_error("the backward is built for bf16 storage");
    return ATTN_ERR_UNSUPPORTED;
  }
  bool empty = false;
  const int64_t need = d ? (int64_t)attn_bwd_workspace_bytes(d, variant) : 0;
  // dout takes the place of out (o_stride describes it)
  int st = validate(d, q, k, v, variant, b_raw, eps_raw, log_tau, causal, dout, mass, max_score,
                    workspace, workspace_bytes, false, &empty, need);
  if (st != ATTN_OK) return st;
  if (!empty) {
    if (!dq || !dk || !dv || (variant == ATTN_SOFTMAX && (!mass || !max_score))) {
      set_error("the backward needs dq, dk, dv and, for softmax, the forward's mass and "
                "max_score");
      return ATTN_ERR_NULL;
    }
    if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv)) {
      set_error("dq, dk and dv must be 16-byte aligned");
      return ATTN_ERR_UNSUPPORTED;
    }
    for (const float* t : {db_raw, deps_raw, dlog_tau})
      if (reinterpret_cast<uintptr_t>(t) & 3u) {
        set_error("parameter gradients must be 4-byte aligned");
        return ATTN_ERR_UNSUPPORTED;
      }
  }
  if (empty && d->B > 0) {
    // T_q == 0: no query rows, so dk and dv are zero; they are still written
    if (!k || !v || !dk || !dv) {
      set_error("k, v, dk and dv are required");
      return ATTN_ERR_NULL;
    }
    if (!aligned16(k) || !aligned16(v) || !aligned16(dk) || !aligned16(dv) ||
        !strides_ok(d->k_stride, d->Tk, d->dk, 2) || !strides_ok(d->v_stride, d->Tk, d->dv, 2)) {
      set_error("k, v, dk, dv must be 16-byte aligned with valid strides");
      return ATTN_ERR_UNSUPPORTED;
    }
  } else if (empty) {
    return ATTN_OK;
  }

  sfs::BwdProblem p{};
  p.q = q; p.k = k; p.v = v; p.dout = dout;
  p.dq = dq; p.dk_ = dk; p.dv_ = dv;
  p.b_raw = b_raw; p.eps_raw = eps_raw; p.log_tau = log_tau;
  p.mass = mass; p.max_score = max_score;
  p.db_raw = db_raw; p.deps_raw = deps_raw; p.dlog_tau = dlog_tau;
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = d->q_stride[i]; p.ks[i] = d->k_stride[i];
    p.vs[i] = d->v_stride[i]; p.os[i] = d->o_stride[i];
  }
  p.B = (int)d->B; p.Hq = (int)d->Hq; p.Hkv = (int)d->Hkv;
  p.Tq = (int)d->Tq; p.Tk = (int)d->Tk; p.dk = (int)d->dk; p.dv = (int)d->dv;
  p.variant = variant;
  p.causal = causal ? 1 : 0;
  const BwdWs w = bwd_ws(d, variant);
  char* ws = static_cast<char*>(workspace);
  p.nk = reinterpret_cast<float*>(ws + w.nk);
  p.nq = reinterpret_cast<float*>(ws + w.nq);
  p.row_d = reinterpret_cast<float*>(ws + w.rd);
  p.row_z = reinterpret_cast<float*>(ws + w.rz);
  const bool params = (variant == ATTN_YAT && (db_raw || deps_raw)) ||
                      (variant == ATTN_STAU && dlog_tau);
  p.prm_part = params ? reinterpret_cast<double*>(ws + w.prm) : nullptr;

  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.Tq > 0) e = sfs::launch_bwd_rows(p, s);  // (no rows: an empty grid)
    if (e == hipSuccess) {
      switch (p.dk) {
        case 16: e = sfs::launch_bwd_bf16_dk16(p, s); break;
        case 32: e = sfs::launch_bwd_bf16_dk32(p, s); break;
        case 64: e = sfs::launch_bwd_bf16_dk64(p, s); break;
        default: e = sfs::launch_bwd_bf16_dk128(p, s); break;
      }
    }
    if (e == hipSuccess && params) e = sfs::launch_bwd_params(p, s);
  }
  if (e != hipSuccess) {
    char msg[256];
    std::snprintf(msg, sizeof msg, "HIP: %s (%s)", hipGetErrorName(e), hipGetErrorString(e));
    set_error(msg);
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape";
    case ATTN_ERR_UNSUPPORTED:
      return "unsupported dtype, variant, head size, option, alignment or size";
    case ATTN_ERR_PARAM: return "a per-head parameter the variant needs is NULL";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* attn_last_error(void) { return g_last_error; }

}  // extern "C"
