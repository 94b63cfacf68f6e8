// attn_bwd_aux.hip -- the small kernels around the attention backward.
//
// bwd_rows: for every query row i the normaliser the forward divided by,
// which every pair (i, j) of the gradient kernels needs:
//   d L / d u_ij = (dout_i . v_j - D_i) / Z_i   for w_ij = u_ij / Z_i.
// Z_i is the mass for s^tau ("s^tau" forum post, core formula), and for
// softmax the weights are exp2(s_ij log2(e) - L_i) with L_i = log2(sum_j
// e^(s_ij - max_i)) + max_i log2(e).  Yat's 1 / (mass + 1e-9) ("Softmax-Free
// Attention in JAX/Flax NNX", "One module, two compatibility functions") is
// formed by the first pass of attn_bwd.hip from its own kappa; here it is
// cleared.  Also clears D (the row sums sum_j w_ij dp_ij that the first pass
// fills in), padding included.
//
// bwd_params: per query head, the parameter gradients from the per-workgroup
// sums of the dq kernel, added in a fixed order in fp64:
//   Yat   d L / d b_raw = sigmoid(b_raw) sum_ij A_ij,
//         d L / d eps_raw = -sigmoid(eps_raw) sum_ij B_ij / 2,
//         A_ij = 2 du_ij (q.k + b) / den, B_ij = 2 du_ij kappa_ij / den
//         (b = softplus(b_raw), eps = softplus(eps_raw), softplus' = sigmoid);
//   s^tau d L / d log_tau = sigmoid(log_tau) ln 2 sum_ij w_ij (dp_ij - D_i)
//         log2(phi_ij)   (d phi^tau / d tau = phi^tau ln phi).
#include "attn_launch.h"

namespace sfs {
namespace {

constexpr float kLog2eF = 1.4426950408889634f;

// One thread per row of B*Hq*nk_pitch(Tq) (padding rows get 0).
__global__ __launch_bounds__(256) void bwd_rows(BwdProblem p) {
  const int64_t pitch = nk_pitch(p.Tq);
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= (int64_t)p.B * p.Hq * pitch) return;
  const int64_t bh = r / pitch, i = r - bh * pitch;
  float z = 0.f;
  if (i < p.Tq) {
    const int64_t ri = bh * p.Tq + i;
    // (Yat and s^tau: the D pass forms Z from its own weights)
    if (p.variant == kSoftmax) z = fmaf(p.max_score[ri], kLog2eF, log2f(p.mass[ri]));
  }
  p.row_d[r] = 0.f;
  p.row_z[r] = z;
}

__device__ double sigmoid_d(double x) { return 1.0 / (1.0 + exp(-x)); }

__global__ __launch_bounds__(64) void bwd_params(BwdProblem p, int n_qt) {
  const int h = blockIdx.x * 64 + threadIdx.x;
  if (h >= p.Hq) return;
  double s0 = 0.0, s1 = 0.0;
  const double* src = p.prm_part + (int64_t)h * p.B * n_qt * 2;
  for (int64_t t = 0; t < (int64_t)p.B * n_qt; ++t) {
    s0 += src[2 * t];
    s1 += src[2 * t + 1];
  }
  if (is_yat(p.variant)) {
    // s0 = sum A/2, s1 = sum B/2 (the dq kernel carries halved terms)
    if (p.db_raw) p.db_raw[h] = (float)(2.0 * sigmoid_d(p.b_raw[h]) * s0);
    if (p.deps_raw) p.deps_raw[h] = (float)(-sigmoid_d(p.eps_raw[h]) * s1);
  } else if (p.variant == kStau) {
    if (p.dlog_tau) p.dlog_tau[h] = (float)(sigmoid_d(p.log_tau[h]) * 0.6931471805599453 * s0);
  }
}

}  // namespace

hipError_t launch_bwd_rows(const BwdProblem& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.Hq * nk_pitch(p.Tq);
  hipLaunchKernelGGL(bwd_rows, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_params(const BwdProblem& p, hipStream_t stream) {
  const int n_qt = (p.Tq + kBwdQRows - 1) / kBwdQRows;
  hipLaunchKernelGGL(bwd_params, dim3((p.Hq + 63) / 64), dim3(64), 0, stream, p, n_qt);
  return hipGetLastError();
}

}  // namespace sfs
