/*
 * sfs_attn.h -- C ABI of the fused attention forward for MI355X (gfx950).
 *
 * One call evaluates, for every batch b, query head h and query row i,
 *
 *     w_ij = normalize_j( score(q_i, k_j) ),   out_i = sum_j w_ij v_j,
 *
 * with one of three score-to-weight maps:
 *
 *   ATTN_YAT      "Softmax-Free Attention in JAX/Flax NNX", section "One module,
 *                 two compatibility functions" (the kernel branch):
 *                 dots = q.k;  d2 = |q|^2 + |k|^2 - 2 dots;
 *                 b = softplus(b_raw[h]), eps = softplus(eps_raw[h]);
 *                 kappa = (dots + b)^2 / (max(d2, 0) + eps); masked kappa = 0;
 *                 mass = sum_j kappa;  w = kappa / (mass + 1e-9).
 *                 No 1/sqrt(d_k) scale.
 *   ATTN_SOFTMAX  "NNX Scaled Dot-Product Attention", the displayed equation
 *                 A = softmax(Q K^T / sqrt(d_k) + M), O = A V, with M = -inf on
 *                 blocked keys ("Mask before softmax").
 *   ATTN_STAU     "s^tau" forum post, core formula:
 *                 s = q.k / sqrt(d_k); phi = softplus(s) + 1e-6;
 *                 tau = softplus(log_tau[h]) + 1; w = phi^tau / sum_j phi^tau.
 *
 * Shapes follow "NNX Scaled Dot-Product Attention", "Shapes and the three
 * steps": queries T_q x d_k, keys T_k x d_k, values T_k x d_v per head; T_q
 * may differ from T_k and d_v from d_k.  Several query heads may share one
 * key/value head (grouped-query attention): query head h reads key/value head
 * h / (Hq / Hkv).
 *
 * Readings of points the pages leave open:
 *   - causal: key j is allowed for query i iff j <= i; it requires T_q == T_k.
 *   - a masked key contributes exactly 0 to numerator and denominator in all
 *     three maps (the s^tau page instead feeds -inf through softplus).
 *   - mass [B,Hq,Tq]: Yat sum(kappa); softmax sum_j exp(s_ij - max_j s_ij);
 *     s^tau sum_j phi^tau.  A row whose s^tau mass underflows to 0 gets out 0.
 *   - max_score [B,Hq,Tq]: Yat max kappa; softmax and s^tau max s (the scaled
 *     logit), over allowed keys.
 *   - s^tau is evaluated in one pass without a running maximum; its supported
 *     domain is tau * ln(phi) < 88 (no fp32 overflow of phi^tau).
 *   - bf16 storage: the weights that multiply V are rounded to bf16 (the
 *     matrix cores take bf16 operands; the decode kernel rounds the same way).
 *     The Yat mass of the matrix-core kernels is the sum of those rounded
 *     weights, so out is normalised by exactly the weights it averages with;
 *     it differs from the fp32 sum of kappa by at most 2^-9 relative.
 */
#ifndef SFS_ATTN_H
#define SFS_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Score-to-weight map. */
typedef enum { ATTN_SOFTMAX = 0, ATTN_YAT = 1, ATTN_STAU = 2 } attn_variant;

/* Storage type of q, k, v and out.  Arithmetic is fp32 in both cases; with
 * ATTN_BF16 the two contractions run on bf16 matrix cores with fp32
 * accumulation and the weights are rounded to bf16 (nearest-even) before the
 * second one. */
typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Status codes: 0 on success, negative on error. */
enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = -2,       /* a size is negative or zero where it may not be,
                                Hq % Hkv != 0, or causal with T_q != T_k */
  ATTN_ERR_UNSUPPORTED = -3, /* dtype, variant, head size, block_rows or
                                kv_splits not built; a base pointer or stride
                                breaks the 16-byte alignment rule; a per-head
                                offset exceeds 2^31 elements */
  ATTN_ERR_PARAM = -4,       /* a per-head parameter the variant needs is NULL */
  ATTN_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required */
  ATTN_ERR_HIP = -6          /* the HIP runtime failed (no device, launch
                                error); see attn_last_error() */
};

/* Problem description.  Sizes: B >= 0 batches, Hq >= 1 query heads,
 * Hkv >= 1 key/value heads with Hq % Hkv == 0, T_q >= 0 query rows,
 * T_k >= 1 key rows, d_k and d_v in {16, 32, 64, 128}.
 *
 * Strides are in elements for the (batch, head, row) axes of q [B,Hq,Tq,dk],
 * k [B,Hkv,Tk,dk], v [B,Hkv,Tk,dv] and out [B,Hq,Tq,dv]; the last axis is
 * contiguous.  Every stride must be a non-negative multiple of 16 bytes
 * (8 bf16 or 4 fp32 elements). */
typedef struct {
  int64_t B, Hq, Hkv, Tq, Tk, dk, dv;
  int32_t dtype; /* attn_dtype */
  /* Query rows per workgroup of the bf16 path: 0 lets the library choose
   * (8 when a key/value head has at most 8 query rows, Hq/Hkv * Tq <= 8;
   * else 256-row workgroups when there are enough to fill the device, else
   * 128 or 64); 8, 64, 128 or 256 force that kernel.  8 is the decode
   * kernel: the query rows of a key/value head packed into one workgroup per
   * 256 keys on the vector ALU, each key and value row read once, partials
   * merged as with kv_splits (it needs Hq/Hkv * Tq <= 8).  Every choice
   * computes the same map; results may differ in the last bits through the
   * order of fp32 additions.  The fp32 path takes 0 only. */
  int32_t block_rows;
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  /* Key splits of the bf16 64- and 128-row kernels.  When a problem has too
   * few query tiles to fill the device (decode, short query blocks against
   * long keys), each workgroup's keys are cut into chunks of whole tiles that
   * run in parallel; each chunk writes unnormalised partials (O, mass,
   * maximum, and for softmax the reference maximum) to the workspace, and a
   * second kernel merges them: plain sums for Yat and s^tau, whose weights
   * need no running maximum, and the log-sum-exp merge for softmax.
   * 0 lets the library choose; 1 switches splitting off; 2 .. 64 force that
   * many chunks (bf16 only, not with block_rows = 256 or 8; the decode
   * kernel always splits into 256-key chunks).  Results differ from
   * the unsplit ones only in the order of fp32 additions. */
  int32_t kv_splits;
  int32_t reserved; /* must be 0 */
} attn_desc;

/* Fill *desc for densely packed [B,H,T,d] tensors.  Returns ATTN_OK or
 * ATTN_ERR_NULL. */
int attn_desc_init(attn_desc* desc, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tq,
                   int64_t Tk, int64_t dk, int64_t dv, int32_t dtype);

/* Device workspace, in bytes, that attn_fwd needs for this problem and map:
 * fp32 |k|^2 + b per key row and query head for ATTN_YAT with bf16 storage
 * (B * Hq * T_k rounded up to 64 rows; not for the decode
 * kernel, block_rows = 8, which forms it itself), and, when the keys are split
 * (see kv_splits; the decode kernel always is, in 256-key chunks), fp32
 * partials of 4 (d_v + 4) bytes per query row and chunk.  Returns 0 when none
 * is needed or the description is invalid. */
size_t attn_fwd_workspace_bytes(const attn_desc* desc, int variant);

/* Attention forward.
 *
 * q, k, v, out   device memory in desc->dtype with the strides of desc; out
 *                must not alias any input.
 * variant        attn_variant.
 * b_raw, eps_raw device fp32 [Hq], raw Yat scalars (softplus is applied here);
 *                required for ATTN_YAT, ignored otherwise (may be NULL).
 *                b_raw = -inf gives the bias-free kernel b = 0.
 * log_tau        device fp32 [Hq]; required for ATTN_STAU, else ignored.
 * causal         nonzero: key j is allowed for query i iff j <= i.
 * mass,          device fp32 [B,Hq,Tq], contiguous; NULL means "do not
 * max_score      store" (they are computed regardless).
 * workspace      device memory of at least attn_fwd_workspace_bytes() bytes,
 *                16-byte aligned; may be NULL when that size is 0.  Its
 *                contents on entry do not matter; it is overwritten.
 * stream         a hipStream_t (NULL = the null stream).
 *
 * Ownership: the caller owns every buffer; the library allocates no device
 * or host memory per call.  The call only validates and enqueues work on
 * `stream`; it returns before the work finishes, and device-side faults
 * surface at the caller's next synchronisation.  On any error nothing is
 * enqueued and no output is written.  Calls on different streams that share
 * a workspace race.  B == 0 or T_q == 0 is a valid empty problem: nothing is
 * enqueued and ATTN_OK is returned. */
int attn_fwd(const attn_desc* desc, const void* q, const void* k, const void* v, int variant,
             const float* b_raw, const float* eps_raw, const float* log_tau, int causal,
             void* out, float* mass, float* max_score, void* workspace,
             size_t workspace_bytes, void* stream);

/* Attention forward that allocates nothing and takes no workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Arguments,
 * layouts, maps, asynchrony and errors are those of attn_fwd without the
 * workspace: the scratch is a library-owned device array of
 * ATTN_NOALLOC_SCRATCH_BYTES per GPU, reserved when the library is loaded on
 * that GPU and held until the process ends.  A problem whose
 * attn_fwd_workspace_bytes() exceeds that size returns ATTN_ERR_WORKSPACE
 * (nothing enqueued).  Every call on one GPU shares that GPU's scratch, which
 * keeps the last call's contents (no call relies on them): calls that may
 * run concurrently on one GPU (different streams) race, so order them.
 * The first call on a GPU looks up the scratch's device address; make it
 * before capturing a graph, whose replays then re-run the captured kernels.
 * Results are identical to attn_fwd's on the same inputs. */
#define ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
int attn_fwd_noalloc(const attn_desc* desc, const void* q, const void* k, const void* v,
                     int variant, const float* b_raw, const float* eps_raw,
                     const float* log_tau, int causal, void* out, float* mass,
                     float* max_score, void* stream);

/* Yat kernel-family options.
 *
 * "The Kernel Between the Roles", section "The run": raising the power of the
 * numerator, (q.k)^(2m), is named as the dial that sharpens the kernel's peak
 * while keeping its structure; the same section measures the b = 0 ablation
 * (the non-universal special case, where an orthogonal query-key pair scores
 * exactly zero).  Here both are options of the Yat map:
 *   kappa = (q.k + b)^(2 power) / (max(|q|^2 + |k|^2 - 2 q.k, 0) + eps),
 * with b = softplus(b_raw[h]), or b = 0 exactly when bias_free is nonzero
 * (b_raw is then not read and may be NULL).  power = 1, bias_free = 0 is the
 * standard kernel that attn_fwd(ATTN_YAT) computes.  Domain: kappa and the
 * row mass must stay finite in fp32, i.e. |q.k + b|^(2 power) / eps summed
 * over a row below ~3e38. */
#define ATTN_YAT_MAX_POWER 8
typedef struct {
  int32_t power;     /* m in 1 .. ATTN_YAT_MAX_POWER */
  int32_t bias_free; /* nonzero: b = 0 exactly */
} attn_yat_opts;

/* The Yat forward with kernel-family options.  Arguments, layouts, workspace
 * (attn_fwd_workspace_bytes(desc, ATTN_YAT)), ownership and errors are those
 * of attn_fwd with variant ATTN_YAT; opts == NULL means {1, 0}.  A power
 * outside 1 .. ATTN_YAT_MAX_POWER returns ATTN_ERR_UNSUPPORTED. */
int attn_fwd_yat(const attn_desc* desc, const void* q, const void* k, const void* v,
                 const float* b_raw, const float* eps_raw, const attn_yat_opts* opts,
                 int causal, void* out, float* mass, float* max_score, void* workspace,
                 size_t workspace_bytes, void* stream);

/* Attention telemetry: one extra pass over the score tiles of a finished
 * forward (same desc, q, k, variant, per-head parameters and mask), given the
 * row statistics that forward returned.  The weights of every allowed pair are
 * recomputed as the forward defines them, and the pass returns:
 *   row_entropy   [B,Hq,Tq]: -sum_j w_ij ln w_ij / ln(n_i) over the n_i allowed
 *                 keys, 0 when n_i = 1 ("The Kernel Between the Roles", "The
 *                 run": 0 for a row on one key, 1 for uniform weights);
 *   row_sparsity  [B,Hq,Tq]: the fraction of allowed keys with w_ij below
 *                 sparsity_threshold (the s^tau post measures weights < 1e-6);
 *   tau_star      [Hq]: Cov(s, ln phi(s)) / Var(ln phi(s)) over all allowed
 *                 pairs of query head h, s = q.k / sqrt(d_k), phi = softplus(s)
 *                 + 1e-6 (the s^tau post's closed form for the tau at which
 *                 s^tau is closest to softmax; NaN when Var = 0).
 * Inputs: mass (all maps) and max_score (softmax) as the forward wrote them,
 * fp32 [B,Hq,Tq], contiguous.  Outputs are device fp32 and may be NULL (not
 * computed); at least one must be given.  v is not read (desc's v fields must
 * still describe a valid tensor shape).  bf16 storage and the standard maps
 * only (the Yat options of attn_fwd_yat are not covered).  Workspace:
 * attn_telemetry_workspace_bytes(desc, variant).  Errors as attn_fwd;
 * sparsity_threshold must be > 0 (else ATTN_ERR_PARAM). */
size_t attn_telemetry_workspace_bytes(const attn_desc* desc, int variant);
int attn_telemetry(const attn_desc* desc, const void* q, const void* k, int variant,
                   const float* b_raw, const float* eps_raw, const float* log_tau, int causal,
                   const float* mass, const float* max_score, float sparsity_threshold,
                   float* row_entropy, float* row_sparsity, float* tau_star, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Attention backward (bf16 storage): the gradients of L = sum(dout * out)
 * for the forward attn_fwd computed with the same desc, inputs, variant,
 * per-head parameters and mask.
 *
 * The pages define the three maps (see the top of this file) and train them
 * by automatic differentiation; the gradients here are the exact derivatives
 * of those closed forms.  With w_ij the forward's weights, Z_i its row
 * normaliser (Yat mass + 1e-9, s^tau mass, softmax sum_j e^(s_ij - max_i)),
 * dp_ij = dout_i . v_j and D_i = sum_j w_ij dp_ij (= dout_i . out_i):
 *   dv_j = sum_i w_ij dout_i, and d L / d u_ij = (dp_ij - D_i) / Z_i for the
 *   unnormalised weight u_ij, which the chain rule carries to q, k and the
 *   parameters through softmax's e^s, s^tau's phi(s)^tau (with
 *   d/dtau = phi^tau ln phi) and Yat's (q.k + b)^2 / (|q - k|^2 + eps).
 * Key/value gradients add over the query heads that share a key/value head.
 * Masked pairs contribute nothing.  The clamp max(d2, 0) of Yat is treated
 * as inactive (it only acts where rounding makes d2 negative, i.e. q = k,
 * where the distance term's derivative 2 (q - k) is 0).  D is recomputed
 * from the weights in fp32 rather than taken from the bf16 output, whose
 * rounding would not cancel where the exact gradient does (a row whose
 * weight sits on one key); the forward's output is therefore not an input.
 *
 * q, k, v        the forward's inputs, device bf16, strides of desc.
 * dout           device bf16 [B,Hq,Tq,dv], strides desc->o_stride.
 * mass,          the forward's row statistics, device fp32 [B,Hq,Tq],
 * max_score      contiguous, read for ATTN_SOFTMAX only.  ATTN_YAT and
 *                ATTN_STAU read neither (may be NULL): they form the row
 *                normaliser again (Yat mass + 1e-9, s^tau mass) from the
 *                weights they differentiate, so that the weights and their
 *                normaliser round alike.
 * dq, dk, dv     device bf16 outputs laid out like q, k and v (q_stride,
 *                k_stride, v_stride); every element is written (dk = dv = 0
 *                when T_q == 0).  They must not alias any input.
 * db_raw,        device fp32 [Hq] outputs for ATTN_YAT (d L / d b_raw and
 * deps_raw       d L / d eps_raw); dlog_tau [Hq] for ATTN_STAU.  NULL means
 * dlog_tau       "not computed"; ignored for the other maps.
 * workspace      attn_bwd_workspace_bytes(desc, variant) bytes, 16-byte
 *                aligned: Yat |q|^2 + b and |k|^2 + b rows per query head,
 *                per-row D and Z, and per-workgroup parameter sums.
 * desc->block_rows and desc->kv_splits are forward launch options and are
 * not used here.  Ownership, asynchrony, errors and empty problems as
 * attn_fwd; ATTN_ERR_UNSUPPORTED for fp32 storage.  The standard maps only
 * (not the options of attn_fwd_yat).  Summation orders are fixed: repeated
 * calls give identical bits. */
size_t attn_bwd_workspace_bytes(const attn_desc* desc, int variant);
int attn_bwd(const attn_desc* desc, const void* q, const void* k, const void* v,
             const void* dout, int variant, const float* b_raw, const float* eps_raw,
             const float* log_tau, int causal, const float* mass, const float* max_score,
             void* dq, void* dk, void* dv, float* db_raw, float* deps_raw, float* dlog_tau,
             void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* attn_status_string(int status);

/* Text of the most recent ATTN_ERR_HIP (or validation detail) on the calling
 * thread; "" if none. */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SFS_ATTN_H */
