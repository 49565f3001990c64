/*
 * muon.h — C ABI of libmuon: the Muon optimizer step and MuonClip's QK-Clip
 * for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [MC] "MuonClip" — 02 Muon from first principles; 03 Making Muon scale;
 *        05 QK-Clip; 06 Multi-head latent attention changes the surgery;
 *        07 One complete training step.
 *   [MM] "Muon and MuonClip: orthogonalised updates for LLM training" —
 *        section 2: "Newton-Schulz: an odd polynomial on singular values",
 *        "The Muon optimizer", "The exploding-logit problem",
 *        "MuonClip: QK-clip, per head, adapted to MLA".
 *   [MS] "About Muon: Muon At Scale" — "Why Not Bernstein's Multiplier?",
 *        "When Softmax Collapses", "What Breaks at Scale" ("The Matrix Does
 *        Not Fit": Dion).
 *
 * Conventions shared by every entry point
 *   - All pointers are DEVICE pointers unless stated otherwise; the structs
 *     passed by pointer (muon_group_t, qkclip_slice_t and adamw_tensor_t
 *     arrays, muon_hparams_t, adamw_hparams_t) are HOST memory read during
 *     the call only.
 *   - Matrices are row-major [rows][cols] with rows = fan-out (the layout of
 *     a Linear weight).  A group is `batch` same-shape matrices, matrix b
 *     starting `batch_stride` elements after matrix b-1.
 *   - bf16 is IEEE binary32's upper half, passed as uint16_t storage.
 *   - The caller owns every buffer.  The library never allocates device
 *     memory.  Scratch space is the caller's `workspace`, sized by the
 *     matching *_workspace_size query; its contents are undefined between
 *     calls except where a layout query below says otherwise.
 *   - Every call is asynchronous on `stream` and never synchronises it.
 *     Argument errors are detected on the host before any launch and are
 *     returned synchronously; nothing is launched then.  Launch failures
 *     return MUON_ERR_HIP.  Data-dependent conditions (non-finite values)
 *     never raise errors: NaN/Inf in gradients propagate into the outputs;
 *     a non-finite S_max is reported through the `clipped` flags.
 *   - Calls on different streams are safe if their workspaces and outputs
 *     do not overlap.  The optional profiler (muon_profile_*) is process-wide
 *     and not thread-safe.
 *   - Every entry point that launches work opens a named roctx range (and
 *     muon_step one per stage), visible to rocprofv3 --marker-trace; the
 *     library links librocprofiler-sdk-roctx for them.
 */
#ifndef MUON_H
#define MUON_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad enum   */
  MUON_ERR_UNSUPPORTED = 2, /* valid but not built (e.g. d_head not 64/128/256) */
  MUON_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required  */
  MUON_ERR_HIP = 4          /* a HIP launch or runtime call failed          */
} muon_status_t;

typedef enum { MUON_DTYPE_F32 = 0, MUON_DTYPE_BF16 = 1 } muon_dtype_t;

/* Multiplier on the orthogonalised update ([MC] 03; [MS] "Why Not Bernstein's
 * Multiplier?"):
 *   MOONLIGHT: rms_target * sqrt(max(rows, cols))  (entry RMS ~ rms_target)
 *   SPECTRAL:  sqrt(rows / cols)                   (sqrt(fan-out / fan-in))
 *   NONE:      1                                                            */
typedef enum {
  MUON_SCALE_MOONLIGHT = 0,
  MUON_SCALE_SPECTRAL = 1,
  MUON_SCALE_NONE = 2
} muon_scale_mode_t;

/* Hyper-parameters of one Muon step.
 *   momentum:  M_t = momentum * M_{t-1} + G_t  ([MC] 02; sum form)
 *   nesterov:  nonzero -> Newton-Schulz input U = G_t + momentum * M_t,
 *              zero    -> U = M_t
 *   ns_*:      ns_steps iterations of X <- a X + (b A + c A A) X, A = X X^T,
 *              on X_0 = U / (||U||_F + ns_eps) in the wide orientation
 *              (transpose when rows > cols)  ([MM] Newton-Schulz subsection)
 *   update:    W <- (1 - lr * weight_decay) W - lr * scale * O  ([MC] 03),
 *              in fp32, rounded once (nearest-even) to the parameter dtype. */
typedef struct {
  float lr;
  float momentum;
  float weight_decay;
  int32_t nesterov;
  int32_t ns_steps; /* 0..64 */
  float ns_a, ns_b, ns_c;
  float ns_eps;
  int32_t scale_mode; /* muon_scale_mode_t */
  float rms_target;   /* used by MUON_SCALE_MOONLIGHT */
} muon_hparams_t;

/* One group of same-shape matrices.  param/grad: param dtype; momentum: fp32;
 * all three [batch][rows][cols] with the same batch_stride (in elements,
 * >= rows*cols).  param and momentum are updated in place; grad is read.
 * Size limit, here and in ns_orthogonalize: rows, cols <= 2^20 and
 * (max(rows, cols) + 256) * (min(rows, cols) + 256) <= 2^31, about 2.1e9
 * elements per matrix (8192 x 253944, 46084 x 46084); beyond it the calls
 * return MUON_ERR_INVALID_ARG and the workspace queries 0.  batch and
 * batch_stride are not limited. */
typedef struct {
  void* param;
  const void* grad;
  float* momentum;
  int32_t batch;
  int32_t rows;
  int32_t cols;
  int32_t reserved; /* must be 0 */
  int64_t batch_stride;
} muon_group_t;

#define MUON_MAX_GROUPS 16

/* ---------------------------------------------------------------- muon_step
 * One full Muon step ([MC] 07 pseudocode order) over n_groups groups sharing
 * one parameter dtype: momentum update and Nesterov lookahead fused with the
 * Frobenius partial sums in one pass; Newton-Schulz on bf16 MFMA with fp32
 * accumulation, every same-shape matrix of every group batched into one
 * launch per stage; then the scaled, decayed parameter write.  X, A = X X^T
 * and B = b A + c A A are stored in bf16 between products, except for wide
 * views of at most 96 rows, whose A and B are kept to about 2^-17 (a bf16
 * pair hi + lo): with so few singular values a bf16 rounding of B is not
 * averaged over directions.
 *   groups:          host array of n_groups descriptors (1..MUON_MAX_GROUPS)
 *   param_dtype:     MUON_DTYPE_F32 or MUON_DTYPE_BF16 (grads share it)
 *   hp:              host pointer, see muon_hparams_t
 *   workspace:       device scratch of >= muon_step_workspace_size(...) bytes,
 *                    256-byte aligned
 * Returns MUON_OK or an error code (see conventions).                       */
size_t muon_step_workspace_size(const muon_group_t* groups, int n_groups);
int muon_step(const muon_group_t* groups, int n_groups, int param_dtype,
              const muon_hparams_t* hp, void* workspace, size_t workspace_bytes,
              hipStream_t stream);

/* Where muon_step leaves its intermediate results, as byte offsets into the
 * workspace of the last call with the same groups (valid until the workspace
 * is reused):
 *   o_offset:       bf16 Newton-Schulz output O of group g, in the group's
 *                   own layout: matrix b, element (i, j) at
 *                   o_offset + 2 * (b * o_batch_stride + i * o_ld + j)
 *   inv_norm_offset: fp32 [batch] values 1 / (||U_b||_F + ns_eps)
 *   x0_offset:       bf16 U (unnormalised, rounded once) in the wide
 *                   orientation: (i, j) of the m x n wide view at
 *                   x0_offset + 2 * (b * x0_batch_stride + i * x0_ld + j);
 *                   only after a call with ns_steps == 1 (later iterations
 *                   reuse that buffer)                                      */
typedef struct {
  size_t o_offset;
  int64_t o_batch_stride;
  int64_t o_ld;
  size_t inv_norm_offset;
  size_t x0_offset;
  int64_t x0_batch_stride;
  int64_t x0_ld;
} muon_ws_layout_t;
int muon_step_workspace_layout(const muon_group_t* groups, int n_groups, int g,
                               int ns_steps, muon_ws_layout_t* out);

/* ---------------------------------------------------------- ns_orthogonalize
 * Newton-Schulz alone ([MM] Newton-Schulz subsection): for each of `batch`
 * matrices in (dtype in_dtype, [rows][cols], batch_stride elements apart),
 * out = NS_steps(in / (||in||_F + eps)) written as bf16 into `out`, dense
 * [batch][rows][cols].  Same arithmetic and kernels as muon_step.          */
size_t ns_workspace_size(int batch, int rows, int cols);
int ns_orthogonalize(const void* in, int in_dtype, uint16_t* out, int batch,
                     int rows, int cols, int64_t batch_stride, int steps,
                     float a, float b, float c, float eps, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------- qkclip_rowmax
 * Per-head maximum pre-softmax logit ([MM] "The exploding-logit problem";
 * [MC] 05 per-head signal):
 *   s_max[h] = logit_scale * max over b < B, i < T, j < T (j <= i if causal)
 *              of sum_t Q[b,i,h,t] * K[b,j,h,t]
 * Q, K: bf16 [B][T][H][d_head] (the forward's projections, row-major).
 * logit_scale is normally 1/sqrt(d_head).  d_head must be 64, 128 or 256.
 * s_max: fp32 [H] device output.  A NaN anywhere in a head's logits makes
 * s_max[h] NaN.  Products are bf16 x bf16 exact, accumulated in fp32.
 * workspace: >= qkclip_rowmax_workspace_size(B, T, H) bytes.               */
size_t qkclip_rowmax_workspace_size(int B, int T, int H);
int qkclip_rowmax(const uint16_t* Q, const uint16_t* K, int B, int T, int H,
                  int d_head, float logit_scale, int causal, float* s_max,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ----------------------------------------------------- qkclip_rowmax_noalloc
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * statistic as qkclip_rowmax, same kernels and results bit for bit, with no
 * workspace argument.  Its partial maxima (B * H * ceil(T / q) floats, with
 * q = 512 queries per block for d_head = 128 and 256 otherwise) live in a
 * 1 MiB array inside the library, one per GPU, held until the process ends;
 * the call allocates nothing.  Limit:
 *   B * H * ceil(T / q) <= qkclip_rowmax_noalloc_max_partials() (262144),
 * else MUON_ERR_WORKSPACE with nothing launched; the other argument errors are
 * qkclip_rowmax's.  Every call on one GPU shares that array: calls that
 * overlap in time on one GPU (concurrent streams, or threads) race and must
 * be serialised by the caller; the array keeps the last call's partials,
 * and nothing in it needs to start at zero.                                 */
size_t qkclip_rowmax_noalloc_max_partials(void);
int qkclip_rowmax_noalloc(const uint16_t* Q, const uint16_t* K, int B, int T,
                          int H, int d_head, float logit_scale, int causal,
                          float* s_max, hipStream_t stream);

/* ------------------------------------------------------------------ attn_fwd
 * Softmax attention forward that also produces QK-Clip's statistic, the way
 * the pages place it ([MC] 05: the per-head signal is read off the forward;
 * [MM] "The exploding-logit problem": the logits that feed the softmax):
 *   s_ij = logit_scale * q_i . k_j  (j <= i if causal, per batch row and head)
 *   O[b,i,h,:] = sum_j softmax_j(s_ij) V[b,j,h,:]
 *   lse[b,h,i] = log sum_j exp(s_ij)               (natural log; optional)
 *   s_max[h]   = max over b, i, j of s_ij           (as qkclip_rowmax)
 * Q, K, V, O: bf16 [B][T][H][d_head], d_head must be 128; lse: fp32
 * [B][H][T] or NULL; s_max: fp32 [H].  Scores and the softmax run in fp32,
 * the probabilities enter the P.V product as bf16, O is rounded once.
 * A NaN logit makes s_max[h] NaN (and propagates into O).
 * workspace: >= attn_fwd_workspace_size(B, T, H) bytes, 16-byte aligned.   */
size_t attn_fwd_workspace_size(int B, int T, int H);
int attn_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int B,
             int T, int H, int d_head, float logit_scale, int causal,
             uint16_t* O, float* lse, float* s_max, void* workspace,
             size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------ qkclip_rescale
 * Balanced MHA QK-Clip ([MC] 05 balanced rescale; [MS] "When Softmax
 * Collapses"): for each head h with finite s_max[h] > tau,
 *   gamma = tau / s_max[h];  rows [h*d_head, (h+1)*d_head) of Wq *= gamma^alpha,
 *   the same rows of Wk *= gamma^(1-alpha)  (fp32 product, one rounding).
 * Heads with s_max <= tau are untouched; NaN/Inf s_max leaves the head
 * untouched.  Wq, Wk: [H*d_head][d_model] of `dtype`, updated in place.
 * s_max: fp32 [H] device input (e.g. from qkclip_rowmax).  clipped: optional
 * int32 [H] device output, 1 clipped, 0 untouched, -1 non-finite s_max.
 * The momentum buffers are not touched ([MC] 07).                          */
int qkclip_rescale(void* Wq, void* Wk, int dtype, int H, int d_head,
                   int d_model, const float* s_max, float tau, float alpha,
                   int32_t* clipped, hipStream_t stream);

/* ---------------------------------------------------- qkclip_rescale_slices
 * The same per-head rule over up to QKCLIP_MAX_SLICES row slices, for any
 * layout in which each head owns a run of consecutive rows: head h owns rows
 * [h*head_pitch, h*head_pitch + rows_per_head) counted from `w` (a device
 * pointer of `dtype`, row-major, `cols` elements per row), and for a clipped
 * head those rows are multiplied by gamma^exponent, exponent in [0, 1].
 * head_pitch > rows_per_head describes fused projections whose per-head
 * blocks interleave several parts (point `w` at the part's first row).
 * Slices must not overlap.  s_max, tau, clipped as for qkclip_rescale.     */
#define QKCLIP_MAX_SLICES 4
typedef struct {
  void* w;
  int64_t head_pitch;   /* rows between the first rows of heads h and h+1 */
  int rows_per_head;
  int cols;
  float exponent;
} qkclip_slice_t;
int qkclip_rescale_slices(const qkclip_slice_t* slices, int n_slices,
                          int dtype, int H, const float* s_max, float tau,
                          int32_t* clipped, hipStream_t stream);

/* -------------------------------------------------------- qkclip_rescale_mla
 * QK-Clip for multi-head latent attention ([MC] 06; [MM] "MuonClip: QK-clip,
 * per head, adapted to MLA"): for a clipped head the head-specific content query rows
 * (Wqc, [H*d_c][q_cols]) and content key rows (Wkc, [H*d_c][kv_cols]) are
 * multiplied by sqrt(gamma), the head-specific rotary query rows (Wqr,
 * [H*d_r][q_cols]) by gamma, and the rotary key shared by all heads is left
 * alone (it takes no argument).  Equivalent to qkclip_rescale_slices with
 * exponents 1/2, 1/2, 1.                                                    */
int qkclip_rescale_mla(void* Wqc, void* Wkc, void* Wqr, int dtype, int H,
                       int d_c, int d_r, int q_cols, int kv_cols,
                       const float* s_max, float tau, int32_t* clipped,
                       hipStream_t stream);

/* ---------------------------------------------------------------- adamw_step
 * Decoupled AdamW for the parameters outside Muon's 2-D hidden matrices
 * (embeddings, output head, norms, biases: [MC] 03 routing and 07 step; the
 * pages name AdamW without writing it out, so this is the standard form):
 *   m <- beta1 m + (1 - beta1) g;   v <- beta2 v + (1 - beta2) g^2
 *   p <- p (1 - lr wd) - lr (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 * with t = hp->step >= 1.  Each tensor is a flat run of `numel` elements:
 * param and grad of `dtype` (bf16 rounds p once, RNE), exp_avg and
 * exp_avg_sq fp32, all updated in place except grad.  Any number of tensors
 * per call; they are packed into as few launches as the argument block
 * allows.  numel == 0 entries are skipped.  fp32 arithmetic.                */
typedef struct {
  float lr;
  float beta1;
  float beta2;
  float eps;
  float weight_decay;
  int step;
} adamw_hparams_t;
typedef struct {
  void* param;
  const void* grad;
  float* exp_avg;
  float* exp_avg_sq;
  int64_t numel;
} adamw_tensor_t;
int adamw_step(const adamw_tensor_t* tensors, int n_tensors, int dtype,
               const adamw_hparams_t* hp, hipStream_t stream);

/* ----------------------------------------------------------------- dion_step
 * One rank-r Dion step ([MS] "What Breaks at Scale", "The Matrix Does Not
 * Fit") on each of `batch` matrices (param and grad of `dtype`, [rows][cols],
 * batch_stride elements apart; momentum fp32 with the same layout):
 *   B = M + G;  P = orth(B Q);  R = B^T P;
 *   M <- B - (1 - mu) P R^T;  Q <- ColNorm(R);  W <- W - lr P Q^T
 *   q:      fp32 [batch][cols][rank], dense, the caller's state between steps
 *           (the power step's warm start): read, then replaced by ColNorm(R).
 *   orth:   the basis of the thin QR of B Q with a positive diagonal,
 *           computed by Cholesky-QR applied twice (Gram matrices and their
 *           Cholesky factors in fp64, products in fp32).  A direction the
 *           columns of B Q do not add (pivot <= 1e-10 x the largest diagonal
 *           entry of the Gram matrix) gets a zero column of P, so it takes no
 *           update and its column of Q becomes zero.
 *   ColNorm: each column of R over its l2 norm; a zero column stays zero.
 *   No scale factor or weight decay (the pages' update has neither).
 *   Arithmetic fp32 (momentum, products, update), param rounded once (RNE).
 * Requirements (else MUON_ERR_UNSUPPORTED): rank a multiple of 8 in 8..128,
 * rank <= min(rows, cols); rows and cols multiples of 8; batch_stride a
 * multiple of 8; every pointer 16-byte aligned.  Other argument errors:
 * MUON_ERR_INVALID_ARG; a missing or short workspace: MUON_ERR_WORKSPACE.   */
size_t dion_workspace_size(int batch, int rows, int cols, int rank);
int dion_step(void* param, int dtype, const void* grad, float* momentum, float* q,
              int batch, int rows, int cols, int rank, int64_t batch_stride,
              float lr, float mu, void* workspace, size_t workspace_bytes,
              hipStream_t stream);

/* -------------------------------------------------------------- diagnostics */
const char* muon_status_string(int status);

/* Matrix-core rate probe (not part of the optimizer): `blocks` workgroups of
 * 256 threads, each wave issuing 32 * iters v_mfma_f32_32x32x16_bf16 on
 * register operands (eight independent accumulators), no memory traffic in
 * the loop; 32768 flop per MFMA, so blocks * 4 * 32 * iters * 32768 flop per
 * launch.  Time it with events on `stream` to get the sustained bf16 MFMA rate
 * at the clock the chip holds under that load.  The matrix cores draw more
 * power on random operands than on smooth ones, so the rate depends on the
 * operand kind: MUON_PROBE_RANDOM (pseudo-random bf16 of both signs, like the
 * Newton-Schulz iterates) or MUON_PROBE_SMOOTH (small positive values that
 * vary slowly across lanes).  sink: device float[blocks], written once per
 * block.  MUON_ERR_INVALID_ARG for blocks outside 1..2^20, iters outside
 * 1..2^24, an unknown operand kind or a null sink. */
#define MUON_PROBE_RANDOM 0
#define MUON_PROBE_SMOOTH 1
int muon_mfma_probe(int blocks, int iters, int operands, float* sink, hipStream_t stream);

/* HBM stream probe (not part of the optimizer): units = min(src_bytes /
 * (16 reads), dst_bytes / (16 writes)); unit u reads the 16-byte chunks
 * src[i * units + u], i < reads, and writes dst[k * units + u], k < writes
 * (the XOR of its loads with k in the first word), all nontemporal, so every
 * wave instruction moves 1 KB of consecutive bytes; each thread takes
 * `unroll` units (1 or 4), all their loads issued first.  Timed with events on
 * `stream`, it gives the HBM rate this chip sustains for a read/write mix:
 * (reads, writes) = (3, 4) is the momentum pass's 6 B read and 8 B written
 * per element, (2, 1) the update pass's, (1, 1) a copy.  src and dst: device,
 * 16-byte aligned, not overlapping.  Returns the bytes the launch moves
 * (units * 16 * (reads + writes)), or minus an error code: an unlisted mix,
 * null or misaligned pointers, another unroll, or units outside 1..2^36 give
 * -MUON_ERR_INVALID_ARG, a failed launch -MUON_ERR_HIP. */
int64_t muon_hbm_probe(const void* src, size_t src_bytes, void* dst, size_t dst_bytes, int reads,
                       int writes, int unroll, hipStream_t stream);

/* Optional per-kernel timing with HIP events recorded around every launch
 * the library makes on the caller's stream.  muon_profile_enable(1) clears
 * and starts recording; muon_profile_collect() waits for the recorded events,
 * fills up to n_kinds entries of total milliseconds and launch counts per
 * kernel kind (index = kind id) and returns the number of kinds.
 * muon_kernel_kind_name(k) names kind k.  Process-wide, not thread-safe.   */
int muon_profile_enable(int on);
int muon_profile_collect(double* total_ms, int64_t* launches, int n_kinds);
const char* muon_kernel_kind_name(int kind);

#ifdef __cplusplus
}
#endif
#endif /* MUON_H */
