/*
 * grpo.h -- C ABI of the fused, chunked GRPO policy loss for AMD MI355X (gfx950).
 *
 * What it computes (sources: Unsloth "Long-context GRPO" blog, Chinese
 * translation at zjt100.com, section on the GRPO maths; Unsloth docs "GRPO
 * with 7x longer context", sections "Flattened sequence length chunking" and
 * "Offloading activations for log softmax"; aibit.im "Mastering GRPO",
 * section "From RLHF and PPO to the efficiency of GRPO"):
 *
 *   tokens   t = b*L + j over B sequences of padded length L (N = B*L)
 *   logits   z_t = W h_t              W: [V, d] LM head, h_t: row t of H [N, d]
 *   lse_t    = log sum_v exp(z_tv)     (max-shifted, float32 or better)
 *   lp_t     = z_{t, y_t} - lse_t      selective log-softmax at the target id
 *   x_t      = ref_lp_t - lp_t
 *   kl_t     = exp(x_t) - x_t - 1      reverse KL, no extra policy factor
 *   l_t      = -(exp(lp_t - stopgrad(lp_t)) * A_{b(t)} - beta * kl_t)
 *              (the ratio's value is 1; its gradient is that of lp_t)
 *   loss     = sum_t m_t l_t / max(sum_t m_t, 1)   masked token mean
 *
 * and the backward of that loss, which recomputes every logit tile instead
 * of keeping a (tokens x vocab) tensor:
 *   c_t  = g * m_t / max(sum m, 1) * (-A_{b(t)} + beta * (1 - exp(x_t)))
 *   dZ_t = c_t * (onehot(y_t) - softmax(z_t))
 *   dH_t = dZ_t W            dW += sum_t dZ_t^T h_t
 *
 * Conventions shared by every call:
 *  - Every pointer argument is a DEVICE pointer unless stated otherwise, to a
 *    dense row-major array owned by the caller.  The library allocates no
 *    memory and keeps no state between calls beyond its loaded code objects.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work and return; nothing is synchronised on the host.
 *  - `dtype` (grpo_dtype) gives the element type of H, H_ref, W and dH
 *    together: GRPO_F32 (float) or GRPO_BF16 (bfloat16).  Logits, log-sum-exp
 *    and every per-token output are float32; dW is always float32.
 *  - Return value: GRPO_OK or a negative grpo_status.  Argument errors are
 *    detected on the host before anything is enqueued; no output is touched
 *    then.  GRPO_ERR_HIP means a launch failed and the outputs are undefined.
 *    grpo_last_error() returns a thread-local text describing the last
 *    failure.
 *  - Device-side preconditions not checked on the host: targets y in
 *    [0, V) (an out-of-range target gives lp = NaN in the forward and an
 *    undefined gradient), mask values in {0, 1}, and no aliasing between
 *    inputs and outputs.
 *  - Shape limits: d must be a multiple of 8 (bf16) or 4 (f32) so that rows
 *    load as 16-byte vectors; N, d, V, chunk >= 1.
 */
#ifndef GRPO_H
#define GRPO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GRPO_F32 = 0, GRPO_BF16 = 1, GRPO_FP8_E4M3 = 2 } grpo_dtype;

typedef enum {
  GRPO_OK = 0,
  GRPO_ERR_INVALID_ARG = -1, /* null pointer, size <= 0, N != B*L, bad dtype, non-finite beta */
  GRPO_ERR_WORKSPACE = -2,   /* workspace pointer null or smaller than grpo_workspace_bytes() */
  GRPO_ERR_UNSUPPORTED = -3, /* shape outside the limits above */
  GRPO_ERR_HIP = -4          /* a HIP launch or runtime call failed */
} grpo_status;

typedef enum {
  GRPO_OP_REF = 0,     /* grpo_ref_logprobs */
  GRPO_OP_FWD = 1,     /* grpo_loss_fwd */
  GRPO_OP_BWD = 2,     /* grpo_loss_bwd, default (fastest) dZ slab */
  GRPO_OP_BWD_MIN = 3  /* grpo_loss_bwd, the least workspace it accepts */
} grpo_op;

/*
 * Workspace bytes that grpo_ref_logprobs (op = GRPO_OP_REF), grpo_loss_fwd
 * (GRPO_OP_FWD) or grpo_loss_bwd (GRPO_OP_BWD, GRPO_OP_BWD_MIN) needs for
 * these sizes.  The workspace is caller-owned device memory with 256-byte
 * alignment; its contents on entry do not matter and are clobbered.  Returns
 * 0 for invalid arguments.  It never scales with N*V: the forward keeps only
 * per-token split partials of one chunk; the backward one chunk of hidden
 * states (and its transpose), per-token scalars, float32 dH partials of one
 * chunk, 8 bytes per token (active-token list, per-sequence counts) and one
 * dZ slab: the gradient of V_s vocabulary columns of the chunk's logits, in
 * H's dtype (bf16 for fp8), stored once, in strips of 256 columns that each
 * hold every active token's 256 values contiguously.
 * The backward plans V_s from the workspace_bytes it is passed: a multiple of
 * 256 columns (up to the whole vocabulary) that fits, the widest one or a
 * narrower one down to half of it where that wastes fewer waves of
 * workgroups, so a caller trades speed for memory by passing any size from
 * grpo_workspace_bytes(GRPO_OP_BWD_MIN, ...) (one 256-column slab) up.
 * GRPO_OP_BWD sizes a slab of at most 1.25 GiB (the whole vocabulary of a
 * 4096-token chunk at the usual LM-head shapes; a wider slab is not faster).
 * The slab's bytes (chunk x V_s) and V_s x d elements of W are each read
 * through one buffer resource, so V_s is also capped below 2^31 bytes for both.
 */
size_t grpo_workspace_bytes(int op, int64_t N, int64_t d, int64_t V, int dtype, int64_t chunk);

/*
 * Automatic chunk size (Unsloth docs, "Flattened sequence length chunking"
 * and "Configuring the parameters": left unset, the chunk multiplier and the
 * hidden-state mini-batch are tuned from the free VRAM and the context
 * length; the multiplier defaults to max(4, context_length // 4096)).  There
 * the chunk's float32 logits are materialised, so memory sets the chunk; here
 * the forward never holds chunk x V logits and the backward's dZ slab has its
 * own bound, so the chunk is chosen for speed within the memory given.
 * Returns the largest multiple of 256 tokens that is at most 8192 (the best
 * measured size at d = 1536 and d = 4096; at 16384 the backward slows down)
 * and at most N = B * L rounded up to 256, for which
 *   grpo_workspace_bytes(GRPO_OP_FWD, ...) + grpo_workspace_bytes(GRPO_OP_BWD, ...)
 * is at most budget_bytes; 256 if no candidate fits.  Pure host arithmetic:
 * no device call, deterministic for given arguments.
 * The caller passes its own budget (for example part of the free HBM) and
 * then uses the result for the workspace query and every call.  Returns 0
 * for invalid arguments.
 */
int64_t grpo_auto_chunk(int64_t B, int64_t L, int64_t d, int64_t V, int dtype, size_t budget_bytes);

/*
 * Group-relative advantages (aibit.im "Mastering GRPO", section "From RLHF
 * and PPO to the efficiency of GRPO": several completions per prompt are
 * scored and the advantage is derived from the group's rewards).
 *   rewards [num_groups * group_size] float32, group-major (group p holds
 *           entries p*group_size .. p*group_size + group_size - 1)
 *   adv     [num_groups * group_size] float32, written:
 *           adv = (r - mean_p) / (std_p + eps), std with divisor n - 1;
 *           a group of one has std 0 (so adv = 0).  NaN rewards propagate
 *           to their own group only.
 */
int grpo_advantages(const float* rewards, int64_t num_groups, int64_t group_size, float eps,
                    float* adv, void* stream);

/*
 * Reference-policy log-probabilities, no gradient (Unsloth blog, GRPO maths:
 * P is the frozen reference model in the reverse-KL term).
 *   H_ref [N, d] dtype; W [V, d] dtype; y [N] int32 target ids.
 *   ref_lp [N] float32, written: log softmax(W h_t)[y_t] for every token.
 *   chunk: flattened tokens per launch (>= 1); the result does not depend on it.
 * Uses exactly the same kernels as grpo_loss_fwd, so H_ref == H gives
 * ref_lp bitwise equal to lp, hence kl == 0 exactly.
 */
int grpo_ref_logprobs(const void* H_ref, const void* W, const int32_t* y, int64_t N, int64_t d,
                      int64_t V, int dtype, int64_t chunk, float* ref_lp, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Forward of the masked token-mean GRPO loss over N = B*L flattened tokens
 * (Unsloth docs, "Flattened sequence length chunking": the (batch x context)
 * axis is flattened and processed `chunk` tokens at a time; no logits are
 * ever written to memory, each vocabulary tile is folded into an online
 * log-sum-exp in registers).
 *   H [N, d] dtype; W [V, d] dtype; y [N] int32; mask [N] uint8 (0/1);
 *   adv [B] float32 (one advantage per sequence); ref_lp [N] float32.
 *   beta: KL weight (0.04 in the pages' setting), finite.
 *   loss [1] float32, written.
 *   lp, kl, lse [N] float32, written for every token, masked or not
 *   (kl unscaled by beta; lse is what grpo_loss_bwd needs back).
 */
int grpo_loss_fwd(const void* H, const void* W, const int32_t* y, const uint8_t* mask,
                  const float* adv, const float* ref_lp, int64_t B, int64_t L, int64_t d,
                  int64_t V, int dtype, float beta, int64_t chunk, float* loss, float* lp,
                  float* kl, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of grpo_loss_fwd's loss with upstream gradient grad_loss (Unsloth
 * docs, "Offloading activations for log softmax": the backward recomputes
 * the chunk's logits rather than keeping them from the forward).  Only
 * unmasked tokens are visited (masked tokens have zero gradient).
 *   H, W, y, mask, adv, ref_lp as in grpo_loss_fwd; lp and lse [N] float32
 *   are the forward's outputs for the same inputs.
 *   dH [N, d] dtype, OVERWRITTEN (rows of masked tokens become 0).
 *   dW [V, d] float32, ACCUMULATED (+=): the caller zeroes it first for a
 *   plain gradient.
 *   workspace_bytes: at least grpo_workspace_bytes(GRPO_OP_BWD_MIN, ...)
 *   (GRPO_ERR_WORKSPACE otherwise); the dZ slab is planned from it (see
 *   grpo_workspace_bytes), so results depend on it only through the
 *   summation order of dH over slabs.
 */
int grpo_loss_bwd(const void* H, const void* W, const int32_t* y, const uint8_t* mask,
                  const float* adv, const float* ref_lp, const float* lp, const float* lse,
                  int64_t B, int64_t L, int64_t d, int64_t V, int dtype, float beta,
                  float grad_loss, int64_t chunk, void* dH, float* dW, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * Options of the _ex calls.  A zero-initialised struct (or a NULL pointer)
 * gives exactly the plain calls.
 *
 * Logit transform (Unsloth docs, "Flattened sequence length chunking": the
 * chunked log-softmax takes logit_scale_multiply, logit_scale_divide,
 * logit_softcapping and temperature, and supports softcapping and
 * temperature).  The pages give no formulas; applied here in the order of
 * those arguments to every logit z = h . w before the log-softmax:
 *   z * multiply, / divide, cap * tanh(z / cap), / temperature.
 * A zero multiply, divide or cap is "off"; a zero temperature means 1.  Every
 * float field must be finite and >= 0 (GRPO_ERR_INVALID_ARG otherwise).  lp,
 * lse, kl and the gradients are those of the transformed logits.
 *
 * Loss variants (Unsloth blog, GRPO maths: the four-run ablation trains the
 * reference loss, the loss with the detach removed, a "full" reverse KL with
 * the extra factor Q and a forward KL; the formulas are lost, so these are
 * the plainest readings), with x = ref_lp - lp and r = exp(x):
 *   kl_estimator  GRPO_KL_REVERSE    kl = r - x - 1 (k3; the default)
 *                 GRPO_KL_FORWARD    kl = r x - (r - 1), the estimator of
 *                                    KL(ref || policy) from policy samples
 *                 GRPO_KL_REVERSE_Q  kl = exp(lp) (r - x - 1), the factor
 *                                    differentiated with the term
 *   no_detach     1: the ratio is exp(lp - lp) -- still 1 in value, but the
 *                 advantage term then carries no gradient
 *   aggregation   GRPO_AGG_TOKEN_MEAN     sum_t m_t l_t / max(sum m, 1)
 *                 GRPO_AGG_SEQUENCE_MEAN  (1/B) sum_b sum_j m l / max(n_b, 1),
 *                                         n_b = sum_j m_{b,j}; an empty
 *                                         sequence adds 0 and counts in B
 * The backward coefficient follows: c_t = g w_t (-[no_detach = 0] A +
 * beta dkl/dlp) with w_t the aggregation weight and dkl/dlp = 1 - r, -x r,
 * -x exp(lp) for the three estimators.  Values outside these sets:
 * GRPO_ERR_INVALID_ARG.  grpo_ref_logprobs_ex uses only the logit transform.
 */
typedef enum { GRPO_KL_REVERSE = 0, GRPO_KL_FORWARD = 1, GRPO_KL_REVERSE_Q = 2 } grpo_kl_estimator;
typedef enum { GRPO_AGG_TOKEN_MEAN = 0, GRPO_AGG_SEQUENCE_MEAN = 1 } grpo_aggregation;

typedef struct grpo_opts {
  float logit_scale_multiply;
  float logit_scale_divide;
  float logit_softcapping;
  float temperature;
  int32_t kl_estimator;   /* grpo_kl_estimator */
  int32_t no_detach;      /* 0 or 1 */
  int32_t aggregation;    /* grpo_aggregation */
} grpo_opts;

/*
 * grpo_ref_logprobs, grpo_loss_fwd and grpo_loss_bwd with options (`opts`
 * may be NULL: exactly the calls above).  Arguments and outputs are otherwise
 * those of the plain calls; grpo_loss_bwd_ex must get the opts of the
 * grpo_loss_fwd_ex call that produced lp and lse, and the reference
 * log-probs are taken with the same logit transform.  kl holds the selected
 * estimator's per-token value.
 */
int grpo_ref_logprobs_ex(const void* H_ref, const void* W, const int32_t* y, int64_t N, int64_t d,
                         int64_t V, int dtype, int64_t chunk, const grpo_opts* opts,
                         float* ref_lp, void* workspace, size_t workspace_bytes, void* stream);
int grpo_loss_fwd_ex(const void* H, const void* W, const int32_t* y, const uint8_t* mask,
                     const float* adv, const float* ref_lp, int64_t B, int64_t L, int64_t d,
                     int64_t V, int dtype, float beta, int64_t chunk, const grpo_opts* opts,
                     float* loss, float* lp, float* kl, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream);
int grpo_loss_bwd_ex(const void* H, const void* W, const int32_t* y, const uint8_t* mask,
                     const float* adv, const float* ref_lp, const float* lp, const float* lse,
                     int64_t B, int64_t L, int64_t d, int64_t V, int dtype, float beta,
                     float grad_loss, int64_t chunk, const grpo_opts* opts, void* dH,
                     float* dW, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8 path (Unsloth docs: FP8 RL training is offered; Unsloth blog, "Unsloth
 * efficient GRPO algorithm": a naive float8 linear cross-entropy breaks loss
 * scaling).  The pages give no recipe; here the LM-head GEMM takes OCP float8
 * e4m3 ("fn": bias 7, 3 mantissa bits, no infinities, largest 448) codes with
 * float32 accumulation (v_mfma_f32_16x16x128_f8f6f4, twice the bf16 rate) and
 * float32 log-sum-exp.  Each hidden-state row (token) has its own scale and
 * the head one scale; the logit is z = (sum_k h8 w8) * w_scale * h_scale[t].
 * Scales are powers of two, so dequantised values are exact.
 *
 * grpo_quantize_fp8: X [rows, cols] (GRPO_F32 or GRPO_BF16, device) ->
 *   codes [rows, cols] uint8 and scales (float32, device): per_row = 1 gives
 *   scales[rows], per_row = 0 one scales[0] for the tensor.  The scale of a
 *   row (or tensor) is 2^e with e the smallest integer such that its largest
 *   |x| <= 448 * 2^e (e = 0 for an all-zero block); codes are x / 2^e rounded
 *   to the nearest e4m3 value, ties to even (the division is exact).  cols must
 *   be a multiple of 16.  per_row = 0 needs grpo_quantize_fp8_workspace_bytes()
 *   of workspace (partial maxima); per_row = 1 needs none (NULL allowed).
 * grpo_dequantize_fp8: out [rows, cols] bfloat16 = codes * scale, exact.
 * grpo_ref_logprobs_fp8, grpo_loss_fwd_fp8: grpo_ref_logprobs_ex and
 *   grpo_loss_fwd_ex on fp8 codes H8 [N, d] (h_scale [N]) and W8 [V, d]
 *   (w_scale [1]); outputs and workspace (grpo_workspace_bytes with dtype
 *   GRPO_FP8_E4M3) as there.  d must be a multiple of 16.
 * grpo_loss_bwd_fp8: the backward of that loss with respect to the dequantised
 *   H and W.  The logits are recomputed from the fp8 codes through the same
 *   MFMA loop as the forward (so they equal the forward's), and dH = dZ W,
 *   dW += dZ^T H run in bfloat16 on exact bfloat16 copies of H and W that it
 *   writes into its workspace (grpo_workspace_bytes(GRPO_OP_BWD, ...,
 *   GRPO_FP8_E4M3, chunk) includes them and one chunk of gathered fp8 rows);
 *   dH [N, d] is bfloat16.
 */
size_t grpo_quantize_fp8_workspace_bytes(void);
int grpo_quantize_fp8(const void* X, int dtype, int64_t rows, int64_t cols, int per_row,
                      uint8_t* codes, float* scales, void* workspace, size_t workspace_bytes,
                      void* stream);
int grpo_dequantize_fp8(const uint8_t* codes, const float* scales, int64_t rows, int64_t cols,
                        int per_row, void* out, void* stream);
int grpo_ref_logprobs_fp8(const uint8_t* H8, const float* h_scale, const uint8_t* W8,
                          const float* w_scale, const int32_t* y, int64_t N, int64_t d, int64_t V,
                          int64_t chunk, const grpo_opts* opts, float* ref_lp, void* workspace,
                          size_t workspace_bytes, void* stream);
int grpo_loss_fwd_fp8(const uint8_t* H8, const float* h_scale, const uint8_t* W8,
                      const float* w_scale, const int32_t* y, const uint8_t* mask,
                      const float* adv, const float* ref_lp, int64_t B, int64_t L, int64_t d,
                      int64_t V, float beta, int64_t chunk, const grpo_opts* opts, float* loss,
                      float* lp, float* kl, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream);
int grpo_loss_bwd_fp8(const uint8_t* H8, const float* h_scale, const uint8_t* W8,
                      const float* w_scale, const int32_t* y, const uint8_t* mask,
                      const float* adv, const float* ref_lp, const float* lp, const float* lse,
                      int64_t B, int64_t L, int64_t d, int64_t V, float beta, float grad_loss,
                      int64_t chunk, const grpo_opts* opts, void* dH, float* dW, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * grpo_loss_fwd_ex without a workspace argument.  Its scratch is a static
 * device array of grpo_noalloc_scratch_bytes() (64 MiB) that each GPU holds
 * for the life of the process; it is located once per device (on the first
 * call there, with that device current) and nothing is allocated, by the
 * library or on its behalf, in any call.  Shapes whose forward workspace
 * (grpo_workspace_bytes(GRPO_OP_FWD, ...)) exceeds it are rejected with
 * GRPO_ERR_WORKSPACE before anything is enqueued; that allows chunks of up
 * to 13 824 tokens at a 151 936-token vocabulary (10 496 at 201 088) for up to
 * 163 840 flattened tokens.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race and give undefined results.  Nothing in the scratch needs to
 * start at zero.  Arguments and results are otherwise exactly those of
 * grpo_loss_fwd_ex, whose kernels it runs.
 */
size_t grpo_noalloc_scratch_bytes(void);
int grpo_loss_fwd_noalloc(const void* H, const void* W, const int32_t* y, const uint8_t* mask,
                          const float* adv, const float* ref_lp, int64_t B, int64_t L, int64_t d,
                          int64_t V, int dtype, float beta, int64_t chunk, const grpo_opts* opts,
                          float* loss, float* lp, float* kl, float* lse, void* stream);

/*
 * Diagnostic: C[M, N] (float32, row-major, written) = A[M, K] . B[N, K]^T,
 * through the same MFMA tile main loop the loss kernels use (A, B dtype
 * elements, both rows contiguous along K).  K times the element size must be
 * a multiple of 16 bytes.  Used by the parity tests to check that loop on
 * its own; not part of the loss itself.
 */
int grpo_gemm_nt(const void* A, const void* B, int64_t M, int64_t N, int64_t K, int dtype,
                 float* C, void* stream);

/*
 * Diagnostics: per-kernel timing with HIP events, off by default.  After
 * grpo_timing_begin(), every kernel launch that this thread's library calls
 * enqueue is bracketed by two HIP events recorded on the launch's own stream.
 * grpo_timing_end() waits for those events and writes, for each kernel that
 * ran, its name (static string), launch count and summed elapsed time in
 * milliseconds into the caller's HOST arrays of max_entries; it returns the
 * number of kernels that ran (entries past max_entries are dropped) and
 * switches timing off.  Used by the benchmark for its roofline figure.
 */
int grpo_timing_begin(void);
int grpo_timing_end(const char** names, int* launches, double* total_ms, int max_entries);

/* Static text for a grpo_status code. */
const char* grpo_strerror(int code);

/* Thread-local text describing the most recent failure on this thread ("" if none). */
const char* grpo_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GRPO_H */
